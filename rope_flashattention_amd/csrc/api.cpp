// C ABI of librope_fa: host-side validation and dispatch.
//
// Every check here runs before any HIP call, so an invalid call enqueues nothing and
// writes nothing.  Constraint sources: the [DynamicNTKOperation] page, section 约束说明
// (table limits) and 参数列表 (UNDEFINED output dtype is unusable); the [RoPE-fusion
// blog]'s warning that a fused operator must not silently fall back (here: unsupported
// shapes, strides and alignments are errors).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "common.h"
#include "rope_fa.h"

namespace ropefa {
hipError_t launch_rope_tables(const int32_t* pos, const float* inv_freq, const int32_t* seq_lens, int32_t batch,
                              int32_t ntokens, int32_t head_size, float pos_scale, rope_dtype out_dtype,
                              int pairing, int angle_mode, void* sin_out, void* cos_out, hipStream_t stream);
hipError_t launch_rope_qk(const rope_attn_params* p, hipStream_t stream);
hipError_t launch_flash_fwd(const rope_attn_params* p, const void* kprime, hipStream_t stream);
hipError_t launch_rope_k_prepass(const rope_attn_params* p, void* kout, hipStream_t stream);
uint64_t flash_fwd_workspace_bytes(const rope_attn_params* p);
hipError_t launch_kv_cache(const rope_kv_cache_params* p, hipStream_t stream);
hipError_t launch_decode(const rope_decode_params* p, hipStream_t stream);
hipError_t launch_flash_bwd(const rope_attn_bwd_params* p, hipStream_t stream);
uint64_t flash_bwd_workspace_bytes(const rope_attn_params* f);
int decode_num_splits(const rope_decode_params* p);
uint64_t decode_workspace_bytes(const rope_decode_params* p, int nsplit);
hipError_t decode_scratch(hipStream_t stream, void** out);
}  // namespace ropefa

using ropefa::dtype_bytes;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(rope_dtype dt) { return dt == ROPE_DT_F16 || dt == ROPE_DT_BF16 || dt == ROPE_DT_F32; }

bool valid_pairing(rope_pairing pr) { return pr == ROPE_PAIR_HALF || pr == ROPE_PAIR_INTERLEAVED; }

constexpr int64_t kMaxTokenStrideBytes = (int64_t)1 << 26;

// Strides {batch, token, head, dim}: dim must be 1; the others non-negative and 16-byte multiples.
rope_status check_strides(const int64_t s[4], int elem_bytes, bool varlen) {
    if (s[3] != 1) return ROPE_ERR_UNSUPPORTED;
    for (int i = 0; i < 3; ++i) {
        if (varlen && i == 0) continue;
        if (s[i] < 0) return ROPE_ERR_SHAPE;
        if ((s[i] * elem_bytes) % 16 != 0) return ROPE_ERR_UNSUPPORTED;
    }
    return ROPE_OK;
}

// Checks shared by rope_qk and rope_flash_attn_fwd.
rope_status check_params(const rope_attn_params* p, bool attention) {
    if (!p) return ROPE_ERR_NULL;
    if (p->struct_size != sizeof(rope_attn_params)) return ROPE_ERR_ABI;
    for (unsigned char c : p->rsv)
        if (c) return ROPE_ERR_ABI;
    if (!valid_dtype(p->dtype)) return ROPE_ERR_DTYPE;
    if (!valid_pairing(p->pairing)) return ROPE_ERR_UNSUPPORTED;
    if (!p->q || !p->k) return ROPE_ERR_NULL;
    if ((p->cos == nullptr) != (p->sin == nullptr)) return ROPE_ERR_NULL;
    const bool gen = p->cos == nullptr && p->pos != nullptr;  // tables formed in the kernel
    if (attention) {
        if (!p->v || !p->out) return ROPE_ERR_NULL;
    } else {
        if (!p->out_q || !p->out_k) return ROPE_ERR_NULL;
        if (!p->cos && !gen) return ROPE_ERR_NULL;  // the Rope op needs its tables
    }
    if (gen) {
        if (!p->inv_freq) return ROPE_ERR_NULL;
        if (!(std::isfinite(p->pos_scale) && p->pos_scale > 0.0f)) return ROPE_ERR_SHAPE;
        if (p->inv_freq_rows != 1 && p->inv_freq_rows != p->batch) return ROPE_ERR_SHAPE;
        // rope_qk finds a packed token's sequence by a scan of at most ROPE_MAX_BATCH entries
        if (!attention && p->cu_seqlens && p->inv_freq_rows > 1 && p->batch > ROPE_MAX_BATCH) return ROPE_ERR_LIMIT;
        if ((reinterpret_cast<uintptr_t>(p->pos) & 3u) || (reinterpret_cast<uintptr_t>(p->inv_freq) & 3u))
            return ROPE_ERR_UNSUPPORTED;
    }
    if (p->batch <= 0 || p->hq <= 0 || p->hkv <= 0 || p->head_dim <= 0) return ROPE_ERR_SHAPE;
    if (p->hq % p->hkv != 0) return ROPE_ERR_SHAPE;
    const bool varlen = p->cu_seqlens != nullptr;
    if (varlen) {
        if (p->max_seqlen <= 0 || p->ntokens <= 0) return ROPE_ERR_SHAPE;
        if (p->max_seqlen > p->ntokens) return ROPE_ERR_SHAPE;
    } else {
        if (p->seqlen <= 0) return ROPE_ERR_SHAPE;
        const int64_t rows = (int64_t)p->batch * p->seqlen;
        if (rows > INT32_MAX) return ROPE_ERR_LIMIT;
        if (p->ntokens != 0 && p->ntokens != rows) return ROPE_ERR_SHAPE;
        if (p->table_seq_rows < 0) return ROPE_ERR_SHAPE;
        if (p->table_seq_rows > 0 && p->table_seq_rows < p->seqlen) return ROPE_ERR_SHAPE;
    }
    if (attention) {
        if (p->head_dim != 64 && p->head_dim != 128) return ROPE_ERR_UNSUPPORTED;
        if (p->dtype == ROPE_DT_F32 && p->head_dim != 64) return ROPE_ERR_UNSUPPORTED;
        if (p->causal != 0 && p->causal != 1) return ROPE_ERR_SHAPE;
        if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.0f)) return ROPE_ERR_SHAPE;
        if (p->batch > 65535) return ROPE_ERR_LIMIT;
    } else {
        if (p->head_dim % 32 != 0) return ROPE_ERR_UNSUPPORTED;
        if (p->head_dim > ROPE_MAX_HEAD_SIZE) return ROPE_ERR_LIMIT;
    }
    if (p->cos && p->table_dtype != p->dtype) return ROPE_ERR_DTYPE;
    const int eb = dtype_bytes(p->dtype);
    rope_status st;
    if ((st = check_strides(p->q_stride, eb, varlen)) != ROPE_OK) return st;
    if ((st = check_strides(p->k_stride, eb, varlen)) != ROPE_OK) return st;
    if (attention) {
        if ((st = check_strides(p->v_stride, eb, varlen)) != ROPE_OK) return st;
        if ((st = check_strides(p->o_stride, eb, varlen)) != ROPE_OK) return st;
        // the fused kernel addresses each 64-key K/V tile as a base pointer plus 32-bit
        // per-lane byte offsets, so a K or V token stride must stay below 2^26 bytes
        if (p->k_stride[1] * eb >= kMaxTokenStrideBytes || p->v_stride[1] * eb >= kMaxTokenStrideBytes)
            return ROPE_ERR_LIMIT;
    }
    if (!aligned16(p->q) || !aligned16(p->k)) return ROPE_ERR_UNSUPPORTED;
    if (attention && (!aligned16(p->v) || !aligned16(p->out))) return ROPE_ERR_UNSUPPORTED;
    if (!attention && (!aligned16(p->out_q) || !aligned16(p->out_k))) return ROPE_ERR_UNSUPPORTED;
    if (p->cos && (!aligned16(p->cos) || !aligned16(p->sin))) return ROPE_ERR_UNSUPPORTED;
    if (p->lse && (reinterpret_cast<uintptr_t>(p->lse) & 3u)) return ROPE_ERR_UNSUPPORTED;
    if (varlen && (reinterpret_cast<uintptr_t>(p->cu_seqlens) & 3u)) return ROPE_ERR_UNSUPPORTED;
    return ROPE_OK;
}

rope_status check_kv_cache(const rope_kv_cache_params* p) {
    if (!p) return ROPE_ERR_NULL;
    if (p->struct_size != sizeof(rope_kv_cache_params)) return ROPE_ERR_ABI;
    for (unsigned char c : p->rsv)
        if (c) return ROPE_ERR_ABI;
    if (!valid_dtype(p->dtype)) return ROPE_ERR_DTYPE;
    if (!valid_pairing(p->pairing)) return ROPE_ERR_UNSUPPORTED;
    if (p->ntokens < 0 || p->hkv <= 0 || p->head_dim <= 0) return ROPE_ERR_SHAPE;
    // the new tokens' arrays may be NULL when there are none (empty allocations)
    if (p->ntokens > 0 && (!p->k || !p->cos || !p->sin || !p->slots)) return ROPE_ERR_NULL;
    if (!p->k_cache) return ROPE_ERR_NULL;
    if (p->ntokens > 0 && (p->v == nullptr) != (p->v_cache == nullptr)) return ROPE_ERR_NULL;
    if (p->block_size <= 0 || p->num_blocks <= 0) return ROPE_ERR_SHAPE;
    if (p->head_dim % 32 != 0) return ROPE_ERR_UNSUPPORTED;
    if (p->head_dim > ROPE_MAX_HEAD_SIZE) return ROPE_ERR_LIMIT;
    if ((int64_t)p->ntokens * p->hkv > INT32_MAX) return ROPE_ERR_LIMIT;
    if (!(std::isfinite(p->eps) && p->eps >= 0.0f)) return ROPE_ERR_SHAPE;
    const int eb = dtype_bytes(p->dtype);
    const int64_t* strides[2] = {p->k_stride, p->v_stride};
    for (int i = 0; i < 2; ++i) {
        if (i == 1 && !p->v_cache) continue;
        for (int j = 0; j < 2; ++j) {
            if (strides[i][j] < 0) return ROPE_ERR_SHAPE;
            if ((strides[i][j] * eb) % 16 != 0) return ROPE_ERR_UNSUPPORTED;
        }
    }
    const int64_t* cstrides[2] = {p->kc_stride, p->vc_stride};
    for (int i = 0; i < 2; ++i) {
        if (i == 1 && !p->v_cache) continue;
        for (int j = 0; j < 3; ++j) {
            if (cstrides[i][j] < 0) return ROPE_ERR_SHAPE;
            if ((cstrides[i][j] * eb) % 16 != 0) return ROPE_ERR_UNSUPPORTED;
        }
    }
    if (!aligned16(p->k) || !aligned16(p->cos) || !aligned16(p->sin) || !aligned16(p->k_cache))
        return ROPE_ERR_UNSUPPORTED;
    if (!aligned16(p->v) || !aligned16(p->v_cache)) return ROPE_ERR_UNSUPPORTED;
    if (p->gamma && !aligned16(p->gamma)) return ROPE_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(p->slots) & 7u) return ROPE_ERR_UNSUPPORTED;
    return ROPE_OK;
}

// Checks of rope_attn_bwd_params up to (not including) the workspace.
rope_status check_bwd_shape(const rope_attn_bwd_params* p) {
    if (!p) return ROPE_ERR_NULL;
    if (p->struct_size != sizeof(rope_attn_bwd_params)) return ROPE_ERR_ABI;
    for (unsigned char c : p->rsv)
        if (c) return ROPE_ERR_ABI;
    const rope_attn_params* f = &p->fwd;
    rope_status st = check_params(f, true);
    if (st != ROPE_OK) return st;
    if (f->dtype == ROPE_DT_F32) return ROPE_ERR_UNSUPPORTED;
    if (!f->cos && f->pos) return ROPE_ERR_UNSUPPORTED;   // tables formed in the kernel: forward only
    if (!f->lse) return ROPE_ERR_NULL;
    if (!p->dout || !p->dq || !p->dk || !p->dv) return ROPE_ERR_NULL;
    const bool varlen = f->cu_seqlens != nullptr;
    const int eb = dtype_bytes(f->dtype);
    if ((st = check_strides(p->do_stride, eb, varlen)) != ROPE_OK) return st;
    if ((st = check_strides(p->dq_stride, eb, varlen)) != ROPE_OK) return st;
    if ((st = check_strides(p->dk_stride, eb, varlen)) != ROPE_OK) return st;
    if ((st = check_strides(p->dv_stride, eb, varlen)) != ROPE_OK) return st;
    if (!aligned16(p->dout) || !aligned16(p->dq) || !aligned16(p->dk) || !aligned16(p->dv))
        return ROPE_ERR_UNSUPPORTED;
    if (f->hq > 65535) return ROPE_ERR_LIMIT;   // grid dimension of the dq kernel
    return ROPE_OK;
}

// Shape checks of rope_decode_params that the workspace size depends on.
rope_status check_decode_shape(const rope_decode_params* p) {
    if (!p) return ROPE_ERR_NULL;
    if (p->struct_size != sizeof(rope_decode_params)) return ROPE_ERR_ABI;
    for (unsigned char c : p->rsv)
        if (c) return ROPE_ERR_ABI;
    if (p->batch <= 0 || p->hq <= 0 || p->hkv <= 0 || p->head_dim <= 0) return ROPE_ERR_SHAPE;
    if (p->hq % p->hkv != 0) return ROPE_ERR_SHAPE;
    if (p->block_size <= 0 || p->max_blocks_per_seq <= 0 || p->num_blocks <= 0) return ROPE_ERR_SHAPE;
    if (p->max_seqlen <= 0 || (int64_t)p->max_seqlen > (int64_t)p->max_blocks_per_seq * p->block_size)
        return ROPE_ERR_SHAPE;
    if (p->num_splits < 0) return ROPE_ERR_SHAPE;
    if (p->num_splits > 256 || p->batch > 65535) return ROPE_ERR_LIMIT;
    const int g = p->hq / p->hkv;
    if ((int64_t)p->hkv * ((g + 31) / 32) > 65535) return ROPE_ERR_LIMIT;
    if ((int64_t)p->batch * p->max_blocks_per_seq > INT32_MAX) return ROPE_ERR_LIMIT;
    if (p->head_dim != 64 && p->head_dim != 128) return ROPE_ERR_UNSUPPORTED;
    return ROPE_OK;
}

rope_status check_decode(const rope_decode_params* p, bool with_workspace = true) {
    rope_status st = check_decode_shape(p);
    if (st != ROPE_OK) return st;
    if (!valid_dtype(p->dtype)) return ROPE_ERR_DTYPE;
    if (p->dtype == ROPE_DT_F32) return ROPE_ERR_UNSUPPORTED;
    if (!valid_pairing(p->pairing)) return ROPE_ERR_UNSUPPORTED;
    if (!p->q || !p->k_cache || !p->v_cache || !p->cache_seqlens || !p->out) return ROPE_ERR_NULL;
    if ((p->cos == nullptr) != (p->sin == nullptr)) return ROPE_ERR_NULL;
    if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.0f)) return ROPE_ERR_SHAPE;
    const int eb = dtype_bytes(p->dtype);
    const int64_t* s2[2] = {p->q_stride, p->o_stride};
    for (const int64_t* s : s2)
        for (int j = 0; j < 2; ++j) {
            if (s[j] < 0) return ROPE_ERR_SHAPE;
            if ((s[j] * eb) % 16 != 0) return ROPE_ERR_UNSUPPORTED;
        }
    const int64_t* s3[2] = {p->kc_stride, p->vc_stride};
    for (const int64_t* s : s3)
        for (int j = 0; j < 3; ++j) {
            if (s[j] < 0) return ROPE_ERR_SHAPE;
            if ((s[j] * eb) % 16 != 0) return ROPE_ERR_UNSUPPORTED;
        }
    if (!aligned16(p->q) || !aligned16(p->out) || !aligned16(p->k_cache) || !aligned16(p->v_cache))
        return ROPE_ERR_UNSUPPORTED;
    if (!aligned16(p->cos) || !aligned16(p->sin)) return ROPE_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(p->block_table) & 3u) || (reinterpret_cast<uintptr_t>(p->cache_seqlens) & 3u) ||
        (reinterpret_cast<uintptr_t>(p->lse) & 3u))
        return ROPE_ERR_UNSUPPORTED;
    if (!with_workspace) return ROPE_OK;
    const uint64_t need = ropefa::decode_workspace_bytes(p, ropefa::decode_num_splits(p));
    if (!p->workspace || (reinterpret_cast<uintptr_t>(p->workspace) & 255u) || p->workspace_bytes < need)
        return ROPE_ERR_WORKSPACE;
    return ROPE_OK;
}

}  // namespace

extern "C" {

const char* rope_status_str(rope_status s) {
    switch (s) {
        case ROPE_OK: return "ROPE_OK";
        case ROPE_ERR_NULL: return "ROPE_ERR_NULL";
        case ROPE_ERR_SHAPE: return "ROPE_ERR_SHAPE";
        case ROPE_ERR_DTYPE: return "ROPE_ERR_DTYPE";
        case ROPE_ERR_LIMIT: return "ROPE_ERR_LIMIT";
        case ROPE_ERR_UNSUPPORTED: return "ROPE_ERR_UNSUPPORTED";
        case ROPE_ERR_ABI: return "ROPE_ERR_ABI";
        case ROPE_ERR_HIP: return "ROPE_ERR_HIP";
        case ROPE_ERR_WORKSPACE: return "ROPE_ERR_WORKSPACE";
    }
    return "ROPE_ERR_UNKNOWN";
}

int32_t rope_abi_version(void) { return ROPE_FA_ABI_VERSION; }

uint32_t rope_attn_params_size(void) { return (uint32_t)sizeof(rope_attn_params); }

uint32_t rope_kv_cache_params_size(void) { return (uint32_t)sizeof(rope_kv_cache_params); }

uint32_t rope_decode_params_size(void) { return (uint32_t)sizeof(rope_decode_params); }

uint32_t rope_attn_bwd_params_size(void) { return (uint32_t)sizeof(rope_attn_bwd_params); }

uint64_t rope_flash_attn_bwd_workspace_size(const rope_attn_bwd_params* p) {
    if (check_bwd_shape(p) != ROPE_OK) return 0;
    return ropefa::flash_bwd_workspace_bytes(&p->fwd);
}

uint64_t rope_decode_workspace_size(const rope_decode_params* p) {
    if (check_decode_shape(p) != ROPE_OK) return 0;
    return ropefa::decode_workspace_bytes(p, ropefa::decode_num_splits(p));
}

rope_status rope_inv_freq(double base, int32_t head_size, const int32_t* seq_lens, int32_t batch, int32_t trained_len,
                          float* out) {
    if (!out) return ROPE_ERR_NULL;
    if (trained_len > 0 && !seq_lens) return ROPE_ERR_NULL;
    if (!(std::isfinite(base) && base > 0.0)) return ROPE_ERR_SHAPE;
    if (head_size <= 0 || head_size % 2 != 0 || batch <= 0) return ROPE_ERR_SHAPE;
    if (head_size > ROPE_MAX_HEAD_SIZE || batch > ROPE_MAX_BATCH) return ROPE_ERR_LIMIT;
    if (seq_lens)
        for (int b = 0; b < batch; ++b)
            if (seq_lens[b] <= 0) return ROPE_ERR_SHAPE;
    const int half = head_size / 2;
    for (int b = 0; b < batch; ++b) {
        double base_b = base;
        if (trained_len > 0 && seq_lens[b] > trained_len)
            base_b = base * std::pow((double)seq_lens[b] / (double)trained_len,
                                     (double)head_size / (double)(head_size - 2));
        for (int i = 0; i < half; ++i)
            out[(int64_t)b * half + i] = (float)(1.0 / std::pow(base_b, (double)(2 * i) / (double)head_size));
    }
    return ROPE_OK;
}

rope_status rope_tables_ex(const int32_t* pos, const float* inv_freq, const int32_t* seq_lens, int32_t batch,
                           int32_t ntokens, int32_t head_size, float pos_scale, rope_dtype out_dtype,
                           rope_pairing pairing, rope_angle_mode angle_mode, void* sin_out, void* cos_out,
                           void* hip_stream) {
    if (!pos || !inv_freq || !seq_lens || !sin_out || !cos_out) return ROPE_ERR_NULL;
    if (batch <= 0 || ntokens <= 0 || head_size <= 0) return ROPE_ERR_SHAPE;
    if (batch > ROPE_MAX_BATCH || ntokens > ROPE_MAX_NTOKENS) return ROPE_ERR_LIMIT;
    if (head_size > ROPE_MAX_HEAD_SIZE || head_size % 32 != 0) return ROPE_ERR_LIMIT;
    int64_t total = 0;
    for (int b = 0; b < batch; ++b) {
        if (seq_lens[b] <= 0) return ROPE_ERR_SHAPE;
        total += seq_lens[b];
    }
    if (total != ntokens) return ROPE_ERR_SHAPE;
    if (!(std::isfinite(pos_scale) && pos_scale > 0.0f)) return ROPE_ERR_SHAPE;
    if (!valid_dtype(out_dtype)) return ROPE_ERR_DTYPE;
    if (!valid_pairing(pairing)) return ROPE_ERR_UNSUPPORTED;
    if (angle_mode != ROPE_ANGLE_F32 && angle_mode != ROPE_ANGLE_EXACT) return ROPE_ERR_UNSUPPORTED;
    if (!aligned16(inv_freq) || !aligned16(sin_out) || !aligned16(cos_out)) return ROPE_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(pos) & 3u) return ROPE_ERR_UNSUPPORTED;
    const hipError_t e = ropefa::launch_rope_tables(pos, inv_freq, seq_lens, batch, ntokens, head_size, pos_scale,
                                                    out_dtype, (int)pairing, (int)angle_mode, sin_out, cos_out,
                                                    (hipStream_t)hip_stream);
    return e == hipSuccess ? ROPE_OK : ROPE_ERR_HIP;
}

rope_status rope_tables(const int32_t* pos, const float* inv_freq, const int32_t* seq_lens, int32_t batch,
                        int32_t ntokens, int32_t head_size, float pos_scale, rope_dtype out_dtype, void* sin_out,
                        void* cos_out, void* hip_stream) {
    return rope_tables_ex(pos, inv_freq, seq_lens, batch, ntokens, head_size, pos_scale, out_dtype, ROPE_PAIR_HALF,
                          ROPE_ANGLE_F32, sin_out, cos_out, hip_stream);
}

rope_status rope_qk(const rope_attn_params* p, void* hip_stream) {
    const rope_status st = check_params(p, false);
    if (st != ROPE_OK) return st;
    const hipError_t e = ropefa::launch_rope_qk(p, (hipStream_t)hip_stream);
    return e == hipSuccess ? ROPE_OK : ROPE_ERR_HIP;
}

rope_status rope_flash_attn_fwd(const rope_attn_params* p, void* hip_stream) {
    const rope_status st = check_params(p, true);
    if (st != ROPE_OK) return st;
    const hipError_t e = ropefa::launch_flash_fwd(p, nullptr, (hipStream_t)hip_stream);
    return e == hipSuccess ? ROPE_OK : ROPE_ERR_HIP;
}

uint64_t rope_flash_attn_fwd_workspace_size(const rope_attn_params* p) {
    if (check_params(p, true) != ROPE_OK) return 0;
    return ropefa::flash_fwd_workspace_bytes(p);
}

rope_status rope_flash_attn_fwd_ws(const rope_attn_params* p, void* workspace, uint64_t workspace_bytes,
                                   void* hip_stream) {
    const rope_status st = check_params(p, true);
    if (st != ROPE_OK) return st;
    const uint64_t need = ropefa::flash_fwd_workspace_bytes(p);
    hipError_t e;
    if (need == 0) {
        e = ropefa::launch_flash_fwd(p, nullptr, (hipStream_t)hip_stream);
    } else {
        if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < need)
            return ROPE_ERR_WORKSPACE;
        e = ropefa::launch_rope_k_prepass(p, workspace, (hipStream_t)hip_stream);
        if (e == hipSuccess) e = ropefa::launch_flash_fwd(p, workspace, (hipStream_t)hip_stream);
    }
    return e == hipSuccess ? ROPE_OK : ROPE_ERR_HIP;
}

rope_status rope_kv_rms_norm_rope_cache(const rope_kv_cache_params* p, void* hip_stream) {
    const rope_status st = check_kv_cache(p);
    if (st != ROPE_OK) return st;
    if (p->ntokens == 0) return ROPE_OK;
    const hipError_t e = ropefa::launch_kv_cache(p, (hipStream_t)hip_stream);
    return e == hipSuccess ? ROPE_OK : ROPE_ERR_HIP;
}

rope_status rope_decode_attn_fwd(const rope_decode_params* p, void* hip_stream) {
    const rope_status st = check_decode(p);
    if (st != ROPE_OK) return st;
    const hipError_t e = ropefa::launch_decode(p, (hipStream_t)hip_stream);
    return e == hipSuccess ? ROPE_OK : ROPE_ERR_HIP;
}

rope_status rope_decode_attn_fwd_noalloc(const rope_decode_params* p, void* hip_stream) {
    const rope_status st = check_decode(p, false);
    if (st != ROPE_OK) return st;
    if (ropefa::decode_workspace_bytes(p, ropefa::decode_num_splits(p)) > ROPE_DECODE_NOALLOC_MAX_BYTES)
        return ROPE_ERR_LIMIT;
    void* ws = nullptr;
    hipError_t e = ropefa::decode_scratch((hipStream_t)hip_stream, &ws);
    if (e != hipSuccess) return ROPE_ERR_HIP;
    rope_decode_params q = *p;
    q.workspace = ws;
    q.workspace_bytes = ROPE_DECODE_NOALLOC_MAX_BYTES;
    e = ropefa::launch_decode(&q, (hipStream_t)hip_stream);
    return e == hipSuccess ? ROPE_OK : ROPE_ERR_HIP;
}

rope_status rope_flash_attn_bwd(const rope_attn_bwd_params* p, void* hip_stream) {
    const rope_status st = check_bwd_shape(p);
    if (st != ROPE_OK) return st;
    const uint64_t need = ropefa::flash_bwd_workspace_bytes(&p->fwd);
    if (!p->workspace || (reinterpret_cast<uintptr_t>(p->workspace) & 255u) || p->workspace_bytes < need)
        return ROPE_ERR_WORKSPACE;
    const hipError_t e = ropefa::launch_flash_bwd(p, (hipStream_t)hip_stream);
    return e == hipSuccess ? ROPE_OK : ROPE_ERR_HIP;
}

}  // extern "C"

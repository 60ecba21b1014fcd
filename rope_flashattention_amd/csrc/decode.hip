// rope_decode_attn_fwd: one decode step of RoPE + GQA attention over a paged KV cache, gfx950.
//
// What is computed: each sequence's new query, rotated with its table row (the rope_qk
// formula), attends to every key in the sequence's cache ([FlashAttention blog]:
// Softmax(QK^T/sqrt(d))V; the keys were rotated when they were written).  The g = hq/hkv
// query heads that share a kv head ([RoPE/GQA tutorial], sections 十一-十二) are served by
// one pass over that head's cache, so the cache is read once per kv head, which is the
// traffic GQA exists to save.  A decode step does a few flops per cached byte, so the
// kernels are bound by HBM bandwidth.
//
// Partial kernel (decode_partial_kernel): one wavefront per (sequence, kv head, group of
// up to 32 q heads, key split).  Per 32-key tile:
//   * S^T = K Q'^T with the 32x32x16 MFMA: the A operand is read straight from the cache,
//     lane l loading 16 bytes of key pi(l % 32) (the permuted row order below), the B
//     operand is the rotated, scaled Q' of the group's heads (head = MFMA column), held in
//     registers for the whole pass; unused columns are zero.
//   * Permuted rows: MFMA row m holds key pi(m) = 16*((m>>2)&1) + 4*(m>>3) + (m&3), which
//     makes lane half h hold the scores of the contiguous keys 16h .. 16h+15 of its head, so
//     the probabilities are already the B operand of the next product.
//   * Online softmax per head in the log2 domain (scale * log2(e) folded into Q').
//   * O^T += V^T P^T with the same MFMA; V rows go through a wave-private LDS tile and the
//     transposing LDS read (ds_read_b64_tr_b16) supplies the V^T operand.
// The wave writes its unnormalised O, running max m and sum l for its key range to the
// workspace.  Combine kernel (decode_combine_kernel): one workgroup per (sequence, q head)
// merges the splits: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
#include "common.h"

namespace ropefa {

struct DecodeArgs {
    const void* q;
    const void* cos;
    const void* sin;
    const void* kc;
    const void* vc;
    const int32_t* block_table;
    const int32_t* seqlens;
    float* ws_o;   // [batch, hq, nsplit, D]
    float* ws_m;   // [batch, hq, nsplit]
    float* ws_l;   // [batch, hq, nsplit]
    void* out;
    float* lse;
    int64_t qs[2], os[2];
    int64_t kcs[3], vcs[3];
    int32_t batch, hq, hkv, g, ngroups, nsplit;
    int32_t block_size, max_blocks, num_blocks, max_seqlen;
    float scale_log2;
    int32_t rotate;
};

template <typename T> struct DMma;
template <> struct DMma<__bf16> {
    __device__ static __forceinline__ f32x16 run(const u32x4& a, const u32x4& b, const f32x16& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};
template <> struct DMma<_Float16> {
    __device__ static __forceinline__ f32x16 run(const u32x4& a, const u32x4& b, const f32x16& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      c, 0, 0, 0);
    }
};

// x combined with its value in the lane 32 apart (the other half of the wavefront); the
// swap returns the lane's own value and its partner's, in an order that depends on the half
__device__ __forceinline__ float dec_halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float dec_halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ i16x4 lds_tr16(const void* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// orders this wave's LDS writes before its later LDS reads (and reads before rewrites)
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// element offset (without the head term) of logical token `key` of sequence b
__device__ __forceinline__ int64_t slot_offset(const DecodeArgs& a, int b, int key, const int64_t (&cs)[3]) {
    const int lb = key / a.block_size;
    const int off = key - lb * a.block_size;
    int pb = a.block_table ? a.block_table[(int64_t)b * a.max_blocks + lb] : b * a.max_blocks + lb;
    pb = min(max(pb, 0), a.num_blocks - 1);
    return (int64_t)pb * cs[0] + (int64_t)off * cs[1];
}

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeArgs a) {
    constexpr int NS = D / 16;   // MFMA k-steps over the head dimension
    constexpr int VP = D + 32;   // padded LDS row of the V tile (elements)
    constexpr float kNegInf = -__builtin_inff();
    __shared__ __attribute__((aligned(16))) T sV[32 * VP];

    const int l = threadIdx.x;
    const int n = l & 31;          // MFMA column: head of the group
    const int hh = l >> 5;         // lane half
    const int split = blockIdx.x;
    const int kvh = blockIdx.y / a.ngroups;
    const int grp = blockIdx.y - kvh * a.ngroups;
    const int b = blockIdx.z;
    const int hin = grp * 32 + n;
    const bool hvalid = hin < a.g;
    const int h = kvh * a.g + (hvalid ? hin : 0);

    int L = min(a.seqlens[b], a.max_seqlen);
    L = max(L, 0);
    int chunk = (L + a.nsplit - 1) / a.nsplit;
    chunk = (chunk + 31) & ~31;
    const int k_begin = min(split * chunk, L);
    const int k_end = min(L, k_begin + chunk);

    // ---- Q'^T operand: rotate-half RoPE in float32, scaled by softmax_scale*log2(e), rounded once
    u32x4 qb[NS];
    {
        const T* qrow = reinterpret_cast<const T*>(a.q) + (int64_t)b * a.qs[0] + (int64_t)h * a.qs[1];
#pragma unroll
        for (int s = 0; s < NS / 2; ++s) {
            const int d = 16 * s + 8 * hh;
            float x[8], y[8];
            unpack<T>(load_chunk<T>(qrow + d), x);
            unpack<T>(load_chunk<T>(qrow + d + D / 2), y);
            if (a.rotate) {
                const T* crow = reinterpret_cast<const T*>(a.cos) + (int64_t)b * D;
                const T* srow = reinterpret_cast<const T*>(a.sin) + (int64_t)b * D;
                float c0[8], s0[8], c1[8], s1[8];
                unpack<T>(load_chunk<T>(crow + d), c0);
                unpack<T>(load_chunk<T>(srow + d), s0);
                unpack<T>(load_chunk<T>(crow + d + D / 2), c1);
                unpack<T>(load_chunk<T>(srow + d + D / 2), s1);
                rotate_pair(x, y, c0, s0, c1, s1);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[e] = hvalid ? x[e] * a.scale_log2 : 0.0f;
                y[e] = hvalid ? y[e] * a.scale_log2 : 0.0f;
            }
            qb[s] = pack<T>(x).w;
            qb[s + NS / 2] = pack<T>(y).w;
        }
    }

    const T* kbase = reinterpret_cast<const T*>(a.kc) + (int64_t)kvh * a.kcs[2];
    const T* vbase = reinterpret_cast<const T*>(a.vc) + (int64_t)kvh * a.vcs[2];
    const int prow = 16 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);   // key of MFMA row n
    const int tr_row = (l & 15) >> 2;
    const int tr_col = ((l >> 4) & 1) * 16 + 4 * (l & 3);

    f32x16 oacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[mb][i] = 0.0f;
    float m_run = kNegInf;
    float l_half = 0.0f;

    for (int k0 = k_begin; k0 < k_end; k0 += 32) {
        // ---- loads: K row pi(n) as the A operand, V row n into registers (ragged tail clamped)
        const T* krow = kbase + slot_offset(a, b, min(k0 + prow, k_end - 1), a.kcs);
        const T* vrow = vbase + slot_offset(a, b, min(k0 + n, k_end - 1), a.vcs);
        u32x4 ka[NS], va[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) ka[s] = load_chunk<T>(krow + 16 * s + 8 * hh).w;
#pragma unroll
        for (int s = 0; s < NS; ++s) va[s] = load_chunk<T>(vrow + 16 * s + 8 * hh).w;

        // ---- S^T = K Q'^T
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s) sacc = DMma<T>::run(ka[s], qb[s], sacc);

        // ---- online softmax: lane half hh holds keys k0 + 16*hh + i
        const int valid = k_end - (k0 + 16 * hh);
        float mt = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i >= valid) sacc[i] = kNegInf;
            mt = fmaxf(mt, sacc[i]);
        }
        mt = dec_halves_max(mt);
        const float m_new = fmaxf(m_run, mt);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        u32x4 pk[2];
        float lt = 0.0f;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = exp2f(sacc[8 * s + j] - m_new);
            pk[s] = pack<T>(p).w;
            float pr[8];
            unpack<T>(Chunk8<T>{pk[s]}, pr);   // the rounded values the product uses
#pragma unroll
            for (int j = 0; j < 8; ++j) lt += pr[j];
        }
        l_half = l_half * alpha + lt;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) oacc[mb] *= alpha;

        // ---- V tile through LDS, O^T += V^T P^T
#pragma unroll
        for (int s = 0; s < NS; ++s) *reinterpret_cast<u32x4*>(&sV[n * VP + 16 * s + 8 * hh]) = va[s];
        wave_lds_sync();
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const T* vp = &sV[(16 * hh + 8 * s + tr_row) * VP + mb * 32 + tr_col];
                const i16x4 lo = lds_tr16(vp);
                const i16x4 hi = lds_tr16(vp + 4 * VP);
                const u32x4 av = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[mb] = DMma<T>::run(av, pk[s], oacc[mb]);
            }
        wave_lds_sync();
    }

    // ---- partial results: O^T row d = mb*32 + 8*(i/4) + 4*hh + i%4, column = head
    const float l_tot = dec_halves_sum(l_half);
    if (hvalid) {
        const int64_t pi = ((int64_t)b * a.hq + h) * a.nsplit + split;
        float* wo = a.ws_o + pi * D;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 v4 = {oacc[mb][4 * q4], oacc[mb][4 * q4 + 1], oacc[mb][4 * q4 + 2], oacc[mb][4 * q4 + 3]};
                *reinterpret_cast<f32x4*>(wo + mb * 32 + 8 * q4 + 4 * hh) = v4;
            }
        if (hh == 0) {
            a.ws_m[pi] = m_run;
            a.ws_l[pi] = l_tot;
        }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
    const int bh = blockIdx.x;
    const int b = bh / a.hq;
    const int h = bh - b * a.hq;
    const int d = threadIdx.x;
    const int64_t p0 = (int64_t)bh * a.nsplit;
    float M = -__builtin_inff();
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.ws_m[p0 + s]);
    float o = 0.0f, lsum = 0.0f;
    if (M != -__builtin_inff()) {
        for (int s = 0; s < a.nsplit; ++s) {
            const float w = exp2f(a.ws_m[p0 + s] - M);   // empty splits: m = -inf, w = 0
            lsum += w * a.ws_l[p0 + s];
            o += w * a.ws_o[(p0 + s) * D + d];
        }
        o = o / lsum;
    }
    T* orow = reinterpret_cast<T*>(a.out) + (int64_t)b * a.os[0] + (int64_t)h * a.os[1];
    orow[d] = (T)o;
    if (a.lse && d == 0)
        a.lse[bh] = M == -__builtin_inff() ? -__builtin_inff() : (M + log2f(lsum)) * 0.69314718055994531f;
}

int decode_num_splits(const rope_decode_params* p) {
    if (p->num_splits > 0) return p->num_splits;
    const int g = p->hq / p->hkv;
    const int64_t units = (int64_t)p->batch * p->hkv * ((g + 31) / 32);
    int64_t ns = (2048 + units - 1) / units;                     // about 8 waves per CU
    const int64_t by_len = ((int64_t)p->max_seqlen + 127) / 128;  // at least 128 keys per split
    ns = ns < by_len ? ns : by_len;
    ns = ns < 256 ? ns : 256;
    return (int)(ns < 1 ? 1 : ns);
}

uint64_t decode_workspace_bytes(const rope_decode_params* p, int nsplit) {
    const uint64_t parts = (uint64_t)p->batch * p->hq * nsplit;
    return parts * (uint64_t)(p->head_dim + 2) * 4u;
}

template <typename T, int D>
static void launch_typed(const DecodeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_partial_kernel<T, D>), dim3(a.nsplit, a.hkv * a.ngroups, a.batch), dim3(64), 0, stream,
                       a);
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.batch * a.hq), dim3(D), 0, stream, a);
}

hipError_t launch_decode(const rope_decode_params* p, hipStream_t stream) {
    DecodeArgs a;
    const int nsplit = decode_num_splits(p);
    a.q = p->q;
    a.cos = p->cos;
    a.sin = p->sin;
    a.rotate = p->cos != nullptr;
    a.kc = p->k_cache;
    a.vc = p->v_cache;
    a.block_table = p->block_table;
    a.seqlens = p->cache_seqlens;
    const uint64_t parts = (uint64_t)p->batch * p->hq * nsplit;
    a.ws_o = reinterpret_cast<float*>(p->workspace);
    a.ws_m = a.ws_o + parts * p->head_dim;
    a.ws_l = a.ws_m + parts;
    a.out = p->out;
    a.lse = p->lse;
    for (int i = 0; i < 2; ++i) {
        a.qs[i] = p->q_stride[i];
        a.os[i] = p->o_stride[i];
    }
    for (int i = 0; i < 3; ++i) {
        a.kcs[i] = p->kc_stride[i];
        a.vcs[i] = p->vc_stride[i];
    }
    a.batch = p->batch;
    a.hq = p->hq;
    a.hkv = p->hkv;
    a.g = p->hq / p->hkv;
    a.ngroups = (a.g + 31) / 32;
    a.nsplit = nsplit;
    a.block_size = p->block_size;
    a.max_blocks = p->max_blocks_per_seq;
    a.num_blocks = p->num_blocks;
    a.max_seqlen = p->max_seqlen;
    a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
    const int key = (p->dtype == ROPE_DT_BF16 ? 0 : 2) + (p->head_dim == 128 ? 1 : 0);
    switch (key) {
        case 0: launch_typed<__bf16, 64>(a, stream); break;
        case 1: launch_typed<__bf16, 128>(a, stream); break;
        case 2: launch_typed<_Float16, 64>(a, stream); break;
        case 3: launch_typed<_Float16, 128>(a, stream); break;
    }
    return hipGetLastError();
}

}  // namespace ropefa

// rope_flash_attn_fwd: RoPE fused into a FlashAttention forward pass on gfx950.
//
// Launch side of the fused kernels (the kernels themselves are in flash_fwd.h); the float32
// kernel is instantiated here, the 16-bit ones in flash_fwd_bf16.hip and flash_fwd_f16.hip.
#include "flash_fwd.h"

namespace ropefa {

// ============================================================================ launch
static void launch32(const FaArgs& a, int rot, dim3 grid, hipStream_t stream) {
    switch (rot) {
        case kRotNone: hipLaunchKernelGGL((flash_fwd32_kernel<64, kRotNone>), grid, dim3(256), 0, stream, a); break;
        case kRotHalfTable: hipLaunchKernelGGL((flash_fwd32_kernel<64, kRotHalfTable>), grid, dim3(256), 0, stream, a); break;
        case kRotInterTable: hipLaunchKernelGGL((flash_fwd32_kernel<64, kRotInterTable>), grid, dim3(256), 0, stream, a); break;
        case kRotHalfGen: hipLaunchKernelGGL((flash_fwd32_kernel<64, kRotHalfGen>), grid, dim3(256), 0, stream, a); break;
        case kRotInterGen: hipLaunchKernelGGL((flash_fwd32_kernel<64, kRotInterGen>), grid, dim3(256), 0, stream, a); break;
    }
}

// Heads packed per workgroup: as many q heads of one kv head as divide the group (<= 8).
int flash_heads_per_wg(int group, rope_dtype dt) {
    if (dt == ROPE_DT_F32) return 1;
    for (int hp = 8; hp > 1; hp >>= 1)
        if (group % hp == 0) return hp;
    return 1;
}

// Rotate K once per key in a pre-pass (into a workspace) instead of in every workgroup that
// stages it.  In-loop, a key is rotated once per (query tile, head group) of its kv head
// that reaches it: on average (group / HP) * (n_qt + 1) / 2 times for causal attention over
// n_qt query tiles (n_qt times without the mask).  The pre-pass reads and writes each k row
// once (4 * head_dim bytes for 16-bit data) plus a launch.  Measured on MI355X (bf16/fp16,
// head_dim 128, per k row and kv head): in-loop rotation costs 12-23 ps per repetition, the
// pre-pass 120-170 ps plus about 5 us per call, so the pre-pass pays from about 8
// repetitions on (a causal S2048 MHA call, 4.5 repetitions, is 9% faster in-loop; causal
// S4096 with 4 q heads per kv head, 32.5 repetitions, 5% faster with the pre-pass).
// Varlen calls whose formed tables use per-sequence inverse frequencies stay in-loop (the
// pre-pass finds a token's sequence by a bounded scan of cu_seqlens).
constexpr double kPrerotMinReps = 8.0;

bool flash_fwd_prerotate_k(const rope_attn_params* p) {
    const bool gen = p->cos == nullptr && p->pos != nullptr;
    if (p->cos == nullptr && !gen) return false;  // no rotation
    if (p->dtype == ROPE_DT_F32) return false;
    if (gen && p->cu_seqlens && p->inv_freq_rows > 1) return false;
    if ((int64_t)p->hkv * p->head_dim * 2 >= ((int64_t)1 << 26)) return false;  // k' token stride limit
    const int group = p->hq / p->hkv;
    const int hp = flash_heads_per_wg(group, p->dtype);
    const int qt = (8 / hp) * 32;
    const int maxlen = p->cu_seqlens ? p->max_seqlen : p->seqlen;
    const double n_qt = (double)((maxlen + qt - 1) / qt);
    const double reps = (double)(group / hp) * (p->causal ? 0.5 * (n_qt + 1.0) : n_qt);
    return reps >= kPrerotMinReps;
}

// k' of the pre-pass: rows x hkv x head_dim values of the dtype, 256-byte multiple.
uint64_t flash_fwd_workspace_bytes(const rope_attn_params* p) {
    if (!flash_fwd_prerotate_k(p)) return 0;
    const uint64_t rows = p->cu_seqlens ? (uint64_t)p->ntokens : (uint64_t)p->batch * (uint64_t)p->seqlen;
    const uint64_t bytes = rows * (uint64_t)p->hkv * (uint64_t)p->head_dim * (uint64_t)dtype_bytes(p->dtype);
    return (bytes + 255u) & ~(uint64_t)255u;
}

hipError_t launch_flash_fwd(const rope_attn_params* p, const void* kprime, hipStream_t stream) {
    FaArgs a;
    a.q = p->q;
    a.k = p->k;
    a.v = p->v;
    a.o = p->out;
    a.lse = p->lse;
    a.cos = p->cos;
    a.sin = p->sin;
    a.cu_seqlens = p->cu_seqlens;
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = p->q_stride[i];
        a.ks[i] = p->k_stride[i];
        a.vs[i] = p->v_stride[i];
        a.os[i] = p->o_stride[i];
    }
    const bool varlen = p->cu_seqlens != nullptr;
    a.seqlen = varlen ? 0 : p->seqlen;
    a.ntokens = varlen ? p->ntokens : p->batch * p->seqlen;
    a.max_seqlen = varlen ? p->max_seqlen : p->seqlen;
    a.group = p->hq / p->hkv;
    a.table_seq_rows = p->table_seq_rows;
    a.lse_stride = varlen ? p->ntokens : p->batch * p->seqlen;
    a.causal = p->causal;
    a.scale_log2 = p->softmax_scale * 1.44269504088896340736f;
    a.pos = p->pos;
    a.inv_freq = p->inv_freq;
    a.pos_scale = p->pos_scale;
    a.inv_freq_rows = p->inv_freq_rows;
    const bool inter = p->pairing == ROPE_PAIR_INTERLEAVED;
    int rot = p->cos ? (inter ? kRotInterTable : kRotHalfTable)
                     : (p->pos ? (inter ? kRotInterGen : kRotHalfGen) : kRotNone);
    if (kprime) {
        // k' written by the pre-pass (launch_rope_k_prepass): dense [batch, hkv, seqlen, D],
        // varlen [hkv, ntokens, D]
        if (rot == kRotNone || p->dtype == ROPE_DT_F32) return hipErrorInvalidValue;
        const int64_t D = p->head_dim;
        const int64_t plane = (varlen ? (int64_t)p->ntokens : (int64_t)p->seqlen) * D;
        a.k = kprime;
        a.ks[0] = varlen ? 0 : (int64_t)p->hkv * plane;
        a.ks[1] = D;
        a.ks[2] = plane;
        rot += kRotQHalfTable - kRotHalfTable;
    }
    const int maxlen = varlen ? p->max_seqlen : p->seqlen;
    if (p->dtype == ROPE_DT_F32) {
        const int qt = 4 * 32;
        const dim3 grid((unsigned)p->hq, (unsigned)((maxlen + qt - 1) / qt), (unsigned)p->batch);
        launch32(a, rot, grid, stream);
        return hipGetLastError();
    }
    const int hp = flash_heads_per_wg(a.group, p->dtype);
    const int qt = (8 / hp) * 32;
    const dim3 grid((unsigned)(p->hq / hp), (unsigned)((maxlen + qt - 1) / qt), (unsigned)p->batch);
    switch (p->dtype) {
        case ROPE_DT_BF16: launch_flash16_bf16(a, hp, p->head_dim, rot, grid, stream); break;
        case ROPE_DT_F16: launch_flash16_f16(a, hp, p->head_dim, rot, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ropefa

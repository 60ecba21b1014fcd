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

hipError_t launch_flash_fwd(const rope_attn_params* p, hipStream_t stream) {
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
    const int rot = p->cos ? (inter ? kRotInterTable : kRotHalfTable)
                           : (p->pos ? (inter ? kRotInterGen : kRotHalfGen) : kRotNone);
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

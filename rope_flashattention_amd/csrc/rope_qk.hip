// rope_qk: standalone rotate-half RoPE of Q and K on gfx950 (the unfused step).
//
// The Rope op of the [DynamicNTKOperation] page (section 算子上下文) takes q, k and the
// sin/cos tables and returns rotated q and k; written per element,
//   x'[j] = x[j] * cos[j] + rotate_half(x)[j] * sin[j],  rotate_half(x) = cat(-x[D/2:], x[:D/2]).
// This is the "RoPE writes to HBM, attention reads it back" step that the [RoPE-fusion
// blog] (section 二) measures as pure data movement, so the kernel is HBM bound:
// it reads q and k, writes q' and k', and reads each table row once per block of heads.
//
// Thread mapping: one thread owns one token and one 8-column chunk j of the first half
// together with its partner chunk j + D/2 (both halves of the rotation live in the same
// thread, no shuffles).  It loads the four table chunks once and then walks a group of
// heads (q heads first, then k heads), so table traffic is amortised over the group.
#include "common.h"

namespace ropefa {

struct QkArgs {
    const void* q;
    const void* k;
    void* oq;
    void* ok;
    const void* cos;
    const void* sin;
    int64_t qs[3];  // {batch, token, head} strides in elements (q and out_q)
    int64_t ks[3];  // (k and out_k)
    int32_t varlen;
    int32_t seqlen;         // dense: tokens per sequence
    int32_t rows;           // token rows processed: dense batch*seqlen, varlen ntokens
    int32_t hq, hkv;
    int32_t head_dim;
    int32_t table_seq_rows; // dense: 0 = shared table
    int32_t heads_per_block;
};

template <typename T>
__global__ __launch_bounds__(256) void rope_qk_kernel(QkArgs a) {
    const int D = a.head_dim;
    const int half = D >> 1;
    const int chunks = half >> 3;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)a.rows * chunks) return;
    const int t = (int)(gid / chunks);
    const int j = (int)(gid - (int64_t)t * chunks) * 8;

    // token -> (sequence, position) offsets and table row
    int64_t qoff, koff, trow;
    if (a.varlen) {
        qoff = (int64_t)t * a.qs[1];
        koff = (int64_t)t * a.ks[1];
        trow = t;
    } else {
        const int b = t / a.seqlen;
        const int s = t - b * a.seqlen;
        qoff = (int64_t)b * a.qs[0] + (int64_t)s * a.qs[1];
        koff = (int64_t)b * a.ks[0] + (int64_t)s * a.ks[1];
        trow = (a.table_seq_rows ? (int64_t)b * a.table_seq_rows : 0) + s;
    }
    const T* crow = reinterpret_cast<const T*>(a.cos) + trow * D;
    const T* srow = reinterpret_cast<const T*>(a.sin) + trow * D;
    float c0[8], s0[8], c1[8], s1[8];
    unpack<T>(load_chunk<T>(crow + j), c0);
    unpack<T>(load_chunk<T>(srow + j), s0);
    unpack<T>(load_chunk<T>(crow + j + half), c1);
    unpack<T>(load_chunk<T>(srow + j + half), s1);

    const int h0 = blockIdx.y * a.heads_per_block;
    const int h1 = min(h0 + a.heads_per_block, a.hq + a.hkv);
    for (int hh = h0; hh < h1; ++hh) {
        const bool isq = hh < a.hq;
        const int h = isq ? hh : hh - a.hq;
        const T* src = reinterpret_cast<const T*>(isq ? a.q : a.k) + (isq ? qoff + (int64_t)h * a.qs[2] : koff + (int64_t)h * a.ks[2]);
        T* dst = reinterpret_cast<T*>(isq ? a.oq : a.ok) + (isq ? qoff + (int64_t)h * a.qs[2] : koff + (int64_t)h * a.ks[2]);
        float x[8], y[8];
        unpack<T>(load_chunk<T>(src + j), x);
        unpack<T>(load_chunk<T>(src + j + half), y);
        rotate_pair(x, y, c0, s0, c1, s1);
        store_chunk<T>(dst + j, pack<T>(x));
        store_chunk<T>(dst + j + half, pack<T>(y));
    }
}

hipError_t launch_rope_qk(const rope_attn_params* p, hipStream_t stream) {
    QkArgs a;
    a.q = p->q;
    a.k = p->k;
    a.oq = p->out_q;
    a.ok = p->out_k;
    a.cos = p->cos;
    a.sin = p->sin;
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = p->q_stride[i];
        a.ks[i] = p->k_stride[i];
    }
    a.varlen = p->cu_seqlens != nullptr;
    a.seqlen = p->seqlen;
    a.rows = a.varlen ? p->ntokens : p->batch * p->seqlen;
    a.hq = p->hq;
    a.hkv = p->hkv;
    a.head_dim = p->head_dim;
    a.table_seq_rows = p->table_seq_rows;
    // heads per block: enough blocks to fill the chip, table reuse across the group
    const int heads = p->hq + p->hkv;
    const int64_t threads = (int64_t)a.rows * (p->head_dim / 16);
    const int64_t blocks_x = (threads + 255) / 256;
    int hpb = 8;
    while (hpb > 1 && blocks_x * ((heads + hpb - 1) / hpb) < 2048) hpb >>= 1;
    a.heads_per_block = hpb;
    const dim3 block(256);
    const dim3 grid((unsigned)blocks_x, (unsigned)((heads + hpb - 1) / hpb));
    switch (p->dtype) {
        case ROPE_DT_BF16: hipLaunchKernelGGL(rope_qk_kernel<__bf16>, grid, block, 0, stream, a); break;
        case ROPE_DT_F16: hipLaunchKernelGGL(rope_qk_kernel<_Float16>, grid, block, 0, stream, a); break;
        case ROPE_DT_F32: hipLaunchKernelGGL(rope_qk_kernel<float>, grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ropefa

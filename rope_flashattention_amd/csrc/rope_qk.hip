// rope_qk: standalone RoPE of Q and K on gfx950 (the unfused step), rotate-half or
// interleaved pairs.
//
// The Rope op of the [DynamicNTKOperation] page (section 算子上下文) takes q, k and the
// sin/cos tables and returns rotated q and k; written per element,
//   x'[j] = x[j] * cos[j] + rotate_half(x)[j] * sin[j],  rotate_half(x) = cat(-x[D/2:], x[:D/2]).
// This is the "RoPE writes to HBM, attention reads it back" step that the [RoPE-fusion
// blog] (section 二) measures as pure data movement, so the kernel is HBM bound:
// it reads q and k, writes q' and k', and reads each table row once per block of heads
// (or forms the row's values in the kernel from positions and inverse frequencies).
//
// Thread mapping: one thread owns one token and one 8-column chunk j of the first half
// together with chunk j + D/2 (for the rotate-half pairing the two are partners; for the
// interleaved pairing each chunk holds whole pairs).  It loads (or forms) the four table
// chunks once and then walks a group of heads (q heads first, then k heads), so table
// traffic is amortised over the group.
#include "common.h"

namespace ropefa {

struct QkArgs {
    const void* q;
    const void* k;
    void* oq;
    void* ok;
    const void* cos;
    const void* sin;
    const int32_t* pos;       // tables formed in the kernel (cos == sin == NULL)
    const float* inv_freq;
    const int32_t* cu_seqlens;
    int64_t qs[3];  // {batch, token, head} strides in elements (q and out_q)
    int64_t ks[3];  // (k and out_k)
    int32_t varlen;
    int32_t seqlen;         // dense: tokens per sequence
    int32_t rows;           // token rows processed: dense batch*seqlen, varlen ntokens
    int32_t batch;
    int32_t hq, hkv;
    int32_t head_dim;
    int32_t table_seq_rows; // dense: 0 = shared table
    int32_t heads_per_block;
    int32_t inv_freq_rows;
    float pos_scale;
};

// Table values of the 16 columns j..j+7 and j+D/2..j+D/2+7 of table row trow: read from
// the tables, or formed here exactly as rope_tables_ex writes them (float32 angle, the
// library's sincos, rounded to T) for sequence b's inverse frequencies.
template <typename T, int PAIR, bool GEN>
__device__ __forceinline__ void qk_table_values(const QkArgs& a, int64_t trow, int b, int j, float (&c0)[8],
                                                float (&s0)[8], float (&c1)[8], float (&s1)[8]) {
    const int D = a.head_dim;
    const int half = D >> 1;
    if (!GEN) {
        const T* crow = reinterpret_cast<const T*>(a.cos) + trow * D;
        const T* srow = reinterpret_cast<const T*>(a.sin) + trow * D;
        unpack<T>(load_chunk<T>(crow + j), c0);
        unpack<T>(load_chunk<T>(srow + j), s0);
        unpack<T>(load_chunk<T>(crow + j + half), c1);
        unpack<T>(load_chunk<T>(srow + j + half), s1);
        return;
    }
    const int32_t p = a.pos[trow];
    const float* f = a.inv_freq + (int64_t)(a.inv_freq_rows > 1 ? b : 0) * half;
    float sv[8], cv[8];
    if (PAIR == ROPE_PAIR_HALF) {
        // columns j.. and j+D/2.. both use frequencies j .. j+7
#pragma unroll
        for (int e = 0; e < 8; ++e) rope_sincos(table_angle(p, a.pos_scale, f[j + e]), sv[e], cv[e]);
        unpack<T>(pack<T>(cv), c0);
        unpack<T>(pack<T>(sv), s0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            c1[e] = c0[e];
            s1[e] = s0[e];
        }
    } else {
        // column m uses frequency m/2: j/2 .. j/2+3 and (j+D/2)/2 .. (j+D/2)/2+3
#pragma unroll
        for (int e = 0; e < 4; ++e) rope_sincos(table_angle(p, a.pos_scale, f[j / 2 + e]), sv[e], cv[e]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            rope_sincos(table_angle(p, a.pos_scale, f[(j + half) / 2 + e]), sv[4 + e], cv[4 + e]);
        float c2[8], s2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            c2[e] = cv[e / 2];
            s2[e] = sv[e / 2];
        }
        unpack<T>(pack<T>(c2), c0);
        unpack<T>(pack<T>(s2), s0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            c2[e] = cv[4 + e / 2];
            s2[e] = sv[4 + e / 2];
        }
        unpack<T>(pack<T>(c2), c1);
        unpack<T>(pack<T>(s2), s1);
    }
}

template <typename T, int PAIR, bool GEN>
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
    int b = 0;
    if (a.varlen) {
        qoff = (int64_t)t * a.qs[1];
        koff = (int64_t)t * a.ks[1];
        trow = t;
        if (GEN && a.inv_freq_rows > 1) {
            // sequence of packed token t (batch <= ROPE_MAX_BATCH here)
#pragma unroll
            for (int i = 1; i < ROPE_MAX_BATCH; ++i) b += (i < a.batch && t >= a.cu_seqlens[i]) ? 1 : 0;
        }
    } else {
        b = t / a.seqlen;
        const int s = t - b * a.seqlen;
        qoff = (int64_t)b * a.qs[0] + (int64_t)s * a.qs[1];
        koff = (int64_t)b * a.ks[0] + (int64_t)s * a.ks[1];
        trow = (a.table_seq_rows ? (int64_t)b * a.table_seq_rows : 0) + s;
    }
    float c0[8], s0[8], c1[8], s1[8];
    qk_table_values<T, PAIR, GEN>(a, trow, b, j, c0, s0, c1, s1);

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
        if (PAIR == ROPE_PAIR_HALF) {
            rotate_pair(x, y, c0, s0, c1, s1);
        } else {
            rotate_interleaved(x, c0, s0);
            rotate_interleaved(y, c1, s1);
        }
        store_chunk<T>(dst + j, pack<T>(x));
        store_chunk<T>(dst + j + half, pack<T>(y));
    }
}

template <typename T>
static void launch_qk_typed(const QkArgs& a, int pairing, bool gen, dim3 grid, hipStream_t stream) {
    const dim3 block(256);
    const int key = pairing * 2 + (gen ? 1 : 0);
    switch (key) {
        case 0: hipLaunchKernelGGL((rope_qk_kernel<T, ROPE_PAIR_HALF, false>), grid, block, 0, stream, a); break;
        case 1: hipLaunchKernelGGL((rope_qk_kernel<T, ROPE_PAIR_HALF, true>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((rope_qk_kernel<T, ROPE_PAIR_INTERLEAVED, false>), grid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL((rope_qk_kernel<T, ROPE_PAIR_INTERLEAVED, true>), grid, block, 0, stream, a); break;
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
    a.pos = p->pos;
    a.inv_freq = p->inv_freq;
    a.cu_seqlens = p->cu_seqlens;
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = p->q_stride[i];
        a.ks[i] = p->k_stride[i];
    }
    a.varlen = p->cu_seqlens != nullptr;
    a.seqlen = p->seqlen;
    a.rows = a.varlen ? p->ntokens : p->batch * p->seqlen;
    a.batch = p->batch;
    a.hq = p->hq;
    a.hkv = p->hkv;
    a.head_dim = p->head_dim;
    a.table_seq_rows = p->table_seq_rows;
    a.inv_freq_rows = p->inv_freq_rows;
    a.pos_scale = p->pos_scale;
    const bool gen = p->cos == nullptr;
    // heads per block: enough blocks to fill the chip, table reuse across the group
    const int heads = p->hq + p->hkv;
    const int64_t threads = (int64_t)a.rows * (p->head_dim / 16);
    const int64_t blocks_x = (threads + 255) / 256;
    int hpb = 8;
    while (hpb > 1 && blocks_x * ((heads + hpb - 1) / hpb) < 2048) hpb >>= 1;
    a.heads_per_block = hpb;
    const dim3 grid((unsigned)blocks_x, (unsigned)((heads + hpb - 1) / hpb));
    switch (p->dtype) {
        case ROPE_DT_BF16: launch_qk_typed<__bf16>(a, p->pairing, gen, grid, stream); break;
        case ROPE_DT_F16: launch_qk_typed<_Float16>(a, p->pairing, gen, grid, stream); break;
        case ROPE_DT_F32: launch_qk_typed<float>(a, p->pairing, gen, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ropefa

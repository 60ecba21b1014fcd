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
// The same kernel with q's heads left out is the fused attention's k' pre-pass (k' rows
// written once per key into a packed workspace).
//
// Thread mapping: one thread owns one token and one 8-column chunk j of the first half
// together with chunk j + D/2 (for the rotate-half pairing the two are partners; for the
// interleaved pairing each chunk holds whole pairs).  It loads (or forms) the four table
// chunks once and then walks a group of heads (q heads first, then k heads), so table
// traffic is amortised over the group.  Calls that move more than twice the last-level
// cache use nontemporal loads and stores (measured on B1 H64/8 S16384, 612 MB: 5.45 -> 5.8
// TB/s; on the smaller workloads, whose output the cache still holds, they are slower).
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
    int64_t ks[3];  // k
    int64_t oks[3]; // out_k (equal to ks for rope_qk; the packed k' rows for the attention pre-pass)
    int32_t varlen;
    int32_t seqlen;         // dense: tokens per sequence
    int32_t rows;           // token rows processed: dense batch*seqlen, varlen ntokens
    int32_t batch;
    int32_t hq, hkv;
    int32_t head_dim;
    int32_t table_seq_rows; // dense: 0 = shared table
    int32_t heads_per_block;
    int32_t inv_freq_rows;
    int32_t half_cols;      // rotate-half tables: columns [0, D/2) read and applied to both halves
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
        if (PAIR == ROPE_PAIR_HALF && a.half_cols) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                c1[e] = c0[e];
                s1[e] = s0[e];
            }
            return;
        }
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

constexpr int kQkMaxHeads = 8;  // heads one thread rotates (heads_per_block <= this)
// Calls that move more than this (q and k read and written) stream past the caches: twice
// the 256 MB last-level cache, so nothing the call writes would still be there when read.
constexpr uint64_t kQkStreamBytes = 512ull << 20;

template <bool NT, typename T>
__device__ __forceinline__ Chunk8<T> qk_load(const T* p) {
    if constexpr (NT) return load_stream<T>(p);
    else return load_chunk<T>(p);
}
template <bool NT, typename T>
__device__ __forceinline__ void qk_store(T* p, const Chunk8<T>& c) {
    if constexpr (NT) store_stream<T>(p, c);
    else store_chunk<T>(p, c);
}

// HEADS_INNER (layouts whose heads are contiguous within a token, BSND and packed TND):
// one thread per (token, head, chunk), the chunk index fastest and then the head, so a
// wave's loads cover whole head rows of one token; the table chunks, the same for all heads
// of a token, are read by every head's lanes from the same addresses.  Otherwise (BNSD,
// where a head's tokens are contiguous): one thread per (token, chunk), walking the
// workgroup's group of heads.
template <typename T, int PAIR, bool GEN, bool NT, bool HEADS_INNER>
__global__ __launch_bounds__(256) void rope_qk_kernel(QkArgs a) {
    const int D = a.head_dim;
    const int half = D >> 1;
    const int chunks = half >> 3;
    const int heads = a.hq + a.hkv;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int t, j, h0, nh;
    if constexpr (HEADS_INNER) {
        if (gid >= (int64_t)a.rows * heads * chunks) return;
        const int64_t th = gid / chunks;
        j = (int)(gid - th * chunks) * 8;
        t = (int)(th / heads);
        h0 = (int)(th - (int64_t)t * heads);
        nh = 1;
    } else {
        if (gid >= (int64_t)a.rows * chunks) return;
        t = (int)(gid / chunks);
        j = (int)(gid - (int64_t)t * chunks) * 8;
        h0 = blockIdx.y * a.heads_per_block;
        nh = min(a.heads_per_block, heads - h0);
    }

    // token -> (sequence, position) offsets and table row
    int64_t qoff, koff, kooff, trow;
    int b = 0;
    if (a.varlen) {
        qoff = (int64_t)t * a.qs[1];
        koff = (int64_t)t * a.ks[1];
        kooff = (int64_t)t * a.oks[1];
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
        kooff = (int64_t)b * a.oks[0] + (int64_t)s * a.oks[1];
        trow = (a.table_seq_rows ? (int64_t)b * a.table_seq_rows : 0) + s;
    }
    float c0[8], s0[8], c1[8], s1[8];
    qk_table_values<T, PAIR, GEN>(a, trow, b, j, c0, s0, c1, s1);

    auto head_ptrs = [&](int hh, const T*& src, T*& dst) {
        const bool isq = hh < a.hq;
        const int h = isq ? hh : hh - a.hq;
        const int64_t off = isq ? qoff + (int64_t)h * a.qs[2] : koff + (int64_t)h * a.ks[2];
        src = reinterpret_cast<const T*>(isq ? a.q : a.k) + off;
        dst = isq ? reinterpret_cast<T*>(a.oq) + off : reinterpret_cast<T*>(a.ok) + kooff + (int64_t)h * a.oks[2];
    };
    auto rotate_store = [&](const Chunk8<T>& xc, const Chunk8<T>& yc, T* dst) {
        float x[8], y[8];
        unpack<T>(xc, x);
        unpack<T>(yc, y);
        if (PAIR == ROPE_PAIR_HALF) {
            rotate_pair(x, y, c0, s0, c1, s1);
        } else {
            rotate_interleaved(x, c0, s0);
            rotate_interleaved(y, c1, s1);
        }
        qk_store<NT, T>(dst + j, pack<T>(x));
        qk_store<NT, T>(dst + j + half, pack<T>(y));
    };
    if constexpr (NT || HEADS_INNER) {
        // streaming (data beyond the caches), or one head per thread: head by head
        for (int i = 0; i < nh; ++i) {
            const T* src;
            T* dst;
            head_ptrs(h0 + i, src, dst);
            const Chunk8<T> xc = qk_load<NT, T>(src + j);
            const Chunk8<T> yc = qk_load<NT, T>(src + j + half);
            rotate_store(xc, yc, dst);
        }
    } else {
        // every load of the thread's heads is issued before the first rotation and store, so
        // a thread keeps 2 * kQkMaxHeads loads in flight instead of 2 (a store may alias the
        // next head's load when the call is in place, which otherwise keeps each head's loads
        // behind the previous head's stores)
        Chunk8<T> xr[kQkMaxHeads], yr[kQkMaxHeads];
#pragma unroll
        for (int i = 0; i < kQkMaxHeads; ++i) {
            if (i < nh) {
                const T* src;
                T* dst;
                head_ptrs(h0 + i, src, dst);
                xr[i] = qk_load<NT, T>(src + j);
                yr[i] = qk_load<NT, T>(src + j + half);
            }
        }
#pragma unroll
        for (int i = 0; i < kQkMaxHeads; ++i) {
            if (i < nh) {
                const T* src;
                T* dst;
                head_ptrs(h0 + i, src, dst);
                rotate_store(xr[i], yr[i], dst);
            }
        }
    }
}

template <typename T, bool NT, bool HI>
static void launch_qk_mode(const QkArgs& a, int pairing, bool gen, dim3 grid, hipStream_t stream) {
    const dim3 block(256);
    const int key = pairing * 2 + (gen ? 1 : 0);
    switch (key) {
        case 0: hipLaunchKernelGGL((rope_qk_kernel<T, ROPE_PAIR_HALF, false, NT, HI>), grid, block, 0, stream, a); break;
        case 1: hipLaunchKernelGGL((rope_qk_kernel<T, ROPE_PAIR_HALF, true, NT, HI>), grid, block, 0, stream, a); break;
        case 2:
            hipLaunchKernelGGL((rope_qk_kernel<T, ROPE_PAIR_INTERLEAVED, false, NT, HI>), grid, block, 0, stream, a);
            break;
        case 3:
            hipLaunchKernelGGL((rope_qk_kernel<T, ROPE_PAIR_INTERLEAVED, true, NT, HI>), grid, block, 0, stream, a);
            break;
    }
}

template <typename T>
static void launch_qk_typed(const QkArgs& a, int pairing, bool gen, bool nt, bool hi, dim3 grid,
                            hipStream_t stream) {
    if (nt)
        hi ? launch_qk_mode<T, true, true>(a, pairing, gen, grid, stream)
           : launch_qk_mode<T, true, false>(a, pairing, gen, grid, stream);
    else
        hi ? launch_qk_mode<T, false, true>(a, pairing, gen, grid, stream)
           : launch_qk_mode<T, false, false>(a, pairing, gen, grid, stream);
}

// hq heads of q (0: k only) and the hkv heads of k; out_k rows at strides oks.
static hipError_t launch_qk(const rope_attn_params* p, int hq, void* ok, const int64_t oks[3], bool half_cols,
                            hipStream_t stream) {
    QkArgs a;
    a.q = p->q;
    a.k = p->k;
    a.oq = p->out_q;
    a.ok = ok;
    a.cos = p->cos;
    a.sin = p->sin;
    a.pos = p->pos;
    a.inv_freq = p->inv_freq;
    a.cu_seqlens = p->cu_seqlens;
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = p->q_stride[i];
        a.ks[i] = p->k_stride[i];
        a.oks[i] = oks[i];
    }
    a.half_cols = half_cols ? 1 : 0;
    a.varlen = p->cu_seqlens != nullptr;
    a.seqlen = p->seqlen;
    a.rows = a.varlen ? p->ntokens : p->batch * p->seqlen;
    a.batch = p->batch;
    a.hq = hq;
    a.hkv = p->hkv;
    a.head_dim = p->head_dim;
    a.table_seq_rows = p->table_seq_rows;
    a.inv_freq_rows = p->inv_freq_rows;
    a.pos_scale = p->pos_scale;
    const bool gen = p->cos == nullptr;
    const int heads = hq + p->hkv;
    const int chunks = p->head_dim / 16;
    // heads contiguous within a token (BSND, packed TND): one thread per (token, head, chunk)
    const bool hi = (hq == 0 || p->q_stride[2] < p->q_stride[1]) && p->k_stride[2] < p->k_stride[1] &&
                    ((int64_t)a.rows * heads * chunks + 255) / 256 <= (int64_t)INT32_MAX;
    dim3 grid;
    if (hi) {
        a.heads_per_block = 1;
        grid = dim3((unsigned)(((int64_t)a.rows * heads * chunks + 255) / 256));
    } else {
        // heads per block: enough blocks to fill the chip, table reuse across the group
        const int64_t blocks_x = ((int64_t)a.rows * chunks + 255) / 256;
        int hpb = kQkMaxHeads;
        while (hpb > 1 && blocks_x * ((heads + hpb - 1) / hpb) < 2048) hpb >>= 1;
        a.heads_per_block = hpb;
        grid = dim3((unsigned)blocks_x, (unsigned)((heads + hpb - 1) / hpb));
    }
    const uint64_t moved = 2ull * (uint64_t)a.rows * (uint64_t)heads * (uint64_t)p->head_dim *
                           (uint64_t)dtype_bytes(p->dtype);
    const bool nt = moved > kQkStreamBytes;
    switch (p->dtype) {
        case ROPE_DT_BF16: launch_qk_typed<__bf16>(a, p->pairing, gen, nt, hi, grid, stream); break;
        case ROPE_DT_F16: launch_qk_typed<_Float16>(a, p->pairing, gen, nt, hi, grid, stream); break;
        case ROPE_DT_F32: launch_qk_typed<float>(a, p->pairing, gen, nt, hi, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_rope_qk(const rope_attn_params* p, hipStream_t stream) {
    return launch_qk(p, p->hq, p->out_k, p->k_stride, false, stream);
}

// The attention pre-pass: k' of every key row and kv head into kout, head-major (dense
// [batch, hkv, seqlen, D], varlen [hkv, ntokens, D], so that a key tile is one contiguous
// block), with the fused kernel's table use (rotate-half tables: columns [0, D/2) only), so
// k' equals what its in-loop rotation stages.
hipError_t launch_rope_k_prepass(const rope_attn_params* p, void* kout, hipStream_t stream) {
    const int64_t D = p->head_dim;
    const int64_t plane = (p->cu_seqlens ? (int64_t)p->ntokens : (int64_t)p->seqlen) * D;
    const int64_t oks[3] = {p->cu_seqlens ? 0 : (int64_t)p->hkv * plane, D, plane};
    return launch_qk(p, 0, kout, oks, true, stream);
}

}  // namespace ropefa

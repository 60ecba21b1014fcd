// rope_flash_attn_bwd: gradients of RoPE fused into FlashAttention, on gfx950.
//
// What is computed (the derivatives of the forward definition; the [FlashAttention blog]
// says the operator serves training): per (sequence, q head) with q' = M q and k' = M k the
// rotated rows (M the token's Rope-op matrix), S = s * q'k'^T, P = softmax(S) recomputed
// from the forward's lse, and dO the output gradient,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),  delta = rowsum(dO * O),
//   dq' = s * dS k',  dk' = s * dS^T q',  dq = M^T dq',  dk = M^T dk'.
// GQA: a kv head's dk and dv sum over the q heads of its group.
//
// Three kernels, no atomics:
//   * bwd_prep_kernel: per (query row, q head) delta and the rotated row q' = M q, per
//     (key row, kv head) k' = M k, into the workspace (so the two main kernels stage plain
//     copies; only their epilogues use the tables).
//   * bwd_dkv_kernel: a workgroup of 8 waves (two per SIMD) owns 128 keys of one (sequence,
//     kv head) and accumulates dV^T and dK'^T over every q head of the group and every
//     query block of 32 rows that can see its keys.  Main waves 0-3 keep their 32 keys'
//     rotated K' and V as MFMA B operands in registers; per block they form S and dP with
//     the 32x32x16 MFMA (A = the block's Q' and dO rows read from LDS in the permuted row
//     order pi, which leaves each lane half with 16 consecutive queries of one key), then
//     P and dS, accumulate dV^T += dO^T P and leave dS in LDS.  Helper waves 4-7 stage the
//     blocks and, one block later, accumulate dK'^T += Q'^T dS for the keys of main wave
//     w - 4.  The transposing LDS read (ds_read_b64_tr_b16) supplies dO^T and Q'^T.
//   * bwd_dq_kernel: a workgroup of 8 waves owns 256 query rows of one (sequence, q head);
//     each wave keeps its 32 rows' Q' and dO as B operands and, per 64-key tile staged in
//     LDS (K', V), forms S^T, dP^T and dS^T and accumulates
//     dQ'^T += K'^T dS^T (K'^T by the transposing read).
// An LDS tile read both ways is stored twice: rows in the pi order for the row reads and
// in natural order for the transposing reads, each at a padded pitch (bank-conflict free
// reads, constant read offsets).  Each kernel loads its blocks two ahead into two register
// sets used in turn (a block's loads then have a whole block's compute to arrive), LDS is
// double-buffered (triple for a copy read one block later) with one barrier per block, and
// the A operands of the row reads are fetched two products ahead; the workgroups that read
// the same rows run on one XCD in step.  The epilogues apply M^T (the transposed Rope op)
// to dq' and dk' before the stores.
#include <type_traits>

#include "common.h"

namespace ropefa {

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    const void* cos;
    const void* sin;
    void* dq;
    void* dk;
    void* dv;
    float* delta;                // workspace [hq, rows]
    void* qrot;                  // workspace [hq, rows, D]: q' of every query row
    void* krot;                  // workspace [hkv, rows, D]: k' of every key row
    const int32_t* cu_seqlens;   // nullptr: dense
    int64_t qs[3], ks[3], vs[3], os[3], dos[3], dqs[3], dks[3], dvs[3];  // {batch, token, head}
    int32_t batch, hq, hkv, group, seqlen, table_seq_rows, lse_stride, causal;
    int32_t rows;                // query rows in total (dense batch*seqlen, varlen ntokens)
    int32_t max_seqlen;          // varlen: host bound of every sequence length (the grid covers it)
    int32_t kv_tiles, q_tiles;   // 128-key tiles (dK/dV grid) and query tiles (dQ grid) per sequence
    float scale, scale_log2;
};

// Workgroups go to the 8 XCDs round robin by linear id.  The workgroups of one group
// (those reading the same rows: one (sequence, kv head)) are kept on one XCD and start
// together, so they share that XCD's L2; item = rank within the group, longest first.
// An XCD's groups are taken K at a time with their items interleaved (item t of each of the
// K groups, then item t + 1): a group dispatched last would otherwise start its longest
// items when the XCD is nearly done and leave the other CUs idle at the end.
template <int K>
__device__ __forceinline__ void xcd_grouped(int id, int per_group, int ngroups, int& grp, int& item) {
    if ((ngroups & 7) == 0) {
        const int slot = id >> 3;       // position in this XCD's dispatch order
        const int G = ngroups >> 3;     // groups per XCD
        const int span = K * per_group;
        int chunk = slot / span, kc = K;
        if (chunk >= G / K) {           // the last, partial chunk of G % K groups
            chunk = G / K;
            kc = G - chunk * K;
        }
        const int rem = slot - chunk * span;
        item = rem / kc;
        grp = (id & 7) + 8 * (chunk * K + rem % kc);
    } else {
        grp = id / per_group;
        item = id - grp * per_group;
    }
}

template <typename T> struct BMma;
template <> struct BMma<__bf16> {
    __device__ static __forceinline__ f32x16 run(const u32x4& a, const u32x4& b, const f32x16& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};
template <> struct BMma<_Float16> {
    __device__ static __forceinline__ f32x16 run(const u32x4& a, const u32x4& b, const f32x16& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      c, 0, 0, 0);
    }
};

__device__ __forceinline__ i16x4 bwd_tr16(const void* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}
// MFMA row m holds row pi(m) of a 32-row block: lane half h then holds rows 16h .. 16h+15
__device__ __forceinline__ int pi_row(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }
__device__ __forceinline__ int pi_inv(int r) { return (r & 3) | (((r >> 4) & 1) << 2) | (((r >> 2) & 3) << 3); }

// LDS tiles.  A tile read as MFMA A operands row by row is stored with its rows in the pi
// order (row m of each 32-row block holds row pi(m)), pitch D + 8: lane n reads row n, so
// every read is the lane's base plus a constant, and a 16-lane group of 16-byte reads
// (rows n .. n+15) starts on 16 distinct 4-bank groups (LDS: 64 banks of 4 bytes).  A tile
// read by ds_read_b64_tr_b16 keeps the natural row order at pitch D + 32: the 32 lanes of
// such a read cover 4 consecutive rows x 64 bytes, which then fall in 4 distinct 16-bank
// quarters.  Stores are at most 2-way bank conflicted.
template <int D> struct BwdLds {
    static constexpr int PA = D + 8;   // row-read copies
    static constexpr int PT = D + 32;  // transposing-read copies
};

struct BwdSeq {
    int L;
    int64_t tok;     // lse / delta index of row 0
    int64_t tab;     // table row of row 0
    int64_t bq, bk, bv, bo, bdo, bdq, bdk, bdv;
};
__device__ __forceinline__ BwdSeq bwd_seq(const BwdArgs& a, int b) {
    // base offset = ib * stride[0] + it * stride[1] with (ib, it) = (b, 0) dense and
    // (0, first token) varlen: constant stride indices (a selected index would put the
    // argument block in scratch memory)
    BwdSeq s;
    int64_t ib, it;
    if (a.cu_seqlens) {
        // device-held lengths are clamped: rows stay inside the packed rows and the grid
        const int64_t c0 = min(max((int64_t)a.cu_seqlens[b], (int64_t)0), (int64_t)a.rows);
        const int64_t len = (int64_t)a.cu_seqlens[b + 1] - c0;
        const int s0 = (int)c0;
        s.L = (int)max((int64_t)0, min(len, min((int64_t)a.max_seqlen, (int64_t)a.rows - c0)));
        s.tok = s0;
        s.tab = s0;
        ib = 0;
        it = s0;
    } else {
        s.L = a.seqlen;
        s.tok = (int64_t)b * a.seqlen;
        s.tab = a.table_seq_rows ? (int64_t)b * a.table_seq_rows : 0;
        ib = b;
        it = 0;
    }
    s.bq = ib * a.qs[0] + it * a.qs[1];
    s.bk = ib * a.ks[0] + it * a.ks[1];
    s.bv = ib * a.vs[0] + it * a.vs[1];
    s.bo = ib * a.os[0] + it * a.os[1];
    s.bdo = ib * a.dos[0] + it * a.dos[1];
    s.bdq = ib * a.dqs[0] + it * a.dqs[1];
    s.bdk = ib * a.dks[0] + it * a.dks[1];
    s.bdv = ib * a.dvs[0] + it * a.dvs[1];
    return s;
}

// The Rope op (M) of the fused forward on a packed chunk pair: x = columns d..d+7, y =
// columns d+D/2..d+D/2+7 of one row, rounded once to T.  Rotate-half uses the table's first
// half only (columns d..d+7 for both halves), as the forward does; interleaved uses both.
template <typename T, int PAIR>
__device__ __forceinline__ void rope_fwd_packed(u32x4& x, u32x4& y, const u32x4& c0, const u32x4& s0, const u32x4& c1,
                                                const u32x4& s1) {
    if (PAIR == 1) {
        u32x4 xo, yo;
        rotate_pair_packed<T>(x, y, c0, s0, xo, yo);
        x = xo;
        y = yo;
    } else if (PAIR == 2) {
        x = rotate_interleaved_packed<T>(x, c0, s0);
        y = rotate_interleaved_packed<T>(y, c1, s1);
    }
}

// Loads chunk pair (d, d + D/2) of row p and rotates it with the row's table values.
template <typename T, int PAIR>
__device__ __forceinline__ void load_rotated_pair(const T* p, const T* crow, const T* srow, int d, int half, u32x4& x,
                                                  u32x4& y) {
    x = load_chunk<T>(p + d).w;
    y = load_chunk<T>(p + d + half).w;
    if (PAIR == 0) return;
    const u32x4 c0 = load_chunk<T>(crow + d).w, s0 = load_chunk<T>(srow + d).w;
    u32x4 c1 = c0, s1 = s0;
    if (PAIR == 2) {
        c1 = load_chunk<T>(crow + d + half).w;
        s1 = load_chunk<T>(srow + d + half).w;
    }
    rope_fwd_packed<T, PAIR>(x, y, c0, s0, c1, s1);
}

// ============================================================================ prep
// Item (j, row) for j < hq: delta of q head j and q'; j >= hq: k' of kv head j - hq.  D/16
// lanes per item, lane c owning columns 8c..8c+7 and their rotation partners + D/2.
template <typename T, int D, int PAIR>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
    constexpr int CH = D / 16;  // lanes per item, a power of two
    constexpr int HALF = D / 2;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t idx = gid / CH;
    const int c = (int)(gid - idx * CH) * 8;
    // head-major items: a wave covers consecutive rows of one head (contiguous in BNSD
    // inputs and in the workspace)
    const int j = (int)(idx / a.rows);
    const int64_t row = idx - (int64_t)j * a.rows;
    if (j >= a.hq + a.hkv) return;  // the whole CH-lane group leaves together
    int64_t b = 0, s = row, tab = row;
    if (!a.cu_seqlens) {
        b = row / a.seqlen;
        s = row - b * a.seqlen;
        tab = (a.table_seq_rows ? b * a.table_seq_rows : 0) + s;
    }
    const T* crow = PAIR ? reinterpret_cast<const T*>(a.cos) + tab * D : nullptr;
    const T* srow = PAIR ? reinterpret_cast<const T*>(a.sin) + tab * D : nullptr;
    u32x4 x, y;
    if (j < a.hq) {
        const int64_t tq = a.cu_seqlens ? row * a.qs[1] : b * a.qs[0] + s * a.qs[1];
        const int64_t to = a.cu_seqlens ? row * a.os[1] : b * a.os[0] + s * a.os[1];
        const int64_t td = a.cu_seqlens ? row * a.dos[1] : b * a.dos[0] + s * a.dos[1];
        load_rotated_pair<T, PAIR>(reinterpret_cast<const T*>(a.q) + tq + (int64_t)j * a.qs[2], crow, srow, c, HALF,
                                   x, y);
        T* dst = reinterpret_cast<T*>(a.qrot) + ((int64_t)j * a.rows + row) * D + c;
        *reinterpret_cast<u32x4*>(dst) = x;
        *reinterpret_cast<u32x4*>(dst + HALF) = y;
        const T* op = reinterpret_cast<const T*>(a.o) + to + (int64_t)j * a.os[2] + c;
        const T* dp = reinterpret_cast<const T*>(a.dout) + td + (int64_t)j * a.dos[2] + c;
        float o0[8], o1[8], d0[8], d1[8];
        unpack<T>(load_chunk<T>(op), o0);
        unpack<T>(load_chunk<T>(op + HALF), o1);
        unpack<T>(load_chunk<T>(dp), d0);
        unpack<T>(load_chunk<T>(dp + HALF), d1);
        float sum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sum = __builtin_fmaf(o0[e], d0[e], sum);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum = __builtin_fmaf(o1[e], d1[e], sum);
#pragma unroll
        for (int m = CH >> 1; m > 0; m >>= 1) sum += __shfl_xor(sum, m, CH);
        if (c == 0) a.delta[(int64_t)j * a.rows + row] = sum;
    } else {
        const int kh = j - a.hq;
        const int64_t tk = a.cu_seqlens ? row * a.ks[1] : b * a.ks[0] + s * a.ks[1];
        load_rotated_pair<T, PAIR>(reinterpret_cast<const T*>(a.k) + tk + (int64_t)kh * a.ks[2], crow, srow, c, HALF,
                                   x, y);
        T* dst = reinterpret_cast<T*>(a.krot) + ((int64_t)kh * a.rows + row) * D + c;
        *reinterpret_cast<u32x4*>(dst) = x;
        *reinterpret_cast<u32x4*>(dst + HALF) = y;
    }
}

// Epilogue helper: scale the 4-value groups of a transposed accumulator (lane holds column
// n; rows d = mb*32 + 8*q4 + 4*hh + e), apply M^T with the table row, and store the row.
template <typename T, int D, int PAIR>
__device__ __forceinline__ void store_grad_row(const f32x16 (&acc)[D / 32], float scale, int hh, const T* crow,
                                               const T* srow, T* dst) {
    float g[D / 32][16];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) g[mb][i] = acc[mb][i] * scale;
    if (PAIR == 1) {
        // M^T for pairs (j, j + D/2) with the table's first half (the forward's M):
        //   g'_j = c_j g_j + s_j g_{j+D/2},  g'_{j+D/2} = c_j g_{j+D/2} - s_j g_j
#pragma unroll
        for (int mb = 0; mb < D / 64; ++mb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d0 = mb * 32 + 8 * q4 + 4 * hh;
                float c0[4], s0[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    c0[e] = (float)crow[d0 + e];
                    s0[e] = (float)srow[d0 + e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = g[mb][4 * q4 + e], y = g[mb + D / 64][4 * q4 + e];
                    g[mb][4 * q4 + e] = __builtin_fmaf(x, c0[e], __fmul_rn(y, s0[e]));
                    g[mb + D / 64][4 * q4 + e] = __builtin_fmaf(y, c0[e], -__fmul_rn(x, s0[e]));
                }
            }
    } else if (PAIR == 2) {
        // M^T for pairs (2k, 2k+1): g'_2k = c_2k g_2k + s_2k+1 g_2k+1, g'_2k+1 = c_2k+1 g_2k+1 - s_2k g_2k
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d0 = mb * 32 + 8 * q4 + 4 * hh;
#pragma unroll
                for (int e = 0; e < 4; e += 2) {
                    const float c0 = (float)crow[d0 + e], s0 = (float)srow[d0 + e];
                    const float c1 = (float)crow[d0 + e + 1], s1 = (float)srow[d0 + e + 1];
                    const float x = g[mb][4 * q4 + e], y = g[mb][4 * q4 + e + 1];
                    g[mb][4 * q4 + e] = __builtin_fmaf(x, c0, __fmul_rn(y, s1));
                    g[mb][4 * q4 + e + 1] = __builtin_fmaf(y, c1, -__fmul_rn(x, s0));
                }
            }
    }
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = mb * 32 + 8 * q4 + 4 * hh;
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<u32x2*>(dst + d0) = u32x2{Elem<T>::pack(g[mb][4 * q4], g[mb][4 * q4 + 1]),
                                                            Elem<T>::pack(g[mb][4 * q4 + 2], g[mb][4 * q4 + 3])};
            }
        }
}

// ============================================================================ staging
// One staging item: the 8-element chunks at columns c and c + D/2 of one row of two
// tensors, loaded one block ahead into registers and written to LDS at the start of the
// next block.
struct StageItem {
    u32x4 a0, a1, b0, b1;
};

template <typename T>
__device__ __forceinline__ void stage_load(StageItem& s, const T* arow, const T* brow, int c, int half) {
    s.a0 = load_chunk<T>(arow + c).w;
    s.a1 = load_chunk<T>(arow + c + half).w;
    s.b0 = load_chunk<T>(brow + c).w;
    s.b1 = load_chunk<T>(brow + c + half).w;
}

// Writes chunk pair (c, c + D/2) (element columns) of row r of a 32-row-block tile: x, y
// into the row-read copy (pi order) and/or the transposing-read copy (natural order).
template <typename T, int D>
__device__ __forceinline__ void store_rowcopy(T* ta, int r, int c, const u32x4& x, const u32x4& y) {
    T* p = ta + ((r & ~31) + pi_inv(r & 31)) * BwdLds<D>::PA + c;
    *reinterpret_cast<u32x4*>(p) = x;
    *reinterpret_cast<u32x4*>(p + D / 2) = y;
}
template <typename T, int D>
__device__ __forceinline__ void store_trcopy(T* tt, int r, int c, const u32x4& x, const u32x4& y) {
    T* p = tt + r * BwdLds<D>::PT + c;
    *reinterpret_cast<u32x4*>(p) = x;
    *reinterpret_cast<u32x4*>(p + D / 2) = y;
}

// ============================================================================ dk, dv
// Eight waves, two per SIMD.  Waves 0-3 (main) own 32 keys each: per block they form S and
// dP, P and dS = P * (dP - delta), accumulate dV^T += dO^T P and leave dS in LDS as the B
// operands of the dK product.  Waves 4-7 (helpers) stage every block into LDS and, one block
// later, accumulate dK'^T += Q'^T dS for the keys of main wave w - 4.  A SIMD then holds one
// wave whose MFMAs can run under the other's vector work; each wave stays within half the
// SIMD's registers.
template <typename T, int D, int PAIR>
__global__ __launch_bounds__(512, 1) void bwd_dkv_kernel(BwdArgs a) {
    constexpr int NS = D / 16;
    constexpr int HALF = D / 2;
    constexpr int CPR = D / 16;        // chunk pairs per row
    constexpr int QITEMS = 32 * CPR;   // staging items of a 32-row block (<= 256)
    static_assert(QITEMS <= 256, "one staging item per helper thread");
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr int PA = BwdLds<D>::PA, PT = BwdLds<D>::PT;
    // row copies and the dO^T copy double-buffered (read in the block's own iteration), the
    // Q'^T copy triple-buffered (read by the helpers one iteration later)
    __shared__ __attribute__((aligned(16))) T sQa[2][32 * PA];
    __shared__ __attribute__((aligned(16))) T sDa[2][32 * PA];
    __shared__ __attribute__((aligned(16))) T sDt[2][32 * PT];
    __shared__ __attribute__((aligned(16))) T sQt[3][32 * PT];
    __shared__ __attribute__((aligned(16))) u32x4 sDS[2][4][2][64];  // dS B operands per key slice and lane
    __shared__ __attribute__((aligned(16))) float sL[2][32];
    __shared__ __attribute__((aligned(16))) float sDel[2][32];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar branches)
    const int l = tid & 63, n = l & 31, hh = l >> 5;
    const int wk = w & 3;  // key slice
    int grp, tile;
    xcd_grouped<2>(blockIdx.x, a.kv_tiles, a.hkv * a.batch, grp, tile);
    const int kvh = grp % a.hkv;
    const int b = grp / a.hkv;
    const BwdSeq sq = bwd_seq(a, b);
    const int L = sq.L;
    const int k0 = tile * 128;
    if (k0 >= L) return;  // whole workgroup
    const int kw0 = k0 + 32 * wk;
    const bool active = kw0 < L;
    const int key = min(kw0 + n, L - 1);

    const int tr_row = (l & 15) >> 2;
    const int tr_col = ((l >> 4) & 1) * 16 + 4 * (l & 3);
    const int mykey = kw0 + n;
    // P of (query qi, this key) is kept iff qi >= qmin
    const int qmin = mykey >= L ? (1 << 30) : (a.causal ? mykey : -(1 << 30));
    const int q_begin = a.causal ? k0 : 0;
    // blocks in order: 32-row query blocks from the last one down, and the group's q heads
    // within each; the workgroups of all key tiles of this (sequence, kv head) start
    // together at the last block and stay in step, reading the same rows at the same time
    const int q_last = q_begin + ((L - 1 - q_begin) >> 5) * 32;
    // the block computes for this slice's keys (wave-uniform)
    auto runs = [&](int q0) { return active && !(a.causal && q0 + 31 < kw0); };
    const T* kp = reinterpret_cast<const T*>(a.krot) + ((int64_t)kvh * a.rows + sq.tok + key) * D;

    if (w < 4) {
        // ================================================================ main waves
        u32x4 kb[NS], vb[NS];
        {
            const T* vp = reinterpret_cast<const T*>(a.v) + sq.bv + (int64_t)key * a.vs[1] + (int64_t)kvh * a.vs[2];
#pragma unroll
            for (int s = 0; s < NS; ++s) kb[s] = load_chunk<T>(kp + 16 * s + 8 * hh).w;
#pragma unroll
            for (int s = 0; s < NS; ++s) vb[s] = load_chunk<T>(vp + 16 * s + 8 * hh).w;
            // complete these loads here: otherwise the loop's first use would wait for
            // every load issued after them
#pragma unroll
            for (int s = 0; s < NS; ++s) asm volatile("" ::"v"(vb[s]));
        }
        f32x16 dvacc[D / 32];
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) dvacc[mb][i] = 0.0f;
        int cq0 = q_last, chi = 0;  // the current block
        int buf = 0;
        for (;;) {
            const int q0 = cq0;
            if (++chi == a.group) {
                chi = 0;
                cq0 -= 32;
            }
            __syncthreads();  // block staged by the helpers
            if (runs(q0)) {
                const T* qa = sQa[buf];
                const T* da = sDa[buf];
                // ---- S and dP: lane (n, hh) gets key kw0 + n against queries q0 + 16hh + i;
                // A operands read two products ahead
                constexpr int PD = 2;
                u32x4 aq[PD + 1], ad[PD + 1];
                auto rd_a = [&](int s) {
                    const int off = n * PA + 16 * s + 8 * hh;
                    aq[s % (PD + 1)] = *reinterpret_cast<const u32x4*>(&qa[off]);
                    ad[s % (PD + 1)] = *reinterpret_cast<const u32x4*>(&da[off]);
                };
#pragma unroll
                for (int s = 0; s < PD; ++s) rd_a(s);
                f32x16 sacc, dpacc;
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[i] = dpacc[i] = 0.0f;
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    if (s + PD < NS) rd_a(s + PD);
                    sacc = BMma<T>::run(aq[s % (PD + 1)], kb[s], sacc);
                    dpacc = BMma<T>::run(ad[s % (PD + 1)], vb[s], dpacc);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // dO^T operands of the dV products, read now so that they arrive during the
                // vector work below
                u32x4 dvop[2][D / 32];
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int mb = 0; mb < D / 32; ++mb) {
                        const T* xt = sDt[buf];
                        const int r = 16 * hh + 8 * s + tr_row;
                        const int e = mb * 32 + tr_col;
                        const i16x4 lo = bwd_tr16(&xt[r * PT + e]);
                        const i16x4 hi = bwd_tr16(&xt[(r + 4) * PT + e]);
                        dvop[s][mb] = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    }
                __builtin_amdgcn_sched_barrier(0);
                // ---- P and dS; the mask matters only for blocks that reach this slice's
                // keys (causal) or for keys past the end: a wave-uniform choice between two
                // copies of this code
                const int thr = qmin - (q0 + 16 * hh);  // query q0 + 16hh + i is masked iff i < thr
                u32x4 pk[2], dsk[2];
                auto probs = [&](auto masked) {
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const f32x4 l0 = *reinterpret_cast<const f32x4*>(&sL[buf][16 * hh + 8 * s]);
                        const f32x4 l1 = *reinterpret_cast<const f32x4*>(&sL[buf][16 * hh + 8 * s + 4]);
                        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&sDel[buf][16 * hh + 8 * s]);
                        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&sDel[buf][16 * hh + 8 * s + 4]);
                        float p[8], ds[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const int i = 8 * s + j;
                            const float lv = j < 4 ? l0[j] : l1[j - 4];
                            const float dl = j < 4 ? d0[j] : d1[j - 4];
                            float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], a.scale_log2, -lv));
                            if (decltype(masked)::value && i < thr) pv = 0.0f;
                            p[j] = pv;
                            ds[j] = pv * (dpacc[i] - dl);
                        }
                        pk[s] = pack<T>(p).w;
                        dsk[s] = pack<T>(ds).w;
                        sDS[buf][wk][s][l] = dsk[s];
                    }
                };
                if (kw0 + 31 >= L || (a.causal && q0 < kw0 + 31))
                    probs(std::true_type{});
                else
                    probs(std::false_type{});
                // dV^T += dO^T P
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int mb = 0; mb < D / 32; ++mb) dvacc[mb] = BMma<T>::run(dvop[s][mb], pk[s], dvacc[mb]);
            }
            buf ^= 1;
            if (cq0 < q_begin) break;
        }
        __syncthreads();  // pairs with the helpers' last barrier
        if (active && kw0 + n < L) {
            const int kr = kw0 + n;
            T* dvp = reinterpret_cast<T*>(a.dv) + sq.bdv + (int64_t)kr * a.dvs[1] + (int64_t)kvh * a.dvs[2];
            store_grad_row<T, D, 0>(dvacc, 1.0f, hh, nullptr, nullptr, dvp);
        }
    } else {
        // ================================================================ helper waves
        const T* Cg = reinterpret_cast<const T*>(a.cos) + sq.tab * D;
        const T* Sg = reinterpret_cast<const T*>(a.sin) + sq.tab * D;
        const T* Qr = reinterpret_cast<const T*>(a.qrot) + sq.tok * D;  // q' rows of this sequence
        const T* Db = reinterpret_cast<const T*>(a.dout) + sq.bdo;
        const int ht = tid - 256;
        // staging: item (row sr, chunk pair sc) of each 32-row block; rows past the end
        // re-read the last row (finite values; their P is exactly 0 through lse = +inf)
        const bool stager = ht < QITEMS;
        const int sr = (ht % QITEMS) / CPR, sc = (ht % CPR) * 8;
        // Every thread issues its loads unconditionally (no branch around a load, so no
        // wait is forced at a join); the loaded values are only used at the block's store.
        StageItem pre[2];
        float pre_l[2], pre_d[2];  // raw lse and delta of row (ht & 31) of the block
        auto load_block = [&](auto slot, int hi, int q0) {
            constexpr int S = decltype(slot)::value;
            const int h = kvh * a.group + hi;
            const int qi = min(q0 + sr, L - 1);
            stage_load<T>(pre[S], Qr + ((int64_t)h * a.rows + qi) * D,
                          Db + (int64_t)qi * a.dos[1] + (int64_t)h * a.dos[2], sc, HALF);
            const int64_t idx = (int64_t)h * a.lse_stride + sq.tok + min(q0 + (ht & 31), L - 1);
            pre_l[S] = a.lse[idx];
            pre_d[S] = a.delta[idx];
        };
        auto store_block = [&](auto slot, int buf, int tbuf, int q0) {
            constexpr int S = decltype(slot)::value;
            if (stager) {
                store_rowcopy<T, D>(sQa[buf], sr, sc, pre[S].a0, pre[S].a1);
                store_trcopy<T, D>(sQt[tbuf], sr, sc, pre[S].a0, pre[S].a1);
                store_rowcopy<T, D>(sDa[buf], sr, sc, pre[S].b0, pre[S].b1);
                store_trcopy<T, D>(sDt[buf], sr, sc, pre[S].b0, pre[S].b1);
            }
            if (ht < 32) {
                // rows past the end get lse = +inf: their P is exactly 0
                const bool ok = q0 + ht < L;
                sL[buf][ht] = ok ? pre_l[S] * kLog2e : __builtin_inff();
                sDel[buf][ht] = ok ? pre_d[S] : 0.0f;
            }
        };
        f32x16 dkacc[D / 32];
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) dkacc[mb][i] = 0.0f;
        // dK'^T += Q'^T dS of a block computed by the main wave of this slice
        auto dk_block = [&](int pbuf, int ptbuf) {
            const u32x4 dsk[2] = {sDS[pbuf][wk][0][l], sDS[pbuf][wk][1][l]};
            // every Q'^T operand first, then the products back to back
            u32x4 qop[2][D / 32];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int mb = 0; mb < D / 32; ++mb) {
                    const T* xt = sQt[ptbuf];
                    const int r = 16 * hh + 8 * s + tr_row;
                    const int e = mb * 32 + tr_col;
                    const i16x4 lo = bwd_tr16(&xt[r * PT + e]);
                    const i16x4 hi = bwd_tr16(&xt[(r + 4) * PT + e]);
                    qop[s][mb] = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int mb = 0; mb < D / 32; ++mb) dkacc[mb] = BMma<T>::run(qop[s][mb], dsk[s], dkacc[mb]);
        };
        // Block loads run two blocks ahead, into two register sets used in turn: block j
        // is stored from its set at iteration j, which then receives block j + 2.
        int ld_hi = 0, ld_q0 = q_last;  // next block to load
        auto load_next = [&](auto slot) {
            const bool ok = ld_q0 >= q_begin;
            load_block(slot, ok ? ld_hi : 0, ok ? ld_q0 : q_begin);  // past the end: a valid dummy, never stored
            const int q = ld_q0;
            if (++ld_hi == a.group) {
                ld_hi = 0;
                ld_q0 -= 32;
            }
            return q;
        };
        int cq0 = load_next(std::integral_constant<int, 0>{});  // block j
        int nq0 = load_next(std::integral_constant<int, 1>{});  // block j + 1 (below q_begin: none)
        int buf = 0, tbuf = 0;
        bool prev = false;  // the previous block ran on this slice: its dK product is due
        int pbuf = 0, ptbuf = 0;
        auto iter = [&](auto slot) {
            const int q0 = cq0;
            store_block(slot, buf, tbuf, q0);
            __syncthreads();  // block visible; the previous block's dS is in LDS
            cq0 = nq0;
            nq0 = load_next(slot);
            if (prev) dk_block(pbuf, ptbuf);
            prev = runs(q0);
            pbuf = buf;
            ptbuf = tbuf;
            buf ^= 1;
            tbuf = tbuf == 2 ? 0 : tbuf + 1;
            return cq0 >= q_begin;
        };
        for (;;) {
            if (!iter(std::integral_constant<int, 0>{})) break;
            if (!iter(std::integral_constant<int, 1>{})) break;
        }
        __syncthreads();  // the last block's dS is in LDS
        if (prev) dk_block(pbuf, ptbuf);
        if (active && kw0 + n < L) {
            const int kr = kw0 + n;
            T* dkp = reinterpret_cast<T*>(a.dk) + sq.bdk + (int64_t)kr * a.dks[1] + (int64_t)kvh * a.dks[2];
            store_grad_row<T, D, PAIR>(dkacc, a.scale, hh, Cg + (int64_t)kr * D, Sg + (int64_t)kr * D, dkp);
        }
    }
}

// ============================================================================ dq
// NW waves of 32 query rows each; key tiles of KT (32 or 64) keys.
template <typename T, int D, int PAIR, int NW, int KT>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_kernel(BwdArgs a) {
    constexpr int NS = D / 16;
    constexpr int HALF = D / 2;
    constexpr int CPR = D / 16;
    constexpr int NT = NW * 64;
    constexpr int KITEMS = KT * CPR;  // staging items of a key tile
    constexpr int NKI = (KITEMS + NT - 1) / NT;
    constexpr int NB = KT / 32;       // 32-key blocks per tile
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr int PA = BwdLds<D>::PA, PT = BwdLds<D>::PT;
    __shared__ __attribute__((aligned(16))) T sKa[2][KT * PA];
    __shared__ __attribute__((aligned(16))) T sKt[2][KT * PT];
    __shared__ __attribute__((aligned(16))) T sVa[2][KT * PA];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar branches)
    const int l = tid & 63, n = l & 31, hh = l >> 5;
    // group = (sequence, kv head); within it: query tiles longest first, the q heads of the
    // kv head next to each other (they read the same K/V tiles in the same order)
    int grp, item;
    xcd_grouped<4>(blockIdx.x, a.q_tiles * a.group, a.hkv * a.batch, grp, item);
    const int kvh = grp % a.hkv;
    const int b = grp / a.hkv;
    const int qt = a.q_tiles - 1 - item / a.group;
    const int h = kvh * a.group + item % a.group;
    const BwdSeq sq = bwd_seq(a, b);
    const int L = sq.L;
    const int q0 = qt * (32 * NW);
    if (q0 >= L) return;  // whole workgroup
    const int qw0 = q0 + 32 * w;
    const bool active = qw0 < L;
    const int qi = qw0 + n;
    const int qrow = min(qi, L - 1);

    const T* Cg = reinterpret_cast<const T*>(a.cos) + sq.tab * D;
    const T* Sg = reinterpret_cast<const T*>(a.sin) + sq.tab * D;
    const T* Kr = reinterpret_cast<const T*>(a.krot) + ((int64_t)kvh * a.rows + sq.tok) * D;  // k' rows
    const T* Vg = reinterpret_cast<const T*>(a.v) + sq.bv + (int64_t)kvh * a.vs[2];

    // ---- staging: NKI items per thread of each key tile; rows past the end re-read the
    // last row (finite, masked below)
    StageItem pre[2][NKI];  // two register sets: tile loads run two tiles ahead
    auto load_tile = [&](auto slot, int k0) {
        constexpr int S = decltype(slot)::value;
#pragma unroll
        for (int j = 0; j < NKI; ++j) {
            const int it = (tid + j * NT) % KITEMS;  // spare threads load a duplicate, never stored
            const int r = it / CPR, c = (it % CPR) * 8;
            const int kr = min(k0 + r, L - 1);
            stage_load<T>(pre[S][j], Kr + (int64_t)kr * D, Vg + (int64_t)kr * a.vs[1], c, HALF);
        }
    };
    auto store_tile = [&](auto slot, int buf) {
        constexpr int S = decltype(slot)::value;
#pragma unroll
        for (int j = 0; j < NKI; ++j) {
            const int it = tid + j * NT;
            if (KITEMS % NT == 0 || it < KITEMS) {
                const int r = it / CPR, c = (it % CPR) * 8;
                store_rowcopy<T, D>(sKa[buf], r, c, pre[S][j].a0, pre[S][j].a1);
                store_trcopy<T, D>(sKt[buf], r, c, pre[S][j].a0, pre[S][j].a1);
                store_rowcopy<T, D>(sVa[buf], r, c, pre[S][j].b0, pre[S][j].b1);
            }
        }
    };

    // ---- this lane's query row: rotated Q' and dO as B operands (column n = query, k = d)
    u32x4 qb[NS], db[NS];
    {
        const T* qp = reinterpret_cast<const T*>(a.qrot) + ((int64_t)h * a.rows + sq.tok + qrow) * D;
        const T* dp = reinterpret_cast<const T*>(a.dout) + sq.bdo + (int64_t)qrow * a.dos[1] + (int64_t)h * a.dos[2];
#pragma unroll
        for (int s = 0; s < NS; ++s) qb[s] = load_chunk<T>(qp + 16 * s + 8 * hh).w;
#pragma unroll
        for (int s = 0; s < NS; ++s) db[s] = load_chunk<T>(dp + 16 * s + 8 * hh).w;
    }
    const float lse2 = a.lse[(int64_t)h * a.lse_stride + sq.tok + qrow] * kLog2e;
    const float del = a.delta[(int64_t)h * a.lse_stride + sq.tok + qrow];
    // complete these loads here: otherwise the loop's first use would wait for every load
    // issued after them, the prefetch included
#pragma unroll
    for (int s = 0; s < NS; ++s) asm volatile("" ::"v"(db[s]));
    asm volatile("" ::"v"(del));

    f32x16 dqacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) dqacc[mb][i] = 0.0f;
    const int tr_row = (l & 15) >> 2;
    const int tr_col = ((l >> 4) & 1) * 16 + 4 * (l & 3);
    const int q_hi = min(q0 + 32 * NW, L);
    const int kend = a.causal ? q_hi : L;
    const int n_kt = (kend + KT - 1) / KT;
    const int wave_kend = a.causal ? min(qw0 + 32, L) : L;

    // key kk of this lane's row is kept iff kk <= kmax
    const int kmax = a.causal ? min(qi, L - 1) : L - 1;

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    load_tile(S0{}, 0);
    load_tile(S1{}, min(KT, (n_kt - 1) * KT));
    auto iter = [&](auto slot, int kt) {
        const int k0 = kt * KT;
        const int buf = kt & 1;
        store_tile(slot, buf);
        __syncthreads();  // tile visible; every read of this buffer two tiles back is done
        // near the end this reloads the last tile (never stored): no branch around the loads
        load_tile(slot, min(k0 + 2 * KT, (n_kt - 1) * KT));
        if (!active || k0 >= wave_kend) return;  // wave-uniform
        const T* ka = sKa[buf];
        const T* ktr = sKt[buf];
        const T* va = sVa[buf];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            // ---- S^T and dP^T: lane (n, hh) gets query qi against keys k0 + 32*blk + 16hh + i
            const int rr = blk * 32 + n;  // pi order: MFMA row n holds key k0 + 32*blk + pi(n)
            f32x16 sacc, dpacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[i] = dpacc[i] = 0.0f;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int off = rr * PA + 16 * s + 8 * hh;
                sacc = BMma<T>::run(*reinterpret_cast<const u32x4*>(&ka[off]), qb[s], sacc);
                dpacc = BMma<T>::run(*reinterpret_cast<const u32x4*>(&va[off]), db[s], dpacc);
            }
            // the K'^T operands of the first dQ' products, read now so that their LDS round trips
            // run under the exponentials below (all of them: the registers spill)
            auto rd_kt = [&](int mb, int s) {
                const int r = blk * 32 + 16 * hh + 8 * s + tr_row;
                const int e = mb * 32 + tr_col;
                const i16x4 lo = bwd_tr16(&ktr[r * PT + e]);
                const i16x4 hi = bwd_tr16(&ktr[(r + 4) * PT + e]);
                return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            };
            u32x4 kto[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) kto[s] = rd_kt(0, s);
            const int thr = kmax - (k0 + 32 * blk + 16 * hh);  // key ... + i is masked iff i > thr
            u32x4 dsk[2];
            auto probs = [&](auto masked) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    float ds[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int i = 8 * s + j;
                        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], a.scale_log2, -lse2));
                        if (decltype(masked)::value && i > thr) pv = 0.0f;
                        ds[j] = pv * (dpacc[i] - del);
                    }
                    dsk[s] = pack<T>(ds).w;
                }
            };
            // wave-uniform: the block's last key against the wave's smallest kept bound
            if (k0 + 32 * blk + 31 > (a.causal ? min(qw0, L - 1) : L - 1))
                probs(std::true_type{});
            else
                probs(std::false_type{});
            // ---- dQ'^T += K'^T dS^T
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
                for (int s = 0; s < 2; ++s) dqacc[mb] = BMma<T>::run(mb == 0 ? kto[s] : rd_kt(mb, s), dsk[s], dqacc[mb]);
        }
    };
    for (int kt = 0; kt < n_kt; kt += 2) {
        iter(S0{}, kt);
        if (kt + 1 < n_kt) iter(S1{}, kt + 1);
    }

    // ---- epilogue: dq = M^T (s * dQ')
    if (active && qi < L) {
        T* dqp = reinterpret_cast<T*>(a.dq) + sq.bdq + (int64_t)qi * a.dqs[1] + (int64_t)h * a.dqs[2];
        store_grad_row<T, D, PAIR>(dqacc, a.scale, hh, Cg + (int64_t)qi * D, Sg + (int64_t)qi * D, dqp);
    }
}

// ============================================================================ launch
#ifndef BWD_DQ_NW
#define BWD_DQ_NW 8
#endif
#ifndef BWD_DQ_KT
#define BWD_DQ_KT 64
#endif
template <typename T, int D, int PAIR>
static void launch_bwd_typed(const BwdArgs& a, int maxlen, hipStream_t stream) {
    constexpr int NW = BWD_DQ_NW, KT = BWD_DQ_KT;
    const int64_t pthreads = (int64_t)a.rows * (a.hq + a.hkv) * (D / 16);
    hipLaunchKernelGGL((bwd_prep_kernel<T, D, PAIR>), dim3((unsigned)((pthreads + 255) / 256)), dim3(256), 0, stream, a);
    BwdArgs g = a;
    g.kv_tiles = (maxlen + 127) / 128;
    g.q_tiles = (maxlen + 32 * NW - 1) / (32 * NW);
    hipLaunchKernelGGL((bwd_dkv_kernel<T, D, PAIR>), dim3((unsigned)(g.kv_tiles * a.hkv * a.batch)), dim3(512), 0,
                       stream, g);
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, PAIR, NW, KT>), dim3((unsigned)(g.q_tiles * a.hq * a.batch)), dim3(NW * 64),
                       0, stream, g);
}

template <typename T, int D>
static void launch_bwd_pair(const BwdArgs& a, int pair, int maxlen, hipStream_t stream) {
    switch (pair) {
        case 0: launch_bwd_typed<T, D, 0>(a, maxlen, stream); break;
        case 1: launch_bwd_typed<T, D, 1>(a, maxlen, stream); break;
        default: launch_bwd_typed<T, D, 2>(a, maxlen, stream); break;
    }
}

// Workspace: delta [hq, rows] float32, then q' [hq, rows, D] and k' [hkv, rows, D] of the
// input dtype, each region starting on a 256-byte boundary.
struct BwdWorkspace {
    uint64_t delta, qrot, krot, total;  // byte offsets and size
};
static BwdWorkspace bwd_workspace(const rope_attn_params* f) {
    const uint64_t rows = f->cu_seqlens ? (uint64_t)f->ntokens : (uint64_t)f->batch * (uint64_t)f->seqlen;
    const uint64_t e = (uint64_t)dtype_bytes(f->dtype);
    auto up = [](uint64_t x) { return (x + 255u) & ~(uint64_t)255u; };
    BwdWorkspace w;
    w.delta = 0;
    w.qrot = up(rows * (uint64_t)f->hq * 4u);
    w.krot = w.qrot + up(rows * (uint64_t)f->hq * (uint64_t)f->head_dim * e);
    w.total = w.krot + up(rows * (uint64_t)f->hkv * (uint64_t)f->head_dim * e);
    return w;
}

uint64_t flash_bwd_workspace_bytes(const rope_attn_params* f) { return bwd_workspace(f).total; }

hipError_t launch_flash_bwd(const rope_attn_bwd_params* p, hipStream_t stream) {
    const rope_attn_params* f = &p->fwd;
    BwdArgs a;
    a.q = f->q;
    a.k = f->k;
    a.v = f->v;
    a.o = f->out;
    a.dout = p->dout;
    a.lse = f->lse;
    a.cos = f->cos;
    a.sin = f->sin;
    a.dq = p->dq;
    a.dk = p->dk;
    a.dv = p->dv;
    const BwdWorkspace ws = bwd_workspace(f);
    char* wsp = reinterpret_cast<char*>(p->workspace);
    a.delta = reinterpret_cast<float*>(wsp + ws.delta);
    a.qrot = wsp + ws.qrot;
    a.krot = wsp + ws.krot;
    a.cu_seqlens = f->cu_seqlens;
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = f->q_stride[i];
        a.ks[i] = f->k_stride[i];
        a.vs[i] = f->v_stride[i];
        a.os[i] = f->o_stride[i];
        a.dos[i] = p->do_stride[i];
        a.dqs[i] = p->dq_stride[i];
        a.dks[i] = p->dk_stride[i];
        a.dvs[i] = p->dv_stride[i];
    }
    const bool varlen = f->cu_seqlens != nullptr;
    a.batch = f->batch;
    a.hq = f->hq;
    a.hkv = f->hkv;
    a.group = f->hq / f->hkv;
    a.seqlen = varlen ? 0 : f->seqlen;
    a.table_seq_rows = f->table_seq_rows;
    a.rows = varlen ? f->ntokens : f->batch * f->seqlen;
    a.max_seqlen = varlen ? f->max_seqlen : f->seqlen;
    a.lse_stride = a.rows;
    a.causal = f->causal;
    a.scale = f->softmax_scale;
    a.scale_log2 = f->softmax_scale * 1.4426950408889634f;
    const int pair = f->cos ? (f->pairing == ROPE_PAIR_INTERLEAVED ? 2 : 1) : 0;
    const int maxlen = varlen ? f->max_seqlen : f->seqlen;
    const int key = (f->dtype == ROPE_DT_BF16 ? 0 : 2) + (f->head_dim == 128 ? 1 : 0);
    switch (key) {
        case 0: launch_bwd_pair<__bf16, 64>(a, pair, maxlen, stream); break;
        case 1: launch_bwd_pair<__bf16, 128>(a, pair, maxlen, stream); break;
        case 2: launch_bwd_pair<_Float16, 64>(a, pair, maxlen, stream); break;
        default: launch_bwd_pair<_Float16, 128>(a, pair, maxlen, stream); break;
    }
    return hipGetLastError();
}

}  // namespace ropefa

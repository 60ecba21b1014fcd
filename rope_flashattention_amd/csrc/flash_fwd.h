// rope_flash_attn_fwd: RoPE fused into a FlashAttention forward pass on gfx950.
//
// What is computed ([RoPE-fusion blog], section 三; [FlashAttention blog], tiling and
// online softmax): for each (sequence, q head, query row) the rotate-half RoPE of q and
// of every key, the scaled scores, a softmax over the causal keys of the sequence and
// the weighted sum of V.  Rotated Q/K exist only in registers and LDS.
//
// bf16/fp16 kernel (flash_fwd16_kernel).  A workgroup is 8 waves (512 threads, one per
// CU).  Each wave owns 32 query rows of one q head; a workgroup holds HP q heads of the
// same kv head (GQA packing) times (8/HP)*32 queries, so every staged K/V tile serves 256
// (head, query) rows and its RoPE is paid once for all of them.  The grid is (head groups,
// query tiles, sequences); query tiles are issued longest-first for causal balance.
//
// Per key tile of 64 keys (LDS double-buffered, one barrier per tile):
//   * S^T = K' Q'^T with 32x32x16 MFMA: A = K' rows from LDS (read four products ahead),
//     B = Q' held in registers since the start (rotated and multiplied by
//     softmax_scale*log2(e) once).  A lane therefore holds 16 scores of one query row and
//     the row statistics need a single exchange between the two halves of the wave
//     (v_permlane32_swap).
//   * Online softmax in the log2 domain with a lazily updated reference m: the MFMA
//     accumulator starts at -m (kept in registers), so S - m comes out of the matrix core
//     and P = exp2(S - m) needs no subtraction and no row max.  The reference (and the O, l
//     rescale by exp2(m_old - m_new)) moves only on the first tile or when a row sum of
//     the tile exceeds 2^16, i.e. when some score has outgrown the reference; then the
//     tile's row max is taken and P recomputed.  P stays below 2^16 otherwise, far inside
//     the float32/bf16 range.  Row sums add the float32 exponentials.
//   * O^T += V^T P^T with the same MFMA: P is already in the B-operand layout, and the
//     V^T operand comes from row-major V in LDS through the transposing LDS read
//     (ds_read_b64_tr_b16).
//   * Meanwhile the next tile, loaded into registers one tile ahead, is rotated (K) and
//     written to the other LDS buffer; the loads for the tile after it are issued.  At
//     head_dim 128 the rotation is cut into 16 slices, one after each P.V MFMA (the four O
//     blocks in turn, operands read three steps ahead), so the vector work issues while
//     the matrix core runs; with tables formed in the kernel the sine and cosine of the
//     staged tile's columns are likewise computed in pieces between the score MFMAs.  No
//     v_dot2 anywhere: on gfx950 those run in the matrix-core pipeline and would serialise
//     with the MFMAs.
// K rotated once per key instead (modes kRotQ*): every workgroup of a kv head stages each
// key tile it needs, so in-loop rotation repeats the rotation of a key once per query tile
// and head group that reaches it (about 256 times on a causal 16384-token GQA sequence
// with 8 q heads per kv head).  Where that repetition costs more than one pass over K, the
// host runs a pre-pass that writes k' (the same arithmetic and rounding as the in-loop
// rotation, so the results are bit-identical) and launches these modes, which rotate only
// Q in registers and stage k' tiles as they are.
// Permuted K' rows: MFMA result row m of S^T is key pi(m) = 16*((m>>2)&1) + 4*(m>>3) + (m&3)
// inside a 32-key block, which makes the 16 scores of lane half h the contiguous keys
// 16h .. 16h+15; K' for key pi(m) is stored at LDS row m so the MFMA reads consecutive rows.
//
// float32 kernel (flash_fwd32_kernel): 4 waves, the 32x32x2 float32 MFMA, a single LDS
// buffer and the straightforward online softmax; it serves the small float32 workload.
#pragma once

#include "common.h"

namespace ropefa {

struct FaArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const void* cos;
    const void* sin;
    const int32_t* pos;         // tables formed in the kernel: positions (table-row indexed)
    const float* inv_freq;      // and inverse frequencies [inv_freq_rows, D/2]
    const int32_t* cu_seqlens;  // nullptr: dense
    int64_t qs[3], ks[3], vs[3], os[3];  // {batch, token, head} strides in elements
    int32_t seqlen;                      // dense sequence length
    int32_t ntokens, max_seqlen;         // varlen: packed rows in total and the host bound of every length
    int32_t group;                       // hq / hkv
    int32_t table_seq_rows;
    int32_t lse_stride;                  // tokens per lse row
    int32_t causal;
    float scale_log2;                    // softmax_scale * log2(e)
    float pos_scale;
    int32_t inv_freq_rows;
};

// Rotation modes of the kernels (template parameter ROT).
enum RotMode : int {
    kRotNone = 0,         // plain attention
    kRotHalfTable = 1,    // rotate-half pairs, tables read (columns [0, D/2) only)
    kRotInterTable = 2,   // interleaved pairs, tables read (all columns)
    kRotHalfGen = 3,      // rotate-half pairs, table values formed in the kernel
    kRotInterGen = 4,     // interleaved pairs, table values formed in the kernel
    // Q rotated in the kernel as by mode m - 4; K read already rotated (a pre-pass wrote k'
    // once per key, instead of every workgroup rotating each tile it stages)
    kRotQHalfTable = 5,
    kRotQInterTable = 6,
    kRotQHalfGen = 7,
    kRotQInterGen = 8
};
constexpr bool rot_inter(int rot) { return rot == kRotInterTable || rot == kRotInterGen; }
constexpr bool rot_gen(int rot) { return rot == kRotHalfGen || rot == kRotInterGen; }
constexpr int q_rot(int rot) { return rot >= kRotQHalfTable ? rot - 4 : rot; }  // rotation of Q
constexpr int k_rot(int rot) { return rot >= kRotQHalfTable ? kRotNone : rot; } // of staged K tiles

// Table values formed in the kernel, rounded to T as a stored table would be:
// cos/sin of frequencies f[0..7] at position p, packed.
template <typename T>
__device__ __forceinline__ void gen_table_chunk(int32_t p, float pos_scale, const float (&f)[8], u32x4& cc,
                                                u32x4& ss) {
    float sv[8], cv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rope_sincos(table_angle(p, pos_scale, f[e]), sv[e], cv[e]);
    cc = pack<T>(cv).w;
    ss = pack<T>(sv).w;
}
// The interleaved layout of frequencies f[0..3] (each value in two adjacent columns).
template <typename T>
__device__ __forceinline__ void gen_table_chunk_inter(int32_t p, float pos_scale, const float* f, u32x4& cc,
                                                      u32x4& ss) {
    float sv[8], cv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        rope_sincos(table_angle(p, pos_scale, f[e]), sv[2 * e], cv[2 * e]);
        sv[2 * e + 1] = sv[2 * e];
        cv[2 * e + 1] = cv[2 * e];
    }
    cc = pack<T>(cv).w;
    ss = pack<T>(sv).w;
}

template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
    typedef bf16x8 vec;
    __device__ static __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<_Float16> {
    typedef f16x8 vec;
    __device__ static __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// x combined with its value in the lane 32 apart (the other half of the wave).
__device__ __forceinline__ float halves_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// LDS row (inside a 64-key tile) that holds key kappa: inverse of pi within each 32-key block.
__device__ __forceinline__ int kprime_row(int kappa) {
    const int blk = kappa >> 5, kl = kappa & 31;
    return blk * 32 + 8 * ((kl >> 2) & 3) + 4 * (kl >> 4) + (kl & 3);
}

constexpr int kBN = 64;  // keys per tile

// Sequence bounds and per-workgroup offsets shared by both kernels.
struct SeqView {
    int seq_start, L;
    int64_t qbase, kbase, vbase, obase, tbase;
    bool varlen;
};
__device__ __forceinline__ SeqView seq_view(const FaArgs& a, int b) {
    SeqView sv;
    sv.varlen = a.cu_seqlens != nullptr;
    sv.seq_start = 0;
    sv.L = a.seqlen;
    if (sv.varlen) {
        // device-held lengths are clamped so that every row stays inside the packed rows
        // and inside the grid (which covers max_seqlen rows per sequence)
        const int64_t s0 = min(max((int64_t)a.cu_seqlens[b], (int64_t)0), (int64_t)a.ntokens);
        const int64_t len = (int64_t)a.cu_seqlens[b + 1] - s0;
        sv.seq_start = (int)s0;
        sv.L = (int)max((int64_t)0, min(len, min((int64_t)a.max_seqlen, (int64_t)a.ntokens - s0)));
    }
    sv.qbase = sv.varlen ? (int64_t)sv.seq_start * a.qs[1] : (int64_t)b * a.qs[0];
    sv.kbase = sv.varlen ? (int64_t)sv.seq_start * a.ks[1] : (int64_t)b * a.ks[0];
    sv.vbase = sv.varlen ? (int64_t)sv.seq_start * a.vs[1] : (int64_t)b * a.vs[0];
    sv.obase = sv.varlen ? (int64_t)sv.seq_start * a.os[1] : (int64_t)b * a.os[0];
    sv.tbase = sv.varlen ? (int64_t)sv.seq_start : (a.table_seq_rows ? (int64_t)b * a.table_seq_rows : 0);
    return sv;
}

// ============================================================================ bf16 / fp16
template <typename T, int D, int HP, int ROT>
__global__ __launch_bounds__(512, 1) void flash_fwd16_kernel(FaArgs a) {
    constexpr int NW = 8, NT = NW * 64;
    constexpr int QT = (NW / HP) * 32;            // queries per workgroup
    constexpr int KP = D + 24;                    // K' LDS row pitch (elements)
    constexpr int VP = D + 32;                    // V LDS row pitch: rows 16 dwords apart mod 64 banks
    constexpr int HALF = D / 2;
    constexpr int KCH = HALF / 8;                 // 8-element chunks per half row
    constexpr int KITEMS = kBN * KCH;             // (key, chunk pair) items per tile
    constexpr int VITEMS = kBN * (D / 8);         // 8-element V chunks per tile
    constexpr int NKI = (KITEMS + NT - 1) / NT;
    constexpr int NVI = (VITEMS + NT - 1) / NT;
    constexpr float kLazySum = 65536.0f;          // tile row sum that forces the reference to move
    constexpr int QROT = q_rot(ROT), KROT = k_rot(ROT);
    // formed tables at head_dim 128: the staged tile's sin/cos are computed between the score
    // MFMAs and its rotation between the P.V MFMAs
    constexpr bool kGenSliced = rot_gen(KROT) && NKI == 1 && KITEMS == NT && D == 128;
    typedef typename Mfma<T>::vec vec;

    __shared__ __attribute__((aligned(16))) T sK[2][kBN * KP];
    __shared__ __attribute__((aligned(16))) T sV[2][kBN * VP];

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, r = l & 31, h = l >> 5;
    const int qt = gridDim.y - 1 - blockIdx.y;  // longest query tiles first
    const int b = blockIdx.z;
    const SeqView sv = seq_view(a, b);
    const int L = sv.L;
    if (qt * QT >= L) return;  // whole workgroup: this sequence is shorter

    const int head = blockIdx.x * HP + (w % HP);
    const int kvh = (blockIdx.x * HP) / a.group;
    const int q0 = qt * QT + (w / HP) * 32;  // first query row of this wave
    const int qi = q0 + r;                     // this lane's query row

    const T* Kg = reinterpret_cast<const T*>(a.k) + sv.kbase + (int64_t)kvh * a.ks[2];
    const T* Vg = reinterpret_cast<const T*>(a.v) + sv.vbase + (int64_t)kvh * a.vs[2];
    const T* Cg = reinterpret_cast<const T*>(a.cos) + sv.tbase * D;
    const T* Sg = reinterpret_cast<const T*>(a.sin) + sv.tbase * D;
    const int32_t* Pg = a.pos + sv.tbase;
    const float* Fg = a.inv_freq + (a.inv_freq_rows > 1 ? (int64_t)b * HALF : 0);

    // ------------------------------------------------------------ tile staging
    const int q_hi = min(qt * QT + QT, L);
    const int kend = a.causal ? q_hi : L;
    const int n_kt = (kend + kBN - 1) / kBN;
    const int wave_kend = a.causal ? min(q0 + 32, L) : L;
    const int kmax = a.causal ? min(qi, L - 1) : L - 1;  // this lane's last key

    u32x4 kx[NKI], ky[NKI], kc[NKI], ks[NKI], kc2[NKI], ks2[NKI], vr[NVI];
    int32_t kpos[NKI];
    float kf[NKI][8];  // formed tables: this thread's frequencies (fixed per item slot)
    if constexpr (rot_gen(KROT)) {
#pragma unroll
        for (int j = 0; j < NKI; ++j) {
            const int it = tid + j * NT;
            const int c = (it % KCH) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                kf[j][e] = KROT == kRotHalfGen ? Fg[c + e] : Fg[(e < 4 ? c : c + HALF) / 2 + (e & 3)];
        }
    }
    // Byte offsets of this thread's staged chunks within a full tile (32-bit, non-negative),
    // so that each load is a uniform tile base plus one per-lane register offset.
    uint32_t kob[NKI], tob[NKI], vob[NVI];
#pragma unroll
    for (int j = 0; j < NKI; ++j) {
        const int it = tid + j * NT;
        const int kap = it / KCH, c = (it % KCH) * 8;
        kob[j] = (uint32_t)(kap * a.ks[1] + c) * (uint32_t)sizeof(T);
        tob[j] = (uint32_t)(kap * D + c) * (uint32_t)sizeof(T);
    }
#pragma unroll
    for (int j = 0; j < NVI; ++j) {
        const int it = tid + j * NT;
        vob[j] = (uint32_t)((it / (D / 8)) * a.vs[1] + (it % (D / 8)) * 8) * (uint32_t)sizeof(T);
    }
    auto stage_load = [&](int kt) {
        const int k0 = kt * kBN;
        const bool full = k0 + kBN <= L;
        const char* kg = reinterpret_cast<const char*>(Kg + (int64_t)k0 * a.ks[1]);
        const char* vg = reinterpret_cast<const char*>(Vg + (int64_t)k0 * a.vs[1]);
        const char* cg = reinterpret_cast<const char*>(Cg + (int64_t)k0 * D);
        const char* sg = reinterpret_cast<const char*>(Sg + (int64_t)k0 * D);
        // rows past the end of the sequence re-read its last row: finite data whose scores
        // the mask removes (their P is exactly 0), so no zero fill is needed
#pragma unroll
        for (int j = 0; j < NKI; ++j) {
            const int it = tid + j * NT;
            if (KITEMS % NT == 0 || it < KITEMS) {
                const int kap = full ? it / KCH : min(it / KCH, L - 1 - k0), c = (it % KCH) * 8;
                const uint32_t ko = full ? kob[j] : (uint32_t)(kap * a.ks[1] + c) * (uint32_t)sizeof(T);
                const uint32_t to = full ? tob[j] : (uint32_t)(kap * D + c) * (uint32_t)sizeof(T);
                kx[j] = *reinterpret_cast<const u32x4*>(kg + ko);
                ky[j] = *reinterpret_cast<const u32x4*>(kg + ko + HALF * sizeof(T));
                if constexpr (KROT == kRotHalfTable || KROT == kRotInterTable) {
                    kc[j] = *reinterpret_cast<const u32x4*>(cg + to);
                    ks[j] = *reinterpret_cast<const u32x4*>(sg + to);
                }
                if constexpr (KROT == kRotInterTable) {
                    kc2[j] = *reinterpret_cast<const u32x4*>(cg + to + HALF * sizeof(T));
                    ks2[j] = *reinterpret_cast<const u32x4*>(sg + to + HALF * sizeof(T));
                }
                if constexpr (rot_gen(KROT)) kpos[j] = Pg[k0 + kap];
            }
        }
#pragma unroll
        for (int j = 0; j < NVI; ++j) {
            const int it = tid + j * NT;
            if (VITEMS % NT == 0 || it < VITEMS) {
                const int kap = full ? it / (D / 8) : min(it / (D / 8), L - 1 - k0), c = (it % (D / 8)) * 8;
                const uint32_t vo = full ? vob[j] : (uint32_t)(kap * a.vs[1] + c) * (uint32_t)sizeof(T);
                vr[j] = *reinterpret_cast<const u32x4*>(vg + vo);
            }
        }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < NKI; ++j) {
            const int it = tid + j * NT;
            if (KITEMS % NT == 0 || it < KITEMS) {
                const int kap = it / KCH, c = (it % KCH) * 8;
                T* dst = &sK[buf][kprime_row(kap) * KP + c];
                if constexpr (KROT == kRotHalfTable) {
                    u32x4 xo, yo;
                    rotate_pair_packed<T>(kx[j], ky[j], kc[j], ks[j], xo, yo);
                    *reinterpret_cast<u32x4*>(dst) = xo;
                    *reinterpret_cast<u32x4*>(dst + HALF) = yo;
                } else if constexpr (KROT == kRotInterTable) {
                    *reinterpret_cast<u32x4*>(dst) = rotate_interleaved_packed<T>(kx[j], kc[j], ks[j]);
                    *reinterpret_cast<u32x4*>(dst + HALF) = rotate_interleaved_packed<T>(ky[j], kc2[j], ks2[j]);
                } else if constexpr (KROT == kRotHalfGen) {
                    u32x4 cc, ss, xo, yo;
                    gen_table_chunk<T>(kpos[j], a.pos_scale, kf[j], cc, ss);
                    rotate_pair_packed<T>(kx[j], ky[j], cc, ss, xo, yo);
                    *reinterpret_cast<u32x4*>(dst) = xo;
                    *reinterpret_cast<u32x4*>(dst + HALF) = yo;
                } else if constexpr (KROT == kRotInterGen) {
                    u32x4 cc, ss;
                    gen_table_chunk_inter<T>(kpos[j], a.pos_scale, &kf[j][0], cc, ss);
                    *reinterpret_cast<u32x4*>(dst) = rotate_interleaved_packed<T>(kx[j], cc, ss);
                    gen_table_chunk_inter<T>(kpos[j], a.pos_scale, &kf[j][4], cc, ss);
                    *reinterpret_cast<u32x4*>(dst + HALF) = rotate_interleaved_packed<T>(ky[j], cc, ss);
                } else {
                    *reinterpret_cast<u32x4*>(dst) = kx[j];
                    *reinterpret_cast<u32x4*>(dst + HALF) = ky[j];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NVI; ++j) {
            const int it = tid + j * NT;
            if (VITEMS % NT == 0 || it < VITEMS) {
                const int kap = it / (D / 8), c = (it % (D / 8)) * 8;
                *reinterpret_cast<u32x4*>(&sV[buf][kap * VP + c]) = vr[j];
            }
        }
    };

    // ------------------------------------------------------------ Q' in registers
    // lane holds Q'[qi][16u + 8h + e], u < D/16, e < 8 (the MFMA B-operand layout);
    // chunk u < D/32 and chunk u + D/32 of the same lane are columns d and d + D/2.
    // The raw rows (and their table values) are loaded first, then the first key tile's
    // loads are issued, and only then is Q rotated: the two memory round trips overlap.
    // Rows past the end load the last row (finite) and are zeroed after the rotation.
    constexpr int QU = D / 32;
    const int qrow = min(qi, L - 1);
    u32x4 qxr[QU], qyr[QU], qcr[QU], qsr[QU], qc2r[QU], qs2r[QU];
    float qf[QU][8];
    int32_t qpos = 0;
    {
        const T* qp = reinterpret_cast<const T*>(a.q) + sv.qbase + (int64_t)qrow * a.qs[1] + (int64_t)head * a.qs[2];
        if constexpr (rot_gen(QROT)) qpos = Pg[qrow];
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            const int d = 16 * u + 8 * h;
            qxr[u] = load_chunk<T>(qp + d).w;
            qyr[u] = load_chunk<T>(qp + d + HALF).w;
            if constexpr (QROT == kRotHalfTable || QROT == kRotInterTable) {
                qcr[u] = load_chunk<T>(Cg + (int64_t)qrow * D + d).w;
                qsr[u] = load_chunk<T>(Sg + (int64_t)qrow * D + d).w;
            }
            if constexpr (QROT == kRotInterTable) {
                qc2r[u] = load_chunk<T>(Cg + (int64_t)qrow * D + d + HALF).w;
                qs2r[u] = load_chunk<T>(Sg + (int64_t)qrow * D + d + HALF).w;
            }
            if constexpr (QROT == kRotHalfGen) {
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[u][e] = Fg[d + e];
            }
            if constexpr (QROT == kRotInterGen) {
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[u][e] = Fg[(e < 4 ? d : d + HALF) / 2 + (e & 3)];
            }
        }
    }
    vec qreg[D / 16];
    auto rotate_q = [&]() {
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            float x[8], y[8];
            unpack<T>(Chunk8<T>{qxr[u]}, x);
            unpack<T>(Chunk8<T>{qyr[u]}, y);
            if constexpr (QROT == kRotHalfTable) {
                float c[8], s[8];
                unpack<T>(Chunk8<T>{qcr[u]}, c);
                unpack<T>(Chunk8<T>{qsr[u]}, s);
                rotate_pair(x, y, c, s, c, s);
            } else if constexpr (QROT == kRotInterTable) {
                float c0[8], s0[8], c1[8], s1[8];
                unpack<T>(Chunk8<T>{qcr[u]}, c0);
                unpack<T>(Chunk8<T>{qsr[u]}, s0);
                unpack<T>(Chunk8<T>{qc2r[u]}, c1);
                unpack<T>(Chunk8<T>{qs2r[u]}, s1);
                rotate_interleaved(x, c0, s0);
                rotate_interleaved(y, c1, s1);
            } else if constexpr (QROT == kRotHalfGen) {
                float c[8], s[8];
                u32x4 cc, ss;
                gen_table_chunk<T>(qpos, a.pos_scale, qf[u], cc, ss);
                unpack<T>(Chunk8<T>{cc}, c);
                unpack<T>(Chunk8<T>{ss}, s);
                rotate_pair(x, y, c, s, c, s);
            } else if constexpr (QROT == kRotInterGen) {
                float c0[8], s0[8], c1[8], s1[8];
                u32x4 cc, ss;
                gen_table_chunk_inter<T>(qpos, a.pos_scale, &qf[u][0], cc, ss);
                unpack<T>(Chunk8<T>{cc}, c0);
                unpack<T>(Chunk8<T>{ss}, s0);
                gen_table_chunk_inter<T>(qpos, a.pos_scale, &qf[u][4], cc, ss);
                unpack<T>(Chunk8<T>{cc}, c1);
                unpack<T>(Chunk8<T>{ss}, s1);
                rotate_interleaved(x, c0, s0);
                rotate_interleaved(y, c1, s1);
            }
            const float sc = qi < L ? a.scale_log2 : 0.0f;  // rows past the end: zero
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[e] *= sc;
                y[e] *= sc;
            }
            qreg[u] = __builtin_bit_cast(vec, pack<T>(x).w);
            qreg[u + D / 32] = __builtin_bit_cast(vec, pack<T>(y).w);
        }
    };

    // ------------------------------------------------------------ main loop
    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 minit = f32x16{};  // -reference, the accumulator start of every score block
    // transposing read: lane l of each 16-lane group supplies row (l%16)/4, columns
    // 4*(l%4)..+3 of a 4x16 tile and receives the tile's column l%16
    const int tr_row = (l & 15) >> 2;
    const int tr_col = ((l >> 4) & 1) * 16 + 4 * (l & 3);

    stage_load(0);
    // q's loads were issued before the first tile's, so the rotation waits for them only and
    // runs while the tile is still in flight (the compiler would otherwise sink it below the
    // barrier, into the critical path before the first MFMA)
    rotate_q();
#pragma unroll
    for (int u = 0; u < D / 16; ++u) asm volatile("" ::"v"(qreg[u]));
    __builtin_amdgcn_sched_barrier(0);
    stage_store(0);
    if (n_kt > 1) stage_load(1);
    __syncthreads();

    for (int kt = 0; kt < n_kt; ++kt) {
        const int buf = kt & 1;
        const int k0 = kt * kBN;
        const bool active = k0 < wave_kend;  // wave-uniform: does this wave need any key here
        vec pk[2][2];
        // formed tables: the staged tile's 8 table columns, each angle's sine half and cosine
        // half one piece after each score MFMA, packed into the table registers in pairs
        float gq = 0.f, gk = 0.f, gr2 = 0.f, gsr = 0.f, gcv[8], gsv[8];
        bool gfar = false;
        auto gen_finish = [&](int e) {
            if constexpr (kGenSliced) {
                rope_sincos_b(gk, gr2, gsr, gsv[e], gcv[e]);
                if constexpr (KROT == kRotHalfGen) {
                    if (e & 1) {
                        kc[0][e >> 1] = Elem<T>::pack(gcv[e - 1], gcv[e]);
                        ks[0][e >> 1] = Elem<T>::pack(gsv[e - 1], gsv[e]);
                        asm volatile("" ::"v"(kc[0][e >> 1]), "v"(ks[0][e >> 1]));
                    } else {
                        asm volatile("" ::"v"(gcv[e]), "v"(gsv[e]));
                    }
                } else {
                    u32x4& tc = e < 4 ? kc[0] : kc2[0];
                    u32x4& ts = e < 4 ? ks[0] : ks2[0];
                    tc[e & 3] = Elem<T>::pack(gcv[e], gcv[e]);
                    ts[e & 3] = Elem<T>::pack(gsv[e], gsv[e]);
                    asm volatile("" ::"v"(tc[e & 3]), "v"(ts[e & 3]));
                }
            }
        };
        auto gen_slice = [&](int j) {
            if constexpr (kGenSliced) {
                // (the empty asm statements keep each piece here: the values are used only
                // under a later branch, into which the compiler would otherwise move them)
                if (j == 0) {
                    gq = __fdiv_rn((float)kpos[0], a.pos_scale);
                    asm volatile("" ::"v"(gq));
                } else if (j & 1) {
                    const int e = (j - 1) >> 1;
                    const float th = __fmul_rn(gq, kf[0][e]);  // the angle table_angle forms
                    gfar |= __builtin_fabsf(th) > kFastPathMax;
                    rope_sincos_a(th, gk, gr2, gsr);
                    asm volatile("" ::"v"(gk), "v"(gr2), "v"(gsr));
                } else {
                    gen_finish((j - 2) >> 1);
                }
            }
        };
        // the first P.V operands are read right after the score MFMAs, so their LDS round
        // trip runs under the softmax
        constexpr int NMBV = D / 32, PDV = 3;
        const T* vpv0 = &sV[buf][(16 * h + tr_row) * VP + tr_col];
        auto rd_v0 = [&](int j) {
            const int kstep = j / NMBV;
            const T* vp = vpv0 + ((kstep >> 1) * 32 + 8 * (kstep & 1)) * VP + (j % NMBV) * 32;
            const i16x4 lo = lds_read_tr16(vp);
            const i16x4 hi = lds_read_tr16(vp + 4 * VP);
            return __builtin_bit_cast(vec, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        vec vpre[PDV];
        if (active) {
            // ---- S^T - m = K' Q'^T - m : lane (r, h) gets keys k0 + 32*blk + 16h + i of query qi
            f32x16 sacc[2];
            {
                // the 2*(D/16) K' operands (block j & 1, column step j >> 1) are read four
                // products ahead, so the MFMAs do not wait on one LDS round trip each
                const T* kp0 = &sK[buf][r * KP + 8 * h];
                auto rd_k = [&](int j) { return *reinterpret_cast<const vec*>(kp0 + (j & 1) * 32 * KP + 16 * (j >> 1)); };
                constexpr int NS = 2 * (D / 16), SPD = 4;
                vec kb[SPD + 1];
#pragma unroll
                for (int j = 0; j < SPD; ++j) kb[j] = rd_k(j);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    if (j + SPD < NS) kb[(j + SPD) % (SPD + 1)] = rd_k(j + SPD);
                    sacc[j & 1] = Mfma<T>::run(kb[j % (SPD + 1)], qreg[j >> 1], j < 2 ? minit : sacc[j & 1]);
                    gen_slice(j);
                    __builtin_amdgcn_sched_barrier(0);
                }
                gen_finish(7);
            }
#pragma unroll
            for (int j = 0; j < PDV; ++j) vpre[j] = rd_v0(j);
            // ---- masks: causal (key > query) and the ragged end of the sequence: key
            // k0 + 32*blk + 16h + i is dropped iff it exceeds this lane's last key kmax
            if ((a.causal && k0 + kBN - 1 > q0) || k0 + kBN > L) {
                const int thr = kmax - (k0 + 16 * h);
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (32 * blk + i > thr) sacc[blk][i] = -INFINITY;
            }
            // ---- P = exp2(S - m) rounded to T, and this lane's part of the tile row sum
            auto exp_pack = [&]() {
                float lsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        u32x4 pw;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float e0 = __builtin_amdgcn_exp2f(sacc[blk][8 * s + 2 * e]);
                            const float e1 = __builtin_amdgcn_exp2f(sacc[blk][8 * s + 2 * e + 1]);
                            pw[e] = Elem<T>::pack(e0, e1);
                            lsum[e] += e0 + e1;
                        }
                        pk[blk][s] = __builtin_bit_cast(vec, pw);
                    }
                return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
            };
            const bool first = m_run == -INFINITY;
            float lt = 0.f;
            bool redo = __builtin_amdgcn_ballot_w64(first) != 0;
            if (!redo) {
                lt = exp_pack();
                redo = __builtin_amdgcn_ballot_w64(!(lt <= kLazySum)) != 0;
            }
            if (redo) {
                // move the reference to the row max (relative to the old one), rescale O and l
                float mx = sacc[0][0];
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[blk][i]);
                mx = halves_max(mx);
                float delta = first ? mx : fmaxf(mx, 0.f);
                if (mx == -INFINITY) delta = 0.f;
                const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(-delta);
                m_run = (first ? 0.f : m_run) + delta;
                l_run *= alpha;
#pragma unroll
                for (int mb = 0; mb < D / 32; ++mb) oacc[mb] *= alpha;
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int i = 0; i < 16; ++i) sacc[blk][i] -= delta;
#pragma unroll
                for (int i = 0; i < 16; ++i) minit[i] = -m_run;
                lt = exp_pack();
            }
            l_run += lt;
        }

        if constexpr (kGenSliced) {
            // waves that skipped the scores, or with an angle beyond the fast path, form the
            // staged tile's table values here in one piece (rounded to T as rope_tables_ex
            // stores them, like the pieces above)
            if (!active || __builtin_amdgcn_ballot_w64(gfar) != 0) {
                if constexpr (KROT == kRotHalfGen) {
                    gen_table_chunk<T>(kpos[0], a.pos_scale, kf[0], kc[0], ks[0]);
                } else {
                    gen_table_chunk_inter<T>(kpos[0], a.pos_scale, &kf[0][0], kc[0], ks[0]);
                    gen_table_chunk_inter<T>(kpos[0], a.pos_scale, &kf[0][4], kc2[0], ks2[0]);
                }
            }
        }
        constexpr bool kSliced = KROT != kRotNone && NKI == 1 && KITEMS == NT && D == 128;
        if constexpr (kSliced) {
            // ---- O^T += V^T P^T, each MFMA followed by a slice of the next tile's K rotation
            // (vector work the matrix core does not wait for); the P.V of inactive waves
            // multiplies P = 0 (set below) so that every wave runs the same straight block
            if (!active) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) pk[i][j] = __builtin_bit_cast(vec, u32x4{0u, 0u, 0u, 0u});
            }
            const T* vp0 = &sV[buf][(16 * h + tr_row) * VP + tr_col];
            auto rd_v = [&](int j) {
                const T* vp = vp0 + ((j >> 3) * 32 + 8 * ((j >> 2) & 1)) * VP + (j & 3) * 32;
                const i16x4 lo = lds_read_tr16(vp);
                const i16x4 hi = lds_read_tr16(vp + 4 * VP);
                return __builtin_bit_cast(vec, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            };
            float rx0 = 0.f, rx1 = 0.f, ry0 = 0.f, ry1 = 0.f, rc0 = 0.f, rc1 = 0.f, rs0 = 0.f, rs1 = 0.f;
            u32x4 kxo, kyo;
            auto rot_slice = [&](int sl) {
                if constexpr (rot_inter(KROT)) {
                    // word w of the x half (w < 4) or of the y half: unpack, then rotate and pack
                    const int w = sl >> 1;
                    const u32x4& src = w < 4 ? kx[0] : ky[0];
                    const u32x4& tc = w < 4 ? kc[0] : kc2[0];
                    const u32x4& ts = w < 4 ? ks[0] : ks2[0];
                    if ((sl & 1) == 0) {
                        rx0 = Elem<T>::lo(src[w & 3]); rx1 = Elem<T>::hi(src[w & 3]);
                        rc0 = Elem<T>::lo(tc[w & 3]); rc1 = Elem<T>::hi(tc[w & 3]);
                        rs0 = Elem<T>::lo(ts[w & 3]); rs1 = Elem<T>::hi(ts[w & 3]);
                    } else {
                        const uint32_t o = Elem<T>::pack(__builtin_fmaf(rx0, rc0, -__fmul_rn(rx1, rs0)),
                                                         __builtin_fmaf(rx1, rc1, __fmul_rn(rx0, rs1)));
                        if (w < 4) kxo[w] = o; else kyo[w & 3] = o;
                    }
                    return;
                }
                const int i = sl >> 2, q = sl & 3;
                if (q == 0) {
                    rx0 = Elem<T>::lo(kx[0][i]); rx1 = Elem<T>::hi(kx[0][i]);
                    ry0 = Elem<T>::lo(ky[0][i]); ry1 = Elem<T>::hi(ky[0][i]);
                } else if (q == 1) {
                    rc0 = Elem<T>::lo(kc[0][i]); rc1 = Elem<T>::hi(kc[0][i]);
                    rs0 = Elem<T>::lo(ks[0][i]); rs1 = Elem<T>::hi(ks[0][i]);
                } else if (q == 2) {
                    kxo[i] = Elem<T>::pack(__builtin_fmaf(rx0, rc0, -__fmul_rn(ry0, rs0)),
                                           __builtin_fmaf(rx1, rc1, -__fmul_rn(ry1, rs1)));
                } else {
                    kyo[i] = Elem<T>::pack(__builtin_fmaf(ry0, rc0, __fmul_rn(rx0, rs0)),
                                           __builtin_fmaf(ry1, rc1, __fmul_rn(rx1, rs1)));
                }
            };
            constexpr int PD = PDV;
            vec vb[PD + 1];
#pragma unroll
            for (int j = 0; j < PD; ++j) vb[j] = vpre[j];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (j + PD < 16) vb[(j + PD) % (PD + 1)] = rd_v(j + PD);
                oacc[j & 3] = Mfma<T>::run(vb[j % (PD + 1)], pk[j >> 3][(j >> 2) & 1], oacc[j & 3]);
                rot_slice(j);
                __builtin_amdgcn_sched_barrier(0);
            }
            // the staged tile's stores (into the other buffers) and the loads of the one after
            {
                T* dst = &sK[buf ^ 1][kprime_row(tid / KCH) * KP + (tid % KCH) * 8];
                *reinterpret_cast<u32x4*>(dst) = kxo;
                *reinterpret_cast<u32x4*>(dst + HALF) = kyo;
#pragma unroll
                for (int j = 0; j < NVI; ++j) {
                    const int it = tid + j * NT;
                    const int kap = it / (D / 8), c = (it % (D / 8)) * 8;
                    *reinterpret_cast<u32x4*>(&sV[buf ^ 1][kap * VP + c]) = vr[j];
                }
            }
            if (kt + 2 < n_kt) stage_load(kt + 2);
        } else {
        if (active) {
            // ---- O^T += V^T P^T: product j updates O block j % NMB with key step j / NMB
            // (the D/32 accumulator chains interleaved), operands read three products ahead
            constexpr int NMB = NMBV, NJ = 4 * NMB, PD = PDV;
            vec vb[PD + 1];
#pragma unroll
            for (int j = 0; j < PD; ++j) vb[j] = vpre[j];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if (j + PD < NJ) vb[(j + PD) % (PD + 1)] = rd_v0(j + PD);
                const int kstep = j / NMB;
                oacc[j % NMB] = Mfma<T>::run(vb[j % (PD + 1)], pk[kstep >> 1][kstep & 1], oacc[j % NMB]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // ---- stage the next tile (rotate K) into the other buffer, prefetch the one after,
        // while the P.V products run
        if (kt + 1 < n_kt) stage_store(buf ^ 1);
        if (kt + 2 < n_kt) stage_load(kt + 2);
        }
        __syncthreads();
    }

    // ------------------------------------------------------------ epilogue
    const float l_tot = halves_sum(l_run);
    if (qi < L) {
        const float inv = 1.0f / l_tot;
        T* op = reinterpret_cast<T*>(a.o) + sv.obase + (int64_t)qi * a.os[1] + (int64_t)head * a.os[2];
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = mb * 32 + 8 * g + 4 * h;
                *reinterpret_cast<u32x2*>(op + d) =
                    u32x2{Elem<T>::pack(oacc[mb][4 * g] * inv, oacc[mb][4 * g + 1] * inv),
                          Elem<T>::pack(oacc[mb][4 * g + 2] * inv, oacc[mb][4 * g + 3] * inv)};
            }
        if (a.lse && h == 0) {
            const int64_t tok = sv.varlen ? (int64_t)sv.seq_start + qi : (int64_t)b * a.seqlen + qi;
            a.lse[(int64_t)head * a.lse_stride + tok] = (m_run + __builtin_log2f(l_tot)) * 0.69314718055994530942f;
        }
    }
}

// ============================================================================ float32
// 4 waves of 32 query rows, one q head per workgroup, head_dim D, 32x32x2 float32 MFMA.
template <int D, int ROT>
__global__ __launch_bounds__(256, 2) void flash_fwd32_kernel(FaArgs a) {
    constexpr int NW = 4, NT = NW * 64;
    constexpr int QT = NW * 32;
    constexpr int KP = D + 4, VP = D + 4;
    constexpr int HALF = D / 2;
    constexpr int KCH = HALF / 8;
    constexpr int NKI = kBN * KCH / NT;
    constexpr int NVI = kBN * (D / 8) / NT;
    static_assert(NKI >= 1 && NVI >= 1, "tile too small for the workgroup");

    __shared__ __attribute__((aligned(16))) float sK[kBN * KP];
    __shared__ __attribute__((aligned(16))) float sV[kBN * VP];

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, r = l & 31, h = l >> 5;
    const int qt = gridDim.y - 1 - blockIdx.y;
    const int b = blockIdx.z;
    const SeqView sv = seq_view(a, b);
    const int L = sv.L;
    if (qt * QT >= L) return;

    const int head = blockIdx.x;
    const int kvh = head / a.group;
    const int q0 = qt * QT + w * 32;
    const int qi = q0 + r;

    const float* Kg = reinterpret_cast<const float*>(a.k) + sv.kbase + (int64_t)kvh * a.ks[2];
    const float* Vg = reinterpret_cast<const float*>(a.v) + sv.vbase + (int64_t)kvh * a.vs[2];
    const float* Cg = reinterpret_cast<const float*>(a.cos) + sv.tbase * D;
    const float* Sg = reinterpret_cast<const float*>(a.sin) + sv.tbase * D;
    const int32_t* Pg = a.pos + sv.tbase;
    const float* Fg = a.inv_freq + (a.inv_freq_rows > 1 ? (int64_t)b * HALF : 0);

    // table values of columns j..j+7 (c0, s0) and j+D/2..j+D/2+7 (c1, s1) of table row t
    auto table_values = [&](int t, int j, float (&c0)[8], float (&s0)[8], float (&c1)[8], float (&s1)[8]) {
        if constexpr (!rot_gen(ROT)) {
            unpack<float>(load_chunk<float>(Cg + (int64_t)t * D + j), c0);
            unpack<float>(load_chunk<float>(Sg + (int64_t)t * D + j), s0);
            if constexpr (rot_inter(ROT)) {
                unpack<float>(load_chunk<float>(Cg + (int64_t)t * D + j + HALF), c1);
                unpack<float>(load_chunk<float>(Sg + (int64_t)t * D + j + HALF), s1);
            }
        } else {
            const int32_t p = Pg[t];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (rot_inter(ROT)) {
                    rope_sincos(table_angle(p, a.pos_scale, Fg[j / 2 + e / 2]), s0[e], c0[e]);
                    rope_sincos(table_angle(p, a.pos_scale, Fg[(j + HALF) / 2 + e / 2]), s1[e], c1[e]);
                } else {
                    rope_sincos(table_angle(p, a.pos_scale, Fg[j + e]), s0[e], c0[e]);
                }
            }
        }
        if constexpr (!rot_inter(ROT)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                c1[e] = c0[e];
                s1[e] = s0[e];
            }
        }
    };
    auto rotate8 = [&](float (&x)[8], float (&y)[8], const float (&c0)[8], const float (&s0)[8],
                       const float (&c1)[8], const float (&s1)[8]) {
        if constexpr (rot_inter(ROT)) {
            rotate_interleaved(x, c0, s0);
            rotate_interleaved(y, c1, s1);
        } else {
            rotate_pair(x, y, c0, s0, c1, s1);
        }
    };

    // lane holds Q'[qi][8u + 4h + e], u < D/8, e < 4 (k-slot h of 4 MFMA steps); group
    // u < D/16 and group u + D/16 are columns d and d + D/2.
    float qreg[D / 2];
    {
        const float* qp = reinterpret_cast<const float*>(a.q) + sv.qbase + (int64_t)qi * a.qs[1] + (int64_t)head * a.qs[2];
#pragma unroll
        for (int u = 0; u < D / 16; ++u) {
            const int d = 8 * u + 4 * h;
            float x[8] = {}, y[8] = {};
            if (qi < L) {
                const f32x4 xv = *reinterpret_cast<const f32x4*>(qp + d);
                const f32x4 yv = *reinterpret_cast<const f32x4*>(qp + d + HALF);
                for (int e = 0; e < 4; ++e) { x[e] = xv[e]; y[e] = yv[e]; }
                if constexpr (ROT != kRotNone) {
                    // 4 columns are used; the helpers work on 8 (d is a multiple of 4, and the
                    // extra 4 columns stay inside the row: d + 8 <= D/2 + 4 for the first half)
                    float c0[8], s0[8], c1[8], s1[8];
                    table_values(qi, d & ~7, c0, s0, c1, s1);
                    float cq0[8] = {}, sq0[8] = {}, cq1[8] = {}, sq1[8] = {};
                    for (int e = 0; e < 4; ++e) {
                        cq0[e] = c0[(d & 7) + e];
                        sq0[e] = s0[(d & 7) + e];
                        cq1[e] = c1[(d & 7) + e];
                        sq1[e] = s1[(d & 7) + e];
                    }
                    rotate8(x, y, cq0, sq0, cq1, sq1);
                }
            }
            for (int e = 0; e < 4; ++e) {
                qreg[4 * u + e] = x[e] * a.scale_log2;
                qreg[4 * (u + D / 16) + e] = y[e] * a.scale_log2;
            }
        }
    }

    const int q_hi = min(qt * QT + QT, L);
    const int kend = a.causal ? q_hi : L;
    const int n_kt = (kend + kBN - 1) / kBN;
    const int wave_kend = a.causal ? min(q0 + 32, L) : L;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * kBN;
        if (kt > 0) __syncthreads();
#pragma unroll
        for (int j = 0; j < NKI; ++j) {
            const int it = tid + j * NT;
            const int kap = it / KCH, c = (it % KCH) * 8;
            const int key = k0 + kap;
            float x[8] = {}, y[8] = {};
            if (key < L) {
                unpack<float>(load_chunk<float>(Kg + (int64_t)key * a.ks[1] + c), x);
                unpack<float>(load_chunk<float>(Kg + (int64_t)key * a.ks[1] + c + HALF), y);
                if constexpr (ROT != kRotNone) {
                    float c0[8], s0[8], c1[8], s1[8];
                    table_values(key, c, c0, s0, c1, s1);
                    rotate8(x, y, c0, s0, c1, s1);
                }
            }
            float* dst = sK + kprime_row(kap) * KP + c;
            store_chunk<float>(dst, pack<float>(x));
            store_chunk<float>(dst + HALF, pack<float>(y));
        }
#pragma unroll
        for (int j = 0; j < NVI; ++j) {
            const int it = tid + j * NT;
            const int kap = it / (D / 8), c = (it % (D / 8)) * 8;
            const int key = k0 + kap;
            store_chunk<float>(sV + kap * VP + c,
                               key < L ? load_chunk<float>(Vg + (int64_t)key * a.vs[1] + c) : zero_chunk<float>());
        }
        __syncthreads();
        if (k0 >= wave_kend) continue;

        f32x16 sacc[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            sacc[blk] = f32x16{};
            const float* kp = sK + (blk * 32 + r) * KP + 4 * h;
#pragma unroll
            for (int u = 0; u < D / 8; ++u) {
                const f32x4 kv = *reinterpret_cast<const f32x4*>(kp + 8 * u);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sacc[blk] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], qreg[4 * u + e], sacc[blk], 0, 0, 0);
            }
        }
        if ((a.causal && k0 + kBN - 1 > q0) || k0 + kBN > L) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + 32 * blk + 16 * h + i;
                    if ((a.causal && key > qi) || key >= L) sacc[blk][i] = -INFINITY;
                }
        }
        float mx = sacc[0][0];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[blk][i]);
        mx = halves_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(sacc[blk][i] - m_use);
                sacc[blk][i] = p;
                psum += p;
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) oacc[mb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    const float av = sV[(blk * 32 + 16 * h + s) * VP + mb * 32 + r];
                    oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, sacc[blk][s], oacc[mb], 0, 0, 0);
                }
    }

    const float l_tot = halves_sum(l_run);
    if (qi < L) {
        const float inv = 1.0f / l_tot;
        float* op = reinterpret_cast<float*>(a.o) + sv.obase + (int64_t)qi * a.os[1] + (int64_t)head * a.os[2];
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = mb * 32 + 8 * g + 4 * h;
                *reinterpret_cast<f32x4*>(op + d) = f32x4{oacc[mb][4 * g] * inv, oacc[mb][4 * g + 1] * inv,
                                                          oacc[mb][4 * g + 2] * inv, oacc[mb][4 * g + 3] * inv};
            }
        if (a.lse && h == 0) {
            const int64_t tok = sv.varlen ? (int64_t)sv.seq_start + qi : (int64_t)b * a.seqlen + qi;
            a.lse[(int64_t)head * a.lse_stride + tok] = (m_run + __builtin_log2f(l_tot)) * 0.69314718055994530942f;
        }
    }
}

// ============================================================================ launch helpers
template <typename T, int D, int HP>
inline void launch16(const FaArgs& a, int rot, dim3 grid, hipStream_t stream) {
    switch (rot) {
        case kRotNone: hipLaunchKernelGGL((flash_fwd16_kernel<T, D, HP, kRotNone>), grid, dim3(512), 0, stream, a); break;
        case kRotHalfTable:
            hipLaunchKernelGGL((flash_fwd16_kernel<T, D, HP, kRotHalfTable>), grid, dim3(512), 0, stream, a);
            break;
        case kRotInterTable:
            hipLaunchKernelGGL((flash_fwd16_kernel<T, D, HP, kRotInterTable>), grid, dim3(512), 0, stream, a);
            break;
        case kRotHalfGen:
            hipLaunchKernelGGL((flash_fwd16_kernel<T, D, HP, kRotHalfGen>), grid, dim3(512), 0, stream, a);
            break;
        case kRotInterGen:
            hipLaunchKernelGGL((flash_fwd16_kernel<T, D, HP, kRotInterGen>), grid, dim3(512), 0, stream, a);
            break;
        case kRotQHalfTable:
            hipLaunchKernelGGL((flash_fwd16_kernel<T, D, HP, kRotQHalfTable>), grid, dim3(512), 0, stream, a);
            break;
        case kRotQInterTable:
            hipLaunchKernelGGL((flash_fwd16_kernel<T, D, HP, kRotQInterTable>), grid, dim3(512), 0, stream, a);
            break;
        case kRotQHalfGen:
            hipLaunchKernelGGL((flash_fwd16_kernel<T, D, HP, kRotQHalfGen>), grid, dim3(512), 0, stream, a);
            break;
        case kRotQInterGen:
            hipLaunchKernelGGL((flash_fwd16_kernel<T, D, HP, kRotQInterGen>), grid, dim3(512), 0, stream, a);
            break;
    }
}

template <typename T, int HP>
inline void launch16_d(const FaArgs& a, int D, int rot, dim3 grid, hipStream_t stream) {
    if (D == 64)
        launch16<T, 64, HP>(a, rot, grid, stream);
    else
        launch16<T, 128, HP>(a, rot, grid, stream);
}

template <typename T>
inline void launch16_hp(const FaArgs& a, int hp, int D, int rot, dim3 grid, hipStream_t stream) {
    switch (hp) {
        case 8: launch16_d<T, 8>(a, D, rot, grid, stream); break;
        case 4: launch16_d<T, 4>(a, D, rot, grid, stream); break;
        case 2: launch16_d<T, 2>(a, D, rot, grid, stream); break;
        default: launch16_d<T, 1>(a, D, rot, grid, stream); break;
    }
}

// one translation unit per element type instantiates the 16-bit kernels
void launch_flash16_bf16(const FaArgs& a, int hp, int D, int rot, dim3 grid, hipStream_t stream);
void launch_flash16_f16(const FaArgs& a, int hp, int D, int rot, dim3 grid, hipStream_t stream);

}  // namespace ropefa

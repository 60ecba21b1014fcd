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
//   * S^T = K' Q'^T with 32x32x16 MFMA: A = K' rows from LDS, B = Q' held in registers
//     since the start (rotated and multiplied by softmax_scale*log2(e) once).  A lane
//     therefore holds 16 scores of one query row and the row statistics need a single
//     exchange between the two halves of the wave (v_permlane32_swap).
//   * Online softmax in the log2 domain with a lazily updated reference m: the MFMA
//     accumulator starts at -m (kept in registers), so S - m comes out of the matrix core
//     and P = exp2(S - m) needs no subtraction and no row max.  The reference (and the O, l
//     rescale by exp2(m_old - m_new)) moves only on the first tile or when a row sum of
//     the tile exceeds 2^16, i.e. when some score has outgrown the reference; then the
//     tile's row max is taken and P recomputed.  P stays below 2^16 otherwise, far inside
//     the float32/bf16 range.  Row sums add the rounded P with v_dot2 (exactly the values
//     the PV product uses).
//   * O^T += V^T P^T with the same MFMA: P is already in the B-operand layout, and the
//     V^T operand comes from row-major V in LDS through the transposing LDS read
//     (ds_read_b64_tr_b16).
//   * Meanwhile the next tile, loaded into registers one tile ahead, is rotated (K) and
//     written to the other LDS buffer; the loads for the tile after it are issued.
// Permuted K' rows: MFMA result row m of S^T is key pi(m) = 16*((m>>2)&1) + 4*(m>>3) + (m&3)
// inside a 32-key block, which makes the 16 scores of lane half h the contiguous keys
// 16h .. 16h+15; K' for key pi(m) is stored at LDS row m so the MFMA reads consecutive rows.
//
// float32 kernel (flash_fwd32_kernel): 4 waves, the 32x32x2 float32 MFMA, a single LDS
// buffer and the straightforward online softmax; it serves the small float32 workload.
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
    const int32_t* cu_seqlens;  // nullptr: dense
    int64_t qs[3], ks[3], vs[3], os[3];  // {batch, token, head} strides in elements
    int32_t seqlen;                      // dense sequence length
    int32_t group;                       // hq / hkv
    int32_t table_seq_rows;
    int32_t lse_stride;                  // tokens per lse row
    int32_t causal;
    float scale_log2;                    // softmax_scale * log2(e)
};

template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
    typedef bf16x8 vec;
    static constexpr uint32_t ones = 0x3f803f80u;  // (1, 1) in bf16
    __device__ static __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<_Float16> {
    typedef f16x8 vec;
    static constexpr uint32_t ones = 0x3c003c00u;  // (1, 1) in fp16
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
        sv.seq_start = a.cu_seqlens[b];
        sv.L = a.cu_seqlens[b + 1] - sv.seq_start;
    }
    sv.qbase = sv.varlen ? (int64_t)sv.seq_start * a.qs[1] : (int64_t)b * a.qs[0];
    sv.kbase = sv.varlen ? (int64_t)sv.seq_start * a.ks[1] : (int64_t)b * a.ks[0];
    sv.vbase = sv.varlen ? (int64_t)sv.seq_start * a.vs[1] : (int64_t)b * a.vs[0];
    sv.obase = sv.varlen ? (int64_t)sv.seq_start * a.os[1] : (int64_t)b * a.os[0];
    sv.tbase = sv.varlen ? (int64_t)sv.seq_start : (a.table_seq_rows ? (int64_t)b * a.table_seq_rows : 0);
    return sv;
}

// ============================================================================ bf16 / fp16
template <typename T, int D, int HP, bool ROT>
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

    // ------------------------------------------------------------ Q' in registers
    // lane holds Q'[qi][16u + 8h + e], u < D/16, e < 8 (the MFMA B-operand layout);
    // the rotate-half partner of chunk u < D/32 is chunk u + D/32 of the same lane.
    vec qreg[D / 16];
    {
        const T* qp = reinterpret_cast<const T*>(a.q) + sv.qbase + (int64_t)qi * a.qs[1] + (int64_t)head * a.qs[2];
#pragma unroll
        for (int u = 0; u < D / 32; ++u) {
            const int d = 16 * u + 8 * h;
            float x[8] = {}, y[8] = {};
            if (qi < L) {
                unpack<T>(load_chunk<T>(qp + d), x);
                unpack<T>(load_chunk<T>(qp + d + HALF), y);
                if (ROT) {
                    float c[8], s[8];
                    unpack<T>(load_chunk<T>(Cg + (int64_t)qi * D + d), c);
                    unpack<T>(load_chunk<T>(Sg + (int64_t)qi * D + d), s);
                    rotate_pair(x, y, c, s, c, s);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[e] *= a.scale_log2;
                y[e] *= a.scale_log2;
            }
            qreg[u] = __builtin_bit_cast(vec, pack<T>(x).w);
            qreg[u + D / 32] = __builtin_bit_cast(vec, pack<T>(y).w);
        }
    }

    // ------------------------------------------------------------ tile staging
    const int q_hi = min(qt * QT + QT, L);
    const int kend = a.causal ? q_hi : L;
    const int n_kt = (kend + kBN - 1) / kBN;
    const int wave_kend = a.causal ? min(q0 + 32, L) : L;

    u32x4 kx[NKI], ky[NKI], kc[NKI], ks[NKI], vr[NVI];
    auto stage_load = [&](int kt) {
        const int k0 = kt * kBN;
        const bool full = k0 + kBN <= L;
        const T* kg = Kg + (int64_t)k0 * a.ks[1];
        const T* vg = Vg + (int64_t)k0 * a.vs[1];
        const T* cg = Cg + (int64_t)k0 * D;
        const T* sg = Sg + (int64_t)k0 * D;
        // rows past the end of the sequence re-read its last row: finite data whose scores
        // the mask removes (their P is exactly 0), so no zero fill is needed
#pragma unroll
        for (int j = 0; j < NKI; ++j) {
            const int it = tid + j * NT;
            if (KITEMS % NT == 0 || it < KITEMS) {
                const int kap = full ? it / KCH : min(it / KCH, L - 1 - k0), c = (it % KCH) * 8;
                const T* kp = kg + (int64_t)kap * a.ks[1] + c;
                kx[j] = *reinterpret_cast<const u32x4*>(kp);
                ky[j] = *reinterpret_cast<const u32x4*>(kp + HALF);
                if (ROT) {
                    kc[j] = *reinterpret_cast<const u32x4*>(cg + kap * D + c);
                    ks[j] = *reinterpret_cast<const u32x4*>(sg + kap * D + c);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NVI; ++j) {
            const int it = tid + j * NT;
            if (VITEMS % NT == 0 || it < VITEMS) {
                const int kap = full ? it / (D / 8) : min(it / (D / 8), L - 1 - k0), c = (it % (D / 8)) * 8;
                vr[j] = *reinterpret_cast<const u32x4*>(vg + (int64_t)kap * a.vs[1] + c);
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
                if (ROT) {
                    u32x4 xo, yo;
                    rotate_pair_packed<T>(kx[j], ky[j], kc[j], ks[j], xo, yo);
                    *reinterpret_cast<u32x4*>(dst) = xo;
                    *reinterpret_cast<u32x4*>(dst + HALF) = yo;
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
    stage_store(0);
    __syncthreads();
    if (n_kt > 1) stage_load(1);

    for (int kt = 0; kt < n_kt; ++kt) {
        const int buf = kt & 1;
        const int k0 = kt * kBN;
        const bool active = k0 < wave_kend;  // wave-uniform: does this wave need any key here
        vec pk[2][2];
        if (active) {
            // ---- S^T - m = K' Q'^T - m : lane (r, h) gets keys k0 + 32*blk + 16h + i of query qi
            f32x16 sacc[2];
            {
                const T* kp0 = &sK[buf][r * KP + 8 * h];
                const T* kp1 = kp0 + 32 * KP;
                sacc[0] = Mfma<T>::run(*reinterpret_cast<const vec*>(kp0), qreg[0], minit);
                sacc[1] = Mfma<T>::run(*reinterpret_cast<const vec*>(kp1), qreg[0], minit);
#pragma unroll
                for (int u = 1; u < D / 16; ++u) {
                    const vec kv0 = *reinterpret_cast<const vec*>(kp0 + 16 * u);
                    const vec kv1 = *reinterpret_cast<const vec*>(kp1 + 16 * u);
                    sacc[0] = Mfma<T>::run(kv0, qreg[u], sacc[0]);
                    sacc[1] = Mfma<T>::run(kv1, qreg[u], sacc[1]);
                }
            }
            // ---- masks: causal (key > query) and the ragged end of the sequence
            if ((a.causal && k0 + kBN - 1 > q0) || k0 + kBN > L) {
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = k0 + 32 * blk + 16 * h + i;
                        if ((a.causal && key > qi) || key >= L) sacc[blk][i] = -INFINITY;
                    }
            }
            // ---- P = exp2(S - m) rounded to T, and this lane's part of the tile row sum
            auto exp_pack = [&]() {
                float lt = 0.f;
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        u32x4 pw;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            pw[e] = Elem<T>::pack(__builtin_amdgcn_exp2f(sacc[blk][8 * s + 2 * e]),
                                                  __builtin_amdgcn_exp2f(sacc[blk][8 * s + 2 * e + 1]));
                            lt = Elem<T>::dot2(pw[e], Mfma<T>::ones, lt);
                        }
                        pk[blk][s] = __builtin_bit_cast(vec, pw);
                    }
                return lt;
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

        // ---- stage the next tile (rotate K) into the other buffer, prefetch the one after
        if (kt + 1 < n_kt) stage_store(buf ^ 1);
        if (kt + 2 < n_kt) stage_load(kt + 2);

        if (active) {
            // ---- O^T += V^T P^T
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const T* vp = &sV[buf][(blk * 32 + 16 * h + 8 * s + tr_row) * VP + mb * 32 + tr_col];
                        const i16x4 lo = lds_read_tr16(vp);
                        const i16x4 hi = lds_read_tr16(vp + 4 * VP);
                        const vec av = __builtin_bit_cast(vec, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                        oacc[mb] = Mfma<T>::run(av, pk[blk][s], oacc[mb]);
                    }
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
template <int D, bool ROT>
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

    // lane holds Q'[qi][8u + 4h + e], u < D/8, e < 4 (k-slot h of 4 MFMA steps); the
    // rotate-half partner of group u < D/16 is group u + D/16.
    float qreg[D / 2];
    {
        const float* qp = reinterpret_cast<const float*>(a.q) + sv.qbase + (int64_t)qi * a.qs[1] + (int64_t)head * a.qs[2];
#pragma unroll
        for (int u = 0; u < D / 16; ++u) {
            const int d = 8 * u + 4 * h;
            float x[8] = {}, y[8] = {}, c[8] = {}, s[8] = {};
            if (qi < L) {
                const f32x4 xv = *reinterpret_cast<const f32x4*>(qp + d);
                const f32x4 yv = *reinterpret_cast<const f32x4*>(qp + d + HALF);
                for (int e = 0; e < 4; ++e) { x[e] = xv[e]; y[e] = yv[e]; }
                if (ROT) {
                    const f32x4 cv = *reinterpret_cast<const f32x4*>(Cg + (int64_t)qi * D + d);
                    const f32x4 sv4 = *reinterpret_cast<const f32x4*>(Sg + (int64_t)qi * D + d);
                    for (int e = 0; e < 4; ++e) { c[e] = cv[e]; s[e] = sv4[e]; }
                    rotate_pair(x, y, c, s, c, s);
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
            float x[8] = {}, y[8] = {}, cc[8] = {}, ss[8] = {};
            if (key < L) {
                unpack<float>(load_chunk<float>(Kg + (int64_t)key * a.ks[1] + c), x);
                unpack<float>(load_chunk<float>(Kg + (int64_t)key * a.ks[1] + c + HALF), y);
                if (ROT) {
                    unpack<float>(load_chunk<float>(Cg + (int64_t)key * D + c), cc);
                    unpack<float>(load_chunk<float>(Sg + (int64_t)key * D + c), ss);
                    rotate_pair(x, y, cc, ss, cc, ss);
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

// ============================================================================ launch
template <typename T, int D, int HP>
static void launch16(const FaArgs& a, bool rot, dim3 grid, hipStream_t stream) {
    if (rot)
        hipLaunchKernelGGL((flash_fwd16_kernel<T, D, HP, true>), grid, dim3(512), 0, stream, a);
    else
        hipLaunchKernelGGL((flash_fwd16_kernel<T, D, HP, false>), grid, dim3(512), 0, stream, a);
}

template <typename T, int HP>
static void launch16_d(const FaArgs& a, int D, bool rot, dim3 grid, hipStream_t stream) {
    if (D == 64)
        launch16<T, 64, HP>(a, rot, grid, stream);
    else
        launch16<T, 128, HP>(a, rot, grid, stream);
}

template <typename T>
static void launch16_hp(const FaArgs& a, int hp, int D, bool rot, dim3 grid, hipStream_t stream) {
    switch (hp) {
        case 8: launch16_d<T, 8>(a, D, rot, grid, stream); break;
        case 4: launch16_d<T, 4>(a, D, rot, grid, stream); break;
        case 2: launch16_d<T, 2>(a, D, rot, grid, stream); break;
        default: launch16_d<T, 1>(a, D, rot, grid, stream); break;
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
    a.group = p->hq / p->hkv;
    a.table_seq_rows = p->table_seq_rows;
    a.lse_stride = varlen ? p->ntokens : p->batch * p->seqlen;
    a.causal = p->causal;
    a.scale_log2 = p->softmax_scale * 1.44269504088896340736f;
    const bool rot = p->cos != nullptr;
    const int maxlen = varlen ? p->max_seqlen : p->seqlen;
    if (p->dtype == ROPE_DT_F32) {
        const int qt = 4 * 32;
        const dim3 grid((unsigned)p->hq, (unsigned)((maxlen + qt - 1) / qt), (unsigned)p->batch);
        if (rot)
            hipLaunchKernelGGL((flash_fwd32_kernel<64, true>), grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((flash_fwd32_kernel<64, false>), grid, dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    const int hp = flash_heads_per_wg(a.group, p->dtype);
    const int qt = (8 / hp) * 32;
    const dim3 grid((unsigned)(p->hq / hp), (unsigned)((maxlen + qt - 1) / qt), (unsigned)p->batch);
    switch (p->dtype) {
        case ROPE_DT_BF16: launch16_hp<__bf16>(a, hp, p->head_dim, rot, grid, stream); break;
        case ROPE_DT_F16: launch16_hp<_Float16>(a, hp, p->head_dim, rot, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ropefa

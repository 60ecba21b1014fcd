// rope_flash_attn_fwd: RoPE fused into a FlashAttention forward pass on gfx950.
//
// What is computed ([RoPE-fusion blog], section 三; [FlashAttention blog], tiling and
// online softmax): for each (sequence, q head, query row) the rotate-half RoPE of q and
// of every key, the scaled scores, a softmax over the causal keys of the sequence and
// the weighted sum of V.  Rotated Q/K exist only in registers and LDS.
//
// Work decomposition.  A workgroup is 4 waves (256 threads).  Each wave owns 32 query
// rows of one q head; a workgroup holds HP q heads of the same kv head (GQA packing)
// times (4/HP)*32 queries, so one staged K/V tile serves 128 (head, query) rows.  The
// grid is (head groups, query tiles, sequences); query tiles are issued longest-first
// for causal balance.
//
// Per key tile of 64 keys:
//   * all threads load K (both rotate-half partners of a chunk in the same thread), the
//     table rows of those keys and V into registers one tile ahead, then rotate K in
//     float32 and write K' and V to LDS;
//   * each wave computes S^T = K' Q'^T with 32x32x16 bf16/fp16 MFMA (A = K' rows from LDS,
//     B = Q' held in registers since the start), so a lane holds 16 scores of one query
//     row; the running max needs one exchange between the two wave halves;
//   * online softmax in the log2 domain (softmax_scale*log2(e) is folded into Q'):
//     m' = max(m, rowmax), P = exp2(S - m'), l = l*exp2(m - m') + rowsum(P), O *= exp2(m - m');
//   * O^T += V^T P^T with the same MFMA: P is already in the B-operand layout, and the
//     V^T operand comes straight from row-major V in LDS through the transposing LDS read.
// Permuted K' rows: MFMA result row m of S^T is key pi(m) = 16*((m>>2)&1) + 4*(m>>3) + (m&3)
// inside a 32-key block, which makes the 16 scores of lane half h the contiguous keys
// 16h .. 16h+15.  K' is stored at LDS row m for key pi(m), so the MFMA still reads
// consecutive LDS rows.
//
// float32 inputs use the 32x32x2 float32 MFMA with the same data flow.
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
template <> struct Mfma<float> {
    typedef float vec;
};

// Value of x in the lane 32 apart (the other half of the wave) combined with x.
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

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBN = 64;  // keys per tile

template <typename T, int D, int HP, bool ROT>
__global__ __launch_bounds__(kThreads, 2) void flash_fwd_kernel(FaArgs a) {
    constexpr bool F32 = Elem<T>::bytes == 4;
    constexpr int QT = (kWaves / HP) * 32;         // queries per workgroup
    constexpr int KP = D + (F32 ? 4 : 8);          // K' LDS row pitch (elements)
    constexpr int VP = D + (F32 ? 4 : 16);         // V LDS row pitch (elements)
    constexpr int HALF = D / 2;
    constexpr int KCH = HALF / 8;                  // 8-element chunks per half row
    constexpr int NKI = kBN * KCH / kThreads;      // K staging items per thread
    constexpr int NVI = kBN * (D / 8) / kThreads;  // V staging items per thread
    static_assert(NKI >= 1 && NVI >= 1, "tile too small for the workgroup");
    typedef typename Mfma<T>::vec vec;

    __shared__ __attribute__((aligned(16))) T sK[kBN * KP];
    __shared__ __attribute__((aligned(16))) T sV[kBN * VP];

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, r = l & 31, h = l >> 5;
    const int qt = gridDim.y - 1 - blockIdx.y;  // longest query tiles first
    const int b = blockIdx.z;

    int seq_start = 0, L = a.seqlen;
    if (a.cu_seqlens) {
        seq_start = a.cu_seqlens[b];
        L = a.cu_seqlens[b + 1] - seq_start;
    }
    if (qt * QT >= L) return;  // whole workgroup: this sequence is shorter

    const int head = blockIdx.x * HP + (w % HP);
    const int kvh = (blockIdx.x * HP) / a.group;
    const int q0 = qt * QT + (w / HP) * 32;  // first query row of this wave
    const int qi = q0 + r;                     // this lane's query row

    const bool varlen = a.cu_seqlens != nullptr;
    const int64_t qbase = varlen ? (int64_t)seq_start * a.qs[1] : (int64_t)b * a.qs[0];
    const int64_t kbase = varlen ? (int64_t)seq_start * a.ks[1] : (int64_t)b * a.ks[0];
    const int64_t vbase = varlen ? (int64_t)seq_start * a.vs[1] : (int64_t)b * a.vs[0];
    const int64_t obase = varlen ? (int64_t)seq_start * a.os[1] : (int64_t)b * a.os[0];
    const int64_t tbase = varlen ? (int64_t)seq_start : (a.table_seq_rows ? (int64_t)b * a.table_seq_rows : 0);

    const T* Kg = reinterpret_cast<const T*>(a.k) + kbase + (int64_t)kvh * a.ks[2];
    const T* Vg = reinterpret_cast<const T*>(a.v) + vbase + (int64_t)kvh * a.vs[2];
    const T* Cg = reinterpret_cast<const T*>(a.cos);
    const T* Sg = reinterpret_cast<const T*>(a.sin);

    // ---------------------------------------------------------------- Q' in registers
    // 16-bit: lane holds Q'[qi][16u + 8h + e], u < D/16, e < 8 (the MFMA B layout).
    // float32: lane holds Q'[qi][8u + 4h + e], u < D/8, e < 4 (k-slot h of 4 MFMA steps).
    constexpr int QV = F32 ? D / 2 : D / 16;
    vec qreg[QV];
    {
        const T* qp = reinterpret_cast<const T*>(a.q) + qbase + (int64_t)qi * a.qs[1] + (int64_t)head * a.qs[2];
        const T* cp = Cg + (tbase + qi) * D;
        const T* sp = Sg + (tbase + qi) * D;
        constexpr int NU = F32 ? D / 16 : D / 32;  // first-half groups per lane
        constexpr int W = F32 ? 4 : 8;             // elements per group
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int d = (F32 ? 8 * u + 4 * h : 16 * u + 8 * h);
            float x[8] = {}, y[8] = {}, c[8] = {}, s[8] = {};
            if (qi < L) {
                if constexpr (F32) {
                    const f32x4 xv = *reinterpret_cast<const f32x4*>(qp + d);
                    const f32x4 yv = *reinterpret_cast<const f32x4*>(qp + d + HALF);
                    for (int e = 0; e < 4; ++e) { x[e] = xv[e]; y[e] = yv[e]; }
                    if (ROT) {
                        const f32x4 cv = *reinterpret_cast<const f32x4*>(cp + d);
                        const f32x4 sv = *reinterpret_cast<const f32x4*>(sp + d);
                        for (int e = 0; e < 4; ++e) { c[e] = cv[e]; s[e] = sv[e]; }
                    }
                } else {
                    unpack<T>(load_chunk<T>(qp + d), x);
                    unpack<T>(load_chunk<T>(qp + d + HALF), y);
                    if (ROT) {
                        unpack<T>(load_chunk<T>(cp + d), c);
                        unpack<T>(load_chunk<T>(sp + d), s);
                    }
                }
                if (ROT) rotate_pair(x, y, c, s, c, s);
            }
#pragma unroll
            for (int e = 0; e < W; ++e) {
                x[e] *= a.scale_log2;
                y[e] *= a.scale_log2;
            }
            if constexpr (F32) {
                for (int e = 0; e < 4; ++e) {
                    qreg[4 * u + e] = x[e];
                    qreg[4 * (u + D / 16) + e] = y[e];
                }
            } else {
                const Chunk8<T> px = pack<T>(x), py = pack<T>(y);
                qreg[u] = __builtin_bit_cast(vec, px.w);
                qreg[u + D / 32] = __builtin_bit_cast(vec, py.w);
            }
        }
    }

    // ---------------------------------------------------------------- main loop
    const int q_hi = min(qt * QT + QT, L);
    const int kend = a.causal ? q_hi : L;
    const int n_kt = (kend + kBN - 1) / kBN;
    const int wave_kend = a.causal ? min(q0 + 32, L) : L;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    Chunk8<T> kx[NKI], ky[NKI], kc[NKI], ks[NKI], vr[NVI];
    auto stage_load = [&](int kt) {
        const int k0 = kt * kBN;
#pragma unroll
        for (int j = 0; j < NKI; ++j) {
            const int it = tid + j * kThreads;
            const int kap = it / KCH, c = (it % KCH) * 8;
            const int key = k0 + kap;
            if (key < L) {
                const T* kp = Kg + (int64_t)key * a.ks[1];
                kx[j] = load_chunk<T>(kp + c);
                ky[j] = load_chunk<T>(kp + c + HALF);
                if (ROT) {
                    kc[j] = load_chunk<T>(Cg + (tbase + key) * D + c);
                    ks[j] = load_chunk<T>(Sg + (tbase + key) * D + c);
                }
            } else {
                kx[j] = zero_chunk<T>();
                ky[j] = zero_chunk<T>();
                kc[j] = zero_chunk<T>();
                ks[j] = zero_chunk<T>();
            }
        }
#pragma unroll
        for (int j = 0; j < NVI; ++j) {
            const int it = tid + j * kThreads;
            const int kap = it / (D / 8), c = (it % (D / 8)) * 8;
            const int key = k0 + kap;
            vr[j] = key < L ? load_chunk<T>(Vg + (int64_t)key * a.vs[1] + c) : zero_chunk<T>();
        }
    };
    auto stage_store = [&]() {
#pragma unroll
        for (int j = 0; j < NKI; ++j) {
            const int it = tid + j * kThreads;
            const int kap = it / KCH, c = (it % KCH) * 8;
            T* dst = sK + kprime_row(kap) * KP + c;
            if (ROT) {
                float x[8], y[8], cc[8], ss[8];
                unpack<T>(kx[j], x);
                unpack<T>(ky[j], y);
                unpack<T>(kc[j], cc);
                unpack<T>(ks[j], ss);
                rotate_pair(x, y, cc, ss, cc, ss);
                store_chunk<T>(dst, pack<T>(x));
                store_chunk<T>(dst + HALF, pack<T>(y));
            } else {
                store_chunk<T>(dst, kx[j]);
                store_chunk<T>(dst + HALF, ky[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NVI; ++j) {
            const int it = tid + j * kThreads;
            const int kap = it / (D / 8), c = (it % (D / 8)) * 8;
            store_chunk<T>(sV + kap * VP + c, vr[j]);
        }
    };

    if (n_kt > 0) stage_load(0);
    for (int kt = 0; kt < n_kt; ++kt) {
        if (kt > 0) __syncthreads();  // every wave is done with the previous tile
        stage_store();
        __syncthreads();
        if (kt + 1 < n_kt) stage_load(kt + 1);
        const int k0 = kt * kBN;
        if (k0 >= wave_kend) continue;  // wave-uniform: no key of this tile is needed here

        // ---- S^T = K' Q'^T : lane (r, h) gets keys k0 + 32*blk + 16h + i for query qi
        f32x16 sacc[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            sacc[blk] = f32x16{};
            if constexpr (F32) {
                const float* kp = sK + (blk * 32 + r) * KP + 4 * h;
#pragma unroll
                for (int u = 0; u < D / 8; ++u) {
                    const f32x4 kv = *reinterpret_cast<const f32x4*>(kp + 8 * u);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sacc[blk] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], qreg[4 * u + e], sacc[blk], 0, 0, 0);
                }
            } else {
                const T* kp = sK + (blk * 32 + r) * KP + 8 * h;
#pragma unroll
                for (int u = 0; u < D / 16; ++u) {
                    const vec kv = *reinterpret_cast<const vec*>(kp + 16 * u);
                    sacc[blk] = Mfma<T>::run(kv, qreg[u], sacc[blk]);
                }
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
        // ---- online softmax (log2 domain)
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

        // ---- O^T += V^T P^T
        if constexpr (F32) {
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int s = 0; s < 16; ++s) {
                        const float av = sV[(blk * 32 + 16 * h + s) * VP + mb * 32 + r];
                        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, sacc[blk][s], oacc[mb], 0, 0, 0);
                    }
        } else {
            vec pk[2][2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    float pv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) pv[e] = sacc[blk][8 * s + e];
                    pk[blk][s] = __builtin_bit_cast(vec, pack<T>(pv).w);
                }
            // transposing read: lane l of each 16-lane group supplies row (l%16)/4, columns
            // 4*(l%4)..+3 of a 4x16 tile and receives the tile's column l%16
            const int tr_row = (l & 15) >> 2;
            const int tr_col = ((l >> 4) & 1) * 16 + 4 * (l & 3);
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const T* vp = sV + (blk * 32 + 16 * h + 8 * s + tr_row) * VP + mb * 32 + tr_col;
                        const i16x4 lo = lds_read_tr16(vp);
                        const i16x4 hi = lds_read_tr16(vp + 4 * VP);
                        const vec av = __builtin_bit_cast(vec, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                        oacc[mb] = Mfma<T>::run(av, pk[blk][s], oacc[mb]);
                    }
        }
    }

    // ---------------------------------------------------------------- epilogue
    const float l_tot = halves_sum(l_run);
    if (qi < L) {
        const float inv = 1.0f / l_tot;
        T* op = reinterpret_cast<T*>(a.o) + obase + (int64_t)qi * a.os[1] + (int64_t)head * a.os[2];
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = mb * 32 + 8 * g + 4 * h;
                const float v0 = oacc[mb][4 * g] * inv, v1 = oacc[mb][4 * g + 1] * inv;
                const float v2 = oacc[mb][4 * g + 2] * inv, v3 = oacc[mb][4 * g + 3] * inv;
                if constexpr (F32) {
                    *reinterpret_cast<f32x4*>(op + d) = f32x4{v0, v1, v2, v3};
                } else {
                    *reinterpret_cast<u32x2*>(op + d) = u32x2{Elem<T>::pack(v0, v1), Elem<T>::pack(v2, v3)};
                }
            }
        if (a.lse && h == 0) {
            const int64_t tok = varlen ? (int64_t)seq_start + qi : (int64_t)b * a.seqlen + qi;
            a.lse[(int64_t)head * a.lse_stride + tok] = (m_run + __builtin_log2f(l_tot)) * 0.69314718055994530942f;
        }
    }
}

template <typename T, int D, int HP>
static void launch_t(const FaArgs& a, bool rot, dim3 grid, hipStream_t stream) {
    if (rot)
        hipLaunchKernelGGL((flash_fwd_kernel<T, D, HP, true>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((flash_fwd_kernel<T, D, HP, false>), grid, dim3(kThreads), 0, stream, a);
}

template <typename T, int HP>
static void launch_d(const FaArgs& a, int D, bool rot, dim3 grid, hipStream_t stream) {
    if (D == 64)
        launch_t<T, 64, HP>(a, rot, grid, stream);
    else
        launch_t<T, 128, HP>(a, rot, grid, stream);
}

// Heads packed per workgroup: as many q heads of one kv head as divide the group.
int flash_heads_per_wg(int group, rope_dtype dt) {
    if (dt == ROPE_DT_F32) return 1;
    if (group % 4 == 0) return 4;
    if (group % 2 == 0) return 2;
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
    const int hp = flash_heads_per_wg(a.group, p->dtype);
    const int qt = (kWaves / hp) * 32;
    const int maxlen = varlen ? p->max_seqlen : p->seqlen;
    const dim3 grid((unsigned)(p->hq / hp), (unsigned)((maxlen + qt - 1) / qt), (unsigned)p->batch);
    switch (p->dtype) {
        case ROPE_DT_BF16:
            if (hp == 4) launch_d<__bf16, 4>(a, p->head_dim, rot, grid, stream);
            else if (hp == 2) launch_d<__bf16, 2>(a, p->head_dim, rot, grid, stream);
            else launch_d<__bf16, 1>(a, p->head_dim, rot, grid, stream);
            break;
        case ROPE_DT_F16:
            if (hp == 4) launch_d<_Float16, 4>(a, p->head_dim, rot, grid, stream);
            else if (hp == 2) launch_d<_Float16, 2>(a, p->head_dim, rot, grid, stream);
            else launch_d<_Float16, 1>(a, p->head_dim, rot, grid, stream);
            break;
        case ROPE_DT_F32: launch_t<float, 64, 1>(a, rot, grid, stream); break;  // head_dim 64 only
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ropefa

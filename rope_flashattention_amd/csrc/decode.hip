// rope_decode_attn_fwd: one decode step of RoPE + GQA attention over a paged KV cache, gfx950.
//
// What is computed: each sequence's new query, rotated with its table row (the rope_qk
// formula, rotate-half or interleaved pairs), attends to every key in the sequence's
// cache ([FlashAttention blog]: Softmax(QK^T/sqrt(d))V; the keys were rotated when they
// were written).  The g = hq/hkv
// query heads that share a kv head ([RoPE/GQA tutorial], sections 十一-十二) are served by
// one pass over that head's cache, so the cache is read once per kv head, which is the
// traffic GQA exists to save.  A decode step does a few flops per cached byte, so the
// kernels are bound by HBM bandwidth.
//
// Partial kernel (decode_partial_kernel): one wavefront per (sequence, kv head, group of
// up to 32 q heads, key split).  Splits have a fixed length, so sequence b has
// ceil(L_b / chunk) non-empty ones; for batches up to kCompactMaxBatch the grid is a list of
// only those items (every wave reads the lengths and finds its item by a prefix sum), so
// every workgroup has the same work up to the last split of a sequence and the
// dispatcher spreads them evenly over the CUs; larger batches use one workgroup per
// (split, unit, sequence) and empty splits exit at once.  Per 32-key tile:
//   * K and V rows arrive by coalesced 16-byte loads (whole 256-byte rows per 16 lanes;
//     every load of a tile issued back to back, the next tile's loads issued as soon as
//     this tile is in LDS) and are stored row-major in a wave-private LDS tile whose
//     16-byte chunks are XOR-swizzled per row, so the reads below are bank-conflict free.
//     The split's block-table entries are read once into one register per lane and
//     fetched per row with a lane shuffle.
//   * S^T = K Q'^T with the 32x32x16 MFMA: the A operand is LDS row pi(m) of the K tile,
//     the B operand the rotated, scaled Q' of the group's heads (head = MFMA column) held
//     in registers for the whole pass; unused columns are zero.
//   * Permuted rows: MFMA row m holds key pi(m) = 16*((m>>2)&1) + 4*(m>>3) + (m&3), which
//     makes lane half h hold the scores of the contiguous keys 16h .. 16h+15 of its head, so
//     the probabilities are already the B operand of the next product.
//   * Online softmax per head in the log2 domain (scale * log2(e) folded into Q'); the
//     reference maximum moves, and O and l are rescaled, only when a tile's maximum
//     exceeds it by more than 2^8 (P <= 2^8 otherwise).
//   * O^T += V^T P^T with the same MFMA; the transposing LDS read (ds_read_b64_tr_b16)
//     supplies the V^T operand.
// The wave writes its unnormalised O, reference m and sum l for its key range to the
// workspace.  Combine kernel (decode_combine_kernel): one workgroup per (sequence, q head)
// merges the splits: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
#include <mutex>

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
    int32_t interleaved;  // query pairing: 0 rotate-half, 1 interleaved
    int32_t chunk;      // keys per split (multiple of 32)
    int32_t bs_shift;   // log2(block_size) when it is a power of two, else -1
    int32_t table_regs; // 1: a split's block-table entries fit one register per lane
    int32_t compact;    // 1: workgroup i takes the i-th non-empty (sequence, unit, split) item
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

__device__ __forceinline__ int logical_block(const DecodeArgs& a, int key) {
    return a.bs_shift >= 0 ? key >> a.bs_shift : key / a.block_size;
}

// physical block of logical block lb of sequence b, clamped into the cache
__device__ __forceinline__ int physical_block(const DecodeArgs& a, int b, int lb) {
    const int pb = a.block_table ? a.block_table[(int64_t)b * a.max_blocks + lb] : b * a.max_blocks + lb;
    return min(max(pb, 0), a.num_blocks - 1);
}

// Sequences up to which the partial kernel's grid lists only non-empty items.
constexpr int kCompactMaxBatch = 1024;

// cached length of sequence b as the kernels use it: clamped to [0, max_seqlen]
__device__ __forceinline__ int seq_len(const DecodeArgs& a, int b) {
    return max(min(a.seqlens[b], a.max_seqlen), 0);
}

template <typename T, int D>
__global__ __launch_bounds__(64, 2) void decode_partial_kernel(DecodeArgs a) {
    constexpr int NS = D / 16;        // MFMA k-steps over the head dimension
    constexpr int CPR = D / 8;        // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;     // rows per coalesced load instruction
    constexpr int NLD = 32 / RPI;     // load instructions per 32-row tile (= D / 16)
    constexpr float kNegInf = -__builtin_inff();
    // K and V tiles, row-major, 16-byte chunks XOR-swizzled per row (conflict-free reads)
    __shared__ __attribute__((aligned(16))) T sK[32 * D];
    __shared__ __attribute__((aligned(16))) T sV[32 * D];

    const int l = threadIdx.x;
    const int n = l & 31;
    const int hh = l >> 5;
    int split, unit, b;
    if (a.compact) {
        // items in the order (sequence, unit, split), non-empty splits only: sequence b owns
        // units * ceil(L_b / chunk) of them; a wave-wide prefix sum over the lengths, 64
        // sequences at a time, finds the one that holds item blockIdx.x
        const int units = a.hkv * a.ngroups;
        const int item = blockIdx.x;
        int base = 0;
        b = -1;
        int local = 0, nb = 1;
        for (int b0 = 0; b0 < a.batch; b0 += 64) {
            const int bi = b0 + l;
            const int cnt = bi < a.batch ? (seq_len(a, bi) + a.chunk - 1) / a.chunk * units : 0;
            int inc = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(inc, o);
                inc += l >= o ? t : 0;
            }
            const int tot = __shfl(inc, 63);
            if (item < base + tot) {
                const int lane = __builtin_ctzll(__builtin_amdgcn_ballot_w64(base + inc > item));
                b = b0 + lane;
                local = __builtin_amdgcn_readfirstlane(item - base - __shfl(inc - cnt, lane));
                nb = __builtin_amdgcn_readfirstlane(__shfl(cnt, lane)) / units;
                break;
            }
            base += tot;
        }
        if (b < 0) return;  // past the last item
        unit = local / nb;
        split = local - unit * nb;
    } else {
        split = blockIdx.x;
        unit = blockIdx.y;
        b = blockIdx.z;
    }
    const int kvh = unit / a.ngroups;
    const int grp = unit - kvh * a.ngroups;
    const int hin = grp * 32 + n;
    const bool hvalid = hin < a.g;
    const int h = kvh * a.g + (hvalid ? hin : 0);

    const int L = seq_len(a, b);
    // splits of a fixed length (from the host bound): every non-empty split has the same
    // work up to a sequence's last one; the combine reads only splits below ceil(L / chunk)
    const int k_begin = min(split * a.chunk, L);
    const int k_end = min(L, k_begin + a.chunk);
    if (k_begin >= k_end) return;  // empty split (wave-uniform)
    const int lb0 = k_begin < k_end ? logical_block(a, k_begin) : 0;
    int tabv = 0;
    if (a.table_regs && k_begin < k_end) {
        const int nlb = logical_block(a, k_end - 1) - lb0 + 1;
        if (l < nlb) tabv = physical_block(a, b, lb0 + l);
    }

    // ---- Q'^T operand
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
                if (a.interleaved) {
                    rotate_interleaved(x, c0, s0);
                    rotate_interleaved(y, c1, s1);
                } else {
                    rotate_pair(x, y, c0, s0, c1, s1);
                }
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
    const int prow = 16 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);   // key (LDS row) of MFMA row n
    const int kswz = (prow & 3) | (((prow >> 4) & 1) << 2);          // its chunk swizzle
    const int tr_row = (l & 15) >> 2;
    const int tr_col = ((l >> 4) & 1) * 16 + 4 * (l & 3);
    const int ld_row = l / CPR;       // + RPI * i
    const int ld_chunk = l % CPR;

    // coalesced loads of one 32-key tile: instruction i, lane l -> row RPI*i + l/CPR, chunk l%CPR
    u32x4 kst[NLD], vst[NLD];
    auto load_tile = [&](int k0) {
        // physical block and offset of every row first (no load in flight is waited on
        // here), then all K and V loads back to back
        int pb[NLD], off[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int key = min(k0 + RPI * i + ld_row, k_end - 1);
            const int lb = logical_block(a, key);
            off[i] = key - lb * a.block_size;
            pb[i] = lb;
        }
        if (a.table_regs) {
#pragma unroll
            for (int i = 0; i < NLD; ++i) pb[i] = __shfl(tabv, pb[i] - lb0);
        } else {
#pragma unroll
            for (int i = 0; i < NLD; ++i) pb[i] = physical_block(a, b, pb[i]);
        }
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            kst[i] = load_stream<T>(kbase + (int64_t)pb[i] * a.kcs[0] + (int64_t)off[i] * a.kcs[1] + ld_chunk * 8).w;
            vst[i] = load_stream<T>(vbase + (int64_t)pb[i] * a.vcs[0] + (int64_t)off[i] * a.vcs[1] + ld_chunk * 8).w;
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[mb][i] = 0.0f;
    float m_run = kNegInf;
    float l_half = 0.0f;

    if (k_begin < k_end) load_tile(k_begin);
    for (int k0 = k_begin; k0 < k_end; k0 += 32) {
        // ---- staged tile -> LDS (K chunk c of row r at slot c ^ fK(r), V at c ^ fV(r))
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int r = RPI * i + ld_row;
            const int fk = (r & 3) | (((r >> 4) & 1) << 2);
            const int fv = 2 * (r & 3);
            *reinterpret_cast<u32x4*>(&sK[r * D + 8 * (ld_chunk ^ fk)]) = kst[i];
            *reinterpret_cast<u32x4*>(&sV[r * D + 8 * (ld_chunk ^ fv)]) = vst[i];
        }
        wave_lds_sync();
        if (k0 + 32 < k_end) load_tile(k0 + 32);   // the next tile streams in while this one is used

        // ---- S^T = K Q'^T, A operand from LDS row prow
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const u32x4 ka = *reinterpret_cast<const u32x4*>(&sK[prow * D + 8 * ((2 * s + hh) ^ kswz)]);
            sacc = DMma<T>::run(ka, qb[s], sacc);
        }

        // ---- online softmax: lane half hh holds keys k0 + 16*hh + i
        const int valid = k_end - (k0 + 16 * hh);
        float mt = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i >= valid) sacc[i] = kNegInf;
            mt = fmaxf(mt, sacc[i]);
        }
        mt = dec_halves_max(mt);
        if (__builtin_amdgcn_ballot_w64(mt > m_run + 8.0f)) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_half *= alpha;
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb) oacc[mb] *= alpha;
        }
        const float m_new = m_run;
        u32x4 pk[2];
        float lt = 0.0f;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(sacc[8 * s + j] - m_new);
            pk[s] = pack<T>(p).w;
            float pr[8];
            unpack<T>(Chunk8<T>{pk[s]}, pr);
#pragma unroll
            for (int j = 0; j < 8; ++j) lt += pr[j];
        }
        l_half += lt;

        // ---- O^T += V^T P^T, V^T operand by the transposing LDS read
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int r = 16 * hh + 8 * s + tr_row;        // rows r and r + 4, r % 4 == tr_row
                const int e = mb * 32 + tr_col;                 // element column, 4 elements
                const int sw = 8 * ((e >> 3) ^ (2 * tr_row)) + (e & 7);
                const i16x4 lo = lds_tr16(&sV[r * D + sw]);
                const i16x4 hi = lds_tr16(&sV[(r + 4) * D + sw]);
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
    // one workgroup of D threads per (sequence, q head); thread d owns output column d.
    // The split statistics are read one split per lane (each wave computes them
    // redundantly).  With at most kPre splits (the usual case) every load of the kernel -
    // the sequence length, the statistics and the partial rows - is issued at once, before
    // the length says which splits hold keys, so the kernel waits for memory once; the
    // partial rows of splits past the last live one are read (the workspace holds them,
    // written or not) and dropped by a select, never by a multiply.
    constexpr float kNegInf = -__builtin_inff();
    constexpr int kPre = 16;
    const int bh = blockIdx.x;
    const int b = bh / a.hq;
    const int h = bh - b * a.hq;
    const int d = threadIdx.x;
    const int lane = d & 63;
    const int64_t p0 = (int64_t)bh * a.nsplit;
    float o = 0.0f, lsum = 0.0f, M = kNegInf;
    int live;
    if (a.nsplit <= kPre) {
        const int ls = min(lane, a.nsplit - 1);
        const float mv = a.ws_m[p0 + ls];
        const float lv = a.ws_l[p0 + ls];
        float v[kPre];
#pragma unroll
        for (int u = 0; u < kPre; ++u) v[u] = a.ws_o[(p0 + min(u, a.nsplit - 1)) * D + d];
        live = (seq_len(a, b) + a.chunk - 1) / a.chunk;  // the splits the partial kernel wrote
        M = lane < live ? mv : kNegInf;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        const float w = lane < live ? exp2f(mv - M) : 0.0f;
        lsum = lane < live ? w * lv : 0.0f;
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
            o += u < live ? wj * v[u] : 0.0f;
        }
    } else {
        live = (seq_len(a, b) + a.chunk - 1) / a.chunk;
        for (int s0 = 0; s0 < live; s0 += 64) M = fmaxf(M, s0 + lane < live ? a.ws_m[p0 + s0 + lane] : kNegInf);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        for (int s0 = 0; s0 < live; s0 += 64) {
            const int s = s0 + lane;
            const float w = s < live ? exp2f(a.ws_m[p0 + s] - M) : 0.0f;
            lsum += s < live ? w * a.ws_l[p0 + s] : 0.0f;
            const int n = min(64, live - s0);
            const float* wo = a.ws_o + (p0 + s0) * D + d;
            for (int j0 = 0; j0 < n; j0 += 8) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = wo[(int64_t)min(j0 + u, n - 1) * D];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), min(j0 + u, 63)));
                    o += j0 + u < n ? wj * v[u] : 0.0f;
                }
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
    if (live > 0) o = o / lsum;
    T* orow = reinterpret_cast<T*>(a.out) + (int64_t)b * a.os[0] + (int64_t)h * a.os[1];
    orow[d] = (T)o;
    if (a.lse && d == 0) a.lse[bh] = live > 0 ? (M + log2f(lsum)) * 0.69314718055994531f : kNegInf;
}

int decode_num_splits(const rope_decode_params* p) {
    if (p->num_splits > 0) return p->num_splits;
    const int g = p->hq / p->hkv;
    const int64_t units = (int64_t)p->batch * p->hkv * ((g + 31) / 32);
    // about 8 waves per CU when every sequence is at the bound (splits have a fixed length,
    // max_seqlen / ns, so shorter sequences leave some of them empty; measured on 32
    // sequences of 1024..8192 keys: 9 splits 4.77 TB/s, 13: 4.46, 17: 4.39, 33: 4.47).  In the
    // grid of all (split, unit, sequence) triples used above kCompactMaxBatch sequences an
    // odd count makes consecutive splits of a sequence fall on different XCDs (workgroups
    // are placed round robin by linear id, split fastest), so empty high splits spread evenly
    int64_t ns = (2048 + units - 1) / units;
    const int64_t by_len = ((int64_t)p->max_seqlen + 127) / 128;  // at least 128 keys per split
    ns = ns < by_len ? ns : by_len;
    if (ns > 1 && (ns & 1) == 0) ns += 1;
    ns = ns < 255 ? ns : 255;
    return (int)(ns < 1 ? 1 : ns);
}

uint64_t decode_workspace_bytes(const rope_decode_params* p, int nsplit) {
    const uint64_t parts = (uint64_t)p->batch * p->hq * nsplit;
    return parts * (uint64_t)(p->head_dim + 2) * 4u;
}

template <typename T, int D>
static void launch_typed(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid = a.compact ? dim3((unsigned)a.nsplit * a.hkv * a.ngroups * a.batch)
                                : dim3(a.nsplit, a.hkv * a.ngroups, a.batch);
    hipLaunchKernelGGL((decode_partial_kernel<T, D>), grid, dim3(64), 0, stream, a);
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.batch * a.hq), dim3(D), 0, stream, a);
}

// ============================================================================ allocation-free entry
// Scratch of rope_decode_attn_fwd_noalloc: the split partials (what rope_decode_attn_fwd keeps
// in the caller's workspace) in a file-scope device array of a fixed size.  Every GPU the
// library runs on holds its own copy, at its own address, until the process ends.  In host
// code the array's name is only a stand-in: kernels and copies use the device address that
// hipGetSymbolAddress returns, looked up once per device.  Nothing in the array must start at
// zero (the partial kernel writes every split that holds keys, the combine kernel reads only
// those), and every call on one GPU shares it, so calls that overlap on a GPU race.
static __device__ __align__(256) unsigned char scratch[ROPE_DECODE_NOALLOC_MAX_BYTES];

hipError_t decode_scratch(hipStream_t stream, void** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (stream) {  // the scratch used is the current device's: the stream must belong to it
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return e;
        if (sdev != dev) return hipErrorInvalidDevice;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = ptr;
    }
    *out = addr[dev];
    return hipSuccess;
}

hipError_t launch_decode(const rope_decode_params* p, hipStream_t stream) {
    DecodeArgs a;
    const int nsplit = decode_num_splits(p);
    a.q = p->q;
    a.cos = p->cos;
    a.sin = p->sin;
    a.rotate = p->cos != nullptr;
    a.interleaved = p->pairing == ROPE_PAIR_INTERLEAVED;
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
    a.chunk = (((p->max_seqlen + nsplit - 1) / nsplit) + 31) & ~31;
    a.bs_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((1 << sh) == p->block_size) a.bs_shift = sh;
    // blocks one split can touch: chunk / block_size + 1 (an unaligned start)
    a.table_regs = (a.chunk / p->block_size + 2) <= 64;
    a.compact = p->batch <= kCompactMaxBatch;
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

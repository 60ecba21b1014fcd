// rope_kv_rms_norm_rope_cache: RMSNorm + RoPE (rotate-half or interleaved pairs) of new K
// rows, written with V into a (possibly paged) KV cache, on gfx950.
//
// The [RoPE-fusion blog] (section 五) names this fused step, the one that runs before
// attention; the RMSNorm is the [RoPE/GQA tutorial]'s (section 八): scale a head row by the
// reciprocal of its root mean square (no mean subtraction), then by the weight gamma.
// Every byte is touched once, so the kernel is HBM bound: per (token, kv head) it reads
// the K and V rows and writes them to the cache; table rows and gamma are shared by all
// heads of a token and stay in the caches.
//
// Thread mapping: a group of G lanes (G a power of two dividing the wavefront) owns one
// (token, head) row; lane l owns the chunks c and c + D/2 with c = l + p*G, 8 columns
// each, so every rotation pair lives in one thread (rotate-half: the two chunks are
// partners; interleaved: each chunk holds whole pairs).  Every load of a thread is issued
// before any arithmetic (more bytes in flight per lane), V is stored straight away, then
// the sum of squares is reduced across the group with xor shuffles.  A whole group leaves
// together (row past the end, or a skipped slot), so every shuffle partner is live.
#include "common.h"

namespace ropefa {

struct KvCacheArgs {
    const void* k;
    const void* v;
    const float* gamma;
    const void* cos;
    const void* sin;
    const int64_t* slots;
    void* kc;
    void* vc;
    int64_t ks[2], vs[2];    // {token, head}
    int64_t kcs[3], vcs[3];  // {block, offset, head}
    int64_t nslots;          // num_blocks * block_size
    int32_t rows;            // ntokens * hkv
    int32_t hkv;
    int32_t head_dim;
    int32_t block_size;
    float eps;
    int32_t group;           // lanes per row, power of two <= 64
    int32_t interleaved;     // pairing: 0 rotate-half, 1 interleaved
};

// K and V are read with load_stream: each byte is read once, and the table rows that the
// other heads of the token re-read stay cached.  The cache rows are written with store_stream
// (nothing here reads them back).

template <typename T, int NP>
__global__ __launch_bounds__(256) void kv_cache_kernel(KvCacheArgs a) {
    const int G = a.group;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = gid / G;
    const int lane = (int)(gid - row * G);
    if (row >= a.rows) return;
    const int t = (int)(row / a.hkv);
    const int h = (int)(row - (int64_t)t * a.hkv);
    const int64_t slot = a.slots[t];
    if (slot < 0 || slot >= a.nslots) return;
    const int64_t blk = slot / a.block_size;
    const int64_t off = slot - blk * a.block_size;

    const int D = a.head_dim;
    const int half = D >> 1;
    const int nchunk = half >> 3;
    const T* krow = reinterpret_cast<const T*>(a.k) + t * a.ks[0] + h * a.ks[1];
    const T* vrow = reinterpret_cast<const T*>(a.v) + t * a.vs[0] + h * a.vs[1];
    const T* crow = reinterpret_cast<const T*>(a.cos) + (int64_t)t * D;
    const T* srow = reinterpret_cast<const T*>(a.sin) + (int64_t)t * D;
    T* kdst = reinterpret_cast<T*>(a.kc) + blk * a.kcs[0] + off * a.kcs[1] + h * a.kcs[2];
    T* vdst = reinterpret_cast<T*>(a.vc) + blk * a.vcs[0] + off * a.vcs[1] + h * a.vcs[2];

    Chunk8<T> kx[NP], ky[NP], vx[NP], vy[NP], cx[NP], cy[NP], sx[NP], sy[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int c = lane + p * G;
        if (c < nchunk) {
            kx[p] = load_stream<T>(krow + c * 8);
            ky[p] = load_stream<T>(krow + c * 8 + half);
            if (a.v) {
                vx[p] = load_stream<T>(vrow + c * 8);
                vy[p] = load_stream<T>(vrow + c * 8 + half);
            }
            cx[p] = load_chunk<T>(crow + c * 8);
            sx[p] = load_chunk<T>(srow + c * 8);
            cy[p] = load_chunk<T>(crow + c * 8 + half);
            sy[p] = load_chunk<T>(srow + c * 8 + half);
        } else {
            kx[p] = ky[p] = zero_chunk<T>();
        }
    }
    if (a.v) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int c = lane + p * G;
            if (c < nchunk) {
                store_stream<T>(vdst + c * 8, vx[p]);
                store_stream<T>(vdst + c * 8 + half, vy[p]);
            }
        }
    }
    float x[NP][8], y[NP][8];
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        unpack<T>(kx[p], x[p]);
        unpack<T>(ky[p], y[p]);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[p][e] * x[p][e] + y[p][e] * y[p][e];
    }
    if (a.gamma) {
        for (int m = G >> 1; m > 0; m >>= 1) ss += __shfl_xor(ss, m, G);
        const float r = rsqrtf(ss / (float)D + a.eps);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int c = lane + p * G;
            if (c < nchunk) {
                float g0[8], g1[8];
                unpack<float>(load_chunk<float>(a.gamma + c * 8), g0);
                unpack<float>(load_chunk<float>(a.gamma + c * 8 + half), g1);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    x[p][e] *= r * g0[e];
                    y[p][e] *= r * g1[e];
                }
            }
        }
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int c = lane + p * G;
        if (c < nchunk) {
            float c0[8], s0[8], c1[8], s1[8];
            unpack<T>(cx[p], c0);
            unpack<T>(sx[p], s0);
            unpack<T>(cy[p], c1);
            unpack<T>(sy[p], s1);
            if (a.interleaved) {
                rotate_interleaved(x[p], c0, s0);
                rotate_interleaved(y[p], c1, s1);
            } else {
                rotate_pair(x[p], y[p], c0, s0, c1, s1);
            }
            store_stream<T>(kdst + c * 8, pack<T>(x[p]));
            store_stream<T>(kdst + c * 8 + half, pack<T>(y[p]));
        }
    }
}

template <typename T>
static void launch_typed(const KvCacheArgs& a, int np, dim3 grid, hipStream_t stream) {
    if (np == 1)
        hipLaunchKernelGGL((kv_cache_kernel<T, 1>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((kv_cache_kernel<T, 2>), grid, dim3(256), 0, stream, a);
}

hipError_t launch_kv_cache(const rope_kv_cache_params* p, hipStream_t stream) {
    KvCacheArgs a;
    a.k = p->k;
    a.v = p->v;
    a.gamma = p->gamma;
    a.cos = p->cos;
    a.sin = p->sin;
    a.slots = p->slots;
    a.kc = p->k_cache;
    a.vc = p->v_cache;
    for (int i = 0; i < 2; ++i) {
        a.ks[i] = p->k_stride[i];
        a.vs[i] = p->v_stride[i];
    }
    for (int i = 0; i < 3; ++i) {
        a.kcs[i] = p->kc_stride[i];
        a.vcs[i] = p->vc_stride[i];
    }
    a.nslots = (int64_t)p->num_blocks * p->block_size;
    a.rows = p->ntokens * p->hkv;
    a.hkv = p->hkv;
    a.head_dim = p->head_dim;
    a.block_size = p->block_size;
    a.eps = p->eps;
    a.interleaved = p->pairing == ROPE_PAIR_INTERLEAVED;
    // chunk pairs per row: head_dim / 16 (2..128); lanes per row: that rounded up to a
    // power of two, at most one wavefront; two pairs per lane above 64 pairs
    const int pairs = p->head_dim / 16;
    int g = 1;
    while (g < pairs && g < 64) g <<= 1;
    a.group = g;
    const int np = (pairs + g - 1) / g;
    if (np > 2) return hipErrorInvalidValue;
    const int64_t threads = (int64_t)a.rows * g;
    const dim3 grid((unsigned)((threads + 255) / 256));
    switch (p->dtype) {
        case ROPE_DT_BF16: launch_typed<__bf16>(a, np, grid, stream); break;
        case ROPE_DT_F16: launch_typed<_Float16>(a, np, grid, stream); break;
        case ROPE_DT_F32: launch_typed<float>(a, np, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ropefa

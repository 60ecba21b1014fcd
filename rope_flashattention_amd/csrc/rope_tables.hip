// rope_tables: the cos/sin tables of the DynamicNTK op, on gfx950.
//
// Formula ([DynamicNTKOperation] page, section 算子功能分析): for each sequence, the
// outer product of its positionIds with its row of InvFreqs gives freq; emb repeats
// freq along the last axis (cat(freq, freq)); the outputs are sin(emb) and cos(emb).
// Linear position scaling ([RoPE-fusion blog], section 5.3) divides positions first.
//
// One thread owns one token and 8 consecutive frequencies i .. i+7: it computes 8
// sin/cos pairs once and stores each pair of 8 results twice (columns i and i + D/2),
// so every transcendental evaluation feeds four stores.  The kernel is bound by HBM
// writes (2 * ntokens * D * sizeof(out)).
#include "common.h"

namespace ropefa {

// Range-reduction constants, derived from pi in extended precision:
//   kHalfPiHi  = fl32(pi/2),  kHalfPiMid = fl32(pi/2 - kHalfPiHi),
//   kHalfPiLo  = fl32(pi/2 - kHalfPiHi - kHalfPiMid),  kTwoOverPi = fl32(2/pi).
// (tests/test_host.py recomputes them.)
constexpr float kHalfPiHi = 0x1.921fb6p+0f;
constexpr float kHalfPiMid = -0x1.777a5cp-25f;
constexpr float kHalfPiLo = -0x1.ee59dap-50f;
constexpr float kTwoOverPi = 0x1.45f306p-1f;
// Arguments up to this magnitude take the fast path below.
constexpr float kFastPathMax = 1048576.0f;  // 2^20

// sin and cos of a float32 angle.
//
// Cody-Waite additive range reduction with fused multiply-adds: k = rint(x * 2/pi),
// r = x - k*pi/2 with pi/2 split in three float32 parts.  The first FMA is exact for
// |x| <= 2^20 (x and k*kHalfPiHi are both multiples of 2^-23 there and |r| < 1), the
// next two add the tail of pi/2, so r keeps nearly full relative precision even close
// to multiples of pi/2.  On |r| <= pi/4 (plus rounding slack) sin and cos are their
// Taylor series truncated after r^11 and r^12 (remainders below 3e-9 relative), in
// Horner form; the quadrant k mod 4 selects and signs the two results.  Larger
// arguments use the device library's sincosf.
__device__ __forceinline__ void rope_sincos(float x, float& s, float& c) {
    if (__builtin_fabsf(x) > kFastPathMax) {
        sincosf(x, &s, &c);
        return;
    }
    const float k = __builtin_rintf(x * kTwoOverPi);
    float r = __builtin_fmaf(-k, kHalfPiHi, x);
    r = __builtin_fmaf(-k, kHalfPiMid, r);
    r = __builtin_fmaf(-k, kHalfPiLo, r);
    const float r2 = r * r;
    // sin r = r + r^3 * (-1/3! + r^2 (1/5! + r^2 (-1/7! + r^2 (1/9! - r^2/11!))))
    float ps = __builtin_fmaf(r2, -1.0f / 39916800.0f, 1.0f / 362880.0f);
    ps = __builtin_fmaf(r2, ps, -1.0f / 5040.0f);
    ps = __builtin_fmaf(r2, ps, 1.0f / 120.0f);
    ps = __builtin_fmaf(r2, ps, -1.0f / 6.0f);
    const float sr = __builtin_fmaf(r * r2, ps, r);
    // cos r = 1 + r^2 * (-1/2! + r^2 (1/4! + r^2 (-1/6! + r^2 (1/8! + r^2 (-1/10! + r^2/12!)))))
    float pc = __builtin_fmaf(r2, 1.0f / 479001600.0f, -1.0f / 3628800.0f);
    pc = __builtin_fmaf(r2, pc, 1.0f / 40320.0f);
    pc = __builtin_fmaf(r2, pc, -1.0f / 720.0f);
    pc = __builtin_fmaf(r2, pc, 1.0f / 24.0f);
    pc = __builtin_fmaf(r2, pc, -0.5f);
    const float cr = __builtin_fmaf(r2, pc, 1.0f);
    const int q = ((int)k) & 3;
    // x = r + q*pi/2:  q=0 (sr, cr)  q=1 (cr, -sr)  q=2 (-sr, -cr)  q=3 (-cr, sr)
    const float a = (q & 1) ? cr : sr;
    const float b = (q & 1) ? sr : cr;
    s = (q & 2) ? -a : a;
    c = ((q + 1) & 2) ? -b : b;
}

struct TablesArgs {
    const int32_t* pos;
    const float* inv_freq;
    void* sin_out;
    void* cos_out;
    int32_t ntokens;
    int32_t head_size;
    int32_t batch;
    float pos_scale;
    int32_t starts[ROPE_MAX_BATCH + 1];  // exclusive prefix sums of seq_lens
};

template <typename TO>
__global__ __launch_bounds__(256) void rope_tables_kernel(TablesArgs a) {
    const int half = a.head_size >> 1;
    const int chunks = half >> 3;  // 8-frequency chunks per row
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)a.ntokens * chunks) return;
    const int t = (int)(gid / chunks);
    const int j = (int)(gid - (int64_t)t * chunks) * 8;
    int b = 0;
#pragma unroll
    for (int i = 1; i < ROPE_MAX_BATCH; ++i) b += (i < a.batch && t >= a.starts[i]) ? 1 : 0;
    // fl32(pos / s): a correctly rounded division
    const float p = __fdiv_rn((float)a.pos[t], a.pos_scale);
    const float* f = a.inv_freq + (int64_t)b * half + j;
    const f32x4 f0 = *reinterpret_cast<const f32x4*>(f);
    const f32x4 f1 = *reinterpret_cast<const f32x4*>(f + 4);
    float sv[8], cv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float fe = e < 4 ? f0[e] : f1[e - 4];
        rope_sincos(__fmul_rn(p, fe), sv[e], cv[e]);  // fl32(p * f), no contraction
    }
    const Chunk8<TO> sc = pack<TO>(sv);
    const Chunk8<TO> cc = pack<TO>(cv);
    TO* so = reinterpret_cast<TO*>(a.sin_out) + (int64_t)t * a.head_size + j;
    TO* co = reinterpret_cast<TO*>(a.cos_out) + (int64_t)t * a.head_size + j;
    store_chunk<TO>(so, sc);
    store_chunk<TO>(so + half, sc);
    store_chunk<TO>(co, cc);
    store_chunk<TO>(co + half, cc);
}

hipError_t launch_rope_tables(const int32_t* pos, const float* inv_freq, const int32_t* seq_lens, int32_t batch,
                              int32_t ntokens, int32_t head_size, float pos_scale, rope_dtype out_dtype,
                              void* sin_out, void* cos_out, hipStream_t stream) {
    TablesArgs a;
    a.pos = pos;
    a.inv_freq = inv_freq;
    a.sin_out = sin_out;
    a.cos_out = cos_out;
    a.ntokens = ntokens;
    a.head_size = head_size;
    a.batch = batch;
    a.pos_scale = pos_scale;
    a.starts[0] = 0;
    for (int i = 0; i < ROPE_MAX_BATCH; ++i) a.starts[i + 1] = a.starts[i] + (i < batch ? seq_lens[i] : 0);
    const int64_t threads = (int64_t)ntokens * (head_size / 16);
    const dim3 block(256);
    const dim3 grid((unsigned)((threads + 255) / 256));
    switch (out_dtype) {
        case ROPE_DT_BF16: hipLaunchKernelGGL(rope_tables_kernel<__bf16>, grid, block, 0, stream, a); break;
        case ROPE_DT_F16: hipLaunchKernelGGL(rope_tables_kernel<_Float16>, grid, block, 0, stream, a); break;
        case ROPE_DT_F32: hipLaunchKernelGGL(rope_tables_kernel<float>, grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ropefa

// Internal helpers shared by the gfx950 kernels of librope_fa (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rope_fa.h"

namespace ropefa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- element conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round-to-nearest-even float -> bf16 / fp16 (hardware conversions on gfx950; fp16 keeps subnormals).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

template <typename T> struct Elem;
template <> struct Elem<__bf16> {
    static constexpr int bytes = 2;
    __device__ static __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ static __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
    // one packed round-to-nearest-even conversion of two floats
    __device__ static __forceinline__ uint32_t pack(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    }
};
template <> struct Elem<_Float16> {
    static constexpr int bytes = 2;
    __device__ static __forceinline__ float lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
    __device__ static __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
    __device__ static __forceinline__ uint32_t pack(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
    }
};
template <> struct Elem<float> { static constexpr int bytes = 4; };

// 8 consecutive elements: 16 bytes for 16-bit types, 32 bytes for float.
template <typename T> struct Chunk8 { u32x4 w; };
template <> struct Chunk8<float> { u32x4 w0, w1; };

template <typename T>
__device__ __forceinline__ Chunk8<T> load_chunk(const T* p) {
    Chunk8<T> c;
    c.w = *reinterpret_cast<const u32x4*>(p);
    return c;
}
template <>
__device__ __forceinline__ Chunk8<float> load_chunk<float>(const float* p) {
    Chunk8<float> c;
    c.w0 = *reinterpret_cast<const u32x4*>(p);
    c.w1 = *reinterpret_cast<const u32x4*>(p + 4);
    return c;
}
// Streaming load of data read once: marked nontemporal, so it does not displace data that is
// re-read (table rows) from the caches.  Measured on this part: a plain copy moves 6.7-7.0
// TB/s with nontemporal loads against 5.5-5.8 with ordinary ones, and the decode step's
// cache reads gain 14%; the rotation of Q and K (rope_qk), which re-reads table rows, is 3%
// slower with them and keeps ordinary loads.
template <typename T>
__device__ __forceinline__ Chunk8<T> load_stream(const T* p) {
    Chunk8<T> c;
    c.w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return c;
}
template <>
__device__ __forceinline__ Chunk8<float> load_stream<float>(const float* p) {
    Chunk8<float> c;
    c.w0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    c.w1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 4));
    return c;
}
// Streaming store of data not read again by this kernel, marked nontemporal.  On this part a
// plain copy gains about 10% when both its loads and its stores are nontemporal (each alone
// gains 1-2%; a write-only fill gains nothing), and the KV-cache step, which reads its rows
// with load_stream, 2.5% from writing the cache this way.
template <typename T>
__device__ __forceinline__ void store_stream(T* p, const Chunk8<T>& c) {
    __builtin_nontemporal_store(c.w, reinterpret_cast<u32x4*>(p));
}
template <>
__device__ __forceinline__ void store_stream<float>(float* p, const Chunk8<float>& c) {
    __builtin_nontemporal_store(c.w0, reinterpret_cast<u32x4*>(p));
    __builtin_nontemporal_store(c.w1, reinterpret_cast<u32x4*>(p + 4));
}
template <typename T>
__device__ __forceinline__ Chunk8<T> zero_chunk() {
    Chunk8<T> c;
    c.w = u32x4{0u, 0u, 0u, 0u};
    return c;
}
template <>
__device__ __forceinline__ Chunk8<float> zero_chunk<float>() {
    Chunk8<float> c;
    c.w0 = u32x4{0u, 0u, 0u, 0u};
    c.w1 = c.w0;
    return c;
}

template <typename T>
__device__ __forceinline__ void unpack(const Chunk8<T>& c, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = Elem<T>::lo(c.w[i]);
        f[2 * i + 1] = Elem<T>::hi(c.w[i]);
    }
}
template <>
__device__ __forceinline__ void unpack<float>(const Chunk8<float>& c, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = __uint_as_float(c.w0[i]);
        f[4 + i] = __uint_as_float(c.w1[i]);
    }
}

template <typename T>
__device__ __forceinline__ Chunk8<T> pack(const float (&f)[8]) {
    Chunk8<T> c;
#pragma unroll
    for (int i = 0; i < 4; ++i) c.w[i] = Elem<T>::pack(f[2 * i], f[2 * i + 1]);
    return c;
}
template <>
__device__ __forceinline__ Chunk8<float> pack<float>(const float (&f)[8]) {
    Chunk8<float> c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        c.w0[i] = __float_as_uint(f[i]);
        c.w1[i] = __float_as_uint(f[4 + i]);
    }
    return c;
}

template <typename T>
__device__ __forceinline__ void store_chunk(T* p, const Chunk8<T>& c) {
    *reinterpret_cast<u32x4*>(p) = c.w;
}
template <>
__device__ __forceinline__ void store_chunk<float>(float* p, const Chunk8<float>& c) {
    *reinterpret_cast<u32x4*>(p) = c.w0;
    *reinterpret_cast<u32x4*>(p + 4) = c.w1;
}

// Rotate-half RoPE of one pair of 8-element chunks: x holds columns [j, j+8) of the
// first half, y the partner columns [j + D/2, j + D/2 + 8); (c0, s0) are the table
// values of the first-half columns and (c1, s1) of the second-half columns.
//   x' = x*c0 - y*s0,   y' = y*c1 + x*s1
// Written as one explicit FMA after one product, so every caller rounds the same way
// whether its table values were loaded or computed.
__device__ __forceinline__ void rotate_pair(float (&x)[8], float (&y)[8], const float (&c0)[8], const float (&s0)[8],
                                            const float (&c1)[8], const float (&s1)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float xv = x[e], yv = y[e];
        x[e] = __builtin_fmaf(xv, c0[e], -__fmul_rn(yv, s0[e]));
        y[e] = __builtin_fmaf(yv, c1[e], __fmul_rn(xv, s1[e]));
    }
}

// The same rotation on packed 16-bit data, 4 dwords (8 elements) per operand, tables in
// the rotate-half form (one cos/sin value per pair): the 16-bit values are widened to
// float32, rotated with a product and an FMA each, and rounded once to T.  Plain VALU
// arithmetic on purpose: gfx950 executes its v_dot2 instructions in the matrix-core
// pipeline, where they neither overlap MFMA work nor issue beside it (measured: a mix of
// MFMAs and dot instructions runs slower than the two one after the other), while
// multiplies and FMAs issue in the gaps between MFMAs.
template <typename T>
__device__ __forceinline__ void rotate_pair_packed(const u32x4& x, const u32x4& y, const u32x4& c, const u32x4& s,
                                                   u32x4& xo, u32x4& yo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float x0 = Elem<T>::lo(x[i]), x1 = Elem<T>::hi(x[i]);
        const float y0 = Elem<T>::lo(y[i]), y1 = Elem<T>::hi(y[i]);
        const float c0 = Elem<T>::lo(c[i]), c1 = Elem<T>::hi(c[i]);
        const float s0 = Elem<T>::lo(s[i]), s1 = Elem<T>::hi(s[i]);
        xo[i] = Elem<T>::pack(__builtin_fmaf(x0, c0, -__fmul_rn(y0, s0)), __builtin_fmaf(x1, c1, -__fmul_rn(y1, s1)));
        yo[i] = Elem<T>::pack(__builtin_fmaf(y0, c0, __fmul_rn(x0, s0)), __builtin_fmaf(y1, c1, __fmul_rn(x1, s1)));
    }
}

// ---------------------------------------------------------------- table values
// Range-reduction constants, derived from pi in extended precision:
//   kHalfPiHi  = fl32(pi/2),  kHalfPiMid = fl32(pi/2 - kHalfPiHi),
//   kHalfPiLo  = fl32(pi/2 - kHalfPiHi - kHalfPiMid),  kTwoOverPi = fl32(2/pi).
// (the host tests recompute them.)
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
//
// The fast path comes in two halves, so that a caller can spread the work of several angles:
// rope_sincos_a reduces the argument and evaluates the sine series, rope_sincos_b the
// cosine series and the quadrant selection.  Run one after the other they are the fast
// path of rope_sincos exactly.
__device__ __forceinline__ void rope_sincos_a(float x, float& k, float& r2, float& sr) {
    k = __builtin_rintf(x * kTwoOverPi);
    float r = __builtin_fmaf(-k, kHalfPiHi, x);
    r = __builtin_fmaf(-k, kHalfPiMid, r);
    r = __builtin_fmaf(-k, kHalfPiLo, r);
    r2 = r * r;
    // sin r = r + r^3 * (-1/3! + r^2 (1/5! + r^2 (-1/7! + r^2 (1/9! - r^2/11!))))
    float ps = __builtin_fmaf(r2, -1.0f / 39916800.0f, 1.0f / 362880.0f);
    ps = __builtin_fmaf(r2, ps, -1.0f / 5040.0f);
    ps = __builtin_fmaf(r2, ps, 1.0f / 120.0f);
    ps = __builtin_fmaf(r2, ps, -1.0f / 6.0f);
    sr = __builtin_fmaf(r * r2, ps, r);
}
__device__ __forceinline__ void rope_sincos_b(float k, float r2, float sr, float& s, float& c) {
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
__device__ __forceinline__ void rope_sincos(float x, float& s, float& c) {
    if (__builtin_fabsf(x) > kFastPathMax) {
        sincosf(x, &s, &c);
        return;
    }
    float k, r2, sr;
    rope_sincos_a(x, k, r2, sr);
    rope_sincos_b(k, r2, sr, s, c);
}

// The angle of one table entry in float32: fl32(fl32(pos / pos_scale) * inv_freq), each
// operation correctly rounded and not contracted ([DynamicNTKOperation], 算子功能分析:
// the outer product of int32 positions with float32 inverse frequencies).
__device__ __forceinline__ float table_angle(int32_t pos, float pos_scale, float inv_freq) {
    return __fmul_rn(__fdiv_rn((float)pos, pos_scale), inv_freq);
}

// Interleaved pairing ([RoPE/GQA tutorial], section 六: adjacent 2-D blocks): elements
// (2k, 2k+1) of a chunk form one pair, rotated with the table values of their own columns,
//   x'_2k = x_2k c_2k - x_2k+1 s_2k,   x'_2k+1 = x_2k+1 c_2k+1 + x_2k s_2k+1.
__device__ __forceinline__ void rotate_interleaved(float (&x)[8], const float (&c)[8], const float (&s)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float a = x[2 * k], b = x[2 * k + 1];
        x[2 * k] = __builtin_fmaf(a, c[2 * k], -__fmul_rn(b, s[2 * k]));
        x[2 * k + 1] = __builtin_fmaf(b, c[2 * k + 1], __fmul_rn(a, s[2 * k + 1]));
    }
}

// The same on packed 16-bit data (4 dwords, one pair per dword), in float32 on the
// vector ALU (see rotate_pair_packed); rounded once to T.
template <typename T>
__device__ __forceinline__ u32x4 rotate_interleaved_packed(const u32x4& x, const u32x4& c, const u32x4& s) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = Elem<T>::lo(x[i]), b = Elem<T>::hi(x[i]);
        o[i] = Elem<T>::pack(__builtin_fmaf(a, Elem<T>::lo(c[i]), -__fmul_rn(b, Elem<T>::lo(s[i]))),
                             __builtin_fmaf(b, Elem<T>::hi(c[i]), __fmul_rn(a, Elem<T>::hi(s[i]))));
    }
    return o;
}

inline int dtype_bytes(rope_dtype dt) {
    switch (dt) {
        case ROPE_DT_F16:
        case ROPE_DT_BF16: return 2;
        case ROPE_DT_F32: return 4;
        default: return 0;
    }
}

}  // namespace ropefa

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
    // a.lo*b.lo + a.hi*b.hi + c in float32
    __device__ static __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
    }
};
template <> struct Elem<_Float16> {
    static constexpr int bytes = 2;
    __device__ static __forceinline__ float lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
    __device__ static __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
    __device__ static __forceinline__ uint32_t pack(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
    }
    __device__ static __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
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
__device__ __forceinline__ void rotate_pair(float (&x)[8], float (&y)[8], const float (&c0)[8], const float (&s0)[8],
                                            const float (&c1)[8], const float (&s1)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float xv = x[e], yv = y[e];
        x[e] = xv * c0[e] - yv * s0[e];
        y[e] = yv * c1[e] + xv * s1[e];
    }
}

// The same rotation on packed 16-bit data, 4 dwords (8 elements) per operand, tables in
// the rotate-half form (one cos/sin value per pair): per element pair (x_j, y_j),
//   x'_j = dot(x_j, y_j ; c_j, -s_j),   y'_j = dot(x_j, y_j ; s_j, c_j)
// with v_perm_b32 building the (x_j, y_j) and table pairs and v_dot2 doing the products in
// float32; results are rounded once to T.
template <typename T>
__device__ __forceinline__ void rotate_pair_packed(const u32x4& x, const u32x4& y, const u32x4& c, const u32x4& s,
                                                   u32x4& xo, u32x4& yo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t xy_e = __builtin_amdgcn_perm(y[i], x[i], 0x05040100u);  // (x_2i,   y_2i)
        const uint32_t xy_o = __builtin_amdgcn_perm(y[i], x[i], 0x07060302u);  // (x_2i+1, y_2i+1)
        const uint32_t ns = s[i] ^ 0x80008000u;                                // -s (both halves)
        const uint32_t cs_e = __builtin_amdgcn_perm(ns, c[i], 0x05040100u);    // (c, -s)
        const uint32_t cs_o = __builtin_amdgcn_perm(ns, c[i], 0x07060302u);
        const uint32_t sc_e = __builtin_amdgcn_perm(c[i], s[i], 0x05040100u);  // (s, c)
        const uint32_t sc_o = __builtin_amdgcn_perm(c[i], s[i], 0x07060302u);
        xo[i] = Elem<T>::pack(Elem<T>::dot2(xy_e, cs_e, 0.0f), Elem<T>::dot2(xy_o, cs_o, 0.0f));
        yo[i] = Elem<T>::pack(Elem<T>::dot2(xy_e, sc_e, 0.0f), Elem<T>::dot2(xy_o, sc_o, 0.0f));
    }
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

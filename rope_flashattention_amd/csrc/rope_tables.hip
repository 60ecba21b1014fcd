// rope_tables: the cos/sin tables of the DynamicNTK op, on gfx950.
//
// Formula ([DynamicNTKOperation] page, section 算子功能分析): for each sequence, the
// outer product of its positionIds with its row of InvFreqs gives freq; emb repeats
// freq along the last axis (cat(freq, freq)); the outputs are sin(emb) and cos(emb).
// Linear position scaling ([RoPE-fusion blog], section 5.3) divides positions first.
//
// One thread evaluates 8 sin/cos pairs and stores each result twice (columns i and
// i + D/2 for the rotate-half layout, 2i and 2i + 1 for the interleaved one); the
// frequencies it takes are chosen so that every store instruction of a wavefront writes
// one contiguous run (see the kernel).  The kernel is bound by HBM writes
// (2 * ntokens * D * sizeof(out)).  The exact-angle mode forms angles and sin/cos in
// float64 and rounds each value once to the output type.
#include "common.h"

namespace ropefa {

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

// float64 -> float32 rounded to odd (truncate, then set the last bit if anything was cut):
// a later round-to-nearest-even to bf16 or fp16 (at least 2 fewer bits) then rounds the
// float64 value correctly, with no double-rounding error.
__device__ __forceinline__ float round_to_odd_f32(double d) {
    const float t = __double2float_rz(d);
    const uint32_t u = __float_as_uint(t) | ((double)t != d ? 1u : 0u);
    return __uint_as_float(u);
}

// 16 bytes of output values (8 16-bit or 4 float32 elements)
template <typename TO>
__device__ __forceinline__ u32x4 piece_bits(const float (&v)[16 / sizeof(TO)]) {
    if constexpr (sizeof(TO) == 4) {
        return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
    } else {
        return pack<TO>(v).w;
    }
}

template <typename TO, int PAIR, bool EXACT>
__global__ __launch_bounds__(256) void rope_tables_kernel(TablesArgs a) {
    // A piece is 16 bytes of one table row: E elements holding FPP frequencies (rotate-half:
    // columns c..c+E-1 of the first half, stored again at c + D/2; interleaved: columns
    // c..c+E-1 = frequencies c/2 .. c/2 + E/2 - 1, each twice).  A thread evaluates 8
    // frequencies, i.e. P pieces; the k-th piece of every lane of a wave is consecutive in
    // memory (pieces wave_base + 64k + lane), so each store instruction writes 1 KB in one run.
    constexpr int E = 16 / sizeof(TO);
    constexpr int FPP = PAIR == ROPE_PAIR_HALF ? E : E / 2;
    constexpr int P = 8 / FPP;
    const int half = a.head_size >> 1;
    const uint32_t npr = (uint32_t)(PAIR == ROPE_PAIR_HALF ? half : a.head_size) / E;  // pieces per row
    const uint32_t total = (uint32_t)a.ntokens * npr;
    const uint32_t wbase = (blockIdx.x * 4u + (threadIdx.x >> 6)) * (64u * P);
    const uint32_t lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < P; ++k) {
        const uint32_t g = wbase + 64u * k + lane;
        if (g >= total) break;
        const int t = (int)(g / npr);
        const int col = (int)(g - (uint32_t)t * npr) * E;  // first column of the piece
        const int fi = PAIR == ROPE_PAIR_HALF ? col : col / 2;  // its first frequency
        int b = 0;
#pragma unroll
        for (int i = 1; i < ROPE_MAX_BATCH; ++i) b += (i < a.batch && t >= a.starts[i]) ? 1 : 0;
        const float* f = a.inv_freq + (int64_t)b * half + fi;
        float fr[FPP];
        if constexpr (FPP == 8) {
            const f32x4 f0 = *reinterpret_cast<const f32x4*>(f);
            const f32x4 f1 = *reinterpret_cast<const f32x4*>(f + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                fr[e] = f0[e];
                fr[e + 4] = f1[e];
            }
        } else if constexpr (FPP == 4) {
            const f32x4 f0 = *reinterpret_cast<const f32x4*>(f);
#pragma unroll
            for (int e = 0; e < 4; ++e) fr[e] = f0[e];
        } else {
            const f32x2 f0 = *reinterpret_cast<const f32x2*>(f);
            fr[0] = f0[0];
            fr[1] = f0[1];
        }
        float sv[FPP], cv[FPP];
        if (EXACT) {
            const double p = (double)a.pos[t] / (double)a.pos_scale;
#pragma unroll
            for (int e = 0; e < FPP; ++e) {
                double sd, cd;
                sincos(p * (double)fr[e], &sd, &cd);
                if (sizeof(TO) == 4) {
                    sv[e] = (float)sd;
                    cv[e] = (float)cd;
                } else {
                    sv[e] = round_to_odd_f32(sd);
                    cv[e] = round_to_odd_f32(cd);
                }
            }
        } else {
            const int32_t pos = a.pos[t];
#pragma unroll
            for (int e = 0; e < FPP; ++e) rope_sincos(table_angle(pos, a.pos_scale, fr[e]), sv[e], cv[e]);
        }
        float se[E], ce[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            se[e] = sv[PAIR == ROPE_PAIR_HALF ? e : e / 2];
            ce[e] = cv[PAIR == ROPE_PAIR_HALF ? e : e / 2];
        }
        const u32x4 sb = piece_bits<TO>(se);
        const u32x4 cb = piece_bits<TO>(ce);
        TO* so = reinterpret_cast<TO*>(a.sin_out) + (int64_t)t * a.head_size + col;
        TO* co = reinterpret_cast<TO*>(a.cos_out) + (int64_t)t * a.head_size + col;
        *reinterpret_cast<u32x4*>(so) = sb;
        *reinterpret_cast<u32x4*>(co) = cb;
        if (PAIR == ROPE_PAIR_HALF) {
            *reinterpret_cast<u32x4*>(so + half) = sb;
            *reinterpret_cast<u32x4*>(co + half) = cb;
        }
    }
}

template <typename TO>
static void launch_tables_typed(const TablesArgs& a, int pairing, int angle_mode, dim3 grid, hipStream_t stream) {
    const int key = pairing * 2 + angle_mode;
    switch (key) {
        case 0: hipLaunchKernelGGL((rope_tables_kernel<TO, ROPE_PAIR_HALF, false>), grid, dim3(256), 0, stream, a); break;
        case 1: hipLaunchKernelGGL((rope_tables_kernel<TO, ROPE_PAIR_HALF, true>), grid, dim3(256), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((rope_tables_kernel<TO, ROPE_PAIR_INTERLEAVED, false>), grid, dim3(256), 0, stream, a); break;
        case 3: hipLaunchKernelGGL((rope_tables_kernel<TO, ROPE_PAIR_INTERLEAVED, true>), grid, dim3(256), 0, stream, a); break;
    }
}

hipError_t launch_rope_tables(const int32_t* pos, const float* inv_freq, const int32_t* seq_lens, int32_t batch,
                              int32_t ntokens, int32_t head_size, float pos_scale, rope_dtype out_dtype,
                              int pairing, int angle_mode, void* sin_out, void* cos_out, hipStream_t stream) {
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
    // 8 frequencies per thread: head_size / 16 threads per row
    const int64_t threads = (int64_t)ntokens * (head_size / 16);
    const dim3 grid((unsigned)((threads + 255) / 256));
    switch (out_dtype) {
        case ROPE_DT_BF16: launch_tables_typed<__bf16>(a, pairing, angle_mode, grid, stream); break;
        case ROPE_DT_F16: launch_tables_typed<_Float16>(a, pairing, angle_mode, grid, stream); break;
        case ROPE_DT_F32: launch_tables_typed<float>(a, pairing, angle_mode, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ropefa

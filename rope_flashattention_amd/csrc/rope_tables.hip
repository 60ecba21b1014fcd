// rope_tables: the cos/sin tables of the DynamicNTK op, on gfx950.
//
// Formula ([DynamicNTKOperation] page, section 算子功能分析): for each sequence, the
// outer product of its positionIds with its row of InvFreqs gives freq; emb repeats
// freq along the last axis (cat(freq, freq)); the outputs are sin(emb) and cos(emb).
// Linear position scaling ([RoPE-fusion blog], section 5.3) divides positions first.
//
// One thread owns one token and 8 consecutive frequencies i .. i+7: it computes 8
// sin/cos pairs once and stores each result twice (columns i and i + D/2 for the
// rotate-half layout, 2i and 2i + 1 for the interleaved one), so every transcendental
// evaluation feeds four stores.  The kernel is bound by HBM writes
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

template <typename TO, int PAIR, bool EXACT>
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
    const float* f = a.inv_freq + (int64_t)b * half + j;
    const f32x4 f0 = *reinterpret_cast<const f32x4*>(f);
    const f32x4 f1 = *reinterpret_cast<const f32x4*>(f + 4);
    float sv[8], cv[8];
    if (EXACT) {
        const double p = (double)a.pos[t] / (double)a.pos_scale;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            double sd, cd;
            sincos(p * (double)(e < 4 ? f0[e] : f1[e - 4]), &sd, &cd);
            if (sizeof(TO) == 4) {
                sv[e] = (float)sd;
                cv[e] = (float)cd;
            } else {
                sv[e] = round_to_odd_f32(sd);
                cv[e] = round_to_odd_f32(cd);
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) rope_sincos(table_angle(a.pos[t], a.pos_scale, e < 4 ? f0[e] : f1[e - 4]), sv[e], cv[e]);
    }
    TO* so = reinterpret_cast<TO*>(a.sin_out) + (int64_t)t * a.head_size;
    TO* co = reinterpret_cast<TO*>(a.cos_out) + (int64_t)t * a.head_size;
    if (PAIR == ROPE_PAIR_HALF) {
        // frequency i fills columns i and i + D/2
        const Chunk8<TO> sc = pack<TO>(sv);
        const Chunk8<TO> cc = pack<TO>(cv);
        store_chunk<TO>(so + j, sc);
        store_chunk<TO>(so + j + half, sc);
        store_chunk<TO>(co + j, cc);
        store_chunk<TO>(co + j + half, cc);
    } else {
        // frequency i fills columns 2i and 2i + 1
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
            float s2[8], c2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                s2[e] = sv[4 * hlf + e / 2];
                c2[e] = cv[4 * hlf + e / 2];
            }
            store_chunk<TO>(so + 2 * j + 8 * hlf, pack<TO>(s2));
            store_chunk<TO>(co + 2 * j + 8 * hlf, pack<TO>(c2));
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

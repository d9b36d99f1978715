// Internal declarations shared by the HIP sources of liblq.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lq.h"

namespace lq {

// Kernel launchers.  Arguments were validated by the C ABI layer; each
// returns the hipError_t of its launch.
hipError_t launch_decode(const lq_dims& d, const lq_state& st, int pos, const float* q,
                         const float* k, const float* v, const float* alpha, const float* beta,
                         float* o, hipStream_t s);
hipError_t launch_flush(const lq_dims& d, const lq_state& st, int n_buffered, float* h_out,
                        hipStream_t s);
hipError_t launch_quantize(const lq_dims& d, const float* h, const lq_state& st, hipStream_t s);
hipError_t launch_dequantize(const lq_dims& d, const lq_state& st, float* h_out, hipStream_t s);
hipError_t launch_fp32_recurrence(const lq_dims& d, float* h, int T, const float* q,
                                  const float* k, const float* v, const float* alpha,
                                  const float* beta, float* o, hipStream_t s);

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

// Workgroup barrier that orders LDS traffic only: global loads issued before
// it stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum / max over aligned groups of G lanes (G a power of two <= 64); every
// lane of the group receives the result.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <int G>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}

// N consecutive floats from an address aligned to 4*N bytes when N is a
// multiple of 4 (or 2), as 128-bit (64-bit) loads.
template <int N>
__device__ __forceinline__ void load_floats(const float* __restrict__ p, float (&x)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            float4 t = reinterpret_cast<const float4*>(p)[i];
            x[4 * i] = t.x; x[4 * i + 1] = t.y; x[4 * i + 2] = t.z; x[4 * i + 3] = t.w;
        }
    } else if constexpr (N % 2 == 0) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            float2 t = reinterpret_cast<const float2*>(p)[i];
            x[2 * i] = t.x; x[2 * i + 1] = t.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = p[i];
    }
}

template <int N>
__device__ __forceinline__ void store_floats(float* __restrict__ p, const float (&x)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i)
            reinterpret_cast<float4*>(p)[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
    } else if constexpr (N % 2 == 0) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i)
            reinterpret_cast<float2*>(p)[i] = make_float2(x[2 * i], x[2 * i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) p[i] = x[i];
    }
}

// Signed byte e (0..3) of a 32-bit word, as float.
__device__ __forceinline__ float sbyte(uint32_t w, int e) {
    return (float)(int32_t)(int8_t)(uint8_t)(w >> (8 * e));
}

// Window-size bucket a kernel is instantiated for.
inline int wbucket(int W) { return W <= 4 ? 4 : W <= 8 ? 8 : W <= 16 ? 16 : 32; }

}  // namespace lq

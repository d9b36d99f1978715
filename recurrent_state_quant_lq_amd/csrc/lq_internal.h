// Internal declarations shared by the HIP sources of liblq.so (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lq.h"

namespace lq {

// Kernel launchers.  Arguments were validated by the C ABI layer; each
// returns the hipError_t of its launch.
// pos_dev / n_dev: per-batch-row device arrays (ragged windows) or null.
hipError_t launch_decode(const lq_dims& d, const lq_state& st, int pos, const int32_t* pos_dev,
                         const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, void* o, hipStream_t s);
hipError_t launch_flush(const lq_dims& d, const lq_state& st, int n_buffered, const int32_t* n_dev,
                        float* h_out, hipStream_t s);
// Decode of one token into slot pos, then the flush of pos + 1 slots, in one launch
// (pos_dev: per-batch-row positions, rows outside [0, W) skipped; or null).
hipError_t launch_decode_flush(const lq_dims& d, const lq_state& st, int pos, const int32_t* pos_dev,
                               const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, void* o, float* h_out, hipStream_t s);
hipError_t launch_quantize(const lq_dims& d, const float* h, const lq_state& st, hipStream_t s);
hipError_t launch_dequantize(const lq_dims& d, const lq_state& st, float* h_out, hipStream_t s);
// Quantized-state records (lq_gdn_state_pack / unpack).
size_t checkpoint_head_bytes(const lq_dims& d);
hipError_t launch_checkpoint(const lq_dims& d, const lq_state& st, void* blob, bool pack, hipStream_t s);
// Chunked fp32 prefill of T tokens, state h updated in place (lq_gdn_prefill).
hipError_t launch_prefill(const lq_dims& d, float* h, int T, const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta, void* o, hipStream_t s);
hipError_t launch_fp32_recurrence(const lq_dims& d, float* h, int T, const void* q,
                                  const void* k, const void* v, const float* alpha,
                                  const float* beta, void* o, hipStream_t s);

// Streaming-read reference (lq_measure_stream_read); arguments validated.
hipError_t launch_stream_read(const void* src, size_t slice_bytes, int n_slices, int mode, int grid,
                              void* sink, size_t write_bytes, hipStream_t s);

// Kernel timing (lq_timing_*): when recording is on, hands out the event
// pair of the next launch of `family` and returns true.
bool timing_slot(int family, hipEvent_t* start, hipEvent_t* stop);

// Every kernel of the library is launched through here.
template <typename... Params, typename... Args>
hipError_t launch_kernel(int family, void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t s,
                         Args... args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (timing_slot(family, &e0, &e1))
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
    return hipGetLastError();
}

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// barriers
// ---------------------------------------------------------------------------

// Workgroup barrier that orders LDS traffic only: global loads issued before
// it may stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Waits for every outstanding memory operation of this wave (LDS copies
// included), then a workgroup barrier with full fences.  Data copied to LDS by
// global_load_lds are readable after it.  (LDS copies and register loads do
// not complete in order with each other, so a partial vmcnt wait cannot tell
// that an LDS copy has landed.)
__device__ __forceinline__ void all_loads_barrier() {
    __builtin_amdgcn_s_waitcnt(0);                              // vmcnt(0) expcnt(0) lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ---------------------------------------------------------------------------
// cross-lane
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <- lane 7-i within 8
constexpr int DPP_MIRROR = 0x140;       // lane i <- lane 15-i within 16
constexpr int DPP_SHL1 = 0x101;         // lane i <- lane i+1 within 16
constexpr int DPP_SHL2 = 0x102;         // lane i <- lane i+2 within 16
constexpr int DPP_ROW_BCAST = 0x150;    // + k: every lane of a 16-lane row <- lane k of that row

// x of lane k * STRIDE of this lane's 16-lane row, for k = 0..N-1, into out[k].
template <int N, int STRIDE = 1, int K = 0>
__device__ __forceinline__ void row_bcast_all(float x, float* out) {
    // every lane has a source lane here, so no fallback value is needed
    out[K] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), DPP_ROW_BCAST + K * STRIDE, 0xf, 0xf, false));
    if constexpr (K + 1 < N) row_bcast_all<N, STRIDE, K + 1>(x, out);
}

__device__ __forceinline__ float swz_xor16(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}

// Totals over the four 16-lane rows of a wave for four values at once, with
// the gfx950 row swaps (v_permlane32_swap: upper half of the first operand
// <-> lower half of the second; v_permlane16_swap: odd rows of the first <->
// even rows of the second).  Row r of the result holds the sum over all 64
// lanes' rows of (a, b, c, d)[r], at the lane's position within the row.
__device__ __forceinline__ float rows_sum4(float a, float b, float c, float d) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(c), false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(b), __float_as_uint(d), false, false);
    // rows of x: a0+a2, a1+a3, c0+c2, c1+c3; of y: the same for b and d
    const float x = __uint_as_float(s0[0]) + __uint_as_float(s0[1]);
    const float y = __uint_as_float(s1[0]) + __uint_as_float(s1[1]);
    const auto s2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(s2[0]) + __uint_as_float(s2[1]);
}

// Sum / max over aligned groups of G lanes (G a power of two <= 64); every
// lane of a group receives the result.  After the two quad steps all lanes
// of a quad agree, so the mirror steps pair whole quads, then whole halves.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (G >= 2) x += dpp<DPP_XOR1>(x);
    if constexpr (G >= 4) x += dpp<DPP_XOR2>(x);
    if constexpr (G >= 8) x += dpp<DPP_HALF_MIRROR>(x);
    if constexpr (G >= 16) x += dpp<DPP_MIRROR>(x);
    if constexpr (G >= 32) x += swz_xor16(x);
    if constexpr (G >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

template <int G>
__device__ __forceinline__ float group_max(float x) {
    if constexpr (G >= 2) x = fmaxf(x, dpp<DPP_XOR1>(x));
    if constexpr (G >= 4) x = fmaxf(x, dpp<DPP_XOR2>(x));
    if constexpr (G >= 8) x = fmaxf(x, dpp<DPP_HALF_MIRROR>(x));
    if constexpr (G >= 16) x = fmaxf(x, dpp<DPP_MIRROR>(x));
    if constexpr (G >= 32) x = fmaxf(x, swz_xor16(x));
    if constexpr (G >= 64) x = fmaxf(x, __shfl_xor(x, 32, 64));
    return x;
}

// Maxima of NON-NEGATIVE floats handled as their bit patterns: for x, y >= 0
// (zeros, subnormals, normals, +inf) x < y exactly when bits(x) < bits(y), and
// the unsigned max folds into one v_max_u32 with a DPP source per step.
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <int G>
__device__ __forceinline__ uint32_t group_umax(uint32_t x) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "groups within a 16-lane row");
    if constexpr (G >= 2) x = umax(x, (uint32_t)dpp_i<DPP_XOR1>((int)x));
    if constexpr (G >= 4) x = umax(x, (uint32_t)dpp_i<DPP_XOR2>((int)x));
    if constexpr (G >= 8) x = umax(x, (uint32_t)dpp_i<DPP_HALF_MIRROR>((int)x));
    if constexpr (G >= 16) x = umax(x, (uint32_t)dpp_i<DPP_MIRROR>((int)x));
    return x;
}

// Wave-uniform unsigned maximum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
    x = group_umax<16>(x);
    const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
    const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
    return umax(umax(a, b), umax(c, d));
}

// Max of |x| over aligned groups of G lanes, as a float (every lane of a
// group receives it).
template <int G>
__device__ __forceinline__ float group_absmax(float x) {
    return __uint_as_float(group_umax<G>(__float_as_uint(x) & 0x7fffffffu));
}

// ---------------------------------------------------------------------------
// rounding to int8 through the 1.5 * 2^23 offset
// ---------------------------------------------------------------------------
// For |y| <= 2^22, y + 1.5*2^23 rounded to fp32 (round to nearest, ties to
// even) is 1.5*2^23 + rint(y) exactly, and the low byte of its bit pattern is
// rint(y) as a two's-complement byte once the sum is clamped to
// 1.5*2^23 +- 127.
constexpr float kRoundOff = 12582912.0f;   // 1.5 * 2^23


// ---------------------------------------------------------------------------
// memory
// ---------------------------------------------------------------------------

// N consecutive floats as 128-bit (64-bit) accesses when N allows it; the
// address must be aligned to the access size.
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

// bf16 token I/O.  A bf16 value is the upper half of an fp32 bit pattern:
// widening is exact; narrowing rounds to nearest, ties to even (adding
// 0x7fff plus the lowest kept bit carries into the kept half exactly when
// the dropped half is above one half, or equal with an odd kept half), and
// keeps NaNs quiet.
__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Streaming loads (non-temporal): data read once per launch (the int8 state,
// the buffered rows), kept out of the caches' working set.
template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }

// Streaming stores (non-temporal): results written once per launch and read
// by a later one.  Written through to memory during the kernel instead of
// staying dirty in the XCD's L2 until the end-of-kernel write-back.
template <typename T>
__device__ __forceinline__ void st_nt(T* p, T v) { __builtin_nontemporal_store(v, p); }
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_nt4(float* p, float a, float b, float c, float d) {
    __builtin_nontemporal_store(f32x4{a, b, c, d}, reinterpret_cast<f32x4*>(p));
}

// Token vectors staged in LDS: fp32 (TI = float), or bf16 (TI = uint16_t)
// packed into the first half of an fp32-sized segment.
template <typename TI>
__device__ __forceinline__ float seg_ld(const float* seg, int i) {
    if constexpr (sizeof(TI) == 4) return seg[i];
    else return bf16_to_f32(reinterpret_cast<const uint16_t*>(seg)[i]);
}
template <int N, typename TI>
__device__ __forceinline__ void seg_ld_n(const float* seg, int i0, float (&x)[N]) {
    if constexpr (sizeof(TI) == 4) {
        load_floats<N>(seg + i0, x);
    } else if constexpr (N % 2 != 0) {
#pragma unroll
        for (int e = 0; e < N; ++e) x[e] = seg_ld<TI>(seg, i0 + e);
    } else {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(seg) + i0 / 2;
#pragma unroll
        for (int e = 0; e < N / 2; ++e) {
            const uint32_t w = p[e];
            x[2 * e] = __uint_as_float(w << 16);
            x[2 * e + 1] = __uint_as_float(w & 0xffff0000u);
        }
    }
}
// One output element (fp32 or bf16, round to nearest even).
template <typename TI>
__device__ __forceinline__ void tok_st(void* base, size_t i, float x) {
    if constexpr (sizeof(TI) == 4) st_nt(reinterpret_cast<float*>(base) + i, x);
    else st_nt(reinterpret_cast<uint16_t*>(base) + i, f32_to_bf16(x));
}
// One input element from global memory.
template <typename TI>
__device__ __forceinline__ float tok_ld(const void* base, size_t i) {
    if constexpr (sizeof(TI) == 4) return reinterpret_cast<const float*>(base)[i];
    else return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
}

// Global -> LDS without registers.  Lane l of the wave writes
// lds_wave_base + 16*l (dma16) or + 4*l (dma4) bytes; lds_wave_base must be
// wave-uniform.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base,
                                     16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* src, void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base,
                                     4, 0, 0);
}

// Signed byte e (0..3) of a 32-bit word, as float.
__device__ __forceinline__ float sbyte(uint32_t w, int e) {
    return (float)(int32_t)(int8_t)(uint8_t)(w >> (8 * e));
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t)(a & 255) | ((uint32_t)(b & 255) << 8) | ((uint32_t)(c & 255) << 16) |
           ((uint32_t)(d & 255) << 24);
}

// ---------------------------------------------------------------------------
// three-digit int8 expansion for the int8 MFMA products
// ---------------------------------------------------------------------------
// With inv = 127 / M (M >= max |x| of the block), x = (M/127)(d0 + d1/254 +
// d2/254^2) to within (M/127)*2^-16, i.e. to fp32 precision relative to the
// block's largest element.  Products of the digits with int8 state bytes sum
// exactly in int32, so the three partial sums recombine to an fp32-accurate
// product with the int8 matrix.
constexpr float kDigitW1 = 1.0f / 254.0f;
constexpr float kDigitW2 = 1.0f / (254.0f * 254.0f);

__device__ __forceinline__ void digits3(float x, float inv, int& d0, int& d1, int& d2) {
    const float u = x * inv;
    const float f0 = fminf(fmaxf(rintf(u), -127.0f), 127.0f);
    const float r1 = (u - f0) * 254.0f;
    const float f1 = fminf(fmaxf(rintf(r1), -127.0f), 127.0f);
    const float r2 = (r1 - f1) * 254.0f;
    const float f2 = fminf(fmaxf(rintf(r2), -127.0f), 127.0f);
    d0 = (int)f0;
    d1 = (int)f1;
    d2 = (int)f2;
}

// The same three digits as offset words (the low byte of each is the digit).
// |x * inv| <= 127 rounds to |d0| <= 127 and each remainder stays within
// 254 * 0.5 = 127, so no clamping is needed.
__device__ __forceinline__ void digits3_words(float x, float inv, uint32_t& w0, uint32_t& w1,
                                              uint32_t& w2) {
    const float u = x * inv;
    const float z0 = u + kRoundOff;
    const float r1 = (u - (z0 - kRoundOff)) * 254.0f;
    const float z1 = r1 + kRoundOff;
    const float r2 = (r1 - (z1 - kRoundOff)) * 254.0f;
    const float z2 = r2 + kRoundOff;
    w0 = __float_as_uint(z0);
    w1 = __float_as_uint(z1);
    w2 = __float_as_uint(z2);
}

// ---------------------------------------------------------------------------
// storage order of the int8 state
// ---------------------------------------------------------------------------
// Byte (i, j) of a head's dk x dv int8 state (key channel i, value channel j)
// sits at sq_off<DK>(i, j) of the head's dk*dv bytes: the A-operand order of
// the decode's v_mfma_i32_16x16x64_i8 tiles, so each wave reads 1 KB
// contiguous bytes per MFMA operand.  Column tile T = j/16 and K step ks =
// i/64 own a block of G*256 bytes (G = min(4, dk/16) groups of 16 channels);
// within it, the 16-byte piece lg*16 + j%16 holds channels ks*64 + lg*16 ..
// +15 of column j, lg = (i%64)/16.  Runs of up to 16 consecutive channels of
// one column (aligned to their length) are contiguous.
// Bytes between the same (row, column-in-tile) of consecutive 16-column tiles:
// sq_off(i, 16 t + c) = sq_off(i, c) + t * sq_tile_stride<DK>().
template <int DK>
__host__ __device__ constexpr uint32_t sq_tile_stride() {
    return (uint32_t)(((DK + 63) / 64) * (DK / 16 < 4 ? DK / 16 : 4) * 256);
}

template <int DK>
__host__ __device__ constexpr uint32_t sq_off(int i, int j) {
    constexpr int G = DK / 16 < 4 ? DK / 16 : 4;
    constexpr int KS = (DK + 63) / 64;
    return (uint32_t)(((((j >> 4) * KS + (i >> 6)) * G + ((i & 63) >> 4)) * 16 + (j & 15)) * 16 + (i & 15));
}

static_assert(sq_off<128>(77, 16 * 5 + 9) == sq_off<128>(77, 9) + 5 * sq_tile_stride<128>(), "tile stride");
static_assert(sq_off<64>(33, 16 * 3 + 2) == sq_off<64>(33, 2) + 3 * sq_tile_stride<64>(), "tile stride");
static_assert(sq_off<16>(11, 4) == sq_off<16>(11, 4) + 0 * sq_tile_stride<16>(), "tile stride");

// Window-size bucket a kernel is instantiated for.
inline int wbucket(int W) { return W <= 4 ? 4 : W <= 8 ? 8 : W <= 16 ? 16 : 32; }

}  // namespace lq

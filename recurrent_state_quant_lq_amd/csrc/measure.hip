// measure.hip -- streaming-read reference kernels (measurement support, not
// part of the method; gfx950).
//
// They read the same number of bytes per workgroup as a decode launch reads
// per head, with nothing else to do, so their duration is what a bare read of
// that shape costs on the GPU at hand: the ceiling any kernel of that launch
// shape can reach.
//
//   one_shot: one 256-lane workgroup per slice (the decode's shape: one
//             workgroup per head, every load issued before any is used);
//   persistent: a fixed grid that walks the slices (grid-stride), the
//             streaming pattern with the fewest launch and tail effects.
//
// Each workgroup XOR-folds what it read and writes `write_bytes` bytes of the
// result (the decode writes about 1.5 KB per head), so no load is dead.
#include "lq_internal.h"

namespace lq {
namespace {

constexpr int NT = 256;

struct ReadArgs {
    const v4i* src;
    v4i* sink;
    uint32_t slice_v4;        // 16-byte pieces per slice
    uint32_t write_v4;        // 16-byte pieces written per slice (<= NT)
    uint32_t n_slices;
};

// Folds slice s into lanes' accumulators: LPL pieces per lane, all issued
// before the first use.
template <int LPL>
__device__ __forceinline__ v4i read_slice(const ReadArgs& a, uint32_t s) {
    const v4i* p = a.src + (size_t)s * a.slice_v4;
    v4i x[LPL];
#pragma unroll
    for (int i = 0; i < LPL; ++i) {
        const uint32_t e = i * NT + threadIdx.x;
        x[i] = e < a.slice_v4 ? ld_nt(p + e) : v4i{0, 0, 0, 0};
    }
    v4i acc = x[0];
#pragma unroll
    for (int i = 1; i < LPL; ++i) acc ^= x[i];
    return acc;
}

__device__ __forceinline__ void write_slice(const ReadArgs& a, uint32_t s, v4i acc) {
    if (threadIdx.x < a.write_v4) st_nt(a.sink + (size_t)s * a.write_v4 + threadIdx.x, acc);
}

template <int LPL>
__global__ __launch_bounds__(NT) void read_one_shot_kernel(ReadArgs a) {
    const uint32_t s = blockIdx.x;
    write_slice(a, s, read_slice<LPL>(a, s));
}

template <int LPL>
__global__ __launch_bounds__(NT) void read_persistent_kernel(ReadArgs a) {
    for (uint32_t s = blockIdx.x; s < a.n_slices; s += gridDim.x) write_slice(a, s, read_slice<LPL>(a, s));
}

template <int LPL>
hipError_t launch_lpl(const ReadArgs& a, int mode, int grid, hipStream_t s) {
    if (mode == 0)
        return launch_kernel(LQ_KERNEL_MEASURE, read_one_shot_kernel<LPL>, dim3(a.n_slices), dim3(NT), s, a);
    return launch_kernel(LQ_KERNEL_MEASURE, read_persistent_kernel<LPL>, dim3(grid), dim3(NT), s, a);
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t slice_bytes, int n_slices, int mode, int grid,
                              void* sink, size_t write_bytes, hipStream_t s) {
    ReadArgs a{static_cast<const v4i*>(src), static_cast<v4i*>(sink), (uint32_t)(slice_bytes / 16),
               (uint32_t)(write_bytes / 16), (uint32_t)n_slices};
    const size_t lpl = (a.slice_v4 + NT - 1) / NT;
    if (lpl <= 2) return launch_lpl<2>(a, mode, grid, s);
    if (lpl <= 4) return launch_lpl<4>(a, mode, grid, s);
    if (lpl <= 8) return launch_lpl<8>(a, mode, grid, s);
    return launch_lpl<16>(a, mode, grid, s);
}

}  // namespace lq

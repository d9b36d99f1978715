// checkpoint.hip -- copy the quantized state to and from a contiguous blob
// (gfx950), e.g. for prefix-cache checkpoints at window boundaries.
//
// News article ("A linear-attention method cuts state ...", paragraph 5): the
// stored state is about 1.19 bytes per value including its scales and
// correction terms; this is that stored form, one contiguous record per head.
//
// Record of one head (head_bytes, a multiple of 16):
//     sq   dk*dv bytes   int8, in the state's storage order (sq_off)
//     r    4*dk          fp32 row scales
//     s    4*dv          fp32 column scales
//     cv   4*C*dv        fp32 compensator rows
//     idx  4*C           int32 compensator row indices
//     zero padding to a multiple of 16 bytes
// Records are in (b, h) order, so the H records of one sequence are adjacent.
// One workgroup per head; 16-byte copies for every segment but idx.
#include "lq_internal.h"

namespace lq {
namespace {

struct CkArgs {
    int8_t* sq;
    float* r;
    float* s;
    int32_t* idx;
    float* cv;
    char* blob;
    size_t head_bytes;
    int dk, dv, C;
    int pack;   // 1: state -> blob, 0: blob -> state
};

__device__ __forceinline__ void copy16(char* dst, const char* src, size_t bytes, int t) {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    for (size_t i = t; i < bytes / 16; i += 256) d4[i] = s4[i];
}

__global__ __launch_bounds__(256) void checkpoint_kernel(CkArgs a) {
    const size_t head = blockIdx.x;
    const int t = threadIdx.x;
    const size_t dk = a.dk, dv = a.dv, C = a.C;
    char* rec = a.blob + head * a.head_bytes;
    char* st[4] = {reinterpret_cast<char*>(a.sq + head * dk * dv), reinterpret_cast<char*>(a.r + head * dk),
                   reinterpret_cast<char*>(a.s + head * dv), reinterpret_cast<char*>(a.cv + head * C * dv)};
    const size_t len[4] = {dk * dv, 4 * dk, 4 * dv, 4 * C * dv};
    size_t off = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        if (a.pack)
            copy16(rec + off, st[g], len[g], t);
        else
            copy16(st[g], rec + off, len[g], t);
        off += len[g];
    }
    int32_t* ri = reinterpret_cast<int32_t*>(rec + off);
    int32_t* si = a.idx + head * C;
    if (t < (int)C) {
        if (a.pack)
            ri[t] = si[t];
        else
            si[t] = ri[t];
    }
    off += 4 * C;
    if (a.pack)
        for (size_t i = off + t; i < a.head_bytes; i += 256) rec[i] = 0;
}

}  // namespace

size_t checkpoint_head_bytes(const lq_dims& d) {
    const size_t b = (size_t)d.dk * d.dv + 4 * (size_t)d.dk + 4 * (size_t)d.dv +
                     4 * (size_t)d.C * d.dv + 4 * (size_t)d.C;
    return (b + 15) / 16 * 16;
}

hipError_t launch_checkpoint(const lq_dims& d, const lq_state& st, void* blob, bool pack, hipStream_t s) {
    CkArgs args{st.sq, st.row_scale, st.col_scale, st.comp_idx, st.comp_val, static_cast<char*>(blob),
                checkpoint_head_bytes(d), d.dk, d.dv, d.C, pack ? 1 : 0};
    return launch_kernel(LQ_KERNEL_CHECKPOINT, checkpoint_kernel, dim3((unsigned)d.B * (unsigned)d.H), dim3(256),
                         s, args);
}

}  // namespace lq

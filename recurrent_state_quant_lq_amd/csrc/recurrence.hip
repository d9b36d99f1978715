// recurrence.hip -- dense fp32-state gated delta rule over T tokens (gfx950).
//
// The FP32-state baseline the LeapQuant abstract (HFEPX paper page,
// "Abstract") compares against, and the prefill that produces a starting
// state.  Per token and (b, h):
//     p = (D H)^T k,  z = (D H)^T q,  u = beta (v - p),
//     H <- D H + k u^T,  o = H^T q = z + u (k . q).
// One workgroup per (b, h) keeps the fp32 state in registers for all T tokens
// (64 KB per head at dk = dv = 128: 64 floats per lane), reads it once and
// writes it once.  Thread t holds rows p*RPP + t/CPR4 (p < PASSES) and the
// four columns 4*(t % CPR4) .. +3.
#include "lq_internal.h"

namespace lq {
namespace {

struct RecArgs {
    float* h;
    const void* q;            // q, k, v, o: fp32 or bf16 (the kernel's TI)
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    void* o;
    int T;
    size_t heads;   // B*H: stride between tokens, in heads
};

template <int DK, int DV, bool KDA, int NT, typename TI>
__global__ __launch_bounds__(NT) void fp32_rec_kernel(RecArgs a) {
    constexpr int CPR4 = DV / 4;
    constexpr int RPP = NT / CPR4;
    constexpr int PASSES = DK / RPP;
    constexpr int NW = NT / 64;
    constexpr int GPW = 64 / CPR4 > 0 ? 64 / CPR4 : 1;   // row groups per wave
    static_assert(NT % CPR4 == 0 && DK % RPP == 0 && CPR4 <= 64, "tiling");
    constexpr int GD = KDA ? DK : 1;

    __shared__ __align__(16) float s_p[NW][DV];
    __shared__ __align__(16) float s_z[NW][DV];
    __shared__ float s_kq[NW];

    const int t = threadIdx.x;
    const int lane = t & 63, w = t >> 6;
    const size_t head = blockIdx.x;
    const int rg = t / CPR4;
    const int c0 = (t % CPR4) * 4;

    float* h = a.h + head * (size_t)DK * DV;
    // the state is read once and written once per launch: streamed (a row's 32
    // lanes cover 512 contiguous bytes, so the stores are whole lines)
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    float4 H[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const f32x4v x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(h + (size_t)(p * RPP + rg) * DV + c0));
        H[p] = make_float4(x[0], x[1], x[2], x[3]);
    }

    for (int tok = 0; tok < a.T; ++tok) {
        const size_t th = (size_t)tok * a.heads + head;
        const float* al = a.alpha + th * GD;
        const float beta = a.beta[th];
        float4 vv;
        if constexpr (sizeof(TI) == 4)
            vv = *reinterpret_cast<const float4*>(static_cast<const float*>(a.v) + th * DV + c0);
        else
            vv = make_float4(tok_ld<TI>(a.v, th * DV + c0), tok_ld<TI>(a.v, th * DV + c0 + 1),
                             tok_ld<TI>(a.v, th * DV + c0 + 2), tok_ld<TI>(a.v, th * DV + c0 + 3));
        float kr[PASSES], qr[PASSES], dr[PASSES];
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int row = p * RPP + rg;
            kr[p] = tok_ld<TI>(a.k, th * DK + row);
            qr[p] = tok_ld<TI>(a.q, th * DK + row);
            dr[p] = KDA ? al[row] : al[0];
        }
        float kq = 0.0f;
        if (t < DK) kq = tok_ld<TI>(a.k, th * DK + t) * tok_ld<TI>(a.q, th * DK + t);
        // decay, then the two column reductions
        float4 pp = make_float4(0.f, 0.f, 0.f, 0.f), zz = pp;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            H[p].x *= dr[p]; H[p].y *= dr[p]; H[p].z *= dr[p]; H[p].w *= dr[p];
            pp.x += H[p].x * kr[p]; pp.y += H[p].y * kr[p]; pp.z += H[p].z * kr[p]; pp.w += H[p].w * kr[p];
            zz.x += H[p].x * qr[p]; zz.y += H[p].y * qr[p]; zz.z += H[p].z * qr[p]; zz.w += H[p].w * qr[p];
        }
#pragma unroll
        for (int m = CPR4; m < 64; m <<= 1) {
            pp.x += __shfl_xor(pp.x, m, 64); pp.y += __shfl_xor(pp.y, m, 64);
            pp.z += __shfl_xor(pp.z, m, 64); pp.w += __shfl_xor(pp.w, m, 64);
            zz.x += __shfl_xor(zz.x, m, 64); zz.y += __shfl_xor(zz.y, m, 64);
            zz.z += __shfl_xor(zz.z, m, 64); zz.w += __shfl_xor(zz.w, m, 64);
        }
        kq = group_sum<64>(kq);
        if (lane < CPR4) {
            *reinterpret_cast<float4*>(&s_p[w][c0]) = pp;
            *reinterpret_cast<float4*>(&s_z[w][c0]) = zz;
        }
        if (lane == 0) s_kq[w] = kq;
        lds_barrier();
        float4 P = make_float4(0.f, 0.f, 0.f, 0.f), Z = P;
        float KQ = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float4 x = *reinterpret_cast<const float4*>(&s_p[ww][c0]);
            const float4 y = *reinterpret_cast<const float4*>(&s_z[ww][c0]);
            P.x += x.x; P.y += x.y; P.z += x.z; P.w += x.w;
            Z.x += y.x; Z.y += y.y; Z.z += y.z; Z.w += y.w;
            KQ += s_kq[ww];
        }
        lds_barrier();   // LDS is rewritten by the next token
        float4 u;
        u.x = beta * (vv.x - P.x); u.y = beta * (vv.y - P.y);
        u.z = beta * (vv.z - P.z); u.w = beta * (vv.w - P.w);
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            H[p].x += kr[p] * u.x; H[p].y += kr[p] * u.y; H[p].z += kr[p] * u.z; H[p].w += kr[p] * u.w;
        }
        if (a.o && rg == 0) {
            float4 ov;
            ov.x = Z.x + u.x * KQ; ov.y = Z.y + u.y * KQ; ov.z = Z.z + u.z * KQ; ov.w = Z.w + u.w * KQ;
            if constexpr (sizeof(TI) == 4) {
                *reinterpret_cast<float4*>(static_cast<float*>(a.o) + th * DV + c0) = ov;
            } else {
                tok_st<TI>(a.o, th * DV + c0, ov.x);
                tok_st<TI>(a.o, th * DV + c0 + 1, ov.y);
                tok_st<TI>(a.o, th * DV + c0 + 2, ov.z);
                tok_st<TI>(a.o, th * DV + c0 + 3, ov.w);
            }
        }
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        __builtin_nontemporal_store(f32x4v{H[p].x, H[p].y, H[p].z, H[p].w},
                                    reinterpret_cast<f32x4v*>(h + (size_t)(p * RPP + rg) * DV + c0));
    (void)GPW;
}

template <int DK, bool KDA>
hipError_t rec_t(const lq_dims& d, const RecArgs& args, hipStream_t s) {
    constexpr int NT = DK >= 64 ? 256 : 64;
    if (d.io_dtype == LQ_IO_BF16)
        return launch_kernel(LQ_KERNEL_FP32_RECURRENCE, fp32_rec_kernel<DK, DK, KDA, NT, uint16_t>,
                             dim3((unsigned)d.B * (unsigned)d.H), dim3(NT), s, args);
    return launch_kernel(LQ_KERNEL_FP32_RECURRENCE, fp32_rec_kernel<DK, DK, KDA, NT, float>,
                         dim3((unsigned)d.B * (unsigned)d.H), dim3(NT), s, args);
}

}  // namespace

hipError_t launch_fp32_recurrence(const lq_dims& d, float* h, int T, const void* q,
                                  const void* k, const void* v, const float* alpha,
                                  const float* beta, void* o, hipStream_t s) {
    RecArgs args{h, q, k, v, alpha, beta, o, T, (size_t)d.B * (size_t)d.H};
    const bool kda = d.decay_mode == LQ_DECAY_PER_KEY;
    switch (d.dk) {
        case 16: return kda ? rec_t<16, true>(d, args, s) : rec_t<16, false>(d, args, s);
        case 64: return kda ? rec_t<64, true>(d, args, s) : rec_t<64, false>(d, args, s);
        default: return kda ? rec_t<128, true>(d, args, s) : rec_t<128, false>(d, args, s);
    }
}

}  // namespace lq

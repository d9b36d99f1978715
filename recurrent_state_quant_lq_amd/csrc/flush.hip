// flush.hip -- window boundary: rebuild the state, extract compensator rows,
// smooth, requantize (gfx950).  Also the standalone codec kernels.
//
// News article ("A linear-attention method cuts state ...", paragraph 3):
// the state is reconstructed and quantized once at the window boundary.
// Forum mirror ("Abstract (translated)", techniques 2 and 3) and paragraph 4
// of the news article: the largest outliers are kept as a few
// high-precision compensator tokens and the residual is smoothed before
// quantization.
//
// Reconstruction from the window-base state Hb and N buffered slots:
//     M = U - Y Hb                     (N x dv,   contraction over dk)
//     H = Gamma Hb + Kt^T M            (dk x dv,  contraction over N)
// with Kt[i][c] = exp(g_{N-1}[c] - g_i[c]) k_i[c] and Gamma = diag exp(g_{N-1}).
// Both are dense fp32 contractions and run on v_mfma_f32_16x16x4_f32.
//
// Register layout ("D layout") of one workgroup: NW waves, wave w owns row
// blocks w*RBW .. w*RBW+RBW-1 (16 rows each) and all DV columns.  Lane l
// (li = l % 16, lg = l / 16) holds, for row block rb, column tile ct and
// v = 0..3,
//     H[(w*RBW + rb)*16 + 4*lg + v][li*CT + ct].
// This is the MFMA accumulator layout with column tile ct made of the
// columns {n*CT + ct}, so one lane's CT columns are contiguous in memory
// (one 8-byte int8 load/store, two 16-byte fp32 loads/stores per row) and the
// first contraction's B operand is the state register itself (its K index
// runs over the 4 rows 4*lg + s a lane already holds).
//
// The codec steps are single IEEE fp32 operations in a fixed order, so the
// int8 bytes, scales and compensator rows are a function of the fp32 H.
#include "lq_internal.h"

#pragma clang fp contract(off)

namespace lq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// Magnitudes below 2^-120 count as zero in the codec: a column that small
// keeps scale 1 and a row that small quantizes to zeros, so 1/s and 127/rho
// (which overflow fp32 below about 2^-121) stay finite.
constexpr float kTiny = 0x1p-120f;

struct CodecOut {
    int8_t* sq;
    float* r;
    float* s;
    int32_t* idx;
    float* cv;
};

template <int DK, int DV>
struct Shape {
    static constexpr int RB = DK / 16;
    static constexpr int CT = DV / 16;
    static constexpr int NW = RB < 4 ? RB : 4;
    static constexpr int NT = 64 * NW;
    static constexpr int RBW = RB / NW;
    static_assert(DK % 16 == 0 && DV % 16 == 0 && RB % NW == 0, "tile shape");
};

template <int CT>
__device__ __forceinline__ void store_bytes(int8_t* p, const int (&b)[CT]) {
    if constexpr (CT == 8) {
        uint2 w;
        w.x = (uint32_t)(b[0] & 255) | ((uint32_t)(b[1] & 255) << 8) | ((uint32_t)(b[2] & 255) << 16) |
              ((uint32_t)(b[3] & 255) << 24);
        w.y = (uint32_t)(b[4] & 255) | ((uint32_t)(b[5] & 255) << 8) | ((uint32_t)(b[6] & 255) << 16) |
              ((uint32_t)(b[7] & 255) << 24);
        *reinterpret_cast<uint2*>(p) = w;
    } else if constexpr (CT == 4) {
        *reinterpret_cast<uint32_t*>(p) = (uint32_t)(b[0] & 255) | ((uint32_t)(b[1] & 255) << 8) |
                                          ((uint32_t)(b[2] & 255) << 16) | ((uint32_t)(b[3] & 255) << 24);
    } else {
#pragma unroll
        for (int i = 0; i < CT; ++i) p[i] = (int8_t)b[i];
    }
}

template <int CT>
__device__ __forceinline__ void load_bytes(const int8_t* p, float (&x)[CT]) {
    if constexpr (CT == 8) {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = sbyte(w.x, e);
            x[4 + e] = sbyte(w.y, e);
        }
    } else if constexpr (CT == 4) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = sbyte(w, e);
    } else {
#pragma unroll
        for (int e = 0; e < CT; ++e) x[e] = (float)p[e];
    }
}

// LDS used by the codec stage.
template <int DK, int DV, int NW>
struct CodecLds {
    float m[DK];        // row magnitudes, later unused
    int pos[DK];        // compensator slot of a row, or -1
    int flag[DK];
    float cm[NW][DV];   // per-wave column maxima
    float sinv[DV];     // 1 / col_scale
};

// Codec of the state held in D layout (H is overwritten).  Writes sq, r, s,
// idx, cv of one head; h_out (nullable) receives H first.
template <int DK, int DV, int RBW, int CT, int NW>
__device__ void codec_store(float (&H)[RBW][CT][4], CodecLds<DK, DV, NW>& L, const CodecOut& out,
                            float* __restrict__ h_out, int C, int smooth) {
    const int t = threadIdx.x;
    const int lane = t & 63, w = t >> 6, li = lane & 15, lg = lane >> 4;
    auto row_of = [&](int rb, int v) { return (w * RBW + rb) * 16 + 4 * lg + v; };

    if (h_out) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float x[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) x[ct] = H[rb][ct][v];
                store_floats<CT>(h_out + (size_t)row_of(rb, v) * DV + li * CT, x);
            }
    }
    // row magnitudes
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float mx = 0.0f;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) mx = fmaxf(mx, fabsf(H[rb][ct][v]));
            mx = group_max<16>(mx);
            if (li == 0) L.m[row_of(rb, v)] = mx;
        }
    lds_barrier();
    // the C largest rows (ties: lower row)
    if (t < DK) {
        const float mt = L.m[t];
        int rank = 0;
        for (int i = 0; i < DK; ++i) {
            const float mi = L.m[i];
            rank += (mi > mt) || (mi == mt && i < t);
        }
        L.flag[t] = rank < C;
    }
    lds_barrier();
    if (t < DK) {
        int p = -1;
        if (L.flag[t]) {
            p = 0;
            for (int i = 0; i < t; ++i) p += L.flag[i];
            out.idx[p] = t;
        }
        L.pos[t] = p;
    }
    lds_barrier();
    // compensator rows out, residual rows zeroed
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int p = L.pos[row_of(rb, v)];
            if (p >= 0) {
                float x[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    x[ct] = H[rb][ct][v];
                    H[rb][ct][v] = 0.0f;
                }
                store_floats<CT>(out.cv + (size_t)p * DV + li * CT, x);
            }
        }
    // column maxima of the residual
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        float mx = 0.0f;
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v) mx = fmaxf(mx, fabsf(H[rb][ct][v]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (lg == 0) L.cm[w][li * CT + ct] = mx;
    }
    lds_barrier();
    if (t < DV) {
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < NW; ++i) mx = fmaxf(mx, L.cm[i][t]);
        const float sj = (smooth && mx >= kTiny) ? mx : 1.0f;
        out.s[t] = sj;
        L.sinv[t] = 1.0f / sj;
    }
    lds_barrier();
    // smoothing, row scales, rounding
    float inv[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) inv[ct] = L.sinv[li * CT + ct];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float rho = 0.0f;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                H[rb][ct][v] = H[rb][ct][v] * inv[ct];
                rho = fmaxf(rho, fabsf(H[rb][ct][v]));
            }
            rho = group_max<16>(rho);
            const int row = row_of(rb, v);
            int b[CT];
            if (rho >= kTiny) {
                const float lam = 127.0f / rho;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    float x = rintf(H[rb][ct][v] * lam);
                    x = fminf(fmaxf(x, -127.0f), 127.0f);
                    b[ct] = (int)x;
                }
                if (li == 0) out.r[row] = rho / 127.0f;
            } else {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) b[ct] = 0;
                if (li == 0) out.r[row] = 0.0f;
            }
            store_bytes<CT>(out.sq + (size_t)row * DV + li * CT, b);
        }
}

// Window-base state Hb of one head in D layout: (sq * r) * s, with the
// compensator rows replaced by their stored values.
template <int DK, int DV, int RBW, int CT>
__device__ void load_base(float (&H)[RBW][CT][4], const int8_t* sq, const float* r, const float* s,
                          const int32_t* idx, const float* cv, int C) {
    const int t = threadIdx.x;
    const int lane = t & 63, w = t >> 6, li = lane & 15, lg = lane >> 4;
    float sc[CT];
    load_floats<CT>(s + li * CT, sc);
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = (w * RBW + rb) * 16 + 4 * lg + v;
            float qb[CT];
            load_bytes<CT>(sq + (size_t)row * DV + li * CT, qb);
            const float rr = r[row];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) H[rb][ct][v] = (qb[ct] * rr) * sc[ct];
        }
    for (int c = 0; c < C; ++c) {
        const int ri = idx[c];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if ((w * RBW + rb) * 16 + 4 * lg + v == ri) {
                    float x[CT];
                    load_floats<CT>(cv + (size_t)c * DV + li * CT, x);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) H[rb][ct][v] = x[ct];
                }
    }
}

struct FlushArgs {
    int8_t* sq;
    float* r;
    float* s;
    int32_t* idx;
    float* cv;
    const float* bk;
    const float* by;
    const float* bu;
    const float* bg;
    float* h_out;
    int W;
    int C;
    int N;
    int smooth;
};

template <int DK, int DV, int WM, bool KDA>
__global__ __launch_bounds__((Shape<DK, DV>::NT)) void flush_kernel(FlushArgs a) {
    using S = Shape<DK, DV>;
    constexpr int RBW = S::RBW, CT = S::CT, NW = S::NW, NT = S::NT;
    constexpr int NPAD = WM <= 16 ? 16 : 32;   // slots padded to the MFMA M size
    constexpr int MB = NPAD / 16;
    constexpr int GD = KDA ? DK : 1;
    constexpr int NU4 = NPAD * DV / 4;         // float4 elements of M
    constexpr int UPT = (NU4 + NT - 1) / NT;

    __shared__ __align__(16) float s_M[NW][NPAD][DV];
    __shared__ __align__(16) CodecLds<DK, DV, NW> L;

    const int t = threadIdx.x;
    const int lane = t & 63, w = t >> 6, li = lane & 15, lg = lane >> 4;
    const size_t head = blockIdx.x;
    const int W = a.W, C = a.C, N = a.N;

    const int8_t* sq = a.sq + head * (DK * DV);
    const float* r = a.r + head * DK;
    const float* s = a.s + head * DV;
    const int32_t* idx = a.idx + head * C;
    const float* cv = a.cv + head * (size_t)C * DV;
    const float* bk = a.bk + head * (size_t)W * DK;
    const float* by = a.by + head * (size_t)W * DK;
    const float* bu = a.bu + head * (size_t)W * DV;
    const float* bg = a.bg + head * (size_t)W * GD;

    // ---- loads -----------------------------------------------------------------
    float H[RBW][CT][4];
    load_base<DK, DV, RBW, CT>(H, sq, r, s, idx, cv, C);

    float4 y4[MB][RBW];                         // A operand of M = Y Hb
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            const int slot = mb * 16 + li;
            y4[mb][rb] = slot < N ? *reinterpret_cast<const float4*>(by + (size_t)slot * DK +
                                                                      (w * RBW + rb) * 16 + 4 * lg)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    float4 u4[UPT];                             // U rows for M
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
        const int e4 = t + i * NT;
        const int slot = (e4 * 4) / DV;
        u4[i] = (e4 < NU4 && slot < N) ? reinterpret_cast<const float4*>(bu)[e4]
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // A operand of Kt^T M: Kt[slot][row] for row = rowbase + li, slot = 4*ks + lg
    float ka[RBW][NPAD / 4];
    float gl[RBW];                              // g_{N-1} of the A-operand rows (KDA)
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
        const int rowa = (w * RBW + rb) * 16 + li;
        gl[rb] = KDA ? bg[(size_t)(N - 1) * DK + rowa] : 0.0f;
#pragma unroll
        for (int ks = 0; ks < NPAD / 4; ++ks) {
            const int slot = 4 * ks + lg;
            float x = 0.0f;
            if (slot < N) {
                const float kx = bk[(size_t)slot * DK + rowa];
                const float gd = KDA ? gl[rb] - bg[(size_t)slot * DK + rowa] : bg[N - 1] - bg[slot];
                x = __expf(gd) * kx;
            }
            ka[rb][ks] = x;
        }
    }

    // ---- M partial = Y Hb over this wave's rows ----------------------------------
    {
        v4f acc[MB][CT];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) acc[mb][ct] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int sidx = 0; sidx < 4; ++sidx)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const float av = sidx == 0 ? y4[mb][rb].x : sidx == 1 ? y4[mb][rb].y
                                   : sidx == 2 ? y4[mb][rb].z : y4[mb][rb].w;
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        acc[mb][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, H[rb][ct][sidx],
                                                                           acc[mb][ct], 0, 0, 0);
                }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float x[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) x[ct] = acc[mb][ct][v];
                store_floats<CT>(&s_M[w][mb * 16 + 4 * lg + v][li * CT], x);
            }
    }
    lds_barrier();
    // M = U - sum over waves (rows >= N stay zero)
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
        const int e4 = t + i * NT;
        if (e4 < NU4) {
            float4 m = u4[i];
            float* base = &s_M[0][0][0] + e4 * 4;
            const int slot = (e4 * 4) / DV;
            if (slot < N) {
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) {
                    const float4 p = *reinterpret_cast<const float4*>(base + ww * NPAD * DV);
                    m.x -= p.x; m.y -= p.y; m.z -= p.z; m.w -= p.w;
                }
            }
            *reinterpret_cast<float4*>(base) = m;
        }
    }
    lds_barrier();

    // ---- H = Gamma Hb + Kt^T M ----------------------------------------------------
    {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = (w * RBW + rb) * 16 + 4 * lg + v;
                const float gam = __expf(KDA ? bg[(size_t)(N - 1) * DK + row] : bg[N - 1]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) H[rb][ct][v] = gam * H[rb][ct][v];
            }
        v4f acc[RBW][CT];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                acc[rb][ct] = v4f{H[rb][ct][0], H[rb][ct][1], H[rb][ct][2], H[rb][ct][3]};
#pragma unroll
        for (int ks = 0; ks < NPAD / 4; ++ks) {
            if (4 * ks < N) {
                float bm[CT];
                load_floats<CT>(&s_M[0][4 * ks + lg][li * CT], bm);
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        acc[rb][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[rb][ks], bm[ct],
                                                                           acc[rb][ct], 0, 0, 0);
            }
        }
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int v = 0; v < 4; ++v) H[rb][ct][v] = acc[rb][ct][v];
    }

    // ---- requantize ------------------------------------------------------------------
    CodecOut out{a.sq + head * (DK * DV), a.r + head * DK, a.s + head * DV, a.idx + head * C,
                 a.cv + head * (size_t)C * DV};
    codec_store<DK, DV, RBW, CT, NW>(H, L, out, a.h_out ? a.h_out + head * (size_t)DK * DV : nullptr, C,
                        a.smooth);
}

struct QuantArgs {
    const float* h;
    int8_t* sq;
    float* r;
    float* s;
    int32_t* idx;
    float* cv;
    int C;
    int smooth;
};

template <int DK, int DV>
__global__ __launch_bounds__((Shape<DK, DV>::NT)) void quantize_kernel(QuantArgs a) {
    using S = Shape<DK, DV>;
    constexpr int RBW = S::RBW, CT = S::CT, NW = S::NW;
    __shared__ __align__(16) CodecLds<DK, DV, NW> L;
    const int t = threadIdx.x;
    const int lane = t & 63, w = t >> 6, li = lane & 15, lg = lane >> 4;
    const size_t head = blockIdx.x;
    const float* h = a.h + head * (size_t)DK * DV;
    float H[RBW][CT][4];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float x[CT];
            load_floats<CT>(h + (size_t)((w * RBW + rb) * 16 + 4 * lg + v) * DV + li * CT, x);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) H[rb][ct][v] = x[ct];
        }
    CodecOut out{a.sq + head * (DK * DV), a.r + head * DK, a.s + head * DV, a.idx + head * a.C,
                 a.cv + head * (size_t)a.C * DV};
    codec_store<DK, DV, RBW, CT, NW>(H, L, out, nullptr, a.C, a.smooth);
}

struct DequantArgs {
    const int8_t* sq;
    const float* r;
    const float* s;
    const int32_t* idx;
    const float* cv;
    float* h;
    int C;
};

template <int DK, int DV>
__global__ __launch_bounds__(256) void dequantize_kernel(DequantArgs a) {
    const size_t head = blockIdx.x;
    const int t = threadIdx.x;
    __shared__ int s_pos[DK];
    for (int i = t; i < DK; i += 256) s_pos[i] = -1;
    __syncthreads();
    if (t < a.C) s_pos[a.idx[head * a.C + t]] = t;
    __syncthreads();
    const int8_t* sq = a.sq + head * (DK * DV);
    const float* r = a.r + head * DK;
    const float* s = a.s + head * DV;
    float* h = a.h + head * (size_t)DK * DV;
    for (int e = t; e < DK * DV; e += 256) {
        const int row = e / DV, col = e % DV;
        const int p = s_pos[row];
        h[e] = p >= 0 ? a.cv[(head * a.C + p) * (size_t)DV + col]
                      : ((float)sq[e] * r[row]) * s[col];
    }
}

template <int DK, int WM, bool KDA>
hipError_t flush_t(const lq_dims& d, const FlushArgs& args, hipStream_t s) {
    hipLaunchKernelGGL((flush_kernel<DK, DK, WM, KDA>), dim3((unsigned)d.B * (unsigned)d.H),
                       dim3(Shape<DK, DK>::NT), 0, s, args);
    return hipGetLastError();
}

template <int DK>
hipError_t flush_dk(const lq_dims& d, const FlushArgs& args, hipStream_t s) {
    const bool kda = d.decay_mode == LQ_DECAY_PER_KEY;
    if (d.W <= 16) return kda ? flush_t<DK, 16, true>(d, args, s) : flush_t<DK, 16, false>(d, args, s);
    return kda ? flush_t<DK, 32, true>(d, args, s) : flush_t<DK, 32, false>(d, args, s);
}

}  // namespace

hipError_t launch_flush(const lq_dims& d, const lq_state& st, int n_buffered, float* h_out,
                        hipStream_t s) {
    FlushArgs args{st.sq, st.row_scale, st.col_scale, st.comp_idx, st.comp_val,
                   st.buf_k, st.buf_y, st.buf_u, st.buf_g, h_out, d.W, d.C, n_buffered, d.smooth};
    switch (d.dk) {
        case 16: return flush_dk<16>(d, args, s);
        case 64: return flush_dk<64>(d, args, s);
        default: return flush_dk<128>(d, args, s);
    }
}

hipError_t launch_quantize(const lq_dims& d, const float* h, const lq_state& st, hipStream_t s) {
    QuantArgs args{h, st.sq, st.row_scale, st.col_scale, st.comp_idx, st.comp_val, d.C, d.smooth};
    const dim3 grid((unsigned)d.B * (unsigned)d.H);
    switch (d.dk) {
        case 16: hipLaunchKernelGGL((quantize_kernel<16, 16>), grid, dim3(Shape<16, 16>::NT), 0, s, args); break;
        case 64: hipLaunchKernelGGL((quantize_kernel<64, 64>), grid, dim3(Shape<64, 64>::NT), 0, s, args); break;
        default: hipLaunchKernelGGL((quantize_kernel<128, 128>), grid, dim3(Shape<128, 128>::NT), 0, s, args); break;
    }
    return hipGetLastError();
}

hipError_t launch_dequantize(const lq_dims& d, const lq_state& st, float* h_out, hipStream_t s) {
    DequantArgs args{st.sq, st.row_scale, st.col_scale, st.comp_idx, st.comp_val, h_out, d.C};
    const dim3 grid((unsigned)d.B * (unsigned)d.H);
    switch (d.dk) {
        case 16: hipLaunchKernelGGL((dequantize_kernel<16, 16>), grid, dim3(256), 0, s, args); break;
        case 64: hipLaunchKernelGGL((dequantize_kernel<64, 64>), grid, dim3(256), 0, s, args); break;
        default: hipLaunchKernelGGL((dequantize_kernel<128, 128>), grid, dim3(256), 0, s, args); break;
    }
    return hipGetLastError();
}

}  // namespace lq

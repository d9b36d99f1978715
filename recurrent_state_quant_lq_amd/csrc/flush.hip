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
//   * Y Hb = ((Y o r) sq) o s + sum_c Y[:, idx_c] cv_c^T: the int8 state is
//     the B operand of v_mfma_i32_16x16x64_i8 as stored (value-column-major
//     sq[j][i]: 16 consecutive key channels of a column are one load) and
//     Y o r enters as three int8 digits per slot (exact int32 sums, recombined
//     in fp32).  Each wave owns whole column tiles, so no cross-wave sums.
//   * Kt^T M is dense fp32 on v_mfma_f32_16x16x4_f32.
//
// Register layout ("D layout") of H in one workgroup: NW waves; lane l
// (li = l % 16, lg = l / 16) of wave w holds, for v4 register (rb, ct),
//     H[row(w, lg, rb, v)][li*CT + ct],   row = w*16*RBW + lg*4*RBW + rb*4 + v,
// i.e. the MFMA accumulator layout with the rows permuted so that a lane's
// 4*RBW rows are consecutive: one column's bytes of those rows are one 8-byte
// access in the value-column-major state, and its CT columns are contiguous
// in row-major fp32 arrays.
//
// The codec steps are single IEEE fp32 operations in a fixed order, so the
// int8 bytes, scales and compensator rows are a function of the fp32 H.
#include "lq_internal.h"

#pragma clang fp contract(off)

namespace lq {
namespace {

// Magnitudes below 2^-120 count as zero in the codec: a column that small
// keeps scale 1 and a row that small quantizes to zeros, so 1/s and 127/rho
// (which overflow fp32 below about 2^-121) stay finite.
constexpr float kTiny = 0x1p-120f;
constexpr int CMAX = 8;

struct CodecOut {
    int8_t* sq;
    float* r;
    float* s;
    int32_t* idx;
    float* cv;
};

template <int DK, int DV>
struct FS {
    static_assert(DK == DV, "square heads");
    static constexpr int RB = DK / 16;
    static constexpr int CT = DV / 16;                 // columns per lane = column tiles
    static constexpr int NW = RB < 4 ? RB : 4;
    static constexpr int NT = 64 * NW;
    static constexpr int RBW = RB / NW;
    static constexpr int RPL = 4 * RBW;                // consecutive rows per lane group
    static constexpr int TPW = CT / NW > 0 ? CT / NW : 1;   // contraction-1 tiles per wave
    static constexpr int KS = (DK + 63) / 64;
    static_assert(DK % 16 == 0 && RB % NW == 0 && (CT % NW == 0 || CT < NW), "tile shape");
};

template <int DK, int DV>
__device__ __forceinline__ int row_of(int w, int lg, int rb, int v) {
    using S = FS<DK, DV>;
    return w * 16 * S::RBW + lg * S::RPL + rb * 4 + v;
}

// RPL bytes of one column for a lane's rows, in row order.
template <int RPL>
struct RowBytes;
template <>
struct RowBytes<8> {
    using T = uint2;
    static __device__ float get(const uint2& x, int k) { return sbyte(k < 4 ? x.x : x.y, k & 3); }
};
template <>
struct RowBytes<4> {
    using T = uint32_t;
    static __device__ float get(const uint32_t& x, int k) { return sbyte(x, k); }
};

// LDS used by the codec stage.
template <int DK, int DV, int NW>
struct CodecLds {
    float m[DK];                 // row magnitudes
    int pos[DK];                 // compensator slot of a row, or -1
    unsigned long long ball[(DK + 63) / 64];
    float cm[NW][DV];            // per-wave column maxima
    float sinv[DV];              // 1 / col_scale
};

// Codec of the state held in D layout (H is overwritten).  Writes sq
// (value-column-major), r, s, idx, cv of one head; h_out (nullable,
// row-major fp32) receives H first.
template <int DK, int DV, int RBW, int CT, int NW>
__device__ void codec_store(v4f (&H)[RBW][CT], CodecLds<DK, DV, NW>& L, const CodecOut& out,
                            float* __restrict__ h_out, int C, int smooth) {
    constexpr int RPL = FS<DK, DV>::RPL;
    const int t = threadIdx.x;
    const int lane = t & 63, w = t >> 6, li = lane & 15, lg = lane >> 4;

    if (h_out) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float x[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) x[ct] = H[rb][ct][v];
                store_floats<CT>(h_out + (size_t)row_of<DK, DV>(w, lg, rb, v) * DV + li * CT, x);
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
            if (li == 0) L.m[row_of<DK, DV>(w, lg, rb, v)] = mx;
        }
    lds_barrier();
    // the C largest rows (ties: lower row), then their ascending positions
    if (t < DK) {
        const float mt = L.m[t];
        int rank = 0;
#pragma unroll 8
        for (int i = 0; i < DK; i += 4) {
            const float4 m4 = *reinterpret_cast<const float4*>(&L.m[i]);
            rank += (m4.x > mt) || (m4.x == mt && i < t);
            rank += (m4.y > mt) || (m4.y == mt && i + 1 < t);
            rank += (m4.z > mt) || (m4.z == mt && i + 2 < t);
            rank += (m4.w > mt) || (m4.w == mt && i + 3 < t);
        }
        const unsigned long long b = __ballot(rank < C);
        if (lane == 0) L.ball[w] = b;
    }
    lds_barrier();
    if (t < DK) {
        const unsigned long long b = L.ball[w];
        int p = -1;
        if ((b >> lane) & 1ull) {
            p = __popcll(b & ((1ull << lane) - 1ull));
            for (int ww = 0; ww < w; ++ww) p += __popcll(L.ball[ww]);
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
            const int p = L.pos[row_of<DK, DV>(w, lg, rb, v)];
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
        mx = fmaxf(mx, swz_xor16(mx));
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
    // smoothing, row scales
    float inv[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) inv[ct] = L.sinv[li * CT + ct];
    float lam[RBW][4];
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
            const bool live = rho >= kTiny;
            lam[rb][v] = live ? 127.0f / rho : 0.0f;
            if (li == 0) out.r[row_of<DK, DV>(w, lg, rb, v)] = live ? rho / 127.0f : 0.0f;
        }
    // rounding; one column's RPL bytes per store
    const int row0 = row_of<DK, DV>(w, lg, 0, 0);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        int b[RBW][4];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float x = rintf(H[rb][ct][v] * lam[rb][v]);
                x = fminf(fmaxf(x, -127.0f), 127.0f);
                b[rb][v] = (int)x;
            }
        int8_t* dst = out.sq + (size_t)(li * CT + ct) * DK + row0;
        if constexpr (RPL == 8)
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack4(b[0][0], b[0][1], b[0][2], b[0][3]),
                                                        pack4(b[1][0], b[1][1], b[1][2], b[1][3]));
        else
            *reinterpret_cast<uint32_t*>(dst) = pack4(b[0][0], b[0][1], b[0][2], b[0][3]);
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
__global__ __launch_bounds__((FS<DK, DV>::NT))
__attribute__((amdgpu_waves_per_eu(WM <= 16 ? 4 : 2, WM <= 16 ? 4 : 2)))
void flush_kernel(FlushArgs a) {
    using S = FS<DK, DV>;
    constexpr int RBW = S::RBW, CT = S::CT, NW = S::NW, NT = S::NT, RPL = S::RPL;
    constexpr int TPW = S::TPW, KS = S::KS;
    constexpr int NPAD = WM <= 16 ? 16 : 32;   // slots padded to the MFMA size
    constexpr int MB = NPAD / 16;
    constexpr int GD = KDA ? DK : 1;
    constexpr int LPS = NT / NPAD;             // lanes per slot in the digit stage
    constexpr int CHD = DK / LPS;              // channels per lane in the digit stage
    static_assert(NT % NPAD == 0 && DK % LPS == 0 && CHD % 4 == 0, "digit tiling");
    using RBy = RowBytes<RPL>;

    __shared__ __align__(16) float s_rs[(2 + CMAX) * DK];  // r, s, compensator rows
    __shared__ __align__(16) int s_misc[16];               // idx[0..7]
    __shared__ __align__(16) int8_t s_dA[3][NPAD][KS * 64];
    __shared__ __align__(16) float s_ysc[NPAD];
    __shared__ __align__(16) float s_yc[CMAX][NPAD];
    __shared__ __align__(16) float s_M[NPAD][DV];
    __shared__ __align__(16) CodecLds<DK, DV, NW> L;
    float* s_r = s_rs;
    float* s_s = s_rs + DK;
    float* s_cv = s_rs + 2 * DK;                            // [CMAX][DV]

    const int t = threadIdx.x;
    const int lane = t & 63, li = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const size_t head = blockIdx.x;
    const int W = a.W, C = a.C, N = a.N;

    const int8_t* sq = a.sq + head * (DK * DV);
    const float* bk = a.bk + head * (size_t)W * DK;
    const float* by = a.by + head * (size_t)W * DK;
    const float* bu = a.bu + head * (size_t)W * DV;
    const float* bg = a.bg + head * (size_t)W * GD;

    // ---- loads --------------------------------------------------------------------------------
    // r, s, compensator rows -> LDS (DK/4 lanes per vector of 16-byte chunks)
    {
        constexpr int SEGL = DK / 4, SPI = 64 / SEGL;
        const int nseg = 2 + C;
        const int my = lane / SEGL;
        for (int s0 = SPI * w; s0 < nseg; s0 += SPI * NW) {
            const float* src = nullptr;
#pragma unroll
            for (int q = 0; q < SPI; ++q) {
                const int sg = s0 + q;
                const float* p = sg == 0 ? a.r + head * DK
                               : sg == 1 ? a.s + head * DV
                               : sg < nseg ? a.cv + (head * C + (sg - 2)) * (size_t)DV : nullptr;
                if (my == q) src = p;
            }
            if (src) lds_dma16(src + 4 * (lane % SEGL), s_rs + s0 * DK);
        }
        if (w == 0 && lane < C) lds_dma4(a.idx + head * C + lane, s_misc);
    }
    // digit stage inputs: Y[slot][c0 .. c0+CHD)
    // (loads below are unconditional, slot indices clamped into the buffer; the
    // values of slots >= N are masked after the barrier)
    const int dslot = t / LPS, dc0 = (t % LPS) * CHD;
    float yv[CHD];
    load_floats<CHD>(by + (size_t)min(dslot, W - 1) * DK + dc0, yv);
    // contraction-1 B operands: column j = tile*16 + li, channels ks*64 + 16*lg .. +15
    v4i bq[TPW][KS];
    constexpr bool FULL = (CT % NW == 0) && (DK % 64 == 0);
#pragma unroll
    for (int tw = 0; tw < TPW; ++tw)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int tile = w * TPW + tw;
            const int i0 = ks * 64 + 16 * lg;
            if (FULL || (tile < CT && i0 < DK))
                bq[tw][ks] = *reinterpret_cast<const v4i*>(sq + (size_t)(tile * 16 + li) * DK + i0);
            else
                bq[tw][ks] = v4i{0, 0, 0, 0};
        }
    // contraction-1 outputs need U[slot][j] at (slot = mb*16 + 4*lg + v, j = tile*16 + li)
    float uv[MB][TPW][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int tw = 0; tw < TPW; ++tw)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int slot = min(mb * 16 + 4 * lg + v, W - 1);
                const int tile = min(w * TPW + tw, CT - 1);
                uv[mb][tw][v] = bu[(size_t)slot * DV + tile * 16 + li];
            }
    // D-layout bytes of the base state: column li*CT + ct, this lane's RPL rows
    const int row0 = row_of<DK, DV>(w, lg, 0, 0);
    typename RBy::T hb[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
        hb[ct] = *reinterpret_cast<const typename RBy::T*>(sq + (size_t)(li * CT + ct) * DK + row0);
    // window log-decay of this lane's rows
    float gam[RBW][4];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            gam[rb][v] = KDA ? bg[(size_t)(N - 1) * DK + row_of<DK, DV>(w, lg, rb, v)] : bg[N - 1];
    // contraction-2 A operands: Kt[slot][rowa], rowa = row(w, li/4, rb, li%4), slot = 4*ks + lg
    float ka[RBW][NPAD / 4], kg[RBW][NPAD / 4], gl[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
        const int rowa = row_of<DK, DV>(w, li >> 2, rb, li & 3);
        gl[rb] = KDA ? bg[(size_t)(N - 1) * DK + rowa] : bg[N - 1];
#pragma unroll
        for (int ks = 0; ks < NPAD / 4; ++ks) {
            const int slot = min(4 * ks + lg, W - 1);
            ka[rb][ks] = bk[(size_t)slot * DK + rowa];
            kg[rb][ks] = KDA ? bg[(size_t)slot * DK + rowa] : bg[slot];
        }
    }
    all_loads_barrier();

    // Kt (decayed keys) of the contraction-2 A operands; slots >= N are zero
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int ks = 0; ks < NPAD / 4; ++ks)
            ka[rb][ks] = 4 * ks + lg < N ? __expf(gl[rb] - kg[rb][ks]) * ka[rb][ks] : 0.0f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int tw = 0; tw < TPW; ++tw)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (mb * 16 + 4 * lg + v >= N) uv[mb][tw][v] = 0.0f;
    if (dslot >= N) {
#pragma unroll
        for (int c = 0; c < CHD; ++c) yv[c] = 0.0f;
    }

    // ---- digits of (Y o r), per slot --------------------------------------------------------------
    {
        float p[CHD];
        float mx = 0.0f;
#pragma unroll
        for (int c = 0; c < CHD; ++c) {
            p[c] = yv[c] * s_r[dc0 + c];
            mx = fmaxf(mx, fabsf(p[c]));
        }
        mx = group_max<LPS>(mx);
        const float inv = mx > 0.0f ? 127.0f / mx : 0.0f;
        int dg[3][CHD];
#pragma unroll
        for (int c = 0; c < CHD; ++c) digits3(p[c], inv, dg[0][c], dg[1][c], dg[2][c]);
#pragma unroll
        for (int d = 0; d < 3; ++d)
#pragma unroll
            for (int c = 0; c < CHD; c += 4)
                *reinterpret_cast<uint32_t*>(&s_dA[d][dslot][dc0 + c]) =
                    pack4(dg[d][c], dg[d][c + 1], dg[d][c + 2], dg[d][c + 3]);
        if (t % LPS == 0) s_ysc[dslot] = mx * (1.0f / 127.0f);
        for (int c = 0; c < C; ++c) {
            const int rc = s_misc[c] - dc0;
#pragma unroll
            for (int cc = 0; cc < CHD; ++cc)
                if (rc == cc) s_yc[c][dslot] = yv[cc];
        }
        // channels past DK in the last K step stay zero
        if constexpr (KS * 64 > DK) {
            constexpr int PADC = KS * 64 - DK;
            for (int e = t; e < 3 * NPAD * PADC; e += NT)
                s_dA[e / (NPAD * PADC)][(e % (NPAD * PADC)) / PADC][DK + e % PADC] = 0;
        }
    }
    lds_barrier();

    // ---- M = U - Y Hb for this wave's column tiles (int8 MFMA) --------------------------------
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        v4i acc[3][TPW];
#pragma unroll
        for (int d = 0; d < 3; ++d)
#pragma unroll
            for (int tw = 0; tw < TPW; ++tw) acc[d][tw] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int d = 0; d < 3; ++d) {
                const v4i aop = *reinterpret_cast<const v4i*>(&s_dA[d][mb * 16 + li][ks * 64 + 16 * lg]);
#pragma unroll
                for (int tw = 0; tw < TPW; ++tw)
                    acc[d][tw] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bq[tw][ks], acc[d][tw], 0, 0, 0);
            }
#pragma unroll
        for (int tw = 0; tw < TPW; ++tw) {
            const int tile = w * TPW + tw;
            if (tile >= CT) break;
            const int jj = tile * 16 + li;
            const float sj = s_s[jj];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int slot = mb * 16 + 4 * lg + v;
                float m = 0.0f;
                if (slot < N) {
                    const float yq = s_ysc[slot] * ((float)acc[0][tw][v] + (float)acc[1][tw][v] * kDigitW1 +
                                                    (float)acc[2][tw][v] * kDigitW2);
                    float comp = 0.0f;
                    for (int c = 0; c < C; ++c) comp += s_yc[c][slot] * s_cv[c * DV + jj];
                    m = uv[mb][tw][v] - (sj * yq + comp);
                }
                s_M[slot][jj] = m;
            }
        }
    }
    lds_barrier();

    // ---- H = Gamma Hb + Kt^T M (fp32 MFMA, accumulating in place) -------------------------------
    v4f H[RBW][CT];
    {
        float sc[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) sc[ct] = s_s[li * CT + ct];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = row_of<DK, DV>(w, lg, rb, v);
                const float rr = s_r[row];
                const float g = __expf(gam[rb][v]);
                float x[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) x[ct] = (RBy::get(hb[ct], rb * 4 + v) * rr) * sc[ct];
                for (int c = 0; c < C; ++c)
                    if (s_misc[c] == row) {
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct) x[ct] += s_cv[c * DV + li * CT + ct];
                    }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) H[rb][ct][v] = g * x[ct];
            }
#pragma unroll
        for (int ks = 0; ks < NPAD / 4; ++ks) {
            if (4 * ks < N) {
                float bm[CT];
                load_floats<CT>(&s_M[4 * ks + lg][li * CT], bm);
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        H[rb][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[rb][ks], bm[ct], H[rb][ct], 0, 0, 0);
            }
        }
    }

    // ---- requantize ---------------------------------------------------------------------------------
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
__global__ __launch_bounds__((FS<DK, DV>::NT)) void quantize_kernel(QuantArgs a) {
    using S = FS<DK, DV>;
    constexpr int RBW = S::RBW, CT = S::CT, NW = S::NW;
    __shared__ __align__(16) CodecLds<DK, DV, NW> L;
    const int t = threadIdx.x;
    const int lane = t & 63, w = t >> 6, li = lane & 15, lg = lane >> 4;
    const size_t head = blockIdx.x;
    const float* h = a.h + head * (size_t)DK * DV;
    v4f H[RBW][CT];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float x[CT];
            load_floats<CT>(h + (size_t)row_of<DK, DV>(w, lg, rb, v) * DV + li * CT, x);
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

// Row-major fp32 state from the codec: (sq * r) * s, plus the compensator rows.
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
        float x = ((float)sq[(size_t)col * DK + row] * r[row]) * s[col];
        if (p >= 0) x += a.cv[(head * a.C + p) * (size_t)DV + col];
        h[e] = x;
    }
}

template <int DK, int WM, bool KDA>
hipError_t flush_t(const lq_dims& d, const FlushArgs& args, hipStream_t s) {
    hipLaunchKernelGGL((flush_kernel<DK, DK, WM, KDA>), dim3((unsigned)d.B * (unsigned)d.H),
                       dim3(FS<DK, DK>::NT), 0, s, args);
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
        case 16: hipLaunchKernelGGL((quantize_kernel<16, 16>), grid, dim3(FS<16, 16>::NT), 0, s, args); break;
        case 64: hipLaunchKernelGGL((quantize_kernel<64, 64>), grid, dim3(FS<64, 64>::NT), 0, s, args); break;
        default: hipLaunchKernelGGL((quantize_kernel<128, 128>), grid, dim3(FS<128, 128>::NT), 0, s, args); break;
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

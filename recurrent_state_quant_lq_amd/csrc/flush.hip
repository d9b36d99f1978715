// flush.hip -- window boundary: rebuild the state, extract compensator rows,
// smooth, requantize (gfx950).  Also the standalone codec kernels.
//
// News article ("A linear-attention method cuts state ...", paragraph 3):
// one rebuild and one rounding of the state per window, at its end.  Forum
// mirror ("Abstract (translated)", techniques 2 and 3) and paragraph 4 of the
// news article: the few biggest outlier entries of the state stay in high
// precision as compensator tokens, and what is left is smoothed, then
// rounded.
//
// Reconstruction from the window-base state Hb and N buffered slots
// (k_i, g_i, m_i; m_i = u_i - Hb^T y_i, see decode.hip):
//     H = Gamma Hb + Kt^T M            (dk x dv,  contraction over N)
// with Kt[i][c] = exp(g_{N-1}[c] - g_i[c]) k_i[c], M = [m_0; ...; m_{N-1}] and
// Gamma = diag exp(g_{N-1}).  Gamma Hb is dequantized into the MFMA
// accumulators; each compensator row gamma(idx_c) cv_c is added to row idx_c
// by the 16 lanes that hold it.  At d = 128 with up to 16 slots Kt^T M runs on
// v_mfma_f32_16x16x32_bf16 over three-way bf16 splits of Kt and M (exact to
// fp32 rounding; split3_bf16), otherwise on v_mfma_f32_16x16x4_f32.
//
// Register layout ("D layout") of H in one workgroup: NW waves; lane l
// (li = l % 16, lg = l / 16) of wave w holds, for v4 register (rb, ct),
//     H[row(w, lg, rb, v)][16*ct + li],   row = w*16*RBW + lg*4*RBW + rb*4 + v,
// i.e. the MFMA accumulator layout (tile ct = columns 16ct..16ct+15) with the
// rows permuted so that a lane's 4*RBW rows are consecutive: one column's
// bytes of those rows are one 8-byte piece of the stored state (sq_off), and
// for one tile the pieces of a wave's 64 lanes are 512 contiguous bytes.
//
// The codec steps are single IEEE fp32 operations in a fixed order, so the
// int8 bytes, scales and compensator rows are a function of the fp32 H.
#include "lq_internal.h"

#include <atomic>

#pragma clang fp contract(off)

namespace lq {
namespace {

// Magnitudes below 2^-120 count as zero in the codec: a column that small
// keeps scale 1 and a row that small quantizes to zeros, so 1/s and 127/rho
// (which overflow fp32 below about 2^-121) stay finite.
constexpr float kTiny = 0x1p-120f;
constexpr int CMAX = 8;

typedef unsigned long long u64;

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
    static constexpr int KS = (DK + 63) / 64;
    static_assert(DK % 16 == 0 && RB % NW == 0 && (CT % NW == 0 || CT < NW), "tile shape");
    // every wave's rows lie in one 64-row half
    static_assert(16 * RBW <= 64 && 64 % (16 * RBW) == 0, "row halves");
    // a lane's RPL rows of one column are one run of the stored state (sq_off)
    static_assert(16 % RPL == 0, "row runs");
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

// A lane's values of one row in the D layout, one per column tile:
// x[ct] = p[16 ct] with p at the lane's column li.
template <int CT>
__device__ __forceinline__ void load_cols(const float* p, float (&x)[CT]) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) x[ct] = p[16 * ct];
}
template <int CT>
__device__ __forceinline__ void store_cols(float* p, const float (&x)[CT]) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) p[16 * ct] = x[ct];
}

__device__ __forceinline__ u64 ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Operands of v_mfma_f32_16x16x32_bf16.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Three-way bf16 split of 8 floats: x = x1 + x2 + x3 + e with x1 = bf16(x),
// x2 = bf16(x - x1), x3 = bf16(x - x1 - x2) (round to nearest even); both
// residuals are exact in fp32 and |e| <= 2^-27 |x|.  The six products
// x1 y1, x1 y2, x2 y1, x1 y3, x2 y2, x3 y1 of two split numbers are exact in
// fp32 and leave out terms of at most about 2^-25 |x y|.  Two values per dword,
// element 2e in the low half (the MFMA operand order).
__device__ __forceinline__ void split3_bf16(const float (&x)[8], uint4& p1, uint4& p2, uint4& p3) {
    uint32_t a[4], b[4], c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const f32x2 v = {x[2 * e], x[2 * e + 1]};
        const bf16x2 h1 = __builtin_convertvector(v, bf16x2);
        const f32x2 r1 = v - __builtin_convertvector(h1, f32x2);
        const bf16x2 h2 = __builtin_convertvector(r1, bf16x2);
        const f32x2 r2 = r1 - __builtin_convertvector(h2, f32x2);
        const bf16x2 h3 = __builtin_convertvector(r2, bf16x2);
        a[e] = __builtin_bit_cast(uint32_t, h1);
        b[e] = __builtin_bit_cast(uint32_t, h2);
        c[e] = __builtin_bit_cast(uint32_t, h3);
    }
    p1 = make_uint4(a[0], a[1], a[2], a[3]);
    p2 = make_uint4(b[0], b[1], b[2], b[3]);
    p3 = make_uint4(c[0], c[1], c[2], c[3]);
}

// Raw buffer over `bytes` bytes from base (gfx9 descriptor: 32-bit data format);
// loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const float* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ float buf_ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Rounding of y through the offset (y + 1.5 * 2^23, round to nearest even)
// with the sum's low byte written into byte B of w and the other bytes of w
// kept: an SDWA destination select with the unused bits preserved, so the
// bytes of four values are packed as they are rounded.
template <int B>
__device__ __forceinline__ void round_into_byte(uint32_t& w, float y, float off) {
    static_assert(B >= 1 && B <= 3, "bytes 1..3");
    if constexpr (B == 1)
        asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
            : "+v"(w) : "v"(y), "v"(off));
    else if constexpr (B == 2)
        asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
            : "+v"(w) : "v"(y), "v"(off));
    else
        asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
            : "+v"(w) : "v"(y), "v"(off));
}

// rint of four values (|y| <= 127) as two's-complement bytes, a first.
__device__ __forceinline__ uint32_t round_pack4(float a, float b, float c, float d) {
    const float off = kRoundOff;
    uint32_t w = __float_as_uint(a + off);       // byte 0; bytes 1..3 are overwritten
    round_into_byte<1>(w, b, off);
    round_into_byte<2>(w, c, off);
    round_into_byte<3>(w, d, off);
    return w;
}

// Maxima over the four 16-lane rows of a wave for four values at once, with
// the gfx950 row swaps (v_permlane32_swap: upper half of the first operand
// <-> lower half of the second; v_permlane16_swap: odd rows of the first <->
// even rows of the second).  Row r of the result holds the maximum over all
// 64 lanes' rows of (a, b, c, d)[r], at the lane's position within the row.
__device__ __forceinline__ uint32_t rows_umax4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(a, c, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(b, d, false, false);
    // rows of x: max(a0,a2), max(a1,a3), max(c0,c2), max(c1,c3); of y: the same for b and d
    const uint32_t x = umax(s0[0], s0[1]);
    const uint32_t y = umax(s1[0], s1[1]);
    const auto s2 = __builtin_amdgcn_permlane16_swap(x, y, false, false);
    return umax(s2[0], s2[1]);
}

// Maximum over the 64 lanes, in every lane: 16-lane rows by DPP, then the
// rows exchanged by the gfx950 row swaps (no scalar round trip).
__device__ __forceinline__ uint32_t wave_umax_v(uint32_t x) {
    x = group_umax<16>(x);
    const auto s = __builtin_amdgcn_permlane32_swap(x, x, false, false);   // rows 2, 3 | rows 0, 1
    x = umax(s[0], s[1]);
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);   // odd | even rows
    return umax(r[0], r[1]);
}

// Maxima over the 16 lanes of a lane group of N values per lane (non-negative
// floats as bit patterns), by halving exchanges: at step S the lanes whose lane
// bit 8 >> S is set keep the second half of their values and pass the first half
// to their partner (row mirror, then half mirror, then quad swaps), the others
// keep the first half; each keeps the maximum of its value and the partner's.
// Once one value is left the remaining steps are plain maxima.  The result at
// lane li is the maximum of value number sum_S bit_S(li) * (N >> (S + 1)), i.e.
// value k sits at the lanes li = k * (16 / N) (+ any of the lower bits).
template <int N, int S = 0>
__device__ __forceinline__ uint32_t halve_umax(const uint32_t* x, int li) {
    constexpr int ctrl = S == 0 ? DPP_MIRROR : S == 1 ? DPP_HALF_MIRROR : S == 2 ? DPP_XOR2 : DPP_XOR1;
    if constexpr (S == 4) {
        static_assert(N == 1, "16 lanes reduce at most 16 values");
        return x[0];
    } else if constexpr (N == 1) {
        const uint32_t v = umax(x[0], (uint32_t)dpp_i<ctrl>((int)x[0]));
        return halve_umax<1, S + 1>(&v, li);
    } else {
        const bool hi = (li & (8 >> S)) != 0;
        uint32_t y[N / 2];
#pragma unroll
        for (int j = 0; j < N / 2; ++j) {
            const uint32_t keep = hi ? x[j + N / 2] : x[j];
            const uint32_t send = hi ? x[j] : x[j + N / 2];
            y[j] = umax(keep, (uint32_t)dpp_i<ctrl>((int)send));
        }
        return halve_umax<N / 2, S + 1>(y, li);
    }
}

// LDS used by the codec stage.
template <int DK, int DV, int NW>
struct CodecLds {
    float m[DK];                 // row magnitudes
    uint32_t cm[NW][DV];         // column maxima per wave (bit patterns of non-negative floats)
    float sinv[DV];              // 1 / col_scale
};

// Codec of the state held in D layout (H is overwritten).  Writes sq
// (stored order, sq_off), r, s, idx, cv of one head; h_out (nullable,
// row-major fp32) receives H first.
template <int DK, int DV, int RBW, int CT, int NW>
__device__ void codec_store(v4f (&H)[RBW][CT], CodecLds<DK, DV, NW>& L, const CodecOut& out,
                            float* __restrict__ h_out, int C, int smooth) {
    constexpr int RPL = FS<DK, DV>::RPL;
    // the lane indices are recomputed here (an opaque copy of the thread id), so
    // the compiler keeps no codec address live through the caller's registers
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const int lane = t & 63, li = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int row0 = row_of<DK, DV>(w, lg, 0, 0);

    if (h_out) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float x[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) x[ct] = H[rb][ct][v];
                store_cols<CT>(h_out + (size_t)(row0 + rb * 4 + v) * DV + li, x);
            }
    }
    // row magnitudes (a lane's maximum starts at +0 and takes only |H|, so its
    // bit pattern orders like the value); lane li ends with row li / (16 / RPL)
    constexpr int LPR = 16 / RPL;             // lanes holding each row's result
    {
        uint32_t m[RPL];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float mx = 0.0f;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) mx = fmaxf(mx, fabsf(H[rb][ct][v]));
                m[rb * 4 + v] = __float_as_uint(mx);
            }
        const uint32_t mr = halve_umax<RPL>(m, li);
        if (li % LPR == 0) L.m[row0 + li / LPR] = __uint_as_float(mr);
    }
    lds_barrier();

    // The C largest rows, ties to the lower row: C rounds of a wave argmax
    // (every wave computes the same set).  A free row's key is its magnitude's
    // bit pattern plus one (same order; at most 0x7f800001), a taken or absent
    // row's key is 0, so the maximum is always a free row (C < DK).
    u64 lo = 0, hi = 0;
    {
        uint32_t ka = lane < DK ? __float_as_uint(L.m[lane]) + 1u : 0u;
        uint32_t kb = lane + 64 < DK ? __float_as_uint(L.m[lane + 64]) + 1u : 0u;
#pragma unroll
        for (int c = 0; c < CMAX; ++c)
            if (c < C) {
                const uint32_t mx = wave_umax_v(umax(ka, kb));
                const u64 ca = ballot(ka == mx), cb = ballot(kb == mx);
                if (ca) {
                    const int r = __builtin_ctzll(ca);
                    lo |= 1ull << r;
                    ka = lane == r ? 0u : ka;
                } else {
                    const int r = __builtin_ctzll(cb);
                    hi |= 1ull << r;
                    kb = lane == r ? 0u : kb;
                }
            }
    }
    // their positions: ascending row order
    if (w == 0) {
        u64 l2 = lo, h2 = hi;
        int mine = 0;
#pragma unroll
        for (int c = 0; c < CMAX; ++c)
            if (c < C) {
                const int r = l2 ? __builtin_ctzll(l2) : 64 + __builtin_ctzll(h2);
                if (l2)
                    l2 &= l2 - 1ull;
                else
                    h2 &= h2 - 1ull;
                if (lane == c) mine = r;
            }
        if (lane < C) st_nt(out.idx + lane, mine);
    }
    // compensator rows stored by the lanes that hold them (one row: 16
    // lanes, one column of each tile), residual rows zeroed
    {
        // a wave's rows lie in one 32-row quarter: its bits, and the set bits below it
        static_assert(16 * RBW <= 32, "row quarters");
        const int wb = w * 16 * RBW;
        const u64 hm = wb >= 64 ? hi : lo;
        const uint32_t qm = (wb & 32) ? (uint32_t)(hm >> 32) : (uint32_t)hm;
        const int o = row0 & 31;
        const uint32_t bits = (qm >> o) & ((1u << RPL) - 1u);
        if (ballot(bits != 0)) {
            const int base = (wb >= 64 ? __popcll(lo) : 0) + ((wb & 32) ? __popc((uint32_t)hm) : 0) +
                             __popc(qm & ((1u << o) - 1u));
#pragma unroll
            for (int k = 0; k < RPL; ++k)
                if ((bits >> k) & 1u) {
                    float* dst = out.cv + (size_t)(base + __popc(bits & ((1u << k) - 1u))) * DV + li;
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) st_nt(dst + 16 * ct, H[k / 4][ct][k % 4]);
                }
        }
        // zeroed; a register is visited only if some lane of the wave holds a
        // compensator row in it
#pragma unroll
        for (int k = 0; k < RPL; ++k)
            if (ballot((bits >> k) & 1u)) {
                const bool z = (bits >> k) & 1u;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) H[k / 4][ct][k % 4] = z ? 0.0f : H[k / 4][ct][k % 4];
            }
    }
    // column maxima of the residual: over this lane's rows, then over the
    // wave's four lane groups (the four lane groups hold the same columns)
    {
        uint32_t cm[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            float mx = 0.0f;
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                for (int v = 0; v < 4; ++v) mx = fmaxf(mx, fabsf(H[rb][ct][v]));
            cm[ct] = __float_as_uint(mx);
        }
        if constexpr (CT % 4 == 0) {
            // lane group lg receives column 16 (4m + lg) + li
#pragma unroll
            for (int m4 = 0; m4 < CT / 4; ++m4)
                L.cm[w][16 * (4 * m4 + lg) + li] = rows_umax4(cm[4 * m4], cm[4 * m4 + 1], cm[4 * m4 + 2], cm[4 * m4 + 3]);
        } else {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                uint32_t x = umax(cm[ct], __float_as_uint(swz_xor16(__uint_as_float(cm[ct]))));
                x = umax(x, (uint32_t)__shfl_xor((int)x, 32, 64));
                if (lg == 0) L.cm[w][16 * ct + li] = x;
            }
        }
    }
    lds_barrier();
    if (t < DV) {
        uint32_t mx = 0u;
#pragma unroll
        for (int i = 0; i < NW; ++i) mx = umax(mx, L.cm[i][t]);
        const float m = __uint_as_float(mx);
        const float sj = (smooth && m >= kTiny) ? m : 1.0f;
        st_nt(out.s + t, sj);
        L.sinv[t] = 1.0f / sj;
    }
    lds_barrier();
    // smoothing and row maxima
    float inv[CT];
    load_cols<CT>(&L.sinv[li], inv);
    uint32_t rho[RPL];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float mx = 0.0f;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                H[rb][ct][v] = H[rb][ct][v] * inv[ct];
                mx = fmaxf(mx, fabsf(H[rb][ct][v]));
            }
            rho[rb * 4 + v] = __float_as_uint(mx);
        }
    // row scales: lane li of a row group holds rho of row row0 + li / LPR and
    // divides for it; the 16 lanes then share the RPL multipliers
    float lam[RPL];
    {
        const float my = __uint_as_float(halve_umax<RPL>(rho, li));
        const bool live = my >= kTiny;
        const float lmy = live ? 127.0f / my : 0.0f;
        if (li % LPR == 0) st_nt(out.r + row0 + li / LPR, live ? my / 127.0f : 0.0f);
        row_bcast_all<RPL, LPR>(lmy, lam);
    }
    // rounding through the offset form; one column's RPL bytes per store,
    // 512 contiguous bytes per tile and wave.
    // The clamp to +-127 never binds: |Y| <= rho and lam = RN(127/rho) give
    // |Y * lam| <= 127 (1 + 2^-24)^2, which rounds to at most 127.
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        float y[RPL];
#pragma unroll
        for (int k = 0; k < RPL; ++k) y[k] = H[k / 4][ct][k % 4] * lam[k];
        int8_t* dst = out.sq + sq_off<DK>(row0, li) + ct * sq_tile_stride<DK>();
        // streamed: a wave's pieces of one tile are 512 contiguous bytes, i.e. whole lines
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        if constexpr (RPL == 8)
            __builtin_nontemporal_store(u32x2{round_pack4(y[0], y[1], y[2], y[3]), round_pack4(y[4], y[5], y[6], y[7])},
                                        reinterpret_cast<u32x2*>(dst));
        else
            __builtin_nontemporal_store(round_pack4(y[0], y[1], y[2], y[3]), reinterpret_cast<uint32_t*>(dst));
    }
}

struct FlushArgs {
    int8_t* sq;
    float* r;
    float* s;
    int32_t* idx;
    float* cv;
    float* bk;                // written only by the fused decode (slot N-1)
    float* bm;
    float* bg;
    float* h_out;
    const int32_t* n_dev;     // per batch row (ragged windows; DEC: positions), or null: N for every row
    int W;
    int C;
    int N;
    int smooth;
    int H;
    // the token decoded into slot N-1 first (decode fused into the flush)
    const void* q;            // q, k, v, o: fp32 or bf16 (the kernel's TI)
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    void* o;
    // staggered start of the first round (0 ticks: none): workgroup b < stag_wgs
    // waits (b / stag_cus) * stag_ticks ticks of the 100 MHz real-time counter
    unsigned stag_ticks;
    unsigned stag_cus;
    unsigned stag_wgs;
};

// Rows 0..NPAD-1 of a [rows][D] fp32 block (row index clamped to rmax) into
// LDS dst[NPAD][D]; 16-byte pieces, one kilobyte per wave-wide copy, copies
// spread over the NW waves.  Row rsub (if >= 0) comes from the vector sub,
// whose first sub_len floats' worth of bytes are copied (D, or D/2 for a
// bf16 vector, which lands in the first half of the row).
template <int NPAD, int D, int NW>
__device__ __forceinline__ void dma_rows(const float* src, int rmax, float* dst, int w, int lane,
                                         int rsub = -1, const float* sub = nullptr, int sub_len = D) {
    constexpr int NCOPY = NPAD * D / 256;
    static_assert((NPAD * D) % 256 == 0, "block of whole copies");
#pragma unroll
    for (int i = 0; i < (NCOPY + NW - 1) / NW; ++i) {
        const int cp = i * NW + w;
        if (cp < NCOPY) {
            const int e = cp * 256 + 4 * lane;
            const int row = min(e / D, rmax);
            if (row != rsub) lds_dma16(src + (size_t)row * D + e % D, dst + cp * 256);
            else if (e % D < sub_len) lds_dma16(sub + e % D, dst + cp * 256);
        }
    }
}

// The window contraction on bf16 MFMAs with three-way operand splits (d = 128,
// up to 16 slots); the fp32 MFMA otherwise.
template <int DK, int NPAD>
struct Bx3 {
    static constexpr bool on = DK == 128 && NPAD == 16;
    static constexpr int SIDE = 3 * NPAD * DK * 2;                 // bytes of one side's three parts
};

// Workgroup LDS of the flush kernel (byte offsets).  With the bf16 contraction
// the buffered rows are loaded into registers, not copied here, and the split
// operands (M parts, then Kt parts) take the rows' region from MB on.
template <int DK, int DV, int NPAD, bool KDA, bool DEC>
struct FlushLds {
    static constexpr int RS = 0;                                   // r | s | cv rows
    static constexpr int MISC = RS + (2 + CMAX) * DK * 4;          // idx; 8: beta, 9: alpha (scalar)
    static constexpr int GS = MISC + 64;                           // scalar log-decays
    static constexpr int MB = GS + 4 * 32;                         // buffered m rows
    static constexpr int KB = MB + NPAD * DV * 4;                  // buffered keys
    static constexpr int GB = KB + NPAD * DK * 4;                  // per-key log-decays
    static constexpr int ROWS_END = GB + (KDA ? NPAD * DK * 4 : 0);
    static constexpr int PARTS = MB;                               // bf16 operand parts (aliasing)
    static constexpr int PARTS_END = Bx3<DK, NPAD>::on ? MB + 2 * Bx3<DK, NPAD>::SIDE : 0;
    static constexpr int TOK = ROWS_END > PARTS_END ? ROWS_END : PARTS_END;   // token q | v | k | alpha (DEC)
    static constexpr int GAM = TOK + (DEC ? 4 * DK * 4 : 0);       // per-key Gamma (KDA)
    static constexpr int CODEC = GAM + (KDA ? DK * 4 : 0);         // codec stage; GEMV partials (DEC)
    static constexpr int NWF = DK / 16 < 4 ? DK / 16 : 4;
    static constexpr int CODEC_BYTES = (int)sizeof(CodecLds<DK, DV, NWF>);
    static constexpr int GEMV_BYTES = DEC ? (2 * DV + 1) * NWF * 4 : 0;     // DEC partials share the region
    static constexpr int BYTES = CODEC + (CODEC_BYTES > GEMV_BYTES ? CODEC_BYTES : GEMV_BYTES);
};

// DEC = true: first decode one token into slot n = N-1 (the window's last
// slot when N = W), then flush N slots, in one launch.  With Gamma =
// diag e^{g_n}, the flush's registers after the window terms of slots i < n
// hold H' = Gamma Hb + sum_{i<n} Kt_i m_i^T, and
//     H'^T q = Hb^T (e^{g_n} o q) + sum_{i<n} a_i m_i,
//     H'^T k = Hb^T (e^{g_n} o k) + sum_{i<n} rr_i m_i
// (compensator rows included), the two sums of the decode step; so
// m_n = beta (v - H'^T k), o = H'^T q + <q, k> m_n, and H = H' + k m_n^T.
// The GEMVs run on the fp32 registers (fma, lane-group rows summed with the
// row swaps, waves through LDS).
// Registers sized for the workgroups per CU (one wave per SIMD each) that the
// LDS allows: 4 with up to 16 slots; with 32, 3 (scalar decay) or 2 (per-key).
template <int DK, int DV, int WM, bool KDA, bool DEC, typename TI>
__global__ __launch_bounds__((FS<DK, DV>::NT))
__attribute__((amdgpu_waves_per_eu(WM <= 16 ? 4 : (KDA ? 2 : 3), WM <= 16 ? 4 : (KDA ? 2 : 3))))
void flush_kernel(FlushArgs a) {
    using S = FS<DK, DV>;
    constexpr int RBW = S::RBW, CT = S::CT, NW = S::NW, RPL = S::RPL;
    constexpr int NPAD = WM <= 16 ? 16 : 32;   // slots padded to the MFMA size
    constexpr bool BX3 = Bx3<DK, NPAD>::on;
    using RBy = RowBytes<RPL>;
    using LY = FlushLds<DK, DV, NPAD, KDA, DEC>;

    __shared__ __align__(16) char smem[LY::BYTES];
    float* s_r = reinterpret_cast<float*>(smem + LY::RS);
    float* s_s = s_r + DK;
    float* s_cv = s_r + 2 * DK;                                    // [CMAX][DV]
    int* s_idx = reinterpret_cast<int*>(smem + LY::MISC);
    float* s_gs = reinterpret_cast<float*>(smem + LY::GS);         // [NPAD] (scalar decay)
    float* s_M = reinterpret_cast<float*>(smem + LY::MB);          // [NPAD][DV]
    float* s_K = reinterpret_cast<float*>(smem + LY::KB);          // [NPAD][DK]
    float* s_G = reinterpret_cast<float*>(smem + LY::GB);          // [NPAD][DK] (per-key decay)
    float* s_tq = reinterpret_cast<float*>(smem + LY::TOK);        // token q [DK] (DEC)
    float* s_tv = s_tq + DK;                                       // token v [DV] (DEC)
    float* s_tk = s_tv + DV;                                       // token k [DK] (DEC)
    float* s_tal = s_tk + DK;                                      // token alpha [DK] (DEC, per-key)
    float* s_gam = reinterpret_cast<float*>(smem + LY::GAM);       // Gamma per row (per-key, bf16 path)
    float* s_pq = reinterpret_cast<float*>(smem + LY::CODEC);      // [2][NW][DV] GEMV partials (DEC)
    float* s_pk = s_pq + NW * DV;
    auto& L = *reinterpret_cast<CodecLds<DK, DV, NW>*>(smem + LY::CODEC);

    const int t = threadIdx.x;
    const int lane = t & 63, li = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const size_t head = blockIdx.x;
    const int W = a.W, C = a.C;
    // n_dev: the slot count per batch row, or (DEC) the decoded token's position
    // (uniform: every value derived from it stays scalar)
    const int N = __builtin_amdgcn_readfirstlane(a.n_dev ? a.n_dev[head / (unsigned)a.H] + (DEC ? 1 : 0) : a.N);
    if (N <= 0 || N > W) return;                  // nothing buffered (or out of range): untouched
    const int n = N - 1;                          // DEC: the decoded token's slot
    // Staggered start.  The dispatcher fills the CUs slot by slot (workgroup b
    // goes to slot b / CUs of its CU), and loads issued together land in about
    // that order, so a first round started all at once computes nothing until
    // most of its loads have landed.  Slot s waits s times the time one slot's
    // loads take to stream in, so the earlier slots compute meanwhile.  The
    // wait is bounded (the counter only advances; at most 4096 sleeps).
    if (a.stag_ticks && blockIdx.x < a.stag_wgs) {
        const unsigned slot = blockIdx.x / a.stag_cus;
        if (slot) {
            const unsigned long long t_end = __builtin_amdgcn_s_memrealtime() + (unsigned long long)a.stag_ticks * slot;
            for (int i = 0; i < 4096 && __builtin_amdgcn_s_memrealtime() < t_end; ++i) __builtin_amdgcn_s_sleep(2);
        }
    }

    const int8_t* sq = a.sq + head * (DK * DV);
    // buffered rows up to the last one read (DEC: slot n's row is the token's); the rows
    // past it repeat it, so they cost no further memory traffic
    const int rlast = __builtin_amdgcn_readfirstlane(max((DEC ? n : N) - 1, 0));
    // slots in the window terms; DEC: slot n (Kt row = k, its m from the decode) is a
    // rank-1 update afterwards
    const int NM = DEC ? n : N;

    // ---- loads (unconditional) --------------------------------------------------------------------
    {
        // r, s, compensator rows (DK/4 lanes per vector of 16-byte pieces)
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
            if (src) lds_dma16(src + 4 * (lane % SEGL), s_r + s0 * DK);
        }
        if constexpr (DEC) {
            // token q, v, k [, alpha]
            constexpr int NTS = KDA ? 4 : 3;
            for (int s0 = SPI * w; s0 < NTS; s0 += SPI * NW) {
                const float* src = nullptr;
#pragma unroll
                for (int q = 0; q < SPI; ++q) {
                    const int sg = s0 + q;
                    const float* p = sg == 0 ? reinterpret_cast<const float*>(static_cast<const TI*>(a.q) + head * DK)
                                   : sg == 1 ? reinterpret_cast<const float*>(static_cast<const TI*>(a.v) + head * DV)
                                   : sg == 2 ? reinterpret_cast<const float*>(static_cast<const TI*>(a.k) + head * DK)
                                   : sg < NTS ? a.alpha + head * DK : nullptr;
                    if (my == q) src = p;
                }
                // bf16 q, v and k fill the first half of their segments
                const bool in_row = sizeof(TI) == 4 || s0 + my >= 3 || 8 * (lane % SEGL) < DK;
                if (src && in_row) lds_dma16(src + 4 * (lane % SEGL), s_tq + s0 * DK);
            }
        }
        if (w == 0) {
            const void* src4 = nullptr;
            if (lane < C) src4 = a.idx + head * C + lane;
            else if (DEC && lane == 8) src4 = a.beta + head;
            else if (DEC && !KDA && lane == 9) src4 = a.alpha + head;
            if (src4) lds_dma4(src4, s_idx);
        }
        if constexpr (!BX3) {
            if (!KDA && w == NW - 1 && lane < NPAD) lds_dma4(a.bg + head * W + min(lane, W - 1), s_gs);
            dma_rows<NPAD, DV, NW>(a.bm + head * (size_t)W * DV, rlast, s_M, w, lane);
            dma_rows<NPAD, DK, NW>(a.bk + head * (size_t)W * DK, rlast, s_K, w, lane);
            if constexpr (KDA) dma_rows<NPAD, DK, NW>(a.bg + head * (size_t)W * DK, rlast, s_G, w, lane);
        }
    }
    // bf16 contraction: lane t holds column j of the buffered m and key rows (and per-key
    // log-decays) for the 8 slots s = 8 hs .. 8 hs + 7 of its half, in registers (no LDS
    // round trip, and no barrier between reading the rows and writing the parts).
    // g_last: the log-decay of the last slot, g_{N-1}, or (DEC) the decoded token's
    // g_n = g_{n-1} + log alpha; per head (scalar decay) or for column j (per-key).
    const int j = t & (DK - 1), hs = __builtin_amdgcn_readfirstlane(t / DK);   // hs: uniform in a wave
    [[maybe_unused]] float mv[8], kv[8], gv[8];
    [[maybe_unused]] float gs_l = 0.0f, g_prev = 0.0f, al = 1.0f;
    if constexpr (BX3) {
        // g_prev: g_{n-1} (DEC; 0 at n = 0) or g_{N-1}; al: the token's decay (DEC);
        // per head (scalar decay) or for column j (per-key)
        if constexpr (KDA) {
            const float* bg = a.bg + head * (size_t)W * DK + j;
            g_prev = DEC ? (n > 0 ? bg[(n - 1) * DK] : 0.0f) : bg[(N - 1) * DK];
            if constexpr (DEC) al = a.alpha[head * DK + j];
        } else {
            const float* bg = a.bg + head * (size_t)W;
            g_prev = DEC ? (n > 0 ? bg[n - 1] : 0.0f) : bg[N - 1];
            if constexpr (DEC) al = a.alpha[head];
            // lane (8 hs + e) % 64 holds slot 8 hs + e's log-decay, e < 8
            gs_l = bg[min(8 * hs + (lane & 7), rlast)];
        }
        // buffer loads: the head's rows as one buffer, the row in the scalar offset and
        // the lane's column in the vector offset (no per-load address arithmetic)
        const uint32_t jb = 4u * (uint32_t)j;
        const auto rm = buf_rsrc(a.bm + head * (size_t)W * DV, W * DV * 4);
        const auto rk = buf_rsrc(a.bk + head * (size_t)W * DK, W * DK * 4);
        [[maybe_unused]] const auto rg = buf_rsrc(a.bg + head * (size_t)W * DK, W * DK * 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int sl = min(8 * hs + e, rlast);               // uniform
            mv[e] = buf_ld(rm, jb, sl * DV * 4);
            kv[e] = buf_ld(rk, jb, sl * DK * 4);
            if constexpr (KDA) gv[e] = buf_ld(rg, jb, sl * DK * 4);
        }
    }
    // D-layout bytes of the base state: column 16 ct + li, this lane's RPL rows
    const int row0 = row_of<DK, DV>(w, lg, 0, 0);
    typename RBy::T hb[CT];
    {
        const auto rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(sq), 0, DK * DV, 0x00020000);
        const uint32_t vo = (uint32_t)sq_off<DK>(row0, li);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            if constexpr (RPL == 8)
                hb[ct] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq, vo, ct * sq_tile_stride<DK>(), 0));
            else
                hb[ct] = __builtin_amdgcn_raw_buffer_load_b32(rq, vo, ct * sq_tile_stride<DK>(), 0);
        }
    }
    // The state-byte loads stay issued ahead of the split: the split's inputs pass through
    // empty asm statements after them, so the compiler cannot start the split (and wait for
    // its loads) before it has issued the state-byte loads.  (With copies to LDS in flight
    // that wait covers every load: the compiler does not order copies to LDS with register
    // loads.)
    asm volatile("" ::: "memory");
    if constexpr (BX3) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            asm volatile("" : "+v"(mv[e]));
            asm volatile("" : "+v"(kv[e]));
            if constexpr (KDA) asm volatile("" : "+v"(gv[e]));
        }
        asm volatile("" : "+v"(g_prev));
        asm volatile("" : "+v"(al));
        if constexpr (!KDA) asm volatile("" : "+v"(gs_l));
    }
    // g_last: the decoded token's g_n = g_{n-1} + log alpha (DEC), else g_{N-1}
    [[maybe_unused]] const float gl_b = DEC ? g_prev + logf(al) : g_prev;
    [[maybe_unused]] const float gl_j = gl_b, gl_h = gl_b;

    if constexpr (BX3) {
        // Kt[s][j] = e^{g_last - g_s} k_s[j], zero from slot NM on (those slots' m rows repeat
        // a written row, so their products are zero); M and Kt split into three bf16 parts
        // each, stored as [part][half][column or row] runs of 8 slots.  The parts region
        // is no copy's target, so it is written before the loads have all landed.
        char* parts = smem + LY::PARTS;
        float ev[8];
        if constexpr (KDA) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ev[e] = 8 * hs + e < NM ? __expf(gl_j - gv[e]) : 0.0f;
            if (hs == 0) s_gam[j] = __expf(gl_j);
        } else {
            // the half's 8 factors, one per lane, then read from lanes 0..7 (hs is uniform in a wave)
            const float es = 8 * hs + (lane & 7) < NM ? __expf(gl_h - gs_l) : 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ev[e] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(es), e));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) kv[e] = ev[e] * kv[e];
        uint4 p[3];
        split3_bf16(mv, p[0], p[1], p[2]);
#pragma unroll
        for (int q = 0; q < 3; ++q) *reinterpret_cast<uint4*>(parts + ((q * 2 + hs) * DV + j) * 16) = p[q];
        split3_bf16(kv, p[0], p[1], p[2]);
#pragma unroll
        for (int q = 0; q < 3; ++q)
            *reinterpret_cast<uint4*>(parts + Bx3<DK, NPAD>::SIDE + ((q * 2 + hs) * DK + j) * 16) = p[q];
    }
    all_loads_barrier();                        // copies landed; parts (and s_gam) written

    // g_last for the fp32-MFMA paths, from the copied rows
    float gn_s = gl_h;
    if constexpr (DEC && !KDA && !BX3) gn_s = (n > 0 ? s_gs[n - 1] : 0.0f) + logf(__int_as_float(s_idx[9]));
    if constexpr (!DEC && !KDA && !BX3) gn_s = s_gs[N - 1];
    auto glast = [&](int row) -> float {
        if constexpr (DEC)
            return KDA ? (n > 0 ? s_G[(n - 1) * DK + row] : 0.0f) + logf(s_tal[row]) : gn_s;
        else
            return KDA ? s_G[(N - 1) * DK + row] : gn_s;
    };
    if constexpr (DEC) {
        // slot n's key and log-decay
        if (t < DK) {
            st_nt(a.bk + head * (size_t)W * DK + (size_t)n * DK + t, seg_ld<TI>(s_tk, t));
            if constexpr (KDA) st_nt(a.bg + head * (size_t)W * DK + (size_t)n * DK + t, BX3 ? gl_j : glast(t));
            else if (t == 0) st_nt(a.bg + head * (size_t)W + n, gn_s);
        }
    }

    // ---- H = Gamma Hb + Kt^T M (MFMA, accumulating in place) ------------------------------------
    // fp32 MFMA: A operands Kt[slot][rowa], rowa = row(w, li/4, rb, li%4), slot = 4*ks + lg
    // (0 from NM on).
    [[maybe_unused]] float ka[RBW][NPAD / 4];
    if constexpr (BX3) {
        // the bf16 parts are in LDS
    } else if constexpr (KDA) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            const int rowa = row_of<DK, DV>(w, li >> 2, rb, li & 3);
            const float gl = glast(rowa);
#pragma unroll
            for (int ks = 0; ks < NPAD / 4; ++ks) {
                const int slot = 4 * ks + lg;
                ka[rb][ks] = slot < NM ? __expf(gl - s_G[slot * DK + rowa]) * s_K[slot * DK + rowa] : 0.0f;
            }
        }
    } else {
        const float gl = glast(0);
#pragma unroll
        for (int ks = 0; ks < NPAD / 4; ++ks) {
            const int slot = 4 * ks + lg;
            const float e = __expf(gl - s_gs[slot]);
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                const int rowa = row_of<DK, DV>(w, li >> 2, rb, li & 3);
                ka[rb][ks] = slot < NM ? e * s_K[slot * DK + rowa] : 0.0f;
            }
        }
    }
    v4f H[RBW][CT];
    {
        float sc[CT], rr[RPL], gm[RPL];
        load_cols<CT>(s_s + li, sc);
        load_floats<RPL>(s_r + row0, rr);
        if constexpr (KDA && BX3) {
            load_floats<RPL>(s_gam + row0, gm);
        } else if constexpr (KDA) {
#pragma unroll
            for (int k = 0; k < RPL; ++k) gm[k] = __expf(glast(row0 + k));
        } else {
            const float g = __expf(glast(0));
#pragma unroll
            for (int k = 0; k < RPL; ++k) gm[k] = g;
        }
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float rg = rr[rb * 4 + v] * gm[rb * 4 + v];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) H[rb][ct][v] = (RBy::get(hb[ct], rb * 4 + v) * rg) * sc[ct];
            }
    }
    // compensator rows: H[idx_c] += gamma(idx_c) cv_c, added by the 16 lanes
    // that hold row idx_c (a uniform branch picks the register)
    for (int c = 0; c < C; ++c) {
        const int ic = __builtin_amdgcn_readfirstlane(s_idx[c]);
        const int r = ic - w * 16 * RBW;                  // row among this wave's rows
        if (r < 0 || r >= 16 * RBW) continue;             // another wave's row
        float g;
        if constexpr (KDA && BX3) g = s_gam[ic];
        else g = __expf(glast(ic));
        float cvv[CT];
        load_cols<CT>(s_cv + c * DV + li, cvv);
        if (lg == r / RPL) {
            const int k = r % RPL;
#pragma unroll
            for (int kk = 0; kk < RPL; ++kk)
                if (kk == k) {
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        H[kk / 4][ct][kk % 4] = __builtin_fmaf(g, cvv[ct], H[kk / 4][ct][kk % 4]);
                }
        }
    }

    // window terms
    if constexpr (BX3) {
        // three K = 32 steps, each lane group pairing one part of Kt with one part of M for
        // its half of the slots: x1 y1, x2 y1, x1 y3 (lane groups 0, 1) and x1 y2, x2 y2,
        // x3 y1 (lane groups 2, 3), x = Kt, y = M
        const char* parts = smem + LY::PARTS;
        const int hs = lg & 1, hi = lg >> 1;
        if (NM > 0) {
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const int pa = m == 0 ? 0 : m == 1 ? 1 : (hi ? 2 : 0);
                const int pb = m < 2 ? hi : (hi ? 0 : 2);
                bf16x8 A[RBW];
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb) {
                    const int rowa = row_of<DK, DV>(w, li >> 2, rb, li & 3);
                    A[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                        parts + Bx3<DK, NPAD>::SIDE + ((pa * 2 + hs) * DK + rowa) * 16));
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const bf16x8 bv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                        parts + ((pb * 2 + hs) * DV + 16 * ct + li) * 16));
#pragma unroll
                    for (int rb = 0; rb < RBW; ++rb)
                        H[rb][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rb], bv, H[rb][ct], 0, 0, 0);
                }
            }
        }
    } else {
        // fp32: B = M rows (rows from NM on are zero; the buffer may hold anything there)
#pragma unroll
        for (int ks = 0; ks < NPAD / 4; ++ks) {
            if (4 * ks < NM) {
                float bm[CT];
                load_cols<CT>(&s_M[(4 * ks + lg) * DV + li], bm);
                if (4 * ks + 4 > NM) {             // uniform: the step runs past slot NM - 1
                    const bool live = 4 * ks + lg < NM;
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) bm[ct] = live ? bm[ct] : 0.0f;
                }
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        H[rb][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[rb][ks], bm[ct], H[rb][ct], 0, 0, 0);
            }
        }
    }

    // ---- DEC: the token of slot n.  H now holds Gamma Hb + sum_{i<n} Kt_i m_i^T, so
    //      H^T q = Hb^T (e^{g_n} o q) + sum_{i<n} a_i m_i and H^T k likewise with rr_i:
    //      m_n = beta (v - H^T k), o = H^T q + <q, k> m_n, then H += k m_n^T ------------------
    if constexpr (DEC) {
        float* s_an = s_pk + NW * DV;                              // [NW] partial <q, k>
        {
            float an = t < DK ? seg_ld<TI>(s_tq, t) * seg_ld<TI>(s_tk, t) : 0.0f;
            an = group_sum<64>(an);
            if (lane == 0) s_an[w] = an;
        }
        // x = q, then k: column partials over this lane's rows, totals over the
        // wave's four lane-group rows, then over the waves in LDS
#pragma unroll
        for (int vec = 0; vec < 2; ++vec) {
            float p[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) p[ct] = 0.0f;
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                float x[4];
                seg_ld_n<4, TI>(vec ? s_tk : s_tq, row0 + 4 * rb, x);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int v = 0; v < 4; ++v) p[ct] = __builtin_fmaf(H[rb][ct][v], x[v], p[ct]);
            }
            float* dst = s_pq + vec * NW * DV + w * DV + li;
            if constexpr (CT % 4 == 0) {
                // row r of rows_sum4's result: the total of tile 4m + r's column
#pragma unroll
                for (int m = 0; m < CT / 4; ++m)
                    dst[16 * (4 * m + lg)] = rows_sum4(p[4 * m], p[4 * m + 1], p[4 * m + 2], p[4 * m + 3]);
            } else {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    p[ct] += swz_xor16(p[ct]);
                    p[ct] += __shfl_xor(p[ct], 32, 64);
                }
                if (lg == 0) store_cols<CT>(dst, p);
            }
        }
        lds_barrier();
        if (t < DV) {
            const int j = t;
            float hq = 0.0f, hk = 0.0f, aq = 0.0f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                hq += s_pq[ww * DV + j];
                hk += s_pk[ww * DV + j];
                aq += s_an[ww];
            }
            const float mn = __int_as_float(s_idx[8]) * (seg_ld<TI>(s_tv, j) - hk);
            s_M[n * DV + j] = mn;
            st_nt(a.bm + head * (size_t)W * DV + (size_t)n * DV + j, mn);
            tok_st<TI>(a.o, head * DV + j, hq + aq * mn);
        }
        lds_barrier();
        {
            float mv[CT];
            load_cols<CT>(s_M + n * DV + li, mv);
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                float xk[4];
                seg_ld_n<4, TI>(s_tk, row0 + 4 * rb, xk);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int v = 0; v < 4; ++v) H[rb][ct][v] = __builtin_fmaf(xk[v], mv[ct], H[rb][ct][v]);
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
            load_cols<CT>(h + (size_t)row_of<DK, DV>(w, lg, rb, v) * DV + li, x);
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
    if (t < a.C) s_pos[a.idx[head * a.C + t] & (DK - 1)] = t;
    __syncthreads();
    const int8_t* sq = a.sq + head * (DK * DV);
    const float* r = a.r + head * DK;
    const float* s = a.s + head * DV;
    float* h = a.h + head * (size_t)DK * DV;
    for (int e = t; e < DK * DV; e += 256) {
        const int row = e / DV, col = e % DV;
        const int p = s_pos[row];
        float x = ((float)sq[sq_off<DK>(row, col)] * r[row]) * s[col];
        if (p >= 0) x += a.cv[(head * a.C + p) * (size_t)DV + col];
        h[e] = x;
    }
}

// Compute units of the current device, cached per device (0 if unknown).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 0;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

// The rate the first round's loads are taken to stream in at when the start
// is staggered: 55,000 bytes per 10 ns tick, i.e. 5.5 TB/s (tuned by
// measurement at B = 64, H = 32, d = 128: slot delays of 1.3-1.7 us, i.e. 256
// heads' loads at 5.5-7 TB/s, were best, 2.1 us worse).
constexpr size_t kStaggerBytesPerTick = 55000;

template <int DK, int WM, bool KDA, bool DEC, typename TI>
hipError_t flush_launch(const lq_dims& d, const FlushArgs& args_in, hipStream_t s) {
    auto kernel = flush_kernel<DK, DK, WM, KDA, DEC, TI>;
    const dim3 grid((unsigned)d.B * (unsigned)d.H), block(FS<DK, DK>::NT);
    // resident workgroups per CU of this kernel (cached; 0 if the query fails)
    static std::atomic<int> occ{-1};
    int slots = occ.load(std::memory_order_relaxed);
    if (slots < 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&slots, kernel, (int)block.x, 0) != hipSuccess) slots = 0;
        occ.store(slots, std::memory_order_relaxed);
    }
    FlushArgs args = args_in;
    const int cus = device_cus();
    // only launches of more than one round in which every head has work: a
    // launch that fits at once may run beside other work (e.g. another stream's),
    // which sleeping workgroups would keep out of their CU slots, and with
    // per-row slot counts most rows may have nothing to do
    if (!args_in.n_dev && cus > 0 && slots > 1 && grid.x > (unsigned)cus * (unsigned)slots) {
        // bytes a head reads before it computes: codec, buffered rows (at most W - 1
        // with a decoded token, W without), the token's vectors
        const size_t gd = KDA ? DK : 1;
        const size_t rows = DEC ? d.W - 1 : d.W;
        size_t head = (size_t)DK * DK + 4 * (2 * DK + (size_t)d.C * DK + d.C) + rows * 4 * (2 * DK + gd);
        if (DEC) head += sizeof(TI) * 3 * DK + (KDA ? 4 * DK : 8);
        args.stag_ticks = (unsigned)((size_t)cus * head / kStaggerBytesPerTick);
        args.stag_cus = (unsigned)cus;
        args.stag_wgs = (unsigned)cus * (unsigned)slots;
    }
    return launch_kernel(DEC ? LQ_KERNEL_DECODE_FLUSH : LQ_KERNEL_FLUSH, kernel, grid, block, s, args);
}

template <int DK, int WM, bool KDA, bool DEC>
hipError_t flush_t(const lq_dims& d, const FlushArgs& args, hipStream_t s) {
    if (DEC && d.io_dtype == LQ_IO_BF16) return flush_launch<DK, WM, KDA, DEC, uint16_t>(d, args, s);
    return flush_launch<DK, WM, KDA, DEC, float>(d, args, s);
}

template <int DK, bool DEC>
hipError_t flush_dk(const lq_dims& d, const FlushArgs& args, hipStream_t s) {
    const bool kda = d.decay_mode == LQ_DECAY_PER_KEY;
    if (d.W <= 16) return kda ? flush_t<DK, 16, true, DEC>(d, args, s) : flush_t<DK, 16, false, DEC>(d, args, s);
    return kda ? flush_t<DK, 32, true, DEC>(d, args, s) : flush_t<DK, 32, false, DEC>(d, args, s);
}

template <bool DEC>
hipError_t flush_any(const lq_dims& d, const FlushArgs& args, hipStream_t s) {
    switch (d.dk) {
        case 16: return flush_dk<16, DEC>(d, args, s);
        case 64: return flush_dk<64, DEC>(d, args, s);
        default: return flush_dk<128, DEC>(d, args, s);
    }
}

}  // namespace

hipError_t launch_flush(const lq_dims& d, const lq_state& st, int n_buffered, const int32_t* n_dev,
                        float* h_out, hipStream_t s) {
    FlushArgs args{st.sq, st.row_scale, st.col_scale, st.comp_idx, st.comp_val,
                   st.buf_k, st.buf_m, st.buf_g, h_out, n_dev, d.W, d.C, n_buffered, d.smooth, d.H,
                   nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, 0};
    return flush_any<false>(d, args, s);
}

hipError_t launch_decode_flush(const lq_dims& d, const lq_state& st, int pos, const int32_t* pos_dev,
                               const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, void* o, float* h_out, hipStream_t s) {
    FlushArgs args{st.sq, st.row_scale, st.col_scale, st.comp_idx, st.comp_val,
                   st.buf_k, st.buf_m, st.buf_g, h_out, pos_dev, d.W, d.C, pos + 1, d.smooth, d.H,
                   q, k, v, alpha, beta, o, 0, 0, 0};
    return flush_any<true>(d, args, s);
}

hipError_t launch_quantize(const lq_dims& d, const float* h, const lq_state& st, hipStream_t s) {
    QuantArgs args{h, st.sq, st.row_scale, st.col_scale, st.comp_idx, st.comp_val, d.C, d.smooth};
    const dim3 grid((unsigned)d.B * (unsigned)d.H);
    switch (d.dk) {
        case 16: return launch_kernel(LQ_KERNEL_QUANTIZE, quantize_kernel<16, 16>, grid, dim3(FS<16, 16>::NT), s, args);
        case 64: return launch_kernel(LQ_KERNEL_QUANTIZE, quantize_kernel<64, 64>, grid, dim3(FS<64, 64>::NT), s, args);
        default: return launch_kernel(LQ_KERNEL_QUANTIZE, quantize_kernel<128, 128>, grid, dim3(FS<128, 128>::NT), s, args);
    }
}

hipError_t launch_dequantize(const lq_dims& d, const lq_state& st, float* h_out, hipStream_t s) {
    DequantArgs args{st.sq, st.row_scale, st.col_scale, st.comp_idx, st.comp_val, h_out, d.C};
    const dim3 grid((unsigned)d.B * (unsigned)d.H);
    switch (d.dk) {
        case 16: return launch_kernel(LQ_KERNEL_DEQUANTIZE, dequantize_kernel<16, 16>, grid, dim3(256), s, args);
        case 64: return launch_kernel(LQ_KERNEL_DEQUANTIZE, dequantize_kernel<64, 64>, grid, dim3(256), s, args);
        default: return launch_kernel(LQ_KERNEL_DEQUANTIZE, dequantize_kernel<128, 128>, grid, dim3(256), s, args);
    }
}

}  // namespace lq

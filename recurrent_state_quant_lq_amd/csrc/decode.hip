// decode.hip -- one decode token over the int8 state (gfx950).
//
// LeapQuant abstract (HFEPX paper page, "Abstract"): while a window is open
// the 8-bit state does not change, and each token's output combines it with
// the window's updates kept in full precision; compensator tokens go through
// the same update as ordinary tokens.  News article ("A linear-attention
// method cuts state ...", paragraph 3): every update is applied, only the
// rounding is deferred.
//
// Buffer form.  With the window-base state Hb (fixed for the window) and the
// window-local log-decays g, slot i of the buffer holds k_i, g_i and
//     m_i = beta_i (v_i - Hb^T (e^{g_i} o k_i) - sum_{l<i} rr_{i,l} m_l),
//     rr_{i,l} = <k_i, E_{i,l} o k_l>,  E_{i,l} = exp(g_i - g_l).
// (m_i = u_i - Hb^T y_i for the WY factors y_i, u_i of the window's delta-rule
// updates: projecting y_i through the fixed Hb once, when the slot is made,
// leaves one dv-vector per slot instead of two.)  The output of slot n is
//     o = Hb^T (e^{g_n} o q) + sum_{i<=n} a_i m_i,   a_i = <q, E_{n,i} o k_i>,
// exactly H_n^T q for the state reached from Hb by the window's n+1 steps,
// and Hb^T x = s o (sq^T (r o x)) + sum_c x[idx_c] cv_c.
//
// One workgroup per (b, h): dk channel lanes and dv value lanes (256 at
// d = 128) with at most 64 VGPRs, so 8 workgroups share a CU and one dispatch
// covers B*H = 2048 heads on 256 CUs.  Loads, all issued up front:
//   * per-head vectors (q, k, v, row and column scales, per-key decay,
//     compensator rows) and the buffered keys go straight to LDS
//     (global_load_lds_dwordx4, no registers);
//   * each value lane loads its column of the buffered m_i;
//   * the int8 state goes to VGPRs last, as the A operands of int8 MFMAs; it
//     is stored in that operand order (sq_off), so each of a wave's state
//     loads reads 1 KB of contiguous bytes.  The first barrier waits for
//     every load: LDS copies and register loads do not complete in order with
//     each other, so no load can be left in flight past the first LDS read.
// Then:
//   A. channel lanes: the int8 digits of r o e^g o q and r o e^g o k per
//      64-channel block; all lanes, in slot groups: rr_i = <k, E_i o k_i>,
//      a_i = <q, E_i o k_i>; slot n's key and log-decay are stored; the
//      last CMAX lanes: the compensator coefficients e^{g_n}[idx_c] q[idx_c]
//      and e^{g_n}[idx_c] k[idx_c]
//   B. int8 MFMA: sq^T x digits for both vectors at once (wave w owns its
//      column tiles); value lanes: sum_i rr_i m_i and sum_i a_i m_i
//   C. value lanes: Hb^T q~, Hb^T k~ with the compensator rows, m_n and o.
#include "lq_internal.h"

#include <utility>

namespace lq {
namespace {

struct DecodeArgs {
    const int8_t* sq;
    const float* r;
    const float* s;
    const int32_t* idx;
    const float* cv;
    float* bk;
    float* bm;
    float* bg;
    const void* q;            // q, k, v, o: fp32 or bf16 (the kernel's TI)
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    void* o;
    const int32_t* pos_dev;   // per batch row (ragged positions), or null: pos for every row
    int W;
    int C;
    int H;
    int pos;
};

constexpr int CMAX = 8;

template <int DK, int DV, int WM, bool KDA>
struct Dec {
    static_assert(DK == DV, "square heads");
    static constexpr int NT = (DK + DV) < 64 ? 64 : DK + DV;
    static constexpr int NW = NT / 64;
    static constexpr int GD = KDA ? DK : 1;
    // int8 MFMA GEMV: 16-column tiles, 64-channel K steps
    static constexpr int NTILE = DV / 16;
    static constexpr int TPW = (NTILE + NW - 1) / NW;    // tiles per wave
    static constexpr int KS = (DK + 63) / 64;            // K steps (= channel waves)
    // slot groups: TPS lanes per slot, CH channels per lane, SPR slots per
    // round, ROUNDS rounds
    static constexpr int TPS0 = NT / WM > 32 ? NT / WM : 32;
    static constexpr int TPS = TPS0 < DK ? TPS0 : DK;
    static constexpr int CH = DK / TPS;
    static constexpr int SPR = NT / TPS;
    static constexpr int ROUNDS = (WM + SPR - 1) / SPR;
    static_assert(TPS <= 64 && CH >= 1 && DK % TPS == 0 && NT % TPS == 0, "slot tiling");
    // LDS vector region: DK-float segments
    //   q k v r s [alpha gprev] cv_0..cv_{CMAX-1} k_0..k_{WM-2}
    static constexpr int SQ = 0, SK = 1, SV = 2, SR = 3, SS = 4, SA = 5, SG = 6;
    static constexpr int SCV = KDA ? 7 : 5;
    static constexpr int SKB = SCV + CMAX;
    static constexpr int NSEG = SKB + (WM > 1 ? WM - 1 : 1);
    static constexpr int SEGL = DK / 4;                  // lanes (16-byte chunks) per segment
    static_assert(DK % 4 == 0 && 64 % SEGL == 0 && SCV * SEGL <= NT, "segments");
    // waves per SIMD the register budget is sized for (8: all 8 workgroups of a
    // CU resident; per-key decay needs more registers for its decay rows; with
    // 32 slots, 6 for scalar decay, whose 77 registers fit there without spills)
    static constexpr int WPE = WM <= 16 ? (KDA ? 6 : 8) : (KDA ? 4 : 6);
};

template <int DK, int DV, int WM, bool KDA, int NB, typename TI>
__global__ __launch_bounds__((Dec<DK, DV, WM, KDA>::NT))
__attribute__((amdgpu_waves_per_eu(Dec<DK, DV, WM, KDA>::WPE, Dec<DK, DV, WM, KDA>::WPE)))
void decode_kernel(DecodeArgs a) {
    using D = Dec<DK, DV, WM, KDA>;
    constexpr int NT = D::NT, GD = D::GD, TPW = D::TPW, KS = D::KS, NTILE = D::NTILE;
    constexpr int TPS = D::TPS, CH = D::CH, SPR = D::SPR, ROUNDS = D::ROUNDS;
    constexpr int SEGL = D::SEGL;

    __shared__ __align__(16) float s_vec[D::NSEG * DK];
    __shared__ __align__(16) float s_rr[WM];
    __shared__ __align__(16) float s_a[WM];
    __shared__ __align__(16) float s_cqk[2][CMAX];            // e^{g_n}[idx_c] q[idx_c], ... k[idx_c]
    __shared__ __align__(16) int8_t s_dig[6][KS * 64];       // digits of q~'' (0..2), k~'' (3..5)
    __shared__ __align__(16) float s_msc[2];                 // digit scales of q~'', k~''

    __shared__ __align__(16) float s_gem[2][DV];             // sq^T q~'', sq^T k~''
    // dwords 0..7: compensator rows; 8: beta; 9: alpha (scalar decay); 10: g_{n-1} (scalar decay)
    __shared__ __align__(16) int s_misc[16];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const size_t head = blockIdx.x;
    const int W = a.W, C = a.C;
    int n = NB;
    if constexpr (NB < 0) {
        n = a.pos_dev ? a.pos_dev[head / (unsigned)a.H] : a.pos;
        if (n < 0 || n >= W) return;              // a row outside its window: untouched
    }

    const float* __restrict__ bkr = a.bk + head * (size_t)W * DK;
    const float* __restrict__ bmr = a.bm + head * (size_t)W * DV;
    const float* __restrict__ bgr = a.bg + head * (size_t)W * GD;

    // ---- per-head vectors, compensator rows and buffered keys -> LDS ----------------------
    // Three contiguous copies, 16-byte chunk c of a region landing at region + 4c floats
    // (lane l of a wave writes its wave's base + 16*l bytes).
    {
        // q k v r s [alpha gprev]: segment sg = t / SEGL, one chunk per lane (bf16 q, k,
        // v fill the first half of their segments)
        constexpr int NVS = D::SCV;
        const int sg = t / SEGL, off = 4 * (t % SEGL);
        const bool tin = sizeof(TI) == 4 || 2 * off < DK;   // this lane's chunk lies in the token row
        const float* src = nullptr;
        switch (sg) {
            case D::SQ: if (tin) src = reinterpret_cast<const float*>(static_cast<const TI*>(a.q) + head * DK); break;
            case D::SK: if (tin) src = reinterpret_cast<const float*>(static_cast<const TI*>(a.k) + head * DK); break;
            case D::SV: if (tin) src = reinterpret_cast<const float*>(static_cast<const TI*>(a.v) + head * DV); break;
            case D::SR: src = a.r + head * DK; break;
            case D::SS: src = a.s + head * DV; break;
            default:
                if constexpr (KDA) {
                    if (sg == D::SA) src = a.alpha + head * DK;
                    else if (sg == D::SG && n > 0) src = bgr + (size_t)(n - 1) * DK;
                }
        }
        if (sg < NVS && src) lds_dma16(src + off, s_vec + 4 * 64 * w);
        // compensator rows: C*DV contiguous floats
        const int ccv = C * DV / 4;
        if (t < ccv) lds_dma16(a.cv + head * (size_t)C * DV + 4 * t, s_vec + D::SCV * DK + 4 * 64 * w);
        // buffered keys k_0 .. k_{n-1}: n*DK contiguous floats
        const int ckb = n * DK / 4;
        for (int base = 0; base < ckb; base += NT) {
            const int c = base + t;
            if (c < ckb) lds_dma16(bkr + 4 * c, s_vec + D::SKB * DK + 4 * (base + 64 * w));
        }
        if (w == 0) {
            const void* src4 = nullptr;
            if (lane < C) src4 = a.idx + head * C + lane;
            else if (lane == 8) src4 = a.beta + head;
            else if (!KDA && lane == 9) src4 = a.alpha + head;
            else if (!KDA && lane == 10 && n > 0) src4 = bgr + (n - 1);
            if (src4) lds_dma4(src4, s_misc);
        }
    }

    // ---- buffer rows -> VGPRs -------------------------------------------------------------
    const int slot0 = t / TPS;
    const int c0 = (t % TPS) * CH;
    // decay rows of the slot groups.  The loads are unconditional: a slot >= n (its
    // value is never used) reads row n - 1 again, a row this workgroup reads anyway,
    // so the rows past it cost no memory traffic
    float gs[ROUNDS][KDA ? CH : 1];
    float gslot[ROUNDS];
    const int glast = max(n - 1, 0);
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
        const int slot = min(slot0 + rd * SPR, glast);
        if constexpr (KDA) load_floats<CH>(bgr + (size_t)slot * DK + c0, gs[rd]);
        else gslot[rd] = bgr[slot];
    }
    const bool is_ch = t < DK;
    const bool is_val = t >= DK && t < DK + DV;
    const int j = t - DK;
    float mcol[WM > 1 ? WM - 1 : 1];              // value lane j: m_i[j], i < n
    if (is_val) {
#pragma unroll
        for (int i = 0; i < WM - 1; ++i)
            if (i < n) mcol[i] = ld_nt(bmr + (size_t)i * DV + j);
    }

    // ---- int8 state -> VGPRs (MFMA A operands), issued last ---------------------------------
    // lane l of wave w: column j = tile*16 + l%16, channels ks*64 + 16*(l/16) .. +15.
    // Every tile and K step is real when the shape divides evenly (the loads are then
    // unconditional).
    constexpr bool FULL = (NTILE % D::NW == 0) && (DK % 64 == 0);
    __builtin_amdgcn_sched_barrier(0);
    v4i sqa[TPW][KS];
    {
        const int8_t* sq = a.sq + head * (DK * DV);
#pragma unroll
        for (int tw = 0; tw < TPW; ++tw)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int tile = w * TPW + tw;
                const int i0 = ks * 64 + 16 * (lane / 16);
                if (FULL || (tile < NTILE && i0 < DK))
                    sqa[tw][ks] = ld_nt(reinterpret_cast<const v4i*>(sq + sq_off<DK>(i0, tile * 16 + lane % 16)));
                else
                    sqa[tw][ks] = v4i{0, 0, 0, 0};
            }
    }
    __builtin_amdgcn_sched_barrier(0);
    all_loads_barrier();

    const float beta = __int_as_float(s_misc[8]);
    float gn_s = 0.0f;
    if constexpr (!KDA) gn_s = (n > 0 ? __int_as_float(s_misc[10]) : 0.0f) + __logf(__int_as_float(s_misc[9]));

    // ---- A. digits of r o e^g o q and r o e^g o k; slot n's key and decay; dot products ----
    float xq = 0.0f, xk = 0.0f;                   // r o e^g o q, r o e^g o k (channel lanes)
    if (is_ch) {
        const float qc = seg_ld<TI>(s_vec + D::SQ * DK, t), kc = seg_ld<TI>(s_vec + D::SK * DK, t);
        const float rc = s_vec[D::SR * DK + t];
        float gn;
        if constexpr (KDA) gn = (n > 0 ? s_vec[D::SG * DK + t] : 0.0f) + __logf(s_vec[D::SA * DK + t]);
        else gn = gn_s;
        const float en = __expf(gn);
        xq = rc * (en * qc);
        xk = rc * (en * kc);
        st_nt(a.bk + head * (size_t)W * DK + (size_t)n * DK + t, kc);
        if constexpr (KDA) st_nt(a.bg + head * (size_t)W * DK + (size_t)n * DK + t, gn);
        else if (t == 0) st_nt(a.bg + head * (size_t)W + n, gn);
    }
    // the compensator rows' coefficients, by the last CMAX lanes (value lanes): the
    // decayed query and key entries at the compensator rows (the same expression the
    // channel lane of row idx_c evaluates)
    if (t >= NT - CMAX && t - (NT - CMAX) < C) {
        const int c = t - (NT - CMAX);
        const int ic = s_misc[c] & (DK - 1);
        float e;
        if constexpr (KDA) e = __expf((n > 0 ? s_vec[D::SG * DK + ic] : 0.0f) + __logf(s_vec[D::SA * DK + ic]));
        else e = __expf(gn_s);
        s_cqk[0][c] = e * seg_ld<TI>(s_vec + D::SQ * DK, ic);
        s_cqk[1][c] = e * seg_ld<TI>(s_vec + D::SK * DK, ic);
    }
    if (w < KS) {
        // wave w's 64 lanes are one 64-channel block (lanes past dk hold zeros):
        // one scale M = max |x| over all dk channels, three int8 digits per
        // channel.  With two blocks each lane also forms the entry of channel
        // t ^ 64 from LDS, so both waves find the same maximum without a barrier,
        // and the int8 products of the two K steps can add up in int32.
        uint32_t aq = __float_as_uint(xq) & 0x7fffffffu, ak = __float_as_uint(xk) & 0x7fffffffu;
        if constexpr (KS == 2) {
            const int p = t ^ 64;
            float ep;
            if constexpr (KDA) ep = __expf((n > 0 ? s_vec[D::SG * DK + p] : 0.0f) + __logf(s_vec[D::SA * DK + p]));
            else ep = __expf(gn_s);
            const float rp = s_vec[D::SR * DK + p];
            aq = umax(aq, __float_as_uint(rp * (ep * seg_ld<TI>(s_vec + D::SQ * DK, p))) & 0x7fffffffu);
            ak = umax(ak, __float_as_uint(rp * (ep * seg_ld<TI>(s_vec + D::SK * DK, p))) & 0x7fffffffu);
        }
        const float mq = __uint_as_float(wave_umax(aq));
        const float mk = __uint_as_float(wave_umax(ak));
        uint32_t d0, d1, d2;
        digits3_words(xq, mq > 0.0f ? 127.0f * __builtin_amdgcn_rcpf(mq) : 0.0f, d0, d1, d2);
        s_dig[0][t] = (int8_t)d0;
        s_dig[1][t] = (int8_t)d1;
        s_dig[2][t] = (int8_t)d2;
        digits3_words(xk, mk > 0.0f ? 127.0f * __builtin_amdgcn_rcpf(mk) : 0.0f, d0, d1, d2);
        s_dig[3][t] = (int8_t)d0;
        s_dig[4][t] = (int8_t)d1;
        s_dig[5][t] = (int8_t)d2;
        if (w == 0 && lane == 0) {
            s_msc[0] = mq * (1.0f / 127.0f);
            s_msc[1] = mk * (1.0f / 127.0f);
        }
    }
    {
        float kq[CH], kk[CH];
        seg_ld_n<CH, TI>(s_vec + D::SQ * DK, c0, kq);
        seg_ld_n<CH, TI>(s_vec + D::SK * DK, c0, kk);
        // per-key decay: g_n of this lane's channels, once for all its slots
        float gnc[KDA ? CH : 1];
        if constexpr (KDA) {
            float al[CH], gp[CH];
            load_floats<CH>(s_vec + D::SA * DK + c0, al);
            if (n > 0) load_floats<CH>(s_vec + D::SG * DK + c0, gp);
#pragma unroll
            for (int c = 0; c < CH; ++c) gnc[c] = (n > 0 ? gp[c] : 0.0f) + __logf(al[c]);
        }
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) {
            const int slot = slot0 + rd * SPR;
            if (rd * SPR > n) break;                      // uniform: no slot <= n left
            float rr = 0.0f, aa = 0.0f;
            if (slot < n) {
                float ks[CH];
                load_floats<CH>(s_vec + (D::SKB + slot) * DK + c0, ks);
                if constexpr (KDA) {
#pragma unroll
                    for (int c = 0; c < CH; ++c) {
                        const float x = ks[c] * __expf(gnc[c] - gs[rd][c]);
                        rr += kk[c] * x;
                        aa += kq[c] * x;
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < CH; ++c) {
                        rr += kk[c] * ks[c];
                        aa += kq[c] * ks[c];
                    }
                    const float e = __expf(gn_s - gslot[rd]);
                    rr *= e;
                    aa *= e;
                }
            } else if (slot == n) {
#pragma unroll
                for (int c = 0; c < CH; ++c) aa += kq[c] * kk[c];
            }
            rr = group_sum<TPS>(rr);
            aa = group_sum<TPS>(aa);
            if ((t % TPS) == 0 && slot <= n) {
                s_rr[slot] = rr;
                s_a[slot] = aa;
            }
        }
    }
    lds_barrier();

    // ---- B. int8 MFMA: both digit sets times sq for this wave's column tiles; buffer sums ------
    // A = the digits (rows 0..2: q~'', rows 4..6: k~'', other rows zero), B = the state
    // bytes (a lane's 16 bytes are 16 channels of value column l % 16: the same bytes it
    // would give as an A operand, so the loaded registers serve as they are).  Lane l
    // then holds digit rows 4 (l/16) .. +3 of value column l % 16: lane group 0 the
    // three digit sums of q~'', lane group 1 those of k~''.
    {
        const int li = lane % 16, lg = lane / 16;
        const int drow = li < 3 ? li : (li >= 4 && li < 7) ? li - 1 : -1;
        v4i aop[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            aop[ks] = drow >= 0 ? *reinterpret_cast<const v4i*>(&s_dig[drow][ks * 64 + 16 * lg])
                                : v4i{0, 0, 0, 0};
        const float sc = lg < 2 ? s_msc[lg] : 0.0f;
#pragma unroll
        for (int tw = 0; tw < TPW; ++tw) {
            const int tile = w * TPW + tw;
            if (tile >= NTILE) break;
            // |digit| <= 127 and |byte| <= 127 over at most 128 channels: the
            // int32 sums stay below 2^21
            v4i dv4 = v4i{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                dv4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[ks], sqa[tw][ks], dv4, 0, 0, 0);
            const float x = __builtin_fmaf((float)dv4[2], kDigitW2, __builtin_fmaf((float)dv4[1], kDigitW1,
                                                                                    (float)dv4[0]));
            if (lg < 2) s_gem[lg][tile * 16 + li] = x * sc;
        }
    }
    float sr = 0.0f, sa = 0.0f;
    if (is_val) {
#pragma unroll
        for (int i = 0; i < WM - 1; ++i)
            if (i < n) {
                sr += s_rr[i] * mcol[i];
                sa += s_a[i] * mcol[i];
            }
    }
    lds_barrier();

    // ---- C. m_n and the output ------------------------------------------------------------------
    if (is_val) {
        const float sj = s_vec[D::SS * DK + j];
        float hq = sj * s_gem[0][j], hk = sj * s_gem[1][j];
#pragma unroll
        for (int c = 0; c < CMAX; ++c)
            if (c < C) {
                const float cvj = s_vec[(D::SCV + c) * DK + j];
                hq += s_cqk[0][c] * cvj;
                hk += s_cqk[1][c] * cvj;
            }
        const float mn = beta * (seg_ld<TI>(s_vec + D::SV * DK, j) - hk - sr);
        st_nt(a.bm + head * (size_t)W * DV + (size_t)n * DV + j, mn);
        tok_st<TI>(a.o, head * DV + j, hq + sa + s_a[n] * mn);
    }
}

// dk = dv = 128: the same step with the waves split by role, so that the token
// work does not wait for the state bytes.  Waves 0-1 (token waves, lane t =
// channel t = value column t) copy the per-head vectors and compensator rows to
// LDS and load the buffered m columns; waves 2-3 (state waves) copy the buffered
// keys to LDS, then, after the first barrier, load the int8 state, wave w the
// column tiles 4 (w - 2) .. + 3.  The first barrier thus waits for the head's
// token data only (each wave's counter of outstanding loads covers only its own
// loads), and the state waves' later waits leave their state loads in flight.  Phase A (digits, slot dot products,
// compensator coefficients) and the buffer sums then run while the state
// streams in; the token waves hand the buffer sums over in LDS and end.  After
// the state lands, only the state waves' MFMAs, two row swaps that bring each
// column's query and key sums to one lane, and the output step remain, with no
// barrier or LDS round trip left on that path.  Each role is its own branch
// (the wave index is uniform), so the register allocator never holds the state
// registers and the m columns at once.
template <int WM, bool KDA, int NB, typename TI>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(Dec<128, 128, WM, KDA>::WPE, Dec<128, 128, WM, KDA>::WPE)))
void decode_split_kernel(DecodeArgs a) {
    constexpr int DK = 128, DV = 128;
    using D = Dec<DK, DV, WM, KDA>;
    constexpr int TPS = D::TPS, CH = D::CH, SPR = D::SPR, ROUNDS = D::ROUNDS, SEGL = D::SEGL;
    constexpr int GD = D::GD;
    constexpr int TPSW = 4;                  // column tiles per state wave
    static_assert(D::NT == 256 && D::KS == 2 && D::NTILE == 2 * TPSW, "two token and two state waves");

    __shared__ __align__(16) float s_vec[D::NSEG * DK];
    __shared__ __align__(16) float s_rr[WM];
    __shared__ __align__(16) float s_a[WM];
    __shared__ __align__(16) float s_cqk[2][CMAX];            // e^{g_n}[idx_c] q[idx_c], ... k[idx_c]
    __shared__ __align__(16) int8_t s_dig[6][128];           // digits of q~'' (0..2), k~'' (3..5)
    __shared__ __align__(16) float s_msc[2];                 // digit scales of q~'', k~''
    __shared__ __align__(16) float s_sum[2][DV];             // sum_i rr_i m_i, sum_i a_i m_i per value column
    // dwords 0..7: compensator rows; 8: beta; 9: alpha (scalar decay); 10: g_{n-1} (scalar decay)
    __shared__ __align__(16) int s_misc[16];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const size_t head = blockIdx.x;
    const int W = a.W, C = a.C;
    int n = NB;
    if constexpr (NB < 0) {
        n = a.pos_dev ? a.pos_dev[head / (unsigned)a.H] : a.pos;
        if (n < 0 || n >= W) return;              // a row outside its window: untouched
    }
    const float* __restrict__ bkr = a.bk + head * (size_t)W * DK;
    const float* __restrict__ bmr = a.bm + head * (size_t)W * DV;
    const float* __restrict__ bgr = a.bg + head * (size_t)W * GD;

    // slot groups of the dot products (all 256 lanes take part)
    const int slot0 = t / TPS;
    const int c0 = (t % TPS) * CH;

    // Dot products rr_i = <k, E_i o k_i>, a_i = <q, E_i o k_i> of this lane's slot
    // group, a_n = <q, k>; results to s_rr, s_a.
    auto dot_products = [&](const float (&gs)[ROUNDS][KDA ? CH : 1], const float (&gslot)[ROUNDS], float gn_s) {
        float kq[CH], kk[CH];
        seg_ld_n<CH, TI>(s_vec + D::SQ * DK, c0, kq);
        seg_ld_n<CH, TI>(s_vec + D::SK * DK, c0, kk);
        float gnc[KDA ? CH : 1];
        if constexpr (KDA) {
            float al[CH], gp[CH];
            load_floats<CH>(s_vec + D::SA * DK + c0, al);
            if (n > 0) load_floats<CH>(s_vec + D::SG * DK + c0, gp);
#pragma unroll
            for (int c = 0; c < CH; ++c) gnc[c] = (n > 0 ? gp[c] : 0.0f) + __logf(al[c]);
        }
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) {
            const int slot = slot0 + rd * SPR;
            if (rd * SPR > n) break;                      // uniform: no slot <= n left
            float rr = 0.0f, aa = 0.0f;
            if (slot < n) {
                float ks[CH];
                load_floats<CH>(s_vec + (D::SKB + slot) * DK + c0, ks);
                if constexpr (KDA) {
#pragma unroll
                    for (int c = 0; c < CH; ++c) {
                        const float x = ks[c] * __expf(gnc[c] - gs[rd][c]);
                        rr += kk[c] * x;
                        aa += kq[c] * x;
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < CH; ++c) {
                        rr += kk[c] * ks[c];
                        aa += kq[c] * ks[c];
                    }
                    const float e = __expf(gn_s - gslot[rd]);
                    rr *= e;
                    aa *= e;
                }
            } else if (slot == n) {
#pragma unroll
                for (int c = 0; c < CH; ++c) aa += kq[c] * kk[c];
            }
            rr = group_sum<TPS>(rr);
            aa = group_sum<TPS>(aa);
            if ((t % TPS) == 0 && slot <= n) {
                s_rr[slot] = rr;
                s_a[slot] = aa;
            }
        }
    };
    // decay rows of this lane's slot groups; a slot >= n (its value is never used)
    // reads row n - 1 again, so the rows past it cost no memory traffic
    auto load_decays = [&](float (&gs)[ROUNDS][KDA ? CH : 1], float (&gslot)[ROUNDS]) {
        const int glast = max(n - 1, 0);
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) {
            const int slot = min(slot0 + rd * SPR, glast);
            if constexpr (KDA) load_floats<CH>(bgr + (size_t)slot * DK + c0, gs[rd]);
            else gslot[rd] = bgr[slot];
        }
    };

    if (w < 2) {
        // ================= token waves: lane t is channel t and value column t =================
        {
            // q k v r s [alpha gprev]: chunk c of segment c / SEGL (bf16 q, k, v fill the
            // first half of their segments)
            constexpr int NVS = D::SCV;
#pragma unroll
            for (int base = 0; base < NVS * SEGL; base += 128) {
                const int c = base + t;
                const int sg = c / SEGL, off = 4 * (c % SEGL);
                const bool tin = sizeof(TI) == 4 || 2 * off < DK;
                const float* src = nullptr;
                switch (sg) {
                    case D::SQ: if (tin) src = reinterpret_cast<const float*>(static_cast<const TI*>(a.q) + head * DK); break;
                    case D::SK: if (tin) src = reinterpret_cast<const float*>(static_cast<const TI*>(a.k) + head * DK); break;
                    case D::SV: if (tin) src = reinterpret_cast<const float*>(static_cast<const TI*>(a.v) + head * DV); break;
                    case D::SR: src = a.r + head * DK; break;
                    case D::SS: src = a.s + head * DV; break;
                    default:
                        if constexpr (KDA) {
                            if (sg == D::SA) src = a.alpha + head * DK;
                            else if (sg == D::SG && n > 0) src = bgr + (size_t)(n - 1) * DK;
                        }
                }
                if (c < NVS * SEGL && src) lds_dma16(src + off, s_vec + 4 * (base + 64 * w));
            }
            // compensator rows: C*DV contiguous floats
            const int ccv = C * DV / 4;
            for (int base = 0; base < ccv; base += 128) {
                const int c = base + t;
                if (c < ccv) lds_dma16(a.cv + head * (size_t)C * DV + 4 * c, s_vec + D::SCV * DK + 4 * (base + 64 * w));
            }
            if (w == 0) {
                const void* src4 = nullptr;
                if (lane < C) src4 = a.idx + head * C + lane;
                else if (lane == 8) src4 = a.beta + head;
                else if (!KDA && lane == 9) src4 = a.alpha + head;
                else if (!KDA && lane == 10 && n > 0) src4 = bgr + (n - 1);
                if (src4) lds_dma4(src4, s_misc);
            }
        }
        float gs[ROUNDS][KDA ? CH : 1], gslot[ROUNDS];
        load_decays(gs, gslot);
        float mcol[WM > 1 ? WM - 1 : 1];          // m_i[t], i < n
#pragma unroll
        for (int i = 0; i < WM - 1; ++i)
            if (i < n) mcol[i] = ld_nt(bmr + (size_t)i * DV + t);
        all_loads_barrier();                                                        // (1)

        float gn_s = 0.0f;
        if constexpr (!KDA) gn_s = (n > 0 ? __int_as_float(s_misc[10]) : 0.0f) + __logf(__int_as_float(s_misc[9]));
        // ---- A. digits of r o e^g o q and r o e^g o k; slot n's key and decay ------------------
        {
            const float qc = seg_ld<TI>(s_vec + D::SQ * DK, t), kc = seg_ld<TI>(s_vec + D::SK * DK, t);
            const float rc = s_vec[D::SR * DK + t];
            float gn;
            if constexpr (KDA) gn = (n > 0 ? s_vec[D::SG * DK + t] : 0.0f) + __logf(s_vec[D::SA * DK + t]);
            else gn = gn_s;
            const float en = __expf(gn);
            const float xq = rc * (en * qc), xk = rc * (en * kc);
            st_nt(a.bk + head * (size_t)W * DK + (size_t)n * DK + t, kc);
            if constexpr (KDA) st_nt(a.bg + head * (size_t)W * DK + (size_t)n * DK + t, gn);
            else if (t == 0) st_nt(a.bg + head * (size_t)W + n, gn);
            // one scale M = max |x| over all 128 channels (each lane also forms the
            // entry of channel t ^ 64 from LDS), three int8 digits per channel
            uint32_t aq = __float_as_uint(xq) & 0x7fffffffu, ak = __float_as_uint(xk) & 0x7fffffffu;
            {
                const int p = t ^ 64;
                float ep;
                if constexpr (KDA) ep = __expf((n > 0 ? s_vec[D::SG * DK + p] : 0.0f) + __logf(s_vec[D::SA * DK + p]));
                else ep = en;
                const float rp = s_vec[D::SR * DK + p];
                aq = umax(aq, __float_as_uint(rp * (ep * seg_ld<TI>(s_vec + D::SQ * DK, p))) & 0x7fffffffu);
                ak = umax(ak, __float_as_uint(rp * (ep * seg_ld<TI>(s_vec + D::SK * DK, p))) & 0x7fffffffu);
            }
            const float mq = __uint_as_float(wave_umax(aq));
            const float mk = __uint_as_float(wave_umax(ak));
            uint32_t d0, d1, d2;
            digits3_words(xq, mq > 0.0f ? 127.0f * __builtin_amdgcn_rcpf(mq) : 0.0f, d0, d1, d2);
            s_dig[0][t] = (int8_t)d0;
            s_dig[1][t] = (int8_t)d1;
            s_dig[2][t] = (int8_t)d2;
            digits3_words(xk, mk > 0.0f ? 127.0f * __builtin_amdgcn_rcpf(mk) : 0.0f, d0, d1, d2);
            s_dig[3][t] = (int8_t)d0;
            s_dig[4][t] = (int8_t)d1;
            s_dig[5][t] = (int8_t)d2;
            if (w == 0 && lane == 0) {
                s_msc[0] = mq * (1.0f / 127.0f);
                s_msc[1] = mk * (1.0f / 127.0f);
            }
        }
        dot_products(gs, gslot, gn_s);
        lds_barrier();                                                              // (2)
        // ---- buffer sums (value column t), handed to the state waves ---------------------------
        float sr = 0.0f, sa = 0.0f;
#pragma unroll
        for (int i = 0; i < WM - 1; ++i)
            if (i < n) {
                sr += s_rr[i] * mcol[i];
                sa += s_a[i] * mcol[i];
            }
        s_sum[0][t] = sr;
        s_sum[1][t] = sa;
        lds_barrier();                                                              // (3)
    } else {
        // ================= state waves ============================================================
        float gs[ROUNDS][KDA ? CH : 1], gslot[ROUNDS];
        {
            // buffered keys k_0 .. k_{n-1}: n*DK contiguous floats.  Copied by these
            // waves, the token waves' share of the head's token loads is issued sooner
            // and the keys stream beside it; this wave waits for its copies at the
            // first barrier, before any wave reads them.
            const int ckb = n * DK / 4;
            const int ts = t - 128;
            for (int base = 0; base < ckb; base += 128) {
                const int c = base + ts;
                if (c < ckb) lds_dma16(bkr + 4 * c, s_vec + D::SKB * DK + 4 * (base + 64 * (w - 2)));
            }
        }
        load_decays(gs, gslot);
        all_loads_barrier();                                                        // (1)
        // The int8 state, requested once this head's token data has landed: every
        // workgroup's token data then reaches the queue ahead of the state streams, so
        // the token work of even the last heads is done before their state arrives.
        // Tile T of this wave, K step ks; lane l: value column T*16 + l%16, channels
        // ks*64 + 16*(l/16) .. +15 (1 KB contiguous per load and wave).
        __builtin_amdgcn_sched_barrier(0);
        v4i sqa[TPSW][2];
        {
            const int8_t* sq = a.sq + head * (DK * DV);
#pragma unroll
            for (int tw = 0; tw < TPSW; ++tw)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    sqa[tw][ks] = ld_nt(reinterpret_cast<const v4i*>(
                        sq + sq_off<DK>(ks * 64 + 16 * (lane / 16), ((w - 2) * TPSW + tw) * 16 + lane % 16)));
        }
        __builtin_amdgcn_sched_barrier(0);
        float gn_s = 0.0f;
        if constexpr (!KDA) gn_s = (n > 0 ? __int_as_float(s_misc[10]) : 0.0f) + __logf(__int_as_float(s_misc[9]));
        // the compensator rows' coefficients, by the last CMAX lanes: the decayed query
        // and key entries at the compensator rows (the expression the channel lane of
        // row idx_c evaluates)
        if (t >= D::NT - CMAX && t - (D::NT - CMAX) < C) {
            const int c = t - (D::NT - CMAX);
            const int ic = s_misc[c] & (DK - 1);
            float e;
            if constexpr (KDA) e = __expf((n > 0 ? s_vec[D::SG * DK + ic] : 0.0f) + __logf(s_vec[D::SA * DK + ic]));
            else e = __expf(gn_s);
            s_cqk[0][c] = e * seg_ld<TI>(s_vec + D::SQ * DK, ic);
            s_cqk[1][c] = e * seg_ld<TI>(s_vec + D::SK * DK, ic);
        }
        dot_products(gs, gslot, gn_s);
        lds_barrier();                                                              // (2)
        // ---- B. int8 MFMA: both digit sets times this wave's state tiles --------------------
        // A = the digits (rows 0..2: q~'', rows 4..6: k~'', other rows zero), B = the state
        // bytes as loaded; lane group 0 ends with the digit sums of q~'' for value column
        // l % 16, lane group 1 those of k~''.
        const int li = lane % 16, lg = lane / 16;
        v4i aop[2];
        {
            const int drow = li < 3 ? li : (li >= 4 && li < 7) ? li - 1 : -1;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                aop[ks] = drow >= 0 ? *reinterpret_cast<const v4i*>(&s_dig[drow][ks * 64 + 16 * lg])
                                    : v4i{0, 0, 0, 0};
        }
        const float sc = lg < 2 ? s_msc[lg] : 0.0f;
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();                                                              // (3)
        __builtin_amdgcn_sched_barrier(0);
        // ---- C. m_n and the output, value column j of lane group lg = this wave's tile lg ----
        // (everything but the GEMV is read while the state is still streaming in)
        const int j = ((w - 2) * TPSW + lg) * 16 + li;
        const float sj = s_vec[D::SS * DK + j];
        const float vj = seg_ld<TI>(s_vec + D::SV * DK, j);
        const float sr = s_sum[0][j], sa = s_sum[1][j];
        const float an = s_a[n];
        const float beta = __int_as_float(s_misc[8]);
        // the compensator rows' share of Hb^T q~ and Hb^T k~ for column j
        float cq = 0.0f, ck = 0.0f;
#pragma unroll
        for (int c = 0; c < CMAX; ++c)
            if (c < C) {
                const float cvj = s_vec[(D::SCV + c) * DK + j];
                cq += s_cqk[0][c] * cvj;
                ck += s_cqk[1][c] * cvj;
            }
        // the MFMAs stay below the barrier and the LDS reads above them: only the
        // MFMAs and what follows wait for the state
        __builtin_amdgcn_sched_barrier(0);
        float x[TPSW];
#pragma unroll
        for (int tw = 0; tw < TPSW; ++tw) {
            // |digit| <= 127 and |byte| <= 127 over 128 channels: int32 sums below 2^21
            v4i dv4 = v4i{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                dv4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[ks], sqa[tw][ks], dv4, 0, 0, 0);
            x[tw] = __builtin_fmaf((float)dv4[2], kDigitW2, __builtin_fmaf((float)dv4[1], kDigitW1, (float)dv4[0])) * sc;
        }
        // Row r of x[tw] holds (q, k, 0, 0)[r] of tile tw.  The row swaps bring tile lg's
        // q and k sums to lane group lg: v_permlane16_swap gives rows (q0, q1, -, -) and
        // (k0, k1, -, -) from tiles 0 and 1 (and the same from tiles 2 and 3), and
        // v_permlane32_swap the upper tiles' rows 0-1 to rows 2-3.
        const auto p01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[0]), __float_as_uint(x[1]), false, false);
        const auto p23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[2]), __float_as_uint(x[3]), false, false);
        const auto pq = __builtin_amdgcn_permlane32_swap(p01[0], p23[0], false, false);
        const auto pk = __builtin_amdgcn_permlane32_swap(p01[1], p23[1], false, false);
        const float hq = sj * __uint_as_float(pq[0]) + cq, hk = sj * __uint_as_float(pk[0]) + ck;
        const float mn = beta * (vj - hk - sr);
        st_nt(a.bm + head * (size_t)W * DV + (size_t)n * DV + j, mn);
        tok_st<TI>(a.o, head * DV + j, hq + sa + an * mn);
    }
}

template <int DK, int WM, bool KDA, int NB>
hipError_t launch_nb(const lq_dims& d, const DecodeArgs& args, hipStream_t s) {
    constexpr int NT = Dec<DK, DK, WM, KDA>::NT;
    const unsigned grid = (unsigned)d.B * (unsigned)d.H;
    if constexpr (DK == 128 && WM <= 16) {      // (with 32 slots the m columns need the registers)
        if (d.io_dtype == LQ_IO_BF16)
            return launch_kernel(LQ_KERNEL_DECODE, decode_split_kernel<WM, KDA, NB, uint16_t>, dim3(grid), dim3(NT),
                                 s, args);
        return launch_kernel(LQ_KERNEL_DECODE, decode_split_kernel<WM, KDA, NB, float>, dim3(grid), dim3(NT), s,
                             args);
    }
    if (d.io_dtype == LQ_IO_BF16)
        return launch_kernel(LQ_KERNEL_DECODE, decode_kernel<DK, DK, WM, KDA, NB, uint16_t>, dim3(grid), dim3(NT),
                             s, args);
    return launch_kernel(LQ_KERNEL_DECODE, decode_kernel<DK, DK, WM, KDA, NB, float>, dim3(grid), dim3(NT), s,
                         args);
}

// dk = 128, W <= 16: one kernel per window position (no runtime guards).
template <bool KDA, int... NBS>
hipError_t launch_fixed(const lq_dims& d, const DecodeArgs& args, hipStream_t s,
                        std::integer_sequence<int, NBS...>) {
    hipError_t e = hipErrorInvalidValue;
    ((args.pos == NBS ? (e = launch_nb<128, 16, KDA, NBS>(d, args, s), 0) : 0), ...);
    return e;
}

template <int DK>
hipError_t launch_dk(const lq_dims& d, const DecodeArgs& args, hipStream_t s) {
    const bool kda = d.decay_mode == LQ_DECAY_PER_KEY;
    switch (wbucket(d.W)) {
        case 4: return kda ? launch_nb<DK, 4, true, -1>(d, args, s) : launch_nb<DK, 4, false, -1>(d, args, s);
        case 8: return kda ? launch_nb<DK, 8, true, -1>(d, args, s) : launch_nb<DK, 8, false, -1>(d, args, s);
        case 16:
            if constexpr (DK == 128)
                if (!args.pos_dev)
                    return kda ? launch_fixed<true>(d, args, s, std::make_integer_sequence<int, 16>{})
                               : launch_fixed<false>(d, args, s, std::make_integer_sequence<int, 16>{});
            return kda ? launch_nb<DK, 16, true, -1>(d, args, s) : launch_nb<DK, 16, false, -1>(d, args, s);
        default: return kda ? launch_nb<DK, 32, true, -1>(d, args, s) : launch_nb<DK, 32, false, -1>(d, args, s);
    }
}

}  // namespace

hipError_t launch_decode(const lq_dims& d, const lq_state& st, int pos, const int32_t* pos_dev,
                         const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, void* o, hipStream_t s) {
    DecodeArgs args{st.sq, st.row_scale, st.col_scale, st.comp_idx, st.comp_val,
                    st.buf_k, st.buf_m, st.buf_g,
                    q, k, v, alpha, beta, o, pos_dev, d.W, d.C, d.H, pos};
    switch (d.dk) {
        case 16: return launch_dk<16>(d, args, s);
        case 64: return launch_dk<64>(d, args, s);
        default: return launch_dk<128>(d, args, s);
    }
}

}  // namespace lq

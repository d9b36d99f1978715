// decode.hip -- one decode token over the int8 state (gfx950).
//
// LeapQuant abstract (HFEPX paper page, "Abstract"): inside a window the
// output is computed from the fixed low-bit state plus high-precision
// buffered updates; the compensator tokens share the update path of real
// tokens.  News article ("A linear-attention method cuts state ...",
// paragraph 3): no update is skipped.  With the window-base state Hb and the
// buffer (k_i, y_i, u_i, g_i), slot n's output is
//     o = Hb^T q' + sum_{i<=n} a_i u_i,   q' = exp(g_n) o q - sum_{i<=n} a_i y_i,
// and Hb^T q' = s o (sq^T (r o q')) + sum_c q'[idx_c] cv_c.
//
// One workgroup per (b, h).  Every global load the step needs is issued at
// the top (the int8 state as 128-bit loads, the buffer rows, the inputs), so
// the dependent chain buffer-dots -> q' -> int8 GEMV runs on data already
// in flight.  Threads play three roles:
//   * slot groups: TPS lanes per buffer slot compute rr_i = <k, E_i o k_i>
//     and a_i = <q, E_i o k_i> (lane-group reductions);
//   * channel threads t < DK own key channel t: y_n[t] and q'[t];
//   * value threads DK <= t < DK+DV own value column j: u_n[j], the buffer
//     part of o[j] and the final output;
//   * all threads: the int8 GEMV, VEC bytes x PASSES rows each, partial sums
//     reduced through LDS.
#include "lq_internal.h"

namespace lq {
namespace {

struct DecodeArgs {
    const int8_t* sq;
    const float* r;
    const float* s;
    const int32_t* idx;
    const float* cv;
    float* bk;
    float* by;
    float* bu;
    float* bg;
    const float* q;
    const float* k;
    const float* v;
    const float* alpha;
    const float* beta;
    float* o;
    int W;
    int C;
    int pos;
};

template <int DK, int DV, int WM, bool KDA, int NT>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeArgs a) {
    static_assert(NT >= DK + DV, "one thread per key channel and per value column");
    constexpr int GD = KDA ? DK : 1;
    // int8 GEMV tiling
    constexpr int VEC = (DK * DV / 16 >= NT) ? 16 : 4;   // bytes per thread per row
    constexpr int CPR = DV / VEC;                         // chunks per row
    constexpr int RPP = NT / CPR;                         // rows per pass
    constexpr int PASSES = DK / RPP;
    static_assert(NT % CPR == 0 && DK % RPP == 0 && PASSES >= 1, "GEMV tiling");
    // buffer-dot tiling
    constexpr int TPS = NT / WM;                          // lanes per slot
    constexpr int CH = DK / TPS;                          // channels per lane
    static_assert(TPS <= 64 && CH >= 1 && DK % TPS == 0, "slot-group tiling");

    __shared__ float s_rr[WM];
    __shared__ float s_a[WM];
    __shared__ float s_q2[DK];
    __shared__ float s_qp[DK];
    __shared__ __align__(16) float s_red[RPP][DV];

    const int t = threadIdx.x;
    const size_t head = blockIdx.x;
    const int n = a.pos;
    const int W = a.W;
    const int C = a.C;

    const int8_t* __restrict__ sq = a.sq + head * (DK * DV);
    const float* __restrict__ bk = a.bk + head * (size_t)W * DK;
    const float* __restrict__ by = a.by + head * (size_t)W * DK;
    const float* __restrict__ bu = a.bu + head * (size_t)W * DV;
    const float* __restrict__ bg = a.bg + head * (size_t)W * GD;
    const float* __restrict__ qv = a.q + head * DK;
    const float* __restrict__ kv = a.k + head * DK;
    const float* __restrict__ av = a.alpha + head * GD;

    // ---- issue loads: int8 state chunks -----------------------------------
    using chunk_t = typename std::conditional<VEC == 16, uint4, uint32_t>::type;
    chunk_t ch[PASSES];
    const int g_row = t / CPR;
    const int g_col = (t % CPR) * VEC;
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        ch[p] = *reinterpret_cast<const chunk_t*>(sq + (size_t)(p * RPP + g_row) * DV + g_col);

    // ---- slot-group loads ----------------------------------------------------
    const int slot = t / TPS;
    const int c0 = (t % TPS) * CH;
    float kq[CH], kk[CH], ks[CH], gs[CH], gp[CH], al[CH];
    load_floats<CH>(qv + c0, kq);
    load_floats<CH>(kv + c0, kk);
    if (slot < n) {
        load_floats<CH>(bk + (size_t)slot * DK + c0, ks);
        if constexpr (KDA) load_floats<CH>(bg + (size_t)slot * DK + c0, gs);
        else gs[0] = bg[slot];
    }
    if constexpr (KDA) {
        load_floats<CH>(av + c0, al);
        if (n > 0) load_floats<CH>(bg + (size_t)(n - 1) * DK + c0, gp);
    }
    const float beta = a.beta[head];
    const float gprev_s = (!KDA && n > 0) ? bg[n - 1] : 0.0f;
    const float gn_s = KDA ? 0.0f : gprev_s + logf(av[0]);

    // ---- channel / value thread loads --------------------------------------
    constexpr int CMAX = 8;
    float col[WM > 1 ? WM - 1 : 1];
    const bool is_ch = t < DK;
    const bool is_val = t >= DK && t < DK + DV;
    const int j = t - DK;
    float x_q = 0.0f, x_k = 0.0f, x_r = 0.0f, x_g = 0.0f;   // channel thread
    float x_v = 0.0f, x_s = 0.0f;                           // value thread
    float cvr[CMAX];
    int cid[CMAX];
    if (is_ch) {
#pragma unroll
        for (int i = 0; i < WM - 1; ++i)
            if (i < n) col[i] = by[(size_t)i * DK + t];
        x_q = qv[t];
        x_k = kv[t];
        x_r = a.r[head * DK + t];
        if constexpr (KDA) x_g = (n > 0 ? bg[(size_t)(n - 1) * DK + t] : 0.0f) + logf(av[t]);
    } else if (is_val) {
#pragma unroll
        for (int i = 0; i < WM - 1; ++i)
            if (i < n) col[i] = bu[(size_t)i * DV + j];
        x_v = a.v[head * DV + j];
        x_s = a.s[head * DV + j];
#pragma unroll
        for (int c = 0; c < CMAX; ++c)
            if (c < C) {
                cid[c] = a.idx[head * C + c];
                cvr[c] = a.cv[(head * C + c) * (size_t)DV + j];
            }
    }

    // ---- 1. buffer inner products -------------------------------------------
    {
        float rr = 0.0f, aa = 0.0f;
        if (slot < n) {
            if constexpr (KDA) {
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const float gnc = (n > 0 ? gp[c] : 0.0f) + logf(al[c]);
                    const float e = __expf(gnc - gs[c]);
                    const float x = ks[c] * e;
                    rr += kk[c] * x;
                    aa += kq[c] * x;
                }
            } else {
                const float e = __expf(gn_s - gs[0]);
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    rr += kk[c] * ks[c];
                    aa += kq[c] * ks[c];
                }
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
    lds_barrier();

    // ---- 2. WY append and transformed query ---------------------------------
    float wsum = 0.0f;   // value threads: sum_{i<=n} a_i u_i[j]
    if (is_ch) {
        const float qc = x_q, kc = x_k;
        const float gn = KDA ? x_g : gn_s;
        const float en = __expf(gn);
        float ay = en * kc, aq = en * qc;
#pragma unroll
        for (int i = 0; i < WM - 1; ++i)
            if (i < n) {
                ay -= s_rr[i] * col[i];
                aq -= s_a[i] * col[i];
            }
        const float yn = beta * ay;
        const float qp = aq - s_a[n] * yn;
        float* byw = a.by + head * (size_t)W * DK + (size_t)n * DK;
        float* bkw = a.bk + head * (size_t)W * DK + (size_t)n * DK;
        byw[t] = yn;
        bkw[t] = kc;
        if constexpr (KDA) a.bg[head * (size_t)W * DK + (size_t)n * DK + t] = gn;
        else if (t == 0) a.bg[head * (size_t)W + n] = gn;
        s_qp[t] = qp;
        s_q2[t] = x_r * qp;
    } else if (is_val) {
        float au = x_v;
#pragma unroll
        for (int i = 0; i < WM - 1; ++i)
            if (i < n) {
                au -= s_rr[i] * col[i];
                wsum += s_a[i] * col[i];
            }
        const float un = beta * au;
        wsum += s_a[n] * un;
        a.bu[head * (size_t)W * DV + (size_t)n * DV + j] = un;
    }
    lds_barrier();

    // ---- 3. int8 GEMV: partial sums of sq^T (r o q') ------------------------
    {
        float acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const float x = s_q2[p * RPP + g_row];
            if constexpr (VEC == 16) {
                const uint32_t w4[4] = {ch[p].x, ch[p].y, ch[p].z, ch[p].w};
#pragma unroll
                for (int wi = 0; wi < 4; ++wi)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[4 * wi + e] += x * sbyte(w4[wi], e);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += x * sbyte(ch[p], e);
            }
        }
        store_floats<VEC>(&s_red[g_row][g_col], acc);
    }
    lds_barrier();

    // ---- 4. output ------------------------------------------------------------
    if (is_val) {
        float gem = 0.0f;
#pragma unroll
        for (int g = 0; g < RPP; ++g) gem += s_red[g][j];
        float out = x_s * gem + wsum;
#pragma unroll
        for (int c = 0; c < CMAX; ++c)
            if (c < C) out += s_qp[cid[c]] * cvr[c];
        a.o[head * DV + j] = out;
    }
}

template <int DK, int WM, bool KDA>
hipError_t launch_t(const lq_dims& d, const DecodeArgs& args, hipStream_t s) {
    constexpr int NT = (2 * DK < 64) ? 64 : 2 * DK;
    const unsigned grid = (unsigned)d.B * (unsigned)d.H;
    hipLaunchKernelGGL((decode_kernel<DK, DK, WM, KDA, NT>), dim3(grid), dim3(NT), 0, s, args);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const lq_dims& d, const DecodeArgs& args, hipStream_t s) {
    const bool kda = d.decay_mode == LQ_DECAY_PER_KEY;
    switch (wbucket(d.W)) {
        case 4: return kda ? launch_t<DK, 4, true>(d, args, s) : launch_t<DK, 4, false>(d, args, s);
        case 8: return kda ? launch_t<DK, 8, true>(d, args, s) : launch_t<DK, 8, false>(d, args, s);
        case 16: return kda ? launch_t<DK, 16, true>(d, args, s) : launch_t<DK, 16, false>(d, args, s);
        default: return kda ? launch_t<DK, 32, true>(d, args, s) : launch_t<DK, 32, false>(d, args, s);
    }
}

}  // namespace

hipError_t launch_decode(const lq_dims& d, const lq_state& st, int pos, const float* q,
                         const float* k, const float* v, const float* alpha, const float* beta,
                         float* o, hipStream_t s) {
    DecodeArgs args{st.sq, st.row_scale, st.col_scale, st.comp_idx, st.comp_val,
                    st.buf_k, st.buf_y, st.buf_u, st.buf_g,
                    q, k, v, alpha, beta, o, d.W, d.C, pos};
    switch (d.dk) {
        case 16: return launch_dk<16>(d, args, s);
        case 64: return launch_dk<64>(d, args, s);
        default: return launch_dk<128>(d, args, s);
    }
}

}  // namespace lq

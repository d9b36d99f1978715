// prefill.hip -- chunked fp32 prefill of a prompt (gfx950): the state after T
// tokens from a given fp32 state, then one quantization into the codec.
//
// LeapQuant abstract (HFEPX paper page, "Abstract"): the low-bit state is
// what decoding reads; News article ("A linear-attention method cuts state
// ...", paragraph 3): it is quantized once per window, not per token.  The
// prompt therefore runs in fp32 and its final state is quantized once.
//
// Chunk form of the gated delta rule.  For a chunk of L = 16 tokens starting
// from state H0, with chunk-local log-decays g_n (prefix sums of log alpha; a
// vector per token for per-key decay) and E_{n,i} = exp(g_n - g_i):
//     rr_{n,i} = <k_n, E_{n,i} o k_i>  (i < n),    a_{n,i} = <q_n, E_{n,i} o k_i>  (i <= n),
//     m_n = beta_n (v_n - H0^T (e^{g_n} o k_n) - sum_{i<n} rr_{n,i} m_i),
//     o_n = H0^T (e^{g_n} o q_n) + sum_{i<=n} a_{n,i} m_i,
//     H   = diag(e^{g_L}) H0 + sum_n (E_{L,n} o k_n) m_n^T,
// the same algebra as a decode window (the m_n are the window slots projected
// through H0).  In matrix form M = T R with T = (I + A)^{-1}, A_{n,i} = beta_n
// rr_{n,i} (strictly lower) and R_n = beta_n (v_n - H0^T (e^{g_n} o k_n)).
//
// One workgroup per (b, h); NW waves, wave w owns the column band
// [w*DV/NW, (w+1)*DV/NW) of H for every row, in v_mfma_f32_16x16x4_f32
// accumulator tiles (tile (rt, ct): rows rt*16 + 4*(lane/16) + v, column
// lane%16 of the band's tile ct).  Every product of the chunk is an fp32 MFMA
// whose register operand is already in place:
//     HK = (e^g o K) H0, HQ = (e^g o Q) H0   (H0 tiles as B operands, K index = row),
//     M  = T R,  O = HQ + (P o mask) M       (R, M in D layout are B operands, K index = token),
//     H  = diag(e^{g_L}) H0 + Kt^T M         (M as B operand, H tiles accumulate),
// so the state never leaves the registers between the first load and the
// final store.  The small L x L products (K K^T, Q K^T; the triangular solve)
// run once per chunk on one or two waves (scalar decay) or on all lanes with a
// per-channel exponential per pair (per-key decay).
#include "lq_internal.h"

namespace lq {
namespace {

struct PrefillArgs {
    float* h;
    const void* q;            // q, k, v, o: fp32 or bf16 (the kernel's TI)
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    void* o;
    int T;
    int heads;     // B*H: stride between tokens, in heads
};

constexpr int CL = 16;   // chunk length (the MFMA tile)

template <int DK, int DV, bool KDA, typename TI>
struct PF {
    static_assert(DK == DV && DK % 16 == 0, "square heads, 16-multiples");
    static constexpr int NW = DV / 16 < 4 ? DV / 16 : 4;   // waves
    static constexpr int NT = 64 * NW;
    static constexpr int RT = DK / 16;                     // row tiles
    static constexpr int CTW = DV / 16 / NW;               // column tiles per wave
    static constexpr int NMAT = KDA ? 4 : 3;               // q, k, v [, alpha] rows per chunk
    // token rows are DKP floats apart in LDS: the 16-byte pad puts row n's word
    // c in bank (4n + c) mod 64, so reads of one column across rows, or of
    // 16-byte pieces of 16 rows, do not collide
    static constexpr int DKP = DK + 4;
    // LDS (floats)
    static constexpr int TOK = 0;                          // [NMAT][CL][DKP]: q | k | v [| alpha -> g]
    static constexpr int XK = TOK + NMAT * CL * DKP;       // per-key: e^g o k, e^g o q, e^{gL-g} o k
    static constexpr int XQ = XK + (KDA ? CL * DKP : 0);
    static constexpr int KT = XQ + (KDA ? CL * DKP : 0);
    static constexpr int DL = KT + (KDA ? CL * DKP : 0);   // per-key: e^{gL} [DK]
    static constexpr int AB = DL + (KDA ? DK : 0);         // alpha [CL] | beta [CL] (raw)
    static constexpr int G = AB + 2 * CL;                  // scalar: g [CL]; beta masked [CL]
    static constexpr int SA = G + 2 * CL;                  // A = beta rr (strictly lower) [CL][CL]
    static constexpr int SP = SA + CL * CL;                // P = a masked [CL][CL]
    static constexpr int ST = SP + CL * CL;                // T = (I + A)^{-1} [CL][CL]
    static constexpr int STG = ST + CL * CL;               // bf16 q | k | v rows as loaded [3][CL][DK]
    static constexpr int FLOATS = STG + (sizeof(TI) == 2 ? 3 * CL * DK / 2 : 0);
    // waves per SIMD the registers are sized for (4: 128 registers, the state
    // tiles take 64 of them at d = 128).  Per-key decay at d = 128 keeps
    // 63-75 KB of LDS per workgroup, i.e. two workgroups (two waves per SIMD)
    // per CU, and is given the registers of that occupancy; at d = 16 with bf16
    // rows it needs 129 registers, i.e. three waves.
    static constexpr int WPE = !KDA ? 4 : DK == 128 ? 2 : (DK == 16 && sizeof(TI) == 2) ? 3 : 4;
};

template <int DK, int DV, bool KDA, typename TI>
__global__ __launch_bounds__((PF<DK, DV, KDA, TI>::NT))
__attribute__((amdgpu_waves_per_eu(PF<DK, DV, KDA, TI>::WPE, PF<DK, DV, KDA, TI>::WPE)))
void prefill_kernel(PrefillArgs a) {
    using P = PF<DK, DV, KDA, TI>;
    constexpr int NW = P::NW, NT = P::NT, RT = P::RT, CTW = P::CTW, DKP = P::DKP;
    __shared__ __align__(16) float sm[P::FLOATS];
    float* sQ = sm + P::TOK;
    float* sK = sQ + CL * DKP;
    float* sV = sK + CL * DKP;
    float* sAl = sV + CL * DKP;               // per-key alpha, then g (in place)
    float* sXk = sm + P::XK;
    float* sXq = sm + P::XQ;
    float* sKt = sm + P::KT;
    float* sDl = sm + P::DL;
    float* sAB = sm + P::AB;
    float* sG = sm + P::G;                    // scalar g [CL], masked beta [CL]
    float* sBm = sG + CL;
    float* sA = sm + P::SA;
    float* sP = sm + P::SP;
    float* sT = sm + P::ST;

    const int t = threadIdx.x;
    const int lane = t & 63, li = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const size_t head = blockIdx.x;
    const size_t heads = (size_t)a.heads;
    const int T = a.T;

    // state tiles: H[rt][ct][v] = H[rt*16 + 4*lg + v][col(ct)], col(ct) = (w*CTW + ct)*16 + li
    float* hp = a.h + head * (size_t)DK * DV;
    v4f H[RT][CTW];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                H[rt][ct][v] = hp[(size_t)(rt * 16 + 4 * lg + v) * DV + (w * CTW + ct) * 16 + li];

    for (int c0 = 0; c0 < T; c0 += CL) {
        const int L = min(CL, T - c0);        // tokens of this chunk; the rest are identity steps
        // ---- chunk tokens -> LDS (rows past T repeat the last token; they are masked) ----
        {
            if constexpr (sizeof(TI) == 4) {
                // one copy per row into its padded LDS row (DK/4 lanes of 16 bytes)
                for (int row = w; row < P::NMAT * CL; row += NW) {
                    const int mat = row / CL, n = row % CL;
                    const size_t th = (size_t)min(c0 + n, T - 1) * heads + head;
                    const float* src = mat == 0 ? static_cast<const float*>(a.q) + th * DK
                                     : mat == 1 ? static_cast<const float*>(a.k) + th * DK
                                     : mat == 2 ? static_cast<const float*>(a.v) + th * DV
                                                : a.alpha + th * DK;
                    if (lane < DK / 4) lds_dma16(src + 4 * lane, sQ + row * DKP);
                }
            } else {
                // bf16 q, k, v rows as they are into the staging rows, whole copies
                constexpr int RB = DK * 2;                   // bytes per token row
                constexpr int RPC = 1024 / RB;               // rows per wave-wide 16-byte copy
                constexpr int NCOPY = (3 * CL + RPC - 1) / RPC;
                char* tdst = reinterpret_cast<char*>(sm + P::STG);
                const int rin = lane / (RB / 16), off = 16 * (lane % (RB / 16));
                for (int cp = w; cp < NCOPY; cp += NW) {
                    const int row = cp * RPC + rin;          // row of the [3][CL] stack
                    if (row >= 3 * CL) continue;
                    // one matrix per copy when its rows divide the chunk (a scalar choice)
                    const int mat = CL % RPC == 0 ? cp * RPC / CL : row / CL, n = row % CL;
                    const size_t th = (size_t)min(c0 + n, T - 1) * heads + head;
                    const void* src = mat == 0 ? a.q : mat == 1 ? a.k : a.v;
                    lds_dma16(reinterpret_cast<const char*>(src) + th * RB + off, tdst + cp * 1024);
                }
                if constexpr (KDA) {
                    for (int n = w; n < CL; n += NW) {
                        const size_t th = (size_t)min(c0 + n, T - 1) * heads + head;
                        if (lane < DK / 4) lds_dma16(a.alpha + th * DK + 4 * lane, sAl + n * DKP);
                    }
                }
            }
            if (w == 0 && lane < 2 * CL) {
                // lanes 0..15: scalar alpha (per-key: unused), lanes 16..31: beta
                const int n = lane % CL;
                const size_t th = (size_t)min(c0 + n, T - 1) * heads + head;
                if (lane < CL) lds_dma4((KDA ? a.beta : a.alpha) + th, sAB);
                else lds_dma4(a.beta + th, sAB);
            }
        }
        all_loads_barrier();
        if constexpr (sizeof(TI) == 2) {
            // bf16 rows -> the fp32 q | k | v rows (exact)
            const uint32_t* stg = reinterpret_cast<const uint32_t*>(sm + P::STG);
#pragma unroll 1
            for (int e = t; e < 3 * CL * DK / 2; e += NT) {
                const uint32_t x = stg[e];
                const int row = 2 * e / DK, col = 2 * e % DK;
                *reinterpret_cast<float2*>(sQ + row * DKP + col) =
                    make_float2(__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u));
            }
            lds_barrier();
        }

        // ---- gates: chunk-local log-decay prefix g, masked beta ------------------------------------
        if constexpr (KDA) {
            if (t < DK) {
                float g = 0.0f;
#pragma unroll
                for (int n = 0; n < CL; ++n) {
                    g += n < L ? logf(sAl[n * DKP + t]) : 0.0f;
                    sAl[n * DKP + t] = g;
                }
                sDl[t] = __expf(g);
#pragma unroll
                for (int n = 0; n < CL; ++n) {
                    const float gn = sAl[n * DKP + t];
                    const float e = __expf(gn);
                    sXk[n * DKP + t] = e * sK[n * DKP + t];
                    sXq[n * DKP + t] = e * sQ[n * DKP + t];
                    sKt[n * DKP + t] = __expf(g - gn) * sK[n * DKP + t];
                }
            }
        } else if (t == 0) {
            float g = 0.0f;
#pragma unroll
            for (int n = 0; n < CL; ++n) {
                g += n < L ? logf(sAB[n]) : 0.0f;
                sG[n] = g;
            }
        }
        if (t < CL) sBm[t] = t < L ? sAB[CL + t] : 0.0f;
        lds_barrier();

        // ---- A = beta rr (strictly lower), P = a (lower incl. diagonal) --------------------------
        if constexpr (KDA) {
            // thread (n, i) = (t/16, t%16) for the 16 x 16 pairs (NT >= 256), or a loop
            for (int pr = t; pr < CL * CL; pr += NT) {
                const int n = pr / CL, i = pr % CL;
                float rr = 0.0f, aa = 0.0f;
                if (i <= n) {
                    for (int c = 0; c < DK; c += 4) {
                        float kn[4], ki[4], qn[4], gn[4], gi[4];
                        load_floats<4>(sK + n * DKP + c, kn);
                        load_floats<4>(sK + i * DKP + c, ki);
                        load_floats<4>(sQ + n * DKP + c, qn);
                        load_floats<4>(sAl + n * DKP + c, gn);
                        load_floats<4>(sAl + i * DKP + c, gi);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float x = ki[e] * __expf(gn[e] - gi[e]);
                            rr = __builtin_fmaf(kn[e], x, rr);
                            aa = __builtin_fmaf(qn[e], x, aa);
                        }
                    }
                }
                sA[pr] = i < n ? sBm[n] * rr : 0.0f;
                sP[pr] = aa;
            }
        } else {
            // K K^T on wave 0, Q K^T on wave 1 (both on wave 0 if there is one wave);
            // A[i=n][k] = X[n][4ks+k], B[k][j] = K[j][4ks+k]
#pragma unroll
            for (int which = 0; which < 2; ++which) {
                if (w != which % NW) continue;
                const float* X = which == 0 ? sK : sQ;
                v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
                for (int ks = 0; ks < DK / 4; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[li * DKP + 4 * ks + lg], sK[li * DKP + 4 * ks + lg],
                                                               acc, 0, 0, 0);
                // D[n = 4lg+v][i = li]
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int n = 4 * lg + v, i = li;
                    const float e = __expf(sG[n] - sG[i]);
                    if (which == 0) sA[n * CL + i] = i < n ? sBm[n] * (e * acc[v]) : 0.0f;
                    else sP[n * CL + i] = i <= n ? e * acc[v] : 0.0f;
                }
            }
        }
        lds_barrier();

        // ---- T = (I + A)^{-1}: lane j < 16 of wave 0 solves column j --------------------------------
        if (t < CL) {
            int j = t;
            asm volatile("" : "+v"(j));          // keeps the unit-row constants out of the chunk loop
            float tc[CL];
#pragma unroll
            for (int n = 0; n < CL; ++n) {
                float arow[CL];
                load_floats<CL>(sA + n * CL, arow);
                float x = n == j ? 1.0f : 0.0f;
#pragma unroll
                for (int i = 0; i < n; ++i) x = __builtin_fmaf(-arow[i], tc[i], x);
                tc[n] = n < j ? 0.0f : x;
                sT[n * CL + j] = tc[n];
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        lds_barrier();

        // ---- per column tile of this wave's band ----------------------------------------------------
        float eg = 0.0f, ekt[4] = {0.f, 0.f, 0.f, 0.f}, egl = 0.0f;
        if constexpr (!KDA) {
            eg = __expf(sG[li]);                          // A rows of HK / HQ: token li
            egl = __expf(sG[CL - 1]);
#pragma unroll
            for (int kv = 0; kv < 4; ++kv) ekt[kv] = __expf(sG[CL - 1] - sG[4 * lg + kv]);   // Kt tokens
        }
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int col = (w * CTW + ct) * 16 + li;
            v4f hk = {0.f, 0.f, 0.f, 0.f}, hq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                // A operands of rows rt*16 + 4*lg + (0..3): one 16-byte read per vector
                float ak[4], aq[4];
                load_floats<4>((KDA ? sXk : sK) + li * DKP + rt * 16 + 4 * lg, ak);
                load_floats<4>((KDA ? sXq : sQ) + li * DKP + rt * 16 + 4 * lg, aq);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    hk = __builtin_amdgcn_mfma_f32_16x16x4f32(KDA ? ak[v] : ak[v] * eg, H[rt][ct][v], hk, 0, 0, 0);
                if (a.o) {                                // HQ only feeds the outputs
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        hq = __builtin_amdgcn_mfma_f32_16x16x4f32(KDA ? aq[v] : aq[v] * eg, H[rt][ct][v], hq, 0, 0, 0);
                }
                if (rt % 2 == 1) __builtin_amdgcn_sched_barrier(0);
            }
            // R = beta (v - HK); M = T R; O = HQ + P M   (token n = 4*lg + v of column col)
            v4f r, m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = 4 * lg + v;
                r[v] = sBm[n] * (sV[n * DKP + col] - hk[v]);
            }
#pragma unroll
            for (int kv = 0; kv < 4; ++kv)
                m = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[li * CL + 4 * lg + kv], r[kv], m, 0, 0, 0);
            if (a.o) {
#pragma unroll
                for (int kv = 0; kv < 4; ++kv)
                    hq = __builtin_amdgcn_mfma_f32_16x16x4f32(sP[li * CL + 4 * lg + kv], m[kv], hq, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int n = 4 * lg + v;
                    if (n < L) tok_st<TI>(a.o, ((size_t)(c0 + n) * heads + head) * DV + col, hq[v]);
                }
            }
            // H = diag(e^{g_L}) H + Kt^T M, Kt[n][row] = e^{g_L - g_n} k_n[row]
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if constexpr (KDA) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) H[rt][ct][v] *= sDl[rt * 16 + 4 * lg + v];
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v) H[rt][ct][v] *= egl;
                }
#pragma unroll
                for (int kv = 0; kv < 4; ++kv) {
                    const int n = 4 * lg + kv, row = rt * 16 + li;
                    const float av = KDA ? sKt[n * DKP + row] : sK[n * DKP + row] * ekt[kv];
                    H[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, m[kv], H[rt][ct], 0, 0, 0);
                }
                if (rt % 2 == 1) __builtin_amdgcn_sched_barrier(0);
            }
        }
        lds_barrier();                                    // LDS is refilled by the next chunk
    }

    // the store addresses are recomputed from an opaque copy of the lane's base, so
    // the load addresses are not kept live through the chunk loop
    int tt = threadIdx.x;
    asm volatile("" : "+v"(tt));
    const int base = 4 * ((tt & 63) >> 4) * DV + (tt >> 6) * CTW * 16 + (tt & 15);
    float* hb = hp + base;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
            for (int v = 0; v < 4; ++v) hb[(rt * 16 + v) * DV + ct * 16] = H[rt][ct][v];
}

template <int DK, bool KDA>
hipError_t prefill_t(const lq_dims& d, const PrefillArgs& args, hipStream_t s) {
    const dim3 grid((unsigned)d.B * (unsigned)d.H);
    if (d.io_dtype == LQ_IO_BF16)
        return launch_kernel(LQ_KERNEL_PREFILL, prefill_kernel<DK, DK, KDA, uint16_t>, grid,
                             dim3(PF<DK, DK, KDA, uint16_t>::NT), s, args);
    return launch_kernel(LQ_KERNEL_PREFILL, prefill_kernel<DK, DK, KDA, float>, grid,
                         dim3(PF<DK, DK, KDA, float>::NT), s, args);
}

}  // namespace

hipError_t launch_prefill(const lq_dims& d, float* h, int T, const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta, void* o, hipStream_t s) {
    PrefillArgs args{h, q, k, v, alpha, beta, o, T, d.B * d.H};
    const bool kda = d.decay_mode == LQ_DECAY_PER_KEY;
    switch (d.dk) {
        case 16: return kda ? prefill_t<16, true>(d, args, s) : prefill_t<16, false>(d, args, s);
        case 64: return kda ? prefill_t<64, true>(d, args, s) : prefill_t<64, false>(d, args, s);
        default: return kda ? prefill_t<128, true>(d, args, s) : prefill_t<128, false>(d, args, s);
    }
}

}  // namespace lq

"""Pins of the oracle's windowed scheme and its WY buffer algebra.

* With quantization off, the WY window route equals the plain recurrence on
  every output and on the state at every boundary (the pages: no update is
  skipped, only the rounding is deferred).
* Brute force at dk = dv = 4: dense products of the explicit transitions
  T_t = (I - beta k k^T) D_t give A_n and U_n, which must match the buffer
  terms y_i, u_i, g_i entry by entry, for every W in 1..4.
* W = 1 with no compensators is per-token quantization (dequantize, one exact
  step, output, quantize); with smoothing off it is the textbook per-row int8
  state.
* The buffer depends on the window's tokens only, an early (partial) flush
  equals the plain recurrence, and the C whole-run runner equals the
  per-window composition of the primitives.
"""
import numpy as np
import pytest

from recurrent_state_quant_lq_amd import inputs


def _tok(seed, T, dk, dv, per_key, outliers=None):
    t = inputs.host_tokens(seed, T, 1, 1, dk, dv, per_key=per_key, beta_lo=0.1, beta_hi=0.9,
                           outliers=outliers)
    return {k: np.ascontiguousarray(v[:, 0, 0]) for k, v in t.items()}


@pytest.mark.parametrize("per_key", [False, True])
@pytest.mark.parametrize("W", [1, 3, 16])
def test_wy_route_equals_recurrence_without_codec(orc, per_key, W):
    dk, dv = 24, 20
    tok = _tok(100 + W, 40, dk, dv, per_key)
    H0 = np.random.default_rng(W).standard_normal((dk, dv))
    o_s, _, H_s, _ = orc.run_head(dk, dv, per_key, W, 0, 1, route=0, use_codec=False, tok=tok, H0=H0)
    o_w, _, H_w, _ = orc.run_head(dk, dv, per_key, W, 0, 1, route=1, use_codec=False, tok=tok, H0=H0)
    sc = np.abs(o_s).max(1, keepdims=True)
    assert (np.abs(o_w - o_s) / sc).max() < 1e-12
    assert np.abs(H_w - H_s).max() / np.abs(H_s).max() < 1e-12


def _explicit_transitions(tok, n_max, per_key, dk):
    Ts = []
    for t in range(n_max):
        k = tok["k"][t].astype(np.float64)
        d = tok["alpha"][t].astype(np.float64) if per_key else np.full(dk, float(tok["alpha"][t]))
        Ts.append((np.eye(dk) - float(tok["beta"][t]) * np.outer(k, k)) @ np.diag(d))
    return Ts


@pytest.mark.parametrize("per_key", [False, True])
@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_bruteforce_d4_buffer_terms(orc, per_key, W):
    dk = dv = 4
    tok = _tok(200 + W + 10 * per_key, W, dk, dv, per_key)
    Ts = _explicit_transitions(tok, W, per_key, dk)
    buf = orc.new_buffer(W, dk, dv, per_key)
    A = np.eye(dk)
    U = np.zeros((dk, dv))
    for n in range(W):
        orc.wy_append(buf, n, tok["k"][n], tok["v"][n], tok["alpha"][n], tok["beta"][n], per_key)
        A = Ts[n] @ A
        U = Ts[n] @ U + float(tok["beta"][n]) * np.outer(tok["k"][n].astype(np.float64),
                                                         tok["v"][n].astype(np.float64))
        g = buf["g"][n] if per_key else np.full(dk, buf["g"][n][0])
        A_wy = np.diag(np.exp(g))
        U_wy = np.zeros((dk, dv))
        for i in range(n + 1):
            gi = buf["g"][i] if per_key else np.full(dk, buf["g"][i][0])
            ek = np.exp(g - gi) * buf["k"][i]
            A_wy -= np.outer(ek, buf["y"][i])
            U_wy += np.outer(ek, buf["u"][i])
        np.testing.assert_allclose(A_wy, A, atol=1e-13)
        np.testing.assert_allclose(U_wy, U, atol=1e-13)
        # the cumulative log-decay is the window-local sum of log alpha
        la = np.log(tok["alpha"][:n + 1].astype(np.float64)).reshape(n + 1, -1).sum(0)
        np.testing.assert_allclose(buf["g"][n], la, rtol=1e-14)


@pytest.mark.parametrize("per_key", [False, True])
@pytest.mark.parametrize("C", [0, 1, 2, 3, 4])
def test_bruteforce_d4_window_outputs(orc, per_key, C):
    """Window outputs from the buffer equal dense-matrix outputs from the
    dequantized base state, for all compensator counts at d = 4."""
    dk = dv = 4
    W = 4
    tok = _tok(300 + C, W, dk, dv, per_key)
    H = np.random.default_rng(C).standard_normal((dk, dv)).astype(np.float32)
    cd = orc.quantize(H, C)
    Hb = orc.dequantize(cd)
    res = orc.window(cd, tok, per_key, W, C, route="wy")
    Ts = _explicit_transitions(tok, W, per_key, dk)
    X = Hb.copy()
    for n in range(W):
        X = Ts[n] @ X + float(tok["beta"][n]) * np.outer(tok["k"][n].astype(np.float64),
                                                         tok["v"][n].astype(np.float64))
        np.testing.assert_allclose(res["o"][n], X.T @ tok["q"][n].astype(np.float64), atol=1e-12)
    np.testing.assert_allclose(res["H"], X, atol=1e-12)


@pytest.mark.parametrize("smooth", [0, 1])
def test_w1_no_compensator_is_per_token_quantization(orc, smooth):
    dk, dv, T = 32, 32, 30
    tok = _tok(400 + smooth, T, dk, dv, False)
    cd0 = orc.quantize(np.zeros((dk, dv), np.float32), 0, smooth)
    # naive per-token scheme written out: dequantize, one exact step, output, quantize
    cd = cd0
    o_naive = []
    for t in range(T):
        H = orc.dequantize(cd)
        o_naive.append(orc.step(H, tok["q"][t], tok["k"][t], tok["v"][t], tok["alpha"][t:t + 1],
                                tok["beta"][t], False))
        cd = orc.quantize(H.astype(np.float32), 0, smooth)
    o_wy, cd_wy, _, _ = orc.run_head(dk, dv, False, 1, 0, smooth, route=1, use_codec=True,
                                     tok=tok, codec=cd0)
    o_naive = np.stack(o_naive)
    sc = np.abs(o_naive).max(1, keepdims=True)
    assert (np.abs(o_wy - o_naive) / sc).max() < 1e-6
    flips = np.abs(cd_wy["sq"].astype(int) - cd["sq"].astype(int))
    assert flips.max() <= 1 and (flips > 0).sum() <= 2
    if not smooth:
        assert (cd_wy["s"] == 1).all()


def test_buffer_depends_only_on_tokens(orc):
    dk, dv, W = 16, 16, 8
    tok = _tok(500, W, dk, dv, True)
    rng = np.random.default_rng(5)
    a = orc.window(orc.quantize(rng.standard_normal((dk, dv)).astype(np.float32), 2), tok, True, W, 2)
    b = orc.window(orc.quantize(rng.standard_normal((dk, dv)).astype(np.float32) * 9, 2), tok, True, W, 2)
    for key in ("k", "y", "u", "g"):
        assert (a["buf"][key] == b["buf"][key]).all()


@pytest.mark.parametrize("N", [1, 5, 11])
def test_early_flush_equals_recurrence(orc, N):
    dk, dv, W = 32, 24, 16
    tok = _tok(600 + N, N, dk, dv, True)
    cd = orc.quantize(np.random.default_rng(N).standard_normal((dk, dv)).astype(np.float32), 4)
    wy = orc.window(cd, tok, True, W, 4, route="wy")
    sq = orc.window(cd, tok, True, W, 4, route="seq")
    assert np.abs(wy["H"] - sq["H"]).max() / np.abs(sq["H"]).max() < 1e-12
    assert (np.abs(wy["o"] - sq["o"]) / np.abs(sq["o"]).max(1, keepdims=True)).max() < 1e-12


@pytest.mark.parametrize("per_key", [False, True])
def test_c_runner_equals_window_composition(orc, per_key):
    dk, dv, W, C, T = 32, 32, 8, 2, 8 * 5
    tok = _tok(700 + per_key, T, dk, dv, per_key)
    cd0 = orc.quantize(np.random.default_rng(7).standard_normal((dk, dv)).astype(np.float32), C)
    o_c, cd_c, _, _ = orc.run_head(dk, dv, per_key, W, C, 1, route=1, use_codec=True, tok=tok,
                                   codec=cd0)
    cd = cd0
    o_py = []
    for w in range(T // W):
        sl = {k: v[w * W:(w + 1) * W] for k, v in tok.items()}
        res = orc.window(cd, sl, per_key, W, C, route="wy")
        o_py.append(res["o"])
        cd = res["codec"]
    assert np.array_equal(np.concatenate(o_py), o_c)
    for key in cd:
        assert np.array_equal(cd[key], cd_c[key])


def test_windowing_beats_per_token_quantization(orc):
    """The pages' premise: rounding the state after every token accumulates
    error, deferring it to once per window with outliers kept aside does not
    (abstract and news article, paragraph 2).  Synthetic stream, error
    against the fp64 recurrence."""
    dk = dv = 64
    T = 256
    out = inputs.make_outliers(1, 1, dk, dv)
    tok = _tok(800, T, dk, dv, False, outliers=out)
    H0 = np.zeros((dk, dv))
    o_ref, _, _, _ = orc.run_head(dk, dv, False, T, 0, 1, route=0, use_codec=False, tok=tok, H0=H0)

    def err(W, C, sm):
        o, _, _, _ = orc.run_head(dk, dv, False, W, C, sm, route=1, use_codec=True, tok=tok,
                                  codec=orc.quantize(np.zeros((dk, dv), np.float32), C, sm))
        return float(np.sqrt(((o - o_ref) ** 2).mean() / (o_ref ** 2).mean()))

    naive, leap = err(1, 0, 0), err(16, 4, 1)
    assert leap < 0.5 * naive


def test_projected_buffer_form(orc):
    """The buffer form the kernels keep, checked on the oracle's WY buffer:
    with m_i = u_i - Hb^T y_i,
        m_n = beta_n (v_n - Hb^T (e^{g_n} o k_n) - sum_{i<n} rr_{n,i} m_i),
        o_n = Hb^T (e^{g_n} o q_n) + sum_{i<=n} a_{n,i} m_i,
    rr_{n,i} = <k_n, E_{n,i} o k_i>, a_{n,i} = <q_n, E_{n,i} o k_i>, in fp64,
    for scalar and per-key decay."""
    import numpy as np
    from recurrent_state_quant_lq_amd import inputs
    for per_key in (False, True):
        dk = dv = 16
        W, C = 6, 2
        tok = inputs.host_tokens(77, W, 1, 1, dk, dv, per_key=per_key, beta_lo=0.1, beta_hi=0.9)
        tok = orc.head_tokens(tok, 0, 0)
        rng = np.random.default_rng(5)
        cd = orc.quantize((rng.standard_normal((dk, dv)) * 0.3).astype(np.float32), C, 1)
        res = orc.window(cd, tok, per_key, W, C, 1)
        Hb = orc.dequantize(cd)
        b = res["buf"]
        m = b["u"] - b["y"] @ Hb
        for n in range(W):
            g = b["g"][n]
            E = np.exp(g[None, :] - b["g"][:n + 1]) if per_key else np.exp(g - b["g"][:n + 1])
            kt = E * b["k"][:n + 1]                                   # E_{n,i} o k_i
            k = tok["k"][n].astype(np.float64)
            q = tok["q"][n].astype(np.float64)
            rr = kt[:n] @ k
            a = kt @ q
            eg = np.exp(g)
            want_m = float(tok["beta"][n]) * (tok["v"][n] - Hb.T @ (eg * k) - rr @ m[:n])
            np.testing.assert_allclose(m[n], want_m, rtol=0, atol=1e-12 * max(1.0, np.abs(m).max()))
            o = Hb.T @ (eg * q) + a @ m[:n + 1]
            np.testing.assert_allclose(o, res["o"][n], rtol=0, atol=1e-12 * max(1.0, np.abs(o).max()))


@pytest.mark.parametrize("per_key", [False, True])
@pytest.mark.parametrize("flush_tail", [False, True])
def test_runner_partial_last_window(orc, per_key, flush_tail):
    """The C runner's last window of T mod W tokens is quantized only when
    asked (an early flush at the end of a sequence).  Asked, its codec is the
    codec of the fp32-rounded state that the plain recurrence reaches from the
    last full window's state over the tail tokens; not asked, the codec stays
    the one the last full window left.  Either way the tail's outputs are the
    recurrence's outputs from that state."""
    dk, dv, W, C = 16, 12, 8, 2
    T = 2 * W + 5
    tok = _tok(900 + per_key, T, dk, dv, per_key)
    cd0 = orc.quantize((np.random.default_rng(9).standard_normal((dk, dv)) * 0.5).astype(np.float32), C)
    o, cd, _, hf = orc.run_head(dk, dv, per_key, W, C, 1, route=0, use_codec=True, tok=tok,
                                codec=cd0, flush_tail=flush_tail)
    head = {k: v[:2 * W] for k, v in tok.items()}
    _, cd2, _, _ = orc.run_head(dk, dv, per_key, W, C, 1, route=0, use_codec=True, tok=head,
                                codec=cd0)
    Hs = orc.dequantize(cd2)
    for t in range(2 * W, T):
        ot = orc.step(Hs, tok["q"][t], tok["k"][t], tok["v"][t], tok["alpha"][t], tok["beta"][t],
                      per_key)
        assert np.array_equal(ot, o[t])
    want = orc.quantize(Hs.astype(np.float32), C, 1) if flush_tail else cd2
    for key in want:
        assert np.array_equal(cd[key], want[key]), key
    if flush_tail:
        assert np.array_equal(hf, Hs.astype(np.float32))
        assert not np.array_equal(cd["sq"], cd2["sq"])

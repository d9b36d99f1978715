"""Pins of the oracle's gated delta-rule step against closed forms.

Each case is a property fixed by the mathematics of the rule
H <- (I - beta k k^T) D H + beta k v^T, o = H^T q, not a retyping of it:
pure decay at beta = 0, the delta rule's write-then-read identity, an
orthonormal-key associative memory with decay, a one-hot key table, KDA with
uniform gates equal to GDN, and joint linearity in (H0, v).  Shapes use
dk != dv so that a transposed operand cannot pass.
"""
import numpy as np
import pytest

DK, DV = 8, 5


def _unit(rng, n):
    x = rng.standard_normal(n)
    return (x / np.linalg.norm(x)).astype(np.float32)


@pytest.mark.parametrize("per_key", [False, True])
def test_beta_zero_is_pure_decay(orc, per_key):
    rng = np.random.default_rng(1)
    H0 = rng.standard_normal((DK, DV))
    H = H0.copy()
    cum = np.ones(DK)
    for t in range(12):
        a = rng.uniform(0.6, 1.0, DK if per_key else 1).astype(np.float32)
        q = rng.standard_normal(DK).astype(np.float32)
        o = orc.step(H, q, _unit(rng, DK), rng.standard_normal(DV).astype(np.float32), a, 0.0, per_key)
        cum = cum * (a.astype(np.float64) if per_key else float(a[0]))
        expect_H = cum[:, None] * H0
        np.testing.assert_allclose(H, expect_H, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(o, expect_H.T @ q.astype(np.float64), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("per_key", [False, True])
def test_write_then_read_returns_v(orc, per_key):
    """beta = 1, |k| = 1: reading the new state with q = k returns v exactly,
    whatever the state and the decay (decay acts before the correction)."""
    rng = np.random.default_rng(2)
    H = rng.standard_normal((DK, DV)) * 3
    for t in range(20):
        k = _unit(rng, DK)
        v = rng.standard_normal(DV).astype(np.float32)
        a = rng.uniform(0.3, 1.0, DK if per_key else 1).astype(np.float32)
        o = orc.step(H, k, k, v, a, 1.0, per_key)
        # |k| = 1 only up to fp32 rounding of k: allow that much
        np.testing.assert_allclose(o, v, rtol=0, atol=2e-6 * (1 + np.abs(H).max()))


@pytest.mark.parametrize("per_key", [False, True])
def test_partial_beta_read(orc, per_key):
    """|k| = 1: H_t^T k = (1 - beta) (D H_{t-1})^T k + beta v."""
    rng = np.random.default_rng(3)
    H = rng.standard_normal((DK, DV))
    for t in range(10):
        k = _unit(rng, DK).astype(np.float64)
        kk = k / np.linalg.norm(k)          # exactly unit in fp64
        k32 = kk.astype(np.float32)
        kk = k32.astype(np.float64)
        nrm2 = kk @ kk
        v = rng.standard_normal(DV).astype(np.float32)
        a = rng.uniform(0.5, 1.0, DK if per_key else 1).astype(np.float32)
        beta = float(np.float32(rng.uniform(0.05, 0.95)))
        d = a.astype(np.float64) if per_key else np.full(DK, float(a[0]))
        before = (d[:, None] * H).T @ kk
        orc.step(H, k32, k32, v, a, beta, per_key)
        read = H.T @ kk
        expect = (1 - beta * nrm2) * before + beta * nrm2 * v.astype(np.float64)
        np.testing.assert_allclose(read, expect, rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_decayed_memory(orc):
    """beta = 1 with orthonormal keys from H0 = 0 stores
    H = sum_i (prod_{t>i} alpha_t) k_i v_i^T."""
    rng = np.random.default_rng(4)
    Q, _ = np.linalg.qr(rng.standard_normal((DK, DK)))
    keys = Q.T.astype(np.float32)                  # rows orthonormal (to fp32 rounding)
    H = np.zeros((DK, DV))
    vs, als = [], []
    for t in range(DK):
        v = rng.standard_normal(DV).astype(np.float32)
        a = np.float32(rng.uniform(0.7, 1.0))
        orc.step(H, keys[t], keys[t], v, np.array([a]), 1.0, False)
        vs.append(v.astype(np.float64))
        als.append(float(a))
    expect = np.zeros((DK, DV))
    for i in range(DK):
        expect += np.prod(als[i + 1:]) * np.outer(keys[i].astype(np.float64), vs[i])
    np.testing.assert_allclose(H, expect, atol=5e-6)


def test_one_hot_keys_make_a_table(orc):
    """alpha = beta = 1 and one-hot keys: each token overwrites row c_t."""
    rng = np.random.default_rng(5)
    H0 = rng.standard_normal((DK, DV))
    H = H0.copy()
    table = {i: H0[i].copy() for i in range(DK)}
    one = np.array([1.0], np.float32)
    for t in range(30):
        c = int(rng.integers(DK))
        k = np.zeros(DK, np.float32)
        k[c] = 1
        v = rng.standard_normal(DV).astype(np.float32)
        orc.step(H, k, k, v, one, 1.0, False)
        table[c] = v.astype(np.float64)
        want = np.stack([table[i] for i in range(DK)])
        others = np.arange(DK) != c
        np.testing.assert_array_equal(H[others], want[others])   # untouched rows
        np.testing.assert_allclose(H[c], want[c], rtol=0, atol=4e-16 * (1 + np.abs(want).max()))
        H[c] = want[c]                                             # keep the table exact


def test_kda_uniform_gate_equals_gdn(orc):
    rng = np.random.default_rng(6)
    H1 = rng.standard_normal((DK, DV))
    H2 = H1.copy()
    for t in range(15):
        q, k = _unit(rng, DK), _unit(rng, DK)
        v = rng.standard_normal(DV).astype(np.float32)
        a = np.float32(rng.uniform(0.8, 1.0))
        beta = rng.uniform(0, 1)
        o1 = orc.step(H1, q, k, v, np.array([a]), beta, False)
        o2 = orc.step(H2, q, k, v, np.full(DK, a, np.float32), beta, True)
        np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(H1, H2)


@pytest.mark.parametrize("per_key", [False, True])
def test_joint_linearity_in_state_and_values(orc, per_key):
    """For fixed (q, k, alpha, beta) the map (H0, v_1..v_T) -> (H_T, o_1..o_T)
    is linear: a dropped or spurious constant term breaks this."""
    rng = np.random.default_rng(7)
    T = 6
    ks = [_unit(rng, DK) for _ in range(T)]
    qs = [_unit(rng, DK) for _ in range(T)]
    als = [rng.uniform(0.5, 1, DK if per_key else 1).astype(np.float32) for _ in range(T)]
    bs = [float(np.float32(rng.uniform(0, 1))) for _ in range(T)]

    def run(H0, V):
        H = H0.copy()
        os_ = [orc.step(H, qs[t], ks[t], V[t], als[t], bs[t], per_key) for t in range(T)]
        return H, np.stack(os_)

    HA, HB = rng.standard_normal((DK, DV)), rng.standard_normal((DK, DV))
    # values restricted to small integers so that a + b is exact in fp32
    VA = rng.integers(-4, 5, (T, DV)).astype(np.float32)
    VB = rng.integers(-4, 5, (T, DV)).astype(np.float32)
    H1, o1 = run(HA, VA)
    H2, o2 = run(HB, VB)
    H3, o3 = run(HA + HB, VA + VB)
    np.testing.assert_allclose(H3, H1 + H2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o3, o1 + o2, rtol=1e-12, atol=1e-12)

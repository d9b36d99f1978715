"""Pins of the oracle's int8 codec (compensator rows, smoothing, rounding).

What fixes it, besides itself: the byte count the pages print (1.19 bytes per
value, 3.4x, ~70 %), exactness of the row extraction, a brute-force top-C
choice, the textbook per-row symmetric int8 quantizer of torch
(``torch.quantize_per_channel``) at C = 0 with smoothing off, the half-LSB
error bound of round-to-nearest, power-of-two scale invariance, an exact
integer round trip, permutation equivariance, and the pages' qualitative
claims that compensators and smoothing reduce the quantization error.
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _rand(rng, dk, dv, outlier_rows=(), outlier_cols=(), scale=1.0):
    H = rng.standard_normal((dk, dv)) * scale
    for r in outlier_rows:
        H[r] *= 40
    for c in outlier_cols:
        H[:, c] *= 25
    return H.astype(np.float32)


def test_page_byte_count(orc):
    g = json.load(open(GOLD))
    d = g["head_dim_assumed"]["value"]
    C = g["compensator_tokens"]["value"]
    bpv = orc.state_bytes(d, d, C) / (d * d)
    assert round(bpv, g["bytes_per_value"]["decimals"]) == g["bytes_per_value"]["value"]
    assert round(g["fp32_bytes_per_value"]["value"] / bpv, 1) == g["reduction_vs_fp32"]["value"]
    assert round(1 - bpv / 4, 1) == g["storage_cut_fraction"]["value"]
    assert orc.state_bytes(128, 128, 4) == 19472


def test_zero_state(orc):
    cd = orc.quantize(np.zeros((16, 16), np.float32), 3)
    assert not cd["sq"].any() and not cd["r"].any() and not cd["cv"].any()
    assert (cd["s"] == 1).all()
    assert list(cd["idx"]) == [0, 1, 2]


@pytest.mark.parametrize("C", [0, 1, 4, 8])
def test_extraction_is_exact(orc, C):
    rng = np.random.default_rng(10 + C)
    H = _rand(rng, 32, 24, outlier_rows=(3, 17, 30))
    cd = orc.quantize(H, C)
    m = np.abs(H).max(1)
    want = sorted(sorted(range(32), key=lambda i: (-m[i], i))[:C])
    assert list(cd["idx"]) == want
    for c, i in enumerate(cd["idx"]):
        assert cd["cv"][c].tobytes() == H[i].tobytes()     # bitwise copy
        assert not cd["sq"][i].any() and cd["r"][i] == 0
    D = orc.dequantize(cd)
    for i in cd["idx"]:
        assert (D[i] == H[i].astype(np.float64)).all()


@pytest.mark.parametrize("C", [0, 1, 2, 3, 4])
def test_top_c_bruteforce_with_ties(orc, C):
    rng = np.random.default_rng(20 + C)
    for trial in range(200):
        H = rng.integers(-3, 4, (4, 4)).astype(np.float32)   # many ties
        cd = orc.quantize(H, C)
        m = np.abs(H).max(1)
        ranked = sorted(range(4), key=lambda i: (-m[i], i))
        assert list(cd["idx"]) == sorted(ranked[:C])


def test_textbook_per_row_int8_matches_torch(orc):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(30)
    H = _rand(rng, 64, 48)
    cd = orc.quantize(H, 0, smooth=0)
    assert (cd["s"] == 1).all()
    amax = np.abs(H).max(1)
    # the scale is the row absmax over 127 (one fp32 division)
    np.testing.assert_array_equal(cd["r"], amax / np.float32(127))
    ref = torch.quantize_per_channel(torch.from_numpy(H), torch.from_numpy(cd["r"]).double(),
                                     torch.zeros(64, dtype=torch.long), 0,
                                     torch.qint8).int_repr().numpy()
    diff = np.abs(ref.astype(int) - cd["sq"].astype(int))
    assert diff.max() <= 1
    # torch divides by the scale, the codec multiplies by 127/rho: the two
    # products differ by an ulp or two, so they may round apart only where
    # the exact quotient lies within a few ulps of a half-integer
    x = H.astype(np.float64) / (amax.astype(np.float64)[:, None] / 127.0)
    near_tie = np.abs(np.abs(x - np.trunc(x)) - 0.5) < 1e-4
    assert not (diff > 0)[~near_tie].any()
    # the row maximum lands on +-127
    rows = np.arange(64)
    assert (np.abs(cd["sq"][rows, np.abs(H).argmax(1)]) == 127).all()


@pytest.mark.parametrize("smooth", [0, 1])
@pytest.mark.parametrize("C", [0, 4])
def test_half_lsb_error_bound(orc, smooth, C):
    rng = np.random.default_rng(40 + smooth + C)
    H = _rand(rng, 128, 128, outlier_rows=(5, 77), outlier_cols=(9, 100))
    cd = orc.quantize(H, C, smooth)
    D = orc.dequantize(cd)
    err = np.abs(D - H.astype(np.float64))
    lsb = cd["r"].astype(np.float64)[:, None] * cd["s"].astype(np.float64)[None, :]
    assert (err <= lsb * (0.5 + 1e-4) + 1e-30).all()
    assert np.abs(cd["sq"].astype(int)).max() <= 127


@pytest.mark.parametrize("smooth", [0, 1])
def test_power_of_two_invariance(orc, smooth):
    rng = np.random.default_rng(50)
    H = _rand(rng, 32, 16, outlier_rows=(2,), outlier_cols=(7,))
    H[:, 3] = 0                                   # a zero column keeps s = 1
    a = orc.quantize(H, 2, smooth)
    for e in (-7, 3, 11):
        b = orc.quantize(H * np.float32(2.0 ** e), 2, smooth)
        assert (a["sq"] == b["sq"]).all() and (a["idx"] == b["idx"]).all()
        np.testing.assert_array_equal(b["cv"], a["cv"] * np.float32(2.0 ** e))
        if smooth:
            assert (a["r"] == b["r"]).all()
            s_expect = a["s"] * np.float32(2.0 ** e)
            s_expect[3] = 1
            np.testing.assert_array_equal(b["s"], s_expect)
        else:
            np.testing.assert_array_equal(b["r"], a["r"] * np.float32(2.0 ** e))


@pytest.mark.parametrize("smooth", [0, 1])
def test_integer_matrix_round_trip(orc, smooth):
    rng = np.random.default_rng(60)
    n = 24
    M = rng.integers(-126, 127, (n, n))
    perm = rng.permutation(n)
    M[np.arange(n), perm] = 127 * rng.choice([-1, 1], n)   # +-127 in every row and column
    H = M.astype(np.float32)
    a = orc.quantize(H, 0, smooth)
    assert (a["sq"] == M).all()
    b = orc.quantize(orc.dequantize(a).astype(np.float32), 0, smooth)
    for key in ("sq", "r", "s"):
        assert (a[key] == b[key]).all()


def test_permutation_equivariance(orc):
    rng = np.random.default_rng(70)
    H = _rand(rng, 32, 20, outlier_rows=(4, 9), outlier_cols=(2,))
    pr, pc = rng.permutation(32), rng.permutation(20)
    a = orc.quantize(H, 3)
    b = orc.quantize(H[pr][:, pc], 3)
    inv = np.argsort(pr)
    assert sorted(pr[b["idx"]]) == sorted(a["idx"])
    assert (b["sq"] == a["sq"][pr][:, pc]).all()
    assert (b["r"] == a["r"][pr]).all() and (b["s"] == a["s"][pc]).all()
    # compensator rows carry the same values, permuted in their columns
    for c, i in enumerate(b["idx"]):
        j = list(a["idx"]).index(pr[i])
        assert (b["cv"][c] == a["cv"][j][pc]).all()
    assert inv.shape == (32,)


def test_compensators_and_smoothing_reduce_error(orc):
    """The pages' claims: holding the biggest outlier entries aside in high
    precision, and smoothing what is left, each lower the quantization error (forum mirror,
    'Abstract (translated)', techniques 2 and 3)."""
    rng = np.random.default_rng(80)
    H = _rand(rng, 128, 128, outlier_rows=(1, 20, 64, 90), outlier_cols=(3, 50))
    H64 = H.astype(np.float64)

    def mse(C, sm):
        return float(((orc.dequantize(orc.quantize(H, C, sm)) - H64) ** 2).mean())

    base, comp, both = mse(0, 0), mse(4, 0), mse(4, 1)
    assert comp < 0.5 * base
    assert both < comp


@pytest.mark.parametrize("smooth", [0, 1])
def test_tiny_magnitudes_stay_finite(orc, smooth):
    """Rows or columns below 2^-120 count as zero: every codec value stays
    finite and the reconstruction error of such a row is below 2^-120."""
    rng = np.random.default_rng(90)
    H = rng.standard_normal((32, 16)).astype(np.float32)
    H[3] *= np.float32(1e-38)                   # a row in the denormal range
    H[7] *= np.float32(2.0 ** -125)
    H[:, 5] *= np.float32(1e-39)                # a tiny column
    D = (rng.standard_normal((16, 16)) * 1e-39).astype(np.float32)   # all denormal
    for M in (H, D, np.full((8, 8), np.float32(2.0 ** -121))):
        cd = orc.quantize(M, 1, smooth)
        for key in ("r", "s", "cv"):
            assert np.isfinite(cd[key]).all()
        assert np.abs(cd["sq"].astype(int)).max() <= 127
        err = np.abs(orc.dequantize(cd) - M.astype(np.float64))
        lsb = cd["r"].astype(np.float64)[:, None] * cd["s"].astype(np.float64)[None, :]
        assert (err <= np.maximum(lsb * (0.5 + 1e-4), 2.0 ** -120)).all()


# Half-integer quotients: the row maximum is 127 (smoothing off), so the row
# multiplier 127/rho is exactly 1 and every entry below is its own quotient.
_TIES = np.array([127.0, 0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5, 62.5, 125.5, 126.5,
                  -126.5, 0.25, -0.75, 0.0], np.float32)
_TIES_HALF_EVEN = np.array([127, 0, 2, 2, 4, 0, -2, -2, -4, 62, 126, 126, -126, 0, -1, 0])


@pytest.mark.parametrize("C", [0, 1])
def test_exact_ties_round_half_to_even(orc, C):
    """The int8 rounding takes exact half-way quotients to the even integer
    (the reading that fixes the otherwise unstated rounding mode).  Rounding
    half away from zero would give 1, 3, 4, -1, ... on the second row."""
    H = np.stack([_TIES * np.float32(0.5), _TIES, -_TIES[::-1]])
    if C:
        H = np.concatenate([np.full((1, _TIES.size), 1000.0, np.float32), H])
    cd = orc.quantize(H, C, smooth=0)
    sq = cd["sq"][C:].astype(int)
    assert cd["r"][C:].tolist() == [0.5, 1.0, 1.0]
    # row 1 is _TIES itself: rho = 127, multiplier 1
    assert (sq[1] == _TIES_HALF_EVEN).all()
    assert (sq[2] == -_TIES_HALF_EVEN[::-1]).all()
    # row 0 is _TIES / 2: rho = 63.5, multiplier 2, quotients = _TIES again
    assert (sq[0] == _TIES_HALF_EVEN).all()


def test_exact_ties_match_torch_rounding(orc):
    """Library pin of the same rounding: torch's per-channel int8 quantizer at
    scale 1 rounds the exact half-way values identically."""
    torch = pytest.importorskip("torch")
    cd = orc.quantize(_TIES[None, :], 0, smooth=0)
    assert cd["r"][0] == np.float32(1.0)
    ref = torch.quantize_per_channel(torch.from_numpy(_TIES[None, :].copy()),
                                     torch.tensor([1.0], dtype=torch.double),
                                     torch.zeros(1, dtype=torch.long), 0, torch.qint8).int_repr().numpy()
    assert (cd["sq"].astype(int) == ref.astype(int)).all()


def test_exact_ties_with_smoothing(orc):
    """Exact ties survive smoothing when every column maximum is a power of
    two: row 0 holds 128 in every column (s_j = 128, an exact division), and
    a row whose largest entry is 127 gets rho = 127/128 and multiplier 128,
    so its quotients are its own entries again."""
    dv = _TIES.size
    H = np.stack([np.full(dv, 128.0, np.float32), _TIES])
    cd = orc.quantize(H, 0, smooth=1)
    assert (cd["s"] == np.float32(128.0)).all()
    assert (cd["sq"][1].astype(int) == _TIES_HALF_EVEN).all()


def test_smoothing_worked_example(orc):
    """A hand-worked 4 x 3 case of compensator extraction then smoothing.

        H = [[ 50, -60, 70  ],      row maxima 70, 2, 4, 2: C = 1 takes row 0
             [  1,  -2, 0.5 ],
             [ -4,   1, 0.25],
             [  2,   0, -1  ]]

    The smoothing factors are the column maxima of the residual (rows 1-3):
    s = [4, 2, 1], not the column maxima of H ([50, 60, 70]).  Then
    Y = R / s = [[.25, -1, .5], [-1, .5, .25], [.5, 0, -1]], each residual row
    has rho = 1 (r = 1/127) and sq = rint(127 Y): 31.75 -> 32, 63.5 -> 64."""
    H = np.array([[50, -60, 70], [1, -2, 0.5], [-4, 1, 0.25], [2, 0, -1]], np.float32)
    cd = orc.quantize(H, 1, smooth=1)
    assert list(cd["idx"]) == [0]
    assert cd["cv"][0].tolist() == [50, -60, 70]
    assert cd["s"].tolist() == [4.0, 2.0, 1.0]
    assert (cd["r"] == np.float32([0.0, 1 / 127, 1 / 127, 1 / 127])).all()
    assert cd["sq"].tolist() == [[0, 0, 0], [32, -127, 64], [-127, 64, 32], [64, 0, -127]]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_smoothing_reaches_full_range_in_every_residual_column(orc, seed):
    """Smoothing by the residual's column maxima puts a value of magnitude
    (about) 1 in every nonzero residual column, in a row whose own maximum it
    then is, so every such column holds a byte of magnitude 127.  The outlier
    rows carry every column's maximum of H here: had the factors come from H,
    the residual columns would reach only about 127/40."""
    rng = np.random.default_rng(300 + seed)
    H = _rand(rng, 64, 48)
    rows = rng.choice(64, 4, replace=False)
    H[rows] = (rng.choice([-1, 1], (4, 48)) * 40 * np.abs(H).max()).astype(np.float32)
    cd = orc.quantize(H, 4, smooth=1)
    assert sorted(cd["idx"]) == sorted(rows)
    keep = np.setdiff1d(np.arange(64), rows)
    colmax = np.abs(H[keep]).max(0)
    assert (cd["s"] == colmax).all()
    assert (np.abs(cd["sq"][keep].astype(int)).max(0) == 127).all()

"""Host-only checks of the C ABI library (no GPU needed, no kernel launched).

The library must load, export every function include/lq.h declares, and
reject bad arguments with the documented status before any HIP call.
"""
import ctypes as ct
import os
import re

import pytest

from recurrent_state_quant_lq_amd import lq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(lq.LIB_PATH), reason="liblq.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lq_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(lq.EXPORTS)


def test_every_declared_symbol_is_exported():
    L = ct.CDLL(lq.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name


def _dims(**kw):
    base = dict(B=2, H=3, dk=128, dv=128, W=16, C=4, decay_mode=0, smooth=1, io_dtype=0)
    base.update(kw)
    return lq.lq_dims(*[base[n] for n in ("B", "H", "dk", "dv", "W", "C", "decay_mode", "smooth",
                                          "io_dtype")])


def test_sizes():
    L = lq.load()
    d = _dims()
    assert L.lq_state_bytes(ct.byref(d)) == 6 * 19472
    # per slot: k (dk) + m (dv) + one log-decay (scalar) or dk of them (per key)
    assert L.lq_buffer_bytes(ct.byref(d)) == 6 * 16 * 4 * (128 + 128 + 1)
    dk = _dims(decay_mode=1)
    assert L.lq_buffer_bytes(ct.byref(dk)) == 6 * 16 * 4 * (3 * 128)
    assert L.lq_state_bytes(None) == 0
    assert L.lq_state_bytes(ct.byref(_dims(dk=0))) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(), lq.LQ_OK),
    (dict(B=0), lq.LQ_ERR_DIMS), (dict(H=-1), lq.LQ_ERR_DIMS), (dict(W=0), lq.LQ_ERR_DIMS),
    (dict(C=-1), lq.LQ_ERR_DIMS), (dict(dk=16, dv=16, C=17), lq.LQ_ERR_DIMS),
    (dict(decay_mode=2), lq.LQ_ERR_DIMS), (dict(smooth=3), lq.LQ_ERR_DIMS),
    (dict(io_dtype=2), lq.LQ_ERR_DIMS), (dict(io_dtype=-1), lq.LQ_ERR_DIMS), (dict(io_dtype=1), lq.LQ_OK),
    (dict(dk=96, dv=96), lq.LQ_ERR_UNSUPPORTED), (dict(dk=128, dv=64), lq.LQ_ERR_UNSUPPORTED),
    (dict(W=33), lq.LQ_ERR_UNSUPPORTED), (dict(C=9), lq.LQ_ERR_UNSUPPORTED),
    (dict(dk=16, dv=16, W=4, C=1), lq.LQ_OK), (dict(dk=64, dv=64, W=32, C=8), lq.LQ_OK),
])
def test_check_dims(kw, status):
    assert lq.load().lq_check_dims(ct.byref(_dims(**kw))) == status


def _fake_state(C=4, misalign=None, null=None):
    names = ("sq", "row_scale", "col_scale", "comp_idx", "comp_val", "buf_k", "buf_m", "buf_g")
    vals = []
    for i, n in enumerate(names):
        p = 0x100000 * (i + 1)
        if n == misalign:
            p += 4
        if n == null:
            p = None
        vals.append(p)
    return lq.lq_state(*vals)


A = ct.c_void_p(0x7000000)      # an aligned address that is never dereferenced
B4 = ct.c_void_p(0x7000004)


def test_decode_argument_errors():
    L = lq.load()
    d = _dims()
    st = _fake_state()
    call = lambda dd, s, pos, *p: L.lq_gdn_decode_step(dd, s, pos, *p, None)
    args = (A, A, A, A, A, A)
    assert call(None, ct.byref(st), 0, *args) == lq.LQ_ERR_NULL
    assert call(ct.byref(d), None, 0, *args) == lq.LQ_ERR_NULL
    assert call(ct.byref(d), ct.byref(st), 16, *args) == lq.LQ_ERR_WINDOW_FULL
    assert call(ct.byref(d), ct.byref(st), 99, *args) == lq.LQ_ERR_WINDOW_FULL
    assert call(ct.byref(d), ct.byref(st), -1, *args) == lq.LQ_ERR_POS
    assert call(ct.byref(d), ct.byref(st), 0, A, A, None, A, A, A) == lq.LQ_ERR_NULL
    assert call(ct.byref(d), ct.byref(st), 0, A, B4, A, A, A, A) == lq.LQ_ERR_ALIGN
    for n in ("sq", "buf_m", "comp_val"):
        assert call(ct.byref(d), ct.byref(_fake_state(null=n)), 0, *args) == lq.LQ_ERR_NULL
        assert call(ct.byref(d), ct.byref(_fake_state(misalign=n)), 0, *args) == lq.LQ_ERR_ALIGN
    # beta and the scalar-mode alpha need only 4-byte alignment
    assert call(ct.byref(d), ct.byref(st), 16, A, A, A, B4, B4, A) == lq.LQ_ERR_WINDOW_FULL
    assert call(ct.byref(_dims(decay_mode=1)), ct.byref(st), 16, A, A, A, B4, A, A) == lq.LQ_ERR_ALIGN
    assert call(ct.byref(d), ct.byref(st), 16, A, A, A, A, ct.c_void_p(0x7000002), A) == lq.LQ_ERR_ALIGN
    # C = 0 does not need compensator arrays
    d0 = _dims(C=0)
    st0 = _fake_state(null="comp_idx")
    assert call(ct.byref(d0), ct.byref(st0), 16, *args) == lq.LQ_ERR_WINDOW_FULL
    assert call(ct.byref(_dims(dk=96, dv=96)), ct.byref(st), 0, *args) == lq.LQ_ERR_UNSUPPORTED


def test_flush_and_codec_argument_errors():
    L = lq.load()
    d = _dims()
    st = _fake_state()
    assert L.lq_gdn_window_flush(ct.byref(d), ct.byref(st), -1, None, None) == lq.LQ_ERR_POS
    assert L.lq_gdn_window_flush(ct.byref(d), ct.byref(st), 17, None, None) == lq.LQ_ERR_POS
    assert L.lq_gdn_window_flush(ct.byref(d), ct.byref(st), 0, None, None) == lq.LQ_OK  # no-op
    assert L.lq_gdn_window_flush(ct.byref(d), ct.byref(st), 3, B4, None) == lq.LQ_ERR_ALIGN
    assert L.lq_gdn_window_flush(ct.byref(d), ct.byref(_fake_state(null="buf_g")), 3, None,
                                 None) == lq.LQ_ERR_NULL
    assert L.lq_gdn_state_quantize(ct.byref(d), None, ct.byref(st), None) == lq.LQ_ERR_NULL
    assert L.lq_gdn_state_quantize(ct.byref(d), B4, ct.byref(st), None) == lq.LQ_ERR_ALIGN
    assert L.lq_gdn_state_dequantize(ct.byref(d), ct.byref(st), None, None) == lq.LQ_ERR_NULL
    # the codec calls do not need the window buffer
    stq = _fake_state(null="buf_k")
    assert L.lq_gdn_state_quantize(ct.byref(_dims(B=0)), A, ct.byref(stq), None) == lq.LQ_ERR_DIMS
    assert L.lq_gdn_fp32_recurrence(ct.byref(d), A, -1, A, A, A, A, A, None, None) == lq.LQ_ERR_POS
    assert L.lq_gdn_fp32_recurrence(ct.byref(d), A, 0, A, A, A, A, A, None, None) == lq.LQ_OK
    assert L.lq_gdn_fp32_recurrence(ct.byref(d), A, 4, A, A, A, A, A, B4, None) == lq.LQ_ERR_ALIGN


def test_status_strings():
    L = lq.load()
    for s in range(8):
        assert L.lq_status_str(s)
    assert L.lq_status_str(1234) == b"unknown status"
    assert L.lq_last_hip_error() == 0


def test_timing_hook_host_side():
    """Recording on/off and collecting with no launches touch no GPU."""
    L = ct.CDLL(lq.LIB_PATH)
    L.lq_timing_collect.argtypes = [ct.c_int32, ct.c_void_p, ct.c_void_p, ct.c_void_p]
    n = ct.c_int32(-1)
    assert L.lq_timing_enable(1) == lq.LQ_OK
    assert L.lq_timing_collect(0, None, None, ct.byref(n)) == lq.LQ_OK
    assert n.value == 0
    assert L.lq_timing_collect(4, None, None, ct.byref(n)) == lq.LQ_ERR_NULL
    assert L.lq_timing_collect(0, None, None, None) == lq.LQ_ERR_NULL
    assert L.lq_timing_enable(0) == lq.LQ_OK


def test_ragged_argument_errors():
    L = lq.load()
    d = _dims()
    st = _fake_state()
    L.lq_gdn_decode_step_ragged.argtypes = [ct.c_void_p] * 10
    L.lq_gdn_window_flush_ragged.argtypes = [ct.c_void_p] * 5
    args = (A, A, A, A, A, A)
    dec = lambda dd, s, p, *a: L.lq_gdn_decode_step_ragged(dd, s, p, *a, None)
    assert dec(ct.byref(d), ct.byref(st), None, *args) == lq.LQ_ERR_NULL
    assert dec(ct.byref(d), ct.byref(st), ct.c_void_p(0x7000002), *args) == lq.LQ_ERR_ALIGN
    assert dec(None, ct.byref(st), A, *args) == lq.LQ_ERR_NULL
    assert dec(ct.byref(_dims(dk=96, dv=96)), ct.byref(st), A, *args) == lq.LQ_ERR_UNSUPPORTED
    fl = lambda dd, s, n, h: L.lq_gdn_window_flush_ragged(dd, s, n, h, None)
    assert fl(ct.byref(d), ct.byref(st), None, None) == lq.LQ_ERR_NULL
    assert fl(ct.byref(d), ct.byref(st), ct.c_void_p(0x7000001), None) == lq.LQ_ERR_ALIGN
    assert fl(ct.byref(d), ct.byref(st), A, B4) == lq.LQ_ERR_ALIGN
    assert fl(ct.byref(d), ct.byref(_fake_state(null="buf_k")), A, None) == lq.LQ_ERR_NULL


def test_decode_flush_argument_errors():
    L = lq.load()
    d = _dims()
    st = _fake_state()
    call = lambda dd, s, pos, *p: L.lq_gdn_decode_step_flush(dd, s, pos, *p, None)
    args = (A, A, A, A, A, A)
    assert call(None, ct.byref(st), 0, *args, None) == lq.LQ_ERR_NULL
    assert call(ct.byref(d), ct.byref(st), 16, *args, None) == lq.LQ_ERR_WINDOW_FULL
    assert call(ct.byref(d), ct.byref(st), -1, *args, None) == lq.LQ_ERR_POS
    assert call(ct.byref(d), ct.byref(st), 15, A, A, A, A, A, None, None) == lq.LQ_ERR_NULL   # o
    assert call(ct.byref(d), ct.byref(st), 15, *args, B4) == lq.LQ_ERR_ALIGN                  # h_out
    assert call(ct.byref(d), ct.byref(_fake_state(null="buf_m")), 15, *args, None) == lq.LQ_ERR_NULL
    assert call(ct.byref(_dims(dk=96, dv=96)), ct.byref(st), 0, *args, None) == lq.LQ_ERR_UNSUPPORTED


def test_decode_flush_ragged_argument_errors():
    L = lq.load()
    d = _dims()
    st = _fake_state()
    L.lq_gdn_decode_step_flush_ragged.argtypes = [ct.c_void_p] * 11
    call = lambda dd, s, p, *a: L.lq_gdn_decode_step_flush_ragged(dd, s, p, *a, None)
    args = (A, A, A, A, A, A, None)
    assert call(ct.byref(d), ct.byref(st), None, *args) == lq.LQ_ERR_NULL
    assert call(ct.byref(d), ct.byref(st), ct.c_void_p(0x7000002), *args) == lq.LQ_ERR_ALIGN
    assert call(ct.byref(d), ct.byref(st), A, A, A, A, A, A, A, B4) == lq.LQ_ERR_ALIGN       # h_out
    assert call(ct.byref(d), ct.byref(_fake_state(null="buf_g")), A, *args) == lq.LQ_ERR_NULL
    assert call(ct.byref(_dims(dk=96, dv=96)), ct.byref(st), A, *args) == lq.LQ_ERR_UNSUPPORTED


def test_prefill_argument_errors():
    L = lq.load()
    d = _dims()
    st = _fake_state()
    call = lambda dd, s, h, T, *p: L.lq_gdn_prefill(dd, s, h, T, *p, None)
    args = (A, A, A, A, A, None)
    assert call(None, ct.byref(st), A, 4, *args) == lq.LQ_ERR_NULL
    assert call(ct.byref(d), ct.byref(st), None, 4, *args) == lq.LQ_ERR_NULL
    assert call(ct.byref(d), ct.byref(st), B4, 4, *args) == lq.LQ_ERR_ALIGN
    assert call(ct.byref(d), ct.byref(st), A, -1, *args) == lq.LQ_ERR_POS
    assert call(ct.byref(d), ct.byref(st), A, 4, A, None, A, A, A, None) == lq.LQ_ERR_NULL
    assert call(ct.byref(d), ct.byref(st), A, 4, A, A, A, A, A, B4) == lq.LQ_ERR_ALIGN          # o
    assert call(ct.byref(d), ct.byref(_fake_state(null="sq")), A, 4, *args) == lq.LQ_ERR_NULL
    assert call(ct.byref(d), None, A, 0, *args) == lq.LQ_OK             # nothing to do
    assert call(ct.byref(_dims(dk=96, dv=96)), ct.byref(st), A, 4, *args) == lq.LQ_ERR_UNSUPPORTED


def test_checkpoint_sizes_and_errors():
    L = lq.load()
    d = _dims()                                   # B=2 H=3 d=128 C=4
    assert lq.lq_checkpoint_bytes(d) == 6 * 19472 == L.lq_state_bytes(ct.byref(d))
    d1 = _dims(C=1)                               # 17,924 bytes padded to 17,936
    assert lq.lq_checkpoint_bytes(d1) == 6 * 17936
    assert lq.lq_checkpoint_bytes(_dims(dk=96, dv=96)) == 0
    st = _fake_state()
    assert L.lq_gdn_state_pack(ct.byref(d), ct.byref(st), None, None) == lq.LQ_ERR_NULL
    assert L.lq_gdn_state_pack(ct.byref(d), ct.byref(st), ct.c_void_p(0x7000004), None) == lq.LQ_ERR_ALIGN
    assert L.lq_gdn_state_unpack(ct.byref(d), A, ct.byref(_fake_state(null="sq")), None) == lq.LQ_ERR_NULL
    assert L.lq_gdn_state_unpack(None, A, ct.byref(st), None) == lq.LQ_ERR_NULL


@pytest.mark.parametrize("dk", [16, 64, 128])
def test_state_storage_order(dk):
    """The stored order of a head's int8 state (include/lq.h): a bijection of
    the dk*dv bytes; byte (i, j) at the position the header's formula gives,
    spelled out here digit by digit; 16-channel runs of a column contiguous;
    value-column-major at dk = 16; row-major round trip through the binding."""
    import numpy as np
    off = lq.sq_order(dk)
    assert off.shape == (dk, dk)
    assert np.array_equal(np.sort(off.ravel()), np.arange(dk * dk))
    G, KS = min(4, dk // 16), (dk + 63) // 64
    for i in range(0, dk, 7):
        for j in range(0, dk, 5):
            tile, jj, ks, lg, e = j // 16, j % 16, i // 64, (i % 64) // 16, i % 16
            assert off[i, j] == (((tile * KS + ks) * G + lg) * 16 + jj) * 16 + e
    # a run of 16 channels of one column is 16 consecutive bytes
    runs = off.T.reshape(dk, dk // 16, 16)
    assert (np.diff(runs, axis=-1) == 1).all()
    if dk == 16:
        assert np.array_equal(off, np.arange(dk)[:, None] + dk * np.arange(dk)[None, :])
    rng = np.random.default_rng(dk)
    rows = rng.integers(-127, 128, size=(2, 3, dk, dk), dtype=np.int8)
    stored = lq.sq_from_rows(rows)
    assert stored.shape == (2, 3, dk * dk)
    assert np.array_equal(lq.sq_to_rows(stored, dk), rows)
    assert stored[1, 2, off[5, 3]] == rows[1, 2, 5, 3]


def test_measure_stream_read_argument_errors():
    L = lq.load()
    f = L.lq_measure_stream_read
    src, sink = 0x100000, 0x200000
    assert f(None, 1024, 4, 0, 0, sink, 16, None) == lq.LQ_ERR_NULL
    assert f(src, 1024, 4, 0, 0, None, 16, None) == lq.LQ_ERR_NULL
    assert f(src + 4, 1024, 4, 0, 0, sink, 16, None) == lq.LQ_ERR_ALIGN
    assert f(src, 1024, 4, 0, 0, sink + 8, 16, None) == lq.LQ_ERR_ALIGN
    for bad in (0, 8, 1000, 65552):
        assert f(src, bad, 4, 0, 0, sink, 16, None) == lq.LQ_ERR_DIMS
    assert f(src, 1024, 0, 0, 0, sink, 16, None) == lq.LQ_ERR_DIMS
    assert f(src, 1024, 4, 2, 0, sink, 16, None) == lq.LQ_ERR_DIMS
    assert f(src, 1024, 4, 1, 0, sink, 16, None) == lq.LQ_ERR_DIMS
    assert f(src, 1024, 4, 0, 0, sink, 4112, None) == lq.LQ_ERR_DIMS
    assert f(src, 1024, 4, 0, 0, sink, 24, None) == lq.LQ_ERR_DIMS


def test_layer_state_rows_are_views():
    """LayerState.rows: rows b0..b1-1 as a state of their own, sharing memory."""
    d = lq.make_dims(6, 2, 16, 16, 4, 1, lq.LQ_DECAY_PER_KEY, 1)
    st = lq.LayerState.allocate(d, "cpu")
    part = st.rows(2, 5)
    assert part.dims.B == 3 and st.dims.B == 6
    assert (part.dims.H, part.dims.dk, part.dims.W, part.dims.C) == (2, 16, 4, 1)
    for f in ("sq", "row_scale", "col_scale", "comp_idx", "comp_val", "buf_k", "buf_m", "buf_g"):
        whole, view = getattr(st, f), getattr(part, f)
        assert view.shape[0] == 3 and view.shape[1:] == whole.shape[1:]
        assert view.is_contiguous()
        assert view.data_ptr() == whole[2].data_ptr()
    part.row_scale.fill_(7.0)
    assert float(st.row_scale[2:5].min()) == 7.0 and float(st.row_scale[:2].abs().max()) == 0.0
    for b0, b1 in ((0, 0), (3, 2), (-1, 2), (0, 7)):
        with pytest.raises(ValueError):
            st.rows(b0, b1)

"""Thin ctypes binding of liblq.so (C ABI declared in include/lq.h).

The functions carry the C names and only marshal arguments: torch device
tensors become device pointers, the current torch stream becomes the HIP
stream.  Before each call the binding checks dtype, device, contiguity and
shape of every tensor against the lq_dims, because the C ABI sees only
pointers.  Every step of the computation runs in the HIP kernels; if the
library is missing, loading fails loudly (there is no fallback).
"""
from __future__ import annotations

import ctypes as ct
import os
from dataclasses import dataclass

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# LQ_LIB may name another build of the same sources (the host-sanitizer build)
LIB_PATH = os.environ.get("LQ_LIB") or os.path.join(_PKG, "liblq.so")

LQ_OK, LQ_ERR_NULL, LQ_ERR_DIMS, LQ_ERR_UNSUPPORTED, LQ_ERR_WINDOW_FULL, LQ_ERR_POS, \
    LQ_ERR_ALIGN, LQ_ERR_HIP = range(8)
LQ_DECAY_SCALAR, LQ_DECAY_PER_KEY = 0, 1
LQ_IO_F32, LQ_IO_BF16 = 0, 1

# every symbol include/lq.h declares
EXPORTS = ("lq_gdn_decode_step", "lq_gdn_window_flush", "lq_gdn_decode_step_ragged",
           "lq_gdn_window_flush_ragged", "lq_gdn_state_quantize",
           "lq_gdn_state_dequantize", "lq_gdn_fp32_recurrence", "lq_state_bytes",
           "lq_buffer_bytes", "lq_status_str", "lq_last_hip_error", "lq_check_dims",
           "lq_timing_enable", "lq_timing_collect", "lq_checkpoint_bytes", "lq_gdn_state_pack",
           "lq_gdn_state_unpack", "lq_gdn_decode_step_flush", "lq_gdn_prefill",
           "lq_gdn_decode_step_flush_ragged", "lq_measure_stream_read")
LQ_KERNEL_DECODE, LQ_KERNEL_FLUSH, LQ_KERNEL_QUANTIZE, LQ_KERNEL_DEQUANTIZE, \
    LQ_KERNEL_FP32_RECURRENCE, LQ_KERNEL_CHECKPOINT, LQ_KERNEL_DECODE_FLUSH, \
    LQ_KERNEL_PREFILL, LQ_KERNEL_MEASURE = range(9)


class lq_dims(ct.Structure):
    _fields_ = [(n, ct.c_int32) for n in ("B", "H", "dk", "dv", "W", "C", "decay_mode", "smooth",
                                          "io_dtype")]


class lq_state(ct.Structure):
    _fields_ = [(n, ct.c_void_p) for n in ("sq", "row_scale", "col_scale", "comp_idx", "comp_val",
                                           "buf_k", "buf_m", "buf_g")]


class LQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib.lq_status_str(status).decode() if _lib is not None else str(status)
        extra = f" (hipError {_lib.lq_last_hip_error()})" if status == LQ_ERR_HIP else ""
        super().__init__(f"{fn}: {msg}{extra} [status {status}]")


_lib = None


def load() -> ct.CDLL:
    """Loads liblq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m recurrent_state_quant_lq_amd.build`")
        L = ct.CDLL(LIB_PATH)
        D, S, P, I = ct.POINTER(lq_dims), ct.POINTER(lq_state), ct.c_void_p, ct.c_int32
        L.lq_gdn_decode_step.argtypes = [D, S, I, P, P, P, P, P, P, P]
        L.lq_gdn_window_flush.argtypes = [D, S, I, P, P]
        L.lq_gdn_decode_step_flush.argtypes = [D, S, I, P, P, P, P, P, P, P, P]
        L.lq_gdn_prefill.argtypes = [D, S, P, I, P, P, P, P, P, P, P]
        L.lq_gdn_decode_step_flush_ragged.argtypes = [D, S, P, P, P, P, P, P, P, P, P]
        L.lq_gdn_decode_step_ragged.argtypes = [D, S, P, P, P, P, P, P, P, P]
        L.lq_gdn_window_flush_ragged.argtypes = [D, S, P, P, P]
        L.lq_gdn_state_quantize.argtypes = [D, P, S, P]
        L.lq_gdn_state_dequantize.argtypes = [D, S, P, P]
        L.lq_gdn_fp32_recurrence.argtypes = [D, P, I, P, P, P, P, P, P, P]
        for f in ("lq_gdn_decode_step", "lq_gdn_window_flush", "lq_gdn_decode_step_flush", "lq_gdn_prefill",
                  "lq_gdn_decode_step_flush_ragged", "lq_gdn_decode_step_ragged",
                  "lq_gdn_window_flush_ragged", "lq_gdn_state_quantize",
                  "lq_gdn_state_dequantize", "lq_gdn_fp32_recurrence", "lq_check_dims",
                  "lq_last_hip_error"):
            getattr(L, f).restype = ct.c_int
        L.lq_check_dims.argtypes = [D]
        L.lq_state_bytes.argtypes = [D]
        L.lq_state_bytes.restype = ct.c_size_t
        L.lq_buffer_bytes.argtypes = [D]
        L.lq_buffer_bytes.restype = ct.c_size_t
        L.lq_status_str.argtypes = [ct.c_int]
        L.lq_status_str.restype = ct.c_char_p
        L.lq_last_hip_error.argtypes = []
        L.lq_checkpoint_bytes.argtypes = [D]
        L.lq_checkpoint_bytes.restype = ct.c_size_t
        L.lq_gdn_state_pack.argtypes = [D, S, P, P]
        L.lq_gdn_state_pack.restype = ct.c_int
        L.lq_gdn_state_unpack.argtypes = [D, P, S, P]
        L.lq_gdn_state_unpack.restype = ct.c_int
        L.lq_measure_stream_read.argtypes = [P, ct.c_size_t, I, I, I, P, ct.c_size_t, P]
        L.lq_measure_stream_read.restype = ct.c_int
        L.lq_timing_enable.argtypes = [ct.c_int32]
        L.lq_timing_enable.restype = ct.c_int
        L.lq_timing_collect.argtypes = [ct.c_int32, ct.POINTER(ct.c_int32), ct.POINTER(ct.c_float),
                                        ct.POINTER(ct.c_int32)]
        L.lq_timing_collect.restype = ct.c_int
        _lib = L
    return _lib


def make_dims(B, H, dk, dv, W, C, decay_mode=LQ_DECAY_SCALAR, smooth=1, io_dtype=LQ_IO_F32) -> lq_dims:
    return lq_dims(B, H, dk, dv, W, C, decay_mode, smooth, io_dtype)


def io_torch_dtype(d: lq_dims):
    """torch dtype of the token vectors q, k, v and outputs o for these dims."""
    return torch.bfloat16 if d.io_dtype == LQ_IO_BF16 else torch.float32


def _dtype_of(d: lq_dims, name: str):
    return io_torch_dtype(d) if name in ("q", "k", "v", "o") else torch.float32


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ct.c_void_p(stream.cuda_stream)


def _check(t: torch.Tensor, name: str, shape, dtype):
    # one fast test of the usual case; the detailed messages below otherwise
    if t is not None and t.dtype == dtype and t.shape == shape and t.is_cuda and t.is_contiguous():
        return
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _raise(fn, rc):
    if rc != LQ_OK:
        raise LQError(fn, rc)


_STATE_FIELDS = ("sq", "row_scale", "col_scale", "comp_idx", "comp_val", "buf_k", "buf_m", "buf_g")

_SQ_ORDER: dict = {}


def sq_order(dk: int) -> np.ndarray:
    """off[i, j]: where byte (i, j) of a head's int8 state (key channel i,
    value channel j) sits in the head's dk*dv stored bytes (the operand order
    of the int8 matrix cores, as include/lq.h states it)."""
    off = _SQ_ORDER.get(dk)
    if off is None:
        i = np.arange(dk, dtype=np.int64)[:, None]
        j = np.arange(dk, dtype=np.int64)[None, :]
        G, KS = min(4, dk // 16), (dk + 63) // 64
        off = ((((j >> 4) * KS + (i >> 6)) * G + ((i & 63) >> 4)) * 16 + (j & 15)) * 16 + (i & 15)
        off.setflags(write=False)
        _SQ_ORDER[dk] = off
    return off


def sq_to_rows(sq: np.ndarray, dk: int) -> np.ndarray:
    """Stored int8 state [..., dk*dv] -> row-major [..., dk, dv]."""
    return np.ascontiguousarray(np.asarray(sq)[..., sq_order(dk)])


def sq_from_rows(rows: np.ndarray) -> np.ndarray:
    """Row-major int8 state [..., dk, dv] -> stored order [..., dk*dv]."""
    rows = np.asarray(rows)
    dk = rows.shape[-2]
    out = np.empty(rows.shape[:-2] + (rows.shape[-2] * rows.shape[-1],), dtype=rows.dtype)
    out[..., sq_order(dk).ravel()] = rows.reshape(out.shape)
    return out


@dataclass
class LayerState:
    """Device tensors of one layer's codec and window buffer (torch-owned).
    ``sq`` is [B,H,dk*dv], each head's bytes in the library's stored order
    (sq_order; sq_to_rows / sq_from_rows convert)."""
    dims: lq_dims
    sq: torch.Tensor
    row_scale: torch.Tensor
    col_scale: torch.Tensor
    comp_idx: torch.Tensor
    comp_val: torch.Tensor
    buf_k: torch.Tensor
    buf_m: torch.Tensor
    buf_g: torch.Tensor

    @staticmethod
    def allocate(d: lq_dims, device="cuda") -> "LayerState":
        B, H, dk, dv, W, C = d.B, d.H, d.dk, d.dv, d.W, d.C
        gd = dk if d.decay_mode == LQ_DECAY_PER_KEY else 1
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
        return LayerState(d, z((B, H, dk * dv), torch.int8), z((B, H, dk), torch.float32),
                          z((B, H, dv), torch.float32), z((B, H, max(C, 1)), torch.int32),
                          z((B, H, max(C, 1), dv), torch.float32),
                          z((B, H, W, dk), torch.float32), z((B, H, W, dv), torch.float32),
                          z((B, H, W, gd), torch.float32))

    def check(self, with_buffer=True):
        d = self.dims
        B, H, dk, dv, W, C = d.B, d.H, d.dk, d.dv, d.W, d.C
        gd = dk if d.decay_mode == LQ_DECAY_PER_KEY else 1
        _check(self.sq, "sq", (B, H, dk * dv), torch.int8)
        _check(self.row_scale, "row_scale", (B, H, dk), torch.float32)
        _check(self.col_scale, "col_scale", (B, H, dv), torch.float32)
        _check(self.comp_idx, "comp_idx", (B, H, max(C, 1)), torch.int32)
        _check(self.comp_val, "comp_val", (B, H, max(C, 1), dv), torch.float32)
        if with_buffer:
            _check(self.buf_k, "buf_k", (B, H, W, dk), torch.float32)
            _check(self.buf_m, "buf_m", (B, H, W, dv), torch.float32)
            _check(self.buf_g, "buf_g", (B, H, W, gd), torch.float32)

    def c_state(self) -> lq_state:
        return lq_state(*[_ptr(getattr(self, n)) for n in _STATE_FIELDS])

    def rows(self, b0: int, b1: int) -> "LayerState":
        """Batch rows b0 .. b1-1 as a state of their own: views of the same device
        memory (no copy) with B = b1 - b0, so that parts of a batch can run as
        separate calls, e.g. as independent chains on separate streams."""
        d = lq_dims.from_buffer_copy(self.dims)
        if not (0 <= b0 < b1 <= d.B):
            raise ValueError(f"rows {b0}..{b1} outside the batch of {d.B}")
        d.B = b1 - b0
        return LayerState(d, *[getattr(self, n)[b0:b1] for n in _STATE_FIELDS])

    def ready(self, with_buffer=True) -> lq_state:
        """The C struct of this state, validated (shapes, dtypes, device) once
        for the tensors the fields hold; a field replaced by another tensor is
        validated again.  In-place writes to the tensors need no revalidation."""
        key = (tuple(id(getattr(self, n)) for n in _STATE_FIELDS), with_buffer)
        c = self.__dict__.get("_ready")
        if c is None or c[0] != key:
            self.check(with_buffer)
            c = (key, self.c_state())
            self.__dict__["_ready"] = c
        return c[1]

    def codec(self) -> dict:
        """Host copies of the codec arrays, int8 matrix row-major [B,H,dk,dv]
        (comp arrays cut to C)."""
        C = self.dims.C
        return dict(sq=sq_to_rows(self.sq.cpu().numpy(), self.dims.dk),
                    r=self.row_scale.cpu().numpy(),
                    s=self.col_scale.cpu().numpy(), idx=self.comp_idx[..., :C].cpu().numpy(),
                    cv=self.comp_val[..., :C, :].cpu().numpy())

    def load_codec(self, cd: dict):
        """Uploads host codec arrays ([B,H,...], int8 matrix row-major
        [B,H,dk,dv], comp arrays with C entries)."""
        C = self.dims.C
        self.sq.copy_(torch.from_numpy(sq_from_rows(cd["sq"])))
        self.row_scale.copy_(torch.as_tensor(cd["r"]))
        self.col_scale.copy_(torch.as_tensor(cd["s"]))
        if C:
            self.comp_idx[..., :C].copy_(torch.as_tensor(cd["idx"]))
            self.comp_val[..., :C, :].copy_(torch.as_tensor(cd["cv"]))


_SHAPES: dict = {}


def _token_shapes(d: lq_dims, T=None):
    key = (d.B, d.H, d.dk, d.dv, d.decay_mode, T)
    sh = _SHAPES.get(key)
    if sh is None:
        pre = (d.B, d.H) if T is None else (T, d.B, d.H)
        ash = pre + ((d.dk,) if d.decay_mode == LQ_DECAY_PER_KEY else ())
        sh = {k: torch.Size(v) for k, v in dict(q=pre + (d.dk,), k=pre + (d.dk,), v=pre + (d.dv,),
                                                alpha=ash, beta=pre, o=pre + (d.dv,)).items()}
        _SHAPES[key] = sh
    return sh


def lq_gdn_decode_step(st: LayerState, pos: int, q, k, v, alpha, beta, o, stream=None):
    d = st.dims
    sh = _token_shapes(d)
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta), ("o", o)):
        _check(t, name, sh[name], _dtype_of(d, name))
    cs = st.ready()
    rc = load().lq_gdn_decode_step(ct.byref(d), ct.byref(cs), int(pos), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(alpha), _ptr(beta), _ptr(o), _stream(stream))
    _raise("lq_gdn_decode_step", rc)


def lq_gdn_window_flush(st: LayerState, n_buffered: int, h_out=None, stream=None):
    d = st.dims
    if h_out is not None:
        _check(h_out, "h_out", (d.B, d.H, d.dk, d.dv), torch.float32)
    cs = st.ready()
    rc = load().lq_gdn_window_flush(ct.byref(d), ct.byref(cs), int(n_buffered), _ptr(h_out),
                                    _stream(stream))
    _raise("lq_gdn_window_flush", rc)


def lq_gdn_decode_step_flush(st: LayerState, pos: int, q, k, v, alpha, beta, o, h_out=None,
                             stream=None):
    """Decode of one token into slot pos, then the flush of pos + 1 slots (one launch)."""
    d = st.dims
    sh = _token_shapes(d)
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta), ("o", o)):
        _check(t, name, sh[name], _dtype_of(d, name))
    if h_out is not None:
        _check(h_out, "h_out", (d.B, d.H, d.dk, d.dv), torch.float32)
    cs = st.ready()
    rc = load().lq_gdn_decode_step_flush(ct.byref(d), ct.byref(cs), int(pos), _ptr(q), _ptr(k),
                                         _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o), _ptr(h_out),
                                         _stream(stream))
    _raise("lq_gdn_decode_step_flush", rc)


def lq_gdn_decode_step_flush_ragged(st: LayerState, pos, q, k, v, alpha, beta, o, h_out=None,
                                    stream=None):
    """pos: device int32 [B]; rows with pos in [0, W) decode slot pos and flush pos + 1 slots."""
    d = st.dims
    _check(pos, "pos", (d.B,), torch.int32)
    sh = _token_shapes(d)
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta), ("o", o)):
        _check(t, name, sh[name], _dtype_of(d, name))
    if h_out is not None:
        _check(h_out, "h_out", (d.B, d.H, d.dk, d.dv), torch.float32)
    cs = st.ready()
    rc = load().lq_gdn_decode_step_flush_ragged(ct.byref(d), ct.byref(cs), _ptr(pos), _ptr(q), _ptr(k),
                                                _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o), _ptr(h_out),
                                                _stream(stream))
    _raise("lq_gdn_decode_step_flush_ragged", rc)


def lq_gdn_decode_step_ragged(st: LayerState, pos, q, k, v, alpha, beta, o, stream=None):
    """pos: device int32 [B], the window position of each batch row."""
    d = st.dims
    _check(pos, "pos", (d.B,), torch.int32)
    sh = _token_shapes(d)
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta), ("o", o)):
        _check(t, name, sh[name], _dtype_of(d, name))
    cs = st.ready()
    rc = load().lq_gdn_decode_step_ragged(ct.byref(d), ct.byref(cs), _ptr(pos), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(alpha), _ptr(beta), _ptr(o), _stream(stream))
    _raise("lq_gdn_decode_step_ragged", rc)


def lq_gdn_window_flush_ragged(st: LayerState, n_buffered, h_out=None, stream=None):
    """n_buffered: device int32 [B], slots to flush per batch row (0 = none)."""
    d = st.dims
    _check(n_buffered, "n_buffered", (d.B,), torch.int32)
    if h_out is not None:
        _check(h_out, "h_out", (d.B, d.H, d.dk, d.dv), torch.float32)
    cs = st.ready()
    rc = load().lq_gdn_window_flush_ragged(ct.byref(d), ct.byref(cs), _ptr(n_buffered), _ptr(h_out),
                                           _stream(stream))
    _raise("lq_gdn_window_flush_ragged", rc)


def lq_gdn_state_quantize(st: LayerState, h, stream=None):
    d = st.dims
    _check(h, "h", (d.B, d.H, d.dk, d.dv), torch.float32)
    cs = st.ready(with_buffer=False)
    rc = load().lq_gdn_state_quantize(ct.byref(d), _ptr(h), ct.byref(cs), _stream(stream))
    _raise("lq_gdn_state_quantize", rc)


def lq_gdn_state_dequantize(st: LayerState, h_out, stream=None):
    d = st.dims
    _check(h_out, "h_out", (d.B, d.H, d.dk, d.dv), torch.float32)
    cs = st.ready(with_buffer=False)
    rc = load().lq_gdn_state_dequantize(ct.byref(d), ct.byref(cs), _ptr(h_out), _stream(stream))
    _raise("lq_gdn_state_dequantize", rc)


def lq_gdn_fp32_recurrence(d: lq_dims, h, T: int, q, k, v, alpha, beta, o=None, stream=None):
    _check(h, "h", (d.B, d.H, d.dk, d.dv), torch.float32)
    sh = _token_shapes(d, T)
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta)):
        _check(t, name, sh[name], _dtype_of(d, name))
    if o is not None:
        _check(o, "o", sh["o"], _dtype_of(d, "o"))
    rc = load().lq_gdn_fp32_recurrence(ct.byref(d), _ptr(h), int(T), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(alpha), _ptr(beta), _ptr(o), _stream(stream))
    _raise("lq_gdn_fp32_recurrence", rc)


def lq_gdn_prefill(d: lq_dims, st, h, T: int, q, k, v, alpha, beta, o=None, stream=None):
    """Chunked fp32 prefill of T tokens (h in/out), then the codec of the final
    state into st (a LayerState, or None for the fp32 state only)."""
    _check(h, "h", (d.B, d.H, d.dk, d.dv), torch.float32)
    sh = _token_shapes(d, T)
    if T > 0:
        for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta)):
            _check(t, name, sh[name], _dtype_of(d, name))
    if o is not None:
        _check(o, "o", sh["o"], _dtype_of(d, "o"))
    cs = None
    if st is not None:
        cs = st.ready(with_buffer=False)
    rc = load().lq_gdn_prefill(ct.byref(d), ct.byref(cs) if cs is not None else None, _ptr(h), int(T),
                               _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o),
                               _stream(stream))
    _raise("lq_gdn_prefill", rc)


def lq_checkpoint_bytes(d: lq_dims) -> int:
    return int(load().lq_checkpoint_bytes(ct.byref(d)))


def lq_gdn_state_pack(st: LayerState, blob, stream=None):
    """blob: device uint8 tensor of lq_checkpoint_bytes(st.dims) bytes."""
    d = st.dims
    _check(blob, "blob", (lq_checkpoint_bytes(d),), torch.uint8)
    cs = st.ready(with_buffer=False)
    _raise("lq_gdn_state_pack", load().lq_gdn_state_pack(ct.byref(d), ct.byref(cs), _ptr(blob),
                                                          _stream(stream)))


def lq_gdn_state_unpack(st: LayerState, blob, stream=None):
    d = st.dims
    _check(blob, "blob", (lq_checkpoint_bytes(d),), torch.uint8)
    cs = st.ready(with_buffer=False)
    _raise("lq_gdn_state_unpack", load().lq_gdn_state_unpack(ct.byref(d), _ptr(blob), ct.byref(cs),
                                                              _stream(stream)))


def lq_state_bytes(d: lq_dims) -> int:
    return int(load().lq_state_bytes(ct.byref(d)))


def lq_buffer_bytes(d: lq_dims) -> int:
    return int(load().lq_buffer_bytes(ct.byref(d)))


def lq_check_dims(d: lq_dims) -> int:
    return int(load().lq_check_dims(ct.byref(d)))


def lq_measure_stream_read(src, slice_bytes: int, n_slices: int, mode: int, grid: int = 0,
                           sink=None, write_bytes: int = 0, stream=None):
    """Streaming-read reference (measurement only): src and sink device
    tensors holding n_slices * slice_bytes and n_slices * write_bytes bytes."""
    if src.numel() * src.element_size() < slice_bytes * n_slices or not src.is_cuda:
        raise ValueError("src: a device tensor of n_slices * slice_bytes bytes is required")
    if write_bytes and (sink is None or not sink.is_cuda or
                        sink.numel() * sink.element_size() < write_bytes * n_slices):
        raise ValueError("sink: a device tensor of n_slices * write_bytes bytes is required")
    rc = load().lq_measure_stream_read(_ptr(src), int(slice_bytes), int(n_slices), int(mode), int(grid),
                                       _ptr(sink), int(write_bytes), _stream(stream))
    _raise("lq_measure_stream_read", rc)


def lq_timing_enable(on: bool = True):
    _raise("lq_timing_enable", load().lq_timing_enable(1 if on else 0))


def lq_timing_collect(max_records: int = 65536):
    """Per-launch kernel durations recorded since lq_timing_enable(True), in
    launch order: (families, milliseconds) as lists; drops the records."""
    fam = (ct.c_int32 * max_records)()
    ms = (ct.c_float * max_records)()
    n = ct.c_int32(0)
    _raise("lq_timing_collect", load().lq_timing_collect(max_records, fam, ms, ct.byref(n)))
    k = min(n.value, max_records)
    return list(fam[:k]), list(ms[:k])

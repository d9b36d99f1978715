"""ctypes front end of the CPU oracle (oracle/lq_oracle.c).

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's
CPU-baseline leg.  Arrays are numpy; states are fp64 (recurrence) and the
codec is (sq int8 [dk,dv], r fp32 [dk], s fp32 [dv], idx int32 [C],
cv fp32 [C,dv]).  Batched helpers take [B,H,...] arrays and loop over heads,
optionally on a thread pool (ctypes releases the GIL during each call).
"""
from __future__ import annotations

import ctypes as ct
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# LQ_ORACLE_LIB may name another build of the same source (the sanitizer build)
_LIB_PATH = os.environ.get("LQ_ORACLE_LIB") or os.path.join(_HERE, "liblq_oracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i8p = np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_vp = ct.c_void_p


def lib():
    """Loads (building first if absent) the oracle library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ct.CDLL(_LIB_PATH)
        I, F, Lg = ct.c_int, ct.c_float, ct.c_long
        L.lqo_step.argtypes = [I, I, I, _f64p, _f32p, _f32p, _f32p, _f32p, F, _f64p]
        L.lqo_step.restype = None
        L.lqo_quantize.argtypes = [I, I, I, I, _f32p, _i8p, _f32p, _f32p, _i32p, _f32p]
        L.lqo_quantize.restype = I
        L.lqo_dequantize.argtypes = [I, I, I, _i8p, _f32p, _f32p, _i32p, _f32p, _f64p]
        L.lqo_dequantize.restype = None
        L.lqo_wy_append.argtypes = [I, I, I, I, _f64p, _f64p, _f64p, _f64p, _f32p, _f32p, _f32p, F]
        L.lqo_wy_append.restype = None
        L.lqo_wy_output.argtypes = [I, I, I, I, _f64p, _f64p, _f64p, _f64p, _f64p, _f32p, _f64p]
        L.lqo_wy_output.restype = None
        L.lqo_wy_reconstruct.argtypes = [I, I, I, I, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p]
        L.lqo_wy_reconstruct.restype = None
        L.lqo_run_head.argtypes = [I] * 10 + [_vp, Lg] * 5 + [_vp] * 8
        L.lqo_run_head.restype = I
        L.lqo_state_bytes.argtypes = [I, I, I]
        L.lqo_state_bytes.restype = Lg
        _lib = L
    return _lib


def _c32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _c64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# per-head primitives
# --------------------------------------------------------------------------

def step(H: np.ndarray, q, k, v, alpha, beta: float, per_key: bool) -> np.ndarray:
    """One token of the gated delta rule on fp64 state H (modified in place);
    returns o = H^T q (fp64)."""
    dk, dv = H.shape
    o = np.zeros(dv, np.float64)
    lib().lqo_step(dk, dv, int(per_key), H, _c32(q), _c32(k), _c32(v),
                   _c32(np.atleast_1d(alpha)), float(beta), o)
    return o


def quantize(H32: np.ndarray, C: int, smooth: int = 1) -> dict:
    """Codec of one fp32 state (dk x dv)."""
    H32 = _c32(H32)
    dk, dv = H32.shape
    out = dict(sq=np.zeros((dk, dv), np.int8), r=np.zeros(dk, np.float32),
               s=np.zeros(dv, np.float32), idx=np.zeros(max(C, 1), np.int32),
               cv=np.zeros((max(C, 1), dv), np.float32))
    rc = lib().lqo_quantize(dk, dv, C, int(smooth), H32, out["sq"], out["r"], out["s"],
                            out["idx"], out["cv"])
    if rc != 0:
        raise ValueError("lqo_quantize: bad sizes")
    out["idx"] = out["idx"][:C].copy()
    out["cv"] = out["cv"][:C].copy()
    return out


def dequantize(cd: dict) -> np.ndarray:
    """fp64 state a codec stands for."""
    dk, dv = cd["sq"].shape
    C = int(cd["idx"].shape[0])
    H = np.zeros((dk, dv), np.float64)
    idx = np.ascontiguousarray(cd["idx"] if C else np.zeros(1, np.int32), dtype=np.int32)
    cv = _c32(cd["cv"] if C else np.zeros((1, dv), np.float32))
    lib().lqo_dequantize(dk, dv, C, np.ascontiguousarray(cd["sq"], dtype=np.int8),
                         _c32(cd["r"]), _c32(cd["s"]), idx, cv, H)
    return H


def new_buffer(W: int, dk: int, dv: int, per_key: bool) -> dict:
    gd = dk if per_key else 1
    return dict(k=np.zeros((W, dk)), y=np.zeros((W, dk)), u=np.zeros((W, dv)), g=np.zeros((W, gd)))


def wy_append(buf: dict, n: int, k, v, alpha, beta: float, per_key: bool) -> None:
    W, dk = buf["k"].shape
    dv = buf["u"].shape[1]
    lib().lqo_wy_append(dk, dv, int(per_key), n, buf["k"], buf["y"], buf["u"], buf["g"],
                        _c32(k), _c32(v), _c32(np.atleast_1d(alpha)), float(beta))


def wy_output(Hb: np.ndarray, buf: dict, n: int, q, per_key: bool) -> np.ndarray:
    dk, dv = Hb.shape
    o = np.zeros(dv, np.float64)
    lib().lqo_wy_output(dk, dv, int(per_key), n, _c64(Hb), buf["k"], buf["y"], buf["u"],
                        buf["g"], _c32(q), o)
    return o


def wy_reconstruct(Hb: np.ndarray, buf: dict, N: int, per_key: bool) -> np.ndarray:
    dk, dv = Hb.shape
    H = np.zeros((dk, dv), np.float64)
    lib().lqo_wy_reconstruct(dk, dv, int(per_key), N, _c64(Hb), buf["k"], buf["y"], buf["u"],
                             buf["g"], H)
    return H


def state_bytes(dk: int, dv: int, C: int) -> int:
    return int(lib().lqo_state_bytes(dk, dv, C))


def window(cd: dict, tok: dict, per_key: bool, W: int, C: int, smooth: int = 1,
           route: str = "wy") -> dict:
    """One window of the quantized scheme for one head, by the primitives.

    ``tok`` holds N <= W tokens of one head (q [N,dk], k, v [N,dv],
    alpha [N] or [N,dk], beta [N]).  Returns o [N,dv] (fp64), the WY buffer,
    the fp64 state after the window, its fp32 rounding and the next codec.
    """
    N = tok["q"].shape[0]
    Hb = dequantize(cd)
    dk, dv = Hb.shape
    buf = new_buffer(W, dk, dv, per_key)
    o = np.zeros((N, dv))
    Hs = Hb.copy()
    for n in range(N):
        wy_append(buf, n, tok["k"][n], tok["v"][n], tok["alpha"][n], tok["beta"][n], per_key)
        if route == "wy":
            o[n] = wy_output(Hb, buf, n, tok["q"][n], per_key)
        else:
            o[n] = step(Hs, tok["q"][n], tok["k"][n], tok["v"][n], tok["alpha"][n],
                        tok["beta"][n], per_key)
    H = wy_reconstruct(Hb, buf, N, per_key) if route == "wy" else Hs
    H32 = H.astype(np.float32)
    return dict(o=o, buf=buf, H=H, H32=H32, codec=quantize(H32, C, smooth))


def run_head(dk: int, dv: int, per_key: bool, W: int, C: int, smooth: int, *, route: int,
             use_codec: bool, tok: dict, codec: dict | None = None, H0=None,
             flush_tail: bool = False):
    """lqo_run_head over T tokens of one head (tok arrays [T, ...] float32).
    Returns (o [T,dv] fp64, codec_out or None, H_out fp64 or None, hf32_last)."""
    T = tok["q"].shape[0]
    q, k, v = _c32(tok["q"]), _c32(tok["k"]), _c32(tok["v"])
    a = _c32(tok["alpha"]).reshape(T, -1)
    b = _c32(tok["beta"]).reshape(T)
    o = np.zeros((T, dv), np.float64)
    hf = np.zeros((dk, dv), np.float32)
    Cm = max(C, 1)
    if use_codec:
        cd = dict(sq=np.array(codec["sq"], np.int8, order="C"), r=_c32(codec["r"]).copy(),
                  s=_c32(codec["s"]).copy(),
                  idx=np.zeros(Cm, np.int32), cv=np.zeros((Cm, dv), np.float32))
        cd["idx"][:C] = codec["idx"]
        cd["cv"][:C] = codec["cv"]
        H = np.zeros((dk, dv))
    else:
        cd = dict(sq=np.zeros((dk, dv), np.int8), r=np.zeros(dk, np.float32),
                  s=np.zeros(dv, np.float32), idx=np.zeros(Cm, np.int32),
                  cv=np.zeros((Cm, dv), np.float32))
        H = np.array(H0 if H0 is not None else np.zeros((dk, dv)), np.float64, order="C")
    P = lambda x: x.ctypes.data
    rc = lib().lqo_run_head(dk, dv, int(per_key), W, C, int(smooth), int(route), int(use_codec),
                            int(flush_tail), T,
                            P(q), dk, P(k), dk, P(v), dv, P(a), a.shape[1], P(b), 1,
                            P(cd["sq"]), P(cd["r"]), P(cd["s"]), P(cd["idx"]), P(cd["cv"]),
                            P(H), P(o), P(hf))
    if rc != 0:
        raise ValueError("lqo_run_head: bad arguments")
    if use_codec:
        cd["idx"] = cd["idx"][:C].copy()
        cd["cv"] = cd["cv"][:C].copy()
        return o, cd, None, hf
    return o, None, H, hf


# --------------------------------------------------------------------------
# batched helpers ([B,H,...] arrays, token arrays [T,B,H,...])
# --------------------------------------------------------------------------

def head_tokens(tok: dict, b: int, h: int, t0: int = 0, t1: int | None = None) -> dict:
    return {key: np.ascontiguousarray(val[t0:t1, b, h]) for key, val in tok.items()}


def _pool_map(fn, items, threads):
    if threads <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))


def prefill(tok: dict, heads, dk: int, dv: int, per_key: bool, threads: int = 1) -> dict:
    """fp64 recurrence from a zero state over all tokens of ``tok`` for the
    listed (b, h) heads; returns {(b,h): H fp64}."""
    T = tok["q"].shape[0]

    def one(bh):
        b, h = bh
        _, _, H, _ = run_head(dk, dv, per_key, max(T, 1), 0, 1, route=0, use_codec=False,
                              tok=head_tokens(tok, b, h))
        return H
    return dict(zip(heads, _pool_map(one, list(heads), threads)))


def quantize_batch(H32: np.ndarray, C: int, smooth: int = 1) -> dict:
    """Codec of a [B,H,dk,dv] fp32 state, as [B,H,...] arrays."""
    B, Hh, dk, dv = H32.shape
    out = dict(sq=np.zeros((B, Hh, dk, dv), np.int8), r=np.zeros((B, Hh, dk), np.float32),
               s=np.zeros((B, Hh, dv), np.float32), idx=np.zeros((B, Hh, C), np.int32),
               cv=np.zeros((B, Hh, C, dv), np.float32))
    for b in range(B):
        for h in range(Hh):
            cd = quantize(H32[b, h], C, smooth)
            for key in out:
                out[key][b, h] = cd[key]
    return out


def codec_of(cb: dict, b: int, h: int) -> dict:
    return {key: np.ascontiguousarray(val[b, h]) for key, val in cb.items()}

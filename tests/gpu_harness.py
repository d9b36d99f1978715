"""Shared runner of the GPU parity tests: runs the HIP path and the CPU oracle
side by side on the same seeded inputs, window by window (resync protocol).

Per window both sides start from the ORACLE's codec bytes.  The HIP path runs
the window's decode steps and the flush; then, for each sampled head:
  * o_t (every step) against the oracle's window outputs, norm-wise:
    max_j |do_j| / max_j |o_j| <= O_TOL;
  * the buffer the kernels wrote (k_i, g_i, m_i = u_i - Hb^T y_i) against the
    same rows formed from the oracle's WY buffer;
  * the fp32 state the flush handed to its rounding step (h_out) against the
    oracle's fp64 state;
  * the flush's codec bytes against the oracle's codec OF THAT SAME fp32
    state: bit-exact;
and the oracle's own next codec is uploaded into those heads.
"""
from __future__ import annotations

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle as O
from recurrent_state_quant_lq_amd import inputs, lq
from recurrent_state_quant_lq_amd.configs import Workload

O_TOL = 2e-3      # max relative error on o_t (norm-wise per token and head)
# bf16 outputs: bf16 keeps 8 significant bits, so rounding to nearest moves
# each element by at most half an ulp, 2^-8 of itself (so of the row's max),
# on top of the fp32 path's error (well under 1e-4)
O_TOL_BF16 = 2.0 ** -8 + 1e-4
H_TOL = 1e-5      # rebuilt fp32 state vs oracle fp64 state (max-abs relative)
BUF_TOL = 1e-5    # WY buffer rows (max-abs relative per slot)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dims_of(wl: Workload, W=None, C=None, smooth=None, io_bf16=False) -> lq.lq_dims:
    return lq.make_dims(wl.B, wl.H, wl.dk, wl.dv, W or wl.W, wl.C if C is None else C,
                        lq.LQ_DECAY_PER_KEY if wl.per_key else lq.LQ_DECAY_SCALAR,
                        wl.smooth if smooth is None else smooth,
                        lq.LQ_IO_BF16 if io_bf16 else lq.LQ_IO_F32)


def io_tokens(tk: dict, bf16: bool) -> dict:
    """q, k, v as the library's token dtype (bf16: rounded once, here)."""
    if not bf16:
        return tk
    return {k: (v.to(torch.bfloat16) if k in ("q", "k", "v") else v) for k, v in tk.items()}


def host(x) -> np.ndarray:
    """Device tensor (fp32 or bf16) -> fp32 numpy (bf16 widens exactly)."""
    return x.float().cpu().numpy()


def rel_err(a, b, axis=-1):
    """max |a-b| / max |b| along axis, maximised over the rest."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    num = np.abs(a - b).max(axis=axis)
    den = np.maximum(np.abs(b).max(axis=axis), 1e-30)
    return float((num / den).max())


def codec_equal(gpu: dict, orc: dict) -> bool:
    for key in ("sq", "r", "s", "idx", "cv"):
        g, o = np.ascontiguousarray(gpu[key]), np.ascontiguousarray(orc[key])
        if g.shape != o.shape or g.tobytes() != o.tobytes():
            return False
    return True


def oracle_buffer(cd: dict, buf: dict, N: int) -> dict:
    """The library's buffer rows from the oracle's WY buffer of one window:
    keys, log-decays and m_i = u_i - Hb^T y_i (Hb: the window-base state the
    codec stands for), all fp64."""
    Hb = O.dequantize(cd)
    return dict(k=buf["k"][:N], g=buf["g"][:N], m=buf["u"][:N] - buf["y"][:N] @ Hb)


def upload_head_codec(st: lq.LayerState, b: int, h: int, cd: dict):
    C = st.dims.C
    st.sq[b, h].copy_(torch.from_numpy(lq.sq_from_rows(cd["sq"])))
    st.row_scale[b, h].copy_(torch.from_numpy(cd["r"]))
    st.col_scale[b, h].copy_(torch.from_numpy(cd["s"]))
    if C:
        st.comp_idx[b, h, :C].copy_(torch.from_numpy(cd["idx"]))
        st.comp_val[b, h, :C].copy_(torch.from_numpy(cd["cv"]))


def head_codec(st: lq.LayerState, b: int, h: int) -> dict:
    C = st.dims.C
    return dict(sq=lq.sq_to_rows(st.sq[b, h].cpu().numpy(), st.dims.dk), r=st.row_scale[b, h].cpu().numpy(),
                s=st.col_scale[b, h].cpu().numpy(), idx=st.comp_idx[b, h, :C].cpu().numpy(),
                cv=st.comp_val[b, h, :C].cpu().numpy())


class TokenSource:
    """Prefill + decode tokens of a workload.  Small workloads draw them on the
    host (numpy Philox), large ones on the device in chunks (torch Philox);
    both come from recurrent_state_quant_lq_amd.inputs."""

    def __init__(self, wl: Workload, host: bool, chunk: int = 256):
        self.wl, self.host, self.chunk = wl, host, chunk
        self._last = (None, None)         # the last device chunk drawn: (index, tensors)
        self.out = inputs.make_outliers(wl.seed, wl.H, wl.dk, wl.dv) if wl.outliers else None
        self._host = None
        if host:
            self._host = inputs.host_tokens(wl.seed, wl.prefill + wl.T, wl.B, wl.H, wl.dk, wl.dv,
                                            per_key=wl.per_key, beta_lo=wl.beta_lo,
                                            beta_hi=wl.beta_hi, outliers=self.out)

    def tokens(self, t0: int, t1: int) -> dict:
        """Device tensors [t1-t0, B, H, ...] of absolute tokens t0..t1-1."""
        wl = self.wl
        if self.host:
            return {k: torch.from_numpy(np.ascontiguousarray(v[t0:t1])).cuda()
                    for k, v in self._host.items()}
        # device chunks of `chunk` tokens, chunk c seeded by (seed, c)
        parts = []
        c0, c1 = t0 // self.chunk, (t1 - 1) // self.chunk
        for c in range(c0, c1 + 1):
            if self._last[0] == c:
                tk = self._last[1]
            else:
                tk = inputs.device_tokens(wl.seed * 1000 + c, self.chunk, wl.B, wl.H, wl.dk, wl.dv,
                                          per_key=wl.per_key, beta_lo=wl.beta_lo, beta_hi=wl.beta_hi,
                                          device="cuda", outliers=self.out)
                self._last = (c, tk)
            a = max(t0, c * self.chunk) - c * self.chunk
            b = min(t1, (c + 1) * self.chunk) - c * self.chunk
            parts.append({k: v[a:b] for k, v in tk.items()})
        return {k: torch.cat([p[k] for p in parts]).contiguous() for k in parts[0]}


@dataclass
class Report:
    o_err: float = 0.0
    h_err: float = 0.0
    buf_err: float = 0.0
    windows: int = 0
    heads: int = 0
    bytes_exact: bool = True
    mismatches: list = field(default_factory=list)


def prefill_state(wl: Workload, src: TokenSource, st: lq.LayerState, sample, chunk=256):
    """Starting codec: the oracle's quantization of its own fp64 prefill for
    the sampled heads; the HIP fp32 recurrence + quantizer for the others."""
    d = st.dims
    B, H, dk, dv = wl.B, wl.H, wl.dk, wl.dv
    start = {}
    if wl.prefill == 0:
        for bh in sample:
            start[bh] = O.quantize(np.zeros((dk, dv), np.float32), d.C, d.smooth)
        st.sq.zero_(); st.row_scale.zero_(); st.col_scale.fill_(1.0)
        st.comp_val.zero_()
        st.comp_idx.copy_(torch.arange(st.comp_idx.shape[-1], dtype=torch.int32).expand_as(st.comp_idx))
    else:
        h = torch.zeros((B, H, dk, dv), dtype=torch.float32, device="cuda")
        Hs = {bh: np.zeros((dk, dv)) for bh in sample}
        for t0 in range(0, wl.prefill, chunk):
            t1 = min(wl.prefill, t0 + chunk)
            tk = io_tokens(src.tokens(t0, t1), d.io_dtype == lq.LQ_IO_BF16)
            lq.lq_gdn_fp32_recurrence(d, h, t1 - t0, tk["q"], tk["k"], tk["v"], tk["alpha"], tk["beta"])
            for (b, hh) in sample:
                ht = {k: host(v[:, b, hh]) for k, v in tk.items()}
                _, _, Hs[(b, hh)], _ = O.run_head(dk, dv, wl.per_key, t1 - t0, 0, 1, route=0,
                                                  use_codec=False, tok=ht, H0=Hs[(b, hh)])
        lq.lq_gdn_state_quantize(st, h)
        for bh in sample:
            start[bh] = O.quantize(Hs[bh].astype(np.float32), d.C, d.smooth)
    for (b, hh), cd in start.items():
        upload_head_codec(st, b, hh, cd)
    torch.cuda.synchronize()
    return start


def resync_run(wl: Workload, sample, *, host_tokens: bool, W=None, C=None, smooth=None,
               T=None, check_buffers=True, log_every=0, fused=False, io_bf16=False) -> Report:
    """fused: each window's last token goes through lq_gdn_decode_step_flush
    (decode + flush in one launch) instead of a decode step and a flush.
    io_bf16: q, k, v and o in bf16 (the oracle gets the bf16 values widened)."""
    d = dims_of(wl, W, C, smooth, io_bf16)
    W, T = d.W, (T if T is not None else wl.T)
    src = TokenSource(wl, host_tokens)
    st = lq.LayerState.allocate(d)
    codec = prefill_state(wl, src, st, sample)
    rep = Report(heads=len(sample))
    iot = lq.io_torch_dtype(d)
    o = torch.empty((wl.B, wl.H, wl.dv), dtype=iot, device="cuda")
    h_out = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    t = 0
    while t < T:
        N = min(W, T - t)
        tk = io_tokens(src.tokens(wl.prefill + t, wl.prefill + t + N), io_bf16)
        outs = torch.empty((N, wl.B, wl.H, wl.dv), dtype=iot, device="cuda")
        for n in range(N):
            args = (tk["q"][n], tk["k"][n], tk["v"][n], tk["alpha"][n], tk["beta"][n], o)
            if fused and n == N - 1:
                lq.lq_gdn_decode_step_flush(st, n, *args, h_out=h_out)
            else:
                lq.lq_gdn_decode_step(st, n, *args)
            outs[n].copy_(o)
        if not fused:
            lq.lq_gdn_window_flush(st, N, h_out)
        # the flush leaves the buffer as the decode steps wrote it
        bufs = ({k: getattr(st, "buf_" + k).clone() for k in ("k", "m", "g")}
                if check_buffers else None)
        torch.cuda.synchronize()
        for (b, h) in sample:
            ht = {k: host(v[:, b, h]) for k, v in tk.items()}
            res = O.window(codec[(b, h)], ht, wl.per_key, W, d.C, d.smooth, route="wy")
            rep.o_err = max(rep.o_err, rel_err(host(outs[:, b, h]), res["o"]))
            hg = h_out[b, h].cpu().numpy()
            rep.h_err = max(rep.h_err, float(np.abs(hg - res["H"]).max() / max(np.abs(res["H"]).max(), 1e-30)))
            if check_buffers:
                ob = oracle_buffer(codec[(b, h)], res["buf"], N)
                for key in ("k", "m", "g"):
                    g = bufs[key][b, h, :N].cpu().numpy()
                    rep.buf_err = max(rep.buf_err, rel_err(g, ob[key]))
            gc = head_codec(st, b, h)
            if not codec_equal(gc, O.quantize(hg, d.C, d.smooth)):
                rep.bytes_exact = False
                rep.mismatches.append((t, b, h))
            codec[(b, h)] = res["codec"]
            upload_head_codec(st, b, h, res["codec"])
        rep.windows += 1
        t += N
        if log_every and rep.windows % log_every == 0:
            say(f"  window {rep.windows}: o_err {rep.o_err:.2e} h_err {rep.h_err:.2e} "
                f"buf_err {rep.buf_err:.2e} exact {rep.bytes_exact}")
    return rep


def free_run(wl: Workload, sample, *, host_tokens: bool, T: int) -> dict:
    """GPU path and oracle each run on their own for T tokens from the same
    starting codec (no resync): per flush, the number of int8 state bytes
    that differ between the two codecs of each sampled head, and the largest
    relative output difference over all tokens.  Two correct fp32 paths differ
    by ulps, which can flip a rounding at a .5 boundary; this measures how far
    such flips carry."""
    d = dims_of(wl)
    W = d.W
    src = TokenSource(wl, host_tokens)
    st = lq.LayerState.allocate(d)
    orc = prefill_state(wl, src, st, sample)          # both sides start from these codecs
    o = torch.empty((wl.B, wl.H, wl.dv), dtype=torch.float32, device="cuda")
    flips, o_err, max_step = [], 0.0, 0
    t = 0
    while t < T:
        N = min(W, T - t)
        tk = src.tokens(wl.prefill + t, wl.prefill + t + N)
        outs = torch.empty((N, wl.B, wl.H, wl.dv), dtype=torch.float32, device="cuda")
        for n in range(N):
            args = (tk["q"][n], tk["k"][n], tk["v"][n], tk["alpha"][n], tk["beta"][n], o)
            if n < N - 1:
                lq.lq_gdn_decode_step(st, n, *args)
            else:
                lq.lq_gdn_decode_step_flush(st, n, *args)
            outs[n].copy_(o)
        torch.cuda.synchronize()
        per = []
        for (b, h) in sample:
            ht = {k: host(v[:, b, h]) for k, v in tk.items()}
            res = O.window(orc[(b, h)], ht, wl.per_key, W, d.C, d.smooth, route="wy")
            o_err = max(o_err, rel_err(host(outs[:, b, h]), res["o"]))
            orc[(b, h)] = res["codec"]
            gc = head_codec(st, b, h)
            diff = gc["sq"].astype(np.int32) - res["codec"]["sq"].astype(np.int32)
            per.append(int(np.count_nonzero(diff)))
            max_step = max(max_step, int(np.abs(diff).max()))
        flips.append(per)
        t += N
    return dict(o_err=o_err, flips=flips, max_byte_diff=max_step, bytes_per_head=wl.dk * wl.dv)


def oracle_threads() -> int:
    """Worker threads for per-head oracle work (ctypes releases the GIL in
    each call); at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def every_head_window(wl: Workload, *, prefill: int, fused: bool, W=None, log=True) -> Report:
    """One full-size window checked against the oracle on EVERY head.

    Start: for every head, the oracle's own fp64 recurrence from a zero state
    over ``prefill`` tokens of the workload's input distribution, rounded to
    fp32 and quantized by the oracle (heads spread over a thread pool); the
    codecs are uploaded in one copy per array.  The GPU then runs one window
    of W tokens (decode steps, then the fused last token or a decode step and
    a flush) on all heads, and every head is checked as in resync_run:
    outputs, buffer rows, the flush's fp32 state and the codec bytes."""
    d = dims_of(wl, W)
    W = d.W
    B, H, dk, dv, C = wl.B, wl.H, wl.dk, wl.dv, d.C
    heads = [(b, h) for b in range(B) for h in range(H)]
    nthr = oracle_threads()
    t_start = time.time()
    src = TokenSource(wl, host=False)
    pre = {k: v.cpu().numpy() for k, v in src.tokens(0, prefill).items()} if prefill else None
    win_dev = src.tokens(prefill, prefill + W)
    win = {k: v.cpu().numpy() for k, v in win_dev.items()}

    def start_codec(bh):
        b, h = bh
        if pre is None:
            Hs = np.zeros((dk, dv))
        else:
            _, _, Hs, _ = O.run_head(dk, dv, wl.per_key, prefill, 0, 1, route=0, use_codec=False,
                                     tok=O.head_tokens(pre, b, h), H0=np.zeros((dk, dv)))
        return O.quantize(Hs.astype(np.float32), C, d.smooth)

    with ThreadPoolExecutor(max_workers=nthr) as ex:
        codecs = list(ex.map(start_codec, heads))
    cb = dict(sq=np.empty((B, H, dk, dv), np.int8), r=np.empty((B, H, dk), np.float32),
              s=np.empty((B, H, dv), np.float32), idx=np.empty((B, H, C), np.int32),
              cv=np.empty((B, H, C, dv), np.float32))
    for (b, h), cd in zip(heads, codecs):
        for key in cb:
            cb[key][b, h] = cd[key]
    if log:
        say(f"  every-head start codecs: {len(heads)} heads, {prefill} prefill tokens, "
            f"{nthr} threads, {time.time() - t_start:.1f} s")
    st = lq.LayerState.allocate(d)
    st.load_codec(cb)
    o = torch.empty((B, H, dv), dtype=torch.float32, device="cuda")
    h_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    outs = torch.empty((W, B, H, dv), dtype=torch.float32, device="cuda")
    for n in range(W):
        args = (win_dev["q"][n], win_dev["k"][n], win_dev["v"][n], win_dev["alpha"][n],
                win_dev["beta"][n], o)
        if fused and n == W - 1:
            lq.lq_gdn_decode_step_flush(st, n, *args, h_out=h_out)
        else:
            lq.lq_gdn_decode_step(st, n, *args)
        outs[n].copy_(o)
    if not fused:
        lq.lq_gdn_window_flush(st, W, h_out)
    torch.cuda.synchronize()
    g_o = outs.cpu().numpy()
    g_h = h_out.cpu().numpy()
    g_buf = {k: getattr(st, "buf_" + k).cpu().numpy() for k in ("k", "m", "g")}
    g_cd = st.codec()

    def check(i):
        b, h = heads[i]
        res = O.window(codecs[i], O.head_tokens(win, b, h), wl.per_key, W, C, d.smooth, route="wy")
        oe = rel_err(g_o[:, b, h], res["o"])
        he = float(np.abs(g_h[b, h] - res["H"]).max() / max(np.abs(res["H"]).max(), 1e-30))
        ob = oracle_buffer(codecs[i], res["buf"], W)
        be = max(rel_err(g_buf[key][b, h, :W], ob[key]) for key in ("k", "m", "g"))
        exact = codec_equal({key: g_cd[key][b, h] for key in g_cd}, O.quantize(g_h[b, h], C, d.smooth))
        return oe, he, be, exact

    with ThreadPoolExecutor(max_workers=nthr) as ex:
        per = list(ex.map(check, range(len(heads))))
    rep = Report(heads=len(heads), windows=1)
    for (b, h), (oe, he, be, exact) in zip(heads, per):
        rep.o_err = max(rep.o_err, oe)
        rep.h_err = max(rep.h_err, he)
        rep.buf_err = max(rep.buf_err, be)
        if not exact:
            rep.bytes_exact = False
            rep.mismatches.append((prefill, b, h))
    if log:
        say(f"  every-head window checked in {time.time() - t_start:.1f} s")
    return rep

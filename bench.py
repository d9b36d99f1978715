#!/usr/bin/env python3
"""Decode throughput of the int8-state Gated DeltaNet path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--layers L] [--workload NAME]

A step is one pass of the whole hot path over one batch: a window of W decode
tokens (lq_gdn_decode_step at positions 0..W-1) followed by the window flush
(lq_gdn_window_flush), for each of L independent GDN layers (default 8, the
layers' states rotated so that the working set, about 720 MB at
B=64 H=32 d=128, exceeds the 256 MB Infinity Cache and every step reads HBM).
Inputs are synthetic, drawn on the device before timing; the starting state
comes from a 512-token fp32 prefill run by the library's fp32 recurrence and
quantized by its quantizer.

Printed (one JSON line): tokens/s through one layer (B * W * L tokens per
step), the decode kernel's roofline (algorithmic bytes over its per-launch
duration measured with HIP events on the launch stream), the flush's, and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F32_PEAK_TFS = 157.3      # MI355X dense fp32 matrix, published
METRIC = "decode tokens/s and state HBM GB/s (% of peak), int8 GDN, B=64 H=32 d=128"
PMC_FILE = os.path.join(ROOT, "profiles", "decode_step_gdn_b64_h32_d128_w16_pmc.md")


def decode_bytes(wl, n: int) -> int:
    """Algorithmic HBM bytes of one decode launch at window slot n: the codec
    (int8 state, scales, compensators), the token inputs and output, the n
    buffered slots read and slot n written."""
    dk, dv, C = wl.dk, wl.dv, wl.C
    a = dk if wl.per_key else 1
    codec = dk * dv + 4 * dk + 4 * dv + C * (4 * dv + 4)
    io = 4 * (2 * dk + dv + a + 1) + 4 * dv
    slot = 4 * (2 * dk + dv + a)
    return wl.B * wl.H * (codec + io + (n + 1) * slot)


def flush_bytes(wl, N: int) -> int:
    """Algorithmic HBM bytes of one flush of N slots: read and write the codec,
    read the N buffered slots."""
    dk, dv, C = wl.dk, wl.dv, wl.C
    a = dk if wl.per_key else 1
    codec = dk * dv + 4 * dk + 4 * dv + C * (4 * dv + 4)
    return wl.B * wl.H * (2 * codec + N * 4 * (2 * dk + dv + a))


def flush_flops(wl, N: int) -> int:
    """The two contractions of the rebuild: 2 * (N*dk*dv) multiply-adds."""
    return wl.B * wl.H * 4 * N * wl.dk * wl.dv


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "lq_internal.h"):
        h.update(open(os.path.join(ROOT, "recurrent_state_quant_lq_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(wl, hsh: str):
    """Measured HBM bytes per decode launch from the committed rocprofv3 PMC
    summary, if it was taken on the current decode kernel."""
    if not os.path.exists(PMC_FILE):
        return None
    for line in open(PMC_FILE):
        line = line.strip()
        if line.startswith("{") and '"kernel_hash"' in line:
            rec = json.loads(line)
            if rec.get("kernel_hash") == hsh:
                return rec.get("hbm_bytes_per_launch")
    return None


def cpu_baseline(wl, windows: int, threads: int):
    """The oracle (plain C, as it is) on the host: the windowed int8 scheme
    for all B*H heads of one layer over `windows` windows."""
    import numpy as np
    import oracle as O
    from recurrent_state_quant_lq_amd import inputs
    tok = inputs.host_tokens(4242, wl.W, wl.B, wl.H, wl.dk, wl.dv, per_key=wl.per_key,
                             beta_lo=wl.beta_lo, beta_hi=wl.beta_hi)
    rng = np.random.default_rng(1)
    H0 = (rng.standard_normal((wl.dk, wl.dv)) * 0.1).astype(np.float32)
    cd0 = O.quantize(H0, wl.C, wl.smooth)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    per_head = {bh: {k: np.ascontiguousarray(np.concatenate([v[:, bh[0], bh[1]]] * windows))
                     for k, v in tok.items()} for bh in heads}

    def one(bh):
        O.run_head(wl.dk, wl.dv, wl.per_key, wl.W, wl.C, wl.smooth, route=0, use_codec=True,
                   tok=per_head[bh], codec=cd0)

    from concurrent.futures import ThreadPoolExecutor
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, heads))
    dt = time.perf_counter() - t0
    return dict(value=wl.B * wl.W * windows / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"one layer, all {len(heads)} heads, {windows} windows of {wl.W} tokens "
                       f"(plain recurrence + codec, fp64/fp32), {dt:.2f} s wall")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--workload", default="gdn_batched")
    ap.add_argument("--W", type=int, default=0, help="override the window length")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-windows", type=int, default=8)
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain device copy of known size (for PMC calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(every (batch, head) state is independent; see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from recurrent_state_quant_lq_amd import inputs, lq
    from recurrent_state_quant_lq_amd.configs import PRESETS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calib:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n}))
        return

    wl = PRESETS[args.workload]
    if args.W:
        wl = wl.with_(W=args.W)
    L, W = args.layers, wl.W
    d = lq.make_dims(wl.B, wl.H, wl.dk, wl.dv, W, wl.C,
                     lq.LQ_DECAY_PER_KEY if wl.per_key else lq.LQ_DECAY_SCALAR, wl.smooth)
    out = inputs.make_outliers(wl.seed, wl.H, wl.dk, wl.dv) if wl.outliers else None
    gen = lambda seed, T: inputs.device_tokens(seed, T, wl.B, wl.H, wl.dk, wl.dv, per_key=wl.per_key,
                                               beta_lo=wl.beta_lo, beta_hi=wl.beta_hi, device=dev,
                                               outliers=out)

    # starting state: fp32 prefill on the device, quantized, copied into L layers
    h = torch.zeros((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=dev)
    for c0 in range(0, wl.prefill, 128):
        T = min(128, wl.prefill - c0)
        tk = gen(wl.seed * 100 + c0, T)
        lq.lq_gdn_fp32_recurrence(d, h, T, tk["q"], tk["k"], tk["v"], tk["alpha"], tk["beta"])
        del tk
    layers = [lq.LayerState.allocate(d, dev) for _ in range(L)]
    for st in layers:
        lq.lq_gdn_state_quantize(st, h)
    del h
    # input ring: W tokens per layer
    ring = [gen(wl.seed * 7 + l, W) for l in range(L)]
    o = torch.empty((wl.B, wl.H, wl.dv), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        for n in range(W):
            for l in range(L):
                tk = ring[l]
                if ev is not None:
                    ev[0][n][l].record()
                lq.lq_gdn_decode_step(layers[l], n, tk["q"][n], tk["k"][n], tk["v"][n],
                                      tk["alpha"][n], tk["beta"][n], o)
                if ev is not None:
                    ev[1][n][l].record()
        for l in range(L):
            if ev is not None:
                ev[2][l].record()
            lq.lq_gdn_window_flush(layers[l], W)
            if ev is not None:
                ev[3][l].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region ---------------------------------------------------------
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    tokens_per_step = wl.B * W * L
    value = tokens_per_step / (ms * 1e-3)

    # ---- per-launch kernel durations (HIP events on the launch stream) ----------
    E = lambda: torch.cuda.Event(enable_timing=True)
    reps = max(2, min(8, args.steps))
    dec_ms = [0.0] * W
    fl_ms = 0.0
    for _ in range(reps):
        ev = ([[E() for _ in range(L)] for _ in range(W)], [[E() for _ in range(L)] for _ in range(W)],
              [E() for _ in range(L)], [E() for _ in range(L)])
        step(ev)
        torch.cuda.synchronize()
        for n in range(W):
            for l in range(L):
                dec_ms[n] += ev[0][n][l].elapsed_time(ev[1][n][l])
        for l in range(L):
            fl_ms += ev[2][l].elapsed_time(ev[3][l])
    launches = reps * L
    dec_avg_us = [1e3 * x / launches for x in dec_ms]
    dec_bytes = [decode_bytes(wl, n) for n in range(W)]
    dec_total_s = sum(dec_avg_us) * 1e-6
    dec_gbs = sum(dec_bytes) / dec_total_s / 1e9
    fl_avg_us = 1e3 * fl_ms / launches
    fl_gbs = flush_bytes(wl, W) / (fl_avg_us * 1e-6) / 1e9
    fl_tfs = flush_flops(wl, W) / (fl_avg_us * 1e-6) / 1e12

    hsh = kernel_hash()
    traffic = read_traffic(wl, hsh)
    roof = {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "lq_gdn_decode_step (decode_kernel<128,128,16,GDN>)",
            "avg_launch_us": round(dec_total_s * 1e6 / W, 3),
            "bytes_per_launch_avg": int(sum(dec_bytes) / W)}

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8-state/f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "dk": wl.dk, "dv": wl.dv, "W": W,
                   "C": wl.C, "decay": "per-key" if wl.per_key else "scalar",
                   "layers_rotated": L, "tokens_per_step": tokens_per_step,
                   "step": f"{W} decode tokens + 1 flush for each of {L} layers",
                   "value_per": "tokens through one GDN layer per second",
                   "prefill": wl.prefill},
        "roofline": roof,
        "state_GBps": round(dec_gbs, 1),
        "flush": {"avg_launch_us": round(fl_avg_us, 3), "hbm_GBps": round(fl_gbs, 1),
                  "hbm_frac": round(fl_gbs / HBM_PEAK_GBS, 4), "mfma_f32_TFLOPs": round(fl_tfs, 2),
                  "mfma_frac": round(fl_tfs / MFMA_F32_PEAK_TFS, 4)},
        "decode_us_by_slot": [round(x, 3) for x in dec_avg_us],
        "kernel_hash": hsh,
    }
    if not args.no_cpu:
        threads = min(16, os.cpu_count() or 1)
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_windows, threads)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

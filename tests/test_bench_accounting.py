"""The benchmark's algorithmic byte counts (the roofline's numerator), pinned
two ways: the codec and buffer terms equal the sizes the C library reports
for the same shapes (lq_state_bytes, lq_buffer_bytes), and the per-launch
totals of the B=64 H=32 d=128 W=16 C=4 step are the figures stated with the
roofline (22,556 + 1,028 n bytes per head at slot n; 60,932,096 bytes per
decode launch over slots 0..14; 117,653,504 per fused last-token launch)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from recurrent_state_quant_lq_amd import lq  # noqa: E402
from recurrent_state_quant_lq_amd.configs import PRESETS  # noqa: E402


def _dims(wl):
    return lq.make_dims(wl.B, wl.H, wl.dk, wl.dv, wl.W, wl.C,
                        lq.LQ_DECAY_PER_KEY if wl.per_key else lq.LQ_DECAY_SCALAR, wl.smooth)


@pytest.mark.parametrize("name", ["gdn_batched", "kda", "gdn_layer", "tiny_gdn"])
def test_terms_match_library_sizes(name):
    wl = PRESETS[name]
    d = _dims(wl)
    heads = wl.B * wl.H
    a = wl.dk if wl.per_key else 1
    io = 4 * (2 * wl.dk + wl.dv + a + 1) + 4 * wl.dv
    slot = 4 * (wl.dk + wl.dv + a)
    state = lq.lq_state_bytes(d)          # the codec arrays of all heads
    buf = lq.lq_buffer_bytes(d)           # W slots of all heads
    assert buf == heads * wl.W * slot
    # decode at slot n: the codec once, the token's I/O, n slots read and one written
    for n in range(wl.W):
        assert bench.decode_bytes(wl, n) == state + heads * io + (n + 1) * heads * slot
    # flush of N slots: the codec read and written, N slots read
    for N in (1, wl.W):
        assert bench.flush_bytes(wl, N) == 2 * state + N * heads * slot
        assert bench.decode_flush_bytes(wl, N) == 2 * state + heads * io + N * heads * slot


def test_headline_step_figures():
    wl = PRESETS["gdn_batched"]
    heads = wl.B * wl.H
    for n in range(wl.W):
        assert bench.decode_bytes(wl, n) == heads * (22556 + 1028 * n)
    assert sum(bench.decode_bytes(wl, n) for n in range(wl.W - 1)) // (wl.W - 1) == 60932096
    assert bench.decode_flush_bytes(wl, wl.W) == 117653504
    assert bench.flush_bytes(wl, wl.W) == heads * 55392


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    """The benchmark times one GPU's share; asked for several (a flag or a
    launcher's WORLD_SIZE) it exits with status 2 and says why, before
    touching a device."""
    import subprocess
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], env=e,
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "runs on one GPU" in r.stderr
    assert r.stdout == ""


def test_scope_table_figures():
    """The scope table's per-head decode bytes at d = 128 (GDN): 23,068 +
    1,540 n (the WY buffer with y and u stored), 69.3 MB per launch over slots
    0..14 at B=64 H=32; the kernel's own count is 512 n + 512 bytes smaller
    per head (one projected vector per slot instead of two)."""
    wl = PRESETS["gdn_batched"]
    heads = wl.B * wl.H
    for n in range(wl.W):
        assert bench.scope_table_decode_bytes(wl, n) == heads * (23068 + 1540 * n)
        assert bench.scope_table_decode_bytes(wl, n) - bench.decode_bytes(wl, n) == heads * 512 * (n + 1)
    mean = sum(bench.scope_table_decode_bytes(wl, n) for n in range(wl.W - 1)) / (wl.W - 1)
    assert round(mean / 1e6, 1) == 69.3
    rd, wr = bench.decode_read_write_bytes(wl, 5)
    assert heads * (rd + wr) == bench.decode_bytes(wl, 5)


def test_host_cpu_fields():
    info = bench.host_cpu()
    assert info["logical_cpus"] >= 1 and 1 <= info["usable_cpus"] <= info["logical_cpus"]
    assert set(info) == {"model", "logical_cpus", "usable_cpus", "cgroup_cpu_quota"}

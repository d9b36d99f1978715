"""The step as independent chains of batch rows on separate streams.

The batch's rows are independent sequences, so a step can run as S chains of
B/S rows each (LayerState.rows views of the same arrays), one per stream, in
one captured graph.  Every result must equal the single-stream run bit for bit:
each head is one workgroup whatever the batch size of its launch.  The graph is
replayed for several windows, with eager copies and synchronizations between
the replays, and every replay is checked.
"""
import pytest
import torch

from recurrent_state_quant_lq_amd import inputs, lq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lq.load()


def _fresh(d, h, L):
    lays = [lq.LayerState.allocate(d, h.device) for _ in range(L)]
    for st in lays:
        lq.lq_gdn_state_quantize(st, h)
    return lays


@pytest.mark.parametrize("per_key", [False, True])
def test_two_stream_chains_match_one_stream(per_key):
    dev = torch.device("cuda:0")
    B, H, dk, W, C, L, S = 8, 8, 128, 16, 4, 2, 2
    d = lq.make_dims(B, H, dk, dk, W, C, lq.LQ_DECAY_PER_KEY if per_key else lq.LQ_DECAY_SCALAR, 1)
    g = torch.Generator(device=dev).manual_seed(11)
    h = torch.randn((B, H, dk, dk), device=dev, generator=g) * 0.3
    ref = _fresh(d, h, L)
    tst = _fresh(d, h, L)
    Bs = B // S
    chains = [[st.rows(i * Bs, (i + 1) * Bs) for st in tst] for i in range(S)]
    side = [torch.cuda.Stream(device=dev) for _ in range(S)]
    # token buffers the graph reads (refilled before every replay), outputs per token
    ring = [inputs.device_tokens(300 + l, W, B, H, dk, dk, per_key=per_key, beta_lo=0.1, beta_hi=0.9, device=dev)
            for l in range(L)]
    o_ref = torch.zeros((L, W, B, H, dk), device=dev)
    o_tst = torch.zeros_like(o_ref)

    def window(lays, o_all, rows=None, stream=None):
        cut = (lambda x: x) if rows is None else (lambda x: x[rows[0]:rows[1]])
        for n in range(W):
            for l in range(L):
                tk = ring[l]
                args = (cut(tk["q"][n]), cut(tk["k"][n]), cut(tk["v"][n]), cut(tk["alpha"][n]),
                        cut(tk["beta"][n]), cut(o_all[l, n]))
                if n < W - 1:
                    lq.lq_gdn_decode_step(lays[l], n, *args, stream=stream)
                else:
                    lq.lq_gdn_decode_step_flush(lays[l], n, *args, stream=stream)

    def chained():
        main = torch.cuda.current_stream()
        for s_ in side:
            s_.wait_stream(main)
        for i, s_ in enumerate(side):
            with torch.cuda.stream(s_):
                window(chains[i], o_tst, rows=(i * Bs, (i + 1) * Bs), stream=s_)
        for s_ in side:
            main.wait_stream(s_)

    # capture on scratch copies of the state, then restore (capture runs nothing)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chained()
    torch.cuda.synchronize()
    for rep in range(3):
        fresh = [inputs.device_tokens(400 + 10 * rep + l, W, B, H, dk, dk, per_key=per_key, beta_lo=0.1,
                                      beta_hi=0.9, device=dev) for l in range(L)]
        for l in range(L):
            for key in ring[l]:
                ring[l][key].copy_(fresh[l][key])
        torch.cuda.synchronize()
        window(ref, o_ref)                      # eager, one stream, all rows
        graph.replay()                          # two chains on two streams
        torch.cuda.synchronize()
        print(f"replay {rep} per_key={per_key}", flush=True)
        assert torch.equal(o_ref, o_tst), f"outputs differ (replay {rep})"
        for a, b in zip(ref, tst):
            for f in ("sq", "row_scale", "col_scale", "comp_idx", "comp_val", "buf_k", "buf_m", "buf_g"):
                assert torch.equal(getattr(a, f), getattr(b, f)), f"{f} differs (replay {rep})"

"""A decode step (a one-token append per sequence, then decode) captured in a
HIP graph through torch's graph API and replayed several times, with eager
work and synchronizations between the replays: every replay's output equals
the eager step's bit for bit and leaves no status flag.  The library's calls
only launch kernels on the caller's stream (no allocation, no memset, no
host synchronization), so a serving loop can capture them; the append of the
same token at the same position is idempotent, so each replay recomputes the
same cache and output.  Modes: uniform INT4 (one attention kernel and the
merge), channel-axis K (the streaming tail, the token V rows, attention,
merge), Oaken (the one-token Oaken append, the K score-share kernel,
attention), paged INT8 and paged Oaken, DSQ (its one-token append into the
tails, then decode), the chunk-mixed cache (decode alone: its cache is
full), and the no-alloc decode entry point."""
import numpy as np
import pytest

import synth
from kvq_harness import i32_device, to_device
from test_gpu_determinism import SM, build

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("quantized_kv_cache_05_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.lib()
    yield


@pytest.mark.parametrize("mode,noalloc", [("uniform_4_a_64", False), ("uniform_4_a_64", True),
                                          ("channel4", False), ("oaken", False), ("paged8", False),
                                          ("paged_oaken", False), ("dsq", False), ("mixed", False)])
@pytest.mark.parametrize("G", [1, 4])
def test_graph_replay_matches_eager_step(mode, noalloc, G):
    print("case graph %s noalloc=%d G=%d" % (mode, noalloc, G), flush=True)
    cache, q, Hq, _, T = build(mode, G)
    torch.cuda.synchronize()
    assert cache.flags() == 0
    B, H = q.shape[0], Hq // G
    wl = {"oaken": 5, "paged_oaken": 5, "channel4": 3, "dsq": 8}.get(mode, 2)
    w = synth.scaled(synth.WORKLOADS[wl], batch=B, kv_heads=H, q_heads=Hq, seq=T + 1, tokens=T + 1)
    k1 = to_device(np.ascontiguousarray(w.kv(0)[:, :, T:T + 1]))
    v1 = to_device(np.ascontiguousarray(w.kv(1)[:, :, T:T + 1]))
    qd = to_device(q)
    pos = i32_device([T] * B)
    append = mode != "mixed"  # (the chunk-mixed cache is full: decode alone)
    max_len = T + 1 if append else T
    lens = i32_device([max_len, T - 57])
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws, n = cache.workspace(Hq, max_len, 0)
    if mode == "dsq":
        score1 = torch.from_numpy(np.ascontiguousarray(w.scores()[:, :, T:T + 1])).cuda()

    def step():
        if mode == "dsq":
            K.kvq_dsq_append(cache.desc, k1, v1, score1, 1, pos)
        elif append:
            K.kvq_quant_append(cache.desc, k1, v1, 1, pos)
        if noalloc:
            K.kvq_decode_attn_noalloc(cache.desc, qd, Hq, lens, max_len, SM, out, 0)
        else:
            K.kvq_decode_attn(cache.desc, qd, Hq, lens, max_len, SM, out, ws, n, 0)

    step()
    torch.cuda.synchronize()
    assert cache.flags() == 0
    ref = out.cpu().numpy().copy()
    assert np.isfinite(ref).all()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # a warm-up on the side stream, as torch's capture recipe asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        out.fill_(float("nan"))
        scratch.mul_(1.0001)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (mode, rep)
        assert cache.flags() == 0

"""Decode determinism and split invariance for every codec and cache mode.

Two decodes of the same cache with the same split count must agree bit for
bit (no atomics whose order varies between runs may touch the output);
decodes with different split counts merge the same per-split results by the
log-sum-exp rule of the Cocktail page (§3.2.3, per-block attention merged
equals attention over the whole sequence), so they agree with the unsplit
decode to binary32 rounding.  That agreement is bounded by half the 1e-4
implementation bar: each split count changes the running-maximum frames, the
rounding of every exp2 and of the fp16 hi / lo weight split, and the order of
the binary32 sums, which moves a row by a few 1e-6 to 2e-5 at 1000 tokens
(per-row relative to max|o|); a merge mistake (a split dropped or counted
twice) moves it by at least ~1/16.
"""
import numpy as np
import pytest

import synth
from kvq_harness import ATTN_TIGHT, i32_device, rel_err_rows, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("quantized_kv_cache_05_amd")

SM = 1.0 / np.sqrt(128.0)
SPLIT_BAR = ATTN_TIGHT / 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.lib()
    yield


def decode(cache, q, Hq, lens, max_len, ns):
    B = q.shape[0]
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws, n = cache.workspace(Hq, max_len, ns)
    K.kvq_decode_attn(cache.desc, to_device(q), Hq, i32_device(lens) if lens is not None else None, max_len,
                      SM, out, ws, n, ns)
    torch.cuda.synchronize()
    assert cache.flags() == 0
    return out.cpu().numpy()


def build(mode, G):
    """(cache, q, Hq, lens, max_len) of a small seeded cache of the given mode."""
    B, H, T, S = 2, 2, 1000, 1024
    if mode == "dsq":
        T = 960
    wl = {"oaken": 5, "paged_oaken": 5, "channel4": 3, "channel8": 3, "mixed": 4, "dsq": 8}.get(mode, 2)
    w = synth.scaled(synth.WORKLOADS[wl], batch=B, kv_heads=H, q_heads=H * G, seq=T, tokens=T)
    k, v, q = w.kv(0), w.kv(1), w.q()
    pos0 = i32_device([0] * B)
    lens = [T, T - 123]
    if mode.startswith("uniform"):
        _, bits, sym, group = mode.split("_")
        cache = K.QuantKVCache(B, H, S, K.KVQ_MODE_UNIFORM, k_bits=int(bits), symmetric=sym == "s",
                               k_group=int(group))
    elif mode in ("e4m3", "e5m2"):
        cache = K.QuantKVCache(B, H, S, K.KVQ_MODE_UNIFORM, k_bits=8, k_group=64,
                               fmt=K.KVQ_FMT_E4M3 if mode == "e4m3" else K.KVQ_FMT_E5M2)
    elif mode.startswith("channel"):
        cache = K.QuantKVCache(B, H, S, K.KVQ_MODE_UNIFORM, k_bits=int(mode[-1]), k_axis=K.KVQ_AXIS_CHANNEL,
                               k_group=64, v_group=64)
        lens = [T, 896]
    elif mode == "paged8":
        order = np.random.default_rng(3).permutation(B * (S // 64) + 5)[:B * (S // 64)].astype(np.int32)
        cache = K.QuantKVCache(B, H, S, K.KVQ_MODE_UNIFORM, k_bits=8, symmetric=True, k_group=128,
                               page_tokens=64, num_pages=B * (S // 64) + 5,
                               block_table=torch.from_numpy(order.reshape(B, -1)).cuda())
    elif mode in ("oaken", "paged_oaken"):
        thr = np.array([-1.59, -0.625, 0.625, 1.59], np.float32)
        kw = {}
        if mode == "paged_oaken":
            order = np.random.default_rng(4).permutation(B * (S // 64)).astype(np.int32)
            kw = dict(page_tokens=64, num_pages=B * (S // 64),
                      block_table=torch.from_numpy(order.reshape(B, -1)).cuda())
        cache = K.QuantKVCache(B, H, S, K.KVQ_MODE_OAKEN, k_bits=4, k_group=64, k_thr=thr, v_thr=thr,
                               sparse_cap=S * 24, **kw)
    elif mode == "mixed":
        C = S // 32
        bits = np.random.default_rng(5).choice(np.array([16, 4, 2], np.uint8), size=(B, C), p=[0.2, 0.4, 0.4])
        w = synth.scaled(synth.WORKLOADS[4], batch=B, kv_heads=H, q_heads=H * G, seq=S, tokens=S, emb_dim=64)
        k, v, q = w.kv(0), w.kv(1), w.q()
        cache = K.QuantKVCache(B, H, S, K.KVQ_MODE_CHUNK_MIXED, k_group=32, chunk_tokens=32)
        K.kvq_reorder_chunks(cache.desc, torch.from_numpy(bits).cuda(), C)
        K.kvq_quant_append(cache.desc, to_device(k), to_device(v), S, pos0)
        return cache, q, H * G, None, S
    elif mode == "dsq":
        cache = K.QuantKVCache(B, H, S, K.KVQ_MODE_DSQ, k_group=32, v_group=32, dsq_sig=13)
        K.kvq_dsq_append(cache.desc, to_device(k), to_device(v), torch.from_numpy(w.scores()).cuda(), T, pos0)
        return cache, q, H * G, [T, 832], T
    else:
        raise ValueError(mode)
    K.kvq_quant_append(cache.desc, to_device(k), to_device(v), T, pos0)
    return cache, q, H * G, lens, T


MODES = ["uniform_8_s_128", "uniform_8_a_64", "uniform_4_a_64", "uniform_4_a_32", "uniform_2_a_128",
         "e4m3", "e5m2", "channel4", "channel8", "paged8", "oaken", "paged_oaken", "mixed", "dsq"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("G", [1, 4])
def test_run_twice_and_split_invariance(mode, G):
    print("case determinism %s G=%d" % (mode, G), flush=True)
    cache, q, Hq, lens, max_len = build(mode, G)
    torch.cuda.synchronize()
    assert cache.flags() == 0
    a = decode(cache, q, Hq, lens, max_len, 1)
    b = decode(cache, q, Hq, lens, max_len, 1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "two runs differ"
    for ns in (0, 2, 4, 16):
        c = decode(cache, q, Hq, lens, max_len, ns)
        d = decode(cache, q, Hq, lens, max_len, ns)
        assert np.array_equal(c.view(np.uint32), d.view(np.uint32)), "two runs differ at %d splits" % ns
        err = float(rel_err_rows(c, a).max())
        print("  splits %d vs 1: %.2e" % (ns, err), flush=True)
        assert err <= SPLIT_BAR, (mode, ns)

"""GPU parity of the FP8 caches, E4M3 and E5M2 (uniform mode, token-axis groups).

Codes and scales must equal the oracle's bit for bit; attention within the
bar.  The encoders are also checked exhaustively: groups whose largest
magnitude is the format's largest finite value (448, 57344) have scale
exactly 1, so every finite fp16 value up to it in magnitude is encoded as
itself and compared with the oracle's encoding.
"""
import numpy as np
import pytest

import oracle
import synth
from kvq_harness import ATTN_BAR, ATTN_TIGHT, host_bytes, i32_device, rel_err_rows, to_device, unpack_layout

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("quantized_kv_cache_05_amd")

SM = 1.0 / np.sqrt(128.0)
LAYOUT = {"k": "K", "v": "V"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.lib()
    yield


def f32bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


# format name -> (format id, oracle quantizer, oracle dequantizer, oracle encoder, largest finite value)
FORMATS = {
    "e4m3": (1, oracle.quant_rows_e4m3, oracle.dequant_rows_e4m3, oracle.e4m3_encode, 448.0),
    "e5m2": (2, oracle.quant_rows_e5m2, oracle.dequant_rows_e5m2, oracle.e5m2_encode, 57344.0),
}


def fp8_cache(B, H, S, group, fmt="e4m3"):
    return K.QuantKVCache(B, H, S, K.KVQ_MODE_UNIFORM, k_bits=8, k_group=group, fmt=FORMATS[fmt][0])


def device_codes(cache, name, B, H, S, group):
    codes = unpack_layout(host_bytes(cache.buf(name + ".codes")).reshape(B, H, S, 128), 8, LAYOUT[name])
    scale = host_bytes(cache.buf(name + ".scale")).view(np.float32).reshape(B, H, S, 128 // group)
    return codes, scale


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_fp8_uniform(group, G, fmt):
    B, H, T, S = 2, 3, 333, 384
    print("case %s group=%d G=%d" % (fmt, group, G), flush=True)
    _, quant, dequant, _, _ = FORMATS[fmt]
    w = synth.scaled(synth.WORKLOADS[1], batch=B, kv_heads=H, q_heads=H * G, seq=T, tokens=T)
    k, v, q = w.kv(0), w.kv(1), w.q()
    cache = fp8_cache(B, H, S, group, fmt)
    K.kvq_quant_append(cache.desc, to_device(k), to_device(v), T, i32_device([0] * B))
    torch.cuda.synchronize()
    assert cache.flags() == 0
    deq = {}
    for name, x in (("k", k), ("v", v)):
        oc, os_ = quant(x, group)
        gc, gs = device_codes(cache, name, B, H, S, group)
        assert np.array_equal(gc[:, :, :T], oc), name + " codes"
        assert np.array_equal(f32bits(gs[:, :, :T]), f32bits(os_)), name + " scales"
        deq[name] = dequant(oc, os_, group)
    seq_len = [T, T - 77]
    for ns in (0, 1, 3):
        out = torch.full((B, H * G, 128), float("nan"), dtype=torch.float32, device="cuda")
        ws, n = cache.workspace(H * G, T, ns)
        K.kvq_decode_attn(cache.desc, to_device(q), H * G, i32_device(seq_len), T, SM, out, ws, n, ns)
        torch.cuda.synchronize()
        refs = np.stack([oracle.attention(q[b], deq["k"][b][:, :L], deq["v"][b][:, :L], SM)
                         for b, L in enumerate(seq_len)])
        err = float(rel_err_rows(out.cpu().numpy(), refs).max())
        print("%s g%d G%d ns%d: max rel err %.3e" % (fmt, group, G, ns, err), flush=True)
        assert err <= ATTN_BAR and err <= ATTN_TIGHT


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_encoder_every_f16_value(fmt):
    """Every finite fp16 value of magnitude <= the format's largest, in groups of 32 led by it
    (scale 1)."""
    print("case %s exhaustive encoder" % fmt, flush=True)
    _, _, _, encode, top = FORMATS[fmt]
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = h.view(np.float16).astype(np.float32)
    vals = h[np.isfinite(f) & (np.abs(f) <= top)]
    per = 31
    n_groups = -(-vals.size // per)
    payload = np.zeros(n_groups * per, np.uint16)
    payload[:vals.size] = vals
    groups = np.concatenate([np.full((n_groups, 1), np.float16(top).view(np.uint16), np.uint16),
                             payload.reshape(n_groups, per)], axis=1)
    rows = -(-n_groups // 4)
    x = np.zeros((rows * 4, 32), np.uint16)
    x[:n_groups] = groups
    x[n_groups:, 0] = np.float16(top).view(np.uint16)
    x = x.reshape(1, 1, rows, 128)
    S = (rows + 63) // 64 * 64
    cache = fp8_cache(1, 1, S, 32, fmt)
    K.kvq_quant_append(cache.desc, to_device(x), to_device(x), rows, i32_device([0]))
    torch.cuda.synchronize()
    assert cache.flags() == 0
    want = encode(x.view(np.float16).astype(np.float32))
    for name in ("k", "v"):
        gc, gs = device_codes(cache, name, 1, 1, S, 32)
        assert np.all(gs[0, 0, :rows] == 1.0)
        assert np.array_equal(gc[:, :, :rows], want), name

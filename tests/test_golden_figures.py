"""The figures the pages print (tests/golden/page_figures.txt, each line
citing its page and section) against the byte calculator, the library's
constants and the oracle.  No GPU."""
import os

import numpy as np

import oracle
import quantized_kv_cache_05_amd as K
from test_abi import make_desc

HERE = os.path.dirname(os.path.abspath(__file__))


def figures():
    out = {}
    with open(os.path.join(HERE, "golden", "page_figures.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (x.strip() for x in line.split("=", 1))
                out[k] = float(v)
    return out


def test_turboquant_size_example_through_the_byte_calculator():
    f = figures()
    layers, H, D, S = 32, 32, 128, 131072
    # an fp16 chunk-mixed cache whose every chunk is FP16 stores 2 bytes per element
    c = make_desc(B=1, H=H, S=S, bits=4, group=64)
    b = K.kvq_cache_bytes(c)
    int4_bytes = sum(getattr(t, n) for t in (b.k, b.v) for n in K.TENSOR_BUFFERS) * layers
    elements = 2 * layers * H * D * S
    assert elements == int(f["turboquant_8b_128k_elements"])
    assert abs(elements * 2 / 1e9 - f["turboquant_8b_128k_fp16_gb"]) < 0.05
    # INT4 with groups of 64: half a byte per element and 5 bytes per group
    assert int4_bytes == elements // 2 + elements // int(f["oaken_group_size"]) * 5


def test_kvo_llm_size_example():
    f = figures()
    per_token = 2 * f["kvo_hidden"] * f["kvo_bytes_per_value"]
    assert per_token == f["kvo_kb_per_token"] * 1024
    per_seq = per_token * f["kvo_context_tokens"]
    assert per_seq == f["kvo_gb_per_sequence"] * 2 ** 30
    assert per_seq * f["kvo_batch"] == f["kvo_gb_total"] * 2 ** 30


def test_oaken_region_shares_are_the_calibration_percentiles():
    f = figures()
    lo_o, lo_i, hi_i, hi_o = (p / 100.0 for p in K.OAKEN_PERCENTILES_BP)
    assert abs((lo_o + (100 - hi_o)) - f["oaken_outer_pct"]) < 1e-9
    assert abs(((lo_i - lo_o) + (hi_o - hi_i)) - f["oaken_middle_pct"]) < 1e-9
    assert abs((hi_i - lo_i) - f["oaken_inner_pct"]) < 1e-9
    assert list(K.OAKEN_PERCENTILES_BP) == list(oracle.OAKEN_PERCENTILES_BP)


def test_cocktail_thresholds_constants():
    f = figures()
    assert K.COCKTAIL_ALPHA == f["cocktail_alpha"] and K.COCKTAIL_BETA == f["cocktail_beta"]
    # the oracle's defaults are the same constants: similarities 0 and 1 fix the
    # range, the others sit between the tenths so that no tie decides a class
    sims = np.concatenate([[0.0, 1.0], np.arange(0.05, 1.0, 0.1)])
    q = np.array([1.0, 0.0])
    c = np.stack([np.array([s, np.sqrt(1 - s * s)]) for s in sims])
    bits, got = oracle.chunk_bits(q, c)
    assert np.allclose(got, sims)
    # T_low = 0.6, T_high = 0.9: above 0.9 -> 16, (0.6, 0.9] -> 4, else 2
    expect = [16 if s > 0.9 else (4 if s > 0.6 else 2) for s in sims]
    assert [int(v) for v in bits] == expect


def test_int8_symmetric_levels():
    f = figures()
    x = np.array([[0x3C00] * 127 + [0xBC00]], np.uint16)  # 1.0 ... , -1.0
    codes, scale, _ = oracle.quant_rows(x, 128, 8, True)
    assert scale[0, 0] == np.float32(1.0) / np.float32(f["int8_sym_levels"])
    assert codes.min() == -127 and codes.max() == 127

#!/usr/bin/env python
"""Benchmark of the quantized KV-cache hot path on one MI355X.

Workload: Llama-2-7B-shaped attention layer, batch 16, 32 MHA heads,
head_dim 128, 4096 cached tokens + 1 appended, fp16 K/V ~ N(0, 1) with 4
outlier channels per (tensor, head) scaled x15, INT8 symmetric per token and
head (scale = amax / 127).  One step = quantize-append of 1 token per
sequence (K and V) followed by one decode query per head over the 4097
cached tokens (fused-dequant split decode + log-sum-exp merge).

Prints one JSON line: value = algorithmic bytes of the step (packed cache +
metadata read, q read, output written, appended token read and written) per
second of step time, in GB/s; roofline = the decode call alone against the
8 TB/s HBM peak; quantize-append throughput (bulk prefill and per-step
append) in tokens/s, a token being one sequence position across all KV heads,
K and V; cpu_baseline = the CPU oracle on a bounded sample of the same work.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn packed-KV GB/s (% of HBM peak) + quantize-append tokens/s"
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--num-splits", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--quiet", action="store_true")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="run one plain device copy of this size first (HBM counter calibration)")
    return p.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def decode_bytes(B, H, Hq, L):
    codes = 2 * B * H * L * 128          # INT8 K and V codes
    scales = 2 * B * H * L * 4           # fp32 scale per token and head, K and V
    q = B * Hq * 128 * 2
    out = B * Hq * 128 * 4
    return codes + scales + q + out


def append_bytes(B, H, t):
    return 2 * B * H * t * (128 * 2 + 128 + 4)  # fp16 in, int8 codes + fp32 scale out, K and V


def cpu_baseline(w, budget_s, args):
    """The oracle (single thread) on whole (b, h) slices until the time budget is spent."""
    import numpy as np
    import oracle

    t_quant = t_dec = 0.0
    slices = 0
    qall = w.q()
    L = w.seq
    sm = 1.0 / np.sqrt(128.0)
    start = time.perf_counter()
    for b in range(w.batch):
        for h in range(w.kv_heads):
            k = w.kv(0, b, b + 1, h, h + 1)
            v = w.kv(1, b, b + 1, h, h + 1)
            t0 = time.perf_counter()
            kc, ks, _ = oracle.quant_rows(k, 128, 8, True)
            vc, vs, _ = oracle.quant_rows(v, 128, 8, True)
            t1 = time.perf_counter()
            kh = oracle.dequant_rows(kc, ks, None, 128, True)[0]
            vh = oracle.dequant_rows(vc, vs, None, 128, True)[0]
            oracle.attention(qall[b, h:h + 1], kh, vh, sm)
            t2 = time.perf_counter()
            t_quant += t1 - t0
            t_dec += t2 - t1
            slices += 1
            if time.perf_counter() - start > budget_s:
                break
        else:
            continue
        break
    dec_bytes = slices * 2 * L * (128 + 4) + slices * (128 * 2 + 128 * 4)
    log(args, "cpu oracle: %d slices, quant %.2fs, decode %.2fs" % (slices, t_quant, t_dec))
    return {
        "value": dec_bytes / t_dec / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "%d of %d (batch, kv-head) slices, %d tokens each: INT8 quantize + dequant + "
                  "binary64 attention, single thread" % (slices, w.batch * w.kv_heads, L),
        "quant_tokens_per_s": slices * L / w.kv_heads / t_quant,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only (--gpus 1); multi-GPU runs are not part of this build",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import quantized_kv_cache_05_amd as K
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from kvq_harness import i32_device, to_device

    torch.cuda.set_device(0)
    w = synth.WORKLOADS[2]
    B, H, Hq, L = w.batch, w.kv_heads, w.q_heads, w.seq  # L = 4097
    T0 = L - 1
    S = (L + 63) // 64 * 64
    log(args, "generating inputs ...")
    t = time.perf_counter()
    k = w.kv(0)
    v = w.kv(1)
    q = w.q()
    log(args, "inputs ready in %.1fs" % (time.perf_counter() - t))
    k_bulk = to_device(np.ascontiguousarray(k[:, :, :T0]))
    v_bulk = to_device(np.ascontiguousarray(v[:, :, :T0]))
    k_new = to_device(np.ascontiguousarray(k[:, :, T0:]))
    v_new = to_device(np.ascontiguousarray(v[:, :, T0:]))
    q_dev = to_device(q)
    del k, v
    cache = K.QuantKVCache(B, H, S, K.KVQ_MODE_UNIFORM, k_bits=8, symmetric=True, k_group=128)
    pos0 = i32_device([0] * B)
    pos_app = i32_device([T0] * B)
    seq_len = i32_device([L] * B)
    out = torch.empty(B, Hq, 128, dtype=torch.float32, device="cuda")
    ws, ws_bytes = cache.workspace(Hq, L, args.num_splits)
    sm = 1.0 / np.sqrt(128.0)
    stream = torch.cuda.current_stream()

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # bulk prefill quantize (also fills the cache)
    for _ in range(2):
        K.kvq_quant_append(cache.desc, k_bulk, v_bulk, T0, pos0)
    torch.cuda.synchronize()
    reps = 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        K.kvq_quant_append(cache.desc, k_bulk, v_bulk, T0, pos0)
    e1.record(stream)
    torch.cuda.synchronize()
    bulk_ms = e0.elapsed_time(e1) / reps
    bulk_tok_s = B * T0 / (bulk_ms / 1e3)
    log(args, "bulk quantize %d x %d tokens: %.3f ms, %.3e tok/s" % (B, T0, bulk_ms, bulk_tok_s))

    def step(ev_a=None, ev_b=None):
        K.kvq_quant_append(cache.desc, k_new, v_new, 1, pos_app)
        if ev_a is not None:
            ev_a.record(stream)
        K.kvq_decode_attn(cache.desc, q_dev, Hq, seq_len, L, sm, out, ws, ws_bytes, args.num_splits)
        if ev_b is not None:
            ev_b.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert cache.flags() == 0, "device status flags %#x" % cache.flags()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s0.record(stream)
    for a, b in evs:
        step(a, b)
    s1.record(stream)
    torch.cuda.synchronize()
    step_ms = s0.elapsed_time(s1) / args.steps
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    dbytes = decode_bytes(B, H, Hq, L)
    abytes = append_bytes(B, H, 1)
    value = (dbytes + abytes) / (step_ms / 1e3) / 1e9
    achieved = dbytes / (dec_ms / 1e3) / 1e9
    append_tok_s = B / ((step_ms - dec_ms) / 1e3) if step_ms > dec_ms else None
    log(args, "step %.4f ms, decode %.4f ms -> %.1f GB/s (%.1f%% of peak)"
        % (step_ms, dec_ms, achieved, 100 * achieved / HBM_PEAK_GBS))

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, args.cpu_seconds, args)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "llama2-7b-layer-int8: batch 16, 32 MHA heads, head_dim 128, 4096 cached + 1 "
                        "appended token, INT8 symmetric per token and head; step = append 1 token per "
                        "sequence + 1 decode query per head",
            "batch": B, "kv_heads": H, "q_heads": Hq, "seq_len": L, "num_splits": args.num_splits,
        },
        "decode_ms": round(dec_ms, 5),
        "decode_gbs": round(achieved, 1),
        "pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "quant_bulk_tokens_per_s": round(bulk_tok_s, 1),
        "quant_bulk_ms": round(bulk_ms, 4),
        "quant_append_tokens_per_s": round(append_tok_s, 1) if append_tok_s else None,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python
"""Benchmark of the quantized KV-cache hot path on one MI355X.

Workloads (seeded synthetic fp16 K/V, head_dim 128; ``--workload N``):
  1 tiny      batch 1, 1 head, 1024 tokens, INT4 asymmetric groups of 64
              along head_dim; step = quantize all 1024 tokens + 1 decode query
  2 llama2    (default) batch 16, 32 MHA heads, 4096 cached + 1 appended
              token, INT8 symmetric per token and head; step = append 1 token
              per sequence + 1 decode query per head over 4097 tokens
  3 gqa128k   batch 1, 32 query / 8 KV heads, 131072 tokens, INT4, K per
              channel over 64-token blocks, V groups of 64 along head_dim;
              step = 1 split-sequence decode query per head (4 cache copies
              rotate so that the 256 MB last-level cache cannot hold the
              working set)
  4 cocktail  batch 8, 40 heads, 32768 tokens in 32-token chunks classed
              FP16 / INT4 / INT2 (groups of 32) by query-chunk cosine
              similarity and reordered contiguous by class; step = 1 chunked
              decode query per head
  5 oaken     (default) batch 256, 40 heads, 2048 tokens of 0.5 * Student-t(3);
              thresholds from a 100-sequence calibration set; dense INT4 +
              sparse shifted outer values; step = append 1 token per
              sequence + 1 decode query per head
  6 e4m3      workload 2's shapes and inputs with FP8 E4M3 codes, one scale
              (max|x| / 448) per token and head
  7 paged     workload 2 in a paged cache: pages of 64 tokens handed out in a
              seeded random order from one pool, read through a block table
  9 e5m2      workload 2's shapes with FP8 E5M2 codes, one scale
              (max|x| / 57344) per token and head
  8 dsq       batch 16, 32 MHA heads, 4096 tokens (workload 2's distribution)
              in KVO-LLM's differential significant-token cache: per 64-token
              group the 13 tokens with the largest seeded scores (exp N(0,1))
              INT8 per channel, the other 51 INT2 in groups of 32 (K as the
              difference from the significant mean); step = 1 decode query
              per head

Prints one JSON line for the headline workload (--workload, default 5, the
largest configuration), with configurations 1-5 each measured in the same run
and summarized under "configs" (--headline-only skips them).  value =
algorithmic bytes of a step (packed cache and metadata read by decode, query
read, output written, appended tokens read and written) per second of step
time, in GB/s.  roofline = the decode kernel
alone: its algorithmic bytes over its average duration (HIP events on the
stream it runs on) against the 8 TB/s HBM peak.  Quantize throughput is in
tokens/s, a token being one sequence position over all KV heads, K and V.
cpu_baseline = the CPU oracle on a bounded sample of the same work, single
thread and all threads.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn packed-KV GB/s (% of HBM peak) + quantize-append tokens/s"
HBM_PEAK_GBS = 8000.0
SM_SCALE = 1.0 / math.sqrt(128.0)
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5, 6, 7, 8, 9],
                   help="the workload of the headline value (default 5, the largest configuration)")
    p.add_argument("--headline-only", action="store_true",
                   help="measure the headline workload only (by default configurations 1-5 are all "
                        "measured and reported under 'configs')")
    p.add_argument("--num-splits", type=int, default=0)
    p.add_argument("--page-tokens", type=int, default=0, choices=[0, 64, 128, 256],
                   help="workloads 3 and 4: the same cache in the paged layout (tokens per page)")
    p.add_argument("--cpu-seconds", type=float, default=16.0,
                   help="budget of the CPU-oracle leg (half single-threaded, half all threads)")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--quiet", action="store_true")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="run one plain device copy of this size first (HBM counter calibration)")
    p.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "BENCH_LOG"),
                   help="no GPU work: turn the counter CSVs of two rocprofv3 --pmc runs of this "
                        "script (FETCH_SIZE, then WRITE_SIZE, both with --copy-probe-mib) and the "
                        "bench line printed by one of them into a traffic summary on stdout")
    p.add_argument("--summarize-busy", nargs=3, metavar=("COUNTER_CSV", "AGENT_CSV", "BENCH_LOG"),
                   help="print VALU / MFMA busy fractions from a rocprofv3 --pmc run of BUSY_COUNTERS")
    p.add_argument("--summarize-stats", nargs=2, metavar=("KERNEL_STATS_CSV", "BENCH_LOG"),
                   help="no GPU work: summarize a rocprofv3 --kernel-trace --stats run of this "
                        "script (its kernel_stats.csv and the output it printed) on stdout")
    return p.parse_args()


ARGS = None


def log(*a):
    if not ARGS.quiet:
        print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# inputs

def upload_kv(w, tensor, torch, chunk_bytes=512 << 20):
    """Device int16 [B][H][T][128] holding the fp16 bits of K (0) or V (1), generated per batch slice."""
    B, H, T = w.batch, w.kv_heads, w.tokens
    out = torch.empty((B, H, T, 128), dtype=torch.int16, device="cuda")
    per = max(1, chunk_bytes // (H * T * 128 * 2))
    for b0 in range(0, B, per):
        b1 = min(B, b0 + per)
        host = w.kv(tensor, b0, b1)
        out[b0:b1].copy_(torch.from_numpy(host.view("int16")))
    return out


def i32(torch, vals):
    import numpy as np
    return torch.tensor(np.asarray(vals, dtype=np.int32), dtype=torch.int32, device="cuda")


# ---------------------------------------------------------------------------
# workloads: each sets up device state and exposes prefill(), step(), byte counts

class Workload:
    rotate = 1

    def __init__(self, w, torch, K):
        self.w, self.torch, self.K = w, torch, K
        self.q = None
        self.out = torch.empty((w.batch, w.q_heads, 128), dtype=torch.float32, device="cuda")

    # decode over cache copy r
    def decode(self, r):
        c = self.caches[r]
        self.K.kvq_decode_attn(c.desc, self.q, self.w.q_heads, self.seq_len, self.max_len, SM_SCALE,
                               self.out, self.ws[r][0], self.ws[r][1], ARGS.num_splits)

    def make_workspaces(self):
        self.ws = [c.workspace(self.w.q_heads, self.max_len, ARGS.num_splits) for c in self.caches]

    def append(self, r):
        pass

    def append_bytes(self):
        return 0

    def flags(self):
        return [c.flags() for c in self.caches]


def page_tables(torch, w, page, tables):
    """Paged layout for a workload: `tables` block tables (one per precision class of a chunk-mixed
    cache) mapping every logical page of every sequence to a page of a pool of batch * pages-per-
    sequence pages, in a seeded random order.  Returns the cache keywords and the table bytes the
    decode workgroups read (an upper bound for chunk-mixed caches, whose classes share the rows)."""
    if not page:
        return {}, 0
    import numpy as np
    B, H, T = w.batch, w.kv_heads, w.tokens
    n = -(-T // page)
    rng = np.random.default_rng(w.seed + page)
    order = np.stack([rng.permutation(B * n).astype(np.int32) for _ in range(tables)])
    kw = dict(page_tokens=page, num_pages=B * n, block_table=torch.from_numpy(order.reshape(-1)).cuda())
    return kw, B * H * n * 4


class UniformToken(Workload):
    """Workloads 1, 2, 6 and 7: token-axis groups, optional 1-token append per step."""

    def __init__(self, w, torch, K, bits, sym, group, append, fmt=0, page=0):
        super().__init__(w, torch, K)
        self.bits, self.sym, self.group, self.app, self.fmt = bits, sym, group, append, fmt
        B, H, T = w.batch, w.kv_heads, w.tokens
        self.T0 = T - 1 if append else T
        S = (T + 63) // 64 * 64
        paging = {}
        self.table_bytes = 0
        if page:
            import numpy as np
            S = (T + page - 1) // page * page
            n = S // page
            order = np.random.default_rng(w.seed).permutation(B * n).astype(np.int32)
            paging = dict(page_tokens=page, num_pages=B * n,
                          block_table=torch.from_numpy(order.reshape(B, n)).cuda())
            self.table_bytes = B * H * (-(-T // page)) * 4  # entries read by the decode workgroups
        kx, vx = upload_kv(w, 0, torch), upload_kv(w, 1, torch)
        self.k_pre = kx[:, :, :self.T0].contiguous()
        self.v_pre = vx[:, :, :self.T0].contiguous()
        if append:
            self.k_new = kx[:, :, self.T0:].contiguous()
            self.v_new = vx[:, :, self.T0:].contiguous()
        del kx, vx
        self.caches = [K.QuantKVCache(B, H, S, K.KVQ_MODE_UNIFORM, k_bits=bits, symmetric=sym,
                                      k_group=group, fmt=fmt, **paging)]
        self.q = torch.from_numpy(w.q().view("int16")).cuda()
        self.pos0 = i32(torch, [0] * B)
        self.pos_app = i32(torch, [self.T0] * B)
        self.seq_len = i32(torch, [T] * B)
        self.max_len = T
        self.make_workspaces()
        self.prefill_tokens = B * self.T0

    def prefill(self, r=0):
        self.K.kvq_quant_append(self.caches[r].desc, self.k_pre, self.v_pre, self.T0, self.pos0)

    def append(self, r):
        if self.app:
            self.K.kvq_quant_append(self.caches[r].desc, self.k_new, self.v_new, 1, self.pos_app)
        else:  # the tiny workload quantizes its whole sequence every step
            self.prefill(r)

    def row_bytes(self):
        ng = 128 // self.group
        return 128 * self.bits // 8 + ng * 4 + (0 if (self.sym or self.fmt) else ng)

    def decode_bytes(self):
        w = self.w
        return (2 * w.batch * w.kv_heads * w.tokens * self.row_bytes()
                + w.batch * w.q_heads * 128 * (2 + 4) + self.table_bytes)

    def append_bytes(self):
        w = self.w
        t = 1 if self.app else self.T0
        return 2 * w.batch * w.kv_heads * t * (256 + self.row_bytes())


class ChannelK(Workload):
    """Workload 3: K per channel over 64-token blocks, V token groups of 64, GQA."""

    def __init__(self, w, torch, K, page=0):
        super().__init__(w, torch, K)
        B, H, T = w.batch, w.kv_heads, w.tokens
        self.kx, self.vx = upload_kv(w, 0, torch), upload_kv(w, 1, torch)
        paging, self.table_bytes = page_tables(torch, w, page, 1)
        one = K.QuantKVCache(B, H, T, K.KVQ_MODE_UNIFORM, k_bits=4, k_axis=K.KVQ_AXIS_CHANNEL,
                             k_group=64, v_group=64, **paging)
        self.rotate = max(1, min(8, -(-2 * MALL_BYTES // one.total_bytes)))
        self.caches = [one] + [K.QuantKVCache(B, H, T, K.KVQ_MODE_UNIFORM, k_bits=4,
                                              k_axis=K.KVQ_AXIS_CHANNEL, k_group=64, v_group=64, **paging)
                               for _ in range(self.rotate - 1)]
        self.q = torch.from_numpy(w.q().view("int16")).cuda()
        self.pos0 = i32(torch, [0] * B)
        self.seq_len = i32(torch, [T] * B)
        self.max_len = T
        self.make_workspaces()
        self.prefill_tokens = B * T

    def prefill(self, r=0):
        self.K.kvq_quant_append(self.caches[r].desc, self.kx, self.vx, self.w.tokens, self.pos0)

    def decode_bytes(self):
        w = self.w
        rows = w.batch * w.kv_heads * w.tokens
        k = rows * 64 + (rows // 64) * 128 * 5
        v = rows * (64 + 2 * 5)
        return k + v + w.batch * w.q_heads * 128 * (2 + 4) + self.table_bytes


class Cocktail(Workload):
    """Workload 4: chunk precision search, reorder, class pools, chunked decode."""

    def __init__(self, w, torch, K, page=0):
        super().__init__(w, torch, K)
        import numpy as np
        B, H, T, CT = w.batch, w.kv_heads, w.tokens, w.chunk_tokens
        self.C = T // CT
        embs = [w.chunk_embeddings(b) for b in range(B)]
        self.q_emb = torch.from_numpy(np.stack([e[0] for e in embs])).cuda()
        self.c_emb = torch.from_numpy(np.stack([e[1] for e in embs])).cuda()
        self.bits = torch.zeros((B, self.C), dtype=torch.uint8, device="cuda")
        self.kx, self.vx = upload_kv(w, 0, torch), upload_kv(w, 1, torch)
        paging, self.table_bytes = page_tables(torch, w, page, 3)
        self.caches = [K.QuantKVCache(B, H, T, K.KVQ_MODE_CHUNK_MIXED, k_group=32, chunk_tokens=CT, **paging)]
        self.q = torch.from_numpy(w.q().view("int16")).cuda()
        self.pos0 = i32(torch, [0] * B)
        self.seq_len = None
        self.max_len = T
        self.make_workspaces()
        self.prefill_tokens = B * T
        self.search()
        torch.cuda.synchronize()

    def search(self):
        w = self.w
        self.K.kvq_chunk_bits(self.q_emb, self.c_emb, w.batch, self.C, w.emb_dim, self.K.COCKTAIL_ALPHA,
                              self.K.COCKTAIL_BETA, self.bits)

    def prefill(self, r=0):
        c = self.caches[r]
        self.K.kvq_reorder_chunks(c.desc, self.bits, self.C)
        self.K.kvq_quant_append(c.desc, self.kx, self.vx, self.w.tokens, self.pos0)

    def seg(self):
        return self.caches[0].buf("seg").cpu().numpy().reshape(self.w.batch, 4)

    def decode_bytes(self):
        w = self.w
        CT, H = w.chunk_tokens, w.kv_heads
        ng = 128 // 32
        total = 0
        for n16, n4, n2, _ in self.seg():
            rows16, rows4, rows2 = n16 * CT, n4 * CT, n2 * CT
            total += 2 * H * (rows16 * 256 + rows4 * (64 + ng * 5) + rows2 * (32 + ng * 5))
            total += 16  # the sequence's segment counts
        return total + w.batch * w.q_heads * 128 * (2 + 4) + self.table_bytes


class Oaken(Workload):
    """Workload 5: calibration, dense INT4 + sparse outer list, 1-token append per step."""

    def __init__(self, w, torch, K):
        super().__init__(w, torch, K)
        B, H, T = w.batch, w.kv_heads, w.tokens
        t = time.perf_counter()
        self.thr = [self.calibrate(0), self.calibrate(1)]
        log("calibration (2 x %d sequences) in %.1fs: K %s V %s" % (
            w.cal_samples, time.perf_counter() - t, self.thr[0], self.thr[1]))
        self.kx, self.vx = upload_kv(w, 0, torch), upload_kv(w, 1, torch)
        self.k_new = self.kx[:, :, T - 1:].contiguous()
        self.v_new = self.vx[:, :, T - 1:].contiguous()
        cap = int(T * 128 * 0.08) // 4 * 4  # outer share ~5 % by construction of the thresholds
        self.caches = [K.QuantKVCache(B, H, T, K.KVQ_MODE_OAKEN, k_bits=4, k_group=64, k_thr=self.thr[0],
                                      v_thr=self.thr[1], sparse_cap=cap)]
        self.q = torch.from_numpy(w.q().view("int16")).cuda()
        self.pos0 = i32(torch, [0] * B)
        self.pos_app = i32(torch, [T - 1] * B)
        self.seq_len = i32(torch, [T] * B)
        self.max_len = T
        self.make_workspaces()
        self.prefill_tokens = B * T

    def calibrate(self, tensor):
        torch, K, w = self.torch, self.K, self.w
        hist = torch.zeros(65536, dtype=torch.int64, device="cuda")
        for s in range(w.cal_samples):
            x = w.calibration(tensor, s)
            K.kvq_hist_f16(torch.from_numpy(x.view("int16")).cuda(), x.size, hist)
        out = torch.zeros(4, dtype=torch.float32, device="cuda")
        K.kvq_hist_percentiles(hist, K.OAKEN_PERCENTILES_BP, out)
        return [float(v) for v in out.cpu()]

    def prefill(self, r=0):
        self.K.kvq_quant_append(self.caches[r].desc, self.kx, self.vx, self.w.tokens, self.pos0)

    def append(self, r):
        self.K.kvq_quant_append(self.caches[r].desc, self.k_new, self.v_new, 1, self.pos_app)

    def entries(self):
        c = self.caches[0]
        T = self.w.tokens
        tot = 0
        for name in ("k", "v"):
            rp = c.buf(name + ".rowptr").view(self.torch.int32).view(-1, T + 1)[:, T]
            tot += int(rp.to(self.torch.int64).sum())
        return tot

    def decode_bytes(self):
        w = self.w
        rows = w.batch * w.kv_heads * w.tokens
        per_row = 64 + 2 * (4 + 1 + 4)  # dense codes, scale, zero-point, outer scale per group
        rowptr = w.batch * w.kv_heads * (w.tokens + 1) * 4
        return 2 * (rows * per_row + rowptr) + 2 * self.entries() + w.batch * w.q_heads * 128 * (2 + 4)

    def append_bytes(self):
        # one token per (b, h) and tensor: fp16 row in; dense codes, group metadata and the row
        # pointer out, plus that row's share of the sparse entries (measured mean)
        w = self.w
        rows = w.batch * w.kv_heads
        per_row_entries = self.entries() / (2 * rows * w.tokens)
        return int(2 * rows * (256 + 64 + 2 * 9 + 4 + 2 * per_row_entries))


DSQ_SIG = 13  # significant tokens per 64-token group (20 % of 64, rounded up)


def dsq_group_bytes(n_sig=DSQ_SIG):
    """Bytes decode reads per 64-token DSQ group and tensor: significant int8 rows, their channel
    scales, the other INT2 rows and their (scale, zero) per 32 channels."""
    n = 64 - n_sig
    return n_sig * 128 + 128 * 4 + n * 32 + n * 4 * 5


class Dsq(Workload):
    """Workload 8: KVO-LLM differential significant-token quantization, decode only per step."""

    def __init__(self, w, torch, K):
        super().__init__(w, torch, K)
        B, H, T = w.batch, w.kv_heads, w.tokens
        self.kx, self.vx = upload_kv(w, 0, torch), upload_kv(w, 1, torch)
        self.sc = torch.from_numpy(w.scores()).cuda()
        self.caches = [K.QuantKVCache(B, H, T, K.KVQ_MODE_DSQ, k_group=32, v_group=32, dsq_sig=DSQ_SIG)]
        self.q = torch.from_numpy(w.q().view("int16")).cuda()
        self.pos0 = i32(torch, [0] * B)
        self.seq_len = i32(torch, [T] * B)
        self.max_len = T
        self.make_workspaces()
        self.prefill_tokens = B * T

    def prefill(self, r=0):
        self.K.kvq_dsq_append(self.caches[r].desc, self.kx, self.vx, self.sc, self.w.tokens, self.pos0)

    def decode_bytes(self):
        w = self.w
        groups = w.batch * w.kv_heads * (w.tokens // 64)
        return 2 * groups * dsq_group_bytes() + w.batch * w.q_heads * 128 * (2 + 4)


def build_workload(idx, torch, K, synth, page=0):
    w = synth.WORKLOADS[idx]
    if page and idx not in (3, 4):
        raise SystemExit("--page-tokens applies to workloads 3 and 4 (workload 7 is the paged INT8 one)")
    if idx == 1:
        return UniformToken(w, torch, K, bits=4, sym=False, group=64, append=False)
    if idx == 2:
        return UniformToken(w, torch, K, bits=8, sym=True, group=128, append=True)
    if idx == 6:
        return UniformToken(w, torch, K, bits=8, sym=False, group=128, append=True, fmt=K.KVQ_FMT_E4M3)
    if idx == 9:
        return UniformToken(w, torch, K, bits=8, sym=False, group=128, append=True, fmt=K.KVQ_FMT_E5M2)
    if idx == 7:
        return UniformToken(w, torch, K, bits=8, sym=True, group=128, append=True, page=64)
    if idx == 3:
        return ChannelK(w, torch, K, page)
    if idx == 4:
        return Cocktail(w, torch, K, page)
    if idx == 8:
        return Dsq(w, torch, K)
    return Oaken(w, torch, K)


WORKLOAD_TEXT = {
    1: "tiny: batch 1, 1 KV head, head_dim 128, 1024 tokens N(0,1) with channels 7 and 93 x20; "
       "INT4 asymmetric groups of 64 along head_dim; step = quantize 1024 tokens + 1 decode query",
    2: "llama2-7b-layer-int8: batch 16, 32 MHA heads, head_dim 128, 4096 cached + 1 appended token, "
       "N(0,1) with 4 outlier channels x15 per head; INT8 symmetric per token and head; "
       "step = append 1 token per sequence + 1 decode query per head",
    3: "llama3-8b-gqa-128k-int4: batch 1, 32 query / 8 KV heads, head_dim 128, 131072 tokens, "
       "N(0,1) with 3 outlier channels x20 per head; INT4 asymmetric, K per channel over 64-token "
       "blocks, V groups of 64; step = 1 split-sequence decode query per head",
    4: "cocktail-13b-mixed: batch 8, 40 heads, head_dim 128, 32768 tokens in 32-token chunks classed "
       "FP16/INT4/INT2 (groups of 32) by 768-d query-chunk cosine similarity (alpha 0.6, beta 0.1), "
       "reordered by class; step = 1 chunked decode query per head",
    5: "oaken-13b-threshold: batch 256, 40 heads, head_dim 128, 2048 tokens of 0.5*t(3); thresholds at "
       "2.5/15/85/97.5 % of a 100-sequence calibration set; dense INT4 groups of 64 + sparse 6-bit "
       "shifted outer values; step = append 1 token per sequence + 1 decode query per head",
    6: "llama2-7b-layer-e4m3: batch 16, 32 MHA heads, head_dim 128, 4096 cached + 1 appended token, "
       "N(0,1) with 4 outlier channels x15 per head; FP8 E4M3 with one scale (max|x| / 448) per token "
       "and head; step = append 1 token per sequence + 1 decode query per head",
    7: "llama2-7b-layer-int8-paged: workload 2 (batch 16, 32 MHA heads, 4096 cached + 1 appended "
       "token, INT8 symmetric per token and head) in a paged cache, 64-token pages in a seeded random "
       "order, block table read by decode; step = append 1 token per sequence + 1 decode query per head",
    9: "llama2-7b-layer-e5m2: batch 16, 32 MHA heads, head_dim 128, 4096 cached + 1 appended token, "
       "N(0,1) with 4 outlier channels x15 per head; FP8 E5M2 with one scale (max|x| / 57344) per token "
       "and head; step = append 1 token per sequence + 1 decode query per head",
    8: "llama2-7b-layer-dsq: batch 16, 32 MHA heads, head_dim 128, 4096 tokens N(0,1) with 4 outlier "
       "channels x15 per head, seeded exp(N(0,1)) token scores; KVO-LLM differential significant-token "
       "quantization: per 64-token group the 13 top-scored tokens INT8 per channel, the other 51 INT2 "
       "in groups of 32 (K as the difference from the significant mean), 1-bit mask; "
       "step = 1 decode query per head",
}


# ---------------------------------------------------------------------------
# CPU oracle leg

def oracle_slice(w, idx, b, h, thr=None):
    """Oracle quantize + dequantize + attention of one (batch, kv head) slice.
    Returns (quantize seconds, decode seconds, decode algorithmic bytes, input generation seconds)."""
    import numpy as np
    import oracle
    tg = time.perf_counter()
    G = w.q_heads // w.kv_heads
    k = w.kv(0, b, b + 1, h, h + 1)[0, 0]
    v = w.kv(1, b, b + 1, h, h + 1)[0, 0]
    q = w.q(b, b + 1)[0, h * G:(h + 1) * G]
    T = w.tokens
    t0 = time.perf_counter()
    if idx in (6, 9):
        q8, dq8 = ((oracle.quant_rows_e4m3, oracle.dequant_rows_e4m3) if idx == 6 else
                   (oracle.quant_rows_e5m2, oracle.dequant_rows_e5m2))
        kc, ks = q8(k, 128)
        vc, vs = q8(v, 128)
        t1 = time.perf_counter()
        kh = dq8(kc, ks, 128)
        vh = dq8(vc, vs, 128)
        nbytes = 2 * T * (128 + 4)
    elif idx in (1, 2, 7):
        bits, sym, g = (4, False, 64) if idx == 1 else (8, True, 128)
        kc, ks, kz = oracle.quant_rows(k, g, bits, sym)
        vc, vs, vz = oracle.quant_rows(v, g, bits, sym)
        t1 = time.perf_counter()
        kh = oracle.dequant_rows(kc, ks, kz, g, sym)
        vh = oracle.dequant_rows(vc, vs, vz, g, sym)
        ng = 128 // g
        nbytes = 2 * T * (128 * bits // 8 + ng * 4 + (0 if sym else ng))
    elif idx == 3:
        kc, ks, kz = oracle.quant_channel_blocks(k, 64, 4)
        vc, vs, vz = oracle.quant_rows(v, 64, 4)
        t1 = time.perf_counter()
        kh = oracle.dequant_channel_blocks(kc, ks, kz, 64)
        vh = oracle.dequant_rows(vc, vs, vz, 64)
        nbytes = T * 64 + (T // 64) * 128 * 5 + T * 74
    elif idx == 8:
        sc = w.scores(b, b + 1)[0, h]
        r = oracle.dsq_quant(k, v, sc, n_sig=DSQ_SIG)
        t1 = time.perf_counter()
        kh, vh = oracle.dsq_dequant(r)
        nbytes = 2 * (T // 64) * dsq_group_bytes()
    elif idx == 4:
        CT = w.chunk_tokens
        bits_c, _ = oracle.chunk_bits(*w.chunk_embeddings(b))
        perm, seg = oracle.reorder(bits_c[None])
        kh = np.zeros((T, 128), np.float32)
        vh = np.zeros((T, 128), np.float32)
        nbytes = 0
        for x, xh in ((k, kh), (v, vh)):
            for c in perm[0]:
                rows = x[c * CT:(c + 1) * CT]
                if bits_c[c] == 16:
                    xh[c * CT:(c + 1) * CT] = rows.view(np.float16).astype(np.float32)
                    nbytes += CT * 256
                else:
                    nb = 4 if bits_c[c] == 4 else 2
                    oc, os_, oz = oracle.quant_rows(rows, 32, nb)
                    xh[c * CT:(c + 1) * CT] = oracle.dequant_rows(oc, os_, oz, 32)
                    nbytes += CT * (128 * nb // 8 + 4 * 5)
        t1 = time.perf_counter()
    else:
        res = []
        for x, tt in ((k, thr[0]), (v, thr[1])):
            res.append(oracle.oaken_rows(x, tt, 64))
        t1 = time.perf_counter()
        kh = oracle.oaken_dequant_rows(*res[0], thr[0], 64)
        vh = oracle.oaken_dequant_rows(*res[1], thr[1], 64)
        nbytes = 2 * (T * (64 + 18) + (T + 1) * 4) + 2 * int(res[0][5].sum() + res[1][5].sum())
    oracle.attention(q, kh[None], vh[None], SM_SCALE)
    t2 = time.perf_counter()
    nbytes += G * 128 * (2 + 4)
    return t1 - t0, t2 - t1, nbytes, t0 - tg


def _oracle_job(idx, b, h, thr):
    import synth
    return oracle_slice(synth.WORKLOADS[idx], idx, b, h, thr=thr)


def cpu_baseline(w, idx, budget_s):
    """The oracle on (batch, kv head) slices: half the budget on one thread, half on worker
    processes (one per available core, at most 16: the host share of one GPU).  Runs before the
    GPU is initialised.  Reports the workers used, the host's core count and CPU model."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor, wait, FIRST_COMPLETED

    import numpy as np
    import oracle
    thr = None
    cal_note = ""
    if idx == 5:
        # thresholds from a reduced calibration set (offline stage, not timed)
        thr = []
        for tensor in (0, 1):
            hist = np.zeros(65536, np.uint64)
            for s in range(2):
                oracle.hist_f16(w.calibration(tensor, s), hist)
            thr.append(oracle.thresholds_from_hist(hist))
        cal_note = "; thresholds from 2 of the 100 calibration sequences"
    slices = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
    rng = np.random.default_rng(0)
    order = [slices[i] for i in rng.permutation(len(slices))]
    # single thread
    tq = td = 0.0
    nb = n1 = 0
    t_start = time.perf_counter()
    while n1 < len(order) and time.perf_counter() - t_start < budget_s / 2:
        a, d, n, _ = oracle_slice(w, idx, *order[n1], thr=thr)
        tq, td, nb, n1 = tq + a, td + d, nb + n, n1 + 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    workers = max(1, min(avail, 16))
    # all cores: worker processes take slices until half the budget has passed
    done = []
    with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
        ex.submit(int, 0).result()  # pay the interpreter start-up before the clock starts
        list(ex.map(int, range(workers)))
        t0 = time.perf_counter()
        pending = set()
        nxt = 0
        while nxt < len(order) and len(pending) < 2 * workers:
            pending.add(ex.submit(_oracle_job, idx, *order[nxt], thr))
            nxt += 1
        while pending:
            fin, pending = wait(pending, return_when=FIRST_COMPLETED)
            done.extend(f.result() for f in fin)
            if time.perf_counter() - t0 < budget_s / 2:
                while nxt < len(order) and len(pending) < 2 * workers:
                    pending.add(ex.submit(_oracle_job, idx, *order[nxt], thr))
                    nxt += 1
        wall = time.perf_counter() - t0
    tq_m = sum(r[0] for r in done)
    td_m = sum(r[1] for r in done)
    nb_m = sum(r[2] for r in done)
    tg_m = sum(r[3] for r in done)
    # the wall time is split between input generation, quantize and attention in proportion to
    # their summed per-slice times; generation is not part of the oracle's rate
    wall_dec = wall * td_m / (tq_m + td_m + tg_m)
    wall_q = wall * tq_m / (tq_m + td_m + tg_m)
    model = "?"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(nb_m / wall_dec / 1e9, 4),
        "unit": "GB/s",
        "cores": workers,
        "host_cores": os.cpu_count(),
        "cores_available": avail,
        "cpu_model": model,
        "kind": "oracle",
        "sample": "%d of %d (batch, kv-head) slices of %d tokens on %d worker processes, %d slices on "
                  "one thread: oracle quantize + dequantize + binary64 attention%s" % (
                      len(done), len(slices), w.tokens, workers, n1, cal_note),
        "single_thread_value": round(nb / td / 1e9, 4),
        "quant_tokens_per_s": round(len(done) * w.tokens / w.kv_heads / wall_q, 1),
        "single_thread_quant_tokens_per_s": round(n1 * w.tokens / w.kv_heads / tq, 1),
    }


# ---------------------------------------------------------------------------
# stored HBM counters of the decode kernel (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)

def code_text(src):
    """C/C++ source without comments and with whitespace collapsed, so that a change to
    comments or layout alone leaves source_hash unchanged (string literals are kept whole)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash():
    """Hash of the code the decode kernels are built from (their headers, the decode
    translation units and the host code that plans their launches), comments and layout
    excluded."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_kv_cache_05_amd", "csrc")
    files = set(glob.glob(os.path.join(csrc, "*.h")) + glob.glob(os.path.join(csrc, "kvq_decode_*.hip")) +
                [os.path.join(csrc, "kvq_api.cpp")])
    for f in sorted(files):
        with open(f, encoding="utf-8") as fh:
            h.update(os.path.basename(f).encode())
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(idx):
    """HBM bytes per decode call from profiles/decode_traffic_w<idx>.txt, if it was taken on the
    current kernel sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", "decode_traffic_w%d.txt" % idx)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash():
        return None
    try:
        return int(float(kv["hbm_bytes_per_call"]))
    except (KeyError, ValueError):
        return None


def decode_kernel(name):
    """The kernels that read the cache in a decode call: the attention kernel and, for Oaken,
    the K outer-value score kernel that runs before it (the split merge reads only partials)."""
    return "k_attn_" in name or "k_oak_kscore" in name


def summarize_pmc(fetch_csv, write_csv, bench_log, copy_mib):
    """Per-call HBM bytes of the decode kernels (decode_kernel) from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), summed over the kernels of one call.  Each counter is scaled by what it
    reads for the plain copy of copy_mib MiB that the same run made (the largest copy
    dispatch): bytes moved / counter KiB."""
    import csv

    def per_dispatch(path):
        out = []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                out.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
        return out

    copy_bytes = copy_mib << 20
    res = {}
    for name, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = per_dispatch(path)
        copies = [r for r in rows if "copyBuffer" in r[0]]
        if not copies:
            raise SystemExit("%s: no copy dispatch; run with --copy-probe-mib" % path)
        probe = max(copies, key=lambda r: r[1])
        attn = [r for r in rows if "k_attn_" in r[0]]
        if not attn:
            raise SystemExit("%s: no attention kernel dispatch" % path)
        dec = [r for r in rows if decode_kernel(r[0])]
        kib = sum(r[2] for r in dec) / len(attn)  # per call: one attention dispatch per call
        factor = copy_bytes / (probe[2] * 1024.0)
        names = sorted({short_kernel_name(r[0]) for r in dec})
        res[name] = (kib, probe[2], factor, len(attn), " + ".join(names))
    bench = None
    with open(bench_log) as fh:
        for line in fh:
            if line.startswith("{"):
                bench = json.loads(line)
    hbm = sum(kib * 1024.0 * f for kib, _, f, _, _ in res.values())
    lines = [
        "kernels (per decode call): %s" % res["fetch"][4],
        "workload: %s" % (bench["config"]["workload"] if bench else "?"),
        "decode calls: %d (FETCH_SIZE run), %d (WRITE_SIZE run)" % (res["fetch"][3], res["write"][3]),
        "copy_probe_bytes: %d" % copy_bytes,
        "copy_probe_fetch_kib: %.1f" % res["fetch"][1],
        "copy_probe_write_kib: %.1f" % res["write"][1],
        "fetch_factor: %.5f" % res["fetch"][2],
        "write_factor: %.5f" % res["write"][2],
        "fetch_kib_per_call: %.1f" % res["fetch"][0],
        "write_kib_per_call: %.1f" % res["write"][0],
        "hbm_bytes_per_call: %d" % round(hbm),
    ]
    if bench:
        lines += ["algorithmic_bytes_per_call: %d" % bench["decode_bytes"],
                  "traffic_over_algorithmic: %.4f" % (hbm / bench["decode_bytes"])]
    lines.append("source_hash: %s" % source_hash())
    print("\n".join(lines))


def short_kernel_name(name):
    name = name.replace("kvq::(anonymous namespace)::", "").replace("kvq::", "")
    if name.startswith("void "):
        name = name[5:]
    if name.startswith("at::native::"):
        return name.split("<")[0] + "<...>"
    cut = name.find("(")
    return name[:cut] if cut > 0 else name


BUSY_COUNTERS = ("SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
                 "SQ_WAVE_CYCLES SQ_INSTS_LDS GRBM_GUI_ACTIVE")


def summarize_busy(counter_csv, agent_csv, bench_log):
    """VALU and MFMA busy fractions of the decode kernels from one rocprofv3 --pmc run of
    BUSY_COUNTERS, averaged over each kernel's dispatches.  GRBM_GUI_ACTIVE is summed over the
    XCDs, so the active cycles of one XCD are GRBM_GUI_ACTIVE / Num_Xcc; a wave64 VALU instruction
    occupies its SIMD for 4 cycles and SQ_ACTIVE_INST_VALU counts those in units of 4 cycles:
      VALU busy = 4 SQ_ACTIVE_INST_VALU / (SIMDs x cycles)
      MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x cycles)
    and the MFMA rate counts 16 x 16 x 32 x 2 flops per instruction (v_mfma_f32_16x16x32_f16)."""
    import csv
    import collections
    with open(agent_csv) as fh:
        gpu = [r for r in csv.DictReader(fh) if r["Agent_Type"] == "GPU"][0]
    simds, xcc = int(gpu["Simd_Count"]), int(gpu["Num_Xcc"])
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    with open(counter_csv) as fh:
        for r in csv.DictReader(fh):
            if not decode_kernel(r["Kernel_Name"]) and "k_merge" not in r["Kernel_Name"]:
                continue
            name = short_kernel_name(r["Kernel_Name"])
            agg[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
            dur[name][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    bench = None
    with open(bench_log) as fh:
        for line in fh:
            if line.startswith("{"):
                bench = json.loads(line)
    lines = []
    if bench:
        lines += ["workload: %s" % bench["config"]["workload"], ""]
    lines.append("SIMDs: %d, XCDs: %d" % (simds, xcc))
    for name, d in agg.items():
        avg = {c: sum(v) / len(v) for c, v in d.items()}
        cyc = avg["GRBM_GUI_ACTIVE"] / xcc
        ns = sum(dur[name].values()) / len(dur[name])
        lines += ["", "kernel: %s (%d dispatches, %.2f us each under the profiler)" % (name, len(dur[name]), ns / 1e3)]
        lines += ["  %s: %.6g" % (c, avg[c]) for c in sorted(avg)]
        lines.append("  VALU busy: %.1f %%" % (100 * 4 * avg["SQ_ACTIVE_INST_VALU"] / (simds * cyc)))
        lines.append("  MFMA busy: %.1f %%" % (100 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * cyc)))
        lines.append("  MFMA rate: %.1f TFLOP/s (dense f16 peak 2500)" % (avg["SQ_INSTS_MFMA"] * 16384 / ns / 1e3))
        lines.append("  VALU instructions per wave: %.0f" % (avg["SQ_INSTS_VALU"] / avg["SQ_WAVES"]))
    lines.append("source_hash: %s" % source_hash())
    print("\n".join(lines))


def summarize_stats(stats_csv, bench_log):
    """Per-kernel durations of one profiled bench run, next to the bench's own event timing."""
    import csv
    with open(stats_csv) as fh:
        rows = list(csv.DictReader(fh))
    bench = None
    with open(bench_log) as fh:
        for line in fh:
            if line.startswith("{"):
                bench = json.loads(line)
    lines = []
    if bench:
        lines += ["workload: %s" % bench["config"]["workload"],
                  "bench decode_ms (HIP events, mean over steps): %.4f" % bench["decode_ms"],
                  "bench decode_bytes: %d" % bench["decode_bytes"],
                  "bench decode GB/s: %.1f (%.2f%% of 8 TB/s)" % (bench["decode_gbs"], bench["pct_hbm_peak"]),
                  "bench quant_prefill_tokens_per_s: %.4g" % bench["quant_prefill_tokens_per_s"],
                  ""]
    lines.append("%-58s %6s %12s %12s %12s %7s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "pct"))
    for r in rows:
        lines.append("%-58s %6s %12.2f %12.2f %12.2f %7.2f" % (
            short_kernel_name(r["Name"])[:58], r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    dec = [r for r in rows if decode_kernel(r["Name"])]
    if dec and bench:
        ns = sum(float(r["AverageNs"]) for r in dec)
        lines += ["", "decode kernels: %s" % " + ".join(short_kernel_name(r["Name"]) for r in dec),
                  "decode kernels avg_us (sum): %.2f -> %.1f GB/s on the decode algorithmic bytes" % (
                      ns / 1e3, bench["decode_bytes"] / ns)]
    lines.append("source_hash: %s" % source_hash())
    print("\n".join(lines))


# ---------------------------------------------------------------------------

def measure(idx, steps, warmup, torch, K, synth, stream, page=0):
    """Set up workload idx, time its bulk prefill quantize and `steps` steps (append + decode) after
    `warmup` untimed ones; returns the per-workload figures.  Device memory is released on return."""
    import numpy as np
    t = time.perf_counter()
    wl = build_workload(idx, torch, K, synth, page)
    torch.cuda.synchronize()
    log("workload %d set up in %.1fs (%d cache cop%s)" % (idx, time.perf_counter() - t, wl.rotate,
                                                        "y" if wl.rotate == 1 else "ies"))
    # bulk prefill (quantize-append of the whole prompt); fills every cache copy
    for r in range(wl.rotate):
        wl.prefill(r)
    torch.cuda.synchronize()
    reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        wl.prefill(i % wl.rotate)
    e1.record(stream)
    torch.cuda.synchronize()
    bulk_ms = e0.elapsed_time(e1) / reps
    bulk_tok_s = wl.prefill_tokens / (bulk_ms / 1e3)
    log("prefill quantize %d tokens: %.3f ms, %.3e tok/s" % (wl.prefill_tokens, bulk_ms, bulk_tok_s))

    def step(i, ev_a=None, ev_b=None):
        r = i % wl.rotate
        wl.append(r)
        if ev_a is not None:
            ev_a.record(stream)
        wl.decode(r)
        if ev_b is not None:
            ev_b.record(stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    flags = wl.flags()
    assert not any(flags), "device status flags %s" % flags
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s0.record(stream)
    for i, (a, b) in enumerate(evs):
        step(i, a, b)
    s1.record(stream)
    torch.cuda.synchronize()
    step_ms = s0.elapsed_time(s1) / steps
    dec_times = [a.elapsed_time(b) for a, b in evs]
    dec_ms = float(np.mean(dec_times))
    dbytes = wl.decode_bytes()
    abytes = wl.append_bytes()
    value = (dbytes + abytes) / (step_ms / 1e3) / 1e9
    achieved = dbytes / (dec_ms / 1e3) / 1e9
    app_ms = step_ms - dec_ms
    w = wl.w
    app_tokens = w.batch * (1 if idx != 1 else w.tokens)
    append_tok_s = app_tokens / (app_ms / 1e3) if (idx in (1, 2, 5, 6, 7, 9) and app_ms > 0) else None
    log("step %.4f ms, decode %.4f ms (median %.4f) -> %.1f GB/s (%.1f%% of peak)"
        % (step_ms, dec_ms, float(np.median(dec_times)), achieved, 100 * achieved / HBM_PEAK_GBS))
    res = {
        "workload": WORKLOAD_TEXT[idx],
        "batch": w.batch, "kv_heads": w.kv_heads, "q_heads": w.q_heads, "seq_len": w.tokens,
        "cache_copies": wl.rotate,
        "steps": steps,
        "value": value,
        "ms_per_step": step_ms,
        "decode_ms": dec_ms,
        "decode_bytes": int(dbytes),
        "decode_gbs": achieved,
        "quant_prefill_tokens_per_s": bulk_tok_s,
        "quant_prefill_ms": bulk_ms,
        "quant_append_tokens_per_s": append_tok_s,
    }
    del wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def config_summary(idx, r):
    """The compact per-configuration record carried in the JSON line."""
    return {
        "workload": WORKLOAD_TEXT[idx].split(":")[0],
        "decode_ms": round(r["decode_ms"], 5),
        "decode_bytes": r["decode_bytes"],
        "decode_gbs": round(r["decode_gbs"], 1),
        "frac_hbm_peak": round(r["decode_gbs"] / HBM_PEAK_GBS, 4),
        "quant_prefill_tokens_per_s": round(r["quant_prefill_tokens_per_s"], 1),
        "quant_append_tokens_per_s": (round(r["quant_append_tokens_per_s"], 1)
                                      if r["quant_append_tokens_per_s"] else None),
        "traffic": stored_traffic(idx),
    }


def main():
    global ARGS
    ARGS = args = parse()
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_busy:
        summarize_busy(*args.summarize_busy)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.copy_probe_mib or 1024)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU (--gpus 1); runs on several GPUs are not part of this "
              "library's scope", file=sys.stderr)
        sys.exit(2)

    import synth

    cpu = None
    if not args.no_cpu:
        t = time.perf_counter()
        cpu = cpu_baseline(synth.WORKLOADS[args.workload], args.workload, args.cpu_seconds)
        log("cpu oracle leg %.1fs: %s" % (time.perf_counter() - t, cpu))

    import torch

    import quantized_kv_cache_05_amd as K

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    idx = args.workload

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    head = measure(idx, args.steps, args.warmup, torch, K, synth, stream, args.page_tokens)
    configs = {}
    if not args.headline_only:
        # the other configurations of the metric, each set up, measured and released in turn
        for j in (1, 2, 3, 4, 5):
            if j == idx:
                configs[str(j)] = config_summary(j, head)
                continue
            configs[str(j)] = config_summary(j, measure(j, min(args.steps, 20), min(args.warmup, 5),
                                                        torch, K, synth, stream))
    achieved = head["decode_gbs"]
    res = {
        "metric": METRIC,
        "value": round(head["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": head["workload"],
            "batch": head["batch"], "kv_heads": head["kv_heads"], "q_heads": head["q_heads"],
            "seq_len": head["seq_len"], "num_splits": args.num_splits, "cache_copies": head["cache_copies"],
            "page_tokens": args.page_tokens,
        },
        "decode_ms": round(head["decode_ms"], 5),
        "decode_bytes": head["decode_bytes"],
        "decode_gbs": round(achieved, 1),
        "pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "quant_prefill_tokens_per_s": round(head["quant_prefill_tokens_per_s"], 1),
        "quant_prefill_ms": round(head["quant_prefill_ms"], 4),
        "quant_append_tokens_per_s": (round(head["quant_append_tokens_per_s"], 1)
                                      if head["quant_append_tokens_per_s"] else None),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if args.page_tokens else stored_traffic(idx),
        },
        "cpu_baseline": cpu,
        "configs": configs or None,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

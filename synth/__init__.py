"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

Holds random-number generation and the workload shapes only: no quantization
or attention arithmetic.  Every value is a pure function of (seed, stream,
flat index) (counter-based SplitMix64 + Box-Muller, see ``synth.c``), so any
(batch, head) slice can be regenerated on its own and both sides see the
same bytes.

Streams: K = 0, V = 1, Q = 2, outlier channels = 3, chunk embeddings = 4,
calibration K = 5, calibration V = 6, token scores = 7.  Seed of workload i (1-based) is
20261200 + i.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lock = threading.Lock()
_lib = None

STREAM_K, STREAM_V, STREAM_Q, STREAM_OUTLIER, STREAM_CHUNK_EMB, STREAM_CAL_K, STREAM_CAL_V, STREAM_SCORE = range(8)
DIST_NORMAL, DIST_T3 = 0, 1


def build(force: bool = True) -> str:
    """Compile libsynth.so next to its source (plain gcc, no GPU)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            L = ctypes.CDLL(_LIB)
            u64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
            L.synth_fill_f16.argtypes = [u64, u64, i32, dbl, u64, u64, i32, u64, i32, vp, vp]
            L.synth_fill_f16.restype = None
            L.synth_fill_f64_normal.argtypes = [u64, u64, u64, u64, vp]
            L.synth_fill_u64.argtypes = [u64, u64, u64, u64, vp]
            L.synth_f16_from_double.argtypes = [dbl]
            L.synth_f16_from_double.restype = ctypes.c_uint16
            _lib = L
    return _lib


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def fill_f16(seed, stream, dist, mult, start, count, dim=128, rows_per_head=1, heads=1,
             chan_scale=None, out=None) -> np.ndarray:
    """fp16 bit patterns (uint16) of flat elements [start, start+count)."""
    L = lib()
    if out is None:
        out = np.empty(count, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size == count and out.flags.c_contiguous
    cs = None
    if chan_scale is not None:
        chan_scale = np.ascontiguousarray(chan_scale, dtype=np.float64)
        assert chan_scale.shape == (heads, dim)
        cs = chan_scale.ctypes.data
    base = out.ctypes.data
    n = _threads() if count >= (1 << 20) else 1
    step = (count + n - 1) // n

    def work(j):
        a = j * step
        c = min(count, a + step) - a
        if c > 0:
            L.synth_fill_f16(seed, stream, dist, mult, start + a, c, dim, rows_per_head, heads, cs,
                             base + 2 * a)

    if n == 1:
        work(0)
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(work, range(n)))
    return out


def fill_f64_normal(seed, stream, start, count) -> np.ndarray:
    out = np.empty(count, dtype=np.float64)
    lib().synth_fill_f64_normal(seed, stream, start, count, out.ctypes.data)
    return out


def fill_u64(seed, stream, start, count) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    lib().synth_fill_u64(seed, stream, start, count, out.ctypes.data)
    return out


@dataclass
class Workload:
    """Shapes and value distributions of one synthetic workload."""
    index: int                 # 1-based workload number
    name: str
    batch: int
    kv_heads: int
    q_heads: int
    seq: int                   # tokens in the cache at decode time
    tokens: int                # tokens generated per (b, h) (seq, or seq + 1 with an append)
    head_dim: int = 128
    dist: int = DIST_NORMAL
    mult: float = 1.0          # global multiplier of the K/V draws
    outlier_mult: float = 1.0  # multiplier of the outlier channels
    outlier_count: int = 0     # random outlier channels per (tensor, head)
    fixed_outliers: tuple = () # fixed outlier channels (same for every head)
    chunk_tokens: int = 0      # chunk-mixed workloads: tokens per chunk
    emb_dim: int = 0           # chunk-mixed workloads: embedding width
    cal_samples: int = 0       # calibration sequences per tensor

    @property
    def seed(self) -> int:
        return 20261200 + self.index

    def channel_scale(self, tensor: int) -> np.ndarray | None:
        """[kv_heads][head_dim] per-channel multiplier (1 or outlier_mult)."""
        if self.fixed_outliers:
            cs = np.ones((self.kv_heads, self.head_dim))
            cs[:, list(self.fixed_outliers)] = self.outlier_mult
            return cs
        if self.outlier_count == 0:
            return None
        cs = np.ones((self.kv_heads, self.head_dim))
        for h in range(self.kv_heads):
            keys = fill_u64(self.seed, STREAM_OUTLIER, (tensor * self.kv_heads + h) * self.head_dim,
                            self.head_dim)
            chans = np.argsort(keys, kind="stable")[: self.outlier_count]
            cs[h, chans] = self.outlier_mult
        return cs

    def kv(self, tensor: int, b0=0, b1=None, h0=0, h1=None, t0=0, t1=None) -> np.ndarray:
        """fp16 bits [b1-b0][h1-h0][t1-t0][head_dim] of K (tensor 0) or V (tensor 1)."""
        b1 = self.batch if b1 is None else b1
        h1 = self.kv_heads if h1 is None else h1
        t1 = self.tokens if t1 is None else t1
        D, T, H = self.head_dim, self.tokens, self.kv_heads
        cs = self.channel_scale(tensor)
        stream = STREAM_K if tensor == 0 else STREAM_V
        out = np.empty((b1 - b0, h1 - h0, t1 - t0, D), dtype=np.uint16)
        full_t = (t0 == 0 and t1 == T)
        if full_t and h0 == 0 and h1 == H:
            flat = out.reshape(-1)
            fill_f16(self.seed, stream, self.dist, self.mult, b0 * H * T * D, flat.size, D, T, H, cs,
                     out=flat)
            return out
        for bi, b in enumerate(range(b0, b1)):
            for hi, h in enumerate(range(h0, h1)):
                start = ((b * H + h) * T + t0) * D
                fill_f16(self.seed, stream, self.dist, self.mult, start, (t1 - t0) * D, D, T, H, cs,
                         out=out[bi, hi].reshape(-1))
        return out

    def q(self, b0=0, b1=None) -> np.ndarray:
        """fp16 bits [b1-b0][q_heads][head_dim] of the decode queries, N(0, 1)."""
        b1 = self.batch if b1 is None else b1
        n = self.q_heads * self.head_dim
        out = fill_f16(self.seed, STREAM_Q, DIST_NORMAL, 1.0, b0 * n, (b1 - b0) * n)
        return out.reshape(b1 - b0, self.q_heads, self.head_dim)

    def chunk_embeddings(self, b: int):
        """(query [emb_dim], chunks [n_chunks][emb_dim]) float64 N(0, 1) vectors of sequence b."""
        n_chunks = self.seq // self.chunk_tokens
        per_seq = (1 + n_chunks) * self.emb_dim
        flat = fill_f64_normal(self.seed, STREAM_CHUNK_EMB, b * per_seq, per_seq)
        return flat[: self.emb_dim], flat[self.emb_dim:].reshape(n_chunks, self.emb_dim)

    def scores(self, b0=0, b1=None) -> np.ndarray:
        """float32 [b1-b0][kv_heads][tokens] per-token importance scores, exp(N(0, 1)): positive and
        heavy-tailed like accumulated attention mass."""
        b1 = self.batch if b1 is None else b1
        n = self.kv_heads * self.tokens
        flat = fill_f64_normal(self.seed, STREAM_SCORE, b0 * n, (b1 - b0) * n)
        return np.exp(flat).astype(np.float32).reshape(b1 - b0, self.kv_heads, self.tokens)

    def calibration(self, tensor: int, sample: int) -> np.ndarray:
        """fp16 bits of calibration sequence `sample`: [kv_heads][seq][head_dim]."""
        n = self.kv_heads * self.seq * self.head_dim
        stream = STREAM_CAL_K if tensor == 0 else STREAM_CAL_V
        return fill_f16(self.seed, stream, self.dist, self.mult, sample * n, n)


WORKLOADS = {
    1: Workload(1, "tiny", batch=1, kv_heads=1, q_heads=1, seq=1024, tokens=1024,
                outlier_mult=20.0, fixed_outliers=(7, 93)),
    2: Workload(2, "llama2-7b-int8", batch=16, kv_heads=32, q_heads=32, seq=4097, tokens=4097,
                outlier_mult=15.0, outlier_count=4),
    3: Workload(3, "llama3-8b-gqa-128k-int4", batch=1, kv_heads=8, q_heads=32, seq=131072,
                tokens=131072, outlier_mult=20.0, outlier_count=3),
    4: Workload(4, "cocktail-13b-mixed", batch=8, kv_heads=40, q_heads=40, seq=32768, tokens=32768,
                chunk_tokens=32, emb_dim=768),
    5: Workload(5, "oaken-13b-threshold", batch=256, kv_heads=40, q_heads=40, seq=2048, tokens=2048,
                dist=DIST_T3, mult=0.5, cal_samples=100),
    6: Workload(6, "llama2-7b-e4m3", batch=16, kv_heads=32, q_heads=32, seq=4097, tokens=4097,
                outlier_mult=15.0, outlier_count=4),
    7: Workload(7, "llama2-7b-int8-paged", batch=16, kv_heads=32, q_heads=32, seq=4097, tokens=4097,
                outlier_mult=15.0, outlier_count=4),
    8: Workload(8, "llama2-7b-dsq", batch=16, kv_heads=32, q_heads=32, seq=4096, tokens=4096,
                outlier_mult=15.0, outlier_count=4),
    9: Workload(9, "llama2-7b-e5m2", batch=16, kv_heads=32, q_heads=32, seq=4097, tokens=4097,
                outlier_mult=15.0, outlier_count=4),
}


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some sizes replaced (same seed and distributions)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    return bits.view(np.float16).astype(np.float32)

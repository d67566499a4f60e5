"""CPU oracle (test infrastructure): numpy marshalling around ``oracle.c``.

Only the tests, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg
use this package; the HIP library never does.  Every function here only
converts arrays and calls the C routine of the same name, whose header
comment cites the page passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            L = ctypes.CDLL(_LIB)
            vp, lg, i32, dbl = ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_double
            sig = {
                "ora_f16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
                "ora_quant_group_asym": ([vp, lg, lg, i32, vp, vp, vp], None),
                "ora_quant_group_sym8": ([vp, lg, lg, vp, vp], None),
                "ora_quant_rows": ([vp, lg, i32, i32, i32, i32, vp, vp, vp], None),
                "ora_quant_channel_blocks": ([vp, lg, lg, i32, i32, i32, vp, vp, vp], None),
                "ora_e4m3_value": ([ctypes.c_uint8], dbl),
                "ora_e4m3_encode": ([ctypes.c_float], ctypes.c_uint8),
                "ora_quant_rows_e4m3": ([vp, lg, i32, i32, vp, vp], None),
                "ora_dequant_rows_e4m3": ([vp, vp, lg, i32, i32, vp], None),
                "ora_e5m2_value": ([ctypes.c_uint8], dbl),
                "ora_e5m2_encode": ([ctypes.c_float], ctypes.c_uint8),
                "ora_quant_rows_e5m2": ([vp, lg, i32, i32, vp, vp], None),
                "ora_dequant_rows_e5m2": ([vp, vp, lg, i32, i32, vp], None),
                "ora_dequant_rows": ([vp, vp, vp, lg, i32, i32, i32, vp], None),
                "ora_dequant_channel_blocks": ([vp, vp, vp, lg, lg, i32, i32, vp], None),
                "ora_oaken_rows": ([vp, lg, i32, i32, vp, vp, vp, vp, vp, vp, vp], None),
                "ora_oaken_dequant_rows": ([vp, vp, vp, vp, vp, vp, lg, i32, i32, vp, vp], None),
                "ora_hist_f16": ([vp, lg, vp], None),
                "ora_hist_percentile": ([vp, lg], ctypes.c_float),
                "ora_chunk_bits": ([vp, vp, lg, i32, dbl, dbl, vp, vp], None),
                "ora_reorder": ([vp, lg, lg, vp, vp], None),
                "ora_attention_partial": ([vp, vp, vp, lg, lg, i32, dbl, vp, vp, vp], None),
                "ora_attention": ([vp, i32, i32, i32, vp, vp, lg, dbl, vp], None),
                "ora_lse_merge": ([i32, vp, vp, vp, i32, vp], None),
                "ora_dsq_group": ([vp, vp, vp, i32, i32, i32, i32] + [vp] * 12, None),
                "ora_dsq_dequant_group": ([ctypes.c_uint64, i32, i32, i32] + [vp] * 13, None),
            }
            for name, (args, res) in sig.items():
                f = getattr(L, name)
                f.argtypes = args
                f.restype = res
            _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def f16_to_f32(bits) -> np.ndarray:
    L = lib()
    flat = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return np.array([L.ora_f16_to_f32(int(b)) for b in flat], dtype=np.float32).reshape(np.shape(bits))


def quant_group_asym(x_bits, bits, stride=1):
    x, px = _c(x_bits, np.uint16)
    n = x.size // stride
    s = np.zeros(1, np.float32)
    z = np.zeros(1, np.uint8)
    q = np.zeros(n, np.uint8)
    lib().ora_quant_group_asym(px, n, stride, bits, s.ctypes.data, z.ctypes.data, q.ctypes.data)
    return s[0], int(z[0]), q


def quant_group_sym8(x_bits):
    x, px = _c(x_bits, np.uint16)
    s = np.zeros(1, np.float32)
    q = np.zeros(x.size, np.int8)
    lib().ora_quant_group_sym8(px, x.size, 1, s.ctypes.data, q.ctypes.data)
    return s[0], q


def quant_rows(x_bits, g, bits, sym=False):
    """x [..., D] fp16 bits -> codes [..., D] (uint8, or int8 if sym), scale/zero [..., D/g]."""
    x, px = _c(x_bits, np.uint16)
    D = x.shape[-1]
    rows = x.size // D
    lead = x.shape[:-1]
    codes = np.zeros(x.shape, np.int8 if sym else np.uint8)
    scale = np.zeros(lead + (D // g,), np.float32)
    zero = np.zeros(lead + (D // g,), np.uint8)
    lib().ora_quant_rows(px, rows, D, g, bits, int(sym), codes.ctypes.data, scale.ctypes.data,
                         zero.ctypes.data)
    return codes, scale, zero


def e4m3_value(codes) -> np.ndarray:
    """binary64 values of E4M3 codes (any shape)."""
    L = lib()
    flat = np.asarray(codes, dtype=np.uint8).reshape(-1)
    return np.array([L.ora_e4m3_value(int(c)) for c in flat], dtype=np.float64).reshape(np.shape(codes))


def e4m3_encode(y) -> np.ndarray:
    """E4M3 codes of binary32 values (any shape)."""
    L = lib()
    flat = np.asarray(y, dtype=np.float32).reshape(-1)
    return np.array([L.ora_e4m3_encode(float(v)) for v in flat], dtype=np.uint8).reshape(np.shape(y))


def quant_rows_e4m3(x_bits, g):
    """x [..., D] fp16 bits -> E4M3 codes [..., D] (uint8), scale [..., D/g]."""
    x, px = _c(x_bits, np.uint16)
    D = x.shape[-1]
    rows = x.size // D
    codes = np.zeros(x.shape, np.uint8)
    scale = np.zeros(x.shape[:-1] + (D // g,), np.float32)
    lib().ora_quant_rows_e4m3(px, rows, D, g, codes.ctypes.data, scale.ctypes.data)
    return codes, scale


def dequant_rows_e4m3(codes, scale, g):
    c, pc = _c(codes, np.uint8)
    s, ps = _c(scale, np.float32)
    D = c.shape[-1]
    out = np.zeros(c.shape, np.float32)
    lib().ora_dequant_rows_e4m3(pc, ps, c.size // D, D, g, out.ctypes.data)
    return out


def e5m2_value(codes) -> np.ndarray:
    """binary64 values of E5M2 codes (any shape)."""
    L = lib()
    flat = np.asarray(codes, dtype=np.uint8).reshape(-1)
    return np.array([L.ora_e5m2_value(int(c)) for c in flat], dtype=np.float64).reshape(np.shape(codes))


def e5m2_encode(y) -> np.ndarray:
    """E5M2 codes of binary32 values (any shape)."""
    L = lib()
    flat = np.asarray(y, dtype=np.float32).reshape(-1)
    return np.array([L.ora_e5m2_encode(float(v)) for v in flat], dtype=np.uint8).reshape(np.shape(y))


def quant_rows_e5m2(x_bits, g):
    """x [..., D] fp16 bits -> E5M2 codes [..., D] (uint8), scale [..., D/g]."""
    x, px = _c(x_bits, np.uint16)
    D = x.shape[-1]
    rows = x.size // D
    codes = np.zeros(x.shape, np.uint8)
    scale = np.zeros(x.shape[:-1] + (D // g,), np.float32)
    lib().ora_quant_rows_e5m2(px, rows, D, g, codes.ctypes.data, scale.ctypes.data)
    return codes, scale


def dequant_rows_e5m2(codes, scale, g):
    c, pc = _c(codes, np.uint8)
    s, ps = _c(scale, np.float32)
    D = c.shape[-1]
    out = np.zeros(c.shape, np.float32)
    lib().ora_dequant_rows_e5m2(pc, ps, c.size // D, D, g, out.ctypes.data)
    return out


def quant_channel_blocks(x_bits, gt, bits):
    """x [..., T, D] -> codes [..., T, D], scale/zero [..., T/gt, D]."""
    x, px = _c(x_bits, np.uint16)
    T, D = x.shape[-2], x.shape[-1]
    lead = x.shape[:-2]
    slices = int(np.prod(lead, dtype=np.int64))
    codes = np.zeros(x.shape, np.uint8)
    scale = np.zeros(lead + (T // gt, D), np.float32)
    zero = np.zeros(lead + (T // gt, D), np.uint8)
    if x.size == 0:
        return codes, scale, zero
    lib().ora_quant_channel_blocks(px, slices, T, D, gt, bits, codes.ctypes.data, scale.ctypes.data,
                                   zero.ctypes.data)
    return codes, scale, zero


def dequant_rows(codes, scale, zero, g, sym=False):
    c, pc = _c(codes, np.int8 if sym else np.uint8)
    s, ps = _c(scale, np.float32)
    z, pz = _c(zero if zero is not None else np.zeros(s.shape, np.uint8), np.uint8)
    D = c.shape[-1]
    out = np.zeros(c.shape, np.float32)
    lib().ora_dequant_rows(pc, ps, pz, c.size // D, D, g, int(sym), out.ctypes.data)
    return out


def dequant_channel_blocks(codes, scale, zero, gt):
    c, pc = _c(codes, np.uint8)
    s, ps = _c(scale, np.float32)
    z, pz = _c(zero, np.uint8)
    T, D = c.shape[-2], c.shape[-1]
    out = np.zeros(c.shape, np.float32)
    if c.size == 0:
        return out
    lib().ora_dequant_channel_blocks(pc, ps, pz, c.size // (T * D), T, D, gt, out.ctypes.data)
    return out


def oaken_rows(x_bits, thr, g=64):
    """-> codes [..., D], scale/zero/oscale [..., D/g], entries [..., D] (first count valid), counts [...]."""
    x, px = _c(x_bits, np.uint16)
    t, pt = _c(thr, np.float32)
    D = x.shape[-1]
    lead = x.shape[:-1]
    rows = x.size // D
    codes = np.zeros(x.shape, np.uint8)
    scale = np.zeros(lead + (D // g,), np.float32)
    zero = np.zeros(lead + (D // g,), np.uint8)
    oscale = np.zeros(lead + (D // g,), np.float32)
    entries = np.zeros(x.shape, np.uint16)
    counts = np.zeros(lead, np.int32)
    lib().ora_oaken_rows(px, rows, D, g, pt, codes.ctypes.data, scale.ctypes.data, zero.ctypes.data,
                         oscale.ctypes.data, entries.ctypes.data, counts.ctypes.data)
    return codes, scale, zero, oscale, entries, counts


def oaken_dequant_rows(codes, scale, zero, oscale, entries, counts, thr, g=64):
    c, pc = _c(codes, np.uint8)
    s, ps = _c(scale, np.float32)
    z, pz = _c(zero, np.uint8)
    so, pso = _c(oscale, np.float32)
    e, pe = _c(entries, np.uint16)
    n, pn = _c(counts, np.int32)
    t, pt = _c(thr, np.float32)
    D = c.shape[-1]
    out = np.zeros(c.shape, np.float32)
    lib().ora_oaken_dequant_rows(pc, ps, pz, pso, pe, pn, c.size // D, D, g, pt, out.ctypes.data)
    return out


def hist_f16(x_bits, hist=None):
    x, px = _c(x_bits, np.uint16)
    if hist is None:
        hist = np.zeros(65536, np.uint64)
    lib().ora_hist_f16(px, x.size, hist.ctypes.data)
    return hist


def hist_percentile(hist, p_bp):
    h, ph = _c(hist, np.uint64)
    return float(lib().ora_hist_percentile(ph, int(p_bp)))


# Oaken threshold percentiles in basis points: lo_outer, lo_inner, hi_inner, hi_outer.
OAKEN_PERCENTILES_BP = (250, 1500, 8500, 9750)


def thresholds_from_hist(hist):
    return np.array([hist_percentile(hist, p) for p in OAKEN_PERCENTILES_BP], np.float32)


def chunk_bits(q_emb, c_emb, alpha=0.6, beta=0.1):
    q, pq = _c(q_emb, np.float64)
    c, pc = _c(c_emb, np.float64)
    n, dim = c.shape
    sims = np.zeros(n, np.float64)
    bits = np.zeros(n, np.uint8)
    lib().ora_chunk_bits(pq, pc, n, dim, alpha, beta, sims.ctypes.data, bits.ctypes.data)
    return bits, sims


def reorder(bits):
    """bits [B][n] -> perm [B][n] int32, seg [B][4] int32."""
    b, pb = _c(bits, np.uint8)
    B, n = b.shape
    perm = np.zeros((B, n), np.int32)
    seg = np.zeros((B, 4), np.int32)
    lib().ora_reorder(pb, B, n, perm.ctypes.data, seg.ctypes.data)
    return perm, seg


def attention_partial(q_bits, khat, vhat, t0, t1, sm_scale):
    q, pq = _c(q_bits, np.uint16)
    k, pk = _c(khat, np.float32)
    v, pv = _c(vhat, np.float32)
    D = q.shape[-1]
    m = np.zeros(1)
    l = np.zeros(1)
    o = np.zeros(D)
    lib().ora_attention_partial(pq, pk, pv, t0, t1, D, sm_scale, m.ctypes.data, l.ctypes.data,
                                o.ctypes.data)
    return m[0], l[0], o


def attention(q_bits, khat, vhat, sm_scale):
    """q [Hq][D] fp16 bits, khat/vhat [Hkv][S][D] float32 -> out [Hq][D] float64."""
    q, pq = _c(q_bits, np.uint16)
    k, pk = _c(khat, np.float32)
    v, pv = _c(vhat, np.float32)
    Hq, D = q.shape
    Hkv, S = k.shape[0], k.shape[1]
    out = np.zeros((Hq, D))
    lib().ora_attention(pq, Hq, Hkv, D, pk, pv, S, sm_scale, out.ctypes.data)
    return out


def lse_merge(m, l, o):
    m_, pm = _c(m, np.float64)
    l_, pl = _c(l, np.float64)
    o_, po = _c(o, np.float64)
    parts, D = o_.shape
    out = np.zeros(D)
    lib().ora_lse_merge(parts, pm, pl, po, D, out.ctypes.data)
    return out


DSQ_GROUP = 64  # tokens per DSQ group


def dsq_quant(k_bits, v_bits, score, n_sig=13, g2=32):
    """DSQ of one (b, kv head): k/v [T][D] fp16 bits, score [T] float32, T a multiple of 64.

    Returns a dict of per-group arrays (G = T / 64, n = 64 - n_sig):
    mask [G] uint64; ksig/vsig [G][n_sig][D] int8; kscale/vscale/base [G][D];
    kc2/vc2 [G][n][D] uint8; ks2/vs2 [G][n][D/g2] float32; kz2/vz2 [G][n][D/g2] uint8.
    """
    k, pk = _c(k_bits, np.uint16)
    v, pv = _c(v_bits, np.uint16)
    sc, _ = _c(score, np.float32)
    T, D = k.shape
    G, n, ng = T // DSQ_GROUP, DSQ_GROUP - n_sig, D // g2
    r = {
        "mask": np.zeros(G, np.uint64),
        "ksig": np.zeros((G, n_sig, D), np.int8), "vsig": np.zeros((G, n_sig, D), np.int8),
        "kscale": np.zeros((G, D), np.float32), "vscale": np.zeros((G, D), np.float32),
        "base": np.zeros((G, D), np.float32),
        "kc2": np.zeros((G, n, D), np.uint8), "vc2": np.zeros((G, n, D), np.uint8),
        "ks2": np.zeros((G, n, ng), np.float32), "vs2": np.zeros((G, n, ng), np.float32),
        "kz2": np.zeros((G, n, ng), np.uint8), "vz2": np.zeros((G, n, ng), np.uint8),
    }
    L = lib()
    for g in range(G):
        o = g * DSQ_GROUP
        L.ora_dsq_group(pk + o * D * 2, pv + o * D * 2, sc.ctypes.data + o * 4, DSQ_GROUP, D, n_sig, g2,
                        r["mask"][g:].ctypes.data, r["ksig"][g].ctypes.data, r["kscale"][g].ctypes.data,
                        r["vsig"][g].ctypes.data, r["vscale"][g].ctypes.data, r["base"][g].ctypes.data,
                        r["kc2"][g].ctypes.data, r["ks2"][g].ctypes.data, r["kz2"][g].ctypes.data,
                        r["vc2"][g].ctypes.data, r["vs2"][g].ctypes.data, r["vz2"][g].ctypes.data)
    return r


def dsq_dequant(r, g2=32):
    """Dequantized K and V [T][D] float32 in token order from a dsq_quant result."""
    G, D = r["kscale"].shape
    khat = np.zeros((G * DSQ_GROUP, D), np.float32)
    vhat = np.zeros((G * DSQ_GROUP, D), np.float32)
    L = lib()
    for g in range(G):
        a = [np.ascontiguousarray(r[x][g]) for x in
             ("ksig", "kscale", "vsig", "vscale", "base", "kc2", "ks2", "kz2", "vc2", "vs2", "vz2")]
        L.ora_dsq_dequant_group(int(r["mask"][g]), DSQ_GROUP, D, g2, *[x.ctypes.data for x in a],
                                khat[g * DSQ_GROUP:].ctypes.data, vhat[g * DSQ_GROUP:].ctypes.data)
    return khat, vhat

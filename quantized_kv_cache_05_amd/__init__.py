"""Python binding of libkvq (the C ABI declared in include/kvq.h).

Argument marshalling only: every computation runs in the HIP kernels of
libkvq.so.  Functions carry the C names; pointer arguments accept torch
tensors (their data_ptr), integers or None, and ``stream=None`` means torch's
current stream.  A negative status raises KVQError.

The library must have been built (``__graft_entry__.build()`` or
``python quantized_kv_cache_05_amd/build.py``); importing the binding without
it raises, there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_HEAD_DIM = 128
KVQ_OK = 0
KVQ_ERR_INVALID_ARG = -1
KVQ_ERR_UNSUPPORTED = -2
KVQ_ERR_CAPACITY = -3
KVQ_ERR_ALIGNMENT = -4
KVQ_ERR_WORKSPACE = -5
KVQ_ERR_HIP = -6

KVQ_MODE_UNIFORM = 0
KVQ_MODE_CHUNK_MIXED = 1
KVQ_MODE_OAKEN = 2
KVQ_MODE_DSQ = 3
KVQ_AXIS_TOKEN = 0
KVQ_AXIS_CHANNEL = 1
KVQ_FMT_INT = 0
KVQ_FMT_E4M3 = 1
KVQ_FMT_E5M2 = 2

KVQ_FLAG_POS_RANGE = 1
KVQ_FLAG_SPARSE_FULL = 2
KVQ_FLAG_LEN_RANGE = 4
KVQ_FLAG_BAD_CHUNK_BITS = 8
KVQ_FLAG_PAGE_RANGE = 16

PART_STRIDE = 132  # floats per split partial in the decode workspace
STATIC_SCRATCH_BYTES = 128 << 20  # KVQ_STATIC_SCRATCH_BYTES: the workspace of kvq_decode_attn_noalloc

_i32, _i64, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

TENSOR_BUFFERS = ("codes", "scale", "zero", "oscale", "rowptr", "sparse", "codes16", "codes2",
                  "scale2", "zero2")


class kvq_tensor(ctypes.Structure):
    _fields_ = [("bits", _i32), ("symmetric", _i32), ("axis", _i32), ("group", _i32),
                ("format", _i32), ("thr", _f32 * 4), ("sparse_cap", _i64)] + [(n, _vp) for n in TENSOR_BUFFERS]


class kvq_cache(ctypes.Structure):
    _fields_ = [("batch", _i32), ("kv_heads", _i32), ("max_seq", _i32), ("head_dim", _i32),
                ("mode", _i32), ("chunk_tokens", _i32), ("k", kvq_tensor), ("v", kvq_tensor),
                ("perm", _vp), ("seg", _vp), ("status", _vp), ("page_tokens", _i32), ("num_pages", _i32),
                ("block_table", _vp), ("dsq_sig", _i32), ("dsq_mask", _vp)]


class kvq_tensor_bytes(ctypes.Structure):
    _fields_ = [(n, _sz) for n in TENSOR_BUFFERS]


class kvq_cache_bytes_t(ctypes.Structure):
    _fields_ = [("k", kvq_tensor_bytes), ("v", kvq_tensor_bytes), ("perm", _sz), ("seg", _sz),
                ("status", _sz), ("dsq_mask", _sz)]


class KVQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%d)" % (where, kvq_status_string(status), status))


_lib = None

EXPORTS = ("kvq_cache_bytes", "kvq_quant_append", "kvq_reorder_chunks", "kvq_append_chunks",
           "kvq_dsq_append", "kvq_decode_workspace_bytes",
           "kvq_decode_attn", "kvq_decode_attn_noalloc", "kvq_chunk_bits", "kvq_hist_f16", "kvq_hist_percentiles",
           "kvq_status_string")


def lib():
    """The loaded libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkvq.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.kvq_cache_bytes.argtypes = [P(kvq_cache), P(kvq_cache_bytes_t)]
        L.kvq_quant_append.argtypes = [P(kvq_cache), _vp, _vp, _i32, _vp, _vp]
        L.kvq_reorder_chunks.argtypes = [P(kvq_cache), _vp, _i32, _vp]
        L.kvq_append_chunks.argtypes = [P(kvq_cache), _vp, _vp, _i32, _vp, _vp, _i32, _vp]
        L.kvq_dsq_append.argtypes = [P(kvq_cache), _vp, _vp, _vp, _i32, _vp, _vp]
        L.kvq_decode_workspace_bytes.argtypes = [P(kvq_cache), _i32, _i32, _i32, P(_sz)]
        L.kvq_decode_attn.argtypes = [P(kvq_cache), _vp, _i32, _vp, _i32, _f32, _vp, _vp, _sz, _i32, _vp]
        L.kvq_decode_attn_noalloc.argtypes = [P(kvq_cache), _vp, _i32, _vp, _i32, _f32, _vp, _i32, _vp]
        L.kvq_chunk_bits.argtypes = [_vp, _vp, _i32, _i32, _i32, ctypes.c_double, ctypes.c_double, _vp,
                                     _vp, _vp]
        L.kvq_hist_f16.argtypes = [_vp, _i64, _vp, _vp]
        L.kvq_hist_percentiles.argtypes = [_vp, _i32, _vp, _vp, _vp]
        L.kvq_status_string.argtypes = [_i32]
        L.kvq_status_string.restype = ctypes.c_char_p
        for n in EXPORTS:
            if n == "kvq_status_string":
                continue
            getattr(L, n).restype = _i32
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> int:
    if status < 0:
        raise KVQError(status, where)
    return status


def kvq_status_string(status: int) -> str:
    return lib().kvq_status_string(int(status)).decode()


def kvq_cache_bytes(cache: kvq_cache) -> kvq_cache_bytes_t:
    out = kvq_cache_bytes_t()
    _check(lib().kvq_cache_bytes(ctypes.byref(cache), ctypes.byref(out)), "kvq_cache_bytes")
    return out


def kvq_quant_append(cache: kvq_cache, k_new, v_new, t_new: int, pos, stream=None) -> int:
    return _check(lib().kvq_quant_append(ctypes.byref(cache), _ptr(k_new), _ptr(v_new), int(t_new),
                                         _ptr(pos), _stream(stream)), "kvq_quant_append")


def kvq_reorder_chunks(cache: kvq_cache, chunk_bits, n_chunks: int, stream=None) -> int:
    return _check(lib().kvq_reorder_chunks(ctypes.byref(cache), _ptr(chunk_bits), int(n_chunks),
                                           _stream(stream)), "kvq_reorder_chunks")


def kvq_append_chunks(cache: kvq_cache, k_new, v_new, t_new: int, pos, new_bits, n_new: int,
                      stream=None) -> int:
    return _check(lib().kvq_append_chunks(ctypes.byref(cache), _ptr(k_new), _ptr(v_new), int(t_new),
                                          _ptr(pos), _ptr(new_bits), int(n_new), _stream(stream)),
                  "kvq_append_chunks")


def kvq_dsq_append(cache: kvq_cache, k_new, v_new, score, t_new: int, pos, stream=None) -> int:
    return _check(lib().kvq_dsq_append(ctypes.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(score), int(t_new),
                                       _ptr(pos), _stream(stream)), "kvq_dsq_append")


def kvq_decode_workspace_bytes(cache: kvq_cache, q_heads: int, max_len: int, num_splits: int = 0) -> int:
    n = _sz(0)
    _check(lib().kvq_decode_workspace_bytes(ctypes.byref(cache), int(q_heads), int(max_len),
                                            int(num_splits), ctypes.byref(n)),
           "kvq_decode_workspace_bytes")
    return n.value


def kvq_decode_attn(cache: kvq_cache, q, q_heads: int, seq_len, max_len: int, sm_scale: float, out,
                    workspace=None, workspace_bytes: int = 0, num_splits: int = 0, stream=None) -> int:
    return _check(lib().kvq_decode_attn(ctypes.byref(cache), _ptr(q), int(q_heads), _ptr(seq_len),
                                        int(max_len), float(sm_scale), _ptr(out), _ptr(workspace),
                                        int(workspace_bytes), int(num_splits), _stream(stream)),
                  "kvq_decode_attn")


def kvq_decode_attn_noalloc(cache: kvq_cache, q, q_heads: int, seq_len, max_len: int, sm_scale: float, out,
                            num_splits: int = 0, stream=None) -> int:
    return _check(lib().kvq_decode_attn_noalloc(ctypes.byref(cache), _ptr(q), int(q_heads), _ptr(seq_len),
                                                int(max_len), float(sm_scale), _ptr(out), int(num_splits),
                                                _stream(stream)),
                  "kvq_decode_attn_noalloc")


def kvq_chunk_bits(q_emb, chunk_emb, batch: int, n_chunks: int, dim: int, alpha: float, beta: float,
                   bits, sims=None, stream=None) -> int:
    return _check(lib().kvq_chunk_bits(_ptr(q_emb), _ptr(chunk_emb), int(batch), int(n_chunks), int(dim),
                                       float(alpha), float(beta), _ptr(sims), _ptr(bits), _stream(stream)),
                  "kvq_chunk_bits")


def kvq_hist_f16(x, n: int, hist, stream=None) -> int:
    return _check(lib().kvq_hist_f16(_ptr(x), int(n), _ptr(hist), _stream(stream)), "kvq_hist_f16")


def kvq_hist_percentiles(hist, p_bp, out, stream=None) -> int:
    arr = (_i32 * len(p_bp))(*[int(p) for p in p_bp])
    return _check(lib().kvq_hist_percentiles(_ptr(hist), len(p_bp), arr, _ptr(out), _stream(stream)),
                  "kvq_hist_percentiles")


# Oaken threshold percentiles in basis points: T_lo_outer, T_lo_inner, T_hi_inner, T_hi_outer.
OAKEN_PERCENTILES_BP = (250, 1500, 8500, 9750)
# Cocktail similarity thresholds recommended by the page (alpha for T_low, beta for T_high).
COCKTAIL_ALPHA = 0.6
COCKTAIL_BETA = 0.1


from .cache import QuantKVCache  # noqa: E402  (allocation helper over the binding)

"""Allocation helper: a kvq_cache descriptor whose buffers are torch tensors.

Sizes come from kvq_cache_bytes; the tensors live as long as this object.
Buffers are plain uint8 device tensors (torch allocations are 256-byte
aligned, above the 16 bytes the library needs).
"""
from __future__ import annotations

import math

from . import (KVQ_AXIS_CHANNEL, KVQ_AXIS_TOKEN, KVQ_MODE_CHUNK_MIXED, KVQ_MODE_OAKEN,
               KVQ_MODE_UNIFORM, TENSOR_BUFFERS, kvq_cache, kvq_cache_bytes,
               kvq_decode_workspace_bytes)


class QuantKVCache:
    def __init__(self, batch: int, kv_heads: int, max_seq: int, mode: int = KVQ_MODE_UNIFORM,
                 k_bits: int = 4, v_bits: int | None = None, symmetric: bool = False,
                 k_axis: int = KVQ_AXIS_TOKEN, k_group: int = 64, v_group: int | None = None,
                 chunk_tokens: int = 32, k_thr=None, v_thr=None, sparse_cap: int = 0,
                 device="cuda", zero_fill: bool = False, fmt: int = 0, page_tokens: int = 0,
                 num_pages: int = 0, block_table=None, dsq_sig: int = 13):
        import torch
        self.torch = torch
        c = kvq_cache()
        c.batch, c.kv_heads, c.max_seq, c.head_dim = batch, kv_heads, max_seq, 128
        c.mode = mode
        c.chunk_tokens = chunk_tokens
        v_bits = k_bits if v_bits is None else v_bits
        v_group = k_group if v_group is None and k_axis == KVQ_AXIS_TOKEN else (v_group or 64)
        for t, bits, axis, group, thr in ((c.k, k_bits, k_axis, k_group, k_thr),
                                          (c.v, v_bits, KVQ_AXIS_TOKEN, v_group, v_thr)):
            t.bits, t.symmetric, t.axis, t.group, t.format = bits, int(symmetric), axis, group, fmt
            if thr is not None:
                for i in range(4):
                    t.thr[i] = float(thr[i])
            t.sparse_cap = sparse_cap
        c.page_tokens, c.num_pages = page_tokens, num_pages
        c.dsq_sig = dsq_sig
        if block_table is not None:
            self.block_table = block_table  # device int32 [batch][max_seq / page_tokens], kept alive here
            c.block_table = block_table.data_ptr()
        self.desc = c
        self.sizes = kvq_cache_bytes(c)
        self.buffers = {}
        alloc = torch.zeros if zero_fill else torch.empty
        for name, t, tb in (("k", c.k, self.sizes.k), ("v", c.v, self.sizes.v)):
            for field in TENSOR_BUFFERS:
                n = getattr(tb, field)
                if n:
                    buf = alloc(n, dtype=torch.uint8, device=device)
                    self.buffers[name + "." + field] = buf
                    setattr(t, field, buf.data_ptr())
        for field in ("perm", "seg"):
            n = getattr(self.sizes, field)
            if n:
                buf = torch.zeros(n // 4, dtype=torch.int32, device=device)
                self.buffers[field] = buf
                setattr(c, field, buf.data_ptr())
        if self.sizes.dsq_mask:
            buf = torch.zeros(self.sizes.dsq_mask // 8, dtype=torch.int64, device=device)
            self.buffers["dsq_mask"] = buf
            c.dsq_mask = buf.data_ptr()
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        c.status = self.status.data_ptr()

    def buf(self, name: str):
        return self.buffers[name]

    def workspace(self, q_heads: int, max_len: int, num_splits: int = 0):
        n = kvq_decode_workspace_bytes(self.desc, q_heads, max_len, num_splits)
        ws = self.torch.empty(max(n, 16), dtype=self.torch.uint8, device=self.status.device)
        return ws, n

    def flags(self) -> int:
        return int(self.status.item()) & 0xFFFFFFFF

    @property
    def total_bytes(self) -> int:
        return sum(b.numel() for b in self.buffers.values())


def round_up(x: int, m: int) -> int:
    return int(math.ceil(x / m) * m)

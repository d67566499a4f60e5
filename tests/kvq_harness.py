"""Test-side helpers: unpack the documented packed layout, move fp16 bits to
the GPU, and compare attention outputs.  Neither the oracle nor the HIP
library is imported here; tests combine the three.
"""
from __future__ import annotations

import numpy as np

# Bar for attention outputs: max relative error 2e-3 per (b, query head) row,
# relative to the row's largest |output| (the per-row infinity norm).
ATTN_BAR = 2e-3
# Tighter implementation check, from the arithmetic: binary32 scores with
# relative error ~1e-6 of |score| <= ~30 (base-2 logits) move each softmax
# weight by <= ~3e-5; binary32 accumulation of a few hundred terms per wave
# adds ~1e-6.  1e-4 leaves 3x margin and still catches a dropped or repeated
# token at the sequence lengths the small tests use (~1/S >= 1e-3).
ATTN_TIGHT = 1e-4


def unpack_codes(packed: np.ndarray, bits: int, signed: bool = False) -> np.ndarray:
    """Packed token rows [..., 128*bits/8] (uint8) -> one code per channel [..., 128]."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    if bits == 8:
        return p.view(np.int8) if signed else p
    if bits == 4:
        out = np.stack([p & 0x0F, p >> 4], axis=-1)
    elif bits == 2:
        out = np.stack([(p >> (2 * j)) & 0x03 for j in range(4)], axis=-1)
    else:
        raise ValueError(bits)
    return out.reshape(p.shape[:-1] + (p.shape[-1] * (8 // bits),))


# Channel order of packed rows (kvq.h).  Unpacking a row naively gives 128
# elements e[0..127]; e[PERM[c]] is the element of channel c.
#  K rows: slot 4q + s (elements 8 (4q + s) + v) holds channels 32 s + 8 q + v.
#  V rows: column word n (elements 8 n + j) holds channels n + 16 j.
#  fp16 K rows of the chunk-mixed FP16 pool: slot order (0, 4, 1, 5, 2, 6, 3, 7)
#  inside each slot.
def _k_perm(order=(0, 1, 2, 3, 4, 5, 6, 7)):
    perm = np.zeros(128, np.int64)
    for q in range(4):
        for s in range(4):
            for k, v in enumerate(order):
                perm[32 * s + 8 * q + v] = 8 * (4 * q + s) + k
    return perm


K_PERM = _k_perm()
K16_PERM = _k_perm((0, 4, 1, 5, 2, 6, 3, 7))
V_PERM = np.array([8 * (c % 16) + c // 16 for c in range(128)], np.int64)


def unpack_layout(packed: np.ndarray, bits: int, layout: str, signed: bool = False) -> np.ndarray:
    """Packed K or V rows [..., 16 * bits] -> codes in channel order [..., 128]."""
    e = unpack_codes(packed, bits, signed)
    return e[..., K_PERM if layout == "K" else V_PERM]


def f16_layout(rows_u16: np.ndarray, layout: str) -> np.ndarray:
    """fp16 rows of the FP16 pool [..., 128] (uint16 bits) -> channel order."""
    return rows_u16[..., K16_PERM if layout == "K" else V_PERM]


def oaken_untag(entries: np.ndarray, rowptr: np.ndarray) -> np.ndarray:
    """One (b, h) Oaken side list as stored by the library -> the entries
    without their row tags (channel | side << 7 | mag << 8).  The stored
    entry carries the token index of its row mod 8 in bits 13-15; this checks
    the tag of every listed entry (rows 0 .. len(rowptr) - 2) against its row
    and strips it."""
    rp = np.asarray(rowptr, np.int64)
    n = int(rp[-1])
    e = np.asarray(entries[:n], np.uint16)
    rows = np.repeat(np.arange(len(rp) - 1), np.diff(rp))
    assert np.array_equal(e >> 13, (rows & 7).astype(np.uint16)), "Oaken entry row tags"
    return e & np.uint16(0x1FFF)


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of unpack_codes (used only to test the unpacker itself)."""
    c = np.ascontiguousarray(codes).astype(np.uint8)
    if bits == 8:
        return c
    per = 8 // bits
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // per, per)).astype(np.uint16)
    out = np.zeros(c.shape[:-1], np.uint16)
    for j in range(per):
        out |= c[..., j] << (bits * j)
    return out.astype(np.uint8)


def rel_err_rows(out: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row max|out - ref| / max|ref| over the last axis."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(out - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return num / den


def to_device(bits: np.ndarray, device="cuda"):
    """fp16 bit patterns (uint16 numpy) -> torch int16 device tensor (same bytes)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def i32_device(values, device="cuda"):
    import torch
    return torch.tensor(np.asarray(values, dtype=np.int32), dtype=torch.int32, device=device)


def host_bytes(t) -> np.ndarray:
    """A uint8 / int32 device tensor -> numpy (synchronizes)."""
    return t.cpu().numpy()

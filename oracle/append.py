"""Appending new tokens' K/V to the paged cache, and FP8 E4M3 encoding.  Test infrastructure only.

Every decode step adds one more key and value per token to the request's
cache, taking one more block whenever the last one is full ("How does
TensorRT-LLM work", outcomeschool.com, section "The paged KV cache"; the
scheduler sketch of "TensorRT-LLM, in depth", aicassindra.com, section
"In-flight batching and the scheduler", makes room for the next token before
the pass).  The host decides where each new token goes; here that decision
arrives as a slot number per token: ``slot = block * block_size + offset``
(-1 = no slot, skip).  Appending is then a scatter of each token's
``[Hkv][D]`` K and V rows into ``pool[block][:, offset, :]``.

For an FP8 cache the stored code is the OCP E4M3 encoding of ``x / scale[g]``
(the quotient computed in float32), saturated to +-448 and rounded to the
nearest representable value with ties to the even code (readings of the
pages, which only say the cache may be FP8: "TensorRT-LLM, in depth",
section "Quantization: fewer bytes per weight and per cached token").
"""
from __future__ import annotations

import functools

import numpy as np

from .fp8_e4m3 import e4m3_decode_table

FP8_MAX = 448.0


@functools.lru_cache(maxsize=1)
def _positive_codes():
    """(values, codes) of the 127 non-negative finite E4M3 codes, ascending by value."""
    t = e4m3_decode_table()
    codes = np.array([c for c in range(0x00, 0x7F)], dtype=np.int64)   # 0x7F is NaN
    vals = t[codes]
    order = np.argsort(vals, kind="stable")
    return vals[order], codes[order]


def e4m3_encode(x) -> np.ndarray:
    """float values -> uint8 E4M3 codes: saturate to +-448, round to nearest, ties to even code.

    The sign is kept (so -0.0 and negative values that round to zero give 0x80).
    NaN encodes as 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    vals, codes = _positive_codes()
    a = np.minimum(np.abs(x), FP8_MAX)
    # nearest of the ascending non-negative values; ties -> the even code
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0) & (hi != lo))
    c = np.where(pick_hi, codes[hi], codes[lo])
    c = np.where(a == vals[hi], codes[hi], c)
    neg = np.signbit(x)
    out = (c | np.where(neg, 0x80, 0)).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), out).astype(np.uint8)


def quantize_e4m3(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """Codes of ``x / scale`` with the quotient rounded to float32 first (as a float32 division)."""
    q = (np.asarray(x_f32, dtype=np.float32) / np.float32(scale)).astype(np.float32)
    return e4m3_encode(q.astype(np.float64))


def append_kv(k_pool, v_pool, k_new, v_new, slot_mapping, block_size, kv_fmt="same",
              k_scale=None, v_scale=None):
    """Return copies of the pools with the new tokens written at their slots.

    ``k_new``/``v_new``: ``[T][Hkv][D]`` in the pools' storage (kv_fmt "same")
    or float32 values to be quantised to E4M3 (kv_fmt "fp8", pools of uint8
    codes, one scale per kv head).  ``slot_mapping[t] = -1`` skips token t.
    """
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    hkv = kp.shape[1]
    for t, slot in enumerate(np.asarray(slot_mapping)):
        slot = int(slot)
        if slot < 0:
            continue
        blk, off = divmod(slot, block_size)
        if kv_fmt == "fp8":
            for g in range(hkv):
                kp[blk, g, off, :] = quantize_e4m3(k_new[t, g], k_scale[g])
                vp[blk, g, off, :] = quantize_e4m3(v_new[t, g], v_scale[g])
        else:
            kp[blk, :, off, :] = k_new[t]
            vp[blk, :, off, :] = v_new[t]
    return kp, vp

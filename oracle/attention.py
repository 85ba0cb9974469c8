"""Paged-KV attention in fp64 on the CPU.  Test infrastructure only.

Steps, in the order the pages describe the problem:

1. gather -- follow the request's block table, in logical order, to the
   physical blocks of one pool of equal blocks ("How does TensorRT-LLM work",
   outcomeschool.com, section "The paged KV cache"; "Introduction to
   TensorRT-LLM", dileepadev.github.io, section "2. Paged KV Cache": block
   tables map virtual to physical blocks);
2. dequantise -- FP8 codes times the per-head scale when the cache is FP8
   ("TensorRT-LLM, in depth", aicassindra.com, section "Quantization: fewer
   bytes per weight and per cached token");
3. attend -- every query looks back at every earlier token and its own
   (outcomeschool, sections "Custom attention kernels" and "The paged KV
   cache"), grouped-query head sharing as in Llama-3-8B (aicassindra, section
   "First principles: where the GPU memory goes"); rows with several new
   tokens are chunked-prefill rows mixed into the same pass (aicassindra,
   section "In-flight batching and the scheduler"), each new token seeing the
   prior context plus the new tokens up to itself.

Softmax is the textbook base-e softmax with max subtraction, computed with
numpy in fp64.  There is no blocking, splitting or reordering beyond what the
definition states.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .fp8_e4m3 import e4m3_decode


def stored_to_f64(arr: np.ndarray, fmt: str) -> np.ndarray:
    """Stored values -> float64.

    ``fmt``: "f32" (float32), "bf16" (uint16 bfloat16 bit patterns: the value
    is the float32 whose upper 16 bits are the pattern and lower 16 bits are
    zero) or "fp8" (uint8 E4M3 codes, unscaled).
    """
    if fmt == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        bits = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if fmt == "fp8":
        return e4m3_decode(arr)
    raise ValueError(f"unknown storage format {fmt!r}")


def gather_kv(pool: np.ndarray, fmt: str, table_row: np.ndarray, L: int, g: int,
              block_size: int, head_scale: Optional[float] = None) -> np.ndarray:
    """Logical tokens [0, L) of kv head g, gathered through one block-table row.

    Token t lives in physical block ``table_row[t // block_size]`` at slot
    ``t % block_size``; pool layout is ``[num_blocks][Hkv][block_size][D]``.
    Returns float64 ``[L, D]``.  Only the first ceil(L / block_size) table
    entries are read.
    """
    t = np.arange(L)
    phys = np.asarray(table_row)[t // block_size]
    slot = t % block_size
    vals = stored_to_f64(pool[phys, g, slot, :], fmt)
    if head_scale is not None:
        vals = vals * np.float64(head_scale)
    return vals


def attend_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                first_pos: int) -> np.ndarray:
    """Causal softmax attention for n consecutive query positions.

    ``q``: float64 [n, D] for positions ``first_pos .. first_pos + n - 1``;
    ``K``, ``V``: float64 [L, D].  Query i sees keys t <= first_pos + i.
    Returns float64 [n, D].
    """
    n = q.shape[0]
    L = K.shape[0]
    s = (q @ K.T) * np.float64(scale)                      # [n, L]
    pos = first_pos + np.arange(n)[:, None]
    visible = np.arange(L)[None, :] <= pos
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.where(visible, np.exp(s - m), 0.0)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ V


def paged_attention_row(w, b: int, fmt_override: Optional[str] = None) -> np.ndarray:
    """Output of row b of workload ``w`` (a ``pa_inputs.Workload``): float64 [q_len, Hq, D]."""
    L = int(w.seq_lens[b])
    n = int(w.q_lens[b])
    q0 = int(w.q_start_loc[b])
    return _row(w.q[q0:q0 + n], w.q_fmt, w.k_pool, w.v_pool, w.kv_fmt, w.block_table[b], L,
                w.block_size, w.num_q_heads, w.num_kv_heads, w.scale, w.k_scale, w.v_scale)


def _row(q_rows, q_fmt, k_pool, v_pool, kv_fmt, table_row, L, bs, Hq, Hkv, scale,
         k_scale, v_scale) -> np.ndarray:
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    n = q_rows.shape[0]
    if not (1 <= n <= L):
        raise ValueError("need 1 <= q_len <= seq_len")
    qf = stored_to_f64(q_rows, q_fmt)                      # [n, Hq, D]
    out = np.empty(qf.shape, dtype=np.float64)
    for g in range(Hkv):
        ks = None if k_scale is None else float(k_scale[g])
        vs = None if v_scale is None else float(v_scale[g])
        K = gather_kv(k_pool, kv_fmt, table_row, L, g, bs, ks)
        V = gather_kv(v_pool, kv_fmt, table_row, L, g, bs, vs)
        for h in range(g * group, (g + 1) * group):
            out[:, h, :] = attend_rows(qf[:, h, :], K, V, scale, L - n)
    return out


def paged_attention(q, q_fmt, k_pool, v_pool, kv_fmt, block_table, seq_lens, block_size,
                    num_q_heads, num_kv_heads, scale, q_lens=None, k_scale=None,
                    v_scale=None, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Paged attention over a batch.  Returns float64 ``[total_q, Hq, D]``.

    ``q`` is ``[total_q, Hq, D]`` with rows packed in order; row b owns
    ``q_lens[b]`` consecutive query tokens (1 for decode).  With ``rows``
    given, only those rows are computed and the others are left NaN.
    """
    seq_lens = np.asarray(seq_lens)
    B = len(seq_lens)
    q_lens = np.ones(B, dtype=np.int64) if q_lens is None else np.asarray(q_lens)
    starts = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    out = np.full((int(starts[-1]), num_q_heads, q.shape[-1]), np.nan, dtype=np.float64)
    for b in (range(B) if rows is None else rows):
        a, e = int(starts[b]), int(starts[b + 1])
        out[a:e] = _row(q[a:e], q_fmt, k_pool, v_pool, kv_fmt, block_table[b], int(seq_lens[b]),
                        block_size, num_q_heads, num_kv_heads, scale, k_scale, v_scale)
    return out


def paged_attention_workload(w, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """``paged_attention`` on a ``pa_inputs.Workload``."""
    return paged_attention(w.q, w.q_fmt, w.k_pool, w.v_pool, w.kv_fmt, w.block_table, w.seq_lens,
                           w.block_size, w.num_q_heads, w.num_kv_heads, w.scale, w.q_lens,
                           w.k_scale, w.v_scale, rows)

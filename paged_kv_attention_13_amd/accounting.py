"""Algorithmic byte and flop counts for paged-KV attention (host arithmetic only).

The per-token KV size follows the pages' own accounting: K and V, per layer,
per KV head, ``head_dim`` elements each ("TensorRT-LLM, in depth",
aicassindra.com, section "First principles: where the GPU memory goes").
One call of this library covers one layer.

Algorithmic bytes of a decode or mixed call are what a perfect kernel must
move through HBM:

* every cached K and V element of every row, once: ``L * Hkv * D * 2 * elem``
  per row (FP8 adds the per-head K and V scales, 4 bytes each, once per call);
* the query and output vectors: ``total_q * Hq * D * elem`` each;
* the block-table entries a row needs: ``4 * ceil(L / bs)`` and ``seq_lens``.

Split-K workspace traffic and any over-fetch are not algorithmic and are
excluded.  Algorithmic flops count 2 per multiply-add of Q.K^T and P.V over
the visible (causal) keys only: ``4 * D * Hq`` per (query, visible key).
"""
from __future__ import annotations

import numpy as np

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    """Bytes of K plus V that one cached token occupies over ``layers`` layers."""
    return 2 * layers * kv_heads * head_dim * bytes_per_elem


def tokens_in_pool(pool_bytes: int, layers: int, kv_heads: int, head_dim: int,
                   bytes_per_elem: int) -> int:
    """Whole tokens that fit in a KV pool of ``pool_bytes``."""
    return pool_bytes // kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_elem)


def kv_bytes(seq_lens, num_kv_heads: int, head_dim: int, kv_fmt: str) -> int:
    """Cached K+V bytes of one layer for the given rows (scales excluded)."""
    tokens = int(np.asarray(seq_lens, dtype=np.int64).sum())
    return tokens * kv_bytes_per_token(1, num_kv_heads, head_dim, ELEM_BYTES[kv_fmt])


def call_bytes(seq_lens, q_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
               block_size: int, q_fmt: str, kv_fmt: str, out_fmt: str) -> dict:
    """Algorithmic HBM bytes of one call, split by kind."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    total_q = int(q_lens.sum())
    kv = kv_bytes(seq_lens, num_kv_heads, head_dim, kv_fmt)
    scales = 2 * 4 * num_kv_heads if kv_fmt == "fp8" else 0
    qb = total_q * num_q_heads * head_dim * ELEM_BYTES[q_fmt]
    ob = total_q * num_q_heads * head_dim * ELEM_BYTES[out_fmt]
    meta = 4 * int(((seq_lens + block_size - 1) // block_size).sum()) + 4 * len(seq_lens)
    return {"kv": kv, "scales": scales, "q": qb, "out": ob, "meta": meta,
            "total": kv + scales + qb + ob + meta}


def call_flops(seq_lens, q_lens, num_q_heads: int, head_dim: int) -> int:
    """Algorithmic flops: 4*D*Hq per (query, visible key) pair, causal part only."""
    total = 0
    for L, n in zip(np.asarray(seq_lens, dtype=np.int64), np.asarray(q_lens, dtype=np.int64)):
        # query i (0-based) of a row with n new tokens sees L - n + i + 1 keys
        visible = n * (L - n) + n * (n + 1) // 2
        total += int(visible)
    return 4 * head_dim * num_q_heads * total


def workload_bytes(w, out_fmt: str | None = None) -> dict:
    """``call_bytes`` for a ``pa_inputs.Workload``."""
    return call_bytes(w.seq_lens, w.q_lens, w.num_q_heads, w.num_kv_heads, w.head_dim,
                      w.block_size, w.q_fmt, w.kv_fmt, out_fmt or w.q_fmt)

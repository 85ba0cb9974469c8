"""fp64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
(no kernels, headers, tables or helpers); the only code both sides consume is
the seeded input generator in ``pa_inputs``, which draws data and does none
of the attention arithmetic.

What it computes.  The pages state the problem in words, not formulas:

* the KV cache keeps one key and one value vector per token, per layer, per
  KV head ("TensorRT-LLM, in depth", aicassindra.com, section "First
  principles: where the GPU memory goes");
* it lives in a pool of equal fixed-size blocks handed out on demand, and a
  per-request table lists the request's blocks in order ("How does
  TensorRT-LLM work", outcomeschool.com, section "The paged KV cache";
  "Introduction to TensorRT-LLM", dileepadev.github.io, section "2. Paged KV
  Cache");
* to produce a token, attention looks back at every token that came before
  (outcomeschool, sections "Custom attention kernels" and "The paged KV
  cache");
* Llama-3-8B groups 32 query heads onto 8 KV heads (grouped-query
  attention; aicassindra, "First principles").

The pages never write the attention formula, so the oracle uses the textbook
scaled-dot-product softmax attention (readings listed in the design notes):

    g      = h // (Hq / Hkv)                       consecutive head groups
    K[t]   = k_pool[table[b][t // bs]][g][t % bs]   t in [0, L)
    s_t    = scale * <q_i,h , K[t]>                 t <= L - n + i  (causal)
    p      = softmax(s)                             base e
    o_i,h  = sum_t p_t V[t]

with L = seq_lens[b] counting every cached token including the row's n new
ones.  FP8 E4M3 KV values are ``decode(code) * scale[g]`` in fp64.

Appending a step's new K/V (a scatter through per-token slot numbers, with
E4M3 quantisation for an FP8 cache) is in ``append.py``; its pins are in
``tests/test_oracle_append.py`` (encoder against its bit format, torch's
``float8_e4m3fn`` cast, ties-to-even, saturation, scatter/gather round trip).

Pins (see ``tests/test_oracle.py``): contiguous triple-loop brute force on
tiny inputs, torch's fp64 ``scaled_dot_product_attention`` special case,
closed-form invariants (constant V, single token, q = 0 mean, one-hot
probes, key-shift invariance), block-permutation invariance, the toy pool of
the outcomeschool figure, and the full E4M3 code table against its bit
format and torch's ``float8_e4m3fn``.
"""
from .fp8_e4m3 import e4m3_decode_table, e4m3_decode
from .append import append_kv, e4m3_encode, quantize_e4m3
from .attention import (
    stored_to_f64,
    gather_kv,
    attend_rows,
    paged_attention,
    paged_attention_row,
    paged_attention_workload,
)

__all__ = [
    "e4m3_decode_table", "e4m3_decode", "append_kv", "e4m3_encode", "quantize_e4m3",
    "stored_to_f64", "gather_kv", "attend_rows",
    "paged_attention", "paged_attention_row", "paged_attention_workload",
]

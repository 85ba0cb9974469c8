"""Seeded synthetic inputs for paged-KV attention.

This module only *draws and lays out* data: random values, sequence lengths,
block tables and pool sizes.  It holds none of the attention arithmetic, so
both the fp64 oracle and the HIP path can consume its output without sharing
any computation.

Storage formats (numpy, host memory):

* ``"f32"``  -- float32 arrays.
* ``"bf16"`` -- uint16 arrays holding bfloat16 bit patterns (numpy has no
  bfloat16); values are N(0,1) float32 samples rounded to nearest-even by
  torch's CPU cast.
* ``"fp8"``  -- uint8 arrays of OCP FP8 E4M3 ("e4m3fn") codes with one float32
  scale per (K or V, kv head): ``scale = amax / 448`` and
  ``code = e4m3(clamp(x / scale, -448, 448))`` via torch's CPU cast.

Pool layout: ``pool[num_blocks][num_kv_heads][block_size][head_dim]``; a
block table row lists, in logical order, the physical block ids of one
request ("a small table remembers which blocks belong to which request and in
what order": "How does TensorRT-LLM work", outcomeschool.com, section "The
paged KV cache").  Table entries past ``ceil(L / block_size)`` are set to -1
because they must never be read.

The five named workloads reproduce the Llama-3-8B decode shapes (32 query
heads, 8 KV heads, head_dim 128: "TensorRT-LLM, in depth", aicassindra.com,
section "First principles: where the GPU memory goes").  Seeds are
``1000 + workload number``.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Optional

import numpy as np

FP8_MAX = 448.0


@dataclasses.dataclass
class Workload:
    """One batch of inputs for a paged-attention call (host numpy arrays)."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_fmt: str                     # "f32" | "bf16"
    kv_fmt: str                    # "f32" | "bf16" | "fp8"
    q: np.ndarray                  # [total_q, Hq, D] in q_fmt storage
    k_pool: np.ndarray             # [num_blocks, Hkv, bs, D] in kv_fmt storage
    v_pool: np.ndarray
    block_table: np.ndarray        # int32 [B, max_blocks_per_seq]
    seq_lens: np.ndarray           # int32 [B], KV tokens incl. the row's new ones
    q_lens: np.ndarray             # int32 [B], 1 for decode rows
    k_scale: Optional[np.ndarray] = None   # float32 [Hkv] (fp8 only)
    v_scale: Optional[np.ndarray] = None
    scale: float = 0.0             # softmax scale; 1/sqrt(D) unless stated
    num_decode_rows: int = 0
    group_start: Optional[np.ndarray] = None   # int32 [groups + 1]: rows sharing a cache prefix
    shared_len: Optional[np.ndarray] = None    # int32 [B]: tokens of the row's cache its group shares

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def q_start_loc(self) -> np.ndarray:
        out = np.zeros(self.num_seqs + 1, dtype=np.int32)
        np.cumsum(self.q_lens, out=out[1:])
        return out

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def is_decode_only(self) -> bool:
        return bool(np.all(self.q_lens == 1))


# ----------------------------------------------------------------------------
# value formats (storage only: rounding of random samples to the stored type)
# ----------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bfloat16 bit patterns, round-to-nearest-even (torch CPU cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quantize_fp8_per_head(x: np.ndarray):
    """Quantise ``x[..., Hkv, bs, D]`` (pool layout) to E4M3 codes with one scale per kv head.

    Returns ``(codes uint8, scales float32[Hkv])``.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    amax = t.abs().amax(dim=(0, 2, 3)).numpy().astype(np.float32)
    amax = np.where(amax > 0, amax, np.float32(1.0))
    scales = (amax / np.float32(FP8_MAX)).astype(np.float32)
    y = t / torch.from_numpy(scales)[None, :, None, None]
    y = y.clamp_(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scales


def _normal(seed_seq: np.random.SeedSequence, shape) -> np.ndarray:
    """N(0,1) float32 samples of ``shape``, filled in fixed 4 Mi-element chunks.

    Chunk i draws from ``default_rng(seed_seq.spawn(...)[i])``, so the result
    depends only on (seed, shape), not on how many threads fill it.
    """
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    n = flat.size
    chunk = 1 << 22
    children = seed_seq.spawn(max(1, (n + chunk - 1) // chunk))

    def fill(i):
        a = i * chunk
        b = min(n, a + chunk)
        np.random.default_rng(children[i]).standard_normal(size=b - a, dtype=np.float32, out=flat[a:b])

    if len(children) == 1:
        fill(0)
    else:
        from concurrent.futures import ThreadPoolExecutor
        workers = min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4)
        with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
            list(ex.map(fill, range(len(children))))
    return out


def _store(x: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if fmt == "bf16":
        return to_bf16_bits(x)
    raise ValueError(fmt)


# ----------------------------------------------------------------------------
# block tables
# ----------------------------------------------------------------------------

def blocks_needed(seq_lens: np.ndarray, block_size: int) -> np.ndarray:
    return (seq_lens.astype(np.int64) + block_size - 1) // block_size


def random_block_table(rng: np.random.Generator, seq_lens: np.ndarray, block_size: int,
                       num_blocks: int, max_blocks_per_seq: Optional[int] = None) -> np.ndarray:
    """Hand each row its blocks from a seeded random permutation of the pool.

    Distinct rows get distinct physical blocks; entries past a row's last
    block are -1.
    """
    need = blocks_needed(seq_lens, block_size)
    total = int(need.sum())
    if total > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks < {total} needed")
    mb = int(need.max()) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    mb = max(mb, 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((len(seq_lens), mb), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += int(n)
    return table


# ----------------------------------------------------------------------------
# generic generator
# ----------------------------------------------------------------------------

def make_workload(*, name: str, seq_lens, q_lens=None, num_q_heads=32, num_kv_heads=8,
                  head_dim=128, block_size=16, q_fmt="bf16", kv_fmt="bf16",
                  pool_factor: float = 1.0, extra_blocks: int = 0, seed: int = 0,
                  poison_unused: bool = False, max_blocks_per_seq: Optional[int] = None,
                  scale: Optional[float] = None) -> Workload:
    """Draw one workload.

    ``seq_lens[b]`` counts every cached token of row b including its
    ``q_lens[b]`` new ones.  The pool holds ``ceil(pool_factor * needed) +
    extra_blocks`` blocks.  With ``poison_unused`` every pool slot no row
    references (unreferenced blocks and slots past L in a row's last block)
    is NaN (fp8: code 0x7F).
    """
    ss_table, ss_q, ss_k, ss_v = np.random.SeedSequence(seed).spawn(4)
    rng = np.random.default_rng(ss_table)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    q_lens = np.ones(B, dtype=np.int32) if q_lens is None else np.asarray(q_lens, dtype=np.int32)
    if np.any(q_lens < 1) or np.any(q_lens > seq_lens):
        raise ValueError("need 1 <= q_len <= seq_len")
    need = int(blocks_needed(seq_lens, block_size).sum())
    num_blocks = int(np.ceil(pool_factor * need)) + int(extra_blocks)
    num_blocks = max(num_blocks, 1)
    table = random_block_table(rng, seq_lens, block_size, num_blocks, max_blocks_per_seq)

    total_q = int(q_lens.sum())
    q = _store(_normal(ss_q, (total_q, num_q_heads, head_dim)), q_fmt)

    kshape = (num_blocks, num_kv_heads, block_size, head_dim)
    kf = _normal(ss_k, kshape)
    vf = _normal(ss_v, kshape)
    k_scale = v_scale = None
    if kv_fmt == "fp8":
        k_pool, k_scale = quantize_fp8_per_head(kf)
        v_pool, v_scale = quantize_fp8_per_head(vf)
    else:
        k_pool, v_pool = _store(kf, kv_fmt), _store(vf, kv_fmt)
    del kf, vf

    w = Workload(name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, block_size=block_size, q_fmt=q_fmt, kv_fmt=kv_fmt,
                 q=q, k_pool=k_pool, v_pool=v_pool, block_table=table, seq_lens=seq_lens,
                 q_lens=q_lens, k_scale=k_scale, v_scale=v_scale,
                 scale=(1.0 / np.sqrt(head_dim)) if scale is None else float(scale),
                 num_decode_rows=leading_decode_rows(q_lens))
    if poison_unused:
        poison_pool(w)
    return w


def make_shared_prefix_workload(*, name: str, group_sizes, shared_lens, own_lens, prefix_ids=None,
                                num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                                extra_blocks: int = 0, seed: int = 0,
                                poison_unused: bool = False) -> Workload:
    """Decode rows in groups whose caches start with the same blocks.

    Group k has ``group_sizes[k]`` consecutive rows whose first ``shared_lens[k]``
    tokens (a multiple of ``block_size``) live in the same physical blocks;
    groups with equal ``prefix_ids`` share the same prefix blocks too (one
    system prompt for many groups).  Row b then has ``own_lens[b] >= 1`` tokens
    of its own in blocks no other row uses, so ``seq_len = shared + own``.
    Physical blocks come from a seeded random permutation of the pool.
    """
    group_sizes = [int(n) for n in group_sizes]
    shared_lens = [int(p) for p in shared_lens]
    own_lens = np.asarray(own_lens, dtype=np.int64)
    prefix_ids = list(range(len(group_sizes))) if prefix_ids is None else [int(i) for i in prefix_ids]
    if any(p % block_size for p in shared_lens) or np.any(own_lens < 1):
        raise ValueError("shared lengths must be whole blocks and every row needs own tokens")
    B = sum(group_sizes)
    if len(own_lens) != B:
        raise ValueError("own_lens needs one entry per row")
    ss_table, ss_q, ss_k, ss_v = np.random.SeedSequence(seed).spawn(4)
    rng = np.random.default_rng(ss_table)
    shared_of_row = np.repeat(np.asarray(shared_lens, dtype=np.int64), group_sizes)
    seq_lens = (shared_of_row + own_lens).astype(np.int32)
    prefix_blocks = {}
    for pid, p in zip(prefix_ids, shared_lens):
        prefix_blocks[pid] = max(prefix_blocks.get(pid, 0), p // block_size)
    own_blocks = (shared_of_row % block_size + own_lens + block_size - 1) // block_size
    need = sum(prefix_blocks.values()) + int(own_blocks.sum())
    num_blocks = need + int(extra_blocks)
    perm = rng.permutation(num_blocks).astype(np.int32)
    pos = 0
    prefix_phys = {}
    for pid in sorted(prefix_blocks):
        prefix_phys[pid] = perm[pos:pos + prefix_blocks[pid]]
        pos += prefix_blocks[pid]
    mb = int(blocks_needed(seq_lens, block_size).max())
    table = np.full((B, mb), -1, dtype=np.int32)
    group_start = np.zeros(len(group_sizes) + 1, dtype=np.int32)
    np.cumsum(group_sizes, out=group_start[1:])
    b = 0
    for k, n in enumerate(group_sizes):
        nshared = shared_lens[k] // block_size
        for _ in range(n):
            table[b, :nshared] = prefix_phys[prefix_ids[k]][:nshared]
            table[b, nshared:nshared + own_blocks[b]] = perm[pos:pos + own_blocks[b]]
            pos += int(own_blocks[b])
            b += 1
    q = _store(_normal(ss_q, (B, num_q_heads, head_dim)), "bf16")
    kshape = (num_blocks, num_kv_heads, block_size, head_dim)
    k_pool = _store(_normal(ss_k, kshape), "bf16")
    v_pool = _store(_normal(ss_v, kshape), "bf16")
    w = Workload(name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                 block_size=block_size, q_fmt="bf16", kv_fmt="bf16", q=q, k_pool=k_pool, v_pool=v_pool,
                 block_table=table, seq_lens=seq_lens, q_lens=np.ones(B, np.int32),
                 scale=1.0 / np.sqrt(head_dim), num_decode_rows=B, group_start=group_start,
                 shared_len=shared_of_row.astype(np.int32))
    if poison_unused:
        poison_pool(w)
    return w


def split_groups(group_sizes, max_rows: int):
    """Cut groups larger than ``max_rows`` into consecutive groups of at most ``max_rows`` rows."""
    out = []
    for n in group_sizes:
        while n > 0:
            out.append(min(n, max_rows))
            n -= out[-1]
    return out


def leading_decode_rows(q_lens: np.ndarray) -> int:
    """Number of leading rows with q_len == 1 (decode rows come first in a mixed batch)."""
    big = np.nonzero(np.asarray(q_lens) != 1)[0]
    return int(big[0]) if len(big) else int(len(q_lens))


def poison_mask(w: Workload) -> np.ndarray:
    """bool [num_blocks, bs]: True where no row's first seq_len tokens live."""
    used = np.zeros((w.num_blocks, w.block_size), dtype=bool)
    bs = w.block_size
    for b in range(w.num_seqs):
        L = int(w.seq_lens[b])
        n = (L + bs - 1) // bs
        for j in range(n):
            hi = min(bs, L - j * bs)
            used[w.block_table[b, j], :hi] = True
    return ~used


def poison_pool(w: Workload) -> None:
    """Overwrite every unreferenced pool slot with NaN (fp8: code 0x7F)."""
    m = poison_mask(w)
    nan = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}[w.kv_fmt]
    for pool in (w.k_pool, w.v_pool):
        view = pool.transpose(0, 2, 1, 3)          # [nb, bs, Hkv, D]
        view[m] = nan


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------

SHARED_PROMPT_7 = 1488      # whole 16-token blocks of workload 7's 1,500-token system prompt

WORKLOAD_NAMES = {
    1: "decode fp32 B1 ctx512 bs16",
    2: "decode bf16 B32 ctxU[1,4096] bs16 pool2x",
    3: "decode bf16 B55 ctx8192 bs64",
    4: "decode fp8kv B128 ctxlogU[128,8192] bs16",
    5: "mixed bf16 8x256-chunk prefill + 96 decode bs16",
    6: "verify bf16 B55 ctx8192 q4 bs64",
    7: "shared-prefix decode bf16 B64 (8 groups of 8) 1488 shared + 312 + U[1,250] bs16",
}


def workload_lengths(i: int, seed: Optional[int] = None):
    """(seq_lens, q_lens) of named workload i, drawn from its own seeded stream."""
    rng = np.random.default_rng((1000 + i) if seed is None else seed)
    if i == 1:
        return np.array([512], np.int32), np.array([1], np.int32)
    if i == 2:
        L = rng.integers(1, 4096 + 1, size=32).astype(np.int32)
        return L, np.ones(32, np.int32)
    if i == 3:
        return np.full(55, 8192, np.int32), np.ones(55, np.int32)
    if i == 4:
        u = rng.uniform(np.log(128.0), np.log(8192.0), size=128)
        L = np.clip(np.rint(np.exp(u)), 128, 8192).astype(np.int32)
        return L, np.ones(128, np.int32)
    if i == 5:
        dec = rng.integers(256, 8192 + 1, size=96).astype(np.int32)
        prior = rng.integers(0, 2048 + 1, size=8).astype(np.int32)
        L = np.concatenate([dec, prior + 256]).astype(np.int32)
        ql = np.concatenate([np.ones(96, np.int32), np.full(8, 256, np.int32)])
        return L, ql
    if i == 6:
        # speculative decoding: every row checks 4 drafted tokens in one pass; the long
        # context of workload 3, so its KV bytes equal that workload's
        return np.full(55, 8192, np.int32), np.full(55, 4, np.int32)
    if i == 7:
        # the support-assistant example: a 1,500-token system prompt shared by every
        # conversation (its 93 full 16-token blocks), then per row the prompt's last 12
        # tokens, a 300-token question and 1..250 tokens generated so far; 64 rows
        # (max_batch_size) in groups of 8
        gen = rng.integers(1, 250 + 1, size=64)
        return (SHARED_PROMPT_7 + 12 + 300 + gen).astype(np.int32), np.ones(64, np.int32)
    raise ValueError(i)


# prefill-only cases (bf16, 32 q / 8 kv heads, 16-token blocks): (seq_lens, q_lens)
PREFILL_CASES = {
    # workload 5's eight prefill-chunk rows alone (its seeded lengths)
    "w5-rows": None,
    # one chunk of 256 new tokens after 8,192 cached ones (few units: the kv-piece path)
    "chunk256-after8192": ([8192 + 256], [256]),
    # one 8,192-token prompt from scratch (many units)
    "prompt8192": ([8192], [8192]),
}


def make_prefill_case(name: str, seed: int = 2024) -> Workload:
    """A prefill-only workload named in PREFILL_CASES."""
    if name == "w5-rows":
        L, ql = workload_lengths(5)
        nd = leading_decode_rows(ql)
        L, ql = L[nd:], ql[nd:]
    else:
        L, ql = PREFILL_CASES[name]
    return make_workload(name=f"prefill {name}", seq_lens=L, q_lens=ql, block_size=16, seed=seed)


def make_config(i: int, seed: Optional[int] = None, poison_unused: bool = False) -> Workload:
    """Named workload i (1..7) at full size."""
    seed = (1000 + i) if seed is None else seed
    L, ql = workload_lengths(i, seed)
    common = dict(name=WORKLOAD_NAMES[i], seq_lens=L, q_lens=ql, seed=seed + 7919,
                  poison_unused=poison_unused)
    if i == 1:
        return make_workload(block_size=16, q_fmt="f32", kv_fmt="f32", **common)
    if i == 2:
        return make_workload(block_size=16, pool_factor=2.0, **common)
    if i == 3:
        return make_workload(block_size=64, **common)
    if i == 4:
        return make_workload(block_size=16, kv_fmt="fp8", **common)
    if i == 5:
        return make_workload(block_size=16, **common)
    if i == 6:
        return make_workload(block_size=64, **common)
    if i == 7:
        return make_shared_prefix_workload(name=WORKLOAD_NAMES[7], group_sizes=[8] * 8,
                                           shared_lens=[SHARED_PROMPT_7] * 8, own_lens=L - SHARED_PROMPT_7,
                                           prefix_ids=[0] * 8, block_size=16, seed=seed + 7919,
                                           poison_unused=poison_unused)
    raise ValueError(i)

"""GPU parity of verify rows (a few new tokens per row, causal) in pa_mixed against the fp64 oracle.

Verify rows are the rows of a speculative-decoding pass: each checks a few
drafted tokens against its whole cache.  Every case prints its name first.
"""
import numpy as np
import pytest

import oracle
import pa_inputs
from gpu_util import TOL_BF16, TOL_FP8, TOL_REL_L2, compare, run_decode, run_mixed

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _verify(rows, dec_lens=(), pre=(), bs=16, hq=32, hkv=8, seed=0, poison=True, kv_fmt="bf16"):
    """rows: (L, n) verify rows; dec_lens: decode rows placed first; pre: (prior, n) prefill rows last."""
    L = list(dec_lens) + [l for l, _ in rows] + [p + n for p, n in pre]
    ql = [1] * len(dec_lens) + [n for _, n in rows] + [n for _, n in pre]
    w = pa_inputs.make_workload(name="verify", seq_lens=L, q_lens=ql, num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=128, block_size=bs, seed=seed, extra_blocks=3,
                                poison_unused=poison, kv_fmt=kv_fmt)
    w.num_decode_rows = len(dec_lens)
    return w


ROWS = [(5, 5), (31, 2), (32, 8), (33, 3), (100, 4), (1000, 8), (4097, 5), (17, 1), (2048, 7), (64, 6)]


@pytest.mark.parametrize("bs", [16, 64])
@pytest.mark.parametrize("workers", [0, 1, 7, 300])
def test_verify_ragged(bs, workers):
    _announce(f"verify ragged bs={bs} workers={workers}")
    w = _verify(ROWS, bs=bs, seed=bs + workers)
    ref = oracle.paged_attention_workload(w)
    got = run_mixed(w, num_workers=workers, num_verify_rows=len(ROWS))
    compare(got, ref, TOL_BF16, what=f"verify bs{bs} W{workers}")


@pytest.mark.parametrize("bs,workers", [(16, 0), (64, 0), (16, 7), (32, 300)])
def test_verify_fp8_kv(bs, workers):
    """FP8-E4M3 pools: decode rows and verify rows of up to 8 new tokens in one call, against the
    oracle fed the dequantised values (NaN codes poison every unused slot)."""
    _announce(f"verify fp8 bs={bs} workers={workers}")
    w = _verify(ROWS, dec_lens=[1, 77, 3000], bs=bs, seed=40 + bs + workers, kv_fmt="fp8")
    ref = oracle.paged_attention_workload(w)
    got = run_mixed(w, num_workers=workers, num_verify_rows=len(ROWS))
    compare(got, ref, TOL_FP8, what=f"verify fp8 bs{bs} W{workers}")


def test_verify_f32_out():
    _announce("verify f32 out")
    w = _verify(ROWS, seed=3)
    ref = oracle.paged_attention_workload(w)
    got = run_mixed(w, out_dtype="f32", num_verify_rows=len(ROWS))
    compare(got, ref, 5e-3, what="verify f32")


@pytest.mark.parametrize("hq,hkv,nmax", [(8, 8, 32), (16, 8, 16), (64, 8, 4), (4, 1, 8), (12, 3, 8)])
def test_verify_group_sizes(hq, hkv, nmax):
    """Column count n x G up to 32 for every group size (1, 2, 4, 8)."""
    _announce(f"verify group hq={hq} hkv={hkv} n<={nmax}")
    rows = [(nmax, nmax), (50, max(1, nmax // 2)), (700, nmax), (1500, 1)]
    w = _verify(rows, hq=hq, hkv=hkv, seed=hq + hkv)
    ref = oracle.paged_attention_workload(w)
    got = run_mixed(w, out_dtype="f32", num_verify_rows=len(rows))
    compare(got, ref, 5e-3, what=f"verify G={hq // hkv}")


def test_verify_one_hot_probes_bit_exact():
    """One key scores ~130 (log2 units) above the rest: each query that sees it returns its V exactly.

    V encodes (physical block, slot) as a small integer, so a wrong gather is a
    wrong integer.  Targets sweep the first and last slot of every block; a target
    among the row's new tokens is seen only by the queries at or after it (causal).
    """
    _announce("verify one-hot probes")
    bs, L, n = 16, 200, 6
    w = _verify([(L, n)], bs=bs, hq=4, hkv=1, seed=8)
    nblk = (L + bs - 1) // bs
    assert w.num_blocks <= 16
    for j in range(nblk):
        phys = w.block_table[0, j]
        for sl in range(bs):
            w.v_pool[phys, 0, sl, :] = pa_inputs.to_bf16_bits(np.full(128, np.float32(phys * 16 + sl)))
    q = np.zeros((n, 4, 128), np.float32)
    q[:, :, 0] = 1.0
    w.q = pa_inputs.to_bf16_bits(q)
    targets = sorted({t for j in range(nblk) for t in (j * bs, min(j * bs + bs - 1, L - 1))}
                     | set(range(L - n, L)))
    for tstar in targets:
        w.k_pool[...] = 0
        phys = w.block_table[0, tstar // bs]
        w.k_pool[phys, 0, tstar % bs, 0] = pa_inputs.to_bf16_bits(np.array([1024.0], np.float32))[0]
        pa_inputs.poison_pool(w)
        got = run_mixed(w, out_dtype="f32", num_workers=3, num_verify_rows=1)
        exp = float(phys * 16 + tstar % bs)
        for i in range(n):
            if tstar <= L - n + i:
                assert np.all(got[i] == exp), (tstar, i, got[i, 0, :4], exp)
            else:     # not visible to query i: all its scores are 0, the mean of its visible V
                ref = oracle.paged_attention_workload(w)
                compare(got[i], ref[i], 1e-4, rel_tol=1e-5, what=f"probe {tstar} query {i}")


def test_verify_constant_v_exact():
    _announce("verify constant V")
    w = _verify([(3, 3), (40, 8), (1000, 4), (3000, 2)], seed=7)
    w.v_pool[...] = np.uint16(0x4000)       # 2.0
    pa_inputs.poison_pool(w)
    for nw in (0, 1, 13, 500):
        got = run_mixed(w, out_dtype="f32", num_workers=nw, num_verify_rows=4)
        np.testing.assert_array_equal(got, 2.0)


def test_verify_split_invariance():
    """Same bound as the decode split test: splits differ only in where P is rounded."""
    _announce("verify split invariance")
    rows = [(50, 4), (1000, 8), (2500, 2), (4096, 5)]
    w = _verify(rows, seed=12)
    ref = oracle.paged_attention_workload(w)
    outs = [run_mixed(w, out_dtype="f32", num_workers=nw, num_verify_rows=4) for nw in (1, 2, 9, 64, 1000, 0)]
    for nw, o in zip((1, 2, 9, 64, 1000, 0), outs):
        compare(o, ref, 5e-3, what=f"verify split {nw}")
        assert np.max(np.abs(o - outs[0])) <= 8e-3


def test_verify_block_permutation_bit_identical():
    _announce("verify block permutation")
    w = _verify([(33, 3), (700, 8), (1500, 5), (16, 8)], seed=10)
    a = run_mixed(w, out_dtype="f32", num_verify_rows=4)
    rng = np.random.default_rng(98)
    perm = rng.permutation(w.num_blocks)
    inv = np.argsort(perm)
    w.k_pool = np.ascontiguousarray(w.k_pool[inv])
    w.v_pool = np.ascontiguousarray(w.v_pool[inv])
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    b = run_mixed(w, out_dtype="f32", num_verify_rows=4)
    np.testing.assert_array_equal(a, b)


def test_verify_queries_match_decode_rows():
    """Query i of a verify row (L, n) is a decode row of length L - n + i + 1 over the same cache."""
    _announce("verify queries vs decode rows")
    L, n = 777, 8
    w = _verify([(L, n)], seed=5, poison=False)
    got = run_mixed(w, out_dtype="f32", num_verify_rows=1)
    d = pa_inputs.make_workload(name="dec", seq_lens=[L - n + i + 1 for i in range(n)], seed=5)
    d.block_table = np.repeat(w.block_table[:1], n, axis=0)
    d.k_pool, d.v_pool, d.q = w.k_pool, w.v_pool, w.q.copy()
    dec = run_decode(d, out_dtype="f32")
    assert np.max(np.abs(got - dec)) <= 5e-3


def test_mixed_three_row_classes():
    """Decode, verify and prefill rows in one pa_mixed call."""
    _announce("mixed decode + verify + prefill")
    w = _verify([(100, 4), (2049, 8), (9, 2)], dec_lens=[1, 300, 4000], pre=[(0, 40), (500, 100)], seed=21)
    ref = oracle.paged_attention_workload(w)
    got = run_mixed(w, num_verify_rows=3)
    compare(got, ref, TOL_BF16, what="three classes")


def test_verify_surplus_workers():
    _announce("verify surplus workers")
    w = _verify([(1, 1), (3, 2), (20, 8)], seed=14)
    ref = oracle.paged_attention_workload(w)
    got = run_mixed(w, out_dtype="f32", num_workers=4000, num_verify_rows=3)
    compare(got, ref, 5e-3, what="verify surplus workers")


def test_verify_full_size_workload():
    _announce(f"workload 6: {pa_inputs.WORKLOAD_NAMES[6]}")
    w = pa_inputs.make_config(6)
    got = run_mixed(w, num_verify_rows=w.num_seqs)
    ref = oracle.paged_attention_workload(w)
    compare(got, ref, TOL_BF16, what=f"workload 6, all {w.num_seqs} rows ({w.total_q} queries)")
    for b in range(w.num_seqs):
        a, e = w.q_start_loc[b], w.q_start_loc[b + 1]
        rel = np.linalg.norm(got[a:e] - ref[a:e]) / np.linalg.norm(ref[a:e])
        assert rel <= TOL_REL_L2, (b, rel)

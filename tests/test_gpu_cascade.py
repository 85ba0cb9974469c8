"""GPU parity of the shared-prefix (cascade) decode call against the fp64 oracle.

Rows in a group alias the same physical prefix blocks; the oracle simply
follows each row's table, so it knows nothing of the sharing.  Every case
prints its name first.
"""
import numpy as np
import pytest

import oracle
import pa_inputs
from gpu_util import TOL_BF16, TOL_REL_L2, compare, run_cascade, run_decode

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _shared(group_sizes, shared_lens, own_lens, prefix_ids=None, bs=16, hq=32, hkv=8, seed=0, poison=True):
    return pa_inputs.make_shared_prefix_workload(name="shared", group_sizes=group_sizes, shared_lens=shared_lens,
                                                 own_lens=own_lens, prefix_ids=prefix_ids, num_q_heads=hq,
                                                 num_kv_heads=hkv, block_size=bs, seed=seed, extra_blocks=3,
                                                 poison_unused=poison)


def _case(bs, seed):
    rng = np.random.default_rng(seed)
    groups = [8, 1, 3, 5, 2, 8]
    shared = [bs * k for k in (20, 0, 3, 64, 1, 5)]
    own = rng.integers(1, 700, size=sum(groups)).tolist()
    own[0], own[1] = 1, 2 * bs               # a single own token; an own part of whole blocks
    return _shared(groups, shared, own, prefix_ids=[0, 1, 2, 3, 4, 0], bs=bs, seed=seed)


@pytest.mark.parametrize("bs", [16, 32, 64, 128])
@pytest.mark.parametrize("workers", [0, 1, 7, 300])
def test_cascade_ragged(bs, workers):
    _announce(f"cascade ragged bs={bs} workers={workers}")
    w = _case(bs, seed=bs + workers)
    ref = oracle.paged_attention_workload(w)
    got = run_cascade(w, num_workers=workers)
    compare(got, ref, TOL_BF16, what=f"cascade bs{bs} W{workers}")


def test_cascade_f32_out_and_equals_decode():
    """Same rows through pa_decode (each row reads its whole cache) and the cascade call."""
    _announce("cascade vs decode, f32 out")
    w = _case(16, seed=3)
    ref = oracle.paged_attention_workload(w)
    got = run_cascade(w, out_dtype="f32")
    dec = run_decode(w, out_dtype="f32")
    compare(got, ref, 5e-3, what="cascade f32")
    compare(dec, ref, 5e-3, what="decode f32")
    assert np.max(np.abs(got - dec)) <= 8e-3


@pytest.mark.parametrize("hq,hkv,gmax", [(8, 8, 32), (16, 8, 16), (64, 8, 4), (4, 1, 8), (12, 3, 8)])
def test_cascade_group_sizes(hq, hkv, gmax):
    """Up to 32 query columns (rows x group size) per kv head for every group size."""
    _announce(f"cascade hq={hq} hkv={hkv} rows<={gmax}")
    groups = [gmax, 1, max(1, gmax // 2)]
    own = list(np.random.default_rng(hq).integers(1, 300, size=sum(groups)))
    w = _shared(groups, [160, 32, 0], own, hq=hq, hkv=hkv, seed=hq + hkv)
    ref = oracle.paged_attention_workload(w)
    got = run_cascade(w, out_dtype="f32")
    compare(got, ref, 5e-3, what=f"cascade G={hq // hkv}")


def test_cascade_constant_v_exact():
    _announce("cascade constant V")
    w = _case(16, seed=7)
    w.v_pool[...] = np.uint16(0x4000)        # 2.0
    pa_inputs.poison_pool(w)
    for nw in (0, 1, 13, 500):
        got = run_cascade(w, out_dtype="f32", num_workers=nw)
        np.testing.assert_array_equal(got, 2.0)


def test_cascade_one_hot_probes_bit_exact():
    """One key scores ~130 (log2 units) above the rest: the output is exactly its V.

    V encodes (physical block, slot) as a small integer.  Targets in the shared
    prefix are seen by every row of the group; targets in a row's own blocks by
    that row only, the others then average the rest (checked against the oracle).
    """
    _announce("cascade one-hot probes")
    bs = 16
    w = _shared([3], [64], [40, 1, 17], hq=4, hkv=1, bs=bs, seed=8)
    assert w.num_blocks <= 16
    for phys in range(w.num_blocks):
        for sl in range(bs):
            w.v_pool[phys, 0, sl, :] = pa_inputs.to_bf16_bits(np.full(128, np.float32(phys * 16 + sl)))
    q = np.zeros((3, 4, 128), np.float32)
    q[:, :, 0] = 1.0
    w.q = pa_inputs.to_bf16_bits(q)
    for r, t in [(0, 0), (0, 15), (0, 16), (0, 63), (0, 64), (0, 103), (1, 64), (2, 80)]:
        w.k_pool[...] = 0
        phys = w.block_table[r, t // bs]
        w.k_pool[phys, 0, t % bs, 0] = pa_inputs.to_bf16_bits(np.array([1024.0], np.float32))[0]
        pa_inputs.poison_pool(w)
        got = run_cascade(w, out_dtype="f32", num_workers=5)
        exp = float(phys * 16 + t % bs)
        for row in range(3):
            if t < 64 or row == r:
                assert np.all(got[row] == exp), (r, t, row, got[row, 0, :4], exp)
            else:
                ref = oracle.paged_attention_workload(w)
                compare(got[row], ref[row], 1e-4, rel_tol=1e-5, what=f"probe {r},{t} row {row}")


def test_cascade_block_permutation_bit_identical():
    _announce("cascade block permutation")
    w = _case(16, seed=10)
    a = run_cascade(w, out_dtype="f32")
    rng = np.random.default_rng(97)
    perm = rng.permutation(w.num_blocks)
    inv = np.argsort(perm)
    w.k_pool = np.ascontiguousarray(w.k_pool[inv])
    w.v_pool = np.ascontiguousarray(w.v_pool[inv])
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    b = run_cascade(w, out_dtype="f32")
    np.testing.assert_array_equal(a, b)


def test_cascade_no_shared_prefix_at_all():
    """Every group with an empty shared part: the prefix kernel has no work."""
    _announce("cascade without shared blocks")
    w = _shared([1, 2, 1], [0, 0, 0], [5, 100, 33, 1], seed=11)
    ref = oracle.paged_attention_workload(w)
    got = run_cascade(w, out_dtype="f32")
    compare(got, ref, 5e-3, what="no prefix")


def test_cascade_full_size_workload():
    _announce(f"workload 7: {pa_inputs.WORKLOAD_NAMES[7]}")
    w = pa_inputs.make_config(7)
    got = run_cascade(w)
    ref = oracle.paged_attention_workload(w)
    compare(got, ref, TOL_BF16, what=f"workload 7, all {w.num_seqs} rows")
    for b in range(w.num_seqs):
        rel = np.linalg.norm(got[b] - ref[b]) / np.linalg.norm(ref[b])
        assert rel <= TOL_REL_L2, (b, rel)

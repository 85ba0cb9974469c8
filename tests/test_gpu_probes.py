"""Bit-exact block-table indexing on the GPU: one-hot probes and the physical-permutation identity.

Every probed query's output must equal, bit for bit, the V vector of its
target slot, which encodes (physical block, kv head, slot) as small integers
(tests/probes.py; tests/test_probes.py checks on the CPU that the oracle gives
exactly these values).  Probes run with 8 kv heads and 4 query heads per kv
head, 16-, 32-, 64- and 128-token blocks, the
library's worker count and an explicit split, for every kernel that reads the cache: the decode kernels (bf16, fp32),
the multi-query kernel (FP8 decode rows, verify rows, shared prefixes) and the
prefill-chunk kernel; then at the full size of every named workload in the
launch configuration the benchmark times.

The permutation identity: relabelling the physical blocks (pool permuted,
table renumbered) must leave every output bit unchanged, because the kernels'
reduction order depends on logical positions only.
"""
import numpy as np
import pytest

import pa_inputs
from gpu_util import run_cascade, run_decode, run_mixed
from probes import DeviceProbe, OneHotProbe

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _workload(seq_lens, q_lens=None, bs=16, kv_fmt="bf16", q_fmt="bf16", hq=32, hkv=8, seed=0, extra_blocks=3):
    return pa_inputs.make_workload(name="probe", seq_lens=seq_lens, q_lens=q_lens, num_q_heads=hq,
                                   num_kv_heads=hkv, head_dim=128, block_size=bs, q_fmt=q_fmt, kv_fmt=kv_fmt,
                                   seed=seed, extra_blocks=extra_blocks, poison_unused=True)


def _sweep(w, run, probe=None, launches=None, what=""):
    """Run the probe's launches through ``run(w, dev)`` and require bit-exact outputs."""
    from paged_kv_attention_13_amd.device import to_device
    probe = probe or OneHotProbe(w)
    probe.prepare()
    d = to_device(w)
    dp = DeviceProbe(probe, d)
    n = launches or probe.num_launches()
    print(f"[{what}] {n} launches", flush=True)
    for r in range(n):
        exp, checked = dp.set_launch(r)
        got = run(w, d)
        bad = np.nonzero(np.any(got[checked] != exp[checked], axis=(1, 2)))[0]
        assert len(bad) == 0, (what, r, np.nonzero(checked)[0][bad[:5]],
                               got[checked][bad[0], :, :8] if len(bad) else None)
    return n


SHORT = [1, 15, 16, 17, 63, 300, 1024]          # one workgroup per unit with the library's count
LONG = [1, 17, 100, 513, 1000, 2049, 3001]      # balanced split with partials and merge


@pytest.mark.parametrize("kv_fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("bs", [16, 64])
@pytest.mark.parametrize("rows", ["short", "long"])
@pytest.mark.parametrize("workers", [0, 37])
def test_decode_probes(kv_fmt, bs, rows, workers):
    _announce(f"decode probes kv={kv_fmt} bs={bs} rows={rows} workers={workers}")
    w = _workload(SHORT if rows == "short" else LONG, bs=bs, kv_fmt=kv_fmt, seed=bs + workers)
    _sweep(w, lambda w, d: run_decode(w, out_dtype="f32", num_workers=workers, dev=d),
           what=f"decode {kv_fmt} bs{bs} {rows} W{workers}")


@pytest.mark.parametrize("kv_fmt", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("bs", [32, 128])
@pytest.mark.parametrize("rows,workers", [("short", 0), ("long", 0), ("long", 37)])
def test_decode_probes_other_block_sizes(kv_fmt, bs, rows, workers):
    """32- and 128-token blocks (page size and slot arithmetic), fp32 pools included."""
    _announce(f"decode probes kv={kv_fmt} bs={bs} rows={rows} workers={workers}")
    q_fmt = "f32" if kv_fmt == "f32" else "bf16"
    w = _workload(SHORT if rows == "short" else LONG, bs=bs, kv_fmt=kv_fmt, q_fmt=q_fmt, seed=3 * bs + workers)
    _sweep(w, lambda w, d: run_decode(w, out_dtype="f32", num_workers=workers, dev=d),
           what=f"decode {kv_fmt} bs{bs} {rows} W{workers}")


@pytest.mark.parametrize("hq,hkv,kv_fmt", [(8, 8, "bf16"), (64, 8, "bf16"), (8, 8, "fp8"), (64, 8, "fp8"),
                                           (32, 8, "f32")])
def test_decode_probes_group_sizes(hq, hkv, kv_fmt):
    _announce(f"decode probes hq={hq} hkv={hkv} kv={kv_fmt}")
    q_fmt = "f32" if kv_fmt == "f32" else "bf16"
    w = _workload([1, 33, 700, 1500], kv_fmt=kv_fmt, q_fmt=q_fmt, hq=hq, hkv=hkv, seed=hq)
    _sweep(w, lambda w, d: run_decode(w, out_dtype="f32", num_workers=0, dev=d), what=f"G={hq // hkv} {kv_fmt}")


@pytest.mark.parametrize("kv_fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("bs", [16, 32, 64, 128])
@pytest.mark.parametrize("workers", [0, 23])
def test_verify_probes(kv_fmt, bs, workers):
    _announce(f"verify probes kv={kv_fmt} bs={bs} workers={workers}")
    ver = [(5, 5), (33, 3), (64, 8), (1000, 8), (2049, 4)]
    dec = [1, 700, 3000]
    w = _workload(dec + [L for L, _ in ver], [1] * len(dec) + [n for _, n in ver], bs=bs, kv_fmt=kv_fmt,
                  seed=bs + workers + 5)
    w.num_decode_rows = len(dec)
    _sweep(w, lambda w, d: run_mixed(w, out_dtype="f32", num_workers=workers, num_verify_rows=len(ver), dev=d),
           what=f"verify {kv_fmt} bs{bs} W{workers}")


@pytest.mark.parametrize("kv_fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("bs", [16, 32, 64, 128])
@pytest.mark.parametrize("workers", [0, 37, None])
def test_mixed_prefill_probes(kv_fmt, bs, workers):
    """Decode rows plus prefill-chunk rows whose kv pieces start in the middle of a page
    (few units: the launch cuts long units into pieces), with the diagonal among the targets.
    workers None: the prefill rows alone."""
    _announce(f"prefill probes kv={kv_fmt} bs={bs} workers={workers}")
    dec = [1, 300, 3000] if workers is not None else []
    workers = workers or 0
    pre = [(0, 64), (100, 256), (1000, 40), (37, 5), (2500, 33)]
    w = _workload(dec + [p + n for p, n in pre], [1] * len(dec) + [n for _, n in pre], bs=bs, kv_fmt=kv_fmt,
                  seed=bs + workers + 9)
    _sweep(w, lambda w, d: run_mixed(w, out_dtype="f32", num_workers=workers, dev=d),
           what=f"prefill {kv_fmt} bs{bs} W{workers}")


def test_prefill_probes_many_units():
    """Prefill rows with more units than resident workgroups (no kv pieces), bf16 output."""
    _announce("prefill probes, many units")
    pre = [(500, 1024), (0, 1024), (61, 700)]
    w = _workload([p + n for p, n in pre], [n for _, n in pre], bs=16, seed=77)
    _sweep(w, lambda w, d: run_mixed(w, dev=d), launches=4, what="prefill many units")


def test_prefill_probes_table_beyond_lds():
    """A prefill launch without kv pieces whose units visit more pages than the 1,024 block-table
    entries staged in LDS (one kv head, 8,224 new tokens after 16,384 cached, 16-token blocks:
    1,026 to 1,538 pages per unit; 257 units of 32 positions, more than half the resident
    workgroups, so no pieces): every load takes its block id from the table in global memory."""
    _announce("prefill probes, block table beyond the LDS staging")
    w = _workload([16384 + 8224], [8224], bs=16, hq=4, hkv=1, seed=91)
    _sweep(w, lambda w, d: run_mixed(w, out_dtype="f32", dev=d), launches=3, what="prefill table beyond LDS")


@pytest.mark.parametrize("bs", [16, 32, 64, 128])
@pytest.mark.parametrize("workers", [0, 7])
def test_cascade_probes(bs, workers):
    _announce(f"cascade probes bs={bs} workers={workers}")
    rng = np.random.default_rng(bs + workers)
    groups = [8, 1, 3, 5, 2, 8]
    shared = [bs * k for k in (20, 0, 3, 40, 1, 5)]
    own = rng.integers(1, 700, size=sum(groups)).tolist()
    own[0], own[1] = 1, 2 * bs
    w = pa_inputs.make_shared_prefix_workload(name="shared", group_sizes=groups, shared_lens=shared, own_lens=own,
                                              prefix_ids=[0, 1, 2, 3, 4, 0], block_size=bs, seed=bs + workers,
                                              extra_blocks=3, poison_unused=True)
    probe = OneHotProbe(w, shared_rows=True)
    _sweep(w, lambda w, d: run_cascade(w, out_dtype="f32", num_workers=workers, dev=d), probe=probe,
           launches=4, what=f"cascade bs{bs} W{workers}")


# ----------------------------------------------------------------------------
# full size, in the benchmark's launch configuration (library worker counts, bf16 out)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("i", [1, 2, 3, 4, 5, 6, 7])
def test_full_size_probes(i):
    _announce(f"full-size probes, workload {i}: {pa_inputs.WORKLOAD_NAMES[i]}")
    w = pa_inputs.make_config(i)
    if i in (1, 2, 3, 4):
        run = lambda w, d: run_decode(w, dev=d)                      # noqa: E731
    elif i == 5:
        run = lambda w, d: run_mixed(w, dev=d)                       # noqa: E731
    elif i == 6:
        run = lambda w, d: run_mixed(w, num_verify_rows=w.num_seqs, dev=d)  # noqa: E731
    else:
        run = lambda w, d: run_cascade(w, dev=d)                     # noqa: E731
    probe = OneHotProbe(w, shared_rows=(i == 7))
    _sweep(w, run, probe=probe, launches=2, what=f"workload {i}")


@pytest.mark.parametrize("case", ["w5-rows", "chunk256-after8192"])
def test_full_size_prefill_rows_probes(case):
    """Prefill rows alone at full size (kv pieces for the single chunk after 8,192 tokens)."""
    _announce(f"full-size prefill probes: {case}")
    w = pa_inputs.make_prefill_case(case)
    _sweep(w, lambda w, d: run_mixed(w, dev=d), launches=2, what=f"prefill {case}")


# ----------------------------------------------------------------------------
# physical-block permutation: bit-identical outputs
# ----------------------------------------------------------------------------

def _permuted(w, seed):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(w.num_blocks)
    inv = np.argsort(perm)
    w2 = pa_inputs.Workload(**{**w.__dict__})
    w2.k_pool = np.ascontiguousarray(w.k_pool[inv])
    w2.v_pool = np.ascontiguousarray(w.v_pool[inv])
    w2.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    return w2


@pytest.mark.parametrize("bs", [16, 64])
@pytest.mark.parametrize("workers", [0, 37])
def test_fp8_decode_block_permutation_bit_identical(bs, workers):
    _announce(f"fp8 decode block permutation bs={bs} workers={workers}")
    w = _workload(LONG, bs=bs, kv_fmt="fp8", seed=300 + bs + workers)
    a = run_decode(w, num_workers=workers)
    b = run_decode(_permuted(w, 7 + bs), num_workers=workers)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("kv_fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("bs", [16, 64])
@pytest.mark.parametrize("dec", [[1, 300, 3000], []])
def test_prefill_block_permutation_bit_identical(kv_fmt, bs, dec):
    _announce(f"prefill block permutation kv={kv_fmt} bs={bs} decode rows {dec}")
    pre = [(0, 64), (100, 256), (1000, 40), (2500, 33)]
    w = _workload(dec + [p + n for p, n in pre], [1] * len(dec) + [n for _, n in pre], bs=bs, kv_fmt=kv_fmt,
                  seed=400 + bs)
    a = run_mixed(w)
    b = run_mixed(_permuted(w, 11 + bs))
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("bs", [16, 64])
def test_fp8_verify_block_permutation_bit_identical(bs):
    _announce(f"fp8 verify block permutation bs={bs}")
    ver = [(5, 5), (700, 8), (1500, 5), (16, 8)]
    w = _workload([L for L, _ in ver], [n for _, n in ver], bs=bs, kv_fmt="fp8", seed=500 + bs)
    w.num_decode_rows = 0
    a = run_mixed(w, num_verify_rows=len(ver))
    b = run_mixed(_permuted(w, 13 + bs), num_verify_rows=len(ver))
    np.testing.assert_array_equal(a, b)

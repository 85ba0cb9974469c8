"""CPU checks of the one-hot probe construction used by the GPU gather tests.

The probe's expected outputs come from the construction alone (the digits of
the target slot).  Here the fp64 oracle, fed the same inputs, must give exactly
those values, on every probed query, for decode, verify, prefill and
shared-prefix rows and for every storage format, so a GPU result that equals
them is the oracle's result bit for bit.
"""
import numpy as np
import pytest

import oracle
import pa_inputs
from probes import OneHotProbe, digit_lut, digit_pool, slot_digits


def test_digit_encodings_are_exact():
    for fmt in ("f32", "bf16", "fp8"):
        lut = digit_lut(fmt)
        np.testing.assert_array_equal(oracle.stored_to_f64(lut, fmt), np.arange(16, dtype=np.float64))


def test_digit_pool_names_its_slot():
    pool = digit_pool(300, 8, 16, "bf16")
    vals = oracle.stored_to_f64(pool, "bf16")
    for p, g, s in [(0, 0, 0), (299, 7, 15), (17, 3, 9), (256, 5, 1)]:
        np.testing.assert_array_equal(vals[p, g, s], slot_digits(p, g, s))
    # distinct slots hold distinct vectors
    flat = vals[:, :, :, :8].reshape(-1, 8)
    assert len(np.unique(flat, axis=0)) == flat.shape[0]


def _check(w, probe, launches=None):
    probe.prepare()
    for r in range(launches or probe.num_launches()):
        exp, checked = probe.apply_host(r)
        ref = oracle.paged_attention_workload(w)
        np.testing.assert_array_equal(ref[checked], exp[checked])


@pytest.mark.parametrize("kv_fmt,q_fmt", [("bf16", "bf16"), ("fp8", "bf16"), ("f32", "f32")])
def test_decode_probe_matches_oracle_exactly(kv_fmt, q_fmt):
    w = pa_inputs.make_workload(name="p", seq_lens=[1, 17, 64, 200], block_size=16, q_fmt=q_fmt, kv_fmt=kv_fmt,
                                seed=3, extra_blocks=2, poison_unused=True)
    _check(w, OneHotProbe(w))


def test_prefill_and_verify_probe_matches_oracle_exactly():
    # decode rows, a verify-like row and prefill rows with more than 128 / G queries
    w = pa_inputs.make_workload(name="p", seq_lens=[5, 90, 40 + 7, 3 + 40], q_lens=[1, 1, 7, 40], block_size=16,
                                seed=4, extra_blocks=2, poison_unused=True)
    _check(w, OneHotProbe(w), launches=3)


def test_shared_prefix_probe_matches_oracle_exactly():
    w = pa_inputs.make_shared_prefix_workload(name="s", group_sizes=[3, 2], shared_lens=[32, 16], own_lens=[5, 1, 20, 9, 2],
                                              prefix_ids=[0, 0], block_size=16, seed=5, extra_blocks=2,
                                              poison_unused=True)
    _check(w, OneHotProbe(w, shared_rows=True), launches=2)


def test_probe_detects_a_planted_gather_mistake():
    """An oracle that reads slot (t + 1) % bs instead of t % bs fails the probe."""
    w = pa_inputs.make_workload(name="p", seq_lens=[40], block_size=16, seed=6, poison_unused=False)
    probe = OneHotProbe(w)
    probe.prepare(poison=False)
    exp, checked = probe.apply_host(0, poison=False)
    bad = pa_inputs.Workload(**{**w.__dict__})
    # shift every block's slots by one (a wrong slot index in the gather)
    bad.k_pool = np.roll(w.k_pool, 1, axis=2)
    bad.v_pool = np.roll(w.v_pool, 1, axis=2)
    ref = oracle.paged_attention_workload(bad)
    assert not np.array_equal(ref[checked], exp[checked])

"""pa_decode_noalloc (the library's static scratch instead of a caller workspace) against pa_decode.

Two calls in a row on one GPU share the static scratch, the second with a
smaller batch, so the second must not depend on what the first left there.
Both must equal pa_decode's output bit for bit (same kernels, same plan) and
match the fp64 oracle within the path's tolerance.
"""
import ctypes

import numpy as np
import pytest

import oracle
import pa_inputs
from gpu_util import TOL_BF16, TOL_FP8, compare


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _args(b, w, d, out, workers=0):
    return b.make_decode_args(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], w.scale,
                              max_seq_len=w.max_seq_len, k_scale=d["k_scale"], v_scale=d["v_scale"], out=out,
                              num_workers=workers)


@pytest.mark.gpu
@pytest.mark.parametrize("kv_fmt", ["bf16", "fp8"])
def test_noalloc_equals_pa_decode_on_two_calls(kv_fmt):
    import torch
    from paged_kv_attention_13_amd import binding as b
    from paged_kv_attention_13_amd.device import to_device
    cases = [(np.random.default_rng(1).integers(1, 6001, size=48).tolist(), 16, 0),     # larger first
             ([3000, 17, 1, 900, 64], 64, 0),                                           # then smaller
             ([2500, 700, 5], 16, 37)]                                                  # explicit split
    for k, (lens, bs, workers) in enumerate(cases):
        _announce(f"noalloc {kv_fmt} call {k}: {len(lens)} rows bs={bs} workers={workers}")
        w = pa_inputs.make_workload(name="noalloc", seq_lens=lens, block_size=bs, kv_fmt=kv_fmt, seed=10 * k + 3,
                                    extra_blocks=3, poison_unused=True)
        d = to_device(w)
        ref_out = torch.empty(d["q"].shape, dtype=torch.bfloat16, device="cuda")
        a = _args(b, w, d, ref_out, workers)
        assert b.decode_workspace_bytes(a) > 0               # the split path: partials are used
        ws = torch.empty(b.decode_workspace_bytes(a), dtype=torch.uint8, device="cuda")
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        b.decode_args_call(a)
        out = torch.full(d["q"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        n = _args(b, w, d, out, workers)
        n.workspace, n.workspace_bytes = 0x10, 1             # ignored by the no-allocation call
        b.decode_noalloc_args_call(n)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), k
        got = out.float().cpu().numpy().astype(np.float64)
        ref = oracle.paged_attention_workload(w)
        compare(got, ref, TOL_FP8 if kv_fmt == "fp8" else TOL_BF16, what=f"noalloc {kv_fmt} call {k}")


@pytest.mark.gpu
@pytest.mark.parametrize("rows", ["whole", "pieces"])
def test_noalloc_short_rows(rows):
    """Rows on the one-workgroup-per-unit path: with whole units (45 rows, 360 units) no
    partials at all; with few units (3 rows, 24 units, each cut over 10 workgroups) the
    pieces' partials go to the static scratch.  Both equal pa_decode bit for bit."""
    _announce(f"noalloc short rows, {rows}")
    import torch
    from paged_kv_attention_13_amd import binding as b
    from paged_kv_attention_13_amd.device import to_device
    lens = [1, 40, 1000] * (15 if rows == "whole" else 1)
    w = pa_inputs.make_workload(name="noalloc", seq_lens=lens, block_size=16, seed=5, extra_blocks=2,
                                poison_unused=True)
    d = to_device(w)
    ref_out = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    a = _args(b, w, d, ref_out)
    nbytes = b.decode_workspace_bytes(a)
    assert (nbytes == 0) == (rows == "whole")
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    b.decode_args_call(a)
    out = torch.full(d["q"].shape, float("nan"), dtype=torch.float32, device="cuda")
    n = _args(b, w, d, out)
    b.decode_noalloc_args_call(n)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    compare(out.cpu().numpy().astype(np.float64), oracle.paged_attention_workload(w), 5e-3, what="noalloc short")


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    """More partials than the 16 MiB static scratch: rejected before any launch (no GPU needed)."""
    from paged_kv_attention_13_amd import binding as b
    a = b.DecodeArgs()
    a.num_seqs, a.num_q_heads, a.num_kv_heads, a.head_dim = 4000, 32, 8, 128
    a.block_size, a.num_blocks, a.max_blocks_per_seq, a.max_seq_len = 16, 1 << 20, 512, 8192
    a.q_dtype = a.kv_dtype = a.out_dtype = b.PA_BF16
    a.q = a.k_pool = a.v_pool = a.out = a.block_table = a.seq_lens = 0x10000
    a.scale = 0.088
    assert b.decode_workspace_bytes(a) > 16 << 20
    rc = b.LIB.pa_decode_noalloc(ctypes.byref(a), None)
    assert b.STATUS_NAMES[rc] == "PA_ERR_WORKSPACE_TOO_SMALL"
    assert "static scratch" in b.LIB.pa_last_error().decode()
    assert b.STATUS_NAMES[b.LIB.pa_decode_noalloc(None, None)] == "PA_ERR_NULL_POINTER"
    a.num_seqs = 55
    a.q = 0x10008                                              # the usual checks still apply
    assert b.STATUS_NAMES[b.LIB.pa_decode_noalloc(ctypes.byref(a), None)] == "PA_ERR_MISALIGNED"

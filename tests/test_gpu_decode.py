"""GPU parity of the decode path (pa_decode and its two stages) against the fp64 oracle.

Every case prints its name before running so that a failing GPU step names
itself.  Inputs are seeded; the oracle never sees anything the GPU produced.
"""
import numpy as np
import pytest

import oracle
import pa_inputs
from gpu_util import TOL_BF16, TOL_F32, TOL_FP8, TOL_REL_L2, compare, run_decode

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _small(seq_lens, bs=16, kv_fmt="bf16", q_fmt="bf16", hq=32, hkv=8, seed=0, poison=True,
           extra_blocks=3):
    return pa_inputs.make_workload(name="small", seq_lens=seq_lens, num_q_heads=hq, num_kv_heads=hkv,
                                   head_dim=128, block_size=bs, q_fmt=q_fmt, kv_fmt=kv_fmt, seed=seed,
                                   extra_blocks=extra_blocks, poison_unused=poison)


RAGGED = [1, 2, 7, 15, 16, 17, 31, 33, 100, 127, 128, 129, 255, 300, 511, 513, 1000]


@pytest.mark.parametrize("bs", [16, 32, 64, 128])
@pytest.mark.parametrize("workers", [0, 1, 7, 300])
def test_bf16_ragged_lengths(bs, workers):
    _announce(f"bf16 ragged bs={bs} workers={workers}")
    w = _small(RAGGED, bs=bs, seed=bs + workers)
    ref = oracle.paged_attention_workload(w)
    got = run_decode(w, num_workers=workers)
    compare(got, ref, TOL_BF16, what=f"bf16 bs{bs} W{workers}")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_bf16_out_dtypes(out):
    _announce(f"bf16 kv, out={out}")
    w = _small([5, 64, 700, 2049], seed=3)
    ref = oracle.paged_attention_workload(w)
    got = run_decode(w, out_dtype=out)
    tol = 5e-3 if out == "f32" else TOL_BF16
    compare(got, ref, tol, what=f"out {out}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (64, 8), (4, 1), (12, 3)])
def test_group_sizes(hq, hkv):
    _announce(f"group size hq={hq} hkv={hkv}")
    w = _small([3, 77, 300, 1100], hq=hq, hkv=hkv, seed=hq * 10 + hkv)
    ref = oracle.paged_attention_workload(w)
    got = run_decode(w, out_dtype="f32")
    compare(got, ref, 5e-3, what=f"G={hq // hkv}")


def test_fp32_path():
    _announce("fp32 ragged")
    w = _small(RAGGED, q_fmt="f32", kv_fmt="f32", seed=11)
    ref = oracle.paged_attention_workload(w)
    got = run_decode(w)
    compare(got, ref, TOL_F32, rel_tol=1e-5, what="fp32")


@pytest.mark.parametrize("hq,hkv,workers", [(8, 8, 0), (16, 8, 77), (64, 8, 0), (64, 8, 300), (12, 3, 5)])
def test_fp32_group_sizes(hq, hkv, workers):
    """fp32 pools for every group size, through the one-workgroup-per-unit kernel (rows within
    1,024 tokens, workers 0) and the balanced split."""
    _announce(f"fp32 group hq={hq} hkv={hkv} workers={workers}")
    w = _small(RAGGED, q_fmt="f32", kv_fmt="f32", hq=hq, hkv=hkv, seed=90 + hq + workers)
    ref = oracle.paged_attention_workload(w)
    got = run_decode(w, num_workers=workers)
    compare(got, ref, TOL_F32, rel_tol=1e-5, what=f"fp32 G={hq // hkv} W{workers}")


@pytest.mark.parametrize("workers", [0, 3, 111])
def test_fp8_ragged(workers):
    _announce(f"fp8 ragged workers={workers}")
    w = _small(RAGGED, kv_fmt="fp8", seed=21 + workers)
    ref = oracle.paged_attention_workload(w)
    got = run_decode(w, num_workers=workers)
    compare(got, ref, TOL_FP8, what=f"fp8 W{workers}")


@pytest.mark.parametrize("hq,hkv,bs", [(8, 8, 16), (16, 8, 32), (64, 8, 16), (12, 3, 64), (4, 1, 128)])
def test_fp8_group_sizes(hq, hkv, bs):
    """FP8 pools for every group size (1, 2, 4, 8 query heads per kv head) and block size."""
    _announce(f"fp8 group hq={hq} hkv={hkv} bs={bs}")
    w = _small(RAGGED, kv_fmt="fp8", hq=hq, hkv=hkv, bs=bs, seed=hq + hkv + bs)
    ref = oracle.paged_attention_workload(w)
    got = run_decode(w, out_dtype="f32")
    compare(got, ref, TOL_FP8, what=f"fp8 G={hq // hkv} bs{bs}")


def test_fp8_every_code_decodes_exactly():
    """Single cached token: out = v_scale * E4M3(code), every one of the 256 codes."""
    _announce("fp8 all codes")
    w = _small([1], kv_fmt="fp8", hq=2, hkv=2, seed=5, poison=False, extra_blocks=0)
    codes = np.arange(256, dtype=np.uint8).reshape(2, 128)
    w.v_pool[0, :, 0, :] = codes
    w.v_scale = np.ones(2, dtype=np.float32)
    got = run_decode(w, out_dtype="f32")[0]
    exp = oracle.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(exp))
    ok = ~np.isnan(exp)
    np.testing.assert_array_equal(got[ok], exp[ok])


def test_single_token_returns_its_value_exactly():
    _announce("single token")
    w = _small([1, 1, 1], seed=6)
    got = run_decode(w, out_dtype="f32")
    ref = oracle.paged_attention_workload(w)
    np.testing.assert_array_equal(got, ref)


def test_constant_v_is_exact():
    _announce("constant V")
    w = _small([1, 40, 1000, 3000], seed=7)
    w.v_pool[...] = np.uint16(0x4000)       # 2.0
    pa_inputs.poison_pool(w)
    for nw in (0, 1, 13, 500):
        got = run_decode(w, out_dtype="f32", num_workers=nw)
        np.testing.assert_array_equal(got, 2.0)


def test_one_hot_probes_bit_exact():
    """One key scores 2^8 above all others: the output is exactly that token's V.

    V holds small integers (exact in bf16) that encode (physical block, slot),
    so a wrong gather shows up as a wrong integer.  t* sweeps the first and
    last slot of every block and the last token.
    """
    _announce("one-hot probes")
    bs = 16
    L = 200
    w = _small([L], bs=bs, hq=4, hkv=1, seed=8)
    nblk = (L + bs - 1) // bs
    # V[phys][0][slot][:] = phys * 16 + slot: integers < 256, exact in bf16
    assert w.num_blocks <= 16
    for j in range(nblk):
        phys = w.block_table[0, j]
        for sl in range(bs):
            val = np.float32(phys * 16 + sl)
            w.v_pool[phys, 0, sl, :] = pa_inputs.to_bf16_bits(np.full(128, val, np.float32))
    q = np.zeros((1, 4, 128), np.float32)
    q[0, :, 0] = 1.0
    w.q = pa_inputs.to_bf16_bits(q)
    targets = sorted({t for j in range(nblk) for t in (j * bs, min(j * bs + bs - 1, L - 1))} | {L - 1})
    for tstar in targets:
        w.k_pool[...] = 0
        phys = w.block_table[0, tstar // bs]
        # score gap: 1024 * scale * log2(e) ~ 130 (log2 units): others underflow to 0
        w.k_pool[phys, 0, tstar % bs, 0] = pa_inputs.to_bf16_bits(np.array([1024.0], np.float32))[0]
        pa_inputs.poison_pool(w)
        got = run_decode(w, out_dtype="f32", num_workers=5)
        exp = float(phys * 16 + tstar % bs)
        assert np.all(got[0] == exp), (tstar, got[0, 0, :4], exp)


def test_uniform_probe_mean():
    """q = 0: every visible token gets the same weight; the output is the mean of V."""
    _announce("q=0 mean")
    w = _small([1, 17, 640, 1500], seed=9)
    w.q[...] = 0
    got = run_decode(w, out_dtype="f32")
    ref = oracle.paged_attention_workload(w)
    compare(got, ref, 1e-5, rel_tol=1e-4, what="mean")


def test_block_permutation_bit_identical():
    _announce("block permutation")
    w = _small([33, 700, 1500, 16], seed=10)
    a = run_decode(w, out_dtype="f32")
    rng = np.random.default_rng(99)
    perm = rng.permutation(w.num_blocks)
    inv = np.argsort(perm)
    w.k_pool = np.ascontiguousarray(w.k_pool[inv])
    w.v_pool = np.ascontiguousarray(w.v_pool[inv])
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    b = run_decode(w, out_dtype="f32")
    np.testing.assert_array_equal(a, b)


def test_split_invariance():
    """The result does not depend on how the work is split across workers.

    Splits differ only in where P is rounded to bf16 (relative 2^-9 per weight,
    at a different running max): |o' - o| <= 2 * 2^-9 * max|v - o| ~ 8e-3 for
    N(0,1) values.  Every split is also checked against the oracle.
    """
    _announce("split invariance")
    w = _small([50, 1000, 2500, 4096], seed=12)
    ref = oracle.paged_attention_workload(w)
    outs = [run_decode(w, out_dtype="f32", num_workers=nw) for nw in (1, 2, 9, 64, 1000, 0)]
    for nw, o in zip((1, 2, 9, 64, 1000, 0), outs):
        compare(o, ref, 5e-3, what=f"split {nw}")
        assert np.max(np.abs(o - outs[0])) <= 8e-3


@pytest.mark.parametrize("rows", ["few", "many"])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (32, 8), (64, 8)])
def test_short_rows_one_workgroup_per_unit(hq, hkv, rows):
    """Rows within 1,024 tokens with the worker count left to the library run one workgroup
    per (row, kv head), its waves merged in LDS; with fewer units than CUs ("few": 72 units,
    each cut over 3 workgroups whose partials the merge kernel combines), else whole units
    and no workspace ("many": 360 units).  Both match the oracle and the balanced split of
    the same rows."""
    _announce(f"one workgroup per unit, hq={hq} hkv={hkv} rows={rows}")
    from paged_kv_attention_13_amd import binding
    lens = [1, 15, 16, 17, 48, 63, 300, 1000, 1024]
    if rows == "many":
        lens = lens * 5
    w = _small(lens, hq=hq, hkv=hkv, seed=60 + hq + len(lens))
    a = binding.DecodeArgs()
    a.num_seqs, a.num_q_heads, a.num_kv_heads, a.head_dim = w.num_seqs, hq, hkv, 128
    a.block_size, a.num_blocks, a.max_blocks_per_seq = w.block_size, w.num_blocks, w.max_blocks_per_seq
    a.max_seq_len, a.q_dtype, a.kv_dtype, a.out_dtype = w.max_seq_len, 1, 1, 1
    pl = binding.plan(a)
    if rows == "many":
        assert pl.workspace_bytes == 0
    else:
        assert pl.workspace_bytes > 0 and pl.num_workers == w.num_seqs * hkv * 3
    ref = oracle.paged_attention_workload(w)
    unit = run_decode(w, out_dtype="f32")
    split = run_decode(w, out_dtype="f32", num_workers=37)
    compare(unit, ref, 5e-3, what="one workgroup per unit")
    compare(split, ref, 5e-3, what="split")
    assert np.max(np.abs(unit - split)) <= 8e-3


def test_short_rows_constant_v_exact():
    _announce("one workgroup per unit, constant V")
    w = _small([1, 40, 1000, 7], seed=71)
    w.v_pool[...] = np.uint16(0x4000)       # 2.0
    pa_inputs.poison_pool(w)
    np.testing.assert_array_equal(run_decode(w, out_dtype="f32"), 2.0)


def test_many_workers_more_than_tiles():
    """More workers than tiles: surplus workers find an empty range and exit."""
    _announce("surplus workers")
    w = _small([1, 3, 20], seed=14)
    ref = oracle.paged_attention_workload(w)
    got = run_decode(w, out_dtype="f32", num_workers=4000)
    compare(got, ref, 5e-3, what="surplus workers")


@pytest.mark.parametrize("workers", [150, 600, 1500])
def test_workers_holding_only_start_up_tiles(workers):
    """Each (row, kv head) unit is charged a few virtual start-up tiles in the work split; with
    many one-token rows and short ranges, some workers hold only virtual tiles (they skip the
    unit) and the real tiles of one unit still go to consecutive workers."""
    _announce(f"virtual start-up tiles, {workers} workers")
    lens = [1] * 40 + [2000] + [1, 17, 1] * 5
    w = _small(lens, seed=19)
    ref = oracle.paged_attention_workload(w)
    got = run_decode(w, out_dtype="f32", num_workers=workers)
    compare(got, ref, 5e-3, what=f"virtual tiles, {workers} workers")
    w.v_pool[...] = np.uint16(0x4000)       # 2.0
    pa_inputs.poison_pool(w)
    np.testing.assert_array_equal(run_decode(w, out_dtype="f32", num_workers=workers), 2.0)


@pytest.mark.parametrize("rows,workers", [(700, 0), (700, 37), (700, 1500), (64, 0), (65, 0)])
def test_many_short_rows(rows, workers):
    """Rows of 1..300 tokens.  700 rows: the split's prefix scan and row search run over 11 chunks
    of 64 rows.  With the worker count left to the library, 64 rows (512 units) still run one
    workgroup per (row, kv head) and 65 rows (520 units) go to the balanced split."""
    _announce(f"{rows} short rows, {workers} workers")
    from paged_kv_attention_13_amd import binding
    from paged_kv_attention_13_amd.device import to_device
    lens = np.random.default_rng(23).integers(1, 301, size=rows)
    w = _small(lens.tolist(), seed=23)
    d = to_device(w)
    a = binding.make_decode_args(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], w.scale,
                                 max_seq_len=w.max_seq_len, num_workers=workers)
    assert (binding.plan(a).workspace_bytes == 0) == (workers == 0 and rows * 8 <= 512)
    ref = oracle.paged_attention_workload(w)
    got = run_decode(w, out_dtype="f32", num_workers=workers, dev=d)
    compare(got, ref, 5e-3, what=f"{rows} rows, {workers} workers")


def test_stages_equal_one_call():
    """pa_decode_partials followed by pa_merge_partials equals pa_decode."""
    _announce("stages")
    import torch
    from paged_kv_attention_13_amd import binding
    from paged_kv_attention_13_amd.device import to_device
    w = _small([300, 1200, 64], seed=13)
    d = to_device(w)
    out1 = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out1)
    a = binding.make_decode_args(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"],
                                 w.scale, max_seq_len=w.max_seq_len, out=out1, num_workers=10)
    pl = binding.plan(a)
    assert pl.num_workers == 10 and pl.workspace_bytes > 0
    ws = torch.empty(pl.workspace_bytes, dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), pl.workspace_bytes
    binding.decode_partials(a)
    binding.merge_partials(a)
    a.out = out2.data_ptr()
    binding.decode_args_call(a)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


@pytest.mark.parametrize("kv_fmt,workers", [("bf16", 37), ("fp8", 0)])
def test_merge_on_a_foreign_workspace_stays_in_bounds(kv_fmt, workers):
    """The merge reads each cut unit's (first worker, count) record from the workspace, and a
    record that did not come from a partials call on that workspace is clamped to the launch's
    slots: pa_merge_partials on random bytes completes (its outputs are meaningless), and the
    library is sound afterwards (a partials call then the merge match the oracle)."""
    _announce(f"merge on a foreign workspace: {kv_fmt} workers={workers}")
    import torch
    from paged_kv_attention_13_amd import binding
    from paged_kv_attention_13_amd.device import to_device
    w = _small([300, 1200, 64, 2500], kv_fmt=kv_fmt, seed=71)
    d = to_device(w)
    out = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    a = binding.make_decode_args(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], w.scale,
                                 max_seq_len=w.max_seq_len, k_scale=d["k_scale"], v_scale=d["v_scale"], out=out,
                                 num_workers=workers)
    pl = binding.plan(a)
    assert pl.workspace_bytes > 0
    gen = torch.Generator(device="cuda").manual_seed(3)
    ws = torch.randint(0, 256, (pl.workspace_bytes,), dtype=torch.uint8, device="cuda", generator=gen)
    a.workspace, a.workspace_bytes = ws.data_ptr(), pl.workspace_bytes
    binding.merge_partials(a)
    torch.cuda.synchronize()
    binding.decode_partials(a)
    binding.merge_partials(a)
    torch.cuda.synchronize()
    compare(out.cpu().numpy().astype(np.float64), oracle.paged_attention_workload(w),
            TOL_FP8 if kv_fmt == "fp8" else 5e-3, what=f"{kv_fmt} after a foreign-workspace merge")


def test_empty_batch_is_a_no_op():
    _announce("empty batch")
    import torch
    from paged_kv_attention_13_amd import binding
    q = torch.zeros((0, 32, 128), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((1, 8, 16, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    sl = torch.zeros((0,), dtype=torch.int32, device="cuda")
    out = binding.decode(q, kp, kp, bt, sl, 0.1, max_seq_len=1)
    assert out.shape == (0, 32, 128)


# ----------------------------------------------------------------------------
# the named workloads at full size: every row against the oracle
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("i", [1, 2, 3, 4])
def test_named_workload_full_size(i):
    _announce(f"workload {i}: {pa_inputs.WORKLOAD_NAMES[i]}")
    w = pa_inputs.make_config(i)
    got = run_decode(w)
    ref = oracle.paged_attention_workload(w)
    tol = {1: TOL_F32, 2: TOL_BF16, 3: TOL_BF16, 4: TOL_FP8}[i]
    compare(got, ref, tol, what=f"workload {i}, all {w.num_seqs} rows")
    # per row too: a single wrong row cannot hide in the workload-wide relative error
    for b in range(w.num_seqs):
        rel = np.linalg.norm(got[b] - ref[b]) / np.linalg.norm(ref[b])
        assert rel <= TOL_REL_L2, (b, rel)


@pytest.mark.parametrize("workers", [0, 9])
def test_one_very_long_row(workers):
    """One row of 131,072 tokens in 128-token blocks (1,024 pages: 16 block-table chunks of 64,
    256 MiB per pool) next to a one-token row."""
    _announce(f"131072-token row, workers={workers}")
    w = _small([131072, 1], bs=128, seed=80 + workers, extra_blocks=1)
    ref = oracle.paged_attention_workload(w)
    got = run_decode(w, out_dtype="f32", num_workers=workers)
    compare(got, ref, 5e-3, what="very long row")

"""GPU parity of pa_mixed (decode rows + causal prefill-chunk rows) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import pa_inputs
from gpu_util import TOL_BF16, TOL_FP8, TOL_REL_L2, compare, run_mixed

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _mixed(dec_lens, pre, bs=16, hq=32, hkv=8, seed=0, poison=True, kv_fmt="bf16"):
    """dec_lens: decode-row lengths; pre: list of (prior, q_len) prefill rows."""
    L = list(dec_lens) + [p + n for p, n in pre]
    ql = [1] * len(dec_lens) + [n for _, n in pre]
    return pa_inputs.make_workload(name="mixed", seq_lens=L, q_lens=ql, num_q_heads=hq, num_kv_heads=hkv,
                                   head_dim=128, block_size=bs, seed=seed, extra_blocks=3,
                                   poison_unused=poison, kv_fmt=kv_fmt)


PRE = [(0, 1), (0, 5), (0, 64), (3, 29), (17, 33), (100, 64), (250, 130), (0, 256), (1000, 96)]


@pytest.mark.parametrize("bs", [16, 32, 64, 128])
def test_mixed_ragged(bs):
    _announce(f"mixed ragged bs={bs}")
    w = _mixed([1, 40, 700, 3000], PRE, bs=bs, seed=bs)
    ref = oracle.paged_attention_workload(w)
    got = run_mixed(w)
    compare(got, ref, TOL_BF16, what=f"mixed bs{bs}")


def test_prefill_only_f32_out():
    _announce("prefill only, f32 out")
    w = _mixed([], PRE, seed=3)
    ref = oracle.paged_attention_workload(w)
    got = run_mixed(w, out_dtype="f32")
    compare(got, ref, 1e-2, what="prefill f32 out")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (64, 8), (32, 8)])
@pytest.mark.parametrize("dec", [[33], []])
def test_prefill_group_sizes(hq, hkv, dec):
    """Every group size, beside a decode row (prefill on the auxiliary stream) and alone."""
    _announce(f"prefill group hq={hq} hkv={hkv} decode rows {dec}")
    w = _mixed(dec, [(0, 40), (70, 100), (5, 200), (300, 333)], hq=hq, hkv=hkv, seed=hq + len(dec))
    ref = oracle.paged_attention_workload(w)
    got = run_mixed(w, out_dtype="f32")
    compare(got, ref, 1e-2, what=f"prefill G={hq // hkv}")


def test_decode_row_equals_last_prefill_query():
    """The last query of a prefill row and a decode row over the same cache agree."""
    _announce("decode vs last prefill query")
    w = _mixed([300], [(299 - 63, 64)], seed=5, poison=False)
    w.block_table[1] = w.block_table[0]          # same cache, L = 300 for both rows
    w.q[0] = w.q[1 + 63]                         # same query vector
    got = run_mixed(w, out_dtype="f32")
    assert np.max(np.abs(got[0] - got[64])) <= 5e-3


def test_single_token_prefill_is_its_value():
    _announce("prefill of one token from scratch")
    w = _mixed([], [(0, 1), (0, 1)], seed=6)
    got = run_mixed(w, out_dtype="f32")
    ref = oracle.paged_attention_workload(w)
    np.testing.assert_array_equal(got, ref)


def test_prefill_constant_v_exact():
    _announce("prefill constant V")
    w = _mixed([9], [(0, 70), (130, 64)], seed=7)
    w.v_pool[...] = np.uint16(0x4000)
    pa_inputs.poison_pool(w)
    got = run_mixed(w, out_dtype="f32")
    np.testing.assert_array_equal(got, 2.0)


def test_prefill_split_matches_unsplit():
    """Few units: long units are cut into kv pieces and merged.  The same rows with a
    max_q_len bound large enough to fill the chip run unsplit; both match the oracle and
    each other (only the order of the sums differs)."""
    _announce("prefill pieces vs one pass")
    w = _mixed([], [(3000, 64), (0, 200), (1500, 33), (40, 1)], seed=41)
    ref = oracle.paged_attention_workload(w)
    got_split = run_mixed(w, out_dtype="f32")
    compare(got_split, ref, 1e-2, what="prefill in pieces")
    import torch
    from paged_kv_attention_13_amd import binding
    from paged_kv_attention_13_amd.device import to_device
    d = to_device(w)
    out = binding.mixed(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], d["q_start_loc"],
                        w.scale, num_decode_rows=0, max_q_len=w.max_seq_len, max_seq_len=w.max_seq_len,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    got_one = out.cpu().numpy().astype(np.float64)
    compare(got_one, ref, 1e-2, what="prefill in one pass")
    assert np.max(np.abs(got_one - got_split)) <= 2e-3


@pytest.mark.parametrize("bs", [32, 128])
@pytest.mark.parametrize("dec", [[], [77]])
def test_prefill_pieces_start_mid_page(bs, dec):
    """Pieces of 64-token tiles over 128-token pages start in the middle of a page, with the
    prefill rows alone and beside a decode row."""
    _announce(f"prefill pieces, bs={bs}, decode rows {dec}")
    w = _mixed(dec, [(5000, 40), (700, 300)], bs=bs, seed=47 + bs)
    ref = oracle.paged_attention_workload(w)
    got = run_mixed(w, out_dtype="f32")
    compare(got, ref, 1e-2, what=f"prefill pieces bs{bs}")


@pytest.mark.parametrize("bs", [16, 64])
def test_prefill_both_workgroup_shapes(bs):
    """Prefill rows alone run in the 8-wave shape (128-token kv tiles as two 64-token sub-tiles;
    here 4 x 8 units, cut into pieces, and 8 x 8 x 8 units of eight 512-token chunks, uncut); beside
    a decode row the same rows run in the 4-wave shape.  All against the oracle."""
    _announce(f"prefill workgroup shapes, bs={bs}")
    pre = [(3000, 40), (700, 64), (1500, 17), (90, 3)]
    for dec in ([], [500]):
        w = _mixed(dec, pre, bs=bs, seed=61 + bs)
        compare(run_mixed(w, out_dtype="f32"), oracle.paged_attention_workload(w), 1e-2,
                what=f"shape test, decode rows {dec}")
    w = _mixed([], [(37 * i, 512) for i in range(8)], bs=bs, seed=67 + bs)     # 8 x 8 x 8 = 512 units
    compare(run_mixed(w, out_dtype="f32"), oracle.paged_attention_workload(w), 1e-2, what="8 chunks of 512")
    # group 8: two head blocks per kv head, 8 x 8 x 2 x 8 = 1,024 units of the 8-wave shape
    w = _mixed([], [(37 * i, 512) for i in range(8)], bs=bs, hq=64, seed=71 + bs)
    compare(run_mixed(w, out_dtype="f32"), oracle.paged_attention_workload(w), 1e-2, what="group 8, 8 x 512")


@pytest.mark.parametrize("bs", [16, 64])
def test_fp8_kv_prefill_rows(bs):
    """FP8-E4M3 pools (NaN codes in every unused slot): prefill-chunk rows beside decode rows
    (4-wave shape), alone and cut into kv pieces, and alone with 512 uncut units (8-wave shape),
    against the oracle fed the dequantised values."""
    _announce(f"fp8 kv prefill rows, bs={bs}")
    for dec in ([1, 300, 3000], []):
        w = _mixed(dec, PRE, bs=bs, seed=81 + bs, kv_fmt="fp8")
        compare(run_mixed(w, out_dtype="f32"), oracle.paged_attention_workload(w), TOL_FP8,
                what=f"fp8 prefill, decode rows {dec}")
    w = _mixed([], [(37 * i, 512) for i in range(8)], bs=bs, seed=83 + bs, kv_fmt="fp8")
    compare(run_mixed(w, out_dtype="f32"), oracle.paged_attention_workload(w), TOL_FP8, what="fp8 8 chunks of 512")


def test_prefill_many_units_unsplit():
    """More units than resident workgroups: no kv split, longest query tiles first."""
    _announce("prefill, 3 rows x 1024 new tokens")
    w = _mixed([7], [(500, 1024), (0, 1024), (2000, 1000)], seed=43)
    got = run_mixed(w)
    rows = [0, 1, 2, 3]
    ref = oracle.paged_attention_workload(w, rows=rows)
    compare(got, ref, TOL_BF16, what="3 x 1024 prefill")


def test_mixed_full_size_workload():
    _announce(f"workload 5: {pa_inputs.WORKLOAD_NAMES[5]}")
    w = pa_inputs.make_config(5)
    got = run_mixed(w)
    ref = oracle.paged_attention_workload(w)
    compare(got, ref, TOL_BF16, what=f"workload 5, all {w.num_seqs} rows ({w.total_q} queries)")
    for b in range(w.num_seqs):
        a, e = w.q_start_loc[b], w.q_start_loc[b + 1]
        rel = np.linalg.norm(got[a:e] - ref[a:e]) / np.linalg.norm(ref[a:e])
        assert rel <= TOL_REL_L2, (b, rel)


def test_mixed_graph_replays_match_eager():
    """A mixed call (decode rows + prefill rows, which fork onto an auxiliary stream and join
    back) recorded into a graph: every replay equals the eager call, with eager work and a
    synchronisation between replays."""
    _announce("mixed call in a graph")
    import torch
    from paged_kv_attention_13_amd import binding
    from paged_kv_attention_13_amd.device import to_device
    w = _mixed([100, 2000, 5], [(0, 64), (300, 100)], seed=31)
    d = to_device(w)
    pre_q = w.q_lens[w.num_decode_rows:]
    out_e = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    out_g = torch.empty_like(out_e)
    kw = dict(num_decode_rows=w.num_decode_rows, max_q_len=int(pre_q.max()), max_seq_len=w.max_seq_len)
    me = binding.make_mixed_args(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"],
                                 d["q_start_loc"], w.scale, out=out_e, **kw)
    mg = binding.make_mixed_args(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"],
                                 d["q_start_loc"], w.scale, out=out_g, **kw)
    ws_e = torch.zeros(binding.mixed_workspace_bytes(me), dtype=torch.uint8, device="cuda")
    ws_g = torch.zeros_like(ws_e)
    me.base.workspace, me.base.workspace_bytes = ws_e.data_ptr(), ws_e.numel()
    mg.base.workspace, mg.base.workspace_bytes = ws_g.data_ptr(), ws_g.numel()
    binding.mixed_args_call(me)
    torch.cuda.synchronize()
    ref = oracle.paged_attention_workload(w)
    compare(out_e.cpu().numpy().astype(np.float64), ref, 5e-3, what="eager mixed")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        binding.mixed_args_call(mg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.mixed_args_call(mg)
    for rep in range(3):
        out_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        binding.mixed_args_call(me)                      # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), rep


def test_prefill_after_a_100k_prefix():
    """64 new tokens after 100,000 cached ones in 16-token blocks: each kv piece spans more
    block-table entries than the kernel stages in LDS, so its loads read the table itself."""
    _announce("prefill after a 100k prefix")
    w = _mixed([], [(100000, 64), (3, 5)], seed=91)
    ref = oracle.paged_attention_workload(w)
    got = run_mixed(w, out_dtype="f32")
    compare(got, ref, 1e-2, what="prefill after 100k")


def test_rows_permuted_within_each_class():
    """Outputs do not depend on the order of rows within each class: decode rows (split path
    and one workgroup per unit) and prefill rows, permuted, give the permuted outputs."""
    _announce("rows permuted within classes")
    dec = [1, 40, 700, 3000, 129]
    pre = [(0, 64), (300, 100), (17, 33)]
    w = _mixed(dec, pre, seed=95)
    rng = np.random.default_rng(95)
    pd, pp = rng.permutation(len(dec)), rng.permutation(len(pre))
    w2 = _mixed([dec[i] for i in pd], [pre[i] for i in pp], seed=95)
    # same cache and queries per row, in the new order
    order = list(pd) + [len(dec) + i for i in pp]
    w2.k_pool, w2.v_pool = w.k_pool, w.v_pool
    w2.block_table = w.block_table[order].copy()
    qs = np.concatenate([np.arange(w.q_start_loc[b], w.q_start_loc[b + 1]) for b in order])
    w2.q = w.q[qs].copy()
    a = run_mixed(w, out_dtype="f32")
    b = run_mixed(w2, out_dtype="f32")
    ref = oracle.paged_attention_workload(w)
    compare(a, ref, 1e-2, what="original order")
    # decode rows on the balanced split may cut their units at other places: within the
    # split-invariance bound; every other row is computed alike in either order
    nd = len(dec)
    assert np.max(np.abs(b - a[qs])) <= 8e-3
    np.testing.assert_array_equal(b[nd:], a[qs][nd:])

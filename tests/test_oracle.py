"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: a contiguous
(unpaged) brute force, torch's fp64 scaled-dot-product attention, closed
forms, invariances, the outcomeschool toy pool, and the FP8 E4M3 format.  The
planted-mistake tests at the end check that these pins really catch the
plausible errors (wrong slot, wrong head group, dropped scale, off-by-one
causal diagonal).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as pa_mod
from pa_inputs import make_workload, random_block_table
import pa_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers (test side): contiguous data -> paged pool
# --------------------------------------------------------------------------

def paged_from_contiguous(rng, kc_rows, vc_rows, bs, extra_blocks=3):
    """kc_rows[b]: float32 [L_b, Hkv, D].  Returns (k_pool, v_pool, table)."""
    Ls = np.array([k.shape[0] for k in kc_rows], dtype=np.int32)
    hkv, d = kc_rows[0].shape[1:]
    need = int(((Ls + bs - 1) // bs).sum())
    nb = need + extra_blocks
    table = random_block_table(rng, Ls, bs, nb)
    kp = np.full((nb, hkv, bs, d), np.nan, dtype=np.float32)
    vp = np.full((nb, hkv, bs, d), np.nan, dtype=np.float32)
    for b, (kc, vc) in enumerate(zip(kc_rows, vc_rows)):
        for t in range(kc.shape[0]):
            kp[table[b, t // bs], :, t % bs, :] = kc[t]
            vp[table[b, t // bs], :, t % bs, :] = vc[t]
    return kp, vp, table


def brute_force(q, kc, vc, scale, hq, hkv, first_pos):
    """Triple-loop softmax attention on contiguous K/V (pure Python floats)."""
    n, _, d = q.shape
    L = kc.shape[0]
    group = hq // hkv
    out = np.zeros((n, hq, d))
    for i in range(n):
        for h in range(hq):
            g = h // group
            vis = first_pos + i + 1
            s = [scale * sum(float(q[i, h, e]) * float(kc[t, g, e]) for e in range(d))
                 for t in range(vis)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            for e in range(d):
                out[i, h, e] = sum(w[t] * float(vc[t, g, e]) for t in range(vis)) / z
    return out


def run_oracle(q, kp, vp, table, Ls, bs, hq, hkv, scale, q_lens, fmt="f32"):
    return oracle.paged_attention(q, "f32", kp, vp, fmt, table, Ls, bs, hq, hkv, scale, q_lens)


# --------------------------------------------------------------------------
# brute force, exhaustive over tiny shapes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bs", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 1), (4, 2), (8, 2)])
@pytest.mark.parametrize("d", [1, 4, 8])
def test_brute_force_sweep(bs, hq, hkv, d):
    rng = np.random.default_rng(bs * 1000 + hq * 100 + hkv * 10 + d)
    Ls = list(range(1, 3 * bs + 2)) if bs <= 4 else [1, 2, 15, 16, 17, 33, 49]
    for L in Ls:
        for n in sorted({1, 2, L} & set(range(1, L + 1))):
            kc = rng.standard_normal((L, hkv, d)).astype(np.float32)
            vc = rng.standard_normal((L, hkv, d)).astype(np.float32)
            q = rng.standard_normal((n, hq, d)).astype(np.float32)
            kp, vp, table = paged_from_contiguous(rng, [kc], [vc], bs)
            scale = 1.0 / math.sqrt(d)
            got = run_oracle(q, kp, vp, table, np.array([L]), bs, hq, hkv, scale, np.array([n]))
            ref = brute_force(q, kc, vc, scale, hq, hkv, L - n)
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_brute_force_batch_of_rows():
    """Several rows with mixed q_len packed in one call, each against its own brute force."""
    rng = np.random.default_rng(5)
    hq, hkv, d, bs = 4, 2, 4, 3
    Ls = [7, 1, 12, 5]
    qls = [1, 1, 4, 5]
    kcs = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in Ls]
    vcs = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in Ls]
    q = rng.standard_normal((sum(qls), hq, d)).astype(np.float32)
    kp, vp, table = paged_from_contiguous(rng, kcs, vcs, bs)
    got = run_oracle(q, kp, vp, table, np.array(Ls), bs, hq, hkv, 0.37, np.array(qls))
    a = 0
    for b, (L, n) in enumerate(zip(Ls, qls)):
        ref = brute_force(q[a:a + n], kcs[b], vcs[b], 0.37, hq, hkv, L - n)
        np.testing.assert_allclose(got[a:a + n], ref, rtol=0, atol=1e-12)
        a += n


# --------------------------------------------------------------------------
# library special cases: torch fp64 scaled_dot_product_attention
# --------------------------------------------------------------------------

def _sdpa(q, kc, vc, scale, first_pos):
    """torch SDPA, fp64 CPU, GQA by torch's own head expansion, lower-right causal mask."""
    import torch.nn.functional as F
    from torch.nn.attention.bias import causal_lower_right
    n, hq, d = q.shape
    L, hkv, _ = kc.shape
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]      # [1, Hq, n, D]
    kt = torch.from_numpy(kc.astype(np.float64)).permute(1, 0, 2)[None]     # [1, Hkv, L, D]
    vt = torch.from_numpy(vc.astype(np.float64)).permute(1, 0, 2)[None]
    assert first_pos == L - n
    mask = causal_lower_right(n, L) if n > 1 else None
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                       enable_gqa=(hq != hkv))
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv", [(4, 4), (32, 8), (8, 1)])
@pytest.mark.parametrize("L,n", [(1, 1), (37, 1), (200, 1), (64, 64), (90, 17), (300, 256)])
def test_against_torch_sdpa(hq, hkv, L, n):
    rng = np.random.default_rng(L * 7 + n + hq)
    d, bs = 32, 16
    kc = rng.standard_normal((L, hkv, d)).astype(np.float32)
    vc = rng.standard_normal((L, hkv, d)).astype(np.float32)
    q = rng.standard_normal((n, hq, d)).astype(np.float32)
    kp, vp, table = paged_from_contiguous(rng, [kc], [vc], bs)
    scale = 1.0 / math.sqrt(d)
    got = run_oracle(q, kp, vp, table, np.array([L]), bs, hq, hkv, scale, np.array([n]))
    ref = _sdpa(q, kc, vc, scale, L - n)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# closed forms and invariants on the named shapes
# --------------------------------------------------------------------------

def _w(seed=1, L=(37, 16, 1, 100), bs=16, kv_fmt="bf16", q_fmt="bf16", q_lens=None):
    return make_workload(name="t", seq_lens=list(L), q_lens=q_lens, num_q_heads=8,
                         num_kv_heads=2, head_dim=16, block_size=bs, q_fmt=q_fmt,
                         kv_fmt=kv_fmt, seed=seed, extra_blocks=2, poison_unused=True)


def test_constant_v_returns_constant():
    w = _w()
    c = np.uint16(0x4040)               # bf16 3.0
    w.v_pool[...] = c
    out = oracle.paged_attention_workload(w)
    np.testing.assert_allclose(out, 3.0, rtol=0, atol=1e-13)


def test_single_token_returns_its_v():
    w = _w(L=(1, 1, 1))
    out = oracle.paged_attention_workload(w)
    for b in range(3):
        for h in range(8):
            g = h // 4
            v = oracle.stored_to_f64(w.v_pool[w.block_table[b, 0], g, 0], "bf16")
            np.testing.assert_array_equal(out[b, h], v)


def test_zero_query_gives_mean_of_values():
    w = _w()
    w.q[...] = 0
    out = oracle.paged_attention_workload(w)
    for b, L in enumerate(w.seq_lens):
        for h in range(8):
            V = np.stack([oracle.stored_to_f64(
                w.v_pool[w.block_table[b, t // w.block_size], h // 4, t % w.block_size], "bf16")
                for t in range(L)])
            np.testing.assert_allclose(out[b, h], V.mean(axis=0), rtol=0, atol=1e-13)


def test_one_hot_probe_picks_one_token():
    """Key t* scores far above the rest: the output is exactly V[t*]."""
    w = _w(L=(50,), bs=4)
    w.k_pool[...] = 0
    w.q[...] = 0
    w.q[0, :, 0] = np.uint16(0x3F80)    # q = e0 for every head (bf16 1.0)
    for tstar in [0, 3, 4, 25, 49]:
        w.k_pool[...] = 0
        w.k_pool[w.block_table[0, tstar // 4], :, tstar % 4, 0] = np.uint16(0x4480)  # 1024
        out = oracle.paged_attention_workload(w)
        for h in range(8):
            v = oracle.stored_to_f64(w.v_pool[w.block_table[0, tstar // 4], h // 4, tstar % 4], "bf16")
            np.testing.assert_array_equal(out[0, h], v)


def test_key_shift_invariance_with_large_logits():
    """Adding one vector u to every key shifts all scores of a query equally."""
    rng = np.random.default_rng(11)
    hq, hkv, d, bs, L = 4, 2, 8, 4, 23
    kc = rng.standard_normal((L, hkv, d))
    vc = rng.standard_normal((L, hkv, d)).astype(np.float32)
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    u = 300.0 * rng.standard_normal(d)
    kp, vp, table = paged_from_contiguous(rng, [kc.astype(np.float32)], [vc], bs)
    kp2 = np.full_like(kp, np.nan)        # same table, shifted keys
    for t in range(L):
        kp2[table[0, t // bs], :, t % bs] = (kc[t] + u).astype(np.float32)
    a = run_oracle(q, kp, vp, table, np.array([L]), bs, hq, hkv, 0.5, np.array([1]))
    b = run_oracle(q, kp2, vp, table, np.array([L]), bs, hq, hkv, 0.5, np.array([1]))
    assert np.all(np.isfinite(b))
    # fp32 rounding of k+u perturbs scores by ~|q||u|*2^-24: loose bound
    np.testing.assert_allclose(a, b, rtol=0, atol=5e-3)


def test_block_permutation_bit_identical():
    w = _w(L=(37, 16, 1, 100, 64))
    ref = oracle.paged_attention_workload(w)
    rng = np.random.default_rng(8)
    perm = rng.permutation(w.num_blocks)           # new id of old block i is perm[i]
    inv = np.argsort(perm)
    w.k_pool = w.k_pool[inv]
    w.v_pool = w.v_pool[inv]
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    got = oracle.paged_attention_workload(w)
    np.testing.assert_array_equal(got, ref)


def test_decode_row_equals_last_query_of_prefill_row():
    """A decode row of length L equals the last query of a prefill row of length L."""
    w = _w(L=(40, 40), q_lens=[7, 1])
    # make row 1 share row 0's blocks and its q equal row 0's last query
    w.block_table[1] = w.block_table[0]
    w.q[7] = w.q[6]
    out = oracle.paged_attention_workload(w)
    # same mathematics; BLAS may sum in another order for a different q count
    np.testing.assert_allclose(out[7], out[6], rtol=0, atol=1e-14)


def test_two_chunks_equal_one_chunk():
    """Queries of chunk [a, a+m) then [a+m, a+m+k) equal one chunk of m+k queries."""
    w = _w(L=(60, 53, 60), q_lens=[13, 6, 7])
    w.block_table[1] = w.block_table[0]
    w.block_table[2] = w.block_table[0]
    w.q[13:19] = w.q[0:6]
    w.q[19:26] = w.q[6:13]
    out = oracle.paged_attention_workload(w)
    np.testing.assert_allclose(out[13:19], out[0:6], rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[19:26], out[6:13], rtol=0, atol=1e-14)


def test_poisoned_slots_never_read():
    w = _w(L=(37, 16, 1, 100))
    out = oracle.paged_attention_workload(w)
    assert np.all(np.isfinite(out))


def test_toy_pool_from_figure():
    with open(os.path.join(GOLDEN, "toy_pool.json")) as f:
        g = json.load(f)
    fx = g["fixture"]
    nb, bs = fx["num_blocks"], fx["block_size"]
    hq = hkv = 1
    d = 2
    kp = np.full((nb, hkv, bs, d), np.nan, dtype=np.float32)
    vp = np.full((nb, hkv, bs, d), np.nan, dtype=np.float32)
    table = np.array(fx["block_table"], dtype=np.int32)
    Ls = np.array(fx["seq_lens"], dtype=np.int32)
    rng = np.random.default_rng(0)
    for b, L in enumerate(Ls):
        for t in range(L):
            blk = table[b, t // bs]
            kp[blk, 0, t % bs] = rng.standard_normal(d)
            vp[blk, 0, t % bs] = blk
    q = np.zeros((3, 1, d), dtype=np.float32)
    out = oracle.paged_attention(q, "f32", kp, vp, "f32", table, Ls, bs, hq, hkv, 0.7)
    exp = g["expected_by_hand"]
    for b, key in enumerate(["A", "B", "C"]):
        np.testing.assert_allclose(out[b, 0], exp[key], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# FP8 E4M3 table
# --------------------------------------------------------------------------

def test_e4m3_table_matches_torch_float8_e4m3fn():
    table = oracle.e4m3_decode_table()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(table), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(table[ok], ref[ok])


def test_e4m3_special_codes():
    t = oracle.e4m3_decode_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9
    assert t[0x08] == 2.0 ** -6           # smallest normal
    assert t[0x07] == 7 * 2.0 ** -9       # largest subnormal
    assert t[0x38] == 1.0
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and math.copysign(1, t[0x80]) < 0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    finite = t[~np.isnan(t)]
    assert finite.max() == 448.0 and len(np.unique(finite)) == 253   # +0/-0 compare equal


def test_fp8_path_uses_scaled_dequant():
    """FP8 rows equal float32 rows holding code value * scale (power-of-two scales: exact)."""
    w = _w(kv_fmt="fp8")
    w.k_scale = np.array([2.0 ** -6, 2.0 ** -3], dtype=np.float32)
    w.v_scale = np.array([2.0 ** -5, 4.0], dtype=np.float32)
    out = oracle.paged_attention_workload(w)
    kf = oracle.e4m3_decode(w.k_pool) * w.k_scale[None, :, None, None]
    vf = oracle.e4m3_decode(w.v_pool) * w.v_scale[None, :, None, None]
    fin = np.isfinite(kf)
    assert np.all(kf[fin] == kf[fin].astype(np.float32))
    ref = oracle.paged_attention(w.q, "bf16", kf.astype(np.float32), vf.astype(np.float32), "f32",
                                 w.block_table, w.seq_lens, w.block_size, 8, 2, w.scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)


def test_bf16_storage_decode():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F80], dtype=np.uint16)
    v = oracle.stored_to_f64(bits, "bf16")
    assert v[0] == 1.0 and v[1] == -1.0
    assert v[2] == 3.140625
    assert v[3] == 2.0 ** -133
    assert v[4] == np.inf


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin above
# --------------------------------------------------------------------------

def _sdpa_pin_passes(monkeypatch_target=None):
    try:
        test_against_torch_sdpa(32, 8, 90, 17)
        test_against_torch_sdpa(4, 4, 37, 1)
        return True
    except AssertionError:
        return False


def _brute_pin_passes():
    try:
        test_brute_force_sweep(3, 4, 2, 4)
        return True
    except AssertionError:
        return False


def test_planted_wrong_slot_is_caught(monkeypatch):
    orig = pa_mod.gather_kv

    def bad(pool, fmt, row, L, g, bs, hs=None):
        t = np.arange(L)
        phys = np.asarray(row)[t // bs]
        slot = (t + 1) % bs                       # off-by-one slot
        v = pa_mod.stored_to_f64(pool[phys, g, slot, :], fmt)
        return v if hs is None else v * hs
    monkeypatch.setattr(pa_mod, "gather_kv", bad)
    assert not _brute_pin_passes()
    monkeypatch.setattr(pa_mod, "gather_kv", orig)
    assert _brute_pin_passes()


def test_planted_wrong_head_group_is_caught(monkeypatch):
    orig = pa_mod._row

    def bad(q_rows, q_fmt, k_pool, v_pool, kv_fmt, table_row, L, bs, Hq, Hkv, scale, ks, vs):
        # interleaved mapping g = h % Hkv instead of consecutive groups
        qf = pa_mod.stored_to_f64(q_rows, q_fmt)
        out = np.empty(qf.shape)
        for h in range(Hq):
            g = h % Hkv
            K = pa_mod.gather_kv(k_pool, kv_fmt, table_row, L, g, bs)
            V = pa_mod.gather_kv(v_pool, kv_fmt, table_row, L, g, bs)
            out[:, h, :] = pa_mod.attend_rows(qf[:, h, :], K, V, scale, L - q_rows.shape[0])
        return out
    monkeypatch.setattr(pa_mod, "_row", bad)
    assert not _sdpa_pin_passes()
    monkeypatch.setattr(pa_mod, "_row", orig)
    assert _sdpa_pin_passes()


@pytest.mark.parametrize("mistake", ["no_scale", "exclusive_diagonal", "no_max_shift_sign"])
def test_planted_attend_mistakes_are_caught(monkeypatch, mistake):
    orig = pa_mod.attend_rows

    def bad(q, K, V, scale, first_pos):
        n, L = q.shape[0], K.shape[0]
        s = q @ K.T * (1.0 if mistake == "no_scale" else scale)
        pos = first_pos + np.arange(n)[:, None]
        vis = (np.arange(L)[None, :] < pos) if mistake == "exclusive_diagonal" else \
            (np.arange(L)[None, :] <= pos)
        vis[:, 0] = True
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.where(vis, np.exp((m - s) if mistake == "no_max_shift_sign" else (s - m)), 0.0)
        return (e / e.sum(axis=1, keepdims=True)) @ V
    monkeypatch.setattr(pa_mod, "attend_rows", bad)
    assert not _sdpa_pin_passes()
    monkeypatch.setattr(pa_mod, "attend_rows", orig)
    assert _sdpa_pin_passes()


# ----------------------------------------------------------------------------
# shared prefixes: rows whose tables alias the same physical prefix blocks
# ----------------------------------------------------------------------------

def test_aliased_prefix_equals_private_copies():
    """Rows pointing at shared prefix blocks get exactly what they get from private copies.

    Prefix reuse ("How does TensorRT-LLM work", section "The paged KV cache")
    stores an identical beginning once; attention must not notice.  The copy
    gives every row its own blocks with the same contents, relabelled in the
    table.
    """
    w = pa_inputs.make_shared_prefix_workload(name="alias", group_sizes=[3, 2, 1], shared_lens=[32, 48, 16],
                                              own_lens=[1, 20, 5, 33, 2, 9], prefix_ids=[0, 0, 1],
                                              num_q_heads=4, num_kv_heads=2, head_dim=8, seed=4)
    ref = oracle.paged_attention_workload(w)
    bs = w.block_size
    used = [(r, j) for r in range(w.num_seqs) for j in range((int(w.seq_lens[r]) + bs - 1) // bs)]
    kp = np.concatenate([w.k_pool[w.block_table[r, j]][None] for r, j in used])
    vp = np.concatenate([w.v_pool[w.block_table[r, j]][None] for r, j in used])
    table = np.full_like(w.block_table, -1)
    for i, (r, j) in enumerate(used):
        table[r, j] = i
    assert len(set(table[table >= 0].tolist())) == len(used)           # now nothing is shared
    got = oracle.paged_attention(w.q, w.q_fmt, kp, vp, w.kv_fmt, table, w.seq_lens, bs, w.num_q_heads,
                                 w.num_kv_heads, w.scale, w.q_lens)
    np.testing.assert_array_equal(got, ref)


def test_split_at_shared_boundary_merges_exactly():
    """Attention over [prefix | own part] equals the log-sum-exp merge of the two parts.

    This is the identity a shared-prefix call relies on (the split-context merge
    named Flash-Decoding, "Introduction to TensorRT-LLM", section "Core
    Optimization Technologies"): with s_j = scale q.k_j over part j,
    m_j = max s_j, l_j = sum exp(s_j - m_j), a_j = sum exp(s_j - m_j) v_j,
    o = sum_j exp(m_j - M) a_j / sum_j exp(m_j - M) l_j.  Checked in fp64 against
    the oracle for every split point.
    """
    rng = np.random.default_rng(3)
    L, D = 40, 8
    q = rng.standard_normal(D)
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    full = oracle.attend_rows(q[None], K, V, 0.3, L - 1)[0]
    for P in range(1, L):
        parts = []
        for lo, hi in ((0, P), (P, L)):
            s = 0.3 * K[lo:hi] @ q
            m = s.max()
            e = np.exp(s - m)
            parts.append((m, e.sum(), e @ V[lo:hi]))
        M = max(p[0] for p in parts)
        o = sum(np.exp(m - M) * a for m, _, a in parts) / sum(np.exp(m - M) * l for m, l, _ in parts)
        np.testing.assert_allclose(o, full, rtol=1e-13, atol=1e-14)

"""GPU tests of the scheduled decode loop: pa_append + pa_mixed per layer, eager and as a HIP graph.

The oracle side keeps host copies of every layer's pools, written with the
oracle's own scatter (oracle.append_kv) through the same slot mapping, and
computes each step's attention with the fp64 oracle.
"""
import numpy as np
import pytest

import oracle
import pa_inputs
from gpu_util import TOL_BF16, compare

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _vec(*key, shape):
    """Seeded N(0,1) values for one (request or token, position, layer, kind) key."""
    return np.random.default_rng(list(key)).standard_normal(shape).astype(np.float32)


def _values(Hq, Hkv, D):
    def fn(rid, tok, pos, layer, kind):
        if kind == "q":
            return _vec(1, rid, pos, layer, shape=(Hq, D))
        # a token's K/V depend on the token and its position: equal prefixes, equal values
        return _vec(2 if kind == "k" else 3, tok, pos, layer, shape=(Hkv, D))
    return fn


def _bits(t):
    import torch
    return t.float().cpu().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_scheduled_loop_matches_oracle():
    """Chunked prefill, prefix reuse and decode over several steps; every output and the pools."""
    _announce("scheduled loop vs oracle")
    import torch
    from paged_kv_attention_13_amd.loop import DecodeLoop, fill_inputs
    Hq, Hkv, D, bs, L = 8, 2, 128, 16, 2
    loop = DecodeLoop(num_layers=L, num_blocks=48, block_size=bs, max_blocks_per_seq=12, max_batch_size=4,
                      max_num_tokens=48, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, prefix_reuse=True)
    vf = _values(Hq, Hkv, D)
    rng = np.random.default_rng(0)
    system = rng.integers(0, 500, size=40)
    prompts = {r: np.concatenate([system, rng.integers(0, 500, size=n)]) for r, n in enumerate([5, 60, 17, 33])}
    arrivals = {0: [0, 1], 3: [2, 3]}
    rep_k = [np.zeros((48, Hkv, bs, D), np.uint16) for _ in range(L)]
    rep_v = [np.zeros((48, Hkv, bs, D), np.uint16) for _ in range(L)]
    for step in range(40):
        for r in arrivals.get(step, []):
            loop.kvm.add_request(r, prompts[r], 6)
        b = loop.schedule()
        if b.num_rows == 0:
            loop.complete([])
            continue
        fill_inputs(loop, b, vf)
        loop.run_batch(b)
        torch.cuda.synchronize()
        T = b.total_q
        for layer in range(L):
            kn, vn = _bits(loop.k_new[layer][:T]), _bits(loop.v_new[layer][:T])
            rep_k[layer], rep_v[layer] = oracle.append_kv(rep_k[layer], rep_v[layer], kn, vn, b.slot_mapping, bs)
            ref = oracle.paged_attention(_bits(loop.q[layer][:T]), "bf16", rep_k[layer], rep_v[layer], "bf16",
                                         b.block_table, b.seq_lens, bs, Hq, Hkv, loop.scale, b.q_lens)
            got = loop.out[layer][:T].float().cpu().numpy().astype(np.float64)
            compare(got, ref, TOL_BF16, what=f"step {step} layer {layer} rows {list(b.request_ids)}")
        loop.complete([(int(r) * 31 + step) % 500 for r in b.request_ids])
    assert all(loop.kvm.info(r)["state"] == "finished" for r in prompts)
    # the two later requests reused the system prompt's two whole blocks
    assert loop.kvm.info(2)["num_reused"] == 2 * bs and loop.kvm.info(3)["num_reused"] == 2 * bs
    for layer in range(L):
        np.testing.assert_array_equal(_bits(loop.k_pools[layer]), rep_k[layer])
        np.testing.assert_array_equal(_bits(loop.v_pools[layer]), rep_v[layer])


def test_graph_replay_matches_eager():
    """A steady decode step recorded once and replayed equals the same step launched eagerly.

    Two loops run the same requests; loop A launches every step, loop B replays
    its graph, with A's eager work and a synchronisation between B's replays.
    Every step's outputs must be bit-identical.
    """
    _announce("graph replay vs eager")
    import torch
    from paged_kv_attention_13_amd.loop import DecodeLoop, fill_inputs
    Hq, Hkv, D, bs, L = 8, 2, 128, 16, 3
    kw = dict(num_layers=L, num_blocks=64, block_size=bs, max_blocks_per_seq=16, max_batch_size=3,
              max_num_tokens=512, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, prefix_reuse=False)
    A, B = DecodeLoop(**kw), DecodeLoop(**kw)
    vf = _values(Hq, Hkv, D)
    for lp in (A, B):
        for r in range(3):
            lp.kvm.add_request(r, np.random.default_rng(r).integers(0, 500, size=100), 25)
    # prefill (one pass for all three), both loops the same way
    for lp in (A, B):
        b = lp.schedule()
        assert b.num_rows == 3 and b.num_decode_rows == 0
        fill_inputs(lp, b, vf)
        lp.run_batch(b)
        torch.cuda.synchronize()
        lp.complete([7, 8, 9])
    A.prepare_decode(3)
    B.prepare_decode(3)
    captured = False
    for step in range(20):
        sampled = [int(x) for x in np.random.default_rng(step).integers(0, 500, size=3)]
        outs = []
        for lp, graph in ((A, False), (B, True)):
            b = lp.schedule()
            assert b.num_rows == 3 and b.num_decode_rows == 3
            fill_inputs(lp, b, vf)
            lp.stage(b)
            if graph:
                if not captured:
                    lp.capture_decode_step()      # warm-up run + recording; replays below
                    captured = True
                lp.decode_step_graph()
            else:
                lp.decode_step_eager()
            torch.cuda.synchronize()
            outs.append([lp.out[layer][:3].clone() for layer in range(L)])
            lp.complete(sampled)
        for layer in range(L):
            assert torch.equal(outs[0][layer], outs[1][layer]), (step, layer)
        for lp in (A, B):
            assert [lp.kvm.info(r)["num_cached"] for r in range(3)] == [100 + step + 1] * 3
    for layer in range(L):
        assert torch.equal(A.k_pools[layer], B.k_pools[layer]) and torch.equal(A.v_pools[layer], B.v_pools[layer])

"""Helpers shared by the GPU tests: run the library on a workload, compare with the oracle."""
import numpy as np

TOL_BF16 = 2e-2        # max |gpu - oracle| on bf16 outputs
TOL_FP8 = 6e-2         # FP8-KV path, oracle fed the dequantised values
TOL_REL_L2 = 1e-2      # ||gpu - oracle||_2 / ||oracle||_2 (catches small systematic errors)
TOL_F32 = 1e-4         # fp32 path (fp32 in, fp32 out)


def run_decode(w, out_dtype=None, num_workers=0, dev=None):
    import torch
    from paged_kv_attention_13_amd import binding
    from paged_kv_attention_13_amd.device import to_device
    d = dev or to_device(w)
    odt = {None: None, "f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    out = binding.decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], w.scale,
                         max_seq_len=w.max_seq_len, k_scale=d["k_scale"], v_scale=d["v_scale"],
                         out_dtype=odt, num_workers=num_workers)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def run_mixed(w, out_dtype=None, num_workers=0, dev=None, num_verify_rows=0):
    """pa_mixed on a workload: rows [0, nd) decode, the next num_verify_rows verify rows, then prefill."""
    import torch
    from paged_kv_attention_13_amd import binding
    from paged_kv_attention_13_amd.device import to_device
    d = dev or to_device(w)
    odt = {None: None, "f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    nd, nv = w.num_decode_rows, num_verify_rows
    verify_q = w.q_lens[nd:nd + nv]
    prefill_q = w.q_lens[nd + nv:]
    out = binding.mixed(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"],
                        d["q_start_loc"], w.scale, num_decode_rows=nd,
                        max_q_len=int(prefill_q.max()) if len(prefill_q) else 1,
                        max_seq_len=w.max_seq_len, out_dtype=odt, num_workers=num_workers,
                        num_verify_rows=nv, max_verify_q_len=int(verify_q.max()) if nv else 0,
                        k_scale=d["k_scale"], v_scale=d["v_scale"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def compare(got, ref, tol, rel_tol=TOL_REL_L2, what=""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    print(f"[{what}] max_abs={mx:.3e} rel_l2={rel:.3e}", flush=True)
    assert mx <= tol, f"{what}: max abs err {mx:.3e} > {tol}"
    assert rel <= rel_tol, f"{what}: relative L2 err {rel:.3e} > {rel_tol}"
    return mx, rel


def run_cascade(w, out_dtype=None, num_workers=0, dev=None, max_group_rows=None):
    """pa_decode_cascade on a shared-prefix workload (``w.group_start``, ``w.shared_len``)."""
    import torch
    from paged_kv_attention_13_amd import binding
    from paged_kv_attention_13_amd.device import to_device
    d = dev or to_device(w)
    odt = {None: None, "f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    if max_group_rows is None:
        max_group_rows = int(np.diff(w.group_start).max())
    out = binding.decode_cascade(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"],
                                 d["group_start"], d["shared_len"], w.scale, max_seq_len=w.max_seq_len,
                                 max_group_rows=max_group_rows, out_dtype=odt, num_workers=num_workers)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)

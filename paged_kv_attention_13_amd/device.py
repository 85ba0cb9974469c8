"""Moving a ``pa_inputs.Workload`` into device tensors (torch as memory plumbing)."""
from __future__ import annotations

import numpy as np


def to_device(w, device="cuda"):
    """Return a dict of device tensors for workload ``w``; layouts as in include/pa.h."""
    import torch

    def dev(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dtype is not None:
            t = t.view(dtype)
        return t.to(device)

    fmt_dtype = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
    q = dev(w.q.view(np.int16) if w.q_fmt == "bf16" else w.q, fmt_dtype[w.q_fmt] if w.q_fmt == "bf16" else None)
    kv_view = (lambda a: a.view(np.int16)) if w.kv_fmt == "bf16" else (lambda a: a)
    kv_dt = fmt_dtype[w.kv_fmt] if w.kv_fmt == "bf16" else None
    out = {
        "q": q,
        "k_pool": dev(kv_view(w.k_pool), kv_dt),
        "v_pool": dev(kv_view(w.v_pool), kv_dt),
        "block_table": dev(w.block_table),
        "seq_lens": dev(w.seq_lens),
        "q_start_loc": dev(w.q_start_loc),
        "k_scale": dev(w.k_scale) if w.k_scale is not None else None,
        "v_scale": dev(w.v_scale) if w.v_scale is not None else None,
    }
    if getattr(w, "group_start", None) is not None:
        out["group_start"] = dev(w.group_start)
        out["shared_len"] = dev(w.shared_len)
    return out

#!/usr/bin/env python3
"""Benchmark of the paged-KV decode attention path on one MI355X.

One step = one call of the library on one batch of synthetic inputs already
resident in HBM: the split-K decode kernel followed by the log-sum-exp merge
(or, for the mixed workload, the prefill-chunk kernel plus both decode
kernels).  The default workload is the long-context decode batch: 55 rows at
8,192 cached tokens, Llama-3-8B GQA shapes (32 q heads, 8 KV heads, head_dim
128), bf16, 64-token blocks -- one layer of the 55-request example on the
"TensorRT-LLM, in depth" page (section "First principles: where the GPU
memory goes").

Prints ONE JSON line.  `value` is the decode-attention KV bandwidth: the
algorithmic KV bytes of one step divided by the measured step time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attention KV GB/s and % of HBM peak; tokens/s per layer at Llama-3-8B GQA"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0
EVENT_STRIDE = 5            # decode workloads: per-kernel HIP events on every 5th timed step


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5, 6],
                    help="named workload (3 = 55 x 8192 bf16 decode, the headline; 6 = the same "
                         "cache with 4 new tokens per row, speculative-decoding verify rows)")
    ap.add_argument("--num-workers", type=int, default=0,
                    help="decode work split into this many waves (0 = library default)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time budget of the oracle baseline sample (0 = skip)")
    ap.add_argument("--loop-batch", type=int, default=1,
                    help="--op loop: decode rows in the steady batch")
    ap.add_argument("--scrub-mib", type=int, default=None,
                    help="decode workloads: read this many MiB between timed steps (outside their events, "
                         "with cache-allocating loads) so no step reads KV left in the caches by the previous "
                         "one; the step time is then the median of the per-step events.  Default: 1024 when "
                         "the workload's KV bytes are under 1 GiB (they could otherwise stay in the 256 MB "
                         "Infinity Cache and the L2s between steps), else 0")
    ap.add_argument("--prewarm-ms", type=float, default=300.0,
                    help="before the warm-up steps, run steps back to back for this long so that the GPU's "
                         "clocks reach their sustained level (a short run otherwise times the clock ramp)")
    ap.add_argument("--skip-probes", action="store_true",
                    help="decode workloads: do not run the stream and gather bandwidth probes after the "
                         "timed steps (for profiler counter passes)")
    ap.add_argument("--prefill-case", default="w5-rows",
                    help="--op prefill: w5-rows, chunk256-after8192 or prompt8192")
    ap.add_argument("--op", default="decode",
                    choices=["decode", "append", "append-fp8", "cascade", "loop", "prefill", "stream"],
                    help="decode: the attention call of --workload (default); append / append-fp8: "
                         "writing the mixed workload's 2,144 new tokens (96 decode + 8 x 256 prefill) "
                         "into their cache slots, bf16 -> bf16 or bf16 -> FP8-E4M3; cascade: the "
                         "shared-prefix decode call on workload 7, with pa_decode on the same rows beside it; "
                         "loop: 32 layers of append + decode per step driven by the host scheduler, launched "
                         "eagerly and replayed as one HIP graph; stream: the streaming-read probe over as "
                         "many bytes as --workload's KV cache (the achievable read bandwidth)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the timed loop, run one device-to-device copy of this many MiB "
                         "(a plain copy kernel of known size, to calibrate HBM byte counters)")
    return ap.parse_args()


class GpuSampler:
    """Shader clock and board power of the GPU, sampled from sysfs in a thread while it runs.

    The card is the amdgpu sysfs device whose PCI slot matches torch's device 0; the current
    shader clock is the ``pp_dpm_sclk`` level marked ``*`` and the power is hwmon's
    ``power1_input`` (microwatts).  Only files are read: no process is started.
    """

    def __init__(self):
        import glob
        import torch
        self.sclk = self.power = None
        p = torch.cuda.get_device_properties(0)
        slot = f"{getattr(p, 'pci_domain_id', 0):04x}:{getattr(p, 'pci_bus_id', 0):02x}:" \
               f"{getattr(p, 'pci_device_id', 0):02x}.0"
        for card in sorted(glob.glob("/sys/class/drm/card*")):
            dev = os.path.join(card, "device")
            try:
                ok = f"PCI_SLOT_NAME={slot}" in open(os.path.join(dev, "uevent")).read()
            except OSError:
                continue
            if ok and os.path.exists(os.path.join(dev, "pp_dpm_sclk")):
                self.sclk = os.path.join(dev, "pp_dpm_sclk")
                pw = sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_input")) +
                            glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_average")))
                self.power = pw[0] if pw else None
                break
        self.samples = []
        self._stop = False
        self._thread = None

    def _read(self):
        import re
        mhz = w = None
        try:
            for line in open(self.sclk).read().splitlines():
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*Mhz", line, re.I)
                    mhz = int(m.group(1)) if m else None
            if self.power:
                w = int(open(self.power).read().strip()) / 1e6
        except (OSError, ValueError):
            pass
        return mhz, w

    def _run(self):
        while not self._stop:
            self.samples.append(self._read())
            time.sleep(0.0005)

    def start(self):
        import threading
        self.samples = []
        self._stop = False
        if self.sclk:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def stop(self, window: str):
        import numpy as np
        self._stop = True
        if self._thread:
            self._thread.join()
        if not self.samples:
            return None
        out = {"window": window, "samples": len(self.samples), "source": self.sclk}
        for key, i in (("sclk_mhz", 0), ("power_w", 1)):
            v = [x[i] for x in self.samples if x[i] is not None]
            if v:
                out[key] = {"min": round(float(np.min(v)), 1), "median": round(float(np.median(v)), 1),
                            "max": round(float(np.max(v)), 1)}
        return out


STREAM_SHAPES = tuple((g, u) for g in (1024, 2048, 4096) for u in (4, 8, 16))


def prewarm(call, ms: float) -> int:
    """Run ``call`` back to back for ``ms`` milliseconds (synchronising every 8 calls)."""
    import torch
    n = 0
    t_end = time.perf_counter() + ms / 1e3
    while time.perf_counter() < t_end:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
        n += 8
    return n


def stream_ceiling(nbytes: int, shapes=STREAM_SHAPES, reps: int = 10, prewarm_ms: float = 100.0):
    """Best streaming-read rate (GB/s) of ``pa_stream_read`` over ``nbytes`` bytes.

    For each launch shape (workgroups, loads in flight per lane), events bracket ``reps``
    back-to-back launches (one event pair per batch, so the pair's own cost is spread over
    the batch); the best shape's mean is kept.
    """
    import torch
    from paged_kv_attention_13_amd import binding
    n = (nbytes + 15) // 16 * 16
    buf = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(3)
    out = torch.empty(4 * max(g for g, _ in shapes), dtype=torch.int32, device="cuda")
    prewarm(lambda: binding.stream_read(buf, out, shapes[0][0], shapes[0][1]), prewarm_ms)
    res = {}
    for g, u in shapes:
        for _ in range(3):
            binding.stream_read(buf, out, g, u)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            binding.stream_read(buf, out, g, u)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[(g, u)] = n / (ms * 1e-3) / 1e9
    del buf, out
    best = max(res, key=res.get)
    return {"GBs": round(res[best], 1), "workgroups": best[0], "loads_in_flight": best[1], "bytes": n,
            "per_shape_GBs": {f"{g}x{u}": round(v, 1) for (g, u), v in res.items()},
            "load": "16-byte non-temporal loads, 256 lanes per workgroup, best launch shape"}


GATHER_SHAPES = tuple((g, f) for g in (256, 512, 1024, 2048) for f in (2, 4, 8))


def gather_ceiling(w, d, shapes=GATHER_SHAPES, reps: int = 10, prewarm_ms: float = 100.0):
    """Best rate (GB/s) of ``pa_gather_read`` over the pages a decode call of workload ``w``
    visits -- every (block, kv head) page of K and of V of every row, in the decode kernels'
    order (row, kv head, block) -- at the workload's own page size."""
    import numpy as np
    import torch
    from paged_kv_attention_13_amd import binding
    kp, vp = d["k_pool"], d["v_pool"]
    elem = kp.element_size()
    page = w.block_size * w.head_dim * elem
    base = min(kp.data_ptr(), vp.data_ptr())
    offs = []
    for b in range(w.num_seqs):
        nblk = (int(w.seq_lens[b]) + w.block_size - 1) // w.block_size
        phys = w.block_table[b, :nblk].astype(np.int64)
        for g in range(w.num_kv_heads):
            pg = (phys * w.num_kv_heads + g) * page
            kv = np.empty(2 * nblk, np.int64)
            kv[0::2] = kp.data_ptr() - base + pg
            kv[1::2] = vp.data_ptr() - base + pg
            offs.append(kv)
    offs = torch.from_numpy(np.concatenate(offs)).cuda()
    basev = kp if kp.data_ptr() == base else vp
    out = torch.empty(4 * max(g for g, _ in shapes), dtype=torch.int32, device="cuda")
    nbytes = offs.numel() * page
    prewarm(lambda: binding.gather_read(basev, offs, page, out, shapes[0][0], shapes[0][1]), prewarm_ms)
    res = {}
    for g, f in shapes:
        for _ in range(3):
            binding.gather_read(basev, offs, page, out, g, f)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            binding.gather_read(basev, offs, page, out, g, f)
        e1.record()
        torch.cuda.synchronize()
        res[(g, f)] = nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    best = max(res, key=res.get)
    return {"GBs": round(res[best], 1), "workgroups": best[0], "pages_in_flight": best[1], "page_bytes": page,
            "pages": int(offs.numel()), "bytes": int(nbytes),
            "per_shape_GBs": {f"{g}x{f}": round(v, 1) for (g, f), v in res.items()},
            "load": "whole (block, kv head) pages in decode order, 16-byte non-temporal loads, best launch shape"}


def bench_stream(args):
    """The streaming-read probe alone over the KV bytes of --workload."""
    import pa_inputs
    from paged_kv_attention_13_amd import accounting
    L, _ = pa_inputs.workload_lengths(args.workload)
    fmt = {1: "f32", 4: "fp8"}.get(args.workload, "bf16")
    nbytes = accounting.kv_bytes(L, 8, 128, fmt)
    sampler = GpuSampler().start()
    st = stream_ceiling(nbytes, reps=max(10, args.steps // 5), prewarm_ms=args.prewarm_ms)
    state = sampler.stop("the pre-warm and the timed launches")
    print(json.dumps({
        "metric": "streaming-read HBM GB/s (the decode kernels' load form, no compute)",
        "value": st["GBs"], "unit": "GB/s", "n_gpus": 1, "steps": max(10, args.steps // 5), "warmup": 3,
        "ms_per_step": round(st["bytes"] / (st["GBs"] * 1e9) * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic (constant bytes)",
        "config": {"workload": f"stream read of {st['bytes']} bytes (the KV bytes of workload {args.workload})",
                   "workgroups": st["workgroups"], "loads_in_flight": st["loads_in_flight"]},
        "stream_read": st,
        "roofline": {"bound": "hbm", "achieved": st["GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(st["GBs"] / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "stream_read_kernel",
                     "bytes_per_launch": st["bytes"]},
        "cpu_baseline": None,
        "gpu_state": state,
    }), flush=True)


def committed_traffic(kv_fmt: str, workload_name: str):
    """HBM bytes per launch of the decode kernel from the committed counter summary.

    Returns None unless the summary covers this workload and the kernel source is
    unchanged since the counters were taken (hash of decode.hip + pa_internal.h).
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode_bf16_55x8192_bs64.md")
    try:
        text = open(path).read()
        block = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    h = hashlib.sha256()
    for f in ("decode.hip", "pa_internal.h"):
        h.update(open(os.path.join(ROOT, "paged_kv_attention_13_amd", "csrc", f), "rb").read())
    if block.get("source_sha256_16") != h.hexdigest()[:16] or block.get("workload") != workload_name:
        return None
    return int(block["traffic_bytes_per_launch"])


def cpu_baseline(w, gpu_out, budget_s):
    """Time the fp64 oracle on whole rows of the same workload, one row at a time."""
    import numpy as np
    import oracle
    from paged_kv_attention_13_amd import accounting
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    rows = []
    errs = []
    t_total = 0.0
    order = np.random.default_rng(0).permutation(w.num_seqs)
    # rows in a seeded order, passing over the workload again while the time budget lasts
    # (the whole long-context workload takes the oracle under 2 s)
    i = 0
    while True:
        b = int(order[i % w.num_seqs])
        i += 1
        t0 = time.perf_counter()
        ref = oracle.paged_attention_row(w, b)
        t_total += time.perf_counter() - t0
        rows.append(b)
        if i <= w.num_seqs:
            a = int(w.q_start_loc[b])
            errs.append(float(np.abs(gpu_out[a:a + ref.shape[0]] - ref).max()))
        if t_total >= budget_s:
            break
    kv = accounting.kv_bytes(w.seq_lens[rows], w.num_kv_heads, w.head_dim, w.kv_fmt)
    tokens = int(w.seq_lens[rows].sum())
    passes, rest = divmod(len(rows), w.num_seqs)
    return {
        "value": kv / t_total / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(rows)} row evaluations ({passes} whole passes over the {w.num_seqs} rows + {rest} "
                  f"rows; {tokens} cached tokens, {kv} KV bytes) of the same workload, one row at a "
                  f"time, fp64 numpy; {t_total:.2f} s",
        "kv_tokens_per_s": tokens / t_total,
        "host_cpus": len(os.sched_getaffinity(0)),
        "max_abs_err_vs_gpu": max(errs),
    }


def bench_append(args):
    """Time pa_append on the mixed workload's step: each row's new tokens go to their slots."""
    import numpy as np
    import torch

    import pa_inputs
    from paged_kv_attention_13_amd import binding

    fp8 = args.op == "append-fp8"
    L, ql = pa_inputs.workload_lengths(5)
    w = pa_inputs.make_workload(name="append", seq_lens=L, q_lens=ql, block_size=16, seed=1005 + 7919,
                                kv_fmt="fp8" if fp8 else "bf16")
    bs = w.block_size
    slots = []
    for b in range(w.num_seqs):
        for pos in range(int(L[b] - ql[b]), int(L[b])):
            slots.append(int(w.block_table[b, pos // bs]) * bs + pos % bs)
    slots = np.array(slots, dtype=np.int32)
    T = len(slots)
    rng = np.random.default_rng(77)
    kn = pa_inputs.to_bf16_bits(rng.standard_normal((T, w.num_kv_heads, w.head_dim)).astype(np.float32))
    vn = pa_inputs.to_bf16_bits(rng.standard_normal((T, w.num_kv_heads, w.head_dim)).astype(np.float32))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    k = dev(kn.view(np.int16)).view(torch.bfloat16)
    v = dev(vn.view(np.int16)).view(torch.bfloat16)
    if fp8:
        kp, vp = dev(w.k_pool), dev(w.v_pool)
        ks, vs = dev(w.k_scale), dev(w.v_scale)
    else:
        kp = dev(w.k_pool.view(np.int16)).view(torch.bfloat16)
        vp = dev(w.v_pool.view(np.int16)).view(torch.bfloat16)
        ks = vs = None
    sm = dev(slots)
    a = binding.make_append_args(k, v, sm, kp, vp, ks, vs)
    import ctypes
    call = lambda: binding.check(binding.LIB.pa_append(  # noqa: E731
        ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # a launch lasts a few microseconds, about as long as an event pair's own overhead, so
    # events bracket batches of `per` back-to-back launches on the launch stream
    per = 10
    nb = max(1, args.steps // per)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nb)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record()
        for _ in range(per):
            call()
        e[1].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / (nb * per)
    k_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) / per
    nbytes = T * w.num_kv_heads * w.head_dim * 2 * (2 + (1 if fp8 else 2)) + 4 * T + (64 if fp8 else 0)
    ach = nbytes / (k_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "paged KV append GB/s (new tokens written to their cache slots)",
        "value": round(nbytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": nb * per, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 -> fp8-e4m3" if fp8 else "bf16",
        "data": "synthetic (seeded N(0,1) values, slots of the mixed workload's new tokens)",
        "config": {"workload": f"append {T} tokens (96 decode + 8x256 prefill rows), 8 kv heads, "
                               f"head_dim 128, bs 16, {'fp8' if fp8 else 'bf16'} pool", "tokens": T},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "append_kernel",
                     "kernel_ms_mean": round(k_ms, 5), "bytes_per_launch": int(nbytes)},
        "cpu_baseline": None,
    }), flush=True)


def _timed(call, steps, warmup, prewarm_ms=0.0):
    """Mean ms per call from events around each call, and wall ms per call over the loop."""
    import numpy as np
    import torch
    prewarm(call, prewarm_ms)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    # events on every EVENT_STRIDE-th call only: each record costs the stream a few microseconds
    stride = max(1, min(EVENT_STRIDE, steps // 8))
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in range(0, steps, stride)}
    t0 = time.perf_counter()
    for i in range(steps):
        e = evs.get(i)
        if e:
            e[0].record()
        call()
        if e:
            e[1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return float(np.mean([e[0].elapsed_time(e[1]) for e in evs.values()])), wall


def bench_cascade(args):
    """Shared-prefix decode (workload 7): pa_decode_cascade, and pa_decode on the same rows."""
    import numpy as np
    import torch

    import pa_inputs
    from paged_kv_attention_13_amd import accounting, binding
    from paged_kv_attention_13_amd.device import to_device

    w = pa_inputs.make_config(7)
    d = to_device(w)
    out = torch.empty(d["q"].shape, dtype=torch.bfloat16, device="cuda")
    rows_per_group = int(np.diff(w.group_start).max())
    c = binding.make_cascade_args(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"],
                                  d["group_start"], d["shared_len"], w.scale, max_seq_len=w.max_seq_len,
                                  max_group_rows=rows_per_group, out=out, num_workers=args.num_workers)
    ws = torch.empty(max(binding.cascade_workspace_bytes(c), 16), dtype=torch.uint8, device="cuda")
    c.base.workspace, c.base.workspace_bytes = ws.data_ptr(), ws.numel()
    out_dec = torch.empty_like(out)
    a = binding.make_decode_args(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], w.scale,
                                 max_seq_len=w.max_seq_len, out=out_dec,
                                 num_workers=args.num_workers)
    wsd = torch.empty(max(binding.plan(a).workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = wsd.data_ptr(), wsd.numel()

    c_ms, c_wall = _timed(lambda: binding.cascade_args_call(c), args.steps, args.warmup, args.prewarm_ms)
    d_ms, d_wall = _timed(lambda: binding.decode_args_call(a), args.steps, args.warmup, args.prewarm_ms)

    Hkv, D = w.num_kv_heads, w.head_dim
    logical = accounting.kv_bytes(w.seq_lens, Hkv, D, "bf16")             # every row's whole cache
    gs = w.group_start
    shared = [int(w.shared_len[gs[k]]) for k in range(len(gs) - 1)]
    own = accounting.kv_bytes(w.seq_lens - w.shared_len, Hkv, D, "bf16")
    physical = own + accounting.kv_bytes(np.array(shared), Hkv, D, "bf16")  # each prefix once per group
    q_bytes = int(w.q.nbytes)
    ach = (physical + q_bytes) / (c_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "shared-prefix decode: effective KV GB/s (every row's whole cache / step time)",
        "value": round(logical / (c_wall * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(c_wall, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) values; 64 rows sharing the blocks of one 1,488-token prefix)",
        "config": {"workload": w.name, "batch": w.num_seqs, "groups": len(gs) - 1,
                   "shared_tokens": shared[0], "context_tokens": int(w.seq_lens.sum()),
                   "block_size": w.block_size, "q_heads": w.num_q_heads, "kv_heads": Hkv, "head_dim": D},
        "logical_kv_bytes": int(logical), "physical_kv_bytes": int(physical),
        "cascade_call_ms": round(c_ms, 5),
        "decode_same_rows": {"call_ms": round(d_ms, 5), "ms_per_step": round(d_wall, 5),
                             "effective_GBs": round(logical / (d_wall * 1e-3) / 1e9, 1)},
        "speedup_vs_decode": round(d_wall / c_wall, 3),
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "pa_decode_cascade call (prefix + row-part + merge kernels)",
                     "kernel_ms_mean": round(c_ms, 5), "bytes_per_launch": int(physical + q_bytes)},
        "cpu_baseline": None,
    }), flush=True)


def bench_prefill(args):
    """Causal prefill-chunk rows alone (pa_mixed with no decode or verify rows)."""
    import torch

    import pa_inputs
    from paged_kv_attention_13_amd import accounting, binding
    from paged_kv_attention_13_amd.device import to_device

    w = pa_inputs.make_prefill_case(args.prefill_case)
    d = to_device(w)
    out = torch.empty(d["q"].shape, dtype=torch.bfloat16, device="cuda")
    m = binding.make_mixed_args(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"],
                                d["q_start_loc"], w.scale, num_decode_rows=0, max_q_len=int(w.q_lens.max()),
                                max_seq_len=w.max_seq_len, out=out)
    ws = torch.empty(max(binding.mixed_workspace_bytes(m), 16), dtype=torch.uint8, device="cuda")
    m.base.workspace, m.base.workspace_bytes = ws.data_ptr(), ws.numel()
    c_ms, wall = _timed(lambda: binding.mixed_args_call(m), args.steps, args.warmup, args.prewarm_ms)
    flops = accounting.call_flops(w.seq_lens, w.q_lens, w.num_q_heads, w.head_dim)
    ach = flops / (c_ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "prefill-chunk attention: algorithmic TFLOP/s (causal part only)",
        "value": round(flops / (wall * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) values)",
        "config": {"workload": w.name, "rows": w.num_seqs, "new_tokens": int(w.q_lens.sum()),
                   "cached_tokens": int(w.seq_lens.sum()), "block_size": w.block_size,
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim},
        "flops_per_call": int(flops),
        "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "pa_mixed call (prefill kernel, plus the piece merge when units are few)",
                     "kernel_ms_mean": round(c_ms, 5)},
        "cpu_baseline": None,
    }), flush=True)


def bench_loop(args):
    """Decode steps of a 32-layer attention stack at small batch: eager launches vs one graph replay."""
    import numpy as np
    import torch

    from paged_kv_attention_13_amd import binding
    from paged_kv_attention_13_amd.loop import DecodeLoop

    B, layers, prompt, bs = args.loop_batch, 32, 511, 16
    mk = lambda: DecodeLoop(num_layers=layers, num_blocks=B * 64 + 8, block_size=bs,  # noqa: E731
                            max_blocks_per_seq=64, max_batch_size=B, max_num_tokens=B * prompt,
                            prefix_reuse=False)
    loops = {"eager": mk(), "graph": mk()}
    rng = np.random.default_rng(11)
    for lp in loops.values():
        for r in range(B):
            lp.kvm.add_request(r, rng.integers(0, 32000, size=prompt), args.warmup + args.steps + 5)
        for layer in range(layers):
            for t in (lp.q[layer], lp.k_new[layer], lp.v_new[layer]):
                t.normal_()
        b = lp.schedule()                        # the whole prompt in one pass
        lp.run_batch(b)
        torch.cuda.synchronize()
        lp.complete(np.zeros(b.num_rows, np.int32))
        lp.prepare_decode(B)
    res = {}
    for mode, lp in loops.items():
        step_ms, gpu_ms = [], []
        for i in range(args.warmup + args.steps):
            b = lp.schedule()
            assert b.num_rows == B and b.num_decode_rows == B
            lp.stage(b)
            if mode == "graph" and lp.graph is None:
                lp.capture_decode_step()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record()
            if mode == "graph":
                lp.decode_step_graph()
            else:
                lp.decode_step_eager()
            e1.record()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            lp.complete(np.zeros(B, np.int32))
            if i >= args.warmup:
                step_ms.append((t1 - t0) * 1e3)
                gpu_ms.append(e0.elapsed_time(e1))
        res[mode] = {"ms_per_step": float(np.mean(step_ms)), "gpu_ms": float(np.mean(gpu_ms)),
                     "p90_ms": float(np.percentile(step_ms, 90))}
    ctx = prompt + args.warmup + args.steps // 2
    kv = layers * B * ctx * 8 * 128 * 2 * 2
    g = res["graph"]["ms_per_step"]
    # one launch per layer when the decode plan runs one workgroup per unit (no workspace)
    fused = binding.plan(loops["graph"]._calls[0][1]).workspace_bytes == 0
    per_layer = 1 if fused else 3
    print(json.dumps({
        "metric": "decode-loop step latency, 32 layers of paged KV append + attention (graph replay)",
        "value": round(B / (g * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(g, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": f"synthetic (seeded N(0,1) q/K/V; {B} request(s) with a {prompt}-token prompt, then decode)",
        "config": {"workload": f"decode loop B{B} ctx~{ctx} 32 layers bs16", "batch": B, "layers": layers,
                   "q_heads": 32, "kv_heads": 8, "head_dim": 128, "block_size": bs,
                   "launches_per_step_eager": layers * per_layer + 4,
                   "per_layer": "pa_append_decode: one launch" if fused else "append + decode + merge"},
        "eager": {k: round(v, 5) for k, v in res["eager"].items()},
        "graph": {k: round(v, 5) for k, v in res["graph"].items()},
        "graph_speedup": round(res["eager"]["ms_per_step"] / g, 3),
        "kv_bytes_per_step": int(kv),
        "roofline": {"bound": "hbm", "achieved": round(kv / (res["graph"]["gpu_ms"] * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kv / (res["graph"]["gpu_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "graph replay (32 x " + ("append + decode in one launch)" if fused else "append + decode + merge)"),
                     "kernel_ms_mean": round(res["graph"]["gpu_ms"], 5), "bytes_per_launch": int(kv)},
        "cpu_baseline": None,
    }), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU (attention over the paged KV cache needs "
              "no exchange between GPUs; see the sharding note in the design document); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    if args.op == "cascade":
        bench_cascade(args)
        return
    if args.op == "loop":
        bench_loop(args)
        return
    if args.op == "prefill":
        bench_prefill(args)
        return
    if args.op == "stream":
        bench_stream(args)
        return
    if args.op != "decode":
        bench_append(args)
        return

    import numpy as np
    import torch

    import pa_inputs
    from paged_kv_attention_13_amd import accounting, binding
    from paged_kv_attention_13_amd.device import to_device

    t_gen = time.perf_counter()
    w = pa_inputs.make_config(args.workload)
    d = to_device(w)
    gen_s = time.perf_counter() - t_gen
    mixed = not w.is_decode_only
    out = torch.empty(d["q"].shape, dtype=d["q"].dtype, device="cuda")

    if mixed:
        n_dec = w.num_decode_rows
        # rows after the decode rows with at most 32 query columns per kv head go to the
        # multi-query (verify) kernel, the rest to the prefill-chunk kernel
        group = w.num_q_heads // w.num_kv_heads
        n_ver = 0
        while n_dec + n_ver < w.num_seqs and w.q_lens[n_dec + n_ver] * group <= 32:
            n_ver += 1
        pre_q = w.q_lens[n_dec + n_ver:]
        m = binding.make_mixed_args(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"],
                                    d["q_start_loc"], w.scale, num_decode_rows=n_dec,
                                    max_q_len=int(pre_q.max()) if len(pre_q) else 1,
                                    max_seq_len=w.max_seq_len, out=out, num_workers=args.num_workers,
                                    num_verify_rows=n_ver,
                                    max_verify_q_len=int(w.q_lens[n_dec:n_dec + n_ver].max()) if n_ver else 0)
        nbytes = binding.mixed_workspace_bytes(m)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        m.base.workspace, m.base.workspace_bytes = ws.data_ptr(), ws.numel()
        dec = binding.make_decode_args(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"],
                                       w.scale, max_seq_len=w.max_seq_len, out=out,
                                       num_workers=args.num_workers)
        dec.num_seqs = n_dec
        pl = binding.plan(dec)
        step = lambda: binding.mixed_args_call(m)  # noqa: E731
        stages = None
    else:
        a = binding.make_decode_args(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"],
                                     w.scale, max_seq_len=w.max_seq_len, k_scale=d["k_scale"],
                                     v_scale=d["v_scale"], out=out, num_workers=args.num_workers)
        pl = binding.plan(a)
        ws = torch.empty(max(pl.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        # rows on the one-workgroup-per-unit path (no workspace) have no merge stage
        unit_path = pl.workspace_bytes == 0
        stages = (lambda: binding.decode_partials(a), None if unit_path else (lambda: binding.merge_partials(a)))
        step = None
        n_dec, n_ver = w.num_seqs, 0

    two_stage = stages is not None and stages[1] is not None

    def run_step(evs=None):
        if evs:
            evs[0].record()
        if stages is None:
            step()
        else:
            stages[0]()
        if evs and evs[1] is not None:
            evs[1].record()
        if two_stage:
            stages[1]()
            if evs:
                evs[2].record()

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    prewarm_steps = prewarm(run_step, args.prewarm_ms)
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # Each event record costs the stream ~6 us on this GPU (measured: the long-context step takes
    # 281 us bare, 286 us with an event pair around the decode kernel, 293 us with a third after
    # the merge), so the per-kernel events are recorded on every EVENT_STRIDE-th timed step only;
    # the step time is the wall clock over all timed steps.  With a scrub between steps the step
    # time is the median of per-step events instead, so every step carries a start and an end
    # event, and only every other step the event between the two kernels (whose own cost would
    # otherwise sit inside the measured step): the kernel time comes from those steps.
    if args.scrub_mib is None:
        args.scrub_mib = 1024 if accounting.workload_bytes(w)["kv"] < (1 << 30) else 0
    # the scrub reads (it does not write): a write would leave the caches full of dirty lines
    # whose write-back then competes with the next step's reads
    scrub = torch.ones((args.scrub_mib << 20) // 4, dtype=torch.int32, device="cuda") if args.scrub_mib > 0 else None
    scrub_out = torch.empty((), dtype=torch.int32, device="cuda")
    stride = 1 if scrub is not None else max(1, min(EVENT_STRIDE, args.steps // 8))
    sampled = list(range(0, args.steps, stride))
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    if scrub is not None and two_stage:
        for i in sampled[1::2]:
            evs[i][1] = None                 # step-time samples: no event between the kernels
    sampler = GpuSampler()
    torch.cuda.synchronize()
    sampler.start()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if scrub is not None:
            torch.amax(scrub, dim=0, out=scrub_out)
        run_step(evs.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gpu_state_summary = sampler.stop("the timed steps")
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    last = 2 if two_stage else 1
    split = [e for e in evs.values() if e[1] is not None]      # steps with the between-kernels event
    if scrub is not None:
        whole = [e for e in evs.values() if e[1] is None] or split
        ms_per_step = float(np.median([e[0].elapsed_time(e[last]) for e in whole]))
    k_ms = [e[0].elapsed_time(e[1]) for e in split]
    m_ms = [e[1].elapsed_time(e[2]) for e in split] if two_stage else []
    kernel_ms = float(np.mean(k_ms))

    cb = accounting.workload_bytes(w)
    kv_bytes = cb["kv"]
    # algorithmic bytes of the split-K kernel (one launch): KV + scales + q + block table
    # entries + seq_lens; the output is written by the merge kernel
    split_bytes = cb["kv"] + cb["scales"] + cb["q"] + cb["meta"]
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = split_bytes / (kernel_ms * 1e-3) / 1e9
    if mixed:
        kernel_label = "pa_mixed call (all kernels)"
    elif w.kv_fmt == "fp8":
        kernel_label = "verify_kernel (multi-query kernel on FP8 decode rows, partials)"
    elif stages[1] is None:
        kernel_label = "decode_unit_kernel (one workgroup per row and kv head, whole call)"
    else:
        kernel_label = "decode_kernel (balanced split, partials)"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if mixed else committed_traffic(w.kv_fmt, w.name),
                "kernel": kernel_label,
                "kernel_ms_mean": round(kernel_ms, 5), "kernel_ms_p10": round(float(np.percentile(k_ms, 10)), 5),
                "kernel_ms_p90": round(float(np.percentile(k_ms, 90)), 5),
                "kernel_launches_timed": len(k_ms),
                "merge_ms_mean": round(float(np.mean(m_ms)), 5) if m_ms else None,
                "bytes_per_launch": int(split_bytes)}
    flops = accounting.call_flops(w.seq_lens, w.q_lens, w.num_q_heads, w.head_dim)

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 kv, bf16 q"}[w.kv_fmt] if w.kv_fmt != "bf16" else "bf16",
        "data": "synthetic (seeded N(0,1) values, random block tables)",
        "config": {"workload": w.name, "batch": w.num_seqs, "total_q": w.total_q,
                   "context_tokens": int(w.seq_lens.sum()), "max_context": w.max_seq_len,
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "kv_dtype": w.kv_fmt,
                   "decode_rows": w.num_decode_rows if mixed else w.num_seqs,
                   "verify_rows": n_ver if mixed else 0,
                   "decode_workers": pl.num_workers if pl.num_workers and (not mixed or n_dec) else None,
                   "tile_tokens": pl.tile_tokens,
                   "scrub_mib_between_steps": args.scrub_mib,
                   "prewarm": f"{prewarm_steps} untimed steps in {args.prewarm_ms:.0f} ms before the warm-up"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(w.total_q / (ms_per_step * 1e-3), 1),
        "kv_tokens_per_s": round(float(w.seq_lens.sum()) / (ms_per_step * 1e-3), 1),
        "kv_bytes_per_step": int(kv_bytes),
        "algorithmic_flops_per_step": int(flops),
        "roofline": roofline,
        "input_generation_s": round(gen_s, 2),
    }
    st = None if args.skip_probes else stream_ceiling(kv_bytes, prewarm_ms=min(100.0, args.prewarm_ms))
    if st is not None:
        res["stream_read"] = st
        res["pct_of_stream"] = round(100 * value / st["GBs"], 2)
        res["kernel_pct_of_stream"] = round(100 * achieved / st["GBs"], 2)
    if not mixed and not args.skip_probes:
        gt = gather_ceiling(w, d, prewarm_ms=min(100.0, args.prewarm_ms))
        res["gather_read"] = gt
        res["pct_of_gather"] = round(100 * value / gt["GBs"], 2)
        res["kernel_pct_of_gather"] = round(100 * achieved / gt["GBs"], 2)
    if args.cpu_seconds > 0:
        gpu_out = out.float().cpu().numpy().astype(np.float64)
        res["cpu_baseline"] = cpu_baseline(w, gpu_out, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    res["gpu_state"] = gpu_state_summary
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

"""A per-layer decode loop driven by the host cache manager, eager or as one HIP graph.

Each step: the manager schedules a pass (decode rows first, then prefill
chunks; "TensorRT-LLM, in depth", aicassindra.com, section "In-flight batching
and the scheduler"), its metadata is copied to the device, and for every layer
the step's new K/V are appended to that layer's paged pools (``pa_append``) and
attention runs over them (``pa_mixed``, or ``pa_decode`` when every row
decodes).  Every step of a steady decode batch issues the same launches, so the
whole step can be recorded once as a graph and replayed with one launch
("How does TensorRT-LLM work", outcomeschool.com, section "CUDA graphs"); the
metadata copies from pinned host buffers are part of the graph, so a replay
picks up the host's new block table and lengths.

Argument marshalling and orchestration only: scheduling is the library's C++
manager, every step of the computation its HIP kernels.
"""
from __future__ import annotations

import ctypes
from typing import Callable, Optional

import numpy as np

from . import binding
from .runtime import Batch, KVManager


class DecodeLoop:
    """``num_layers`` layers of paged attention (bf16), one K and one V pool per layer."""

    def __init__(self, *, num_layers: int, num_blocks: int, block_size: int, max_blocks_per_seq: int,
                 max_batch_size: int, max_num_tokens: int, num_q_heads: int = 32, num_kv_heads: int = 8,
                 head_dim: int = 128, prefix_reuse: bool = True, device: str = "cuda"):
        import torch
        self.torch = torch
        self.L, self.bs, self.mbps = num_layers, block_size, max_blocks_per_seq
        self.max_bs, self.max_tok = max_batch_size, max_num_tokens
        self.Hq, self.Hkv, self.D = num_q_heads, num_kv_heads, head_dim
        self.kvm = KVManager(num_blocks, block_size, max_blocks_per_seq, prefix_reuse)
        bf = torch.bfloat16
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.k_pools = [torch.zeros(shape, dtype=bf, device=device) for _ in range(num_layers)]
        self.v_pools = [torch.zeros(shape, dtype=bf, device=device) for _ in range(num_layers)]
        # device metadata (fixed addresses) and pinned host staging for it
        i32 = torch.int32
        self.d_table = torch.full((max_batch_size, max_blocks_per_seq), -1, dtype=i32, device=device)
        self.d_seq = torch.ones(max_batch_size, dtype=i32, device=device)
        self.d_qsl = torch.zeros(max_batch_size + 1, dtype=i32, device=device)
        self.d_slots = torch.full((max_num_tokens,), -1, dtype=i32, device=device)
        self.h_table = torch.full((max_batch_size, max_blocks_per_seq), -1, dtype=i32).pin_memory()
        self.h_seq = torch.ones(max_batch_size, dtype=i32).pin_memory()
        self.h_qsl = torch.zeros(max_batch_size + 1, dtype=i32).pin_memory()
        self.h_slots = torch.full((max_num_tokens,), -1, dtype=i32).pin_memory()
        # per-layer step inputs and outputs
        self.q = [torch.zeros((max_num_tokens, num_q_heads, head_dim), dtype=bf, device=device)
                  for _ in range(num_layers)]
        self.k_new = [torch.zeros((max_num_tokens, num_kv_heads, head_dim), dtype=bf, device=device)
                      for _ in range(num_layers)]
        self.v_new = [torch.zeros((max_num_tokens, num_kv_heads, head_dim), dtype=bf, device=device)
                      for _ in range(num_layers)]
        self.out = [torch.zeros((max_num_tokens, num_q_heads, head_dim), dtype=bf, device=device)
                    for _ in range(num_layers)]
        self.scale = 1.0 / float(np.sqrt(head_dim))
        self.max_seq_bound = max_blocks_per_seq * block_size
        self._ws = None
        self.graph = None
        self._graph_rows = None

    # ---- metadata --------------------------------------------------------------------
    def _stage(self, b: Batch) -> None:
        """Write a batch's metadata into the pinned staging buffers (host side)."""
        B, T = b.num_rows, b.total_q
        self.h_table.fill_(-1)
        self.h_table[:B].copy_(self.torch.from_numpy(b.block_table))
        self.h_seq.fill_(1)
        self.h_seq[:B].copy_(self.torch.from_numpy(b.seq_lens))
        self.h_qsl.zero_()
        self.h_qsl[:B + 1].copy_(self.torch.from_numpy(b.q_start_loc))
        self.h_qsl[B + 1:] = int(b.q_start_loc[-1])
        self.h_slots.fill_(-1)
        self.h_slots[:T].copy_(self.torch.from_numpy(b.slot_mapping))

    def _upload(self) -> None:
        for d, h in ((self.d_table, self.h_table), (self.d_seq, self.h_seq), (self.d_qsl, self.h_qsl),
                     (self.d_slots, self.h_slots)):
            d.copy_(h, non_blocking=True)

    def _workspace(self, nbytes: int):
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = self.torch.empty(max(nbytes, 256), dtype=self.torch.uint8, device=self.d_seq.device)
        return self._ws

    # ---- one step, any batch -----------------------------------------------------------
    def schedule(self) -> Batch:
        return self.kvm.schedule(self.max_bs, self.max_tok)

    def run_batch(self, b: Batch) -> None:
        """Queue one pass over every layer for batch ``b`` (inputs already in q/k_new/v_new)."""
        torch = self.torch
        self._stage(b)
        self._upload()
        B, T = b.num_rows, b.total_q
        if B == 0:
            return
        n_dec = b.num_decode_rows
        n_pre = B - n_dec
        for layer in range(self.L):
            kp, vp = self.k_pools[layer], self.v_pools[layer]
            a = binding.make_append_args(self.k_new[layer][:T], self.v_new[layer][:T], self.d_slots[:T], kp, vp)
            binding.check(binding.LIB.pa_append(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
            m = binding.make_mixed_args(self.q[layer][:T], kp, vp, self.d_table[:B], self.d_seq[:B], self.d_qsl[:B + 1],
                                        self.scale, num_decode_rows=n_dec, max_q_len=max(b.max_q_len, 1) if n_pre else 1,
                                        max_seq_len=self.max_seq_bound, out=self.out[layer][:T])
            ws = self._workspace(binding.mixed_workspace_bytes(m))
            m.base.workspace, m.base.workspace_bytes = ws.data_ptr(), ws.numel()
            binding.mixed_args_call(m)

    # ---- steady decode: fixed rows, prebuilt arguments, optional graph ------------------
    def _decode_calls(self, B: int):
        """Prebuilt (append, decode) argument structs per layer for B decode rows."""
        calls = []
        for layer in range(self.L):
            kp, vp = self.k_pools[layer], self.v_pools[layer]
            a = binding.make_append_args(self.k_new[layer][:B], self.v_new[layer][:B], self.d_slots[:B], kp, vp)
            d = binding.make_decode_args(self.q[layer][:B], kp, vp, self.d_table[:B], self.d_seq[:B], self.scale,
                                         max_seq_len=self.max_seq_bound, out=self.out[layer][:B])
            ws = self.torch.empty(max(binding.plan(d).workspace_bytes, 256), dtype=self.torch.uint8,
                                  device=self.d_seq.device)
            d.workspace, d.workspace_bytes = ws.data_ptr(), ws.numel()
            calls.append((a, d, ws))
        return calls

    def _launch_decode(self, calls) -> None:
        # one pa_append_decode per layer: for short rows a single launch appends the new
        # token and attends over it; otherwise it queues the append and the decode
        s = ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        for a, d, _ in calls:
            binding.check(binding.LIB.pa_append_decode(ctypes.byref(a), ctypes.byref(d), s))

    def prepare_decode(self, B: int) -> None:
        self._calls = self._decode_calls(B)
        self._calls_rows = B

    def decode_step_eager(self) -> None:
        """Upload the staged metadata and launch every layer's append + decode."""
        self._upload()
        self._launch_decode(self._calls)

    def capture_decode_step(self) -> None:
        """Record upload + every layer's append + decode as one graph (fixed rows).

        The step runs once eagerly first (so every kernel is loaded before the
        recording); appending the same tokens at the same slots again in the
        first replay writes the same values, so that replay computes the same step.
        """
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):                  # warm the launch path outside the capture
            self.decode_step_eager()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.decode_step_eager()
        self.graph = g

    def decode_step_graph(self) -> None:
        self.graph.replay()

    def stage(self, b: Batch) -> None:
        self._stage(b)

    def complete(self, sampled) -> None:
        self.kvm.complete(sampled)


def fill_inputs(loop: DecodeLoop, b: Batch, value_fn: Callable[..., np.ndarray]) -> None:
    """Fill each layer's q / k_new / v_new rows for batch ``b``.

    ``value_fn(request_id, token_id, position, layer, kind)`` returns a float32
    vector (kind "q": [Hq, D]; "k" / "v": [Hkv, D]).
    """
    torch = loop.torch
    T = b.total_q
    if T == 0:
        return
    rows = np.repeat(b.request_ids, b.q_lens)
    for layer in range(loop.L):
        for kind, buf in (("q", loop.q[layer]), ("k", loop.k_new[layer]), ("v", loop.v_new[layer])):
            x = np.stack([value_fn(int(rows[t]), int(b.token_ids[t]), int(b.positions[t]), layer, kind)
                          for t in range(T)])
            buf[:T].copy_(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16))


__all__ = ["DecodeLoop", "fill_inputs"]

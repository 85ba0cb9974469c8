"""ctypes binding of the host-side cache manager and scheduler (``include/pa_runtime.h``).

Argument marshalling only: block allocation, prefix reuse and scheduling run
in the library's C++ code.
"""
from __future__ import annotations

import ctypes
import dataclasses

import numpy as np

from .binding import LIB, PagedAttentionError, check

P = ctypes.POINTER


class KvmBatch(ctypes.Structure):
    _fields_ = [
        ("num_rows", ctypes.c_int32),
        ("num_decode_rows", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("request_ids", P(ctypes.c_int64)),
        ("seq_lens", P(ctypes.c_int32)),
        ("q_start_loc", P(ctypes.c_int32)),
        ("block_table", P(ctypes.c_int32)),
        ("slot_mapping", P(ctypes.c_int32)),
        ("positions", P(ctypes.c_int32)),
        ("token_ids", P(ctypes.c_int32)),
    ]


class KvmRequestInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("state", "prompt_len", "num_cached", "num_reused", "num_generated", "num_blocks")]


_SIGS = {
    "pa_kvm_create": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P(ctypes.c_void_p)],
                      ctypes.c_int),
    "pa_kvm_destroy": ([ctypes.c_void_p], None),
    "pa_kvm_add_request": ([ctypes.c_void_p, ctypes.c_int64, P(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32],
                           ctypes.c_int),
    "pa_kvm_schedule": ([ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, P(KvmBatch)], ctypes.c_int),
    "pa_kvm_complete": ([ctypes.c_void_p, P(ctypes.c_int32)], ctypes.c_int),
    "pa_kvm_num_free_blocks": ([ctypes.c_void_p], ctypes.c_int32),
    "pa_kvm_num_used_blocks": ([ctypes.c_void_p], ctypes.c_int32),
    "pa_kvm_request_info_get": ([ctypes.c_void_p, ctypes.c_int64, P(KvmRequestInfo)], ctypes.c_int),
    "pa_kvm_generated": ([ctypes.c_void_p, ctypes.c_int64, P(ctypes.c_int32), ctypes.c_int32, P(ctypes.c_int32)],
                         ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(LIB, _name)
    _fn.argtypes = _args
    _fn.restype = _res

STATES = {0: "waiting", 1: "prefilling", 2: "decoding", 3: "finished"}


@dataclasses.dataclass
class Batch:
    """One pass's metadata, copied out of the manager (numpy arrays)."""
    request_ids: np.ndarray
    num_decode_rows: int
    seq_lens: np.ndarray
    q_start_loc: np.ndarray
    block_table: np.ndarray
    slot_mapping: np.ndarray
    positions: np.ndarray
    token_ids: np.ndarray
    max_q_len: int
    max_seq_len: int

    @property
    def num_rows(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q_start_loc[-1])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.q_start_loc)


def _arr(ptr, n, dtype):
    if n == 0:
        return np.zeros(0, dtype=dtype)
    return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dtype, copy=True)


class KVManager:
    """Owner of one ``pa_kvm`` manager."""

    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int, prefix_reuse: bool = True):
        h = ctypes.c_void_p()
        check(LIB.pa_kvm_create(num_blocks, block_size, max_blocks_per_seq, int(prefix_reuse), ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size, self.max_blocks_per_seq = num_blocks, block_size, max_blocks_per_seq

    def close(self):
        if self._h:
            LIB.pa_kvm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover
            pass

    def add_request(self, rid: int, prompt, max_new_tokens: int) -> None:
        p = np.ascontiguousarray(prompt, dtype=np.int32)
        check(LIB.pa_kvm_add_request(self._h, int(rid), p.ctypes.data_as(P(ctypes.c_int32)), len(p),
                                     int(max_new_tokens)))

    def schedule(self, max_batch_size: int, max_num_tokens: int) -> Batch:
        b = KvmBatch()
        check(LIB.pa_kvm_schedule(self._h, int(max_batch_size), int(max_num_tokens), ctypes.byref(b)))
        B, T, mb = b.num_rows, b.total_q, b.max_blocks_per_seq
        return Batch(request_ids=_arr(b.request_ids, B, np.int64), num_decode_rows=b.num_decode_rows,
                     seq_lens=_arr(b.seq_lens, B, np.int32), q_start_loc=_arr(b.q_start_loc, B + 1, np.int32),
                     block_table=_arr(b.block_table, B * mb, np.int32).reshape(B, mb),
                     slot_mapping=_arr(b.slot_mapping, T, np.int32), positions=_arr(b.positions, T, np.int32),
                     token_ids=_arr(b.token_ids, T, np.int32), max_q_len=b.max_q_len, max_seq_len=b.max_seq_len)

    def complete(self, sampled) -> None:
        s = np.ascontiguousarray(sampled, dtype=np.int32)
        check(LIB.pa_kvm_complete(self._h, s.ctypes.data_as(P(ctypes.c_int32))))

    @property
    def free_blocks(self) -> int:
        return int(LIB.pa_kvm_num_free_blocks(self._h))

    @property
    def used_blocks(self) -> int:
        return int(LIB.pa_kvm_num_used_blocks(self._h))

    def info(self, rid: int) -> dict:
        i = KvmRequestInfo()
        check(LIB.pa_kvm_request_info_get(self._h, int(rid), ctypes.byref(i)))
        return {"state": STATES[i.state], "prompt_len": i.prompt_len, "num_cached": i.num_cached,
                "num_reused": i.num_reused, "num_generated": i.num_generated, "num_blocks": i.num_blocks}

    def generated(self, rid: int) -> np.ndarray:
        n = ctypes.c_int32()
        check(LIB.pa_kvm_generated(self._h, int(rid), None, 0, ctypes.byref(n)))
        out = np.zeros(n.value, dtype=np.int32)
        check(LIB.pa_kvm_generated(self._h, int(rid), out.ctypes.data_as(P(ctypes.c_int32)), n.value,
                                   ctypes.byref(n)))
        return out


__all__ = ["KVManager", "Batch", "PagedAttentionError"]

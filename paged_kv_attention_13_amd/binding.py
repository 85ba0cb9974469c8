"""ctypes binding of ``libpa_kv.so`` (the C ABI declared in ``include/pa.h``).

Argument marshalling only: torch tensors are turned into device pointers and
the current HIP stream, outputs and workspaces are allocated with torch, and
the call goes straight to the library.  Every step of the computation runs
in the library's HIP kernels; there is no fallback.  If the library is not
built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# PA_LIB_PATH selects another build of the same ABI (the tests load the host-only
# sanitizer build this way); by default the in-tree HIP library.
LIB_PATH = os.environ.get("PA_LIB_PATH") or os.path.join(PKG, "libpa_kv.so")

PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_NULL_POINTER", 2: "PA_ERR_BAD_SHAPE", 3: "PA_ERR_BAD_DTYPE",
                4: "PA_ERR_UNSUPPORTED", 5: "PA_ERR_WORKSPACE_TOO_SMALL", 6: "PA_ERR_MISALIGNED",
                7: "PA_ERR_BAD_METADATA", 8: "PA_ERR_HIP"}

EXPORTED = ["pa_abi_version", "pa_decode_plan", "pa_mixed_workspace_size", "pa_decode",
            "pa_decode_partials", "pa_merge_partials", "pa_mixed", "pa_append", "pa_check_decode_metadata",
            "pa_check_mixed_metadata", "pa_check_append_metadata", "pa_cascade_workspace_size",
            "pa_decode_cascade", "pa_check_cascade_metadata", "pa_append_decode",
            "pa_check_append_decode_metadata", "pa_status_string", "pa_last_error",
            "pa_decode_workspace_size", "pa_check_metadata", "pa_stream_read", "pa_decode_noalloc",
            "pa_gather_read", "pa_device_checks", "pa_device_check_flags"]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("num_workers", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("scale", ctypes.c_float),
        ("out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class MixedArgs(ctypes.Structure):
    _fields_ = [
        ("base", DecodeArgs),
        ("q_start_loc", ctypes.c_void_p),
        ("total_q", ctypes.c_int32),
        ("num_decode_rows", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("num_verify_rows", ctypes.c_int32),
        ("max_verify_q_len", ctypes.c_int32),
    ]


class CascadeArgs(ctypes.Structure):
    _fields_ = [
        ("base", DecodeArgs),
        ("group_start", ctypes.c_void_p),
        ("shared_len", ctypes.c_void_p),
        ("num_groups", ctypes.c_int32),
        ("max_group_rows", ctypes.c_int32),
    ]


class AppendArgs(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("src_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("slot_mapping", ctypes.c_void_p),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


class Plan(ctypes.Structure):
    _fields_ = [("num_workers", ctypes.c_int32), ("tile_tokens", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message or STATUS_NAMES.get(status, str(status)))
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m paged_kv_attention_13_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sigs = {
        "pa_abi_version": ([], ctypes.c_int),
        "pa_decode_plan": ([P(DecodeArgs), P(Plan)], ctypes.c_int),
        "pa_decode_workspace_size": ([P(DecodeArgs)], ctypes.c_size_t),
        "pa_check_metadata": ([P(MixedArgs)], ctypes.c_int),
        "pa_stream_read": ([ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                            ctypes.c_void_p], ctypes.c_int),
        "pa_gather_read": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                            ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p], ctypes.c_int),
        "pa_mixed_workspace_size": ([P(MixedArgs), P(ctypes.c_size_t)], ctypes.c_int),
        "pa_decode": ([P(DecodeArgs), ctypes.c_void_p], ctypes.c_int),
        "pa_decode_partials": ([P(DecodeArgs), ctypes.c_void_p], ctypes.c_int),
        "pa_decode_noalloc": ([P(DecodeArgs), ctypes.c_void_p], ctypes.c_int),
        "pa_merge_partials": ([P(DecodeArgs), ctypes.c_void_p], ctypes.c_int),
        "pa_mixed": ([P(MixedArgs), ctypes.c_void_p], ctypes.c_int),
        "pa_append": ([P(AppendArgs), ctypes.c_void_p], ctypes.c_int),
        "pa_check_append_metadata": ([P(AppendArgs)], ctypes.c_int),
        "pa_append_decode": ([P(AppendArgs), P(DecodeArgs), ctypes.c_void_p], ctypes.c_int),
        "pa_check_append_decode_metadata": ([P(AppendArgs), P(DecodeArgs)], ctypes.c_int),
        "pa_check_decode_metadata": ([P(DecodeArgs)], ctypes.c_int),
        "pa_check_mixed_metadata": ([P(MixedArgs)], ctypes.c_int),
        "pa_cascade_workspace_size": ([P(CascadeArgs), P(ctypes.c_size_t)], ctypes.c_int),
        "pa_decode_cascade": ([P(CascadeArgs), ctypes.c_void_p], ctypes.c_int),
        "pa_check_cascade_metadata": ([P(CascadeArgs)], ctypes.c_int),
        "pa_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "pa_last_error": ([], ctypes.c_char_p),
        "pa_device_checks": ([], ctypes.c_int),
        "pa_device_check_flags": ([P(ctypes.c_uint32)], ctypes.c_int),
    }
    for name, (argtypes, restype) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    return lib


LIB = _load()


def check(status: int) -> None:
    if status != 0:
        raise PagedAttentionError(status, LIB.pa_last_error().decode())


CHECK_BLOCK_ID, CHECK_SEQ_LEN, CHECK_Q_LEN, CHECK_SLOT = 1, 2, 4, 8


def device_check_flags() -> int:
    """``pa_device_check_flags``: synchronise the device and return (and clear) the PA_CHECK_*
    bits the kernels of a debug build (``pa_device_checks() == 1``) recorded; 0 otherwise."""
    v = ctypes.c_uint32(0)
    check(LIB.pa_device_check_flags(ctypes.byref(v)))
    return int(v.value)


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class _on_stream:
    """Make ``stream`` (if given) torch's current stream for the duration of a call, so that the
    output and workspace the call allocates belong to the stream its kernels run on: the caching
    allocator then does not hand that memory to other streams' work while the kernels use it."""

    def __init__(self, stream):
        self.ctx = None if stream is None else _torch().cuda.stream(stream)

    def __enter__(self):
        if self.ctx is not None:
            self.ctx.__enter__()

    def __exit__(self, *exc):
        if self.ctx is not None:
            return self.ctx.__exit__(*exc)
        return False


def _hold(struct, *objs):
    """Keep the tensors whose addresses a struct carries alive as long as the struct.

    The C structs hold plain addresses; without this a temporary tensor passed in
    (``out=torch.empty(...)``) would be freed at once and its memory handed to the
    next allocation while the library still writes there.
    """
    keep = getattr(struct, "_keep", None)
    if keep is None:
        keep = []
        struct._keep = keep
    keep.extend(o for o in objs if o is not None)
    return struct


def make_decode_args(q, k_pool, v_pool, block_table, seq_lens, scale, *, max_seq_len: int,
                     k_scale=None, v_scale=None, out=None, num_workers: int = 0,
                     workspace=None) -> DecodeArgs:
    a = DecodeArgs()
    a.num_seqs = int(seq_lens.shape[0])
    a.num_q_heads = int(q.shape[1])
    a.num_kv_heads = int(k_pool.shape[1])
    a.head_dim = int(q.shape[2])
    a.block_size = int(k_pool.shape[2])
    a.num_blocks = int(k_pool.shape[0])
    a.max_blocks_per_seq = int(block_table.shape[1])
    a.max_seq_len = int(max_seq_len)
    a.num_workers = int(num_workers)
    a.q_dtype = dtype_code(q)
    a.kv_dtype = dtype_code(k_pool)
    a.out_dtype = dtype_code(out) if out is not None else a.q_dtype
    a.q = _ptr(q)
    a.k_pool = _ptr(k_pool)
    a.v_pool = _ptr(v_pool)
    a.k_scale = _ptr(k_scale)
    a.v_scale = _ptr(v_scale)
    a.block_table = _ptr(block_table)
    a.seq_lens = _ptr(seq_lens)
    a.scale = float(scale)
    a.out = _ptr(out)
    if workspace is not None:
        a.workspace = _ptr(workspace)
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return _hold(a, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, out, workspace)


def plan(args: DecodeArgs) -> Plan:
    p = Plan()
    check(LIB.pa_decode_plan(ctypes.byref(args), ctypes.byref(p)))
    return p


SIZE_MAX = ctypes.c_size_t(-1).value


def decode_workspace_bytes(args: DecodeArgs) -> int:
    """``pa_decode_workspace_size``: bytes of workspace a decode call needs."""
    n = int(LIB.pa_decode_workspace_size(ctypes.byref(args)))
    if n == SIZE_MAX:
        raise PagedAttentionError(2, LIB.pa_last_error().decode())
    return n


def _alloc_out(q, out_dtype):
    torch = _torch()
    return torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)


def _alloc_workspace(nbytes: int, device):
    torch = _torch()
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def decode(q, k_pool, v_pool, block_table, seq_lens, scale, *, max_seq_len: int,
           k_scale=None, v_scale=None, out=None, out_dtype=None, num_workers: int = 0,
           workspace=None, stream=None):
    """Decode attention (``pa_decode``).  Returns ``out`` [B, Hq, D]."""
    with _on_stream(stream):
        if out is None:
            out = _alloc_out(q, out_dtype)
        a = make_decode_args(q, k_pool, v_pool, block_table, seq_lens, scale, max_seq_len=max_seq_len,
                             k_scale=k_scale, v_scale=v_scale, out=out, num_workers=num_workers)
        if workspace is None:
            workspace = _alloc_workspace(decode_workspace_bytes(a), q.device)
        if workspace is not None:
            a.workspace = _ptr(workspace)
            a.workspace_bytes = workspace.numel() * workspace.element_size()
        check(LIB.pa_decode(ctypes.byref(a), ctypes.c_void_p(_stream(stream))))
    return out


def decode_noalloc_args_call(args: DecodeArgs, stream=None) -> None:
    """``pa_decode_noalloc``: pa_decode with the library's static scratch (args.workspace ignored)."""
    check(LIB.pa_decode_noalloc(ctypes.byref(args), ctypes.c_void_p(_stream(stream))))


def decode_partials(args: DecodeArgs, stream=None) -> None:
    check(LIB.pa_decode_partials(ctypes.byref(args), ctypes.c_void_p(_stream(stream))))


def merge_partials(args: DecodeArgs, stream=None) -> None:
    check(LIB.pa_merge_partials(ctypes.byref(args), ctypes.c_void_p(_stream(stream))))


def decode_args_call(args: DecodeArgs, stream=None) -> None:
    check(LIB.pa_decode(ctypes.byref(args), ctypes.c_void_p(_stream(stream))))


def make_mixed_args(q, k_pool, v_pool, block_table, seq_lens, q_start_loc, scale, *,
                    num_decode_rows: int, max_q_len: int, max_seq_len: int, out=None,
                    num_workers: int = 0, num_verify_rows: int = 0,
                    max_verify_q_len: int = 0, k_scale=None, v_scale=None) -> MixedArgs:
    m = MixedArgs()
    base = make_decode_args(q, k_pool, v_pool, block_table, seq_lens, scale, max_seq_len=max_seq_len,
                            k_scale=k_scale, v_scale=v_scale, out=out, num_workers=num_workers)
    m.base = base
    m.q_start_loc = _ptr(q_start_loc)
    m.total_q = int(q.shape[0])
    m.num_decode_rows = int(num_decode_rows)
    m.max_q_len = int(max_q_len)
    m.num_verify_rows = int(num_verify_rows)
    m.max_verify_q_len = int(max_verify_q_len)
    return _hold(m, *base._keep, q_start_loc)


def mixed_workspace_bytes(m: MixedArgs) -> int:
    n = ctypes.c_size_t()
    check(LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n)))
    return int(n.value)


def mixed(q, k_pool, v_pool, block_table, seq_lens, q_start_loc, scale, *, num_decode_rows: int,
          max_q_len: int, max_seq_len: int, out=None, out_dtype=None, num_workers: int = 0,
          num_verify_rows: int = 0, max_verify_q_len: int = 0, k_scale=None, v_scale=None,
          workspace=None, stream=None):
    """Mixed batch (``pa_mixed``): decode rows, then verify rows, then prefill-chunk rows.
    Returns ``out`` [total_q, Hq, D]."""
    with _on_stream(stream):
        if out is None:
            out = _alloc_out(q, out_dtype)
        m = make_mixed_args(q, k_pool, v_pool, block_table, seq_lens, q_start_loc, scale,
                            num_decode_rows=num_decode_rows, max_q_len=max_q_len,
                            max_seq_len=max_seq_len, out=out, num_workers=num_workers,
                            num_verify_rows=num_verify_rows, max_verify_q_len=max_verify_q_len,
                            k_scale=k_scale, v_scale=v_scale)
        if workspace is None:
            workspace = _alloc_workspace(mixed_workspace_bytes(m), q.device)
        if workspace is not None:
            m.base.workspace = _ptr(workspace)
            m.base.workspace_bytes = workspace.numel() * workspace.element_size()
        check(LIB.pa_mixed(ctypes.byref(m), ctypes.c_void_p(_stream(stream))))
    return out


def mixed_args_call(m: MixedArgs, stream=None) -> None:
    check(LIB.pa_mixed(ctypes.byref(m), ctypes.c_void_p(_stream(stream))))


def check_decode_metadata(block_table, seq_lens, *, num_q_heads: int, num_kv_heads: int,
                          head_dim: int, block_size: int, num_blocks: int, max_seq_len: int,
                          q_dtype: int = PA_BF16, kv_dtype: int = PA_BF16) -> None:
    """Host-side precondition check (``pa_check_decode_metadata``) on numpy int32 arrays."""
    import numpy as np
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    a = DecodeArgs()
    a.num_seqs, a.num_q_heads, a.num_kv_heads = len(sl), num_q_heads, num_kv_heads
    a.head_dim, a.block_size, a.num_blocks = head_dim, block_size, num_blocks
    a.max_blocks_per_seq, a.max_seq_len = bt.shape[1], max_seq_len
    a.q_dtype, a.kv_dtype, a.out_dtype = q_dtype, kv_dtype, q_dtype
    a.block_table = bt.ctypes.data
    a.seq_lens = sl.ctypes.data
    check(LIB.pa_check_decode_metadata(ctypes.byref(a)))


def check_mixed_metadata(block_table, seq_lens, q_start_loc, *, num_decode_rows: int, max_q_len: int,
                         num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                         num_blocks: int, max_seq_len: int, num_verify_rows: int = 0,
                         max_verify_q_len: int = 0) -> None:
    import numpy as np
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qs = np.ascontiguousarray(q_start_loc, dtype=np.int32)
    m = MixedArgs()
    a = m.base
    a.num_seqs, a.num_q_heads, a.num_kv_heads = len(sl), num_q_heads, num_kv_heads
    a.head_dim, a.block_size, a.num_blocks = head_dim, block_size, num_blocks
    a.max_blocks_per_seq, a.max_seq_len = bt.shape[1], max_seq_len
    a.q_dtype = a.kv_dtype = a.out_dtype = PA_BF16
    a.block_table = bt.ctypes.data
    a.seq_lens = sl.ctypes.data
    m.q_start_loc = qs.ctypes.data
    m.total_q = int(qs[-1])
    m.num_decode_rows = num_decode_rows
    m.max_q_len = max_q_len
    m.num_verify_rows = num_verify_rows
    m.max_verify_q_len = max_verify_q_len
    check(LIB.pa_check_metadata(ctypes.byref(m)))


def make_cascade_args(q, k_pool, v_pool, block_table, seq_lens, group_start, shared_len, scale, *,
                      max_seq_len: int, max_group_rows: int, out=None, num_workers: int = 0) -> CascadeArgs:
    c = CascadeArgs()
    base = make_decode_args(q, k_pool, v_pool, block_table, seq_lens, scale, max_seq_len=max_seq_len,
                            out=out, num_workers=num_workers)
    c.base = base
    c.group_start = _ptr(group_start)
    c.shared_len = _ptr(shared_len)
    c.num_groups = int(group_start.shape[0]) - 1
    c.max_group_rows = int(max_group_rows)
    return _hold(c, *base._keep, group_start, shared_len)


def cascade_workspace_bytes(c: CascadeArgs) -> int:
    n = ctypes.c_size_t()
    check(LIB.pa_cascade_workspace_size(ctypes.byref(c), ctypes.byref(n)))
    return int(n.value)


def decode_cascade(q, k_pool, v_pool, block_table, seq_lens, group_start, shared_len, scale, *,
                   max_seq_len: int, max_group_rows: int, out=None, out_dtype=None, num_workers: int = 0,
                   workspace=None, stream=None):
    """Shared-prefix decode (``pa_decode_cascade``).  Returns ``out`` [B, Hq, D]."""
    with _on_stream(stream):
        if out is None:
            out = _alloc_out(q, out_dtype)
        c = make_cascade_args(q, k_pool, v_pool, block_table, seq_lens, group_start, shared_len, scale,
                              max_seq_len=max_seq_len, max_group_rows=max_group_rows, out=out,
                              num_workers=num_workers)
        if workspace is None:
            workspace = _alloc_workspace(cascade_workspace_bytes(c), q.device)
        if workspace is not None:
            c.base.workspace = _ptr(workspace)
            c.base.workspace_bytes = workspace.numel() * workspace.element_size()
        check(LIB.pa_decode_cascade(ctypes.byref(c), ctypes.c_void_p(_stream(stream))))
    return out


def cascade_args_call(c: CascadeArgs, stream=None) -> None:
    check(LIB.pa_decode_cascade(ctypes.byref(c), ctypes.c_void_p(_stream(stream))))


def check_cascade_metadata(block_table, seq_lens, group_start, shared_len, *, max_group_rows: int,
                           num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                           num_blocks: int, max_seq_len: int) -> None:
    """Host-side precondition check (``pa_check_cascade_metadata``) on numpy int32 arrays."""
    import numpy as np
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    gs = np.ascontiguousarray(group_start, dtype=np.int32)
    sh = np.ascontiguousarray(shared_len, dtype=np.int32)
    c = CascadeArgs()
    a = c.base
    a.num_seqs, a.num_q_heads, a.num_kv_heads = len(sl), num_q_heads, num_kv_heads
    a.head_dim, a.block_size, a.num_blocks = head_dim, block_size, num_blocks
    a.max_blocks_per_seq, a.max_seq_len = bt.shape[1], max_seq_len
    a.q_dtype = a.kv_dtype = a.out_dtype = PA_BF16
    a.block_table = bt.ctypes.data
    a.seq_lens = sl.ctypes.data
    c.group_start = gs.ctypes.data
    c.shared_len = sh.ctypes.data
    c.num_groups = len(gs) - 1
    c.max_group_rows = max_group_rows
    check(LIB.pa_check_cascade_metadata(ctypes.byref(c)))


def make_append_args(k, v, slot_mapping, k_pool, v_pool, k_scale=None, v_scale=None) -> AppendArgs:
    a = AppendArgs()
    a.num_tokens = int(k.shape[0])
    a.num_kv_heads = int(k.shape[1])
    a.head_dim = int(k.shape[2])
    a.block_size = int(k_pool.shape[2])
    a.num_blocks = int(k_pool.shape[0])
    a.src_dtype = dtype_code(k)
    a.kv_dtype = dtype_code(k_pool)
    a.k = _ptr(k)
    a.v = _ptr(v)
    a.slot_mapping = _ptr(slot_mapping)
    a.k_pool = _ptr(k_pool)
    a.v_pool = _ptr(v_pool)
    a.k_scale = _ptr(k_scale)
    a.v_scale = _ptr(v_scale)
    return _hold(a, k, v, slot_mapping, k_pool, v_pool, k_scale, v_scale)


def append_decode_args_call(app: AppendArgs, dec: DecodeArgs, stream=None) -> None:
    """``pa_append_decode``: append each decode row's new token, then attend (one launch for short rows)."""
    check(LIB.pa_append_decode(ctypes.byref(app), ctypes.byref(dec), ctypes.c_void_p(_stream(stream))))


def append(k, v, slot_mapping, k_pool, v_pool, k_scale=None, v_scale=None, stream=None) -> None:
    """Write new tokens' K/V into their pool slots in place (``pa_append``)."""
    a = make_append_args(k, v, slot_mapping, k_pool, v_pool, k_scale, v_scale)
    check(LIB.pa_append(ctypes.byref(a), ctypes.c_void_p(_stream(stream))))


def check_append_metadata(slot_mapping, *, num_kv_heads: int, head_dim: int, block_size: int,
                          num_blocks: int, src_dtype: int = PA_BF16, kv_dtype: int = PA_BF16) -> None:
    import numpy as np
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    a = AppendArgs()
    a.num_tokens, a.num_kv_heads, a.head_dim = len(sm), num_kv_heads, head_dim
    a.block_size, a.num_blocks, a.src_dtype, a.kv_dtype = block_size, num_blocks, src_dtype, kv_dtype
    a.slot_mapping = sm.ctypes.data
    check(LIB.pa_check_append_metadata(ctypes.byref(a)))


def stream_read(src, out, num_workgroups: int, loads_in_flight: int = 8, stream=None) -> None:
    """``pa_stream_read``: read every byte of the device tensor ``src`` once (the bandwidth
    probe); ``out`` is a device uint32/int32 tensor of 4 * num_workgroups words."""
    nbytes = src.numel() * src.element_size()
    check(LIB.pa_stream_read(_ptr(src), nbytes, _ptr(out), int(num_workgroups), int(loads_in_flight),
                             ctypes.c_void_p(_stream(stream))))


def gather_read(base, page_offsets, page_bytes: int, out, num_workgroups: int, pages_in_flight: int = 4,
                stream=None) -> None:
    """``pa_gather_read``: read the pages ``base + page_offsets[i]`` (an int64 device tensor of
    byte offsets) of ``page_bytes`` each, in list order (the paged-read bandwidth probe)."""
    check(LIB.pa_gather_read(_ptr(base), _ptr(page_offsets), int(page_offsets.numel()), int(page_bytes),
                             _ptr(out), int(num_workgroups), int(pages_in_flight), ctypes.c_void_p(_stream(stream))))

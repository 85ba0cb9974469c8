"""CPU checks of the C ABI: the library loads, exports every declared call, and
rejects bad arguments with the documented status before anything is launched.
No call in this file reaches a kernel launch."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header=None):
    """Functions declared in include/*.h (or in one header)."""
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in ([header] if header else sorted(os.listdir(inc))):
        if not h.endswith(".h"):
            continue
        src = open(os.path.join(inc, h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def b():
    from paged_kv_attention_13_amd import binding
    return binding


def test_header_declares_the_calls():
    names = _declared_functions("pa.h")
    for n in ["pa_decode", "pa_mixed", "pa_decode_plan", "pa_decode_partials", "pa_merge_partials",
              "pa_check_decode_metadata", "pa_check_mixed_metadata", "pa_mixed_workspace_size",
              "pa_append", "pa_check_append_metadata", "pa_decode_workspace_size", "pa_check_metadata",
              "pa_status_string", "pa_last_error", "pa_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(b):
    for n in _declared_functions():
        assert hasattr(b.LIB, n), n
    out = os.popen(f"nm -D --defined-only {b.LIB_PATH}").read()
    for n in _declared_functions():
        assert re.search(rf"\bT {n}\b", out), f"{n} not exported"


def test_abi_version(b):
    assert b.LIB.pa_abi_version() == 4


def test_struct_layout_matches_header(b):
    # field offsets of the C struct on x86-64 (12 int32, then pointers, float, ...)
    assert b.DecodeArgs.q.offset == 48
    assert b.DecodeArgs.num_workers.offset == 32
    assert b.DecodeArgs.scale.offset == 48 + 7 * 8
    assert ctypes.sizeof(b.DecodeArgs) == 48 + 7 * 8 + 8 + 3 * 8
    assert b.MixedArgs.q_start_loc.offset == ctypes.sizeof(b.DecodeArgs)
    nb = ctypes.sizeof(b.DecodeArgs)
    assert b.MixedArgs.num_verify_rows.offset == nb + 8 + 3 * 4
    assert b.MixedArgs.max_verify_q_len.offset == nb + 8 + 4 * 4
    assert ctypes.sizeof(b.MixedArgs) == nb + 8 + 5 * 4 + 4      # padded to 8 bytes
    assert b.CascadeArgs.group_start.offset == nb
    assert b.CascadeArgs.shared_len.offset == nb + 8
    assert b.CascadeArgs.num_groups.offset == nb + 16
    assert b.CascadeArgs.max_group_rows.offset == nb + 20
    assert ctypes.sizeof(b.CascadeArgs) == nb + 24


def _args(b, **kw):
    a = b.DecodeArgs()
    a.num_seqs, a.num_q_heads, a.num_kv_heads, a.head_dim = 2, 32, 8, 128
    a.block_size, a.num_blocks, a.max_blocks_per_seq, a.max_seq_len = 16, 64, 8, 128
    a.q_dtype = a.kv_dtype = a.out_dtype = b.PA_BF16
    fake = 0x10000
    a.q = a.k_pool = a.v_pool = a.out = a.block_table = a.seq_lens = fake
    a.scale = 0.088
    for k, v in kw.items():
        setattr(a, k, v)
    return a


BAD = [
    (dict(num_q_heads=30), "PA_ERR_BAD_SHAPE"),
    (dict(num_q_heads=24, num_kv_heads=2), "PA_ERR_UNSUPPORTED"),     # group 12
    (dict(head_dim=64), "PA_ERR_UNSUPPORTED"),
    (dict(block_size=24), "PA_ERR_UNSUPPORTED"),
    (dict(block_size=8), "PA_ERR_UNSUPPORTED"),
    (dict(max_seq_len=129), "PA_ERR_BAD_SHAPE"),
    (dict(num_seqs=-1), "PA_ERR_BAD_SHAPE"),
    (dict(q_dtype=0), "PA_ERR_BAD_DTYPE"),
    (dict(out_dtype=2), "PA_ERR_BAD_DTYPE"),
    (dict(kv_dtype=0), "PA_ERR_BAD_DTYPE"),
    (dict(k_scale=0x20000), "PA_ERR_BAD_DTYPE"),
    (dict(kv_dtype=2), "PA_ERR_NULL_POINTER"),                       # fp8 without scales
    (dict(q=None), "PA_ERR_NULL_POINTER"),
    (dict(out=None), "PA_ERR_NULL_POINTER"),
    (dict(q=0x10008), "PA_ERR_MISALIGNED"),
    (dict(k_pool=0x10004), "PA_ERR_MISALIGNED"),
    (dict(num_workers=-1), "PA_ERR_UNSUPPORTED"),
    (dict(num_workers=70000), "PA_ERR_UNSUPPORTED"),
    (dict(max_seq_len=2000, max_blocks_per_seq=128), "PA_ERR_WORKSPACE_TOO_SMALL"),
]


@pytest.mark.parametrize("kw,status", BAD)
@pytest.mark.parametrize("entry", ["pa_decode", "pa_decode_partials", "pa_merge_partials"])
def test_bad_arguments_rejected_before_launch(b, kw, status, entry):
    a = _args(b, **kw)
    rc = getattr(b.LIB, entry)(ctypes.byref(a), None)
    assert b.STATUS_NAMES[rc] == status, (kw, b.LIB.pa_last_error())
    assert b.LIB.pa_last_error().decode().startswith(status)


def test_null_struct(b):
    assert b.STATUS_NAMES[b.LIB.pa_decode(None, None)] == "PA_ERR_NULL_POINTER"
    assert b.STATUS_NAMES[b.LIB.pa_mixed(None, None)] == "PA_ERR_NULL_POINTER"


def test_plan_choices(b):
    # one worker per SIMD at most
    a = _args(b, num_seqs=55, block_size=64, max_blocks_per_seq=128, max_seq_len=8192)
    p = b.plan(a)
    assert p.num_workers == 1024 and p.tile_tokens == 16
    units = 55 * 8
    slots = (units + 1024) * 4
    r256 = lambda x: (x + 255) // 256 * 256
    # (first worker, count) records, then m, l and acc of every partial slot
    assert p.workspace_bytes == r256(2 * units * 4) + 2 * r256(slots * 4) + r256(slots * 512)
    # FP8 KV uses 32-token tiles
    a.kv_dtype = 2
    a.k_scale = a.v_scale = 0x10000
    assert b.plan(a).tile_tokens == 32
    a = _args(b, num_seqs=8, block_size=16, max_blocks_per_seq=128, max_seq_len=2048)
    assert b.plan(a).num_workers == 1024
    a = _args(b, num_seqs=32, block_size=16, max_blocks_per_seq=256, max_seq_len=4096)
    assert b.plan(a).num_workers == 1024
    # FP8 pools: the multi-query kernel, up to two waves per SIMD
    a.kv_dtype = 2
    a.k_scale = a.v_scale = 0x10000
    assert b.plan(a).num_workers == 2048
    # an explicit worker count is honoured
    a = _args(b, num_seqs=55, block_size=64, max_blocks_per_seq=128, max_seq_len=8192, num_workers=7)
    assert b.plan(a).num_workers == 7
    # tiny work with an explicit split: fewer workers, at least a few tiles each
    a = _args(b, num_seqs=1, max_seq_len=2048, max_blocks_per_seq=128)
    p = b.plan(a)
    assert p.num_workers == 8 * (128 + 4) // 4       # each unit's 4 virtual start-up tiles count
    # rows within 1,024 tokens and at most 512 (row, kv head) units: one workgroup per unit
    a = _args(b, num_seqs=64, max_seq_len=300, max_blocks_per_seq=64)
    assert b.plan(a).workspace_bytes == 0
    a = _args(b, num_seqs=65, max_seq_len=300, max_blocks_per_seq=64)
    assert b.plan(a).workspace_bytes > 0
    # many short units (at most 32 tiles each): two waves per SIMD
    assert b.plan(a).num_workers == 2048
    a = _args(b, num_seqs=2048, max_seq_len=128, max_blocks_per_seq=8)
    assert b.plan(a).num_workers == 2048
    a = _args(b, num_seqs=2048, max_seq_len=513, max_blocks_per_seq=33)
    assert b.plan(a).num_workers == 1024
    # short units between one and two waves per SIMD round up to two
    a = _args(b, num_seqs=130, max_seq_len=64, max_blocks_per_seq=4)   # 1,040 units x 8 tiles
    assert b.plan(a).num_workers == 2048
    # rows within 1,024 tokens: one workgroup of 8 waves per (row, kv head), no workspace ...
    a = _args(b, num_seqs=40, max_seq_len=1024, max_blocks_per_seq=64)
    p = b.plan(a)
    assert p.num_workers == 40 * 8 * 8 and p.workspace_bytes == 0
    # ... or, with fewer units than CUs, each unit cut over S = min(CUs / units, tiles / 4, 8)
    # workgroups (24 units: S = 8), whose partials take the split layout with S x units slots
    a = _args(b, num_seqs=3, max_seq_len=1024, max_blocks_per_seq=64)
    p = b.plan(a)
    units, S = 3 * 8, 8
    slots = (units + units * S) * 4
    r256 = lambda x: (x + 255) // 256 * 256
    assert p.num_workers == units * S
    assert p.workspace_bytes == r256(2 * units * 4) + 2 * r256(slots * 4) + r256(slots * 512)
    a = _args(b, num_seqs=1, max_seq_len=48, max_blocks_per_seq=4)      # 3 tiles: one piece per unit
    assert b.plan(a).workspace_bytes == 0
    a = _args(b, num_seqs=3, max_seq_len=1024, max_blocks_per_seq=64)
    a.num_workers = 5                                         # an explicit count keeps the split
    assert b.plan(a).num_workers == 5 and b.plan(a).workspace_bytes > 0
    a.num_workers = 0
    a.kv_dtype, a.k_scale, a.v_scale = 2, 0x10000, 0x10000   # FP8 runs on the multi-query kernel
    assert b.plan(a).workspace_bytes > 0
    # no rows: no workspace
    a = _args(b, num_seqs=0)
    assert b.plan(a).workspace_bytes == 0


def test_mixed_validation(b):
    m = b.MixedArgs()
    m.base = _args(b)
    m.q_start_loc = 0x10000
    m.total_q = 5
    m.num_decode_rows = 3            # > num_seqs = 2
    m.max_q_len = 4
    assert b.STATUS_NAMES[b.LIB.pa_mixed(ctypes.byref(m), None)] == "PA_ERR_BAD_SHAPE"
    m.num_decode_rows = 1
    m.max_q_len = 0
    assert b.STATUS_NAMES[b.LIB.pa_mixed(ctypes.byref(m), None)] == "PA_ERR_BAD_SHAPE"
    m.max_q_len = 4
    # prefill-chunk rows take bf16 q with a bf16 or FP8 cache: FP8 pools pass validation (the
    # call then stops at the missing workspace), fp32 pools are rejected
    m.base.kv_dtype = 2
    m.base.k_scale = m.base.v_scale = 0x10000
    assert b.STATUS_NAMES[b.LIB.pa_mixed(ctypes.byref(m), None)] == "PA_ERR_WORKSPACE_TOO_SMALL"
    m.base.kv_dtype = m.base.q_dtype = m.base.out_dtype = 0
    m.base.k_scale = m.base.v_scale = None
    assert b.STATUS_NAMES[b.LIB.pa_mixed(ctypes.byref(m), None)] == "PA_ERR_UNSUPPORTED"
    m.base.kv_dtype = m.base.q_dtype = m.base.out_dtype = 1
    m.q_start_loc = None
    assert b.STATUS_NAMES[b.LIB.pa_mixed(ctypes.byref(m), None)] == "PA_ERR_NULL_POINTER"


def _mixed_args(b, **kw):
    m = b.MixedArgs()
    m.base = _args(b, num_seqs=4, max_seq_len=128)
    m.q_start_loc = 0x10000
    m.total_q = 12
    m.num_decode_rows = 1
    m.num_verify_rows = 2
    m.max_verify_q_len = 4
    m.max_q_len = 8
    for k, v in kw.items():
        setattr(m, k, v)
    return m


@pytest.mark.parametrize("kw,status", [
    (dict(num_verify_rows=4), "PA_ERR_BAD_SHAPE"),            # 1 decode + 4 verify > 4 rows
    (dict(num_verify_rows=-1), "PA_ERR_BAD_SHAPE"),
    (dict(max_verify_q_len=0), "PA_ERR_UNSUPPORTED"),
    (dict(max_verify_q_len=9), "PA_ERR_UNSUPPORTED"),          # 9 x group 4 > 32 columns
    (dict(total_q=3), "PA_ERR_BAD_SHAPE"),
])
def test_mixed_verify_class_validation(b, kw, status):
    m = _mixed_args(b, **kw)
    assert b.STATUS_NAMES[b.LIB.pa_mixed(ctypes.byref(m), None)] == status


def test_mixed_rows_take_bf16_or_fp8_kv(b):
    m = _mixed_args(b, num_decode_rows=2, num_verify_rows=2)   # no prefill rows
    m.base.kv_dtype = b.PA_FP8_E4M3
    m.base.k_scale = m.base.v_scale = 0x10000
    # accepted (it only lacks a workspace)
    assert b.STATUS_NAMES[b.LIB.pa_mixed(ctypes.byref(m), None)] == "PA_ERR_WORKSPACE_TOO_SMALL"
    n = ctypes.c_size_t()
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n)) == 0 and n.value > 0
    # prefill-chunk rows too
    m.num_verify_rows = 1
    assert b.STATUS_NAMES[b.LIB.pa_mixed(ctypes.byref(m), None)] == "PA_ERR_WORKSPACE_TOO_SMALL"
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n)) == 0 and n.value > 0


def test_mixed_group_bounds_verify_q_len(b):
    # group 8: at most 4 queries per verify row; group 1: up to 32
    m = _mixed_args(b, max_verify_q_len=5)
    m.base.num_q_heads = 64
    assert b.STATUS_NAMES[b.LIB.pa_mixed(ctypes.byref(m), None)] == "PA_ERR_UNSUPPORTED"
    m.max_verify_q_len = 4
    n = ctypes.c_size_t()
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n)) == 0
    m.base.num_q_heads = 8
    m.max_verify_q_len = 32
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n)) == 0
    m.max_verify_q_len = 33
    assert b.STATUS_NAMES[b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n))] == \
        "PA_ERR_UNSUPPORTED"


def test_mixed_workspace_holds_verify_partials(b):
    """Workspace = decode part (rounded to 256 B) + verify records and partial slots."""
    n0, n1 = ctypes.c_size_t(), ctypes.c_size_t()
    m = _mixed_args(b, num_verify_rows=0)
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n0)) == 0
    m = _mixed_args(b)
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n1)) == 0
    r256 = lambda x: (x + 255) // 256 * 256
    units = 2 * 8                                             # verify rows x kv heads
    workers = min(1024, max(1, (units * 4 + 3) // 4))         # max_seq_len 128 = 4 tiles of 32
    slots = (units + workers) * 4 * 4                         # max_verify_q_len 4 x group 4
    vbytes = r256(2 * units * 4) + 2 * r256(slots * 4) + r256(slots * 128 * 4)
    assert n1.value == r256(n0.value) + vbytes
    # an explicit worker count applies to the verify rows too
    m.base.num_workers = 3
    n2 = ctypes.c_size_t()
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n2)) == 0
    m.num_verify_rows = 0
    n3 = ctypes.c_size_t()
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n3)) == 0
    slots = (units + 3) * 16
    assert n2.value == r256(n3.value) + r256(2 * units * 4) + 2 * r256(slots * 4) + r256(slots * 512)


def test_mixed_workspace_holds_prefill_pieces(b):
    """Prefill rows with fewer units than resident workgroups get kv pieces: one slot of
    4 waves x 32 queries x (128 + 2) fp32 per (unit, piece); with many units, none."""
    r256 = lambda x: (x + 255) // 256 * 256
    m = _mixed_args(b, num_verify_rows=0)                     # 1 decode row + 3 prefill rows
    m.base.max_blocks_per_seq, m.base.max_seq_len = 256, 4096
    n = ctypes.c_size_t()
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n)) == 0
    dec = b.plan(_args(b, num_seqs=1, max_blocks_per_seq=256, max_seq_len=4096)).workspace_bytes
    units = 3 * 8 * 1 * 1          # rows x kv heads x head blocks (group 4) x query tiles of 32
    splits = min(8, -(-2 * 512 // units), max(1, (4096 // 64) // 4))
    assert splits == 8
    slots = units * splits
    assert n.value == r256(dec) + r256(slots * 4 * 32 * 128 * 4) + r256(slots * 4 * 32 * 2 * 4)
    m.max_q_len = 4096                                        # 3 x 8 x 128 units > 512
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n)) == 0
    assert n.value == dec
    m.max_q_len = 8
    m.base.max_seq_len = 128                                  # 2 tiles: pieces would be too short
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n)) == 0
    assert n.value == b.plan(_args(b, num_seqs=1, max_blocks_per_seq=256, max_seq_len=128)).workspace_bytes


def test_prefill_alone_workgroup_shape(b):
    """Prefill rows alone take the 8-wave shape (64 query positions per workgroup at group 4,
    128-token kv tiles, one workgroup per CU) when its units fill at least two rounds of its
    256 resident workgroups or at most half a round (then cut into pieces: slots of 8 waves);
    in between, and beside decode rows, the 4-wave shape."""
    r256 = lambda x: (x + 255) // 256 * 256
    m = _mixed_args(b, num_decode_rows=0, num_verify_rows=0, max_verify_q_len=0, total_q=4 * 4096)
    m.base.max_blocks_per_seq, m.base.max_seq_len = 256, 4096
    n = ctypes.c_size_t()
    # 4 rows x 8 kv heads x one 64-position tile = 32 units <= 128: 8 pieces of >= 4 tiles each
    m.max_q_len = 8
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n)) == 0
    slots = 32 * min(8, (2 * 256 + 31) // 32, (4096 // 128) // 4)
    assert n.value == r256(slots * 8 * 32 * 128 * 4) + r256(slots * 8 * 32 * 2 * 4)
    # 4 x 8 x 64 = 2,048 units >= 512: no pieces
    m.max_q_len = 4096
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n)) == 0
    assert n.value == 0
    # 4 x 8 x 8 = 256 units of the 8-wave shape, in neither range: 4-wave shape, 4 x 8 x 16 = 512
    # units on its 512 slots, no pieces
    m.max_q_len = 512
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n)) == 0
    assert n.value == 0
    # the same few units beside a decode row: 4-wave shape, 3 x 8 x 1 = 24 units, pieces of 4 waves
    m.num_decode_rows, m.max_q_len = 1, 8
    assert b.LIB.pa_mixed_workspace_size(ctypes.byref(m), ctypes.byref(n)) == 0
    dec = b.plan(_args(b, num_seqs=1, max_blocks_per_seq=256, max_seq_len=4096)).workspace_bytes
    slots = 24 * min(8, (2 * 512 + 23) // 24, (4096 // 64) // 4)
    assert n.value == r256(dec) + r256(slots * 4 * 32 * 128 * 4) + r256(slots * 4 * 32 * 2 * 4)


def _cascade_args(b, **kw):
    c = b.CascadeArgs()
    c.base = _args(b, num_seqs=4, max_seq_len=128)
    c.group_start = c.shared_len = 0x10000
    c.num_groups = 2
    c.max_group_rows = 3
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("kw,status", [
    (dict(num_groups=0), "PA_ERR_BAD_SHAPE"),
    (dict(num_groups=5), "PA_ERR_BAD_SHAPE"),                 # more groups than rows
    (dict(max_group_rows=0), "PA_ERR_UNSUPPORTED"),
    (dict(max_group_rows=9), "PA_ERR_UNSUPPORTED"),           # 9 rows x group 4 > 32 columns
    (dict(group_start=None), "PA_ERR_NULL_POINTER"),
    (dict(shared_len=None), "PA_ERR_NULL_POINTER"),
    (dict(), "PA_ERR_WORKSPACE_TOO_SMALL"),                   # no workspace
])
def test_cascade_validation(b, kw, status):
    c = _cascade_args(b, **kw)
    assert b.STATUS_NAMES[b.LIB.pa_decode_cascade(ctypes.byref(c), None)] == status


def test_cascade_needs_bf16(b):
    c = _cascade_args(b)
    c.base.kv_dtype = b.PA_FP8_E4M3
    c.base.k_scale = c.base.v_scale = 0x10000
    assert b.STATUS_NAMES[b.LIB.pa_decode_cascade(ctypes.byref(c), None)] == "PA_ERR_UNSUPPORTED"


def test_cascade_workspace_size(b):
    """Decode part (every row's own tokens) then the prefix part, 256-byte aligned."""
    c = _cascade_args(b)
    n = ctypes.c_size_t()
    assert b.LIB.pa_cascade_workspace_size(ctypes.byref(c), ctypes.byref(n)) == 0
    r256 = lambda x: (x + 255) // 256 * 256
    c.base.num_workers = min(b.plan(c.base).num_workers, 1024)   # row parts: one worker per SIMD at most
    dec = b.plan(c.base).workspace_bytes
    c.base.num_workers = 0
    units = 2 * 8
    workers = min(1024, max(1, (units * 4 + 3) // 4))
    slots = (units + workers) * 3 * 4
    assert n.value == r256(dec) + r256(2 * units * 4) + 2 * r256(slots * 4) + r256(slots * 512)


def _cmeta(b, table, lens, gs, shared, max_group_rows=4, **kw):
    args = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=20, max_seq_len=64)
    args.update(kw)
    b.check_cascade_metadata(np.array(table), np.array(lens), np.array(gs), np.array(shared),
                             max_group_rows=max_group_rows, **args)


def test_cascade_metadata_checker(b):
    table = [[0, 1, 2, -1], [0, 1, 3, -1], [4, 5, -1, -1]]
    _cmeta(b, table, [40, 33, 20], [0, 2, 3], [32, 32, 0])
    _cmeta(b, table, [40, 33, 20], [0, 2, 3], [16, 16, 16])            # a shorter shared part is fine
    with pytest.raises(b.PagedAttentionError, match="differs"):
        _cmeta(b, table, [40, 33, 20], [0, 2, 3], [32, 16, 0])
    with pytest.raises(b.PagedAttentionError, match="multiple of block_size"):
        _cmeta(b, table, [40, 33, 20], [0, 2, 3], [24, 24, 0])
    with pytest.raises(b.PagedAttentionError, match="below seq_len"):
        _cmeta(b, table, [40, 32, 20], [0, 2, 3], [32, 32, 0])         # row 1 would have no own token
    with pytest.raises(b.PagedAttentionError, match="shared prefix"):
        _cmeta(b, [[0, 1, 2, 6], [0, 1, 3, 7], [4, 5, -1, -1]], [60, 60, 20], [0, 2, 3],
               [48, 48, 0])                                            # third block differs
    with pytest.raises(b.PagedAttentionError, match="empty"):
        _cmeta(b, table, [40, 33, 20], [0, 2, 2, 3], [32, 32, 0])
    with pytest.raises(b.PagedAttentionError, match="max_group_rows"):
        _cmeta(b, table, [40, 33, 20], [0, 2, 3], [32, 32, 0], max_group_rows=1)
    with pytest.raises(b.PagedAttentionError, match="group_start"):
        _cmeta(b, table, [40, 33, 20], [0, 2, 2], [32, 32, 0])


def test_shared_prefix_inputs_pass_the_checker(b):
    import pa_inputs
    w = pa_inputs.make_shared_prefix_workload(name="t", group_sizes=[3, 1, 2, 8], shared_lens=[32, 0, 48, 64],
                                              own_lens=[1, 5, 17, 3, 16, 40] + [7] * 8, prefix_ids=[0, 1, 0, 2],
                                              seed=1, extra_blocks=2)
    b.check_cascade_metadata(w.block_table, w.seq_lens, w.group_start, w.shared_len, max_group_rows=8,
                             num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                             num_blocks=w.num_blocks, max_seq_len=w.max_seq_len)
    # own blocks belong to one row only; prefix blocks only to rows of groups with that prefix
    owners = {}
    for r in range(w.num_seqs):
        nb = (int(w.seq_lens[r]) + 15) // 16
        for j in range(nb):
            owners.setdefault(int(w.block_table[r, j]), set()).add(r)
    for r in range(w.num_seqs):
        nsh = int(w.shared_len[r]) // 16
        nb = (int(w.seq_lens[r]) + 15) // 16
        for j in range(nsh, nb):
            assert owners[int(w.block_table[r, j])] == {r}
    assert set(w.block_table[0, :2]) == set(w.block_table[4, :2])     # prefix id 0 shared across groups


def _meta(b, table, lens, **kw):
    args = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=10,
                max_seq_len=64)
    args.update(kw)
    b.check_decode_metadata(np.array(table), np.array(lens), **args)


def test_metadata_checker(b):
    _meta(b, [[0, 1, -1, -1], [2, -1, -1, -1]], [20, 16])          # ok: trailing -1 never read
    with pytest.raises(b.PagedAttentionError, match="outside"):
        _meta(b, [[0, -1, -1, -1], [2, -1, -1, -1]], [20, 16])      # needs 2 blocks, second is -1
    with pytest.raises(b.PagedAttentionError, match="outside"):
        _meta(b, [[0, 10, -1, -1]], [20])                           # id == num_blocks
    with pytest.raises(b.PagedAttentionError, match="< 1"):
        _meta(b, [[0, 1, -1, -1]], [0])
    with pytest.raises(b.PagedAttentionError, match="max_seq_len"):
        _meta(b, [[0, 1, 2, 3]], [60], max_seq_len=50)


def test_mixed_metadata_checker(b):
    kw = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=10,
              max_seq_len=64)
    table = np.array([[0, -1, -1, -1], [1, 2, -1, -1], [3, 4, 5, -1]])
    b.check_mixed_metadata(table, [5, 20, 40], [0, 1, 9, 49], num_decode_rows=1, max_q_len=40, **kw)
    with pytest.raises(b.PagedAttentionError, match="decode row"):
        b.check_mixed_metadata(table, [5, 20, 40], [0, 2, 9, 49], num_decode_rows=1, max_q_len=40, **kw)
    with pytest.raises(b.PagedAttentionError, match="q_len"):
        b.check_mixed_metadata(table, [5, 20, 40], [0, 1, 30, 49], num_decode_rows=1, max_q_len=40, **kw)
    with pytest.raises(b.PagedAttentionError, match="max_q_len"):
        b.check_mixed_metadata(table, [5, 20, 40], [0, 1, 9, 49], num_decode_rows=1, max_q_len=30, **kw)
    # row 1 as a verify row (q_len 8)
    b.check_mixed_metadata(table, [5, 20, 40], [0, 1, 9, 49], num_decode_rows=1, max_q_len=40,
                           num_verify_rows=1, max_verify_q_len=8, **kw)
    with pytest.raises(b.PagedAttentionError, match="max_verify_q_len"):
        b.check_mixed_metadata(table, [5, 20, 40], [0, 1, 9, 49], num_decode_rows=1, max_q_len=40,
                               num_verify_rows=1, max_verify_q_len=7, **kw)
    with pytest.raises(b.PagedAttentionError, match="do not fit"):
        b.check_mixed_metadata(table, [5, 20, 40], [0, 1, 9, 49], num_decode_rows=1, max_q_len=40,
                               num_verify_rows=3, max_verify_q_len=8, **kw)


def test_status_strings(b):
    for code, name in b.STATUS_NAMES.items():
        assert b.LIB.pa_status_string(code).decode() == name


def _append_args(b, **kw):
    a = b.AppendArgs()
    a.num_tokens, a.num_kv_heads, a.head_dim, a.block_size, a.num_blocks = 4, 8, 128, 16, 10
    a.src_dtype = a.kv_dtype = b.PA_BF16
    a.k = a.v = a.slot_mapping = a.k_pool = a.v_pool = 0x10000
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(num_tokens=-1), "PA_ERR_BAD_SHAPE"),
    (dict(num_kv_heads=0), "PA_ERR_BAD_SHAPE"),
    (dict(head_dim=64), "PA_ERR_UNSUPPORTED"),
    (dict(block_size=12), "PA_ERR_UNSUPPORTED"),
    (dict(src_dtype=2), "PA_ERR_BAD_DTYPE"),
    (dict(src_dtype=0), "PA_ERR_BAD_DTYPE"),              # f32 -> bf16 not offered
    (dict(kv_dtype=2), "PA_ERR_NULL_POINTER"),            # fp8 without scales
    (dict(k_scale=0x10000), "PA_ERR_BAD_DTYPE"),
    (dict(slot_mapping=None), "PA_ERR_NULL_POINTER"),
    (dict(v_pool=0x10002), "PA_ERR_MISALIGNED"),
])
def test_append_bad_arguments(b, kw, status):
    a = _append_args(b, **kw)
    assert b.STATUS_NAMES[b.LIB.pa_append(ctypes.byref(a), None)] == status, b.LIB.pa_last_error()


def test_append_metadata_checker(b):
    kw = dict(num_kv_heads=8, head_dim=128, block_size=16, num_blocks=4)
    b.check_append_metadata([0, 17, -1, 63], **kw)
    with pytest.raises(b.PagedAttentionError, match="outside"):
        b.check_append_metadata([0, 64], **kw)
    with pytest.raises(b.PagedAttentionError, match="outside"):
        b.check_append_metadata([-2], **kw)
    with pytest.raises(b.PagedAttentionError, match="two tokens"):
        b.check_append_metadata([5, 6, 5], **kw)


def test_append_struct_layout(b):
    assert b.AppendArgs.k.offset == 32
    assert ctypes.sizeof(b.AppendArgs) == 32 + 7 * 8


def test_argument_structs_keep_their_tensors_alive(b):
    """The C structs carry plain addresses: the builders must hold the tensors they point at.

    A temporary passed inline (out=torch.empty(...)) would otherwise be freed at once and its
    memory handed to the next allocation while a kernel still writes there.
    """
    import gc
    import torch
    q = torch.zeros(2, 32, 128, dtype=torch.bfloat16)
    kp = torch.zeros(4, 8, 16, 128, dtype=torch.bfloat16)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    sl = torch.ones(2, dtype=torch.int32)
    qs = torch.tensor([0, 1, 2], dtype=torch.int32)
    structs = [
        b.make_decode_args(q, kp, kp, bt, sl, 0.1, max_seq_len=16, out=torch.empty(2, 32, 128, dtype=torch.bfloat16)),
        b.make_mixed_args(q, kp, kp, bt, sl, qs, 0.1, num_decode_rows=2, max_q_len=1, max_seq_len=16,
                          out=torch.empty(2, 32, 128, dtype=torch.bfloat16)),
        b.make_cascade_args(q, kp, kp, bt, sl, torch.tensor([0, 2], dtype=torch.int32),
                            torch.zeros(2, dtype=torch.int32), 0.1, max_seq_len=16, max_group_rows=2,
                            out=torch.empty(2, 32, 128, dtype=torch.bfloat16)),
    ]
    gc.collect()
    for s in structs:
        out_ptr = s.out if hasattr(s, "out") else s.base.out
        assert any(t.data_ptr() == out_ptr for t in s._keep)
    a = b.make_append_args(torch.zeros(3, 8, 128), torch.zeros(3, 8, 128), torch.zeros(3, dtype=torch.int32),
                           torch.zeros(4, 8, 16, 128), torch.zeros(4, 8, 16, 128))
    gc.collect()
    assert any(t.data_ptr() == a.slot_mapping for t in a._keep)


def _pair(b, **kw):
    """Append args for 4 tokens and decode args for 4 rows over the same pools."""
    app = _append_args(b)
    dec = _args(b, num_seqs=4, num_blocks=10, max_blocks_per_seq=8)
    dec.k_pool = dec.v_pool = app.k_pool
    for k, v in kw.items():
        setattr(app, k, v)
    return app, dec


@pytest.mark.parametrize("kw,status", [
    (dict(num_tokens=3), "PA_ERR_BAD_SHAPE"),                 # one new token per decode row
    (dict(k_pool=0x20000), "PA_ERR_BAD_SHAPE"),               # a different pool
    (dict(block_size=32), "PA_ERR_BAD_SHAPE"),
    (dict(num_blocks=11), "PA_ERR_BAD_SHAPE"),
    (dict(head_dim=64), "PA_ERR_UNSUPPORTED"),                # the append args are validated too
])
def test_append_decode_pair_validation(b, kw, status):
    app, dec = _pair(b, **kw)
    rc = b.LIB.pa_append_decode(ctypes.byref(app), ctypes.byref(dec), None)
    assert b.STATUS_NAMES[rc] == status, b.LIB.pa_last_error()


def test_append_decode_metadata_checker(b):
    """Token b must go to the slot of row b's newest position."""
    import numpy as np
    bs = 16
    table = np.array([[3, 1, -1], [0, 2, 4]], dtype=np.int32)
    lens = np.array([20, 33], dtype=np.int32)
    slots = np.array([1 * bs + 3, 4 * bs + 0], dtype=np.int32)   # positions 19 and 32
    app = b.AppendArgs()
    app.num_tokens, app.num_kv_heads, app.head_dim, app.block_size, app.num_blocks = 2, 8, 128, bs, 5
    app.src_dtype = app.kv_dtype = b.PA_BF16
    app.slot_mapping = slots.ctypes.data
    dec = _args(b, num_seqs=2, num_blocks=5, max_blocks_per_seq=3, max_seq_len=48)
    dec.block_table, dec.seq_lens = table.ctypes.data, lens.ctypes.data
    dec.k_pool = dec.v_pool = app.k_pool = app.v_pool = None
    assert b.LIB.pa_check_append_decode_metadata(ctypes.byref(app), ctypes.byref(dec)) == 0, b.LIB.pa_last_error()
    slots[1] = 4 * bs + 1                                       # one past row 1's newest position
    rc = b.LIB.pa_check_append_decode_metadata(ctypes.byref(app), ctypes.byref(dec))
    assert b.STATUS_NAMES[rc] == "PA_ERR_BAD_METADATA"
    slots[1] = -1                                               # a skipped token is allowed
    assert b.LIB.pa_check_append_decode_metadata(ctypes.byref(app), ctypes.byref(dec)) == 0


def test_decode_workspace_size_is_the_plans(b):
    """pa_decode_workspace_size returns the plan's workspace bytes (0 where no workspace is
    needed) and SIZE_MAX, with the reason in pa_last_error, for invalid arguments."""
    shapes = [dict(num_seqs=55, block_size=64, max_blocks_per_seq=128, max_seq_len=8192),
              dict(num_seqs=32, max_blocks_per_seq=256, max_seq_len=4096),
              dict(num_seqs=40, max_seq_len=1024, max_blocks_per_seq=64),         # one workgroup per unit
              dict(num_seqs=3, max_seq_len=1024, max_blocks_per_seq=64),          # units cut over workgroups
              dict(num_seqs=55, block_size=64, max_blocks_per_seq=128, max_seq_len=8192, num_workers=7),
              dict(num_seqs=0)]
    for kw in shapes:
        a = _args(b, **kw)
        n = b.LIB.pa_decode_workspace_size(ctypes.byref(a))
        assert n == b.plan(a).workspace_bytes, kw
    a = _args(b, num_seqs=40, max_seq_len=1024, max_blocks_per_seq=64)
    assert b.LIB.pa_decode_workspace_size(ctypes.byref(a)) == 0
    a = _args(b, kv_dtype=2, k_scale=0x10000, v_scale=0x10000, num_seqs=128, max_seq_len=8192,
              max_blocks_per_seq=512)
    assert b.LIB.pa_decode_workspace_size(ctypes.byref(a)) == b.plan(a).workspace_bytes > 0
    for kw, status in [(dict(num_q_heads=30), "PA_ERR_BAD_SHAPE"), (dict(head_dim=64), "PA_ERR_UNSUPPORTED")]:
        a = _args(b, **kw)
        assert b.LIB.pa_decode_workspace_size(ctypes.byref(a)) == b.SIZE_MAX
        assert b.LIB.pa_last_error().decode().startswith(status)
        with pytest.raises(b.PagedAttentionError):
            b.decode_workspace_bytes(a)
    assert b.LIB.pa_decode_workspace_size(None) == b.SIZE_MAX


def test_check_metadata_is_the_batch_validator(b):
    """pa_check_metadata validates a whole mixed batch on host copies, like
    pa_check_mixed_metadata, and reports the first violation."""
    table = np.array([[0, -1, -1, -1], [1, 2, -1, -1], [3, 4, 5, -1]], np.int32)
    lens = np.array([5, 20, 40], np.int32)

    def call(qsl, fn, **kw):
        qsl = np.asarray(qsl, np.int32)
        m = b.MixedArgs()
        a = m.base
        a.num_seqs, a.num_q_heads, a.num_kv_heads, a.head_dim = 3, 32, 8, 128
        a.block_size, a.num_blocks, a.max_blocks_per_seq, a.max_seq_len = 16, 10, 4, 64
        a.q_dtype = a.kv_dtype = a.out_dtype = b.PA_BF16
        a.block_table, a.seq_lens = table.ctypes.data, lens.ctypes.data
        m.q_start_loc, m.total_q = qsl.ctypes.data, int(qsl[-1])
        m.num_decode_rows, m.max_q_len = 1, 40
        for k, v in kw.items():
            setattr(m, k, v)
        rc = getattr(b.LIB, fn)(ctypes.byref(m))
        return b.STATUS_NAMES[rc], b.LIB.pa_last_error().decode()

    for fn in ("pa_check_metadata", "pa_check_mixed_metadata"):
        assert call([0, 1, 9, 49], fn)[0] == "PA_OK"
        st, msg = call([0, 2, 9, 49], fn)
        assert st == "PA_ERR_BAD_METADATA" and "decode row" in msg
        st, msg = call([0, 1, 30, 49], fn)
        assert st == "PA_ERR_BAD_METADATA" and "q_len" in msg
        st, msg = call([0, 1, 9, 49], fn, max_q_len=30)
        assert st == "PA_ERR_BAD_METADATA" and "max_q_len" in msg
    bad = table.copy()
    bad[2, 1] = 10                                         # block id == num_blocks
    table[:] = bad
    st, msg = call([0, 1, 9, 49], "pa_check_metadata")
    assert st == "PA_ERR_BAD_METADATA" and "outside" in msg
    assert b.STATUS_NAMES[b.LIB.pa_check_metadata(None)] == "PA_ERR_NULL_POINTER"


@pytest.mark.parametrize("scale", [0.0, -0.088, float("nan"), float("inf")])
def test_scale_must_be_positive_and_finite(b, scale):
    """The launching calls reject a scale that is not finite and > 0 before any launch."""
    a = _args(b, scale=scale)
    for entry in ("pa_decode", "pa_decode_partials", "pa_merge_partials"):
        rc = getattr(b.LIB, entry)(ctypes.byref(a), None)
        assert b.STATUS_NAMES[rc] == "PA_ERR_UNSUPPORTED", entry
        assert "scale" in b.LIB.pa_last_error().decode()
    m = b.MixedArgs()
    m.base = _args(b, scale=scale)
    m.q_start_loc, m.total_q, m.num_decode_rows, m.max_q_len = 0x10000, 2, 2, 1
    assert b.STATUS_NAMES[b.LIB.pa_mixed(ctypes.byref(m), None)] == "PA_ERR_UNSUPPORTED"
    # the plan does not depend on the scale
    assert b.plan(_args(b, scale=scale)).num_workers > 0


def test_allocations_follow_the_launch_stream(b, monkeypatch):
    """With an explicit stream, the output and workspace a call allocates are allocated with
    that stream current (so torch's caching allocator ties them to it), and the launch goes to
    that stream.  Runs on the CPU with a stand-in for torch.cuda and for the library."""
    import types

    import torch
    events = []

    class Stream:
        def __init__(self, h):
            self.cuda_stream = h

    mine, default = Stream(0x1234), Stream(0x99)
    current = [default]

    class StreamCtx:
        def __init__(self, s):
            self.s = s

        def __enter__(self):
            self.prev = current[0]
            current[0] = self.s

        def __exit__(self, *e):
            current[0] = self.prev
            return False

    def empty(*a, **kw):
        kw["device"] = "cpu"
        events.append(("alloc", current[0].cuda_stream))
        return torch.empty(*a, **kw)

    fake = types.SimpleNamespace(float32=torch.float32, bfloat16=torch.bfloat16, uint8=torch.uint8,
                                 float8_e4m3fn=torch.float8_e4m3fn, empty=empty,
                                 cuda=types.SimpleNamespace(stream=StreamCtx, current_stream=lambda: current[0]))

    class Lib:
        def pa_decode_workspace_size(self, a):
            return 4096

        def pa_mixed_workspace_size(self, m, n):
            n._obj.value = 4096
            return 0

        def pa_cascade_workspace_size(self, c, n):
            n._obj.value = 4096
            return 0

        def _launch(self, a, st):
            events.append(("launch", st.value))
            return 0

        pa_decode = pa_mixed = pa_decode_cascade = _launch

    monkeypatch.setattr(b, "_torch", lambda: fake)
    monkeypatch.setattr(b, "LIB", Lib())
    q = torch.zeros((2, 32, 128), dtype=torch.bfloat16)
    kp = torch.zeros((4, 8, 16, 128), dtype=torch.bfloat16)
    bt = torch.zeros((2, 2), dtype=torch.int32)
    sl = torch.ones(2, dtype=torch.int32)
    qsl = torch.arange(3, dtype=torch.int32)
    gs = torch.tensor([0, 2], dtype=torch.int32)
    for call in (lambda st: b.decode(q, kp, kp, bt, sl, 0.1, max_seq_len=16, stream=st),
                 lambda st: b.mixed(q, kp, kp, bt, sl, qsl, 0.1, num_decode_rows=2, max_q_len=1,
                                    max_seq_len=16, stream=st),
                 lambda st: b.decode_cascade(q, kp, kp, bt, sl, gs, sl, 0.1, max_seq_len=16,
                                             max_group_rows=2, stream=st)):
        events.clear()
        call(mine)
        assert events == [("alloc", 0x1234), ("alloc", 0x1234), ("launch", 0x1234)], events
        assert current[0] is default
        events.clear()
        call(None)
        assert events == [("alloc", 0x99), ("alloc", 0x99), ("launch", 0x99)], events


def test_stream_probe_rejects_bad_arguments(b):
    """pa_stream_read (include/pa_probe.h) validates before any launch."""
    f = b.LIB.pa_stream_read
    cases = [((None, 1024, 0x10000, 4, 8), "PA_ERR_NULL_POINTER"),
             ((0x10000, 1024, None, 4, 8), "PA_ERR_NULL_POINTER"),
             ((0x10008, 1024, 0x10000, 4, 8), "PA_ERR_MISALIGNED"),
             ((0x10000, 1000, 0x10000, 4, 8), "PA_ERR_BAD_SHAPE"),
             ((0x10000, 0, 0x10000, 4, 8), "PA_ERR_BAD_SHAPE"),
             ((0x10000, 1024, 0x10000, 0, 8), "PA_ERR_BAD_SHAPE"),
             ((0x10000, 1024, 0x10000, 70000, 8), "PA_ERR_BAD_SHAPE"),
             ((0x10000, 1024, 0x10000, 4, 5), "PA_ERR_UNSUPPORTED")]
    for args, status in cases:
        assert b.STATUS_NAMES[f(*args, None)] == status, args


def test_gather_probe_rejects_bad_arguments(b):
    f = b.LIB.pa_gather_read
    cases = [((None, 0x10000, 4, 2048, 0x10000, 4, 4), "PA_ERR_NULL_POINTER"),
             ((0x10000, None, 4, 2048, 0x10000, 4, 4), "PA_ERR_NULL_POINTER"),
             ((0x10008, 0x10000, 4, 2048, 0x10000, 4, 4), "PA_ERR_MISALIGNED"),
             ((0x10000, 0x10004, 4, 2048, 0x10000, 4, 4), "PA_ERR_MISALIGNED"),
             ((0x10000, 0x10000, 0, 2048, 0x10000, 4, 4), "PA_ERR_BAD_SHAPE"),
             ((0x10000, 0x10000, 4, 1000, 0x10000, 4, 4), "PA_ERR_BAD_SHAPE"),
             ((0x10000, 0x10000, 4, 2048, 0x10000, 0, 4), "PA_ERR_BAD_SHAPE"),
             ((0x10000, 0x10000, 4, 2048, 0x10000, 4, 3), "PA_ERR_UNSUPPORTED")]
    for args, status in cases:
        assert b.STATUS_NAMES[f(*args, None)] == status, args


def test_device_checks_only_in_the_debug_build(b):
    """The library reports its checks off and no flags without touching a device; the debug
    build (PA_DEVICE_CHECKS=1) exports the same calls and reports its checks on."""
    import ctypes as ct
    assert b.LIB.pa_device_checks() == 0
    assert b.device_check_flags() == 0
    assert b.STATUS_NAMES[b.LIB.pa_device_check_flags(None)] == "PA_ERR_NULL_POINTER"
    if os.path.basename(b.LIB_PATH).startswith("libpa_host"):
        return                               # the host-only (sanitizer) build: no HIP library here
    path = os.path.join(os.path.dirname(b.LIB_PATH), "libpa_kv_checked.so")
    assert os.path.exists(path), "build() also builds libpa_kv_checked.so"
    lib = ct.CDLL(path)
    lib.pa_device_checks.restype = ct.c_int
    assert lib.pa_device_checks() == 1
    lib.pa_abi_version.restype = ct.c_int
    assert lib.pa_abi_version() == b.LIB.pa_abi_version()

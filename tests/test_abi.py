"""The C ABI loads, exports what include/qknr.h declares, and rejects bad
arguments on the host before anything is enqueued (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import qk_norm_rope_amd as Q
from qk_norm_rope_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "qknr.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_the_expected_entry_points():
    assert set(_declared_functions()) == set(L.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert Q.status_str(0) == "ok"
    assert "invalid" in Q.status_str(-1)
    assert "workspace" in Q.status_str(-3)


def test_rope_table_matches_oracle_bitwise():
    # the library's host helper and the oracle compute the table independently
    cos, sin = Q.rope_table(1e6, 40960, 128)
    ocos, osin = O.rope_table(1e6, 40960, 128)
    assert np.array_equal(cos, ocos)
    assert np.array_equal(sin, osin)
    for r in (2, 32, 64, 96):   # partial rotary: the table of an r-wide head
        cos, sin = Q.rope_table(1e6, 300, r)
        ocos, osin = O.rope_table(1e6, 300, r)
        assert np.array_equal(cos, ocos) and np.array_equal(sin, osin)


def _pool(**kw):
    p = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, num_pages=16,
             dtype=L.QKR_BF16, reserved=0)
    p.update(kw)
    return L.Pool(**p)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks


def _append(pool, n=1, **kw):
    args = dict(stream=None, n=n, q=FAKE, k=FAKE, v=FAKE, in_dtype=L.QKR_BF16, qg=FAKE, kg=FAKE,
                eps=1e-6, cos=FAKE, sin=FAKE, rope_rows=100, pos=FAKE, slots=FAKE, n_slotted=n,
                table=None, ppr=0, q_out=FAKE, kp=FAKE, vp=FAKE)
    args.update(kw)
    return L.LIB.qknorm_rope_append(args["stream"], ctypes.byref(pool), args["n"], args["q"], args["k"],
                                    args["v"], args["in_dtype"], args["qg"], args["kg"], args["eps"],
                                    args["cos"], args["sin"], args["rope_rows"], args["pos"],
                                    args["slots"], args["n_slotted"], args["table"], args["ppr"],
                                    args["q_out"], args["kp"], args["vp"])


def test_append_host_checks():
    assert _append(_pool(head_dim=64)) == -2
    assert _append(_pool(page_size=32)) == -2
    assert _append(_pool(num_q_heads=30)) == -1          # not a multiple of kv heads
    assert _append(_pool(num_q_heads=16)) == -2          # group of 2 is not built
    assert _append(_pool(reserved=1)) == -1
    assert _append(_pool(), in_dtype=7) == -2
    assert _append(_pool(), q=None) == -1
    assert _append(_pool(), n=-1) == -1
    assert _append(_pool(), n_slotted=2) == -1           # more slotted tokens than tokens
    assert _append(_pool(), n=2, n_slotted=1) == -1      # decode tokens need a table
    assert _append(_pool(), rope_rows=0) == -1
    assert _append(_pool(), eps=float("nan")) == -1
    assert _append(_pool(), n=0, q=None) == 0            # empty batch is a no-op


def test_decode_and_prefill_host_checks():
    pool = _pool()
    lib = L.LIB
    assert lib.paged_decode_attn(None, ctypes.byref(pool), 0, None, None, None, None, 0, None,
                                 0.1, None, None, 0) == 0
    assert lib.paged_decode_attn(None, ctypes.byref(pool), 2, FAKE, FAKE, FAKE, None, 4, FAKE,
                                 0.1, FAKE, FAKE, 1 << 20) == -1
    need = lib.paged_decode_attn_workspace(ctypes.byref(pool), 2, 4)
    assert need > 0
    assert lib.paged_decode_attn(None, ctypes.byref(pool), 2, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                                 0.1, FAKE, FAKE, need - 1) == -3
    assert lib.paged_decode_attn(None, ctypes.byref(pool), 2, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                                 0.1, FAKE, None, need) == -3
    assert lib.paged_decode_attn(None, ctypes.byref(pool), 2, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                                 float("inf"), FAKE, FAKE, need) == -1
    pneed = lib.paged_prefill_attn_workspace(ctypes.byref(pool), 100)
    assert pneed >= 2 * 4
    assert lib.paged_prefill_attn(None, ctypes.byref(pool), 100, FAKE, FAKE, FAKE, FAKE, 3, 4, None,
                                  FAKE, 0.1, FAKE, FAKE, pneed) == -1
    assert lib.paged_prefill_attn(None, ctypes.byref(pool), 100, FAKE, FAKE, FAKE, FAKE, 3, 4, FAKE,
                                  FAKE, 0.1, FAKE, FAKE, pneed - 1) == -3
    assert lib.paged_prefill_attn(None, ctypes.byref(_pool(head_dim=256)), 100, FAKE, FAKE, FAKE,
                                  FAKE, 3, 4, FAKE, FAKE, 0.1, FAKE, FAKE, pneed) == -2


def _append_ex(pool, opts, **kw):
    args = dict(stream=None, n=1, q=FAKE, k=FAKE, v=FAKE, in_dtype=L.QKR_BF16, qg=FAKE, kg=FAKE,
                eps=1e-6, cos=FAKE, sin=FAKE, rope_rows=100, pos=FAKE, slots=FAKE, n_slotted=1,
                table=None, ppr=0, q_out=FAKE, kp=FAKE, vp=FAKE)
    args.update(kw)
    return L.LIB.qknorm_rope_append_ex(args["stream"], ctypes.byref(pool), args["n"], args["q"], args["k"],
                                       args["v"], args["in_dtype"], args["qg"], args["kg"], args["eps"],
                                       args["cos"], args["sin"], args["rope_rows"], args["pos"],
                                       args["slots"], args["n_slotted"], args["table"], args["ppr"],
                                       args["q_out"], args["kp"], args["vp"],
                                       ctypes.byref(opts) if opts is not None else None)


def test_append_options_host_checks():
    n0 = dict(n=0, n_slotted=0)   # valid options on an empty batch: no-op
    assert _append_ex(_pool(), None, **n0) == 0
    assert _append_ex(_pool(), L.AppendOpts(1, 64), **n0) == 0
    assert _append_ex(_pool(), L.AppendOpts(2, 0)) == -1            # qk_norm_whole is 0 or 1
    for bad in (1, 3, 130, -2):                                      # odd, too wide, negative
        assert _append_ex(_pool(), L.AppendOpts(0, bad)) == -1
    o = L.AppendOpts(0, 0)
    o.reserved[2] = 1
    assert _append_ex(_pool(), o) == -1
    assert _append_ex(_pool(num_q_heads=256, num_kv_heads=64), L.AppendOpts(1, 0)) == -2


def test_attention_options_host_checks():
    pool = _pool()
    lib = L.LIB
    o = L.AttnOpts(None)
    o.reserved[0] = 5
    need = lib.paged_decode_attn_workspace(ctypes.byref(pool), 2, 4)
    assert lib.paged_decode_attn_ex(None, ctypes.byref(pool), 2, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                                    0.1, FAKE, FAKE, need, ctypes.byref(o)) == -1
    assert lib.paged_prefill_attn_ex(None, ctypes.byref(pool), 100, FAKE, FAKE, FAKE, FAKE, 3, 4, FAKE,
                                     FAKE, 0.1, FAKE, FAKE, 1 << 20, ctypes.byref(o)) == -1
    assert lib.packed_prefill_attn_ex(None, ctypes.byref(pool), 100, FAKE, FAKE, FAKE, FAKE, 3, 4, FAKE,
                                      FAKE, FAKE, 0.1, FAKE, FAKE, 1 << 20, ctypes.byref(o)) == -1
    # the packed form needs segments, and its workspace also holds first positions
    assert lib.packed_prefill_attn(None, ctypes.byref(pool), 100, FAKE, FAKE, FAKE, FAKE, 3, 4, FAKE,
                                   FAKE, None, 0.1, FAKE, FAKE, 1 << 20) == -1
    assert lib.packed_prefill_attn_workspace(ctypes.byref(pool), 100) > \
        lib.paged_prefill_attn_workspace(ctypes.byref(pool), 100)
    assert lib.packed_prefill_attn_workspace(ctypes.byref(_pool(dtype=L.QKR_F32)), 100) >= 400


def test_workspace_sizes_grow_with_work():
    pool = _pool()
    a = L.LIB.paged_decode_attn_workspace(ctypes.byref(pool), 8, 65)
    b = L.LIB.paged_decode_attn_workspace(ctypes.byref(pool), 64, 640)
    assert 0 < a < b
    assert L.LIB.paged_decode_attn_workspace(ctypes.byref(_pool(dtype=L.QKR_F32)), 8, 65) == 0
    assert L.LIB.paged_prefill_attn_workspace(ctypes.byref(pool), 4096) >= 64 * 4


def test_decode_kernel_name_host_cases():
    # a float32 pool and invalid sizes need no device; the bfloat16 choice is checked on the GPU
    assert L.LIB.paged_decode_attn_kernel(ctypes.byref(_pool(dtype=L.QKR_F32)), 8, 65) == b"attention_generic_kernel"
    assert L.LIB.paged_decode_attn_kernel(ctypes.byref(_pool()), 0, 65) == b""
    assert L.LIB.paged_decode_attn_kernel(ctypes.byref(_pool()), 8, 0) == b""
    assert L.LIB.paged_decode_attn_kernel(None, 8, 65) == b""


def test_read_probe_host_checks():
    lib = L.LIB
    assert lib.qkr_read_probe(None, None, 16, ctypes.c_void_p(0x1000)) == -1            # null buffer
    assert lib.qkr_read_probe(None, ctypes.c_void_p(0x1008), 16, ctypes.c_void_p(0x1000)) == -1   # misaligned
    assert lib.qkr_read_probe(None, ctypes.c_void_p(0x1000), 15, ctypes.c_void_p(0x1000)) == -1   # size
    assert lib.qkr_read_probe(None, ctypes.c_void_p(0x1000), 16, None) == -1            # null out
    assert lib.qkr_read_probe(None, ctypes.c_void_p(0x1000), 0, ctypes.c_void_p(0x1000)) == 0     # nothing to read


def test_mfma_probe_host_checks():
    lib = L.LIB
    flops = ctypes.c_int64(0)
    assert lib.qkr_mfma_probe(None, 10, None, ctypes.byref(flops)) == -1             # null out
    assert lib.qkr_mfma_probe(None, 10, ctypes.c_void_p(0x1000), None) == -1        # null flops
    assert lib.qkr_mfma_probe(None, -1, ctypes.c_void_p(0x1000), ctypes.byref(flops)) == -1   # negative count


def test_rope_table_rejects_bad_arguments():
    buf = np.zeros(4, np.float32)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    assert L.LIB.qkr_rope_table(1e6, 1, 3, p, p) == -1
    assert L.LIB.qkr_rope_table(-1.0, 1, 8, p, p) == -1
    assert L.LIB.qkr_rope_table(1e6, 1, 8, None, p) == -1


def _step(pool, **kw):
    args = dict(P=100, R=2, q=FAKE, k=FAKE, v=FAKE, in_dtype=L.QKR_BF16, qg=FAKE, kg=FAKE, eps=1e-6,
                cos=FAKE, sin=FAKE, rope_rows=100, pos=FAKE, rows=FAKE, slots=FAKE, spos=FAKE, table=FAKE,
                n_table_rows=4, ppr=4, row0=2, scale=0.1, q_out=FAKE, kp=FAKE, vp=FAKE, pout=FAKE, dout=FAKE,
                ws=FAKE, ws_bytes=1 << 24)
    args.update(kw)
    a = args
    return L.LIB.step_paged(None, ctypes.byref(pool), a["P"], a["R"], a["q"], a["k"], a["v"], a["in_dtype"],
                            a["qg"], a["kg"], a["eps"], a["cos"], a["sin"], a["rope_rows"], a["pos"],
                            a["rows"], a["slots"], a["spos"], a["table"], a["n_table_rows"], a["ppr"],
                            a["row0"], a["scale"], a["q_out"], a["kp"], a["vp"], a["pout"], a["dout"],
                            a["ws"], a["ws_bytes"])


def test_step_host_checks():
    pool = _pool()
    assert _step(pool, P=0, R=0) == 0                                   # empty step: no-op
    assert _step(_pool(dtype=L.QKR_F32)) == -2                          # bfloat16 pools only
    assert _step(pool, in_dtype=L.QKR_F32) == -2                        # bfloat16 inputs only
    assert _step(pool, P=-1) == -1
    assert _step(pool, table=None) == -1
    assert _step(pool, rows=None) == -1                                 # prompt tokens need rows
    assert _step(pool, spos=None) == -1                                 # decode rows need positions
    assert _step(pool, row0=3) == -1                                    # rows 3..4 of a 4-row table
    assert _step(pool, row0=-1) == -1
    assert _step(pool, scale=float("nan")) == -1
    assert _step(pool, R=8193, n_table_rows=9000, row0=0) == -2        # decode rows per step
    assert _step(pool, ppr=4096) == -2                                  # pages per row
    need = L.LIB.step_paged_workspace(ctypes.byref(pool), 100, 2, 4)
    assert need >= 64 * 4 + L.LIB.paged_decode_attn_workspace(ctypes.byref(pool), 2, 4)
    assert _step(pool, ws_bytes=need - 1) == -3
    assert _step(pool, ws=None, ws_bytes=need) == -3
    assert L.LIB.step_paged_workspace(ctypes.byref(_pool(dtype=L.QKR_F32)), 100, 2, 4) == 0
    assert L.LIB.step_paged_workspace(ctypes.byref(pool), 100, 0, 4) < need


def test_size_limits_host_checks():
    pool = _pool()
    lib = L.LIB
    need = lib.paged_decode_attn_workspace(ctypes.byref(pool), 12289, 4)
    assert lib.paged_decode_attn(None, ctypes.byref(pool), 12289, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                                 0.1, FAKE, FAKE, need) == -2          # more rows than one call takes
    # rows x KV heads x (5 x pages per row + 12) must stay below 2^31 (the decode
    # split's cost scale): 12288 rows of 8 KV heads take 4366 pages per row, not 4367
    need = lib.paged_decode_attn_workspace(ctypes.byref(pool), 12288, 4367)
    assert lib.paged_decode_attn(None, ctypes.byref(pool), 12288, FAKE, FAKE, FAKE, FAKE, 4367, FAKE,
                                 0.1, FAKE, FAKE, need) == -2
    assert lib.paged_decode_attn_noalloc(None, ctypes.byref(pool), 12288, FAKE, FAKE, FAKE, FAKE, 4367, FAKE,
                                         0.1, FAKE) == -2
    pneed = lib.paged_prefill_attn_workspace(ctypes.byref(pool), 100)
    assert lib.paged_prefill_attn(None, ctypes.byref(pool), 100, FAKE, FAKE, FAKE, FAKE, 3, 2049, FAKE,
                                  FAKE, 0.1, FAKE, FAKE, pneed) == -2   # longer page table than prefill takes


def test_noalloc_decode_host_checks():
    # the allocation-free decode takes no workspace; its checks run before any
    # device call, including the limit of its library-owned scratch
    pool = _pool()
    lib = L.LIB
    assert lib.paged_decode_attn_noalloc(None, ctypes.byref(pool), 0, None, None, None, None, 0, None,
                                         0.1, None) == 0
    assert lib.paged_decode_attn_noalloc(None, ctypes.byref(pool), -1, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                                         0.1, FAKE) == -1
    assert lib.paged_decode_attn_noalloc(None, ctypes.byref(pool), 2, FAKE, FAKE, FAKE, None, 4, FAKE,
                                         0.1, FAKE) == -1
    assert lib.paged_decode_attn_noalloc(None, ctypes.byref(pool), 2, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                                         float("nan"), FAKE) == -1
    assert lib.paged_decode_attn_noalloc(None, ctypes.byref(_pool(head_dim=64)), 2, FAKE, FAKE, FAKE, FAKE,
                                         4, FAKE, 0.1, FAKE) == -2
    # 8 KV heads: the scratch holds exactly the kernel's 12288 rows
    rows = L.NOALLOC_MAX_ROW_HEADS // 8 + 1
    assert lib.paged_decode_attn_noalloc(None, ctypes.byref(pool), rows, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                                         0.1, FAKE) == -2
    # 16 KV heads: half the rows reach the scratch limit
    p16 = _pool(num_q_heads=64, num_kv_heads=16)
    assert lib.paged_decode_attn_noalloc(None, ctypes.byref(p16), L.NOALLOC_MAX_ROW_HEADS // 16 + 1, FAKE,
                                         FAKE, FAKE, FAKE, 4, FAKE, 0.1, FAKE) == -2
    assert "scratch" in L.last_error()
    # fewer KV heads: the kernel's own row limit still holds
    p4 = _pool(num_q_heads=16, num_kv_heads=4)
    assert lib.paged_decode_attn_noalloc(None, ctypes.byref(p4), 12289, FAKE, FAKE, FAKE, FAKE, 4, FAKE,
                                         0.1, FAKE) == -2


def _check(pool, **kw):
    a = dict(table=FAKE, n_table_rows=4, ppr=8, n=3, rows=FAKE, pos=FAKE, slots=FAKE, r=2, spos=FAKE,
             row0=2, rope_rows=100, counts=FAKE, wait=0)
    a.update(kw)
    return L.LIB.qkr_check_indices(None, ctypes.byref(pool), a["table"], a["n_table_rows"], a["ppr"], a["n"],
                                   a["rows"], a["pos"], a["slots"], a["r"], a["spos"], a["row0"],
                                   a["rope_rows"], a["counts"], a["wait"])


def test_check_indices_host_checks():
    pool = _pool()
    assert _check(pool, counts=None) == -1
    assert _check(pool, table=None) == -1
    assert _check(pool, rows=None) == -1               # prompt tokens need rows and positions
    assert _check(pool, spos=None) == -1               # decode rows need positions
    assert _check(pool, row0=3) == -1                  # decode rows 3..4 of a 4-row table
    assert _check(pool, n=-1) == -1
    assert _check(pool, rope_rows=-1) == -1
    assert _check(_pool(head_dim=64)) == -2
    assert Q.status_str(L.QKR_EDATA) == "device data out of range"

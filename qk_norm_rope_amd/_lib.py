"""ctypes binding of libqknr (include/qknr.h). Argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks dtype,
shape and contiguity, and passes raw pointers and the current HIP stream to the
C ABI. All computation happens in the library's kernels; if the library is not
built the import fails loudly.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqknr.so")

QKR_F32 = 0
QKR_BF16 = 1
HEAD_DIM = 128
PAGE_SIZE = 64
NOALLOC_MAX_ROW_HEADS = 98304   # QKR_NOALLOC_MAX_ROW_HEADS: rows x KV heads of paged_decode_attn_noalloc
QKR_EDATA = -5
CHECK_NAMES = ("row", "position", "page", "slot_range", "slot_mismatch")   # QKR_CHECK_* order
CHECK_COUNTS = 8

EXPORTED = (
    "qknorm_rope_append",
    "qknorm_rope_append_ex",
    "paged_decode_attn",
    "paged_decode_attn_ex",
    "paged_decode_attn_workspace",
    "paged_decode_attn_kernel",
    "paged_decode_attn_noalloc",
    "paged_prefill_attn",
    "paged_prefill_attn_ex",
    "paged_prefill_attn_workspace",
    "packed_prefill_attn",
    "packed_prefill_attn_ex",
    "packed_prefill_attn_workspace",
    "step_paged",
    "step_paged_workspace",
    "qkr_check_indices",
    "qkr_read_probe",
    "qkr_mfma_probe",
    "qkr_rope_table",
    "qkr_status_str",
    "qkr_last_error",
    "qkr_version",
)


class Pool(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class AppendOpts(ctypes.Structure):
    _fields_ = [
        ("qk_norm_whole", ctypes.c_int32),
        ("rotary_dim", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 6),
    ]


class AttnOpts(ctypes.Structure):
    _fields_ = [
        ("gate", ctypes.c_void_p),
        ("reserved", ctypes.c_int32 * 6),
    ]


class QknrError(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = LIB.qkr_last_error().decode() if status in (-2, -4) else ""
        super().__init__(f"{where}: {status_str(status)} ({status}){': ' + detail if detail else ''}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m qk_norm_rope_amd.build`")
    # PyTorch ships its own HIP runtime (soname libamdhip64.so.7). Loading torch
    # first makes the library's libamdhip64.so.7 dependency resolve to that same
    # runtime, so torch's streams and allocations are valid in the library's
    # calls; two HIP runtimes in one process do not share devices.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    pool_p = ctypes.POINTER(Pool)
    app_p = ctypes.POINTER(AppendOpts)
    att_p = ctypes.POINTER(AttnOpts)
    lib.qknorm_rope_append_ex.restype = ctypes.c_int
    lib.qknorm_rope_append_ex.argtypes = [vp, pool_p, i32, vp, vp, vp, i32, vp, vp, f32, vp, vp, i32,
                                          vp, vp, i32, vp, i32, vp, vp, vp, app_p]
    lib.paged_decode_attn_ex.restype = ctypes.c_int
    lib.paged_decode_attn_ex.argtypes = [vp, pool_p, i32, vp, vp, vp, vp, i32, vp, f32, vp, vp, sz, att_p]
    lib.paged_prefill_attn_ex.restype = ctypes.c_int
    lib.paged_prefill_attn_ex.argtypes = [vp, pool_p, i32, vp, vp, vp, vp, i32, i32, vp, vp, f32, vp, vp, sz,
                                          att_p]
    lib.packed_prefill_attn_ex.restype = ctypes.c_int
    lib.packed_prefill_attn_ex.argtypes = [vp, pool_p, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp, f32, vp, vp,
                                           sz, att_p]
    lib.qknorm_rope_append.restype = ctypes.c_int
    lib.qknorm_rope_append.argtypes = [vp, pool_p, i32, vp, vp, vp, i32, vp, vp, f32, vp, vp, i32,
                                       vp, vp, i32, vp, i32, vp, vp, vp]
    lib.paged_decode_attn.restype = ctypes.c_int
    lib.paged_decode_attn.argtypes = [vp, pool_p, i32, vp, vp, vp, vp, i32, vp, f32, vp, vp, sz]
    lib.paged_decode_attn_noalloc.restype = ctypes.c_int
    lib.paged_decode_attn_noalloc.argtypes = [vp, pool_p, i32, vp, vp, vp, vp, i32, vp, f32, vp]
    lib.paged_decode_attn_workspace.restype = sz
    lib.paged_decode_attn_workspace.argtypes = [pool_p, i32, i32]
    lib.paged_decode_attn_kernel.restype = ctypes.c_char_p
    lib.paged_decode_attn_kernel.argtypes = [pool_p, i32, i32]
    lib.paged_prefill_attn.restype = ctypes.c_int
    lib.paged_prefill_attn.argtypes = [vp, pool_p, i32, vp, vp, vp, vp, i32, i32, vp, vp, f32, vp, vp, sz]
    lib.paged_prefill_attn_workspace.restype = sz
    lib.paged_prefill_attn_workspace.argtypes = [pool_p, i32]
    lib.packed_prefill_attn.restype = ctypes.c_int
    lib.packed_prefill_attn.argtypes = [vp, pool_p, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp, f32, vp, vp, sz]
    lib.packed_prefill_attn_workspace.restype = sz
    lib.packed_prefill_attn_workspace.argtypes = [pool_p, i32]
    lib.step_paged.restype = ctypes.c_int
    lib.step_paged.argtypes = [vp, pool_p, i32, i32, vp, vp, vp, i32, vp, vp, f32, vp, vp, i32,
                               vp, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp, sz]
    lib.step_paged_workspace.restype = sz
    lib.step_paged_workspace.argtypes = [pool_p, i32, i32, i32]
    lib.qkr_check_indices.restype = ctypes.c_int
    lib.qkr_check_indices.argtypes = [vp, pool_p, vp, i32, i32, i32, vp, vp, vp, i32, vp, i32, i32, vp, i32]
    lib.qkr_rope_table.restype = ctypes.c_int
    lib.qkr_rope_table.argtypes = [ctypes.c_double, i32, i32, vp, vp]
    lib.qkr_status_str.restype = ctypes.c_char_p
    lib.qkr_status_str.argtypes = [ctypes.c_int]
    lib.qkr_last_error.restype = ctypes.c_char_p
    lib.qkr_last_error.argtypes = []
    lib.qkr_mfma_probe.restype = ctypes.c_int
    lib.qkr_mfma_probe.argtypes = [vp, i32, vp, ctypes.POINTER(ctypes.c_int64)]
    lib.qkr_read_probe.restype = ctypes.c_int
    lib.qkr_read_probe.argtypes = [vp, vp, sz, vp]
    lib.qkr_version.restype = ctypes.c_int
    lib.qkr_version.argtypes = []
    return lib


LIB = _load()


def status_str(status: int) -> str:
    return LIB.qkr_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise QknrError(status, where)


# ------------------------------------------------------------------ helpers

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return QKR_BF16
    if t.dtype == torch.float32:
        return QKR_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t, name, dtype=None, numel=None):
    """Device pointer of a contiguous CUDA/HIP tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def pool_desc(k_pool, num_q_heads: int) -> Pool:
    """Pool descriptor for pools shaped [num_kv_heads, num_pages*64, 128]."""
    if k_pool.dim() != 3 or k_pool.shape[1] % PAGE_SIZE != 0:
        raise ValueError("pools must be [num_kv_heads, num_pages*64, head_dim]")
    return Pool(num_q_heads, k_pool.shape[0], k_pool.shape[2], PAGE_SIZE,
                k_pool.shape[1] // PAGE_SIZE, _dtype_code(k_pool), 0)


# -------------------------------------------------------------- the C ABI

def rope_table(theta: float, rope_rows: int, head_dim: int = HEAD_DIM):
    """qkr_rope_table: float32 numpy (cos, sin), each [rope_rows, head_dim/2]."""
    import numpy as np
    cos = np.empty((rope_rows, head_dim // 2), dtype=np.float32)
    sin = np.empty((rope_rows, head_dim // 2), dtype=np.float32)
    _check(LIB.qkr_rope_table(float(theta), int(rope_rows), int(head_dim),
                              cos.ctypes.data_as(ctypes.c_void_p), sin.ctypes.data_as(ctypes.c_void_p)),
           "qkr_rope_table")
    return cos, sin


def qknorm_rope_append(q, k, v, q_gain, k_gain, rope_cos, rope_sin, positions, q_out, k_pool,
                       v_pool, slots=None, table=None, eps: float = 1e-6, stream=None,
                       qk_norm_whole: bool = False, rotary_dim: int = 0) -> None:
    """QK-norm + RoPE of every token of q/k; q_out <- rotated q; k/v written into the pools.

    The first ``len(slots)`` tokens write at ``slots``; the rest are decode rows
    whose slot comes from ``table`` (row b = token index - len(slots)).
    ``qk_norm_whole`` / ``rotary_dim`` select qknorm_rope_append_ex's variants
    (gains of width heads*head_dim; rope tables of width rotary_dim/2).
    """
    import torch
    n = int(positions.numel())
    n_q = q_out.shape[-1] // HEAD_DIM if q_out.dim() == 2 else 0
    pool = pool_desc(k_pool, n_q)
    n_slotted = 0 if slots is None else int(slots.numel())
    ppr = 0 if table is None else int(table.shape[-1])
    in_dt = _dtype_code(q)
    gq = HEAD_DIM * (n_q if qk_norm_whole else 1)
    gk = HEAD_DIM * (pool.num_kv_heads if qk_norm_whole else 1)
    rd = int(rotary_dim) or HEAD_DIM
    opts = AppendOpts(1 if qk_norm_whole else 0, int(rotary_dim))
    st = LIB.qknorm_rope_append_ex(
        _stream(stream), ctypes.byref(pool), n,
        _ptr(q, "q", q.dtype, n * n_q * HEAD_DIM), _ptr(k, "k", q.dtype, n * pool.num_kv_heads * HEAD_DIM),
        _ptr(v, "v", q.dtype, n * pool.num_kv_heads * HEAD_DIM), in_dt,
        _ptr(q_gain, "q_gain", torch.float32, gq), _ptr(k_gain, "k_gain", torch.float32, gk),
        float(eps), _ptr(rope_cos, "rope_cos", torch.float32), _ptr(rope_sin, "rope_sin", torch.float32),
        int(rope_cos.numel() // (rd // 2)), _ptr(positions, "positions", torch.int32),
        _ptr(slots, "slots", torch.int32), n_slotted,
        _ptr(table, "table", torch.int32, (n - n_slotted) * ppr), ppr,
        _ptr(q_out, "q_out", k_pool.dtype, n * n_q * HEAD_DIM), _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool", k_pool.dtype),
        ctypes.byref(opts))
    _check(st, "qknorm_rope_append")


def decode_workspace_bytes(k_pool, num_q_heads: int, n_rows: int, pages_per_row: int) -> int:
    pool = pool_desc(k_pool, num_q_heads)
    return int(LIB.paged_decode_attn_workspace(ctypes.byref(pool), int(n_rows), int(pages_per_row)))


def decode_kernel_name(k_pool, num_q_heads: int, n_rows: int, pages_per_row: int) -> str:
    """The kernel paged_decode_attn launches for this batch on the current device."""
    pool = pool_desc(k_pool, num_q_heads)
    return LIB.paged_decode_attn_kernel(ctypes.byref(pool), int(n_rows), int(pages_per_row)).decode()


def prefill_workspace_bytes(k_pool, num_q_heads: int, n_tokens: int) -> int:
    pool = pool_desc(k_pool, num_q_heads)
    return int(LIB.paged_prefill_attn_workspace(ctypes.byref(pool), int(n_tokens)))


def _attn_opts(gate, dtype, n):
    return AttnOpts(_ptr(gate, "gate", dtype, n))


def paged_decode_attn(q, k_pool, v_pool, table, positions, scale: float, out, workspace=None,
                      stream=None, gate=None) -> None:
    """out[b] <- attention of row b's query over positions 0..positions[b] of table[b]
    (times sigmoid(gate) when a gate is given)."""
    import torch
    n_q = q.shape[-1] // HEAD_DIM
    pool = pool_desc(k_pool, n_q)
    n_rows = int(positions.numel())
    ppr = int(table.shape[-1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    opts = _attn_opts(gate, k_pool.dtype, n_rows * n_q * HEAD_DIM)
    st = LIB.paged_decode_attn_ex(
        _stream(stream), ctypes.byref(pool), n_rows, _ptr(q, "q", k_pool.dtype, n_rows * n_q * HEAD_DIM),
        _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool", k_pool.dtype),
        _ptr(table, "table", torch.int32, n_rows * ppr), ppr, _ptr(positions, "positions", torch.int32),
        float(scale), _ptr(out, "out", torch.float32, n_rows * n_q * HEAD_DIM),
        _ptr(workspace, "workspace"), ws_bytes, ctypes.byref(opts))
    _check(st, "paged_decode_attn")


def paged_decode_attn_noalloc(q, k_pool, v_pool, table, positions, scale: float, out, stream=None) -> None:
    """paged_decode_attn on the library's own per-GPU scratch: no workspace, no
    allocation; calls that overlap on one GPU race (order them on one stream)."""
    import torch
    n_q = q.shape[-1] // HEAD_DIM
    pool = pool_desc(k_pool, n_q)
    n_rows = int(positions.numel())
    ppr = int(table.shape[-1])
    st = LIB.paged_decode_attn_noalloc(
        _stream(stream), ctypes.byref(pool), n_rows, _ptr(q, "q", k_pool.dtype, n_rows * n_q * HEAD_DIM),
        _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool", k_pool.dtype),
        _ptr(table, "table", torch.int32, n_rows * ppr), ppr, _ptr(positions, "positions", torch.int32),
        float(scale), _ptr(out, "out", torch.float32, n_rows * n_q * HEAD_DIM))
    _check(st, "paged_decode_attn_noalloc")


def paged_prefill_attn(q, k_pool, v_pool, table, rows, positions, scale: float, out, workspace=None,
                       stream=None, gate=None) -> None:
    """out[p] <- attention of token p over positions 0..positions[p] of table[rows[p]]
    (times sigmoid(gate) when a gate is given)."""
    import torch
    n_q = q.shape[-1] // HEAD_DIM
    pool = pool_desc(k_pool, n_q)
    n = int(positions.numel())
    ppr = int(table.shape[-1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    opts = _attn_opts(gate, k_pool.dtype, n * n_q * HEAD_DIM)
    st = LIB.paged_prefill_attn_ex(
        _stream(stream), ctypes.byref(pool), n, _ptr(q, "q", k_pool.dtype, n * n_q * HEAD_DIM),
        _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool", k_pool.dtype),
        _ptr(table, "table", torch.int32), int(table.shape[0]), ppr,
        _ptr(rows, "rows", torch.int32, n), _ptr(positions, "positions", torch.int32, n),
        float(scale), _ptr(out, "out", torch.float32, n * n_q * HEAD_DIM),
        _ptr(workspace, "workspace"), ws_bytes, ctypes.byref(opts))
    _check(st, "paged_prefill_attn")


def packed_workspace_bytes(k_pool, num_q_heads: int, n_tokens: int) -> int:
    pool = pool_desc(k_pool, num_q_heads)
    return int(LIB.packed_prefill_attn_workspace(ctypes.byref(pool), int(n_tokens)))


def packed_prefill_attn(q, k_pool, v_pool, table, rows, positions, segments, scale: float, out,
                        workspace=None, stream=None, gate=None) -> None:
    """out[p] <- attention of token p over the tokens of its own prompt (segment) up to its position."""
    import torch
    n_q = q.shape[-1] // HEAD_DIM
    pool = pool_desc(k_pool, n_q)
    n = int(positions.numel())
    ppr = int(table.shape[-1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    opts = _attn_opts(gate, k_pool.dtype, n * n_q * HEAD_DIM)
    st = LIB.packed_prefill_attn_ex(
        _stream(stream), ctypes.byref(pool), n, _ptr(q, "q", k_pool.dtype, n * n_q * HEAD_DIM),
        _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool", k_pool.dtype),
        _ptr(table, "table", torch.int32), int(table.shape[0]), ppr,
        _ptr(rows, "rows", torch.int32, n), _ptr(positions, "positions", torch.int32, n),
        _ptr(segments, "segments", torch.int32, n),
        float(scale), _ptr(out, "out", torch.float32, n * n_q * HEAD_DIM),
        _ptr(workspace, "workspace"), ws_bytes, ctypes.byref(opts))
    _check(st, "packed_prefill_attn")


def step_workspace_bytes(k_pool, num_q_heads: int, n_prefill: int, n_decode: int, pages_per_row: int) -> int:
    pool = pool_desc(k_pool, num_q_heads)
    return int(LIB.step_paged_workspace(ctypes.byref(pool), int(n_prefill), int(n_decode), int(pages_per_row)))


def step_paged(q, k, v, q_gain, k_gain, rope_cos, rope_sin, positions, rows, slots, step_positions,
               table, decode_row0: int, scale: float, q_out, k_pool, v_pool, prefill_out, decode_out,
               workspace, eps: float = 1e-6, stream=None) -> None:
    """One mixed step in a single launch: append over the prompt tokens (positions,
    rows, slots) and the decode rows (step_positions, table rows decode_row0 + b),
    then prefill attention into prefill_out and decode attention into decode_out."""
    import torch
    n_q = q_out.shape[-1] // HEAD_DIM
    pool = pool_desc(k_pool, n_q)
    P = 0 if positions is None else int(positions.numel())
    R = 0 if step_positions is None else int(step_positions.numel())
    n = P + R
    ppr = int(table.shape[-1])
    ws_bytes = workspace.numel() * workspace.element_size()
    st = LIB.step_paged(
        _stream(stream), ctypes.byref(pool), P, R,
        _ptr(q, "q", torch.bfloat16, n * n_q * HEAD_DIM), _ptr(k, "k", torch.bfloat16, n * pool.num_kv_heads * HEAD_DIM),
        _ptr(v, "v", torch.bfloat16, n * pool.num_kv_heads * HEAD_DIM), _dtype_code(q),
        _ptr(q_gain, "q_gain", torch.float32, HEAD_DIM), _ptr(k_gain, "k_gain", torch.float32, HEAD_DIM),
        float(eps), _ptr(rope_cos, "rope_cos", torch.float32), _ptr(rope_sin, "rope_sin", torch.float32),
        int(rope_cos.numel() // (HEAD_DIM // 2)),
        _ptr(positions, "positions", torch.int32, P) if P else None,
        _ptr(rows, "rows", torch.int32, P) if P else None,
        _ptr(slots, "slots", torch.int32, P) if P else None,
        _ptr(step_positions, "step_positions", torch.int32, R) if R else None,
        _ptr(table, "table", torch.int32), int(table.shape[0]), ppr, int(decode_row0), float(scale),
        _ptr(q_out, "q_out", torch.bfloat16, n * n_q * HEAD_DIM), _ptr(k_pool, "k_pool", torch.bfloat16),
        _ptr(v_pool, "v_pool", torch.bfloat16),
        _ptr(prefill_out, "prefill_out", torch.float32, P * n_q * HEAD_DIM) if P else None,
        _ptr(decode_out, "decode_out", torch.float32, R * n_q * HEAD_DIM) if R else None,
        _ptr(workspace, "workspace"), ws_bytes)
    _check(st, "step_paged")


def check_indices(k_pool, num_q_heads: int, table, rows=None, positions=None, slots=None, step_positions=None,
                  decode_row0: int = 0, rope_rows: int = 0, counts=None, wait: bool = True, stream=None):
    """qkr_check_indices: count out-of-range rows, positions, visited page ids and
    slots, and slots that differ from their row's page table, for prompt tokens
    (rows, positions, slots) and decode rows (step_positions, table rows
    decode_row0 + b). Returns (status, counts): with wait, status is 0 or
    QKR_EDATA and counts a dict; without it, status 0 and counts the device
    int32 tensor the counts land in (nothing synchronises)."""
    import torch
    pool = pool_desc(k_pool, num_q_heads)
    P = 0 if positions is None else int(positions.numel())
    R = 0 if step_positions is None else int(step_positions.numel())
    if counts is None:
        counts = torch.zeros(CHECK_COUNTS, dtype=torch.int32, device=table.device)
    st = LIB.qkr_check_indices(
        _stream(stream), ctypes.byref(pool), _ptr(table, "table", torch.int32), int(table.shape[0]),
        int(table.shape[-1]), P, _ptr(rows, "rows", torch.int32, P) if P else None,
        _ptr(positions, "positions", torch.int32, P) if P else None,
        _ptr(slots, "slots", torch.int32, P) if (P and slots is not None) else None,
        R, _ptr(step_positions, "step_positions", torch.int32, R) if R else None, int(decode_row0),
        int(rope_rows), _ptr(counts, "counts", torch.int32, CHECK_COUNTS), 1 if wait else 0)
    if st not in (0, QKR_EDATA):
        _check(st, "qkr_check_indices")
    if not wait:
        return st, counts
    c = counts.cpu().tolist()
    return st, {name: int(c[i]) for i, name in enumerate(CHECK_NAMES)}


def read_probe(buf, out, stream=None) -> None:
    """qkr_read_probe: one streaming read (non-temporal loads) of the device tensor
    buf (a measurement helper, not part of the attention path); out: 1 float32 on
    the same device."""
    import torch
    if not buf.is_cuda or not out.is_cuda or out.dtype != torch.float32 or out.numel() < 1:
        raise ValueError("read_probe needs a device buffer and one device float32")
    if not buf.is_contiguous():
        raise ValueError("read_probe needs a contiguous buffer")
    s = stream if stream is not None else torch.cuda.current_stream()
    _check(LIB.qkr_read_probe(ctypes.c_void_p(s.cuda_stream), ctypes.c_void_p(buf.data_ptr()),
                              buf.numel() * buf.element_size(), ctypes.c_void_p(out.data_ptr())), "qkr_read_probe")


def mfma_probe(iters, out, stream=None) -> int:
    """qkr_mfma_probe: a loop of bf16 MFMAs on every CU (a measurement helper, not
    part of the attention path); out: 1 float32 on the device. Returns the FLOPs."""
    import torch
    if not out.is_cuda or out.dtype != torch.float32 or out.numel() < 1:
        raise ValueError("mfma_probe needs one device float32")
    s = stream if stream is not None else torch.cuda.current_stream()
    flops = ctypes.c_int64(0)
    _check(LIB.qkr_mfma_probe(ctypes.c_void_p(s.cuda_stream), int(iters), ctypes.c_void_p(out.data_ptr()),
                              ctypes.byref(flops)), "qkr_mfma_probe")
    return int(flops.value)


def version() -> int:
    return int(LIB.qkr_version())


def last_error() -> str:
    return LIB.qkr_last_error().decode()

"""Shared helpers of the GPU parity tests: run a workload through the library
(through its C ABI binding) and build the oracle's view of the same pool."""
from __future__ import annotations

import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle as O
import workloads as W

DEV = "cuda"
TOL_F32 = 1e-4   # max abs error, float32 pool
TOL_BF16 = 2e-2  # max abs error, bfloat16 K/V with float32 accumulation

_ROPE = {}


def lib():
    import qk_norm_rope_amd as Q
    return Q


def rope_tables():
    if "t" not in _ROPE:
        cos, sin = lib().rope_table(O.ROPE_THETA, W.MAX_POSITIONS, W.HEAD_DIM)
        _ROPE["t"] = (torch.from_numpy(cos).to(DEV), torch.from_numpy(sin).to(DEV))
    return _ROPE["t"]


def bits(t: torch.Tensor) -> torch.Tensor:
    """Integer view of a float tensor, for bitwise comparisons (NaN == NaN)."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def host_values(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor -> the oracle's representation (float32, or bf16 bits)."""
    if dtype == "bf16":
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


class OraclePool:
    """The oracle's view of one pool (K: which=0, V: which=1).

    ``pool[g, slots]`` returns the stored values at ``slots`` of KV head g: the
    pre-step history regenerated on the host from the seeded generator, then the
    oracle's own writes of the step (``pool[:, s, :] = rows``). Nothing comes
    from the GPU.
    """

    def __init__(self, w: W.Workload, which: int):
        self.w = w
        self.which = which
        self.writes = {}

    def __setitem__(self, key, rows):
        _, s, _ = key
        self.writes[int(s)] = np.array(rows)

    def __getitem__(self, key):
        g, slots = key
        slots = np.asarray(slots, dtype=np.int64)
        vals = W.host_history(self.w, self.which, g, slots)
        if self.writes:
            for i, s in enumerate(slots):
                r = self.writes.get(int(s))
                if r is not None:
                    vals[i] = r[g]
        return vals


class SnapshotPool:
    """The oracle's view of one pool, read from a copy of the generator's pool that
    was taken on the device before any library kernel ran (``Run.k_pre`` /
    ``Run.v_pre``), plus the oracle's own writes of the step.

    ``check_append`` turns that copy into the expected post-append pool (the
    pre-step values with the oracle's rows at the oracle's slots), so after it the
    writes are already in place and applying them again changes nothing. Each
    thread keeps the host copy of the last slot list it read, so the oracle's
    per-KV-head reads of one row cost one device gather.
    """

    def __init__(self, pre: torch.Tensor, dtype: str):
        self.pre = pre
        self.dtype = dtype
        self.writes = {}
        self._local = threading.local()

    def __setitem__(self, key, rows):
        _, s, _ = key
        self.writes[int(s)] = np.array(rows)

    def __getitem__(self, key):
        g, slots = key
        slots = np.asarray(slots, dtype=np.int64)
        c = getattr(self._local, "c", None)
        if c is None or c[0].shape != slots.shape or not np.array_equal(c[0], slots):
            idx = torch.as_tensor(slots, device=self.pre.device)
            vals = host_values(self.pre.index_select(1, idx), self.dtype)
            if self.writes:
                for i, s in enumerate(slots.tolist()):
                    r = self.writes.get(s)
                    if r is not None:
                        vals[:, i] = r
            c = (slots.copy(), vals)
            self._local.c = c
        return c[1][g]


def oracle_workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def oracle_parallel(fn, tokens):
    """fn(tokens_subset) -> [len(subset), n] for interleaved subsets of ``tokens`` on
    threads (the oracle's NumPy calls release the interpreter lock; BLAS runs one
    thread per worker); the rows come back in the order of ``tokens``."""
    from threadpoolctl import threadpool_limits
    tokens = list(tokens)
    n = max(1, min(oracle_workers(), len(tokens)))
    parts_in = [tokens[i::n] for i in range(n)]
    with threadpool_limits(1), ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(fn, parts_in))
    out = np.empty((len(tokens), parts[0].shape[1]), dtype=np.float64)
    for i in range(n):
        out[i::n] = parts[i]
    return out


def report(name: str, got: np.ndarray, ref: np.ndarray, tol: float) -> float:
    """Max and mean abs error and NaN count of got against ref; asserts no NaN and
    max abs error <= tol. Returns the max abs error."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    d = np.abs(got.astype(np.float64) - ref)
    n_nan = int(np.isnan(got).sum())
    n_inf = int(np.isinf(got).sum())
    mx = float(np.nanmax(d)) if d.size else 0.0
    mean = float(np.nanmean(d)) if d.size else 0.0
    print(f"[parity] {name}: {got.shape[0]} x {got.shape[1] if got.ndim > 1 else 1} outputs, "
          f"max abs err {mx:.3e}, mean abs err {mean:.3e}, NaN {n_nan}, Inf {n_inf}", flush=True)
    assert n_nan == 0 and n_inf == 0, f"{name}: non-finite outputs"
    assert mx <= tol, f"{name}: max abs err {mx} > {tol}"
    return mx


class Run:
    """One workload on the GPU: inputs, pre-step pools, and the library's outputs."""

    def __init__(self, w: W.Workload, keep_pre: bool = True):
        self.w = w
        self.t = W.upload(w, DEV)
        self.k_pool, self.v_pool = W.make_pools(w, DEV)
        self.k_pre = self.k_pool.clone() if keep_pre else None
        self.v_pre = self.v_pool.clone() if keep_pre else None
        self.td = W.torch_dtype(w.dtype)
        self.rope = None   # (cos, sin) device tables; None: rope_tables() (W.MAX_POSITIONS rows)
        self.q_out = None
        self.pre_out = None
        self.dec_out = None

    def positions_all(self):
        return torch.cat([self.t["positions"], self.t["step_positions"]])

    def append(self):
        Q = lib()
        w, t = self.w, self.t
        cos, sin = self.rope or rope_tables()
        self.q_out = torch.empty((w.n_tokens, w.n_q_heads * W.HEAD_DIM), dtype=self.td, device=DEV)
        Q.qknorm_rope_append(t["q"], t["k"], t["v"], t["q_gain"], t["k_gain"], cos, sin,
                             self.positions_all(), self.q_out, self.k_pool, self.v_pool,
                             slots=t["slots"] if w.n_prefill else None,
                             table=t["decode_table"] if w.n_decode else None)

    def prefill(self):
        Q = lib()
        w, t = self.w, self.t
        P = w.n_prefill
        self.pre_out = torch.empty((P, w.n_q_heads * W.HEAD_DIM), dtype=torch.float32, device=DEV)
        ws = torch.zeros(max(1, Q.prefill_workspace_bytes(self.k_pool, w.n_q_heads, P)),
                         dtype=torch.uint8, device=DEV)
        Q.paged_prefill_attn(self.q_out[:P], self.k_pool, self.v_pool, t["table"], t["rows"],
                             t["positions"], W.SCALE, self.pre_out, ws)

    def decode(self, workspace=None):
        Q = lib()
        w, t = self.w, self.t
        P, R = w.n_prefill, w.n_decode
        self.dec_out = torch.empty((R, w.n_q_heads * W.HEAD_DIM), dtype=torch.float32, device=DEV)
        if workspace is None:
            workspace = decode_workspace(self.k_pool, R, w.pages_per_row)
        Q.paged_decode_attn(self.q_out[P:], self.k_pool, self.v_pool, t["decode_table"],
                            t["step_positions"], W.SCALE, self.dec_out, workspace)

    def fused_step(self, workspace=None):
        """The whole step through step_paged (one launch)."""
        Q = lib()
        w, t = self.w, self.t
        cos, sin = rope_tables()
        P, R = w.n_prefill, w.n_decode
        n_q = w.n_q_heads * W.HEAD_DIM
        self.q_out = torch.empty((w.n_tokens, n_q), dtype=self.td, device=DEV)
        self.pre_out = torch.empty((P, n_q), dtype=torch.float32, device=DEV)
        self.dec_out = torch.empty((R, n_q), dtype=torch.float32, device=DEV)
        if workspace is None:
            workspace = step_workspace(self.k_pool, P, R, w.pages_per_row)
        Q.step_paged(t["q"], t["k"], t["v"], t["q_gain"], t["k_gain"], cos, sin,
                     t["positions"] if P else None, t["rows"] if P else None, t["slots"] if P else None,
                     t["step_positions"] if R else None, t["table"], w.decode_row0, W.SCALE,
                     self.q_out, self.k_pool, self.v_pool, self.pre_out, self.dec_out, workspace)

    def step_nosync(self):
        self.append()
        if self.w.n_prefill:
            self.prefill()
        if self.w.n_decode:
            self.decode()

    def step(self):
        self.step_nosync()
        torch.cuda.synchronize()


def decode_workspace(k_pool, n_rows, pages_per_row):
    Q = lib()
    n = Q.decode_workspace_bytes(k_pool, 4 * k_pool.shape[0], n_rows, pages_per_row)
    return torch.zeros(max(1, n), dtype=torch.uint8, device=DEV)


def step_workspace(k_pool, n_prefill, n_decode, pages_per_row):
    Q = lib()
    n = Q.step_workspace_bytes(k_pool, 4 * k_pool.shape[0], n_prefill, n_decode, pages_per_row)
    return torch.zeros(max(1, n), dtype=torch.uint8, device=DEV)


def oracle_append(w: W.Workload):
    """Oracle q_out and stored k/v rows for every token of the step, and their slots."""
    every_at = np.concatenate([w.positions, w.step_positions]).astype(np.int64)
    dec_slots = [O.page_slot(w.decode_table[b], int(w.step_positions[b])) for b in range(w.n_decode)]
    every_slot = np.concatenate([w.slots.astype(np.int64), np.asarray(dec_slots, dtype=np.int64)])
    q_out, k_rows, v_rows = O.append(w.q, w.k, w.v, w.dtype, w.dtype, w.q_gain, w.k_gain, every_at,
                                     n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads)
    return q_out, k_rows, v_rows, every_slot


def oracle_pools(w: W.Workload, k_rows, v_rows, every_slot, run=None):
    """The oracle's pools after the step's writes: from the run's pre-step copies
    when it kept them (SnapshotPool), else regenerated on the host (OraclePool)."""
    if run is not None and run.k_pre is not None:
        kp, vp = SnapshotPool(run.k_pre, w.dtype), SnapshotPool(run.v_pre, w.dtype)
    else:
        kp, vp = OraclePool(w, 0), OraclePool(w, 1)
    O.apply_writes(kp, vp, every_slot, k_rows, v_rows)
    return kp, vp


def oracle_decode(w: W.Workload, ref_q, kp, vp, rows=None):
    """Oracle decode of the step's rows (all by default), threads over rows."""
    P = w.n_prefill
    rows = range(w.n_decode) if rows is None else rows
    heads = {"n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads}
    return oracle_parallel(lambda part: O.decode(ref_q[P:], w.dtype, kp, vp, w.dtype, w.decode_table,
                                                 w.step_positions, W.SCALE, tokens=part, **heads), rows)


def oracle_prefill(w: W.Workload, ref_q, kp, vp, toks=None):
    """Oracle prefill of the step's prompt tokens (all by default), threads over tokens."""
    P = w.n_prefill
    toks = range(P) if toks is None else toks
    heads = {"n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads}
    return oracle_parallel(lambda part: O.prefill(ref_q[:P], w.dtype, kp, vp, w.dtype, w.table, w.rows,
                                                  w.positions, W.SCALE, tokens=part, **heads), toks)


def max_abs_err(got: np.ndarray, ref: np.ndarray) -> float:
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), "non-finite output"
    return float(np.max(np.abs(got.astype(np.float64) - ref)))


def check_append(run, ref_q, k_rows, v_rows, slots):
    """q_out bit-exact, and every pool byte: the written slots hold the oracle's
    rows, all others their pre-step values (needs a Run with keep_pre)."""
    w = run.w
    assert np.array_equal(host_values(run.q_out, w.dtype), ref_q), "q_out bytes differ"
    idx = torch.as_tensor(slots[slots >= 0], device=DEV)
    td = run.td
    keep = slots >= 0
    for pool, pre, rows in ((run.k_pool, run.k_pre, k_rows), (run.v_pool, run.v_pre, v_rows)):
        exp = pre
        r = rows[keep]
        if w.dtype == "bf16":
            rt = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16).to(DEV)
        else:
            rt = torch.from_numpy(r).to(DEV)
        exp[:, idx] = rt.permute(1, 0, 2).to(td)
        assert torch.equal(bits(pool), bits(exp)), "pool bytes differ"

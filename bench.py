"""Benchmark of the paged QK-norm + RoPE + GQA attention step on one MI355X.

One step = the whole path over one batch: qknorm_rope_append over every token
(prompt chunks + decode rows), paged_prefill_attn over the prompt tokens,
paged_decode_attn over the decode rows, all on one stream. The default
workload is the mixed step (2 prompt chunks of 2048 tokens at positions 8192
and 0, 128 decode rows at positions uniform in [1, 16384], 65536-page bfloat16
pool), the one workload that exercises every part of the path.

Prints one JSON line. ``value`` is the paged-decode attention throughput in
algorithmic GB/s (K/V bytes of every visible position + q + out, divided by the
decode kernel's time, measured with HIP events on the launch stream around each
call, averaged over the timed steps); the prefill TFLOP/s (visible (query, key)
pairs x 16384 FLOP) and the append GB/s are reported beside it. By default a
1 GiB read evicts the 256 MB MALL and the L2 before every timed step (outside
the timed windows); the warm back-to-back figures follow under ``warm``. The
other standard workloads (8 decode rows, 64 ragged decode rows with a shared
prefix, the 4-prompt packed prefill) are timed the same way under
``workloads``.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn GB/s (% HBM peak) + prefill TFLOP/s (% MFMA peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
COPY_PROBE_BYTES = 1 << 30
MFMA_BF16_PEAK_TFLOPS = 2500.0


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "step_2x2048_plus_128rows_hbm_traffic.txt")
DECODE_SOURCES = ("decode.hip", "decode_body.h", "common.h")


def sources_sha256(sources) -> str:
    """sha256 over the named csrc files, in order (a kernel, its device code, helpers)."""
    import hashlib
    h = hashlib.sha256()
    for s in sources:
        h.update(open(os.path.join(ROOT, "qk_norm_rope_amd", "csrc", s), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel: str, sources):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel's sources have changed since the counters were taken."""
    try:
        kv = dict(line.split(": ", 1) for line in open(TRAFFIC_FILE).read().splitlines()
                  if line and not line.startswith("#"))
        sha = sources_sha256(sources)
        if kv.get(f"{kernel}.source_sha256") != sha:
            return None
        return int(float(kv[f"{kernel}.traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def algorithmic_work(w):
    """Bytes / FLOPs each part of one step must move or compute.

    Decode: K and V of every visible position of every row ("logical"; a page
    shared by several rows counts once per row), plus q, out and the table rows;
    "unique" counts each visible pool slot once. Prefill: visible (query, key)
    pairs x 4 x head_dim x query heads. Append: q, k, v in and q_out, k, v out,
    the cos/sin row, position and slot of every token.
    """
    import numpy as np
    D, HQ, HKV = 128, w.n_q_heads, w.n_kv_heads
    dec_pos = w.step_positions.astype(np.int64)
    R = len(dec_pos)
    per_pos = HKV * D * 2 * 2                                     # K and V, bf16
    dec_kv = int((dec_pos + 1).sum()) * per_pos
    extra = R * HQ * D * 2 + R * HQ * D * 4 + R * 4 * (1 + w.pages_per_row)
    if R:
        tab = w.decode_table.astype(np.int64)
        slots = np.concatenate([tab[b][np.arange(p + 1) // 64] * 64 + np.arange(p + 1) % 64
                                for b, p in enumerate(dec_pos)])
        dec_kv_unique = int(len(np.unique(slots))) * per_pos
    else:
        dec_kv_unique = 0
    pre_pairs = int((w.positions.astype(np.int64) + 1).sum())
    pre_flops = pre_pairs * 4 * D * HQ
    n = w.n_tokens
    app_bytes = n * ((HQ + 2 * HKV) * D * 2 * 2 + D * 4 + 4 + 4)  # q,k,v in + q_out,k,v out, cos/sin, pos, slot
    return {"decode_bytes": dec_kv + extra, "decode_kv_bytes": dec_kv,
            "decode_bytes_unique": dec_kv_unique + extra, "decode_kv_bytes_unique": dec_kv_unique,
            "prefill_flops": pre_flops, "prefill_pairs": pre_pairs, "append_bytes": app_bytes}


class Step:
    """One workload on the GPU: inputs, pools, outputs, and one step's launches."""

    def __init__(self, Q, W, w, dev, cos, sin):
        import torch
        self.Q, self.W, self.w = Q, W, w
        self.t = W.upload(w, dev)
        self.k_pool, self.v_pool = W.make_pools(w, dev)
        self.cos, self.sin = cos, sin
        P, R = w.n_prefill, w.n_decode
        self.P, self.R = P, R
        self.positions_all = torch.cat([self.t["positions"], self.t["step_positions"]])
        nq = w.n_q_heads * 128
        self.q_out = torch.empty((P + R, nq), dtype=torch.bfloat16, device=dev)
        self.pre_out = torch.empty((max(P, 1), nq), dtype=torch.float32, device=dev)
        self.dec_out = torch.empty((max(R, 1), nq), dtype=torch.float32, device=dev)
        self.ws_p = torch.zeros(max(1, Q.prefill_workspace_bytes(self.k_pool, w.n_q_heads, max(P, 1))),
                                dtype=torch.uint8, device=dev)
        self.ws_d = torch.zeros(max(1, Q.decode_workspace_bytes(self.k_pool, w.n_q_heads, max(R, 1),
                                                                w.pages_per_row)), dtype=torch.uint8, device=dev)

    def append(self):
        t = self.t
        self.Q.qknorm_rope_append(t["q"], t["k"], t["v"], t["q_gain"], t["k_gain"], self.cos, self.sin,
                                  self.positions_all, self.q_out, self.k_pool, self.v_pool,
                                  slots=t["slots"] if self.P else None,
                                  table=t["decode_table"] if self.R else None)

    def prefill(self):
        t = self.t
        self.Q.paged_prefill_attn(self.q_out[:self.P], self.k_pool, self.v_pool, t["table"], t["rows"],
                                  t["positions"], self.W.SCALE, self.pre_out, self.ws_p)

    def decode(self):
        t = self.t
        self.Q.paged_decode_attn(self.q_out[self.P:], self.k_pool, self.v_pool, t["decode_table"],
                                 t["step_positions"], self.W.SCALE, self.dec_out, self.ws_d)

    def run(self, stream, ev=None):
        """append, prefill, decode; ev: four events recorded between the calls."""
        if ev is not None:
            ev[0].record(stream)
        self.append()
        if ev is not None:
            ev[1].record(stream)
        if self.P:
            self.prefill()
        if ev is not None:
            ev[2].record(stream)
        if self.R:
            self.decode()
        if ev is not None:
            ev[3].record(stream)


def time_steps(step, stream, steps, warmup, scratch):
    """Per-kernel ms (event windows averaged over the timed steps), the step time
    and the wall time. With ``scratch`` (a 1 GiB tensor) every timed step is
    preceded by a read of it (evicting the MALL and the L2; a read leaves no dirty
    lines), outside the windows, and the step time is the sum of the windows;
    without it the steps run back to back and the step time is first start to
    last end over the steps."""
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for _ in range(warmup):
        step.run(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if scratch is not None:
            scratch.amax()   # reads every byte, writes 4
        step.run(stream, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = {"append": 0.0, "prefill": 0.0, "decode": 0.0}
    for ev in evs:
        times["append"] += ev[0].elapsed_time(ev[1])
        times["prefill"] += ev[1].elapsed_time(ev[2])
        times["decode"] += ev[2].elapsed_time(ev[3])
    for k in times:
        times[k] /= steps
    step_ms = sum(times.values()) if scratch is not None else evs[0][0].elapsed_time(evs[-1][3]) / steps
    return times, step_ms, wall


def rates(w, times):
    """GB/s and TFLOP/s of the step's kernels from their per-launch times."""
    work = algorithmic_work(w)
    out = {}
    if w.n_decode:
        gbs = work["decode_bytes"] / (times["decode"] * 1e-3) / 1e9
        out["decode"] = {"gbs": round(gbs, 2), "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "bytes_per_launch": work["decode_bytes"], "ms_per_launch": round(times["decode"], 5),
                         "bound": "hbm"}
        if work["decode_kv_bytes_unique"] != work["decode_kv_bytes"]:
            u = work["decode_bytes_unique"] / (times["decode"] * 1e-3) / 1e9
            out["decode"].update({"gbs_unique": round(u, 2), "frac_unique": round(u / HBM_PEAK_GBS, 4),
                                  "bytes_per_launch_unique": work["decode_bytes_unique"]})
    if w.n_prefill:
        tf = work["prefill_flops"] / (times["prefill"] * 1e-3) / 1e12
        out["prefill"] = {"tflops": round(tf, 2), "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                          "flops_per_launch": work["prefill_flops"], "ms_per_launch": round(times["prefill"], 5),
                          "bound": "mfma"}
    gbs = work["append_bytes"] / (times["append"] * 1e-3) / 1e9
    out["append"] = {"gbs": round(gbs, 2), "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": work["append_bytes"], "ms_per_launch": round(times["append"], 5),
                     "bound": "hbm"}
    return out


def measure_fused(step, stream, steps, scratch):
    """The same step through step_paged (one launch), timed like the three calls:
    one event window per step, flushed before each when ``scratch`` is given, else
    back to back."""
    import torch
    Q, W, w, t = step.Q, step.W, step.w, step.t
    P, R = step.P, step.R
    ws = torch.zeros(max(1, Q.step_workspace_bytes(step.k_pool, w.n_q_heads, P, R, w.pages_per_row)),
                     dtype=torch.uint8, device=step.q_out.device)

    def f():
        Q.step_paged(t["q"], t["k"], t["v"], t["q_gain"], t["k_gain"], step.cos, step.sin,
                     t["positions"] if P else None, t["rows"] if P else None, t["slots"] if P else None,
                     t["step_positions"] if R else None, t["table"], w.decode_row0, W.SCALE,
                     step.q_out, step.k_pool, step.v_pool, step.pre_out, step.dec_out, ws)
    for _ in range(3):
        f()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        if scratch is not None:
            scratch.amax()
        a.record(stream)
        f()
        b.record(stream)
    torch.cuda.synchronize()
    if scratch is not None:
        ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    else:
        ms = evs[0][0].elapsed_time(evs[-1][1]) / steps
    fault = int(ws[20:24].view(torch.int32).item())
    return {"ms_per_step": round(ms, 4), "kernel": "step_paged_kernel", "launches": 1, "wait_gave_up": fault}


def measure_hbm_reference(Q, dev, reps=5):
    """What plain streaming kernels reach on this GPU: the library's read probe (a
    grid-stride read with non-temporal loads, as decode's K/V loads; no paging,
    masking or attention arithmetic) over 4 GiB, and
    torch's copy_ (a read and a write) over 1 GiB, both far beyond the 256 MB MALL.
    The roofline peak stays the published 8 TB/s; these say how much of it the
    simplest kernels get on the same GPU."""
    import torch
    big = torch.ones(4 * COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    x = big[:COPY_PROBE_BYTES // 4]
    y = torch.empty_like(x)
    for _ in range(2):
        Q.read_probe(big, sink)
        y.copy_(x)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        Q.read_probe(big, sink)
    ev[1].record()
    for _ in range(reps):
        y.copy_(x)
    ev[2].record()
    torch.cuda.synchronize()
    read_ms = ev[0].elapsed_time(ev[1]) / reps
    copy_ms = ev[1].elapsed_time(ev[2]) / reps
    del big, x, y, sink
    torch.cuda.empty_cache()
    return {"read_gbs": round(4 * COPY_PROBE_BYTES / (read_ms * 1e-3) / 1e9, 1),
            "copy_gbs": round(2 * COPY_PROBE_BYTES / (copy_ms * 1e-3) / 1e9, 1),
            "source": "qkr_read_probe over 4 GiB (non-temporal read); torch copy_ over 1 GiB (read + write); "
                      "HIP events"}


def measure_mfma_reference(Q, dev, iters=4000, reps=5):
    """What the matrix cores sustain on this GPU: the library's MFMA probe (bf16
    32x32x16 MFMAs from registers, eight independent accumulators per wave, two
    waves per SIMD, no memory traffic). The roofline peak stays the published
    2.5 PFLOP/s dense bf16."""
    import torch
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    Q.mfma_probe(iters, sink)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    flops = 0
    for _ in range(reps):
        flops += Q.mfma_probe(iters, sink)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    return {"tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "source": "qkr_mfma_probe: bf16 32x32x16 MFMAs from registers on every CU, HIP events"}


def measure_append_steady(step, stream, reps=50):
    """The step's append, launched back to back (its in-step event window also holds
    the launch gap after the previous step's last kernel)."""
    import torch
    step.append()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        step.append()
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / reps


def measure_packed(step, stream, reps=10):
    """The step's prompt tokens through packed_prefill_attn (each chunk its own
    prompt, attending only among itself), timed after the step's timed region."""
    import torch
    Q, W, w, t = step.Q, step.W, step.w, step.t
    P = w.n_prefill
    seg = t["rows"]   # one prompt per chunk, one row per prompt
    ws = torch.zeros(max(1, Q.packed_workspace_bytes(step.k_pool, w.n_q_heads, P)), dtype=torch.uint8,
                     device=step.q_out.device)

    def f():
        Q.packed_prefill_attn(step.q_out[:P], step.k_pool, step.v_pool, t["table"], t["rows"], t["positions"],
                              seg, W.SCALE, step.pre_out, ws)
    for _ in range(2):
        f()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        f()
    b.record(stream)
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    first = {}
    for r, p in zip(w.rows.tolist(), w.positions.tolist()):
        first[r] = min(first.get(r, p), p)
    pairs = int(sum(p - first[r] + 1 for r, p in zip(w.rows.tolist(), w.positions.tolist())))
    flops = pairs * 4 * 128 * w.n_q_heads
    tf = flops / (ms * 1e-3) / 1e12
    return {"tflops": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_per_launch": flops, "ms_per_launch": round(ms, 5), "bound": "mfma",
            "form": "each chunk attends only to itself (no history)"}


def measure_variants(step, stream, reps=10):
    """The attention variants on the step's inputs, timed after the step's timed
    region: the append with one norm over all heads and a 64-wide rotation, and
    the decode with the sigmoid output gate."""
    import numpy as np
    import torch
    Q, W, w, t = step.Q, step.W, step.w, step.t
    dev = step.q_out.device
    work = algorithmic_work(w)
    rng = np.random.default_rng(7)
    gq = torch.from_numpy(rng.uniform(0.5, 1.5, w.n_q_heads * 128).astype(np.float32)).to(dev)
    gk = torch.from_numpy(rng.uniform(0.5, 1.5, w.n_kv_heads * 128).astype(np.float32)).to(dev)
    c64, s64 = Q.rope_table(1e6, W.MAX_POSITIONS, 64)
    c64, s64 = torch.from_numpy(c64).to(dev), torch.from_numpy(s64).to(dev)
    P, R = w.n_prefill, w.n_decode

    def timed(fn):
        fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / reps

    app_ms = timed(lambda: Q.qknorm_rope_append(
        t["q"], t["k"], t["v"], gq, gk, c64, s64, step.positions_all, step.q_out, step.k_pool, step.v_pool,
        slots=t["slots"] if P else None, table=t["decode_table"] if R else None,
        qk_norm_whole=True, rotary_dim=64))
    # the extra gain bytes of the whole-vector norm are read once per token from cache; not counted
    out = {"append_whole_norm_rotary64": {"gbs": round(work["append_bytes"] / (app_ms * 1e-3) / 1e9, 2),
                                          "ms_per_launch": round(app_ms, 5), "bound": "hbm"}}
    if R:
        gate = torch.randn((R, w.n_q_heads * 128), device=dev).to(torch.bfloat16)
        dec_ms = timed(lambda: Q.paged_decode_attn(step.q_out[P:], step.k_pool, step.v_pool, t["decode_table"],
                                                   t["step_positions"], W.SCALE, step.dec_out, step.ws_d,
                                                   gate=gate))
        gbs = (work["decode_bytes"] + R * w.n_q_heads * 128 * 2) / (dec_ms * 1e-3) / 1e9
        out["decode_gated"] = {"gbs": round(gbs, 2), "frac": round(gbs / HBM_PEAK_GBS, 4),
                               "ms_per_launch": round(dec_ms, 5), "bound": "hbm"}
    return out


# ---------------------------------------------------------------- the oracle

def oracle_snapshot(w, k_pool, v_pool, sample_rows=128, prefill_tokens=256, seed=0):
    """Host copies of the pool slots the oracle sample reads, taken from the
    generator's pre-step pools before any library kernel has run."""
    import numpy as np
    import torch
    rng = np.random.default_rng(seed)
    rows = sorted(rng.choice(w.n_decode, size=min(sample_rows, w.n_decode), replace=False).tolist()) \
        if w.n_decode else []
    toks = sorted(rng.choice(w.n_prefill, size=min(prefill_tokens, w.n_prefill), replace=False).tolist()) \
        if w.n_prefill else []

    def grab(row, n):
        sl = torch.as_tensor(w.row_slot_list(row, n), device=k_pool.device)
        k = k_pool[:, sl].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        v = v_pool[:, sl].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return k, v

    dec = {b: grab(w.decode_row0 + b, int(w.step_positions[b])) for b in rows}
    pre_rows = sorted(set(int(w.rows[t]) for t in toks))
    hist = dict(w.history)
    pre = {r: grab(r, hist.get(r, 0)) for r in pre_rows}
    return {"rows": rows, "toks": toks, "dec": dec, "pre": pre}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def _host_pools(w, O, W, q_out, k_rows, v_rows):
    """Dense host pools of a small workload: history regenerated on the host, then
    the oracle's writes of the step."""
    import numpy as np
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    kp = np.zeros((w.n_kv_heads, w.pool_slots, 128), dt)
    vp = np.zeros_like(kp)
    hs = w.history_slots()
    for g in range(w.n_kv_heads):
        if len(hs):
            kp[g, hs] = W.host_history(w, 0, g, hs)
            vp[g, hs] = W.host_history(w, 1, g, hs)
    dec_slots = [O.page_slot(w.decode_table[b], int(w.step_positions[b])) for b in range(w.n_decode)]
    every_slot = np.concatenate([w.slots.astype(np.int64), np.asarray(dec_slots, dtype=np.int64)])
    O.apply_writes(kp, vp, every_slot, k_rows, v_rows)
    return kp, vp


def cpu_small_workloads():
    """The oracle on the small standard workloads, whole: all cores, then one thread.

    1 decode row (float32), 8 decode rows (bfloat16, all of them) and the 4-prompt
    packed prefill (all 4096 tokens). Each timed region is the oracle's attention
    call only (the append and the pools are prepared before it).
    """
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle as O
    import workloads as W
    res = {}
    for cfg in (0, 1, 3):
        w = W.config(cfg)
        every_at = np.concatenate([w.positions, w.step_positions]).astype(np.int64)
        q_out, k_rows, v_rows = O.append(w.q, w.k, w.v, w.dtype, w.dtype, w.q_gain, w.k_gain, every_at)
        kp, vp = _host_pools(w, O, W, q_out, k_rows, v_rows)
        work = algorithmic_work(w)
        per_pos = 8 * 128 * 2 * (2 if w.dtype == "bf16" else 4)
        entry = {}
        for label, threads in (("all_cores", None), ("one_thread", 1)):
            with threadpool_limits(threads):
                t0 = time.perf_counter()
                if w.n_decode:
                    O.decode(q_out, w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE)
                else:
                    O.prefill(q_out, w.dtype, kp, vp, w.dtype, w.table, w.rows, w.positions, W.SCALE)
                dt = time.perf_counter() - t0
            if w.n_decode:
                nbytes = int((w.step_positions.astype(np.int64) + 1).sum()) * per_pos
                entry[label] = {"seconds": round(dt, 4), "gbs": round(nbytes / dt / 1e9, 4)}
            else:
                entry[label] = {"seconds": round(dt, 4), "tflops": round(work["prefill_flops"] / dt / 1e12, 6)}
        res[w.name] = entry
    return res


def cpu_baseline(w, snap, passes=2):
    """The oracle on a bounded sample of the benchmarked workload, on the host cores.

    Decode: the sampled decode rows, ``passes`` times. Prefill: the sampled
    prompt tokens. The oracle computes the step's own q/k/v rows itself; the
    history comes from the snapshot; the timed regions are the oracle's
    attention calls only. The small standard workloads follow, whole, with all
    cores and with one thread.
    """
    import numpy as np
    import oracle as O
    import workloads as W
    rows, toks = snap["rows"], snap["toks"]
    P = w.n_prefill
    heads = {"n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads}
    res = {"unit": "GB/s", "cores": int(_blas_threads()), "nproc": int(os.cpu_count() or 1),
           "cpu_model": _cpu_model(), "kind": "oracle"}
    if rows:
        every_at = np.concatenate([w.positions, w.step_positions]).astype(np.int64)
        sel = [P + b for b in rows]
        q_out, k_rows, v_rows = O.append(w.q[sel], w.k[sel], w.v[sel], w.dtype, w.dtype,
                                         w.q_gain, w.k_gain, every_at[sel], **heads)
        pos_s = w.step_positions[rows].astype(np.int64)
        ppr = -(-(int(pos_s.max()) + 1) // 64)
        table = np.arange(len(rows) * ppr, dtype=np.int32).reshape(len(rows), ppr)
        kp = np.zeros((w.n_kv_heads, len(rows) * ppr * 64, 128), np.uint16)
        vp = np.zeros_like(kp)
        for i, b in enumerate(rows):
            n = int(pos_s[i])      # history positions 0..n-1, then the row's new token
            base = i * ppr * 64
            kp[:, base:base + n], vp[:, base:base + n] = snap["dec"][b]
            kp[:, base + n] = k_rows[i]
            vp[:, base + n] = v_rows[i]
        t0 = time.perf_counter()
        for _ in range(passes):
            O.decode(q_out, w.dtype, kp, vp, w.dtype, table, pos_s, W.SCALE, **heads)
        dt = (time.perf_counter() - t0) / passes
        del kp, vp
        nbytes = int((pos_s + 1).sum()) * w.n_kv_heads * 128 * 2 * 2
        res.update({"value": round(nbytes / dt / 1e9, 4), "seconds": round(dt * passes, 3),
                    "sample": f"float64 oracle decode of {len(rows)} of the {w.n_decode} decode rows "
                              f"({int((pos_s + 1).sum())} visible positions, {nbytes / 1e9:.3f} GB of K/V), "
                              f"{passes} passes, BLAS threads = {res['cores']}"})
    if toks:
        q_pre, k_pre, v_pre = O.append(w.q[:P], w.k[:P], w.v[:P], w.dtype, w.dtype, w.q_gain,
                                       w.k_gain, w.positions, **heads)
        pre_rows = sorted(snap["pre"])
        nvis = {r: max(int(w.positions[t]) for t in toks if int(w.rows[t]) == r) + 1 for r in pre_rows}
        ppr2 = max(-(-n // 64) for n in nvis.values())
        tab2 = np.zeros((max(pre_rows) + 1, ppr2), np.int32)
        kp2 = np.zeros((w.n_kv_heads, len(pre_rows) * ppr2 * 64, 128), np.uint16)
        vp2 = np.zeros_like(kp2)
        for i, r in enumerate(pre_rows):
            base = i * ppr2 * 64
            kh, vh = snap["pre"][r]
            kp2[:, base:base + kh.shape[1]] = kh
            vp2[:, base:base + vh.shape[1]] = vh
            tab2[r] = np.arange(i * ppr2, (i + 1) * ppr2)
        # the chunk's own keys/values, as the oracle computed them, at their positions
        for t in range(P):
            r = int(w.rows[t])
            if r in nvis and int(w.positions[t]) < nvis[r]:
                base = pre_rows.index(r) * ppr2 * 64
                kp2[:, base + int(w.positions[t])] = k_pre[t]
                vp2[:, base + int(w.positions[t])] = v_pre[t]
        t0 = time.perf_counter()
        O.prefill(q_pre, w.dtype, kp2, vp2, w.dtype, tab2, w.rows, w.positions, W.SCALE, tokens=toks, **heads)
        dtp = time.perf_counter() - t0
        flops = sum(int(w.positions[t]) + 1 for t in toks) * 4 * 128 * w.n_q_heads
        res["prefill"] = {"tflops": round(flops / dtp / 1e12, 6), "unit": "TFLOP/s", "seconds": round(dtp, 3),
                          "sample": f"float64 oracle prefill of {len(toks)} of the {P} prompt tokens"}
    res["workloads"] = cpu_small_workloads()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4, help="standard workload index (default: mixed step)")
    ap.add_argument("--kv-heads", type=int, default=8, choices=(1, 2, 4, 8),
                    help="KV heads of the workload (4 query heads each): 8 / S is one GPU's share "
                         "when the heads are sharded over S GPUs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip everything after the timed steps (warm pass, other workloads, packed form, "
                         "variants, back-to-back append); for profiler runs that average per kernel name")
    ap.add_argument("--warm", action="store_true",
                    help="time the steps back to back with no cache flush between them (default: a 1 GiB read "
                         "evicts the 256 MB MALL and the L2 before every timed step, outside the timed windows)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run a plain 1 GiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path has no "
              "cross-GPU part; see the sharding notes in the design document.", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as W
    import qk_norm_rope_amd as Q

    dev = "cuda"
    torch.cuda.set_device(0)
    w = W.config(args.workload, kv_heads=args.kv_heads)
    if w.dtype != "bf16":
        print("bench.py measures the bfloat16 workloads (1..4)", file=sys.stderr)
        sys.exit(2)
    cos, sin = Q.rope_table(1e6, W.MAX_POSITIONS)
    cos, sin = torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev)
    step = Step(Q, W, w, dev, cos, sin)
    snap = None if args.no_cpu_baseline else oracle_snapshot(w, step.k_pool, step.v_pool)
    stream = torch.cuda.current_stream()

    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    scratch = None if args.warm else torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
    times, step_ms, wall = time_steps(step, stream, args.steps, args.warmup, scratch)
    r = rates(w, times)
    extras = not args.no_extras
    flushed = scratch is not None
    warm = None
    if extras and flushed:
        wt, wms, _ = time_steps(step, stream, args.steps, 1, None)
        wr = rates(w, wt)
        warm = {"ms_per_step": round(wms, 4)}
        for k, v in wr.items():
            warm[k] = {"gbs" if "gbs" in v else "tflops": v.get("gbs", v.get("tflops")),
                       "ms_per_launch": v["ms_per_launch"]}
    fused = measure_fused(step, stream, args.steps, scratch) if extras else None
    app_steady_ms = measure_append_steady(step, stream) if extras else None
    packed = measure_packed(step, stream) if (step.P and extras) else None
    variants = measure_variants(step, stream) if extras else None
    hbm_ref = measure_hbm_reference(Q, dev) if extras else None
    mfma_ref = measure_mfma_reference(Q, dev) if extras else None
    others = None
    if extras and args.workload == 4 and args.kv_heads == 8:
        others = {}
        for cfg in (1, 2, 3):
            wo = W.config(cfg)
            so = Step(Q, W, wo, dev, cos, sin)
            to, ms_o, _ = time_steps(so, stream, args.steps, args.warmup, scratch)
            others[wo.name] = {"ms_per_step": round(ms_o, 4), **rates(wo, to)}
            del so
            torch.cuda.empty_cache()
    del scratch

    if step.R:   # the dominant kernel: decode when the step has decode rows, else prefill
        dec_kernel = Q.decode_kernel_name(step.k_pool, w.n_q_heads, step.R, w.pages_per_row)
        roofline = {"bound": "hbm", "achieved": r["decode"]["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(r["decode"]["gbs"] / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(dec_kernel, DECODE_SOURCES)
                    if (args.workload == 4 and args.kv_heads == 8) else None,
                    "kernel": dec_kernel,
                    "bytes_per_launch": r["decode"]["bytes_per_launch"],
                    "ms_per_launch": round(times["decode"], 5)}
    else:
        roofline = {"bound": "mfma", "achieved": r["prefill"]["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": r["prefill"]["frac"], "traffic": None,
                    "kernel": "paged_prefill_bf16_kernel", "flops_per_launch": r["prefill"]["flops_per_launch"],
                    "ms_per_launch": r["prefill"]["ms_per_launch"]}
    result = {
        "metric": METRIC,
        "value": roofline["achieved"],
        "unit": roofline["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "prefill_tokens": step.P, "decode_rows": step.R,
                   "prefill_chunks": "2x2048 at positions 8192 and 0" if args.workload == 4 else None,
                   "decode_positions": "uniform [1, 16384]" if args.workload == 4 else None,
                   "pool_pages": w.num_pages, "page_size": 64, "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads,
                   "head_dim": 128,
                   "caches": "MALL and L2 flushed before every step" if flushed else "warm (back to back)"},
        "roofline": roofline,
    }
    if step.P:
        result["prefill"] = {**r["prefill"], "peak": MFMA_BF16_PEAK_TFLOPS}
    result["append"] = r["append"]
    if step.R and "gbs_unique" in r["decode"]:
        result["decode_unique"] = {k: r["decode"][k] for k in ("gbs_unique", "frac_unique", "bytes_per_launch_unique")}
    if app_steady_ms is not None:
        work = algorithmic_work(w)
        result["append"]["steady_gbs"] = round(work["append_bytes"] / (app_steady_ms * 1e-3) / 1e9, 2)
        result["append"]["steady_ms_per_launch"] = round(app_steady_ms, 5)
    if fused is not None:
        fused["ms_per_step_three_calls"] = round(step_ms, 4)
        fused["speedup"] = round(step_ms / fused["ms_per_step"], 4)
        result["fused_step"] = fused
    if warm is not None:
        result["warm"] = warm
    if others is not None:
        result["workloads"] = others
    if packed is not None:
        result["packed_prefill"] = packed
    if variants is not None:
        result["variants"] = variants
    if hbm_ref is not None:
        if roofline["unit"] == "GB/s":
            hbm_ref["decode_frac_of_read"] = round(roofline["achieved"] / hbm_ref["read_gbs"], 4)
        result["hbm_reference"] = hbm_ref
    if mfma_ref is not None:
        if "prefill" in result:
            mfma_ref["prefill_frac_of_probe"] = round(result["prefill"]["tflops"] / mfma_ref["tflops"], 4)
        result["mfma_reference"] = mfma_ref
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, snap)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

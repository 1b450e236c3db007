"""The attention variants of the pages through the C ABI: the whole-vector
QK-norm and partial rotary (qknorm_rope_append_ex, bit-exact against the
oracle's append with the same options) and the sigmoid output gate (the *_ex
attention calls, against the oracle's output_gate of its attention)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_support import (DEV, TOL_BF16, TOL_F32, Run, bits, decode_workspace, host_values, lib,
                         max_abs_err, oracle_append, oracle_pools)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    lib().version()  # loads libqknr.so; fails loudly when it is not built
    yield
    torch.cuda.empty_cache()


def _workload(dtype, seed):
    return W.build("variants", seed, dtype, num_pages=32, pages_per_row=8, n_table_rows=5,
                   chunks=[(0, 0, 100), (1, 37, 60)], decode=[(2, 10), (3, 200), (4, 0)],
                   decode_row0=2)


@pytest.mark.parametrize("dtype,whole,rotary", [("bf16", True, 0), ("bf16", False, 64),
                                                ("bf16", True, 32), ("bf16", False, 96),
                                                ("bf16", False, 2), ("f32", True, 64)])
def test_append_variants_bit_exact(dtype, whole, rotary):
    Q = lib()
    w = _workload(dtype, 51)
    R = rotary or W.HEAD_DIM
    print(f"append variant {dtype} whole={whole} rotary_dim={R}", flush=True)
    rng = np.random.default_rng(52)
    gq = rng.uniform(0.5, 1.5, (W.NUM_Q_HEADS if whole else 1) * W.HEAD_DIM).astype(np.float32)
    gk = rng.uniform(0.5, 1.5, (W.NUM_KV_HEADS if whole else 1) * W.HEAD_DIM).astype(np.float32)
    cos, sin = Q.rope_table(O.ROPE_THETA, 512, R)
    run = Run(w, keep_pre=False)
    t = run.t
    q_out = torch.empty((w.n_tokens, W.NUM_Q_HEADS * W.HEAD_DIM), dtype=run.td, device=DEV)
    Q.qknorm_rope_append(t["q"], t["k"], t["v"], torch.from_numpy(gq).to(DEV), torch.from_numpy(gk).to(DEV),
                         torch.from_numpy(cos).to(DEV), torch.from_numpy(sin).to(DEV), run.positions_all(),
                         q_out, run.k_pool, run.v_pool, slots=t["slots"], table=t["decode_table"],
                         qk_norm_whole=whole, rotary_dim=rotary)
    torch.cuda.synchronize()
    every_at = np.concatenate([w.positions, w.step_positions]).astype(np.int64)
    oq, ok_, ov = O.append(w.q, w.k, w.v, w.dtype, w.dtype, gq, gk, every_at, norm_whole=whole,
                           rotary_dim=R)
    assert np.array_equal(host_values(q_out, w.dtype), oq)
    _, _, _, every_slot = oracle_append(w)
    sl = torch.from_numpy(every_slot).to(DEV)
    kp = host_values(run.k_pool[:, sl].permute(1, 0, 2).contiguous(), w.dtype)
    vp = host_values(run.v_pool[:, sl].permute(1, 0, 2).contiguous(), w.dtype)
    assert np.array_equal(kp, ok_)
    assert np.array_equal(vp, ov)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_output_gate_decode_prefill_packed(dtype):
    Q = lib()
    w = _workload(dtype, 53)
    print(f"output gate {dtype}", flush=True)
    run = Run(w, keep_pre=False)
    run.append()
    t = run.t
    P, R = w.n_prefill, w.n_decode
    rng = np.random.default_rng(54)
    gate32 = rng.standard_normal((w.n_tokens, W.NUM_Q_HEADS * W.HEAD_DIM)).astype(np.float32)
    gate_host = O.store(gate32, w.dtype)   # the pool dtype's bytes
    gate = torch.from_numpy(gate_host.view(np.int16) if dtype == "bf16" else gate_host).to(DEV)
    if dtype == "bf16":
        gate = gate.view(torch.bfloat16)
    q_out, k_rows, v_rows, every_slot = oracle_append(w)
    kp, vp = oracle_pools(w, k_rows, v_rows, every_slot)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16

    dec = torch.empty((R, W.NUM_Q_HEADS * W.HEAD_DIM), dtype=torch.float32, device=DEV)
    Q.paged_decode_attn(run.q_out[P:], run.k_pool, run.v_pool, t["decode_table"], t["step_positions"],
                        W.SCALE, dec, decode_workspace(run.k_pool, R, w.pages_per_row), gate=gate[P:])
    ref = O.decode(q_out[P:], w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE)
    assert max_abs_err(dec.cpu().numpy(), O.output_gate(ref, gate_host[P:], w.dtype)) <= tol

    pre = torch.empty((P, W.NUM_Q_HEADS * W.HEAD_DIM), dtype=torch.float32, device=DEV)
    ws = torch.zeros(max(1, Q.packed_workspace_bytes(run.k_pool, W.NUM_Q_HEADS, P)), dtype=torch.uint8,
                     device=DEV)
    Q.paged_prefill_attn(run.q_out[:P], run.k_pool, run.v_pool, t["table"], t["rows"], t["positions"],
                         W.SCALE, pre, ws, gate=gate[:P])
    ref = O.prefill(q_out[:P], w.dtype, kp, vp, w.dtype, w.table, w.rows, w.positions, W.SCALE)
    assert max_abs_err(pre.cpu().numpy(), O.output_gate(ref, gate_host[:P], w.dtype)) <= tol

    seg = t["rows"]
    Q.packed_prefill_attn(run.q_out[:P], run.k_pool, run.v_pool, t["table"], t["rows"], t["positions"],
                          seg, W.SCALE, pre, ws, gate=gate[:P])
    ref = O.packed(q_out[:P], w.dtype, k_rows[:P], v_rows[:P], w.dtype, w.rows, w.positions, W.SCALE)
    torch.cuda.synchronize()
    assert max_abs_err(pre.cpu().numpy(), O.output_gate(ref, gate_host[:P], w.dtype)) <= tol


@pytest.mark.parametrize("kv,rotary", [(3, 0), (5, 64), (17, 0), (40, 32)])
def test_whole_norm_append_head_counts(kv, rotary):
    # head counts that are not powers of two (the head sums are added pairwise with
    # an odd one carried up) and above 64 (several sums per lane in the reduction)
    Q = lib()
    w = W.build(f"variants_kv{kv}", 60 + kv, "bf16", num_pages=16, pages_per_row=8, n_table_rows=3,
                chunks=[(0, 0, 40), (1, 9, 30)], decode=[(2, 77)], decode_row0=2, n_kv_heads=kv)
    R = rotary or W.HEAD_DIM
    nq, nk = w.n_q_heads, w.n_kv_heads
    print(f"whole-norm append: {nq} query heads, {nk} KV heads, rotary_dim={R}", flush=True)
    rng = np.random.default_rng(61 + kv)
    gq = rng.uniform(0.5, 1.5, nq * W.HEAD_DIM).astype(np.float32)
    gk = rng.uniform(0.5, 1.5, nk * W.HEAD_DIM).astype(np.float32)
    cos, sin = Q.rope_table(O.ROPE_THETA, 512, R)
    run = Run(w, keep_pre=False)
    t = run.t
    q_out = torch.empty((w.n_tokens, nq * W.HEAD_DIM), dtype=run.td, device=DEV)
    Q.qknorm_rope_append(t["q"], t["k"], t["v"], torch.from_numpy(gq).to(DEV), torch.from_numpy(gk).to(DEV),
                         torch.from_numpy(cos).to(DEV), torch.from_numpy(sin).to(DEV), run.positions_all(),
                         q_out, run.k_pool, run.v_pool, slots=t["slots"], table=t["decode_table"],
                         qk_norm_whole=True, rotary_dim=rotary)
    torch.cuda.synchronize()
    every_at = np.concatenate([w.positions, w.step_positions]).astype(np.int64)
    oq, ok_, ov = O.append(w.q, w.k, w.v, w.dtype, w.dtype, gq, gk, every_at, n_q_heads=nq, n_kv_heads=nk,
                           norm_whole=True, rotary_dim=R)
    assert np.array_equal(host_values(q_out, w.dtype), oq)
    _, _, _, every_slot = oracle_append(w)
    sl = torch.from_numpy(every_slot).to(DEV)
    kp = host_values(run.k_pool[:, sl].permute(1, 0, 2).contiguous(), w.dtype)
    vp = host_values(run.v_pool[:, sl].permute(1, 0, 2).contiguous(), w.dtype)
    assert np.array_equal(kp, ok_)
    assert np.array_equal(vp, ov)

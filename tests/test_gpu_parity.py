"""GPU vs oracle parity through the C ABI, on the five standard workloads at
their full sizes and on small ragged cases.

* q_out and every pool byte: bit-exact (the pool outside the written slots is
  unchanged, the written slots hold the oracle's bytes).
* attention outputs: max abs error <= 1e-4 (float32 pool) or 2e-2 (bfloat16
  K/V, float32 accumulation), on every output of the small workloads and on
  sampled rows / tokens of the large ones.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_support import (DEV, TOL_BF16, TOL_F32, OraclePool, Run, bits, check_append, decode_workspace,
                         host_values, max_abs_err, oracle_append, oracle_pools)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import qk_norm_rope_amd
    qk_norm_rope_amd.version()  # loads libqknr.so; fails loudly when it is not built
    yield
    torch.cuda.empty_cache()


def _tol(w):
    return TOL_F32 if w.dtype == "f32" else TOL_BF16


def _sample(n, k, rng, must=()):
    if n <= k:
        return list(range(n))
    pick = set(int(x) for x in must if 0 <= x < n)
    pick.update(int(x) for x in rng.choice(n, size=k - len(pick), replace=False))
    return sorted(pick)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_standard_workload(cfg):
    w = W.config(cfg)
    print(f"[parity] workload {cfg} {w.name}: P={w.n_prefill} R={w.n_decode}", flush=True)
    run = Run(w)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    check_append(run, ref_q, k_rows, v_rows, slots)
    del run.k_pre, run.v_pre
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    rng = np.random.default_rng(100 + cfg)
    tol = _tol(w)
    P, R = w.n_prefill, w.n_decode
    if R:
        rows = _sample(R, 8, rng, must=[int(np.argmax(w.step_positions)), int(np.argmin(w.step_positions))])
        ref = O.decode(ref_q[P:], w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE,
                       tokens=rows)
        got = run.dec_out[rows].cpu().numpy()
        err = max_abs_err(got, ref)
        print(f"[parity] decode rows {len(rows)} max abs err {err:.3e}", flush=True)
        assert err <= tol
    if P:
        toks = _sample(P, 256, rng, must=[0, P - 1, 2047, 2048, 63, 64, 511, 512, 2535, 2536])
        ref = O.prefill(ref_q[:P], w.dtype, kp, vp, w.dtype, w.table, w.rows, w.positions, W.SCALE,
                        tokens=toks)
        got = run.pre_out[toks].cpu().numpy()
        err = max_abs_err(got, ref)
        print(f"[parity] prefill tokens {len(toks)} max abs err {err:.3e}", flush=True)
        assert err <= tol


def test_prefill_every_token_of_packed_workload():
    # every output of the packed prefill workload, not a sample
    w = W.config(3)
    run = Run(w, keep_pre=False)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    assert np.array_equal(host_values(run.q_out, w.dtype), ref_q)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    ref = O.prefill(ref_q, w.dtype, kp, vp, w.dtype, w.table, w.rows, w.positions, W.SCALE)
    err = max_abs_err(run.pre_out.cpu().numpy(), ref)
    print(f"[parity] packed prefill all tokens max abs err {err:.3e}", flush=True)
    assert err <= TOL_BF16


RAGGED_DECODE = [0, 1, 2, 15, 16, 63, 64, 65, 127, 128, 129, 1000, 4095]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_decode_positions(dtype):
    dec = [(b, p) for b, p in enumerate(RAGGED_DECODE)]
    w = W.build("ragged_decode", 21, dtype, num_pages=512, pages_per_row=64,
                n_table_rows=len(dec), decode=dec)
    run = Run(w)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    check_append(run, ref_q, k_rows, v_rows, slots)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    ref = O.decode(ref_q, w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE)
    err = max_abs_err(run.dec_out.cpu().numpy(), ref)
    print(f"[parity] ragged decode {dtype} max abs err {err:.3e}", flush=True)
    assert err <= _tol(w)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_prefill_chunks(dtype):
    # chunks of odd lengths at odd offsets, several rows inside one 64-token tile,
    # a chunk continuing after history, a single-token chunk
    chunks = [(0, 0, 1), (1, 0, 63), (2, 5, 65), (3, 100, 130), (4, 64, 64), (5, 3, 2), (6, 700, 37)]
    w = W.build("ragged_prefill", 22, dtype, num_pages=256, pages_per_row=16,
                n_table_rows=7, chunks=chunks)
    run = Run(w)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    check_append(run, ref_q, k_rows, v_rows, slots)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    ref = O.prefill(ref_q, w.dtype, kp, vp, w.dtype, w.table, w.rows, w.positions, W.SCALE)
    err = max_abs_err(run.pre_out.cpu().numpy(), ref)
    print(f"[parity] ragged prefill {dtype} max abs err {err:.3e}", flush=True)
    assert err <= _tol(w)


def test_mixed_step_small():
    w = W.build("step_small", 23, "bf16", num_pages=256, pages_per_row=20, n_table_rows=6,
                chunks=[(0, 130, 70), (1, 0, 90)], decode=[(2, 0), (3, 64), (4, 777), (5, 1200)],
                decode_row0=2)
    run = Run(w)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    check_append(run, ref_q, k_rows, v_rows, slots)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    P = w.n_prefill
    ref_p = O.prefill(ref_q[:P], w.dtype, kp, vp, w.dtype, w.table, w.rows, w.positions, W.SCALE)
    ref_d = O.decode(ref_q[P:], w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE)
    assert max_abs_err(run.pre_out.cpu().numpy(), ref_p) <= TOL_BF16
    assert max_abs_err(run.dec_out.cpu().numpy(), ref_d) <= TOL_BF16


def test_negative_slot_skips_the_write():
    w = W.build("skip", 24, "bf16", num_pages=16, pages_per_row=4, n_table_rows=1,
                chunks=[(0, 0, 10)])
    w.slots[3] = -1
    w.slots[7] = -1
    run = Run(w)
    run.append()
    torch.cuda.synchronize()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    check_append(run, ref_q, k_rows, v_rows, slots)


def test_empty_batch_is_a_noop():
    import qk_norm_rope_amd as Q
    w = W.config(1)
    run = Run(w, keep_pre=False)
    from gpu_support import rope_tables
    cos, sin = rope_tables()
    before = run.k_pool.clone()
    e = torch.empty(0, dtype=torch.int32, device=DEV)
    q = torch.empty((0, 4096), dtype=torch.bfloat16, device=DEV)
    kv = torch.empty((0, 1024), dtype=torch.bfloat16, device=DEV)
    Q.qknorm_rope_append(q, kv, kv, run.t["q_gain"], run.t["k_gain"], cos, sin, e, q.clone(),
                         run.k_pool, run.v_pool, slots=e)
    out = torch.empty((0, 4096), dtype=torch.float32, device=DEV)
    Q.paged_decode_attn(q, run.k_pool, run.v_pool, run.t["decode_table"][:0], e, W.SCALE, out,
                        decode_workspace(run.k_pool, 1, w.pages_per_row))
    torch.cuda.synchronize()
    assert torch.equal(bits(before), bits(run.k_pool))


def _permute_pages(run, perm):
    """Move every page p of both pools to page perm[p]; returns the new pools."""
    n = run.w.num_pages
    src = torch.arange(n, device=DEV)
    dst = torch.as_tensor(perm, device=DEV)
    out = []
    for pool in (run.k_pool, run.v_pool):
        pg = pool.view(pool.shape[0], n, 64, pool.shape[2])
        new = torch.empty_like(pg)
        new[:, dst] = pg[:, src]
        out.append(new.view_as(pool))
    return out


def test_shuffled_pages_give_bitwise_equal_outputs():
    w = W.build("shuffle", 25, "bf16", num_pages=300, pages_per_row=40, n_table_rows=6,
                chunks=[(0, 200, 150), (1, 0, 100)], decode=[(2, 5), (3, 900), (4, 2000), (5, 64)],
                decode_row0=2)
    run = Run(w, keep_pre=False)
    run.step()
    perm = np.random.default_rng(5).permutation(w.num_pages)
    kp2, vp2 = _permute_pages(run, perm)
    table2 = torch.as_tensor(perm[w.table], dtype=torch.int32, device=DEV).contiguous()
    import qk_norm_rope_amd as Q
    P = w.n_prefill
    pre2 = torch.empty_like(run.pre_out)
    ws = torch.zeros(Q.prefill_workspace_bytes(kp2, 32, P), dtype=torch.uint8, device=DEV)
    Q.paged_prefill_attn(run.q_out[:P], kp2, vp2, table2, run.t["rows"], run.t["positions"], W.SCALE,
                         pre2, ws)
    dec2 = torch.empty_like(run.dec_out)
    Q.paged_decode_attn(run.q_out[P:], kp2, vp2, table2[2:].contiguous(), run.t["step_positions"],
                        W.SCALE, dec2, decode_workspace(kp2, w.n_decode, w.pages_per_row))
    torch.cuda.synchronize()
    assert torch.equal(pre2, run.pre_out)
    assert torch.equal(dec2, run.dec_out)


def test_decode_split_and_batch_invariance():
    # a row decoded alone (few items, other split) vs inside a large batch
    w = W.config(1)
    run = Run(w, keep_pre=False)
    run.step()
    import qk_norm_rope_amd as Q
    P = w.n_prefill
    for b in (0, 3):
        out1 = torch.empty((1, 4096), dtype=torch.float32, device=DEV)
        Q.paged_decode_attn(run.q_out[P + b:P + b + 1], run.k_pool, run.v_pool,
                            run.t["decode_table"][b:b + 1].contiguous(),
                            run.t["step_positions"][b:b + 1].contiguous(), W.SCALE, out1,
                            decode_workspace(run.k_pool, 1, w.pages_per_row))
        torch.cuda.synchronize()
        diff = (out1[0] - run.dec_out[b]).abs().max().item()
        assert diff <= 1e-5, diff


def test_decode_workspace_is_reusable():
    w = W.config(2)
    run = Run(w, keep_pre=False)
    run.append()
    ws = decode_workspace(run.k_pool, w.n_decode, w.pages_per_row)
    run.decode(ws)
    first = run.dec_out.clone()
    for _ in range(3):
        run.decode(ws)
        torch.cuda.synchronize()
        assert torch.equal(first, run.dec_out)
    # counters are back at zero after every call
    n_pairs = w.n_decode * 8
    assert int(ws[:4 * n_pairs].view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("positions", [[0], [5, 70], [63, 64, 65], [200] * 3])
def test_decode_with_fewer_pages_than_workgroups(positions):
    # far fewer (row, KV head, page) units than resident workgroups: segments cut
    # into single pages, many workgroups with nothing to do
    dec = [(b, p) for b, p in enumerate(positions)]
    w = W.build("few_units", 26, "bf16", num_pages=64, pages_per_row=8, n_table_rows=len(dec),
                decode=dec)
    run = Run(w, keep_pre=False)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    ref = O.decode(ref_q, w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE)
    assert max_abs_err(run.dec_out.cpu().numpy(), ref) <= TOL_BF16


def test_decode_many_short_segments_per_workgroup():
    # 1024 rows of 1-5 pages: each workgroup's slice holds many (row, KV head)
    # segments of odd and even page counts, so every segment's first page is
    # fetched during the previous segment's last page; every output is checked
    rng = np.random.default_rng(47)
    n = 1024
    pos = rng.integers(0, 320, size=n)
    pos[:6] = [0, 63, 64, 127, 128, 319]
    w = W.build("many_segments", 47, "bf16", num_pages=n * 5 + 8, pages_per_row=5, n_table_rows=n,
                decode=[(b, int(p)) for b, p in enumerate(pos)])
    print(f"[parity] {n} decode rows of 1-5 pages", flush=True)
    run = Run(w, keep_pre=False)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    ref = O.decode(ref_q, w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE)
    err = max_abs_err(run.dec_out.cpu().numpy(), ref)
    print(f"[parity] many short segments max abs err {err:.3e}", flush=True)
    assert err <= TOL_BF16

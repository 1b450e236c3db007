"""GPU vs oracle parity through the C ABI, on the five standard workloads at
their full sizes and on small ragged cases.

* q_out and every pool byte: bit-exact (the pool outside the written slots is
  unchanged, the written slots hold the oracle's bytes).
* attention outputs: max abs error <= 1e-4 (float32 pool) or 2e-2 (bfloat16
  K/V, float32 accumulation), on every output; the mean abs error and the count of
  non-finite outputs (required to be 0) are printed beside the max.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_support import (DEV, TOL_BF16, TOL_F32, Run, bits, check_append, decode_workspace, host_values,
                         max_abs_err, oracle_append, oracle_decode, oracle_pools, oracle_prefill, report)

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


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_standard_workload(cfg):
    # every output of every standard workload at its full size
    w = W.config(cfg)
    print(f"[parity] workload {cfg} {w.name}: P={w.n_prefill} R={w.n_decode}", flush=True)
    run = Run(w)
    # the pre-step copy the oracle reads is the generator's: spot-check it against
    # the host regeneration, bit for bit
    hs = w.history_slots()
    if len(hs):
        pick = np.random.default_rng(cfg).choice(hs, size=min(512, len(hs)), replace=False)
        for g in (0, w.n_kv_heads - 1):
            dev = host_values(run.k_pre[g, torch.as_tensor(pick, device=DEV)], w.dtype)
            assert np.array_equal(dev.view(np.uint8), W.host_history(w, 0, g, pick).view(np.uint8))
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    check_append(run, ref_q, k_rows, v_rows, slots)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots, run)
    tol = _tol(w)
    if w.n_decode:
        report(f"workload {cfg} decode", run.dec_out.cpu().numpy(), oracle_decode(w, ref_q, kp, vp), tol)
    if w.n_prefill:
        report(f"workload {cfg} prefill", run.pre_out.cpu().numpy(), oracle_prefill(w, ref_q, kp, vp), tol)


def _scores_log2(ref_q, kp, w, q_row, table_row, pos, head):
    """Scaled scores (log2 units) of one query head over positions 0..pos, float64."""
    q = O.widen(ref_q[q_row], w.dtype).reshape(w.n_q_heads, 128)[head]
    sl = O.row_slots(table_row, pos + 1)
    K = O.widen(kp[head // 4, sl], w.dtype)
    return (K @ q) * W.SCALE * 1.4426950408889634


def test_wide_score_range():
    # large QK-norm gains (uniform in [8, 16]) give scores of hundreds of log2 units:
    # the step's own keys score far above the history's, so a run's running max
    # moves by far more than 8 log2 units after its first page (the prefill kernel
    # then rescales a non-empty accumulator) and decode rows meet their largest
    # score on their last page
    # (a prompt of one page: the page max must cover both halves of each query's
    # keys, which sit in lanes l and l ^ 32, or the exponent overflows)
    w = W.build("wide_scores", 31, "bf16", num_pages=256, pages_per_row=24, n_table_rows=8,
                chunks=[(0, 700, 200), (1, 0, 300), (2, 64, 64), (3, 0, 64)],
                decode=[(4, 0), (5, 130), (6, 1000), (7, 1463)], decode_row0=4, gain_range=(8.0, 16.0))
    run = Run(w)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    check_append(run, ref_q, k_rows, v_rows, slots)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots, run)
    P = w.n_prefill
    # the case exists: token 150 of chunk 0 (position 850) sees its run's first page
    # (positions 0..63, history) far below the chunk's own keys
    s = _scores_log2(ref_q, kp, w, 150, w.table[0], 850, 5)
    jump = s.max() - s[:64].max()
    print(f"[parity] wide scores: range {s.max() - s.min():.0f} log2 units, max above the first page's by "
          f"{jump:.0f}", flush=True)
    assert jump > 8
    report("wide scores prefill", run.pre_out.cpu().numpy(), oracle_prefill(w, ref_q, kp, vp), TOL_BF16)
    report("wide scores decode", run.dec_out.cpu().numpy(), oracle_decode(w, ref_q, kp, vp), TOL_BF16)


def test_decode_every_output_on_a_large_batch():
    # 600 rows of up to 40 pages (192000 units at most): the cost-cut slices cut
    # many segments, with odd and even page counts, and hold many short ones whole
    rng = np.random.default_rng(48)
    n = 600
    pos = rng.integers(0, 40 * 64, size=n)
    pos[:8] = [0, 63, 64, 127, 128, 2559, 2495, 2496]
    w = W.build("large_batch", 48, "bf16", num_pages=n * 40 + 8, pages_per_row=40, n_table_rows=n,
                decode=[(b, int(p)) for b, p in enumerate(pos)])
    print(f"[parity] {n} decode rows of up to 40 pages, every output", flush=True)
    run = Run(w)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    check_append(run, ref_q, k_rows, v_rows, slots)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots, run)
    report("large-batch decode", run.dec_out.cpu().numpy(), oracle_decode(w, ref_q, kp, vp), TOL_BF16)


RAGGED_DECODE = [0, 1, 2, 15, 16, 63, 64, 65, 127, 128, 129, 300, 1000, 3000, 4095]


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
    report(f"ragged decode {dtype}", run.dec_out.cpu().numpy(), ref, _tol(w))


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
    report(f"ragged prefill {dtype}", run.pre_out.cpu().numpy(), ref, _tol(w))


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
    report("small step prefill", run.pre_out.cpu().numpy(), ref_p, TOL_BF16)
    report("small step decode", run.dec_out.cpu().numpy(), ref_d, TOL_BF16)


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


@pytest.mark.parametrize("positions", [[0], [5, 70], [63, 64, 65], [200] * 3, [130, 300, 450]])
def test_decode_with_fewer_pages_than_workgroups(positions):
    # far fewer (row, KV head, page) units than resident workgroups: many workgroups
    # with nothing to do; rows of 1 to 8 pages, odd counts included (a row's last
    # 2-page chunk then holds a single page)
    dec = [(b, p) for b, p in enumerate(positions)]
    w = W.build("few_units", 26, "bf16", num_pages=64, pages_per_row=8, n_table_rows=len(dec),
                decode=dec)
    run = Run(w, keep_pre=False)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    ref = O.decode(ref_q, w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE)
    report(f"few units {positions}", run.dec_out.cpu().numpy(), ref, TOL_BF16)


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
    report("many short segments", run.dec_out.cpu().numpy(), ref, TOL_BF16)


def test_decode_kernel_choice_on_the_standard_workloads():
    # 8 rows take the (row, KV head, 2-page chunk) kernel, 64 and 128 rows the split-K grid
    import qk_norm_rope_amd as Q
    names = {}
    for cfg in (1, 2, 4):
        w = W.config(cfg)
        pool = torch.empty((w.n_kv_heads, 64, 128), dtype=torch.bfloat16, device=DEV)
        names[cfg] = Q.decode_kernel_name(pool, w.n_q_heads, w.n_decode, w.pages_per_row)
    print(f"[parity] decode kernels: {names}", flush=True)
    assert names == {1: "paged_decode_small_kernel", 2: "paged_decode_bf16_kernel", 4: "paged_decode_bf16_kernel"}

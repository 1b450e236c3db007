"""Out-of-range device indices stay inside the buffers (GPU, through the C ABI).

The kernels range-check every index they read from device memory: a page id
outside the pool, a position outside the page table or the rotation table, a
table row outside the table, a slot outside the pool. The token or row that
carries it gets NaN outputs when its position or row is out of range (as with a
float32 pool) and unspecified values for a bad page, and nothing is read or
written outside the buffers. These tests corrupt a few rows and tokens of valid
workloads and check that every other row and token still matches the oracle
bit for bit (q_out, pool bytes) or within the bfloat16 tolerance (attention).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_support import (DEV, TOL_BF16, Run, bits, decode_workspace, host_values, lib, max_abs_err,
                         oracle_append, oracle_pools)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import qk_norm_rope_amd
    qk_norm_rope_amd.version()
    yield
    torch.cuda.empty_cache()


def test_decode_rows_with_bad_pages_and_positions():
    dec = [(b, p) for b, p in enumerate([70, 300, 5, 129, 900, 64, 1000, 33])]
    w = W.build("bad_decode", 51, "bf16", num_pages=256, pages_per_row=16, n_table_rows=8, decode=dec)
    run = Run(w)
    t = run.t
    tab, pos = t["decode_table"], t["step_positions"]
    tab[1, 2] = w.num_pages + 3     # row 1: a page past the pool (its keys are skipped)
    tab[3, 2] = -7                  # row 3: the page of its own position (no write, keys skipped)
    pos[5] = -4                     # row 5: negative position (no rotation, no write, no output)
    pos[7] = 16 * 64 + 10           # row 7: past its table (q_out written, no pool write, no output)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    got_q = host_values(run.q_out, w.dtype)
    for b in (0, 1, 2, 3, 4, 6):   # row 7 was rotated at its corrupted position
        assert np.array_equal(got_q[b], ref_q[b]), f"q_out of row {b}"
    # pool: the written slots of rows 0, 1, 2, 4, 6; rows 3, 5, 7 write nothing
    keep = np.array([b in (0, 1, 2, 4, 6) for b in range(8)])
    exp_k, exp_v = run.k_pre, run.v_pre
    idx = torch.as_tensor(slots[keep], device=DEV)
    for exp, rows in ((exp_k, k_rows), (exp_v, v_rows)):
        rt = torch.from_numpy(rows[keep].view(np.int16)).view(torch.bfloat16).to(DEV)
        exp[:, idx] = rt.permute(1, 0, 2)
    assert torch.equal(bits(run.k_pool), bits(exp_k)), "K pool bytes differ"
    assert torch.equal(bits(run.v_pool), bits(exp_v)), "V pool bytes differ"
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    good = [0, 2, 4, 6]
    ref = O.decode(ref_q, w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE, tokens=good)
    got = run.dec_out[good].cpu().numpy()
    err = max_abs_err(got, ref)
    print(f"[bad] decode: valid rows max abs err {err:.3e}", flush=True)
    assert err <= TOL_BF16
    # a row with an out-of-pool page still attends over its other pages: finite
    assert torch.isfinite(run.dec_out[1]).all()
    # rows whose position is outside the table get NaN outputs (as for a float32
    # pool), written over whatever the output held
    out = torch.zeros_like(run.dec_out)
    lib().paged_decode_attn(run.q_out, run.k_pool, run.v_pool, tab, pos, W.SCALE, out,
                            decode_workspace(run.k_pool, w.n_decode, w.pages_per_row))
    torch.cuda.synchronize()
    assert torch.isnan(out[5]).all() and torch.isnan(out[7]).all()
    assert torch.isfinite(out[[0, 1, 2, 3, 4, 6]]).all()


def test_prefill_tokens_with_bad_rows_positions_and_pages():
    chunks = [(0, 0, 70), (1, 30, 50), (2, 0, 20), (3, 0, 10)]
    w = W.build("bad_prefill", 52, "bf16", num_pages=128, pages_per_row=4, n_table_rows=4, chunks=chunks)
    run = Run(w, keep_pre=False)
    t = run.t
    t["table"][1, 1] = w.num_pages + 1   # row 1 (tokens 70..119): a page past the pool
    t["positions"][125] = -3             # row 2: a negative position
    t["positions"][130] = 10 ** 6        # row 2: past the table and the rotation table
    t["rows"][145] = 99                  # row 3: a table row that does not exist
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    got_q = host_values(run.q_out, w.dtype)
    skipped = {125, 130}                 # no rotation exists for them: q_out is not written
    ok = [i for i in range(w.n_prefill) if i not in skipped]
    assert np.array_equal(got_q[ok], ref_q[ok]), "q_out of the valid tokens"
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    good = list(range(0, 70)) + [i for i in range(140, 150) if i != 145]
    ref = O.prefill(ref_q, w.dtype, kp, vp, w.dtype, w.table, w.rows, w.positions, W.SCALE, tokens=good)
    got = run.pre_out[good].cpu().numpy()
    err = max_abs_err(got, ref)
    print(f"[bad] prefill: {len(good)} valid tokens max abs err {err:.3e}", flush=True)
    assert err <= TOL_BF16
    # tokens with an out-of-range position or row get NaN outputs (as for a float32 pool)
    out = torch.zeros_like(run.pre_out)
    ws = torch.zeros(lib().prefill_workspace_bytes(run.k_pool, 32, w.n_prefill), dtype=torch.uint8, device=DEV)
    lib().paged_prefill_attn(run.q_out, run.k_pool, run.v_pool, t["table"], t["rows"], t["positions"], W.SCALE,
                             out, ws)
    torch.cuda.synchronize()
    assert torch.isnan(out[[125, 130, 145]]).all()
    assert torch.isfinite(out[good]).all()


def test_decode_large_batch_with_rows_outside_their_tables():
    # a batch for the split-K kernel (200 rows of up to 40 pages) whose positions
    # put some rows outside their tables: the first and the last row, a run of
    # three, and scattered ones. Such rows hold no pages but keep their per-segment
    # charge on the slices' cost scale; every other row must still match the oracle
    # and the bad rows must come out NaN
    rng = np.random.default_rng(53)
    n, ppr = 200, 40
    pos = rng.integers(0, ppr * 64, size=n)
    w = W.build("bad_large", 53, "bf16", num_pages=n * ppr + 8, pages_per_row=ppr, n_table_rows=n,
                decode=[(b, int(p)) for b, p in enumerate(pos)])
    import qk_norm_rope_amd as Q
    assert Q.decode_kernel_name(torch.empty((8, 64, 128), dtype=torch.bfloat16, device=DEV), 32, n,
                                ppr) == "paged_decode_bf16_kernel"
    run = Run(w, keep_pre=False)
    bad = [0, 17, 18, 19, 77, 150, n - 1]
    for b in bad:
        run.t["step_positions"][b] = -1 if b % 2 else ppr * 64 + 5
    print(f"[bad] {n} decode rows, {len(bad)} of them outside their tables", flush=True)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    good = [b for b in range(n) if b not in bad]
    ref = O.decode(ref_q, w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE, tokens=good)
    got = run.dec_out[good].cpu().numpy()
    err = max_abs_err(got, ref)
    print(f"[bad] large batch: valid rows max abs err {err:.3e}", flush=True)
    assert err <= TOL_BF16
    assert torch.isnan(run.dec_out[bad]).all()

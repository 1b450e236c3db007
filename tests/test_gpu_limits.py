"""Parity at the library's size limits, on the GPU through the C ABI.

* decode: the most rows one call takes (12288; the launcher keeps a prefix table
  of the rows in LDS), with the doubled workgroup grid of large batches;
* the longest page table (2048 pages, positions up to 131071): a prompt chunk on
  the last page of its row (prefill work items of 2048 pages) and a decode row at
  position 131071, whose 16384 units are split over ~1000 workgroups so that each
  of its segments merges ~128 partial softmax states.
q_out is compared bit for bit with the oracle; attention outputs within the
bfloat16 tolerance (2e-2 max abs error), on sampled rows and tokens.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_support import DEV, TOL_BF16, Run, host_values, lib, max_abs_err, oracle_append, oracle_pools

pytestmark = pytest.mark.gpu

MAX_DECODE_ROWS = 12288
MAX_PAGES_PER_ROW = 2048


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import qk_norm_rope_amd
    qk_norm_rope_amd.version()
    yield
    torch.cuda.empty_cache()


def test_decode_at_the_row_limit():
    rng = np.random.default_rng(41)
    pos = rng.integers(0, 200, size=MAX_DECODE_ROWS)
    pos[:4] = [0, 63, 64, 199]
    w = W.build("limit_rows", 41, "bf16", num_pages=MAX_DECODE_ROWS * 4 + 8, pages_per_row=4,
                n_table_rows=MAX_DECODE_ROWS, decode=[(b, int(p)) for b, p in enumerate(pos)])
    print(f"[limits] {MAX_DECODE_ROWS} decode rows", flush=True)
    run = Run(w, keep_pre=False)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    assert np.array_equal(host_values(run.q_out, w.dtype), ref_q), "q_out bytes differ"
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    rows = sorted(set([0, 1, 2, 3, MAX_DECODE_ROWS - 1] + [int(x) for x in rng.choice(MAX_DECODE_ROWS, 19, replace=False)]))
    ref = O.decode(ref_q, w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE, tokens=rows)
    err = max_abs_err(run.dec_out[rows].cpu().numpy(), ref)
    print(f"[limits] decode rows {len(rows)} max abs err {err:.3e}", flush=True)
    assert err <= TOL_BF16


def test_prefill_and_decode_at_the_page_table_limit():
    last = MAX_PAGES_PER_ROW * W.PAGE_SIZE   # positions 0 .. last-1
    w = W.build("limit_pages", 42, "bf16", num_pages=2 * MAX_PAGES_PER_ROW + 8,
                pages_per_row=MAX_PAGES_PER_ROW, n_table_rows=2,
                chunks=[(0, last - 64, 64)], decode=[(1, last - 1)], decode_row0=1)
    print(f"[limits] {MAX_PAGES_PER_ROW} pages per row: prompt chunk at {last - 64}..{last - 1}, "
          f"decode row at {last - 1}", flush=True)
    run = Run(w, keep_pre=False)
    # a rotation table that reaches the last position (the standard one stops at
    # the model's 40960 positions, and the append skips tokens beyond its table)
    cos, sin = lib().rope_table(O.ROPE_THETA, last, W.HEAD_DIM)
    run.rope = (torch.from_numpy(cos).to(DEV), torch.from_numpy(sin).to(DEV))
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    assert np.array_equal(host_values(run.q_out, w.dtype), ref_q), "q_out bytes differ"
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    ref_d = O.decode(ref_q[64:], w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE)
    err = max_abs_err(run.dec_out.cpu().numpy(), ref_d)
    print(f"[limits] decode at position {last - 1}: max abs err {err:.3e}", flush=True)
    assert err <= TOL_BF16
    toks = [0, 63]
    ref_p = O.prefill(ref_q[:64], w.dtype, kp, vp, w.dtype, w.table, w.rows, w.positions, W.SCALE, tokens=toks)
    err = max_abs_err(run.pre_out[toks].cpu().numpy(), ref_p)
    print(f"[limits] prefill tokens {toks}: max abs err {err:.3e}", flush=True)
    assert err <= TOL_BF16

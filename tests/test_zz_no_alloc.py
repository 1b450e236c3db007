"""paged_decode_attn_noalloc (no workspace argument, no allocation: the library's
own per-GPU scratch) against paged_decode_attn with a caller workspace, through
the C ABI: the same kernel and split, so the outputs must be bitwise equal, on
calls in a row that reuse the scratch, the later ones with fewer rows."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_support import DEV, TOL_BF16, TOL_F32, Run, decode_workspace, max_abs_err, oracle_append, oracle_pools

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import qk_norm_rope_amd
    qk_norm_rope_amd.version()
    yield
    torch.cuda.empty_cache()


def _both(run, rows):
    """Decode of the first `rows` rows through both entry points."""
    import qk_norm_rope_amd as Q
    w, t = run.w, run.t
    P = w.n_prefill
    nq = w.n_q_heads * W.HEAD_DIM
    q = run.q_out[P:P + rows]
    table = t["decode_table"][:rows].contiguous()
    pos = t["step_positions"][:rows].contiguous()
    ref = torch.full((rows, nq), float("nan"), dtype=torch.float32, device=DEV)
    got = torch.full((rows, nq), float("nan"), dtype=torch.float32, device=DEV)
    Q.paged_decode_attn(q, run.k_pool, run.v_pool, table, pos, W.SCALE, ref,
                        decode_workspace(run.k_pool, rows, w.pages_per_row))
    Q.paged_decode_attn_noalloc(q, run.k_pool, run.v_pool, table, pos, W.SCALE, got)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_workspace_call_on_consecutive_calls():
    # first call: 64 ragged rows (cost-cut slices, many cut segments and
    # merges); then 8 rows, then 3 of them, on the scratch the first call left behind
    big = W.config(2)
    print(f"[noalloc] {big.name}: {big.n_decode} rows", flush=True)
    run_big = Run(big, keep_pre=False)
    run_big.append()
    ref, got = _both(run_big, big.n_decode)
    assert torch.equal(ref, got), "64 rows: outputs differ"
    del run_big, ref, got
    torch.cuda.empty_cache()

    small = W.config(1)
    print(f"[noalloc] {small.name}: {small.n_decode} rows, then 3", flush=True)
    run = Run(small, keep_pre=False)
    run.append()
    ref8, got8 = _both(run, small.n_decode)
    assert torch.equal(ref8, got8), "8 rows: outputs differ"
    ref3, got3 = _both(run, 3)
    assert torch.equal(ref3, got3), "3 rows: outputs differ"
    # and both agree with the oracle
    ref_q, k_rows, v_rows, slots = oracle_append(small)
    kp, vp = oracle_pools(small, k_rows, v_rows, slots)
    exp = O.decode(ref_q, small.dtype, kp, vp, small.dtype, small.decode_table, small.step_positions, W.SCALE)
    err = max_abs_err(got8.cpu().numpy(), exp)
    print(f"[noalloc] 8 rows vs oracle max abs err {err:.3e}", flush=True)
    assert err <= TOL_BF16
    # 3 rows split the work differently from 8: equal up to float32 rounding
    assert (got3 - got8[:3]).abs().max().item() <= 1e-5


def test_noalloc_float32_pool():
    w = W.config(0)
    run = Run(w, keep_pre=False)
    run.append()
    ref, got = _both(run, 1)
    assert torch.equal(ref, got)
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    exp = O.decode(ref_q, w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE)
    assert max_abs_err(got.cpu().numpy(), exp) <= TOL_F32


def test_noalloc_rejects_batches_beyond_the_scratch():
    import qk_norm_rope_amd as Q
    from qk_norm_rope_amd import _lib as L
    # 16 KV heads (64 query heads): the scratch holds 6144 rows
    rows = L.NOALLOC_MAX_ROW_HEADS // 16 + 1
    k_pool = torch.zeros((16, 64, 128), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((rows, 64 * 128), dtype=torch.bfloat16, device=DEV)
    table = torch.zeros((rows, 1), dtype=torch.int32, device=DEV)
    pos = torch.zeros(rows, dtype=torch.int32, device=DEV)
    out = torch.zeros((rows, 64 * 128), dtype=torch.float32, device=DEV)
    with pytest.raises(Q.QknrError) as e:
        Q.paged_decode_attn_noalloc(q, k_pool, k_pool, table, pos, W.SCALE, out)
    assert e.value.status == -2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert int(out.abs().sum().item()) == 0   # nothing ran

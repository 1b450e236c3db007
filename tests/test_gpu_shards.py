"""One GPU's share of the step when the heads are sharded over S GPUs (nest
"models/qwen3-8b/files", README Shards paragraph: heads and KV heads split over
the devices). GPU s holds 8/S KV heads, their 4 query heads each, and its slice of
both pools; the library takes the head counts at run time, so the path runs
unchanged at 1, 2 or 4 KV heads. Checked against the oracle at those shapes:
q_out and every pool byte bit for bit, attention within the bfloat16 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_support import TOL_BF16, Run, check_append, host_values, max_abs_err, oracle_append, oracle_pools

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import qk_norm_rope_amd
    qk_norm_rope_amd.version()
    yield
    torch.cuda.empty_cache()


def _heads(w):
    return {"n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads}


@pytest.mark.parametrize("kv", [1, 2, 4])
def test_mixed_step_at_a_shard_shape(kv):
    w = W.build("shard_step", 60 + kv, "bf16", num_pages=256, pages_per_row=20, n_table_rows=8,
                chunks=[(0, 130, 70), (1, 0, 90), (2, 5, 3)],
                decode=[(3, 0), (4, 63), (5, 64), (6, 777), (7, 1200)], decode_row0=3, n_kv_heads=kv)
    print(f"[shard] {kv} KV heads, {w.n_q_heads} query heads: P={w.n_prefill} R={w.n_decode}", flush=True)
    run = Run(w)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    check_append(run, ref_q, k_rows, v_rows, slots)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    P = w.n_prefill
    ref_p = O.prefill(ref_q[:P], w.dtype, kp, vp, w.dtype, w.table, w.rows, w.positions, W.SCALE, **_heads(w))
    ref_d = O.decode(ref_q[P:], w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE,
                     **_heads(w))
    ep = max_abs_err(run.pre_out.cpu().numpy(), ref_p)
    ed = max_abs_err(run.dec_out.cpu().numpy(), ref_d)
    print(f"[shard] prefill err {ep:.3e} decode err {ed:.3e}", flush=True)
    assert ep <= TOL_BF16 and ed <= TOL_BF16


def test_standard_step_one_kv_head():
    # the mixed-step workload as one of 8 shards: same rows, positions and pages, 1 KV head
    w = W.config(4, kv_heads=1)
    run = Run(w, keep_pre=False)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    assert np.array_equal(host_values(run.q_out, w.dtype), ref_q), "q_out bytes differ"
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    rng = np.random.default_rng(64)
    P, R = w.n_prefill, w.n_decode
    rows = sorted(set([int(np.argmax(w.step_positions))] + [int(x) for x in rng.choice(R, 7, replace=False)]))
    ref_d = O.decode(ref_q[P:], w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE,
                     tokens=rows, **_heads(w))
    ed = max_abs_err(run.dec_out[rows].cpu().numpy(), ref_d)
    toks = sorted(set([0, 2047, 2048, P - 1] + [int(x) for x in rng.choice(P, 60, replace=False)]))
    ref_p = O.prefill(ref_q[:P], w.dtype, kp, vp, w.dtype, w.table, w.rows, w.positions, W.SCALE,
                      tokens=toks, **_heads(w))
    ep = max_abs_err(run.pre_out[toks].cpu().numpy(), ref_p)
    print(f"[shard] step at 1 KV head: decode rows {len(rows)} err {ed:.3e}, prefill tokens {len(toks)} "
          f"err {ep:.3e}", flush=True)
    assert ed <= TOL_BF16 and ep <= TOL_BF16

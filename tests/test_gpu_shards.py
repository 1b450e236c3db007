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
from gpu_support import (TOL_BF16, Run, check_append, oracle_append, oracle_decode, oracle_pools, oracle_prefill,
                         report)

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
    report(f"shard {kv} KV heads prefill", run.pre_out.cpu().numpy(), ref_p, TOL_BF16)
    report(f"shard {kv} KV heads decode", run.dec_out.cpu().numpy(), ref_d, TOL_BF16)


def test_standard_step_one_kv_head():
    # the mixed-step workload as one of 8 shards: same rows, positions and pages,
    # 1 KV head; every output
    w = W.config(4, kv_heads=1)
    run = Run(w)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    check_append(run, ref_q, k_rows, v_rows, slots)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots, run)
    report("step at 1 KV head decode", run.dec_out.cpu().numpy(), oracle_decode(w, ref_q, kp, vp), TOL_BF16)
    report("step at 1 KV head prefill", run.pre_out.cpu().numpy(), oracle_prefill(w, ref_q, kp, vp), TOL_BF16)

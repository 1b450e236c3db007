"""Prefill passes with more tiles than one wave plans (nest "models/qwen3-8b/files",
Entries table, prefill_paged: prompts packed end to end, each token attending over
its row's pages up to its position).

Up to 64 tiles of 64 tokens, one wave sorts the tiles by cost and assigns key
splits; above that the whole planning workgroup sorts and scans, above 512 tiles
the plan orders tiles without splitting any, and above 8192 tiles there is no plan
(tiles run in pack order). These cases run those paths at 8 KV heads and at 1 KV
head (one GPU's share of heads sharded 8 ways). The pool bytes are checked bit for
bit; attention outputs within the bfloat16 tolerance on sampled tokens that include
the first and last token of every prompt (of the first and last few prompts when
there are many), so the longest tiles (the first ones in the plan's order) are
covered.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_support import TOL_BF16, Run, check_append, max_abs_err, oracle_append, oracle_pools

pytestmark = pytest.mark.gpu

# (row, first position, length): 8360 tokens = 131 tiles; one prompt continues a
# row at position 500 (its history is in the pool), tiles straddle prompts
CHUNKS_131 = [(0, 0, 1560), (1, 0, 3000), (2, 500, 900), (3, 0, 2900)]
# 33000 tokens = 516 tiles
CHUNKS_516 = [(0, 0, 8250), (1, 0, 8250), (2, 0, 8250), (3, 0, 8250)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import qk_norm_rope_amd
    qk_norm_rope_amd.version()
    yield
    torch.cuda.empty_cache()


def _check(w, chunks, seed, n_random, max_ends=None):
    run = Run(w)
    run.step()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    check_append(run, ref_q, k_rows, v_rows, slots)
    del run.k_pre, run.v_pre
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    P = w.n_prefill
    ends, start = [], 0
    for _, _, n in chunks:
        ends += [start, start + n - 1]
        start += n
    if max_ends is not None and len(ends) > max_ends:
        ends = ends[:max_ends // 2] + ends[-(max_ends // 2):]
    rng = np.random.default_rng(seed)
    toks = sorted(set(ends + [int(x) for x in rng.choice(P, n_random, replace=False)]))
    ref = O.prefill(ref_q[:P], w.dtype, kp, vp, w.dtype, w.table, w.rows, w.positions, W.SCALE, tokens=toks,
                    n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads)
    err = max_abs_err(run.pre_out[toks].cpu().numpy(), ref)
    print(f"[many tiles] {w.name}: {(P + 63) // 64} tiles, {w.n_kv_heads} KV heads, {len(toks)} tokens, "
          f"max abs err {err:.3e}", flush=True)
    assert err <= TOL_BF16


@pytest.mark.parametrize("kv", [8, 1])
def test_prefill_with_131_tiles(kv):
    w = W.build(f"many_tiles_131_kv{kv}", 70 + kv, "bf16", num_pages=512, pages_per_row=64, n_table_rows=4,
                chunks=CHUNKS_131, n_kv_heads=kv)
    print(f"[many tiles] P={w.n_prefill}, {kv} KV heads", flush=True)
    _check(w, CHUNKS_131, 170 + kv, 56)


def test_prefill_with_516_tiles():
    w = W.build("many_tiles_516", 81, "bf16", num_pages=1024, pages_per_row=160, n_table_rows=4,
                chunks=CHUNKS_516)
    print(f"[many tiles] P={w.n_prefill}, 8 KV heads", flush=True)
    _check(w, CHUNKS_516, 181, 40)


def test_prefill_with_8200_tiles_without_a_plan():
    # 128 prompts of 4100 tokens (524800 tokens, 8200 tiles) at 1 KV head
    chunks = [(r, 0, 4100) for r in range(128)]
    w = W.build("many_tiles_8200", 91, "bf16", num_pages=8400, pages_per_row=65, n_table_rows=128,
                chunks=chunks, n_kv_heads=1)
    print(f"[many tiles] P={w.n_prefill}, 1 KV head", flush=True)
    _check(w, chunks, 191, 40, max_ends=16)

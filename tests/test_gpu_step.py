"""step_paged (the whole mixed step in one launch) against the three-call
composition and the oracle, through the C ABI.

* q_out and every pool byte: bit-exact with the composition (whose bytes the
  oracle pins in test_gpu_parity) and with the oracle's append.
* prefill_out: bit-exact with paged_prefill_attn (the same work items).
* decode_out: within the bfloat16 tolerance of the oracle (2e-2 max abs error),
  and within 1e-4 of paged_decode_attn (the page ranges are split differently,
  so only float32 rounding differs).
* the workspace's control words are zero again after every call, and the
  bounded wait never gave up.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_support import (DEV, TOL_BF16, Run, bits, host_values, max_abs_err, oracle_append,
                         oracle_pools, step_workspace)

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="step_paged's kernel is switched off: an earlier form hung on the GPU "
                            "(its ticket loop was compiled into a nest where only thread 0 took new "
                            "tickets); the corrected form has not run on a GPU yet"),
]

SPLIT_TOL = 1e-4   # decode: fused step vs paged_decode_attn, same inputs


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import qk_norm_rope_amd
    qk_norm_rope_amd.version()
    yield
    torch.cuda.empty_cache()


def _control_words_clear(ws):
    words = ws[:64 * 4].view(torch.int32).cpu().numpy()
    assert words[5] == 0, f"a workgroup gave up waiting for the writes (saw {words[6]}, {words[7]})"
    assert not words.any(), f"control words not cleared: {words[:8]}"


def _compare(w, fused, ref, oracle_rows=8, seed=0, oracle=True):
    """fused vs composition (bitwise / split tolerance) and decode vs the oracle."""
    P, R = w.n_prefill, w.n_decode
    assert torch.equal(bits(fused.q_out), bits(ref.q_out)), "q_out differs from the composition"
    assert torch.equal(bits(fused.k_pool), bits(ref.k_pool)), "K pool differs from the composition"
    assert torch.equal(bits(fused.v_pool), bits(ref.v_pool)), "V pool differs from the composition"
    if P:
        assert torch.equal(bits(fused.pre_out), bits(ref.pre_out)), "prefill_out differs"
    if R:
        d = float((fused.dec_out - ref.dec_out).abs().max())
        print(f"[step] decode fused vs three calls max abs diff {d:.3e}", flush=True)
        assert d <= SPLIT_TOL
        if not oracle:
            return
        ref_q, k_rows, v_rows, slots = oracle_append(w)
        assert np.array_equal(host_values(fused.q_out, w.dtype), ref_q)
        kp, vp = oracle_pools(w, k_rows, v_rows, slots)
        rng = np.random.default_rng(seed)
        rows = sorted(set([int(np.argmax(w.step_positions)), int(np.argmin(w.step_positions))]
                          + [int(x) for x in rng.choice(R, size=min(R, oracle_rows), replace=False)]))
        ref_d = O.decode(ref_q[P:], w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE,
                         tokens=rows)
        err = max_abs_err(fused.dec_out[rows].cpu().numpy(), ref_d)
        print(f"[step] decode rows {len(rows)} vs oracle max abs err {err:.3e}", flush=True)
        assert err <= TOL_BF16


def _pair(w):
    ref = Run(w, keep_pre=False)
    ref.step()
    fused = Run(w, keep_pre=False)
    ws = step_workspace(fused.k_pool, w.n_prefill, w.n_decode, w.pages_per_row)
    fused.fused_step(ws)
    torch.cuda.synchronize()
    _control_words_clear(ws)
    return fused, ref, ws


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_step_matches_three_calls_on_standard_workloads(cfg):
    w = W.config(cfg)
    print(f"[step] workload {cfg} {w.name}: P={w.n_prefill} R={w.n_decode}", flush=True)
    fused, ref, _ = _pair(w)
    _compare(w, fused, ref, seed=200 + cfg)


def test_step_small_mixed_against_the_oracle_everywhere():
    # several rows inside one tile, a chunk after history, decode rows at page edges
    w = W.build("step_small", 31, "bf16", num_pages=256, pages_per_row=20, n_table_rows=8,
                chunks=[(0, 130, 70), (1, 0, 90), (2, 5, 3)],
                decode=[(3, 0), (4, 63), (5, 64), (6, 777), (7, 1200)], decode_row0=3)
    fused = Run(w, keep_pre=False)
    fused.fused_step()
    torch.cuda.synchronize()
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    assert np.array_equal(host_values(fused.q_out, w.dtype), ref_q)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    P = w.n_prefill
    ref_p = O.prefill(ref_q[:P], w.dtype, kp, vp, w.dtype, w.table, w.rows, w.positions, W.SCALE)
    ref_d = O.decode(ref_q[P:], w.dtype, kp, vp, w.dtype, w.decode_table, w.step_positions, W.SCALE)
    ep = max_abs_err(fused.pre_out.cpu().numpy(), ref_p)
    ed = max_abs_err(fused.dec_out.cpu().numpy(), ref_d)
    print(f"[step] small mixed: prefill err {ep:.3e} decode err {ed:.3e}", flush=True)
    assert ep <= TOL_BF16 and ed <= TOL_BF16


def test_step_decode_only_and_prefill_only():
    dec = W.build("step_dec", 32, "bf16", num_pages=512, pages_per_row=64, n_table_rows=13,
                  decode=[(b, p) for b, p in enumerate([0, 1, 2, 15, 16, 63, 64, 65, 127, 128, 129, 1000, 4095])])
    fused, ref, _ = _pair(dec)
    _compare(dec, fused, ref, oracle_rows=13)
    pre = W.build("step_pre", 33, "bf16", num_pages=256, pages_per_row=16, n_table_rows=7,
                  chunks=[(0, 0, 1), (1, 0, 63), (2, 5, 65), (3, 100, 130), (4, 64, 64), (5, 3, 2), (6, 700, 37)])
    fused, ref, _ = _pair(pre)
    _compare(pre, fused, ref)


def test_step_workspace_reused_by_a_smaller_step():
    big = W.build("step_big", 34, "bf16", num_pages=1024, pages_per_row=40, n_table_rows=12,
                  chunks=[(0, 512, 700), (1, 0, 300)], decode=[(2 + b, 97 * b + 5) for b in range(10)],
                  decode_row0=2)
    small = W.build("step_little", 35, "bf16", num_pages=1024, pages_per_row=40, n_table_rows=5,
                    chunks=[(0, 0, 40)], decode=[(1, 3), (2, 640), (3, 64), (4, 2000)], decode_row0=1)
    ws = step_workspace(Run(big, keep_pre=False).k_pool, big.n_prefill, big.n_decode, big.pages_per_row)
    for w in (big, small, small):
        fused = Run(w, keep_pre=False)
        fused.fused_step(ws)
        torch.cuda.synchronize()
        _control_words_clear(ws)
        ref = Run(w, keep_pre=False)
        ref.step()
        _compare(w, fused, ref)


def test_step_without_the_tile_plan():
    # more tiles than the in-kernel plan sorts: tiles run in pack order
    n_rows = 1030
    w = W.build("step_many_tiles", 36, "bf16", num_pages=2048, pages_per_row=2, n_table_rows=n_rows + 2,
                chunks=[(r, 0, 64) for r in range(n_rows)], decode=[(n_rows, 70), (n_rows + 1, 5)],
                decode_row0=n_rows)
    assert (w.n_prefill + 63) // 64 > 1024
    fused, ref, _ = _pair(w)
    _compare(w, fused, ref, oracle=False)   # the composition's bytes are oracle-pinned elsewhere

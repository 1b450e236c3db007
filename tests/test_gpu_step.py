"""step_paged (the whole mixed step in one launch) against the three-call
composition and the oracle, through the C ABI.

* q_out and every pool byte: bit-exact with the composition (qknorm_rope_append
  then paged_prefill_attn and paged_decode_attn), whose bytes test_gpu_parity
  pins to the oracle.
* prefill_out and decode_out: every output within the bfloat16 tolerance of the
  oracle (2e-2 max abs error, no NaN). Against the composition: decode within
  1e-4 (its page ranges are split differently, so only float32 rounding
  differs); prefill within the bfloat16 tolerance (the composition's plan may
  split a long tile's keys over several workgroups and merge them, which rounds
  the bfloat16 probabilities against other maxima), and bitwise when it does not
  split (the standard workloads at 8 KV heads).
* the workspace's control words are zero again after every call, and the
  bounded wait never gave up.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_support import (TOL_BF16, Run, bits, oracle_append, oracle_decode, oracle_pools, oracle_prefill, report,
                         step_workspace)

pytestmark = pytest.mark.gpu

SPLIT_TOL = 1e-4   # decode: fused step vs paged_decode_attn, same inputs


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import qk_norm_rope_amd
    qk_norm_rope_amd.version()
    yield
    torch.cuda.empty_cache()


CTL_INTS = 64 + 256 * 8   # the control area: 64 words, then 8 append counters 256 ints apart


def _control_words_clear(ws):
    words = ws[:CTL_INTS * 4].view(torch.int32).cpu().numpy()
    assert words[5] == 0, f"a workgroup gave up waiting for the writes (saw {words[6]}, {words[7]})"
    assert not words.any(), f"control words not cleared: {words[:8]}, counters {words[64::256]}"


def _fused(w, ws=None, keep_pre=True):
    fused = Run(w, keep_pre=keep_pre)
    if ws is None:
        ws = step_workspace(fused.k_pool, w.n_prefill, w.n_decode, w.pages_per_row)
    print(f"[step] {w.name}: P={w.n_prefill} R={w.n_decode}, one launch", flush=True)
    fused.fused_step(ws)
    torch.cuda.synchronize()
    _control_words_clear(ws)
    return fused, ws


def _compare(w, fused, prefill_bitwise=False, oracle=True):
    """fused vs the three calls (bitwise / rounding bounds) and every output vs the oracle."""
    ref = Run(w, keep_pre=False)
    ref.step()
    P, R = w.n_prefill, w.n_decode
    assert torch.equal(bits(fused.q_out), bits(ref.q_out)), "q_out differs from the composition"
    assert torch.equal(bits(fused.k_pool), bits(ref.k_pool)), "K pool differs from the composition"
    assert torch.equal(bits(fused.v_pool), bits(ref.v_pool)), "V pool differs from the composition"
    if P:
        d = float((fused.pre_out - ref.pre_out).abs().max())
        print(f"[step] prefill fused vs three calls max abs diff {d:.3e}", flush=True)
        if prefill_bitwise:
            assert torch.equal(bits(fused.pre_out), bits(ref.pre_out)), "prefill_out differs"
        assert d <= TOL_BF16
    if R:
        d = float((fused.dec_out - ref.dec_out).abs().max())
        print(f"[step] decode fused vs three calls max abs diff {d:.3e}", flush=True)
        assert d <= SPLIT_TOL
    del ref
    if not oracle:
        return
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots, fused)
    if P:
        report(f"step {w.name} prefill", fused.pre_out.cpu().numpy(), oracle_prefill(w, ref_q, kp, vp), TOL_BF16)
    if R:
        report(f"step {w.name} decode", fused.dec_out.cpu().numpy(), oracle_decode(w, ref_q, kp, vp), TOL_BF16)


def test_step_small_mixed():
    # several rows inside one tile, a chunk after history, decode rows at page edges
    w = W.build("step_small", 31, "bf16", num_pages=256, pages_per_row=20, n_table_rows=8,
                chunks=[(0, 130, 70), (1, 0, 90), (2, 5, 3)],
                decode=[(3, 0), (4, 63), (5, 64), (6, 777), (7, 1200)], decode_row0=3)
    fused, _ = _fused(w)
    _compare(w, fused)


def test_step_decode_only_and_prefill_only():
    dec = W.build("step_dec", 32, "bf16", num_pages=512, pages_per_row=64, n_table_rows=13,
                  decode=[(b, p) for b, p in enumerate([0, 1, 2, 15, 16, 63, 64, 65, 127, 128, 129, 1000, 4095])])
    fused, _ = _fused(dec)
    _compare(dec, fused)
    pre = W.build("step_pre", 33, "bf16", num_pages=256, pages_per_row=16, n_table_rows=7,
                  chunks=[(0, 0, 1), (1, 0, 63), (2, 5, 65), (3, 100, 130), (4, 64, 64), (5, 3, 2), (6, 700, 37)])
    fused, _ = _fused(pre)
    _compare(pre, fused)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_step_on_standard_workloads(cfg):
    w = W.config(cfg)
    fused, _ = _fused(w)
    _compare(w, fused, prefill_bitwise=True)


def test_step_workspace_reused_by_a_smaller_step():
    big = W.build("step_big", 34, "bf16", num_pages=1024, pages_per_row=40, n_table_rows=12,
                  chunks=[(0, 512, 700), (1, 0, 300)], decode=[(2 + b, 97 * b + 5) for b in range(10)],
                  decode_row0=2)
    small = W.build("step_little", 35, "bf16", num_pages=1024, pages_per_row=40, n_table_rows=5,
                    chunks=[(0, 0, 40)], decode=[(1, 3), (2, 640), (3, 64), (4, 2000)], decode_row0=1)
    ws = None
    for w in (big, small, small):
        fused, ws = _fused(w, ws)
        _compare(w, fused)


def test_step_without_the_tile_plan():
    # more tiles than the in-kernel plan sorts: tiles run in pack order
    n_rows = 1030
    w = W.build("step_many_tiles", 36, "bf16", num_pages=2048, pages_per_row=2, n_table_rows=n_rows + 2,
                chunks=[(r, 0, 64) for r in range(n_rows)], decode=[(n_rows, 70), (n_rows + 1, 5)],
                decode_row0=n_rows)
    assert (w.n_prefill + 63) // 64 > 1024
    fused, _ = _fused(w, keep_pre=False)
    _compare(w, fused, oracle=False)   # the composition's outputs are oracle-checked in test_gpu_parity
    # the decode rows against the oracle
    ref_q, k_rows, v_rows, slots = oracle_append(w)
    kp, vp = oracle_pools(w, k_rows, v_rows, slots)
    report("step without plan decode", fused.dec_out.cpu().numpy(), oracle_decode(w, ref_q, kp, vp), TOL_BF16)
    P = w.n_prefill
    toks = sorted(set([0, 63, 64, P - 1] + list(np.random.default_rng(36).choice(P, 200, replace=False))))
    report("step without plan prefill (200 tokens)", fused.pre_out[toks].cpu().numpy(),
           oracle_prefill(w, ref_q, kp, vp, toks), TOL_BF16)

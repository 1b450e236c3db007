"""Packed prompts attending only among themselves (nest attention.linnet,
prefill_packed / packed) through the C ABI, against the oracle's ``packed``,
which reads the pass's own keys and values rather than the pool.

The pack mixes a chunk with history (positions from 300), a prompt from 0, a
second prompt in the same row right after it, and a prompt from 64, so 64-token
tiles span prompts, rows and differing first visible positions.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_support import DEV, TOL_BF16, TOL_F32, Run, bits, lib, max_abs_err, oracle_append

pytestmark = pytest.mark.gpu

CHUNKS = [(0, 300, 150), (1, 0, 100), (1, 100, 37), (2, 64, 90)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    lib().version()  # loads libqknr.so; fails loudly when it is not built
    yield
    torch.cuda.empty_cache()


def _workload(dtype, seed, chunks=CHUNKS):
    w = W.build("packed", seed, dtype, num_pages=64, pages_per_row=12, n_table_rows=3,
                chunks=chunks)
    seg = np.concatenate([np.full(n, i) for i, (_, _, n) in enumerate(chunks)]).astype(np.int32)
    return w, seg


def _packed(run, seg):
    Q = lib()
    w, t = run.w, run.t
    P = w.n_prefill
    out = torch.empty((P, W.NUM_Q_HEADS * W.HEAD_DIM), dtype=torch.float32, device=DEV)
    ws = torch.zeros(max(1, Q.packed_workspace_bytes(run.k_pool, W.NUM_Q_HEADS, P)),
                     dtype=torch.uint8, device=DEV)
    Q.packed_prefill_attn(run.q_out[:P], run.k_pool, run.v_pool, t["table"], t["rows"],
                          t["positions"], torch.from_numpy(seg).to(DEV), W.SCALE, out, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_packed_prefill_matches_oracle(dtype):
    w, seg = _workload(dtype, 41)
    print(f"packed prefill {dtype}: {w.n_prefill} tokens, chunks {CHUNKS}", flush=True)
    run = Run(w, keep_pre=False)
    run.append()
    got = _packed(run, seg).cpu().numpy()
    q_out, k_rows, v_rows, _ = oracle_append(w)
    ref = O.packed(q_out, w.dtype, k_rows, v_rows, w.dtype, seg, w.positions, W.SCALE)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    err = max_abs_err(got, ref)
    assert err <= tol, err


def test_packed_equals_paged_without_history_bitwise():
    # every prompt from position 0 in its own row: the packed and the paged
    # forms compute the same thing
    chunks = [(0, 0, 150), (1, 0, 100), (2, 0, 127)]
    w, seg = _workload("bf16", 42, chunks)
    run = Run(w, keep_pre=False)
    run.append()
    got = _packed(run, seg)
    run.prefill()
    torch.cuda.synchronize()
    assert torch.equal(bits(got), bits(run.pre_out))


def test_packed_history_does_not_change_the_result_bitwise():
    # the same pack over two different histories in the pools
    w, seg = _workload("bf16", 43)
    outs = []
    for fill in (None, 7.0):
        run = Run(w, keep_pre=False)
        if fill is not None:
            # overwrite every slot before the step's writes; the pass's own keys land on top
            run.k_pool.fill_(fill)
            run.v_pool.fill_(-fill)
        run.append()
        outs.append(_packed(run, seg))
    assert torch.equal(bits(outs[0]), bits(outs[1]))


@pytest.mark.parametrize("fill_bits", [0x7FC0, 0x7F80, 0xFF80])
def test_packed_ignores_non_finite_history_bitwise(fill_bits):
    # history the packed form does not see may hold anything, NaN and +-Inf
    # included (an uninitialised scratch pool of the training form): the result is
    # bitwise the one over a clean history. The chunks start mid-page (300, 100,
    # 64 + 90 tokens), so a run's first page mixes unseen history and its own keys.
    w, seg = _workload("bf16", 44)
    outs = []
    for fill in (None, fill_bits):
        run = Run(w, keep_pre=False)
        if fill is not None:
            val = torch.from_numpy(np.array([fill], np.uint16).view(np.int16)).view(torch.bfloat16).item()
            run.k_pool.fill_(val)
            run.v_pool.fill_(val)
        run.append()
        outs.append(_packed(run, seg))
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(bits(outs[0]), bits(outs[1]))

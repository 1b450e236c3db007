"""The prefill softmax's three page paths, on the GPU through the C ABI.

The paged prefill kernel evaluates a page's exponentials against the running max
m as it stands and takes the page max only when some lane's sum of them exceeds
2^7 (or a query has no finite max yet); the running max then moves when the page
max exceeds m by more than 8 log2 units. Scores built directly (q and the pools
are inputs of paged_prefill_attn) put each KV head's queries on a chosen path:

* even KV heads: a key on page 1 scores 7.49 above page 0 (sum above 2^7, max
  within 8: the page is redone against the same m), a key on page 2 scores 9.5
  above (the max moves);
* odd KV heads: the page-1 key scores 8.5 above (the max moves on page 1), the
  page-2 key 1.0 above the new max (the sum stays small: no page max taken).

Outputs must match the oracle within the bfloat16 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_support import DEV, TOL_BF16, host_values, lib, max_abs_err

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    lib().version()
    yield
    torch.cuda.empty_cache()


def _bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def test_prefill_page_max_paths():
    Q = lib()
    n_q, n_kv, hd, ps = W.NUM_Q_HEADS, W.NUM_KV_HEADS, W.HEAD_DIM, W.PAGE_SIZE
    num_pages, ppr = 4, 4
    c = W.SCALE * LOG2E   # log2 units of score per unit of q . k
    # 64 prompt tokens at positions 192..255 of one row whose pages are 0..3
    positions = np.arange(192, 256, dtype=np.int32)
    n = len(positions)
    rows = np.zeros(n, dtype=np.int32)
    table = np.arange(ppr, dtype=np.int32)[None, :]
    # every query head: q = e_0
    q = np.zeros((n, n_q * hd), dtype=np.float32)
    q[:, ::hd] = 1.0
    # k: dim 0 sets each key's score (all other dims 0)
    k = np.zeros((n_kv, num_pages * ps, hd), dtype=np.float32)
    for g in range(n_kv):
        s1, s2 = (7.5, 9.5) if g % 2 == 0 else (8.5, 9.5)
        k[g, 1 * ps + 5, 0] = s1 / c
        k[g, 2 * ps + 17, 0] = s2 / c
    rng = np.random.default_rng(57)
    v = rng.standard_normal((n_kv, num_pages * ps, hd)).astype(np.float32)
    q_t, k_t, v_t = _bf16(q), _bf16(k), _bf16(v)
    # the cases exist after rounding to bfloat16
    kb = host_values(k_t, "bf16")
    s = O.widen(kb, "bf16")[:, :, 0] * c
    for g in range(n_kv):
        p0, p1, p2 = (s[g, i * ps:(i + 1) * ps].max() for i in range(3))
        if g % 2 == 0:
            assert 7.0 < p1 - p0 < 8.0 and p2 - p0 > 8.0, (g, p0, p1, p2)
        else:
            assert p1 - p0 > 8.0 and p2 - p1 < 7.0, (g, p0, p1, p2)
    out = torch.empty((n, n_q * hd), dtype=torch.float32, device=DEV)
    ws = torch.zeros(max(1, Q.prefill_workspace_bytes(k_t, n_q, n)), dtype=torch.uint8, device=DEV)
    Q.paged_prefill_attn(q_t, k_t, v_t, torch.from_numpy(table).to(DEV), torch.from_numpy(rows).to(DEV),
                         torch.from_numpy(positions).to(DEV), W.SCALE, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = O.prefill(host_values(q_t, "bf16"), "bf16", kb, host_values(v_t, "bf16"), "bf16", table, rows,
                    positions, W.SCALE)
    assert np.isfinite(got).all()
    err = max_abs_err(got, ref)
    print(f"[softmax paths] prefill max abs err {err:.3e}", flush=True)
    assert err <= TOL_BF16

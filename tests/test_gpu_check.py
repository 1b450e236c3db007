"""qkr_check_indices on the GPU through the C ABI: a valid step has no
violations; corrupted rows, positions, page ids and slots are counted exactly
(the expected counts are found by brute force on the host); the no-wait form
only enqueues, and the waiting form returns QKR_EDATA."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_support import DEV, lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    lib().version()
    yield
    torch.cuda.empty_cache()


def _expected(w, table, rows, positions, slots, step_positions, rope_rows):
    """Brute force over every query: the QKR_CHECK_* counts."""
    n_rows, ppr = table.shape
    max_pos = min(ppr * 64, rope_rows) if rope_rows > 0 else ppr * 64
    c = dict(row=0, position=0, page=0, slot_range=0, slot_mismatch=0)
    queries = [(int(r), int(p), int(s)) for r, p, s in zip(rows, positions, slots)]
    queries += [(w.decode_row0 + b, int(p), None) for b, p in enumerate(step_positions)]
    for i, (r, p, s) in enumerate(queries):
        prompt = i < len(rows)
        row_bad = not (0 <= r < n_rows)
        pos_bad = not (0 <= p < max_pos)
        c["row"] += prompt and row_bad
        c["position"] += pos_bad
        if not row_bad and not pos_bad:
            c["page"] += any(not (0 <= table[r][j] < w.num_pages) for j in range(p // 64 + 1))
        if prompt and s >= 0:
            c["slot_range"] += s >= w.num_pages * 64
            if not row_bad and not pos_bad:
                c["slot_mismatch"] += s != table[r][p // 64] * 64 + p % 64
    return c


def _call(w, t, **kw):
    k_pool = torch.empty((w.n_kv_heads, w.pool_slots, 128), dtype=torch.bfloat16, device=DEV)
    return lib().check_indices(k_pool, w.n_q_heads, t["table"], rows=t["rows"], positions=t["positions"],
                               slots=t["slots"], step_positions=t["step_positions"], decode_row0=w.decode_row0,
                               **kw)


def test_valid_step_has_no_violations():
    w = W.config(4)
    t = W.upload(w, DEV)
    st, counts = _call(w, t, rope_rows=W.MAX_POSITIONS)
    print(f"[check] {w.name}: {counts}", flush=True)
    assert st == 0 and not any(counts.values())


def test_corrupted_indices_are_counted_exactly():
    w = W.build("check", 71, "bf16", num_pages=300, pages_per_row=20, n_table_rows=8,
                chunks=[(0, 130, 70), (1, 0, 90), (2, 5, 40)], decode=[(3, 0), (4, 64), (5, 777), (6, 1200),
                                                                       (7, 300)], decode_row0=3)
    table, rows, positions = w.table.copy(), w.rows.copy(), w.positions.copy()
    slots, step_positions = w.slots.copy(), w.step_positions.copy()
    rows[3] = 8                        # a table row that does not exist
    rows[4] = -1
    positions[10] = -5                 # a negative position
    positions[100] = 20 * 64           # past the page table
    table[1, 0] = w.num_pages + 2      # row 1's first page: every token of row 1 sees it
    table[6, 18] = -3                  # decode row 6 (position 1200, page 18) sees it
    table[5, 19] = -4                  # beyond decode row 5's last page (12): not seen
    slots[20] = w.num_pages * 64 + 7   # outside the pool
    slots[30] = slots[31]              # another slot of the pool: differs from its row's table
    slots[40] = -1                     # padding: not counted
    step_positions[4] = 40960          # past the rotation table (and the 20-page table)
    exp = _expected(w, table, rows, positions, slots, step_positions, W.MAX_POSITIONS)
    t = W.upload(w, DEV)
    for name, arr in (("table", table), ("rows", rows), ("positions", positions), ("slots", slots),
                      ("step_positions", step_positions)):
        t[name] = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32)).to(DEV)
    st, counts = _call(w, t, rope_rows=W.MAX_POSITIONS)
    print(f"[check] corrupted: {counts}, expected {exp}", flush=True)
    assert st == lib().QKR_EDATA
    assert counts == exp
    assert all(v > 0 for v in exp.values())
    assert "bad rows" in lib().last_error()
    # without waiting: the counts land in the device buffer, nothing else happens
    st, dev_counts = _call(w, t, rope_rows=W.MAX_POSITIONS, wait=False)
    assert st == 0
    torch.cuda.synchronize()
    assert dev_counts.cpu().tolist()[:5] == [exp[k] for k in ("row", "position", "page", "slot_range",
                                                             "slot_mismatch")]
    # a smaller rotation table makes more positions out of range
    exp2 = _expected(w, table, rows, positions, slots, step_positions, 1000)
    st, counts = _call(w, t, rope_rows=1000)
    assert counts == exp2 and exp2["position"] > exp["position"]

"""Seeded synthetic inputs for the paged QK-norm + RoPE + attention step.

This module only draws inputs: activations, gains, page tables, positions, rows,
slots and the pool contents that stand in for earlier steps. It holds none of
the step's arithmetic and serves both the oracle (on the CPU) and the GPU
library (through torch device tensors).

The five standard workloads follow the shapes of the nest ``qwen3-8b`` page
(README architecture paragraph and Entries table: 32 query heads over 8 KV heads,
head_dim 128, pages of 64 positions, at most 40960 positions per row):

0. one decode row at position 63 over one page, float32 everywhere;
1. 8 decode rows at positions uniform in [256, 4096], 1024-page bfloat16 pool;
2. 64 decode rows at positions log-uniform in [64, 32768], 8 shared prefix
   pages, a pool of 40960 pages (40960 positions per row);
3. packed prefill of 4 prompts (512, 1024, 1000, 1560 tokens) from position 0;
4. a mixed step: chunks of 2048 tokens at positions 8192 (row 0) and 0 (row 1),
   plus 128 decode rows at positions uniform in [1, 16384], 65536-page pool.

Pool contents before the step ("history") come from a counter-based hash of
(seed, k-or-v, kv head, slot, element) so that any page can be regenerated on
the host without copying the pool back. The top 16 bits of the hash pick one of
65536 standard normal quantiles (at probabilities (i + 1/2) / 65536, float32), so
the history is N(0, 1) to within that discretisation (tails to about 4.3), and
the same table lookup gives identical values on the CPU and on the GPU. Slots
that hold neither history nor a write of the step are NaN so that a wrong read
shows up in the output.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 64
HEAD_DIM = 128
NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
MAX_POSITIONS = 40960
SCALE = float(np.float32(1.0 / np.sqrt(np.float32(HEAD_DIM))))

CONFIG_NAMES = [
    "decode_1row_pos63_f32",
    "decode_8rows_u256_4096_bf16",
    "decode_64rows_logu64_32768_prefix8_bf16",
    "prefill_packed_4096_bf16",
    "step_2x2048_plus_128rows_bf16",
]


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str                     # "f32" or "bf16": input, q_out and pool dtype
    num_pages: int
    pages_per_row: int
    table: np.ndarray              # int32 [n_table_rows, pages_per_row]
    positions: np.ndarray          # int32 [P]   prompt tokens
    rows: np.ndarray               # int32 [P]
    slots: np.ndarray              # int32 [P]
    step_positions: np.ndarray     # int32 [R]   decode rows
    decode_row0: int               # decode row b uses table row decode_row0 + b
    q: np.ndarray                  # [P+R, 32*128] float32 or bf16 bits (uint16)
    k: np.ndarray                  # [P+R, 8*128]
    v: np.ndarray                  # [P+R, 8*128]
    q_gain: np.ndarray             # float32 [128]
    k_gain: np.ndarray             # float32 [128]
    history: list = field(default_factory=list)   # (row, n) : positions 0..n-1 pre-filled
    row_pages: dict = field(default_factory=dict)  # row -> allocated page ids, in order
    n_kv_heads: int = NUM_KV_HEADS   # one GPU's share when the heads are sharded (8 / S)
    _history_slots: np.ndarray = field(default=None, repr=False)

    @property
    def n_q_heads(self) -> int:
        return self.n_kv_heads * (NUM_Q_HEADS // NUM_KV_HEADS)

    @property
    def n_prefill(self) -> int:
        return int(len(self.positions))

    @property
    def n_decode(self) -> int:
        return int(len(self.step_positions))

    @property
    def n_tokens(self) -> int:
        return self.n_prefill + self.n_decode

    @property
    def decode_table(self) -> np.ndarray:
        return self.table[self.decode_row0:self.decode_row0 + self.n_decode]

    @property
    def pool_slots(self) -> int:
        return self.num_pages * PAGE_SIZE

    def row_slot_list(self, row: int, n: int) -> np.ndarray:
        """Slots the allocator gave to positions 0..n-1 of ``row``."""
        pages = np.asarray(self.row_pages[row], dtype=np.int64)
        expanded = (pages[:, None] * PAGE_SIZE + np.arange(PAGE_SIZE)[None, :]).reshape(-1)
        return expanded[:n]

    def history_slots(self) -> np.ndarray:
        """Every slot that holds a pre-step value (shared prefix pages once), sorted."""
        if self._history_slots is None:
            s = [self.row_slot_list(r, n) for r, n in self.history if n > 0]
            self._history_slots = (np.unique(np.concatenate(s)) if s
                                   else np.zeros(0, dtype=np.int64))
        return self._history_slots


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def build(name: str, seed: int, dtype: str, num_pages: int, pages_per_row: int,
          n_table_rows: int, chunks=(), decode=(), decode_row0: int = 0,
          shared_prefix_pages: int = 0, reserve_page0: bool = True,
          n_kv_heads: int = NUM_KV_HEADS, gain_range=(0.5, 1.5)) -> Workload:
    """General builder.

    ``chunks``: sequence of (row, first_position, length) prompt chunks, packed
    in this order; positions before ``first_position`` of that row are history.
    ``decode``: sequence of (row, position); positions before it are history.
    ``shared_prefix_pages``: that many page ids are common to every row, and a
    row uses min(shared, position // 64) of them, so the page it writes is its own.
    ``n_kv_heads``: KV heads of the workload (4 query heads each); fewer than 8 is
    one GPU's share of the heads when they are sharded over 8 / n_kv_heads GPUs.
    ``gain_range``: the QK-norm gains are uniform in it ((0.5, 1.5) by default;
    large gains give wide score ranges).
    """
    rng = np.random.default_rng(seed)
    need = {}      # row -> number of positions the row spans after the step
    hist = {}      # row -> number of history positions
    for r, p0, n in chunks:
        need[r] = max(need.get(r, 0), p0 + n)
        hist[r] = p0
    for r, p in decode:
        need[r] = max(need.get(r, 0), p + 1)
        hist[r] = p
    first = 1 if (reserve_page0 and num_pages > 1) else 0
    free = list(rng.permutation(np.arange(first, num_pages)))
    prefix = [int(free.pop()) for _ in range(shared_prefix_pages)]
    table = np.zeros((n_table_rows, pages_per_row), dtype=np.int32)
    row_pages = {}
    for r in sorted(need):
        n_pages = -(-need[r] // PAGE_SIZE)
        assert n_pages <= pages_per_row, (r, n_pages, pages_per_row)
        first_new = hist[r]
        n_shared = min(shared_prefix_pages, first_new // PAGE_SIZE)
        pages = prefix[:n_shared] + [int(free.pop()) for _ in range(n_pages - n_shared)]
        row_pages[r] = pages
        table[r, :n_pages] = pages

    def slot_of(r, pos):
        return row_pages[r][pos // PAGE_SIZE] * PAGE_SIZE + pos % PAGE_SIZE

    positions, rows, slots = [], [], []
    for r, p0, n in chunks:
        for pos in range(p0, p0 + n):
            positions.append(pos)
            rows.append(r)
            slots.append(slot_of(r, pos))
    step_positions = [p for _, p in decode]
    for b, (r, _) in enumerate(decode):
        assert r == decode_row0 + b, "decode row b must use table row decode_row0 + b"

    n_tok = len(positions) + len(step_positions)
    n_q_heads = n_kv_heads * (NUM_Q_HEADS // NUM_KV_HEADS)
    q = rng.standard_normal((n_tok, n_q_heads * HEAD_DIM), dtype=np.float32)
    k = rng.standard_normal((n_tok, n_kv_heads * HEAD_DIM), dtype=np.float32)
    v = rng.standard_normal((n_tok, n_kv_heads * HEAD_DIM), dtype=np.float32)
    q_gain = rng.uniform(gain_range[0], gain_range[1], HEAD_DIM).astype(np.float32)
    k_gain = rng.uniform(gain_range[0], gain_range[1], HEAD_DIM).astype(np.float32)
    if dtype == "bf16":
        q, k, v = _bf16_bits(q), _bf16_bits(k), _bf16_bits(v)
    history = sorted(hist.items())
    return Workload(
        name=name, seed=seed, dtype=dtype, num_pages=num_pages, pages_per_row=pages_per_row,
        table=table, positions=np.asarray(positions, np.int32), rows=np.asarray(rows, np.int32),
        slots=np.asarray(slots, np.int32), step_positions=np.asarray(step_positions, np.int32),
        decode_row0=decode_row0, q=q, k=k, v=v, q_gain=q_gain, k_gain=k_gain,
        history=history, row_pages=row_pages, n_kv_heads=n_kv_heads)


def config(i: int, seed: int | None = None, kv_heads: int = NUM_KV_HEADS) -> Workload:
    """Standard workload ``i`` (0..4); the seed defaults to ``i``. ``kv_heads`` < 8
    gives one GPU's share of it when the heads are sharded (same rows and positions)."""
    s = i if seed is None else seed
    rng = np.random.default_rng(10_000 + s)
    name = CONFIG_NAMES[i] + ("" if kv_heads == NUM_KV_HEADS else f"_kv{kv_heads}")
    kw = {"n_kv_heads": kv_heads}
    if i == 0:
        return build(name, s, "f32", num_pages=1, pages_per_row=1, n_table_rows=1,
                     decode=[(0, 63)], reserve_page0=False, **kw)
    if i == 1:
        pos = rng.integers(256, 4096, size=8, endpoint=True)
        return build(name, s, "bf16", num_pages=1024, pages_per_row=65, n_table_rows=8,
                     decode=[(b, int(p)) for b, p in enumerate(pos)], **kw)
    if i == 2:
        pos = np.floor(np.exp(rng.uniform(np.log(64), np.log(32768), size=64))).astype(int)
        return build(name, s, "bf16", num_pages=40960, pages_per_row=640, n_table_rows=64,
                     decode=[(b, int(p)) for b, p in enumerate(pos)], shared_prefix_pages=8, **kw)
    if i == 3:
        lens = [512, 1024, 1000, 1560]
        return build(name, s, "bf16", num_pages=1024, pages_per_row=25, n_table_rows=4,
                     chunks=[(r, 0, n) for r, n in enumerate(lens)], **kw)
    if i == 4:
        pos = rng.integers(1, 16384, size=128, endpoint=True)
        return build(name, s, "bf16", num_pages=65536, pages_per_row=257, n_table_rows=130,
                     chunks=[(0, 8192, 2048), (1, 0, 2048)],
                     decode=[(2 + b, int(p)) for b, p in enumerate(pos)], decode_row0=2, **kw)
    raise IndexError(i)


# --------------------------------------------------------------------------
# History values: counter-based, identical on CPU and GPU (integer ops, an exact
# int -> float conversion and a power-of-two scale, then torch's bfloat16 cast).
# --------------------------------------------------------------------------

_M32 = 0xFFFFFFFF
_NORMAL_TABLE = None
_TABLE_ON = {}   # device -> the quantile table as a torch tensor there


def normal_quantiles() -> np.ndarray:
    """float32 [65536]: the standard normal quantile at (i + 1/2) / 65536."""
    global _NORMAL_TABLE
    if _NORMAL_TABLE is None:
        from statistics import NormalDist
        nd = NormalDist()
        _NORMAL_TABLE = np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)],
                                 dtype=np.float64).astype(np.float32)
        _NORMAL_TABLE.flags.writeable = False
    return _NORMAL_TABLE


def _mix32(x):
    x = x ^ (x >> 16)
    x = (x * 0x45D9F3B) & _M32
    x = x ^ (x >> 16)
    x = (x * 0x45D9F3B) & _M32
    x = x ^ (x >> 16)
    return x


def history_values(seed: int, which: int, kv_head: int, slots, device="cpu"):
    """float32 torch tensor [len(slots), 128] of pre-step pool values.

    ``which`` is 0 for K, 1 for V. Values depend only on (seed, which, kv_head,
    slot, element), never on the row that owns the slot.
    """
    import torch
    s = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=device)
    key = int(_mix32(np.int64(((seed * 2 + which) * 64 + kv_head + 1) & _M32)))
    idx = s[:, None] * HEAD_DIM + torch.arange(HEAD_DIM, device=device, dtype=torch.int64)[None, :]
    h = _mix32(_mix32(idx & _M32) ^ key)
    dev = str(torch.device(device))
    if dev not in _TABLE_ON:
        _TABLE_ON[dev] = torch.from_numpy(normal_quantiles().copy()).to(device)
    return _TABLE_ON[dev][h >> 16]


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def make_pools(w: Workload, device, chunk_slots: int = 1 << 16):
    """K and V pools [n_kv_heads, num_pages*64, 128] on ``device`` holding the pre-step state."""
    import torch
    td = torch_dtype(w.dtype)
    shape = (w.n_kv_heads, w.pool_slots, HEAD_DIM)
    k_pool = torch.full(shape, float("nan"), dtype=td, device=device)
    v_pool = torch.full(shape, float("nan"), dtype=td, device=device)
    hs = w.history_slots()
    for a in range(0, len(hs), chunk_slots):
        part = hs[a:a + chunk_slots]
        idx = torch.as_tensor(part, device=device)
        for g in range(w.n_kv_heads):
            k_pool[g].index_copy_(0, idx, history_values(w.seed, 0, g, part, device).to(td))
            v_pool[g].index_copy_(0, idx, history_values(w.seed, 1, g, part, device).to(td))
    return k_pool, v_pool


def host_history(w: Workload, which: int, kv_head: int, slots) -> np.ndarray:
    """Pre-step stored values at ``slots`` as the pool holds them (float32, or
    bfloat16 bits as uint16); NaN where no history was written."""
    import torch
    slots = np.asarray(slots, dtype=np.int64)
    hs = w.history_slots()
    pos = np.searchsorted(hs, slots)
    present = (pos < len(hs)) & (hs[np.minimum(pos, max(len(hs) - 1, 0))] == slots) if len(hs) else \
        np.zeros(len(slots), dtype=bool)
    vals = history_values(w.seed, which, kv_head, slots)
    vals[torch.as_tensor(~present)] = float("nan")
    t = vals.to(torch_dtype(w.dtype))
    if w.dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def upload(w: Workload, device):
    """Activations, gains and index arrays as torch tensors on ``device``."""
    import torch

    def act(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
        return torch.from_numpy(a.copy()).to(device)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

    return {
        "q": act(w.q), "k": act(w.k), "v": act(w.v),
        "q_gain": torch.from_numpy(w.q_gain.copy()).to(device),
        "k_gain": torch.from_numpy(w.k_gain.copy()).to(device),
        "table": i32(w.table), "positions": i32(w.positions), "rows": i32(w.rows),
        "slots": i32(w.slots), "step_positions": i32(w.step_positions),
        "decode_table": i32(w.decode_table),
    }

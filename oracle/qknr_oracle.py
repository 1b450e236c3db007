"""Plain, slow CPU oracle for the paged QK-norm + RoPE + GQA attention step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. It shares
no code with the HIP library and imports nothing from it.

What it computes, and where the pages state it:

* fantasma, ``src/inference/model.zig`` (tangled.org), ``fullAttentionForward``:
  per-head RMSNorm of q and k with one ``[head_dim]`` gain each (QK-norm), then
  RoPE at the token's position, then the k/v append, then for every query head
  ``h`` the scaled dot product with every cached key of KV head
  ``h / (heads / kv_heads)``, a max-subtracted softmax and the weighted sum of
  the cached values. ``applyRope`` fixes the non-interleaved ("rotate_half")
  pairing of element ``i`` with ``i + head_dim/2``; ``loadWeights`` builds the
  cos/sin table from ``inv_freq = 1 / theta^(2i/dim)``.
* nest, ``models/qwen3-8b/files``: the README's architecture paragraph (32 query
  heads, 8 KV heads, head_dim 128, rope base 1e6, RMS eps 1e-6; QK-norm after the
  split into heads and before rope), its Entries table (``decode_paged``,
  ``prefill_paged``, ``step_paged``; page size 64), ``src/attention.linnet``
  (``decode``: a key is visible when its position is at most the query's;
  ``decode_paged`` / ``prefill_paged`` / ``step_paged``: the writes go into the
  pool before attention reads it), ``src/norm.linnet`` (``rms_norm`` over the
  last axis, eps 1e-6) and ``src/rope.linnet`` (``tables``: each frequency
  repeated for both halves).
* logicaffeine, ``logicaffeine_compile/model/author.rs``, ``attention``: the same
  order (norm across heads, rope across heads, write the row, attend up to pos).

Floating-point contract. The pages fix no intermediate precision for QK-norm and
RoPE, so this oracle pins one float32 recipe (every step an IEEE round-to-nearest
float32 operation, no fused multiply-add) and the library must reproduce its
bytes exactly:

1. ``p_l = x_l*x_l + x_{l+64}*x_{l+64}`` for ``l < 64`` (products rounded, then the sum);
2. pairwise sum of the 64 ``p_l``, neighbours first (``p0+p1``, ``p2+p3``, ...);
3. ``ms = ss / 128`` (exact), ``r = 1 / sqrt(ms + eps)`` (sqrt and division rounded);
4. ``y_d = (x_d * r) * g_d``;
5. ``y'_i = y_i*c_i - y_{i+64}*s_i`` and ``y'_{i+64} = y_{i+64}*c_i + y_i*s_i``;
6. the store rounds to the pool dtype (bfloat16: round to nearest even).

Attention is computed in float64 from the pool contents after the append.
"""
from __future__ import annotations

import math
from functools import lru_cache

import numpy as np

PAGE_SIZE = 64
HEAD_DIM = 128
NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
ROPE_THETA = 1.0e6
RMS_EPS = 1.0e-6


# --------------------------------------------------------------------------
# bfloat16 storage (the pool dtype of the nest package's generics, T = "bf16")
# --------------------------------------------------------------------------

def f32_from_bf16_bits(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_from_f32(x) -> np.ndarray:
    """Round float32 to bfloat16 with round-to-nearest-even; returns uint16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        rounded = np.where(nan, np.uint16(0x7FC0), rounded)
    return rounded


def widen(a, dtype: str) -> np.ndarray:
    """Stored values (float32 array, bfloat16 bits, or float64) as float64."""
    if dtype == "bf16":
        return f32_from_bf16_bits(a).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f64":   # exact float64 inputs (brute-force checks)
        return np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


def as_f32(a, dtype: str) -> np.ndarray:
    """Input activations as float32 (bfloat16 inputs widen exactly)."""
    if dtype == "bf16":
        return f32_from_bf16_bits(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    raise ValueError(dtype)


def store(a_f32, dtype: str) -> np.ndarray:
    """Round float32 values to the pool dtype (step 6 of the recipe)."""
    if dtype == "bf16":
        return bf16_bits_from_f32(a_f32)
    if dtype == "f32":
        return np.asarray(a_f32, dtype=np.float32).copy()
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Slot resolution: nest README, Entries table (decode_paged: row b's positions
# lie in the pages table[b] lists, PageSize 64); attention.linnet page_slots.
# --------------------------------------------------------------------------

def page_slot(table_row, pos: int, page_size: int = PAGE_SIZE) -> int:
    """Pool slot of position ``pos`` of a row whose page list is ``table_row``."""
    return int(table_row[pos // page_size]) * page_size + pos % page_size


def row_slots(table_row, n_pos: int, page_size: int = PAGE_SIZE) -> np.ndarray:
    """Slots of positions 0 .. n_pos-1 of one row, in position order."""
    return np.array([page_slot(table_row, j, page_size) for j in range(n_pos)],
                    dtype=np.int64)


# --------------------------------------------------------------------------
# RoPE table: fantasma model.zig, loadWeights (inv_freq = 1/theta^(2i/dim),
# angle = pos * inv_freq); nest rope.linnet, tables (THETA = 1e6, the same
# frequency for both halves). Evaluated in float64, rounded once to float32;
# only the half-width [pos][D/2] table is kept since both halves are equal.
# --------------------------------------------------------------------------

def rope_inv_freq(theta: float, head_dim: int) -> list:
    return [1.0 / math.pow(theta, (2.0 * i) / head_dim) for i in range(head_dim // 2)]


@lru_cache(maxsize=65536)
def _rope_row_cached(theta: float, pos: int, head_dim: int):
    inv = rope_inv_freq(theta, head_dim)
    c = np.array([math.cos(pos * f) for f in inv], dtype=np.float64).astype(np.float32)
    s = np.array([math.sin(pos * f) for f in inv], dtype=np.float64).astype(np.float32)
    c.flags.writeable = False
    s.flags.writeable = False
    return c, s


def rope_row(theta: float, pos: int, head_dim: int = HEAD_DIM):
    """(cos, sin) float32 vectors of length head_dim/2 for one position."""
    return _rope_row_cached(float(theta), int(pos), int(head_dim))


def rope_table(theta: float, n_pos: int, head_dim: int = HEAD_DIM):
    """(cos, sin) float32 tables of shape [n_pos, head_dim/2]."""
    inv = rope_inv_freq(theta, head_dim)
    half = head_dim // 2
    cos = np.empty((n_pos, half), dtype=np.float32)
    sin = np.empty((n_pos, half), dtype=np.float32)
    for pos in range(n_pos):
        for i in range(half):
            a = pos * inv[i]
            cos[pos, i] = math.cos(a)
            sin[pos, i] = math.sin(a)
    return cos, sin


# --------------------------------------------------------------------------
# QK-norm: nest README and norm.linnet (RmsNorm over the last axis at width
# head_dim, eps 1e-6, applied per head after split_heads); fantasma
# fullAttentionForward (rmsNorm of each head slice with q_norm / k_norm).
# --------------------------------------------------------------------------

def _pair_sums(p) -> np.ndarray:
    """Pairwise float32 sum along the last axis, neighbours first; an odd last
    element is carried up a level unchanged."""
    while p.shape[-1] > 1:
        n = p.shape[-1]
        m = n - n % 2
        q = p[..., 0:m:2] + p[..., 1:m:2]
        if n % 2:
            q = np.concatenate([q, p[..., m:]], axis=-1)
        p = q
    return p[..., 0]


def _head_square_sums(x) -> np.ndarray:
    """Per head (last axis, width D): sum of squares by recipe steps 1-2."""
    d = x.shape[-1]
    half = d // 2
    assert half & (half - 1) == 0, "head_dim/2 must be a power of two"
    sq = x * x
    return _pair_sums(sq[..., :half] + sq[..., half:])


def qk_norm(x, gain, eps: float = RMS_EPS) -> np.ndarray:
    """RMS-normalise the last axis of ``x`` (float32 recipe steps 1-4)."""
    x = np.asarray(x, dtype=np.float32)
    g = np.asarray(gain, dtype=np.float32)
    d = x.shape[-1]
    ss = _head_square_sums(x)
    ms = ss / np.float32(d)
    r = np.float32(1.0) / np.sqrt(ms + np.float32(eps))
    return (x * r[..., None]) * g


def qk_norm_whole(x, gain, eps: float = RMS_EPS) -> np.ndarray:
    """RMS-normalise all heads of a token together: ``x`` [..., H, D], ``gain`` [H*D].

    logicaffeine ``author.rs``, ``qk_norm_segments``: with ``qk_norm_whole`` the
    q and k norms run over one segment of width heads*head_dim (kv_heads*head_dim)
    instead of one per head. Pinned float32 order: each head's sum of squares by
    recipe steps 1-2, the head sums added pairwise (neighbours first, an odd last
    one carried up), ``ms = total / (H*D)``, ``r = 1/sqrt(ms + eps)``,
    ``y = (x*r)*g``.
    """
    x = np.asarray(x, dtype=np.float32)
    h, d = x.shape[-2], x.shape[-1]
    g = np.asarray(gain, dtype=np.float32).reshape(h, d)
    total = _pair_sums(_head_square_sums(x))
    ms = total / np.float32(h * d)
    r = np.float32(1.0) / np.sqrt(ms + np.float32(eps))
    return (x * r[..., None, None]) * g


def rope_rotate(y, cos, sin, rotary_dim: int | None = None) -> np.ndarray:
    """Rotate pairs (i, i + R/2) of the first R = rotary_dim elements by the angle
    whose cos/sin are given (recipe step 5); the other elements pass unchanged.

    ``cos``/``sin`` broadcast against ``y[..., :R/2]``. fantasma ``applyRope``:
    ``x*cos + rotate_half(x)*sin`` with ``rotate_half(x) = cat(-x2, x1)`` over the
    first ``rotary_dim`` elements (R = D: the whole head).
    """
    y = np.asarray(y, dtype=np.float32)
    r = y.shape[-1] if rotary_dim is None else int(rotary_dim)
    half = r // 2
    a = y[..., :half]
    b = y[..., half:r]
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    return np.concatenate([a * c - b * s, b * c + a * s, y[..., r:]], axis=-1)


def append(q, k, v, in_dtype: str, pool_dtype: str, q_gain, k_gain, positions,
           eps: float = RMS_EPS, theta: float = ROPE_THETA,
           n_q_heads: int = NUM_Q_HEADS, n_kv_heads: int = NUM_KV_HEADS,
           head_dim: int = HEAD_DIM, norm_whole: bool = False, rotary_dim: int | None = None):
    """QK-norm + RoPE of every token, and the values to store.

    ``q``: [n, n_q_heads*head_dim], ``k``/``v``: [n, n_kv_heads*head_dim], token
    major with head h at columns h*D .. h*D+D-1 (nest attention.linnet,
    split_heads). Returns ``(q_out, k_rows, v_rows)`` in the pool dtype with
    shapes [n, n_q_heads*D], [n, n_kv_heads, D], [n, n_kv_heads, D].
    ``norm_whole``: one RMS norm over all heads (gains [n_heads*D]);
    ``rotary_dim``: rotate only the first R elements of every head, with the
    table of an R-wide head (``inv_freq = 1/theta^(2i/R)``).
    """
    n = len(positions)
    D = head_dim
    R = D if rotary_dim is None else int(rotary_dim)
    qf = as_f32(q, in_dtype).reshape(n, n_q_heads, D)
    kf = as_f32(k, in_dtype).reshape(n, n_kv_heads, D)
    vf = as_f32(v, in_dtype).reshape(n, n_kv_heads, D)
    cos = np.stack([rope_row(theta, int(p), R)[0] for p in positions]) if n else np.zeros((0, R // 2), np.float32)
    sin = np.stack([rope_row(theta, int(p), R)[1] for p in positions]) if n else np.zeros((0, R // 2), np.float32)
    norm = qk_norm_whole if norm_whole else qk_norm
    qn = rope_rotate(norm(qf, q_gain, eps), cos[:, None, :], sin[:, None, :], R)
    kn = rope_rotate(norm(kf, k_gain, eps), cos[:, None, :], sin[:, None, :], R)
    q_out = store(qn.reshape(n, n_q_heads * D), pool_dtype)
    k_rows = store(kn, pool_dtype)
    v_rows = store(vf, pool_dtype)
    return q_out, k_rows, v_rows


def apply_writes(k_pool, v_pool, slots, k_rows, v_rows) -> None:
    """Write each token's k/v rows at its slot of every KV head; slot < 0 is skipped.

    Pools are indexed ``pool[kv_head, slot, d]`` (nest attention.linnet, cache_k /
    cache_v of shape [Batch=1, KvHeads, MaxSeq, HeadDim]).
    """
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        k_pool[:, s, :] = k_rows[t]
        v_pool[:, s, :] = v_rows[t]


# --------------------------------------------------------------------------
# Attention: fantasma fullAttentionForward (per query head, dot with every
# cached key of its KV head, max-subtracted exp, normalise, weighted V sum);
# nest attention.linnet decode (visible when position <= the query's),
# paged_attention / paged_prefill_attention over table[row].
# --------------------------------------------------------------------------

def attend(q_heads, keys, values, scale: float):
    """Softmax attention of a few query heads over one KV head's visible keys.

    q_heads [G, D], keys/values [L, D], all float64. Returns (out [G, D],
    weights [G, L]).
    """
    s = (q_heads @ keys.T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    w = e / e.sum(axis=1, keepdims=True)
    return w @ values, w


def attention(q_out, q_dtype: str, k_pool, v_pool, pool_dtype: str, table, rows,
              positions, scale: float, n_q_heads: int = NUM_Q_HEADS,
              n_kv_heads: int = NUM_KV_HEADS, head_dim: int = HEAD_DIM,
              page_size: int = PAGE_SIZE, tokens=None, return_weights: bool = False):
    """Attention of tokens over their rows' pages, float64.

    Token ``t`` (row ``rows[t]``, position ``positions[t]``) attends with query
    head h over positions 0 .. positions[t] (inclusive) of its row, read through
    ``table[rows[t]]`` from KV head h // (n_q_heads // n_kv_heads). ``k_pool`` /
    ``v_pool`` are indexed ``pool[kv_head, slots]`` -> [len(slots), D].
    ``tokens`` selects a subset of tokens (default: all). Returns
    out [len(tokens), n_q_heads*D] (and per-token weights if asked).
    """
    D = head_dim
    group = n_q_heads // n_kv_heads
    if tokens is None:
        tokens = range(len(positions))
    tokens = list(tokens)
    out = np.zeros((len(tokens), n_q_heads * D), dtype=np.float64)
    weights = []
    by_row = {}
    for i, t in enumerate(tokens):
        by_row.setdefault(int(rows[t]), []).append((i, t))
    for r, items in by_row.items():
        n_vis = max(int(positions[t]) for _, t in items) + 1
        slots = row_slots(table[r], n_vis, page_size)
        kv = [(widen(k_pool[g, slots], pool_dtype), widen(v_pool[g, slots], pool_dtype))
              for g in range(n_kv_heads)]
        for i, t in items:
            pi = int(positions[t])
            q = widen(q_out[t], q_dtype).reshape(n_q_heads, D)
            wt = []
            for g in range(n_kv_heads):
                K, V = kv[g]
                o, w = attend(q[g * group:(g + 1) * group], K[:pi + 1], V[:pi + 1], scale)
                out[i, g * group * D:(g + 1) * group * D] = o.reshape(-1)
                wt.append(w)
            if return_weights:
                weights.append(np.concatenate(wt, axis=0))
    if return_weights:
        return out, weights
    return out


def decode(q_out, q_dtype, k_pool, v_pool, pool_dtype, table, positions, scale, **kw):
    """Paged decode (nest attention.linnet, decode_paged): row b reads table[b]."""
    rows = np.arange(len(positions))
    return attention(q_out, q_dtype, k_pool, v_pool, pool_dtype, table, rows,
                     positions, scale, **kw)


def prefill(q_out, q_dtype, k_pool, v_pool, pool_dtype, table, rows, positions, scale, **kw):
    """Paged prefill (nest attention.linnet, prefill_paged): token p reads table[rows[p]]."""
    return attention(q_out, q_dtype, k_pool, v_pool, pool_dtype, table, rows,
                     positions, scale, **kw)


def output_gate(out, gate, gate_dtype: str) -> np.ndarray:
    """The sigmoid output gate, float64: fantasma fullAttentionForward multiplies
    every element of the attention output by ``sigmoid(gate)`` (the gate half of
    the q projection, same [n, heads*head_dim] layout)."""
    g = widen(gate, gate_dtype)
    return np.asarray(out, dtype=np.float64) * (1.0 / (1.0 + np.exp(-g)))


def packed(q_out, q_dtype: str, k_rows, v_rows, kv_dtype: str, segments, positions,
           scale: float, n_q_heads: int = NUM_Q_HEADS, n_kv_heads: int = NUM_KV_HEADS,
           head_dim: int = HEAD_DIM, tokens=None, return_weights: bool = False):
    """Prompts packed end to end attending only among themselves, float64.

    nest attention.linnet, ``prefill_packed`` and its training form ``packed``:
    token i attends with query head h over the pass's own tokens j that pass the
    mask ``own[i, j] = segments[i] == segments[j] and positions[j] <= positions[i]``,
    using the pass's keys and values ``k_rows`` / ``v_rows`` ([n, n_kv_heads, D]
    as stored) rather than the cache; the visible keys are taken in pack order.
    Returns out [len(tokens), n_q_heads*D] (and per-token weights if asked).
    """
    D = head_dim
    group = n_q_heads // n_kv_heads
    seg = np.asarray(segments)
    pos = np.asarray(positions)
    K = widen(k_rows, kv_dtype)
    V = widen(v_rows, kv_dtype)
    if tokens is None:
        tokens = range(len(pos))
    tokens = list(tokens)
    out = np.zeros((len(tokens), n_q_heads * D), dtype=np.float64)
    weights = []
    for i, t in enumerate(tokens):
        vis = np.nonzero((seg == seg[t]) & (pos <= pos[t]))[0]
        q = widen(q_out[t], q_dtype).reshape(n_q_heads, D)
        wt = []
        for g in range(n_kv_heads):
            o, w = attend(q[g * group:(g + 1) * group], K[vis, g], V[vis, g], scale)
            out[i, g * group * D:(g + 1) * group * D] = o.reshape(-1)
            wt.append(w)
        if return_weights:
            weights.append(np.concatenate(wt, axis=0))
    if return_weights:
        return out, weights
    return out


def step(q, k, v, in_dtype, pool_dtype, q_gain, k_gain, k_pool, v_pool, table,
         positions, rows, slots, step_positions, step_table, scale,
         eps: float = RMS_EPS, theta: float = ROPE_THETA, prefill_tokens=None,
         decode_rows=None):
    """The mixed step (nest attention.linnet, step_paged).

    One QK-norm + RoPE over the P prompt tokens followed by the R decode tokens;
    every write (prompt tokens at ``slots``, decode row b at its page slot of
    ``step_table[b]``) lands in the pools before any attention reads them; then
    prefill attention for the prompt tokens and paged decode for the rows.
    Mutates the pools. Returns (q_out, prefill_out, decode_out).
    """
    P = len(positions)
    R = len(step_positions)
    every_at = np.concatenate([np.asarray(positions), np.asarray(step_positions)])
    decode_slots = [page_slot(step_table[b], int(step_positions[b])) for b in range(R)]
    every_slot = np.concatenate([np.asarray(slots, dtype=np.int64),
                                 np.asarray(decode_slots, dtype=np.int64)])
    q_out, k_rows, v_rows = append(q, k, v, in_dtype, pool_dtype, q_gain, k_gain,
                                   every_at, eps=eps, theta=theta)
    apply_writes(k_pool, v_pool, every_slot, k_rows, v_rows)
    pre = prefill(q_out[:P], pool_dtype, k_pool, v_pool, pool_dtype, table, rows,
                  positions, scale, tokens=prefill_tokens)
    dec = decode(q_out[P:], pool_dtype, k_pool, v_pool, pool_dtype, step_table,
                 step_positions, scale, tokens=decode_rows)
    return q_out, pre, dec

"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test checks the oracle against what the pages or the mathematics fix:
library routines (torch CPU rms_norm, scaled_dot_product_attention, the
bfloat16 cast), closed forms, invariants and the constants the nest
qwen3-8b page prints.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- constants

def test_constants_match_page():
    vals = {}
    with open(os.path.join(GOLDEN, "qwen3_8b_constants.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    assert O.NUM_Q_HEADS == vals["num_q_heads"] == W.NUM_Q_HEADS
    assert O.NUM_KV_HEADS == vals["num_kv_heads"] == W.NUM_KV_HEADS
    assert O.HEAD_DIM == vals["head_dim"] == W.HEAD_DIM
    assert O.ROPE_THETA == vals["rope_theta"]
    assert O.RMS_EPS == vals["rms_eps"]
    assert O.PAGE_SIZE == vals["page_size"] == W.PAGE_SIZE
    assert W.MAX_POSITIONS == vals["max_positions"]


# ------------------------------------------------------------------ bfloat16

def test_bf16_round_matches_torch_cast():
    rng = _rng(1)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    # exact ties: low half 0x8000 with even and odd upper halves
    ties = (np.arange(2000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32).view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1e-40, -1e-40, 3.4e38])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits_from_f32(x), ref)
    back = O.f32_from_bf16_bits(ref)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


# --------------------------------------------------------------------- slots

def test_page_slot_brute_force():
    # a table whose pages are listed out of order: position p of row r lives in
    # page table[r][p // 64] at offset p % 64
    table = np.array([[5, 2, 7], [0, 6, 1]], dtype=np.int32)
    pool = {}
    for r in range(2):
        for page_idx, page in enumerate(table[r]):
            for off in range(64):
                pool[(r, page_idx * 64 + off)] = page * 64 + off
    for (r, p), s in pool.items():
        assert O.page_slot(table[r], p) == s
    assert list(O.row_slots(table[1], 66)[-3:]) == [63, 6 * 64, 6 * 64 + 1]


# ---------------------------------------------------------------- rope table

def test_rope_inv_freq_agrees_with_exp_log_form():
    # fantasma loadWeights writes 1/theta^(2i/dim); nest rope.linnet writes
    # exp(-(2i/D) * ln theta). Equal in real arithmetic.
    inv = O.rope_inv_freq(1e6, 128)
    alt = [math.exp(-(2.0 * i / 128) * math.log(1e6)) for i in range(64)]
    np.testing.assert_allclose(inv, alt, rtol=1e-14, atol=0)
    assert inv[0] == 1.0


def test_rope_table_closed_forms():
    cos, sin = O.rope_table(1e6, 300, 128)
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)
    # frequency 0 is exactly 1 rad per position
    np.testing.assert_allclose(cos[:, 0], np.cos(np.arange(300.0)), atol=6e-8)
    # unit circle and the angle-addition identity, in float64 from the f32 table
    c = cos.astype(np.float64)
    s = sin.astype(np.float64)
    assert np.max(np.abs(c * c + s * s - 1.0)) < 3e-7
    a, b = 117, 150
    np.testing.assert_allclose(c[a + b], c[a] * c[b] - s[a] * s[b], atol=3e-7)
    np.testing.assert_allclose(s[a + b], s[a] * c[b] + c[a] * s[b], atol=3e-7)
    # rows from rope_row agree with the table
    for p in (0, 1, 63, 299):
        rc, rs = O.rope_row(1e6, p, 128)
        assert np.array_equal(rc, cos[p]) and np.array_equal(rs, sin[p])


# ------------------------------------------------------------------- QK-norm

def test_qk_norm_matches_torch_rms_norm():
    rng = _rng(2)
    g = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    # ordinary scale, and small vectors where eps is not negligible
    x = np.concatenate([rng.standard_normal((200, 128)),
                        rng.standard_normal((200, 128)) * 1e-3]).astype(np.float32)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (128,),
                                       torch.from_numpy(g).double(), 1e-6).numpy()
    y = O.qk_norm(x, g, 1e-6)
    np.testing.assert_allclose(y, ref, rtol=2e-6, atol=1e-30)
    # eps really matters for the small rows: dropping it would be 40% off
    y_no_eps = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (128,),
                                            torch.from_numpy(g).double(), 0.0).numpy()
    assert np.max(np.abs(y_no_eps[200:] / ref[200:] - 1)) > 0.05


def test_qk_norm_invariants():
    rng = _rng(3)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    ones = np.ones(128, np.float32)
    y = O.qk_norm(x, ones, 1e-6).astype(np.float64)
    ms = np.mean(x.astype(np.float64) ** 2, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + 1e-6), rtol=2e-6)
    # scale invariance far above eps
    y2 = O.qk_norm(x * np.float32(64.0), ones, 1e-6).astype(np.float64)
    np.testing.assert_allclose(y2, y, rtol=2e-6, atol=1e-7)
    # normalises each head slice on its own, not the whole projection
    xs = np.concatenate([x[0], x[1] * np.float32(10)])  # two heads side by side
    per_head = O.qk_norm(xs.reshape(2, 128), ones, 1e-6)
    assert np.allclose(per_head[1], y[1], rtol=2e-6)


def test_qk_norm_zero_vector():
    y = O.qk_norm(np.zeros((1, 128), np.float32), np.ones(128, np.float32), 1e-6)
    assert np.all(y == 0.0)


# ---------------------------------------------------------------------- RoPE

def test_rope_is_complex_rotation_of_half_pairs():
    rng = _rng(4)
    y = rng.standard_normal((64, 128)).astype(np.float32)
    pos = rng.integers(0, 40960, 64)
    cs = np.stack([O.rope_row(1e6, int(p))[0] for p in pos])
    sn = np.stack([O.rope_row(1e6, int(p))[1] for p in pos])
    out = O.rope_rotate(y, cs, sn).astype(np.float64)
    z = (y[:, :64].astype(np.float64) + 1j * y[:, 64:].astype(np.float64)) * \
        (cs.astype(np.float64) + 1j * sn.astype(np.float64))
    np.testing.assert_allclose(out[:, :64], z.real, atol=2e-6)
    np.testing.assert_allclose(out[:, 64:], z.imag, atol=2e-6)


def test_rope_position_zero_is_identity_bitwise():
    rng = _rng(5)
    y = rng.standard_normal((10, 128)).astype(np.float32)
    c, s = O.rope_row(1e6, 0)
    assert np.array_equal(O.rope_rotate(y, c, s), y)


def test_rope_preserves_pair_norms():
    rng = _rng(6)
    y = rng.standard_normal((100, 128)).astype(np.float32)
    c, s = O.rope_row(1e6, 12345)
    out = O.rope_rotate(y, c, s).astype(np.float64)
    y = y.astype(np.float64)
    n0 = y[:, :64] ** 2 + y[:, 64:] ** 2
    n1 = out[:, :64] ** 2 + out[:, 64:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=3e-6, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    rng = _rng(7)
    q = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal(128).astype(np.float32)

    def score(m, n):
        cq, sq = O.rope_row(1e6, m)
        ck, sk = O.rope_row(1e6, n)
        return float(O.rope_rotate(q, cq, sq).astype(np.float64) @
                     O.rope_rotate(k, ck, sk).astype(np.float64))

    base = score(700, 300)
    for shift in (1, 64, 5000, 30000):
        assert abs(score(700 + shift, 300 + shift) - base) < 5e-4
    assert abs(score(700, 300) - score(300, 700)) > 1e-3


# -------------------------------------------------------------------- append

def _small_append_case(dtype, n=5, seed=8):
    rng = _rng(seed)
    q = rng.standard_normal((n, 32 * 128)).astype(np.float32)
    k = rng.standard_normal((n, 8 * 128)).astype(np.float32)
    v = rng.standard_normal((n, 8 * 128)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = (O.bf16_bits_from_f32(a) for a in (q, k, v))
    qg = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    kg = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    pos = rng.integers(0, 40960, n)
    return q, k, v, qg, kg, pos


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_matches_float64_norm_and_rotation(dtype):
    q, k, v, qg, kg, pos = _small_append_case(dtype)
    q_out, k_rows, v_rows = O.append(q, k, v, dtype, dtype, qg, kg, pos)
    # float64 reference of the same maths with torch routines: rms_norm per
    # head, then a complex rotation of (i, i+64) pairs
    qf = torch.from_numpy(O.as_f32(q, dtype).reshape(-1, 32, 128)).double()
    ref = torch.nn.functional.rms_norm(qf, (128,), torch.from_numpy(qg).double(), 1e-6).numpy()
    ang = np.array([[p * f for f in O.rope_inv_freq(1e6, 128)] for p in pos])
    z = (ref[..., :64] + 1j * ref[..., 64:]) * np.exp(1j * ang)[:, None, :]
    refq = np.concatenate([z.real, z.imag], axis=-1).reshape(len(pos), -1)
    got = O.widen(q_out, dtype)
    tol = 1e-5 if dtype == "f32" else 8e-3
    np.testing.assert_allclose(got, refq, rtol=tol, atol=tol)
    # V is stored as given (cast only)
    assert np.array_equal(v_rows.reshape(len(pos), -1), O.store(O.as_f32(v, dtype), dtype))


def test_apply_writes_skips_negative_slots():
    kp = np.zeros((8, 10, 128), np.float32)
    vp = np.zeros((8, 10, 128), np.float32)
    rows = np.ones((3, 8, 128), np.float32) * np.arange(1, 4, dtype=np.float32)[:, None, None]
    O.apply_writes(kp, vp, [4, -1, 9], rows, rows * 2)
    assert np.all(kp[:, 4] == 1) and np.all(kp[:, 9] == 3) and np.all(vp[:, 9] == 6)
    assert np.count_nonzero(kp) == 2 * 8 * 128


# ----------------------------------------------------------------- attention

def _tiny_pool(rng, n_pages, dtype="f32"):
    kp = rng.standard_normal((8, n_pages * 64, 128)).astype(np.float32)
    vp = rng.standard_normal((8, n_pages * 64, 128)).astype(np.float32)
    if dtype == "bf16":
        kp, vp = O.bf16_bits_from_f32(kp), O.bf16_bits_from_f32(vp)
    return kp, vp


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_matches_torch_sdpa(dtype):
    rng = _rng(9)
    kp, vp = _tiny_pool(rng, 6, dtype)
    table = np.array([[3, 0, 5], [1, 4, 2]], dtype=np.int32)
    positions = np.array([130, 7])
    q = rng.standard_normal((2, 32 * 128)).astype(np.float32)
    if dtype == "bf16":
        q = O.bf16_bits_from_f32(q)
    scale = W.SCALE
    out = O.decode(q, dtype, kp, vp, dtype, table, positions, scale)
    for b in range(2):
        n = positions[b] + 1
        slots = [table[b][j // 64] * 64 + j % 64 for j in range(n)]
        K = torch.from_numpy(O.widen(kp[:, slots], dtype))      # [8, n, 128]
        V = torch.from_numpy(O.widen(vp[:, slots], dtype))
        Q = torch.from_numpy(O.widen(q[b], dtype).reshape(32, 1, 128))
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None], K.repeat_interleave(4, dim=0)[None], V.repeat_interleave(4, dim=0)[None],
            scale=scale)[0, :, 0, :].reshape(-1).numpy()
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def test_attention_weights_sum_to_one_and_single_key():
    rng = _rng(10)
    kp, vp = _tiny_pool(rng, 2)
    table = np.array([[1, 0]], dtype=np.int32)
    q = rng.standard_normal((1, 32 * 128)).astype(np.float32)
    out, w = O.decode(q, "f32", kp, vp, "f32", table, np.array([100]), W.SCALE,
                      return_weights=True)
    np.testing.assert_allclose(w[0].sum(axis=1), 1.0, atol=1e-12)
    assert w[0].shape == (32, 101)
    # position 0: the only visible key is the token's own, so o = V_0 exactly
    out0 = O.decode(q, "f32", kp, vp, "f32", table, np.array([0]), W.SCALE)
    v0 = vp[:, 64].astype(np.float64)          # slot of position 0 = page 1, offset 0
    assert np.array_equal(out0[0].reshape(32, 128), np.repeat(v0, 4, axis=0))


def test_attention_uniform_when_query_is_zero_or_keys_equal():
    rng = _rng(11)
    kp, vp = _tiny_pool(rng, 2)
    table = np.array([[0, 1]], dtype=np.int32)
    n = 90
    vis = vp[:, :n].astype(np.float64)
    zero_q = np.zeros((1, 32 * 128), np.float32)
    out = O.decode(zero_q, "f32", kp, vp, "f32", table, np.array([n - 1]), W.SCALE)
    np.testing.assert_allclose(out[0].reshape(32, 128), np.repeat(vis.mean(axis=1), 4, axis=0),
                               rtol=1e-12, atol=1e-13)
    kp2 = kp.copy()
    kp2[:, :n] = kp2[:, :1]
    q = rng.standard_normal((1, 32 * 128)).astype(np.float32)
    out2 = O.decode(q, "f32", kp2, vp, "f32", table, np.array([n - 1]), W.SCALE)
    np.testing.assert_allclose(out2[0].reshape(32, 128), np.repeat(vis.mean(axis=1), 4, axis=0),
                               rtol=1e-12, atol=1e-13)


def test_gqa_grouping_uses_consecutive_query_heads():
    # query heads 4g..4g+3 read KV head g: change KV head 5 only and only
    # query heads 20..23 move
    rng = _rng(12)
    kp, vp = _tiny_pool(rng, 1)
    table = np.array([[0]], dtype=np.int32)
    q = rng.standard_normal((1, 32 * 128)).astype(np.float32)
    a = O.decode(q, "f32", kp, vp, "f32", table, np.array([40]), W.SCALE)
    vp2 = vp.copy()
    vp2[5] += 1.0
    b = O.decode(q, "f32", kp, vp2, "f32", table, np.array([40]), W.SCALE)
    moved = np.abs(a - b).reshape(32, 128).max(axis=1) > 0
    assert list(np.nonzero(moved)[0]) == [20, 21, 22, 23]


def test_paged_equals_contiguous_bitwise():
    rng = _rng(13)
    n_pages = 12
    kp, vp = _tiny_pool(rng, n_pages, "bf16")
    positions = np.array([250, 64, 5])
    q = O.bf16_bits_from_f32(rng.standard_normal((3, 32 * 128)).astype(np.float32))
    perm = rng.permutation(n_pages)
    # contiguous: row b owns pages 4b..4b+3 in order; paged: same data moved to
    # shuffled page ids
    ident = np.arange(12, dtype=np.int32).reshape(3, 4)
    shuf = perm[ident].astype(np.int32)
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    for p in range(n_pages):
        kp2[:, perm[p] * 64:(perm[p] + 1) * 64] = kp[:, p * 64:(p + 1) * 64]
        vp2[:, perm[p] * 64:(perm[p] + 1) * 64] = vp[:, p * 64:(p + 1) * 64]
    a = O.decode(q, "bf16", kp, vp, "bf16", ident, positions, W.SCALE)
    b = O.decode(q, "bf16", kp2, vp2, "bf16", shuf, positions, W.SCALE)
    assert np.array_equal(a, b)


def test_packed_prefill_equals_separate_prompts_bitwise():
    rng = _rng(14)
    kp, vp = _tiny_pool(rng, 8, "bf16")
    table = np.array([[0, 1, 2], [3, 4, 5]], dtype=np.int32)
    lens = [150, 70]
    rows = np.concatenate([np.zeros(lens[0], int), np.ones(lens[1], int)])
    positions = np.concatenate([np.arange(lens[0]), np.arange(lens[1])])
    q = O.bf16_bits_from_f32(rng.standard_normal((sum(lens), 32 * 128)).astype(np.float32))
    packed = O.prefill(q, "bf16", kp, vp, "bf16", table, rows, positions, W.SCALE)
    sep0 = O.prefill(q[:150], "bf16", kp, vp, "bf16", table, rows[:150], positions[:150], W.SCALE)
    sep1 = O.prefill(q[150:], "bf16", kp, vp, "bf16", table, rows[150:], positions[150:], W.SCALE)
    assert np.array_equal(packed, np.concatenate([sep0, sep1]))
    # a decode of the last token of a prompt is the same computation
    dec = O.decode(q[149:150], "bf16", kp, vp, "bf16", table[:1], positions[149:150], W.SCALE)
    assert np.array_equal(dec[0], packed[149])


def test_segment_mask_equals_paged_rows():
    # the packed, segment-masked form (nest attention.linnet prefill_packed:
    # own[i, j] = same segment and pos[j] <= pos[i], over the pass's own k/v)
    # equals the paged form when each prompt has its own row and starts at 0
    rng = _rng(15)
    lens = [40, 90, 30]
    seg = np.concatenate([np.full(n, s) for s, n in enumerate(lens)])
    pos = np.concatenate([np.arange(n) for n in lens])
    P = len(seg)
    k = rng.standard_normal((P, 8, 128)).astype(np.float32)
    v = rng.standard_normal((P, 8, 128)).astype(np.float32)
    q = rng.standard_normal((P, 32 * 128)).astype(np.float32)
    # pool: prompt s on page s (positions < 64 for the 40/30 prompts, two pages for 90)
    table = np.array([[0, 5], [1, 2], [3, 6]], dtype=np.int32)
    kp = np.full((8, 7 * 64, 128), np.nan, np.float32)
    vp = np.full((8, 7 * 64, 128), np.nan, np.float32)
    slots = [O.page_slot(table[s], p) for s, p in zip(seg, pos)]
    O.apply_writes(kp, vp, slots, k, v)
    paged = O.prefill(q, "f32", kp, vp, "f32", table, seg, pos, W.SCALE)
    Q = torch.from_numpy(q.reshape(P, 32, 128).transpose(1, 0, 2).copy()).double()
    K = torch.from_numpy(k.transpose(1, 0, 2).copy()).double().repeat_interleave(4, dim=0)
    V = torch.from_numpy(v.transpose(1, 0, 2).copy()).double().repeat_interleave(4, dim=0)
    own = torch.from_numpy((seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None]))
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=own,
                                                           scale=W.SCALE)
    ref = ref.permute(1, 0, 2).reshape(P, -1).numpy()
    np.testing.assert_allclose(paged, ref, rtol=1e-12, atol=1e-12)


def test_qk_norm_whole_matches_torch_rms_norm_over_all_heads():
    rng = _rng(20)
    x = rng.standard_normal((5, 32, 128)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 32 * 128).astype(np.float32)
    got = O.qk_norm_whole(x, g, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x.reshape(5, -1)).double(), (4096,),
                                       weight=torch.from_numpy(g).double(), eps=1e-6)
    np.testing.assert_allclose(got.reshape(5, -1), ref.numpy(), rtol=2e-6, atol=1e-6)


def test_qk_norm_whole_single_head_is_the_per_head_recipe_bitwise():
    rng = _rng(21)
    x = rng.standard_normal((7, 1, 128)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    assert np.array_equal(O.qk_norm_whole(x, g), O.qk_norm(x, g))


def test_qk_norm_whole_unit_gain_invariant():
    # with g = 1: mean of y^2 over all heads = ms / (ms + eps)
    rng = _rng(22)
    x = (0.01 * rng.standard_normal((3, 8, 128))).astype(np.float32)
    y = O.qk_norm_whole(x, np.ones(8 * 128, np.float32)).astype(np.float64)
    ms = (x.astype(np.float64) ** 2).reshape(3, -1).mean(axis=1)
    np.testing.assert_allclose((y ** 2).reshape(3, -1).mean(axis=1), ms / (ms + 1e-6), rtol=1e-5)


def test_partial_rotary_leaves_the_tail_and_rotates_the_head_bitwise():
    # fantasma applyRope with rotary_dim R: the first R elements rotate as an
    # R-wide head would, the others are unchanged
    rng = _rng(23)
    y = rng.standard_normal((6, 128)).astype(np.float32)
    for R in (32, 64, 96):
        c, s = O.rope_table(O.ROPE_THETA, 6, R)
        got = O.rope_rotate(y, c, s, R)
        assert np.array_equal(got[:, R:], y[:, R:])
        assert np.array_equal(got[:, :R], O.rope_rotate(y[:, :R], c, s))
    c, s = O.rope_table(O.ROPE_THETA, 6, 128)
    assert np.array_equal(O.rope_rotate(y, c, s, 128), O.rope_rotate(y, c, s))


def test_partial_rotary_scores_depend_on_relative_position_of_rotated_part():
    # <R(m)q, R(n)k> through the oracle's rope_rotate with rotary_dim R depends on
    # m - n only (up to float32 rounding); the unrotated tail adds the same
    # position-free term at any positions
    rng = _rng(24)
    R = 32
    q = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal(128).astype(np.float32)

    def rot(x, pos):
        c, s = O.rope_row(O.ROPE_THETA, pos, R)
        return O.rope_rotate(x, c, s, R).astype(np.float64)

    d1 = rot(q, 100) @ rot(k, 40)
    d2 = rot(q, 1060) @ rot(k, 1000)
    assert abs(d1 - d2) < 1e-4
    assert abs(d1 - rot(q, 40) @ rot(k, 100)) > 1e-3       # the sign of m - n matters
    tail = q[R:].astype(np.float64) @ k[R:].astype(np.float64)
    assert rot(q, 5)[R:] @ rot(k, 900)[R:] == tail
    # against the complex rotation of the first R elements in float64
    c, s = O.rope_row(O.ROPE_THETA, 777, R)
    z = (q[:R // 2] + 1j * q[R // 2:R]) * (c.astype(np.float64) + 1j * s.astype(np.float64))
    np.testing.assert_allclose(rot(q, 777)[:R], np.concatenate([z.real, z.imag]), atol=2e-6)


# ------------------------------------------------- the pinned float32 order
# The pages fix no intermediate precision for QK-norm; the oracle pins one float32
# order (neighbours-first pairwise sum of p_l = x_l^2 + x_{l+64}^2, an odd last
# element carried up). Below, a scalar transcription of that order in plain
# Python over numpy float32 scalars, and three other plausible orders. The inputs
# spread their squares over many octaves, so the orders round differently; the
# oracle must equal the pinned one bit for bit and differ from each other one.

F32 = np.float32


def _tree_neighbours(vals):
    vals = list(vals)
    while len(vals) > 1:
        nxt = [F32(vals[i] + vals[i + 1]) for i in range(0, len(vals) - 1, 2)]
        if len(vals) % 2:
            nxt.append(vals[-1])
        vals = nxt
    return vals[0]


def _xor_butterfly(vals):
    # s_l <- s_l + s_{l xor k} for k = 32, 16, ..., 1 over 64 lanes; lane 0's value
    s = list(vals)
    k = len(s) // 2
    while k >= 1:
        s = [F32(s[l] + s[l ^ k]) for l in range(len(s))]
        k //= 2
    return s[0]


def _sequential(vals):
    acc = F32(0.0)
    for v in vals:
        acc = F32(acc + v)
    return acc


def _numpy_sum(vals):
    return np.sum(np.array(vals, dtype=np.float32))


def _scalar_norm(x, g, eps, order):
    """One head (or, with ``order`` applied to head sums, see below) by the recipe."""
    d = len(x)
    half = d // 2
    p = [F32(F32(x[l] * x[l]) + F32(x[l + half] * x[l + half])) for l in range(half)]
    ss = order(p)
    ms = F32(ss / F32(d))
    r = F32(F32(1.0) / np.sqrt(F32(ms + F32(eps))))
    return np.array([F32(F32(x[i] * r) * g[i]) for i in range(d)], dtype=np.float32)


def _octave_vectors(rng, n, d=128):
    mag = np.exp2(rng.uniform(-8, 8, size=(n, d)))
    return (rng.standard_normal((n, d)) * mag).astype(np.float32)


def test_qk_norm_float32_order_is_the_pinned_one_bitwise():
    rng = _rng(30)
    x = _octave_vectors(rng, 200)
    g = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    got = O.qk_norm(x, g, 1e-6)
    differ = {"butterfly": 0, "sequential": 0, "numpy": 0}
    for i in range(len(x)):
        pinned = _scalar_norm(x[i], g, 1e-6, _tree_neighbours)
        assert np.array_equal(got[i].view(np.uint32), pinned.view(np.uint32)), i
        for name, order in (("butterfly", _xor_butterfly), ("sequential", _sequential),
                            ("numpy", _numpy_sum)):
            differ[name] += not np.array_equal(_scalar_norm(x[i], g, 1e-6, order).view(np.uint32),
                                               pinned.view(np.uint32))
    # each other order gives other bits on these inputs, so the check discriminates
    assert all(c > 0 for c in differ.values()), differ


def _scalar_norm_whole(x, g, eps, order=_tree_neighbours):
    """All heads of one token: per-head sums of squares by the recipe, then the head
    sums by ``order``, ms = total / (H*D)."""
    h, d = x.shape
    half = d // 2
    heads = [_tree_neighbours([F32(F32(x[j, l] * x[j, l]) + F32(x[j, l + half] * x[j, l + half]))
                               for l in range(half)]) for j in range(h)]
    total = order(heads)
    ms = F32(total / F32(h * d))
    r = F32(F32(1.0) / np.sqrt(F32(ms + F32(eps))))
    gg = np.asarray(g, np.float32).reshape(h, d)
    return np.array([[F32(F32(x[j, i] * r) * gg[j, i]) for i in range(d)] for j in range(h)], np.float32)


@pytest.mark.parametrize("heads", [3, 5, 12, 17, 20, 40, 68, 160])
def test_qk_norm_whole_at_odd_and_uneven_head_counts(heads):
    # the head counts the whole-vector variant is run at on the GPU (query heads
    # 12, 20, 68, 160; KV heads 3, 5, 17, 40): pinned order bit for bit, torch
    # rms_norm over all heads in float64, and a sequential head sum differs
    rng = _rng(31 + heads)
    n = 12
    x = (rng.standard_normal((n, heads, 128)) *
         np.exp2(rng.uniform(-10, 10, size=(n, heads, 1)))).astype(np.float32)
    g = rng.uniform(0.5, 1.5, heads * 128).astype(np.float32)
    got = O.qk_norm_whole(x, g, 1e-6)
    seq_differs = 0
    for t in range(n):
        pinned = _scalar_norm_whole(x[t], g, 1e-6)
        assert np.array_equal(got[t].view(np.uint32), pinned.view(np.uint32)), t
        seq_differs += not np.array_equal(_scalar_norm_whole(x[t], g, 1e-6, _sequential).view(np.uint32),
                                          pinned.view(np.uint32))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x.reshape(n, -1)).double(), (heads * 128,),
                                       weight=torch.from_numpy(g).double(), eps=1e-6).numpy()
    np.testing.assert_allclose(got.reshape(n, -1), ref, rtol=2e-6, atol=1e-30)
    if heads >= 5:
        assert seq_differs > 0


def test_output_gate_closed_forms():
    rng = _rng(25)
    out = rng.standard_normal((3, 256))
    zero = np.zeros((3, 256), np.float32)
    assert np.array_equal(O.output_gate(out, zero, "f32"), out * 0.5)
    g = rng.standard_normal((3, 256)).astype(np.float32)
    ref = torch.sigmoid(torch.from_numpy(g).double()).numpy() * out
    np.testing.assert_allclose(O.output_gate(out, g, "f32"), ref, rtol=1e-14, atol=1e-15)


def _packed_case(rng, lens, firsts, seg_ids, dtype="f32"):
    seg = np.concatenate([np.full(n, s) for s, n in zip(seg_ids, lens)])
    pos = np.concatenate([np.arange(f, f + n) for f, n in zip(firsts, lens)])
    P = len(seg)
    k = rng.standard_normal((P, 8, 128)).astype(np.float32)
    v = rng.standard_normal((P, 8, 128)).astype(np.float32)
    q = rng.standard_normal((P, 32 * 128)).astype(np.float32)
    if dtype == "bf16":
        k, v, q = O.bf16_bits_from_f32(k), O.bf16_bits_from_f32(v), O.bf16_bits_from_f32(q)
    return seg, pos, q, k, v


def test_packed_matches_sdpa_with_own_mask():
    # nest attention.linnet prefill_packed / packed: own[i, j] = same segment and
    # positions[j] <= positions[i], over the pass's own keys; segment ids need not
    # be ordered and a prompt may start past position 0 (its history is not seen)
    rng = _rng(16)
    seg, pos, q, k, v = _packed_case(rng, [40, 90, 30], [0, 300, 7], [7, 2, 5])
    P = len(seg)
    got = O.packed(q, "f32", k, v, "f32", seg, pos, W.SCALE)
    Q = torch.from_numpy(q.reshape(P, 32, 128).transpose(1, 0, 2).copy()).double()
    K = torch.from_numpy(k.transpose(1, 0, 2).copy()).double().repeat_interleave(4, dim=0)
    V = torch.from_numpy(v.transpose(1, 0, 2).copy()).double().repeat_interleave(4, dim=0)
    own = torch.from_numpy((seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None]))
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=own, scale=W.SCALE)
    ref = ref.permute(1, 0, 2).reshape(P, -1).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_packed_brute_force_tiny():
    # pure-Python loops with math.exp at Hq=4, Hkv=2, D=8
    rng = _rng(17)
    seg = np.array([3, 3, 3, 1, 1, 4, 4, 4, 4])
    pos = np.array([5, 6, 7, 0, 1, 2, 3, 4, 5])
    n, hq, hk, d = len(seg), 4, 2, 8
    q = rng.standard_normal((n, hq * d))
    k = rng.standard_normal((n, hk, d))
    v = rng.standard_normal((n, hk, d))
    got = O.packed(q, "f64", k, v, "f64", seg, pos, 0.3, n_q_heads=hq, n_kv_heads=hk, head_dim=d)
    for i in range(n):
        for h in range(hq):
            g = h // (hq // hk)
            js = [j for j in range(n) if seg[j] == seg[i] and pos[j] <= pos[i]]
            sc = [0.3 * sum(q[i, h * d + e] * k[j, g, e] for e in range(d)) for j in js]
            mx = max(sc)
            ex = [math.exp(x - mx) for x in sc]
            tot = sum(ex)
            for e in range(d):
                ref = sum(ex[a] * v[j, g, e] for a, j in enumerate(js)) / tot
                assert abs(got[i, h * d + e] - ref) < 1e-12


def test_packed_equals_paged_when_prompts_start_at_zero_bitwise():
    # every prompt at positions 0.. on private pages: the packed form and the
    # paged form see the same keys in the same order
    rng = _rng(18)
    seg, pos, q, k, v = _packed_case(rng, [70, 20, 130], [0, 0, 0], [0, 1, 2], "bf16")
    table = np.array([[4, 0, 9], [2, 7, 8], [1, 3, 5]], dtype=np.int32)
    kp = np.zeros((8, 10 * 64, 128), np.uint16)
    vp = np.zeros((8, 10 * 64, 128), np.uint16)
    O.apply_writes(kp, vp, [O.page_slot(table[s], p) for s, p in zip(seg, pos)], k, v)
    a = O.packed(q, "bf16", k, v, "bf16", seg, pos, W.SCALE)
    b = O.prefill(q, "bf16", kp, vp, "bf16", table, seg, pos, W.SCALE)
    assert np.array_equal(a, b)


def test_packed_ignores_history_bitwise():
    # a prompt chunk at positions 300.. attends only to itself: the same as the
    # paged form of the same keys placed at positions 0.. of a fresh row (the
    # mask uses positions only through their order within the prompt)
    rng = _rng(19)
    seg, pos, q, k, v = _packed_case(rng, [100, 50], [300, 64], [0, 1], "bf16")
    a = O.packed(q, "bf16", k, v, "bf16", seg, pos, W.SCALE)
    rel = np.concatenate([np.arange(100), np.arange(50)])
    table = np.array([[0, 1], [2, 3]], dtype=np.int32)
    kp = np.zeros((8, 4 * 64, 128), np.uint16)
    vp = np.zeros((8, 4 * 64, 128), np.uint16)
    O.apply_writes(kp, vp, [O.page_slot(table[s], p) for s, p in zip(seg, rel)], k, v)
    b = O.prefill(q, "bf16", kp, vp, "bf16", table, seg, rel, W.SCALE)
    assert np.array_equal(a, b)


def test_step_writes_before_reads():
    # a prompt chunk sees its own keys through the pool: the first token of a
    # chunk at position 0 attends to exactly its own value
    w = W.build("t", 3, "f32", num_pages=4, pages_per_row=2, n_table_rows=2,
                chunks=[(0, 0, 3)], decode=[(1, 0)], decode_row0=1)
    kp = np.full((8, w.pool_slots, 128), np.nan, np.float32)
    vp = np.full((8, w.pool_slots, 128), np.nan, np.float32)
    q_out, pre, dec = O.step(w.q, w.k, w.v, "f32", "f32", w.q_gain, w.k_gain, kp, vp,
                             w.table, w.positions, w.rows, w.slots, w.step_positions,
                             w.decode_table, W.SCALE)
    v0 = w.v[0].reshape(8, 128).astype(np.float64)
    assert np.array_equal(pre[0].reshape(32, 128), np.repeat(v0, 4, axis=0))
    vd = w.v[3].reshape(8, 128).astype(np.float64)
    assert np.array_equal(dec[0].reshape(32, 128), np.repeat(vd, 4, axis=0))
    assert not np.isnan(pre).any()

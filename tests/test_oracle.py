"""Pins for the fp64 oracle: closed forms, invariants the pages state, textbook
library routines and brute force. CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- rotation

def test_theta_closed_form():
    # base ** (-2i/d): d=4, base=1e4 -> [1, 1e-2]; d=8, base=1e6 -> 1e6**[0,-1/4,-1/2,-3/4]
    assert np.allclose(O.rope_theta(4, 1e4), [1.0, 0.01], rtol=0, atol=1e-15)
    assert np.allclose(O.rope_theta(8, 1e6), [1.0, 10 ** -1.5, 1e-3, 10 ** -4.5], rtol=1e-14, atol=0)


def test_rotation_sign_and_angle_d2():
    # d = 2: theta_0 = 1, the angle is r radians; the block [[c,-s],[s,c]] maps
    # (1,0) -> (cos r, sin r) and (0,1) -> (-sin r, cos r)  (P-RoPE page Eq. (2)).
    for r in (0, 1, 3, -5, 8191, 131071):
        y = O.rotate(np.array([1.0, 0.0]), r, 1e4)
        assert np.allclose(y, [math.cos(r), math.sin(r)], atol=1e-12)
        y = O.rotate(np.array([0.0, 1.0]), r, 1e6)
        assert np.allclose(y, [-math.sin(r), math.cos(r)], atol=1e-12)


def test_rotation_closed_form_d4():
    # d = 4, base 1e4: angles (3, 0.03) for r = 3
    x = np.array([1.0, 2.0, -0.5, 4.0])
    c0, s0, c1, s1 = math.cos(3), math.sin(3), math.cos(0.03), math.sin(0.03)
    want = [c0 * 1 - s0 * 2, s0 * 1 + c0 * 2, c1 * -0.5 - s1 * 4, s1 * -0.5 + c1 * 4]
    assert np.allclose(O.rotate(x, 3, 1e4), want, atol=1e-14)


def test_rotation_matches_complex_multiplication():
    # independent construction: pair (a, b) as a + ib times exp(i r theta_i)
    rng = _rng(1)
    d = 16
    x = rng.standard_normal((7, d))
    r = rng.integers(-200000, 200000, size=7)
    th = np.array([1e6 ** (-(2 * i) / d) for i in range(d // 2)])
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * r[:, None] * th[None, :])
    want = np.empty_like(x)
    want[:, 0::2], want[:, 1::2] = z.real, z.imag
    assert np.allclose(O.rotate(x, r, 1e6), want, atol=1e-11)


def test_rotation_norm_identity_composition():
    rng = _rng(2)
    x = rng.standard_normal((50, 128))
    r = rng.integers(0, 131072, size=50)
    y = O.rotate(x, r, 1e6)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.array_equal(O.rotate(x, 0, 1e4), x)
    a = rng.integers(-5000, 5000, size=50)
    b = rng.integers(-5000, 5000, size=50)
    # R_a R_b = R_{a+b}  (Jet-Long page, section 3.2)
    assert np.allclose(O.rotate(O.rotate(x, b, 1e4), a, 1e4), O.rotate(x, a + b, 1e4), atol=1e-11)
    assert np.allclose(O.rotate(O.rotate(x, a, 1e4), -a, 1e4), x, atol=1e-11)


def test_relative_offset_property():
    # (R_t q)^T (R_s k) = q^T R_{s-t} k  (P-RoPE page, Eq. (3), with the sign of
    # the offset written so that it holds; the printed R_{t-s} is a sign slip)
    rng = _rng(3)
    q = rng.standard_normal((20, 64))
    k = rng.standard_normal((20, 64))
    t = rng.integers(0, 10000, size=20)
    s = rng.integers(0, 10000, size=20)
    lhs = np.sum(O.rotate(q, t, 1e4) * O.rotate(k, s, 1e4), axis=1)
    rhs = np.sum(q * O.rotate(k, s - t, 1e4), axis=1)
    assert np.allclose(lhs, rhs, atol=1e-10)


def test_rope_apply_negative_ids_undo():
    rng = _rng(4)
    x = rng.standard_normal((2, 5, 3, 8))
    p = rng.integers(0, 70000, size=(2, 5))
    y = O.rope_apply_ref(O.rope_apply_ref(x, p, 1e6), -p, 1e6)
    assert np.allclose(y, x, atol=1e-11)


# ----------------------------------------------------------------- rounding

def test_bf16_rounding_matches_torch_on_float32_values():
    rng = _rng(5)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # plant exact ties: 1 + 2^-8 -> 1 (even), 1 + 3*2^-8 -> 1 + 2^-6 (even)
    x[:4] = [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3 * 2 ** -9 + 1]
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
    assert got[0] == 1.0 and got[1] == 1 + 2 ** -6


def test_bf16_rounding_exact_rational():
    # float64 inputs not representable in float32: nearest multiple of the
    # bf16 spacing in the value's binade, ties to even, by exact rationals
    rng = _rng(6)
    vals = rng.standard_normal(300) * 10.0 ** rng.integers(-3, 4, 300)
    for x in vals:
        fx = Fraction(float(x))
        e = math.floor(math.log2(abs(x)))
        spacing = Fraction(2) ** (e - 7)
        q, rem = divmod(fx, spacing)
        if rem * 2 > spacing or (rem * 2 == spacing and q % 2 == 1):
            q += 1
        assert float(q * spacing) == O.round_to_bf16(np.array([x]))[0]


# ----------------------------------------------------------------- id maps

def test_periodic_index_eq4():
    assert list(O.periodic_index([0, 1023, 1024, 2049, 8191], 1024)) == [0, 1023, 0, 1, 1023]
    assert list(O.periodic_index([5, 7], 0)) == [5, 7]


def test_group_size_eq2_golden():
    g = json.load(open(os.path.join(GOLDEN, "group_size.json")))
    for L, G in g["cases"]:
        assert O.group_size(L, g["w_pretrained"]) == G


def test_remote_index_eq3():
    assert list(O.remote_index([0, 1, 2, 3, 7, 131071], 4)) == [0, 0, 0, 0, 1, 32767]
    assert list(O.remote_index([0, 5, 9], 1)) == [0, 5, 9]


def test_endprompt_ids_golden():
    import workloads
    g = json.load(open(os.path.join(GOLDEN, "endprompt_ids.json")))
    ids = workloads.endprompt_ids()
    assert ids.shape[0] == g["length"]
    assert ids[0] == g["first_segment"][0] and ids[191] == g["first_segment"][1]
    assert ids[192] == g["second_segment"][0] and ids[-1] == g["second_segment"][1]
    assert np.all(np.diff(ids[:192]) == 1) and np.all(np.diff(ids[192:]) == 1)


def test_prop1_same_phi_never_share_window():
    # P-RoPE Prop. 1: with period W and a window of W keys (i - j <= W - 1),
    # the periodic indices inside any window are distinct.
    W = 16
    t = np.arange(200)
    phi = O.periodic_index(t, W)
    for i in range(200):
        win = phi[max(0, i - W + 1): i + 1]
        assert len(set(win.tolist())) == len(win)


def test_case2_offset_off_by_period():
    # P-RoPE Case 2: across a period boundary phi(t) - phi(t') = (t - t') - W, so the
    # periodic score equals a plain-RoPE score with the key moved W later.
    rng = _rng(7)
    W = 64
    q = rng.standard_normal((1, 32))
    k = rng.standard_normal((1, 32))
    for t, tp in [(130, 100), (64, 63), (200, 150)]:
        assert t // W != tp // W and t - tp <= W - 1
        s_per = float(np.sum(O.rotate(q, t % W, 1e4) * O.rotate(k, tp % W, 1e4)))
        s_shift = float(np.sum(O.rotate(q, t, 1e4) * O.rotate(k, tp + W, 1e4)))
        assert abs(s_per - s_shift) < 1e-10
    # Case 1: same period block, the offset is exact
    t, tp = 70, 66
    s_per = float(np.sum(O.rotate(q, t % W, 1e4) * O.rotate(k, tp % W, 1e4)))
    s_plain = float(np.sum(O.rotate(q, t, 1e4) * O.rotate(k, tp, 1e4)))
    assert abs(s_per - s_plain) < 1e-10


# ----------------------------------------------------------------- attention

def _rand_qkv(B, S, Hq, Hkv, d, seed):
    rng = _rng(seed)
    return (rng.standard_normal((B, S, Hq, d)), rng.standard_normal((B, S, Hkv, d)),
            rng.standard_normal((B, S, Hkv, d)))


def _sdpa(q, k, v, mask=None, causal=False):
    """torch scaled_dot_product_attention in float64 on CPU; [B,S,H,d] layout, GQA by
    repeating each KV head over its contiguous group of query heads."""
    grp = q.shape[2] // k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).repeat_interleave(grp, dim=2).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).repeat_interleave(grp, dim=2).permute(0, 2, 1, 3)
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal)
    return o.permute(0, 2, 1, 3).numpy()


def test_nope_equals_sdpa_causal_gqa():
    q, k, v = _rand_qkv(2, 37, 8, 2, 16, 10)
    pos = np.tile(np.arange(37), (2, 1))
    o, lse = O.prefill_ref(q, k, v, pos, "nope")
    assert np.allclose(o, _sdpa(q, k, v, causal=True), atol=1e-12)
    # LSE against torch.logsumexp of the causal scores
    grp = 4
    sc = np.einsum("bihd,bjhd->bhij", q, np.repeat(k, grp, axis=2)) / 4.0
    sc = np.where(np.tril(np.ones((37, 37), bool)), sc, -np.inf)
    want = torch.logsumexp(torch.from_numpy(sc), dim=-1).numpy()
    assert np.allclose(lse, want, atol=1e-12)


def test_rope_equals_sdpa_on_prerotated_inputs():
    # rotate with complex multiplication (independent of O.rotate), then SDPA
    B, S, Hq, Hkv, d, base = 1, 29, 4, 2, 8, 1e4
    q, k, v = _rand_qkv(B, S, Hq, Hkv, d, 11)
    pos = np.array([[0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18,
                     900, 901, 902, 903, 904, 905, 906, 907, 908, 909]])
    th = np.array([base ** (-(2 * i) / d) for i in range(d // 2)])

    def crot(x):
        z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos[:, :, None, None] * th)
        y = np.empty_like(x)
        y[..., 0::2], y[..., 1::2] = z.real, z.imag
        return y

    o, _ = O.prefill_ref(q, k, v, pos, "rope", rope_base=base)
    assert np.allclose(o, _sdpa(crot(q), crot(k), v, causal=True), atol=1e-12)


def test_window_equals_sdpa_with_boolean_mask():
    q, k, v = _rand_qkv(1, 40, 2, 2, 8, 12)
    pos = np.arange(40)[None]
    W = 7                                     # window of W keys including self
    i = np.arange(40)[:, None]
    j = np.arange(40)[None, :]
    mask = (j <= i) & (j >= i - (W - 1))      # P-RoPE window {t-W+1, ..., t}
    o, _ = O.prefill_ref(q, k, v, pos, "nope", window_left=W - 1)
    assert np.allclose(o, _sdpa(q, k, v, mask=mask), atol=1e-12)


def test_window_uniform_closed_form():
    # q = 0 -> uniform weights over kept keys; v_j = (j, 1) -> O_i = mean kept j, LSE = log count
    S, W = 50, 9
    q = np.zeros((1, S, 1, 2))
    k = _rng(13).standard_normal((1, S, 1, 2))
    v = np.zeros((1, S, 1, 2))
    v[0, :, 0, 0] = np.arange(S)
    v[0, :, 0, 1] = 1.0
    o, lse = O.prefill_ref(q, k, v, np.arange(S)[None], "rope", window_left=W - 1)
    for i in range(S):
        lo = max(0, i - W + 1)
        assert abs(o[0, i, 0, 0] - (lo + i) / 2) < 1e-12
        assert abs(lse[0, 0, i] - math.log(i - lo + 1)) < 1e-12


def test_bifocal_closed_form_golden():
    g = json.load(open(os.path.join(GOLDEN, "bifocal_d2_closed_form.json")))
    S, w0, s, row = g["S"], g["w0"], g["s"], g["row"]
    q = np.zeros((1, S, 1, 2)); q[..., 0] = 1.0
    k = np.zeros((1, S, 1, 2)); k[..., 0] = 1.0
    v = np.zeros((1, S, 1, 2)); v[0, :, 0, 0] = np.arange(S); v[0, :, 0, 1] = 1.0
    o, lse = O.prefill_ref(q, k, v, np.arange(S)[None], "bifocal", rope_base=1e6,
                           remap_scale=s, window_left=w0, softmax_scale=1.0)
    sc = [eval(e, {"cos": math.cos}) for e in g["key_scores_expr"]]
    w = [math.exp(x) for x in sc]
    assert abs(lse[0, 0, row] - math.log(sum(w))) < 1e-13
    assert abs(o[0, row, 0, 0] - sum(j * wj for j, wj in enumerate(w)) / sum(w)) < 1e-13
    assert abs(o[0, row, 0, 1] - 1.0) < 1e-13


@pytest.mark.parametrize("mode,kw", [
    ("nope", dict()),
    ("nope", dict(window_left=3)),
    ("rope", dict(rope_base=1e4)),
    ("rope", dict(rope_base=1e4, period=5, window_left=4)),
    ("rope", dict(rope_base=1e6, window_left=0)),
    ("bifocal", dict(rope_base=1e6, remap_scale=3, window_left=4)),
    ("bifocal", dict(rope_base=1e4, remap_scale=2, window_left=0)),
    ("bifocal", dict(rope_base=1e4, remap_scale=4, window_left=-1)),
])
def test_vectorized_equals_brute_force(mode, kw):
    B, S, Hq, Hkv, d = 2, 12, 4, 2, 6
    q, k, v = _rand_qkv(B, S, Hq, Hkv, d, 14)
    pos = np.stack([np.arange(S), np.concatenate([np.arange(6), np.arange(100, 106)])])
    o, _ = O.prefill_ref(q, k, v, pos, mode, **kw)
    bf = np.array(O.brute_force_prefill(q, k, v, pos, mode, kw.get("rope_base", 1e4),
                                        period=kw.get("period", 0),
                                        remap_scale=kw.get("remap_scale", 1),
                                        window_left=kw.get("window_left", -1)))
    assert np.allclose(o, bf, atol=1e-12)


def test_rows_subset_matches_full():
    q, k, v = _rand_qkv(1, 70, 4, 2, 8, 15)
    pos = np.arange(70)[None]
    o, l = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=1e6, remap_scale=2, window_left=9)
    rows = np.array([0, 5, 9, 10, 11, 69])
    o2, l2 = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=1e6, remap_scale=2, window_left=9,
                           rows=rows, max_block_elems=100)
    assert np.allclose(o2, o[:, rows], atol=1e-13)
    assert np.allclose(l2, l[:, :, rows], atol=1e-13)


# ----------------------------------------------------------------- invariants

def test_shift_invariance_rope():
    q, k, v = _rand_qkv(1, 33, 2, 1, 16, 16)
    pos = np.arange(33)[None]
    o1, _ = O.prefill_ref(q, k, v, pos, "rope", rope_base=1e4)
    o2, _ = O.prefill_ref(q, k, v, pos + 12345, "rope", rope_base=1e4)
    assert np.allclose(o1, o2, atol=1e-9)


def test_shift_by_multiple_of_s_invariance_bifocal():
    q, k, v = _rand_qkv(1, 33, 2, 1, 16, 17)
    pos = np.arange(33)[None]
    kw = dict(rope_base=1e6, remap_scale=3, window_left=5)
    o1, _ = O.prefill_ref(q, k, v, pos, "bifocal", **kw)
    o2, _ = O.prefill_ref(q, k, v, pos + 3 * 4000, "bifocal", **kw)
    assert np.allclose(o1, o2, atol=1e-9)


def test_period_at_least_S_is_plain_rope():
    q, k, v = _rand_qkv(1, 30, 2, 2, 8, 18)
    pos = np.arange(30)[None]
    o1, _ = O.prefill_ref(q, k, v, pos, "rope", rope_base=1e4, period=30, window_left=10)
    o2, _ = O.prefill_ref(q, k, v, pos, "rope", rope_base=1e4, period=0, window_left=10)
    assert np.allclose(o1, o2, atol=1e-13)


def test_period_applied_equals_prereduced_ids():
    q, k, v = _rand_qkv(1, 40, 2, 2, 8, 19)
    pos = np.arange(40)[None]
    o1, _ = O.prefill_ref(q, k, v, pos, "rope", period=16, window_left=15)
    o2, _ = O.prefill_ref(q, k, v, pos % 16, "rope", period=0, window_left=15)
    assert np.array_equal(o1, o2)


def test_full_window_equals_causal():
    q, k, v = _rand_qkv(1, 25, 2, 1, 8, 20)
    pos = np.arange(25)[None]
    for mode in ("nope", "rope"):
        o1, _ = O.prefill_ref(q, k, v, pos, mode, window_left=24)
        o2, _ = O.prefill_ref(q, k, v, pos, mode, window_left=-1)
        assert np.array_equal(o1, o2)


def test_bifocal_reductions_to_plain_rope():
    q, k, v = _rand_qkv(1, 31, 4, 2, 8, 21)
    pos = np.arange(31)[None]
    plain, _ = O.prefill_ref(q, k, v, pos, "rope", rope_base=1e6)
    # s = 1: f(x) = x, the base model (Jet-Long page, section 3)
    o, _ = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=1e6, remap_scale=1, window_left=4)
    assert np.allclose(o, plain, atol=1e-12)
    # w0 >= S - 1: all keys local
    o, _ = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=1e6, remap_scale=3, window_left=30)
    assert np.allclose(o, plain, atol=1e-12)
    # w0 = -1: all keys remote, plain RoPE at ids floor(p/s)
    o, _ = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=1e6, remap_scale=3, window_left=-1)
    o_r, _ = O.prefill_ref(q, k, v, pos // 3, "rope", rope_base=1e6)
    assert np.allclose(o, o_r, atol=1e-12)


def test_bifocal_w0_zero_self_only_local():
    # Jet-Long section 4.4: w0 = 0 keeps only the query's own key in the local window
    S = 9
    q, k, v = _rand_qkv(1, S, 1, 1, 4, 22)
    pos = np.arange(S)[None]
    o, _ = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=1e4, remap_scale=2, window_left=0)
    i = S - 1
    qb = O.rotate(q[0, i, 0], i, 1e4)
    kb = O.rotate(k[0, i, 0], i, 1e4)
    sc = [float(qb @ kb) / 2]
    for j in range(i):
        sc.insert(j, float(O.rotate(q[0, i, 0], i // 2, 1e4) @ O.rotate(k[0, j, 0], j // 2, 1e4)) / 2)
    w = np.exp(np.array(sc) - max(sc))
    assert np.allclose(o[0, i, 0], (w[:, None] * v[0, :, 0]).sum(0) / w.sum(), atol=1e-13)


def test_eq7_merge_equals_direct():
    q, k, v = _rand_qkv(1, 48, 4, 2, 8, 23)
    pos = np.arange(48)[None]
    for w0, s in [(5, 2), (0, 3), (47, 4), (-1, 2), (10, 1)]:
        direct, _ = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=1e6, remap_scale=s, window_left=w0)
        eq7 = O.bifocal_eq7_ref(q, k, v, pos, rope_base=1e6, remap_scale=s, window_left=w0)
        assert np.allclose(eq7, direct, atol=1e-10), (w0, s)


# ----------------------------------------------------------------- decode

@pytest.mark.parametrize("L,s,w0", [(40, 4, 6), (33, 2, 0), (17, 3, -1), (25, 1, 5), (20, 4, 30)])
def test_decode_equals_last_prefill_row(L, s, w0):
    # cache of base-rotated keys (Jet-Long Eq. (4)) plus the correction rotation
    # (Eq. (5)-(6)) reproduces the last row of direct bifocal attention
    B, Hq, Hkv, d, base = 2, 4, 2, 16, 1e6
    q, k, v = _rand_qkv(B, L, Hq, Hkv, d, 24)
    pos = np.tile(np.arange(L), (B, 1))
    o_pre, l_pre = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=base, remap_scale=s, window_left=w0)
    kc = O.rope_apply_ref(k, pos, base)
    ql = O.rope_apply_ref(q[:, -1:], pos[:, -1:], base)[:, 0]
    o_dec, l_dec = O.decode_ref(ql, kc, v, np.full(B, L), "bifocal", rope_base=base,
                                remap_scale=s, window_left=w0)
    assert np.allclose(o_dec, o_pre[:, -1], atol=1e-10)
    assert np.allclose(l_dec, l_pre[:, :, -1], atol=1e-10)


def test_decode_rope_window_equals_prefill_last_row():
    B, L, Hq, Hkv, d = 1, 30, 2, 1, 8
    q, k, v = _rand_qkv(B, L, Hq, Hkv, d, 25)
    pos = np.arange(L)[None]
    o_pre, _ = O.prefill_ref(q, k, v, pos, "rope", rope_base=1e4, period=8, window_left=7)
    r = pos % 8
    kc = O.rope_apply_ref(k, r, 1e4)
    ql = O.rope_apply_ref(q[:, -1:], r[:, -1:], 1e4)[:, 0]
    o_dec, _ = O.decode_ref(ql, kc, v, [L], "rope", window_left=7)
    assert np.allclose(o_dec, o_pre[:, -1], atol=1e-12)


def test_decode_ragged_kv_len():
    B, L, Hq, Hkv, d = 3, 20, 2, 2, 8
    q, k, v = _rand_qkv(B, L, Hq, Hkv, d, 26)
    lens = [20, 1, 7]
    o, l = O.decode_ref(q[:, 0], k, v, lens, "bifocal", rope_base=1e4, remap_scale=2, window_left=3)
    for b, n in enumerate(lens):
        o1, l1 = O.decode_ref(q[b:b + 1, 0], k[b:b + 1, :n], v[b:b + 1, :n], [n], "bifocal",
                              rope_base=1e4, remap_scale=2, window_left=3)
        assert np.allclose(o[b], o1[0], atol=1e-14) and np.allclose(l[b], l1[0], atol=1e-14)
    # one key: output is that value row
    assert np.allclose(o[1], v[1, 0][np.arange(Hq) // 1], atol=1e-14)


def test_decode_empty_sequence():
    """kv_len 0 (an empty slot in a batch): no key, so O = 0 and LSE = -inf, and the
    other sequences' results are what they are alone."""
    B, L, Hq, Hkv, d = 3, 20, 4, 2, 8
    q, k, v = _rand_qkv(B, L, Hq, Hkv, d, 27)
    lens = [0, 13, 0]
    o, l = O.decode_ref(q[:, 0], k, v, lens, "bifocal", rope_base=1e4, remap_scale=2, window_left=3)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert np.all(np.isneginf(l[0])) and np.all(np.isneginf(l[2]))
    o1, l1 = O.decode_ref(q[1:2, 0], k[1:2, :13], v[1:2, :13], [13], "bifocal",
                          rope_base=1e4, remap_scale=2, window_left=3)
    assert np.allclose(o[1], o1[0], atol=1e-14) and np.allclose(l[1], l1[0], atol=1e-14)
    # nope/rope go through the same masked softmax
    o, l = O.decode_ref(q[:, 0], k, v, lens, "nope", window_left=5)
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[2])) and np.all(np.isfinite(l[1]))


def test_operand_rounding_identity_on_bf16_inputs():
    rng = _rng(27)
    q = O.round_to_bf16(rng.standard_normal((1, 20, 2, 8)))
    k = O.round_to_bf16(rng.standard_normal((1, 20, 2, 8)))
    v = rng.standard_normal((1, 20, 2, 8))
    pos = np.arange(20)[None]
    a, _ = O.prefill_ref(q, k, v, pos, "nope", operand_round="bf16")
    b, _ = O.prefill_ref(q, k, v, pos, "nope")
    assert np.array_equal(a, b)
    c, _ = O.prefill_ref(q, k, v, pos, "rope", operand_round="bf16")
    d_, _ = O.prefill_ref(q, k, v, pos, "rope")
    assert 0 < np.max(np.abs(c - d_)) < 0.05


# ---------------------------------------------------------------- interpolated remote mapping
# (Jet-Long page, section 4.5: remote view with frequencies theta_i / s at the
# original positions instead of aliased positions floor(p / s))

def test_interp_all_remote_equals_sdpa_on_complex_rotation():
    # w0 = -1: every key remote; rotate at angle p * theta_i / s with complex
    # multiplication (independent of O.rotate), then the library's SDPA
    B, S, Hq, Hkv, d, base, s = 1, 27, 4, 2, 8, 1e6, 3
    q, k, v = _rand_qkv(B, S, Hq, Hkv, d, 31)
    pos = np.arange(S)[None] * 7 + 5
    th = np.array([base ** (-(2 * i) / d) for i in range(d // 2)]) / s

    def crot(x):
        z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos[:, :, None, None] * th)
        y = np.empty_like(x)
        y[..., 0::2], y[..., 1::2] = z.real, z.imag
        return y

    o, _ = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=base, remap_scale=s, window_left=-1,
                         remote_map="interp")
    assert np.allclose(o, _sdpa(crot(q), crot(k), v, causal=True), atol=1e-12)


def test_interp_vectorized_equals_brute_force():
    B, S, Hq, Hkv, d = 1, 11, 2, 1, 6
    q, k, v = _rand_qkv(B, S, Hq, Hkv, d, 32)
    pos = np.arange(S)[None] + 3
    o, _ = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=1e4, remap_scale=3, window_left=2,
                         remote_map="interp")
    bf = np.array(O.brute_force_prefill(q, k, v, pos, "bifocal", 1e4, remap_scale=3, window_left=2,
                                        remote_map="interp"))
    assert np.allclose(o, bf, atol=1e-12)


def test_interp_scale_one_and_shift_invariance():
    q, k, v = _rand_qkv(1, 25, 4, 2, 8, 33)
    pos = np.arange(25)[None]
    plain, _ = O.prefill_ref(q, k, v, pos, "rope", rope_base=1e6)
    o1, _ = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=1e6, remap_scale=1, window_left=5,
                          remote_map="interp")
    assert np.allclose(o1, plain, atol=1e-12)
    # unlike aliasing (invariant only under shifts by multiples of s), the
    # interpolated view depends on id differences alone: any shift leaves it unchanged
    o3, _ = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=1e6, remap_scale=3, window_left=5,
                          remote_map="interp")
    o3s, _ = O.prefill_ref(q, k, v, pos + 1001, "bifocal", rope_base=1e6, remap_scale=3, window_left=5,
                           remote_map="interp")
    assert np.allclose(o3, o3s, atol=1e-10)
    oa, _ = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=1e6, remap_scale=3, window_left=5)
    assert not np.allclose(o3, oa, atol=1e-6)  # a different mapping indeed


@pytest.mark.parametrize("L,s,w0", [(40, 3, 7), (33, 4, -1)])
def test_interp_decode_equals_last_prefill_row(L, s, w0):
    B, Hq, Hkv, d, base = 1, 4, 2, 16, 1e6
    q, k, v = _rand_qkv(B, L, Hq, Hkv, d, 34)
    pos = np.tile(np.arange(L), (B, 1))
    o_pre, l_pre = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=base, remap_scale=s, window_left=w0,
                                 remote_map="interp")
    kc = O.rope_apply_ref(k, pos, base)
    ql = O.rope_apply_ref(q[:, -1:], pos[:, -1:], base)[:, 0]
    o_dec, l_dec = O.decode_ref(ql, kc, v, np.full(B, L), "bifocal", rope_base=base, remap_scale=s,
                                window_left=w0, remote_map="interp")
    assert np.allclose(o_dec, o_pre[:, -1], atol=1e-10)
    assert np.allclose(l_dec, l_pre[:, :, -1], atol=1e-10)


# ---------------------------------------------------------------- negative ids
# Ids may be any integer: a negative id rotates backwards, the period takes the
# mathematical remainder in [0, P) and the remote map the floor.

def test_periodic_and_remote_index_of_negative_ids():
    # P-RoPE Eq. (4) phi(t) = t mod W lies in [0, W); Jet-Long Eq. (3) is a floor
    assert list(O.periodic_index([-1, -8, -9, 7], 8)) == [7, 0, 7, 7]
    assert list(O.remote_index([-1, -2, -3, -4, -5, 5], 2)) == [-1, -1, -2, -2, -3, 2]


def test_negative_shift_invariance_rope_and_bifocal():
    # relative-offset property (P-RoPE Eq. (3)) for ids pushed below zero; for the
    # bifocal map only shifts by a multiple of s keep floor(p / s) differences,
    # which a truncating division of negative ids would break
    q, k, v = _rand_qkv(1, 33, 2, 1, 16, 41)
    pos = np.arange(33)[None]
    o1, _ = O.prefill_ref(q, k, v, pos, "rope", rope_base=1e4)
    o2, _ = O.prefill_ref(q, k, v, pos - 20, "rope", rope_base=1e4)
    assert np.allclose(o1, o2, atol=1e-9)
    p1, _ = O.prefill_ref(q, k, v, pos, "rope", rope_base=1e4, period=8, window_left=5)
    p2, _ = O.prefill_ref(q, k, v, pos - 8 * 9, "rope", rope_base=1e4, period=8, window_left=5)
    assert np.allclose(p1, p2, atol=1e-12)
    kw = dict(rope_base=1e6, remap_scale=3, window_left=5)
    b1, _ = O.prefill_ref(q, k, v, pos, "bifocal", **kw)
    b2, _ = O.prefill_ref(q, k, v, pos - 3 * 7, "bifocal", **kw)
    assert np.allclose(b1, b2, atol=1e-9)
    trunc = pos - 3 * 7
    # the same ids with a truncating division differ for the negative ones
    assert np.any(np.trunc(trunc / 3) != O.remote_index(trunc, 3))


def test_negative_ids_vectorized_equals_brute_force():
    B, S, Hq, Hkv, d = 1, 10, 2, 1, 6
    q, k, v = _rand_qkv(B, S, Hq, Hkv, d, 42)
    pos = np.array([[-7, -6, -5, -3, -1, 0, 2, 4, -100, 9]])
    for mode, kw in (("rope", dict(rope_base=1e4, period=4)), ("bifocal", dict(rope_base=1e4, remap_scale=3,
                                                                                   window_left=2))):
        o, _ = O.prefill_ref(q, k, v, pos, mode, **kw)
        bf = np.array(O.brute_force_prefill(q, k, v, pos, mode, kw["rope_base"], period=kw.get("period", 0),
                                            remap_scale=kw.get("remap_scale", 1),
                                            window_left=kw.get("window_left", -1)))
        assert np.allclose(o, bf, atol=1e-12), mode


# ---------------------------------------------------------------- ALiBi on a sliding window
# (P-RoPE page, section 1: SWA with ALiBi, the linear distance penalty clamped
# to the window of W keys, with a manually set slope per head)

def _alibi_mask(S, W, slopes):
    """Additive float mask [H, S, S]: - m_h (i - j) on the W kept keys, -inf elsewhere."""
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    dist = i - j
    kept = (dist >= 0) & ((dist <= W - 1) if W > 0 else True)
    bias = -np.asarray(slopes, dtype=np.float64)[:, None, None] * dist[None]
    return np.where(kept[None], bias, -np.inf)


@pytest.mark.parametrize("W", [6, 0])
def test_alibi_equals_sdpa_with_float_mask(W):
    # W = 0: no window (global ALiBi over the causal keys)
    B, S, Hq, Hkv, d = 1, 31, 4, 2, 8
    q, k, v = _rand_qkv(B, S, Hq, Hkv, d, 43)
    slopes = np.array([0.5, 0.25, 0.125, 0.0625])
    pos = np.arange(S)[None]
    o, _ = O.prefill_ref(q, k, v, pos, "nope", window_left=W - 1, alibi_slopes=slopes)
    want = _sdpa(q, k, v, mask=_alibi_mask(S, W, slopes)[None])
    assert np.allclose(o, want, atol=1e-12)
    # rope on the same window: SDPA on inputs rotated by complex multiplication
    base = 1e4
    th = np.array([base ** (-(2 * i) / d) for i in range(d // 2)])

    def crot(x):
        z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos[:, :, None, None] * th)
        y = np.empty_like(x)
        y[..., 0::2], y[..., 1::2] = z.real, z.imag
        return y

    o_r, _ = O.prefill_ref(q, k, v, pos, "rope", rope_base=base, window_left=W - 1, alibi_slopes=slopes)
    assert np.allclose(o_r, _sdpa(crot(q), crot(k), v, mask=_alibi_mask(S, W, slopes)[None]), atol=1e-12)


def test_alibi_geometric_closed_form():
    # q = 0: the logits of row i are - m * delta for delta = 0 .. n - 1 with
    # n = min(i + 1, W) kept keys, so the weights are a geometric sequence r^delta,
    # r = exp(-m): LSE = log((1 - r^n) / (1 - r)), and with v_j = (j, 1)
    # O_i = i - sum(delta r^delta) / sum(r^delta)
    #     = i - r (1 - n r^(n-1) + (n-1) r^n) / ((1 - r)(1 - r^n)).
    S, W, m = 40, 11, 0.3
    q = np.zeros((1, S, 1, 2))
    k = _rng(44).standard_normal((1, S, 1, 2))
    v = np.zeros((1, S, 1, 2))
    v[0, :, 0, 0] = np.arange(S)
    v[0, :, 0, 1] = 1.0
    o, lse = O.prefill_ref(q, k, v, np.arange(S)[None], "nope", window_left=W - 1, alibi_slopes=[m])
    r = math.exp(-m)
    for i in range(S):
        n = min(i + 1, W)
        assert abs(lse[0, 0, i] - math.log((1 - r ** n) / (1 - r))) < 1e-12
        mean_delta = r * (1 - n * r ** (n - 1) + (n - 1) * r ** n) / ((1 - r) * (1 - r ** n))
        assert abs(o[0, i, 0, 0] - (i - mean_delta)) < 1e-11
        assert abs(o[0, i, 0, 1] - 1.0) < 1e-13


def test_alibi_zero_and_large_slopes():
    q, k, v = _rand_qkv(1, 25, 2, 1, 8, 45)
    pos = np.arange(25)[None]
    plain, lp = O.prefill_ref(q, k, v, pos, "rope", rope_base=1e4, window_left=7)
    zero, lz = O.prefill_ref(q, k, v, pos, "rope", rope_base=1e4, window_left=7, alibi_slopes=[0.0, 0.0])
    assert np.array_equal(plain, zero) and np.array_equal(lp, lz)
    # a steep slope leaves only the key at distance 0: O_i = v_i
    big, _ = O.prefill_ref(q, k, v, pos, "rope", rope_base=1e4, window_left=7, alibi_slopes=[80.0, 80.0])
    assert np.allclose(big[0, :, 0], v[0, :, 0], atol=1e-12)
    assert np.allclose(big[0, :, 1], v[0, :, 0], atol=1e-12)


@pytest.mark.parametrize("mode,kw", [
    ("nope", dict(window_left=3)),
    ("rope", dict(rope_base=1e4, period=5, window_left=4)),
    ("rope", dict(rope_base=1e4)),
])
def test_alibi_vectorized_equals_brute_force(mode, kw):
    B, S, Hq, Hkv, d = 2, 12, 4, 2, 6
    q, k, v = _rand_qkv(B, S, Hq, Hkv, d, 46)
    slopes = np.array([0.7, 0.2, 1.3, 0.05])
    pos = np.stack([np.arange(S), np.concatenate([np.arange(6), np.arange(100, 106)])])
    o, _ = O.prefill_ref(q, k, v, pos, mode, alibi_slopes=slopes, **kw)
    bf = np.array(O.brute_force_prefill(q, k, v, pos, mode, kw.get("rope_base", 1e4), period=kw.get("period", 0),
                                        window_left=kw.get("window_left", -1), alibi_slopes=slopes))
    assert np.allclose(o, bf, atol=1e-12)


@pytest.mark.parametrize("mode,w", [("rope", 9), ("nope", -1)])
def test_alibi_decode_equals_last_prefill_row(mode, w):
    B, L, Hq, Hkv, d = 1, 30, 4, 2, 8
    q, k, v = _rand_qkv(B, L, Hq, Hkv, d, 47)
    slopes = np.array([0.4, 0.1, 0.9, 0.02])
    pos = np.arange(L)[None]
    kw = dict(rope_base=1e4) if mode == "rope" else {}
    o_pre, l_pre = O.prefill_ref(q, k, v, pos, mode, window_left=w, alibi_slopes=slopes, **kw)
    kc = O.rope_apply_ref(k, pos, 1e4) if mode == "rope" else k
    ql = O.rope_apply_ref(q[:, -1:], pos[:, -1:], 1e4)[:, 0] if mode == "rope" else q[:, -1]
    o_dec, l_dec = O.decode_ref(ql, kc, v, [L], mode, window_left=w, alibi_slopes=slopes)
    assert np.allclose(o_dec, o_pre[:, -1], atol=1e-12)
    assert np.allclose(l_dec, l_pre[:, :, -1], atol=1e-12)


def test_alibi_rejected_for_bifocal():
    q, k, v = _rand_qkv(1, 5, 1, 1, 4, 48)
    with pytest.raises(ValueError):
        O.prefill_ref(q, k, v, np.arange(5)[None], "bifocal", remap_scale=2, window_left=1, alibi_slopes=[0.1])


# ---------------------------------------------------------------- real-valued interpolation scale
# (Jet-Long page, section 3.1: s = max(1, L / w_pretrained) for continuous-style
# rescaling; section 4.5: frequency interpolation as the remote map)

def test_continuous_scale_values():
    assert O.continuous_scale(10, 32) == 1.0
    assert O.continuous_scale(32, 32) == 1.0
    assert O.continuous_scale(48, 32) == 1.5
    assert O.continuous_scale(131072, 32768) == 4.0
    assert O.continuous_scale(100000, 32768) == 100000 / 32768
    # the integer group size of Eq. (2) is its ceiling
    for L in (1, 31, 32, 33, 100000):
        assert O.group_size(L, 32) == math.ceil(O.continuous_scale(L, 32))


@pytest.mark.parametrize("s", [1.5, 2.5, 131072 / 40000])
def test_interp_real_scale_equals_sdpa_on_complex_rotation(s):
    B, S, Hq, Hkv, d, base = 1, 27, 4, 2, 8, 1e6
    q, k, v = _rand_qkv(B, S, Hq, Hkv, d, 49)
    pos = np.arange(S)[None] * 5 + 3
    th = np.array([base ** (-(2 * i) / d) for i in range(d // 2)]) / s

    def crot(x):
        z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos[:, :, None, None] * th)
        y = np.empty_like(x)
        y[..., 0::2], y[..., 1::2] = z.real, z.imag
        return y

    o, _ = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=base, remap_scale=s, window_left=-1,
                         remote_map="interp")
    assert np.allclose(o, _sdpa(crot(q), crot(k), v, causal=True), atol=1e-12)


def test_interp_real_scale_brute_force_and_eq7():
    B, S, Hq, Hkv, d = 1, 11, 2, 1, 6
    q, k, v = _rand_qkv(B, S, Hq, Hkv, d, 50)
    pos = np.arange(S)[None] + 3
    o, _ = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=1e4, remap_scale=1.75, window_left=2,
                         remote_map="interp")
    bf = np.array(O.brute_force_prefill(q, k, v, pos, "bifocal", 1e4, remap_scale=1.75, window_left=2,
                                        remote_map="interp"))
    assert np.allclose(o, bf, atol=1e-12)
    q2, k2, v2 = _rand_qkv(1, 48, 4, 2, 8, 51)
    pos2 = np.arange(48)[None]
    for w0, s in [(5, 1.5), (0, 2.25), (-1, 3.1), (47, 1.2)]:
        direct, _ = O.prefill_ref(q2, k2, v2, pos2, "bifocal", rope_base=1e6, remap_scale=s, window_left=w0,
                                  remote_map="interp")
        eq7 = O.bifocal_eq7_ref(q2, k2, v2, pos2, rope_base=1e6, remap_scale=s, window_left=w0,
                                remote_map="interp")
        assert np.allclose(eq7, direct, atol=1e-10), (w0, s)


@pytest.mark.parametrize("L,w_pre,w0", [(40, 16, 7), (33, 30, -1), (50, 64, 4)])
def test_interp_continuous_decode_equals_last_prefill_row(L, w_pre, w0):
    # the dynamic factor at the sequence's own length, s = max(1, L / w_pre)
    s = O.continuous_scale(L, w_pre)
    B, Hq, Hkv, d, base = 1, 4, 2, 16, 1e6
    q, k, v = _rand_qkv(B, L, Hq, Hkv, d, 52)
    pos = np.tile(np.arange(L), (B, 1))
    o_pre, l_pre = O.prefill_ref(q, k, v, pos, "bifocal", rope_base=base, remap_scale=s, window_left=w0,
                                 remote_map="interp")
    kc = O.rope_apply_ref(k, pos, base)
    ql = O.rope_apply_ref(q[:, -1:], pos[:, -1:], base)[:, 0]
    o_dec, l_dec = O.decode_ref(ql, kc, v, np.full(B, L), "bifocal", rope_base=base, remap_scale=s,
                                window_left=w0, remote_map="interp")
    assert np.allclose(o_dec, o_pre[:, -1], atol=1e-10)
    assert np.allclose(l_dec, l_pre[:, :, -1], atol=1e-10)


def test_alias_rejects_real_scale():
    q, k, v = _rand_qkv(1, 5, 1, 1, 4, 53)
    with pytest.raises(ValueError):
        O.prefill_ref(q, k, v, np.arange(5)[None], "bifocal", remap_scale=1.5, window_left=1)

"""Plain float64 CPU oracle for causal attention under remapped RoPE positions.

TEST INFRASTRUCTURE ONLY. Nothing in the library may import or call this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg
do. It is deliberately slow and literal: explicit per-pair rotations from the
definitions, a full masked softmax, NumPy float64 throughout. It shares no code,
constant or table with the HIP library.

Sources (page titles; sections and equations named where each step is used):

* "Periodic RoPE for Infinite Context LLMs" (P-RoPE), section 3.1, Eq. (1)-(3):
  RoPE frequencies and the 2x2 block rotation; section 3.2, Eq. (4)-(5): the
  periodic index t mod W with causal sliding-window attention; section 3.3,
  Eq. (6): NoPE global attention scaled by 1/sqrt(d_h).
* "Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal RoPE",
  section 3, Eq. (1): the bifocal score; section 3.1, Eq. (2)-(3): group size
  and the floor-division remote map; section 3.2, Eq. (4)-(6): a cache of
  base-rotated keys and the correction rotation; section 3.3, Eq. (7): the
  inclusion-exclusion merge of three attention calls.
* EndPrompt (abstract): a two-segment sequence whose second segment carries
  ids near the target length; attention over it is ordinary causal RoPE
  attention on those ids.
* "Periodic RoPE for Infinite Context LLMs", section 1: the earlier layer
  design of sliding-window attention with ALiBi, its linear distance penalty
  clamped to the window, with a manually set slope.

Readings taken where the pages leave a step open:

* RoPE pairs adjacent coordinates (2i, 2i+1) with frequency theta_i, which is
  what the block-diagonal matrix of Eq. (2) (P-RoPE page) prints.
* Scores are scaled by 1/sqrt(d) in every mode (Eq. (6), P-RoPE page) unless a
  scale is given.
* Masks and bifocal routing use token indices (i for the query, j for the
  key); position ids drive the rotation only.
* ``window_left`` is the largest kept distance i - j. For the P-RoPE window of
  W keys it is W - 1; for Jet-Long it is w0 (local iff i - j <= w0).
* ``remap_scale`` is the integer group size G of Jet-Long Eq. (2)-(3) for the
  aliasing map. For the interpolation map it may be any real s >= 1; the
  continuous dynamic factor of Jet-Long section 3.1 is s = max(1, L / w_pre)
  (``continuous_scale``).
* ALiBi (``alibi_slopes``, one slope m_h per query head, nope/rope modes): the
  scaled score of a kept key gets - m_h * (i - j) added; keys beyond the window
  are masked, so the penalty only acts on distances 0 .. window_left.
* ``operand_round``: the rotated query and key that enter the score product are
  rounded once to the given type ("bf16" or "fp32"), the rest stays float64.
  This models a model that stores RoPE'd vectors in its own dtype (the Jet-Long
  cache of Eq. (4) is such a tensor). ``None`` keeps everything in float64.

Parity pinning: every function here is pinned by tests against closed forms,
invariants the pages state, textbook library routines or brute force (see
tests/test_oracle.py); none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

MODES = ("nope", "rope", "bifocal")


# --------------------------------------------------------------------------
# RoPE (P-RoPE page, section 3.1)
# --------------------------------------------------------------------------

def rope_theta(d: int, base: float) -> np.ndarray:
    """theta_i = base ** (-2i/d), i = 0 .. d/2-1  (P-RoPE page, Eq. (1))."""
    if d % 2:
        raise ValueError("head dimension must be even")
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / d)


def rotate(x: np.ndarray, r, base: float) -> np.ndarray:
    """Apply R_r to the last axis of ``x`` (P-RoPE page, Eq. (2)).

    Each adjacent pair (x_{2i}, x_{2i+1}) is multiplied by the 2x2 block
    [[cos r*theta_i, -sin r*theta_i], [sin r*theta_i, cos r*theta_i]].
    ``r`` broadcasts against ``x[..., 0]`` (one rotation index per vector).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    th = rope_theta(d, base)
    r = np.asarray(r, dtype=np.float64)[..., None]        # exact for |r| < 2**53
    ang = r * th                                           # (..., d/2)
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    y = np.empty(np.broadcast_shapes(x.shape, c.shape[:-1] + (d,)), dtype=np.float64)
    y[..., 0::2] = c * xe - s * xo
    y[..., 1::2] = s * xe + c * xo
    return y


def periodic_index(t, period: int):
    """phi(t) = t mod P (P-RoPE page, Eq. (4)); P = 0 means no period."""
    t = np.asarray(t, dtype=np.int64)
    return t if period == 0 else np.mod(t, period)


def group_size(L: int, w_pretrained: int) -> int:
    """G = max(1, ceil(L / w_pretrained)) (Jet-Long page, section 3.1, Eq. (2))."""
    return max(1, -(-int(L) // int(w_pretrained)))


def continuous_scale(L: int, w_pretrained: int) -> float:
    """s = max(1, L / w_pretrained), the continuous-style dynamic factor (Jet-Long
    page, section 3.1, stated beside Eq. (2) for frequency-rescaling methods)."""
    return max(1.0, float(L) / float(w_pretrained))


def remote_index(p, G: int):
    """f(x) = floor(x / G) (Jet-Long page, section 3.1, Eq. (3))."""
    return np.floor_divide(np.asarray(p, dtype=np.int64), int(G))


def remote_position(p, G: int, remote_map: str = "alias"):
    """The remote view's rotation position of position p.

    "alias": floor(p / G), the default mapping (Jet-Long page, Eq. (3));
    "interp": p / G unfloored, i.e. every frequency theta_i divided by G at the
    original positions: the frequency-interpolation mapping the same page
    compares against aliasing in section 4.5 (Table 6), taken in its plainest
    (uniform, linear) form. G may be any real number >= 1 here.
    """
    if remote_map == "alias":
        return remote_index(p, G)
    if remote_map == "interp":
        return np.asarray(p, dtype=np.float64) / float(G)
    raise ValueError(remote_map)


def rope_apply_ref(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """y = R_pos x per token: x [B,S,H,d], pos int [B,S] (negative ids allowed)."""
    return rotate(x, np.asarray(pos, dtype=np.int64)[:, :, None], base)


# --------------------------------------------------------------------------
# Rounding of rotated operands (a reading, see module docstring)
# --------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits), ties to even.

    Written from the format's definition: with x = m * 2**e, 0.5 <= |m| < 1,
    keep m rounded to a multiple of 2**-8. Valid for the normal range, which
    is all the workloads reach.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def round_operand(x: np.ndarray, kind: Optional[str]) -> np.ndarray:
    if kind is None:
        return np.asarray(x, dtype=np.float64)
    if kind == "bf16":
        return round_to_bf16(x)
    if kind == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(kind)


# --------------------------------------------------------------------------
# Masked softmax attention for a block of query rows
# --------------------------------------------------------------------------

def _softmax_rows(scores: np.ndarray, keep: np.ndarray, vals: np.ndarray):
    """Full masked softmax over the last axis, then P @ V.

    scores, keep: [R, S]; vals: [S, d]. Returns (O [R, d], lse [R]).
    Rows with no kept key give O = 0 and lse = -inf.
    """
    s = np.where(keep, scores, -np.inf)
    if s.shape[-1] == 0:  # no key at all (an empty sequence)
        return np.zeros((s.shape[0], vals.shape[-1])), np.full(s.shape[0], -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    p = np.where(keep, np.exp(s - m), 0.0)
    l = np.sum(p, axis=-1, keepdims=True)
    safe_l = np.where(l > 0, l, 1.0)
    o = (p @ vals) / safe_l
    lse = np.where(l[:, 0] > 0, m[:, 0] + np.log(safe_l[:, 0]), -np.inf)
    return o, lse


def _check_mode(mode, period, remap_scale, window_left, remote_map="alias", alibi_slopes=None):
    if mode not in MODES:
        raise ValueError(f"mode must be one of {MODES}")
    if period < 0 or remap_scale < 1 or window_left < -1:
        raise ValueError("bad period / remap_scale / window_left")
    if remote_map not in ("alias", "interp") or (remote_map == "interp" and mode != "bifocal"):
        raise ValueError("bad remote_map")
    if remote_map == "alias" and int(remap_scale) != remap_scale:
        raise ValueError("the aliasing map takes an integer group size")
    if alibi_slopes is not None and mode == "bifocal":
        raise ValueError("ALiBi biases apply to the nope/rope modes")


def prefill_ref(q, k, v, pos, mode: str, rope_base: float = 1e4, period: int = 0,
                remap_scale: int = 1, window_left: int = -1,
                softmax_scale: Optional[float] = None, operand_round: Optional[str] = None,
                rows: Optional[np.ndarray] = None, max_block_elems: int = 1 << 24,
                remote_map: str = "alias",
                alibi_slopes: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Causal attention with RoPE under remapped ids, computed directly.

    q [B,S,Hq,d], k/v [B,S,Hkv,d] (unrotated), pos int [B,S]. The KV head of
    query head h is h // (Hq // Hkv). Returns O [B,R,Hq,d] and LSE [B,Hq,R]
    for the query rows ``rows`` (default all S rows, R = S).

    Per mode, for query index i and key index j <= i:
      nope:    s_ij = q_i . k_j                          (P-RoPE page, Eq. (6))
      rope:    s_ij = (R_{r_i} q_i) . (R_{r_j} k_j), r = pos mod P if P > 0
                                                         (P-RoPE page, Eq. (3)-(5))
      bifocal: i - j <= w0: (R_{p_i} q_i) . (R_{p_j} k_j)
               i - j >  w0: (R_{f(p_i)} q_i) . (R_{f(p_j)} k_j), f(x) = floor(x/s)
                                                         (Jet-Long page, Eq. (1), (3)),
                            or f(x) = x / s with remote_map="interp" (section 4.5)
    then scaled by softmax_scale (default 1/sqrt(d)). In nope/rope modes a
    window_left >= 0 also drops keys with i - j > window_left, and
    ``alibi_slopes`` (length Hq) adds - m_h * (i - j) to the scaled score of
    each kept key: the sliding-window ALiBi layer of the P-RoPE page, section 1,
    whose penalty the window clamps to distances 0 .. window_left.
    """
    _check_mode(mode, period, remap_scale, window_left, remote_map, alibi_slopes)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    grp = Hq // Hkv
    scale = (1.0 / math.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    slopes = None if alibi_slopes is None else np.asarray(alibi_slopes, dtype=np.float64).reshape(Hq)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    o_out = np.zeros((B, R, Hq, d))
    lse_out = np.full((B, Hq, R), -np.inf)
    j_all = np.arange(S)

    for b in range(B):
        p = pos[b]
        # rotation indices for queries and keys
        if mode == "nope":
            kb = round_operand(k[b], operand_round)                      # [S,Hkv,d]
            qb = round_operand(q[b][rows], operand_round)                # [R,Hq,d]
        elif mode == "rope":
            r = periodic_index(p, period)
            kb = round_operand(rotate(k[b], r[:, None], rope_base), operand_round)
            qb = round_operand(rotate(q[b][rows], r[rows][:, None], rope_base), operand_round)
        else:  # bifocal: base rotation at p, remote rotation at f(p)
            rr = remote_position(p, remap_scale, remote_map)
            kb = round_operand(rotate(k[b], p[:, None], rope_base), operand_round)
            qb = round_operand(rotate(q[b][rows], p[rows][:, None], rope_base), operand_round)
            kr = round_operand(rotate(k[b], rr[:, None], rope_base), operand_round)
            qr = round_operand(rotate(q[b][rows], rr[rows][:, None], rope_base), operand_round)

        chunk = max(1, max_block_elems // S)
        for c0 in range(0, R, chunk):
            sel = slice(c0, min(R, c0 + chunk))
            ri = rows[sel]
            jmax = int(ri.max()) + 1                    # keys beyond the last row are never kept
            jj = j_all[:jmax]
            dist = ri[:, None] - jj[None, :]            # i - j
            keep = dist >= 0
            if mode != "bifocal" and window_left >= 0:
                keep &= dist <= window_left
            for h in range(Hq):
                g = h // grp
                sc = qb[sel, h, :] @ kb[:jmax, g, :].T
                if mode == "bifocal":
                    sc_remote = qr[sel, h, :] @ kr[:jmax, g, :].T
                    sc = np.where(dist <= window_left, sc, sc_remote)
                logits = sc * scale
                if slopes is not None:
                    logits = logits - slopes[h] * dist
                o, lse = _softmax_rows(logits, keep, v[b, :jmax, g, :])
                o_out[b, sel, h, :] = o
                lse_out[b, h, sel] = lse
    return o_out, lse_out


def decode_ref(q, k_cache, v_cache, kv_len, mode: str = "bifocal", rope_base: float = 1e6,
               remap_scale: int = 1, window_left: int = -1,
               softmax_scale: Optional[float] = None, operand_round: Optional[str] = None,
               remote_map: str = "alias",
               alibi_slopes: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One decode step against a cache of base-rotated keys.

    q [B,Hq,d] is the query already rotated at its own position p_q = kv_len-1;
    k_cache/v_cache [B,L,Hkv,d] hold keys rotated at their index j (Jet-Long
    page, section 3.2, Eq. (4)). Returns O [B,Hq,d] and LSE [B,Hq].

    bifocal: local keys (p_q - j <= w0) score q . k_j; remote keys score
    RoPE(q, dq) . RoPE(k_j, dk_j) with dq = floor(p_q/s) - p_q and
    dk_j = floor(j/s) - j (Jet-Long page, Eq. (5)-(6)); with remote_map="interp"
    the remote positions are p_q / s and j / s, so dq = p_q/s - p_q and
    dk_j = j/s - j.
    nope/rope: the cache and q already carry whatever rotation the layer uses,
    so scores are q . k_j, with keys p_q - j > window_left dropped if
    window_left >= 0 and, with ``alibi_slopes``, - m_h * (p_q - j) added to
    each scaled score (as in prefill_ref).
    A real remap_scale s with remote_map="interp" gives dq = p_q/s - p_q.
    """
    _check_mode(mode, 0, remap_scale, window_left, remote_map, alibi_slopes)
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    B, Hq, d = q.shape
    Hkv = kc.shape[2]
    grp = Hq // Hkv
    scale = (1.0 / math.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    slopes = None if alibi_slopes is None else np.asarray(alibi_slopes, dtype=np.float64).reshape(Hq)
    o_out = np.zeros((B, Hq, d))
    lse_out = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(kv_len[b])
        pq = L - 1
        j = np.arange(L)
        dist = pq - j
        keep = np.ones(L, dtype=bool)
        if mode != "bifocal" and window_left >= 0:
            keep = dist <= window_left
        if mode == "bifocal":
            dq = remote_position(pq, remap_scale, remote_map) - pq       # Eq. (5)
            dk = remote_position(j, remap_scale, remote_map) - j
            k_rem = round_operand(rotate(kc[b, :L], dk[:, None], rope_base), operand_round)
            q_rem = round_operand(rotate(q[b], dq, rope_base), operand_round)
        for h in range(Hq):
            g = h // grp
            sc = kc[b, :L, g, :] @ q[b, h]
            if mode == "bifocal":
                sc = np.where(dist <= window_left, sc, k_rem[:, g, :] @ q_rem[h])
            logits = sc * scale
            if slopes is not None:
                logits = logits - slopes[h] * dist
            o, lse = _softmax_rows(logits[None, :], keep[None, :], vc[b, :L, g, :])
            o_out[b, h] = o[0]
            lse_out[b, h] = lse[0]
    return o_out, lse_out


# --------------------------------------------------------------------------
# Independent formulations used as self-checks
# --------------------------------------------------------------------------

def _window_call(qrot, krot, v, lo_dist, hi_dist, scale):
    """Attention of one head restricted to keys with lo_dist <= i - j <= hi_dist.

    qrot [S,d], krot [S,d], v [S,d]. Returns (O [S,d], lse [S]).
    """
    S = qrot.shape[0]
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    dist = i - j
    keep = (dist >= lo_dist) & (dist <= hi_dist)
    return _softmax_rows((qrot @ krot.T) * scale, keep, v)


def bifocal_eq7_ref(q, k, v, pos, rope_base: float, remap_scale: int, window_left: int,
                    softmax_scale: Optional[float] = None, remote_map: str = "alias"):
    """Bifocal attention by the three-call inclusion-exclusion merge.

    (A) window w0 with base q/k, (B) full causal with remote q/k, (C) window w0
    with remote q/k; M = max(lse_A, lse_B, lse_C), W_X = exp(lse_X - M),
    O = (W_A O_A + W_B O_B - W_C O_C) / (W_A + W_B - W_C)
    (Jet-Long page, section 3.3, Eq. (7)). Float64, no operand rounding. The
    remote q/k are rotated at remote_position(p, s, remote_map).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    B, S, Hq, d = q.shape
    grp = Hq // k.shape[2]
    scale = (1.0 / math.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    w0 = window_left
    out = np.zeros_like(q)
    for b in range(B):
        p = pos[b]
        rr = remote_position(p, remap_scale, remote_map)
        for h in range(Hq):
            g = h // grp
            qb = rotate(q[b, :, h], p, rope_base)
            kb = rotate(k[b, :, g], p, rope_base)
            qr = rotate(q[b, :, h], rr, rope_base)
            kr = rotate(k[b, :, g], rr, rope_base)
            oa, la = _window_call(qb, kb, v[b, :, g], 0, w0, scale)
            ob, lb = _window_call(qr, kr, v[b, :, g], 0, S, scale)
            oc, lc = _window_call(qr, kr, v[b, :, g], 0, w0, scale)
            M = np.maximum(np.maximum(la, lb), lc)
            wa, wb, wc = (np.exp(l - M) for l in (la, lb, lc))
            num = wa[:, None] * oa + wb[:, None] * ob - wc[:, None] * oc
            den = wa + wb - wc
            out[b, :, h] = num / den[:, None]
    return out


def brute_force_prefill(q, k, v, pos, mode: str, rope_base: float, period: int = 0,
                        remap_scale: int = 1, window_left: int = -1,
                        softmax_scale: Optional[float] = None, remote_map: str = "alias",
                        alibi_slopes=None):
    """Pure-Python loops over (b, h, i, j, pair) with explicit 2x2 rotation blocks.

    For tiny inputs only. Returns O as nested float lists shaped [B][S][Hq][d].
    ``alibi_slopes`` adds - m_h * (i - j) to each kept score (nope/rope).
    """
    q = np.asarray(q, dtype=np.float64).tolist()
    k = np.asarray(k, dtype=np.float64).tolist()
    v = np.asarray(v, dtype=np.float64).tolist()
    pos = np.asarray(pos, dtype=np.int64).tolist()
    B, S, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0][0])
    grp = Hq // Hkv
    scale = (1.0 / math.sqrt(d)) if softmax_scale is None else softmax_scale

    def block_rotate(vec, r):
        out = []
        for i in range(d // 2):
            th = rope_base ** (-2.0 * i / d)
            a = r * th
            m = [[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]]
            x0, x1 = vec[2 * i], vec[2 * i + 1]
            out += [m[0][0] * x0 + m[0][1] * x1, m[1][0] * x0 + m[1][1] * x1]
        return out

    def dot(a, b_):
        return sum(x * y for x, y in zip(a, b_))

    O = [[[[0.0] * d for _ in range(Hq)] for _ in range(S)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            for i in range(S):
                scores, idx = [], []
                for j in range(i + 1):
                    dist = i - j
                    if mode == "nope":
                        if window_left >= 0 and dist > window_left:
                            continue
                        s_ij = dot(q[b][i][h], k[b][j][g])
                    elif mode == "rope":
                        if window_left >= 0 and dist > window_left:
                            continue
                        ri = pos[b][i] % period if period else pos[b][i]
                        rj = pos[b][j] % period if period else pos[b][j]
                        s_ij = dot(block_rotate(q[b][i][h], ri), block_rotate(k[b][j][g], rj))
                    else:
                        if dist <= window_left:
                            ri, rj = pos[b][i], pos[b][j]
                        elif remote_map == "alias":
                            ri, rj = pos[b][i] // remap_scale, pos[b][j] // remap_scale
                        else:
                            ri, rj = pos[b][i] / remap_scale, pos[b][j] / remap_scale
                        s_ij = dot(block_rotate(q[b][i][h], ri), block_rotate(k[b][j][g], rj))
                    bias = 0.0 if alibi_slopes is None else -float(alibi_slopes[h]) * dist
                    scores.append(s_ij * scale + bias)
                    idx.append(j)
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = sum(w)
                for c in range(d):
                    O[b][i][h][c] = sum(wj * v[b][j][g][c] for wj, j in zip(w, idx)) / tot
    return O

"""GPU parity for the layer variants beyond the base workloads, through the C ABI
against the fp64 oracle on the same seeded inputs:

* position ids of any sign (floor semantics of the period and the remote map);
* sliding-window ALiBi biases on the nope/rope layers (P-RoPE page, section 1);
* the frequency-interpolation remote map with a real scale s, fixed or the
  continuous factor max(1, L / w_pretrained) of Jet-Long section 3.1, in the
  fused prefill, the unfused Eq. (7) composition and decode;
* prefill graphs captured on one stream and replayed in either order.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
import position_remapped_rope_amd as P
import workloads as W
from parity import LSE_TOL, assert_close, log, oracle_decode, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs(B, S, Hq, Hkv, d, dtype, seed, ids=None):
    w = W.Workload("t", "prefill", B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, mode="rope", rope_base=1e4, seed=seed)
    inp = W.make_prefill_inputs(w)
    if ids is not None:
        inp["pos"] = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(ids, (B, S)).astype(np.int32)))
    return inp


def _np(inp):
    return to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), inp["pos"].numpy()


def _compare(o, lse, o_ref, lse_ref, dtype, what):
    assert_close(to_np(o), o_ref, dtype, what)
    lerr = float(np.max(np.abs(lse.cpu().numpy() - lse_ref)))
    log(f"{what}: lse max_abs={lerr:.3e}")
    assert lerr <= LSE_TOL[dtype], what


def _slopes(Hq, seed):
    # a spread of slopes around the geometric ALiBi family, one per query head
    rng = np.random.default_rng(seed)
    return (2.0 ** (-8.0 * (np.arange(Hq) + 1) / Hq) * rng.uniform(0.5, 2.0, Hq)).astype(np.float32)


# ------------------------------------------------------------------ negative ids

NEG = [
    # name, (B, S, Hq, Hkv, d, dtype), mode, kwargs, first id
    ("rope_period_crossing_zero", (1, 500, 4, 2, 128, "bf16"), "rope", dict(rope_base=1e4, period=96, window_left=80), -250),
    ("rope_below_zero_d64", (2, 300, 8, 2, 64, "bf16"), "rope", dict(rope_base=1e6), -1000),
    ("rope_min_int", (1, 200, 4, 4, 128, "bf16"), "rope", dict(rope_base=1e4, period=1000), -(1 << 31)),
    ("bifocal_alias_crossing_zero", (1, 700, 8, 2, 128, "bf16"), "bifocal",
     dict(rope_base=1e6, remap_scale=3, window_left=100), -333),
    ("bifocal_alias_far_below_zero", (1, 400, 4, 1, 128, "bf16"), "bifocal",
     dict(rope_base=1e6, remap_scale=4, window_left=64), -(1 << 30)),
    ("bifocal_interp_crossing_zero", (1, 500, 4, 2, 64, "bf16"), "bifocal",
     dict(rope_base=1e6, remap_scale=2, window_left=50, remote_map="interp"), -260),
    ("fp32_rope_period", (1, 120, 4, 2, 64, "fp32"), "rope", dict(rope_base=1e4, period=16, window_left=30), -70),
    ("fp32_bifocal", (1, 150, 4, 2, 128, "fp32"), "bifocal", dict(rope_base=1e6, remap_scale=3, window_left=20), -77),
    # ids that run past INT32_MAX and wrap to INT32_MIN mid-sequence: two K rows a
    # thread stages 16 keys apart can then have ids 16 apart modulo 2^32 only,
    # which must not be taken for an affine step
    ("rope_ids_wrap_int32", (1, 300, 4, 2, 128, "bf16"), "rope", dict(rope_base=1e4), (1 << 31) - 150),
    ("bifocal_ids_wrap_int32", (1, 400, 4, 2, 128, "bf16"), "bifocal",
     dict(rope_base=1e6, remap_scale=2, window_left=64), (1 << 31) - 200),
    ("bifocal_interp_ids_wrap_int32", (1, 300, 4, 2, 64, "bf16"), "bifocal",
     dict(rope_base=1e6, remap_scale=2, window_left=40, remote_map="interp"), (1 << 31) - 120),
    ("fp32_rope_ids_wrap_int32", (1, 100, 4, 2, 64, "fp32"), "rope", dict(rope_base=1e4), (1 << 31) - 50),
    # periods at or below the 16-key step between a thread's two staged K rows:
    # the second row's index never follows from the first's, so every tile takes
    # the exact path for it
    ("rope_period_below_row_step", (1, 300, 4, 2, 128, "bf16"), "rope", dict(rope_base=1e4, period=10, window_left=150),
     -37),
    ("rope_period_equal_row_step", (1, 300, 4, 2, 128, "bf16"), "rope", dict(rope_base=1e4, period=16), 5),
]


@pytest.mark.parametrize("name,shape,mode,kw,first", NEG, ids=[c[0] for c in NEG])
def test_prefill_negative_ids(name, shape, mode, kw, first):
    B, S, Hq, Hkv, d, dtype = shape
    ids = (np.arange(S, dtype=np.int64) + first).astype(np.int32)
    inp = _inputs(B, S, Hq, Hkv, d, dtype, seed=zlib.crc32(name.encode()) % 1000, ids=ids)
    q, k, v, pos = (inp[n].to(DEV) for n in ("q", "k", "v", "pos"))
    o, lse = P.prefill(q, k, v, pos, mode=mode, return_lse=True, **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = O.prefill_ref(*_np(inp), mode, operand_round=dtype, **kw)
    _compare(o, lse, o_ref, lse_ref, dtype, name)


def test_unfused_negative_ids():
    S = 600
    ids = (np.arange(S) - 300).astype(np.int32)
    inp = _inputs(1, S, 8, 2, 128, "bf16", seed=501, ids=ids)
    kw = dict(rope_base=1e6, remap_scale=3, window_left=90)
    q, k, v, pos = (inp[n].to(DEV) for n in ("q", "k", "v", "pos"))
    o, lse = P.prefill_bifocal_unfused(q, k, v, pos, return_lse=True, **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = O.prefill_ref(*_np(inp), "bifocal", operand_round="bf16", **kw)
    _compare(o, lse, o_ref, lse_ref, "bf16", "unfused negative ids")


# ------------------------------------------------------------------ scores that rise tile by tile

# Log2-unit scores of the keys of each 64-key tile (plus a little jitter): a
# tile 7.5 or 7.9 above the reference leaves it in place although the tile's P
# sum is far above 2^8; tiles 20 and 40 higher raise it; a low tile at the end.
RISING_LOG2 = [0.0, 7.5, 7.9, 20.0, 27.5, 40.0, 40.5, 3.0]


def _rising_inputs(S=512, Hq=4, Hkv=2, d=128, seed=77):
    """q and k whose scores follow RISING_LOG2 by key tile for every query row.
    The signal sits in the last rotary pair, whose angle stays below 1e-3 rad
    at these ids and base 1e6, so RoPE leaves the scores almost unchanged; the
    other dims hold small noise. The oracle takes the same bf16 inputs."""
    rng = np.random.default_rng(seed)
    a = 16.0
    q = rng.normal(0.0, 0.05, (1, S, Hq, d)).astype(np.float32)
    k = rng.normal(0.0, 0.05, (1, S, Hkv, d)).astype(np.float32)
    v = rng.normal(0.0, 1.0, (1, S, Hkv, d)).astype(np.float32)
    q[..., d - 2] = a
    q[..., d - 1] = 0.0
    log2s = np.asarray(RISING_LOG2)[np.arange(S) // 64] + rng.uniform(-0.3, 0.3, S)
    k[0, :, :, d - 2] = (log2s / np.log2(np.e) * np.sqrt(d) / a)[:, None]
    k[..., d - 1] = 0.0
    pos = np.arange(S, dtype=np.int32)[None, :]
    return {"q": W.to_dtype_tensor(q, "bf16"), "k": W.to_dtype_tensor(k, "bf16"),
            "v": W.to_dtype_tensor(v, "bf16"), "pos": torch.from_numpy(np.ascontiguousarray(pos))}


@pytest.mark.parametrize("mode,kw", [
    ("bifocal", dict(rope_base=1e6, remap_scale=2, window_left=64)),
    ("bifocal", dict(rope_base=1e6, remap_scale=2, window_left=-1)),
    ("rope", dict(rope_base=1e6)),
    ("nope", dict()),
], ids=["bifocal", "bifocal_remote_only", "rope", "nope"])
def test_prefill_rising_scores(mode, kw):
    """The reference max's rare branches (a large P sum with no raise, and a
    raise) against the oracle, in the bifocal kernel (P before the max) and in
    the max-first kernels."""
    inp = _rising_inputs()
    q, k, v, pos = (inp[n].to(DEV) for n in ("q", "k", "v", "pos"))
    o, lse = P.prefill(q, k, v, pos if mode != "nope" else None, mode=mode, return_lse=True, **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = O.prefill_ref(*_np(inp), mode, operand_round="bf16", **kw)
    _compare(o, lse, o_ref, lse_ref, "bf16", f"rising scores {mode} {kw}")


# ------------------------------------------------------------------ ALiBi on a sliding window

ALIBI = [
    # name, (B, S, Hq, Hkv, d, dtype), mode, kwargs
    ("nope_swa_gqa4", (1, 900, 8, 2, 128, "bf16"), "nope", dict(window_left=200)),
    ("nope_global_ragged", (2, 333, 4, 4, 128, "bf16"), "nope", dict(window_left=-1)),
    ("rope_period_swa", (1, 1500, 16, 16, 128, "bf16"), "rope", dict(rope_base=1e4, period=512, window_left=255)),
    ("rope_swa_d64_gqa2", (1, 700, 4, 2, 64, "bf16"), "rope", dict(rope_base=1e4, window_left=63)),
    ("rope_self_only", (1, 130, 4, 1, 128, "bf16"), "rope", dict(rope_base=1e4, window_left=0)),
    ("fp32_rope_swa", (1, 200, 4, 2, 64, "fp32"), "rope", dict(rope_base=1e4, window_left=40)),
    ("fp32_nope_global", (1, 150, 4, 4, 128, "fp32"), "nope", dict(window_left=-1)),
]


@pytest.mark.parametrize("name,shape,mode,kw", ALIBI, ids=[c[0] for c in ALIBI])
def test_prefill_alibi(name, shape, mode, kw):
    B, S, Hq, Hkv, d, dtype = shape
    seed = zlib.crc32(name.encode()) % 1000
    inp = _inputs(B, S, Hq, Hkv, d, dtype, seed=seed)
    slopes = _slopes(Hq, seed)
    q, k, v, pos = (inp[n].to(DEV) for n in ("q", "k", "v", "pos"))
    sl = torch.from_numpy(slopes).to(DEV)
    o, lse = P.prefill(q, k, v, pos if mode != "nope" else None, mode=mode, return_lse=True, alibi_slopes=sl, **kw)
    o_s, _ = P.prefill(q, k, v, pos if mode != "nope" else None, mode=mode, return_lse=True, alibi_slopes=sl,
                       schedule="static", **kw)
    torch.cuda.synchronize()
    if dtype == "bf16":
        assert torch.equal(o, o_s), "queued and static schedules differ"
    o_ref, lse_ref = O.prefill_ref(*_np(inp), mode, operand_round=dtype, alibi_slopes=slopes.astype(np.float64), **kw)
    _compare(o, lse, o_ref, lse_ref, dtype, name)


def test_prefill_alibi_zero_slopes_equal_plain():
    inp = _inputs(1, 500, 8, 2, 128, "bf16", seed=511)
    q, k, v, pos = (inp[n].to(DEV) for n in ("q", "k", "v", "pos"))
    kw = dict(rope_base=1e4, period=128, window_left=100)
    o_a = P.prefill(q, k, v, pos, mode="rope", alibi_slopes=torch.zeros(8, device=DEV), **kw)
    o_p = P.prefill(q, k, v, pos, mode="rope", **kw)
    torch.cuda.synchronize()
    assert_close(to_np(o_a), to_np(o_p), "bf16", "zero slopes vs plain")


DEC_ALIBI = [
    # name, (B, L, Hq, Hkv, d), mode, kwargs, lens
    ("nope_swa_split", (2, 3000, 8, 2, 128), "nope", dict(window_left=500), [3000, 777]),
    ("rope_global_rows_layout", (1, 4500, 32, 8, 128), "rope", dict(window_left=-1), [4500]),
    ("nope_swa_d64", (2, 1500, 8, 4, 64), "nope", dict(window_left=100), [1500, 1]),
]


@pytest.mark.parametrize("name,shape,mode,kw,lens", DEC_ALIBI, ids=[c[0] for c in DEC_ALIBI])
def test_decode_alibi(name, shape, mode, kw, lens):
    B, L, Hq, Hkv, d = shape
    seed = zlib.crc32(name.encode()) % 1000
    w = W.Workload("t", "decode", B=B, S=L, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", mode=mode, rope_base=1e4, seed=seed)
    inp = W.make_decode_inputs(w)
    inp["kv_len"] = torch.tensor(lens, dtype=torch.int32)
    slopes = _slopes(Hq, seed)
    q, kc, vc, kv = (inp[n].to(DEV) for n in ("q", "k_cache", "v_cache", "kv_len"))
    o, lse = P.decode(q, kc, vc, kv, mode=mode, return_lse=True, alibi_slopes=torch.from_numpy(slopes).to(DEV), **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_decode(inp, mode, alibi_slopes=slopes.astype(np.float64), **kw)
    _compare(o, lse, o_ref, lse_ref, "bf16", f"decode {name}")


def test_decode_alibi_matches_prefill_last_row():
    """A P-RoPE-style SWA + ALiBi layer: cache of keys rotated at t mod P, decode at
    the last position == the last row of the prefill oracle."""
    S, Hq, Hkv, d, Pp, Wl = 900, 8, 2, 128, 256, 199
    inp = _inputs(1, S, Hq, Hkv, d, "bf16", seed=512)
    slopes = _slopes(Hq, 512)
    q, k, v, pos = (inp[n].to(DEV) for n in ("q", "k", "v", "pos"))
    phi = (pos % Pp).to(torch.int32)
    kc = P.rope_apply(k, phi, 1e4)
    ql = P.rope_apply(q[:, -1:].contiguous(), phi[:, -1:].contiguous(), 1e4)[:, 0].contiguous()
    o = P.decode(ql, kc, v, torch.tensor([S], dtype=torch.int32, device=DEV), mode="rope", window_left=Wl,
                 alibi_slopes=torch.from_numpy(slopes).to(DEV))
    torch.cuda.synchronize()
    ref, _ = O.prefill_ref(*_np(inp), "rope", rope_base=1e4, period=Pp, window_left=Wl, rows=[S - 1],
                           alibi_slopes=slopes.astype(np.float64))
    assert_close(to_np(o), ref[:, 0], "bf16", "SWA + ALiBi decode vs prefill oracle last row")


# ------------------------------------------------------------------ real-valued interpolation scale

INTERP_REAL = [
    # name, (B, S, Hq, Hkv, d, dtype), kwargs (interp_scale or w_pretrained), oracle s
    ("s1p5_gqa4", (1, 700, 8, 2, 128, "bf16"), dict(window_left=150, interp_scale=1.5), 1.5),
    ("s2p37_d64", (2, 333, 4, 2, 64, "bf16"), dict(window_left=40, interp_scale=2.37), 2.37),
    ("all_remote_s3p2", (1, 260, 4, 1, 128, "bf16"), dict(window_left=-1, interp_scale=3.2), 3.2),
    ("continuous_w_pre", (1, 1000, 8, 2, 128, "bf16"), dict(window_left=100, w_pretrained=384), 1000 / 384),
    ("continuous_below_w_pre", (1, 300, 4, 2, 128, "bf16"), dict(window_left=30, w_pretrained=512), 1.0),
    ("fp32_s1p75", (1, 150, 4, 2, 128, "fp32"), dict(window_left=20, interp_scale=1.75), 1.75),
]


@pytest.mark.parametrize("name,shape,kw,s", INTERP_REAL, ids=[c[0] for c in INTERP_REAL])
@pytest.mark.parametrize("unfused", [False, True])
def test_prefill_interp_real_scale(name, shape, kw, s, unfused):
    B, S, Hq, Hkv, d, dtype = shape
    inp = _inputs(B, S, Hq, Hkv, d, dtype, seed=zlib.crc32(name.encode()) % 1000)
    q, k, v, pos = (inp[n].to(DEV) for n in ("q", "k", "v", "pos"))
    if unfused:
        o, lse = P.prefill_bifocal_unfused(q, k, v, pos, rope_base=1e6, remote_map="interp", return_lse=True, **kw)
    else:
        o, lse = P.prefill(q, k, v, pos, mode="bifocal", rope_base=1e6, remote_map="interp", return_lse=True, **kw)
    torch.cuda.synchronize()
    assert abs(s - (O.continuous_scale(S, kw["w_pretrained"]) if "w_pretrained" in kw else s)) < 1e-15
    o_ref, lse_ref = O.prefill_ref(*_np(inp), "bifocal", rope_base=1e6, remap_scale=s,
                                   window_left=kw["window_left"], remote_map="interp", operand_round=dtype)
    _compare(o, lse, o_ref, lse_ref, dtype, f"{name}{' unfused' if unfused else ''}")


def test_decode_interp_real_scale():
    B, L, Hq, Hkv, d = 2, 3000, 32, 8, 128
    w = W.Workload("t", "decode", B=B, S=L, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", mode="bifocal", rope_base=1e6, seed=521)
    inp = W.make_decode_inputs(w)
    inp["kv_len"] = torch.tensor([3000, 1234], dtype=torch.int32)
    kw = dict(rope_base=1e6, window_left=300, remote_map="interp")
    q, kc, vc, kv = (inp[n].to(DEV) for n in ("q", "k_cache", "v_cache", "kv_len"))
    o, lse = P.decode(q, kc, vc, kv, return_lse=True, interp_scale=2.6, **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_decode(inp, "bifocal", remap_scale=2.6, **kw)
    _compare(o, lse, o_ref, lse_ref, "bf16", "decode interp s = 2.6")


def test_decode_interp_continuous_scale_per_sequence():
    """w_pretrained with the interpolation map: each sequence's own continuous
    factor s = max(1, kv_len / w_pre), formed in the kernel; a batch straddles 1."""
    B, L, Hq, Hkv, d, w_pre = 4, 2100, 8, 2, 128, 512
    w = W.Workload("t", "decode", B=B, S=L, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", mode="bifocal", rope_base=1e6, seed=522)
    inp = W.make_decode_inputs(w)
    lens = [300, 512, 700, 2100]
    inp["kv_len"] = torch.tensor(lens, dtype=torch.int32)
    kw = dict(rope_base=1e6, window_left=150, remote_map="interp")
    q, kc, vc, kv = (inp[n].to(DEV) for n in ("q", "k_cache", "v_cache", "kv_len"))
    o, lse = P.decode(q, kc, vc, kv, return_lse=True, w_pretrained=w_pre, **kw)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        s = O.continuous_scale(n, w_pre)
        sub = {x: inp[x][b:b + 1] for x in ("q", "k_cache", "v_cache", "kv_len")}
        o_ref, lse_ref = oracle_decode(sub, "bifocal", remap_scale=s, **kw)
        _compare(o[b:b + 1], lse[b:b + 1], o_ref, lse_ref, "bf16", f"len {n} s {s:.4f}")


def test_interp_continuous_generation_matches_prefill():
    """Prefill at s(S0), then decode across L = w_pre with the cache untouched: each
    decode at length L uses s = max(1, L / w_pre) and equals the last row of the
    direct interpolated bifocal oracle over the first L tokens."""
    w_pre, S0, n = 256, 200, 330
    Hq, Hkv, d = 4, 2, 128
    kw = dict(rope_base=1e6, window_left=60)
    inp = _inputs(1, n, Hq, Hkv, d, "bf16", seed=523)
    q_all, k_all, v_all, pos_all = (inp[x].to(DEV) for x in ("q", "k", "v", "pos"))
    kc = P.rope_apply(k_all, pos_all, kw["rope_base"])
    outs = {}
    for L in (S0, w_pre, w_pre + 1, 300, n):
        ql = P.rope_apply(q_all[:, L - 1:L].contiguous(), pos_all[:, L - 1:L].contiguous(), kw["rope_base"])
        outs[L] = P.decode(ql[:, 0].contiguous(), kc, v_all, torch.tensor([L], dtype=torch.int32, device=DEV),
                           mode="bifocal", remote_map="interp", w_pretrained=w_pre, **kw)
    torch.cuda.synchronize()
    qn, kn, vn, pn = _np(inp)
    for L, o in outs.items():
        s = O.continuous_scale(L, w_pre)
        ref, _ = O.prefill_ref(qn[:, :L], kn[:, :L], vn[:, :L], pn[:, :L], "bifocal", remap_scale=s,
                               remote_map="interp", rows=[L - 1], **kw)
        assert_close(to_np(o), ref[:, 0], "bf16", f"decode at L = {L} (s = {s:.4f})")


# ------------------------------------------------------------------ graph capture of the queued prefill

def test_two_graphs_on_one_capture_stream_replay_in_any_order():
    """Two prefill graphs captured on the same side stream (each capture gets its
    own zero-filled queue buffer) replay in either order, and back to back, to the
    eager results."""
    outs, refs, graphs, keep = [], [], [], []
    side = torch.cuda.Stream(device=DEV)
    for i, (mode, kw) in enumerate([("bifocal", dict(rope_base=1e6, remap_scale=2, window_left=300)),
                                    ("rope", dict(rope_base=1e4, period=256, window_left=127))]):
        inp = _inputs(1, 2500, 8, 2, 128, "bf16", seed=530 + i)
        q, k, v, pos = (inp[n].to(DEV) for n in ("q", "k", "v", "pos"))
        o = torch.empty_like(q)
        keep.append((q, k, v, pos))  # a graph does not keep its inputs alive
        run = (lambda q=q, k=k, v=v, pos=pos, o=o, mode=mode, kw=kw:
               P.prefill(q, k, v, pos, mode=mode, out=o, **kw))
        run()
        torch.cuda.synchronize()
        refs.append(o.clone())
        outs.append(o)
        side.wait_stream(torch.cuda.current_stream(DEV))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            run()
        torch.cuda.synchronize()
        graphs.append(g)
    for order in ((0, 1), (1, 0), (1, 1, 0, 0)):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for gi in order:
            graphs[gi].replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(o, ref), order

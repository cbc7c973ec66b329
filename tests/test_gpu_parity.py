"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded inputs. Small shapes span several tiles, ragged tails and the
degenerate cases; the full-size workloads are checked on all rows (EndPrompt,
P-RoPE/NoPE, every sequence of the 128K decode batches) or on about 512
stratified sampled rows (64K/128K bifocal)."""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
import position_remapped_rope_amd as P
import workloads as W
from parity import (LSE_TOL, assert_close, check_prefill, gpu_decode, log, oracle_decode, to_np)

pytestmark = pytest.mark.gpu


def _inputs(B, S, Hq, Hkv, d, dtype, seed, ids=None):
    w = W.Workload("t", "prefill", B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, mode="rope",
                   rope_base=1e4, seed=seed)
    inp = W.make_prefill_inputs(w)
    if ids is not None:
        inp["pos"] = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(ids, (B, S)).astype(np.int32)))
    return inp


# ------------------------------------------------------------------ rope_apply

# (heads go in groups of 8 loads: H = 8 and 16 are whole groups, 12 a group and a
# rest of 4, 3, 2 and 1 a rest only)
@pytest.mark.parametrize("dtype,d,H", [("bf16", 128, 8), ("fp32", 64, 3), ("bf16", 6, 2), ("fp32", 256, 1),
                                       ("bf16", 128, 12), ("fp32", 128, 16)])
def test_rope_apply_matches_oracle(dtype, d, H):
    rng = np.random.default_rng(d + H)
    B, S = 2, 300
    x32 = rng.standard_normal((B, S, H, d)).astype(np.float32)
    x = W.to_dtype_tensor(x32, dtype)
    pos = rng.integers(-140000, 140000, size=(B, S)).astype(np.int32)
    pos[0, :4] = [0, 1, 2**31 - 1, -2**31 + 1]
    base = 1e6
    y = P.rope_apply(x.cuda(), torch.from_numpy(pos).cuda(), base)
    torch.cuda.synchronize()
    ref = O.rope_apply_ref(to_np(x), pos.astype(np.int64), base)
    got = to_np(y)
    if dtype == "bf16":
        # one rounding of an fp32-accurate result: within one bf16 ulp of the exact value
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        assert np.all(np.abs(got - ref) <= ulp * 1.0 + 1e-6), float(np.max(np.abs(got - ref) / ulp))
    else:
        err = float(np.max(np.abs(got - ref)))
        log(f"rope_apply fp32 d={d}: max_abs={err:.3e}")
        assert err < 2e-6 * max(1.0, float(np.max(np.abs(ref))))


@pytest.mark.parametrize("H", [4, 12])
def test_rope_apply_in_place(H):
    x = W.to_dtype_tensor(np.random.default_rng(5).standard_normal((1, 64, H, 128)).astype(np.float32), "bf16").cuda()
    pos = torch.arange(64, dtype=torch.int32).reshape(1, 64).cuda()
    y = P.rope_apply(x, pos, 1e4)
    x2 = x.clone()
    P.rope_apply(x2, pos, 1e4, out=x2)
    torch.cuda.synchronize()
    assert torch.equal(y, x2)


# ------------------------------------------------------------------ prefill, small shapes

SMALL = [
    # name, (B, S, Hq, Hkv, d, dtype), mode, kwargs, ids
    ("nope_gqa4_ragged", (2, 300, 8, 2, 128, "bf16"), "nope", {}, None),
    ("nope_mha_d64", (1, 130, 2, 2, 64, "bf16"), "nope", {}, None),
    ("rope_period_window", (1, 517, 4, 4, 64, "bf16"), "rope", dict(rope_base=1e4, period=128, window_left=100), None),
    ("rope_self_only", (1, 200, 6, 3, 128, "bf16"), "rope", dict(rope_base=1e4, window_left=0), None),
    ("rope_gqa3", (1, 190, 6, 2, 128, "bf16"), "rope", dict(rope_base=1e6), None),
    ("rope_endprompt_ids", (1, 256, 4, 4, 128, "bf16"), "rope", dict(rope_base=1e4), W.endprompt_ids()),
    ("rope_huge_ids", (1, 160, 4, 2, 128, "bf16"), "rope", dict(rope_base=1e4),
     (np.arange(160) + (1 << 30)).astype(np.int32)),
    ("bifocal_gqa8", (1, 700, 8, 1, 128, "bf16"), "bifocal", dict(rope_base=1e6, remap_scale=3, window_left=150), None),
    ("bifocal_w0_zero", (1, 333, 4, 2, 64, "bf16"), "bifocal", dict(rope_base=1e6, remap_scale=2, window_left=0), None),
    ("bifocal_all_remote", (1, 260, 4, 1, 128, "bf16"), "bifocal", dict(rope_base=1e6, remap_scale=4, window_left=-1), None),
    ("bifocal_all_local", (1, 130, 4, 1, 128, "bf16"), "bifocal", dict(rope_base=1e6, remap_scale=4, window_left=500), None),
    ("bifocal_s1", (2, 257, 4, 2, 128, "bf16"), "bifocal", dict(rope_base=1e6, remap_scale=1, window_left=64), None),
    ("bifocal_scale_arg", (1, 200, 4, 4, 128, "bf16"), "bifocal",
     dict(rope_base=1e6, remap_scale=2, window_left=33, softmax_scale=0.05), None),
    ("one_token", (1, 1, 4, 2, 128, "bf16"), "bifocal", dict(rope_base=1e6, remap_scale=2, window_left=8), None),
    ("tile_plus_one", (1, 65, 4, 4, 128, "bf16"), "rope", dict(rope_base=1e4, window_left=31), None),
    ("fp32_nope", (1, 100, 4, 2, 64, "fp32"), "nope", {}, None),
    ("fp32_bifocal_d128", (1, 150, 4, 2, 128, "fp32"), "bifocal", dict(rope_base=1e6, remap_scale=2, window_left=20), None),
    ("fp32_rope_period", (2, 90, 2, 1, 64, "fp32"), "rope", dict(rope_base=1e4, period=16, window_left=15), None),
]


@pytest.mark.parametrize("name,shape,mode,kw,ids", SMALL, ids=[c[0] for c in SMALL])
def test_prefill_small(name, shape, mode, kw, ids):
    B, S, Hq, Hkv, d, dtype = shape
    inp = _inputs(B, S, Hq, Hkv, d, dtype, seed=zlib.crc32(name.encode()) % 1000, ids=ids)
    check_prefill(inp, mode, dtype, what=name, **kw)


# Work-queue schedule: the same items as the static one, so the same bits.
# Items = B * Hkv * (G / HG) * ceil(S / (256 / HG)), HG = 4, 2 or 1 dividing G.
QUEUED = [
    # fewer items (5) than XCD queues
    ("five_items", (1, 300, 4, 1, 128), "bifocal", dict(rope_base=1e6, remap_scale=2, window_left=40)),
    # 72 items: queues of 9 that split head groups (claims in item order)
    ("split_groups", (3, 1000, 6, 2, 64), "rope", dict(rope_base=1e4, period=64, window_left=200)),
    # 512 items, more than the compute units: queues of two whole head groups each
    ("more_items_than_cus", (2, 8192, 8, 8, 128), "nope", {}),
    # 1024 items, bifocal with GQA 4
    ("bifocal_gqa4_1024_items", (1, 16384, 16, 4, 128), "bifocal", dict(rope_base=1e6, remap_scale=4, window_left=1000)),
]


@pytest.mark.parametrize("name,shape,mode,kw", QUEUED, ids=[c[0] for c in QUEUED])
def test_queued_schedule_equals_static(name, shape, mode, kw):
    B, S, Hq, Hkv, d = shape
    inp = _inputs(B, S, Hq, Hkv, d, "bf16", seed=zlib.crc32(name.encode()) % 1000)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    pos = inp["pos"].to(dev) if mode != "nope" else None
    o_s, l_s = P.prefill(q, k, v, pos, mode=mode, return_lse=True, schedule="static", **kw)
    queue = P.prefill_queue(dev, torch.cuda.current_stream(dev).cuda_stream)
    for rep in range(2):  # the second call reuses the buffer the first left zero
        o_q, l_q = P.prefill(q, k, v, pos, mode=mode, return_lse=True, schedule="queue", **kw)
        torch.cuda.synchronize()
        assert torch.equal(o_q, o_s) and torch.equal(l_q, l_s), (name, rep)
        assert int(queue.count_nonzero()) == 0, (name, rep)
    log(f"{name}: queued == static, queue left zero")


def test_queued_schedule_two_streams():
    """Two streams, each with its own queue buffer, running at the same time."""
    dev = torch.device("cuda:0")
    cases = []
    for i, (S, mode, kw) in enumerate([(12288, "bifocal", dict(rope_base=1e6, remap_scale=3, window_left=2000)),
                                       (12288, "nope", {})]):
        inp = _inputs(1, S, 8, 2, 128, "bf16", seed=700 + i)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        pos = inp["pos"].to(dev) if mode != "nope" else None
        ref = P.prefill(q, k, v, pos, mode=mode, schedule="static", **kw)
        cases.append((q, k, v, pos, mode, kw, ref))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in cases]
    outs = []
    for st, (q, k, v, pos, mode, kw, _) in zip(streams, cases):
        with torch.cuda.stream(st):
            outs.append([P.prefill(q, k, v, pos, mode=mode, schedule="queue", **kw) for _ in range(3)])
    torch.cuda.synchronize()
    for st, got, case in zip(streams, outs, cases):
        for o in got:
            assert torch.equal(o, case[-1])
        assert int(P.prefill_queue(dev, st.cuda_stream).count_nonzero()) == 0


def test_queued_fp32_runs_static_and_leaves_queue():
    inp = _inputs(1, 150, 4, 2, 64, "fp32", seed=17)
    dev = torch.device("cuda:0")
    q, k, v, pos = (inp[n].to(dev) for n in ("q", "k", "v", "pos"))
    kw = dict(rope_base=1e6, remap_scale=2, window_left=20)
    queue = P.prefill_queue(dev, torch.cuda.current_stream(dev).cuda_stream)
    queue.fill_(7)
    o_q = P.prefill(q, k, v, pos, mode="bifocal", schedule="queue", **kw)
    o_s = P.prefill(q, k, v, pos, mode="bifocal", schedule="static", **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_q, o_s)
    assert bool((queue == 7).all())
    queue.zero_()
    torch.cuda.synchronize()


def test_prefill_period_equals_prereduced_ids():
    inp = _inputs(1, 300, 4, 4, 128, "bf16", seed=9)
    o1 = P.prefill(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["pos"].cuda(), mode="rope",
                   rope_base=1e4, period=64, window_left=63)
    red = (inp["pos"] % 64).to(torch.int32)
    o2 = P.prefill(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), red.cuda(), mode="rope",
                   rope_base=1e4, period=0, window_left=63)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# ------------------------------------------------------------------ unfused bifocal (Jet-Long Eq. (7))

UNFUSED = [c for c in SMALL if c[2] == "bifocal"] + [
    ("unfused_w0_at_tile_edge", (1, 400, 8, 2, 128, "bf16"), "bifocal", dict(rope_base=1e6, remap_scale=2, window_left=63), None),
    ("unfused_d64_gqa2", (2, 250, 4, 2, 64, "bf16"), "bifocal", dict(rope_base=1e4, remap_scale=3, window_left=40), None),
]


@pytest.mark.parametrize("name,shape,mode,kw,ids", UNFUSED, ids=[c[0] for c in UNFUSED])
def test_unfused_bifocal_small(name, shape, mode, kw, ids):
    """Three attention calls merged by Eq. (7) on the device == the direct oracle."""
    B, S, Hq, Hkv, d, dtype = shape
    inp = _inputs(B, S, Hq, Hkv, d, dtype, seed=zlib.crc32(name.encode()) % 1000, ids=ids)
    check_prefill(inp, "bifocal", dtype, what=f"{name} unfused", unfused=True, **kw)


def test_unfused_matches_fused():
    inp = _inputs(1, 1000, 8, 2, 128, "bf16", seed=71)
    kw = dict(rope_base=1e6, remap_scale=2, window_left=300)
    from parity import gpu_prefill
    o_f, l_f = gpu_prefill(inp, "bifocal", **kw)
    o_u, l_u = gpu_prefill(inp, "bifocal", unfused=True, **kw)
    assert_close(to_np(o_u), to_np(o_f), "bf16", "unfused vs fused")
    assert float((l_u - l_f).abs().max()) < LSE_TOL["bf16"]


def test_unfused_full_window_reduces_to_call_a():
    """w0 >= S - 1: calls B and C see the same keys, W_B - W_C is exactly zero
    and the merge returns call A (plain RoPE attention) unchanged."""
    inp = _inputs(1, 300, 4, 2, 128, "bf16", seed=72)
    from parity import gpu_prefill
    o_u, _ = gpu_prefill(inp, "bifocal", unfused=True, rope_base=1e6, remap_scale=3, window_left=299)
    o_r, _ = gpu_prefill(inp, "rope", rope_base=1e6, window_left=299)
    assert torch.equal(o_u, o_r)


# ------------------------------------------------------------------ P-RoPE generation with a ring-buffer cache

def test_prope_ring_buffer_generation():
    """P-RoPE decode (P-RoPE page, section 3.2): keys rotated at phi(t) = t mod P are
    kept in a W-slot ring buffer (slot t mod W, overwritten cyclically); the decode
    at step t attends to the min(t+1, W) live slots, in any order, with no mask.
    Each step equals row t of the direct windowed P-RoPE oracle."""
    W, Pp, n = 128, 256, 420
    Hq, Hkv, d, base = 8, 4, 128, 1e4
    inp = _inputs(1, n, Hq, Hkv, d, "bf16", seed=91)
    dev = torch.device("cuda:0")
    q_all, k_all, v_all = (inp[x].to(dev) for x in ("q", "k", "v"))
    kc = torch.zeros((1, W, Hkv, d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    outs = {}
    for t in range(n):
        phi = torch.tensor([[t % Pp]], dtype=torch.int32, device=dev)
        slot = t % W
        P.rope_apply(k_all[:, t:t + 1].contiguous(), phi, base, out=kc[:, slot:slot + 1])
        vc[:, slot] = v_all[:, t]
        qt = P.rope_apply(q_all[:, t:t + 1].contiguous(), phi, base)[:, 0].contiguous()
        outs[t] = P.decode(qt, kc, vc, torch.tensor([min(t + 1, W)], dtype=torch.int32, device=dev),
                           mode="rope", rope_base=base, window_left=-1)
    torch.cuda.synchronize()
    checks = [0, 5, W - 2, W - 1, W, Pp - 1, Pp, Pp + W, n - 1]
    ref, _ = O.prefill_ref(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), inp["pos"].numpy(), "rope",
                           rope_base=base, period=Pp, window_left=W - 1, rows=checks)
    for c, t in enumerate(checks):
        assert_close(to_np(outs[t]), ref[:, c], "bf16", f"ring step t = {t}")


# ------------------------------------------------------------------ interpolated remote mapping

INTERP = [
    ("interp_gqa4", (1, 700, 8, 2, 128, "bf16"), dict(rope_base=1e6, remap_scale=2, window_left=150), None),
    ("interp_s3_d64", (2, 333, 4, 2, 64, "bf16"), dict(rope_base=1e4, remap_scale=3, window_left=40), None),
    ("interp_all_remote", (1, 260, 4, 1, 128, "bf16"), dict(rope_base=1e6, remap_scale=4, window_left=-1), None),
    ("interp_huge_ids", (1, 300, 4, 2, 128, "bf16"), dict(rope_base=1e6, remap_scale=5, window_left=70),
     (np.arange(300) + (1 << 20)).astype(np.int32)),
    ("interp_fp32", (1, 150, 4, 2, 128, "fp32"), dict(rope_base=1e6, remap_scale=2, window_left=20), None),
]


@pytest.mark.parametrize("name,shape,kw,ids", INTERP, ids=[c[0] for c in INTERP])
def test_interp_prefill_small(name, shape, kw, ids):
    B, S, Hq, Hkv, d, dtype = shape
    inp = _inputs(B, S, Hq, Hkv, d, dtype, seed=zlib.crc32(name.encode()) % 1000, ids=ids)
    check_prefill(inp, "bifocal", dtype, what=name, remote_map="interp", **kw)


def test_interp_decode_matches_prefill_last_row():
    B, S, Hq, Hkv, d = 1, 900, 8, 2, 128
    inp = _inputs(B, S, Hq, Hkv, d, "bf16", seed=35)
    kw = dict(rope_base=1e6, remap_scale=3, window_left=120, remote_map="interp")
    q, k, v, pos = (inp[n].cuda() for n in ("q", "k", "v", "pos"))
    kc = P.rope_apply(k, pos, kw["rope_base"])
    ql = P.rope_apply(q[:, -1:].contiguous(), pos[:, -1:].contiguous(), kw["rope_base"])[:, 0].contiguous()
    o_dec = P.decode(ql, kc, v, torch.tensor([S], dtype=torch.int32).cuda(), mode="bifocal", **kw)
    torch.cuda.synchronize()
    o_pre, _ = O.prefill_ref(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), inp["pos"].numpy(), "bifocal",
                             rows=[S - 1], **kw)
    assert_close(to_np(o_dec), o_pre[:, 0], "bf16", "interp decode vs prefill oracle last row")


# ------------------------------------------------------------------ full-size workloads

def test_endprompt_fp32_full():
    w = W.get("endprompt_fp32")
    inp = W.make_prefill_inputs(w)
    check_prefill(inp, "rope", "fp32", what=w.name, rope_base=w.rope_base, window_left=-1)


@pytest.mark.parametrize("name", ["prope_local_8k", "nope_global_8k"])
def test_prope_nope_8k_full(name):
    w = W.get(name)
    inp = W.make_prefill_inputs(w)
    kw = dict(window_left=w.window_left)
    if w.mode == "rope":
        kw.update(rope_base=w.rope_base, period=w.period)
    check_prefill(inp, w.mode, "bf16", what=w.name, **kw)


@pytest.mark.parametrize("name,unfused", [("bifocal_64k", False), ("bifocal_128k", False), ("bifocal_64k", True)])
def test_bifocal_full_size_sampled_rows(name, unfused):
    w = W.get(name)
    log(f"{name}: generating inputs")
    inp = W.make_prefill_inputs(w)
    # 64 first rows, 64 last, 65 straddling w0, 64 at tile edges and 258 uniform
    # draws (a few coincide with the others): at least 512 distinct rows
    rows = W.stratified_rows(w.S, w.window_left, n_uniform=258, seed=w.seed, n_edge=64)
    assert len(rows) >= 512, len(rows)
    log(f"{name}: {len(rows)} sampled rows")
    check_prefill(inp, "bifocal", "bf16", rows=rows, what=w.name + (" unfused" if unfused else ""),
                  unfused=unfused, report_exact=not unfused, rope_base=w.rope_base, remap_scale=w.remap_scale,
                  window_left=w.window_left)


# ------------------------------------------------------------------ decode

DEC_SMALL = [
    ("bifocal_ragged", (3, 2000, 8, 2, 128), "bifocal", dict(rope_base=1e6, remap_scale=4, window_left=300), [2000, 1, 777]),
    ("bifocal_gqa4_d64", (2, 1500, 8, 2, 64), "bifocal", dict(rope_base=1e4, remap_scale=3, window_left=0), [1500, 513]),
    ("bifocal_all_remote", (1, 700, 4, 4, 128), "bifocal", dict(rope_base=1e6, remap_scale=2, window_left=-1), [700]),
    ("nope_window", (2, 1030, 4, 1, 128), "nope", dict(window_left=100), [1030, 40]),
    ("rope_full", (1, 600, 16, 2, 128), "rope", dict(rope_base=1e4), [600]),
    ("gqa3", (1, 900, 6, 2, 128), "bifocal", dict(rope_base=1e6, remap_scale=2, window_left=50), [900]),
    # several 2048-key chunks per sequence, lengths on and next to chunk edges
    ("multi_chunk_ragged", (4, 6200, 8, 2, 128), "bifocal", dict(rope_base=1e6, remap_scale=4, window_left=2500),
     [6200, 2048, 2049, 4097]),
    ("multi_chunk_s3_d64", (2, 4500, 16, 4, 64), "bifocal", dict(rope_base=1e6, remap_scale=3, window_left=1000),
     [4500, 4096]),
    ("multi_chunk_nope_window", (1, 5000, 8, 8, 128), "nope", dict(window_left=2100), [5000]),
    # Hkv % 4 == 0 and a grid of at most one workgroup per CU: each workgroup
    # takes 4 KV heads of 1024-key chunks, one wave per head, no LDS merge
    ("rows_layout_ragged", (3, 5000, 32, 8, 128), "bifocal", dict(rope_base=1e6, remap_scale=4, window_left=1500),
     [5000, 1, 2049]),
    ("rows_layout_interp_d64", (2, 3100, 16, 4, 64), "bifocal",
     dict(rope_base=1e4, remap_scale=2, window_left=100, remote_map="interp"), [3100, 1024]),
    ("rows_layout_rope_window", (1, 4500, 8, 4, 128), "rope", dict(rope_base=1e4, window_left=1030), [4500]),
    # interpolated remote frequencies (Jet-Long section 4.5)
    ("interp_multi_chunk", (3, 5000, 8, 2, 128), "bifocal",
     dict(rope_base=1e6, remap_scale=4, window_left=300, remote_map="interp"), [5000, 1, 4097]),
    ("interp_s3_d64", (2, 1500, 8, 2, 64), "bifocal",
     dict(rope_base=1e4, remap_scale=3, window_left=0, remote_map="interp"), [1500, 513]),
    # one sequence, 32/8 heads over a 20K-key cache: the short-cache policy takes
    # 128-key chunks, so the combine merges 157 partials (all of them) or 133 (a
    # shorter kv_len), more than one round of its per-thread batches of 4 x 32
    ("combine_two_rounds", (1, 20000, 32, 8, 128), "bifocal", dict(rope_base=1e6, remap_scale=4, window_left=4096),
     [20000]),
    ("combine_partial_round", (1, 20000, 32, 8, 128), "bifocal", dict(rope_base=1e6, remap_scale=4, window_left=4096),
     [16999]),
]


@pytest.mark.parametrize("name,shape,mode,kw,lens", DEC_SMALL, ids=[c[0] for c in DEC_SMALL])
def test_decode_small(name, shape, mode, kw, lens):
    B, L, Hq, Hkv, d = shape
    w = W.Workload("t", "decode", B=B, S=L, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", mode=mode,
                   rope_base=kw.get("rope_base", 1e4), seed=zlib.crc32(name.encode()) % 1000)
    inp = W.make_decode_inputs(w)
    inp["kv_len"] = torch.tensor(lens, dtype=torch.int32)
    o, lse = gpu_decode(inp, mode=mode, **kw)
    o_ref, lse_ref = oracle_decode(inp, mode, **kw)
    assert_close(to_np(o), o_ref, "bf16", name)
    assert float(np.max(np.abs(lse.cpu().numpy() - lse_ref))) < LSE_TOL["bf16"]


def test_decode_one_head_layout_waves_without_keys():
    """The 1-head decode layout (Hkv = 2, not a multiple of 4) issues each wave's
    first K/V loads before the query rotation whatever its key count: in the
    last chunk of the 13333-key sequence (512-key chunks, 128 keys per wave)
    only 21 keys remain, so three of its four waves have none and their loads
    fall past the buffer span. Both sequences match the oracle."""
    B, L, Hq, Hkv, d = 2, 20000, 8, 2, 128
    kw = dict(rope_base=1e6, remap_scale=4, window_left=700)
    w = W.Workload("t", "decode", B=B, S=L, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", mode="bifocal",
                   rope_base=1e6, seed=517)
    inp = W.make_decode_inputs(w)
    inp["kv_len"] = torch.tensor([20000, 13333], dtype=torch.int32)
    o, lse = gpu_decode(inp, mode="bifocal", **kw)
    o_ref, lse_ref = oracle_decode(inp, "bifocal", **kw)
    assert_close(to_np(o), o_ref, "bf16", "1-head layout, waves without keys")
    assert float(np.max(np.abs(lse.cpu().numpy() - lse_ref))) < LSE_TOL["bf16"]


@pytest.mark.parametrize("mode,kw", [
    ("bifocal", dict(rope_base=1e6, remap_scale=4, window_left=300)),
    ("nope", dict(window_left=100)),
])
def test_decode_empty_sequences(mode, kw):
    """Empty slots (kv_len 0) in a batch give O = 0 and LSE = -inf; the other
    sequences match the oracle."""
    B, L, Hq, Hkv, d = 4, 3000, 8, 2, 128
    w = W.Workload("t", "decode", B=B, S=L, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", mode=mode,
                   rope_base=kw.get("rope_base", 1e4), seed=515)
    inp = W.make_decode_inputs(w)
    inp["kv_len"] = torch.tensor([0, 3000, 0, 1], dtype=torch.int32)
    o, lse = gpu_decode(inp, mode=mode, **kw)
    o_ref, lse_ref = oracle_decode(inp, mode, **kw)
    o, lse = to_np(o), lse.cpu().numpy()
    for b in (0, 2):
        assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b])), b
    assert_close(o[[1, 3]], o_ref[[1, 3]], "bf16", f"{mode} with empty slots")
    assert float(np.max(np.abs(lse[[1, 3]] - lse_ref[[1, 3]]))) < LSE_TOL["bf16"]


def _replay_checks(graph, out, ref, eager_fn, reps=3):
    """Replay a captured graph several times, with eager work and synchronisation
    between replays, and check every replay against the eager result."""
    for r in range(reps):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        eager_fn()
        torch.cuda.synchronize()


def test_decode_graph_replay_matches_eager():
    """Decode captured in a HIP graph (both layouts: 4 heads per workgroup, and
    1 head with the LDS merge) replays to the eager result."""
    dev = torch.device("cuda:0")
    for B, L, Hq, Hkv, lens in ((2, 3000, 32, 8, [3000, 1700]), (2, 3000, 8, 2, [3000, 5])):
        w = W.Workload("t", "decode", B=B, S=L, Hq=Hq, Hkv=Hkv, d=128, dtype="bf16", mode="bifocal",
                       rope_base=1e6, seed=616)
        inp = W.make_decode_inputs(w)
        q, kc, vc = (inp[n].to(dev) for n in ("q", "k_cache", "v_cache"))
        kv_len = torch.tensor(lens, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        ws = torch.empty(P.decode_workspace_size(B, L, Hq, 128), dtype=torch.uint8, device=dev)
        kw = dict(rope_base=1e6, remap_scale=4, window_left=600)
        run = lambda: P.decode(q, kc, vc, kv_len, mode="bifocal", out=o, workspace=ws, **kw)
        run()
        torch.cuda.synchronize()
        ref = o.clone()
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            run()
        torch.cuda.synchronize()
        _replay_checks(g, o, ref, run)


def test_prefill_queued_graph_replay_matches_eager():
    """The queued prefill captured in a HIP graph: the capture stream's queue
    buffer is left zero by every replay, so replays keep matching."""
    dev = torch.device("cuda:0")
    inp = _inputs(1, 3000, 8, 2, 128, "bf16", seed=617)
    q, k, v, pos = (inp[n].to(dev) for n in ("q", "k", "v", "pos"))
    o = torch.empty_like(q)
    kw = dict(rope_base=1e6, remap_scale=2, window_left=500)
    run = lambda: P.prefill(q, k, v, pos, mode="bifocal", out=o, **kw)
    run()
    torch.cuda.synchronize()
    ref = o.clone()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        run()  # creates the side stream's queue buffer before capture
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    _replay_checks(g, o, ref, run)
    assert int(P.prefill_queue(dev, side.cuda_stream).count_nonzero()) == 0


def test_decode_workspace_reuse():
    """One workspace serves consecutive calls with other lengths: each result is
    bit-identical to a call with a fresh workspace (no state survives a call)."""
    B, L, Hq, Hkv, d = 2, 5000, 8, 2, 128
    w = W.Workload("t", "decode", B=B, S=L, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", mode="bifocal",
                   rope_base=1e6, seed=404)
    inp = W.make_decode_inputs(w)
    dev = torch.device("cuda:0")
    q, kc, vc = (inp[n].to(dev) for n in ("q", "k_cache", "v_cache"))
    kw = dict(rope_base=1e6, remap_scale=2, window_left=700)
    ws = torch.full((P.decode_workspace_size(B, L, Hq, d),), 0x7f, dtype=torch.uint8, device=dev)
    for lens in ([5000, 3000], [1, 4097], [5000, 5000], [2048, 2049]):
        kv_len = torch.tensor(lens, dtype=torch.int32, device=dev)
        o_reuse = P.decode(q, kc, vc, kv_len, mode="bifocal", workspace=ws, **kw)
        o_fresh = P.decode(q, kc, vc, kv_len, mode="bifocal", **kw)
        torch.cuda.synchronize()
        assert torch.equal(o_reuse, o_fresh), lens
    sub = dict(inp, kv_len=torch.tensor([2048, 2049], dtype=torch.int32))
    o_ref, _ = oracle_decode(sub, "bifocal", **kw)
    assert_close(to_np(o_reuse), o_ref, "bf16", "reused workspace vs oracle")


# ------------------------------------------------------------------ dynamic group size (Jet-Long Eq. (2))

def test_dynamic_g_prefill_equals_fixed_scale():
    """w_pretrained > 0 uses s = G(S); with G(S) = 3 the result is the fixed-s call's, bit for bit."""
    inp = _inputs(1, 700, 4, 2, 128, "bf16", seed=81)
    from parity import gpu_prefill
    kw = dict(rope_base=1e6, window_left=100)
    o_dyn, _ = gpu_prefill(inp, "bifocal", w_pretrained=256, **kw)  # ceil(700 / 256) = 3
    o_fix, _ = gpu_prefill(inp, "bifocal", remap_scale=3, **kw)
    assert torch.equal(o_dyn, o_fix)
    o_un, _ = gpu_prefill(inp, "bifocal", unfused=True, w_pretrained=256, **kw)
    o_unf, _ = gpu_prefill(inp, "bifocal", unfused=True, remap_scale=3, **kw)
    assert torch.equal(o_un, o_unf)


def test_dynamic_g_decode_batch_straddles_boundaries():
    """One decode call whose sequences sit on both sides of w_pretrained multiples:
    each uses its own s = G(kv_len)."""
    B, L, Hq, Hkv, d = 4, 1600, 8, 2, 128
    w = W.Workload("t", "decode", B=B, S=L, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", mode="bifocal", rope_base=1e6, seed=82)
    inp = W.make_decode_inputs(w)
    lens = [512, 513, 1025, 1600]
    inp["kv_len"] = torch.tensor(lens, dtype=torch.int32)
    kw = dict(rope_base=1e6, window_left=200)
    o, lse = gpu_decode(inp, mode="bifocal", w_pretrained=512, **kw)
    for b, n in enumerate(lens):
        G = O.group_size(n, 512)
        sub = {"q": inp["q"][b:b + 1], "k_cache": inp["k_cache"][b:b + 1], "v_cache": inp["v_cache"][b:b + 1],
               "kv_len": inp["kv_len"][b:b + 1]}
        o_ref, lse_ref = oracle_decode(sub, "bifocal", remap_scale=G, **kw)
        assert_close(to_np(o[b:b + 1]), o_ref, "bf16", f"len {n} G {G}")
        assert float(np.max(np.abs(lse.cpu().numpy()[b] - lse_ref[0]))) < LSE_TOL["bf16"]


def test_generation_across_group_size_boundaries():
    """Prefill a prompt, then generate token by token across L = w_pre and 2 w_pre:
    each new key is rotated at its own position into the cache (Jet-Long Eq. (4)),
    the cache is never rewritten, and the decode at length L (s = G(L) from the
    kernel) equals the last row of the direct bifocal oracle over the first L tokens."""
    w_pre, S0, steps = 256, 240, 290
    Hq, Hkv, d = 4, 2, 128
    kw = dict(rope_base=1e6, window_left=100)
    n = S0 + steps
    inp = _inputs(1, n, Hq, Hkv, d, "bf16", seed=83)
    dev = torch.device("cuda:0")
    q_all, k_all, v_all, pos_all = (inp[x].to(dev) for x in ("q", "k", "v", "pos"))
    # prompt: bifocal prefill at G(S0) = 1, and the base-rotated cache
    o_pre = P.prefill(q_all[:, :S0].contiguous(), k_all[:, :S0].contiguous(), v_all[:, :S0].contiguous(),
                      pos_all[:, :S0].contiguous(), mode="bifocal", w_pretrained=w_pre, **kw)
    kc = torch.zeros((1, n, Hkv, d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    P.rope_apply(k_all[:, :S0].contiguous(), pos_all[:, :S0].contiguous(), kw["rope_base"], out=kc[:, :S0])
    vc[:, :S0] = v_all[:, :S0]
    outs = {}
    for L in range(S0 + 1, n + 1):
        p = pos_all[:, L - 1:L].contiguous()
        P.rope_apply(k_all[:, L - 1:L].contiguous(), p, kw["rope_base"], out=kc[:, L - 1:L])
        vc[:, L - 1] = v_all[:, L - 1]
        ql = P.rope_apply(q_all[:, L - 1:L].contiguous(), p, kw["rope_base"])[:, 0].contiguous()
        o = P.decode(ql, kc, vc, torch.tensor([L], dtype=torch.int32, device=dev), mode="bifocal",
                     w_pretrained=w_pre, **kw)
        outs[L] = o
    torch.cuda.synchronize()
    qn, kn, vn, pn = (to_np(inp[x]) if x != "pos" else inp[x].numpy() for x in ("q", "k", "v", "pos"))
    ref0, _ = O.prefill_ref(qn[:, :S0], kn[:, :S0], vn[:, :S0], pn[:, :S0], "bifocal", remap_scale=1,
                            operand_round="bf16", **kw)
    assert_close(to_np(o_pre), ref0, "bf16", "prompt prefill at G = 1")
    for L in (S0 + 1, w_pre, w_pre + 1, 2 * w_pre, 2 * w_pre + 1, n):
        G = O.group_size(L, w_pre)
        ref, _ = O.prefill_ref(qn[:, :L], kn[:, :L], vn[:, :L], pn[:, :L], "bifocal", remap_scale=G,
                               rows=[L - 1], **kw)
        assert_close(to_np(outs[L]), ref[:, 0], "bf16", f"decode at L = {L} (G = {G})")


def test_decode_matches_prefill_last_row():
    """Cache built with rope_apply (Jet-Long Eq. (4)) + decode == last prefill row."""
    B, S, Hq, Hkv, d = 1, 1100, 8, 2, 128
    inp = _inputs(B, S, Hq, Hkv, d, "bf16", seed=31)
    kw = dict(rope_base=1e6, remap_scale=4, window_left=200)
    q, k, v, pos = (inp[n].cuda() for n in ("q", "k", "v", "pos"))
    kc = P.rope_apply(k, pos, kw["rope_base"])
    ql = P.rope_apply(q[:, -1:].contiguous(), pos[:, -1:].contiguous(), kw["rope_base"])[:, 0].contiguous()
    o_dec = P.decode(ql, kc, v, torch.tensor([S], dtype=torch.int32).cuda(), mode="bifocal", **kw)
    torch.cuda.synchronize()
    # the decode oracle on the exact same (rounded) cache and query
    ref, _ = O.decode_ref(to_np(ql), to_np(kc), to_np(v), [S], "bifocal", operand_round="bf16", **kw)
    assert_close(to_np(o_dec), ref, "bf16", "decode vs oracle on rope_apply cache")
    # and the direct prefill oracle's last row (the Eq. (4)-(6) identity), bf16 cache rounding included
    o_pre, _ = O.prefill_ref(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]), inp["pos"].numpy(),
                             "bifocal", **kw)
    assert_close(to_np(o_dec), o_pre[:, -1], "bf16", "decode vs prefill oracle last row")


@pytest.mark.parametrize("name,check_elems", [("bifocal_decode_128k_b1", [0]),
                                              ("bifocal_decode_128k_b8", list(range(8)))])
def test_decode_128k_full(name, check_elems):
    w = W.get(name)
    log(f"{name}: generating inputs")
    inp = W.make_decode_inputs(w)
    kw = dict(rope_base=w.rope_base, remap_scale=w.remap_scale, window_left=w.window_left)
    o, lse = gpu_decode(inp, mode="bifocal", **kw)
    o = to_np(o)
    for b in check_elems:
        sub = {"q": inp["q"][b:b + 1], "k_cache": inp["k_cache"][b:b + 1], "v_cache": inp["v_cache"][b:b + 1],
               "kv_len": inp["kv_len"][b:b + 1]}
        o_ref, lse_ref = oracle_decode(sub, "bifocal", **kw)
        assert_close(o[b:b + 1], o_ref, "bf16", f"{name} seq {b}")
        assert float(np.max(np.abs(lse.cpu().numpy()[b] - lse_ref[0]))) < LSE_TOL["bf16"]

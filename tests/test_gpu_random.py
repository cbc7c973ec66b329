"""Seeded random configurations against the oracle: shapes, head groupings,
head dims, modes and their parameters, id arrays and lengths drawn from fixed
seeds, so that combinations the hand-picked cases do not name are covered too.
Prefill also checks that the work-queue and static schedules give the same bits."""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
import position_remapped_rope_amd as P
import workloads as W
from parity import LSE_TOL, assert_close, check_prefill, gpu_decode, log, oracle_decode, to_np

pytestmark = pytest.mark.gpu


def _prefill_config(i):
    rng = np.random.default_rng(zlib.crc32(f"prefill-{i}".encode()))
    mode = str(rng.choice(["nope", "rope", "bifocal"], p=[0.2, 0.35, 0.45]))
    dtype = "fp32" if rng.random() < 0.15 else "bf16"
    d = int(rng.choice([64, 128]))
    while True:
        Hkv, G = int(rng.choice([1, 2, 3, 4, 8])), int(rng.choice([1, 2, 3, 4, 8]))
        if Hkv * G <= 24:
            break
    B, S = int(rng.integers(1, 4)), int(rng.integers(1, 650))
    kw = {}
    ids = None
    if mode != "nope":
        kind = rng.integers(0, 4)
        if kind == 1:    # shifted by a large constant
            ids = np.arange(S) + int(rng.integers(1, 1 << 30))
        elif kind == 2:  # increasing with random gaps
            ids = np.cumsum(rng.integers(0, 5, size=S))
        elif kind == 3:  # any non-negative ids, unordered
            ids = rng.integers(0, 100000, size=S)
        kw["rope_base"] = float(rng.choice([1e4, 1e6]))
    if mode == "rope":
        kw["period"] = int(rng.choice([0, int(rng.integers(1, 300))]))
        kw["window_left"] = int(rng.choice([-1, int(rng.integers(0, S))]))
    elif mode == "nope":
        kw["window_left"] = int(rng.choice([-1, int(rng.integers(0, S))]))
    else:
        kw["remap_scale"] = int(rng.integers(1, 6))
        kw["window_left"] = int(rng.choice([-1, 0, int(rng.integers(0, S))]))
        if rng.random() < 0.3:
            kw["remote_map"] = "interp"
    if rng.random() < 0.2:
        kw["softmax_scale"] = float(rng.uniform(0.03, 0.3))
    seed = int(rng.integers(0, 1000))
    return (B, S, G * Hkv, Hkv, d, dtype), mode, kw, ids, seed


@pytest.mark.parametrize("i", range(24))
def test_random_prefill_config(i):
    (B, S, Hq, Hkv, d, dtype), mode, kw, ids, seed = _prefill_config(i)
    what = f"random prefill {i}: B{B} S{S} H{Hq}/{Hkv} d{d} {dtype} {mode} {kw}"
    w = W.Workload("t", "prefill", B=B, S=S, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, mode="rope", rope_base=1e4,
                   seed=seed)
    inp = W.make_prefill_inputs(w)
    if ids is not None:
        inp["pos"] = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(ids, (B, S)).astype(np.int32)))
    check_prefill(inp, mode, dtype, what=what, **kw)
    # the two schedules run the same items: identical bits
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    pos = inp["pos"].to(dev) if mode != "nope" else None
    o_q, l_q = P.prefill(q, k, v, pos, mode=mode, return_lse=True, schedule="queue", **kw)
    o_s, l_s = P.prefill(q, k, v, pos, mode=mode, return_lse=True, schedule="static", **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_q, o_s) and torch.equal(l_q, l_s), what


def _decode_config(i):
    rng = np.random.default_rng(zlib.crc32(f"decode-{i}".encode()))
    mode = str(rng.choice(["nope", "rope", "bifocal"], p=[0.15, 0.15, 0.7]))
    d = int(rng.choice([64, 128]))
    Hkv, G = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2, 3, 4, 8, 16]))
    B, L = int(rng.integers(1, 5)), int(rng.integers(1, 5000))
    lens = [int(x) for x in rng.integers(0, L + 1, size=B)]
    if rng.random() < 0.5:
        lens[int(rng.integers(0, B))] = L
    if B > 1 and rng.random() < 0.25:  # an empty slot
        lens[int(rng.integers(0, B))] = 0
    kw = {"rope_base": float(rng.choice([1e4, 1e6]))}
    if mode == "bifocal":
        kw["window_left"] = int(rng.choice([-1, 0, int(rng.integers(0, L))]))
        r = rng.random()
        if r < 0.2:    # Jet-Long Eq. (2): s from each sequence's length
            kw["remap_scale"] = 1
            kw["w_pretrained"] = int(rng.integers(100, 2000))
        else:
            kw["remap_scale"] = int(rng.integers(1, 7))
            if r > 0.8:
                kw["remote_map"] = "interp"
    else:
        kw["window_left"] = int(rng.choice([-1, int(rng.integers(0, L))]))
    seed = int(rng.integers(0, 1000))
    return (B, L, G * Hkv, Hkv, d), mode, kw, lens, seed


@pytest.mark.parametrize("i", range(16))
def test_random_decode_config(i):
    (B, L, Hq, Hkv, d), mode, kw, lens, seed = _decode_config(i)
    what = f"random decode {i}: B{B} L{L} H{Hq}/{Hkv} d{d} {mode} lens {lens} {kw}"
    w = W.Workload("t", "decode", B=B, S=L, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", mode=mode,
                   rope_base=kw["rope_base"], seed=seed)
    inp = W.make_decode_inputs(w)
    inp["kv_len"] = torch.tensor(lens, dtype=torch.int32)
    o, lse = gpu_decode(inp, mode=mode, **kw)
    o, lse = to_np(o), lse.cpu().numpy()
    if kw.get("w_pretrained", 0) > 0:
        # the oracle takes s itself: Jet-Long Eq. (2) per sequence, s = G(kv_len)
        okw = {k: v for k, v in kw.items() if k != "w_pretrained"}
        refs = []
        for b in range(B):
            sub = {n: inp[n][b:b + 1] for n in ("q", "k_cache", "v_cache", "kv_len")}
            refs.append(oracle_decode(sub, mode, **dict(okw, remap_scale=O.group_size(max(lens[b], 0),
                                                                                   kw["w_pretrained"]))))
        o_ref = np.concatenate([r[0] for r in refs])
        lse_ref = np.concatenate([r[1] for r in refs])
    else:
        o_ref, lse_ref = oracle_decode(inp, mode, **kw)
    live = [b for b in range(B) if lens[b] > 0]
    for b in range(B):
        if lens[b] == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b])), what
    if live:
        assert_close(o[live], o_ref[live], "bf16", what)
        assert float(np.max(np.abs(lse[live] - lse_ref[live]))) < LSE_TOL["bf16"], what
    log(f"{what}: ok")

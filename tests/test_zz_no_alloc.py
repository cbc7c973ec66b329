"""The decode entry point that allocates nothing (prope_attn_decode_noalloc),
through the C ABI: its results equal prope_attn_decode's bit for bit (and the
oracle's to the bf16 bar) on two calls in a row, the second with a smaller
input; it replays under HIP graph capture; and a launch whose partials exceed
the fixed array is refused."""
import numpy as np
import pytest
import torch

import position_remapped_rope_amd as P
import workloads as W
from parity import assert_close, oracle_decode, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _case(B, L, Hq, Hkv, lens, seed):
    w = W.Workload("t", "decode", B=B, S=L, Hq=Hq, Hkv=Hkv, d=128, dtype="bf16", mode="bifocal", rope_base=1e6,
                   seed=seed)
    inp = W.make_decode_inputs(w)
    inp["kv_len"] = torch.tensor(lens, dtype=torch.int32)
    return inp


def test_noalloc_equals_workspace_decode_two_calls():
    kw = dict(mode="bifocal", rope_base=1e6, remap_scale=4, window_left=700)
    # the second call is smaller (fewer sequences, a shorter cache, another layout)
    for B, L, Hq, Hkv, lens, seed in ((2, 9000, 32, 8, [9000, 4321], 901), (1, 1500, 8, 2, [1500], 902)):
        inp = _case(B, L, Hq, Hkv, lens, seed)
        q, kc, vc, kv = (inp[n].to(DEV) for n in ("q", "k_cache", "v_cache", "kv_len"))
        o_na, l_na = P.decode_noalloc(q, kc, vc, kv, return_lse=True, **kw)
        o_ws, l_ws = P.decode(q, kc, vc, kv, return_lse=True, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), (B, L)
        o_ref, _ = oracle_decode(inp, "bifocal", **{k: v for k, v in kw.items() if k != "mode"})
        assert_close(to_np(o_na), o_ref, "bf16", f"no-alloc decode B={B} L={L}")


def test_noalloc_under_graph_capture():
    inp = _case(2, 6000, 32, 8, [6000, 2500], 903)
    kw = dict(mode="bifocal", rope_base=1e6, remap_scale=4, window_left=500)
    q, kc, vc, kv = (inp[n].to(DEV) for n in ("q", "k_cache", "v_cache", "kv_len"))
    o = torch.empty_like(q)
    run = lambda: P.decode_noalloc(q, kc, vc, kv, out=o, **kw)
    run()
    torch.cuda.synchronize()
    ref = o.clone()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    for r in range(3):
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref), r
        run()  # eager work between replays
        torch.cuda.synchronize()


def test_noalloc_refuses_partials_beyond_the_array():
    # 64 sequences of 128K keys with 32 query heads: 64 * 32 * 64 chunks * 130 * 4 B = 68 MB > 16 MiB
    B, L, Hq, Hkv = 64, 131072, 32, 8
    assert P.decode_workspace_size(B, L, Hq, 128) > P.DECODE_SCRATCH_BYTES
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((1, 1, Hkv, 128), dtype=torch.bfloat16, device=DEV).expand(B, L, Hkv, 128)
    kv = torch.full((B,), L, dtype=torch.int32, device=DEV)
    with pytest.raises(P.PropeError, match="WORKSPACE"):
        # the refusal comes before any launch, so the (unreadable) expanded caches are never touched
        P.lib()  # noqa
        import ctypes
        p = P._params("bifocal", 1e6, 0, 4, 4096, 0.0)
        o = torch.empty_like(q)
        rc = P.lib().prope_attn_decode_noalloc(q.data_ptr(), kc.data_ptr(), kc.data_ptr(), o.data_ptr(), None,
                                               kv.data_ptr(), B, L, Hq, Hkv, 128, P.BF16, ctypes.byref(p), None)
        P._check(rc)

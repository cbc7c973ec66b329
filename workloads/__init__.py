"""Seeded synthetic inputs for remapped-position RoPE attention.

This module is shared by the tests, the benchmark and the smoke check. It
holds workload shapes, parameters and random-number generation only: no
rotation, no masking, no softmax, nothing the attention method computes. The
oracle (``oracle/``) and the HIP library both consume what it produces.

Recipe (used for every workload):

* Each tensor gets its own child of ``numpy.random.SeedSequence(seed)``
  (spawned in a fixed order), drawn with PCG64 as float32 N(0, 1).
* bf16 workloads round those float32 draws to bfloat16 with round-to-nearest-
  even (PyTorch's CPU conversion), so the oracle and the GPU read identical
  bits; fp32 workloads use the draws as they are.
* Position ids are int32 arrays built from the workload's description
  (EndPrompt two-segment ids, or plain token indices). Any remapping of ids
  (period, aliasing) is left to the code under test.
* "Peaky" K (the 128K bifocal workload): round(frac * B * S * Hkv) K rows,
  a row being one (batch, token, KV head) head_dim vector, chosen uniformly
  without replacement, are multiplied by a factor before rounding.
* Decode caches are drawn per batch element, so a check of one sequence can
  regenerate just that sequence.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_prefill_inputs", "make_decode_inputs",
           "endprompt_ids", "to_dtype_tensor", "stratified_rows"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str              # "prefill" or "decode"
    B: int
    S: int                 # sequence length (prefill) or cache length L (decode)
    Hq: int
    Hkv: int
    d: int
    dtype: str             # "bf16" or "fp32"
    mode: str              # "nope", "rope", "bifocal"
    rope_base: float
    period: int = 0        # P for periodic ids (0 = none)
    remap_scale: int = 1   # s (integer group size) for bifocal
    window_left: int = -1  # max kept i - j (rope/nope), or w0 (bifocal)
    seed: int = 0
    ids: str = "index"     # "index" or "endprompt"
    peaky_frac: float = 0.0
    peaky_factor: float = 1.0
    description: str = ""

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the method is evaluated on (shapes from the pages'
# settings: an 8B-like 32/8-head and a 1.7B-like 16/8-head layer, a tiny
# EndPrompt case and a P-RoPE/NoPE pair).
WORKLOADS = {
    "endprompt_fp32": Workload(
        "endprompt_fp32", "prefill", B=1, S=256, Hq=4, Hkv=4, d=64, dtype="fp32", mode="rope",
        rope_base=1e4, window_left=-1, seed=0, ids="endprompt",
        description="two-segment ids 0..191 then 8128..8191, full causal, fp32"),
    "prope_local_8k": Workload(
        "prope_local_8k", "prefill", B=1, S=8192, Hq=16, Hkv=16, d=128, dtype="bf16", mode="rope",
        rope_base=1e4, period=1024, window_left=511, seed=1,
        description="P-RoPE sliding-window layer: ids t, period 1024, window 512 keys"),
    "nope_global_8k": Workload(
        "nope_global_8k", "prefill", B=1, S=8192, Hq=16, Hkv=16, d=128, dtype="bf16", mode="nope",
        rope_base=1e4, window_left=-1, seed=1,
        description="NoPE global layer over the same tensors, full causal"),
    "bifocal_64k": Workload(
        "bifocal_64k", "prefill", B=1, S=65536, Hq=32, Hkv=8, d=128, dtype="bf16", mode="bifocal",
        rope_base=1e6, remap_scale=2, window_left=4096, seed=2,
        description="bifocal prefill, 8B-like heads, w0 4096, s 2"),
    "bifocal_128k": Workload(
        "bifocal_128k", "prefill", B=1, S=131072, Hq=16, Hkv=8, d=128, dtype="bf16", mode="bifocal",
        rope_base=1e6, remap_scale=4, window_left=4096, seed=3, peaky_frac=0.01, peaky_factor=8.0,
        description="bifocal prefill, 1.7B-like heads, w0 4096, s 4, 1% of K rows x8"),
    "bifocal_decode_128k_b1": Workload(
        "bifocal_decode_128k_b1", "decode", B=1, S=131072, Hq=32, Hkv=8, d=128, dtype="bf16",
        mode="bifocal", rope_base=1e6, remap_scale=4, window_left=4096, seed=4,
        description="bifocal decode against a 128K cache, batch 1"),
    "bifocal_decode_128k_b8": Workload(
        "bifocal_decode_128k_b8", "decode", B=8, S=131072, Hq=32, Hkv=8, d=128, dtype="bf16",
        mode="bifocal", rope_base=1e6, remap_scale=4, window_left=4096, seed=4,
        description="bifocal decode against a 128K cache, batch 8"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def endprompt_ids(seg1: int = 192, seg2: int = 64, target_len: int = 8192) -> np.ndarray:
    """Two-segment ids: 0..seg1-1, then the last seg2 ids below target_len."""
    return np.concatenate([np.arange(seg1), np.arange(target_len - seg2, target_len)]).astype(np.int32)


def _normal(seq: np.random.SeedSequence, shape) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seq))
    return rng.standard_normal(size=shape, dtype=np.float32)


def to_dtype_tensor(a: np.ndarray, dtype: str):
    """float32 array -> torch CPU tensor of the workload dtype (RNE for bf16)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "fp32":
        return t
    raise ValueError(dtype)


def _ids(w: Workload, S: int) -> np.ndarray:
    if w.ids == "endprompt":
        ids = endprompt_ids()
        assert ids.shape[0] == S, (ids.shape, S)
        return ids
    return np.arange(S, dtype=np.int32)


def make_prefill_inputs(w: Workload, S: Optional[int] = None, B: Optional[int] = None):
    """Returns dict of torch CPU tensors q, k, v ([B,S,H,d], workload dtype) and pos (int32 [B,S]).

    ``S``/``B`` override the workload's sizes (smaller parity cases drawn with
    the same recipe and seed).
    """
    import torch
    S = w.S if S is None else S
    B = w.B if B is None else B
    cq, ck, cv, cp = np.random.SeedSequence(w.seed).spawn(4)
    q = _normal(cq, (B, S, w.Hq, w.d))
    k = _normal(ck, (B, S, w.Hkv, w.d))
    v = _normal(cv, (B, S, w.Hkv, w.d))
    if w.peaky_frac > 0:
        n_rows = B * S * w.Hkv
        n_peaky = int(round(w.peaky_frac * n_rows))
        rng = np.random.Generator(np.random.PCG64(cp))
        rows = rng.choice(n_rows, size=n_peaky, replace=False)
        k.reshape(n_rows, w.d)[rows] *= np.float32(w.peaky_factor)
    pos = np.broadcast_to(_ids(w, S), (B, S)).astype(np.int32).copy()
    return {
        "q": to_dtype_tensor(q, w.dtype),
        "k": to_dtype_tensor(k, w.dtype),
        "v": to_dtype_tensor(v, w.dtype),
        "pos": torch.from_numpy(pos),
    }


def make_decode_inputs(w: Workload, L: Optional[int] = None, B: Optional[int] = None,
                       batch_elems=None):
    """Decode inputs: q [B,Hq,d], k_cache/v_cache [B,L,Hkv,d], kv_len int32 [B].

    Values are N(0,1) drawn per batch element (``batch_elems`` selects which
    elements to draw; default all). The cache tensors are treated by the method
    as already base-rotated keys and values, and q as the base-rotated query.
    """
    import torch
    L = w.S if L is None else L
    B = w.B if B is None else B
    elems = list(range(B)) if batch_elems is None else list(batch_elems)
    root = np.random.SeedSequence(w.seed)
    children = root.spawn(B)
    qs, ks, vs = [], [], []
    for b in elems:
        cq, ck, cv = children[b].spawn(3)
        qs.append(_normal(cq, (w.Hq, w.d)))
        ks.append(_normal(ck, (L, w.Hkv, w.d)))
        vs.append(_normal(cv, (L, w.Hkv, w.d)))
    q = np.stack(qs)
    k = np.stack(ks)
    v = np.stack(vs)
    kv_len = np.full((len(elems),), L, dtype=np.int32)
    return {
        "q": to_dtype_tensor(q, w.dtype),
        "k_cache": to_dtype_tensor(k, w.dtype),
        "v_cache": to_dtype_tensor(v, w.dtype),
        "kv_len": torch.from_numpy(kv_len),
    }


def stratified_rows(S: int, window_left: int, n_uniform: int, seed: int, tile: int = 64,
                    n_edge: int = 16) -> np.ndarray:
    """Sampled query rows for checks at sizes where every row is too costly.

    First and last ``n_edge`` rows, rows straddling the first row that has a
    key beyond the window, rows on both sides of tile edges, and ``n_uniform``
    seeded uniform rows; sorted and unique.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed + 1000)))
    parts = [np.arange(min(n_edge, S)), np.arange(max(0, S - n_edge), S)]
    if 0 <= window_left < S:
        lo = window_left
        parts.append(np.arange(lo - n_edge // 2, lo + n_edge // 2 + 1))
    edges = rng.choice(max(1, S // tile), size=min(n_edge // 2, max(1, S // tile)), replace=False) * tile
    parts.append(edges)
    parts.append(edges - 1)
    parts.append(rng.integers(0, S, size=n_uniform))
    rows = np.concatenate(parts)
    rows = rows[(rows >= 0) & (rows < S)]
    return np.unique(rows).astype(np.int64)

"""Helpers shared by the GPU parity tests: run the HIP library through its
binding, run the oracle on the same seeded inputs, compare."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle as O
import position_remapped_rope_amd as P
import workloads as W

# bf16 gate stated for the method: max-abs 2e-2 and mean-relative (L1 ratio) 5e-3;
# fp32 gate: max-abs 1e-4.
TOL = {"bf16": dict(max_abs=2e-2, mean_rel=5e-3), "fp32": dict(max_abs=1e-4, mean_rel=1e-5)}
# LSE is a smooth maximum of a row's scores, so its error is at most the largest
# score error. A bf16 score can move by one operand ulp times the other operand
# where the GPU's fp32 rotation and the oracle's fp64 rotation round to different
# bf16 neighbours: with |q| ~ 3 and keys scaled by 8 that is ~3 * 8 * 2^-8 / sqrt(128)
# ~ 8e-3 for one flipped coordinate. The gate is 1e-2 (bf16) and 1e-5 (fp32).
LSE_TOL = {"bf16": 1e-2, "fp32": 1e-5}


def log(msg: str):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


def errors(got: np.ndarray, ref: np.ndarray):
    diff = np.abs(got - ref)
    return float(diff.max()), float(diff.sum() / max(np.abs(ref).sum(), 1e-300))


def assert_close(got, ref, dtype, what=""):
    mx, mr = errors(np.asarray(got, np.float64), np.asarray(ref, np.float64))
    tol = TOL[dtype]
    log(f"{what}: max_abs={mx:.3e} mean_rel={mr:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= tol["max_abs"] and mr <= tol["mean_rel"], f"{what}: max_abs={mx} mean_rel={mr}"
    return mx, mr


def to_np(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def gpu_prefill(inputs, mode, unfused=False, **kw):
    dev = torch.device("cuda:0")
    q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
    pos = inputs["pos"].to(dev)
    if unfused:
        assert mode == "bifocal"
        o, lse = P.prefill_bifocal_unfused(q, k, v, pos, return_lse=True, **kw)
    else:
        o, lse = P.prefill(q, k, v, pos if mode != "nope" else None, mode=mode, return_lse=True, **kw)
    torch.cuda.synchronize()
    return o, lse


def oracle_prefill(inputs, mode, dtype, rows=None, operand_round="same", **kw):
    """Prefill oracle. By default the rotated operands are rounded to the input dtype
    (the parity contract); operand_round=None gives the exact fp64 result."""
    q, k, v = (to_np(inputs[n]) for n in ("q", "k", "v"))
    pos = inputs["pos"].numpy()
    kw = {("softmax_scale" if k_ == "softmax_scale" else k_): v_ for k_, v_ in kw.items()}
    if kw.get("softmax_scale", 0.0) == 0.0:
        kw.pop("softmax_scale", None)
    rnd = dtype if operand_round == "same" else operand_round
    return O.prefill_ref(q, k, v, pos, mode, operand_round=rnd, rows=rows, **kw)


def check_prefill(inputs, mode, dtype, rows=None, what="", unfused=False, report_exact=False, **kw):
    t0 = time.time()
    o, lse = gpu_prefill(inputs, mode, unfused=unfused, **kw)
    t1 = time.time()
    o_ref, lse_ref = oracle_prefill(inputs, mode, dtype, rows=rows, **kw)
    t2 = time.time()
    o_np, lse_np = to_np(o), lse.cpu().numpy()
    if rows is not None:
        o_np = o_np[:, rows]
        lse_np = lse_np[:, :, rows]
    log(f"{what}: gpu {t1 - t0:.2f}s oracle {t2 - t1:.2f}s")
    if report_exact and dtype == "bf16":
        # for the record only: the same rows against the oracle with unrounded operands
        o_ex, lse_ex = oracle_prefill(inputs, mode, dtype, rows=rows, operand_round=None, **kw)
        mx, mr = errors(o_np, o_ex)
        log(f"{what}: vs exact-operand oracle (not gated) max_abs={mx:.3e} mean_rel={mr:.3e} "
            f"lse max_abs={float(np.max(np.abs(lse_np - lse_ex))):.3e}")
    res = assert_close(o_np, o_ref, dtype, what)
    lerr = float(np.max(np.abs(lse_np - lse_ref)))
    log(f"{what}: lse max_abs={lerr:.3e}")
    assert lerr <= LSE_TOL[dtype], f"{what}: lse error {lerr}"
    return res


def gpu_decode(inputs, **kw):
    dev = torch.device("cuda:0")
    q, kc, vc = (inputs[n].to(dev) for n in ("q", "k_cache", "v_cache"))
    kv_len = inputs["kv_len"].to(dev)
    o, lse = P.decode(q, kc, vc, kv_len, return_lse=True, **kw)
    torch.cuda.synchronize()
    return o, lse


def oracle_decode(inputs, mode, **kw):
    """Decode oracle; the remote view's rotated q and k enter the score rounded to
    bf16, as they do on the GPU's bf16 MFMA (same contract as prefill)."""
    kw = dict(kw)
    kw.setdefault("operand_round", "bf16")
    if kw.get("softmax_scale", 0.0) == 0.0:
        kw.pop("softmax_scale", None)
    return O.decode_ref(to_np(inputs["q"]), to_np(inputs["k_cache"]), to_np(inputs["v_cache"]),
                        inputs["kv_len"].numpy(), mode, **kw)

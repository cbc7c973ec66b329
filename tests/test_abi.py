"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import json
import os
import re
import subprocess

import pytest

import position_remapped_rope_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prope.h")

pytestmark = pytest.mark.skipif(not os.path.exists(P.lib_path()),
                                reason="libprope.so not built (python -m position_remapped_rope_amd.build)")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, -1, -2, -3, -4
FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced by rejected calls


def _header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(prope_[a-z_]+)\s*\(", txt)))


def test_header_symbols_exported():
    names = _header_functions()
    assert set(names) == set(P.EXPORTED_SYMBOLS)
    L = ctypes.CDLL(P.lib_path())
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", P.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (prope_[a-z_]+)\b", out))
    assert set(names) <= exported


def test_status_strings_and_version():
    L = P.lib()
    assert L.prope_version() == 2
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, 12345):
        assert isinstance(P.status_string(code), str) and P.status_string(code)


def test_group_size_golden():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "group_size.json")))
    for L_, G in g["cases"]:
        assert P.group_size(L_, g["w_pretrained"]) == G
    assert P.group_size(10, 0) == -1 and P.group_size(-1, 5) == -1
    # ceil(L / w) near the top of int64 (no overflow), and results beyond int32
    assert P.group_size(2 ** 63 - 1, 2) == -1
    assert P.group_size(2 ** 63 - 1, 2 ** 62) == 2
    assert P.group_size(2 ** 31 - 1, 1) == 2 ** 31 - 1


def _params(**kw):
    d = dict(mode=P.BIFOCAL, period=0, remap_scale=2, window_left=8, rope_base=1e6, softmax_scale=0.0, w_pretrained=0,
             remote_map=0, reserved=0, interp_scale=0.0, alibi_slopes=None)
    d.update(kw)
    return P.PropeParams(d["mode"], d["period"], d["remap_scale"], d["window_left"], d["rope_base"],
                         d["softmax_scale"], d["w_pretrained"], d["remote_map"], d["reserved"], d["interp_scale"],
                         d["alibi_slopes"])


def test_params_layout_matches_header(tmp_path):
    """The binding's ctypes struct has the C struct's size and field offsets."""
    import shutil
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "layout.c"
    fields = [f for f, _ in P.PropeParams._fields_]
    body = "".join(f'  printf("{f} %zu\\n", offsetof(prope_params, {f}));\n' for f in fields)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "prope.h"\nint main(void) {\n'
                   '  printf("sizeof %zu\\n", sizeof(prope_params));\n' + body + '  return 0;\n}\n')
    exe = tmp_path / "layout"
    r = subprocess.run([cc, "-std=c99", f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    assert int(got["sizeof"]) == ctypes.sizeof(P.PropeParams)
    for f in fields:
        assert int(got[f]) == getattr(P.PropeParams, f).offset, f


def _prefill(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, pos=FAKE, B=1, S=16, Hq=4, Hkv=2, d=128, dt=0,
             params=None, byref=True):
    L = P.lib()
    p = _params() if params is None else params
    return L.prope_attn_prefill(q, k, v, o, lse, pos, B, S, Hq, Hkv, d, dt,
                                ctypes.byref(p) if byref else None, None)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(pos=None),
    dict(B=0), dict(S=0), dict(Hq=0), dict(Hkv=0), dict(Hq=6, Hkv=4),
    dict(d=96), dict(d=256), dict(d=32), dict(dt=7),
    dict(q=FAKE + 8),
    dict(params=_params(remap_scale=0)), dict(params=_params(period=-1)),
    dict(params=_params(period=8)),                       # period only with ROPE
    dict(params=_params(mode=P.ROPE, remap_scale=2)),     # remap_scale only with BIFOCAL
    dict(params=_params(window_left=-2)), dict(params=_params(mode=5)),
    dict(params=_params(rope_base=1.0)), dict(params=_params(rope_base=float("nan"))),
    dict(params=_params(softmax_scale=-1.0)), dict(params=_params(w_pretrained=-1)),
    dict(params=_params(w_pretrained=64)),                              # dynamic G needs remap_scale 1
    dict(params=_params(mode=P.ROPE, remap_scale=1, w_pretrained=64)),  # dynamic G is bifocal only
    dict(params=_params(remote_map=2)), dict(params=_params(remote_map=-1)),
    dict(params=_params(mode=P.ROPE, remap_scale=1, remote_map=1)),     # interpolation is bifocal only
    dict(params=_params(reserved=1)),
    dict(params=_params(remap_scale=1, remote_map=1, interp_scale=0.5)),           # s >= 1
    dict(params=_params(remap_scale=1, remote_map=1, interp_scale=float("nan"))),
    dict(params=_params(remap_scale=1, remote_map=1, interp_scale=float("inf"))),
    dict(params=_params(remap_scale=1, remote_map=0, interp_scale=1.5)),           # real s is interpolation only
    dict(params=_params(remap_scale=2, remote_map=1, interp_scale=1.5)),           # one source of s
    dict(params=_params(remap_scale=1, remote_map=1, interp_scale=1.5, w_pretrained=64)),
    dict(params=_params(alibi_slopes=FAKE)),                                        # ALiBi is nope/rope only
    dict(byref=False),
])
def test_prefill_rejects(kw):
    assert _prefill(**kw) == INVALID


def test_prefill_rejects_grids_beyond_the_launch_limit():
    # a 1-D launch holds at most 2^32 - 1 work-items; the checks return before any HIP call
    rope = _params(mode=P.ROPE, remap_scale=1)
    # fp32 at d = 128: 4 (row, head) pairs per 512-thread workgroup, so 2^25 pairs need 2^32 threads
    assert _prefill(B=64, S=16384, Hq=32, Hkv=32, d=128, dt=1, params=rope) == UNSUPPORTED
    assert _prefill_queued(B=64, S=16384, Hq=32, Hkv=32, d=128, dt=1) == UNSUPPORTED
    # bf16: 256 pairs per workgroup, 2^31 pairs (256 GiB of q at d = 64)
    assert _prefill(B=256, S=1 << 17, Hq=64, Hkv=64, d=64, dt=0, params=rope) == UNSUPPORTED
    # the unfused merge takes a thread per 8 outputs: 2^28 rows at d = 128, while its calls fit
    assert _unfused(B=64, S=1 << 16, Hq=64, Hkv=64, d=128, dt=0) == UNSUPPORTED
    assert _unfused(B=64, S=16384, Hq=32, Hkv=32, d=128, dt=1) == UNSUPPORTED


def test_prefill_nope_allows_null_pos_but_rope_does_not():
    assert _prefill(pos=None, params=_params(mode=P.ROPE, remap_scale=1)) == INVALID


def _decode(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, kv_len=FAKE, B=1, Lmax=4096, Hq=32, Hkv=8, d=128, dt=0,
            params=None, ws=FAKE, ws_bytes=None):
    L = P.lib()
    p = _params() if params is None else params
    if ws_bytes is None:
        ws_bytes = L.prope_decode_workspace_size(B, Lmax, Hq, d)
    return L.prope_attn_decode(q, kc, vc, o, None, kv_len, B, Lmax, Hq, Hkv, d, dt, ctypes.byref(p),
                               ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(kv_len=None), INVALID), (dict(ws=None), INVALID),
    (dict(Lmax=0), INVALID), (dict(Hq=30, Hkv=8), INVALID), (dict(d=80), INVALID),
    (dict(params=_params(mode=P.ROPE, remap_scale=1, period=16)), INVALID),
    (dict(dt=1), UNSUPPORTED), (dict(Hq=64, Hkv=2), UNSUPPORTED),
    (dict(Lmax=1 << 21, Hkv=8, Hq=32), UNSUPPORTED),
    (dict(B=65536, Lmax=1024), UNSUPPORTED), (dict(Hq=65536, Hkv=65536, Lmax=16, d=64), UNSUPPORTED),
    (dict(ws_bytes=100), WORKSPACE),
    (dict(params=_params(alibi_slopes=FAKE)), INVALID),
    (dict(params=_params(remap_scale=1, remote_map=1, interp_scale=0.99)), INVALID),
])
def test_decode_rejects(kw, code):
    assert _decode(**kw) == code


def _unfused(q=FAKE, k=FAKE, v=FAKE, o=FAKE, pos=FAKE, B=1, S=1000, Hq=4, Hkv=2, d=64, dt=0, params=None,
             ws=FAKE, ws_bytes=None):
    L = P.lib()
    p = _params() if params is None else params
    if ws_bytes is None:
        ws_bytes = L.prope_bifocal_unfused_workspace_size(B, S, Hq, d, dt)
    return L.prope_attn_prefill_bifocal_unfused(q, k, v, o, None, pos, B, S, Hq, Hkv, d, dt, ctypes.byref(p),
                                                ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(params=_params(mode=P.ROPE, remap_scale=1)), INVALID), (dict(params=_params(mode=P.NOPE, remap_scale=1)), INVALID),
    (dict(pos=None), INVALID), (dict(ws=None), INVALID), (dict(ws=FAKE + 16), INVALID),
    (dict(ws_bytes=1000), WORKSPACE), (dict(d=96), INVALID), (dict(Hq=5, Hkv=2), INVALID),
    (dict(params=_params(remap_scale=1, remote_map=1, interp_scale=0.5)), INVALID),
])
def test_unfused_rejects(kw, code):
    assert _unfused(**kw) == code


def test_unfused_workspace_size_formula():
    L = P.lib()
    up = lambda x: (x + 255) // 256 * 256
    for B, S, Hq, d, dt in [(1, 1000, 4, 64, 0), (2, 65536, 32, 128, 0), (1, 77, 3, 128, 1)]:
        ob = up(B * S * Hq * d * (2 if dt == 0 else 4))
        lb = up(B * Hq * S * 4)
        queue = up(17 * 128)  # the three calls' work queue (fp32 leaves it unused)
        assert L.prope_bifocal_unfused_workspace_size(B, S, Hq, d, dt) == 2 * ob + 3 * lb + up(B * S * 4) + queue
    assert L.prope_bifocal_unfused_workspace_size(0, 10, 4, 64, 0) == 0


def _prefill_queued(queue=FAKE + (1 << 20), **kw):
    L = P.lib()
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, pos=FAKE, B=1, S=16, Hq=4, Hkv=2, d=128, dt=0)
    a.update(kw)
    p = _params()
    return L.prope_attn_prefill_queued(a["q"], a["k"], a["v"], a["o"], a["lse"], a["pos"], a["B"], a["S"], a["Hq"],
                                       a["Hkv"], a["d"], a["dt"], ctypes.byref(p), queue, None)


def test_prefill_queue_size():
    # 8 per-XCD item counters, 8 per-XCD done counts, 1 global done count, one 128-byte line each
    assert P.lib().prope_prefill_queue_size() == 17 * 128


@pytest.mark.parametrize("kw", [dict(queue=None), dict(queue=FAKE + (1 << 20) + 64), dict(S=0), dict(d=96),
                                dict(q=None), dict(Hq=6, Hkv=4)])
def test_prefill_queued_rejects(kw):
    assert _prefill_queued(**kw) == INVALID


def test_workspace_size_formula():
    L = P.lib()
    # [B][Hq][chunks][d + 2] float32 partials, chunks = max(ceil(Lmax / 1024), min(512, ceil(Lmax / 128)))
    assert L.prope_decode_workspace_size(1, 131072, 32, 128) == 1 * 32 * 512 * 130 * 4
    assert L.prope_decode_workspace_size(8, 3000, 4, 64) == 8 * 4 * 24 * 66 * 4
    assert L.prope_decode_workspace_size(1, 1 << 20, 8, 128) == 1 * 8 * 1024 * 130 * 4
    assert L.prope_decode_workspace_size(0, 10, 4, 64) == 0


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(pos=None), dict(d=3), dict(d=258), dict(B=0), dict(base=0.5), dict(dt=2),
    dict(y=FAKE + 64),  # partial overlap with x
])
def test_rope_apply_rejects(kw):
    L = P.lib()
    a = dict(x=FAKE, y=FAKE + (1 << 24), pos=FAKE, B=1, S=8, H=2, d=64, dt=0, base=1e4)
    a.update(kw)
    assert L.prope_rope_apply(a["x"], a["y"], a["pos"], a["B"], a["S"], a["H"], a["d"], a["dt"],
                              a["base"], None) == INVALID


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(P, "_lib", None)
    monkeypatch.setattr(P, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(P.PropeError):
        P.lib()


# ---------------------------------------------------------------- binding argument checks
# The C ABI cannot see buffer sizes, so the binding checks every caller-supplied
# output and the operand dtypes before it calls into the library. Device checks
# are switched off here (no GPU), so CPU tensors reach the shape checks; every
# case raises before a library call.

@pytest.fixture
def cpu_binding(monkeypatch):
    monkeypatch.setattr(P, "_dev", lambda t, name: None)
    return P


def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


@pytest.mark.parametrize("case", ["out_shape", "out_dtype", "lse_shape", "lse_dtype", "slopes_shape", "slopes_dtype"])
def test_binding_prefill_rejects_mismatched_outputs(cpu_binding, case):
    import torch
    q, k, v = _t(1, 16, 4, 64), _t(1, 16, 2, 64), _t(1, 16, 2, 64)
    pos = torch.zeros((1, 16), dtype=torch.int32)
    kw = {
        "out_shape": dict(out=_t(1, 15, 4, 64)),
        "out_dtype": dict(out=_t(1, 16, 4, 64, dtype=torch.float32)),
        "lse_shape": dict(lse=_t(1, 16, 4, dtype=torch.float32)),
        "lse_dtype": dict(lse=_t(1, 4, 16)),
        "slopes_shape": dict(alibi_slopes=_t(3, dtype=torch.float32)),
        "slopes_dtype": dict(alibi_slopes=_t(4)),
    }[case]
    with pytest.raises(P.PropeError):
        P.prefill(q, k, v, pos, mode="rope", **kw)


@pytest.mark.parametrize("case", ["out_shape", "lse_shape", "q_dtype", "cache_dtype", "slopes"])
def test_binding_decode_rejects_mismatched_operands(cpu_binding, case):
    import torch
    q, kc, vc = _t(2, 8, 64), _t(2, 100, 2, 64), _t(2, 100, 2, 64)
    kv_len = torch.zeros((2,), dtype=torch.int32)
    kw = {}
    if case == "out_shape":
        kw = dict(out=_t(2, 8, 32))
    elif case == "lse_shape":
        kw = dict(lse=_t(2, 4, dtype=torch.float32))
    elif case == "q_dtype":
        q = _t(2, 8, 64, dtype=torch.float32)
    elif case == "cache_dtype":
        vc = _t(2, 100, 2, 64, dtype=torch.float32)
    else:
        kw = dict(mode="nope", alibi_slopes=_t(2, dtype=torch.float32))
    with pytest.raises(P.PropeError):
        P.decode(q, kc, vc, kv_len, **kw)


def test_binding_rope_apply_and_unfused_reject_mismatched_outputs(cpu_binding):
    import torch
    x = _t(1, 8, 2, 64)
    pos = torch.zeros((1, 8), dtype=torch.int32)
    with pytest.raises(P.PropeError):
        P.rope_apply(x, pos, 1e4, out=_t(1, 8, 2, 32))
    q, k, v = _t(1, 16, 4, 64), _t(1, 16, 2, 64), _t(1, 16, 2, 64)
    with pytest.raises(P.PropeError):
        P.prefill_bifocal_unfused(q, k, v, torch.zeros((1, 16), dtype=torch.int32), remap_scale=2, window_left=3,
                                  lse=_t(1, 4, 15, dtype=torch.float32))


def _decode_noalloc(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, kv_len=FAKE, B=1, Lmax=4096, Hq=32, Hkv=8, d=128, dt=0,
                    params=None):
    L = P.lib()
    p = _params() if params is None else params
    return L.prope_attn_decode_noalloc(q, kc, vc, o, None, kv_len, B, Lmax, Hq, Hkv, d, dt, ctypes.byref(p), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(kv_len=None), INVALID), (dict(o=FAKE + 8), INVALID), (dict(d=80), INVALID),
    (dict(dt=1), UNSUPPORTED),
    # partials beyond the fixed 16 MiB array: 64 x 32 heads x 64 chunks x 130 x 4 B
    (dict(B=64, Lmax=131072), WORKSPACE),
])
def test_decode_noalloc_rejects(kw, code):
    assert _decode_noalloc(**kw) == code

"""Host-side logic of the library that needs no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "position_remapped_rope_amd", "csrc")


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_fastdiv_matches_integer_division(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    exe = tmp_path / "fastdiv_check"
    src = os.path.join(ROOT, "tests", "host", "fastdiv_check.cpp")
    r = subprocess.run([hipcc, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", f"-I{CSRC}",
                        src, "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok ")


# Kernels that may keep a few values in scratch, with the most bytes per lane:
# the bifocal bf16 prefill at d = 128 keeps a tile's scores live while it forms
# P (it takes the row max only when a sum of P is large), and the compiler
# moves some item-invariant values to scratch, reloaded once per item.
SCRATCH_ALLOWED = {"prefill_bf16_kernelILi128ELi2ELb0E": 32}


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_kernel_spills_in_inner_loops(tmp_path):
    """Every gfx950 kernel keeps its per-iteration state in registers and LDS: a
    scratch access in an inner loop (or a kernel-argument table indexed per
    lane, which goes to private memory) runs far slower. Kernels use no scratch
    at all, except the listed ones within their bound, and those never touch it
    inside a nested loop (the prefill's tile loop sits inside its item loop).
    Reads the compiler's resource remarks and the loop depths it notes on the
    block labels of the assembly."""
    import re
    import sys
    sys.path.insert(0, ROOT)
    from position_remapped_rope_amd import build as b
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    seen = 0
    for src in (s for s in b.SOURCES if s.endswith(".hip")):
        asm = tmp_path / (src + ".s")
        r = subprocess.run([hipcc, *b.FLAGS, "-x", "hip", "-fno-honor-nans", "--cuda-device-only", "-S",
                            os.path.join(CSRC, src), "-o", str(asm), "-Rpass-analysis=kernel-resource-usage"],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        names = re.findall(r"Function Name: (\S+)", r.stderr)
        scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
        assert len(names) == len(scratch), src  # (a source may hold no kernel)
        lines = asm.read_text().splitlines()
        for n, sc in zip(names, scratch):
            bound = next((v for k, v in SCRATCH_ALLOWED.items() if k in n), 0)
            assert sc <= bound, f"{src}: {n} uses {sc} bytes of scratch per lane"
            if sc == 0:
                continue
            i0 = next(i for i, l in enumerate(lines) if l.startswith(n + ":"))
            depth, n_ops = 0, 0
            for l in lines[i0 + 1:]:
                if l.startswith(".Lfunc_end"):
                    break
                if re.match(r"^\.LBB\w+:", l):
                    m = re.search(r"Depth=(\d+)", l)
                    depth = int(m.group(1)) if m else 0
                elif l.strip().startswith("scratch_"):
                    n_ops += 1
                    assert depth < 2, f"{src}: {n} touches scratch in a nested loop: {l.strip()}"
            assert n_ops > 0, n
        seen += len(names)
    assert seen >= 20


def test_item_trace_summary_phases():
    """bench.py's item-trace summary on a synthetic table: two workgroups, two
    items each, known phase lengths (100 counter ticks = 1 us)."""
    import sys
    import numpy as np
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    t = np.zeros((4, 64), dtype=np.uint64)
    for w, base in ((0, 1000), (1, 1050)):
        t[w, 0] = base
        x = base + 100  # claim of item 0 done at +1 us
        for k in range(2):
            # setup 3 us, prologue 1 us, loop 20 us, finalize 1.5 us, then a 0.5 us claim gap
            pts = [x, x + 300, x + 400, x + 2400, x + 2550]
            t[w, 1 + 5 * k: 6 + 5 * k] = pts
            x = pts[-1] + 50
        t[w, 63] = x + 10
    s = bench.summarize_item_trace(t)
    assert s["workgroups"] == 2 and s["items_traced"] == 4
    m = s["median_us"]
    assert (m["setup"], m["prologue"], m["loop"], m["finalize"], m["claim_gap"]) == (3.0, 1.0, 20.0, 1.5, 0.5)
    # each workgroup: entry to the end of its last item = 1 + 25.5 + 0.5 + 25.5 = 52.5 us, 40 us of it in
    # the tile loops; exit 0.6 us later; the second workgroup starts 0.5 us after the first
    assert abs(s["non_loop_share_median"] - (1 - 40 / 52.5)) < 1e-3  # reported to 3 decimals
    assert s["launch_span_us"] == 53.6 and s["workgroup_exit_us"] == [53.1, 53.35, 53.6]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_trace_build_compiles_and_exports_reader(tmp_path):
    """The item-phase trace build (build.py --trace) of the bf16 prefill keeps
    compiling, defines prope_item_trace_read, and the default build does not."""
    import sys
    sys.path.insert(0, ROOT)
    from position_remapped_rope_amd import build as b
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    src = os.path.join(CSRC, "prefill_bf16.hip")
    syms = {}
    for tag, extra in (("trace", b.TRACE_FLAGS), ("default", [])):
        obj = tmp_path / f"prefill_{tag}.o"
        r = subprocess.run([hipcc, *b.FLAGS, *extra, "-x", "hip", "-fno-honor-nans", "-c", src, "-o", str(obj)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        nm = subprocess.run(["nm", "-g", "--defined-only", str(obj)], capture_output=True, text=True)
        assert nm.returncode == 0, nm.stderr
        syms[tag] = nm.stdout
    assert "prope_item_trace_read" in syms["trace"]
    assert "prope_item_trace_read" not in syms["default"]

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


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_kernel_spills_to_scratch(tmp_path):
    """Every gfx950 kernel keeps its state in registers and LDS: a kernel that
    spills (or indexes a kernel-argument table per lane and so copies it to
    private memory) runs far slower. Reads the compiler's resource remarks."""
    import re
    import sys
    sys.path.insert(0, ROOT)
    from position_remapped_rope_amd import build as b
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    seen = 0
    for src in (s for s in b.SOURCES if s.endswith(".hip")):
        r = subprocess.run([hipcc, *b.FLAGS, "-x", "hip", "-fno-honor-nans", "-c", os.path.join(CSRC, src),
                            "-o", str(tmp_path / (src + ".o")), "-Rpass-analysis=kernel-resource-usage"],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        names = re.findall(r"Function Name: (\S+)", r.stderr)
        scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
        assert len(names) == len(scratch), src  # (a source may hold no kernel)
        for n, sc in zip(names, scratch):
            assert sc == 0, f"{src}: {n} uses {sc} bytes of scratch per lane"
        seen += len(names)
    assert seen >= 20

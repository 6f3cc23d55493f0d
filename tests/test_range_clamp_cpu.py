"""The attention kernels' key/query range helpers, built for the host with
hipcc: ranges stay inside [0, N) for any cu_seqlens table, so a table the
host did not check gives wrong values rather than out-of-range tile
addresses, and valid tables give each token's document range. The scanning
variants the kernels use (document found from that of an earlier token)
give the same ranges as the binary search for valid tables, from every
earlier token, and stay in bounds for invalid ones."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_range_helpers_clamp_on_host(tmp_path):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "range_check")
    src = os.path.join(ROOT, "tests", "native", "range_check.hip")
    csrc = os.path.join(ROOT, "long_context_attention_ulysses_amd", "csrc")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", csrc, "-o", exe, src],
                          stderr=subprocess.DEVNULL)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout
    assert out.stdout.strip().endswith("OK")

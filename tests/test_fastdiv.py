"""The multiply-and-shift divisors the attention kernel takes for its
launch constants (column groups, splits, KV heads, q-heads per KV head, tile
count, block length): built for the host from the library's own header and
checked against integer division (see tests/hostcheck/fastdiv_check.cpp)."""
import os
import subprocess
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


def test_fastdiv_matches_integer_division():
    src = os.path.join(ROOT, "tests", "hostcheck", "fastdiv_check.cpp")
    inc = os.path.join(ROOT, "block_diffusion_draft_vocab_amd", "csrc")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "fastdiv_check")
        # host code only: the header's device functions are not instantiated
        subprocess.run([HIPCC, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
                        "-I", inc, "-I", os.path.join(ROOT, "include"), src, "-o", exe],
                       check=True, capture_output=True, text=True, timeout=600)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 mismatches" in r.stdout

"""Host check of the split attention's escape indexing (no GPU): tests/escape_bounds.cpp is built
host-only from the kernels' own helpers in csrc/codec_dev.h and walks the rebuild's per-lane
steps for random, dense, all-raw, all-wide and corrupt tag words against every count of stored
escape pieces, for 16-token groups (escape units of two bytes) and 8-token groups (units of one
byte, four groups per CODE unit).  A corrupt tile's escape reads stay inside its staged escape bytes (or, for the
always-issued plane read, at most one unused unit past them, inside the workgroup's LDS)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_escape_reads_stay_inside_the_staged_pieces(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    exe = tmp_path / "escape_bounds"
    subprocess.check_call([hipcc, "-x", "hip", "--offload-host-only", "-O1", "-std=c++17",
                           "-I", os.path.join(ROOT, "decode_attention_calibrate_amd", "csrc"),
                           "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "escape_bounds.cpp"), "-o", str(exe)])
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.startswith("ok"), res.stdout + res.stderr

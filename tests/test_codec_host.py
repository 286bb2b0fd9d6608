"""Exhaustive host-side check of the HIP library's codec arithmetic.

tests/host/codec_check.hip includes the library's device codec header
(quantization_aware_attention_nvfp4_amd/csrc/aq_device.hpp, whose functions are
__host__ __device__) and compares it on the CPU with the oracle (dlopen of
liboracle.so): every fp32 for the 1/6 quotient, 11 binades x 8 significands for
the Markstein quotient, all E4M3/E2M1 rounding decisions, and every
(bf16 amax, bf16 x) pair of a unit-scale block.  CPU and gfx950 both round
fp32 add/mul/fma/div to nearest-even, so agreement here carries over."""
import os
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "codec_check.hip")
CSRC = os.path.join(ROOT, "quantization_aware_attention_nvfp4_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_device_codec_matches_oracle_exhaustively(tmp_path):
    exe = tmp_path / "codec_check"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-fopenmp", "-ffp-contract=off", "-I", CSRC, SRC,
                    "-o", str(exe), "-ldl"], check=True, capture_output=True)
    r = subprocess.run([str(exe), oracle.build()], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(": ok") == 6

"""The library's fp32 -> bf16 rounding (the layer output's last step), run on the host.

bf16_bits_rne is compiled for the host from the library's own device header and checked
against torch's fp32 -> bfloat16 conversion (round to nearest even) on every special class
and on random bit patterns; a NaN must come out a NaN of the same sign (torch canonicalises
NaNs, so for them only the class and the sign are compared)."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = r"""
#include <cstdio>
#include <cstdint>
#include <vector>
#include "moe_dev.h"
int main() {
  std::vector<uint32_t> in;
  uint32_t u;
  while (fread(&u, 4, 1, stdin) == 1) in.push_back(u);
  for (uint32_t v : in) {
    uint16_t o = moe::bf16_bits_rne(v);
    fwrite(&o, 2, 1, stdout);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def rounder(tmp_path_factory):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not shutil.which(hipcc):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("bf16")
    src = d / "round.cpp"
    src.write_text(SRC)
    exe = d / "round"
    inc = os.path.join(ROOT, "expert_cache_offload_amd", "csrc")
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
                    f"-I{inc}", str(src), "-o", str(exe)], check=True, capture_output=True)

    def run(bits: np.ndarray) -> np.ndarray:
        r = subprocess.run([str(exe)], input=bits.astype("<u4").tobytes(), capture_output=True,
                           check=True)
        return np.frombuffer(r.stdout, dtype="<u2")
    return run


def _torch_bf16(bits: np.ndarray) -> np.ndarray:
    f = torch.from_numpy(bits.astype(np.uint32).view(np.float32).copy())
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_finite_and_inf_match_torch(rounder):
    rng = np.random.default_rng(0)
    special = np.array([0, 0x80000000, 0x7f800000, 0xff800000, 1, 0x807fffff, 0x3f808000,
                        0x3f818000, 0x3f80ffff, 0x7f7fffff, 0x7f7f8000, 0xff7f8000, 0x00008000,
                        0x0001ffff, 0x3f7fffff, 0x477fe000], dtype=np.uint32)
    bits = np.concatenate([special, rng.integers(0, 2**32, 200_000, dtype=np.uint64)
                           .astype(np.uint32)])
    bits = bits[(bits & 0x7fffffff) <= 0x7f800000]  # finite values and infinities
    assert np.array_equal(rounder(bits), _torch_bf16(bits))


def test_nan_stays_nan_with_its_sign(rounder):
    rng = np.random.default_rng(1)
    mant = rng.integers(1, 2**23, 5000, dtype=np.uint64).astype(np.uint32)
    mant = np.concatenate([mant, np.array([1, 0x7fff, 0x8000, 0xffff, 0x7fffff, 0x400000,
                                           0x3fffff], np.uint32)])
    for sign in (0, 0x80000000):
        bits = (sign | 0x7f800000 | mant).astype(np.uint32)
        out = rounder(bits).astype(np.uint32)
        assert np.all((out & 0x7f80) == 0x7f80), "exponent must stay all ones"
        assert np.all((out & 0x007f) != 0), "mantissa must stay non-zero (a NaN, not an inf)"
        assert np.all((out & 0x8000) == (sign >> 16)), "sign kept"
        assert np.all(np.isnan(_torch_bf16(bits).view(np.uint16).astype(np.uint32)
                               .__lshift__(16).view(np.float32)))

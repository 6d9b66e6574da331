"""The library's float64 exponential (exp_le0 in csrc/device.hpp) on the CPU.

Every float64 mass of the speculative draws and of the whole-row selections
goes through exp_le0: a Cody-Waite reduction x = k ln2/64 + r with ln2/64
split in two, the Taylor series of e^r to r^6 (|r| <= ln2/128, truncation
below 1e-19 relative), a table entry 2^((k mod 64)/64) and an exponent shift.
A host build of the same function (the table from the host's exp2) is
compared with mpmath at 120 bits:
  * x in [-708, 0] (normal results): at most 2 units in the last place -- the
    table entry (within 1 ulp), the polynomial's last fused multiply-add (half
    an ulp) and the product with the entry (half an ulp);
  * x in [-745, -708) (subnormal results): within 2 x 2^-1074;
  * x < -745 and -inf: exactly 0; x = 0: exactly 1.
The points are seeded uniform draws over the whole range and near zero, and
the float64 neighbours of the reduction's interval ends k ln2/64.
"""
import os
import subprocess

import mpmath as mp
import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "exp_le0_host.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def exp_host(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    exe = str(tmp_path_factory.mktemp("exp") / "exp_le0_host")
    subprocess.run([HIPCC, "-O2", "-std=c++17", "--offload-host-only", "-x", "hip", SRC, "-o", exe], check=True,
                   capture_output=True)

    def run(xs):
        inp = "\n".join(float(x).hex() for x in xs) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split()
        assert len(out) == len(xs)
        return [float.fromhex(o) for o in out]
    return run


def test_exp_le0_error_bound(exp_host):
    mp.mp.prec = 120
    rng = np.random.default_rng(20261202)
    xs = list(-rng.random(30000) * 745.0) + list(-rng.random(3000) * 1e-3) + list(-rng.random(3000) * 8.0)
    step = float(mp.log(2) / 64)
    for k in range(0, 745 * 93, 37):
        b = -k * step
        xs += [float(np.nextafter(b, -np.inf)), b, float(np.nextafter(b, 0.0))]
    got = exp_host(xs)
    worst_ulp, worst_sub = 0.0, 0.0
    for x, v in zip(xs, got):
        e = mp.exp(mp.mpf(x))
        if x >= -708.0:
            ulp = mp.mpf(2) ** (mp.floor(mp.log(e, 2)) - 52)
            worst_ulp = max(worst_ulp, float(abs(mp.mpf(v) - e) / ulp))
        elif x >= -745.0:
            worst_sub = max(worst_sub, float(abs(mp.mpf(v) - e) / mp.mpf(2) ** -1074))
    assert worst_ulp <= 2.0, worst_ulp
    assert worst_sub <= 2.0, worst_sub


def test_exp_le0_special_points(exp_host):
    xs = [0.0, -0.0, -5e-324, -1e-300, -745.0000001, -746.0, -1000.0, -1e308, float("-inf")]
    got = exp_host(xs)
    assert got[0] == 1.0 and got[1] == 1.0
    assert got[2] == 1.0 and got[3] == 1.0
    assert all(v == 0.0 for v in got[4:])

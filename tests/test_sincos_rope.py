"""CPU check of the fp64 sine/cosine the move kernel uses for the rotation
angle delta * theta_i (sincos_rope in akv_rope.h, a Cody-Waite reduction by
pi/2 and Taylor series).  The same source is compiled for the host with hipcc
and compared with the C library's sin and cos on the same double argument:
the reposition's one-ulp bf16 bound needs the angle's sine and cosine to
fp64 accuracy, and these are the values every re-rotated key is built from."""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

PROG = r"""
#include <cstdio>
#include <cstdlib>
#include "akv_rope.h"
int main() {
  long long delta; double theta;
  while (std::scanf("%lld %la", &delta, &theta) == 2) {
    double s, c;
    akv::sincos_rope((double)delta * theta, &s, &c);
    std::printf("%a %a\n", s, c);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def sincos_exe(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("sincos")
    src = d / "sincos.hip"
    src.write_text(PROG)
    exe = d / "sincos"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17",
                        "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROOT, "agent_kv_cache_amd", "csrc"),
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return str(exe)


def _run(exe, deltas, thetas):
    inp = "".join(f"{int(dl)} {float(th).hex()}\n" for dl, th in zip(deltas, thetas))
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    vals = [tuple(float.fromhex(x) for x in line.split()) for line in out.splitlines()]
    return np.array(vals)


def test_sincos_matches_libm(sincos_exe):
    rng = np.random.default_rng(11)
    deltas, thetas = [], []
    # RoPE frequency tables (bases 1e4 .. 5e5, d = 64 / 128) times deltas of
    # every magnitude up to 2^31 - 1
    for base in (1.0e4, 1.5e5, 5.0e5):
        for dim in (64, 128):
            th = base ** (-2.0 * np.arange(dim // 2) / dim)
            for mag in (1, 3, 255, 4096, 131071, 2 ** 20 + 7, 2 ** 31 - 1):
                for sgn in (1, -1):
                    deltas += [sgn * mag] * len(th)
                    thetas += list(th)
    n = 20000
    deltas += list(rng.integers(-(2 ** 31) + 1, 2 ** 31, size=n))
    thetas += list(rng.uniform(0.0, 1.0, size=n))
    deltas += list(rng.integers(-200000, 200000, size=n))
    thetas += list(np.exp(rng.uniform(np.log(1e-7), 0.0, size=n)))
    # arguments next to multiples of pi/2 (quadrant edges): delta * 1.0
    k = rng.integers(1, 2 ** 20, size=2000)
    deltas += list(np.rint(k * (math.pi / 2)).astype(np.int64))
    thetas += [1.0] * len(k)
    got = _run(sincos_exe, deltas, thetas)
    x = np.array([float(dl) * float(th) for dl, th in zip(deltas, thetas)])
    ref_s = np.array([math.sin(v) for v in x])
    ref_c = np.array([math.cos(v) for v in x])
    err = np.maximum(np.abs(got[:, 0] - ref_s), np.abs(got[:, 1] - ref_c))
    # a few fp64 ulps of values in [-1, 1]
    assert err.max() <= 4.5e-16, (err.max(), int(err.argmax()), x[err.argmax()])


def test_sincos_zero_and_sign(sincos_exe):
    got = _run(sincos_exe, [0, 1, -1], [0.5, 1.0, 1.0])
    assert got[0, 0] == 0.0 and got[0, 1] == 1.0          # delta 0: the identity rotation
    assert abs(got[1, 0] - math.sin(1.0)) <= 2.3e-16 and abs(got[1, 1] - math.cos(1.0)) <= 2.3e-16
    assert got[2, 0] == -got[1, 0] and got[2, 1] == got[1, 1]   # odd sine, even cosine

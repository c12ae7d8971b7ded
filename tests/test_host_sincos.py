"""CPU pin of the library's own rotary sine and cosine (csrc/common.h).

The kernels take the sin/cos of every rotary angle with the library's own
routines (Cody-Waite reduction by pi/2 in three parts, then Taylor series of
sin and cos on |r| <= pi/4): KVCMAS App. A.3 "Correction Weighting and
Positional Alignment" defines re-alignment by these angles.  The routines
are host-callable; this test compiles them for the host from the same
header and compares them with the C library's long-double sinl/cosl (64-bit
significand, so the reference itself errs by about 2^-64) over angles of
shifts up to the documented limit of 2^23 positions.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc")
                                  else None)


@pytest.fixture(scope="module")
def host_lib(tmp_path_factory):
    if HIPCC is None:
        pytest.skip("hipcc is not installed")
    out = str(tmp_path_factory.mktemp("sincos") / "host_sincos.so")
    cmd = [HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", os.path.join(HERE, "host_sincos.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return ctypes.CDLL(out)


def run(lib, x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    n = len(x)
    s, c = np.empty(n), np.empty(n)
    sf, cf = np.empty(n, np.float32), np.empty(n, np.float32)
    D, F = ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_float)
    lib.host_rope_sincos(x.ctypes.data_as(D), n, s.ctypes.data_as(D), c.ctypes.data_as(D),
                         sf.ctypes.data_as(F), cf.ctypes.data_as(F))
    return s, c, sf, cf


def rotary_angles(rng, count, theta=5e5, hd=128, limit=2 ** 23):
    """delta * theta^(-2i/hd) for shifts |delta| < limit and every pair i."""
    inv = theta ** (-2.0 * np.arange(hd // 2) / hd)
    d = rng.integers(-(limit - 1), limit, count).astype(np.float64)
    return d * inv[rng.integers(0, hd // 2, count)]


def errors(lib, x):
    s, c, sf, cf = run(lib, x)
    xl = x.astype(np.longdouble)
    rs, rc = np.sin(xl), np.cos(xl)
    e64 = max(np.abs(s.astype(np.longdouble) - rs).max(), np.abs(c.astype(np.longdouble) - rc).max())
    e32 = max(np.abs(sf.astype(np.longdouble) - rs).max(), np.abs(cf.astype(np.longdouble) - rc).max())
    return float(e64) * 2.0 ** 53, float(e32) * 2.0 ** 24


def test_long_double_reference_is_finer_than_double():
    assert np.finfo(np.longdouble).nmant >= 63


def test_sincos_within_two_units_of_libm_up_to_the_shift_limit(host_lib):
    rng = np.random.default_rng(2024)
    x = np.concatenate([
        rotary_angles(rng, 20000),                        # rotary angles, theta 5e5
        rotary_angles(rng, 10000, theta=1e6),             # theta 1e6
        rng.uniform(-(2.0 ** 23), 2.0 ** 23, 10000),      # the largest angles (pair 0)
        rng.uniform(-4.0, 4.0, 5000),                     # around the first quadrants
    ])
    e64, e32 = errors(host_lib, x)
    print(f"max abs error: fp64 {e64:.3f} x 2^-53, fp32 table {e32:.3f} x 2^-24")
    assert e64 <= 2.0
    assert e32 <= 2.0


def test_sincos_near_multiples_of_a_quarter_turn(host_lib):
    # the reduction's hardest inputs: x close to k pi/2, where r is tiny and
    # the quadrant decides signs; and the shift limit itself
    k = np.arange(-2000, 2001, dtype=np.float64)
    x = np.concatenate([k * (np.pi / 2), np.nextafter(k * (np.pi / 2), np.inf),
                        np.nextafter(k * (np.pi / 2), -np.inf),
                        [2.0 ** 23 - 1, -(2.0 ** 23 - 1), 8388606.5]])
    e64, e32 = errors(host_lib, x)
    assert e64 <= 2.0 and e32 <= 2.0


def test_sincos_exact_at_zero(host_lib):
    s, c, sf, cf = run(host_lib, np.array([0.0, -0.0]))
    assert s.tolist() == [0.0, 0.0] and c.tolist() == [1.0, 1.0]
    assert sf.tolist() == [0.0, 0.0] and cf.tolist() == [1.0, 1.0]

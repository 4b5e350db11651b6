"""The bf16 layers' GeLU (gelu_bf16 in csrc/common.hpp) meets its stated bound.

GeLU(a) = a * Phi(a) with Phi the standard normal distribution function
(the erf form, 0.5 * (1 + erf(a / sqrt(2)))). The kernel takes u = min(|a|, 6)
and q = Phi(-u) as 2^p(u), p a degree-6 polynomial, and returns
max(a, 0) - u * q in one fma (a * (1 - q) for 0 <= a <= 6, a * q below 0). The coefficients are read from the kernel source and
the device arithmetic is replayed in float32 (each fma rounded once; exp2
rounded to float32; the bound leaves room for the hardware exp2, within 1 ulp):

  * relative error <= 1e-4 for |a| <= 6 (the bf16 result's step is 2^-8),
  * absolute error <= |a| * 2e-9 beyond,
  * exact special values: GeLU(0) = 0, NaN stays NaN, +inf stays +inf.
The reference is scipy's log_ndtr / ndtr (float64), not the fit itself.
"""
import os
import re

import numpy as np
from scipy.special import ndtr

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "sparse_mixture_experts_05_amd", "csrc", "common.hpp")


def _coefficients():
    body = open(SRC).read()
    body = body[body.index("float gelu_bf16(float a)"):]
    body = body[: body.index("\n}\n")]
    lits = [float(v) for v in re.findall(r"(-?\d+\.\d+(?:e-?\d+)?)f", body)]
    # lits: the clamp's bounds 0.0 and 6.0, then c6, c5, c4, ..., c0 in Horner order
    assert lits[:2] == [0.0, 6.0]
    return np.array(lits[2:9][::-1], dtype=np.float32)  # c0..c6


def _gelu_device(a):
    c = _coefficients()
    a = np.asarray(a, dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        u = np.minimum(np.abs(a), np.float32(6.0))
        u = np.where(np.isnan(a), np.float32(6.0), u)  # whatever med3 makes of a NaN: r decides
        p = np.float32(c[6])
        for k in range(5, -1, -1):
            p = np.float32(p.astype(np.float64) * u.astype(np.float64) + np.float64(c[k]))
        q = np.float32(np.exp2(p.astype(np.float64)))
        r = np.where(~(a <= 0), a, np.float32(0.0))  # NaN passes through
        # one fma: the product u * q is exact in float64, one rounding to float32
        g = (-u.astype(np.float64) * q.astype(np.float64) + r.astype(np.float64)).astype(np.float32)
        return g, q


def test_coefficients_fit_log2_phi():
    """p(u) stays within 6.6e-5 of log2 Phi(-u) on [0, 6] (float64)."""
    c = _coefficients().astype(np.float64)
    u = np.linspace(0.0, 6.0, 100001)
    p = np.polyval(c[::-1], u)
    ref = np.log2(ndtr(-u))
    assert np.max(np.abs(p - ref)) <= 6.6e-5
    assert abs(c[0] + 1.0) < 1e-4  # log2 Phi(0) = -1


def test_relative_error_bound():
    a = np.concatenate([np.linspace(-6, 6, 400001), -np.logspace(-8, 0.77, 2000),
                        np.logspace(-8, 0.77, 2000)]).astype(np.float32)
    got, _ = _gelu_device(a)
    x = a.astype(np.float64)
    ref = x * ndtr(x)
    nz = ref != 0
    rel = np.abs(got[nz] - ref[nz]) / np.abs(ref[nz])
    assert rel.max() <= 1e-4, rel.max()
    assert np.all(got[~nz] == 0)


def test_tail_bound():
    a = np.concatenate([np.linspace(6, 60, 5001), np.linspace(-60, -6, 5001)]).astype(np.float32)
    got, _ = _gelu_device(a)
    x = a.astype(np.float64)
    ref = x * ndtr(x)
    assert np.all(np.abs(got - ref) <= np.abs(x) * 2e-9 + np.abs(ref) * 1e-6)


def test_special_values():
    got, _ = _gelu_device(np.array([0.0, -0.0, np.nan, np.inf], dtype=np.float32))
    assert got[0] == 0 and got[1] == 0
    assert np.isnan(got[2])
    assert got[3] == np.inf

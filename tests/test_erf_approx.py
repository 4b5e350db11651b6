"""The kernel's erf (Abramowitz & Stegun 7.1.26) meets its published error bound.

The constants are read from the kernel source, so this checks exactly what the
GPU code uses: |erf_AS(x) - erf(x)| <= 1.5e-7 (the handbook's bound; float64
evaluation here, the device adds fp32 rounding, far below the bf16 output step).
"""
import math
import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "sparse_mixture_experts_05_amd", "csrc", "common.hpp")


def _constants():
    body = open(SRC).read()
    body = body[body.index("float erf_as7126"):]
    body = body[: body.index("\n}\n")]
    nums = [float(v) for v in re.findall(r"(-?\d+\.\d+)f", body) if float(v) != 1.0]
    # p, then a5, a4, a3, a2, a1 in Horner order (the literal 1.0s are structure)
    p, a5, a4, a3, a2, a1 = nums[:6]
    return p, (a1, a2, a3, a4, a5)


def test_constants_are_the_handbooks():
    p, a = _constants()
    assert p == 0.3275911
    assert a == (0.254829592, -0.284496736, 1.421413741, -1.453152027, 1.061405429)


def test_error_bound():
    p, a = _constants()
    x = np.concatenate([np.linspace(-6, 6, 200001), np.array([0.0, 1e-8, -1e-8, 10.0, -10.0])])
    ax = np.abs(x)
    t = 1.0 / (1.0 + p * ax)
    poly = t * (a[0] + t * (a[1] + t * (a[2] + t * (a[3] + t * a[4]))))
    y = np.sign(x) * (1.0 - poly * np.exp(-ax * ax))
    ref = np.array([math.erf(v) for v in x])
    assert np.max(np.abs(y - ref)) <= 1.5e-7

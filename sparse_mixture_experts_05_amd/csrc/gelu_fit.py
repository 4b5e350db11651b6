"""Fit of the bf16 GeLU's normal-tail polynomial (the device function gelu_bf16 in common.hpp):
p(u) ~ log2 Phi(-u) on [0, 6], degree 6, near-minimax in the absolute error of
p (so in the relative error of 2^p), by Lawson's iteratively reweighted least
squares on Chebyshev points. Prints the coefficients c0..c6 as float32."""
import numpy as np
from scipy.special import log_ndtr

U, DEG, N = 6.0, 6, 4000
t = np.cos(np.pi * (np.arange(N) + 0.5) / N)
u = (t + 1) * U / 2
f = log_ndtr(-u) / np.log(2)
A = np.stack([u ** i for i in range(DEG + 1)], 1)
w = np.full(N, 1.0 / N)
for _ in range(200):
    c, *_ = np.linalg.lstsq(A * np.sqrt(w)[:, None], f * np.sqrt(w), rcond=None)
    e = np.abs(A @ c - f)
    w = w * e
    w /= w.sum()
for i, v in enumerate(np.float32(c)):
    print(f"c{i} = {float(v):.9g}")
print("max |p - log2 Phi(-u)| =", np.abs(A @ c - f).max())

"""Coefficients of the epilogue GELU's erf (gelu_fast in moe_internal.h).

erfc(u / sqrt 2) = exp2(Q(u)) for u = |v| in [0, 6], Q(u) = sum_{k=1..6} c_k u^k
(no constant term, so erf(0) = 0 exactly).  Fitted by least squares on 8000
Chebyshev nodes, each residual weighted by max(u, 1/2) erfc(u / sqrt 2): the
size of its effect on GELU(v) = max(v, 0) - |v| erfc(|v| / sqrt 2) / 2, held
up near 0 so the error relative to |v| stays small there too.  Evaluated in
float32 as the kernel does, the result is within 2.5e-7 of GELU in absolute
terms and 4.8e-7 |v| over [-10, 10] (checked by tests/test_gelu_fast.py);
degrees 7 to 9 gain nothing in absolute terms, degree 5 is ten times worse.

    python sparse_mixture_experts_28_amd/csrc/fit_gelu.py   # prints the c_k
"""
import numpy as np
from scipy.special import erfc

U = 6.0


def fit(n_nodes: int = 8000, degree: int = 6) -> np.ndarray:
    x = np.cos(np.pi * (np.arange(n_nodes) + 0.5) / n_nodes) * U / 2 + U / 2
    y = np.log2(erfc(x / np.sqrt(2.0)))
    w = np.maximum(np.maximum(x, 0.5) * erfc(x / np.sqrt(2.0)), 1e-4)
    a = np.stack([x ** k for k in range(1, degree + 1)], 1)
    c, *_ = np.linalg.lstsq(a * w[:, None], y * w, rcond=None)
    return c.astype(np.float32)


if __name__ == "__main__":
    print(", ".join(f"{v:.9e}f" for v in fit()))

"""The epilogue GELU's approximation (gelu_fast in csrc/moe_internal.h),
evaluated in float32 the way the kernel evaluates it, against the exact erf
form; and its coefficients against the fit that produced them."""
import os
import re
import sys

import numpy as np
from scipy.special import erf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "sparse_mixture_experts_28_amd", "csrc", "moe_internal.h")


def _coefficients():
    src = open(HDR).read()
    body = src[src.index("float gelu_fast(float v)"):]
    body = body[:body.index("\n}\n")]
    nums = [float(x) for x in re.findall(r"([-+]?\d\.\d+e[-+]\d+)f", body)]
    # Horner from the highest power: the first fma holds c_n, c_(n-1); then c_(n-2) .. c_1
    return np.array(nums[::-1], dtype=np.float32)   # c_1 .. c_n


def _gelu_fast(v: np.ndarray, c: np.ndarray) -> np.ndarray:
    f = np.float32
    # med3(|v|, 0, 6): NaN gives 6
    u = np.where(np.isnan(v), f(6.0), np.minimum(np.abs(v), f(6.0))).astype(np.float32)
    # fused multiply-adds round once: the float64 product of two float32 values is exact
    u64 = u.astype(np.float64)
    q = (u64 * c[-1] + c[-2]).astype(np.float32)
    for k in range(len(c) - 3, -1, -1):
        q = (u64 * q + c[k]).astype(np.float32)
    t = (q.astype(np.float64) * u - 1.0).astype(np.float32)
    e = np.exp2(t.astype(np.float64)).astype(np.float32)
    m = np.maximum(v, f(0.0))              # propagates NaN, as the kernel's maximum does
    with np.errstate(invalid="ignore"):
        return (-(u.astype(np.float64)) * e + m).astype(np.float32)


def test_gelu_fast_error_bound():
    c = _coefficients()
    assert c.shape == (6,)
    v = np.concatenate([np.linspace(-10, 10, 200001), np.linspace(-1e-3, 1e-3, 2001)]).astype(np.float32)
    exact = 0.5 * v.astype(np.float64) * (1.0 + erf(v.astype(np.float64) / np.sqrt(2.0)))
    err = np.abs(_gelu_fast(v, c) - exact)
    assert err.max() <= 2.6e-7
    nz = np.abs(v) > 0
    assert (err[nz] / np.abs(v[nz])).max() <= 5e-7
    assert _gelu_fast(np.array([0.0], np.float32), c)[0] == 0.0
    special = _gelu_fast(np.array([np.inf, np.nan, -np.inf], np.float32), c)
    assert special[0] == np.inf and np.isnan(special[1])
    assert -1e-8 < special[2] <= 0.0


def test_gelu_fast_coefficients_match_fit():
    sys.path.insert(0, os.path.dirname(HDR))
    try:
        import fit_gelu
    finally:
        sys.path.pop(0)
    assert np.allclose(fit_gelu.fit(), _coefficients(), rtol=1e-6, atol=0)

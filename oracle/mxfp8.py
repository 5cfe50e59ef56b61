"""CPU oracle of the MXFP8 (OCP microscaling, E4M3 elements) expert path.

TEST INFRASTRUCTURE ONLY, like ``oracle.moe_ref``: used by tests, smoke() and
the bench's cpu_baseline leg, never by the product path; shares no code with
the HIP library.

The pages name FP8 expert weights as a serving option (the MoE training
guide's section 9.2 on inference: vLLM's ``quantization="fp8"``, roughly
20-30% more throughput and under 1% accuracy loss) and fix no encoding or
scaling convention.  Reading taken: the Open Compute Project's microscaling
format MXFP8, because it is the FP8 form the target's scaled matrix
instructions consume:

  * an element is an FP8 E4M3 value (1 sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN; no
    infinities; largest finite 448);
  * every block of 32 consecutive elements along the contracted dimension
    shares one power-of-two scale X = 2^s stored as an E8M0 byte s + 127;
  * quantizing a block V: s = floor(log2(max|V|)) - 8 (8 = the exponent of
    E4M3's largest power of two), element = V_i / X rounded to the nearest
    E4M3 value (ties to even mantissa), magnitudes above 448 clamped to 448;
    an all-zero block gets s = -127 and zero elements.

The layer in this form (W8A8): the activations entering each expert Linear
(x for the first, act(x W1^T + b1) for the second) and both expert weight
matrices are MXFP8 along their contracted dimension; products are exact
(everything is dequantized to float64); biases, the router and the combine
are as in ``oracle.moe_ref``.  Nothing here rounds an intermediate except the
quantization steps themselves.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from . import moe_ref

E4M3_MAX = 448.0
E4M3_EMAX = 8            # exponent of 256, the largest power of two below 448
BLOCK = 32
E8M0_BIAS = 127


def e4m3_decode(code: int) -> float:
    """Value of an E4M3 code (NaN for S.1111.111)."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    v = math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7)
    return -v if s else v


# every finite non-negative E4M3 value and its code, ascending
_POS = sorted((e4m3_decode(c), c) for c in range(0x7F))
_POS_VALUES = np.array([v for v, _ in _POS])
_POS_CODES = np.array([c for _, c in _POS], dtype=np.uint8)
_DECODE = np.array([e4m3_decode(c) for c in range(256)])


def e4m3_encode(v: float) -> int:
    """Nearest E4M3 code to v, ties to the even mantissa (even code), magnitudes
    above 448 clamped to 448; the sign of zero is kept."""
    if math.isnan(v):
        raise ValueError("NaN has no E4M3 encoding here")
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = min(abs(v), E4M3_MAX)
    i = int(np.searchsorted(_POS_VALUES, a))           # first value >= a
    if i < len(_POS_VALUES) and _POS_VALUES[i] == a:
        return sign | int(_POS_CODES[i])
    lo, hi = i - 1, i
    dlo, dhi = a - _POS_VALUES[lo], _POS_VALUES[hi] - a
    if dlo < dhi or (dlo == dhi and int(_POS_CODES[lo]) % 2 == 0):
        return sign | int(_POS_CODES[lo])
    return sign | int(_POS_CODES[hi])


def block_exponent(amax: float) -> int:
    """s = floor(log2(amax)) - 8 for amax > 0, -127 for an all-zero block,
    clamped to the E8M0 range [-127, 127]."""
    if amax == 0.0:
        return -E8M0_BIAS
    m, e = math.frexp(amax)          # amax = m 2^e, 0.5 <= m < 1: floor(log2 amax) = e - 1
    return max(-E8M0_BIAS, min(E8M0_BIAS, (e - 1) - E4M3_EMAX))


def quantize(a: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 of a [R, K] float64 array (K a multiple of 32) along its rows:
    codes uint8 [R, K] and E8M0 scale bytes uint8 [R, K/32].  The block
    exponent is floor(log2 amax) - 8 (frexp, exact); each element is
    v * 2^-s (exact) encoded as e4m3_encode does, elementwise."""
    a = np.asarray(a, dtype=np.float64)
    R, K = a.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = a.reshape(R, K // BLOCK, BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    _, e = np.frexp(amax)
    s = np.where(amax > 0, np.clip((e - 1) - E4M3_EMAX, -E8M0_BIAS, E8M0_BIAS), -E8M0_BIAS)
    y = np.ldexp(blocks, -s[:, :, None]).reshape(R, K)
    return _encode_array(y), (s + E8M0_BIAS).astype(np.uint8)


def _encode_array(y: np.ndarray) -> np.ndarray:
    """e4m3_encode over an array: the nearest finite value by binary search of
    the sorted value table, ties to the even code, magnitudes clamped to 448."""
    a = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a)                 # first table value >= a
    hi_c = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi_c] - a
    exact = _POS_VALUES[hi_c] == a
    pick_lo = (dlo < dhi) | ((dlo == dhi) & (_POS_CODES[lo] % 2 == 0))
    code = np.where(exact, _POS_CODES[hi_c], np.where(pick_lo, _POS_CODES[lo], _POS_CODES[hi_c]))
    sign = np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 [R, K] values of MXFP8 codes and scales."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    R, K = codes.shape
    x = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - E8M0_BIAS), BLOCK, axis=1)
    return _DECODE[codes] * x


def moe_forward_mxfp8_ref(x, W_g, experts_q, E: int, k: int, capacity_factor: float = 0.0, n_shared: int = 0,
                          b_g=None, kind: str = "bf16", rows: Optional[Sequence[int]] = None,
                          override_idx: Optional[np.ndarray] = None, activation: str = "gelu",
                          min_capacity: int = 0, b_sel=None):
    """The layer with MXFP8 expert Linears, in float64.

    ``experts_q(e)`` returns (W1 codes [h,d], W1 scales [h,d/32], b1 [h] or
    None, W2 codes [d,h], W2 scales [d,h/32], b2 [d] or None) with biases as
    raw inputs of ``kind``.  Routing, capacity, aux and z-loss are exactly
    those of ``oracle.moe_ref.moe_forward_ref`` (the router stays in x's own
    precision).  For each kept (token, expert) and each shared expert:
      xq  = dequantize(quantize(x rows))
      H   = act(xq W1q^T + b1);  Hq = dequantize(quantize(H))
      y   = Hq W2q^T + b2
    and the combine weights y as in the plain layer."""
    xf = moe_ref.widen(x, kind)
    T, d = xf.shape
    rows_arr = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    # routing, capacity, aux and z-loss of the plain layer; its expert outputs
    # are not needed (no rows asked), the MXFP8 experts follow below
    base = moe_ref.moe_forward_ref(x, W_g, lambda e: _no_ffn(experts_q, e, kind), E, k, capacity_factor,
                                   n_shared, b_g, kind=kind, rows=np.zeros(0, dtype=np.int64),
                                   override_idx=override_idx, activation=activation, min_capacity=min_capacity,
                                   b_sel=b_sel)
    base.rows = rows_arr
    xq = dequantize(*quantize(xf))
    want = np.zeros(T, dtype=bool)
    want[rows_arr] = True
    row_of = np.full(T, -1, dtype=np.int64)
    row_of[rows_arr] = np.arange(rows_arr.size)
    out = np.zeros((rows_arr.size, d), dtype=np.float64)
    for e in range(E + n_shared):
        if e < E:
            tok, slot = np.nonzero((base.idx == e) & base.slot_kept & want[:, None])
            if tok.size == 0:
                continue
            wts = base.w[tok, slot]
        else:
            tok, wts = rows_arr, np.ones(rows_arr.size)
        out[row_of[tok]] += wts[:, None] * expert_ffn_mxfp8(xq[tok], experts_q(e), kind, activation)
    base.out = out
    return base


def expert_ffn_mxfp8(xq: np.ndarray, eq, kind: str, activation: str) -> np.ndarray:
    """One expert on already-quantized input rows: act(xq W1q^T + b1), quantized
    along h, then times W2q^T plus b2 (all float64 except the quantization)."""
    W1c, W1s, b1, W2c, W2s, b2 = eq
    u = xq @ dequantize(W1c, W1s).T
    if b1 is not None:
        u = u + moe_ref.widen(b1, kind)[None, :]
    hq = dequantize(*quantize(moe_ref.ACTIVATIONS[activation](u)))
    y = hq @ dequantize(W2c, W2s).T
    if b2 is not None:
        y = y + moe_ref.widen(b2, kind)[None, :]
    return y


def _no_ffn(experts_q, e, kind):
    """Shapes-only stand-in for the routing pass (its outputs are replaced)."""
    W1c, _, _, W2c, _, _ = experts_q(e)
    h, d = W1c.shape
    return (np.zeros((h, d)), None, np.zeros((d, h)), None)

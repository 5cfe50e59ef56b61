"""Pins of the MXFP8 oracle (oracle/mxfp8.py) against what the format's
definition and independent routines fix, and planted mistakes that a pin must
catch.  CPU only."""
import math
import os
import sys
import types

import numpy as np
import pytest

import oracle.mxfp8 as mx
from oracle import moe_ref

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "mxfp8.py")


def _brute_encode(v):
    """Nearest finite E4M3 value by exhaustive search over all 254 finite codes,
    ties to the even code, |v| > 448 clamped (an independent derivation)."""
    best, bd = None, math.inf
    a = min(abs(v), 448.0)
    for c in range(0x7F):
        m, e = c & 7, (c >> 3) & 15
        val = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        d = abs(val - a)
        if d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best | (0x80 if math.copysign(1.0, v) < 0 else 0)


def check_codec_table(m=None):
    m = m or mx
    vals = [m.e4m3_decode(c) for c in range(256)]
    assert sum(math.isnan(v) for v in vals) == 2 and math.isnan(vals[0x7F]) and math.isnan(vals[0xFF])
    assert vals[0x38] == 1.0 and vals[0x7E] == 448.0 and vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6
    assert vals[0xB8] == -1.0 and vals[0x36] == 0.875 and vals[0x00] == 0.0
    for c in range(256):
        if not math.isnan(vals[c]):
            assert m.e4m3_encode(vals[c]) == c, hex(c)          # round trip on every finite code


def check_encode_against_torch_and_brute(m=None):
    """In-range values agree with torch's float8_e4m3fn conversion (round to
    nearest even) and with the exhaustive search; the grid's midpoints test ties."""
    import torch
    m = m or mx
    rng = np.random.default_rng(20)
    pos = sorted(v for v in (m.e4m3_decode(c) for c in range(0x7F)))
    mids = [(a + b) / 2 for a, b in zip(pos, pos[1:])]
    xs = np.concatenate([rng.standard_normal(3000) * 40, rng.standard_normal(500) * 0.01, mids, -np.array(mids)])
    xs = xs[np.abs(xs) <= 448]
    ref = torch.tensor(xs, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([m.e4m3_encode(float(v)) for v in xs], dtype=np.uint8)
    brute = np.array([_brute_encode(float(v)) for v in xs], dtype=np.uint8)
    assert np.array_equal(ours, brute) and np.array_equal(ours, ref)
    assert m.e4m3_encode(449.0) == 0x7E and m.e4m3_encode(1e6) == 0x7E and m.e4m3_encode(-1e6) == 0xFE


def check_block_scale_rule(m=None):
    """OCP MX: X = 2^(floor(log2 amax) - 8) for E4M3 (its largest power of two
    is 2^8), so the block maximum lands in [256, 512) before rounding."""
    m = m or mx
    assert m.block_exponent(448.0) == 0 and m.block_exponent(256.0) == 0 and m.block_exponent(255.9) == -1
    assert m.block_exponent(1.0) == -8 and m.block_exponent(0.75) == -9 and m.block_exponent(2.0 ** -100) == -108
    assert m.block_exponent(0.0) == -127
    rng = np.random.default_rng(21)
    for amax in rng.uniform(1e-3, 1e3, 200):
        s = m.block_exponent(float(amax))
        assert 256.0 <= amax * 2.0 ** -s < 512.0


def check_quantize_roundtrip_and_bound(m=None):
    m = m or mx
    rng = np.random.default_rng(22)
    # values on the grid of a block whose largest element is a power of two >= 256 * 2^s: exact
    s = -5
    codes = rng.integers(0, 0x7E, (4, 64)).astype(np.uint8) | (rng.integers(0, 2, (4, 64)).astype(np.uint8) << 7)
    codes[:, 0] = 0x40 | (codes[:, 0] & 0x80)          # +-256 anchors the block maximum
    codes[:, 32] = 0x40
    vals = np.array([[m.e4m3_decode(int(c)) for c in row] for row in codes]) * 2.0 ** s
    qc, qs = m.quantize(vals)
    assert np.all(qs == s + 127) and np.array_equal(m.dequantize(qc, qs), vals)
    # error bound: half a unit in the last place of E4M3 relative to each element's binade,
    # except where the clamp at 448 applies (elements in [448, 512) X)
    a = rng.standard_normal((8, 256)) * np.exp(rng.standard_normal((8, 1)))
    qc, qs = m.quantize(a)
    dq = m.dequantize(qc, qs)
    X = np.repeat(2.0 ** (qs.astype(np.int64) - 127), 32, axis=1)
    y = a / X
    clamped = np.abs(y) > 448
    ulp = np.where(np.abs(y) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(dq - a)[~clamped] <= (ulp / 2 * X)[~clamped] * (1 + 1e-12))
    assert np.all(np.abs(dq[clamped]) == 448 * X[clamped])
    z, zs = m.quantize(np.zeros((2, 64)))
    assert np.all(zs == 0) and np.all(m.dequantize(z, zs) == 0)


def _brute_quantize_block(vals):
    """Scalar MXFP8 of one 32-element block from the definition: the exponent by
    repeated halving/doubling, the elements by exhaustive search."""
    amax = max(abs(v) for v in vals)
    if amax == 0:
        return [0] * 32, 0
    e = 0
    while 2.0 ** (e + 1) <= amax:
        e += 1
    while 2.0 ** e > amax:
        e -= 1
    s = e - 8
    return [_brute_encode(v / 2.0 ** s) for v in vals], s + 127


def check_quantize_against_brute(m=None):
    m = m or mx
    rng = np.random.default_rng(23)
    a = rng.standard_normal((3, 96)) * np.array([[1e-3], [1.0], [300.0]])
    qc, qs = m.quantize(a)
    for r in range(3):
        for b in range(3):
            codes, sc = _brute_quantize_block(list(a[r, 32 * b:32 * b + 32]))
            assert qc[r, 32 * b:32 * b + 32].tolist() == codes and int(qs[r, b]) == sc


def _layer_case(m, activation="gelu", bias=True, S=0):
    rng = np.random.default_rng(24)
    T, d, h, E, k = 40, 64, 96, 4, 2
    x = rng.standard_normal((T, d))
    W_g = rng.standard_normal((E, d))
    ex = []
    for _ in range(E + S):
        W1 = rng.standard_normal((h, d)) * 0.3
        W2 = rng.standard_normal((d, h)) * 0.3
        b1 = rng.standard_normal(h) * 0.1 if bias else None
        b2 = rng.standard_normal(d) * 0.1 if bias else None
        ex.append((W1, b1, W2, b2))
    exq = [(*m.quantize(W1), b1, *m.quantize(W2), b2) for (W1, b1, W2, b2) in ex]
    return x, W_g, ex, exq, E, k


def check_layer_properties(m=None):
    """The MXFP8 layer routes exactly like the plain one, and its output stays
    within a few E4M3 quantization steps of the plain layer's (three roundings
    of about 2^-4 relative each), without being equal to it."""
    m = m or mx
    for act, bias, S in [("gelu", True, 0), ("silu", False, 1)]:
        x, W_g, ex, exq, E, k = _layer_case(m, act, bias, S)
        r = m.moe_forward_mxfp8_ref(x, W_g, lambda e: exq[e], E, k, 0.0, S, kind="f64", activation=act)
        p = moe_ref.moe_forward_ref(x, W_g, lambda e: ex[e], E, k, 0.0, S, kind="f64", activation=act)
        assert r.idx.tolist() == p.idx.tolist() and np.allclose(r.w, p.w, rtol=0, atol=0)
        rel = np.max(np.abs(r.out - p.out)) / np.max(np.abs(p.out))
        assert 1e-4 < rel < 0.15, rel


def check_layer_against_scalar_brute(m=None):
    """One token through one expert, scalar loops from the definition."""
    m = m or mx
    x, W_g, ex, exq, E, k = _layer_case(m)
    W1, b1, W2, b2 = ex[0]
    W1c, W1s, _, W2c, W2s, _ = exq[0]
    dq = lambda c, s: m.e4m3_decode(int(c)) * 2.0 ** (int(s) - 127)
    xt = x[3]
    xc, xs = [], []
    for b in range(2):
        cc, ss = _brute_quantize_block(list(xt[32 * b:32 * b + 32]))
        xc += cc
        xs.append(ss)
    xq = [m.e4m3_decode(xc[i]) * 2.0 ** (xs[i // 32] - 127) for i in range(64)]
    u = [sum(xq[i] * dq(W1c[j, i], W1s[j, i // 32]) for i in range(64)) + b1[j] for j in range(96)]
    g = [0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in u]
    hc, hs = [], []
    for b in range(3):
        cc, ss = _brute_quantize_block(g[32 * b:32 * b + 32])
        hc += cc
        hs.append(ss)
    hq = [m.e4m3_decode(hc[i]) * 2.0 ** (hs[i // 32] - 127) for i in range(96)]
    y = [sum(hq[j] * dq(W2c[c, j], W2s[c, j // 32]) for j in range(96)) + b2[c] for c in range(64)]
    got = m.expert_ffn_mxfp8(m.dequantize(*m.quantize(x[3:4])), exq[0], "f64", "gelu")[0]
    assert np.allclose(got, y, rtol=0, atol=1e-12)
    # and through the layer: token 3's output is its routing weights times the
    # scalar expert outputs (the quantization of x happens inside the layer)
    r = m.moe_forward_mxfp8_ref(x, W_g, lambda e: exq[e], E, k, kind="f64", rows=[3])
    want = np.zeros(64)
    for j in range(k):
        e = int(r.idx[3, j])
        W1c, W1s, b1e, W2c, W2s, b2e = exq[e]
        u = [sum(xq[i] * dq(W1c[jj, i], W1s[jj, i // 32]) for i in range(64)) + b1e[jj] for jj in range(96)]
        g = [0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in u]
        hc, hs = [], []
        for b in range(3):
            cc, ss = _brute_quantize_block(g[32 * b:32 * b + 32])
            hc += cc
            hs.append(ss)
        hq = [m.e4m3_decode(hc[i]) * 2.0 ** (hs[i // 32] - 127) for i in range(96)]
        want += r.w[3, j] * np.array([sum(hq[jj] * dq(W2c[c, jj], W2s[c, jj // 32]) for jj in range(96)) + b2e[c]
                                      for c in range(64)])
    assert np.allclose(r.out[0], want, rtol=0, atol=1e-12)


def check_array_encoder_matches_scalar(m=None):
    m = m or mx
    pos = sorted(v for v in (m.e4m3_decode(c) for c in range(0x7F)))
    mids = [(a + b) / 2 for a, b in zip(pos, pos[1:])]
    rng = np.random.default_rng(25)
    y = np.concatenate([mids, -np.array(mids), pos, rng.standard_normal(2000) * 100, [500.0, -1e9, 0.0, -0.0]])
    assert m._encode_array(y).tolist() == [m.e4m3_encode(float(v)) for v in y]


CHECKS = [check_array_encoder_matches_scalar, check_codec_table, check_encode_against_torch_and_brute, check_block_scale_rule,
          check_quantize_roundtrip_and_bound, check_quantize_against_brute, check_layer_properties,
          check_layer_against_scalar_brute]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_pin(check):
    check()


MUTANTS = [
    ("emax_7", "E4M3_EMAX = 8 ", "E4M3_EMAX = 7 "),
    ("emax_9", "E4M3_EMAX = 8 ", "E4M3_EMAX = 9 "),
    ("ceil_log2", "return max(-E8M0_BIAS, min(E8M0_BIAS, (e - 1) - E4M3_EMAX))",
     "return max(-E8M0_BIAS, min(E8M0_BIAS, e - E4M3_EMAX))"),
    ("no_clamp", "a = min(abs(v), E4M3_MAX)", "a = abs(v)"),
    ("ties_to_lower", "if dlo < dhi or (dlo == dhi and int(_POS_CODES[lo]) % 2 == 0):", "if dlo <= dhi:"),
    ("ties_to_upper", "if dlo < dhi or (dlo == dhi and int(_POS_CODES[lo]) % 2 == 0):", "if dlo < dhi:"),
    ("scale_sign", "y = np.ldexp(blocks, -s[:, :, None]).reshape(R, K)", "y = np.ldexp(blocks, s[:, :, None]).reshape(R, K)"),
    ("array_ties_to_lower", "pick_lo = (dlo < dhi) | ((dlo == dhi) & (_POS_CODES[lo] % 2 == 0))", "pick_lo = dlo <= dhi"),
    ("array_sign_dropped", "sign = np.where(np.signbit(y), 0x80, 0).astype(np.uint8)",
     "sign = np.zeros(y.shape, dtype=np.uint8)"),
    ("array_ceil_log2", "s = np.where(amax > 0, np.clip((e - 1) - E4M3_EMAX, -E8M0_BIAS, E8M0_BIAS), -E8M0_BIAS)",
     "s = np.where(amax > 0, np.clip(e - E4M3_EMAX, -E8M0_BIAS, E8M0_BIAS), -E8M0_BIAS)"),
    ("block_16", "BLOCK = 32", "BLOCK = 16"),
    ("bias_126", "E8M0_BIAS = 127", "E8M0_BIAS = 126"),
    ("subnormal_exp", "v = math.ldexp(m / 8.0, -6) if e == 0", "v = math.ldexp(m / 8.0, -7) if e == 0"),
    ("h_not_quantized", "hq = dequantize(*quantize(moe_ref.ACTIVATIONS[activation](u)))",
     "hq = moe_ref.ACTIVATIONS[activation](u)"),
    ("x_not_quantized", "xq = dequantize(*quantize(xf))", "xq = xf"),
]


def _mutant(old, new, monkeypatch):
    src = open(SRC_PATH, encoding="utf-8").read()
    assert src.count(old) == 1, old
    name = "oracle.mxfp8_mutant"
    mod = types.ModuleType(name)
    mod.__dict__["__name__"] = name
    mod.__dict__["__package__"] = "oracle"
    monkeypatch.setitem(sys.modules, name, mod)
    exec(compile(src.replace(old, new), name, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, monkeypatch):
    mod = _mutant(old, new, monkeypatch)
    caught = False
    for check in CHECKS:
        try:
            check(mod)
        except Exception:
            caught = True
            break
    assert caught, f"mutant {name} passed every pin"

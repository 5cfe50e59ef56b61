"""The seeded workload generator: deterministic per seed, per-expert streams,
shapes and bfloat16 rounding (round to nearest, ties to even)."""
import numpy as np

from synthetic import CONFIGS, f32_to_bf16_bits, make_inputs


def test_deterministic_and_per_expert():
    a = make_inputs("tiny", seed=0)
    b = make_inputs("tiny", seed=0)
    c = make_inputs("tiny", seed=1)
    assert np.array_equal(a.x, b.x) and not np.array_equal(a.x, c.x)
    for e in range(4):
        for u, v in zip(a.expert(e), b.expert(e)):
            assert np.array_equal(u, v)
    assert not np.array_equal(a.expert(0)[0], a.expert(1)[0])
    W1, b1, W2, b2 = a.stacked()
    assert np.array_equal(W1[2], a.expert(2)[0]) and np.array_equal(W2[3], a.expert(3)[2])
    assert not b1.any() and not b2.any()             # tiny: zero biases


def test_shapes():
    for name, cfg in CONFIGS.items():
        inp = make_inputs(cfg.replace(T=16, d=16, h=32) if cfg.T > 64 else cfg)
        c = inp.cfg
        assert inp.x.shape == (c.T, c.d) and inp.W_g.shape == (c.E, c.d)
        W1, b1, W2, b2 = inp.expert(0)
        assert W1.shape == (c.h, c.d) and W2.shape == (c.d, c.h) and b1.shape == (c.h,) and b2.shape == (c.d,)
        assert inp.x.dtype == (np.uint16 if c.dtype == "bf16" else np.float32)
        assert (inp.b_g is not None) == (name == "glam")


def test_bf16_rounding():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 0.0], dtype=np.float32)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6... i.e. mantissa 0x02)
    assert f32_to_bf16_bits(f).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000]

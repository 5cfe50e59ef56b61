"""Expert-choice routing on the GPU vs the CPU oracle, through the C ABI.

Reduced shapes (the oracle computes every output) cover every GEMM tile
height, the split tail, the float32 SIMT path, shared experts, C = 1 and
C = T (the dense limit), E = 256, a skewed router with untaken tokens, the
Mixtral expert form and exact ties between duplicate tokens; two workloads run
at full size with C = ceil(k T / E) (the same expert rows as their top-k
routing) and the oracle computing every output row.
"""
import math
import sys

import numpy as np
import pytest

from synthetic import CONFIGS, make_inputs
from tests.parity import compare_ec, run_gpu_ec

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mixture_experts_28_amd  # noqa: F401  (fails loudly if libmoe.so is missing)
    yield


def _C(cfg, per_token):
    return min(cfg.T, math.ceil(per_token * cfg.T / cfg.E))


# name: (base workload, overrides, tokens per expert as a multiple of T / E, or an int C)
REDUCED = {
    "ec_bm256": ("mixtral", dict(T=2100, d=256, h=512, E=4), 2.0),
    "ec_T600": ("mixtral", dict(T=600, d=512, h=1024), 2.0),
    "ec_fine_shared": ("deepseek", dict(T=512, d=256, h=512, E=32, S=1), 8.0),
    "ec_skewed_untaken": ("glam", dict(T=1000, d=256, h=512, E=16), 2.0),
    "ec_tail_split_deep_K": ("mixtral", dict(T=512, d=2048, h=512, E=4), 2.0),
    "ec_f32_shared": ("switch", dict(T=500, d=64, h=128, E=8, S=1), 1.6),
    "ec_tiny": ("tiny", {}, 2.0),
    "ec_dense_C_eq_T": ("mixtral", dict(T=130, d=256, h=256, E=4), 4.0),
    "ec_C1": ("glam", dict(T=300, d=256, h=256, E=8), 1),
    "ec_E256": ("deepseek", dict(T=128, d=256, h=256, E=256, S=0), 8.0),
    "ec_silu_nobias": ("mixtral", dict(T=600, d=512, h=1024, activation="silu", expert_bias=False), 2.0),
    "ec_single_token": ("mixtral", dict(T=1, d=256, h=256, E=8), 1),
    "ec_d32_bf16_simt": ("mixtral", dict(T=100, d=32, h=64, E=6), 3.0),
}


def _run(inp, C, rows=None):
    stacked = inp.stacked()
    gpu = run_gpu_ec(inp, C, stacked=stacked)
    return gpu, compare_ec(inp, C, gpu, stacked=stacked, rows=rows)


@pytest.mark.parametrize("case", sorted(REDUCED))
def test_ec_reduced_full_oracle(case):
    base, kw, per = REDUCED[case]
    inp = make_inputs(CONFIGS[base].replace(name=case, **kw) if kw else CONFIGS[base], seed=0)
    c = inp.cfg
    C = per if isinstance(per, int) else _C(c, per)
    _say(f"[ec] {case}: T={c.T} d={c.d} h={c.h} E={c.E} C={C} S={c.S} {c.activation} bias={c.expert_bias} {c.dtype}")
    _, rep = _run(inp, C)
    _say(f"[ec] {case}: {rep}")


def test_ec_duplicate_tokens_tie_to_lower_index():
    """Tokens 10..19 repeat tokens 0..9 exactly, so every column has exact
    ties; the lower token index wins them on the GPU as in the oracle."""
    inp = make_inputs(CONFIGS["mixtral"].replace(name="ec_dup", T=200, d=256, h=256, E=8), seed=3)
    x = inp.x.copy()
    x[10:20] = x[0:10]
    x[150:200] = x[100:150]
    inp._x = x
    _say("[ec] duplicate tokens")
    gpu, rep = _run(inp, 40)
    _say(f"[ec] duplicate tokens: {rep}")


def test_ec_deterministic_bitwise():
    inp = make_inputs(CONFIGS["glam"].replace(name="ec_det", T=700, d=256, h=512, E=16), seed=0)
    stacked = inp.stacked()
    _say("[ec] determinism: two calls")
    a = run_gpu_ec(inp, 88, stacked=stacked)
    b = run_gpu_ec(inp, 88, stacked=stacked)
    for key in ("out", "tok", "w"):
        assert np.array_equal(a[key], b[key]), key
    assert a["aux"] == b["aux"] and a["z"] == b["z"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral", "glam"])
def test_ec_full_size(name):
    inp = make_inputs(name, seed=0)
    c = inp.cfg
    C = _C(c, c.k)
    _say(f"[ec-full] {name}: T={c.T} d={c.d} h={c.h} E={c.E} C={C} {c.dtype}")
    gpu, rep = _run(inp, C, rows=None)
    # every expert holds exactly C distinct tokens, on every expert
    assert all(len(set(r.tolist())) == C for r in gpu["tok"])
    _say(f"[ec-full] {name}: {rep}")


def test_ec_constant_column_takes_lowest_indices():
    """Expert 0's router row is zero, so all its logits are equal: its bucket
    holds every token (more than the directly ranked 1024), the exact radix
    path runs, and every tie goes to the lower token index: tokens 0..C-1."""
    inp = make_inputs(CONFIGS["mixtral"].replace(name="ec_const", T=3000, d=256, h=256, E=8), seed=1)
    W_g = inp.W_g.copy()
    W_g[0] = 0
    inp._wg = W_g
    C = 700
    _say("[ec] constant column (radix path)")
    gpu, rep = _run(inp, C)
    assert gpu["tok"][0].tolist() == list(range(C))
    _say(f"[ec] constant column: {rep}")


def test_ec_long_column_unstaged():
    """T above the 16384 tokens staged in LDS: the column is read from L2."""
    inp = make_inputs(CONFIGS["mixtral"].replace(name="ec_long", T=20000, d=256, h=256, E=8), seed=2)
    C = _C(inp.cfg, 2.0)
    _say(f"[ec] long column T=20000 C={C}")
    gpu, rep = _run(inp, C, rows=None)
    _say(f"[ec] long column: {rep}")

"""The parity comparison itself, on the CPU: results built from the oracle pass,
and planted discrepancies (a wrong count, a shifted slot, a wrong expert, an
output, aux or z-loss off by more than the tolerance, a near-tie resolved the
other way) are judged as the rules say."""
import numpy as np
import pytest

from synthetic import CONFIGS, make_inputs
from tests.parity import compare, compare_ec, oracle_ec_for, oracle_for


def fake_gpu(r, dtype):
    out = r.out.astype(np.float32).astype(np.float64)
    return dict(out=out, idx=r.idx.copy(), w=r.w.astype(np.float32).astype(np.float64), aux=float(np.float32(r.aux)),
                z=float(np.float32(r.z)), counts=r.counts.copy(), kept=r.kept.copy(), slot_pos=r.slot_pos.copy())


@pytest.fixture(scope="module")
def case():
    inp = make_inputs(CONFIGS["switch"].replace(T=300, d=32, h=64, E=8, k=2, cf=0.5), seed=3)
    stacked = inp.stacked()
    return inp, stacked, oracle_for(inp, stacked)


def test_oracle_results_pass(case):
    inp, stacked, r = case
    rep = compare(inp, fake_gpu(r, "f32"), stacked=stacked)
    assert rep["dropped"] > 0 and not rep["rerun"]


@pytest.mark.parametrize("what", ["counts", "kept", "slot", "expert", "out", "aux", "z", "weight", "order"])
def test_discrepancy_fails(case, what):
    inp, stacked, r = case
    g = fake_gpu(r, "f32")
    if what == "counts":
        g["counts"][0] += 1
    elif what == "kept":
        g["kept"][1] -= 1
    elif what == "slot":
        i = np.argwhere(g["slot_pos"] >= 0)[5]
        g["slot_pos"][tuple(i)] += 1
    elif what == "expert":
        t = int(np.nonzero(~r.tie_flag)[0][3])
        g["idx"][t, 1] = next(e for e in range(8) if e not in g["idx"][t])
    elif what == "out":
        g["out"][7, 3] += 2e-5 * np.abs(r.out).max()
    elif what == "aux":
        g["aux"] += 2e-5
    elif what == "z":
        g["z"] += 2e-5 * max(1.0, r.z)
    elif what == "weight":
        g["w"][4, 0] += 2e-5
    elif what == "order":
        t = int(np.nonzero(~r.order_flag)[0][0])
        g["idx"][t] = g["idx"][t][::-1]
        g["w"][t] = g["w"][t][::-1]
        g["slot_pos"][t] = g["slot_pos"][t][::-1]
    with pytest.raises(AssertionError):
        compare(inp, g, stacked=stacked)


def test_near_tie_resolved_the_other_way_is_accepted():
    """Build a token whose 2nd and 3rd logits tie exactly; a GPU that picks the
    other expert passes through the conditioned re-run."""
    inp = make_inputs(CONFIGS["tiny"].replace(T=16, d=8, h=16, E=4, k=2), seed=5)
    inp.W_g  # materialise
    x = inp.x.copy()
    Wg = inp.W_g.copy()
    Wg[3] = Wg[2]                       # experts 2 and 3 have identical router rows
    inp._wg = Wg
    stacked = inp.stacked()
    r = oracle_for(inp, stacked)
    t = int(np.nonzero(r.tie_flag)[0][0])
    g_idx = r.idx.copy()
    row = list(g_idx[t])
    if 2 in row:
        row[row.index(2)] = 3
    else:
        row[row.index(3)] = 2
    g_idx[t] = row
    r2 = oracle_for(inp, stacked, override_idx=g_idx)
    g = fake_gpu(r2, "f32")
    rep = compare(inp, g, stacked=stacked)
    assert rep["rerun"] and rep["flagged"] >= 1
    del x


# ------------------------------------------------------------ expert choice --
def fake_gpu_ec(r):
    return dict(out=r.out.astype(np.float32).astype(np.float64), tok=r.tok.copy(),
                w=r.w.astype(np.float32).astype(np.float64), aux=float(np.float32(r.aux)), z=float(np.float32(r.z)))


@pytest.fixture(scope="module")
def case_ec():
    inp = make_inputs(CONFIGS["switch"].replace(T=200, d=32, h=64, E=8, k=1, S=1), seed=4)
    stacked = inp.stacked()
    return inp, stacked, oracle_ec_for(inp, 30, stacked)


def test_ec_oracle_results_pass(case_ec):
    inp, stacked, r = case_ec
    rep = compare_ec(inp, 30, fake_gpu_ec(r), stacked=stacked)
    assert not rep["rerun"] and rep["untaken"] > 0


@pytest.mark.parametrize("what", ["token", "order", "weight", "out", "aux", "z"])
def test_ec_discrepancy_fails(case_ec, what):
    inp, stacked, r = case_ec
    g = fake_gpu_ec(r)
    if what == "token":
        e = int(np.nonzero(~r.flag)[0][0])
        spare = next(t for t in range(inp.cfg.T) if t not in g["tok"][e])
        row = sorted(list(g["tok"][e][:-1]) + [spare])
        g["tok"][e] = row
    elif what == "order":
        g["tok"][2] = g["tok"][2][::-1]
    elif what == "weight":
        g["w"][3, 5] += 2e-5
    elif what == "out":
        g["out"][11, 4] += 2e-5 * np.abs(r.out).max()
    elif what == "aux":
        g["aux"] += 2e-5
    elif what == "z":
        g["z"] += 2e-5 * max(1.0, r.z)
    with pytest.raises(AssertionError):
        compare_ec(inp, 30, g, stacked=stacked)


def test_ec_near_tie_resolved_the_other_way_is_accepted():
    """Two tokens with identical rows tie in every column; a GPU that takes
    the later one of a tied pair at an expert's boundary passes through the
    conditioned re-run."""
    inp = make_inputs(CONFIGS["tiny"].replace(T=16, d=8, h=16, E=4, k=1), seed=6)
    x = inp.x.copy()
    r0 = oracle_ec_for(inp, 4)
    e = 0
    order = np.argsort(-r0.logits[:, e], kind="stable")
    a_, b_ = int(order[3]), int(order[4])           # the 4th and 5th best of expert 0
    x[b_] = x[a_]                                     # now they tie exactly
    inp._x = x
    stacked = inp.stacked()
    r = oracle_ec_for(inp, 4, stacked)
    assert r.flag[e]
    g_tok = r.tok.copy()
    lo, hi = min(a_, b_), max(a_, b_)
    assert lo in g_tok[e] and hi not in g_tok[e]
    g_tok[e] = np.sort([t if t != lo else hi for t in g_tok[e]])
    r2 = oracle_ec_for(inp, 4, stacked, override_tok=g_tok)
    rep = compare_ec(inp, 4, fake_gpu_ec(r2), stacked=stacked)
    assert rep["rerun"] and rep["flagged"] >= 1

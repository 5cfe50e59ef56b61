"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of the pages prints a worked numeric example of the layer, so the
oracle is pinned by: hand-derived closed-form fixtures (tests/golden, each
citing the passage it follows), brute force on tiny inputs (oracle.brute,
an independent scalar derivation), library routines (torch CPU float64
topk / gelu / linear), closed forms of the balance loss, capacity
invariants, and symmetry properties of the combine.  Each check is a plain
function so ``test_oracle_mutants`` can plant mistakes in the oracle and
show that some pin catches every one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle.moe_ref as ref
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ helpers --
def rand_case(rng, T, d, h, E, k, S=0, wscale=1.0, bias=True):
    x = rng.standard_normal((T, d))
    W_g = rng.standard_normal((E, d)) * wscale
    experts = []
    for _ in range(E + S):
        W1 = rng.standard_normal((h, d)) * 0.5
        b1 = rng.standard_normal(h) * 0.3 if bias else np.zeros(h)
        W2 = rng.standard_normal((d, h)) * 0.5
        b2 = rng.standard_normal(d) * 0.3 if bias else np.zeros(d)
        experts.append((W1, b1, W2, b2))
    return x, W_g, experts


def run_ref(x, W_g, experts, E, k, cf=0.0, S=0, b_g=None, **kw):
    return ref.moe_forward_ref(x, W_g, lambda e: experts[e], E, k, cf, S, b_g, kind="f64", **kw)


def to_lists(a):
    return [list(map(float, r)) for r in np.asarray(a)]


def brute_case(x, W_g, experts, k, cap=None, S=0, b_g=None, activation="gelu"):
    vec = lambda b: None if b is None else list(map(float, b))
    ex = [(to_lists(W1), vec(b1), to_lists(W2), vec(b2)) for (W1, b1, W2, b2) in experts]
    return brute.brute_layer(to_lists(x), to_lists(W_g), ex, k, cap=cap, n_shared=S,
                             b_g=vec(b_g), activation=activation)


def ffn_torch(xr, W1, b1, W2, b2):
    """Library-routine expert FFN: torch CPU float64 linear + exact GELU."""
    import torch
    import torch.nn.functional as F
    t = lambda a: torch.as_tensor(np.asarray(a), dtype=torch.float64)
    u = F.linear(t(xr), t(W1), t(b1))
    return F.linear(F.gelu(u, approximate="none"), t(W2), t(b2)).numpy()


# --------------------------------------------------------------- checks --
def check_weights_sum_to_one():
    """Renormalised top-k weights sum to 1 per token ([guide] §3.1 comment on the
    renormalisation; §4.1 diagram 0.6 + 0.4); k = 1 gives weight 1 exactly."""
    rng = np.random.default_rng(1)
    for (T, d, E, k) in [(50, 8, 6, 2), (40, 5, 7, 3), (30, 4, 4, 1), (20, 6, 9, 9)]:
        x, W_g, ex = rand_case(rng, T, d, 3, E, k)
        r = run_ref(x, W_g, ex, E, k)
        assert np.allclose(r.w.sum(1), 1.0, atol=1e-12, rtol=0)
        assert np.all(r.w > 0)
        if k == 1:
            assert np.all(r.w == 1.0)
        # weights follow the selection order (descending logits)
        assert np.all(np.diff(r.w, axis=1) <= 1e-15)


def check_against_brute():
    """Oracle == brute force (subset enumeration, explicit queues, scalar loops)."""
    rng = np.random.default_rng(2)
    cases = [(6, 4, 3, 4, 2, 0, None), (8, 3, 2, 5, 3, 0, None), (7, 2, 4, 3, 1, 0, 0.5),
             (8, 3, 3, 5, 2, 1, 1.0), (5, 4, 2, 2, 2, 2, None), (8, 2, 3, 4, 2, 0, 0.5),
             (8, 3, 2, 5, 1, 0, 1.0), (4, 3, 3, 3, 3, 1, 0.5)]
    for (T, d, h, E, k, S, cf) in cases:
        for trial in range(3):
            x, W_g, ex = rand_case(rng, T, d, h, E, k, S)
            b_g = rng.standard_normal(E) if trial == 2 else None
            r = run_ref(x, W_g, ex, E, k, cf or 0.0, S, b_g)
            assert not r.tie_flag.any()
            cap = None if not cf else int(math.ceil(cf * T / E))
            b = brute_case(x, W_g, ex, k, cap=cap, S=S, b_g=b_g)
            assert r.idx.tolist() == b["idx"]
            assert np.allclose(r.w, np.array(b["w"]), rtol=0, atol=1e-13)
            assert r.counts.tolist() == b["counts"]
            assert r.kept.tolist() == b["kept"]
            assert (r.counts - r.kept).tolist() == b["dropped"]
            assert r.slot_kept.tolist() == b["slot_kept"]
            assert abs(r.aux - b["aux"]) < 1e-13
            assert abs(r.z - b["z"]) < 1e-12
            assert np.allclose(r.out, np.array(b["out"]), rtol=0, atol=1e-11)


def check_topk_vs_torch():
    """The top-k set and order equal torch.topk (CPU float64) on unflagged tokens."""
    import torch
    rng = np.random.default_rng(3)
    for (T, d, E, k) in [(300, 16, 8, 2), (200, 32, 64, 1), (100, 24, 256, 8), (64, 8, 5, 5)]:
        x, W_g, _ = rand_case(rng, T, d, 2, E, k)
        l = ref.router_logits(x, W_g)
        sel = ref.select_topk(l, k)
        v, i = torch.topk(torch.as_tensor(l), k, dim=1)
        i = i.numpy()
        for t in range(T):
            if sel.tie_flag[t]:
                continue
            assert set(sel.idx[t]) == set(i[t])
            if not sel.order_flag[t]:
                assert list(sel.idx[t]) == list(i[t])


def check_tie_rule():
    """Exact ties go to the lower expert index and are flagged."""
    l = np.array([[1.0, 2.0, 2.0, 0.5], [3.0, 3.0, 3.0, 3.0], [0.0, 5.0, 1.0, 1.0 + 2e-7]])
    sel = ref.select_topk(l, 2)
    assert sel.idx.tolist() == [[1, 2], [0, 1], [1, 3]]
    assert sel.tie_flag.tolist() == [False, True, True]
    assert sel.order_flag.tolist() == [True, True, False]
    assert ref.is_valid_topk(l[1], [2, 3]) and ref.is_valid_topk(l[2], [1, 2])
    assert not ref.is_valid_topk(l[0], [0, 1]) and not ref.is_valid_topk(l[0], [1, 1])


def check_dense_limit():
    """k = E without capacity: out = sum_e softmax(l)_e FFN_e(x) ([ch7] §7.1),
    computed here with no top-k and no permutation, through torch library calls."""
    rng = np.random.default_rng(4)
    for (T, d, h, E) in [(20, 6, 10, 4), (9, 3, 5, 7)]:
        x, W_g, ex = rand_case(rng, T, d, h, E, E)
        r = run_ref(x, W_g, ex, E, E)
        l = x @ W_g.T
        p = np.exp(l - l.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        dense = sum(p[:, e:e + 1] * ffn_torch(x, *ex[e]) for e in range(E))
        assert np.allclose(r.out, dense, rtol=0, atol=1e-12)


def check_aux_closed_forms():
    """Balance loss E sum f P ([guide] §4.3, [ch7] §7.4) on closed-form cases."""
    rng = np.random.default_rng(5)
    # (i) zero router: P uniform (1/E) so aux = E * sum f / E = 1, whatever the routing
    for (E, k) in [(8, 2), (5, 1), (64, 1), (6, 3)]:
        x = rng.standard_normal((40, 4))
        r = run_ref(x, np.zeros((E, 4)), [(np.zeros((2, 4)), np.zeros(2), np.zeros((4, 2)), np.zeros(4))] * E, E, k)
        assert abs(r.aux - 1.0) < 1e-14
        assert r.idx[:, 0].tolist() == [0] * 40      # everyone ties -> lowest indices
    # (ii) cyclic one-hot tokens and a circulant router W_g[e, c] = a[(e - c) mod E]
    # with a strictly decreasing: token c picks experts c, c+1, .., c+k-1 (mod E),
    # so f is uniform, and P_e averages every rotation of softmax(a), so P is uniform
    for (E, k, m) in [(4, 1, 3), (6, 2, 2), (8, 3, 1)]:
        x = np.tile(np.eye(E), (m, 1))
        a = 3.0 - 0.5 * np.arange(E)
        W_g = np.array([[a[(e - c) % E] for c in range(E)] for e in range(E)])
        ex = [(np.zeros((2, E)), np.zeros(2), np.zeros((E, 2)), np.zeros(E))] * E
        r = run_ref(x, W_g, ex, E, k)
        assert np.allclose(r.f, 1.0 / E) and np.allclose(r.P, 1.0 / E)
        assert abs(r.aux - 1.0) < 1e-14
    # (iii) every token to expert 0 with p -> 1: aux -> E (k = 1)
    E = 8
    x = np.ones((10, 1))
    W_g = np.array([[60.0]] + [[0.0]] * (E - 1))
    ex = [(np.zeros((2, 1)), np.zeros(2), np.zeros((1, 2)), np.zeros(1))] * E
    r = run_ref(x, W_g, ex, E, 1)
    assert abs(r.aux - E) < 1e-9
    # (iv) the definition: aux = E * sum_e (c_e / (T k)) * mean_t p[t, e], by explicit loops
    x, W_g, ex = rand_case(rng, 30, 5, 2, 6, 2)
    r = run_ref(x, W_g, ex, 6, 2)
    c = [sum(1 for t in range(30) for j in range(2) if r.idx[t, j] == e) for e in range(6)]
    Pm = [math.fsum(r.probs[t, e] for t in range(30)) / 30 for e in range(6)]
    assert abs(r.aux - 6 * math.fsum(c[e] / 60 * Pm[e] for e in range(6))) < 1e-14
    # (v) f uniform gives exactly 1 whatever P is; a skewed f can push it above 1
    ex = [(np.zeros((2, 2)), np.zeros(2), np.zeros((2, 2)), np.zeros(2))] * 2
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    W_g = np.array([[2.0, 0.0], [0.0, 0.1]])
    r = run_ref(x, W_g, ex[:2], 2, 1)
    assert r.counts.tolist() == [1, 1] and abs(r.aux - 1.0) < 1e-14   # f uniform -> exactly 1
    W_g = np.array([[2.0, -1.0], [0.0, 0.0]])
    r = run_ref(np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 1.0]]), W_g, ex[:2], 2, 1)
    f = np.array([2 / 3, 1 / 3])
    assert np.allclose(r.f, f) and abs(r.aux - 2 * np.dot(f, r.P)) < 1e-14 and r.aux > 1.0
    # (vi) and it can fall below 1: each token nearly ties its choice with expert 2,
    # which no token picks, so f = (1/2, 1/2, 0) while P ~ (1/4, 1/4, 1/2): aux ~ 3/4
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    W_g = np.array([[0.0, -30.0], [-30.0, 0.0], [-0.01, -0.01]])
    ex3 = [(np.zeros((2, 2)), np.zeros(2), np.zeros((2, 2)), np.zeros(2))] * 3
    r = run_ref(x, W_g, ex3, 3, 1)
    assert r.idx[:, 0].tolist() == [0, 1]
    assert abs(r.aux - 3 * (0.5 * r.P[0] + 0.5 * r.P[1])) < 1e-14 and 0.74 < r.aux < 0.76


def check_capacity():
    """Capacity = ceil(cf T / E) counted in tokens ([guide] §8.2; [ch7] §7.4);
    drops in token order; invariants and brute-force queues."""
    assert ref.capacity_of(1.25, 4096, 64) == 80     # switch-shaped workload
    assert ref.capacity_of(1.5, 16384, 64) == 384    # glam-shaped workload
    assert ref.capacity_of(1.0, 6, 4) == 2           # ceil(1.5)
    assert ref.capacity_of(0.0, 10, 2) is None and ref.capacity_of(-1.0, 10, 2) is None
    rng = np.random.default_rng(6)
    for (T, E, k) in [(60, 5, 2), (80, 8, 1), (50, 4, 3)]:
        x, W_g, ex = rand_case(rng, T, 4, 2, E, k)
        W_g[0] += 1.5                          # skew toward expert 0 so caps bind
        prev = None
        for cf in [0.1, 0.25, 0.5, 1.0, 2.0, float(E)]:
            r = run_ref(x, W_g, ex, E, k, cf)
            cap = ref.capacity_of(cf, T, E)
            assert r.kept.sum() + (r.counts - r.kept).sum() == T * k
            assert np.all(r.kept <= cap) and np.all(r.kept == np.minimum(r.counts, cap))
            assert r.slot_kept.sum() == r.kept.sum()
            if prev is not None:
                assert np.all(r.kept >= prev)                          # monotone in cf
                assert np.all(r.slot_kept[prev_mask])                  # kept sets grow
            prev, prev_mask = r.kept, r.slot_kept
            if cf >= E:
                assert r.slot_kept.all()                               # cap >= T
            # the kept assignments of an expert are its first ``cap`` tokens
            for e in range(E):
                toks = [t for t in range(T) for j in range(k) if r.idx[t, j] == e]
                kept_toks = [t for t in range(T) for j in range(k) if r.idx[t, j] == e and r.slot_kept[t, j]]
                assert kept_toks == toks[:cap]
            # slot_pos: contiguous per-expert segments in expert order
            pos = np.sort(r.slot_pos[r.slot_kept])
            assert pos.tolist() == list(range(int(r.kept.sum())))
        # cap = 1: each expert keeps only its first token
        r = run_ref(x, W_g, ex, E, k, 0.5 * E / T)
        assert r.cap == 1 and np.all(r.kept == np.minimum(r.counts, 1))
        for e in range(E):
            first = [t for t in range(T) if e in r.idx[t]][:1]
            assert [t for t in range(T) for j in range(k) if r.idx[t, j] == e and r.slot_kept[t, j]] == first


def check_dropped_contribute_nothing():
    """A dropped assignment adds nothing and the others are not renormalised."""
    rng = np.random.default_rng(7)
    x, W_g, ex = rand_case(rng, 40, 4, 3, 4, 2)
    W_g[1] += 2.0
    full = run_ref(x, W_g, ex, 4, 2)
    r = run_ref(x, W_g, ex, 4, 2, 0.5)
    assert (~r.slot_kept).any()
    for t in range(40):
        acc = np.zeros(4)
        for j in range(2):
            if r.slot_kept[t, j]:
                acc += full.w[t, j] * ffn_torch(x[t:t + 1], *ex[full.idx[t, j]])[0]
        assert np.allclose(r.out[t], acc, rtol=0, atol=1e-12)


def check_ffn_library():
    """Expert FFN == torch F.linear + F.gelu(approximate='none') in float64, and
    GELU == u * Phi(u) from math.erf."""
    rng = np.random.default_rng(8)
    W1, b1, W2, b2 = (rng.standard_normal(s) for s in [(12, 5), 12, (5, 12), 5])
    xr = rng.standard_normal((7, 5))
    assert np.allclose(ref.expert_ffn(xr, W1, b1, W2, b2), ffn_torch(xr, W1, b1, W2, b2), rtol=0, atol=1e-13)
    for u in [-3.0, -1.0, -0.1, 0.0, 0.3, 1.0, 2.5]:
        assert abs(float(ref.gelu(np.array([u]))[0]) - u * 0.5 * (1 + math.erf(u / math.sqrt(2)))) < 1e-15


def check_combine_symmetries():
    """Identical experts; relabelling experts; permuting tokens."""
    rng = np.random.default_rng(9)
    T, d, h, E, k = 32, 5, 7, 6, 2
    x, W_g, ex = rand_case(rng, T, d, h, E, k)
    same = [ex[0]] * E
    y = ffn_torch(x, *ex[0])
    r = run_ref(x, W_g, same, E, k)
    assert np.allclose(r.out, y, rtol=0, atol=1e-12)                     # sum of weights is 1
    r = run_ref(x, W_g, same, E, k, 0.5)
    kept_w = (r.w * r.slot_kept).sum(1, keepdims=True)
    assert np.allclose(r.out, kept_w * y, rtol=0, atol=1e-12)            # drops: kept weight only
    # relabel experts: permute router rows and expert params together
    perm = rng.permutation(E)
    r0 = run_ref(x, W_g, ex, E, k)
    r1 = run_ref(x, W_g[perm], [ex[p] for p in perm], E, k)
    ok = ~r0.tie_flag
    assert np.allclose(r0.out[ok], r1.out[ok], rtol=0, atol=1e-12)
    assert np.all(perm[r1.idx[ok]] == r0.idx[ok])
    # token permutation equivariance (no capacity)
    tp = rng.permutation(T)
    r2 = run_ref(x[tp], W_g, ex, E, k)
    assert np.allclose(r2.out, r0.out[tp], rtol=0, atol=1e-12)


def check_shared():
    """Shared experts: always on, weight 1 ([guide] §7.1; [ch7] §7.3)."""
    rng = np.random.default_rng(10)
    T, d, h, E, k = 20, 4, 6, 5, 2
    x, W_g, ex = rand_case(rng, T, d, h, E, k, S=2)
    zeroed = [(W1, b1, np.zeros_like(W2), np.zeros_like(b2)) for (W1, b1, W2, b2) in ex[:E]] + ex[E:]
    r = run_ref(x, W_g, zeroed, E, k, 0.0, 2)
    assert np.allclose(r.out, ffn_torch(x, *ex[E]) + ffn_torch(x, *ex[E + 1]), rtol=0, atol=1e-12)
    r0 = run_ref(x, W_g, ex, E, k, 0.0, 0)
    r1 = run_ref(x, W_g, ex, E, k, 0.5, 1)
    r1n = run_ref(x, W_g, ex, E, k, 0.5, 0)
    assert np.allclose(r1.out - r1n.out, ffn_torch(x, *ex[E]), rtol=0, atol=1e-12)   # never capacity-limited
    assert r1.kept.tolist() == r1n.kept.tolist() and r0.counts.sum() == T * k


def check_golden_fixtures():
    """Hand-derived closed forms (tests/golden): the 0.6 / 0.4 diagram of the
    [guide] §4.1 flow, and the first-come capacity queue of [guide] §8.2."""
    Phi1 = 0.5 * (1.0 + math.erf(1.0 / math.sqrt(2.0)))
    g = json.load(open(os.path.join(GOLDEN, "two_of_three_experts.json")))
    x = np.array(g["x"])
    W_g = np.array([[0.0 if v is None else math.log(v)] for v in g["W_g_logs"]])
    ex = [tuple(np.array(e[n], dtype=np.float64) for n in ("W1", "b1", "W2", "b2")) for e in g["experts"]]
    r = run_ref(x, W_g, ex, 3, g["k"])
    assert r.idx.tolist() == g["expected"]["idx"]
    assert np.allclose(r.w, [[0.6, 0.4]], rtol=0, atol=1e-15)
    assert r.counts.tolist() == g["expected"]["counts"]
    assert abs(r.aux - 1.25) < 1e-15
    assert abs(r.out[0, 0] - (0.6 * (2 * Phi1 - 1) + 0.4 * 1.5)) < 1e-15

    g = json.load(open(os.path.join(GOLDEN, "capacity_queue.json")))
    x = np.array(g["x"])
    W_g = np.array(g["W_g"])
    ex = [tuple(np.array(e[n], dtype=np.float64) for n in ("W1", "b1", "W2", "b2")) for e in g["experts"]]
    r = run_ref(x, W_g, ex, 2, g["k"], g["capacity_factor"])
    e_ = g["expected"]
    assert r.cap == e_["cap"] and r.idx.tolist() == e_["idx"]
    assert r.counts.tolist() == e_["counts"] and r.kept.tolist() == e_["kept"]
    assert r.slot_pos.tolist() == e_["slot_pos"]
    want = [Phi1] * 3 + [0.0] * 2 + [-(1 - Phi1)]
    assert np.allclose(r.out[:, 0], want, rtol=0, atol=1e-15)
    s = math.e / (math.e + 1 / math.e)
    P = [(5 * s + (1 - s)) / 6, (5 * (1 - s) + s) / 6]
    assert abs(r.aux - 2 * (5 / 6 * P[0] + 1 / 6 * P[1])) < 1e-15


def check_rows_and_override():
    """Restricting outputs to some rows, and overriding the selection, are consistent."""
    rng = np.random.default_rng(11)
    x, W_g, ex = rand_case(rng, 30, 4, 5, 6, 2, S=1)
    full = run_ref(x, W_g, ex, 6, 2, 0.7, 1)
    rows = [0, 3, 17, 29]
    part = run_ref(x, W_g, ex, 6, 2, 0.7, 1, rows=rows)
    assert np.allclose(part.out, full.out[rows], rtol=0, atol=1e-14)
    assert part.slot_pos.tolist() == full.slot_pos.tolist()
    same = run_ref(x, W_g, ex, 6, 2, 0.7, 1, override_idx=full.idx)
    assert np.array_equal(same.out, full.out)
    alt = full.idx.copy()
    alt[5] = alt[5][::-1]
    swapped = run_ref(x, W_g, ex, 6, 2, 0.7, 1, override_idx=alt)
    assert np.allclose(swapped.w[5], full.w[5][::-1])


def check_widen_bf16():
    """bf16 bit patterns widen exactly: 0x3F80 = 1, 0xC000 = -2, 0x3E80 = 0.25,
    0x0001 = 2^-133 (smallest subnormal), 0x7F7F = largest finite."""
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0001, 0x7F7F], dtype=np.uint16)
    v = ref.widen(bits, "bf16")
    assert v.tolist() == [1.0, -2.0, 0.25, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127]


def _no_ffn(E, d):
    """E experts that output 0 (bias-free), for checks of the router alone."""
    return [(np.zeros((2, d)), None, np.zeros((d, 2)), None)] * E


def check_z_loss_closed_forms():
    """Router z-loss (1/T) sum_t logsumexp(l_t)^2 ([guide] §4.3) on closed forms."""
    rng = np.random.default_rng(12)
    # (i) zero router: every logit is 0, so logsumexp = log E for every token
    for E in [1, 2, 8, 64, 256]:
        r = run_ref(rng.standard_normal((17, 3)), np.zeros((E, 3)), _no_ffn(E, 3), E, 1)
        assert abs(r.z - math.log(E) ** 2) <= 1e-14 * max(1.0, math.log(E) ** 2)
    # (ii) router bias only, l_t = log [1, 2, 3, 4] for every token: (log 10)^2
    b = np.log(np.array([1.0, 2.0, 3.0, 4.0]))
    r = run_ref(rng.standard_normal((9, 2)), np.zeros((4, 2)), _no_ffn(4, 2), 4, 2, b_g=b)
    assert abs(r.z - math.log(10.0) ** 2) < 1e-14
    # (iii) two experts with logits (a_t, 0): logsumexp = log(1 + e^a_t), the softplus
    a = np.array([-3.0, -0.5, 0.0, 0.7, 2.0, 5.0])
    r = run_ref(a[:, None], np.array([[1.0], [0.0]]), _no_ffn(2, 1), 2, 1)
    assert abs(r.z - sum(math.log1p(math.exp(v)) ** 2 for v in a) / len(a)) < 1e-14
    # (iv) large equal logits L: logsumexp = L + log E, without overflow
    for (L, E) in [(1000.0, 8), (-1000.0, 3)]:
        r = run_ref(np.ones((4, 1)), np.full((E, 1), L), _no_ffn(E, 1), E, 1)
        assert abs(r.z - (L + math.log(E)) ** 2) <= 1e-13 * (L + math.log(E)) ** 2
    # (v) a common logit shift c moves every logsumexp by c, so z(c) is a quadratic
    # in c with leading coefficient 1: unit-step second differences are exactly 2
    x, W_g, ex = rand_case(rng, 11, 4, 2, 5, 2)
    z = [run_ref(x, W_g, ex, 5, 2, b_g=np.full(5, c)).z for c in (-1.0, 0.0, 1.0, 2.0)]
    assert abs((z[2] - 2 * z[1] + z[0]) - 2.0) < 1e-12 and abs((z[3] - 2 * z[2] + z[1]) - 2.0) < 1e-12
    # (vi) it depends on the router alone: not on k, the capacity or the experts
    r1 = run_ref(x, W_g, ex, 5, 1, 0.5)
    r2 = run_ref(x, W_g, _no_ffn(5, 4), 5, 3)
    assert r1.z == r2.z == run_ref(x, W_g, ex, 5, 2).z


def check_silu_and_bias_free():
    """SiLU = u sigmoid(u) ([guide] §6.1): closed values, the identity
    silu(u) - silu(-u) = u, torch's F.silu; the bias-free SiLU expert equals
    torch F.linear without bias around F.silu; a None bias equals a zero bias."""
    import torch
    import torch.nn.functional as F
    s = lambda u: float(ref.silu(np.array([u]))[0])
    assert s(0.0) == 0.0
    assert abs(s(1.0) - math.e / (math.e + 1.0)) < 1e-16
    assert abs(s(-1.0) + 1.0 / (math.e + 1.0)) < 1e-16
    assert s(800.0) == 800.0 and abs(s(-800.0)) < 1e-300 and math.isfinite(s(-800.0))
    u = np.linspace(-30.0, 30.0, 241)
    assert np.allclose(ref.silu(u) - ref.silu(-u), u, rtol=0, atol=1e-13)
    assert np.allclose(ref.silu(u), F.silu(torch.as_tensor(u)).numpy(), rtol=1e-14, atol=1e-300)
    rng = np.random.default_rng(13)
    W1, W2 = rng.standard_normal((12, 5)), rng.standard_normal((5, 12))
    xr = rng.standard_normal((7, 5))
    t = lambda a: torch.as_tensor(a, dtype=torch.float64)
    want = F.linear(F.silu(F.linear(t(xr), t(W1))), t(W2)).numpy()
    assert np.allclose(ref.expert_ffn(xr, W1, None, W2, None, "silu"), want, rtol=0, atol=1e-13)
    for act in ("gelu", "silu"):
        assert np.array_equal(ref.expert_ffn(xr, W1, None, W2, None, act),
                              ref.expert_ffn(xr, W1, np.zeros(12), W2, np.zeros(5), act))


def check_min_capacity():
    """Capacity floor min_capacity ([guide] §5.1 DeepSpeed block, with the §8.2
    formula): cap = max(ceil(cf T / E), min_capacity); no limit stays no limit."""
    assert ref.capacity_of(1.0, 8, 4, 4) == 4          # ceil(2) = 2: the floor binds
    assert ref.capacity_of(1.25, 4096, 64, 4) == 80    # ceil(80) = 80: it does not
    assert ref.capacity_of(2.0, 4096, 64, 4) == 128    # the eval capacity factor 2.0 of §5.1
    assert ref.capacity_of(0.01, 100, 4, 3) == 3       # ceil(0.25) = 1 -> 3
    assert ref.capacity_of(0.0, 10, 2, 4) is None and ref.capacity_of(-1.0, 10, 2, 7) is None
    assert ref.capacity_of(1.0, 6, 4, 0) == 2          # no floor: ceil(1.5)
    rng = np.random.default_rng(15)
    x, W_g, ex = rand_case(rng, 40, 3, 2, 4, 2)
    W_g[0] += 1.5
    r0 = run_ref(x, W_g, ex, 4, 2, 0.2)                # ceil(2) = 2
    r1 = run_ref(x, W_g, ex, 4, 2, 0.2, min_capacity=7)
    assert r0.cap == 2 and r1.cap == 7
    assert np.all(r1.kept == np.minimum(r1.counts, 7)) and np.all(r1.slot_kept[r0.slot_kept])
    big = run_ref(x, W_g, ex, 4, 2, 0.2, min_capacity=40)   # floor >= T: nothing dropped
    assert big.slot_kept.all() and np.allclose(big.out, run_ref(x, W_g, ex, 4, 2).out, rtol=0, atol=0)


def check_mixtral_expert_against_brute():
    """Bias-free SiLU experts with a capacity floor == brute force (scalar loops,
    subset enumeration, explicit first-come queues)."""
    rng = np.random.default_rng(14)
    # (T, d, h, E, k, S, cf, min_capacity, cap worked out by hand)
    cases = [(8, 3, 4, 4, 2, 0, 0.0, 0, None), (8, 3, 3, 5, 2, 1, 0.5, 3, 3),
             (7, 2, 4, 3, 1, 0, 0.3, 2, 2), (6, 4, 2, 4, 2, 1, 1.0, 0, 2), (9, 2, 3, 3, 2, 0, 0.4, 5, 5)]
    for (T, d, h, E, k, S, cf, mc, cap) in cases:
        for trial in range(2):
            x, W_g, ex = rand_case(rng, T, d, h, E, k, S)
            ex = [(W1, None, W2, None) for (W1, _, W2, _) in ex]
            b_g = rng.standard_normal(E) if trial == 1 else None
            r = run_ref(x, W_g, ex, E, k, cf, S, b_g, activation="silu", min_capacity=mc)
            assert not r.tie_flag.any() and r.cap == cap
            b = brute_case(x, W_g, ex, k, cap=cap, S=S, b_g=b_g, activation="silu")
            assert r.idx.tolist() == b["idx"] and r.kept.tolist() == b["kept"]
            assert r.slot_kept.tolist() == b["slot_kept"]
            assert abs(r.aux - b["aux"]) < 1e-13 and abs(r.z - b["z"]) < 1e-12
            assert np.allclose(r.out, np.array(b["out"]), rtol=0, atol=1e-11)


def check_golden_silu_min_capacity():
    """Hand-derived fixture (tests/golden/silu_min_capacity.json): Mixtral expert
    form of [guide] §6.1, a capacity floor, and the z-loss of [guide] §4.3."""
    g = json.load(open(os.path.join(GOLDEN, "silu_min_capacity.json")))
    vec = lambda v: None if v is None else np.array(v, dtype=np.float64)
    ex = [tuple(vec(e[n]) for n in ("W1", "b1", "W2", "b2")) for e in g["experts"]]
    r = run_ref(np.array(g["x"]), np.array(g["W_g"]), ex, 2, g["k"], g["capacity_factor"],
                activation=g["activation"], min_capacity=g["min_capacity"])
    e_ = g["expected"]
    assert r.cap == e_["cap"] and r.idx.tolist() == e_["idx"]
    assert r.counts.tolist() == e_["counts"] and r.kept.tolist() == e_["kept"]
    assert r.slot_pos.tolist() == e_["slot_pos"]
    want = [math.e / (math.e + 1)] * 4 + [0.0] + [-1 / (math.e + 1)]
    assert np.allclose(r.out[:, 0], want, rtol=0, atol=1e-15)
    assert abs(r.z - math.log(math.e + 1 / math.e) ** 2) < 1e-15


def run_ec(x, W_g, experts, E, C, S=0, b_g=None, **kw):
    return ref.moe_forward_expert_choice_ref(x, W_g, lambda e: experts[e], E, C, S, b_g, kind="f64", **kw)


def check_ec_against_brute():
    """Expert choice == brute force (per-expert subset enumeration, scalar loops)."""
    rng = np.random.default_rng(16)
    # (T, d, h, E, C, S, activation)
    cases = [(6, 3, 3, 3, 2, 0, "gelu"), (7, 2, 4, 4, 1, 0, "gelu"), (8, 3, 2, 2, 4, 1, "silu"),
             (5, 4, 3, 3, 5, 0, "gelu"), (9, 2, 3, 4, 3, 1, "gelu"), (6, 3, 2, 5, 3, 0, "silu")]
    for (T, d, h, E, C, S, act) in cases:
        for trial in range(2):
            x, W_g, ex = rand_case(rng, T, d, h, E, 1, S)
            b_g = rng.standard_normal(E) if trial == 1 else None
            r = run_ec(x, W_g, ex, E, C, S, b_g, activation=act)
            assert not r.flag.any()
            vec = lambda b: None if b is None else list(map(float, b))
            exl = [(to_lists(W1), vec(b1), to_lists(W2), vec(b2)) for (W1, b1, W2, b2) in ex]
            b = brute.brute_expert_choice_layer(to_lists(x), to_lists(W_g), exl, C, S, vec(b_g), act)
            assert r.tok.tolist() == b["tok"] and r.per_token.tolist() == b["per_token"]
            assert np.allclose(r.w, np.array(b["w"]), rtol=0, atol=1e-14)
            assert abs(r.aux - b["aux"]) < 1e-13 and abs(r.z - b["z"]) < 1e-12
            assert np.allclose(r.out, np.array(b["out"]), rtol=0, atol=1e-11)


def check_ec_dense_limit_and_balance():
    """C = T: every expert takes every token, so the layer is the dense softmax
    mixture sum_e p_e FFN_e(x) ([ch7] §7.1), computed here through torch; any
    C: each expert takes exactly C distinct tokens (perfect balance, [ch7]
    §7.2), the taken logits dominate the untaken ones, and the balance loss is 1."""
    rng = np.random.default_rng(17)
    for (T, d, h, E) in [(20, 6, 10, 4), (9, 3, 5, 7)]:
        x, W_g, ex = rand_case(rng, T, d, h, E, 1)
        r = run_ec(x, W_g, ex, E, T)
        l = x @ W_g.T
        p = np.exp(l - l.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        dense = sum(p[:, e:e + 1] * ffn_torch(x, *ex[e]) for e in range(E))
        assert np.allclose(r.out, dense, rtol=0, atol=1e-12)
        assert np.all(r.per_token == E)
    for (T, E, C) in [(50, 4, 7), (33, 8, 1), (40, 3, 20)]:
        x, W_g, ex = rand_case(rng, T, 5, 2, E, 1)
        r = run_ec(x, W_g, ex, E, C)
        assert r.tok.shape == (E, C) and r.per_token.sum() == E * C
        for e in range(E):
            assert len(set(r.tok[e].tolist())) == C and np.all(np.diff(r.tok[e]) > 0)
            un = np.setdiff1d(np.arange(T), r.tok[e])
            assert un.size == 0 or r.logits[r.tok[e], e].min() >= r.logits[un, e].max()
            assert np.allclose(r.w[e], r.probs[r.tok[e], e], rtol=0, atol=0)
        assert abs(r.aux - 1.0) < 1e-12
    # ties go to the lower token index; near-ties are flagged
    l = np.array([[1.0, 0.0], [2.0, 0.0], [2.0, 5.0], [0.5, 5.0 - 5e-7]])
    sel = ref.select_expert_choice(l, 2)
    assert sel.tok.tolist() == [[1, 2], [2, 3]] and sel.flag.tolist() == [False, False]
    sel = ref.select_expert_choice(l, 1)
    assert sel.tok.tolist() == [[1], [2]] and sel.flag.tolist() == [True, True]
    assert ref.is_valid_expert_choice(l[:, 0], [2]) and not ref.is_valid_expert_choice(l[:, 0], [0])
    # capacity: ceil(cf T / E), floored by min_capacity, at most T
    assert ref.expert_choice_capacity(2.0, 16384, 64) == 512
    assert ref.expert_choice_capacity(1.0, 10, 4, 4) == 4 and ref.expert_choice_capacity(8.0, 10, 2) == 10


def check_golden_expert_choice():
    """Hand-derived fixture (tests/golden/expert_choice_four_tokens.json): [guide]
    §4.2 / [ch7] §7.2 expert choice with a token that no expert takes."""
    g = json.load(open(os.path.join(GOLDEN, "expert_choice_four_tokens.json")))
    ex = [tuple(np.array(e[n], dtype=np.float64) for n in ("W1", "b1", "W2", "b2")) for e in g["experts"]]
    Phi = lambda u: 0.5 * (1.0 + math.erf(u / math.sqrt(2.0)))
    gelu = lambda u: u * Phi(u)
    sig = lambda u: 1.0 / (1.0 + math.exp(-u))
    x, W_g = np.array(g["x"]), np.array(g["W_g"])
    r = run_ec(x, W_g, ex, 2, 1)
    assert r.tok.tolist() == g["expected"]["C1"]["tok"] and r.per_token.tolist() == g["expected"]["C1"]["per_token"]
    assert np.allclose(r.out[:, 0], [0.0, sig(4) * gelu(2), sig(2) * gelu(-1), 0.0], rtol=0, atol=1e-15)
    r = run_ec(x, W_g, ex, 2, 2)
    assert r.tok.tolist() == g["expected"]["C2"]["tok"] and r.per_token.tolist() == g["expected"]["C2"]["per_token"]
    want = [sig(2) * gelu(1), sig(4) * gelu(2), sig(2) * gelu(-1), sig(-1) * gelu(0.5)]
    assert np.allclose(r.out[:, 0], want, rtol=0, atol=1e-15)


def check_selection_bias_closed_form():
    """A selection-only router bias ([guide] §4.3 / §7.1 and [bee]: DeepSeek-V3
    corrects expert usage with a bias on the router logits; this is the reading
    where only the choice sees it).  One token, logits (2, 1, 0), b_sel =
    (0, 0, 3), k = 2: the keys (2, 1, 3) choose experts 2 then 0; their weights
    are the plain softmax probabilities renormalised, 1/(e^2+1) and
    e^2/(e^2+1); f = (1/2, 0, 1/2) with P the plain softmax, so aux =
    1.5 (e^2+1)/(e^2+e+1); z = log(e^2+e+1)^2.  Expert e maps x = 1 to
    GELU(e + 1)."""
    Phi = lambda u: 0.5 * (1.0 + math.erf(u / math.sqrt(2.0)))
    gelu = lambda u: u * Phi(u)
    e2 = math.e ** 2
    x = np.array([[1.0]])
    W_g = np.array([[2.0], [1.0], [0.0]])
    ex = [(np.array([[e + 1.0]]), np.zeros(1), np.array([[1.0]]), np.zeros(1)) for e in range(3)]
    r = run_ref(x, W_g, ex, 3, 2, b_sel=np.array([0.0, 0.0, 3.0], dtype=np.float32))
    assert r.idx.tolist() == [[2, 0]]
    assert np.allclose(r.w[0], [1.0 / (e2 + 1.0), e2 / (e2 + 1.0)], rtol=0, atol=1e-15)
    assert r.counts.tolist() == [1, 0, 1]
    assert abs(r.aux - 1.5 * (e2 + 1.0) / (e2 + math.e + 1.0)) < 1e-14
    assert abs(r.z - math.log(e2 + math.e + 1.0) ** 2) < 1e-14
    assert np.allclose(r.P, np.array([e2, math.e, 1.0]) / (e2 + math.e + 1.0), rtol=0, atol=1e-15)
    want = (gelu(3.0) + e2 * gelu(1.0)) / (e2 + 1.0)
    assert abs(r.out[0, 0] - want) < 1e-14
    assert np.array_equal(r.keys, np.array([[2.0, 1.0, 3.0]]))
    # without it the plain top-2 (experts 0, 1)
    assert run_ref(x, W_g, ex, 3, 2).idx.tolist() == [[0, 1]]


def check_selection_bias_invariants_and_brute():
    """A zero or constant selection bias changes nothing; a random one agrees
    with brute force (the subset search ranks l + b_sel, weights, P and z from l)
    with capacity, shared experts and a router offset."""
    rng = np.random.default_rng(31)
    x, W_g, ex = rand_case(rng, 30, 5, 3, 6, 2, 1)
    base = run_ref(x, W_g, ex, 6, 2, 1.25, 1)
    for b in (np.zeros(6, dtype=np.float32), np.full(6, 5.0, dtype=np.float32)):
        r = run_ref(x, W_g, ex, 6, 2, 1.25, 1, b_sel=b)
        assert np.array_equal(r.idx, base.idx) and np.array_equal(r.w, base.w)
        assert np.array_equal(r.kept, base.kept) and r.aux == base.aux and r.z == base.z
        assert np.array_equal(r.out, base.out)
    for (T, d, h, E, k, S, cf) in [(8, 3, 2, 5, 2, 0, None), (7, 2, 3, 4, 3, 1, 0.75), (8, 3, 2, 6, 1, 0, 1.0)]:
        for trial in range(3):
            x, W_g, ex = rand_case(rng, T, d, h, E, k, S)
            b_sel = (rng.standard_normal(E) * 2.0).astype(np.float32)
            b_g = rng.standard_normal(E) if trial == 1 else None
            r = run_ref(x, W_g, ex, E, k, cf or 0.0, S, b_g, b_sel=b_sel)
            assert not r.tie_flag.any()
            cap = None if not cf else int(math.ceil(cf * T / E))
            vec = lambda b: None if b is None else list(map(float, b))
            exl = [(to_lists(W1), vec(b1), to_lists(W2), vec(b2)) for (W1, b1, W2, b2) in ex]
            b = brute.brute_layer(to_lists(x), to_lists(W_g), exl, k, cap=cap, n_shared=S, b_g=vec(b_g),
                                  b_sel=vec(b_sel))
            assert r.idx.tolist() == b["idx"]
            assert np.allclose(r.w, np.array(b["w"]), rtol=0, atol=1e-13)
            assert r.kept.tolist() == b["kept"] and r.slot_kept.tolist() == b["slot_kept"]
            assert abs(r.aux - b["aux"]) < 1e-13 and abs(r.z - b["z"]) < 1e-12
            assert np.allclose(r.out, np.array(b["out"]), rtol=0, atol=1e-12)
        # some selections do change
        assert not np.array_equal(run_ref(x, W_g, ex, E, k, cf or 0.0, S).idx, r.idx) or k == E


# ------------------------------------------------- the pages' own loops --
def _page_form_cases():
    """(label, x, W_g, experts, shared, k, activation, kind) on the tiny fp32
    workload and reduced shapes (float64 arrays; bf16 cases hold bf16-exact values)."""
    from synthetic import CONFIGS, make_inputs
    cases = []
    tiny = make_inputs("tiny", seed=0)
    c = tiny.cfg
    ex = [tuple(None if a is None else ref.widen(a, "f32") for a in tiny.expert(e)) for e in range(c.E)]
    cases.append(("tiny", ref.widen(tiny.x, "f32"), ref.widen(tiny.W_g, "f32"), ex, [], c.k, "gelu"))
    for label, base, kw in [
        ("mixtral-reduced-bf16", "mixtral", dict(T=160, d=64, h=256, E=8, k=2, w_std=0.2)),
        ("switch-top1", "switch", dict(T=120, d=32, h=64, E=16, k=1, cf=0.0, w_std=0.3)),
        ("deepseek-shared", "deepseek", dict(T=100, d=64, h=128, E=16, k=4, S=2, w_std=0.2)),
        ("mixtral-expert-form", "mixtral", dict(T=90, d=32, h=96, E=8, k=2, w_std=0.3, activation="silu",
                                                expert_bias=False)),
    ]:
        inp = make_inputs(CONFIGS[base].replace(name=label, **kw), seed=5)
        c = inp.cfg
        wide = lambda a: None if a is None else ref.widen(a, c.dtype)
        ex = [tuple(wide(a) for a in inp.expert(e)) for e in range(c.E + c.S)]
        cases.append((label, wide(inp.x), wide(inp.W_g), ex[:c.E], ex[c.E:], c.k, c.activation))
    return cases


def check_pages_own_loops():
    """The layer as the pages' sketches compute it (tests/page_forms.py: torch
    CPU float64, torch.topk on the softmax, the guide's §3.1 slot-major loop,
    the tutorial's part-5 expert-major indexed add, the guide's §7.1 shared
    plus routed sum) equals the oracle on every unflagged token: the chosen
    set, the renormalised weights, the output; the tutorial's balance loss is
    k times the oracle's (its fractions count all k choices per token, summing
    to k); the router z-loss is the guide's §4.3 logsumexp form."""
    from tests.page_forms import page_form_layer
    for label, x, W_g, experts, shared, k, act in _page_form_cases():
        E, S = len(experts), len(shared)
        allx = experts + shared
        r = ref.moe_forward_ref(x, W_g, lambda e: allx[e], E, k, 0.0, S, None, kind="f64", activation=act)
        assert not r.tie_flag.any(), label
        for order in ("slot", "expert"):
            pf = page_form_layer(x, W_g, experts, k, order=order, shared=shared, activation=act)
            assert np.array_equal(np.sort(pf.idx, 1), np.sort(r.idx, 1)), (label, order)
            wa = np.take_along_axis(pf.w, np.argsort(pf.idx, 1), 1)
            wb = np.take_along_axis(r.w, np.argsort(r.idx, 1), 1)
            assert np.max(np.abs(wa - wb)) <= 1e-13, (label, order)
            scale = float(np.max(np.abs(r.out)))
            assert np.max(np.abs(pf.out - r.out)) <= 1e-12 * scale, (label, order)
            assert abs(pf.aux_tutorial - k * r.aux) <= 1e-12 * k * r.aux, (label, order)
            assert abs(pf.z - r.z) <= 1e-12 * max(1.0, r.z), (label, order)


ALL_CHECKS = [check_weights_sum_to_one, check_against_brute, check_topk_vs_torch, check_tie_rule,
              check_dense_limit, check_aux_closed_forms, check_capacity, check_dropped_contribute_nothing,
              check_ffn_library, check_combine_symmetries, check_shared, check_golden_fixtures,
              check_rows_and_override, check_widen_bf16, check_z_loss_closed_forms,
              check_silu_and_bias_free, check_min_capacity, check_mixtral_expert_against_brute,
              check_golden_silu_min_capacity, check_ec_against_brute, check_ec_dense_limit_and_balance,
              check_golden_expert_choice, check_selection_bias_closed_form,
              check_selection_bias_invariants_and_brute, check_pages_own_loops]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_pin(check):
    check()

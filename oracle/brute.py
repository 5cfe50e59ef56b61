"""Brute-force scalar model of the sparse-MoE layer forward, for tiny inputs.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.moe_ref``: used by tests
alone, never by the product path).  It is a second, deliberately naive
derivation of the layer used to pin ``oracle.moe_ref``: pure-Python scalar
loops with ``math.exp``/``math.erf``, the top-k set found by enumerating all
C(E, k) expert subsets, and capacity modelled as one explicit first-come
queue per expert.  It shares no helper with ``oracle.moe_ref``.

Definitions followed: the pages' layer of "AI-Research-SKILLs MoE 训练实战…全指南"
§3.1 (router, softmax, top-k, renormalise, weighted expert sum), its §4.3
balance loss and router z-loss, its §8.2 / "第7章 Mixture of Experts" §7.4
capacity, the shared experts of its §7.1 and the SiLU, bias-free Mixtral
expert of its §6.1.
"""
from __future__ import annotations

import itertools
import math
from typing import List, Optional, Sequence


def _dot(a: Sequence[float], b: Sequence[float]) -> float:
    s = 0.0
    for u, v in zip(a, b):
        s += u * v
    return s


def brute_topk(logits: Sequence[float], k: int):
    """Among all k-subsets of experts choose the one with the largest logit sum;
    among equal sums the lexicographically smallest sorted index tuple.  The
    chosen experts are then listed by descending logit, ties by index."""
    E = len(logits)
    best = None
    best_sum = -math.inf
    for combo in itertools.combinations(range(E), k):   # ascending lexicographic order
        s = math.fsum(logits[e] for e in combo)
        if s > best_sum:                                 # strict: the first of equals wins
            best, best_sum = combo, s
    return sorted(best, key=lambda e: (-logits[e], e))


def brute_layer(x: List[List[float]], W_g: List[List[float]], experts, k: int,
                cap: Optional[int] = None, n_shared: int = 0,
                b_g: Optional[Sequence[float]] = None, activation: str = "gelu",
                b_sel: Optional[Sequence[float]] = None):
    """x: T lists of d floats; W_g: E lists of d floats; experts: list of
    (W1 [h][d], b1 [h] or None, W2 [d][h], b2 [d] or None) for E routed then
    n_shared shared; activation "gelu" (erf form) or "silu" (u / (1 + e^-u),
    the Mixtral expert of the guide's §6.1); b_sel a per-expert bias that
    enters the choice of experts only (the subset search ranks l + b_sel; the
    weights, P and z come from l).

    Returns dict(out, idx, w, counts, kept, dropped, slot_kept, aux, z)."""
    T = len(x)
    E = len(W_g)
    d = len(x[0])

    logits = []
    probs = []
    for t in range(T):
        lt = [_dot(x[t], W_g[e]) + (b_g[e] if b_g is not None else 0.0) for e in range(E)]
        m = max(lt)
        ex = [math.exp(v - m) for v in lt]
        z = math.fsum(ex)
        logits.append(lt)
        probs.append([v / z for v in ex])

    if b_sel is None:
        idx = [brute_topk(logits[t], k) for t in range(T)]
    else:
        idx = [brute_topk([logits[t][e] + b_sel[e] for e in range(E)], k) for t in range(T)]
    w = []
    for t in range(T):
        sel = [probs[t][e] for e in idx[t]]
        z = math.fsum(sel)
        w.append([v / z for v in sel])

    counts = [0] * E
    for t in range(T):
        for e in idx[t]:
            counts[e] += 1

    # capacity: one first-come queue per expert, tokens arriving in order
    queues = [[] for _ in range(E)]
    slot_kept = [[False] * k for _ in range(T)]
    for t in range(T):
        for j, e in enumerate(idx[t]):
            if cap is None or len(queues[e]) < cap:
                queues[e].append((t, j))
                slot_kept[t][j] = True
    kept = [len(q) for q in queues]
    dropped = [counts[e] - kept[e] for e in range(E)]

    def ffn(e, xt):
        W1, b1, W2, b2 = experts[e]
        h = len(W1)
        g = []
        for i in range(h):
            u = _dot(W1[i], xt) + (b1[i] if b1 is not None else 0.0)
            if activation == "silu":
                g.append(u / (1.0 + math.exp(-u)))
            else:
                g.append(0.5 * u * (1.0 + math.erf(u / math.sqrt(2.0))))
        return [_dot(W2[c], g) + (b2[c] if b2 is not None else 0.0) for c in range(d)]

    out = [[0.0] * d for _ in range(T)]
    for t in range(T):
        for j, e in enumerate(idx[t]):
            if not slot_kept[t][j]:
                continue
            y = ffn(e, x[t])
            for c in range(d):
                out[t][c] += w[t][j] * y[c]
        for s in range(n_shared):
            y = ffn(E + s, x[t])
            for c in range(d):
                out[t][c] += y[c]

    aux = 0.0
    for e in range(E):
        f_e = counts[e] / (T * k)
        P_e = math.fsum(probs[t][e] for t in range(T)) / T
        aux += f_e * P_e
    aux *= E

    # router z-loss ([guide] §4.3): mean over tokens of log(sum_e exp l)^2,
    # summed directly (tiny inputs only: no overflow guard)
    z = math.fsum(math.log(math.fsum(math.exp(v) for v in logits[t])) ** 2 for t in range(T)) / T

    return dict(out=out, idx=idx, w=w, counts=counts, kept=kept, dropped=dropped,
                slot_kept=slot_kept, aux=aux, z=z, logits=logits, probs=probs)


def brute_expert_choice_layer(x: List[List[float]], W_g: List[List[float]], experts, C: int,
                              n_shared: int = 0, b_g: Optional[Sequence[float]] = None,
                              activation: str = "gelu"):
    """Expert-choice routing ([guide] §4.2; "第7章 Mixture of Experts" §7.2),
    scalar loops: every expert's column of logits goes through the subset
    enumeration of brute_topk (the C-subset of tokens with the largest logit
    sum, the lexicographically smallest among equals); a chosen token is
    weighted by its softmax probability of that expert.

    Returns dict(out, tok [E][C] ascending, w [E][C], per_token, aux, z)."""
    T = len(x)
    E = len(W_g)
    d = len(x[0])
    logits = [[_dot(x[t], W_g[e]) + (b_g[e] if b_g is not None else 0.0) for e in range(E)] for t in range(T)]
    probs = []
    for t in range(T):
        m = max(logits[t])
        ex = [math.exp(v - m) for v in logits[t]]
        z = math.fsum(ex)
        probs.append([v / z for v in ex])

    tok = [sorted(brute_topk([logits[t][e] for t in range(T)], C)) for e in range(E)]
    w = [[probs[t][e] for t in tok[e]] for e in range(E)]
    per_token = [sum(1 for e in range(E) if t in tok[e]) for t in range(T)]

    def ffn(e, xt):
        W1, b1, W2, b2 = experts[e]
        g = []
        for i in range(len(W1)):
            u = _dot(W1[i], xt) + (b1[i] if b1 is not None else 0.0)
            g.append(u / (1.0 + math.exp(-u)) if activation == "silu" else 0.5 * u * (1.0 + math.erf(u / math.sqrt(2.0))))
        return [_dot(W2[c], g) + (b2[c] if b2 is not None else 0.0) for c in range(d)]

    out = [[0.0] * d for _ in range(T)]
    for e in range(E):
        for c, t in enumerate(tok[e]):
            y = ffn(e, x[t])
            for i in range(d):
                out[t][i] += w[e][c] * y[i]
    for s in range(n_shared):
        for t in range(T):
            y = ffn(E + s, x[t])
            for i in range(d):
                out[t][i] += y[i]

    # every expert receives C of the E*C assignments: f_e = 1/E
    aux = E * math.fsum((1.0 / E) * (math.fsum(probs[t][e] for t in range(T)) / T) for e in range(E))
    z = math.fsum(math.log(math.fsum(math.exp(v) for v in logits[t])) ** 2 for t in range(T)) / T
    return dict(out=out, tok=tok, w=w, per_token=per_token, aux=aux, z=z)

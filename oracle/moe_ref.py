"""CPU oracle of the sparse Mixture-of-Experts FFN layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``sparse_mixture_experts_28_amd``) and never imports it.

The layer reaches exactly (up to rounding order) a result with a plain
definition, MoE(x) = sum_i G(x)_i * E_i(x) with G the renormalised top-k
softmax gate, plus the capacity cap and the shared experts.  So this oracle
is that definition written out in float64, one step per function, with no
blocking, fusion or reordering.  bfloat16 inputs (uint16 bit patterns) are
widened exactly to float64 first; no intermediate is ever rounded.

Pages cited (each by its title and its own section):
  [guide]    "AI-Research-SKILLs MoE 训练实战：稀疏专家模型的架构、路由、负载均衡与推理优化全指南"
             (news.rkmt.cn) -- §3.1 basic MoE layer, §4.1 data-flow diagram,
             §4.2 routing mechanisms, §4.3 auxiliary loss, §7.1 DeepSeekMoE,
             §7.2 Switch Transformers, §8.2 capacity factor.
  [tutorial] "混合专家大模型MoE架构选型与部署实践教程" (developer.baidu.com) --
             part 5, the generic gate / layer pseudo-code (SparseMoEGate, SimpleMoELayer).
  [bee]      "[BEE-30064] 混合專家架構與服務" -- "專家路由工作原理" (how routing works).
  [ch7]      "第7章 Mixture of Experts（MoE）架构" (glsqs.com) -- §7.1 formal
             definition, §7.2 Top-K gating, §7.3 shared experts, §7.4 balance loss
             and capacity, and the tensor-shape trace.

Readings taken where the pages are silent or disagree (every one is listed
with its reason in the design notes of this repository):
  * selection is made on the logits, descending, ties to the lower expert
    index; softmax-then-top-k and top-k-then-softmax agree exactly;
  * a token is flagged when its k-th and (k+1)-th largest logits differ by
    less than TIE_EPS (its routing is then decided by rounding, not by the
    method); "order-ambiguous" when two adjacent logits inside its top k do;
  * aux = E * sum_e f_e P_e with f_e = c_e / (T k) over all k choices before
    any capacity drop, P_e the mean full softmax over all T tokens, no alpha;
  * capacity cap = ceil(cf * T / E) in double, counting tokens (not T*k);
    per expert, assignments are kept in ascending token order; a dropped
    assignment contributes nothing and the surviving weights are not
    renormalised;
  * GELU is the exact erf form; the expert output b2 sits inside the
    weighted term;
  * shared experts are stored after the routed ones, weight 1, no capacity;
  * the router z-loss is the mean over tokens of the squared log-sum-exp of
    that token's logits (router bias included), unscaled;
  * SiLU is u * sigmoid(u); a missing expert bias (None) is a bias-free
    Linear; min_capacity raises the capacity to at least that many tokens and
    only applies when there is a capacity limit (cf > 0);
  * expert-choice routing: each expert takes the C tokens with the largest
    router logits (ties to the lower token index), listed in ascending token
    order; a chosen token is weighted by its softmax probability of that
    expert (the gate G(x) of the layer), not renormalised; a token may be
    taken by several experts or by none.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np
from scipy.special import erf

TIE_EPS = 1e-6


# ---------------------------------------------------------------- inputs --
def widen(a, kind: str) -> np.ndarray:
    """Exact conversion of an input array to float64.

    kind "bf16": ``a`` holds bfloat16 bit patterns (uint16); a bfloat16 is
    the top half of a float32, so shifting left by 16 gives that float32
    exactly, and float32 -> float64 is exact.  kind "f32": a float32 array.
    """
    if kind == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if kind == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if kind == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(f"unknown input kind {kind!r}")


# ---------------------------------------------------------------- router --
def router_logits(x: np.ndarray, W_g: np.ndarray, b_g: Optional[np.ndarray] = None) -> np.ndarray:
    """l[t,e] = sum_c x[t,c] W_g[e,c] (+ b_g[e]).

    The router is one linear layer d -> E ([bee] "how routing works": bias-free;
    [guide] §6.1 and [tutorial] part 5 likewise); W_g has the nn.Linear layout
    [E, d].  The optional b_g is a fixed logit offset used only to skew loads
    in a synthetic workload ([guide] §4.3 mentions a bias on the logits).
    """
    l = x @ W_g.T
    if b_g is not None:
        l = l + np.asarray(b_g, dtype=np.float64)[None, :]
    return l


def softmax(l: np.ndarray) -> np.ndarray:
    """p[t,e] = exp(l[t,e] - m_t) / sum_e' exp(l[t,e'] - m_t), m_t = max_e l[t,e]
    ([guide] §3.1; [tutorial] part 5: softmax over the expert axis)."""
    m = l.max(axis=1, keepdims=True)
    z = np.exp(l - m)
    return z / z.sum(axis=1, keepdims=True)


def router_z_loss(l: np.ndarray) -> float:
    """Router z-loss: (1/T) sum_t (log sum_e exp l[t,e])^2, unscaled.

    [guide] §4.3 adds it to the balance loss to keep the router's logits small
    (the training loss weights it by 0.001, as its §8.5 repeats); it acts on
    the logits themselves, so a router bias is included.  The log-sum-exp is
    taken with the row maximum factored out, which cannot overflow."""
    m = l.max(axis=1)
    lse = m + np.log(np.exp(l - m[:, None]).sum(axis=1))
    return float(np.mean(lse * lse))


@dataclass
class Selection:
    idx: np.ndarray          # [T,k] int64, slot 0 = largest logit
    tie_flag: np.ndarray     # [T] bool: k-th vs (k+1)-th logit gap < TIE_EPS
    order_flag: np.ndarray   # [T] bool: an adjacent gap inside the top k < TIE_EPS


def select_topk(l: np.ndarray, k: int, eps: float = TIE_EPS) -> Selection:
    """The k experts with the largest logits, descending, ties to the lower index.

    ([guide] §3.1 and §4.2; [bee] "how routing works" step 2; [ch7] §7.2 Top-K
    gating.)  A stable sort of the negated logits keeps equal logits in
    ascending expert order, which is the tie rule.
    """
    T, E = l.shape
    order = np.argsort(-l, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int64)
    s = np.take_along_axis(l, order, axis=1)
    if k < E:
        tie = (s[:, k - 1] - s[:, k]) < eps
    else:
        tie = np.zeros(T, dtype=bool)
    if k > 1:
        order_amb = np.any((s[:, : k - 1] - s[:, 1:k]) < eps, axis=1)
    else:
        order_amb = np.zeros(T, dtype=bool)
    return Selection(idx=idx, tie_flag=tie, order_flag=order_amb)


def is_valid_topk(l_row: np.ndarray, chosen: Sequence[int], eps: float = TIE_EPS) -> bool:
    """True iff ``chosen`` is a set of k distinct experts that is a top-k set
    of ``l_row`` up to near-ties: no expert left out has a logit more than
    ``eps`` above the smallest chosen logit."""
    chosen = [int(c) for c in chosen]
    E = l_row.shape[0]
    if len(set(chosen)) != len(chosen) or any(c < 0 or c >= E for c in chosen):
        return False
    rest = [e for e in range(E) if e not in set(chosen)]
    if not rest:
        return True
    return float(max(l_row[rest])) <= float(min(l_row[chosen])) + eps


def renormalised_weights(p: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w[t,j] = p[t, idx[t,j]] / sum_j' p[t, idx[t,j']] ([guide] §3.1: the k
    scores are divided by their sum; [tutorial] part 5 likewise).  Equals the
    softmax over the k selected logits ([bee] step 3; [ch7] §7.2)."""
    sel = np.take_along_axis(p, idx, axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def expert_counts(idx: np.ndarray, E: int) -> np.ndarray:
    """c_e = number of (token, slot) assignments routed to expert e, before capacity."""
    return np.bincount(idx.ravel(), minlength=E).astype(np.int64)


def aux_loss(counts: np.ndarray, p: np.ndarray, k: int) -> tuple[float, np.ndarray, np.ndarray]:
    """Switch balance loss E * sum_e f_e P_e, unscaled ([guide] §4.3; [ch7] §7.4).

    f_e = c_e / (T k): the fraction of the T*k assignments sent to e;
    P_e = (1/T) sum_t p[t,e]: the mean router probability of e.
    Returns (aux, f, P)."""
    T, E = p.shape
    f = counts.astype(np.float64) / float(T * k)
    P = p.mean(axis=0)
    return float(E * np.sum(f * P)), f, P


# -------------------------------------------------------------- capacity --
def capacity_of(capacity_factor: float, T: int, E: int, min_capacity: int = 0) -> Optional[int]:
    """cap = max(ceil(cf * T / E), min_capacity), the ceiling computed in
    double; None (no limit) when cf <= 0, whatever min_capacity is.

    [guide] §8.2 and [ch7] §7.4 give C = CF * tokens / experts, counting
    tokens; the ceiling follows the switch-style workload's own statement.
    [guide] §5.1's DeepSpeed block names a ``min_capacity`` knob without
    defining it; it is read as a floor under the computed capacity."""
    if capacity_factor is None or capacity_factor <= 0:
        return None
    return max(int(math.ceil(float(capacity_factor) * float(T) / float(E))), int(min_capacity))


def capacity_ranks(idx: np.ndarray, E: int) -> np.ndarray:
    """rank[t,j] = number of earlier tokens t' < t that were routed to idx[t,j].

    Each expert receives its assignments in ascending token order; a token's
    k experts are distinct, so the slot index never breaks a tie."""
    T, k = idx.shape
    rank = np.empty((T, k), dtype=np.int64)
    seen = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            rank[t, j] = seen[e]
            seen[e] += 1
    return rank


# ---------------------------------------------------------------- experts --
def gelu(u: np.ndarray) -> np.ndarray:
    """GELU, exact erf form: 0.5 u (1 + erf(u / sqrt 2)) (nn.GELU's default,
    used by the expert FFN of [guide] §3.1)."""
    return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))


def silu(u: np.ndarray) -> np.ndarray:
    """SiLU: u * sigmoid(u) = u / (1 + exp(-u)) ([guide] §6.1, the activation
    of the Mixtral expert).  Written with exp(-|u|) so neither sign overflows."""
    e = np.exp(-np.abs(u))
    return np.where(u >= 0, u / (1.0 + e), u * e / (1.0 + e))


ACTIVATIONS = {"gelu": gelu, "silu": silu}


def expert_ffn(xr: np.ndarray, W1: np.ndarray, b1: Optional[np.ndarray], W2: np.ndarray,
               b2: Optional[np.ndarray], activation: str = "gelu") -> np.ndarray:
    """y = W2 act(W1 x + b1) + b2 for each row of xr.

    [guide] §3.1: Linear(d, h), GELU, Linear(h, d), both with bias ([tutorial]
    part 5 likewise); [guide] §6.1's Mixtral expert: Linear(d, h) without bias,
    SiLU, Linear(h, d) without bias.  A bias given as None is absent.
    W1 is [h, d] and W2 is [d, h] (nn.Linear layout)."""
    u = xr @ W1.T
    if b1 is not None:
        u = u + b1[None, :]
    y = ACTIVATIONS[activation](u) @ W2.T
    if b2 is not None:
        y = y + b2[None, :]
    return y


# ------------------------------------------------------------------ layer --
@dataclass
class MoERef:
    logits: np.ndarray       # [T,E]
    probs: np.ndarray        # [T,E]
    idx: np.ndarray          # [T,k]
    w: np.ndarray            # [T,k]
    tie_flag: np.ndarray     # [T]
    order_flag: np.ndarray   # [T]
    counts: np.ndarray       # [E] before capacity
    kept: np.ndarray         # [E] after capacity
    rank: np.ndarray         # [T,k] token-order rank within the expert
    slot_kept: np.ndarray    # [T,k] bool
    slot_pos: np.ndarray     # [T,k] row in the expert-sorted buffer, -1 if dropped
    offsets: np.ndarray      # [E+1] exclusive scan of kept
    cap: Optional[int]
    aux: float
    z: float                 # router z-loss
    f: np.ndarray
    P: np.ndarray
    rows: np.ndarray         # token ids whose outputs are in ``out``
    out: np.ndarray          # [len(rows), d] float64
    keys: Optional[np.ndarray] = None   # [T,E] what the top-k ranks: logits (+ b_sel)


def selection_keys(l: np.ndarray, b_sel=None) -> np.ndarray:
    """What the top-k ranks: the logits, plus an optional float32 per-expert
    bias b_sel that changes which experts are chosen but not their weights.

    [guide] §4.3 and §7.1 and [bee] (DeepSeek-V3): the balance loss is
    replaced by a bias on the router logits that is adjusted during training
    to correct the experts' usage.  The pages write it inside the logits
    (``b_g`` here); this is the other reading, where only the choice sees it:
    the softmax weights, the balance loss's P and the z-loss use l."""
    if b_sel is None:
        return l
    return l + np.asarray(b_sel, dtype=np.float32).astype(np.float64)[None, :]


def moe_forward_ref(x, W_g, get_expert: Callable[[int], tuple], E: int, k: int,
                    capacity_factor: float = 0.0, n_shared: int = 0, b_g=None,
                    kind: str = "f32", rows: Optional[Sequence[int]] = None,
                    override_idx: Optional[np.ndarray] = None, activation: str = "gelu",
                    min_capacity: int = 0, b_sel=None) -> MoERef:
    """The whole layer forward in float64.

    x [T,d] and W_g [E,d] are raw inputs of ``kind`` ("f32", "bf16" bit
    patterns, or "f64"); ``get_expert(e)`` returns the raw (W1 [h,d], b1 [h],
    W2 [d,h], b2 [d]) of expert e, routed for e < E and shared for
    E <= e < E + n_shared, either bias possibly None (bias-free Linear);
    b_g is an optional float32 logit offset [E]; b_sel an optional float32
    selection-only bias [E] (see selection_keys).  ``activation`` is "gelu"
    or "silu"; ``min_capacity`` floors the capacity (see capacity_of).

    ``rows`` restricts the expert computation to those tokens (routing,
    counts, capacity and aux always use all T tokens).  ``override_idx``
    replaces the selection with a given [T,k] choice (used to continue the
    comparison after a near-tie was resolved the other way by rounding).

    Steps ([guide] §3.1 and §7.1; [ch7] §7.1 MoE(x) = sum G_i E_i(x)):
      1 logits  2 softmax  3 top-k (of the logits, + b_sel)  4 renormalise
      5 counts, aux and z-loss  6 capacity in token order  7 weighted routed
      experts  8 shared experts.
    """
    xf = widen(x, kind)
    T, d = xf.shape
    l = router_logits(xf, widen(W_g, kind), b_g)
    p = softmax(l)
    keys = selection_keys(l, b_sel)
    sel = select_topk(keys, k)
    idx = sel.idx if override_idx is None else np.asarray(override_idx, dtype=np.int64).reshape(T, k)
    w = renormalised_weights(p, idx)
    counts = expert_counts(idx, E)
    aux, f, P = aux_loss(counts, p, k)
    z = router_z_loss(l)

    cap = capacity_of(capacity_factor, T, E, min_capacity)
    rank = capacity_ranks(idx, E)
    slot_kept = np.ones((T, k), dtype=bool) if cap is None else (rank < cap)
    kept = counts.copy() if cap is None else np.minimum(counts, cap)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    slot_pos = np.where(slot_kept, offsets[idx] + rank, -1)

    rows_arr = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    want = np.zeros(T, dtype=bool)
    want[rows_arr] = True
    row_of = np.full(T, -1, dtype=np.int64)
    row_of[rows_arr] = np.arange(rows_arr.size)
    out = np.zeros((rows_arr.size, d), dtype=np.float64)

    for e in range(E):
        tok, slot = np.nonzero((idx == e) & slot_kept & want[:, None])
        if tok.size == 0:
            continue
        W1, b1, W2, b2 = (None if a is None else widen(a, kind) for a in get_expert(e))
        y = expert_ffn(xf[tok], W1, b1, W2, b2, activation)
        # a token occurs at most once per expert, so this scatter has no collisions
        out[row_of[tok]] += w[tok, slot][:, None] * y

    for s in range(n_shared):
        W1, b1, W2, b2 = (None if a is None else widen(a, kind) for a in get_expert(E + s))
        out += expert_ffn(xf[rows_arr], W1, b1, W2, b2, activation)

    return MoERef(logits=l, probs=p, idx=idx, w=w, tie_flag=sel.tie_flag,
                  order_flag=sel.order_flag, counts=counts, kept=kept, rank=rank,
                  slot_kept=slot_kept, slot_pos=slot_pos, offsets=offsets, cap=cap,
                  aux=aux, z=z, f=f, P=P, rows=rows_arr, out=out, keys=keys)


# --------------------------------------------------------- expert choice --
@dataclass
class ExpertChoice:
    tok: np.ndarray          # [E, C] int64: expert e's tokens, ascending token order
    flag: np.ndarray         # [E] bool: C-th vs (C+1)-th largest logit of the column < TIE_EPS apart


def select_expert_choice(l: np.ndarray, C: int, eps: float = TIE_EPS) -> ExpertChoice:
    """Expert choice: expert e takes the C tokens t with the largest l[t, e],
    ties to the lower token index ([guide] §4.2, the router scores transposed
    to (experts, tokens) and a top-k over tokens with k = the per-expert
    capacity; [ch7] §7.2, each expert picks its top-C tokens).  The chosen
    set is listed in ascending token order."""
    T, E = l.shape
    order = np.argsort(-l, axis=0, kind="stable")        # per expert: descending, ties -> lower token
    tok = np.sort(order[:C, :], axis=0).T
    s = np.take_along_axis(l, order, axis=0)
    flag = np.zeros(E, dtype=bool) if C >= T else (s[C - 1, :] - s[C, :]) < eps
    return ExpertChoice(tok=tok.astype(np.int64), flag=flag)


def is_valid_expert_choice(l_col: np.ndarray, chosen: Sequence[int], eps: float = TIE_EPS) -> bool:
    """True when ``chosen`` are distinct tokens and none of them has a logit
    more than eps below an unchosen token's (a top-C set up to near-ties)."""
    chosen = list(map(int, chosen))
    if len(set(chosen)) != len(chosen):
        return False
    rest = np.delete(l_col, chosen)
    return rest.size == 0 or float(l_col[chosen].min()) >= float(rest.max()) - eps


def expert_choice_capacity(capacity_factor: float, T: int, E: int, min_capacity: int = 0) -> int:
    """C = min(T, max(ceil(cf T / E), min_capacity)) for cf > 0: the capacity
    formula of [guide] §8.2 (with the floor of its §5.1), an expert cannot
    take more than the T tokens there are."""
    cap = capacity_of(capacity_factor, T, E, min_capacity)
    if cap is None:
        raise ValueError("expert choice needs a capacity factor > 0")
    return min(T, cap)


@dataclass
class ExpertChoiceRef:
    logits: np.ndarray       # [T,E]
    probs: np.ndarray        # [T,E]
    tok: np.ndarray          # [E,C]
    w: np.ndarray            # [E,C] probs[tok[e,c], e]
    flag: np.ndarray         # [E]
    per_token: np.ndarray    # [T] how many experts took each token
    aux: float
    z: float
    P: np.ndarray
    rows: np.ndarray
    out: np.ndarray          # [len(rows), d]


def moe_forward_expert_choice_ref(x, W_g, get_expert: Callable[[int], tuple], E: int, C: int,
                                  n_shared: int = 0, b_g=None, kind: str = "f32",
                                  rows: Optional[Sequence[int]] = None,
                                  override_tok: Optional[np.ndarray] = None,
                                  activation: str = "gelu") -> ExpertChoiceRef:
    """The layer with expert-choice routing, in float64.

    Inputs as moe_forward_ref; C (1..T) tokens per expert.  Steps: 1 logits
    2 softmax over experts 3 each expert's top-C tokens 4 weights
    w[e,c] = p[tok[e,c], e] 5 balance loss and z-loss 6 out[t] = sum over the
    experts that took t of w FFN_e(x_t) 7 shared experts, weight 1.
    ``override_tok`` replaces the selection ([E, C], used after a near-tie was
    resolved the other way by rounding).

    The balance loss keeps the layer's definition E sum_e f_e P_e with f_e the
    fraction of all assignments that expert e receives: every expert receives
    C of the E C, so f is uniform and the loss is sum_e P_e = 1."""
    xf = widen(x, kind)
    T, d = xf.shape
    if not 1 <= C <= T:
        raise ValueError("C must be in 1..T")
    l = router_logits(xf, widen(W_g, kind), b_g)
    p = softmax(l)
    sel = select_expert_choice(l, C)
    tok = sel.tok if override_tok is None else np.asarray(override_tok, dtype=np.int64).reshape(E, C)
    w = p[tok, np.arange(E)[:, None]]
    counts = np.full(E, C, dtype=np.int64)
    f = counts / float(counts.sum())
    P = np.mean(p, axis=0)
    aux = float(E * np.sum(f * P))
    z_ec = router_z_loss(l)
    per_token = np.bincount(tok.ravel(), minlength=T).astype(np.int64)

    rows_arr = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    want = np.zeros(T, dtype=bool)
    want[rows_arr] = True
    row_of = np.full(T, -1, dtype=np.int64)
    row_of[rows_arr] = np.arange(rows_arr.size)
    out = np.zeros((rows_arr.size, d), dtype=np.float64)
    for e in range(E):
        sel_c = np.nonzero(want[tok[e]])[0]
        if sel_c.size == 0:
            continue
        toks = tok[e, sel_c]
        W1, b1, W2, b2 = (None if a is None else widen(a, kind) for a in get_expert(e))
        # the tokens of one expert are distinct, so this scatter has no collisions
        out[row_of[toks]] += w[e, sel_c][:, None] * expert_ffn(xf[toks], W1, b1, W2, b2, activation)
    for s_ in range(n_shared):
        W1, b1, W2, b2 = (None if a is None else widen(a, kind) for a in get_expert(E + s_))
        out = out + expert_ffn(xf[rows_arr], W1, b1, W2, b2, activation)
    return ExpertChoiceRef(logits=l, probs=p, tok=tok, w=w, flag=sel.flag, per_token=per_token, aux=aux,
                           z=z_ec, P=P, rows=rows_arr, out=out)


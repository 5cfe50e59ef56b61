"""The layer in the data-flow forms the pages use, in torch (CPU, float64).

A second, independent derivation that pins the oracle: where the oracle is
numpy with its own top-k (a stable sort of the logits), capacity ranks and
an expert-major loop, these forms use torch's library routines the way the
pages' layer sketches do -- a router Linear, ``torch.softmax`` over experts,
``torch.topk`` on the probabilities, the chosen scores divided by their sum,
experts built as ``nn.Sequential(Linear, GELU/SiLU, Linear)`` -- and walk the
experts in the three orders the pages show:

  * slot-major ("AI-Research-SKILLs MoE 训练实战…全指南" §3.1, the basic MoE
    layer): for each of the k slots, for each expert, the tokens whose slot
    picked that expert are run through it and added with their weight;
  * expert-major with an indexed add ("混合专家大模型MoE架构选型与部署实践教程"
    part 5, the generic gate and layer): for each expert, every (token, slot)
    that picked it, gathered, run once, scaled and index-added;
  * shared plus routed (the guide's §7.1 DeepSeekMoE module): the always-on
    shared experts summed over every token, plus the routed output.

The balance loss is formed as the tutorial's gate forms it (a one-hot over
the k choices summed per token, averaged over tokens, times the mean router
probability, times E): that counts every expert a token picked, so its
fractions sum to k, and it equals k times the loss of the reading this
repository takes (fractions of the T k assignments).  The router z-loss is
the guide's §4.3 form, the token mean of logsumexp(logits) squared.

No capacity limit (the pages' sketches have none).  This module is test
code written for this repository from the pages' descriptions; it shares
nothing with the oracle or the HIP library.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np


def _t(a):
    import torch
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def expert_module(W1, b1, W2, b2, activation: str = "gelu"):
    """nn.Sequential(Linear(d, h), act, Linear(h, d)) holding the given float64
    weights (nn.Linear layout [out, in]); a None bias is a bias-free Linear."""
    import torch
    from torch import nn
    h, d = np.asarray(W1).shape
    act = nn.GELU(approximate="none") if activation == "gelu" else nn.SiLU()
    first = nn.Linear(d, h, bias=b1 is not None, dtype=torch.float64)
    second = nn.Linear(h, d, bias=b2 is not None, dtype=torch.float64)
    with torch.no_grad():
        first.weight.copy_(_t(W1))
        second.weight.copy_(_t(W2))
        if b1 is not None:
            first.bias.copy_(_t(b1))
        if b2 is not None:
            second.bias.copy_(_t(b2))
    return nn.Sequential(first, act, second)


@dataclass
class PageFormResult:
    out: np.ndarray        # [T, d]
    idx: np.ndarray        # [T, k] torch.topk's order on the probabilities
    w: np.ndarray          # [T, k] the chosen probabilities over their sum
    aux_tutorial: float    # E sum_e (mean_t onehot_k count)_e (mean_t p)_e: k x the repository's reading
    z: float               # mean_t logsumexp(l_t)^2


def page_form_layer(x, W_g, experts: Sequence, k: int, order: str = "slot", shared: Sequence = (),
                    activation: str = "gelu") -> PageFormResult:
    """The layer on float64 arrays x [T, d], W_g [E, d]; ``experts`` and
    ``shared`` are (W1, b1, W2, b2) tuples; ``order`` is "slot" (the guide's
    loop over slots, then experts) or "expert" (the tutorial's loop over
    experts with an indexed add)."""
    import torch
    with torch.no_grad():
        X = _t(x)
        T = X.shape[0]
        E = np.asarray(W_g).shape[0]
        router = torch.nn.Linear(X.shape[1], E, bias=False, dtype=torch.float64)
        router.weight.copy_(_t(W_g))
        logits = router(X)
        probs = torch.softmax(logits, dim=-1)
        scores, chosen = torch.topk(probs, k, dim=-1)
        scores = scores / scores.sum(dim=-1, keepdim=True)
        mods = [expert_module(*e, activation=activation) for e in experts]

        routed = torch.zeros_like(X)
        if order == "slot":
            for j in range(k):
                for e, f in enumerate(mods):
                    hit = chosen[:, j] == e
                    if bool(hit.any()):
                        routed[hit] += scores[hit, j].unsqueeze(-1) * f(X[hit])
        elif order == "expert":
            for e, f in enumerate(mods):
                tok, slot = torch.where(chosen == e)
                if tok.numel():
                    routed.index_add_(0, tok, f(X[tok]) * scores[tok, slot].unsqueeze(-1))
        else:
            raise ValueError(order)

        out = routed
        if len(shared):
            out = routed + sum(expert_module(*s, activation=activation)(X) for s in shared)

        picked = torch.nn.functional.one_hot(chosen, E).sum(dim=1).to(torch.float64)   # [T, E]
        aux_tutorial = float(E * torch.sum(picked.mean(dim=0) * probs.mean(dim=0)))
        z = float(torch.logsumexp(logits, dim=-1).pow(2).mean())
    return PageFormResult(out=out.numpy(), idx=chosen.numpy().astype(np.int64), w=scores.numpy(),
                          aux_tutorial=aux_tutorial, z=z)

"""Plant plausible mistakes in the oracle and show that some pin catches each.

Each mutant is one textual edit of oracle/moe_ref.py (a dropped term, a
wrong sign, an off-by-one, another page's reading of a formula, a reordered
loop).  The mutated source is executed as a throw-away module on the CPU and
the pin checks of test_oracle_pins run against it; at least one of them must
fail (an assertion or any exception) for every mutant.
"""
import os
import sys
import types

import pytest

import tests.test_oracle_pins as pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moe_ref.py")
SRC = open(SRC_PATH, encoding="utf-8").read()

MUTANTS = [
    ("softmax_unnormalised", "return z / z.sum(axis=1, keepdims=True)", "return z"),
    ("softmax_no_max_shift_wrong_sign", "z = np.exp(l - m)", "z = np.exp(m - l)"),
    ("topk_smallest", 'order = np.argsort(-l, axis=1, kind="stable")', 'order = np.argsort(l, axis=1, kind="stable")'),
    ("ties_to_higher_index", 'order = np.argsort(-l, axis=1, kind="stable")',
     'order = np.argsort(l, axis=1, kind="stable")[:, ::-1]'),
    ("tie_flag_off_by_one", "tie = (s[:, k - 1] - s[:, k]) < eps", "tie = (s[:, k - 2] - s[:, k - 1]) < eps"),
    ("weights_not_renormalised", "return sel / sel.sum(axis=1, keepdims=True)", "return sel"),
    ("aux_f_over_T_not_Tk", "f = counts.astype(np.float64) / float(T * k)", "f = counts.astype(np.float64) / float(T)"),
    ("aux_missing_E", "return float(E * np.sum(f * P)), f, P", "return float(np.sum(f * P)), f, P"),
    ("aux_P_drops_a_token", "P = p.mean(axis=0)", "P = p[:-1].mean(axis=0)"),
    ("capacity_floor", "int(math.ceil(float(capacity_factor) * float(T) / float(E)))",
     "int(float(capacity_factor) * float(T) / float(E))"),
    ("capacity_off_by_one", "(rank < cap)", "(rank <= cap)"),
    ("capacity_slot_major_order", "    for t in range(T):\n        for j in range(k):\n            e = int(idx[t, j])",
     "    for j in range(k):\n        for t in range(T):\n            e = int(idx[t, j])"),
    ("offsets_use_counts", "offsets[1:] = np.cumsum(kept)", "offsets[1:] = np.cumsum(counts)"),
    ("gelu_tanh_approx", "return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))",
     "return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)))"),
    ("gelu_wrong_sign", "return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))", "return 0.5 * u * (1.0 - erf(u / math.sqrt(2.0)))"),
    ("ffn_drops_b1", "u = u + b1[None, :]", "u = u"),
    ("ffn_drops_b2", "y = y + b2[None, :]", "y = y"),
    # a transposed operand that only shows where the matrix is square (h == d)
    ("ffn_W1_transposed_when_square", "u = xr @ W1.T",
     "u = xr @ (W1 if W1.shape[0] == W1.shape[1] else W1.T)"),
    ("ffn_W2_transposed_when_square", "y = ACTIVATIONS[activation](u) @ W2.T",
     "y = ACTIVATIONS[activation](u) @ (W2 if W2.shape[0] == W2.shape[1] else W2.T)"),
    ("router_W_g_transposed_when_square", "l = x @ W_g.T", "l = x @ (W_g if W_g.shape[0] == W_g.shape[1] else W_g.T)"),
    ("router_drops_bias", "l = l + np.asarray(b_g, dtype=np.float64)[None, :]", "l = l"),
    ("b2_outside_weight", "out[row_of[tok]] += w[tok, slot][:, None] * y",
     "out[row_of[tok]] += w[tok, slot][:, None] * (y - b2[None, :]) + b2[None, :]"),
    ("survivors_renormalised", "out[row_of[tok]] += w[tok, slot][:, None] * y",
     "out[row_of[tok]] += (w[tok, slot] / (w * slot_kept).sum(1)[tok])[:, None] * y"),
    ("dropped_slots_still_added", "tok, slot = np.nonzero((idx == e) & slot_kept & want[:, None])",
     "tok, slot = np.nonzero((idx == e) & want[:, None])"),
    ("shared_weighted_half", "out += expert_ffn(xf[rows_arr], W1, b1, W2, b2, activation)",
     "out += 0.5 * expert_ffn(xf[rows_arr], W1, b1, W2, b2, activation)"),
    ("bf16_widen_wrong_shift", "<< np.uint32(16)", "<< np.uint32(15)"),
    ("z_loss_not_squared", "return float(np.mean(lse * lse))", "return float(np.mean(lse))"),
    ("z_loss_square_of_mean", "return float(np.mean(lse * lse))", "return float(np.mean(lse) ** 2)"),
    ("z_loss_sum_not_mean", "return float(np.mean(lse * lse))", "return float(np.sum(lse * lse))"),
    ("z_loss_drops_max", "lse = m + np.log(", "lse = np.log("),
    ("z_loss_no_max_shift", "lse = m + np.log(np.exp(l - m[:, None]).sum(axis=1))",
     "lse = np.log(np.exp(l).sum(axis=1))"),
    ("z_loss_on_probs", "z = router_z_loss(l)", "z = router_z_loss(p)"),
    ("z_loss_without_router_bias", "z = router_z_loss(l)", "z = router_z_loss(xf @ widen(W_g, kind).T)"),
    ("silu_negative_branch", "u * e / (1.0 + e))", "u / (1.0 + e))"),
    ("silu_is_sigmoid", "return np.where(u >= 0, u / (1.0 + e), u * e / (1.0 + e))",
     "return np.where(u >= 0, 1.0 / (1.0 + e), e / (1.0 + e))"),
    ("activation_ignored", "y = ACTIVATIONS[activation](u) @ W2.T", "y = gelu(u) @ W2.T"),
    ("min_capacity_ignored", "return max(int(math.ceil(float(capacity_factor) * float(T) / float(E))), int(min_capacity))",
     "return int(math.ceil(float(capacity_factor) * float(T) / float(E)))"),
    ("min_capacity_is_a_ceiling", "return max(int(math.ceil(float(capacity_factor) * float(T) / float(E))), int(min_capacity))",
     "return min(int(math.ceil(float(capacity_factor) * float(T) / float(E))), int(min_capacity) or 2 ** 31)"),
    ("min_capacity_applies_without_limit", "    if capacity_factor is None or capacity_factor <= 0:\n        return None\n    return max(",
     "    if capacity_factor is None or capacity_factor <= 0:\n        return int(min_capacity) or None\n    return max("),
    ("ec_takes_smallest", 'order = np.argsort(-l, axis=0, kind="stable")', 'order = np.argsort(l, axis=0, kind="stable")'),
    ("ec_ties_to_higher_token", 'order = np.argsort(-l, axis=0, kind="stable")',
     'order = np.argsort(-l[::-1], axis=0, kind="stable"); order = l.shape[0] - 1 - order'),
    ("ec_one_token_short", "tok = np.sort(order[:C, :], axis=0).T", "tok = np.sort(order[:max(C - 1, 1), :], axis=0).T"),
    ("ec_flag_off_by_one", "(s[C - 1, :] - s[C, :]) < eps", "(s[C - 2, :] - s[C - 1, :]) < eps"),
    ("ec_weight_softmax_over_tokens", "w = p[tok, np.arange(E)[:, None]]",
     "w = (np.exp(l - l.max(0)) / np.exp(l - l.max(0)).sum(0))[tok, np.arange(E)[:, None]]"),
    ("ec_weight_wrong_expert", "w = p[tok, np.arange(E)[:, None]]", "w = p[tok, (np.arange(E)[:, None] + 1) % E]"),
    ("ec_weights_renormalised", "        out[row_of[toks]] += w[e, sel_c][:, None] * expert_ffn(",
     "        out[row_of[toks]] += (w[e, sel_c] / np.maximum(np.bincount(tok.ravel(), weights=w.ravel(), minlength=T)[toks], 1e-300))[:, None] * expert_ffn("),
    ("ec_capacity_not_clipped", "    return min(T, cap)", "    return cap"),
    ("ec_shared_weighted_half", "        out = out + expert_ffn(xf[rows_arr], W1, b1, W2, b2, activation)",
     "        out = out + 0.5 * expert_ffn(xf[rows_arr], W1, b1, W2, b2, activation)"),
    ("sel_bias_ignored", "return l + np.asarray(b_sel, dtype=np.float32).astype(np.float64)[None, :]", "return l"),
    ("sel_bias_subtracted", "return l + np.asarray(b_sel, dtype=np.float32).astype(np.float64)[None, :]",
     "return l - np.asarray(b_sel, dtype=np.float32).astype(np.float64)[None, :]"),
    ("sel_bias_in_weights", "    p = softmax(l)\n    keys = selection_keys(l, b_sel)",
     "    p = softmax(selection_keys(l, b_sel))\n    keys = selection_keys(l, b_sel)"),
    ("sel_bias_in_z_loss", "z = router_z_loss(l)", "z = router_z_loss(keys)"),
]


def _mutant_module(old, new, monkeypatch):
    assert SRC.count(old) == 1, f"mutation anchor not unique/absent: {old!r}"
    name = "oracle_mutant_under_test"
    mod = types.ModuleType(name)
    mod.__dict__["__name__"] = name
    monkeypatch.setitem(sys.modules, name, mod)
    exec(compile(SRC.replace(old, new), name, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, monkeypatch):
    mod = _mutant_module(old, new, monkeypatch)
    monkeypatch.setattr(pins, "ref", mod)
    failures = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except Exception as exc:  # an assertion or a crash both count as caught
            failures.append((check.__name__, type(exc).__name__))
            break
    assert failures, f"mutant {name} passed every pin"


def test_unmutated_source_passes(monkeypatch):
    mod = _mutant_module("TIE_EPS = 1e-6", "TIE_EPS = 1e-6", monkeypatch)
    monkeypatch.setattr(pins, "ref", mod)
    for check in pins.ALL_CHECKS:
        check()

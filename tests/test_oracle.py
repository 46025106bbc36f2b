"""The oracle against its pins (hand examples, closed forms, invariants,
brute force, library routines), and planted mistakes that the pins catch."""
import importlib.util
import os
import types

import pytest

from oracle import lemo_oracle as O
from tests import oracle_pins as P

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "lemo_oracle.py")


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    failures = check(O)
    assert not failures, failures


def mutant(old: str, new: str):
    """A copy of the oracle with one planted mistake (text replacement)."""
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


MUTATIONS = [
    ("no_diagonal_exclusion", "Sbar[out] = -np.inf", "pass", [P.check_exact_hand]),
    ("headmax_keeps_diagonal", "S[:, out] = -np.inf", "pass", [P.check_exact_bruteforce]),
    ("causal_keeps_diagonal", "(j_abs[None, :] >= i_abs[:, None]) if causal", "(j_abs[None, :] > i_abs[:, None]) if causal",
     [P.check_exact_hand]),
    ("causal_reversed", "(j_abs[None, :] >= i_abs[:, None]) if causal", "(j_abs[None, :] <= i_abs[:, None]) if causal",
     [P.check_exact_hand]),
    ("tail_block_dropped", "nb = -(-n_tok // block)\n    Q = bf16_decode(q)", "nb = n_tok // block\n    Q = bf16_decode(q)",
     [P.check_exact_hand]),
    ("pool_tail_divides_by_block", "mean[m] = acc / np.float32(len(rows))", "mean[m] = acc / np.float32(block)",
     [P.check_ragged_tail]),
    ("pool_tail_dropped", "nb = -(-n_tok // block)\n    mean = np.empty", "nb = n_tok // block\n    mean = np.empty",
     [P.check_ragged_tail]),
    ("kept_rows_tail_full", "R = (n_kept - 1) * block + min(block, n_tokens - int(kept[-1]) * block)",
     "R = n_kept * block", [P.check_ragged_tail]),
    ("kept_rows_misplaced_not_skipped", "rows[rows >= n_tokens] = -1", "rows[rows >= n_tokens] = 0",
     [P.check_ragged_tail]),
    ("tail_block_full_width", "rows_of = [np.arange(m * block, min((m + 1) * block, n_tok)) for m in kb]",
     "rows_of = [np.arange(m * block, (m + 1) * block) % n_tok for m in kb]", [P.check_exact_bruteforce]),
    ("empty_block_pair_not_zero", "M[a] = np.maximum(best, 0.0)", "M[a] = best", [P.check_exact_hand]),
    ("batch_shares_first_sequence", "res = [exact_block_scores(q[b], k[b],", "res = [exact_block_scores(q[0], k[0],",
     [P.check_exact_invariants]),
    ("transposed_column_sum", "I = M.sum(axis=0) if query_blocks", "I = M.sum(axis=1) if query_blocks",
     [P.check_exact_hand]),
    ("column_takes_query_block", "key_blocks=[key_block], query_blocks=None, causal=causal)",
     "query_blocks=[key_block], key_blocks=None, causal=causal)", [P.check_exact_column]),
    ("column_ignores_causal", "key_blocks=[key_block], query_blocks=None, causal=causal)",
     "key_blocks=[key_block], query_blocks=None, causal=False)", [P.check_exact_column]),
    ("column_sums_first_row", "return float(M[:, 0].sum()), M[:, 0]", "return float(M[0].sum()), M[:, 0]",
     [P.check_exact_column]),
    ("no_sqrt_scale", "scale = 1.0 / math.sqrt(head_dim)", "scale = 1.0", [P.check_exact_closed_form]),
    ("no_head_mean", ".sum(axis=0) / n_heads", ".sum(axis=0)", [P.check_exact_closed_form, P.check_exact_hand]),
    ("max_before_clamp_swapped", "M[a] = np.maximum(per_head, 0.0).sum(axis=0)", "M[a] = np.maximum(per_head.sum(axis=0), 0.0)",
     [P.check_exact_closed_form]),
    ("predictor_no_clamp", "M = np.maximum(q_hat @ k_hat.T, 0.0)", "M = q_hat @ k_hat.T", [P.check_predictor]),
    ("pool_sum_not_mean", "mean[m] = acc / np.float32(len(rows))", "mean[m] = acc", [P.check_predictor]),
    ("predictor_no_relu", "hid = np.maximum(bf16_decode(xbar) @ bf16_decode(u), 0.0)",
     "hid = bf16_decode(xbar) @ bf16_decode(u)", [P.check_predictor]),
    ("predictor_transposed_v", "return bf16_decode(hid_bf16) @ bf16_decode(v)",
     "return bf16_decode(hid_bf16) @ bf16_decode(v).T", [P.check_predictor]),
    ("token_no_final_round", "return bf16_round(est.astype(np.float32).astype(np.float64))",
     "return bf16_round(np.trunc(est * 64) / 64)", [P.check_token_predictor]),
    ("token_uses_transposed_u", "est = predictor_embeddings(x, u, v)", "est = predictor_embeddings(x, u.T, v)",
     [P.check_token_predictor]),
    ("linear_weight_not_transposed", "prod = bf16_decode(a) @ bf16_decode(weight).T", "prod = bf16_decode(a) @ bf16_decode(weight)",
     [P.check_fused_movement]),
    ("gather_linear_dense_rows", "dst[live, :width] = linear_bf16(np.asarray(x)[rows[live]], weight)",
     "dst[live, :width] = linear_bf16(np.asarray(x)[live], weight)", [P.check_fused_movement]),
    ("gather_linear_no_pad", "        dst[p, :width] = 0\n    return dst, n_pad > cap\n\n\ndef linear_scatter",
     "        pass\n    return dst, n_pad > cap\n\n\ndef linear_scatter", [P.check_fused_movement]),
    ("threshold_strict", "keep = s >= theta\n    elif mode == SELECT_MEAN", "keep = s > theta\n    elif mode == SELECT_MEAN",
     [P.check_select]),
    ("mean_exact_sum", "        for v in s:\n            total += float(v)", "        total = math.fsum(float(v) for v in s)",
     [P.check_select]),
    ("mean_reversed_order", "        for v in s:\n            total += float(v)", "        for v in s[::-1]:\n            total += float(v)",
     [P.check_select]),
    ("topk_ties_high_index", "-float(s[c]) if not np.isnan(s[c]) else 0.0, c))",
     "-float(s[c]) if not np.isnan(s[c]) else 0.0, -c))", [P.check_select]),
    ("round_truncates", "r = np.rint(np.ldexp(ax, -qexp))", "r = np.floor(np.ldexp(ax, -qexp))",
     [P.check_bf16_round, P.check_bf16_add]),
    ("round_ties_away", "r = np.rint(np.ldexp(ax, -qexp))", "r = np.floor(np.ldexp(ax, -qexp) + 0.5)",
     [P.check_bf16_round]),
    ("round_no_subnormals", "qexp = np.maximum(e - 8, -133)", "qexp = e - 8", [P.check_bf16_round]),
    ("gather_wrong_block", "rows = (kept[:, None] * block + np.arange(block)[None, :]).reshape(-1)",
     "rows = ((kept[:, None] + 1) * block + np.arange(block)[None, :]).reshape(-1) % 6", [P.check_movement]),
    ("pad_not_zeroed", "        dst[p, :width] = 0\n    return dst, n_pad > cap\n\n\ndef linear_bf16",
     "        pass\n    return dst, n_pad > cap\n\n\ndef linear_bf16", [P.check_movement]),
    ("scatter_into_dense_rows", "for p, t in enumerate(rows):\n        if t >= 0:\n            out[t] = bf16_round(bf16_decode(out[t]) +",
     "for p, t in enumerate(range(rows.size)):\n        if t >= 0:\n            out[t] = bf16_round(bf16_decode(out[t]) +", [P.check_movement]),
    ("recompute_adds", "bf16_decode(out[t]) - bf16_decode(y[p, :width])", "bf16_decode(out[t]) + bf16_decode(y[p, :width])",
     [P.check_recompute]),
    ("recompute_into_dense_rows", "for p, t in enumerate(rows):\n        if t >= 0:\n            out[t] = bf16_round(bf16_decode(out[t]) -",
     "for p, t in enumerate(range(rows.size)):\n        if t >= 0:\n            out[t] = bf16_round(bf16_decode(out[t]) -", [P.check_recompute]),
    ("recompute_y_misaligned", "bf16_decode(out[t]) - bf16_decode(y[p, :width])", "bf16_decode(out[t]) - bf16_decode(y[t, :width])",
     [P.check_recompute]),
    ("mlp_no_magnitude", "_block_channel_max_sum(np.abs(bf16_decode(act)), block)", "_block_channel_max_sum(bf16_decode(act), block)",
     [P.check_mlp_scores]),
    ("mlp_mean_not_max", ".max(axis=0).sum() for m in range(nb)", ".mean(axis=0).sum() for m in range(nb)", [P.check_mlp_scores]),
    ("mlp_ragged_block_dropped", "nb = -(-n // block)\n    return np.array([mag", "nb = n // block\n    return np.array([mag",
     [P.check_mlp_scores]),
    ("silu_wrong_sign", "g / (1.0 + np.exp(-g)) * u", "g / (1.0 + np.exp(g)) * u", [P.check_mlp_scores]),
    ("gated_uses_gate_twice", "g / (1.0 + np.exp(-g)) * u", "g / (1.0 + np.exp(-g)) * g", [P.check_mlp_scores]),
]


@pytest.mark.parametrize("name,old,new,checks", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, checks):
    mod = mutant(old, new)
    failures = []
    for c in checks:
        try:
            failures += c(mod)
        except Exception as e:  # a crash also counts as caught
            failures.append(f"{c.__name__} raised {e!r}")
    assert failures, f"planted mistake {name} went unnoticed"

"""Planted mistakes in the oracle: each one must make at least one pin fail.

Each case rewrites one snippet of oracle/sol_oracle.py into a plausible
mistake (a dropped term, a wrong sign, index, operand or constant), loads the
result as a separate module, points the pin module at it and runs the named
pins; at least one of them must raise AssertionError.  The snippet must occur
exactly once in the oracle, so that a mutation cannot silently stop applying
when the oracle changes.  Everything here runs on the CPU.
"""

import math
import os
import types

import pytest

import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "sol_oracle.py")

HAND = [(c,) for c in P._golden_cases()]
CONST = [(dict(tau=1.0), 200), (dict(topk_ratio=0.25), 333), (dict(tau=1.0, prefix_len=70), 256)]
BRUTE = [(256, 2, 64, dict(tau=1.0)), (200, 2, 64, dict(topk_ratio=0.25, prefix_len=70)),
         (100, 3, 64, dict(tau=math.inf, prefix_len=10))]

# (name, snippet, replacement, [(pin, [argument tuples])])
MUTATIONS = [
    ("sample_std",
     "sigma = np.sqrt(((S - mu[..., None]) ** 2).mean(axis=-1))",
     "sigma = np.sqrt(((S - mu[..., None]) ** 2).sum(axis=-1) / max(S.shape[-1] - 1, 1))",
     [("test_route_hand_examples", HAND)]),
    ("strict_threshold",
     "sel = S >= thr[..., None]",
     "sel = S > thr[..., None]",
     [("test_route_hand_examples", HAND)]),
    ("ties_to_higher_index",
     'order = np.argsort(-S, axis=-1, kind="stable")',
     'order = (S.shape[-1] - 1) - np.argsort(-S[..., ::-1], axis=-1, kind="stable")',
     [("test_route_hand_examples", HAND)]),
    ("no_sink",
     "sel[..., :pb] = True",
     "sel[..., :pb] = sel[..., :pb]",
     [("test_topk_counts_with_sink", [()]), ("test_route_hand_examples", HAND)]),
    ("tail_mean_over_64",
     "out[:, :, c, :] = rows.sum(axis=1) / rows.shape[1]",
     "out[:, :, c, :] = rows.sum(axis=1) / BLOCK",
     [("test_constant_key_blocks_reproduce_dense", CONST), ("test_brute_force_small", BRUTE)]),
    ("exact_logit_unscaled",
     "logits = [q_rows @ kx.T * scale]",
     "logits = [q_rows @ kx.T]",
     [("test_dense_limit_matches_softmax_and_sdpa", [(1, 200, 2, 64)])]),
    ("centroid_logit_unscaled",
     "y = q_rows @ kbar_head[missed].T * scale",
     "y = q_rows @ kbar_head[missed].T",
     [("test_constant_key_blocks_reproduce_dense", CONST)]),
    ("centroid_logit_from_pooled_q",
     "y = q_rows @ kbar_head[missed].T * scale",
     "y = q_rows.mean(axis=0, keepdims=True) @ kbar_head[missed].T * scale + 0.0 * q_rows[:, :1]",
     [("test_brute_force_small", BRUTE)]),
    ("no_log_mass",
     "y = y + np.log(sizes[missed].astype(np.float64))[None, :]",
     "y = y + 0.0 * np.log(sizes[missed].astype(np.float64))[None, :]",
     [("test_constant_key_blocks_reproduce_dense", CONST)]),
    ("reweight_anchor_over_all_rows",
     "first = int(prefix_len) if 0 <= int(prefix_len) < N else 0",
     "first = 0",
     [("test_reweight_is_exact_for_the_anchor_query", [(70,)])]),
    ("reweight_bias_without_logsumexp",
     "cb[b, h, c] = (m + math.log(e.sum())) - float(kt[b, h, c] @ a) * scale",
     "cb[b, h, c] = m - float(kt[b, h, c] @ a) * scale",
     [("test_reweight_equal_keys_reduce_to_log_mass", [()]), ("test_reweight_bias_is_the_weight_entropy", [()])]),
    ("reweight_value_is_the_mean",
     "vt[b, h, c] = w @ vc",
     "vt[b, h, c] = vc.mean(axis=0)",
     [("test_reweight_is_exact_for_the_anchor_query", [(0,), (70,)])]),
    ("int8_scale_over_255",
     "ks = amax / np.float32(127)",
     "ks = amax / np.float32(255)",
     [("test_int8_codes_round_to_nearest", [()])]),
    ("int8_floor_instead_of_rint",
     "code = np.rint(res / safe[:, :, None, :, None])",
     "code = np.floor(res / safe[:, :, None, :, None])",
     [("test_int8_codes_round_to_nearest", [()])]),
    ("int8_mean_term_dropped",
     "return mean_term + sq * sk * dots",
     "return sq * sk * dots",
     [("test_int8_equal_keys_are_exact", [()]), ("test_int8_logit_error_bound", [()])]),
    ("int8_whole_keys",
     "res = kb - base[:, :, None]",
     "res = kb - 0.0 * base[:, :, None]",
     [("test_int8_equal_keys_are_exact", [()])]),
    ("reblock_metric_of_own_side",
     "M = other.T @ other",
     "M = x.T @ x",
     [("test_reblock_metric_is_score_pattern_cosine", [()])]),
    ("reblock_keys_own_partition",
     "pk[b, h] = pq[b, h]",
     "pk[b, h] = _reblock_head(k[b, :, h], q[b, :, h], r0)",
     [("test_reblock_q_reuse_k_shares_the_query_partition", [()])]),
    ("pivot_a_most_similar",
     "a = int(np.argmin(s))",
     "a = int(np.argmax(s))",
     [("test_pivot_split_hand_example", [()])]),
    ("pivot_b_most_similar",
     "b = int(np.argmin(t))",
     "b = int(np.argmax(t))",
     [("test_pivot_split_hand_example", [()])]),
    ("pivot_rank_sign",
     "p = mu @ (u[b] - u[a])",
     "p = mu @ (u[a] - u[b])",
     [("test_pivot_split_hand_example", [()])]),
]


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"snippet not found exactly once: {old!r}"
    mod = types.ModuleType("sol_oracle_mutant")
    exec(compile(src.replace(old, new), "sol_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, old, new, pins):
    monkeypatch.setattr(P, "O", _mutant(old, new))
    for pin, arglist in pins:
        for args in arglist:
            try:
                getattr(P, pin)(*args)
            except AssertionError:
                return
    pytest.fail(f"no pin caught the planted mistake {name}")


def test_unmutated_oracle_passes_the_same_pins(monkeypatch):
    """The same pins with the oracle as it stands (through the same loader)."""
    monkeypatch.setattr(P, "O", _mutant("BLOCK = 64", "BLOCK = 64"))
    seen = set()
    for _, _, _, pins in MUTATIONS:
        for pin, arglist in pins:
            for args in arglist:
                key = (pin, repr(args))
                if key not in seen:
                    seen.add(key)
                    getattr(P, pin)(*args)

"""Plant plausible mistakes in a copy of the oracle; the pins must catch each.

Each mutation edits one expression of oracle/attention.py's source text (a
dropped term, a wrong sign, a wrong index or axis, a transposed operand),
executes the edited copy as a throwaway module on the CPU, points the pin
tests of test_oracle.py at it, and asserts that at least one pin fails.
The real oracle is never modified.
"""

import os
import types

import pytest

import test_oracle as T

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "attention.py")

MUTATIONS = [
    ("scale dropped from scores", "s = scale * (qc @ k.T)", "s = (qc @ k.T)"),
    ("causal direction flipped", "np.arange(n_keys)[None, :] <= q_pos[:, None]",
     "np.arange(n_keys)[None, :] >= q_pos[:, None]"),
    ("causal hides the diagonal", "np.arange(n_keys)[None, :] <= q_pos[:, None]",
     "np.arange(n_keys)[None, :] < q_pos[:, None]"),
    ("window left bound off by one", "lo = keys >= q_pos[:, None] - left",
     "lo = keys > q_pos[:, None] - left"),
    ("window right bound off by one", "hi = keys <= q_pos[:, None] + right",
     "hi = keys < q_pos[:, None] + right"),
    ("window sides swapped", "lo = keys >= q_pos[:, None] - left",
     "lo = keys >= q_pos[:, None] - right"),
    ("grouped heads interleaved instead of blocked",
     "return np.repeat(k, group, axis=-3), np.repeat(v, group, axis=-3)",
     "return np.tile(k, (group, 1, 1)), np.tile(v, (group, 1, 1))"),
    ("grouped K/V gradient averaged instead of summed",
     "+ g.shape[-2:]).sum(axis=-3)", "+ g.shape[-2:]).mean(axis=-3)"),
    ("max over the wrong axis", "m = s.max(axis=1, keepdims=True)             # pass 1",
     "m = s.max(axis=0, keepdims=True)             # pass 1"),
    ("block mask transposed",
     "vis = bm[q_pos[:, None] // mask_block, np.arange(n_keys)[None, :] // mask_block]",
     "vis = bm[np.arange(n_keys)[None, :] // mask_block, q_pos[:, None] // mask_block]"),
    ("block mask replaces the causal rule", "vis = c if vis is None else vis & c",
     "vis = c if vis is None else vis"),
    ("empty rows get LSE 0", "lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)",
     "lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), 0.0)"),
    ("empty rows keep a uniform P", "p = np.where(l > 0, e / np.where(l > 0, l, 1.0), 0.0)",
     "p = np.where(l > 0, e / np.where(l > 0, l, 1.0), 1.0 / s.shape[1])"),
    ("LSE without the max", "lse[r0:r1] = (m + np.log(l))[:, 0]",
     "lse[r0:r1] = (np.log(l))[:, 0]"),
    ("LSE without the log", "lse[r0:r1] = (m + np.log(l))[:, 0]",
     "lse[r0:r1] = (m + l)[:, 0]"),
    ("unnormalized output", "o[r0:r1] = p @ v", "o[r0:r1] = e @ v"),
    ("backward drops the D term", "ds = p * (dp - d_i)", "ds = p * dp"),
    ("backward sign flipped", "ds = p * (dp - d_i)", "ds = p * (d_i - dp)"),
    ("dK without scale", "dk += scale * (ds.T @ q[r0:r1])", "dk += (ds.T @ q[r0:r1])"),
    ("dQ without scale", "dq[r0:r1] = scale * (ds @ k)", "dq[r0:r1] = (ds @ k)"),
    ("dV with P not transposed", "dv += p.T @ do[r0:r1]", "dv += p @ do[r0:r1]"),
    ("dP uses K in place of V", "dp = do[r0:r1] @ v.T", "dp = do[r0:r1] @ k.T"),
    ("recurrence keeps the larger normalizer instead of their sum",
     "new_lse = np.logaddexp(acc_lse, tile_lse)", "new_lse = np.maximum(acc_lse, tile_lse)"),
    ("recurrence skips needed tiles", "if causal and keys[0] > rows[-1]:",
     "if causal and keys[0] > rows[0]:"),
    ("recurrence forgets the old output",
     "acc_o = keep_acc[:, None] * acc_o + keep_tile[:, None] * tile_o",
     "acc_o = keep_tile[:, None] * tile_o"),
    ("recurrence does not reweight the tile",
     "acc_o = keep_acc[:, None] * acc_o + keep_tile[:, None] * tile_o",
     "acc_o = keep_acc[:, None] * acc_o + tile_o"),
    ("tile output left unnormalized", "tile_o = (w @ v[keys]) / tot[:, None]",
     "tile_o = (w @ v[keys])"),
    ("merge weight inverted", "w_a = np.exp(lse_a - lse)[..., None]",
     "w_a = np.exp(lse - lse_a)[..., None]"),
]

ORACLE_NAMES = ["attention_forward", "attention_backward", "attention_forward_blockwise",
                "attention_probabilities", "merge_partials"]

# (pin function, kwargs) -- the parametrized pins of test_oracle.py, one set each.
PINS = [
    (T.test_golden_forward_hand_example, {}),
    (T.test_golden_backward_hand_example, {}),
    (T.test_brute_force_tiny, dict(n=5, d=2, causal=False)),
    (T.test_brute_force_tiny, dict(n=5, d=2, causal=True)),
    (T.test_rectangular_and_batched_shapes, {}),
    (T.test_rows_of_p_sum_to_one, dict(causal=True)),
    (T.test_identical_keys_give_mean_of_v, dict(causal=True)),
    (T.test_causal_row0_returns_v0, {}),
    (T.test_scale_zero_is_uniform_average, dict(causal=False)),
    (T.test_single_key, {}),
    (T.test_one_hot_dominant_score_selects_row, {}),
    (T.test_key_permutation_invariance_and_query_equivariance, {}),
    (T.test_key_shift_and_value_affinity, dict(causal=False)),
    (T.test_blockwise_online_softmax_equals_full, dict(causal=True, bq=7, bk=5)),
    (T.test_blockwise_online_softmax_equals_full, dict(causal=False, bq=16, bk=64)),
    (T.test_two_shard_merge_equals_full, {}),
    (T.test_gradients_match_finite_differences, dict(causal=False)),
    (T.test_gradient_invariants, dict(causal=True)),
    (T.test_matches_torch_cpu_float64_attention_and_autograd, dict(causal=True)),
    (T.test_brute_force_window_and_groups, dict(window=(2, 1), causal=False, hq=4, hkv=2)),
    (T.test_brute_force_window_and_groups, dict(window=(1, 0), causal=True, hq=2, hkv=1)),
    (T.test_window_closed_forms, {}),
    (T.test_grouped_heads_equal_repeated_heads_and_mqa_closed_form, {}),
    (T.test_window_gradients_match_finite_differences, dict(window=(2, 1))),
    (T.test_grouped_window_matches_torch_float64_and_autograd, dict(window=(5, 3), causal=False)),
    (T.test_block_mask_brute_force, dict(causal=True, n=7, mb=2)),
    (T.test_block_mask_brute_force, dict(causal=False, n=12, mb=4)),
    (T.test_all_ones_block_mask_equals_dense, {}),
    (T.test_block_diagonal_mask_is_attention_within_each_block, {}),
    (T.test_hidden_blocks_do_not_matter, {}),
    (T.test_block_mask_gradients_match_finite_differences, {}),
]


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "<oracle mutant>", "exec"), mod.__dict__)
    return mod


def _failures(mod, monkeypatch):
    for name in ORACLE_NAMES:
        monkeypatch.setattr(T, name, getattr(mod, name))
    failed = []
    for fn, kw in PINS:
        try:
            fn(**kw)
        except Exception:  # noqa: BLE001 -- any failure means the pin caught it
            failed.append(fn.__name__)
    return failed


def test_unmutated_copy_passes_every_pin(monkeypatch):
    mod = _mutant("ROW_CHUNK = 2048", "ROW_CHUNK = 2048")
    assert _failures(mod, monkeypatch) == []


@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(label, old, new, monkeypatch):
    assert _failures(_mutant(old, new), monkeypatch), f"no pin caught: {label}"

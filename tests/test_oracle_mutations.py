"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Each mutation replaces one small oracle helper through monkeypatching; the named pin
test must then fail.  This shows the pins are not vacuous: a dropped term, a wrong
index or sign, a transposed operand or a wrong tie rule anywhere in the oracle turns
at least one of them red.
"""
import numpy as np
import pytest

from oracle import blockwise, dense, select, sparse
import test_oracle_backward as tb
import test_oracle_blockwise as tw
import test_oracle_dense as td
import test_oracle_select_sparse as ts
import test_oracle_sink as tk
import test_oracle_bias as tbias
import test_oracle_dropout as tdrop


def _mut_gqa_modulo(monkeypatch):
    monkeypatch.setattr(dense, "kv_head_of", lambda hq, G: hq % G)
    monkeypatch.setattr(blockwise, "kv_head_of", lambda hq, G: hq % G)


def _mut_drop_scale(monkeypatch):
    monkeypatch.setattr(dense, "scores", lambda q, k, scale: q @ k.T)


def _mut_transposed_scores(monkeypatch):
    monkeypatch.setattr(dense, "scores", lambda q, k, scale: scale * (k @ q.T).T[::-1, ::-1])


def _mut_strict_causal(monkeypatch):
    orig = dense.visible

    def vis(q_pos, k_pos, causal, wl=-1, wr=-1):
        ok = orig(q_pos, k_pos, False, wl, wr)
        if causal:
            ok &= np.asarray(k_pos)[None, :] < np.asarray(q_pos)[:, None]
        return ok
    monkeypatch.setattr(dense, "visible", vis)


def _mut_window_exclusive(monkeypatch):
    orig = dense.visible

    def vis(q_pos, k_pos, causal, wl=-1, wr=-1):
        return orig(q_pos, k_pos, causal, wl - 1 if wl > 0 else wl, wr)
    monkeypatch.setattr(dense, "visible", vis)


def _mut_grad_sign(monkeypatch):
    monkeypatch.setattr(dense, "grad_scores", lambda P, dP, Di: P * (dP + Di[:, None]))


def _mut_grad_drop_d(monkeypatch):
    monkeypatch.setattr(dense, "grad_scores", lambda P, dP, Di: P * dP)


def _mut_correction_inverted(monkeypatch):
    monkeypatch.setattr(blockwise, "correction_factor", lambda prev, new: np.exp(new - prev))


def _mut_ties_to_higher_index(monkeypatch):
    monkeypatch.setattr(select, "rank_candidates",
                        lambda sc: sc.shape[1] - 1 - np.argsort(-sc[:, ::-1], axis=1, kind="stable"))


def _mut_window_off_by_one(monkeypatch):
    orig = sparse.candidate_positions

    def cand(t, sel_row, *, window, block_size, seqlen=None):
        return orig(t - 1, sel_row, window=window, block_size=block_size, seqlen=seqlen)
    monkeypatch.setattr(sparse, "candidate_positions", cand)


def _mut_clamp_to_last(monkeypatch):
    orig = sparse.candidate_positions

    def cand(t, sel_row, *, window, block_size, seqlen=None):
        pos, pad = orig(t, sel_row, window=window, block_size=block_size, seqlen=seqlen)
        n_w = window
        fixed = [p if (i < n_w or c >= 0) else block_size - 1
                 for i, (p, c) in enumerate(zip(pos, [0] * n_w + [c for c in sel_row for _ in range(block_size)]))]
        return np.asarray(fixed), pad
    monkeypatch.setattr(sparse, "candidate_positions", cand)


def _mut_sink_sign(monkeypatch):
    orig = dense._sink_weight
    monkeypatch.setattr(dense, "_sink_weight", lambda z, m, l: orig(None if z is None else -z, m, l))


def _mut_sink_in_log2_units(monkeypatch):
    orig = dense._sink_weight
    monkeypatch.setattr(dense, "_sink_weight",
                        lambda z, m, l: orig(None if z is None else z * 1.4426950408889634, m, l))


def _mut_clamped_slots_pass_no_gradient(monkeypatch):
    """The -1 clamp reads token 0, so token 0 must also collect those slots' gradients."""
    orig = sparse.candidate_positions

    def cand(t, sel_row, *, window, block_size, seqlen=None):
        pos, pad = orig(t, sel_row, window=window, block_size=block_size, seqlen=seqlen)
        neg = np.concatenate([np.zeros(window, bool), np.repeat(np.asarray(sel_row) < 0, block_size)])
        return pos, pad | neg
    monkeypatch.setattr(sparse, "candidate_positions", cand)


def _mut_bias_scaled_with_logits(monkeypatch):
    """The bias is added to the scaled logits, not scaled with them."""
    orig = dense._bias_rows
    monkeypatch.setattr(dense, "_bias_rows", lambda *a: orig(*a) / np.sqrt(8.0))


def _mut_dropout_ignored(monkeypatch):
    """The dropout array is read but never applied."""
    orig = dense._drop_rows
    monkeypatch.setattr(dense, "_drop_rows", lambda drop, b, h, rows, Skv: orig(None, b, h, rows, Skv))


def _mut_dropout_inverted(monkeypatch):
    """True read as kept instead of dropped."""
    orig = dense._drop_rows
    monkeypatch.setattr(dense, "_drop_rows", lambda drop, b, h, rows, Skv:
                        ~orig(drop, b, h, rows, Skv) if drop is not None else orig(drop, b, h, rows, Skv))


MUTATIONS = [
    (_mut_gqa_modulo, lambda: td.test_forward_matches_torch_sdpa(td.CASES[0])),
    (_mut_drop_scale, lambda: td.test_forward_matches_torch_sdpa(td.CASES[1])),
    (_mut_transposed_scores, lambda: td.test_forward_matches_torch_sdpa(td.CASES[1])),
    (_mut_strict_causal, td.test_window_zero_left_returns_own_value),
    (_mut_window_exclusive, td.test_zero_queries_average_visible_values),
    (_mut_grad_sign, lambda: tb.test_finite_differences(True, (-1, -1), 0, 0, 4)),
    (_mut_grad_drop_d, tb.test_gradient_sums),
    (_mut_correction_inverted, lambda: tw.test_ring_carry_equals_definition(4, 8, 8, True, (-1, -1), 8)),
    (_mut_ties_to_higher_index, ts.test_select_ties_go_to_lower_index),
    (_mut_window_off_by_one, ts.test_sparse_equals_materialised_candidate_list),
    (_mut_clamp_to_last, ts.test_sparse_zero_keys_closed_form),
    (_mut_sink_sign, tk.test_sink_with_zero_left_window_closed_form),
    (_mut_bias_scaled_with_logits, lambda: tbias.test_bias_matches_torch_sdpa_and_autograd((2, 4, 19, 19), True, (-1, -1))),
    (_mut_dropout_ignored, lambda: tdrop.test_dropout_matches_torch_sdpa_and_autograd((2, 4, 19, 19), True, (-1, -1))),
    (_mut_dropout_inverted, lambda: tdrop.test_dropout_matches_torch_sdpa_and_autograd((2, 4, 19, 19), True, (-1, -1))),
    (_mut_clamped_slots_pass_no_gradient, lambda: ts.test_sparse_backward_matches_autograd_of_materialised_list(8, 3)),
    (_mut_sink_in_log2_units, lambda: tk.test_sink_forward_and_backward_match_torch(True, (-1, -1), 2, 8)),
]


@pytest.mark.parametrize("mutate,pin", MUTATIONS, ids=[m.__name__ for m, _ in MUTATIONS])
def test_pin_catches_mutation(monkeypatch, mutate, pin):
    pin()                                   # green before the mutation
    mutate(monkeypatch)
    with pytest.raises(AssertionError):
        pin()

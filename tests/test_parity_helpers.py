"""The comparison helpers of tests/parity.py are not vacuous: a wrong result confined to
the late rows of a long causal sequence (whose outputs are small, |o_t| ~ 0.5/sqrt(t+1)
for the long-context inputs) passes the element bound and the whole-tensor Frobenius
bound, and must fail the per-(batch, head, row block) Frobenius bound."""
import numpy as np
import pytest

from parity import check_close


def decaying_output(B=1, S=4096, H=2, D=16, seed=0):
    g = np.random.default_rng(seed)
    t = np.arange(S, dtype=np.float64)[None, :, None, None]
    return g.standard_normal((B, S, H, D)) * 0.5 / np.sqrt(t + 1.0)


def test_late_block_error_is_caught_only_per_block():
    ref = decaying_output(S=131072)
    gpu = ref.copy()
    gpu[:, -4096:, 1] *= 1.2                        # 20 % off on the last block of one head
    # the element bound and the whole-tensor Frobenius bound alone would pass
    assert np.all(np.abs(gpu - ref) <= 2e-2 + 2.0 ** -8 * np.abs(ref))
    assert np.linalg.norm(gpu - ref) / np.linalg.norm(ref) <= 1e-2
    with pytest.raises(AssertionError, match="row block 31"):
        check_close("o", gpu, ref, "bf16", blocks=4096)


def test_sampled_rows_are_grouped_by_position():
    ref = decaying_output(S=512)
    rows = np.sort(np.random.default_rng(1).choice(131072, 512, replace=False))
    gpu = ref.copy()
    late = rows >= 65536
    gpu[:, late, 0] *= 0.7
    with pytest.raises(AssertionError, match="relative Frobenius"):
        check_close("o", gpu, ref, "bf16", blocks=4096, rows=rows)
    check_close("o", ref * (1 + 1e-4), ref, "bf16", blocks=4096, rows=rows)


def test_nan_entries_of_the_reference_are_skipped():
    ref = decaying_output(S=256)
    ref[:, 100:] = np.nan                           # rows the oracle did not evaluate
    gpu = np.where(np.isnan(ref), 123.0, ref)
    check_close("o", gpu, ref, "bf16", blocks=64)

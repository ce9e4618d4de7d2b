"""The decision rule of the bf16-bound selection, checked on the CPU against a full sort.

The GPU selection for up to 256 key blocks scores every candidate approximately, with
|s~ - s| <= Eb, and from the n-th and (n+1)-th largest approximate scores v_n >= v_n+1
(counted with multiplicity) decides: s~ > v_n+1 + 2 Eb is in the top n, s~ < v_n - 2 Eb
is out, the rest are ranked by their exact scores (then the lower index) to fill the
list.  This is a plain restatement of that rule in numpy, fed exact scores with
adversarial errors of up to Eb / 1.25 (the analytic bound: the kernel's Eb is 1.25 times
it, the room its own rounding of the thresholds needs) -- at that bound, random inside
it, and pushing near-ties apart or together -- and compared with the exact top n of a
stable sort.  It shares no
code with the kernel or the oracle; it pins the rule, not an implementation of it.
"""
import numpy as np
import pytest


def exact_top(s, n):
    order = sorted(range(len(s)), key=lambda c: (-s[c], c))   # score descending, lower index first
    return sorted(order[:n])


def rule_top(s, approx, eb, n):
    if len(s) <= n:
        return list(range(len(s)))
    srt = np.sort(approx)[::-1]
    vn, vn1 = srt[n - 1], srt[n]                               # with multiplicity
    hi, lo = vn1 + 2 * eb, vn - 2 * eb
    sure = [c for c in range(len(s)) if approx[c] > hi]
    und = [c for c in range(len(s)) if approx[c] <= hi and approx[c] >= lo]
    assert len(sure) <= n and len(sure) + len(und) >= n
    und.sort(key=lambda c: (-s[c], c))
    return sorted(sure + und[:n - len(sure)])


def perturb(s, eb, mode, rng):
    e = eb / 1.25                                            # the error the rule must tolerate
    if mode == "random":
        return s + rng.uniform(-e, e, size=s.shape)
    if mode == "edge":
        return s + e * rng.choice([-1.0, 1.0], size=s.shape)
    # push the larger of each near pair down and the smaller up (order flips inside the bound)
    med = np.median(s)
    return s + np.where(s > med, -e, e)


@pytest.mark.parametrize("mode", ["random", "edge", "squeeze"])
@pytest.mark.parametrize("n", [1, 3, 8, 16])
def test_rule_matches_sort(mode, n):
    rng = np.random.default_rng(1000 * n + len(mode))
    for trial in range(300):
        m = int(rng.integers(1, 257))
        kind = trial % 4
        if kind == 0:                                            # spread scores
            s = rng.normal(0.0, 4.0, size=m)
        elif kind == 1:                                          # near ties, inside the bound
            s = 1.0 + rng.integers(-3, 4, size=m) * 1e-4
        elif kind == 2:                                          # exact ties (integers)
            s = rng.integers(-2, 3, size=m).astype(np.float64)
        else:                                                    # a few groups of equal values
            s = rng.choice(rng.normal(0.0, 1.0, size=5), size=m)
        eb = float(rng.choice([1e-6, 1e-4, 1e-2, 0.5]))
        approx = perturb(s, eb, mode, rng)
        assert rule_top(s, approx, eb, n) == exact_top(s, n), (trial, m, kind, eb)


def test_rule_needs_the_full_margin():
    """A narrower margin goes wrong: candidate 0 is pushed up by the error bound and 1
    down, so 0 leads the approximate scores by half a bound although 1 is the top one; a
    margin under that half would declare 0 surely in, the rule's 2 Eb leaves both
    undecided and the exact scores pick 1."""
    eb = 1e-3
    s = np.array([1.0, 1.0 + 1.5 * eb])
    approx = s + np.array([eb, -eb])                     # 1 + eb, 1 + 0.5 eb
    n = 1
    assert exact_top(s, n) == [1]
    vn1 = np.sort(approx)[::-1][n]
    assert approx[0] > vn1 + 0.4 * eb                    # a 0.4 eb margin would keep 0
    assert rule_top(s, approx, eb, n) == [1]

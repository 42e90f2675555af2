"""Pins for the oracle's lenience variant and its throughput analytics.

Lenience (the Leviathan review, "Lenience"): q(x) is multiplied by l in the
acceptance decision; the page's guarantee is that no token is then sampled
with more than 1/l times its probability, and alpha grows as l falls; l = 1
is the exact method, whose output follows the target exactly.  The checks
integrate the oracle's decisions over the uniforms exactly (as the coupling
example's pin does).  The analytics are pinned to the review's printed table
(operations and speed at c = c_hat = 0) and figure readings."""
import json
import math
import os

import numpy as np
import pytest

from oracle import analytics
from oracle.verify import verify_sequence

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def logits_of(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


def one_step(target, draft_dist, x, u, lenience):
    zp = np.stack([logits_of(target), logits_of(target)])
    zq = np.stack([logits_of(draft_dist)])
    return verify_sequence(zp, zq, np.array([x], np.int32), np.asarray(u, np.float64), 1.0, 0, 1.0, 1, lenience)


def accept_measure(target, draft_dist, x, lenience):
    """Measure of u_1 in [0, 1) for which the oracle accepts draft x (bisection)."""
    acc = lambda u0: one_step(target, draft_dist, x, [u0, 0.5], lenience).n == 1
    if not acc(0.0):
        return 0.0
    hi = np.nextafter(1.0, 0.0)
    if acc(hi):
        return 1.0
    lo = 0.0
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        lo, hi = (mid, hi) if acc(mid) else (lo, mid)
    return 0.5 * (lo + hi)


def residual_measure(target, draft_dist, x, lenience, th):
    """Distribution of the token drawn after a rejection of x (integrated over u_res)."""
    u_rej = th + 0.5 * (1.0 - th)
    V = len(target)
    out = np.zeros(V)

    def tok(ur):
        return int(one_step(target, draft_dist, x, [u_rej, ur], lenience).tokens[0])

    def walk(lo, hi, depth=0):
        a, b = tok(lo), tok(np.nextafter(hi, 0.0))
        if a == b:
            out[a] += hi - lo
            return
        if depth > 60:
            out[a] += 0.5 * (hi - lo)
            out[b] += 0.5 * (hi - lo)
            return
        mid = 0.5 * (lo + hi)
        walk(lo, mid, depth + 1)
        walk(mid, hi, depth + 1)
    walk(0.0, 1.0)
    return out


def exact_output(target, draft_dist, lenience):
    V = len(target)
    out = np.zeros(V)
    acc_rate = 0.0
    for x in range(V):
        if draft_dist[x] == 0.0:
            continue
        th = accept_measure(target, draft_dist, x, lenience)
        out[x] += draft_dist[x] * th
        acc_rate += draft_dist[x] * th
        if th < 1.0:
            out += draft_dist[x] * (1.0 - th) * residual_measure(target, draft_dist, x, lenience, th)
    return out, acc_rate


CASES = [
    ([0.2, 0.5, 0.3], [0.6, 0.3, 0.1]),            # the worked coupling example (target, draft)
    ([0.05, 0.15, 0.4, 0.4], [0.4, 0.3, 0.2, 0.1]),
    ([0.7, 0.1, 0.1, 0.1, 0.0], [0.25, 0.25, 0.2, 0.1, 0.2]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_lenience_guarantee_and_rising_acceptance(case):
    p, q = map(np.asarray, CASES[case])
    prev = -1.0
    for l in (1.0, 0.7, 0.5, 0.3, 0.1, 0.0):
        out, acc = exact_output(p, q, l)
        assert abs(out.sum() - 1.0) < 1e-9
        if l == 1.0:
            assert np.abs(out - p).max() < 1e-9            # exact method: the target itself
            assert abs(acc - np.minimum(p, q).sum()) < 1e-9
        else:
            assert (out <= p / l + 1e-9).all() if l > 0 else True   # no token above 1/l of its probability
        # The acceptance rate is E_{x~q}[min(1, p(x) / (l q(x)))] = sum min(q, p / l).
        expect = float(np.minimum(q, p / l).sum()) if l > 0 else float(q[p > 0].sum())
        assert abs(acc - expect) < 1e-9, (l, acc, expect)
        assert acc >= prev - 1e-12                          # alpha grows as l falls
        prev = acc


def test_lenience_out_of_range_is_invalid():
    p, q = CASES[0]
    for l in (-0.1, 1.5, float("nan")):
        assert one_step(p, q, 0, [0.3, 0.5], l).n == -1


def test_analytics_match_the_review_table():
    table = gold("ops_speed_table.json")
    for alpha, gamma, ops, speed in table["rows"]:
        assert round(analytics.expected_tokens(alpha, gamma), 2) == pytest.approx(speed, abs=1e-9)
        assert round(analytics.speedup(alpha, gamma, 0.0), 2) == pytest.approx(speed, abs=1e-9)
        assert round(analytics.operations(alpha, gamma, 0.0), 2) == pytest.approx(ops, abs=1e-9)


def test_analytics_figure_readings():
    f = gold("tokens_per_round_figure.json")
    assert f["tokens_per_round_low"] <= analytics.expected_tokens(f["alpha"], f["gamma"]) <= f["tokens_per_round_high"]
    g = gold("optimal_gamma_example.json")
    assert analytics.optimal_gamma(g["alpha"], g["c"], 200) == g["optimal_gamma"]
    # Cheaper or better drafters favour longer drafts.
    assert analytics.optimal_gamma(0.9, 0.05, 200) < analytics.optimal_gamma(0.9, 0.01, 200)
    assert analytics.optimal_gamma(0.7, 0.01, 200) < analytics.optimal_gamma(0.9, 0.01, 200)
    assert analytics.optimal_gamma(0.5, 2.0, 200) == 1


def test_acceptance_length_by_simulation():
    # tau = 1 + sum_k prod_{i<=k} alpha_k with position-dependent acceptance:
    # simulate rounds that stop at the first rejection.
    rng = np.random.default_rng(5)
    alphas = [0.9, 0.8, 0.7, 0.6, 0.5]
    N = 200000
    acc = rng.random((N, len(alphas))) < np.array(alphas)[None, :]
    n = np.argmin(np.concatenate([acc, np.zeros((N, 1), bool)], axis=1), axis=1)
    tok = n + 1.0
    tau = analytics.acceptance_length(alphas)
    assert abs(tok.mean() - tau) < 4.5 * tok.std() / math.sqrt(N)
    # Constant alpha: tau is the expected-tokens law.
    assert abs(analytics.acceptance_length([0.8] * 5) - analytics.expected_tokens(0.8, 5)) < 1e-12

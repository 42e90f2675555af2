"""Pins for the K-SEQ / SpecTr oracle ("SpecTr: Fast Speculative Decoding
via Optimal Transport", mtandhj.com; that page calls the draft p and the
target q, here p is the target and q the draft).

Facts used: the output of K-SEQ follows the target exactly (section
"Residual distribution": A(x) + (1 - P_A) q_res(x) = target); the
candidates' direct mass A_rho*(x) = min(rho* q(x), p(x)) is never below the
single-candidate min(p, q) and never above the target; the naive repeat of
the single-candidate test overshoots (the page's 3/4 > 1/2 example) and
K-SEQ does not; the page's two-token example bounds the hit rate between the
single-candidate 0.7 and the optimal-transport 0.94; with one candidate the
method is the single-candidate test, and a SpecTr round with K = 1 is the
ordinary verify.  Exact integration runs over the oracle's own decisions
(thresholds found by bisection), not over re-typed formulas.

The SpecTr walk (section "SpecTr": candidates filtered by the output prefix,
the walk ends when the output misses the candidates) is pinned on its own
output: over candidate sets drawn from a prefix-dependent drafter, the
round's tokens, completed by fresh target draws where the round ended early,
must follow the target's chain p0(y1) p1(y2 | y1) p2(y3 | y1, y2), and every
round must obey the stop rule.  Planted mistakes in a copy of the walk (a
filter on the wrong depth, rows taken from the wrong candidate, no stop) must
fail the pin."""
import inspect
import itertools
import math
import multiprocessing as mp
import os
import textwrap

import numpy as np
import pytest
from scipy import stats

from oracle import kseq
from oracle.verify import verify_sequence


def logit(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


def threshold(f):
    """Measure of u in [0, 1) with f(u) True, for f true on an initial interval."""
    if not f(0.0):
        return 0.0
    hi = np.nextafter(1.0, 0.0)
    if f(hi):
        return 1.0
    lo = 0.0
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        lo, hi = (mid, hi) if f(mid) else (lo, mid)
    return 0.5 * (lo + hi)


def residual_measure(p, q, cands, u_rej):
    V = len(p)
    k = len(cands)
    out = np.zeros(V)

    def tok(ur):
        return kseq.kseq_position(p, q, cands, list(u_rej) + [ur]).token

    def walk(lo, hi, d=0):
        a, b = tok(lo), tok(np.nextafter(hi, 0.0))
        if a == b:
            out[a] += hi - lo
            return
        if d > 60:
            out[a] += 0.5 * (hi - lo)
            out[b] += 0.5 * (hi - lo)
            return
        m = 0.5 * (lo + hi)
        walk(lo, m, d + 1)
        walk(m, hi, d + 1)
    walk(0.0, 1.0)
    return out


def exact_kseq(p, q, k):
    """(output distribution, direct-acceptance mass per token, hit rate),
    integrating the oracle over the candidate tuples and every uniform."""
    V = len(p)
    out = np.zeros(V)
    direct = np.zeros(V)
    hit = 0.0
    for tup in itertools.product(range(V), repeat=k):
        w = float(np.prod([q[x] for x in tup]))
        if w == 0.0:
            continue
        cands = list(tup)
        reach = 1.0                      # probability that candidates before i were all rejected
        u_rej = []
        for i, x in enumerate(cands):
            def acc(ui, i=i):
                r = kseq.kseq_position(p, q, cands, u_rej + [ui] + [0.999999999] * (k - i - 1) + [0.5])
                return r.accepted == i
            a = threshold(acc)
            direct[x] += w * reach * a
            out[x] += w * reach * a
            hit += w * reach * a
            reach *= 1.0 - a
            u_rej.append(a + 0.5 * (1.0 - a) if a < 1.0 else 0.0)
            if reach == 0.0:
                break
        if reach > 0.0:
            res = residual_measure(p, q, cands, u_rej)
            out += w * reach * res
            hit += w * reach * res[sorted(set(cands))].sum()
    return out, direct, hit


CASES = [
    ([0.3, 0.7], [0.6, 0.4]),                       # the page's two-token example (target, draft)
    ([0.5, 0.5], [1.0, 0.0]),                       # the page's over-allocation example
    ([0.1, 0.2, 0.3, 0.4], [0.4, 0.3, 0.2, 0.1]),
    ([0.05, 0.6, 0.35, 0.0], [0.25, 0.25, 0.25, 0.25]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("k", [1, 2, 3])
def test_output_follows_the_target_exactly(case, k):
    p, q = map(np.asarray, CASES[case])
    out, direct, hit = exact_kseq(p, q, k)
    assert np.abs(out - p).max() < 1e-9, (out, p)
    assert (direct <= p + 1e-9).all()                             # never above the target's budget
    assert (direct >= np.minimum(p, q) - 1e-9).all()              # never below one candidate
    rho = kseq.rho_star(p, q, k)
    assert np.abs(direct - np.minimum(rho * q, p)).max() < 1e-9   # A_rho*(x) = min(rho* q, p)
    if k == 1:
        assert abs(hit - np.minimum(p, q).sum()) < 1e-9


def test_two_token_example_hit_rate_between_the_pages_bounds():
    p, q = np.array([0.3, 0.7]), np.array([0.6, 0.4])
    _, _, hit = exact_kseq(p, q, 2)
    assert 0.7 - 1e-12 <= hit <= 0.94 + 1e-12, hit
    assert hit > 0.7 + 1e-3                                       # two candidates help here


def test_naive_repeat_overshoots_and_kseq_does_not():
    # Draft puts all mass on A, target is (1/2, 1/2), two candidates (both A).
    p, q = np.array([0.5, 0.5]), np.array([1.0, 0.0])
    naive = 0.5 + 0.5 * 0.5
    assert naive == 0.75 > p[0]
    _, direct, _ = exact_kseq(p, q, 2)
    assert direct[0] <= p[0] + 1e-12


def test_rho_star_is_the_smallest_root():
    rng = np.random.default_rng(2)
    for _ in range(30):
        V = int(rng.integers(2, 12))
        p, q = rng.dirichlet(np.ones(V)), rng.dirichlet(np.ones(V))
        k = int(rng.integers(1, 9))
        r = kseq.rho_star(p, q, k)
        assert 1.0 <= r <= k
        g = lambda x: x * kseq.beta_of(p, q, x) - (1 - (1 - kseq.beta_of(p, q, x)) ** k)
        assert g(r) >= -1e-12
        if r > 1.0:
            assert g(r * (1 - 1e-9)) < 1e-9


def test_one_candidate_is_the_single_candidate_test():
    rng = np.random.default_rng(4)
    V = 6
    for _ in range(200):
        p, q = rng.dirichlet(np.ones(V)), rng.dirichlet(np.ones(V))
        x = int(rng.integers(0, V))
        u = rng.random(2)
        r = kseq.kseq_position(p, q, [x], u)
        zp = np.stack([logit(p), logit(p)])
        zq = np.stack([logit(q)])
        s = verify_sequence(zp, zq, np.array([x], np.int32), u, 1.0, 0, 1.0, 1)
        if s.margin > 1e-9:
            assert (r.accepted == 0) == (s.n == 1)
            assert r.token == (x if s.n == 1 else s.tokens[0])


def test_spectr_with_one_candidate_is_the_ordinary_verify():
    rng = np.random.default_rng(6)
    L, V = 4, 40
    for trial in range(40):
        zp = rng.normal(size=(L + 1, V)) * 2
        zq = zp[:L] + rng.normal(size=(L, V)) * 0.7
        T = float(rng.choice([0.0, 0.8, 1.2]))
        draft = rng.integers(0, V, size=L).astype(np.int32)
        draft[::2] = np.argmax(zq[::2], axis=1)
        u = rng.random(L + 1)
        s = verify_sequence(zp, zq, draft, u, T, 0, 1.0, L)
        us = np.zeros((L + 1, 2))
        us[:L, 0] = u[:L]
        us[:, 1] = u[L]
        us[L, 0] = u[L]
        r = kseq.spectr_sequence(zp[None], zq[None], draft[None], us, T, 0, 1.0)
        if min(s.margin, r.margin) > 1e-9:
            assert r.n == s.n and (r.tokens == s.tokens).all(), (trial, r, s.n, s.tokens)


def test_spectr_first_token_follows_the_target():
    rng = np.random.default_rng(8)
    K, L, V = 3, 2, 5
    zp1 = rng.normal(size=V) * 1.2
    p1 = np.exp(zp1 - zp1.max())
    p1 /= p1.sum()
    zq1 = zp1 + rng.normal(size=V)
    q1 = np.exp(zq1 - zq1.max())
    q1 /= q1.sum()
    N = 20000
    counts = np.zeros(V)
    for _ in range(N):
        cand = np.stack([rng.choice(V, size=L, p=q1) for _ in range(K)]).astype(np.int32)
        zp = np.broadcast_to(zp1, (K, L + 1, V)).copy()
        zq = np.broadcast_to(zq1, (K, L, V)).copy()
        r = kseq.spectr_sequence(zp, zq, cand, rng.random((L + 1, K + 1)), 1.0, 0, 1.0)
        counts[r.tokens[0]] += 1
    pv = stats.chisquare(counts, p1 * N).pvalue
    assert pv > 1e-4, pv


def test_rho_star_at_large_k_is_the_saturation_point():
    """For large k, (1 - beta)^k is below any rounding of rho beta - 1, so
    the root sits where every element saturates: for rho < r_max =
    max p/q, D(rho) = sum max(0, p - rho q) >= (r_max - rho) q(x_max) > 0,
    which exceeds (1 - beta)^k once r_max - rho > (1 - beta)^k / q(x_max).
    So rho* = r_max to far better than 1e-9 (it is never above r_max: there
    D = 0 and (1 - beta)^k > 0)."""
    rng = np.random.default_rng(7)
    checked = 0
    for trial in range(20):
        V = int(rng.integers(50, 600))
        q = rng.dirichlet(np.ones(V))
        p = q * np.exp(0.3 * rng.standard_normal(V))
        p /= p.sum()
        r_max = float((p / q).max())
        beta_rmax = kseq.beta_of(p, q, r_max)
        for k in (48, 64):
            if (1.0 - beta_rmax) ** k > 1e-15:
                continue
            rho = kseq.rho_star(p, q, k)
            assert abs(rho - r_max) <= 1e-9 * r_max, (trial, k, rho, r_max)
            checked += 1
    assert checked >= 10


# --------------------------------------------------------------------------
# The SpecTr walk beyond the first depth, K > 1.
# --------------------------------------------------------------------------
WV, WL = 3, 2
W_P0 = np.array([0.5, 0.3, 0.2])                                     # target at depth 0
W_P1 = np.array([[0.1, 0.2, 0.7], [0.6, 0.1, 0.3], [0.3, 0.6, 0.1]])  # target after y1
W_P2 = np.array([[np.roll([0.7, 0.2, 0.1], (a + 2 * b) % 3) for b in range(3)] for a in range(3)])  # after (y1, y2)
W_Q0 = np.array([0.2, 0.5, 0.3])                                     # drafter at depth 0
W_Q1 = np.array([np.roll([0.5, 0.3, 0.2], a) for a in range(3)])      # drafter after y1

# Planted mistakes: (text in the walk, replacement).
WALK_MUTATIONS = {
    "filter on the first depth": ("if int(cand[c, j]) == r.token", "if int(cand[c, 0]) == r.token"),
    "rows of candidate 0": ("c0 = alive[0]", "c0 = 0"),
    "no stop when the output misses": ("        if not alive:\n            return SpecTrResult(out, j, margin)",
                                       "        if not alive:\n            alive = list(range(K))"),
}


def _walk(mutation):
    if mutation is None:
        return kseq.spectr_sequence
    src = textwrap.dedent(inspect.getsource(kseq.spectr_sequence))
    old, new = WALK_MUTATIONS[mutation]
    assert old in src, mutation
    ns = dict(vars(kseq))
    exec(compile(src.replace(old, new, 1), "<planted mistake>", "exec"), ns)
    return ns["spectr_sequence"]


def _walk_rounds(args):
    """Counts of the completed (y1, y2, y3) and the number of rounds that
    break the stop rule, over n rounds."""
    mutation, K, seed, n = args
    walk = _walk(mutation)
    rng = np.random.default_rng(seed)
    counts = np.zeros((WV, WV, WV))
    broken = 0
    for _ in range(n):
        first = rng.choice(WV, size=K, p=W_Q0)
        cand = np.stack([first, [rng.choice(WV, p=W_Q1[a]) for a in first]], axis=1).astype(np.int32)
        # Row j of candidate c: the model after c's first j tokens.
        zp = np.stack([np.stack([logit(W_P0), logit(W_P1[a]), logit(W_P2[a, b])]) for a, b in cand])
        zq = np.stack([np.stack([logit(W_Q0), logit(W_Q1[a])]) for a, b in cand])
        r = walk(zp, zq, cand, rng.random((WL + 1, K + 1)), 1.0, 0, 1.0)
        y = [int(t) for t in r.tokens[: r.n + 1]]
        # Stop rule: every output before the last continues a candidate
        # prefix; a round that ended before depth L ended on an output that
        # is not one.
        prefixes = {tuple(int(t) for t in cand[c, :j]) for c in range(K) for j in range(1, WL + 1)}
        ok = len(y) == r.n + 1 and all(tuple(y[: j + 1]) in prefixes for j in range(r.n))
        if r.n < WL:
            ok = ok and tuple(y) not in prefixes
        broken += not ok
        # The next rounds would continue from the target: complete with it.
        if len(y) < 2:
            y.append(int(rng.choice(WV, p=W_P1[y[0]])))
        if len(y) < 3:
            y.append(int(rng.choice(WV, p=W_P2[y[0], y[1]])))
        counts[tuple(y)] += 1
    return counts, broken


def walk_law(mutation, K, rounds, seed):
    """(chi-square p-value of the completed outputs against the target's
    chain, rounds breaking the stop rule)."""
    chunks = 8
    args = [(mutation, K, seed * 100 + c, rounds // chunks) for c in range(chunks)]
    with mp.get_context("fork").Pool(min(chunks, os.cpu_count() or 1)) as pool:
        parts = pool.map(_walk_rounds, args)
    counts = sum(c for c, _ in parts)
    broken = sum(b for _, b in parts)
    expected = W_P0[:, None, None] * W_P1[:, :, None] * W_P2 * counts.sum()
    return stats.chisquare(counts.ravel(), expected.ravel()).pvalue, broken


@pytest.mark.parametrize("K", [2, 3])
def test_spectr_walk_follows_the_target_chain(K):
    pv, broken = walk_law(None, K, 24000, seed=K)
    assert broken == 0
    assert pv > 1e-4, pv


@pytest.mark.parametrize("mutation", sorted(WALK_MUTATIONS))
def test_spectr_walk_pin_rejects_planted_mistakes(mutation):
    for K in (2, 3):
        pv, broken = walk_law(mutation, K, 8000, seed=10 + K)
        assert broken > 0 or pv < 1e-8, (mutation, K, pv, broken)

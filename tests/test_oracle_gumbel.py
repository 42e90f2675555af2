"""Pins for the shared-noise (Gumbel coupling) verify of the CPU oracle.

Facts used ("Speculative Decoding: the art of guessing well", section
"Sampling with shared noise"): argmax of logits plus Gumbel noise samples the
softmax; with the noise shared, the drafter's and the target's samples agree
with probability sum_j 1 / sum_i max(p(i)/p(j), q(i)/q(j)), at least
(1 - TV) / (1 + TV); with independent noise they agree with probability
sum_i p(i) q(i); the output is the target's own sample under that noise,
whatever the drafter; greedy decoding is the T = 0 case.  The decision
margin (the best two scores' gap relative to the size of their terms) is
pinned by float32 scoring computed here: outside the margin it picks the
oracle's token at every temperature, and a planted mistake in the margin
fails that pin.  None of these tests re-types the oracle's own code path."""
import inspect
import json
import math
import os
import textwrap

import numpy as np
from scipy import stats

import oracle
from oracle import verify as verify_mod
from oracle.verify import gumbel_target_token, gumbel_verify_sequence, verify_sequence

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gumbel(rng, shape):
    return (-np.log(-np.log(rng.random(shape).clip(1e-300, 1 - 1e-16)))).astype(np.float32)


def logit(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


def match_closed_form(p, q):
    """The page's agreement probability of two Gumbel-max samples under shared noise."""
    p, q = np.asarray(p, float), np.asarray(q, float)
    tot = 0.0
    for j in range(len(p)):
        if p[j] > 0 and q[j] > 0:
            with np.errstate(divide="ignore"):
                tot += 1.0 / np.maximum(p / p[j], q / q[j]).sum()
    return tot


def test_closed_form_on_the_coupling_example_respects_the_bound():
    # The worked coupling example (draft (0.6, 0.3, 0.1), target (0.2, 0.5, 0.3)):
    # TV = 0.4, so the page's bound is 0.6 / 1.4.
    ex = json.load(open(os.path.join(GOLD, "coupling_example.json")))
    p, q = ex["target"], ex["draft"]
    tv = 0.5 * np.abs(np.subtract(p, q)).sum()
    assert abs(tv - 0.4) < 1e-12
    m = match_closed_form(p, q)
    assert (1 - tv) / (1 + tv) - 1e-12 <= m <= 1 - tv + 1e-12


def _match_rate(p, q, n, seed, shared=True, T=1.0):
    rng = np.random.default_rng(seed)
    zp, zq = logit(p), logit(q)
    hits = 0
    for _ in range(n):
        g = gumbel(rng, len(p))
        gq = g if shared else gumbel(rng, len(p))
        tp, _ = gumbel_target_token(zp, g, T, 0, 1.0)
        tq, _ = gumbel_target_token(zq, gq, T, 0, 1.0)
        hits += tp == tq
    return hits / n


def test_shared_noise_match_rate_equals_closed_form():
    ex = json.load(open(os.path.join(GOLD, "coupling_example.json")))
    p, q = ex["target"], ex["draft"]
    n = 40000
    rate = _match_rate(p, q, n, seed=1)
    m = match_closed_form(p, q)
    assert abs(rate - m) < 4.5 * math.sqrt(m * (1 - m) / n), (rate, m)


def test_shared_noise_match_rate_random_distributions():
    rng = np.random.default_rng(3)
    for trial in range(3):
        p = rng.dirichlet(np.ones(6))
        q = rng.dirichlet(np.ones(6))
        n = 20000
        rate = _match_rate(p, q, n, seed=10 + trial)
        m = match_closed_form(p, q)
        tv = 0.5 * np.abs(p - q).sum()
        assert (1 - tv) / (1 + tv) <= m + 1e-12
        assert abs(rate - m) < 4.5 * math.sqrt(m * (1 - m) / n), (trial, rate, m)


def test_independent_noise_match_rate_is_sum_pq():
    ex = json.load(open(os.path.join(GOLD, "coupling_example.json")))
    p, q = np.array(ex["target"]), np.array(ex["draft"])
    n = 40000
    rate = _match_rate(p, q, n, seed=2, shared=False)
    m = float((p * q).sum())
    assert abs(rate - m) < 4.5 * math.sqrt(m * (1 - m) / n), (rate, m)


def test_gumbel_max_samples_the_processed_softmax():
    # Temperature, top-k and top-p change the law exactly as the processed
    # distribution says: chi-square against softmax(z / T) restricted to the
    # support and renormalised.
    rng = np.random.default_rng(4)
    z = np.array([1.2, 0.3, -0.5, 2.0, 0.9, -1.4, 0.1, 1.5])
    for T, k, tp in ((1.0, 0, 1.0), (0.6, 0, 1.0), (1.7, 5, 1.0), (1.0, 0, 0.7), (0.8, 6, 0.85)):
        n = 30000
        counts = np.zeros(len(z))
        for _ in range(n):
            t, _ = gumbel_target_token(z, gumbel(rng, len(z)), T, k, tp)
            counts[t] += 1
        s = z / T
        keep = np.ones(len(z), bool)
        if 0 < k < len(z):
            keep &= s >= np.sort(s)[::-1][k - 1]
        w = np.where(keep, np.exp(s - s.max()), 0.0)
        if tp < 1.0:
            order = np.argsort(-s)
            c = np.cumsum((w / w.sum())[order])
            cut = order[: int(np.searchsorted(c, tp)) + 1]
            keep2 = np.zeros(len(z), bool)
            keep2[cut] = True
            w = np.where(keep2, w, 0.0)
        prob = w / w.sum()
        assert counts[prob == 0].sum() == 0, (T, k, tp)
        sel = prob > 0
        pv = stats.chisquare(counts[sel], prob[sel] * n).pvalue
        assert pv > 1e-4, (T, k, tp, pv)


def test_tokens_per_round_law_under_shared_noise():
    # Identical (p, q) at every position, fresh noise per position: positions
    # agree independently with the closed-form probability m, so the mean
    # number of tokens per round is (1 - m^(gamma+1)) / (1 - m).
    rng = np.random.default_rng(6)
    p = np.array([0.5, 0.3, 0.15, 0.05])
    q = np.array([0.35, 0.4, 0.05, 0.2])
    m = match_closed_form(p, q)
    G, N = 4, 6000
    zp = np.tile(logit(p), (G + 1, 1))
    zq = np.tile(logit(q), (G, 1))
    tot = []
    for _ in range(N):
        g = gumbel(rng, (G + 1, 4))
        draft = np.array([gumbel_target_token(zq[i], g[i], 1.0, 0, 1.0)[0] for i in range(G)], np.int32)
        r = gumbel_verify_sequence(zp, g, draft, 1.0, 0, 1.0, G)
        tot.append(r.n + 1)
    tot = np.array(tot, float)
    expect = (1 - m ** (G + 1)) / (1 - m)
    assert abs(tot.mean() - expect) < 4.5 * tot.std() / math.sqrt(N), (tot.mean(), expect)


def test_output_is_the_targets_own_sample_for_any_drafter():
    rng = np.random.default_rng(7)
    G, V = 5, 50
    zp = rng.normal(size=(G + 1, V)) * 2
    g = gumbel(rng, (G + 1, V))
    targets = None
    for sigma in (0.0, 0.3, 1.0, 3.0):
        zq = zp[:G] + sigma * rng.normal(size=(G, V))
        draft = np.array([gumbel_target_token(zq[i], g[i], 0.9, 0, 1.0)[0] for i in range(G)], np.int32)
        r = gumbel_verify_sequence(zp, g, draft, 0.9, 0, 1.0, G)
        assert (r.tokens[: r.n + 1] == r.target[: r.n + 1]).all()
        if sigma == 0.0:
            assert r.n == G                      # a drafter equal to the target is always right
        if targets is None:
            targets = r.target.copy()
        assert (r.target == targets).all()       # the target's samples do not depend on the drafter


def test_greedy_is_exact_matching():
    rng = np.random.default_rng(8)
    G, V = 4, 30
    for trial in range(50):
        zp = rng.integers(-3, 4, size=(G + 1, V)).astype(float)
        zq = zp[:G] + rng.integers(-1, 2, size=(G, V))
        draft = rng.integers(0, V, size=G).astype(np.int32)
        draft[::2] = np.argmax(zq[::2], axis=1)
        g = gumbel(rng, (G + 1, V))
        a = gumbel_verify_sequence(zp, g, draft, 0.0, 0, 1.0, G)
        b = verify_sequence(zp, zq, draft, np.full(G + 1, 0.5), 0.0, 0, 1.0, G)
        assert a.n == b.n and (a.tokens == b.tokens).all(), trial


def float32_sample(z, g, T, kept):
    """The argmax, lowest id on ties, of the score T (z / T + g) formed in
    float32 as fl(z + fl(T g)): the same decision at another precision."""
    sc = (np.float32(z) + (np.float32(T) * np.asarray(g, np.float32)).astype(np.float32)).astype(np.float32)
    return int(np.argmax(np.where(kept, sc, np.float32(-np.inf))))


def margin_pin_disagreements(token_fn, seed=21, rows=1200):
    """Rows where float32 scoring picks another token although the margin
    says the decision is not near (margin >= 1e-5), and the near count.
    Half the rows have a tied maximum: at tiny T the noise then decides
    between values that float32 can hardly tell apart."""
    rng = np.random.default_rng(seed)
    bad = near = 0
    for r in range(rows):
        V = int(rng.integers(50, 2000))
        z = np.round(rng.normal(size=V) * 3 * 128) / 128            # bf16-like values: many ties
        if r % 2:
            z[int(rng.integers(V))] = z.max()
        g = gumbel(rng, V)
        T = float(rng.choice([1e-7, 1e-6, 1e-5, 1e-3, 0.6, 1.0, 1.4, 50.0]))
        k = int(rng.choice([0, 0, 40]))
        tp = float(rng.choice([1.0, 1.0, 0.9]))
        t, m = token_fn(z, g, T, k, tp)
        kept = oracle.process(z, T, k, tp).kept
        if m < 1e-5:
            near += 1
        elif float32_sample(z, g, T, kept) != t:
            bad += 1
    return bad, near


def test_margin_covers_float32_scoring():
    bad, near = margin_pin_disagreements(gumbel_target_token)
    assert bad == 0
    assert near < 300          # mostly rows at T <= 1e-5 with a tied maximum, and top-p boundaries


def test_margin_pin_rejects_an_unscaled_gap():
    src = textwrap.dedent(inspect.getsource(verify_mod.gumbel_target_token))
    old = "gap = (sc[t] - sc[t2]) / max(1.0, size(t), size(t2))"
    assert old in src
    ns = dict(vars(verify_mod))
    exec(compile(src.replace(old, "gap = sc[t] - sc[t2]"), "<planted mistake>", "exec"), ns)
    bad, _ = margin_pin_disagreements(ns["gumbel_target_token"])
    assert bad > 0


def test_margin_of_a_tie_and_of_a_single_survivor():
    z = np.array([1.0, 3.0, 3.0, -2.0])
    g = np.zeros(4, np.float32)
    t, m = gumbel_target_token(z, g, 1.0, 0, 1.0)
    assert t == 1 and m == 0.0                 # an exact tie: lowest id, no margin
    t, m = gumbel_target_token(z, g, 1.0, 1, 1.0)
    assert t == 1 and m == 0.0                 # top-1 keeps both tied values
    t, m = gumbel_target_token(np.array([1.0, 3.0, 2.0]), g[:3], 1.0, 1, 1.0)
    assert t == 1 and m == math.inf            # one survivor: nothing to decide
    t, m = gumbel_target_token(z, g, 0.0, 0, 1.0)
    assert t == 1 and m == math.inf            # greedy: exact on the logits


def test_ties_go_to_the_lowest_id_and_bad_inputs_are_flagged():
    z = np.zeros((2, 6))
    g = np.zeros((2, 6), np.float32)
    g[:, 2] = g[:, 4] = 1.0
    r = gumbel_verify_sequence(z, g, np.array([2], np.int32), 1.0, 0, 1.0, 1)
    assert r.target[0] == 2 and r.n == 1 and r.tokens[1] == 2
    g2 = g.copy()
    g2[1, 3] = np.nan
    assert gumbel_verify_sequence(z, g2, np.array([2], np.int32), 1.0, 0, 1.0, 1).n == -1
    # Off the support (top-k 1 keeps only id 0 of a strictly decreasing row) the noise is never used.
    zd = np.tile(-np.arange(6.0), (2, 1))
    g3 = np.zeros((2, 6), np.float32)
    g3[:, 3] = np.nan
    assert gumbel_verify_sequence(zd, g3, np.array([0], np.int32), 1.0, 1, 1.0, 1).n == 1
    assert gumbel_verify_sequence(zd, g3, np.array([0], np.int32), 1.0, 4, 1.0, 1).n == -1
    assert gumbel_verify_sequence(z, g2, np.array([0], np.int32), 0.0, 0, 1.0, 1).n == 1   # noise unused at T = 0
    assert gumbel_verify_sequence(z, g, np.array([6], np.int32), 1.0, 0, 1.0, 1).n == -1
    z2 = z.copy()
    z2[0, 1] = np.nan
    assert gumbel_verify_sequence(z2, g, np.array([2], np.int32), 1.0, 0, 1.0, 1).n == -1

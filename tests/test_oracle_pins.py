"""Pins for the CPU oracle: values and laws that the pages and the mathematics
fix, checked against the oracle's outputs.  None of these re-types the
oracle's own formula: they use the pages' printed numbers, exact integration
over the uniforms, brute-force definitions on tiny inputs, distributional
tests and special cases that reduce to a textbook routine."""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle.verify import process, inverse_cdf, verify_sequence, verify_batch, decode_row

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def logits_of(p):
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p)


def one_step(target_rows, draft_rows, draft, u, T=1.0, k=0, top_p=1.0, gamma_b=None):
    zp = np.stack([logits_of(r) for r in target_rows])
    zq = np.stack([logits_of(r) for r in draft_rows])
    g = zq.shape[0] if gamma_b is None else gamma_b
    return verify_sequence(zp, zq, np.asarray(draft, np.int32), np.asarray(u, np.float64), T, k, top_p, g)


def accept_threshold(target, draft_dist, x):
    """Bisection on u_1 for the point where the oracle stops accepting draft x
    (gamma = 1).  Returns the measure of accepting uniforms."""
    def acc(u0):
        return one_step([target, target], [draft_dist], [x], [u0, 0.5]).n == 1
    if not acc(0.0):
        return 0.0
    hi = np.nextafter(1.0, 0.0)
    if acc(hi):
        return 1.0
    lo = 0.0
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        if acc(mid):
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def token_intervals(f, lo=0.0, hi=None, depth=0):
    """Measure of u in [lo, hi) mapped to each value of a monotone step function f."""
    if hi is None:
        hi = 1.0
    hi_in = np.nextafter(hi, 0.0)
    a, b = f(lo), f(hi_in)
    if a == b:
        return {a: hi - lo}
    if depth > 60 or hi - lo < 1e-15:
        return {a: 0.5 * (hi - lo), b: 0.5 * (hi - lo)}
    mid = 0.5 * (lo + hi)
    out = token_intervals(f, lo, mid, depth + 1)
    for t, m in token_intervals(f, mid, hi, depth + 1).items():
        out[t] = out.get(t, 0.0) + m
    return out


def exact_output_distribution(target, draft_dist, bonus):
    """P(first emitted token = y) for gamma = 1, integrating the oracle's
    piecewise-constant decisions over both uniforms exactly."""
    V = len(target)
    out = np.zeros(V)
    for x in range(V):
        if draft_dist[x] == 0.0:
            continue
        th = accept_threshold(target, draft_dist, x)
        out[x] += draft_dist[x] * th
        if th < 1.0:
            u_rej = max(th, 0.0) + 0.5 * (1.0 - max(th, 0.0))

            def tok(ur, x=x, u_rej=u_rej):
                return int(one_step([target, bonus], [draft_dist], [x], [u_rej, ur]).tokens[0])
            for y, m in token_intervals(tok).items():
                out[y] += draft_dist[x] * (1.0 - th) * m
    return out


# ----------------------------------------------------------------------------
# P1: the worked coupling example.
# ----------------------------------------------------------------------------
def test_worked_coupling_example():
    g = gold("coupling_example.json")
    q = np.array(g["draft"])
    p = np.array(g["target"])
    pr = process(logits_of(p), 1.0, 0, 1.0).prob
    assert np.allclose(pr, p, atol=1e-15)
    res = one_step([p, p], [q], [0], [0.0, 0.5])
    assert abs(res.alpha[0] - g["diagonal_total"]) < 1e-12
    # Acceptance measure per draft token, then the residual on rejection.
    coupling = np.zeros((3, 3))
    for x in range(3):
        th = accept_threshold(p, q, x)
        coupling[x, x] += q[x] * th
        if th < 1.0:
            u_rej = th + 0.5 * (1 - th)

            def tok(ur, x=x, u_rej=u_rej):
                return int(one_step([p, p], [q], [x], [u_rej, ur]).tokens[0])
            for y, m in token_intervals(tok).items():
                coupling[x, y] += q[x] * (1 - th) * m
    assert np.allclose(coupling, np.array(g["optimal_coupling_rows_draft_cols_output"]), atol=1e-12)
    assert abs(coupling.trace() - g["diagonal_total"]) < 1e-12
    assert abs(coupling[0, 1:].sum() - g["leftover_draft_row_A"]) < 1e-12
    assert np.allclose(coupling[0, 1:], g["missing_target_B_C"], atol=1e-12)
    assert np.allclose(coupling.sum(axis=0), p, atol=1e-12)   # output marginal is the target


def test_two_token_overlap_example():
    g = gold("two_token_example.json")
    res = one_step([g["target"], g["target"]], [g["draft"]], [0], [0.0, 0.5])
    assert abs(res.alpha[0] - g["single_candidate_acceptance"]) < 1e-12


# ----------------------------------------------------------------------------
# P3: alpha = 1 - sum max(0, p-q) = sum min(p,q) = 1 - TV(p, q).
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(5))
def test_alpha_identities(seed):
    rng = np.random.default_rng(seed)
    V = 50
    zp = rng.normal(size=(2, V)) * 2
    zq = zp[:1] + rng.normal(size=(1, V))
    res = verify_sequence(zp, zq, np.array([3], np.int32), np.array([0.3, 0.6]), 0.9, 0, 1.0, 1)
    p = np.exp(zp[0] / 0.9) / np.exp(zp[0] / 0.9).sum()
    q = np.exp(zq[0] / 0.9) / np.exp(zq[0] / 0.9).sum()
    tv = 0.5 * np.abs(p - q).sum()
    assert abs(res.alpha[0] - (1 - tv)) < 1e-12
    # The acceptance probability averaged over x ~ q is the same number.
    acc = sum(q[x] * accept_threshold(p, q, x) for x in range(V))
    assert abs(acc - res.alpha[0]) < 1e-10


# ----------------------------------------------------------------------------
# P4: the output follows the target for any draft.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(4))
def test_output_is_target_exact_integration(seed):
    rng = np.random.default_rng(100 + seed)
    V = 5
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V) * 0.5)
    if seed == 3:
        q[1] = 0.0      # drafter leaves out a token the target keeps
        q /= q.sum()
    bonus = rng.dirichlet(np.ones(V))
    out = exact_output_distribution(p, q, bonus)
    assert np.allclose(out, p, atol=1e-10), (out, p)


def _draw(dist, u):
    return int(np.searchsorted(np.cumsum(dist), u * np.sum(dist), side="right"))


def _run_batch(zp, zq, draft, u, T=1.0, k=0, top_p=1.0, gamma=None):
    N = draft.shape[0]
    G = zq.shape[0]
    Pb = np.broadcast_to(zp, (N,) + zp.shape)
    Qb = np.broadcast_to(zq, (N,) + zq.shape)
    gl = np.full(N, G if gamma is None else gamma, np.int32)
    return verify_batch(Pb, Qb, draft, u, np.full(N, T), np.full(N, k, np.int32), np.full(N, top_p), gl)


@pytest.mark.slow
def test_output_is_target_chi_square():
    rng = np.random.default_rng(7)
    V, G, N = 8, 2, 60000
    zp = rng.normal(size=(G + 1, V)) * 1.5
    zq = zp[:G] + rng.normal(size=(G, V)) * 1.2
    P = np.stack([process(zp[j], 1.0, 0, 1.0).prob for j in range(G + 1)])
    Q = np.stack([process(zq[i], 1.0, 0, 1.0).prob for i in range(G)])
    ud = rng.random((N, G))
    draft = np.array([[_draw(Q[i], ud[n, i]) for i in range(G)] for n in range(N)], np.int32)
    u = rng.random((N, G + 1))
    r = _run_batch(zp, zq, draft, u)
    first = r.tokens[:, 0]
    obs = np.bincount(first, minlength=V)
    assert stats.chisquare(obs, P[0] * N).pvalue > 1e-4
    sel = r.n >= 1
    second = r.tokens[sel, 1]
    obs2 = np.bincount(second, minlength=V)
    assert stats.chisquare(obs2, P[1] * sel.sum()).pvalue > 1e-4


# ----------------------------------------------------------------------------
# P5 / P6: tokens per round.
# ----------------------------------------------------------------------------
def _overlap_pair(alpha, V=4):
    """Target and draft with overlap exactly alpha: shared mass alpha on
    token 0, the rest on disjoint tokens."""
    p = np.zeros(V)
    q = np.zeros(V)
    p[0] = q[0] = alpha
    p[1] = 1 - alpha
    q[2] = 1 - alpha
    return p, q


@pytest.mark.slow
def test_tokens_per_round_matches_page_table():
    table = gold("ops_speed_table.json")
    rng = np.random.default_rng(11)
    N = 6000
    for alpha, gamma, _ops, speed in table["rows"]:
        p, q = _overlap_pair(alpha)
        zp = np.stack([logits_of(p)] * (gamma + 1))
        zq = np.stack([logits_of(q)] * gamma)
        draft = np.where(rng.random((N, gamma)) < alpha, 0, 2).astype(np.int32)
        u = rng.random((N, gamma + 1))
        r = _run_batch(zp, zq, draft, u)
        assert (r.alpha[:, :gamma] - alpha).__abs__().max() < 1e-12
        tok = r.n + 1.0
        sem = tok.std(ddof=1) / math.sqrt(N)
        assert abs(tok.mean() - speed) < 4 * sem + 0.005, (alpha, gamma, tok.mean(), speed)


@pytest.mark.slow
def test_tokens_per_round_figure_reading():
    f = gold("tokens_per_round_figure.json")
    rng = np.random.default_rng(12)
    N = 6000
    alpha, gamma = f["alpha"], f["gamma"]
    p, q = _overlap_pair(alpha)
    zp = np.stack([logits_of(p)] * (gamma + 1))
    zq = np.stack([logits_of(q)] * gamma)
    draft = np.where(rng.random((N, gamma)) < alpha, 0, 2).astype(np.int32)
    r = _run_batch(zp, zq, draft, rng.random((N, gamma + 1)))
    mean = (r.n + 1.0).mean()
    assert f["tokens_per_round_low"] <= mean <= f["tokens_per_round_high"]


@pytest.mark.slow
def test_acceptance_length_position_dependent():
    rng = np.random.default_rng(13)
    alphas = [0.9, 0.8, 0.7, 0.55, 0.4]
    G = len(alphas)
    N = 20000
    pairs = [_overlap_pair(a, V=4) for a in alphas]
    zp = np.stack([logits_of(p) for p, _ in pairs] + [logits_of(pairs[0][0])])
    zq = np.stack([logits_of(q) for _, q in pairs])
    draft = np.stack([np.where(rng.random(N) < a, 0, 2) for a in alphas], axis=1).astype(np.int32)
    r = _run_batch(zp, zq, draft, rng.random((N, G + 1)))
    # P(n >= k) = prod_{i <= k} alpha_i  =>  histogram of n.
    surv = np.concatenate([[1.0], np.cumprod(alphas)])
    pmf = surv[:-1] - surv[1:]
    pmf = np.append(pmf, surv[-1])
    obs = np.bincount(r.n, minlength=G + 1)
    assert stats.chisquare(obs, pmf * N).pvalue > 1e-4
    tau = 1 + np.cumprod(alphas).sum()
    assert abs((r.n + 1.0).mean() - tau) < 4 * (r.n.std() / math.sqrt(N))


# ----------------------------------------------------------------------------
# P7: greedy decoding is exact prefix matching.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(20))
def test_greedy_prefix_matching(seed):
    rng = np.random.default_rng(200 + seed)
    V, G = 6, 4
    zp = rng.integers(-3, 4, size=(G + 1, V)).astype(np.float64)   # integer logits: ties happen
    zq = rng.integers(-3, 4, size=(G, V)).astype(np.float64)
    draft = rng.integers(0, V, size=G).astype(np.int32)
    am = [min(np.nonzero(zp[j] == zp[j].max())[0]) for j in range(G + 1)]
    if seed % 3 == 0:
        draft[:2] = am[:2]
    n_bf = 0
    while n_bf < G and draft[n_bf] == am[n_bf]:
        n_bf += 1
    res = verify_sequence(zp, zq, draft, rng.random(G + 1), 0.0, 0, 1.0, G)
    assert res.n == n_bf
    assert list(res.tokens[:n_bf]) == list(draft[:n_bf])
    assert res.tokens[n_bf] == am[n_bf]
    amq = [min(np.nonzero(zq[i] == zq[i].max())[0]) for i in range(G)]
    assert list(res.alpha) == [1.0 if am[i] == amq[i] else 0.0 for i in range(G)]


# ----------------------------------------------------------------------------
# P8: special cases.
# ----------------------------------------------------------------------------
def test_identical_distributions_accept_everything():
    rng = np.random.default_rng(5)
    V, G = 16, 5
    zp = rng.normal(size=(G + 1, V))
    zq = zp[:G].copy()
    P = [process(zp[j], 1.0, 0, 1.0).prob for j in range(G + 1)]
    for trial in range(20):
        draft = np.array([_draw(P[i], rng.random()) for i in range(G)], np.int32)
        u = rng.random(G + 1)
        res = verify_sequence(zp, zq, draft, u, 1.0, 0, 1.0, G)
        assert res.n == G
        assert np.allclose(res.alpha[:G], 1.0, atol=1e-12)
        assert res.tokens[G] == _draw(P[G], u[G])


def test_disjoint_supports_reject_first():
    V, G = 6, 3
    p = np.array([0.5, 0.5, 0, 0, 0, 0.0])
    q = np.array([0, 0, 0.2, 0.3, 0.5, 0.0])
    zp = np.stack([logits_of(p)] * (G + 1))
    zq = np.stack([logits_of(q)] * G)
    for ur in (0.1, 0.7):
        res = verify_sequence(zp, zq, np.array([3, 2, 4], np.int32), np.array([0.2, 0.3, 0.4, ur]), 1.0, 0, 1.0, G)
        assert res.n == 0
        assert np.allclose(res.alpha, 0.0)
        assert res.tokens[0] == (0 if ur < 0.5 else 1)     # residual is the target itself


def test_zero_residual_falls_back_to_target():
    # Draft token outside both supports while p == q: rejection with Z = 0.
    p = np.array([0.25, 0.75, 0.0])
    zp = np.stack([logits_of(p)] * 2)
    zq = np.stack([logits_of(p)])
    res = verify_sequence(zp, zq, np.array([2], np.int32), np.array([0.5, 0.5]), 1.0, 0, 1.0, 1)
    assert res.n == 0 and res.zero_residual and res.tokens[0] == 1


# ----------------------------------------------------------------------------
# P9 / P10: filters that reduce to something else.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(10))
def test_topk1_equals_greedy(seed):
    rng = np.random.default_rng(300 + seed)
    V, G = 40, 4
    zp = rng.normal(size=(G + 1, V)) * 2
    zq = zp[:G] + rng.normal(size=(G, V))
    draft = np.array([int(np.argmax(zq[i])) if rng.random() < 0.7 else int(rng.integers(V)) for i in range(G)], np.int32)
    u = rng.random(G + 1)
    a = verify_sequence(zp, zq, draft, u, 0.8, 1, 1.0, G)
    b = verify_sequence(zp, zq, draft, u, 0.0, 0, 1.0, G)
    assert a.n == b.n and list(a.tokens) == list(b.tokens)
    assert np.allclose(a.alpha, b.alpha)


@pytest.mark.parametrize("seed", range(5))
def test_noop_filters(seed):
    rng = np.random.default_rng(400 + seed)
    V, G = 64, 3
    zp = rng.normal(size=(G + 1, V)) * 2
    zq = zp[:G] + rng.normal(size=(G, V))
    draft = rng.integers(0, V, size=G).astype(np.int32)
    u = rng.random(G + 1)
    base = verify_sequence(zp, zq, draft, u, 1.1, 0, 1.0, G)
    for k, tp in ((V, 1.0), (V + 5, 1.0), (-1, 1.0), (0, 1.5)):
        r = verify_sequence(zp, zq, draft, u, 1.1, k, tp, G)
        assert r.n == base.n and list(r.tokens) == list(base.tokens)
        assert np.array_equal(r.alpha, base.alpha)


# ----------------------------------------------------------------------------
# Filters against brute-force definitions on tiny vocabularies.
# ----------------------------------------------------------------------------
def _bf_topk(s, k):
    return np.array([sum(s[w] > s[v] for w in range(len(s))) < k for v in range(len(s))])


def _bf_topp(s, kept, top_p):
    e = np.where(kept, np.exp(s - s[kept].max()), 0.0)
    P = e / e.sum()
    best = None
    for t in sorted(set(s[kept].tolist())):
        mass = sum(P[v] for v in range(len(s)) if kept[v] and s[v] >= t)
        if mass >= top_p:
            best = t
    return kept & (s >= best)


@pytest.mark.parametrize("seed", range(30))
def test_filters_brute_force(seed):
    rng = np.random.default_rng(500 + seed)
    V = 12
    z = rng.integers(-4, 5, size=V).astype(np.float64) * 0.5     # many ties
    T = [0.5, 1.0, 1.7][seed % 3]
    k = int(rng.integers(1, V + 1))
    tp = float(rng.choice([0.3, 0.6, 0.9, 0.95]))
    s = z / T
    pr = process(z, T, k, 1.0)
    assert np.array_equal(pr.kept, _bf_topk(s, k) if k < V else np.ones(V, bool))
    pr2 = process(z, T, k, tp)
    assert np.array_equal(pr2.kept, _bf_topp(s, pr.kept, tp))
    e = np.where(pr2.kept, np.exp(s - s.max()), 0.0)
    assert np.allclose(pr2.prob, e / e.sum(), atol=1e-15)


def test_argmax_lowest_index():
    z = np.array([1.0, 3.0, 0.0, 3.0])
    assert process(z, 0.0, 0, 1.0).prob.tolist() == [0, 1, 0, 0]


# ----------------------------------------------------------------------------
# Control flow: the first rejection ends the round (Algorithm 1, step 3; the
# tests are made left to right and the extra token is drawn at the rejected
# position).  Rows and uniforms after it decide nothing: cutting the round at
# the rejection, or spoiling what follows it, changes no output.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(40))
def test_the_first_rejection_ends_the_round(seed):
    rng = np.random.default_rng(600 + seed)
    V = int(rng.integers(3, 40))
    G = int(rng.integers(2, 7))
    zp = rng.normal(size=(G + 1, V)) * 2
    zq = zp[:G] + rng.normal(size=(G, V)) * rng.choice([0.3, 1.0, 3.0])
    T = float(rng.choice([0.0, 0.5, 1.0, 1.3]))
    k = int(rng.choice([0, 1, 3, V]))
    tp = float(rng.choice([1.0, 0.9, 0.5]))
    draft = rng.integers(0, V, size=G).astype(np.int32)
    u = rng.random(G + 1)
    a = verify_sequence(zp, zq, draft, u, T, k, tp, G)
    if a.n >= G - 1:
        return
    n = a.n
    cut = verify_sequence(zp, zq, draft, u, T, k, tp, n + 1)                # the round ends at the rejection
    assert cut.n == n and list(cut.tokens[: n + 1]) == list(a.tokens[: n + 1])
    zp2, zq2, d2, u2 = zp.copy(), zq.copy(), draft.copy(), u.copy()
    zp2[n + 1:] = rng.normal(size=(G - n, V)) * 5                           # spoil everything after it
    zq2[n + 1:] = rng.normal(size=(G - n - 1, V)) * 5
    d2[n + 1:] = rng.integers(0, V, size=G - n - 1)
    u2[n + 1:G] = rng.random(G - n - 1)
    b = verify_sequence(zp2, zq2, d2, u2, T, k, tp, G)
    assert b.n == n and list(b.tokens) == list(a.tokens)
    assert np.array_equal(b.alpha[: n + 1], a.alpha[: n + 1]) and np.array_equal(b.pq[: n + 1], a.pq[: n + 1])


# ----------------------------------------------------------------------------
# Inverse CDF and decoding.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(5))
def test_inverse_cdf_measures(seed):
    rng = np.random.default_rng(700 + seed)
    w = rng.random(9) * (rng.random(9) < 0.7)
    w[3] = 0.4
    meas = token_intervals(lambda u: inverse_cdf(w, u)[0])
    got = np.zeros(9)
    for t, m in meas.items():
        got[t] = m
    assert np.allclose(got, w / w.sum(), atol=1e-12)
    for u in rng.random(50):
        t = inverse_cdf(w, u)[0]
        assert t == int(np.searchsorted(np.cumsum(w), u * np.cumsum(w)[-1], side="right"))
        assert w[t] > 0


def test_bf16_decoding():
    bits = np.array([0x3F80, 0xC000, 0xFF80, 0x7F80, 0x0001, 0x4049, 0x8000], np.uint16)
    v = decode_row(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == -np.inf and v[3] == np.inf
    assert v[4] == 2.0 ** -133 and v[5] == 3.140625 and v[6] == 0.0 and math.copysign(1, v[6]) < 0


# ----------------------------------------------------------------------------
# Invalid rows get sentinels.
# ----------------------------------------------------------------------------
def test_invalid_rows():
    rng = np.random.default_rng(9)
    V, G = 10, 3
    zp = rng.normal(size=(G + 1, V))
    zq = rng.normal(size=(G, V))
    d = np.array([1, 2, 3], np.int32)
    u = np.array([0.1, 0.2, 0.3, 0.4])
    ok = verify_sequence(zp, zq, d, u, 1.0, 0, 1.0, G)
    assert ok.n >= 0
    bad = []
    z2 = zp.copy(); z2[1, 4] = np.nan; bad.append((z2, zq, d, u, 1.0, G))
    z2 = zp.copy(); z2[0, 4] = np.inf; bad.append((z2, zq, d, u, 1.0, G))
    z2 = zq.copy(); z2[2, :] = -np.inf; bad.append((zp, z2, d, u, 1.0, G))
    bad.append((zp, zq, np.array([1, V, 3], np.int32), u, 1.0, G))
    bad.append((zp, zq, d, u, -0.5, G))
    bad.append((zp, zq, d, u, 1.0, 0))
    bad.append((zp, zq, d, np.array([0.1, 1.0, 0.3, 0.4]), 1.0, G))
    for a in bad:
        r = verify_sequence(a[0], a[1], a[2], a[3], a[4], 0, 1.0, a[5])
        assert r.n == -1 and (r.tokens == -1).all() and np.isnan(r.alpha).all()
    # Padding beyond gamma_b is never read.
    z2 = zp.copy(); z2[3, :] = np.nan
    zq2 = zq.copy(); zq2[2, :] = np.nan
    d2 = d.copy(); d2[2] = -7
    r = verify_sequence(z2, zq2, d2, u, 1.0, 0, 1.0, 2)
    assert r.n >= 0 and r.alpha[2] == 0.0


def test_neg_inf_logits_allowed():
    zp = np.array([[0.0, -np.inf, 1.0], [2.0, 0.0, -np.inf]])
    zq = np.array([[0.0, 0.5, -np.inf]])
    r = verify_sequence(zp, zq, np.array([0], np.int32), np.array([0.99, 0.3]), 1.0, 0, 1.0, 1)
    assert r.n in (0, 1) and r.tokens[r.n] in (0, 2) if r.n == 0 else True
    assert r.pq[0, 0] > 0 and r.pq[0, 1] > 0


def test_inverse_cdf_never_picks_zero_mass():
    # Leading zero-mass entries and u = 0: the draw must land on the first
    # token that carries mass (a token of zero probability is never sampled).
    w = np.array([0.0, 0.0, 0.3, 0.0, 0.7])
    assert inverse_cdf(w, 0.0)[0] == 2
    zp = np.stack([logits_of([0.0, 0.0, 0.3, 0.0, 0.7])] * 2)
    zq = np.stack([logits_of([0.0, 0.0, 0.3, 0.0, 0.7])])
    r = verify_sequence(zp, zq, np.array([2], np.int32), np.array([0.0, 0.0]), 1.0, 0, 1.0, 1)
    assert r.n == 1 and r.tokens[1] == 2


@pytest.mark.parametrize("cut", [0, 1, 2, 4])
def test_topp_mass_exactly_at_threshold(cut):
    # When the mass of the top (cut+1) values equals top_p exactly, those
    # values already reach top_p and form the nucleus.
    rng = np.random.default_rng(800 + cut)
    z = rng.normal(size=10) * 2
    base = process(z, 1.0, 0, 1.0).prob
    order = np.argsort(-z, kind="stable")
    cum = np.cumsum(base[order])
    pr = process(z, 1.0, 0, float(cum[cut]))
    assert pr.kept.sum() == cut + 1
    assert set(np.nonzero(pr.kept)[0]) == set(order[: cut + 1].tolist())


# ----------------------------------------------------------------------------
# Decision margins against the oracle's own decisions.  A margin says how far
# a uniform (or top_p) is from the point where the output would change; the
# change points are found by bisection on the outputs, with nothing re-typed.
# The pins must also reject planted mistakes (margins in unnormalised units,
# a missing side) in copies of the oracle's functions.
# ----------------------------------------------------------------------------
import inspect
import textwrap

from oracle import verify as verify_mod


def oracle_with(replacements):
    """verify_sequence and process of a copy of the oracle module in which
    each (function name, old text, new text) replacement has been made."""
    ns = dict(vars(verify_mod))
    for fname in ("process", "inverse_cdf", "verify_sequence"):
        src = textwrap.dedent(inspect.getsource(getattr(verify_mod, fname)))
        for name, old, new in replacements:
            if name == fname:
                assert old in src, (fname, old)
                src = src.replace(old, new)
        exec(compile(src, f"<oracle copy: {fname}>", "exec"), ns)
    return ns["verify_sequence"], ns["process"]


def bisect_edge(pred, good, bad, steps=90):
    """The point between `good` (pred True) and `bad` (pred False) where pred
    changes, for pred True on an interval around `good`."""
    for _ in range(steps):
        mid = 0.5 * (good + bad)
        if pred(mid):
            good = mid
        else:
            bad = mid
    return 0.5 * (good + bad)


def margin_cases(n_cases, seed):
    rng = np.random.default_rng(seed)
    for _ in range(n_cases):
        V = int(rng.integers(5, 16))
        G = int(rng.integers(1, 5))
        T = float(rng.choice([0.7, 1.0, 1.4]))
        zp = rng.normal(size=(G + 1, V)) * 1.5
        zq = zp[:G] + rng.normal(size=(G, V)) * 0.8
        Q = [process(zq[i], T, 0, 1.0).prob for i in range(G)]
        draft = np.array([int(rng.choice(V, p=Q[i])) for i in range(G)], np.int32)   # on the draft's support
        yield zp, zq, draft, rng.random(G + 1), T, G


def acc_margin_by_bisection(vfn, zp, zq, draft, u, T, G, i):
    """(change point of the test at position i in u_i, or None when the test
    accepts on all of [0, 1))."""
    def accepted(x):
        uu = u.copy()
        uu[i] = x
        return vfn(zp, zq, draft, uu, T, 0, 1.0, G).n > i
    if not accepted(0.0):
        return 0.0
    if accepted(np.nextafter(1.0, 0.0)):
        return None
    return bisect_edge(accepted, 0.0, 1.0)


def check_margin_acc(vfn, cases):
    for zp, zq, draft, u, T, G in cases:
        r = vfn(zp, zq, draft, u, T, 0, 1.0, G)
        flip, edge = np.inf, np.inf
        for i in range(min(r.n + 1, G)):            # the tests that were made
            a = acc_margin_by_bisection(vfn, zp, zq, draft, u, T, G, i)
            if a is None:
                edge = min(edge, 1.0 - u[i])        # ratio >= 1: |u - ratio| >= 1 - u
            else:
                flip = min(flip, abs(u[i] - a))
        assert r.margin_acc <= flip + 1e-12, (r.margin_acc, flip)
        assert r.margin_acc >= min(flip, edge) - 1e-12, (r.margin_acc, flip, edge)


def check_margin_cdf(vfn, cases):
    for zp, zq, draft, u, T, G in cases:
        r = vfn(zp, zq, draft, u, T, 0, 1.0, G)
        ur = float(u[G])

        def token(x):
            uu = u.copy()
            uu[G] = x
            return int(vfn(zp, zq, draft, uu, T, 0, 1.0, G).tokens[r.n])
        t = token(ur)
        same = lambda x: token(x) == t
        lo = 0.0 if same(0.0) else bisect_edge(same, ur, 0.0)
        hi = 1.0 if same(np.nextafter(1.0, 0.0)) else bisect_edge(same, ur, 1.0)
        assert abs(r.margin_cdf - min(ur - lo, hi - ur)) < 1e-12, (r.margin_cdf, ur, lo, hi)


def check_margin_topp(pfn, n_cases, seed):
    rng = np.random.default_rng(seed)
    for _ in range(n_cases):
        V = int(rng.integers(4, 14))
        z = rng.normal(size=V) * 1.5
        if rng.random() < 0.3:
            z = np.round(z)                          # ties at the cut
        T = float(rng.choice([0.6, 1.0, 1.5]))
        k = int(rng.choice([0, V - 2, V // 2]))
        tp = float(rng.uniform(0.2, 0.98))
        kept = pfn(z, T, k, tp).kept
        same = lambda x: np.array_equal(pfn(z, T, k, x).kept, kept)
        # The kept set grows with top_p; at top_p = 0 it is the maximum with
        # its ties, and top_p = 1 turns the filter off.
        lo_dist = np.inf if same(0.0) else tp - bisect_edge(same, tp, 0.0)
        hi_dist = 1.0 - tp if same(1.0) else bisect_edge(same, tp, 1.0) - tp
        assert abs(pfn(z, T, k, tp).topp_margin - min(lo_dist, hi_dist)) < 1e-12, (z, T, k, tp)


def test_margin_acc_is_the_distance_to_the_acceptance_change():
    check_margin_acc(verify_sequence, margin_cases(40, 901))


def test_margin_cdf_is_the_distance_to_the_token_change():
    check_margin_cdf(verify_sequence, margin_cases(40, 902))


def test_topp_margin_is_the_distance_to_the_nucleus_change():
    check_margin_topp(process, 60, 903)


def _change_distance(sig, tp):
    """Distance from tp to the nearest top_p in [0, 1] where sig(top_p)
    changes (sig constant on an interval around tp; top_p = 1 turns the
    filter off, so the upper side ends there)."""
    s0 = sig(tp)
    same = lambda x: sig(x) == s0
    lo = np.inf if same(0.0) else tp - bisect_edge(same, tp, 0.0)
    hi = 1.0 - tp if same(1.0) else bisect_edge(same, tp, 1.0) - tp
    return min(lo, hi)


def test_topp_margins_of_positions_and_decisions():
    """topp_pos[i] is the distance of top_p to the nearest change of the
    nucleus of position i's rows, so no change of alpha_i or
    (p_i(x_i), q_i(x_i)) is nearer; the token margin's top-p part is the
    same for the rows of the tests made and of the draw, so no change of n
    or the tokens is nearer."""
    rng = np.random.default_rng(904)
    for _ in range(30):
        V, G = int(rng.integers(5, 12)), int(rng.integers(1, 4))
        zp = np.round(rng.normal(size=(G + 1, V)) * 3) / 2
        zq = zp[:G] + np.round(rng.normal(size=(G, V)) * 2) / 2
        draft = rng.integers(0, V, size=G).astype(np.int32)
        u, T, tp = rng.random(G + 1), 1.0, float(rng.uniform(0.3, 0.95))
        run = lambda x: verify_sequence(zp, zq, draft, u, T, 0, x, G)
        kept = lambda row, x: tuple(np.nonzero(process(row, T, 0, x).kept)[0])
        r = run(tp)
        for i in range(G):
            d_kept = _change_distance(lambda x: (kept(zp[i], x), kept(zq[i], x)), tp)
            d_out = _change_distance(lambda x: (run(x).alpha[i], tuple(run(x).pq[i])), tp)
            assert abs(r.topp_pos[i] - d_kept) < 1e-12, (i, r.topp_pos[i], d_kept)
            assert r.topp_pos[i] <= d_out + 1e-12
        rows = [zp[j] for j in range(r.n + 1)] + [zq[i] for i in range(min(r.n + 1, G))]
        d_kept = _change_distance(lambda x: tuple(kept(row, x) for row in rows), tp)
        d_out = _change_distance(lambda x: (run(x).n, tuple(run(x).tokens)), tp)
        assert abs(r.margin_topp - d_kept) < 1e-12, (r.margin_topp, d_kept)
        assert r.margin_topp <= d_out + 1e-12


MARGIN_MISTAKES = {
    "acceptance margin in unnormalised units": (
        "acc", [("verify_sequence", "abs(ui - px / (lenience * qx))", "abs(ui * lenience * qx - px)")]),
    "CDF margin in unnormalised units": (
        "cdf", [("inverse_cdf", "margin = min(u - lo / Z, c[t] / Z - u)", "margin = min(u * Z - lo, c[t] - u * Z)")]),
    "CDF margin on one side only": (
        "cdf", [("inverse_cdf", "margin = min(u - lo / Z, c[t] / Z - u)", "margin = c[t] / Z - u")]),
    "top-p margin without the lower side": (
        "topp", [("process", "margin = min(margin, top_p - prob[above].sum())", "pass")]),
}


@pytest.mark.parametrize("name", sorted(MARGIN_MISTAKES))
def test_margin_pins_reject_planted_mistakes(name):
    kind, repl = MARGIN_MISTAKES[name]
    vfn, pfn = oracle_with(repl)
    with pytest.raises(AssertionError):
        if kind == "acc":
            check_margin_acc(vfn, margin_cases(40, 901))
        elif kind == "cdf":
            check_margin_cdf(vfn, margin_cases(40, 902))
        else:
            check_margin_topp(pfn, 60, 903)

"""CPU oracle for the batched speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run this module; the product path
never does.  It shares no code with the HIP library (no kernels, headers,
helpers or tables) and does not import it.

Everything here is plain float64 numpy, one sequence at a time, written from
the definitions on the pages (cited by page title and section):

* Processing (temperature, top-k, top-p, normalisation): both distributions
  are the *adjusted, normalised* ones -- "Fast Inference from Transformers via
  Speculative Decoding" (mtandhj.com summary), "Speculative Sampling:
  theoretical basis", first bullet; the Leviathan review (dongryeollee1),
  "Method: Speculative Decoding / Overview", preprocessing remark (argmax,
  top-k, nucleus and temperature all reduce to standard sampling from an
  adjusted distribution).
* Acceptance: accept x ~ q when u < min(1, p(x)/q(x)) -- llm-compass
  "Speculative Decoding", section 4 (speculative_step), and "Speculative
  Decoding: the art of guessing well", section "Speculative sampling".
* First rejection: n = min({i-1 : r_i > p_i(x_i)/q_i(x_i)} U {gamma}) --
  Leviathan review, Algorithm 1, step 3.
* Residual p'(x) = norm(max(0, p(x) - q(x))), bonus from p_{gamma+1} --
  Algorithm 1, steps 4-5; mtandhj summary, "Speculative Sampling: theoretical
  basis" (residual), "Core idea" (bonus token).
* Sampling by inverse CDF (normalise, cumulative sum, invert one uniform) --
  "the art of guessing well", section "Sampling with shared noise", first
  paragraph.
* Overlap alpha = sum_x min(p(x), q(x)) -- mtandhj summary, "How to choose
  gamma"; "the art of guessing well", section "Speculative sampling".

Readings taken where the pages leave a point open (each is listed with its
reason in the design notes): strict '<' in the acceptance test, written
division-free as u*q < p; a draft token with q(x) = 0 is accepted iff
p(x) > 0; argmax ties go to the lowest vocabulary id; top-k keeps every value
>= the k-th largest (ties kept); top-p keeps every value >= t*, the largest
value whose upper mass reaches top_p (ties kept), applied after top-k;
the inverse CDF runs over ascending vocabulary id and returns the first v
with C(v) > u*Z; a zero residual mass falls back to p_{n+1}; the residual or
bonus draw is u[gamma_max]; invalid rows get sentinel outputs.
"""
from __future__ import annotations

import dataclasses
import math
import multiprocessing as mp
import os
from typing import Optional, Sequence

import numpy as np

INF = float("inf")


# ----------------------------------------------------------------------------
# Input decoding.
# ----------------------------------------------------------------------------
def decode_row(row: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or float32 -> float64 values (exact)."""
    if row.dtype == np.uint16:
        return (row.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(row, dtype=np.float64)


def row_is_valid(z: np.ndarray) -> bool:
    """A logit row is usable when it has no NaN, no +inf and at least one
    finite value (so the softmax is defined)."""
    if np.isnan(z).any() or np.isposinf(z).any():
        return False
    return bool(np.isfinite(z).any())


# ----------------------------------------------------------------------------
# Processing: temperature -> top-k -> top-p -> normalise.
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Processed:
    prob: np.ndarray          # float64 [V], sums to 1
    kept: np.ndarray          # bool [V], the support after filtering
    topp_margin: float        # distance of top_p from the nucleus boundary masses


def process(z: np.ndarray, T: float, top_k: int, top_p: float) -> Processed:
    """The adjusted, normalised distribution for one logit row.

    T == 0 is argmax: all mass on the largest logit (the lowest id among
    equal maxima).  For T > 0 the scores are s = z / T; top-k (0 < k < V)
    keeps s >= the k-th largest s; top-p (top_p < 1) then keeps s >= t*,
    where t* is the largest kept value whose mass at-or-above reaches
    top_p; the kept scores are normalised with a softmax."""
    V = z.shape[0]
    if T == 0.0:
        prob = np.zeros(V)
        prob[int(np.argmax(z))] = 1.0
        return Processed(prob, prob > 0, INF)
    s = z / T
    kept = np.ones(V, dtype=bool)
    if 0 < top_k < V:
        kth = np.partition(s, V - top_k)[V - top_k]     # the k-th largest value
        kept = s >= kth
    m = s[kept].max()
    e = np.where(kept, np.exp(s - m), 0.0)
    prob = e / e.sum()
    margin = INF
    if top_p < 1.0:
        vals = s[kept]
        order = np.argsort(-vals, kind="stable")
        cum = np.cumsum(prob[kept][order])
        hit = np.nonzero(cum >= top_p)[0]
        if hit.size:
            t_star = vals[order[hit[0]]]
            above = kept & (s > t_star)
            at = kept & (s >= t_star)
            m_at = prob[at].sum()
            margin = m_at - top_p
            if above.any():
                margin = min(margin, top_p - prob[above].sum())
            kept = at
            e = np.where(kept, e, 0.0)
            prob = e / e.sum()
    return Processed(prob, kept, float(margin))


def inverse_cdf(r: np.ndarray, u: float):
    """Inverse-CDF draw from the (unnormalised) non-negative weights r.

    Returns (token, margin): token = min{v : C(v) > u * Z} over ascending
    vocabulary id with C the running sum and Z = C(V-1); if rounding leaves
    no such v, the last v with r(v) > 0.  The margin is the distance of u
    from the two CDF values that bracket the chosen token, in normalised
    units."""
    c = np.cumsum(r)
    Z = c[-1]
    target = u * Z
    idx = np.nonzero(c > target)[0]
    if idx.size:
        t = int(idx[0])
    else:
        t = int(np.nonzero(r > 0)[0][-1])
    lo = c[t - 1] if t > 0 else 0.0
    margin = min(u - lo / Z, c[t] / Z - u)
    return t, float(margin)


# ----------------------------------------------------------------------------
# One sequence (Algorithm 1 form).
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class SeqResult:
    tokens: np.ndarray        # int32 [gamma_max+1], -1 padded
    n: int                    # accepted drafts, -1 for an invalid row
    alpha: np.ndarray         # float64 [gamma_max], 0 in padded slots
    pq: np.ndarray            # float64 [gamma_max, 2] = p_i(x_i), q_i(x_i)
    margin_acc: float
    margin_cdf: float
    margin_topp: float        # top-p margin of the rows that decided n and the drawn token
    zero_residual: bool       # Z == 0 fallback taken
    topp_pos: np.ndarray      # float64 [gamma_max]: top-p margin of position i's two rows (alpha_i, pq_i)

    @property
    def margin(self):
        """Decision margin of n and the tokens."""
        return min(self.margin_acc, self.margin_cdf, self.margin_topp)


def invalid_result(gamma_max: int) -> SeqResult:
    return SeqResult(np.full(gamma_max + 1, -1, np.int32), -1, np.full(gamma_max, np.nan),
                     np.full((gamma_max, 2), np.nan), INF, INF, INF, False, np.full(gamma_max, INF))


def _inputs_valid(zp, zq, draft, u, T, top_p, gamma_b, V, gamma_max, lenience=1.0) -> bool:
    if not (1 <= gamma_b <= gamma_max):
        return False
    if not (T >= 0.0) or math.isnan(top_p):
        return False
    if not (0.0 <= lenience <= 1.0):
        return False
    x = draft[:gamma_b]
    if (x < 0).any() or (x >= V).any():
        return False
    uu = np.concatenate([u[:gamma_b], u[gamma_max:gamma_max + 1]]).astype(np.float64)
    if not ((uu >= 0.0) & (uu < 1.0)).all():
        return False
    for j in range(gamma_b + 1):
        if not row_is_valid(zp[j]):
            return False
    for i in range(gamma_b):
        if not row_is_valid(zq[i]):
            return False
    return True


def verify_sequence(zp: np.ndarray, zq: np.ndarray, draft: np.ndarray, u: np.ndarray,
                    T: float, top_k: int, top_p: float, gamma_b: int, lenience: float = 1.0) -> SeqResult:
    """Verify one sequence.

    zp: [gamma_max+1, V] target logits (float64), zq: [gamma_max, V] draft
    logits, draft: [gamma_max] tokens, u: [gamma_max+1] uniforms where
    u[i] (i < gamma_b) tests draft i and u[gamma_max] drives the residual or
    bonus draw.  Positions at and beyond gamma_b (drafts) and gamma_b+1
    (targets) are padding and are never read.

    lenience l in [0, 1] multiplies q(x) in the acceptance test (the
    Leviathan review, "Lenience"): accept iff u * l * q(x) < p(x).  l = 1 is
    the exact method.  Reading: the page changes only the acceptance
    decision, so the residual stays max(0, p - q); with it no token's output
    probability exceeds p(x) / l, the page's guarantee."""
    gamma_max = zq.shape[0]
    V = zp.shape[1]
    T = float(T)
    top_p = float(top_p)
    lenience = float(lenience)
    if not _inputs_valid(zp, zq, draft, u, T, top_p, gamma_b, V, gamma_max, lenience):
        return invalid_result(gamma_max)
    P = [process(zp[j], T, top_k, top_p) for j in range(gamma_b + 1)]
    Q = [process(zq[i], T, top_k, top_p) for i in range(gamma_b)]

    alpha = np.zeros(gamma_max)
    pq = np.zeros((gamma_max, 2))
    for i in range(gamma_b):
        alpha[i] = np.minimum(P[i].prob, Q[i].prob).sum()
        pq[i] = (P[i].prob[draft[i]], Q[i].prob[draft[i]])

    # Left-to-right acceptance; stop at the first rejection.
    n = gamma_b
    margin_acc = INF
    for i in range(gamma_b):
        px, qx = pq[i]
        ui = float(u[i])
        if T > 0.0 and lenience * qx > 0.0:
            margin_acc = min(margin_acc, abs(ui - px / (lenience * qx)))
        if not (ui * lenience * qx < px):
            n = i
            break

    # Residual at the rejected position, else the bonus position.
    if n < gamma_b:
        r = np.maximum(P[n].prob - Q[n].prob, 0.0)
    else:
        r = P[gamma_b].prob.copy()
    zero_residual = False
    if not (r.sum() > 0.0):
        zero_residual = True
        r = P[n].prob.copy()
    t, margin_cdf = inverse_cdf(r, float(u[gamma_max]))
    if T == 0.0:
        margin_cdf = INF

    # A nucleus boundary moves what is computed from its row: alpha_i and
    # (p_i(x_i), q_i(x_i)) depend on position i's two rows only; n and the
    # tokens on the rows of the tests that were made (positions 0..n, the
    # last of them the rejection) and of the draw (position n, or the bonus
    # row).  Rows after the first rejection decide nothing.
    topp_pos = np.full(gamma_max, INF)
    for i in range(gamma_b):
        topp_pos[i] = min(P[i].topp_margin, Q[i].topp_margin)
    deciding = [P[j].topp_margin for j in range(n + 1)] + [Q[i].topp_margin for i in range(min(n + 1, gamma_b))]
    margin_topp = min(deciding)

    tokens = np.full(gamma_max + 1, -1, np.int32)
    tokens[:n] = draft[:n]
    tokens[n] = t
    return SeqResult(tokens, n, alpha, pq, margin_acc, margin_cdf, margin_topp, zero_residual, topp_pos)


# ----------------------------------------------------------------------------
# Batched driver (rows in parallel across host cores).
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class BatchResult:
    tokens: np.ndarray        # int32 [B, gamma_max+1]
    n: np.ndarray             # int32 [B]
    alpha: np.ndarray         # float64 [B, gamma_max]
    pq: np.ndarray            # float64 [B, gamma_max, 2]
    margin: np.ndarray        # float64 [B] = min of the three margins (decides n and the tokens)
    margin_acc: np.ndarray
    margin_cdf: np.ndarray
    margin_topp: np.ndarray
    zero_residual: np.ndarray
    topp_pos: np.ndarray      # float64 [B, gamma_max]: per-position top-p margin (alpha_i, pq_i)


_SHARED = {}


def _one(b: int) -> SeqResult:
    a = _SHARED
    return verify_sequence(decode_row(a["p"][b]), decode_row(a["q"][b]), a["draft"][b], a["u"][b],
                           float(a["T"][b]), int(a["k"][b]), float(a["top_p"][b]), int(a["g"][b]),
                           float(a["l"][b]))


def verify_batch(p_logits, q_logits, draft, u, temperature, top_k, top_p, gamma_len,
                 rows: Optional[Sequence[int]] = None, processes: Optional[int] = None,
                 lenience=None) -> BatchResult:
    """Run the oracle over the sequences in ``rows`` (default: all).

    processes: worker processes (fork); None -> all host cores, 1 -> serial.
    lenience: [B] per-sequence lenience, None -> 1 (the exact method)."""
    B = p_logits.shape[0]
    gamma_max = q_logits.shape[1]
    rows = list(range(B)) if rows is None else list(rows)
    _SHARED.update(p=p_logits, q=q_logits, draft=np.asarray(draft), u=np.asarray(u),
                   T=np.asarray(temperature), k=np.asarray(top_k), top_p=np.asarray(top_p),
                   g=np.asarray(gamma_len),
                   l=np.ones(B, np.float32) if lenience is None else np.asarray(lenience))
    nproc = os.cpu_count() if processes is None else processes
    nproc = max(1, min(nproc, len(rows)))
    if nproc == 1:
        res = [_one(b) for b in rows]
    else:
        with mp.get_context("fork").Pool(nproc) as pool:
            res = pool.map(_one, rows, chunksize=max(1, len(rows) // (4 * nproc)))
    R = len(rows)
    out = BatchResult(np.full((R, gamma_max + 1), -1, np.int32), np.zeros(R, np.int32),
                      np.zeros((R, gamma_max)), np.zeros((R, gamma_max, 2)), np.zeros(R),
                      np.zeros(R), np.zeros(R), np.zeros(R), np.zeros(R, bool), np.full((R, gamma_max), INF))
    for k, r in enumerate(res):
        out.tokens[k] = r.tokens
        out.n[k] = r.n
        out.alpha[k] = r.alpha
        out.pq[k] = r.pq
        out.margin[k] = r.margin
        out.margin_acc[k] = r.margin_acc
        out.margin_cdf[k] = r.margin_cdf
        out.margin_topp[k] = r.margin_topp
        out.zero_residual[k] = r.zero_residual
        out.topp_pos[k] = r.topp_pos
    _SHARED.clear()
    return out


# ----------------------------------------------------------------------------
# Verify with shared Gumbel noise (Gumbel coupling).
# ----------------------------------------------------------------------------
# "Speculative Decoding: the art of guessing well", section "Sampling with
# shared noise": the drafter and the target use the same noise vector g_k at
# draft position k.  The drafter proposes argmax_i(log q_k(i) + g_k,i); the
# target's own sample is argmax_i(log p_k(i) + g_k,i); the verify keeps the
# longest prefix on which the two agree and appends the target's token at the
# first disagreement (the target's token after the last draft when all
# agree).  Gumbel-max sampling itself (argmax of logits plus independent
# Gumbel noise follows the softmax) is the same section's first part.
#
# log p_k(i) = z_i / T - log S over the processed support, so the argmax only
# needs the support and the score z_i / T + g_i (log S is common to every i).
# The scores are formed in float64.  Ties go to the lowest id; T = 0 is exact
# argmax matching (the noise is unused, as in "Draft and verify").
# Decision margin of one position: the gap between the best and the
# second-best score over the support, divided by the magnitude of the terms
# that form them, max(1, |z/T| + |g|) of either: a score computed in any
# precision with relative rounding e is off by about e times that, so the
# argmax can only differ from this one where the gap is that small.

def gumbel_scores(z: np.ndarray, g: np.ndarray, T: float) -> np.ndarray:
    """float64 scores z / T + g of one row (z decoded logits, g the row's
    noise, T > 0): log p + g up to the row's common -log S."""
    return np.asarray(z, dtype=np.float64) / T + np.asarray(g, dtype=np.float64)


def gumbel_target_token(z: np.ndarray, g: np.ndarray, T: float, top_k: int, top_p: float, parts: bool = False):
    """The target's sample at one position: the lowest id maximising the
    score over the processed support.  Returns (token, margin), the margin
    being the smaller of the score-gap margin and the top-p margin; with
    parts, (token, margin, top-p margin)."""
    if T == 0.0:
        return (int(np.argmax(z)), INF, INF) if parts else (int(np.argmax(z)), INF)
    pr = process(z, T, top_k, top_p)
    sc = np.where(pr.kept, gumbel_scores(z, g, T), -np.inf)
    t = int(np.argmax(sc))
    margin = pr.topp_margin
    if pr.kept.sum() > 1:
        rest = sc.copy()
        rest[t] = -np.inf
        t2 = int(np.argmax(rest))
        size = lambda i: abs(float(z[i]) / T) + abs(float(g[i]))
        gap = (sc[t] - sc[t2]) / max(1.0, size(t), size(t2))
        margin = min(margin, float(gap))
    return (t, margin, pr.topp_margin) if parts else (t, margin)


@dataclasses.dataclass
class GumbelResult:
    tokens: np.ndarray        # int32 [gamma_max+1]: x_1..x_n, then target[n], -1 padded
    n: int                    # drafts kept, -1 for an invalid sequence
    target: np.ndarray        # int32 [gamma_max+1]: the target's sample at each used position
    margin: float             # decision margin of n and the tokens (positions 0..n)
    margin_pos: np.ndarray    # float64 [gamma_max+1]: decision margin of each position's sample
    topp_pos: np.ndarray      # float64 [gamma_max+1]: its top-p part alone


def gumbel_verify_sequence(zp: np.ndarray, g: np.ndarray, draft: np.ndarray, T: float, top_k: int,
                           top_p: float, gamma_b: int) -> GumbelResult:
    """One sequence.  zp: [gamma_max+1, V] target logits (float64), g:
    [gamma_max+1, V] noise, draft: [gamma_max] proposed tokens.  Rows beyond
    gamma_b are padding and are never read."""
    gamma_max = zp.shape[0] - 1
    V = zp.shape[1]
    T = float(T)
    top_p = float(top_p)
    bad = GumbelResult(np.full(gamma_max + 1, -1, np.int32), -1, np.full(gamma_max + 1, -1, np.int32), INF,
                       np.full(gamma_max + 1, INF), np.full(gamma_max + 1, INF))
    if not (1 <= gamma_b <= gamma_max) or not (T >= 0.0) or math.isnan(top_p):
        return bad
    x = np.asarray(draft[:gamma_b])
    if (x < 0).any() or (x >= V).any():
        return bad
    for j in range(gamma_b + 1):
        if not row_is_valid(zp[j]):
            return bad
    target = np.full(gamma_max + 1, -1, np.int32)
    margin_pos = np.full(gamma_max + 1, INF)
    topp_pos = np.full(gamma_max + 1, INF)
    for j in range(gamma_b + 1):
        # Noise off the processed support never takes part in the argmax;
        # a NaN or infinite value on it makes the sequence invalid.
        if T > 0.0:
            kept = process(zp[j], T, top_k, top_p).kept
            if not np.isfinite(np.asarray(g[j], dtype=np.float64)[kept]).all():
                return bad
        target[j], margin_pos[j], topp_pos[j] = gumbel_target_token(zp[j], g[j], T, top_k, top_p, parts=True)
    n = gamma_b
    for k in range(gamma_b):
        if int(x[k]) != int(target[k]):
            n = k
            break
    tokens = np.full(gamma_max + 1, -1, np.int32)
    tokens[:n] = x[:n]
    tokens[n] = target[n]
    return GumbelResult(tokens, n, target, float(margin_pos[: n + 1].min()), margin_pos, topp_pos)


@dataclasses.dataclass
class GumbelBatchResult:
    tokens: np.ndarray        # int32 [B, gamma_max+1]
    n: np.ndarray             # int32 [B]
    target: np.ndarray        # int32 [B, gamma_max+1]
    margin: np.ndarray        # float64 [B]: decision margin of n and the tokens
    margin_pos: np.ndarray    # float64 [B, gamma_max+1]: decision margin of each target sample
    topp_pos: np.ndarray      # float64 [B, gamma_max+1]: its top-p part alone


_GSHARED = {}


def _gumbel_one(b: int) -> GumbelResult:
    a = _GSHARED
    return gumbel_verify_sequence(decode_row(a["p"][b]), a["noise"][b], np.asarray(a["draft"][b]), float(a["T"][b]),
                                  int(a["k"][b]), float(a["top_p"][b]), int(a["g"][b]))


def gumbel_verify_batch(p_logits, noise, draft, temperature, top_k, top_p, gamma_len,
                        rows: Optional[Sequence[int]] = None, processes: int = 1) -> GumbelBatchResult:
    """The Gumbel-coupling verify over the sequences in ``rows`` (default:
    all), on `processes` worker processes (fork; 1 = serial)."""
    B = p_logits.shape[0]
    G1 = p_logits.shape[1]
    rows = list(range(B)) if rows is None else list(rows)
    R = len(rows)
    _GSHARED.update(p=p_logits, noise=noise, draft=draft, T=np.asarray(temperature), k=np.asarray(top_k),
                    top_p=np.asarray(top_p), g=np.asarray(gamma_len))
    nproc = max(1, min(processes, R))
    if nproc == 1:
        res = [_gumbel_one(b) for b in rows]
    else:
        with mp.get_context("fork").Pool(nproc) as pool:
            res = pool.map(_gumbel_one, rows, chunksize=max(1, R // (4 * nproc)))
    _GSHARED.clear()
    out = GumbelBatchResult(np.full((R, G1), -1, np.int32), np.zeros(R, np.int32), np.full((R, G1), -1, np.int32),
                            np.zeros(R), np.full((R, G1), INF), np.full((R, G1), INF))
    for k, r in enumerate(res):
        out.tokens[k] = r.tokens
        out.n[k] = r.n
        out.target[k] = r.target
        out.margin[k] = r.margin
        out.margin_pos[k] = r.margin_pos
        out.topp_pos[k] = r.topp_pos
    return out


# ----------------------------------------------------------------------------
# Sampling one token per row (the drafter's step before a verify).
# ----------------------------------------------------------------------------
# x ~ the processed distribution ("Fast Inference from Transformers via
# Speculative Decoding", mtandhj.com summary, "Speculative Sampling:
# theoretical basis": both models sample from their adjusted distributions),
# drawn by the inverse CDF at one uniform ("Speculative Decoding: the art of
# guessing well", "Sampling with shared noise", textbook method).

@dataclasses.dataclass
class SampleBatchResult:
    tokens: np.ndarray        # int32 [R], -1 for an invalid row
    margin: np.ndarray        # float64 [R]: min of the CDF and top-p margins


def sample_row(z: np.ndarray, u: float, T: float, top_k: int, top_p: float):
    """Returns (token, margin) for one row; (-1, inf) for invalid input."""
    T = float(T)
    top_p = float(top_p)
    if not row_is_valid(z) or not (T >= 0.0) or math.isnan(top_p) or not (0.0 <= u < 1.0):
        return -1, INF
    pr = process(z, T, top_k, top_p)
    t, m_cdf = inverse_cdf(pr.prob, float(u))
    if T == 0.0:
        m_cdf = INF
    return t, min(m_cdf, pr.topp_margin)


def sample_batch(logits, u, temperature, top_k, top_p) -> SampleBatchResult:
    R = logits.shape[0]
    out = SampleBatchResult(np.full(R, -1, np.int32), np.full(R, INF))
    for r in range(R):
        t, m = sample_row(decode_row(logits[r]), float(u[r]), float(temperature[r]), int(top_k[r]), float(top_p[r]))
        out.tokens[r] = t
        out.margin[r] = m
    return out

"""K-SEQ multi-candidate verify and the SpecTr walk (CPU oracle).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

Written from "SpecTr: Fast Speculative Decoding via Optimal Transport"
(mtandhj.com), sections "K-SEQ" (equations 4-7), "Residual distribution" and
"SpecTr".  That page names the draft distribution p and the target q; here,
as everywhere in this build, p is the TARGET and q the DRAFT, so the page's
formulas appear with the two letters exchanged:

    a_rho(x) = min(1, p(x) / (rho q(x)))          acceptance of one candidate
    m_rho(x) = q(x) a_rho(x) = min(q(x), p(x)/rho) mass of "draw x and accept it"
    beta(rho) = sum_x m_rho(x)
    P_A = 1 - (1 - beta)^k                         some candidate is accepted
    A_rho(x) = (P_A / beta) m_rho(x)               mass the candidates give x
    rho* in [1, k] with 1 - (1 - beta(rho*))^k = rho* beta(rho*)
    residual  (p(x) - A_rho*(x)) / (1 - P_A)

Candidates X_1..X_k (i.i.d. draws of the draft, repeats kept) are tested in
order with uniforms u_1..u_k; the first accepted one is the output; if all
are rejected the output is drawn from the residual.  beta = 0 draws from the
target; P_A = 1 never reaches the residual.

Readings where the page leaves a step open:
* rho* is the smallest root: rho beta(rho) - (1 - (1 - beta(rho))^k) is
  non-decreasing in rho (rho beta(rho) = sum min(rho q, p) grows, beta falls),
  non-positive at rho = 1 and non-negative at rho = k, so the roots form an
  interval; the page's "rho >= rho* is valid, and rho* maximises the direct
  acceptance" picks its left end.  Found by bisection (80 halvings).
* The root is located on the same function written without cancellation:
  as p sums to 1, 1 - rho beta(rho) = sum max(0, p - rho q) =: D(rho), so
  rho beta - (1 - (1 - beta)^k) = (1 - beta)^k - D(rho).  For large k the
  term (1 - beta)^k falls below 1e-16 while rho beta - 1 can only be formed
  to about 1e-16; D is a sum of non-negative terms, exactly 0 once every
  element is saturated (rho q >= p), so the sign is never decided by
  rounding.
* The acceptance test is strict, u_i < a(X_i) (as for the single-candidate
  test); the residual draw is the same inverse CDF over ascending id at the
  residual uniform u_{k+1}, with Z the sum of the clamped residual weights.
* The processed distributions (temperature, top-k, top-p) are those of the
  single-candidate verify.
* SpecTr: at each depth the candidates are the next tokens of the candidate
  sequences that agree with the output so far; their rows (target and draft
  distributions after that common prefix) are taken from the first such
  sequence; the walk continues while the output is one of the candidates and
  ends with a bonus draw from the target after the last depth.  One uniform
  vector u[j] (K + 1 values) is used at depth j, whichever node is reached.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

from .verify import INF, decode_row, inverse_cdf, process, row_is_valid


def beta_of(p: np.ndarray, q: np.ndarray, rho: float) -> float:
    return float(np.minimum(q, p / rho).sum())


def deficit_of(p: np.ndarray, q: np.ndarray, rho: float) -> float:
    """D(rho) = sum max(0, p - rho q) = 1 - rho beta(rho) for normalised p."""
    return float(np.maximum(p - rho * q, 0.0).sum())


def rho_star(p: np.ndarray, q: np.ndarray, k: int) -> float:
    """Smallest rho in [1, k] with rho beta(rho) >= 1 - (1 - beta(rho))^k,
    i.e. (1 - beta(rho))^k >= D(rho)."""
    def g(rho):
        b = beta_of(p, q, rho)
        return (1.0 - b) ** k - deficit_of(p, q, rho)
    if k <= 1 or g(1.0) >= 0.0:
        return 1.0
    lo, hi = 1.0, float(k)
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        if g(mid) >= 0.0:
            hi = mid
        else:
            lo = mid
    return hi


@dataclasses.dataclass
class KseqResult:
    token: int                 # output Y
    accepted: int              # index of the accepted candidate, -1 when the residual drew Y
    rho: float
    beta: float
    p_accept: float            # P_A
    margin: float              # min distance of a deciding uniform from its threshold


def kseq_position(p: np.ndarray, q: np.ndarray, cands, u) -> KseqResult:
    """One K-SEQ step: target p, draft q (processed, normalised), candidate
    tokens (repeats kept), uniforms u[0..k-1] for the candidates and u[k]
    for the residual."""
    k = len(cands)
    rho = rho_star(p, q, k)
    beta = beta_of(p, q, rho)
    p_acc = 1.0 - (1.0 - beta) ** k
    margin = INF
    for i, x in enumerate(cands):
        qx, px = q[x], p[x]
        a = 1.0 if qx * rho <= px else px / (rho * qx)     # min(1, p / (rho q)), q > 0 here
        if qx == 0.0:
            a = 1.0 if px > 0.0 else 0.0
        margin = min(margin, abs(float(u[i]) - a))
        if float(u[i]) < a:
            return KseqResult(int(x), i, rho, beta, p_acc, margin)
    if beta > 0.0:
        r = p - (p_acc / beta) * np.minimum(q, p / rho)
        r = np.maximum(r, 0.0)
        if not (r.sum() > 0.0):
            r = p.copy()
    else:
        r = p.copy()
    t, m = inverse_cdf(r, float(u[k]))
    return KseqResult(t, -1, rho, beta, p_acc, min(margin, m))


@dataclasses.dataclass
class SpecTrResult:
    tokens: np.ndarray         # int32 [L+1]: output tokens, -1 padded
    n: int                     # positions whose output was one of the candidates (<= L); -1 invalid
    margin: float


def spectr_sequence(zp, zq, cand, u, T, top_k, top_p) -> SpecTrResult:
    """One SpecTr round.  zp: [K, L+1, V] target logits per candidate
    sequence (row j = the target after the candidate's first j tokens), zq:
    [K, L, V] draft logits, cand: [K, L] candidate tokens, u: [L+1, K+1]
    uniforms (depth L: u[L, 0] is the bonus draw)."""
    K, L = cand.shape
    V = zp.shape[-1]
    T, top_p = float(T), float(top_p)
    bad = SpecTrResult(np.full(L + 1, -1, np.int32), -1, INF)
    if not (T >= 0.0) or math.isnan(top_p) or (cand < 0).any() or (cand >= V).any():
        return bad
    if not ((u >= 0.0) & (u < 1.0)).all():
        return bad
    out = np.full(L + 1, -1, np.int32)
    alive = list(range(K))
    margin = INF
    for j in range(L):
        c0 = alive[0]
        if not (row_is_valid(zp[c0, j]) and row_is_valid(zq[c0, j])):
            return bad
        P = process(zp[c0, j], T, top_k, top_p)
        Q = process(zq[c0, j], T, top_k, top_p)
        margin = min(margin, P.topp_margin, Q.topp_margin)
        xs = [int(cand[c, j]) for c in alive]
        r = kseq_position(P.prob, Q.prob, xs, u[j])
        if T > 0.0:
            margin = min(margin, r.margin)
        out[j] = r.token
        alive = [c for c in alive if int(cand[c, j]) == r.token]
        if not alive:
            return SpecTrResult(out, j, margin)
    c0 = alive[0]
    if not row_is_valid(zp[c0, L]):
        return bad
    P = process(zp[c0, L], T, top_k, top_p)
    t, m = inverse_cdf(P.prob, float(u[L, 0]))
    if T > 0.0:
        margin = min(margin, m, P.topp_margin)
    out[L] = t
    return SpecTrResult(out, L, margin)


@dataclasses.dataclass
class SpecTrBatchResult:
    tokens: np.ndarray         # int32 [B, L+1]
    n: np.ndarray              # int32 [B]
    margin: np.ndarray         # float64 [B]


def spectr_batch(p_logits, q_logits, cand, u, temperature, top_k, top_p, rows=None) -> SpecTrBatchResult:
    B, K, L1, V = p_logits.shape
    rows = list(range(B)) if rows is None else list(rows)
    out = SpecTrBatchResult(np.full((len(rows), L1), -1, np.int32), np.zeros(len(rows), np.int32),
                            np.zeros(len(rows)))
    for i, b in enumerate(rows):
        zp = np.stack([np.stack([decode_row(p_logits[b, c, j]) for j in range(L1)]) for c in range(K)])
        zq = np.stack([np.stack([decode_row(q_logits[b, c, j]) for j in range(L1 - 1)]) for c in range(K)])
        r = spectr_sequence(zp, zq, np.asarray(cand[b]), np.asarray(u[b], np.float64), float(temperature[b]),
                            int(top_k[b]), float(top_p[b]))
        out.tokens[i] = r.tokens
        out.n[i] = r.n
        out.margin[i] = r.margin
    return out

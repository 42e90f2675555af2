"""Expected-throughput analytics of speculative decoding (CPU oracle side).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the library's own
analytics entry points are checked against these and against the pages'
printed numbers.

Definitions (page titles and sections):
* Expected tokens per round with i.i.d. acceptance alpha and gamma drafts:
  (1 - alpha^(gamma+1)) / (1 - alpha) -- "Fast Inference from Transformers
  via Speculative Decoding" (mtandhj.com summary and the Leviathan review),
  "Analysis / expected generated tokens"; "Speculative Decoding: the art of
  guessing well", "How many tokens do we get?".
* Walltime speedup with cost ratio c: the expected tokens divided by
  (gamma c + 1) -- Leviathan review, "Analysis / walltime".
* Expected arithmetic operations relative to plain decoding, with the
  drafter's operations ratio c_hat: (1 - alpha)(gamma c_hat + gamma + 1) /
  (1 - alpha^(gamma+1)) -- Leviathan review, "Analysis / operations".
* Optimal gamma: the integer gamma >= 1 maximising the speedup (ties to the
  smaller gamma) -- Leviathan review, "Optimal gamma".
* Acceptance length tau = 1 + sum_k prod_{i<=k} alpha_i with per-position
  acceptance alpha_k -- "the art of guessing well", "How many tokens do we
  get?".
"""
from __future__ import annotations

from typing import Sequence


def expected_tokens(alpha: float, gamma: int) -> float:
    if alpha >= 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def speedup(alpha: float, gamma: int, c: float) -> float:
    return expected_tokens(alpha, gamma) / (gamma * c + 1.0)


def operations(alpha: float, gamma: int, c_hat: float) -> float:
    return (gamma * c_hat + gamma + 1.0) / expected_tokens(alpha, gamma)


def optimal_gamma(alpha: float, c: float, gamma_max: int) -> int:
    best, best_s = 1, -1.0
    for g in range(1, gamma_max + 1):
        s = speedup(alpha, g, c)
        if s > best_s:
            best, best_s = g, s
    return best


def acceptance_length(alphas: Sequence[float]) -> float:
    tau, run = 1.0, 1.0
    for a in alphas:
        run *= a
        tau += run
    return tau

"""Helpers shared by the GPU tests: upload a synthetic batch, run the HIP
path through the C ABI, run the oracle, compare under the parity rules."""
import dataclasses
import sys

import numpy as np

from speculative_sampling_verification_verify_amd import binding, synth
import oracle

TOL = 1e-5          # probability / overlap tolerance and decision-margin threshold


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def logits_to_dev(arr, dev):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16), binding.SV_BF16
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev), binding.SV_FP32


@dataclasses.dataclass
class GpuOut:
    tokens: np.ndarray
    n: np.ndarray
    alpha: np.ndarray
    pq: np.ndarray


def run_gpu(bt, dev="cuda:0", verifier=None, with_params=True, pass_gamma=True):
    import torch
    P, dt = logits_to_dev(bt.p_logits, dev)
    Q, _ = logits_to_dev(bt.q_logits, dev)
    ver = verifier or binding.Verifier(bt.B, bt.gamma_max, bt.V, dt, device=dev)
    tok, n, alpha, pq = ver(P, Q, to_dev(bt.draft, dev), to_dev(bt.u, dev), to_dev(bt.temperature, dev),
                            to_dev(bt.top_k, dev) if with_params else None,
                            to_dev(bt.top_p, dev) if with_params else None,
                            to_dev(bt.gamma_len, dev) if pass_gamma else None)
    torch.cuda.synchronize()
    return GpuOut(tok.cpu().numpy(), n.cpu().numpy(), alpha.cpu().numpy(), pq.cpu().numpy())


def run_oracle(bt, processes=1):
    return oracle.verify_batch(bt.p_logits, bt.q_logits, bt.draft, bt.u, bt.temperature, bt.top_k, bt.top_p,
                               bt.gamma_len, processes=processes)


@dataclasses.dataclass
class Report:
    rows: int
    near: int            # sequences whose n / tokens decision margin is below TOL
    near_differ: int     # of those, sequences whose n or tokens differ
    max_alpha_err: float
    max_pq_err: float
    invalid: int
    positions: int       # used draft positions of the valid sequences
    compared: int        # of those, positions whose alpha and p(x), q(x) were compared

    @property
    def compared_share(self):
        return self.compared / self.positions if self.positions else 1.0


def compare(bt, g: GpuOut, ref, label="", min_compared_share=None):
    """Assert the parity rules; return counts for reporting.

    n and the tokens must match wherever the oracle's decision margin (the
    acceptance tests made, the draw, and the nucleus boundaries of the rows
    that decided them) is at least TOL.  alpha_i and (p_i(x_i), q_i(x_i))
    must be within TOL at every position whose two rows have no nucleus
    boundary within TOL; padded positions must hold 0.  With
    min_compared_share, at least that share of the valid sequences' used
    positions must have been compared."""
    near = ref.margin < TOL
    same = (g.n == ref.n) & (g.tokens == ref.tokens).all(axis=1)
    bad = ~same & ~near
    if bad.any():
        i = int(np.nonzero(bad)[0][0])
        raise AssertionError(
            f"{label}: {int(bad.sum())} rows differ outside the margin; first b={i}: gpu n={g.n[i]} "
            f"tokens={g.tokens[i].tolist()} | oracle n={ref.n[i]} tokens={ref.tokens[i].tolist()} "
            f"margin={ref.margin[i]:.3g} T={bt.temperature[i]} k={bt.top_k[i]} top_p={bt.top_p[i]} "
            f"gamma={bt.gamma_len[i]}")
    invalid = ref.n < 0
    assert (g.n[invalid] == -1).all() and (g.tokens[invalid] == -1).all(), f"{label}: sentinel rows"
    assert np.isnan(g.alpha[invalid]).all(), f"{label}: sentinel alpha"
    # Overlap and probabilities, position by position.
    G = ref.alpha.shape[1]
    used = np.arange(G)[None, :] < np.asarray(bt.gamma_len)[:, None]
    cmp_pos = ~invalid[:, None] & (ref.topp_pos >= TOL)
    ea = np.where(cmp_pos, np.abs(g.alpha - ref.alpha), 0.0)
    ep = np.where(cmp_pos[:, :, None], np.abs(g.pq - ref.pq), 0.0)
    max_a = float(ea.max()) if ea.size else 0.0
    max_p = float(ep.max()) if ep.size else 0.0
    if max_a > TOL or max_p > TOL or np.isnan(max_a) or np.isnan(max_p):
        ia = np.unravel_index(int(np.nanargmax(ea)), g.alpha.shape)
        raise AssertionError(f"{label}: alpha err {max_a:.3g}, pq err {max_p:.3g}; worst alpha at {ia}: "
                             f"gpu {g.alpha[ia]} oracle {ref.alpha[ia]}")
    positions = int((used & ~invalid[:, None]).sum())
    compared = int((used & cmp_pos).sum())
    rep = Report(int(len(g.n)), int(near.sum()), int((near & ~same).sum()), max_a, max_p, int(invalid.sum()),
                 positions, compared)
    if min_compared_share is not None:
        assert rep.compared_share >= min_compared_share, \
            f"{label}: alpha / pq compared on {compared} of {positions} positions ({rep.compared_share:.3f})"
    return rep

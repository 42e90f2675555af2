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
    near: int            # rows with a decision margin below TOL
    near_differ: int     # of those, rows whose n or tokens differ
    max_alpha_err: float
    max_pq_err: float
    invalid: int


def compare(bt, g: GpuOut, ref, label=""):
    """Assert the parity rules; return counts for reporting."""
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
    # Overlap and probabilities: every valid row whose top-p boundaries are
    # not within the margin.
    cmp_rows = ~invalid & (ref.margin_topp >= TOL)
    ea = np.abs(g.alpha[cmp_rows] - ref.alpha[cmp_rows])
    ep = np.abs(g.pq[cmp_rows] - ref.pq[cmp_rows])
    max_a = float(ea.max()) if ea.size else 0.0
    max_p = float(ep.max()) if ep.size else 0.0
    if max_a > TOL or max_p > TOL:
        ia = np.unravel_index(int(np.argmax(np.abs(g.alpha - ref.alpha) * cmp_rows[:, None])), g.alpha.shape)
        raise AssertionError(f"{label}: alpha err {max_a:.3g}, pq err {max_p:.3g}; worst alpha at {ia}: "
                             f"gpu {g.alpha[ia]} oracle {ref.alpha[ia]}")
    return Report(int(len(g.n)), int(near.sum()), int((near & ~same).sum()), max_a, max_p, int(invalid.sum()))

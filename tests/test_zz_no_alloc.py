"""spec_verify_noalloc (the allocation-free entry point, whose workspace is a
fixed per-GPU array inside the library) against spec_verify_ex with a caller
workspace: the same kernels, so the outputs must be identical.  Two calls in
a row on each shape, the second with a smaller input, so the second call runs
on what the first left in the shared array."""
import numpy as np
import pytest
import torch

from speculative_sampling_verification_verify_amd import binding, synth
from gpu_util import compare, log, logits_to_dev, run_oracle, to_dev

pytestmark = pytest.mark.gpu


def _inputs(bt, dev):
    P, dt = logits_to_dev(bt.p_logits, dev)
    Q, _ = logits_to_dev(bt.q_logits, dev)
    return P, Q, dt, to_dev(bt.draft, dev), to_dev(bt.u, dev), to_dev(bt.temperature, dev), \
        to_dev(bt.top_k, dev), to_dev(bt.top_p, dev), to_dev(bt.gamma_len, dev)


def _run_both(bt, hints, dev="cuda:0"):
    P, Q, dt, d, u, T, k, tp, gl = _inputs(bt, dev)
    B, G, V = bt.B, bt.gamma_max, bt.V
    ref = binding.Verifier(B, G, V, dt, device=dev, hints=hints)
    rt, rn, ra, rpq = ref(P, Q, d, u, T, k, tp, gl)
    out_t = torch.full((B, G + 1), -7, dtype=torch.int32, device=dev)
    out_n = torch.full((B,), -7, dtype=torch.int32, device=dev)
    out_a = torch.full((B, G), -7.0, dtype=torch.float32, device=dev)
    out_pq = torch.full((B, G, 2), -7.0, dtype=torch.float32, device=dev)
    binding.spec_verify_noalloc(P, Q, d, gl, u, T, k, tp, out_t, out_n, out_a, out_pq, hints=hints)
    torch.cuda.synchronize()
    return (rt.cpu().numpy(), rn.cpu().numpy(), ra.cpu().numpy(), rpq.cpu().numpy()), \
        (out_t.cpu().numpy(), out_n.cpu().numpy(), out_a.cpu().numpy(), out_pq.cpu().numpy())


def _same(label, a, b):
    for name, x, y in zip(("tokens", "n", "alpha", "pq"), a, b):
        assert np.array_equal(x, y, equal_nan=True), f"{label}: {name} differs from the workspace entry point"


# (workload, first (B, V), second (B, V), hints): each pair of calls shrinks.
CASES = [
    (3, (48, 40000), (12, 9000), binding.SV_HINT_NO_DENSE),     # top-k sequences: select + finisher
    (4, (24, 60000), (8, 20000), 0),                            # mixed: argmax and dense top-p rows in one launch
    (1, (16, 32000), (6, 3000), binding.SV_HINT_ALL_DENSE),     # unfiltered: pair kernel, rows in LDS
    (0, (64, 1000), (5, 700), 0),                               # fp32 rows
]


@pytest.mark.parametrize("cid,first,second,hints", CASES)
def test_noalloc_matches_workspace_entry_point(cid, first, second, hints):
    for step, (B, V) in enumerate((first, second)):
        bt = synth.make_batch(cid, B=B, V=V, seed=synth.BASE_SEED + 1000 + 17 * step + cid)
        log(f"noalloc: workload {cid} call {step} B={B} V={V} hints={hints}")
        ref, got = _run_both(bt, hints)
        _same(f"workload {cid} call {step}", ref, got)
        # And the parity rules against the oracle, for the allocation-free outputs.
        g = type("G", (), {})()
        g.tokens, g.n, g.alpha, g.pq = got
        r = compare(bt, g, run_oracle(bt), label=f"noalloc workload {cid} call {step}")
        log(f"noalloc: workload {cid} call {step}: {r}")


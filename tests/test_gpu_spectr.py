"""Multi-candidate verify (K-SEQ at every node, SpecTr walk) on the GPU,
through the C ABI, against the CPU oracle on the same seeded inputs.  n and
every output token must be identical except in sequences whose oracle
decision margin (acceptance threshold, CDF boundary, top-p boundary) is
below 1e-5."""
import numpy as np
import pytest

from speculative_sampling_verification_verify_amd import synth
import oracle
from gpu_util import TOL, log, logits_to_dev, to_dev

pytestmark = pytest.mark.gpu


def run_gpu_spectr(sb, dev="cuda:0"):
    import torch
    from speculative_sampling_verification_verify_amd import binding
    P, _ = logits_to_dev(sb.p_logits, dev)
    Q, _ = logits_to_dev(sb.q_logits, dev)
    ver = binding.SpectrVerifier(sb.B, sb.K, sb.L, device=dev)
    tok, n = ver(P, Q, to_dev(sb.cand, dev), to_dev(sb.u, dev), to_dev(sb.temperature, dev),
                 to_dev(sb.top_k, dev), to_dev(sb.top_p, dev))
    torch.cuda.synchronize()
    return tok.cpu().numpy(), n.cpu().numpy()


def check_spectr(sb, label, rows=None):
    log(f"[spectr] {label}: B={sb.B} K={sb.K} L={sb.L} V={sb.V} dtype={sb.p_logits.dtype}")
    tok, n = run_gpu_spectr(sb)
    rows = list(range(sb.B)) if rows is None else list(rows)
    ref = oracle.kseq.spectr_batch(sb.p_logits, sb.q_logits, sb.cand, sb.u, sb.temperature, sb.top_k, sb.top_p,
                                   rows=rows)
    near = ref.margin < TOL
    same = (n[rows] == ref.n) & (tok[rows] == ref.tokens).all(1)
    bad = ~same & ~near
    if bad.any():
        i = int(np.nonzero(bad)[0][0])
        b = rows[i]
        raise AssertionError(f"{label}: {int(bad.sum())} sequences differ; first b={b}: gpu n={n[b]} "
                             f"tokens={tok[b].tolist()} | oracle n={ref.n[i]} tokens={ref.tokens[i].tolist()} "
                             f"margin={ref.margin[i]:.3g} T={sb.temperature[b]} k={sb.top_k[b]} top_p={sb.top_p[b]}")
    log(f"[spectr] {label}: ok, {len(rows)} sequences, near-margin {int(near.sum())} "
        f"(differ {int((near & ~same).sum())}), mean tokens per round {np.mean(ref.n[ref.n >= 0] + 1):.3f}")
    return tok, n, ref


@pytest.mark.parametrize("B,K,L,V,dtype", [
    (12, 4, 4, 32000, "bf16"),     # rows in LDS, vector path
    (40, 8, 3, 1000, "fp32"),      # small fp32 rows
    (6, 3, 2, 50000, "bf16"),      # rows streamed from global memory
    (8, 2, 5, 7001, "bf16"),       # odd V: scalar elements
    (10, 1, 4, 4000, "bf16"),      # one candidate: the ordinary verify
])
def test_spectr_shapes(B, K, L, V, dtype):
    rng = np.random.default_rng(V + K)
    T = rng.choice(np.array([0.0, 0.6, 1.0, 1.3], np.float32), size=B)
    k = rng.choice(np.array([0, 0, 40, 700], np.int32), size=B)
    tp = rng.choice(np.array([1.0, 1.0, 0.9], np.float32), size=B)
    sb = synth.make_spectr_batch(B, K, L, V, dtype=dtype, seed=100 + V, temperature=T, top_k=k, top_p=tp)
    check_spectr(sb, f"B{B}-K{K}-L{L}-V{V}-{dtype}")


def test_spectr_duplicates_and_invalid():
    sb = synth.make_spectr_batch(8, 4, 3, 3000, sigma=0.05, temperature=0.9)   # near-identical drafter: repeats
    P, cand, u, T = sb.p_logits.copy(), sb.cand.copy(), sb.u.copy(), sb.temperature.copy()
    cand[1, 2, 1] = sb.V                   # candidate out of range
    u[2, 1, 0] = 1.0                       # uniform out of range
    T[3] = -1.0                            # bad temperature
    P[4, :, 0, 11] = 0x7FC0                # NaN on the root node's target row
    cand[5] = cand[5, :1]                  # all candidates identical
    sb2 = synth.SpectrBatch(sb.name, P, sb.q_logits, cand, u, T, sb.top_k, sb.top_p, sb.seed)
    tok, n, ref = check_spectr(sb2, "duplicates-invalid")
    assert (n[1:5] == -1).all() and (tok[1:5] == -1).all()
    assert n[0] >= 0 and n[5] >= 0


def test_spectr_bench_shape_sampled():
    """The benchmark's shape and launch (B = 32, K = 8, L = 8, V = 32000, bf16,
    T = 0.8), every sequence checked against the oracle (the candidates of a
    close drafter share prefixes, so the rho* search with its LDS list runs at
    the shallow nodes)."""
    sb = synth.make_spectr_batch(32, 8, 8, 32000, dtype="bf16", temperature=0.8)
    check_spectr(sb, "bench-shape")


@pytest.mark.parametrize("B,K,L,V,dtype", [
    (3, 64, 2, 500, "bf16"),    # K at its limit: the walk's 64-bit class masks, 64 lanes of candidates
    (2, 2, 64, 300, "fp32"),    # L at its limit: 65 depths staged in the walk's LDS
])
def test_spectr_size_limits(B, K, L, V, dtype):
    sb = synth.make_spectr_batch(B, K, L, V, dtype=dtype, seed=300 + K + L, sigma=0.2, temperature=0.9)
    check_spectr(sb, f"limits-B{B}-K{K}-L{L}-V{V}-{dtype}")


def test_spectr_extreme_temperatures():
    """Near-one-hot (T = 1e-3) and near-uniform (T = 30) processed rows, with
    and without top-p, in the K-SEQ nodes."""
    T = np.array([1e-3, 30.0, 1e-3, 30.0, 0.05, 8.0], np.float32)
    tp = np.array([1.0, 1.0, 0.9, 0.9, 1.0, 0.95], np.float32)
    sb = synth.make_spectr_batch(6, 6, 3, 4000, dtype="bf16", seed=77, sigma=0.3, temperature=T, top_p=tp)
    check_spectr(sb, "extreme-T")

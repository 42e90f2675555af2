"""GPU paths of the lenient verify (spec_verify_ex), the one-token sampler
(spec_sample) and the shared-noise drafter's sampler (spec_sample_gumbel),
through the C ABI, against the CPU oracle on the same seeded inputs.  Tokens
and n must be identical except where the oracle's decision margin is below
1e-5; overlap and p(x), q(x) within 1e-5."""
import numpy as np
import pytest

from speculative_sampling_verification_verify_amd import synth
import oracle
from gpu_util import TOL, compare, log, logits_to_dev, to_dev

pytestmark = pytest.mark.gpu


def run_gpu_lenient(bt, lenience, dev="cuda:0"):
    import torch
    from speculative_sampling_verification_verify_amd import binding
    from gpu_util import GpuOut
    P, dt = logits_to_dev(bt.p_logits, dev)
    Q, _ = logits_to_dev(bt.q_logits, dev)
    ver = binding.Verifier(bt.B, bt.gamma_max, bt.V, dt, device=dev)
    tok, n, alpha, pq = ver(P, Q, to_dev(bt.draft, dev), to_dev(bt.u, dev), to_dev(bt.temperature, dev),
                            to_dev(bt.top_k, dev), to_dev(bt.top_p, dev), to_dev(bt.gamma_len, dev),
                            lenience=to_dev(np.asarray(lenience, np.float32), dev))
    torch.cuda.synchronize()
    return GpuOut(tok.cpu().numpy(), n.cpu().numpy(), alpha.cpu().numpy(), pq.cpu().numpy())


@pytest.mark.parametrize("cid,B,V", [(3, 12, 30000), (1, 12, 32000), (4, 24, 20000), (0, 64, 1000)])
def test_lenient_verify(cid, B, V):
    bt = synth.make_batch(cid, B=B, V=V)
    rng = np.random.default_rng(cid)
    lv = rng.choice(np.array([1.0, 0.8, 0.5, 0.3, 0.1, 0.0], np.float32), size=bt.B)
    log(f"[lenient] workload{cid} B={bt.B} V={bt.V}")
    g = run_gpu_lenient(bt, lv)
    ref = oracle.verify_batch(bt.p_logits, bt.q_logits, bt.draft, bt.u, bt.temperature, bt.top_k, bt.top_p,
                              bt.gamma_len, processes=1, lenience=lv)
    rep = compare(bt, g, ref, f"lenient-{cid}")
    log(f"[lenient] workload{cid}: ok {rep}; mean n at l<1: {ref.n[(lv < 1) & (ref.n >= 0)].mean():.3f}, "
        f"at l=1: {ref.n[(lv == 1) & (ref.n >= 0)].mean() if (lv == 1).any() else float('nan'):.3f}")


def test_lenience_out_of_range_rows_are_invalid():
    bt = synth.make_batch(3, B=6, V=9000)
    lv = np.array([1.0, -0.5, 1.5, np.nan, 0.0, 0.5], np.float32)
    g = run_gpu_lenient(bt, lv)
    ref = oracle.verify_batch(bt.p_logits, bt.q_logits, bt.draft, bt.u, bt.temperature, bt.top_k, bt.top_p,
                              bt.gamma_len, processes=1, lenience=lv)
    compare(bt, g, ref, "lenience-range")
    assert (g.n[1:4] == -1).all() and (g.n[[0, 4, 5]] >= 0).all()


def _sample_inputs(R, V, dtype, seed):
    rng = np.random.default_rng(seed)
    rank = np.stack([rng.permutation(V) for _ in range(R)])
    z = (3.0 * rng.normal(size=(R, V)) - 1.1 * np.log1p(rank)).astype(np.float32)
    T = rng.choice(np.array([0.0, 0.6, 1.0, 1.3], np.float32), size=R)
    k = rng.choice(np.array([0, 0, 1, 50, 700], np.int32), size=R)
    tp = rng.choice(np.array([1.0, 1.0, 0.9, 0.5], np.float32), size=R)
    u = rng.random(R).astype(np.float32)
    logits = synth.f32_to_bf16_bits(z) if dtype == "bf16" else z
    return logits, u, T, k, tp


@pytest.mark.parametrize("dtype,V,R", [("bf16", 152064, 64), ("bf16", 32000, 96), ("fp32", 1000, 300),
                                       ("bf16", 5001, 40), ("bf16", 70000, 24)])
def test_sampler_against_oracle(dtype, V, R):
    import torch
    from speculative_sampling_verification_verify_amd import binding
    logits, u, T, k, tp = _sample_inputs(R, V, dtype, seed=V % 101)
    u[3] = 1.0                                       # invalid uniform
    if dtype == "bf16":
        logits[5, 7] = 0x7FC0                        # NaN logit
    log(f"[sample] {dtype} V={V} R={R}")
    L, dt = logits_to_dev(logits, "cuda:0")
    smp = binding.Sampler(R, V, dt, device="cuda:0")
    tok = smp(L, to_dev(u, "cuda:0"), to_dev(T, "cuda:0"), to_dev(k, "cuda:0"), to_dev(tp, "cuda:0"))
    torch.cuda.synchronize()
    tok = tok.cpu().numpy()
    ref = oracle.sample_batch(logits, u, T, k, tp)
    near = ref.margin < TOL
    bad = (tok != ref.tokens) & ~near
    assert not bad.any(), (np.nonzero(bad)[0][:5], tok[bad][:5], ref.tokens[bad][:5])
    assert tok[3] == -1 and ref.tokens[3] == -1
    log(f"[sample] {dtype} V={V}: ok, near-margin {int(near.sum())} (differ {int((near & (tok != ref.tokens)).sum())})")


def test_sampler_follows_processed_softmax():
    import torch
    from scipy import stats
    from speculative_sampling_verification_verify_amd import binding
    N, V = 40000, 10
    rng = np.random.default_rng(4)
    z = (1.4 * rng.normal(size=V)).astype(np.float32)
    logits = np.broadcast_to(z, (N, V)).copy()
    u = rng.random(N).astype(np.float32)
    T = np.full(N, 0.9, np.float32)
    smp = binding.Sampler(N, V, binding.SV_FP32, device="cuda:0")
    tok = smp(to_dev(logits, "cuda:0"), to_dev(u, "cuda:0"), to_dev(T, "cuda:0")).cpu().numpy()
    s = z.astype(np.float64) / 0.9
    p = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    pv = stats.chisquare(np.bincount(tok, minlength=V), p * N).pvalue
    log(f"[sample] chi-square p-value {pv:.3g}")
    assert pv > 1e-4


@pytest.mark.parametrize("dtype,V,R", [("bf16", 152064, 48), ("fp32", 1000, 200), ("bf16", 7001, 40)])
def test_gumbel_sampler_and_coupled_round(dtype, V, R):
    # The drafter samples with spec_sample_gumbel; the verify then runs with
    # the same noise: every position must match the oracle exactly.
    import torch
    from speculative_sampling_verification_verify_amd import binding
    logits, _, T, k, tp = _sample_inputs(R, V, dtype, seed=V % 53)
    noise = synth.gumbel_noise_rows(9, 0, R, V)
    Ld, _ = logits_to_dev(logits, "cuda:0")
    tok = binding.spec_sample_gumbel(Ld, to_dev(noise, "cuda:0"), to_dev(T, "cuda:0"), to_dev(k, "cuda:0"),
                                     to_dev(tp, "cuda:0"))
    torch.cuda.synchronize()
    tok = tok.cpu().numpy()
    ref = np.array([oracle.gumbel_target_token(oracle.decode_row(logits[r]), noise[r], float(T[r]), int(k[r]),
                                               float(tp[r])) for r in range(R)], dtype=object)
    ref_tok = np.array([int(t) for t, _ in ref])
    near = np.array([m < TOL for _, m in ref])
    assert ((tok == ref_tok) | near).all(), np.nonzero((tok != ref_tok) & ~near)[0][:5]
    log(f"[gumbel-sample] {dtype} V={V}: ok, near-margin {int(near.sum())}")
    # One coupled round: 6 sequences of gamma = 3 built from the same rows.
    if R >= 24:
        G, Bq = 3, 6
        rows = np.arange(Bq * (G + 1)).reshape(Bq, G + 1)
        P = logits[rows]
        Nz = noise[rows]
        draft = tok[rows[:, :G]].astype(np.int32)
        draft[::2, 1] = (draft[::2, 1] + 1) % V              # some disagreements
        base = synth.make_gumbel_batch(0, B=2, V=64)
        Tb = T[rows[:, 0]]
        kb, tpb = k[rows[:, 0]], tp[rows[:, 0]]
        # rows of one sequence share the sequence's parameters: rebuild drafts accordingly
        for b in range(Bq):
            for i in range(G):
                draft[b, i] = oracle.gumbel_target_token(oracle.decode_row(P[b, i]), Nz[b, i], float(Tb[b]),
                                                         int(kb[b]), float(tpb[b]))[0]
        draft[::2, 1] = (draft[::2, 1] + 1) % V
        gb = synth.GumbelBatch(base.workload, P, Nz, draft, np.full(Bq, G, np.int32), Tb, kb, tpb, 0)
        from test_gpu_gumbel import check_gumbel
        check_gumbel(gb, f"coupled-round-{dtype}-V{V}")


def test_no_dense_hint_keeps_dense_rows_exact():
    # The hint only skips the dense-pair launch; dense sequences in such a
    # call take the one-workgroup-per-sequence path and still match.
    import torch
    from speculative_sampling_verification_verify_amd import binding
    from gpu_util import GpuOut
    bt = synth.make_batch(4, B=16, V=20000)          # mixed greedy and top-p rows: some dense
    P, dt = logits_to_dev(bt.p_logits, "cuda:0")
    Q, _ = logits_to_dev(bt.q_logits, "cuda:0")
    ver = binding.Verifier(bt.B, bt.gamma_max, bt.V, dt, device="cuda:0", hints=binding.SV_HINT_NO_DENSE)
    tok, n, alpha, pq = ver(P, Q, to_dev(bt.draft, "cuda:0"), to_dev(bt.u, "cuda:0"),
                            to_dev(bt.temperature, "cuda:0"), to_dev(bt.top_k, "cuda:0"), to_dev(bt.top_p, "cuda:0"),
                            to_dev(bt.gamma_len, "cuda:0"))
    torch.cuda.synchronize()
    g = GpuOut(tok.cpu().numpy(), n.cpu().numpy(), alpha.cpu().numpy(), pq.cpu().numpy())
    ref = oracle.verify_batch(bt.p_logits, bt.q_logits, bt.draft, bt.u, bt.temperature, bt.top_k, bt.top_p,
                              bt.gamma_len, processes=1)
    compare(bt, g, ref, "no-dense-hint")

"""A seeded sweep of shapes and sampling settings across the kernels' regimes
(rows held in LDS, value-histogram rows, streamed fp32 rows, split pairs
under the unfiltered hint, top-k lists), against the oracle under the
parity rules.  Each case draws its sizes, temperatures, filters and
special entries (-inf, ties) from its own seed, so the sweep is the same
on every run."""
import numpy as np
import pytest

from speculative_sampling_verification_verify_amd import binding, synth
from gpu_util import compare, log, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

# (regime, seed): V ranges per regime.
REGIMES = {
    "lds": (2000, 32768, "bf16"),
    "hist": (32776, 131072, "bf16"),
    "fp32": (9000, 40000, "fp32"),
    "split": (40000, 152064, "bf16"),
    "topk": (30000, 160000, "bf16"),
}
CASES = [(r, s) for r in REGIMES for s in range(4)]


def _case(regime, seed):
    rng = np.random.default_rng(7000 + 97 * list(REGIMES).index(regime) + seed)
    lo, hi, dtype = REGIMES[regime]
    V = int(rng.integers(lo, hi + 1))
    if dtype == "bf16" and regime in ("hist", "split"):
        V -= V % 8                                  # whole 16-byte units: these kernels' rows
    B = int(rng.integers(1, 7))
    G = int(rng.integers(1, 6))
    T = rng.choice([0.0, 0.3, 0.7, 1.0, 1.4, 3.0], size=B).astype(np.float32)
    if regime == "split":
        T = np.maximum(T, 0.3).astype(np.float32)
        k = np.zeros(B, np.int32)
        tp = np.ones(B, np.float32)
    elif regime == "topk":
        k = rng.choice([1, 8, 50, 200, 512], size=B).astype(np.int32)
        tp = rng.choice([1.0, 0.9, 0.5], size=B).astype(np.float32)
    else:
        k = rng.choice([0, 0, 600, V + 5], size=B).astype(np.int32)
        tp = rng.choice([1.0, 1.0, 0.95, 0.8, 0.3], size=B).astype(np.float32)
    rank = np.stack([rng.permutation(V) for _ in range(B)])[:, None, :]
    scale = rng.uniform(1.0, 4.0)
    zp = (scale * rng.normal(size=(B, G + 1, V)) - 1.1 * np.log1p(rank)).astype(np.float32)
    zq = (zp[:, :G] + rng.uniform(0.2, 1.5) * rng.normal(size=(B, G, V))).astype(np.float32)
    # Special entries: a block of -inf in one sequence, a tie group at the top of another.
    if B > 1:
        zp[0, :, : V // 7] = -np.inf
        zq[0, :, V // 9: V // 5] = -np.inf
    last = zp[-1]                                    # a view: the assignment below writes zp
    last[:, rng.integers(0, V, size=40)] = last.max(axis=-1, keepdims=True)
    gl = rng.integers(1, G + 1, size=B).astype(np.int32)
    gum = -np.log(-np.log(rng.random(size=zq.shape)))
    draft = np.argmax(zq / np.maximum(T, 1e-3)[:, None, None] + gum, axis=2).astype(np.int32)
    cast = (lambda x: synth.f32_to_bf16_bits(np.asarray(x, np.float32))) if dtype == "bf16" else \
        (lambda x: np.asarray(x, np.float32))
    w = synth.make_batch(0, B=1, V=8).workload
    return synth.Batch(w, cast(zp), cast(zq), draft, synth.uniforms(100 + seed, B, G), gl, T, k, tp, seed)


@pytest.mark.parametrize("regime,seed", CASES)
def test_sweep(regime, seed):
    bt = _case(regime, seed)
    hints = binding.SV_HINT_UNFILTERED if regime == "split" else 0
    dt = binding.SV_BF16 if bt.p_logits.dtype == np.uint16 else binding.SV_FP32
    log(f"[sweep] {regime} seed {seed}: B={bt.B} G={bt.gamma_max} V={bt.V} {bt.p_logits.dtype} hints={hints}")
    ver = binding.Verifier(bt.B, bt.gamma_max, bt.V, dt, device="cuda:0", hints=hints)
    ref = run_oracle(bt)
    for call in range(2):
        rep = compare(bt, run_gpu(bt, verifier=ver), ref, f"sweep-{regime}-{seed}-call{call}")
    log(f"[sweep] {regime} seed {seed}: ok {rep}")

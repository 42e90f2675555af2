"""Seeded synthetic inputs for the batched speculative-sampling verify step.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It only *makes inputs*: logits for the target (gamma+1 positions)
and the drafter (gamma positions), the drafter's proposed tokens, per-row
sampling parameters, and the counter-based uniforms that the verify step
consumes.  It computes none of the verify step itself (no acceptance test, no
residual, no overlap).

The drafter's proposal x_i is, by the method's own definition, a sample from
the drafter's processed distribution (Leviathan et al., as summarised on the
speculative-decoding review page, "Speculative Sampling": x ~ q after the
sampling adjustments).  The drafter is outside the verify step, so this module
simulates it with its own small sampler (Gumbel-max over the drafter's
candidate set, see ``_drafter_sample``).  Nothing that the verify step outputs
is derived from that sampler: any token in [0, V) is a legal input.

Value recipe (one sequence b, position j, vocab entry v):
    z_p[b, j, v] = scale * g[b, j, v] - slope * log(1 + pi_b(v))
    z_q[b, i, v] = z_p[b, i, v] + sigma_b * n[b, i, v]
with g, n ~ N(0, 1) and pi_b a seeded permutation of the vocabulary (a
Zipf-like rank profile placed at random vocabulary ids).  bf16 configurations
round the float32 values to bfloat16 with round-to-nearest-even; the stored
bf16 bits are the ground truth for every consumer.

Uniforms: u[b, j] for j < gamma_max are the acceptance draws r_1..r_gamma; the
single residual/bonus draw sits at u[b, gamma_max].  Each is the first 64-bit
word of Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11) at counter
(b, j, 4, 0) under key (seed, 0), shifted right by 40 bits and scaled by 2^-24,
so every uniform is an exact float32 in [0, 1).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BASE_SEED = 20261202

# Counter-stream ids.
(STREAM_PERM, STREAM_TARGET, STREAM_DRAFT_NOISE, STREAM_DRAFT_SAMPLE, STREAM_UNIFORM, STREAM_ROWPARAM,
 STREAM_GUMBEL) = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload shape (sizes, value recipe, sampling settings)."""
    cid: int
    name: str
    B: int
    V: int
    gamma_max: int
    dtype: str                 # "bf16" or "fp32"
    scale: float
    slope: float
    sigma: float               # drafter noise; ignored when sigma_choices is set
    temperature: float         # ignored when t_choices is set
    top_k: int = 0             # <= 0 => off
    top_p: float = 1.0         # >= 1 => off
    ragged_gamma: bool = False  # per-row gamma_b ~ U{1..gamma_max}
    t_choices: tuple = ()
    sigma_choices: tuple = ()


WORKLOADS = {
    # Tiny reference: 1000 independent single-sequence rounds, fp32 logits.
    0: Workload(0, "tiny-fp32-V1000-g4", B=1000, V=1000, gamma_max=4, dtype="fp32",
                scale=2.0, slope=1.0, sigma=1.0, temperature=1.0),
    1: Workload(1, "B32-V32000-g5-T0.8", B=32, V=32000, gamma_max=5, dtype="bf16",
                scale=3.0, slope=1.1, sigma=0.5, temperature=0.8),
    2: Workload(2, "B64-V128256-g4-topk50", B=64, V=128256, gamma_max=4, dtype="bf16",
                scale=3.0, slope=1.1, sigma=1.0, temperature=1.0, top_k=50),
    3: Workload(3, "B256-V152064-g7-T0.7-topk64", B=256, V=152064, gamma_max=7, dtype="bf16",
                scale=3.0, slope=1.2, sigma=0.5, temperature=0.7, top_k=64),
    4: Workload(4, "B128-V128256-mixed-g1..8-topp0.9", B=128, V=128256, gamma_max=8, dtype="bf16",
                scale=3.0, slope=1.1, sigma=1.0, temperature=1.0, top_p=0.9, ragged_gamma=True,
                t_choices=(0.0, 0.6, 1.0, 1.3), sigma_choices=(0.3, 1.0, 2.0)),
}


# ----------------------------------------------------------------------------
# Philox4x64-10, vectorised over counters (published definition, SC'11).
# ----------------------------------------------------------------------------
_PHILOX_M0 = np.uint64(0xD2E7470EE14C6C93)
_PHILOX_M1 = np.uint64(0xCA5A826395121157)
_PHILOX_W0 = np.uint64(0x9E3779B97F4A7C15)
_PHILOX_W1 = np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)


def _mulhilo64(a: np.uint64, b: np.ndarray):
    """Full 64x64 -> 128-bit product of a scalar and an array, as (hi, lo)."""
    a_lo, a_hi = a & _LO32, a >> np.uint64(32)
    b_lo, b_hi = b & _LO32, b >> np.uint64(32)
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> np.uint64(32)) + (lh & _LO32) + (hl & _LO32)
    lo = (ll & _LO32) | ((mid & _LO32) << np.uint64(32))
    hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64_10(c0, c1, c2, c3, k0, k1):
    """Philox4x64 with 10 rounds on arrays of counters; returns the 4 output words."""
    with np.errstate(over="ignore"):
        x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64).copy() for c in (c0, c1, c2, c3))
        x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
        x0, x1, x2, x3 = x0.copy(), x1.copy(), x2.copy(), x3.copy()
        k0 = np.uint64(k0)
        k1 = np.uint64(k1)
        for _ in range(10):
            hi0, lo0 = _mulhilo64(_PHILOX_M0, x0)
            hi1, lo1 = _mulhilo64(_PHILOX_M1, x2)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
            k0 = k0 + _PHILOX_W0
            k1 = k1 + _PHILOX_W1
    return x0, x1, x2, x3


def uniforms(seed: int, B: int, gamma_max: int, row0: int = 0) -> np.ndarray:
    """[B, gamma_max+1] float32 uniforms in [0, 1): Philox(seed, row, pos)."""
    rows = np.arange(row0, row0 + B, dtype=np.uint64)[:, None]
    pos = np.arange(gamma_max + 1, dtype=np.uint64)[None, :]
    w0, _, _, _ = philox4x64_10(rows, pos, np.uint64(STREAM_UNIFORM), np.uint64(0), seed, 0)
    return ((w0 >> np.uint64(40)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


# ----------------------------------------------------------------------------
# bf16 storage helpers (bit manipulation only).
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits.

    NaN inputs become a quiet NaN of the same sign."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = ((b[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Generation.
# ----------------------------------------------------------------------------
def _rng(seed: int, stream: int, row: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=[seed, stream], counter=[0, row, 0, 0]))


@dataclasses.dataclass
class Batch:
    """Host copy of one verify call's inputs.

    p_logits: [B, gamma_max+1, V] (uint16 bf16 bits, or float32)
    q_logits: [B, gamma_max, V]
    draft:    [B, gamma_max] int32 (padded slots hold 0)
    u:        [B, gamma_max+1] float32
    gamma_len, temperature, top_k, top_p: [B] per-row parameters
    """
    workload: Workload
    p_logits: np.ndarray
    q_logits: np.ndarray
    draft: np.ndarray
    u: np.ndarray
    gamma_len: np.ndarray
    temperature: np.ndarray
    top_k: np.ndarray
    top_p: np.ndarray
    seed: int

    @property
    def B(self):
        return self.p_logits.shape[0]

    @property
    def V(self):
        return self.p_logits.shape[2]

    @property
    def gamma_max(self):
        return self.q_logits.shape[1]

    def logits_f64(self, which: str, b: int) -> np.ndarray:
        arr = self.p_logits if which == "p" else self.q_logits
        row = arr[b]
        if row.dtype == np.uint16:
            return bf16_bits_to_f32(row).astype(np.float64)
        return row.astype(np.float64)


def row_params(w: Workload, seed: int, B: int, row0: int = 0):
    """Per-row gamma_b, temperature, sigma, top-k and top-p."""
    gamma_len = np.full(B, w.gamma_max, dtype=np.int32)
    temperature = np.full(B, w.temperature, dtype=np.float32)
    sigma = np.full(B, w.sigma, dtype=np.float64)
    if w.ragged_gamma or w.t_choices or w.sigma_choices:
        for k in range(B):
            g = _rng(seed, STREAM_ROWPARAM, row0 + k)
            gl = int(g.integers(1, w.gamma_max + 1))
            ti = int(g.integers(0, len(w.t_choices))) if w.t_choices else -1
            si = int(g.integers(0, len(w.sigma_choices))) if w.sigma_choices else -1
            if w.ragged_gamma:
                gamma_len[k] = gl
            if ti >= 0:
                temperature[k] = w.t_choices[ti]
            if si >= 0:
                sigma[k] = w.sigma_choices[si]
    top_k = np.full(B, w.top_k, dtype=np.int32)
    top_p = np.full(B, w.top_p, dtype=np.float32)
    return gamma_len, temperature, sigma, top_k, top_p


def _drafter_sample(zq: np.ndarray, T: float, k: int, top_p: float, rng: np.random.Generator) -> int:
    """The drafter's own token choice for one position (simulated drafter).

    T == 0: the drafter's highest-scoring token (lowest id among equals).
    T > 0: Gumbel-max over the drafter's candidate set: the k highest logits
    when k is active, then the shortest high-to-low prefix holding top_p of
    the tempered mass when top_p < 1."""
    if T == 0.0:
        return int(np.argmax(zq))
    V = zq.shape[0]
    if 0 < k < V:
        part = np.argpartition(-zq, k - 1)[:k]
        order = part[np.argsort(-zq[part], kind="stable")]
    else:
        order = np.argsort(-zq, kind="stable")
    s = zq[order] / T
    if top_p < 1.0:
        w = np.exp(s - s[0])
        c = np.cumsum(w) / w.sum()
        cut = int(np.searchsorted(c, top_p, side="left")) + 1
        order, s = order[:cut], s[:cut]
    gum = -np.log(-np.log(rng.random(s.shape[0]).clip(1e-300, 1.0 - 1e-16)))
    return int(order[int(np.argmax(s + gum))])


def make_sequence(w: Workload, seed: int, b: int, gamma_b: int, T: float, sigma: float,
                  top_k: int, top_p: float):
    """Logits and drafter tokens for one sequence; returns (zp, zq, draft) in storage dtype."""
    V, G = w.V, w.gamma_max
    perm = _rng(seed, STREAM_PERM, b).permutation(V)
    zipf = (w.slope * np.log1p(perm.astype(np.float64))).astype(np.float32)
    g = _rng(seed, STREAM_TARGET, b).standard_normal((G + 1, V), dtype=np.float32)
    zp32 = np.float32(w.scale) * g - zipf[None, :]
    n = _rng(seed, STREAM_DRAFT_NOISE, b).standard_normal((G, V), dtype=np.float32)
    zq32 = zp32[:G] + np.float32(sigma) * n
    if w.dtype == "bf16":
        zp = f32_to_bf16_bits(zp32)
        zq = f32_to_bf16_bits(zq32)
        zq_val = bf16_bits_to_f32(zq).astype(np.float64)
    else:
        zp = zp32
        zq = zq32
        zq_val = zq32.astype(np.float64)
    rng = _rng(seed, STREAM_DRAFT_SAMPLE, b)
    draft = np.zeros(G, dtype=np.int32)
    for i in range(gamma_b):
        draft[i] = _drafter_sample(zq_val[i], float(T), int(top_k), float(top_p), rng)
    return zp, zq, draft


def make_batch(cid: int, B: Optional[int] = None, V: Optional[int] = None, seed: Optional[int] = None,
               row0: int = 0, out_p: Optional[np.ndarray] = None, out_q: Optional[np.ndarray] = None) -> Batch:
    """Generate one call's inputs for workload ``cid``.

    B and V may be overridden to get smaller instances with the same recipe;
    row0 offsets the sequence ids (so that sub-batches of a workload are
    slices of the same stream).  out_p / out_q may be preallocated arrays."""
    w = WORKLOADS[cid]
    if V is not None and V != w.V:
        w = dataclasses.replace(w, V=V, top_k=min(w.top_k, V) if w.top_k else 0)
    B = w.B if B is None else B
    seed = BASE_SEED + cid if seed is None else seed
    G, Vv = w.gamma_max, w.V
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    P = out_p if out_p is not None else np.empty((B, G + 1, Vv), dtype=dt)
    Q = out_q if out_q is not None else np.empty((B, G, Vv), dtype=dt)
    gamma_len, temperature, sigma, top_k, top_p = row_params(w, seed, B, row0)
    draft = np.zeros((B, G), dtype=np.int32)
    for k in range(B):
        zp, zq, d = make_sequence(w, seed, row0 + k, int(gamma_len[k]), float(temperature[k]),
                                  float(sigma[k]), int(top_k[k]), float(top_p[k]))
        P[k] = zp
        Q[k] = zq
        draft[k] = d
    u = uniforms(seed, B, G, row0)
    return Batch(w, P, Q, draft, u, gamma_len, temperature, top_k, top_p, seed)


def algorithmic_bytes(batch: Batch) -> int:
    """Bytes the verify step must read: every used logit row once, plus the
    tokens and uniforms, plus the outputs it writes."""
    el = 2 if batch.p_logits.dtype == np.uint16 else 4
    g = batch.gamma_len.astype(np.int64)
    rows = int((2 * g + 1).sum())
    B, G = batch.B, batch.gamma_max
    small = B * G * 4 + B * (G + 1) * 4 + B * 4 * 3 + B * (G + 1) * 4 + B * 4 + B * G * 4
    return rows * batch.V * el + small


# ----------------------------------------------------------------------------
# Shared-noise (Gumbel coupling) inputs.
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class GumbelBatch:
    """Host copy of one shared-noise verify call's inputs.

    p_logits: [B, gamma_max+1, V] target logits (uint16 bf16 bits, or float32)
    noise:    [B, gamma_max+1, V] float32 Gumbel noise, one vector per position,
              shared by the drafter and the target
    draft:    [B, gamma_max] int32 proposals of a drafter that used the same noise
    gamma_len, temperature, top_k, top_p: [B] per-row parameters
    q_logits: the simulated drafter's logits (inputs of the drafter only)
    """
    workload: Workload
    p_logits: np.ndarray
    noise: np.ndarray
    draft: np.ndarray
    gamma_len: np.ndarray
    temperature: np.ndarray
    top_k: np.ndarray
    top_p: np.ndarray
    seed: int
    q_logits: Optional[np.ndarray] = None

    @property
    def B(self):
        return self.p_logits.shape[0]

    @property
    def V(self):
        return self.p_logits.shape[2]

    @property
    def gamma_max(self):
        return self.p_logits.shape[1] - 1


def gumbel_noise_rows(seed: int, b: int, rows: int, V: int) -> np.ndarray:
    """[rows, V] float32 standard Gumbel noise -log(-log u) of sequence b,
    u uniform in (0, 1) from the sequence's own counter stream."""
    u = _rng(seed, STREAM_GUMBEL, b).random((rows, V))
    u = np.clip(u, 2.0 ** -60, 1.0 - 2.0 ** -53)
    return (-np.log(-np.log(u))).astype(np.float32)


def _coupled_drafter(zq: np.ndarray, g: np.ndarray, T: float, k: int, top_p: float) -> int:
    """The simulated drafter's proposal under shared noise: the highest
    drafter score plus noise over the drafter's candidate set (T == 0: the
    highest drafter logit)."""
    if T == 0.0:
        return int(np.argmax(zq))
    V = zq.shape[0]
    cand = np.ones(V, dtype=bool)
    if 0 < k < V:
        cand &= zq >= np.partition(zq, V - k)[V - k]
    if top_p < 1.0:
        order = np.argsort(-np.where(cand, zq, -np.inf), kind="stable")
        s = zq[order] / T
        w = np.where(np.isfinite(s), np.exp(s - s[0]), 0.0)
        c = np.cumsum(w) / w.sum()
        cut = int(np.searchsorted(c, top_p, side="left")) + 1
        keep = np.zeros(V, dtype=bool)
        keep[order[:cut]] = True
        cand &= keep
    score = (zq.astype(np.float32) + np.float32(T) * g).astype(np.float32)
    return int(np.argmax(np.where(cand, score, np.float32(-np.inf))))


def make_gumbel_batch(cid: int, B: Optional[int] = None, V: Optional[int] = None,
                      seed: Optional[int] = None) -> GumbelBatch:
    """Inputs of the shared-noise verify on workload ``cid``'s shapes and value
    recipe: the same target logits, one noise vector per position, and the
    proposals of a drafter that scored its own logits with the same noise."""
    base = make_batch(cid, B=B, V=V, seed=seed)
    Bn, G, Vv = base.B, base.gamma_max, base.V
    noise = np.empty((Bn, G + 1, Vv), dtype=np.float32)
    draft = np.zeros((Bn, G), dtype=np.int32)
    for b in range(Bn):
        noise[b] = gumbel_noise_rows(base.seed, b, G + 1, Vv)
        zq = base.logits_f64("q", b)
        for i in range(int(base.gamma_len[b])):
            draft[b, i] = _coupled_drafter(zq[i], noise[b, i], float(base.temperature[b]), int(base.top_k[b]),
                                           float(base.top_p[b]))
    w = dataclasses.replace(base.workload, name=base.workload.name + "-gumbel")
    return GumbelBatch(w, base.p_logits, noise, draft, base.gamma_len, base.temperature, base.top_k, base.top_p,
                       base.seed, base.q_logits)


# ----------------------------------------------------------------------------
# Multi-candidate (K-SEQ / SpecTr) inputs.
# ----------------------------------------------------------------------------
STREAM_SPECTR = 7


@dataclasses.dataclass
class SpectrBatch:
    """Host copy of one multi-candidate verify call's inputs.

    p_logits: [B, K, L+1, V] target logits; row j of candidate c is the target
              after c's first j tokens (equal prefixes give identical rows)
    q_logits: [B, K, L, V] draft logits, same layout
    cand:     [B, K, L] int32 candidate tokens (K independent drafter samples)
    u:        [B, L+1, K+1] float32 uniforms
    temperature, top_k, top_p: [B]
    """
    name: str
    p_logits: np.ndarray
    q_logits: np.ndarray
    cand: np.ndarray
    u: np.ndarray
    temperature: np.ndarray
    top_k: np.ndarray
    top_p: np.ndarray
    seed: int

    @property
    def B(self):
        return self.p_logits.shape[0]

    @property
    def K(self):
        return self.p_logits.shape[1]

    @property
    def L(self):
        return self.q_logits.shape[2]

    @property
    def V(self):
        return self.p_logits.shape[3]


def _prefix_rng(seed: int, b: int, prefix) -> np.random.Generator:
    h = 1469598103934665603
    for t in (b,) + tuple(int(x) for x in prefix) + (len(prefix),):
        h = ((h ^ (t & 0xFFFFFFFFFFFF)) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return np.random.Generator(np.random.Philox(key=[seed, STREAM_SPECTR], counter=[0, h, 0, 0]))


def make_spectr_batch(B: int, K: int, L: int, V: int, dtype: str = "bf16", seed: int = BASE_SEED + 10,
                      scale: float = 3.0, slope: float = 1.1, sigma: float = 0.5, temperature=0.8, top_k=0,
                      top_p=1.0) -> SpectrBatch:
    """K candidate sequences per sequence, each drawn token by token from the
    drafter's processed distribution after its own prefix (Gumbel-max over the
    drafter's candidate set); target and draft rows are functions of the
    prefix, so candidates with a common prefix share them."""
    dt = np.uint16 if dtype == "bf16" else np.float32
    P = np.empty((B, K, L + 1, V), dtype=dt)
    Q = np.empty((B, K, L, V), dtype=dt)
    cand = np.zeros((B, K, L), dtype=np.int32)
    T = np.broadcast_to(np.asarray(temperature, np.float32), (B,)).copy()
    kk = np.broadcast_to(np.asarray(top_k, np.int32), (B,)).copy()
    tp = np.broadcast_to(np.asarray(top_p, np.float32), (B,)).copy()
    for b in range(B):
        perm = _rng(seed, STREAM_PERM, b).permutation(V)
        zipf = (slope * np.log1p(perm.astype(np.float64))).astype(np.float32)
        cache = {}

        def rows(prefix):
            key = tuple(prefix)
            if key not in cache:
                g = _prefix_rng(seed, b, key)
                zp = np.float32(scale) * g.standard_normal(V, dtype=np.float32) - zipf
                zq = zp + np.float32(sigma) * g.standard_normal(V, dtype=np.float32)
                if dtype == "bf16":
                    zp, zq = f32_to_bf16_bits(zp), f32_to_bf16_bits(zq)
                cache[key] = (zp, zq)
            return cache[key]
        drng = _rng(seed, STREAM_DRAFT_SAMPLE, b)
        for c in range(K):
            for j in range(L + 1):
                zp, zq = rows(cand[b, c, :j])
                P[b, c, j] = zp
                if j < L:
                    Q[b, c, j] = zq
                    zqv = bf16_bits_to_f32(zq).astype(np.float64) if dtype == "bf16" else zq.astype(np.float64)
                    cand[b, c, j] = _drafter_sample(zqv, float(T[b]), int(kk[b]), float(tp[b]), drng)
    u = np.random.default_rng([seed, STREAM_UNIFORM]).random((B, L + 1, K + 1)).astype(np.float32)
    return SpectrBatch(f"spectr-B{B}-K{K}-L{L}-V{V}-{dtype}", P, Q, cand, u, T, kk, tp, seed)

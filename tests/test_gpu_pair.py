"""Dense rows (temperature > 0, no top-k up to 512) through every launch shape
of the pair kernel, against the oracle: rows held in LDS by 64-, 256- and
1024-thread workgroups, rows streamed from global memory, vector and scalar
element paths, bf16 and fp32, with unfiltered, large-top-k and nucleus rows,
and the nucleus corner cases (tie groups at the cut, a crossing bin too
large to gather, point masses)."""
import numpy as np
import pytest

from speculative_sampling_verification_verify_amd import synth
from gpu_util import compare, log, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _bf(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def dense_batch(V, dtype, B=6, G=3, seed=0, T=None, k=None, tp=None, zp=None, zq=None):
    """Zipf-shaped target logits (scale 3, slope 1.1 over a seeded
    permutation), draft logits = target + noise, drafts by Gumbel-max from
    the draft logits at the row temperature, Philox uniforms."""
    rng = np.random.default_rng(1000 + seed)
    if zp is None:
        rank = np.stack([rng.permutation(V) for _ in range(B)])[:, None, :]
        zp = (3.0 * rng.normal(size=(B, G + 1, V)) - 1.1 * np.log1p(rank)).astype(np.float32)
    if zq is None:
        zq = (zp[:, :G] + 0.7 * rng.normal(size=(B, G, V))).astype(np.float32)
    T = np.full(B, 1.0, np.float32) if T is None else np.asarray(T, np.float32)
    k = np.zeros(B, np.int32) if k is None else np.asarray(k, np.int32)
    tp = np.ones(B, np.float32) if tp is None else np.asarray(tp, np.float32)
    gum = -np.log(-np.log(rng.random(size=zq.shape)))
    draft = np.argmax(zq / np.maximum(T, 1e-3)[:, None, None] + gum, axis=2).astype(np.int32)
    cast = _bf if dtype == "bf16" else (lambda x: np.asarray(x, np.float32))
    w = synth.make_batch(0, B=1, V=8).workload
    return synth.Batch(w, cast(zp), cast(zq), draft, synth.uniforms(seed, B, G), np.full(B, G, np.int32),
                       T, k, tp, seed)


# (dtype, V): one case per launch shape.
SHAPES = [
    ("fp32", 1000),      # 4000-byte rows: 64-thread workgroup, vector loads
    ("fp32", 1001),      # 64 threads, scalar elements
    ("bf16", 2048),      # 64 threads, exactly 4 KB
    ("bf16", 6000),      # 256 threads
    ("bf16", 32768),     # 1024 threads, exactly 64 KB in LDS
    ("bf16", 32769),     # streamed, scalar elements
    ("fp32", 20000),     # streamed, vector, fp32 keys
    ("bf16", 96000),     # streamed, vector
]


@pytest.mark.parametrize("dtype,V", SHAPES)
def test_dense_launch_shapes(dtype, V):
    B = 8
    T = np.array([1.0, 0.6, 1.3, 0.8, 1.0, 0.7, 1.1, 2.0], np.float32)
    k = np.array([0, 0, 0, 600, 600, 0, V + 3, 0], np.int32)
    k = np.where(k >= V, V + 3, k).astype(np.int32)
    tp = np.array([1.0, 0.9, 0.9, 1.0, 0.85, 0.5, 0.95, 0.99], np.float32)
    bt = dense_batch(V, dtype, B=B, G=3, seed=V % 97, T=T, k=k, tp=tp)
    log(f"[pair] shape {dtype} V={V}")
    check = compare(bt, run_gpu(bt), run_oracle(bt), f"pair-{dtype}-V{V}")
    log(f"[pair] shape {dtype} V={V}: ok {check}")


@pytest.mark.parametrize("V", [5000, 70000])
def test_point_mass_rows_and_zero_residual(V):
    # top_p <= 0 keeps only the maximum (and its ties); where p and q share
    # it, the residual is empty and a rejected draft is replaced from p.
    B, G = 6, 4
    rng = np.random.default_rng(9)
    zp = rng.normal(size=(B, G + 1, V)).astype(np.float32)
    zq = zp[:, :G].copy()
    zq[1] += 0.3 * rng.normal(size=(G, V)).astype(np.float32)   # a different maximum on some positions
    bt = dense_batch(V, "bf16", B=B, G=G, seed=4, zp=zp, zq=zq, T=np.full(B, 0.9),
                     tp=np.array([0.0, 0.0, -1.0, 0.0, 1.0, 0.0], np.float32))
    d = bt.draft.copy()
    d[::2, 1] = (np.argmax(zq[::2, 1], axis=1) + 1) % V     # drafts off the maximum: q(x) = 0 -> rejected
    bt = synth.Batch(bt.workload, bt.p_logits, bt.q_logits, d, bt.u, bt.gamma_len, bt.temperature, bt.top_k,
                     bt.top_p, bt.seed)
    compare(bt, run_gpu(bt), run_oracle(bt), f"point-mass-V{V}")


@pytest.mark.parametrize("dtype,V", [("bf16", 40000), ("bf16", 8000), ("fp32", 30000)])
def test_nucleus_cut_inside_tie_group(dtype, V):
    # 3000 equal logits hold most of the mass; the cut falls inside them, so
    # the whole tie group is kept.
    B, G = 4, 2
    rng = np.random.default_rng(21)
    zp = (rng.normal(size=(B, G + 1, V)) - 4).astype(np.float32)
    zp[:, :, 100:3100] = 2.0
    zq = (zp[:, :G] + 0.5 * rng.normal(size=(B, G, V))).astype(np.float32)
    bt = dense_batch(V, dtype, B=B, G=G, seed=8, zp=zp, zq=zq, T=np.full(B, 1.0),
                     tp=np.array([0.5, 0.9, 0.2, 0.99], np.float32))
    compare(bt, run_gpu(bt), run_oracle(bt), f"tie-group-{dtype}-V{V}")


def test_nucleus_crossing_bin_too_large_to_gather():
    # fp32 logits packed into a band far narrower than one value bin: more
    # than 2048 distinct keys share the crossing bin, so the exact cut is
    # found by radix passes over the row.
    B, G, V = 3, 2, 30000
    rng = np.random.default_rng(5)
    zp = (rng.normal(size=(B, G + 1, V)) - 8).astype(np.float32)
    zp[:, :, :6000] = (4.0 + 1e-4 * rng.random(size=(B, G + 1, 6000))).astype(np.float32)
    zq = (zp[:, :G] + 0.3 * rng.normal(size=(B, G, V))).astype(np.float32)
    bt = dense_batch(V, "fp32", B=B, G=G, seed=6, zp=zp, zq=zq, T=np.full(B, 1.0),
                     tp=np.array([0.5, 0.3, 0.8], np.float32))
    compare(bt, run_gpu(bt), run_oracle(bt), "crossing-bin-overflow")


def test_rows_beyond_the_tile_table_use_multipass():
    # Odd V above 65536 elements: scalar streamed rows exceed the residual
    # tile table, so these dense rows take the finisher's multi-pass path.
    V = 70001
    bt = dense_batch(V, "bf16", B=3, G=2, seed=3, T=np.array([1.0, 0.7, 1.2]),
                     tp=np.array([1.0, 0.9, 0.8], np.float32))
    compare(bt, run_gpu(bt), run_oracle(bt), "multipass-V70001")


def test_streamed_pairs_beyond_one_round():
    """More streamed pairs (200 sequences x 4 positions = 800) than the pair
    kernel's resident workgroups (512): the leftovers are taken from the shared
    counter, bonus positions last, by whichever workgroups finish first."""
    B = 200
    rng = np.random.default_rng(5)
    T = rng.choice(np.array([0.6, 1.0, 1.3], np.float32), size=B)
    tp = rng.choice(np.array([1.0, 0.9], np.float32), size=B)
    bt = dense_batch(40000, "bf16", B=B, G=3, seed=11, T=T, tp=tp)
    compare(bt, run_gpu(bt), run_oracle(bt), "streamed-800-pairs")


# ---- the all-dense hint: no select launch, pairs taken in a fixed order --------

@pytest.mark.parametrize("cid,B,V,label", [
    (1, 8, None, "rows in LDS, 1024 threads (unfiltered bf16, V 32000)"),
    (0, 64, None, "rows in LDS, 64 threads (fp32, V 1000)"),
    (1, 4, 70000, "streamed rows (bf16, V 70000)"),
    (4, 16, 20000, "ragged drafts with argmax sequences: the promise broken"),
    (2, 4, 20000, "top-k 50 sequences only: the promise broken everywhere"),
])
def test_all_dense_hint_matches_oracle(cid, B, V, label):
    # The hint skips the select launch; the pair kernel then walks every
    # (sequence, position) itself, and sequences that are not dense after all
    # go to the finisher's multi-pass path.  Two calls in a row check that
    # the pair queue counter is left cleared.
    from speculative_sampling_verification_verify_amd import binding
    bt = synth.make_batch(cid, B=B, V=V)
    log(f"all-dense hint: {label}: B={bt.B} V={bt.V} G={bt.gamma_max}")
    dt = binding.SV_BF16 if bt.p_logits.dtype == np.uint16 else binding.SV_FP32
    ver = binding.Verifier(bt.B, bt.gamma_max, bt.V, dt, device="cuda:0", hints=binding.SV_HINT_ALL_DENSE)
    ref = run_oracle(bt)
    for call in range(2):
        compare(bt, run_gpu(bt, verifier=ver), ref, f"all-dense-{label}-call{call}")


# ---- bf16 rows counted in an LDS histogram of their values -------------------

@pytest.mark.parametrize("V", [32776, 65544, 131072])
def test_histogram_rows_sizes_and_filters(V):
    """Streamed bf16 rows from just above the LDS-held size to the largest
    the histogram variant takes (V = 131072, 16 units per thread, partial
    last tile at 32776 and 65544), with unfiltered, top-p (including 0),
    large top-k, top-k plus top-p, -inf entries and extreme temperatures."""
    B, G = 10, 3
    T = np.array([1.0, 0.6, 1.3, 0.8, 1.0, 0.7, 1e-3, 50.0, 1.1, 0.9], np.float32)
    k = np.array([0, 0, 0, 600, 5000, 0, 0, 0, 700, 0], np.int32)
    tp = np.array([1.0, 0.9, 0.0, 1.0, 0.85, 0.3, 0.95, 0.9, 1.0, 0.99], np.float32)
    rng = np.random.default_rng(V % 1009)
    rank = np.stack([rng.permutation(V) for _ in range(B)])[:, None, :]
    zp = (3.0 * rng.normal(size=(B, G + 1, V)) - 1.1 * np.log1p(rank)).astype(np.float32)
    zq = (zp[:, :G] + 0.7 * rng.normal(size=(B, G, V))).astype(np.float32)
    zp[9, :, ::7] = -np.inf                    # -inf entries carry no mass
    zq[9, :, 3::11] = -np.inf
    bt = dense_batch(V, "bf16", B=B, G=G, seed=V % 89, T=T, k=k, tp=tp, zp=zp, zq=zq)
    log(f"[pair-hist] V={V}")
    rep = compare(bt, run_gpu(bt), run_oracle(bt), f"pair-hist-V{V}")
    log(f"[pair-hist] V={V}: ok {rep}")


def test_histogram_reread_lists():
    """The units read again after the histograms are those whose largest
    target value reaches the target's nucleus: draft rows equal to the target
    rows (zero residual everywhere, so the draw sums p), a nucleus held only
    by the last, partial tile, a nucleus of most units (more list entries
    than one batch of the weights pass holds), and a large top-k whose cut
    lies below the floor of the unfiltered rows."""
    B, G, V = 4, 2, 65544
    rng = np.random.default_rng(45)
    rank = np.stack([rng.permutation(V) for _ in range(B)])[:, None, :]
    zp = (3.0 * rng.normal(size=(B, G + 1, V)) - 1.1 * np.log1p(rank)).astype(np.float32)
    zq = (zp[:, :G] + 0.7 * rng.normal(size=(B, G, V))).astype(np.float32)
    zq[0] = zp[0, :G]
    zp[1, :, V - 12:] = 40.0 + rng.normal(size=(G + 1, 12))
    zq[1, :, V - 12:] = 40.0 + rng.normal(size=(G, 12))
    zp[2] = (0.3 * rng.normal(size=(G + 1, V))).astype(np.float32)
    zq[2] = (zp[2, :G] + 0.1 * rng.normal(size=(G, V))).astype(np.float32)
    bt = dense_batch(V, "bf16", B=B, G=G, seed=15, zp=zp, zq=zq,
                     T=np.array([1.0, 0.8, 1.3, 1.0]), k=np.array([0, 0, 0, 40000]),
                     tp=np.array([0.9, 0.95, 0.97, 1.0], np.float32))
    rep = compare(bt, run_gpu(bt), run_oracle(bt), "hist-lists")
    log(f"[pair-hist] reread lists: ok {rep}")


def test_histogram_count_overflow_takes_the_multipass_path():
    """More than 65535 equal values in one row overflow its 16-bit count: the
    pair is marked for the finisher, which computes the sequence from the
    logits.  Rows of sequence 0 overflow in both, sequence 1 only in the
    draft rows, sequence 2 only in the target rows; sequence 3 is ordinary."""
    B, G, V = 4, 2, 131072
    rng = np.random.default_rng(44)
    zp = (2.0 * rng.normal(size=(B, G + 1, V))).astype(np.float32)
    zq = (zp[:, :G] + 0.5 * rng.normal(size=(B, G, V))).astype(np.float32)
    zp[0, :, :70000] = 0.25
    zq[0, :, :70000] = 0.25
    zq[1, :, 1000:67000] = -1.0
    zp[2, :, 500:66500] = 0.5
    bt = dense_batch(V, "bf16", B=B, G=G, seed=12, zp=zp, zq=zq, T=np.array([1.0, 0.8, 1.2, 1.0]),
                     tp=np.array([1.0, 0.9, 0.8, 0.9], np.float32))
    rep = compare(bt, run_gpu(bt), run_oracle(bt), "hist-overflow")
    log(f"[pair-hist] overflow: ok {rep}")


def test_histogram_row_with_nan_is_invalid_and_others_exact():
    B, G, V = 4, 2, 50000
    bt = dense_batch(V, "bf16", B=B, G=G, seed=13, T=np.array([1.0, 0.8, 1.2, 1.0]),
                     tp=np.array([1.0, 0.9, 0.8, 0.9], np.float32))
    P, Q = bt.p_logits.copy(), bt.q_logits.copy()
    Q[1, 1, 777] = 0x7FC1                     # NaN in a draft row
    P[2, 2, 5] = 0x7F80                       # +inf in the bonus row
    bt = synth.Batch(bt.workload, P, Q, bt.draft, bt.u, bt.gamma_len, bt.temperature, bt.top_k, bt.top_p, bt.seed)
    g = run_gpu(bt)
    ref = run_oracle(bt)
    assert ref.n[1] == -1 and ref.n[2] == -1
    compare(bt, g, ref, "hist-invalid")


# ---- calls with dense and streamed sequences on the histogram variant --------

def _mixed_logits(B, G, V, seed):
    rng = np.random.default_rng(seed)
    rank = np.stack([rng.permutation(V) for _ in range(B)])[:, None, :]
    zp = (3.0 * rng.normal(size=(B, G + 1, V)) - 1.1 * np.log1p(rank)).astype(np.float32)
    zq = (zp[:, :G] + 0.7 * rng.normal(size=(B, G, V))).astype(np.float32)
    return zp, zq


def test_mixed_call_select_units_beside_histogram_pairs():
    """Dense top-p sequences beside argmax and top-k sequences at V = 65544,
    no hint: the select units run in the histogram pairs' launch.  The last
    top-k sequence has more ties at its k-th value than the select's buffer
    holds (demoted to the finisher's multi-pass path).  Two calls in a row on
    one verifier check the counters the finisher clears."""
    from speculative_sampling_verification_verify_amd import binding
    B, G, V = 8, 3, 65544
    zp, zq = _mixed_logits(B, G, V, 61)
    zp[7, :, :20000] = 3.0
    bt = dense_batch(V, "bf16", B=B, G=G, seed=61, zp=zp, zq=zq,
                     T=np.array([1.0, 0.0, 0.8, 1.0, 0.6, 1.3, 0.0, 1.0]),
                     k=np.array([0, 0, 0, 64, 0, 0, 0, 50]),
                     tp=np.array([0.9, 1.0, 0.95, 1.0, 0.8, 0.9, 1.0, 1.0], np.float32))
    ver = binding.Verifier(B, G, V, binding.SV_BF16, device="cuda:0")
    ref = run_oracle(bt)
    for call in range(2):
        rep = compare(bt, run_gpu(bt, verifier=ver), ref, f"mixed-call{call}")
    log(f"[pair-hist] mixed call: ok {rep}")


def test_mixed_kernel_without_dense_sequences():
    """Only argmax and top-k sequences at a histogram-variant V, no hint: the
    listing finds no dense pair, and the select units are taken one per
    wavefront, spread over the CUs, instead of in groups of 16."""
    from speculative_sampling_verification_verify_amd import binding
    B, G, V = 40, 4, 65544
    zp, zq = _mixed_logits(B, G, V, 62)
    T = np.where(np.arange(B) % 2 == 0, 0.0, 0.8).astype(np.float32)
    k = np.where(np.arange(B) % 4 == 1, 64, np.where(np.arange(B) % 4 == 3, 200, 0)).astype(np.int32)
    bt = dense_batch(V, "bf16", B=B, G=G, seed=62, zp=zp, zq=zq, T=T, k=k)
    ver = binding.Verifier(B, G, V, binding.SV_BF16, device="cuda:0")
    ref = run_oracle(bt)
    for call in range(2):
        rep = compare(bt, run_gpu(bt, verifier=ver), ref, f"mixed-no-dense-call{call}")
    log(f"[pair-hist] mixed kernel, no dense sequence: ok {rep}")


def test_streamed_rows_beyond_the_histogram_variant():
    # 17500 units per row: more than the histogram variant holds, so the
    # value-binned streamed variant takes these rows.
    V = 140000
    bt = dense_batch(V, "bf16", B=3, G=2, seed=14, T=np.array([1.0, 0.7, 1.2]),
                     tp=np.array([1.0, 0.9, 0.8], np.float32))
    compare(bt, run_gpu(bt), run_oracle(bt), "streamed-V140000")


# ---- dense pairs of unfiltered rows split over several workgroups -------------

def _split_verifier(bt, hints):
    from speculative_sampling_verification_verify_amd import binding
    dt = binding.SV_BF16 if bt.p_logits.dtype == np.uint16 else binding.SV_FP32
    return binding.Verifier(bt.B, bt.gamma_max, bt.V, dt, device="cuda:0", hints=hints)


@pytest.mark.parametrize("dtype,V,B,G", [
    ("bf16", 128256, 2, 3),     # 8 pairs: 31 chunks of 518 units
    ("bf16", 152064, 1, 7),     # 8 pairs: 32 chunks of 594 units
    ("bf16", 65544, 4, 3),      # 16 chunks, a ragged last chunk
    ("bf16", 40000, 3, 2),      # 9 chunks of 556 units
    ("fp32", 20000, 8, 3),      # fp32 rows of 80 KB, 9 chunks
    ("bf16", 32000, 32, 5),     # rows held in LDS: no split, the hint changes nothing
])
def test_split_pairs_match_oracle(dtype, V, B, G):
    """Unfiltered dense rows under the unfiltered hint (with and without the
    all-dense hint): per-chunk maxima and normalisers, per-chunk weights, and
    the draw from the crossing chunk, against the oracle; two calls in a row
    reuse the chunk records."""
    from speculative_sampling_verification_verify_amd import binding
    T = np.resize(np.array([1.0, 0.6, 1.3, 0.8, 2.0, 1e-3, 50.0, 0.9], np.float32), B)
    bt = dense_batch(V, dtype, B=B, G=G, seed=V % 97, T=T)
    ref = run_oracle(bt)
    for hints in (binding.SV_HINT_UNFILTERED, binding.SV_HINT_ALL_DENSE | binding.SV_HINT_UNFILTERED):
        ver = _split_verifier(bt, hints)
        for call in range(2):
            log(f"[split] {dtype} V={V} B={B} G={G} hints={hints} call {call}")
            rep = compare(bt, run_gpu(bt, verifier=ver), ref, f"split-{dtype}-V{V}-h{hints}-c{call}")
        log(f"[split] ok {rep}")


@pytest.mark.parametrize("V,dtype", [(40000, "bf16"), (1000, "fp32"), (2000, "bf16"), (520, "fp32")])
def test_split_pairs_edge_cases(V, dtype):
    """Under the unfiltered hint: equal draft and target rows (zero residual:
    the draw falls back to p), -inf entries, a NaN row (invalid), short
    drafts (padding positions), and sequences that break the promise (top-p,
    top-k above 512, top-k 20, argmax), which take the finisher's paths.
    V = 40000 runs the split kernels; the short rows run the 64-thread pair
    kernel with its rows in registers and no row LDS (top-k 600 is a filter
    only where V > 600)."""
    from speculative_sampling_verification_verify_amd import binding
    B, G = 8, 3
    rng = np.random.default_rng(46)
    rank = np.stack([rng.permutation(V) for _ in range(B)])[:, None, :]
    zp = (3.0 * rng.normal(size=(B, G + 1, V)) - 1.1 * np.log1p(rank)).astype(np.float32)
    zq = (zp[:, :G] + 0.7 * rng.normal(size=(B, G, V))).astype(np.float32)
    zq[0] = zp[0, :G]                          # zero residual
    zp[1, :, ::5] = -np.inf                    # -inf entries
    zq[1, :, 2::7] = -np.inf
    T = np.array([1.0, 0.9, 1.1, 0.8, 1.0, 0.7, 1.2, 0.0], np.float32)
    k = np.array([0, 0, 0, 0, 600, 20, 0, 0], np.int32)
    tp = np.array([1.0, 1.0, 1.0, 0.9, 1.0, 1.0, 1.0, 1.0], np.float32)
    bt = dense_batch(V, dtype, B=B, G=G, seed=47, T=T, k=k, tp=tp, zp=zp, zq=zq)
    gl = np.array([3, 3, 1, 3, 2, 3, 3, 3], np.int32)
    P = bt.p_logits.copy()
    P[2, 1, 99] = 0x7FC1 if dtype == "bf16" else np.nan   # NaN in a target row of sequence 2 (position 1 is used)
    bt = synth.Batch(bt.workload, P, bt.q_logits, bt.draft, bt.u, gl, bt.temperature, bt.top_k, bt.top_p,
                     bt.seed)
    ref = run_oracle(bt)
    assert ref.n[2] == -1
    for hints in (binding.SV_HINT_UNFILTERED, binding.SV_HINT_ALL_DENSE | binding.SV_HINT_UNFILTERED):
        ver = _split_verifier(bt, hints)
        for call in range(2):
            log(f"[split] edge cases V={V} {dtype} hints={hints} call {call}")
            compare(bt, run_gpu(bt, verifier=ver), ref, f"split-edges-V{V}-h{hints}-c{call}")

"""Benchmark of the batched speculative-sampling verify step on one MI355X.

One step = one spec_verify call over one batch of synthetic inputs that are
already resident in HBM.  The default workload is the headline one:
B = 256 sequences, V = 152064, gamma = 7, bf16 logits, temperature 0.7,
top-k 64 (1.17 GB of logits per call).

Prints one JSON line with verify-rows/s (a row is one sequence), the
achieved HBM bandwidth of the kernel that reads most of the logits (the
streaming select for top-k and argmax sequences, the pair kernel for dense
ones) against the 8 TB/s peak, timed with HIP events recorded around that
kernel on the call's stream, and the CPU oracle timed on a bounded sample
on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from speculative_sampling_verification_verify_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "spec-verify rows/sec + achieved HBM GB/s vs peak at B=256,V=152064,γ=7"
# rocprofv3 HBM-counter summaries, by (kernel, workload name).
PMC_SUMMARIES = {
    ("select_kernel", "B256-V152064-g7-T0.7-topk64"): "select_kernel_B256_V152064_g7_pmc.txt",
    ("mixed_hist_kernel", "B128-V128256-mixed-g1..8-topp0.9"): "mixed_hist_kernel_B128_V128256_mixed_topp_pmc.txt",
    ("select_kernel", "B64-V128256-g4-topk50"): "select_kernel_B64_V128256_g4_topk50_pmc.txt",
    ("pair_kernel", "B32-V32000-g5-T0.8"): "pair_kernel_B32_V32000_g5_pmc.txt",
    ("pair_kernel", "tiny-fp32-V1000-g4"): "pair_kernel_B1000_V1000_g4_fp32_pmc.txt",
    ("gumbel_mixed_kernel", "B128-V128256-mixed-g1..8-topp0.9-gumbel"): "gumbel_mixed_kernel_B128_V128256_mixed_topp_pmc.txt",
}
CSRC = os.path.join(ROOT, "speculative_sampling_verification_verify_amd", "csrc")
ROTATE_BYTES = 768 << 20     # rotate input copies until this many bytes are in flight
CPU_REPEAT = 16              # the CPU baseline's sample may pass over a batch this many times
EVENT_EVERY = 10             # timed calls per call that carries the kernel's HIP events


# The sources that determine a kernel's code and launch: its own header, the
# shared device headers and the host file.  A counter summary stays valid
# while these are unchanged.
KERNEL_SOURCES = {
    "select_kernel": ("spec_verify.hip", "sv_common.h", "sv_device.h", "sv_wave.h"),
    "pair_kernel": ("spec_verify.hip", "sv_common.h", "sv_device.h", "sv_pair.h"),
    "pair_hist_kernel": ("spec_verify.hip", "sv_common.h", "sv_device.h", "sv_pair.h", "sv_phist.h"),
    "mixed_hist_kernel": ("spec_verify.hip", "sv_common.h", "sv_device.h", "sv_pair.h", "sv_phist.h", "sv_wave.h"),
    "gumbel_hist_kernel": ("spec_verify.hip", "sv_common.h", "sv_device.h", "sv_pair.h", "sv_phist.h", "sv_finish.h",
                           "sv_gumbel.h"),
    "gumbel_mixed_kernel": ("spec_verify.hip", "sv_common.h", "sv_device.h", "sv_pair.h", "sv_phist.h", "sv_finish.h",
                            "sv_gumbel.h", "sv_wave.h"),
}


def _code_text(text: str) -> str:
    """The source with comments removed and whitespace runs collapsed, so that
    an edit of comments or layout does not mark a profile stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(kernel: str | None = None) -> str:
    """Hash of the code (not the comments) of the sources a kernel is built
    from; profiles/ records it beside the counters taken on that code."""
    names = KERNEL_SOURCES.get(kernel) or sorted(os.listdir(CSRC))
    h = hashlib.sha256()
    for name in sorted(names):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_text(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str, workload: str):
    """Per-launch HBM bytes (read + write) of `kernel` on `workload` from the
    committed rocprofv3 counter summary, if one exists and was taken on the
    current kernel sources; else None."""
    name = PMC_SUMMARIES.get((kernel, workload))
    path = os.path.join(ROOT, "profiles", name) if name else None
    if not path or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash(kernel):
        return None
    try:
        return float(kv["hbm_read_bytes_per_launch"]) + float(kv["hbm_write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> int:
    try:
        return min(16, len(os.sched_getaffinity(0)))
    except AttributeError:
        return min(16, os.cpu_count() or 1)


def oracle_reference(bt, cores: int):
    """The oracle's outputs for every sequence of the batch, computed before
    the GPU is touched (worker processes are forked), to check the timed
    calls' outputs afterwards."""
    import oracle
    return oracle.verify_batch(bt.p_logits, bt.q_logits, bt.draft, bt.u, bt.temperature, bt.top_k, bt.top_p,
                               bt.gamma_len, processes=cores)


def output_check(bt, ref, tokens, n, alpha, pq, tol=1e-5):
    """The parity rules on one call's outputs: n and the tokens identical
    wherever the oracle's decision margin is at least tol; alpha and
    (p(x), q(x)) within tol at every position whose rows have no nucleus
    boundary within tol.  Returns the counts for the JSON line."""
    near = ref.margin < tol
    same = (n == ref.n) & (tokens == ref.tokens).all(axis=1)
    G = bt.gamma_max
    used = (np.arange(G)[None, :] < bt.gamma_len[:, None]) & (ref.n >= 0)[:, None]
    cmp = used & (ref.topp_pos >= tol)
    ea = np.abs(alpha - ref.alpha)[cmp]
    ep = np.abs(pq - ref.pq)[cmp]
    max_a = float(ea.max()) if ea.size else 0.0
    max_p = float(ep.max()) if ep.size else 0.0
    ok = bool((same | near).all() and max_a <= tol and max_p <= tol)
    return {"sequences_checked": int(len(n)), "near": int(near.sum()), "near_differ": int((near & ~same).sum()),
            "differ_outside_margin": int((~same & ~near).sum()), "positions": int(used.sum()),
            "positions_compared": int(cmp.sum()), "max_alpha_err": max_a, "max_pq_err": max_p, "ok": ok}


def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "speculative_sampling_verification_verify_amd", "libsvprobe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; build it with __graft_entry__.build()")
    L = ctypes.CDLL(path)
    vp, sz, i, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32
    L.sv_read_probe.argtypes = [vp, sz, vp, sz, vp, i, i, u32, vp]
    L.sv_read_probe.restype = i
    return L


def read_ceiling(A, B, launches: int = 10):
    """Streaming-read ceiling on the call's own logit buffers: a plain
    read of A and B (each once per launch) in a few launch shapes, timed with
    events on the current stream; the best shape's GB/s."""
    import torch
    L = _probe_lib()
    nbytes = A.numel() * A.element_size() + B.numel() * B.element_size()
    out = torch.zeros(16384, dtype=torch.int32, device=A.device)
    stream = torch.cuda.current_stream().cuda_stream or None
    best = None
    for grid in (1024, 2048, 4096, 8192, 16384):
        for unroll in (8, 16):
            def launch():
                rc = L.sv_read_probe(A.data_ptr(), A.numel() * A.element_size(), B.data_ptr(),
                                     B.numel() * B.element_size(), out.data_ptr(), grid, unroll, 0x9E3779B9, stream)
                if rc != 0:
                    raise RuntimeError(f"sv_read_probe failed with {rc}")
            launch()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
            for a, b in evs:
                a.record()
                launch()
                b.record()
            torch.cuda.synchronize()
            us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
            gbs = nbytes / (us * 1e-6) / 1e9
            if best is None or gbs > best["achieved"]:
                best = {"achieved": gbs, "unit": "GB/s", "frac_of_peak": gbs / HBM_PEAK_GBS, "bytes": nbytes,
                        "avg_us": us, "grid": grid, "unroll": unroll}
    return best


def kernel_bytes(bt):
    """Logit bytes read by the streaming select (argmax and top-k <= 512
    sequences) and by the pair kernel (every other sequence with T > 0)."""
    g = bt.gamma_len.astype(np.int64)
    rows = (2 * g + 1) * bt.V * bt.p_logits.itemsize
    T, k = bt.temperature, bt.top_k
    sel = (T == 0) | ((T > 0) & (k > 0) & (k < bt.V) & (k <= 512))
    dense = (T > 0) & ~sel
    return int(rows[sel].sum()), int(rows[dense].sum())


def timed_calls(step, kern: int, n: int, every: int = EVENT_EVERY):
    """n calls step(0..n-1) between two device synchronisations, with HIP
    events around kernel `kern` (SV_KERNEL_*, on the call's stream) on every
    `every`-th call.  An event recorded between two kernels of a call delays
    the second by about 5 us, so sampling keeps the call rate a measure of
    the calls.  Returns (wall seconds, per-launch ms of the sampled calls)."""
    import torch
    from speculative_sampling_verification_verify_amd import binding
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(0, n, every)]
    for a, b in evs:     # materialise the underlying hipEvent_t handles
        a.record()
        b.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(n):
        if j % every == 0:
            a, b = evs[j // every]
            binding.spec_verify_set_stage_events(a, b, kern)
        step(j)
        if j % every == 0:
            binding.spec_verify_set_stage_events(None, None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, np.array([a.elapsed_time(b) for a, b in evs])


def pair_kernel_name(bt, mixed: bool = False) -> str:
    """The kernel of the pair stage for this batch's rows: bf16 rows longer
    than the 64 KB held in LDS, of whole 16-byte units and at most 16384 of
    them, are counted into a histogram (pair_hist_kernel; mixed_hist_kernel,
    which also streams the select's rows, when the call has both kinds of
    sequence); other dense rows take pair_kernel (the library makes the same
    choice)."""
    V = bt.V
    if bt.p_logits.dtype == np.uint16 and V * 2 > 65536 and V % 8 == 0 and V // 8 <= 16384:
        return "mixed_hist_kernel" if mixed else "pair_hist_kernel"
    return "pair_kernel"


def cpu_baseline(bt, seconds_target: float, cores: int):
    """Time the CPU oracle (as it stands) on whole sequences of the same
    workload, in worker processes (fork) on `cores` host cores."""
    import oracle
    # Estimate the per-sequence cost on a few sequences, then size the sample.
    t0 = time.perf_counter()
    oracle.verify_batch(bt.p_logits, bt.q_logits, bt.draft, bt.u, bt.temperature, bt.top_k, bt.top_p,
                        bt.gamma_len, rows=range(2), processes=1)
    per_seq = max((time.perf_counter() - t0) / 2, 1e-4)
    # The sample cycles through the batch's sequences until it holds about
    # seconds_target of CPU work (at most CPU_REPEAT passes over the batch).
    n = int(min(CPU_REPEAT * bt.B, max(cores, seconds_target / per_seq)))
    rows = [i % bt.B for i in range(n)]
    t0 = time.perf_counter()
    oracle.verify_batch(bt.p_logits, bt.q_logits, bt.draft, bt.u, bt.temperature, bt.top_k, bt.top_p,
                        bt.gamma_len, rows=rows, processes=cores)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "rows/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{n} sequences cycling through the workload's {bt.B} (float64 numpy oracle, {cores} worker processes, "
                      f"{dt:.2f} s wall, about {per_seq * n:.1f} s of CPU work)"}


def _gumbel_rows(args):
    import oracle
    (p, noise, draft, T, k, tp, gl), rows = args
    r = oracle.gumbel_verify_batch(p, noise, draft, T, k, tp, gl, rows=rows)
    return len(rows), int((r.n >= 0).sum())


def cpu_baseline_gumbel(gb, seconds_target: float, cores: int):
    """Time the CPU oracle of the shared-noise verify on whole sequences of
    the same workload, in worker processes (fork)."""
    import multiprocessing as mp
    import oracle
    data = (gb.p_logits, gb.noise, gb.draft, gb.temperature, gb.top_k, gb.top_p, gb.gamma_len)
    t0 = time.perf_counter()
    oracle.gumbel_verify_batch(*data, rows=[0])
    per_seq = max(time.perf_counter() - t0, 1e-4)
    n = int(min(CPU_REPEAT * gb.B, max(cores, seconds_target / per_seq)))
    chunks = [[j % gb.B for j in range(i, n, cores)] for i in range(cores) if i < n]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(len(chunks)) as pool:
        pool.map(_gumbel_rows, [(data, c) for c in chunks])
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "rows/s", "cores": len(chunks), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{n} sequences cycling through the workload's {gb.B} (shared-noise oracle, {len(chunks)} worker processes, "
                      f"{dt:.2f} s wall, about {per_seq * n:.1f} s of CPU work)"}


def main_gumbel(args):
    """The shared-noise verify on workload `args.workload`'s shapes."""
    t_gen = time.perf_counter()
    gb = synth.make_gumbel_batch(args.workload)
    t_gen = time.perf_counter() - t_gen
    es = gb.p_logits.itemsize
    g1 = gb.gamma_len.astype(np.int64) + 1
    T, k = gb.temperature, gb.top_k
    listed = (T == 0) | ((T > 0) & (k > 0) & (k < gb.V) & (k <= 512))
    # The streaming select reads the listed sequences' logits once (noise only
    # at their few kept ids); the dense kernel reads logits and noise.
    sel_bytes = int((g1[listed] * gb.V * es).sum())
    dense_bytes = int((g1[~listed] * gb.V * (es + 4)).sum())
    kbytes = max(sel_bytes, dense_bytes)
    cpu = None
    if not args.no_cpu:
        try:
            cores = min(16, len(os.sched_getaffinity(0)))
        except AttributeError:
            cores = min(16, os.cpu_count() or 1)
        cpu = cpu_baseline_gumbel(gb, args.cpu_seconds, cores)
    import torch
    from speculative_sampling_verification_verify_amd import binding
    dev = torch.device("cuda:0")
    if gb.p_logits.dtype == np.uint16:
        P = torch.from_numpy(gb.p_logits.view(np.int16)).to(dev).view(torch.bfloat16)
        dtype_name = "bf16"
    else:
        P = torch.from_numpy(gb.p_logits).to(dev)
        dtype_name = "fp32"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    N = t(gb.noise)
    draft, temp, topk, topp, gl = t(gb.draft), t(gb.temperature), t(gb.top_k), t(gb.top_p), t(gb.gamma_len)
    # The call says what it knows of its sequences (host-side facts): with no
    # argmax or small-top-k sequence the select and list launches are skipped;
    # with only such sequences the list kernel finishes the call.
    ghints = binding.SV_HINT_ALL_DENSE if sel_bytes == 0 else (binding.SV_HINT_NO_DENSE if dense_bytes == 0 else 0)
    ver = binding.GumbelVerifier(gb.B, gb.gamma_max, gb.V,
                                 binding.SV_BF16 if dtype_name == "bf16" else binding.SV_FP32, device=dev, hints=ghints)
    nsets = int(min(32, max(1, -(-ROTATE_BYTES // max(kbytes, 1)))))
    sets = [(P, N)] + [(P.clone(), N.clone()) for _ in range(nsets - 1)]
    torch.cuda.synchronize()

    def step(j):
        Pj, Nj = sets[j % nsets]
        ver(Pj, Nj, draft, temp, topk, topp, gl)

    for j in range(args.warmup):
        step(j)
    torch.cuda.synchronize()
    K = args.steps
    # The dense stage is the histogram kernel for filtered bf16 rows of 32K-131K
    # values (16-byte aligned), else the per-(sequence, position) kernel.  With
    # both kinds of sequence on the histogram rows (no hint), one launch,
    # gumbel_mixed_kernel, streams the select's rows and takes the histogram
    # rows: it reads both kinds of bytes.
    hist_rows = dtype_name == "bf16" and 32768 < gb.V <= 131072 and gb.V % 8 == 0
    gmixed = hist_rows and ghints == 0
    kern = binding.SV_KERNEL_SELECT if sel_bytes >= dense_bytes and not gmixed else binding.SV_KERNEL_GUMBEL
    kname = ("select_kernel" if kern == binding.SV_KERNEL_SELECT
             else ("gumbel_mixed_kernel" if gmixed else ("gumbel_hist_kernel" if hist_rows else "gumbel_kernel")))
    if gmixed:
        kbytes = sel_bytes + dense_bytes
    wall, k_ms = timed_calls(step, kern, K)
    ms_per_step = wall * 1e3 / K
    n_acc = ver.n_accepted.cpu().numpy()
    k_avg = float(k_ms.mean())
    achieved = kbytes / (k_avg * 1e-3) / 1e9
    w = gb.workload
    out = {
        "metric": "shared-noise spec-verify rows/sec + achieved HBM GB/s vs peak",
        "value": gb.B / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic",
        "config": {"workload": w.name, "B": gb.B, "V": gb.V, "gamma": gb.gamma_max,
                   "temperature": float(w.temperature), "top_k": int(w.top_k), "top_p": float(w.top_p),
                   "parallelism": "single-gpu", "hints": {binding.SV_HINT_ALL_DENSE: "all-dense",
                                                             binding.SV_HINT_NO_DENSE: "no-dense"}.get(ghints, "none")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_from_profile(kname, w.name),
                     "kernel": kname, "kernel_bytes_per_launch": kbytes, "kernel_avg_us": k_avg * 1e3,
                     "kernel_p10_us": float(np.percentile(k_ms, 10) * 1e3),
                     "kernel_p90_us": float(np.percentile(k_ms, 90) * 1e3),
                     "kernel_timed_launches": int(len(k_ms)), "event_every": EVENT_EVERY},
        "cpu_baseline": cpu,
        "extra": {"mean_tokens_per_round": float((n_acc[n_acc >= 0] + 1).mean()),
                  "input_sets_rotated": nsets, "input_generation_s": t_gen},
    }
    print(json.dumps(out))


def _spectr_rows(args):
    import oracle
    (p, q, cand, u, T, k, tp), rows = args
    oracle.kseq.spectr_batch(p, q, cand, u, T, k, tp, rows=rows)
    return len(rows)


def main_spectr(args):
    """Multi-candidate verify (K-SEQ / SpecTr) at K = 8 candidates of L = 8
    tokens (the configuration the SpecTr page reports), B = 32 sequences,
    V = 32000 bf16, T = 0.8."""
    import multiprocessing as mp
    t_gen = time.perf_counter()
    sb = synth.make_spectr_batch(32, 8, 8, 32000, dtype="bf16", temperature=0.8)
    t_gen = time.perf_counter() - t_gen
    es = sb.p_logits.itemsize
    # Algorithmic bytes of the first node launch, the timed kernel: the target
    # and draft rows (the target row alone after depth L) of every node whose
    # class holds two or more candidates, each read once.  The single-
    # candidate nodes the walk reaches are computed by a second, small launch.
    nodes = 0
    for b in range(sb.B):
        for j in range(sb.L + 1):
            sizes = {}
            for c in range(sb.K):
                key = tuple(sb.cand[b, c, :j])
                sizes[key] = sizes.get(key, 0) + 1
            nodes += sum(1 for v in sizes.values() if v >= 2) * (2 if j < sb.L else 1)
    kbytes = nodes * sb.V * es
    cpu = None
    if not args.no_cpu:
        import oracle
        try:
            cores = min(16, len(os.sched_getaffinity(0)))
        except AttributeError:
            cores = min(16, os.cpu_count() or 1)
        data = (sb.p_logits, sb.q_logits, sb.cand, sb.u, sb.temperature, sb.top_k, sb.top_p)
        t0 = time.perf_counter()
        oracle.kseq.spectr_batch(*data, rows=[0])
        per_seq = max(time.perf_counter() - t0, 1e-4)
        n = int(min(CPU_REPEAT * sb.B, max(cores, args.cpu_seconds / per_seq)))
        chunks = [[j % sb.B for j in range(i, n, cores)] for i in range(cores) if i < n]
        t0 = time.perf_counter()
        with mp.get_context("fork").Pool(len(chunks)) as pool:
            pool.map(_spectr_rows, [(data, c) for c in chunks])
        dt = time.perf_counter() - t0
        cpu = {"value": n / dt, "unit": "rows/s", "cores": len(chunks), "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"{n} sequences cycling through the workload's {sb.B} (K-SEQ / SpecTr oracle, {len(chunks)} worker "
                         f"processes, {dt:.2f} s wall, about {per_seq * n:.1f} s of CPU work)"}
    import torch
    from speculative_sampling_verification_verify_amd import binding
    dev = torch.device("cuda:0")
    P = torch.from_numpy(sb.p_logits.view(np.int16)).to(dev).view(torch.bfloat16)
    Q = torch.from_numpy(sb.q_logits.view(np.int16)).to(dev).view(torch.bfloat16)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    cand, u, temp, topk, topp = t(sb.cand), t(sb.u), t(sb.temperature), t(sb.top_k), t(sb.top_p)
    ver = binding.SpectrVerifier(sb.B, sb.K, sb.L, device=dev)
    logit_bytes = sb.p_logits.nbytes + sb.q_logits.nbytes
    nsets = int(min(32, max(1, -(-ROTATE_BYTES // logit_bytes))))
    sets = [(P, Q)] + [(P.clone(), Q.clone()) for _ in range(nsets - 1)]
    torch.cuda.synchronize()

    def step(j):
        Pj, Qj = sets[j % nsets]
        ver(Pj, Qj, cand, u, temp, topk, topp)

    for j in range(args.warmup):
        step(j)
    torch.cuda.synchronize()
    K = args.steps
    wall, k_ms = timed_calls(step, binding.SV_KERNEL_KSEQ, K)
    ms_per_step = wall * 1e3 / K
    n_out = ver.n.cpu().numpy()
    k_avg = float(k_ms.mean())
    achieved = kbytes / (k_avg * 1e-3) / 1e9
    out = {
        "metric": "multi-candidate (K-SEQ / SpecTr) verify rows/sec + achieved HBM GB/s vs peak",
        "value": sb.B / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": sb.name, "B": sb.B, "K": sb.K, "L": sb.L, "V": sb.V, "temperature": 0.8,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_from_profile("kseq_node_kernel", sb.name),
                     "kernel": "kseq_node_kernel", "kernel_bytes_per_launch": kbytes, "kernel_avg_us": k_avg * 1e3,
                     "kernel_p10_us": float(np.percentile(k_ms, 10) * 1e3),
                     "kernel_p90_us": float(np.percentile(k_ms, 90) * 1e3),
                     "kernel_timed_launches": int(len(k_ms)), "event_every": EVENT_EVERY},
        "cpu_baseline": cpu,
        "extra": {"mean_tokens_per_round": float((n_out[n_out >= 0] + 1).mean()), "shared_node_rows": nodes,
                  "input_sets_rotated": nsets, "input_generation_s": t_gen},
    }
    print(json.dumps(out))


def main_small_batch(args):
    """Per-call latency of small batches (B = 1, 4, 8; gamma 4, V = 128256;
    B = 1, gamma 7, V = 152064) of unfiltered bf16 rows at T = 1, all dense:
    one workgroup per (sequence, position) pair against the pairs split over
    several workgroups (SV_HINT_UNFILTERED).  Synthetic logits: target
    N(0, 3^2), draft = target + N(0, 0.7^2), seeded; random drafts and
    uniforms.  The two forms' tokens must agree."""
    import torch
    from speculative_sampling_verification_verify_amd import binding
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    rows = []
    for B, G, V in ((1, 4, 128256), (4, 4, 128256), (8, 4, 128256), (1, 7, 152064)):
        rng = np.random.default_rng(1000 * B + G)
        zp = (3.0 * rng.normal(size=(B, G + 1, V))).astype(np.float32)
        zq = (zp[:, :G] + 0.7 * rng.normal(size=(B, G, V))).astype(np.float32)
        P = torch.from_numpy(synth.f32_to_bf16_bits(zp).view(np.int16)).to(dev).view(torch.bfloat16)
        Q = torch.from_numpy(synth.f32_to_bf16_bits(zq).view(np.int16)).to(dev).view(torch.bfloat16)
        call = (t(rng.integers(0, V, size=(B, G)).astype(np.int32)), t(rng.random((B, G + 1)).astype(np.float32)),
                t(np.ones(B, np.float32)), t(np.zeros(B, np.int32)), t(np.ones(B, np.float32)),
                t(np.full(B, G, np.int32)))
        # Rotated copies keep the rows out of the last-level cache between calls.
        nsets = int(min(32, max(1, -(-ROTATE_BYTES // (zp.nbytes // 2 + zq.nbytes // 2)))))
        sets = [(P, Q)] + [(P.clone(), Q.clone()) for _ in range(nsets - 1)]
        out = {"B": B, "gamma": G, "V": V}
        toks = {}
        for name, hints in (("one_workgroup_per_pair_us", binding.SV_HINT_ALL_DENSE),
                            ("split_us", binding.SV_HINT_ALL_DENSE | binding.SV_HINT_UNFILTERED)):
            ver = binding.Verifier(B, G, V, binding.SV_BF16, device=dev, hints=hints)
            for j in range(args.warmup):
                ver(*sets[j % nsets], *call)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for j in range(args.steps):
                ver(*sets[j % nsets], *call)
            torch.cuda.synchronize()
            out[name] = (time.perf_counter() - t0) / args.steps * 1e6
            ver(P, Q, *call)
            toks[name] = ver.tokens.cpu().numpy().copy()
        out["same_tokens"] = bool((toks["split_us"] == toks["one_workgroup_per_pair_us"]).all())
        rows.append(out)
    print(json.dumps({"metric": "verify call latency, small batches of unfiltered bf16 rows", "unit": "us",
                      "higher_is_better": False, "steps": args.steps, "warmup": args.warmup, "rows": rows}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, help="synthetic workload id (3 = headline)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--gumbel", action="store_true",
                    help="the shared-noise (Gumbel coupling) verify on the workload's shapes instead")
    ap.add_argument("--spectr", action="store_true",
                    help="the multi-candidate (K-SEQ / SpecTr) verify at K = 8, L = 8 instead")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (HBM counter calibration)")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the oracle check of the last timed call's outputs")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read ceiling on the call's logit buffers")
    ap.add_argument("--small-batch", action="store_true",
                    help="call latency of small batches of long unfiltered rows, with and without the split pairs")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the verify step on one GPU; runs on more than one GPU are not supported "
              "(sequences shard across GPUs with no exchange, so per-GPU throughput is the figure).",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        import torch
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": args.steps}))
        return

    if args.gumbel:
        main_gumbel(args)
        return
    if args.spectr:
        main_spectr(args)
        return
    if args.small_batch:
        main_small_batch(args)
        return

    t_gen = time.perf_counter()
    bt = synth.make_batch(args.workload)
    t_gen = time.perf_counter() - t_gen
    alg_bytes = synth.algorithmic_bytes(bt)
    logit_bytes = int((2 * bt.gamma_len.astype(np.int64) + 1).sum()) * bt.V * bt.p_logits.itemsize

    # CPU work first: worker processes are forked before the GPU is touched.
    # The oracle's outputs for every sequence, to check the timed calls' outputs.
    cores = host_cores()
    t_ref = time.perf_counter()
    ref = None if args.no_check else oracle_reference(bt, cores)
    t_ref = time.perf_counter() - t_ref
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(bt, args.cpu_seconds, cores)

    import torch
    from speculative_sampling_verification_verify_amd import binding

    dev = torch.device("cuda:0")
    if bt.p_logits.dtype == np.uint16:
        P = torch.from_numpy(bt.p_logits.view(np.int16)).to(dev).view(torch.bfloat16)
        Q = torch.from_numpy(bt.q_logits.view(np.int16)).to(dev).view(torch.bfloat16)
        dt_code, dtype_name = binding.SV_BF16, "bf16"
    else:
        P = torch.from_numpy(bt.p_logits).to(dev)
        Q = torch.from_numpy(bt.q_logits).to(dev)
        dt_code, dtype_name = binding.SV_FP32, "fp32"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    draft, u, temp, topk, topp, gl = (t(bt.draft), t(bt.u), t(bt.temperature), t(bt.top_k), t(bt.top_p),
                                      t(bt.gamma_len))
    # The sampling settings are known on the host: when no sequence is dense
    # (every one argmax or top-k <= 512) the call says so and the empty
    # dense-pair launch is skipped; when every sequence is dense it says that,
    # and the select launch (which would only list the pairs) is skipped.
    sel_bytes, pair_bytes = kernel_bytes(bt)
    hints = binding.SV_HINT_NO_DENSE if pair_bytes == 0 else (binding.SV_HINT_ALL_DENSE if sel_bytes == 0 else 0)
    # No top-k and no top-p anywhere: the unfiltered hint (a host-side fact as well).
    if pair_bytes > 0 and not ((bt.top_k > 0) & (bt.top_k < bt.V)).any() and not (bt.top_p < 1.0).any():
        hints |= binding.SV_HINT_UNFILTERED
    ver = binding.Verifier(bt.B, bt.gamma_max, bt.V, dt_code, device=dev, hints=hints)
    # Copies of the logits, rotated step by step, so that a workload smaller
    # than the 256 MB last-level cache is still read from HBM.
    nsets = int(min(32, max(1, -(-ROTATE_BYTES // max(logit_bytes, 1)))))
    sets = [(P, Q)] + [(P.clone(), Q.clone()) for _ in range(nsets - 1)]
    torch.cuda.synchronize()

    def step(j):
        Pj, Qj = sets[j % nsets]
        ver(Pj, Qj, draft, u, temp, topk, topp, gl)

    # The kernel that reads most of the logit bytes: the streaming select for
    # top-k / argmax sequences, the pair kernel for dense ones; with both kinds
    # on the histogram variant, the pair-stage kernel that reads them all (the
    # select launch then only lists the dense pairs).
    mixed = sel_bytes > 0 and pair_bytes > 0 and pair_kernel_name(bt) == "pair_hist_kernel"
    kernel = binding.SV_KERNEL_PAIR if pair_bytes > sel_bytes or mixed else binding.SV_KERNEL_SELECT
    kname = "select_kernel" if kernel == binding.SV_KERNEL_SELECT else pair_kernel_name(bt, mixed)
    kbytes = sel_bytes + pair_bytes if mixed else max(sel_bytes, pair_bytes)

    for j in range(args.warmup):
        step(j)
    torch.cuda.synchronize()
    K = args.steps

    wall, k_ms = timed_calls(step, kernel, K)
    ms_per_step = wall * 1e3 / K
    n_acc = ver.n_accepted.cpu().numpy()
    alpha = ver.alpha.cpu().numpy()
    # Outside the timed region: the last timed call's outputs against the oracle.
    check = None
    if ref is not None:
        check = output_check(bt, ref, ver.tokens.cpu().numpy(), n_acc, alpha, ver.pq.cpu().numpy())
    # Outside the timed region: the other kernels' durations, for the record.
    other_us = {}
    for kern, name in ((binding.SV_KERNEL_SELECT, "select_kernel (dense-pair listing only)" if mixed else "select_kernel"),
                       (binding.SV_KERNEL_PAIR, pair_kernel_name(bt, mixed)), (binding.SV_KERNEL_FINISH, "finish_kernel")):
        if (kern == binding.SV_KERNEL_PAIR and hints & binding.SV_HINT_NO_DENSE) or \
                (kern == binding.SV_KERNEL_SELECT and hints & binding.SV_HINT_ALL_DENSE):
            other_us[name] = None      # not launched
        elif kern != kernel:
            _, ms = timed_calls(step, kern, min(K, 20), every=1)
            other_us[name] = float(ms.mean() * 1e3) if (ms > 0).all() else None
    k_avg = float(k_ms.mean())
    achieved = kbytes / (k_avg * 1e-3) / 1e9
    traffic = traffic_from_profile(kname, bt.workload.name)
    w = bt.workload
    ceiling = None if args.no_ceiling else read_ceiling(P, Q)
    single = single_round_latency(bt, P, Q, draft, u, temp, topk, topp, gl, dt_code, hints, ver) \
        if args.workload == 0 else None
    out = {
        "metric": METRIC,
        "value": bt.B / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic",
        "config": {"workload": w.name, "B": bt.B, "V": bt.V, "gamma": bt.gamma_max,
                   "temperature": float(w.temperature), "top_k": int(w.top_k), "top_p": float(w.top_p),
                   "logit_bytes_per_call": logit_bytes, "parallelism": "single-gpu",
                   "hints": "+".join(n for f, n in ((binding.SV_HINT_NO_DENSE, "no-dense"),
                                                     (binding.SV_HINT_ALL_DENSE, "all-dense"),
                                                     (binding.SV_HINT_UNFILTERED, "unfiltered")) if hints & f) or "none"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kname, "kernel_bytes_per_launch": kbytes, "kernel_avg_us": k_avg * 1e3,
                     "kernel_p10_us": float(np.percentile(k_ms, 10) * 1e3),
                     "kernel_p90_us": float(np.percentile(k_ms, 90) * 1e3),
                     "kernel_timed_launches": int(len(k_ms)), "event_every": EVENT_EVERY},
        "cpu_baseline": cpu,
        "cpu_model": cpu_model(),
        "near_margin": check,
        "read_ceiling": ceiling,
        "extra": {"call_GBps": alg_bytes / (ms_per_step * 1e-3) / 1e9,
                  "kernel_frac_of_read_ceiling": achieved / ceiling["achieved"] if ceiling else None,
                  "single_round_B1": single,
                  "oracle_reference_s": t_ref,
                  "logit_rows_per_s": int((2 * bt.gamma_len.astype(np.int64) + 1).sum()) / (ms_per_step * 1e-3),
                  "mean_alpha": float(alpha[alpha > 0].mean()) if (alpha > 0).any() else None,
                  "mean_tokens_per_round": float((n_acc[n_acc >= 0] + 1).mean()),
                  "other_kernels_avg_us": other_us,
                  "input_sets_rotated": nsets,
                  "input_generation_s": t_gen},
    }
    print(json.dumps(out))
    if check is not None and not check["ok"]:
        print("bench.py: the timed call's outputs break the parity rules against the oracle", file=sys.stderr)
        sys.exit(3)


def single_round_latency(bt, P, Q, draft, u, temp, topk, topp, gl, dt_code, hints, batched, rounds=1000):
    """The tiny workload as it is stated: one sequence per call, `rounds`
    calls in a row (round r takes sequence r of the batch), each call timed
    with events on the stream; the outputs must equal the batched call's."""
    import torch
    from speculative_sampling_verification_verify_amd import binding
    rounds = min(rounds, bt.B)
    one = binding.Verifier(1, bt.gamma_max, bt.V, dt_code, device=P.device, hints=hints)
    toks = torch.empty((rounds, bt.gamma_max + 1), dtype=torch.int32, device=P.device)
    ns = torch.empty((rounds,), dtype=torch.int32, device=P.device)
    sl = lambda t, r: t[r:r + 1]

    def call(r):
        return one(sl(P, r), sl(Q, r), sl(draft, r), sl(u, r), sl(temp, r), sl(topk, r), sl(topp, r), sl(gl, r))

    # An untimed pass keeps every round's outputs for the comparison.
    for r in range(rounds):
        tok, n, _, _ = call(r)
        toks[r:r + 1].copy_(tok)
        ns[r:r + 1].copy_(n)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(rounds)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r, (a, b) in enumerate(evs):
        a.record()
        call(r)
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    same = bool(torch.equal(toks, batched.tokens[:rounds]) and torch.equal(ns, batched.n_accepted[:rounds]))
    return {"calls": rounds, "B": 1, "us_per_call_events_mean": float(us.mean()),
            "us_per_call_events_p50": float(np.median(us)), "us_per_call_events_p90": float(np.percentile(us, 90)),
            "us_per_call_wall": wall * 1e6 / rounds, "outputs_equal_batched_call": same}


if __name__ == "__main__":
    main()

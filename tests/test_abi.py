"""The C ABI library: it loads, exports every entry point declared in
include/spec_verify.h, and rejects bad arguments on the host before touching
the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

from speculative_sampling_verification_verify_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def _ensure_built():
    if not os.path.exists(binding.LIB_PATH):
        from speculative_sampling_verification_verify_amd import build
        build.build_library()
    return binding.lib()


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(spec_\w*)\s*\(", txt, flags=re.M)))


def test_header_declares_entry_points():
    names = declared_functions()
    assert set(names) == set(binding.EXPORTED), names


def test_library_exports_every_declared_symbol():
    L = _ensure_built()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert binding.spec_verify_version() == 11


def test_workspace_bytes():
    _ensure_built()
    ws = binding.spec_verify_workspace_bytes
    assert ws(256, 7, 152064, binding.SV_BF16) > 0
    assert ws(256, 7, 152064, binding.SV_BF16) >= ws(128, 7, 152064, binding.SV_BF16)
    assert ws(1, 1, 1, binding.SV_FP32) > 0
    assert ws(0, 4, 100, binding.SV_BF16) > 0
    for bad in [(-1, 4, 100, 0), (4, 0, 100, 0), (4, 65, 100, 0), (4, 4, 0, 0), (4, 4, (1 << 20) + 1, 0),
                (4, 4, 100, 7)]:
        assert ws(*bad) == 0, bad


def test_workspace_bytes_sweep():
    """The plan of parts per row and the workspace layout over a spread of
    shapes: every valid shape gets a size that holds at least one survivor
    list (1024 entries of 8 bytes) per logit row, for the verify (2G+1 rows
    per sequence) and the shared-noise verify (G+1).  (Small batches get more
    parts per row, so the size need not grow with B.)"""
    L = _ensure_built()
    ws = binding.spec_verify_workspace_bytes
    gws = L.spec_verify_gumbel_workspace_bytes
    for dt in (binding.SV_BF16, binding.SV_FP32):
        for V in (1, 7, 8, 1000, 2048, 32000, 32769, 65544, 131072, 152064, 1 << 20):
            for G in (1, 2, 7, 8, 31, 64):
                for B in (0, 1, 2, 7, 64, 256, 1000, 4096):
                    assert ws(B, G, V, dt) >= max(1, B * (2 * G + 1) * 8192), (B, G, V, dt)
                    assert gws(B, G, V, dt) >= max(1, B * (G + 1) * 8192), (B, G, V, dt)


def test_host_argument_errors():
    L = _ensure_built()
    fake = ctypes.c_void_p(0x100000)   # never dereferenced: every case below fails on the host
    nul = None
    B, G, V = 2, 3, 64
    need = binding.spec_verify_workspace_bytes(B, G, V, binding.SV_BF16)

    def call(p=fake, q=fake, dt=binding.SV_BF16, draft=fake, u=fake, temp=fake, B=B, G=G, V=V, out=fake,
             ws=fake, wsb=need):
        return L.spec_verify(p, q, dt, draft, nul, u, temp, nul, nul, B, G, V, out, out, out, nul, ws, wsb, nul)

    assert call(dt=5) == binding.SV_ERR_UNSUPPORTED
    assert call(G=65) == binding.SV_ERR_UNSUPPORTED
    assert call(V=(1 << 20) + 1) == binding.SV_ERR_UNSUPPORTED
    assert call(G=0) == binding.SV_ERR_ARG
    assert call(V=0) == binding.SV_ERR_ARG
    assert call(B=-3) == binding.SV_ERR_ARG
    assert call(p=nul) == binding.SV_ERR_ARG
    assert call(draft=nul) == binding.SV_ERR_ARG
    assert call(u=nul) == binding.SV_ERR_ARG
    assert call(temp=nul) == binding.SV_ERR_ARG
    assert call(out=nul) == binding.SV_ERR_ARG
    assert call(p=ctypes.c_void_p(0x100001)) == binding.SV_ERR_ARG          # misaligned bf16
    assert call(ws=nul) == binding.SV_ERR_WORKSPACE
    assert call(wsb=need - 1) == binding.SV_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(0x100010)) == binding.SV_ERR_WORKSPACE   # not 256-byte aligned
    assert call(B=0) == binding.SV_OK                                         # empty batch: nothing to do
    rc = L.spec_verify_workspace_init(nul, 0, B, G, V, binding.SV_BF16, nul)
    assert rc == binding.SV_ERR_WORKSPACE
    assert L.spec_verify_workspace_init(fake, need, B, 0, V, binding.SV_BF16, nul) == binding.SV_ERR_ARG


def test_gumbel_host_argument_errors():
    L = _ensure_built()
    fake = ctypes.c_void_p(0x100000)   # never dereferenced: every case below fails on the host
    nul = None
    B, G, V = 2, 3, 64

    need = binding.lib().spec_verify_gumbel_workspace_bytes(B, G, V, binding.SV_BF16)
    assert need > 0

    def call(p=fake, dt=binding.SV_BF16, noise=fake, draft=fake, temp=fake, B=B, G=G, V=V, out=fake, tgt=fake,
             ws=fake, wsb=need):
        return L.spec_verify_gumbel(p, dt, noise, draft, nul, temp, nul, nul, B, G, V, out, out, tgt, ws, wsb, nul)

    assert call(ws=nul) == binding.SV_ERR_WORKSPACE
    assert call(wsb=need - 1) == binding.SV_ERR_WORKSPACE

    assert call(dt=3) == binding.SV_ERR_UNSUPPORTED
    assert call(G=65) == binding.SV_ERR_UNSUPPORTED
    assert call(V=(1 << 20) + 1) == binding.SV_ERR_UNSUPPORTED
    assert call(G=0) == binding.SV_ERR_ARG
    assert call(B=-1) == binding.SV_ERR_ARG
    assert call(p=nul) == binding.SV_ERR_ARG
    assert call(noise=nul) == binding.SV_ERR_ARG
    assert call(draft=nul) == binding.SV_ERR_ARG
    assert call(temp=nul) == binding.SV_ERR_ARG
    assert call(out=nul) == binding.SV_ERR_ARG
    assert call(tgt=nul) == binding.SV_ERR_ARG
    assert call(noise=ctypes.c_void_p(0x100002)) == binding.SV_ERR_ARG      # misaligned float noise
    assert call(p=ctypes.c_void_p(0x100001)) == binding.SV_ERR_ARG          # misaligned bf16
    assert call(B=0) == binding.SV_OK

    def call_ex(hints, B=B):
        return L.spec_verify_gumbel_ex(fake, binding.SV_BF16, fake, fake, nul, fake, nul, nul, hints, B, G, V, fake,
                                       fake, fake, fake, need, nul)

    assert call_ex(binding.SV_HINT_NO_DENSE | binding.SV_HINT_ALL_DENSE) == binding.SV_ERR_ARG
    assert call_ex(binding.SV_HINT_NO_DENSE, B=0) == binding.SV_OK
    assert call_ex(4) == binding.SV_ERR_ARG
    assert call_ex(binding.SV_HINT_ALL_DENSE, B=0) == binding.SV_OK
    assert call_ex(binding.SV_HINT_ALL_DENSE, B=-1) == binding.SV_ERR_ARG


def test_sample_and_lenient_host_argument_errors():
    L = _ensure_built()
    fake = ctypes.c_void_p(0x100000)
    nul = None
    R, V = 4, 64
    need = binding.spec_sample_workspace_bytes(R, V, binding.SV_BF16)
    assert need > 0 and binding.spec_sample_workspace_bytes(R, 0, binding.SV_BF16) == 0
    assert binding.spec_sample_workspace_bytes(-1, V, binding.SV_BF16) == 0

    def sample(p=fake, dt=binding.SV_BF16, u=fake, temp=fake, R=R, V=V, out=fake, ws=fake, wsb=need):
        return L.spec_sample(p, dt, u, temp, nul, nul, R, V, out, ws, wsb, nul)

    assert sample(dt=9) == binding.SV_ERR_UNSUPPORTED
    assert sample(V=(1 << 20) + 1) == binding.SV_ERR_UNSUPPORTED
    assert sample(R=-1) == binding.SV_ERR_ARG
    assert sample(V=0) == binding.SV_ERR_ARG
    assert sample(p=nul) == binding.SV_ERR_ARG
    assert sample(u=nul) == binding.SV_ERR_ARG
    assert sample(temp=nul) == binding.SV_ERR_ARG
    assert sample(out=nul) == binding.SV_ERR_ARG
    assert sample(ws=nul) == binding.SV_ERR_WORKSPACE
    assert sample(wsb=need - 1) == binding.SV_ERR_WORKSPACE
    assert sample(R=0) == binding.SV_OK
    assert L.spec_sample_workspace_init(nul, 0, R, V, binding.SV_BF16, nul) == binding.SV_ERR_WORKSPACE

    gneed = binding.lib().spec_verify_gumbel_workspace_bytes(R, 0, V, binding.SV_BF16)

    def gsample(p=fake, noise=fake, temp=fake, R=R, V=V, out=fake):
        return L.spec_sample_gumbel(p, binding.SV_BF16, noise, temp, nul, nul, R, V, out, fake, gneed, nul)

    assert gsample(noise=nul) == binding.SV_ERR_ARG
    assert gsample(out=nul) == binding.SV_ERR_ARG
    assert gsample(R=-2) == binding.SV_ERR_ARG
    assert gsample(R=0) == binding.SV_OK

    B, G = 2, 3
    wneed = binding.spec_verify_workspace_bytes(B, G, V, binding.SV_BF16)
    ex = lambda q=fake, draft=fake, G=G, hints=0: L.spec_verify_ex(fake, q, binding.SV_BF16, draft, nul, fake, fake,
                                                                   nul, nul, nul, hints, B, G, V, fake, fake, fake,
                                                                   nul, fake, wneed, nul)
    assert ex(q=nul) == binding.SV_ERR_ARG
    assert ex(draft=nul) == binding.SV_ERR_ARG
    assert ex(G=0) == binding.SV_ERR_ARG
    assert ex(hints=8) == binding.SV_ERR_ARG
    assert ex(hints=binding.SV_HINT_ALL_DENSE | binding.SV_HINT_UNFILTERED | 16) == binding.SV_ERR_ARG
    assert ex(hints=binding.SV_HINT_NO_DENSE | binding.SV_HINT_ALL_DENSE) == binding.SV_ERR_ARG


def test_spectr_host_argument_errors():
    L = _ensure_built()
    fake = ctypes.c_void_p(0x100000)
    nul = None

    def call(p=fake, q=fake, dt=binding.SV_BF16, cand=fake, u=fake, temp=fake, B=2, K=4, Ln=3, V=64, out=fake):
        return L.spec_verify_spectr(p, q, dt, cand, u, temp, nul, nul, B, K, Ln, V, out, out, out, nul)

    assert call(dt=4) == binding.SV_ERR_UNSUPPORTED
    assert call(K=65) == binding.SV_ERR_UNSUPPORTED
    assert call(Ln=65) == binding.SV_ERR_UNSUPPORTED
    assert call(V=(1 << 20) + 1) == binding.SV_ERR_UNSUPPORTED
    assert call(K=0) == binding.SV_ERR_ARG
    assert call(Ln=0) == binding.SV_ERR_ARG
    assert call(V=0) == binding.SV_ERR_ARG
    assert call(B=-1) == binding.SV_ERR_ARG
    for kw in ("p", "q", "cand", "u", "temp", "out"):
        assert call(**{kw: nul}) == binding.SV_ERR_ARG, kw
    assert call(p=ctypes.c_void_p(0x100001)) == binding.SV_ERR_ARG
    assert call(V=600001) == binding.SV_ERR_UNSUPPORTED     # odd V above 64 KB rows: beyond the streamed limit
    assert call(B=0) == binding.SV_OK


def test_stage_events_kernel_selector():
    L = _ensure_built()
    assert L.spec_verify_set_stage_events(7, None, None) == binding.SV_ERR_ARG
    assert L.spec_verify_set_stage_events(5, None, None) == binding.SV_ERR_ARG
    assert L.spec_verify_set_stage_events(-1, None, None) == binding.SV_ERR_ARG
    for k in (binding.SV_KERNEL_SELECT, binding.SV_KERNEL_PAIR, binding.SV_KERNEL_FINISH, binding.SV_KERNEL_GUMBEL,
              binding.SV_KERNEL_KSEQ):
        assert L.spec_verify_set_stage_events(k, None, None) == binding.SV_OK


def test_strerror():
    _ensure_built()
    for code in (0, -1, -2, -3, -4, 17):
        assert isinstance(binding.spec_verify_strerror(code), str)
    assert "workspace" in binding.spec_verify_strerror(binding.SV_ERR_WORKSPACE)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()


def test_noalloc_host_errors():
    """The allocation-free entry point checks its arguments, and that the call
    fits its fixed buffer, before any HIP call (no GPU is touched here)."""
    L = _ensure_built()
    fake = ctypes.c_void_p(0x100000)
    nul = None
    bf = binding.SV_BF16

    def call(p=fake, q=fake, dt=bf, draft=fake, u=fake, temp=fake, hints=0, B=2, G=3, V=64, out=fake):
        return L.spec_verify_noalloc(p, q, dt, draft, nul, u, temp, nul, nul, nul, hints, B, G, V, out, out, out,
                                     nul, nul)

    assert call(dt=5) == binding.SV_ERR_UNSUPPORTED
    assert call(G=65) == binding.SV_ERR_UNSUPPORTED
    assert call(V=0) == binding.SV_ERR_ARG
    assert call(p=nul) == binding.SV_ERR_ARG
    assert call(out=nul) == binding.SV_ERR_ARG
    assert call(p=ctypes.c_void_p(0x100001)) == binding.SV_ERR_ARG
    assert call(hints=3) == binding.SV_ERR_ARG
    assert call(B=0) == binding.SV_OK
    # Sizes whose workspace exceeds the fixed buffer: a clear error, nothing enqueued.
    big = (512, 8, 152064)
    assert binding.spec_verify_workspace_bytes(*big, bf) > binding.SV_NOALLOC_SCRATCH_BYTES
    rc = call(B=big[0], G=big[1], V=big[2])
    assert rc == binding.SV_ERR_SCRATCH
    assert "fixed buffer" in binding.spec_verify_strerror(rc)
    # The benchmark's workloads fit.
    for B, G, V, dt in ((1, 4, 1000, binding.SV_FP32), (32, 5, 32000, bf), (64, 4, 128256, bf),
                        (256, 7, 152064, bf), (128, 8, 128256, bf)):
        assert binding.spec_verify_workspace_bytes(B, G, V, dt) <= binding.SV_NOALLOC_SCRATCH_BYTES

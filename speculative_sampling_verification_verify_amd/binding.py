"""ctypes binding of libspecverify.so (the C ABI in include/spec_verify.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the verify computation runs in the HIP
kernels.  The functions keep the C names; ``Verifier`` owns a workspace and
output tensors for repeated calls.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; SV_LIBRARY names another build of the same source (the
# host-sanitized one the ABI tests also run against).
LIB_PATH = os.environ.get("SV_LIBRARY") or os.path.join(_HERE, "libspecverify.so")

SV_BF16, SV_FP32 = 0, 1
SV_OK, SV_ERR_ARG, SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE, SV_ERR_HIP, SV_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
SV_NOALLOC_SCRATCH_BYTES = 64 << 20
SV_KERNEL_SELECT, SV_KERNEL_PAIR, SV_KERNEL_FINISH, SV_KERNEL_GUMBEL, SV_KERNEL_KSEQ = 0, 1, 2, 3, 4
SV_MAX_CANDIDATES = 64
SV_HINT_NO_DENSE = 1
SV_HINT_ALL_DENSE = 2
SV_HINT_UNFILTERED = 4
SV_MAX_GAMMA = 64
SV_MAX_VOCAB = 1 << 20

EXPORTED = ("spec_verify_workspace_bytes", "spec_verify_workspace_init", "spec_verify", "spec_verify_ex",
            "spec_verify_strerror", "spec_verify_version", "spec_verify_set_stage_events", "spec_verify_gumbel",
            "spec_sample_workspace_bytes", "spec_sample_workspace_init", "spec_sample", "spec_sample_gumbel",
            "spec_verify_expected_tokens", "spec_verify_speedup", "spec_verify_operations",
            "spec_verify_optimal_gamma", "spec_verify_acceptance_length", "spec_verify_spectr",
            "spec_verify_gumbel_workspace_bytes", "spec_verify_gumbel_workspace_init", "spec_verify_gumbel_ex",
            "spec_verify_noalloc")

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where} failed with {code}: {spec_verify_strerror(code)}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.spec_verify_workspace_bytes.argtypes = [i, i, i, i]
        L.spec_verify_workspace_bytes.restype = sz
        L.spec_verify_workspace_init.argtypes = [vp, sz, i, i, i, i, vp]
        L.spec_verify_workspace_init.restype = i
        L.spec_verify.argtypes = [vp, vp, i, vp, vp, vp, vp, vp, vp, i, i, i, vp, vp, vp, vp, vp, sz, vp]
        L.spec_verify.restype = i
        L.spec_verify_strerror.argtypes = [i]
        L.spec_verify_strerror.restype = ctypes.c_char_p
        L.spec_verify_version.argtypes = []
        L.spec_verify_version.restype = i
        L.spec_verify_set_stage_events.argtypes = [i, vp, vp]
        L.spec_verify_gumbel.argtypes = [vp, i, vp, vp, vp, vp, vp, vp, i, i, i, vp, vp, vp, vp, sz, vp]
        L.spec_verify_gumbel_workspace_bytes.argtypes = [i, i, i, i]
        L.spec_verify_gumbel_workspace_bytes.restype = sz
        L.spec_verify_gumbel_workspace_init.argtypes = [vp, sz, i, i, i, i, vp]
        L.spec_verify_gumbel_workspace_init.restype = i
        L.spec_verify_gumbel.restype = i
        L.spec_verify_gumbel_ex.argtypes = [vp, i, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, vp, vp, vp, sz, vp]
        L.spec_verify_gumbel_ex.restype = i
        L.spec_verify_ex.argtypes = [vp, vp, i, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, vp, vp, vp, vp, sz, vp]
        L.spec_verify_ex.restype = i
        L.spec_verify_noalloc.argtypes = [vp, vp, i, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, vp, vp, vp, vp]
        L.spec_verify_noalloc.restype = i
        L.spec_sample_workspace_bytes.argtypes = [i, i, i]
        L.spec_sample_workspace_bytes.restype = sz
        L.spec_sample_workspace_init.argtypes = [vp, sz, i, i, i, vp]
        L.spec_sample_workspace_init.restype = i
        L.spec_sample.argtypes = [vp, i, vp, vp, vp, vp, i, i, vp, vp, sz, vp]
        L.spec_sample.restype = i
        L.spec_sample_gumbel.argtypes = [vp, i, vp, vp, vp, vp, i, i, vp, vp, sz, vp]
        L.spec_sample_gumbel.restype = i
        L.spec_verify_spectr.argtypes = [vp, vp, i, vp, vp, vp, vp, vp, i, i, i, i, vp, vp, vp, vp]
        L.spec_verify_spectr.restype = i
        d = ctypes.c_double
        L.spec_verify_expected_tokens.argtypes = [d, i]
        L.spec_verify_expected_tokens.restype = d
        L.spec_verify_speedup.argtypes = [d, i, d]
        L.spec_verify_speedup.restype = d
        L.spec_verify_operations.argtypes = [d, i, d]
        L.spec_verify_operations.restype = d
        L.spec_verify_optimal_gamma.argtypes = [d, d, i]
        L.spec_verify_optimal_gamma.restype = i
        L.spec_verify_acceptance_length.argtypes = [ctypes.POINTER(d), i]
        L.spec_verify_acceptance_length.restype = d
        L.spec_verify_set_stage_events.restype = i
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    h = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return h or None


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype in (torch.bfloat16, torch.int16):
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_FP32
    raise TypeError(f"logits must be bfloat16 (or int16 bf16 bit patterns) or float32, got {t.dtype}")


def spec_verify_workspace_bytes(B: int, gamma_max: int, V: int, dtype: int) -> int:
    return int(lib().spec_verify_workspace_bytes(B, gamma_max, V, dtype))


def spec_verify_strerror(code: int) -> str:
    return lib().spec_verify_strerror(code).decode()


def spec_verify_version() -> int:
    return int(lib().spec_verify_version())


def spec_verify_set_stage_events(begin, end, kernel: int = SV_KERNEL_SELECT) -> None:
    """Record hipEvent_t handles (ints, or torch.cuda.Event already recorded
    once) around one kernel (SV_KERNEL_*) of the following calls; pass
    None, None to stop."""
    h = lambda e: None if e is None else (e.cuda_event if hasattr(e, "cuda_event") else int(e))
    rc = lib().spec_verify_set_stage_events(kernel, h(begin), h(end))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_set_stage_events")


def spec_verify_workspace_init(workspace: torch.Tensor, B: int, gamma_max: int, V: int, dtype: int,
                               stream=None) -> None:
    rc = lib().spec_verify_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                          B, gamma_max, V, dtype, _stream_handle(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_workspace_init")


def _check(t: Optional[torch.Tensor], name: str, dtype, shape, device):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def spec_verify(p_logits: torch.Tensor, q_logits: torch.Tensor, draft_tokens: torch.Tensor,
                gamma_len: Optional[torch.Tensor], uniforms: torch.Tensor, temperature: torch.Tensor,
                top_k: Optional[torch.Tensor], top_p: Optional[torch.Tensor],
                out_tokens: torch.Tensor, out_n_accepted: torch.Tensor, out_alpha: torch.Tensor,
                out_pq: Optional[torch.Tensor], workspace: torch.Tensor, stream=None,
                lenience: Optional[torch.Tensor] = None, hints: int = 0) -> None:
    """Enqueue one verify call (see include/spec_verify.h for the contract);
    with `lenience` ([B] float32) or `hints` (SV_HINT_* flags) the call goes
    to spec_verify_ex."""
    if p_logits.dim() != 3 or q_logits.dim() != 3:
        raise ValueError("p_logits must be [B, gamma_max+1, V] and q_logits [B, gamma_max, V]")
    B, G1, V = p_logits.shape
    G = G1 - 1
    dev = p_logits.device
    if dev.type != "cuda":
        raise ValueError("logits must live in GPU memory")
    dt = _dtype_code(p_logits)
    _check(q_logits, "q_logits", p_logits.dtype, (B, G, V), dev)
    _check(p_logits, "p_logits", p_logits.dtype, (B, G + 1, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, G), dev)
    _check(gamma_len, "gamma_len", torch.int32, (B,), dev)
    _check(uniforms, "uniforms", torch.float32, (B, G + 1), dev)
    _check(temperature, "temperature", torch.float32, (B,), dev)
    _check(top_k, "top_k", torch.int32, (B,), dev)
    _check(top_p, "top_p", torch.float32, (B,), dev)
    _check(out_tokens, "out_tokens", torch.int32, (B, G + 1), dev)
    _check(out_n_accepted, "out_n_accepted", torch.int32, (B,), dev)
    _check(out_alpha, "out_alpha", torch.float32, (B, G), dev)
    _check(out_pq, "out_pq", torch.float32, (B, G, 2), dev)
    _check(lenience, "lenience", torch.float32, (B,), dev)
    wsb = workspace.numel() * workspace.element_size()
    if lenience is None and not hints:
        rc = lib().spec_verify(_ptr(p_logits), _ptr(q_logits), dt, _ptr(draft_tokens), _ptr(gamma_len),
                               _ptr(uniforms), _ptr(temperature), _ptr(top_k), _ptr(top_p), B, G, V,
                               _ptr(out_tokens), _ptr(out_n_accepted), _ptr(out_alpha), _ptr(out_pq),
                               _ptr(workspace), wsb, _stream_handle(stream))
    else:
        rc = lib().spec_verify_ex(_ptr(p_logits), _ptr(q_logits), dt, _ptr(draft_tokens), _ptr(gamma_len),
                                  _ptr(uniforms), _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(lenience),
                                  int(hints), B, G, V, _ptr(out_tokens), _ptr(out_n_accepted), _ptr(out_alpha), _ptr(out_pq),
                                  _ptr(workspace), wsb, _stream_handle(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify")


def spec_verify_noalloc(p_logits: torch.Tensor, q_logits: torch.Tensor, draft_tokens: torch.Tensor,
                        gamma_len: Optional[torch.Tensor], uniforms: torch.Tensor, temperature: torch.Tensor,
                        top_k: Optional[torch.Tensor], top_p: Optional[torch.Tensor],
                        out_tokens: torch.Tensor, out_n_accepted: torch.Tensor, out_alpha: torch.Tensor,
                        out_pq: Optional[torch.Tensor], stream=None, lenience: Optional[torch.Tensor] = None,
                        hints: int = 0) -> None:
    """Enqueue one verify call on the library's fixed per-GPU buffer
    (spec_verify_noalloc: no workspace argument, nothing allocated)."""
    if p_logits.dim() != 3 or q_logits.dim() != 3:
        raise ValueError("p_logits must be [B, gamma_max+1, V] and q_logits [B, gamma_max, V]")
    B, G1, V = p_logits.shape
    G = G1 - 1
    dev = p_logits.device
    if dev.type != "cuda":
        raise ValueError("logits must live in GPU memory")
    dt = _dtype_code(p_logits)
    _check(q_logits, "q_logits", p_logits.dtype, (B, G, V), dev)
    _check(p_logits, "p_logits", p_logits.dtype, (B, G + 1, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, G), dev)
    _check(gamma_len, "gamma_len", torch.int32, (B,), dev)
    _check(uniforms, "uniforms", torch.float32, (B, G + 1), dev)
    _check(temperature, "temperature", torch.float32, (B,), dev)
    _check(top_k, "top_k", torch.int32, (B,), dev)
    _check(top_p, "top_p", torch.float32, (B,), dev)
    _check(out_tokens, "out_tokens", torch.int32, (B, G + 1), dev)
    _check(out_n_accepted, "out_n_accepted", torch.int32, (B,), dev)
    _check(out_alpha, "out_alpha", torch.float32, (B, G), dev)
    _check(out_pq, "out_pq", torch.float32, (B, G, 2), dev)
    _check(lenience, "lenience", torch.float32, (B,), dev)
    rc = lib().spec_verify_noalloc(_ptr(p_logits), _ptr(q_logits), dt, _ptr(draft_tokens), _ptr(gamma_len),
                                   _ptr(uniforms), _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(lenience),
                                   int(hints), B, G, V, _ptr(out_tokens), _ptr(out_n_accepted), _ptr(out_alpha),
                                   _ptr(out_pq), _stream_handle(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_noalloc")


class Verifier:
    """Owns a workspace and output buffers for calls of one shape."""

    def __init__(self, B: int, gamma_max: int, V: int, dtype: int = SV_BF16, device="cuda", with_pq=True,
                 hints: int = 0):
        self.B, self.G, self.V, self.dtype, self.hints = B, gamma_max, V, dtype, hints
        dev = torch.device(device)
        nbytes = spec_verify_workspace_bytes(B, gamma_max, V, dtype)
        if nbytes == 0:
            raise ValueError("unsupported sizes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        spec_verify_workspace_init(self.workspace, B, gamma_max, V, dtype)
        self.tokens = torch.empty((B, gamma_max + 1), dtype=torch.int32, device=dev)
        self.n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
        self.alpha = torch.empty((B, gamma_max), dtype=torch.float32, device=dev)
        self.pq = torch.empty((B, gamma_max, 2), dtype=torch.float32, device=dev) if with_pq else None

    def __call__(self, p_logits, q_logits, draft_tokens, uniforms, temperature, top_k=None, top_p=None,
                 gamma_len=None, stream=None, lenience=None):
        spec_verify(p_logits, q_logits, draft_tokens, gamma_len, uniforms, temperature, top_k, top_p,
                    self.tokens, self.n_accepted, self.alpha, self.pq, self.workspace, stream, lenience, self.hints)
        return self.tokens, self.n_accepted, self.alpha, self.pq


def gumbel_workspace(B: int, gamma_max: int, V: int, dtype: int, device) -> torch.Tensor:
    """A prepared workspace for spec_verify_gumbel (gamma_max = 0: spec_sample_gumbel)."""
    nbytes = int(lib().spec_verify_gumbel_workspace_bytes(B, gamma_max, V, dtype))
    if nbytes == 0:
        raise ValueError("unsupported sizes")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    rc = lib().spec_verify_gumbel_workspace_init(_ptr(ws), nbytes, B, gamma_max, V, dtype, _stream_handle(None))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_gumbel_workspace_init")
    return ws


def spec_verify_gumbel(p_logits: torch.Tensor, noise: torch.Tensor, draft_tokens: torch.Tensor,
                       gamma_len: Optional[torch.Tensor], temperature: torch.Tensor, top_k: Optional[torch.Tensor],
                       top_p: Optional[torch.Tensor], out_tokens: torch.Tensor, out_n_accepted: torch.Tensor,
                       out_target: torch.Tensor, workspace: torch.Tensor, stream=None, hints: int = 0) -> None:
    """Enqueue one shared-noise verify call (see include/spec_verify.h); with
    `hints` (SV_HINT_ALL_DENSE or SV_HINT_NO_DENSE) the call goes through
    spec_verify_gumbel_ex."""
    if p_logits.dim() != 3:
        raise ValueError("p_logits must be [B, gamma_max+1, V]")
    B, G1, V = p_logits.shape
    G = G1 - 1
    dev = p_logits.device
    if dev.type != "cuda":
        raise ValueError("logits must live in GPU memory")
    dt = _dtype_code(p_logits)
    _check(p_logits, "p_logits", p_logits.dtype, (B, G + 1, V), dev)
    _check(noise, "noise", torch.float32, (B, G + 1, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, G), dev)
    _check(gamma_len, "gamma_len", torch.int32, (B,), dev)
    _check(temperature, "temperature", torch.float32, (B,), dev)
    _check(top_k, "top_k", torch.int32, (B,), dev)
    _check(top_p, "top_p", torch.float32, (B,), dev)
    _check(out_tokens, "out_tokens", torch.int32, (B, G + 1), dev)
    _check(out_n_accepted, "out_n_accepted", torch.int32, (B,), dev)
    _check(out_target, "out_target", torch.int32, (B, G + 1), dev)
    head = (_ptr(p_logits), dt, _ptr(noise), _ptr(draft_tokens), _ptr(gamma_len), _ptr(temperature), _ptr(top_k),
            _ptr(top_p))
    tail = (B, G, V, _ptr(out_tokens), _ptr(out_n_accepted), _ptr(out_target), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if hints:
        rc, name = lib().spec_verify_gumbel_ex(*head, int(hints), *tail), "spec_verify_gumbel_ex"
    else:
        rc, name = lib().spec_verify_gumbel(*head, *tail), "spec_verify_gumbel"
    if rc != SV_OK:
        raise SpecVerifyError(rc, name)


class GumbelVerifier:
    """Workspace and output buffers for shared-noise verify calls of one shape."""

    def __init__(self, B: int, gamma_max: int, V: int, dtype: int = SV_BF16, device="cuda", hints: int = 0):
        dev = torch.device(device)
        self.hints = hints
        self.workspace = gumbel_workspace(B, gamma_max, V, dtype, dev)
        self.tokens = torch.empty((B, gamma_max + 1), dtype=torch.int32, device=dev)
        self.n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
        self.target = torch.empty((B, gamma_max + 1), dtype=torch.int32, device=dev)

    def __call__(self, p_logits, noise, draft_tokens, temperature, top_k=None, top_p=None, gamma_len=None,
                 stream=None):
        spec_verify_gumbel(p_logits, noise, draft_tokens, gamma_len, temperature, top_k, top_p, self.tokens,
                           self.n_accepted, self.target, self.workspace, stream, self.hints)
        return self.tokens, self.n_accepted, self.target


def spec_sample_workspace_bytes(R: int, V: int, dtype: int) -> int:
    return int(lib().spec_sample_workspace_bytes(R, V, dtype))


class Sampler:
    """One token per row from the processed distribution, by inverse CDF at a
    uniform (spec_sample); owns the workspace and the output for one shape."""

    def __init__(self, R: int, V: int, dtype: int = SV_BF16, device="cuda"):
        self.R, self.V, self.dtype = R, V, dtype
        dev = torch.device(device)
        nbytes = spec_sample_workspace_bytes(R, V, dtype)
        if nbytes == 0:
            raise ValueError("unsupported sizes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        rc = lib().spec_sample_workspace_init(_ptr(self.workspace), nbytes, R, V, dtype,
                                              _stream_handle(None))
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_sample_workspace_init")
        self.tokens = torch.empty((R,), dtype=torch.int32, device=dev)

    def __call__(self, logits, uniforms, temperature, top_k=None, top_p=None, stream=None):
        if logits.dim() != 2:
            raise ValueError("logits must be [R, V]")
        R, V = logits.shape
        dev = logits.device
        dt = _dtype_code(logits)
        _check(logits, "logits", logits.dtype, (self.R, self.V), dev)
        _check(uniforms, "uniforms", torch.float32, (R,), dev)
        _check(temperature, "temperature", torch.float32, (R,), dev)
        _check(top_k, "top_k", torch.int32, (R,), dev)
        _check(top_p, "top_p", torch.float32, (R,), dev)
        rc = lib().spec_sample(_ptr(logits), dt, _ptr(uniforms), _ptr(temperature), _ptr(top_k), _ptr(top_p), R, V,
                               _ptr(self.tokens), _ptr(self.workspace),
                               self.workspace.numel() * self.workspace.element_size(), _stream_handle(stream))
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_sample")
        return self.tokens


def spec_sample_gumbel(logits: torch.Tensor, noise: torch.Tensor, temperature: torch.Tensor,
                       top_k: Optional[torch.Tensor] = None, top_p: Optional[torch.Tensor] = None,
                       out_tokens: Optional[torch.Tensor] = None, stream=None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The shared-noise drafter's sample per row (spec_sample_gumbel); a
    workspace is made for the call when none is given."""
    if logits.dim() != 2:
        raise ValueError("logits must be [R, V]")
    R, V = logits.shape
    dev = logits.device
    dt = _dtype_code(logits)
    _check(noise, "noise", torch.float32, (R, V), dev)
    _check(temperature, "temperature", torch.float32, (R,), dev)
    _check(top_k, "top_k", torch.int32, (R,), dev)
    _check(top_p, "top_p", torch.float32, (R,), dev)
    if out_tokens is None:
        out_tokens = torch.empty((R,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", torch.int32, (R,), dev)
    if workspace is None:
        workspace = gumbel_workspace(R, 0, V, dt, dev)
    rc = lib().spec_sample_gumbel(_ptr(logits), dt, _ptr(noise), _ptr(temperature), _ptr(top_k), _ptr(top_p), R, V,
                                  _ptr(out_tokens), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream_handle(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_sample_gumbel")
    return out_tokens


# Throughput analytics (host functions of the library).
def spec_verify_expected_tokens(alpha: float, gamma: int) -> float:
    return float(lib().spec_verify_expected_tokens(alpha, gamma))


def spec_verify_speedup(alpha: float, gamma: int, c: float) -> float:
    return float(lib().spec_verify_speedup(alpha, gamma, c))


def spec_verify_operations(alpha: float, gamma: int, c_hat: float) -> float:
    return float(lib().spec_verify_operations(alpha, gamma, c_hat))


def spec_verify_optimal_gamma(alpha: float, c: float, gamma_max: int) -> int:
    return int(lib().spec_verify_optimal_gamma(alpha, c, gamma_max))


def spec_verify_acceptance_length(alphas) -> float:
    arr = (ctypes.c_double * len(alphas))(*[float(a) for a in alphas])
    return float(lib().spec_verify_acceptance_length(arr, len(alphas)))


class SpectrVerifier:
    """Output buffers for multi-candidate (K-SEQ / SpecTr) verify calls of one
    shape (spec_verify_spectr)."""

    def __init__(self, B: int, K: int, L: int, device="cuda"):
        dev = torch.device(device)
        self.B, self.K, self.L = B, K, L
        self.tokens = torch.empty((B, L + 1), dtype=torch.int32, device=dev)
        self.n = torch.empty((B,), dtype=torch.int32, device=dev)
        self.node_tokens = torch.empty((B, K, L + 1), dtype=torch.int32, device=dev)

    def __call__(self, p_logits, q_logits, candidates, uniforms, temperature, top_k=None, top_p=None, stream=None):
        if p_logits.dim() != 4 or q_logits.dim() != 4:
            raise ValueError("p_logits must be [B, K, L+1, V] and q_logits [B, K, L, V]")
        B, K, L1, V = p_logits.shape
        L = L1 - 1
        dev = p_logits.device
        dt = _dtype_code(p_logits)
        _check(p_logits, "p_logits", p_logits.dtype, (self.B, self.K, self.L + 1, V), dev)
        _check(q_logits, "q_logits", p_logits.dtype, (B, K, L, V), dev)
        _check(candidates, "candidates", torch.int32, (B, K, L), dev)
        _check(uniforms, "uniforms", torch.float32, (B, L + 1, K + 1), dev)
        _check(temperature, "temperature", torch.float32, (B,), dev)
        _check(top_k, "top_k", torch.int32, (B,), dev)
        _check(top_p, "top_p", torch.float32, (B,), dev)
        rc = lib().spec_verify_spectr(_ptr(p_logits), _ptr(q_logits), dt, _ptr(candidates), _ptr(uniforms),
                                      _ptr(temperature), _ptr(top_k), _ptr(top_p), B, K, L, V, _ptr(self.tokens),
                                      _ptr(self.n), _ptr(self.node_tokens), _stream_handle(stream))
        if rc != SV_OK:
            raise SpecVerifyError(rc, "spec_verify_spectr")
        return self.tokens, self.n

"""MI355X-native Kimi Delta Attention (KDA) forward: Python binding.

Thin ctypes binding over ``libkda.so`` (the C ABI declared in include/kda.h).
It only marshals arguments: every step of the computation runs in the HIP
kernels.  PyTorch supplies device memory and the current stream.

    o, S_T = kda_fwd_chunked(q, k, v, alpha, beta, S0, chunk=64)
    o      = kda_decode_step(q, k, v, alpha, beta, S)   # S updated in place

There is no fallback: if the library is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "KDA_F32", "KDA_BF16", "GATES", "RULES", "KdaError", "lib", "library_path", "exported_symbols",
    "kda_fwd_chunked", "kda_decode_step", "kda_fwd_chunked_raw", "kda_decode_step_raw",
    "kda_fwd_chunked_noalloc_raw",
    "kda_fwd_chunked_fused", "kda_decode_step_fused", "attnres_forward", "attnres_forward_raw",
    "status_string", "version", "workspace_bytes", "set_wait_limit", "wait_limit",
    "set_ring_cap", "ring_cap",
]

KDA_F32 = 0
KDA_BF16 = 1
# kda_gate / kda_rule of include/kda.h
GATES = {"channel": 0, "head": 1, "none": 2}
RULES = {"delta": 0, "linear": 1}
STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED",
          3: "KDA_ERR_WORKSPACE", 4: "KDA_ERR_HIP", 5: "KDA_ERR_CHECK"}
# Every symbol include/kda.h declares.
ABI_SYMBOLS = ("kda_version", "kda_status_string", "kda_fwd_chunked", "kda_fwd_chunked_ex",
               "kda_fwd_chunked_fused", "kda_fwd_chunked_workspace_bytes", "kda_decode_step",
               "kda_decode_step_ex", "kda_decode_step_fused", "attnres_forward",
               "kda_fwd_chunked_noalloc",
               "kda_testing_set_wait_limit", "kda_testing_wait_limit",
               "kda_testing_set_ring_cap", "kda_testing_ring_cap",
               "kda_build_checked", "kda_check_sites", "kda_testing_check_probe")

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")
CHECKED_LIB_PATH = os.path.join(_PKG, "libkda_checked.so")  # bounds-checked debugging build
_LIB_PATH = LIB_PATH
_lib = None


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def select_build(checked: bool = False) -> str:
    """Route every later call through libkda.so (default) or the
    bounds-checked debugging build libkda_checked.so (include/kda.h, "Checked
    build": synchronous, returns KDA_ERR_CHECK if a kernel index leaves its
    buffer).  Returns the library path now in use."""
    global _LIB_PATH, _lib
    path = CHECKED_LIB_PATH if checked else LIB_PATH
    if path != _LIB_PATH:
        _LIB_PATH, _lib = path, None
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libkda.so once.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m gated_delta_rule_76_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.kda_version.argtypes = []
        L.kda_version.restype = i
        L.kda_status_string.argtypes = [i]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_fwd_chunked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i,
                                      vp, sz, vp]
        L.kda_fwd_chunked.restype = i
        L.kda_fwd_chunked_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.kda_fwd_chunked_workspace_bytes.restype = sz
        L.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
        L.kda_decode_step.restype = i
        L.kda_fwd_chunked_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i,
                                         i, i, vp, sz, vp]
        L.kda_fwd_chunked_ex.restype = i
        L.kda_decode_step_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
        L.kda_decode_step_ex.restype = i
        f = ctypes.c_float
        L.kda_fwd_chunked_fused.argtypes = [vp, vp, vp, vp, vp, f, vp, vp, vp, i, i, i, i, i, i,
                                            i, i, i, vp, sz, vp]
        L.kda_fwd_chunked_fused.restype = i
        L.kda_decode_step_fused.argtypes = [vp, vp, vp, vp, vp, f, vp, vp, i, i, i, i, i, i, i, vp]
        L.kda_decode_step_fused.restype = i
        L.attnres_forward.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
        L.attnres_forward.restype = i
        L.kda_fwd_chunked_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i,
                                              i, i, vp]
        L.kda_fwd_chunked_noalloc.restype = i
        L.kda_testing_set_wait_limit.argtypes = [i]
        L.kda_testing_set_wait_limit.restype = i
        L.kda_testing_wait_limit.argtypes = []
        L.kda_testing_wait_limit.restype = i
        L.kda_testing_set_ring_cap.argtypes = [sz]
        L.kda_testing_set_ring_cap.restype = i
        L.kda_testing_ring_cap.argtypes = []
        L.kda_testing_ring_cap.restype = sz
        L.kda_build_checked.argtypes = []
        L.kda_build_checked.restype = i
        L.kda_check_sites.argtypes = []
        L.kda_check_sites.restype = ctypes.c_uint
        L.kda_testing_check_probe.argtypes = [vp]
        L.kda_testing_check_probe.restype = i
        _lib = L
    return _lib


def exported_symbols() -> Tuple[str, ...]:
    L = lib()
    return tuple(s for s in ABI_SYMBOLS if hasattr(L, s))


def version() -> int:
    return int(lib().kda_version())


def set_wait_limit(polls: int) -> int:
    """Test hook (include/kda_testing.h): polls before a prefill output wave
    gives up on a chunk's hand-over and writes NaN for it.  Returns the status."""
    return int(lib().kda_testing_set_wait_limit(int(polls)))


def wait_limit() -> int:
    return int(lib().kda_testing_wait_limit())


def set_ring_cap(nbytes: int) -> int:
    """Test hook (include/kda_testing.h): slot budget of the prefill's segment
    ring in bytes (0 restores the default).  Returns the status."""
    return int(lib().kda_testing_set_ring_cap(int(nbytes)))


def ring_cap() -> int:
    return int(lib().kda_testing_ring_cap())


def build_checked() -> bool:
    """True when the library in use is the bounds-checked build."""
    return bool(lib().kda_build_checked())


def check_sites() -> int:
    """Site mask of the last call that returned KDA_ERR_CHECK (checked build)."""
    return int(lib().kda_check_sites())


def check_probe(stream=None) -> int:
    """Test hook: one bounds check that fails on purpose without touching
    memory; KDA_ERR_CHECK (5) in the checked build, 0 otherwise."""
    return int(lib().kda_testing_check_probe(stream))


def status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


# ---------------------------------------------------------------- raw calls
def kda_fwd_chunked_raw(q, k, v, alpha, beta, S0, o, S_T, B, T, H, d_k, d_v, chunk, dtype,
                        workspace=None, workspace_bytes=0, stream=None, gate=0, rule=0) -> int:
    """Direct C call with integer pointers (0/None for NULL); returns the status."""
    return int(lib().kda_fwd_chunked_ex(q, k, v, alpha, beta, S0, o, S_T, B, T, H, d_k, d_v,
                                        chunk, dtype, gate, rule, workspace, workspace_bytes,
                                        stream))


def kda_fwd_chunked_noalloc_raw(q, k, v, alpha, beta, S0, o, S_T, B, T, H, d_k, d_v, chunk,
                                dtype, gate=0, rule=0, stream=None) -> int:
    """kda_fwd_chunked_noalloc with integer pointers: no workspace argument,
    the library's own device array holds the operand slots."""
    return int(lib().kda_fwd_chunked_noalloc(q, k, v, alpha, beta, S0, o, S_T, B, T, H, d_k, d_v,
                                             chunk, dtype, gate, rule, stream))


def kda_decode_step_raw(q, k, v, alpha, beta, S, o, B, H, d_k, d_v, dtype, stream=None,
                        gate=0, rule=0) -> int:
    return int(lib().kda_decode_step_ex(q, k, v, alpha, beta, S, o, B, H, d_k, d_v, dtype, gate,
                                        rule, stream))


def kda_fwd_chunked_fused_raw(q_raw, k_raw, v, g_raw, b_raw, gate_scale, S0, o, S_T, B, T, H,
                              d_k, d_v, chunk, dtype, gate, rule, workspace=None,
                              workspace_bytes=0, stream=None) -> int:
    return int(lib().kda_fwd_chunked_fused(q_raw, k_raw, v, g_raw, b_raw, float(gate_scale), S0, o,
                                           S_T, B, T, H, d_k, d_v, chunk, dtype, gate, rule,
                                           workspace, workspace_bytes, stream))


def kda_decode_step_fused_raw(q_raw, k_raw, v, g_raw, b_raw, gate_scale, S, o, B, H, d_k, d_v,
                              dtype, gate, rule, stream=None) -> int:
    return int(lib().kda_decode_step_fused(q_raw, k_raw, v, g_raw, b_raw, float(gate_scale), S, o,
                                           B, H, d_k, d_v, dtype, gate, rule, stream))


# ---------------------------------------------------------- torch front end
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"KDA tensors must be bfloat16 or float32, got {t.dtype}")


def _check(t, name, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _variant(gate: str, rule: str):
    if gate not in GATES:
        raise ValueError(f"gate must be one of {sorted(GATES)}, got {gate!r}")
    if rule not in RULES:
        raise ValueError(f"rule must be one of {sorted(RULES)}, got {rule!r}")
    return GATES[gate], RULES[rule]


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def workspace_bytes(B: int, T: int, H: int, d_k: int, d_v: int, chunk: int, dtype: int) -> int:
    return int(lib().kda_fwd_chunked_workspace_bytes(B, T, H, d_k, d_v, chunk, dtype))


def kda_fwd_chunked(q, k, v, alpha, beta, S0=None, *, chunk: int = 64, o=None, S_T=None,
                    return_state: bool = True, workspace=None, gate: str = "channel",
                    rule: str = "delta"):
    """Chunked KDA prefill on the GPU.

    q, k, alpha: [B,T,H,d_k]; v: [B,T,H,d_v]; beta: [B,T,H] (all bf16 or all
    fp32, CUDA/HIP tensors); S0: [B,H,d_k,d_v] fp32 or None.  Returns (o, S_T);
    S_T is None when return_state is False.  ``S_T`` may be S0 (in place).
    ``workspace`` is an optional uint8 device tensor of at least
    workspace_bytes(...) bytes; by default one is taken from torch's caching
    allocator for the call.  ``gate``: "channel" (alpha [B,T,H,d_k], KDA),
    "head" (alpha [B,T,H], Gated DeltaNet) or "none" (alpha ignored, may be
    None).  ``rule``: "delta" (error-correcting write) or "linear" (no
    correction).
    """
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,d_k]")
    B, T, H, d_k = q.shape
    d_v = v.shape[-1]
    dt, dev = q.dtype, q.device
    _dtype_code(q)
    g, r = _variant(gate, rule)
    _check(k, "k", (B, T, H, d_k), dt, dev)
    if g == GATES["channel"]:
        _check(alpha, "alpha", (B, T, H, d_k), dt, dev)
    elif g == GATES["head"]:
        _check(alpha, "alpha", (B, T, H), dt, dev)
    _check(v, "v", (B, T, H, d_v), dt, dev)
    _check(beta, "beta", (B, T, H), dt, dev)
    _check(q, "q", (B, T, H, d_k), dt, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, d_k, d_v), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, d_v), dtype=dt, device=dev)
    else:
        _check(o, "o", (B, T, H, d_v), dt, dev)
    if return_state and S_T is None:
        S_T = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=dev)
    if S_T is not None:
        _check(S_T, "S_T", (B, H, d_k, d_v), torch.float32, dev)
    need = workspace_bytes(B, T, H, d_k, d_v, chunk, _dtype_code(q))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need or workspace.device != dev:
        raise ValueError(f"workspace must hold {need} bytes on {dev}")
    ap = alpha.data_ptr() if (alpha is not None and g != GATES["none"]) else None
    st = kda_fwd_chunked_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), ap,
                             beta.data_ptr(), S0.data_ptr() if S0 is not None else None,
                             o.data_ptr(), S_T.data_ptr() if S_T is not None else None,
                             B, T, H, d_k, d_v, chunk, _dtype_code(q), workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), _stream_handle(dev),
                             g, r)
    if st != 0:
        raise KdaError(st, "kda_fwd_chunked")
    return o, S_T


def kda_decode_step(q, k, v, alpha, beta, S, *, o=None, gate: str = "channel",
                    rule: str = "delta"):
    """One T=1 decode step; S [B,H,d_k,d_v] fp32 is updated in place.  Returns o.
    ``gate``/``rule`` as for kda_fwd_chunked (a "head" gate is alpha [B,H])."""
    torch = _torch()
    if q.dim() != 3:
        raise ValueError("q must be [B,H,d_k]")
    B, H, d_k = q.shape
    d_v = v.shape[-1]
    dt, dev = q.dtype, q.device
    _dtype_code(q)
    g, r = _variant(gate, rule)
    _check(k, "k", (B, H, d_k), dt, dev)
    if g == GATES["channel"]:
        _check(alpha, "alpha", (B, H, d_k), dt, dev)
    elif g == GATES["head"]:
        _check(alpha, "alpha", (B, H), dt, dev)
    _check(v, "v", (B, H, d_v), dt, dev)
    _check(beta, "beta", (B, H), dt, dev)
    _check(S, "S", (B, H, d_k, d_v), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, d_v), dtype=dt, device=dev)
    else:
        _check(o, "o", (B, H, d_v), dt, dev)
    ap = alpha.data_ptr() if (alpha is not None and g != GATES["none"]) else None
    st = kda_decode_step_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), ap,
                             beta.data_ptr(), S.data_ptr(), o.data_ptr(), B, H, d_k, d_v,
                             _dtype_code(q), _stream_handle(dev), g, r)
    if st != 0:
        raise KdaError(st, "kda_decode_step")
    return o


def kda_fwd_chunked_fused(q_raw, k_raw, v, g_raw, b_raw, S0=None, *, gate_scale: float,
                          chunk: int = 64, o=None, S_T=None, return_state: bool = True,
                          workspace=None, gate: str = "channel", rule: str = "delta"):
    """kda_fwd_chunked from raw projections: the kernels L2-normalise q_raw and
    k_raw, map the gate as alpha = exp(-gate_scale * softplus(g_raw)) and beta =
    sigmoid(b_raw).  Shapes as kda_fwd_chunked (g_raw [B,T,H] for gate "head")."""
    torch = _torch()
    if q_raw.dim() != 4:
        raise ValueError("q_raw must be [B,T,H,d_k]")
    B, T, H, d_k = q_raw.shape
    d_v = v.shape[-1]
    dt, dev = q_raw.dtype, q_raw.device
    code = _dtype_code(q_raw)
    g, r = _variant(gate, rule)
    _check(k_raw, "k_raw", (B, T, H, d_k), dt, dev)
    if g == GATES["channel"]:
        _check(g_raw, "g_raw", (B, T, H, d_k), dt, dev)
    elif g == GATES["head"]:
        _check(g_raw, "g_raw", (B, T, H), dt, dev)
    _check(v, "v", (B, T, H, d_v), dt, dev)
    _check(b_raw, "b_raw", (B, T, H), dt, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, d_k, d_v), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, d_v), dtype=dt, device=dev)
    else:
        _check(o, "o", (B, T, H, d_v), dt, dev)
    if return_state and S_T is None:
        S_T = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=dev)
    if S_T is not None:
        _check(S_T, "S_T", (B, H, d_k, d_v), torch.float32, dev)
    need = workspace_bytes(B, T, H, d_k, d_v, chunk, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need or workspace.device != dev:
        raise ValueError(f"workspace must hold {need} bytes on {dev}")
    gp = g_raw.data_ptr() if (g_raw is not None and g != GATES["none"]) else None
    st = kda_fwd_chunked_fused_raw(q_raw.data_ptr(), k_raw.data_ptr(), v.data_ptr(), gp,
                                   b_raw.data_ptr(), gate_scale,
                                   S0.data_ptr() if S0 is not None else None, o.data_ptr(),
                                   S_T.data_ptr() if S_T is not None else None, B, T, H, d_k, d_v,
                                   chunk, code, g, r, workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(),
                                   _stream_handle(dev))
    if st != 0:
        raise KdaError(st, "kda_fwd_chunked_fused")
    return o, S_T


def kda_decode_step_fused(q_raw, k_raw, v, g_raw, b_raw, S, *, gate_scale: float, o=None,
                          gate: str = "channel", rule: str = "delta"):
    """kda_decode_step from raw projections (maps as kda_fwd_chunked_fused).
    S [B,H,d_k,d_v] fp32 is updated in place; returns o."""
    torch = _torch()
    if q_raw.dim() != 3:
        raise ValueError("q_raw must be [B,H,d_k]")
    B, H, d_k = q_raw.shape
    d_v = v.shape[-1]
    dt, dev = q_raw.dtype, q_raw.device
    code = _dtype_code(q_raw)
    g, r = _variant(gate, rule)
    _check(k_raw, "k_raw", (B, H, d_k), dt, dev)
    if g == GATES["channel"]:
        _check(g_raw, "g_raw", (B, H, d_k), dt, dev)
    elif g == GATES["head"]:
        _check(g_raw, "g_raw", (B, H), dt, dev)
    _check(v, "v", (B, H, d_v), dt, dev)
    _check(b_raw, "b_raw", (B, H), dt, dev)
    _check(S, "S", (B, H, d_k, d_v), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, d_v), dtype=dt, device=dev)
    else:
        _check(o, "o", (B, H, d_v), dt, dev)
    gp = g_raw.data_ptr() if (g_raw is not None and g != GATES["none"]) else None
    st = kda_decode_step_fused_raw(q_raw.data_ptr(), k_raw.data_ptr(), v.data_ptr(), gp,
                                   b_raw.data_ptr(), gate_scale, S.data_ptr(), o.data_ptr(), B, H,
                                   d_k, d_v, code, g, r, _stream_handle(dev))
    if st != 0:
        raise KdaError(st, "kda_decode_step_fused")
    return o


def attnres_forward_raw(q, k, h, out, L, N, d_k, d, dtype, stream=None) -> int:
    return int(lib().attnres_forward(q, k, h, out, L, N, d_k, d, dtype, stream))


def attnres_forward(q, k, h, *, out=None):
    """AttnRes depth aggregation: out[n] = sum_i softmax_i(q[n] . k[i, n]) h[i, n].
    q [N,d_k], k [L,N,d_k], h [L,N,d] (bf16 or fp32, one dtype).  Returns out [N,d]."""
    torch = _torch()
    if k.dim() != 3 or h.dim() != 3:
        raise ValueError("k must be [L,N,d_k] and h [L,N,d]")
    L, N, d_k = k.shape
    d = h.shape[-1]
    dt, dev = q.dtype, q.device
    code = _dtype_code(q)
    _check(q, "q", (N, d_k), dt, dev)
    _check(k, "k", (L, N, d_k), dt, dev)
    _check(h, "h", (L, N, d), dt, dev)
    if out is None:
        out = torch.empty((N, d), dtype=dt, device=dev)
    else:
        _check(out, "out", (N, d), dt, dev)
    st = attnres_forward_raw(q.data_ptr(), k.data_ptr(), h.data_ptr(), out.data_ptr(), L, N, d_k, d,
                             code, _stream_handle(dev))
    if st != 0:
        raise KdaError(st, "attnres_forward")
    return out

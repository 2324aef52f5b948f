"""MI355X-native fused GEMM-Residual-RMSNorm-GEMM block, SwiGLU block, the two
chained as an MLP sub-layer, and the LM-head GEMM with cross-entropy.

Thin Python binding over the C-ABI library ``libcoda.so`` (include/coda.h).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensors, allocates outputs and workspaces with torch, and passes
raw device pointers and torch's current HIP stream.  There is no CPU or
PyTorch fallback: without the built library every call raises.

Low-level calls (same names and argument order as the C functions, outputs
preallocated by the caller):
    coda_fwd, coda_fwd_noalloc, coda_bwd, coda_swiglu_fwd, coda_swiglu_bwd, coda_mlp_fwd, coda_mlp_bwd,
    coda_ce_fwd, coda_ce_bwd, coda_rope_fwd, coda_rope_bwd
Convenience calls (allocate outputs):
    fwd(X, W1, R, gamma, W2, eps)        -> (z, y, r)
    bwd(X, W1, gamma, W2, y, r, dz)      -> (dX, dW1, dR, dW2, dgamma)
    swiglu_fwd(X, W, Wd)                 -> (z, gu, a)
    swiglu_bwd(X, W, Wd, gu, a, dz)      -> (dX, dW, dWd)
    mlp_fwd(X, W1, R, gamma, W, Wd, eps) -> (z, y, r, gu, a)
    mlp_bwd(X, W1, gamma, W, Wd, y, r, gu, a, dz, dy_in=None)
                                         -> (dX, dW1, dR, dW, dWd, dgamma)
    ce_fwd(h, Wv, labels)                -> (loss, lse, logits)
    ce_bwd(h, Wv, labels, logits, lse, dloss) -> (dh, dWv)
    rope_fwd(X, W, N_rot, D, S, base)    -> Y
    rope_bwd(X, W, dY, N_rot, D, S, base) -> (dX, dW)
    bwd_mx8(X, W1, gamma, W2, y, r, dz)  -> (dX, dW1, dR, dW2, dgamma), MXFP8 GEMMs
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "CodaError", "lib_path", "load_library", "coda_fwd", "coda_fwd_noalloc", "coda_bwd", "coda_swiglu_fwd",
    "coda_swiglu_bwd", "coda_mlp_fwd", "coda_mlp_bwd", "fwd", "bwd", "swiglu_fwd",
    "swiglu_bwd", "mlp_fwd", "mlp_bwd", "coda_ce_fwd", "coda_ce_bwd", "ce_fwd", "ce_bwd",
    "ce_fwd_workspace_bytes", "ce_bwd_workspace_bytes", "coda_rope_fwd", "coda_rope_bwd", "rope_fwd",
    "rope_bwd", "rope_fwd_workspace_bytes", "rope_bwd_workspace_bytes", "fwd_workspace_bytes", "bwd_workspace_bytes",
    "swiglu_bwd_workspace_bytes", "mlp_fwd_workspace_bytes", "mlp_bwd_workspace_bytes",
    "coda_mx8_quantize", "coda_fwd_mx8", "mx8_quantize", "fwd_mx8", "fwd_mx8_workspace_bytes",
    "coda_bwd_mx8", "bwd_mx8", "bwd_mx8_workspace_bytes", "coda_swiglu_fwd_mx8", "coda_swiglu_bwd_mx8",
    "swiglu_fwd_mx8", "swiglu_bwd_mx8", "swiglu_fwd_mx8_workspace_bytes", "swiglu_bwd_mx8_workspace_bytes",
    "coda_mlp_fwd_mx8", "coda_mlp_bwd_mx8", "mlp_fwd_mx8", "mlp_bwd_mx8", "mlp_fwd_mx8_workspace_bytes",
    "mlp_bwd_mx8_workspace_bytes",
    "mx8_scales_to_rowmajor", "mx8_scales_from_rowmajor",
    "version", "trace_start", "trace_read", "trace_stop",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None

CODA_F32, CODA_BF16 = 0, 1


class CodaError(RuntimeError):
    """A non-zero coda_status from the library."""

    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {msg}")
        self.status = status


def lib_path() -> str:
    return os.path.join(_PKG, "libcoda.so")


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libcoda.so (built in-tree by build.py), or another build of the
    same sources at `path` (the first call decides).  torch is imported first
    so that the library binds to the HIP runtime torch already loaded."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m gemm_epilogue_fusion_gemm1_amd.build`; "
            "there is no fallback implementation")
    import torch  # noqa: F401  (binds libamdhip64 before the library is loaded)
    L = ctypes.CDLL(path)
    i64, sz, vp, f32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    i32 = ctypes.c_int
    L.coda_status_str.restype = ctypes.c_char_p
    L.coda_status_str.argtypes = [i32]
    L.coda_version.restype = ctypes.c_char_p
    L.coda_version.argtypes = []
    for name, args in {
        "coda_fwd_workspace_bytes": [i32, i64, i64, i64, i64],
        "coda_bwd_workspace_bytes": [i32, i64, i64, i64, i64],
        "coda_swiglu_fwd_workspace_bytes": [i32, i64, i64, i64],
        "coda_swiglu_bwd_workspace_bytes": [i32, i64, i64, i64],
        "coda_mlp_fwd_workspace_bytes": [i32, i64, i64, i64, i64],
        "coda_mlp_bwd_workspace_bytes": [i32, i64, i64, i64, i64],
        "coda_ce_fwd_workspace_bytes": [i32, i64, i64, i64],
        "coda_ce_bwd_workspace_bytes": [i32, i64, i64, i64],
        "coda_rope_fwd_workspace_bytes": [i32, i64, i64, i64, i64, i64, i64],
        "coda_rope_bwd_workspace_bytes": [i32, i64, i64, i64, i64, i64, i64],
        "coda_fwd_mx8_workspace_bytes": [i64, i64, i64, i64],
        "coda_bwd_mx8_workspace_bytes": [i64, i64, i64, i64],
        "coda_swiglu_fwd_mx8_workspace_bytes": [i64, i64, i64],
        "coda_swiglu_bwd_mx8_workspace_bytes": [i64, i64, i64],
        "coda_mlp_fwd_mx8_workspace_bytes": [i64, i64, i64, i64],
        "coda_mlp_bwd_mx8_workspace_bytes": [i64, i64, i64, i64],
    }.items():
        getattr(L, name).restype = sz
        getattr(L, name).argtypes = args
    L.coda_fwd.restype = i32
    L.coda_fwd.argtypes = [i32, i64, i64, i64, i64, f32] + [vp] * 8 + [vp, sz, vp]
    L.coda_fwd_noalloc.restype = i32
    L.coda_fwd_noalloc.argtypes = [i32, i64, i64, i64, i64, f32] + [vp] * 8 + [vp]
    L.coda_bwd.restype = i32
    L.coda_bwd.argtypes = [i32, i64, i64, i64, i64] + [vp] * 12 + [vp, sz, vp]
    L.coda_swiglu_fwd.restype = i32
    L.coda_swiglu_fwd.argtypes = [i32, i64, i64, i64] + [vp] * 6 + [vp, sz, vp]
    L.coda_swiglu_bwd.restype = i32
    L.coda_swiglu_bwd.argtypes = [i32, i64, i64, i64] + [vp] * 9 + [vp, sz, vp]
    L.coda_mlp_fwd.restype = i32
    L.coda_mlp_fwd.argtypes = [i32, i64, i64, i64, i64, f32] + [vp] * 11 + [vp, sz, vp]
    L.coda_mlp_bwd.restype = i32
    L.coda_mlp_bwd.argtypes = [i32, i64, i64, i64, i64] + [vp] * 17 + [vp, sz, vp]
    L.coda_ce_fwd.restype = i32
    L.coda_ce_fwd.argtypes = [i32, i64, i64, i64] + [vp] * 6 + [vp, sz, vp]
    L.coda_ce_bwd.restype = i32
    L.coda_ce_bwd.argtypes = [i32, i64, i64, i64] + [vp] * 8 + [vp, sz, vp]
    L.coda_rope_fwd.restype = i32
    L.coda_rope_fwd.argtypes = [i32, i64, i64, i64, i64, i64, i64, f32] + [vp] * 3 + [vp, sz, vp]
    L.coda_rope_bwd.restype = i32
    L.coda_rope_bwd.argtypes = [i32, i64, i64, i64, i64, i64, i64, f32] + [vp] * 5 + [vp, sz, vp]
    L.coda_mx8_quantize.restype = i32
    L.coda_mx8_quantize.argtypes = [i64, i64, vp, i64, vp, vp, vp]
    L.coda_bwd_mx8.restype = i32
    L.coda_bwd_mx8.argtypes = [i64, i64, i64, i64] + [vp] * 12 + [vp, sz, vp]
    L.coda_swiglu_fwd_mx8.restype = i32
    L.coda_swiglu_fwd_mx8.argtypes = [i64, i64, i64] + [vp] * 6 + [vp, sz, vp]
    L.coda_swiglu_bwd_mx8.restype = i32
    L.coda_swiglu_bwd_mx8.argtypes = [i64, i64, i64] + [vp] * 9 + [vp, sz, vp]
    L.coda_mlp_fwd_mx8.restype = i32
    L.coda_mlp_fwd_mx8.argtypes = [i64, i64, i64, i64, f32] + [vp] * 11 + [vp, sz, vp]
    L.coda_mlp_bwd_mx8.restype = i32
    L.coda_mlp_bwd_mx8.argtypes = [i64, i64, i64, i64] + [vp] * 17 + [vp, sz, vp]
    L.coda_fwd_mx8.restype = i32
    L.coda_fwd_mx8.argtypes = [i64, i64, i64, i64, f32] + [vp] * 11 + [vp, sz, vp]
    L.coda_trace_start.restype = i32
    L.coda_trace_start.argtypes = [i32]
    L.coda_trace_count.restype = i32
    L.coda_trace_count.argtypes = []
    L.coda_trace_get.restype = i32
    L.coda_trace_get.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float),
                                 ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    L.coda_trace_stop.restype = i32
    L.coda_trace_stop.argtypes = []
    _LIB = L
    return L


def version() -> str:
    return load_library().coda_version().decode()


# ----------------------------------------------------------------- helpers

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return CODA_BF16
    if t.dtype == torch.float32:
        return CODA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: expected torch.bfloat16 or torch.float32")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("every tensor must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError("every tensor must be contiguous (row-major)")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, status):
    if status != 0:
        msg = load_library().coda_status_str(status).decode()
        raise CodaError(fn, status, msg)


def _shape(t, *dims, name=""):
    if tuple(t.shape) != tuple(dims):
        raise ValueError(f"{name}: expected shape {tuple(dims)}, got {tuple(t.shape)}")


class _Args:
    """Checks every tensor of one call before any pointer is taken: its dtype,
    its exact shape, that it lives on the first tensor's device and is
    contiguous.  The library reads and writes exactly the extents these
    shapes imply, so a tensor of another dtype or a smaller size is refused
    here instead of being reinterpreted or overrun."""

    def __init__(self, fn, first, name):
        if first is None:
            raise ValueError(f"{fn}: {name} is required")
        if not first.is_cuda:
            raise ValueError(f"{fn}: {name} must be a device (HIP) tensor")
        self.fn, self.dev = fn, first.device

    def __call__(self, t, name, shape, dtype, optional=False):
        if t is None:
            if optional:
                return None
            raise ValueError(f"{self.fn}: {name} is required")
        if t.dtype != dtype:
            raise TypeError(f"{self.fn}: {name} must be {dtype}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{self.fn}: {name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if t.device != self.dev:
            raise ValueError(f"{self.fn}: {name} is on {t.device}, expected {self.dev}")
        if not t.is_contiguous():
            raise ValueError(f"{self.fn}: {name} must be contiguous (row-major)")
        return ctypes.c_void_p(t.data_ptr())

    def ws(self, t, name="workspace", optional=False):
        """A workspace: a 1-D uint8 tensor on the device; returns (pointer, bytes)."""
        import torch
        if t is None:
            if optional:
                return None, 0
            raise ValueError(f"{self.fn}: {name} is required")
        if t.dtype != torch.uint8 or t.dim() != 1:
            raise TypeError(f"{self.fn}: {name} must be a 1-D torch.uint8 tensor, got {t.dtype} {tuple(t.shape)}")
        if t.device != self.dev:
            raise ValueError(f"{self.fn}: {name} is on {t.device}, expected {self.dev}")
        if not t.is_contiguous():
            raise ValueError(f"{self.fn}: {name} must be contiguous")
        return ctypes.c_void_p(t.data_ptr()), t.numel()


def _workspace(nbytes, device):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def fwd_workspace_bytes(dtype_code, M, K, d, N) -> int:
    return int(load_library().coda_fwd_workspace_bytes(dtype_code, M, K, d, N))


def bwd_workspace_bytes(dtype_code, M, K, d, N) -> int:
    return int(load_library().coda_bwd_workspace_bytes(dtype_code, M, K, d, N))


def swiglu_bwd_workspace_bytes(dtype_code, M, d, F) -> int:
    return int(load_library().coda_swiglu_bwd_workspace_bytes(dtype_code, M, d, F))


def mlp_fwd_workspace_bytes(dtype_code, M, K, d, F) -> int:
    return int(load_library().coda_mlp_fwd_workspace_bytes(dtype_code, M, K, d, F))


def mlp_bwd_workspace_bytes(dtype_code, M, K, d, F) -> int:
    return int(load_library().coda_mlp_bwd_workspace_bytes(dtype_code, M, K, d, F))


def ce_fwd_workspace_bytes(dtype_code, M, d, V) -> int:
    return int(load_library().coda_ce_fwd_workspace_bytes(dtype_code, M, d, V))


def ce_bwd_workspace_bytes(dtype_code, M, d, V) -> int:
    return int(load_library().coda_ce_bwd_workspace_bytes(dtype_code, M, d, V))


def rope_fwd_workspace_bytes(dtype_code, M, K, N, N_rot, D, S) -> int:
    return int(load_library().coda_rope_fwd_workspace_bytes(dtype_code, M, K, N, N_rot, D, S))


def rope_bwd_workspace_bytes(dtype_code, M, K, N, N_rot, D, S) -> int:
    return int(load_library().coda_rope_bwd_workspace_bytes(dtype_code, M, K, N, N_rot, D, S))


# ------------------------------------------------------------ tracing

def fwd_mx8_workspace_bytes(M, K, d, N) -> int:
    return int(load_library().coda_fwd_mx8_workspace_bytes(M, K, d, N))


def trace_start(capacity: int) -> None:
    """Bracket every kernel launch with HIP events (see coda_trace_start)."""
    _check("coda_trace_start", load_library().coda_trace_start(int(capacity)))


def trace_read():
    """[(kernel name, ms, flops, bytes)] for every launch recorded so far (waits for them)."""
    L = load_library()
    out = []
    name, ms = ctypes.c_char_p(), ctypes.c_float()
    fl, by = ctypes.c_double(), ctypes.c_double()
    for i in range(L.coda_trace_count()):
        _check("coda_trace_get", L.coda_trace_get(i, ctypes.byref(name), ctypes.byref(ms),
                                                  ctypes.byref(fl), ctypes.byref(by)))
        out.append((name.value.decode(), float(ms.value), float(fl.value), float(by.value)))
    return out


def trace_stop() -> None:
    _check("coda_trace_stop", load_library().coda_trace_stop())


# ------------------------------------------------------ C-ABI passthroughs
#
# Same names and argument order as the C functions; outputs are caller-owned
# and are checked like the inputs (dtype, exact shape, device).  Float tensors
# share the dtype of the first argument; r, dgamma, lse, loss and dloss are
# float32, labels int32, workspaces 1-D uint8.

def coda_fwd(X, W1, R, gamma, W2, eps, y, r, z, workspace):
    """coda_fwd with caller-owned outputs y [M,d], r [M] (fp32), z [M,N]."""
    import torch
    a = _Args("coda_fwd", X, "X")
    dt = X.dtype
    _dtype_code(X)
    M, K = X.shape
    d, N = W1.shape[1], W2.shape[1]
    p = [a(X, "X", (M, K), dt), a(W1, "W1", (K, d), dt), a(R, "R", (M, d), dt), a(gamma, "gamma", (d,), dt),
         a(W2, "W2", (d, N), dt), a(y, "y", (M, d), dt), a(r, "r", (M,), torch.float32),
         a(z, "z", (M, N), dt)]
    wp, wn = a.ws(workspace)
    _check("coda_fwd", load_library().coda_fwd(_dtype_code(X), M, K, d, N, float(eps), *p, wp, wn, _stream()))


def coda_fwd_noalloc(X, W1, R, gamma, W2, eps, y, r, z):
    """coda_fwd without a workspace: the library's built-in device scratch
    (80 MiB per device) holds the intermediates, so the call allocates
    nothing.  Calls that overlap on one device race on that scratch."""
    import torch
    a = _Args("coda_fwd_noalloc", X, "X")
    dt = X.dtype
    _dtype_code(X)
    M, K = X.shape
    d, N = W1.shape[1], W2.shape[1]
    p = [a(X, "X", (M, K), dt), a(W1, "W1", (K, d), dt), a(R, "R", (M, d), dt), a(gamma, "gamma", (d,), dt),
         a(W2, "W2", (d, N), dt), a(y, "y", (M, d), dt), a(r, "r", (M,), torch.float32),
         a(z, "z", (M, N), dt)]
    _check("coda_fwd_noalloc", load_library().coda_fwd_noalloc(_dtype_code(X), M, K, d, N, float(eps), *p,
                                                                _stream()))


def coda_bwd(X, W1, gamma, W2, y, r, dz, dX, dW1, dR, dW2, dgamma, workspace):
    import torch
    a = _Args("coda_bwd", X, "X")
    dt = X.dtype
    _dtype_code(X)
    M, K = X.shape
    d, N = W1.shape[1], W2.shape[1]
    p = [a(X, "X", (M, K), dt), a(W1, "W1", (K, d), dt), a(gamma, "gamma", (d,), dt), a(W2, "W2", (d, N), dt),
         a(y, "y", (M, d), dt), a(r, "r", (M,), torch.float32), a(dz, "dz", (M, N), dt),
         a(dX, "dX", (M, K), dt), a(dW1, "dW1", (K, d), dt), a(dR, "dR", (M, d), dt),
         a(dW2, "dW2", (d, N), dt), a(dgamma, "dgamma", (d,), torch.float32)]
    wp, wn = a.ws(workspace)
    _check("coda_bwd", load_library().coda_bwd(_dtype_code(X), M, K, d, N, *p, wp, wn, _stream()))


def coda_swiglu_fwd(X, W, Wd, gu, a, z, workspace=None):
    c = _Args("coda_swiglu_fwd", X, "X")
    dt = X.dtype
    _dtype_code(X)
    M, d = X.shape
    F = Wd.shape[0]
    p = [c(X, "X", (M, d), dt), c(W, "W", (d, 2 * F), dt), c(Wd, "Wd", (F, d), dt),
         c(gu, "gu", (M, 2 * F), dt), c(a, "a", (M, F), dt), c(z, "z", (M, d), dt)]
    wp, wn = c.ws(workspace, optional=True)
    _check("coda_swiglu_fwd", load_library().coda_swiglu_fwd(_dtype_code(X), M, d, F, *p, wp, wn, _stream()))


def coda_swiglu_bwd(X, W, Wd, gu, a, dz, dX, dW, dWd, workspace):
    c = _Args("coda_swiglu_bwd", X, "X")
    dt = X.dtype
    _dtype_code(X)
    M, d = X.shape
    F = Wd.shape[0]
    p = [c(X, "X", (M, d), dt), c(W, "W", (d, 2 * F), dt), c(Wd, "Wd", (F, d), dt),
         c(gu, "gu", (M, 2 * F), dt), c(a, "a", (M, F), dt), c(dz, "dz", (M, d), dt),
         c(dX, "dX", (M, d), dt), c(dW, "dW", (d, 2 * F), dt), c(dWd, "dWd", (F, d), dt)]
    wp, wn = c.ws(workspace)
    _check("coda_swiglu_bwd", load_library().coda_swiglu_bwd(_dtype_code(X), M, d, F, *p, wp, wn, _stream()))


def coda_mlp_fwd(X, W1, R, gamma, W, Wd, eps, y, r, gu, a, z, workspace):
    import torch
    c = _Args("coda_mlp_fwd", X, "X")
    dt = X.dtype
    _dtype_code(X)
    M, K = X.shape
    d = W1.shape[1]
    F = Wd.shape[0]
    p = [c(X, "X", (M, K), dt), c(W1, "W1", (K, d), dt), c(R, "R", (M, d), dt), c(gamma, "gamma", (d,), dt),
         c(W, "W", (d, 2 * F), dt), c(Wd, "Wd", (F, d), dt), c(y, "y", (M, d), dt),
         c(r, "r", (M,), torch.float32), c(gu, "gu", (M, 2 * F), dt), c(a, "a", (M, F), dt),
         c(z, "z", (M, d), dt)]
    wp, wn = c.ws(workspace)
    _check("coda_mlp_fwd", load_library().coda_mlp_fwd(_dtype_code(X), M, K, d, F, float(eps), *p, wp, wn,
                                                        _stream()))


def coda_mlp_bwd(X, W1, gamma, W, Wd, y, r, gu, a, dz, dy_in, dX, dW1, dR, dW, dWd, dgamma,
                 workspace):
    import torch
    c = _Args("coda_mlp_bwd", X, "X")
    dt = X.dtype
    _dtype_code(X)
    M, K = X.shape
    d = W1.shape[1]
    F = Wd.shape[0]
    p = [c(X, "X", (M, K), dt), c(W1, "W1", (K, d), dt), c(gamma, "gamma", (d,), dt),
         c(W, "W", (d, 2 * F), dt), c(Wd, "Wd", (F, d), dt), c(y, "y", (M, d), dt),
         c(r, "r", (M,), torch.float32), c(gu, "gu", (M, 2 * F), dt), c(a, "a", (M, F), dt),
         c(dz, "dz", (M, d), dt), c(dy_in, "dy_in", (M, d), dt, optional=True),
         c(dX, "dX", (M, K), dt), c(dW1, "dW1", (K, d), dt), c(dR, "dR", (M, d), dt),
         c(dW, "dW", (d, 2 * F), dt), c(dWd, "dWd", (F, d), dt), c(dgamma, "dgamma", (d,), torch.float32)]
    wp, wn = c.ws(workspace)
    _check("coda_mlp_bwd", load_library().coda_mlp_bwd(_dtype_code(X), M, K, d, F, *p, wp, wn, _stream()))


def coda_ce_fwd(h, Wv, labels, logits, lse, loss, workspace):
    import torch
    c = _Args("coda_ce_fwd", h, "h")
    dt = h.dtype
    _dtype_code(h)
    M, d = h.shape
    V = Wv.shape[1]
    p = [c(h, "h", (M, d), dt), c(Wv, "Wv", (d, V), dt), c(labels, "labels", (M,), torch.int32),
         c(logits, "logits", (M, V), dt), c(lse, "lse", (M,), torch.float32), c(loss, "loss", (M,), torch.float32)]
    wp, wn = c.ws(workspace)
    _check("coda_ce_fwd", load_library().coda_ce_fwd(_dtype_code(h), M, d, V, *p, wp, wn, _stream()))


def coda_ce_bwd(h, Wv, labels, logits, lse, dloss, dh, dWv, workspace):
    import torch
    c = _Args("coda_ce_bwd", h, "h")
    dt = h.dtype
    _dtype_code(h)
    M, d = h.shape
    V = Wv.shape[1]
    p = [c(h, "h", (M, d), dt), c(Wv, "Wv", (d, V), dt), c(labels, "labels", (M,), torch.int32),
         c(logits, "logits", (M, V), dt), c(lse, "lse", (M,), torch.float32),
         c(dloss, "dloss", (M,), torch.float32), c(dh, "dh", (M, d), dt), c(dWv, "dWv", (d, V), dt)]
    wp, wn = c.ws(workspace)
    _check("coda_ce_bwd", load_library().coda_ce_bwd(_dtype_code(h), M, d, V, *p, wp, wn, _stream()))


def coda_rope_fwd(X, W, N_rot, D, S, base, Y, workspace):
    c = _Args("coda_rope_fwd", X, "X")
    dt = X.dtype
    _dtype_code(X)
    M, K = X.shape
    N = W.shape[1]
    p = [c(X, "X", (M, K), dt), c(W, "W", (K, N), dt), c(Y, "Y", (M, N), dt)]
    wp, wn = c.ws(workspace)
    _check("coda_rope_fwd", load_library().coda_rope_fwd(_dtype_code(X), M, K, N, N_rot, D, S, float(base),
                                                          *p, wp, wn, _stream()))


def coda_rope_bwd(X, W, dY, N_rot, D, S, base, dX, dW, workspace):
    c = _Args("coda_rope_bwd", X, "X")
    dt = X.dtype
    _dtype_code(X)
    M, K = X.shape
    N = W.shape[1]
    p = [c(X, "X", (M, K), dt), c(W, "W", (K, N), dt), c(dY, "dY", (M, N), dt), c(dX, "dX", (M, K), dt),
         c(dW, "dW", (K, N), dt)]
    wp, wn = c.ws(workspace)
    _check("coda_rope_bwd", load_library().coda_rope_bwd(_dtype_code(X), M, K, N, N_rot, D, S, float(base),
                                                          *p, wp, wn, _stream()))


def coda_mx8_quantize(src, codes, scales):
    """MXFP8 quantisation of the bf16 rows of src [rows, cols] into codes
    [rows, cols] and step-blocked scales [cols/128, rows, 4] (uint8)."""
    import torch
    c = _Args("coda_mx8_quantize", src, "src")
    rows, cols = src.shape
    p = [c(src, "src", (rows, cols), torch.bfloat16), c(codes, "codes", (rows, cols), torch.uint8),
         c(scales, "scales", (cols // 128, rows, 4), torch.uint8)]
    _check("coda_mx8_quantize", load_library().coda_mx8_quantize(rows, cols, p[0], cols, p[1], p[2], _stream()))


def coda_fwd_mx8(Xq, Xs, W1tq, W1ts, R, gamma, W2tq, W2ts, eps, y, r, z, workspace):
    """coda_fwd_mx8 with caller-owned outputs y [M,d] (bf16), r [M] (fp32), z [M,N] (bf16)."""
    import torch
    c = _Args("coda_fwd_mx8", Xq, "Xq")
    u8, bf = torch.uint8, torch.bfloat16
    M, K = Xq.shape
    d, N = W1tq.shape[0], W2tq.shape[0]
    p = [c(Xq, "Xq", (M, K), u8), c(Xs, "Xs", (K // 128, M, 4), u8), c(W1tq, "W1tq", (d, K), u8),
         c(W1ts, "W1ts", (K // 128, d, 4), u8), c(R, "R", (M, d), bf), c(gamma, "gamma", (d,), bf),
         c(W2tq, "W2tq", (N, d), u8), c(W2ts, "W2ts", (d // 128, N, 4), u8), c(y, "y", (M, d), bf),
         c(r, "r", (M,), torch.float32), c(z, "z", (M, N), bf)]
    wp, wn = c.ws(workspace)
    _check("coda_fwd_mx8", load_library().coda_fwd_mx8(M, K, d, N, float(eps), *p, wp, wn, _stream()))


def coda_bwd_mx8(X, W1, gamma, W2, y, r, dz, dX, dW1, dR, dW2, dgamma, workspace):
    """coda_bwd_mx8: the block backward on MXFP8 GEMM operands (bf16 tensors in
    and out, as coda_bwd)."""
    import torch
    a = _Args("coda_bwd_mx8", X, "X")
    bf = torch.bfloat16
    M, K = X.shape
    d, N = W1.shape[1], W2.shape[1]
    p = [a(X, "X", (M, K), bf), a(W1, "W1", (K, d), bf), a(gamma, "gamma", (d,), bf), a(W2, "W2", (d, N), bf),
         a(y, "y", (M, d), bf), a(r, "r", (M,), torch.float32), a(dz, "dz", (M, N), bf),
         a(dX, "dX", (M, K), bf), a(dW1, "dW1", (K, d), bf), a(dR, "dR", (M, d), bf),
         a(dW2, "dW2", (d, N), bf), a(dgamma, "dgamma", (d,), torch.float32)]
    wp, wn = a.ws(workspace)
    _check("coda_bwd_mx8", load_library().coda_bwd_mx8(M, K, d, N, *p, wp, wn, _stream()))


def coda_swiglu_fwd_mx8(X, W, Wd, gu, a, z, workspace):
    """coda_swiglu_fwd_mx8: the SwiGLU block forward on MXFP8 GEMM operands
    (bf16 tensors in and out, as coda_swiglu_fwd)."""
    import torch
    c = _Args("coda_swiglu_fwd_mx8", X, "X")
    bf = torch.bfloat16
    M, d = X.shape
    F = Wd.shape[0]
    p = [c(X, "X", (M, d), bf), c(W, "W", (d, 2 * F), bf), c(Wd, "Wd", (F, d), bf),
         c(gu, "gu", (M, 2 * F), bf), c(a, "a", (M, F), bf), c(z, "z", (M, d), bf)]
    wp, wn = c.ws(workspace)
    _check("coda_swiglu_fwd_mx8", load_library().coda_swiglu_fwd_mx8(M, d, F, *p, wp, wn, _stream()))


def coda_swiglu_bwd_mx8(X, W, Wd, gu, a, dz, dX, dW, dWd, workspace):
    """coda_swiglu_bwd_mx8: the SwiGLU block backward on MXFP8 GEMM operands
    (bf16 tensors in and out, as coda_swiglu_bwd)."""
    import torch
    c = _Args("coda_swiglu_bwd_mx8", X, "X")
    bf = torch.bfloat16
    M, d = X.shape
    F = Wd.shape[0]
    p = [c(X, "X", (M, d), bf), c(W, "W", (d, 2 * F), bf), c(Wd, "Wd", (F, d), bf),
         c(gu, "gu", (M, 2 * F), bf), c(a, "a", (M, F), bf), c(dz, "dz", (M, d), bf),
         c(dX, "dX", (M, d), bf), c(dW, "dW", (d, 2 * F), bf), c(dWd, "dWd", (F, d), bf)]
    wp, wn = c.ws(workspace)
    _check("coda_swiglu_bwd_mx8", load_library().coda_swiglu_bwd_mx8(M, d, F, *p, wp, wn, _stream()))


def coda_mlp_fwd_mx8(X, W1, R, gamma, W, Wd, eps, y, r, gu, a, z, workspace):
    """coda_mlp_fwd_mx8: the MLP sub-layer forward on MXFP8 GEMM operands
    (bf16 tensors in and out, r float32, as coda_mlp_fwd)."""
    import torch
    c = _Args("coda_mlp_fwd_mx8", X, "X")
    bf = torch.bfloat16
    M, K = X.shape
    d = W1.shape[1]
    F = Wd.shape[0]
    p = [c(X, "X", (M, K), bf), c(W1, "W1", (K, d), bf), c(R, "R", (M, d), bf), c(gamma, "gamma", (d,), bf),
         c(W, "W", (d, 2 * F), bf), c(Wd, "Wd", (F, d), bf), c(y, "y", (M, d), bf),
         c(r, "r", (M,), torch.float32), c(gu, "gu", (M, 2 * F), bf), c(a, "a", (M, F), bf), c(z, "z", (M, d), bf)]
    wp, wn = c.ws(workspace)
    _check("coda_mlp_fwd_mx8", load_library().coda_mlp_fwd_mx8(M, K, d, F, float(eps), *p, wp, wn, _stream()))


def coda_mlp_bwd_mx8(X, W1, gamma, W, Wd, y, r, gu, a, dz, dy_in, dX, dW1, dR, dW, dWd, dgamma, workspace):
    """coda_mlp_bwd_mx8: the MLP sub-layer backward on MXFP8 GEMM operands
    (dy_in may be None)."""
    import torch
    c = _Args("coda_mlp_bwd_mx8", X, "X")
    bf = torch.bfloat16
    M, K = X.shape
    d = W1.shape[1]
    F = Wd.shape[0]
    p = [c(X, "X", (M, K), bf), c(W1, "W1", (K, d), bf), c(gamma, "gamma", (d,), bf),
         c(W, "W", (d, 2 * F), bf), c(Wd, "Wd", (F, d), bf), c(y, "y", (M, d), bf),
         c(r, "r", (M,), torch.float32), c(gu, "gu", (M, 2 * F), bf), c(a, "a", (M, F), bf),
         c(dz, "dz", (M, d), bf), c(dy_in, "dy_in", (M, d), bf, optional=True), c(dX, "dX", (M, K), bf),
         c(dW1, "dW1", (K, d), bf), c(dR, "dR", (M, d), bf), c(dW, "dW", (d, 2 * F), bf),
         c(dWd, "dWd", (F, d), bf), c(dgamma, "dgamma", (d,), torch.float32)]
    wp, wn = c.ws(workspace)
    _check("coda_mlp_bwd_mx8", load_library().coda_mlp_bwd_mx8(M, K, d, F, *p, wp, wn, _stream()))


# ------------------------------------------------------ convenience calls

def mx8_scales_to_rowmajor(scales):
    """Step-blocked scales [cols/128, rows, 4] as the row-major [rows, cols/32]
    (a view permutation, made contiguous)."""
    t, rows, _ = scales.shape
    return scales.permute(1, 0, 2).reshape(rows, 4 * t).contiguous()


def mx8_scales_from_rowmajor(scales):
    """Row-major scales [rows, cols/32] in the step-blocked layout [cols/128, rows, 4]."""
    rows, nb = scales.shape
    return scales.reshape(rows, nb // 4, 4).permute(1, 0, 2).contiguous()


def mx8_quantize(src):
    """MXFP8 codes [rows, cols] and step-blocked scales [cols/128, rows, 4]
    (uint8 tensors) of the bf16 rows of src."""
    import torch
    rows, cols = src.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=src.device)
    scales = torch.empty((cols // 128, rows, 4), dtype=torch.uint8, device=src.device)
    coda_mx8_quantize(src, codes, scales)
    return codes, scales


def fwd_mx8(Xq, Xs, W1tq, W1ts, R, gamma, W2tq, W2ts, eps):
    """The fused block forward on MXFP8 operands (weights stored [out, in]).
    Returns (z, y, r)."""
    import torch
    M, K = Xq.shape
    d, N = W1tq.shape[0], W2tq.shape[0]
    _shape(Xs, K // 128, M, 4, name="Xs"); _shape(W1tq, d, K, name="W1tq")
    _shape(W1ts, K // 128, d, 4, name="W1ts")
    _shape(W2tq, N, d, name="W2tq"); _shape(W2ts, d // 128, N, 4, name="W2ts")
    _shape(R, M, d, name="R"); _shape(gamma, d, name="gamma")
    y = torch.empty((M, d), dtype=torch.bfloat16, device=R.device)
    r = torch.empty((M,), dtype=torch.float32, device=R.device)
    z = torch.empty((M, N), dtype=torch.bfloat16, device=R.device)
    ws = _workspace(fwd_mx8_workspace_bytes(M, K, d, N), R.device)
    coda_fwd_mx8(Xq, Xs, W1tq, W1ts, R, gamma, W2tq, W2ts, eps, y, r, z, ws)
    return z, y, r


def bwd_mx8_workspace_bytes(M, K, d, N) -> int:
    return int(load_library().coda_bwd_mx8_workspace_bytes(M, K, d, N))


def bwd_mx8(X, W1, gamma, W2, y, r, dz):
    """The block backward with every GEMM on MXFP8 operands (bf16 in and out).
    Returns (dX, dW1, dR, dW2, dgamma)."""
    import torch
    M, K = X.shape
    d, N = W1.shape[1], W2.shape[1]
    dX = torch.empty_like(X)
    dW1 = torch.empty_like(W1)
    dR = torch.empty((M, d), dtype=X.dtype, device=X.device)
    dW2 = torch.empty_like(W2)
    dgamma = torch.empty((d,), dtype=torch.float32, device=X.device)
    ws = _workspace(bwd_mx8_workspace_bytes(M, K, d, N), X.device)
    coda_bwd_mx8(X, W1, gamma, W2, y, r, dz, dX, dW1, dR, dW2, dgamma, ws)
    return dX, dW1, dR, dW2, dgamma


def swiglu_fwd_mx8_workspace_bytes(M, d, F) -> int:
    return int(load_library().coda_swiglu_fwd_mx8_workspace_bytes(M, d, F))


def swiglu_bwd_mx8_workspace_bytes(M, d, F) -> int:
    return int(load_library().coda_swiglu_bwd_mx8_workspace_bytes(M, d, F))


def swiglu_fwd_mx8(X, W, Wd):
    """The SwiGLU block forward with both GEMMs on MXFP8 operands (bf16 in and
    out).  Returns (z, gu, a)."""
    import torch
    M, d = X.shape
    F = Wd.shape[0]
    gu = torch.empty((M, 2 * F), dtype=X.dtype, device=X.device)
    a = torch.empty((M, F), dtype=X.dtype, device=X.device)
    z = torch.empty((M, d), dtype=X.dtype, device=X.device)
    ws = _workspace(swiglu_fwd_mx8_workspace_bytes(M, d, F), X.device)
    coda_swiglu_fwd_mx8(X, W, Wd, gu, a, z, ws)
    return z, gu, a


def swiglu_bwd_mx8(X, W, Wd, gu, a, dz):
    """The SwiGLU block backward with every GEMM on MXFP8 operands.  Returns
    (dX, dW, dWd)."""
    import torch
    M, d = X.shape
    F = Wd.shape[0]
    dX = torch.empty_like(X)
    dW = torch.empty((d, 2 * F), dtype=X.dtype, device=X.device)
    dWd = torch.empty((F, d), dtype=X.dtype, device=X.device)
    ws = _workspace(swiglu_bwd_mx8_workspace_bytes(M, d, F), X.device)
    coda_swiglu_bwd_mx8(X, W, Wd, gu, a, dz, dX, dW, dWd, ws)
    return dX, dW, dWd


def mlp_fwd_mx8_workspace_bytes(M, K, d, F) -> int:
    return int(load_library().coda_mlp_fwd_mx8_workspace_bytes(M, K, d, F))


def mlp_bwd_mx8_workspace_bytes(M, K, d, F) -> int:
    return int(load_library().coda_mlp_bwd_mx8_workspace_bytes(M, K, d, F))


def mlp_fwd_mx8(X, W1, R, gamma, W, Wd, eps):
    """The MLP sub-layer forward with its GEMMs on MXFP8 operands.  Returns
    (z, y, r, gu, a)."""
    import torch
    M, K = X.shape
    d = W1.shape[1]
    F = Wd.shape[0]
    y = torch.empty((M, d), dtype=X.dtype, device=X.device)
    r = torch.empty((M,), dtype=torch.float32, device=X.device)
    gu = torch.empty((M, 2 * F), dtype=X.dtype, device=X.device)
    a = torch.empty((M, F), dtype=X.dtype, device=X.device)
    z = torch.empty((M, d), dtype=X.dtype, device=X.device)
    ws = _workspace(mlp_fwd_mx8_workspace_bytes(M, K, d, F), X.device)
    coda_mlp_fwd_mx8(X, W1, R, gamma, W, Wd, eps, y, r, gu, a, z, ws)
    return z, y, r, gu, a


def mlp_bwd_mx8(X, W1, gamma, W, Wd, y, r, gu, a, dz, dy_in=None):
    """The MLP sub-layer backward with its GEMMs on MXFP8 operands.  Returns
    (dX, dW1, dR, dW, dWd, dgamma)."""
    import torch
    M, K = X.shape
    d = W1.shape[1]
    F = Wd.shape[0]
    dX = torch.empty_like(X)
    dW1 = torch.empty_like(W1)
    dR = torch.empty((M, d), dtype=X.dtype, device=X.device)
    dW = torch.empty_like(W)
    dWd = torch.empty_like(Wd)
    dgamma = torch.empty((d,), dtype=torch.float32, device=X.device)
    ws = _workspace(mlp_bwd_mx8_workspace_bytes(M, K, d, F), X.device)
    coda_mlp_bwd_mx8(X, W1, gamma, W, Wd, y, r, gu, a, dz, dy_in, dX, dW1, dR, dW, dWd, dgamma, ws)
    return dX, dW1, dR, dW, dWd, dgamma


def fwd(X, W1, R, gamma, W2, eps):
    """z = RMSNorm(X W1 + R) * gamma @ W2, fused.  Returns (z, y, r)."""
    import torch
    M, K = X.shape
    d, N = W1.shape[1], W2.shape[1]
    _shape(W1, K, d, name="W1"); _shape(R, M, d, name="R")
    _shape(gamma, d, name="gamma"); _shape(W2, d, N, name="W2")
    y = torch.empty((M, d), dtype=X.dtype, device=X.device)
    r = torch.empty((M,), dtype=torch.float32, device=X.device)
    z = torch.empty((M, N), dtype=X.dtype, device=X.device)
    ws = _workspace(fwd_workspace_bytes(_dtype_code(X), M, K, d, N), X.device)
    coda_fwd(X, W1, R, gamma, W2, eps, y, r, z, ws)
    return z, y, r


def bwd(X, W1, gamma, W2, y, r, dz):
    """Gradients of <dz, z> from the saved (y, r).  Returns (dX, dW1, dR, dW2, dgamma)."""
    import torch
    M, K = X.shape
    d, N = W1.shape[1], W2.shape[1]
    _shape(y, M, d, name="y"); _shape(r, M, name="r"); _shape(dz, M, N, name="dz")
    dX = torch.empty_like(X)
    dW1 = torch.empty_like(W1)
    dR = torch.empty((M, d), dtype=X.dtype, device=X.device)
    dW2 = torch.empty_like(W2)
    dgamma = torch.empty((d,), dtype=torch.float32, device=X.device)
    ws = _workspace(bwd_workspace_bytes(_dtype_code(X), M, K, d, N), X.device)
    coda_bwd(X, W1, gamma, W2, y, r, dz, dX, dW1, dR, dW2, dgamma, ws)
    return dX, dW1, dR, dW2, dgamma


def swiglu_fwd(X, W, Wd):
    """z = (silu(X W_gate) * (X W_up)) @ Wd, fused.  Returns (z, gu, a)."""
    import torch
    M, d = X.shape
    F = Wd.shape[0]
    _shape(W, d, 2 * F, name="W"); _shape(Wd, F, d, name="Wd")
    gu = torch.empty((M, 2 * F), dtype=X.dtype, device=X.device)
    a = torch.empty((M, F), dtype=X.dtype, device=X.device)
    z = torch.empty((M, d), dtype=X.dtype, device=X.device)
    coda_swiglu_fwd(X, W, Wd, gu, a, z)
    return z, gu, a


def swiglu_bwd(X, W, Wd, gu, a, dz):
    """Gradients of <dz, z> from the saved (gu, a).  Returns (dX, dW, dWd)."""
    import torch
    M, d = X.shape
    F = Wd.shape[0]
    _shape(gu, M, 2 * F, name="gu"); _shape(a, M, F, name="a"); _shape(dz, M, d, name="dz")
    dX = torch.empty_like(X)
    dW = torch.empty_like(W)
    dWd = torch.empty_like(Wd)
    ws = _workspace(swiglu_bwd_workspace_bytes(_dtype_code(X), M, d, F), X.device)
    coda_swiglu_bwd(X, W, Wd, gu, a, dz, dX, dW, dWd, ws)
    return dX, dW, dWd


def mlp_fwd(X, W1, R, gamma, W, Wd, eps):
    """The MLP sub-layer: z = silu(g) u Wd with [g | u] = RMSNorm(X W1 + R) * gamma @ W,
    fused.  Returns (z, y, r, gu, a)."""
    import torch
    M, K = X.shape
    d = W1.shape[1]
    F = Wd.shape[0]
    _shape(W1, K, d, name="W1"); _shape(R, M, d, name="R"); _shape(gamma, d, name="gamma")
    _shape(W, d, 2 * F, name="W"); _shape(Wd, F, d, name="Wd")
    y = torch.empty((M, d), dtype=X.dtype, device=X.device)
    r = torch.empty((M,), dtype=torch.float32, device=X.device)
    gu = torch.empty((M, 2 * F), dtype=X.dtype, device=X.device)
    a = torch.empty((M, F), dtype=X.dtype, device=X.device)
    z = torch.empty((M, d), dtype=X.dtype, device=X.device)
    ws = _workspace(mlp_fwd_workspace_bytes(_dtype_code(X), M, K, d, F), X.device)
    coda_mlp_fwd(X, W1, R, gamma, W, Wd, eps, y, r, gu, a, z, ws)
    return z, y, r, gu, a


def mlp_bwd(X, W1, gamma, W, Wd, y, r, gu, a, dz, dy_in=None):
    """Gradients of <dz, z> + <dy_in, y> from the saved (y, r, gu, a).
    Returns (dX, dW1, dR, dW, dWd, dgamma)."""
    import torch
    M, K = X.shape
    d = W1.shape[1]
    F = Wd.shape[0]
    _shape(y, M, d, name="y"); _shape(r, M, name="r"); _shape(gu, M, 2 * F, name="gu")
    _shape(a, M, F, name="a"); _shape(dz, M, d, name="dz")
    if dy_in is not None:
        _shape(dy_in, M, d, name="dy_in")
    dX = torch.empty_like(X)
    dW1 = torch.empty_like(W1)
    dR = torch.empty((M, d), dtype=X.dtype, device=X.device)
    dW = torch.empty_like(W)
    dWd = torch.empty_like(Wd)
    dgamma = torch.empty((d,), dtype=torch.float32, device=X.device)
    ws = _workspace(mlp_bwd_workspace_bytes(_dtype_code(X), M, K, d, F), X.device)
    coda_mlp_bwd(X, W1, gamma, W, Wd, y, r, gu, a, dz, dy_in, dX, dW1, dR, dW, dWd, dgamma, ws)
    return dX, dW1, dR, dW, dWd, dgamma


def ce_fwd(h, Wv, labels):
    """Per-row cross-entropy of the logits h Wv against labels (int32).
    Returns (loss, lse, logits); lse and logits are saved for the backward."""
    import torch
    M, d = h.shape
    V = Wv.shape[1]
    _shape(Wv, d, V, name="Wv"); _shape(labels, M, name="labels")
    logits = torch.empty((M, V), dtype=h.dtype, device=h.device)
    lse = torch.empty((M,), dtype=torch.float32, device=h.device)
    loss = torch.empty((M,), dtype=torch.float32, device=h.device)
    ws = _workspace(ce_fwd_workspace_bytes(_dtype_code(h), M, d, V), h.device)
    coda_ce_fwd(h, Wv, labels, logits, lse, loss, ws)
    return loss, lse, logits


def ce_bwd(h, Wv, labels, logits, lse, dloss):
    """Gradients of sum_i dloss_i loss_i.  Returns (dh, dWv)."""
    import torch
    M, d = h.shape
    V = Wv.shape[1]
    _shape(logits, M, V, name="logits"); _shape(lse, M, name="lse"); _shape(dloss, M, name="dloss")
    dh = torch.empty_like(h)
    dWv = torch.empty_like(Wv)
    ws = _workspace(ce_bwd_workspace_bytes(_dtype_code(h), M, d, V), h.device)
    coda_ce_bwd(h, Wv, labels, logits, lse, dloss, dh, dWv, ws)
    return dh, dWv


def rope_fwd(X, W, N_rot, D, S, base=10000.0):
    """Y = X W with rotary positions on the first N_rot columns (interleaved
    pairs per D-wide head, position = row mod S)."""
    import torch
    M, K = X.shape
    N = W.shape[1]
    _shape(W, K, N, name="W")
    Y = torch.empty((M, N), dtype=X.dtype, device=X.device)
    ws = _workspace(rope_fwd_workspace_bytes(_dtype_code(X), M, K, N, N_rot, D, S), X.device)
    coda_rope_fwd(X, W, N_rot, D, S, base, Y, ws)
    return Y


def rope_bwd(X, W, dY, N_rot, D, S, base=10000.0):
    """Gradients of <dY, Y>.  Returns (dX, dW)."""
    import torch
    M, K = X.shape
    N = W.shape[1]
    _shape(dY, M, N, name="dY")
    dX = torch.empty_like(X)
    dW = torch.empty_like(W)
    ws = _workspace(rope_bwd_workspace_bytes(_dtype_code(X), M, K, N, N_rot, D, S), X.device)
    coda_rope_bwd(X, W, dY, N_rot, D, S, base, dX, dW, ws)
    return dX, dW

"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects bad arguments with the documented status before any HIP
call (so no GPU is needed; the pointers below are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coda.h")

OK, NULL, SHAPE, ALIGN, ALIAS, DTYPE, EPS, WORKSPACE, UNSUPPORTED, HIP = range(10)
F32, BF16 = 0, 1


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(coda_[a-z_0-9]+)\s*\(", src)))


def _lib_under_test():
    """libcoda.so, or the build named by CODA_ABI_TEST_LIB (the sanitized
    copy that test_abi_asan.py runs this file against)."""
    from gemm_epilogue_fusion_gemm1_amd import lib_path
    return os.environ.get("CODA_ABI_TEST_LIB") or lib_path()


@pytest.fixture(scope="module")
def L():
    from gemm_epilogue_fusion_gemm1_amd import lib_path, load_library
    if not os.path.exists(_lib_under_test()) and _lib_under_test() == lib_path():
        import __graft_entry__
        __graft_entry__.build()
    return load_library(_lib_under_test())


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("coda_fwd", "coda_bwd", "coda_swiglu_fwd", "coda_swiglu_bwd"):
        assert fn in names


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib_under_test()], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (coda_[a-z_0-9]+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for f in declared_functions():
        assert hasattr(L, f)


def test_status_strings_and_version(L):
    for s in range(10):
        assert L.coda_status_str(s).decode().startswith("CODA_")
    assert b"gfx950" in L.coda_version()


def test_workspace_sizes(L):
    M, K, d, N = 8192, 4096, 4096, 11008
    fw = L.coda_fwd_workspace_bytes(BF16, M, K, d, N)
    # partials [M, d/256] fp32 + y * gamma [M, d] bf16
    assert fw >= M * (d // 256) * 4 + M * d * 2
    bw = L.coda_bwd_workspace_bytes(BF16, M, K, d, N)
    assert bw >= M * d * 2 + M * (d // 256) * 4 + (M // 256) * d * 4 + M * 4
    assert L.coda_swiglu_bwd_workspace_bytes(BF16, 8192, 4096, 14336) >= 8192 * 2 * 14336 * 2
    assert L.coda_bwd_workspace_bytes(F32, M, K, d, N) == 0
    assert L.coda_fwd_workspace_bytes(7, M, K, d, N) == 0


class FakeMem:
    """Distinct, 16-byte aligned fake device addresses, never dereferenced."""

    def __init__(self):
        self.next = 1 << 40

    def __call__(self, nbytes):
        p = self.next
        self.next += (nbytes + 4095) // 4096 * 4096 + 4096
        return ctypes.c_void_p(p)


def fwd_args(dtype=BF16, M=64, K=32, d=48, N=80, eps=1e-6):
    m = FakeMem()
    e = 2 if dtype == BF16 else 4
    a = dict(dtype=dtype, M=M, K=K, d=d, N=N, eps=eps,
             X=m(M * K * e), W1=m(K * d * e), R=m(M * d * e), gamma=m(d * e), W2=m(d * N * e),
             y=m(M * d * e), r=m(M * 4), z=m(M * N * e))
    a["ws_bytes"] = 1 << 20
    a["ws"] = m(a["ws_bytes"])
    return a


def call_fwd(L, a):
    return L.coda_fwd(a["dtype"], a["M"], a["K"], a["d"], a["N"], a["eps"], a["X"], a["W1"], a["R"],
                      a["gamma"], a["W2"], a["y"], a["r"], a["z"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 5, DTYPE),
    ("X", None, NULL), ("W2", None, NULL), ("r", None, NULL), ("z", None, NULL),
    ("M", 0, SHAPE), ("M", -8, SHAPE), ("K", 12, SHAPE), ("d", 4, SHAPE), ("N", 81, SHAPE),
    ("eps", 0.0, EPS), ("eps", -1e-6, EPS), ("eps", float("nan"), EPS), ("eps", float("inf"), EPS),
    ("ws", None, WORKSPACE), ("ws_bytes", 16, WORKSPACE),
])
def test_fwd_rejects(L, field, value, status):
    a = fwd_args()
    a[field] = value
    assert call_fwd(L, a) == status


def test_fwd_rejects_misalignment_and_alias(L):
    a = fwd_args()
    a["R"] = ctypes.c_void_p(a["R"].value + 2)
    assert call_fwd(L, a) == ALIGN
    a = fwd_args()
    a["z"] = ctypes.c_void_p(a["X"].value)          # output over an input
    assert call_fwd(L, a) == ALIAS
    a = fwd_args()
    a["y"] = ctypes.c_void_p(a["ws"].value + 256)   # output inside the workspace
    assert call_fwd(L, a) == ALIAS
    a = fwd_args()
    a["r"] = ctypes.c_void_p(a["y"].value + 16)     # two outputs overlap
    assert call_fwd(L, a) == ALIAS


def test_fwd_f32_multiple_of_four(L):
    a = fwd_args(dtype=F32, M=12, K=20, d=28, N=36)
    a["ws_bytes"] = 16
    assert call_fwd(L, a) == WORKSPACE               # shapes 12/20/28/36 pass for f32 ...
    a = fwd_args(dtype=F32, M=12, K=20, d=30, N=36)
    assert call_fwd(L, a) == SHAPE                   # ... 30 is not a multiple of 4


def test_size_limits(L):
    """Tensors past 2 GiB are accepted (the call here then stops at the
    missing workspace, before any HIP call); row lengths past 2^21 and row
    counts past 2^23 are refused."""
    a = fwd_args(M=1 << 16, N=1 << 15)               # z is 4 GiB of bf16
    assert call_fwd(L, a) == WORKSPACE
    a = fwd_args(N=(1 << 21) + 8)                    # a row length past 2^21
    assert call_fwd(L, a) == SHAPE
    a = fwd_args(M=(1 << 23) + 8)                    # a row count past 2^23
    assert call_fwd(L, a) == SHAPE
    a = fwd_args(M=1 << 23, K=8, d=8, N=8)           # at the row-count limit
    assert call_fwd(L, a) == WORKSPACE


def call_fwd_noalloc(L, a):
    return L.coda_fwd_noalloc(a["dtype"], a["M"], a["K"], a["d"], a["N"], a["eps"], a["X"], a["W1"], a["R"],
                              a["gamma"], a["W2"], a["y"], a["r"], a["z"], None)


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 5, DTYPE), ("X", None, NULL), ("z", None, NULL), ("M", 0, SHAPE), ("N", 81, SHAPE),
    ("eps", 0.0, EPS), ("eps", float("nan"), EPS),
])
def test_fwd_noalloc_rejects(L, field, value, status):
    """The workspace-free forward checks its arguments like coda_fwd, before
    any HIP call."""
    a = fwd_args()
    a[field] = value
    assert call_fwd_noalloc(L, a) == status


def test_fwd_noalloc_scratch_limit_and_alias(L):
    """A forward whose workspace would exceed the built-in 80 MiB scratch is
    refused with CODA_ERR_WORKSPACE before any HIP call; the LLaMA-7B- and
    70B-hidden-shaped forwards fit.  Outputs over inputs are still refused."""
    limit = 80 << 20
    assert L.coda_fwd_workspace_bytes(BF16, 8192, 4096, 4096, 11008) <= limit
    assert L.coda_fwd_workspace_bytes(BF16, 4096, 8192, 8192, 28672) <= limit
    a = fwd_args(M=8192, K=64, d=8192, N=64)          # y * gamma alone is 128 MiB
    assert L.coda_fwd_workspace_bytes(BF16, 8192, 64, 8192, 64) > limit
    assert call_fwd_noalloc(L, a) == WORKSPACE
    a = fwd_args()
    a["z"] = ctypes.c_void_p(a["X"].value)
    assert call_fwd_noalloc(L, a) == ALIAS


def bwd_call(L, **over):
    m = FakeMem()
    M, K, d, N = 64, 32, 48, 80
    a = dict(dtype=BF16, M=M, K=K, d=d, N=N, X=m(M * K * 2), W1=m(K * d * 2), gamma=m(d * 2),
             W2=m(d * N * 2), y=m(M * d * 2), r=m(M * 4), dz=m(M * N * 2), dX=m(M * K * 2),
             dW1=m(K * d * 2), dR=m(M * d * 2), dW2=m(d * N * 2), dgamma=m(d * 4),
             ws=m(1 << 20), ws_bytes=1 << 20)
    a.update(over)
    return L.coda_bwd(a["dtype"], a["M"], a["K"], a["d"], a["N"], a["X"], a["W1"], a["gamma"], a["W2"],
                      a["y"], a["r"], a["dz"], a["dX"], a["dW1"], a["dR"], a["dW2"], a["dgamma"],
                      a["ws"], a["ws_bytes"], None)


def test_bwd_rejects(L):
    assert bwd_call(L, dtype=9) == DTYPE
    assert bwd_call(L, dz=None) == NULL
    assert bwd_call(L, dgamma=None) == NULL
    assert bwd_call(L, N=84) == SHAPE
    assert bwd_call(L, dtype=F32) == UNSUPPORTED
    assert bwd_call(L, ws_bytes=64) == WORKSPACE
    assert bwd_call(L, ws=None) == WORKSPACE
    assert bwd_call(L, dgamma=ctypes.c_void_p((1 << 41) + 4)) == ALIGN


def test_bwd_alias(L):
    m = FakeMem()
    p = m(1 << 16)
    assert bwd_call(L, dX=p, dW1=ctypes.c_void_p(p.value + 64)) == ALIAS


def test_swiglu_rejects(L):
    m = FakeMem()
    M, d, F = 64, 32, 40
    X, W, Wd = m(M * d * 2), m(d * 2 * F * 2), m(F * d * 2)
    gu, a, z = m(M * 2 * F * 2), m(M * F * 2), m(M * d * 2)
    assert L.coda_swiglu_fwd(BF16, M, d, F, X, W, Wd, gu, a, None, None, 0, None) == NULL
    assert L.coda_swiglu_fwd(BF16, M, d, 44, X, W, Wd, gu, a, z, None, 0, None) == SHAPE
    assert L.coda_swiglu_fwd(F32, M, d, F, X, W, Wd, gu, a, z, None, 0, None) == UNSUPPORTED
    assert L.coda_swiglu_fwd(BF16, M, d, F, X, W, Wd, gu, gu, z, None, 0, None) == ALIAS
    dX, dW, dWd, ws = m(M * d * 2), m(d * 2 * F * 2), m(F * d * 2), m(M * 2 * F * 2)
    need = L.coda_swiglu_bwd_workspace_bytes(BF16, M, d, F)
    assert L.coda_swiglu_bwd(BF16, M, d, F, X, W, Wd, gu, a, z, dX, dW, dWd, ws, need - 16, None) == WORKSPACE
    assert L.coda_swiglu_bwd(BF16, M, d, F, X, W, Wd, gu, a, z, dX, dW, X, ws, need, None) == ALIAS


def _mlp_mem(m, M, K, d, F):
    return dict(X=m(M * K * 2), W1=m(K * d * 2), R=m(M * d * 2), gamma=m(d * 2), W=m(d * 2 * F * 2),
                Wd=m(F * d * 2), y=m(M * d * 2), r=m(M * 4), gu=m(M * 2 * F * 2), a=m(M * F * 2),
                z=m(M * d * 2), dz=m(M * d * 2), dy_in=m(M * d * 2), dX=m(M * K * 2), dW1=m(K * d * 2),
                dR=m(M * d * 2), dW=m(d * 2 * F * 2), dWd=m(F * d * 2), dgamma=m(d * 4),
                ws=m(1 << 22), ws_bytes=1 << 22)


def mlp_fwd_call(L, **over):
    M, K, d, F = 64, 32, 48, 40
    a = dict(dtype=BF16, M=M, K=K, d=d, F=F, eps=1e-6, **_mlp_mem(FakeMem(), M, K, d, F))
    a.update(over)
    return L.coda_mlp_fwd(a["dtype"], a["M"], a["K"], a["d"], a["F"], a["eps"], a["X"], a["W1"], a["R"],
                          a["gamma"], a["W"], a["Wd"], a["y"], a["r"], a["gu"], a["a"], a["z"], a["ws"],
                          a["ws_bytes"], None)


def mlp_bwd_call(L, **over):
    M, K, d, F = 64, 32, 48, 40
    a = dict(dtype=BF16, M=M, K=K, d=d, F=F, **_mlp_mem(FakeMem(), M, K, d, F))
    a.update(over)
    return L.coda_mlp_bwd(a["dtype"], a["M"], a["K"], a["d"], a["F"], a["X"], a["W1"], a["gamma"], a["W"],
                          a["Wd"], a["y"], a["r"], a["gu"], a["a"], a["dz"], a["dy_in"], a["dX"], a["dW1"],
                          a["dR"], a["dW"], a["dWd"], a["dgamma"], a["ws"], a["ws_bytes"], None)


def test_mlp_workspace_sizes(L):
    M, K, d, F = 8192, 4096, 4096, 11008
    assert L.coda_mlp_fwd_workspace_bytes(BF16, M, K, d, F) == L.coda_fwd_workspace_bytes(BF16, M, K, d, 1)
    # dgu [M, 2F] bf16 + the block backward's workspace
    assert (L.coda_mlp_bwd_workspace_bytes(BF16, M, K, d, F)
            >= M * 2 * F * 2 + L.coda_bwd_workspace_bytes(BF16, M, K, d, 2 * F))
    assert L.coda_mlp_fwd_workspace_bytes(F32, M, K, d, F) == 0
    assert L.coda_mlp_bwd_workspace_bytes(F32, M, K, d, F) == 0


def test_mlp_rejects(L):
    assert mlp_fwd_call(L, dtype=9) == DTYPE
    assert mlp_fwd_call(L, Wd=None) == NULL
    assert mlp_fwd_call(L, F=44) == SHAPE
    assert mlp_fwd_call(L, eps=0.0) == EPS
    assert mlp_fwd_call(L, eps=float("nan")) == EPS
    assert mlp_fwd_call(L, dtype=F32) == UNSUPPORTED
    assert mlp_fwd_call(L, ws_bytes=64) == WORKSPACE
    assert mlp_fwd_call(L, gu=ctypes.c_void_p((1 << 41) + 8)) == ALIGN
    m = FakeMem()
    m.next = 1 << 44                  # away from the helpers' own fake addresses
    p = m(1 << 20)
    assert mlp_fwd_call(L, a=p, z=ctypes.c_void_p(p.value + 64)) == ALIAS
    assert mlp_bwd_call(L, dtype=9) == DTYPE
    assert mlp_bwd_call(L, dgamma=None) == NULL
    assert mlp_bwd_call(L, K=36) == SHAPE
    assert mlp_bwd_call(L, dtype=F32) == UNSUPPORTED
    assert mlp_bwd_call(L, ws=None) == WORKSPACE
    assert mlp_bwd_call(L, dy_in=ctypes.c_void_p((1 << 41) + 4)) == ALIGN
    d_R = m(64 * 48 * 2)
    assert mlp_bwd_call(L, dR=d_R, dy_in=d_R) == ALIAS          # dy_in may not overlap an output


def test_ce_rejects(L):
    m = FakeMem()
    M, d, V = 64, 32, 200
    h, Wv, lab = m(M * d * 2), m(d * V * 2), m(M * 4)
    logits, lse, loss, ws = m(M * V * 2), m(M * 4), m(M * 4), m(1 << 20)
    need = L.coda_ce_fwd_workspace_bytes(BF16, M, d, V)
    assert need >= 2 * M * ((V + 255) // 256) * 4 + M * 4
    assert L.coda_ce_fwd(BF16, M, d, V, h, Wv, None, logits, lse, loss, ws, need, None) == NULL
    assert L.coda_ce_fwd(BF16, M, d, 204, h, Wv, lab, logits, lse, loss, ws, need, None) == SHAPE
    assert L.coda_ce_fwd(F32, M, d, V, h, Wv, lab, logits, lse, loss, ws, need, None) == UNSUPPORTED
    assert L.coda_ce_fwd(BF16, M, d, V, h, Wv, lab, logits, lse, loss, ws, need - 16, None) == WORKSPACE
    assert L.coda_ce_fwd(BF16, M, d, V, h, Wv, lab, logits, lse, lse, ws, need, None) == ALIAS
    assert L.coda_ce_fwd(BF16, M, d, V, h, Wv, ctypes.c_void_p(lab.value + 4), logits, lse, loss, ws, need,
                         None) == ALIGN
    dl, dh, dWv = m(M * 4), m(M * d * 2), m(d * V * 2)
    nb = L.coda_ce_bwd_workspace_bytes(BF16, M, d, V)
    assert nb >= M * V * 2
    assert L.coda_ce_bwd(BF16, M, d, V, h, Wv, lab, logits, lse, dl, dh, dWv, ws, nb - 16, None) == WORKSPACE
    assert L.coda_ce_bwd(BF16, M, d, V, h, Wv, lab, logits, lse, dl, dh, h, ws, nb, None) == ALIAS
    assert L.coda_ce_bwd(9, M, d, V, h, Wv, lab, logits, lse, dl, dh, dWv, ws, nb, None) == DTYPE


def test_rope_rejects(L):
    m = FakeMem()
    M, K, N = 64, 32, 96
    X, W, Y = m(M * K * 2), m(K * N * 2), m(M * N * 2)
    ws = m(1 << 20)
    need = L.coda_rope_fwd_workspace_bytes(BF16, M, K, N, 64, 32, 16)
    assert need >= 16 * 32 * 4
    ok = dict(N_rot=64, D=32, S=16, base=10000.0)

    def fwd(**o):
        a = {**ok, **o}
        return L.coda_rope_fwd(a.get("dtype", BF16), M, K, N, a["N_rot"], a["D"], a["S"], a["base"], X, W,
                               a.get("Y", Y), ws, a.get("ws_bytes", need), None)
    assert fwd(D=12) == SHAPE            # head width not a multiple of 8
    assert fwd(N_rot=48) == SHAPE        # rotated columns not whole heads
    assert fwd(N_rot=128) == SHAPE       # more rotated columns than N
    assert fwd(S=0) == SHAPE
    assert fwd(base=-1.0) == SHAPE
    assert fwd(base=float("inf")) == SHAPE
    assert fwd(dtype=F32) == UNSUPPORTED
    assert fwd(ws_bytes=need - 16) == WORKSPACE
    assert fwd(Y=X) == ALIAS
    assert L.coda_rope_fwd(BF16, M, K, N, 64, 32, 16, 10000.0, X, None, Y, ws, need, None) == NULL
    dY, dX, dW = m(M * N * 2), m(M * K * 2), m(K * N * 2)
    nb = L.coda_rope_bwd_workspace_bytes(BF16, M, K, N, 64, 32, 16)
    assert nb >= need + M * N * 2
    assert L.coda_rope_bwd(BF16, M, K, N, 64, 32, 16, 10000.0, X, W, dY, dX, dW, ws, nb - 16, None) == WORKSPACE
    assert L.coda_rope_bwd(BF16, M, K, N, 64, 32, 16, 10000.0, X, W, dY, dX, X, ws, nb, None) == ALIAS


def test_mx8_rejects(L):
    m = FakeMem()
    M, K, d, N = 64, 256, 384, 96
    Xq, Xs = m(M * K), m(M * K // 32)
    W1q, W1s = m(d * K), m(d * K // 32)
    W2q, W2s = m(N * d), m(N * d // 32)
    R, g, y, r, z = m(M * d * 2), m(d * 2), m(M * d * 2), m(M * 4), m(M * N * 2)
    need = L.coda_fwd_mx8_workspace_bytes(M, K, d, N)
    # partial sums, codes and scales of y * gamma
    assert need >= M * 2 * 4 + M * d + M * d // 32
    ws = m(need)

    def fwd(**o):
        a = dict(M=M, K=K, d=d, N=N, eps=1e-6, Xq=Xq, R=R, y=y, z=z, ws_bytes=need)
        a.update(o)
        return L.coda_fwd_mx8(a["M"], a["K"], a["d"], a["N"], a["eps"], a["Xq"], Xs, W1q, W1s, a["R"], g,
                              W2q, W2s, a["y"], r, a["z"], ws, a["ws_bytes"], None)
    assert fwd(K=200) == SHAPE           # K not whole steps of 128
    assert fwd(d=320) == SHAPE           # d not whole steps of 128
    assert fwd(M=60) == SHAPE
    assert fwd(N=0) == SHAPE
    assert fwd(eps=0.0) == EPS
    assert fwd(ws_bytes=need - 1) == WORKSPACE
    assert fwd(Xq=None) == NULL
    assert fwd(y=R) == ALIAS
    assert fwd(z=ctypes.c_void_p(z.value + 8)) == ALIGN
    q_src, q_codes, q_scales = m(M * K * 2), m(M * K), m(M * K // 32)
    assert L.coda_mx8_quantize(M, 48, q_src, 48, q_codes, q_scales, None) == SHAPE
    assert L.coda_mx8_quantize(M, 96, q_src, 96, q_codes, q_scales, None) == SHAPE   # not whole 128-k steps
    assert L.coda_mx8_quantize(M, K, q_src, K - 8, q_codes, q_scales, None) == SHAPE
    assert L.coda_mx8_quantize(0, K, q_src, K, q_codes, q_scales, None) == SHAPE
    assert L.coda_mx8_quantize(M, K, q_src, K, q_src, q_scales, None) == ALIAS
    assert L.coda_mx8_quantize(M, K, None, K, q_codes, q_scales, None) == NULL
    assert L.coda_mx8_quantize(M, K, ctypes.c_void_p(q_src.value + 4), K, q_codes, q_scales, None) == ALIGN

def bwd_mx8_call(L, **over):
    m = FakeMem()
    M, K, d, N = 256, 40, 128, 384
    a = dict(M=M, K=K, d=d, N=N, X=m(M * K * 2), W1=m(K * d * 2), gamma=m(d * 2), W2=m(d * N * 2),
             y=m(M * d * 2), r=m(M * 4), dz=m(M * N * 2), dX=m(M * K * 2), dW1=m(K * d * 2), dR=m(M * d * 2),
             dW2=m(d * N * 2), dg=m(d * 4))
    a["ws_bytes"] = L.coda_bwd_mx8_workspace_bytes(M, K, d, N)
    a["ws"] = m(a["ws_bytes"])
    a.update(over)
    return L.coda_bwd_mx8(a["M"], a["K"], a["d"], a["N"], a["X"], a["W1"], a["gamma"], a["W2"], a["y"], a["r"],
                          a["dz"], a["dX"], a["dW1"], a["dR"], a["dW2"], a["dg"], a["ws"], a["ws_bytes"], None)


def test_bwd_mx8_rejects(L):
    """The MXFP8 backward checks like coda_bwd, and needs M, d, N in whole
    128-element K steps; every rejection comes before any HIP call."""
    assert L.coda_bwd_mx8_workspace_bytes(256, 40, 128, 384) > 256 * 384 * 2
    assert L.coda_bwd_mx8_workspace_bytes(200, 40, 128, 384) == 0
    assert bwd_mx8_call(L, X=None) == NULL
    assert bwd_mx8_call(L, dg=None) == NULL
    assert bwd_mx8_call(L, M=200) == SHAPE
    assert bwd_mx8_call(L, d=136) == SHAPE
    assert bwd_mx8_call(L, N=392) == SHAPE
    assert bwd_mx8_call(L, K=12) == SHAPE
    assert bwd_mx8_call(L, ws_bytes=1024) == WORKSPACE
    assert bwd_mx8_call(L, ws=None) == WORKSPACE
    m = FakeMem()
    x = m(1 << 20)
    assert bwd_mx8_call(L, X=x, dX=x) == ALIAS
    assert bwd_mx8_call(L, r=ctypes.c_void_p(m(4096).value + 4)) == ALIGN



def swiglu_mx8_call(L, bwd, **over):
    m = FakeMem()
    M, d, F = 256, 128, 384
    a = dict(M=M, d=d, F=F, X=m(M * d * 2), W=m(d * 2 * F * 2), Wd=m(F * d * 2), gu=m(M * 2 * F * 2),
             a=m(M * F * 2), z=m(M * d * 2), dz=m(M * d * 2), dX=m(M * d * 2), dW=m(d * 2 * F * 2),
             dWd=m(F * d * 2))
    q = L.coda_swiglu_bwd_mx8_workspace_bytes if bwd else L.coda_swiglu_fwd_mx8_workspace_bytes
    a["ws_bytes"] = q(M, d, F)
    a["ws"] = m(a["ws_bytes"])
    a.update(over)
    if bwd:
        return L.coda_swiglu_bwd_mx8(a["M"], a["d"], a["F"], a["X"], a["W"], a["Wd"], a["gu"], a["a"], a["dz"],
                                     a["dX"], a["dW"], a["dWd"], a["ws"], a["ws_bytes"], None)
    return L.coda_swiglu_fwd_mx8(a["M"], a["d"], a["F"], a["X"], a["W"], a["Wd"], a["gu"], a["a"], a["z"],
                                 a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("bwd", [False, True], ids=["fwd", "bwd"])
def test_swiglu_mx8_rejects(L, bwd):
    """The MXFP8 SwiGLU calls need M, d, F in whole 128-element blocks and
    check pointers, alignment, aliasing and the workspace before any HIP
    call; the workspace query returns 0 for a refused shape."""
    q = L.coda_swiglu_bwd_mx8_workspace_bytes if bwd else L.coda_swiglu_fwd_mx8_workspace_bytes
    assert q(256, 128, 384) > 0
    for bad in ((200, 128, 384), (256, 136, 384), (256, 128, 392), (0, 128, 384)):
        assert q(*bad) == 0
    assert swiglu_mx8_call(L, bwd, X=None) == NULL
    assert swiglu_mx8_call(L, bwd, Wd=None) == NULL
    assert swiglu_mx8_call(L, bwd, M=200) == SHAPE
    assert swiglu_mx8_call(L, bwd, d=136) == SHAPE
    assert swiglu_mx8_call(L, bwd, F=392) == SHAPE
    assert swiglu_mx8_call(L, bwd, ws_bytes=1024) == WORKSPACE
    assert swiglu_mx8_call(L, bwd, ws=None) == WORKSPACE
    m = FakeMem()
    x = m(1 << 22)
    out = "dX" if bwd else "z"
    assert swiglu_mx8_call(L, bwd, X=x, **{out: x}) == ALIAS
    assert swiglu_mx8_call(L, bwd, W=ctypes.c_void_p(m(4096).value + 4)) == ALIGN


def mlp_mx8_call(L, bwd, **over):
    m = FakeMem()
    M, K, d, F = 256, 128, 128, 256
    a = dict(M=M, K=K, d=d, F=F, eps=1e-6, X=m(M * K * 2), W1=m(K * d * 2), R=m(M * d * 2), gamma=m(d * 2),
             W=m(d * 2 * F * 2), Wd=m(F * d * 2), y=m(M * d * 2), r=m(M * 4), gu=m(M * 2 * F * 2),
             a=m(M * F * 2), z=m(M * d * 2), dz=m(M * d * 2), dy_in=m(M * d * 2), dX=m(M * K * 2),
             dW1=m(K * d * 2), dR=m(M * d * 2), dW=m(d * 2 * F * 2), dWd=m(F * d * 2), dg=m(d * 4))
    q = L.coda_mlp_bwd_mx8_workspace_bytes if bwd else L.coda_mlp_fwd_mx8_workspace_bytes
    a["ws_bytes"] = q(M, K, d, F)
    a["ws"] = m(a["ws_bytes"])
    a.update(over)
    if bwd:
        return L.coda_mlp_bwd_mx8(a["M"], a["K"], a["d"], a["F"], a["X"], a["W1"], a["gamma"], a["W"], a["Wd"],
                                  a["y"], a["r"], a["gu"], a["a"], a["dz"], a["dy_in"], a["dX"], a["dW1"], a["dR"],
                                  a["dW"], a["dWd"], a["dg"], a["ws"], a["ws_bytes"], None)
    return L.coda_mlp_fwd_mx8(a["M"], a["K"], a["d"], a["F"], a["eps"], a["X"], a["W1"], a["R"], a["gamma"],
                              a["W"], a["Wd"], a["y"], a["r"], a["gu"], a["a"], a["z"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("bwd", [False, True], ids=["fwd", "bwd"])
def test_mlp_mx8_rejects(L, bwd):
    """The MXFP8 MLP calls need M, K, d, F in whole 128-element blocks and
    check pointers, eps, alignment, aliasing and the workspace before any HIP
    call; dy_in is optional."""
    q = L.coda_mlp_bwd_mx8_workspace_bytes if bwd else L.coda_mlp_fwd_mx8_workspace_bytes
    assert q(256, 128, 128, 256) > 0
    for bad in ((200, 128, 128, 256), (256, 136, 128, 256), (256, 128, 136, 256), (256, 128, 128, 264)):
        assert q(*bad) == 0
    assert mlp_mx8_call(L, bwd, X=None) == NULL
    assert mlp_mx8_call(L, bwd, gamma=None) == NULL
    assert mlp_mx8_call(L, bwd, M=200) == SHAPE
    assert mlp_mx8_call(L, bwd, K=136) == SHAPE
    assert mlp_mx8_call(L, bwd, F=264) == SHAPE
    assert mlp_mx8_call(L, bwd, ws_bytes=1024) == WORKSPACE
    m = FakeMem()
    x = m(1 << 22)
    out = "dX" if bwd else "z"
    assert mlp_mx8_call(L, bwd, X=x, **{out: x}) == ALIAS
    assert mlp_mx8_call(L, bwd, W1=ctypes.c_void_p(m(4096).value + 4)) == ALIGN
    if bwd:
        d_ = m(1 << 20)
        assert mlp_mx8_call(L, bwd, dy_in=d_, dR=d_) == ALIAS
        assert mlp_mx8_call(L, bwd, dy_in=ctypes.c_void_p(m(4096).value + 8)) == ALIGN
    else:
        assert mlp_mx8_call(L, bwd, eps=0.0) == EPS

"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an object ``O`` exposing the oracle's functions and
raises AssertionError when the oracle disagrees with the pinned fact.  The
oracle tests call them with the real oracle; the mutation tests call them with
copies that carry one planted mistake and require that some pin fails.

Kinds of pin used here:
  * brute force: pure-Python loops over tiny inputs, written from the
    definitions independently of numpy;
  * finite differences: the backward against central differences of the
    forward's loss L = <dz, z>;
  * library routines: torch CPU float64 ``F.rms_norm``, ``F.silu`` and autograd;
  * closed forms and hand-worked examples (tests/golden/);
  * invariants of the mathematics (homogeneity, linearity in a weight).
"""
from __future__ import annotations

import json
import math
import os
from types import SimpleNamespace

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def oracle_namespace(**overrides):
    import oracle
    ns = {k: getattr(oracle, k) for k in oracle.__all__}
    ns.update(overrides)
    return SimpleNamespace(**ns)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol:.1e} * {scale:.3g}"


def _rng(seed):
    return np.random.default_rng(seed)


def _coda_case(seed, M, K, d, N, eps=1e-6):
    g = _rng(seed)
    return dict(X=g.standard_normal((M, K)), W1=g.standard_normal((K, d)) / math.sqrt(K),
                R=g.standard_normal((M, d)), gamma=1 + 0.1 * g.standard_normal(d),
                W2=g.standard_normal((d, N)) / math.sqrt(d), dz=g.standard_normal((M, N)),
                eps=eps)


def _loss_fwd(O, c):
    z = O.ref_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W2"], c["eps"])["z"]
    return float(np.sum(c["dz"] * z))


def _bwd_exact(O, c):
    f = O.ref_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W2"], c["eps"])
    return O.ref_bwd(c["X"], c["W1"], c["gamma"], c["W2"], f["y"], f["r"], c["dz"]), f


# ---------------------------------------------------------------- forward pins

def pin_fwd_bruteforce(O):
    """Pure-Python loops at M,K,d,N = 3,4,5,6 against ref_fwd (y, r, z)."""
    c = _coda_case(11, 3, 4, 5, 6, eps=1e-3)
    X, W1, R, gm, W2 = (c[k].tolist() for k in ("X", "W1", "R", "gamma", "W2"))
    M, K, d, N = 3, 4, 5, 6
    y = [[sum(X[i][k] * W1[k][j] for k in range(K)) + R[i][j] for j in range(d)] for i in range(M)]
    r = [1.0 / math.sqrt(sum(v * v for v in y[i]) / d + c["eps"]) for i in range(M)]
    z = [[sum(r[i] * y[i][j] * gm[j] * W2[j][n] for j in range(d)) for n in range(N)] for i in range(M)]
    f = O.ref_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W2"], c["eps"])
    _close(f["y"], y, 1e-13, "y vs loops")
    _close(f["r"], r, 1e-13, "r vs loops")
    _close(f["z"], z, 1e-13, "z vs loops")


def pin_fwd_torch_rmsnorm(O):
    """torch CPU float64: F.rms_norm(X W1 + R, (d,), gamma, eps) @ W2 (library routine)."""
    import torch
    import torch.nn.functional as F
    c = _coda_case(12, 16, 24, 40, 56, eps=1e-5)
    t = {k: torch.from_numpy(np.asarray(c[k])) for k in ("X", "W1", "R", "gamma", "W2")}
    yt = t["X"] @ t["W1"] + t["R"]
    ht = F.rms_norm(yt, (yt.shape[1],), t["gamma"], c["eps"])
    zt = ht @ t["W2"]
    f = O.ref_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W2"], c["eps"])
    _close(f["h"], ht.numpy(), 1e-13, "h vs torch rms_norm")
    _close(f["z"], zt.numpy(), 1e-13, "z vs torch rms_norm")


def pin_fwd_constant_rows(O):
    """W1 = 0 and rows of R constant (c_i): r_i = (c_i^2 + eps)^-1/2 and
    z_i = r_i c_i sum_j gamma_j W2[j, :] (closed form)."""
    g = _rng(13)
    M, K, d, N, eps = 5, 7, 9, 4, 0.3
    cvals = np.array([0.0, 1.0, -2.0, 0.5, 3.0])
    R = np.repeat(cvals[:, None], d, axis=1)
    gamma = 1 + 0.1 * g.standard_normal(d)
    W2 = g.standard_normal((d, N))
    f = O.ref_fwd(g.standard_normal((M, K)), np.zeros((K, d)), R, gamma, W2, eps)
    r_cf = 1.0 / np.sqrt(cvals ** 2 + eps)
    _close(f["r"], r_cf, 1e-14, "r closed form")
    _close(f["z"], (r_cf * cvals)[:, None] * (gamma @ W2)[None, :], 1e-13, "z closed form")


def pin_fwd_scale_invariance(O):
    """With eps = 0, z(aX, aR) = z(X, R) for a > 0 (RMSNorm is 0-homogeneous)."""
    c = _coda_case(14, 6, 8, 10, 12, eps=0.0)
    z1 = O.ref_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W2"], 0.0)["z"]
    z2 = O.ref_fwd(3.7 * c["X"], c["W1"], 3.7 * c["R"], c["gamma"], c["W2"], 0.0)["z"]
    _close(z2, z1, 1e-13, "scale invariance")


def pin_partials(O):
    """P from loops at a ragged tile width, and sum_t P[i, t] = d * ms_i."""
    g = _rng(15)
    y = g.standard_normal((4, 23))
    BN = 8
    P = O.ref_partials(y, BN)
    loops = [[sum(float(y[i, j]) ** 2 for j in range(t * BN, min(t * BN + BN, 23))) for t in range(3)]
             for i in range(4)]
    _close(P, loops, 1e-14, "partials vs loops")
    c = _coda_case(16, 5, 6, 40, 7)
    f = O.ref_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W2"], c["eps"])
    _close(O.ref_partials(f["y"], 16).sum(axis=1), 40 * f["ms"], 1e-13, "sum of partials")


def pin_rewrite_equals_unfused(O):
    """z = diag(r) (y (diag(gamma) W2)) with r from partials equals the unfused z."""
    c = _coda_case(17, 9, 16, 48, 20, eps=1e-5)
    a = O.ref_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W2"], c["eps"])
    b = O.ref_fwd_rewritten(c["X"], c["W1"], c["R"], c["gamma"], c["W2"], c["eps"], BN=16)
    _close(b["r"], a["r"], 1e-14, "r rewritten")
    _close(b["z"], a["z"], 1e-13, "z rewritten")
    # and both agree with plain loops on a tiny case
    pin_fwd_bruteforce(O)


def _golden_eval(expr, env):
    return eval(expr, {"__builtins__": {}}, env)  # expressions from a committed fixture


def pin_golden_coda(O):
    """The hand-worked 2x2 cases of tests/golden/coda_worked_example.json."""
    with open(os.path.join(GOLDEN, "coda_worked_example.json")) as fh:
        gold = json.load(fh)
    inp = {k: np.array(v, dtype=np.float64) for k, v in gold["inputs"].items()}
    env = {"rho": math.sqrt(0.4)}
    for case in gold["cases"]:
        eps = case["eps"]
        f = O.ref_fwd(inp["X"], inp["W1"], inp["R"], inp["gamma"], inp["W2"], eps)
        b = O.ref_bwd(inp["X"], inp["W1"], inp["gamma"], inp["W2"], f["y"], f["r"], inp["dz"])
        got = {"y": f["y"], "r": f["r"], "z": f["z"], **{k: b[k] for k in
               ("dgamma", "dR", "dX", "dW1", "dW2")}}
        for k, v in case["expect"].items():
            want = np.vectorize(lambda e: _golden_eval(e, env), otypes=[float])(np.array(v))
            _close(got[k], want, 1e-14, f"golden eps={eps} {k}")


# --------------------------------------------------------------- backward pins

def pin_bwd_finite_differences(O):
    """Central differences of L = <dz, z> for every input element, tiny shape."""
    c = _coda_case(21, 3, 4, 5, 6, eps=1e-2)
    b, _ = _bwd_exact(O, c)
    grads = {"X": b["dX"], "W1": b["dW1"], "R": b["dR"], "gamma": b["dgamma"], "W2": b["dW2"]}
    for name, grad in grads.items():
        base = c[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            hstep = 1e-6 * max(1.0, abs(base[idx]))
            cp = dict(c)
            arr = base.copy(); arr[idx] += hstep; cp[name] = arr
            lp = _loss_fwd(O, cp)
            arr = base.copy(); arr[idx] -= hstep; cp[name] = arr
            lm = _loss_fwd(O, cp)
            fd[idx] = (lp - lm) / (2 * hstep)
        _close(grad, fd, 1e-7, f"d{name} vs finite differences")


def pin_bwd_torch_autograd(O):
    """torch CPU float64 autograd through matmul + add + F.rms_norm + matmul."""
    import torch
    import torch.nn.functional as F
    c = _coda_case(22, 12, 20, 32, 28, eps=1e-5)
    t = {k: torch.tensor(np.asarray(c[k]), requires_grad=True) for k in ("X", "W1", "R", "gamma", "W2")}
    y = t["X"] @ t["W1"] + t["R"]
    z = F.rms_norm(y, (y.shape[1],), t["gamma"], c["eps"]) @ t["W2"]
    (z * torch.from_numpy(c["dz"])).sum().backward()
    b, _ = _bwd_exact(O, c)
    for k, g in (("X", "dX"), ("W1", "dW1"), ("R", "dR"), ("gamma", "dgamma"), ("W2", "dW2")):
        _close(b[g], t[k].grad.numpy(), 1e-12, f"{g} vs torch autograd")


def pin_bwd_invariants(O):
    """Identities of the mathematics:
    <dW2, W2> = <dgamma, gamma> = <dz, z> (z linear in W2 and in gamma);
    sum_j dy_ij y_ij = eps r_i^3 s_i (derivative of z(a y) at a = 1);
    <dX, X> + <dR, R> = <dW1, W1> + <dR, R> = eps sum_i r_i^3 s_i;
    dgamma_j = sum_n (n^T dz)_jn W2_jn (second route);
    s_i = (1/r_i) sum_n dz_in z_in.
    """
    c = _coda_case(23, 10, 14, 18, 22, eps=0.05)
    b, f = _bwd_exact(O, c)
    L = float(np.sum(c["dz"] * f["z"]))
    _close(np.sum(b["dW2"] * c["W2"]), L, 1e-12, "<dW2,W2>")
    _close(np.sum(b["dgamma"] * c["gamma"]), L, 1e-12, "<dgamma,gamma>")
    # s from its definition, independent of O's intermediate values
    dn = (c["dz"] @ c["W2"].T) * c["gamma"][None, :]
    s = np.sum(dn * f["y"], axis=1)
    rhs = c["eps"] * f["r"] ** 3 * s
    _close(np.sum(b["dR"] * f["y"], axis=1), rhs, 1e-12, "row identity")
    tot = float(np.sum(rhs))
    _close(np.sum(b["dX"] * c["X"]) + np.sum(b["dR"] * c["R"]), tot, 1e-12, "<dX,X>+<dR,R>")
    _close(np.sum(b["dW1"] * c["W1"]) + np.sum(b["dR"] * c["R"]), tot, 1e-12, "<dW1,W1>+<dR,R>")
    n = f["y"] * f["r"][:, None]
    _close(b["dgamma"], np.sum((n.T @ c["dz"]) * c["W2"], axis=1), 1e-12, "dgamma second route")
    _close(s, np.sum(c["dz"] * f["z"], axis=1) / f["r"], 1e-12, "s from z")


def pin_sampled_forms(O):
    """The row/column-restricted forms equal the corresponding slices of the
    full forms (which the pins above tie to the mathematics)."""
    c = _coda_case(24, 20, 12, 16, 24, eps=1e-4)
    f = O.ref_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W2"], c["eps"])
    rows = np.array([0, 7, 19])
    fr = O.ref_fwd_rows(c["X"], c["W1"], c["R"], c["gamma"], c["W2"], c["eps"], rows)
    for k in ("y", "r", "z"):
        _close(fr[k], f[k][rows], 1e-14, f"rows {k}")
    yr = O.ref_y_r(c["X"], c["W1"], c["R"], c["eps"])
    _close(yr["y"], f["y"], 1e-14, "ref_y_r y")
    _close(yr["r"], f["r"], 1e-14, "ref_y_r r")
    b = O.ref_bwd(c["X"], c["W1"], c["gamma"], c["W2"], f["y"], f["r"], c["dz"])
    cd, cn = np.array([1, 5, 15]), np.array([0, 11, 23])
    bs = O.ref_bwd_sampled(c["X"], c["W1"], c["gamma"], c["W2"], f["y"], f["r"], c["dz"], rows, cd, cn)
    _close(bs["dX_rows"], b["dX"][rows], 1e-13, "sampled dX")
    _close(bs["dR_rows"], b["dR"][rows], 1e-13, "sampled dR")
    _close(bs["dW1_cols"], b["dW1"][:, cd], 1e-13, "sampled dW1")
    _close(bs["dW2_cols"], b["dW2"][:, cn], 1e-13, "sampled dW2")
    _close(bs["dgamma"], b["dgamma"], 1e-13, "sampled dgamma")


# ----------------------------------------------------------------- SwiGLU pins

def _swiglu_case(seed, M, d, F):
    g = _rng(seed)
    return dict(X=g.standard_normal((M, d)), W=g.standard_normal((d, 2 * F)) / math.sqrt(d),
                Wd=g.standard_normal((F, d)) / math.sqrt(F), dz=g.standard_normal((M, d)))


def _swiglu_loss(O, c):
    return float(np.sum(c["dz"] * O.ref_swiglu_fwd(c["X"], c["W"], c["Wd"])["z"]))


def _swiglu_bwd(O, c):
    f = O.ref_swiglu_fwd(c["X"], c["W"], c["Wd"])
    return O.ref_swiglu_bwd(c["X"], c["W"], c["Wd"], f["gu"], f["a"], c["dz"]), f


def pin_swiglu_bruteforce(O):
    """Loops at M, d, F = 3, 4, 5 against ref_swiglu_fwd (gate columns first)."""
    c = _swiglu_case(31, 3, 4, 5)
    X, W, Wd = (c[k].tolist() for k in ("X", "W", "Wd"))
    M, d, F = 3, 4, 5
    gu = [[sum(X[i][k] * W[k][j] for k in range(d)) for j in range(2 * F)] for i in range(M)]
    a = [[gu[i][j] / (1.0 + math.exp(-gu[i][j])) * gu[i][F + j] for j in range(F)] for i in range(M)]
    z = [[sum(a[i][j] * Wd[j][n] for j in range(F)) for n in range(d)] for i in range(M)]
    f = O.ref_swiglu_fwd(c["X"], c["W"], c["Wd"])
    _close(f["gu"], gu, 1e-13, "gu vs loops")
    _close(f["a"], a, 1e-13, "a vs loops")
    _close(f["z"], z, 1e-13, "z vs loops")


def pin_swiglu_finite_differences(O):
    c = _swiglu_case(32, 3, 4, 5)
    b, _ = _swiglu_bwd(O, c)
    for name, grad in (("X", b["dX"]), ("W", b["dW"]), ("Wd", b["dWd"])):
        base = c[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            hstep = 1e-6 * max(1.0, abs(base[idx]))
            cp = dict(c)
            arr = base.copy(); arr[idx] += hstep; cp[name] = arr
            lp = _swiglu_loss(O, cp)
            arr = base.copy(); arr[idx] -= hstep; cp[name] = arr
            lm = _swiglu_loss(O, cp)
            fd[idx] = (lp - lm) / (2 * hstep)
        _close(grad, fd, 1e-7, f"swiglu d{name} vs finite differences")


def pin_swiglu_torch(O):
    """torch CPU float64: F.silu(g) * u with autograd (library routine)."""
    import torch
    import torch.nn.functional as Fn
    c = _swiglu_case(33, 16, 24, 40)
    t = {k: torch.tensor(c[k], requires_grad=True) for k in ("X", "W", "Wd")}
    gu = t["X"] @ t["W"]
    F = c["W"].shape[1] // 2
    z = (Fn.silu(gu[:, :F]) * gu[:, F:]) @ t["Wd"]
    (z * torch.from_numpy(c["dz"])).sum().backward()
    f = O.ref_swiglu_fwd(c["X"], c["W"], c["Wd"])
    _close(f["z"], z.detach().numpy(), 1e-13, "swiglu z vs torch")
    b, _ = _swiglu_bwd(O, c)
    for k in ("X", "W", "Wd"):
        _close(b["d" + k], t[k].grad.numpy(), 1e-12, f"swiglu d{k} vs torch")


def pin_swiglu_invariants(O):
    """<dWd, Wd> = <dz, z>; <dW[:, F:], W[:, F:]> = <dz, z> (z linear in Wd and
    in W_up); at g = 0, dg = da u / 2; a huge negative gate gives no NaN."""
    c = _swiglu_case(34, 9, 12, 14)
    b, f = _swiglu_bwd(O, c)
    L = float(np.sum(c["dz"] * f["z"]))
    F = 14
    _close(np.sum(b["dWd"] * c["Wd"]), L, 1e-12, "<dWd,Wd>")
    _close(np.sum(b["dW"][:, F:] * c["W"][:, F:]), L, 1e-12, "<dWu,Wu>")
    W = c["W"].copy(); W[:, :F] = 0.0
    f0 = O.ref_swiglu_fwd(c["X"], W, c["Wd"])
    b0 = O.ref_swiglu_bwd(c["X"], W, c["Wd"], f0["gu"], f0["a"], c["dz"])
    da = c["dz"] @ c["Wd"].T
    _close(b0["dgu"][:, :F], 0.5 * da * f0["gu"][:, F:], 1e-13, "g=0 gate gradient")
    s = O.sigmoid(np.array([-800.0, -30.0, 0.0, 30.0, 800.0]))
    assert np.all(np.isfinite(s)), "sigmoid overflow"
    _close(s, [0.0, math.exp(-30) / (1 + math.exp(-30)), 0.5, 1 / (1 + math.exp(-30)), 1.0], 1e-15, "sigmoid")


def pin_golden_swiglu(O):
    with open(os.path.join(GOLDEN, "swiglu_worked_example.json")) as fh:
        gold = json.load(fh)
    env = {"L3": math.log(3.0)}
    ev = np.vectorize(lambda e: _golden_eval(e, env), otypes=[float])
    for case in gold["cases"]:
        inp = {k: ev(np.array(v)) for k, v in case["inputs"].items()}
        f = O.ref_swiglu_fwd(inp["X"], inp["W"], inp["Wd"])
        b = O.ref_swiglu_bwd(inp["X"], inp["W"], inp["Wd"], f["gu"], f["a"], inp["dz"])
        got = {**f, **b}
        for k, v in case["expect"].items():
            _close(got[k], ev(np.array(v)), 1e-14, f"swiglu golden {k}")


def pin_swiglu_sampled(O):
    """Row/column-restricted SwiGLU forms equal slices of the full forms, both
    with exact saved activations and with saved activations rounded to bf16."""
    c = _swiglu_case(35, 20, 8, 12)
    f = O.ref_swiglu_fwd(c["X"], c["W"], c["Wd"])
    rows, cw, rd = np.array([0, 9, 19]), np.array([0, 5, 12, 23]), np.array([1, 7, 11])
    fr = O.ref_swiglu_fwd_rows(c["X"], c["W"], c["Wd"], rows)
    for k in ("gu", "a", "z"):
        _close(fr[k], f[k][rows], 1e-14, f"swiglu rows {k}")
    for saved_bf16 in (False, True):
        keep = O.bf16_rne if saved_bf16 else (lambda v: v)
        b = O.ref_swiglu_bwd(c["X"], c["W"], c["Wd"], keep(f["gu"]), keep(f["a"]), c["dz"])
        s = O.ref_swiglu_bwd_sampled(c["X"], c["W"], c["Wd"], c["dz"], rows, cw, rd, saved_bf16)
        _close(s["dX_rows"], b["dX"][rows], 1e-13, "swiglu sampled dX")
        _close(s["dgu_rows"], b["dgu"][rows], 1e-13, "swiglu sampled dgu")
        _close(s["dW_cols"], b["dW"][:, cw], 1e-13, "swiglu sampled dW")
        _close(s["dWd_rows"], b["dWd"][rd], 1e-13, "swiglu sampled dWd")


# -------------------------------------------------- MLP sub-layer (chained) pins

def _mlp_case(seed, M, K, d, F, eps=1e-2):
    g = _rng(seed)
    return dict(X=g.standard_normal((M, K)), W1=g.standard_normal((K, d)) / math.sqrt(K),
                R=g.standard_normal((M, d)), gamma=1 + 0.1 * g.standard_normal(d),
                W=g.standard_normal((d, 2 * F)) / math.sqrt(d),
                Wd=g.standard_normal((F, d)) / math.sqrt(F), dz=g.standard_normal((M, d)),
                dy_in=g.standard_normal((M, d)), eps=eps)


def _mlp_loss(O, c):
    f = O.ref_mlp_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W"], c["Wd"], c["eps"])
    return float(np.sum(c["dz"] * f["z"]) + np.sum(c["dy_in"] * f["y"]))


def _mlp_bwd(O, c, dy_in=True):
    f = O.ref_mlp_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W"], c["Wd"], c["eps"])
    b = O.ref_mlp_bwd(c["X"], c["W1"], c["gamma"], c["W"], c["Wd"], f["y"], f["r"], f["gu"], f["a"],
                      c["dz"], c["dy_in"] if dy_in else None)
    return b, f


def pin_mlp_finite_differences(O):
    """Central differences of L = <dz, z> + <dy_in, y> through the whole chain
    (projection + residual, RMS norm, SwiGLU, down projection), tiny shape."""
    c = _mlp_case(51, 3, 4, 5, 3)
    b, _ = _mlp_bwd(O, c)
    grads = {"X": b["dX"], "W1": b["dW1"], "R": b["dR"], "gamma": b["dgamma"], "W": b["dW"],
             "Wd": b["dWd"]}
    for name, grad in grads.items():
        base = c[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            hstep = 1e-6 * max(1.0, abs(base[idx]))
            cp = dict(c)
            arr = base.copy(); arr[idx] += hstep; cp[name] = arr
            lp = _mlp_loss(O, cp)
            arr = base.copy(); arr[idx] -= hstep; cp[name] = arr
            lm = _mlp_loss(O, cp)
            fd[idx] = (lp - lm) / (2 * hstep)
        _close(grad, fd, 1e-7, f"mlp d{name} vs finite differences")


def pin_mlp_torch(O):
    """torch CPU float64: matmul + add, F.rms_norm, matmul, F.silu(g) * u,
    matmul, with autograd of <dz, z> + <dy_in, y> (library routines)."""
    import torch
    import torch.nn.functional as Fn
    c = _mlp_case(52, 12, 20, 16, 12, eps=1e-5)
    t = {k: torch.tensor(np.asarray(c[k]), requires_grad=True) for k in ("X", "W1", "R", "gamma", "W", "Wd")}
    y = t["X"] @ t["W1"] + t["R"]
    gu = Fn.rms_norm(y, (y.shape[1],), t["gamma"], c["eps"]) @ t["W"]
    F = c["W"].shape[1] // 2
    z = (Fn.silu(gu[:, :F]) * gu[:, F:]) @ t["Wd"]
    ((z * torch.from_numpy(c["dz"])).sum() + (y * torch.from_numpy(c["dy_in"])).sum()).backward()
    b, f = _mlp_bwd(O, c)
    _close(f["z"], z.detach().numpy(), 1e-13, "mlp z vs torch")
    _close(f["gu"], gu.detach().numpy(), 1e-13, "mlp gu vs torch")
    for k in ("X", "W1", "R", "gamma", "W", "Wd"):
        _close(b["d" + k], t[k].grad.numpy(), 1e-12, f"mlp d{k} vs torch")


def pin_mlp_invariants(O):
    """<dWd, Wd> = <dW[:, F:], W[:, F:]> = <dz, z> (z is linear in Wd and in
    W_up); without dy_in, sum_j dy_ij y_ij = eps r_i^3 s_i (z depends on y only
    through diag(r) y, which is homogeneous of degree 0 at eps = 0); dy_in
    passes into dR, dX and dW1 unchanged: dR(dy_in) - dR(0) = dy_in."""
    c = _mlp_case(53, 9, 10, 12, 7, eps=0.05)
    b, f = _mlp_bwd(O, c, dy_in=False)
    L = float(np.sum(c["dz"] * f["z"]))
    F = 7
    _close(np.sum(b["dWd"] * c["Wd"]), L, 1e-12, "mlp <dWd,Wd>")
    _close(np.sum(b["dW"][:, F:] * c["W"][:, F:]), L, 1e-12, "mlp <dWu,Wu>")
    _close(np.sum(b["dR"] * f["y"], axis=1), c["eps"] * f["r"] ** 3 * b["s"], 1e-12, "mlp row identity")
    b1, _ = _mlp_bwd(O, c, dy_in=True)
    _close(b1["dR"] - b["dR"], c["dy_in"], 1e-12, "dy_in into dR")
    _close(b1["dX"] - b["dX"], c["dy_in"] @ c["W1"].T, 1e-12, "dy_in into dX")
    _close(b1["dW"], b["dW"], 1e-13, "dy_in does not reach dW")


def pin_mlp_sampled(O):
    """Row/column-restricted MLP forms equal slices of the full forms."""
    c = _mlp_case(54, 20, 12, 16, 10, eps=1e-4)
    f = O.ref_mlp_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W"], c["Wd"], c["eps"])
    rows = np.array([0, 7, 19])
    fr = O.ref_mlp_fwd_rows(c["X"], c["W1"], c["R"], c["gamma"], c["W"], c["Wd"], c["eps"], rows)
    for k in ("y", "r", "gu", "a", "z"):
        _close(fr[k], f[k][rows], 1e-14, f"mlp rows {k}")
    fq = O.ref_mlp_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W"], c["Wd"], c["eps"], O.bf16_rne)
    fqr = O.ref_mlp_fwd_rows(c["X"], c["W1"], c["R"], c["gamma"], c["W"], c["Wd"], c["eps"], rows, O.bf16_rne)
    for k in ("gu", "a", "z"):
        _close(fqr[k], fq[k][rows], 1e-14, f"mlp rows (stored operand) {k}")
    cd, c2, rf = np.array([1, 5, 15]), np.array([0, 9, 11, 19]), np.array([2, 3, 9])
    for dy_in, rnd in ((None, None), (c["dy_in"], None), (c["dy_in"], O.bf16_rne)):
        b = O.ref_mlp_bwd(c["X"], c["W1"], c["gamma"], c["W"], c["Wd"], f["y"], f["r"], f["gu"], f["a"],
                          c["dz"], dy_in, rnd)
        bs = O.ref_mlp_bwd_sampled(c["X"], c["W1"], c["gamma"], c["W"], c["Wd"], f["y"], f["r"], f["gu"],
                                   f["a"], c["dz"], dy_in, rows, cd, c2, rf, rnd)
        _close(bs["dX_rows"], b["dX"][rows], 1e-13, "mlp sampled dX")
        _close(bs["dR_rows"], b["dR"][rows], 1e-13, "mlp sampled dR")
        _close(bs["dW1_cols"], b["dW1"][:, cd], 1e-13, "mlp sampled dW1")
        _close(bs["dW_cols"], b["dW"][:, c2], 1e-13, "mlp sampled dW")
        _close(bs["dWd_rows"], b["dWd"][rf], 1e-13, "mlp sampled dWd")
        _close(bs["dgamma"], b["dgamma"], 1e-13, "mlp sampled dgamma")


def pin_mlp_dgu_rounding(O):
    """With dgu rounded for storage, the second half is the block backward of
    ``ref_bwd`` fed that rounded dgu (the MLP's dh GEMM input), and the
    rounding only moves what depends on dgu: dWd and dgu's own first half
    stay as without it."""
    c = _mlp_case(55, 10, 12, 16, 9, eps=1e-3)
    f = O.ref_mlp_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W"], c["Wd"], c["eps"])
    b0 = O.ref_mlp_bwd(c["X"], c["W1"], c["gamma"], c["W"], c["Wd"], f["y"], f["r"], f["gu"], f["a"],
                       c["dz"], c["dy_in"])
    b1 = O.ref_mlp_bwd(c["X"], c["W1"], c["gamma"], c["W"], c["Wd"], f["y"], f["r"], f["gu"], f["a"],
                       c["dz"], c["dy_in"], O.bf16_rne)
    # dgu from its definition, independent of O's intermediates
    F = 9
    g, u = f["gu"][:, :F], f["gu"][:, F:]
    sg = 1.0 / (1.0 + np.exp(-g))
    da = c["dz"] @ c["Wd"].T
    dgu = np.concatenate([da * u * sg * (1 + g * (1 - sg)), da * g * sg], axis=1)
    dgu_r = O.bf16_rne(dgu)           # pinned on its own by pin_bf16_rne
    ref = O.ref_bwd(c["X"], c["W1"], c["gamma"], c["W"], f["y"], f["r"], dgu_r, c["dy_in"])
    _close(b1["dW"], ref["dW2"], 1e-12, "rounded dgu: dW")
    _close(b1["dgamma"], ref["dgamma"], 1e-12, "rounded dgu: dgamma")
    _close(b1["dX"], ref["dX"], 1e-12, "rounded dgu: dX")
    _close(b1["dWd"], b0["dWd"], 1e-15, "rounding dgu leaves dWd")
    assert float(np.max(np.abs(b1["dgamma"] - b0["dgamma"]))) > 0.0, "rounding had no effect"


def pin_mlp_stored_operand_bruteforce(O):
    """With the gate/up GEMM's stored input rounded (h_round = bf16_rne),
    pure-Python loops over a tiny case: y = X W1 + R, r from y,
    gu_ij = r_i * sum_k round(y_ik gamma_k) W_kj, a = g sigmoid(g) u, z = a Wd;
    y and r do not depend on the rounding."""
    c = _mlp_case(56, 3, 4, 5, 2, eps=1e-3)
    X, W1, R, gm, W, Wd = (c[k] for k in ("X", "W1", "R", "gamma", "W", "Wd"))
    M, K = X.shape
    d, F = W1.shape[1], 2
    f = O.ref_mlp_fwd(X, W1, R, gm, W, Wd, c["eps"], O.bf16_rne)
    f0 = O.ref_mlp_fwd(X, W1, R, gm, W, Wd, c["eps"])
    for i in range(M):
        y = [sum(X[i][k] * W1[k][j] for k in range(K)) + R[i][j] for j in range(d)]
        r = 1.0 / math.sqrt(sum(v * v for v in y) / d + c["eps"])
        hy = [float(O.bf16_rne(np.array([y[k] * gm[k]]))[0]) for k in range(d)]
        gu = [r * sum(hy[k] * W[k][j] for k in range(d)) for j in range(2 * F)]
        a = [gu[j] / (1.0 + math.exp(-gu[j])) * gu[F + j] for j in range(F)]
        z = [sum(a[j] * Wd[j][m] for j in range(F)) for m in range(d)]
        _close(f["y"][i], y, 1e-13, "stored operand: y")
        _close(f["r"][i], r, 1e-13, "stored operand: r")
        _close(f["gu"][i], gu, 1e-13, "stored operand: gu")
        _close(f["a"][i], a, 1e-13, "stored operand: a")
        _close(f["z"][i], z, 1e-13, "stored operand: z")
    _close(f["y"], f0["y"], 0.0, "rounding leaves y")
    assert float(np.max(np.abs(f["gu"] - f0["gu"]))) > 0.0, "rounding had no effect"


# ---------------------------------------------------- cross-entropy LM-head pins

def _ce_case(seed, M, d, V, scale=1.0):
    g = _rng(seed)
    return dict(h=g.standard_normal((M, d)) * scale, Wv=g.standard_normal((d, V)) / math.sqrt(d),
                labels=g.integers(0, V, M), dloss=g.standard_normal(M))


def pin_ce_torch(O):
    """torch CPU float64 F.cross_entropy (reduction='none') with autograd of
    sum_i dloss_i loss_i (library routine)."""
    import torch
    import torch.nn.functional as Fn
    c = _ce_case(61, 12, 16, 300, scale=3.0)
    th = torch.tensor(c["h"], requires_grad=True)
    tw = torch.tensor(c["Wv"], requires_grad=True)
    loss = Fn.cross_entropy(th @ tw, torch.tensor(c["labels"]), reduction="none")
    (loss * torch.from_numpy(c["dloss"])).sum().backward()
    f = O.ref_ce_fwd(c["h"], c["Wv"], c["labels"])
    _close(f["loss"], loss.detach().numpy(), 1e-13, "ce loss vs torch")
    for logits in (None, f["logits"]):
        b = O.ref_ce_bwd(c["h"], c["Wv"], c["labels"], f["lse"], c["dloss"], logits)
        _close(b["dh"], th.grad.numpy(), 1e-12, "ce dh vs torch")
        _close(b["dWv"], tw.grad.numpy(), 1e-12, "ce dWv vs torch")


def pin_ce_ignored_rows(O):
    """Ignored rows (labels outside [0, V)): torch CPU float64
    F.cross_entropy with ignore_index=-100 and reduction='none' (library
    routine) gives loss 0 and zero gradients for the rows labelled -100; the
    other out-of-range labels (-1, V, a large index) give the same loss 0 and
    zero dlogits row, and the remaining rows equal the result of the call
    without the ignored rows."""
    import torch
    import torch.nn.functional as Fn
    c = _ce_case(67, 10, 8, 60, scale=2.0)
    lab = c["labels"].copy()
    lab[[1, 6]] = -100
    th = torch.tensor(c["h"], requires_grad=True)
    tw = torch.tensor(c["Wv"], requires_grad=True)
    loss = Fn.cross_entropy(th @ tw, torch.tensor(lab), reduction="none", ignore_index=-100)
    (loss * torch.from_numpy(c["dloss"])).sum().backward()
    f = O.ref_ce_fwd(c["h"], c["Wv"], lab)
    _close(f["loss"], loss.detach().numpy(), 1e-13, "ce ignored rows: loss vs torch")
    b = O.ref_ce_bwd(c["h"], c["Wv"], lab, f["lse"], c["dloss"])
    _close(b["dh"], th.grad.numpy(), 1e-12, "ce ignored rows: dh vs torch")
    _close(b["dWv"], tw.grad.numpy(), 1e-12, "ce ignored rows: dWv vs torch")
    lab2 = c["labels"].copy()
    bad = [0, 4, 9]
    lab2[bad] = [-1, 60, 1 << 30]
    f2 = O.ref_ce_fwd(c["h"], c["Wv"], lab2)
    b2 = O.ref_ce_bwd(c["h"], c["Wv"], lab2, f2["lse"], c["dloss"])
    assert np.all(f2["loss"][bad] == 0.0), "ce ignored rows: loss not 0"
    assert np.all(b2["dlogits"][bad] == 0.0), "ce ignored rows: dlogits row not 0"
    keep = np.setdiff1d(np.arange(10), bad)
    fk = O.ref_ce_fwd(c["h"][keep], c["Wv"], c["labels"][keep])
    bk = O.ref_ce_bwd(c["h"][keep], c["Wv"], c["labels"][keep], fk["lse"], c["dloss"][keep])
    _close(f2["loss"][keep], fk["loss"], 1e-14, "ce ignored rows: other losses")
    _close(f2["lse"], O.ref_ce_fwd(c["h"], c["Wv"], c["labels"])["lse"], 1e-14, "ce ignored rows: lse kept")
    _close(b2["dWv"], bk["dWv"], 1e-12, "ce ignored rows: dWv from the other rows")
    _close(b2["dh"][keep], bk["dh"], 1e-12, "ce ignored rows: dh of the other rows")
    assert np.all(b2["dh"][bad] == 0.0), "ce ignored rows: dh row not 0"
    s = O.ref_ce_bwd_sampled(c["h"], c["Wv"], lab2, f2["lse"], c["dloss"], np.arange(10), np.arange(60))
    _close(s["dh_rows"], b2["dh"], 1e-12, "ce ignored rows: sampled dh")
    _close(s["dWv_cols"], b2["dWv"], 1e-12, "ce ignored rows: sampled dWv")


def pin_ce_finite_differences(O):
    """Central differences of L = sum_i dloss_i loss_i, tiny shape."""
    c = _ce_case(62, 3, 4, 7)

    def L(h, Wv):
        return float(np.sum(c["dloss"] * O.ref_ce_fwd(h, Wv, c["labels"])["loss"]))
    f = O.ref_ce_fwd(c["h"], c["Wv"], c["labels"])
    b = O.ref_ce_bwd(c["h"], c["Wv"], c["labels"], f["lse"], c["dloss"])
    for name, grad in (("h", b["dh"]), ("Wv", b["dWv"])):
        base = c[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            hstep = 1e-6 * max(1.0, abs(base[idx]))
            hp, wp = c["h"], c["Wv"]
            arr = base.copy(); arr[idx] += hstep
            lp = L(arr, wp) if name == "h" else L(hp, arr)
            arr = base.copy(); arr[idx] -= hstep
            lm = L(arr, wp) if name == "h" else L(hp, arr)
            fd[idx] = (lp - lm) / (2 * hstep)
        _close(grad, fd, 1e-7, f"ce d{name} vs finite differences")


def pin_ce_closed_forms(O):
    """Wv = 0: every logit is 0, lse = log V, loss = log V, softmax uniform so
    dlogits = dloss (1/V - onehot).  Equal large logits (1000 + shift) give
    lse = 1000 + shift + log V without overflow.  Adding a constant to every
    logit of a row (an extra input column of ones) moves lse by it and leaves
    the loss."""
    c = _ce_case(63, 5, 6, 40)
    V = 40
    f = O.ref_ce_fwd(c["h"], np.zeros((6, V)), c["labels"])
    _close(f["lse"], np.full(5, math.log(V)), 1e-14, "ce zero weights lse")
    _close(f["loss"], np.full(5, math.log(V)), 1e-14, "ce zero weights loss")
    b = O.ref_ce_bwd(c["h"], np.zeros((6, V)), c["labels"], f["lse"], c["dloss"])
    want = np.full((5, V), 1.0 / V)
    want[np.arange(5), c["labels"]] -= 1.0
    _close(b["dlogits"], want * c["dloss"][:, None], 1e-14, "ce uniform dlogits")
    hb = np.ones((5, 1))
    Wb = np.full((1, V), 1000.0)
    fb = O.ref_ce_fwd(hb, Wb, c["labels"])
    _close(fb["lse"], np.full(5, 1000.0 + math.log(V)), 1e-14, "ce large logits lse")
    assert np.all(np.isfinite(fb["loss"])), "ce overflow"
    shift = np.array([0.5, -3.0, 7.0, 0.0, 100.0])
    ha = np.concatenate([c["h"], shift[:, None]], axis=1)
    Wa = np.concatenate([c["Wv"], np.ones((1, V))], axis=0)
    f0 = O.ref_ce_fwd(c["h"], c["Wv"], c["labels"])
    fa = O.ref_ce_fwd(ha, Wa, c["labels"])
    _close(fa["lse"], f0["lse"] + shift, 1e-12, "ce shift lse")
    _close(fa["loss"], f0["loss"], 1e-12, "ce shift loss")


def pin_ce_invariants(O):
    """Softmax rows sum to 1, so every row of dlogits sums to 0 and so does
    every row of dWv (its columns sum to zero vectors); <dh, h> = <dlogits,
    logits> = sum_i dloss_i (E_p[logits_i] - logits_i,label), with p from
    scipy's softmax (library routine)."""
    from scipy.special import softmax
    c = _ce_case(64, 9, 8, 50, scale=2.0)
    f = O.ref_ce_fwd(c["h"], c["Wv"], c["labels"])
    b = O.ref_ce_bwd(c["h"], c["Wv"], c["labels"], f["lse"], c["dloss"])
    _close(np.sum(b["dlogits"], axis=1), np.zeros(9), 1e-13, "ce dlogits rows sum to 0")
    _close(np.sum(b["dWv"], axis=1), np.zeros(8), 1e-12, "ce dWv rows sum to 0")
    lg = c["h"] @ c["Wv"]
    p = softmax(lg, axis=1)
    want = np.sum(c["dloss"] * (np.sum(p * lg, axis=1) - lg[np.arange(9), c["labels"]]))
    _close(np.sum(b["dh"] * c["h"]), want, 1e-12, "ce <dh,h>")


def pin_ce_partials(O):
    """The tiled running (max, sum-exp) state reaches scipy's logsumexp
    (library routine), for tile widths that divide V and ones that do not,
    and with one tile holding the row's largest logits by far."""
    from scipy.special import logsumexp
    g = _rng(65)
    x = g.standard_normal((6, 700)) * 5.0
    x[2, 650:] += 80.0
    for BN in (256, 128, 100, 700, 1):
        p = O.ref_ce_partials(x, BN)
        _close(p["lse"], logsumexp(x, axis=1), 1e-12, f"ce partials BN={BN}")
        T = -(-700 // BN)
        assert p["m"].shape == (6, T) and p["s"].shape == (6, T)
        _close(p["m"][:, 0], np.max(x[:, :BN], axis=1), 0.0, "ce partial max")


def pin_ce_sampled(O):
    """Row/column-restricted forms equal slices of the full forms, with the
    logits recomputed and with saved logits passed in."""
    c = _ce_case(66, 20, 8, 90)
    f = O.ref_ce_fwd(c["h"], c["Wv"], c["labels"])
    rows, cols = np.array([0, 7, 19]), np.array([0, 3, 44, 89])
    fr = O.ref_ce_fwd_rows(c["h"], c["Wv"], c["labels"], rows)
    for k in ("logits", "lse", "loss"):
        _close(fr[k], f[k][rows], 1e-14, f"ce rows {k}")
    b = O.ref_ce_bwd(c["h"], c["Wv"], c["labels"], f["lse"], c["dloss"])
    for logits in (None, f["logits"]):
        bs = O.ref_ce_bwd_sampled(c["h"], c["Wv"], c["labels"], f["lse"], c["dloss"], rows, cols, logits)
        _close(bs["dh_rows"], b["dh"][rows], 1e-13, "ce sampled dh")
        _close(bs["dWv_cols"], b["dWv"][:, cols], 1e-13, "ce sampled dWv")


# ------------------------------------------------------------------- RoPE pins

def _rope_case(seed, M, K, N, N_rot, D, S, base=10000.0):
    g = _rng(seed)
    return dict(X=g.standard_normal((M, K)), W=g.standard_normal((K, N)) / math.sqrt(K),
                dY=g.standard_normal((M, N)), N_rot=N_rot, D=D, S=S, base=base)


def _rope_args(c):
    return (c["N_rot"], c["D"], c["S"], c["base"])


def pin_rope_bruteforce(O):
    """Pure-Python loops: P = X W, then for rotated head columns
    y_2i = p_2i cos - p_2i+1 sin, y_2i+1 = p_2i sin + p_2i+1 cos with the angle
    (m mod S) base^(-2i/D); other columns unchanged."""
    c = _rope_case(71, 5, 3, 14, 8, 4, 3, base=100.0)
    X, W = c["X"], c["W"]
    f = O.ref_rope_fwd(X, W, *_rope_args(c))
    for m in range(5):
        P = [sum(X[m][k] * W[k][j] for k in range(3)) for j in range(14)]
        want = list(P)
        for h0 in range(0, 8, 4):
            for i in range(2):
                ang = (m % 3) * 100.0 ** (-2.0 * i / 4)
                a, b = P[h0 + 2 * i], P[h0 + 2 * i + 1]
                want[h0 + 2 * i] = a * math.cos(ang) - b * math.sin(ang)
                want[h0 + 2 * i + 1] = a * math.sin(ang) + b * math.cos(ang)
        _close(f["Y"][m], want, 1e-13, f"rope brute force row {m}")


def pin_rope_torch(O):
    """torch CPU float64 complex form: pairs as complex numbers times
    polar(1, angle) (torch.polar, view_as_complex), with autograd of <dY, Y>."""
    import torch
    c = _rope_case(72, 12, 16, 40, 32, 8, 5)
    N_rot, D, S, base = _rope_args(c)
    tX = torch.tensor(c["X"], requires_grad=True)
    tW = torch.tensor(c["W"], requires_grad=True)
    P = tX @ tW
    pos = (torch.arange(12) % S).double()
    theta = base ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
    rot = torch.polar(torch.ones(12, D // 2, dtype=torch.float64), pos[:, None] * theta[None, :])
    q = torch.view_as_complex(P[:, :N_rot].reshape(12, N_rot // D, D // 2, 2).contiguous())
    qr = torch.view_as_real(q * rot[:, None, :]).reshape(12, N_rot)
    Y = torch.cat([qr, P[:, N_rot:]], dim=1)
    (Y * torch.from_numpy(c["dY"])).sum().backward()
    f = O.ref_rope_fwd(c["X"], c["W"], N_rot, D, S, base)
    _close(f["Y"], Y.detach().numpy(), 1e-13, "rope Y vs torch")
    b = O.ref_rope_bwd(c["X"], c["W"], c["dY"], N_rot, D, S, base)
    _close(b["dX"], tX.grad.numpy(), 1e-12, "rope dX vs torch")
    _close(b["dW"], tW.grad.numpy(), 1e-12, "rope dW vs torch")


def pin_rope_finite_differences(O):
    c = _rope_case(73, 3, 4, 10, 8, 4, 2)
    args = _rope_args(c)
    b = O.ref_rope_bwd(c["X"], c["W"], c["dY"], *args)

    def L(X, W):
        return float(np.sum(c["dY"] * O.ref_rope_fwd(X, W, *args)["Y"]))
    for name, grad in (("X", b["dX"]), ("W", b["dW"])):
        base_ = c[name]
        fd = np.zeros_like(base_)
        for idx in np.ndindex(base_.shape):
            hstep = 1e-6 * max(1.0, abs(base_[idx]))
            arr = base_.copy(); arr[idx] += hstep
            lp = L(arr, c["W"]) if name == "X" else L(c["X"], arr)
            arr = base_.copy(); arr[idx] -= hstep
            lm = L(arr, c["W"]) if name == "X" else L(c["X"], arr)
            fd[idx] = (lp - lm) / (2 * hstep)
        _close(grad, fd, 1e-7, f"rope d{name} vs finite differences")


def pin_rope_properties(O):
    """Rows at position 0 are left unchanged; the rotation keeps every pair's
    length; the inverse undoes it; unrotated columns pass through; and the
    relative-position property: <rot(q, m), rot(k, n)> over a head depends only
    on m - n (rows of equal content at positions (1, 4) and (3, 6))."""
    g = _rng(74)
    N_rot, D, S, base = 16, 8, 7, 10000.0
    Y = g.standard_normal((14, 20))
    R = O.ref_rope_rotate(Y, N_rot, D, S, base)
    _close(R[0], Y[0], 0.0, "position 0")
    _close(R[7], Y[7], 0.0, "position 0 of the second sequence")
    _close(R[:, N_rot:], Y[:, N_rot:], 0.0, "unrotated columns")
    _close(R[:, 0:N_rot:2] ** 2 + R[:, 1:N_rot:2] ** 2, Y[:, 0:N_rot:2] ** 2 + Y[:, 1:N_rot:2] ** 2,
           1e-13, "pair lengths")
    _close(O.ref_rope_rotate(R, N_rot, D, S, base, inverse=True), Y, 1e-13, "inverse")
    q, k = g.standard_normal(20), g.standard_normal(20)
    Z = np.zeros((7, 20))
    Z[1], Z[3], Z[4], Z[6] = q, q, k, k
    RZ = O.ref_rope_rotate(Z, N_rot, D, S, base)
    for h0 in range(0, N_rot, D):
        a = float(np.dot(RZ[1, h0:h0 + D], RZ[4, h0:h0 + D]))
        b = float(np.dot(RZ[3, h0:h0 + D], RZ[6, h0:h0 + D]))
        _close(a, b, 1e-13, "relative position")


def pin_rope_sampled(O):
    c = _rope_case(75, 20, 6, 24, 16, 8, 6)
    args = _rope_args(c)
    f = O.ref_rope_fwd(c["X"], c["W"], *args)
    rows, cols = np.array([0, 5, 6, 13, 19]), np.array([0, 1, 7, 15, 16, 23])
    fr = O.ref_rope_fwd_rows(c["X"], c["W"], *args, rows)
    _close(fr["Y"], f["Y"][rows], 1e-14, "rope rows Y")
    b = O.ref_rope_bwd(c["X"], c["W"], c["dY"], *args)
    bs = O.ref_rope_bwd_sampled(c["X"], c["W"], c["dY"], *args, rows, cols)
    _close(bs["dX_rows"], b["dX"][rows], 1e-13, "rope sampled dX")
    _close(bs["dW_cols"], b["dW"][:, cols], 1e-13, "rope sampled dW")


def pin_bwd_dy_in_finite_differences(O):
    """``ref_bwd`` with dy_in: central differences of <dz, z> + <dy_in, y> for
    the block's own forward, tiny shape."""
    c = _coda_case(25, 3, 4, 5, 6, eps=1e-2)
    dy_in = _rng(26).standard_normal((3, 5))

    def loss(cc):
        f = O.ref_fwd(cc["X"], cc["W1"], cc["R"], cc["gamma"], cc["W2"], cc["eps"])
        return float(np.sum(cc["dz"] * f["z"]) + np.sum(dy_in * f["y"]))
    f = O.ref_fwd(c["X"], c["W1"], c["R"], c["gamma"], c["W2"], c["eps"])
    b = O.ref_bwd(c["X"], c["W1"], c["gamma"], c["W2"], f["y"], f["r"], c["dz"], dy_in)
    for name, grad in (("X", b["dX"]), ("W1", b["dW1"]), ("R", b["dR"])):
        base = c[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            hstep = 1e-6 * max(1.0, abs(base[idx]))
            cp = dict(c)
            arr = base.copy(); arr[idx] += hstep; cp[name] = arr
            lp = loss(cp)
            arr = base.copy(); arr[idx] -= hstep; cp[name] = arr
            lm = loss(cp)
            fd[idx] = (lp - lm) / (2 * hstep)
        _close(grad, fd, 1e-7, f"dy_in: d{name} vs finite differences")


# ------------------------------------------------------------------- bf16 pins

def pin_bf16_rne(O):
    """Known values, ties to even, one rounding from float64, range ends, and
    agreement with torch's float32 -> bfloat16 conversion (round-to-nearest-even)
    on values that are exact in float32."""
    import torch
    cases = {
        1.0: 1.0,
        1.0 + 2.0 ** -8: 1.0,                           # tie -> even (1.0)
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,           # tie -> even (mantissa 2)
        1.0 + 2.0 ** -8 + 2.0 ** -40: 1.0 + 2.0 ** -7,  # above the tie: one rounding from f64
        -1.0 - 2.0 ** -8 - 2.0 ** -40: -1.0 - 2.0 ** -7,
        2.0 ** -130 + 2.0 ** -134: 2.0 ** -130,          # subnormal spacing 2^-133
        3.0 * 2.0 ** -134: 2.0 ** -132,                  # 1.5 steps -> tie -> even (2 steps)
        float(np.ldexp(255.0, 120)): float(np.ldexp(255.0, 120)),
        float(np.ldexp(511.0, 119)): math.inf,           # rounds up past the largest value
        0.0: 0.0,
    }
    for x, want in cases.items():
        g = float(O.bf16_rne(np.array([x]))[0])
        assert g == want, f"bf16_rne({x!r}) = {g!r}, want {want!r}"
    v = _rng(41).standard_normal(20000).astype(np.float32) * np.float32(37.0)
    t = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_rne(v.astype(np.float64)), t), "bf16_rne vs torch"


# ------------------------------------------------------------------ MXFP8 pins

def _e4m3_table():
    """All finite E4M3 (FN) values by code, built by pure-Python loops from the
    format's bit fields (sign, 4 exponent bits with bias 7, 3 mantissa bits)."""
    tab = {}
    for code in range(256):
        if code & 0x7F == 0x7F:
            continue
        e, m = (code >> 3) & 15, code & 7
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        tab[code] = -mag if code & 0x80 else mag
    return tab


def _e4m3_nearest(x, tab):
    """Brute force: the finite code nearest to x (|x| clamped to 448), ties to
    the even mantissa; the sign of x is kept for zero."""
    a = min(abs(x), 448.0)
    best = None
    for code, v in tab.items():
        if code & 0x80:
            continue
        dv = abs(v - a)
        if best is None or dv < best[0] or (dv == best[0] and (code & 1) == 0):
            best = (dv, code)
    code = best[1]
    return code | 0x80 if (x < 0 or (x == 0 and math.copysign(1.0, x) < 0)) else code


def _shared_exp_loop(amax):
    """floor(log2(amax)) - 8 clamped to [-127, 127] by repeated halving and
    doubling (no frexp or log); -127 for amax == 0."""
    if amax == 0:
        return -127
    e = 0
    while amax >= 2.0 ** (e + 1):
        e += 1
    while amax < 2.0 ** e:
        e -= 1
    return max(-127, min(127, e - 8))


def pin_e4m3_codes(O):
    """E4M3 (FN) decoding against the bit fields (pure Python) and torch's
    float8_e4m3fn on all 256 codes; known values; encoding against brute-force
    nearest-code search (ties to even, saturation at 448) and against torch's
    float32 -> float8_e4m3fn conversion (round to nearest even) up to 464."""
    import torch
    tab = _e4m3_table()
    codes = np.arange(256, dtype=np.uint8)
    dec = O.e4m3_decode(codes)
    for c in range(256):
        if c in tab:
            assert dec[c] == tab[c] and math.copysign(1, dec[c]) == math.copysign(1, tab[c]), f"decode {c:#x}"
        else:
            assert np.isnan(dec[c]), f"decode {c:#x} should be NaN"
    t = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = ~np.isnan(t)
    assert np.array_equal(np.isnan(dec), ~fin) and np.array_equal(dec[fin], t[fin]), "decode vs torch"
    for c, v in ((0x38, 1.0), (0x7E, 448.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6), (0x07, 7 * 2.0 ** -9),
                 (0xC0, -2.0), (0x78, 256.0)):
        assert dec[c] == v, f"decode {c:#x} = {dec[c]!r}, want {v!r}"
    g = _rng(81)
    pos = sorted(v for c, v in tab.items() if not c & 0x80)
    xs = [0.0, -0.0, 448.0, 449.0, 463.9, 464.0, 465.0, 479.0, 480.0, 1e6, -1e6, 2.0 ** -10, 2.0 ** -11,
          3 * 2.0 ** -10, 5 * 2.0 ** -10]
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (a + b) / 2
        xs += [mid, -mid, mid * (1 + 1e-12), mid * (1 - 1e-12)]
    xs += list(g.uniform(-500, 500, 200)) + list(g.uniform(-0.05, 0.05, 200))
    enc = O.e4m3_encode(np.array(xs))
    for x, c in zip(xs, enc):
        want = _e4m3_nearest(x, tab)
        assert int(c) == want, f"e4m3_encode({x!r}) = {int(c):#x}, want {want:#x}"
    v = (g.standard_normal(50000) * np.exp2(g.integers(-12, 9, 50000))).astype(np.float32)
    v = v[np.abs(v) <= 464]      # above 464 torch rounds to 480, which E4M3 FN spends on NaN
    tt = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(v.astype(np.float64)), tt), "e4m3_encode vs torch"


def pin_mx_quantize(O):
    """MXFP8 block quantisation: E8M0 decoding; hand-worked blocks (all ones,
    amax 448, saturation at 500, an all-zero block, a tiny block whose shared
    exponent clamps at -127); brute force (scale by halving/doubling loops,
    codes by nearest-code search) on random blocks; exact round trip of blocks
    that are MXFP8 values; the element error bound of one E4M3 rounding."""
    assert O.e8m0_decode(np.array([0], np.uint8))[0] == 2.0 ** -127
    assert O.e8m0_decode(np.array([127], np.uint8))[0] == 1.0
    assert O.e8m0_decode(np.array([254], np.uint8))[0] == 2.0 ** 127
    assert np.isnan(O.e8m0_decode(np.array([255], np.uint8))[0])
    blk = np.ones((1, 32))
    q, s = O.mx_quantize(blk)
    assert s[0, 0] == 119 and np.all(q == 0x78), "all-ones block: 2^-8 scale, code 256"
    blk = np.zeros((1, 32)); blk[0, 0] = 448.0; blk[0, 1] = -1.0; blk[0, 2] = 500.0 / 512 * 448
    q, s = O.mx_quantize(blk)
    assert s[0, 0] == 127 and q[0, 0] == 0x7E and q[0, 1] == 0xB8, "amax 448: scale 1"
    blk[0, 3] = 500.0
    q, s = O.mx_quantize(blk)
    assert s[0, 0] == 127 and q[0, 3] == 0x7E, "500 saturates to 448 under scale 1"
    q, s = O.mx_quantize(np.zeros((2, 64)))
    assert np.all(s == 0) and np.all(q == 0), "zero blocks"
    q, s = O.mx_quantize(np.full((1, 32), 2.0 ** -130))
    assert s[0, 0] == 0 and np.all(q == 0x20), "clamped shared exponent: 2^-130 / 2^-127 = 2^-3"
    tab = _e4m3_table()
    g = _rng(82)
    V = g.standard_normal((3, 96)) * np.exp2(g.integers(-20, 20, (3, 1)))
    V[1, 32:64] = 0.0
    q, s = O.mx_quantize(V)
    for i in range(3):
        for b in range(3):
            blkv = [float(x) for x in V[i, 32 * b:32 * b + 32]]
            e = _shared_exp_loop(max(abs(x) for x in blkv))
            assert int(s[i, b]) == e + 127, f"scale of block ({i},{b})"
            for j, x in enumerate(blkv):
                assert int(q[i, 32 * b + j]) == _e4m3_nearest(x / 2.0 ** e, tab), f"code ({i},{32 * b + j})"
    # MXFP8 values round-trip exactly (a code with exponent field 15 and
    # mantissa <= 6 sets the block maximum)
    codes = g.integers(0, 0x7F, (4, 64)).astype(np.uint8) | (g.integers(0, 2, (4, 64)) << 7).astype(np.uint8)
    codes[codes & 0x7F == 0x7F] = 0x10
    codes[:, ::32] = 0x78 | (codes[:, ::32] & 0x80)
    codes[(codes & 0x78) == 0x78] &= 0xFE                  # exponent field 15: mantissa <= 6 (no 480)
    codes[(codes & 0x7F) == 0x7E] = 0x7C
    scales = g.integers(100, 150, (4, 2)).astype(np.uint8)
    V = O.mx_dequantize(codes, scales)
    q, s = O.mx_quantize(V)
    assert np.array_equal(s, scales) and np.array_equal(q, codes), "MXFP8 values must round-trip"
    V = g.standard_normal((8, 256)) * 3.0
    q, s = O.mx_quantize(V)
    D = O.mx_dequantize(q, s)
    sc = np.repeat(O.e8m0_decode(s), 32, axis=1)
    u = np.abs(V) / sc
    bound = np.where(u >= 2.0 ** -6, 2.0 ** -4 * np.abs(V), 2.0 ** -10 * sc)
    bound = np.where(u > 448.0, np.abs(V) - 448.0 * sc + 1e-300, bound)
    assert np.all(np.abs(D - V) <= bound * (1 + 1e-12)), "one E4M3 rounding per element"
    assert np.all(u < 512.0) and np.all(np.max(u.reshape(8, 8, 32), axis=2) >= 256.0), "block max lands in [256, 512)"


def _mx8_case(seed, M, K, d, N, eps=1e-6):
    g = _rng(seed)
    X = g.standard_normal((M, K))
    W1t = g.standard_normal((d, K)) / math.sqrt(K)
    W2t = g.standard_normal((N, d)) / math.sqrt(d)
    return dict(X=X, W1t=W1t, W2t=W2t, R=g.standard_normal((M, d)), gamma=1 + 0.1 * g.standard_normal(d),
                eps=eps)


def _mx8_quantised(O, c):
    Xq, Xs = O.mx_quantize(c["X"])
    W1q, W1s = O.mx_quantize(c["W1t"])
    W2q, W2s = O.mx_quantize(c["W2t"])
    return Xq, Xs, W1q, W1s, W2q, W2s


def pin_fwd_mx8_exact(O):
    """With W1 = 0 and gamma = 1, y = R; R made of MXFP8 values makes the
    quantisation of y gamma exact, so z and r must equal the real-valued
    forward (ref_fwd, itself pinned) of the dequantised weights exactly, up to
    float64 rounding: this fixes r applied after the second GEMM, on the
    unquantised y gamma."""
    g = _rng(83)
    M, K, d, N = 5, 64, 96, 7
    Xq, Xs = O.mx_quantize(g.standard_normal((M, K)))
    W1q = np.zeros((d, K), np.uint8); W1s = np.full((d, K // 32), 127, np.uint8)
    codes = g.integers(0, 0x7E, (M, d)).astype(np.uint8) | (g.integers(0, 2, (M, d)) << 7).astype(np.uint8)
    codes[codes & 0x7F == 0x7F] = 0x11
    codes[codes == 0x80] = 0x00                             # y = 0 + R turns -0 into +0
    codes[:, ::32] = 0x70 | (codes[:, ::32] & 0x80)         # block max 128..: exponent field 14
    codes[:, 1::32] = 0x78 | (codes[:, 1::32] & 0x80)       # exponent field 15, mantissa 0
    scales = g.integers(115, 130, (M, d // 32)).astype(np.uint8)
    R = O.mx_dequantize(codes, scales)
    W2q, W2s = O.mx_quantize(g.standard_normal((N, d)))
    out = O.ref_fwd_mx8(Xq, Xs, W1q, W1s, R, np.ones(d), W2q, W2s, 1e-6)
    ref = O.ref_fwd(np.zeros((M, K)), np.zeros((K, d)), R, np.ones(d), O.mx_dequantize(W2q, W2s).T, 1e-6)
    assert np.array_equal(out["yg_q"], codes) and np.array_equal(out["yg_s"], scales), "exact quantisation"
    _close(out["z"], ref["z"], 1e-13, "mx8 exact z")
    _close(out["r"], ref["r"], 1e-13, "mx8 exact r")


def pin_fwd_mx8_bruteforce(O):
    """Pure-Python loops on a tiny case: dequantise the operands from their
    bit fields, y = X W1^T + R, r, quantise y*gamma per 32-block by the loop
    scale and nearest-code search, z = r * (q W2^T)."""
    tab = _e4m3_table()
    c = _mx8_case(84, 3, 64, 64, 4)
    Xq, Xs, W1q, W1s, W2q, W2s = _mx8_quantised(O, c)
    M, K, d, N = 3, 64, 64, 4

    def deq(codes, scales, i, k):
        return tab[int(codes[i, k])] * 2.0 ** (int(scales[i, k // 32]) - 127)

    out = O.ref_fwd_mx8(Xq, Xs, W1q, W1s, c["R"], c["gamma"], W2q, W2s, c["eps"])
    for i in range(M):
        y = [sum(deq(Xq, Xs, i, k) * deq(W1q, W1s, j, k) for k in range(K)) + c["R"][i, j] for j in range(d)]
        r = 1.0 / math.sqrt(sum(v * v for v in y) / d + c["eps"])
        assert abs(out["r"][i] - r) <= 1e-12 * r, "mx8 r"
        hq = []
        for b in range(d // 32):
            blk = [y[j] * c["gamma"][j] for j in range(32 * b, 32 * b + 32)]
            e = _shared_exp_loop(max(abs(v) for v in blk))
            hq += [tab[_e4m3_nearest(v / 2.0 ** e, tab)] * 2.0 ** e for v in blk]
        for n in range(N):
            z = r * sum(hq[j] * deq(W2q, W2s, n, j) for j in range(d))
            assert abs(out["z"][i, n] - z) <= 1e-12 * max(1.0, abs(z)), f"mx8 z[{i},{n}]"
        assert max(abs(out["y"][i, j] - y[j]) for j in range(d)) <= 1e-12, "mx8 y"


def pin_fwd_mx8_rows(O):
    """The row form equals the matching rows of the full forward."""
    c = _mx8_case(85, 40, 64, 96, 24)
    Xq, Xs, W1q, W1s, W2q, W2s = _mx8_quantised(O, c)
    full = O.ref_fwd_mx8(Xq, Xs, W1q, W1s, c["R"], c["gamma"], W2q, W2s, c["eps"])
    rows = np.array([0, 7, 39, 20])
    part = O.ref_fwd_mx8_rows(Xq, Xs, W1q, W1s, c["R"], c["gamma"], W2q, W2s, c["eps"], rows)
    for k in ("y", "r", "z", "yg_q", "yg_s"):
        assert np.array_equal(part[k], full[k][rows]), f"mx8 rows {k}"


def _bf16_loop(x):
    """Nearest bfloat16 value of a float (8 significant bits, ties to even), by
    frexp and Python's round (banker's rounding) - no numpy, no oracle code."""
    if x == 0.0 or not math.isfinite(x):
        return x
    m, e = math.frexp(x)                      # x = m 2**e, 0.5 <= |m| < 1
    e = max(e, -125)                          # below 2**-126 the spacing stays 2**-133
    return math.ldexp(round(math.ldexp(x, 8 - e)), e - 8)


def _mx_block_loop(vals, tab):
    """MXFP8 of one 32-block by loops: scale exponent from the block max,
    nearest code per element; returns the dequantised values."""
    e = _shared_exp_loop(max(abs(v) for v in vals))
    return [tab[_e4m3_nearest(v / 2.0 ** e, tab)] * 2.0 ** e for v in vals]


def _mx_matmul_loop(A, B, tab):
    """A [m][k] B [k][n] with A's rows and B's columns quantised in 32-blocks
    along k, by loops."""
    m, k, n = len(A), len(A[0]), len(B[0])
    Aq = [sum((_mx_block_loop(A[i][b:b + 32], tab) for b in range(0, k, 32)), []) for i in range(m)]
    Bq = [sum((_mx_block_loop([B[kk][j] for kk in range(b, b + 32)], tab) for b in range(0, k, 32)), [])
          for j in range(n)]
    return [[sum(Aq[i][kk] * Bq[j][kk] for kk in range(k)) for j in range(n)] for i in range(m)]


def _mx_grid(g, shape):
    """Values exactly representable in MXFP8 along the last axis: per 32-block
    a power of two 2**e and E4M3 values v (|v| <= 448) with the block's largest
    |v| in [256, 448], so that the block maximum gives back exponent e."""
    tab = _e4m3_table()
    vals = np.array(sorted(v for v in tab.values()))
    top = vals[(np.abs(vals) >= 256.0)]
    nb = shape[-1] // 32
    out = g.choice(vals[np.abs(vals) < 256.0], size=shape[:-1] + (nb, 32))
    lead = g.integers(0, 32, size=shape[:-1] + (nb,))
    np.put_along_axis(out, lead[..., None], g.choice(top, size=shape[:-1] + (nb, 1)), axis=-1)
    blk = 2.0 ** g.integers(-14, -6, size=shape[:-1] + (nb, 1))
    return (out * blk).reshape(shape)


def pin_mx_matmul(O):
    """The MXFP8 product against loops (each operand quantised along the
    contraction index from the format's bit fields); grid-exact operands give
    the exact product; the product of the transposes is the transpose."""
    tab = _e4m3_table()
    g = _rng(90)
    A = g.standard_normal((3, 64)) * 3.0
    B = g.standard_normal((64, 2)) * 0.2
    A[1, 40] = 0.0
    got = O.mx_matmul(A, B)
    want = np.array(_mx_matmul_loop(A.tolist(), B.tolist(), tab))
    _close(got, want, 1e-12, "mx_matmul vs loops")
    Ag, Bg = _mx_grid(g, (5, 96)), _mx_grid(g, (7, 96)).T
    _close(O.mx_matmul(Ag, Bg), Ag @ Bg, 1e-13, "mx_matmul of grid-exact operands")
    C = g.standard_normal((64, 4))
    assert np.array_equal(O.mx_matmul(A, C), O.mx_matmul(C.T, A.T).T), "mx_matmul transposition"


def _bwd_mx8_case(seed, M, K, d, N):
    g = _rng(seed)
    return dict(X=g.standard_normal((M, K)), W1=g.standard_normal((K, d)) / math.sqrt(K),
                gamma=1 + 0.1 * g.standard_normal(d), W2=g.standard_normal((d, N)) / math.sqrt(d),
                y=g.standard_normal((M, d)) * 1.5, dz=g.standard_normal((M, N)))


def _bwd_mx8_loops(X, W1, gamma, W2, y, r, dz, dy_in, tab):
    """The MXFP8 block backward by loops (lists in, lists out): dh, dgamma, c,
    the stored dy, dW2, dX, dW1."""
    M, d, N = len(y), len(y[0]), len(dz[0])
    W2T = [[W2[j][k] for j in range(d)] for k in range(N)]          # [N][d]: the product dz W2^T
    dh = _mx_matmul_loop(dz, W2T, tab)
    dgam = [sum(dh[i][j] * r[i] * y[i][j] for i in range(M)) for j in range(d)]
    dn = [[dh[i][j] * gamma[j] for j in range(d)] for i in range(M)]
    s_ = [sum(dn[i][j] * y[i][j] for j in range(d)) for i in range(M)]
    cc = [r[i] ** 3 * s_[i] / d for i in range(M)]
    dy = [[_bf16_loop(r[i] * _bf16_loop(dn[i][j]) - cc[i] * y[i][j] + (dy_in[i][j] if dy_in else 0.0))
           for j in range(d)] for i in range(M)]
    nT = [[_bf16_loop(r[i] * y[i][j]) for i in range(M)] for j in range(d)]
    dW2 = _mx_matmul_loop(nT, dz, tab)
    dW2 = [[dW2[j][k] * gamma[j] for k in range(N)] for j in range(d)]
    W1T = [[W1[k][j] for k in range(len(W1))] for j in range(d)]
    XT = [[X[i][k] for i in range(M)] for k in range(len(X[0]))]
    return {"dh": dh, "dgamma": dgam, "c": cc, "dy": dy, "dW2": dW2,
            "dX": _mx_matmul_loop(dy, W1T, tab), "dW1": _mx_matmul_loop(XT, dy, tab)}


def pin_bwd_mx8_bruteforce(O):
    """The MXFP8 backward by pure-Python loops on a tiny case (every dimension
    two 32-blocks): each GEMM's operands quantised along its contraction
    index, dn, n and dy rounded to bf16 before they are quantised."""
    tab = _e4m3_table()
    M = K = d = N = 64
    c = _bwd_mx8_case(91, M, K, d, N)
    y = c["y"]
    r = 1.0 / np.sqrt(np.mean(y * y, axis=1) + 1e-6)
    out = O.ref_bwd_mx8(c["X"], c["W1"], c["gamma"], c["W2"], y, r, c["dz"])
    L = _bwd_mx8_loops(c["X"].tolist(), c["W1"].tolist(), c["gamma"].tolist(), c["W2"].tolist(), y.tolist(),
                       r.tolist(), c["dz"].tolist(), None, tab)
    _close(out["dh"], np.array(L["dh"]), 1e-12, "mx8 bwd dh")
    _close(out["dgamma"], np.array(L["dgamma"]), 1e-12, "mx8 bwd dgamma")
    _close(out["c"], np.array(L["c"]), 1e-12, "mx8 bwd c")
    _close(O.bf16_rne(out["dy"]), np.array(L["dy"]), 1e-12, "mx8 bwd dy (stored)")
    _close(out["dW2"], np.array(L["dW2"]), 1e-12, "mx8 bwd dW2")
    _close(out["dX"], np.array(L["dX"]), 1e-12, "mx8 bwd dX")
    _close(out["dW1"], np.array(L["dW1"]), 1e-12, "mx8 bwd dW1")


def pin_bwd_mx8_grid_exact(O):
    """With dz and W2 on the MXFP8 grid the dh product is exact, so dh,
    dgamma, s and c equal those of the unquantised backward (ref_bwd, pinned by
    finite differences and torch autograd); with every quantised operand on
    the grid and the identity as storage, dX, dW1 and dW2 equal ref_bwd's
    products of the same operands."""
    g = _rng(92)
    M, K, d, N = 64, 32, 64, 96
    c = _bwd_mx8_case(93, M, K, d, N)
    dz = _mx_grid(g, (M, N))
    W2 = _mx_grid(g, (d, N))
    y = c["y"]
    r = 1.0 / np.sqrt(np.mean(y * y, axis=1) + 1e-6)
    q = O.ref_bwd_mx8(c["X"], c["W1"], c["gamma"], W2, y, r, dz, store=lambda v: v)
    e = O.ref_bwd(c["X"], c["W1"], c["gamma"], W2, y, r, dz)
    for k in ("dh", "dgamma", "s", "c"):
        _close(q[k], e[k], 1e-12, f"mx8 bwd {k} on grid operands")
    _close(q["dR"], e["dR"], 1e-12, "mx8 bwd dR (identity storage)")


def pin_bwd_mx8_sampled(O):
    """The sampled form equals slices of the full MXFP8 backward."""
    M, K, d, N = 96, 64, 64, 128
    c = _bwd_mx8_case(94, M, K, d, N)
    y = O.bf16_rne(c["y"])
    r = 1.0 / np.sqrt(np.mean(y * y, axis=1) + 1e-6)
    full = O.ref_bwd_mx8(c["X"], c["W1"], c["gamma"], c["W2"], y, r, c["dz"])
    rows, cd, cn = np.array([0, 17, 95]), np.array([1, 63]), np.array([0, 5, 127])
    sm = O.ref_bwd_mx8_sampled(c["X"], c["W1"], c["gamma"], c["W2"], y, r, c["dz"], rows, cd, cn)
    _close(sm["dX_rows"], full["dX"][rows], 1e-12, "mx8 sampled dX rows")
    _close(sm["dR_rows"], full["dR"][rows], 1e-12, "mx8 sampled dR rows")
    _close(sm["dW1_cols"], full["dW1"][:, cd], 1e-12, "mx8 sampled dW1 cols")
    _close(sm["dW2_cols"], full["dW2"][:, cn], 1e-12, "mx8 sampled dW2 cols")
    _close(sm["dgamma"], full["dgamma"], 1e-12, "mx8 sampled dgamma")


def pin_bwd_mx8_row_blocks(O):
    """MXFP8 blocks along M are local: with dz zero outside a few rows, dn,
    s, c and dy vanish there, so dX and dR are zero on every other row, and
    the backward on the whole aligned 32-row blocks holding those rows alone
    equals the full backward exactly (their quantisation along M is the same
    inside the full matrix).  The GPU test at the largest row count relies on
    this."""
    M, K, d, N = 512, 32, 64, 96
    c = _bwd_mx8_case(95, M, K, d, N)
    y = O.bf16_rne(c["y"])
    r = 1.0 / np.sqrt(np.mean(y * y, axis=1) + 1e-6)
    hot = np.array([0, 45, 200, M - 100, M - 1])
    dz = np.zeros((M, N))
    dz[hot] = c["dz"][hot]
    full = O.ref_bwd_mx8(c["X"], c["W1"], c["gamma"], c["W2"], y, r, dz)
    blocks = np.unique(hot // 32)
    rows = (blocks[:, None] * 32 + np.arange(32)[None, :]).ravel()
    rest = np.setdiff1d(np.arange(M), rows)
    sub = O.ref_bwd_mx8(c["X"][rows], c["W1"], c["gamma"], c["W2"], y[rows], r[rows], dz[rows])
    if np.any(full["dX"][rest]) or np.any(full["dR"][rest]):
        raise AssertionError("mx8 bwd: dX / dR nonzero outside the rows with a gradient")
    for k in ("dW1", "dW2", "dgamma"):
        _close(sub[k], full[k], 1e-12, f"mx8 bwd {k} from the gathered row blocks")
    _close(sub["dX"], full["dX"][rows], 1e-12, "mx8 bwd dX on the gathered row blocks")
    _close(sub["dR"], full["dR"][rows], 1e-12, "mx8 bwd dR on the gathered row blocks")


def _swiglu_mx8_case(seed, M, d, F):
    g = _rng(seed)
    return dict(X=g.standard_normal((M, d)), W=g.standard_normal((d, 2 * F)) / math.sqrt(d),
                Wd=g.standard_normal((F, d)) / math.sqrt(F), dz=g.standard_normal((M, d)))


def pin_swiglu_mx8_bruteforce(O):
    """The MXFP8 SwiGLU forward and backward by pure-Python loops (every
    dimension whole 32-blocks): each GEMM's operands quantised along its
    contraction index from the format's bit fields, a = silu(g) u from the
    unrounded gu, a and dgu rounded to bf16 before they are quantised."""
    tab = _e4m3_table()
    M, d, F = 64, 64, 32
    c = _swiglu_mx8_case(95, M, d, F)
    X, W, Wd, dz = (c[k].tolist() for k in ("X", "W", "Wd", "dz"))
    sig = lambda t: 1.0 / (1.0 + math.exp(-t))  # noqa: E731
    gu = _mx_matmul_loop(X, W, tab)
    a = [[gu[i][j] * sig(gu[i][j]) * gu[i][F + j] for j in range(F)] for i in range(M)]
    a_s = [[_bf16_loop(v) for v in row] for row in a]
    z = _mx_matmul_loop(a_s, Wd, tab)
    f = O.ref_swiglu_fwd_mx8(c["X"], c["W"], c["Wd"])
    _close(f["gu"], np.array(gu), 1e-12, "swiglu mx8 gu vs loops")
    _close(f["a"], np.array(a), 1e-12, "swiglu mx8 a vs loops")
    _close(f["z"], np.array(z), 1e-12, "swiglu mx8 z vs loops")
    gu_s = [[_bf16_loop(v) for v in row] for row in gu]
    b = O.ref_swiglu_bwd_mx8(c["X"], c["W"], c["Wd"], np.array(gu_s), np.array(a_s), c["dz"])
    WdT = [[Wd[j][k] for j in range(F)] for k in range(d)]            # [d][F]
    da = _mx_matmul_loop(dz, WdT, tab)
    dgu = []
    for i in range(M):
        row_g, row_u = [], []
        for j in range(F):
            g_, u_ = gu_s[i][j], gu_s[i][F + j]
            sg = sig(g_)
            row_g.append(da[i][j] * u_ * sg * (1.0 + g_ * (1.0 - sg)))
            row_u.append(da[i][j] * g_ * sg)
        dgu.append(row_g + row_u)
    dgu_s = [[_bf16_loop(v) for v in row] for row in dgu]
    aT = [[a_s[i][j] for i in range(M)] for j in range(F)]
    WT = [[W[k][j] for k in range(d)] for j in range(2 * F)]
    XT = [[X[i][k] for i in range(M)] for k in range(d)]
    _close(b["da"], np.array(da), 1e-12, "swiglu mx8 da vs loops")
    _close(b["dgu"], np.array(dgu), 1e-12, "swiglu mx8 dgu vs loops")
    _close(b["dWd"], np.array(_mx_matmul_loop(aT, dz, tab)), 1e-12, "swiglu mx8 dWd vs loops")
    _close(b["dX"], np.array(_mx_matmul_loop(dgu_s, WT, tab)), 1e-12, "swiglu mx8 dX vs loops")
    _close(b["dW"], np.array(_mx_matmul_loop(XT, dgu_s, tab)), 1e-12, "swiglu mx8 dW vs loops")


def _mx_grid_both(g, shape):
    """A matrix exactly representable in MXFP8 along both axes: E4M3 values
    times one power of two, with |v| = 256 wherever i % 32 == j % 32, so that
    every 32-block of a row and of a column has its maximum in [256, 448]."""
    tab = _e4m3_table()
    vals = np.array(sorted(v for v in tab.values() if abs(v) <= 256.0))
    out = g.choice(vals, size=shape)
    i, j = np.indices(shape)
    out[(i % 32) == (j % 32)] = 256.0 * g.choice([-1.0, 1.0], size=int(np.sum((i % 32) == (j % 32))))
    return out * 2.0 ** -12


def pin_swiglu_mx8_row_blocks(O):
    """As pin_bwd_mx8_row_blocks for the SwiGLU block: with dz zero outside
    a few rows, da, dgu and dX vanish there, and the backward on the whole
    aligned 32-row blocks holding those rows equals the full one."""
    g = _rng(96)
    M, d, F = 512, 64, 96
    c = _swiglu_mx8_case(97, M, d, F)
    f = O.ref_swiglu_fwd_mx8(c["X"], c["W"], c["Wd"])
    gu, a = O.bf16_rne(f["gu"]), O.bf16_rne(f["a"])
    hot = np.array([0, 45, 200, M - 100, M - 1])
    dz = np.zeros((M, d))
    dz[hot] = g.standard_normal((len(hot), d))
    full = O.ref_swiglu_bwd_mx8(c["X"], c["W"], c["Wd"], gu, a, dz)
    blocks = np.unique(hot // 32)
    rows = (blocks[:, None] * 32 + np.arange(32)[None, :]).ravel()
    rest = np.setdiff1d(np.arange(M), rows)
    sub = O.ref_swiglu_bwd_mx8(c["X"][rows], c["W"], c["Wd"], gu[rows], a[rows], dz[rows])
    if np.any(full["dX"][rest]) or np.any(full["dgu"][rest]):
        raise AssertionError("swiglu mx8 bwd: dX / dgu nonzero outside the rows with a gradient")
    for k in ("dW", "dWd"):
        _close(sub[k], full[k], 1e-12, f"swiglu mx8 bwd {k} from the gathered row blocks")
    _close(sub["dX"], full["dX"][rows], 1e-12, "swiglu mx8 bwd dX on the gathered row blocks")


def pin_swiglu_mx8_grid_exact(O):
    """With operands on the MXFP8 grid the quantised products are exact, so
    the MXFP8 SwiGLU reduces to the pinned ref_swiglu_fwd / ref_swiglu_bwd:
    gu and a (X, W on the grid along d); da, dgu (dz, Wd on the grid along d)
    and dWd (the saved a and dz on the grid along M)."""
    g = _rng(96)
    M, d, F = 64, 64, 96
    X = _mx_grid(g, (M, d))
    W = _mx_grid(g, (2 * F, d)).T.copy()
    Wd = _mx_grid(g, (F, d))
    dz = _mx_grid_both(g, (M, d))
    a_saved = _mx_grid(g, (F, M)).T.copy()
    q = O.ref_swiglu_fwd_mx8(X, W, Wd, store=lambda v: v)
    e = O.ref_swiglu_fwd(X, W, Wd)
    _close(q["gu"], e["gu"], 1e-13, "swiglu mx8 gu on grid operands")
    _close(q["a"], e["a"], 1e-13, "swiglu mx8 a on grid operands")
    qb = O.ref_swiglu_bwd_mx8(X, W, Wd, e["gu"], a_saved, dz, store=lambda v: v)
    eb = O.ref_swiglu_bwd(X, W, Wd, e["gu"], a_saved, dz)
    for k in ("da", "dgu", "dWd"):
        _close(qb[k], eb[k], 1e-13, f"swiglu mx8 {k} on grid operands")


def pin_swiglu_mx8_sampled(O):
    """The sampled forms equal slices of the full MXFP8 SwiGLU forward and
    backward (with the saved gu and a rounded to bf16)."""
    M, d, F = 96, 64, 64
    c = _swiglu_mx8_case(97, M, d, F)
    f = O.ref_swiglu_fwd_mx8(c["X"], c["W"], c["Wd"])
    rows = np.array([0, 33, 95])
    fr = O.ref_swiglu_fwd_mx8_rows(c["X"], c["W"], c["Wd"], rows)
    for k in ("gu", "a", "z"):
        _close(fr[k], f[k][rows], 1e-13, f"swiglu mx8 rows {k}")
    b = O.ref_swiglu_bwd_mx8(c["X"], c["W"], c["Wd"], O.bf16_rne(f["gu"]), O.bf16_rne(f["a"]), c["dz"])
    cols_W, rows_Wd = np.array([0, 63, 64, 127]), np.array([1, 62])
    sm = O.ref_swiglu_bwd_mx8_sampled(c["X"], c["W"], c["Wd"], c["dz"], rows, cols_W, rows_Wd)
    _close(sm["dX_rows"], b["dX"][rows], 1e-12, "swiglu mx8 sampled dX rows")
    _close(sm["dgu_rows"], b["dgu"][rows], 1e-12, "swiglu mx8 sampled dgu rows")
    _close(sm["dW_cols"], b["dW"][:, cols_W], 1e-12, "swiglu mx8 sampled dW cols")
    _close(sm["dWd_rows"], b["dWd"][rows_Wd], 1e-12, "swiglu mx8 sampled dWd rows")


def _mlp_mx8_case(seed, M, K, d, F):
    g = _rng(seed)
    return dict(X=g.standard_normal((M, K)), W1=g.standard_normal((K, d)) / math.sqrt(K),
                R=g.standard_normal((M, d)), gamma=1 + 0.1 * g.standard_normal(d),
                W=g.standard_normal((d, 2 * F)) / math.sqrt(d), Wd=g.standard_normal((F, d)) / math.sqrt(F),
                dz=g.standard_normal((M, d)), dy_in=0.3 * g.standard_normal((M, d)), eps=1e-6)


def pin_mlp_mx8_bruteforce(O):
    """The MXFP8 MLP sub-layer by pure-Python loops (M = 64, K = d = F = 32):
    y from the MXFP8 product, r, gu = r (y gamma quantised along d) W, a, z
    from the stored a; the backward's SwiGLU part, then the block backward by
    loops with dgu (stored) as its output gradient and dy_in added to dy."""
    tab = _e4m3_table()
    M, K, d, F = 64, 32, 32, 32
    c = _mlp_mx8_case(98, M, K, d, F)
    L = {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    sig = lambda t: 1.0 / (1.0 + math.exp(-t))  # noqa: E731
    xw = _mx_matmul_loop(L["X"], L["W1"], tab)
    y = [[xw[i][j] + L["R"][i][j] for j in range(d)] for i in range(M)]
    r = [1.0 / math.sqrt(sum(v * v for v in y[i]) / d + c["eps"]) for i in range(M)]
    yg = [[y[i][j] * L["gamma"][j] for j in range(d)] for i in range(M)]
    p = _mx_matmul_loop(yg, L["W"], tab)
    gu = [[r[i] * p[i][j] for j in range(2 * F)] for i in range(M)]
    a = [[gu[i][j] * sig(gu[i][j]) * gu[i][F + j] for j in range(F)] for i in range(M)]
    z = _mx_matmul_loop([[_bf16_loop(v) for v in row] for row in a], L["Wd"], tab)
    f = O.ref_mlp_fwd_mx8(c["X"], c["W1"], c["R"], c["gamma"], c["W"], c["Wd"], c["eps"])
    for k, v in (("y", y), ("r", r), ("gu", gu), ("a", a), ("z", z)):
        _close(f[k], np.array(v), 1e-12, f"mlp mx8 {k} vs loops")
    y_s = [[_bf16_loop(v) for v in row] for row in y]
    gu_s = [[_bf16_loop(v) for v in row] for row in gu]
    a_s = [[_bf16_loop(v) for v in row] for row in a]
    b = O.ref_mlp_bwd_mx8(c["X"], c["W1"], c["gamma"], c["W"], c["Wd"], np.array(y_s), np.array(r),
                          np.array(gu_s), np.array(a_s), c["dz"], c["dy_in"])
    WdT = [[L["Wd"][j][k] for j in range(F)] for k in range(d)]
    da = _mx_matmul_loop(L["dz"], WdT, tab)
    dgu = []
    for i in range(M):
        rg, ru = [], []
        for j in range(F):
            g_, u_ = gu_s[i][j], gu_s[i][F + j]
            sg = sig(g_)
            rg.append(da[i][j] * u_ * sg * (1.0 + g_ * (1.0 - sg)))
            ru.append(da[i][j] * g_ * sg)
        dgu.append(rg + ru)
    dgu_s = [[_bf16_loop(v) for v in row] for row in dgu]
    B = _bwd_mx8_loops(L["X"], L["W1"], L["gamma"], L["W"], y_s, r, dgu_s, L["dy_in"], tab)
    aT = [[a_s[i][j] for i in range(M)] for j in range(F)]
    _close(b["dgu"], np.array(dgu), 1e-12, "mlp mx8 dgu vs loops")
    _close(b["dWd"], np.array(_mx_matmul_loop(aT, L["dz"], tab)), 1e-12, "mlp mx8 dWd vs loops")
    _close(b["dgamma"], np.array(B["dgamma"]), 1e-12, "mlp mx8 dgamma vs loops")
    _close(O.bf16_rne(b["dR"]), np.array(B["dy"]), 1e-12, "mlp mx8 dR (stored) vs loops")
    for k, kk in (("dW", "dW2"), ("dX", "dX"), ("dW1", "dW1")):
        _close(b[k], np.array(B[kk]), 1e-12, f"mlp mx8 {k} vs loops")


def pin_mlp_mx8_grid_exact(O):
    """On the MXFP8 grid the MLP's quantised products are exact: X and W1 on
    the grid along K give ref_mlp_fwd's y and r; dz and Wd on it along d,
    the saved a and dz along M, give ref_mlp_bwd's da, dgu and dWd (with the
    same saved gu and identity storage); and with dy_in, dR moves by dy_in
    exactly (identity storage)."""
    g = _rng(99)
    M, K, d, F = 64, 64, 64, 64
    c = _mlp_mx8_case(100, M, K, d, F)
    X, W1 = _mx_grid(g, (M, K)), _mx_grid(g, (d, K)).T.copy()
    q = O.ref_mlp_fwd_mx8(X, W1, c["R"], c["gamma"], c["W"], c["Wd"], c["eps"], store=lambda v: v)
    e = O.ref_mlp_fwd(X, W1, c["R"], c["gamma"], c["W"], c["Wd"], c["eps"])
    _close(q["y"], e["y"], 1e-13, "mlp mx8 y on grid operands")
    _close(q["r"], e["r"], 1e-13, "mlp mx8 r on grid operands")
    dz = _mx_grid_both(g, (M, d))
    Wd = _mx_grid(g, (F, d))
    a_saved = _mx_grid(g, (F, M)).T.copy()
    gu = e["gu"]
    ident = lambda v: v  # noqa: E731
    qb = O.ref_mlp_bwd_mx8(X, W1, c["gamma"], c["W"], Wd, e["y"], e["r"], gu, a_saved, dz, None, ident)
    eb = O.ref_mlp_bwd(X, W1, c["gamma"], c["W"], Wd, e["y"], e["r"], gu, a_saved, dz)
    for k in ("da", "dgu", "dWd"):
        _close(qb[k], eb[k], 1e-13, f"mlp mx8 {k} on grid operands")
    qi = O.ref_mlp_bwd_mx8(X, W1, c["gamma"], c["W"], Wd, e["y"], e["r"], gu, a_saved, dz, c["dy_in"], ident)
    _close(qi["dR"] - qb["dR"], c["dy_in"], 1e-13, "mlp mx8 dR moves by dy_in")


def pin_mlp_mx8_sampled(O):
    """The row and sampled forms equal slices of the full MXFP8 MLP forward
    and backward."""
    M, K, d, F = 96, 64, 64, 64
    c = _mlp_mx8_case(101, M, K, d, F)
    f = O.ref_mlp_fwd_mx8(c["X"], c["W1"], c["R"], c["gamma"], c["W"], c["Wd"], c["eps"])
    rows = np.array([0, 45, 95])
    fr = O.ref_mlp_fwd_mx8_rows(c["X"], c["W1"], c["R"], c["gamma"], c["W"], c["Wd"], c["eps"], rows)
    for k in ("y", "r", "gu", "a", "z"):
        _close(fr[k], f[k][rows], 1e-13, f"mlp mx8 rows {k}")
    sv = {k: O.bf16_rne(f[k]) for k in ("y", "gu", "a")}
    b = O.ref_mlp_bwd_mx8(c["X"], c["W1"], c["gamma"], c["W"], c["Wd"], sv["y"], f["r"], sv["gu"], sv["a"],
                          c["dz"], c["dy_in"])
    cd, c2, rF = np.array([0, 63]), np.array([1, 64, 127]), np.array([3, 60])
    sm = O.ref_mlp_bwd_mx8_sampled(c["X"], c["W1"], c["gamma"], c["W"], c["Wd"], sv["y"], f["r"], sv["gu"],
                                   sv["a"], c["dz"], c["dy_in"], rows, cd, c2, rF)
    _close(sm["dX_rows"], b["dX"][rows], 1e-12, "mlp mx8 sampled dX rows")
    _close(sm["dR_rows"], b["dR"][rows], 1e-12, "mlp mx8 sampled dR rows")
    _close(sm["dW1_cols"], b["dW1"][:, cd], 1e-12, "mlp mx8 sampled dW1 cols")
    _close(sm["dW_cols"], b["dW"][:, c2], 1e-12, "mlp mx8 sampled dW cols")
    _close(sm["dWd_rows"], b["dWd"][rF], 1e-12, "mlp mx8 sampled dWd rows")
    _close(sm["dgamma"], b["dgamma"], 1e-12, "mlp mx8 sampled dgamma")


ALL_PINS = [
    pin_fwd_bruteforce, pin_fwd_torch_rmsnorm, pin_fwd_constant_rows,
    pin_fwd_scale_invariance, pin_partials, pin_rewrite_equals_unfused,
    pin_golden_coda, pin_bwd_finite_differences, pin_bwd_torch_autograd,
    pin_bwd_invariants, pin_sampled_forms, pin_swiglu_bruteforce,
    pin_swiglu_finite_differences, pin_swiglu_torch, pin_swiglu_invariants,
    pin_golden_swiglu, pin_swiglu_sampled, pin_bf16_rne, pin_mlp_finite_differences,
    pin_mlp_torch, pin_mlp_invariants, pin_mlp_sampled, pin_mlp_dgu_rounding,
    pin_mlp_stored_operand_bruteforce, pin_ce_torch, pin_ce_ignored_rows, pin_ce_finite_differences,
    pin_ce_closed_forms, pin_ce_invariants, pin_ce_partials, pin_ce_sampled,
    pin_rope_bruteforce, pin_rope_torch, pin_rope_finite_differences, pin_rope_properties,
    pin_rope_sampled,
    pin_bwd_dy_in_finite_differences, pin_e4m3_codes, pin_mx_quantize, pin_fwd_mx8_exact,
    pin_fwd_mx8_bruteforce, pin_fwd_mx8_rows, pin_mx_matmul, pin_bwd_mx8_bruteforce,
    pin_bwd_mx8_grid_exact, pin_bwd_mx8_sampled, pin_bwd_mx8_row_blocks, pin_swiglu_mx8_bruteforce,
    pin_swiglu_mx8_grid_exact, pin_swiglu_mx8_row_blocks,
    pin_swiglu_mx8_sampled, pin_mlp_mx8_bruteforce, pin_mlp_mx8_grid_exact, pin_mlp_mx8_sampled,
]

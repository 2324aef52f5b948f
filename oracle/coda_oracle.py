"""CPU oracle for the fused GEMM-Residual-RMSNorm-GEMM block and the SwiGLU
gate/up block: plain, unfused definitions in numpy float64.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import or call this module.  The library's
product path (its HIP kernels, C-ABI and Python binding) never imports it, and
this module imports nothing from the library.

Sources.  The pages are three news articles on the paper "CODA: Rewriting
Transformer Blocks as GEMM-Epilogue Programs":
  [JA]  toolin.ai blog, "CODA：LLMと初心者が光速のGPUカーネルを書けるようにする"
  [RU]  kucoin.com news flash (Russian) on the same paper
  [FR]  kucoin.com news flash (French) on the same paper
Their sections are cited by heading: [JA] 核心の洞察 = the insight section,
[RU] "CODA: В «Финале» спрятаны сокровища", [FR] "CODA : « La fin » cache
un trésor", [JA] 組み合わせ可能な5種類の「積み木」 / [RU] "Пять «кирпичиков»"
/ [FR] "Cinq « blocs »" = the five epilogue primitives.

What the pages fix, and the readings taken where they are silent:
  * GEMM-RMSNorm-GEMM: a GEMM, a residual add, RMS normalisation, then a second
    GEMM ([RU] insight section: the pattern runs a matmul, a residual add, RMS
    normalisation, another matmul).  The pages give no formula.  Reading: y =
    X W1 + R; r_i = (mean_j y_ij^2 + eps)^(-1/2), the mean over the normalised
    width d, eps inside the root; h = diag(r) y diag(gamma) (a plain scale by
    gamma, no bias); z = h W2.
  * The row scale r is one scalar per row and commutes with the second GEMM, so
    it can be applied after it; the first GEMM only leaves per-tile partial sums
    of squares that a small kernel combines ([JA] 核心の洞察; [RU] and [FR]
    insight sections).  ``ref_fwd_rewritten`` and ``ref_partials`` write that
    rewrite out; it reaches the same z up to rounding order.
  * The backward is the exact gradient of L = <dz, z>; the pages state a
    theorem that the backward inherits the forward's block-local structure but
    not its content ([RU]/[FR] insight sections).  ``ref_bwd`` is the
    hand-derived gradient of the definitions above, written unfused.
  * SwiGLU in the activation epilogue ([JA]/[RU]/[FR] primitives sections,
    "elementwise transform ... activation").  Reading: gu = X W with W =
    [W_gate | W_up] (gate columns first), a = silu(g) * u with silu(t) =
    t * sigmoid(t), z = a Wd.
  * Saved activations are stored for the backward ([JA]/[RU]/[FR] primitives
    sections, "matrix tile load/store ... saving intermediates").  Reading: the
    backward functions take the saved tensors (y and r; gu and a) as inputs, so
    a caller can pass them rounded to the storage dtype.
  * The two patterns chained as in a LLaMA MLP sub-layer (``ref_mlp_*``): the
    pages name both inside a transformer block (the residual add and RMS
    normalisation around a matmul, and SwiGLU as the activation epilogue,
    [RU]/[FR] insight and primitives sections).  Reading: the normalised h
    feeds the gate/up GEMM in place of the second GEMM, h W = [g | u], a =
    silu(g) u, z = a Wd; y is the residual stream, so its gradient may also
    receive a term dy_in from later layers, added to dy.
  * Cross-entropy over an LM-head GEMM (``ref_ce_*``): the pages' stateful
    epilogue primitive keeps a running max and sum of exponentials across the
    tiles of a row, which cross-entropy uses ([JA]/[RU]/[FR] primitives
    sections).  Reading: logits = h Wv; lse_i = log sum_j exp(logits_ij);
    loss_i = lse_i - logits_i,label_i (mean-free, one loss per row); the
    backward of L = sum_i dloss_i loss_i.  A label outside [0, V) marks an
    ignored row (loss 0, no gradient), the usual ignore-index convention.
  * A rotary-position epilogue on a QKV projection (``ref_rope_*``): the
    pages list position encodings among the elementwise transforms an
    epilogue can carry ([JA]/[RU]/[FR] primitives sections).  Reading: Y = X W,
    then the first N_rot columns (q and k) are rotated head by head (head
    width D) on the interleaved pairs (2i, 2i+1) by the angle p theta_i, theta_i
    = base^(-2i/D), p = row mod S (rows are S-token sequences one after
    another); the remaining columns (v) pass through.
  * An FP8 forward of the fused block (``ref_fwd_mx8``): the pages note that
    faster FP8/FP4 matrix units make the data movement around a GEMM relatively
    more costly ([JA] 課題：大モデル訓練の「手抜き税」; [RU] "Налог на лень
    при обучении больших моделей"; [FR] "Le « impôt de la paresse » pour
    l'entraînement des grands modèles") but fix no format.  Reading: OCP MXFP8 (E4M3 elements, one E8M0
    power-of-two scale per 32 along the contraction index), both GEMMs' operands
    in it; the second GEMM's operand is y diag(gamma) quantised by the first
    GEMM's epilogue, with r still applied after the second GEMM.
  * An FP8 backward of the block (``ref_bwd_mx8``): the same format; the
    gradient of the unquantised block (the forward's quantisation passes the
    gradient straight through), each backward GEMM on MXFP8 operands quantised
    along its own contraction index, the intermediates that feed a quantiser
    (dn, n, dy) held in bf16 first, as the bf16 backward stores them.
  * The SwiGLU block on MXFP8 (``ref_swiglu_fwd_mx8``, ``ref_swiglu_bwd_mx8``):
    the same reading for the gate/up pattern; a = silu(g) u from the GEMM's
    unrounded result, a and dgu held in bf16 before they are quantised.
  * The MLP sub-layer on MXFP8 (``ref_mlp_fwd_mx8``, ``ref_mlp_bwd_mx8``): the
    two readings composed, y diag(gamma) quantised as in the block's MXFP8
    forward, dy_in added to dy as in the bf16 MLP.

Every function here is pinned by a test against something other than itself
(brute-force loops, finite differences, torch CPU autograd, closed forms and
invariants, a hand-worked example); see the ``tests/test_oracle_*.py`` files.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_rne", "ref_fwd", "ref_fwd_rewritten", "ref_partials", "ref_bwd",
    "ref_y_r", "ref_fwd_rows", "ref_bwd_sampled", "sigmoid", "ref_swiglu_fwd",
    "ref_swiglu_bwd", "ref_swiglu_fwd_rows", "ref_swiglu_bwd_sampled",
    "ref_mlp_fwd", "ref_mlp_bwd", "ref_mlp_fwd_rows", "ref_mlp_bwd_sampled",
    "ref_ce_fwd", "ref_ce_bwd", "ref_ce_partials", "ref_ce_fwd_rows", "ref_ce_bwd_sampled",
    "rope_angles", "ref_rope_rotate", "ref_rope_fwd", "ref_rope_bwd", "ref_rope_fwd_rows",
    "ref_rope_bwd_sampled",
    "E4M3_MAX", "MX_BLOCK", "e4m3_decode", "e4m3_encode", "e8m0_decode", "mx_quantize",
    "mx_dequantize", "ref_fwd_mx8", "ref_fwd_mx8_rows", "mx_matmul", "ref_bwd_mx8",
    "ref_bwd_mx8_sampled", "ref_swiglu_fwd_mx8", "ref_swiglu_bwd_mx8", "ref_swiglu_fwd_mx8_rows",
    "ref_swiglu_bwd_mx8_sampled", "ref_mlp_fwd_mx8", "ref_mlp_fwd_mx8_rows", "ref_mlp_bwd_mx8",
    "ref_mlp_bwd_mx8_sampled",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# bf16 rounding (storage contract of saved activations and outputs)
# ---------------------------------------------------------------------------

def bf16_rne(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and fp32's exponent range.  A finite x is
    written m * 2**e with 0.5 <= |m| < 1 (frexp); below 2**-126 the spacing
    stays at that of the smallest normal binade.  The value is scaled so that
    one bf16 step is 1, rounded with numpy's rint (ties to even), and scaled
    back.  Results beyond the largest bf16 value become +-inf.  This is one
    rounding straight from float64, not via float32.
    """
    x = _f64(x)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xm = x[fin]
    _, e = np.frexp(xm)
    e = np.maximum(e, -125)           # |x| < 2**-126: subnormal spacing 2**-133
    step_exp = e - 8                  # 8 significant bits
    q = np.rint(np.ldexp(xm, -step_exp))
    v = np.ldexp(q, step_exp)
    max_bf16 = np.ldexp(255.0, 120)   # (2 - 2**-7) * 2**127
    v = np.where(np.abs(v) > max_bf16, np.copysign(np.inf, v), v)
    out[fin] = v
    return out


# ---------------------------------------------------------------------------
# GEMM-Residual-RMSNorm-GEMM, forward
# ---------------------------------------------------------------------------

def ref_fwd(X, W1, R, gamma, W2, eps: float) -> dict:
    """Unfused forward: y = X W1 + R; r = (mean_j y^2 + eps)^-1/2;
    h = diag(r) y diag(gamma); z = h W2.

    Returns y, ms (row mean squares), r, h and z, all float64.
    The pattern follows [RU]/[FR] insight sections (matmul, residual add, RMS
    normalisation, matmul); the formula of r is the reading stated in the module
    header.
    """
    X, W1, R, gamma, W2 = map(_f64, (X, W1, R, gamma, W2))
    y = X @ W1 + R
    ms = np.mean(y * y, axis=1)
    r = 1.0 / np.sqrt(ms + eps)
    h = (y * r[:, None]) * gamma[None, :]
    z = h @ W2
    return {"y": y, "ms": ms, "r": r, "h": h, "z": z}


def ref_partials(y, BN: int) -> np.ndarray:
    """Per-row, per-column-tile partial sums of squares.

    P[i, t] = sum of y[i, j]**2 over j in [t*BN, min((t+1)*BN, d)); the last
    tile may be ragged.  This is the tile-wise reduction the first GEMM's
    epilogue leaves behind ([RU] insight section: a local "partial RMS" at the
    end of the first GEMM, combined by a light reduction kernel; [FR] same
    section).
    """
    y = _f64(y)
    M, d = y.shape
    T = -(-d // BN)
    P = np.zeros((M, T))
    for t in range(T):
        blk = y[:, t * BN:min((t + 1) * BN, d)]
        P[:, t] = np.sum(blk * blk, axis=1)
    return P


def ref_fwd_rewritten(X, W1, R, gamma, W2, eps: float, BN: int = 256) -> dict:
    """The rewritten forward of the pages' insight section: the row scale is
    deferred past the second GEMM.

    y = X W1 + R; P = per-tile partial sums of squares of y; r_i = (sum_t
    P[i,t] / d + eps)^-1/2; W2' = diag(gamma) W2; z = diag(r) (y W2').
    ([JA] 核心の洞察: r commutes with the following matmul so applying it moves
    into the second GEMM's epilogue; [RU]/[FR] insight sections add the partial
    RMS and the reduction kernel.)  Same z as ``ref_fwd`` up to rounding order.
    """
    X, W1, R, gamma, W2 = map(_f64, (X, W1, R, gamma, W2))
    y = X @ W1 + R
    d = y.shape[1]
    P = ref_partials(y, BN)
    r = 1.0 / np.sqrt(P.sum(axis=1) / d + eps)
    W2f = gamma[:, None] * W2
    z = r[:, None] * (y @ W2f)
    return {"y": y, "P": P, "r": r, "W2f": W2f, "z": z}


# ---------------------------------------------------------------------------
# GEMM-Residual-RMSNorm-GEMM, backward
# ---------------------------------------------------------------------------

def ref_bwd(X, W1, gamma, W2, y, r, dz, dy_in=None) -> dict:
    """Exact gradient of L = <dz, z> (+ <dy_in, y>) for the forward of
    ``ref_fwd``, given the saved y and r.

    With n = diag(r) y and h = n diag(gamma):
      dW2 = h^T dz;  dh = dz W2^T;  dgamma_j = sum_i dh_ij n_ij;
      dn = dh diag(gamma);  s_i = sum_j dn_ij y_ij;  c_i = r_i^3 s_i / d;
      dy = diag(r) dn - diag(c) y (+ dy_in);  dR = dy;  dX = dy W1^T;
      dW1 = X^T dy.
    (dr_i/dy_ik = -r_i^3 y_ik / d gives the -c y term.)  Without dy_in the
    gradient reaches y only through z, so dR = dy; dy_in is the gradient the
    residual stream y receives from elsewhere, and it adds to dy.
    """
    X, W1, gamma, W2, y, r, dz = map(_f64, (X, W1, gamma, W2, y, r, dz))
    d = y.shape[1]
    n = y * r[:, None]
    h = n * gamma[None, :]
    dW2 = h.T @ dz
    dh = dz @ W2.T
    dgamma = np.sum(dh * n, axis=0)
    dn = dh * gamma[None, :]
    s = np.sum(dn * y, axis=1)
    c = r ** 3 * s / d
    dy = dn * r[:, None] - c[:, None] * y
    if dy_in is not None:
        dy = dy + _f64(dy_in)
    dX = dy @ W1.T
    dW1 = X.T @ dy
    return {"dX": dX, "dW1": dW1, "dR": dy, "dW2": dW2, "dgamma": dgamma,
            "dh": dh, "dn": dn, "n": n, "s": s, "c": c, "dy": dy}


# ---------------------------------------------------------------------------
# Sampled forms for workloads too large to evaluate whole on the host.
# They restrict the same definitions to chosen rows or columns.
# ---------------------------------------------------------------------------

def ref_y_r(X, W1, R, eps: float) -> dict:
    """The first half of ``ref_fwd``: y = X W1 + R and r, without the second GEMM."""
    X, W1, R = map(_f64, (X, W1, R))
    y = X @ W1 + R
    r = 1.0 / np.sqrt(np.mean(y * y, axis=1) + eps)
    return {"y": y, "r": r}


def ref_fwd_rows(X, W1, R, gamma, W2, eps: float, rows) -> dict:
    """``ref_fwd`` evaluated for the given rows only (rows are independent)."""
    rows = np.asarray(rows)
    X = _f64(X[rows])
    R = _f64(R[rows])
    out = ref_fwd(X, W1, R, gamma, W2, eps)
    out["rows"] = rows
    return out


def ref_bwd_sampled(X, W1, gamma, W2, y, r, dz, rows, cols_d, cols_N) -> dict:
    """``ref_bwd`` with dX and dR restricted to ``rows``, dW1 to the columns
    ``cols_d`` and dW2 to the columns ``cols_N``; dgamma, s and c in full.

    s and c need every row's dh, so dh = dz W2^T is formed whole (the one
    large product).  The rest is the definitions restricted.
    """
    X, W1, gamma, W2, y, r = map(_f64, (X, W1, gamma, W2, y, r))
    dz = _f64(dz)
    d = y.shape[1]
    n = y * r[:, None]
    dh = dz @ W2.T
    dgamma = np.sum(dh * n, axis=0)
    dn = dh * gamma[None, :]
    s = np.sum(dn * y, axis=1)
    c = r ** 3 * s / d
    rows = np.asarray(rows)
    cols_d = np.asarray(cols_d)
    cols_N = np.asarray(cols_N)
    dy_rows = dn[rows] * r[rows, None] - c[rows, None] * y[rows]
    dX_rows = dy_rows @ W1.T
    dy_cols = dn[:, cols_d] * r[:, None] - c[:, None] * y[:, cols_d]
    dW1_cols = X.T @ dy_cols
    h = n * gamma[None, :]
    dW2_cols = h.T @ dz[:, cols_N]
    return {"rows": rows, "cols_d": cols_d, "cols_N": cols_N,
            "dR_rows": dy_rows, "dX_rows": dX_rows, "dW1_cols": dW1_cols,
            "dW2_cols": dW2_cols, "dgamma": dgamma, "s": s, "c": c}


# ---------------------------------------------------------------------------
# SwiGLU gate/up GEMM with the activation in the epilogue
# ---------------------------------------------------------------------------

def sigmoid(t) -> np.ndarray:
    """Logistic function 1/(1+exp(-t)), using exp(t)/(1+exp(t)) for t < 0 so
    that no exp overflows."""
    t = _f64(t)
    out = np.empty_like(t)
    pos = t >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-t[pos]))
    et = np.exp(t[~pos])
    out[~pos] = et / (1.0 + et)
    return out


def ref_swiglu_fwd(X, W, Wd) -> dict:
    """gu = X W; g = gu[:, :F], u = gu[:, F:]; a = g sigmoid(g) u; z = a Wd."""
    X, W, Wd = map(_f64, (X, W, Wd))
    F = W.shape[1] // 2
    gu = X @ W
    g, u = gu[:, :F], gu[:, F:]
    a = g * sigmoid(g) * u
    z = a @ Wd
    return {"gu": gu, "a": a, "z": z}


def ref_swiglu_bwd(X, W, Wd, gu, a, dz) -> dict:
    """Exact gradient of L = <dz, z> for ``ref_swiglu_fwd`` given saved gu, a.

    da = dz Wd^T; with sg = sigmoid(g):
      dg = da u sg (1 + g (1 - sg));  du = da g sg;
      dWd = a^T dz;  dgu = [dg | du];  dW = X^T dgu;  dX = dgu W^T.
    """
    X, W, Wd, gu, a, dz = map(_f64, (X, W, Wd, gu, a, dz))
    F = W.shape[1] // 2
    g, u = gu[:, :F], gu[:, F:]
    sg = sigmoid(g)
    da = dz @ Wd.T
    dg = da * u * sg * (1.0 + g * (1.0 - sg))
    du = da * g * sg
    dgu = np.concatenate([dg, du], axis=1)
    return {"dX": dgu @ W.T, "dW": X.T @ dgu, "dWd": a.T @ dz,
            "dgu": dgu, "da": da}


def ref_swiglu_fwd_rows(X, W, Wd, rows) -> dict:
    """``ref_swiglu_fwd`` for the given rows only."""
    rows = np.asarray(rows)
    out = ref_swiglu_fwd(_f64(X[rows]), W, Wd)
    out["rows"] = rows
    return out


def ref_swiglu_bwd_sampled(X, W, Wd, dz, rows, cols_W, rows_Wd, saved_bf16: bool = True) -> dict:
    """``ref_swiglu_bwd`` restricted: dX and dgu on ``rows``, dW on the columns
    ``cols_W`` (indices into [0, 2F)), dWd on the rows ``rows_Wd`` (indices
    into [0, F)).

    The saved gu and a are recomputed here from X and W, only where needed,
    and rounded to bf16 when ``saved_bf16`` (the storage contract of the
    saved activations); the arithmetic is that of ``ref_swiglu_bwd``.
    """
    X, W, Wd, dz = map(_f64, (X, W, Wd, dz))
    F = W.shape[1] // 2
    keep = bf16_rne if saved_bf16 else (lambda v: v)
    rows = np.asarray(rows)
    cols_W = np.asarray(cols_W)
    rows_Wd = np.asarray(rows_Wd)
    # rows: the whole gradient chain for these tokens
    gu_r = X[rows] @ W
    g_r, u_r = gu_r[:, :F], gu_r[:, F:]
    a_r = g_r * sigmoid(g_r) * u_r
    sub = ref_swiglu_bwd(X[rows], W, Wd, keep(gu_r), keep(a_r), dz[rows])
    # dW columns: dgu[:, c] over every token
    jg = cols_W % F
    is_gate = cols_W < F
    g = keep(X @ W[:, jg])
    u = keep(X @ W[:, F + jg])
    da = dz @ Wd[jg, :].T
    sg = sigmoid(g)
    dgu_c = np.where(is_gate[None, :], da * u * sg * (1.0 + g * (1.0 - sg)), da * g * sg)
    # dWd rows: a[:, j] over every token
    gj = X @ W[:, rows_Wd]
    uj = X @ W[:, F + rows_Wd]
    a_c = keep(gj * sigmoid(gj) * uj)
    return {"rows": rows, "cols_W": cols_W, "rows_Wd": rows_Wd,
            "dX_rows": sub["dX"], "dgu_rows": sub["dgu"],
            "dW_cols": X.T @ dgu_c, "dWd_rows": a_c.T @ dz}


# ---------------------------------------------------------------------------
# The two patterns chained: a LLaMA MLP sub-layer
# ---------------------------------------------------------------------------

def ref_mlp_fwd(X, W1, R, gamma, W, Wd, eps: float, h_round=None) -> dict:
    """Projection + residual, RMS normalisation, SwiGLU gate/up, down projection.

    y = X W1 + R;  r_i = (mean_j y_ij^2 + eps)^(-1/2);  h = diag(r) y diag(gamma);
    gu = h W (W = [W_gate | W_up]);  g = gu[:, :F], u = gu[:, F:];
    a = g sigmoid(g) u;  z = a Wd.
    ([RU]/[FR] insight sections for the residual + RMS pattern around a
    matmul; [JA]/[RU]/[FR] primitives sections for SwiGLU as the activation.)

    With the row scale deferred past the gate/up GEMM (the insight sections'
    rewrite), the GEMM's input is y diag(gamma), an intermediate a fused path
    stores between the two GEMMs; ``h_round``, if given, is applied to it:
    gu = diag(r) (h_round(y diag(gamma)) W).  Without it, gu = h W exactly.
    """
    X, W1, R, gamma, W, Wd = map(_f64, (X, W1, R, gamma, W, Wd))
    y = X @ W1 + R
    r = 1.0 / np.sqrt(np.mean(y * y, axis=1) + eps)
    h = y * r[:, None] * gamma[None, :]
    F = W.shape[1] // 2
    if h_round is None:
        gu = h @ W
    else:
        gu = r[:, None] * (_f64(h_round(y * gamma[None, :])) @ W)
    g, u = gu[:, :F], gu[:, F:]
    a = g * sigmoid(g) * u
    z = a @ Wd
    return {"y": y, "r": r, "h": h, "gu": gu, "a": a, "z": z}


def ref_mlp_bwd(X, W1, gamma, W, Wd, y, r, gu, a, dz, dy_in=None, dgu_round=None) -> dict:
    """Exact gradient of L = <dz, z> (+ <dy_in, y>) for ``ref_mlp_fwd``, given
    the saved y, r, gu and a.

    dgu is the one intermediate of this backward that a fused path must store
    between its two halves (the primitives sections' tile store of
    intermediates); ``dgu_round``, if given, is applied to it before the second
    half, so that the oracle can follow the storage contract the way the
    callers pass the saved y rounded (e.g. ``bf16_rne``).

    The SwiGLU part first, from the saved gu and a (as ``ref_swiglu_bwd``):
      da = dz Wd^T;  dg = da u sg (1 + g (1 - sg));  du = da g sg;
      dgu = [dg | du];  dWd = a^T dz.
    Then h W is the second GEMM of the RMS-normalised block with dgu as its
    output gradient, so the rest is ``ref_bwd`` with W2 = W and dz = dgu:
      dW = h^T dgu;  dh = dgu W^T;  dgamma;  dy (+ dy_in);  dR;  dX;  dW1.
    """
    X, W1, gamma, W, Wd, y, r, gu, a, dz = map(_f64, (X, W1, gamma, W, Wd, y, r, gu, a, dz))
    F = W.shape[1] // 2
    g, u = gu[:, :F], gu[:, F:]
    sg = sigmoid(g)
    da = dz @ Wd.T
    dg = da * u * sg * (1.0 + g * (1.0 - sg))
    du = da * g * sg
    dgu = np.concatenate([dg, du], axis=1)
    dWd = a.T @ dz
    if dgu_round is not None:
        dgu = _f64(dgu_round(dgu))
    b = ref_bwd(X, W1, gamma, W, y, r, dgu, dy_in)
    return {"dX": b["dX"], "dW1": b["dW1"], "dR": b["dR"], "dW": b["dW2"], "dWd": dWd,
            "dgamma": b["dgamma"], "dgu": dgu, "da": da, "dh": b["dh"], "s": b["s"], "c": b["c"]}


def ref_mlp_fwd_rows(X, W1, R, gamma, W, Wd, eps: float, rows, h_round=None) -> dict:
    """``ref_mlp_fwd`` evaluated for the given rows only (rows are independent)."""
    rows = np.asarray(rows)
    out = ref_mlp_fwd(_f64(X[rows]), W1, _f64(R[rows]), gamma, W, Wd, eps, h_round)
    out["rows"] = rows
    return out


def ref_mlp_bwd_sampled(X, W1, gamma, W, Wd, y, r, gu, a, dz, dy_in, rows, cols_d, cols_2F,
                        rows_F, dgu_round=None) -> dict:
    """``ref_mlp_bwd`` with dX and dR restricted to ``rows``, dW1 to the columns
    ``cols_d``, dW to the columns ``cols_2F``, dWd to the rows ``rows_F``;
    dgamma, s and c in full.

    s and c need every row's dh, so dgu (from da = dz Wd^T) and dh = dgu W^T
    are formed whole.  The rest is the definitions restricted.  dy_in may be
    None.  ``dgu_round`` as in ``ref_mlp_bwd``.
    """
    X, W1, gamma, W, Wd, y, r, gu, a, dz = map(_f64, (X, W1, gamma, W, Wd, y, r, gu, a, dz))
    d = y.shape[1]
    F = W.shape[1] // 2
    g, u = gu[:, :F], gu[:, F:]
    sg = sigmoid(g)
    da = dz @ Wd.T
    dgu = np.concatenate([da * u * sg * (1.0 + g * (1.0 - sg)), da * g * sg], axis=1)
    if dgu_round is not None:
        dgu = _f64(dgu_round(dgu))
    n = y * r[:, None]
    dh = dgu @ W.T
    dgamma = np.sum(dh * n, axis=0)
    dn = dh * gamma[None, :]
    s = np.sum(dn * y, axis=1)
    c = r ** 3 * s / d
    rows, cols_d, cols_2F, rows_F = map(np.asarray, (rows, cols_d, cols_2F, rows_F))
    dy_rows = dn[rows] * r[rows, None] - c[rows, None] * y[rows]
    dy_cols = dn[:, cols_d] * r[:, None] - c[:, None] * y[:, cols_d]
    if dy_in is not None:
        dy_in = _f64(dy_in)
        dy_rows = dy_rows + dy_in[rows]
        dy_cols = dy_cols + dy_in[:, cols_d]
    h = n * gamma[None, :]
    return {"rows": rows, "cols_d": cols_d, "cols_2F": cols_2F, "rows_F": rows_F,
            "dR_rows": dy_rows, "dX_rows": dy_rows @ W1.T, "dW1_cols": X.T @ dy_cols,
            "dW_cols": h.T @ dgu[:, cols_2F], "dWd_rows": a[:, rows_F].T @ dz,
            "dgamma": dgamma, "s": s, "c": c}


# ---------------------------------------------------------------------------
# Cross-entropy over an LM-head GEMM
# ---------------------------------------------------------------------------

def _logsumexp_rows(x) -> np.ndarray:
    """log sum_j exp(x_ij) per row, shifted by the row max so nothing overflows."""
    m = np.max(x, axis=1)
    return m + np.log(np.sum(np.exp(x - m[:, None]), axis=1))


def _ce_valid(labels, V):
    """Rows whose label is a column index; the others are ignored rows."""
    labels = np.asarray(labels, dtype=np.int64)
    return labels, (labels >= 0) & (labels < V)


def ref_ce_fwd(h, Wv, labels) -> dict:
    """logits = h Wv;  lse_i = log sum_j exp(logits_ij);
    loss_i = lse_i - logits_i,label_i.  ([JA]/[RU]/[FR] primitives sections:
    cross-entropy over the stateful max / sum-exp epilogue.)
    A label outside [0, V) marks an ignored row (reading: the pages define no
    label format; the usual ignore-index convention): its loss is 0 and it
    contributes no gradient; its lse is still the row's."""
    h, Wv = _f64(h), _f64(Wv)
    logits = h @ Wv
    labels, valid = _ce_valid(labels, logits.shape[1])
    lse = _logsumexp_rows(logits)
    picked = logits[np.arange(logits.shape[0]), np.where(valid, labels, 0)]
    loss = np.where(valid, lse - picked, 0.0)
    return {"logits": logits, "lse": lse, "loss": loss}


def ref_ce_partials(logits, BN: int = 256) -> dict:
    """The stateful primitive's per-tile state: for each row i and tile t of BN
    columns, m[i,t] = max_{j in t} logits_ij and s[i,t] = sum_{j in t}
    exp(logits_ij - m[i,t]); and their combination, the running (max, sum)
    update m' = max(m, m_t), s' = s exp(m - m') + s_t exp(m_t - m'), taken
    over the tiles in order, giving lse = m + log s.  Same lse as the
    definition up to rounding."""
    x = _f64(logits)
    M, V = x.shape
    T = -(-V // BN)
    m = np.empty((M, T))
    s = np.empty((M, T))
    for t in range(T):
        blk = x[:, t * BN:min((t + 1) * BN, V)]
        m[:, t] = np.max(blk, axis=1)
        s[:, t] = np.sum(np.exp(blk - m[:, t:t + 1]), axis=1)
    run_m = m[:, 0].copy()
    run_s = s[:, 0].copy()
    for t in range(1, T):
        new_m = np.maximum(run_m, m[:, t])
        run_s = run_s * np.exp(run_m - new_m) + s[:, t] * np.exp(m[:, t] - new_m)
        run_m = new_m
    return {"m": m, "s": s, "lse": run_m + np.log(run_s)}


def ref_ce_bwd(h, Wv, labels, lse, dloss, logits=None) -> dict:
    """Exact gradient of L = sum_i dloss_i loss_i for ``ref_ce_fwd``, given the
    saved lse (and the saved logits, if passed; else they are recomputed):
      p = exp(logits - lse) (softmax by rows);  dlogits = diag(dloss) (p - onehot(labels));
      dh = dlogits Wv^T;  dWv = h^T dlogits.
    An ignored row (label outside [0, V)) has loss 0, so its dlogits row is 0."""
    h, Wv = _f64(h), _f64(Wv)
    lse, dloss = _f64(lse), _f64(dloss)
    logits = h @ Wv if logits is None else _f64(logits)
    labels, valid = _ce_valid(labels, logits.shape[1])
    p = np.exp(logits - lse[:, None])
    dlogits = p
    rows = np.nonzero(valid)[0]
    dlogits[rows, labels[rows]] -= 1.0
    dlogits = dlogits * np.where(valid, dloss, 0.0)[:, None]
    return {"dh": dlogits @ Wv.T, "dWv": h.T @ dlogits, "dlogits": dlogits}


def ref_ce_fwd_rows(h, Wv, labels, rows) -> dict:
    """``ref_ce_fwd`` for the given rows only (rows are independent)."""
    rows = np.asarray(rows)
    out = ref_ce_fwd(_f64(h[rows]), Wv, np.asarray(labels)[rows])
    out["rows"] = rows
    return out


def ref_ce_bwd_sampled(h, Wv, labels, lse, dloss, rows, cols_V, logits=None) -> dict:
    """``ref_ce_bwd`` with dh restricted to ``rows`` and dWv to the columns
    ``cols_V``: dh rows need only those rows' dlogits; dWv columns need every
    row's dlogits in those columns."""
    h, Wv = _f64(h), _f64(Wv)
    labels, valid = _ce_valid(labels, Wv.shape[1])
    lse, dloss = _f64(lse), _f64(dloss)
    dloss = np.where(valid, dloss, 0.0)
    rows, cols_V = np.asarray(rows), np.asarray(cols_V)

    def dlog(lg, lab, ls, dl, cols):
        p = np.exp(lg - ls[:, None])
        hit = lab[:, None] == cols[None, :]
        return (p - hit) * dl[:, None]
    lg_rows = h[rows] @ Wv if logits is None else _f64(logits[rows])
    dlr = dlog(lg_rows, labels[rows], lse[rows], dloss[rows], np.arange(Wv.shape[1]))
    lg_cols = h @ Wv[:, cols_V] if logits is None else _f64(logits[:, cols_V])
    dlc = dlog(lg_cols, labels, lse, dloss, cols_V)
    return {"rows": rows, "cols_V": cols_V, "dh_rows": dlr @ Wv.T, "dWv_cols": h.T @ dlc}


# ---------------------------------------------------------------------------
# Rotary position embedding in the epilogue of a QKV projection
# ---------------------------------------------------------------------------

def rope_angles(M: int, D: int, S: int, base: float) -> np.ndarray:
    """phi[m, i] = (m mod S) * base^(-2i/D), i = 0..D/2-1."""
    p = (np.arange(M) % S).astype(np.float64)
    theta = base ** (-2.0 * np.arange(D // 2, dtype=np.float64) / D)
    return p[:, None] * theta[None, :]


def ref_rope_rotate(Y, N_rot: int, D: int, S: int, base: float, inverse: bool = False) -> np.ndarray:
    """Rotate the pairs (2i, 2i+1) of every D-wide head in the first N_rot
    columns by phi[m, i] (by -phi[m, i] when ``inverse``); other columns are
    copied."""
    Y = _f64(Y)
    M = Y.shape[0]
    out = Y.copy()
    phi = rope_angles(M, D, S, base)
    c, sn = np.cos(phi), np.sin(phi)
    if inverse:
        sn = -sn
    for h0 in range(0, N_rot, D):
        x0 = Y[:, h0:h0 + D:2]
        x1 = Y[:, h0 + 1:h0 + D:2]
        out[:, h0:h0 + D:2] = x0 * c - x1 * sn
        out[:, h0 + 1:h0 + D:2] = x0 * sn + x1 * c
    return out


def ref_rope_fwd(X, W, N_rot: int, D: int, S: int, base: float) -> dict:
    """Y = rope(X W): the projection, then the rotation of its first N_rot
    columns ([JA]/[RU]/[FR] primitives sections: elementwise transforms in
    the epilogue)."""
    P = _f64(X) @ _f64(W)
    return {"P": P, "Y": ref_rope_rotate(P, N_rot, D, S, base)}


def ref_rope_bwd(X, W, dY, N_rot: int, D: int, S: int, base: float) -> dict:
    """Exact gradient of L = <dY, Y>: the rotation is orthogonal, so
    dP = rotate(dY, -phi) on the rotated columns (dY elsewhere);
    dX = dP W^T;  dW = X^T dP."""
    X, W = _f64(X), _f64(W)
    dP = ref_rope_rotate(dY, N_rot, D, S, base, inverse=True)
    return {"dP": dP, "dX": dP @ W.T, "dW": X.T @ dP}


def ref_rope_fwd_rows(X, W, N_rot: int, D: int, S: int, base: float, rows) -> dict:
    """``ref_rope_fwd`` for the given rows (their positions kept)."""
    rows = np.asarray(rows)
    P = _f64(X[rows]) @ _f64(W)
    M_all = int(np.max(rows)) + 1
    phi_all = rope_angles(M_all, D, S, base)[rows]
    c, sn = np.cos(phi_all), np.sin(phi_all)
    Y = P.copy()
    for h0 in range(0, N_rot, D):
        x0, x1 = P[:, h0:h0 + D:2], P[:, h0 + 1:h0 + D:2]
        Y[:, h0:h0 + D:2] = x0 * c - x1 * sn
        Y[:, h0 + 1:h0 + D:2] = x0 * sn + x1 * c
    return {"rows": rows, "P": P, "Y": Y}


def ref_rope_bwd_sampled(X, W, dY, N_rot: int, D: int, S: int, base: float, rows, cols_N) -> dict:
    """``ref_rope_bwd`` with dX restricted to ``rows`` and dW to the columns
    ``cols_N`` (dP is row-local, so it is formed whole)."""
    X, W = _f64(X), _f64(W)
    dP = ref_rope_rotate(dY, N_rot, D, S, base, inverse=True)
    rows, cols_N = np.asarray(rows), np.asarray(cols_N)
    return {"rows": rows, "cols_N": cols_N, "dX_rows": dP[rows] @ W.T, "dW_cols": X.T @ dP[:, cols_N]}


# ---------------------------------------------------------------------------
# MX-FP8 (OCP microscaling, E4M3 elements with one E8M0 scale per 32) forward
# of the fused block
# ---------------------------------------------------------------------------
# The pages say that faster low-precision (FP8, FP4) matrix units raise the
# relative cost of the memory-bound work around a GEMM (the "tax" sections:
# [JA] 課題：大モデル訓練の「手抜き税」, [RU] "Налог на лень ...", [FR] "Le
# « impôt de la paresse » ...").  They fix no FP8 format
# or scaling.  Reading: the OCP Microscaling (MX) v1.0 MXFP8 format.  An
# element is FP8 E4M3 (the "FN" variant: bias 7, no infinities, S.1111.111 is
# NaN, largest finite 448); every 32 consecutive elements along the contraction
# index share one E8M0 scale byte s meaning 2**(s - 127) (255 is NaN).  A block
# is quantised with the shared exponent floor(log2(amax)) - 8 (8 = E4M3's
# largest normal exponent), clamped to [-127, 127]; an all-zero block takes
# exponent -127; each element divided by 2**shared_exp is rounded to the
# nearest E4M3 value, ties to even, and saturated to +-448.

E4M3_MAX = 448.0
MX_BLOCK = 32


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 (FN) byte -> float64: sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent 0 is subnormal (m/8 * 2**-6); 0x7F and 0xFF
    are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(x) -> np.ndarray:
    """float64 -> nearest E4M3 (FN) byte, ties to even, saturating at +-448.

    Normal values keep 4 significant bits (spacing 2**(e-3) in the binade
    [2**e, 2**(e+1)), e >= -6); below 2**-6 the spacing stays 2**-9
    (subnormals).  The value is scaled so that one step is 1, rounded with
    numpy's rint (ties to even) and the code is assembled from the rounded
    magnitude.  NaN is not accepted.
    """
    x = _f64(x)
    if np.isnan(x).any():
        raise ValueError("e4m3_encode: NaN input")
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, fe = np.frexp(a)                       # a = f * 2**fe, 0.5 <= f < 1; a in [2**(fe-1), 2**fe)
    e = np.maximum(fe - 1, -6)                # binade exponent, subnormals use -6
    q = np.rint(np.ldexp(a, 3 - e))           # magnitude in steps of 2**(e-3): 8..16 normal, 0..8 subnormal
    # a carry to 16 steps moves to the next binade (16 * 2**(e-3) = 2**(e+1))
    carry = q >= 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, q / 2, q)
    sub = q < 8                               # only possible with e == -6
    exp_field = np.where(sub, 0, e + 7).astype(np.int64)
    mant = np.where(sub, q, q - 8).astype(np.int64)
    mag_code = (exp_field << 3) | mant
    mag_code = np.minimum(mag_code, 0x7E)     # saturate (448 = 0x7E); rounding can reach 480 only above 464
    code = np.where(np.signbit(x), 0x80, 0) | mag_code
    return code.astype(np.uint8)


def e8m0_decode(scales) -> np.ndarray:
    """E8M0 scale byte s -> 2**(s - 127); 255 is NaN."""
    s = np.asarray(scales, dtype=np.uint8).astype(np.float64)
    return np.where(s == 255, np.nan, np.exp2(s - 127.0))


def mx_quantize(V, block: int = MX_BLOCK):
    """Quantise the rows of V [rows, K] to MXFP8 along K (K % block == 0).

    Per block of ``block`` consecutive elements of a row: amax = max |v|;
    shared_exp = floor(log2(amax)) - 8, clamped to [-127, 127] (amax == 0 ->
    -127); scale byte = shared_exp + 127; element codes = e4m3_encode(v /
    2**shared_exp).  Returns (codes uint8 [rows, K], scales uint8 [rows,
    K / block]).
    """
    V = _f64(V)
    rows, K = V.shape
    if K % block:
        raise ValueError("mx_quantize: K must be a multiple of the block")
    B = V.reshape(rows, K // block, block)
    amax = np.max(np.abs(B), axis=2)
    _, fe = np.frexp(amax)                    # amax in [2**(fe-1), 2**fe): floor(log2) = fe - 1
    sexp = np.where(amax > 0, fe - 1 - 8, -127)
    sexp = np.clip(sexp, -127, 127)
    codes = e4m3_encode(np.ldexp(B, -sexp[:, :, None]))
    return codes.reshape(rows, K), (sexp + 127).astype(np.uint8)


def mx_dequantize(codes, scales, block: int = MX_BLOCK) -> np.ndarray:
    """MXFP8 [rows, K] codes with [rows, K / block] scales -> float64."""
    c = np.asarray(codes)
    rows, K = c.shape
    v = e4m3_decode(c).reshape(rows, K // block, block) * e8m0_decode(scales)[:, :, None]
    return v.reshape(rows, K)


def ref_fwd_mx8(Xq, Xs, W1q, W1s, R, gamma, W2q, W2s, eps: float) -> dict:
    """Forward of the fused block with MXFP8 GEMM operands.

    X is [M, K] (codes Xq, scales Xs along K).  The weights are stored with
    their contraction index contiguous, as [out, in]: W1q [d, K] with W1s
    [d, K/32], W2q [N, d] with W2s [N, d/32].  R [M, d] and gamma [d] are real.

      y  = deq(X) deq(W1)^T + R;   r_i = (mean_j y_ij^2 + eps)^-1/2;
      (q, s) = mx_quantize(y diag(gamma))   (blocks along j, the second
                                             GEMM's contraction index);
      z  = diag(r) (deq(q, s) deq(W2)^T).

    This is the rewrite of ``ref_fwd_rewritten`` (r deferred past the second
    GEMM) with its second operand stored in MXFP8.  Reading: what is
    quantised is y diag(gamma), the tensor the first GEMM's epilogue holds,
    not the normalised h = diag(r) y diag(gamma); the two differ by one E4M3
    rounding per element because r is not a power of two.
    """
    Xh = mx_dequantize(Xq, Xs)
    W1h = mx_dequantize(W1q, W1s)
    W2h = mx_dequantize(W2q, W2s)
    R, gamma = _f64(R), _f64(gamma)
    y = Xh @ W1h.T + R
    r = 1.0 / np.sqrt(np.mean(y * y, axis=1) + eps)
    q, s = mx_quantize(y * gamma[None, :])
    z = r[:, None] * (mx_dequantize(q, s) @ W2h.T)
    return {"y": y, "r": r, "yg_q": q, "yg_s": s, "yg": y * gamma[None, :], "z": z}


def mx_matmul(A, B) -> np.ndarray:
    """A B with both operands in MXFP8, quantised along the contraction index:
    deq(mx_quantize(A)) deq(mx_quantize(B^T))^T, A [m, k], B [k, n],
    k % 32 == 0 (each operand's 32-blocks run along k, as block-scaled
    matrix units require)."""
    Aq, As = mx_quantize(A)
    Bq, Bs = mx_quantize(np.ascontiguousarray(_f64(B).T))
    return mx_dequantize(Aq, As) @ mx_dequantize(Bq, Bs).T


def ref_bwd_mx8(X, W1, gamma, W2, y, r, dz, store=bf16_rne, dy_in=None) -> dict:
    """Backward of the block with every GEMM on MXFP8 operands.

    The pages argue that FP8 matrix units make the memory-bound work around a
    GEMM relatively costlier ([JA] 課題; [RU] "Налог на лень"); they give no
    FP8 training recipe.  Reading: the gradient is the calculus of the
    unquantised block (``ref_bwd``: the forward's quantisation passes the
    gradient straight through), and each of the four backward GEMMs runs on
    MXFP8 operands quantised along its own contraction index (``mx_matmul``):
      dh  = mx(dz, W2^T)                 (contraction over N)
      dgamma_j = sum_i dh_ij r_i y_ij;  dn = dh diag(gamma);
      s_i = sum_j dn_ij y_ij;  c_i = r_i^3 s_i / d;
      dy  = diag(r) store(dn) - diag(c) y (+ dy_in);  dR = store(dy)
      dW2 = diag(gamma) mx(store(n)^T, dz),  n = diag(r) y   (contraction over M)
      dX  = mx(store(dy), W1^T)          (contraction over d)
      dW1 = mx(X^T, store(dy))           (contraction over M)
    ``store`` is the storage contract of the intermediates that feed a
    quantiser (dn, n and dy are kept in bf16): bf16_rne by default; pass the
    identity for unrounded intermediates.  y and r are the saved forward
    tensors; X, W1, W2 the unquantised (bf16) inputs; dy_in (optional) the
    gradient that reaches y from later layers (the MLP sub-layer's residual
    stream), added to dy as in ``ref_bwd``.
    """
    X, W1, gamma, W2, y, r, dz = map(_f64, (X, W1, gamma, W2, y, r, dz))
    d = y.shape[1]
    dh = mx_matmul(dz, W2.T)
    n = y * r[:, None]
    dgamma = np.sum(dh * n, axis=0)
    dn = dh * gamma[None, :]
    s = np.sum(dn * y, axis=1)
    c = r ** 3 * s / d
    dy = r[:, None] * store(dn) - c[:, None] * y
    if dy_in is not None:
        dy = dy + _f64(dy_in)
    dy_s = store(dy)
    dW2 = gamma[:, None] * mx_matmul(store(n).T, dz)
    dX = mx_matmul(dy_s, W1.T)
    dW1 = mx_matmul(X.T, dy_s)
    return {"dX": dX, "dW1": dW1, "dR": dy, "dW2": dW2, "dgamma": dgamma,
            "dh": dh, "dn": dn, "n": n, "s": s, "c": c, "dy": dy}


def ref_bwd_mx8_sampled(X, W1, gamma, W2, y, r, dz, rows, cols_d, cols_N, store=bf16_rne, dy_in=None) -> dict:
    """``ref_bwd_mx8`` with dX and dR restricted to ``rows``, dW1 to the columns
    ``cols_d`` and dW2 to the columns ``cols_N``; dgamma, s and c in full.

    A quantisation block runs along its GEMM's contraction index, so a row of
    dX needs only that row of dy (blocks along d) and the whole of W1; a
    column of dW1 needs that column of dy over every row (blocks along M);
    a column of dW2 that column of dz over every row.  dh is formed whole.
    """
    X, W1, gamma, W2, y, r, dz = map(_f64, (X, W1, gamma, W2, y, r, dz))
    d = y.shape[1]
    rows, cols_d, cols_N = map(np.asarray, (rows, cols_d, cols_N))
    dh = mx_matmul(dz, W2.T)
    n = y * r[:, None]
    dgamma = np.sum(dh * n, axis=0)
    dn = dh * gamma[None, :]
    s = np.sum(dn * y, axis=1)
    c = r ** 3 * s / d
    dy = r[:, None] * store(dn) - c[:, None] * y
    if dy_in is not None:
        dy = dy + _f64(dy_in)
    dy_s = store(dy)
    dX_rows = mx_matmul(dy_s[rows], W1.T)
    dW1_cols = mx_matmul(X.T, dy_s[:, cols_d])
    dW2_cols = gamma[:, None] * mx_matmul(store(n).T, dz[:, cols_N])
    dR_rows = dy[rows]
    return {"rows": rows, "cols_d": cols_d, "cols_N": cols_N, "dX_rows": dX_rows, "dR_rows": dR_rows,
            "dW1_cols": dW1_cols, "dW2_cols": dW2_cols, "dgamma": dgamma, "s": s, "c": c}


def ref_swiglu_fwd_mx8(X, W, Wd, store=bf16_rne) -> dict:
    """SwiGLU block with both GEMMs on MXFP8 operands quantised along their
    contraction index (the format of ``mx_matmul``; the reading of the FP8
    block carried over to the SwiGLU pattern, [JA] 課題; [RU] "Налог на лень"):
      gu = mx(X, W)                 (contraction over d)
      a  = silu(g) u, from the unrounded gu = [g | u] (the activation epilogue
           works on the GEMM's fp32 result)
      z  = mx(store(a), Wd)         (contraction over F; a is stored in bf16
           and quantised from there)
    X, W, Wd are the unquantised (bf16) inputs."""
    X, W, Wd = map(_f64, (X, W, Wd))
    F = W.shape[1] // 2
    gu = mx_matmul(X, W)
    g, u = gu[:, :F], gu[:, F:]
    a = g * sigmoid(g) * u
    return {"gu": gu, "a": a, "z": mx_matmul(store(a), Wd)}


def ref_swiglu_bwd_mx8(X, W, Wd, gu, a, dz, store=bf16_rne) -> dict:
    """Backward of ``ref_swiglu_fwd_mx8``: the gradient of the unquantised
    block (``ref_swiglu_bwd``; quantisation passes it straight through), each
    GEMM on MXFP8 operands quantised along its own contraction index:
      da  = mx(dz, Wd^T)            (contraction over d)
      dg  = da u sg (1 + g (1 - sg)), du = da g sg, sg = sigmoid(g), from the
            saved gu = [g | u];  dgu = [dg | du]
      dWd = mx(a^T, dz)             (contraction over M; a the saved a)
      dX  = mx(store(dgu), W^T)     (contraction over 2F)
      dW  = mx(X^T, store(dgu))     (contraction over M)
    ``store`` is the storage of dgu before it is quantised (bf16)."""
    X, W, Wd, gu, a, dz = map(_f64, (X, W, Wd, gu, a, dz))
    F = W.shape[1] // 2
    g, u = gu[:, :F], gu[:, F:]
    sg = sigmoid(g)
    da = mx_matmul(dz, Wd.T)
    dgu = np.concatenate([da * u * sg * (1.0 + g * (1.0 - sg)), da * g * sg], axis=1)
    dgu_s = store(dgu)
    return {"dX": mx_matmul(dgu_s, W.T), "dW": mx_matmul(X.T, dgu_s), "dWd": mx_matmul(a.T, dz),
            "dgu": dgu, "da": da}


def ref_swiglu_fwd_mx8_rows(X, W, Wd, rows, store=bf16_rne) -> dict:
    """``ref_swiglu_fwd_mx8`` for the given rows only (X's blocks run along
    its rows, a's along its rows: every step is row-local)."""
    rows = np.asarray(rows)
    out = ref_swiglu_fwd_mx8(_f64(X)[rows], W, Wd, store)
    out["rows"] = rows
    return out


def ref_swiglu_bwd_mx8_sampled(X, W, Wd, dz, rows, cols_W, rows_Wd, store=bf16_rne) -> dict:
    """``ref_swiglu_bwd_mx8`` restricted: dX and dgu on ``rows``, dW on the
    columns ``cols_W`` (indices into [0, 2F)), dWd on the rows ``rows_Wd``
    (indices into [0, F)), with the saved gu and a those of
    ``ref_swiglu_fwd_mx8`` rounded by ``store`` (recomputed here where needed).

    The columns of a product with B's blocks along the contraction index are
    independent (mx(A, B[:, c]) = mx(A, B)[:, c]), and so are the rows of one
    with A's blocks along it; a column of dW needs that column of dgu over
    every row (its blocks run along M)."""
    X, W, Wd, dz = map(_f64, (X, W, Wd, dz))
    F = W.shape[1] // 2
    rows, cols_W, rows_Wd = map(np.asarray, (rows, cols_W, rows_Wd))
    # rows: dgu and dX for these tokens (row-local: blocks along d and 2F)
    gu_r = store(ref_swiglu_fwd_mx8(X[rows], W, Wd, store)["gu"])
    g_r, u_r = gu_r[:, :F], gu_r[:, F:]
    sg_r = sigmoid(g_r)
    da_r = mx_matmul(dz[rows], Wd.T)
    dgu_r = np.concatenate([da_r * u_r * sg_r * (1.0 + g_r * (1.0 - sg_r)), da_r * g_r * sg_r], axis=1)
    # dW columns: dgu[:, c] over every token
    jg = cols_W % F
    g = store(mx_matmul(X, W[:, jg]))
    u = store(mx_matmul(X, W[:, F + jg]))
    da = mx_matmul(dz, Wd[jg, :].T)
    sg = sigmoid(g)
    dgu_c = np.where((cols_W < F)[None, :], da * u * sg * (1.0 + g * (1.0 - sg)), da * g * sg)
    # dWd rows: a[:, j] over every token
    gj = mx_matmul(X, W[:, rows_Wd])
    uj = mx_matmul(X, W[:, F + rows_Wd])
    a_c = store(gj * sigmoid(gj) * uj)
    return {"rows": rows, "cols_W": cols_W, "rows_Wd": rows_Wd, "dX_rows": mx_matmul(store(dgu_r), W.T),
            "dgu_rows": dgu_r, "dW_cols": mx_matmul(X.T, store(dgu_c)), "dWd_rows": mx_matmul(a_c.T, dz)}


def ref_mlp_fwd_mx8(X, W1, R, gamma, W, Wd, eps: float, store=bf16_rne) -> dict:
    """The MLP sub-layer (``ref_mlp_fwd``) with its three GEMMs on MXFP8
    operands quantised along their contraction index:
      y  = mx(X, W1) + R                    (contraction over K)
      r_i = (mean_j y_ij^2 + eps)^-1/2
      gu = diag(r) mx(y diag(gamma), W)     (contraction over d; as in
           ``ref_fwd_mx8``, y diag(gamma) is quantised from the unrounded y
           and r applied after the product)
      a  = silu(g) u;  z = mx(store(a), Wd) (contraction over F)
    X, W1, R, gamma, W, Wd are the unquantised (bf16) inputs."""
    X, W1, R, gamma, W, Wd = map(_f64, (X, W1, R, gamma, W, Wd))
    F = W.shape[1] // 2
    y = mx_matmul(X, W1) + R
    r = 1.0 / np.sqrt(np.mean(y * y, axis=1) + eps)
    gu = r[:, None] * mx_matmul(y * gamma[None, :], W)
    g, u = gu[:, :F], gu[:, F:]
    a = g * sigmoid(g) * u
    return {"y": y, "r": r, "gu": gu, "a": a, "z": mx_matmul(store(a), Wd)}


def ref_mlp_fwd_mx8_rows(X, W1, R, gamma, W, Wd, eps: float, rows, store=bf16_rne) -> dict:
    """``ref_mlp_fwd_mx8`` for the given rows only (every quantisation block
    of X, y diag(gamma) and a runs along a row)."""
    rows = np.asarray(rows)
    out = ref_mlp_fwd_mx8(_f64(X)[rows], W1, _f64(R)[rows], gamma, W, Wd, eps, store)
    out["rows"] = rows
    return out


def ref_mlp_bwd_mx8(X, W1, gamma, W, Wd, y, r, gu, a, dz, dy_in=None, store=bf16_rne) -> dict:
    """Backward of ``ref_mlp_fwd_mx8``: the SwiGLU part of
    ``ref_swiglu_bwd_mx8`` (da = mx(dz, Wd^T), dgu from the saved gu, dWd =
    mx(a^T, dz)), then, with dgu rounded by ``store`` as the second GEMM's
    output gradient, the block backward ``ref_bwd_mx8`` with W2 = W (dW = its
    dW2) and dy_in added to dy."""
    X, W1, gamma, W, Wd, y, r, gu, a, dz = map(_f64, (X, W1, gamma, W, Wd, y, r, gu, a, dz))
    F = W.shape[1] // 2
    g, u = gu[:, :F], gu[:, F:]
    sg = sigmoid(g)
    da = mx_matmul(dz, Wd.T)
    dgu = np.concatenate([da * u * sg * (1.0 + g * (1.0 - sg)), da * g * sg], axis=1)
    b = ref_bwd_mx8(X, W1, gamma, W, y, r, store(dgu), store, dy_in)
    return {"dX": b["dX"], "dW1": b["dW1"], "dR": b["dR"], "dW": b["dW2"], "dWd": mx_matmul(a.T, dz),
            "dgamma": b["dgamma"], "dgu": dgu, "da": da, "dh": b["dh"], "s": b["s"], "c": b["c"]}


def ref_mlp_bwd_mx8_sampled(X, W1, gamma, W, Wd, y, r, gu, a, dz, dy_in, rows, cols_d, cols_2F, rows_F,
                            store=bf16_rne) -> dict:
    """``ref_mlp_bwd_mx8`` with dX and dR on ``rows``, dW1 on the columns
    ``cols_d``, dW on the columns ``cols_2F``, dWd on the rows ``rows_F``;
    dgamma, s and c in full (they need every row, so dgu is formed whole and
    the block part is ``ref_bwd_mx8_sampled``)."""
    X, W1, gamma, W, Wd, y, r, gu, a, dz = map(_f64, (X, W1, gamma, W, Wd, y, r, gu, a, dz))
    F = W.shape[1] // 2
    g, u = gu[:, :F], gu[:, F:]
    sg = sigmoid(g)
    da = mx_matmul(dz, Wd.T)
    dgu = np.concatenate([da * u * sg * (1.0 + g * (1.0 - sg)), da * g * sg], axis=1)
    rows_F = np.asarray(rows_F)
    b = ref_bwd_mx8_sampled(X, W1, gamma, W, y, r, store(dgu), rows, cols_d, cols_2F, store, dy_in)
    return {"rows": b["rows"], "cols_d": b["cols_d"], "cols_2F": b["cols_N"], "rows_F": rows_F,
            "dX_rows": b["dX_rows"], "dR_rows": b["dR_rows"], "dW1_cols": b["dW1_cols"],
            "dW_cols": b["dW2_cols"], "dWd_rows": mx_matmul(a[:, rows_F].T, dz), "dgamma": b["dgamma"],
            "s": b["s"], "c": b["c"]}


def ref_fwd_mx8_rows(Xq, Xs, W1q, W1s, R, gamma, W2q, W2s, eps: float, rows) -> dict:
    """``ref_fwd_mx8`` for the given rows only (every step is row-local)."""
    rows = np.asarray(rows)
    out = ref_fwd_mx8(np.asarray(Xq)[rows], np.asarray(Xs)[rows], W1q, W1s, _f64(R[rows]), gamma,
                      W2q, W2s, eps)
    out["rows"] = rows
    return out

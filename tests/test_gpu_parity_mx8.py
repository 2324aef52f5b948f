"""GPU parity of the MXFP8 path through the C-ABI against the CPU oracle.

The oracle quantises the inputs (bf16 draws) to MXFP8 on the host; both sides
then start from the same codes and scales.

Bars:
  * the quantiser (bf16 -> MXFP8): bit-exact codes and scales (a bf16 value,
    its block maximum and the power-of-two scaling are exact in fp32 and in
    float64, so both sides round the same value);
  * y, z: max|gpu - ref| / max|ref| <= 2e-2 (bf16 outputs, fp32 accumulation);
    r per element |dr|/r <= 1e-3;
  * y * gamma quantised in the first GEMM's epilogue: the value rounded there
    is the kernel's fp32 y, accumulated by the MXFP8 matrix instruction with
    reduced precision, while the oracle's is exact, so a code may differ where
    the exact value lies near a rounding boundary.  Required: every GPU value
    is the correct rounding (under the GPU's scale) of a value within a slack
    of the exact one (the slack bounds the accumulation error, see
    ``accumulation_slack``); a scale differs from the oracle's only where the
    block's exact maximum lies within that slack of a power of two; at most
    1e-2 of the codes and scales differ.
"""
import numpy as np
import pytest

import oracle
from gemm_epilogue_fusion_gemm1_amd import synth

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
R_TOL = 1e-3
FLIP_FRAC = 1e-2


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_epilogue_fusion_gemm1_amd as coda
    coda.load_library()       # raises when the HIP library is missing: no fallback
    return torch, torch.device("cuda:0")


def rel(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 1.0
    return float(np.max(np.abs(got - ref))) / max(den, 1e-300)


def report(name, errs):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.2e}" if isinstance(v, float) else f"{k}={v}"
                                          for k, v in errs.items()), flush=True)


def u8(torch, dev, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev)


def blocked(s):
    """Row-major scales [rows, K/32] in the library's step-blocked layout [K/128, rows, 4]."""
    rows, nb = s.shape
    return np.ascontiguousarray(s.reshape(rows, nb // 4, 4).transpose(1, 0, 2))


def unblocked(s):
    """Step-blocked scales [K/128, rows, 4] as row-major [rows, K/32]."""
    t, rows, _ = s.shape
    return np.ascontiguousarray(s.transpose(1, 0, 2).reshape(rows, 4 * t))


def bf(torch, dev, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(torch.bfloat16)


def quantised(h):
    Xq, Xs = oracle.mx_quantize(h["X"])
    W1q, W1s = oracle.mx_quantize(h["W1t"])
    W2q, W2s = oracle.mx_quantize(h["W2t"])
    return dict(Xq=Xq, Xs=Xs, W1q=W1q, W1s=W1s, W2q=W2q, W2s=W2s)


def run_fwd(torch, dev, h, q, eps):
    import gemm_epilogue_fusion_gemm1_amd as coda
    M, K = h["X"].shape
    d, N = h["W1t"].shape[0], h["W2t"].shape[0]
    y = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    r = torch.empty((M,), dtype=torch.float32, device=dev)
    z = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    nb = coda.fwd_mx8_workspace_bytes(M, K, d, N)
    ws = torch.empty((nb,), dtype=torch.uint8, device=dev)
    coda.coda_fwd_mx8(u8(torch, dev, q["Xq"]), u8(torch, dev, blocked(q["Xs"])), u8(torch, dev, q["W1q"]),
                      u8(torch, dev, blocked(q["W1s"])), bf(torch, dev, h["R"]), bf(torch, dev, h["gamma"]),
                      u8(torch, dev, q["W2q"]), u8(torch, dev, blocked(q["W2s"])), eps, y, r, z, ws)
    torch.cuda.synchronize()
    # workspace layout (coda.h): partial sums, then q [M, d], then qs
    # (step-blocked [d/128, M, 4]), each at a 256-byte boundary
    def ru(x):
        return (x + 255) // 256 * 256
    off_q = ru(M * ((d + 255) // 256) * 4)
    off_qs = off_q + ru(M * d)
    w = ws.cpu().numpy()
    yq = w[off_q:off_q + M * d].reshape(M, d)
    ys = unblocked(w[off_qs:off_qs + M * (d // 32)].reshape(d // 128, M, 4))
    return y.float().cpu().numpy(), r.cpu().numpy(), z.float().cpu().numpy(), yq, ys


def accumulation_slack(Xq, Xs, W1q, W1s, gamma):
    """Per element (i, j) of y*gamma, the deviation allowed between the
    kernel's fp32 value and the exact one: 2^-10 times the sum, over the 64-k
    groups of one MFMA instruction, of the group's largest |X_ik W1_jk|, times
    |gamma_j|.  The MXFP8 matrix instruction sums its 64 products with
    reduced precision (an in-bounds probe measured up to 2^-12.6 of the
    largest product per instruction), so this is 4x that measurement."""
    X = oracle.mx_dequantize(Xq, Xs)
    W = oracle.mx_dequantize(W1q, W1s)
    rows, K = X.shape
    d = W.shape[0]
    out = np.empty((rows, d))
    Wg = np.abs(W).reshape(d, K // 64, 64)
    for i in range(rows):
        prod = np.abs(X[i]).reshape(1, K // 64, 64) * Wg          # [d, groups, 64]
        out[i] = prod.max(axis=2).sum(axis=1)
    return 2.0 ** -10 * out * np.abs(np.asarray(gamma, dtype=np.float64))[None, :]


def check_quantised_yg(name, yq, ys, ref, slack):
    """Codes and scales of y*gamma against the exact value (see the module
    docstring).  Each GPU element must be a correct rounding (under the GPU's
    scale) of a value within `slack` of the exact y*gamma; a scale may differ
    from the oracle's only where the exact block maximum is within the block's
    slack of a power of two; at most 1e-2 of the codes may differ."""
    ora_q, ora_s, yg = ref["yg_q"], ref["yg_s"], ref["yg"]
    rows, d = yg.shape
    amax = np.max(np.abs(yg.reshape(rows, d // 32, 32)), axis=2)
    bslack = np.max(slack.reshape(rows, d // 32, 32), axis=2)
    p2 = np.exp2(np.round(np.log2(np.maximum(amax, 1e-300))))
    s_diff = ys != ora_s
    assert np.all(np.abs(amax - p2)[s_diff] <= bslack[s_diff]), \
        f"{name}: a scale differs away from a power-of-two boundary"
    sc = np.repeat(oracle.e8m0_decode(ys), 32, axis=1)
    got = oracle.e4m3_decode(yq) * sc
    u = np.abs(yg) / sc
    half_step = 0.5 * np.where(u >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(u, 2.0 ** -6))) - 3),
                               2.0 ** -9) * sc
    err = np.abs(got - yg)
    sat = (u > 448.0) & (np.abs(got) == 448.0 * sc) & (np.sign(got) == np.sign(yg))
    ok = (err <= half_step * (1 + 1e-9) + slack) | sat
    if not ok.all():
        i, j = (int(v) for v in np.argwhere(~ok)[0])
        raise AssertionError(
            f"{name}: {int((~ok).sum())} codes are not a rounding of a value within the slack; first at "
            f"({i},{j}): exact {yg[i, j]!r}, gpu code {int(yq[i, j]):#x} -> {got[i, j]!r}, oracle code "
            f"{int(ora_q[i, j]):#x}, scale byte {int(ys[i, j // 32])}, slack {slack[i, j]:.3e}")
    nf_c, nf_s = float((yq != ora_q).mean()), float(s_diff.mean())
    assert nf_c <= FLIP_FRAC and nf_s <= FLIP_FRAC, (nf_c, nf_s)
    return nf_c, nf_s


# --------------------------------------------------------------- quantiser

def _quant_cases():
    g = np.random.default_rng(7)
    a = (g.standard_normal((300, 1152)) * np.exp2(g.integers(-20, 20, (300, 1)))).astype(np.float32)
    a[3, :64] = 0.0                                   # all-zero blocks
    a[4, :32] = -0.0
    a[5, :32] = 1e-39                                 # fp32-subnormal block maximum
    a[6, 7] = 3.0e38                                  # largest exponents
    a[7, :32] = np.linspace(-470, 470, 32)            # saturating elements under scale 1
    a[8, :32] = 2.0 ** -133                           # the smallest bf16 subnormal
    return [("ragged", synth.round_to_bf16(a)),
            ("one_step", synth.round_to_bf16(g.standard_normal((7, 128)).astype(np.float32))),
            ("wide", synth.round_to_bf16(g.standard_normal((64, 4096)).astype(np.float32)))]


@pytest.mark.parametrize("case", _quant_cases(), ids=lambda c: c[0])
def test_mx8_quantize_bit_exact(torch_dev, case):
    torch, dev = torch_dev
    import gemm_epilogue_fusion_gemm1_amd as coda
    name, a = case
    codes, scales = coda.mx8_quantize(bf(torch, dev, a))
    torch.cuda.synchronize()
    oq, os_ = oracle.mx_quantize(a.astype(np.float64))
    gq, gs = codes.cpu().numpy(), unblocked(scales.cpu().numpy())
    nq, ns = int((gq != oq).sum()), int((gs != os_).sum())
    report(f"mx8 quantize {name} {a.shape}", {"code_mismatches": nq, "scale_mismatches": ns})
    assert ns == 0 and nq == 0


# --------------------------------------------------------------- the block

SMALL_MX8 = [
    # M, K, d, N
    (520, 256, 384, 776),       # 3 x 2 x 4 tiles, M and N ragged, d a partial tile
    (8, 128, 128, 8),           # smallest accepted
    (256, 256, 256, 256),       # exactly one tile
    (264, 1152, 128, 40),       # long K loop, narrow d and N
    (768, 512, 1024, 520),      # several full tiles, 4 partials per row
]


@pytest.mark.parametrize("shape", SMALL_MX8, ids=lambda s: "x".join(map(str, s)))
def test_fwd_mx8(torch_dev, shape):
    torch, dev = torch_dev
    M, K, d, N = shape
    eps = 1e-6
    h = synth.mx8_inputs(M, K, d, N, seed=300 + M + K)
    q = quantised(h)
    y, r, z, yq, ys = run_fwd(torch, dev, h, q, eps)
    f = oracle.ref_fwd_mx8(q["Xq"], q["Xs"], q["W1q"], q["W1s"], h["R"], h["gamma"], q["W2q"], q["W2s"], eps)
    errs = {"y": rel(y, f["y"]), "z": rel(z, f["z"]),
            "r": float(np.max(np.abs(r - f["r"]) / f["r"]))}
    report(f"mx8 fwd {shape} (before the code check)", errs)
    slack = accumulation_slack(q["Xq"], q["Xs"], q["W1q"], q["W1s"], h["gamma"])
    nf_c, nf_s = check_quantised_yg(f"mx8 {shape}", yq, ys, f, slack)
    report(f"mx8 fwd {shape}", {**errs, "yg_code_flips": nf_c, "yg_scale_flips": nf_s})
    assert errs["y"] <= BF16_TOL and errs["z"] <= BF16_TOL and errs["r"] <= R_TOL


def test_full_workload_mx8(torch_dev):
    """LLaMA-7B-shaped block forward on MXFP8 operands, in the launch
    configuration the benchmark times: y, r, z and the quantised y*gamma on
    sampled rows (r for every row); the quantiser checked bit-exact on X."""
    torch, dev = torch_dev
    import gemm_epilogue_fusion_gemm1_amd as coda
    w = synth.WORKLOADS["llama7b_fwd_mx8"]
    h = synth.workload_inputs(w)
    q = quantised(h)
    gq, gs = coda.mx8_quantize(bf(torch, dev, h["X"]))
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), q["Xq"]) and np.array_equal(unblocked(gs.cpu().numpy()), q["Xs"])
    del gq, gs
    y, r, z, yq, ys = run_fwd(torch, dev, h, q, w.eps)
    # one row from every 128-row band (each wave row of every 256-row tile);
    # a row spans every column tile of both GEMMs
    rng = np.random.default_rng(w.seed)
    rows = np.unique(np.concatenate([[0, w.M - 1], [rng.integers(b, min(b + 128, w.M)) for b in range(0, w.M, 128)]]))
    f = oracle.ref_fwd_mx8_rows(q["Xq"], q["Xs"], q["W1q"], q["W1s"], h["R"], h["gamma"], q["W2q"],
                                q["W2s"], w.eps, rows)
    errs = {"y_rows": rel(y[rows], f["y"]), "z_rows": rel(z[rows], f["z"]),
            "r_rows": float(np.max(np.abs(r[rows] - f["r"]) / f["r"]))}
    report(f"{w.name} (before the code check)", errs)
    slack = accumulation_slack(q["Xq"][rows], q["Xs"][rows], q["W1q"], q["W1s"], h["gamma"])
    nf_c, nf_s = check_quantised_yg("mx8 7B rows", yq[rows], ys[rows], f, slack)
    report(w.name, {**errs, "yg_code_flips": nf_c, "yg_scale_flips": nf_s})
    assert errs["y_rows"] <= BF16_TOL and errs["z_rows"] <= BF16_TOL and errs["r_rows"] <= R_TOL
    assert np.all(np.isfinite(z)) and np.all(r > 0)

# ----------------------------------------------------------- MXFP8 backward

SMALL_BWD_MX8 = [
    # M, K, d, N (M, d, N whole 128-k steps; K ragged)
    (256, 136, 256, 384),
    (128, 8, 128, 128),          # smallest accepted
    (640, 1032, 384, 1152),      # several tiles, K tail, d and N not multiples of 256
    (384, 264, 512, 256),
]


def _mx8_bwd_inputs(M, K, d, N, seed, eps=1e-6):
    """The backward's inputs: the draws of the bf16 block and its saved y
    (rounded to bf16) and r from the oracle's forward."""
    h = synth.coda_inputs(M, K, d, N, seed=seed, dtype="bf16")
    yr = oracle.ref_y_r(h["X"], h["W1"], h["R"], eps)
    return h, oracle.bf16_rne(yr["y"]), yr["r"]


def _run_bwd_mx8(torch, dev, h, y, r):
    import gemm_epilogue_fusion_gemm1_amd as coda
    t = {k: bf(torch, dev, v) for k, v in h.items() if k != "R"}
    ty = bf(torch, dev, y)
    tr = torch.from_numpy(np.asarray(r, np.float32)).to(dev)
    out = coda.bwd_mx8(t["X"], t["W1"], t["gamma"], t["W2"], ty, tr, t["dz"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("shape", SMALL_BWD_MX8, ids=lambda s: "x".join(map(str, s)))
def test_bwd_mx8(torch_dev, shape):
    torch, dev = torch_dev
    M, K, d, N = shape
    h, y, r = _mx8_bwd_inputs(M, K, d, N, seed=800 + M + K)
    dX, dW1, dR, dW2, dg = _run_bwd_mx8(torch, dev, h, y, r)
    b = oracle.ref_bwd_mx8(h["X"], h["W1"], h["gamma"], h["W2"], y, r, h["dz"])
    f = lambda t: t.float().cpu().numpy()  # noqa: E731
    errs = {"dX": rel(f(dX), b["dX"]), "dW1": rel(f(dW1), b["dW1"]), "dR": rel(f(dR), b["dR"]),
            "dW2": rel(f(dW2), b["dW2"]), "dgamma": rel(dg.cpu().numpy(), b["dgamma"])}
    # beside it: the distance from the unquantised backward (the MXFP8 error itself)
    e = oracle.ref_bwd(h["X"], h["W1"], h["gamma"], h["W2"], y, r, h["dz"])
    info = {f"{k}_vs_unquantised": rel(f(v), e[k]) for k, v in (("dX", dX), ("dW1", dW1), ("dW2", dW2))}
    report(f"mx8 bwd {shape}", {**errs, **info})
    for k in ("dX", "dW1", "dR", "dW2"):
        assert errs[k] <= BF16_TOL, (k, errs[k])
    assert errs["dgamma"] <= 1e-3


def test_bwd_mx8_deterministic(torch_dev):
    torch, dev = torch_dev
    h, y, r = _mx8_bwd_inputs(640, 1032, 384, 1152, seed=820)
    a = _run_bwd_mx8(torch, dev, h, y, r)
    b = _run_bwd_mx8(torch, dev, h, y, r)
    for x_, y_ in zip(a, b):
        assert torch.equal(x_, y_)


def test_full_workload_bwd_mx8(torch_dev):
    """LLaMA-7B-shaped MXFP8 backward: dX and dR on stratified rows (one per
    128-row band), dW1 and dW2 on stratified columns (one per 64-column
    band), dgamma in full."""
    torch, dev = torch_dev
    w = synth.WORKLOADS["llama7b_fwdbwd_mx8"]
    print(f"[parity] {w.name}: inputs and the oracle's forward", flush=True)
    h, y, r = _mx8_bwd_inputs(w.M, w.K, w.d, w.N, seed=w.seed, eps=w.eps)
    dX, dW1, dR, dW2, dg = _run_bwd_mx8(torch, dev, h, y, r)
    rng = np.random.default_rng(w.seed)
    strata = lambda n, band: np.unique(np.concatenate([[0, n - 1], [rng.integers(b0, min(b0 + band, n)) for b0 in range(0, n, band)]]))  # noqa: E731
    rows, cd, cn = strata(w.M, 128), strata(w.d, 64), strata(w.N, 64)
    print(f"[parity] {w.name}: oracle backward (sampled)", flush=True)
    b = oracle.ref_bwd_mx8_sampled(h["X"], h["W1"], h["gamma"], h["W2"], y, r, h["dz"], rows, cd, cn)
    f = lambda t: t.float().cpu().numpy()  # noqa: E731
    errs = {"dX_rows": rel(f(dX[rows]), b["dX_rows"]), "dR_rows": rel(f(dR[rows]), b["dR_rows"]),
            "dW1_cols": rel(f(dW1[:, cd]), b["dW1_cols"]), "dW2_cols": rel(f(dW2[:, cn]), b["dW2_cols"]),
            "dgamma": rel(dg.cpu().numpy(), b["dgamma"])}
    report(w.name, errs)
    for k in ("dX_rows", "dR_rows", "dW1_cols", "dW2_cols"):
        assert errs[k] <= BF16_TOL, (k, errs[k])
    assert errs["dgamma"] <= 1e-3


def test_bwd_mx8_max_rows(torch_dev):
    """The largest accepted token count, M = 2^23: the passes that quantise
    along M run over 65536 blocks of 128 rows.  K = 8, d = N = 128, and dz
    is nonzero in six rows only (the first, the last, one in the last
    128-row block and three between), so every gradient vanishes outside
    those rows (dn = 0 there, hence s = c = 0 and dy = 0) and every sum over
    M gets terms from their 32-row quantisation blocks alone.  Whole aligned
    32-row blocks quantise along M as they do inside the full matrix, so the
    oracle's backward on the gathered blocks is the full one: dX and dR are
    compared on those rows and must be exactly zero on every other row;
    dW1, dW2 and dgamma are compared in full.  The bulk inputs come from
    torch's seeded generator on the device; W1, W2 and gamma from the
    workload draws."""
    torch, dev = torch_dev
    import gemm_epilogue_fusion_gemm1_amd as coda
    M, K, d, N = 1 << 23, 8, 128, 128
    hot = np.array([0, 77, 123457, (1 << 22) + 3, M - 100, M - 1])
    blocks = np.unique(hot // 32)
    rows = (blocks[:, None] * 32 + np.arange(32)[None, :]).ravel()
    print(f"[parity] mx8 bwd M=2^23: inputs ({len(rows)} rows in {len(blocks)} blocks checked)", flush=True)
    g = torch.Generator(device=dev)
    g.manual_seed(9090)
    X = torch.randn((M, K), generator=g, device=dev, dtype=torch.bfloat16)
    y = torch.randn((M, d), generator=g, device=dev, dtype=torch.bfloat16)
    r = 0.5 + torch.rand((M,), generator=g, device=dev, dtype=torch.float32)
    dz = torch.zeros((M, N), dtype=torch.bfloat16, device=dev)
    hot_t = torch.from_numpy(hot).to(dev)
    dz[hot_t] = torch.randn((len(hot), N), generator=g, device=dev, dtype=torch.bfloat16)
    w = synth.coda_inputs(128, K, d, N, seed=9091, dtype="bf16")
    W1, gamma, W2 = bf(torch, dev, w["W1"]), bf(torch, dev, w["gamma"]), bf(torch, dev, w["W2"])
    print("[parity] mx8 bwd M=2^23: coda_bwd_mx8", flush=True)
    dX, dW1, dR, dW2, dg = coda.bwd_mx8(X, W1, gamma, W2, y, r, dz)
    torch.cuda.synchronize()
    rows_t = torch.from_numpy(rows).to(dev)
    rest = torch.ones((M,), dtype=torch.bool, device=dev)
    rest[rows_t] = False
    zero_dX = int(torch.count_nonzero(dX[rest]))
    zero_dR = int(torch.count_nonzero(dR[rest]))
    f = lambda t: t.float().cpu().numpy()  # noqa: E731
    print("[parity] mx8 bwd M=2^23: oracle on the gathered blocks", flush=True)
    b = oracle.ref_bwd_mx8(f(X[rows_t]), f(W1), f(gamma), f(W2), f(y[rows_t]), r[rows_t].cpu().numpy(),
                           f(dz[rows_t]))
    errs = {"dX_rows": rel(f(dX[rows_t]), b["dX"]), "dR_rows": rel(f(dR[rows_t]), b["dR"]),
            "dW1": rel(f(dW1), b["dW1"]), "dW2": rel(f(dW2), b["dW2"]),
            "dgamma": rel(dg.cpu().numpy(), b["dgamma"]), "nonzero_dX_elsewhere": zero_dX,
            "nonzero_dR_elsewhere": zero_dR}
    report("mx8 bwd M=2^23", errs)
    del X, y, r, dz, dX, dR, rest                      # ~14 GB: give it back before the next test
    torch.cuda.empty_cache()
    assert zero_dX == 0 and zero_dR == 0
    for k in ("dX_rows", "dR_rows", "dW1", "dW2"):
        assert errs[k] <= BF16_TOL, (k, errs[k])
    assert errs["dgamma"] <= 1e-3


# ---------------------------------------------------------------- SwiGLU block

SMALL_SWIGLU_MX8 = [
    (128, 128, 128),           # smallest accepted: one gated tile, one K step
    (256, 384, 256),
    (384, 256, 640),           # F not a multiple of the 256-column tile
    (640, 1152, 384),          # several tiles, d not a multiple of 256
    (1024, 512, 1280),
]


def _run_swiglu_mx8(torch, dev, h, gu=None, a=None):
    import gemm_epilogue_fusion_gemm1_amd as coda
    t = {k: bf(torch, dev, v) for k, v in h.items()}
    if gu is None:
        out = coda.swiglu_fwd_mx8(t["X"], t["W"], t["Wd"])
    else:
        out = coda.swiglu_bwd_mx8(t["X"], t["W"], t["Wd"], bf(torch, dev, gu), bf(torch, dev, a), t["dz"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("shape", SMALL_SWIGLU_MX8, ids=lambda s: "x".join(map(str, s)))
def test_swiglu_mx8(torch_dev, shape):
    """Forward outputs against ``ref_swiglu_fwd_mx8``; the backward, fed the
    oracle's saved gu and a (bf16), against ``ref_swiglu_bwd_mx8``; the
    distance from the unquantised block reported beside them."""
    torch, dev = torch_dev
    M, d, F = shape
    h = synth.swiglu_inputs(M, d, F, seed=830 + M + F)
    z, gu, a = _run_swiglu_mx8(torch, dev, h)
    f = oracle.ref_swiglu_fwd_mx8(h["X"], h["W"], h["Wd"])
    g = lambda v: v.float().cpu().numpy()  # noqa: E731
    errs = {"z": rel(g(z), f["z"]), "gu": rel(g(gu), f["gu"]), "a": rel(g(a), f["a"])}
    gu_s, a_s = oracle.bf16_rne(f["gu"]), oracle.bf16_rne(f["a"])
    dX, dW, dWd = _run_swiglu_mx8(torch, dev, h, gu_s, a_s)
    b = oracle.ref_swiglu_bwd_mx8(h["X"], h["W"], h["Wd"], gu_s, a_s, h["dz"])
    errs.update(dX=rel(g(dX), b["dX"]), dW=rel(g(dW), b["dW"]), dWd=rel(g(dWd), b["dWd"]))
    e = oracle.ref_swiglu_bwd(h["X"], h["W"], h["Wd"], gu_s, a_s, h["dz"])
    info = {f"{k}_vs_unquantised": rel(g(v), e[k]) for k, v in (("dX", dX), ("dW", dW), ("dWd", dWd))}
    report(f"swiglu mx8 {shape}", {**errs, **info})
    for k, v in errs.items():
        assert v <= BF16_TOL, (k, v)


def test_swiglu_mx8_deterministic(torch_dev):
    torch, dev = torch_dev
    h = synth.swiglu_inputs(384, 256, 640, seed=850)
    f1 = _run_swiglu_mx8(torch, dev, h)
    f2 = _run_swiglu_mx8(torch, dev, h)
    gu, a = f1[1].float().cpu().numpy(), f1[2].float().cpu().numpy()
    b1 = _run_swiglu_mx8(torch, dev, h, gu, a)
    b2 = _run_swiglu_mx8(torch, dev, h, gu, a)
    for x_, y_ in zip(f1 + b1, f2 + b2):
        assert torch.equal(x_, y_)


def test_full_workload_swiglu_mx8(torch_dev):
    """The SwiGLU shape (M = 8192, d = 4096, F = 14336) on MXFP8: forward rows
    and the backward (fed the GPU forward's saved gu and a, as in training)
    on stratified rows, dW columns and dWd rows, one from every 128-row /
    64-column band, against the oracle's chain."""
    torch, dev = torch_dev
    w = synth.WORKLOADS["swiglu_fwdbwd_mx8"]
    print(f"[parity] {w.name}: inputs", flush=True)
    h = synth.workload_inputs(w)
    z, gu, a = _run_swiglu_mx8(torch, dev, h)
    t = {k: bf(torch, dev, v) for k, v in h.items()}
    import gemm_epilogue_fusion_gemm1_amd as coda
    dX, dW, dWd = coda.swiglu_bwd_mx8(t["X"], t["W"], t["Wd"], gu, a, t["dz"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    strata = lambda n, band: np.unique(np.concatenate([[0, n - 1], [rng.integers(b0, min(b0 + band, n)) for b0 in range(0, n, band)]]))  # noqa: E731
    rows, cols_W, rows_Wd = strata(w.M, 128), strata(2 * w.F, 64), strata(w.F, 64)
    print(f"[parity] {w.name}: oracle (sampled)", flush=True)
    fr = oracle.ref_swiglu_fwd_mx8_rows(h["X"], h["W"], h["Wd"], rows)
    b = oracle.ref_swiglu_bwd_mx8_sampled(h["X"], h["W"], h["Wd"], h["dz"], rows, cols_W, rows_Wd)
    g = lambda v: v.float().cpu().numpy()  # noqa: E731
    errs = {"z_rows": rel(g(z[rows]), fr["z"]), "gu_rows": rel(g(gu[rows]), fr["gu"]),
            "a_rows": rel(g(a[rows]), fr["a"]), "dX_rows": rel(g(dX[rows]), b["dX_rows"]),
            "dW_cols": rel(g(dW[:, cols_W]), b["dW_cols"]), "dWd_rows": rel(g(dWd[rows_Wd]), b["dWd_rows"])}
    report(w.name, errs)
    for k, v in errs.items():
        assert v <= BF16_TOL, (k, v)


def test_swiglu_mx8_max_rows(torch_dev):
    """The SwiGLU block on MXFP8 at the largest accepted token count, M =
    2^23 (d = F = 128): gu is 4 GiB and the MXFP8 dgu 2 GiB, so the backward
    GEMMs reach dgu through buffer windows, and the passes along M (a, X and
    dz, and dgu in the da GEMM's epilogue) run over 65536 row blocks.  The
    forward on sampled rows (row-local: X, a and the weights are quantised
    along d and F).  The backward, fed the forward's gu and a, with dz
    nonzero in six rows: da, dgu and dX vanish on every other row and the
    sums over M take terms from those rows' 32-row quantisation blocks alone,
    so the oracle on the gathered blocks is the full one (a CPU pin checks
    this); dX must be exactly zero outside those blocks.  The bulk inputs
    come from torch's seeded generator on the device; W and Wd from the
    workload draws."""
    torch, dev = torch_dev
    import gemm_epilogue_fusion_gemm1_amd as coda
    M, d, F = 1 << 23, 128, 128
    hot = np.array([0, 77, 123457, (1 << 22) + 3, M - 100, M - 1])
    blocks = np.unique(hot // 32)
    brows = (blocks[:, None] * 32 + np.arange(32)[None, :]).ravel()
    print("[parity] swiglu mx8 M=2^23: inputs", flush=True)
    g = torch.Generator(device=dev)
    g.manual_seed(9290)
    X = torch.randn((M, d), generator=g, device=dev, dtype=torch.bfloat16)
    dz = torch.zeros((M, d), dtype=torch.bfloat16, device=dev)
    hot_t = torch.from_numpy(hot).to(dev)
    dz[hot_t] = torch.randn((len(hot), d), generator=g, device=dev, dtype=torch.bfloat16)
    w = synth.swiglu_inputs(128, d, F, seed=9291)
    W, Wd = bf(torch, dev, w["W"]), bf(torch, dev, w["Wd"])
    print("[parity] swiglu mx8 M=2^23: forward and backward", flush=True)
    z, gu, a = coda.swiglu_fwd_mx8(X, W, Wd)
    dX, dW, dWd = coda.swiglu_bwd_mx8(X, W, Wd, gu, a, dz)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M), np.arange(5, M, 1 << 20), hot]))
    rows_t, brows_t = torch.from_numpy(rows).to(dev), torch.from_numpy(brows).to(dev)
    rest = torch.ones((M,), dtype=torch.bool, device=dev)
    rest[brows_t] = False
    nz_dX = int(torch.count_nonzero(dX[rest]))
    h = lambda v: v.float().cpu().numpy()  # noqa: E731
    Wh, Wdh = h(W), h(Wd)
    print("[parity] swiglu mx8 M=2^23: oracle on the sampled rows and gathered blocks", flush=True)
    f = oracle.ref_swiglu_fwd_mx8(h(X[rows_t]), Wh, Wdh)
    b = oracle.ref_swiglu_bwd_mx8(h(X[brows_t]), Wh, Wdh, h(gu[brows_t]), h(a[brows_t]), h(dz[brows_t]))
    errs = {"z_rows": rel(h(z[rows_t]), f["z"]), "gu_rows": rel(h(gu[rows_t]), f["gu"]),
            "a_rows": rel(h(a[rows_t]), f["a"]), "dX_blocks": rel(h(dX[brows_t]), b["dX"]),
            "dW": rel(h(dW), b["dW"]), "dWd": rel(h(dWd), b["dWd"])}
    report("swiglu mx8 M=2^23", {**errs, "nonzero_dX_elsewhere": nz_dX})
    del X, dz, z, gu, a, dX, rest                      # ~25 GB: give it back before the next test
    torch.cuda.empty_cache()
    assert nz_dX == 0
    for k, v in errs.items():
        assert v <= BF16_TOL, (k, v)


# ----------------------------------------------------------- MLP sub-layer

SMALL_MLP_MX8 = [
    (128, 128, 128, 128),        # smallest accepted
    (256, 384, 256, 384),
    (384, 256, 384, 640),        # F not a multiple of the 256-column tile
    (640, 1152, 256, 128),       # several row tiles, long K
]
R_ELEM_TOL = 1e-3
# Behind a quantisation point (y*gamma, a, dgu, dn/n/dy) the GPU rounds values
# that differ from the oracle's by the matrix instruction's accumulation
# error, so an E4M3 code flips wherever a value lies that close to a rounding
# boundary, and a flip moves its element by one E4M3 step.  Four such points
# in a row make the outputs' max-norm error a matter of which flips land
# where; the bar there is normwise (Frobenius) 2e-2, with 1e-1 on the
# max-norm as a guard.  An emulation of the chain with every GPU-computed
# product perturbed by 2^-12 (relative) gives 1.0-1.8e-2 normwise and up to
# 6e-2 max-norm at these shapes; a wiring mistake (an operand, a scale
# layout, dy_in) moves the normwise error far beyond 5e-2.
CHAIN_NORM_TOL = 2e-2
CHAIN_MAX_TOL = 1e-1


def nrel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref)) / max(float(np.linalg.norm(ref)), 1e-300)


def _check_chain(errs, nerrs, keys):
    for k in keys:
        assert nerrs[k] <= CHAIN_NORM_TOL, (k, "normwise", nerrs[k])
        assert errs[k] <= CHAIN_MAX_TOL, (k, "max-norm", errs[k])


def _mlp_mx8_gpu(torch, dev, h, saved=None):
    import gemm_epilogue_fusion_gemm1_amd as coda
    t = {k: bf(torch, dev, v) for k, v in h.items()}
    if saved is None:
        out = coda.mlp_fwd_mx8(t["X"], t["W1"], t["R"], t["gamma"], t["W"], t["Wd"], 1e-6)
    else:
        y, r, gu, a = saved
        out = coda.mlp_bwd_mx8(t["X"], t["W1"], t["gamma"], t["W"], t["Wd"], y, r, gu, a, t["dz"], t["dy_in"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("shape", SMALL_MLP_MX8, ids=lambda s: "x".join(map(str, s)))
def test_mlp_mx8(torch_dev, shape):
    """Forward against ``ref_mlp_fwd_mx8``; the backward (with dy_in), fed the
    oracle's saved y, r, gu and a, against ``ref_mlp_bwd_mx8``."""
    torch, dev = torch_dev
    M, K, d, F = shape
    h = synth.mlp_inputs(M, K, d, F, seed=860 + M + F)
    z, y, r, gu, a = _mlp_mx8_gpu(torch, dev, h)
    f = oracle.ref_mlp_fwd_mx8(h["X"], h["W1"], h["R"], h["gamma"], h["W"], h["Wd"], 1e-6)
    g = lambda v: v.float().cpu().numpy()  # noqa: E731
    errs = {"y": rel(g(y), f["y"]), "gu": rel(g(gu), f["gu"]), "a": rel(g(a), f["a"]), "z": rel(g(z), f["z"])}
    rr = float(np.max(np.abs(r.cpu().numpy() - f["r"]) / f["r"]))
    sv = {k: oracle.bf16_rne(f[k]) for k in ("y", "gu", "a")}
    saved = (bf(torch, dev, sv["y"]), torch.from_numpy(np.asarray(f["r"], np.float32)).to(dev),
             bf(torch, dev, sv["gu"]), bf(torch, dev, sv["a"]))
    dX, dW1, dR, dW, dWd, dg = _mlp_mx8_gpu(torch, dev, h, saved)
    b = oracle.ref_mlp_bwd_mx8(h["X"], h["W1"], h["gamma"], h["W"], h["Wd"], sv["y"], f["r"], sv["gu"], sv["a"],
                               h["dz"], h["dy_in"])
    errs.update(dX=rel(g(dX), b["dX"]), dW1=rel(g(dW1), b["dW1"]), dR=rel(g(dR), b["dR"]), dW=rel(g(dW), b["dW"]),
                dWd=rel(g(dWd), b["dWd"]), dgamma=rel(dg.cpu().numpy(), b["dgamma"]))
    outs = {"gu": (gu, f["gu"]), "a": (a, f["a"]), "z": (z, f["z"]), "dX": (dX, b["dX"]), "dW1": (dW1, b["dW1"]),
            "dR": (dR, b["dR"]), "dW": (dW, b["dW"]), "dWd": (dWd, b["dWd"]), "dgamma": (dg, b["dgamma"])}
    nerrs = {k: nrel(g(v), ref) for k, (v, ref) in outs.items()}
    report(f"mlp mx8 {shape}", {**errs, "r": rr})
    report(f"mlp mx8 {shape} normwise", nerrs)
    assert rr <= R_ELEM_TOL
    assert errs["y"] <= BF16_TOL
    _check_chain(errs, nerrs, outs)


def test_mlp_mx8_deterministic(torch_dev):
    torch, dev = torch_dev
    h = synth.mlp_inputs(384, 256, 384, 640, seed=870)
    f1 = _mlp_mx8_gpu(torch, dev, h)
    f2 = _mlp_mx8_gpu(torch, dev, h)
    b1 = _mlp_mx8_gpu(torch, dev, h, f1[1:])
    b2 = _mlp_mx8_gpu(torch, dev, h, f1[1:])
    for x_, y_ in zip(f1 + b1, f2 + b2):
        assert torch.equal(x_, y_)


def test_full_workload_mlp_mx8(torch_dev):
    """The LLaMA-7B MLP shape on MXFP8 (M = 8192, K = d = 4096, F = 11008, with
    dy_in): forward rows; the backward, fed the GPU forward's saved tensors,
    on stratified rows and columns with dgamma in full, against the oracle's
    chain (its own forward, saved tensors rounded to bf16)."""
    torch, dev = torch_dev
    import gemm_epilogue_fusion_gemm1_amd as coda
    w = synth.WORKLOADS["llama7b_mlp_fwdbwd_mx8"]
    print(f"[parity] {w.name}: inputs", flush=True)
    h = synth.workload_inputs(w)
    t = {k: bf(torch, dev, v) for k, v in h.items()}
    z, y, r, gu, a = coda.mlp_fwd_mx8(t["X"], t["W1"], t["R"], t["gamma"], t["W"], t["Wd"], w.eps)
    dX, dW1, dR, dW, dWd, dg = coda.mlp_bwd_mx8(t["X"], t["W1"], t["gamma"], t["W"], t["Wd"], y, r, gu, a, t["dz"],
                                               t["dy_in"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    strata = lambda n, band: np.unique(np.concatenate([[0, n - 1], [rng.integers(b0, min(b0 + band, n)) for b0 in range(0, n, band)]]))  # noqa: E731
    rows, cd, c2, rF = strata(w.M, 128), strata(w.d, 64), strata(2 * w.F, 64), strata(w.F, 64)
    print(f"[parity] {w.name}: oracle forward (full: the backward needs every row)", flush=True)
    f = oracle.ref_mlp_fwd_mx8(h["X"], h["W1"], h["R"], h["gamma"], h["W"], h["Wd"], w.eps)
    g = lambda v: v.float().cpu().numpy()  # noqa: E731
    errs = {"z_rows": rel(g(z[rows]), f["z"][rows]), "y_rows": rel(g(y[rows]), f["y"][rows]),
            "gu_rows": rel(g(gu[rows]), f["gu"][rows]), "a_rows": rel(g(a[rows]), f["a"][rows])}
    rr = float(np.max(np.abs(r.cpu().numpy() - f["r"]) / f["r"]))
    print(f"[parity] {w.name}: oracle backward (sampled)", flush=True)
    sv = {k: oracle.bf16_rne(f[k]) for k in ("y", "gu", "a")}
    b = oracle.ref_mlp_bwd_mx8_sampled(h["X"], h["W1"], h["gamma"], h["W"], h["Wd"], sv["y"], f["r"], sv["gu"],
                                       sv["a"], h["dz"], h["dy_in"], rows, cd, c2, rF)
    outs = {"z_rows": (z[rows], f["z"][rows]), "gu_rows": (gu[rows], f["gu"][rows]),
            "a_rows": (a[rows], f["a"][rows]), "dX_rows": (dX[rows], b["dX_rows"]),
            "dR_rows": (dR[rows], b["dR_rows"]), "dW1_cols": (dW1[:, cd], b["dW1_cols"]),
            "dW_cols": (dW[:, c2], b["dW_cols"]), "dWd_rows": (dWd[rF], b["dWd_rows"]),
            "dgamma": (dg, b["dgamma"])}
    errs.update({k: rel(g(v), ref) for k, (v, ref) in outs.items()})
    nerrs = {k: nrel(g(v), ref) for k, (v, ref) in outs.items()}
    report(w.name, {**errs, "r": rr})
    report(f"{w.name} normwise", nerrs)
    assert rr <= R_ELEM_TOL
    assert errs["y_rows"] <= BF16_TOL
    _check_chain(errs, nerrs, outs)


def test_mx8_graph_capture_replays_match_eager(torch_dev):
    """The MXFP8 SwiGLU and MLP steps (forward + backward; the calls quantise
    their inputs, so every quantiser runs too) captured into a HIP graph
    replay bitwise equal to the eager calls, on every replay, with eager
    calls and synchronisations between the replays."""
    torch, dev = torch_dev
    import gemm_epilogue_fusion_gemm1_amd as coda
    M, K, d, F = 384, 256, 384, 640
    hs = synth.swiglu_inputs(M, d, F, seed=880)
    hm = synth.mlp_inputs(M, K, d, F, seed=881)
    ts = {k: bf(torch, dev, v) for k, v in hs.items()}
    tm = {k: bf(torch, dev, v) for k, v in hm.items()}
    e = lambda *shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
    b = dict(gu=e(M, 2 * F), a=e(M, F), z=e(M, d), dX=e(M, d), dW=e(d, 2 * F), dWd=e(F, d),
             y=e(M, d), r=e(M, dt=torch.float32), gu2=e(M, 2 * F), a2=e(M, F), z2=e(M, d), dX2=e(M, K),
             dW1=e(K, d), dR=e(M, d), dW2=e(d, 2 * F), dWd2=e(F, d), dg=e(d, dt=torch.float32))
    u8 = lambda n: torch.empty((n,), dtype=torch.uint8, device=dev)  # noqa: E731
    ws = [u8(coda.swiglu_fwd_mx8_workspace_bytes(M, d, F)), u8(coda.swiglu_bwd_mx8_workspace_bytes(M, d, F)),
          u8(coda.mlp_fwd_mx8_workspace_bytes(M, K, d, F)), u8(coda.mlp_bwd_mx8_workspace_bytes(M, K, d, F))]

    def step():
        coda.coda_swiglu_fwd_mx8(ts["X"], ts["W"], ts["Wd"], b["gu"], b["a"], b["z"], ws[0])
        coda.coda_swiglu_bwd_mx8(ts["X"], ts["W"], ts["Wd"], b["gu"], b["a"], ts["dz"], b["dX"], b["dW"], b["dWd"],
                                 ws[1])
        coda.coda_mlp_fwd_mx8(tm["X"], tm["W1"], tm["R"], tm["gamma"], tm["W"], tm["Wd"], 1e-6, b["y"], b["r"],
                              b["gu2"], b["a2"], b["z2"], ws[2])
        coda.coda_mlp_bwd_mx8(tm["X"], tm["W1"], tm["gamma"], tm["W"], tm["Wd"], b["y"], b["r"], b["gu2"], b["a2"],
                              tm["dz"], tm["dy_in"], b["dX2"], b["dW1"], b["dR"], b["dW2"], b["dWd2"], b["dg"], ws[3])

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in b.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in b.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in b.items():
            assert torch.equal(v, ref[k]), f"replay {rep}: {k} differs from the eager result"
        step()
        torch.cuda.synchronize()
    report("mx8 graph capture", {"replays": 3.0})

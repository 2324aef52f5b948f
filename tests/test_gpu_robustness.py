"""GPU behaviour beyond plain parity, each against the oracle or the library's
own contract:

  * non-finite inputs: a NaN or an infinity placed in an input reaches exactly
    the outputs the oracle's IEEE arithmetic sends it to (the same NaN / +inf /
    -inf pattern), and every finite output stays within the bf16 bar;
  * bitwise run-to-run determinism of every fused pattern (no atomics);
  * the binding refuses tensors of the wrong dtype, shape or device before
    any launch (outputs keep their contents);
  * cross-entropy rows whose label lies outside [0, V) are ignored.
"""
import numpy as np
import pytest

import oracle
from gemm_epilogue_fusion_gemm1_amd import synth

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_epilogue_fusion_gemm1_amd as coda
    coda.load_library()
    return torch, torch.device("cuda:0"), coda


def up(torch, dev, arr):
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev).to(torch.bfloat16)


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def same_nonfinite(name, got, ref):
    """The NaN, +inf and -inf positions agree; the finite entries are within
    the bf16 bar of the finite reference entries."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    for kind, f in (("nan", np.isnan), ("+inf", np.isposinf), ("-inf", np.isneginf)):
        g, r = f(got), f(ref)
        assert np.array_equal(g, r), f"{name}: {kind} at {np.argwhere(g != r)[:4].tolist()} differs"
    fin = np.isfinite(ref)
    if fin.any():
        den = max(float(np.max(np.abs(ref[fin]))), 1e-300)
        err = float(np.max(np.abs(got[fin] - ref[fin]))) / den
        assert err <= BF16_TOL, (name, err)
    return int(np.count_nonzero(~fin))


# ------------------------------------------------------------ non-finite inputs

CODA_NONFINITE = [
    ("X", (3, 5), np.nan),
    ("R", (7, 2), np.inf),
    ("W2", (4, 9), -np.inf),
    ("dz", (11, 1), np.nan),
]


@pytest.mark.parametrize("where", CODA_NONFINITE, ids=lambda c: f"{c[0]}{c[1]}={c[2]}")
def test_coda_nonfinite_propagates(env, where):
    torch, dev, coda = env
    M, K, d, N, eps = 264, 136, 272, 520, 1e-6
    h = synth.coda_inputs(M, K, d, N, seed=700, dtype="bf16")
    name, idx, val = where
    h[name][idx] = val
    t = {k: up(torch, dev, v) for k, v in h.items()}
    z, y, r = coda.fwd(t["X"], t["W1"], t["R"], t["gamma"], t["W2"], eps)
    dX, dW1, dR, dW2, dg = coda.bwd(t["X"], t["W1"], t["gamma"], t["W2"], y, r, t["dz"])
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        f = oracle.ref_fwd(h["X"], h["W1"], h["R"], h["gamma"], h["W2"], eps)
        b = oracle.ref_bwd(h["X"], h["W1"], h["gamma"], h["W2"], oracle.bf16_rne(f["y"]), f["r"], h["dz"])
    n = {}
    for k, g_, ref in (("y", y, f["y"]), ("z", z, f["z"]), ("dX", dX, b["dX"]), ("dW1", dW1, b["dW1"]),
                       ("dR", dR, b["dR"]), ("dW2", dW2, b["dW2"])):
        n[k] = same_nonfinite(k, host(g_), ref)
    for k, g_, ref in (("r", r, f["r"]), ("dgamma", dg, b["dgamma"])):
        got = g_.cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.array_equal(np.isinf(got), np.isinf(ref)), k
        n[k] = int(np.count_nonzero(~np.isfinite(ref)))
    print(f"[nonfinite] coda {where}: non-finite counts {n}", flush=True)
    assert sum(n.values()) > 0


def test_swiglu_mlp_ce_rope_nonfinite(env):
    torch, dev, coda = env
    # SwiGLU: NaN in X
    hs = synth.swiglu_inputs(264, 136, 200, seed=701)
    hs["X"][5, 7] = np.nan
    ts = {k: up(torch, dev, v) for k, v in hs.items()}
    z, gu, a = coda.swiglu_fwd(ts["X"], ts["W"], ts["Wd"])
    dX, dW, dWd = coda.swiglu_bwd(ts["X"], ts["W"], ts["Wd"], gu, a, ts["dz"])
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        f = oracle.ref_swiglu_fwd(hs["X"], hs["W"], hs["Wd"])
        b = oracle.ref_swiglu_bwd(hs["X"], hs["W"], hs["Wd"], oracle.bf16_rne(f["gu"]), oracle.bf16_rne(f["a"]),
                                  hs["dz"])
    for k, g_, ref in (("gu", gu, f["gu"]), ("a", a, f["a"]), ("z", z, f["z"]), ("dX", dX, b["dX"]),
                       ("dW", dW, b["dW"]), ("dWd", dWd, b["dWd"])):
        same_nonfinite(f"swiglu {k}", host(g_), ref)
    # MLP sub-layer: +inf in R
    hm = synth.mlp_inputs(264, 136, 272, 200, seed=702)
    hm["R"][9, 3] = np.inf
    tm = {k: up(torch, dev, v) for k, v in hm.items()}
    eps = 1e-6
    z, y, r, gu, a = coda.mlp_fwd(tm["X"], tm["W1"], tm["R"], tm["gamma"], tm["W"], tm["Wd"], eps)
    grads = coda.mlp_bwd(tm["X"], tm["W1"], tm["gamma"], tm["W"], tm["Wd"], y, r, gu, a, tm["dz"], tm["dy_in"])
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        fq = oracle.ref_mlp_fwd(hm["X"], hm["W1"], hm["R"], hm["gamma"], hm["W"], hm["Wd"], eps, oracle.bf16_rne)
        bm = oracle.ref_mlp_bwd(hm["X"], hm["W1"], hm["gamma"], hm["W"], hm["Wd"], oracle.bf16_rne(fq["y"]),
                                fq["r"], oracle.bf16_rne(fq["gu"]), oracle.bf16_rne(fq["a"]), hm["dz"],
                                hm["dy_in"], dgu_round=oracle.bf16_rne)
    for k, g_, ref in (("y", y, fq["y"]), ("gu", gu, fq["gu"]), ("a", a, fq["a"]), ("z", z, fq["z"])):
        same_nonfinite(f"mlp {k}", host(g_), ref)
    for k, g_ in zip(("dX", "dW1", "dR", "dW", "dWd"), grads[:5]):
        same_nonfinite(f"mlp {k}", host(g_), bm[k])
    # cross-entropy: NaN in h (its row's logits, lse and loss are NaN)
    hc = synth.ce_inputs(264, 136, 1000, seed=703)
    hc["h"][4, 2] = np.nan
    th, tW = up(torch, dev, hc["h"]), up(torch, dev, hc["Wv"])
    tl = torch.from_numpy(hc["labels"]).to(dev)
    td = torch.from_numpy(hc["dloss"]).to(dev)
    loss, lse, logits = coda.ce_fwd(th, tW, tl)
    dh, dWv = coda.ce_bwd(th, tW, tl, logits, lse, td)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        fc = oracle.ref_ce_fwd(hc["h"], hc["Wv"], hc["labels"])
        bc = oracle.ref_ce_bwd(hc["h"], hc["Wv"], hc["labels"], fc["lse"], hc["dloss"], oracle.bf16_rne(fc["logits"]))
    assert np.isnan(fc["lse"][4]) and np.isnan(fc["loss"][4])
    for k, g_, ref in (("loss", loss, fc["loss"]), ("lse", lse, fc["lse"])):
        same_nonfinite(f"ce {k}", g_.cpu().numpy(), ref)
    for k, g_, ref in (("logits", logits, fc["logits"]), ("dh", dh, bc["dh"]), ("dWv", dWv, bc["dWv"])):
        same_nonfinite(f"ce {k}", host(g_), ref)
    # rotary projection: NaN in X
    hr = synth.rope_inputs(264, 136, 392, seed=704)
    hr["X"][6, 6] = np.nan
    tr = {k: up(torch, dev, v) for k, v in hr.items()}
    Y = coda.rope_fwd(tr["X"], tr["W"], 256, 128, 100)
    dXr, dWr = coda.rope_bwd(tr["X"], tr["W"], tr["dY"], 256, 128, 100)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        fr = oracle.ref_rope_fwd(hr["X"], hr["W"], 256, 128, 100, 10000.0)
        br = oracle.ref_rope_bwd(hr["X"], hr["W"], hr["dY"], 256, 128, 100, 10000.0)
    for k, g_, ref in (("Y", Y, fr["Y"]), ("dX", dXr, br["dX"]), ("dW", dWr, br["dW"])):
        same_nonfinite(f"rope {k}", host(g_), ref)


# ------------------------------------------------------------ determinism

def _twice(torch, fn):
    outs = []
    for _ in range(2):
        res = fn()
        torch.cuda.synchronize()
        outs.append([x.clone() for x in res])
    for i, (a_, b_) in enumerate(zip(*outs)):
        assert torch.equal(a_, b_), f"output {i} differs between two runs"


def test_determinism_every_pattern(env):
    """Two runs of each fused pattern give bitwise equal outputs (every
    reduction has a fixed order; no atomics)."""
    torch, dev, coda = env
    hs = {k: up(torch, dev, v) for k, v in synth.swiglu_inputs(520, 392, 200, seed=710).items()}

    def swiglu():
        z, gu, a = coda.swiglu_fwd(hs["X"], hs["W"], hs["Wd"])
        return (z, gu, a, *coda.swiglu_bwd(hs["X"], hs["W"], hs["Wd"], gu, a, hs["dz"]))
    _twice(torch, swiglu)
    hm = {k: up(torch, dev, v) for k, v in synth.mlp_inputs(520, 264, 392, 200, seed=711).items()}

    def mlp():
        z, y, r, gu, a = coda.mlp_fwd(hm["X"], hm["W1"], hm["R"], hm["gamma"], hm["W"], hm["Wd"], 1e-6)
        return (z, y, r, gu, a, *coda.mlp_bwd(hm["X"], hm["W1"], hm["gamma"], hm["W"], hm["Wd"], y, r, gu, a,
                                               hm["dz"], hm["dy_in"]))
    _twice(torch, mlp)
    hc = synth.ce_inputs(520, 264, 1000, seed=712)
    th, tW = up(torch, dev, hc["h"]), up(torch, dev, hc["Wv"])
    tl, td = torch.from_numpy(hc["labels"]).to(dev), torch.from_numpy(hc["dloss"]).to(dev)

    def ce():
        loss, lse, logits = coda.ce_fwd(th, tW, tl)
        return (loss, lse, logits, *coda.ce_bwd(th, tW, tl, logits, lse, td))
    _twice(torch, ce)
    hr = {k: up(torch, dev, v) for k, v in synth.rope_inputs(520, 264, 776, seed=713).items()}

    def rope():
        Y = coda.rope_fwd(hr["X"], hr["W"], 512, 128, 200)
        return (Y, *coda.rope_bwd(hr["X"], hr["W"], hr["dY"], 512, 128, 200))
    _twice(torch, rope)
    hq = synth.mx8_inputs(264, 256, 384, 520, seed=714)
    tq = {k: up(torch, dev, v) for k, v in hq.items()}

    def mx8():
        xq, xs = coda.mx8_quantize(tq["X"])
        w1q, w1s = coda.mx8_quantize(tq["W1t"])
        w2q, w2s = coda.mx8_quantize(tq["W2t"])
        z, y, r = coda.fwd_mx8(xq, xs, w1q, w1s, tq["R"], tq["gamma"], w2q, w2s, 1e-6)
        return (xq, xs, z, y, r)
    _twice(torch, mx8)


# ------------------------------------------------------------ binding checks

def test_binding_refuses_mismatched_tensors(env):
    """Every tensor's dtype, shape and device is checked before a pointer is
    taken: nothing is launched, outputs keep their contents."""
    torch, dev, coda = env
    M, K, d, N = 264, 136, 272, 520
    h = synth.coda_inputs(M, K, d, N, seed=720, dtype="bf16", with_dz=False)
    t = {k: up(torch, dev, v) for k, v in h.items()}
    bf, f32 = torch.bfloat16, torch.float32

    def outs():
        return dict(y=torch.full((M, d), 5.0, dtype=bf, device=dev), r=torch.full((M,), 5.0, dtype=f32, device=dev),
                    z=torch.full((M, N), 5.0, dtype=bf, device=dev),
                    ws=torch.empty(coda.fwd_workspace_bytes(1, M, K, d, N), dtype=torch.uint8, device=dev))

    cases = [
        ("gamma float32", dict(gamma=t["gamma"].float()), {}, TypeError),
        ("W2 float32", dict(W2=t["W2"].float()), {}, TypeError),
        ("r bf16", {}, dict(r=torch.empty((M,), dtype=bf, device=dev)), TypeError),
        ("r short", {}, dict(r=torch.empty((M - 8,), dtype=f32, device=dev)), ValueError),
        ("z short", {}, dict(z=torch.empty((M - 8, N), dtype=bf, device=dev)), ValueError),
        ("y transposed shape", {}, dict(y=torch.empty((d, M), dtype=bf, device=dev)), ValueError),
        ("R wrong shape", dict(R=t["R"][:, :d - 8].contiguous()), {}, ValueError),
        ("workspace float", {}, dict(ws=torch.empty(64, dtype=f32, device=dev)), TypeError),
        ("z on the host", {}, dict(z=torch.empty((M, N), dtype=bf)), ValueError),
        ("R not contiguous", dict(R=torch.empty((d, M), dtype=bf, device=dev).t()), {}, ValueError),
    ]
    for label, ins, outs_over, exc in cases:
        o = outs()
        o.update(outs_over)
        a = {**t, **ins}
        with pytest.raises(exc):
            coda.coda_fwd(a["X"], a["W1"], a["R"], a["gamma"], a["W2"], 1e-6, o["y"], o["r"], o["z"], o["ws"])
        torch.cuda.synchronize()
        for k in ("y", "r", "z"):
            if o[k].is_cuda and o[k].dtype in (bf, f32) and o[k].numel():
                assert torch.all(o[k] == 5.0) or k in outs_over, f"{label}: {k} was written"
    # a backward output of another dtype, and the cross-entropy labels' dtype
    z, y, r = coda.fwd(t["X"], t["W1"], t["R"], t["gamma"], t["W2"], 1e-6)
    dz = up(torch, dev, synth.coda_inputs(M, K, d, N, seed=721)["dz"])
    dgamma_bf16 = torch.empty((d,), dtype=bf, device=dev)
    ws = torch.empty(coda.bwd_workspace_bytes(1, M, K, d, N), dtype=torch.uint8, device=dev)
    with pytest.raises(TypeError):
        coda.coda_bwd(t["X"], t["W1"], t["gamma"], t["W2"], y, r, dz, torch.empty_like(t["X"]),
                      torch.empty_like(t["W1"]), torch.empty_like(y), torch.empty_like(t["W2"]), dgamma_bf16, ws)
    hc = synth.ce_inputs(264, 136, 1000, seed=722)
    th, tW = up(torch, dev, hc["h"]), up(torch, dev, hc["Wv"])
    with pytest.raises(TypeError):
        coda.ce_fwd(th, tW, torch.from_numpy(hc["labels"]).long().to(dev))


# ------------------------------------------------------ ignored CE labels

def test_ce_ignored_labels(env):
    """Rows labelled outside [0, V) (-100, -1, V, a large index) have loss 0
    and a zero dlogits row; the rest match the oracle."""
    torch, dev, coda = env
    M, d, V = 520, 264, 776
    hc = synth.ce_inputs(M, d, V, seed=730)
    bad = np.array([0, 3, 257, 519])
    hc["labels"][bad] = [-100, -1, V, 1 << 30]
    th, tW = up(torch, dev, hc["h"]), up(torch, dev, hc["Wv"])
    tl, td = torch.from_numpy(hc["labels"]).to(dev), torch.from_numpy(hc["dloss"]).to(dev)
    loss, lse, logits = coda.ce_fwd(th, tW, tl)
    dh, dWv = coda.ce_bwd(th, tW, tl, logits, lse, td)
    torch.cuda.synchronize()
    f = oracle.ref_ce_fwd(hc["h"], hc["Wv"], hc["labels"])
    b = oracle.ref_ce_bwd(hc["h"], hc["Wv"], hc["labels"], f["lse"], hc["dloss"], oracle.bf16_rne(f["logits"]))
    lg = loss.cpu().numpy()
    assert np.all(lg[bad] == 0.0)
    assert np.all(host(dh)[bad] == 0.0)
    den = float(np.max(np.abs(f["loss"])))
    assert float(np.max(np.abs(lg - f["loss"]))) / den <= 1e-4
    assert float(np.max(np.abs(lse.cpu().numpy() - f["lse"]))) / float(np.max(np.abs(f["lse"]))) <= 1e-4
    for k, g_ in (("dh", dh), ("dWv", dWv)):
        ref = b[k]
        assert float(np.max(np.abs(host(g_) - ref))) / float(np.max(np.abs(ref))) <= BF16_TOL, k


def _nonfinite_split(clean, dirty, mask):
    """dirty is non-finite exactly where mask says, and bitwise the clean
    result elsewhere."""
    import torch
    bad = ~torch.isfinite(dirty.float())
    m = torch.as_tensor(mask, device=dirty.device)
    assert bool(bad[m].all()), "a dependent element stayed finite"
    assert not bool(bad[~m].any()), "a non-finite value reached an independent element"
    assert torch.equal(dirty[~m], clean[~m]), "an independent element changed"


def test_mx8_nonfinite_propagates(env):
    """The MXFP8 quantisers keep a NaN or an infinity (as the NaN code; a
    saturating clamp would turn it into a finite bound): it reaches every
    output element that depends on it, and every other element is bitwise
    the clean run's.  Block forward (NaN in X, Inf in R), block backward (NaN
    in dz), SwiGLU forward and backward (NaN in X, in dz)."""
    torch, dev, coda = env
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(torch.bfloat16)  # noqa: E731
    M, K, d, N = 256, 256, 256, 384
    h = synth.mx8_inputs(M, K, d, N, seed=717, with_dz=True)

    def fwd(X, R):
        xq, xs = coda.mx8_quantize(bf(X))
        w1q, w1s = coda.mx8_quantize(bf(h["W1t"]))
        w2q, w2s = coda.mx8_quantize(bf(h["W2t"]))
        z, y, r = coda.fwd_mx8(xq, xs, w1q, w1s, bf(R), bf(h["gamma"]), w2q, w2s, 1e-6)
        torch.cuda.synchronize()
        return z, y, r
    X, R = h["X"].copy(), h["R"].copy()
    X[3, 5] = np.nan
    R[9, 7] = np.inf
    zc, yc, rc = fwd(h["X"], h["R"])
    zd, yd, rd = fwd(X, R)
    rows = np.zeros((M, N), bool)
    rows[[3, 9]] = True
    _nonfinite_split(zc, zd, rows)

    def bwd(dz):
        y = yc
        out = coda.bwd_mx8(bf(h["X"]), bf(h["W1"]), bf(h["gamma"]), bf(h["W2"]), y, rc, bf(dz))
        torch.cuda.synchronize()
        return out
    dz = h["dz"].copy()
    dz[7, 2] = np.nan
    cl, di = bwd(h["dz"]), bwd(dz)
    r7 = np.zeros((M, K), bool)
    r7[7] = True
    _nonfinite_split(cl[0], di[0], r7)                                  # dX: row 7
    rd7 = np.zeros((M, d), bool)
    rd7[7] = True
    _nonfinite_split(cl[2], di[2], rd7)                                 # dR: row 7
    c2 = np.zeros((d, N), bool)
    c2[:, 2] = True
    _nonfinite_split(cl[3], di[3], c2)                                  # dW2: column 2
    _nonfinite_split(cl[1], di[1], np.ones((K, d), bool))              # dW1: every column sums over row 7
    _nonfinite_split(cl[4], di[4], np.ones((d,), bool))                # dgamma: sums over every row

    Ms, ds, F = 256, 256, 256
    hs = synth.swiglu_inputs(Ms, ds, F, seed=718)
    Xs = hs["X"].copy()
    Xs[4, 9] = np.nan
    zc, guc, ac = coda.swiglu_fwd_mx8(bf(hs["X"]), bf(hs["W"]), bf(hs["Wd"]))
    zd, gud, ad = coda.swiglu_fwd_mx8(bf(Xs), bf(hs["W"]), bf(hs["Wd"]))
    torch.cuda.synchronize()
    for c_, d_, w_ in ((zc, zd, ds), (guc, gud, 2 * F), (ac, ad, F)):
        m = np.zeros((Ms, w_), bool)
        m[4] = True
        _nonfinite_split(c_, d_, m)
    dzs = hs["dz"].copy()
    dzs[6, 3] = np.nan
    cl = coda.swiglu_bwd_mx8(bf(hs["X"]), bf(hs["W"]), bf(hs["Wd"]), guc, ac, bf(hs["dz"]))
    di = coda.swiglu_bwd_mx8(bf(hs["X"]), bf(hs["W"]), bf(hs["Wd"]), guc, ac, bf(dzs))
    torch.cuda.synchronize()
    m = np.zeros((Ms, ds), bool)
    m[6] = True
    _nonfinite_split(cl[0], di[0], m)                                   # dX: row 6
    _nonfinite_split(cl[1], di[1], np.ones((ds, 2 * F), bool))         # dW: every column sums over row 6
    m = np.zeros((F, ds), bool)
    m[:, 3] = True
    _nonfinite_split(cl[2], di[2], m)                                   # dWd: column 3

"""The workspace-free forward (coda_fwd_noalloc, built-in device scratch)
against coda_fwd with a caller workspace: the same kernels, so the outputs
must be bitwise equal, and both within the oracle's bar.  Two calls in a row,
the second smaller, so the second runs on scratch the first left behind."""
import numpy as np
import pytest

import oracle
from gemm_epilogue_fusion_gemm1_amd import synth

pytestmark = pytest.mark.gpu


def _rel(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref))) / float(np.max(np.abs(ref)))


def test_fwd_noalloc_matches_fwd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_epilogue_fusion_gemm1_amd as coda
    coda.load_library()
    dev = torch.device("cuda:0")
    eps = 1e-6
    for (M, K, d, N), seed in (((520, 264, 392, 776), 31), ((264, 136, 272, 520), 32)):
        print(f"[noalloc] M={M} K={K} d={d} N={N}", flush=True)
        h = synth.coda_inputs(M, K, d, N, seed=seed, dtype="bf16", with_dz=False)
        t = {k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in h.items()}
        z0, y0, r0 = coda.fwd(t["X"], t["W1"], t["R"], t["gamma"], t["W2"], eps)
        y = torch.full((M, d), 7.0, dtype=torch.bfloat16, device=dev)
        r = torch.full((M,), 7.0, dtype=torch.float32, device=dev)
        z = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=dev)
        coda.coda_fwd_noalloc(t["X"], t["W1"], t["R"], t["gamma"], t["W2"], eps, y, r, z)
        torch.cuda.synchronize()
        assert torch.equal(y, y0) and torch.equal(r, r0) and torch.equal(z, z0), "noalloc differs from coda_fwd"
        f = oracle.ref_fwd(h["X"], h["W1"], h["R"], h["gamma"], h["W2"], eps)
        assert _rel(z.float().cpu().numpy(), f["z"]) <= 2e-2
        assert _rel(y.float().cpu().numpy(), f["y"]) <= 2e-2
        assert float(np.max(np.abs(r.cpu().numpy() - f["r"]) / f["r"])) <= 1e-3


def test_fwd_noalloc_refuses_oversize():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemm_epilogue_fusion_gemm1_amd as coda
    dev = torch.device("cuda:0")
    M, K, d, N = 8192, 64, 8192, 64      # y * gamma alone needs 128 MiB
    bf = torch.bfloat16
    X = torch.zeros((M, K), dtype=bf, device=dev)
    W1 = torch.zeros((K, d), dtype=bf, device=dev)
    R = torch.zeros((M, d), dtype=bf, device=dev)
    g = torch.ones((d,), dtype=bf, device=dev)
    W2 = torch.zeros((d, N), dtype=bf, device=dev)
    y = torch.full((M, d), 3.0, dtype=bf, device=dev)
    r = torch.full((M,), 3.0, dtype=torch.float32, device=dev)
    z = torch.full((M, N), 3.0, dtype=bf, device=dev)
    with pytest.raises(coda.CodaError) as e:
        coda.coda_fwd_noalloc(X, W1, R, g, W2, 1e-6, y, r, z)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert torch.all(z == 3.0) and torch.all(r == 3.0)

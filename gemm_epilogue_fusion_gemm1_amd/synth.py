"""Seeded synthetic inputs and the workload table.

This module draws random numbers and quantises them to the storage dtype.
It holds none of the block's arithmetic.  Both the HIP path (through the
Python binding) and the CPU oracle are fed from here.  The two share nothing
else.

Recipe.  Each workload has one integer seed.  ``numpy.random.SeedSequence(seed)``
is spawned into six child streams, one per tensor, in the fixed order
X, R, W1, W2, gamma, dz (a SwiGLU workload uses X, W, Wd, dz).  Each stream
feeds a ``numpy.random.Generator(PCG64)`` that draws standard normals in fp32.
The draws are scaled, to std 1/sqrt(fan-in) for weights, and then rounded to
nearest-even bf16 when the workload stores bf16.  The arrays returned are fp32
and hold values exactly representable in the storage dtype, so an upload to
a bf16 device tensor is exact.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: its shapes, dtype, epsilon and seed."""

    name: str
    kind: str            # "coda" (GEMM-Residual-RMSNorm-GEMM), "swiglu", "mlp" (the two
                         # chained), "ce" (LM-head GEMM + cross-entropy), "rope"
                         # (QKV projection with rotary positions in its epilogue),
                         # "mx8" (the coda block on MXFP8 operands), "swiglu_mx8"
                         # (the SwiGLU block on MXFP8 operands) or "mlp_mx8" (the MLP
                         # sub-layer on MXFP8 operands)
    dtype: str           # "f32", "bf16" or "mxfp8" (bf16 draws, quantised by the caller)
    M: int
    K: int = 0           # coda, mlp: GEMM1 reduction width
    d: int = 0           # coda, mlp: normalised width; swiglu: model width
    N: int = 0           # coda: GEMM2 output width; ce: vocabulary size V
    F: int = 0           # swiglu, mlp: hidden width (gate and up halves)
    eps: float = 0.0
    rot: int = 0         # rope: rotated leading columns (q and k)
    head: int = 0        # rope: head width
    seq: int = 0         # rope: tokens per sequence (position = row mod seq)
    base: float = 0.0    # rope: frequency base
    seed: int = 0
    backward: bool = True
    note: str = ""

    def flops_fwd(self) -> float:
        """Algorithmic GEMM flops of the forward pass (elementwise work excluded)."""
        if self.kind in ("coda", "mx8"):
            return 2.0 * self.M * (self.K * self.d + self.d * self.N)
        if self.kind == "ce":
            return 2.0 * self.M * self.d * self.N
        if self.kind == "rope":
            return 2.0 * self.M * self.K * self.N
        swiglu = 2.0 * self.M * self.d * 2 * self.F + 2.0 * self.M * self.F * self.d
        if self.kind in ("mlp", "mlp_mx8"):
            return 2.0 * self.M * self.K * self.d + swiglu
        return swiglu

    def flops_bwd(self) -> float:
        """Algorithmic GEMM flops of the backward pass: two products per forward GEMM."""
        return 2.0 * self.flops_fwd()


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32_fwd", "coda", "f32", M=128, K=256, d=256, N=512,
                 eps=1e-6, seed=1000, backward=False,
                 note="tiny forward-only block in fp32"),
        Workload("llama1b_fwd", "coda", "bf16", M=8192, K=2048, d=2048, N=8192,
                 eps=1e-6, seed=1001, backward=False,
                 note="LLaMA-3-1B-shaped block forward, 4 x 2048 tokens"),
        Workload("llama7b_fwdbwd", "coda", "bf16", M=8192, K=4096, d=4096, N=11008,
                 eps=1e-6, seed=1002, backward=True,
                 note="LLaMA-7B-shaped block forward+backward"),
        Workload("llama70b_fwdbwd", "coda", "bf16", M=4096, K=8192, d=8192, N=28672,
                 eps=1e-5, seed=1003, backward=True,
                 note="LLaMA-70B-hidden-shaped block forward+backward"),
        Workload("swiglu_fwdbwd", "swiglu", "bf16", M=8192, d=4096, F=14336,
                 seed=1004, backward=True,
                 note="SwiGLU gate/up GEMM with fused epilogue, then down-projection"),
        Workload("llama7b_mlp_fwdbwd", "mlp", "bf16", M=8192, K=4096, d=4096, F=11008,
                 eps=1e-6, seed=1005, backward=True,
                 note="LLaMA-7B-shaped MLP sub-layer: projection + residual, RMS norm, "
                      "SwiGLU gate/up, down projection; forward+backward with dy_in"),
        Workload("llama7b_ce_fwdbwd", "ce", "bf16", M=8192, d=4096, N=32000,
                 seed=1006, backward=True,
                 note="LLaMA-7B-shaped LM head (vocabulary 32000) with cross-entropy, "
                      "forward+backward"),
        Workload("llama3_8b_ce_fwdbwd", "ce", "bf16", M=16384, d=4096, N=128256,
                 seed=1009, backward=True,
                 note="LLaMA-3-8B-shaped LM head (vocabulary 128256) over two 8192-token "
                      "sequences, with cross-entropy, forward+backward; logits and dlogits "
                      "are 4.2 GB each"),
        Workload("llama7b_qkv_rope_fwdbwd", "rope", "bf16", M=8192, K=4096, N=12288,
                 rot=8192, head=128, seq=4096, base=10000.0, seed=1007, backward=True,
                 note="LLaMA-7B-shaped QKV projection with rotary positions on q and k "
                      "(two 4096-token sequences), forward+backward"),
        Workload("llama7b_fwd_mx8", "mx8", "mxfp8", M=8192, K=4096, d=4096, N=11008,
                 eps=1e-6, seed=1008, backward=False,
                 note="LLaMA-7B-shaped block forward with MXFP8 operands (weights "
                      "stored [out, in])"),
        Workload("llama7b_fwdbwd_mx8", "mx8", "mxfp8", M=8192, K=4096, d=4096, N=11008,
                 eps=1e-6, seed=1010, backward=True,
                 note="LLaMA-7B-shaped block forward+backward with every GEMM on MXFP8 "
                      "operands (the backward quantises its bf16 inputs along each "
                      "GEMM's contraction index)"),
        Workload("swiglu_fwdbwd_mx8", "swiglu_mx8", "mxfp8", M=8192, d=4096, F=14336,
                 seed=1011, backward=True,
                 note="SwiGLU block forward+backward (the swiglu_fwdbwd shape) with every "
                      "GEMM on MXFP8 operands (bf16 draws, quantised by the calls)"),
        Workload("llama7b_mlp_fwdbwd_mx8", "mlp_mx8", "mxfp8", M=8192, K=4096, d=4096, F=11008,
                 eps=1e-6, seed=1012, backward=True,
                 note="LLaMA-7B-shaped MLP sub-layer forward+backward with dy_in (the "
                      "llama7b_mlp_fwdbwd shape) with every GEMM on MXFP8 operands"),
    ]
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Quantise fp32 values to the nearest bf16 (ties to even); returns fp32.

    Works on the fp32 bit pattern: add 0x7FFF plus the lowest kept bit, then
    clear the low 16 bits.  The inputs drawn here are finite normals, so the
    NaN case never arises.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _normal(stream: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(stream))
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _quantise(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def coda_inputs(M: int, K: int, d: int, N: int, seed: int, dtype: str = "bf16",
                with_dz: bool = True) -> dict:
    """X, R ~ N(0,1); W1 ~ N(0,1/K); W2 ~ N(0,1/d); gamma = 1 + 0.1 N(0,1); dz ~ N(0,1)."""
    s = np.random.SeedSequence(seed).spawn(6)
    out = {
        "X": _normal(s[0], (M, K), 1.0),
        "R": _normal(s[1], (M, d), 1.0),
        "W1": _normal(s[2], (K, d), 1.0 / math.sqrt(K)),
        "W2": _normal(s[3], (d, N), 1.0 / math.sqrt(d)),
        "gamma": np.float32(1.0) + np.float32(0.1) * _normal(s[4], (d,), 1.0),
    }
    if with_dz:
        out["dz"] = _normal(s[5], (M, N), 1.0)
    return {k: _quantise(v, dtype) for k, v in out.items()}


def swiglu_inputs(M: int, d: int, F: int, seed: int, dtype: str = "bf16",
                  with_dz: bool = True) -> dict:
    """X ~ N(0,1); W = [W_gate | W_up] ~ N(0,1/d); Wd ~ N(0,1/F); dz ~ N(0,1)."""
    s = np.random.SeedSequence(seed).spawn(4)
    out = {
        "X": _normal(s[0], (M, d), 1.0),
        "W": _normal(s[1], (d, 2 * F), 1.0 / math.sqrt(d)),
        "Wd": _normal(s[2], (F, d), 1.0 / math.sqrt(F)),
    }
    if with_dz:
        out["dz"] = _normal(s[3], (M, d), 1.0)
    return {k: _quantise(v, dtype) for k, v in out.items()}


def mlp_inputs(M: int, K: int, d: int, F: int, seed: int, dtype: str = "bf16",
               with_dz: bool = True) -> dict:
    """X, R ~ N(0,1); W1 ~ N(0,1/K); gamma = 1 + 0.1 N(0,1); W = [W_gate | W_up]
    ~ N(0,1/d); Wd ~ N(0,1/F); dz, dy_in ~ N(0,1)."""
    s = np.random.SeedSequence(seed).spawn(8)
    out = {
        "X": _normal(s[0], (M, K), 1.0),
        "R": _normal(s[1], (M, d), 1.0),
        "W1": _normal(s[2], (K, d), 1.0 / math.sqrt(K)),
        "gamma": np.float32(1.0) + np.float32(0.1) * _normal(s[3], (d,), 1.0),
        "W": _normal(s[4], (d, 2 * F), 1.0 / math.sqrt(d)),
        "Wd": _normal(s[5], (F, d), 1.0 / math.sqrt(F)),
    }
    if with_dz:
        out["dz"] = _normal(s[6], (M, d), 1.0)
        out["dy_in"] = _normal(s[7], (M, d), 1.0)
    return {k: _quantise(v, dtype) for k, v in out.items()}


def ce_inputs(M: int, d: int, V: int, seed: int, dtype: str = "bf16", with_dz: bool = True) -> dict:
    """h ~ N(0,1) (final hidden states); Wv ~ N(0,1/d); labels uniform in
    [0, V) (int32); dloss = U(0.5, 1.5) / M (a mean reduction's gradient,
    varied per row; float32)."""
    s = np.random.SeedSequence(seed).spawn(4)
    out = {"h": _quantise(_normal(s[0], (M, d), 1.0), dtype),
           "Wv": _quantise(_normal(s[1], (d, V), 1.0 / math.sqrt(d)), dtype),
           "labels": np.random.Generator(np.random.PCG64(s[2])).integers(0, V, M).astype(np.int32)}
    if with_dz:
        u = np.random.Generator(np.random.PCG64(s[3])).random(M, dtype=np.float32)
        out["dloss"] = ((np.float32(0.5) + u) / np.float32(M)).astype(np.float32)
    return out


def rope_inputs(M: int, K: int, N: int, seed: int, dtype: str = "bf16", with_dz: bool = True) -> dict:
    """X ~ N(0,1); W = [Wq | Wk | Wv] ~ N(0,1/K); dY ~ N(0,1)."""
    s = np.random.SeedSequence(seed).spawn(3)
    out = {"X": _normal(s[0], (M, K), 1.0), "W": _normal(s[1], (K, N), 1.0 / math.sqrt(K))}
    if with_dz:
        out["dY"] = _normal(s[2], (M, N), 1.0)
    return {k: _quantise(v, dtype) for k, v in out.items()}


def mx8_inputs(M: int, K: int, d: int, N: int, seed: int, with_dz: bool = False) -> dict:
    """The draws of ``coda_inputs`` (bf16) with the weights transposed to
    [out, in], the layout an MXFP8 weight is quantised from (blocks run along
    the contraction index), and (for a backward) the weights as drawn and dz.
    The quantisation itself is the caller's."""
    h = coda_inputs(M, K, d, N, seed, "bf16", with_dz=with_dz)
    out = {"X": h["X"], "R": h["R"], "gamma": h["gamma"],
           "W1t": np.ascontiguousarray(h["W1"].T), "W2t": np.ascontiguousarray(h["W2"].T)}
    if with_dz:
        out.update(W1=h["W1"], W2=h["W2"], dz=h["dz"])
    return out


def workload_inputs(w: Workload, with_dz: bool | None = None) -> dict:
    """Inputs of a named workload (dz only when it has a backward pass)."""
    if with_dz is None:
        with_dz = w.backward
    if w.kind == "coda":
        return coda_inputs(w.M, w.K, w.d, w.N, w.seed, w.dtype, with_dz)
    if w.kind == "mlp":
        return mlp_inputs(w.M, w.K, w.d, w.F, w.seed, w.dtype, with_dz)
    if w.kind == "ce":
        return ce_inputs(w.M, w.d, w.N, w.seed, w.dtype, with_dz)
    if w.kind == "rope":
        return rope_inputs(w.M, w.K, w.N, w.seed, w.dtype, with_dz)
    if w.kind == "mx8":
        return mx8_inputs(w.M, w.K, w.d, w.N, w.seed, with_dz)
    if w.kind == "swiglu_mx8":     # bf16 draws; the MXFP8 calls quantise them
        return swiglu_inputs(w.M, w.d, w.F, w.seed, "bf16", with_dz)
    if w.kind == "mlp_mx8":
        return mlp_inputs(w.M, w.K, w.d, w.F, w.seed, "bf16", with_dz)
    return swiglu_inputs(w.M, w.d, w.F, w.seed, w.dtype, with_dz)

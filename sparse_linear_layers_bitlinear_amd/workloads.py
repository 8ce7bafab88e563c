"""Seeded synthetic inputs for the Sparse-BitLinear forward path.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic (no quantizer, mask, GEMM or dequant). Both the CPU oracle
(through the tests) and the HIP path consume the buffers it returns, so the
two sides always see identical inputs.

Shapes follow the layers the pages evaluate: Qwen2.5 0.5B / 1.5B / 3B FFN
projections (Sparse-BitNet summary, section 5 "Experimental Analysis" and
Table 3) and the BitNet b1.58 2B4T transformer (BitNet b1.58 2B4T technical
report summary, section 3.2 "Big-Picture Architecture"). The pages publish no
data for this path, so every tensor is drawn here:

* master weights: fp32, 0.02 * N(0, 1), generated first, row-major, one
  tensor after another in the listed order;
* activations: N(0, 1) in fp32, generated after all weights, then rounded to
  bf16 (round-to-nearest-even); a config may then overwrite a seeded set of
  channels (outliers x10, or Student-t df=4 "heavy-tailed" channels).

All randomness comes from ``numpy.random.default_rng(seed)`` (PCG64).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Linear", "Workload", "WORKLOADS", "bf16_round", "bf16_bits",
    "make_workload", "make_linear_inputs",
]


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as bf16-exact fp32.

    Used only to produce the bf16 activations the configs call for.
    Inputs are finite by construction.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Bit pattern (uint16) of a bf16-exact fp32 array."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class Linear:
    """One projection: y[T, O] = Sparse-BitLinear(x[T, K]; W[O, K])."""
    name: str
    O: int
    K: int
    x_name: str  # which activation tensor feeds it


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    T: int
    N: int
    M: int
    linears: tuple
    x_specs: tuple          # (name, K) in generation order
    outliers: int = 0       # number of x10 outlier channels per x tensor
    heavy_tail_frac: float = 0.0  # fraction of channels drawn from Student-t df=4
    seed: int = 0
    nm_sweep: tuple = field(default_factory=tuple)


def _ffn(hidden: int, inter: int, gate: bool = True):
    ls = []
    if gate:
        ls.append(Linear("gate", inter, hidden, "x_gu"))
    ls.append(Linear("up", inter, hidden, "x_gu"))
    ls.append(Linear("down", hidden, inter, "x_down"))
    return tuple(ls), (("x_gu", hidden), ("x_down", inter))


_q05_l, _q05_x = _ffn(896, 4864)
_q15_l, _q15_x = _ffn(1536, 8960, gate=False)
_q3_l, _q3_x = _ffn(2048, 11008)

WORKLOADS = {
    "tiny": Workload(
        "tiny", "single Sparse-BitLinear, 16 tokens, K=256, O=128, 6:8",
        T=16, N=6, M=8, linears=(Linear("proj", 128, 256, "x"),),
        x_specs=(("x", 256),), outliers=2),
    "qwen05b_ffn": Workload(
        "qwen05b_ffn", "Qwen2.5-0.5B-shaped FFN gate+up+down, T=2048 (4x512), 6:8",
        T=2048, N=6, M=8, linears=_q05_l, x_specs=_q05_x),
    "qwen15b_ffn": Workload(
        "qwen15b_ffn", "Qwen2.5-1.5B-shaped FFN up+down, T=4096, 2:4",
        T=4096, N=2, M=4, linears=_q15_l, x_specs=_q15_x),
    "qwen3b_sweep": Workload(
        "qwen3b_sweep", "Qwen2.5-3B-shaped FFN, T=8192, N:8 sweep 7..2",
        T=8192, N=6, M=8, linears=_q3_l, x_specs=_q3_x, heavy_tail_frac=0.02,
        nm_sweep=((7, 8), (6, 8), (5, 8), (4, 8), (3, 8), (2, 8))),
    "bitnet_decode": Workload(
        "bitnet_decode", "BitNet-2B4T-shaped decode layer, T in {1,4,8}, prepacked 2:4",
        T=8, N=2, M=4,
        linears=(Linear("q", 2560, 2560, "x_attn"), Linear("k", 640, 2560, "x_attn"),
                 Linear("v", 640, 2560, "x_attn"), Linear("o", 2560, 2560, "x_o"),
                 Linear("gate", 6912, 2560, "x_ffn"), Linear("up", 6912, 2560, "x_ffn"),
                 Linear("down", 2560, 6912, "x_down")),
        x_specs=(("x_attn", 2560), ("x_o", 2560), ("x_ffn", 2560), ("x_down", 6912))),
}


def make_workload(name: str, T: int | None = None, seed: int | None = None,
                  scale_T: int | None = None):
    """Draw every tensor of a workload.

    Returns (W, X): dicts name -> fp32 array. W[name] is the fp32 master weight
    [O, K]; X[x_name] is the bf16-exact fp32 activation [T, K].
    ``T`` overrides the token count (e.g. a bounded sample for CPU timing).
    """
    wl = WORKLOADS[name]
    T = wl.T if T is None else int(T)
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    W = {}
    for lin in wl.linears:
        W[lin.name] = (rng.standard_normal((lin.O, lin.K), dtype=np.float32)
                       * np.float32(0.02))
    X = {}
    for xn, K in wl.x_specs:
        X[xn] = rng.standard_normal((T, K), dtype=np.float32)
    for xn, K in wl.x_specs:
        x = X[xn]
        if wl.outliers:
            ch = rng.choice(K, wl.outliers, replace=False)
            x[:, ch] *= np.float32(10.0)
        if wl.heavy_tail_frac:
            nch = int(math.ceil(wl.heavy_tail_frac * K))
            ch = rng.choice(K, nch, replace=False)
            x[:, ch] = rng.standard_t(4, size=(T, nch)).astype(np.float32)
        X[xn] = bf16_round(x)
    return W, X


def make_linear_inputs(T: int, O: int, K: int, seed: int = 0,
                       w_scale: float = 0.02, outliers: int = 0):
    """One (W fp32 [O,K], x bf16-exact fp32 [T,K]) pair of arbitrary shape,
    drawn in the same order and distributions as the workloads."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((O, K), dtype=np.float32) * np.float32(w_scale)
    x = rng.standard_normal((T, K), dtype=np.float32)
    if outliers:
        ch = rng.choice(K, outliers, replace=False)
        x[:, ch] *= np.float32(10.0)
    return W, bf16_round(x)

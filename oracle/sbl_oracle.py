"""CPU oracle for the Sparse-BitLinear forward path and its Dual-STE backward
-- TEST INFRASTRUCTURE ONLY.

This is the plain, slow, step-by-step definition of what the HIP library must
compute. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it. The library never calls it and shares no
code with it (no headers, tables, helpers or constants).

Sources ("the pages"):
  [SB]  Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to
        Semi-Structured Sparsity -- paper-graph-ui summary, section 3.4
        "Detailed, Sentence-Based Technical Breakdown".
  [SB2] the paperlayer.ai summary of the same paper (section 2 "Sparse-BitNet").
  [B2T] BitNet b1.58 2B4T Technical Report -- paper-graph-ui summary,
        section 3.4 (activation quantization; GPU inference kernel).

Precision. The pages fix no arithmetic precision. Where a floating-point
value decides an integer (the int8 activation code, the ternary code) the
decision is taken in IEEE fp32 -- the precision the kernels compute in -- so
both sides take it identically. The absmean sum is exact (correctly rounded
to fp64). The dequantized output is computed in fp64 from the exact int32
accumulator; the bf16 output is the bf16 rounding of the same product
taken in the reading's fixed fp32 order (``dequant_f32``).

Pins (what checks this file against something other than itself) live in
tests/test_oracle_pins.py: brute-force integer GEMM, exhaustive mask
permutations and tie patterns, the pages' master-vs-ternary ranking example,
exact-rational absmean, the Gaussian zero-fraction and N:M density closed
forms, activation-quantizer invariants and error bounds, the N = M textbook
reduction, packed-format round trips and a hand-written packed fixture.
Every function below is pinned; none is "parity unpinned". The one
unpinnable choice is a convention, not a function: the weight dequant factor
is sw = gamma + eps (the value used to divide), see ``dequant``.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "quant_act", "absmean", "nm_mask", "ternary_codes", "apply_mask",
    "quant_mask_weight", "gemm_int", "gemm_int_bruteforce", "dequant", "dequant_f32",
    "to_bf16", "linear_fwd", "packed_row_bytes", "packed_bytes", "pack",
    "unpack", "INDEX_FORM", "mask_words", "mask_flips", "group_threshold",
    "rms_scale", "sum_squares", "rmsnorm_quant_act", "dropped_max",
    "act_dequant_bf16", "linear_bwd_dx", "linear_bwd_dw",
]

F32 = np.float32


# ---------------------------------------------------------------------------
# a1. Activation quantizer Q_a, per token, absmax -> int8
# ---------------------------------------------------------------------------
def quant_act(x: np.ndarray, eps_a: float = 1e-5):
    """Per-token absmax int8 quantization.

    [SB] "Activation quantization" paragraph: x~ = Clip(x * 127/(max|x| + eps),
    -128, 127). [B2T] "Activation Quantization: Per-Token Absmax to 8-Bit
    Integers": one scale per token (row), values rounded to the nearest
    integer. Readings: the scale is s = 127 / (m + eps) evaluated in fp32
    first, then x * s in fp32, rounded half-to-even, then clipped to
    [-128, 127]. The dequant factor is sx = (m + eps) / 127 in fp32.

    x: [T, K] float32 (bf16 inputs are passed as their exact fp32 values).
    Returns xq int8 [T, K], sx float32 [T].
    """
    x = np.asarray(x, dtype=F32)
    eps = F32(eps_a)
    m = np.max(np.abs(x), axis=1)                       # exact in fp32
    d = (m + eps).astype(F32)                           # fp32 add
    s = (F32(127.0) / d).astype(F32)                    # fp32 IEEE division
    v = (x * s[:, None]).astype(F32)                    # fp32 multiply
    q = np.clip(np.rint(v), -128, 127).astype(np.int8)  # round half to even, clip
    sx = (d / F32(127.0)).astype(F32)
    return q, sx


# ---------------------------------------------------------------------------
# a2. gamma = absmean of the whole master weight
# ---------------------------------------------------------------------------
def absmean(w: np.ndarray, eps_w: float = 1e-5):
    """gamma = ||W||_1 / (d_out * d_in); sw = gamma + eps.

    [SB] "Step 1: Compute the Rescaling Factor" (mean absolute value over the
    whole matrix) and "Step 2: Rescale and RoundClip" (the divisor is
    gamma + eps). [B2T] "Weight Quantization: Absolute Mean" gives the same
    mean. Reading: the sum is exact -- math.fsum returns the correctly
    rounded fp64 of the exact sum -- then one fp64 division by n, then
    rounding to fp32; sw = fp32(gamma + eps).
    Returns (gamma, sw) as np.float32.
    """
    a = np.abs(np.asarray(w, dtype=F32)).astype(np.float64).ravel()
    n = a.size
    S = math.fsum(a)
    gamma = F32(S / n)
    sw = F32(gamma + F32(eps_w))
    return gamma, sw


# ---------------------------------------------------------------------------
# a3. N:M keep-mask from master-weight magnitudes
# ---------------------------------------------------------------------------
def nm_mask(w: np.ndarray, N: int, M: int) -> np.ndarray:
    """Pi_{N:M}(|W|): per row, per contiguous group of M along the input
    dimension, keep the N entries of largest magnitude.

    [SB] "N:M Mask Generation" / "The Masking Operation". Tie rule (the page
    allows any; reading): among equal magnitudes the lower index is kept
    first, so exactly N are kept in every group. +0 and -0 tie.
    Implemented as a stable sort of -|w| inside each group.
    w: [O, K] with K % M == 0. Returns uint8 [O, K] of 0/1.
    """
    w = np.asarray(w, dtype=F32)
    O, K = w.shape
    assert K % M == 0 and 1 <= N <= M
    a = np.abs(w).reshape(O, K // M, M)
    order = np.argsort(-a, axis=2, kind="stable")       # descending, stable
    mask = np.zeros_like(a, dtype=np.uint8)
    np.put_along_axis(mask, order[:, :, :N], 1, axis=2)
    return mask.reshape(O, K)


# ---------------------------------------------------------------------------
# a4. RoundClip to ternary, then apply the mask (quant-then-mask)
# ---------------------------------------------------------------------------
def ternary_codes(w: np.ndarray, sw) -> np.ndarray:
    """W_q = RoundClip(W / (gamma + eps), -1, +1).

    [SB] "Step 2: Rescale and RoundClip" (Eq. 1). Readings: IEEE fp32
    division, round half to even, clip to [-1, 1]. Returns int8 [O, K].
    """
    w = np.asarray(w, dtype=F32)
    r = (w / F32(sw)).astype(F32)
    return np.clip(np.rint(r), -1, 1).astype(np.int8)


def apply_mask(codes: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """W_eff = W_q (elementwise) M. [SB] "Composition Order: Quant-Then-Mask"."""
    return (codes.astype(np.int8) * mask.astype(np.int8)).astype(np.int8)


def quant_mask_weight(w: np.ndarray, N: int, M: int, eps_w: float = 1e-5,
                      variant: str = "method"):
    """The whole weight side of the forward, in the order [SB] gives in
    "The Full Sparse-BitLinear Layer": mask from master |W|, gamma from the
    full unmasked W, RoundClip, then the mask applied to the ternary codes.

    variant="ternary" is the ablation of [SB] "Where the mask is computed" /
    Figure 3a: the mask is ranked on the ternary magnitudes |W_q| instead
    (ties, which are the rule here, go to the lower index).

    variant="mask_then_quant" is the ablation of [SB] "Composition Order":
    W_eff = Q_t(W (.) M) -- the same master-ranked mask, but gamma is the mean
    |w| over the kept (Top-N) weights only, n = O * K/M * N, then RoundClip
    of the masked weight (pruned entries are 0 and stay 0).
    Returns (w_eff int8, mask uint8, gamma f32, sw f32)."""
    if variant == "mask_then_quant":
        mask = nm_mask(w, N, M)
        w = np.asarray(w, dtype=F32)
        gamma, sw = absmean(w[mask == 1], eps_w)
        w_masked = np.where(mask == 1, w, F32(0.0)).astype(F32)
        return ternary_codes(w_masked, sw), mask, gamma, sw
    gamma, sw = absmean(w, eps_w)
    codes = ternary_codes(w, sw)
    if variant == "method":
        mask = nm_mask(w, N, M)
    elif variant == "ternary":
        mask = nm_mask(np.abs(codes).astype(F32), N, M)
    else:
        raise ValueError(variant)
    return apply_mask(codes, mask), mask, gamma, sw


# ---------------------------------------------------------------------------
# a5. int8 x ternary GEMM with an exact integer accumulator
# ---------------------------------------------------------------------------
def gemm_int(xq: np.ndarray, w_eff: np.ndarray) -> np.ndarray:
    """acc[t, o] = sum_k xq[t, k] * W_eff[o, k], exact, as int32.

    [SB] "The Full Sparse-BitLinear Layer", output step: y = s * (W_eff x~).
    Computed with an fp64 matrix product, which is exact here: every partial
    sum is an integer of magnitude <= 128 * K < 2**53.
    """
    xq = np.asarray(xq)
    w_eff = np.asarray(w_eff)
    assert xq.shape[1] == w_eff.shape[1] and xq.shape[1] * 128 < 2 ** 53
    acc = xq.astype(np.float64) @ w_eff.astype(np.float64).T
    acc = acc.astype(np.int64)
    assert np.all(np.abs(acc) < 2 ** 31)
    return acc.astype(np.int32)


def gemm_int_bruteforce(xq: np.ndarray, w_eff: np.ndarray) -> np.ndarray:
    """The same contraction as a plain integer triple loop (tiny inputs only)."""
    T, K = xq.shape
    O = w_eff.shape[0]
    out = np.zeros((T, O), dtype=np.int64)
    for t in range(T):
        for o in range(O):
            s = 0
            for k in range(K):
                s += int(xq[t, k]) * int(w_eff[o, k])
            out[t, o] = s
    return out.astype(np.int32)


# ---------------------------------------------------------------------------
# a6. dequant
# ---------------------------------------------------------------------------
def dequant(acc: np.ndarray, sx: np.ndarray, sw) -> np.ndarray:
    """y[t, o] = acc[t, o] * sx[t] * sw[o], in fp64.

    [SB] "The Full Sparse-BitLinear Layer": one scalar multiply per output
    absorbs both scales (Eq. 4). Reading (convention, not fixed by the
    pages): the weight factor is sw = gamma + eps, the value the weights
    were divided by (Algorithm 2 "multiplied back by scale"); the activation
    factor is sx = (m + eps)/127. ``sw`` may be a scalar or a per-row [O]
    array (gate and up concatenated).
    """
    sw = np.broadcast_to(np.asarray(sw, dtype=np.float64), (acc.shape[1],))
    return (acc.astype(np.float64) * np.asarray(sx, dtype=np.float64)[:, None]
            * sw[None, :])


def dequant_f32(acc: np.ndarray, sx: np.ndarray, sw) -> np.ndarray:
    """y[t, o] = fp32(fp32(fp32(acc) * sx[t]) * sw[o]): the same product as
    ``dequant`` taken in IEEE fp32, left to right, each step rounded to
    nearest (the reading of the dequant arithmetic: one fixed fp32 order, no
    fused multiply-add). fp32(acc) is exact (|acc| < 2^24). Returns float32;
    ``to_bf16`` of it is the bf16 output."""
    sw = np.broadcast_to(np.asarray(sw, dtype=F32), (acc.shape[1],))
    a = np.asarray(acc).astype(F32)
    return ((a * np.asarray(sx, dtype=F32)[:, None]).astype(F32) * sw[None, :]).astype(F32)


def to_bf16(y: np.ndarray) -> np.ndarray:
    """fp64 -> bf16, correctly rounded (ties to even), as bf16-exact fp32.

    fp64 -> fp32 with round-to-odd, then fp32 -> bf16 RNE: since fp32 keeps
    more than two extra bits over bf16, this equals direct RNE from fp64.
    """
    y = np.asarray(y, dtype=np.float64)
    r = y.astype(F32)
    over = np.abs(r.astype(np.float64)) > np.abs(y)
    r = np.where(over, np.nextafter(r, F32(0)), r).astype(F32)   # truncate
    inexact = r.astype(np.float64) != y
    u = r.view(np.uint32) | inexact.astype(np.uint32)            # odd if inexact
    u = u.astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(F32)


def linear_fwd(x: np.ndarray, w: np.ndarray, N: int, M: int,
               eps_a: float = 1e-5, eps_w: float = 1e-5):
    """The four steps end to end ([SB] "The Full Sparse-BitLinear Layer";
    Algorithm 1 forward). Returns a dict with every intermediate."""
    xq, sx = quant_act(x, eps_a)
    w_eff, mask, gamma, sw = quant_mask_weight(w, N, M, eps_w)
    acc = gemm_int(xq, w_eff)
    y = dequant(acc, sx, sw)
    return dict(xq=xq, sx=sx, w_eff=w_eff, mask=mask, gamma=gamma, sw=sw,
                acc=acc, y=y)


# ---------------------------------------------------------------------------
# a7. Backward under the Dual straight-through estimator
# ---------------------------------------------------------------------------
# [SB] "Gradient Estimation: The Dual Straight-Through Estimator" and the
# backward steps of the Algorithm 1 walk-through: the forward is the product
# y = x~ W~^T of x~ = sx * xq and W~ = sw * W_eff. The STE of Q_a hands the
# gradient at x~ to x unchanged; the Dual STE hands the gradient at W~ (=
# W_eff up to the scale) to every master weight unchanged -- pruned ones too,
# no mask gating, and (Algorithm 2's backward returns its input gradient) no
# clip window. The pages fix no precision; readings: dY is bf16 (the pages'
# training dtype) and x~ enters the weight gradient as bf16 of fp32(sx * q).
def act_dequant_bf16(xq: np.ndarray, sx: np.ndarray) -> np.ndarray:
    """x~ as the weight gradient consumes it: fp32(xq * sx[t]), then rounded
    to bf16 (nearest, ties to even). Returns bf16-exact float32 [T, K]."""
    v = (np.asarray(xq).astype(F32) * np.asarray(sx, dtype=F32)[:, None]).astype(F32)
    return to_bf16(v.astype(np.float64))


def linear_bwd_dx(dy: np.ndarray, w_eff: np.ndarray, sw) -> np.ndarray:
    """dX[t, k] = sum_o dY[t, o] * sw[o] * W_eff[o, k], in fp64: the gradient
    at x~ of sum(dY * y). sw: scalar or per-row [O] (tensors concatenated)."""
    w_eff = np.asarray(w_eff)
    sw = np.broadcast_to(np.asarray(sw, dtype=np.float64), (w_eff.shape[0],))
    return np.asarray(dy, dtype=np.float64) @ (w_eff.astype(np.float64) * sw[:, None])


def linear_bwd_dw(dy: np.ndarray, xt: np.ndarray, mask=None) -> np.ndarray:
    """dW[o, k] = sum_t dY[t, o] * x~[t, k], in fp64, at every (o, k): the
    gradient at W~, passed to the master weights whether kept or pruned.

    mask: the estimator [SB] "Gradient Estimation" ablates against (the
    mask-gated gradients of prior N:M training; "mask without grad" in
    Figure 3): dW = M (.) dY^T x~, zero at every pruned weight."""
    dw = np.asarray(dy, dtype=np.float64).T @ np.asarray(xt, dtype=np.float64)
    return dw if mask is None else dw * (np.asarray(mask) != 0)


# ---------------------------------------------------------------------------
# Packed ternary-plus-index weight format
# ---------------------------------------------------------------------------
# The pages fix only that four ternary values fit in one int8 ([B2T] "Inference
# Implementation: GPU") and that the structured-sparse kernels share one weight
# layout ([SB2] appendix A.2). The format below is this project's definition,
# restated here from its specification (the library implements it separately):
#
# 2-bit code: 0 -> 0b00, +1 -> 0b01, -1 -> 0b11 (two's complement).
# Byte-sliced word: 16 two-bit fields; field u sits at bit 8*(u%4) + 2*(u//4).
# Rows are records of fixed pitch, concatenable along O.
#
# INDEX FORM (N = 2 with M = 4 or M = 8): pitch = ceil(K/128) * 32 bytes,
#   plus ceil(K/128) * 16 for M = 8. Chunk c covers k in [32c, 32c+32) = 8
#   groups q of 4; it is two little-endian uint32: word 0 (codes): compressed
#   value v = 2q + j (j = 0, 1) holds the code of the j-th selected slot of
#   group q (ascending), as field v of a byte-sliced word; word 1 (indices):
#   bits [4q+1:4q] = first selected slot, [4q+3:4q+2] = second. For 2:4 the
#   selected slots are the kept ones. For 2:8 a group of 4 holds 0, 1 or 2 kept
#   slots: they are selected, then the lowest unselected slots until there are
#   two (their code is 0), and the mask follows the chunks as in the dense form
#   (bit j of word c = mask[32c + j]), since the selection alone does not tell
#   which slots were kept. Groups past K: slots (0, 1), codes 0.
# DENSE FORM (every other N:M): pitch = ceil(K/64)*16 + ceil(K/128)*16 bytes.
#   First ceil(K/64)*4 uint32 code words: word c holds W_eff codes of
#   k = 16c + u as field u (byte-sliced); then ceil(K/128)*4 uint32 mask
#   words: bit j of word c = mask[32c + j]. Everything past K is zero.
def INDEX_FORM(N: int, M: int) -> bool:
    return N == 2 and M in (4, 8)


def _ceil(a, b):
    return -(-a // b)


def packed_row_bytes(K: int, N: int, M: int) -> int:
    if INDEX_FORM(N, M):
        return _ceil(K, 128) * 32 + (_ceil(K, 128) * 16 if M == 8 else 0)
    return _ceil(K, 64) * 16 + _ceil(K, 128) * 16


def packed_bytes(O: int, K: int, N: int, M: int) -> int:
    return O * packed_row_bytes(K, N, M)


def _field_shift(u):
    u = np.asarray(u, dtype=np.uint32)
    return (8 * (u % 4) + 2 * (u // 4)).astype(np.uint32)


def pack(w_eff: np.ndarray, mask: np.ndarray, N: int, M: int) -> np.ndarray:
    """(W_eff, mask) -> packed bytes (uint8 [O, pitch])."""
    w_eff = np.asarray(w_eff, dtype=np.int8)
    mask = np.asarray(mask, dtype=np.uint8)
    O, K = w_eff.shape
    code2 = (w_eff.astype(np.int32) & 3).astype(np.uint32)
    if INDEX_FORM(N, M):
        Kc = _ceil(K, 128) * 128
        c2 = np.zeros((O, Kc), np.uint32)
        c2[:, :K] = code2
        mk = np.zeros((O, Kc), np.uint8)
        mk[:, :K] = mask
        pad = np.zeros((O, Kc - K), np.uint8)
        pad.reshape(O, -1, 4)[:, :, :2] = 1                 # padding groups keep (0, 1)
        mk[:, K:] = pad
        g_c = c2.reshape(O, Kc // 4, 4)
        g_m = mk.reshape(O, Kc // 4, 4).copy()
        for _ in range(2):                                  # 2:8: select the lowest free slots
            short = g_m.sum(axis=2) < 2
            free = np.argmax(g_m == 0, axis=2)
            rows, grp = np.nonzero(short)
            g_m[rows, grp, free[rows, grp]] = 1
        assert np.all(g_m.sum(axis=2) == 2)
        i0 = np.argmax(g_m, axis=2)                         # first kept slot
        i1 = 3 - np.argmax(g_m[:, :, ::-1], axis=2)         # last kept slot
        c0 = np.take_along_axis(g_c, i0[:, :, None], 2)[:, :, 0]
        c1 = np.take_along_axis(g_c, i1[:, :, None], 2)[:, :, 0]
        q = np.arange(8, dtype=np.uint32)
        i0 = i0.reshape(O, Kc // 32, 8).astype(np.uint32)
        i1 = i1.reshape(O, Kc // 32, 8).astype(np.uint32)
        c0 = c0.reshape(O, Kc // 32, 8)
        c1 = c1.reshape(O, Kc // 32, 8)
        idx = np.bitwise_or.reduce((i0 | (i1 << 2)) << (4 * q), axis=2)
        cw = np.bitwise_or.reduce((c0 << _field_shift(2 * q))
                                  | (c1 << _field_shift(2 * q + 1)), axis=2)
        rec = np.stack([cw, idx], axis=2).reshape(O, -1).astype("<u4")
        if M == 8:                                          # the 2:8 mask follows the chunks
            mk8 = np.zeros((O, Kc), np.uint32)
            mk8[:, :K] = mask
            mw = np.bitwise_or.reduce(mk8.reshape(O, Kc // 32, 32)
                                      << np.arange(32, dtype=np.uint32), axis=2)
            rec = np.concatenate([rec, mw.astype("<u4")], axis=1)
        return rec.view(np.uint8).reshape(O, -1)
    Kc = _ceil(K, 64) * 64
    Km = _ceil(K, 128) * 128
    c2 = np.zeros((O, Kc), np.uint32)
    c2[:, :K] = code2
    cw = np.bitwise_or.reduce(c2.reshape(O, Kc // 16, 16)
                              << _field_shift(np.arange(16)), axis=2)
    mk = np.zeros((O, Km), np.uint32)
    mk[:, :K] = mask
    mw = np.bitwise_or.reduce(mk.reshape(O, Km // 32, 32)
                              << np.arange(32, dtype=np.uint32), axis=2)
    rec = np.concatenate([cw, mw], axis=1).astype("<u4")
    return rec.view(np.uint8).reshape(O, -1)


def _sext2(c):
    c = np.asarray(c, dtype=np.int32) & 3
    return np.where(c >= 2, c - 4, c).astype(np.int8)


def unpack(packed: np.ndarray, O: int, K: int, N: int, M: int):
    """packed bytes -> (W_eff int8 [O, K], mask uint8 [O, K])."""
    pitch = packed_row_bytes(K, N, M)
    words = np.ascontiguousarray(np.asarray(packed, np.uint8).reshape(O, pitch))
    words = words.view("<u4").astype(np.uint32)
    if INDEX_FORM(N, M):
        nch = _ceil(K, 128) * 4
        cw = words[:, 0:2 * nch:2]
        idx = words[:, 1:2 * nch:2]
        q = np.arange(8, dtype=np.uint32)
        i0 = (idx[:, :, None] >> (4 * q)) & 3
        i1 = (idx[:, :, None] >> (4 * q + 2)) & 3
        c0 = _sext2(cw[:, :, None] >> _field_shift(2 * q))
        c1 = _sext2(cw[:, :, None] >> _field_shift(2 * q + 1))
        G = nch * 8
        i0 = i0.reshape(O, G)
        i1 = i1.reshape(O, G)
        c0 = c0.reshape(O, G)
        c1 = c1.reshape(O, G)
        w = np.zeros((O, G, 4), np.int8)
        mk = np.zeros((O, G, 4), np.uint8)
        np.put_along_axis(w, i0[:, :, None].astype(np.int64), c0[:, :, None], 2)
        np.put_along_axis(w, i1[:, :, None].astype(np.int64), c1[:, :, None], 2)
        np.put_along_axis(mk, i0[:, :, None].astype(np.int64), 1, 2)
        np.put_along_axis(mk, i1[:, :, None].astype(np.int64), 1, 2)
        if M == 8:                                          # the mask is stored, not implied
            mw = words[:, 2 * nch:]
            mk = ((mw[:, :, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(np.uint8)
        return w.reshape(O, -1)[:, :K].copy(), mk.reshape(O, -1)[:, :K].copy()
    ncw = _ceil(K, 64) * 4
    cw = words[:, :ncw]
    mw = words[:, ncw:]
    w = _sext2(cw[:, :, None] >> _field_shift(np.arange(16))).reshape(O, -1)
    mk = ((mw[:, :, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(np.uint8)
    return w[:, :K].copy(), mk.reshape(O, -1)[:, :K].copy()


# ---------------------------------------------------------------------------
# Mask diagnostics: flip count (for the flip rate r_t) and per-group threshold
# ---------------------------------------------------------------------------
def mask_words(mask: np.ndarray) -> np.ndarray:
    """The library's bit layout of a keep-mask: uint32 [O, C] with
    C = ceil(K/128)*4 words per row; bit e of word c is the mask of column
    k = 32c + e (0 for k >= K). (A storage layout of the library, not a
    definition of the pages.)"""
    mask = np.asarray(mask, dtype=np.uint8)
    O, K = mask.shape
    C = _ceil(K, 128) * 4
    full = np.zeros((O, 32 * C), np.uint64)
    full[:, :K] = mask
    bits = full.reshape(O, C, 32) << np.arange(32, dtype=np.uint64)
    return bits.sum(axis=2).astype(np.uint32)


def mask_flips(mask_prev: np.ndarray, mask_cur: np.ndarray) -> int:
    """Number of mask positions that changed between two steps.

    [SB] section 3.4 (Dual STE discussion) and the analysis of Figure 3b: the
    mask flip rate r_t (Eq. 6) measures how many mask positions change
    between consecutive steps. Reading: r_t = mask_flips / (O*K) (the
    equation itself is not printed on the pages)."""
    a = np.asarray(mask_prev, dtype=np.uint8)
    b = np.asarray(mask_cur, dtype=np.uint8)
    assert a.shape == b.shape
    return int(np.count_nonzero(a != b))


def dropped_max(w: np.ndarray, mask: np.ndarray, M: int) -> np.ndarray:
    """Largest |w| among the dropped slots of each group of M under a given
    mask (0 when nothing is dropped); equals group_threshold for the mask
    ranked on |w|. float32 [O, K/M]."""
    w = np.asarray(w, dtype=F32)
    O, K = w.shape
    a = np.where(np.asarray(mask).reshape(O, K // M, M) == 0, np.abs(w).reshape(O, K // M, M),
                 F32(0))
    return a.max(axis=2).astype(F32)


def group_threshold(w: np.ndarray, N: int, M: int) -> np.ndarray:
    """Per-block pruning threshold of the magnitude-stratification analysis.

    [SB] Figure 6 discussion: for each block (group of M along the input
    dimension) the threshold t is the magnitude of the (N+1)-th largest
    weight. With N == M nothing is pruned; reading: t = 0 then.
    Returns float32 [O, K/M] (the master magnitude itself, not normalized)."""
    w = np.asarray(w, dtype=F32)
    O, K = w.shape
    assert K % M == 0 and 1 <= N <= M
    a = np.abs(w).reshape(O, K // M, M)
    if N == M:
        return np.zeros((O, K // M), F32)
    desc = -np.sort(-a, axis=2)                         # magnitudes, largest first
    return desc[:, :, N].astype(F32)


# ---------------------------------------------------------------------------
# Q_a(Norm(x)): RMS normalization before the activation quantizer
# ---------------------------------------------------------------------------
def rms_scale(x: np.ndarray, eps_n: float) -> np.ndarray:
    """Per-row r = fp32(1 / sqrt(S / K + eps_n)), S = sum_k fp32(x_k * x_k).

    [SB] Algorithm 1 walk-through: x~ = Q_a(Norm(x)), Norm likely RMSNorm;
    [B2T] section 3.2: subln normalization without bias terms. The pages fix
    no arithmetic; reading: the squares are fp32 products; S is their exact
    sum rounded once to fp64 (math.fsum, so no summation order is implied);
    then fp64 division by K, addition of eps_n, square root and reciprocal,
    rounded once to fp32. x: [T, K] float32 with finite squares. Returns
    float32 [T]."""
    x = np.asarray(x, dtype=F32)
    K = x.shape[1]
    S = sum_squares(x)
    r = 1.0 / np.sqrt(S / float(K) + float(np.float32(eps_n)))
    return r.astype(F32)


def sum_squares(x: np.ndarray) -> np.ndarray:
    """Per row, S = sum_k fp32(x_k * x_k), the exact sum rounded once to
    fp64 (math.fsum). Returns float64 [T]."""
    x = np.asarray(x, dtype=F32)
    sq = (x * x).astype(F32).astype(np.float64)         # fp32 products, exact in fp64
    return np.array([math.fsum(sq[t]) for t in range(x.shape[0])], dtype=np.float64)


def rmsnorm_quant_act(x: np.ndarray, gain, eps_n: float, eps_a: float):
    """z = fp32(fp32(x * r) * gain) per element (gain None: fp32(x * r)),
    then quant_act(z). Returns (xq int8 [T, K], sx float32 [T])."""
    x = np.asarray(x, dtype=F32)
    r = rms_scale(x, eps_n)
    z = (x * r[:, None]).astype(F32)
    if gain is not None:
        z = (z * np.asarray(gain, dtype=F32)[None, :]).astype(F32)
    return quant_act(z, eps_a)

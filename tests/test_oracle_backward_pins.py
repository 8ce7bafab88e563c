"""Pins of the oracle's Dual-STE backward (act_dequant_bf16, linear_bwd_dx,
linear_bwd_dw) against what the pages and mathematics fix: exact finite
differences of the forward's bilinear loss (pruned positions included),
torch autograd of the straight-through formulation, the Euler identity of a
bilinear form tied to the forward oracle, and bf16 rounding cases."""
from fractions import Fraction

import numpy as np
import torch

import oracle as o
from sparse_linear_layers_bitlinear_amd.workloads import bf16_round, make_linear_inputs

F32 = np.float32


def _loss(dy, xt, wt):
    """sum_{t,o} dY[t,o] * y[t,o], y[t,o] = sum_k x~[t,k] W~[o,k], as exact
    rationals by plain loops (no matrix product)."""
    T, K = len(xt), len(xt[0])
    O = len(wt)
    total = Fraction(0)
    for t in range(T):
        for oo in range(O):
            y = sum((xt[t][k] * wt[oo][k] for k in range(K)), Fraction(0))
            total += dy[t][oo] * y
    return total


def _fr(a):
    return [[Fraction(float(v)) for v in row] for row in np.asarray(a, dtype=np.float64)]


def test_bwd_exact_finite_differences_including_pruned():
    """The loss is linear in each operand, so a unit step gives the exact
    partial derivative. dW must equal it at every (o, k), pruned positions
    included (the Dual STE hands the gradient to weights the mask removed)."""
    rng = np.random.default_rng(11)
    T, O, K, N, M = 3, 4, 8, 6, 8
    W, _ = make_linear_inputs(T, O, K, seed=5)
    w_eff, mask, gamma, sw = o.quant_mask_weight(W, N, M)
    assert (mask == 0).sum() == O * 2
    xq = rng.integers(-128, 128, size=(T, K)).astype(np.int8)
    sx = np.array([0.5, 0.25, 2.0], F32)
    xt = o.act_dequant_bf16(xq, sx)                      # exact: sx is a power of two
    dy = rng.integers(-3, 4, size=(T, O)).astype(np.float64)
    wt = w_eff.astype(np.float64) * float(sw)
    dX = o.linear_bwd_dx(dy, w_eff, sw)
    dW = o.linear_bwd_dw(dy, xt)
    DY, XT, WT = _fr(dy), _fr(xt), _fr(wt)
    L0 = _loss(DY, XT, WT)
    for t in range(T):
        for k in range(K):
            XT[t][k] += 1
            assert _loss(DY, XT, WT) - L0 == Fraction(float(dX[t, k]))
            XT[t][k] -= 1
    for oo in range(O):
        for k in range(K):
            WT[oo][k] += 1
            assert _loss(DY, XT, WT) - L0 == Fraction(float(dW[oo, k]))
            WT[oo][k] -= 1
    assert np.any(dW[mask == 0] != 0)                  # pruned weights get gradient


def test_bwd_matches_autograd_of_straight_through_form():
    """Algorithm 2's straight-through form: the forward uses W~ and x~, the
    backward hands the gradient to the master W and to x unchanged."""
    rng = np.random.default_rng(12)
    for N, M in [(6, 8), (2, 4)]:
        T, O, K = 5, 16, 32
        W, x = make_linear_inputs(T, O, K, seed=21 + N)
        xq, sx = o.quant_act(x)
        w_eff, mask, gamma, sw = o.quant_mask_weight(W, N, M)
        xt = o.act_dequant_bf16(xq, sx)
        dy = bf16_round(rng.standard_normal((T, O)).astype(F32)).astype(np.float64)
        Wm = torch.tensor(W, dtype=torch.float64, requires_grad=True)
        xm = torch.tensor(x, dtype=torch.float64, requires_grad=True)
        w_used = Wm + (torch.tensor(w_eff * float(sw), dtype=torch.float64) - Wm).detach()
        x_used = xm + (torch.tensor(xt, dtype=torch.float64) - xm).detach()
        (x_used @ w_used.T * torch.tensor(dy)).sum().backward()
        dX = o.linear_bwd_dx(dy, w_eff, sw)
        # autograd's dX uses W~ as fp64; the oracle the same product
        assert np.allclose(xm.grad.numpy(), dX, rtol=1e-12, atol=1e-12)
        assert np.allclose(Wm.grad.numpy(), o.linear_bwd_dw(dy, xt), rtol=1e-12, atol=1e-12)


def test_bwd_euler_identity_with_forward():
    """For y = x~ W~^T: <dX, x~> = <dY, y> = <dW, W~>, with y from the forward
    oracle's exact integer GEMM and dequant (x~ = sx * xq unrounded here)."""
    rng = np.random.default_rng(13)
    for N, M in [(6, 8), (2, 4), (3, 8)]:
        T, O, K = 7, 24, 64
        W, x = make_linear_inputs(T, O, K, seed=40 + N)
        r = o.linear_fwd(x, W, N, M)
        xt = r["xq"].astype(np.float64) * r["sx"].astype(np.float64)[:, None]
        dy = rng.standard_normal((T, O))
        dX = o.linear_bwd_dx(dy, r["w_eff"], r["sw"])
        dW = o.linear_bwd_dw(dy, xt)
        wt = r["w_eff"].astype(np.float64) * float(r["sw"])
        a, b, c = (dX * xt).sum(), (dy * r["y"]).sum(), (dW * wt).sum()
        assert abs(a - b) <= 1e-10 * abs(b) and abs(c - b) <= 1e-10 * abs(b)


def test_bwd_mask_enters_dx_only():
    """dW does not depend on the mask (dense gradient flow); dX does: with
    N = M it is the product with the unmasked ternary codes, and a sparser
    mask changes it."""
    rng = np.random.default_rng(14)
    T, O, K = 6, 16, 64
    W, x = make_linear_inputs(T, O, K, seed=77)
    xq, sx = o.quant_act(x)
    xt = o.act_dequant_bf16(xq, sx)
    dy = rng.standard_normal((T, O))
    dw = o.linear_bwd_dw(dy, xt)
    assert np.array_equal(dw, dy.T @ xt.astype(np.float64))
    full = o.quant_mask_weight(W, 8, 8)
    codes = o.ternary_codes(W, full[3])
    assert np.array_equal(o.linear_bwd_dx(dy, full[0], full[3]),
                          dy @ (codes.astype(np.float64) * float(full[3])))
    sparse = o.quant_mask_weight(W, 2, 8)
    assert not np.allclose(o.linear_bwd_dx(dy, sparse[0], sparse[3]),
                           o.linear_bwd_dx(dy, full[0], full[3]))
    # per-row sw of two concatenated tensors = the sum of the two products
    W2, _ = make_linear_inputs(T, 8, K, seed=78)
    a = o.quant_mask_weight(W, 6, 8)
    b = o.quant_mask_weight(W2, 6, 8)
    dy2 = rng.standard_normal((T, O + 8))
    cat = o.linear_bwd_dx(dy2, np.concatenate([a[0], b[0]]),
                          np.concatenate([np.full(O, a[3]), np.full(8, b[3])]))
    assert np.allclose(cat, o.linear_bwd_dx(dy2[:, :O], a[0], a[3])
                       + o.linear_bwd_dx(dy2[:, O:], b[0], b[3]), rtol=1e-13, atol=1e-13)


def test_act_dequant_bf16_rounding():
    """Exact when sx is a power of two (|q| <= 128 fits bf16's 8 bits); ties
    go to even; otherwise within half a bf16 step."""
    xq = np.array([[1, -1, 127, -128, 3, 0, 65, -77]], np.int8)
    assert np.array_equal(o.act_dequant_bf16(xq, np.array([0.125], F32)),
                          xq.astype(F32) * F32(0.125))
    # q * sx exactly halfway between two bf16 values
    one_tie = F32(1 + 2 ** -8)                  # between 1 and 1 + 2^-7: even is 1
    odd_tie = F32(1 + 3 * 2 ** -8)              # between 1 + 2^-7 and 1 + 2^-6: even is the upper
    r = o.act_dequant_bf16(np.array([[1], [1]], np.int8), np.array([one_tie, odd_tie], F32))
    assert r[0, 0] == F32(1.0) and r[1, 0] == F32(1 + 2 ** -6)
    rng = np.random.default_rng(15)
    xq = rng.integers(-128, 128, size=(9, 40)).astype(np.int8)
    sx = rng.uniform(1e-3, 1e-1, 9).astype(F32)
    v = xq.astype(F32) * sx[:, None]
    r = o.act_dequant_bf16(xq, sx).astype(np.float64)
    err = np.abs(r - v.astype(np.float64))
    ulp = 2.0 ** (np.floor(np.log2(np.abs(v.astype(np.float64)) + (v == 0))) - 7)
    assert np.all(err <= ulp / 2)                               # half a bf16 step
    assert np.any(err > ulp / 4)                                # and not exact
    assert np.array_equal(r.astype(F32), bf16_round(v))   # bf16-representable


def test_bwd_mask_gated_estimator():
    """The gated ablation: exact finite differences of the loss in W~ where
    the mask keeps the weight, zero where it prunes; with N = M it is the
    dense gradient."""
    rng = np.random.default_rng(16)
    T, O, K, N, M = 3, 4, 8, 6, 8
    W, _ = make_linear_inputs(T, O, K, seed=9)
    w_eff, mask, gamma, sw = o.quant_mask_weight(W, N, M)
    xq = rng.integers(-128, 128, size=(T, K)).astype(np.int8)
    xt = o.act_dequant_bf16(xq, np.array([0.5, 0.25, 2.0], F32))
    dy = rng.integers(-3, 4, size=(T, O)).astype(np.float64)
    gated = o.linear_bwd_dw(dy, xt, mask=mask)
    DY, XT, WT = _fr(dy), _fr(xt), _fr(w_eff.astype(np.float64) * float(sw))
    L0 = _loss(DY, XT, WT)
    for oo in range(O):
        for k in range(K):
            if mask[oo, k]:
                WT[oo][k] += 1
                assert _loss(DY, XT, WT) - L0 == Fraction(float(gated[oo, k]))
                WT[oo][k] -= 1
            else:
                assert gated[oo, k] == 0
    full = o.nm_mask(W, 8, 8)
    assert np.array_equal(o.linear_bwd_dw(dy, xt, mask=full), o.linear_bwd_dw(dy, xt))


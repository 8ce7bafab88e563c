"""The bound behind the fused RMSNorm kernel's fast exact sum of squares.

The kernel sums fp32(x * x) over a row exactly (the reading: S = the exact
sum rounded once to fp64, as math.fsum gives). Its fast case rests on a
fact of arithmetic, checked here on the host, independently of the kernel:
a square of a bf16 value has at most 16 significant bits (of an fp32 value,
after fp32 rounding, 24), so squares whose exponents lie within W binades
of each other are integer multiples of the window's lowest unit; with
W = 54 - SB - ceil(log2 K), K of them sum below 2^53 units, so fp64
accumulation of one window is exact in any order, and the sum of two such
windows needs one rounding only (one IEEE addition). Rows whose nonzero
squares are normal and span fewer than 2W binades take that path.
"""
import math

import numpy as np
import pytest

from sparse_linear_layers_bitlinear_amd.workloads import bf16_round

F32 = np.float32


def _window(K, sb):
    return 54 - sb - math.ceil(math.log2(K))


def _squares(x):
    return (x.astype(F32) * x.astype(F32)).astype(F32)


def _exp(sq):
    return (sq.view(np.uint32) >> 23).astype(np.int64)


def _seq_sum(vals):
    s = 0.0
    for v in vals:
        s += float(v)
    return s


def _row(rng, K, emax_x, span_x, bf16):
    """Row of random signs and mantissas whose |x| exponents cover
    [emax_x - span_x, emax_x], with both ends present."""
    e = rng.integers(emax_x - span_x, emax_x + 1, K)
    e[0], e[1] = emax_x, emax_x - span_x
    # (mantissas below 1.99: bf16 rounding never carries into the next binade)
    x = (rng.uniform(1.0, 1.99, K) * np.exp2(e.astype(np.float64))).astype(F32)
    x *= np.where(rng.random(K) < 0.5, -1, 1).astype(F32)
    x[1] = F32(np.exp2(float(emax_x - span_x)))
    return bf16_round(x) if bf16 else x


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("K", [1024, 11008])
def test_two_window_fp64_sum_is_exact(bf16, K):
    sb = 16 if bf16 else 24
    W = _window(K, sb)
    rng = np.random.default_rng(K + sb)
    checked = 0
    for trial in range(40):
        # |x| exponents over about W binades, so the squares span up to 2W - 1
        x = _row(rng, K, int(rng.integers(-8, 8)), W - 1, bf16)
        sq = _squares(x)
        nz = sq[sq != 0]
        ex = _exp(nz)
        emax, emin = int(ex.max()), int(ex.min())
        if not (emin >= 1 and emax - emin < 2 * W):
            continue
        split = emax - W + 1
        hi, lo = nz[ex >= split], nz[ex < split]
        exact_hi = math.fsum(map(float, hi))
        exact_lo = math.fsum(map(float, lo))
        for _ in range(3):                       # any order: every partial sum exact
            assert _seq_sum(rng.permutation(hi)) == exact_hi
            assert _seq_sum(rng.permutation(lo)) == exact_lo
        # the one rounding: the sum of the two windows is the correctly rounded total
        assert exact_hi + exact_lo == math.fsum(map(float, nz))
        checked += 1
    assert checked >= 30


def test_one_fp64_accumulator_is_not_exact_there():
    """The split is needed: one square of 2^12 and many of about 2^-35 with 16
    significant bits (down to 2^-50), 47 binades apart (within 2W = 48 at
    K = 11008): in a single fp64 sum near 2^12 (unit 2^-40) the small
    squares lose their low bits."""
    K, W = 11008, _window(11008, 16)
    x = np.full(K, F32(1.5078125 * 2.0 ** -18), dtype=F32)    # bf16: 1 + 65/128
    x[0] = F32(2.0 ** 6)
    x = bf16_round(x)
    sq = _squares(x)
    ex = _exp(sq[sq != 0])
    assert ex.max() - ex.min() == 47 < 2 * W
    assert _seq_sum(sq) != math.fsum(map(float, sq))
    split = int(ex.max()) - W + 1
    hi, lo = sq[_exp(sq) >= split], sq[_exp(sq) < split]
    assert _seq_sum(hi) + _seq_sum(lo) == math.fsum(map(float, sq))

"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: brute force,
exact rational arithmetic, closed forms, invariants, the pages' worked
example, and hand-encoded fixtures. A plausible mistake in the oracle (a
dropped eps, a wrong sign, an off-by-one in the mask rank, a transposed GEMM
operand, a mask-then-quant order, a ternary-ranked mask) fails at least one.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import ndtr
from scipy.stats import binom

import oracle as o
from sparse_linear_layers_bitlinear_amd.workloads import (
    WORKLOADS, bf16_round, make_linear_inputs, make_workload)

F32 = np.float32


# --------------------------------------------------------------- GEMM (a5) --
def test_gemm_bruteforce_tiny():
    rng = np.random.default_rng(3)
    for T, O, K in [(1, 1, 4), (3, 5, 40), (7, 2, 96)]:
        xq = rng.integers(-128, 128, size=(T, K)).astype(np.int8)
        w = rng.integers(-1, 2, size=(O, K)).astype(np.int8)
        assert np.array_equal(o.gemm_int(xq, w), o.gemm_int_bruteforce(xq, w))
        # a transposed operand would not even produce [T, O] for T != O
        assert o.gemm_int(xq, w).shape == (T, O)


def test_gemm_extremes_exact():
    K = 11008
    xq = np.full((2, K), -128, np.int8)
    xq[1] = 127
    w = np.ones((3, K), np.int8)
    w[1] = -1
    w[2, ::2] = 0
    acc = o.gemm_int(xq, w)
    ref = xq.astype(np.int64) @ w.astype(np.int64).T     # numpy integer matmul
    assert np.array_equal(acc.astype(np.int64), ref)
    assert acc[0, 0] == -128 * K and acc[1, 1] == -127 * K


def test_gemm_config1_bruteforce():
    """Config 1 (16 x 256 -> 128, 6:8) through the whole oracle; its int32
    accumulator against a plain integer triple loop."""
    W, X = make_workload("tiny")
    r = o.linear_fwd(X["x"], W["proj"], 6, 8)
    assert np.array_equal(r["acc"], o.gemm_int_bruteforce(r["xq"], r["w_eff"]))


def test_N_equals_M_is_plain_int8_gemm():
    """N = M: the mask keeps everything and a5 is an int8 x int8 GEMM."""
    W, x = make_linear_inputs(9, 24, 64, seed=5)
    for M in (4, 8):
        r = o.linear_fwd(x, W, M, M)
        assert r["mask"].all()
        codes = o.ternary_codes(W, r["sw"])
        ref = r["xq"].astype(np.int64) @ codes.astype(np.int64).T
        assert np.array_equal(r["acc"].astype(np.int64), ref)


# ---------------------------------------------------------------- mask (a3) --
@pytest.mark.parametrize("M", [4, 8])
def test_mask_all_permutations(M):
    """Distinct magnitudes: the kept set is exactly the N largest."""
    perms = np.array(list(itertools.permutations(range(1, M + 1))), np.float32)
    rng = np.random.default_rng(0)
    signs = rng.choice([-1.0, 1.0], size=perms.shape).astype(np.float32)
    W = perms * signs * F32(0.01)
    for N in range(1, M + 1):
        mask = o.nm_mask(W, N, M)
        assert np.array_equal(mask, (perms > M - N).astype(np.uint8))


def _rank_rule_keep(vals, N):
    """Rank rule written out: slot i is kept iff fewer than N slots beat it;
    j beats i if |w_j| > |w_i|, or |w_j| == |w_i| and j < i."""
    keep = []
    for i, a in enumerate(vals):
        beats = sum(1 for j, b in enumerate(vals) if b > a or (b == a and j < i))
        keep.append(1 if beats < N else 0)
    return keep


def test_mask_all_tie_patterns():
    """Every magnitude pattern in {0,1,2}^8, every N, against the rank rule;
    zeros carry a random sign so -0 and +0 must tie."""
    pats = np.array(list(itertools.product([0, 1, 2], repeat=8)), np.float32)
    rng = np.random.default_rng(1)
    signs = rng.choice([-1.0, 1.0], size=pats.shape).astype(np.float32)
    W = pats * signs          # includes -0.0
    for N in range(1, 9):
        mask = o.nm_mask(W, N, 8)
        exp = np.array([_rank_rule_keep(list(p), N) for p in pats], np.uint8)
        assert np.array_equal(mask, exp), N
    # M = 4 groups of the same patterns
    W4 = W.reshape(-1, 4)
    P4 = pats.reshape(-1, 4)
    for N in range(1, 5):
        exp = np.array([_rank_rule_keep(list(p), N) for p in P4], np.uint8)
        assert np.array_equal(o.nm_mask(W4, N, 4), exp)


def test_mask_invariants():
    rng = np.random.default_rng(2)
    W = rng.standard_normal((64, 256)).astype(np.float32) * F32(0.02)
    Wi = rng.integers(-50, 51, size=(64, 256)).astype(np.float32)  # many ties
    for N, M in [(1, 4), (2, 4), (3, 4), (2, 8), (5, 8), (6, 8), (7, 8)]:
        for A in (W, Wi):
            m = o.nm_mask(A, N, M)
            assert np.all(m.reshape(64, -1, M).sum(axis=2) == N)   # exactly N
            assert np.array_equal(m, o.nm_mask(-A, N, M))           # sign-blind
            assert np.array_equal(m, o.nm_mask(A * F32(4), N, M))   # scale-blind
        # strictly increasing map of |w| (exact on these integers)
        f = np.sign(Wi) * (Wi * Wi + 3 * np.abs(Wi))
        assert np.array_equal(o.nm_mask(Wi, N, M), o.nm_mask(f, N, M))
        # the mask does not depend on gamma / eps
        wq1 = o.quant_mask_weight(W, N, M, 1e-5)[1]
        wq2 = o.quant_mask_weight(W, N, M, 1e-1)[1]
        assert np.array_equal(wq1, wq2)


def test_master_vs_ternary_worked_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "master_vs_ternary_ranking.json")))
    w = np.array([ex["w_master"]], np.float32)
    N, M = ex["N"], ex["M"]
    w_eff, mask, gamma, sw = o.quant_mask_weight(w, N, M, 1e-5)
    assert gamma == F32(0.7)
    codes = o.ternary_codes(w, sw)
    assert codes[0].tolist() == ex["expected_codes"]
    assert mask[0].tolist() == ex["expected_mask_from_master"]
    # ranking the ternary values instead: ties broken by index pick slot 3
    m_t = o.nm_mask(codes.astype(np.float32), N, M)
    assert m_t[0].tolist() == ex["expected_mask_from_ternary_lower_index_ties"]
    assert not np.array_equal(m_t, mask)
    # quant-then-mask: W_eff keeps the zero code at the kept slot 5
    assert w_eff[0].tolist() == [1, -1, 1, 0, 1, 0, -1, 0]
    # the ablated recipe of the weight side gives exactly that ternary-ranked mask
    w2, m2, g2, sw2 = o.quant_mask_weight(w, N, M, 1e-5, variant="ternary")
    assert m2[0].tolist() == ex["expected_mask_from_ternary_lower_index_ties"]
    assert g2 == gamma and sw2 == sw
    assert w2[0].tolist() == (codes * m2)[0].tolist()
    # largest dropped magnitude: 0.2 (slot 7) under the master mask, 0.3 under the ternary one
    assert o.dropped_max(w, mask, M)[0].tolist() == [np.float32(0.2)]
    assert o.dropped_max(w, m2, M)[0].tolist() == [np.float32(0.3)]
    assert np.array_equal(o.dropped_max(w, mask, M), o.group_threshold(w, N, M))


def test_mask_then_quant_worked_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "composition_order.json")))
    w = np.array([ex["w_master"]], np.float32)
    N, M = ex["N"], ex["M"]
    q_eff, q_mask, q_gamma, _ = o.quant_mask_weight(w, N, M, 1e-5)
    m_eff, m_mask, m_gamma, m_sw = o.quant_mask_weight(w, N, M, 1e-5, variant="mask_then_quant")
    assert q_mask[0].tolist() == ex["expected_mask"] and np.array_equal(m_mask, q_mask)
    assert q_gamma == F32(0.4609375) and m_gamma == F32(0.875)
    assert m_sw == F32(F32(0.875) + F32(1e-5))
    assert q_eff[0].tolist() == ex["expected_w_eff_quant_then_mask"]
    assert m_eff[0].tolist() == ex["expected_w_eff_mask_then_quant"]


def test_mask_then_quant_properties():
    """gamma over the Top-N of each group is at least the full mean (each
    group's Top-N mean is at least its mean); the exact rational mean of the
    kept |w|; RoundClip is monotone in 1/sw, so the nonzero codes are a subset
    of quant-then-mask's; N = M keeps all and reduces to the method."""
    rng = np.random.default_rng(31)
    for N, M, K in [(2, 4, 64), (6, 8, 96), (5, 8, 40), (1, 4, 32)]:
        w = (rng.standard_normal((9, K)) * 0.02).astype(np.float32)
        q_eff, q_mask, q_gamma, _ = o.quant_mask_weight(w, N, M)
        m_eff, m_mask, m_gamma, m_sw = o.quant_mask_weight(w, N, M, variant="mask_then_quant")
        assert np.array_equal(m_mask, q_mask)
        assert m_gamma >= q_gamma
        g, sw = _gamma_exact(w[q_mask == 1], 1e-5)
        assert m_gamma == g and m_sw == sw
        assert np.all(m_eff[q_mask == 0] == 0)
        assert np.all((m_eff != 0) <= (q_eff != 0))
        assert np.all(m_eff[m_eff != 0] == q_eff[m_eff != 0])
        assert (m_eff != 0).sum() < (q_eff != 0).sum()       # strictly sparser here
    w = (rng.standard_normal((5, 64)) * 0.02).astype(np.float32)
    for a, b in zip(o.quant_mask_weight(w, 8, 8), o.quant_mask_weight(w, 8, 8, variant="mask_then_quant")):
        assert np.array_equal(a, b)


# ------------------------------------------------------------ absmean (a2) --
def _gamma_exact(w, eps):
    S = sum((Fraction(float(v)) for v in np.abs(w.astype(np.float64)).ravel()),
            Fraction(0))
    S64 = float(S)                       # correctly rounded (CPython)
    g = F32(S64 / w.size)
    return g, F32(g + F32(eps))


def test_absmean_matches_exact_rational():
    rng = np.random.default_rng(4)
    cases = [
        rng.standard_normal((7, 33)).astype(np.float32) * F32(0.02),
        # very wide exponent range, denormals included
        (rng.standard_normal(500) * np.exp2(rng.integers(-149, 100, 500))
         ).astype(np.float32),
        np.array([1e-45, 3e38, 1.0, 2e-38, 7e-46], np.float32),
        bf16_round(rng.standard_normal(301).astype(np.float32)),
    ]
    for w in cases:
        assert o.absmean(w, 1e-5) == _gamma_exact(w, 1e-5)


def test_absmean_closed_forms_and_order_independence():
    c = F32(0.0123)
    w = np.full((37, 64), c, np.float32)
    w[::3] *= -1
    g, sw = o.absmean(w, 1e-5)
    assert g == c and sw == F32(c + F32(1e-5))
    # dyadic values: the mean is exact
    w = np.array([0.5, -0.25, 0.125, 1.0], np.float32)
    assert o.absmean(w, 0.0)[0] == F32(1.875 / 4)
    # all-zero weights: gamma = 0, sw = eps
    assert o.absmean(np.zeros((4, 8), np.float32), 1e-5) == (F32(0), F32(1e-5))
    # permutation invariance, bit for bit
    rng = np.random.default_rng(5)
    w = (rng.standard_normal(20000) * np.exp2(rng.integers(-40, 10, 20000))
         ).astype(np.float32)
    g0 = o.absmean(w)
    for _ in range(3):
        assert o.absmean(rng.permutation(w)) == g0


# ------------------------------------------------------- ternary codes (a4) --
def test_codes_against_exact_rationals():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal(4000) * 0.05).astype(np.float32)
    for sw in [F32(0.0159), F32(0.02), F32(1.0), F32(3e-7)]:
        ws = (w * (sw / F32(0.02))).astype(np.float32)
        codes = o.ternary_codes(ws, sw)
        for v, c in zip(ws, codes):
            r = Fraction(float(abs(v))) / Fraction(float(sw))
            if abs(r - Fraction(1, 2)) < Fraction(1, 2 ** 20):
                continue                                   # boundary band
            exp = (1 if r > Fraction(1, 2) else 0) * (1 if v > 0 else -1)
            assert c == exp


def test_codes_round_half_even_and_clip():
    sw = F32(0.25)
    w = np.array([0.125, -0.125, 0.375, -0.375, 0.625, 5.0, -5.0, 0.0, -0.0],
                 np.float32)
    # 0.5 -> 0 (ties to even), 1.5 -> 2 -> clip 1, 2.5 -> 2 -> clip 1
    assert o.ternary_codes(w, sw).tolist() == [0, 0, 1, -1, 1, 1, -1, 0, 0]


def test_gaussian_zero_fraction_closed_form():
    """For W ~ N(0, s^2): P(code = 0) = P(|w| < sw/2) = 2 Phi(sw / (2 s)) - 1
    (about 0.310 at sw ~ s sqrt(2/pi))."""
    rng = np.random.default_rng(7)
    s = 0.02
    W = rng.standard_normal((2048, 2048)).astype(np.float32) * F32(s)
    g, sw = o.absmean(W)
    p0 = 2 * ndtr(float(sw) / (2 * s)) - 1
    frac = float((o.ternary_codes(W, sw) == 0).mean())
    sd = math.sqrt(p0 * (1 - p0) / W.size)
    assert abs(frac - p0) < 5 * sd
    assert abs(p0 - 0.31006) < 2e-3


@pytest.mark.parametrize("N,M", [(7, 8), (6, 8), (5, 8), (4, 8), (3, 8),
                                 (2, 8), (2, 4), (1, 4)])
def test_nm_density_closed_form(N, M):
    """Quant-then-mask with a master-ranked mask: a group keeps min(#{|w| >=
    threshold}, N) nonzeros, #{..} ~ Binomial(M, p). Density = E[min(B, N)]/M.
    A mask-then-quant order (gamma over kept weights) fails this."""
    rng = np.random.default_rng(8)
    s = 0.02
    W = rng.standard_normal((1024, 4096)).astype(np.float32) * F32(s)
    w_eff, mask, g, sw = o.quant_mask_weight(W, N, M)
    p = 1 - (2 * ndtr(float(sw) / (2 * s)) - 1)
    j = np.arange(M + 1)
    pm = binom.pmf(j, M, p)
    mean = float((np.minimum(j, N) * pm).sum()) / M
    var = float(((np.minimum(j, N) / M - mean) ** 2 * pm).sum())
    groups = W.size // M
    dens = float((w_eff != 0).mean())
    assert abs(dens - mean) < 5 * math.sqrt(var / groups)


# ---------------------------------------------------------- Q_a (a1) ------
def _all_positive_bf16():
    u = np.arange(1, 0x7F80, dtype=np.uint32) << 16        # finite, > 0
    return u.view(np.float32)


def test_quant_act_every_bf16_scale():
    """Every finite positive bf16 row maximum m; invariants and the rounding
    error bound against exact fp64 arithmetic."""
    eps = 1e-5
    ms = _all_positive_bf16()                 # 32639 values
    rng = np.random.default_rng(9)
    K = 40
    frac = rng.uniform(-1, 1, size=(ms.size, K - 3))
    x = np.empty((ms.size, K), np.float32)
    x[:, 0] = ms
    x[:, 1] = -ms
    x[:, 2] = 0.0
    x[:, 3:] = bf16_round((frac * ms[:, None]).astype(np.float32))
    x[:, 3:] = np.clip(x[:, 3:], -ms[:, None], ms[:, None])
    q, sx = o.quant_act(x, eps)
    qi = q.astype(np.int64)
    assert np.all(np.abs(qi) <= 127)
    assert np.all((qi == 0) | (np.sign(qi) == np.sign(x)))
    big = ms >= 300 * eps
    assert np.all(qi[big, 0] == 127) and np.all(qi[big, 1] == -127)
    assert np.all(qi[:, 2] == 0)
    d64 = ms.astype(np.float64) + eps
    exact = x.astype(np.float64) * 127.0 / d64[:, None]
    assert np.all(np.abs(qi - exact) <= 0.5 + 1e-4)
    # monotone in x within a row
    order = np.argsort(x, axis=1, kind="stable")
    qs = np.take_along_axis(qi, order, 1)
    assert np.all(np.diff(qs, axis=1) >= 0)
    # dequant factor: sx * 127 = m + eps to fp32 accuracy
    assert np.all(np.abs(sx.astype(np.float64) * 127 - d64) <= 4e-7 * d64)


def test_quant_act_eps_placement_and_zero_rows():
    # eps is added to the max: with eps = m the scale halves; 63.5 -> 64 (even)
    q, sx = o.quant_act(np.array([[1.0, 0.5, -0.25]], np.float32), eps_a=1.0)
    assert q.tolist() == [[64, 32, -16]] and sx[0] == F32(2.0 / 127)
    # all-zero token: codes 0, sx = eps/127 (eps prevents division by zero)
    q, sx = o.quant_act(np.zeros((2, 16), np.float32), eps_a=1e-5)
    assert not q.any() and np.all(sx == F32(F32(1e-5) / F32(127)))


# -------------------------------------------------------- end to end (a6) --
def test_end_to_end_error_bound():
    """y against the unquantized-activation product x (sw W_eff)^T: the only
    difference is activation rounding, at most half an int8 step per term."""
    W, X = make_workload("tiny")
    x, w = X["x"], W["proj"]
    r = o.linear_fwd(x, w, 6, 8)
    ref = x.astype(np.float64) @ (float(r["sw"]) * r["w_eff"].astype(np.float64)).T
    bound = (0.5 * r["sx"].astype(np.float64)[:, None] * float(r["sw"])
             * np.abs(r["w_eff"]).sum(axis=1)[None, :]) * (1 + 1e-5) + 1e-12
    assert np.all(np.abs(r["y"] - ref) <= bound)


def test_to_bf16_is_nearest_even():
    rng = np.random.default_rng(10)
    y = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))
    # include exact bf16 midpoints (ties) and values just off them
    base = bf16_round(rng.standard_normal(200).astype(np.float32)).astype(np.float64)
    ulp = np.abs(base) * 2.0 ** -8
    y = np.concatenate([y, base + ulp / 2, base - ulp / 2, base + ulp / 2 * (1 + 2 ** -40)])
    b = o.to_bf16(y).astype(np.float64)
    # neighbours in bf16
    bu = b.astype(np.float32).view(np.uint32)
    up = ((bu + 0x10000)).view(np.float32).astype(np.float64)
    dn = ((bu - 0x10000)).view(np.float32).astype(np.float64)
    err = np.abs(b - y)
    assert np.all(err <= np.abs(up - y)) and np.all(err <= np.abs(dn - y))
    tie = (np.abs(up - y) == err) | (np.abs(dn - y) == err)
    assert np.all(((bu[tie] >> 16) & 1) == 0)         # ties -> even


def test_dequant_f32_rounds_each_step():
    """dequant_f32 against exact rational arithmetic: each product of two
    fp32 values is exact in Fraction, and np.float32(float(.)) of it is the
    nearest fp32 (the fp64 conversion is exact: 48 significant bits), so
    fp32(fp32(acc * sx) * sw) is fixed independently of numpy's float32
    multiply; it stays within two fp32 roundings of the fp64 ``dequant``."""
    from fractions import Fraction
    rng = np.random.default_rng(12)
    acc = rng.integers(-(127 * 8192), 127 * 8192, size=(6, 7)).astype(np.int32)
    acc[0, 0] = 0
    sx = rng.uniform(1e-4, 1.0, 6).astype(np.float32)
    sw = rng.uniform(1e-3, 0.1, 7).astype(np.float32)
    y = o.dequant_f32(acc, sx, sw)
    assert y.dtype == np.float32
    for t in range(6):
        for j in range(7):
            p1 = np.float32(float(Fraction(int(acc[t, j])) * Fraction(float(sx[t]))))
            p2 = np.float32(float(Fraction(float(p1)) * Fraction(float(sw[j]))))
            assert y[t, j] == p2
    ref = o.dequant(acc, sx, sw)
    assert np.all(np.abs(y - ref) <= 2.0 ** -23 * np.abs(ref))
    # scalar sw broadcasts like a per-row vector of equal values
    assert np.array_equal(o.dequant_f32(acc, sx, sw[2]), o.dequant_f32(acc, sx, np.full(7, sw[2])))


# ------------------------------------------------------------ packed format --
@pytest.mark.parametrize("M", [4, 8])
def test_pack_roundtrip_all_nm(M):
    rng = np.random.default_rng(11)
    for N in range(1, M + 1):
        for K in sorted({M, 2 * M, 32, 64 + M, 128, 136, 200 - 200 % M, 264}):
            if K % M:
                continue
            W = rng.standard_normal((6, K)).astype(np.float32)
            w_eff, mask, _, _ = o.quant_mask_weight(W, N, M)
            p = o.pack(w_eff, mask, N, M)
            assert p.size == o.packed_bytes(6, K, N, M)
            assert p.shape[1] % 16 == 0
            w2, m2 = o.unpack(p, 6, K, N, M)
            assert np.array_equal(w2, w_eff) and np.array_equal(m2, mask)
            # rows are independent records: concatenating along O commutes
            p_top = o.pack(w_eff[:2], mask[:2], N, M)
            assert np.array_equal(p[:2], p_top)


def test_pack_bits_per_weight():
    # 2:4 index form is 2 bits/weight; dense form 2 + 1 bits/weight
    assert o.packed_bytes(1, 1024, 2, 4) * 8 == 2 * 1024
    assert o.packed_bytes(1, 1024, 6, 8) * 8 == 3 * 1024
    # 2:8 in the index form: 2 bits/weight of selected codes + indices, 1 of mask
    assert o.packed_bytes(1, 1024, 2, 8) * 8 == 3 * 1024


def test_pack_hand_encoded_rows(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "packed_rows.json")))
    for c in ex["cases"]:
        w = np.array([c["w_eff"]], np.int8)
        m = np.array([c["mask"]], np.uint8)
        p = o.pack(w, m, c["N"], c["M"])
        assert p.tobytes().hex() == c["packed_hex"]
        w2, m2 = o.unpack(np.frombuffer(bytes.fromhex(c["packed_hex"]), np.uint8),
                          1, c["K"], c["N"], c["M"])
        assert np.array_equal(w2, w) and np.array_equal(m2, m)


def test_workload_shapes():
    W, X = make_workload("tiny")
    assert W["proj"].shape == (128, 256) and X["x"].shape == (16, 256)
    assert np.array_equal(X["x"], bf16_round(X["x"]))
    wl = WORKLOADS["qwen3b_sweep"]
    assert [l.K for l in wl.linears] == [2048, 2048, 11008]
    assert all(l.O % 128 == 0 and l.K % 128 == 0
               for w in WORKLOADS.values() for l in w.linears if w.name != "tiny")


# ------------------------------------------------------ mask diagnostics ---
@pytest.mark.parametrize("N,M", [(6, 8), (2, 4), (1, 8), (7, 8), (8, 8), (4, 4)])
def test_group_threshold_bruteforce_and_mask_relation(N, M):
    """The (N+1)-th largest |w| per group, by a plain sort of Python floats,
    and its relation to the mask: every kept magnitude >= t = the largest
    dropped magnitude (whatever the tie rule)."""
    rng = np.random.default_rng(N * 10 + M)
    w = rng.standard_normal((5, 8 * M)).astype(np.float32)
    w[0, :M] = 0.25                       # a group of ties
    w[1, M:2 * M] = np.float32(-0.0)      # signed zeros
    t = o.group_threshold(w, N, M)
    mask = o.nm_mask(w, N, M)
    for r in range(w.shape[0]):
        for g in range(w.shape[1] // M):
            mags = [abs(float(v)) for v in w[r, g * M:(g + 1) * M]]
            want = 0.0 if N == M else sorted(mags, reverse=True)[N]
            assert float(t[r, g]) == want
            kept = [m for m, k in zip(mags, mask[r, g * M:(g + 1) * M]) if k]
            dropped = [m for m, k in zip(mags, mask[r, g * M:(g + 1) * M]) if not k]
            if dropped:
                assert min(kept) >= float(t[r, g]) == max(dropped)


def test_mask_flips_hamming_and_pairs():
    a = np.array([[1, 1, 0, 0, 1, 0, 1, 0]], np.uint8)
    b = np.array([[0, 1, 1, 0, 1, 0, 1, 0]], np.uint8)
    assert o.mask_flips(a, b) == 2 == o.mask_flips(b, a)
    assert o.mask_flips(a, a) == 0
    rng = np.random.default_rng(3)
    w1 = rng.standard_normal((6, 64)).astype(np.float32)
    w2 = w1 + np.float32(0.3) * rng.standard_normal((6, 64)).astype(np.float32)
    m1, m2 = o.nm_mask(w1, 6, 8), o.nm_mask(w2, 6, 8)
    brute = sum(int(x != y) for x, y in zip(m1.ravel().tolist(), m2.ravel().tolist()))
    assert o.mask_flips(m1, m2) == brute
    # both masks keep exactly N per group: flips come in pairs within a group
    d = (m1 != m2).reshape(6, 8, 8).sum(axis=2)
    assert np.all(d % 2 == 0) and brute > 0


def test_mask_words_hand_layout():
    m = np.zeros((2, 40), np.uint8)
    m[0, [0, 31, 32, 39]] = 1
    m[1, 5] = 1
    words = o.mask_words(m)
    assert words.shape == (2, 4) and words.dtype == np.uint32
    assert words[0].tolist() == [0x80000001, 0x81, 0, 0]
    assert words[1].tolist() == [0x20, 0, 0, 0]


# ------------------------------------------------------- Q_a(Norm(x)) ------
def test_sum_squares_exact_rational():
    """S against exact rational arithmetic (fractions.Fraction, converted to
    fp64 with correct rounding), on rows whose squares span many binades --
    including sums a running fp64 total gets wrong (2^60 + 256 ones) and
    squares that are fp32 denormals -- and invariant under any permutation."""
    from fractions import Fraction
    rng = np.random.default_rng(11)
    rows = [rng.standard_normal(1000).astype(np.float32) * np.float32(3.0),
            np.concatenate([[np.float32(2.0 ** 30)], np.ones(256, np.float32)]),
            (rng.standard_normal(600) * np.exp2(rng.integers(-70, 60, 600))).astype(np.float32),
            np.array([2.0 ** -70, 2.0 ** -75, 3.0 * 2.0 ** -80, 0.0, -0.0], np.float32),
            np.zeros(16, np.float32)]
    for row in rows:
        S = o.sum_squares(row[None, :])[0]
        sq = (row * row).astype(np.float32)
        exact = sum((Fraction(float(v)) for v in sq), Fraction(0))
        assert S == float(exact)
        perm = row[rng.permutation(row.size)]
        assert o.sum_squares(perm[None, :])[0] == S
    # a running fp64 total loses every +1 next to 2^60: the exact sum does not
    assert o.sum_squares(rows[1][None, :])[0] == 2.0 ** 60 + 256.0


def test_rms_scale_closed_form():
    """r = fp32(1 / sqrt(S / K + eps)) with S exact: rows of c (r = 1/|c| up
    to eps) and the hand value of a row with two nonzero entries."""
    for c in (1.0, 0.5, 3.0, 2.0 ** 20):
        x = np.full((1, 64), c, np.float32)
        r = o.rms_scale(x, 1e-30)
        assert r[0] == np.float32(1.0 / c)
    x = np.zeros((1, 8), np.float32)
    x[0, :2] = [3.0, 4.0]
    r = o.rms_scale(x, 1e-6)
    assert r[0] == np.float32(1.0 / math.sqrt(25.0 / 8 + float(np.float32(1e-6))))


def test_rmsnorm_quant_act_hand_example_and_unit_rms():
    x = np.zeros((1, 8), np.float32)
    x[0, :2] = [3.0, 4.0]                     # S = 25, mean 25/8
    xq, sx = o.rmsnorm_quant_act(x, None, 1e-6, 1e-5)
    r = np.float32(1.0 / math.sqrt(25.0 / 8 + float(np.float32(1e-6))))
    z = (x * r).astype(np.float32)
    xq2, sx2 = o.quant_act(z)
    assert np.array_equal(xq, xq2) and np.array_equal(sx, sx2)
    assert xq[0, 1] == 127 and xq[0, 0] == round(127 * 3 / 4)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    r = o.rms_scale(x, 1e-12)
    z = x * r[:, None]
    assert np.allclose(np.mean(z.astype(np.float64) ** 2, axis=1), 1.0, rtol=1e-5)


def test_rmsnorm_quant_act_power_of_two_invariance():
    """Scaling x by 2 and eps_n by 4 scales S and S/K + eps exactly: r halves
    exactly, z and the codes are unchanged (with and without a gain)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(256)).astype(np.float32)
    for gain in (None, g):
        a = o.rmsnorm_quant_act(x, gain, float(np.float32(1e-5)), 1e-5)
        b = o.rmsnorm_quant_act(2 * x, gain, 4 * float(np.float32(1e-5)), 1e-5)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])

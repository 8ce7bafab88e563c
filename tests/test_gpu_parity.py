"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Integer stages (int8 activation codes, gamma/sw bits, masks, W_eff, packed
bytes, int32 accumulators) must match bit for bit; fp32 outputs within 1e-3
relative; bf16 outputs bit-identical to the bf16 rounding of the dequant
product taken in the reading's fixed fp32 order.
Inputs are seeded synthetic tensors from the workload generators; no expected
value comes from the HIP path.
"""
import math

import numpy as np
import pytest
import torch

import oracle as o
from sparse_linear_layers_bitlinear_amd.workloads import (
    WORKLOADS, bf16_round, make_linear_inputs, make_workload)
from gpu_helpers import (assert_bf16_exact, assert_f32_close, bf16_tensor, f32_bits, host,
                         log_case, to_dev)

pytestmark = pytest.mark.gpu
F32 = np.float32


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from sparse_linear_layers_bitlinear_amd import sbl
    return sbl


# ------------------------------------------------------------------ helpers --
def oracle_rows(W, N, M, rows, eps_w=1e-5):
    """Oracle weight side on a subset of rows (gamma from the full W)."""
    gamma, sw = o.absmean(W, eps_w)
    Wr = W[rows]
    mask = o.nm_mask(Wr, N, M)
    w_eff = o.apply_mask(o.ternary_codes(Wr, sw), mask)
    return w_eff, mask, gamma, sw


def packed_rows(packed_t, O, K, N, M, rows):
    pitch = o.packed_row_bytes(K, N, M)
    return host(packed_t).reshape(O, pitch)[rows]


# ------------------------------------------------------------ a1: Q_a -------
@pytest.mark.parametrize("dt,T,K,ldx", [
    ("bf16", 16, 256, 256), ("bf16", 7, 100, 100), ("bf16", 33, 896, 1024),
    ("bf16", 1, 11008, 11008), ("fp32", 5, 4864, 4864), ("fp32", 3, 12, 16),
    ("fp32", 130, 36, 36), ("bf16", 257, 2048, 2048)])
def test_quant_act_parity(S, dt, T, K, ldx):
    log_case("quant_act", dt, T, K, ldx)
    rng = np.random.default_rng(T * 131 + K)
    xf = rng.standard_normal((T, ldx)).astype(F32) * F32(rng.uniform(0.01, 50))
    xf[:, rng.choice(K, min(2, K), replace=False)] *= F32(10)
    if dt == "bf16":
        xf = bf16_round(xf)
        xt = bf16_tensor(xf)
    else:
        xt = to_dev(xf)
    xq, sx = S.sbl_quant_act(xt[:, :K] if ldx != K else xt)
    q_ref, sx_ref = o.quant_act(xf[:, :K])
    assert np.array_equal(host(xq), q_ref)
    assert np.array_equal(f32_bits(host(sx)), f32_bits(sx_ref))


def test_quant_act_every_bf16_scale(S):
    """Every finite positive bf16 row maximum, plus an all-zero row."""
    log_case("quant_act every bf16 max")
    u = np.arange(1, 0x7F80, dtype=np.uint32) << 16
    ms = u.view(np.float32)
    rng = np.random.default_rng(0)
    K = 64
    x = np.empty((ms.size + 1, K), np.float32)
    x[:-1, 0] = ms
    x[:-1, 1] = -ms
    x[:-1, 2:] = bf16_round((rng.uniform(-1, 1, (ms.size, K - 2)) * ms[:, None]).astype(F32))
    x[:-1, 2:] = np.clip(x[:-1, 2:], -ms[:, None], ms[:, None])
    x[-1] = 0
    for eps in (1e-5, 1e-8):
        xq, sx = S.sbl_quant_act(bf16_tensor(x), eps_a=eps)
        q_ref, sx_ref = o.quant_act(x, eps)
        assert np.array_equal(host(xq), q_ref)
        assert np.array_equal(f32_bits(host(sx)), f32_bits(sx_ref))


def test_quant_act_empty_and_errors(S):
    log_case("quant_act empty")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    xq, sx = S.sbl_quant_act(x)
    assert xq.shape == (0, 64)
    with pytest.raises(S.SblError):
        S.sbl_quant_act(torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda:0"), eps_a=0.0)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("T,K,gain", [(1, 896, True), (7, 4864, True), (64, 2048, False),
                                      (3, 8200, True), (5, 16, False), (33, 20000, True)])
def test_rmsnorm_quant_act_parity(S, dt, T, K, gain):
    """Q_a(RMSNorm(x) * g) in one pass: codes and scales bit for bit against
    the oracle (sum of squares exact, rounded once), rows longer than the
    register cache included."""
    if dt == "fp32" and K % 4:
        pytest.skip("K % 4")
    log_case("rmsnorm_quant_act", dt, T, K, gain)
    rng = np.random.default_rng(T * 7 + K)
    x = (rng.standard_normal((T, K), dtype=np.float32) * np.float32(2.0)).astype(F32)
    if dt == "bf16":
        x = bf16_round(x)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(F32) if gain else None
    xt = bf16_tensor(x) if dt == "bf16" else to_dev(x)
    xq, sx = S.sbl_rmsnorm_quant_act(xt, to_dev(g) if gain else None, eps_n=1e-6)
    rq, rs = o.rmsnorm_quant_act(x, g, 1e-6, 1e-5)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(f32_bits(host(sx)), f32_bits(rs))


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_rmsnorm_quant_act_extreme_ranges(S, dt):
    """Rows whose squares span many 32-binade windows of the exact sum (from
    fp32 denormals up to 2^120), a row of one huge value plus many small
    ones, zero rows and single nonzero entries: codes and scales bit for
    bit against the oracle's exactly rounded sum."""
    log_case("rmsnorm_quant_act extreme", dt)
    rng = np.random.default_rng(3)
    T, K = 12, 1024
    x = (rng.standard_normal((T, K)) * np.exp2(rng.integers(-70, 60, (T, K)))).astype(F32)
    x[1] = (rng.standard_normal(K) * np.exp2(rng.integers(-75, -60, K))).astype(F32)
    x[2] = 1.0
    x[2, 5] = 2.0 ** 30
    x[3] = 0.0
    x[4] = 0.0
    x[4, 1000] = -3.0
    x[5] = (rng.standard_normal(K) * 1e-3).astype(F32)
    x[5, :8] = 2.0 ** 50
    if dt == "bf16":
        x = bf16_round(x)
    xt = bf16_tensor(x) if dt == "bf16" else to_dev(x)
    for eps_n in (1e-6, 1e-30):
        xq, sx = S.sbl_rmsnorm_quant_act(xt, None, eps_n=eps_n)
        rq, rs = o.rmsnorm_quant_act(x, None, eps_n, 1e-5)
        assert np.array_equal(host(xq), rq)
        assert np.array_equal(f32_bits(host(sx)), f32_bits(rs))


@pytest.mark.parametrize("dt,K", [("bf16", 1024), ("bf16", 11008), ("fp32", 1024), ("fp32", 11008)])
def test_rmsnorm_quant_act_window_boundary(S, dt, K):
    """Rows at the edge of the kernel's fast exact sum (two fp64 windows of
    W = 54 - SB - ceil(log2 K) binades below the largest square, SB = 16 for
    bf16 and 24 for fp32): squares spanning 2W - 1 binades (fast, both
    windows used), 2W (general sum), squares exactly at the split and one
    binade below it, and one large square with many small ones 47 binades
    down whose low bits a single fp64 sum would lose. Codes and scales bit
    for bit against the oracle's exactly rounded sum."""
    sb = 16 if dt == "bf16" else 24
    W = 54 - sb - math.ceil(math.log2(K))
    log_case("rmsnorm_quant_act window boundary", dt, K, W)
    rng = np.random.default_rng(K + sb)
    rows = []
    for span2 in (2 * W - 1, 2 * W):             # largest square 2.25 * 2^(2 e_hi), smallest set by r[1]
        e_hi = 3
        e = rng.integers(e_hi - W + 1, e_hi + 1, K)
        r = (rng.uniform(1.0, 1.99, K) * np.exp2(e.astype(np.float64))).astype(F32)
        r *= np.where(rng.random(K) < 0.5, -1, 1).astype(F32)
        r[0] = F32(1.5 * 2.0 ** e_hi)                                   # square exponent 2 e_hi + 1
        r[1] = F32(2.0 ** (e_hi - span2 // 2)) if span2 % 2 else F32(1.5 * 2.0 ** (e_hi - span2 // 2))
        rows.append(r)
    r = (rng.uniform(1.0, 1.99, K) * np.exp2(rng.integers(-2, 3, K).astype(np.float64))).astype(F32)
    r[0] = F32(1.5 * 2.0 ** 4)                                          # largest square: exponent 9
    split = 9 - W + 1                                                   # squares at 2^split go high
    r[2:40] = F32(2.0 ** (split / 2)) if split % 2 == 0 else F32(2.0 ** ((split - 1) / 2) * 1.5)
    r[40:80] = F32(2.0 ** ((split - 1) / 2)) if (split - 1) % 2 == 0 else F32(2.0 ** ((split - 2) / 2) * 1.5)
    rows.append(r)
    r = np.full(K, F32(1.5078125 * 2.0 ** -18), dtype=F32)
    r[0] = F32(2.0 ** 6)
    rows.append(r)
    x = np.stack(rows).astype(F32)
    if dt == "bf16":
        x = bf16_round(x)
    xt = bf16_tensor(x) if dt == "bf16" else to_dev(x)
    for eps_n in (1e-6, 1e-30):
        xq, sx = S.sbl_rmsnorm_quant_act(xt, None, eps_n=eps_n)
        rq, rs = o.rmsnorm_quant_act(x, None, eps_n, 1e-5)
        assert np.array_equal(host(xq), rq)
        assert np.array_equal(f32_bits(host(sx)), f32_bits(rs))


def test_rmsnorm_quant_act_errors(S):
    x = torch.zeros((4, 12), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(S.SblError):
        S.sbl_rmsnorm_quant_act(x)                    # K % 8 != 0
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(S.SblError):
        S.sbl_rmsnorm_quant_act(x, eps_n=0.0)
    xq, sx = S.sbl_rmsnorm_quant_act(x[:0])
    assert xq.shape == (0, 64)


# ------------------------------------------------------ a2-a4: weight side --
NM_ALL = [(n, 4) for n in range(1, 5)] + [(n, 8) for n in range(1, 9)]


@pytest.mark.parametrize("N,M", NM_ALL)
@pytest.mark.parametrize("O,K,dt", [(128, 256, "fp32"), (37, 264, "fp32"), (19, 136, "bf16"),
                                    (5, 1032, "fp32"), (3, 8, "bf16")])
def test_quant_mask_weight_parity(S, N, M, O, K, dt):
    if K % M:
        pytest.skip("K % M")
    log_case("quant_mask_weight", N, M, O, K, dt)
    W, _ = make_linear_inputs(1, O, K, seed=O * 7 + K + N)
    if dt == "bf16":
        W = bf16_round(W)
        wt = bf16_tensor(W)
    else:
        wt = to_dev(W)
    r = S.sbl_quant_mask_weight(wt, N, M, want_w_eff=True, want_mask=True, want_sw_rows=True)
    w_eff, mask, gamma, sw = o.quant_mask_weight(W, N, M)
    gs = host(r["gamma_sw"])
    assert f32_bits(gs[0]) == f32_bits(gamma) and f32_bits(gs[1]) == f32_bits(sw)
    assert np.array_equal(host(r["mask"]), mask)
    assert np.array_equal(host(r["w_eff"]), w_eff)
    assert np.array_equal(host(r["packed"]).reshape(O, -1), o.pack(w_eff, mask, N, M))
    assert np.all(f32_bits(host(r["sw_rows"])) == f32_bits(sw))


@pytest.mark.parametrize("N,M", [(6, 8), (2, 4), (3, 8), (1, 4)])
@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_quant_mask_weight_batch_parity(S, N, M, dt):
    """Several tensors of different shapes (and scales, so every gamma
    differs) in one batched preparation: each equals the oracle and the
    single-tensor call bit for bit."""
    shapes = [(128, 256), (37, 264), (300, 1032), (5, 8), (64, 4096)]
    shapes = [(O, K) for O, K in shapes if K % M == 0]
    log_case("quant_mask_weight batch", N, M, dt, shapes)
    Ws, items = [], []
    for i, (O, K) in enumerate(shapes):
        W, _ = make_linear_inputs(1, O, K, seed=1000 + 17 * i + N, w_scale=0.01 * (i + 1))
        if dt == "bf16":
            W = bf16_round(W)
        Ws.append(W)
        items.append({"w": bf16_tensor(W) if dt == "bf16" else to_dev(W),
                      "w_eff": torch.empty((O, K), dtype=torch.int8, device="cuda:0"),
                      "mask": torch.empty((O, K), dtype=torch.uint8, device="cuda:0"),
                      "sw_rows": torch.empty(O, dtype=torch.float32, device="cuda:0")})
    outs = S.sbl_quant_mask_weight_batch(items, N, M)
    for W, it, r in zip(Ws, items, outs):
        O, K = W.shape
        w_eff, mask, gamma, sw = o.quant_mask_weight(W, N, M)
        gs = host(r["gamma_sw"])
        assert f32_bits(gs[0]) == f32_bits(gamma) and f32_bits(gs[1]) == f32_bits(sw)
        assert np.array_equal(host(r["mask"]), mask)
        assert np.array_equal(host(r["w_eff"]), w_eff)
        assert np.array_equal(host(r["packed"]).reshape(O, -1), o.pack(w_eff, mask, N, M))
        assert np.all(f32_bits(host(r["sw_rows"])) == f32_bits(sw))
        one = S.sbl_quant_mask_weight(it["w"], N, M)
        assert np.array_equal(host(one["packed"]), host(r["packed"]))
        assert np.array_equal(host(one["gamma_sw"]), gs)


@pytest.mark.parametrize("N,M", [(6, 8), (2, 4), (3, 8), (7, 8), (8, 8), (1, 4)])
@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_mask_diagnostics_parity(S, N, M, dt):
    """Mask diagnostics computed with the mask: the keep bits, the number of
    positions that flipped against a previous step's mask, and the (N+1)-th
    largest magnitude of every group -- bit for bit against the oracle."""
    shapes = [(37, 264), (64, 1024), (19, 136), (5, 8)]
    shapes = [(O, K) for O, K in shapes if K % M == 0]
    log_case("mask diagnostics", N, M, dt, shapes)
    rng = np.random.default_rng(N * 8 + M)
    cases, items = [], []
    for i, (O, K) in enumerate(shapes):
        W0, _ = make_linear_inputs(1, O, K, seed=2000 + i)
        W1 = (W0 + np.float32(0.01) * rng.standard_normal((O, K), dtype=np.float32)).astype(F32)
        if i == 0:
            W1[0, :M] = W1[0, 0]                 # a tied group
        if dt == "bf16":
            W0, W1 = bf16_round(W0), bf16_round(W1)
        prev = o.mask_words(o.nm_mask(W0, N, M))
        cases.append((W0, W1, prev))
        items.append({"w": bf16_tensor(W1) if dt == "bf16" else to_dev(W1),
                      "prev_mask_bits": to_dev(prev.view(np.int32)),
                      "want_mask_bits": True, "want_group_thr": True})
    outs = S.sbl_quant_mask_weight_batch(items, N, M)
    for (W0, W1, prev), r in zip(cases, outs):
        m0, m1 = o.nm_mask(W0, N, M), o.nm_mask(W1, N, M)
        assert np.array_equal(host(r["mask_bits"]).view(np.uint32), o.mask_words(m1))
        assert int(host(r["flips"])[0]) == o.mask_flips(m0, m1)
        assert np.array_equal(f32_bits(host(r["group_thr"])), f32_bits(o.group_threshold(W1, N, M)))
    # the flip counter starts from zero on every call
    outs2 = S.sbl_quant_mask_weight_batch(
        [dict(it, flips=r["flips"]) for it, r in zip(items, outs)], N, M)
    for (W0, W1, prev), r in zip(cases, outs2):
        assert int(host(r["flips"])[0]) == o.mask_flips(o.nm_mask(W0, N, M), o.nm_mask(W1, N, M))


@pytest.mark.parametrize("N,M", [(6, 8), (2, 4), (3, 8), (5, 8), (1, 4)])
@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_mask_from_ternary_variant_parity(S, N, M, dt):
    """The ablated recipe (mask ranked on |W_q|): mask, codes, packing and the
    diagnostics against the oracle; the method's prep of the same W differs."""
    shapes = [(37, 264), (64, 1024), (5, 8)]
    shapes = [(O, K) for O, K in shapes if K % M == 0]
    log_case("mask from ternary", N, M, dt, shapes)
    Ws, items = [], []
    for i, (O, K) in enumerate(shapes):
        W, _ = make_linear_inputs(1, O, K, seed=3000 + i + N)
        if dt == "bf16":
            W = bf16_round(W)
        Ws.append(W)
        items.append({"w": bf16_tensor(W) if dt == "bf16" else to_dev(W), "variant": 1,
                      "w_eff": torch.empty((O, K), dtype=torch.int8, device="cuda:0"),
                      "mask": torch.empty((O, K), dtype=torch.uint8, device="cuda:0"),
                      "want_mask_bits": True, "want_group_thr": True})
    outs = S.sbl_quant_mask_weight_batch(items, N, M)
    differs = False
    for W, r in zip(Ws, outs):
        w_eff, mask, gamma, sw = o.quant_mask_weight(W, N, M, variant="ternary")
        assert np.array_equal(host(r["mask"]), mask)
        assert np.array_equal(host(r["w_eff"]), w_eff)
        assert np.array_equal(host(r["packed"]).reshape(W.shape[0], -1), o.pack(w_eff, mask, N, M))
        assert np.array_equal(host(r["mask_bits"]).view(np.uint32), o.mask_words(mask))
        assert np.array_equal(f32_bits(host(r["group_thr"])), f32_bits(o.dropped_max(W, mask, M)))
        differs |= not np.array_equal(mask, o.nm_mask(W, N, M))
    assert differs


@pytest.mark.parametrize("N,M", [(6, 8), (2, 4), (7, 8), (8, 8), (3, 8), (1, 4), (2, 8)])
@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_mask_then_quant_variant_parity(S, N, M, dt):
    """The composition-order ablation (gamma over the kept weights): gamma and
    sw bit for bit, codes, mask, packing and the dropped maximum against the
    oracle, in one batch of ragged shapes; the last item spans a wide exponent
    range so the exact sum leaves its main window. K = 100 (M = 4 only) leaves
    bf16 rows unaligned, so that batch takes the element-wise loads."""
    shapes = [(37, 264), (64, 1024), (5, 8), (11, 100), (19, 72)]
    shapes = [(O, K) for O, K in shapes if K % M == 0]
    log_case("mask then quant", N, M, dt, shapes)
    rng = np.random.default_rng(77 + N)
    Ws, items = [], []
    for i, (O, K) in enumerate(shapes):
        W, _ = make_linear_inputs(1, O, K, seed=4000 + i + N)
        if i == len(shapes) - 1:
            W = (W * np.exp2(rng.integers(-60, 60, W.shape))).astype(np.float32)
        if dt == "bf16":
            W = bf16_round(W)
        Ws.append(W)
        items.append({"w": bf16_tensor(W) if dt == "bf16" else to_dev(W), "variant": 2,
                      "w_eff": torch.empty((O, K), dtype=torch.int8, device="cuda:0"),
                      "mask": torch.empty((O, K), dtype=torch.uint8, device="cuda:0"),
                      "want_group_thr": True})
    outs = S.sbl_quant_mask_weight_batch(items, N, M)
    for W, r in zip(Ws, outs):
        w_eff, mask, gamma, sw = o.quant_mask_weight(W, N, M, variant="mask_then_quant")
        gs = host(r["gamma_sw"])
        assert f32_bits(gs[0]) == f32_bits(gamma) and f32_bits(gs[1]) == f32_bits(sw)
        assert np.array_equal(host(r["mask"]), mask)
        assert np.array_equal(host(r["w_eff"]), w_eff)
        assert np.array_equal(host(r["packed"]).reshape(W.shape[0], -1), o.pack(w_eff, mask, N, M))
        assert np.array_equal(f32_bits(host(r["group_thr"])), f32_bits(o.dropped_max(W, mask, M)))


def test_mask_then_quant_full_size(S):
    """The Qwen2.5-0.5B FFN projections under mask-then-quant, one batch."""
    from sparse_linear_layers_bitlinear_amd.workloads import WORKLOADS, make_workload
    log_case("mask then quant full", "qwen05b_ffn")
    wl = WORKLOADS["qwen05b_ffn"]
    W, _ = make_workload("qwen05b_ffn")
    items = [{"w": to_dev(W[l.name]), "variant": 2} for l in wl.linears]
    outs = S.sbl_quant_mask_weight_batch(items, wl.N, wl.M)
    for l, r in zip(wl.linears, outs):
        w_eff, mask, gamma, sw = o.quant_mask_weight(W[l.name], wl.N, wl.M, variant="mask_then_quant")
        gs = host(r["gamma_sw"])
        assert f32_bits(gs[0]) == f32_bits(gamma) and f32_bits(gs[1]) == f32_bits(sw)
        assert np.array_equal(host(r["packed"]).reshape(l.O, -1), o.pack(w_eff, mask, wl.N, wl.M))


def test_quant_mask_weight_batch_full_size(S):
    """The three projections of the Qwen2.5-0.5B FFN prepared in one batch
    (K differs between them), as the benchmark step does."""
    from sparse_linear_layers_bitlinear_amd.workloads import WORKLOADS, make_workload
    log_case("quant_mask_weight batch full", "qwen05b_ffn")
    wl = WORKLOADS["qwen05b_ffn"]
    W, _ = make_workload("qwen05b_ffn")
    items = [{"w": to_dev(W[l.name])} for l in wl.linears]
    outs = S.sbl_quant_mask_weight_batch(items, wl.N, wl.M)
    for l, r in zip(wl.linears, outs):
        w_eff, mask, gamma, sw = o.quant_mask_weight(W[l.name], wl.N, wl.M)
        gs = host(r["gamma_sw"])
        assert f32_bits(gs[0]) == f32_bits(gamma) and f32_bits(gs[1]) == f32_bits(sw)
        assert np.array_equal(host(r["packed"]).reshape(l.O, -1), o.pack(w_eff, mask, wl.N, wl.M))


def test_roundclip_boundary(S):
    """Weights within a few ulps of the zero/one rounding boundary sw/2 (and
    exact ties, which round to even = 0)."""
    log_case("roundclip boundary")
    rng = np.random.default_rng(42)
    O, K = 64, 512
    W = rng.standard_normal((O, K)).astype(F32) * F32(0.02)
    idx = rng.choice(O * K, 4096, replace=False)
    offs = np.arange(-8, 9)
    for _ in range(10):  # fixed point: boundary values relative to the final sw
        _, sw = o.absmean(W)
        half = np.float32(sw) * F32(0.5)
        vals = (half.view(np.uint32) + offs[np.arange(idx.size) % offs.size]).astype(np.uint32)
        vals = vals.view(np.float32) * np.where(np.arange(idx.size) % 2, F32(-1), F32(1))
        W.reshape(-1)[idx] = vals
        if o.absmean(W)[1] == sw:
            break
    _, sw = o.absmean(W)
    assert np.all(np.abs(W.reshape(-1)[idx]) == np.abs(vals))
    for N, M in [(6, 8), (2, 4), (8, 8)]:
        r = S.sbl_quant_mask_weight(to_dev(W), N, M, want_w_eff=True, want_mask=True)
        w_eff, mask, _, sw_ref = o.quant_mask_weight(W, N, M)
        assert f32_bits(host(r["gamma_sw"])[1]) == f32_bits(sw_ref)
        assert np.array_equal(host(r["w_eff"]), w_eff)
        assert np.array_equal(host(r["mask"]), mask)


def test_absmean_extreme_ranges(S):
    log_case("absmean extreme ranges")
    rng = np.random.default_rng(5)
    cases = {
        "wide": (rng.standard_normal((16, 1024)) * np.exp2(rng.integers(-149, 120, (16, 1024)))
                 ).astype(F32),
        "denormal": (rng.standard_normal((8, 256)) * F32(1e-41)).astype(F32),
        "huge": (rng.standard_normal((8, 256)) * F32(1e37)).astype(F32),
        "zero": np.zeros((4, 64), F32),
        "ties": np.round(rng.standard_normal((32, 128)) * 3).astype(F32) * F32(0.01),
    }
    for name, W in cases.items():
        for N, M in [(6, 8), (2, 4)]:
            r = S.sbl_quant_mask_weight(to_dev(W), N, M, want_w_eff=True, want_mask=True)
            w_eff, mask, gamma, sw = o.quant_mask_weight(W, N, M)
            gs = host(r["gamma_sw"])
            assert f32_bits(gs[0]) == f32_bits(gamma), name
            assert f32_bits(gs[1]) == f32_bits(sw), name
            assert np.array_equal(host(r["mask"]), mask), name
            assert np.array_equal(host(r["w_eff"]), w_eff), name


@pytest.mark.parametrize("dt", [np.float32, "bf16"])
def test_absmean_outliers_in_some_blocks(S, dt):
    """Tensors large enough for many partial-pass workgroups, with a few
    magnitudes outside [2^-31, 2) (and zeros) in some of them only: gamma
    stays exact whether every workgroup's terms lie in that window or not,
    alone and in a batch that mixes both kinds of tensor."""
    log_case("absmean outliers in some blocks", dt)
    rng = np.random.default_rng(6)
    clean = (rng.standard_normal((1536, 1024)) * 0.02).astype(F32)
    dirty = clean.copy()
    flat = dirty.reshape(-1)
    pos = rng.choice(flat.size, 7, replace=False)
    flat[pos] = np.array([3.0, -1e5, 2.0, 1e-20, -3e-30, 0.0, 7e3], F32)
    if dt == "bf16":
        clean, dirty = bf16_round(clean), bf16_round(dirty)
    dev = lambda a: to_dev(a) if dt == np.float32 else to_dev(a).to(torch.bfloat16)
    wide = (rng.standard_normal((512, 1024)) * 0.02).astype(F32)
    wide[::37, ::53] *= F32(1e6)
    if dt == "bf16":
        wide = bf16_round(wide)
    for W in (clean, dirty, wide):
        g_ref, sw_ref = o.absmean(W)
        r = S.sbl_quant_mask_weight(dev(W), 6, 8)
        gs = host(r["gamma_sw"])
        assert f32_bits(gs[0]) == f32_bits(g_ref) and f32_bits(gs[1]) == f32_bits(sw_ref)
    for order in ((clean, dirty, wide), (dirty, clean), (clean, clean, wide, clean),
                  (clean, dirty, clean, wide, dirty, clean, wide, clean)):   # the largest batch
        outs = S.sbl_quant_mask_weight_batch([{"w": dev(W)} for W in order], 6, 8)
        for W, r in zip(order, outs):
            g_ref, sw_ref = o.absmean(W)
            gs = host(r["gamma_sw"])
            assert f32_bits(gs[0]) == f32_bits(g_ref) and f32_bits(gs[1]) == f32_bits(sw_ref)


@pytest.mark.parametrize("M", [8, 4])
def test_mask_every_tie_pattern(S, M):
    """Every group of M magnitudes drawn from {0, 1, 2} (M = 8: 6561 groups)
    or {0, 1, 2, 3} (M = 4: 256 groups), with random signs and signed zeros,
    for every N: the GPU mask (and codes) equal the oracle's rank rule."""
    log_case("mask tie patterns", M)
    levels = 3 if M == 8 else 4
    pats = np.array(np.meshgrid(*[np.arange(levels)] * M, indexing="ij")).reshape(M, -1).T
    rng = np.random.default_rng(11)
    sign = np.where(rng.random(pats.shape) < 0.5, -1.0, 1.0)
    W = (pats * sign).astype(F32) * F32(0.01)
    W = W.reshape(-1, (81 if M == 8 else 16) * M)   # 81 (16) groups per row
    for N in range(1, M + 1):
        r = S.sbl_quant_mask_weight(to_dev(W), N, M, want_w_eff=True, want_mask=True)
        w_eff, mask, gamma, sw = o.quant_mask_weight(W, N, M)
        assert np.array_equal(host(r["mask"]), mask), N
        assert np.array_equal(host(r["w_eff"]), w_eff), N


def test_weight_prep_errors(S):
    log_case("quant_mask_weight errors")
    w = torch.zeros((4, 12), dtype=torch.float32, device="cuda:0")
    with pytest.raises(S.SblError):       # K % M
        S.sbl_quant_mask_weight(w, 6, 8)
    with pytest.raises(S.SblError):       # N > M
        S.sbl_quant_mask_weight(w, 5, 4)


# ------------------------------------------------------------- pack/unpack --
@pytest.mark.parametrize("N,M", NM_ALL)
def test_pack_unpack_parity(S, N, M):
    log_case("pack/unpack", N, M)
    for O, K in [(9, 8 * M), (4, 136), (2, 1024)]:
        if K % M:
            continue
        W, _ = make_linear_inputs(1, O, K, seed=N * 11 + M + K)
        w_eff, mask, _, _ = o.quant_mask_weight(W, N, M)
        p = S.sbl_pack(to_dev(w_eff), to_dev(mask), N, M)
        ref = o.pack(w_eff, mask, N, M)
        assert np.array_equal(host(p).reshape(O, -1), ref)
        w2, m2 = S.sbl_unpack(to_dev(ref.reshape(-1)), O, K, N, M)
        assert np.array_equal(host(w2), w_eff) and np.array_equal(host(m2), mask)


# ------------------------------------------------------------- a5+a6: GEMM --
def _gemm_case(S, T, O, K, N, M, ydt, seed, sw_per_row):
    rng = np.random.default_rng(seed)
    xq = rng.integers(-128, 128, size=(T, K)).astype(np.int8)
    W = rng.standard_normal((O, K)).astype(F32)
    w_eff, mask, _, _ = o.quant_mask_weight(W, N, M)
    packed = o.pack(w_eff, mask, N, M)
    sx = rng.uniform(1e-3, 1.0, T).astype(F32)
    sw = (rng.uniform(1e-3, 0.1, O) if sw_per_row else rng.uniform(1e-3, 0.1, 1)).astype(F32)
    y, acc = S.sbl_gemm(to_dev(xq), to_dev(sx), to_dev(packed.reshape(-1)), to_dev(sw), O, N, M,
                        out_dtype=ydt, want_acc=True)
    acc_ref = o.gemm_int(xq, w_eff)
    assert np.array_equal(host(acc), acc_ref)
    y_ref = o.dequant(acc_ref, sx, sw if sw_per_row else sw[0])
    if ydt == torch.float32:
        assert_f32_close(host(y), y_ref)
    else:
        assert_bf16_exact(host(y), acc_ref, sx, sw if sw_per_row else sw[0])
        # without the int32 output the prefill kernel stages the bf16 tile in
        # LDS and writes whole row segments: a separate epilogue
        y2 = S.sbl_gemm(to_dev(xq), to_dev(sx), to_dev(packed.reshape(-1)), to_dev(sw), O, N, M,
                        out_dtype=ydt)
        assert_bf16_exact(host(y2), acc_ref, sx, sw if sw_per_row else sw[0])


@pytest.mark.parametrize("N,M", [(6, 8), (2, 4), (2, 8), (1, 4), (8, 8), (4, 8), (3, 8), (7, 8)])
@pytest.mark.parametrize("T,O,K", [(1, 7, 64), (5, 130, 264), (16, 128, 256), (33, 200, 1024),
                                   (130, 67, 136), (257, 256, 512), (64, 1, 128), (40, 96, 1000)])
def test_gemm_parity(S, N, M, T, O, K):
    if K % M:
        pytest.skip("K % M")
    log_case("gemm", N, M, T, O, K)
    _gemm_case(S, T, O, K, N, M, torch.float32, seed=T + O + K + N, sw_per_row=True)
    _gemm_case(S, T, O, K, N, M, torch.bfloat16, seed=T + O + K + N + 1, sw_per_row=False)


def test_gemm_empty_and_deterministic(S):
    log_case("gemm empty / determinism")
    xq = torch.zeros((0, 64), dtype=torch.int8, device="cuda:0")
    sx = torch.zeros((0,), dtype=torch.float32, device="cuda:0")
    pk = torch.zeros(o.packed_bytes(8, 64, 6, 8), dtype=torch.uint8, device="cuda:0")
    sw = torch.ones(1, dtype=torch.float32, device="cuda:0")
    y = S.sbl_gemm(xq, sx, pk, sw, 8, 6, 8)
    assert y.shape == (0, 8)
    rng = np.random.default_rng(9)
    T, O, K = 300, 520, 768
    for N, M in [(6, 8), (2, 4)]:
        xq = to_dev(rng.integers(-128, 128, size=(T, K)).astype(np.int8))
        W = rng.standard_normal((O, K)).astype(F32)
        r = S.sbl_quant_mask_weight(to_dev(W), N, M)
        sx = to_dev(rng.uniform(0.01, 1, T).astype(F32))
        outs = [host(S.sbl_gemm(xq, sx, r["packed"], r["gamma_sw"][1:], O, N, M,
                                want_acc=True)[1]) for _ in range(3)]
        assert all(np.array_equal(outs[0], x) for x in outs[1:])


# -------------------------------------------------------------- end to end --
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16])
def test_linear_fwd_tiny_config(S, ydt):
    """16 tokens, K=256, O=128, 6:8, two x10 outlier channels."""
    log_case("linear_fwd tiny", ydt)
    W, X = make_workload("tiny")
    w, x = W["proj"], X["x"]
    y = S.sbl_linear_fwd(bf16_tensor(x), 6, 8, w_master=to_dev(w), out_dtype=ydt)
    ref = o.linear_fwd(x, w, 6, 8)
    if ydt == torch.float32:
        assert_f32_close(host(y), ref["y"])
    else:
        assert_bf16_exact(host(y), ref["acc"], ref["sx"], ref["sw"])
    # the same through the separate calls, with every intermediate
    xq, sx = S.sbl_quant_act(bf16_tensor(x))
    r = S.sbl_quant_mask_weight(to_dev(w), 6, 8, want_w_eff=True, want_mask=True)
    yy, acc = S.sbl_gemm(xq, sx, r["packed"], r["gamma_sw"][1:], 128, 6, 8,
                         out_dtype=torch.float32, want_acc=True)
    assert np.array_equal(host(xq), ref["xq"])
    assert np.array_equal(f32_bits(host(sx)), f32_bits(ref["sx"]))
    assert np.array_equal(host(r["w_eff"]), ref["w_eff"])
    assert np.array_equal(host(r["mask"]), ref["mask"])
    assert np.array_equal(host(acc), ref["acc"])
    assert_f32_close(host(yy), ref["y"])
    # prepacked path
    y2 = S.sbl_linear_fwd(bf16_tensor(x), 6, 8, prepacked=r["packed"], sw=r["gamma_sw"][1:],
                          O=128, out_dtype=torch.float32)
    assert_f32_close(host(y2), ref["y"])


def _full_projection(S, W, x, N, M, rows_t, rows_o, sw_full=None):
    """GPU weight prep + act quant + GEMM at full size; oracle on sampled rows."""
    O, K = W.shape
    r = S.sbl_quant_mask_weight(to_dev(W), N, M, want_w_eff=False, want_mask=False)
    xq, sx = S.sbl_quant_act(bf16_tensor(x))
    y, acc = S.sbl_gemm(xq, sx, r["packed"], r["gamma_sw"][1:], O, N, M,
                        out_dtype=torch.bfloat16, want_acc=True)
    w_eff_s, mask_s, gamma, sw = oracle_rows(W, N, M, rows_o)
    gs = host(r["gamma_sw"])
    assert f32_bits(gs[0]) == f32_bits(gamma) and f32_bits(gs[1]) == f32_bits(sw)
    assert np.array_equal(packed_rows(r["packed"], O, K, N, M, rows_o),
                          o.pack(w_eff_s, mask_s, N, M))
    xq_s, sx_s = o.quant_act(x[rows_t])
    assert np.array_equal(host(xq)[rows_t], xq_s)
    assert np.array_equal(f32_bits(host(sx)[rows_t]), f32_bits(sx_s))
    acc_s = o.gemm_int(xq_s, w_eff_s)
    acc_g = host(acc)[np.ix_(rows_t, rows_o)]
    assert np.array_equal(acc_g, acc_s)
    assert_bf16_exact(host(y)[np.ix_(rows_t, rows_o)], acc_s, sx_s, sw)
    # bf16 y alone (the staged epilogue the benchmark times)
    y2 = S.sbl_gemm(xq, sx, r["packed"], r["gamma_sw"][1:], O, N, M, out_dtype=torch.bfloat16)
    assert_bf16_exact(host(y2)[np.ix_(rows_t, rows_o)], acc_s, sx_s, sw)


def _sample(n, k, seed):
    rng = np.random.default_rng(seed)
    s = np.unique(np.concatenate([[0, n - 1], rng.choice(n, min(n, k), replace=False)]))
    return s


@pytest.mark.parametrize("wl", ["qwen05b_ffn", "qwen15b_ffn"])
def test_full_size_ffn(S, wl):
    W, X = make_workload(wl)
    w = WORKLOADS[wl]
    for lin in w.linears:
        log_case("full size", wl, lin.name, w.T, lin.O, lin.K, f"{w.N}:{w.M}")
        _full_projection(S, W[lin.name], X[lin.x_name], w.N, w.M,
                         _sample(w.T, 64, 1), _sample(lin.O, 192, 2))


def test_full_size_qwen3b_sweep(S):
    wl = WORKLOADS["qwen3b_sweep"]
    W, X = make_workload("qwen3b_sweep")
    for (N, M) in wl.nm_sweep:
        for lin in wl.linears:
            if lin.name == "up" and (N, M) != (6, 8):
                continue
            log_case("full size qwen3b", lin.name, f"{N}:{M}", wl.T, lin.O, lin.K)
            _full_projection(S, W[lin.name], X[lin.x_name], N, M,
                             _sample(wl.T, 32, N), _sample(lin.O, 96, N + 1))


@pytest.mark.parametrize("wl,nm", [("qwen05b_ffn", None), ("qwen15b_ffn", None),
                                   ("qwen3b_sweep", (6, 8)), ("qwen3b_sweep", (2, 4)),
                                   ("qwen3b_sweep", (2, 8))])
def test_prefill_bench_launches(S, wl, nm):
    """The GEMM calls the prefill benchmark times, as it makes them: per input
    one sbl_gemm over the group's tensors concatenated along O (gate|up) with
    per-row sw written by each tensor's preparation, int8 x from
    sbl_quant_act, bf16 y into a preallocated buffer, no int32 output. Sampled
    rows and columns of each segment against the oracle, bit for bit."""
    w = WORKLOADS[wl]
    N, M = nm if nm else (w.N, w.M)
    W, X = make_workload(wl)
    groups = {}
    for lin in w.linears:
        groups.setdefault(lin.x_name, []).append(lin)
    for xn, lins in groups.items():
        K = dict(w.x_specs)[xn]
        O = sum(l.O for l in lins)
        log_case("prefill bench launch", wl, f"{N}:{M}", "+".join(l.name for l in lins), w.T, O, K)
        packed = torch.empty(S.sbl_packed_bytes(O, K, N, M), dtype=torch.uint8, device="cuda:0")
        swr = torch.empty(O, dtype=torch.float32, device="cuda:0")
        op, oo = 0, 0
        for l in lins:
            nb = S.sbl_packed_bytes(l.O, l.K, N, M)
            S.sbl_quant_mask_weight(to_dev(W[l.name]), N, M, packed=packed[op:op + nb],
                                    sw_rows=swr[oo:oo + l.O])
            op += nb
            oo += l.O
        x = X[xn]
        xq, sx = S.sbl_quant_act(bf16_tensor(x))
        y = torch.empty((w.T, O), dtype=torch.bfloat16, device="cuda:0")
        S.sbl_gemm(xq, sx, packed, swr, O, N, M, y=y)
        yh = host(y)
        rows_t = _sample(w.T, 24, O)
        xq_s, sx_s = o.quant_act(x[rows_t])
        oo = 0
        for i, l in enumerate(lins):
            rows_o = _sample(l.O, 64, i + 3)
            w_eff_s, _, _, sw = oracle_rows(W[l.name], N, M, rows_o)
            acc_s = o.gemm_int(xq_s, w_eff_s)
            assert_bf16_exact(yh[np.ix_(rows_t, oo + rows_o)], acc_s, sx_s, sw)
            oo += l.O


@pytest.mark.parametrize("T", [1, 4, 8])
def test_decode_bitnet_layer(S, T):
    """Prepacked 2:4 decode projections of a BitNet-2B4T-shaped layer."""
    wl = WORKLOADS["bitnet_decode"]
    W, X = make_workload("bitnet_decode", T=T)
    for lin in wl.linears:
        log_case("decode", T, lin.name, lin.O, lin.K)
        w = W[lin.name]
        r = S.sbl_quant_mask_weight(to_dev(w), 2, 4)
        x = X[lin.x_name]
        y = S.sbl_linear_fwd(bf16_tensor(x), 2, 4, prepacked=r["packed"], sw=r["gamma_sw"][1:],
                             O=lin.O, out_dtype=torch.float32)
        ref = o.linear_fwd(x, w, 2, 4)
        assert_f32_close(host(y), ref["y"])


# ---------------------------------------------- decode path (T <= 16 tokens) --
def _x_tensor(x, xdt):
    return bf16_tensor(x) if xdt == "bf16" else to_dev(x)


def _x_host(x, xdt):
    """The activations the library sees (bf16 inputs round to bf16 first)."""
    return bf16_round(x) if xdt == "bf16" else x


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("xdt", ["bf16", "fp32"])
@pytest.mark.parametrize("N,M,O,K", [(2, 4, 200, 2560), (6, 8, 37, 1000), (2, 4, 64, 6912),
                                     (6, 8, 130, 8192), (2, 4, 48, 264), (1, 4, 16, 128),
                                     (2, 8, 96, 1000)])
def test_decode_fused_linear(S, T, xdt, N, M, O, K):
    """Decode-sized batches: sbl_linear_fwd quantizes the activations inside
    the GEMV. Against the oracle, and bit-identical to the separate
    activation-quantization and GEMM calls."""
    log_case("decode fused", T, xdt, N, M, O, K)
    W, x = make_linear_inputs(T, O, K, seed=T * 31 + O + K + N)
    if xdt == "fp32":   # full fp32 values, not bf16-exact ones
        x = np.random.default_rng(T + K).standard_normal((T, K), dtype=np.float32)
    xt = _x_tensor(x, xdt)
    r = S.sbl_quant_mask_weight(to_dev(W), N, M)
    y = S.sbl_linear_fwd(xt, N, M, prepacked=r["packed"], sw=r["gamma_sw"][1:], O=O,
                         out_dtype=torch.float32)
    yb = S.sbl_linear_fwd(xt, N, M, prepacked=r["packed"], sw=r["gamma_sw"][1:], O=O,
                          out_dtype=torch.bfloat16)
    ref = o.linear_fwd(_x_host(x, xdt), W, N, M)
    assert_f32_close(host(y), ref["y"])
    assert_bf16_exact(host(yb), ref["acc"], ref["sx"], ref["sw"])
    xq, sx = S.sbl_quant_act(xt)
    assert np.array_equal(host(xq), ref["xq"])
    y2, acc = S.sbl_gemm(xq, sx, r["packed"], r["gamma_sw"][1:], O, N, M,
                         out_dtype=torch.float32, want_acc=True)
    assert np.array_equal(host(acc), ref["acc"])
    assert np.array_equal(f32_bits(host(y)), f32_bits(host(y2)))
    # from master weights (weight preparation, then the fused decode)
    y3 = S.sbl_linear_fwd(xt, N, M, w_master=to_dev(W), out_dtype=torch.float32)
    assert np.array_equal(f32_bits(host(y3)), f32_bits(host(y)))


@pytest.mark.parametrize("R", [2, 3, 9, 20])
def test_decode_tiles_per_workgroup(S, R, monkeypatch):
    """Several 16-row tiles per decode workgroup, forced through the
    workgroup count (ceil(tiles / R) workgroups), ragged O, per-row sw; R = 9
    and 20 take more tiles than a workgroup has wavefronts."""
    for (T, O, K, N, M) in [(4, 1000, 512, 2, 4), (16, 333, 1024, 6, 8), (1, 17, 128, 2, 4),
                            (7, 130, 2688, 4, 8), (8, 700, 256, 2, 4)]:
        tiles = -(-O // 16)
        monkeypatch.setenv("SBL_DECODE_BLOCKS", str(-(-tiles // R)))
        log_case("decode R", R, T, O, K, N, M)
        _gemm_case(S, T, O, K, N, M, torch.bfloat16, seed=R * 13 + T + O, sw_per_row=True)
        W, x = make_linear_inputs(T, O, K, seed=R + O)
        r = S.sbl_quant_mask_weight(to_dev(W), N, M, want_sw_rows=True)
        xr = bf16_round(x)
        ref = o.linear_fwd(xr, W, N, M)
        y = S.sbl_linear_fwd(bf16_tensor(x), N, M, prepacked=r["packed"],
                             sw=r["sw_rows"], O=O, out_dtype=torch.float32)
        assert_f32_close(host(y), ref["y"])
        yb = S.sbl_linear_fwd(bf16_tensor(x), N, M, prepacked=r["packed"],
                              sw=r["sw_rows"], O=O, out_dtype=torch.bfloat16)
        assert_bf16_exact(host(yb), ref["acc"], ref["sx"], ref["sw"])


@pytest.mark.parametrize("tg", [1, 2, 3, 5])
def test_decode_token_groups(S, tg, monkeypatch):
    """Token groups of the decode GEMV forced (the last group ragged), with
    forced slice counts too: every group quantizes its own rows and stores its
    own outputs."""
    monkeypatch.setenv("SBL_DECODE_TG", str(tg))
    for (T, O, K, N, M, slices) in [(16, 333, 1024, 6, 8, 0), (7, 1000, 2560, 2, 4, 0),
                                    (8, 130, 6912, 2, 4, 3), (5, 64, 512, 4, 8, 0)]:
        if slices:
            monkeypatch.setenv("SBL_DECODE_BLOCKS", str(slices))
        else:
            monkeypatch.delenv("SBL_DECODE_BLOCKS", raising=False)
        log_case("decode token groups", tg, T, O, K, N, M, slices)
        W, x = make_linear_inputs(T, O, K, seed=tg * 17 + O)
        r = S.sbl_quant_mask_weight(to_dev(W), N, M, want_sw_rows=True)
        ref = o.linear_fwd(bf16_round(x), W, N, M)
        yb = S.sbl_linear_fwd(bf16_tensor(x), N, M, prepacked=r["packed"], sw=r["sw_rows"], O=O,
                              out_dtype=torch.bfloat16)
        assert_bf16_exact(host(yb), ref["acc"], ref["sx"], ref["sw"])
        xq, sx = S.sbl_quant_act(bf16_tensor(x))
        y2, acc = S.sbl_gemm(xq, sx, r["packed"], r["sw_rows"], O, N, M,
                             out_dtype=torch.float32, want_acc=True)
        assert np.array_equal(host(acc), ref["acc"])
        assert_f32_close(host(y2), ref["y"])


@pytest.mark.parametrize("T", [1, 4, 8])
def test_decode_bench_launches(S, T):
    """The calls the decode benchmark times, as it makes them: per projection
    group of a BitNet-2B4T-shaped layer one sbl_linear_fwd on prepacked 2:4
    weights, the group's tensors concatenated along O (q|k|v, gate|up) with
    per-row sw written by each tensor's preparation (sw_inc = 1), bf16 x
    quantized inside the GEMV, bf16 y. Each segment against the oracle."""
    wl = WORKLOADS["bitnet_decode"]
    W, X = make_workload("bitnet_decode", T=T)
    groups = {}
    for lin in wl.linears:
        groups.setdefault(lin.x_name, []).append(lin)
    for xn, lins in groups.items():
        K = dict(wl.x_specs)[xn]
        O = sum(l.O for l in lins)
        log_case("decode bench launch", T, "+".join(l.name for l in lins), O, K)
        packed = torch.empty(S.sbl_packed_bytes(O, K, 2, 4), dtype=torch.uint8, device="cuda:0")
        swr = torch.empty(O, dtype=torch.float32, device="cuda:0")
        op, oo = 0, 0
        for l in lins:
            nb = S.sbl_packed_bytes(l.O, l.K, 2, 4)
            S.sbl_quant_mask_weight(to_dev(W[l.name]), 2, 4, packed=packed[op:op + nb],
                                    sw_rows=swr[oo:oo + l.O])
            op += nb
            oo += l.O
        x = X[xn]
        y = S.sbl_linear_fwd(bf16_tensor(x), 2, 4, prepacked=packed, sw=swr, O=O)
        yh = host(y)
        oo = 0
        for l in lins:
            ref = o.linear_fwd(x, W[l.name], 2, 4)
            assert_bf16_exact(yh[:, oo:oo + l.O], ref["acc"], ref["sx"], ref["sw"])
            oo += l.O


def test_decode_large_k_falls_back(S):
    """16 tokens with K too long to stage in LDS take the tiled path."""
    T, O, K, N, M = 16, 40, 12288, 2, 4
    log_case("decode fallback", T, O, K)
    W, x = make_linear_inputs(T, O, K, seed=5)
    r = S.sbl_quant_mask_weight(to_dev(W), N, M)
    y = S.sbl_linear_fwd(bf16_tensor(x), N, M, prepacked=r["packed"], sw=r["gamma_sw"][1:],
                         O=O, out_dtype=torch.float32)
    assert_f32_close(host(y), o.linear_fwd(bf16_round(x), W, N, M)["y"])


@pytest.mark.parametrize("cfg", list(range(28)))
def test_gemm_every_tile_config(S, cfg, monkeypatch):
    """Each workgroup-tile configuration of the GEMM, forced, on ragged shapes."""
    monkeypatch.setenv("SBL_GEMM_TILE", str(cfg))
    for (N, M) in [(6, 8), (2, 4), (2, 8)]:
        for (T, O, K) in [(70, 300, 520), (300, 520, 1024), (17, 1000, 264), (200, 136, 1280),
                          (40, 260, 64)]:
            if K % M:
                continue
            log_case("gemm tile", cfg, N, M, T, O, K)
            _gemm_case(S, T, O, K, N, M, torch.bfloat16, seed=cfg * 7 + T + O, sw_per_row=True)

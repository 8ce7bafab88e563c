"""GPU parity of the Dual-STE backward (sbl_act_dequant, sbl_linear_bwd_dx,
sbl_linear_bwd_dw) against the oracle, through the C ABI.

x~ in bf16 is an integer-like stage (a rounding decision) and must match bit
for bit. The gradient products are fp32-accumulated contractions of exact
bf16 products, so the bound is derived from the arithmetic: with S the sum of
the |terms| of an output (computed by the oracle in fp64) and n the number of
terms, |gpu - exact| <= (n + 8) * 2^-24 * S (fp32 accumulation and the
scale), plus the output rounding (2^-23 |exact| for fp32, 2^-8 for bf16).
fp32 outputs must in addition stay within 1e-3 of max |exact|.
"""
import numpy as np
import pytest
import torch

import oracle as o
from sparse_linear_layers_bitlinear_amd.workloads import (
    WORKLOADS, bf16_round, make_linear_inputs, make_workload)
from gpu_helpers import bf16_tensor, f32_bits, host, log_case, to_dev

pytestmark = pytest.mark.gpu
F32 = np.float32


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from sparse_linear_layers_bitlinear_amd import sbl
    return sbl


def assert_grad_close(g, ref, abs_sum, n_terms, out_bf16):
    g = np.asarray(g, np.float64)
    acc = (n_terms + 8) * 2.0 ** -24 * np.asarray(abs_sum, np.float64)
    rnd = np.abs(ref) * (2.0 ** -8 if out_bf16 else 2.0 ** -23)
    err = np.abs(g - ref)
    bad = err > acc * 1.01 + rnd
    assert not bad.any(), (f"{int(bad.sum())} outputs beyond the bound; worst excess "
                           f"{float((err - acc - rnd).max())}")
    if not out_bf16:        # (one bf16 rounding alone can exceed 1e-3 relative)
        scale = max(float(np.abs(ref).max(initial=0.0)), 1e-30)
        assert float(err.max(initial=0.0)) / scale <= 1e-3


def _dy(rng, T, O):
    return bf16_round(rng.standard_normal((T, O)).astype(F32))


@pytest.mark.parametrize("T,K", [(1, 8), (37, 264), (300, 1536)])
def test_act_dequant_bit_exact(S, T, K):
    log_case("act_dequant", T, K)
    rng = np.random.default_rng(T + K)
    xq = rng.integers(-128, 128, size=(T, K)).astype(np.int8)
    xq[0, :2] = [-128, 127]
    sx = rng.uniform(1e-4, 1.0, T).astype(F32)
    sx[0] = F32(1 + 3 * 2 ** -8)                     # rounding ties in row 0 (q odd)
    xt = S.sbl_act_dequant(to_dev(xq), to_dev(sx))
    ref = o.act_dequant_bf16(xq, sx)
    assert np.array_equal(f32_bits(host(xt)), f32_bits(ref))


def _dx_case(S, T, O, K, N, M, out_bf16, seed, accumulate=False, nseg=1):
    """dX for nseg weight tensors of O rows each, concatenated (own sw each)."""
    rng = np.random.default_rng(seed)
    Ws = [make_linear_inputs(1, O, K, seed=seed + 10 * i)[0] for i in range(nseg)]
    preps = [S.sbl_quant_mask_weight(to_dev(W), N, M, want_sw_rows=True) for W in Ws]
    packed = torch.cat([p["packed"] for p in preps])
    swr = torch.cat([p["sw_rows"] for p in preps])
    refs = [o.quant_mask_weight(W, N, M) for W in Ws]
    w_eff = np.concatenate([r[0] for r in refs])
    sw = np.concatenate([np.full(O, r[3], np.float64) for r in refs])
    dy = _dy(rng, T, O * nseg)
    odt = torch.bfloat16 if out_bf16 else torch.float32
    dx0 = rng.standard_normal((T, K)).astype(F32)
    if out_bf16:
        dx0 = bf16_round(dx0)
    dx = to_dev(dx0).to(odt) if accumulate else None
    dx = S.sbl_linear_bwd_dx(bf16_tensor(dy), packed, swr, K, N, M, seg_rows=[O] * nseg,
                             out_dtype=odt, dx=dx, accumulate=accumulate)
    ref = o.linear_bwd_dx(dy, w_eff, sw)
    abs_sum = o.linear_bwd_dx(np.abs(dy), np.abs(w_eff), sw)
    if accumulate:
        ref = ref + dx0
        abs_sum = abs_sum + np.abs(dx0)
    assert_grad_close(host(dx), ref, abs_sum, O * nseg, out_bf16)


@pytest.mark.parametrize("N,M", [(6, 8), (2, 4), (1, 4), (8, 8), (3, 8), (7, 8), (2, 8)])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_bwd_dx_parity(S, N, M, out_bf16):
    for T, O, K in [(50, 136, 264), (130, 392, 520), (1, 8, 8)]:
        if K % M:
            continue
        log_case("bwd_dx", N, M, out_bf16, T, O, K)
        _dx_case(S, T, O, K, N, M, out_bf16, seed=T + O + N)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("N,M", [(6, 8), (2, 4)])
def test_bwd_dx_every_tile_config(S, cfg, N, M, monkeypatch):
    monkeypatch.setenv("SBL_BWD_TILE", str(cfg))
    monkeypatch.setenv("SBL_BWD_DMA", "0")                 # the register-staged kernel
    for T, O, K in [(200, 264, 392), (70, 520, 136)]:
        log_case("bwd_dx tile", cfg, N, M, T, O, K)
        _dx_case(S, T, O, K, N, M, False, seed=cfg + T)


@pytest.mark.parametrize("wide", ["0", "1"])
@pytest.mark.parametrize("N,M", [(6, 8), (2, 4), (2, 8)])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_bwd_dx_dma_kernel(S, wide, N, M, out_bf16, monkeypatch):
    """The single-tensor dX kernels with dY landed by LDS DMA, 128x128 and
    256x128 tiles: T tails (one row, past a tile), O tails (a last step of 8
    rows, steps past one round of the three- and four-stage rings), K tails
    (partial tile columns), and accumulation into dx."""
    monkeypatch.setenv("SBL_BWD_TILE", "0")
    monkeypatch.setenv("SBL_BWD_DX_DMA", "1")
    monkeypatch.setenv("SBL_BWD_DX_WIDE", wide)
    for T, O, K, acc in [(1, 8, 16, False), (33, 136, 264, False), (150, 264, 392, True),
                         (300, 392, 520, False), (257, 520, 136, False), (97, 40, 16, True)]:
        log_case("bwd_dx dma", wide, N, M, out_bf16, T, O, K, acc)
        _dx_case(S, T, O, K, N, M, out_bf16, seed=T + O + K + N, accumulate=acc)


@pytest.mark.parametrize("N,M", [(6, 8), (2, 4)])
def test_bwd_dx_segments_and_accumulate(S, N, M):
    """Two and three concatenated tensors with their own sw (gate+up style),
    with and without accumulation into dx."""
    for nseg, acc, odt in [(2, False, False), (3, True, False), (2, True, True)]:
        log_case("bwd_dx segments", N, M, nseg, acc, odt)
        _dx_case(S, 96, 136, 264, N, M, odt, seed=nseg * 11 + N, accumulate=acc, nseg=nseg)


def _dw_case(S, T, O, K, out_bf16, seed):
    rng = np.random.default_rng(seed)
    _, x = make_linear_inputs(T, 8, K, seed=seed)
    x = bf16_round(x)
    xq, sx = S.sbl_quant_act(bf16_tensor(x))
    xt = S.sbl_act_dequant(xq, sx)
    dy = _dy(rng, T, O)
    odt = torch.bfloat16 if out_bf16 else torch.float32
    dw = S.sbl_linear_bwd_dw(bf16_tensor(dy), xt, out_dtype=odt)
    oq, osx = o.quant_act(x)
    oxt = o.act_dequant_bf16(oq, osx)
    ref = o.linear_bwd_dw(dy, oxt)
    abs_sum = o.linear_bwd_dw(np.abs(dy), np.abs(oxt))
    assert_grad_close(host(dw), ref, abs_sum, T, out_bf16)


@pytest.mark.parametrize("out_bf16", [False, True])
def test_bwd_dw_parity(S, out_bf16):
    for T, O, K in [(77, 136, 264), (200, 392, 520), (1, 8, 8), (513, 64, 128)]:
        log_case("bwd_dw", out_bf16, T, O, K)
        _dw_case(S, T, O, K, out_bf16, seed=T + O)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_bwd_dw_every_tile_config(S, cfg, monkeypatch):
    monkeypatch.setenv("SBL_BWD_TILE", str(cfg))
    monkeypatch.setenv("SBL_BWD_DMA", "0")                 # the register-staged kernel
    for T, O, K in [(150, 264, 392), (64, 520, 136)]:
        log_case("bwd_dw tile", cfg, T, O, K)
        _dw_case(S, T, O, K, False, seed=cfg + T)


@pytest.mark.parametrize("wide", ["0", "1"])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_bwd_dw_dma_kernel(S, out_bf16, wide, monkeypatch):
    """The dW kernels with direct-to-LDS loads, 128x128 and 256x128 tiles:
    T tails of every size class (one row, one past a step, many steps, past
    one round of the three- and four-stage rings), tiles smaller than O and
    K (clamped edge loads), several tile-order groups."""
    monkeypatch.setenv("SBL_BWD_TILE", "0")
    monkeypatch.setenv("SBL_BWD_DW_WIDE", wide)
    for T, O, K, grp in [(1, 8, 8, 1), (33, 136, 264, 1), (150, 264, 392, 3), (97, 8, 16, 1),
                         (300, 392, 520, 2), (256, 128, 128, 1), (65, 520, 136, 1),
                         (160, 776, 264, 2)]:
        monkeypatch.setenv("SBL_BWD_GROUP", str(grp))
        log_case("bwd_dw dma", out_bf16, wide, T, O, K, grp)
        _dw_case(S, T, O, K, out_bf16, seed=T + O + K)


@pytest.mark.parametrize("group", [1, 3, 7, 64])
def test_bwd_tile_order_groups(S, group, monkeypatch):
    """The grouped tile order forced to several group sizes (ragged last
    groups included): every tile is computed exactly once."""
    monkeypatch.setenv("SBL_BWD_GROUP", str(group))
    log_case("bwd tile order", group)
    _dx_case(S, 300, 264, 520, 6, 8, False, seed=group)
    _dx_case(S, 130, 392, 264, 2, 4, False, seed=group + 1)
    _dw_case(S, 150, 520, 392, False, seed=group + 2)


@pytest.mark.parametrize("N,M", [(6, 8), (2, 4), (8, 8)])
@pytest.mark.parametrize("cfg", [0, 2])
def test_bwd_dw_mask_gated(S, N, M, cfg, monkeypatch):
    """The gated-gradient ablation: dW with the weight preparation's keep bits
    equals the oracle's M (.) dW (M from the oracle's own mask), and is the
    dense dW exactly wherever the mask keeps the weight."""
    monkeypatch.setenv("SBL_BWD_TILE", str(cfg))
    rng = np.random.default_rng(N + cfg)
    for T, O, K in [(150, 264, 392), (33, 136, 264)]:
        if K % M:
            continue
        log_case("bwd_dw gated", N, M, cfg, T, O, K)
        W, x = make_linear_inputs(T, O, K, seed=T + N)
        x = bf16_round(x)
        prep = S.sbl_quant_mask_weight_batch([{"w": to_dev(W), "want_mask_bits": True}], N, M)[0]
        xq, sx = S.sbl_quant_act(bf16_tensor(x))
        xt = S.sbl_act_dequant(xq, sx)
        dy = _dy(rng, T, O)
        dyt = bf16_tensor(dy)
        gated = host(S.sbl_linear_bwd_dw(dyt, xt, keep_bits=prep["mask_bits"]))
        dense = host(S.sbl_linear_bwd_dw(dyt, xt))
        mask = o.nm_mask(W, N, M)
        assert np.array_equal(gated, np.where(mask == 1, dense, 0.0).astype(np.float32))
        oxt = o.act_dequant_bf16(*o.quant_act(x))
        ref = o.linear_bwd_dw(dy, oxt, mask=mask)
        abs_sum = o.linear_bwd_dw(np.abs(dy), np.abs(oxt), mask=mask)
        assert_grad_close(gated, ref, abs_sum, T, False)


def test_bwd_empty_and_zero_tokens(S):
    """T = 0: dW is all zeros (an empty sum); dX is left as it is."""
    log_case("bwd empty")
    dev = torch.device("cuda:0")
    dw = torch.full((16, 24), 7.0, device=dev)
    S.lib.sbl_linear_bwd_dw(None, 16, None, 0, 16, 24, None, S._ptr(dw), S.SBL_FP32, None)
    assert np.array_equal(host(dw), np.zeros((16, 24), F32))
    dx = torch.full((0, 24), 1.0, device=dev)
    dy = torch.zeros((0, 16), dtype=torch.bfloat16, device=dev)
    W, _ = make_linear_inputs(1, 16, 24, seed=1)
    p = S.sbl_quant_mask_weight(to_dev(W), 6, 8, want_sw_rows=True)
    S.sbl_linear_bwd_dx(dy, p["packed"], p["sw_rows"], 24, 6, 8, out_dtype=torch.float32, dx=dx)


def test_bwd_full_size_sampled(S):
    """The Qwen2.5-1.5B training-step shapes (T = 4096, 2:4): dX of the up
    projection (8960 x 1536, reduction over 8960) and dW of the down
    projection (1536 x 8960, reduction over 4096), in the launch
    configuration the benchmark uses, checked on sampled rows."""
    wl = WORKLOADS["qwen15b_ffn"]
    W, X = make_workload("qwen15b_ffn")
    rng = np.random.default_rng(5)
    up = next(l for l in wl.linears if l.name == "up")
    down = next(l for l in wl.linears if l.name == "down")
    log_case("bwd full dx", up.O, up.K, wl.T)
    p = S.sbl_quant_mask_weight(to_dev(W["up"]), wl.N, wl.M, want_sw_rows=True)
    dy = _dy(rng, wl.T, up.O)
    dx = S.sbl_linear_bwd_dx(bf16_tensor(dy), p["packed"], p["sw_rows"], up.K, wl.N, wl.M,
                             out_dtype=torch.bfloat16)
    w_eff, _, _, sw = o.quant_mask_weight(W["up"], wl.N, wl.M)
    rows = rng.choice(wl.T, 48, replace=False)
    ref = o.linear_bwd_dx(dy[rows], w_eff, sw)
    abs_sum = o.linear_bwd_dx(np.abs(dy[rows]), np.abs(w_eff), sw)
    assert_grad_close(host(dx)[rows], ref, abs_sum, up.O, True)
    log_case("bwd full dw", down.O, down.K, wl.T)
    x = bf16_round(X[down.x_name])
    xq, sx = S.sbl_quant_act(bf16_tensor(x))
    xt = S.sbl_act_dequant(xq, sx)
    dy2 = _dy(rng, wl.T, down.O)
    dw = S.sbl_linear_bwd_dw(bf16_tensor(dy2), xt)
    oq, osx = o.quant_act(x)
    oxt = o.act_dequant_bf16(oq, osx)
    assert np.array_equal(f32_bits(host(xt)), f32_bits(oxt))
    orow = rng.choice(down.O, 48, replace=False)
    ref = o.linear_bwd_dw(dy2[:, orow], oxt)
    abs_sum = o.linear_bwd_dw(np.abs(dy2[:, orow]), np.abs(oxt))
    assert_grad_close(host(dw)[orow], ref, abs_sum, wl.T, False)


def test_bwd_dx_dma_full_size_sampled(S):
    """dX of a Qwen2.5-3B-shaped up projection (T = 8192 tokens, 11008 x
    2048 weights, 6:8), the shape class that takes the LDS-DMA dX kernel
    with 256-row tiles, in the launch configuration chosen for it; checked on
    sampled rows."""
    T, O, K, N, M = 8192, 11008, 2048, 6, 8
    rng = np.random.default_rng(17)
    W, _ = make_linear_inputs(1, O, K, seed=17)
    log_case("bwd full dx dma", T, O, K)
    p = S.sbl_quant_mask_weight(to_dev(W), N, M, want_sw_rows=True)
    dy = _dy(rng, T, O)
    dx = S.sbl_linear_bwd_dx(bf16_tensor(dy), p["packed"], p["sw_rows"], K, N, M,
                             out_dtype=torch.float32)
    w_eff, _, _, sw = o.quant_mask_weight(W, N, M)
    rows = rng.choice(T, 48, replace=False)
    ref = o.linear_bwd_dx(dy[rows], w_eff, sw)
    abs_sum = o.linear_bwd_dx(np.abs(dy[rows]), np.abs(w_eff), sw)
    assert_grad_close(host(dx)[rows], ref, abs_sum, O, False)


@pytest.mark.parametrize("wl_name", ["qwen05b_ffn", "qwen15b_ffn"])
def test_bwd_bench_launches(S, wl_name):
    """The backward calls the training-step benchmark times, as it makes them:
    per input, x~ from sbl_act_dequant, one sbl_linear_bwd_dx over the group's
    tensors concatenated along O (gate|up: two segments with their own sw)
    into a preallocated bf16 dx, and one sbl_linear_bwd_dw of the group's dY
    against x~ into a preallocated fp32 dW. Sampled rows against the oracle,
    the segments' products summed in fp64."""
    wl = WORKLOADS[wl_name]
    N, M, T = wl.N, wl.M, wl.T
    W, X = make_workload(wl_name)
    rng = np.random.default_rng(23)
    dev = torch.device("cuda:0")
    groups = {}
    for lin in wl.linears:
        groups.setdefault(lin.x_name, []).append(lin)
    for xn, lins in groups.items():
        K = dict(wl.x_specs)[xn]
        O = sum(l.O for l in lins)
        log_case("bwd bench launch", wl_name, "+".join(l.name for l in lins), T, O, K)
        packed = torch.empty(S.sbl_packed_bytes(O, K, N, M), dtype=torch.uint8, device=dev)
        swr = torch.empty(O, dtype=torch.float32, device=dev)
        op, oo = 0, 0
        for l in lins:
            nb = S.sbl_packed_bytes(l.O, l.K, N, M)
            S.sbl_quant_mask_weight(to_dev(W[l.name]), N, M, packed=packed[op:op + nb],
                                    sw_rows=swr[oo:oo + l.O])
            op += nb
            oo += l.O
        x = X[xn]
        xq, sx = S.sbl_quant_act(bf16_tensor(x))
        xt = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
        S.sbl_act_dequant(xq, sx, xt=xt)
        dy = _dy(rng, T, O)
        dx = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((O, K), dtype=torch.float32, device=dev)
        S.sbl_linear_bwd_dx(bf16_tensor(dy), packed, swr, K, N, M, seg_rows=[l.O for l in lins],
                            dx=dx)
        S.sbl_linear_bwd_dw(bf16_tensor(dy), xt, dw=dw)
        oq, osx = o.quant_act(x)
        oxt = o.act_dequant_bf16(oq, osx)
        assert np.array_equal(f32_bits(host(xt)), f32_bits(oxt))
        rows = rng.choice(T, 32, replace=False)
        ref = np.zeros((len(rows), K))
        abs_sum = np.zeros((len(rows), K))
        oo = 0
        for l in lins:
            w_eff, _, _, sw = o.quant_mask_weight(W[l.name], N, M)
            d = dy[rows][:, oo:oo + l.O]
            ref += o.linear_bwd_dx(d, w_eff, sw)
            abs_sum += o.linear_bwd_dx(np.abs(d), np.abs(w_eff), sw)
            oo += l.O
        assert_grad_close(host(dx)[rows], ref, abs_sum, O, True)
        orow = rng.choice(O, 48, replace=False)
        ref = o.linear_bwd_dw(dy[:, orow], oxt)
        abs_sum = o.linear_bwd_dw(np.abs(dy[:, orow]), np.abs(oxt))
        assert_grad_close(host(dw)[orow], ref, abs_sum, T, False)

"""HIP-graph capture of the library calls: every replay must equal the eager
result (the bench times graph replays). The library records no memset nodes;
this checks replays after the first, with eager work and input changes in
between."""
import numpy as np
import pytest
import torch

import oracle as o
from sparse_linear_layers_bitlinear_amd.workloads import make_linear_inputs
from gpu_helpers import bf16_tensor, host, log_case, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from sparse_linear_layers_bitlinear_amd import sbl
    return sbl


@pytest.mark.parametrize("N,M,T,O,K", [(6, 8, 64, 256, 512), (2, 4, 48, 384, 640),
                                       (2, 4, 4, 512, 1024)])
def test_graph_replays_match_eager(S, N, M, T, O, K):
    log_case("graph replay", N, M, T, O, K)
    dev = torch.device("cuda:0")
    xs, Ws = [], []
    for i in range(4):
        W, x = make_linear_inputs(T, O, K, seed=100 + i)
        xs.append(x)
        Ws.append(W)
    x_in = bf16_tensor(xs[0]).clone()
    w_in = to_dev(Ws[0]).clone()
    xq = torch.empty((T, K), dtype=torch.int8, device=dev)
    sx = torch.empty(T, dtype=torch.float32, device=dev)
    packed = torch.empty(S.sbl_packed_bytes(O, K, N, M), dtype=torch.uint8, device=dev)
    swr = torch.empty(O, dtype=torch.float32, device=dev)
    ws = torch.empty(S.sbl_quant_mask_weight_workspace(O, K), dtype=torch.uint8, device=dev)
    y = torch.empty((T, O), dtype=torch.float32, device=dev)

    def step():
        S.sbl_quant_act(x_in, xq=xq, sx=sx)
        S.sbl_quant_mask_weight(w_in, N, M, packed=packed, sw_rows=swr, ws=ws)
        S.sbl_gemm(xq, sx, packed, swr, O, N, M, out_dtype=torch.float32, y=y)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in [1, 2, 3, 0, 2]:
        x_in.copy_(bf16_tensor(xs[i]))
        w_in.copy_(to_dev(Ws[i]))
        g.replay()
        y_graph = host(y).copy()
        packed_graph = host(packed).copy()
        step()                                  # eager, same inputs
        assert np.array_equal(host(y), y_graph)
        assert np.array_equal(host(packed), packed_graph)
        ref = o.linear_fwd(xs[i], Ws[i], N, M)
        assert np.array_equal(packed_graph.reshape(O, -1), o.pack(ref["w_eff"], ref["mask"], N, M))
        _ = torch.zeros(1000, device=dev).sum()  # unrelated eager work between replays


def test_graph_multistream_matches_eager(S):
    """Weight preparation of two projections on two side streams, forked from
    and joined back into the capturing stream (the schedule the benchmark
    times); every replay equals the eager sequential result."""
    log_case("graph multistream", 6, 8, 96, 320, 512)
    dev = torch.device("cuda:0")
    N, M, T, K = 6, 8, 96, 512
    Os = [320, 192]
    Wa, x = make_linear_inputs(T, Os[0], K, seed=7)
    Wb, _ = make_linear_inputs(T, Os[1], K, seed=8)
    Ws = [to_dev(Wa), to_dev(Wb)]
    x_in = bf16_tensor(x).clone()
    O = sum(Os)
    nb = [S.sbl_packed_bytes(o, K, N, M) for o in Os]
    xq = torch.empty((T, K), dtype=torch.int8, device=dev)
    sx = torch.empty(T, dtype=torch.float32, device=dev)
    packed = torch.empty(sum(nb), dtype=torch.uint8, device=dev)
    swr = torch.empty(O, dtype=torch.float32, device=dev)
    wss = [torch.empty(S.sbl_quant_mask_weight_workspace(o, K), dtype=torch.uint8, device=dev)
           for o in Os]
    y = torch.empty((T, O), dtype=torch.float32, device=dev)
    sides = [torch.cuda.Stream(), torch.cuda.Stream()]

    def prep(i):
        off_p, off_o = sum(nb[:i]), sum(Os[:i])
        S.sbl_quant_mask_weight(Ws[i], N, M, packed=packed[off_p:off_p + nb[i]],
                                sw_rows=swr[off_o:off_o + Os[i]], ws=wss[i])

    def step():
        main = torch.cuda.current_stream()
        for i, side in enumerate(sides):
            side.wait_stream(main)
            with torch.cuda.stream(side):
                prep(i)
        S.sbl_quant_act(x_in, xq=xq, sx=sx)
        for side in sides:
            main.wait_stream(side)
        S.sbl_gemm(xq, sx, packed, swr, O, N, M, out_dtype=torch.float32, y=y)

    def eager_sequential():
        prep(0)
        prep(1)
        S.sbl_quant_act(x_in, xq=xq, sx=sx)
        S.sbl_gemm(xq, sx, packed, swr, O, N, M, out_dtype=torch.float32, y=y)
        torch.cuda.synchronize()
        return host(y).copy(), host(packed).copy()

    y_ref, p_ref = eager_sequential()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        y.zero_()
        packed.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), y_ref)
        assert np.array_equal(host(packed), p_ref)
        _ = torch.zeros(1000, device=dev).sum()
    for i, Wi in enumerate([Wa, Wb]):
        r = o.quant_mask_weight(Wi, N, M)
        off_p = sum(nb[:i])
        assert np.array_equal(p_ref[off_p:off_p + nb[i]].reshape(Os[i], -1),
                              o.pack(r[0], r[1], N, M))


def test_graph_backward_replays_match_eager(S):
    """The backward calls (x~, dX over two segments, dW) captured in a graph:
    every replay, with new inputs and eager work in between, equals the eager
    result bit for bit."""
    log_case("graph backward", 6, 8, 96, 2 * 136, 264)
    dev = torch.device("cuda:0")
    N, M, T, O, K = 6, 8, 96, 136, 264
    rng = np.random.default_rng(3)
    Ws = [to_dev(make_linear_inputs(1, O, K, seed=50 + i)[0]) for i in range(2)]
    preps = [S.sbl_quant_mask_weight(w, N, M, want_sw_rows=True) for w in Ws]
    packed = torch.cat([p["packed"] for p in preps])
    swr = torch.cat([p["sw_rows"] for p in preps])
    xs = [bf16_tensor(make_linear_inputs(T, 8, K, seed=60 + i)[1]) for i in range(3)]
    dys = [bf16_tensor(rng.standard_normal((T, 2 * O)).astype(np.float32)) for _ in range(3)]
    x_in, dy_in = xs[0].clone(), dys[0].clone()
    xq = torch.empty((T, K), dtype=torch.int8, device=dev)
    sx = torch.empty(T, dtype=torch.float32, device=dev)
    xt = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((2 * O, K), dtype=torch.float32, device=dev)

    def step():
        S.sbl_quant_act(x_in, xq=xq, sx=sx)
        S.sbl_act_dequant(xq, sx, xt=xt)
        S.sbl_linear_bwd_dx(dy_in, packed, swr, K, N, M, seg_rows=[O, O], dx=dx)
        S.sbl_linear_bwd_dw(dy_in, xt, dw=dw)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in [1, 2, 0, 2]:
        x_in.copy_(xs[i])
        dy_in.copy_(dys[i])
        g.replay()
        got = [host(t).copy() for t in (xt, dx, dw)]
        step()                                   # eager, same inputs
        for a, t in zip(got, (xt, dx, dw)):
            assert np.array_equal(a, host(t))
        _ = torch.zeros(1000, device=dev).sum()  # unrelated eager work between replays

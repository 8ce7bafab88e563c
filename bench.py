"""Throughput of the Sparse-BitLinear forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--nm N:M]
                    [--decode-T T] [--layers L] [--no-cpu-baseline] [--eager]

A step is one pass of the whole forward hot path over one batch:
  prefill workloads (Qwen2.5-shaped FFN, mask recomputed every call):
    per-token int8 quantization of each FFN input, absmean + N:M mask +
    RoundClip + pack of every master weight, the int8 x ternary GEMMs with
    dequant epilogue (gate and up fused into one GEMM over concatenated rows);
    all projections' weights are prepared by one batched call;
  decode workload (BitNet-2B4T-shaped layer, prepacked 2:4 weights): for each
    of L distinct layer copies, the q|k|v, o, gate|up and down projections of
    T bf16 tokens, each one sbl_linear_fwd call (per-token int8 quantization
    inside the GEMV).
The step is captured once into a HIP graph and replayed (the library launches
stay the same kernels; the graph only removes Python/ctypes launch cost).
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from sparse_linear_layers_bitlinear_amd import sbl  # noqa: E402
from sparse_linear_layers_bitlinear_amd.workloads import (  # noqa: E402
    WORKLOADS, bf16_round, make_workload)

# MI355X published peaks
PEAK_INT8_DENSE_TOPS = 5000.0     # dense int8 MFMA, TOPS
PEAK_HBM_GBS = 8000.0             # HBM3E, GB/s
PEAK_BF16_DENSE_TFLOPS = 2500.0   # dense bf16 MFMA, TFLOP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="qwen3b_sweep",
                   choices=["qwen05b_ffn", "qwen15b_ffn", "qwen3b_sweep", "bitnet_decode", "tiny"])
    p.add_argument("--nm", default=None, help="override N:M, e.g. 2:8")
    p.add_argument("--decode-T", type=int, default=8)
    p.add_argument("--layers", type=int, default=30)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--eager", action="store_true", help="time eager launches instead of a graph")
    p.add_argument("--fused-norm", action="store_true",
                   help="prefill: quantize each FFN input as Q_a(RMSNorm(x) * g) in one pass "
                        "(sbl_rmsnorm_quant_act) instead of Q_a(x)")
    p.add_argument("--mask-from-ternary", action="store_true",
                   help="prefill: the ablated recipe, mask ranked on the ternary codes")
    p.add_argument("--backward", action="store_true",
                   help="prefill: the step adds the Dual-STE backward of every projection (x~ in "
                        "bf16, dX and dW on the bf16 matrix cores) to the forward: a training step")
    p.add_argument("--overlap-backward", action="store_true",
                   help="with --backward: each group's dW on a second stream beside its dX "
                        "(default: every call on one stream)")
    p.add_argument("--mask-gated-grad", action="store_true",
                   help="with --backward: the ablated estimator, dW gated by the mask (the weight "
                        "preparation also writes the keep bits)")
    p.add_argument("--mask-then-quant", action="store_true",
                   help="prefill: the composition-order ablation, gamma over the kept weights only")
    p.add_argument("--diagnostics", action="store_true",
                   help="prefill: the weight preparation also emits the mask diagnostics (keep bits, "
                        "flips against the previous step's mask, per-group pruning threshold)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    return p.parse_args()


# ---------------------------------------------------------------- prefill --
class PrefillStep:
    def __init__(self, wl_name, N, M, diagnostics=False, fused_norm=False, variant=0,
                 backward=False, gated=False, overlap_backward=False):
        wl = WORKLOADS[wl_name]
        self.wl, self.N, self.M, self.diag, self.norm = wl, N, M, diagnostics, fused_norm
        self.bwd, self.gated = backward, gated and backward
        # with overlap_backward: dW on a second stream (default priority), beside dX
        self.side = torch.cuda.Stream() if backward and overlap_backward else None
        W, X = make_workload(wl_name)
        dev = torch.device("cuda:0")
        self.T = wl.T
        self.x = {k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in X.items()}
        self.W = {k: torch.from_numpy(v).to(dev) for k, v in W.items()}
        self.K_of = dict(wl.x_specs)
        self.xq = {k: torch.empty((self.T, K), dtype=torch.int8, device=dev)
                   for k, K in self.K_of.items()}
        self.sx = {k: torch.empty(self.T, dtype=torch.float32, device=dev) for k in self.K_of}
        # RMSNorm gains for the fused-norm variant (seeded, 1 + 0.1 N(0,1))
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        self.gain = {k: 1 + 0.1 * torch.randn(K, generator=gen, device=dev)
                     for k, K in self.K_of.items()}
        # group projections that share an input into one GEMM over concatenated rows
        self.groups = {}
        for lin in wl.linears:
            self.groups.setdefault(lin.x_name, []).append(lin)
        self.packed, self.swr, self.y = {}, {}, {}
        for xn, lins in self.groups.items():
            K = self.K_of[xn]
            O = sum(l.O for l in lins)
            self.packed[xn] = torch.empty(sbl.sbl_packed_bytes(O, K, N, M), dtype=torch.uint8,
                                          device=dev)
            self.swr[xn] = torch.empty(O, dtype=torch.float32, device=dev)
            self.y[xn] = torch.empty((self.T, O), dtype=torch.bfloat16, device=dev)
        # all projections' weights are prepared by one batched call
        self.ws = torch.empty(sbl.sbl_quant_mask_weight_batch_workspace(len(wl.linears)),
                              dtype=torch.uint8, device=dev)
        self.prep_items = []
        for xn, lins in self.groups.items():
            off_p, off_o = 0, 0
            for l in lins:
                nb = sbl.sbl_packed_bytes(l.O, l.K, N, M)
                self.prep_items.append({
                    "w": self.W[l.name], "packed": self.packed[xn][off_p:off_p + nb],
                    "sw_rows": self.swr[xn][off_o:off_o + l.O],
                    "gamma_sw": torch.empty(2, dtype=torch.float32, device=dev),
                    "variant": variant})
                off_p += nb
                off_o += l.O
        if diagnostics:
            # the previous step's mask: the same preparation on slightly moved weights
            prev = [dict(it, w=(it["w"] * 1.001 + 1e-4).contiguous(), want_mask_bits=True)
                    for it in self.prep_items]
            prev = sbl.sbl_quant_mask_weight_batch(prev, N, M, ws=self.ws)
            for it, pv in zip(self.prep_items, prev):
                O, K = it["w"].shape
                it["prev_mask_bits"] = pv["mask_bits"]
                it["mask_bits"] = torch.empty_like(pv["mask_bits"])
                it["flips"] = torch.empty(1, dtype=torch.int64, device=dev)
                it["group_thr"] = torch.empty((O, K // M), dtype=torch.float32, device=dev)
            torch.cuda.synchronize()
        self.ops = sum(2.0 * self.T * l.O * l.K for l in wl.linears)
        if backward:
            # upstream gradient of each group's output (seeded bf16 N(0,1)), x~, dX and dW
            self.dy, self.xt, self.dx, self.dw = {}, {}, {}, {}
            for xn, lins in self.groups.items():
                K, O = self.K_of[xn], sum(l.O for l in lins)
                self.dy[xn] = torch.randn((self.T, O), generator=gen, device=dev).to(torch.bfloat16)
                self.xt[xn] = torch.empty((self.T, K), dtype=torch.bfloat16, device=dev)
                self.dx[xn] = torch.empty((self.T, K), dtype=torch.bfloat16, device=dev)
                self.dw[xn] = torch.empty((O, K), dtype=torch.float32, device=dev)
            self.ops *= 3.0       # forward + dX + dW, each 2 T O K per projection
            self.keep = {}
            if self.gated:
                # the preparation writes each weight's keep bits into its group's buffer
                items = iter(self.prep_items)
                for xn, lins in self.groups.items():
                    C = -(-self.K_of[xn] // 128) * 4
                    self.keep[xn] = torch.empty((sum(l.O for l in lins), C), dtype=torch.int32,
                                                device=dev)
                    off = 0
                    for l in lins:
                        next(items)["mask_bits"] = self.keep[xn][off:off + l.O]
                        off += l.O

    def calls(self):
        """The step as an ordered list of (name, launch) pairs."""
        N, M = self.N, self.M
        out = []
        for xn in self.groups:
            if self.norm:
                out.append((f"quant_act[{xn}]", lambda xn=xn: sbl.sbl_rmsnorm_quant_act(
                    self.x[xn], self.gain[xn], xq=self.xq[xn], sx=self.sx[xn])))
            else:
                out.append((f"quant_act[{xn}]", lambda xn=xn: sbl.sbl_quant_act(
                    self.x[xn], xq=self.xq[xn], sx=self.sx[xn])))
        out.append((f"quant_mask_weight[{'+'.join(l.name for l in self.wl.linears)}]",
                    lambda: sbl.sbl_quant_mask_weight_batch(self.prep_items, N, M, ws=self.ws)))
        for xn, lins in self.groups.items():
            O = sum(l.O for l in lins)
            out.append((f"gemm[{'+'.join(l.name for l in lins)}]",
                        lambda xn=xn, O=O: sbl.sbl_gemm(self.xq[xn], self.sx[xn], self.packed[xn],
                                                        self.swr[xn], O, N, M, y=self.y[xn])))
        if self.bwd:
            for xn, lins in reversed(list(self.groups.items())):
                K, tag = self.K_of[xn], '+'.join(l.name for l in lins)
                out.append((f"act_dequant[{xn}]", lambda xn=xn: sbl.sbl_act_dequant(
                    self.xq[xn], self.sx[xn], xt=self.xt[xn])))
                out.append((f"bwd_dx[{tag}]", lambda xn=xn, K=K, lins=lins: sbl.sbl_linear_bwd_dx(
                    self.dy[xn], self.packed[xn], self.swr[xn], K, N, M,
                    seg_rows=[l.O for l in lins], dx=self.dx[xn])))
                out.append((f"bwd_dw[{tag}]", lambda xn=xn: sbl.sbl_linear_bwd_dw(
                    self.dy[xn], self.xt[xn], dw=self.dw[xn], keep_bits=self.keep.get(xn))))
        return out

    cold_weights = True    # each replay starts from a flushed last-level cache

    def run(self):
        """One step: act quant of the FFN input, one batched preparation of every
        weight, the grouped GEMMs in order (a later group's input, e.g. the down
        projection's, would come from the earlier GEMM in a real FFN)."""
        calls = self.calls()
        order = [c for c in calls if c[0].startswith("quant_mask_weight")]
        for xn in self.groups:
            order += [c for c in calls if c[0] in (f"quant_act[{xn}]",) or
                      (c[0].startswith("gemm[") and c[0] == self._gemm_name(xn))]
        if self.side is None:
            order += [c for c in calls if c[0].split("[")[0] in ("act_dequant", "bwd_dx", "bwd_dw")]
            run_all(order)
            return
        run_all(order)
        self._backward_two_streams(dict(calls))

    def _backward_two_streams(self, f):
        """The backward with each projection group's dW beside its dX: the
        launch stream runs the groups' dX in reverse order (a group's upstream
        gradient comes from the dX of the group after it, through the FFN's
        activation), a second stream the x~ of every group and the dW of each
        group once that group's upstream gradient exists (for all but the last
        group: once the dX before it has run). The streams join at the end."""
        main, side = torch.cuda.current_stream(), self.side
        groups = list(reversed(list(self.groups.items())))
        side.wait_stream(main)                       # after the forward
        with torch.cuda.stream(side):
            for xn, _ in groups:
                f[f"act_dequant[{xn}]"]()
        for gi, (xn, lins) in enumerate(groups):
            tag = '+'.join(l.name for l in lins)
            if gi > 0:
                side.wait_stream(main)               # the previous group's dX has run
            with torch.cuda.stream(side):
                f[f"bwd_dw[{tag}]"]()
            f[f"bwd_dx[{tag}]"]()
        main.wait_stream(side)

    def _gemm_name(self, xn):
        return f"gemm[{'+'.join(l.name for l in self.groups[xn])}]"

    def call_info(self, name):
        """(bound, algorithmic units per launch, unit) of a named call."""
        T = self.T
        if name.startswith("bwd_"):
            tag = name[name.index("[") + 1:-1]
            ops = sum(2.0 * T * l.O * l.K for l in self.wl.linears if l.name in tag.split("+"))
            return "mfma_bf16", ops, "flops"
        if name.startswith("act_dequant["):
            K = self.K_of[name[12:-1]]
            return "hbm", 3.0 * T * K + 4.0 * T, "bytes"
        if name.startswith("gemm["):
            xn = [k for k, ls in self.groups.items()
                  if name == f"gemm[{'+'.join(l.name for l in ls)}]"][0]
            ops = sum(2.0 * T * l.O * l.K for l in self.groups[xn])
            return "mfma", ops, "ops"
        if name.startswith("quant_act["):
            K = self.K_of[name[10:-1]]
            return "hbm", 2.0 * T * K + T * K + 4.0 * T + (4.0 * K if self.norm else 0.0), "bytes"
        # weight preparation: W read twice (absmean pass, mask/code pass), packed written;
        # with diagnostics also the keep bits written, the previous ones read, the thresholds
        diag = sum(2.0 * 4 * l.O * (-(-l.K // 128) * 4) + 4.0 * l.O * l.K / self.M
                   for l in self.wl.linears) if self.diag else (
            sum(4.0 * l.O * (-(-l.K // 128) * 4) for l in self.wl.linears) if self.gated else 0.0)
        return "hbm", diag + sum(2.0 * l.O * l.K * self.W[l.name].element_size() +
                                 sbl.sbl_packed_bytes(l.O, l.K, self.N, self.M)
                                 for l in self.wl.linears), "bytes"


# ----------------------------------------------------------------- decode --
class DecodeStep:
    def __init__(self, T, L):
        wl = WORKLOADS["bitnet_decode"]
        self.wl, self.N, self.M, self.T, self.L = wl, 2, 4, T, L
        dev = torch.device("cuda:0")
        W, X = make_workload("bitnet_decode", T=T)
        self.x = {k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in X.items()}
        self.K_of = dict(wl.x_specs)
        self.groups = {}
        for lin in wl.linears:
            self.groups.setdefault(lin.x_name, []).append(lin)
        # L distinct prepacked copies: copy 0 from the seeded workload weights, copies
        # l > 0 from seeded torch draws of the same distribution (not timed)
        g = torch.Generator(device=dev)
        self.packed, self.swr = [], []
        ws = torch.empty(sbl.sbl_quant_mask_weight_workspace(6912, 2560), dtype=torch.uint8,
                         device=dev)
        for li in range(L):
            g.manual_seed(1000 + li)
            pk, sr = {}, {}
            for xn, lins in self.groups.items():
                K = self.K_of[xn]
                O = sum(l.O for l in lins)
                pk[xn] = torch.empty(sbl.sbl_packed_bytes(O, K, 2, 4), dtype=torch.uint8,
                                     device=dev)
                sr[xn] = torch.empty(O, dtype=torch.float32, device=dev)
                op, oo = 0, 0
                for l in lins:
                    if li == 0:
                        w = torch.from_numpy(W[l.name]).to(dev)
                    else:
                        w = torch.randn((l.O, l.K), generator=g, device=dev) * 0.02
                    nb = sbl.sbl_packed_bytes(l.O, l.K, 2, 4)
                    sbl.sbl_quant_mask_weight(w, 2, 4, packed=pk[xn][op:op + nb],
                                              sw_rows=sr[xn][oo:oo + l.O], ws=ws)
                    op += nb
                    oo += l.O
            self.packed.append(pk)
            self.swr.append(sr)
        torch.cuda.synchronize()
        self.y = {xn: torch.empty((T, sum(l.O for l in ls)), dtype=torch.bfloat16, device=dev)
                  for xn, ls in self.groups.items()}
        self.ws = {xn: torch.empty(max(1, sbl.sbl_linear_fwd_workspace(
            T, sum(l.O for l in ls), self.K_of[xn], 2, 4, True)), dtype=torch.uint8, device=dev)
            for xn, ls in self.groups.items()}
        self.weights = sum(l.O * l.K for l in wl.linears)
        self.bytes_layer = sum(self.call_bytes(xn) for xn in self.groups)
        self.ops = 2.0 * T * self.weights * L

    def call_bytes(self, xn):
        """Algorithmic HBM bytes of one projection group: packed W, bf16 x,
        per-row weight scales and the bf16 output."""
        T = self.T
        K = self.K_of[xn]
        O = sum(l.O for l in self.groups[xn])
        return sbl.sbl_packed_bytes(O, K, 2, 4) + 2 * T * K + 4 * O + 2 * T * O

    def calls(self):
        """Per layer and projection group one sbl_linear_fwd on the prepacked
        weights (the activation quantization runs inside the GEMV)."""
        out = []
        for li in range(self.L):
            for xn in self.groups:
                O = sum(l.O for l in self.groups[xn])
                out.append((f"linear[{'+'.join(l.name for l in self.groups[xn])}]",
                            lambda xn=xn, O=O, li=li: sbl.sbl_linear_fwd(
                                self.x[xn], 2, 4, prepacked=self.packed[li][xn],
                                sw=self.swr[li][xn], O=O, y=self.y[xn], ws=self.ws[xn])))
        return out

    cold_weights = True    # 30 layers of packed weights exceed the last-level cache

    def run(self):
        """One step: the layers' calls in order (each depends on the previous
        one in a real decoder)."""
        run_all(self.calls())

    def call_info(self, name):
        xn = [k for k, ls in self.groups.items()
              if name == f"linear[{'+'.join(l.name for l in ls)}]"][0]
        return "hbm", float(self.call_bytes(xn)), "bytes"


# ------------------------------------------------------------------ timing --
def run_all(calls):
    for _, f in calls:
        f()


def capture(fn):
    """Capture fn's launches into a HIP graph (after one eager warm-up run on a
    side stream, as graph capture requires)."""
    stream = torch.cuda.current_stream()
    s = torch.cuda.Stream()
    s.wait_stream(stream)
    with torch.cuda.stream(s):
        fn()
    stream.wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


FLUSH_BYTES = 1 << 30     # > the 256 MB last-level cache (MALL) and the L2s


class CacheFlush:
    """Evicts every cache level by reading 1 GiB (a sum over a buffer written
    once at set-up). A read leaves only clean lines behind: a 1 GiB write
    would leave the last-level cache full of dirty lines whose write-back
    lands in the next kernel's time (measured: +57 us on the 3B step's first
    kernel), which is the flush's cost, not the kernel's."""

    def __init__(self):
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")

    def __call__(self):
        self.sink = self.buf.sum()


def flush_buffer():
    return CacheFlush()


def time_steps(step, steps, warmup, eager):
    """Device ms per step: HIP events on the launch stream around each step;
    before each step (outside the events) a 1 GiB read evicts every cache
    level, so each step reads its inputs and weights from HBM."""
    run = step.run if eager else capture(step.run).replay
    flush = flush_buffer()
    for _ in range(warmup):
        flush()
        run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        flush()
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / steps


def per_call_times(step, reps):
    """Device time per launch of every named call, from HIP events on the
    library's stream around graph replays of that call alone: for each name, a
    graph of all of the step's launches of that name in step order (decode:
    one launch per layer, distinct weights), repeated so that a replay holds
    at least 8 launches. A 1 GiB read precedes every replay (outside the
    events), so the replay's first launch finds no input in any cache."""
    calls = step.calls()
    names = list(dict.fromkeys(n for n, _ in calls))
    flush = flush_buffer() if step.cold_weights else None
    out, per_step = {}, {}
    for name in names:
        fs = [f for n, f in calls if n == name]
        per_step[name] = len(fs)
        rep = max(1, -(-8 // len(fs)))
        graph = capture(lambda: [f() for _ in range(rep) for f in fs])
        launches = rep * len(fs)
        graph.replay()
        ms = []
        for _ in range(reps):
            if flush is not None:
                flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            graph.replay()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b) / launches)
        out[name] = float(np.median(ms))
        del graph
    return out, per_step


def cpu_baseline(wl_name, N, M, seconds, decode_T=None, backward=False):
    import oracle as o
    from threadpoolctl import threadpool_info
    if wl_name == "bitnet_decode":
        W, X = make_workload(wl_name, T=decode_T)
        wl = WORKLOADS[wl_name]
        # decode path: prepacked weights; the oracle's act quant + GEMM + dequant
        prep = {l.name: o.quant_mask_weight(W[l.name], 2, 4) for l in wl.linears}
        def one():
            for l in wl.linears:
                xq, sx = o.quant_act(X[l.x_name])
                o.dequant(o.gemm_int(xq, prep[l.name][0]), sx, prep[l.name][3])
        units = sum(l.O * l.K * 0.25 + decode_T * l.K + 2 * decode_T * l.O
                    for l in wl.linears)
        unit, sample = "GB/s", f"one BitNet-2B4T decode layer, T={decode_T}, prepacked 2:4"
    else:
        W, X = make_workload(wl_name)
        wl = WORKLOADS[wl_name]
        rng = np.random.default_rng(7)
        dys = {l.name: bf16_round(rng.standard_normal((wl.T, l.O)).astype(np.float32))
               for l in wl.linears} if backward else {}
        def one():
            for l in wl.linears:
                r = o.linear_fwd(X[l.x_name], W[l.name], N, M)
                if backward:
                    o.linear_bwd_dx(dys[l.name], r["w_eff"], r["sw"])
                    o.linear_bwd_dw(dys[l.name], o.act_dequant_bf16(r["xq"], r["sx"]))
        units = sum(2.0 * wl.T * l.O * l.K for l in wl.linears) * (3.0 if backward else 1.0)
        unit = "TOPS"
        sample = (f"full {wl_name} step (T={wl.T}, {N}:{M}, every projection, mask "
                  f"recomputed{', forward + backward' if backward else ''}), repeated")
    times = []
    t_end = time.time() + seconds
    while time.time() < t_end or len(times) < 1:
        t0 = time.perf_counter()
        one()
        times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    val = units / med / (1e12 if unit == "TOPS" else 1e9)
    return {"value": round(val, 6), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{sample} x{len(times)}, median {med * 1e3:.1f} ms per step",
            "cpu_model": _cpu_model(), "nproc": os.cpu_count()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


TRAFFIC_FILES = [os.path.join(ROOT, "profiles", f)
                 for f in ("traffic_qwen3b_sweep.txt", "traffic_qwen05b_ffn.txt",
                           "traffic_qwen15b_ffn.txt", "traffic_bitnet_decode_t8.txt",
                           "traffic_qwen15b_ffn_train.txt")]
def measured_traffic(workload, kernel_call):
    """HBM bytes per launch of the dominant call from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (scaled by the same counters on a plain
    copy of known size). None if the call has no entry or its kernels' source
    has changed since the counters were taken."""
    import hashlib
    text = ""
    for path in TRAFFIC_FILES:
        try:
            text += open(path).read() + "\n\n"
        except OSError:
            pass
    for block in text.split("\n\n"):
        kv = dict(line.split("=", 1) for line in block.split("\n")
                  if "=" in line and not line.startswith("#"))
        if kv.get("call", "").strip() != kernel_call or kv.get("workload", "").strip() != workload:
            continue
        try:
            src = os.path.join(ROOT, kv["src"].strip())
            if hashlib.sha256(open(src, "rb").read()).hexdigest() != kv["src_sha256"].strip():
                return None
            return float(kv["hbm_bytes_per_launch"])
        except (OSError, KeyError, ValueError):
            return None
    return None


def calibrate_copy():
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n,
                      "bytes_written_per_copy": n, "copies": 3}))


def copy_bandwidth():
    """HBM bandwidth a plain device copy reaches on this GPU (GB/s, read + written
    bytes): a 1 GiB device-to-device copy, one warm-up then five timed copies
    between HIP events on the current stream. The practical ceiling the
    HBM-bound calls are also compared with."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(5):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    rate = 2.0 * n * 5 / (s.elapsed_time(e) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return rate


def traffic_tag(a, N, M):
    """Workload key of the committed counter summaries."""
    if a.workload == "bitnet_decode":
        return f"bitnet_decode T={a.decode_T} L={a.layers}"
    return (f"{a.workload} T={WORKLOADS[a.workload].T} {N}:{M}" + (" diag" if a.diagnostics else "")
            + (" norm" if a.fused_norm else "") + (" ternary-mask" if a.mask_from_ternary else "")
            + (" mask-then-quant" if a.mask_then_quant else "") + (" backward" if a.backward else "")
            + (" gated" if a.mask_gated_grad and a.backward else ""))


def per_call_rates(step, per_call, copy_gbs=None):
    """Device time of one launch of each call and its rate against the call's
    own roofline (HBM GB/s or effective TOPS); HBM-bound calls also against
    the measured device-copy bandwidth."""
    out = {}
    for k, ms in per_call.items():
        bound, units, _ = step.call_info(k)
        rate = units / (ms * 1e-3)
        if bound == "hbm":
            out[k] = {"us": round(ms * 1e3, 2), "GB/s": round(rate / 1e9, 1),
                      "frac": round(rate / 1e9 / PEAK_HBM_GBS, 4)}
            if copy_gbs:
                out[k]["frac_of_copy"] = round(rate / 1e9 / copy_gbs, 4)
        elif bound == "mfma_bf16":
            out[k] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(rate / 1e12, 1),
                      "frac": round(rate / 1e12 / PEAK_BF16_DENSE_TFLOPS, 4)}
        else:
            # effective (dense-equivalent) TOPS against the dense int8 peak; also the
            # algorithmic rate (kept weights only, x N/M) and, where the GEMM runs on
            # the 2:4 sparse instruction (2:4, 2:8), the fraction of its 2x peak
            N, M = getattr(step, "N", None), getattr(step, "M", None)
            out[k] = {"us": round(ms * 1e3, 2), "TOPS": round(rate / 1e12, 1),
                      "frac": round(rate / 1e12 / PEAK_INT8_DENSE_TOPS, 4)}
            if N and M:
                out[k]["algorithmic_TOPS"] = round(rate * N / M / 1e12, 1)
                if (N, M) in ((2, 4), (2, 8)):
                    out[k]["frac_of_sparse_peak"] = round(rate / 1e12 / (2 * PEAK_INT8_DENSE_TOPS), 4)
    return out


def main():
    a = parse()
    if a.calibrate_copy:
        calibrate_copy()
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU (no multi-GPU path); --gpus must be 1",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    torch.cuda.init()
    wl = WORKLOADS[a.workload]
    N, M = wl.N, wl.M
    if a.nm:
        N, M = (int(v) for v in a.nm.split(":"))
    if a.mask_from_ternary and a.mask_then_quant:
        sys.exit("bench.py: --mask-from-ternary and --mask-then-quant are two separate ablations")
    if a.workload == "bitnet_decode":
        step = DecodeStep(a.decode_T, a.layers)
    else:
        step = PrefillStep(a.workload, N, M, a.diagnostics, a.fused_norm,
                           1 if a.mask_from_ternary else 2 if a.mask_then_quant else 0,
                           a.backward, a.mask_gated_grad, a.overlap_backward)
    ms = time_steps(step, a.steps, a.warmup, a.eager)
    per_call, calls_per_step = per_call_times(step, max(5, min(a.steps, 20)))
    share = {k: per_call[k] * calls_per_step[k] for k in per_call}
    dom = max(share, key=share.get)
    bound, units, kind = step.call_info(dom)
    achieved = units / (per_call[dom] * 1e-3)
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(achieved / 1e12, 2),
                "peak": PEAK_INT8_DENSE_TOPS, "unit": "TFLOP/s"}
    elif bound == "mfma_bf16":
        roof = {"bound": "mfma", "achieved": round(achieved / 1e12, 2),
                "peak": PEAK_BF16_DENSE_TFLOPS, "unit": "TFLOP/s", "dtype": "bf16"}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    copy_gbs = copy_bandwidth()
    if roof["bound"] == "hbm":
        roof["frac_of_copy"] = round(roof["achieved"] / copy_gbs, 4)
    roof["traffic"] = measured_traffic(traffic_tag(a, N, M), dom)
    roof["kernel"] = dom
    roof["avg_ms"] = round(per_call[dom], 5)

    if a.workload == "bitnet_decode":
        total_bytes = step.bytes_layer * step.L
        value = total_bytes / (ms * 1e-3) / 1e9
        metric, unit = "Sparse-BitLinear decode GB/s (prepacked 2:4, whole layer stream)", "GB/s"
        config = {"workload": "bitnet_decode", "tokens": a.decode_T, "layers": a.layers,
                  "nm": "2:4", "bytes_per_step": total_bytes,
                  "weights_per_layer": step.weights}
    else:
        value = step.ops / (ms * 1e-3) / 1e12
        metric = ("Sparse-BitLinear effective TOPS (training step: prefill forward + Dual-STE "
                  "backward)" if a.backward else "Sparse-BitLinear effective TOPS (prefill)")
        unit = "TOPS"
        config = {"workload": a.workload, "tokens": step.T, "nm": f"{N}:{M}",
                  "mask_diagnostics": bool(a.diagnostics), "fused_rmsnorm": bool(a.fused_norm),
                  "mask_from": "ternary codes (ablation)" if a.mask_from_ternary else "master |W|",
                  "composition": "mask-then-quant (ablation)" if a.mask_then_quant else "quant-then-mask",
                  "projections": [f"{l.name} {l.O}x{l.K}" for l in wl.linears],
                  "mask": "recomputed every step", "dense_equiv_ops_per_step": step.ops,
                  "backward": bool(a.backward),
                  "gradient": ("mask-gated (ablation)" if a.mask_gated_grad and a.backward else
                               "dense (Dual STE)") if a.backward else None,
                  "backward_schedule": (("dW on a second stream beside dX" if a.overlap_backward
                                         else "one stream") if a.backward else None)}
    out = {
        "metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("int8xternary->int32 fwd, bf16 MFMA (fp32 acc) bwd" if getattr(a, "backward", False)
                  else "int8xternary->int32 (bf16 in/out)"), "data": "synthetic",
        "config": config, "roofline": roof,
        "breakdown_ms": {k: round(share[k], 5) for k in share},
        "per_call": per_call_rates(step, per_call, copy_gbs),
        "breakdown_note": "per-step device ms of each call, from graph replays of that call alone",
        "timing": "eager launches" if a.eager else "HIP graph replay",
        "copy_GBs": round(copy_gbs, 1),
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(a.workload, N, M, a.cpu_seconds, a.decode_T,
                                           a.backward and a.workload != "bitnet_decode")
    print(json.dumps(out))


if __name__ == "__main__":
    main()

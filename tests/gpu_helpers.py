"""Shared helpers of the GPU parity tests (comparison rules, case logging)."""
import sys

import numpy as np
import torch

import oracle as o


def log_case(*parts):
    """Name the case before the GPU runs it (flushed, so a crash still shows it)."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    return t if dtype is None else t.to(dtype)


def bf16_tensor(x_f32):
    """bf16-exact fp32 numpy array -> bf16 device tensor (exact)."""
    return to_dev(x_f32).to(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def assert_f32_close(y_gpu, y_ref64, rtol=1e-3):
    """fp32 output: |d| / max(|ref|, 1e-6 * max|ref|) <= rtol."""
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref64 = np.asarray(y_ref64, np.float64)
    floor = 1e-6 * max(float(np.abs(y_ref64).max(initial=0.0)), 1e-30)
    rel = np.abs(y_gpu - y_ref64) / np.maximum(np.abs(y_ref64), floor)
    assert float(rel.max(initial=0.0)) <= rtol, f"max rel err {rel.max()}"


def assert_bf16_exact(y_gpu_f32, acc, sx, sw):
    """bf16 output: bit-identical to the bf16 rounding (nearest even) of
    fp32(fp32(acc * sx[t]) * sw[o]) -- the dequant product in the reading's
    fixed fp32 order, from the oracle's exact int32 accumulator."""
    ref = o.to_bf16(o.dequant_f32(acc, sx, sw).astype(np.float64))
    got = np.asarray(y_gpu_f32, np.float32)
    assert got.shape == ref.shape
    bad = got.view(np.uint32) != ref.view(np.uint32)
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} bf16 outputs differ, first at "
                           f"{np.argwhere(bad)[0].tolist()}")


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)

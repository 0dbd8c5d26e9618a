"""Helpers shared by the GPU tests: run the HIP path through the binding and
the oracle on the same seeded inputs."""
import numpy as np

import oracle
from block_scaled_fp4_act_amd import inputs

FMT = {"nvfp4": 0, "mxfp4": 1}


def dev_x(x_np, bf16):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_np, np.float32))
    if bf16:
        t = t.to(torch.bfloat16)
    return t.cuda()


def gpu_quantize(x_np, fmt, bf16, with_residue=True):
    import torch
    import block_scaled_fp4_act_amd as rs
    M, K = x_np.shape
    act = rs.quantize_act_with_residue(dev_x(x_np, bf16), fmt, with_residue)
    codes, scales, globs = rs.act_views(act, fmt, M, K, with_residue)
    torch.cuda.synchronize()
    return act, codes.cpu().numpy(), scales.cpu().numpy(), globs.cpu().numpy()


def assert_quant_equal(x_np, fmt, bf16, with_residue=True):
    """Bit-exact comparison of codes, scale bytes and fp32 tensor scales."""
    xin = inputs.round_to_bf16(x_np) if bf16 else np.ascontiguousarray(x_np, np.float32)
    act, c, s, g = gpu_quantize(xin, fmt, bf16, with_residue)
    q = oracle.quantize_act(xin, fmt, with_residue)
    assert np.array_equal(c, q["codes"]), _first_diff(c, q["codes"])
    assert np.array_equal(s, q["scales"]), _first_diff(s, q["scales"])
    assert np.array_equal(g.view(np.uint32), q["globals"].view(np.uint32)), _first_diff(g, q["globals"])
    return act, q


def _first_diff(a, b):
    idx = np.argwhere(a != b)
    if len(idx) == 0:
        return "equal"
    i = tuple(idx[0])
    return f"{len(idx)} mismatches; first at {i}: gpu={a[i]!r} oracle={b[i]!r}"


def check_linear(y_gpu, y_orc, beta, tol=1e-4):
    """|y_gpu - y_oracle| <= tol * beta elementwise (beta = sum of |terms|)."""
    err = np.abs(y_gpu.astype(np.float64) - y_orc)
    bad = err > tol * beta
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} outside tolerance; worst ratio "
                           f"{float((err / np.maximum(beta, 1e-300)).max()):.3e}")


def sample_channels(N, M, seed, min_outputs=4096, floor=192):
    """Sorted output channels for a sampled full-size check: enough that the
    sample holds at least min_outputs elements of y [M, N] (and floor
    channels), always including the first and the last channel."""
    n = min(N, max(floor, -(-min_outputs // M)))
    rows = np.sort(np.random.default_rng(seed).choice(N, n, replace=False))
    rows[0], rows[-1] = 0, N - 1
    return rows

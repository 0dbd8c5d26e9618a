"""GPU check of rsfp4_nvfp4_linear_compensated_noalloc (the library's own
scratch as the workspace) through the C ABI: bit for bit the output
of rsfp4_nvfp4_linear_compensated given a caller's workspace of the size that
the scratch holds of it, on calls in a
row whose second is smaller, and within the oracle's tolerance."""
import numpy as np
import pytest

import oracle
from block_scaled_fp4_act_amd import inputs
from gpu_util import check_linear, dev_x

pytestmark = pytest.mark.gpu


def _case(M, N, K, seed):
    import torch
    import block_scaled_fp4_act_amd as rs
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    W = inputs.weights(N, K, seed + 1)
    blob = rs.prepack_weights(torch.from_numpy(W).cuda(), 0)
    act = rs.quantize_act_with_residue(dev_x(x, True), 0, True)
    return x, W, blob, act


def test_noalloc_matches_workspace_entry():
    import torch
    import block_scaled_fp4_act_amd as rs
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    rs.lib()
    oracle.build()
    # the MLP down projection (K split in four on a 256-CU device), then a
    # smaller split call, a shape whose plan does not split, two row tiles
    # split in two, wide operands whose rewritten activations and split
    # partials fit in the scratch (1 + 2 MB; 8-wave tiles over N = 16400,
    # 0.4 + 8.3 MB) and one whose do not (32 MB: it runs without them, with
    # the records path's bits)
    for i, (M, N, K) in enumerate([(8, 4096, 14336), (3, 512, 8192), (4, 1024, 4096), (16, 2048, 8192),
                                   (64, 1024, 4096), (20, 16400, 4096), (1024, 256, 8192)]):
        x, W, blob, act = _case(M, N, K, 40 + i)
        # the workspace entry given what the scratch holds of the workspace
        nb = min(rs.workspace_bytes(0, M, N, K, True), 16384 + 16777216)
        ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
        y_ref = torch.empty((M, N), device="cuda")
        rs.fp4_linear_compensated(act, blob, M, N, K, 0, out=y_ref, ws=ws)
        y = torch.full((M, N), float("nan"), device="cuda")
        rs.nvfp4_linear_compensated_noalloc(act, blob, M, N, K, y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), (M, N, K)
        y2 = torch.full((M, N), float("nan"), device="cuda")
        rs.nvfp4_linear_compensated_noalloc(act, blob, M, N, K, y2)    # scratch reused: counters were left zero
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int32), y_ref.view(torch.int32)), (M, N, K)
        if N <= 1024:
            xin = inputs.round_to_bf16(x)
            q = oracle.quantize_act(xin, 0, True)
            w = oracle.quantize_weight(W, 0)
            yo, beta = oracle.linear(q["deq"], w["deq"], M, True)
            check_linear(y.cpu().numpy(), yo, beta)

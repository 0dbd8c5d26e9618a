"""GPU parity of the grouped (mixture of experts) linear: one launch over E
experts, expert e taking rows offsets[e] .. offsets[e+1] of one activation
buffer and the e-th of E stacked weight blobs.  Each expert's rows must equal,
bit for bit, the ordinary linear on those rows alone with that expert's
weights, and agree with the oracle within 1e-4 * sum_k |term_k|."""
import numpy as np
import pytest

import oracle
from block_scaled_fp4_act_amd import inputs
from gpu_util import _first_diff, check_linear, dev_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import block_scaled_fp4_act_amd as rs
    rs.lib()
    oracle.build()


def _rs():
    import block_scaled_fp4_act_amd as rs
    return rs


def _setup(fmt, E, counts, N, K, seed):
    import torch
    rs = _rs()
    rng = np.random.default_rng(seed)
    M_total = int(sum(counts))
    x = rng.standard_normal((M_total, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    Ws = [inputs.weights(N, K, seed * 100 + e) for e in range(E)]
    blobs = [rs.prepack_weights(torch.from_numpy(W).cuda(), fmt) for W in Ws]
    stacked = torch.cat(blobs)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return x, Ws, blobs, stacked, offs


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("comp", [True, False])
@pytest.mark.parametrize("case", [
    (1, [3], 80, 256), (4, [2, 0, 3, 1], 72, 512), (8, [1, 2, 1, 0, 2, 1, 1, 3], 528, 1024),
    (3, [8, 5, 8], 40, 4096), (2, [1, 1], 4112, 256),
], ids=lambda c: f"E{c[0]}_N{c[2]}_K{c[3]}")
def test_grouped_vs_per_expert(fmt, comp, case):
    import torch
    rs = _rs()
    E, counts, N, K = case
    x, Ws, blobs, stacked, offs = _setup(fmt, E, counts, N, K, E + N)
    M_total = x.shape[0]
    max_rows = max(counts)
    act = rs.quantize_act_with_residue(dev_x(x, True), fmt, with_residue=comp)
    y = torch.full((M_total, N), float("nan"), dtype=torch.float32, device="cuda")
    rs.fp4_grouped_linear(act, stacked, M_total, E, torch.from_numpy(offs).cuda(), max_rows, N, K, fmt, comp, out=y)
    torch.cuda.synchronize()
    yg = y.cpu().numpy()
    xin = inputs.round_to_bf16(x)
    for e in range(E):
        lo, hi = offs[e], offs[e + 1]
        if hi == lo:
            continue
        # the ordinary linear on the expert's rows alone
        act_e = rs.quantize_act_with_residue(dev_x(x[lo:hi], True), fmt, with_residue=comp)
        f = rs.fp4_linear_compensated if comp else rs.fp4_linear
        ye = f(act_e, blobs[e], hi - lo, N, K, fmt)
        torch.cuda.synchronize()
        a, b = yg[lo:hi].view(np.int32), ye.cpu().numpy().view(np.int32)
        assert np.array_equal(a, b), (e, _first_diff(a, b))
        q = oracle.quantize_act(xin[lo:hi], fmt, with_residue=comp)
        w = oracle.quantize_weight(Ws[e], fmt)
        yo, beta = oracle.linear(q["deq"], w["deq"], hi - lo, comp)
        check_linear(yg[lo:hi], yo, beta)


def test_grouped_rows_past_max_rows_untouched():
    """Rows of an expert past max_rows and rows no expert covers keep their
    values; offsets outside [0, M_total] are clamped."""
    import torch
    rs = _rs()
    E, N, K = 3, 64, 256
    counts = [2, 3, 1]
    x, Ws, blobs, stacked, _ = _setup(0, E, counts, N, K, 9)
    M_total = x.shape[0]
    act = rs.quantize_act_with_residue(dev_x(x, True), 0, with_residue=True)
    # expert 0: rows 0-1, expert 1: rows 2-4 but max_rows = 2, expert 2: [5, 99) clamped to [5, 6)
    offs = torch.tensor([0, 2, 5, 99], dtype=torch.int32, device="cuda")
    y = torch.full((M_total, N), 7.0, dtype=torch.float32, device="cuda")
    rs.fp4_grouped_linear(act, stacked, M_total, E, offs, 2, N, K, 0, True, out=y)
    torch.cuda.synchronize()
    yg = y.cpu().numpy()
    assert (yg[4] == 7.0).all()                      # expert 1's third row: past max_rows
    assert not (yg[[0, 1, 2, 3, 5]] == 7.0).any()


def test_grouped_graph_replays():
    """Grouped calls in a HIP graph, replayed with new offsets written by a
    device kernel between replays (as a router would): every replay equals
    the eager result for the offsets it saw."""
    import torch
    rs = _rs()
    E, N, K = 4, 96, 512
    counts = [2, 2, 2, 2]
    x, Ws, blobs, stacked, offs = _setup(1, E, counts, N, K, 3)
    M_total = x.shape[0]
    act = rs.quantize_act_with_residue(dev_x(x, True), 1, with_residue=True)
    offs_dev = torch.from_numpy(offs).cuda()
    variants = [torch.tensor(v, dtype=torch.int32, device="cuda") for v in
                ([0, 2, 4, 6, 8], [0, 1, 3, 6, 8], [0, 0, 4, 4, 8])]
    eager = []
    for v in variants:
        offs_dev.copy_(v)
        eager.append(rs.fp4_grouped_linear(act, stacked, M_total, E, offs_dev, 4, N, K, 1, True).clone())
    torch.cuda.synchronize()
    y = torch.zeros((M_total, N), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            rs.fp4_grouped_linear(act, stacked, M_total, E, offs_dev, 4, N, K, 1, True, out=y)
    torch.cuda.synchronize()
    for rep in range(2):
        for v, e in zip(variants, eager):
            offs_dev.copy_(v)
            y.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int32), e.view(torch.int32)), (rep, v.tolist())

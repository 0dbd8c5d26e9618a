"""GPU parity of the narrow linear with K split across workgroups: the K
slices' partial sums meet in the workspace of rsfp4_workspace_bytes and the
slice that completes a channel group's count sums them in slice order.
Against the oracle elementwise, bit for bit across repeated calls and graph
replays, with the workspace's counters left at zero, and equal (within the
tolerance) to the unsplit plan that a call without a workspace runs."""
import numpy as np
import pytest

import oracle
from block_scaled_fp4_act_amd import inputs
from gpu_util import check_linear, dev_x

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


def _cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


# (M, N, K) of compensated NVFP4 calls whose plan splits K on a 256-CU device:
# few channel groups with K of 64+ steps (four slices, two steps per wave;
# ragged N)
SPLIT_CASES = [(1, 512, 8192), (8, 512, 8192), (3, 1000, 12288), (6, 16, 16384), (8, 4096, 12288),
               # two row tiles (17..32 operand rows): slices of up to 32 steps
               (16, 2048, 8192), (12, 1000, 12288), (9, 520, 16384), (16, 4096, 14336), (10, 48, 4608)]


def _setup(M, N, K, seed):
    import torch
    rs = _rs()
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    W = inputs.weights(N, K, seed + 1)
    blob = rs.prepack_weights(torch.from_numpy(W).cuda(), 0)
    act = rs.quantize_act_with_residue(dev_x(x, True), 0, True)
    return x, W, blob, act


def _ws(M, N, K):
    import torch
    nb = _rs().workspace_bytes(0, M, N, K, True)
    return torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda"), nb


COUNTER_BYTES = 16384     # the workspace's fixed counter area (4096 groups)


def _counters_zero(ws, N):
    return int(ws[:COUNTER_BYTES].count_nonzero()) == 0


@pytest.mark.parametrize("MNK", SPLIT_CASES, ids=lambda t: "M%dN%dK%d" % t)
def test_split_vs_oracle(MNK):
    import torch
    if _cus() != 256:
        pytest.skip("the split cases are chosen for a 256-CU device")
    rs = _rs()
    M, N, K = MNK
    x, W, blob, act = _setup(M, N, K, M + N + K)
    ws, nb = _ws(M, N, K)
    assert nb > 0, "this shape's plan should split K"
    y = rs.fp4_linear_compensated(act, blob, M, N, K, 0, ws=ws)
    torch.cuda.synchronize()
    assert _counters_zero(ws, N)
    xin = inputs.round_to_bf16(x)
    q = oracle.quantize_act(xin, 0, True)
    w = oracle.quantize_weight(W, 0)
    yo, beta = oracle.linear(q["deq"], w["deq"], M, True)
    check_linear(y.cpu().numpy(), yo, beta)
    # without a workspace (or with one too small) the unsplit plan runs: the
    # same sums up to the order in which the slices are added
    y0 = rs.fp4_linear_compensated(act, blob, M, N, K, 0, ws=ws[:0])
    y1 = rs.fp4_linear_compensated(act, blob, M, N, K, 0, ws=ws[: nb - 256])
    torch.cuda.synchronize()
    check_linear(y0.cpu().numpy(), yo, beta)
    assert torch.equal(y0, y1)


def test_split_repeats_and_graph_replays():
    """Twenty calls in a row give the same bits (the slices are summed in a
    fixed order whatever their arrival order) and leave the counters zero;
    a captured graph replayed with eager calls between replays does too."""
    import torch
    if _cus() != 256:
        pytest.skip("the split case is chosen for a 256-CU device")
    rs = _rs()
    M, N, K = 8, 4096, 14336                   # the MLP down projection's shape
    _, _, blob, act = _setup(M, N, K, 11)
    ws, nb = _ws(M, N, K)
    assert nb > 0
    ref = rs.fp4_linear_compensated(act, blob, M, N, K, 0, ws=ws).clone()
    for _ in range(20):
        y = rs.fp4_linear_compensated(act, blob, M, N, K, 0, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32))
    assert _counters_zero(ws, N)
    out = torch.empty((M, N), device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            rs.fp4_linear_compensated(act, blob, M, N, K, 0, out=out, ws=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"replay {rep}"
        rs.fp4_linear_compensated(act, blob, M, N, K, 0, ws=ws)     # eager work between replays
        torch.cuda.synchronize()
    assert _counters_zero(ws, N)


def test_split_shapes_share_one_workspace():
    """Calls of different shapes (different channel-group counts, four, three
    and two slices, and one that does not split) in turn through one
    workspace: each leaves the shared counter area zero, so the next shape's
    counts start from zero (a layout that moved the partials with N would hand
    one call's partials to the next call's counters)."""
    import torch
    if _cus() != 256:
        pytest.skip("the split cases are chosen for a 256-CU device")
    rs = _rs()
    shapes = [(8, 4096, 14336), (8, 14336, 4096), (1, 512, 8192), (12, 1000, 12288), (16, 2048, 8192)]
    nb = max(rs.workspace_bytes(0, M, N, K, True) for M, N, K in shapes)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    data = []
    for i, (M, N, K) in enumerate(shapes):
        _, _, blob, act = _setup(M, N, K, 20 + i)
        ref = rs.fp4_linear_compensated(act, blob, M, N, K, 0, ws=ws[:0])
        data.append((M, N, K, blob, act, ref))
    for rep in range(3):
        for M, N, K, blob, act, ref in data:
            y = torch.full((M, N), float("nan"), device="cuda")
            rs.fp4_linear_compensated(act, blob, M, N, K, 0, out=y, ws=ws)
            torch.cuda.synchronize()
            tol = 1e-5 * float(ref.abs().max())
            assert float((y - ref).abs().max()) <= tol, (rep, M, N, K)
            assert _counters_zero(ws, N)


def test_workspace_query():
    """Nonzero for the split shapes, zero where the plan does not split."""
    if _cus() != 256:
        pytest.skip("the split shapes are chosen for a 256-CU device")
    rs = _rs()
    assert rs.workspace_bytes(0, 8, 4096, 14336, True) > 0        # MLP down
    assert rs.workspace_bytes(0, 8, 14336, 4096, True) == 0       # MLP up (half a round of groups: unsplit)
    assert rs.workspace_bytes(0, 4, 4096, 4096, True) == 0        # attention projection
    assert rs.workspace_bytes(0, 8, 28672, 8192, True) == 0       # large MLP (balanced)
    assert rs.workspace_bytes(1, 8, 4096, 14336, True) == 0       # MXFP4
    assert rs.workspace_bytes(0, 8, 4096, 14336, False) == 0      # plain
    assert rs.workspace_bytes(0, 16, 4096, 14336, True) > 0       # two row tiles, 4 slices of 28 steps
    assert rs.workspace_bytes(0, 16, 4096, 4096, True) == 0       # two row tiles, 32 steps: one pass
    assert rs.workspace_bytes(0, 17, 4096, 4096, True) == 0       # four row tiles
    assert rs.workspace_bytes(0, 17, 4096, 8192, True) > 0        # tiled, rewritten operand

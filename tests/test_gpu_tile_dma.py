"""GPU parity of the wide MXFP4 linear over LDS-DMA streamed operands: the
activation records are rewritten into the packed-weight layout (in the
workspace of rsfp4_workspace_bytes, after its counter area), then both tiled
operands are multiplied.  Against the oracle elementwise, and bit for bit
against the register-staged tiled kernel that a call with a smaller workspace
runs (both sum the same MFMAs in the same order); the workspace's counters
stay zero, and graph replays match the eager call."""
import numpy as np
import pytest

import oracle
from block_scaled_fp4_act_amd import inputs
from gpu_util import check_linear, dev_x, sample_channels

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


# (M, N, K, compensated): more than 32 stacked rows; ragged row tiles (rows
# past the operand), ragged channel tiles (N not a multiple of 16 or 256),
# K tails (K not a multiple of 128, or of 512: a partial last quad), a long K,
# and N past one channel tile many times over
CASES = [(17, 264, 384, True), (33, 130, 160, False), (40, 512, 1056, True), (64, 128, 256, True),
         (100, 72, 2048, False), (129, 300, 512, True), (40, 64, 24576, True), (30, 16400, 256, True),
         (200, 1000, 1184, True), (48, 520, 5152, False), (300, 40, 96, True), (37, 2056, 4096, True)]


def _setup(M, N, K, comp, seed):
    import torch
    rs = _rs()
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    W = inputs.weights(N, K, seed + 1)
    blob = rs.prepack_weights(torch.from_numpy(W).cuda(), 1)
    act = rs.quantize_act_with_residue(dev_x(x, True), 1, comp)
    return x, W, blob, act


def _call(act, blob, M, N, K, comp, ws, bf16=False):
    import torch
    rs = _rs()
    if bf16:
        f = rs.fp4_linear_compensated_bf16 if comp else rs.fp4_linear_bf16
    else:
        f = rs.fp4_linear_compensated if comp else rs.fp4_linear
    y = f(act, blob, M, N, K, 1, ws=ws)
    torch.cuda.synchronize()
    return y


def _ws(M, N, K, comp):
    import torch
    nb = _rs().workspace_bytes(1, M, N, K, comp)
    B = 2 * M if comp else M
    assert nb == 16384 + -(-B // 16) * _group_bytes(K)
    return torch.zeros(nb, dtype=torch.uint8, device="cuda")


def _group_bytes(K):
    quads = -(-K // 512)
    return quads * (4 * 1024 + 256)


def _small_ws():
    import torch
    return torch.zeros(256, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("case", CASES, ids=lambda c: "M%dN%dK%d%s" % (c[0], c[1], c[2], "c" if c[3] else "p"))
def test_dma_path_matches_oracle(case):
    M, N, K, comp = case
    x, W, blob, act = _setup(M, N, K, comp, M * 7 + N + K)
    ws = _ws(M, N, K, comp)
    y = _call(act, blob, M, N, K, comp, ws).cpu().numpy()
    xin = inputs.round_to_bf16(x)
    q = oracle.quantize_act(xin, 1, with_residue=comp)
    w = oracle.quantize_weight(W, 1)
    yo, beta = oracle.linear(q["deq"], w["deq"], M, comp)
    check_linear(y, yo, beta)
    assert int(ws[:16384].count_nonzero()) == 0, "the workspace's counter area must stay zero"


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "M%dN%dK%d%s" % (c[0], c[1], c[2], "c" if c[3] else "p"))
def test_dma_path_bitwise_equals_register_staged(case, bf16):
    M, N, K, comp = case
    _, _, blob, act = _setup(M, N, K, comp, M * 11 + N + 3 * K)
    import torch
    y_dma = _call(act, blob, M, N, K, comp, _ws(M, N, K, comp), bf16)
    y_reg = _call(act, blob, M, N, K, comp, _small_ws(), bf16)
    it = torch.int16 if bf16 else torch.int32
    a, b = y_dma.view(it), y_reg.view(it)
    assert torch.equal(a, b), f"{int((a != b).sum())} of {a.numel()} outputs differ"


@pytest.mark.parametrize("M", [17, 32, 64, 128, 256])
def test_dma_path_workload(M):
    """The MXFP4 workload at full size (K = 5120, N = 25600) as the bench
    launches it: bit for bit against the register-staged kernel, and a sample
    of output channels against the oracle."""
    import torch
    wl = inputs.MX.with_m(M)
    rs = _rs()
    x, W = wl.draw_x(), wl.draw_w()
    blob = rs.prepack_weights(torch.from_numpy(W).cuda(), 1)
    act = rs.quantize_act_with_residue(dev_x(x, wl.bf16), 1, True)
    y_dma = _call(act, blob, M, wl.N, wl.K, True, _ws(M, wl.N, wl.K, True))
    y_reg = _call(act, blob, M, wl.N, wl.K, True, _small_ws())
    assert torch.equal(y_dma.view(torch.int32), y_reg.view(torch.int32))
    rows = sample_channels(wl.N, M, 5)
    xin = inputs.round_to_bf16(x) if wl.bf16 else x
    q = oracle.quantize_act(xin, 1, with_residue=True)
    w = oracle.quantize_weight(W, 1, rows=rows)
    yo, beta = oracle.linear(q["deq"], w["deq"], M, True)
    check_linear(y_dma.cpu().numpy()[:, rows], yo, beta)


# Ragged shapes large enough for the 256-row tiles on a 256-CU device:
# 256 x 256 tiles (3 row tiles, the last with 8 rows; 65 channel tiles, the
# last with one group) and 256 x 128 tiles (one row tile of 240 rows)
WIDE_CASES = [(260, 16400, 1184, True), (120, 24600, 1056, True), (250, 24600, 672, False)]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: "M%dN%dK%d%s" % (c[0], c[1], c[2], "c" if c[3] else "p"))
def test_dma_path_large_tiles(case):
    import torch
    M, N, K, comp = case
    x, W, blob, act = _setup(M, N, K, comp, M + N + 5 * K)
    y_dma = _call(act, blob, M, N, K, comp, _ws(M, N, K, comp))
    y_reg = _call(act, blob, M, N, K, comp, _small_ws())
    assert torch.equal(y_dma.view(torch.int32), y_reg.view(torch.int32))
    rows = sample_channels(N, M, 3)
    rows = np.unique(np.concatenate([rows, np.arange(N - 40, N)]))   # the ragged last channel tile
    xin = inputs.round_to_bf16(x)
    q = oracle.quantize_act(xin, 1, with_residue=comp)
    w = oracle.quantize_weight(W, 1, rows=rows)
    yo, beta = oracle.linear(q["deq"], w["deq"], M, comp)
    check_linear(y_dma.cpu().numpy()[:, rows], yo, beta)


def test_dma_path_graph_replays():
    """Rewrite + product captured in a HIP graph: every replay (with eager
    work between them) equals the eager call bit for bit."""
    import torch
    M, N, K = 96, 2056, 2048
    _, _, blob, act = _setup(M, N, K, True, 99)
    ws = _ws(M, N, K, True)
    y_eager = _call(act, blob, M, N, K, True, ws).clone()
    rs = _rs()
    out = torch.empty(M, N, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        rs.fp4_linear_compensated(act, blob, M, N, K, 1, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rs.fp4_linear_compensated(act, blob, M, N, K, 1, out=out, ws=ws)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), y_eager.view(torch.int32))
        _ = _call(act, blob, M, N, K, True, ws)    # eager work between replays

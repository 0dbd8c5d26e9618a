"""GPU parity of the wide linear over LDS-DMA streamed activations: the
activation records are rewritten in tiles (MXFP4: the packed-weight layout,
both operands then streamed into LDS; NVFP4: exact f16 MFMA fragments) in the
workspace of rsfp4_workspace_bytes, after its counter area, then multiplied.  Against the oracle elementwise, and bit for bit
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


# (M, N, K, compensated): more than 32 stacked rows (NVFP4 64-row tiles up to
# 64 rows and from 97 to 128, and up to 256 below N = 16384: 180 rows in three); ragged row tiles (rows
# past the operand), ragged channel tiles (N not a multiple of 16 or 256),
# K tails (K not a multiple of 128, or of 512: a partial last quad), a long K,
# and N past one channel tile many times over
CASES = [(17, 264, 384, True), (33, 130, 160, False), (40, 512, 1056, True), (64, 128, 256, True),
         (100, 72, 2048, False), (129, 300, 512, True), (40, 64, 24576, True), (30, 16400, 256, True),
         (200, 1000, 1184, True), (48, 520, 5152, False), (300, 40, 96, True), (37, 2056, 4096, True),
         (20, 16400, 4096, True), (90, 520, 1184, True),
         # 65..96 stacked rows at wide N: one 128-row tile (split in K when few)
         (40, 16400, 4096, True), (90, 16400, 1184, False)]
# NVFP4 compensated with 33..64 stacked rows, N <= 4096 and K <= 4096 runs
# the narrow kernel with four row tiles instead: those shapes are left out
NV_NARROW4 = lambda M, N, K, comp: comp and 2 * M <= 64 and N <= 4096 and K <= 4096
FMT_CASES = [(f,) + c for f in (0, 1) for c in CASES if not (f == 0 and NV_NARROW4(*c))]


def _cid(c):
    return "%s-M%dN%dK%d%s" % ("nv" if c[0] == 0 else "mx", c[1], c[2], c[3], "c" if c[4] else "p")


def _setup(fmt, M, N, K, comp, seed):
    import torch
    rs = _rs()
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    W = inputs.weights(N, K, seed + 1)
    blob = rs.prepack_weights(torch.from_numpy(W).cuda(), fmt)
    act = rs.quantize_act_with_residue(dev_x(x, True), fmt, comp)
    return x, W, blob, act


def _call(fmt, act, blob, M, N, K, comp, ws, bf16=False):
    import torch
    rs = _rs()
    if bf16:
        f = rs.fp4_linear_compensated_bf16 if comp else rs.fp4_linear_bf16
    else:
        f = rs.fp4_linear_compensated if comp else rs.fp4_linear
    y = f(act, blob, M, N, K, fmt, ws=ws)
    torch.cuda.synchronize()
    return y


def _ws(fmt, M, N, K, comp, split=True):
    """The workspace rsfp4_workspace_bytes asks for: the counter area and the
    rewritten activations, and for an NVFP4 product with few tiles room for
    its K slices' partial sums.  split=False: the counter area and the
    rewritten activations only (the product then runs unsplit)."""
    import torch
    nb = _rs().workspace_bytes(fmt, M, N, K, comp)
    B = 2 * M if comp else M
    base = 16384 + -(-B // 16) * _group_bytes(fmt, K)
    assert nb == base or (fmt == 0 and nb > base), (nb, base)
    return torch.zeros(nb if split else base, dtype=torch.uint8, device="cuda")


def _splits(fmt, M, N, K, comp):
    B = 2 * M if comp else M
    return _rs().workspace_bytes(fmt, M, N, K, comp) > 16384 + -(-B // 16) * _group_bytes(fmt, K)


def _group_bytes(fmt, K):
    """Bytes of 16 rows of the rewritten activations: MXFP4 quads of 4 steps
    (4 KB of codes + 256 B of scale words), NVFP4 4 KB of f16 per step."""
    if fmt == 1:
        return -(-K // 512) * (4 * 1024 + 256)
    return -(-K // 128) * 4096


def _small_ws():
    import torch
    return torch.zeros(256, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("case", FMT_CASES, ids=_cid)
def test_dma_path_matches_oracle(case):
    fmt, M, N, K, comp = case
    x, W, blob, act = _setup(fmt, M, N, K, comp, M * 7 + N + K)
    ws = _ws(fmt, M, N, K, comp)
    y = _call(fmt, act, blob, M, N, K, comp, ws).cpu().numpy()
    xin = inputs.round_to_bf16(x)
    q = oracle.quantize_act(xin, fmt, with_residue=comp)
    w = oracle.quantize_weight(W, fmt)
    yo, beta = oracle.linear(q["deq"], w["deq"], M, comp)
    check_linear(y, yo, beta)
    assert int(ws[:16384].count_nonzero()) == 0, "the workspace's counter area must stay zero"


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", FMT_CASES, ids=_cid)
def test_dma_path_bitwise_equals_register_staged(case, bf16):
    fmt, M, N, K, comp = case
    _, _, blob, act = _setup(fmt, M, N, K, comp, M * 11 + N + 3 * K)
    import torch
    y_dma = _call(fmt, act, blob, M, N, K, comp, _ws(fmt, M, N, K, comp, split=False), bf16)
    y_reg = _call(fmt, act, blob, M, N, K, comp, _small_ws(), bf16)
    it = torch.int16 if bf16 else torch.int32
    a, b = y_dma.view(it), y_reg.view(it)
    assert torch.equal(a, b), f"{int((a != b).sum())} of {a.numel()} outputs differ"


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", [c for c in FMT_CASES if c[0] == 0], ids=_cid)
def test_split_deterministic(case, bf16):
    """NVFP4 products with few tiles split K across workgroups (the shapes
    where the workspace has room for partial sums): the last slice to arrive
    adds all slices in slice order, so repeated calls agree bit for bit, the
    counters are left zero, and the result agrees with the unsplit product
    to within the summation order (both against the oracle in the test
    above).  Shapes that do not split give the unsplit product's bits."""
    import torch
    fmt, M, N, K, comp = case
    splits = _splits(fmt, M, N, K, comp)
    _, _, blob, act = _setup(fmt, M, N, K, comp, M * 13 + N + K)
    ws = _ws(fmt, M, N, K, comp)
    ys = [_call(fmt, act, blob, M, N, K, comp, ws, bf16) for _ in range(3)]
    it = torch.int16 if bf16 else torch.int32
    for y in ys[1:]:
        assert torch.equal(y.view(it), ys[0].view(it))
    assert int(ws[:16384].count_nonzero()) == 0, "the split's counters must be left zero"
    y1 = _call(fmt, act, blob, M, N, K, comp, _ws(fmt, M, N, K, comp, split=False), bf16)
    if not splits:
        assert torch.equal(ys[0].view(it), y1.view(it))
        return
    y1 = y1.float()
    # fp32 sums that differ in the last bits may round to neighbouring bf16
    # values: one bf16 ulp, at most 2^-7 of the value
    tol = 1e-4 * max(1.0, y1.abs().max().item()) + (2.0 ** -7 if bf16 else 0.0) * y1.abs()
    d = (ys[0].float() - y1).abs()
    assert bool((d <= tol).all()), float(d.max())


@pytest.mark.parametrize("wl", [inputs.MX.with_m(m) for m in (17, 32, 64, 128, 256)]
                         + [inputs.LARGE_MLP.with_m(m) for m in (17, 32, 64, 128)], ids=lambda w: f"{w.name}_M{w.M}")
def test_dma_path_workload(wl):
    """The MXFP4 and large-MLP NVFP4 workloads at full size, as the bench
    launches them: bit for bit against the register-staged kernel, and a
    sample of output channels against the oracle."""
    import torch
    fmt = 1 if wl.fmt == "mxfp4" else 0
    M = wl.M
    rs = _rs()
    x, W = wl.draw_x(), wl.draw_w()
    blob = rs.prepack_weights(torch.from_numpy(W).cuda(), fmt)
    act = rs.quantize_act_with_residue(dev_x(x, wl.bf16), fmt, True)
    y_dma = _call(fmt, act, blob, M, wl.N, wl.K, True, _ws(fmt, M, wl.N, wl.K, True, split=False))
    y_reg = _call(fmt, act, blob, M, wl.N, wl.K, True, _small_ws())
    assert torch.equal(y_dma.view(torch.int32), y_reg.view(torch.int32))
    rows = sample_channels(wl.N, M, 5)
    xin = inputs.round_to_bf16(x) if wl.bf16 else x
    q = oracle.quantize_act(xin, fmt, with_residue=True)
    w = oracle.quantize_weight(W, fmt, rows=rows)
    yo, beta = oracle.linear(q["deq"], w["deq"], M, True)
    check_linear(y_dma.cpu().numpy()[:, rows], yo, beta)


# Ragged shapes large enough for the 256-row tiles on a 256-CU device:
# 256 x 256 tiles (3 row tiles, the last with 8 rows; 65 channel tiles, the
# last with one group) and 256 x 128 tiles (one row tile of 240 rows)
WIDE_CASES = [(1, 260, 16400, 1184, True), (1, 120, 24600, 1056, True), (1, 250, 24600, 672, False),
              (0, 130, 28700, 1184, True), (0, 200, 16400, 800, False)]


@pytest.mark.parametrize("case", WIDE_CASES, ids=_cid)
def test_dma_path_large_tiles(case):
    import torch
    fmt, M, N, K, comp = case
    x, W, blob, act = _setup(fmt, M, N, K, comp, M + N + 5 * K)
    y_dma = _call(fmt, act, blob, M, N, K, comp, _ws(fmt, M, N, K, comp, split=False))
    y_reg = _call(fmt, act, blob, M, N, K, comp, _small_ws())
    assert torch.equal(y_dma.view(torch.int32), y_reg.view(torch.int32))
    rows = sample_channels(N, M, 3)
    rows = np.unique(np.concatenate([rows, np.arange(N - 40, N)]))   # the ragged last channel tile
    xin = inputs.round_to_bf16(x)
    q = oracle.quantize_act(xin, fmt, with_residue=comp)
    w = oracle.quantize_weight(W, fmt, rows=rows)
    yo, beta = oracle.linear(q["deq"], w["deq"], M, comp)
    check_linear(y_dma.cpu().numpy()[:, rows], yo, beta)


@pytest.mark.parametrize("wl", [inputs.MLP_DOWN.with_m(64), inputs.MLP_DOWN.with_m(128), inputs.ATTN.with_m(64),
                                inputs.ATTN.with_m(128)], ids=lambda w: f"{w.name}_M{w.M}")
def test_split_workload(wl):
    """Full-size NVFP4 shapes with few tiles (N = 4096; 64- and 128-row
    tiles), compensated: K split across workgroups; a
    sample of output channels against the oracle, repeat calls bit for bit,
    the counters left zero."""
    import torch
    M = wl.M
    rs = _rs()
    x, W = wl.draw_x(), wl.draw_w()
    blob = rs.prepack_weights(torch.from_numpy(W).cuda(), 0)
    act = rs.quantize_act_with_residue(dev_x(x, wl.bf16), 0, True)
    ws = _ws(0, M, wl.N, wl.K, True)
    assert _splits(0, M, wl.N, wl.K, True)
    if M == 64 and wl.K == 14336 and torch.cuda.get_device_properties(0).multi_processor_count == 256:
        # 64-row tiles: 2 x 32 tiles, K in 4 slices of 32 steps; per tile,
        # wave and slice 64 lanes x 4 x 2 x 2 folded partial sums
        assert ws.numel() == 16384 + 8 * 112 * 4096 + 64 * 4 * 4 * 64 * 16 * 4
    y = _call(0, act, blob, M, wl.N, wl.K, True, ws)
    y2 = _call(0, act, blob, M, wl.N, wl.K, True, ws)
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    assert int(ws[:16384].count_nonzero()) == 0
    rows = sample_channels(wl.N, M, 5)
    xin = inputs.round_to_bf16(x) if wl.bf16 else x
    q = oracle.quantize_act(xin, 0, with_residue=True)
    w = oracle.quantize_weight(W, 0, rows=rows)
    yo, beta = oracle.linear(q["deq"], w["deq"], M, True)
    check_linear(y.cpu().numpy()[:, rows], yo, beta)


@pytest.mark.parametrize("fmt", [0, 1], ids=["nv", "mx"])
def test_dma_path_graph_replays(fmt):
    """Rewrite + product captured in a HIP graph: every replay (with eager
    work between them) equals the eager call bit for bit."""
    import torch
    M, N, K = 96, 2056, 2048
    _, _, blob, act = _setup(fmt, M, N, K, True, 99)
    ws = _ws(fmt, M, N, K, True)
    y_eager = _call(fmt, act, blob, M, N, K, True, ws).clone()
    rs = _rs()
    out = torch.empty(M, N, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        rs.fp4_linear_compensated(act, blob, M, N, K, fmt, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rs.fp4_linear_compensated(act, blob, M, N, K, fmt, out=out, ws=ws)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), y_eager.view(torch.int32))
        _ = _call(fmt, act, blob, M, N, K, True, ws)    # eager work between replays

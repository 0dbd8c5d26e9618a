"""GPU parity of the one-call quantize + linear (rsfp4_*_linear*_from_x): one
launch in which every workgroup quantizes the rows itself (bf16 x, K <= 8192,
MXFP4 or plain NVFP4 with M <= 4), two launches otherwise.  Checked against the oracle
(y within 1e-4 * sum_k |term_k|) and, bit for bit, against the quantize and
linear calls made in turn."""
import numpy as np
import pytest

import oracle
from block_scaled_fp4_act_amd import inputs
from gpu_util import FMT, _first_diff, check_linear, dev_x, sample_channels

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


def _run(x_np, W, fmt, comp, x_bf16=True, bf16_out=False, blob=None):
    """from_x and the two calls on the same inputs; y must agree bit for bit.
    The act buffer starts as a sentinel: afterwards it is untouched (one
    launch) or holds the quantize call's records (two launches)."""
    import torch
    rs = _rs()
    M, K = x_np.shape
    N = W.shape[0]
    if blob is None:
        blob = rs.prepack_weights(torch.from_numpy(W).cuda(), fmt)
    x = dev_x(x_np, x_bf16)
    dt = torch.bfloat16 if bf16_out else torch.float32
    act = torch.full((rs.packed_act_bytes(fmt, M, K, comp),), 0xA5, dtype=torch.uint8, device="cuda")
    y = rs.fp4_linear_from_x(x, blob, N, fmt, comp, out_dtype=dt, act=act)
    act2 = rs.quantize_act_with_residue(x, fmt, with_residue=comp)
    if bf16_out:
        f = rs.fp4_linear_compensated_bf16 if comp else rs.fp4_linear_bf16
    else:
        f = rs.fp4_linear_compensated if comp else rs.fp4_linear
    y2 = f(act2, blob, M, N, K, fmt)
    torch.cuda.synchronize()
    iv = torch.int16 if bf16_out else torch.int32
    yb, y2b = y.view(iv).cpu().numpy(), y2.view(iv).cpu().numpy()
    assert np.array_equal(yb, y2b), _first_diff(yb, y2b)
    a = act.cpu().numpy()
    if not (a == 0xA5).all():
        for u, v in zip(rs.act_views(act, fmt, M, K, comp), rs.act_views(act2, fmt, M, K, comp)):
            un, vn = u.cpu().numpy(), v.cpu().numpy()
            assert np.array_equal(un.view(np.uint8), vn.view(np.uint8)), _first_diff(un, vn)
    return y


CASES = [  # (M, N, K): one launch (bf16 x, B <= 16, K <= 8192) and two-launch shapes
    (1, 512, 512), (2, 72, 160), (3, 1000, 384), (4, 256, 4096), (5, 48, 640), (8, 320, 1024),
    (8, 100, 2080), (6, 16, 32), (4, 80, 8192), (8, 4112, 256), (16, 64, 512), (1, 40, 7936),
    # two launches: 17..32 operand rows, a wide operand, K past 8192
    (12, 64, 256), (17, 264, 384), (40, 130, 160), (4, 72, 12288),
]


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("comp", [True, False])
@pytest.mark.parametrize("MNK", CASES, ids=lambda t: "M%dN%dK%d" % t)
def test_from_x_small_vs_oracle(fmt, comp, MNK):
    M, N, K = MNK
    rng = np.random.default_rng(7 * M + N + 3 * K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    W = inputs.weights(N, K, K + N + 1)
    y = _run(x, W, fmt, comp)
    xin = inputs.round_to_bf16(x)
    q = oracle.quantize_act(xin, fmt, with_residue=comp)
    w = oracle.quantize_weight(W, fmt)
    yo, beta = oracle.linear(q["deq"], w["deq"], M, comp)
    check_linear(y.cpu().numpy(), yo, beta)


def _adversarial(M, K, seed):
    """Rows that exercise the quantizer's corner paths inside the linear: zero,
    tiny, huge, exact E2M1 grid and ties, one dominant outlier."""
    rng = np.random.default_rng(seed)
    rows = [np.zeros(K, np.float32), (rng.standard_normal(K) * 1e-30).astype(np.float32),
            (rng.standard_normal(K) * 1e30).astype(np.float32)]
    e = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    rows.append(np.tile(np.concatenate([e, -e]), K // 16) * np.float32(0.4375))
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    rows.append(np.tile(np.concatenate([ties, -ties]), K // 16))
    w = rng.standard_normal(K).astype(np.float32)
    w[rng.integers(0, K)] = 1e4
    rows.append(w)
    x = np.stack(rows)
    return np.concatenate([x, rng.standard_normal((max(0, M - len(rows)), K)).astype(np.float32)])[:M]


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M", [6, 8])
def test_from_x_adversarial_rows(fmt, M):
    K, N = 1024, 96
    _run(_adversarial(M, K, M), inputs.weights(N, K, 5), fmt, True)
    _run(_adversarial(M, K, M + 1), inputs.weights(N, K, 5), fmt, False)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("MNK", [(4, 96, 4096), (8, 64, 1024), (1, 48, 8192)], ids=lambda t: "M%dN%dK%d" % t)
def test_from_x_fp32_input_and_bf16_output(fmt, MNK):
    M, N, K = MNK
    rng = np.random.default_rng(M + N + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    W = inputs.weights(N, K, 11)
    _run(x, W, fmt, True, x_bf16=False)
    _run(x, W, fmt, True, x_bf16=True, bf16_out=True)
    _run(x, W, fmt, False, x_bf16=False, bf16_out=True)


def _workloads():
    wls = [inputs.ATTN, inputs.ATTN.with_m(1), inputs.MLP_UP, inputs.MLP_DOWN]
    wls += [inputs.LARGE_MLP.with_m(m) for m in (1, 4, 8)]
    wls += [inputs.MX.with_m(m) for m in (1, 8)]
    return wls


@pytest.mark.parametrize("wl", _workloads(), ids=lambda w: f"{w.name}_M{w.M}")
def test_from_x_workload_sampled(wl):
    """Full-size workloads as the bench runs them; sampled output channels
    against the oracle, all of y against the two calls."""
    fmt = FMT[wl.fmt]
    x, W = wl.draw_x(), wl.draw_w()
    y = _run(x, W, fmt, True, x_bf16=wl.bf16)
    rows = sample_channels(wl.N, wl.M, 5)
    xin = inputs.round_to_bf16(x) if wl.bf16 else x
    q = oracle.quantize_act(xin, fmt, with_residue=True)
    w = oracle.quantize_weight(W, fmt, rows=rows)
    yo, beta = oracle.linear(q["deq"], w["deq"], wl.M, True)
    check_linear(y.cpu().numpy()[:, rows], yo, beta)


def test_from_x_graph_replays():
    """Three calls captured in one HIP graph, replayed three times with eager
    work between the replays; every replay equals the eager result."""
    import torch
    rs = _rs()
    M, N, K = 4, 1040, 4096
    W = inputs.weights(N, K, 3)
    blob = rs.prepack_weights(torch.from_numpy(W).cuda(), 0)
    xs = [dev_x(np.random.default_rng(i).standard_normal((M, K)).astype(np.float32), True) for i in range(3)]
    act = torch.empty(rs.packed_act_bytes(0, M, K, True), dtype=torch.uint8, device="cuda")
    ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _ in range(3)]
    eager = [rs.fp4_linear_from_x(x, blob, N, 0, True, act=act).clone() for x in xs]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for x, y in zip(xs, ys):
                rs.fp4_linear_from_x(x, blob, N, 0, True, out=y, act=act)
    torch.cuda.synchronize()
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y.view(torch.int32), e.view(torch.int32)), f"replay {rep}"
        rs.fp4_linear_from_x(xs[rep], blob, N, 0, True, act=act)   # eager work between replays
        torch.cuda.synchronize()


def test_from_x_launch_count():
    """The launch-count query follows the rule: bf16 x, K <= 8192 and MXFP4
    with M <= 4 or plain NVFP4 with M <= 4 run as one launch; compensated
    NVFP4 always as two."""
    import torch
    rs = _rs()
    assert rs.from_x_launches(0, 2, 4096, 4096, True) == 2
    assert rs.from_x_launches(0, 4, 4096, 4096, False) == 1
    assert rs.from_x_launches(0, 8, 4096, 4096, False) == 2
    assert rs.from_x_launches(1, 4, 4096, 4096, True) == 1
    assert rs.from_x_launches(1, 8, 25600, 5120, True) == 2
    assert rs.from_x_launches(0, 1, 4096, 16384, False) == 2         # K past 8192
    assert rs.from_x_launches(0, 1, 4096, 4096, False, x_dtype=torch.float32) == 2
    assert rs.from_x_launches(0, 1, 4096, 100, False) == 0           # K not a multiple of 32

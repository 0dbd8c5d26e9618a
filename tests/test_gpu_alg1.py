"""GPU parity of the paper-numerics NVFP4 quantizer (ResServe, Appendix B.2:
Eq. 8 with a given tensor scale alpha, Algorithm 1's multiplier scale and
residue, alpha shared by x and r) and of the bf16-output linears.  Codes, scale
bytes and tensor scales bit-exact; fp32 outputs within 1e-4 * sum|terms|; bf16
outputs equal to the fp32 result rounded to nearest even."""
import numpy as np
import pytest

import oracle
from block_scaled_fp4_act_amd import inputs
from gpu_util import check_linear, dev_x, _first_diff

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


def _alpha_dev(a):
    import torch
    return torch.tensor([np.float32(a)], dtype=torch.float32, device="cuda")


# ----------------------------------------------------------- tensor alpha --

@pytest.mark.parametrize("wl", [inputs.SMALL, inputs.ATTN, inputs.MLP_DOWN], ids=lambda w: w.name)
def test_tensor_alpha_bitexact(wl):
    import torch
    x = wl.draw_x()
    xin = inputs.round_to_bf16(x) if wl.bf16 else x
    a = _rs().nvfp4_tensor_alpha(dev_x(xin, wl.bf16))
    torch.cuda.synchronize()
    want = oracle.nvfp4_alpha(xin)
    assert a.cpu().numpy().view(np.uint32)[0] == np.float32(want).view(np.uint32)


def test_tensor_alpha_zero_and_large():
    import torch
    rs = _rs()
    assert rs.nvfp4_tensor_alpha(torch.zeros(3, 64, device="cuda")).item() == 0.0
    x = np.zeros((2, 4096), np.float32)
    x[1, 4000] = -2688.0 * 2.0 ** 7
    a = rs.nvfp4_tensor_alpha(dev_x(x, False))
    torch.cuda.synchronize()
    assert a.item() == 2.0 ** 7


# ------------------------------------------------------------- quantize ----

def _check_alpha_quant(xin, alpha, bf16, with_residue=True):
    import torch
    rs = _rs()
    M, K = xin.shape
    act = rs.nvfp4_quantize_act_alpha(dev_x(xin, bf16), _alpha_dev(alpha), with_residue)
    codes, scales, globs = rs.act_views(act, 0, M, K, with_residue)
    torch.cuda.synchronize()
    q = oracle.quantize_act_alg1(xin, alpha, with_residue)
    c, s, g = codes.cpu().numpy(), scales.cpu().numpy(), globs.cpu().numpy()
    assert np.array_equal(c, q["codes"]), _first_diff(c, q["codes"])
    assert np.array_equal(s, q["scales"]), _first_diff(s, q["scales"])
    assert np.array_equal(g.view(np.uint32), q["globals"].view(np.uint32))
    return act, q


@pytest.mark.parametrize("wl", inputs.ALL, ids=lambda w: w.name)
@pytest.mark.parametrize("with_residue", [True, False])
def test_quantize_alpha_workload_bitexact(wl, with_residue):
    x = wl.draw_x() if not wl.x_rows else inputs.activations(
        wl.x_rows, wl.K, wl.x_seed, wl.outlier_frac, wl.outlier_scale, wl.o_seed, wl.bf16)
    xin = inputs.round_to_bf16(x) if wl.bf16 else x
    _check_alpha_quant(xin, oracle.nvfp4_alpha(xin), wl.bf16, with_residue)


@pytest.mark.parametrize("alpha", [1e-3, 0.01, 2.0 ** -5, 0.37, 3.0e-6])
@pytest.mark.parametrize("K", [32, 160, 4096, 14336, 32768])
def test_quantize_alpha_static_scales(alpha, K):
    """Static (calibrated) alphas far from the data's own: block scales
    saturate at 448 or fall to E4M3 subnormals, codes saturate."""
    x = inputs.activations(3, K, K + 1, 0.01, 20.0, 2, False)
    _check_alpha_quant(x, np.float32(alpha), False)


def test_quantize_alpha_edge_rows():
    K = 512
    rng = np.random.default_rng(41)
    rows = [np.zeros(K, np.float32), -np.zeros(K, np.float32)]
    g = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    grid = (rng.choice(g, K) * rng.choice([-1, 1], K)).astype(np.float32)
    rows.append(grid * np.float32(0.01 * 2.25))         # values at multiplier ties
    rows.append((rng.standard_normal(K) * 1e-30).astype(np.float32))
    spike = rng.standard_normal(K).astype(np.float32)
    spike[3] = 4.0e5
    rows.append(spike)
    x = np.stack(rows)
    for alpha in (np.float32(0.01), oracle.nvfp4_alpha(x), np.float32(0.0), np.float32(1e-38)):
        _check_alpha_quant(x, alpha, False)


def test_golden_alg1_on_gpu():
    """The hand-worked page example, through the kernel."""
    from conftest import load_golden
    gd = load_golden("nvfp4_alg1_worked.txt")
    x = np.zeros((1, 32), np.float32)
    x[0, :16] = gd["x"]
    act, q = _check_alpha_quant(x, np.float32(gd["alpha"][0]), False)
    assert np.array_equal(q["codes"][0, :8], gd["codes"])
    assert np.array_equal(q["codes"][1, :8], gd["res_codes"])


# --------------------------------------------------------------- linear ----

@pytest.mark.parametrize("M,N,K", [(1, 512, 512), (4, 264, 4096), (8, 100, 1024), (40, 130, 768)])
def test_alpha_linear_compensated(M, N, K):
    import torch
    rs = _rs()
    x = inputs.activations(M, K, M + K, 0.01, 20.0, 3, True)
    W = inputs.weights(N, K, 9)
    xin = inputs.round_to_bf16(x)
    alpha = oracle.nvfp4_alpha(xin)
    blob = rs.prepack_weights(torch.from_numpy(W).cuda(), 0)
    act = rs.nvfp4_quantize_act_alpha(dev_x(xin, True), _alpha_dev(alpha), True)
    y = rs.fp4_linear_compensated(act, blob, M, N, K, 0)
    torch.cuda.synchronize()
    q = oracle.quantize_act_alg1(xin, alpha, True)
    yo, beta = oracle.linear(q["deq"], oracle.quantize_weight(W, 0)["deq"], M, True)
    check_linear(y.cpu().numpy(), yo, beta)


BF16_CASES = [(1, 512, 512), (4, 300, 4096), (16, 64, 1024), (40, 130, 768), (129, 72, 512),
              (4, 64, 20480)]


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("comp", [True, False])
@pytest.mark.parametrize("MNK", BF16_CASES, ids=lambda t: "M%dN%dK%d" % t)
def test_linear_bf16_output(fmt, comp, MNK):
    import torch
    rs = _rs()
    M, N, K = MNK
    x = inputs.activations(M, K, M * 3 + K, 0.01, 20.0, 3, True)
    W = inputs.weights(N, K, K + N)
    xin = inputs.round_to_bf16(x)
    blob = rs.prepack_weights(torch.from_numpy(W).cuda(), fmt)
    act = rs.quantize_act_with_residue(dev_x(xin, True), fmt, comp)
    f32 = rs.fp4_linear_compensated if comp else rs.fp4_linear
    b16 = rs.fp4_linear_compensated_bf16 if comp else rs.fp4_linear_bf16
    y32 = f32(act, blob, M, N, K, fmt)
    y16 = b16(act, blob, M, N, K, fmt)
    torch.cuda.synchronize()
    assert y16.dtype == torch.bfloat16
    if K <= 16384 or 2 * M > 32:
        # same kernel and summation order: bf16 = RNE(fp32 result) exactly
        assert torch.equal(y16, y32.to(torch.bfloat16))
    q = oracle.quantize_act(xin, fmt, with_residue=comp)
    yo, beta = oracle.linear(q["deq"], oracle.quantize_weight(W, fmt)["deq"], M, comp)
    err = np.abs(y16.float().cpu().numpy().astype(np.float64) - yo)
    assert np.all(err <= 2.0 ** -8 * np.abs(yo) + 1e-4 * beta)

"""GPU parity of selective compensation (K-Ext; ResServe Section 5.3, Eq. 6 and
Appendix B.1, Eq. 7 / Algorithm 1): calibration sums, masks, the [W | W_S]
prepack and the extended activation records must equal the oracle's bit for
bit; the product over K_eff must satisfy |y_gpu - y_oracle| <= 1e-4 * sum|terms|
elementwise."""
import numpy as np
import pytest

import oracle
from block_scaled_fp4_act_amd import inputs
from gpu_util import FMT, check_linear, dev_x, _first_diff, sample_channels

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


def _t(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ---------------------------------------------------------- calibration ----

@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("TK", [(64, 4096), (37, 5120), (5, 14336), (200, 72)])
def test_channel_abs_sum_bitexact(bf16, TK):
    import torch
    T, K = TK
    x = inputs.activations(T, K, 11 + T, 0.01, 20.0, 12, bf16)
    s = _rs().channel_abs_sum(dev_x(x, bf16))
    torch.cuda.synchronize()
    want = oracle.channel_abs_sum(x)
    got = s.cpu().numpy()
    assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), _first_diff(got, want)


def test_channel_abs_sum_accumulates_batches():
    import torch
    rs = _rs()
    a = inputs.activations(19, 512, 1, 0.01, 20.0, 2, True)
    b = inputs.activations(23, 512, 3, 0.01, 20.0, 2, True)
    s = rs.channel_abs_sum(dev_x(a, True))
    rs.channel_abs_sum(dev_x(b, True), out=s, accumulate=True)
    torch.cuda.synchronize()
    want = oracle.channel_abs_sum(np.concatenate([a, b]))
    assert np.array_equal(s.cpu().numpy().view(np.uint64), want.view(np.uint64))


@pytest.mark.parametrize("k", [1, 2, 4, 8])
@pytest.mark.parametrize("K", [64, 4096, 14336])
def test_select_bitexact(k, K):
    import torch
    rng = np.random.default_rng(K + k)
    score = rng.integers(0, 5, size=K).astype(np.float64)        # many ties
    score[: K // 2] += rng.standard_normal(K // 2)
    m = _rs().kext_select(_t(score), k)
    torch.cuda.synchronize()
    want = oracle.kext_select(score, k)
    assert np.array_equal(m.cpu().numpy(), want), _first_diff(m.cpu().numpy(), want)


def test_select_from_calibration_end_to_end():
    import torch
    rs = _rs()
    w = inputs.LARGE_MLP
    xc = inputs.calibration_rows(w)
    m = rs.kext_select(rs.channel_abs_sum(dev_x(xc, True)), 2)
    torch.cuda.synchronize()
    want = oracle.kext_select(oracle.channel_abs_sum(xc), 2)
    assert np.array_equal(m.cpu().numpy(), want)


# -------------------------------------------------------------- prepack ----

def _oracle_weight_ext(W, fmt, masks, k, rows=None):
    """Oracle [W | W_S] quantized as one tensor; with rows, only those rows
    (its NVFP4 tensor scale is W's: the appended columns repeat W's values)."""
    if rows is None:
        return oracle.quantize_weight(oracle.kext_extend_weight(W, masks, k), fmt)
    s_gw = oracle.nvfp4_global_scale(oracle.absmax(W)) if fmt == 0 else 0.0
    out = oracle.quantize_weight_rows(oracle.kext_extend_weight(W[np.asarray(rows)], masks, k), fmt, s_gw)
    out["s_g"] = np.float32(s_gw)
    return out


def _prepack_kext_check(W, fmt, masks, k, rows=None, bf16=False):
    import torch
    rs = _rs()
    N, K = W.shape
    KE = rs.kext_dim(K, k)
    Wd = _t(W)
    if bf16:
        Wd = Wd.to(torch.bfloat16)
    blob = rs.prepack_weights_kext(Wd, fmt, _t(masks), k)
    codes, scales, s_g = rs.unpack_weights_canonical(blob, fmt, N, KE)
    torch.cuda.synchronize()
    q = _oracle_weight_ext(W, fmt, masks, k, rows)
    sel = slice(None) if rows is None else torch.as_tensor(np.asarray(rows)).cuda()
    c = codes[sel].cpu().numpy()
    s = scales[sel].cpu().numpy()
    assert np.array_equal(c, q["codes"]), _first_diff(c, q["codes"])
    assert np.array_equal(s, q["scales"]), _first_diff(s, q["scales"])
    if fmt == 0:
        assert s_g.cpu().numpy()[0].view(np.uint32) == np.float32(q["s_g"]).view(np.uint32)
    return blob


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("k", [1, 2, 4, 8])
@pytest.mark.parametrize("NK", [(72, 256), (33, 1024), (16, 512)])
def test_prepack_kext_bitexact_small(fmt, k, NK):
    N, K = NK
    W = inputs.weights(N, K, 7 + k)
    _prepack_kext_check(W, fmt, inputs.random_masks(K, k, 3 + k), k)


def test_prepack_kext_bf16():
    W = inputs.round_to_bf16(inputs.weights(40, 512, 4))
    for fmt in (0, 1):
        _prepack_kext_check(W, fmt, inputs.random_masks(512, 2, 5), 2, bf16=True)


@pytest.mark.parametrize("wl,k", [(inputs.LARGE_MLP, 1), (inputs.LARGE_MLP, 4), (inputs.MX, 2)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_prepack_kext_workload_sampled(wl, k):
    W = _weights(wl)
    rows = np.sort(np.random.default_rng(5).choice(wl.N, 64, replace=False))
    rows[-1] = wl.N - 1
    masks = inputs.random_masks(wl.K, k, 17)
    _prepack_kext_check(W, FMT[wl.fmt], masks, k, rows=rows)


# ------------------------------------------------------------- quantize ----

def _quant_kext_check(x, fmt, masks, k, bf16):
    import torch
    rs = _rs()
    M, K = x.shape
    KE = rs.kext_dim(K, k)
    xin = inputs.round_to_bf16(x) if bf16 else np.ascontiguousarray(x, np.float32)
    act = rs.quantize_act_kext(dev_x(xin, bf16), fmt, _t(masks), k)
    codes, scales, globs = rs.act_views(act, fmt, M, KE, with_residue=False)
    torch.cuda.synchronize()
    q = oracle.kext_quantize_act(xin, fmt, masks, k)
    c, s, g = codes.cpu().numpy(), scales.cpu().numpy(), globs.cpu().numpy()
    assert np.array_equal(c, q["codes"]), _first_diff(c, q["codes"])
    assert np.array_equal(s, q["scales"]), _first_diff(s, q["scales"])
    assert np.array_equal(g.view(np.uint32), q["globals"].view(np.uint32)), _first_diff(g, q["globals"])
    return act, q


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("k", [1, 2, 4, 8])
@pytest.mark.parametrize("K", [256, 768, 4096, 5120, 8192, 14336])
def test_quantize_kext_bitexact(fmt, k, K):
    if oracle.kext_dim(K, k) > 32768 or (K // 8 * k) % 32:
        pytest.skip("no whole-block extension of this width")
    x = inputs.activations(6, K, K + k, 0.01, 20.0, 3, False)
    masks = inputs.random_masks(K, k, K * 10 + k)
    _quant_kext_check(x, fmt, masks, k, bf16=(K % 512 == 0))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("k", [1, 8])
def test_quantize_kext_longest_rows(fmt, k):
    """K_eff = 32768 (k = 8) and the four-chunks-per-thread launch (K > 16384)."""
    K = 16384 if k == 8 else 24576
    x = inputs.activations(2, K, 5, 0.005, 30.0, 6, True)
    _quant_kext_check(x, fmt, inputs.random_masks(K, k, 8), k, bf16=True)


@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_kext_edge_rows(fmt):
    """Zero rows, -0 rows, exactly representable rows (zero residues), one
    huge channel, tiny values: the extension's scales and codes still match."""
    K, k = 512, 2
    rng = np.random.default_rng(31)
    rows = [np.zeros(K, np.float32), -np.zeros(K, np.float32)]
    base = rng.standard_normal((1, K)).astype(np.float32)
    rows.append(oracle.quantize_act(base, fmt, with_residue=False)["deq"][0])
    spike = rng.standard_normal(K).astype(np.float32)
    spike[77] = 3.0e4
    rows.append(spike)
    rows.append((rng.standard_normal(K) * 1e-30).astype(np.float32))
    x = np.stack(rows).astype(np.float32)
    _quant_kext_check(x, fmt, inputs.random_masks(K, k, 2), k, bf16=False)


# --------------------------------------------------------------- linear ----

def _kext_pipeline(x, W, fmt, masks, k, bf16):
    import torch
    rs = _rs()
    M = x.shape[0]
    N, K = W.shape
    KE = rs.kext_dim(K, k)
    m = _t(masks)
    blob = rs.prepack_weights_kext(_t(W), fmt, m, k)
    xin = inputs.round_to_bf16(x) if bf16 else x
    act = rs.quantize_act_kext(dev_x(xin, bf16), fmt, m, k)
    y = rs.fp4_linear(act, blob, M, N, KE, fmt)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _oracle_kext(x, W, fmt, masks, k, bf16, rows=None):
    xin = inputs.round_to_bf16(x) if bf16 else x
    q = oracle.kext_quantize_act(xin, fmt, masks, k)
    w = _oracle_weight_ext(W, fmt, masks, k, rows)
    return oracle.linear(q["deq"], w["deq"], x.shape[0], False)


_W_CACHE = {}


def _weights(wl):
    key = (wl.N, wl.K, wl.w_seed)
    if key not in _W_CACHE:
        _W_CACHE.clear()
        _W_CACHE[key] = wl.draw_w()
    return _W_CACHE[key]


KEXT_CASES = [  # (M, N, K, k): narrow and tiled kernels, ragged N, K tails of a quad,
    # and (NVFP4) a tiled product split in K (K_eff = 5120: 40 steps in slices of 16, 16, 8)
    (1, 512, 512, 1), (4, 264, 512, 2), (8, 100, 1024, 4), (16, 72, 256, 8),
    (33, 130, 768, 2), (64, 128, 256, 4), (129, 300, 512, 1), (200, 64, 1024, 2),
    (64, 200, 4096, 2),
]


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("case", KEXT_CASES, ids=lambda t: "M%dN%dK%dk%d" % t)
def test_kext_linear_small_full(fmt, case):
    M, N, K, k = case
    rng = np.random.default_rng(M * 7 + N + K + k)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    W = inputs.weights(N, K, K + N + k)
    masks = oracle.kext_select(oracle.channel_abs_sum(x), k)
    y = _kext_pipeline(x, W, fmt, masks, k, True)
    yo, beta = _oracle_kext(x, W, fmt, masks, k, True)
    check_linear(y, yo, beta)


def _kext_workloads():
    out = []
    for m in (8, 128):
        for k in inputs.KEXT_K:
            out.append((inputs.LARGE_MLP.with_m(m), k))
    for m in (8, 256):
        for k in inputs.KEXT_K:
            out.append((inputs.MX.with_m(m), k))
    out.append((inputs.MLP_DOWN, 2))      # K_eff = 17920: past the narrow kernel's K
    return out


@pytest.mark.parametrize("wl,k", _kext_workloads(),
                         ids=lambda v: f"{v.name}_M{v.M}" if hasattr(v, "name") else f"k{v}")
def test_kext_linear_workload_sampled(wl, k):
    """Full-size workloads with calibration-chosen masks, launched as the bench
    launches them; the oracle computes a sample of output channels."""
    fmt = FMT[wl.fmt]
    x, W = wl.draw_x(), _weights(wl)
    masks = oracle.kext_select(oracle.channel_abs_sum(inputs.calibration_rows(wl)), k)
    y = _kext_pipeline(x, W, fmt, masks, k, wl.bf16)
    rows = sample_channels(wl.N, wl.M, 9)
    yo, beta = _oracle_kext(x, W, fmt, masks, k, wl.bf16, rows=rows)
    check_linear(y[:, rows], yo, beta)


@pytest.mark.parametrize("fmt", [0, 1])
def test_kext_full_ratio_matches_compensated_mxfp4(fmt):
    """k = 8: MXFP4 K-Ext is the full-residue product (same codes in another
    order of the sum); NVFP4 K-Ext differs only in the residue's tensor scale,
    and is checked against its own oracle."""
    import torch
    rs = _rs()
    M, N, K = 8, 256, 1024
    x = inputs.activations(M, K, 3, 0.01, 20.0, 4, True)
    W = inputs.weights(N, K, 5)
    masks = np.full(K // 8, 0xFF, np.uint8)
    yk = _kext_pipeline(x, W, fmt, masks, 8, True)
    if fmt == 1:
        blob = rs.prepack_weights(_t(W), fmt)
        act = rs.quantize_act_with_residue(dev_x(inputs.round_to_bf16(x), True), fmt, True)
        ym = rs.fp4_linear_compensated(act, blob, M, N, K, fmt)
        torch.cuda.synchronize()
        yo, beta = oracle.linear(oracle.quantize_act(inputs.round_to_bf16(x), fmt, True)["deq"],
                                 oracle.quantize_weight(W, fmt)["deq"], M, True)
        check_linear(yk, yo, beta)
        check_linear(ym.cpu().numpy(), yo, beta)
    else:
        yo, beta = _oracle_kext(x, W, fmt, masks, 8, True)
        check_linear(yk, yo, beta)

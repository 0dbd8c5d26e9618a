"""Pins of the oracle's compensated linear (ResServe, Section 4.2 Eq. 1 and
Section 4.3 Eq. 2: Y = X^ W^ + R^ W^ as the stacked product [X^; R^] W^ with the
Fold Y_j = Z_j + Z_{M+j}) against exact rational brute force, an independent
float64 matmul, a reduction to pure dequantization, and the error ordering the
method exists for.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest

from block_scaled_fp4_act_amd import inputs


def _bruteforce(dx, dw, M, comp):
    N, K = dw.shape
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(float(dx[m, k])) * Fraction(float(dw[n, k]))
                if comp:
                    s += Fraction(float(dx[M + m, k])) * Fraction(float(dw[n, k]))
            y[m, n] = float(s)
    return y


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("comp", [False, True])
def test_linear_bruteforce_tiny(orc, fmt, comp):
    rng = np.random.default_rng(21 + fmt)
    M, N, K = 2, 3, 64
    x = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    q = orc.quantize_act(x, fmt, with_residue=comp)
    w = orc.quantize_weight(W, fmt)
    y, beta = orc.linear(q["deq"], w["deq"], M, comp)
    yb = _bruteforce(q["deq"], w["deq"], M, comp)
    # fp64 accumulation of exact products: within a few ulps of the exact sum
    assert np.all(np.abs(y - yb) <= 1e-13 * beta)
    # beta is the sum of |products|
    bb = np.abs(q["deq"][:M]).astype(np.float64) @ np.abs(w["deq"]).T.astype(np.float64)
    if comp:
        bb += np.abs(q["deq"][M:]).astype(np.float64) @ np.abs(w["deq"]).T.astype(np.float64)
    assert np.allclose(beta, bb, rtol=1e-12, atol=0)


@pytest.mark.parametrize("fmt", [0, 1])
def test_linear_matches_matmul(orc, fmt):
    rng = np.random.default_rng(3)
    M, N, K = 4, 96, 512
    x = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    q = orc.quantize_act(x, fmt)
    w = orc.quantize_weight(W, fmt)
    y, beta = orc.linear(q["deq"], w["deq"], M, True)
    dx = q["deq"].astype(np.float64)
    dw = w["deq"].astype(np.float64)
    ref = dx[:M] @ dw.T + dx[M:] @ dw.T
    assert np.all(np.abs(y - ref) <= 1e-12 * beta)
    yp, _ = orc.linear(q["deq"][:M], w["deq"], M, False)
    assert np.all(np.abs(yp - dx[:M] @ dw.T) <= 1e-12 * beta)


@pytest.mark.parametrize("fmt,diag", [(0, 2.625), (1, 4.0)])
def test_identity_weight_is_dequantization(orc, fmt, diag):
    """With W = c*I and c exactly representable (NVFP4: 2.625 gives s_gw = 2^-10
    and an effective scale 0.4375; MXFP4: 4 gives X = 1), the weights dequantize
    exactly and the compensated linear reduces to c * (x^ + r^) elementwise."""
    K = 256
    W = np.eye(K, dtype=np.float32) * np.float32(diag)
    w = orc.quantize_weight(W, fmt)
    assert np.array_equal(w["deq"], W)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, K)).astype(np.float32)
    q = orc.quantize_act(x, fmt)
    y, _ = orc.linear(q["deq"], w["deq"], 3, True)
    d = q["deq"].astype(np.float64)
    assert np.array_equal(y, d[:3] * diag + d[3:] * diag)
    yp, _ = orc.linear(q["deq"][:3], w["deq"], 3, False)
    assert np.array_equal(yp, d[:3] * diag)


def test_exact_activations_comp_equals_plain(orc):
    """A representable x has r = 0, so compensated == plain bit for bit."""
    e = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, 0, -0.5, -1, -1.5, -2, -3, -4, -6], np.float32) * np.float32(0.4375)
    x = np.tile(e, (2, 4))
    W = inputs.weights(16, 64, 0)
    q = orc.quantize_act(x, 0)
    w = orc.quantize_weight(W, 0)
    yc, _ = orc.linear(q["deq"], w["deq"], 2, True)
    yp, _ = orc.linear(q["deq"][:2], w["deq"], 2, False)
    assert np.array_equal(yc, yp)


def _nmse(y, ref):
    return float(((y - ref) ** 2).sum() / (ref ** 2).sum())


@pytest.mark.parametrize("fmt", [0, 1])
def test_compensation_lowers_error_exact_weights(orc, fmt):
    """With exactly representable weights only activation error remains, and
    compensation must lower the output NMSE against x W^T (pooled NMSE as in
    ResServe Appendix C.2)."""
    rng = np.random.default_rng(31)
    M, N, K = 4, 64, 512
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, 5, replace=False)] *= 20
    # weights drawn from the FP4 grid times a power of two: exact in both formats
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    W = (grid[rng.integers(0, 8, (N, K))] * np.where(rng.random((N, K)) < 0.5, -1, 1)).astype(np.float32)
    W[:, ::32] = 6.0  # every 32-block reaches 6, so MXFP4 picks X = 1
    w = orc.quantize_weight(W, fmt)
    if fmt == 1:
        assert np.array_equal(w["deq"], W)
    q = orc.quantize_act(x, fmt)
    ref = x.astype(np.float64) @ w["deq"].astype(np.float64).T
    yc, _ = orc.linear(q["deq"], w["deq"], M, True)
    yp, _ = orc.linear(q["deq"][:M], w["deq"], M, False)
    assert _nmse(yc, ref) < 0.25 * _nmse(yp, ref)


@pytest.mark.parametrize("wl", [inputs.SMALL, inputs.MX.with_m(4)])
def test_compensation_lowers_error_on_workload(orc, wl):
    """On the seeded workloads (weight error included, as in ResServe Table 3's
    protocol), compensation lowers pooled NMSE against the fp32 product."""
    if wl.N * wl.K > 4096 * 1024:
        wl = inputs.Workload(wl.name, wl.fmt, wl.M, wl.K, 512, wl.w_seed, wl.x_seed, wl.o_seed,
                             wl.outlier_frac, wl.outlier_scale, wl.bf16, wl.x_rows)
    fmt = 0 if wl.fmt == "nvfp4" else 1
    x, W = wl.draw_x(), wl.draw_w()
    q = orc.quantize_act(x, fmt)
    w = orc.quantize_weight(W, fmt)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    yc, _ = orc.linear(q["deq"], w["deq"], wl.M, True)
    yp, _ = orc.linear(q["deq"][:wl.M], w["deq"], wl.M, False)
    assert _nmse(yc, ref) < _nmse(yp, ref)


def test_tiny_grid_bruteforce_error_order(orc):
    """Brute force over many tiny rows drawn from a small grid: the compensated
    operand is never farther from x than the plain one, elementwise."""
    rng = np.random.default_rng(41)
    vals = np.array([-7, -3.3, -1, -0.2, 0, 0.1, 0.9, 2.2, 5.1, 11], np.float32)
    for fmt in (0, 1):
        for _ in range(50):
            x = vals[rng.integers(0, len(vals), (1, 32))]
            q = orc.quantize_act(x, fmt)
            e_plain = np.abs(x.astype(np.float64) - q["deq"][0])
            e_comp = np.abs(x.astype(np.float64) - q["deq"][0] - q["deq"][1])
            assert (e_comp <= e_plain).all()


def test_threaded_timing_build_same_bits(orc):
    """The OpenMP timing build of the oracle (the linear's channels and the
    weight rows spread over threads) returns the plain build's bits."""
    rng = np.random.default_rng(17)
    x = inputs.activations(3, 1024, 5, 0.01, 20.0, 6, True)
    W = inputs.weights(96, 1024, 8)
    for fmt in (0, 1):
        q = orc.quantize_act(x, fmt, True)
        w1 = orc.quantize_weight(W, fmt)
        w8 = orc.quantize_weight(W, fmt, threads=True)
        assert np.array_equal(w1["codes"], w8["codes"]) and np.array_equal(w1["scales"], w8["scales"])
        y1, b1 = orc.linear(q["deq"], w1["deq"], 3, True)
        y8, b8 = orc.linear(q["deq"], w8["deq"], 3, True, threads=True)
        assert np.array_equal(y1, y8) and np.array_equal(b1, b8)
    assert orc.threads() >= 1
    del rng

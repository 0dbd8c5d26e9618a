"""Pins of the oracle's paper-numerics NVFP4 quantizer (ResServe, Appendix B.2:
Eq. 8 with a given tensor scale alpha, and Algorithm 1: the block scale from
(Max/6)/alpha, the multiplier scale 1/(alpha S_b), codes of x * scale and the
residue x - e / scale, the residue sharing alpha).  CPU only."""
import numpy as np
import pytest

from conftest import load_golden


def test_golden_alg1(orc):
    g = load_golden("nvfp4_alg1_worked.txt")
    alpha = np.float32(g["alpha"][0])
    q = orc.quantize_row_alg1(g["x"], alpha)
    assert np.array_equal(q["scales"], g["scales"])
    assert np.array_equal(q["codes"], g["codes"])
    assert np.array_equal(q["resid"], g["resid"])
    r = orc.quantize_row_alg1(q["resid"], alpha)
    assert np.array_equal(r["scales"], g["res_scales"])
    assert np.array_equal(r["codes"], g["res_codes"])
    # the stacked form: rows [x; r] with alpha in every record
    qa = orc.quantize_act_alg1(g["x"][None, :], alpha, with_residue=True)
    assert np.array_equal(qa["codes"][0], g["codes"]) and np.array_equal(qa["codes"][1], g["res_codes"])
    assert np.all(qa["globals"] == alpha)
    assert np.array_equal(qa["resid"][0], g["resid"])


def test_alpha_closed_form(orc):
    for k in range(-20, 21, 5):
        amax = np.float32(2688.0 * 2.0 ** k)      # 6 * 448 * 2^k
        x = np.zeros(64, np.float32)
        x[17] = -amax
        assert orc.nvfp4_alpha(x) == np.float32(2.0 ** k)
    assert orc.nvfp4_alpha(np.zeros(32, np.float32)) == 0.0


def _pow2_case(seed, K=256):
    """Rows whose every block maximum is 6 * alpha * 2^j (so S_b is a power of
    two) with a power-of-two alpha: all scalings are exact."""
    rng = np.random.default_rng(seed)
    alpha = np.float32(2.0 ** -7)
    x = (rng.standard_normal(K) * 0.5).astype(np.float32)
    for b in range(K // 16):
        j = int(rng.integers(-3, 4))
        blk = x[16 * b:16 * b + 16]
        blk[:] = np.clip(blk, -5.9, 5.9) * np.float32(alpha * 2.0 ** j)
        blk[int(rng.integers(16))] = np.float32(6.0 * alpha * 2.0 ** j)
    return x, alpha


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_power_of_two_scales_match_division_path(orc, seed):
    """With alpha and every S_b powers of two, scale = 1/(alpha S_b) is exact,
    x * scale = x / s~ and e / scale = s~ e, so Algorithm 1 gives the codes,
    scale bytes and exact residue x - deq of the division path (Eqs. 9-10)."""
    x, alpha = _pow2_case(seed)
    q = orc.quantize_row_alg1(x, alpha)
    codes = np.zeros(x.size // 2, np.uint8)
    scales = np.zeros(x.size // 16, np.uint8)
    deq = np.zeros(x.size, np.float32)
    orc.lib().oracle_nvfp4_quantize_row(orc.oracle._p(x), x.size, float(alpha), orc.oracle._p(codes),
                                        orc.oracle._p(scales), orc.oracle._p(deq))
    assert np.array_equal(q["scales"], scales)
    assert np.array_equal(q["codes"], codes)
    assert np.array_equal(q["deq"], deq)
    assert np.array_equal(q["resid"], x - deq)


def test_codes_differ_from_division_only_at_ties(orc):
    """On random data with a data-derived alpha, the multiplier's codes equal
    E2M1_RNE(x / s~) except where x / s~ lies within 2^-21 (relative) of a
    rounding tie of the E2M1 grid."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal(16 * 4096).astype(np.float32)
    x[::97] *= 20
    alpha = orc.nvfp4_alpha(x)
    q = orc.quantize_row_alg1(x, alpha)
    sb = np.array([orc.e4m3_value(int(b)) for b in range(256)], np.float32)[q["scales"]]
    st = (np.float32(alpha) * sb).astype(np.float32)
    st16 = np.repeat(st, 16)
    u = (x.astype(np.float64) / st16.astype(np.float64))
    codes = orc.unpack_codes(q["codes"][None, :], x.size)[0]
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    mag = np.array([orc.e2m1_encode_mag(float(v)) for v in np.abs(u).astype(np.float32)])
    diff = np.nonzero((codes & 7) != mag)[0]
    assert diff.size < 20
    for i in diff:
        rel = np.min(np.abs(np.abs(u[i]) - ties) / ties)
        assert rel < 2.0 ** -21, (i, u[i])


def test_residue_bounded_by_half_step(orc):
    """|r| <= s~ (the largest half-step of the E2M1 grid is 1, between 4 and 6)
    wherever x * scale does not saturate."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal(16 * 512).astype(np.float32)
    alpha = orc.nvfp4_alpha(x)
    q = orc.quantize_row_alg1(x, alpha)
    sb = np.array([orc.e4m3_value(int(b)) for b in range(256)], np.float32)[q["scales"]]
    st16 = np.repeat((np.float32(alpha) * sb).astype(np.float32), 16)
    assert np.all(np.abs(q["resid"]) <= st16 * 1.0001)


def test_zero_block_and_zero_alpha(orc):
    x = np.zeros(32, np.float32)
    x[16:] = np.linspace(-1, 1, 16, dtype=np.float32)
    q = orc.quantize_row_alg1(x, np.float32(0.01))
    assert q["scales"][0] == 0 and np.all(q["codes"][:8] == 0)
    assert np.array_equal(q["resid"][:16], x[:16])
    q0 = orc.quantize_row_alg1(x, np.float32(0.0))   # s/alpha = inf -> 448, scale 0
    assert np.all((q0["codes"] & 0x77) == 0) and np.array_equal(q0["resid"], x)


def test_alg1_compensation_reduces_error(orc):
    """The compensated product with the shared-alpha residue beats plain."""
    from block_scaled_fp4_act_amd import inputs
    x = inputs.activations(8, 512, 3, 0.01, 20.0, 4, True)
    W = inputs.weights(64, 512, 5)
    alpha = orc.nvfp4_alpha(x)
    q = orc.quantize_act_alg1(x, alpha, with_residue=True)
    w = orc.quantize_weight(W, 0)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    yp, _ = orc.linear(q["deq"][:8], w["deq"], 8, False)
    yc, _ = orc.linear(q["deq"], w["deq"], 8, True)
    e = lambda y: np.sum((y - ref) ** 2) / np.sum(ref ** 2)
    assert e(yc) < 0.7 * e(yp)

"""Pins of the oracle's codecs and row quantizers against what the ResServe page
(arXiv 2611.08713) fixes: the E2M1 magnitudes and maxima of Section 2 / Figure 1,
the scale rules of Appendix B.2 (Eqs. 8-10), the residue of Section 2, and
closed-form properties of round-to-nearest-even.  CPU only."""
import math
import struct

import numpy as np
import pytest

from conftest import load_golden

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def f32(v):
    return struct.unpack("<f", struct.pack("<f", v))[0]


def nextup(v):
    return float(np.nextafter(np.float32(v), np.float32(np.inf)))


def nextdown(v):
    return float(np.nextafter(np.float32(v), np.float32(-np.inf)))


# ---------------------------------------------------------------- E2M1 ----

def test_e2m1_values_and_roundtrip(orc):
    for c in range(16):
        v = orc.e2m1_value(c)
        mag = E2M1[c & 7]
        assert abs(v) == mag
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)
    for c in range(8):  # the eight magnitudes round-trip exactly
        assert orc.e2m1_encode_mag(E2M1[c]) == c


def test_e2m1_ties_and_neighbours(orc):
    for lo in range(7):
        mid = (E2M1[lo] + E2M1[lo + 1]) / 2  # exact in binary32
        even = lo if lo % 2 == 0 else lo + 1
        assert orc.e2m1_encode_mag(mid) == even, mid
        assert orc.e2m1_encode_mag(nextdown(mid)) == lo
        assert orc.e2m1_encode_mag(nextup(mid)) == lo + 1


def test_e2m1_saturation_and_specials(orc):
    for u in (6.0, nextup(6.0), 7.0, 1e30, float("inf")):
        assert orc.e2m1_encode_mag(u) == 7
    assert orc.e2m1_encode_mag(float("nan")) == 0
    assert orc.e2m1_encode_mag(0.0) == 0
    assert orc.e2m1_encode_mag(1e-45) == 0


# ---------------------------------------------------------------- E4M3 ----

def _e4m3_positive_grid():
    """All finite non-negative E4M3FN values from the format's structure:
    subnormals k*2^-9 (k=0..7) and normals (8+m)*2^(e-10), e=1..15, with
    (e=15, m=7) reserved for NaN."""
    vals = [k * 2.0 ** -9 for k in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append((8 + m) * 2.0 ** (e - 10))
    return vals


def test_e4m3_decode_matches_structure(orc):
    grid = _e4m3_positive_grid()
    assert len(grid) == 127
    for c in range(127):
        assert orc.e4m3_value(c) == grid[c]
        assert orc.e4m3_value(c | 0x80) == -grid[c]
    assert math.isnan(orc.e4m3_value(0x7F)) and math.isnan(orc.e4m3_value(0xFF))
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x08) == 2.0 ** -6
    assert orc.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_encode_identity_ties_neighbours(orc):
    grid = _e4m3_positive_grid()
    for c in range(127):
        assert orc.e4m3_encode(grid[c]) == (c if c else 0)
    for c in range(126):
        mid = (grid[c] + grid[c + 1]) / 2
        assert f32(mid) == mid  # 5 significant bits: exact in binary32
        even = c if c % 2 == 0 else c + 1
        assert orc.e4m3_encode(mid) == even
        if c > 0 or nextdown(mid) > 0:
            assert orc.e4m3_encode(nextdown(mid)) == c
        assert orc.e4m3_encode(nextup(mid)) == c + 1


def test_e4m3_saturation_and_specials(orc):
    for t in (448.0, 464.0, 479.0, 1e10, float("inf")):
        assert orc.e4m3_encode(t) == 0x7E
    for t in (0.0, -0.0, -1.0, float("nan")):
        assert orc.e4m3_encode(t) == 0
    rng = np.random.default_rng(7)
    ts = np.exp(rng.uniform(-12, 8, 4000)).astype(np.float32)
    codes = {orc.e4m3_encode(float(t)) for t in ts}
    assert 0x7F not in codes and max(codes) <= 0x7E


def test_e4m3_is_nearest_bruteforce(orc):
    """Brute force: the chosen code minimizes |t - value| on random arguments."""
    grid = np.array(_e4m3_positive_grid())
    rng = np.random.default_rng(11)
    for t in np.exp(rng.uniform(-9, 6.2, 2000)).astype(np.float32):
        c = orc.e4m3_encode(float(t))
        d = np.abs(grid - float(t))
        assert d[c] == d.min()


# ---------------------------------------------------------------- E8M0 ----

def test_e8m0_rule(orc):
    for j in range(-120, 127):
        a = 2.0 ** j
        assert orc.e8m0_for_amax(a) == j - 2 + 127
        if j > -126:
            assert orc.e8m0_for_amax(nextdown(a)) == j - 3 + 127
        assert orc.e8m0_for_amax(a * 1.999) == j - 2 + 127
    assert orc.e8m0_for_amax(0.0) == 0
    assert orc.e8m0_for_amax(2.0 ** -149) == 0      # clamped at 2^-127
    assert orc.e8m0_for_amax(2.0 ** -130) == 0
    assert orc.e8m0_for_amax(f32(3.4e38)) == 127 + 127 - 2
    for b in range(255):
        assert orc.e8m0_value(b) == 2.0 ** (b - 127)


# ------------------------------------------------------ golden examples ----

def _row_q(orc, x, fmt):
    q = orc.quantize_act(x.reshape(1, -1), fmt, with_residue=True)
    return q


@pytest.mark.parametrize("name,fmt", [("nvfp4_roundtrip.txt", 0), ("mxfp4_roundtrip.txt", 1),
                                      ("nvfp4_worked.txt", 0), ("mxfp4_worked.txt", 1)])
def test_golden(orc, name, fmt):
    g = load_golden(name)
    x = g["x"]
    q = _row_q(orc, x, fmt)
    assert (q["codes"][0] == g["codes"]).all()
    assert (q["scales"][0] == g["scales"]).all()
    assert (q["codes"][1] == g["res_codes"]).all()
    assert (q["scales"][1] == g["res_scales"]).all()
    if "s_g" in g:
        assert q["globals"][0] == g["s_g"][0]
    if "res_s_g" in g:
        assert q["globals"][1] == g["res_s_g"][0]
    if "deq" in g:
        assert (q["deq"][0].view(np.uint32) == g["deq"].view(np.uint32)).all()
    if "resid" in g:
        assert np.array_equal(q["resid"][0], g["resid"])
    if name.endswith("roundtrip.txt"):
        assert (q["resid"] == 0).all() and not np.signbit(q["resid"]).any()


# ------------------------------------------------------- invariants ----

def _data(seed, M, K, scale=1.0, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32) * np.float32(scale)
    if outliers:
        x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    return x


@pytest.mark.parametrize("fmt", [0, 1])
def test_residue_exact_in_fp32(orc, fmt):
    """x = d + r exactly: r = x - d is a Sterbenz-exact subtraction."""
    for seed in range(3):
        x = _data(seed, 4, 4096)
        q = orc.quantize_act(x, fmt)
        d = q["deq"][:4]
        r = q["resid"]
        assert np.array_equal((d + r).astype(np.float32), x)
        assert np.array_equal((x - d).astype(np.float32), r)


@pytest.mark.parametrize("fmt", [0, 1])
def test_power_of_two_equivariance(orc, fmt):
    x = _data(5, 3, 1024)
    q0 = orc.quantize_act(x, fmt)
    for j in (-20, -3, 1, 7, 30):
        qj = orc.quantize_act(x * np.float32(2.0 ** j), fmt)
        assert np.array_equal(qj["codes"], q0["codes"])
        if fmt == 0:
            assert np.array_equal(qj["scales"], q0["scales"])
            assert np.array_equal(qj["globals"], (q0["globals"] * np.float32(2.0 ** j)).astype(np.float32))
        else:
            assert np.array_equal(qj["scales"].astype(int), q0["scales"].astype(int) + j)


@pytest.mark.parametrize("fmt", [0, 1])
def test_sign_symmetry(orc, fmt):
    x = _data(6, 2, 512)
    q0 = orc.quantize_act(x, fmt)
    q1 = orc.quantize_act(-x, fmt)
    # base rows: every sign bit flips (x has no zeros)
    assert np.array_equal(q1["codes"][:2], q0["codes"][:2] ^ 0x88)
    # residue rows: r(-x) = -r(x) except that an exact zero residue is +0 both ways
    c0 = orc.unpack_codes(q0["codes"][2:], 512)
    c1 = orc.unpack_codes(q1["codes"][2:], 512)
    nz = q0["resid"] != 0
    assert np.array_equal(c1 & 7, c0 & 7)
    assert np.array_equal(c1[nz], c0[nz] ^ 8)
    assert np.array_equal(c1[~nz], c0[~nz])
    assert np.array_equal(q1["scales"], q0["scales"])
    assert np.array_equal(q1["globals"], q0["globals"])


def test_nvfp4_amax_block(orc):
    """The block holding the row amax encodes t ~= 448 to 0x7e, and the amax
    element gets magnitude 6 (Appendix B.2: alpha normalizes max s_i to 448)."""
    x = _data(8, 6, 2048)
    q = orc.quantize_act(x, 0, with_residue=False)
    codes = orc.unpack_codes(q["codes"], 2048)
    for m in range(6):
        k = int(np.argmax(np.abs(x[m])))
        assert q["scales"][m, k // 16] == 0x7E
        assert codes[m, k] & 7 == 7
        assert q["globals"][m] == np.float32(np.abs(x[m]).max()) / np.float32(2688.0)


def test_mxfp4_block_max_code(orc):
    """Each MXFP4 block's largest element has magnitude 4 or 6: q = a / 2^(E-2)
    lies in [4, 8) for a in [2^E, 2^(E+1))."""
    x = _data(9, 4, 2048)
    q = orc.quantize_act(x, 1, with_residue=False)
    codes = orc.unpack_codes(q["codes"], 2048)
    for m in range(4):
        for b in range(2048 // 32):
            blk = np.abs(x[m, 32 * b:32 * b + 32])
            k = 32 * b + int(np.argmax(blk))
            assert codes[m, k] & 7 in (6, 7)


@pytest.mark.parametrize("fmt", [0, 1])
def test_zero_rows(orc, fmt):
    x = np.zeros((2, 256), np.float32)
    x[1] = -0.0
    q = orc.quantize_act(x, fmt)
    assert (q["scales"] == 0).all() and (q["globals"] == 0).all()
    assert (q["codes"][0] == 0).all()
    assert (q["codes"][1] == 0x88).all()         # sign of -0 is kept
    assert (q["deq"] == 0).all() and (q["resid"] == 0).all()
    assert not np.signbit(q["resid"]).any()      # -0 - (-0) = +0
    assert (q["codes"][2:] == 0).all()


def test_nvfp4_tiny_row_sign(orc):
    """Tiny values far below a block's scale get code 0 with the input's sign."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    x[0, 1] = -1e-6
    x[0, 2] = 1e-6
    q = orc.quantize_act(x, 0)
    c = orc.unpack_codes(q["codes"], 32)[0]
    assert c[0] == 7 and c[1] == 8 and c[2] == 0
    assert q["resid"][0, 1] == np.float32(-1e-6)


def test_exact_input_has_zero_residue(orc):
    """A row whose values are already representable has r = 0, so the
    compensated operand equals the plain one."""
    g = load_golden("nvfp4_roundtrip.txt")
    x = np.tile(g["x"], (2, 8))
    q = orc.quantize_act(x, 0)
    assert (q["resid"] == 0).all() and (q["codes"][2:] == 0).all()


@pytest.mark.parametrize("fmt", [0, 1])
def test_dequant_consistent_with_codes(orc, fmt):
    """The stored codes/scales/globals rebuild exactly the dequantized values."""
    x = _data(12, 3, 1024)
    q = orc.quantize_act(x, fmt)
    d = orc.dequant_rows(q["codes"], q["scales"], q["globals"], fmt, 1024)
    assert np.array_equal(d.view(np.uint32), q["deq"].view(np.uint32))


@pytest.mark.parametrize("fmt", [0, 1])
def test_residue_never_hurts(orc, fmt):
    """0 is on every grid, so each residue element is quantized no farther from
    r than 0 is: the compensated activation error never exceeds the plain one."""
    x = _data(13, 8, 1024)
    q = orc.quantize_act(x, fmt)
    d, dr, r = q["deq"][:8], q["deq"][8:], q["resid"]
    plain = np.abs(x.astype(np.float64) - d)
    comp = np.abs(x.astype(np.float64) - d - dr)
    assert (np.abs(r.astype(np.float64) - dr) <= np.abs(r.astype(np.float64))).all()
    assert (comp <= plain + 1e-30).all()
    assert comp.sum() < plain.sum()


def test_nvfp4_weight_tensor_scale(orc):
    """Weights share one tensor scale from max|W| (Appendix B.2, Eq. 8)."""
    W = _data(14, 32, 256, scale=0.02)
    out = orc.quantize_weight(W, 0)
    assert out["s_g"] == np.float32(np.abs(W).max()) / np.float32(2688.0)
    rows = orc.quantize_weight_rows(W, 0, float(out["s_g"]))
    assert np.array_equal(rows["codes"], out["codes"])
    sub = orc.quantize_weight(W, 0, rows=[3, 17])
    assert np.array_equal(sub["codes"], out["codes"][[3, 17]])

"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same
seeded inputs.  Codes, scale bytes and tensor scales must be bit-exact; outputs
must satisfy |y_gpu - y_oracle| <= 1e-4 * sum_k |term_k| elementwise."""
import numpy as np
import pytest

import oracle
from block_scaled_fp4_act_amd import inputs
from gpu_util import FMT, assert_quant_equal, check_linear, dev_x, sample_channels

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import block_scaled_fp4_act_amd as rs
    rs.lib()  # raises if the HIP library was not built
    oracle.build()
    torch.manual_seed(0)


def _rs():
    import block_scaled_fp4_act_amd as rs
    return rs


_W_CACHE = {}


def _weights(wl):
    """W of a workload, drawn once and kept (one at a time: they are large)."""
    key = (wl.N, wl.K, wl.w_seed)
    if key not in _W_CACHE:
        _W_CACHE.clear()
        _W_CACHE[key] = wl.draw_w()
    return _W_CACHE[key]


# ------------------------------------------------------------- quantize ----

@pytest.mark.parametrize("wl", inputs.ALL, ids=lambda w: w.name)
@pytest.mark.parametrize("with_residue", [True, False])
def test_quantize_workload_bitexact(wl, with_residue):
    x = wl.draw_x() if not wl.x_rows else inputs.activations(
        wl.x_rows, wl.K, wl.x_seed, wl.outlier_frac, wl.outlier_scale, wl.o_seed, wl.bf16)
    fmt = FMT[wl.fmt]
    assert_quant_equal(x, fmt, wl.bf16, with_residue)
    # the other format on the same activations as well
    assert_quant_equal(x, 1 - fmt, wl.bf16, with_residue)


def _adversarial(K, seed):
    rng = np.random.default_rng(seed)
    rows = []
    rows.append(np.zeros(K, np.float32))                        # all zero
    rows.append(-np.zeros(K, np.float32))                       # all -0
    e = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    rows.append(np.tile(np.concatenate([e, -e]), K // 16) * np.float32(0.4375))  # exact grid
    r = rng.standard_normal(K).astype(np.float32)
    r[::7] = 0.0
    r[1::11] *= np.float32(1e-6)                                # tiny values beside big ones
    rows.append(r)
    rows.append((rng.standard_normal(K) * 1e-30).astype(np.float32))    # tiny row, normal scale math
    rows.append((rng.standard_normal(K) * 1e-41).astype(np.float32))    # subnormal row
    rows.append((rng.standard_normal(K) * 1e30).astype(np.float32))     # huge row
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    rows.append(np.tile(np.concatenate([ties, -ties]), K // 16))        # E2M1 ties at scale 1
    z = rng.standard_normal(K).astype(np.float32)
    z[: K // 2] = 0.0                                           # half the blocks empty
    rows.append(z)
    w = rng.standard_normal(K).astype(np.float32)
    w[rng.integers(0, K)] = 1e4                                 # one dominant outlier
    rows.append(w)
    return np.stack(rows)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("K", [32, 160, 4096, 32768])
def test_quantize_adversarial_bitexact(fmt, K):
    x = _adversarial(K, K)
    assert_quant_equal(x, fmt, False, True)
    assert_quant_equal(x, fmt, True, True)


def _near_tie_rows(K, n_rows, seed):
    """Rows whose element quotients v / s~ sit on and within three ulps of
    every E2M1 rounding tie, with s~ = S_b s_g not a power of two: the cases
    where the one-division quotient must reproduce the IEEE division exactly."""
    rng = np.random.default_rng(seed)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    rows = []
    for _ in range(n_rows):
        amax = np.float32(rng.uniform(50.0, 900.0))
        s_g = np.float32(oracle.nvfp4_global_scale(float(amax)))
        row = np.zeros(K, np.float32)
        for b in range(K // 16):
            bm = np.float32(amax if b == 0 else amax * rng.uniform(0.05, 1.0))
            sb = oracle.e4m3_value(oracle.e4m3_encode(float(np.float32(bm / np.float32(np.float32(6.0) * s_g)))))
            st = np.float32(np.float32(sb) * s_g)
            blk = np.empty(16, np.float32)
            blk[0] = bm
            for j in range(1, 16):
                x = np.float32(np.float32(rng.choice(ties)) * st)
                for _ in range(int(rng.integers(-3, 4))):
                    x = np.nextafter(x, np.float32(np.inf))
                x = min(x, bm)
                blk[j] = x if rng.random() < 0.5 else -x
            row[16 * b:16 * b + 16] = blk
        rows.append(row)
    return np.stack(rows)


@pytest.mark.parametrize("K", [256, 4096])
def test_quantize_quotient_near_ties(K):
    x = _near_tie_rows(K, 8, K + 3)
    assert_quant_equal(x, 0, False, True)


# NVFP4 rows shared by several workgroups (at most 256 rows x parts on a
# 256-CU device): two to eight parts of whole waves, a ragged last part
# (K = 8224: 1028 chunks of 8 in parts of 320), the part count cut by M
# (M = 100: two parts) and none left (M = 300), with and without residue
@pytest.mark.parametrize("MK", [(1, 8224), (3, 16384), (5, 14336), (40, 4096), (100, 8192), (300, 4160)],
                         ids=lambda t: "M%dK%d" % t)
def test_quantize_row_parts_bitexact(MK):
    M, K = MK
    rng = np.random.default_rng(M + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    x[0, :16] = 0.0
    assert_quant_equal(x, 0, True, True)
    assert_quant_equal(x, 0, False, True)
    assert_quant_equal(x, 0, True, False)


@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_exact_residue_identity(fmt):
    """The buffer's base and residue rows dequantize to d and d_r with
    x = d + r exactly; the oracle's residue is compared element by element."""
    x = inputs.ATTN.draw_x()
    _, q = assert_quant_equal(x, fmt, True, True)
    assert np.array_equal(q["deq"][:4] + q["resid"], inputs.round_to_bf16(x))


# -------------------------------------------------------------- prepack ----

def _prepack_check(W, fmt, rows=None):
    import torch
    rs = _rs()
    N, K = W.shape
    Wd = torch.from_numpy(W).cuda()
    blob = rs.prepack_weights(Wd, fmt)
    codes, scales, s_g = rs.unpack_weights_canonical(blob, fmt, N, K)
    torch.cuda.synchronize()
    q = oracle.quantize_weight(W, fmt, rows=rows, want_deq=False)
    sel = slice(None) if rows is None else torch.as_tensor(np.asarray(rows)).cuda()
    c = codes[sel].cpu().numpy()
    s = scales[sel].cpu().numpy()
    assert np.array_equal(c, q["codes"])
    assert np.array_equal(s, q["scales"])
    if fmt == 0:
        assert s_g.cpu().numpy()[0].view(np.uint32) == np.float32(q["s_g"]).view(np.uint32)
    return blob


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("NK", [(512, 512), (72, 160), (16, 32), (1000, 384), (33, 4096)])
def test_prepack_bitexact_small(fmt, NK):
    N, K = NK
    W = inputs.weights(N, K, 7)
    _prepack_check(W, fmt)


@pytest.mark.parametrize("wl", [inputs.ATTN, inputs.MLP_DOWN, inputs.LARGE_MLP, inputs.MX], ids=lambda w: w.name)
def test_prepack_bitexact_workload_sampled(wl):
    W = _weights(wl)
    rows = np.sort(np.random.default_rng(5).choice(wl.N, 96, replace=False))
    rows[-1] = wl.N - 1
    _prepack_check(W, FMT[wl.fmt], rows=rows)


def test_prepack_bf16_weights():
    import torch
    rs = _rs()
    W = inputs.round_to_bf16(inputs.weights(96, 512, 3))
    for fmt in (0, 1):
        blob = rs.prepack_weights(torch.from_numpy(W).cuda().to(torch.bfloat16), fmt)
        codes, scales, _ = rs.unpack_weights_canonical(blob, fmt, 96, 512)
        q = oracle.quantize_weight(W, fmt, want_deq=False)
        assert np.array_equal(codes.cpu().numpy(), q["codes"])
        assert np.array_equal(scales.cpu().numpy(), q["scales"])


# --------------------------------------------------------------- linear ----

def _run_linear(x, W, fmt, bf16, comp, M=None):
    import torch
    rs = _rs()
    M = x.shape[0] if M is None else M
    N, K = W.shape
    blob = rs.prepack_weights(torch.from_numpy(W).cuda(), fmt)
    act = rs.quantize_act_with_residue(dev_x(x, bf16), fmt, with_residue=comp)
    f = rs.fp4_linear_compensated if comp else rs.fp4_linear
    y = f(act, blob, M, N, K, fmt)
    torch.cuda.synchronize()
    return y.cpu().numpy(), blob, act


def _oracle_linear(x, W, fmt, bf16, comp, rows=None):
    xin = inputs.round_to_bf16(x) if bf16 else x
    q = oracle.quantize_act(xin, fmt, with_residue=comp)
    w = oracle.quantize_weight(W, fmt, rows=rows)
    return oracle.linear(q["deq"], w["deq"], xin.shape[0], comp)


SMALL_CASES = [  # (M, N, K): several tiles, ragged N and K tails, both row-tile counts
    (1, 512, 512), (2, 72, 160), (3, 1000, 384), (4, 256, 4096), (5, 48, 640),
    (8, 320, 1024), (8, 100, 2080), (11, 64, 256), (16, 64, 512), (6, 16, 32),
    # wide operands (more than 32 tile rows): the 2-D tiled kernel, with ragged
    # row tiles, channel tiles and K tails
    (17, 264, 384), (33, 130, 160), (40, 512, 1056), (64, 128, 256), (100, 72, 2048),
    (129, 300, 512),
    # K past one narrow launch (two launches over the K steps, the second
    # adding to y), up to the longest supported K, and a wide operand there
    (4, 200, 20480), (2, 64, 32768), (40, 64, 24576),
    # two row tiles, compensated NVFP4: launches of 32 steps adding into y
    # (two full ones; one full and a ragged one; four)
    (12, 80, 8192), (16, 48, 5120), (9, 40, 16384),
    # four row tiles (compensated NVFP4, 33..64 operand rows, K and N at most
    # 4096): one launch of 32 steps and a ragged one of 17; the tiled kernel
    # past K = 4096 and past N = 4096
    (20, 72, 4096), (24, 40, 2112), (32, 48, 8192), (25, 40, 5120), (30, 16400, 256),
]


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("comp", [True, False])
@pytest.mark.parametrize("MNK", SMALL_CASES, ids=lambda t: "M%dN%dK%d" % t)
def test_linear_small_full(fmt, comp, MNK):
    M, N, K = MNK
    rng = np.random.default_rng(M * 1000 + N + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    W = inputs.weights(N, K, K + N)
    y, _, _ = _run_linear(x, W, fmt, True, comp)
    yo, beta = _oracle_linear(x, W, fmt, True, comp)
    check_linear(y, yo, beta)


def _workload_cases():
    wls = [inputs.SMALL, inputs.ATTN, inputs.MLP_UP, inputs.MLP_DOWN]
    wls += [inputs.LARGE_MLP.with_m(m) for m in inputs.LARGE_MLP_M]
    wls += [inputs.MX.with_m(m) for m in inputs.MX_M]
    return [(wl, comp) for wl in wls for comp in (True, False)]


@pytest.mark.parametrize("wl,comp", _workload_cases(),
                         ids=lambda v: f"{v.name}_M{v.M}" if hasattr(v, "name") else ("comp" if v else "plain"))
def test_linear_workload_sampled(wl, comp):
    """Full-size workloads, launched exactly as the bench launches them; the
    oracle computes a sample of output channels one by one (at least 4096
    outputs of y)."""
    fmt = FMT[wl.fmt]
    x, W = wl.draw_x(), _weights(wl)
    y, _, _ = _run_linear(x, W, fmt, wl.bf16, comp)
    rows = sample_channels(wl.N, wl.M, 9)
    xin = inputs.round_to_bf16(x) if wl.bf16 else x
    q = oracle.quantize_act(xin, fmt, with_residue=comp)
    w = oracle.quantize_weight(W, fmt, rows=rows)
    yo, beta = oracle.linear(q["deq"], w["deq"], wl.M, comp)
    check_linear(y[:, rows], yo, beta)


@pytest.mark.parametrize("fmt", [0, 1])
def test_linear_deterministic(fmt):
    x = inputs.ATTN.draw_x()
    W = inputs.weights(1024, 4096, 1)
    y1, blob, act = _run_linear(x, W, fmt, True, True)
    rs = _rs()
    import torch
    y2 = rs.fp4_linear_compensated(act, blob, 4, 1024, 4096, fmt)
    torch.cuda.synchronize()
    assert np.array_equal(y1.view(np.uint32), y2.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("fmt", [0, 1])
def test_linear_zero_activations(fmt):
    """A zero row gives exactly zero outputs (beta = 0 there)."""
    x = np.zeros((2, 512), np.float32)
    x[1] = inputs.activations(1, 512, 3, 0.01, 20.0, 4, False)[0]
    W = inputs.weights(64, 512, 2)
    y, _, _ = _run_linear(x, W, fmt, False, True)
    assert (y[0] == 0).all()
    yo, beta = _oracle_linear(x, W, fmt, False, True)
    check_linear(y, yo, beta)


def test_plain_reads_first_rows_of_compensated_buffer():
    """A with-residue buffer's first M records are a valid plain buffer."""
    import torch
    rs = _rs()
    x = inputs.ATTN.draw_x()
    W = inputs.weights(256, 4096, 4)
    blob = rs.prepack_weights(torch.from_numpy(W).cuda(), 0)
    a2 = rs.quantize_act_with_residue(dev_x(x, True), 0, True)
    a1 = rs.quantize_act_with_residue(dev_x(x, True), 0, False)
    y2 = rs.fp4_linear(a2, blob, 4, 256, 4096, 0)
    y1 = rs.fp4_linear(a1, blob, 4, 256, 4096, 0)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_linear_limits_rejected():
    import torch
    rs = _rs()
    act = torch.zeros(rs.packed_act_bytes(0, 17, 512, True), dtype=torch.uint8, device="cuda")
    blob = torch.zeros(rs.packed_weight_bytes(0, 64, 512), dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="unsupported"):
        rs.fp4_linear_compensated(act, blob, 1, 64, 32800, 0)
    with pytest.raises(RuntimeError, match="outside"):
        rs.fp4_linear_compensated(act, blob, 65536, 64, 512, 0)
    with pytest.raises(RuntimeError, match="too small"):
        rs.fp4_linear_compensated(act[:100], blob, 1, 64, 512, 0)
    with pytest.raises(RuntimeError, match="too small"):
        rs.fp4_linear_compensated(act, blob, 18, 64, 512, 0)


@pytest.mark.parametrize("fmt", [0, 1])
def test_validate_packed(fmt):
    """A prepacked blob's header reads back its format, N and K; a corrupted
    magic, a short buffer and a wrong tensor scale are rejected."""
    import torch
    rs = _rs()
    N, K = 48, 160
    blob = rs.prepack_weights(torch.from_numpy(inputs.weights(N, K, 3)).cuda(), fmt)
    assert rs.validate_packed(blob) == (fmt, N, K)
    with pytest.raises(RuntimeError, match="buffer too small"):
        rs.validate_packed(blob[: rs.packed_weight_bytes(fmt, N, K) - 16])
    bad = blob.clone()
    bad[0] ^= 0xFF
    with pytest.raises(RuntimeError, match="unknown format or dtype"):
        rs.validate_packed(bad)
    bad = blob.clone()
    bad[32:36] = torch.tensor([0, 0, 0x80, 0xFF], dtype=torch.uint8)   # s_g = -inf
    with pytest.raises(RuntimeError, match="unknown format or dtype"):
        rs.validate_packed(bad)

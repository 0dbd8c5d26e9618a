"""GPU parity of compensated decode attention (ResAttn; ResServe Section 4.3
Eq. 3 and Section 5.2) over the paged NVFP4 KV cache: the cache writer must
match the oracle's NVFP4 rows bit for bit; the attention output must satisfy
|o_gpu - o_oracle| <= 2^-10 * (sum_t p_t |v_t| / sum_t p_t)
                      + (1e-6 + L * 2^-25) * max|v|
elementwise.  The probabilities enter the P V product rounded to f16 (on the
numerator only; the row sum l stays fp32): a normal f16 p carries a relative
error of at most 2^-11, which the first term covers twice over; a p below
2^-14 is an f16 subnormal with an absolute error of at most 2^-25, and L such
terms add at most L * 2^-25 * max|v| / l to the output, with l >= 1 (the
token with the largest score contributes p = 1, and a split's weight
2^(m_s - M) keeps that).  Scores are exact products summed in fp32; the 1e-6
term covers the fp32 sums."""
import math

import numpy as np
import pytest

import oracle
from block_scaled_fp4_act_amd import inputs

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


def _rand(shape, seed, scale=1.0):
    return (np.random.Generator(np.random.PCG64(seed)).standard_normal(shape, dtype=np.float32) * np.float32(scale))


class Problem:
    """B sequences of given lengths in a shuffled paged cache."""

    def __init__(self, lens, H_q, H_kv, D, seed, k_scale=1.0, v_scale=1.0, spare_pages=3, bf16=True):
        import torch
        rs = _rs()
        self.lens, self.H_q, self.H_kv, self.D = list(lens), H_q, H_kv, D
        self.B = len(lens)
        self.k_scale, self.v_scale = k_scale, v_scale
        npg = [(L + 31) // 32 for L in lens]
        self.max_pages = max(max(npg), 1)
        total = sum(npg) + spare_pages
        perm = np.random.default_rng(seed).permutation(total)
        self.table = np.zeros((self.B, self.max_pages), np.int32)
        slots, ks, vs = [], [], []
        pos = 0
        for b, L in enumerate(lens):
            pages = perm[pos:pos + npg[b]]
            pos += npg[b]
            self.table[b, :npg[b]] = pages
            t = np.arange(L)
            slots.append(pages[t // 32] * 32 + t % 32)
        self.k = [_rand((L, H_kv, D), seed * 10 + b + 1) for b, L in enumerate(lens)]
        self.v = [_rand((L, H_kv, D), seed * 10 + b + 101) for b, L in enumerate(lens)]
        if bf16:
            self.k = [inputs.round_to_bf16(x) for x in self.k]
            self.v = [inputs.round_to_bf16(x) for x in self.v]
        self.cache = torch.full((total * rs.kv_page_bytes(H_kv, D),), 0x5A, dtype=torch.uint8, device="cuda")
        kk = np.concatenate(self.k) if sum(lens) else np.zeros((0, H_kv, D), np.float32)
        vv = np.concatenate(self.v) if sum(lens) else np.zeros((0, H_kv, D), np.float32)
        sl = np.concatenate(slots).astype(np.int32)
        if len(sl):
            dt = torch.bfloat16 if bf16 else torch.float32
            rs.kv_cache_write(_t(kk).to(dt), _t(vv).to(dt), _t(sl), self.cache, k_scale, v_scale)
        self.slots = sl
        q = _rand((self.B * H_q, D), seed + 7)
        q[:, ::29] *= 20.0                       # outlier channels, then bf16 (what the kernel receives)
        self.q = inputs.round_to_bf16(q)

    def run(self, comp=True, splits=0, out_bf16=False):
        import torch
        rs = _rs()
        qa = rs.quantize_act_with_residue(_t(self.q).to(torch.bfloat16), 0, comp)
        out = rs.resattn_decode(qa, self.cache, _t(self.table), _t(np.array(self.lens, np.int32)),
                                max(max(self.lens), 1), self.B, self.H_q, self.H_kv, self.D, compensated=comp,
                                k_scale=self.k_scale, v_scale=self.v_scale, splits=splits, out_bf16=out_bf16)
        torch.cuda.synchronize()
        return out

    def reference(self, comp=True):
        q = oracle.quantize_act(self.q, 0, with_residue=comp)
        n = self.B * self.H_q
        ref = np.zeros((self.B, self.H_q, self.D))
        mag = np.zeros_like(ref)
        slack = np.zeros((self.B,))
        sm = 1.0 / math.sqrt(self.D)
        for b, L in enumerate(self.lens):
            if L == 0:
                continue
            kd = oracle.kv_quantize(self.k[b], self.k_scale)["deq"]
            vd = oracle.kv_quantize(self.v[b], self.v_scale)["deq"]
            rows = slice(b * self.H_q, (b + 1) * self.H_q)
            qb = q["deq"][rows]
            qr = q["deq"][n + b * self.H_q: n + (b + 1) * self.H_q] if comp else None
            ref[b] = oracle.attention_decode(qb, qr, kd, vd, sm)
            mag[b] = oracle.attention_decode(qb, qr, kd, np.abs(vd), sm)
            slack[b] = (1e-6 + L * 2.0 ** -25) * np.abs(vd).max()
        return ref, mag, slack


def _check(out, ref, mag, slack):
    """slack[b]: (1e-6 + L_b 2^-25) max|v| of sequence b (the module docstring)."""
    o = out.float().cpu().numpy().astype(np.float64)
    bound = 2.0 ** -10 * mag + slack[:, None, None]
    err = np.abs(o - ref)
    bad = err > bound
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} outside; worst ratio "
                           f"{float((err / np.maximum(bound, 1e-30)).max()):.3e}")


def _kv_slot(t):
    """k-slot of page row t in the attention kernel's P V operand."""
    return 8 * (t >> 2) + (t & 3) if t < 16 else 8 * ((t - 16) >> 2) + 4 + (t & 3)


def _read_token(pg, base, row, D):
    """One token's K codes, K scales, V codes and V scales read back from the
    page region of one KV head, following the documented page layout; codes
    come back token-major (element 2k in the low nibble of byte k)."""
    nc = D // 128
    kc = pg[base + row * D // 2: base + (row + 1) * D // 2]
    kso = base + 16 * D + row * (D // 16)
    ksc = np.array([pg[kso + 2 * nc * ((b & 7) >> 1) + 2 * (b >> 3) + (b & 1)] for b in range(D // 16)], np.uint8)
    sl = _kv_slot(row)
    q, u = sl >> 3, sl & 7
    nib = []
    for d in range(D):
        c, a, e = d >> 7, (d & 127) >> 3, d & 7
        off = base + 18 * D + 2048 * c + 1024 * (e >> 2) + 16 * (a + 16 * q) + 4 * (e & 3)
        nib.append((int.from_bytes(bytes(pg[off:off + 4]), "little") >> (4 * u)) & 0xF)
    vc = np.array([nib[2 * k] | (nib[2 * k + 1] << 4) for k in range(D // 2)], np.uint8)
    vsc = np.array([pg[base + 34 * D + 32 * b + sl] for b in range(D // 16)], np.uint8)
    return kc, ksc, vc, vsc


def test_kv_slot_is_a_permutation():
    assert sorted(_kv_slot(t) for t in range(32)) == list(range(32))


@pytest.mark.parametrize("D", [128, 256])
def test_kv_cache_write_bitexact(D):
    P = Problem([70, 33], 8, 2, D, seed=3, k_scale=1.0, v_scale=0.5)
    pb = _rs().kv_page_bytes(2, D)
    cache = P.cache.cpu().numpy().reshape(-1, pb)
    for b in range(P.B):
        qk = oracle.kv_quantize(P.k[b], 1.0)
        qv = oracle.kv_quantize(P.v[b], 0.5)
        for t in range(P.lens[b]):
            page, row = divmod(int(P.table[b, t // 32]) * 32 + t % 32, 32)
            for h in range(2):
                kc, ksc, vc, vsc = _read_token(cache[page], h * 36 * D, row, D)
                assert np.array_equal(kc, qk["codes"][t, h]) and np.array_equal(ksc, qk["scales"][t, h])
                assert np.array_equal(vc, qv["codes"][t, h]) and np.array_equal(vsc, qv["scales"][t, h])


@pytest.mark.parametrize("D", [128, 256])
def test_kv_cache_write_across_calls(D):
    """Decode-style writes: tokens arrive over several calls (odd rows first,
    then even rows, then one token per call) into pages that hold other bytes;
    each call must clear and set only its tokens' nibbles of the shared V
    words, so every token reads back bit-exact at the end."""
    import torch
    rs = _rs()
    H_kv, T = 2, 40
    pb = rs.kv_page_bytes(H_kv, D)
    cache = torch.full((3 * pb,), 0xA7, dtype=torch.uint8, device="cuda")
    k = inputs.round_to_bf16(_rand((T, H_kv, D), 31 + D))
    v = inputs.round_to_bf16(_rand((T, H_kv, D), 32 + D))
    slots = (np.arange(T) + 32).astype(np.int32)          # pages 1 and 2
    order = [np.arange(1, 32, 2), np.arange(0, 32, 2)] + [np.array([t]) for t in range(32, T)]
    for idx in order:
        rs.kv_cache_write(_t(k[idx]).to(torch.bfloat16), _t(v[idx]).to(torch.bfloat16), _t(slots[idx]), cache,
                          1.0, 1.0)
    torch.cuda.synchronize()
    pages = cache.cpu().numpy().reshape(-1, pb)
    assert (pages[0] == 0xA7).all()                        # page 0 untouched
    qk, qv = oracle.kv_quantize(k, 1.0), oracle.kv_quantize(v, 1.0)
    for t in range(T):
        page, row = divmod(int(slots[t]), 32)
        for h in range(H_kv):
            kc, ksc, vc, vsc = _read_token(pages[page], h * 36 * D, row, D)
            assert np.array_equal(kc, qk["codes"][t, h]) and np.array_equal(ksc, qk["scales"][t, h])
            assert np.array_equal(vc, qv["codes"][t, h]) and np.array_equal(vsc, qv["scales"][t, h])


CASES = [  # (lens, H_q, H_kv, D)
    ([1, 37, 300], 16, 2, 128),      # GQA 8, one token, a partial page, several pages
    ([64, 5, 129], 8, 2, 128),       # GQA 4
    ([45, 200], 12, 2, 256),         # GQA 6, D = 256
    ([1000], 8, 1, 128),
]


@pytest.mark.parametrize("comp", [True, False])
@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "L%s_Hq%d_Hkv%d_D%d" % ("-".join(map(str, c[0])), c[1], c[2], c[3]))
def test_resattn_parity(case, splits, comp):
    lens, H_q, H_kv, D = case
    P = Problem(lens, H_q, H_kv, D, seed=sum(lens) + H_q)
    out = P.run(comp=comp, splits=splits)
    _check(out, *P.reference(comp=comp))


@pytest.mark.parametrize("splits", [64, 100, 130])
@pytest.mark.parametrize("D", [128, 256])
def test_resattn_many_splits(D, splits):
    """64 and more splits take the sixteen-wave combine: a split count that is
    not a multiple of 16, and more splits than pages (empty splits)."""
    import torch
    P = Problem([4000, 1500], 16, 2, D, seed=splits + D)
    o32 = P.run(splits=splits)
    _check(o32, *P.reference())
    o16 = P.run(splits=splits, out_bf16=True)
    assert torch.equal(o16, o32.to(torch.bfloat16))
    _check(P.run(comp=False, splits=splits), *P.reference(comp=False))


@pytest.mark.parametrize("splits", [1500, 4096])
@pytest.mark.parametrize("D", [128, 256])
def test_resattn_split_extremes(D, splits):
    """1500 and 4096 splits (the most the kernel accepts) over short sequences:
    nearly every split is empty, and the combine's per-thread (m, l) loop runs
    its later iterations (past 1024 splits)."""
    import torch
    P = Problem([300, 45], 16, 2, D, seed=splits + 3 * D)
    o32 = P.run(splits=splits)
    _check(o32, *P.reference())
    o16 = P.run(splits=splits, out_bf16=True)
    assert torch.equal(o16, o32.to(torch.bfloat16))
    _check(P.run(comp=False, splits=splits), *P.reference(comp=False))


def test_resattn_long_peaked_sequence():
    """32768 tokens with peaked scores (outlier query channels at 20x): many
    probabilities fall below 2^-14 and round to f16 subnormals, which the
    L * 2^-25 * max|v| term of the bound covers; preset split rule."""
    P = Problem([32768], 8, 1, 128, seed=21)
    _check(P.run(), *P.reference())
    _check(P.run(splits=256), *P.reference())


def test_resattn_global_scales_and_bf16_output():
    import torch
    P = Problem([77, 150], 16, 2, 128, seed=5, k_scale=0.75, v_scale=2.0)
    o32 = P.run(splits=1)
    o16 = P.run(splits=1, out_bf16=True)
    assert o16.dtype == torch.bfloat16 and torch.equal(o16, o32.to(torch.bfloat16))
    _check(o32, *P.reference())


def test_resattn_zero_length_and_empty_splits():
    """A sequence of length 0 gives zeros; splits beyond a short sequence are
    empty and weigh nothing."""
    P = Problem([0, 40, 2], 8, 1, 128, seed=9)
    out = P.run(splits=5)
    assert (out[0] == 0).all()
    ref, mag, slack = P.reference()
    _check(out[1:], ref[1:], mag[1:], slack[1:])


def test_resattn_compensation_reduces_error():
    """Against attention with the unquantized query over the same cache, the
    compensated scores beat the plain ones (the page's Fig. 10d comparison)."""
    P = Problem([512, 512], 16, 2, 128, seed=11)
    ref_exact = np.zeros((2, 16, 128))
    sm = 1 / math.sqrt(128)
    for b in range(2):
        kd = oracle.kv_quantize(P.k[b], 1.0)["deq"]
        vd = oracle.kv_quantize(P.v[b], 1.0)["deq"]
        ref_exact[b] = oracle.attention_decode(P.q[b * 16:(b + 1) * 16], None, kd, vd, sm)
    e = lambda o: float(np.sum((o.float().cpu().numpy() - ref_exact) ** 2))
    assert e(P.run(comp=True)) < 0.6 * e(P.run(comp=False))


@pytest.mark.parametrize("cfg", [(8, 64, 8, 128, 8192), (2, 24, 4, 256, 4096)],
                         ids=["D128_GQA8_B8_L8192", "D256_GQA6_B2_L4096"])
def test_resattn_workload_sampled(cfg):
    """Decode shapes of the page's Figure 10 at moderate length, with the
    preset split rule; heads of the first and last sequences checked."""
    B, H_q, H_kv, D, L = cfg
    P = Problem([L] * B, H_q, H_kv, D, seed=L + B)
    out = P.run()
    keep = [0, B - 1]
    sub = Problem.__new__(Problem)
    sub.__dict__.update(P.__dict__)
    sub.lens = [P.lens[b] for b in keep]
    sub.k = [P.k[b] for b in keep]
    sub.v = [P.v[b] for b in keep]
    sub.q = np.concatenate([P.q[b * H_q:(b + 1) * H_q] for b in keep])
    sub.B = len(keep)
    ref, mag, slack = sub.reference()
    _check(out[keep], ref, mag, slack)


def test_resattn_split_rule():
    """The preset split count, a power of two: at most ~8 waves per compute
    unit over B * H_kv items, and the smallest p with p^2 B > 8 pages (256
    compute units)."""
    import torch
    rs = _rs()
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("rule values are for a 256-unit device")
    assert rs.resattn_splits(1, 8, 8192) == 64          # 256 pages: 64^2 > 2048 >= 32^2
    assert rs.resattn_splits(1, 8, 131072) == 256       # 4096 pages
    assert rs.resattn_splits(1, 8, 16384) == 128        # 512 pages: 64^2 = 4096 is not above 4096
    assert rs.resattn_splits(4, 8, 8192) == 32          # 32^2 * 4 > 2048
    assert rs.resattn_splits(8, 8, 8192) == 32          # 16^2 * 8 = 2048 is not above 2048
    assert rs.resattn_splits(4, 8, 65536) == 64         # capped: 8 waves per unit over 32 items
    assert rs.resattn_splits(32, 8, 8192) == 8          # capped: 8 waves per unit over 256 items
    assert rs.resattn_splits(1, 8, 32) == 1             # one page
    assert rs.resattn_splits(1, 8, 100) == 4            # 4 pages: 8, capped at the pages

"""Pins of the oracle's compensated decode attention (ResServe, Section 4.3
Eq. 3 and Section 5.2: scores Q^K^T + R^K^T folded before softmax, output
softmax(S) V^ over the dequantized NVFP4 cache) and of its KV quantization.
CPU only."""
import numpy as np
import pytest

from block_scaled_fp4_act_amd import inputs


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def test_single_token_returns_its_value(orc):
    q = _rand((8, 128), 1)
    k = _rand((1, 2, 128), 2)
    v = _rand((1, 2, 128), 3)
    out = orc.attention_decode(q, None, k, v, 1 / np.sqrt(128))
    for h in range(8):
        assert np.array_equal(out[h], v[0, h // 4].astype(np.float64))


def test_zero_keys_average_values_per_kv_head(orc):
    """All scores equal: the output is the mean of V; query head h reads KV
    head h // (H_q / H_kv)."""
    L, H_kv, d = 37, 4, 64
    k = np.zeros((L, H_kv, d), np.float32)
    v = _rand((L, H_kv, d), 4)
    q = _rand((24, d), 5)
    out = orc.attention_decode(q, _rand((24, d), 6), k, v, 0.125)
    for h in range(24):
        np.testing.assert_allclose(out[h], v[:, h // 6].astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)


def test_matches_numpy_softmax_attention(orc):
    L, H_q, H_kv, d = 300, 8, 1, 128
    q, r = _rand((H_q, d), 7), _rand((H_q, d), 8, 0.05)
    k, v = _rand((L, H_kv, d), 9), _rand((L, H_kv, d), 10)
    sm = 1 / np.sqrt(d)
    out = orc.attention_decode(q, r, k, v, sm)
    s = (q.astype(np.float64) + r.astype(np.float64)) @ k[:, 0].astype(np.float64).T * sm
    p = np.exp(s - s.max(axis=1, keepdims=True))
    want = (p @ v[:, 0].astype(np.float64)) / p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-13)


def test_dominant_token(orc):
    L, d = 50, 128
    k = np.zeros((L, 1, d), np.float32)
    k[17, 0, :] = 1.0
    q = np.full((4, d), 2.0, np.float32)           # score 256 * sm for token 17, 0 elsewhere
    v = _rand((L, 1, d), 11)
    out = orc.attention_decode(q, None, k, v, 1.0)
    np.testing.assert_allclose(out, np.repeat(v[17].astype(np.float64), 4, axis=0), rtol=0, atol=1e-12)


def test_kv_quantize_uses_given_global_scale(orc):
    """With g = 1 a block whose maximum is 6 * S (S on the E4M3 grid) keeps
    S as its scale and grid values exactly."""
    x = np.zeros((2, 3, 32), np.float32)
    x[0, 1, :16] = np.array([6, 3, -1.5, 0.5] + [0] * 12, np.float32) * 0.75
    q = orc.kv_quantize(x, 1.0)
    assert q["scales"][0, 1, 0] == 0x34                  # 0.75 = 1.5 * 2^-1: exponent field 6, mantissa 4
    assert np.array_equal(q["deq"], x)


def test_compensated_scores_closer_to_unquantized_query(orc):
    """Folding the quantized residue into the scores brings the output closer
    to attention with the unquantized query (same NVFP4 cache)."""
    L, H_q, H_kv, d = 512, 8, 1, 128
    qx = inputs.activations(H_q, d, 3, 0.02, 20.0, 4, True)
    k = orc.kv_quantize(_rand((L, H_kv, d), 12), 1.0)["deq"]
    v = orc.kv_quantize(_rand((L, H_kv, d), 13), 1.0)["deq"]
    sm = 1 / np.sqrt(d)
    ref = orc.attention_decode(qx, None, k, v, sm)
    qq = orc.quantize_act(qx, 0, with_residue=True)
    plain = orc.attention_decode(qq["deq"][:H_q], None, k, v, sm)
    comp = orc.attention_decode(qq["deq"][:H_q], qq["deq"][H_q:], k, v, sm)
    e = lambda o: np.sum((o - ref) ** 2)
    assert e(comp) < 0.5 * e(plain)

"""ctypes binding of the plain C oracle (``rsfp4_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Every function here marshals numpy arrays into the C
oracle and back; the arithmetic lives in the C file, which follows the ResServe
page (arXiv 2611.08713): Section 2 / Figure 1 for the formats, Appendix B.2
Eqs. 8-10 for the NVFP4 scale computation, Section 4.2 Eq. 1 and Section 4.3
Eq. 2 for the compensated product and its Fold; Section 5.3, Eq. 6 and
Appendix B.1, Eq. 7 for selective compensation (K-Ext); Appendix B.2 (Eq. 8 and
Algorithm 1) for the paper-numerics NVFP4 quantizer with a tensor scale alpha;
Section 4.3 Eq. 3 and Section 5.2 for compensated decode attention (ResAttn).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rsfp4_oracle.c")
_LIB = os.path.join(_HERE, "librsfp4_oracle.so")
_LIB_OMP = os.path.join(_HERE, "librsfp4_oracle_omp.so")    # timing build: the linear's channels over threads
FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

NVFP4, MXFP4 = 0, 1
BLOCK = {NVFP4: 16, MXFP4: 32}

__all__ = [
    "NVFP4", "MXFP4", "BLOCK", "build", "lib",
    "e2m1_value", "e2m1_encode_mag", "e4m3_value", "e4m3_encode",
    "e8m0_for_amax", "e8m0_value", "nvfp4_global_scale", "absmax",
    "quantize_act", "quantize_weight", "quantize_weight_rows", "dequant_rows",
    "linear", "threads", "unpack_codes",
    "channel_abs_sum", "kext_select", "kext_dim", "kext_extend_weight", "kext_quantize_act",
    "nvfp4_alpha", "quantize_row_alg1", "quantize_act_alg1",
    "kv_quantize", "attention_decode",
]


def build(force=False):
    """Compile the oracle with gcc (-O2, no contraction, no fast-math), and the
    same source with -fopenmp as the multi-threaded timing build."""
    for path, extra in ((_LIB, []), (_LIB_OMP, ["-fopenmp"])):
        if force or not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            tmp = path + ".tmp"
            subprocess.check_call(["gcc"] + FLAGS + extra + ["-o", tmp, _SRC, "-lm"])
            os.replace(tmp, path)
    return _LIB


_lib = None
_lib_omp = None


def lib(threads=False):
    """The oracle library; threads=True: the OpenMP timing build (same results)."""
    global _lib, _lib_omp
    if threads:
        if _lib_omp is None:
            if not os.path.exists(_LIB_OMP):
                build()
            _lib_omp = _load(_LIB_OMP)
        return _lib_omp
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _load(_LIB)
    return _lib


def _load(path):
    L = ctypes.CDLL(path)
    if True:
        f32, u8, i64, i32, dbl = ctypes.c_float, ctypes.c_uint8, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        P = ctypes.c_void_p
        L.oracle_e2m1_value.restype, L.oracle_e2m1_value.argtypes = f32, [u8]
        L.oracle_e2m1_encode_mag.restype, L.oracle_e2m1_encode_mag.argtypes = u8, [f32]
        L.oracle_e4m3_value.restype, L.oracle_e4m3_value.argtypes = f32, [u8]
        L.oracle_e4m3_encode.restype, L.oracle_e4m3_encode.argtypes = u8, [f32]
        L.oracle_e8m0_for_amax.restype, L.oracle_e8m0_for_amax.argtypes = u8, [f32]
        L.oracle_e8m0_value.restype, L.oracle_e8m0_value.argtypes = f32, [u8]
        L.oracle_nvfp4_global_scale.restype, L.oracle_nvfp4_global_scale.argtypes = f32, [f32]
        L.oracle_absmax.restype, L.oracle_absmax.argtypes = f32, [P, i64]
        L.oracle_nvfp4_quantize_row.restype = None
        L.oracle_nvfp4_quantize_row.argtypes = [P, i64, f32, P, P, P]
        L.oracle_mxfp4_quantize_row.restype = None
        L.oracle_mxfp4_quantize_row.argtypes = [P, i64, P, P, P]
        L.oracle_quantize_act.restype = None
        L.oracle_quantize_act.argtypes = [i32, P, i64, i64, i32, P, P, P, P, P]
        L.oracle_quantize_weight_rows.restype = None
        L.oracle_quantize_weight_rows.argtypes = [i32, P, i64, i64, f32, P, P, P]
        L.oracle_linear.restype = None
        L.oracle_linear.argtypes = [P, P, i64, i64, i64, i32, P, P]
        L.oracle_channel_abs_sum.restype = None
        L.oracle_channel_abs_sum.argtypes = [P, i64, i64, P]
        L.oracle_kext_select.restype = None
        L.oracle_kext_select.argtypes = [P, i64, i32, P]
        L.oracle_kext_extend_weight.restype = None
        L.oracle_kext_extend_weight.argtypes = [P, i64, i64, P, i32, P]
        L.oracle_kext_quantize_act.restype = None
        L.oracle_kext_quantize_act.argtypes = [i32, P, i64, i64, P, i32, P, P, P, P, P]
        L.oracle_nvfp4_alpha.restype, L.oracle_nvfp4_alpha.argtypes = f32, [P, i64]
        L.oracle_nvfp4_quantize_row_alg1.restype = None
        L.oracle_nvfp4_quantize_row_alg1.argtypes = [P, i64, f32, P, P, P, P]
        L.oracle_quantize_act_alg1.restype = None
        L.oracle_quantize_act_alg1.argtypes = [P, i64, i64, f32, i32, P, P, P, P, P, P]
        L.oracle_attention_decode.restype = None
        L.oracle_attention_decode.argtypes = [P, P, P, P, i64, i64, i64, i64, dbl, P, P]
        L.oracle_threads.restype, L.oracle_threads.argtypes = i32, []
        return L


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def e2m1_value(code):
    return lib().oracle_e2m1_value(int(code))


def e2m1_encode_mag(u):
    return lib().oracle_e2m1_encode_mag(float(u))


def e4m3_value(code):
    return lib().oracle_e4m3_value(int(code))


def e4m3_encode(t):
    return lib().oracle_e4m3_encode(float(t))


def e8m0_for_amax(a):
    return lib().oracle_e8m0_for_amax(float(a))


def e8m0_value(b):
    return lib().oracle_e8m0_value(int(b))


def nvfp4_global_scale(amax):
    return lib().oracle_nvfp4_global_scale(float(amax))


def absmax(v):
    v = _f32(v).ravel()
    return lib().oracle_absmax(_p(v), v.size)


def quantize_act(x, fmt, with_residue=True):
    """Quantize activation rows x[M, K] (fp32 values; bf16 inputs already widened).

    Returns a dict with stacked rows R = 2M (with residue) or M:
      codes [R, K/2] u8, scales [R, K/blk] u8, globals [R] f32 (zeros for MXFP4),
      deq [R, K] f32 (dequantized values), resid [M, K] f32 (fp32 residue) or None.
    """
    x = _f32(x)
    M, K = x.shape
    blk = BLOCK[fmt]
    assert K % blk == 0
    R = 2 * M if with_residue else M
    codes = np.zeros((R, K // 2), np.uint8)
    scales = np.zeros((R, K // blk), np.uint8)
    globs = np.zeros((R,), np.float32)
    deq = np.zeros((R, K), np.float32)
    resid = np.zeros((M, K), np.float32) if with_residue else None
    lib().oracle_quantize_act(fmt, _p(x), M, K, 1 if with_residue else 0, _p(codes), _p(scales),
                              _p(globs), _p(deq), _p(resid) if with_residue else None)
    return {"codes": codes, "scales": scales, "globals": globs, "deq": deq, "resid": resid}


def quantize_weight_rows(W_rows, fmt, s_gw=0.0, want_deq=True, threads=False):
    """Quantize weight rows W_rows[n, K] with a given NVFP4 tensor scale s_gw
    (threads=True: the OpenMP timing build, the same bits)."""
    W_rows = _f32(W_rows)
    n, K = W_rows.shape
    blk = BLOCK[fmt]
    codes = np.zeros((n, K // 2), np.uint8)
    scales = np.zeros((n, K // blk), np.uint8)
    deq = np.zeros((n, K), np.float32) if want_deq else None
    lib(threads).oracle_quantize_weight_rows(fmt, _p(W_rows), n, K, float(s_gw), _p(codes), _p(scales),
                                             _p(deq) if want_deq else None)
    return {"codes": codes, "scales": scales, "deq": deq}


def quantize_weight(W, fmt, rows=None, want_deq=True, threads=False):
    """Quantize a weight tensor W[N, K] (NVFP4: one tensor scale from max|W|).

    rows: optional index array; only those rows are quantized (the tensor scale
    still comes from the whole tensor).  Returns codes, scales, deq, s_g.
    """
    W = _f32(W)
    s_gw = nvfp4_global_scale(absmax(W)) if fmt == NVFP4 else 0.0
    sub = W if rows is None else W[np.asarray(rows)]
    out = quantize_weight_rows(sub, fmt, s_gw, want_deq, threads)
    out["s_g"] = np.float32(s_gw)
    return out


def unpack_codes(codes, K):
    """[R, K/2] packed nibbles -> [R, K] u8 codes (low nibble = even index)."""
    lo = codes & 15
    hi = codes >> 4
    out = np.empty((codes.shape[0], K), np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def dequant_rows(codes, scales, globals_, fmt, K):
    """Dequantize rows from codes/scales/globals with the oracle's codecs,
    fl(fl(S_b * s_g) * e) for NVFP4 and fl(X * e) for MXFP4."""
    L = lib()
    c = unpack_codes(codes, K)
    e = np.array([L.oracle_e2m1_value(i) for i in range(16)], np.float32)[c]
    blk = BLOCK[fmt]
    if fmt == NVFP4:
        tab = np.array([L.oracle_e4m3_value(i) for i in range(256)], np.float32)
        sb = tab[scales]
        st = (sb * np.asarray(globals_, np.float32).reshape(-1, 1)).astype(np.float32)
    else:
        tab = np.array([L.oracle_e8m0_value(i) for i in range(256)], np.float32)
        st = tab[scales]
    return (np.repeat(st, blk, axis=1) * e).astype(np.float32)


def linear(dx, dw, M, compensated, want_beta=True, threads=False):
    """fp64 linear over dequantized rows: dx [R, K] stacked (R = 2M when
    compensated), dw [N, K].  Returns (y [M, N] f64, beta [M, N] f64).
    threads=True runs the OpenMP timing build (the same bits)."""
    dx = _f32(dx)
    dw = _f32(dw)
    N, K = dw.shape
    y = np.zeros((M, N), np.float64)
    beta = np.zeros((M, N), np.float64) if want_beta else None
    lib(threads).oracle_linear(_p(dx), _p(dw), M, N, K, 1 if compensated else 0, _p(y),
                               _p(beta) if want_beta else None)
    return y, beta


def threads():
    """Threads the OpenMP timing build uses."""
    return int(lib(True).oracle_threads())


# ---------------------------------------------------------------- K-Ext --

def channel_abs_sum(x, prev=None):
    """Calibration score: per-channel sum of |x| over the rows of x[T, K] in
    binary64, rows in order, continuing from prev (a [K] f64 array) if given."""
    x = _f32(x)
    T, K = x.shape
    out = np.zeros((K,), np.float64) if prev is None else np.array(prev, np.float64, copy=True)
    lib().oracle_channel_abs_sum(_p(x), T, K, _p(out))
    return out


def kext_select(score, k):
    """Top-k channels of every 8-channel group (ties to the lower index) as
    K/8 mask bytes."""
    score = np.ascontiguousarray(score, dtype=np.float64)
    K = score.size
    assert K % 8 == 0 and k in (1, 2, 4, 8)
    masks = np.zeros((K // 8,), np.uint8)
    lib().oracle_kext_select(_p(score), K, int(k), _p(masks))
    return masks


def kext_dim(K, k):
    """Effective reduction length K_eff = K + (K/8) k."""
    return K + (K // 8) * k


def _check_masks(masks, K, k):
    masks = np.ascontiguousarray(masks, dtype=np.uint8)
    assert masks.size == K // 8
    pop = np.unpackbits(masks.reshape(-1, 1), axis=1).sum(axis=1)
    assert np.all(pop == k), "every mask byte must select exactly k channels"
    return masks


def kext_extend_weight(W, masks, k):
    """[W | W[:, S]] with the selected columns in extension order (fp32)."""
    W = _f32(W)
    N, K = W.shape
    masks = _check_masks(masks, K, k)
    out = np.zeros((N, kext_dim(K, k)), np.float32)
    lib().oracle_kext_extend_weight(_p(W), N, K, _p(masks), int(k), _p(out))
    return out


def kext_quantize_act(x, fmt, masks, k):
    """K-Ext activation records: codes [M, K_eff/2], scales [M, K_eff/blk],
    globals [M] (NVFP4 base tensor scale), deq [M, K_eff]."""
    x = _f32(x)
    M, K = x.shape
    masks = _check_masks(masks, K, k)
    KE = kext_dim(K, k)
    blk = BLOCK[fmt]
    assert (KE - K) % blk == 0, "the extension must hold whole blocks"
    codes = np.zeros((M, KE // 2), np.uint8)
    scales = np.zeros((M, KE // blk), np.uint8)
    globs = np.zeros((M,), np.float32)
    deq = np.zeros((M, KE), np.float32)
    work = np.zeros((KE - K,), np.float32)
    lib().oracle_kext_quantize_act(fmt, _p(x), M, K, _p(masks), int(k), _p(codes), _p(scales),
                                   _p(globs), _p(deq), _p(work))
    return {"codes": codes, "scales": scales, "globals": globs, "deq": deq}


# ------------------------------------------------- paper numerics (alg1) --

def nvfp4_alpha(x):
    """alpha = fl(fl(amax / 6) / 448) over the whole tensor."""
    x = _f32(x).ravel()
    return np.float32(lib().oracle_nvfp4_alpha(_p(x), x.size))


def quantize_row_alg1(v, alpha):
    """One NVFP4 row with tensor scale alpha: codes, scales, deq, resid."""
    v = _f32(v).ravel()
    K = v.size
    codes = np.zeros((K // 2,), np.uint8)
    scales = np.zeros((K // 16,), np.uint8)
    deq = np.zeros((K,), np.float32)
    resid = np.zeros((K,), np.float32)
    lib().oracle_nvfp4_quantize_row_alg1(_p(v), K, float(alpha), _p(codes), _p(scales), _p(deq), _p(resid))
    return {"codes": codes, "scales": scales, "deq": deq, "resid": resid}


def quantize_act_alg1(x, alpha, with_residue=True):
    """Rows of x[M, K] with one tensor scale alpha (rows stacked [X^; R^])."""
    x = _f32(x)
    M, K = x.shape
    R = 2 * M if with_residue else M
    codes = np.zeros((R, K // 2), np.uint8)
    scales = np.zeros((R, K // 16), np.uint8)
    globs = np.zeros((R,), np.float32)
    deq = np.zeros((R, K), np.float32)
    resid = np.zeros((M, K), np.float32) if with_residue else None
    work = np.zeros((K,), np.float32)
    lib().oracle_quantize_act_alg1(_p(x), M, K, float(alpha), 1 if with_residue else 0, _p(codes), _p(scales),
                                   _p(globs), _p(deq), _p(resid) if with_residue else None, _p(work))
    return {"codes": codes, "scales": scales, "globals": globs, "deq": deq, "resid": resid}


# ------------------------------------------------- decode attention (ResAttn) --

def kv_quantize(x, g):
    """NVFP4 rows of a K or V tensor [..., d] with a given global scale g (the
    cache's tensor scale): codes [..., d/2], scales [..., d/16], deq [..., d]."""
    x = _f32(x)
    shp = x.shape
    d = shp[-1]
    rows = x.reshape(-1, d)
    q = quantize_weight_rows(rows, NVFP4, float(g), True)
    return {"codes": q["codes"].reshape(shp[:-1] + (d // 2,)),
            "scales": q["scales"].reshape(shp[:-1] + (d // 16,)),
            "deq": q["deq"].reshape(shp)}


def attention_decode(qb, qr, kd, vd, sm_scale):
    """binary64 decode attention of one sequence: qb, qr [H_q, d] dequantized
    query base / residue (qr None: uncompensated), kd, vd [L, H_kv, d]."""
    qb = _f32(qb)
    H_q, d = qb.shape
    kd = _f32(kd)
    vd = _f32(vd)
    L, H_kv, _ = kd.shape
    out = np.zeros((H_q, d), np.float64)
    work = np.zeros((max(L, 1),), np.float64)
    qrp = _p(_f32(qr)) if qr is not None else None
    if qr is not None:
        qr = _f32(qr)
        qrp = _p(qr)
    lib().oracle_attention_decode(_p(qb), qrp, _p(kd), _p(vd), L, H_q, H_kv, d, float(sm_scale), _p(out),
                                  _p(work))
    return out

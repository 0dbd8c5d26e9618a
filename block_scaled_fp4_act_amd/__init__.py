"""Residue-compensated block-scaled FP4 linear for AMD Instinct MI355X (gfx950).

A thin binding over the C ABI in include/rsfp4.h (librsfp4.so): it only
marshals torch tensors (device memory) and the current HIP stream into the C
calls; every step of the path runs in the library's HIP kernels.  There is no
CPU fallback: a missing library raises.

Names follow the C ABI: ``nvfp4_prepack_weights``, ``nvfp4_quantize_act_with_residue``,
``nvfp4_linear``, ``nvfp4_linear_compensated`` and the ``mxfp4_`` twins, plus the
format-generic ``prepack_weights``, ``quantize_act_with_residue``, ``fp4_linear``
and ``fp4_linear_compensated``.  Selective compensation (K-Ext):
``channel_abs_sum``, ``kext_select``, ``kext_dim``, ``prepack_weights_kext``,
``quantize_act_kext`` (and the ``nvfp4_`` / ``mxfp4_`` forms); the product is
then the plain ``fp4_linear`` over K_eff = kext_dim(K, k).  Paper numerics:
``nvfp4_tensor_alpha``, ``nvfp4_quantize_act_alpha`` and the bf16-output
``fp4_linear_bf16`` / ``fp4_linear_compensated_bf16``.  Decode attention:
``kv_cache_write`` and ``resattn_decode`` (queries quantized with
``nvfp4_quantize_act_with_residue``).
"""
import ctypes

from ._lib import lib

NVFP4, MXFP4 = 0, 1
F32, BF16 = 0, 1
BLOCK = {NVFP4: 16, MXFP4: 32}
_FMT_NAME = {NVFP4: "nvfp4", MXFP4: "mxfp4"}


def _fmt(fmt):
    if isinstance(fmt, str):
        fmt = {"nvfp4": NVFP4, "mxfp4": MXFP4}[fmt.lower()]
    return int(fmt)


def _check(status):
    if status != 0:
        L = lib()
        raise RuntimeError(f"rsfp4: {L.rsfp4_status_string(status).decode()}: "
                           f"{L.rsfp4_last_error().decode()}")


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


# ------------------------------------------------------------------ sizes --

def act_row_bytes(fmt, K):
    return int(lib().rsfp4_act_row_bytes(_fmt(fmt), K))


def packed_act_bytes(fmt, M, K, with_residue=True):
    return int(lib().rsfp4_packed_act_bytes(_fmt(fmt), M, K, 1 if with_residue else 0))


def packed_weight_bytes(fmt, N, K):
    return int(lib().rsfp4_packed_weight_bytes(_fmt(fmt), N, K))


def workspace_bytes(fmt, M, N, K, compensated=True):
    return int(lib().rsfp4_workspace_bytes(_fmt(fmt), M, N, K, 1 if compensated else 0))


_WS = {}


def _workspace(fmt, M, N, K, comp, ws, device):
    """The linear's workspace: `ws` when given (a uint8 cuda tensor, zero-filled
    before its first use), else one zero-filled buffer per device kept here and
    shared by every call that passes none (the library leaves its counters
    zero after each call, so calls in stream order can share it; calls that
    may run concurrently on other streams must pass their own)."""
    import torch
    need = workspace_bytes(fmt, M, N, K, comp)
    if ws is not None:
        return ws
    if need == 0:
        return None
    key = torch.device(device).index if torch.device(device).index is not None else torch.cuda.current_device()
    buf = _WS.get(key)
    if buf is None or buf.numel() < need:
        buf = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf


# ---------------------------------------------------------------- prepack --

def prepack_weights(W, fmt, out=None):
    """Quantize W[N, K] (cuda, fp32/bf16) into a packed uint8 blob (offline step)."""
    import torch
    fmt = _fmt(fmt)
    assert W.is_cuda and W.dim() == 2 and W.is_contiguous()
    N, K = W.shape
    nbytes = packed_weight_bytes(fmt, N, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    fn = getattr(lib(), f"rsfp4_{_FMT_NAME[fmt]}_prepack_weights")
    _check(fn(_ptr(W), _dtype_code(W), N, K, _ptr(out), out.numel(), _stream(W)))
    return out


def nvfp4_prepack_weights(W, out=None):
    return prepack_weights(W, NVFP4, out)


def mxfp4_prepack_weights(W, out=None):
    return prepack_weights(W, MXFP4, out)


# --------------------------------------------------------------- quantize --

def quantize_act_with_residue(x, fmt, with_residue=True, out=None):
    """Quantize x[M, K] (cuda, fp32/bf16) into the activation buffer (uint8)."""
    import torch
    fmt = _fmt(fmt)
    assert x.is_cuda and x.dim() == 2 and x.is_contiguous()
    M, K = x.shape
    nbytes = packed_act_bytes(fmt, M, K, with_residue)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    fn = getattr(lib(), f"rsfp4_{_FMT_NAME[fmt]}_quantize_act_with_residue")
    _check(fn(_ptr(x), _dtype_code(x), M, K, 1 if with_residue else 0, _ptr(out), out.numel(), _stream(x)))
    return out


def nvfp4_quantize_act_with_residue(x, with_residue=True, out=None):
    return quantize_act_with_residue(x, NVFP4, with_residue, out)


def mxfp4_quantize_act_with_residue(x, with_residue=True, out=None):
    return quantize_act_with_residue(x, MXFP4, with_residue, out)


def act_views(act, fmt, M, K, with_residue=True):
    """Canonical views into an activation buffer: codes [R, K/2], scales
    [R, K/blk] (uint8) and the per-row fp32 tensor scales [R] (slicing only)."""
    fmt = _fmt(fmt)
    R = 2 * M if with_residue else M
    rb = act_row_bytes(fmt, K)
    rows = act[: R * rb].view(R, rb)
    codes = rows[:, 16:16 + K // 2]
    scales = rows[:, 16 + K // 2:16 + K // 2 + K // BLOCK[fmt]]
    globs = rows[:, 0:4].contiguous().view(-1).view(__import__("torch").float32)
    return codes, scales, globs


# ----------------------------------------------------------------- linear --

def _linear(act, w_packed, M, N, K, fmt, comp, out, bf16=False, ws=None):
    import torch
    fmt = _fmt(fmt)
    dt = torch.bfloat16 if bf16 else torch.float32
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=act.device)
    assert out.is_cuda and out.dtype == dt and out.is_contiguous() and out.numel() >= M * N
    ws = _workspace(fmt, M, N, K, comp, ws, act.device)
    name = f"rsfp4_{_FMT_NAME[fmt]}_linear" + ("_compensated" if comp else "") + ("_bf16" if bf16 else "")
    _check(getattr(lib(), name)(_ptr(act), act.numel(), _ptr(w_packed), w_packed.numel(), M, N, K,
                                _ptr(out), _ptr(ws), ws.numel() if ws is not None else 0, _stream(act)))
    return out


def fp4_linear(act, w_packed, M, N, K, fmt, out=None, ws=None):
    """y = deq(q(x)) W^T (plain W4A4), fp32 [M, N]."""
    return _linear(act, w_packed, M, N, K, fmt, False, out, ws=ws)


def fp4_linear_compensated(act, w_packed, M, N, K, fmt, out=None, ws=None):
    """y = deq(q(x)) W^T + deq(q(r)) W^T (residue-compensated), fp32 [M, N].
    ws: the split-K workspace (workspace_bytes; a shared one when omitted)."""
    return _linear(act, w_packed, M, N, K, fmt, True, out, ws=ws)


def fp4_linear_bf16(act, w_packed, M, N, K, fmt, out=None, ws=None):
    """As fp4_linear, bf16 output (round to nearest even)."""
    return _linear(act, w_packed, M, N, K, fmt, False, out, bf16=True, ws=ws)


def fp4_linear_compensated_bf16(act, w_packed, M, N, K, fmt, out=None, ws=None):
    """As fp4_linear_compensated, bf16 output (round to nearest even)."""
    return _linear(act, w_packed, M, N, K, fmt, True, out, bf16=True, ws=ws)


def nvfp4_linear(act, w_packed, M, N, K, out=None):
    return _linear(act, w_packed, M, N, K, NVFP4, False, out)


def nvfp4_linear_compensated(act, w_packed, M, N, K, out=None):
    return _linear(act, w_packed, M, N, K, NVFP4, True, out)


def nvfp4_linear_compensated_noalloc(act, w_packed, M, N, K, out):
    """rsfp4_nvfp4_linear_compensated_noalloc: the compensated NVFP4 linear
    with the library's own scratch as workspace (no allocation in the call);
    out: the caller's fp32 [M, N] cuda tensor."""
    import torch
    assert out.is_cuda and out.dtype == torch.float32 and out.is_contiguous() and out.numel() >= M * N
    _check(lib().rsfp4_nvfp4_linear_compensated_noalloc(_ptr(act), act.numel(), _ptr(w_packed), w_packed.numel(),
                                                        M, N, K, _ptr(out), _stream(act)))
    return out


def mxfp4_linear(act, w_packed, M, N, K, out=None):
    return _linear(act, w_packed, M, N, K, MXFP4, False, out)


def mxfp4_linear_compensated(act, w_packed, M, N, K, out=None):
    return _linear(act, w_packed, M, N, K, MXFP4, True, out)


# ------------------------------------ grouped linear (mixture of experts) --

def fp4_grouped_linear(act, w_packed, M_total, E, offsets, max_rows, N, K, fmt, compensated=True, out=None):
    """Expert e: rows offsets[e] .. offsets[e+1]-1 of act (M_total quantized
    rows, with residue rows when compensated) times the e-th of E stacked
    blobs in w_packed -> the same rows of y [M_total, N] (fp32).  offsets:
    int32 cuda tensor [E + 1]; max_rows bounds every expert's rows."""
    import torch
    fmt = _fmt(fmt)
    assert offsets.is_cuda and offsets.dtype == torch.int32 and offsets.numel() >= E + 1
    if out is None:
        out = torch.zeros((M_total, N), dtype=torch.float32, device=act.device)
    assert out.is_cuda and out.dtype == torch.float32 and out.is_contiguous() and out.numel() >= M_total * N
    name = f"rsfp4_{_FMT_NAME[fmt]}_grouped_linear" + ("_compensated" if compensated else "")
    _check(getattr(lib(), name)(_ptr(act), act.numel(), M_total, _ptr(w_packed), w_packed.numel(), E, _ptr(offsets),
                                max_rows, N, K, _ptr(out), _stream(act)))
    return out


# ------------------------------------------- quantize + linear in one call --

def from_x_launches(fmt, M, N, K, compensated=True, x_dtype=None):
    """1 or 2: the kernel launches fp4_linear_from_x makes for this shape."""
    import torch
    xt = _dtype_code(torch.empty(0, dtype=x_dtype if x_dtype is not None else torch.bfloat16))
    return lib().rsfp4_from_x_launches(_fmt(fmt), xt, M, N, K, 1 if compensated else 0)


def fp4_linear_from_x(x, w_packed, N, fmt, compensated=True, out=None, out_dtype=None, act=None, ws=None):
    """Quantize x[M, K] (cuda, fp32/bf16) and apply the linear in one call:
    y [M, N] (fp32, or bf16 with out_dtype=torch.bfloat16).  act: an
    activation buffer of packed_act_bytes(fmt, M, K, compensated) bytes that
    the call uses where the quantizer and the linear run as two launches
    (allocated here when omitted); ws: the linear's workspace, as for
    fp4_linear_compensated."""
    import torch
    fmt = _fmt(fmt)
    assert x.is_cuda and x.dim() == 2 and x.is_contiguous()
    M, K = x.shape
    dt = out_dtype if out_dtype is not None else (out.dtype if out is not None else torch.float32)
    assert dt in (torch.float32, torch.bfloat16)
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=x.device)
    assert out.is_cuda and out.dtype == dt and out.is_contiguous() and out.numel() >= M * N
    if act is None:
        act = torch.empty(packed_act_bytes(fmt, M, K, compensated), dtype=torch.uint8, device=x.device)
    ws = _workspace(fmt, M, N, K, compensated, ws, x.device)
    name = f"rsfp4_{_FMT_NAME[fmt]}_linear" + ("_compensated" if compensated else "") + "_from_x"
    _check(getattr(lib(), name)(_ptr(x), _dtype_code(x), M, N, K, _ptr(w_packed), w_packed.numel(), _ptr(out),
                                _dtype_code(out), _ptr(act), act.numel(), _ptr(ws),
                                ws.numel() if ws is not None else 0, _stream(x)))
    return out


# ------------------------------------------- paper numerics (tensor scale) --

def nvfp4_tensor_alpha(x, out=None):
    """alpha = ((max|x|) / 6) / 448 of a whole tensor, as a 1-element fp32 tensor."""
    import torch
    assert x.is_cuda and x.is_contiguous()
    M = x.shape[0] if x.dim() > 1 else 1
    K = x.numel() // M
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(lib().rsfp4_nvfp4_tensor_alpha(_ptr(x), _dtype_code(x), M, K, _ptr(out), _stream(x)))
    return out


def nvfp4_quantize_act_alpha(x, alpha, with_residue=True, out=None):
    """Paper-numerics NVFP4 quantization of x[M, K] with tensor scale alpha
    (a 1-element fp32 cuda tensor), shared by x and r."""
    import torch
    assert x.is_cuda and x.dim() == 2 and x.is_contiguous()
    assert alpha.is_cuda and alpha.dtype == torch.float32
    M, K = x.shape
    nbytes = packed_act_bytes(NVFP4, M, K, with_residue)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    _check(lib().rsfp4_nvfp4_quantize_act_alpha(_ptr(x), _dtype_code(x), M, K, _ptr(alpha),
                                                1 if with_residue else 0, _ptr(out), out.numel(), _stream(x)))
    return out


# ------------------------------------------------ decode attention (ResAttn) --

def kv_page_bytes(H_kv, D):
    return int(lib().rsfp4_kv_page_bytes(H_kv, D))


def kv_cache_write(k, v, slots, cache, k_scale=1.0, v_scale=1.0):
    """Quantize k, v [T, H_kv, D] (cuda, fp32/bf16) into the paged NVFP4 cache
    (uint8 cuda tensor) at slots [T] (int32: page * 32 + row)."""
    import torch
    assert k.is_cuda and k.dim() == 3 and k.is_contiguous() and v.shape == k.shape and v.dtype == k.dtype
    assert slots.is_cuda and slots.dtype == torch.int32 and cache.is_cuda and cache.dtype == torch.uint8
    T, H_kv, D = k.shape
    _check(lib().rsfp4_kv_cache_write(_ptr(k), _ptr(v.contiguous()), _dtype_code(k), T, H_kv, D, _ptr(slots),
                                      float(k_scale), float(v_scale), _ptr(cache), cache.numel(), _stream(k)))
    return cache


def resattn_splits(B, H_kv, max_seq_len):
    return int(lib().rsfp4_resattn_splits(B, H_kv, max_seq_len))


def resattn_decode(q_act, cache, block_table, seq_lens, max_seq_len, B, H_q, H_kv, D, compensated=True,
                   k_scale=1.0, v_scale=1.0, sm_scale=None, splits=0, out=None, out_bf16=False, ws=None):
    """Compensated (or plain) decode attention; returns out [B, H_q, D]."""
    import math
    import torch
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if splits <= 0:
        splits = resattn_splits(B, H_kv, max_seq_len)
    need = int(lib().rsfp4_resattn_workspace_bytes(B, H_q, D, splits))
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=cache.device)
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.bfloat16 if out_bf16 else torch.float32, device=cache.device)
    max_pages = block_table.shape[1]
    _check(lib().rsfp4_resattn_decode(_ptr(q_act), q_act.numel(), 1 if compensated else 0, _ptr(cache),
                                      cache.numel(), _ptr(block_table), max_pages, _ptr(seq_lens), max_seq_len, B,
                                      H_q, H_kv, D, float(k_scale), float(v_scale), float(sm_scale), int(splits),
                                      _ptr(out), 1 if out_bf16 else 0, _ptr(ws) if ws is not None else None,
                                      ws.numel() if ws is not None else 0, _stream(cache)))
    return out


# ---------------------------------------------------------------- K-Ext --

def kext_dim(K, k):
    """K_eff = K + (K/8) k (raises for an unsupported K, k)."""
    ke = int(lib().rsfp4_kext_dim(K, k))
    if ke < 0:
        raise ValueError(f"K = {K}, k = {k}: no whole-block extension (see rsfp4_kext_dim)")
    return ke


def channel_abs_sum(x, out=None, accumulate=False):
    """Per-channel sum of |x| over the rows of x[T, K] in float64 (calibration)."""
    import torch
    assert x.is_cuda and x.dim() == 2 and x.is_contiguous()
    T, K = x.shape
    if out is None:
        out = torch.zeros(K, dtype=torch.float64, device=x.device)
    assert out.dtype == torch.float64 and out.is_contiguous() and out.numel() >= K
    _check(lib().rsfp4_channel_abs_sum(_ptr(x), _dtype_code(x), T, K, _ptr(out), 1 if accumulate else 0,
                                       _stream(x)))
    return out


def kext_select(score, k, out=None):
    """K/8 mask bytes: the k best channels of every group of 8."""
    import torch
    assert score.is_cuda and score.dtype == torch.float64 and score.is_contiguous()
    K = score.numel()
    if out is None:
        out = torch.empty(K // 8, dtype=torch.uint8, device=score.device)
    _check(lib().rsfp4_kext_select(_ptr(score), K, int(k), _ptr(out), _stream(score)))
    return out


def prepack_weights_kext(W, fmt, masks, k, out=None):
    """Pack [W | W_S] (width K_eff) into a blob for the plain linear."""
    import torch
    fmt = _fmt(fmt)
    assert W.is_cuda and W.dim() == 2 and W.is_contiguous() and masks.is_cuda and masks.dtype == torch.uint8
    N, K = W.shape
    nbytes = packed_weight_bytes(fmt, N, kext_dim(K, k))
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    fn = getattr(lib(), f"rsfp4_{_FMT_NAME[fmt]}_prepack_weights_kext")
    _check(fn(_ptr(W), _dtype_code(W), N, K, _ptr(masks), int(k), _ptr(out), out.numel(), _stream(W)))
    return out


def quantize_act_kext(x, fmt, masks, k, out=None):
    """Quantize x[M, K] into M records of width K_eff (base + selected residues)."""
    import torch
    fmt = _fmt(fmt)
    assert x.is_cuda and x.dim() == 2 and x.is_contiguous() and masks.is_cuda and masks.dtype == torch.uint8
    M, K = x.shape
    nbytes = packed_act_bytes(fmt, M, kext_dim(K, k), False)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    fn = getattr(lib(), f"rsfp4_{_FMT_NAME[fmt]}_quantize_act_kext")
    _check(fn(_ptr(x), _dtype_code(x), M, K, _ptr(masks), int(k), _ptr(out), out.numel(), _stream(x)))
    return out


def nvfp4_prepack_weights_kext(W, masks, k, out=None):
    return prepack_weights_kext(W, NVFP4, masks, k, out)


def mxfp4_prepack_weights_kext(W, masks, k, out=None):
    return prepack_weights_kext(W, MXFP4, masks, k, out)


def nvfp4_quantize_act_kext(x, masks, k, out=None):
    return quantize_act_kext(x, NVFP4, masks, k, out)


def mxfp4_quantize_act_kext(x, masks, k, out=None):
    return quantize_act_kext(x, MXFP4, masks, k, out)


# ------------------------------------------------------------ test/debug --

def validate_packed(w_packed):
    """(fmt, N, K) from a packed weight blob's header after checking it;
    raises RuntimeError on a bad header (synchronizes the current stream)."""
    f, n, k = ctypes.c_int(0), ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().rsfp4_validate_packed(_ptr(w_packed), w_packed.numel(), ctypes.byref(f), ctypes.byref(n),
                                       ctypes.byref(k), _stream(w_packed)))
    return f.value, n.value, k.value


def unpack_weights_canonical(w_packed, fmt, N, K):
    """Canonical codes [N, K/2], scales [N, K/blk] and the NVFP4 tensor scale."""
    import torch
    fmt = _fmt(fmt)
    dev = w_packed.device
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, K // BLOCK[fmt]), dtype=torch.uint8, device=dev)
    s_g = torch.zeros(1, dtype=torch.float32, device=dev)
    _check(lib().rsfp4_unpack_weights_canonical(_ptr(w_packed), w_packed.numel(), fmt, N, K, _ptr(codes),
                                                _ptr(scales), _ptr(s_g), _stream(w_packed)))
    return codes, scales, s_g


# ------------------------------------------------------------ measurement --

def stream_read(src, sink=None):
    """Read the uint8 cuda tensor src once with the library's streaming-read
    kernel (the reference read rate); sink: a 1-element int32 cuda tensor that
    the kernel xors the xor of all 32-bit words of src into."""
    import torch
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=src.device)
    _check(lib().rsfp4_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(src)))
    return sink

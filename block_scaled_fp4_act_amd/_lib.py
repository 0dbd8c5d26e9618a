"""ctypes loader of librsfp4.so and the signatures of include/rsfp4.h."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librsfp4.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "rsfp4.h")

_lib = None

P = ctypes.c_void_p
I64 = ctypes.c_int64
INT = ctypes.c_int
SZ = ctypes.c_size_t

SIGNATURES = {
    "rsfp4_abi_version": (INT, []),
    "rsfp4_status_string": (ctypes.c_char_p, [INT]),
    "rsfp4_last_error": (ctypes.c_char_p, []),
    "rsfp4_act_row_bytes": (SZ, [INT, I64]),
    "rsfp4_packed_act_bytes": (SZ, [INT, I64, I64, INT]),
    "rsfp4_packed_weight_bytes": (SZ, [INT, I64, I64]),
    "rsfp4_workspace_bytes": (SZ, [INT, I64, I64, I64, INT]),
    "rsfp4_nvfp4_prepack_weights": (INT, [P, INT, I64, I64, P, SZ, P]),
    "rsfp4_mxfp4_prepack_weights": (INT, [P, INT, I64, I64, P, SZ, P]),
    "rsfp4_nvfp4_quantize_act_with_residue": (INT, [P, INT, I64, I64, INT, P, SZ, P]),
    "rsfp4_mxfp4_quantize_act_with_residue": (INT, [P, INT, I64, I64, INT, P, SZ, P]),
    "rsfp4_nvfp4_linear": (INT, [P, SZ, P, SZ, I64, I64, I64, P, P, SZ, P]),
    "rsfp4_nvfp4_linear_compensated": (INT, [P, SZ, P, SZ, I64, I64, I64, P, P, SZ, P]),
    "rsfp4_nvfp4_linear_compensated_noalloc": (INT, [P, SZ, P, SZ, I64, I64, I64, P, P]),
    "rsfp4_stream_read": (INT, [P, SZ, P, P]),
    "rsfp4_mxfp4_linear": (INT, [P, SZ, P, SZ, I64, I64, I64, P, P, SZ, P]),
    "rsfp4_mxfp4_linear_compensated": (INT, [P, SZ, P, SZ, I64, I64, I64, P, P, SZ, P]),
    "rsfp4_unpack_weights_canonical": (INT, [P, SZ, INT, I64, I64, P, P, P, P]),
    "rsfp4_validate_packed": (INT, [P, SZ, P, P, P, P]),
    "rsfp4_nvfp4_linear_bf16": (INT, [P, SZ, P, SZ, I64, I64, I64, P, P, SZ, P]),
    "rsfp4_nvfp4_linear_compensated_bf16": (INT, [P, SZ, P, SZ, I64, I64, I64, P, P, SZ, P]),
    "rsfp4_mxfp4_linear_bf16": (INT, [P, SZ, P, SZ, I64, I64, I64, P, P, SZ, P]),
    "rsfp4_mxfp4_linear_compensated_bf16": (INT, [P, SZ, P, SZ, I64, I64, I64, P, P, SZ, P]),
    "rsfp4_from_x_launches": (INT, [INT, INT, I64, I64, I64, INT]),
    "rsfp4_nvfp4_grouped_linear": (INT, [P, SZ, I64, P, SZ, I64, P, I64, I64, I64, P, P]),
    "rsfp4_nvfp4_grouped_linear_compensated": (INT, [P, SZ, I64, P, SZ, I64, P, I64, I64, I64, P, P]),
    "rsfp4_mxfp4_grouped_linear": (INT, [P, SZ, I64, P, SZ, I64, P, I64, I64, I64, P, P]),
    "rsfp4_mxfp4_grouped_linear_compensated": (INT, [P, SZ, I64, P, SZ, I64, P, I64, I64, I64, P, P]),
    "rsfp4_nvfp4_linear_from_x": (INT, [P, INT, I64, I64, I64, P, SZ, P, INT, P, SZ, P, SZ, P]),
    "rsfp4_nvfp4_linear_compensated_from_x": (INT, [P, INT, I64, I64, I64, P, SZ, P, INT, P, SZ, P, SZ, P]),
    "rsfp4_mxfp4_linear_from_x": (INT, [P, INT, I64, I64, I64, P, SZ, P, INT, P, SZ, P, SZ, P]),
    "rsfp4_mxfp4_linear_compensated_from_x": (INT, [P, INT, I64, I64, I64, P, SZ, P, INT, P, SZ, P, SZ, P]),
    "rsfp4_nvfp4_quantize_act_alpha": (INT, [P, INT, I64, I64, P, INT, P, SZ, P]),
    "rsfp4_nvfp4_tensor_alpha": (INT, [P, INT, I64, I64, P, P]),
    "rsfp4_kv_page_bytes": (SZ, [I64, I64]),
    "rsfp4_kv_cache_write": (INT, [P, P, INT, I64, I64, I64, P, ctypes.c_float, ctypes.c_float, P, SZ, P]),
    "rsfp4_resattn_splits": (INT, [I64, I64, I64]),
    "rsfp4_resattn_workspace_bytes": (SZ, [I64, I64, I64, INT]),
    "rsfp4_resattn_decode": (INT, [P, SZ, INT, P, SZ, P, I64, P, I64, I64, I64, I64, I64, ctypes.c_float,
                                   ctypes.c_float, ctypes.c_float, INT, P, INT, P, SZ, P]),
    "rsfp4_kext_dim": (I64, [I64, INT]),
    "rsfp4_channel_abs_sum": (INT, [P, INT, I64, I64, P, INT, P]),
    "rsfp4_kext_select": (INT, [P, I64, INT, P, P]),
    "rsfp4_nvfp4_prepack_weights_kext": (INT, [P, INT, I64, I64, P, INT, P, SZ, P]),
    "rsfp4_mxfp4_prepack_weights_kext": (INT, [P, INT, I64, I64, P, INT, P, SZ, P]),
    "rsfp4_nvfp4_quantize_act_kext": (INT, [P, INT, I64, I64, P, INT, P, SZ, P]),
    "rsfp4_mxfp4_quantize_act_kext": (INT, [P, INT, I64, I64, P, INT, P, SZ, P]),
}


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"librsfp4.so is missing at {LIB_PATH}: build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'` (there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib

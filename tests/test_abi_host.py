"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/rsfp4.h declares, answers the size queries, and rejects
bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import block_scaled_fp4_act_amd as rs
from block_scaled_fp4_act_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "rsfp4.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rsfp4_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = rs.lib()
    names = _declared()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_version_and_strings():
    L = rs.lib()
    assert L.rsfp4_abi_version() == 1
    for s in range(8):
        assert L.rsfp4_status_string(s)
    assert L.rsfp4_status_string(99) == b"unknown status"


def test_size_queries():
    # act records: 16-byte head + K/2 codes + K/blk scales, padded to 16
    assert rs.act_row_bytes(0, 4096) == 16 + 2048 + 256
    assert rs.act_row_bytes(1, 4096) == 16 + 2048 + 128
    assert rs.act_row_bytes(0, 32) == 48 and rs.act_row_bytes(1, 32) == 48
    assert rs.packed_act_bytes(0, 4, 4096, True) == 8 * 2320
    assert rs.packed_act_bytes(0, 4, 4096, False) == 4 * 2320
    # weights: header + groups(16 ch) x quads(4 steps of 128 K) x (4 KB codes + scales)
    assert rs.packed_weight_bytes(0, 4096, 4096) == 256 + 256 * 8 * (4096 + 512)
    assert rs.packed_weight_bytes(1, 25600, 5120) == 256 + 1600 * 10 * (4096 + 256)
    assert rs.packed_weight_bytes(0, 17, 160) == 256 + 2 * 1 * (4096 + 512)   # padded quad
    assert rs.workspace_bytes(0, 4, 4096, 4096, True) == 0
    # wide MXFP4 operands (more than 32 stacked rows): the 16 KB counter area,
    # then the activation operand rewritten as groups of 16 rows x quads of
    # 4 steps (4 KB codes + 256 B scale words)
    assert rs.workspace_bytes(1, 256, 25600, 5120, True) == 16384 + 32 * 10 * (4096 + 256)
    assert rs.workspace_bytes(1, 40, 64, 1056, False) == 16384 + 3 * 3 * (4096 + 256)
    assert rs.workspace_bytes(1, 17, 64, 1056, True) == 16384 + 3 * 3 * (4096 + 256)
    # NVFP4: 4 KB of f16 fragments per 16 rows and step (33..64 compensated
    # rows with N, K <= 4096 take the narrow kernel and no such workspace;
    # without a device the size leaves out a split's partial sums)
    assert rs.workspace_bytes(0, 128, 28672, 8192, True) == 16384 + 16 * 64 * 4096
    assert rs.workspace_bytes(0, 40, 64, 1056, False) == 16384 + 3 * 9 * 4096
    assert rs.workspace_bytes(0, 20, 28672, 8192, True) == 16384 + 3 * 64 * 4096
    assert rs.workspace_bytes(0, 20, 4096, 8192, True) == 16384 + 3 * 64 * 4096
    assert rs.workspace_bytes(0, 20, 4096, 4096, True) == 0
    # invalid requests size to 0
    assert rs.packed_weight_bytes(0, 16, 48) == 0
    assert rs.packed_weight_bytes(2, 16, 64) == 0
    assert rs.act_row_bytes(0, 0) == 0


def _err():
    return rs.lib().rsfp4_last_error().decode()


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first


def test_validation_errors_without_device():
    L = rs.lib()
    # null pointers
    assert L.rsfp4_nvfp4_linear(None, 0, None, 0, 1, 16, 128, None, None, 0, None) == 1
    assert "non-NULL" in _err()
    # bad K
    assert L.rsfp4_nvfp4_linear(FAKE, 1 << 20, FAKE, 1 << 20, 1, 16, 100, FAKE, None, 0, None) == 2
    assert L.rsfp4_mxfp4_quantize_act_with_residue(FAKE, 0, 1, 48, 1, FAKE, 1 << 20, None) == 2
    # K above the linear's limit, M outside [1, 65535]
    assert L.rsfp4_nvfp4_linear(FAKE, 1 << 30, FAKE, 1 << 30, 1, 16, 32800, FAKE, None, 0, None) == 6
    # the tiled kernel's activation operand must stay below 2^31 bytes
    big = 1 << 40
    assert L.rsfp4_nvfp4_linear_compensated(FAKE, big, FAKE, big, 65535, 16, 32768, FAKE, None, 0, None) == 6
    assert "2^31" in _err()
    assert L.rsfp4_mxfp4_linear_compensated(FAKE, 1 << 30, FAKE, 1 << 30, 65536, 16, 512, FAKE, None, 0, None) == 2
    assert L.rsfp4_mxfp4_linear(FAKE, 1 << 30, FAKE, 1 << 30, 0, 16, 512, FAKE, None, 0, None) == 2
    # a wide operand's buffer is checked like a narrow one's
    assert L.rsfp4_mxfp4_linear_compensated(FAKE, 1000, FAKE, 1 << 30, 40, 16, 512, FAKE, None, 0, None) == 5
    # quantize K limit and M limit
    assert L.rsfp4_nvfp4_quantize_act_with_residue(FAKE, 0, 1, 32800, 1, FAKE, 1 << 30, None) == 2
    assert L.rsfp4_nvfp4_quantize_act_with_residue(FAKE, 0, 0, 512, 1, FAKE, 1 << 30, None) == 2
    # unknown dtype / format
    assert L.rsfp4_nvfp4_quantize_act_with_residue(FAKE, 5, 1, 512, 1, FAKE, 1 << 30, None) == 4
    assert L.rsfp4_unpack_weights_canonical(FAKE, 1 << 30, 3, 16, 512, FAKE, FAKE, None, None) == 4
    # alignment
    odd = ctypes.c_void_p(0x100001)
    assert L.rsfp4_nvfp4_quantize_act_with_residue(odd, 0, 1, 512, 1, FAKE, 1 << 30, None) == 3
    assert L.rsfp4_nvfp4_prepack_weights(FAKE, 0, 16, 512, ctypes.c_void_p(0x100010), 1 << 30, None) == 3
    # buffer sizes
    assert L.rsfp4_nvfp4_quantize_act_with_residue(FAKE, 0, 4, 512, 1, FAKE, 100, None) == 5
    assert "needs" in _err()
    assert L.rsfp4_nvfp4_prepack_weights(FAKE, 0, 16, 512, FAKE, 100, None) == 5
    assert L.rsfp4_nvfp4_linear_compensated(FAKE, 100, FAKE, 1 << 30, 2, 16, 512, FAKE, None, 0, None) == 5
    assert L.rsfp4_nvfp4_linear(FAKE, 1 << 30, FAKE, 100, 2, 16, 512, FAKE, None, 0, None) == 5


def test_binding_raises_on_error():
    with pytest.raises(RuntimeError, match="bad shape"):
        rs._check(2) if False else rs._check(rs.lib().rsfp4_nvfp4_linear(
            FAKE, 1 << 20, FAKE, 1 << 20, 1, 16, 100, FAKE, None, 0, None))


def test_product_path_does_not_import_oracle():
    """The package never reaches the oracle: no module under it names it."""
    pkg = os.path.dirname(rs.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                txt = open(os.path.join(root, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "rsfp4_oracle" not in txt, f


def test_kext_dim_and_validation():
    L = rs.lib()
    assert rs.kext_dim(4096, 1) == 4096 + 512
    assert rs.kext_dim(4096, 2) == 5120 and rs.kext_dim(4096, 4) == 6144 and rs.kext_dim(4096, 8) == 8192
    assert rs.kext_dim(128, 2) == 160 and rs.kext_dim(64, 4) == 96 and rs.kext_dim(32, 8) == 64
    for K, k in ((160, 1), (4096, 3), (96, 2), (48, 8), (0, 1)):
        assert L.rsfp4_kext_dim(K, k) == -1
        with pytest.raises(ValueError):
            rs.kext_dim(K, k)
    # the extended calls check like the plain ones, against K_eff
    assert L.rsfp4_nvfp4_quantize_act_kext(FAKE, 0, 4, 512, FAKE, 3, FAKE, 1 << 30, None) == 2
    assert "1, 2, 4 or 8" in _err()
    assert L.rsfp4_mxfp4_quantize_act_kext(FAKE, 0, 4, 160, FAKE, 1, FAKE, 1 << 30, None) == 2
    assert L.rsfp4_nvfp4_quantize_act_kext(FAKE, 0, 4, 512, None, 2, FAKE, 1 << 30, None) == 1
    need = rs.packed_act_bytes(0, 4, 640, False)
    assert L.rsfp4_nvfp4_quantize_act_kext(FAKE, 0, 4, 512, FAKE, 2, FAKE, need - 1, None) == 5
    assert L.rsfp4_nvfp4_quantize_act_kext(FAKE, 0, 4, 32768, FAKE, 1, FAKE, 1 << 40, None) == 2
    wneed = rs.packed_weight_bytes(1, 64, 768)
    assert L.rsfp4_mxfp4_prepack_weights_kext(FAKE, 0, 64, 512, FAKE, 4, FAKE, wneed - 1, None) == 5
    assert L.rsfp4_mxfp4_prepack_weights_kext(FAKE, 0, 64, 512, FAKE, 4, ctypes.c_void_p(0x100010), wneed, None) == 3
    assert L.rsfp4_kext_select(FAKE, 100, 2, FAKE, None) == 2
    assert L.rsfp4_kext_select(FAKE, 64, 5, FAKE, None) == 2
    assert L.rsfp4_channel_abs_sum(FAKE, 0, 0, 64, FAKE, 0, None) == 2
    assert L.rsfp4_channel_abs_sum(FAKE, 0, 4, 64, ctypes.c_void_p(0x100004), 0, None) == 3


def test_from_x_validation():
    """The one-call quantize + linear: host-side checks, which fail before
    anything touches a device."""
    L = rs.lib()
    f = L.rsfp4_nvfp4_linear_compensated_from_x
    act_need = rs.packed_act_bytes(0, 2, 512, True)
    # null act, unknown output dtype, misaligned act, small act, small weights
    assert f(FAKE, 1, 2, 16, 512, FAKE, 1 << 30, FAKE, 0, None, 0, None, 0, None) == 1
    assert f(FAKE, 1, 2, 16, 512, FAKE, 1 << 30, FAKE, 7, FAKE, 1 << 30, None, 0, None) == 4
    assert f(FAKE, 1, 2, 16, 512, FAKE, 1 << 30, FAKE, 0, ctypes.c_void_p(0x100008), 1 << 30, None, 0, None) == 3
    assert f(FAKE, 1, 2, 16, 512, FAKE, 1 << 30, FAKE, 0, FAKE, act_need - 1, None, 0, None) == 5
    assert "act holds" in _err()
    assert f(FAKE, 1, 2, 16, 512, FAKE, 100, FAKE, 0, FAKE, 1 << 30, None, 0, None) == 5
    # shapes: K past the quantizer, M outside [1, 65535], bad K
    assert L.rsfp4_mxfp4_linear_from_x(FAKE, 1, 2, 16, 32800, FAKE, 1 << 30, FAKE, 0, FAKE, 1 << 30, None, 0, None) == 2
    assert L.rsfp4_mxfp4_linear_from_x(FAKE, 1, 0, 16, 512, FAKE, 1 << 30, FAKE, 0, FAKE, 1 << 30, None, 0, None) == 2
    assert L.rsfp4_mxfp4_linear_from_x(FAKE, 1, 2, 16, 100, FAKE, 1 << 30, FAKE, 0, FAKE, 1 << 30, None, 0, None) == 2


def test_validate_packed_host_checks():
    """rsfp4_validate_packed: the checks made before the header is read."""
    L = rs.lib()
    assert L.rsfp4_validate_packed(None, 1 << 20, None, None, None, None) == 1
    assert L.rsfp4_validate_packed(ctypes.c_void_p(0x100010), 1 << 20, None, None, None, None) == 3
    assert L.rsfp4_validate_packed(FAKE, 255, None, None, None, None) == 5
    assert "header" in _err()


def test_grouped_validation():
    """The grouped linear's host-side checks."""
    L = rs.lib()
    f = L.rsfp4_nvfp4_grouped_linear_compensated
    big = 1 << 30
    assert f(None, big, 8, FAKE, big, 4, FAKE, 2, 64, 512, FAKE, None) == 1
    assert f(FAKE, big, 0, FAKE, big, 4, FAKE, 2, 64, 512, FAKE, None) == 2       # M_total
    assert f(FAKE, big, 8, FAKE, big, 0, FAKE, 2, 64, 512, FAKE, None) == 2       # E
    assert f(FAKE, big, 8, FAKE, big, 4, FAKE, 9, 64, 512, FAKE, None) == 2       # max_rows > M_total
    assert f(FAKE, big, 40, FAKE, big, 4, FAKE, 17, 64, 512, FAKE, None) == 6     # 34 operand rows
    assert f(FAKE, big, 8, FAKE, big, 4, FAKE, 2, 64, 20480, FAKE, None) == 6     # K past one launch
    assert f(FAKE, 100, 8, FAKE, big, 4, FAKE, 2, 64, 512, FAKE, None) == 5       # act too small
    need = rs.packed_weight_bytes(0, 64, 512)
    assert f(FAKE, big, 8, FAKE, 4 * need - 1, 4, FAKE, 2, 64, 512, FAKE, None) == 5
    assert "blobs need" in _err()


def test_stream_read_host_checks():
    """rsfp4_stream_read: null, alignment and size checks come before any
    device call."""
    L = rs.lib()
    sink = ctypes.c_void_p(0x100000)
    assert L.rsfp4_stream_read(None, 4096, sink, None) == 1
    assert L.rsfp4_stream_read(FAKE, 4096, None, None) == 1
    assert L.rsfp4_stream_read(ctypes.c_void_p(0x100008), 4096, sink, None) == 3       # src not 16-aligned
    assert L.rsfp4_stream_read(FAKE, 4096, ctypes.c_void_p(0x100002), None) == 3       # sink not 4-aligned
    assert L.rsfp4_stream_read(FAKE, 4088, sink, None) == 2                             # not whole 16 bytes
    assert "multiple of 16" in _err()


def test_noalloc_host_checks():
    """The no-allocation linear validates like the workspace call (null and
    shape errors before any device call)."""
    L = rs.lib()
    assert L.rsfp4_nvfp4_linear_compensated_noalloc(None, 0, None, 0, 1, 16, 128, None, None) == 1

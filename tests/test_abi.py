"""C ABI checks that need no GPU: the library loads, exports every entry point
include/qmoe.h declares, sizes its tensors as the oracle's layout does, and
rejects bad arguments on the host before launching anything."""
import ctypes
import os
import re

import pytest

from oracle import formats as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(",
                           text, flags=re.M))
    for fmt in fm.FORMATS:
        names |= {f"qquantize_{fmt}", f"qdequant_{fmt}", f"qgemv_{fmt}"}
    names.discard("QMOE_DECLARE_FORMAT")
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    from decode_moe_mul_amd import qmoe
    return qmoe.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 30
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_strings(L):
    assert L.qmoe_abi_version() == 1
    assert L.qmoe_status_string(0) == b"ok"
    assert L.qmoe_status_string(-3) == b"workspace too small"


@pytest.mark.parametrize("fmt", fm.FORMATS)
@pytest.mark.parametrize("N,K", [(1, 256), (640, 2048), (2048, 640), (14336, 4096), (7, 512)])
def test_tensor_bytes_matches_oracle_layout(L, fmt, N, K):
    from decode_moe_mul_amd import qmoe
    if K % fm.BLOCK[fmt]:
        assert L.qmoe_tensor_bytes(qmoe.FORMATS[fmt], N, K) == 0
        return
    assert L.qmoe_tensor_bytes(qmoe.FORMATS[fmt], N, K) == fm.tensor_bytes(fmt, N, K)
    assert qmoe.plane_offsets(fmt, N, K) == fm.plane_offsets(fmt, N, K)[0]


def test_block_sizes(L):
    assert [L.qmoe_block_size(i) for i in range(5)] == [32, 32, 32, 256, 256]
    assert L.qmoe_block_size(7) == 0


def test_host_validation_rejects_before_launch(L):
    from decode_moe_mul_amd import qmoe
    fake = ctypes.c_void_p(256 * 1000)  # never dereferenced: every call below fails validation
    # K not a multiple of the block
    assert L.qgemv_q4_k(fake, 4, 100, fake, 0, 1, fake, None) == -1
    # unknown activation dtype
    assert L.qgemv_q8_0(fake, 4, 64, fake, 7, 1, fake, None) == -2
    # null pointers
    assert L.qgemv_q8_0(None, 4, 64, fake, 0, 1, fake, None) == -1
    # misaligned weights
    assert L.qgemv_q8_0(ctypes.c_void_p(256 * 1000 + 4), 4, 64, fake, 0, 1, fake, None) == -1
    # router: k > E, k > 64, E too large
    assert L.moe_route(fake, 0, 4, 64, fake, None, 8, 9, 0, fake, fake, None, fake, 1 << 20, None) == -1
    assert L.moe_route(fake, 0, 4, 64, fake, None, 8192, 4, 0, fake, fake, None, fake, 1 << 30, None) == -2
    # router: workspace too small
    need = L.moe_route_workspace_size(4, 64, 16)
    assert need > 0
    assert L.moe_route(fake, 0, 4, 64, fake, None, 16, 2, 0, fake, fake, None, fake, need - 1, None) == -3
    # fused decode routing: too many rows, workspace too small
    need = L.moe_route_decode_workspace_size(4, 64, 16)
    assert need >= L.moe_route_workspace_size(4, 64, 16)
    assert L.moe_route_decode(fake, 0, 17, 64, fake, None, 16, 2, 0, fake, fake, None, fake,
                              fake, fake, fake, 1 << 30, None) == -2
    assert L.moe_route_decode(fake, 0, 4, 64, fake, None, 16, 2, 0, fake, fake, None, fake,
                              fake, fake, fake, need - 1, None) == -3
    assert L.moe_route_decode(fake, 0, 16, 64, fake, None, 512, 64, 8000, fake, fake, None,
                              fake, fake, fake, fake, 1 << 30, None) == -2
    assert L.moe_route_decode(fake, 0, 1, 64, fake, None, 513, 8, 0, fake, fake, None,
                              fake, fake, fake, fake, 1 << 30, None) == -2
    # batched GEMV: too many matrices, unknown format, bad K
    from decode_moe_mul_amd import qmoe as qm
    descs = (qm.GemvDesc * 17)()
    assert L.qgemv_batch(descs, 17, None) == -1
    assert L.qgemv_batch(None, 0, None) == 0
    descs[0] = qm.GemvDesc(9, 8, 64, 0, 1, 0, 256 * 1000, 256 * 1000, 256 * 1000)
    assert L.qgemv_batch(descs, 1, None) == -2
    descs[0] = qm.GemvDesc(0, 8, 100, 0, 1, 0, 256 * 1000, 256 * 1000, 256 * 1000)
    assert L.qgemv_batch(descs, 1, None) == -1
    assert b"matrix 0" in L.qmoe_last_error()
    # permute: E too large
    assert L.moe_permute(fake, 4, 2, 9000, fake, fake, fake, None) == -2
    # combine: H not a multiple of 4
    assert L.moe_combine(fake, fake, fake, 4, 2, 6, None, fake, None) == -1
    # tiers that do not cover [0, E)
    tier = qmoe.Tier(0, 4, 0, 0, 256 * 1000, 256 * 1000, 256 * 1000)
    arr = (qmoe.Tier * 1)(tier)
    ws_need = L.moe_ffn_workspace_size(2, 2, 64)
    assert L.moe_ffn_tiered(arr, 1, 8, 64, 64, fake, 0, 2, 2, fake, fake, fake, fake,
                            ws_need, None) == -1
    assert b"cover" in L.qmoe_last_error()
    # overlapping tiers
    arr2 = (qmoe.Tier * 2)(qmoe.Tier(0, 4, 0, 0, 256000, 256000, 256000),
                           qmoe.Tier(3, 8, 0, 0, 256000, 256000, 256000))
    assert L.moe_ffn_tiered(arr2, 2, 8, 64, 64, fake, 0, 2, 2, fake, fake, fake, fake,
                            ws_need, None) == -1
    # unknown format in a tier
    arr3 = (qmoe.Tier * 1)(qmoe.Tier(0, 8, 9, 0, 256000, 256000, 256000))
    assert L.moe_ffn_tiered(arr3, 1, 8, 64, 64, fake, 0, 2, 2, fake, fake, fake, fake,
                            ws_need, None) == -2
    # workspace too small
    arr4 = (qmoe.Tier * 1)(qmoe.Tier(0, 8, 0, 0, 256000, 256000, 256000))
    assert L.moe_ffn_tiered(arr4, 1, 8, 64, 64, fake, 0, 2, 2, fake, fake, fake, fake,
                            ws_need - 1, None) == -3
    assert L.qgemm_grouped_prefill(arr4, 1, 8, 64, 64, fake, 0, 2, 2, fake, fake, fake, fake,
                                   16, None) == -3


def test_zero_rows_are_noops(L):
    fake = ctypes.c_void_p(256 * 1000)
    assert L.qgemv_q8_0(fake, 0, 64, fake, 0, 1, fake, None) == 0
    assert L.qgemv_q8_0(fake, 4, 64, fake, 0, 0, fake, None) == 0
    assert L.moe_route(fake, 0, 0, 64, fake, None, 16, 2, 0, fake, fake, None, None, 0, None) == 0
    assert L.moe_combine(None, None, None, 0, 2, 64, None, fake, None) == 0
    arr = (ctypes.c_byte * 1)()
    from decode_moe_mul_amd import qmoe
    t = (qmoe.Tier * 1)(qmoe.Tier(0, 8, 0, 0, 256000, 256000, 256000))
    assert L.moe_ffn_tiered(t, 1, 8, 64, 64, fake, 0, 0, 2, fake, fake, fake, None, 0, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from decode_moe_mul_amd import qmoe
    monkeypatch.setattr(qmoe, "_lib", None)
    monkeypatch.setattr(qmoe, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(qmoe.QmoeError):
        qmoe.lib()


def test_t5_ternary_entry_points_and_limits(L):
    """The ternary format's layout queries and host-side checks (no launch)."""
    from decode_moe_mul_amd import qmoe
    T5 = qmoe.FORMATS["t5"]
    fake = ctypes.c_void_p(256 * 1000)
    assert L.qmoe_block_size(T5) == 128
    for N, K in [(1, 128), (3, 384), (4096, 4096), (640, 2048)]:
        assert L.qmoe_tensor_bytes(T5, N, K) == fm.tensor_bytes("t5", N, K)
    assert L.qmoe_tensor_bytes(T5, 4, 100) == 0
    assert L.qgemv_t5(fake, 4, 100, fake, 0, 1, fake, None) == -1     # K % 128
    assert L.qgemv_t5(fake, 4, 256, fake, 0, 17, fake, None) == -1    # R > 16
    assert L.qgemv_t5(fake, 4, 20224, fake, 0, 1, fake, None) == -2   # staged row > LDS
    assert L.qgemv_t5(fake, 0, 256, fake, 0, 1, fake, None) == 0      # no rows: no-op
    # T5 is not a tier format
    tier = qmoe.Tier(0, 8, T5, 0, 256000, 256000, 256000)
    arr = (qmoe.Tier * 1)(tier)
    ws_need = L.moe_ffn_workspace_size(2, 2, 256)
    assert L.moe_ffn_tiered(arr, 1, 8, 256, 256, fake, 0, 2, 2, fake, fake, fake, fake,
                            ws_need, None) == -2
    # qgemv_batch takes batches of T5 matrices (checked as qgemv_t5 checks)
    # but not T5 mixed with other formats
    descs = (qmoe.GemvDesc * 2)(qmoe.GemvDesc(T5, 8, 256, 0, 1, 0, 256000, 256000, 256000),
                                qmoe.GemvDesc(T5, 8, 100, 0, 1, 0, 256000, 256000, 256000))
    assert L.qgemv_batch(descs, 2, None) == -1
    assert b"matrix 1" in L.qmoe_last_error()
    descs[1] = qmoe.GemvDesc(3, 8, 256, 0, 1, 0, 256000, 256000, 256000)
    assert L.qgemv_batch(descs, 2, None) == -2


def test_one_launch_layer_validation(L):
    from decode_moe_mul_amd import qmoe
    fake = ctypes.c_void_p(256 * 1000)  # never dereferenced: every call below fails validation
    arr = (qmoe.Tier * 1)(qmoe.Tier(0, 16, 0, 0, 256000, 256000, 256000))
    need = L.moe_layer_decode_workspace_size(4, 64, 16, 64, 2, 0)
    # counter block + split-K partials + h [A, F] + o [A, H], each 256-aligned
    assert need == 16384 + 256 + 2048 + 2048 + 512   # + schedule table (64 entries)
    args = lambda T, E, k, ns, ws: (arr, 1, E, 64, 64, fake, 0, T, fake, None, k, ns, fake, fake,
                                    fake, fake, fake, fake, fake, ws, None)
    assert L.moe_layer_decode(*args(17, 16, 2, 0, 1 << 30)) == -2      # rows beyond 16
    assert L.moe_layer_decode(*args(4, 16, 0, 0, 1 << 30)) == -1       # k = 0
    assert L.moe_layer_decode(*args(4, 16, 17, 0, 1 << 30)) == -1      # k > E
    assert L.moe_layer_decode(*args(4, 600, 8, 0, 1 << 30)) == -2      # E > 512
    assert L.moe_layer_decode(*args(4, 16, 2, 0, need - 1)) == -3      # workspace
    # tiers must cover the shared experts too
    assert L.moe_layer_decode(*args(4, 16, 2, 1, 1 << 30)) == -1
    assert b"cover" in L.qmoe_last_error()
    assert L.moe_layer_decode_workspace_size(-1, 64, 16, 64, 2, 0) == 0


def test_mx_gemm_validation(L):
    fake = ctypes.c_void_p(256 * 1000)  # never dereferenced: every call below fails validation
    assert L.qquantize_act_mxfp8(fake, 0, 4, 48, fake, fake, None) == -1     # K % 32
    assert L.qquantize_act_mxfp8(fake, 5, 4, 64, fake, fake, None) == -2     # dtype
    assert L.qquantize_act_mxfp8(None, 0, 4, 64, fake, fake, None) == -1     # null
    assert L.qquantize_act_mxfp8(fake, 0, 0, 64, fake, fake, None) == 0      # no rows
    assert L.qgemm_mxfp4_mxfp8(fake, 16, 96, fake, fake, 4, fake, None) == -1  # K % 128
    assert L.qgemm_mxfp4_mxfp8(ctypes.c_void_p(256 * 1000 + 16), 16, 128, fake, fake, 4, fake,
                               None) == -1                                    # W alignment
    assert L.qgemm_mxfp4_mxfp8(fake, 0, 128, fake, fake, 4, fake, None) == 0


def test_int8_gemv_validation(L):
    fake = ctypes.c_void_p(256 * 1000)  # never dereferenced: every call below fails validation
    assert L.qquantize_act_q8(fake, 0, 4, 48, fake, fake, None) == -1      # K % 32
    assert L.qquantize_act_q8(fake, 3, 4, 64, fake, fake, None) == -2      # dtype
    assert L.qgemv_q8_0_i8(fake, 16, 64, fake, fake, 17, fake, None) == -1  # R > 16
    assert L.qgemv_q8_0_i8(fake, 16, 48, fake, fake, 2, fake, None) == -1   # K % 32
    assert L.qgemv_q8_0_i8(fake, 0, 64, fake, fake, 2, fake, None) == 0


def test_newer_entry_points_validate_on_the_host(L):
    """Argument errors of the int8 GEMM, the streaming read, the one-launch
    layer and the allocation-free routing are caught before any launch."""
    from decode_moe_mul_amd import qmoe
    fake = ctypes.c_void_p(256 * 1000)
    # qgemm_q8_0_i8: K not a multiple of 32, negative sizes, null pointers
    assert L.qgemm_q8_0_i8(fake, 64, 48, fake, fake, 16, fake, None) == -1
    assert L.qgemm_q8_0_i8(fake, -1, 64, fake, fake, 16, fake, None) == -1
    assert L.qgemm_q8_0_i8(fake, 0, 64, fake, fake, 16, fake, None) == 0      # no rows: no-op
    assert L.qgemm_q8_0_i8(None, 64, 64, fake, fake, 16, fake, None) == -1
    assert L.qgemm_q8_0_i8(ctypes.c_void_p(256 * 1000 + 16), 64, 64, fake, fake, 16, fake,
                           None) == -1                                          # W misaligned
    # qmoe_wave_latency: its output pointer
    assert L.qmoe_wave_latency(None, None) == -1
    # qmoe_stream_read: sizes, alignment, blocks per CU
    assert L.qmoe_stream_read(fake, 0, 8, fake, None) == 0
    assert L.qmoe_stream_read(fake, 24, 8, fake, None) == -1
    assert L.qmoe_stream_read(ctypes.c_void_p(256 * 1000 + 4), 64, 8, fake, None) == -1
    assert L.qmoe_stream_read(fake, 64, 0, fake, None) == -1
    assert L.qmoe_stream_read(fake, 64, 65, fake, None) == -1
    assert L.qmoe_stream_read(fake, 64, 8, None, None) == -1
    # moe_layer_decode: more than 16 rows, more than 512 experts
    t = (qmoe.Tier * 1)(qmoe.Tier(0, 8, 0, 0, 256000, 256000, 256000))
    args = (fake, fake, fake, fake, fake, fake, fake, 1 << 20, None)
    assert L.moe_layer_decode(t, 1, 8, 64, 64, fake, 0, 17, fake, None, 2, 0, *args) == -2
    assert L.moe_layer_decode(t, 1, 600, 64, 64, fake, 0, 4, fake, None, 2, 0, *args) == -2
    # moe_route_decode_noalloc: more rows than the fused routing takes
    assert L.moe_route_decode_noalloc(fake, 0, 17, 64, fake, None, 16, 2, 0, fake, fake, None,
                                      fake, fake, fake, None) == -2

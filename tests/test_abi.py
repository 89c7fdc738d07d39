"""The C ABI: every symbol the header declares is exported, and arguments,
shapes and the device are validated before anything is launched."""

import ctypes
import os
import re

import pytest

import bit_quantized_diffusion_amd as bq

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "svdq.h")


def _gpu_present():
    import torch
    return torch.cuda.is_available()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SVDQ_API\s+[\w\s\*]+?\b(svdq_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_symbols()
    for must in ("svdq_pack_weights", "svdq_quantize_act_lora_down", "svdq_gemm_w4a4_lora_up"):
        assert must in names
    assert set(names) == set(bq.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bq.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_internal_launchers_are_hidden():
    lib = ctypes.CDLL(bq.LIB_PATH)
    assert not hasattr(lib, "svdq_launch_gemm_w4a4_lora_up")


def test_status_strings():
    for st in (0, -1, -2, -3, -4):
        assert bq.status_string(st).startswith("svdq:")
    assert "unknown" in bq.status_string(123)
    assert bq.version() >= 100


def test_sizes():
    s = bq.packed_sizes(3072, 12288, 32)
    assert s == (3072 * 4, 32 * 3072 * 2, 12288 * 32 * 2, 12288 * 1536, 48 * 12288 * 2)
    s = bq.packed_sizes(3072, 12288, 32, bq.MXFP4)
    assert s[4] == 96 * 12288
    a = bq.act_sizes(4608, 3072, 32)
    assert a == (4608 * 1536, 48 * 4608 * 2, 4608 * 32 * 4)


@pytest.mark.parametrize("K,N,rank,prec,want", [
    (100, 64, 16, bq.INT4, bq.SVDQ_ERR_SHAPE),      # K % 64
    (0, 64, 0, bq.INT4, bq.SVDQ_ERR_SHAPE),
    (128, 0, 0, bq.INT4, bq.SVDQ_ERR_SHAPE),
    (128, 64, 8, bq.INT4, bq.SVDQ_ERR_SHAPE),       # rank % 16
    (128, 64, 80, bq.INT4, bq.SVDQ_ERR_SHAPE),      # rank > min(K, N)
    (4096, 4096, 272, bq.INT4, bq.SVDQ_ERR_SHAPE),  # rank > 256
    (192, 64, 16, bq.MXFP4, bq.SVDQ_ERR_SHAPE),     # MXFP4 needs K % 128
    (128, 64, 16, 7, bq.SVDQ_ERR_INVALID_ARG),
])
def test_shape_rules(K, N, rank, prec, want):
    out = (ctypes.c_size_t * 5)()
    assert bq.lib.svdq_packed_sizes(K, N, rank, prec, out) == want


FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced (validation fails first)
MIS = ctypes.c_void_p(0x10004)       # misaligned


def test_hot_calls_reject_null_and_misaligned():
    L = bq.lib
    assert L.svdq_quantize_act_lora_down(None, 16, 64, FAKE, FAKE, 16, 0, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_INVALID_ARG
    assert L.svdq_quantize_act_lora_down(MIS, 16, 64, FAKE, FAKE, 16, 0, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_INVALID_ARG
    assert L.svdq_quantize_act_lora_down(FAKE, 16, 64, FAKE, None, 16, 0, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_INVALID_ARG
    assert L.svdq_gemm_w4a4_lora_up(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, MIS, FAKE, 16, 16, 64, 16, 0, None) == bq.SVDQ_ERR_INVALID_ARG
    assert L.svdq_gemm_w4a4_lora_up(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 16, 16, 64, 16, 0, None) == bq.SVDQ_ERR_INVALID_ARG
    assert L.svdq_debug_group_partials(FAKE, None, 16, 16, 64, 0, 0, 1, 1, FAKE, None) == bq.SVDQ_ERR_INVALID_ARG
    uf = L.svdq_unfused_linear
    assert uf(None, 16, 64, FAKE, FAKE, 16, FAKE, FAKE, FAKE, None, 16, 0, FAKE, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_INVALID_ARG
    assert uf(FAKE, 16, 64, FAKE, FAKE, 16, FAKE, FAKE, None, None, 16, 0, FAKE, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_INVALID_ARG
    assert uf(FAKE, 16, 64, FAKE, FAKE, 16, FAKE, FAKE, FAKE, MIS, 16, 0, FAKE, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_INVALID_ARG


def test_hot_calls_reject_bad_shapes():
    L = bq.lib
    assert L.svdq_quantize_act_lora_down(FAKE, 0, 64, FAKE, FAKE, 16, 0, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_SHAPE
    assert L.svdq_quantize_act_lora_down(FAKE, 16, 96, FAKE, FAKE, 16, 0, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_SHAPE
    assert L.svdq_quantize_act_lora_down(FAKE, 16, 64, FAKE, FAKE, 24, 0, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_SHAPE
    assert L.svdq_gemm_w4a4_lora_up(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, 0, 64, 16, 0, None) == bq.SVDQ_ERR_SHAPE
    assert L.svdq_gemm_w4a4_lora_up(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, 8, 64, 16, 0, None) == bq.SVDQ_ERR_SHAPE
    uf = L.svdq_unfused_linear
    assert uf(FAKE, 16, 64, FAKE, FAKE, 16, FAKE, FAKE, FAKE, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_SHAPE
    assert uf(FAKE, 16, 100, FAKE, FAKE, 16, FAKE, FAKE, FAKE, None, 16, 0, FAKE, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_SHAPE
    assert uf(FAKE, 16, 64, FAKE, FAKE, 24, FAKE, FAKE, FAKE, None, 16, 0, FAKE, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_SHAPE
    # window outside the matrix
    assert L.svdq_debug_group_partials(FAKE, FAKE, 16, 16, 64, 10, 0, 7, 1, FAKE, None) == bq.SVDQ_ERR_SHAPE


def test_oversize_operands_are_refused():
    """The GEMMs address a 4-bit operand and its scales with 32-bit byte
    offsets, so an operand of 2^31 code bytes or more is refused with
    SVDQ_ERR_SHAPE before anything is launched (never a wrong Y): M = N =
    349,526 at K = 12288 is the first such size; one token fewer passes the
    shape rules (and then stops at the device check here)."""
    L = bq.lib
    K = 12288
    big, ok = 349526, 349525
    assert big * (K // 2) >= 2 ** 31 > ok * (K // 2)
    for prec in (bq.INT4, bq.MXFP4):
        g = L.svdq_gemm_w4a4_lora_up
        assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, big, 64, K, 16, prec, None) == bq.SVDQ_ERR_SHAPE
        assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, big, K, 16, prec, None) == bq.SVDQ_ERR_SHAPE
        assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ok, 64, K, 16, prec, None) != bq.SVDQ_ERR_SHAPE
    assert L.svdq_gemm_w4a4_lora_up_gelu(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, big, 64, K, 16, 0, None) \
        == bq.SVDQ_ERR_SHAPE
    assert L.svdq_unfused_linear(FAKE, big, K, FAKE, FAKE, 16, FAKE, FAKE, FAKE, None, 64, 0, FAKE, FAKE, FAKE, FAKE,
                                 None) == bq.SVDQ_ERR_SHAPE
    assert L.svdq_gemm_w4a16(FAKE, FAKE, FAKE, None, FAKE, 64, big, K, None) == bq.SVDQ_ERR_SHAPE
    assert L.svdq_debug_group_partials(FAKE, FAKE, big, 16, K, 0, 0, 1, 1, FAKE, None) == bq.SVDQ_ERR_SHAPE
    f = L.svdq_mlp_gemm_gelu_quant
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, big, 256, K, 16, FAKE, FAKE, 16, 0, FAKE, FAKE, FAKE,
             None) == bq.SVDQ_ERR_SHAPE


def test_noalloc_validates_and_refuses_beyond_its_array():
    """The no-allocation unfused call: NULL / misaligned pointers, MXFP4,
    and a layer whose intermediates exceed the library's 32 MiB device array
    (M = 4608, K = 16384: 36 MiB of codes) -> SVDQ_ERR_SHAPE, before any
    device work."""
    f = bq.lib.svdq_unfused_linear_noalloc
    assert bq.NOALLOC_SCRATCH_BYTES == 32 << 20
    assert f(None, 16, 64, FAKE, FAKE, 16, FAKE, FAKE, FAKE, None, 16, 0, FAKE, None) == bq.SVDQ_ERR_INVALID_ARG
    assert f(FAKE, 16, 64, FAKE, FAKE, 16, FAKE, FAKE, FAKE, MIS, 16, 0, FAKE, None) == bq.SVDQ_ERR_INVALID_ARG
    assert f(FAKE, 16, 128, FAKE, FAKE, 16, FAKE, FAKE, FAKE, None, 16, bq.MXFP4, FAKE, None) == bq.SVDQ_ERR_INVALID_ARG
    assert f(FAKE, 4608, 16384, FAKE, FAKE, 32, FAKE, FAKE, FAKE, None, 64, 0, FAKE, None) == bq.SVDQ_ERR_SHAPE
    # FLUX fc2 (4608 x 12288, rank 32) fits: it stops at the device check here, not at the size
    assert f(FAKE, 4608, 12288, FAKE, FAKE, 32, FAKE, FAKE, FAKE, None, 64, 0, FAKE, None) != bq.SVDQ_ERR_SHAPE


def test_mlp_calls_validate():
    """The GELU and fused-MLP calls: NULL / misaligned pointers, MXFP4
    (INT4 only), N not a multiple of 128 for the fused pair, rank rules."""
    L = bq.lib
    g = L.svdq_gemm_w4a4_lora_up_gelu
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 16, 16, 64, 16, 0, None) == bq.SVDQ_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, MIS, FAKE, 16, 16, 64, 16, 0, None) == bq.SVDQ_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, 16, 128, 16, bq.MXFP4, None) == bq.SVDQ_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, 16, 96, 16, 0, None) == bq.SVDQ_ERR_SHAPE
    f = L.svdq_mlp_gemm_gelu_quant
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 16, 256, 64, 16, FAKE, FAKE, 16, 0, FAKE, FAKE, FAKE, None)
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a11=None) == bq.SVDQ_ERR_INVALID_ARG          # smooth_inv2
    assert call(a12=None) == bq.SVDQ_ERR_INVALID_ARG          # lora_down2 with rank2 > 0
    assert call(a15=MIS) == bq.SVDQ_ERR_INVALID_ARG           # xq2
    assert call(a14=bq.MXFP4) == bq.SVDQ_ERR_INVALID_ARG
    assert call(a8=192) == bq.SVDQ_ERR_SHAPE                  # N % 128 != 0
    assert call(a13=24) == bq.SVDQ_ERR_SHAPE                  # rank2 not a multiple of 16
    assert call(a12=None, a13=0, a17=None) != bq.SVDQ_ERR_INVALID_ARG   # rank2 == 0 needs no L1 / lora_act2


def test_w4a16_calls_validate():
    """The W4A16 comparison GEMM and its pack: NULL / misaligned pointers,
    K not a multiple of 64, empty shapes."""
    g = bq.lib.svdq_gemm_w4a16
    assert g(None, FAKE, FAKE, None, FAKE, 16, 16, 64, None) == bq.SVDQ_ERR_INVALID_ARG
    assert g(FAKE, FAKE, None, None, FAKE, 16, 16, 64, None) == bq.SVDQ_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, MIS, FAKE, 16, 16, 64, None) == bq.SVDQ_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, None, FAKE, 16, 16, 96, None) == bq.SVDQ_ERR_SHAPE
    assert g(FAKE, FAKE, FAKE, None, FAKE, 0, 16, 64, None) == bq.SVDQ_ERR_SHAPE
    assert g(FAKE, FAKE, FAKE, None, FAKE, 16, 0, 64, None) == bq.SVDQ_ERR_SHAPE
    p = bq.lib.svdq_pack_w4a16
    assert p(None, 64, 4, FAKE, FAKE) == bq.SVDQ_ERR_INVALID_ARG
    assert p(FAKE, 100, 4, FAKE, FAKE) == bq.SVDQ_ERR_SHAPE


def test_workspace_gemm_validates():
    """svdq_gemm_w4a4_lora_up_ws applies the rules of svdq_gemm_w4a4_lora_up
    and refuses a misaligned workspace; svdq_gemm_workspace_size checks its
    shape and output pointer."""
    L = bq.lib
    g = L.svdq_gemm_w4a4_lora_up_ws
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, 16, 64, 16, 0, MIS, 1 << 20, None) == bq.SVDQ_ERR_INVALID_ARG
    assert g(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, 16, 64, 16, 0, FAKE, 1 << 20, None) == bq.SVDQ_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 16, 16, 64, 16, 0, FAKE, 1 << 20, None) == bq.SVDQ_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, 8, 64, 16, 0, FAKE, 1 << 20, None) == bq.SVDQ_ERR_SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, 16, 96, 16, 0, None, 0, None) == bq.SVDQ_ERR_SHAPE
    out = ctypes.c_size_t(7)
    assert L.svdq_gemm_workspace_size(16, 16, 64, 0, None) == bq.SVDQ_ERR_INVALID_ARG
    assert L.svdq_gemm_workspace_size(0, 16, 64, 0, ctypes.byref(out)) == bq.SVDQ_ERR_SHAPE
    assert L.svdq_gemm_workspace_size(16, 16, 96, 0, ctypes.byref(out)) == bq.SVDQ_ERR_SHAPE
    assert L.svdq_gemm_workspace_size(16, 16, 64, 2, ctypes.byref(out)) == bq.SVDQ_ERR_INVALID_ARG
    assert out.value == 0


@pytest.mark.skipif(_gpu_present(), reason="checks the no-device path")
def test_no_device_gives_unsupported_device_not_a_crash():
    L = bq.lib
    assert L.svdq_device_check(0) == bq.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert not bq.device_check(0)
    # fully valid arguments: the device check is what refuses
    assert L.svdq_quantize_act_lora_down(FAKE, 16, 64, FAKE, FAKE, 16, 0, FAKE, FAKE, FAKE, None) == bq.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert L.svdq_gemm_w4a4_lora_up(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, 16, 64, 16, 0, None) == bq.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert L.svdq_debug_group_partials(FAKE, FAKE, 16, 16, 64, 0, 0, 1, 1, FAKE, None) == bq.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert L.svdq_gemm_w4a4_lora_up_ws(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, 16, 64, 16, 0, FAKE, 1 << 20,
                                       None) == bq.SVDQ_ERR_UNSUPPORTED_DEVICE
    out = ctypes.c_size_t(0)
    assert L.svdq_gemm_workspace_size(576, 3072, 12288, 0, ctypes.byref(out)) == bq.SVDQ_ERR_UNSUPPORTED_DEVICE
    with pytest.raises(bq.SvdqError) as ei:
        bq.check(bq.SVDQ_ERR_UNSUPPORTED_DEVICE)
    assert ei.value.status == bq.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert L.svdq_device_check(-1) == bq.SVDQ_ERR_UNSUPPORTED_DEVICE


def test_pack_validates_on_host():
    import numpy as np
    w = np.zeros((64, 100), np.uint16)
    with pytest.raises(bq.SvdqError):
        bq.pack_weights(w, np.ones(100, np.float32), 16)
    with pytest.raises(ValueError):
        bq.pack_weights(np.zeros((64, 128), np.uint16), np.ones(64, np.float32), 16)


def test_mfma_ceiling_validates():
    """The measurement hook: NULL / misaligned output, unknown precision,
    empty launch."""
    f = bq.lib.svdq_bench_mfma_ceiling
    assert f(bq.INT4, 4, 4, None, None) == bq.SVDQ_ERR_INVALID_ARG
    assert f(bq.INT4, 4, 4, MIS, None) == bq.SVDQ_ERR_INVALID_ARG
    assert f(7, 4, 4, FAKE, None) == bq.SVDQ_ERR_INVALID_ARG
    assert f(bq.INT4, 0, 4, FAKE, None) == bq.SVDQ_ERR_SHAPE
    assert f(bq.MXFP4, 4, 0, FAKE, None) == bq.SVDQ_ERR_SHAPE

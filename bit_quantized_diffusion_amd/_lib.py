"""ctypes loader for the in-tree libsvdq.so.

Importing this module fails loudly when the library has not been built:
there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsvdq.so")

SVDQ_OK = 0
SVDQ_ERR_INVALID_ARG = -1
SVDQ_ERR_SHAPE = -2
SVDQ_ERR_UNSUPPORTED_DEVICE = -3
SVDQ_ERR_HIP = -4

INT4 = 0
MXFP4 = 1

EXPORTED = (
    "svdq_version", "svdq_status_string", "svdq_device_check",
    "svdq_packed_sizes", "svdq_act_sizes", "svdq_pack_weights",
    "svdq_quantize_act_lora_down", "svdq_gemm_w4a4_lora_up",
    "svdq_unfused_linear", "svdq_debug_group_partials", "svdq_merge_lora",
    "svdq_gemm_w4a4_lora_up_gelu", "svdq_mlp_gemm_gelu_quant",
    "svdq_pack_w4a16", "svdq_gemm_w4a16", "svdq_bench_mfma_ceiling",
    "svdq_unfused_linear_noalloc", "svdq_gemm_workspace_size", "svdq_gemm_w4a4_lora_up_ws",
)


class SvdqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python bit_quantized_diffusion_amd/build.py` (hipcc, gfx950)")
    # The tensors handed to the library come from torch, which ships its own
    # HIP runtime.  Load torch first so that libsvdq.so binds to that same
    # runtime (the dynamic loader reuses the already loaded libamdhip64);
    # loaded the other way round the process ends up with two HIP runtimes
    # and the library's device queries fail.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "svdq_version": ([], i),
        "svdq_status_string": ([i], ctypes.c_char_p),
        "svdq_device_check": ([i], i),
        "svdq_packed_sizes": ([i, i, i, i, sz], i),
        "svdq_act_sizes": ([i, i, i, i, sz], i),
        "svdq_pack_weights": ([vp, vp, i, i, i, i, vp, vp, vp, vp, vp, vp], i),
        "svdq_quantize_act_lora_down": ([vp, i, i, vp, vp, i, i, vp, vp, vp, vp], i),
        "svdq_gemm_w4a4_lora_up": ([vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp], i),
        "svdq_unfused_linear": ([vp, i, i, vp, vp, i, vp, vp, vp, vp, i, i, vp, vp, vp, vp, vp], i),
        "svdq_debug_group_partials": ([vp, vp, i, i, i, i, i, i, i, vp, vp], i),
        "svdq_merge_lora": ([vp, vp, i, vp, vp, vp, i, i, i, vp, vp], i),
        "svdq_gemm_w4a4_lora_up_gelu": ([vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp], i),
        "svdq_mlp_gemm_gelu_quant": ([vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, vp, i, i, vp, vp, vp, vp], i),
        "svdq_pack_w4a16": ([vp, i, i, vp, vp], i),
        "svdq_gemm_w4a16": ([vp, vp, vp, vp, vp, i, i, i, vp], i),
        "svdq_bench_mfma_ceiling": ([i, i, i, vp, vp], i),
        "svdq_unfused_linear_noalloc": ([vp, i, i, vp, vp, i, vp, vp, vp, vp, i, i, vp, vp], i),
        "svdq_gemm_workspace_size": ([i, i, i, i, sz], i),
        "svdq_gemm_w4a4_lora_up_ws": ([vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp, ctypes.c_size_t, vp], i),
    }
    for name, (args, ret) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ret
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.svdq_status_string(int(status)).decode()


def check(status: int) -> None:
    if status != SVDQ_OK:
        raise SvdqError(status, status_string(status))

"""SVDQuant W4A4 linear layer for AMD Instinct MI355X (gfx950).

A thin binding over the C ABI of ``libsvdq.so`` (``include/svdq.h``).  It only
marshals arguments: torch tensors supply device memory and the current HIP
stream, every step of the layer runs in the library's HIP kernels, and the
offline pack runs in the library's C++ code.  A missing library is an import
error; there is no fallback.

    Y = X^ L1 L2 + dequant(Q4(X^) Q4(R)^T) + b,   X^ = X diag(lambda)^-1

(model card "svdq-int4-flux.1-dev": "Overview of SVDQuant" caption, stages
2-3; Nunchaku engine caption (b): the two fused kernels.)
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import numpy as np

from ._lib import (INT4, MXFP4, SVDQ_ERR_HIP, SVDQ_ERR_INVALID_ARG,  # noqa: F401
                   SVDQ_ERR_SHAPE, SVDQ_ERR_UNSUPPORTED_DEVICE, SVDQ_OK,
                   EXPORTED, LIB_PATH, SvdqError, check, lib, status_string)

__all__ = [
    "INT4", "MXFP4", "SvdqError", "lib", "LIB_PATH", "status_string", "merge_lora",
    "version", "device_check", "packed_sizes", "act_sizes", "pack_weights",
    "quantize_act_lora_down", "gemm_w4a4_lora_up", "debug_group_partials", "unfused_linear",
    "unfused_linear_noalloc", "NOALLOC_SCRATCH_BYTES",
    "PackedLinear", "linear", "gemm_w4a4_lora_up_gelu", "mlp_gemm_gelu_quant", "mlp",
    "pack_w4a16", "gemm_w4a16", "mfma_ceiling",
]


def version() -> int:
    return lib.svdq_version()


def device_check(device: int = 0) -> bool:
    return lib.svdq_device_check(int(device)) == SVDQ_OK


def packed_sizes(K: int, N: int, rank: int, precision: int = INT4):
    out = (ctypes.c_size_t * 5)()
    check(lib.svdq_packed_sizes(K, N, rank, precision, out))
    return tuple(int(v) for v in out)


def act_sizes(M: int, K: int, rank: int, precision: int = INT4):
    out = (ctypes.c_size_t * 3)()
    check(lib.svdq_act_sizes(M, K, rank, precision, out))
    return tuple(int(v) for v in out)


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def pack_weights(w_bf16: np.ndarray, act_absmax: np.ndarray, rank: int,
                 precision: int = INT4, want_residual: bool = False) -> dict:
    """Offline pack on the CPU.  w_bf16: uint16 bf16 bits [N][K] (nn.Linear
    layout); act_absmax: float32 [K].  Returns host numpy arrays:
    smooth_inv [K] f32, lora_down [rank][K] u16, lora_up [N][rank] u16,
    wq [N][K/2] u8, ws [K/64][N] f16 (INT4) or [K/32][N] u8 (MXFP4), and the
    residual r [K][N] f32 when asked for."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    ax = np.ascontiguousarray(act_absmax, dtype=np.float32)
    if w.ndim != 2 or ax.ndim != 1 or ax.shape[0] != w.shape[1]:
        raise ValueError("w_bf16 must be [N][K] and act_absmax [K]")
    N, K = w.shape
    packed_sizes(K, N, rank, precision)          # validates the shape
    out = dict(
        smooth_inv=np.empty(K, np.float32),
        lora_down=np.empty((rank, K), np.uint16),
        lora_up=np.empty((N, rank), np.uint16),
        wq=np.empty((N, K // 2), np.uint8),
        ws=np.empty(_scale_shape(K, N, precision), np.float16 if precision == INT4 else np.uint8),
    )
    r = np.empty((K, N), np.float32) if want_residual else None
    check(lib.svdq_pack_weights(
        _np_ptr(w), _np_ptr(ax), K, N, rank, precision,
        _np_ptr(out["smooth_inv"]), _np_ptr(out["lora_down"]) if rank else None,
        _np_ptr(out["lora_up"]) if rank else None, _np_ptr(out["wq"]),
        _np_ptr(out["ws"]), _np_ptr(r)))
    if want_residual:
        out["r"] = r
    return out


def merge_lora(lora_down: Optional[np.ndarray], lora_up: Optional[np.ndarray], smooth_inv: np.ndarray,
               a_bf16: np.ndarray, b_bf16: np.ndarray):
    """Merge an off-the-shelf LoRA (Y += X A B) into the packed 16-bit branch
    on the CPU, leaving the 4-bit residual as it is.  lora_down [rank][K] and
    lora_up [N][rank] are bf16 bits from pack_weights (None for rank 0);
    a_bf16 [K][ra], b_bf16 [ra][N] bf16 bits.  Returns (lora_down'
    [rank+ra][K], lora_up' [N][rank+ra])."""
    sinv = np.ascontiguousarray(smooth_inv, dtype=np.float32)
    a = np.ascontiguousarray(a_bf16, dtype=np.uint16)
    b = np.ascontiguousarray(b_bf16, dtype=np.uint16)
    K, ra = a.shape
    N = b.shape[1]
    if b.shape[0] != ra or sinv.shape != (K,):
        raise ValueError("a must be [K][ra], b [ra][N] and smooth_inv [K]")
    rank = 0 if lora_down is None else int(np.asarray(lora_down).shape[0])
    ld = None if rank == 0 else np.ascontiguousarray(lora_down, dtype=np.uint16)
    lu = None if rank == 0 else np.ascontiguousarray(lora_up, dtype=np.uint16)
    if rank and (ld.shape != (rank, K) or lu.shape != (N, rank)):
        raise ValueError("lora_down must be [rank][K] and lora_up [N][rank]")
    down = np.empty((rank + ra, K), np.uint16)
    up = np.empty((N, rank + ra), np.uint16)
    check(lib.svdq_merge_lora(_np_ptr(ld), _np_ptr(lu), rank, _np_ptr(sinv), _np_ptr(a), _np_ptr(b), ra, K, N,
                              _np_ptr(down), _np_ptr(up)))
    return down, up


# ---------------------------------------------------------------------------
# device calls (torch tensors as device memory)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dptr(t, dtype, shape, name):
    """Device pointer of a contiguous CUDA tensor with the given dtype/shape."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _scale_dtype(precision):
    torch = _torch()
    return torch.float16 if precision == INT4 else torch.uint8


def _scale_shape(K, rows, precision):
    """Scales are group-major: [K/64][rows] (INT4), [K/32][rows] (MXFP4)."""
    return (K // 64, rows) if precision == INT4 else (K // 32, rows)


def quantize_act_lora_down(x, smooth_inv, lora_down, rank: int, precision: int = INT4,
                           xq=None, xs=None, lora_act=None):
    """First fused kernel.  x: bf16 [M][K]; smooth_inv: f32 [K];
    lora_down: bf16 [rank][K] or None when rank == 0.
    Returns (xq u8 [M][K/2], xs (INT4 [K/64][M] f16, MXFP4 [K/32][M] u8),
    lora_act f32 [M][rank] or None)."""
    torch = _torch()
    M, K = x.shape
    dev = x.device
    if xq is None:
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if xs is None:
        xs = torch.empty(_scale_shape(K, M, precision), dtype=_scale_dtype(precision), device=dev)
    if rank and lora_act is None:
        lora_act = torch.empty((M, rank), dtype=torch.float32, device=dev)
    check(lib.svdq_quantize_act_lora_down(
        _dptr(x, torch.bfloat16, (M, K), "x"), M, K,
        _dptr(smooth_inv, torch.float32, (K,), "smooth_inv"),
        _dptr(lora_down, torch.bfloat16, (rank, K), "lora_down") if rank else None,
        rank, precision,
        _dptr(xq, torch.uint8, (M, K // 2), "xq"),
        _dptr(xs, _scale_dtype(precision), _scale_shape(K, M, precision), "xs"),
        _dptr(lora_act, torch.float32, (M, rank), "lora_act") if rank else None,
        _stream(dev)))
    return xq, xs, (lora_act if rank else None)


def gemm_workspace_size(M: int, N: int, K: int, precision: int = INT4) -> int:
    """Bytes of workspace svdq_gemm_w4a4_lora_up_ws can use for this shape
    on the current device (0: the single-pass schedule runs anyway)."""
    out = ctypes.c_size_t(0)
    check(lib.svdq_gemm_workspace_size(M, N, K, precision, ctypes.byref(out)))
    return int(out.value)


_WS_BYTES = {}


def _workspace_bytes(dev, M, N, K, precision):
    """gemm_workspace_size, asked once per device and shape (the answer
    depends on nothing else), so that the per-call cost is a lookup."""
    key = (dev.index, M, N, K, precision)
    n = _WS_BYTES.get(key)
    if n is None:
        n = _WS_BYTES[key] = gemm_workspace_size(M, N, K, precision)
    return n


def gemm_w4a4_lora_up(xq, xs, wq, ws, lora_act, lora_up, bias, M: int, N: int, K: int,
                      rank: int, precision: int = INT4, y=None, workspace="auto"):
    """Second fused kernel.  Returns y bf16 [M][N].

    workspace: "auto" allocates (from torch's allocator, on the call's
    stream) the bytes gemm_workspace_size asks for, so that grids that would
    leave the device mostly idle run split along K; None calls the entry
    point without a workspace (single-pass schedule); a uint8 device tensor
    is used as given."""
    torch = _torch()
    dev = xq.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    sd = _scale_dtype(precision)
    args = (_dptr(xq, torch.uint8, (M, K // 2), "xq"), _dptr(xs, sd, _scale_shape(K, M, precision), "xs"),
            _dptr(wq, torch.uint8, (N, K // 2), "wq"), _dptr(ws, sd, _scale_shape(K, N, precision), "ws"),
            _dptr(lora_act, torch.float32, (M, rank), "lora_act") if rank else None,
            _dptr(lora_up, torch.bfloat16, (N, rank), "lora_up") if rank else None,
            _dptr(bias, torch.bfloat16, (N,), "bias"),
            _dptr(y, torch.bfloat16, (M, N), "y"),
            M, N, K, rank, precision)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a uint8 device tensor")
        nbytes = _workspace_bytes(dev, M, N, K, precision)
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=dev) if nbytes else None
    if workspace is None:
        check(lib.svdq_gemm_w4a4_lora_up(*args, _stream(dev)))
    else:
        n = workspace.numel()
        check(lib.svdq_gemm_w4a4_lora_up_ws(*args, _dptr(workspace, torch.uint8, (n,), "workspace"), n,
                                            _stream(dev)))
    return y


def gemm_w4a4_lora_up_gelu(xq, xs, wq, ws, lora_act, lora_up, bias, M: int, N: int, K: int, rank: int, y=None):
    """Second fused kernel with the MLP's GELU fused: y = bf16(GELU(bf16(Y)))
    (INT4).  Returns y bf16 [M][N]."""
    torch = _torch()
    dev = xq.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    check(lib.svdq_gemm_w4a4_lora_up_gelu(
        _dptr(xq, torch.uint8, (M, K // 2), "xq"), _dptr(xs, torch.float16, (K // 64, M), "xs"),
        _dptr(wq, torch.uint8, (N, K // 2), "wq"), _dptr(ws, torch.float16, (K // 64, N), "ws"),
        _dptr(lora_act, torch.float32, (M, rank), "lora_act") if rank else None,
        _dptr(lora_up, torch.bfloat16, (N, rank), "lora_up") if rank else None,
        _dptr(bias, torch.bfloat16, (N,), "bias"),
        _dptr(y, torch.bfloat16, (M, N), "y"),
        M, N, K, rank, INT4, _stream(dev)))
    return y


def mlp_gemm_gelu_quant(xq, xs, wq, ws, lora_act, lora_up, bias, M: int, N: int, K: int, rank: int,
                        smooth_inv2, lora_down2, rank2: int, xq2=None, xs2=None, lora_act2=None):
    """First layer's second kernel fused with GELU and the second layer's
    first kernel (INT4): returns (xq2 u8 [M][N/2], xs2 f16 [N/64][M],
    lora_act2 f32 [M][rank2] or None)."""
    torch = _torch()
    dev = xq.device
    if xq2 is None:
        xq2 = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
    if xs2 is None:
        xs2 = torch.empty((N // 64, M), dtype=torch.float16, device=dev)
    if rank2 and lora_act2 is None:
        lora_act2 = torch.empty((M, rank2), dtype=torch.float32, device=dev)
    check(lib.svdq_mlp_gemm_gelu_quant(
        _dptr(xq, torch.uint8, (M, K // 2), "xq"), _dptr(xs, torch.float16, (K // 64, M), "xs"),
        _dptr(wq, torch.uint8, (N, K // 2), "wq"), _dptr(ws, torch.float16, (K // 64, N), "ws"),
        _dptr(lora_act, torch.float32, (M, rank), "lora_act") if rank else None,
        _dptr(lora_up, torch.bfloat16, (N, rank), "lora_up") if rank else None,
        _dptr(bias, torch.bfloat16, (N,), "bias"), M, N, K, rank,
        _dptr(smooth_inv2, torch.float32, (N,), "smooth_inv2"),
        _dptr(lora_down2, torch.bfloat16, (rank2, N), "lora_down2") if rank2 else None, rank2, INT4,
        _dptr(xq2, torch.uint8, (M, N // 2), "xq2"), _dptr(xs2, torch.float16, (N // 64, M), "xs2"),
        _dptr(lora_act2, torch.float32, (M, rank2), "lora_act2") if rank2 else None, _stream(dev)))
    return xq2, xs2, (lora_act2 if rank2 else None)


def mfma_ceiling(precision: int = INT4, blocks: int = 512, iters: int = 4096, out=None):
    """Launch the matrix-core ceiling kernel once (measurement only); returns
    (ops per launch, the checksum tensor).  The caller times the launch."""
    torch = _torch()
    if out is None:
        out = torch.empty((blocks,), dtype=torch.float32, device="cuda")
    check(lib.svdq_bench_mfma_ceiling(precision, blocks, iters, _dptr(out, torch.float32, (blocks,), "out"),
                                      _stream(out.device)))
    return float(blocks) * 4 * 8 * iters * 131072, out


def pack_w4a16(w_bf16: np.ndarray):
    """W4A16 comparison weights on the CPU: w_bf16 uint16 bf16 bits [N][K] ->
    (wq uint8 [N][K/2], ws float16 [K/64][N])."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    N, K = w.shape
    wq = np.empty((N, K // 2), np.uint8)
    ws = np.empty((K // 64, N), np.float16)
    check(lib.svdq_pack_w4a16(_np_ptr(w), K, N, _np_ptr(wq), _np_ptr(ws)))
    return wq, ws


def gemm_w4a16(x, wq, ws, bias, N: int, y=None):
    """W4A16 comparison GEMM: y = bf16(x . dequant(W)^T + bias), x bf16 [M][K]."""
    torch = _torch()
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    check(lib.svdq_gemm_w4a16(
        _dptr(x, torch.bfloat16, (M, K), "x"), _dptr(wq, torch.uint8, (N, K // 2), "wq"),
        _dptr(ws, torch.float16, (K // 64, N), "ws"), _dptr(bias, torch.bfloat16, (N,), "bias"),
        _dptr(y, torch.bfloat16, (M, N), "y"), M, N, K, _stream(x.device)))
    return y


def unfused_linear(x, layer: "PackedLinear", y=None, xq=None, xs=None, lora_act=None):
    """The same layer as four separate kernels (quantize, down projection,
    4-bit GEMM, up projection): the baseline the two fusions are measured
    against.  INT4 only.  Returns y bf16 [M][N]."""
    torch = _torch()
    M, K = x.shape
    N, r, dev = layer.N, layer.rank, x.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if xq is None:
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if xs is None:
        xs = torch.empty((K // 64, M), dtype=torch.float16, device=dev)
    if r and lora_act is None:
        lora_act = torch.empty((M, r), dtype=torch.float32, device=dev)
    check(lib.svdq_unfused_linear(
        _dptr(x, torch.bfloat16, (M, K), "x"), M, K,
        _dptr(layer.smooth_inv, torch.float32, (K,), "smooth_inv"),
        _dptr(layer.lora_down, torch.bfloat16, (r, K), "lora_down") if r else None, r,
        _dptr(layer.wq, torch.uint8, (N, K // 2), "wq"), _dptr(layer.ws, torch.float16, (K // 64, N), "ws"),
        _dptr(layer.lora_up, torch.bfloat16, (N, r), "lora_up") if r else None,
        _dptr(layer.bias, torch.bfloat16, (N,), "bias"), N, layer.precision,
        _dptr(xq, torch.uint8, (M, K // 2), "xq"), _dptr(xs, torch.float16, (K // 64, M), "xs"),
        _dptr(lora_act, torch.float32, (M, r), "lora_act") if r else None,
        _dptr(y, torch.bfloat16, (M, N), "y"), _stream(dev)))
    return y


NOALLOC_SCRATCH_BYTES = 32 << 20


def unfused_linear_noalloc(x, layer: "PackedLinear", y):
    """unfused_linear with its intermediates in the library's own device
    array (svdq_unfused_linear_noalloc): the caller passes y and nothing is
    allocated.  Calls that overlap on one GPU race."""
    torch = _torch()
    M, K = x.shape
    N, r, dev = layer.N, layer.rank, x.device
    check(lib.svdq_unfused_linear_noalloc(
        _dptr(x, torch.bfloat16, (M, K), "x"), M, K,
        _dptr(layer.smooth_inv, torch.float32, (K,), "smooth_inv"),
        _dptr(layer.lora_down, torch.bfloat16, (r, K), "lora_down") if r else None, r,
        _dptr(layer.wq, torch.uint8, (N, K // 2), "wq"), _dptr(layer.ws, torch.float16, (K // 64, N), "ws"),
        _dptr(layer.lora_up, torch.bfloat16, (N, r), "lora_up") if r else None,
        _dptr(layer.bias, torch.bfloat16, (N,), "bias"), N, layer.precision,
        _dptr(y, torch.bfloat16, (M, N), "y"), _stream(dev)))
    return y


def debug_group_partials(xq, wq, M: int, N: int, K: int, m0: int, n0: int, mt: int, nt: int, out=None):
    """Exact INT4 per-group partials for a window: int32 [mt][nt][K/64]."""
    torch = _torch()
    if out is None:
        out = torch.empty((mt, nt, K // 64), dtype=torch.int32, device=xq.device)
    check(lib.svdq_debug_group_partials(
        _dptr(xq, torch.uint8, (M, K // 2), "xq"), _dptr(wq, torch.uint8, (N, K // 2), "wq"),
        M, N, K, m0, n0, mt, nt, _dptr(out, torch.int32, (mt, nt, K // 64), "out"),
        _stream(xq.device)))
    return out


@dataclass
class PackedLinear:
    """Packed weights of one layer, resident on a device."""
    K: int
    N: int
    rank: int
    precision: int
    smooth_inv: object
    lora_down: object
    lora_up: object
    wq: object
    ws: object
    bias: object = None

    @classmethod
    def from_host(cls, packed: dict, bias_bf16: Optional[np.ndarray], rank: int,
                  precision: int = INT4, device="cuda"):
        torch = _torch()
        N, K2 = packed["wq"].shape

        def dev(a, dtype):
            t = torch.from_numpy(np.ascontiguousarray(a))
            if dtype in (torch.bfloat16,):
                t = t.view(torch.int16).view(torch.bfloat16)
            elif dtype == torch.float16 and t.dtype != torch.float16:
                t = t.view(torch.float16)
            return t.to(device)

        return cls(
            K=K2 * 2, N=N, rank=rank, precision=precision,
            smooth_inv=dev(packed["smooth_inv"], torch.float32),
            lora_down=dev(packed["lora_down"], torch.bfloat16) if rank else None,
            lora_up=dev(packed["lora_up"], torch.bfloat16) if rank else None,
            wq=dev(packed["wq"], torch.uint8),
            ws=dev(packed["ws"], torch.float16 if precision == INT4 else torch.uint8),
            bias=None if bias_bf16 is None else dev(bias_bf16, torch.bfloat16),
        )


def mlp(x, fc1: "PackedLinear", fc2: "PackedLinear", y=None):
    """The MLP pair fc2(GELU(fc1(x))) with the activation and fc2's first
    kernel fused into fc1's second kernel (INT4): three launches, no fc1
    output in memory."""
    M = x.shape[0]
    xq, xs, la = quantize_act_lora_down(x, fc1.smooth_inv, fc1.lora_down, fc1.rank)
    xq2, xs2, la2 = mlp_gemm_gelu_quant(xq, xs, fc1.wq, fc1.ws, la, fc1.lora_up, fc1.bias, M, fc1.N, fc1.K,
                                        fc1.rank, fc2.smooth_inv, fc2.lora_down, fc2.rank)
    return gemm_w4a4_lora_up(xq2, xs2, fc2.wq, fc2.ws, la2, fc2.lora_up, fc2.bias, M, fc2.N, fc2.K, fc2.rank, y=y)


def linear(x, layer: PackedLinear, y=None):
    """Y = layer(x) for x bf16 [M][K] on the device: both fused kernels."""
    M = x.shape[0]
    xq, xs, la = quantize_act_lora_down(x, layer.smooth_inv, layer.lora_down, layer.rank, layer.precision)
    return gemm_w4a4_lora_up(xq, xs, layer.wq, layer.ws, la, layer.lora_up, layer.bias,
                             M, layer.N, layer.K, layer.rank, layer.precision, y=y)

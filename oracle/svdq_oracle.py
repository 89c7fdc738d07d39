"""Plain CPU oracle of the SVDQuant W4A4 linear layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may use this module.  It shares no code with the HIP
path and never takes an input or an expected value from it.

What it computes, in the pages' order:

  Y = X^ . L1 . L2  +  dequant( Q4(X^) . Q4(R)^T )  +  b
  X^ = X . diag(lambda)^-1 ,   W^ = diag(lambda) . W = L1 . L2 + R

* Stage 2 of the "Overview of SVDQuant" figure caption (model card
  "svdq-int4-flux.1-dev"): outliers migrate from activations to weights
  (X^ = X diag(lambda)^-1, W^ = diag(lambda) W, so X^ W^ = X W).
* Stage 3 of the same caption and the SVDQuant abstract: W^ splits by SVD
  into a 16-bit low-rank branch L1 L2 and a residual R that is quantized to
  4 bits; activations are quantized to 4 bits as well (W4A4).
* Nunchaku engine figure caption (b): the down projection X^ L1 and the
  activation quantization read the same input; the up projection and the
  4-bit GEMM write the same output.  Fusion only moves data, so the oracle
  computes the unfused steps.

The pages give no formula for lambda, the quantizer, its group size, scale
dtype, rounding or packing.  The readings taken here (each one applies to
both this oracle and the GPU path):

  R1  lambda_j = sqrt(max(ax_j,1e-5)) / sqrt(max(aw_j,1e-5)) in fp64
      (migration strength 0.5), ax_j = max_m |X[m,j]| of the calibration
      activations, aw_j = max_n |W[j,n]|; the kernels multiply by the stored
      smooth_inv_j = fp32(1/lambda_j).
  R2  W^[j,n] = W[j,n] / smooth_inv_j in fp64 (the stored fp32 value).
  R3  top-r SVD W^ = U S V^T; L1 = bf16(fp32(U_r S_r)), L2 = bf16(fp32(V_r^T))
      (only the product L1 L2 is unique).
  R4  R = fp32(W^ - L1 L2) with the bf16-rounded factors (fp64 product).
  R5  INT4 groups of 64 along K: per token for X^, per output channel for R.
      s = fp16(fp32(amax / 7)) with round-to-nearest-even and saturation at
      65504; s == 0 -> all codes 0; otherwise inv = fp32(1/s) and
      q = clamp(rint(fp32(v * inv)), -7, 7), ties to even.
  R6  codes take 4 bits each, row-major [rows][K/2], in units of 16
      consecutive k stored as two little-endian 32-bit words (I0, I1).  A
      code q has the 6-bit image f(q) = 32 [q < 0] + |q| (sign in bit 5,
      |q| in bits 0-2, bits 3-4 zero: the FP6 E2M3 pattern of q/8).  The 16
      images of a unit, the j-th at bits 6j..6j+5, form a 96-bit string
      D0 | D1 << 32 | D2 << 64; then I0 = D0 | (D2 & Z0) and
      I1 = D1 | (D2 & Z1) with Z0 = 0x18618618 and Z1 = 0x86186186 -- the
      zero bits 3-4 of the images in D0 and D1, which together are exactly
      the 21 data bits of D2.  Sign and magnitude hold the quantizer's
      symmetric range [-7, 7]; zero carries no sign.  Scales are
      group-major [K/64][rows].
  R7  x^ = bf16(fp32(x * smooth_inv)), rounded once and used by both branches.
  R8  down projection t = X^ L1 in fp64 (the GPU keeps it in fp32 [M][r]);
      the up projection uses bf16(fp32(t)).
  R9  Y = bf16(fp32(acc + up + bias)) with acc = sum_g P_g s_x s_w.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "GROUP",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "f32_to_f16_sat",
    "quantize_groups", "pack_int4", "unpack_int4",
    "smoothing", "pack_weights", "smooth_act", "quantize_act_lora_down",
    "group_partials", "dequant_accumulate", "lora_up", "gemm_w4a4_lora_up",
    "gemm_dequant_form", "svdq_linear", "merge_lora", "gelu_tanh",
    "reference_linear", "relative_error",
]

GROUP = 64          # INT4 quantization group along K (reading R5)
QMAX = 7            # symmetric code range [-7, 7] (reading R5)
F16_MAX = 65504.0


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even.

    Worked out on the fp32 bit pattern: add 0x7FFF plus the lowest kept bit,
    then drop the 16 low bits.  NaN stays a quiet NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + keep_lsb) >> 16) & 0xFFFF
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40) & 0xFFFF
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """bf16 bit pattern -> fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_sat(a) -> np.ndarray:
    """fp32 -> fp16, round to nearest even, finite values saturate to +-65504
    (subnormal fp16 results are kept, never flushed)."""
    a = np.asarray(a, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = a.astype(np.float16)
    over = np.isinf(h) & np.isfinite(a)
    if np.any(over):
        h = np.array(h, copy=True)
        h[over] = np.where(a[over] > 0, np.float16(F16_MAX), np.float16(-F16_MAX))
    return h


# ---------------------------------------------------------------------------
# 4-bit quantizer (reading R5) and packing (reading R6)
# ---------------------------------------------------------------------------

def quantize_groups(v):
    """Symmetric INT4 quantization of fp32 rows in groups of 64 along K.

    v: fp32 [rows][K], K % 64 == 0.
    Returns (codes int8 [rows][K] in [-7, 7], scales fp16 [rows][K/64])."""
    v = np.asarray(v, dtype=np.float32)
    rows, K = v.shape
    assert K % GROUP == 0
    g = v.reshape(rows, K // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)                             # exact in fp32
    s = f32_to_f16_sat(amax / np.float32(QMAX))              # IEEE fp32 division
    s32 = s.astype(np.float32)
    zero = s32 == 0
    with np.errstate(divide="ignore"):
        inv = np.float32(1.0) / s32                          # IEEE fp32 division
    inv = np.where(zero, np.float32(0.0), inv).astype(np.float32)
    q = np.rint(g * inv[:, :, None])                          # fp32 product, ties to even
    q = np.clip(q, -QMAX, QMAX).astype(np.int8)
    q[zero] = 0
    return q.reshape(rows, K), s


_Z0 = 0x18618618     # bits 3,4 9,10 15,16 21,22 27,28: the zero bits 3-4 of the images in D0
_Z1 = 0x86186186     # bits 1,2 7,8 13,14 19,20 25,26 31: the same in D1
_UNIT = 16           # codes per unit (two 32-bit words)


def _images(q) -> np.ndarray:
    """int codes in [-7, 7] -> 6-bit images 32 [q < 0] + |q| (zero has no sign)."""
    q = np.asarray(q).astype(np.int64)
    assert np.all(np.abs(q) <= 7), "4-bit codes hold [-7, 7]"
    return np.where(q < 0, 32 - q, q).astype(np.uint64)


def pack_int4(q) -> np.ndarray:
    """int codes [rows][K] (K % 16 == 0) in [-7, 7] -> uint8 [rows][K/2]
    (reading R6): per unit of 16 consecutive k, the images f_j at bits
    6j..6j+5 of the 96-bit string D0 | D1 << 32 | D2 << 64, stored as
    I0 = D0 | (D2 & Z0), I1 = D1 | (D2 & Z1)."""
    f = _images(q)
    rows, K = f.shape
    assert K % _UNIT == 0
    f = f.reshape(rows, K // _UNIT, _UNIT)
    D = [np.zeros((rows, K // _UNIT), np.uint64) for _ in range(3)]
    for j in range(_UNIT):
        bit = 6 * j
        w, o = bit // 32, bit % 32
        D[w] |= (f[:, :, j] << np.uint64(o)) & np.uint64(0xFFFFFFFF)
        if o + 6 > 32:                              # the image straddles two words
            D[w + 1] |= f[:, :, j] >> np.uint64(32 - o)
    z0, z1 = np.uint64(_Z0), np.uint64(_Z1)
    assert not np.any(D[0] & z0) and not np.any(D[1] & z1)
    assert not np.any(D[2] & ~(z0 | z1) & np.uint64(0xFFFFFFFF))
    words = np.stack([D[0] | (D[2] & z0), D[1] | (D[2] & z1)], axis=2).astype("<u4")
    return np.ascontiguousarray(words).view(np.uint8).reshape(rows, K // 2)


def unpack_int4(p) -> np.ndarray:
    """Inverse of pack_int4: D0 = I0 & ~Z0, D1 = I1 & ~Z1,
    D2 = (I0 & Z0) | (I1 & Z1); image j = bits 6j..6j+5 of the 96-bit
    string, read as sign (bit 5) and magnitude (bits 0-2)."""
    p = np.ascontiguousarray(p, dtype=np.uint8)
    rows, nb = p.shape
    assert nb % 8 == 0
    w = p.view("<u4").astype(np.uint64).reshape(rows, nb // 8, 2)
    z0, z1, m32 = np.uint64(_Z0), np.uint64(_Z1), np.uint64(0xFFFFFFFF)
    D = [w[:, :, 0] & ~z0 & m32, w[:, :, 1] & ~z1 & m32, (w[:, :, 0] & z0) | (w[:, :, 1] & z1)]
    out = np.empty((rows, nb // 8, _UNIT), dtype=np.int8)
    for j in range(_UNIT):
        bit = 6 * j
        wd, o = bit // 32, bit % 32
        f = D[wd] >> np.uint64(o)
        if o + 6 > 32:
            f = f | (D[wd + 1] << np.uint64(32 - o))
        f = f & np.uint64(63)
        mag = (f & np.uint64(7)).astype(np.int8)
        out[:, :, j] = np.where(f & np.uint64(32), -mag, mag)
    return out.reshape(rows, nb * 2)


# ---------------------------------------------------------------------------
# offline side: smoothing, SVD, residual quantization (stages 2 and 3)
# ---------------------------------------------------------------------------

def smoothing(act_absmax, w_bits):
    """Reading R1.  act_absmax fp32 [K]; w_bits bf16 [N][K] (nn.Linear
    layout, W = W_lin^T).  Returns (lambda fp64 [K], smooth_inv fp32 [K])."""
    w = bf16_bits_to_f32(w_bits).astype(np.float64)
    aw = np.abs(w).max(axis=0)
    ax = np.asarray(act_absmax, dtype=np.float32).astype(np.float64)
    lam = np.sqrt(np.maximum(ax, 1e-5)) / np.sqrt(np.maximum(aw, 1e-5))
    smooth_inv = (1.0 / lam).astype(np.float32)
    return lam, smooth_inv


def pack_weights(w_bits, act_absmax, rank):
    """Offline pack (readings R1-R6).

    Returns a dict with smooth_inv fp32 [K], l1 bf16 bits [K][r],
    l2 bf16 bits [r][N], wq uint8 [N][K/2], ws fp16 [K/64][N], r fp32 [K][N],
    w_hat fp64 [K][N] and the singular values of W^."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    _, smooth_inv = smoothing(act_absmax, w_bits)
    w = bf16_bits_to_f32(w_bits).astype(np.float64).T            # K x N
    w_hat = w / smooth_inv.astype(np.float64)[:, None]           # R2
    if rank > 0:
        u, sig, vt = np.linalg.svd(w_hat, full_matrices=False)   # R3
        l1 = f32_to_bf16_bits((u[:, :rank] * sig[:rank]).astype(np.float32))
        l2 = f32_to_bf16_bits(vt[:rank].astype(np.float32))
        low = bf16_bits_to_f32(l1).astype(np.float64) @ bf16_bits_to_f32(l2).astype(np.float64)
    else:
        sig = None
        l1 = np.zeros((K, 0), dtype=np.uint16)
        l2 = np.zeros((0, N), dtype=np.uint16)
        low = 0.0
    r = (w_hat - low).astype(np.float32)                        # R4
    q, s = quantize_groups(np.ascontiguousarray(r.T))           # per output channel
    return dict(smooth_inv=smooth_inv, l1=l1, l2=l2, wq=pack_int4(q),
                ws=np.ascontiguousarray(s.T), r=r, w_hat=w_hat, sigma=sig)


# ---------------------------------------------------------------------------
# online side, first fused kernel: smoothing + quantize + down projection
# ---------------------------------------------------------------------------

def smooth_act(x_bits, smooth_inv) -> np.ndarray:
    """Reading R7: x^ = bf16(fp32(x * smooth_inv)).  Returns bf16 bits."""
    x = bf16_bits_to_f32(x_bits)
    return f32_to_bf16_bits(x * np.asarray(smooth_inv, np.float32)[None, :])


def quantize_act_lora_down(x_bits, smooth_inv, l1_bits):
    """What the first fused kernel computes: X^, Q4(X^) and X^ L1.

    Returns dict(xhat bf16 bits [M][K], xq uint8 [M][K/2],
    xs fp16 [K/64][M], t fp64 [M][r])."""
    xh_bits = smooth_act(x_bits, smooth_inv)
    xh = bf16_bits_to_f32(xh_bits)
    q, s = quantize_groups(xh)
    l1 = bf16_bits_to_f32(l1_bits).astype(np.float64)
    t = xh.astype(np.float64) @ l1 if l1.shape[1] else np.zeros((xh.shape[0], 0))
    return dict(xhat=xh_bits, xq=pack_int4(q), xs=np.ascontiguousarray(s.T), t=t)


# ---------------------------------------------------------------------------
# online side, second fused kernel: 4-bit GEMM + dequant + up projection
# ---------------------------------------------------------------------------

def group_partials(xq, wq) -> np.ndarray:
    """P[m, n, g] = sum over k in group g of qx[m,k] qw[n,k], exact integers.

    Each group's product is an fp64 matmul of integer-valued arrays; every
    partial sum is an integer below 2^53, so it is exact."""
    qx = unpack_int4(xq).astype(np.float64)
    qw = unpack_int4(wq).astype(np.float64)
    M, K = qx.shape
    N = qw.shape[0]
    G = K // GROUP
    P = np.empty((M, N, G), dtype=np.int64)
    for g in range(G):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        P[:, :, g] = np.rint(qx[:, sl] @ qw[:, sl].T).astype(np.int64)
    return P


def dequant_accumulate(P, xs, ws) -> np.ndarray:
    """acc[m,n] = sum_g P[m,n,g] * s_x[m,g] * s_w[n,g] in fp64."""
    sx = np.asarray(xs).astype(np.float64)      # [G][M]
    sw = np.asarray(ws).astype(np.float64)      # [G][N]
    M, N, G = P.shape
    acc = np.zeros((M, N), dtype=np.float64)
    for g in range(G):
        acc += P[:, :, g].astype(np.float64) * sx[g][:, None] * sw[g][None, :]
    return acc


def lora_up(t, l2_bits) -> np.ndarray:
    """Reading R8: up = bf16(fp32(t)) L2 in fp64."""
    l2 = bf16_bits_to_f32(l2_bits).astype(np.float64)
    if l2.shape[0] == 0:
        return np.zeros((np.asarray(t).shape[0], l2.shape[1]))
    tb = bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(t).astype(np.float32)))
    return tb.astype(np.float64) @ l2


def _bias64(bias_bits, N):
    if bias_bits is None:
        return np.zeros(N)
    return bf16_bits_to_f32(bias_bits).astype(np.float64)


def gemm_w4a4_lora_up(xq, xs, wq, ws, t, l2_bits, bias_bits=None):
    """What the second fused kernel computes (readings R8, R9).

    Returns dict(y bf16 bits [M][N], y64 fp64 pre-rounding sum, P, acc, up)."""
    P = group_partials(xq, wq)
    acc = dequant_accumulate(P, xs, ws)
    up = lora_up(t, l2_bits)
    y64 = acc + up + _bias64(bias_bits, acc.shape[1])[None, :]
    return dict(y=f32_to_bf16_bits(y64.astype(np.float32)), y64=y64,
                P=P, acc=acc, up=up)


def gemm_dequant_form(xq, xs, wq, ws, t, l2_bits, bias_bits=None):
    """Same result as gemm_w4a4_lora_up for large inputs.

    Uses the identity sum_g s_x s_w sum_{k in g} qx qw
    = sum_k (qx s_x)(qw s_w): one fp64 matmul of the decoded operands
    instead of one matmul per group.  Agrees with the per-group form to
    fp64 rounding."""
    qx = unpack_int4(xq).astype(np.float64)
    qw = unpack_int4(wq).astype(np.float64)
    sx = np.repeat(np.asarray(xs).astype(np.float64).T, GROUP, axis=1)   # [M][K]
    sw = np.repeat(np.asarray(ws).astype(np.float64).T, GROUP, axis=1)   # [N][K]
    acc = (qx * sx) @ (qw * sw).T
    up = lora_up(t, l2_bits)
    y64 = acc + up + _bias64(bias_bits, acc.shape[1])[None, :]
    return dict(y=f32_to_bf16_bits(y64.astype(np.float32)), y64=y64, acc=acc, up=up)


def svdq_linear(x_bits, packed, bias_bits=None, per_group=True):
    """Whole layer: first fused kernel, then second fused kernel."""
    a = quantize_act_lora_down(x_bits, packed["smooth_inv"], packed["l1"])
    f = gemm_w4a4_lora_up if per_group else gemm_dequant_form
    b = f(a["xq"], a["xs"], packed["wq"], packed["ws"], a["t"], packed["l2"], bias_bits)
    b.update(a)
    return b


# ---------------------------------------------------------------------------
# LoRA without re-quantization (SVDQuant abstract; Nunchaku Lite keeps the
# LoRA loading hooks working)
# ---------------------------------------------------------------------------

def merge_lora(l1_bits, l2_bits, smooth_inv, a_bits, b_bits):
    """Concatenate an off-the-shelf LoRA (Y += X A B) to the low-rank branch.

    The branch sees X^ = X diag(smooth_inv), so A is folded with
    diag(1/smooth_inv): L1' = [L1 | bf16(fp32(A / smooth_inv))],
    L2' = [L2 ; B].  The 4-bit residual is left as it is."""
    a = bf16_bits_to_f32(a_bits).astype(np.float64)
    a_fold = a / np.asarray(smooth_inv, np.float32).astype(np.float64)[:, None]
    l1n = np.concatenate([np.asarray(l1_bits, np.uint16),
                          f32_to_bf16_bits(a_fold.astype(np.float32))], axis=1)
    l2n = np.concatenate([np.asarray(l2_bits, np.uint16),
                          np.asarray(b_bits, np.uint16)], axis=0)
    return l1n, l2n


# ---------------------------------------------------------------------------
# helpers for building the second layer of the MLP pair and for quality
# ---------------------------------------------------------------------------

def gelu_tanh(y):
    """tanh-approximated GELU in fp64 (FLUX's MLP activation):
    0.5 y (1 + tanh(u)), u = sqrt(2/pi) (y + 0.044715 y^3).  Evaluated as
    y / (1 + exp(-2u)), the same function, so that negative y do not lose
    everything to the cancellation in 1 + tanh(u) (which is 0 in fp64 once
    u < -19); exp overflowing to inf gives -0 for very negative y."""
    y = np.asarray(y, dtype=np.float64)
    u = np.sqrt(2.0 / np.pi) * (y + 0.044715 * y ** 3)
    with np.errstate(over="ignore"):
        return y / (1.0 + np.exp(-2.0 * u))


def reference_linear(x_bits, w_bits, bias_bits=None) -> np.ndarray:
    """Unquantized X W + b in fp64 (W given in nn.Linear layout)."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    w = bf16_bits_to_f32(w_bits).astype(np.float64)
    y = x @ w.T
    return y + _bias64(bias_bits, y.shape[1])[None, :]


def relative_error(y_bits, y_ref64) -> float:
    y = bf16_bits_to_f32(y_bits).astype(np.float64)
    return float(np.linalg.norm(y - y_ref64) / np.linalg.norm(y_ref64))

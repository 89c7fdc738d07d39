"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: bit-exact on packed 4-bit codes, fp16 scales and per-group int32
partials; the fp32 down projection within rtol 1e-3; Y within
max|Y - Y_oracle| <= 1e-2 * max|Y_oracle| (bf16 output rounding)."""

import sys

import numpy as np
import pytest
import torch

import bit_quantized_diffusion_amd as bq
import oracle as O
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu

Y_TOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def device_layer(case):
    pk, r = case["pk"], case["rank"]
    return bq.PackedLinear(
        K=case["x"].shape[1], N=pk["wq"].shape[0], rank=r, precision=bq.INT4,
        smooth_inv=dev(pk["smooth_inv"]),
        lora_down=dev_bf16(pk["l1"].T) if r else None,
        lora_up=dev_bf16(pk["l2"].T) if r else None,
        wq=dev(pk["wq"]), ws=dev(pk["ws"]),
        bias=None if case["bias"] is None else dev_bf16(case["bias"]))


def assert_y_close(y_bits, ref_bits, what, slack=None, y64=None):
    """The stated bound, max|dY| <= 1e-2 max|Y_oracle|, always; with `slack`
    (per-element fp32 slack of the pre-rounding sum, from the oracle's own
    terms) and the oracle's exact sum `y64` also the per-element bound
    |dY| <= ulp_bf16(|y64| + slack) + slack: the GPU's fp32 sum is within
    `slack` of the exact one, and two round-to-nearest bf16 roundings of
    values that close differ by at most that plus one bf16 step."""
    y = O.bf16_bits_to_f32(y_bits).astype(np.float64)
    r = O.bf16_bits_to_f32(ref_bits).astype(np.float64)
    err = np.max(np.abs(y - r))
    bound = Y_TOL * np.max(np.abs(r))
    msg = (f"  {what}: max|dY| = {err:.3e}  bound {bound:.3e}  "
           f"exact-bf16 fraction {np.mean(y_bits == ref_bits):.4f}")
    if slack is not None:
        per = C.ulp_bf16(np.abs(y64) + slack) + slack
        worst = np.max(np.abs(y - r) / per)
        msg += f"  per-element worst |dY|/bound {worst:.3f}"
    say(msg)
    assert err <= bound
    if slack is not None:
        bad = np.abs(y - r) > per
        assert not bad.any(), f"{int(bad.sum())} elements outside the per-element bound"


SMALL = [
    (256, 512, 512, 16, 0, False),    # tiny config shape, no bias
    (300, 576, 200, 32, 1, True),     # ragged M, 9 groups (ragged K step)
    (129, 192, 131, 48, 2, True),     # rank 48, odd N (element stores)
    (1, 64, 1, 0, 3, True),           # single token, single channel, rank 0
    (64, 256, 64, 64, 4, False),
    (520, 1024, 264, 16, 5, True),
    (40, 4096, 272, 256, 6, True),    # largest rank
    (136, 8192, 144, 16, 7, True),    # long K loop: the fused GEMM's coarse schedule
    (72, 8256, 136, 32, 8, True),     # long K loop, odd group count
    (130, 64, 150, 16, 9, True),      # one group (one half stage) with the low-rank branch
    (257, 128, 129, 32, 10, False),   # one stage, ragged M and N
    (33, 8192, 131, 16, 11, True),    # coarse schedule with odd N (element stores)
    (70, 320, 131, 32, 12, True),     # rank 32 (up projection and bias via LDS), odd N, odd group count
    (65, 256, 34, 32, 13, True),      # rank 32, two stages, ragged even N (bias via LDS)
    (40, 128, 45, 32, 14, True),      # rank 32, one stage (operands issued with stage 0), odd N
    (130, 128, 160, 32, 15, False),   # rank 32, one stage, no bias
]


def _small(p):
    return C.small_case(*p)


@pytest.fixture(autouse=True)
def _require_device():
    assert bq.device_check(0), "gfx950 device required for the GPU tests"


@pytest.mark.parametrize("p", SMALL, ids=lambda p: "M%dK%dN%dr%d" % p[:4])
def test_k1_parity(p):
    case = _small(p)
    say(f"k1 {p}")
    pk, r = case["pk"], case["rank"]
    layer = device_layer(case)
    xq, xs, la = bq.quantize_act_lora_down(dev_bf16(case["x"]), layer.smooth_inv, layer.lora_down, r)
    torch.cuda.synchronize()
    ref = O.quantize_act_lora_down(case["x"], pk["smooth_inv"], pk["l1"])
    assert np.array_equal(xq.cpu().numpy(), ref["xq"])
    assert np.array_equal(host_u16(xs), ref["xs"].view(np.uint16))
    if r:
        t = ref["t"]
        got = la.cpu().numpy().astype(np.float64)
        assert np.allclose(got, t, rtol=1e-3, atol=1e-4 * np.max(np.abs(t)))


def test_k1_quantizer_edge_values():
    """Magnitudes across the bf16 range, exact ties, zero groups, groups
    whose fp16 scale is subnormal, flushes to zero or saturates."""
    rng = np.random.default_rng(99)
    M, K = 96, 512
    x = np.zeros((M, K), np.float32)
    for m in range(M):
        e = -40 + (m * 61) // M          # 2^-40 .. 2^20
        row = rng.standard_normal(K).astype(np.float32) * np.float32(2.0 ** e)
        if m % 5 == 1:                   # exact ties after scaling
            row = ((rng.integers(-6, 6, K) + 0.5) * 2.0 ** (e - 3)).astype(np.float32)
            row[::64] = np.float32(7 * 2.0 ** (e - 3))
        if m % 7 == 2:
            row[64:128] = 0
        x[m] = row
    x[3, :64] = np.float32(458752.0)     # saturating scale
    x[4, :2] = [np.float32(7 * 2.0 ** -25), 0]   # scale ties to zero
    xb = O.f32_to_bf16_bits(x)
    sinv = np.ones(K, np.float32)
    xq, xs, _ = bq.quantize_act_lora_down(dev_bf16(xb), dev(sinv), None, 0)
    torch.cuda.synchronize()
    ref = O.quantize_act_lora_down(xb, sinv, np.zeros((K, 0), np.uint16))
    assert np.array_equal(xq.cpu().numpy(), ref["xq"])
    assert np.array_equal(host_u16(xs), ref["xs"].view(np.uint16))


@pytest.mark.parametrize("p", SMALL, ids=lambda p: "M%dK%dN%dr%d" % p[:4])
def test_partials_exact(p):
    case = _small(p)
    say(f"partials {p}")
    pk = case["pk"]
    ref_a = O.quantize_act_lora_down(case["x"], pk["smooth_inv"], pk["l1"])
    M, K = case["x"].shape
    N = pk["wq"].shape[0]
    xq, wq = dev(ref_a["xq"]), dev(pk["wq"])
    P = bq.debug_group_partials(xq, wq, M, N, K, 0, 0, M, N)
    torch.cuda.synchronize()
    ref = O.group_partials(ref_a["xq"], pk["wq"])
    assert np.array_equal(P.cpu().numpy().astype(np.int64), ref)
    if M > 3 and N > 3:      # an interior window
        m0, n0, mt, nt = M // 3, N // 3, max(1, M // 2), max(1, N // 2)
        Pw = bq.debug_group_partials(xq, wq, M, N, K, m0, n0, mt, nt)
        torch.cuda.synchronize()
        assert np.array_equal(Pw.cpu().numpy().astype(np.int64), ref[m0:m0 + mt, n0:n0 + nt])


@pytest.mark.parametrize("p", SMALL, ids=lambda p: "M%dK%dN%dr%d" % p[:4])
def test_k2_parity(p):
    case = _small(p)
    say(f"k2 {p}")
    pk, r = case["pk"], case["rank"]
    M, K = case["x"].shape
    N = pk["wq"].shape[0]
    ref = C.oracle_rows(case, np.arange(M))
    layer = device_layer(case)
    la = dev(ref["t"].astype(np.float32)) if r else None
    y = bq.gemm_w4a4_lora_up(dev(ref["xq"]), dev(ref["xs"]), layer.wq, layer.ws, la, layer.lora_up,
                             layer.bias, M, N, K, r)
    torch.cuda.synchronize()
    sl = C.int4_slack(ref, ref["xs"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=False)
    assert_y_close(host_u16(y), ref["y"], "k2", sl, ref["y64"])


# scale regimes for the GEMM's exponent/significand split of s_w * s_x
_SCALE_KINDS = ("subnormal", "huge", "mixed")


def _scales(rng, kind, shape):
    """fp16 scale arrays that span the format: zero, subnormal, normal and
    the largest finite value, as bit patterns."""
    if kind == "subnormal":
        bits = rng.integers(1, 0x0400, size=shape)                       # 2^-24 .. just below 2^-14
        bits[..., ::7] = 0x0001
        bits[..., 3::11] = 0x03FF
    elif kind == "huge":
        bits = rng.integers(0x7000, 0x7C00, size=shape)                  # 2^13 .. 65504
        bits[..., ::5] = 0x7BFF
    else:
        bits = rng.integers(0, 0x7C00, size=shape)                        # every finite positive value
        bits[..., ::13] = 0x0000
        bits[..., 1::17] = 0x0001
        bits[..., 2::19] = 0x0400
        bits[..., 3::23] = 0x7BFF
    return bits.astype(np.uint16).view(np.float16)


@pytest.mark.parametrize("kind", _SCALE_KINDS)
@pytest.mark.parametrize("rank", [0, 16])
def test_k2_scale_extremes(kind, rank):
    """The GEMM on hand-made codes and scales across the whole fp16 range
    (zero scales with non-zero codes included: their products are zero)."""
    say(f"k2 scales {kind} rank {rank}")
    rng = np.random.default_rng([77, rank, _SCALE_KINDS.index(kind)])
    M, K, N = 131, 640, 140
    G = K // 64
    qx = rng.integers(-7, 8, size=(M, K))
    qw = rng.integers(-7, 8, size=(N, K))
    xq, wq = O.pack_int4(qx), O.pack_int4(qw)
    xs, ws = _scales(rng, kind, (G, M)), _scales(rng, kind, (G, N))
    t = rng.standard_normal((M, rank)).astype(np.float32)
    l2 = O.f32_to_bf16_bits((rng.standard_normal((rank, N)) * 0.05).astype(np.float32))
    bias = O.f32_to_bf16_bits((rng.standard_normal(N) * 0.01).astype(np.float32))
    if kind == "subnormal":
        # products near 2^-48: keep the output made of them alone
        bias, t, l2 = None, t * 0, l2 * 0
    ref = O.gemm_w4a4_lora_up(xq, xs, wq, ws, t.astype(np.float64), l2, bias)
    y = bq.gemm_w4a4_lora_up(dev(xq), dev(xs), dev(wq), dev(ws), dev(t) if rank else None,
                             dev_bf16(np.ascontiguousarray(l2.T)) if rank else None,
                             None if bias is None else dev_bf16(bias), M, N, K, rank)
    torch.cuda.synchronize()
    yb = host_u16(y)
    assert np.all(np.isfinite(O.bf16_bits_to_f32(yb)))
    sl = C.int4_slack(ref, xs, ws, t, l2, bias, t_from_kernel=False)
    assert_y_close(yb, ref["y"], f"k2 scales {kind}", sl, ref["y64"])


@pytest.mark.parametrize("kind", _SCALE_KINDS)
def test_k2_single_group_scales_bit_exact(kind):
    """K = 64 (one group), rank 0, no bias: Y = bf16(P s_x s_w) with the
    product P s_x s_w rounded once to fp32 on both sides (P has at most 12
    significant bits and each scale 11, so the fp64 product is exact), so
    every element must be bit-exact -- every (s_x, s_w) pair and every
    partial is checked on its own, whatever its magnitude."""
    say(f"k2 one group, scales {kind}")
    rng = np.random.default_rng([78, _SCALE_KINDS.index(kind)])
    M, K, N = 200, 64, 160
    qx = rng.integers(-7, 8, size=(M, K))
    qw = rng.integers(-7, 8, size=(N, K))
    qx[0, :] = 7
    qw[0, :] = -7                      # P = -3136 at (0, 0)
    xq, wq = O.pack_int4(qx), O.pack_int4(qw)
    xs, ws = _scales(rng, kind, (1, M)), _scales(rng, kind, (1, N))
    ref = O.gemm_w4a4_lora_up(xq, xs, wq, ws, np.zeros((M, 0)), np.zeros((0, N), np.uint16), None)
    y = bq.gemm_w4a4_lora_up(dev(xq), dev(xs), dev(wq), dev(ws), None, None, None, M, N, K, 0)
    torch.cuda.synchronize()
    yb = host_u16(y)
    same = yb == ref["y"]
    say(f"  exact-bf16 fraction {np.mean(same):.5f}")
    assert same.all(), f"{int((~same).sum())} of {same.size} outputs differ"


@pytest.mark.parametrize("p", SMALL, ids=lambda p: "M%dK%dN%dr%d" % p[:4])
def test_layer_end_to_end(p):
    case = _small(p)
    say(f"layer {p}")
    M = case["x"].shape[0]
    ref = C.oracle_rows(case, np.arange(M))
    y = bq.linear(dev_bf16(case["x"]), device_layer(case))
    torch.cuda.synchronize()
    pk = case["pk"]
    sl = C.int4_slack(ref, ref["xs"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    assert_y_close(host_u16(y), ref["y"], "layer", sl, ref["y64"])


@pytest.mark.parametrize("p", SMALL, ids=lambda p: "M%dK%dN%dr%d" % p[:4])
def test_unfused_baseline(p):
    """The four-kernel baseline computes the same layer: against the oracle
    to the same tolerance (its Y is rounded to bf16 twice), and its codes
    and scales are the fused path's bit for bit."""
    case = _small(p)
    say(f"unfused {p}")
    M = case["x"].shape[0]
    ref = C.oracle_rows(case, np.arange(M))
    layer = device_layer(case)
    x = dev_bf16(case["x"])
    y = bq.unfused_linear(x, layer)
    xq, xs, _ = bq.quantize_act_lora_down(x, layer.smooth_inv, layer.lora_down, layer.rank)
    xq_u = torch.empty_like(xq)
    xs_u = torch.empty_like(xs)
    bq.unfused_linear(x, layer, xq=xq_u, xs=xs_u)
    torch.cuda.synchronize()
    assert torch.equal(xq, xq_u) and torch.equal(xs.view(torch.int16), xs_u.view(torch.int16))
    pk = case["pk"]
    sl = C.int4_slack(ref, ref["xs"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    sl = sl + 0.5 * C.ulp_bf16(np.abs(ref["acc"]) + sl)     # the GEMM's own bf16 rounding before the up projection
    assert_y_close(host_u16(y), ref["y"], "unfused", sl, ref["y64"])


@pytest.mark.parametrize("name", ["fc1", "fc2"])
def test_unfused_baseline_full_size(name):
    """The four-kernel baseline on the FLUX MLP layers the fusion ablation
    times: codes and scales equal to the fused path's on every row, Y on
    sampled rows against the oracle (bound as in the small-shape test)."""
    case = _full_case(name)
    pk = case["pk"]
    M = case["x"].shape[0]
    say(f"unfused full-size {name}")
    layer = device_layer(case)
    x = dev_bf16(case["x"])
    xq_u = torch.empty((M, x.shape[1] // 2), dtype=torch.uint8, device=x.device)
    xs_u = torch.empty((x.shape[1] // 64, M), dtype=torch.float16, device=x.device)
    y = bq.unfused_linear(x, layer, xq=xq_u, xs=xs_u)
    xq, xs, _ = bq.quantize_act_lora_down(x, layer.smooth_inv, layer.lora_down, layer.rank)
    torch.cuda.synchronize()
    assert torch.equal(xq, xq_u) and torch.equal(xs.view(torch.int16), xs_u.view(torch.int16))
    rows = _sample_rows(M, seed=3)
    ref = C.oracle_rows(case, rows)
    sl = C.int4_slack(ref, ref["xs"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    sl = sl + 0.5 * C.ulp_bf16(np.abs(ref["acc"]) + sl)
    assert_y_close(host_u16(y)[rows], ref["y"], f"unfused {name}", sl, ref["y64"])


def test_outputs_reused_buffers_and_streams():
    """Caller-owned outputs are written in place; a side stream works."""
    case = _small(SMALL[1])
    M = case["x"].shape[0]
    layer = device_layer(case)
    x = dev_bf16(case["x"])
    ref = C.oracle_rows(case, np.arange(M))
    y = torch.full((M, layer.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        bq.linear(x, layer, y=y)
    s.synchronize()
    pk = case["pk"]
    sl = C.int4_slack(ref, ref["xs"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    assert_y_close(host_u16(y), ref["y"], "stream", sl, ref["y64"])


# ---------------------------------------------------------------------------
# full FLUX sizes: whole tensors on the GPU, oracle on sampled rows
# ---------------------------------------------------------------------------

def _sample_rows(M, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 17, 1000, 2047, 4095, 4096, M - 2, M - 1]
    rest = rng.choice(M, 23, replace=False)
    return np.unique(np.concatenate([fixed, rest]))


def _full_case(name):
    if name == "fc2":
        return C.mlp_pair()[1]
    return C.named_case(name)


@pytest.mark.parametrize("name", ["qkv", "fc1", "fc1_lora", "fc2"])
def test_full_size_layer(name):
    say(f"full-size {name}: building oracle case")
    case = _full_case(name)
    pk, r = case["pk"], case["rank"]
    M, K = case["x"].shape
    N = pk["wq"].shape[0]
    say(f"full-size {name}: M={M} K={K} N={N} rank={r}")
    layer = device_layer(case)
    x = dev_bf16(case["x"])
    xq, xs, la = bq.quantize_act_lora_down(x, layer.smooth_inv, layer.lora_down, r)
    y = bq.gemm_w4a4_lora_up(xq, xs, layer.wq, layer.ws, la, layer.lora_up, layer.bias, M, N, K, r)
    torch.cuda.synchronize()
    # first kernel on every row: exact codes and scales
    ref_a = O.quantize_act_lora_down(case["x"], pk["smooth_inv"], pk["l1"])
    assert np.array_equal(xq.cpu().numpy(), ref_a["xq"])
    assert np.array_equal(host_u16(xs), ref_a["xs"].view(np.uint16))
    t = ref_a["t"]
    assert np.allclose(la.cpu().numpy().astype(np.float64), t, rtol=1e-3, atol=1e-4 * np.max(np.abs(t)))
    # exact partials on windows, including the ragged corner
    for (m0, n0) in [(0, 0), (M - 70, N - 70), (M // 2, N // 3)]:
        mt, nt = 64, 64
        P = bq.debug_group_partials(xq, layer.wq, M, N, K, m0, n0, mt, nt)
        torch.cuda.synchronize()
        refP = O.group_partials(ref_a["xq"][m0:m0 + mt], pk["wq"][n0:n0 + nt])
        assert np.array_equal(P.cpu().numpy().astype(np.int64), refP)
    # Y on sampled rows
    rows = _sample_rows(M)
    ref = C.oracle_rows(case, rows)
    sl = C.int4_slack(ref, ref["xs"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    assert_y_close(host_u16(y)[rows], ref["y"], f"{name} end to end", sl, ref["y64"])


@pytest.mark.parametrize("name", ["fc1", "fc2"])
def test_per_gpu_share_every_row(name):
    """The FLUX MLP layers at M = 576, the token rows each of eight GPUs
    holds when the 4608 rows are split (fc2's 120 tiles fill under a
    quarter of the workgroup slots): codes, scales and Y of every row
    against the oracle."""
    case = _full_case(name)
    pk, r = case["pk"], case["rank"]
    M, K = 576, case["x"].shape[1]
    N = pk["wq"].shape[0]
    say(f"per-GPU share {name}: M={M} K={K} N={N} rank={r}")
    layer = device_layer(case)
    x = dev_bf16(case["x"][:M])
    xq, xs, la = bq.quantize_act_lora_down(x, layer.smooth_inv, layer.lora_down, r)
    y = bq.gemm_w4a4_lora_up(xq, xs, layer.wq, layer.ws, la, layer.lora_up, layer.bias, M, N, K, r)
    torch.cuda.synchronize()
    ref = C.oracle_rows(case, np.arange(M))
    assert np.array_equal(xq.cpu().numpy(), ref["xq"])
    assert np.array_equal(host_u16(xs), ref["xs"].view(np.uint16))
    sl = C.int4_slack(ref, ref["xs"], pk["ws"], ref["t"], pk["l2"], case["bias"], t_from_kernel=True)
    assert_y_close(host_u16(y), ref["y"], f"{name} M=576", sl, ref["y64"])


def test_layer_with_merged_lora():
    """A rank-32 layer with a rank-16 adapter merged by the library's host
    call (svdq_merge_lora): the rank-48 hot path against the oracle of the
    merged layer."""
    spec_case = C.small_case(200, 768, 264, 32, 21, True, 16)
    x = spec_case["x"]
    M, K = x.shape
    lay_pk = spec_case["pk"]          # oracle-packed, LoRA merged by the oracle
    say("merged LoRA layer")
    # the library's merge of the same adapter onto the same unmerged factors
    spec = spec_case["spec"]
    a_bits, b_bits = synth.gen_lora(spec)
    base = O.pack_weights(spec_case["w"], spec_case["ax"], 32)
    down, up = bq.merge_lora(np.ascontiguousarray(base["l1"].T), np.ascontiguousarray(base["l2"].T),
                             base["smooth_inv"], a_bits, b_bits)
    assert np.array_equal(down, np.ascontiguousarray(lay_pk["l1"].T))
    assert np.array_equal(up, np.ascontiguousarray(lay_pk["l2"].T))
    layer = bq.PackedLinear(K=K, N=base["wq"].shape[0], rank=48, precision=bq.INT4,
                            smooth_inv=dev(base["smooth_inv"]), lora_down=dev_bf16(down), lora_up=dev_bf16(up),
                            wq=dev(base["wq"]), ws=dev(base["ws"]), bias=dev_bf16(spec_case["bias"]))
    ref = C.oracle_rows(spec_case, np.arange(M))
    y = bq.linear(dev_bf16(x), layer)
    torch.cuda.synchronize()
    sl = C.int4_slack(ref, ref["xs"], lay_pk["ws"], ref["t"], lay_pk["l2"], spec_case["bias"], t_from_kernel=True)
    assert_y_close(host_u16(y), ref["y"], "merged lora", sl, ref["y64"])

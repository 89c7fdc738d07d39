"""Pins for the CPU oracle: it is checked against things other than itself --
hand-derived fixtures, an exact-rational re-derivation of IEEE rounding,
brute-force integer loops, independent library routines (torch casts,
a symmetric eigensolver) and invariants of the method."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# exact-rational IEEE rounding (independent of numpy's float arithmetic)
# ---------------------------------------------------------------------------

def round_to_format(x: Fraction, p: int, emin: int) -> Fraction:
    """Round an exact rational to the nearest binary float with p significant
    bits and minimum normal exponent emin (gradual underflow), ties to even,
    unbounded exponent range above."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    n = a / ulp
    m = math.floor(n)
    rem = n - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return sign * m * ulp


def f32r(x):
    return round_to_format(Fraction(x), 24, -126)


def f16r_sat(x):
    r = round_to_format(Fraction(x), 11, -14)
    if abs(r) > 65504:
        r = Fraction(65504) * (1 if r > 0 else -1)
    return r


def rint_even(x: Fraction) -> int:
    m = math.floor(x)
    rem = x - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return m


def brute_quantize_group(vals):
    """One 64-group by the quantizer reading, in exact rationals."""
    fr = [Fraction(float(v)) for v in vals]
    amax = max(abs(v) for v in fr)
    s = f16r_sat(f32r(amax / 7))
    if s == 0:
        return [0] * len(vals), s
    inv = f32r(1 / s)
    return [max(-7, min(7, rint_even(f32r(v * inv)))) for v in fr], s


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_bf16_roundtrip_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_bits_to_f32(bits)
    back = O.f32_to_bf16_bits(f)
    finite = ~np.isnan(f)
    assert np.array_equal(back[finite], bits[finite])
    assert np.all(np.isnan(O.bf16_bits_to_f32(back[~finite])))


def test_bf16_matches_torch_cast_random_and_ties():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # force a quarter of them to exact ties (low half = 0x8000)
    u[: len(u) // 4] = (u[: len(u) // 4] & 0xFFFF0000) | 0x8000
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ours = O.f32_to_bf16_bits(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # torch may turn values that overflow bf16 into inf the same way (RNE)
    assert np.array_equal(ours, ref)


def test_f16_saturating_known_values():
    cases = {
        65504.0: 65504.0, 65519.0: 65504.0, 65520.0: 65504.0, 1e6: 65504.0,
        -1e6: -65504.0, 2.0 ** -24: 2.0 ** -24, 2.0 ** -25: 0.0,
        3 * 2.0 ** -25: 2.0 ** -23, 1 + 2.0 ** -11: 1.0, 1 + 3 * 2.0 ** -11: 1 + 2.0 ** -9,
    }
    a = np.array(list(cases.keys()), dtype=np.float32)
    h = O.f32_to_f16_sat(a).astype(np.float64)
    assert list(h) == list(cases.values())


def test_f16_matches_torch_half_cast():
    rng = np.random.default_rng(8)
    f = (rng.standard_normal(1 << 18) * np.exp2(rng.uniform(-30, 17, 1 << 18))).astype(np.float32)
    ours = O.f32_to_f16_sat(f)
    ref = torch.from_numpy(f).to(torch.float16).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin].view(np.uint16), ref[fin].view(np.uint16))
    assert np.all(np.abs(ours[~fin]) == np.float16(65504))


# ---------------------------------------------------------------------------
# quantizer and packing
# ---------------------------------------------------------------------------

def _golden(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


def _group_from(case, n=64):
    v = np.zeros(n, dtype=np.float32)
    for k, hx in case["values"].items():
        v[int(k)] = np.float32(float.fromhex(hx))
    return v


@pytest.mark.parametrize("case", _golden("int4_groups.json")["cases"], ids=lambda c: c["name"])
def test_quantizer_golden(case):
    v = _group_from(case)
    q, s = O.quantize_groups(v[None, :])
    assert int(s.view(np.uint16)[0, 0]) == int(case["scale_f16_bits"], 16)
    want = np.zeros(64, dtype=np.int8)
    for k, c in case["codes"].items():
        want[int(k)] = c
    assert np.array_equal(q[0], want)
    packed = O.pack_int4(q)
    want_b = np.zeros(32, dtype=np.uint8)
    for k, b in case["packed_bytes"].items():
        want_b[int(k)] = int(b, 16)
    assert np.array_equal(packed[0], want_b)


def test_quantizer_vs_exact_rational_bruteforce():
    rng = np.random.default_rng(11)
    groups = []
    for i in range(48):
        scale = 2.0 ** rng.integers(-30, 12)
        g = (rng.standard_normal(64) * scale).astype(np.float32)
        if i % 4 == 1:     # plant exact ties after scaling by a power-of-two s
            s = 2.0 ** rng.integers(-10, 5)
            k = rng.integers(-6, 6, 64) + 0.5
            k[0] = 7
            g = (k * s).astype(np.float32)
        if i % 4 == 2:
            g[rng.integers(0, 64, 40)] = 0
        groups.append(g)
    v = np.stack(groups)
    q, s = O.quantize_groups(v)
    for i in range(len(groups)):
        codes, sref = brute_quantize_group(v[i])
        assert Fraction(float(s[i, 0])) == sref
        assert list(q[i]) == codes, i


def test_quantizer_grid_lossless():
    rng = np.random.default_rng(12)
    for e in range(-14, 12):
        s = 2.0 ** e
        k = rng.integers(-7, 8, (4, 64))
        k[:, 5] = 7 * np.where(rng.random(4) < 0.5, 1, -1)
        q, sc = O.quantize_groups((k * s).astype(np.float32))
        assert np.array_equal(q, k)
        assert np.all(sc.astype(np.float64) == s)


def test_quantizer_error_bound():
    rng = np.random.default_rng(13)
    v = (rng.standard_normal((64, 256)) * 3).astype(np.float32)
    q, s = O.quantize_groups(v)
    deq = q.reshape(64, 4, 64).astype(np.float64) * s.astype(np.float64)[:, :, None]
    err = np.abs(deq - v.reshape(64, 4, 64))
    assert np.all(err <= s.astype(np.float64)[:, :, None] * 0.5 * (1 + 1e-3))


def test_pack_bytes_and_roundtrip():
    # Unit [1, -1, -7, 7, 0, -5, 3, -3, 2, -2, 4, -4, 5, 6, -6, 0], worked by
    # hand: images f = [1, 33, 39, 7, 0, 37, 3, 35, 2, 34, 4, 36, 5, 6, 38, 0].
    # D0 = 1 + 33<<6 + 39<<12 + 7<<18 + 0<<24 + (37 & 3)<<30 = 0x401e7841;
    # D1 = 37>>2 + 3<<4 + 35<<10 + 2<<16 + 34<<22 + (4 & 15)<<28 = 0x48828c39;
    # D2 = 4>>4 + 36<<2 + 5<<8 + 6<<14 + 38<<20 + 0<<26 = 0x02618590.
    # I0 = D0 | (D2 & 0x18618618) = 0x401e7841 | 0x00618410 = 0x407ffc51,
    # I1 = D1 | (D2 & 0x86186186) = 0x48828c39 | 0x02000180 = 0x4a828db9.
    q = np.array([[1, -1, -7, 7, 0, -5, 3, -3, 2, -2, 4, -4, 5, 6, -6, 0]], dtype=np.int8)
    assert list(O.pack_int4(q)[0]) == [0x51, 0xFC, 0x7F, 0x40, 0xB9, 0x8D, 0x82, 0x4A]
    # all +7: D0 = 0xc71c71c7, D1 = 0x71c71c71, D2 = 0x1c71c71c -> I0 = 0xdf7df7df, I1 = 0x75d75d75
    assert list(O.pack_int4(np.full((1, 16), 7, np.int8))[0]) == [0xDF, 0xF7, 0x7D, 0xDF, 0x75, 0x5D, 0xD7, 0x75]
    rng = np.random.default_rng(1)
    q = rng.integers(-7, 8, (9, 128)).astype(np.int8)
    assert np.array_equal(O.unpack_int4(O.pack_int4(q)), q)
    # a sign bit on a zero magnitude decodes to 0
    d2 = 0x20 << 2                                   # image 11 = 0x20 (-0) at bits 2..7 of D2
    z1 = d2 & 0x86186186                             # its sign bit 7 lies in Z1
    w = np.array([[0, 0, 0, 0] + list(int(z1).to_bytes(4, "little"))], np.uint8)
    assert O.unpack_int4(w).tolist() == [[0] * 16]


def test_packed_unit_reads_as_fp6_e2m3():
    """The unit's three words D0, D1, D2, recovered from I0, I1 with the
    masks, hold the codes as FP6 E2M3 values q/8 (sign bit 5, exponent
    bits 3-4, mantissa bits 0-2; exponent 0 = subnormal m/8), the j-th at
    bits 6j of the 96-bit string: decoded by the E2M3 definition, not by
    unpack_int4."""
    rng = np.random.default_rng(2)
    q = rng.integers(-7, 8, (5, 64)).astype(np.int8)
    p = O.pack_int4(q).view("<u4").reshape(5, 4, 2).astype(np.uint64)
    for r in range(5):
        for u in range(4):
            i0, i1 = int(p[r, u, 0]), int(p[r, u, 1])
            d = (i0 & ~0x18618618 & 0xFFFFFFFF) | ((i1 & ~0x86186186 & 0xFFFFFFFF) << 32) | \
                (((i0 & 0x18618618) | (i1 & 0x86186186)) << 64)
            for j in range(16):
                f = (d >> (6 * j)) & 63
                sign, e, m = f >> 5, (f >> 3) & 3, f & 7
                val = (m / 8.0) if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 1)
                assert e == 0
                assert (-val if sign else val) == q[r, 16 * u + j] / 8.0


# ---------------------------------------------------------------------------
# smoothing (stage 2) and SVD (stage 3)
# ---------------------------------------------------------------------------

def test_smoothing_closed_form():
    ax = np.array([4.0, 1.0, 1e-7, 0.0], dtype=np.float32)
    w = np.array([[1.0, -4.0, 0.5, 0.0], [-0.5, 2.0, -1.0, 0.0]], dtype=np.float32)
    wb = O.f32_to_bf16_bits(w)
    lam, sinv = O.smoothing(ax, wb)
    # lambda = sqrt(max(ax,1e-5))/sqrt(max(aw,1e-5)): [2, 1/2, sqrt(1e-5), 1]
    assert sinv[0] == np.float32(0.5) and sinv[1] == np.float32(2.0)
    assert sinv[2] == np.float32(float.fromhex("0x1.3c3a4ep+8"))   # fp32 nearest sqrt(1e5)
    assert sinv[3] == np.float32(1.0)


def test_smoothing_preserves_product():
    spec = synth.layer_spec("tiny")
    lay = synth.gen_layer(spec)
    x = O.bf16_bits_to_f32(lay["x"]).astype(np.float64)
    ax = np.abs(O.bf16_bits_to_f32(lay["x"])).max(axis=0)
    _, sinv = O.smoothing(ax, lay["w"])
    w = O.bf16_bits_to_f32(lay["w"]).astype(np.float64).T
    xh = x * sinv.astype(np.float64)[None, :]
    wh = w / sinv.astype(np.float64)[:, None]
    ref = x @ w
    assert np.max(np.abs(xh @ wh - ref)) <= 1e-12 * np.max(np.abs(ref))
    # the activation outliers shrink after migration
    assert np.abs(xh).max() < 0.5 * np.abs(x).max()


@pytest.fixture(scope="module")
def tiny_pack():
    spec = synth.layer_spec("tiny")
    lay = synth.gen_layer(spec)
    ax = np.abs(O.bf16_bits_to_f32(lay["x"])).max(axis=0)
    pk = O.pack_weights(lay["w"], ax, spec.rank)
    return spec, lay, ax, pk


def test_svd_eckart_young_against_eigh(tiny_pack):
    spec, lay, ax, pk = tiny_pack
    wh = pk["w_hat"]
    # singular values from a symmetric eigensolver of the Gram matrix
    ev = np.sort(np.linalg.eigvalsh(wh @ wh.T))[::-1]
    sig = np.sqrt(np.maximum(ev, 0))
    r = spec.rank
    l1 = O.bf16_bits_to_f32(pk["l1"]).astype(np.float64)
    l2 = O.bf16_bits_to_f32(pk["l2"]).astype(np.float64)
    low = l1 @ l2
    s_low = np.linalg.eigvalsh(low @ low.T)[::-1][:r]
    assert np.allclose(np.sqrt(np.maximum(s_low, 0)), sig[:r], rtol=2e-3)
    tail = np.sum(sig[r:] ** 2)
    res2 = np.sum((wh - low) ** 2)
    assert abs(res2 - tail) <= 2e-2 * tail
    # L2 rows orthonormal up to bf16 rounding
    assert np.allclose(l2 @ l2.T, np.eye(r), atol=2e-2)


def test_residual_reconstructs(tiny_pack):
    _, _, _, pk = tiny_pack
    l1 = O.bf16_bits_to_f32(pk["l1"]).astype(np.float64)
    l2 = O.bf16_bits_to_f32(pk["l2"]).astype(np.float64)
    recon = l1 @ l2 + pk["r"].astype(np.float64)
    ulp = np.spacing(np.abs(pk["r"]).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(recon - pk["w_hat"]) <= ulp)


def test_full_rank_gives_tiny_residual():
    rng = np.random.default_rng(3)
    w = O.f32_to_bf16_bits((rng.standard_normal((48, 64)) * 0.02).astype(np.float32))
    ax = np.ones(64, dtype=np.float32)
    pk = O.pack_weights(w, ax, 48)
    assert np.linalg.norm(pk["r"]) <= 1e-2 * np.linalg.norm(pk["w_hat"])


# ---------------------------------------------------------------------------
# partials, dequant, whole layer
# ---------------------------------------------------------------------------

def test_group_partials_bruteforce():
    rng = np.random.default_rng(5)
    M, N, K = 5, 7, 192
    qx = rng.integers(-7, 8, (M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, (N, K)).astype(np.int8)
    P = O.group_partials(O.pack_int4(qx), O.pack_int4(qw))
    for m in range(M):
        for n in range(N):
            for g in range(K // 64):
                s = 0
                for k in range(64 * g, 64 * g + 64):
                    s += int(qx[m, k]) * int(qw[n, k])
                assert P[m, n, g] == s
    extreme = np.full((1, 64), 7, dtype=np.int8)
    assert O.group_partials(O.pack_int4(extreme), O.pack_int4(-extreme))[0, 0, 0] == -3136


def test_unit_scales_sum_partials():
    rng = np.random.default_rng(6)
    M, N, K = 8, 16, 256
    qx = O.pack_int4(rng.integers(-7, 8, (M, K)))
    qw = O.pack_int4(rng.integers(-7, 8, (N, K)))
    ones_x = np.ones((K // 64, M), dtype=np.float16)
    ones_w = np.ones((K // 64, N), dtype=np.float16)
    P = O.group_partials(qx, qw)
    acc = O.dequant_accumulate(P, ones_x, ones_w)
    assert np.array_equal(acc, P.sum(axis=2).astype(np.float64))


def _layer(spec):
    lay = synth.gen_layer(spec)
    ax = np.abs(O.bf16_bits_to_f32(lay["x"])).max(axis=0)
    return lay, ax


def test_rank0_is_plain_w4a4():
    spec = synth.custom_spec(32, 256, 64, 0, seed=1)
    lay, ax = _layer(spec)
    pk = O.pack_weights(lay["w"], ax, 0)
    out = O.svdq_linear(lay["x"], pk, lay["bias"])
    # plain W4A4: dequantize both operands elementwise and multiply
    a = O.quantize_act_lora_down(lay["x"], pk["smooth_inv"], pk["l1"])
    qx = O.unpack_int4(a["xq"]).astype(np.float64)
    qw = O.unpack_int4(pk["wq"]).astype(np.float64)
    xd = qx * np.repeat(a["xs"].astype(np.float64).T, 64, axis=1)
    wd = qw * np.repeat(pk["ws"].astype(np.float64).T, 64, axis=1)
    ref = xd @ wd.T + O.bf16_bits_to_f32(lay["bias"]).astype(np.float64)[None, :]
    assert np.allclose(out["y64"], ref, rtol=1e-12, atol=1e-12)
    assert np.all(out["up"] == 0)


def test_dequant_form_matches_per_group():
    spec = synth.custom_spec(40, 320, 96, 16, seed=2)
    lay, ax = _layer(spec)
    pk = O.pack_weights(lay["w"], ax, 16)
    a = O.svdq_linear(lay["x"], pk, lay["bias"], per_group=True)
    b = O.svdq_linear(lay["x"], pk, lay["bias"], per_group=False)
    assert np.allclose(a["y64"], b["y64"], rtol=1e-12, atol=1e-12 * np.abs(a["y64"]).max())


def test_low_rank_branch_reduces_error_on_outliers():
    """Stage 3 of the overview caption: the 16-bit low-rank branch eases the
    4-bit quantization of the migrated weights."""
    spec = synth.layer_spec("tiny")
    lay, ax = _layer(spec)
    ref = O.reference_linear(lay["x"], lay["w"], lay["bias"])
    e0 = O.relative_error(O.svdq_linear(lay["x"], O.pack_weights(lay["w"], ax, 0))["y"], ref)
    er = O.relative_error(O.svdq_linear(lay["x"], O.pack_weights(lay["w"], ax, spec.rank))["y"], ref)
    assert er < e0
    assert er < 0.2


def test_smoothing_helps_w4a4_on_outliers():
    """Stage 2 of the overview caption: migrating outliers from X to W makes
    the activations easier to quantize.  Compare against no migration
    (smooth_inv = 1) at rank 0."""
    spec = synth.layer_spec("tiny")
    lay, ax = _layer(spec)
    ref = O.reference_linear(lay["x"], lay["w"], lay["bias"])
    pk = O.pack_weights(lay["w"], ax, 0)
    e_s = O.relative_error(O.svdq_linear(lay["x"], pk)["y"], ref)
    flat = O.pack_weights(lay["w"], np.full_like(ax, 1.0), 0)
    flat_ones = dict(flat)
    flat_ones["smooth_inv"] = np.ones_like(flat["smooth_inv"])
    w = O.bf16_bits_to_f32(lay["w"]).astype(np.float32)
    q, s = O.quantize_groups(w)
    flat_ones["wq"] = O.pack_int4(q)
    flat_ones["ws"] = np.ascontiguousarray(s.T)
    e_n = O.relative_error(O.svdq_linear(lay["x"], flat_ones)["y"], ref)
    assert e_s < e_n


def test_lora_merge_adds_xab():
    spec = synth.custom_spec(48, 256, 128, 16, seed=4, lora_rank=16)
    lay, ax = _layer(spec)
    a_bits, b_bits = synth.gen_lora(spec)
    pk = O.pack_weights(lay["w"], ax, 16)
    base = O.svdq_linear(lay["x"], pk, lay["bias"])
    l1n, l2n = O.merge_lora(pk["l1"], pk["l2"], pk["smooth_inv"], a_bits, b_bits)
    pk2 = dict(pk, l1=l1n, l2=l2n)
    merged = O.svdq_linear(lay["x"], pk2, lay["bias"])
    x = O.bf16_bits_to_f32(lay["x"]).astype(np.float64)
    xab = x @ O.bf16_bits_to_f32(a_bits).astype(np.float64) @ O.bf16_bits_to_f32(b_bits).astype(np.float64)
    d = merged["y64"] - base["y64"]
    assert np.max(np.abs(d - xab)) <= 2e-2 * np.max(np.abs(xab))
    # the 4-bit residual is untouched
    assert np.array_equal(pk2["wq"], pk["wq"]) and np.array_equal(pk2["ws"], pk["ws"])


# ---------------------------------------------------------------------------
# MXFP4 rules
# ---------------------------------------------------------------------------

def test_mx_decode_table():
    g = _golden("mxfp4_blocks.json")
    codes = np.arange(16, dtype=np.uint8).reshape(1, 16)
    codes = np.concatenate([codes, np.zeros((1, 16), np.uint8)], axis=1)
    dec = O.mx_decode(codes, np.array([[127]], np.uint8))
    assert list(dec[0, :16]) == g["decode_table"]
    dec2 = O.mx_decode(codes, np.array([[130]], np.uint8))
    assert list(dec2[0, :16]) == [8 * v for v in g["decode_table"]]


def test_mx_ties_golden():
    g = _golden("mxfp4_blocks.json")["ties"]
    for v, c in zip(g["values"], g["codes"]):
        blk = np.zeros((1, 32), np.float32)
        blk[0, 0] = 6.0
        blk[0, 1] = v
        codes, sb = O.mx_quantize_blocks(blk)
        assert sb[0, 0] == 127 and codes[0, 1] == c, v


@pytest.mark.parametrize("case", _golden("mxfp4_blocks.json")["cases"], ids=lambda c: c["name"])
def test_mx_blocks_golden(case):
    v = _group_from(case, 32)
    codes, sb = O.mx_quantize_blocks(v[None, :])
    assert int(sb[0, 0]) == case["scale_byte"]
    want = np.zeros(32, np.uint8)
    for k, c in case["codes"].items():
        want[int(k)] = c
    assert np.array_equal(codes[0], want)


def test_mx_power_of_two_grid_lossless():
    rng = np.random.default_rng(21)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for e in range(-20, 20, 3):
        mags = grid[rng.integers(0, 8, (3, 32))]
        mags[:, 0] = 6.0
        vals = mags * np.where(rng.random((3, 32)) < 0.5, -1, 1) * 2.0 ** e
        codes, sb = O.mx_quantize_blocks(vals.astype(np.float32))
        assert np.all(sb == e + 127)
        assert np.array_equal(O.mx_decode(codes, sb), vals)


# ---------------------------------------------------------------------------
# GELU of the MLP pair
# ---------------------------------------------------------------------------

def test_gelu_tanh_form():
    """The logistic evaluation is the tanh form: against math.tanh where the
    tanh form has no cancellation, odd part y, limits, and the tail that the
    tanh form loses to cancellation."""
    import math
    ys = np.linspace(-6.0, 8.0, 561)
    want = [0.5 * y * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (y + 0.044715 * y ** 3))) for y in ys]
    got = O.gelu_tanh(ys)
    big = np.abs(ys) < 3.0
    assert np.allclose(got[big], np.array(want)[big], rtol=1e-13, atol=1e-15)
    # gelu(y) - gelu(-y) = y (the odd part of 0.5 y tanh(u) vanishes)
    assert np.allclose(O.gelu_tanh(ys) - O.gelu_tanh(-ys), ys, rtol=1e-13, atol=1e-13)
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert O.gelu_tanh(np.array([50.0]))[0] == 50.0
    t = O.gelu_tanh(np.array([-10.0, -1e4]))
    assert t[0] < 0 and t[0] > -1e-30          # tiny, not rounded to 0 by cancellation
    assert t[1] == 0.0 and np.signbit(t[1])    # exp overflow: -0


# ---------------------------------------------------------------------------
# smoothing of the activations: one rounding to fp32, then one to bf16 (R7)
# ---------------------------------------------------------------------------

def _bf16r(x: Fraction) -> Fraction:
    return round_to_format(x, 8, -126)


def _double_rounding_pairs(n_want=24, seed=31):
    """(x, s) pairs, x bf16 and s fp32, whose exact product rounds to a
    different bf16 value directly than through fp32: the fp32 rounding lands
    on a bf16 halfway point.  Found by a seeded search over products that
    are exact in fp64 (8 x 24 significant bits)."""
    rng = np.random.default_rng(seed)
    found = []
    while len(found) < n_want:
        x = O.bf16_bits_to_f32(rng.integers(0x3C00, 0x4300, 1 << 16).astype(np.uint16))
        s = (1.0 + rng.random(1 << 16)).astype(np.float32)
        p = x.astype(np.float64) * s.astype(np.float64)      # exact
        p32 = p.astype(np.float32).view(np.uint32)
        tie = (p32 & 0xFFFF) == 0x8000                        # fp32 value is a bf16 halfway point
        for i in np.nonzero(tie)[0]:
            exact = Fraction(float(x[i])) * Fraction(float(s[i]))
            if _bf16r(exact) != _bf16r(f32r(exact)):
                found.append((np.float32(x[i]), np.float32(s[i])))
    return found[:n_want]


def test_smooth_act_rounds_through_fp32_then_bf16():
    """x^ = bf16(fp32(x * smooth_inv)): checked in exact rationals on products
    where rounding straight from the exact (or fp64) product, or skipping
    the bf16 step, gives a different value."""
    pairs = _double_rounding_pairs()
    x = np.array([p[0] for p in pairs], np.float32)
    s = np.array([p[1] for p in pairs], np.float32)
    # one row per pair, smooth_inv per column: put pair i on the diagonal
    n = len(pairs)
    xb = np.zeros((n, n), np.uint16)
    xb[np.arange(n), np.arange(n)] = O.f32_to_bf16_bits(x)
    got = O.smooth_act(xb, s)
    for i in range(n):
        exact = Fraction(float(x[i])) * Fraction(float(s[i]))
        want = _bf16r(f32r(exact))
        assert Fraction(float(O.bf16_bits_to_f32(got[i:i + 1, i])[0])) == want
        assert want != _bf16r(exact)          # the single rounding would differ
        assert want != f32r(exact)            # and the unrounded fp32 value too
    # off-diagonal zeros stay zero
    off = got.copy()
    off[np.arange(n), np.arange(n)] = 0
    assert not off.any()


def test_smooth_act_random_against_rationals():
    rng = np.random.default_rng(32)
    xb = rng.integers(0, 0x7F00, (6, 40)).astype(np.uint16) | (rng.integers(0, 2, (6, 40)) << 15).astype(np.uint16)
    s = (rng.standard_normal(40) * np.exp2(rng.integers(-8, 8, 40))).astype(np.float32)
    got = O.smooth_act(xb, s)
    xf = O.bf16_bits_to_f32(xb)
    for m in range(6):
        for k in range(40):
            want = _bf16r(f32r(Fraction(float(xf[m, k])) * Fraction(float(s[k]))))
            assert Fraction(float(O.bf16_bits_to_f32(got[m:m + 1, k])[0])) == want


# ---------------------------------------------------------------------------
# MXFP4: several blocks of one row with their own scales
# ---------------------------------------------------------------------------

def test_mx_decode_multi_block_row():
    """A row of 4 blocks with scale bytes 127, 120, 133, 0: each element is
    sign * grid[code & 7] * 2^(byte - 127) of its own block (hand sum)."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    rng = np.random.default_rng(41)
    codes = rng.integers(0, 16, (2, 128)).astype(np.uint8)
    sb = np.array([[127, 120, 133, 0], [1, 254, 126, 128]], np.uint8)
    dec = O.mx_decode(codes, sb)
    for r in range(2):
        for k in range(128):
            c = int(codes[r, k])
            want = (-1.0 if c & 8 else 1.0) * grid[c & 7] * 2.0 ** (int(sb[r, k // 32]) - 127)
            assert dec[r, k] == want, (r, k)


def test_mx_gemm_multi_block_hand_sum():
    """mx_gemm_lora_up on rows with distinct per-block scales against an
    explicit double loop over k with each element decoded by hand."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    rng = np.random.default_rng(42)
    M, N, K = 3, 4, 128
    cx = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cw = rng.integers(0, 16, (N, K)).astype(np.uint8)
    bx = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    bw = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    out = O.mx_gemm_lora_up(pack(cx), np.ascontiguousarray(bx.T), pack(cw), np.ascontiguousarray(bw.T),
                            np.zeros((M, 0)), np.zeros((0, N), np.uint16), None)

    def dec(c, b):
        return (-1.0 if c & 8 else 1.0) * grid[c & 7] * 2.0 ** (int(b) - 127)

    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(dec(int(cx[m, k]), bx[m, k // 32])) * Fraction(dec(int(cw[n, k]), bw[n, k // 32]))
            assert out["y64"][m, n] == float(s)      # exact: dyadic values well inside fp64
            assert out["y"][m, n] == O.f32_to_bf16_bits(np.array([float(s)], np.float32))[0]


# ---------------------------------------------------------------------------
# R8 (the up projection reads bf16(t)) and R9 (one rounding of acc + up + b)
# ---------------------------------------------------------------------------

def _one_code_group(q_x, q_w, s_x, s_w):
    """One token, one channel, K = 64: a single non-zero code pair at k 0."""
    qx = np.zeros((1, 64), np.int8)
    qw = np.zeros((1, 64), np.int8)
    qx[0, 0], qw[0, 0] = q_x, q_w
    xs = np.array([[s_x]], np.float16)
    ws = np.array([[s_w]], np.float16)
    return O.pack_int4(qx), xs, O.pack_int4(qw), ws


def test_up_projection_uses_bf16_of_t():
    """acc = 1 * 1 * 2^-4 * 2^-4 = 2^-8; t = 1 + 2^-10 is not a bf16 value
    and rounds to 1; L2 = 1.  With bf16(t): y = 1 + 2^-8, a bf16 halfway
    point, which rounds to the even 1.0 (0x3F80).  With t unrounded the sum
    is above the halfway point and would give 1 + 2^-7 (0x3F81)."""
    xq, xs, wq, ws = _one_code_group(1, 1, 2.0 ** -4, 2.0 ** -4)
    t = np.array([[1.0 + 2.0 ** -10]])
    l2 = O.f32_to_bf16_bits(np.array([[1.0]], np.float32))
    out = O.gemm_w4a4_lora_up(xq, xs, wq, ws, t, l2, None)
    assert out["acc"][0, 0] == 2.0 ** -8
    assert out["up"][0, 0] == 1.0
    assert int(out["y"][0, 0]) == 0x3F80


def test_output_rounded_once_after_bias():
    """acc = 2^-8 (one code pair, scales 2^-4), up = 1 (t = 1, L2 = 1),
    bias = 2^-12: the exact sum 1 + 2^-8 + 2^-12 lies above the bf16
    halfway point 1 + 2^-8 and rounds up to 1 + 2^-7 (0x3F81).  Rounding
    acc + up first (to the even 1.0) and then adding the bias would give
    0x3F80."""
    xq, xs, wq, ws = _one_code_group(1, 1, 2.0 ** -4, 2.0 ** -4)
    t = np.array([[1.0]])
    l2 = O.f32_to_bf16_bits(np.array([[1.0]], np.float32))
    bias = O.f32_to_bf16_bits(np.array([2.0 ** -12], np.float32))
    out = O.gemm_w4a4_lora_up(xq, xs, wq, ws, t, l2, bias)
    assert out["y64"][0, 0] == 1.0 + 2.0 ** -8 + 2.0 ** -12
    assert int(out["y"][0, 0]) == 0x3F81
    # the per-group partial times both scales, by hand: 1 * 2^-4 * 2^-4
    assert out["P"][0, 0, 0] == 1 and out["acc"][0, 0] == 2.0 ** -8

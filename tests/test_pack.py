"""The library's offline pack (C++) against the oracle.

What is unique is compared exactly: smooth_inv, and at rank 0 (no SVD) the
packed codes and scales.  With a low-rank branch the SVD factors are not
unique, so the product L1 L2 is checked through its singular values and the
residual norm, and the rest through invariants (L1 L2 + R = W^, the codes
are a valid 4-bit quantization of R)."""

import numpy as np
import pytest

import bit_quantized_diffusion_amd as bq
import oracle as O
import synth


def _absmax(x_bits):
    return np.abs(O.bf16_bits_to_f32(x_bits)).max(axis=0).astype(np.float32)


def _layer(spec):
    lay = synth.gen_layer(spec)
    return lay, _absmax(lay["x"])


@pytest.mark.parametrize("spec", [
    synth.layer_spec("tiny"),
    synth.custom_spec(64, 448, 200, 0, seed=3),
    synth.custom_spec(64, 1024, 96, 0, seed=4),
], ids=lambda s: s.name)
def test_rank0_pack_bit_exact(spec):
    lay, ax = _layer(spec)
    ref = O.pack_weights(lay["w"], ax, 0)
    got = bq.pack_weights(lay["w"], ax, 0, want_residual=True)
    assert np.array_equal(got["smooth_inv"].view(np.uint32), ref["smooth_inv"].view(np.uint32))
    assert np.array_equal(got["r"].view(np.uint32), ref["r"].view(np.uint32))
    assert np.array_equal(got["wq"], ref["wq"])
    assert np.array_equal(got["ws"].view(np.uint16), ref["ws"].view(np.uint16))


def test_rank0_mxfp4_pack_bit_exact():
    spec = synth.custom_spec(64, 512, 160, 0, seed=5)
    lay, ax = _layer(spec)
    ref = O.mx_pack_weights(lay["w"], ax, 0)
    got = bq.pack_weights(lay["w"], ax, 0, precision=bq.MXFP4)
    assert np.array_equal(got["wq"], ref["wq"])
    assert np.array_equal(got["ws"], ref["ws"])


def _check_low_rank(spec, lay, ax, got, ref, tol_sig=2e-3, tol_res=1e-3):
    r = spec.rank
    # smoothing is exact
    assert np.array_equal(got["smooth_inv"].view(np.uint32), ref["smooth_inv"].view(np.uint32))
    l1 = O.bf16_bits_to_f32(got["lora_down"]).astype(np.float64).T      # K x r
    l2 = O.bf16_bits_to_f32(got["lora_up"]).astype(np.float64).T        # r x N
    low = l1 @ l2
    wh = ref["w_hat"]
    # singular values of the library's low-rank product match the top-r of W^
    s_low = np.linalg.svd(low, compute_uv=False)[:r]
    assert np.allclose(s_low, ref["sigma"][:r], rtol=tol_sig)
    # Eckart-Young: the residual is as small as the oracle's
    res_lib = np.linalg.norm(wh - low)
    res_ref = np.linalg.norm(ref["r"].astype(np.float64))
    assert abs(res_lib - res_ref) <= tol_res * res_ref
    # L1 L2 + R = W^ to fp32 rounding of R
    R = got["r"].astype(np.float64)
    ulp = np.spacing(np.abs(got["r"])).astype(np.float64)
    assert np.all(np.abs(low + R - wh) <= ulp)
    # rows of L2 are orthonormal up to bf16 rounding
    assert np.allclose(l2 @ l2.T, np.eye(r), atol=2e-2)
    # the codes are a valid 4-bit quantization of R: |R - s q| <= s/2 for
    # normal fp16 scales, and s is amax/7 rounded to fp16
    K, N = R.shape
    q = O.unpack_int4(got["wq"]).astype(np.float64)                     # N x K
    s = got["ws"].astype(np.float64)                                     # G x N
    sfull = np.repeat(s.T, 64, axis=1)                                   # N x K
    err = np.abs(R.T - q * sfull)
    normal = sfull >= 2.0 ** -14
    assert np.all(err[normal] <= 0.5 * sfull[normal] * (1 + 2e-3))
    amax = np.abs(R.T.reshape(N, K // 64, 64)).max(axis=2)
    assert np.allclose(s.T, amax / 7, rtol=2.0 ** -10, atol=2.0 ** -24)


@pytest.mark.parametrize("spec", [
    synth.layer_spec("tiny"),                                   # K <= N: Gram over K
    synth.custom_spec(96, 512, 128, 16, seed=6),                # K > N: Gram over N
    synth.custom_spec(96, 256, 320, 48, seed=7),                # rank 48
], ids=lambda s: s.name)
def test_low_rank_pack_against_oracle(spec):
    lay, ax = _layer(spec)
    ref = O.pack_weights(lay["w"], ax, spec.rank)
    got = bq.pack_weights(lay["w"], ax, spec.rank, want_residual=True)
    _check_low_rank(spec, lay, ax, got, ref)


def test_full_rank_pack_reconstructs():
    spec = synth.custom_spec(32, 128, 64, 64, seed=8)
    lay, ax = _layer(spec)
    got = bq.pack_weights(lay["w"], ax, 64, want_residual=True)
    ref = O.pack_weights(lay["w"], ax, 64)
    assert np.linalg.norm(got["r"]) <= 1e-2 * np.linalg.norm(ref["w_hat"])


def test_pack_is_deterministic():
    spec = synth.custom_spec(32, 256, 128, 32, seed=9)
    lay, ax = _layer(spec)
    a = bq.pack_weights(lay["w"], ax, 32)
    b = bq.pack_weights(lay["w"], ax, 32)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


# ---------------------------------------------------------------------------
# LoRA merge (host entry point) against the oracle's merge
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rank,lora_rank", [(16, 16), (0, 16), (32, 32)])
def test_merge_lora_bit_exact(rank, lora_rank):
    """Same concatenation and the same fp64 fold with 1/smooth_inv, rounded
    once to fp32 then to bf16: bit for bit the oracle's merge."""
    spec = synth.custom_spec(40, 256, 96, rank, seed=7, lora_rank=lora_rank)
    lay, ax = _layer(spec)
    pk = bq.pack_weights(lay["w"], ax, rank)
    a_bits, b_bits = synth.gen_lora(spec)
    down, up = bq.merge_lora(pk["lora_down"] if rank else None, pk["lora_up"] if rank else None,
                             pk["smooth_inv"], a_bits, b_bits)
    l1 = np.ascontiguousarray(pk["lora_down"].T) if rank else np.zeros((spec.K, 0), np.uint16)
    l2 = np.ascontiguousarray(pk["lora_up"].T) if rank else np.zeros((0, spec.N), np.uint16)
    l1n, l2n = O.merge_lora(l1, l2, pk["smooth_inv"], a_bits, b_bits)
    assert down.shape == (rank + lora_rank, spec.K) and up.shape == (spec.N, rank + lora_rank)
    assert np.array_equal(down, np.ascontiguousarray(l1n.T))
    assert np.array_equal(up, np.ascontiguousarray(l2n.T))


def test_merge_lora_adds_the_adapter():
    """The merged branch adds X A B (up to the bf16 roundings of the fold):
    X^ L1' L2' - X^ L1 L2 = X A B."""
    spec = synth.custom_spec(32, 256, 64, 16, seed=8, lora_rank=16)
    lay, ax = _layer(spec)
    pk = bq.pack_weights(lay["w"], ax, 16)
    a_bits, b_bits = synth.gen_lora(spec)
    down, up = bq.merge_lora(pk["lora_down"], pk["lora_up"], pk["smooth_inv"], a_bits, b_bits)
    x = O.bf16_bits_to_f32(lay["x"]).astype(np.float64)
    xh = x * pk["smooth_inv"].astype(np.float64)[None, :]
    f = lambda t: O.bf16_bits_to_f32(t).astype(np.float64)
    delta = xh @ f(down.T) @ f(up.T) - xh @ f(pk["lora_down"].T) @ f(pk["lora_up"].T)
    want = x @ f(a_bits) @ f(b_bits)
    assert np.max(np.abs(delta - want)) <= 1e-2 * np.max(np.abs(want))


def test_merge_lora_rejects_bad_arguments():
    K, N = 128, 64
    sinv = np.ones(K, np.float32)
    a = np.zeros((K, 8), np.uint16)
    b = np.zeros((8, N), np.uint16)
    with pytest.raises(bq.SvdqError) as e:        # merged rank 8 is not a multiple of 16
        bq.merge_lora(None, None, sinv, a, b)
    assert e.value.status == bq.SVDQ_ERR_SHAPE
    st = bq.lib.svdq_merge_lora(None, None, 0, None, None, None, 16, K, N, None, None)
    assert st == bq.SVDQ_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# The library's pack at the FLUX MLP sizes (slow: about a minute of CPU per
# case; run with SVDQ_RUN_SLOW=1).  X only supplies the per-channel absmax,
# so a few hundred rows of the layer's distribution stand in for it (fc2's
# own X would be fc1's GELU output).  The singular values are those of the
# bf16 factors: each factor is rounded to bf16 (relative 2^-9 per element),
# which moves a singular value of the product by up to about 2 * 2^-9 of it
# -- the oracle's own bf16 factors sit 2.2e-3 off the exact values at fc1 --
# so against the exact SVD the bound is 2^-8, and against the oracle's bf16
# factors (the same roundings of nearly the same subspace) 1e-4.
# ---------------------------------------------------------------------------

@pytest.mark.slow
@pytest.mark.parametrize("name", ["fc1", "fc2"])
def test_pack_flux_mlp_size(name):
    spec = synth.layer_spec(name, M=256, x_from_prev=False)
    lay, ax = _layer(spec)
    ref = O.pack_weights(lay["w"], ax, spec.rank)
    got = bq.pack_weights(lay["w"], ax, spec.rank, want_residual=True)
    _check_low_rank(spec, lay, ax, got, ref, tol_sig=2.0 ** -8)
    r = spec.rank
    low_lib = O.bf16_bits_to_f32(got["lora_down"]).astype(np.float64).T @ \
        O.bf16_bits_to_f32(got["lora_up"]).astype(np.float64).T
    low_ref = O.bf16_bits_to_f32(ref["l1"]).astype(np.float64) @ O.bf16_bits_to_f32(ref["l2"]).astype(np.float64)
    s_lib = np.linalg.svd(low_lib, compute_uv=False)[:r]
    s_ref = np.linalg.svd(low_ref, compute_uv=False)[:r]
    assert np.allclose(s_lib, s_ref, rtol=1e-4)

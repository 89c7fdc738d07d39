// HIP kernels of the SVDQuant W4A4 linear layer for gfx950 (MI355X).
//
// Kernel 1 (quantize + down projection) and kernel 2 (4-bit GEMM + up
// projection) are the two fusions of the Nunchaku engine figure, caption
// (b), on the "svdq-int4-flux.1-dev" model card: the down projection and
// the quantizer share their input X, the up projection and the 4-bit compute
// share their output Y.
//
// Layout conventions are those of include/svdq.h.  Matrix-core layouts used
// here (CDNA3/CDNA4 16x16 MFMA family, wave64):
//   A operand  lane l holds row (l % 16) and a lane-group (l / 16) slice of K,
//   B operand  lane l holds column (l % 16) and the same K slice,
//   D result   lane l, element i holds row 4*(l/16)+i, column l % 16.
// Which k inside the slice an element stands for does not matter as long as
// A and B are filled the same way, which every kernel here does.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "svdq_internal.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// number formats on the device
// ---------------------------------------------------------------------------

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// two fp32 -> packed bf16 pair (lo, hi), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const v2bf b = __builtin_convertvector((v2f{lo, hi}), v2bf);
  return __builtin_bit_cast(uint32_t, b);
}

// fp32 -> fp16 bits with round to nearest even; finite values saturate to
// 65504; subnormal results are kept (fp16 denormals are not flushed).
__device__ __forceinline__ uint32_t f16_sat_bits(float f) {
  const _Float16 h = static_cast<_Float16>(f);
  uint32_t b = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
  if ((b & 0x7FFFu) == 0x7C00u && __builtin_isfinite(f)) b = (b & 0x8000u) | 0x7BFFu;
  return b;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// fp32 -> packed bf16 pair with round to nearest even
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) { return cvt_pk_bf16(lo, hi); }

// ---------------------------------------------------------------------------
// Kernel 1: smoothing + INT4 activation quantization + down projection.
//
// A workgroup of 4 waves owns 64 rows (16 per wave: one row tile of the
// down projection's 16x16 MFMA) and one slice of K (a multiple of 128 k;
// blockIdx.y).  A wave step covers its 16 rows x 128 k: lane l owns row
// l % 16 and the 32 contiguous k at (l/16)*32, half of one group, read as 4
// chunks of 8 k.  The group absmax needs one lane exchange (the other half
// is 16 lanes away), and the lane's 32 codes leave as one 16-byte store.
// X^ is rounded to bf16 by v_cvt_pk_bf16_f32; chunk c of the 4 lanes of a
// row is the A operand of one bf16 MFMA with L1 (K = 32: k at q*32 + c*8 +
// 0..7 for lane group q; the L1 fragment is loaded with the same k), so X is
// read once.  The four waves of a workgroup read the same L1 fragments, so
// the L1 (lora_down) traffic to L2 is that of 64 rows, not 16.
//
// With more than one K slice, each workgroup adds its 64 x rank partial
// X^ L1 into lora_act with fp32 atomics (lora_act is cleared first by a
// small fill kernel); the order of those additions is not fixed, so
// lora_act can differ in its last bits between runs.  With one slice the
// partial is stored directly.
//
// The kernel is bound by HBM reads of X, so every load is unconditional
// (row and k clamped into the matrix; data of a clamped chunk is zeroed
// before use, stores are predicated) and the X of a wave's next step is
// requested before the current step is processed.
// ---------------------------------------------------------------------------

constexpr int kK1Rows = 64;       // rows per workgroup (4 waves x 16)

// Quantizer of kernel 1 (QMODE): kQuantNone = down projection only (the
// unfused baseline's second kernel), kQuantInt4 = INT4 groups of 64 with fp16
// scales, kQuantMx = MXFP4 blocks of 32 with E8M0 scales.
constexpr int kQuantNone = 0, kQuantInt4 = 1, kQuantMx = 2;

// Bits of 2^e as fp32 for e in [-127, 127] (2^-127 is a subnormal).
__device__ __forceinline__ float exp2i_f32(int e) {
  return e >= -126 ? __uint_as_float(static_cast<uint32_t>(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// ---------------------------------------------------------------------------
// INT4 code layout (shared by kernel 1, the fused MLP tail and the GEMMs).
//
// A unit of 16 consecutive k is two little-endian words I0, I1.  Code q has
// the 6-bit image 32 [q < 0] + |q|, which is the FP6 E2M3 pattern of q/8
// (bits 3-4, the exponent, are zero: a subnormal); image j of the unit sits
// at bits 6j..6j+5 of the 96-bit string D0 | D1 << 32 | D2 << 64, the
// layout in which the matrix core reads 16 FP6 values from three VGPRs.
// Stored: I0 = D0 | (D2 & kZ0), I1 = D1 | (D2 & kZ1) -- the masks are the
// zero exponent bits of the images in D0 and D1, which together are exactly
// the data bits of D2 -- so the matrix-core words come back with four
// operations per unit: D0 = I0 & ~kZ0, D1 = I1 & ~kZ1,
// D2 = (I0 & kZ0) | (I1 & kZ1).
// ---------------------------------------------------------------------------
constexpr uint32_t kZ0 = 0x18618618u;     // bits 3,4 9,10 15,16 21,22 27,28
constexpr uint32_t kZ1 = 0x86186186u;     // bits 1,2 7,8 13,14 19,20 25,26 31

typedef __bf16 v32bf __attribute__((ext_vector_type(32)));
typedef unsigned v6u __attribute__((ext_vector_type(6)));
typedef float v32f __attribute__((ext_vector_type(32)));

// 32 values (x[c][e] = value 8c + e) -> their INT4 codes in the code layout,
// q = clamp(rint(fp32(x * inv)), -7, 7) with ties to even, as 16 bytes (two
// units).  invs = inv / 8 (exact), so v = x * invs is fp32(x * inv) / 8 and
// (v + 1.5 * 2^20) - 1.5 * 2^20 rounds it to the 1/8 grid with ties to even
// -- q/8 -- and gives +0 for a negative value that rounds to zero; clamped
// to +-7/8 it is exact in bf16, and v_cvt_scalef32_pk32_fp6_bf16 (scale 1)
// writes the 32 values as FP6 images in order, D0..D5.
__device__ __forceinline__ uint4 pack_codes_fp6(const float (&x)[4][8], float invs) {
#pragma clang fp contract(off)
  constexpr float kMagic = 1572864.0f;           // 1.5 * 2^20: ulp 1/8 on [2^20, 2^21)
  v32bf h;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float r0 = (x[c][e] * invs + kMagic) - kMagic;
      float r1 = (x[c][e + 1] * invs + kMagic) - kMagic;
      r0 = __builtin_amdgcn_fmed3f(r0, -0.875f, 0.875f);
      r1 = __builtin_amdgcn_fmed3f(r1, -0.875f, 0.875f);
      const v2bf b = __builtin_convertvector((v2f{r0, r1}), v2bf);
      h[8 * c + e] = b[0];
      h[8 * c + e + 1] = b[1];
    }
  const v6u d = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(h, 1.0f);
  return make_uint4(d[0] | (d[2] & kZ0), d[1] | (d[2] & kZ1), d[3] | (d[5] & kZ0), d[4] | (d[5] & kZ1));
}

// Ranks up to 48 are held to four workgroups per CU (at most 128 VGPRs,
// four waves per SIMD): unbounded, the compiler took 136 VGPRs at rank 32,
// three waves per SIMD, and the launch slots fell under the ~1024-workgroup
// grid (bounded: FLUX fc1 17.3 -> 15.9 us, fc2 45 -> 43 us, no spill).
// Larger ranks would spill under that bound and keep the compiler's choice.
template <int RT, bool ATOMIC, int QMODE = kQuantInt4>
__global__ __launch_bounds__(256, (RT <= 3 ? 4 : 1)) void k1_quant_down_int4(
    const uint16_t* __restrict__ x, int M, int K, const float* __restrict__ sinv,
    const uint16_t* __restrict__ ldown, uint8_t* __restrict__ xq, void* __restrict__ xs_,
    float* __restrict__ lact, int ks) {
  constexpr int RANK = RT * 16;
  constexpr int TB = RT < 2 ? (RT > 0 ? RT : 1) : 2;    // L1 fragments per batch of loads (ranks of 16)
  // ranks up to 64: the step's L1 slice [RANK][128 k] is loaded once per
  // workgroup into a two-slot LDS ring and shared by the 4 waves (one
  // barrier per step); larger ranks load their fragments per wave
  constexpr bool L1S = RT > 0 && RT <= 4;
  constexpr int kL1Row = 128 + 8;                       // bf16 elements per L1 row in LDS (16 bytes padding)
  constexpr int kL1Chunks = L1S ? RANK * 16 / 256 : 1;  // 16-byte chunks per thread and step (1..4)
  extern __shared__ float lds_sinv[];                   // smooth_inv of this workgroup's K slice
  __shared__ __attribute__((aligned(16))) uint16_t lds_l1[L1S ? 2 : 1][L1S ? RANK : 1][kL1Row];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int row0 = blockIdx.x * kK1Rows + wave * 16;
  const int row = row0 + r16;
  const bool row_ok = row < M;
  const int k_begin = blockIdx.y * ks;
  const int k_end = min(K, k_begin + ks);
  const size_t xrow = static_cast<size_t>(row) * K;
  const uint16_t* xr = x + static_cast<size_t>(min(row, M - 1)) * K;
  // k of chunk c of the step at kbase for this lane, clamped into the row
  auto kof = [&](int kbase, int c) { return min(kbase + q * 32 + c * 8, K - 8); };

  v4f acc[RT > 0 ? RT : 1];
#pragma unroll
  for (int t = 0; t < (RT > 0 ? RT : 1); ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  // the first step's X is requested before the LDS staging below, so that
  // its latency overlaps that of the staging loads and barriers
  uint4 xn[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) xn[c] = *reinterpret_cast<const uint4*>(xr + kof(k_begin, c));

  // smooth_inv is read by every step of every wave: stage the slice in LDS
  for (int i = threadIdx.x; i < (k_end - k_begin) / 4; i += blockDim.x)
    reinterpret_cast<float4*>(lds_sinv)[i] = reinterpret_cast<const float4*>(sinv + k_begin)[i];
  __syncthreads();
  // LDS copy of smooth_inv at k (k inside the slice; clamped k of the last
  // chunk can fall 8 below the slice start only when the slice is the
  // whole, shorter-than-128 row, and then it is still inside the slice)
  auto sv = [&](int k) { return lds_sinv + (k - k_begin); };

  // L1 slice of the step at kbase: chunk id = threadIdx.x + 256 i is row
  // id/16, k kbase + 8 (id%16) (clamped into the row)
  struct L1Regs {
    uint4 v0, v1, v2, v3;
  };
  auto l1_chunk = [&](int kbase, int i) {
    const int id = static_cast<int>(threadIdx.x) + 256 * i;
    return *reinterpret_cast<const uint4*>(ldown + static_cast<size_t>(id >> 4) * K + min(kbase + 8 * (id & 15), K - 8));
  };
  auto l1_gload = [&](int kbase) {
    L1Regs L;
    L.v0 = l1_chunk(kbase, 0);
    if constexpr (kL1Chunks > 1) L.v1 = l1_chunk(kbase, 1);
    if constexpr (kL1Chunks > 2) L.v2 = l1_chunk(kbase, 2);
    if constexpr (kL1Chunks > 3) L.v3 = l1_chunk(kbase, 3);
    return L;
  };
  auto l1_put = [&](int slot, int i, const uint4& v) {
    const int id = static_cast<int>(threadIdx.x) + 256 * i;
    *reinterpret_cast<uint4*>(&lds_l1[slot][id >> 4][8 * (id & 15)]) = v;
  };
  auto l1_lstore = [&](int slot, L1Regs L) {
    l1_put(slot, 0, L.v0);
    if constexpr (kL1Chunks > 1) l1_put(slot, 1, L.v1);
    if constexpr (kL1Chunks > 2) l1_put(slot, 2, L.v2);
    if constexpr (kL1Chunks > 3) l1_put(slot, 3, L.v3);
  };
  L1Regs l1n;
  if constexpr (L1S) {
    l1n = l1_gload(k_begin);
    l1_lstore(0, l1n);
    __syncthreads();
  }

  auto load_l1 = [&](v4i (&dst)[4][TB], int kbase, int t0) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < TB; ++t)
        if (t0 + t < RT)
          dst[c][t] = *reinterpret_cast<const v4i*>(ldown + static_cast<size_t>((t0 + t) * 16 + r16) * K + kof(kbase, c));
  };

  int slot = 0;
  for (int kbase = k_begin; kbase < k_end; kbase += 128, slot ^= 1) {
    uint4 xc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) xc[c] = xn[c];
    // L1 of this step (per wave) or of the next step (shared), issued
    // before the next step's X so that waiting for them (in order) does not
    // also wait for the X prefetch
    v4i lb[4][TB];
    const bool more = kbase + 128 < k_end;
    if constexpr (L1S) {
      if (more) l1n = l1_gload(kbase + 128);
    } else if constexpr (RT > 0) {
      load_l1(lb, kbase, 0);
    }
    {
      const int nxt = kbase + 128 < k_end ? kbase + 128 : kbase;   // the last step re-reads itself (unused)
#pragma unroll
      for (int c = 0; c < 4; ++c) xn[c] = *reinterpret_cast<const uint4*>(xr + kof(nxt, c));
    }
    // lane (row, q) holds the 32 k at kbase + q*32: half of group
    // kbase/64 + q/2, whose other half sits in lane q^1 (16 lanes away)
    const bool valid = kbase + q * 32 < k_end;         // false only in a slice's odd last group
    float4 s0[4], s1[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = valid ? kbase + q * 32 + c * 8 : k_begin;
      s0[c] = *reinterpret_cast<const float4*>(sv(k));
      s1[c] = *reinterpret_cast<const float4*>(sv(k) + 4);
    }

    // lanes past the slice's end compute on in-bounds data and zero it
    // with a mask (a select would become a branch per element)
    uint32_t vmask = valid ? 0xFFFFFFFFu : 0u;
    asm volatile("" : "+v"(vmask));
    float xh[4][8];
    uint32_t pk[4][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t ws[4] = {xc[c].x, xc[c].y, xc[c].z, xc[c].w};
      const float ss[8] = {s0[c].x, s0[c].y, s0[c].z, s0[c].w, s1[c].x, s1[c].y, s1[c].z, s1[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(ws[e] << 16) * ss[2 * e];
        const float hi = __uint_as_float(ws[e] & 0xFFFF0000u) * ss[2 * e + 1];
        const uint32_t p = cvt_pk_bf16(lo, hi) & vmask;
        pk[c][e] = p;
        xh[c][2 * e] = __uint_as_float(p << 16);
        xh[c][2 * e + 1] = __uint_as_float(p & 0xFFFF0000u);
      }
    }

    if constexpr (QMODE == kQuantInt4) {
      uint16_t* xs = static_cast<uint16_t*>(xs_);
      const int g = kbase / 64 + (q >> 1);
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(xh[c][e]));
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      const uint32_t sbits = f16_sat_bits(__fdiv_rn(amax, 7.0f));
      const float s = f16_bits_to_f32(sbits);
      const float inv = (s == 0.f) ? 0.f : __fdiv_rn(1.0f, s);
      // the lane's 32 codes are 16 contiguous bytes of the packed row: two
      // units of 16 codes in the layer's code layout (pack_codes_fp6)
      const uint4 packed = pack_codes_fp6(xh, inv * 0.125f);
      if (row_ok && valid) *reinterpret_cast<uint4*>(xq + xrow / 2 + (kbase + q * 32) / 2) = packed;
      if (row_ok && valid && (q & 1) == 0) xs[static_cast<size_t>(g) * M + row] = static_cast<uint16_t>(sbits);
    } else if constexpr (QMODE == kQuantMx) {
      // MXFP4 (OCP MX): the lane's 32 k are one block.  e = floor(log2
      // amax) - 2 from the fp32 exponent field, clamped to [-127, 127];
      // scale byte e + 127 (amax == 0 gives byte 0 and zero codes).  The
      // elements x^ / 2^e are rounded to E2M1 by v_cvt_scalef32_pk_fp4_f32
      // (nearest, ties to the even code, saturating at 6); a value that
      // rounds to zero keeps no sign.  For the two smallest exponents the
      // elements are scaled by 2^64 first so that the scale stays normal.
      uint8_t* xs = static_cast<uint8_t*>(xs_);
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(xh[c][e]));
      int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu) - 127 - 2;
      e = max(-127, min(127, e));
      const bool tiny = e < -125;
      const float pre = tiny ? 18446744073709551616.0f : 1.0f;     // 2^64
      const float scale = exp2i_f32(tiny ? e + 64 : e);
      uint32_t word[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // byte b of the word = codes of k 2b (low nibble) and 2b + 1
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xh[c][0] * pre, xh[c][1] * pre, scale, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xh[c][2] * pre, xh[c][3] * pre, scale, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xh[c][4] * pre, xh[c][5] * pre, scale, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xh[c][6] * pre, xh[c][7] * pre, scale, 3);
        // clear the sign of zero magnitudes: bit 3 of a nibble survives
        // only where its magnitude (bits 0-2) is non-zero
        const uint32_t mag = w & 0x77777777u;
        w = mag | (w & ((mag + 0x77777777u) & 0x88888888u));
        word[c] = w;
      }
      if (row_ok && valid) {
        *reinterpret_cast<uint4*>(xq + xrow / 2 + (kbase + q * 32) / 2) = make_uint4(word[0], word[1], word[2], word[3]);
        xs[static_cast<size_t>(kbase / 32 + q) * M + row] = static_cast<uint8_t>(e + 127);
      }
    }

    if constexpr (L1S) {
      // fragments from the shared slice: L1 row t*16 + r16, k q*32 + c*8
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const v8bf a = __builtin_bit_cast(v8bf, (v4i{static_cast<int>(pk[c][0]), static_cast<int>(pk[c][1]),
                                                     static_cast<int>(pk[c][2]), static_cast<int>(pk[c][3])}));
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const v4i b = *reinterpret_cast<const v4i*>(&lds_l1[slot][t * 16 + r16][q * 32 + c * 8]);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf, b), acc[t], 0, 0, 0);
        }
      }
      if (more) l1_lstore(slot ^ 1, l1n);
      __syncthreads();
    } else if constexpr (RT > 0) {
#pragma unroll
      for (int t0 = 0; t0 < RT; t0 += TB) {
        if (t0 > 0) load_l1(lb, kbase, t0);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const v8bf a = __builtin_bit_cast(v8bf, (v4i{static_cast<int>(pk[c][0]), static_cast<int>(pk[c][1]),
                                                       static_cast<int>(pk[c][2]), static_cast<int>(pk[c][3])}));
#pragma unroll
          for (int t = 0; t < TB; ++t)
            if (t0 + t < RT)    // compile-time after unrolling (odd RT)
              acc[t0 + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf, lb[c][t]),
                                                                    acc[t0 + t], 0, 0, 0);
        }
      }
    }
  }

  if constexpr (RT > 0) {
    // D layout: lane (q, r16), element i -> row 4q + i, column r16 of tile t
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = row0 + 4 * q + i;
        if (rr < M) {
          float* dst = lact + static_cast<size_t>(rr) * RANK + t * 16 + r16;
          if constexpr (ATOMIC)
            atomicAdd(dst, acc[t][i]);
          else
            *dst = acc[t][i];
        }
      }
  }
}

// lora_act cleared before kernel 1's atomic slice sums: 16 bytes per thread
// (n is a multiple of 16 floats: the rank is)
__global__ void fill_zero_f32(float* __restrict__ p, size_t n) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (4 * i < n) reinterpret_cast<float4*>(p)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------------------
// Kernel 2 (both precisions): 4-bit GEMM + dequant + up projection + bias.
//
// Output tile 128 (n) x 128 (m) per workgroup of 4 waves, 64 x 64 per wave
// (2 x 2 MFMA tiles of 32 x 32).  The MFMA computes Y^T tiles (A = W codes,
// B = X codes), so a lane ends up with groups of 4 consecutive output
// channels of one token; the epilogue turns the tile around in LDS so that
// Y is written in 16-byte row segments.
//
// INT4 codes reach the matrix core as FP6 E2M3 values q/8 (the code
// layout is built for that: four operations per 16 codes recover the
// matrix core's words); for one K-group of 64,
// v_mfma_scale_f32_32x32x64_f8f6f4 then returns the group's integer partial
// P / 64 times its two E8M0 block scales, exactly.  MXFP4 codes are the
// matrix core's own FP4.
// ---------------------------------------------------------------------------

constexpr int kTile = 128;      // output tile edge (both n and m)
constexpr unsigned kUnitScales = 0x7F7F7F7Fu;   // E8M0 127 = 1.0 in every byte

// Raw buffer resource over [base, base + bytes) (bytes clamped to 32 bits;
// callers keep every access inside the range).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  const int n = static_cast<int>(bytes > 0xFFFFFFFFull ? 0xFFFFFFFFull : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n, 0x00020000);
}

// chunk swizzle of a 128-byte LDS row: over any 8 consecutive rows
// (r0 = 0 mod 8) the swizzle takes all 8 values, and over any 16 (r0 = 0
// mod 16) r mod 2 and the swizzle take all 16 combinations: the 16-byte
// reads of consecutive rows at one chunk are conflict-free for 32 and for
// 64 four-byte banks.
__device__ __forceinline__ int swz8(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

typedef unsigned v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 buffer_load_u4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
template <int S>
struct Slot {
  static constexpr int value = S;
};

struct TileCoord {
  int n0, m0;
};

// Blocks are dispatched round-robin over the 8 XCDs.  Give every XCD a
// contiguous range of the logical tile order, and walk that order in groups
// of 8 tile-rows so that tiles running together share operand panels in the
// XCD's L2.
__device__ __forceinline__ TileCoord tile_coord(int pid, int tiles_n, int tiles_m) {
  const int total = tiles_n * tiles_m;
  const int q = total / 8, rem = total % 8;
  const int xcd = pid % 8, idx = pid / 8;
  const int logical = xcd * q + min(xcd, rem) + idx;
  constexpr int GROUP = 8;
  const int group_size = GROUP * tiles_m;
  const int gid = logical / group_size;
  const int first_n = gid * GROUP;
  const int gn = min(tiles_n - first_n, GROUP);
  const int within = logical - gid * group_size;
  TileCoord tc;
  tc.n0 = (first_n + within % gn) * kTile;
  tc.m0 = (within / gn) * kTile;
  return tc;
}

// ---------------------------------------------------------------------------
// Kernel 2, MXFP4: FP4 GEMM with E8M0 block scales + up projection + bias.
//
// The packed E2M1 nibbles are the matrix core's own FP4 format and the E8M0
// bytes are its block scales, so v_mfma_scale_f32_32x32x64_f8f6f4 (A and B
// as FP4) takes both straight from LDS: no conversion and no dequant work.
// One instruction covers 64 k = two MX blocks: lane half h holds the 32 k of
// block h of its row (16 bytes) and supplies that block's scale byte.
//
// Output tile 128 (n) x 128 (m) per workgroup of 4 waves, 64 x 64 per wave
// (2 x 2 MFMA tiles, Y^T orientation as in the INT4 kernel).  A pipeline
// stage is 256 k: 128 code bytes and 8 scale bytes per row (the last stage
// is a half stage when K % 256 == 128).  Per stage every thread loads four
// 16-byte chunks of W and four of X (eight lanes cover one 128-byte row
// segment) and one dword (4 rows of one block) of the W and of the X scales,
// which stay group-major in LDS ([block][row] bytes).
//
// Two-slot LDS ring: at the top of iteration g the registers holding stage
// g+1 (loaded during iteration g-1) are stored into slot (g+1)%2, the loads
// of stage g+2 are issued and stage g is computed from slot g%2; one barrier
// per stage.  A global load so has a whole stage of MFMA work plus the
// barrier to arrive before anything waits for it.
//
// Epilogue: the up projection on the accumulators, the bias, one rounding
// to bf16; the tile then goes through LDS so that each store writes 16
// contiguous bytes and eight lanes fill a 128-byte segment of a Y row.
// ---------------------------------------------------------------------------
constexpr int kMxStage = 256;                    // k per pipeline stage
constexpr int kMxStageB = kMxStage / 2;          // code bytes per row and stage
constexpr int kMxRow = kMxStageB + 16;           // LDS row stride in bytes (16 bytes of padding)
constexpr int kMxSlot = 2 * kTile * kMxRow;      // one ring slot: W rows, then X rows
constexpr int kMxThreads = 256;
constexpr int kMxYRow = kTile + 8;               // staging row stride of the output tile (bf16 elements)
static_assert(2 * kMxSlot >= kTile * kMxYRow * 2, "output staging fits in the ring");

// The staged 128-row output tile of the epilogue: rows 0-63 at lo, rows
// 64-127 at hi, kMxYRow bf16 per row (the halves may sit in different LDS
// arrays).
struct StageTile {
  uint16_t* lo;
  uint16_t* hi;
  __device__ __forceinline__ uint16_t* row(int r) const { return r < 64 ? lo + r * kMxYRow : hi + (r - 64) * kMxYRow; }
};
__device__ __forceinline__ StageTile stage_tile(uint16_t* base) { return StageTile{base, base + 64 * kMxYRow}; }

// tanh-form GELU, 0.5 y (1 + tanh(u)) with u = sqrt(2/pi) (y + 0.044715 y^3),
// evaluated as y / (1 + exp(-2u)) with the hardware exp2 and reciprocal
// (relative error a few ulp of fp32).
__device__ __forceinline__ float gelu_tanh_f32(float y) {
  const float u = 0.7978845608028654f * __builtin_fmaf(0.044715f * y, y * y, y);
  const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * u);     // exp(-2u)
  return y * __builtin_amdgcn_rcpf(1.0f + e);
}

// Second layer of an MLP pair, fed by the first layer's epilogue: its
// smoothing, L1 (lora_down2 [rank2][N]) and kernel-1 outputs.
struct MlpOut {
  const float* sinv2;
  const uint16_t* ldown2;
  int rank2;
  uint8_t* xq2;
  uint16_t* xs2;
  float* lact2;
};

// The second layer's kernel 1 on a staged 128 x 128 tile of X2 (bf16,
// [m][n] with row stride kMxYRow); N % 128 == 0.
__device__ __forceinline__ void mlp_tail(const StageTile& stg, int M, int N, int n0, int m0, int tid,
                                         const MlpOut& mo) {
  // thread t owns one 64-column group of one tile row: row t/2, columns
  // 64 (t%2) .. +64, so the group's absmax and scale stay in its registers
  const int r = tid >> 1, c0 = (tid & 1) * 64;
  const int m = m0 + r;
  const size_t rowb2 = static_cast<size_t>(N / 2);
  uint16_t* srow = stg.row(r) + c0;
  float xh[2][4][8];            // the group's 64 values: two halves of 32 (the code layout's 16-byte runs)
  float amax = 0.f;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    const uint4 v = *reinterpret_cast<const uint4*>(srow + 8 * ch);
    const float4 sa = *reinterpret_cast<const float4*>(mo.sinv2 + n0 + c0 + 8 * ch);
    const float4 sb = *reinterpret_cast<const float4*>(mo.sinv2 + n0 + c0 + 8 * ch + 4);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    const float sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
    uint32_t p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = cvt_pk_bf16(__uint_as_float(w4[e] << 16) * sv[2 * e], __uint_as_float(w4[e] & 0xFFFF0000u) * sv[2 * e + 1]);
      xh[ch >> 2][ch & 3][2 * e] = __uint_as_float(p[e] << 16);
      xh[ch >> 2][ch & 3][2 * e + 1] = __uint_as_float(p[e] & 0xFFFF0000u);
      amax = fmaxf(amax, fmaxf(fabsf(xh[ch >> 2][ch & 3][2 * e]), fabsf(xh[ch >> 2][ch & 3][2 * e + 1])));
    }
    *reinterpret_cast<uint4*>(srow + 8 * ch) = make_uint4(p[0], p[1], p[2], p[3]);   // x^2 for the MFMA
  }
  const uint32_t sbits = f16_sat_bits(__fdiv_rn(amax, 7.0f));
  const float sc = f16_bits_to_f32(sbits);
  const float invs = ((sc == 0.f) ? 0.f : __fdiv_rn(1.0f, sc)) * 0.125f;
  const uint4 w0 = pack_codes_fp6(xh[0], invs);
  const uint4 w1 = pack_codes_fp6(xh[1], invs);
  if (m < M) {
    uint4* dst = reinterpret_cast<uint4*>(mo.xq2 + static_cast<size_t>(m) * rowb2 + (n0 + c0) / 2);
    dst[0] = w0;
    dst[1] = w1;
    mo.xs2[static_cast<size_t>((n0 + c0) / 64) * M + m] = static_cast<uint16_t>(sbits);
  }
  __syncthreads();
  // partial down projection over the tile's 128 columns: wave w, rows
  // 32w .. +32 (two 16-row MFMA tiles), 16 ranks per MFMA, K = 128 in 4
  // steps of 32; lane (r16, q) holds row r16, columns 32s + 8q .. +8
  const int lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, qq = lane >> 4;
  for (int rt = 0; rt < mo.rank2 / 16; ++rt) {
    v4f d[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const v4i b = *reinterpret_cast<const v4i*>(mo.ldown2 + static_cast<size_t>(rt * 16 + r16) * N + n0 + 32 * ks + 8 * qq);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const v4i a = *reinterpret_cast<const v4i*>(stg.row(32 * wave + 16 * mt + r16) + 32 * ks + 8 * qq);
        d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), d[mt],
                                                       0, 0, 0);
      }
    }
    float dv[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dv[mt][i] = d[mt][i];
        asm volatile("" : "+v"(dv[mt][i]));     // read the MFMA results before the predicated atomics
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 32 * wave + 16 * mt + 4 * qq + i;
        if (m < M) atomicAdd(mo.lact2 + static_cast<size_t>(m) * mo.rank2 + rt * 16 + r16, dv[mt][i]);
      }
  }
}

// acc += bf16(lora_act) . L2 (16 ranks per v_mfma_f32_32x32x16_bf16) on the
// accumulators of a 128 x 128 tile (4 waves of 64 x 64, Y^T MFMA layout).
__device__ __forceinline__ void lora_up_acc(v16f (&acc)[2][2], const float* __restrict__ lact,
                                            const uint16_t* __restrict__ lup, int M, int N, int rank, int n0, int m0,
                                            int wn, int wm, int l32, int h) {
  for (int c0 = 0; c0 < rank; c0 += 16) {
    const int j = c0 + 8 * h;
    v4i ub[2], ua[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      const int m = m0 + wm * 64 + jt * 32 + l32;
      ub[jt] = v4i{0, 0, 0, 0};
      if (m < M) {
        const float4* src = reinterpret_cast<const float4*>(lact + static_cast<size_t>(m) * rank + j);
        const float4 f0 = src[0], f1 = src[1];
        ub[jt] = v4i{static_cast<int>(pack_bf16_rne(f0.x, f0.y)), static_cast<int>(pack_bf16_rne(f0.z, f0.w)),
                     static_cast<int>(pack_bf16_rne(f1.x, f1.y)), static_cast<int>(pack_bf16_rne(f1.z, f1.w))};
      }
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int n = n0 + wn * 64 + it * 32 + l32;
      ua[it] = n < N ? *reinterpret_cast<const v4i*>(lup + static_cast<size_t>(n) * rank + j) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
        acc[it][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ua[it]),
                                                              __builtin_bit_cast(v8bf, ub[jt]), acc[it][jt], 0, 0, 0);
  }
}

// The tile's bias values: lane element 4j+i of tile it is channel
// n0 + wn*64 + it*32 + 8j + 4h + i (zero without a bias).
__device__ __forceinline__ void load_bias(float (&bv)[2][4][4], const uint16_t* __restrict__ bias, int N, int n0, int wn,
                                          int h) {
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nb = n0 + wn * 64 + it * 32 + 8 * j + 4 * h;
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[it][j][i] = 0.f;
      if (bias) {
        if ((N % 4) == 0 && nb + 3 < N) {
          const uint2 b2 = *reinterpret_cast<const uint2*>(bias + nb);
          bv[it][j][0] = __uint_as_float(b2.x << 16);
          bv[it][j][1] = __uint_as_float(b2.x & 0xFFFF0000u);
          bv[it][j][2] = __uint_as_float(b2.y << 16);
          bv[it][j][3] = __uint_as_float(b2.y & 0xFFFF0000u);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (nb + i < N) bv[it][j][i] = __uint_as_float(static_cast<uint32_t>(bias[nb + i]) << 16);
        }
      }
    }
}

// Shared epilogue of the 128 x 128 GEMM tiles (4 waves of 64 x 64, Y^T
// MFMA layout): acc += bf16(lora_act) . L2 on the accumulators (16 ranks per
// v_mfma_f32_32x32x16_bf16), the bias, one rounding to bf16, then the tile
// goes through LDS (stg: kTile rows of kMxYRow bf16) so that each store
// writes 16 contiguous bytes and eight lanes fill a 128-byte segment of a Y
// row.  Every wave must be past its last LDS read of the main loop.
//
// EPI = 0 writes Y.  EPI = 1 writes bf16(GELU(Y)) (Y rounded to bf16 first,
// as the next layer would read it).  EPI = 2 writes nothing of Y: the tile
// of X2 = bf16(GELU(Y)) becomes the second layer's kernel-1 input --
// x^2 = bf16(X2 * smooth_inv2), its 4-bit codes and fp16 scales per 64
// columns (tile-local: a group lies inside the 128-column tile), and its
// partial down projection x^2 . L1_2 over the tile's 128 columns, summed
// into lact2 with fp32 atomics (lact2 cleared beforehand).
// UPL: rank 32, and the tile's lora_act rows (128 x 32 fp32, 128-byte rows,
// 16-byte chunk c of row r at chunk c ^ swz8(r)) and L2 rows (128 x 32 bf16
// at byte 16384, 64-byte rows, chunk c of row r at c ^ ((r / 4) % 4)) are
// already in LDS at upl.
// PRE: the low-rank term and the bias are already in acc (lora_up_acc and
// load_bias at the start of the tile).
template <int EPI, bool UPL = false, bool PRE = false, bool UPL_SYNC = false>
__device__ __forceinline__ void epilogue_tile128(v16f (&acc)[2][2], const StageTile& stg,
                                                 const float* __restrict__ lact, const uint16_t* __restrict__ lup,
                                                 const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M,
                                                 int N, int rank, int n0, int m0, int wn, int wm, int l32, int h,
                                                 int tid, const MlpOut& mo, const uint8_t* upl = nullptr,
                                                 const uint8_t* upl_hi = nullptr, const uint8_t* upl_u = nullptr,
                                                 const uint8_t* upl_b = nullptr) {
  float bv[2][4][4];
  if constexpr (UPL) {
    // lora_act rows 64-127 and the L2 rows may sit apart from rows 0-63
    const uint8_t* const a_hi = upl_hi ? upl_hi : upl + 64 * 128;
    const uint8_t* const u_rows = upl_u ? upl_u : upl + 16384;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      v4i ub[2], ua[2];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const int r = wm * 64 + jt * 32 + l32;
        const uint8_t* row = (wm ? a_hi : upl) + (jt * 32 + l32) * 128;
        const float4 f0 = *reinterpret_cast<const float4*>(row + (((4 * c + 2 * h) ^ swz8(r)) << 4));
        const float4 f1 = *reinterpret_cast<const float4*>(row + (((4 * c + 2 * h + 1) ^ swz8(r)) << 4));
        ub[jt] = m0 + r < M ? v4i{static_cast<int>(pack_bf16_rne(f0.x, f0.y)), static_cast<int>(pack_bf16_rne(f0.z, f0.w)),
                                  static_cast<int>(pack_bf16_rne(f1.x, f1.y)), static_cast<int>(pack_bf16_rne(f1.z, f1.w))}
                            : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int r = wn * 64 + it * 32 + l32;
        ua[it] = n0 + r < N ? *reinterpret_cast<const v4i*>(u_rows + r * 64 + (((2 * c + h) ^ ((r >> 2) & 3)) << 4))
                            : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
          acc[it][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ua[it]),
                                                                __builtin_bit_cast(v8bf, ub[jt]), acc[it][jt], 0, 0, 0);
    }
    // the bias of the tile's channels from LDS (bf16, channel n0 + i at
    // byte 2 i) or, without upl_b, from memory (zeros without a bias);
    // with UPL_SYNC read before the barrier: the staging below overwrites
    // LDS that other waves may still be reading
    if (upl_b) {
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int nl = wn * 64 + it * 32 + 8 * j + 4 * h;
          const uint2 b2 = *reinterpret_cast<const uint2*>(upl_b + 2 * nl);
          bv[it][j][0] = __uint_as_float(b2.x << 16);
          bv[it][j][1] = __uint_as_float(b2.x & 0xFFFF0000u);
          bv[it][j][2] = __uint_as_float(b2.y << 16);
          bv[it][j][3] = __uint_as_float(b2.y & 0xFFFF0000u);
        }
    } else {
      load_bias(bv, bias, N, n0, wn, h);
    }
    if constexpr (UPL_SYNC) {
      __syncthreads();
    }
  }
  if constexpr (!PRE) lora_up_acc(acc, lact, lup, M, N, UPL ? 0 : rank, n0, m0, wn, wm, l32, h);

  if constexpr (!UPL) load_bias(bv, PRE ? nullptr : bias, N, n0, wn, h);

  // Y = bf16(acc + bias), one rounding, into the staging tile [m][n]
#pragma unroll
  for (int jt = 0; jt < 2; ++jt)
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ml = wm * 64 + jt * 32 + l32;
        const int nl = wn * 64 + it * 32 + 8 * j + 4 * h;
        uint32_t p01 = cvt_pk_bf16(acc[it][jt][4 * j + 0] + bv[it][j][0], acc[it][jt][4 * j + 1] + bv[it][j][1]);
        uint32_t p23 = cvt_pk_bf16(acc[it][jt][4 * j + 2] + bv[it][j][2], acc[it][jt][4 * j + 3] + bv[it][j][3]);
        if constexpr (EPI >= 1) {
          p01 = cvt_pk_bf16(gelu_tanh_f32(__uint_as_float(p01 << 16)), gelu_tanh_f32(__uint_as_float(p01 & 0xFFFF0000u)));
          p23 = cvt_pk_bf16(gelu_tanh_f32(__uint_as_float(p23 << 16)), gelu_tanh_f32(__uint_as_float(p23 & 0xFFFF0000u)));
        }
        *reinterpret_cast<uint2*>(stg.row(ml) + nl) = make_uint2(p01, p23);
      }
  __syncthreads();

  if constexpr (EPI == 2) {
    mlp_tail(stg, M, N, n0, m0, tid, mo);
    return;
  }

  // 16-byte stores: thread t writes channels 8(t%16) .. +7 of tile rows t/16 + 16i
  const int c8 = (tid & 15) * 8;
  const int n = n0 + c8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 4) + 16 * i;
    const int m = m0 + r;
    if (m < M && n < N) {
      const uint4 v = *reinterpret_cast<const uint4*>(stg.row(r) + c8);
      uint16_t* dst = y + static_cast<size_t>(m) * N + n;
      if ((N % 8) == 0) {
        // non-temporal: Y is not read again here, and streaming it past the
        // caches keeps the operand panels resident (measured: INT4 fc1 -3 %,
        // MXFP4 fc1 -7 %, bit-identical output)
        __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(dst));
      } else {
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < N) dst[e] = static_cast<uint16_t>(vv[e / 2] >> (16 * (e % 2)));
      }
    }
  }
}

// One FP4 x FP4 MFMA over 64 k with per-lane block scales (byte 0 of sa, sb).
__device__ __forceinline__ v16f mfma_fp4(const v4i& a, const v4i& b, const v16f& c, uint32_t sa, uint32_t sb) {
  const v8i a8 = __builtin_shufflevector(a, v4i{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
  const v8i b8 = __builtin_shufflevector(b, v4i{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, static_cast<int>(sa), 0,
                                                         static_cast<int>(sb));
}

constexpr int kMxdRowB = 128;                      // LDS bytes per row and stage (no padding)
constexpr int kMxdOp = kTile * kMxdRowB;           // one operand's rows
constexpr int kMxdSlot = 2 * kMxdOp + 2 * 8 * kTile;   // W rows, X rows, then scales [W|X][block][row]
static_assert(kMxdSlot >= kTile * kMxYRow * 2, "output staging fits in one slot of the ring");
static_assert(kMxdSlot >= 16384 + 8192 + 1024, "rank-32 up-projection operands and the bias fit in one slot");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Rank 32: a tile's lora_act rows m0 .. +127 (fp32, 16 KB) and L2 rows
// n0 .. +127 (bf16, 8 KB) straight from memory into LDS at dst, in the
// layout of epilogue_tile128's UPL mode; rows past the edge read zero.
// Wave w (wave-uniform) moves lora_act rows 32 w .. +31 (four loads of 8
// rows) and L2 rows 32 w .. +31 (two loads of 16 rows); the caller waits
// (vmcnt) and synchronises before the epilogue reads them.
__device__ __forceinline__ void upl_issue(uint8_t* dst, const float* __restrict__ lact,
                                          const uint16_t* __restrict__ lup, const uint16_t* __restrict__ bias,
                                          int M, int N, int m0, int n0, int wave, int lane) {
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(lact + static_cast<size_t>(m0) * 32, static_cast<size_t>(M - m0) * 128);
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(lup + static_cast<size_t>(n0) * 32, static_cast<size_t>(N - n0) * 64);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int blk = 4 * wave + j, r = 8 * blk + (lane >> 3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(dst + blk * 1024), 16,
                                             r * 128 + (((lane & 7) ^ swz8(r)) << 4), 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int blk = 2 * wave + j, r = 16 * blk + (lane >> 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (lds_ptr_t)(dst + 16384 + blk * 1024), 16,
                                             r * 64 + (((lane & 3) ^ ((r >> 2) & 3)) << 4), 0, 0, 0);
  }
  // wave 0: the bias of channels n0 .. n0+511 (the tile uses the first 128)
  // into the kilobyte after the L2 rows; even N only (a buffer load bounds
  // each dword, so with odd N the last channel's dword would read zero)
  if (wave == 0 && bias && (N & 1) == 0) {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias + n0, static_cast<size_t>(N - n0) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(dst + 16384 + 8192), 16, 16 * lane, 0, 0, 0);
  }
}

__global__ __launch_bounds__(kMxThreads, 2) void k2_gemm_mxfp4(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws,
    const float* __restrict__ lact, const uint16_t* __restrict__ lup,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M, int N, int K, int rank) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_c[2][kMxdSlot];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int wn = wave >> 1, wm = wave & 1;
  const int S = (K + kMxStage - 1) / kMxStage;
  const int kb = K / 2;

  const TileCoord tc = tile_coord(blockIdx.x, (N + kTile - 1) / kTile, (M + kTile - 1) / kTile);
  const int n0 = tc.n0, m0 = tc.m0;

  // Direct-to-LDS loads.  Waves 0, 1 load W rows, waves 2, 3 X rows: load j
  // of a wave fills rows 64 (wave % 2) + 8 j .. + 7 of its operand, lane i
  // row + i/8, 16-byte LDS chunk i%8, which holds the row's chunk
  // (i%8) ^ swz8(row) (the XOR spreads a column of rows over the banks).
  // Rows past the matrix edge are clamped to its last row; the resources
  // bound every access.
  const bool is_w = wave < 2;
  const int rows = is_w ? N : M;
  const int r0 = is_w ? n0 : m0;
  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(is_w ? wq : xq, static_cast<size_t>(rows) * static_cast<size_t>(kb));
  const int lrow = 64 * (wave & 1) + (lane >> 3);          // + 8 j
  int vcode[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = lrow + 8 * j;
    vcode[j] = min(r0 + r, rows - 1) * kb + (((lane & 7) ^ swz8(r)) << 4);
  }
  const int lds_op = is_w ? 0 : kMxdOp;
  // scales of a stage: 8 blocks x 128 rows = 256 dwords per operand; the
  // operand's two waves load dwords d = 128 i + 64 (wave % 2) + lane
  // (i = 0, 1): block d / 32, rows 4 (d % 32) .. + 3, as one dword where
  // the 4 rows are inside the matrix (row count a multiple of 4), else as
  // bytes from rows clamped into the matrix
  const __amdgpu_buffer_rsrc_t rsc =
      make_rsrc(is_w ? ws : xs, static_cast<size_t>(K / 32) * static_cast<size_t>(rows));
  const int srow = r0 + 4 * (lane & 31);
  const bool s_dw = (rows % 4) == 0 && srow + 3 < rows;
  const int lds_sc = 2 * kMxdOp + (is_w ? 0 : 8 * kTile);

  auto issue = [&](int st, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int so = st * kMxStageB;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lds_ptr_t dst = (lds_ptr_t)(&lds_c[buf][lds_op + (lrow - (lane >> 3) + 8 * j) * kMxdRowB]);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, dst, 16, vcode[j] + so, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d0 = 128 * i + 64 * (wave & 1);          // first dword of this load
      const int blk = 8 * st + ((d0 + lane) >> 5);
      if (s_dw) {
        lds_ptr_t sdst = (lds_ptr_t)(&lds_c[buf][lds_sc + 4 * d0]);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, sdst, 4, blk * rows + srow, 0, 0, 0);
      } else {
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v |= static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b8(rsc, blk * rows + min(srow + e, rows - 1), 0, 0))
               << (8 * e);
        *reinterpret_cast<uint32_t*>(&lds_c[buf][lds_sc + 4 * (d0 + lane)]) = v;
      }
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[it][jt][r] = 0.f;

  // 64-k substep s: logical chunk 2s + h of the row (block 2s + h of the
  // stage), stored at chunk (2s + h) ^ swz8(row); swz8(row) = swz8(l32)
  // (rows differ from l32 by multiples of 32)
  auto compute = [&](auto buf_c, bool half) {
    constexpr int buf = decltype(buf_c)::value;
    const uint8_t* wb = &lds_c[buf][0] + (wn * 64 + l32) * kMxdRowB;
    const uint8_t* xb = &lds_c[buf][kMxdOp] + (wm * 64 + l32) * kMxdRowB;
    const uint8_t* wsc = &lds_c[buf][2 * kMxdOp] + wn * 64 + l32;
    const uint8_t* xsc = &lds_c[buf][2 * kMxdOp + 8 * kTile] + wm * 64 + l32;
    auto sub = [&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
      const int ch = ((2 * s + h) ^ swz8(l32)) << 4;
      v4i a[2], b[2];
      uint32_t sa[2], sb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *reinterpret_cast<const v4i*>(wb + t * 32 * kMxdRowB + ch);
        b[t] = *reinterpret_cast<const v4i*>(xb + t * 32 * kMxdRowB + ch);
        sa[t] = wsc[(2 * s + h) * kTile + t * 32];
        sb[t] = xsc[(2 * s + h) * kTile + t * 32];
      }
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
          acc[it][jt] = mfma_fp4(a[it], b[jt], acc[it][jt], sa[it], sb[jt]);
    };
    sub(Slot<0>{});
    sub(Slot<1>{});
    if (!half) {
      sub(Slot<2>{});
      sub(Slot<3>{});
    }
  };

  const bool half_last = (K % kMxStage) != 0;
  // Rank 32: during the last stage the tile's up-projection operands come
  // straight into the slot that stage does not use (upl_issue), and the
  // output is staged in the other slot.
  const bool upl = rank == 32;
  auto issue_up = [&](auto buf_c) {
    upl_issue(&lds_c[decltype(buf_c)::value][0], lact, lup, bias, M, N, m0, n0, wave, lane);
  };
  issue(0, Slot<0>{});
  __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): this wave's stage-0 data is in LDS
  __syncthreads();
  auto iteration = [&](int st, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    if (st + 1 < S) issue(st + 1, Slot<1 - buf>{});
    else if (upl) issue_up(Slot<1 - buf>{});
    compute(buf_c, half_last && st == S - 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };
  for (int st = 0; st < S; st += 2) {
    iteration(st, Slot<0>{});
    if (st + 1 < S) iteration(st + 1, Slot<1>{});
  }

  const int last = (S - 1) & 1;
  if (upl)
    epilogue_tile128<0, true>(acc, stage_tile(reinterpret_cast<uint16_t*>(&lds_c[last][0])), lact, lup, bias, y, M, N, rank, n0,
                              m0, wn, wm, l32, h, tid, MlpOut{}, &lds_c[1 - last][0], nullptr, nullptr,
                              bias && (N & 1) == 0 ? &lds_c[1 - last][16384 + 8192] : nullptr);
  else
    epilogue_tile128<0>(acc, stage_tile(reinterpret_cast<uint16_t*>(&lds_c[0][0])), lact, lup, bias, y, M, N, rank, n0,
                        m0, wn, wm, l32, h, tid, MlpOut{});
}

// Kernel 2, INT4: 4-bit GEMM + per-group dequant + up projection + bias.
//
// Same tiling and epilogue as the MXFP4 kernel: output tile 128 (n) x 128
// (m) per workgroup of 4 waves, 64 x 64 per wave.  A stage is 128 k = two
// K-groups: per row 64 packed bytes and two fp16 scales.
//
// Operands: the packed codes travel straight from memory into LDS
// (buffer_load ... lds, 16 bytes per lane: no staging registers, no LDS
// stores) through a three-slot ring, two stages ahead of their use.  Rows
// are 64 bytes, unpadded; logical 16-byte chunk j of row r (group j/2, half
// j%2) sits at chunk j ^ swz4(r), so that the 16-byte reads of 32
// consecutive rows at one chunk fall in distinct banks.  Each wave reads
// its operands' packed chunks and turns each into the six words in which
// v_mfma_scale_f32_32x32x64_f8f6f4 reads 32 FP6 E2M3 values q/8 (four
// operations per unit of 16 codes, see the code layout), so one FP6 MFMA
// over a group (K = 64) returns sum qw qx / 64 = P / 64 with the two scales'
// exponents applied as E8M0 block scales, exactly: every product is a
// multiple of 2^-6 and |P| <= 3136.
//
// Dequant: a scale s = m 2^e (m in [0.5, 1), v_frexp) gives the MFMA its
// exponent (+6 on the W side cancels the 1/64; -1 on the X side cancels
// the doubled product below); the significand products m_w(n) m_x(m) of a
// 32 x 32 tile-group are a rank-1 matrix, which one v_mfma_f32_32x32x8_f16
// returns exactly in fp32 and in P's layout (both lane halves carry the
// significands, so it comes out doubled); one fp32 FMA per element then adds
// P' * (2 m_w m_x) into the accumulators.  The scales are split once per
// workgroup (one row per thread) into a three-slot LDS ring of their own.
//
// DEBUG = true is a test hook on the same loads, LDS ring, code conversion
// and FP6 MFMA: unit scales, and the exact integer partial of every K-group
// written for a window [win_m0, +win_mt) x [win_n0, +win_nt) of the output
// instead of Y.
// ---------------------------------------------------------------------------
constexpr int kI4Stage = 128;                    // k per pipeline stage (2 groups)
constexpr int kI4RowB = kI4Stage / 2;            // packed bytes per row and stage
constexpr int kI4Op = kTile * kI4RowB;           // one operand's rows in a slot (8 KB)
constexpr int kI4Slots = 3;                      // ring depth: loads run two stages ahead
constexpr int kI4CoarseMinK = 8192;              // K from which the fused GEMM takes the coarse schedule
// every slot's W rows and X rows are LDS arrays of their own (so that the
// compiler tells a stage's reads from the loads landing in another slot and
// waits for neither); slot 0's two arrays also hold the epilogue's output
// tile, a half each
constexpr int kI4Half = 64 * kMxYRow * 2;        // 64 staged output rows
static_assert(kI4Half >= kI4Op, "slot 0's arrays hold both code rows and output rows");

// chunk swizzle of a 64-byte LDS row: bits (r1 ^ r3, r2) of the row index.
// Over any 8 consecutive rows (r0 = 0 mod 8) r mod 2 and the swizzle take all
// 8 combinations, and over any 16 (r0 = 0 mod 16) r mod 4 and the swizzle
// take all 16: conflict-free 16-byte reads for 32 and for 64 four-byte banks.
__device__ __forceinline__ int swz4(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | ((r >> 1) & 2); }

// one packed chunk (two units, 32 codes) -> the six matrix-core words
__device__ __forceinline__ v8i fp6_words(const uint4& w) {
  return v8i{static_cast<int>(w.x & ~kZ0), static_cast<int>(w.y & ~kZ1), static_cast<int>((w.x & kZ0) | (w.y & kZ1)),
             static_cast<int>(w.z & ~kZ0), static_cast<int>(w.w & ~kZ1), static_cast<int>((w.z & kZ0) | (w.w & kZ1)),
             0, 0};
}

// LDS address of a __shared__ object: the low 32 bits of its flat address.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

// buffer_load ... lds written as inline asm, so that the compiler neither
// counts these loads nor waits for them: a kernel that issues them orders
// them itself with s_waitcnt vmcnt and barriers (lds_wait_barrier).  M0
// holds the LDS address (one wait state between its write and the load).
// 16 bytes per lane land at M0 + 16 lane; 2 bytes per lane land,
// zero-extended, in the 4-byte slot M0 + 4 lane.
__device__ __forceinline__ void dma_b128(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff, int soff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(r), "s"(soff), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void dma_u16(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff, int soff) {
  asm volatile("s_nop 0\n\tbuffer_load_ushort %0, %1, %2 offen lds"
               :: "v"(voff), "s"(r), "s"(soff), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
// wait until at most N of the wave's vector-memory loads are outstanding
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// the wave's LDS accesses done and at most N loads outstanding, then the
// workgroup barrier
template <int N>
__device__ __forceinline__ void lds_wait_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

// Split-K (EPI = kEpiPartial): block (tile, y) computes stages
// [y per, min(S, (y + 1) per)) of the tile and writes its fp32 accumulators
// to part[(y * tiles + tile) * 4096 + i * 256 + thread], i = 0..15 (the
// thread's 64 values in accumulator order); the low-rank term, the bias and
// the rounding are left to k_splitk_finish.
constexpr int kEpiPartial = 3;
struct SplitOut {
  float4* part;
  int per;
};

template <bool DEBUG, int EPI = 0, bool COARSE = false, bool UPL = false>
__global__ __launch_bounds__(kMxThreads, 2) void k2_gemm_int4(
    const uint8_t* __restrict__ xq, const uint16_t* __restrict__ xs,
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
    const float* __restrict__ lact, const uint16_t* __restrict__ lup,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M, int N, int K, int rank,
    int win_m0, int win_n0, int win_mt, int win_nt, int32_t* __restrict__ dbg, MlpOut mo, SplitOut so) {
  __shared__ __attribute__((aligned(16))) uint8_t w_ring0[kI4Half];
  __shared__ __attribute__((aligned(16))) uint8_t x_ring0[kI4Half];
  __shared__ __attribute__((aligned(16))) uint8_t w_ring1[kI4Op];
  __shared__ __attribute__((aligned(16))) uint8_t x_ring1[kI4Op];
  __shared__ __attribute__((aligned(16))) uint8_t w_ring2[kI4Op];
  __shared__ __attribute__((aligned(16))) uint8_t x_ring2[kI4Op];
  auto wring = [&](int slot) __attribute__((always_inline)) { return slot == 0 ? w_ring0 : slot == 1 ? w_ring1 : w_ring2; };
  auto xring = [&](int slot) __attribute__((always_inline)) { return slot == 0 ? x_ring0 : slot == 1 ? x_ring1 : x_ring2; };
  // raw fp16 scales as loaded, [slot][operand W, X][group][row], one per
  // 4-byte slot; two slots (stage st lands in slot st % 2)
  __shared__ __attribute__((aligned(16))) uint32_t s_raw[2][2][2][kTile];
  // split scale words, [slot][operand W, X][row]: {g0 word0, g0 word1,
  // g1 word0, g1 word1} (split); stage st's in slot st % 2
  __shared__ __attribute__((aligned(16))) uint4 s_words[2][2][kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int wn = wave >> 1, wm = wave & 1;
  const int G = K / 64;
  const int S = (G + 1) / 2;                   // the last stage holds one group when G is odd
  const int kb = K / 2;
  // the stages this block computes: [s_lo, s_lo + SL) (all of them but in
  // the split-K pass)
  const int s_lo = EPI == kEpiPartial ? static_cast<int>(blockIdx.y) * so.per : 0;
  const int SL = EPI == kEpiPartial ? min(so.per, S - s_lo) : S;

  int n0, m0;
  if constexpr (DEBUG) {
    const int tiles_m = (win_mt + kTile - 1) / kTile;
    n0 = win_n0 + (blockIdx.x / tiles_m) * kTile;
    m0 = win_m0 + (blockIdx.x % tiles_m) * kTile;
  } else {
    const TileCoord tc = tile_coord(blockIdx.x, (N + kTile - 1) / kTile, (M + kTile - 1) / kTile);
    n0 = tc.n0;
    m0 = tc.m0;
  }

  // Loads: waves 0, 1 load W rows, waves 2, 3 X rows; wave w owns rows
  // 64 (w % 2) .. +63 of its operand.  Per stage a wave issues six loads,
  // in this order: its rows' fp16 scales of the stage's two groups (lane i
  // -> row 64 (w % 2) + i), then four code loads, load j filling rows
  // 64 (w % 2) + 16 j .. +15: lane i writes LDS chunk i % 4 of row i / 4 and
  // reads global chunk (i % 4) ^ swz4(row) of that row.  Rows past the
  // matrix edge are clamped to its last row; the resources bound every
  // access (a missing second group of an odd-G last stage reads zeros or
  // the next row, never used).
  const int op = wave >> 1;                    // wave-uniform: 0 W, 1 X
  const int ld_rows = op == 0 ? N - n0 : M - m0;
  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(op == 0 ? wq + static_cast<size_t>(n0) * kb : xq + static_cast<size_t>(m0) * kb,
                static_cast<size_t>(ld_rows) * static_cast<size_t>(kb));
  int vcode[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 64 * (wave & 1) + 16 * j + (lane >> 2);
    vcode[j] = min(r, ld_rows - 1) * kb + (((lane & 3) ^ swz4(r)) << 4);
  }
  const int s_rows = op == 0 ? N : M;
  const int s_row = tid & (kTile - 1);         // = 64 (wave % 2) + lane
  const int gbytes = 2 * s_rows;               // bytes per group of the scale array
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(op == 0 ? ws : xs, DEBUG ? 0 : static_cast<size_t>(G) * static_cast<size_t>(gbytes));
  const int vs = 2 * min((op == 0 ? n0 : m0) + s_row, s_rows - 1);
  auto dma = [&](int st, auto slot_c) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    const int gst = s_lo + st;                 // the stage's index in the tile's K loop
    const int sso = 2 * gst * gbytes;
    dma_u16(rs, lds_addr(&s_raw[st & 1][op][0][64 * (wave & 1)]), vs, sso);
    dma_u16(rs, lds_addr(&s_raw[st & 1][op][1][64 * (wave & 1)]), vs, sso + gbytes);
    const uint8_t* base = (op == 0 ? wring(slot) : xring(slot)) + 64 * (wave & 1) * kI4RowB;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma_b128(rc, lds_addr(base + 16 * j * kI4RowB), vcode[j], gst * kI4RowB);
  };
  // A scale s (fp16 >= 0) splits as s = m 2^e with m in [0.5, 1)
  // (v_frexp_mant_f16, v_frexp_exp_i16_f16, subnormals included; s == 0
  // gives m = 0, and its codes are zero too).  Two words per row and group:
  //   W: word0 = m | (e + 127 + 6) << 16, word1 = 0
  //   X: word0 = m,                       word1 = (e + 127 - 1) << 16
  // Byte 2 of W's word0 and of X's word1 is the E8M0 scale of the FP6 MFMA
  // (op_sel 2); as f16 operands of the rank-1 MFMA ({word0, word1} = k 0-3,
  // the same in k 4-7) W gives [m_w, e_w, 0, 0] and X [m_x, 0, 0, e_x], so
  // only k 0 and k 4 contribute: 2 m_w m_x, exactly.  Thread t splits the
  // row its own wave loaded (s_row of operand op).
  auto split = [&](int st) __attribute__((always_inline)) {
    if constexpr (DEBUG) return;
    const uint32_t raw[2] = {s_raw[st & 1][op][0][s_row], s_raw[st & 1][op][1][s_row]};
    uint32_t wv[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const _Float16 sv = __builtin_bit_cast(_Float16, static_cast<uint16_t>(raw[i]));
      const uint32_t m = __builtin_bit_cast(uint16_t, __builtin_amdgcn_frexp_manth(sv));
      const uint32_t e = static_cast<uint32_t>(__builtin_amdgcn_frexp_exph(sv) + (op == 0 ? 127 + 6 : 127 - 1)) & 0xFFu;
      wv[2 * i] = op == 0 ? (m | (e << 16)) : m;
      wv[2 * i + 1] = op == 0 ? 0u : (e << 16);
    }
    s_words[st & 1][op][s_row] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  };
  // UPL (rank 32, plain epilogue): the tile's lora_act rows (128 x 32 fp32)
  // and L2 rows (128 x 32 bf16) come straight into LDS while the K loop
  // runs, in the layout of epilogue_tile128's UPL mode: lora_act rows 0-63
  // into the W half and rows 64-127 into the X half of the ring slot that
  // stage SL % 3 would use (no stage uses it after stage SL - 3), the L2
  // rows into the tail of x_ring0 (past its code rows; only the epilogue's
  // staging writes there).  Wave w moves lora_act rows 32 w .. +31 (four
  // loads of 8 rows) and L2 rows 32 w .. +31 (two loads of 16 rows); rows
  // past the matrix edge read zero; wave 0 adds one load of the bias.
  // Six loads per wave (seven in wave 0), ordered by the kernel's own
  // waits.
  uint8_t* const upl_lo = wring(SL % kI4Slots);
  uint8_t* const upl_hi = xring(SL % kI4Slots);
  uint8_t* const upl_u = x_ring0 + kI4Op;
  uint8_t* const upl_b = x_ring0 + kI4Op + 8192;
  static_assert(kI4Op + 8192 + 1024 <= kI4Half, "L2 rows and bias fit in x_ring0 past its code rows");
  auto upl_dma = [&]() __attribute__((always_inline)) {
    if constexpr (UPL) {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(lact + static_cast<size_t>(m0) * 32, static_cast<size_t>(M - m0) * 128);
      const __amdgpu_buffer_rsrc_t ru = make_rsrc(lup + static_cast<size_t>(n0) * 32, static_cast<size_t>(N - n0) * 64);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int blk = 4 * wave + j, r = 8 * blk + (lane >> 3);
        dma_b128(ra, lds_addr((blk < 8 ? upl_lo : upl_hi) + (blk & 7) * 1024), r * 128 + (((lane & 7) ^ swz8(r)) << 4), 0);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int blk = 2 * wave + j, r = 16 * blk + (lane >> 2);
        dma_b128(ru, lds_addr(upl_u + blk * 1024), r * 64 + (((lane & 3) ^ ((r >> 2) & 3)) << 4), 0);
      }
      // wave 0 also moves the bias of channels n0 .. n0+511 (the tile uses
      // the first 128; past N it reads zero) to the kilobyte after the L2
      // rows.  Even N only: the buffer bounds a load dword by dword, so with
      // odd N the last channel's dword would read zero; odd N takes the
      // bias from memory in the epilogue.
      if (wave == 0 && bias && (N & 1) == 0) {
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias + n0, static_cast<size_t>(N - n0) * 2);
        dma_b128(rb, lds_addr(upl_b), 16 * lane, 0);
      }
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[it][jt][r] = 0.f;

  // packed chunks of group g for the lane: W rows (tiles 0, 1) and X rows
  struct Raw {
    uint4 a0, a1, b0, b1;
  };
  const int ch_off = swz4(l32) << 4;           // the lane's rows are l32 mod 32
  auto load_raw = [&](int slot, auto g_c) __attribute__((always_inline)) {
    constexpr int g = decltype(g_c)::value;
    const int off = ((2 * g + h) << 4) ^ ch_off;
    const uint8_t* wr = wring(slot) + (wn * 64 + l32) * kI4RowB + off;
    const uint8_t* xr = xring(slot) + (wm * 64 + l32) * kI4RowB + off;
    Raw o;
    o.a0 = *reinterpret_cast<const uint4*>(wr);
    o.a1 = *reinterpret_cast<const uint4*>(wr + 32 * kI4RowB);
    o.b0 = *reinterpret_cast<const uint4*>(xr);
    o.b1 = *reinterpret_cast<const uint4*>(xr + 32 * kI4RowB);
    return o;
  };
  struct Ops {
    v8i a0, a1, b0, b1;
  };
  auto cvt = [&](const Raw& r) __attribute__((always_inline)) {
    Ops o;
    o.a0 = fp6_words(r.a0);
    o.a1 = fp6_words(r.a1);
    o.b0 = fp6_words(r.b0);
    o.b1 = fp6_words(r.b1);
    return o;
  };
  // the stage's scale words of the lane's W rows (tiles 0, 1) and X rows
  struct Scl {
    uint4 w0, w1, x0, x1;
  };
  auto load_scl = [&](int wslot) __attribute__((always_inline)) {
    Scl c;
    c.w0 = s_words[wslot][0][wn * 64 + l32];
    c.w1 = s_words[wslot][0][wn * 64 + 32 + l32];
    c.x0 = s_words[wslot][1][wm * 64 + l32];
    c.x1 = s_words[wslot][1][wm * 64 + 32 + l32];
    return c;
  };
  // tile-group t = 2 it + jt of group g: the partial P of W tile it and X
  // tile jt, times 2^(e_w + e_x) / 2 (exact)
  auto mf = [&](const Ops& o, const Scl& c, auto g_c, auto t_c) __attribute__((always_inline)) {
    constexpr int g = decltype(g_c)::value;
    constexpr int t = decltype(t_c)::value;
    constexpr int it = t >> 1, jt = t & 1;
    const uint4& sw = it ? c.w1 : c.w0;
    const uint4& sx = jt ? c.x1 : c.x0;
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(it ? o.a1 : o.a0, jt ? o.b1 : o.b0, v16f{}, 2, 2, 2,
                                                           static_cast<int>(g ? sw.z : sw.x), 2,
                                                           static_cast<int>(g ? sx.w : sx.y));
  };
  // the rank-1 product 2 m_w m_x of the same tile-group
  const v16f zero16 = {};
  auto rk = [&](const Scl& c, auto g_c, auto t_c) __attribute__((always_inline)) {
    constexpr int g = decltype(g_c)::value;
    constexpr int t = decltype(t_c)::value;
    constexpr int it = t >> 1, jt = t & 1;
    const uint4& sw = it ? c.w1 : c.w0;
    const uint4& sx = jt ? c.x1 : c.x0;
    const h4 a = __builtin_bit_cast(h4, g ? make_uint2(sw.z, sw.w) : make_uint2(sw.x, sw.y));
    const h4 b = __builtin_bit_cast(h4, g ? make_uint2(sx.z, sx.w) : make_uint2(sx.x, sx.y));
    return __builtin_amdgcn_mfma_f32_32x32x8f16(a, b, zero16, 0, 0, 0);
  };
  auto dqc = [&](auto t_c, const v16f& p, const v16f& c) __attribute__((always_inline)) {
    constexpr int t = decltype(t_c)::value;
    constexpr int it = t >> 1, jt = t & 1;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[it][jt][r] = __builtin_fmaf(p[r], c[r], acc[it][jt][r]);
  };
  using I0 = Slot<0>;
  using I1 = Slot<1>;
  using I2 = Slot<2>;
  using I3 = Slot<3>;

  // A stage (one group on an odd-G last stage) runs its tile-groups in one
  // of two schedules; in both the second group's chunks are read and
  // converted while the first group computes, and the stage's last two
  // tile-groups leave compute with their MFMAs in flight, their dequant
  // (finish) running after the stage barrier.
  //  - fine (default): both MFMAs of tile-group t+1 (the FP6 product and the
  //    scale outer product) are issued before the dequant of tile-group t,
  //    and the compiler interleaves MFMAs and FMAs freely;
  //  - COARSE: the four MFMAs of two tile-groups back to back, then their 32
  //    dequant FMAs and the other VALU work, with scheduling barriers between
  //    the phases, so that with two waves per SIMD one wave's MFMA phase can
  //    run under the other's VALU phase.  Measured on FLUX's MLP layers it
  //    is faster over a 96-stage K loop and slower over a 24-stage one, so
  //    only long K loops take it.
  // Per output element the FMAs run in the same order in both.
  v16f pa, pb, ca, cb;
  auto finish = [&]() __attribute__((always_inline)) {
    dqc(I2{}, pa, ca);
    dqc(I3{}, pb, cb);
  };
  auto compute = [&](int slot, int wslot, bool one, int g0, auto&& pre) __attribute__((always_inline)) {
    if constexpr (DEBUG) {
      pre();
      auto group = [&](auto g_c) __attribute__((always_inline)) {
        constexpr int g = decltype(g_c)::value;
        const Ops o = cvt(load_raw(slot, g_c));
        const v8i a[2] = {o.a0, o.a1}, b[2] = {o.b0, o.b1};
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[it], b[jt], v16f{}, 2, 2, 0,
                                                                           kUnitScales, 0, kUnitScales);
            int32_t pi[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              pi[r] = static_cast<int32_t>(p[r] * 64.0f);     // exact: P / 64 * 64
              asm volatile("" : "+v"(pi[r]));               // read the MFMA result before the predicated stores
            }
            const int m = m0 + wm * 64 + jt * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int n = n0 + wn * 64 + it * 32 + 8 * (r / 4) + 4 * h + (r % 4);
              if (m < win_m0 + win_mt && n < win_n0 + win_nt)
                dbg[(static_cast<size_t>(m - win_m0) * win_nt + (n - win_n0)) * G + g0 + g] = pi[r];
            }
          }
      };
      group(I0{});
      if (!one) group(I1{});
    } else if constexpr (COARSE) {
      const Raw r0 = load_raw(slot, I0{});
      const Scl c = load_scl(wslot);
      pre();
      const Ops o0 = cvt(r0);
      __builtin_amdgcn_sched_barrier(0);
      pa = mf(o0, c, I0{}, I0{});
      ca = rk(c, I0{}, I0{});
      pb = mf(o0, c, I0{}, I1{});
      cb = rk(c, I0{}, I1{});
      __builtin_amdgcn_sched_barrier(0);
      dqc(I0{}, pa, ca);
      dqc(I1{}, pb, cb);
      __builtin_amdgcn_sched_barrier(0);
      pa = mf(o0, c, I0{}, I2{});
      ca = rk(c, I0{}, I2{});
      pb = mf(o0, c, I0{}, I3{});
      cb = rk(c, I0{}, I3{});
      __builtin_amdgcn_sched_barrier(0);
      if (one) return;
      const Ops o1 = cvt(load_raw(slot, I1{}));
      dqc(I2{}, pa, ca);
      dqc(I3{}, pb, cb);
      __builtin_amdgcn_sched_barrier(0);
      pa = mf(o1, c, I1{}, I0{});
      ca = rk(c, I1{}, I0{});
      pb = mf(o1, c, I1{}, I1{});
      cb = rk(c, I1{}, I1{});
      __builtin_amdgcn_sched_barrier(0);
      dqc(I0{}, pa, ca);
      dqc(I1{}, pb, cb);
      __builtin_amdgcn_sched_barrier(0);
      pa = mf(o1, c, I1{}, I2{});
      ca = rk(c, I1{}, I2{});
      pb = mf(o1, c, I1{}, I3{});
      cb = rk(c, I1{}, I3{});
    } else {
      const Raw r0 = load_raw(slot, I0{});
      const Scl c = load_scl(wslot);
      pre();
      const Ops o0 = cvt(r0);
      pa = mf(o0, c, I0{}, I0{});
      ca = rk(c, I0{}, I0{});
      pb = mf(o0, c, I0{}, I1{});
      cb = rk(c, I0{}, I1{});
      dqc(I0{}, pa, ca);
      pa = mf(o0, c, I0{}, I2{});
      ca = rk(c, I0{}, I2{});
      dqc(I1{}, pb, cb);
      pb = mf(o0, c, I0{}, I3{});
      cb = rk(c, I0{}, I3{});
      if (one) return;
      const Ops o1 = cvt(load_raw(slot, I1{}));
      dqc(I2{}, pa, ca);
      pa = mf(o1, c, I1{}, I0{});
      ca = rk(c, I1{}, I0{});
      dqc(I3{}, pb, cb);
      pb = mf(o1, c, I1{}, I1{});
      cb = rk(c, I1{}, I1{});
      dqc(I0{}, pa, ca);
      pa = mf(o1, c, I1{}, I2{});
      ca = rk(c, I1{}, I2{});
      dqc(I1{}, pb, cb);
      pb = mf(o1, c, I1{}, I3{});
      cb = rk(c, I1{}, I3{});
    }
  };

  // Pipeline: at the top of iteration st, stage st (codes and scale words)
  // is in LDS for every wave and stage st+1's six loads per wave may still
  // be out.  The iteration reads stage st's first group and scale words,
  // issues stage st+2's loads (when there is one), finishes stage st-1 and
  // computes stage st; then, once the wave's own scale loads of stage st+1
  // have landed (at most the four code loads of stage st+1 and the six of
  // stage st+2 still out), it splits stage st+1's scales, and it ends with
  // stage st+1 complete (at most stage st+2's six loads out) and the
  // barrier.
  // Prologue: stage 0 in flight; meanwhile the tile's low-rank term and
  // bias go into the accumulators (the main loop adds the 4-bit products to
  // them).  Stage 1 is issued only after that, so that the compiler's wait
  // for the low-rank operands (it counts only its own loads, hence waits
  // for every load issued before them) does not also wait for stage 1;
  // then stage 0 complete and split.
  dma(0, Slot<0>{});
  if constexpr (UPL) {
    if (SL == 1) upl_dma();
  } else if constexpr (!DEBUG && EPI != kEpiPartial) {
    lora_up_acc(acc, lact, lup, M, N, rank, n0, m0, wn, wm, l32, h);
    float bv[2][4][4];
    load_bias(bv, bias, N, n0, wn, h);
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[it][jt][r] += bv[it][r / 4][r % 4];
  }
  if (SL > 1) dma(1, Slot<1>{});
  if (SL > 1)
    vm_wait<6>();
  else
    vm_wait<0>();
  split(0);
  lds_wait_barrier<6>();                       // stage 1's loads may stay out
  auto iteration = [&](int st, auto slot_c) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    constexpr int slot2 = (slot + 2) % kI4Slots;
    const bool ahead = st + 2 < SL;            // uniform
    // UPL: the up-projection operands are issued with the second-to-last
    // stage (six loads per wave behind stage st+1's, in the place of a
    // stage st+2), so the waits below count them like a stage's loads
    const bool up_now = UPL && st + 2 == SL;
    compute(slot, st & 1, 2 * (s_lo + st) + 1 >= G, 2 * st, [&]() __attribute__((always_inline)) {
      if (ahead) dma(st + 2, Slot<slot2>{});
      if constexpr (UPL)
        if (up_now) upl_dma();
      if constexpr (!DEBUG)
        if (st > 0) finish();
    });
    if (st + 1 < SL) {
      if (ahead || up_now)
        vm_wait<10>();
      else
        vm_wait<4>();
      split(st + 1);
    }
    if (ahead || up_now)
      lds_wait_barrier<6>();
    else
      lds_wait_barrier<0>();
  };
  for (int st = 0; st < SL; st += 3) {
    iteration(st, Slot<0>{});
    if (st + 1 < SL) iteration(st + 1, Slot<1>{});
    if (st + 2 < SL) iteration(st + 2, Slot<2>{});
  }

  if constexpr (!DEBUG) finish();
  if constexpr (EPI == kEpiPartial) {
    float4* dst = so.part + (static_cast<size_t>(blockIdx.y) * gridDim.x + blockIdx.x) * 4096 + tid;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const v16f& a = acc[i >> 3][(i >> 2) & 1];
      const int r = 4 * (i & 3);
      dst[i * 256] = make_float4(a[r], a[r + 1], a[r + 2], a[r + 3]);
    }
  } else if constexpr (UPL) {
    epilogue_tile128<EPI, true, false, true>(acc, StageTile{reinterpret_cast<uint16_t*>(w_ring0), reinterpret_cast<uint16_t*>(x_ring0)},
                                             lact, lup, bias, y, M, N, rank, n0, m0, wn, wm, l32, h, tid, mo, upl_lo,
                                             upl_hi, upl_u, bias && (N & 1) == 0 ? upl_b : nullptr);
  } else if constexpr (!DEBUG) {
    epilogue_tile128<EPI, false, true>(acc, StageTile{reinterpret_cast<uint16_t*>(w_ring0), reinterpret_cast<uint16_t*>(x_ring0)}, lact,
                          lup, bias, y, M, N, rank, n0, m0, wn, wm, l32, h, tid, mo);
  }
}

// Second pass of the split-K schedule: the splits' fp32 partials of a tile
// summed in split order, then the shared epilogue (the up projection on the
// accumulators, the bias, one rounding to bf16, full-line stores).
__global__ __launch_bounds__(kMxThreads) void k_splitk_finish(const float4* __restrict__ part, int splits,
                                                         const float* __restrict__ lact,
                                                         const uint16_t* __restrict__ lup,
                                                         const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
                                                         int M, int N, int rank) {
  __shared__ __attribute__((aligned(16))) uint16_t stg_lo[64 * kMxYRow];
  __shared__ __attribute__((aligned(16))) uint16_t stg_hi[64 * kMxYRow];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int wn = wave >> 1, wm = wave & 1;
  const TileCoord tc = tile_coord(blockIdx.x, (N + kTile - 1) / kTile, (M + kTile - 1) / kTile);
  v16f acc[2][2];
  const float4* src = part + static_cast<size_t>(blockIdx.x) * 4096 + tid;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 v = src[i * 256];
    v16f& a = acc[i >> 3][(i >> 2) & 1];
    const int r = 4 * (i & 3);
    a[r] = v.x;
    a[r + 1] = v.y;
    a[r + 2] = v.z;
    a[r + 3] = v.w;
  }
  for (int sp = 1; sp < splits; ++sp) {
    src += static_cast<size_t>(gridDim.x) * 4096;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 v = src[i * 256];
      v16f& a = acc[i >> 3][(i >> 2) & 1];
      const int r = 4 * (i & 3);
      a[r] += v.x;
      a[r + 1] += v.y;
      a[r + 2] += v.z;
      a[r + 3] += v.w;
    }
  }
  epilogue_tile128<0>(acc, StageTile{stg_lo, stg_hi}, lact, lup, bias, y, M, N, rank, tc.n0, tc.m0, wn, wm, l32, h,
                      tid, MlpOut{});
}

// ---------------------------------------------------------------------------
// W4A16 comparison GEMM: 4-bit weights (the layer's INT4 codes and fp16
// group scales), bf16 activations, bf16 matrix-core products.
//
// Same tiling, XCD map, two-slot ring and epilogue as the 4-bit kernels; a
// stage is one K-group of 64.  The loader turns each 16 packed bytes of W
// into 32 bf16 weights on their way into LDS: the two units' matrix-core
// words (code layout) hold the codes as FP6 E2M3 values q/8, which
// v_cvt_scalef32_pk32_f32_fp6 decodes exactly, in k order; the product with
// 8 s is q s exactly in fp32 and one rounding makes it bf16.  X tiles go to
// LDS as they are.  v_mfma_f32_32x32x16_bf16 accumulates in fp32.
// ---------------------------------------------------------------------------
constexpr int kW16Row = 64 * 2 + 16;            // LDS row: 64 bf16 + 16 bytes padding
constexpr int kW16Slot = 2 * kTile * kW16Row;   // W rows, then X rows
static_assert(2 * kW16Slot >= kTile * kMxYRow * 2, "output staging fits in the ring");

__global__ __launch_bounds__(kMxThreads, 2) void k2_gemm_w4a16(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) int8_t lds_c[2][kW16Slot];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int wn = wave >> 1, wm = wave & 1;
  const int G = K / 64;
  const size_t kb = static_cast<size_t>(K / 2);

  const TileCoord tc = tile_coord(blockIdx.x, (N + kTile - 1) / kTile, (M + kTile - 1) / kTile);
  const int n0 = tc.n0, m0 = tc.m0;

  // W: thread t dequantizes half (t%2) of the group's 64 codes of row t/2;
  // rows past the matrix edge are clamped to its last row (never stored)
  const int wr = tid >> 1, wc = tid & 1;
  const int wrow = min(n0 + wr, N - 1);
  const uint8_t* wsrc = wq + static_cast<size_t>(wrow) * kb + wc * 16;
  const uint16_t* wsc = ws + wrow;
  const int wdst = wr * kW16Row + wc * 64;
  // X: rows wave*32 + 8i + lane/8 (i = 0..3), 16-byte chunk lane%8 of the
  // group's 128 bytes (eight lanes per row)
  const int xr = wave * 32 + (lane >> 3), xc = lane & 7;
  const uint16_t* xsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xsrc[i] = x + static_cast<size_t>(min(m0 + xr + 8 * i, M - 1)) * K + xc * 8;
  const int xdst = kTile * kW16Row + xr * kW16Row + xc * 16;

  struct LoadRegs {
    uint4 w, x0, x1, x2, x3;
    uint32_t s;
  };
  auto gload = [&](int g) {
    LoadRegs L;
    L.w = *reinterpret_cast<const uint4*>(wsrc + g * 32);
    L.s = wsc[static_cast<size_t>(g) * N];
    L.x0 = *reinterpret_cast<const uint4*>(xsrc[0] + g * 64);
    L.x1 = *reinterpret_cast<const uint4*>(xsrc[1] + g * 64);
    L.x2 = *reinterpret_cast<const uint4*>(xsrc[2] + g * 64);
    L.x3 = *reinterpret_cast<const uint4*>(xsrc[3] + g * 64);
    return L;
  };
  auto lstore = [&](auto buf_c, LoadRegs L) {
    constexpr int buf = decltype(buf_c)::value;
    const float sc = f16_bits_to_f32(L.s) * 8.0f;          // 8 s: (q/8) (8 s) = q s exactly
    const v6u d = {L.w.x & ~kZ0, L.w.y & ~kZ1, (L.w.x & kZ0) | (L.w.y & kZ1),
                   L.w.z & ~kZ0, L.w.w & ~kZ1, (L.w.z & kZ0) | (L.w.w & kZ1)};
    const v32f v = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(d, 1.0f);   // q/8 of the 32 codes, in k order
    uint32_t o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = cvt_pk_bf16(v[2 * i] * sc, v[2 * i + 1] * sc);
    uint4* wd = reinterpret_cast<uint4*>(&lds_c[buf][0] + wdst);
    wd[0] = make_uint4(o[0], o[1], o[2], o[3]);
    wd[1] = make_uint4(o[4], o[5], o[6], o[7]);
    wd[2] = make_uint4(o[8], o[9], o[10], o[11]);
    wd[3] = make_uint4(o[12], o[13], o[14], o[15]);
    int8_t* xd = &lds_c[buf][0] + xdst;
    *reinterpret_cast<uint4*>(xd) = L.x0;
    *reinterpret_cast<uint4*>(xd + 8 * kW16Row) = L.x1;
    *reinterpret_cast<uint4*>(xd + 16 * kW16Row) = L.x2;
    *reinterpret_cast<uint4*>(xd + 24 * kW16Row) = L.x3;
  };

  v16f acc[2][2];
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[it][jt][r] = 0.f;

  // 16-k step s of the group: lane half h holds k 16s + 8h .. +8 of its row
  auto compute = [&](auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int8_t* wb = &lds_c[buf][0] + (wn * 64 + l32) * kW16Row + 16 * h;
    const int8_t* xb = &lds_c[buf][kTile * kW16Row] + (wm * 64 + l32) * kW16Row + 16 * h;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *reinterpret_cast<const v4i*>(wb + t * 32 * kW16Row + 32 * s);
        b[t] = *reinterpret_cast<const v4i*>(xb + t * 32 * kW16Row + 32 * s);
      }
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
          acc[it][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[it]),
                                                                __builtin_bit_cast(v8bf, b[jt]), acc[it][jt], 0, 0, 0);
    }
  };

  LoadRegs ld = gload(0);
  lstore(Slot<0>{}, ld);
  if (G > 1) ld = gload(1);
  __syncthreads();

  auto iteration = [&](int g, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    if (g + 1 < G) lstore(Slot<1 - buf>{}, ld);
    if (g + 2 < G) ld = gload(g + 2);
    compute(buf_c);
    __syncthreads();
  };
  for (int g = 0; g < G; g += 2) {
    iteration(g, Slot<0>{});
    if (g + 1 < G) iteration(g + 1, Slot<1>{});
  }

  epilogue_tile128<0>(acc, stage_tile(reinterpret_cast<uint16_t*>(&lds_c[0][0])), nullptr, nullptr, bias, y, M, N, 0,
                      n0, m0, wn, wm, l32, h, tid, MlpOut{});
}

// K1 grid: 64-row blocks x K slices.  The slice count is chosen so that
// the grid holds about four workgroups per CU (256 CUs), with slices of
// whole 128-k steps and at most kK1MaxSliceSteps steps, which bounds the
// slice's smooth_inv staging in LDS at 8 KB for any M and K.
template <int RT, int QMODE = kQuantInt4>
hipError_t launch_k1(const void* x, int M, int K, const float* sinv, const void* ldown, uint8_t* xq, void* xs,
                     float* lact, hipStream_t st) {
  const int row_blocks = (M + kK1Rows - 1) / kK1Rows;
  const int steps = (K + 127) / 128;
  constexpr int kK1MaxSliceSteps = 16;
  int slices = (1024 + row_blocks - 1) / row_blocks;
  if (slices > steps) slices = steps;
  if (slices < 1) slices = 1;
  if (slices < (steps + kK1MaxSliceSteps - 1) / kK1MaxSliceSteps) slices = (steps + kK1MaxSliceSteps - 1) / kK1MaxSliceSteps;
  const int steps_per_slice = (steps + slices - 1) / slices;
  const int ks = steps_per_slice * 128;
  slices = (steps + steps_per_slice - 1) / steps_per_slice;
  const size_t lds = static_cast<size_t>(ks) * sizeof(float);
  dim3 grid(row_blocks, slices), block(256);
  const bool atomic = RT > 0 && slices > 1;
  if (atomic) {
    const size_t n = static_cast<size_t>(M) * RT * 16;
    hipLaunchKernelGGL(fill_zero_f32, dim3(static_cast<unsigned>((n / 4 + 255) / 256)), dim3(256), 0, st, lact, n);
    hipLaunchKernelGGL((k1_quant_down_int4<RT, true, QMODE>), grid, block, lds, st, static_cast<const uint16_t*>(x), M, K,
                       sinv, static_cast<const uint16_t*>(ldown), xq, xs, lact, ks);
  } else {
    hipLaunchKernelGGL((k1_quant_down_int4<RT, false, QMODE>), grid, block, lds, st, static_cast<const uint16_t*>(x), M, K,
                       sinv, static_cast<const uint16_t*>(ldown), xq, xs, lact, ks);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Unfused baseline (engine caption (a) of the "svdq-int4-flux.1-dev" card:
// the low-rank branch as separate kernels): quantize (K1 without the down
// projection), down projection (K1's loop without the quantizer, reading X a
// second time), 4-bit GEMM (K2 without the up projection and bias, writing
// a bf16 Y) and this up projection, which reads Y back, adds
// bf16(lora_act) . L2 and the bias, and writes Y again.  Same arithmetic as
// the fused path except that the GEMM's output is rounded to bf16 before the
// up projection is added (a second rounding).
//
// Tile 64 (n) x 64 (m) per workgroup of 4 waves, 32 x 32 per wave, Y^T
// orientation as in kernel 2 (a lane holds 4 consecutive channels of one
// token: 8-byte loads and stores of Y).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_up_proj(const float* __restrict__ lact, const uint16_t* __restrict__ lup,
                                                 const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M,
                                                 int N, int rank) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * 64 + (wave & 1) * 32;
  const int m0 = blockIdx.y * 64 + (wave >> 1) * 32;
  const int m = m0 + l32, n = n0 + l32;
  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int c0 = 0; c0 < rank; c0 += 16) {
    const int j = c0 + 8 * h;
    v4i ub = v4i{0, 0, 0, 0}, ua = v4i{0, 0, 0, 0};
    if (m < M) {
      const float4* src = reinterpret_cast<const float4*>(lact + static_cast<size_t>(m) * rank + j);
      const float4 f0 = src[0], f1 = src[1];
      ub = v4i{static_cast<int>(pack_bf16_rne(f0.x, f0.y)), static_cast<int>(pack_bf16_rne(f0.z, f0.w)),
               static_cast<int>(pack_bf16_rne(f1.x, f1.y)), static_cast<int>(pack_bf16_rne(f1.z, f1.w))};
    }
    if (n < N) ua = *reinterpret_cast<const v4i*>(lup + static_cast<size_t>(n) * rank + j);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ua), __builtin_bit_cast(v8bf, ub), acc, 0,
                                                  0, 0);
  }
  float out[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    out[r] = acc[r];
    asm volatile("" : "+v"(out[r]));     // read the MFMA result before the predicated code below
  }
  if (m >= M) return;
  const bool vec_ok = (N % 4) == 0;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int nb = n0 + 8 * jj + 4 * h;
    uint16_t* dst = y + static_cast<size_t>(m) * N + nb;
    if (vec_ok && nb + 3 < N) {
      const uint2 old = *reinterpret_cast<const uint2*>(dst);
      const uint32_t ov[4] = {old.x & 0xFFFFu, old.x >> 16, old.y & 0xFFFFu, old.y >> 16};
      uint32_t nv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float b = bias ? __uint_as_float(static_cast<uint32_t>(bias[nb + i]) << 16) : 0.f;
        nv[i] = bf16_rne_bits(__uint_as_float(ov[i] << 16) + out[4 * jj + i] + b);
      }
      *reinterpret_cast<uint2*>(dst) = make_uint2(nv[0] | (nv[1] << 16), nv[2] | (nv[3] << 16));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (nb + i < N) {
          const float b = bias ? __uint_as_float(static_cast<uint32_t>(bias[nb + i]) << 16) : 0.f;
          dst[i] = static_cast<uint16_t>(bf16_rne_bits(__uint_as_float(static_cast<uint32_t>(dst[i]) << 16) +
                                                       out[4 * jj + i] + b));
        }
    }
  }
}

template <int RT>
hipError_t launch_unfused(const void* x, int M, int K, const float* sinv, const void* ldown, const uint8_t* wq,
                          const void* ws, const void* lup, const void* bias, int N, uint8_t* xq, void* xs,
                          float* lact, void* y, hipStream_t st) {
  hipError_t e = launch_k1<0>(x, M, K, sinv, nullptr, xq, xs, nullptr, st);           // 1: quantize
  if (e != hipSuccess) return e;
  if constexpr (RT > 0) {
    e = launch_k1<RT, kQuantNone>(x, M, K, sinv, ldown, xq, xs, lact, st);            // 2: down projection
    if (e != hipSuccess) return e;
  }
  const int tiles = ((N + kTile - 1) / kTile) * ((M + kTile - 1) / kTile);               // 3: 4-bit GEMM
  hipLaunchKernelGGL(k2_gemm_int4<false>, dim3(tiles), dim3(kMxThreads), 0, st, xq, static_cast<const uint16_t*>(xs),
                     wq, static_cast<const uint16_t*>(ws), nullptr, nullptr, nullptr, static_cast<uint16_t*>(y), M, N,
                     K, 0, 0, 0, 0, 0, nullptr, MlpOut{}, SplitOut{});
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_up_proj, dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, st, lact,  // 4: up projection
                     static_cast<const uint16_t*>(lup), static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y),
                     M, N, RT * 16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Matrix-core ceiling, for the measurement only: every wave issues 8
// independent v_mfma_scale_f32_32x32x64_f8f6f4 per iteration (FP8 operands,
// or FP4 with PREC = SVDQ_MXFP4) on lane-dependent operand bits, so the rate
// is that of dense MFMA issue at the clock this load sustains.  Two
// workgroups of 4 waves per CU (2 waves per SIMD, as in the GEMMs).  out[b]
// receives one sum per workgroup so nothing is dead code.
// ---------------------------------------------------------------------------
template <int PREC>
__global__ __launch_bounds__(256, 2) void k_mfma_ceiling(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const uint32_t seed = 0x9E3779B9u * static_cast<uint32_t>(lane + 1 + threadIdx.x);
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // FP8: bytes 0x08..0x37 (normal, moderate); FP4: any nibble
    const uint32_t r = seed * (2u * i + 1u) ^ (seed >> 13);
    a[i] = static_cast<int>(PREC == 1 ? r : (r & 0x37373737u) | 0x08080808u);
    b[i] = static_cast<int>(PREC == 1 ? (r >> 3) | (r << 29) : ((r >> 3) & 0x37373737u) | 0x08080808u);
  }
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
  constexpr int F = PREC == 1 ? 4 : 0;
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, F, F, 0, 0x70707070, 0, 0x70707070);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, F, F, 0, 0x70707070, 0, 0x70707070);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, F, F, 0, 0x70707070, 0, 0x70707070);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, F, F, 0, 0x70707070, 0, 0x70707070);
    c4 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c4, F, F, 0, 0x71717171, 0, 0x70707070);
    c5 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c5, F, F, 0, 0x71717171, 0, 0x70707070);
    c6 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c6, F, F, 0, 0x71717171, 0, 0x70707070);
    c7 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c7, F, F, 0, 0x71717171, 0, 0x70707070);
  }
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) sum += c0[r] + c1[r] + c2[r] + c3[r] + c4[r] + c5[r] + c6[r] + c7[r];
  sum += __shfl_xor(sum, 32);
  if (threadIdx.x == 0) out[blockIdx.x] = sum;
}

}  // namespace

extern "C" int svdq_launch_quantize_act_lora_down(const void* x, int M, int K, const float* smooth_inv,
                                                  const void* lora_down, int rank, int precision, uint8_t* xq,
                                                  void* xs, float* lora_act, void* stream) {
  if (precision != SVDQ_INT4 && precision != SVDQ_MXFP4) return static_cast<int>(hipErrorInvalidValue);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool mx = precision == SVDQ_MXFP4;
  hipError_t e;
  switch (rank / 16) {
#define SVDQ_K1_CASE(R)                                                                        \
  case R:                                                                                      \
    e = mx ? launch_k1<R, kQuantMx>(x, M, K, smooth_inv, lora_down, xq, xs, lora_act, st)      \
           : launch_k1<R, kQuantInt4>(x, M, K, smooth_inv, lora_down, xq, xs, lora_act, st); \
    break;
    SVDQ_K1_CASE(0) SVDQ_K1_CASE(1) SVDQ_K1_CASE(2) SVDQ_K1_CASE(3) SVDQ_K1_CASE(4) SVDQ_K1_CASE(5)
    SVDQ_K1_CASE(6) SVDQ_K1_CASE(7) SVDQ_K1_CASE(8) SVDQ_K1_CASE(9) SVDQ_K1_CASE(10) SVDQ_K1_CASE(11)
    SVDQ_K1_CASE(12) SVDQ_K1_CASE(13) SVDQ_K1_CASE(14) SVDQ_K1_CASE(15) SVDQ_K1_CASE(16)
#undef SVDQ_K1_CASE
    default:
      return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(e);
}

extern "C" int svdq_launch_gemm_w4a4_lora_up(const uint8_t* xq, const void* xs, const uint8_t* wq, const void* ws,
                                             const float* lora_act, const void* lora_up, const void* bias, void* y,
                                             int M, int N, int K, int rank, int precision, void* stream) {
  if (precision != SVDQ_INT4 && precision != SVDQ_MXFP4) return static_cast<int>(hipErrorInvalidValue);
  const int tiles = ((N + kTile - 1) / kTile) * ((M + kTile - 1) / kTile);
  if (precision == SVDQ_MXFP4) {
    hipLaunchKernelGGL(k2_gemm_mxfp4, dim3(tiles), dim3(kMxThreads), 0, static_cast<hipStream_t>(stream), xq,
                       static_cast<const uint8_t*>(xs), wq, static_cast<const uint8_t*>(ws), lora_act,
                       static_cast<const uint16_t*>(lora_up), static_cast<const uint16_t*>(bias),
                       static_cast<uint16_t*>(y), M, N, K, rank);
    return static_cast<int>(hipGetLastError());
  }
  // long K loops take the coarse MFMA/VALU phases (see k2_gemm_int4); on
  // the fine schedule rank 32 brings its up-projection operands and the
  // bias into LDS during the K loop (on the coarse one that measured ~1 %
  // slower, on the fine one ~4 % faster, FLUX fc2 / fc1)
  if (K >= kI4CoarseMinK)
    hipLaunchKernelGGL((k2_gemm_int4<false, 0, true>), dim3(tiles), dim3(kMxThreads), 0,
                       static_cast<hipStream_t>(stream), xq, static_cast<const uint16_t*>(xs), wq,
                       static_cast<const uint16_t*>(ws), lora_act, static_cast<const uint16_t*>(lora_up),
                       static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), M, N, K, rank, 0, 0, 0, 0,
                       nullptr, MlpOut{}, SplitOut{});
  else if (rank == 32)
    hipLaunchKernelGGL((k2_gemm_int4<false, 0, false, true>), dim3(tiles), dim3(kMxThreads), 0,
                       static_cast<hipStream_t>(stream), xq, static_cast<const uint16_t*>(xs), wq,
                       static_cast<const uint16_t*>(ws), lora_act, static_cast<const uint16_t*>(lora_up),
                       static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), M, N, K, rank, 0, 0, 0, 0,
                       nullptr, MlpOut{}, SplitOut{});
  else
    hipLaunchKernelGGL(k2_gemm_int4<false>, dim3(tiles), dim3(kMxThreads), 0, static_cast<hipStream_t>(stream), xq,
                       static_cast<const uint16_t*>(xs), wq, static_cast<const uint16_t*>(ws), lora_act,
                       static_cast<const uint16_t*>(lora_up), static_cast<const uint16_t*>(bias),
                       static_cast<uint16_t*>(y), M, N, K, rank, 0, 0, 0, 0, nullptr, MlpOut{}, SplitOut{});
  return static_cast<int>(hipGetLastError());
}

// Split-K plan of the fused INT4 GEMM for the current device: a grid whose
// tiles fill under half the workgroup slots (two per CU) and whose K loop
// is long (at least kSplitMinStages stages of 128 k) is cut along K into
// `splits` runs of `per` stages (each at least 8); otherwise splits = 1.
constexpr int kSplitMinStages = 16;
constexpr int kSplitMax = 8;
extern "C" int svdq_gemm_split_plan(int M, int N, int K, int precision, int* splits, int* per, size_t* bytes) {
  *splits = 1;
  *per = 0;
  *bytes = 0;
  if (precision != SVDQ_INT4) return 0;
  static int slots_of[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (slots_of[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 0;
    slots_of[dev] = 2 * cus;
  }
  const int slots = slots_of[dev];
  const int tiles = ((N + kTile - 1) / kTile) * ((M + kTile - 1) / kTile);
  const int S = (K / 64 + 1) / 2;
  if (2 * tiles > slots || S < kSplitMinStages) return 0;
  int sp = min(min(slots / tiles, S / 8), kSplitMax);
  if (sp < 2) return 0;
  const int p = (S + sp - 1) / sp;
  sp = (S + p - 1) / p;
  *splits = sp;
  *per = p;
  *bytes = static_cast<size_t>(sp) * static_cast<size_t>(tiles) * 4096 * sizeof(float4);
  return 0;
}

extern "C" int svdq_launch_gemm_w4a4_lora_up_ws(const uint8_t* xq, const void* xs, const uint8_t* wq, const void* ws,
                                                const float* lora_act, const void* lora_up, const void* bias, void* y,
                                                int M, int N, int K, int rank, int precision, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  int splits = 1, per = 0;
  size_t need = 0;
  svdq_gemm_split_plan(M, N, K, precision, &splits, &per, &need);
  if (splits < 2 || workspace == nullptr || workspace_bytes < need)
    return svdq_launch_gemm_w4a4_lora_up(xq, xs, wq, ws, lora_act, lora_up, bias, y, M, N, K, rank, precision, stream);
  const int tiles = ((N + kTile - 1) / kTile) * ((M + kTile - 1) / kTile);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float4* part = static_cast<float4*>(workspace);
  const SplitOut so{part, per};
  if (K >= kI4CoarseMinK)
    hipLaunchKernelGGL((k2_gemm_int4<false, kEpiPartial, true>), dim3(tiles, splits), dim3(kMxThreads), 0, st, xq,
                       static_cast<const uint16_t*>(xs), wq, static_cast<const uint16_t*>(ws), nullptr, nullptr,
                       nullptr, static_cast<uint16_t*>(y), M, N, K, 0, 0, 0, 0, 0, nullptr, MlpOut{}, so);
  else
    hipLaunchKernelGGL((k2_gemm_int4<false, kEpiPartial, false>), dim3(tiles, splits), dim3(kMxThreads), 0, st, xq,
                       static_cast<const uint16_t*>(xs), wq, static_cast<const uint16_t*>(ws), nullptr, nullptr,
                       nullptr, static_cast<uint16_t*>(y), M, N, K, 0, 0, 0, 0, 0, nullptr, MlpOut{}, so);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return static_cast<int>(e);
  hipLaunchKernelGGL(k_splitk_finish, dim3(tiles), dim3(kMxThreads), 0, st, part, splits, lora_act,
                     static_cast<const uint16_t*>(lora_up), static_cast<const uint16_t*>(bias),
                     static_cast<uint16_t*>(y), M, N, rank);
  return static_cast<int>(hipGetLastError());
}

extern "C" int svdq_launch_gemm_int4_gelu(const uint8_t* xq, const void* xs, const uint8_t* wq, const void* ws,
                                          const float* lora_act, const void* lora_up, const void* bias, void* y, int M,
                                          int N, int K, int rank, void* stream) {
  const int tiles = ((N + kTile - 1) / kTile) * ((M + kTile - 1) / kTile);
  hipLaunchKernelGGL((k2_gemm_int4<false, 1>), dim3(tiles), dim3(kMxThreads), 0, static_cast<hipStream_t>(stream), xq,
                     static_cast<const uint16_t*>(xs), wq, static_cast<const uint16_t*>(ws), lora_act,
                     static_cast<const uint16_t*>(lora_up), static_cast<const uint16_t*>(bias),
                     static_cast<uint16_t*>(y), M, N, K, rank, 0, 0, 0, 0, nullptr, MlpOut{}, SplitOut{});
  return static_cast<int>(hipGetLastError());
}

extern "C" int svdq_launch_mlp_gemm_gelu_quant(const uint8_t* xq, const void* xs, const uint8_t* wq, const void* ws,
                                               const float* lora_act, const void* lora_up, const void* bias, int M,
                                               int N, int K, int rank, const float* smooth_inv2,
                                               const void* lora_down2, int rank2, uint8_t* xq2, void* xs2,
                                               float* lora_act2, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rank2 > 0) {
    const size_t n = static_cast<size_t>(M) * rank2;
    hipLaunchKernelGGL(fill_zero_f32, dim3(static_cast<unsigned>((n / 4 + 255) / 256)), dim3(256), 0, st, lora_act2, n);
  }
  const int tiles = ((N + kTile - 1) / kTile) * ((M + kTile - 1) / kTile);
  const MlpOut mo{smooth_inv2, static_cast<const uint16_t*>(lora_down2), rank2, xq2, static_cast<uint16_t*>(xs2),
                  lora_act2};
  hipLaunchKernelGGL((k2_gemm_int4<false, 2>), dim3(tiles), dim3(kMxThreads), 0, st, xq,
                     static_cast<const uint16_t*>(xs), wq, static_cast<const uint16_t*>(ws), lora_act,
                     static_cast<const uint16_t*>(lora_up), static_cast<const uint16_t*>(bias), nullptr, M, N, K, rank,
                     0, 0, 0, 0, nullptr, mo, SplitOut{});
  return static_cast<int>(hipGetLastError());
}

extern "C" int svdq_launch_gemm_w4a16(const void* x, const uint8_t* wq, const void* ws, const void* bias, void* y,
                                      int M, int N, int K, void* stream) {
  const int tiles = ((N + kTile - 1) / kTile) * ((M + kTile - 1) / kTile);
  hipLaunchKernelGGL(k2_gemm_w4a16, dim3(tiles), dim3(kMxThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(x), wq, static_cast<const uint16_t*>(ws),
                     static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), M, N, K);
  return static_cast<int>(hipGetLastError());
}

extern "C" int svdq_launch_mfma_ceiling(int precision, int blocks, int iters, float* out, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (precision == SVDQ_MXFP4)
    hipLaunchKernelGGL(k_mfma_ceiling<1>, dim3(blocks), dim3(256), 0, st, iters, out);
  else
    hipLaunchKernelGGL(k_mfma_ceiling<0>, dim3(blocks), dim3(256), 0, st, iters, out);
  return static_cast<int>(hipGetLastError());
}

extern "C" int svdq_launch_unfused_linear(const void* x, int M, int K, const float* smooth_inv, const void* lora_down,
                                          int rank, const uint8_t* wq, const void* ws, const void* lora_up,
                                          const void* bias, int N, int precision, uint8_t* xq, void* xs,
                                          float* lora_act, void* y, void* stream) {
  if (precision != SVDQ_INT4) return static_cast<int>(hipErrorInvalidValue);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (rank / 16) {
#define SVDQ_UF_CASE(R) \
  case R:               \
    e = launch_unfused<R>(x, M, K, smooth_inv, lora_down, wq, ws, lora_up, bias, N, xq, xs, lora_act, y, st); \
    break;
    SVDQ_UF_CASE(0) SVDQ_UF_CASE(1) SVDQ_UF_CASE(2) SVDQ_UF_CASE(3) SVDQ_UF_CASE(4) SVDQ_UF_CASE(5)
    SVDQ_UF_CASE(6) SVDQ_UF_CASE(7) SVDQ_UF_CASE(8) SVDQ_UF_CASE(9) SVDQ_UF_CASE(10) SVDQ_UF_CASE(11)
    SVDQ_UF_CASE(12) SVDQ_UF_CASE(13) SVDQ_UF_CASE(14) SVDQ_UF_CASE(15) SVDQ_UF_CASE(16)
#undef SVDQ_UF_CASE
    default:
      return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(e);
}

extern "C" int svdq_launch_debug_group_partials(const uint8_t* xq, const uint8_t* wq, int M, int N, int K, int m0,
                                                int n0, int mt, int nt, int32_t* out, void* stream) {
  const int tiles = ((nt + kTile - 1) / kTile) * ((mt + kTile - 1) / kTile);
  hipLaunchKernelGGL(k2_gemm_int4<true>, dim3(tiles), dim3(kMxThreads), 0, static_cast<hipStream_t>(stream), xq,
                     nullptr, wq, nullptr, nullptr, nullptr, nullptr, nullptr, M, N, K, 0, m0, n0, mt, nt, out, MlpOut{},
                     SplitOut{});
  return static_cast<int>(hipGetLastError());
}

// ---------------------------------------------------------------------------
// The unfused layer without workspace arguments, for callers that cannot
// allocate: its intermediates (codes, scales, lora_act) live in one
// file-scope device array of kNoAllocScratchBytes, the same array for every
// call on a device.  Host code never uses the array's name as an address:
// the device address comes from hipGetSymbolAddress, taken once per device
// (with that device current) on the first call there, and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[svdq::kNoAllocScratchBytes];

namespace {

constexpr int kScratchDevices = 64;
void* g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mutex;

hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int svdq_launch_unfused_linear_noalloc(const void* x, int M, int K, const float* smooth_inv,
                                                  const void* lora_down, int rank, const uint8_t* wq, const void* ws,
                                                  const void* lora_up, const void* bias, int N, int precision, void* y,
                                                  void* stream) {
  void* base = nullptr;
  const hipError_t e = scratch_ptr(&base);
  if (e != hipSuccess) return static_cast<int>(e);
  size_t off[3];
  svdq::noalloc_layout(M, K, rank, off);
  uint8_t* b = static_cast<uint8_t*>(base);
  return svdq_launch_unfused_linear(x, M, K, smooth_inv, lora_down, rank, wq, ws, lora_up, bias, N, precision,
                                    b + off[0], b + off[1], rank > 0 ? reinterpret_cast<float*>(b + off[2]) : nullptr,
                                    y, stream);
}

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

#include "svdq_internal.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// number formats on the device
// ---------------------------------------------------------------------------

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_round(float f) {
  return __uint_as_float(bf16_rne_bits(f) << 16);
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

// two bf16 values that are exact in fp32 -> one packed dword (lo, hi)
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// fp32 -> packed bf16 pair with round to nearest even
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  return bf16_rne_bits(lo) | (bf16_rne_bits(hi) << 16);
}

// ---------------------------------------------------------------------------
// Kernel 1: smoothing + INT4 activation quantization + down projection.
//
// One workgroup = 4 waves over 16 rows and all of K.  A wave step covers the
// 16 rows x 4 groups of 64 k; lane l owns row l % 16 and group l / 16 of the
// step, so the group's absmax, scale and codes are lane-local.  The same
// bf16 X^ registers feed the bf16 MFMA with L1 (8 MFMAs of K = 32 per step
// and rank tile).  Waves take steps round-robin; their partial X^ L1 tiles
// are summed in LDS at the end (a fixed order, so the result is
// deterministic).
// ---------------------------------------------------------------------------

template <int RT>
__global__ __launch_bounds__(256) void k1_quant_down_int4(
    const uint16_t* __restrict__ x, int M, int K, const float* __restrict__ sinv,
    const uint16_t* __restrict__ ldown, uint8_t* __restrict__ xq, uint16_t* __restrict__ xs,
    float* __restrict__ lact) {
  constexpr int RANK = RT * 16;
  __shared__ float red[RT > 0 ? 4 * 16 * RANK : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int row = row0 + r16;
  const bool row_ok = row < M;
  const int G = K / 64;
  const int nsteps = (G + 3) / 4;

  v4f acc[RT > 0 ? RT : 1];
#pragma unroll
  for (int t = 0; t < (RT > 0 ? RT : 1); ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int step = wave; step < nsteps; step += 4) {
    const int g = step * 4 + q;
    const bool g_ok = g < G;
    const bool ok = row_ok && g_ok;
    const int k0 = g * 64;
    float v[64];
    if (ok) {
      const uint4* src = reinterpret_cast<const uint4*>(x + static_cast<size_t>(row) * K + k0);
      const float4* sp = reinterpret_cast<const float4*>(sinv + k0);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 w = src[c];
        const float4 s0 = sp[2 * c], s1 = sp[2 * c + 1];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(ws[e] << 16);
          const float hi = __uint_as_float(ws[e] & 0xFFFF0000u);
          v[8 * c + 2 * e] = bf16_round(lo * ss[2 * e]);
          v[8 * c + 2 * e + 1] = bf16_round(hi * ss[2 * e + 1]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = 0.f;
    }

    // per-group absmax -> fp16 scale -> codes
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t sbits = f16_sat_bits(__fdiv_rn(amax, 7.0f));
    const float s = f16_bits_to_f32(sbits);
    const float inv = (s == 0.f) ? 0.f : __fdiv_rn(1.0f, s);
    uint32_t packed[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float qf = __builtin_rintf(v[8 * c + e] * inv);
        qf = fminf(7.f, fmaxf(-7.f, qf));
        const int qi = static_cast<int>(qf);
        word |= (static_cast<uint32_t>(qi) & 0xFu) << (4 * e);
      }
      packed[c] = word;
    }
    if (ok) {
      uint4* dst = reinterpret_cast<uint4*>(xq + static_cast<size_t>(row) * (K / 2) + k0 / 2);
      dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
      xs[static_cast<size_t>(g) * M + row] = static_cast<uint16_t>(sbits);
    }

    if constexpr (RT > 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v4i araw;
        araw.x = static_cast<int>(pack_bf16_exact(v[8 * j + 0], v[8 * j + 1]));
        araw.y = static_cast<int>(pack_bf16_exact(v[8 * j + 2], v[8 * j + 3]));
        araw.z = static_cast<int>(pack_bf16_exact(v[8 * j + 4], v[8 * j + 5]));
        araw.w = static_cast<int>(pack_bf16_exact(v[8 * j + 6], v[8 * j + 7]));
        const v8bf a = __builtin_bit_cast(v8bf, araw);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          v4i braw = v4i{0, 0, 0, 0};
          if (g_ok) {
            braw = *reinterpret_cast<const v4i*>(ldown + static_cast<size_t>(t * 16 + r16) * K + k0 + 8 * j);
          }
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(v8bf, braw), acc[t], 0, 0, 0);
        }
      }
    }
  }

  if constexpr (RT > 0) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * q + i) * RANK + t * 16 + r16] = acc[t][i];
    __syncthreads();
    for (int e = threadIdx.x; e < 16 * RANK; e += 256) {
      const int rr = e / RANK;
      const float sum = ((red[e] + red[16 * RANK + e]) + red[2 * 16 * RANK + e]) + red[3 * 16 * RANK + e];
      if (row0 + rr < M) lact[static_cast<size_t>(row0 + rr) * RANK + (e - rr * RANK)] = sum;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: INT4 GEMM + per-group dequant + up projection + bias.
//
// Output tile 128 (n) x 128 (m) per workgroup of 4 waves; each wave owns a
// 64 x 64 sub-tile = 4 x 4 MFMA tiles.  The MFMA computes Y^T tiles (A = W
// codes, B = X codes) so that a lane ends up with 4 consecutive output
// channels of one token, which it stores as one 8-byte write.
//
// Per K-group of 64: the packed int4 tiles are read from global memory
// (16 B per thread per operand), unpacked to int8 with the x16 nibble trick
// ((w << 4) & 0xF0F0F0F0 holds 16*q of the even codes, w & 0xF0F0F0F0 16*q
// of the odd codes, both exact int8), written to LDS (double buffered) and
// fed to v_mfma_i32_16x16x64_i8.  Each MFMA returns 256 * P for the group,
// an exact int32; the 1/256 is folded into the activation scale, and the
// fp32 accumulator gets fma(float(256 P), s_w * s_x / 256, acc).  After the
// K loop the bf16 up projection runs on the same accumulators (MFMA srcC),
// then the bias is added and Y is rounded to bf16 and stored once.
// ---------------------------------------------------------------------------

constexpr int kTile = 128;      // output tile edge (both n and m)
constexpr int kLdsRow = 80;     // 64 bytes of int8 codes + 16 bytes padding

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

__device__ __forceinline__ void unpack_store(int8_t* dst, const uint4& w) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = (ws[i] << 4) & 0xF0F0F0F0u;
    o[2 * i + 1] = ws[i] & 0xF0F0F0F0u;
  }
  uint4* d = reinterpret_cast<uint4*>(dst);
  d[0] = make_uint4(o[0], o[1], o[2], o[3]);
  d[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

template <bool DEBUG>
__global__ __launch_bounds__(256, 2) void k2_gemm_int4(
    const uint8_t* __restrict__ xq, const uint16_t* __restrict__ xs,
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
    const float* __restrict__ lact, const uint16_t* __restrict__ lup,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int M, int N, int K, int rank,
    int win_m0, int win_n0, int win_mt, int win_nt, int32_t* __restrict__ dbg) {
  __shared__ __attribute__((aligned(16))) int8_t lds_w[2][kTile * kLdsRow];
  __shared__ __attribute__((aligned(16))) int8_t lds_x[2][kTile * kLdsRow];
  __shared__ __attribute__((aligned(16))) float lds_sw[2][kTile];
  __shared__ __attribute__((aligned(16))) float lds_sx[2][kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int wn = wave >> 1, wm = wave & 1;
  const int G = K / 64;
  const size_t rowb = static_cast<size_t>(K / 2);

  int n0, m0, row_lim_n, row_lim_m;
  if constexpr (DEBUG) {
    const int tiles_m = (win_mt + kTile - 1) / kTile;
    n0 = win_n0 + (blockIdx.x / tiles_m) * kTile;
    m0 = win_m0 + (blockIdx.x % tiles_m) * kTile;
  } else {
    const TileCoord tc = tile_coord(blockIdx.x, (N + kTile - 1) / kTile, (M + kTile - 1) / kTile);
    n0 = tc.n0;
    m0 = tc.m0;
  }
  row_lim_n = N;
  row_lim_m = M;

  // loader role: thread t moves 16 packed bytes of row t/2, half t%2
  const int lrow = tid >> 1, lhalf = tid & 1;
  const bool w_ok = n0 + lrow < row_lim_n;
  const bool x_ok = m0 + lrow < row_lim_m;
  const uint8_t* wsrc = wq + static_cast<size_t>(n0 + lrow) * rowb + lhalf * 16;
  const uint8_t* xsrc = xq + static_cast<size_t>(m0 + lrow) * rowb + lhalf * 16;
  // scale role: threads 0..127 move s_w of row n0+t, 128..255 s_x of m0+t-128
  const bool sc_is_w = tid < kTile;
  const int sc_i = sc_is_w ? tid : tid - kTile;
  const bool sc_ok = sc_is_w ? (n0 + sc_i < N) : (m0 + sc_i < M);
  const uint16_t* scsrc = sc_is_w ? (ws + n0 + sc_i) : (xs + m0 + sc_i);
  const size_t sc_stride = sc_is_w ? static_cast<size_t>(N) : static_cast<size_t>(M);

  uint4 wreg = make_uint4(0, 0, 0, 0), xreg = make_uint4(0, 0, 0, 0);
  float screg = 0.f;
  auto gload = [&](int g) {
    wreg = w_ok ? *reinterpret_cast<const uint4*>(wsrc + g * 32) : make_uint4(0, 0, 0, 0);
    xreg = x_ok ? *reinterpret_cast<const uint4*>(xsrc + g * 32) : make_uint4(0, 0, 0, 0);
    if constexpr (!DEBUG) screg = sc_ok ? f16_bits_to_f32(scsrc[static_cast<size_t>(g) * sc_stride]) : 0.f;
  };
  auto lstore = [&](int buf) {
    unpack_store(&lds_w[buf][lrow * kLdsRow + lhalf * 32], wreg);
    unpack_store(&lds_x[buf][lrow * kLdsRow + lhalf * 32], xreg);
    if (sc_is_w) lds_sw[buf][sc_i] = screg;
    else lds_sx[buf][sc_i] = screg * 0.00390625f;   // 1/256, exact
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    if (g + 1 < G) gload(g + 1);

    v4i a[4], b[4];
    v4f sw4[4];
    float sx1[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      a[it] = *reinterpret_cast<const v4i*>(&lds_w[buf][(wn * 64 + it * 16 + r16) * kLdsRow + q * 16]);
      sw4[it] = *reinterpret_cast<const v4f*>(&lds_sw[buf][wn * 64 + it * 16 + 4 * q]);
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      b[jt] = *reinterpret_cast<const v4i*>(&lds_x[buf][(wm * 64 + jt * 16 + r16) * kLdsRow + q * 16]);
      sx1[jt] = lds_sx[buf][wm * 64 + jt * 16 + r16];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[it], b[jt], v4i{0, 0, 0, 0}, 0, 0, 0);
        if constexpr (DEBUG) {
          const int m = m0 + wm * 64 + jt * 16 + r16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = n0 + wn * 64 + it * 16 + 4 * q + i;
            if (m < win_m0 + win_mt && n < win_n0 + win_nt) {
              dbg[(static_cast<size_t>(m - win_m0) * win_nt + (n - win_n0)) * G + g] = p[i] >> 8;
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float s = sw4[it][i] * sx1[jt];
            acc[it][jt][i] = __builtin_fmaf(static_cast<float>(p[i]), s, acc[it][jt][i]);
          }
        }
      }
    }
    if (g + 1 < G) lstore(buf ^ 1);
    __syncthreads();
  }

  if constexpr (!DEBUG) {
    // up projection: acc += bf16(lora_act) . L2 on the same tiles
    for (int c0 = 0; c0 < rank; c0 += 32) {
      const int j = c0 + 8 * q;          // this lane's 8 k-slots
      const bool j_ok = j < rank;
      v4i ua[4], ub[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int n = n0 + wn * 64 + it * 16 + r16;
        ua[it] = (j_ok && n < N) ? *reinterpret_cast<const v4i*>(lup + static_cast<size_t>(n) * rank + j)
                                 : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int m = m0 + wm * 64 + jt * 16 + r16;
        if (j_ok && m < M) {
          const float4* src = reinterpret_cast<const float4*>(lact + static_cast<size_t>(m) * rank + j);
          const float4 f0 = src[0], f1 = src[1];
          ub[jt] = v4i{static_cast<int>(pack_bf16_rne(f0.x, f0.y)), static_cast<int>(pack_bf16_rne(f0.z, f0.w)),
                       static_cast<int>(pack_bf16_rne(f1.x, f1.y)), static_cast<int>(pack_bf16_rne(f1.z, f1.w))};
        } else {
          ub[jt] = v4i{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
          acc[it][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, ua[it]),
                                                               __builtin_bit_cast(v8bf, ub[jt]), acc[it][jt], 0, 0, 0);
    }

    const bool vec_ok = (N % 4) == 0;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int nb = n0 + wn * 64 + it * 16 + 4 * q;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (nb + i < N) bv[i] = __uint_as_float(static_cast<uint32_t>(bias[nb + i]) << 16);
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int m = m0 + wm * 64 + jt * 16 + r16;
        if (m >= M) continue;
        uint16_t* dst = y + static_cast<size_t>(m) * N + nb;
        const uint32_t h0 = bf16_rne_bits(acc[it][jt][0] + bv[0]);
        const uint32_t h1 = bf16_rne_bits(acc[it][jt][1] + bv[1]);
        const uint32_t h2 = bf16_rne_bits(acc[it][jt][2] + bv[2]);
        const uint32_t h3 = bf16_rne_bits(acc[it][jt][3] + bv[3]);
        if (vec_ok && nb + 3 < N) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
        } else {
          const uint32_t hs[4] = {h0, h1, h2, h3};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (nb + i < N) dst[i] = static_cast<uint16_t>(hs[i]);
        }
      }
    }
  }
}

template <int RT>
hipError_t launch_k1(const void* x, int M, int K, const float* sinv, const void* ldown, uint8_t* xq, void* xs,
                     float* lact, hipStream_t st) {
  dim3 grid((M + 15) / 16), block(256);
  hipLaunchKernelGGL(k1_quant_down_int4<RT>, grid, block, 0, st, static_cast<const uint16_t*>(x), M, K, sinv,
                     static_cast<const uint16_t*>(ldown), xq, static_cast<uint16_t*>(xs), lact);
  return hipGetLastError();
}

}  // namespace

extern "C" int svdq_launch_quantize_act_lora_down(const void* x, int M, int K, const float* smooth_inv,
                                                  const void* lora_down, int rank, int precision, uint8_t* xq,
                                                  void* xs, float* lora_act, void* stream) {
  if (precision != SVDQ_INT4) return static_cast<int>(hipErrorInvalidValue);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (rank / 16) {
#define SVDQ_K1_CASE(R) \
  case R:               \
    e = launch_k1<R>(x, M, K, smooth_inv, lora_down, xq, xs, lora_act, st); \
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
  if (precision != SVDQ_INT4) return static_cast<int>(hipErrorInvalidValue);
  const int tiles = ((N + kTile - 1) / kTile) * ((M + kTile - 1) / kTile);
  hipLaunchKernelGGL(k2_gemm_int4<false>, dim3(tiles), dim3(256), 0, static_cast<hipStream_t>(stream), xq,
                     static_cast<const uint16_t*>(xs), wq, static_cast<const uint16_t*>(ws), lora_act,
                     static_cast<const uint16_t*>(lora_up), static_cast<const uint16_t*>(bias),
                     static_cast<uint16_t*>(y), M, N, K, rank, 0, 0, 0, 0, nullptr);
  return static_cast<int>(hipGetLastError());
}

extern "C" int svdq_launch_debug_group_partials(const uint8_t* xq, const uint8_t* wq, int M, int N, int K, int m0,
                                                int n0, int mt, int nt, int32_t* out, void* stream) {
  const int tiles = ((nt + kTile - 1) / kTile) * ((mt + kTile - 1) / kTile);
  hipLaunchKernelGGL(k2_gemm_int4<true>, dim3(tiles), dim3(256), 0, static_cast<hipStream_t>(stream), xq, nullptr,
                     wq, nullptr, nullptr, nullptr, nullptr, nullptr, M, N, K, 0, m0, n0, mt, nt, out);
  return static_cast<int>(hipGetLastError());
}

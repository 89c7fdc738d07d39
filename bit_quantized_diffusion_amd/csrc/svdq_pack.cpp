// Offline weight pack of the SVDQuant W4A4 layer, on the host CPU.
//
// Stage 2 of the "Overview of SVDQuant" caption (model card
// "svdq-int4-flux.1-dev") migrates activation outliers into the weights:
// W^ = diag(lambda) W.  Stage 3 splits W^ by SVD into a 16-bit low-rank
// branch L1 L2 and a residual R that is quantized to 4 bits.  No LAPACK is
// linked: the top-r singular subspace comes from block subspace iteration on
// the Gram matrix of the smaller side of W^, with a Rayleigh-Ritz step
// (cyclic Jacobi) each iteration.  Everything runs in fp64 until the factors
// are rounded to bf16.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <random>
#include <thread>
#include <vector>

#include "svdq_internal.h"

namespace svdq {

// ---------------------------------------------------------------------------
// host number formats
// ---------------------------------------------------------------------------

uint16_t f32_to_bf16_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  return static_cast<uint16_t>((u + 0x7FFFu + lsb) >> 16);
}

float bf16_bits_to_f32(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// fp32 -> fp16 bits, round to nearest even, finite values saturate to 65504,
// subnormal results kept.
uint16_t f32_to_f16_sat_bits(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax > 0x7F800000u) return static_cast<uint16_t>(sign | 0x7E00u);   // NaN
  if (ax == 0x7F800000u) return static_cast<uint16_t>(sign | 0x7C00u);  // inf stays inf
  const int e = static_cast<int>(ax >> 23) - 127;
  if (e > 15) return static_cast<uint16_t>(sign | 0x7BFFu);
  if (e >= -14) {
    const uint32_t mant = ax & 0x7FFFFFu;
    uint32_t h = (static_cast<uint32_t>(e + 15) << 10) | (mant >> 13);
    const uint32_t rem = mant & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1;
    if (h >= 0x7C00u) h = 0x7BFFu;
    return static_cast<uint16_t>(sign | h);
  }
  if (e < -25) return static_cast<uint16_t>(sign);
  const uint32_t mant = (ax & 0x7FFFFFu) | 0x800000u;  // value = mant * 2^(e-23)
  const int sh = -e - 1;                               // value * 2^24 = mant >> sh
  uint32_t m = mant >> sh;
  const uint32_t rem = mant & ((1u << sh) - 1u);
  const uint32_t half = 1u << (sh - 1);
  if (rem > half || (rem == half && (m & 1u))) m += 1;
  return static_cast<uint16_t>(sign | m);
}

float f16_bits_to_f32(uint16_t h) {
  const uint32_t sign = static_cast<uint32_t>(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu;
  const uint32_t m = h & 0x3FFu;
  float out;
  if (e == 0) {
    out = std::ldexp(static_cast<float>(m), -24);
    uint32_t u;
    std::memcpy(&u, &out, 4);
    u |= sign;
    std::memcpy(&out, &u, 4);
    return out;
  }
  uint32_t u;
  if (e == 31) {
    u = sign | 0x7F800000u | (m << 13);
  } else {
    u = sign | ((e - 15 + 127) << 23) | (m << 13);
  }
  std::memcpy(&out, &u, 4);
  return out;
}

// ---------------------------------------------------------------------------
// validation helpers (shared with the ABI translation unit)
// ---------------------------------------------------------------------------

int check_precision(int precision) {
  return (precision == SVDQ_INT4 || precision == SVDQ_MXFP4) ? SVDQ_OK : SVDQ_ERR_INVALID_ARG;
}

int check_k(int K, int precision) {
  if (K < 64) return SVDQ_ERR_SHAPE;
  if (precision == SVDQ_INT4 && K % kInt4Group != 0) return SVDQ_ERR_SHAPE;
  if (precision == SVDQ_MXFP4 && K % 128 != 0) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}

// The GEMM kernels address a 4-bit operand and its scale array with 32-bit
// byte offsets: rows * K/2 code bytes and (K / group) * rows scale bytes
// must stay below 2^31 (M or N up to ~349,000 at K = 12288).
int check_operand_extent(int rows, int K, int precision) {
  const long long codes = static_cast<long long>(rows) * (K / 2);
  const long long scales = precision == SVDQ_INT4 ? static_cast<long long>(K / kInt4Group) * rows * 2
                                                  : static_cast<long long>(K / kMxBlock) * rows;
  return (codes < (1LL << 31) && scales < (1LL << 31)) ? SVDQ_OK : SVDQ_ERR_SHAPE;
}

int check_rank(int rank, int K, int N) {
  if (rank < 0 || rank % 16 != 0 || rank > kMaxRank) return SVDQ_ERR_SHAPE;
  if (rank > std::min(K, N)) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}

int host_threads() {
  for (const char* name : {"SVDQ_NUM_THREADS", "OMP_NUM_THREADS"}) {
    const char* v = std::getenv(name);
    if (v && std::atoi(v) > 0) return std::min(64, std::atoi(v));
  }
  unsigned hc = std::thread::hardware_concurrency();
  return static_cast<int>(std::max(1u, std::min(64u, hc)));
}

namespace {

// Run body(i) for i in [0, n) over a small pool of threads (dynamic chunks).
void parallel_for(int64_t n, const std::function<void(int64_t)>& body, int64_t chunk = 1) {
  const int nt = static_cast<int>(std::min<int64_t>(host_threads(), (n + chunk - 1) / chunk));
  if (nt <= 1) {
    for (int64_t i = 0; i < n; ++i) body(i);
    return;
  }
  std::atomic<int64_t> next{0};
  auto worker = [&]() {
    for (;;) {
      const int64_t s = next.fetch_add(chunk);
      if (s >= n) break;
      const int64_t e = std::min(n, s + chunk);
      for (int64_t i = s; i < e; ++i) body(i);
    }
  };
  std::vector<std::thread> pool;
  pool.reserve(nt - 1);
  for (int t = 0; t < nt - 1; ++t) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
}

// G = A A^T for A [d][L] row-major (fp64); G is d x d, both triangles filled.
void gram(const double* A, int d, int64_t L, double* G) {
  constexpr int B = 32;
  const int nb = (d + B - 1) / B;
  std::vector<std::pair<int, int>> tiles;
  for (int bi = 0; bi < nb; ++bi)
    for (int bj = bi; bj < nb; ++bj) tiles.emplace_back(bi, bj);
  parallel_for(static_cast<int64_t>(tiles.size()), [&](int64_t t) {
    const int i0 = tiles[t].first * B, j0 = tiles[t].second * B;
    const int i1 = std::min(d, i0 + B), j1 = std::min(d, j0 + B);
    double acc[B][B];
    for (int i = 0; i < B; ++i)
      for (int j = 0; j < B; ++j) acc[i][j] = 0.0;
    constexpr int64_t C = 512;
    for (int64_t l0 = 0; l0 < L; l0 += C) {
      const int64_t l1 = std::min(L, l0 + C);
      for (int i = i0; i < i1; ++i) {
        const double* ai = A + static_cast<int64_t>(i) * L;
        for (int j = j0; j < j1; ++j) {
          const double* aj = A + static_cast<int64_t>(j) * L;
          double s0 = 0, s1 = 0, s2 = 0, s3 = 0;
          int64_t l = l0;
          for (; l + 4 <= l1; l += 4) {
            s0 += ai[l] * aj[l];
            s1 += ai[l + 1] * aj[l + 1];
            s2 += ai[l + 2] * aj[l + 2];
            s3 += ai[l + 3] * aj[l + 3];
          }
          for (; l < l1; ++l) s0 += ai[l] * aj[l];
          acc[i - i0][j - j0] += (s0 + s1) + (s2 + s3);
        }
      }
    }
    for (int i = i0; i < i1; ++i)
      for (int j = j0; j < j1; ++j) {
        G[static_cast<int64_t>(i) * d + j] = acc[i - i0][j - j0];
        G[static_cast<int64_t>(j) * d + i] = acc[i - i0][j - j0];
      }
  });
}

// Z[c][:] = G * Q[c][:] for b vectors stored as rows (Q, Z are [b][d]).
void sym_apply(const double* G, int d, const double* Q, int b, double* Z) {
  parallel_for(d, [&](int64_t i) {
    const double* gi = G + i * d;
    for (int c = 0; c < b; ++c) {
      const double* q = Q + static_cast<int64_t>(c) * d;
      double s0 = 0, s1 = 0;
      int k = 0;
      for (; k + 2 <= d; k += 2) {
        s0 += gi[k] * q[k];
        s1 += gi[k + 1] * q[k + 1];
      }
      for (; k < d; ++k) s0 += gi[k] * q[k];
      Z[static_cast<int64_t>(c) * d + i] = s0 + s1;
    }
  }, 16);
}

double dot(const double* a, const double* b, int n) {
  double s0 = 0, s1 = 0;
  int k = 0;
  for (; k + 2 <= n; k += 2) {
    s0 += a[k] * b[k];
    s1 += a[k + 1] * b[k + 1];
  }
  for (; k < n; ++k) s0 += a[k] * b[k];
  return s0 + s1;
}

// Modified Gram-Schmidt, applied twice, on b row vectors of length d.
// A vector that collapses is replaced by a fresh unit vector orthogonal to
// the previous ones (keeps the basis full when W^ is rank-deficient).
void orthonormalize(double* Q, int b, int d, std::mt19937_64& rng) {
  std::normal_distribution<double> nd;
  for (int c = 0; c < b; ++c) {
    double* v = Q + static_cast<int64_t>(c) * d;
    const double n0 = std::sqrt(dot(v, v, d));
    for (int tries = 0; tries < 4; ++tries) {
      for (int pass = 0; pass < 2; ++pass) {
        for (int p = 0; p < c; ++p) {
          const double* u = Q + static_cast<int64_t>(p) * d;
          const double h = dot(u, v, d);
          for (int k = 0; k < d; ++k) v[k] -= h * u[k];
        }
      }
      const double nrm = std::sqrt(dot(v, v, d));
      if (nrm > 1e-10 * std::max(n0, 1e-300) && nrm > 0) {
        for (int k = 0; k < d; ++k) v[k] /= nrm;
        break;
      }
      for (int k = 0; k < d; ++k) v[k] = nd(rng);
    }
  }
}

// Cyclic Jacobi eigen-decomposition of a symmetric n x n matrix H (row-major,
// destroyed).  On return evals[i] and the columns of V (row-major n x n) are
// sorted by decreasing eigenvalue.
void jacobi_eig(std::vector<double>& H, int n, std::vector<double>& evals, std::vector<double>& V) {
  V.assign(static_cast<size_t>(n) * n, 0.0);
  for (int i = 0; i < n; ++i) V[static_cast<size_t>(i) * n + i] = 1.0;
  auto at = [&](int i, int j) -> double& { return H[static_cast<size_t>(i) * n + j]; };
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0, diag = 0;
    for (int i = 0; i < n; ++i) {
      diag += at(i, i) * at(i, i);
      for (int j = i + 1; j < n; ++j) off += at(i, j) * at(i, j);
    }
    if (off <= 1e-30 * diag || off == 0) break;
    for (int p = 0; p < n - 1; ++p) {
      for (int q = p + 1; q < n; ++q) {
        const double apq = at(p, q);
        if (std::fabs(apq) < 1e-300) continue;
        const double app = at(p, p), aqq = at(q, q);
        const double theta = (aqq - app) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < n; ++k) {
          const double hkp = at(k, p), hkq = at(k, q);
          at(k, p) = c * hkp - s * hkq;
          at(k, q) = s * hkp + c * hkq;
        }
        for (int k = 0; k < n; ++k) {
          const double hpk = at(p, k), hqk = at(q, k);
          at(p, k) = c * hpk - s * hqk;
          at(q, k) = s * hpk + c * hqk;
        }
        for (int k = 0; k < n; ++k) {
          double& vkp = V[static_cast<size_t>(k) * n + p];
          double& vkq = V[static_cast<size_t>(k) * n + q];
          const double a = vkp, b2 = vkq;
          vkp = c * a - s * b2;
          vkq = s * a + c * b2;
        }
      }
    }
  }
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::sort(order.begin(), order.end(), [&](int a, int b) { return at(a, a) > at(b, b); });
  evals.resize(n);
  std::vector<double> Vs(static_cast<size_t>(n) * n);
  for (int c = 0; c < n; ++c) {
    evals[c] = at(order[c], order[c]);
    for (int k = 0; k < n; ++k) Vs[static_cast<size_t>(k) * n + c] = V[static_cast<size_t>(k) * n + order[c]];
  }
  V.swap(Vs);
}

// Top-r eigenpairs of the d x d symmetric PSD matrix G.  Returns r eigen
// vectors as rows of U ([r][d]) and their eigenvalues.  With the environment
// variable SVDQ_PACK_STATS=1 the iteration count goes to stderr.
void top_eigs(const double* G, int d, int r, std::vector<double>& U, std::vector<double>& evals) {
  const int b = std::min(d, r + std::max(16, r / 2));
  std::mt19937_64 rng(0x5D0C7E11u);
  std::normal_distribution<double> nd;
  std::vector<double> Q(static_cast<size_t>(b) * d), Z(static_cast<size_t>(b) * d);
  for (auto& v : Q) v = nd(rng);
  orthonormalize(Q.data(), b, d, rng);
  std::vector<double> H(static_cast<size_t>(b) * b), S, theta;
  double prev = -1;
  for (int it = 0; it < 3000; ++it) {
    sym_apply(G, d, Q.data(), b, Z.data());
    // Rayleigh quotient H = Q^T G Q
    for (int i = 0; i < b; ++i)
      for (int j = i; j < b; ++j) {
        const double h = dot(Q.data() + static_cast<int64_t>(i) * d, Z.data() + static_cast<int64_t>(j) * d, d);
        H[static_cast<size_t>(i) * b + j] = h;
        H[static_cast<size_t>(j) * b + i] = h;
      }
    jacobi_eig(H, b, theta, S);
    double captured = 0;
    for (int i = 0; i < r; ++i) captured += std::max(theta[i], 0.0);
    const bool done = it >= 8 && std::fabs(captured - prev) <= 1e-13 * std::max(captured, 1e-300);
    prev = captured;
    if (done || it == 2999) {
      if (const char* e = std::getenv("SVDQ_PACK_STATS"); e && e[0] == '1')
        std::fprintf(stderr, "svdq_pack: Gram order %d, rank %d, block %d, %d subspace iterations\n", d, r, b, it + 1);
      // Ritz vectors of the current basis: U = S^T Q (rows)
      U.assign(static_cast<size_t>(r) * d, 0.0);
      for (int c = 0; c < r; ++c) {
        double* u = U.data() + static_cast<int64_t>(c) * d;
        for (int j = 0; j < b; ++j) {
          const double w = S[static_cast<size_t>(j) * b + c];
          const double* q = Q.data() + static_cast<int64_t>(j) * d;
          for (int k = 0; k < d; ++k) u[k] += w * q[k];
        }
      }
      evals.assign(theta.begin(), theta.begin() + r);
      return;
    }
    // power step on the rotated basis: Q = orth(Z S)
    parallel_for(d, [&](int64_t k) {
      double tmp[512];
      double* t = b <= 512 ? tmp : nullptr;
      std::vector<double> heap;
      if (!t) {
        heap.resize(b);
        t = heap.data();
      }
      for (int c = 0; c < b; ++c) {
        double s = 0;
        for (int j = 0; j < b; ++j) s += Z[static_cast<size_t>(j) * d + k] * S[static_cast<size_t>(j) * b + c];
        t[c] = s;
      }
      for (int c = 0; c < b; ++c) Q[static_cast<size_t>(c) * d + k] = t[c];
    }, 64);
    orthonormalize(Q.data(), b, d, rng);
  }
}

// --------------------------- quantizers ------------------------------------

// Code layout of the INT4 codes: units of 16 consecutive k in two
// little-endian 32-bit words.  Code q has the 6-bit image 32 [q < 0] + |q|
// (the FP6 E2M3 pattern of q/8); image j of a unit sits at bits 6j..6j+5 of
// the 96-bit string D0 | D1 << 32 | D2 << 64, and the unit is stored as
// I0 = D0 | (D2 & 0x18618618), I1 = D1 | (D2 & 0x86186186): the two masks
// are the always-zero bits 3-4 of the images in D0 and D1, which together
// are exactly the data bits of D2.  n codes (n % 16 == 0) -> n / 2 bytes.
void pack_int4_units(const int* q, int n, uint8_t* out) {
  for (int u = 0; u < n / 16; ++u) {
    uint32_t d[3] = {0, 0, 0};
    for (int j = 0; j < 16; ++j) {
      const int c = q[16 * u + j];
      const uint32_t f = c < 0 ? 32u + static_cast<uint32_t>(-c) : static_cast<uint32_t>(c);
      const int bit = 6 * j, w = bit / 32, o = bit % 32;
      d[w] |= f << o;
      if (o + 6 > 32) d[w + 1] |= f >> (32 - o);
    }
    const uint32_t i0 = d[0] | (d[2] & 0x18618618u), i1 = d[1] | (d[2] & 0x86186186u);
    for (int b = 0; b < 4; ++b) {
      out[8 * u + b] = static_cast<uint8_t>(i0 >> (8 * b));
      out[8 * u + 4 + b] = static_cast<uint8_t>(i1 >> (8 * b));
    }
  }
}

void quant_int4_row(const float* v, int K, uint8_t* q_packed, uint16_t* scale_bits, int64_t scale_stride) {
  for (int g = 0; g < K / kInt4Group; ++g) {
    const float* gv = v + g * kInt4Group;
    float amax = 0.0f;
    for (int i = 0; i < kInt4Group; ++i) amax = std::max(amax, std::fabs(gv[i]));
    const uint16_t sb = f32_to_f16_sat_bits(amax / 7.0f);
    scale_bits[g * scale_stride] = sb;
    const float s = f16_bits_to_f32(sb);
    uint8_t* out = q_packed + g * (kInt4Group / 2);
    if (s == 0.0f) {
      std::memset(out, 0, kInt4Group / 2);
      continue;
    }
    const float inv = 1.0f / s;
    int q[kInt4Group];
    for (int i = 0; i < kInt4Group; ++i)
      q[i] = std::min(7, std::max(-7, static_cast<int>(std::nearbyint(gv[i] * inv))));
    pack_int4_units(q, kInt4Group, out);
  }
}

uint8_t e2m1_code(double a) {
  if (a <= 0.25) return 0;
  if (a < 0.75) return 1;
  if (a <= 1.25) return 2;
  if (a < 1.75) return 3;
  if (a <= 2.5) return 4;
  if (a < 3.5) return 5;
  if (a <= 5.0) return 6;
  return 7;
}

void quant_mxfp4_row(const float* v, int K, uint8_t* q_packed, uint8_t* scale_bytes, int64_t scale_stride) {
  for (int g = 0; g < K / kMxBlock; ++g) {
    const float* gv = v + g * kMxBlock;
    float amax = 0.0f;
    for (int i = 0; i < kMxBlock; ++i) amax = std::max(amax, std::fabs(gv[i]));
    uint8_t* out = q_packed + g * (kMxBlock / 2);
    if (amax == 0.0f) {
      scale_bytes[g * scale_stride] = 0;
      std::memset(out, 0, kMxBlock / 2);
      continue;
    }
    uint32_t bits;
    std::memcpy(&bits, &amax, 4);
    int e = static_cast<int>((bits >> 23) & 0xFFu) - 127 - 2;
    e = std::min(127, std::max(-127, e));
    scale_bytes[g * scale_stride] = static_cast<uint8_t>(e + 127);
    for (int i = 0; i < kMxBlock; i += 2) {
      uint8_t c[2];
      for (int h = 0; h < 2; ++h) {
        const double sv = std::ldexp(static_cast<double>(gv[i + h]), -e);
        uint8_t m = e2m1_code(std::fabs(sv));
        if (sv < 0 && m) m |= 8;
        c[h] = m;
      }
      out[i / 2] = static_cast<uint8_t>(c[0] | (c[1] << 4));
    }
  }
}

}  // namespace
}  // namespace svdq

using namespace svdq;

extern "C" int svdq_pack_weights(const uint16_t* w_bf16, const float* act_absmax, int K, int N, int rank,
                                 int precision, float* smooth_inv, uint16_t* lora_down, uint16_t* lora_up,
                                 uint8_t* wq, void* ws, float* r_out) {
  int st = check_precision(precision);
  if (st) return st;
  if (!w_bf16 || !act_absmax || !smooth_inv || !wq || !ws) return SVDQ_ERR_INVALID_ARG;
  if (N < 1) return SVDQ_ERR_SHAPE;
  if ((st = check_k(K, precision))) return st;
  if ((st = check_rank(rank, K, N))) return st;
  if (rank > 0 && (!lora_down || !lora_up)) return SVDQ_ERR_INVALID_ARG;

  const int64_t KN = static_cast<int64_t>(K) * N;
  // -- stage 2: smoothing --------------------------------------------------
  std::vector<double> aw(K, 0.0);
  for (int n = 0; n < N; ++n) {
    const uint16_t* row = w_bf16 + static_cast<int64_t>(n) * K;
    for (int j = 0; j < K; ++j) aw[j] = std::max(aw[j], static_cast<double>(std::fabs(bf16_bits_to_f32(row[j]))));
  }
  std::vector<double> sinv64(K);
  for (int j = 0; j < K; ++j) {
    const double ax = static_cast<double>(act_absmax[j]);
    const double lam = std::sqrt(std::max(ax, 1e-5)) / std::sqrt(std::max(aw[j], 1e-5));
    smooth_inv[j] = static_cast<float>(1.0 / lam);
    sinv64[j] = static_cast<double>(smooth_inv[j]);
  }
  // W^ [K][N] (math layout), fp64
  std::vector<double> what(KN);
  parallel_for(K, [&](int64_t j) {
    for (int n = 0; n < N; ++n)
      what[j * N + n] = static_cast<double>(bf16_bits_to_f32(w_bf16[static_cast<int64_t>(n) * K + j])) / sinv64[j];
  }, 16);

  // -- stage 3: top-r SVD --------------------------------------------------
  std::vector<float> l1f(static_cast<size_t>(K) * rank), l2f(static_cast<size_t>(rank) * N);  // bf16-rounded, as fp32
  if (rank > 0) {
    const bool rows_small = K <= N;           // Gram of the smaller side
    const int d = rows_small ? K : N;
    const int64_t L = rows_small ? N : K;
    std::vector<double> At;
    const double* A = what.data();
    if (!rows_small) {
      At.resize(KN);
      parallel_for(N, [&](int64_t n) {
        for (int j = 0; j < K; ++j) At[n * K + j] = what[static_cast<int64_t>(j) * N + n];
      }, 16);
      A = At.data();
    }
    std::vector<double> G(static_cast<size_t>(d) * d);
    gram(A, d, L, G.data());
    std::vector<double> U, ev;
    top_eigs(G.data(), d, rank, U, ev);
    G.clear();
    G.shrink_to_fit();
    // P = U A  ([r][L]): the projections of A's columns on the eigenvectors
    std::vector<double> P(static_cast<size_t>(rank) * L, 0.0);
    parallel_for(rank, [&](int64_t c) {
      const double* u = U.data() + c * d;
      double* p = P.data() + c * L;
      for (int i = 0; i < d; ++i) {
        const double ui = u[i];
        const double* a = A + static_cast<int64_t>(i) * L;
        for (int64_t l = 0; l < L; ++l) p[l] += ui * a[l];
      }
    });
    for (int c = 0; c < rank; ++c) {
      const double sig = std::sqrt(std::max(ev[c], 0.0));
      const double* u = U.data() + static_cast<int64_t>(c) * d;
      const double* p = P.data() + static_cast<int64_t>(c) * L;
      const bool live = sig > 0.0;
      if (rows_small) {
        // W^ = U S V^T with U over K: L1 = U S, L2 = V^T = P / sigma
        for (int j = 0; j < K; ++j) l1f[static_cast<size_t>(j) * rank + c] = bf16_bits_to_f32(f32_to_bf16_bits(static_cast<float>(u[j] * sig)));
        for (int n = 0; n < N; ++n) l2f[static_cast<size_t>(c) * N + n] = live ? bf16_bits_to_f32(f32_to_bf16_bits(static_cast<float>(p[n] / sig))) : 0.0f;
      } else {
        // eigenvectors over N: L2 = V^T = u, L1 = W^ V = P^T
        for (int n = 0; n < N; ++n) l2f[static_cast<size_t>(c) * N + n] = bf16_bits_to_f32(f32_to_bf16_bits(static_cast<float>(u[n])));
        for (int j = 0; j < K; ++j) l1f[static_cast<size_t>(j) * rank + c] = bf16_bits_to_f32(f32_to_bf16_bits(static_cast<float>(p[j])));
      }
    }
    for (int c = 0; c < rank; ++c) {
      for (int j = 0; j < K; ++j) lora_down[static_cast<int64_t>(c) * K + j] = f32_to_bf16_bits(l1f[static_cast<size_t>(j) * rank + c]);
      for (int n = 0; n < N; ++n) lora_up[static_cast<int64_t>(n) * rank + c] = f32_to_bf16_bits(l2f[static_cast<size_t>(c) * N + n]);
    }
  }

  // -- residual R = fp32(W^ - L1 L2), then its 4-bit codes per output channel
  std::vector<float> rT(KN);   // [N][K]
  parallel_for(K, [&](int64_t j) {
    const float* l1row = l1f.data() + j * rank;
    for (int n = 0; n < N; ++n) {
      double low = 0.0;
      for (int c = 0; c < rank; ++c) low += static_cast<double>(l1row[c]) * static_cast<double>(l2f[static_cast<size_t>(c) * N + n]);
      const float r = static_cast<float>(what[j * N + n] - low);
      rT[static_cast<int64_t>(n) * K + j] = r;
      if (r_out) r_out[j * N + n] = r;
    }
  }, 8);
  if (precision == SVDQ_INT4) {
    uint16_t* wsb = static_cast<uint16_t*>(ws);
    parallel_for(N, [&](int64_t n) {
      quant_int4_row(rT.data() + n * K, K, wq + n * (K / 2), wsb + n, N);
    }, 16);
  } else {
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    parallel_for(N, [&](int64_t n) {
      quant_mxfp4_row(rT.data() + n * K, K, wq + n * (K / 2), wsb + n, N);
    }, 16);
  }
  return SVDQ_OK;
}

// Off-the-shelf LoRA merged into the 16-bit branch without re-quantizing
// the residual (SVDQuant abstract: the engine supports low-rank adapters
// without re-quantization).  The branch reads X^ = X diag(smooth_inv), so
// the adapter's down factor is folded with 1/smooth_inv:
// L1' = [L1 | A diag(1/smooth_inv)], L2' = [L2 ; B]; then X^ L1' L2' =
// X^ L1 L2 + X A B.  Each folded element is a[k][j] / smooth_inv[k] in fp64,
// rounded to fp32 and then to bf16 (nearest even).
extern "C" int svdq_merge_lora(const uint16_t* lora_down, const uint16_t* lora_up, int rank,
                               const float* smooth_inv, const uint16_t* a, const uint16_t* b, int lora_rank, int K,
                               int N, uint16_t* lora_down_out, uint16_t* lora_up_out) {
  if (!smooth_inv || !a || !b || !lora_down_out || !lora_up_out) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_down || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (K < 1 || N < 1 || lora_rank < 1 || rank < 0) return SVDQ_ERR_SHAPE;
  int st;
  if ((st = check_rank(rank, K, N))) return st;
  if ((st = check_rank(rank + lora_rank, K, N))) return st;
  const int r2 = rank + lora_rank;
  const int64_t k64 = K;
  // L1'^T = [L1^T ; (A diag(1/smooth_inv))^T]: rows 0..rank-1 copied
  if (rank > 0) std::memcpy(lora_down_out, lora_down, sizeof(uint16_t) * static_cast<size_t>(rank) * K);
  for (int j = 0; j < lora_rank; ++j) {
    uint16_t* dst = lora_down_out + static_cast<int64_t>(rank + j) * k64;
    for (int k = 0; k < K; ++k) {
      const double v = static_cast<double>(bf16_bits_to_f32(a[static_cast<int64_t>(k) * lora_rank + j])) /
                       static_cast<double>(smooth_inv[k]);
      dst[k] = f32_to_bf16_bits(static_cast<float>(v));
    }
  }
  // L2'^T [N][r2] = [L2^T | B^T]
  for (int n = 0; n < N; ++n) {
    uint16_t* dst = lora_up_out + static_cast<int64_t>(n) * r2;
    for (int c = 0; c < rank; ++c) dst[c] = lora_up[static_cast<int64_t>(n) * rank + c];
    for (int j = 0; j < lora_rank; ++j) dst[rank + j] = b[static_cast<int64_t>(j) * N + n];
  }
  return SVDQ_OK;
}

// W4A16 comparison layer: the weights quantized with the layer's INT4 rule
// per output channel in groups of 64 along K, with no smoothing and no
// low-rank branch (the 4-bit weight-only baseline the SVDQuant abstract
// measures W4A4 against).
extern "C" int svdq_pack_w4a16(const uint16_t* w_bf16, int K, int N, uint8_t* wq, void* ws) {
  if (!w_bf16 || !wq || !ws) return SVDQ_ERR_INVALID_ARG;
  if (N < 1) return SVDQ_ERR_SHAPE;
  int st;
  if ((st = check_k(K, SVDQ_INT4))) return st;
  uint16_t* wsb = static_cast<uint16_t*>(ws);
  parallel_for(N, [&](int64_t n) {
    std::vector<float> row(K);
    for (int k = 0; k < K; ++k) row[k] = bf16_bits_to_f32(w_bf16[n * K + k]);
    quant_int4_row(row.data(), K, wq + n * (K / 2), wsb + n, N);
  }, 16);
  return SVDQ_OK;
}

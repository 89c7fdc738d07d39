// C ABI entry points of libsvdq.so: argument and device validation, then the
// kernel launchers.  Nothing here throws; every failure is a status code.
//
// The device check follows the "Hardware support" section of the blog
// "Nunchaku 4-bit inference in Diffusers": the capability of the GPU is
// checked when the layer is used and an unsupported GPU gets a clear error
// instead of wrong output.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "svdq_internal.h"

using namespace svdq;

static_assert(kNoAllocScratchBytes == SVDQ_NOALLOC_SCRATCH_BYTES, "scratch size of the header and the library agree");

namespace {

constexpr int kMaxDevices = 64;
// 0 = not probed yet, 1 = gfx950, 2 = not usable
std::atomic<int> g_dev_state[kMaxDevices];
std::mutex g_dev_mutex;

int probe_device(int device) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return SVDQ_ERR_UNSUPPORTED_DEVICE;
  if (device < 0 || device >= count || device >= kMaxDevices) return SVDQ_ERR_UNSUPPORTED_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return SVDQ_ERR_UNSUPPORTED_DEVICE;
  return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? SVDQ_OK : SVDQ_ERR_UNSUPPORTED_DEVICE;
}

int current_device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return SVDQ_ERR_UNSUPPORTED_DEVICE;
  }
  return svdq_device_check(dev);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(int e) { return e == 0 ? SVDQ_OK : SVDQ_ERR_HIP; }

}  // namespace

extern "C" {

int svdq_version(void) { return 100; }

const char* svdq_status_string(int status) {
  switch (status) {
    case SVDQ_OK: return "svdq: ok";
    case SVDQ_ERR_INVALID_ARG: return "svdq: invalid argument (NULL or misaligned pointer, or unknown precision)";
    case SVDQ_ERR_SHAPE: return "svdq: unsupported shape (check M, N >= 1, K and rank rules)";
    case SVDQ_ERR_UNSUPPORTED_DEVICE: return "svdq: no usable gfx950 (MI355X) device; the 4-bit kernels need gfx950";
    case SVDQ_ERR_HIP: return "svdq: HIP runtime error (launch failed)";
    default: return "svdq: unknown status";
  }
}

int svdq_device_check(int device) {
  if (device < 0 || device >= kMaxDevices) return SVDQ_ERR_UNSUPPORTED_DEVICE;
  int s = g_dev_state[device].load(std::memory_order_acquire);
  if (s == 0) {
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    s = g_dev_state[device].load(std::memory_order_relaxed);
    if (s == 0) {
      s = probe_device(device) == SVDQ_OK ? 1 : 2;
      (void)hipGetLastError();
      g_dev_state[device].store(s, std::memory_order_release);
    }
  }
  return s == 1 ? SVDQ_OK : SVDQ_ERR_UNSUPPORTED_DEVICE;
}

int svdq_packed_sizes(int K, int N, int rank, int precision, size_t* out) {
  int st = check_precision(precision);
  if (st) return st;
  if (!out) return SVDQ_ERR_INVALID_ARG;
  if (N < 1) return SVDQ_ERR_SHAPE;
  if ((st = check_k(K, precision))) return st;
  if ((st = check_rank(rank, K, N))) return st;
  const size_t k = static_cast<size_t>(K), n = static_cast<size_t>(N), r = static_cast<size_t>(rank);
  out[0] = k * 4;
  out[1] = r * k * 2;
  out[2] = n * r * 2;
  out[3] = n * k / 2;
  out[4] = precision == SVDQ_INT4 ? (k / kInt4Group) * n * 2 : (k / kMxBlock) * n;
  return SVDQ_OK;
}

int svdq_act_sizes(int M, int K, int rank, int precision, size_t* out) {
  int st = check_precision(precision);
  if (st) return st;
  if (!out) return SVDQ_ERR_INVALID_ARG;
  if (M < 1) return SVDQ_ERR_SHAPE;
  if ((st = check_k(K, precision))) return st;
  if ((st = check_rank(rank, K, K))) return st;
  const size_t m = static_cast<size_t>(M), k = static_cast<size_t>(K), r = static_cast<size_t>(rank);
  out[0] = m * k / 2;
  out[1] = precision == SVDQ_INT4 ? (k / kInt4Group) * m * 2 : (k / kMxBlock) * m;
  out[2] = m * r * 4;
  return SVDQ_OK;
}

int svdq_quantize_act_lora_down(const void* x, int M, int K, const float* smooth_inv, const void* lora_down,
                                int rank, int precision, uint8_t* xq, void* xs, float* lora_act, void* stream) {
  int st = check_precision(precision);
  if (st) return st;
  if (!x || !smooth_inv || !xq || !xs) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_down || !lora_act)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(smooth_inv) || !aligned16(xq) || !aligned16(xs)) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!aligned16(lora_down) || !aligned16(lora_act))) return SVDQ_ERR_INVALID_ARG;
  if (M < 1) return SVDQ_ERR_SHAPE;
  if ((st = check_k(K, precision))) return st;
  if ((st = check_rank(rank, K, K))) return st;
  if ((st = current_device_ok())) return st;
  return hip_status(svdq_launch_quantize_act_lora_down(x, M, K, smooth_inv, lora_down, rank, precision, xq, xs,
                                                       lora_act, stream));
}

int svdq_gemm_w4a4_lora_up(const uint8_t* xq, const void* xs, const uint8_t* wq, const void* ws,
                           const float* lora_act, const void* lora_up, const void* bias, void* y, int M, int N,
                           int K, int rank, int precision, void* stream) {
  int st = check_precision(precision);
  if (st) return st;
  if (!xq || !xs || !wq || !ws || !y) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(wq) || !aligned16(ws) || !aligned16(y))
    return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!aligned16(lora_act) || !aligned16(lora_up))) return SVDQ_ERR_INVALID_ARG;
  if (bias && !aligned16(bias)) return SVDQ_ERR_INVALID_ARG;
  if (M < 1 || N < 1) return SVDQ_ERR_SHAPE;
  if ((st = check_k(K, precision))) return st;
  if ((st = check_rank(rank, K, N))) return st;
  if ((st = check_operand_extent(M, K, precision)) || (st = check_operand_extent(N, K, precision))) return st;
  if ((st = current_device_ok())) return st;
  return hip_status(svdq_launch_gemm_w4a4_lora_up(xq, xs, wq, ws, lora_act, lora_up, bias, y, M, N, K, rank,
                                                  precision, stream));
}

int svdq_gemm_workspace_size(int M, int N, int K, int precision, size_t* out_bytes) {
  int st = check_precision(precision);
  if (st) return st;
  if (!out_bytes) return SVDQ_ERR_INVALID_ARG;
  *out_bytes = 0;
  if (M < 1 || N < 1) return SVDQ_ERR_SHAPE;
  if ((st = check_k(K, precision))) return st;
  if ((st = check_operand_extent(M, K, precision)) || (st = check_operand_extent(N, K, precision))) return st;
  if ((st = current_device_ok())) return st;
  int splits = 1, per = 0;
  svdq_gemm_split_plan(M, N, K, precision, &splits, &per, out_bytes);
  return SVDQ_OK;
}

int svdq_gemm_w4a4_lora_up_ws(const uint8_t* xq, const void* xs, const uint8_t* wq, const void* ws,
                              const float* lora_act, const void* lora_up, const void* bias, void* y, int M, int N,
                              int K, int rank, int precision, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_precision(precision);
  if (st) return st;
  if (!xq || !xs || !wq || !ws || !y) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(wq) || !aligned16(ws) || !aligned16(y))
    return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!aligned16(lora_act) || !aligned16(lora_up))) return SVDQ_ERR_INVALID_ARG;
  if (bias && !aligned16(bias)) return SVDQ_ERR_INVALID_ARG;
  if (workspace && !aligned16(workspace)) return SVDQ_ERR_INVALID_ARG;
  if (M < 1 || N < 1) return SVDQ_ERR_SHAPE;
  if ((st = check_k(K, precision))) return st;
  if ((st = check_rank(rank, K, N))) return st;
  if ((st = check_operand_extent(M, K, precision)) || (st = check_operand_extent(N, K, precision))) return st;
  if ((st = current_device_ok())) return st;
  return hip_status(svdq_launch_gemm_w4a4_lora_up_ws(xq, xs, wq, ws, lora_act, lora_up, bias, y, M, N, K, rank,
                                                     precision, workspace, workspace_bytes, stream));
}

int svdq_gemm_w4a4_lora_up_gelu(const uint8_t* xq, const void* xs, const uint8_t* wq, const void* ws,
                                const float* lora_act, const void* lora_up, const void* bias, void* y, int M, int N,
                                int K, int rank, int precision, void* stream) {
  int st = check_precision(precision);
  if (st) return st;
  if (precision != SVDQ_INT4) return SVDQ_ERR_INVALID_ARG;
  if (!xq || !xs || !wq || !ws || !y) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(wq) || !aligned16(ws) || !aligned16(y))
    return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!aligned16(lora_act) || !aligned16(lora_up))) return SVDQ_ERR_INVALID_ARG;
  if (bias && !aligned16(bias)) return SVDQ_ERR_INVALID_ARG;
  if (M < 1 || N < 1) return SVDQ_ERR_SHAPE;
  if ((st = check_k(K, precision))) return st;
  if ((st = check_rank(rank, K, N))) return st;
  if ((st = check_operand_extent(M, K, precision)) || (st = check_operand_extent(N, K, precision))) return st;
  if ((st = current_device_ok())) return st;
  return hip_status(svdq_launch_gemm_int4_gelu(xq, xs, wq, ws, lora_act, lora_up, bias, y, M, N, K, rank, stream));
}

int svdq_mlp_gemm_gelu_quant(const uint8_t* xq, const void* xs, const uint8_t* wq, const void* ws,
                             const float* lora_act, const void* lora_up, const void* bias, int M, int N, int K,
                             int rank, const float* smooth_inv2, const void* lora_down2, int rank2, int precision,
                             uint8_t* xq2, void* xs2, float* lora_act2, void* stream) {
  int st = check_precision(precision);
  if (st) return st;
  if (precision != SVDQ_INT4) return SVDQ_ERR_INVALID_ARG;
  if (!xq || !xs || !wq || !ws || !smooth_inv2 || !xq2 || !xs2) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (rank2 > 0 && (!lora_down2 || !lora_act2)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(wq) || !aligned16(ws) || !aligned16(smooth_inv2) ||
      !aligned16(xq2) || !aligned16(xs2))
    return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!aligned16(lora_act) || !aligned16(lora_up))) return SVDQ_ERR_INVALID_ARG;
  if (rank2 > 0 && (!aligned16(lora_down2) || !aligned16(lora_act2))) return SVDQ_ERR_INVALID_ARG;
  if (bias && !aligned16(bias)) return SVDQ_ERR_INVALID_ARG;
  if (M < 1 || N < 128 || N % 128 != 0) return SVDQ_ERR_SHAPE;
  if ((st = check_k(K, precision))) return st;
  if ((st = check_rank(rank, K, N))) return st;
  if ((st = check_rank(rank2, N, N))) return st;
  if ((st = check_operand_extent(M, K, precision)) || (st = check_operand_extent(N, K, precision)) ||
      (st = check_operand_extent(M, N, precision)))
    return st;
  if ((st = current_device_ok())) return st;
  return hip_status(svdq_launch_mlp_gemm_gelu_quant(xq, xs, wq, ws, lora_act, lora_up, bias, M, N, K, rank,
                                                    smooth_inv2, lora_down2, rank2, xq2, xs2, lora_act2, stream));
}

int svdq_gemm_w4a16(const void* x, const uint8_t* wq, const void* ws, const void* bias, void* y, int M, int N,
                    int K, void* stream) {
  if (!x || !wq || !ws || !y) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(ws) || !aligned16(y)) return SVDQ_ERR_INVALID_ARG;
  if (bias && !aligned16(bias)) return SVDQ_ERR_INVALID_ARG;
  if (M < 1 || N < 1) return SVDQ_ERR_SHAPE;
  int st;
  if ((st = check_k(K, SVDQ_INT4))) return st;
  if ((st = check_operand_extent(N, K, SVDQ_INT4))) return st;
  if ((st = current_device_ok())) return st;
  return hip_status(svdq_launch_gemm_w4a16(x, wq, ws, bias, y, M, N, K, stream));
}

int svdq_unfused_linear(const void* x, int M, int K, const float* smooth_inv, const void* lora_down, int rank,
                        const uint8_t* wq, const void* ws, const void* lora_up, const void* bias, int N,
                        int precision, uint8_t* xq, void* xs, float* lora_act, void* y, void* stream) {
  int st = check_precision(precision);
  if (st) return st;
  if (!x || !smooth_inv || !wq || !ws || !xq || !xs || !y) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_down || !lora_up || !lora_act)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(smooth_inv) || !aligned16(wq) || !aligned16(ws) || !aligned16(xq) ||
      !aligned16(xs) || !aligned16(y))
    return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!aligned16(lora_down) || !aligned16(lora_up) || !aligned16(lora_act))) return SVDQ_ERR_INVALID_ARG;
  if (bias && !aligned16(bias)) return SVDQ_ERR_INVALID_ARG;
  if (M < 1 || N < 1) return SVDQ_ERR_SHAPE;
  if ((st = check_k(K, precision))) return st;
  if ((st = check_rank(rank, K, N))) return st;
  if (precision != SVDQ_INT4) return SVDQ_ERR_INVALID_ARG;
  if ((st = check_operand_extent(M, K, precision)) || (st = check_operand_extent(N, K, precision))) return st;
  if ((st = current_device_ok())) return st;
  return hip_status(svdq_launch_unfused_linear(x, M, K, smooth_inv, lora_down, rank, wq, ws, lora_up, bias, N,
                                               precision, xq, xs, lora_act, y, stream));
}

int svdq_unfused_linear_noalloc(const void* x, int M, int K, const float* smooth_inv, const void* lora_down,
                                int rank, const uint8_t* wq, const void* ws, const void* lora_up, const void* bias,
                                int N, int precision, void* y, void* stream) {
  int st = check_precision(precision);
  if (st) return st;
  if (!x || !smooth_inv || !wq || !ws || !y) return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!lora_down || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(smooth_inv) || !aligned16(wq) || !aligned16(ws) || !aligned16(y))
    return SVDQ_ERR_INVALID_ARG;
  if (rank > 0 && (!aligned16(lora_down) || !aligned16(lora_up))) return SVDQ_ERR_INVALID_ARG;
  if (bias && !aligned16(bias)) return SVDQ_ERR_INVALID_ARG;
  if (M < 1 || N < 1) return SVDQ_ERR_SHAPE;
  if ((st = check_k(K, precision))) return st;
  if ((st = check_rank(rank, K, N))) return st;
  if (precision != SVDQ_INT4) return SVDQ_ERR_INVALID_ARG;
  if ((st = check_operand_extent(M, K, precision)) || (st = check_operand_extent(N, K, precision))) return st;
  size_t off[3];
  if (noalloc_layout(M, K, rank, off) > kNoAllocScratchBytes) return SVDQ_ERR_SHAPE;
  if ((st = current_device_ok())) return st;
  return hip_status(svdq_launch_unfused_linear_noalloc(x, M, K, smooth_inv, lora_down, rank, wq, ws, lora_up, bias, N,
                                                       precision, y, stream));
}

int svdq_bench_mfma_ceiling(int precision, int blocks, int iters, float* out, void* stream) {
  if (!out || !aligned16(out)) return SVDQ_ERR_INVALID_ARG;
  if (precision != SVDQ_INT4 && precision != SVDQ_MXFP4) return SVDQ_ERR_INVALID_ARG;
  if (blocks < 1 || iters < 1) return SVDQ_ERR_SHAPE;
  int st;
  if ((st = current_device_ok())) return st;
  return hip_status(svdq_launch_mfma_ceiling(precision, blocks, iters, out, stream));
}

int svdq_debug_group_partials(const uint8_t* xq, const uint8_t* wq, int M, int N, int K, int m0, int n0, int mt,
                              int nt, int32_t* out, void* stream) {
  if (!xq || !wq || !out) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(wq) || !aligned16(out)) return SVDQ_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || mt < 1 || nt < 1) return SVDQ_ERR_SHAPE;
  int st = check_k(K, SVDQ_INT4);
  if (st) return st;
  if (m0 < 0 || n0 < 0 || m0 + static_cast<long long>(mt) > M || n0 + static_cast<long long>(nt) > N)
    return SVDQ_ERR_SHAPE;
  if ((st = check_operand_extent(M, K, SVDQ_INT4)) || (st = check_operand_extent(N, K, SVDQ_INT4))) return st;
  if ((st = current_device_ok())) return st;
  return hip_status(svdq_launch_debug_group_partials(xq, wq, M, N, K, m0, n0, mt, nt, out, stream));
}

}  // extern "C"

// Internal declarations shared by the host-side translation units of
// libsvdq.so.  Not part of the public ABI (that is include/svdq.h).
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/svdq.h"

namespace svdq {

constexpr int kInt4Group = 64;    // INT4 quantization group along K
constexpr int kMxBlock = 32;      // MXFP4 block along K
constexpr int kMaxRank = 256;

// Number of host threads for the offline pack.
int host_threads();

// Shape rules of the ABI; return SVDQ_OK or SVDQ_ERR_SHAPE / _INVALID_ARG.
int check_precision(int precision);
int check_k(int K, int precision);
int check_rank(int rank, int K, int N);
int check_operand_extent(int rows, int K, int precision);

// Device scratch of svdq_unfused_linear_noalloc: its codes, scales and
// lora_act, each at a 256-byte aligned offset.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
inline size_t noalloc_align(size_t v) { return (v + 255) & ~size_t(255); }
// off[0] xq, off[1] xs, off[2] lora_act; returns the bytes the call needs.
inline size_t noalloc_layout(int M, int K, int rank, size_t off[3]) {
  const size_t m = static_cast<size_t>(M), k = static_cast<size_t>(K), r = static_cast<size_t>(rank);
  off[0] = 0;
  off[1] = noalloc_align(m * k / 2);
  off[2] = off[1] + noalloc_align((k / kInt4Group) * m * 2);
  return off[2] + m * r * 4;
}

// Host-side number-format helpers used by the offline pack.
uint16_t f32_to_bf16_bits(float f);
float bf16_bits_to_f32(uint16_t b);
uint16_t f32_to_f16_sat_bits(float f);
float f16_bits_to_f32(uint16_t h);

}  // namespace svdq

// Kernel launchers (defined in svdq_kernels.hip).  They assume validated
// arguments and return a hipError_t value as int.
extern "C" {
int svdq_launch_quantize_act_lora_down(const void* x, int M, int K,
                                       const float* smooth_inv,
                                       const void* lora_down, int rank,
                                       int precision, uint8_t* xq, void* xs,
                                       float* lora_act, void* stream);
int svdq_launch_gemm_w4a4_lora_up(const uint8_t* xq, const void* xs,
                                  const uint8_t* wq, const void* ws,
                                  const float* lora_act, const void* lora_up,
                                  const void* bias, void* y, int M, int N,
                                  int K, int rank, int precision,
                                  void* stream);
// Split-K plan of svdq_launch_gemm_w4a4_lora_up_ws for the current device
// (splits = 1 and bytes = 0 when the single-pass schedule runs); returns 0.
int svdq_gemm_split_plan(int M, int N, int K, int precision, int* splits, int* per, size_t* bytes);
int svdq_launch_gemm_w4a4_lora_up_ws(const uint8_t* xq, const void* xs, const uint8_t* wq, const void* ws,
                                     const float* lora_act, const void* lora_up, const void* bias, void* y, int M,
                                     int N, int K, int rank, int precision, void* workspace, size_t workspace_bytes,
                                     void* stream);
int svdq_launch_gemm_int4_gelu(const uint8_t* xq, const void* xs, const uint8_t* wq, const void* ws,
                               const float* lora_act, const void* lora_up, const void* bias, void* y, int M, int N,
                               int K, int rank, void* stream);
int svdq_launch_mlp_gemm_gelu_quant(const uint8_t* xq, const void* xs, const uint8_t* wq, const void* ws,
                                    const float* lora_act, const void* lora_up, const void* bias, int M, int N, int K,
                                    int rank, const float* smooth_inv2, const void* lora_down2, int rank2,
                                    uint8_t* xq2, void* xs2, float* lora_act2, void* stream);
int svdq_launch_gemm_w4a16(const void* x, const uint8_t* wq, const void* ws, const void* bias, void* y, int M,
                           int N, int K, void* stream);
int svdq_launch_unfused_linear(const void* x, int M, int K,
                               const float* smooth_inv, const void* lora_down,
                               int rank, const uint8_t* wq, const void* ws,
                               const void* lora_up, const void* bias, int N,
                               int precision, uint8_t* xq, void* xs,
                               float* lora_act, void* y, void* stream);
int svdq_launch_mfma_ceiling(int precision, int blocks, int iters, float* out, void* stream);
int svdq_launch_unfused_linear_noalloc(const void* x, int M, int K, const float* smooth_inv, const void* lora_down,
                                       int rank, const uint8_t* wq, const void* ws, const void* lora_up,
                                       const void* bias, int N, int precision, void* y, void* stream);
int svdq_launch_debug_group_partials(const uint8_t* xq, const uint8_t* wq,
                                     int M, int N, int K, int m0, int n0,
                                     int mt, int nt, int32_t* out,
                                     void* stream);
}

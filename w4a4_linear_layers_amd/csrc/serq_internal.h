// Internal declarations of libserq: kernel launchers called by the C ABI
// layer (serq_abi.cpp) and device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace serq {

// Arguments of one serq_linear call (device pointers, validated sizes).
struct LinearArgs {
  const uint8_t* Xq;   // M x K/2 bytes (a_bits 4) or M x K int8 (a_bits 8)
  const float* sx;     // M
  const uint8_t* Wq;   // N x K/2 bytes
  const float* sw;     // N
  const uint8_t* Rq;   // N x rq_row_bytes(r) bytes (may be null when r == 0)
  const float* sr;     // N (may be null when r == 0)
  void* Y;             // M x N, fp32 or bf16
  int32_t* dbg_main;   // optional M x N int32
  int32_t* dbg_res;    // optional M x N int32
  int M, K, N, r;
  int a_bits;
  int y_bf16;
};

// Row bytes of the packed Q(R): r codes padded with zero codes to a
// multiple of 32 codes (16 bytes).
__host__ __device__ constexpr int rq_row_bytes(int r) { return (r + 31) / 32 * 16; }

// Kernel families serq_linear chooses between.
enum class LinearKernel { kGemv, kDecode16, kDecode32, kTile, kGeneric };

struct LinearPlan {
  LinearKernel kind;
  int tn, tm;          // per-wave 32x32 block counts (kTile only)
  int wgm;             // wave rows (token direction) per k-group (kTile only)
  int kg;              // k-groups per workgroup, each a k-tile of every stage (kTile only)
  const char* name;
};

LinearPlan plan_linear(int M, int K, int N, int r, int a_bits);

hipError_t launch_quant_act(const void* X, int x_bf16, int M, int K, const float* s_hat_inv,
                            int a_bits, void* Xq, float* sx, hipStream_t stream);
hipError_t launch_linear(const LinearArgs& a, const LinearPlan& plan, hipStream_t stream);
hipError_t launch_silu_mul_quant_act(const void* G, const void* U, int ld, int x_bf16, int M, int K,
                                     const float* s_hat_inv, int a_bits, void* Xq, float* sx,
                                     hipStream_t stream);

// The bf6 route (serq_act_bf6, serq_linear_bf6): operands in the bf6 tile
// layout; LinearArgs carries X6 / W6 / R6 in place of Xq / Wq / Rq.
hipError_t launch_act_bf6(const void* Xq, int M, int K, void* X6, hipStream_t stream);
hipError_t launch_linear_bf6(const LinearArgs& a, hipStream_t stream);
int bf6_tile_kind(int M, int N, int r);   // serq_linear_bf6's tile: 0 128x128, 2 256x256

// The MXFP4 layer (serq_quant_act_mx, serq_linear_mx): FP4 E2M1 codes two
// per byte with one E8M0 exponent byte per 32 elements along K.
struct MxArgs {
  const uint8_t* Xq;   // M x K/2
  const uint8_t* Xsc;  // M x K/32
  const uint8_t* Wq;   // N x K/2
  const uint8_t* Wsc;  // N x K/32
  const uint8_t* Rq;   // N x r/2 (may be null when r == 0)
  const uint8_t* Rsc;  // N x r/32
  void* Y;             // M x N, fp32 or bf16
  float* dbg_main;     // optional M x N fp32 accumulators
  float* dbg_res;
  int M, K, N, r;
  int y_bf16;
};

hipError_t launch_quant_act_mx(const void* X, int x_bf16, int M, int K, const float* s_hat_inv, uint8_t* Xq,
                               uint8_t* Xsc, hipStream_t stream);
hipError_t launch_linear_mx(const MxArgs& a, hipStream_t stream);
int mx_kernel_kind(int M, int K, int N);   // 0 plain, 1 pipelined 128 x 128, 2 pipelined 256 x 256

}  // namespace serq

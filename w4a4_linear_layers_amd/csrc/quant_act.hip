// Per-token activation quantization for the SERQ linear (gfx950).
//
// The activations arrive already in the saliency order (papernotes.org SERQ
// notes, 关键设计 3: the previous layer's columns were permuted offline), so
// each row is read once, contiguously:
//     x^[m, k] = fl32(X[m, k] * s_hat_inv[k])
//     m_row    = max_k |x^[m, k]|,  scale = fl32(m_row / qmax),
//     code     = clamp(rne(fl32(x^ * fl32(qmax / m_row))))
// with qmax = 7 (int4, packed two codes per byte) or 127 (int8). A row whose
// reciprocal overflows (all-zero row) gets scale 0 and zero codes.
//
// This is a streaming scan, bound by HBM: one workgroup of 256 lanes per row,
// 16-byte loads, the flattened row kept in registers between the absmax
// reduction (wave shuffles, then LDS across the four waves) and the
// quantization, so X is read exactly once.

#include <cfloat>

#include "serq_internal.h"

namespace serq {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;                       // elements per lane per pass
constexpr int kPassElems = kThreads * kVec;   // 2048 elements per pass

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16lo(a.x); v[1] = bf16hi(a.x); v[2] = bf16lo(a.y); v[3] = bf16hi(a.y);
  v[4] = bf16lo(a.z); v[5] = bf16hi(a.z); v[6] = bf16lo(a.w); v[7] = bf16hi(a.w);
}

__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

template <int QMAX>
__device__ __forceinline__ int qcode(float v, float inv) {
  float q = __builtin_rintf(v * inv);
  q = fminf(fmaxf(q, static_cast<float>(-QMAX - 1)), static_cast<float>(QMAX));
  return static_cast<int>(q);
}

// Fast path: K % 8 == 0, K <= NP * 2048, 16-byte aligned rows.
template <typename T, int A_BITS, int NP>
__global__ __launch_bounds__(kThreads) void quant_act_rows(const T* __restrict__ X,
                                                           const float* __restrict__ sinv, int K,
                                                           uint8_t* __restrict__ Xq,
                                                           float* __restrict__ sx) {
  constexpr int QMAX = A_BITS == 4 ? 7 : 127;
  __shared__ float red[kThreads / 64];
  const size_t row = blockIdx.x;
  const T* xr = X + row * static_cast<size_t>(K);
  float v[NP][kVec];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c = (p * kThreads + static_cast<int>(threadIdx.x)) * kVec;
    if (c < K) {
      float s[kVec];
      load8(xr + c, v[p]);
      load8(sinv + c, s);
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        v[p][i] = v[p][i] * s[i];
        amax = fmaxf(amax, fabsf(v[p][i]));
      }
    }
  }
  amax = block_max(amax, red);
  float inv = static_cast<float>(QMAX) / amax;
  const bool zero = !(inv <= FLT_MAX);
  if (zero) inv = 0.0f;
  if (threadIdx.x == 0) sx[row] = zero ? 0.0f : amax / static_cast<float>(QMAX);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c = (p * kThreads + static_cast<int>(threadIdx.x)) * kVec;
    if (c < K) {
      int q[kVec];
#pragma unroll
      for (int i = 0; i < kVec; ++i) q[i] = qcode<QMAX>(v[p][i], inv);
      if (A_BITS == 4) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < kVec; ++i) w |= static_cast<uint32_t>(q[i] & 0xF) << (4 * i);
        *reinterpret_cast<uint32_t*>(Xq + row * static_cast<size_t>(K / 2) + c / 2) = w;
      } else {
        uint2 w;
        w.x = (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) | (static_cast<uint32_t>(q[3] & 0xFF) << 24);
        w.y = (q[4] & 0xFF) | ((q[5] & 0xFF) << 8) | ((q[6] & 0xFF) << 16) | (static_cast<uint32_t>(q[7] & 0xFF) << 24);
        *reinterpret_cast<uint2*>(Xq + row * static_cast<size_t>(K) + c) = w;
      }
    }
  }
}

// General path: any even K, any alignment; two reads of the row.
template <typename T, int A_BITS>
__global__ __launch_bounds__(kThreads) void quant_act_rows_generic(const T* __restrict__ X,
                                                                   const float* __restrict__ sinv,
                                                                   int K, uint8_t* __restrict__ Xq,
                                                                   float* __restrict__ sx) {
  constexpr int QMAX = A_BITS == 4 ? 7 : 127;
  __shared__ float red[kThreads / 64];
  const size_t row = blockIdx.x;
  const T* xr = X + row * static_cast<size_t>(K);
  float amax = 0.0f;
  for (int k = threadIdx.x; k < K; k += kThreads) amax = fmaxf(amax, fabsf(load1(xr + k) * sinv[k]));
  amax = block_max(amax, red);
  float inv = static_cast<float>(QMAX) / amax;
  const bool zero = !(inv <= FLT_MAX);
  if (zero) inv = 0.0f;
  if (threadIdx.x == 0) sx[row] = zero ? 0.0f : amax / static_cast<float>(QMAX);
  for (int k2 = 2 * threadIdx.x; k2 < K; k2 += 2 * kThreads) {
    const int q0 = qcode<QMAX>(load1(xr + k2) * sinv[k2], inv);
    const int q1 = qcode<QMAX>(load1(xr + k2 + 1) * sinv[k2 + 1], inv);
    if (A_BITS == 4) {
      Xq[row * static_cast<size_t>(K / 2) + k2 / 2] = static_cast<uint8_t>((q0 & 0xF) | ((q1 & 0xF) << 4));
    } else {
      Xq[row * static_cast<size_t>(K) + k2] = static_cast<uint8_t>(q0 & 0xFF);
      Xq[row * static_cast<size_t>(K) + k2 + 1] = static_cast<uint8_t>(q1 & 0xFF);
    }
  }
}

template <typename T, int A_BITS>
hipError_t launch_typed(const T* X, int M, int K, const float* sinv, uint8_t* Xq, float* sx,
                        hipStream_t st) {
  const dim3 grid(M), block(kThreads);
  const bool aligned = (K % kVec == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0) &&
                       ((reinterpret_cast<uintptr_t>(sinv) & 15) == 0) &&
                       ((reinterpret_cast<uintptr_t>(Xq) & 15) == 0);
  const int passes = (K + kPassElems - 1) / kPassElems;
  if (!aligned || passes > 16) {
    quant_act_rows_generic<T, A_BITS><<<grid, block, 0, st>>>(X, sinv, K, Xq, sx);
  } else if (passes <= 1) {
    quant_act_rows<T, A_BITS, 1><<<grid, block, 0, st>>>(X, sinv, K, Xq, sx);
  } else if (passes <= 2) {
    quant_act_rows<T, A_BITS, 2><<<grid, block, 0, st>>>(X, sinv, K, Xq, sx);
  } else if (passes <= 4) {
    quant_act_rows<T, A_BITS, 4><<<grid, block, 0, st>>>(X, sinv, K, Xq, sx);
  } else if (passes <= 8) {
    quant_act_rows<T, A_BITS, 8><<<grid, block, 0, st>>>(X, sinv, K, Xq, sx);
  } else {
    quant_act_rows<T, A_BITS, 16><<<grid, block, 0, st>>>(X, sinv, K, Xq, sx);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_act(const void* X, int x_bf16, int M, int K, const float* s_hat_inv,
                            int a_bits, void* Xq, float* sx, hipStream_t stream) {
  uint8_t* q = static_cast<uint8_t*>(Xq);
  if (x_bf16) {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    return a_bits == 4 ? launch_typed<uint16_t, 4>(x, M, K, s_hat_inv, q, sx, stream)
                       : launch_typed<uint16_t, 8>(x, M, K, s_hat_inv, q, sx, stream);
  }
  const float* x = static_cast<const float*>(X);
  return a_bits == 4 ? launch_typed<float, 4>(x, M, K, s_hat_inv, q, sx, stream)
                     : launch_typed<float, 8>(x, M, K, s_hat_inv, q, sx, stream);
}

}  // namespace serq

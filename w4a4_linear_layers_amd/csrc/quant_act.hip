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
// This is a streaming scan, bound by HBM: one workgroup of 256 or 512 lanes
// per row, 16-byte loads, the flattened row kept in registers between the
// absmax reduction (wave shuffles, then LDS across the waves) and the
// quantization, so X is read exactly once.

#include <cfloat>

#include "serq_internal.h"

namespace serq {
namespace {

constexpr int kThreads = 256;                 // lanes of the generic kernel
constexpr int kVec = 8;                       // elements per lane per pass
constexpr int kPassElems = kThreads * kVec;   // 2048: the split path's row-length unit

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

template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

template <int QMAX>
__device__ __forceinline__ int qcode(float v, float inv) {
  float q = __builtin_rintf(v * inv);
  q = fminf(fmaxf(q, static_cast<float>(-QMAX - 1)), static_cast<float>(QMAX));
  return static_cast<int>(q);
}

// The MLP activation h = silu(g) * u, evaluated by one fixed fp32 recipe so
// that the codes it feeds the quantizer are reproducible bit for bit (the
// LLaMA MLP's silu(g) = g / (1 + e^-g); its input order is already down's
// saliency order, the permutation having been pushed into gate and up
// offline -- papernotes.org SERQ notes, 关键设计 3). e^x by Cody and Waite's
// reduction: e^x = 2^n e^r, n = rne(x log2 e), r = fma(-n, c_lo,
// fma(-n, c_hi, x)) with c_hi + c_lo = ln 2 and c_hi = 22713 * 2^-15 of 15
// significant bits (|n| <= 116 after the clamp, so n c_hi has at most 22
// significant bits and is exact), then the degree-7 Taylor polynomial of e^r in Horner form,
// one fused multiply-add per degree, and an exact scaling by 2^n; the
// argument is clamped to [-80, 80] so every step stays a normal number.
// Every other operation is one fp32 op (the build disables contraction into
// fused multiply-adds, so only the ones written here exist); the division is
// IEEE.
constexpr double kLn2 = 0.6931471805599453;
constexpr float kLog2e = static_cast<float>(1.0 / kLn2);
constexpr float kLn2Hi = 0.693145751953125f;
constexpr float kLn2Lo = static_cast<float>(kLn2 - 0.693145751953125);
constexpr float kInvFact[8] = {1.0f, 1.0f, static_cast<float>(1.0 / 2), static_cast<float>(1.0 / 6),
                               static_cast<float>(1.0 / 24), static_cast<float>(1.0 / 120),
                               static_cast<float>(1.0 / 720), static_cast<float>(1.0 / 5040)};

__device__ __forceinline__ float exp32(float x) {
#pragma clang fp contract(off)
  x = fminf(fmaxf(x, -80.0f), 80.0f);
  const float n = __builtin_rintf(x * kLog2e);
  float r = __builtin_fmaf(-n, kLn2Hi, x);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float p = kInvFact[7];
#pragma unroll
  for (int k = 6; k >= 0; --k) p = __builtin_fmaf(p, r, kInvFact[k]);
  return __builtin_ldexpf(p, static_cast<int>(n));
}

__device__ __forceinline__ float silu_mul(float g, float u) {
#pragma clang fp contract(off)
  const float s = 1.0f + exp32(-g);
  const float sg = g / s;
  return sg * u;
}

// Where a row's values come from: the activations themselves (ACT false:
// row m of x at a + m * ld), or h = silu(g) * u (ACT true: g at a, u at b,
// both with row stride ld).
template <typename T, bool ACT>
struct RowSrc {
  const T* a;
  const T* b;
  int ld;
  __device__ __forceinline__ void load8(size_t row, int c, float (&v)[8]) const {
    if constexpr (!ACT) {
      serq::load8(a + row * ld + c, v);
    } else {
      float g[8], u[8];
      serq::load8(a + row * ld + c, g);
      serq::load8(b + row * ld + c, u);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = silu_mul(g[i], u[i]);
    }
  }
  __device__ __forceinline__ float load1(size_t row, int k) const {
    if constexpr (!ACT) return serq::load1(a + row * ld + k);
    else return silu_mul(serq::load1(a + row * ld + k), serq::load1(b + row * ld + k));
  }
};

// Fast path: K % 8 == 0, K <= NP * NT * 8, 16-byte aligned rows; NT lanes
// per row.
template <typename T, int A_BITS, int NP, bool ACT, int NT>
__global__ __launch_bounds__(NT) void quant_act_rows(RowSrc<T, ACT> src,
                                                           const float* __restrict__ sinv, int K,
                                                           uint8_t* __restrict__ Xq,
                                                           float* __restrict__ sx) {
  constexpr int QMAX = A_BITS == 4 ? 7 : 127;
  __shared__ float red[NT / 64];
  const size_t row = blockIdx.x;
  float v[NP][kVec];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c = (p * NT + static_cast<int>(threadIdx.x)) * kVec;
    if (c < K) {
      float s[kVec];
      src.load8(row, c, v[p]);
      load8(sinv + c, s);
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        v[p][i] = v[p][i] * s[i];
        amax = fmaxf(amax, fabsf(v[p][i]));
      }
    }
  }
  amax = block_max<NT>(amax, red);
  float inv = static_cast<float>(QMAX) / amax;
  const bool zero = !(inv <= FLT_MAX);
  if (zero) inv = 0.0f;
  if (threadIdx.x == 0) sx[row] = zero ? 0.0f : amax / static_cast<float>(QMAX);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c = (p * NT + static_cast<int>(threadIdx.x)) * kVec;
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
template <typename T, int A_BITS, bool ACT>
__global__ __launch_bounds__(kThreads) void quant_act_rows_generic(RowSrc<T, ACT> src,
                                                                   const float* __restrict__ sinv,
                                                                   int K, uint8_t* __restrict__ Xq,
                                                                   float* __restrict__ sx) {
  constexpr int QMAX = A_BITS == 4 ? 7 : 127;
  __shared__ float red[kThreads / 64];
  const size_t row = blockIdx.x;
  float amax = 0.0f;
  for (int k = threadIdx.x; k < K; k += kThreads) amax = fmaxf(amax, fabsf(src.load1(row, k) * sinv[k]));
  amax = block_max<kThreads>(amax, red);
  float inv = static_cast<float>(QMAX) / amax;
  const bool zero = !(inv <= FLT_MAX);
  if (zero) inv = 0.0f;
  if (threadIdx.x == 0) sx[row] = zero ? 0.0f : amax / static_cast<float>(QMAX);
  for (int k2 = 2 * threadIdx.x; k2 < K; k2 += 2 * kThreads) {
    const int q0 = qcode<QMAX>(src.load1(row, k2) * sinv[k2], inv);
    const int q1 = qcode<QMAX>(src.load1(row, k2 + 1) * sinv[k2 + 1], inv);
    if (A_BITS == 4) {
      Xq[row * static_cast<size_t>(K / 2) + k2 / 2] = static_cast<uint8_t>((q0 & 0xF) | ((q1 & 0xF) << 4));
    } else {
      Xq[row * static_cast<size_t>(K) + k2] = static_cast<uint8_t>(q0 & 0xFF);
      Xq[row * static_cast<size_t>(K) + k2 + 1] = static_cast<uint8_t>(q1 & 0xFF);
    }
  }
}

// Few long rows: one workgroup per row would leave most CUs idle while each
// works through K elements alone, so each row is cut into C chunks of
// 512 * NP elements, one wave each, in two launches. The first writes every
// chunk's max |x^|; the second reduces the row's C maxima, recomputes its
// chunk's x^ (the same operations, so the same values) and writes the codes;
// chunk 0 writes the scale. Codes and scales equal the one-pass kernels' bit
// for bit (a max does not depend on the order it is taken in). The chunk
// maxima sit in a library-held device array (each device has its own copy),
// fully written by the first launch before the second reads it: calls that
// overlap on one device must not both take this path.
constexpr int kSplitMaxRows = 128;
constexpr int kSplitMaxChunks = 64;
constexpr int kChunkElems = 64 * kVec;        // one wave, 8 elements per lane

__device__ float g_chunk_max[kSplitMaxRows * kSplitMaxChunks];

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

template <typename T, int NP, bool ACT>
__device__ __forceinline__ float chunk_values(const RowSrc<T, ACT>& src, const float* __restrict__ sinv,
                                              size_t row, int c0, int K, float (&v)[NP][kVec]) {
  const int lane = static_cast<int>(threadIdx.x);
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c = c0 + (p * 64 + lane) * kVec;
    if (c < K) {
      float s[kVec];
      src.load8(row, c, v[p]);
      load8(sinv + c, s);
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        v[p][i] = v[p][i] * s[i];
        amax = fmaxf(amax, fabsf(v[p][i]));
      }
    }
  }
  return amax;
}

template <typename T, int NP, bool ACT>
__global__ __launch_bounds__(64) void chunk_max_kernel(RowSrc<T, ACT> src, const float* __restrict__ sinv,
                                                       int K, int C) {
  const int chunk = blockIdx.x;
  const size_t row = blockIdx.y;
  float v[NP][kVec];
  const float amax = wave_max(chunk_values<T, NP, ACT>(src, sinv, row, chunk * kChunkElems * NP, K, v));
  if (threadIdx.x == 0) g_chunk_max[row * C + chunk] = amax;
}

template <typename T, int A_BITS, int NP, bool ACT>
__global__ __launch_bounds__(64) void chunk_quant_kernel(RowSrc<T, ACT> src, const float* __restrict__ sinv,
                                                         int K, int C, uint8_t* __restrict__ Xq,
                                                         float* __restrict__ sx) {
  constexpr int QMAX = A_BITS == 4 ? 7 : 127;
  const int lane = static_cast<int>(threadIdx.x);
  const int chunk = blockIdx.x;
  const size_t row = blockIdx.y;
  const int c0 = chunk * kChunkElems * NP;
  float v[NP][kVec];
  chunk_values<T, NP, ACT>(src, sinv, row, c0, K, v);
  const float amax = wave_max(lane < C ? g_chunk_max[row * C + lane] : 0.0f);
  float inv = static_cast<float>(QMAX) / amax;
  const bool zero = !(inv <= FLT_MAX);
  if (zero) inv = 0.0f;
  if (chunk == 0 && lane == 0) sx[row] = zero ? 0.0f : amax / static_cast<float>(QMAX);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c = c0 + (p * 64 + lane) * kVec;
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

template <typename T, int A_BITS, int NP, bool ACT>
hipError_t launch_split_np(RowSrc<T, ACT> src, int M, int K, const float* sinv, uint8_t* Xq, float* sx,
                           hipStream_t st) {
  const int C = (K + kChunkElems * NP - 1) / (kChunkElems * NP);
  const dim3 grid(C, M), block(64);
  chunk_max_kernel<T, NP, ACT><<<grid, block, 0, st>>>(src, sinv, K, C);
  chunk_quant_kernel<T, A_BITS, NP, ACT><<<grid, block, 0, st>>>(src, sinv, K, C, Xq, sx);
  return hipGetLastError();
}

// The split path's share (measured against the one-pass kernel): up to 64
// rows, or kSplitMaxRows rows of the fused activation beyond 16384 elements,
// chunks of up to 2048 elements, at most kSplitMaxChunks of them; rows short
// enough for one workgroup's pass gain nothing from it.
template <bool ACT>
bool use_split(int M, int K) {
  const int max_rows = ACT && K > 16384 ? kSplitMaxRows : 64;
  return M <= max_rows && K > (ACT ? 2 : 4) * kPassElems && K <= kSplitMaxChunks * 4 * kChunkElems;
}

template <typename T, int A_BITS, bool ACT>
hipError_t launch_split(RowSrc<T, ACT> src, int M, int K, const float* sinv, uint8_t* Xq, float* sx,
                        hipStream_t st) {
  if (K <= kSplitMaxChunks * kChunkElems) return launch_split_np<T, A_BITS, 1, ACT>(src, M, K, sinv, Xq, sx, st);
  if (K <= kSplitMaxChunks * 2 * kChunkElems)
    return launch_split_np<T, A_BITS, 2, ACT>(src, M, K, sinv, Xq, sx, st);
  return launch_split_np<T, A_BITS, 4, ACT>(src, M, K, sinv, Xq, sx, st);
}

template <typename T, int A_BITS, bool ACT, int NT>
hipError_t launch_rows(RowSrc<T, ACT> src, int M, int K, const float* sinv, uint8_t* Xq, float* sx,
                       hipStream_t st) {
  const dim3 grid(M), block(NT);
  const int passes = (K + NT * kVec - 1) / (NT * kVec);
  if (passes <= 1) {
    quant_act_rows<T, A_BITS, 1, ACT, NT><<<grid, block, 0, st>>>(src, sinv, K, Xq, sx);
  } else if (passes <= 2) {
    quant_act_rows<T, A_BITS, 2, ACT, NT><<<grid, block, 0, st>>>(src, sinv, K, Xq, sx);
  } else if (passes <= 4) {
    quant_act_rows<T, A_BITS, 4, ACT, NT><<<grid, block, 0, st>>>(src, sinv, K, Xq, sx);
  } else if (passes <= 8) {
    quant_act_rows<T, A_BITS, 8, ACT, NT><<<grid, block, 0, st>>>(src, sinv, K, Xq, sx);
  } else if constexpr (NT < 1024) {       // 1024 lanes hold at most 8 passes in their registers
    quant_act_rows<T, A_BITS, 16, ACT, NT><<<grid, block, 0, st>>>(src, sinv, K, Xq, sx);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int A_BITS, bool ACT>
hipError_t launch_typed(RowSrc<T, ACT> src, int M, int K, const float* sinv, uint8_t* Xq, float* sx,
                        hipStream_t st) {
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool aligned = (K % kVec == 0) && (src.ld % kVec == 0) && al16(src.a) && (!ACT || al16(src.b)) &&
                       al16(sinv) && al16(Xq);
  if (aligned && use_split<ACT>(M, K)) return launch_split<T, A_BITS, ACT>(src, M, K, sinv, Xq, sx, st);
  // 512 lanes per row while the rows are few or long (more waves in flight
  // per row, fewer values per lane; measured 1.3x at 256 rows of 14336),
  // 1024 for many rows beyond 16384 (1.05-1.15x at 1024-4096 rows of 28672;
  // at 14336 it was slower), 256 for many short rows (more rows resident
  // per CU).
  if (aligned && M > 512 && K > 16384 && K <= 8 * 1024 * kVec)
    return launch_rows<T, A_BITS, ACT, 1024>(src, M, K, sinv, Xq, sx, st);
  if (aligned && K <= 16 * 512 * kVec && (M <= 512 || K > 8192))
    return launch_rows<T, A_BITS, ACT, 512>(src, M, K, sinv, Xq, sx, st);
  if (aligned && K <= 16 * kThreads * kVec) return launch_rows<T, A_BITS, ACT, kThreads>(src, M, K, sinv, Xq, sx, st);
  quant_act_rows_generic<T, A_BITS, ACT><<<dim3(M), dim3(kThreads), 0, st>>>(src, sinv, K, Xq, sx);
  return hipGetLastError();
}

template <bool ACT>
hipError_t launch_any(const void* A, const void* B, int ld, int x_bf16, int M, int K, const float* sinv,
                      int a_bits, void* Xq, float* sx, hipStream_t st) {
  uint8_t* q = static_cast<uint8_t*>(Xq);
  if (x_bf16) {
    const RowSrc<uint16_t, ACT> src{static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), ld};
    return a_bits == 4 ? launch_typed<uint16_t, 4, ACT>(src, M, K, sinv, q, sx, st)
                       : launch_typed<uint16_t, 8, ACT>(src, M, K, sinv, q, sx, st);
  }
  const RowSrc<float, ACT> src{static_cast<const float*>(A), static_cast<const float*>(B), ld};
  return a_bits == 4 ? launch_typed<float, 4, ACT>(src, M, K, sinv, q, sx, st)
                     : launch_typed<float, 8, ACT>(src, M, K, sinv, q, sx, st);
}

}  // namespace

hipError_t launch_quant_act(const void* X, int x_bf16, int M, int K, const float* s_hat_inv,
                            int a_bits, void* Xq, float* sx, hipStream_t stream) {
  return launch_any<false>(X, nullptr, K, x_bf16, M, K, s_hat_inv, a_bits, Xq, sx, stream);
}

hipError_t launch_silu_mul_quant_act(const void* G, const void* U, int ld, int x_bf16, int M, int K,
                                     const float* s_hat_inv, int a_bits, void* Xq, float* sx,
                                     hipStream_t stream) {
  return launch_any<true>(G, U, ld, x_bf16, M, K, s_hat_inv, a_bits, Xq, sx, stream);
}

}  // namespace serq

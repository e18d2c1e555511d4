// The MXFP4 variant of the SERQ layer on gfx950 (serq_quant_act_mx,
// serq_linear_mx).
//
// The pages run the method on integer and on microscaling-FP4 matrix
// hardware alike (gist.science/de/paper/2603.08185, "Technische
// Zusammenfassung" 3: compatible with INT4 and MXFP4; 4, Performance &
// Latenz: the speed is measured on hardware FP4 products, the residual
// adding about 1 %). Format: OCP Microscaling (MX) -- blocks of 32 elements
// along K share an E8M0 exponent (byte e + 127, the scale 2^e), elements are
// FP4 E2M1 packed two per byte, element 2t in the low nibble. This is
// exactly the operand format of gfx950's scaled matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands: a lane's operand is 32
// consecutive elements of one row (16 bytes, the packed row as stored) and
// its scale operand the E8M0 byte of that block, so rows go from memory to
// the matrix core with no re-encoding at all.
//
//   acc_main[m, n] = sum over K-blocks b of 2^(ex_mb + ew_nb) sum_{k in b} x_mk w_nk
//   acc_res[m, n]  = sum over the first r/32 blocks of 2^(ex_mb + er_nb) sum x_mk rho_nk
//   Y = acc_main + acc_res                    (fp32, stored as fp32 or bf16)
//
// The residual reuses the activation blocks of the first r channels (no
// second quantization; papernotes.org SERQ notes, 关键设计 2). Accumulation
// is in fp32 inside the matrix instruction, so unlike the integer layer the
// sums are rounded (bounded by the usual fp32 summation bound).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "serq_internal.h"

namespace serq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------ quantization

// E2M1 code of t (|t| < 8): nearest of 0, .5, 1, 1.5, 2, 3, 4, 6, ties to
// the even mantissa (0, 1, 2, 4), saturated at 6; zero is code 0.
__device__ __forceinline__ uint32_t e2m1_code(float t) {
  const float a = fabsf(t);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return (t < 0.0f && c != 0u) ? (c | 8u) : c;
}

// One lane per 32-element block of one row: x^ = fl32(x * s_hat_inv), the
// block's exponent e = floor(log2(max |x^|)) - 2 (clamped to [-127, 127],
// -127 for a zero block) from the binary32 exponent field, then the codes of
// x^ * 2^-e (an exact scaling: |x^ 2^-e| < 8).
template <typename T>
__global__ __launch_bounds__(256) void serq_quant_act_mx_kernel(const T* __restrict__ X, const float* __restrict__ sinv,
                                                                int M, int K, uint8_t* __restrict__ Xq,
                                                                uint8_t* __restrict__ Xsc) {
  const int nb = K / 32;
  const long long g = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (g >= static_cast<long long>(M) * nb) return;
  const int m = static_cast<int>(g / nb), b = static_cast<int>(g % nb);
  const T* x = X + static_cast<size_t>(m) * K + 32 * b;
  const float* si = sinv + 32 * b;
  float v[32];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = reinterpret_cast<const uint4*>(x)[q];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = __uint_as_float(w[i] << 16);
        v[8 * q + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 u = reinterpret_cast<const float4*>(x)[q];
      v[4 * q] = u.x;
      v[4 * q + 1] = u.y;
      v[4 * q + 2] = u.z;
      v[4 * q + 3] = u.w;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 s4 = reinterpret_cast<const float4*>(si)[q];
    v[4 * q] *= s4.x;
    v[4 * q + 1] *= s4.y;
    v[4 * q + 2] *= s4.z;
    v[4 * q + 3] *= s4.w;
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(v[4 * q + i]));
  }
  const int biased = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);
  const int e = biased == 0 ? -127 : max(-127, biased - 127 - 2);
  const float down = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);    // 2^-e, a normal number
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t p = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) p |= e2m1_code(v[8 * q + i] * down) << (4 * i);
    w[q] = p;
  }
  reinterpret_cast<uint4*>(Xq + static_cast<size_t>(m) * (K / 2))[b] = make_uint4(w[0], w[1], w[2], w[3]);
  Xsc[static_cast<size_t>(m) * nb + b] = static_cast<uint8_t>(e + 127);
}

// ------------------------------------------------------------ the GEMM

// Workgroup tile: 128 output channels x 128 tokens, four waves of 64 x 64
// (2 x 2 blocks of 32 x 32; A = weight rows, B = token rows, so lane l of a
// block holds token l % 32 and channels 8 q + 4 (l / 32) + i). K runs in
// k-tiles of 128 elements (64 bytes and four E8M0 bytes per row), double
// buffered in LDS: the next k-tile's global loads are in flight while the
// current one's eight MFMAs per wave run. A k-tile is two MFMA steps of 64
// elements; in step s lane half h takes elements [64 s + 32 h, +32) of its
// row (16 bytes) and the scale of block 4 kt + 2 s + h. 16-byte row parts
// are stored XOR-swizzled (slot = part ^ swz(row)), so the 16 rows a
// fragment read touches hit distinct banks. Rows past M or N and elements
// past K load as zero codes.
constexpr int kMxTile = 128;
constexpr int kMxThreads = 256;

__device__ __forceinline__ int mx_swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

__device__ __forceinline__ v16f mfma_mx(uint4 a, uint4 b, int sa, int sb, v16f c) {
  const v8i av = v8i{static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z), static_cast<int>(a.w), 0, 0, 0, 0};
  const v8i bv = v8i{static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z), static_cast<int>(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

__device__ __forceinline__ uint32_t mx_pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// Workgroup -> tile: each XCD (workgroup b runs on XCD b % 8) takes a
// contiguous run of the tile order, which walks groups of 8 tile rows with
// the tile column fastest, so co-resident tiles share operand blocks in L2.
__device__ __forceinline__ void mx_tile_coords(int b, int nb, int n_tiles, int& tn, int& tm) {
  int l = b;
  if (nb % 8 == 0) l = (b % 8) * (nb / 8) + b / 8;
  const int m_tiles = nb / n_tiles;
  const int per_group = 8 * n_tiles;
  const int grp = l / per_group;
  const int first_m = grp * 8;
  const int gm = min(8, m_tiles - first_m);
  const int in = l - grp * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

struct MxStage {
  uint4 w[2], x[2];        // this thread's two 16-byte parts of each operand tile
  uint32_t ws, xs;         // one row's four scale bytes (threads 0..127: weights, 128..255: tokens)
};

__global__ __launch_bounds__(kMxThreads, 2) void serq_mx_tile_kernel(MxArgs a, int n_tiles) {
  __shared__ uint4 sW[2][kMxTile * 4];
  __shared__ uint4 sX[2][kMxTile * 4];
  __shared__ uint32_t sWs[2][kMxTile];
  __shared__ uint32_t sXs[2][kMxTile];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  int tn, tm;
  mx_tile_coords(blockIdx.x, gridDim.x, n_tiles, tn, tm);
  const int n0 = tn * kMxTile, m0 = tm * kMxTile;

  v16f acc[2][2], res[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = v16f{};
      res[i][j] = v16f{};
    }

  // One pass over `klen` elements of weight rows W (pitch wp bytes, scales
  // pitch wsp) against the first klen elements of the activation rows.
  auto pass = [&](const uint8_t* W, const uint8_t* Wsc, int wp, int wsp, int klen, v16f (&out)[2][2]) {
    const int nkt = (klen + kMxTile - 1) / kMxTile;
    const int xp = a.K / 2, xsp = a.K / 32;
    auto load = [&](int kt, MxStage& st) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int idx = tid + kMxThreads * i, row = idx >> 2, part = idx & 3;
        const int k0 = kt * kMxTile + 32 * part;           // first element of the part
        const int n = n0 + row, m = m0 + row;
        st.w[i] = (n < a.N && k0 < klen) ? *reinterpret_cast<const uint4*>(W + static_cast<size_t>(n) * wp + k0 / 2)
                                         : make_uint4(0, 0, 0, 0);
        st.x[i] = (m < a.M && k0 < klen) ? *reinterpret_cast<const uint4*>(a.Xq + static_cast<size_t>(m) * xp + k0 / 2)
                                         : make_uint4(0, 0, 0, 0);
      }
      const int row = tid & 127;
      const bool xside = tid >= 128;
      uint32_t sc = 0x7F7F7F7Fu;                           // unit scales for blocks past the end
      const int srow = (xside ? m0 : n0) + row;
      if (srow < (xside ? a.M : a.N)) {
        const uint8_t* p = xside ? a.Xsc + static_cast<size_t>(srow) * xsp : Wsc + static_cast<size_t>(srow) * wsp;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int blk = 4 * kt + q;
          if (32 * blk < klen) sc = (sc & ~(0xFFu << (8 * q))) | (static_cast<uint32_t>(p[blk]) << (8 * q));
        }
      }
      if (xside) st.xs = sc;
      else st.ws = sc;
    };
    auto store = [&](int buf, const MxStage& st) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int idx = tid + kMxThreads * i, row = idx >> 2, part = idx & 3;
        sW[buf][row * 4 + (part ^ mx_swz(row))] = st.w[i];
        sX[buf][row * 4 + (part ^ mx_swz(row))] = st.x[i];
      }
      if (tid >= 128) sXs[buf][tid & 127] = st.xs;
      else sWs[buf][tid] = st.ws;
    };
    MxStage st;
    load(0, st);
    store(0, st);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nkt) load(kt + 1, st);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int part = 2 * s + h;
        uint4 wa[2], xb[2];
        int sa[2], sb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int rw = wn * 64 + i * 32 + l32;
          wa[i] = sW[buf][rw * 4 + (part ^ mx_swz(rw))];
          sa[i] = static_cast<int>((sWs[buf][rw] >> (8 * part)) & 0xFFu);
          const int rx = wm * 64 + i * 32 + l32;
          xb[i] = sX[buf][rx * 4 + (part ^ mx_swz(rx))];
          sb[i] = static_cast<int>((sXs[buf][rx] >> (8 * part)) & 0xFFu);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) out[i][j] = mfma_mx(wa[i], xb[j], sa[i], sb[j], out[i][j]);
      }
      // buffer buf ^ 1 was last read in iteration kt - 1, which every wave
      // has left (the barrier below)
      if (kt + 1 < nkt) store(buf ^ 1, st);
      __syncthreads();
    }
  };

  pass(a.Wq, a.Wsc, a.K / 2, a.K / 32, a.K, acc);
  if (a.r > 0) pass(a.Rq, a.Rsc, a.r / 2, a.r / 32, a.r, res);

  // epilogue: y = acc_main + acc_res; lane holds token m and channels
  // n .. n + 3 of each group q
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = m0 + wm * 64 + j * 32 + l32;
      if (m >= a.M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 64 + i * 32 + 8 * q + 4 * h;
        float y[4], am[4], ar[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          am[e] = acc[i][j][4 * q + e];
          ar[e] = res[i][j][4 * q + e];
          y[e] = am[e] + ar[e];
        }
        const size_t base = static_cast<size_t>(m) * a.N + n;
        if (n + 3 < a.N && (a.N & 3) == 0) {
          if (a.y_bf16)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.Y) + base) =
                make_uint2(mx_pack_bf16x2(y[0], y[1]), mx_pack_bf16x2(y[2], y[3]));
          else
            *reinterpret_cast<float4*>(static_cast<float*>(a.Y) + base) = make_float4(y[0], y[1], y[2], y[3]);
          if (a.dbg_main) {
            *reinterpret_cast<float4*>(a.dbg_main + base) = make_float4(am[0], am[1], am[2], am[3]);
            *reinterpret_cast<float4*>(a.dbg_res + base) = make_float4(ar[0], ar[1], ar[2], ar[3]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (n + e >= a.N) break;
            if (a.y_bf16)
              static_cast<uint16_t*>(a.Y)[base + e] = static_cast<uint16_t>(mx_pack_bf16x2(y[e], 0.0f));
            else
              static_cast<float*>(a.Y)[base + e] = y[e];
            if (a.dbg_main) {
              a.dbg_main[base + e] = am[e];
              a.dbg_res[base + e] = ar[e];
            }
          }
        }
      }
    }
}

}  // namespace

hipError_t launch_quant_act_mx(const void* X, int x_bf16, int M, int K, const float* s_hat_inv, uint8_t* Xq,
                               uint8_t* Xsc, hipStream_t st) {
  const long long blocks = static_cast<long long>(M) * (K / 32);
  const long long grid = (blocks + 255) / 256;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if (x_bf16)
    serq_quant_act_mx_kernel<uint16_t><<<dim3(static_cast<unsigned>(grid)), dim3(256), 0, st>>>(
        static_cast<const uint16_t*>(X), s_hat_inv, M, K, Xq, Xsc);
  else
    serq_quant_act_mx_kernel<float><<<dim3(static_cast<unsigned>(grid)), dim3(256), 0, st>>>(
        static_cast<const float*>(X), s_hat_inv, M, K, Xq, Xsc);
  return hipGetLastError();
}

hipError_t launch_linear_mx(const MxArgs& a, hipStream_t st) {
  const int n_tiles = (a.N + kMxTile - 1) / kMxTile;
  const int m_tiles = (a.M + kMxTile - 1) / kMxTile;
  if (static_cast<long long>(n_tiles) * m_tiles > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  serq_mx_tile_kernel<<<dim3(n_tiles * m_tiles), dim3(kMxThreads), 0, st>>>(a, n_tiles);
  return hipGetLastError();
}

}  // namespace serq

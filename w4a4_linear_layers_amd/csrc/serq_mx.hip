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

typedef int v4i __attribute__((ext_vector_type(4)));
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

__device__ __forceinline__ v16f mfma_mx(v4i a, v4i b, int sa, int sb, v16f c) {
  const v8i av = v8i{a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  const v8i bv = v8i{b.x, b.y, b.z, b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

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

// ------------------------------------------------------------ pipelined GEMM

// The same product with a deeper pipeline, for K a multiple of 128: k-tiles
// of 128 elements (64 bytes of codes and 4 exponent bytes per row) stream
// through STAGES LDS buffers by direct global->LDS loads, as in the integer
// and bf6 tile kernels: every wave issues the same loads per k-tile (1 KB
// chunks of 16 rows x 64 bytes, one 256-byte chunk of 64 rows' exponent
// dwords), waits with s_waitcnt vmcnt, and one LDS-only barrier per k-tile
// publishes k-tile t + 1 and frees buffer t, which the loads of k-tile
// t + STAGES go into. Past the last k-tile the loads repeat it into a buffer
// that is never read again, so the wait counts are branch-free. A wave holds
// TN x TM blocks of 32 x 32. Fragment k: in MFMA step s lane half h takes
// elements [64 s + 32 h, +32) of its row (16 bytes; 16-byte row parts sit at
// slot part ^ swz(row), conflict-free) and the exponent byte 2 s + h of the
// row's dword, shifted down to the low byte the instruction reads. The
// residual (r/64 MFMA steps at most 4) runs in the epilogue from fragments
// read straight from memory, one weight block row at a time, and the output
// is y = acc_main + acc_res.

constexpr int kMxKt = 128;                    // elements per k-tile

// M0 is written in the asm and declared clobbered; the compiler sets it
// itself before every instruction of its own that reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void mx_dma16(const void* sbase, uint32_t voff, uint32_t lds_chunk) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(sbase), "s"(lds_chunk)
               : "memory", "m0");
}
__device__ __forceinline__ void mx_dma4(const void* sbase, uint32_t voff, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" :: "v"(voff), "s"(sbase), "s"(lds_dst)
               : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void mx_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0) only
  asm volatile("s_barrier" ::: "memory");
}
template <int N>
__device__ __forceinline__ void mx_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// Output-tile swizzle for bf16 rows (16-byte chunks XOR-ed with the row's
// low bits): the 8-byte half a lane writes moves to the other half of its
// chunk when mx_half_swap(row), which keeps the 8-byte writes of 16 (and 32)
// consecutive rows at one column on distinct banks.
__device__ __forceinline__ int mx_half_swap(int row) { return ((row >> 3) ^ (row >> 4)) & 1; }
// 16-byte part slot of a 64-byte row (bits 1-3 of the row): the 16-byte
// reads of 16 consecutive rows at one part hit distinct bank groups.
__device__ __forceinline__ int mx_swz64(int row) {
  return (((row >> 1) ^ (row >> 2)) & 1) | ((((row >> 2) ^ (row >> 3)) & 1) << 1);
}

template <int TN, int TM, int WNW, int WMW, int STAGES, int OCC>
struct MxCfg {
  static constexpr int NW = WNW * WMW, NT = 64 * NW;
  static constexpr int BN = 32 * TN * WNW, BM = 32 * TM * WMW;
  static constexpr int W_BYTES = BN * 64, X_BYTES = BM * 64;
  static constexpr int WS_OFF = W_BYTES + X_BYTES, XS_OFF = WS_OFF + BN * 4;
  static constexpr int STAGE = XS_OFF + BM * 4;
  static constexpr int CW = W_BYTES / 1024 / NW, CX = X_BYTES / 1024 / NW;   // 1 KB chunks per wave
  static constexpr int LOADS = CW + CX + 1;                                  // + one exponent chunk
  static constexpr int LDS = STAGES * STAGE;
  static constexpr bool F32_VIA_LDS = BM * BN * 4 <= LDS;    // else fp32 outputs are stored element-wise
  static_assert(BM * BN * 2 <= LDS && BN * 2 / 16 >= 16, "bf16 output tile in LDS");
  static_assert(CW * NW * 1024 == W_BYTES && CX * NW * 1024 == X_BYTES, "operand chunks split over the waves");
  static_assert((BN + BM) / 64 == NW, "one exponent chunk per wave");
  static_assert(OCC * LDS <= 160 * 1024 && (STAGES - 1) * LOADS < 64, "LDS, vmcnt range");
};

template <int TN, int TM, int WNW, int WMW, int STAGES, int OCC>
__global__ __launch_bounds__(64 * WNW * WMW, OCC) void serq_mx_pipe_kernel(MxArgs a, int n_tiles) {
  using C = MxCfg<TN, TM, WNW, WMW, STAGES, OCC>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int wn = wv / WMW, wm = wv % WMW;
  const int l32 = lane & 31, h = lane >> 5;
  int tile_n, tile_m;
  mx_tile_coords(blockIdx.x, gridDim.x, n_tiles, tile_n, tile_m);
  const int n0 = __builtin_amdgcn_readfirstlane(tile_n * C::BN);
  const int m0 = __builtin_amdgcn_readfirstlane(tile_m * C::BM);
  const int nk = a.K / kMxKt;
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const uint8_t* const Wq = a.Wq;
  const uint8_t* const Xq = a.Xq;
  const uint8_t* const Wsc = a.Wsc;
  const uint8_t* const Xsc = a.Xsc;
  const uint32_t rowb = static_cast<uint32_t>(a.K / 2), scb = static_cast<uint32_t>(a.K / 32);

  // Per-lane source offsets of this wave's chunks at k-tile 0 (rows past
  // the matrix read its last row; those outputs are never stored).
  const int part = (lane & 3) ^ mx_swz64(lane >> 2);
  uint32_t woff[C::CW], xoff[C::CX];
#pragma unroll
  for (int c = 0; c < C::CW; ++c) {
    const int row = (wv * C::CW + c) * 16 + (lane >> 2);
    woff[c] = static_cast<uint32_t>(min(n0 + row, a.N - 1)) * rowb + part * 16;
  }
#pragma unroll
  for (int c = 0; c < C::CX; ++c) {
    const int row = (wv * C::CX + c) * 16 + (lane >> 2);
    xoff[c] = static_cast<uint32_t>(min(m0 + row, a.M - 1)) * rowb + part * 16;
  }
  // exponent chunk: waves [0, BN/64) take weight rows, the rest token rows
  const bool ws_side = wv < C::BN / 64;
  const uint8_t* const sc_src = ws_side ? Wsc : Xsc;
  const int sc_row = ws_side ? n0 + wv * 64 + lane : m0 + (wv - C::BN / 64) * 64 + lane;
  const uint32_t scoff = static_cast<uint32_t>(min(sc_row, (ws_side ? a.N : a.M) - 1)) * scb;
  const uint32_t sc_dst = ws_side ? C::WS_OFF + wv * 256 : C::XS_OFF + (wv - C::BN / 64) * 256;

  auto issue = [&](int t) {
    const int kt = min(t, nk - 1);
    const uint32_t dst = lds_base + (t % STAGES) * C::STAGE;
#pragma unroll
    for (int c = 0; c < C::CW; ++c) mx_dma16(Wq + kt * 64, woff[c], dst + (wv * C::CW + c) * 1024);
#pragma unroll
    for (int c = 0; c < C::CX; ++c) mx_dma16(Xq + kt * 64, xoff[c], dst + C::W_BYTES + (wv * C::CX + c) * 1024);
    mx_dma4(sc_src + kt * 4, scoff, dst + sc_dst);
  };
  struct Frags {
    v4i w[TN], x[TM];
    int ws[TN], xs[TM];
  };
  auto read = [&](int buf, int s, Frags& f) {
    const uint8_t* sb = lds + buf * C::STAGE;
    const int p = 2 * s + h;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int row = wn * 32 * TN + 32 * i + l32;
      f.w[i] = *reinterpret_cast<const v4i*>(sb + row * 64 + ((p ^ mx_swz64(row)) * 16));
      f.ws[i] = static_cast<int>(*reinterpret_cast<const uint32_t*>(sb + C::WS_OFF + row * 4) >> (8 * p));
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int row = wm * 32 * TM + 32 * j + l32;
      f.x[j] = *reinterpret_cast<const v4i*>(sb + C::W_BYTES + row * 64 + ((p ^ mx_swz64(row)) * 16));
      f.xs[j] = static_cast<int>(*reinterpret_cast<const uint32_t*>(sb + C::XS_OFF + row * 4) >> (8 * p));
    }
  };
  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v16f{};
  auto mm = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = mfma_mx(f.w[i], f.x[j], f.ws[i], f.xs[j], acc[i][j]);
  };
  // The MFMAs are pure values the compiler could move past the barrier:
  // empty asm statements on the accumulators and the next fragments keep
  // them in program order, so the matrix core has work while the wave waits.
  auto pin = [&]() {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) asm volatile("" : "+v"(acc[i][j]));
  };
  auto pin_frags = [&](Frags& f) {
#pragma unroll
    for (int i = 0; i < TN; ++i) asm volatile("" : "+v"(f.w[i]), "+v"(f.ws[i]));
#pragma unroll
    for (int j = 0; j < TM; ++j) asm volatile("" : "+v"(f.x[j]), "+v"(f.xs[j]));
  };

#pragma unroll
  for (int p = 0; p < STAGES; ++p) issue(p);
  mx_wait_vmcnt<(STAGES - 1) * C::LOADS>();
  mx_lds_barrier();
  Frags f0, f1;
  read(0, 0, f0);
  for (int t = 0; t < nk - 1; ++t) {
    read(t % STAGES, 1, f1);
    mm(f0);
    pin();
    mx_wait_vmcnt<(STAGES - 2) * C::LOADS>();
    mx_lds_barrier();
    issue(t + STAGES);
    pin_frags(f1);
    read((t + 1) % STAGES, 0, f0);
    mm(f1);
  }
  read((nk - 1) % STAGES, 1, f1);
  mm(f0);
  mm(f1);
  mx_wait_vmcnt<0>();                            // the repeated loads past the end, unused

  // Epilogue, one weight block row at a time: its residual MFMAs (fragments
  // read from memory; elements past r contribute zero), then
  // y = acc_main + acc_res, into an output tile in LDS (the stages are free
  // once every wave is here) that is then written with 16-byte row stores;
  // element-wise stores with the debug sums, or for fp32 tiles larger than
  // the LDS.
  const bool direct = a.dbg_main != nullptr || (!a.y_bf16 && !C::F32_VIA_LDS);
  if (!direct) mx_lds_barrier();
  const int nw = n0 + wn * 32 * TN, mw = m0 + wm * 32 * TM;
  const int rsteps = (a.r + 63) / 64;
  const uint32_t rrow = static_cast<uint32_t>(a.r / 2), rsc = static_cast<uint32_t>(a.r / 32);
  // Up to kRS residual steps (r <= 128 on the 256 tile, whose registers are
  // fuller, 256 on the 128 tile) the fragments wait in registers: the
  // activation side's, the same for every block row, loaded once, and each
  // block row's weight side loaded while the row before it is finished, so
  // that the epilogue waits for one load latency instead of one per block
  // row. Longer residuals load step by step.
  constexpr int kRS = TN * TM >= 8 ? 2 : 4;
  const bool rreg = rsteps <= kRS;
  uint4 rxf[TM][kRS];
  int rxs[TM][kRS];
  uint4 rwf[2][kRS];
  int rws[2][kRS];
  auto load_w = [&](int i, int buf) {
    const int nr = min(nw + 32 * i + l32, a.N - 1);
#pragma unroll
    for (int s = 0; s < kRS; ++s) {
      const int k0 = 64 * s + 32 * h;
      const bool in = s < rsteps && k0 < a.r;
      rwf[buf][s] = in ? *reinterpret_cast<const uint4*>(a.Rq + nr * rrow + k0 / 2) : make_uint4(0, 0, 0, 0);
      rws[buf][s] = in ? a.Rsc[nr * rsc + k0 / 32] : 127;
    }
  };
  if (rreg) {
#pragma unroll
    for (int s = 0; s < kRS; ++s) {
      const int k0 = 64 * s + 32 * h;
      const bool in = s < rsteps && k0 < a.r;
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int mr = min(mw + 32 * j + l32, a.M - 1);
        rxf[j][s] = in ? *reinterpret_cast<const uint4*>(Xq + mr * rowb + k0 / 2) : make_uint4(0, 0, 0, 0);
        rxs[j][s] = in ? Xsc[mr * scb + k0 / 32] : 127;
      }
    }
    load_w(0, 0);
  }
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    v16f res[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j) res[j] = v16f{};
    if (rreg) {
      if (i + 1 < TN) load_w(i + 1, (i + 1) & 1);
#pragma unroll
      for (int s = 0; s < kRS; ++s) {
        if (s >= rsteps) break;
#pragma unroll
        for (int j = 0; j < TM; ++j) res[j] = mfma_mx(rwf[i & 1][s], rxf[j][s], rws[i & 1][s], rxs[j][s], res[j]);
      }
    } else {
      const int nr = min(nw + 32 * i + l32, a.N - 1);
      for (int s = 0; s < rsteps; ++s) {
        const int k0 = 64 * s + 32 * h;
        const bool in = k0 < a.r;
        const uint4 wf = in ? *reinterpret_cast<const uint4*>(a.Rq + nr * rrow + k0 / 2) : make_uint4(0, 0, 0, 0);
        const int wsv = in ? a.Rsc[nr * rsc + k0 / 32] : 127;
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          const int mr = min(mw + 32 * j + l32, a.M - 1);
          const uint4 xf = in ? *reinterpret_cast<const uint4*>(Xq + mr * rowb + k0 / 2) : make_uint4(0, 0, 0, 0);
          const int xsv = in ? Xsc[mr * scb + k0 / 32] : 127;
          res[j] = mfma_mx(wf, xf, wsv, xsv, res[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = mw + 32 * j + l32;
      if (m >= a.M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nw + 32 * i + 8 * q + 4 * h;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * q + e] + res[j][4 * q + e];
        if (!direct) {
          const int row = wm * 32 * TM + 32 * j + l32;   // token within the tile
          if (a.y_bf16) {
            uint8_t* rp = lds + row * (C::BN * 2);
            const int c = (wn * 32 * TN + 32 * i) / 8 + q;
            *reinterpret_cast<uint2*>(rp + 16 * (c ^ (row & 15)) + (h ^ mx_half_swap(row)) * 8) =
                make_uint2(mx_pack_bf16x2(y[0], y[1]), mx_pack_bf16x2(y[2], y[3]));
          } else if constexpr (C::F32_VIA_LDS) {
            uint8_t* rp = lds + row * (C::BN * 4);
            const int c = (wn * 32 * TN + 32 * i + 8 * q + 4 * h) / 4;
            *reinterpret_cast<float4*>(rp + 16 * (c ^ (row & 15))) = make_float4(y[0], y[1], y[2], y[3]);
          }
          continue;
        }
        const size_t base = static_cast<size_t>(m) * a.N + n;
        if (n + 3 < a.N && (a.N & 3) == 0) {
          if (a.y_bf16)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.Y) + base) =
                make_uint2(mx_pack_bf16x2(y[0], y[1]), mx_pack_bf16x2(y[2], y[3]));
          else
            *reinterpret_cast<float4*>(static_cast<float*>(a.Y) + base) = make_float4(y[0], y[1], y[2], y[3]);
          if (a.dbg_main) {
            *reinterpret_cast<float4*>(a.dbg_main + base) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            *reinterpret_cast<float4*>(a.dbg_res + base) =
                make_float4(res[j][4 * q], res[j][4 * q + 1], res[j][4 * q + 2], res[j][4 * q + 3]);
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
              a.dbg_main[base + e] = acc[i][j][4 * q + e];
              a.dbg_res[base + e] = res[j][4 * q + e];
            }
          }
        }
      }
    }
  }
  if (direct) return;
  __syncthreads();
  // 16-byte chunks along the rows of Y (every LDS read first, then the
  // stores); ragged tails element by element.
  auto copy_out = [&](auto ebc) {
    constexpr int EB = decltype(ebc)::value;   // bytes per element
    constexpr int CPR = C::BN * EB / 16;       // chunks per tile row
    constexpr int EPC = 16 / EB;               // elements per chunk
    constexpr int RPP = C::NT / CPR;           // rows per pass
    constexpr int PASSES = C::BM / RPP;
    const int tid = threadIdx.x;
    const int c = tid % CPR;
    const int n = n0 + c * EPC;
    const bool vec = (a.N % EPC) == 0 && n + EPC <= a.N;
    uint4 v[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = p * RPP + tid / CPR;
      v[p] = *reinterpret_cast<const uint4*>(lds + row * C::BN * EB + 16 * (c ^ (row & 15)));
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = p * RPP + tid / CPR;
      if (m0 + row >= a.M) break;
      if (n >= a.N) continue;
      uint4 w = v[p];
      if (EB == 2 && mx_half_swap(row)) w = make_uint4(w.z, w.w, w.x, w.y);
      uint8_t* dst = static_cast<uint8_t*>(a.Y) + (static_cast<size_t>(m0 + row) * a.N + n) * EB;
      if (vec) {
        *reinterpret_cast<uint4*>(dst) = w;
      } else {
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
        for (int e = 0; e < EPC && n + e < a.N; ++e) {
          if (EB == 2)
            reinterpret_cast<uint16_t*>(dst)[e] = static_cast<uint16_t>(d[e >> 1] >> (16 * (e & 1)));
          else
            reinterpret_cast<uint32_t*>(dst)[e] = d[e];
        }
      }
    }
  };
  if (a.y_bf16)
    copy_out(std::integral_constant<int, 2>{});
  else if constexpr (C::F32_VIA_LDS)
    copy_out(std::integral_constant<int, 4>{});
}

// ---------------------------------------------------------------------------
// MX GEMV (one or two tokens, K a multiple of 128). Per 32-element block
// the FP4 codes of both operands become bf16 pairs by gfx950's scaled
// conversion (scale 1: the E2M1 values exactly), and v_dot2c_f32_bf16
// multiplies and sums them -- exactly, since every product is a multiple of
// 1/4 below 36 in magnitude and a block's sum stays below 2^11 -- then the
// block sum is scaled by 2^(ex + ew) (exact) and added to the token's fp32
// sum: one rounding per block, as in the matrix instruction. A wave streams
// 8 weight rows over a K range: each load instruction takes one 128-byte
// line (8 blocks) of each of the 8 rows, lane (row l / 8, block l % 8) 16
// bytes of it, plus that block's exponent byte. A workgroup of KP waves
// covers one row octet in KP K ranges; the activation codes and exponents
// are copied into LDS once per workgroup and converted at each use (a
// variant that converted them once into 64-byte bf16 blocks in LDS measured
// slower: four times the LDS reads per use). The residual's blocks (Q(R)
// and its exponents against the first activation blocks) are more lines of
// the last K range. Partial sums are added over a row's 8 lanes, then over
// the waves, in a fixed order.
// ---------------------------------------------------------------------------

constexpr int kMxGemvMaxTokens = 2;
// Lines per unit and lane, two units in flight. One line per unit measured
// fastest at one token (8B gate/up 14.5 us against 17.5 with four, 8B down
// 8.1 against 9.8, q_proj 4.5 against 5.0; the 70B-shaped layers 24.5-25.3
// against 26.5-26.8); eight was slower still.
constexpr int kMxGemvUnit = 1;
constexpr int kMxGemvMaxX = 96 * 1024;       // LDS bytes for the activation codes and exponents

typedef __bf16 mx_bf16x2 __attribute__((ext_vector_type(2)));

// The 16 bf16 pairs of a 32-element FP4 block (16 bytes).
__device__ __forceinline__ void mx_block_bf16(const uint4& v, mx_bf16x2 (&o)[16]) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[4 * i + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 0);
    o[4 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 1);
    o[4 * i + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 2);
    o[4 * i + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 3);
  }
}

template <int MT, int KP>
__global__ __launch_bounds__(64 * KP) void serq_mx_gemv_kernel(MxArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];   // [MT][K/2] codes, then [MT][K/32] exponents
  __shared__ float red[KP][2][MT][8];                             // [wave][main, residual][token][row]
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int r8 = lane >> 3, part = lane & 7;
  const int Kb = a.K / 2, Kblk = a.K / 32, rblk = a.r / 32;
  const int n = static_cast<int>(blockIdx.x) * 8 + r8;           // this lane's channel
  const int nrow = min(n, a.N - 1);
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int xe_off = MT * Kb;                                     // a multiple of 64

  // Activation codes (1 KB per load instruction) and exponents (256 bytes
  // per instruction) into LDS, spread over the waves: older than every
  // weight load of the wave.
  for (int q = wv; q < (MT * Kb + 1023) / 1024; q += KP) {
    const int off = 1024 * q + 16 * lane;
    if (off < MT * Kb) mx_dma16(a.Xq, static_cast<uint32_t>(off), lds_base + 1024 * q);
  }
  for (int q = wv; q < (MT * Kblk + 255) / 256; q += KP) {
    const int off = 256 * q + 4 * lane;
    if (off < MT * Kblk) mx_dma4(a.Xsc, static_cast<uint32_t>(off), lds_base + xe_off + 256 * q);
  }

  // This wave's lines [l0, l1) of its 8 rows, then (last K range) the
  // residual's lines. Line i of the wave: main line l0 + i, or residual
  // line l0 + i - l1.
  const int lines = (Kb + 127) / 128;
  const int per = (lines + KP - 1) / KP;
  const int l0 = min(wv * per, lines), l1 = min(l0 + per, lines);
  const bool res_here = a.r > 0 && wv == KP - 1;
  const int total = (l1 - l0) + (res_here ? (rblk + 7) / 8 : 0);
  const uint8_t* wrow = a.Wq + static_cast<size_t>(nrow) * Kb;
  const uint8_t* wsc = a.Wsc + static_cast<size_t>(nrow) * Kblk;
  const uint8_t* rrow = a.r > 0 ? a.Rq + static_cast<size_t>(nrow) * (a.r / 2) : wrow;
  const uint8_t* rsc = a.r > 0 ? a.Rsc + static_cast<size_t>(nrow) * rblk : wsc;
  // Block of line i for this lane (main or residual), and whether it counts.
  auto block_of = [&](int i, bool& res) {
    const int ii = min(i, max(total - 1, 0));
    res = res_here && l0 + ii >= l1;
    return (res ? l0 + ii - l1 : min(l0 + ii, lines - 1)) * 8 + part;
  };
  // Every load is issued (lines past the end and blocks past a row's end
  // reload a valid block), so the compiler's load counters stay exact.
  struct Unit {
    uint4 w[kMxGemvUnit];
    uint32_t e[kMxGemvUnit];
  };
  auto issue = [&](int u, Unit& b) {
#pragma unroll
    for (int k = 0; k < kMxGemvUnit; ++k) {
      bool res;
      const int blk = block_of(u * kMxGemvUnit + k, res);
      const int cb = min(blk, (res ? rblk : Kblk) - 1);
      b.w[k] = *reinterpret_cast<const uint4*>((res ? rrow : wrow) + 16 * cb);
      b.e[k] = (res ? rsc : wsc)[cb];
    }
  };
  float acc[MT], accr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = accr[t] = 0.0f;
  auto consume = [&](int u, const Unit& b) {
#pragma unroll
    for (int k = 0; k < kMxGemvUnit; ++k) {
      const int i = u * kMxGemvUnit + k;
      bool res;
      const int blk = block_of(i, res);
      if (i >= total || blk >= (res ? rblk : Kblk)) continue;
      mx_bf16x2 wc[16];
      mx_block_bf16(b.w[k], wc);
      const int ew = static_cast<int>(b.e[k] & 0xFFu);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        mx_bf16x2 xc[16];
        mx_block_bf16(*reinterpret_cast<const uint4*>(lds + t * Kb + 16 * blk), xc);
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) s = __builtin_amdgcn_fdot2_f32_bf16(wc[q], xc[q], s, false);
        const int ex = lds[xe_off + t * Kblk + blk];
        const float v = ldexpf(s, ew + ex - 254);
        if (res) accr[t] += v; else acc[t] += v;
      }
    }
  };
  auto fence_sums = [&]() {
#pragma unroll
    for (int t = 0; t < MT; ++t) asm volatile("" : "+v"(acc[t]), "+v"(accr[t]) :: "memory");
  };
  Unit A, B;
  issue(0, A);
  // The activation copies are older than the weight loads (two per line):
  // once only those are outstanding, this wave's copies have landed.
  mx_wait_vmcnt<2 * kMxGemvUnit>();
  mx_lds_barrier();
  const int units = (total + kMxGemvUnit - 1) / kMxGemvUnit;
  int u = 0;
  for (; u + 2 <= units; u += 2) {
    issue(u + 1, B);
    consume(u, A);
    fence_sums();
    issue(u + 2, A);
    consume(u + 1, B);
    fence_sums();
  }
  if (u < units) consume(u, A);
  mx_wait_vmcnt<0>();                            // the last issue, past the end, unused

  // Over the row's 8 lanes (fixed order), then over the waves in order.
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      acc[t] += __shfl_xor(acc[t], o);
      accr[t] += __shfl_xor(accr[t], o);
    }
  }
  if (part == 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      red[wv][0][t][r8] = acc[t];
      red[wv][1][t][r8] = accr[t];
    }
  }
  __syncthreads();
  if (wv == 0 && lane < 8 * MT) {
    const int t = lane >> 3, row = lane & 7;
    const int nn = static_cast<int>(blockIdx.x) * 8 + row;
    if (t < a.M && nn < a.N) {
      float sm = red[0][0][t][row], sr = red[0][1][t][row];
#pragma unroll
      for (int w = 1; w < KP; ++w) {
        sm += red[w][0][t][row];
        sr += red[w][1][t][row];
      }
      const float y = sm + sr;
      const size_t o = static_cast<size_t>(t) * a.N + nn;
      if (a.y_bf16)
        static_cast<uint16_t*>(a.Y)[o] = static_cast<uint16_t>(mx_pack_bf16x2(y, 0.0f));
      else
        static_cast<float*>(a.Y)[o] = y;
      if (a.dbg_main) {
        a.dbg_main[o] = sm;
        a.dbg_res[o] = sr;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MX skinny kernel (up to 16 tokens, K a multiple of 128): one eight-wave
// workgroup per 16 output channels, on v_mfma_scale_f32_16x16x128_f8f6f4
// with FP4 operands -- A the 16 weight rows, B the (zero-padded) 16 token
// rows, a lane's operand the 16 stored bytes of its row's 32-element block
// (row l % 16, block l / 16 of the 128-element chunk) and its scale operand
// that block's exponent byte, so nothing is converted. Wave w takes pairs
// of chunks w, w + 8, ... of the main K and of the residual, a lane loading
// two adjacent blocks of its rows (a 128-byte line of a row per four lanes),
// the next pair's loads issued as the current pair's two MFMAs go out (two
// blocks per lane with one pair in flight measured faster than four chunks
// of single blocks in flight, 20 % on q_proj at 16 tokens, 11 % on
// 28672 x 8192; deeper rings and wider lanes were slower), and keeps its two
// 16 x 16 sums in registers; the eight waves' sums are added through LDS in
// a fixed order (deterministic; one rounding per block in the matrix
// instruction, eight more).
// ---------------------------------------------------------------------------

constexpr int kMxSkinnyMaxTokens = 16;
constexpr int kMxSkinnyWaves = 8;
constexpr int kMxSkinnyRing = 1;              // items in flight per wave
constexpr int kMxSkinnyP = 2;                 // consecutive blocks per lane and item

typedef float mx_v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ mx_v4f mfma_mx16(const uint4& a, const uint4& b, int sa, int sb, mx_v4f c) {
  const v8i av = v8i{static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z), static_cast<int>(a.w), 0, 0, 0, 0};
  const v8i bv = v8i{static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z), static_cast<int>(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

__global__ __launch_bounds__(64 * kMxSkinnyWaves) void serq_mx_skinny_kernel(MxArgs a) {
  __shared__ mx_v4f red[kMxSkinnyWaves][2][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int l16 = lane & 15, kq = lane >> 4;
  const int Kb = a.K / 2, Kblk = a.K / 32;
  const int rblk = a.r / 32;
  const int nch = a.K / 128;                       // main chunks
  const int rch = (a.r + 127) / 128;               // residual chunks (the last may be partial)
  const int ch = min(static_cast<int>(blockIdx.x) * 16 + l16, a.N - 1);   // this lane's weight row
  const int tk = min(l16, a.M - 1);                                      // this lane's token row
  const bool tok_in = l16 < a.M;
  const uint8_t* wrow = a.Wq + static_cast<size_t>(ch) * Kb;
  const uint8_t* wsc = a.Wsc + static_cast<size_t>(ch) * Kblk;
  const uint8_t* rrow = a.r > 0 ? a.Rq + static_cast<size_t>(ch) * (a.r / 2) : wrow;
  const uint8_t* rsc = a.r > 0 ? a.Rsc + static_cast<size_t>(ch) * rblk : wsc;
  const uint8_t* xrow = a.Xq + static_cast<size_t>(tk) * Kb;
  const uint8_t* xsc = a.Xsc + static_cast<size_t>(tk) * Kblk;
  // This wave's items: P consecutive main chunks (blocks 4 P p .. 4 P p +
  // 4 P - 1 of the row), p = wv, wv + 8, ..., then P residual chunks at a
  // time. A lane loads the 16 P contiguous bytes of blocks P kq .. P kq + P - 1
  // of its rows, so four lanes read 64 P contiguous bytes of a row per
  // request; MFMA e of the item takes every lane's block P kq + e -- the same
  // products, the same block on both sides.
  constexpr int P = kMxSkinnyP;
  const int npm = (nch + P - 1) / P, npr = (rch + P - 1) / P;   // main and residual items
  const int nmain = npm > wv ? (npm - wv + kMxSkinnyWaves - 1) / kMxSkinnyWaves : 0;
  const int nres = npr > wv ? (npr - wv + kMxSkinnyWaves - 1) / kMxSkinnyWaves : 0;
  const int total = nmain + nres;
  struct Item {
    uint4 w[P], x[P];
    uint32_t ew[P], ex[P];
  };
  // Item i's loads (past the end: the last item's, never used); a block past
  // the row (K or r) reads block 0 of the row and is zeroed before use.
  auto load = [&](int i, Item& it) {
    const int ii = min(i, max(total - 1, 0));
    const bool res = ii >= nmain;
    const int pp = wv + kMxSkinnyWaves * (res ? ii - nmain : ii);
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const int blk = 4 * P * pp + P * kq + e;
      const int b = blk < (res ? rblk : Kblk) ? blk : 0;
      it.w[e] = *reinterpret_cast<const uint4*>((res ? rrow : wrow) + 16 * b);
      it.ew[e] = (res ? rsc : wsc)[b];
      it.x[e] = *reinterpret_cast<const uint4*>(xrow + 16 * b);
      it.ex[e] = xsc[b];
    }
  };
  mx_v4f acc = mx_v4f{0.f, 0.f, 0.f, 0.f}, accr = mx_v4f{0.f, 0.f, 0.f, 0.f};
  auto use = [&](int i, const Item& it) {
    if (i >= total) return;
    const bool res = i >= nmain;
    const int pp = wv + kMxSkinnyWaves * (res ? i - nmain : i);
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const bool blk_in = 4 * P * pp + P * kq + e < (res ? rblk : Kblk);
      const uint4 z = make_uint4(0, 0, 0, 0);
      const uint4 w = blk_in ? it.w[e] : z;
      const uint4 x = (blk_in && tok_in) ? it.x[e] : z;
      const int ew = static_cast<int>(it.ew[e] & 0xFFu), ex = static_cast<int>(it.ex[e] & 0xFFu);
      if (res)
        accr = mfma_mx16(w, x, ew, ex, accr);
      else
        acc = mfma_mx16(w, x, ew, ex, acc);
    }
  };
  Item ring[kMxSkinnyRing];
#pragma unroll
  for (int k = 0; k < kMxSkinnyRing; ++k) load(k, ring[k]);
  for (int i0 = 0; i0 < total; i0 += kMxSkinnyRing) {
#pragma unroll
    for (int k = 0; k < kMxSkinnyRing; ++k) {
      use(i0 + k, ring[k]);
      load(i0 + k + kMxSkinnyRing, ring[k]);
    }
  }
  red[wv][0][lane] = acc;
  red[wv][1][lane] = accr;
  __syncthreads();
  if (wv == 0) {
    mx_v4f sm = red[0][0][lane], sr = red[0][1][lane];
#pragma unroll
    for (int w = 1; w < kMxSkinnyWaves; ++w) {
      sm += red[w][0][lane];
      sr += red[w][1][lane];
    }
    // lane: token l16, channels 16 g + 4 kq + (0..3)
    const int n = static_cast<int>(blockIdx.x) * 16 + 4 * kq;
    if (tok_in) {
      const size_t o = static_cast<size_t>(l16) * a.N + n;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = sm[e] + sr[e];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n + e >= a.N) break;
        if (a.y_bf16)
          static_cast<uint16_t*>(a.Y)[o + e] = static_cast<uint16_t>(mx_pack_bf16x2(y[e], 0.0f));
        else
          static_cast<float*>(a.Y)[o + e] = y[e];
        if (a.dbg_main) {
          a.dbg_main[o + e] = sm[e];
          a.dbg_res[o + e] = sr[e];
        }
      }
    }
  }
}

// LDS bytes of the GEMV's activations: codes, then exponents.
inline long long mx_gemv_lds(int M, int K) {
  return static_cast<long long>(M) * (K / 2) + static_cast<long long>(M) * (K / 32);
}

template <int MT, int KP>
hipError_t launch_mx_gemv_kp(const MxArgs& a, hipStream_t st) {
  static bool set = false;                    // idempotent: setting it again is harmless
  auto* fn = &serq_mx_gemv_kernel<MT, KP>;
  if (!set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kMxGemvMaxX);
    if (e != hipSuccess) return e;
    set = true;
  }
  fn<<<dim3((a.N + 7) / 8), dim3(64 * KP), static_cast<size_t>(mx_gemv_lds(a.M, a.K)), st>>>(a);
  return hipGetLastError();
}

// Eight K ranges per row octet when the layer has few octets (so that it
// still keeps about sixteen waves per CU loading), else four.
template <int MT>
hipError_t launch_mx_gemv(const MxArgs& a, hipStream_t st) {
  if ((a.N + 7) / 8 < 4 * 256) return launch_mx_gemv_kp<MT, 8>(a, st);
  return launch_mx_gemv_kp<MT, 4>(a, st);
}

template <int TN, int TM, int WNW, int WMW, int STAGES, int OCC>
hipError_t launch_mx_pipe(const MxArgs& a, hipStream_t st) {
  using C = MxCfg<TN, TM, WNW, WMW, STAGES, OCC>;
  auto* fn = &serq_mx_pipe_kernel<TN, TM, WNW, WMW, STAGES, OCC>;
  static bool attr_set = false;              // idempotent: setting it again is harmless
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       C::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int n_tiles = (a.N + C::BN - 1) / C::BN;
  const int m_tiles = (a.M + C::BM - 1) / C::BM;
  if (static_cast<long long>(n_tiles) * m_tiles > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  fn<<<dim3(n_tiles * m_tiles), dim3(C::NT), C::LDS, st>>>(a, n_tiles);
  return hipGetLastError();
}

}  // namespace

// Which MXFP4 kernel serq_linear_mx launches: 0 the plain double-buffered
// one (K not a multiple of 128, or 32-bit row offsets not enough), 1 the
// pipelined 128 x 128 tile, 2 the pipelined 256 x 256 tile (when it still
// gives every CU a tile).
int mx_kernel_kind(int M, int K, int N) {
  if (K % kMxKt != 0 || static_cast<uint64_t>(N) * (K / 2) >= (1ull << 32) ||
      static_cast<uint64_t>(M) * (K / 2) >= (1ull << 32))
    return 0;
  const long long t256 = static_cast<long long>((M + 255) / 256) * ((N + 255) / 256);
  return t256 >= 256 ? 2 : 1;
}

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
  // the pipelined kernels load exponent dwords, so those arrays must be 4-byte aligned
  const bool sc_aligned = ((reinterpret_cast<uintptr_t>(a.Wsc) | reinterpret_cast<uintptr_t>(a.Xsc)) & 3u) == 0;
  // Few tokens. On layers whose 128-channel tiles would leave half the CUs
  // idle or more (N < 16384): the GEMV up to two tokens, the skinny kernel
  // up to sixteen (its time grows slowly with the tokens, the GEMV's by a
  // conversion pass per token: 8B down at four tokens 17.2 us on the GEMV,
  // 14.9 at five on the skinny kernel; q_proj at 16 tokens 9.2 against 15.1
  // tiled, 8B down 19.9 against 41.5). On wider layers the tile kernel
  // fills the CUs and from two tokens on is faster than both (4096 x 28672:
  // 20.3 us at four tokens, 29.4 on the GEMV; 21.0 at sixteen, 48.5 on the
  // skinny kernel); one token takes the GEMV there too.
  const bool narrow = a.N < 16384;
  if (sc_aligned && (a.M == 1 || (a.M <= kMxGemvMaxTokens && narrow)) && a.K % kMxKt == 0 &&
      mx_gemv_lds(a.M, a.K) <= kMxGemvMaxX &&
      static_cast<uint64_t>(a.N) * (a.K / 2) < (1ull << 32)) {
    switch (a.M) {
      case 1: return launch_mx_gemv<1>(a, st);
      default: return launch_mx_gemv<2>(a, st);
    }
  }
  if (narrow && a.M <= kMxSkinnyMaxTokens && a.K % kMxKt == 0 &&
      static_cast<uint64_t>(a.N) * (a.K / 2) < (1ull << 32)) {
    serq_mx_skinny_kernel<<<dim3((a.N + 15) / 16), dim3(64 * kMxSkinnyWaves), 0, st>>>(a);
    return hipGetLastError();
  }
  const int kind = sc_aligned ? mx_kernel_kind(a.M, a.K, a.N) : 0;
  if (kind == 2) return launch_mx_pipe<4, 2, 2, 4, 4, 1>(a, st);
  // 128 x 128 tiles with three stages: 1-4 % faster than four on 512-2048
  // tokens of q_proj, 8B gate/up and down (fewer loads in flight per CU)
  if (kind == 1) return launch_mx_pipe<2, 2, 2, 2, 3, 2>(a, st);
  const int n_tiles = (a.N + kMxTile - 1) / kMxTile;
  const int m_tiles = (a.M + kMxTile - 1) / kMxTile;
  if (static_cast<long long>(n_tiles) * m_tiles > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  serq_mx_tile_kernel<<<dim3(n_tiles * m_tiles), dim3(kMxThreads), 0, st>>>(a, n_tiles);
  return hipGetLastError();
}

}  // namespace serq

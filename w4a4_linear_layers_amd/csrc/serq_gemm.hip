// The fused SERQ linear for gfx950:
//     acc_main = Xq . Q(W^)        over all K        (the pure 4-bit GEMM)
//     acc_res  = Xq[:, :r] . Q(R)  over the r salient channels
//     Y = sx[m] * (sw[n] * acc_main + sr[n] * acc_res)
// (papernotes.org SERQ notes, 关键设计 2: the residual is one
// (tokens x r)(r x d) product on the salient activation channels, computed
// beside the main path and added, with R quantized and no intermediate
// quantization; gist.science/ja "技術概要" 2 contrasts this single product
// with the serial two-factor form.)
//
// CDNA4 has no int4 matrix instruction, so 4-bit codes are widened to int8 in
// registers right before v_mfma_i32_16x16x64_i8. The widening keeps the
// nibble in the high half of each byte: for a packed dword w,
//     (w << 4) & 0xF0F0F0F0  = 16 * (codes 0, 2, 4, 6)
//      w       & 0xF0F0F0F0  = 16 * (codes 1, 3, 5, 7)
// two VALU ops per four int8 lanes and no sign extension. Both operands go
// through the same widening, so the k order inside a fragment is the same
// permutation on both sides and the dot product is unchanged; the int32 sum
// is exactly 256 * (true sum) for W4A4 (16 * for W4A8, where the int8
// activations are byte-shuffled into the same order). |acc| stays below
// 2^31 for K up to 2^17.
//
// MFMA operand roles: A = weight rows (16 output channels), B = activation
// rows (16 tokens), so D[n][m]; lane l of a 16x16 block holds tokens
// m = l % 16 and four consecutive channels n = 4 (l / 16) + i, which the
// epilogue writes as one 16- or 8-byte vector per lane.
//
// Fragment k layout: within a 128-code k-tile, lane group g = l / 16 of both
// operands holds codes [32 g, 32 g + 32) (16 packed bytes); MFMA step 0 uses
// its first 16 codes and step 1 the next 16.

#include <utility>

#include "serq_internal.h"

typedef int v4i __attribute__((ext_vector_type(4)));

namespace serq {
namespace {

constexpr int kThreads = 256;
constexpr int kKTileCodes = 128;            // codes per k-tile
constexpr int kKTileW = kKTileCodes / 2;    // packed weight bytes per row per k-tile
constexpr int kMaxResidual = 256;           // largest r handled by the tile kernels

// Compile-time loop: f(std::integral_constant<int, I>) for I in [0, N). Keeps
// register-array indices static where #pragma unroll may give up.
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 16 packed int4 codes (two dwords) -> 16 int8 lanes (x16), split order.
__device__ __forceinline__ v4i widen16(uint32_t p0, uint32_t p1) {
  v4i r;
  r.x = static_cast<int>((p0 << 4) & 0xF0F0F0F0u);
  r.y = static_cast<int>(p0 & 0xF0F0F0F0u);
  r.z = static_cast<int>((p1 << 4) & 0xF0F0F0F0u);
  r.w = static_cast<int>(p1 & 0xF0F0F0F0u);
  return r;
}

// Two packed int4 dwords -> split-order int8 (x16) as a uint2 (for LDS).
__device__ __forceinline__ uint2 widen8(uint32_t p) {
  return make_uint2((p << 4) & 0xF0F0F0F0u, p & 0xF0F0F0F0u);
}

// 8 int8 codes in natural order (two dwords) -> even codes, odd codes.
__device__ __forceinline__ uint2 split8(uint32_t d0, uint32_t d1) {
  return make_uint2(__builtin_amdgcn_perm(d1, d0, 0x06040200u),
                    __builtin_amdgcn_perm(d1, d0, 0x07050301u));
}

// 16 int8 codes in natural order -> the split order of widen16.
__device__ __forceinline__ v4i split16(uint4 d) {
  const uint2 a = split8(d.x, d.y), b = split8(d.z, d.w);
  v4i r;
  r.x = static_cast<int>(a.x);
  r.y = static_cast<int>(a.y);
  r.z = static_cast<int>(b.x);
  r.w = static_cast<int>(b.y);
  return r;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Bytes [off, off + 4) of a row with `valid` bytes; zero beyond. Dword load
// when the row length keeps dwords aligned.
__device__ __forceinline__ uint32_t load_dword_masked(const uint8_t* row, int off, int valid) {
  if (off >= valid) return 0u;
  if ((valid & 3) == 0) return *reinterpret_cast<const uint32_t*>(row + off);
  uint32_t w = 0;
  for (int b = 0; b < 4 && off + b < valid; ++b) w |= static_cast<uint32_t>(row[off + b]) << (8 * b);
  return w;
}

// Epilogue for one 16x16 block: lane owns token m and channels n..n+3.
template <int SHIFT>
__device__ __forceinline__ void store_block(const LinearArgs& a, v4i am, v4i ar, int m, int n,
                                            bool has_res) {
  if (m >= a.M) return;
  const float sxm = a.sx[m];
  const size_t base = static_cast<size_t>(m) * a.N + n;
  if (a.dbg_main) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (n + i < a.N) {
        a.dbg_main[base + i] = am[i] >> SHIFT;
        a.dbg_res[base + i] = ar[i] >> SHIFT;
      }
    }
  }
  float y[4];
  if (n + 3 < a.N && (a.N & 3) == 0) {
    const float4 w4 = *reinterpret_cast<const float4*>(a.sw + n);
    float4 r4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (has_res) r4 = *reinterpret_cast<const float4*>(a.sr + n);
    const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
    const float rv[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float fm = static_cast<float>(am[i] >> SHIFT);
      const float fr = static_cast<float>(ar[i] >> SHIFT);
      y[i] = sxm * __builtin_fmaf(rv[i], fr, wv[i] * fm);
    }
    if (a.y_bf16) {
      uint2 o;
      o.x = f32_to_bf16_rne(y[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(y[1])) << 16);
      o.y = f32_to_bf16_rne(y[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(y[3])) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.Y) + base) = o;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.Y) + base) = make_float4(y[0], y[1], y[2], y[3]);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (n + i >= a.N) break;
    const float fm = static_cast<float>(am[i] >> SHIFT);
    const float fr = static_cast<float>(ar[i] >> SHIFT);
    const float srn = has_res ? a.sr[n + i] : 0.0f;
    const float yi = sxm * __builtin_fmaf(srn, fr, a.sw[n + i] * fm);
    if (a.y_bf16)
      static_cast<uint16_t*>(a.Y)[base + i] = f32_to_bf16_rne(yi);
    else
      static_cast<float*>(a.Y)[base + i] = yi;
  }
}

// ---------------------------------------------------------------------------
// Macro-tile kernel (prefill-sized M): a 256-lane workgroup computes a
// (32 TM tokens) x (32 TN channels) tile with 2 x 2 waves; each wave owns
// TN x TM blocks of 16 x 16. Packed tiles are staged through LDS with a
// two-stage pipeline (global loads for k-tile t+1 in flight while the MFMAs of
// k-tile t run). After the K loop the LDS is reused for the residual: the
// r salient activation columns and Q(R) are widened once into LDS, and each
// block's residual MFMAs run right before its epilogue, so the residual needs
// only one 4-register accumulator at a time.
// ---------------------------------------------------------------------------

template <int TN, int TM, int A_BITS>
struct TileCfg {
  static constexpr int WN = 16 * TN, WM = 16 * TM;       // wave tile
  static constexpr int BN = 2 * WN, BM = 2 * WM;         // workgroup tile
  static constexpr int XB = kKTileCodes * A_BITS / 8;    // activation bytes / row / k-tile
  static constexpr int WS = kKTileW + 16;                // LDS row strides (bank-conflict free
  static constexpr int XS = XB + 16;                     //  16-byte reads)
  static constexpr int STAGE = BN * WS + BM * XS;
  static constexpr int W_CHUNKS = BN * kKTileW / 16 / kThreads;
  static constexpr int X_CHUNKS = BM * XB / 16 / kThreads;
  static constexpr int SHIFT = A_BITS == 4 ? 8 : 4;
  static constexpr int pipeline_bytes() { return 2 * STAGE; }
  static constexpr int residual_bytes(int rp) { return (BN + BM) * (rp + 16); }
};

template <int TN, int TM, int A_BITS>
__global__ __launch_bounds__(kThreads) void serq_tile_kernel(LinearArgs a, int n_tiles) {
  using C = TileCfg<TN, TM, A_BITS>;
  static_assert(C::W_CHUNKS * kThreads * 16 == C::BN * kKTileW, "W tile must split evenly");
  static_assert(C::X_CHUNKS * kThreads * 16 == C::BM * C::XB, "X tile must split evenly");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int l16 = lane & 15, g = lane >> 4;
  const int tile_n = blockIdx.x % n_tiles, tile_m = blockIdx.x / n_tiles;
  const int n0 = tile_n * C::BN, m0 = tile_m * C::BM;
  const int Kb = a.K / 2;                      // packed weight bytes per row
  const int Xrow = a.K * A_BITS / 8;           // activation bytes per row
  const int nkt = (Kb + kKTileW - 1) / kKTileW;

  // global -> register staging assignment (16-byte chunks)
  const uint8_t* wsrc[C::W_CHUNKS];
  int wdst[C::W_CHUNKS], woff[C::W_CHUNKS];
#pragma unroll
  for (int i = 0; i < C::W_CHUNKS; ++i) {
    const int c = tid + i * kThreads, row = c >> 2, part = c & 3;
    wsrc[i] = a.Wq + static_cast<size_t>(min(n0 + row, a.N - 1)) * Kb + part * 16;
    woff[i] = part * 16;
    wdst[i] = row * C::WS + part * 16;
  }
  const uint8_t* xsrc[C::X_CHUNKS];
  int xdst[C::X_CHUNKS], xoff[C::X_CHUNKS];
  constexpr int XPARTS = C::XB / 16;
#pragma unroll
  for (int i = 0; i < C::X_CHUNKS; ++i) {
    const int c = tid + i * kThreads, row = c / XPARTS, part = c % XPARTS;
    xsrc[i] = a.Xq + static_cast<size_t>(min(m0 + row, a.M - 1)) * Xrow + part * 16;
    xoff[i] = part * 16;
    xdst[i] = C::BN * C::WS + row * C::XS + part * 16;
  }
  uint4 wreg[C::W_CHUNKS], xreg[C::X_CHUNKS];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::W_CHUNKS; ++i) {
      const int o = kt * kKTileW + woff[i];
      wreg[i] = o < Kb ? *reinterpret_cast<const uint4*>(wsrc[i] + kt * kKTileW) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::X_CHUNKS; ++i) {
      const int o = kt * C::XB + xoff[i];
      xreg[i] = o < Xrow ? *reinterpret_cast<const uint4*>(xsrc[i] + kt * C::XB) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* base = lds + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::W_CHUNKS; ++i) *reinterpret_cast<uint4*>(base + wdst[i]) = wreg[i];
#pragma unroll
    for (int i = 0; i < C::X_CHUNKS; ++i) *reinterpret_cast<uint4*>(base + xdst[i]) = xreg[i];
  };

  v4i acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int wrow0 = (wn * C::WN + l16) * C::WS + g * 16;
  const int xrow0 = C::BN * C::WS + (wm * C::WM + l16) * C::XS + g * (A_BITS == 4 ? 16 : 32);

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    const uint8_t* sb = lds + buf * C::STAGE;
    uint4 wf[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) wf[i] = *reinterpret_cast<const uint4*>(sb + wrow0 + i * 16 * C::WS);
    if constexpr (A_BITS == 4) {
      uint4 xf[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j) xf[j] = *reinterpret_cast<const uint4*>(sb + xrow0 + j * 16 * C::XS);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v4i wa[TN], xb[TM];
#pragma unroll
        for (int i = 0; i < TN; ++i) wa[i] = s ? widen16(wf[i].z, wf[i].w) : widen16(wf[i].x, wf[i].y);
#pragma unroll
        for (int j = 0; j < TM; ++j) xb[j] = s ? widen16(xf[j].z, xf[j].w) : widen16(xf[j].x, xf[j].y);
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j) acc[i][j] = mfma(wa[i], xb[j], acc[i][j]);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v4i wa[TN], xb[TM];
#pragma unroll
        for (int j = 0; j < TM; ++j)
          xb[j] = split16(*reinterpret_cast<const uint4*>(sb + xrow0 + j * 16 * C::XS + s * 16));
#pragma unroll
        for (int i = 0; i < TN; ++i) wa[i] = s ? widen16(wf[i].z, wf[i].w) : widen16(wf[i].x, wf[i].y);
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j) acc[i][j] = mfma(wa[i], xb[j], acc[i][j]);
      }
    }
    if (kt + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- residual operands, widened once into LDS (reusing the pipeline space)
  const int r = a.r;
  const bool has_res = r > 0;
  const int rp = (r + 63) & ~63;             // padded with zero codes
  const int RS = rp + 16;
  uint8_t* Rw = lds;
  uint8_t* Rx = lds + C::BN * RS;
  if (has_res) {
    const int groups = rp / 8;               // 8 codes per group
    const int rbytes = r / 2;
    for (int e = tid; e < C::BN * groups; e += kThreads) {
      const int row = e / groups, gi = e - row * groups;
      const uint8_t* src = a.Rq + static_cast<size_t>(min(n0 + row, a.N - 1)) * rbytes;
      *reinterpret_cast<uint2*>(Rw + row * RS + gi * 8) = widen8(load_dword_masked(src, gi * 4, rbytes));
    }
    for (int e = tid; e < C::BM * groups; e += kThreads) {
      const int row = e / groups, gi = e - row * groups;
      const uint8_t* src = a.Xq + static_cast<size_t>(min(m0 + row, a.M - 1)) * Xrow;
      uint2 v;
      if constexpr (A_BITS == 4) {
        v = widen8(load_dword_masked(src, gi * 4, rbytes));
      } else {
        v = split8(load_dword_masked(src, gi * 8, r), load_dword_masked(src, gi * 8 + 4, r));
      }
      *reinterpret_cast<uint2*>(Rx + row * RS + gi * 8) = v;
    }
    __syncthreads();
  }
  const int nks = rp / 64;

  // ---- per block: residual MFMAs, then the epilogue
  static_for<TM>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    v4i xr[kMaxResidual / 64];
#pragma unroll
    for (int s = 0; s < kMaxResidual / 64; ++s)
      xr[s] = s < nks ? *reinterpret_cast<const v4i*>(Rx + (wm * C::WM + j * 16 + l16) * RS + s * 64 + g * 16)
                      : v4i{0, 0, 0, 0};
    static_for<TN>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      v4i ar = v4i{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < kMaxResidual / 64; ++s)
        if (s < nks)
          ar = mfma(*reinterpret_cast<const v4i*>(Rw + (wn * C::WN + i * 16 + l16) * RS + s * 64 + g * 16),
                    xr[s], ar);
      store_block<C::SHIFT>(a, acc[i][j], ar, m0 + wm * C::WM + j * 16 + l16,
                            n0 + wn * C::WN + i * 16 + 4 * g, has_res);
    });
  });
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 32): the packed weights are streamed from HBM exactly
// once. A workgroup owns 16 output channels; its four waves take interleaved
// 128-code chunks of K, so together they read 256 contiguous bytes of each
// weight row per step. Activations (a few KB) come through L2. The residual
// chunks are spread over the waves the same way, then the partial int32
// accumulators are summed through LDS and wave 0 runs the epilogue.
// ---------------------------------------------------------------------------

template <int MG, int A_BITS>
__global__ __launch_bounds__(kThreads) void serq_decode_kernel(LinearArgs a) {
  constexpr int SHIFT = A_BITS == 4 ? 8 : 4;
  constexpr int XCB = kKTileCodes * A_BITS / 8;       // activation bytes per chunk
  constexpr int UNROLL = 4;
  __shared__ v4i red[2][kThreads / 64 - 1][MG][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int Kb = a.K / 2, Xrow = a.K * A_BITS / 8;
  const uint8_t* wp = a.Wq + static_cast<size_t>(min(n0 + l16, a.N - 1)) * Kb + g * 16;
  const uint8_t* xp[MG];
  bool xv[MG];
#pragma unroll
  for (int j = 0; j < MG; ++j) {
    const int m = j * 16 + l16;
    xv[j] = m < a.M;
    xp[j] = a.Xq + static_cast<size_t>(min(m, a.M - 1)) * Xrow + g * (XCB / 4);
  }
  const int nchunks = (Kb + kKTileW - 1) / kKTileW;

  auto chunk = [&](int c, v4i (&acc)[MG], const uint8_t* wbase, int wlimit, int xlimit) {
    const int wo = c * kKTileW + g * 16;
    const uint4 w = wo < wlimit ? *reinterpret_cast<const uint4*>(wbase + c * kKTileW)
                                : make_uint4(0, 0, 0, 0);
    const v4i w0 = widen16(w.x, w.y), w1 = widen16(w.z, w.w);
#pragma unroll
    for (int j = 0; j < MG; ++j) {
      const int xo = c * XCB + g * (XCB / 4);
      if constexpr (A_BITS == 4) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (xv[j] && xo < xlimit) x = *reinterpret_cast<const uint4*>(xp[j] + c * XCB);
        acc[j] = mfma(w0, widen16(x.x, x.y), acc[j]);
        acc[j] = mfma(w1, widen16(x.z, x.w), acc[j]);
      } else {
        uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
        if (xv[j] && xo < xlimit) {
          x0 = *reinterpret_cast<const uint4*>(xp[j] + c * XCB);
          x1 = *reinterpret_cast<const uint4*>(xp[j] + c * XCB + 16);
        }
        acc[j] = mfma(w0, split16(x0), acc[j]);
        acc[j] = mfma(w1, split16(x1), acc[j]);
      }
    }
  };

  v4i acc[MG];
#pragma unroll
  for (int j = 0; j < MG; ++j) acc[j] = v4i{0, 0, 0, 0};
  int c = wave;
  for (; c + 4 * (UNROLL - 1) < nchunks; c += 4 * UNROLL) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) chunk(c + 4 * u, acc, wp, Kb, Xrow);
  }
  for (; c < nchunks; c += 4) chunk(c, acc, wp, Kb, Xrow);

  // residual: r codes against Q(R), chunks of 128 codes spread over the waves
  v4i accr[MG];
#pragma unroll
  for (int j = 0; j < MG; ++j) accr[j] = v4i{0, 0, 0, 0};
  const int r = a.r;
  if (r > 0) {
    const int rb = r / 2;
    const uint8_t* rrow = a.Rq + static_cast<size_t>(min(n0 + l16, a.N - 1)) * rb;
    const int rchunks = (rb + kKTileW - 1) / kKTileW;
    const int xlim = r * A_BITS / 8;
    for (int cr = wave; cr < rchunks; cr += 4) {
      const int wo = cr * kKTileW + g * 16;
      uint4 w;
      w.x = load_dword_masked(rrow, wo, rb);
      w.y = load_dword_masked(rrow, wo + 4, rb);
      w.z = load_dword_masked(rrow, wo + 8, rb);
      w.w = load_dword_masked(rrow, wo + 12, rb);
      const v4i w0 = widen16(w.x, w.y), w1 = widen16(w.z, w.w);
#pragma unroll
      for (int j = 0; j < MG; ++j) {
        const uint8_t* xrow = xp[j] - g * (XCB / 4);
        const int xo = cr * XCB + g * (XCB / 4);
        if constexpr (A_BITS == 4) {
          uint4 x = make_uint4(0, 0, 0, 0);
          if (xv[j]) {
            x.x = load_dword_masked(xrow, xo, xlim);
            x.y = load_dword_masked(xrow, xo + 4, xlim);
            x.z = load_dword_masked(xrow, xo + 8, xlim);
            x.w = load_dword_masked(xrow, xo + 12, xlim);
          }
          accr[j] = mfma(w0, widen16(x.x, x.y), accr[j]);
          accr[j] = mfma(w1, widen16(x.z, x.w), accr[j]);
        } else {
          uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
          if (xv[j]) {
            x0.x = load_dword_masked(xrow, xo, xlim);
            x0.y = load_dword_masked(xrow, xo + 4, xlim);
            x0.z = load_dword_masked(xrow, xo + 8, xlim);
            x0.w = load_dword_masked(xrow, xo + 12, xlim);
            x1.x = load_dword_masked(xrow, xo + 16, xlim);
            x1.y = load_dword_masked(xrow, xo + 20, xlim);
            x1.z = load_dword_masked(xrow, xo + 24, xlim);
            x1.w = load_dword_masked(xrow, xo + 28, xlim);
          }
          accr[j] = mfma(w0, split16(x0), accr[j]);
          accr[j] = mfma(w1, split16(x1), accr[j]);
        }
      }
    }
  }

  // cross-wave reduction through LDS
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < MG; ++j) {
      red[0][wave - 1][j][lane] = acc[j];
      red[1][wave - 1][j][lane] = accr[j];
    }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kThreads / 64 - 1; ++w)
#pragma unroll
    for (int j = 0; j < MG; ++j) {
      acc[j] += red[0][w][j][lane];
      accr[j] += red[1][w][j][lane];
    }
#pragma unroll
  for (int j = 0; j < MG; ++j) store_block<SHIFT>(a, acc[j], accr[j], j * 16 + l16, n0 + 4 * g, r > 0);
}

// ---------------------------------------------------------------------------
// Generic kernel: one lane per output, any even K and r, any alignment. Used
// only for shapes the fast kernels do not cover (K % 32 != 0, r % 8 != 0,
// r > 256, unaligned buffers).
// ---------------------------------------------------------------------------

__device__ __forceinline__ int code_at(const uint8_t* row, int k, int bits) {
  if (bits == 8) return static_cast<int>(static_cast<int8_t>(row[k]));
  const int b = row[k >> 1];
  const int nib = (k & 1) ? (b >> 4) : (b & 15);
  return nib >= 8 ? nib - 16 : nib;
}

__global__ __launch_bounds__(kThreads) void serq_generic_kernel(LinearArgs a) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= static_cast<size_t>(a.M) * a.N) return;
  const int m = static_cast<int>(idx / a.N), n = static_cast<int>(idx % a.N);
  const uint8_t* xr = a.Xq + static_cast<size_t>(m) * (static_cast<size_t>(a.K) * a.a_bits / 8);
  const uint8_t* wr = a.Wq + static_cast<size_t>(n) * (a.K / 2);
  int am = 0;
  for (int k = 0; k < a.K; ++k) am += code_at(xr, k, a.a_bits) * code_at(wr, k, 4);
  int ar = 0;
  float srn = 0.0f;
  if (a.r > 0) {
    const uint8_t* rr = a.Rq + static_cast<size_t>(n) * (a.r / 2);
    for (int k = 0; k < a.r; ++k) ar += code_at(xr, k, a.a_bits) * code_at(rr, k, 4);
    srn = a.sr[n];
  }
  if (a.dbg_main) {
    a.dbg_main[idx] = am;
    a.dbg_res[idx] = ar;
  }
  const float y = a.sx[m] * __builtin_fmaf(srn, static_cast<float>(ar), a.sw[n] * static_cast<float>(am));
  if (a.y_bf16)
    static_cast<uint16_t*>(a.Y)[idx] = f32_to_bf16_rne(y);
  else
    static_cast<float*>(a.Y)[idx] = y;
}

template <int TN, int TM, int A_BITS>
hipError_t launch_tile(const LinearArgs& a, hipStream_t st) {
  using C = TileCfg<TN, TM, A_BITS>;
  const int rp = (a.r + 63) & ~63;
  const int lds = max(C::pipeline_bytes(), a.r > 0 ? C::residual_bytes(rp) : 0);
  static bool attr_set = false;  // idempotent; the attribute is per function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&serq_tile_kernel<TN, TM, A_BITS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       C::residual_bytes(kMaxResidual) > C::pipeline_bytes()
                                           ? C::residual_bytes(kMaxResidual)
                                           : C::pipeline_bytes());
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int n_tiles = (a.N + C::BN - 1) / C::BN;
  const int m_tiles = (a.M + C::BM - 1) / C::BM;
  serq_tile_kernel<TN, TM, A_BITS><<<dim3(n_tiles * m_tiles), dim3(kThreads), lds, st>>>(a, n_tiles);
  return hipGetLastError();
}

template <int A_BITS>
hipError_t launch_tile_bits(const LinearArgs& a, const LinearPlan& p, hipStream_t st) {
  if (p.tn == 8 && p.tm == 8) return launch_tile<8, 8, A_BITS>(a, st);
  if (p.tn == 8 && p.tm == 4) return launch_tile<8, 4, A_BITS>(a, st);
  if (p.tn == 4 && p.tm == 4) return launch_tile<4, 4, A_BITS>(a, st);
  if (p.tn == 4 && p.tm == 2) return launch_tile<4, 2, A_BITS>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace

LinearPlan plan_linear(int M, int K, int N, int r, int a_bits) {
  (void)a_bits;
  const bool fast = (K % 32 == 0) && (r % 8 == 0) && r <= kMaxResidual;
  if (!fast) return {LinearKernel::kGeneric, 0, 0, "generic"};
  if (M <= 16) return {LinearKernel::kDecode16, 0, 0, "decode16"};
  if (M <= 32) return {LinearKernel::kDecode32, 0, 0, "decode32"};
  // Macro tiles: prefer the largest tile that still gives every CU work.
  auto tiles = [&](int bm, int bn) {
    return static_cast<long>((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  };
  constexpr long kCUs = 256;
  if (M > 128 && tiles(256, 256) >= kCUs) return {LinearKernel::kTile, 8, 8, "tile256x256"};
  if (M > 64 && tiles(128, 256) >= kCUs) return {LinearKernel::kTile, 8, 4, "tile128x256"};
  if (M > 64) return {LinearKernel::kTile, 4, 4, "tile128x128"};
  return {LinearKernel::kTile, 4, 2, "tile64x128"};
}

hipError_t launch_linear(const LinearArgs& a, const LinearPlan& p, hipStream_t st) {
  switch (p.kind) {
    case LinearKernel::kDecode16: {
      const dim3 grid((a.N + 15) / 16);
      if (a.a_bits == 4)
        serq_decode_kernel<1, 4><<<grid, dim3(kThreads), 0, st>>>(a);
      else
        serq_decode_kernel<1, 8><<<grid, dim3(kThreads), 0, st>>>(a);
      return hipGetLastError();
    }
    case LinearKernel::kDecode32: {
      const dim3 grid((a.N + 15) / 16);
      if (a.a_bits == 4)
        serq_decode_kernel<2, 4><<<grid, dim3(kThreads), 0, st>>>(a);
      else
        serq_decode_kernel<2, 8><<<grid, dim3(kThreads), 0, st>>>(a);
      return hipGetLastError();
    }
    case LinearKernel::kTile:
      return a.a_bits == 4 ? launch_tile_bits<4>(a, p, st) : launch_tile_bits<8>(a, p, st);
    case LinearKernel::kGeneric: {
      const size_t total = static_cast<size_t>(a.M) * a.N;
      const dim3 grid(static_cast<unsigned>((total + kThreads - 1) / kThreads));
      serq_generic_kernel<<<grid, dim3(kThreads), 0, st>>>(a);
      return hipGetLastError();
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace serq

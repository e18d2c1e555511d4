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

// Epilogue for four consecutive output channels n..n+3 of token m, given
// the token scale and the four channel scales (no memory reads here).
template <int SHIFT>
__device__ __forceinline__ void store4(const LinearArgs& a, v4i am, v4i ar, int m, int n, float sxm,
                                       float4 w4, float4 r4) {
  if (m >= a.M) return;
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
  const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
  const float rv[4] = {r4.x, r4.y, r4.z, r4.w};
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float fm = static_cast<float>(am[i] >> SHIFT);
    const float fr = static_cast<float>(ar[i] >> SHIFT);
    y[i] = sxm * __builtin_fmaf(rv[i], fr, wv[i] * fm);
  }
  if (n + 3 < a.N && (a.N & 3) == 0) {
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
    if (a.y_bf16)
      static_cast<uint16_t*>(a.Y)[base + i] = f32_to_bf16_rne(y[i]);
    else
      static_cast<float*>(a.Y)[base + i] = y[i];
  }
}

// The scales of channels n..n+3 (zero past N), from global memory.
__device__ __forceinline__ float4 load_scales4(const float* p, int n, int N) {
  if (n + 3 < N && (N & 3) == 0) return *reinterpret_cast<const float4*>(p + n);
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = n + i < N ? p[n + i] : 0.0f;
  return make_float4(v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------------------
// Macro-tile kernel (prefill-sized M): a 256-lane workgroup computes a
// (64 TM tokens) x (64 TN channels) tile with 2 x 2 waves; each wave owns
// TN x TM blocks of 32 x 32 (v_mfma_i32_32x32x32_i8, A = weights, B = tokens).
//
// K loop: 128-code k-tiles streamed through STAGES LDS buffers with gfx950's
// direct global->LDS loads (global_load_lds_dwordx4: each lane moves 16
// bytes into its own slot of a 1 KB wave chunk, no registers involved), so
// k-tile t + STAGES - 1 is in flight while the MFMAs of k-tile t run. The
// loads are issued from inline assembly and waited for explicitly (s_waitcnt
// vmcnt + s_barrier, no fence): at the top of iteration t each wave waits
// until only its loads for later k-tiles are outstanding, then one barrier
// both publishes k-tile t and frees the buffer read in iteration t - 1, which
// the next load is issued into. (Left to itself the compiler would drain every
// outstanding load before each LDS read, serializing the pipeline.)
//
// LDS rows are 64 bytes (packed int4, 128 codes) or 128 bytes (int8). A
// 16-byte slot is placed at position part ^ f(row) -- (row >> 1) & 3 for 64-byte
// rows, row & 7 for 128-byte rows -- so the lanes that read the same part of
// consecutive rows hit distinct bank groups.
//
// Fragment k layout inside a k-tile: lane half h = lane / 32 of both operands
// holds codes [64 h, 64 h + 64); MFMA step s (0..3) takes its codes
// [64 h + 16 s, 64 h + 16 s + 16). The two halves together cover 32 codes per
// step and the four steps cover the 128 codes of the k-tile.
//
// After the K loop the LDS is reused for the residual: the r salient
// activation columns and Q(R) are widened once into LDS, and each block's
// residual MFMAs run right before its epilogue, so the residual needs only
// one 16-register accumulator at a time.
// ---------------------------------------------------------------------------

typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16i mfma32(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// One 16-byte direct global->LDS load per lane, from sbase + voff (sbase
// wave-uniform, voff a per-lane byte offset), into the wave's 1 KB chunk at
// `lds_chunk` (wave-uniform); lane i lands at lds_chunk + 16 i.
// M0 is written here and declared clobbered; the compiler sets M0 itself
// before every instruction of its own that reads it, so nothing relies on
// M0 surviving this statement.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_chunk) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_chunk) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with vmcnt <= n (n < 64) and no wait on lgkm/exp counters.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int TN, int TM, int A_BITS>
struct TileCfg {
  static constexpr int WN = 32 * TN, WM = 32 * TM;       // wave tile
  static constexpr int BN = 2 * WN, BM = 2 * WM;         // workgroup tile
  static constexpr int XB = kKTileCodes * A_BITS / 8;    // activation bytes / row / k-tile
  static constexpr int W_BYTES = BN * kKTileW;
  static constexpr int STAGE = W_BYTES + BM * XB;        // bytes per LDS stage
  static constexpr int W_CHUNKS = W_BYTES / 1024;        // 1 KB wave chunks per stage
  static constexpr int X_CHUNKS = BM * XB / 1024;
  static constexpr int CW = W_CHUNKS / 4;                // weight chunks per wave and stage
  static constexpr int CX = X_CHUNKS / 4;                // activation chunks per wave and stage
  static constexpr int CHUNKS_PER_WAVE = CW + CX;
  // Two workgroups share a CU: keep each under 80 KB of LDS.
  static constexpr int STAGES = (4 * STAGE <= 73728) ? 4 : (3 * STAGE <= 73728 ? 3 : 2);
  static constexpr int SHIFT = A_BITS == 4 ? 8 : 4;
  static constexpr int pipeline_bytes() { return STAGES * STAGE; }
  static constexpr int residual_bytes(int rp) { return (BN + BM) * (rp + 16) + 4 * (2 * BN + BM); }
  static_assert(W_CHUNKS % 4 == 0 && X_CHUNKS % 4 == 0, "stage must split over four waves");
  static_assert(STAGES * STAGE <= 80 * 1024, "LDS");
  static_assert(BN * 0 + (BN + BM) * (kMaxResidual + 16) + 4 * (2 * BN + BM) <= 80 * 1024, "LDS");
};

template <int TN, int TM, int A_BITS>
__global__ __launch_bounds__(kThreads, 2) void serq_tile_kernel(LinearArgs a, int n_tiles) {
  using C = TileCfg<TN, TM, A_BITS>;
  constexpr int STAGES = C::STAGES;
  constexpr int CPW = C::CHUNKS_PER_WAVE;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int tile_n = blockIdx.x % n_tiles, tile_m = blockIdx.x / n_tiles;
  const int n0 = tile_n * C::BN, m0 = tile_m * C::BM;
  const int Kb = a.K / 2;                      // packed weight bytes per row
  const int Xrow = a.K * A_BITS / 8;           // activation bytes per row
  const int nkt = (Kb + kKTileW - 1) / kKTileW;
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  // Wave w loads weight chunks [w CW, (w + 1) CW) and activation chunks
  // [w CX, (w + 1) CX) of every stage: 16 rows x 64 bytes per chunk (8 rows x
  // 128 bytes for int8 activations). Per lane: the byte offset of its row and
  // swizzled part at k-tile 0; the k-tile advances the (scalar) base pointer.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int part64 = (lane & 3) ^ ((lane >> 3) & 3);   // row (lane >> 2): (row >> 1) & 3
  const int part128 = (lane & 7) ^ ((lane >> 3) & 7);  // row (lane >> 3): row & 7
  uint32_t woff[C::CW], xoff[C::CX];
#pragma unroll
  for (int i = 0; i < C::CW; ++i) {
    const int row = (wv * C::CW + i) * 16 + (lane >> 2);
    woff[i] = static_cast<uint32_t>(min(n0 + row, a.N - 1)) * Kb + part64 * 16;
  }
#pragma unroll
  for (int i = 0; i < C::CX; ++i) {
    if constexpr (A_BITS == 4) {
      const int row = (wv * C::CX + i) * 16 + (lane >> 2);
      xoff[i] = static_cast<uint32_t>(min(m0 + row, a.M - 1)) * Xrow + part64 * 16;
    } else {
      const int row = (wv * C::CX + i) * 8 + (lane >> 3);
      xoff[i] = static_cast<uint32_t>(min(m0 + row, a.M - 1)) * Xrow + part128 * 16;
    }
  }
  // Issue the loads of k-tile kt into LDS stage `stage`. Only the last
  // k-tile can run past the end of K; its missing slots are zero-filled with
  // an ordinary LDS store instead.
  const bool k_exact = (Kb % kKTileW) == 0;
  auto issue = [&](int kt, int stage) {
    const uint32_t sbase = lds_base + stage * C::STAGE;
    const uint8_t* wsrc = a.Wq + static_cast<size_t>(kt) * kKTileW;
    const uint8_t* xsrc = a.Xq + static_cast<size_t>(kt) * C::XB;
    const bool full = k_exact || kt + 1 < nkt;
    const int wpos = kt * kKTileW + part64 * 16;                       // this lane's k byte
    const int xpos = kt * C::XB + (A_BITS == 4 ? part64 : part128) * 16;
#pragma unroll
    for (int i = 0; i < C::CW; ++i) {
      const uint32_t chunk = sbase + (wv * C::CW + i) * 1024;
      if (full || wpos < Kb)
        dma16(wsrc, woff[i], chunk);
      else
        *reinterpret_cast<uint4*>(lds + (chunk - lds_base) + lane * 16) = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::CX; ++i) {
      const uint32_t chunk = sbase + C::W_BYTES + (wv * C::CX + i) * 1024;
      if (full || xpos < Xrow)
        dma16(xsrc, xoff[i], chunk);
      else
        *reinterpret_cast<uint4*>(lds + (chunk - lds_base) + lane * 16) = make_uint4(0, 0, 0, 0);
    }
  };

  v16i acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v16i{};

  // fragment read offsets within a stage (the swizzle depends on l32 only)
  constexpr int XP = A_BITS == 4 ? 2 : 4;    // 16-byte parts per activation row and lane
  int wrd[2], xrd[XP];
#pragma unroll
  for (int p = 0; p < 2; ++p)
    wrd[p] = (wn * C::WN + l32) * kKTileW + (((2 * h + p) ^ ((l32 >> 1) & 3)) * 16);
#pragma unroll
  for (int p = 0; p < XP; ++p) {
    if constexpr (A_BITS == 4)
      xrd[p] = C::W_BYTES + (wm * C::WM + l32) * C::XB + (((2 * h + p) ^ ((l32 >> 1) & 3)) * 16);
    else
      xrd[p] = C::W_BYTES + (wm * C::WM + l32) * C::XB + (((4 * h + p) ^ (l32 & 7)) * 16);
  }

  // This lane's packed fragments of one k-tile: two 16-byte parts per weight
  // row, two (int4) or four (int8) per activation row.
  struct Frags {
    uint4 w[2][TN];
    uint4 x[XP][TM];
  };
  auto read_frags = [&](int stage, Frags& f) {
    const uint8_t* sb = lds + stage * C::STAGE;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int i = 0; i < TN; ++i) f.w[p][i] = *reinterpret_cast<const uint4*>(sb + wrd[p] + i * 32 * kKTileW);
#pragma unroll
    for (int p = 0; p < XP; ++p)
#pragma unroll
      for (int j = 0; j < TM; ++j) f.x[p][j] = *reinterpret_cast<const uint4*>(sb + xrd[p] + j * 32 * C::XB);
  };
  // MFMA step s takes dwords (2 (s & 1), 2 (s & 1) + 1) of weight part s >> 1.
  auto unpack = [&](const Frags& f, int s, v4i (&wa)[TN], v4i (&xb)[TM]) {
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const uint4 w = f.w[s >> 1][i];
      wa[i] = (s & 1) ? widen16(w.z, w.w) : widen16(w.x, w.y);
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      if constexpr (A_BITS == 4) {
        const uint4 x = f.x[s >> 1][j];
        xb[j] = (s & 1) ? widen16(x.z, x.w) : widen16(x.x, x.y);
      } else {
        xb[j] = split16(f.x[s][j]);
      }
    }
  };
  // The four MFMA steps of one k-tile, software-pipelined: the widening for
  // step s + 1 is issued between the MFMAs of step s, so the VALU work runs
  // while the matrix core is busy.
  auto compute = [&](const Frags& f) {
    v4i wa[TN], xb[TM];
    unpack(f, 0, wa, xb);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i wn2[TN], xn2[TM];
      if (s < 3) unpack(f, s + 1, wn2, xn2);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = mfma32(wa[i], xb[j], acc[i][j]);
      if (s < 3) {
        constexpr int kValuPerMfma = (6 * (TN + TM) + TN * TM - 1) / (TN * TM);
#pragma unroll
        for (int q = 0; q < TN * TM; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // then VALU
        }
#pragma unroll
        for (int i = 0; i < TN; ++i) wa[i] = wn2[i];
#pragma unroll
        for (int j = 0; j < TM; ++j) xb[j] = xn2[j];
      }
    }
  };
  // One k-tile: publish k-tile kt + 1 (own loads done, then a barrier), reuse
  // the buffer of k-tile kt -- its fragments are already in registers -- for
  // the loads of k-tile kt + STAGES, read k-tile kt + 1's fragments into
  // `next`, then run k-tile kt's MFMAs from `cur` while those reads land.
  auto step = [&](int kt, const Frags& cur, Frags& next) {
    if (kt + 1 < nkt) {
      const int ahead = min(STAGES - 2, nkt - 2 - kt);   // later k-tiles still in flight
      if (ahead >= 2) {
        wait_vmcnt<CPW * 2>();
      } else if (ahead == 1) {
        wait_vmcnt<CPW>();
      } else {
        wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): earlier fragment reads and zero-fills done
      __builtin_amdgcn_s_barrier();
      if (kt + STAGES < nkt) issue(kt + STAGES, kt % STAGES);
      read_frags((kt + 1) % STAGES, next);
    }
    compute(cur);
  };

#pragma unroll
  for (int st = 0; st < STAGES; ++st)
    if (st < nkt) issue(st, st);
  {
    const int inflight = min(STAGES, nkt);     // wait for k-tile 0 only
    if (inflight >= 4) {
      wait_vmcnt<CPW * 3>();
    } else if (inflight == 3) {
      wait_vmcnt<CPW * 2>();
    } else if (inflight == 2) {
      wait_vmcnt<CPW>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
  }
  Frags f0, f1;
  read_frags(0, f0);
  for (int kt = 0; kt < nkt; kt += 2) {
    step(kt, f0, f1);
    if (kt + 1 < nkt) step(kt + 1, f1, f0);
  }
  __syncthreads();                              // every wave is done with the pipeline buffers

  // ---- Epilogue operands, staged once into LDS (reusing the pipeline space)
  // with back-to-back wide loads: the widened residual operands -- Q(R) rows
  // and the r salient activation codes of the tile's tokens -- and the
  // token and channel scales. The per-block epilogue then reads only LDS.
  const int r = a.r;
  const bool has_res = r > 0;
  const int rp = (r + 31) & ~31;             // padded with zero codes to the MFMA depth
  const int RS = rp + 16;                    // LDS row stride of the widened operands
  uint8_t* Rw = lds;
  uint8_t* Rx = lds + C::BN * RS;
  float* s_sw = reinterpret_cast<float*>(lds + (C::BN + C::BM) * RS);
  float* s_sr = s_sw + C::BN;
  float* s_sx = s_sr + C::BN;
  if (tid < C::BN) {
    const int n = min(n0 + tid, a.N - 1);
    s_sw[tid] = a.sw[n];
    s_sr[tid] = has_res ? a.sr[n] : 0.0f;
  }
  if (tid < C::BM) s_sx[tid] = a.sx[min(m0 + tid, a.M - 1)];
  if (has_res) {
    const int rbytes = r / 2;
    const bool wide = (r % 32) == 0;         // packed rows 16-byte aligned
    for (int row = tid; row < C::BN + C::BM; row += kThreads) {
      const bool is_w = row < C::BN;
      const uint8_t* src = is_w ? a.Rq + static_cast<size_t>(min(n0 + row, a.N - 1)) * rbytes
                                : a.Xq + static_cast<size_t>(min(m0 + row - C::BN, a.M - 1)) * Xrow;
      uint8_t* dst = is_w ? Rw + row * RS : Rx + (row - C::BN) * RS;
#pragma unroll
      for (int q = 0; q < kMaxResidual / 32; ++q) {   // 32 codes per piece
        if (32 * q >= rp) break;
        uint4 lo, hi;                        // widened codes 32q .. 32q + 31
        if (A_BITS == 8 && !is_w) {
          uint4 d0, d1;
          if (wide && 32 * q + 32 <= r) {
            d0 = *reinterpret_cast<const uint4*>(src + 32 * q);
            d1 = *reinterpret_cast<const uint4*>(src + 32 * q + 16);
          } else {
            d0 = make_uint4(load_dword_masked(src, 32 * q, r), load_dword_masked(src, 32 * q + 4, r),
                            load_dword_masked(src, 32 * q + 8, r), load_dword_masked(src, 32 * q + 12, r));
            d1 = make_uint4(load_dword_masked(src, 32 * q + 16, r), load_dword_masked(src, 32 * q + 20, r),
                            load_dword_masked(src, 32 * q + 24, r), load_dword_masked(src, 32 * q + 28, r));
          }
          const uint2 e0 = split8(d0.x, d0.y), e1 = split8(d0.z, d0.w);
          const uint2 e2 = split8(d1.x, d1.y), e3 = split8(d1.z, d1.w);
          lo = make_uint4(e0.x, e0.y, e1.x, e1.y);
          hi = make_uint4(e2.x, e2.y, e3.x, e3.y);
        } else {
          uint4 p;
          if (wide && 16 * q + 16 <= rbytes) {
            p = *reinterpret_cast<const uint4*>(src + 16 * q);
          } else {
            p = make_uint4(load_dword_masked(src, 16 * q, rbytes), load_dword_masked(src, 16 * q + 4, rbytes),
                           load_dword_masked(src, 16 * q + 8, rbytes), load_dword_masked(src, 16 * q + 12, rbytes));
          }
          const uint2 e0 = widen8(p.x), e1 = widen8(p.y), e2 = widen8(p.z), e3 = widen8(p.w);
          lo = make_uint4(e0.x, e0.y, e1.x, e1.y);
          hi = make_uint4(e2.x, e2.y, e3.x, e3.y);
        }
        *reinterpret_cast<uint4*>(dst + 32 * q) = lo;
        *reinterpret_cast<uint4*>(dst + 32 * q + 16) = hi;
      }
    }
  }
  __syncthreads();
  const int nks = rp / 32;                   // 32-code MFMA steps; lane half h takes 16 of each

  // ---- per block: residual MFMAs, then the epilogue
  static_for<TM>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    v4i xr[kMaxResidual / 32];
#pragma unroll
    for (int s = 0; s < kMaxResidual / 32; ++s)
      xr[s] = s < nks ? *reinterpret_cast<const v4i*>(Rx + (wm * C::WM + j * 32 + l32) * RS + s * 32 + h * 16)
                      : v4i{0, 0, 0, 0};
    const int mt = wm * C::WM + j * 32 + l32;   // token within the tile
    const float sxm = s_sx[mt];
    static_for<TN>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      v16i ar = v16i{};
#pragma unroll
      for (int s = 0; s < kMaxResidual / 32; ++s)
        if (s < nks)
          ar = mfma32(*reinterpret_cast<const v4i*>(Rw + (wn * C::WN + i * 32 + l32) * RS + s * 32 + h * 16),
                      xr[s], ar);
      const int nt = wn * C::WN + i * 32 + 4 * h;   // channel within the tile
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 w4 = *reinterpret_cast<const float4*>(s_sw + nt + 8 * q);
        const float4 r4 = *reinterpret_cast<const float4*>(s_sr + nt + 8 * q);
        const v4i am4 = v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        const v4i ar4 = v4i{ar[4 * q], ar[4 * q + 1], ar[4 * q + 2], ar[4 * q + 3]};
        store4<C::SHIFT>(a, am4, ar4, m0 + mt, n0 + nt + 8 * q, sxm, w4, r4);
      }
    });
  });
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 32): the packed weights are streamed from HBM exactly
// once. A workgroup owns 16 output channels; its four waves take interleaved
// 256-code chunks of K (128 bytes of each of the 16 weight rows), with two
// register groups of chunks in flight per wave. Activations (a few KB) come
// through L2. One wave also takes the residual (r <= 256 codes: one chunk),
// then the partial int32 accumulators are summed through LDS and wave 0 runs
// the epilogue.
// ---------------------------------------------------------------------------

template <int MG, int A_BITS>
__global__ __launch_bounds__(kThreads) void serq_decode_kernel(LinearArgs a) {
  constexpr int SHIFT = A_BITS == 4 ? 8 : 4;
  constexpr int CC = 256;                             // codes per chunk
  constexpr int CWB = CC / 2;                         // weight bytes per row and chunk
  constexpr int CXB = CC * A_BITS / 8;                // activation bytes per row and chunk
  constexpr int LW = CWB / 4 / 16;                    // 16-byte weight loads per lane and chunk (2)
  constexpr int LX = CXB / 4 / 16;                    // 16-byte activation loads per lane and chunk
  constexpr int U = MG * LX <= 2 ? 2 : 1;             // chunks per register group
  static_assert(kMaxResidual <= CC, "the residual fits in one chunk");
  __shared__ v4i red[2][kThreads / 64 - 1][MG][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int Kb = a.K / 2, Xrow = a.K * A_BITS / 8;
  const int nrow = min(n0 + l16, a.N - 1);
  // Lane (row l16, group g) holds codes [CC c + 64 g, CC c + 64 g + 64) of
  // chunk c for both operands: 32 contiguous weight bytes, so the four lanes
  // of a row cover its whole 128-byte chunk.
  const uint8_t* wp = a.Wq + static_cast<size_t>(nrow) * Kb + g * (CWB / 4);
  const uint8_t* xp[MG];
  bool xv[MG];
#pragma unroll
  for (int j = 0; j < MG; ++j) {
    const int m = j * 16 + l16;
    xv[j] = m < a.M;
    xp[j] = a.Xq + static_cast<size_t>(min(m, a.M - 1)) * Xrow + g * (CXB / 4);
  }
  const int nchunks = (a.K + CC - 1) / CC;

  // Everything but the streamed weights is loaded up front so that its
  // latency overlaps the K loop: the epilogue scales and, in wave 1, the
  // (at most one chunk of) Q(R) and salient activation codes.
  float sxv[MG];
#pragma unroll
  for (int j = 0; j < MG; ++j) sxv[j] = a.sx[min(j * 16 + l16, a.M - 1)];
  const float4 sw4 = load_scales4(a.sw, n0 + 4 * g, a.N);
  const float4 sr4 = a.r > 0 ? load_scales4(a.sr, n0 + 4 * g, a.N) : make_float4(0.f, 0.f, 0.f, 0.f);
  const int r = a.r;
  const int rb = r / 2;                                 // packed residual bytes per row
  constexpr int kResWave = 1;
  uint4 rw[LW];
  uint4 rx[MG][LX];
#pragma unroll
  for (int l = 0; l < LW; ++l) rw[l] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < MG; ++j)
#pragma unroll
    for (int l = 0; l < LX; ++l) rx[j][l] = make_uint4(0, 0, 0, 0);
  if (r > 0 && wave == kResWave) {
    const uint8_t* rrow = a.Rq + static_cast<size_t>(nrow) * rb;
#pragma unroll
    for (int l = 0; l < LW; ++l) {
      const int wo = g * (CWB / 4) + 16 * l;
      rw[l] = make_uint4(load_dword_masked(rrow, wo, rb), load_dword_masked(rrow, wo + 4, rb),
                         load_dword_masked(rrow, wo + 8, rb), load_dword_masked(rrow, wo + 12, rb));
    }
    const int xlim = r * A_BITS / 8;
#pragma unroll
    for (int j = 0; j < MG; ++j) {
      if (!xv[j]) continue;
      const uint8_t* xrow = xp[j] - g * (CXB / 4);
#pragma unroll
      for (int l = 0; l < LX; ++l) {
        const int xo = g * (CXB / 4) + 16 * l;
        rx[j][l] = make_uint4(load_dword_masked(xrow, xo, xlim), load_dword_masked(xrow, xo + 4, xlim),
                              load_dword_masked(xrow, xo + 8, xlim), load_dword_masked(xrow, xo + 12, xlim));
      }
    }
  }

  // The K loop streams groups of U chunks per wave (chunk c = wave + 4 u);
  // the loads of the next group are issued into a second register buffer
  // before the current group is consumed.
  struct Group {
    uint4 w[U][LW];
    uint4 x[U][MG][LX];
  };
  auto load_group = [&](int c0, Group& gr) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 4 * u;
#pragma unroll
      for (int l = 0; l < LW; ++l) {
        const int o = c * CWB + g * (CWB / 4) + 16 * l;
        gr.w[u][l] = (c < nchunks && o < Kb) ? *reinterpret_cast<const uint4*>(wp + c * CWB + 16 * l)
                                             : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < MG; ++j)
#pragma unroll
        for (int l = 0; l < LX; ++l) {
          const int o = c * CXB + g * (CXB / 4) + 16 * l;
          gr.x[u][j][l] = (c < nchunks && xv[j] && o < Xrow)
                              ? *reinterpret_cast<const uint4*>(xp[j] + c * CXB + 16 * l)
                              : make_uint4(0, 0, 0, 0);
        }
    }
  };
  // One chunk: four MFMA steps of 16 codes per lane.
  auto dot_chunk = [&](const uint4 (&w)[LW], const uint4 (&x)[MG][LX], v4i (&acc)[MG]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 ww = w[s >> 1];
      const v4i wa = (s & 1) ? widen16(ww.z, ww.w) : widen16(ww.x, ww.y);
#pragma unroll
      for (int j = 0; j < MG; ++j) {
        v4i xb;
        if constexpr (A_BITS == 4) {
          const uint4 xx = x[j][s >> 1];
          xb = (s & 1) ? widen16(xx.z, xx.w) : widen16(xx.x, xx.y);
        } else {
          xb = split16(x[j][s]);
        }
        acc[j] = mfma(wa, xb, acc[j]);
      }
    }
  };

  v4i acc[MG];
#pragma unroll
  for (int j = 0; j < MG; ++j) acc[j] = v4i{0, 0, 0, 0};
  {
    Group g0, g1;
    int c0 = wave;
    load_group(c0, g0);
    for (; c0 < nchunks; c0 += 8 * U) {
      if (c0 + 4 * U < nchunks) load_group(c0 + 4 * U, g1);
#pragma unroll
      for (int u = 0; u < U; ++u) dot_chunk(g0.w[u], g0.x[u], acc);
      if (c0 + 4 * U >= nchunks) break;
      if (c0 + 8 * U < nchunks) load_group(c0 + 8 * U, g0);
#pragma unroll
      for (int u = 0; u < U; ++u) dot_chunk(g1.w[u], g1.x[u], acc);
    }
  }
  v4i accr[MG];
#pragma unroll
  for (int j = 0; j < MG; ++j) accr[j] = v4i{0, 0, 0, 0};
  if (r > 0 && wave == kResWave) dot_chunk(rw, rx, accr);

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
  for (int j = 0; j < MG; ++j) store4<SHIFT>(a, acc[j], accr[j], j * 16 + l16, n0 + 4 * g, sxv[j], sw4, sr4);
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
  const int rp = (a.r + 31) & ~31;
  const int lds = max(C::pipeline_bytes(), C::residual_bytes(rp));
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
  if (p.tn == 2 && p.tm == 2) return launch_tile<2, 2, A_BITS>(a, st);
  if (p.tn == 2 && p.tm == 1) return launch_tile<2, 1, A_BITS>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace

LinearPlan plan_linear(int M, int K, int N, int r, int a_bits) {
  // The fast kernels address rows with 32-bit byte offsets.
  const bool small = static_cast<uint64_t>(N) * (K / 2) < (1ull << 32) &&
                     static_cast<uint64_t>(M) * K * a_bits / 8 < (1ull << 32);
  const bool fast = (K % 32 == 0) && (r % 8 == 0) && r <= kMaxResidual && small;
  if (!fast) return {LinearKernel::kGeneric, 0, 0, "generic"};
  if (M <= 16) return {LinearKernel::kDecode16, 0, 0, "decode16"};
  if (M <= 32) return {LinearKernel::kDecode32, 0, 0, "decode32"};
  // Macro tiles of 128 x 128 (64 x 128 for up to 64 tokens), two
  // workgroups per CU.
  if (M > 64) return {LinearKernel::kTile, 2, 2, "tile128x128"};
  return {LinearKernel::kTile, 2, 1, "tile64x128"};
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

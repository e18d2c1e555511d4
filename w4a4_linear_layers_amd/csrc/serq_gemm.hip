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

// Two fp32 values -> two bf16 (round to nearest even) packed in a dword,
// `lo` in the low half: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f));
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
      const uint2 o = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
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
// The residual rides in the same pipeline: after the K/128 main k-tiles come
// ceil(r / 128) residual k-tiles (rows of Q(R) for the weights, the first
// codes of the same activation rows), loaded by the same instructions, so
// they are already in LDS when the K loop ends. The epilogue scales are
// loaded into LDS at kernel start, before the first k-tile. Every wave issues
// the same number of load instructions per k-tile, which is what the vmcnt
// thresholds count.
//
// LDS rows are 64 bytes (packed int4, 128 codes) or 128 bytes (int8); each
// 16-byte part is stored at a row-dependent XOR-swizzled slot (swz64,
// swz128) so that the lanes that read the same part of consecutive rows hit
// distinct bank groups.
//
// Fragment k layout inside a k-tile: lane half h = lane / 32 of both operands
// holds codes [64 h, 64 h + 64); MFMA step s (0..3) takes its codes
// [64 h + 16 s, 64 h + 16 s + 16). The two halves together cover 32 codes per
// step and the four steps cover the 128 codes of the k-tile.
//
// Epilogue: each block's residual MFMAs run from the residual k-tiles, the
// scales turn the two accumulators into fp32 outputs in place, the output
// tile is written to LDS (swizzled, conflict-free) and then copied to Y with
// 16-byte stores along its rows.
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

// LDS slot swizzles. A 16-byte part of a 64-byte row goes to slot
// part ^ swz64(row); of a 128-byte row to part ^ swz128(row). Chosen so that
// the 16-byte reads of 16 consecutive rows at one part hit distinct bank
// groups whether the LDS serves 8 or 16 lanes of a ds_read_b128 per cycle.
__device__ __forceinline__ int swz64(int row) {
  return (((row >> 1) ^ (row >> 2)) & 1) | ((((row >> 2) ^ (row >> 3)) & 1) << 1);
}
__device__ __forceinline__ int swz128(int row) {
  return ((row >> 1) & 3) | ((((row >> 3) ^ row) & 1) << 2);
}

// Workgroup -> tile order. Workgroups are dispatched round-robin over the
// eight XCDs (each with its own L2), so workgroup b runs on XCD b % 8. The
// grid is first regrouped so that each XCD gets a contiguous range of the
// tile order, and the tile order walks groups of kGroupM tile rows with the
// tile column fastest inside a group: the tiles resident on one XCD then
// share a few weight column blocks and activation row blocks.
constexpr int kXcds = 8;
constexpr int kGroupM = 8;
__device__ __forceinline__ void tile_coords(int b, int nb, int n_tiles, int& tn, int& tm) {
  int l = b;
  if (nb % kXcds == 0) l = (b % kXcds) * (nb / kXcds) + b / kXcds;
  const int m_tiles = nb / n_tiles;
  const int per_group = kGroupM * n_tiles;
  const int grp = l / per_group;
  const int first_m = grp * kGroupM;
  const int gm = min(kGroupM, m_tiles - first_m);      // rows in this (possibly last) group
  const int in = l - grp * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}


// One 4-byte direct global->LDS load per lane: lane i moves the dword at
// sbase + voff into lds_dst + 4 i (same conventions as dma16).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_dst) : "memory", "m0");
}
#pragma clang diagnostic pop

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
  static constexpr int SCALE_BYTES = 4 * (2 * BN + BM);  // sw, sr, sx of the tile
  // Two workgroups share a CU: keep each within 80 KB of LDS.
  static constexpr int kLdsCap = 80 * 1024;
  static constexpr int STAGES = (4 * STAGE + SCALE_BYTES <= kLdsCap) ? 4 : (3 * STAGE + SCALE_BYTES <= kLdsCap ? 3 : 2);
  static constexpr int SCALE_OFF = STAGES * STAGE;
  static constexpr int OUT_BYTES = BM * BN * 4;          // fp32 output tile (bf16 takes half)
  static constexpr int LDS_BYTES = SCALE_OFF + SCALE_BYTES > OUT_BYTES ? SCALE_OFF + SCALE_BYTES : OUT_BYTES;
  static constexpr int SHIFT = A_BITS == 4 ? 8 : 4;
  static_assert(W_CHUNKS % 4 == 0 && X_CHUNKS % 4 == 0, "stage must split over four waves");
  static_assert(BN % 64 == 0 && BM % 64 == 0, "scale rows are loaded 64 at a time");
  // The residual k-tiles (at most two) stay in their buffers while the last
  // main k-tile is computed from another one.
  static_assert(STAGES >= (kMaxResidual / 2 + kKTileW - 1) / kKTileW + 1, "residual k-tiles need free stages");
  static_assert(LDS_BYTES <= kLdsCap, "LDS");
};

// Output-tile swizzle for bf16 rows (16 chunks of 16 bytes): the 8-byte half
// a lane writes moves to the other half of its chunk when half_swap(row).
// With chunk ^ (row & 15) this keeps the eight-byte writes of 16 (and of 32)
// consecutive rows at one column on distinct banks.
__device__ __forceinline__ int half_swap(int row) { return ((row >> 3) ^ (row >> 4)) & 1; }

template <int TN, int TM, int A_BITS>
__global__ __launch_bounds__(kThreads, 2) void serq_tile_kernel(LinearArgs a, int n_tiles) {
  using C = TileCfg<TN, TM, A_BITS>;
  constexpr int STAGES = C::STAGES;
  constexpr int CPW = C::CHUNKS_PER_WAVE;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  int tile_n, tile_m;
  tile_coords(blockIdx.x, gridDim.x, n_tiles, tile_n, tile_m);
  const int n0 = __builtin_amdgcn_readfirstlane(tile_n * C::BN);
  const int m0 = __builtin_amdgcn_readfirstlane(tile_m * C::BM);
  const int Kb = a.K / 2;                      // packed weight bytes per row
  const int Xrow = a.K * A_BITS / 8;           // activation bytes per row
  const int Rb = rq_row_bytes(a.r);            // Q(R) bytes per row (zero-padded)
  const int nkt = (Kb + kKTileW - 1) / kKTileW;  // main k-tiles
  const int ntot = nkt + (Rb + kKTileW - 1) / kKTileW;   // plus residual k-tiles
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // Epilogue scales into LDS first, so that every wave's k-tile waits below
  // also cover them: wave 0 loads sw, wave 1 sr, wave 2 sx of the tile.
  {
    const uint32_t sbase = lds_base + C::SCALE_OFF;
    if (wv == 0) {
#pragma unroll
      for (int c = 0; c < C::BN / 64; ++c)
        if (n0 + 64 * c + lane < a.N) dma4(a.sw + n0 + 64 * c, 4 * lane, sbase + 256 * c);
    } else if (wv == 1) {
      if (a.r > 0) {
#pragma unroll
        for (int c = 0; c < C::BN / 64; ++c)
          if (n0 + 64 * c + lane < a.N) dma4(a.sr + n0 + 64 * c, 4 * lane, sbase + 4 * C::BN + 256 * c);
      } else {                                  // no residual: sr = 0
#pragma unroll
        for (int c = 0; c < C::BN / 64; ++c)
          reinterpret_cast<float*>(lds + C::SCALE_OFF + 4 * C::BN)[64 * c + lane] = 0.0f;
      }
    } else if (wv == 2) {
#pragma unroll
      for (int c = 0; c < C::BM / 64; ++c)
        if (m0 + 64 * c + lane < a.M) dma4(a.sx + m0 + 64 * c, 4 * lane, sbase + 8 * C::BN + 256 * c);
    }
  }

  // Wave w loads weight chunks [w CW, (w + 1) CW) and activation chunks
  // [w CX, (w + 1) CX) of every stage: 16 rows x 64 bytes per chunk (8 rows x
  // 128 bytes for int8 activations). Per lane: the byte offset of its row and
  // swizzled part at k-tile 0; the k-tile advances the (scalar) base pointer.
  const int part64 = (lane & 3) ^ swz64(lane >> 2);    // 16-row chunks: row & 15 = lane >> 2
  uint32_t woff[C::CW], roff[C::CW], xoff[C::CX];
  int xpart[C::CX];                                     // this lane's 16-byte part of each activation chunk
#pragma unroll
  for (int i = 0; i < C::CW; ++i) {
    const int row = min(n0 + (wv * C::CW + i) * 16 + (lane >> 2), a.N - 1);
    woff[i] = static_cast<uint32_t>(row) * Kb + part64 * 16;
    roff[i] = static_cast<uint32_t>(row) * Rb + part64 * 16;
  }
#pragma unroll
  for (int i = 0; i < C::CX; ++i) {
    if constexpr (A_BITS == 4) {
      const int row = (wv * C::CX + i) * 16 + (lane >> 2);
      xpart[i] = part64;
      xoff[i] = static_cast<uint32_t>(min(m0 + row, a.M - 1)) * Xrow + part64 * 16;
    } else {
      const int row = (wv * C::CX + i) * 8 + (lane >> 3);
      xpart[i] = (lane & 7) ^ swz128(row);
      xoff[i] = static_cast<uint32_t>(min(m0 + row, a.M - 1)) * Xrow + xpart[i] * 16;
    }
  }
  // Issue the loads of k-tile kt (main k-tiles, then residual ones) into LDS
  // stage `stage`. A k-tile that runs past the end of its rows (the last
  // main one when K % 128 != 0, the last residual one) zero-fills its missing
  // 16-byte slots with an ordinary LDS store instead; every instruction still
  // has at least one loading lane, so the per-wave load count is the same
  // for every k-tile.
  auto issue = [&](int kt, int stage) {
    const uint32_t sbase = lds_base + stage * C::STAGE;
    const bool res = kt >= nkt;
    const int kx = res ? kt - nkt : kt;        // k-tile index within its source rows
    const uint8_t* wsrc = (res ? a.Rq : a.Wq) + kx * kKTileW;
    const uint8_t* xsrc = a.Xq + kx * C::XB;
    const int wleft = (res ? Rb : Kb) - kx * kKTileW;     // row bytes left from the k-tile start
    const int xleft = Xrow - kx * C::XB;
#pragma unroll
    for (int i = 0; i < C::CW; ++i) {
      const uint32_t chunk = sbase + (wv * C::CW + i) * 1024;
      const uint32_t off = res ? roff[i] : woff[i];
      if (wleft >= kKTileW || part64 * 16 < wleft)
        dma16(wsrc, off, chunk);
      else
        *reinterpret_cast<uint4*>(lds + (chunk - lds_base) + lane * 16) = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::CX; ++i) {
      const uint32_t chunk = sbase + C::W_BYTES + (wv * C::CX + i) * 1024;
      if (xleft >= C::XB || xpart[i] * 16 < xleft)
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
    wrd[p] = (wn * C::WN + l32) * kKTileW + (((2 * h + p) ^ swz64(l32)) * 16);
#pragma unroll
  for (int p = 0; p < XP; ++p) {
    if constexpr (A_BITS == 4)
      xrd[p] = C::W_BYTES + (wm * C::WM + l32) * C::XB + (((2 * h + p) ^ swz64(l32)) * 16);
    else
      xrd[p] = C::W_BYTES + (wm * C::WM + l32) * C::XB + (((4 * h + p) ^ swz128(l32)) * 16);
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
  // Widened MFMA operands of step s from a weight / activation fragment.
  auto wop = [&](const uint4& w0, const uint4& w1, int s) {
    const uint4 w = (s >> 1) ? w1 : w0;
    return (s & 1) ? widen16(w.z, w.w) : widen16(w.x, w.y);
  };
  auto xop = [&](const uint4 (&x)[XP], int s) {
    if constexpr (A_BITS == 4) {
      const uint4 v = x[s >> 1];
      return (s & 1) ? widen16(v.z, v.w) : widen16(v.x, v.y);
    } else {
      return split16(x[s]);
    }
  };
  // MFMA step s takes dwords (2 (s & 1), 2 (s & 1) + 1) of weight part s >> 1.
  auto unpack = [&](const Frags& f, int s, v4i (&wa)[TN], v4i (&xb)[TM]) {
#pragma unroll
    for (int i = 0; i < TN; ++i) wa[i] = wop(f.w[0][i], f.w[1][i], s);
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      uint4 xj[XP];
#pragma unroll
      for (int p = 0; p < XP; ++p) xj[p] = f.x[p][j];
      xb[j] = xop(xj, s);
    }
  };
  // The four MFMA steps of one k-tile, software-pipelined: the widening for
  // step s + 1 is issued between the MFMAs of step s, so the VALU work runs
  // while the matrix core is busy.
  auto compute = [&](const Frags& f, v16i (&acc)[TN][TM]) {
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
      const int ahead = min(STAGES - 2, ntot - 2 - kt);   // later k-tiles still in flight
      if (ahead >= 2) {
        wait_vmcnt<CPW * 2>();
      } else if (ahead == 1) {
        wait_vmcnt<CPW>();
      } else {
        wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): earlier fragment reads and zero-fills done
      __builtin_amdgcn_s_barrier();
      if (kt + STAGES < ntot) issue(kt + STAGES, kt % STAGES);
      read_frags((kt + 1) % STAGES, next);
    }
    compute(cur, acc);
  };

#pragma unroll
  for (int st = 0; st < STAGES; ++st)
    if (st < ntot) issue(st, st);
  {
    const int inflight = min(STAGES, ntot);    // wait for k-tile 0 (and the scales) only
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

  // ---- Epilogue. The residual k-tiles were issued during the last main
  // iterations; wait for them, then publish them (and the zero-fills).
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  const float* s_sw = reinterpret_cast<const float*>(lds + C::SCALE_OFF);
  const float* s_sr = s_sw + C::BN;
  const float* s_sx = s_sr + C::BN;
  const int nres = ntot - nkt;
  // Residual MFMAs for all blocks, from the residual k-tiles.
  v16i ar[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) ar[i][j] = v16i{};
  for (int t = 0; t < nres; ++t) {
    Frags fr;
    read_frags((nkt + t) % STAGES, fr);
    compute(fr, ar);
  }
  if (a.dbg_main) {                            // exact accumulators, for tests
    static_for<TM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int m = m0 + wm * C::WM + j * 32 + l32;
      static_for<TN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int nb = n0 + wn * C::WN + i * 32 + 4 * h;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int n = nb + 8 * (e >> 2) + (e & 3);
          if (m < a.M && n < a.N) {
            a.dbg_main[static_cast<size_t>(m) * a.N + n] = acc[i][j][e] >> C::SHIFT;
            a.dbg_res[static_cast<size_t>(m) * a.N + n] = ar[i][j][e] >> C::SHIFT;
          }
        }
      });
    });
  }
  // y = sx (sw acc_main + sr acc_res) in fp32, kept in place of the main
  // accumulator. The scales of a channel block are read once for its TM
  // token blocks.
  float sxm[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) sxm[j] = s_sx[wm * C::WM + j * 32 + l32];
  static_for<TN>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int nt = wn * C::WN + i * 32 + 4 * h;   // first channel (within the tile) of group q = 0
    float4 w4[4], r4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w4[q] = *reinterpret_cast<const float4*>(s_sw + nt + 8 * q);
      r4[q] = *reinterpret_cast<const float4*>(s_sr + nt + 8 * q);
    }
    static_for<TM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float wv4[4] = {w4[q].x, w4[q].y, w4[q].z, w4[q].w};
        const float rv4[4] = {r4[q].x, r4[q].y, r4[q].z, r4[q].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float fm = static_cast<float>(acc[i][j][4 * q + c] >> C::SHIFT);
          const float fr = static_cast<float>(ar[i][j][4 * q + c] >> C::SHIFT);
          acc[i][j][4 * q + c] = __float_as_int(sxm[j] * __builtin_fmaf(rv4[c], fr, wv4[c] * fm));
        }
      }
    });
  });
  __syncthreads();                              // residual buffers and scales no longer read

  // Output tile into LDS, row = token, swizzled 16-byte chunks.
  if (a.y_bf16) {
    constexpr int RB = C::BN * 2;
    static_for<TM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int row = wm * C::WM + j * 32 + l32;
      uint8_t* rp = lds + row * RB;
      const int hs = (h ^ half_swap(row)) * 8;
      static_for<TN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = (wn * C::WN + i * 32) / 8 + q;
          const uint2 o = make_uint2(
              pack_bf16x2(__int_as_float(acc[i][j][4 * q]), __int_as_float(acc[i][j][4 * q + 1])),
              pack_bf16x2(__int_as_float(acc[i][j][4 * q + 2]), __int_as_float(acc[i][j][4 * q + 3])));
          *reinterpret_cast<uint2*>(rp + 16 * (c ^ (row & 15)) + hs) = o;
        }
      });
    });
  } else {
    constexpr int RB = C::BN * 4;
    static_for<TM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int row = wm * C::WM + j * 32 + l32;
      uint8_t* rp = lds + row * RB;
      static_for<TN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = (wn * C::WN + i * 32 + 8 * q + 4 * h) / 4;
          *reinterpret_cast<v4i*>(rp + 16 * (c ^ (row & 15))) =
              v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        }
      });
    });
  }
  __syncthreads();

  // Copy-out: 16-byte chunks along the rows of Y (every LDS read first, then
  // the stores); ragged tails element by element.
  auto copy_out = [&](auto ebc) {
    constexpr int EB = decltype(ebc)::value;  // bytes per element
    constexpr int CPR = C::BN * EB / 16;      // chunks per tile row
    constexpr int EPC = 16 / EB;              // elements per chunk
    constexpr int RPP = kThreads / CPR;       // rows per pass
    constexpr int PASSES = C::BM / RPP;
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
      uint4 w = v[p];
      if (EB == 2 && half_swap(row)) w = make_uint4(w.z, w.w, w.x, w.y);
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
  else
    copy_out(std::integral_constant<int, 4>{});
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
  const int rb = rq_row_bytes(r);                       // Q(R) row stride (zero-padded)
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
    const uint8_t* rr = a.Rq + static_cast<size_t>(n) * rq_row_bytes(a.r);
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
  static bool attr_set = false;  // idempotent; the attribute is per function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&serq_tile_kernel<TN, TM, A_BITS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int n_tiles = (a.N + C::BN - 1) / C::BN;
  const int m_tiles = (a.M + C::BM - 1) / C::BM;
  serq_tile_kernel<TN, TM, A_BITS><<<dim3(n_tiles * m_tiles), dim3(kThreads), C::LDS_BYTES, st>>>(a, n_tiles);
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

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
// activations are byte-shuffled into the same order). The scaled sum stays
// below 2^31 for K < 2^17 (|true sum| <= 64 K for W4A4, 1024 K for W4A8);
// longer rows take the generic kernel.
//
// MFMA operand roles: A = weight rows (16 output channels), B = activation
// rows (16 tokens), so D[n][m]; lane l of a 16x16 block holds tokens
// m = l % 16 and four consecutive channels n = 4 (l / 16) + i, which the
// epilogue writes as one 16- or 8-byte vector per lane.
//
// Fragment k layout: within a 128-code k-tile, lane group g = l / 16 of both
// operands holds codes [32 g, 32 g + 32) (16 packed bytes); MFMA step 0 uses
// its first 16 codes and step 1 the next 16.

#include <atomic>
#include <utility>

#include "serq_internal.h"

typedef int v4i __attribute__((ext_vector_type(4)));

namespace serq {
namespace {

constexpr int kThreads = 256;
constexpr int kCUs = 256;                   // compute units of an MI355X
constexpr int kKTileCodes = 128;            // codes per k-tile
constexpr int kKTileW = kKTileCodes / 2;    // packed weight bytes per row per k-tile
constexpr int kMaxResidual = 256;           // largest r handled by the tile kernels
constexpr int kWidenMaxK = 1 << 17;         // K bound of the kernels that sum widened codes

// Lambdas that touch a kernel's register arrays must be inlined: a call
// would pass the arrays by address and put them in scratch memory.
#define SERQ_INLINE __attribute__((always_inline))

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

// Workgroup barrier for LDS data only: this wave's LDS accesses complete,
// then s_barrier. Unlike __syncthreads it does not wait for outstanding
// global loads, so prefetches stay in flight. The wait is the builtin, so the
// compiler knows every earlier LDS read has landed; the memory clobber on the
// barrier keeps it from moving LDS accesses across.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0), no vmcnt / expcnt wait
  asm volatile("s_barrier" ::: "memory");
}

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

// Tile shape: each wave owns TN x TM blocks of 32 x 32; a k-group is a
// 2 (channels) x WGM (tokens) grid of waves, and the workgroup holds KG
// k-groups, group g taking k-tile g of every KG-k-tile stage (their sums are
// added through LDS at the end). OCC workgroups share a CU: two waves per
// SIMD in every shape.
template <int TN, int TM, int A_BITS, int WGM, int KG>
struct TileCfg {
  static constexpr int NWG = 2 * WGM;                    // waves per k-group
  static constexpr int NW = NWG * KG;                    // waves per workgroup
  static constexpr int NT = 64 * NW;                     // lanes per workgroup
  static constexpr int OCC = 8 / NW;                     // workgroups per CU
  static constexpr int WN = 32 * TN, WM = 32 * TM;       // wave tile
  static constexpr int BN = 2 * WN, BM = WGM * WM;       // workgroup tile
  static constexpr int XB = kKTileCodes * A_BITS / 8;    // activation bytes / row / k-tile
  static constexpr int W_BYTES = BN * kKTileW;
  static constexpr int SUB = W_BYTES + BM * XB;          // one k-tile of the tile in LDS
  static constexpr int STAGE = KG * SUB;                 // bytes per LDS stage (KG k-tiles)
  static constexpr int W_CHUNKS = W_BYTES / 1024;        // 1 KB wave chunks per k-tile
  static constexpr int X_CHUNKS = BM * XB / 1024;
  static constexpr int CW = KG * W_CHUNKS / NW;          // weight chunks per wave and stage
  static constexpr int CX = KG * X_CHUNKS / NW;          // activation chunks per wave and stage
  static constexpr int CHUNKS_PER_WAVE = CW + CX;
  static constexpr int SCALE_BYTES = 4 * (2 * BN + BM);  // sw, sr, sx of the tile
  static constexpr int TRASH_BYTES = KG > 1 ? 1024 : 0;  // sink of the loads that only keep counts even
  static constexpr int kLdsCap = 160 * 1024 / OCC;       // the CU's LDS split between its workgroups
  static constexpr int kMaxStages = 8;
  static constexpr int stages() {
    int st = kMaxStages;
    while (st > 2 && st * STAGE + SCALE_BYTES + TRASH_BYTES > kLdsCap) --st;
    return st;
  }
  static constexpr int STAGES = stages();
  static constexpr int SCALE_OFF = STAGES * STAGE;
  static constexpr int TRASH_OFF = SCALE_OFF + SCALE_BYTES;
  static constexpr int OUT_BYTES = BM * BN * 4;          // fp32 output tile (bf16 takes half)
  static constexpr int RED_BYTES = (KG - 1) * NWG * 64 * TN * TM * 2 * 64;   // other groups' sums
  static constexpr int lds_bytes() {
    int b = TRASH_OFF + TRASH_BYTES;
    if (OUT_BYTES > b) b = OUT_BYTES;
    if (RED_BYTES > b) b = RED_BYTES;
    return b;
  }
  static constexpr int LDS_BYTES = lds_bytes();
  static constexpr int SHIFT = A_BITS == 4 ? 8 : 4;
  // Output-tile chunk swizzle mask for rows of `eb`-byte elements: XOR with
  // the row's low bits, within the row's 16-byte chunks.
  static constexpr int out_swz(int eb) { return BN * eb / 16 >= 16 ? 15 : BN * eb / 16 - 1; }
  static_assert((KG * W_CHUNKS) % NW == 0 && (KG * X_CHUNKS) % NW == 0, "stage must split over the waves");
  static_assert(RED_BYTES <= SCALE_OFF, "group sums fit in the stages");
  static_assert(BN % 64 == 0 && (BM % 64 == 0 || BM == 32), "scale rows are loaded 64 at a time");
  static_assert(CHUNKS_PER_WAVE * (STAGES - 1) < 64, "vmcnt range");
  // The residual k-tiles (at most two) stay in their buffers while the last
  // main k-tile is computed from another one.
  static_assert(STAGES >= ((kMaxResidual / 2 + kKTileW - 1) / kKTileW + KG - 1) / KG + 1,
                "residual k-tiles need free stages");
  static_assert(LDS_BYTES <= kLdsCap, "LDS");
};

// Output-tile swizzle for bf16 rows (16 chunks of 16 bytes): the 8-byte half
// a lane writes moves to the other half of its chunk when half_swap(row).
// With chunk ^ (row & 15) this keeps the eight-byte writes of 16 (and of 32)
// consecutive rows at one column on distinct banks.
__device__ __forceinline__ int half_swap(int row) { return ((row >> 3) ^ (row >> 4)) & 1; }

template <int TN, int TM, int A_BITS, int WGM, int KG>
__global__ __launch_bounds__(128 * WGM * KG, 2)   // NT lanes; two waves per SIMD (OCC workgroups per CU)
void serq_tile_kernel(LinearArgs a, int n_tiles) {
  using C = TileCfg<TN, TM, A_BITS, WGM, KG>;
  static_assert(C::NT == 128 * WGM * KG && C::OCC * C::NW == 8, "launch bounds");
  constexpr int STAGES = C::STAGES;
  constexpr int CPW = C::CHUNKS_PER_WAVE;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = wave / C::NWG, wl = wave % C::NWG;     // k-group, and wave within it
  const int wn = wl / WGM, wm = wl % WGM;
  const int l32 = lane & 31, h = lane >> 5;
  int tile_n, tile_m;
  tile_coords(blockIdx.x, gridDim.x, n_tiles, tile_n, tile_m);
  const int n0 = __builtin_amdgcn_readfirstlane(tile_n * C::BN);
  const int m0 = __builtin_amdgcn_readfirstlane(tile_m * C::BM);
  const int Kb = a.K / 2;                      // packed weight bytes per row
  const int Xrow = a.K * A_BITS / 8;           // activation bytes per row
  const int Rb = rq_row_bytes(a.r);            // Q(R) bytes per row (zero-padded)
  // Stages of KG k-tiles: main ones, then the residual ones.
  const int nkt = ((Kb + kKTileW - 1) / kKTileW + KG - 1) / KG;
  const int ntot = nkt + ((Rb + kKTileW - 1) / kKTileW + KG - 1) / KG;
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // The operand bases, held in registers: selecting between fields of the
  // argument block inside the loop would reload them from memory (a scalar
  // load, whose out-of-order return forces lgkmcnt(0) waits that also drain
  // the fragment reads in flight).
  const uint8_t* const Wq = a.Wq;
  const uint8_t* const Rq = a.Rq;
  const uint8_t* const Xq = a.Xq;

  // Epilogue scales into LDS first, so that every wave's k-tile waits below
  // also cover them: wave 0 loads sw, wave 1 sr, wave 2 (wave 0 in a
  // two-wave workgroup) sx of the tile.
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
    }
    if (wv == (C::NW > 2 ? 2 : 0)) {
#pragma unroll
      for (int c = 0; c < (C::BM + 63) / 64; ++c)
        if (64 * c + lane < C::BM && m0 + 64 * c + lane < a.M)
          dma4(a.sx + m0 + 64 * c, 4 * lane, sbase + 8 * C::BN + 256 * c);
    }
  }

  // Wave w loads weight chunks [w CW, (w + 1) CW) and activation chunks
  // [w CX, (w + 1) CX) of every stage: 16 rows x 64 bytes per chunk (8 rows x
  // 128 bytes for int8 activations) of one of the stage's KG k-tiles. Per
  // lane: the byte offset of its row and swizzled part at stage 0, and the
  // chunk's place in the stage; the stage advances the (scalar) base pointer.
  const int part64 = (lane & 3) ^ swz64(lane >> 2);    // 16-row chunks: row & 15 = lane >> 2
  uint32_t woff[C::CW], roff[C::CW], xoff[C::CX], wdst[C::CW], xdst[C::CX];
  int xpart[C::CX];                                     // this lane's 16-byte part of each activation chunk
  int wsub[C::CW], xsub[C::CX], wrow[C::CW], xrow[C::CX];   // k-tile within the stage, source row
#pragma unroll
  for (int i = 0; i < C::CW; ++i) {
    const int c = wv * C::CW + i, sub = c / C::W_CHUNKS, cc = c % C::W_CHUNKS;
    const int row = min(n0 + cc * 16 + (lane >> 2), a.N - 1);
    wsub[i] = sub;
    wrow[i] = row;
    wdst[i] = sub * C::SUB + cc * 1024;
    woff[i] = static_cast<uint32_t>(row) * Kb + part64 * 16 + sub * kKTileW;
    roff[i] = static_cast<uint32_t>(row) * Rb + part64 * 16 + sub * kKTileW;
  }
#pragma unroll
  for (int i = 0; i < C::CX; ++i) {
    const int c = wv * C::CX + i, sub = c / C::X_CHUNKS, cc = c % C::X_CHUNKS;
    xsub[i] = sub;
    xdst[i] = sub * C::SUB + C::W_BYTES + cc * 1024;
    if constexpr (A_BITS == 4) {
      const int row = cc * 16 + (lane >> 2);
      xpart[i] = part64;
      xrow[i] = min(m0 + row, a.M - 1);
    } else {
      const int row = cc * 8 + (lane >> 3);
      xpart[i] = (lane & 7) ^ swz128(row);
      xrow[i] = min(m0 + row, a.M - 1);
    }
    xoff[i] = static_cast<uint32_t>(xrow[i]) * Xrow + xpart[i] * 16 + sub * C::XB;
  }
  // Issue the loads of stage kt (main stages, then residual ones) into LDS
  // stage `stage`. A k-tile that runs past the end of its rows (the last
  // main one when K % 128 != 0, the last residual one) zero-fills its missing
  // 16-byte slots with an ordinary LDS store instead. Every load instruction
  // keeps at least one loading lane, and a chunk wholly past the end (a
  // stage's trailing k-tiles) still issues one load, of valid bytes into a
  // scratch kilobyte of LDS, so the per-wave load count is the same for every
  // stage.
  auto issue = [&](int kt, int stage) {
    const uint32_t sbase = lds_base + stage * C::STAGE;
    const bool res = kt >= nkt;
    const int kx = res ? kt - nkt : kt;        // stage index within its source rows
    const uint8_t* wsrc = (res ? Rq : Wq) + kx * KG * kKTileW;
    const uint8_t* xsrc = Xq + kx * KG * C::XB;
    const int wleft = (res ? Rb : Kb) - kx * KG * kKTileW;     // row bytes left from the stage start
    const int xleft = Xrow - kx * KG * C::XB;
    // Full main stages take a path with no per-lane masks.
    if (!res && wleft >= KG * kKTileW && xleft >= KG * C::XB) {
#pragma unroll
      for (int i = 0; i < C::CW; ++i) dma16(wsrc, woff[i], sbase + wdst[i]);
#pragma unroll
      for (int i = 0; i < C::CX; ++i) dma16(xsrc, xoff[i], sbase + xdst[i]);
      return;
    }
#pragma unroll
    for (int i = 0; i < C::CW; ++i) {
      const uint32_t chunk = sbase + wdst[i];
      const uint32_t off = res ? roff[i] : woff[i];
      const int wl = wleft - wsub[i] * kKTileW;             // bytes of this k-tile's rows left
      if (wl > 0 && (wl >= kKTileW || part64 * 16 < wl)) {
        dma16(wsrc, off, chunk);
      } else {
        if (KG > 1 && wl <= 0)
          dma16(res ? Rq : Wq, static_cast<uint32_t>(wrow[i]) * (res ? Rb : Kb), lds_base + C::TRASH_OFF);
        *reinterpret_cast<uint4*>(lds + (chunk - lds_base) + lane * 16) = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < C::CX; ++i) {
      const uint32_t chunk = sbase + xdst[i];
      const int xl = xleft - xsub[i] * C::XB;
      if (xl > 0 && (xl >= C::XB || xpart[i] * 16 < xl)) {
        dma16(xsrc, xoff[i], chunk);
      } else {
        if (KG > 1 && xl <= 0) dma16(Xq, static_cast<uint32_t>(xrow[i]) * Xrow, lds_base + C::TRASH_OFF);
        *reinterpret_cast<uint4*>(lds + (chunk - lds_base) + lane * 16) = make_uint4(0, 0, 0, 0);
      }
    }
  };

  // With fewer than four blocks per wave, consecutive MFMA steps go to AS
  // separate accumulator sets (added up after the loop), so that no MFMA
  // waits for the previous one's result.
  constexpr int AS = TN * TM >= 4 ? 1 : 4 / (TN * TM);
  v16i accs[AS][TN][TM];
#pragma unroll
  for (int k = 0; k < AS; ++k)
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) accs[k][i][j] = v16i{};

  // fragment read offsets within a stage (the swizzle depends on l32 only)
  constexpr int XP = A_BITS == 4 ? 2 : 4;    // 16-byte parts per activation row and lane
  int wrd[2], xrd[XP];
#pragma unroll
  for (int p = 0; p < 2; ++p)
    wrd[p] = kg * C::SUB + (wn * C::WN + l32) * kKTileW + (((2 * h + p) ^ swz64(l32)) * 16);
#pragma unroll
  for (int p = 0; p < XP; ++p) {
    if constexpr (A_BITS == 4)
      xrd[p] = kg * C::SUB + C::W_BYTES + (wm * C::WM + l32) * C::XB + (((2 * h + p) ^ swz64(l32)) * 16);
    else
      xrd[p] = kg * C::SUB + C::W_BYTES + (wm * C::WM + l32) * C::XB + (((4 * h + p) ^ swz128(l32)) * 16);
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
  // while the matrix core is busy. The wave raises its issue priority for the
  // k-tile's MFMA sequence, so that of the two waves on a SIMD the one feeding
  // the matrix core goes first: 2-3 % on the one-k-group prefill tiles, 3-7 %
  // on the 64x64 four-k-group tile, up to 6 % on the 64x64 two-k-group tile
  // when two of its workgroups share a CU; on the 32x64 four-k-group tile and
  // the two-k-group 128x128 tile it cost 1-2 %, so those leave it alone.
  static constexpr bool kRaisePrio = KG == 1 || (KG == 4 && TM == 2) || (KG == 2 && WGM == 1);
  auto compute = [&](const Frags& f, v16i (&acc)[AS][TN][TM]) {
    v4i wa[TN], xb[TM];
    unpack(f, 0, wa, xb);
    if constexpr (kRaisePrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i wn2[TN], xn2[TM];
      if (s < 3) unpack(f, s + 1, wn2, xn2);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[s % AS][i][j] = mfma32(wa[i], xb[j], acc[s % AS][i][j]);
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
    if constexpr (kRaisePrio) __builtin_amdgcn_s_setprio(0);
  };
  // One k-tile: publish k-tile kt + 1 (own loads done, then a barrier), reuse
  // the buffer of k-tile kt -- its fragments are already in registers -- for
  // the loads of k-tile kt + STAGES, read k-tile kt + 1's fragments into
  // `next`, then run k-tile kt's MFMAs from `cur` while those reads land.
  // Wait until at most `n` k-tiles of this wave's loads are outstanding
  // (n < STAGES, wave-uniform): vmcnt counts instructions, CPW per k-tile.
  auto wait_tiles = [&](int n) {
    if (n >= STAGES - 2) {                       // the steady state, tested first
      wait_vmcnt<CPW * (STAGES - 2)>();
      return;
    }
    static_for<STAGES>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if (n == k) wait_vmcnt<CPW * k>();
    });
  };
  // k-tile kt lives in stage st = kt % STAGES (a constant at every call).
  auto step = [&](int kt, int st, const Frags& cur, Frags& next) {
    // cur's fragment reads and the last zero-fills have landed (on every
    // path, so the compiler does not wait again after the next reads).
    __builtin_amdgcn_s_waitcnt(0xC07F);
    if (kt + 1 < nkt) {
      wait_tiles(min(STAGES - 2, ntot - 2 - kt));   // later k-tiles may stay in flight
      asm volatile("s_barrier" ::: "memory");
      if (kt + STAGES < ntot) issue(kt + STAGES, st);
      read_frags((st + 1) % STAGES, next);
    }
    compute(cur, accs);
  };

#pragma unroll
  for (int st = 0; st < STAGES; ++st)
    if (st < ntot) issue(st, st);
  wait_tiles(min(STAGES, ntot) - 1);           // k-tile 0 (and the scales) landed
  lds_barrier();
  // Steady state: k-tile kt + 1 is the oldest load still awaited, STAGES - 2
  // more are in flight, and k-tile kt + STAGES is a full main k-tile -- no
  // test at all.
  auto fast_step = [&](int kt, int st, const Frags& cur, Frags& next) {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    wait_vmcnt<CPW * (STAGES - 2)>();
    asm volatile("s_barrier" ::: "memory");
    const uint32_t sbase = lds_base + st * C::STAGE;
    const uint8_t* wsrc = Wq + (kt + STAGES) * KG * kKTileW;
    const uint8_t* xsrc = Xq + (kt + STAGES) * KG * C::XB;
#pragma unroll
    for (int i = 0; i < C::CW; ++i) dma16(wsrc, woff[i], sbase + wdst[i]);
#pragma unroll
    for (int i = 0; i < C::CX; ++i) dma16(xsrc, xoff[i], sbase + xdst[i]);
    read_frags((st + 1) % STAGES, next);
    compute(cur, accs);
  };

  // The loop is unrolled over a whole period of (stage, fragment buffer)
  // pairs so that every LDS offset is a constant.
  Frags f0, f1;
  read_frags(0, f0);
  constexpr int UNR = STAGES % 2 ? 2 * STAGES : STAGES;
  const int nfull = min(Kb / kKTileW, Xrow / C::XB) / KG;   // main stages with no ragged end
  int kt0 = 0;
  for (; kt0 + UNR <= nfull - STAGES; kt0 += UNR) {
    static_for<UNR>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i % 2 == 0)
        fast_step(kt0 + i, i % STAGES, f0, f1);
      else
        fast_step(kt0 + i, i % STAGES, f1, f0);
    });
  }
  for (; kt0 < nkt; kt0 += UNR) {
    static_for<UNR>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (kt0 + i < nkt) {
        if constexpr (i % 2 == 0)
          step(kt0 + i, i % STAGES, f0, f1);
        else
          step(kt0 + i, i % STAGES, f1, f0);
      }
    });
  }

  // ---- Epilogue. The residual k-tiles were issued during the last main
  // iterations; wait for them, then publish them (and the zero-fills).
  wait_vmcnt<0>();
  lds_barrier();
  const float* s_sw = reinterpret_cast<const float*>(lds + C::SCALE_OFF);
  const float* s_sr = s_sw + C::BN;
  const float* s_sx = s_sr + C::BN;
  const int nres = ntot - nkt;
  // Residual MFMAs for all blocks, from the residual k-tiles.
  v16i ars[AS][TN][TM];
#pragma unroll
  for (int k = 0; k < AS; ++k)
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) ars[k][i][j] = v16i{};
  for (int t = 0; t < nres; ++t) {
    Frags fr;
    read_frags((nkt + t) % STAGES, fr);
    compute(fr, ars);
  }
  v16i (&acc)[TN][TM] = accs[0];
  v16i (&ar)[TN][TM] = ars[0];
#pragma unroll
  for (int k = 1; k < AS; ++k)
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        acc[i][j] += accs[k][i][j];
        ar[i][j] += ars[k][i][j];
      }
  // Which k-group finishes block (i, j): with two k-groups and an even
  // number of blocks per wave, each group takes every other block (the
  // epilogue's scaling and LDS writes split between them); otherwise group 0
  // takes them all.
  constexpr bool kSplitEpi = KG == 2 && (TN * TM) % 2 == 0;
  auto owns = [&](int i, int j) { return kSplitEpi ? ((i * TM + j) & 1) == kg : kg == 0; };
  if constexpr (kSplitEpi) {
    // Each wave leaves the sums of the blocks the other group finishes in LDS
    // (the stages are free once every wave is here; lane-contiguous words, no
    // bank conflicts) and adds the other group's sums of its own blocks.
    constexpr int NH = TN * TM / 2, PL = NH * 16;
    lds_barrier();
    int* red = reinterpret_cast<int*>(lds);
    int* dst = red + (kg * C::NWG + wl) * 2 * PL * 64 + lane;
    const int* src = red + ((1 - kg) * C::NWG + wl) * 2 * PL * 64 + lane;
    static_for<TN * TM>([&](auto bc) {
      constexpr int b = decltype(bc)::value, i = b / TM, j = b % TM, t = b / 2;
      if ((b & 1) != kg) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          dst[(t * 16 + e) * 64] = acc[i][j][e];
          dst[(PL + t * 16 + e) * 64] = ar[i][j][e];
        }
      }
    });
    lds_barrier();
    static_for<TN * TM>([&](auto bc) {
      constexpr int b = decltype(bc)::value, i = b / TM, j = b % TM, t = b / 2;
      if ((b & 1) == kg) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          acc[i][j][e] += src[(t * 16 + e) * 64];
          ar[i][j][e] += src[(PL + t * 16 + e) * 64];
        }
      }
    });
  } else if constexpr (KG > 1) {
    // The other k-groups' sums through LDS (the stages are free once every
    // wave is here; lane-contiguous words, no bank conflicts), added up by
    // group 0, which runs the epilogue.
    constexpr int PL = TN * TM * 16;
    lds_barrier();
    int* red = reinterpret_cast<int*>(lds);
    if (kg > 0) {
      int* dst = red + ((kg - 1) * C::NWG + wl) * 2 * PL * 64 + lane;
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            dst[((i * TM + j) * 16 + e) * 64] = acc[i][j][e];
            dst[(PL + (i * TM + j) * 16 + e) * 64] = ar[i][j][e];
          }
    }
    lds_barrier();
    if (kg == 0) {
      for (int g = 1; g < KG; ++g) {
        const int* src = red + ((g - 1) * C::NWG + wl) * 2 * PL * 64 + lane;
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              acc[i][j][e] += src[((i * TM + j) * 16 + e) * 64];
              ar[i][j][e] += src[(PL + (i * TM + j) * 16 + e) * 64];
            }
      }
    }
  }
  if (a.dbg_main) {                            // exact accumulators, for tests
    static_for<TM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int m = m0 + wm * C::WM + j * 32 + l32;
      static_for<TN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if (!owns(i, j)) return;
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
  // The accumulators hold 2^SHIFT times the code dot products; the factor is
  // taken out of the token scale instead of shifting every accumulator. A
  // power-of-two factor commutes with fp32 rounding, so the result is the
  // same as converting the shifted integers.
  float sxm[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) sxm[j] = s_sx[wm * C::WM + j * 32 + l32] * (1.0f / (1 << C::SHIFT));
  if (kSplitEpi || kg == 0) static_for<TN>([&](auto ic) {
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
      if (!owns(i, j)) return;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float wv4[4] = {w4[q].x, w4[q].y, w4[q].z, w4[q].w};
        const float rv4[4] = {r4[q].x, r4[q].y, r4[q].z, r4[q].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float fm = static_cast<float>(acc[i][j][4 * q + c]);
          const float fr = static_cast<float>(ar[i][j][4 * q + c]);
          acc[i][j][4 * q + c] = __float_as_int(sxm[j] * __builtin_fmaf(rv4[c], fr, wv4[c] * fm));
        }
      }
    });
  });
  __syncthreads();                              // residual buffers and scales no longer read

  // Output tile into LDS, row = token, swizzled 16-byte chunks.
  if (!kSplitEpi && kg > 0) {
    // the other k-groups only help with the copy-out
  } else if (a.y_bf16) {
    constexpr int RB = C::BN * 2, SWZ = C::out_swz(2);
    static_for<TM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int row = wm * C::WM + j * 32 + l32;
      uint8_t* rp = lds + row * RB;
      const int hs = (h ^ half_swap(row)) * 8;
      static_for<TN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if (!owns(i, j)) return;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = (wn * C::WN + i * 32) / 8 + q;
          const uint2 o = make_uint2(
              pack_bf16x2(__int_as_float(acc[i][j][4 * q]), __int_as_float(acc[i][j][4 * q + 1])),
              pack_bf16x2(__int_as_float(acc[i][j][4 * q + 2]), __int_as_float(acc[i][j][4 * q + 3])));
          *reinterpret_cast<uint2*>(rp + 16 * (c ^ (row & SWZ)) + hs) = o;
        }
      });
    });
  } else {
    constexpr int RB = C::BN * 4, SWZ = C::out_swz(4);
    static_for<TM>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int row = wm * C::WM + j * 32 + l32;
      uint8_t* rp = lds + row * RB;
      static_for<TN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if (!owns(i, j)) return;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = (wn * C::WN + i * 32 + 8 * q + 4 * h) / 4;
          *reinterpret_cast<v4i*>(rp + 16 * (c ^ (row & SWZ))) =
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
    constexpr int RPP = C::NT / CPR;          // rows per pass
    constexpr int PASSES = (C::BM + RPP - 1) / RPP;
    const int c = tid % CPR;
    const int n = n0 + c * EPC;
    const bool vec = (a.N % EPC) == 0 && n + EPC <= a.N;
    uint4 v[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = min(p * RPP + tid / CPR, C::BM - 1);
      v[p] = *reinterpret_cast<const uint4*>(lds + row * C::BN * EB + 16 * (c ^ (row & C::out_swz(EB))));
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = p * RPP + tid / CPR;
      if (row >= C::BM || m0 + row >= a.M) break;
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
// 256 x 256 tile kernel (W4A4 prefill on layers with a tile for every CU):
// one four-wave workgroup per CU, so each wave is its SIMD's only wave and
// has the SIMD's whole register file: its 4 x 4 blocks of 32 x 32 (128
// channels x 128 tokens) keep their 256 int32 sums in the accumulation
// registers and the fragments and widened operands in the vector registers.
//
// With 2 x 2 blocks per wave, each MFMA step widens four operands for four
// MFMAs (six VALU per MFMA), and the two waves of a SIMD together issue
// nearly as many VALU cycles as the matrix core runs, so the widening sets
// the pace. With 4 x 4 blocks a step widens eight operands for sixteen
// MFMAs (three per MFMA), issued by the wave between its own MFMAs. The
// tile also halves the L2 -> LDS bytes per output.
//
// The k pipeline is the macro-tile kernel's: 128-code k-tiles through four
// 32 KB LDS stages by direct global->LDS loads (eight 1 KB chunks per wave
// and k-tile), vmcnt-counted waits, one barrier per k-tile, and the residual
// k-tiles last in the same stream. The residual has no accumulators of its
// own (they would need 256 more registers): the epilogue runs, per channel
// block, the residual MFMAs of its four token blocks from the residual
// k-tiles still in LDS, combines them with the main sums and stores the
// block's outputs from registers.
// ---------------------------------------------------------------------------

struct Tile256Cfg {
  static constexpr int TN = 4, TM = 4;                   // 32 x 32 blocks per wave
  static constexpr int NW = 4, NT = 64 * NW;
  static constexpr int BN = 256, BM = 256;
  static constexpr int XB = kKTileCodes / 2;             // int4 activation bytes per row and k-tile
  static constexpr int W_BYTES = BN * kKTileW;
  static constexpr int STAGE = W_BYTES + BM * XB;        // 32 KB
  static constexpr int CW = W_BYTES / 1024 / NW;         // weight chunks per wave and k-tile
  static constexpr int CX = BM * XB / 1024 / NW;         // activation chunks per wave and k-tile
  static constexpr int CPW = CW + CX;
  static constexpr int STAGES = 4;
  static constexpr int SCALE_OFF = STAGES * STAGE;
  static constexpr int SCALE_BYTES = 4 * (2 * BN + BM);
  static constexpr int LDS_BYTES = SCALE_OFF + SCALE_BYTES;
  static constexpr int SHIFT = 8;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(CPW * (STAGES - 1) < 64, "vmcnt range");
  static_assert(STAGES >= (kMaxResidual / 2 + kKTileW - 1) / kKTileW + 1, "residual k-tiles need free stages");
};

// Store target of the lanes of a partial tile whose outputs fall outside Y
// (written, never read): 16 bytes per lane.
__device__ __align__(16) uint8_t tile_store_sink[64 * 16];

__global__ __launch_bounds__(256, 1) void serq_tile256_kernel(LinearArgs a, int n_tiles) {
  using C = Tile256Cfg;
  constexpr int STAGES = C::STAGES, CPW = C::CPW, TN = C::TN, TM = C::TM;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  int tile_n, tile_m;
  tile_coords(blockIdx.x, gridDim.x, n_tiles, tile_n, tile_m);
  const int n0 = __builtin_amdgcn_readfirstlane(tile_n * C::BN);
  const int m0 = __builtin_amdgcn_readfirstlane(tile_m * C::BM);
  const int Kb = a.K / 2;                      // packed bytes per weight and activation row
  const int Rb = rq_row_bytes(a.r);
  const int nkt = (Kb + kKTileW - 1) / kKTileW;
  const int ntot = nkt + (Rb + kKTileW - 1) / kKTileW;
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint8_t* const Wq = a.Wq;
  const uint8_t* const Rq = a.Rq;
  const uint8_t* const Xq = a.Xq;

  // Epilogue scales first (older than every k-tile load, so the first
  // k-tile wait covers them): wave 0 sw, wave 1 sr, wave 2 sx.
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
  // [w CX, (w + 1) CX) of every k-tile: 16 rows x 64 bytes each, the lane's
  // 16-byte part at its swizzled slot (rows past the end clamped to the last).
  const int part64 = (lane & 3) ^ swz64(lane >> 2);
  uint32_t woff[C::CW], roff[C::CW], xoff[C::CX];
#pragma unroll
  for (int i = 0; i < C::CW; ++i) {
    const int row = min(n0 + (wv * C::CW + i) * 16 + (lane >> 2), a.N - 1);
    woff[i] = static_cast<uint32_t>(row) * Kb + part64 * 16;
    roff[i] = static_cast<uint32_t>(row) * Rb + part64 * 16;
  }
#pragma unroll
  for (int i = 0; i < C::CX; ++i) {
    const int row = min(m0 + (wv * C::CX + i) * 16 + (lane >> 2), a.M - 1);
    xoff[i] = static_cast<uint32_t>(row) * Kb + part64 * 16;
  }
  auto wdst = [&](int i) { return static_cast<uint32_t>((wv * C::CW + i) * 1024); };
  auto xdst = [&](int i) { return static_cast<uint32_t>(C::W_BYTES + (wv * C::CX + i) * 1024); };
  // k-tile kt (main ones, then residual ones) into stage `stage`; a k-tile
  // running past the end of its rows zero-fills its missing 16-byte slots
  // with LDS stores (every load instruction keeps a loading lane: part 0 of
  // a row is always in range).
  auto issue = [&](int kt, int stage) SERQ_INLINE {
    const uint32_t sbase = lds_base + stage * C::STAGE;
    const bool res = kt >= nkt;
    const int kx = res ? kt - nkt : kt;
    const uint8_t* wsrc = (res ? Rq : Wq) + kx * kKTileW;
    const uint8_t* xsrc = Xq + kx * C::XB;
    const int wleft = (res ? Rb : Kb) - kx * kKTileW;
    const int xleft = Kb - kx * C::XB;
    if (!res && wleft >= kKTileW) {
#pragma unroll
      for (int i = 0; i < C::CW; ++i) dma16(wsrc, woff[i], sbase + wdst(i));
#pragma unroll
      for (int i = 0; i < C::CX; ++i) dma16(xsrc, xoff[i], sbase + xdst(i));
      return;
    }
#pragma unroll
    for (int i = 0; i < C::CW; ++i) {
      if (wleft >= kKTileW || part64 * 16 < wleft)
        dma16(wsrc, res ? roff[i] : woff[i], sbase + wdst(i));
      else
        *reinterpret_cast<uint4*>(lds + stage * C::STAGE + wdst(i) + lane * 16) = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::CX; ++i) {
      if (xleft >= C::XB || part64 * 16 < xleft)
        dma16(xsrc, xoff[i], sbase + xdst(i));
      else
        *reinterpret_cast<uint4*>(lds + stage * C::STAGE + xdst(i) + lane * 16) = make_uint4(0, 0, 0, 0);
    }
  };

  v16i acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v16i{};

  int wrd[2], xrd[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    wrd[p] = (wn * 32 * TN + l32) * kKTileW + (((2 * h + p) ^ swz64(l32)) * 16);
    xrd[p] = C::W_BYTES + (wm * 32 * TM + l32) * C::XB + (((2 * h + p) ^ swz64(l32)) * 16);
  }
  struct Frags {
    uint4 w[2][TN];
    uint4 x[2][TM];
  };
  // Part p (16 bytes per row and lane) of every block's fragments of the
  // k-tile in `stage`.
  auto read_part = [&](int stage, int p, Frags& f) SERQ_INLINE {
    const uint8_t* sb = lds + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < TN; ++i) f.w[p][i] = *reinterpret_cast<const uint4*>(sb + wrd[p] + i * 32 * kKTileW);
#pragma unroll
    for (int j = 0; j < TM; ++j) f.x[p][j] = *reinterpret_cast<const uint4*>(sb + xrd[p] + j * 32 * C::XB);
  };
  // MFMA step s takes dwords (2 (s & 1), 2 (s & 1) + 1) of part s >> 1.
  auto op = [&](const uint4& v0, const uint4& v1, int s) SERQ_INLINE {
    const uint4 v = (s >> 1) ? v1 : v0;
    return (s & 1) ? widen16(v.z, v.w) : widen16(v.x, v.y);
  };
  auto unpack = [&](const Frags& f, int s, v4i (&wa)[TN], v4i (&xb)[TM]) SERQ_INLINE {
#pragma unroll
    for (int i = 0; i < TN; ++i) wa[i] = op(f.w[0][i], f.w[1][i], s);
#pragma unroll
    for (int j = 0; j < TM; ++j) xb[j] = op(f.x[0][j], f.x[1][j], s);
  };
  // The four MFMA steps of the k-tile whose step-0 operands are in wa, xb
  // and whose fragments are in `f`; step s + 1's widening is issued between
  // step s's MFMAs. One fragment buffer: once steps 0 and 1 are widened,
  // part 0 of the next k-tile (stage `next`) is read into its place, and
  // part 1 once steps 2 and 3 are; step 3's MFMAs cover the widening of the
  // next k-tile's step 0, so the matrix core has operands right after the
  // next barrier.
  v4i wa[TN], xb[TM];
  auto compute = [&](Frags& f, int next, bool read_next) SERQ_INLINE {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i wn2[TN], xn2[TM];
      const bool widen = s < 3 || read_next;
      if (widen) unpack(f, (s + 1) & 3, wn2, xn2);
      if (s == 0 || s == 2)
        if (read_next) read_part(next, s >> 1, f);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = mfma32(wa[i], xb[j], acc[i][j]);
      if (widen) {
        constexpr int kValuPerMfma = (6 * (TN + TM) + TN * TM - 1) / (TN * TM);
#pragma unroll
        for (int q = 0; q < TN * TM; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
          if (q == 0 && (s == 0 || s == 2)) __builtin_amdgcn_sched_group_barrier(0x100, TN + TM, 0);
        }
#pragma unroll
        for (int i = 0; i < TN; ++i) wa[i] = wn2[i];
#pragma unroll
        for (int j = 0; j < TM; ++j) xb[j] = xn2[j];
      }
      // nothing moves across steps: hoisting later steps' widening would
      // need more registers than the wave has
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto wait_tiles = [&](int n) SERQ_INLINE {
    if (n >= STAGES - 2) {
      wait_vmcnt<CPW * (STAGES - 2)>();
      return;
    }
    static_for<STAGES>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if (n == k) wait_vmcnt<CPW * k>();
    });
  };
  // One k-tile, as in the macro-tile kernel: publish kt + 1 (own loads
  // done, then a barrier), refill kt's buffer (its fragments are in
  // registers) with kt + STAGES, then run kt's MFMAs while kt + 1's
  // fragments are read.
  auto step = [&](int kt, int st, Frags& f) SERQ_INLINE {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    const bool more = kt + 1 < nkt;
    if (more) {
      wait_tiles(min(STAGES - 2, ntot - 2 - kt));
      asm volatile("s_barrier" ::: "memory");
      if (kt + STAGES < ntot) issue(kt + STAGES, st);
    }
    compute(f, (st + 1) % STAGES, more);
  };
  auto fast_step = [&](int kt, int st, Frags& f) SERQ_INLINE {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    wait_vmcnt<CPW * (STAGES - 2)>();
    asm volatile("s_barrier" ::: "memory");
    const uint32_t sbase = lds_base + st * C::STAGE;
    const uint8_t* wsrc = Wq + (kt + STAGES) * kKTileW;
    const uint8_t* xsrc = Xq + (kt + STAGES) * C::XB;
#pragma unroll
    for (int i = 0; i < C::CW; ++i) dma16(wsrc, woff[i], sbase + wdst(i));
#pragma unroll
    for (int i = 0; i < C::CX; ++i) dma16(xsrc, xoff[i], sbase + xdst(i));
    compute(f, (st + 1) % STAGES, true);
  };

#pragma unroll
  for (int st = 0; st < STAGES; ++st)
    if (st < ntot) issue(st, st);
  wait_tiles(min(STAGES, ntot) - 1);
  lds_barrier();
  Frags f;
  read_part(0, 0, f);
  read_part(0, 1, f);
  unpack(f, 0, wa, xb);
  const int nfull = Kb / kKTileW;              // main k-tiles with no ragged end
  int kt0 = 0;
  for (; kt0 + STAGES <= nfull - STAGES; kt0 += STAGES)
    static_for<STAGES>([&](auto ic) { fast_step(kt0 + decltype(ic)::value, decltype(ic)::value, f); });
  for (; kt0 < nkt; kt0 += STAGES) {
    static_for<STAGES>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (kt0 + i < nkt) step(kt0 + i, i, f);
    });
  }

  // ---- Epilogue: the residual k-tiles (issued during the last main
  // iterations) and zero-fills published, then channel block by channel
  // block: t = sw acc_main in fp32, the block's accumulators reused for its
  // residual MFMAs, y = sx (sr acc_res + t), stores.
  wait_vmcnt<0>();
  lds_barrier();
  const float* s_sw = reinterpret_cast<const float*>(lds + C::SCALE_OFF);
  const float* s_sr = s_sw + C::BN;
  const float* s_sx = s_sr + C::BN;
  const int nres = ntot - nkt;
  // The sums are 2^SHIFT times the code dot products; the factor comes out
  // of the token scale (a power of two commutes with fp32 rounding).
  float sxm[TM];
  int mrow[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    mrow[j] = m0 + wm * 32 * TM + j * 32 + l32;
    sxm[j] = s_sx[wm * 32 * TM + j * 32 + l32] * (1.0f / (1 << C::SHIFT));
  }
  // Channel block i: t = sw acc_main (fp32), then the block's accumulators
  // are reused for its residual sums (four independent MFMA chains, one per
  // token block).
  auto residual = [&](auto ic, float (&t)[TM][16], const float4 (&w4)[4]) SERQ_INLINE {
    constexpr int i = decltype(ic)::value;
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float wv4[4] = {w4[q].x, w4[q].y, w4[q].z, w4[q].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) t[j][4 * q + c] = wv4[c] * static_cast<float>(acc[i][j][4 * q + c]);
      }
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v16i{};
    for (int u = 0; u < nres; ++u) {
      const uint8_t* sb = lds + ((nkt + u) % STAGES) * C::STAGE;
      const uint4 w0 = *reinterpret_cast<const uint4*>(sb + wrd[0] + i * 32 * kKTileW);
      const uint4 w1 = *reinterpret_cast<const uint4*>(sb + wrd[1] + i * 32 * kKTileW);
      uint4 x0[TM], x1[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        x0[j] = *reinterpret_cast<const uint4*>(sb + xrd[0] + j * 32 * C::XB);
        x1[j] = *reinterpret_cast<const uint4*>(sb + xrd[1] + j * 32 * C::XB);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const v4i wa = op(w0, w1, s);
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = mfma32(wa, op(x0[j], x1[j], s), acc[i][j]);
      }
    }
  };
  auto load_scales = [&](int nt, float4 (&w4)[4], float4 (&r4)[4]) SERQ_INLINE {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w4[q] = *reinterpret_cast<const float4*>(s_sw + nt + 8 * q);
      r4[q] = *reinterpret_cast<const float4*>(s_sr + nt + 8 * q);
    }
  };
  if (!a.dbg_main && (a.N & 3) == 0) {
    // Common case: four-channel vector stores with no branches. A lane
    // whose token or channel group is past the end writes its vector to a
    // dummy slot instead, so every store instruction is issued.
    const bool wide = (a.N & 7) == 0;            // bf16: eight-channel groups whole or past the end
    auto epi = [&](auto ebc) SERQ_INLINE {
      constexpr int EB = decltype(ebc)::value;
      uint8_t* yrow[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j)
        yrow[j] = mrow[j] < a.M ? static_cast<uint8_t*>(a.Y) + static_cast<size_t>(mrow[j]) * a.N * EB : nullptr;
      uint8_t* const sink = reinterpret_cast<uint8_t*>(tile_store_sink) + 16 * lane;
      static_for<TN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int nt = wn * 32 * TN + i * 32 + 4 * h;
        float4 w4[4], r4[4];
        load_scales(nt, w4, r4);
        float t[TM][16];
        residual(ic, t, w4);
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          float y[4][4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float rv4[4] = {r4[q].x, r4[q].y, r4[q].z, r4[q].w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
              y[q][c] = sxm[j] * __builtin_fmaf(rv4[c], static_cast<float>(acc[i][j][4 * q + c]), t[j][4 * q + c]);
          }
          if constexpr (EB == 2) {
            if (wide) {
              // Lane half h holds channels 8 q + 4 h + (0..3); one swap of the
              // halves' packed groups per dword gives half 0 channels
              // 16 p + (0..7) and half 1 channels 16 p + 8 + (0..7): one
              // 16-byte store per lane and pair of groups.
#pragma unroll
              for (int p = 0; p < 2; ++p) {
                const uint32_t g0[2] = {pack_bf16x2(y[2 * p][0], y[2 * p][1]), pack_bf16x2(y[2 * p][2], y[2 * p][3])};
                const uint32_t g1[2] = {pack_bf16x2(y[2 * p + 1][0], y[2 * p + 1][1]),
                                        pack_bf16x2(y[2 * p + 1][2], y[2 * p + 1][3])};
                uint32_t lo[2], hi[2];
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                  const auto sw2 = __builtin_amdgcn_permlane32_swap(g0[d], g1[d], false, false);
                  lo[d] = sw2[0];
                  hi[d] = sw2[1];
                }
                const int n = n0 + nt - 4 * h + 16 * p + 8 * h;
                uint8_t* dst = (yrow[j] != nullptr && n < a.N) ? yrow[j] + 2 * n : sink;
                *reinterpret_cast<uint4*>(dst) = make_uint4(lo[0], lo[1], hi[0], hi[1]);
              }
              continue;
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + nt + 8 * q;
            uint8_t* dst = (yrow[j] != nullptr && n < a.N) ? yrow[j] + EB * n : sink;
            if constexpr (EB == 2)
              *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(y[q][0], y[q][1]), pack_bf16x2(y[q][2], y[q][3]));
            else
              *reinterpret_cast<float4*>(dst) = make_float4(y[q][0], y[q][1], y[q][2], y[q][3]);
          }
        }
      });
    };
    if (a.y_bf16)
      epi(std::integral_constant<int, 2>{});
    else
      epi(std::integral_constant<int, 4>{});
    return;
  }
  // Debug sums or N % 4 != 0: element-wise checks.
  const int esz = a.y_bf16 ? 2 : 4;
  static_for<TN>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int nt = wn * 32 * TN + i * 32 + 4 * h;   // first channel (within the tile) of group q = 0
    float4 w4[4], r4[4];
    load_scales(nt, w4, r4);
    if (a.dbg_main) {                            // exact main sums, for tests
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int n = n0 + nt + 8 * (e >> 2) + (e & 3);
          if (mrow[j] < a.M && n < a.N) a.dbg_main[static_cast<size_t>(mrow[j]) * a.N + n] = acc[i][j][e] >> C::SHIFT;
        }
    }
    float t[TM][16];
    residual(ic, t, w4);
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = mrow[j];
      if (m >= a.M) continue;
      if (a.dbg_res) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int n = n0 + nt + 8 * (e >> 2) + (e & 3);
          if (n < a.N) a.dbg_res[static_cast<size_t>(m) * a.N + n] = acc[i][j][e] >> C::SHIFT;
        }
      }
      uint8_t* yrow = static_cast<uint8_t*>(a.Y) + static_cast<size_t>(m) * a.N * esz;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float rv4[4] = {r4[q].x, r4[q].y, r4[q].z, r4[q].w};
        float y[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          y[c] = sxm[j] * __builtin_fmaf(rv4[c], static_cast<float>(acc[i][j][4 * q + c]), t[j][4 * q + c]);
        const int n = n0 + nt + 8 * q;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (n + c >= a.N) break;
          if (a.y_bf16)
            reinterpret_cast<uint16_t*>(yrow)[n + c] = f32_to_bf16_rne(y[c]);
          else
            reinterpret_cast<float*>(yrow)[n + c] = y[c];
        }
      }
    }
  });
}

// ---------------------------------------------------------------------------
// Skinny kernel (4..32 tokens, and W4A8 from one token): eight-wave
// workgroups, each owning G <= 8 16-channel groups and one K
// slice of `seg` 256-code chunks (KS slices in all). The workgroup's slice of
// the activation rows is loaded into LDS once and shared by its G groups.
// Few groups per workgroup with the whole of K would reload the activations
// for every group (for 16 tokens as many bytes as the weights themselves);
// the host picks G and KS to keep that traffic, plus the partial sums below,
// small while still launching about one workgroup per CU.
//
// The workgroup's work is the flat list of G x Ts items, group-major: an
// item is 256 codes of a group's 16 weight rows (128 bytes of each row) or,
// last in slice 0, the zero-padded Q(R) rows against the first activation
// codes. Wave w takes items w, w + 8, ... in units of IPW, issues a unit's
// loads, then computes it while the next unit's loads are in flight (a unit
// is two or three items). So at
// any moment a CU's loads fall in a few tens of KB of contiguous weight rows
// (measured faster than deeper per-wave rings spread over several groups,
// whose scattered requests streamed at about two thirds of the rate). Every
// load is unconditional (clamped addresses, zeroed activation side) and
// every slot is computed, so the compiler's load counters stay exact. Lane
// (row l16, quarter g) of an item holds weight bytes [32 g, 32 g + 32) of its
// row's 128 (codes [64 g, 64 g + 64)) and reads the activation codes at the
// same positions for tokens l16 and 16 + l16 from LDS (rows padded by 16
// bytes: the 16 tokens of a read hit distinct banks); v_mfma_i32_16x16x64_i8
// takes them in four steps, and the item's sums are added into its group's
// LDS slot.
//
// With one slice, wave j then writes group j. With several, every
// workgroup stores its int32 slot sums in a workspace, and the last of a
// group set's KS workgroups to finish (an agent-scope counter) adds the KS
// partial sums, writes the outputs and resets the counter for the next call.
// ---------------------------------------------------------------------------

constexpr int kSkxWaves = 8;
constexpr int kSkxMaxGroups = 8;            // groups per workgroup
constexpr int kSkxLds = 159 * 1024;         // dynamic LDS bytes: activation slice + group slots
                                            // (the rest of the 160 KB holds the static flag)

template <int MG>
constexpr int skx_slot_bytes() { return 2 * MG * 64 * 16; }

// Scratch of the K split (KS > 1): one counter per group set and the slices'
// int32 partial sums, KS x ngroups x [main, residual][token block][lane].
// Both are file-scope device arrays, so each device holds its own copy from
// the moment the code object is loaded, zero-filled, and no call allocates:
// a plan whose partial sums would not fit takes a tile kernel instead. Every
// counter is zero when a launch starts (zero at load; the last workgroup of
// a group set puts its counter back to zero, and the next launch on the
// stream starts after that one has ended). Launches that take the split
// path on one device share the arrays, so they must not overlap in time.
constexpr int kSkxCounters = 16384;                       // group sets per split launch, at most
constexpr size_t kSkxPartBytes = size_t{16} << 20;        // partial sums per split launch, at most
__device__ __align__(256) int skx_counters[kSkxCounters];
__device__ __align__(256) v4i skx_partials[kSkxPartBytes / sizeof(v4i)];

struct SkinnySplit {
  int G, nb, KS, seg;       // groups per workgroup, group sets, K slices, chunks per slice
};

// f / d for 0 <= f with f d < 2^32, d >= 1, as one high multiply by
// mul = floor((2^32 - 1) / d) + 1 (mul = 2^32 / d when d is a power of two,
// else ceil(2^32 / d), whose excess over 2^32 / d, times f, stays below
// one): the skinny kernel's per-item divisions by wave-uniform divisors are
// then single scalar multiplies instead of the ~25-instruction sequence of a
// general division.
struct SmallDiv {
  int d;
  uint32_t mul;
  __device__ explicit SmallDiv(int d_) : d(d_), mul(d_ > 1 ? 0xFFFFFFFFu / static_cast<uint32_t>(d_) + 1u : 0u) {}
  __device__ int operator()(int f) const {
    return d > 1 ? static_cast<int>(__umulhi(static_cast<uint32_t>(f), mul)) : f;
  }
};

template <int MG, int A_BITS, int IPW>
__global__ __launch_bounds__(64 * kSkxWaves, 1) void serq_skinny_kernel(LinearArgs a, SkinnySplit sp) {
  constexpr int SHIFT = A_BITS == 4 ? 8 : 4;
  constexpr int CWB = 128;                  // weight bytes per row and item
  constexpr int CXB = 2 * A_BITS * 16;      // activation bytes per row and item
  constexpr int LW = 2;                     // 16-byte weight loads per lane and item
  constexpr int LX = CXB / 64;              // 16-byte activation reads per lane and item
  constexpr int SLOT = skx_slot_bytes<MG>() / 16;   // v4i per group slot
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int Kb = a.K / 2, Xrow = a.K * A_BITS / 8;
  const int Rb = rq_row_bytes(a.r);
  const bool has_res = a.r > 0;
  const int ngroups = (a.N + 15) / 16;
  const int b = static_cast<int>(blockIdx.x) % sp.nb, ks = static_cast<int>(blockIdx.x) / sp.nb;
  // Group j of this workgroup is b + nb j: at any moment the CUs stream rows
  // spread over the whole matrix rather than each its own contiguous block.
  auto grp = [&](int j) { return b + sp.nb * j; };
  const int Gb = (ngroups - b + sp.nb - 1) / sp.nb;   // groups of this workgroup
  const int C = (a.K + 255) / 256;
  const int c0 = ks * sp.seg;                         // first chunk of the slice
  const int Cs = min(sp.seg, C - c0);                 // main items per group
  const bool res_here = has_res && ks == 0;
  const int Ts = Cs + (res_here ? 1 : 0);             // items per group
  const int NI = Gb * Ts;                             // items of the workgroup
  const int XS = sp.seg * CXB + 16;                   // LDS row stride of the activation slice
  const int xoff = c0 * CXB;                          // slice start within an activation row
  const int xlen = min(Cs * CXB, Xrow - xoff);        // slice bytes per row
  v4i* slots = reinterpret_cast<v4i*>(lds + a.M * XS);   // [Gb][main, residual][token block][lane]
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  // Scales of the group this wave writes at the end (group wv), then the
  // activation slice into LDS (direct loads); both are older than every
  // weight load.
  float wsc[4], rsc[4], sxv[MG];
  {
    const int nb = grp(min(wv, Gb - 1)) * 16;
    const float* srp = has_res ? a.sr : a.sw;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int n = min(nb + 4 * g + e, a.N - 1);
      wsc[e] = a.sw[n];
      rsc[e] = srp[n];                      // replaced by zeros at the end when r == 0
    }
#pragma unroll
    for (int t = 0; t < MG; ++t) sxv[t] = a.sx[min(t * 16 + l16, a.M - 1)];
  }
  {
    const int per_row = (xlen + 1023) / 1024;
    const SmallDiv by_row(max(per_row, 1));
    for (int q = wv; q < a.M * per_row; q += kSkxWaves) {
      const int t = by_row(q), c = q - t * per_row;
      if (1024 * c + 16 * lane < xlen)
        dma16(a.Xq + static_cast<size_t>(t) * Xrow + xoff, 1024 * c + 16 * lane, lds_base + t * XS + 1024 * c);
    }
  }
  for (int i = threadIdx.x; i < Gb * SLOT; i += 64 * kSkxWaves) slots[i] = v4i{0, 0, 0, 0};

  // Item f (group f / Ts, item f % Ts of it). Past the list the loads read
  // the last item's bytes and the item is computed against zero
  // activations. The group and item index travel with the loaded data.
  struct Buf {
    uint4 w[IPW][LW];
    int j[IPW], t[IPW];
  };
  const SmallDiv by_item(Ts);
  auto issue = [&](int u, Buf& bf) {
    static_for<IPW>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const int f = min(wv + kSkxWaves * (u * IPW + k), NI - 1);
      const int j = by_item(f), t = f - j * Ts;
      bf.j[k] = j;
      bf.t[k] = t;
      const bool res = t >= Cs;
      const int nrow = min(grp(j) * 16 + l16, a.N - 1);
      const uint8_t* wp = res ? a.Rq + static_cast<size_t>(nrow) * Rb : a.Wq + static_cast<size_t>(nrow) * Kb;
      const int wlim = res ? Rb : Kb;
      const int c = res ? 0 : c0 + t;
#pragma unroll
      for (int l = 0; l < LW; ++l) {
        const int o = c * CWB + g * (CWB / 4) + 16 * l;
        bf.w[k][l] = *reinterpret_cast<const uint4*>(wp + min(o, wlim - 16));
      }
    });
  };
  auto consume = [&](int u, const Buf& bf) {
    static_for<IPW>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const bool used = wv + kSkxWaves * (u * IPW + k) < NI;
      const int j = bf.j[k], t = bf.t[k];
      const bool res = t >= Cs;
      // Activation bytes of the item within the slice row, and the bytes
      // that take part (the row's end, or the residual's codes).
      const int xo = res ? 0 : t * CXB;
      const int xlim = !used ? 0 : (res ? Rb * A_BITS / 4 : xlen);
      uint4 xs[MG][LX];
#pragma unroll
      for (int tb = 0; tb < MG; ++tb)
#pragma unroll
        for (int l = 0; l < LX; ++l) {
          const int o = xo + g * (CXB / 4) + 16 * l;
          const int m = tb * 16 + l16;
          xs[tb][l] = (m < a.M && o < xlim) ? *reinterpret_cast<const uint4*>(lds + m * XS + o)
                                            : make_uint4(0, 0, 0, 0);
        }
      v4i p[MG];
#pragma unroll
      for (int tb = 0; tb < MG; ++tb) p[tb] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint4 ww = bf.w[k][st >> 1];
        const v4i wa = (st & 1) ? widen16(ww.z, ww.w) : widen16(ww.x, ww.y);
#pragma unroll
        for (int tb = 0; tb < MG; ++tb) {
          v4i xv;
          if constexpr (A_BITS == 4) {
            const uint4 xx = xs[tb][st >> 1];
            xv = (st & 1) ? widen16(xx.z, xx.w) : widen16(xx.x, xx.y);
          } else {
            xv = split16(xs[tb][st]);
          }
          p[tb] = mfma(wa, xv, p[tb]);
        }
      }
      if (used) {
        int* dst = reinterpret_cast<int*>(slots + j * SLOT + (res ? MG : 0) * 64 + lane);
#pragma unroll
        for (int tb = 0; tb < MG; ++tb)
#pragma unroll
          for (int e = 0; e < 4; ++e) atomicAdd(dst + tb * 256 + e, p[tb][e]);
      }
    });
  };

  // Unit 0's loads go out first; then this wave's scale and direct loads
  // (older) are waited for and one barrier publishes the activation slice
  // and the cleared slots. Unit u + 1 is issued before unit u is computed,
  // the loop unrolled by two so each buffer keeps its registers.
  const int units = ((NI + kSkxWaves - 1) / kSkxWaves + IPW - 1) / IPW;
  Buf A, B;
  issue(0, A);
  wait_vmcnt<IPW * LW>();
  lds_barrier();
  int u = 0;
  for (; u + 2 <= units; u += 2) {
    issue(u + 1, B);
    consume(u, A);
    issue(u + 2, A);
    consume(u + 1, B);
  }
  if (u < units) consume(u, A);
  wait_vmcnt<0>();                           // the last issue, past the end, unused
  lds_barrier();

  if (sp.KS > 1) {
    // Partial sums out, counter, last workgroup reads them back. Every byte
    // that crosses workgroups (partial sums, counters) is accessed only by
    // agent-scope atomic operations, never by plain loads or stores. On
    // gfx950 (the gfx942 memory model) the relaxed agent-scope store and load
    // are global_store / global_load with sc1, which write through to and
    // read from the point where all XCDs are coherent, and the counter RMW is
    // performed there too. The ordering that a release / acquire pair would
    // give is made by the hardware sequence instead: s_waitcnt vmcnt(0) waits
    // for every partial-sum store's acknowledgement (the data is at the
    // coherence point) before the counter RMW is issued; the group set's last
    // workgroup sees KS - 1 returned only after all KS RMWs, and issues its
    // loads after that return (vmcnt wait, then barrier), so they observe
    // every slice's stores. What release / acquire would add -- a write-back
    // of the whole L2 before the RMW and an invalidation of it after -- only
    // matters for data moved by plain stores and loads, of which there is
    // none here (and each costs more than the whole split saves). Slice 0
    // alone holds residual sums.
    if (wv < Gb) {
      long long* dst = reinterpret_cast<long long*>(skx_partials + (static_cast<size_t>(ks) * ngroups + grp(wv)) * SLOT);
      const long long* src = reinterpret_cast<const long long*>(slots + wv * SLOT);
      const int hn = ks == 0 && has_res ? 2 * MG : MG;
      for (int h = 0; h < hn; ++h)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          __hip_atomic_store(dst + (h * 64 + lane) * 2 + e, src[(h * 64 + lane) * 2 + e], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vmcnt<0>();
    lds_barrier();
    if (threadIdx.x == 0)
      s_last = __hip_atomic_fetch_add(skx_counters + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == sp.KS - 1;
    lds_barrier();
    if (!s_last) return;
    if (threadIdx.x == 0) __hip_atomic_store(skx_counters + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (wv >= Gb) return;
  v4i sm[MG], sr[MG];
  if (sp.KS == 1) {
#pragma unroll
    for (int t = 0; t < MG; ++t) {
      sm[t] = slots[wv * SLOT + t * 64 + lane];
      sr[t] = slots[wv * SLOT + (MG + t) * 64 + lane];
    }
  } else {
    auto ld = [&](int q, int h) {
      const long long* src = reinterpret_cast<const long long*>(skx_partials + (static_cast<size_t>(q) * ngroups + grp(wv)) * SLOT);
      const long long lo = __hip_atomic_load(src + (h * 64 + lane) * 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const long long hi = __hip_atomic_load(src + (h * 64 + lane) * 2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return v4i{static_cast<int>(lo), static_cast<int>(lo >> 32), static_cast<int>(hi), static_cast<int>(hi >> 32)};
    };
#pragma unroll
    for (int t = 0; t < MG; ++t) {
      sm[t] = v4i{0, 0, 0, 0};
      sr[t] = has_res ? ld(0, MG + t) : v4i{0, 0, 0, 0};
    }
    for (int q = 0; q < sp.KS; ++q)
#pragma unroll
      for (int t = 0; t < MG; ++t) sm[t] += ld(q, t);
  }
  const float4 w4 = make_float4(wsc[0], wsc[1], wsc[2], wsc[3]);
  const float4 r4 = has_res ? make_float4(rsc[0], rsc[1], rsc[2], rsc[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
  const int nb = grp(wv) * 16;
#pragma unroll
  for (int t = 0; t < MG; ++t) store4<SHIFT>(a, sm[t], sr[t], t * 16 + l16, nb + 4 * g, sxv[t], w4, r4);
}

// ---------------------------------------------------------------------------
// GEMV kernel (W4A4, M <= 3 tokens): v_dot8c_i32_i4 multiplies eight packed
// int4 codes of each operand and adds to an int32, in the canonical nibble
// order of both Q(W^) and the activation codes, so the packed bytes are used
// as loaded -- no widening, and no matrix-core work thrown away on missing
// tokens.
//
// A wave streams 8 weight rows over a K range: each load instruction takes
// 128 contiguous bytes (one cache line) of each of the 8 rows, lane (row
// l / 8, part l % 8) 16 of them, with two units of kGemvUnit instructions
// in flight. A workgroup of KP waves covers one row octet split into KP K
// ranges (KP = 8 for narrow layers, so that they still keep about sixteen
// waves per CU loading, else 4). The
// activation rows (M x K/2 bytes) are loaded into LDS once per workgroup and
// read back in broadcast. At the end each row's partial sums are added over
// its 8 lanes, then over the KP waves through LDS, and the K range 0 wave
// writes the outputs. The salient-row residual is one more instruction of the
// last K range: the zero-padded Q(R) rows (at most 128 bytes) against the
// first activation codes.
// ---------------------------------------------------------------------------

constexpr int kGemvUnit = 4;                // load instructions per unit (two units in flight per wave)
constexpr int kGemvMaxX = 64 * 1024;        // LDS bytes for the activation rows
constexpr int kGemvMaxTokens = 3;          // from four tokens the skinny kernel measured faster

template <int MT, int KP>
__global__ __launch_bounds__(64 * KP) void serq_gemv_kernel(LinearArgs a) {
  constexpr int OCT = 1;                              // row octets per workgroup
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];   // [MT][Kb] activation codes
  __shared__ int red[KP][2][MT][64];                  // [wave][main, residual][token][lane]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int oct = wv / KP, kp = wv % KP;
  const int r8 = lane >> 3, part = lane & 7;
  const int Kb = a.K / 2;
  const int Rb = rq_row_bytes(a.r);
  const int n = (static_cast<int>(blockIdx.x) * OCT + oct) * 8 + r8;   // this lane's channel
  const int nrow = min(n, a.N - 1);
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  // Scales of this lane's channel and the token scales, oldest loads first.
  const float swn = a.sw[nrow];
  const float srn = a.r > 0 ? a.sr[nrow] : 0.0f;
  float sxv[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) sxv[t] = a.sx[t];
  // Activation rows into LDS, 1 KB per load instruction over the four waves.
  const int nx = (MT * Kb + 1023) / 1024;
  for (int q = wv; q < nx; q += KP) {
    const int off = 1024 * q + 16 * lane;
    if (off < MT * Kb) dma16(a.Xq, static_cast<uint32_t>(off), lds_base + 1024 * q);
  }

  // This wave's K range: 128-byte lines [l0, l1) of its 8 rows, plus the
  // residual line for the last range.
  const int lines = (Kb + 127) / 128;
  const int per = (lines + KP - 1) / KP;
  const int l0 = min(kp * per, lines), l1 = min(l0 + per, lines);
  const bool res_here = a.r > 0 && kp == KP - 1;
  const int total = (l1 - l0) + (res_here ? 1 : 0);
  const uint8_t* wrow = a.Wq + static_cast<size_t>(nrow) * Kb;
  const uint8_t* rrow = a.Rq + static_cast<size_t>(nrow) * Rb;   // read only when r > 0
  // Item i of this wave: line l0 + i, or the residual line after the last.
  // Every load is issued (items past the end reload the last one, pieces
  // past a row's end read its last 16 bytes) and every item is computed,
  // with the activation side zeroed where the weight bytes do not count:
  // the compiler's load counters then stay exact and the ring never drains.
  auto load = [&](int i, uint4& w) {
    const int ii = min(i, max(total - 1, 0));
    const bool res = res_here && l0 + ii >= l1;
    const uint8_t* p = res ? rrow : wrow;
    const int lim = res ? Rb : Kb;
    const int off = (res ? 0 : 128 * (l0 + ii)) + 16 * part;
    w = *reinterpret_cast<const uint4*>(p + min(off, lim - 16));
  };
  // Units of kGemvUnit items, double-buffered: unit u + 1 is issued before
  // unit u is computed; the loop is unrolled by two so each buffer keeps its
  // registers (a single rotating ring got its loads hoisted into fresh
  // registers and copied back at the loop end, which waits for them).
  struct Unit {
    uint4 w[kGemvUnit];
  };
  auto issue = [&](int u, Unit& b) {
    static_for<kGemvUnit>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      load(u * kGemvUnit + k, b.w[k]);
    });
  };
  Unit A, B;
  issue(0, A);
  // This wave's activation loads are older than its weight loads: once at
  // most the weight loads are outstanding, its part of LDS is written.
  wait_vmcnt<kGemvUnit>();
  lds_barrier();

  int acc[MT], accr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = accr[t] = 0;
  auto consume1 = [&](int i, const uint4& w) {
    const bool used = i < total;
    const int ii = min(i, max(total - 1, 0));
    const bool res = res_here && l0 + ii >= l1;
    const int off = (res ? 0 : 128 * (l0 + ii)) + 16 * part;
    const bool inx = used && off < (res ? Rb : Kb);   // (Q(R)'s padding is zero)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint4 x = inx ? *reinterpret_cast<const uint4*>(lds + t * Kb + off) : make_uint4(0, 0, 0, 0);
      int d = 0;
      d = __builtin_amdgcn_sdot8(static_cast<int>(w.x), static_cast<int>(x.x), d, false);
      d = __builtin_amdgcn_sdot8(static_cast<int>(w.y), static_cast<int>(x.y), d, false);
      d = __builtin_amdgcn_sdot8(static_cast<int>(w.z), static_cast<int>(x.z), d, false);
      d = __builtin_amdgcn_sdot8(static_cast<int>(w.w), static_cast<int>(x.w), d, false);
      if (res) accr[t] += d; else acc[t] += d;
    }
  };
  auto consume = [&](int u, const Unit& b) {
    static_for<kGemvUnit>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      consume1(u * kGemvUnit + k, b.w[k]);
    });
  };
  // fence_sums: an empty asm that takes the sums, so a unit's dot products
  // are done before the next issue into its registers (the compiler would
  // otherwise sink them, load into fresh registers and copy back at the loop
  // end, waiting for the loads).
  auto fence_sums = [&]() {
#pragma unroll
    for (int t = 0; t < MT; ++t) asm volatile("" : "+v"(acc[t]), "+v"(accr[t]) :: "memory");
  };
  const int units = (total + kGemvUnit - 1) / kGemvUnit;
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
  wait_vmcnt<0>();                               // the last issue, past the end, unused

  // Sum over the row's 8 lanes, then over the KP waves of the row octet.
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      acc[t] += __shfl_xor(acc[t], off, 64);
      accr[t] += __shfl_xor(accr[t], off, 64);
    }
  }
  if (KP > 1) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      red[wv][0][t][lane] = acc[t];
      red[wv][1][t][lane] = accr[t];
    }
    lds_barrier();
    if (kp != 0) return;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int k = 1; k < KP; ++k) {
        acc[t] += red[wv + k][0][t][lane];
        accr[t] += red[wv + k][1][t][lane];
      }
  }
  if (part != 0 || n >= a.N) return;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (t >= a.M) break;
    const size_t idx = static_cast<size_t>(t) * a.N + n;
    if (a.dbg_main) {
      a.dbg_main[idx] = acc[t];
      a.dbg_res[idx] = accr[t];
    }
    const float y = sxv[t] * __builtin_fmaf(srn, static_cast<float>(accr[t]), swn * static_cast<float>(acc[t]));
    if (a.y_bf16)
      static_cast<uint16_t*>(a.Y)[idx] = f32_to_bf16_rne(y);
    else
      static_cast<float*>(a.Y)[idx] = y;
  }
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

// Raise a kernel's dynamic-LDS limit once per device (the attribute is set
// with the device current; `done` holds one bit per device).
hipError_t ensure_max_lds(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const uint64_t bit = uint64_t{1} << dev;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

template <int TN, int TM, int A_BITS, int WGM, int KG>
hipError_t launch_tile(const LinearArgs& a, hipStream_t st) {
  using C = TileCfg<TN, TM, A_BITS, WGM, KG>;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_max_lds(reinterpret_cast<const void*>(&serq_tile_kernel<TN, TM, A_BITS, WGM, KG>),
                                C::LDS_BYTES, lds_set);
  if (e != hipSuccess) return e;
  const int n_tiles = (a.N + C::BN - 1) / C::BN;
  const int m_tiles = (a.M + C::BM - 1) / C::BM;
  serq_tile_kernel<TN, TM, A_BITS, WGM, KG><<<dim3(n_tiles * m_tiles), dim3(C::NT), C::LDS_BYTES, st>>>(a, n_tiles);
  return hipGetLastError();
}

// G and KS: about one workgroup per CU, the slice fitting LDS beside the
// group slots; one slice if the activations fit, else the choice with the
// least activation traffic (every workgroup loads its slice of the M rows)
// plus partial-sum traffic (KS x the outputs, written and read back). Between
// two choices whose slices both hold eight chunks or more, that traffic is
// weighted by the padding of the work grid (groups per workgroup times
// workgroups, slices times their length, over the layer's groups and
// chunks): every workgroup runs as many items as the fullest one, so a
// ragged last slice or group set costs its padding in time (8B down at 32
// tokens: 4 x 4 even slices 13.6 us against 15.9 for 5 x 5 of 12, 8 of the
// last; 1.2-1.5x on the 28672-, 14336- and 11008-long rows at 9-32 tokens;
// with shorter slices the split's fixed tail outweighs it).
template <int MG, int A_BITS>
SkinnySplit plan_skinny(const LinearArgs& a) {
  constexpr int CXB = 2 * A_BITS * 16;
  const int ngroups = (a.N + 15) / 16;
  const int C = (a.K + 255) / 256;
  SkinnySplit best{0, 0, 0, 0};
  double best_cost = 0.0, best_pad = 1.0;
  for (int G = 1; G <= kSkxMaxGroups; ++G) {
    const int nb = (ngroups + G - 1) / G;
    if (G > 1 && (ngroups + G - 2) / (G - 1) == nb) continue;   // same group sets as G - 1
    int KS = max(1, min(C, (kCUs + nb - 1) / nb));
    if (ngroups > kCUs * kSkxMaxGroups) KS = 1;
    for (;; ++KS) {
      const int seg = (C + KS - 1) / KS;
      if (static_cast<long>(a.M) * (seg * CXB + 16) + G * skx_slot_bytes<MG>() <= kSkxLds || KS >= C) break;
    }
    const int seg = (C + KS - 1) / KS;
    if (static_cast<long>(a.M) * (seg * CXB + 16) + G * skx_slot_bytes<MG>() > kSkxLds) continue;
    const int ks_used = (C + seg - 1) / seg;
    if (ks_used > 1 && (nb > kSkxCounters ||
                        static_cast<size_t>(ks_used) * ngroups * skx_slot_bytes<MG>() > kSkxPartBytes))
      continue;
    const double xbytes = static_cast<double>(nb) * a.M * (a.K * A_BITS / 8);
    const double pbytes = ks_used > 1 ? 2.0 * ks_used * ngroups * skx_slot_bytes<MG>() : 0.0;
    const double cost = xbytes + pbytes;
    const double pad = static_cast<double>(nb) * G * ks_used * seg / (static_cast<double>(ngroups) * C);
    const bool long_slices = seg >= 8 && best.seg >= 8;
    const double cmp_new = long_slices ? cost * pad : cost, cmp_best = long_slices ? best_cost * best_pad : best_cost;
    // One slice whenever the activations fit: the split's tail (partial sums
    // out, counter, the last workgroup's reads) measured several us.
    const bool better = best.G == 0 || (ks_used == 1 && best.KS > 1) ||
                        (cmp_new < cmp_best && !(ks_used > 1 && best.KS == 1));
    if (better) {
      best = SkinnySplit{G, nb, ks_used, seg};
      best_cost = cost;
      best_pad = pad;
    }
  }
  return best;
}

template <int MG, int A_BITS, int IPW>
hipError_t launch_skinny_ipw(const LinearArgs& a, const SkinnySplit& sp, hipStream_t st) {
  constexpr int CXB = 2 * A_BITS * 16;
  const int lds = a.M * (sp.seg * CXB + 16) + sp.G * skx_slot_bytes<MG>();
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_max_lds(reinterpret_cast<const void*>(&serq_skinny_kernel<MG, A_BITS, IPW>), kSkxLds,
                                lds_set);
  if (e != hipSuccess) return e;
  serq_skinny_kernel<MG, A_BITS, IPW><<<dim3(sp.nb * sp.KS), dim3(64 * kSkxWaves), lds, st>>>(a, sp);
  return hipGetLastError();
}

template <int MG, int A_BITS>
hipError_t launch_skinny(const LinearArgs& a, hipStream_t st) {
  const SkinnySplit sp = plan_skinny<MG, A_BITS>(a);
  if (sp.G == 0) return hipErrorInvalidValue;   // plan_linear only picks the skinny kernel when a plan exists
  // A wave's items of one group in a single unit when they are three or
  // fewer (q_proj-sized rows: 4.95 us at 8 tokens against 5.6 in units of
  // two), else units of two items (two units in flight): on long rows fewer
  // loads in flight stream faster than a group's items at once (8B down at
  // 16 tokens 9.0 against 9.8 us in units of eight; 28672 x 8192 at 8 tokens
  // 24.6 against 30.1; 8192 x 28672 at 32 tokens 27.7 against 32.0).
  const int per = max(2, (sp.seg + (a.r > 0 ? 1 : 0) + kSkxWaves - 1) / kSkxWaves);
  if (per == 3) return launch_skinny_ipw<MG, A_BITS, 3>(a, sp, st);
  return launch_skinny_ipw<MG, A_BITS, 2>(a, sp, st);
}

template <int MT, int KP>
hipError_t launch_gemv_kp(const LinearArgs& a, hipStream_t st) {
  const int octets = (a.N + 7) / 8;
  const int grid = octets;
  const int lds = (MT * (a.K / 2) + 15) / 16 * 16;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_max_lds(reinterpret_cast<const void*>(&serq_gemv_kernel<MT, KP>), kGemvMaxX, lds_set);
  if (e != hipSuccess) return e;
  serq_gemv_kernel<MT, KP><<<dim3(grid), dim3(64 * KP), lds, st>>>(a);
  return hipGetLastError();
}

// Four K ranges per row octet, eight when there are few octets (so that
// narrow layers still keep about sixteen waves per CU loading).
template <int MT>
hipError_t launch_gemv(const LinearArgs& a, hipStream_t st) {
  const int octets = (a.N + 7) / 8;
  if (octets < 4 * kCUs) return launch_gemv_kp<MT, 8>(a, st);
  return launch_gemv_kp<MT, 4>(a, st);
}

hipError_t launch_tile256(const LinearArgs& a, hipStream_t st) {
  using C = Tile256Cfg;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_max_lds(reinterpret_cast<const void*>(&serq_tile256_kernel), C::LDS_BYTES, lds_set);
  if (e != hipSuccess) return e;
  const int n_tiles = (a.N + C::BN - 1) / C::BN;
  const int m_tiles = (a.M + C::BM - 1) / C::BM;
  serq_tile256_kernel<<<dim3(n_tiles * m_tiles), dim3(C::NT), C::LDS_BYTES, st>>>(a, n_tiles);
  return hipGetLastError();
}

template <int A_BITS>
hipError_t launch_tile_bits(const LinearArgs& a, const LinearPlan& p, hipStream_t st) {
  if constexpr (A_BITS == 4)
    if (p.tn == 4 && p.tm == 4) return launch_tile256(a, st);
  if (p.tn == 2 && p.tm == 2 && p.wgm == 2 && p.kg == 1) return launch_tile<2, 2, A_BITS, 2, 1>(a, st);
  if (p.tn == 2 && p.tm == 2 && p.wgm == 2 && p.kg == 2) return launch_tile<2, 2, A_BITS, 2, 2>(a, st);
  if (p.tn == 2 && p.tm == 1 && p.wgm == 2 && p.kg == 1) return launch_tile<2, 1, A_BITS, 2, 1>(a, st);
  if (p.tn == 1 && p.tm == 1 && p.wgm == 2 && p.kg == 1) return launch_tile<1, 1, A_BITS, 2, 1>(a, st);
  if (p.tn == 1 && p.tm == 1 && p.wgm == 1 && p.kg == 4) return launch_tile<1, 1, A_BITS, 1, 4>(a, st);
  if (p.tn == 1 && p.tm == 2 && p.wgm == 1 && p.kg == 4) return launch_tile<1, 2, A_BITS, 1, 4>(a, st);
  if constexpr (A_BITS == 4)
    if (p.tn == 1 && p.tm == 2 && p.wgm == 1 && p.kg == 2) return launch_tile<1, 2, A_BITS, 1, 2>(a, st);
  return hipErrorInvalidValue;
}


// ---------------------------------------------------------------------------
// bf6 route: the same linear on v_mfma_scale_f32_32x32x64_f8f6f4 with both
// operands as E3M2 six-bit values and unit block scales (E8M0 127 = 2^0).
// Every int4 code is exactly such a value, a product of two codes is at most
// 64 in magnitude and every partial sum an integer of magnitude <= 64 K <=
// 2^24, so the fp32 accumulators hold the exact integer dot products and the
// epilogue is serq_linear's on those integers.
//
// Operands come in the bf6 tile layout (weights prepacked on the host,
// activations re-encoded by serq_act_bf6): for one 128-code k-tile the 128
// rows of a tile are 12 KB of contiguous 24-byte lane fragments, in the
// order the MFMA takes them. So the direct global->LDS loads move contiguous
// 1 KB chunks, and each fragment read is three 8-byte LDS reads at a 24-byte
// lane stride (16 lanes cover the 32 banks once: no conflicts).
//
// Workgroup: 128 x 128 outputs, four waves of 64 x 64 (2 x 2 blocks of
// 32 x 32; A = weight rows, B = tokens, the output layout of the integer
// 32 x 32 MFMA). Three LDS stages of one k-tile (12 KB of weights, then 12 KB
// of activations); waves 0-1 load the weight half, 2-3 the activation half,
// six 1 KB chunks each per stage, so every wave counts the same loads per
// k-tile. The k-tile pipeline is the integer tile kernel's: wait until only
// the next k-tile's loads are outstanding, one barrier publishes k-tile t and
// frees the buffer of t - 1, which the loads of t + 2 go into. The residual
// k-tiles (Q(R) against the first activation k-tiles) follow the main ones
// in the same pipeline, into a second set of accumulators.
// ---------------------------------------------------------------------------

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kB6Tile = 128;                        // row padding of the layout, codes per k-tile
constexpr int kB6Frag = 24;                         // bytes of one lane fragment (32 codes)
constexpr int kB6Step = 64 * kB6Frag;               // one MFMA operand of a 32-row block
constexpr int kB6Block = 2 * kB6Step;               // 32 rows x 128 codes

// Tile shape: each wave owns TN x TM blocks of 32 x 32, the workgroup a
// WNW x WMW grid of waves; STAGES LDS buffers of one k-tile each, OCC
// workgroups per CU. Every wave loads an equal share of both halves of a
// stage (WB weight and XB activation bytes): 1 KB instructions, the last one
// of a share with 32 lanes when the share ends on a half kilobyte, so each
// wave issues LOADS instructions per k-tile.
template <int TN, int TM, int WNW, int WMW, int STAGES, int OCC>
struct B6Cfg {
  static constexpr int NW = WNW * WMW, NT = 64 * NW;
  static constexpr int BN = 32 * TN * WNW, BM = 32 * TM * WMW;
  static constexpr int W_HALF = BN / 32 * kB6Block, X_HALF = BM / 32 * kB6Block;
  static constexpr int STAGE = W_HALF + X_HALF;
  static constexpr int WB = W_HALF / NW, XB = X_HALF / NW;
  static constexpr int WI = (WB + 1023) / 1024, XI = (XB + 1023) / 1024;
  static constexpr int LOADS = WI + XI;
  static constexpr int LDS = STAGES * STAGE;
  static constexpr bool F32_VIA_LDS = BM * BN * 4 <= LDS;     // else fp32 outputs are stored element-wise
  static constexpr int MAX_RES = (STAGES - 1) * kB6Tile;      // residual k-tiles must fit beside the last main one
  static_assert(WB * NW == W_HALF && XB * NW == X_HALF && WB % 512 == 0 && XB % 512 == 0, "load split");
  static_assert(OCC * LDS <= 160 * 1024 && (STAGES - 1) * LOADS < 64, "LDS, vmcnt range");
  static_assert(BM * BN * 2 <= LDS && BN * 2 / 16 >= 16, "bf16 output tile in LDS");
};

__device__ __forceinline__ v16f mfma_bf6(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 3, 3, 0, 127, 0, 127);
}

// One lane fragment from LDS: 32 six-bit fields in the low six dwords.
__device__ __forceinline__ v8i ld_frag(const uint8_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  const uint2 v = *reinterpret_cast<const uint2*>(p + 8);
  const uint2 w = *reinterpret_cast<const uint2*>(p + 16);
  return v8i{static_cast<int>(u.x), static_cast<int>(u.y), static_cast<int>(v.x), static_cast<int>(v.y),
             static_cast<int>(w.x), static_cast<int>(w.y), 0, 0};
}

// The layout pads rows to 128 only: a launch needs BN | Np and BM | Mp (the
// host picks the shape accordingly), so every load stays inside the buffers.
template <int TN, int TM, int WNW, int WMW, int STAGES, int OCC>
__global__ __launch_bounds__(64 * WNW * WMW, OCC) void serq_bf6_tile_kernel(LinearArgs a, int n_tiles) {
  using C = B6Cfg<TN, TM, WNW, WMW, STAGES, OCC>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int wn = wv / WMW, wm = wv % WMW;
  const int l32 = lane & 31, h = lane >> 5;
  int tile_n, tile_m;
  tile_coords(blockIdx.x, gridDim.x, n_tiles, tile_n, tile_m);
  const int n0 = __builtin_amdgcn_readfirstlane(tile_n * C::BN);
  const int m0 = __builtin_amdgcn_readfirstlane(tile_m * C::BM);
  const int rbn = (a.N + kB6Tile - 1) / kB6Tile * (kB6Tile / 32);   // 32-row blocks per k-tile
  const int rbm = (a.M + kB6Tile - 1) / kB6Tile * (kB6Tile / 32);
  const int nk = (a.K + kB6Tile - 1) / kB6Tile;
  const int ntot = nk + (a.r + kB6Tile - 1) / kB6Tile;
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const uint8_t* const W6 = a.Wq;
  const uint8_t* const R6 = a.Rq;
  const uint8_t* const X6 = a.Xq;

  // k-tile t (main for t < nk, else residual t - nk) into buffer t % STAGES.
  // Past the last k-tile the loads repeat the last one into a buffer that is
  // never read again, so every wave issues the same loads per k-tile and the
  // wait counts below hold without branches.
  auto issue = [&](int t) {
    const int tl = min(t, ntot - 1);
    const int kt = tl < nk ? tl : tl - nk;
    const uint8_t* wsrc = (tl < nk ? W6 : R6) + (static_cast<size_t>(kt) * rbn + n0 / 32) * kB6Block + wv * C::WB;
    const uint8_t* xsrc = X6 + (static_cast<size_t>(kt) * rbm + m0 / 32) * kB6Block + wv * C::XB;
    const uint32_t dst = lds_base + (t % STAGES) * C::STAGE;
#pragma unroll
    for (int c = 0; c < C::WI; ++c) {
      if (C::WB - 1024 * c >= 1024 || lane < 32)
        dma16(wsrc + c * 1024, 16 * lane, dst + wv * C::WB + c * 1024);
    }
#pragma unroll
    for (int c = 0; c < C::XI; ++c) {
      if (C::XB - 1024 * c >= 1024 || lane < 32)
        dma16(xsrc + c * 1024, 16 * lane, dst + C::W_HALF + wv * C::XB + c * 1024);
    }
  };
  // One MFMA step (64 codes) of a k-tile: the wave's TN weight and TM
  // activation fragments, then its TN x TM MFMAs.
  auto read = [&](int buf, int st, v8i (&wf)[TN], v8i (&xf)[TM]) {
    const uint8_t* wb = lds + buf * C::STAGE + wn * TN * kB6Block + st * kB6Step + lane * kB6Frag;
    const uint8_t* xb = lds + buf * C::STAGE + C::W_HALF + wm * TM * kB6Block + st * kB6Step + lane * kB6Frag;
#pragma unroll
    for (int i = 0; i < TN; ++i) wf[i] = ld_frag(wb + i * kB6Block);
#pragma unroll
    for (int j = 0; j < TM; ++j) xf[j] = ld_frag(xb + j * kB6Block);
  };
  auto mm = [&](const v8i (&wf)[TN], const v8i (&xf)[TM], v16f (&acc)[TN][TM]) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = mfma_bf6(wf[i], xf[j], acc[i][j]);
  };

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Every buffer starts loading; step 0 of k-tile 0 goes into registers.
#pragma unroll
  for (int p = 0; p < STAGES; ++p) issue(p);
  wait_vmcnt<(STAGES - 1) * C::LOADS>();
  lds_barrier();
  v8i w0[TN], x0[TM], w1[TN], x1[TM];
  read(0, 0, w0, x0);
  // Main k-tile t: step 1's fragments are read while step 0's MFMAs run;
  // then (this wave's k-tile t + 1 loads done, one barrier) k-tile t + 1 is
  // published and buffer t, fully read by every wave, takes k-tile
  // t + STAGES; step 0 of k-tile t + 1 is read while step 1's MFMAs run.
  // The MFMAs are pure values that the compiler would otherwise move past
  // the barrier: empty asm statements that take the accumulators (after step
  // 0) and step 1's fragments (after the barrier) pin them in program order,
  // so the matrix core has step 0's work while the wave waits.
  auto pin = [&](v16f (&ac)[TN][TM]) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) asm volatile("" : "+v"(ac[i][j]));
  };
  auto pin_frags = [&](v8i (&wf)[TN], v8i (&xf)[TM]) {
#pragma unroll
    for (int i = 0; i < TN; ++i) asm volatile("" : "+v"(wf[i]));
#pragma unroll
    for (int j = 0; j < TM; ++j) asm volatile("" : "+v"(xf[j]));
  };
  for (int t = 0; t < nk - 1; ++t) {
    read(t % STAGES, 1, w1, x1);
    mm(w0, x0, acc);
    pin(acc);
    wait_vmcnt<(STAGES - 2) * C::LOADS>();
    lds_barrier();
    issue(t + STAGES);
    pin_frags(w1, x1);
    read((t + 1) % STAGES, 0, w0, x0);
    mm(w1, x1, acc);
  }
  read((nk - 1) % STAGES, 1, w1, x1);
  mm(w0, x0, acc);
  mm(w1, x1, acc);
  // The residual k-tiles (at most STAGES - 1, the host checks, in buffers
  // the last main k-tile does not use) are complete and published.
  wait_vmcnt<0>();
  lds_barrier();

  // The accumulators are exact integers: serq_linear's epilogue on them,
  // one weight block row at a time: its blocks' residual MFMAs into TM
  // temporaries (independent chains), then
  //   y = sx (sw acc_main + sr acc_res)
  // in fp32 in place of the main accumulator (already the fp32 value of the
  // integer sum), or element-wise stores (with the exact sums for tests, or
  // fp32 outputs too large for LDS).
  const int nw = n0 + wn * 32 * TN, mw = m0 + wm * 32 * TM;
  const int nr = ntot - nk;
  const bool direct = a.dbg_main != nullptr || (!a.y_bf16 && !C::F32_VIA_LDS);
  float sxm[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) sxm[j] = a.sx[min(mw + 32 * j + l32, a.M - 1)];
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    v16f res[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) res[j][e] = 0.0f;
    for (int q = 0; q < nr; ++q) {
      const uint8_t* bp = lds + ((nk + q) % STAGES) * C::STAGE + lane * kB6Frag;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const v8i wf = ld_frag(bp + (wn * TN + i) * kB6Block + st * kB6Step);
#pragma unroll
        for (int j = 0; j < TM; ++j)
          res[j] = mfma_bf6(wf, ld_frag(bp + C::W_HALF + (wm * TM + j) * kB6Block + st * kB6Step), res[j]);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = nw + 32 * i + 8 * q + 4 * h;
      float wv4[4], rv4[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int nc = min(n + c, a.N - 1);
        wv4[c] = a.sw[nc];
        rv4[c] = nr > 0 ? a.sr[nc] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        if (direct) {
          v4i am, ar;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            am[c] = static_cast<int>(acc[i][j][4 * q + c]);
            ar[c] = static_cast<int>(res[j][4 * q + c]);
          }
          store4<0>(a, am, ar, mw + 32 * j + l32, n, sxm[j], make_float4(wv4[0], wv4[1], wv4[2], wv4[3]),
                    make_float4(rv4[0], rv4[1], rv4[2], rv4[3]));
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[i][j][4 * q + c] =
                sxm[j] * __builtin_fmaf(rv4[c], res[j][4 * q + c], wv4[c] * acc[i][j][4 * q + c]);
        }
      }
    }
  }
  if (direct) return;
  // Output tile into LDS (the stages are free once every wave is here), row =
  // token, 16-byte chunks swizzled as in the integer tile kernel; then 16-byte
  // stores along the rows of Y.
  lds_barrier();
  const bool bf = a.y_bf16;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int row = wm * 32 * TM + 32 * j + l32;
    if (bf) {
      uint8_t* rp = lds + row * (C::BN * 2);
      const int hs = (h ^ half_swap(row)) * 8;
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = (wn * 32 * TN + 32 * i) / 8 + q;
          const uint2 o = make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                     pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
          *reinterpret_cast<uint2*>(rp + 16 * (c ^ (row & 15)) + hs) = o;
        }
    } else if constexpr (C::F32_VIA_LDS) {
      uint8_t* rp = lds + row * (C::BN * 4);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = (wn * 32 * TN + 32 * i + 8 * q + 4 * h) / 4;
          *reinterpret_cast<float4*>(rp + 16 * (c ^ (row & 15))) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
    }
  }
  __syncthreads();
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
  if (bf) {
    copy_out(std::integral_constant<int, 2>{});
  } else if constexpr (C::F32_VIA_LDS) {
    copy_out(std::integral_constant<int, 4>{});
  }
}

// E3M2 pattern of a stored nibble (4-bit two's complement code): byte c of
// the first constant for codes 0..7, of the second for nibbles 8..15 (codes
// -8..-1).
__device__ __forceinline__ uint64_t bf6_of_nibble(uint32_t nib) {
  constexpr uint64_t kPos = 0x1716151412100C00ull;
  constexpr uint64_t kNeg = 0x2C30323435363738ull;
  return (((nib & 8u) ? kNeg : kPos) >> (8 * (nib & 7u))) & 0x3Full;
}

// serq_act_bf6: lane f writes fragment f of the bf6 tile layout (32 codes of
// one row, zero past the M x K codes).
__global__ __launch_bounds__(256) void serq_act_bf6_kernel(const uint8_t* Xq, int M, int K, uint8_t* X6, int rbm,
                                                           int nfrag) {
  const int f = static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x);
  if (f >= nfrag) return;
  const int l = f & 63, s = (f >> 6) & 1, blk = f >> 7;
  const int rb = blk % rbm, kt = blk / rbm;
  const int row = rb * 32 + (l & 31);
  const int k0 = kt * kB6Tile + 64 * s + 32 * (l >> 5);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (row < M && k0 < K) {
    const uint8_t* src = Xq + static_cast<size_t>(row) * (K / 2) + k0 / 2;
    if ((K & 31) == 0) {
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      w[0] = v.x;
      w[1] = v.y;
      w[2] = v.z;
      w[3] = v.w;
    } else {
      for (int b = 0; b < 16 && k0 + 2 * b < K; ++b) w[b >> 2] |= static_cast<uint32_t>(src[b]) << (8 * (b & 3));
    }
  }
  uint64_t o[3] = {0ull, 0ull, 0ull};
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const uint64_t p = bf6_of_nibble((w[c >> 3] >> (4 * (c & 7))) & 15u);
    const int bit = 6 * c;
    o[bit >> 6] |= p << (bit & 63);
    if ((bit & 63) > 58) o[(bit >> 6) + 1] |= p >> (64 - (bit & 63));
  }
  uint2* dst = reinterpret_cast<uint2*>(X6 + static_cast<size_t>(f) * kB6Frag);
#pragma unroll
  for (int q = 0; q < 3; ++q) dst[q] = make_uint2(static_cast<uint32_t>(o[q]), static_cast<uint32_t>(o[q] >> 32));
}

}  // namespace

LinearPlan plan_linear(int M, int K, int N, int r, int a_bits) {
  // The fast kernels address rows with 32-bit byte offsets.
  const bool small = static_cast<uint64_t>(N) * (K / 2) < (1ull << 32) &&
                     static_cast<uint64_t>(M) * K * a_bits / 8 < (1ull << 32);
  const bool fast = (K % 32 == 0) && (r % 8 == 0) && r <= kMaxResidual && small;
  if (!fast) return {LinearKernel::kGeneric, 0, 0, 0, 1, "generic"};
  // A few tokens of W4A4 whose activation rows fit in LDS: int4 dot products.
  if (a_bits == 4 && M <= kGemvMaxTokens && static_cast<long>(M) * (K / 2) <= kGemvMaxX)
    return {LinearKernel::kGemv, 0, 0, 0, 1, "gemv"};
  // The MFMA kernels sum the widened codes, 256 (W4A4) or 16 (W4A8) times the
  // true products: exact in int32 while |acc| < 2^23, i.e. for K < 2^17.
  if (K >= kWidenMaxK) return {LinearKernel::kGeneric, 0, 0, 0, 1, "generic"};
  // Up to 32 tokens: the skinny kernel, unless its K split would need more
  // partial-sum scratch than the library holds (then a tile kernel).
  if (M <= 32) {
    LinearArgs s{};
    s.M = M;
    s.K = K;
    s.N = N;
    s.r = r;
    s.a_bits = a_bits;
    const SkinnySplit sp = M <= 16 ? (a_bits == 4 ? plan_skinny<1, 4>(s) : plan_skinny<1, 8>(s))
                                   : (a_bits == 4 ? plan_skinny<2, 4>(s) : plan_skinny<2, 8>(s));
    if (sp.G > 0) {
      if (M <= 16)
        return {LinearKernel::kDecode16, 0, 0, 0, 1, sp.KS > 1 ? "decode16_ksplit" : "decode16"};
      return {LinearKernel::kDecode32, 0, 0, 0, 1, sp.KS > 1 ? "decode32_ksplit" : "decode32"};
    }
  }
  // Macro tiles, two four-wave workgroups per CU: the two run independently,
  // so one's barrier and load waits are covered by the other's MFMAs. (One
  // eight-wave 256 x 128 workgroup per CU, lockstep at every k-tile barrier,
  // measured 12-20 % slower on the LLaMA shapes.) The largest tile that still
  // gives every CU a workgroup; smaller tiles keep more k-tiles in flight.
  auto tiles = [&](int bm, int bn) { return static_cast<long>((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  // W4A4: 256 x 256 tiles (one four-wave workgroup per CU, 4 x 4 blocks per
  // wave: half the widening per MFMA) where their rounds of 256 tiles take
  // less time than the rounds of 512 128 x 128 tiles: a round of the large
  // tiles does twice the work of one of the small ones, measured at 0.93-0.95
  // of the time on the LLaMA prefill shapes. Padding and a partial last
  // round count as full ones.
  const long rounds256 = (tiles(256, 256) + kCUs - 1) / kCUs;
  const long rounds128 = (tiles(128, 128) + 2 * kCUs - 1) / (2 * kCUs);
  if (a_bits == 4 && M > 128 && rounds256 * 19 < rounds128 * 10)
    return {LinearKernel::kTile, 4, 4, 2, 1, "tile256x256"};
  // Exactly one 128 x 128 tile per CU and K of 64 k-tiles or more (W4A4):
  // the two-k-group tile below, whose eight waves share each CU's one tile
  // (1.03x on 14336 x 4096 at 1024 tokens, 1.07x on 28672 x 8192 at 512;
  // even with K = 4096).
  const bool one_tile_per_cu = a_bits == 4 && tiles(128, 128) == kCUs && K >= 64 * kKTileCodes;
  if (M > 64 && tiles(128, 128) >= kCUs && !one_tile_per_cu)
    return {LinearKernel::kTile, 2, 2, 2, 1, "tile128x128"};
  // Three quarters of the CUs or more with one 128 x 128 tile each: two
  // k-groups of four waves per tile, one eight-wave workgroup per CU
  // (1.1-1.2x on 4096 x 28672, 8192 x 28672 at 65-128 tokens and on
  // 4096 x 4096 at 768; with half the CUs it lost to the 64-row tiles).
  if (M > 64 && tiles(128, 128) >= 3 * kCUs / 4) return {LinearKernel::kTile, 2, 2, 2, 2, "tile128x128k2"};
  // W4A4 from 256 tokens whose 64 x 64 tiles are one round of two per CU:
  // those tiles with two k-groups (below) rather than 64 x 128 tiles
  // (1.06x on 4096 x 4096 and 1.15x on 14336 x 4096 at 512 tokens, 1.09x
  // on 28672 x 8192 at 256).
  const bool k2_round = a_bits == 4 && M >= 256 && K >= 8 * kKTileCodes && tiles(64, 64) <= 2 * kCUs;
  if (tiles(64, 128) >= kCUs && !k2_round) return {LinearKernel::kTile, 2, 1, 2, 1, "tile64x128"};
  // When 64 x 64 tiles would leave half the CUs idle, 32 x 64 tiles whose
  // eight waves form four k-groups (each a k-tile of every four-k-tile
  // stage): every CU gets work and all four SIMDs of a CU share one tile's
  // k-loop, at twice the weight traffic into LDS (measured 1.1x faster than
  // 64 x 64 at 40-128 tokens of 4096 x 4096, 1.25x on 14336 x 4096; four
  // k-groups beat one two-wave group per tile by the same margins). Two
  // k-groups of 64 x 64 tiles measured slower than one wherever 64 x 64
  // tiles fill the CUs (one eight-wave workgroup per CU against two
  // four-wave ones).
  if (tiles(64, 64) <= kCUs / 2) return {LinearKernel::kTile, 1, 1, 1, 4, "tile32x64k4"};
  // Up to one 64 x 64 tile per CU and K of 64 k-tiles or more: two waves of
  // 32 x 64 per k-group, four k-groups (1.12x on 14336 x 4096 at 192-256
  // tokens; with K = 4096 its eight four-k-tile stages left it even or a
  // few % behind the single group).
  if (tiles(64, 64) <= kCUs && K >= 64 * kKTileCodes)
    return {LinearKernel::kTile, 1, 2, 1, 4, "tile64x64k4"};
  // Two k-groups of two 32 x 64 waves (each wave 1 x 2 blocks: 9 VALU per
  // MFMA against 12 for single blocks, the four waves splitting the
  // epilogue): 0.87-0.89x the time of four single-block waves on 4096 x 4096
  // at 160-256 tokens and on 8192 x 4096 at 256, 0.94x at 320 tiles; with
  // fewer than eight k-tiles the group reduction costs more than it saves.
  if (a_bits == 4 && K >= 8 * kKTileCodes) return {LinearKernel::kTile, 1, 2, 1, 2, "tile64x64k2"};
  return {LinearKernel::kTile, 1, 1, 2, 1, "tile64x64"};
}

hipError_t launch_linear(const LinearArgs& a, const LinearPlan& p, hipStream_t st) {
  switch (p.kind) {
    case LinearKernel::kGemv:
      switch (a.M) {
        case 1: return launch_gemv<1>(a, st);
        case 2: return launch_gemv<2>(a, st);
        default: return launch_gemv<3>(a, st);
      }
    case LinearKernel::kDecode16:
      return a.a_bits == 4 ? launch_skinny<1, 4>(a, st) : launch_skinny<1, 8>(a, st);
    case LinearKernel::kDecode32:
      return a.a_bits == 4 ? launch_skinny<2, 4>(a, st) : launch_skinny<2, 8>(a, st);
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

hipError_t launch_act_bf6(const void* Xq, int M, int K, void* X6, hipStream_t st) {
  const int rbm = (M + kB6Tile - 1) / kB6Tile * (kB6Tile / 32);
  const long long nfrag = static_cast<long long>((K + kB6Tile - 1) / kB6Tile) * rbm * 128;
  if (nfrag > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const int nf = static_cast<int>(nfrag);
  serq_act_bf6_kernel<<<dim3((nf + 255) / 256), dim3(256), 0, st>>>(static_cast<const uint8_t*>(Xq), M, K,
                                                                   static_cast<uint8_t*>(X6), rbm, nf);
  return hipGetLastError();
}

namespace {

template <int TN, int TM, int WNW, int WMW, int STAGES, int OCC>
hipError_t launch_bf6_tile(const LinearArgs& a, hipStream_t st) {
  using C = B6Cfg<TN, TM, WNW, WMW, STAGES, OCC>;
  static std::atomic<uint64_t> lds_set{0};
  auto* fn = &serq_bf6_tile_kernel<TN, TM, WNW, WMW, STAGES, OCC>;
  hipError_t e = ensure_max_lds(reinterpret_cast<const void*>(fn), C::LDS, lds_set);
  if (e != hipSuccess) return e;
  const int n_tiles = (a.N + C::BN - 1) / C::BN;
  const int m_tiles = (a.M + C::BM - 1) / C::BM;
  if (static_cast<long long>(n_tiles) * m_tiles > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  fn<<<dim3(n_tiles * m_tiles), dim3(C::NT), C::LDS, st>>>(a, n_tiles);
  return hipGetLastError();
}

}  // namespace

// Tiles: 256 x 256 (eight waves of 4 x 2 blocks, one workgroup per CU:
// half the L2->LDS bytes per output of 128 x 128 and twice the MFMA work per
// barrier) when the padded sizes split into them and they give every CU a
// tile; else 128 x 128, two workgroups per CU (a 256 x 128 tile of eight
// 2 x 2-block waves, one workgroup per CU, measured 5-10 % slower than it on
// q_proj at 2048 tokens: with one workgroup per CU nothing overlaps the
// prologue and the epilogue). The layout pads rows to 128 only, so a 256 side
// needs the padded size to be a multiple of 256.
int bf6_tile_kind(int M, int N, int r) {
  const int mp = (M + kB6Tile - 1) / kB6Tile * kB6Tile, np = (N + kB6Tile - 1) / kB6Tile * kB6Tile;
  if (mp % 256 == 0 && np % 256 == 0 && static_cast<long>(mp / 256) * (np / 256) >= kCUs &&
      r <= B6Cfg<4, 2, 2, 4, 3, 1>::MAX_RES)
    return 2;
  return 0;
}

hipError_t launch_linear_bf6(const LinearArgs& a, hipStream_t st) {
  if (bf6_tile_kind(a.M, a.N, a.r) == 2) return launch_bf6_tile<4, 2, 2, 4, 3, 1>(a, st);
  return launch_bf6_tile<2, 2, 2, 2, 3, 2>(a, st);
}

}  // namespace serq

// Offline SERQ calibration and output-channel permutation (host code).
//
// Calibration follows the pages' three offline steps (papernotes.org ICLR
// 2026 notes on SERQ, 方法详解 / 整体框架 and 关键设计 1-3):
//   1. static activation flattening: a SmoothQuant-style per-channel factor
//      s_j folded into the weight rows, W~ = diag(s) W (关键设计 1);
//   2. saliency: rows ranked by their scale, permuted in descending order,
//      W^ = P W~ = [W~_s; W~_r]; the single compensator R = W~_s - Q(W~_s)
//      on the first r rows, itself quantized (关键设计 2, 核心 idea);
//   3. the permutation is merged into the stored weights; a later layer's
//      order can be pushed into this layer's output channels (关键设计 3).
//
// Every floating-point step is one IEEE binary32 operation with
// round-to-nearest-even (the library is built with -ffp-contract=off), so the
// results are reproducible bit for bit. Output columns are independent once
// s and P are known, so the column range is split over host threads; the
// result does not depend on the thread count.

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

#include "serq.h"

namespace {

inline float bf16_bits_to_float(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

struct WeightView {
  const void* p;
  serq_dtype dt;
  int N;
  inline float at(int row, int col) const {
    size_t idx = static_cast<size_t>(row) * N + col;
    if (dt == SERQ_F32) return static_cast<const float*>(p)[idx];
    return bf16_bits_to_float(static_cast<const uint16_t*>(p)[idx]);
  }
};

// Symmetric quantizer of one group with absolute maximum m.
struct Quantizer {
  float scale;
  float inv;
  bool zero;
  Quantizer(float m, float qmax) {
    inv = qmax / m;
    zero = !(inv <= FLT_MAX);  // +inf: m == 0 or too small to invert
    scale = zero ? 0.0f : m / qmax;
    if (zero) inv = 0.0f;
  }
  inline int code(float v, int lo, int hi) const {
    if (zero) return 0;
    float t = v * inv;
    float q = std::nearbyint(t);  // round half to even (default rounding mode)
    if (q < static_cast<float>(lo)) q = static_cast<float>(lo);
    if (q > static_cast<float>(hi)) q = static_cast<float>(hi);
    return static_cast<int>(q);
  }
};

inline uint8_t pack2(int c0, int c1) {
  return static_cast<uint8_t>((c0 & 0xF) | ((c1 & 0xF) << 4));
}

int worker_count(int N) {
  unsigned hc = std::thread::hardware_concurrency();
  int t = hc ? static_cast<int>(hc) : 1;
  t = std::min(t, 16);
  t = std::min(t, std::max(1, N / 64));
  return std::max(1, t);
}

// Quantize output columns [n0, n1): fills Wq, sw, Rq, sr for them.
void calibrate_columns(const WeightView& W, int K, int r, const float* s, const int32_t* perm,
                       int n0, int n1, uint8_t* Wq, float* sw, uint8_t* Rq, float* sr) {
  const int nb = n1 - n0;
  if (nb <= 0) return;
  // column maxima of the folded weight (order independent)
  std::vector<float> cmax(nb, 0.0f);
  for (int j = 0; j < K; ++j) {
    const float sj = s[j];
    for (int c = 0; c < nb; ++c) {
      float v = sj * W.at(j, n0 + c);
      cmax[c] = std::max(cmax[c], std::fabs(v));
    }
  }
  std::vector<Quantizer> qw;
  qw.reserve(nb);
  for (int c = 0; c < nb; ++c) {
    qw.emplace_back(cmax[c], 7.0f);
    sw[n0 + c] = qw[c].scale;
  }
  const size_t Kb = static_cast<size_t>(K) / 2;
  std::vector<float> R(static_cast<size_t>(r) * nb);
  std::vector<int> prev(nb);
  // rows in saliency order, two at a time (one packed byte per column)
  for (int i = 0; i < K; ++i) {
    const int j = perm[i];
    const float sj = s[j];
    for (int c = 0; c < nb; ++c) {
      float v = sj * W.at(j, n0 + c);
      int q = qw[c].code(v, -8, 7);
      if (i < r) {
        float deq = static_cast<float>(q) * qw[c].scale;
        R[static_cast<size_t>(i) * nb + c] = v - deq;
      }
      if (i & 1) {
        Wq[static_cast<size_t>(n0 + c) * Kb + (i >> 1)] = pack2(prev[c], q);
      } else {
        prev[c] = q;
      }
    }
  }
  if (r == 0) {
    if (sr)
      for (int c = 0; c < nb; ++c) sr[n0 + c] = 0.0f;
    return;
  }
  const size_t rb = static_cast<size_t>(SERQ_RQ_ROW_BYTES(r));
  for (int c = 0; c < nb; ++c) {
    float m = 0.0f;
    for (int i = 0; i < r; ++i) m = std::max(m, std::fabs(R[static_cast<size_t>(i) * nb + c]));
    Quantizer qr(m, 7.0f);
    sr[n0 + c] = qr.scale;
    uint8_t* row = Rq + static_cast<size_t>(n0 + c) * rb;
    std::memset(row, 0, rb);                    // zero codes in the padding
    for (int i = 0; i < r; i += 2) {
      int c0 = qr.code(R[static_cast<size_t>(i) * nb + c], -8, 7);
      int c1 = qr.code(R[static_cast<size_t>(i + 1) * nb + c], -8, 7);
      row[i >> 1] = pack2(c0, c1);
    }
  }
}

}  // namespace

extern "C" int serq_calibrate(const void* W, serq_dtype w_dtype, int K, int N,
                              const float* act_absmax, float alpha, int r,
                              int32_t* perm, float* s_hat_inv,
                              uint8_t* Wq, float* sw, uint8_t* Rq, float* sr) {
  if (!W || !act_absmax || !perm || !s_hat_inv || !Wq || !sw) return SERQ_EINVAL;
  if (w_dtype != SERQ_F32 && w_dtype != SERQ_BF16) return SERQ_EINVAL;
  if (K <= 0 || N <= 0 || (K & 1) || (r & 1) || r < 0 || r > K) return SERQ_EINVAL;
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return SERQ_EINVAL;
  if (r > 0 && (!Rq || !sr)) return SERQ_EINVAL;

  const WeightView wv{W, w_dtype, N};

  // 1. smoothing factors from the channel maxima (double, rounded once)
  std::vector<float> s(K), s_inv(K);
  for (int j = 0; j < K; ++j) {
    float wmax = 0.0f;
    for (int n = 0; n < N; ++n) wmax = std::max(wmax, std::fabs(wv.at(j, n)));
    const double a = std::max(static_cast<double>(act_absmax[j]), 1e-5);
    const double w = std::max(static_cast<double>(wmax), 1e-5);
    double sv;
    if (alpha == 0.5f) {
      sv = std::sqrt(a) / std::sqrt(w);
    } else {
      const double al = static_cast<double>(alpha);
      sv = std::pow(a, al) / std::pow(w, 1.0 - al);
    }
    s[j] = static_cast<float>(sv);
    s_inv[j] = 1.0f / s[j];
  }

  // 2. saliency order: descending s, ties keep the lower channel first
  std::vector<int32_t> idx(K);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) { return s[x] > s[y]; });
  for (int i = 0; i < K; ++i) {
    perm[i] = idx[i];
    s_hat_inv[i] = s_inv[idx[i]];
  }

  // 3. fold, permute, quantize per output column, compensator
  const int T = worker_count(N);
  const int per = (N + T - 1) / T;
  std::vector<std::thread> pool;
  for (int t = 1; t < T; ++t) {
    int n0 = t * per, n1 = std::min(N, n0 + per);
    if (n0 >= n1) break;
    pool.emplace_back(calibrate_columns, std::cref(wv), K, r, s.data(), perm, n0, n1, Wq, sw, Rq, sr);
  }
  calibrate_columns(wv, K, r, s.data(), perm, 0, std::min(N, per), Wq, sw, Rq, sr);
  for (auto& th : pool) th.join();
  return SERQ_OK;
}

extern "C" int serq_permute_outputs(const int32_t* perm_next, int K, int N, int r,
                                    uint8_t* Wq, float* sw, uint8_t* Rq, float* sr) {
  if (!perm_next || !Wq || !sw) return SERQ_EINVAL;
  if (N <= 0 || K <= 0 || (K & 1) || (r & 1) || r < 0 || r > K) return SERQ_EINVAL;
  if (r > 0 && (!Rq || !sr)) return SERQ_EINVAL;
  std::vector<char> seen(N, 0);
  for (int i = 0; i < N; ++i) {
    int p = perm_next[i];
    if (p < 0 || p >= N || seen[p]) return SERQ_EINVAL;
    seen[p] = 1;
  }
  const size_t Kb = static_cast<size_t>(K) / 2, rb = static_cast<size_t>(SERQ_RQ_ROW_BYTES(r));
  std::vector<uint8_t> wtmp(static_cast<size_t>(N) * Kb);
  std::vector<float> ftmp(N);
  for (int i = 0; i < N; ++i)
    std::memcpy(&wtmp[static_cast<size_t>(i) * Kb], Wq + static_cast<size_t>(perm_next[i]) * Kb, Kb);
  std::memcpy(Wq, wtmp.data(), wtmp.size());
  for (int i = 0; i < N; ++i) ftmp[i] = sw[perm_next[i]];
  std::memcpy(sw, ftmp.data(), sizeof(float) * N);
  if (r > 0) {
    std::vector<uint8_t> rtmp(static_cast<size_t>(N) * rb);
    for (int i = 0; i < N; ++i)
      std::memcpy(&rtmp[static_cast<size_t>(i) * rb], Rq + static_cast<size_t>(perm_next[i]) * rb, rb);
    std::memcpy(Rq, rtmp.data(), rtmp.size());
    for (int i = 0; i < N; ++i) ftmp[i] = sr[perm_next[i]];
    std::memcpy(sr, ftmp.data(), sizeof(float) * N);
  }
  return SERQ_OK;
}

// bf6 tile layout of a packed int4 matrix (the layout and the E3M2 patterns
// are stated with serq_prepack_bf6 in serq.h): each 24-byte fragment holds
// 32 codes of one row as six-bit fields, low field first.
namespace {

constexpr int kBf6Tile = 128;

// E3M2 pattern of a 4-bit two's complement code (the nibble as stored).
inline uint32_t bf6_pattern(uint32_t nib) {
  static const uint8_t kMag[9] = {0x00, 0x0C, 0x10, 0x12, 0x14, 0x15, 0x16, 0x17, 0x18};   // |v| = 0..8
  const int v = nib < 8 ? static_cast<int>(nib) : static_cast<int>(nib) - 16;
  return v < 0 ? (0x20u | kMag[-v]) : kMag[v];
}

}  // namespace

extern "C" int64_t serq_bf6_bytes(int rows, int k) {
  if (rows < 0 || k < 0) return -1;
  return static_cast<int64_t>(SERQ_BF6_BYTES(rows, k));
}

extern "C" int serq_prepack_bf6(const uint8_t* codes, int rows, int k, int pitch, uint8_t* out) {
  if (!codes || !out) return SERQ_EINVAL;
  if (rows <= 0 || k <= 0 || (k & 1) || pitch <= 0 || k > 2 * pitch) return SERQ_EINVAL;
  const int rp = (rows + kBf6Tile - 1) / kBf6Tile * kBf6Tile;
  const int nkt = (k + kBf6Tile - 1) / kBf6Tile, nrb = rp / 32;
  for (int kt = 0; kt < nkt; ++kt)
    for (int rb = 0; rb < nrb; ++rb)
      for (int s = 0; s < 2; ++s)
        for (int l = 0; l < 64; ++l) {
          const int row = rb * 32 + l % 32;
          const int k0 = kt * kBf6Tile + 64 * s + 32 * (l / 32);
          uint64_t word[3] = {0, 0, 0};       // the fragment as a little-endian 192-bit integer
          for (int f = 0; f < 32 && row < rows; ++f) {
            const int kk = k0 + f;
            if (kk >= k) break;
            const uint8_t byte = codes[static_cast<size_t>(row) * pitch + kk / 2];
            const uint64_t pat = bf6_pattern((kk & 1) ? (byte >> 4) : (byte & 15u));
            const int bit = 6 * f;
            word[bit / 64] |= pat << (bit % 64);
            if (bit % 64 > 58) word[bit / 64 + 1] |= pat >> (64 - bit % 64);
          }
          uint8_t frag[24];
          for (int b = 0; b < 24; ++b) frag[b] = static_cast<uint8_t>(word[b / 8] >> (8 * (b % 8)));
          const size_t off = ((static_cast<size_t>(kt) * nrb + rb) * 2 + s) * 1536 + static_cast<size_t>(l) * 24;
          std::memcpy(out + off, frag, sizeof frag);
        }
  return SERQ_OK;
}

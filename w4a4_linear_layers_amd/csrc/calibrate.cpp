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
#include <atomic>
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

// s_j = fl32(max(a_j, 1e-5)^alpha / max(w_j, 1e-5)^(1 - alpha)) in double
// (exactly sqrt(a) / sqrt(w) for alpha = 1/2), s_inv_j = fl32(1 / s_j).
void smoothing_factors(const WeightView& wv, int K, int N, const float* act_absmax, float alpha, float* s,
                       float* s_inv) {
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
  smoothing_factors(wv, K, N, act_absmax, alpha, s.data(), s_inv.data());

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

// ---------------------------------------------------------------------------
// SERQ with GPTQ weight codes (serq_calibrate_gptq). GPTQ (Frantar,
// Ashkboos, Hoefler and Alistarh, ICLR 2023) quantizes the rows of the
// folded, permuted weight one at a time in the saliency order and moves each
// row's quantization error onto the rows not yet quantized, weighted by the
// upper Cholesky factor U of H^-1, H = X^T X over the layer's calibration
// inputs (gist.science/de "Technische Zusammenfassung" 3: SERQ works with
// RTN and with GPTQ). The r salient rows come first and their error is left
// to the compensator R (it would otherwise be corrected twice), so their
// codes, R, Q(R) and every scale are serq_calibrate's; GPTQ re-quantizes
// rows r..K-1 on the same per-column grid.
//
// All of it is fp64 with every element updated by the same sequence of
// single operations in the same order as the reference statement of the
// algorithm (compiled with -ffp-contract=off: no fused multiply-adds), so the
// codes do not depend on the thread count:
//   H[i][j]  = sum over t in order of x^[t][i] x^[t][j], then damp * mean(diag)
//              on the diagonal (all-zero H: the identity);
//   V upper with H = V V^T, eliminating from the last index:
//              V[k][k] = sqrt(A[k][k]), V[i][k] = A[i][k] / V[k][k],
//              A[i][j] -= V[i][k] V[j][k] (i <= j < k);
//   U = V^-1 by back substitution: row k divided by V[k][k], then
//              B[i][c] -= V[i][k] B[k][c] (i < k <= c);
//   per row i: codes of fl32(w_i), e = (w_i - deq) / U[i][i] (i >= r),
//              w_j -= U[i][j] e for j > i.
// ---------------------------------------------------------------------------

namespace {

// Spinning barrier for the factorizations' per-step synchronization.
class StepBarrier {
 public:
  explicit StepBarrier(int n) : n_(n) {}
  void arrive_and_wait() {
    const int gen = gen_.load(std::memory_order_acquire);
    if (count_.fetch_add(1, std::memory_order_acq_rel) + 1 == n_) {
      count_.store(0, std::memory_order_relaxed);
      gen_.fetch_add(1, std::memory_order_acq_rel);
    } else {
      while (gen_.load(std::memory_order_acquire) == gen) std::this_thread::yield();
    }
  }

 private:
  const int n_;
  std::atomic<int> count_{0};
  std::atomic<int> gen_{0};
};

// Run f(t, T) on T threads (t = 0 on the calling thread).
template <typename Fn>
void run_threads(int T, Fn f) {
  std::vector<std::thread> pool;
  for (int t = 1; t < T; ++t) pool.emplace_back(f, t, T);
  f(0, T);
  for (auto& th : pool) th.join();
}

int gptq_threads(int work) {
  unsigned hc = std::thread::hardware_concurrency();
  int t = hc ? static_cast<int>(hc) : 1;
  return std::max(1, std::min({t, 16, work}));
}

}  // namespace

extern "C" int serq_calibrate_gptq(const void* W, serq_dtype w_dtype, int K, int N,
                                   const float* act_absmax, float alpha, int r,
                                   const void* X_cal, serq_dtype x_dtype, int T, float damp,
                                   int32_t* perm, float* s_hat_inv,
                                   uint8_t* Wq, float* sw, uint8_t* Rq, float* sr) {
  if (!X_cal || T <= 0) return SERQ_EINVAL;
  if (x_dtype != SERQ_F32 && x_dtype != SERQ_BF16) return SERQ_EINVAL;
  if (!(damp >= 0.0f && damp <= FLT_MAX)) return SERQ_EINVAL;
  const int st = serq_calibrate(W, w_dtype, K, N, act_absmax, alpha, r, perm, s_hat_inv, Wq, sw, Rq, sr);
  if (st != SERQ_OK) return st;

  const WeightView wv{W, w_dtype, N};
  const WeightView xv{X_cal, x_dtype, K};
  std::vector<float> s(K), s_inv(K);
  smoothing_factors(wv, K, N, act_absmax, alpha, s.data(), s_inv.data());
  const size_t KK = static_cast<size_t>(K) * K;

  // the inputs the layer sees: flattened and permuted, x^ = fl32(x[perm] * s^-1)
  std::vector<double> xh(static_cast<size_t>(T) * K);
  for (int t = 0; t < T; ++t)
    for (int i = 0; i < K; ++i) xh[static_cast<size_t>(t) * K + i] = static_cast<double>(xv.at(t, perm[i]) * s_hat_inv[i]);

  // H, upper triangle, rows dealt cyclically (row i holds K - i entries)
  std::vector<double> A(KK, 0.0);
  const int TH = gptq_threads(K);
  run_threads(TH, [&](int tid, int nth) {
    for (int t = 0; t < T; ++t) {
      const double* x = &xh[static_cast<size_t>(t) * K];
      for (int i = tid; i < K; i += nth) {
        const double xi = x[i];
        double* row = &A[static_cast<size_t>(i) * K];
        for (int j = i; j < K; ++j) row[j] += xi * x[j];
      }
    }
  });
  double d = 0.0;
  for (int i = 0; i < K; ++i) d += A[static_cast<size_t>(i) * K + i];
  d = d / K;
  if (d == 0.0) {
    std::fill(A.begin(), A.end(), 0.0);
    for (int i = 0; i < K; ++i) A[static_cast<size_t>(i) * K + i] = 1.0;
  } else {
    const double lam = static_cast<double>(damp) * d;
    for (int i = 0; i < K; ++i) A[static_cast<size_t>(i) * K + i] += lam;
  }

  // V (upper, H = V V^T) from the last index; then U = V^-1 in B
  std::vector<double> V(KK, 0.0), B(KK, 0.0);
  for (int i = 0; i < K; ++i) B[static_cast<size_t>(i) * K + i] = 1.0;
  std::atomic<int> not_pd{0};
  {
    StepBarrier bar(TH);
    run_threads(TH, [&](int tid, int nth) {
      std::vector<double> col(K);
      for (int k = K - 1; k >= 0; --k) {
        bar.arrive_and_wait();                        // step k + 1's updates are done
        const double akk = A[static_cast<size_t>(k) * K + k];
        if (!(akk > 0.0)) {
          not_pd.store(1, std::memory_order_relaxed);
          return;                                     // every thread sees the same value
        }
        const double v = std::sqrt(akk);
        for (int i = 0; i < k; ++i) col[i] = A[static_cast<size_t>(i) * K + k] / v;
        if (tid == 0) V[static_cast<size_t>(k) * K + k] = v;
        for (int i = tid; i < k; i += nth) {
          V[static_cast<size_t>(i) * K + k] = col[i];
          double* row = &A[static_cast<size_t>(i) * K];
          const double ci = col[i];
          for (int j = i; j < k; ++j) row[j] -= ci * col[j];
        }
      }
    });
  }
  if (not_pd.load()) return SERQ_EINVAL;
  {
    StepBarrier bar(TH);
    run_threads(TH, [&](int tid, int nth) {
      std::vector<double> rowk(K);
      for (int k = K - 1; k >= 0; --k) {
        bar.arrive_and_wait();                        // row k has all its updates
        const double vkk = V[static_cast<size_t>(k) * K + k];
        const double* bk = &B[static_cast<size_t>(k) * K];
        for (int c = k; c < K; ++c) rowk[c] = bk[c] / vkk;
        bar.arrive_and_wait();                        // every thread has read row k
        if (k % nth == tid)
          for (int c = k; c < K; ++c) B[static_cast<size_t>(k) * K + c] = rowk[c];
        for (int i = tid; i < k; i += nth) {
          const double vik = V[static_cast<size_t>(i) * K + k];
          double* bi = &B[static_cast<size_t>(i) * K];
          for (int c = k; c < K; ++c) bi[c] -= vik * rowk[c];
        }
      }
    });
  }
  std::vector<double>().swap(A);
  std::vector<double>().swap(V);

  // the folded, permuted weight and its per-column grid
  std::vector<double> Wk(static_cast<size_t>(K) * N);
  std::vector<float> cmax(N, 0.0f);
  for (int i = 0; i < K; ++i) {
    const int j = perm[i];
    const float sj = s[j];
    for (int n = 0; n < N; ++n) {
      const float v = sj * wv.at(j, n);
      Wk[static_cast<size_t>(i) * N + n] = static_cast<double>(v);
      cmax[n] = std::max(cmax[n], std::fabs(v));
    }
  }
  std::vector<int8_t> codes(static_cast<size_t>(K) * N);
  const int TC = gptq_threads(std::max(1, N / 16));
  run_threads(TC, [&](int tid, int nth) {
    const int per = (N + nth - 1) / nth, n0 = tid * per, n1 = std::min(N, n0 + per);
    if (n0 >= n1) return;
    std::vector<Quantizer> qz;
    for (int n = n0; n < n1; ++n) qz.emplace_back(cmax[n], 7.0f);
    std::vector<double> err(n1 - n0);
    for (int i = 0; i < K; ++i) {
      double* wi = &Wk[static_cast<size_t>(i) * N];
      for (int n = n0; n < n1; ++n) {
        const Quantizer& q = qz[n - n0];
        const int c = q.code(static_cast<float>(wi[n]), -8, 7);
        codes[static_cast<size_t>(i) * N + n] = static_cast<int8_t>(c);
        if (i >= r) {
          const double deq = static_cast<double>(static_cast<float>(c) * q.scale);
          err[n - n0] = (wi[n] - deq) / B[static_cast<size_t>(i) * K + i];
        }
      }
      if (i < r) continue;
      const double* ui = &B[static_cast<size_t>(i) * K];
      for (int j = i + 1; j < K; ++j) {
        const double uij = ui[j];
        double* wj = &Wk[static_cast<size_t>(j) * N];
        for (int n = n0; n < n1; ++n) wj[n] -= uij * err[n - n0];
      }
    }
  });
  const size_t Kb = static_cast<size_t>(K) / 2;
  for (int n = 0; n < N; ++n)
    for (int i = 0; i < K; i += 2)
      Wq[static_cast<size_t>(n) * Kb + (i >> 1)] =
          pack2(codes[static_cast<size_t>(i) * N + n], codes[static_cast<size_t>(i + 1) * N + n]);
  return SERQ_OK;
}

// ---------------------------------------------------------------------------
// The MXFP4 layer (serq_calibrate_mx). The pages run SERQ on MXFP4 as well as
// INT4 (gist.science/de "Technische Zusammenfassung" 3 and 4); the format
// is the OCP Microscaling (MX) one: blocks of 32 elements along the
// reduction dimension share an E8M0 exponent e = floor(log2(max |v|)) - 2,
// clamped to [-127, 127] (-127 for an all-zero block), and each element is
// the FP4 E2M1 value nearest to v / 2^e, ties to the even mantissa,
// saturated at 6 (a value that rounds to zero is code 0). The scaling by
// 2^-e is exact, so the code depends only on the binary32 value of v.
// ---------------------------------------------------------------------------

namespace {

inline int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int ex = 0;
  (void)std::frexp(amax, &ex);                 // amax = m 2^ex, m in [1/2, 1)
  return std::max(-127, std::min(127, ex - 1 - 2));
}

// E2M1 code of t (|t| < 8 by construction): nearest of 0, .5, 1, 1.5, 2, 3,
// 4, 6, ties to the even mantissa (0, 1, 2, 4), saturated at 6.
inline int e2m1_code(double t) {
  const double a = std::fabs(t);
  int c;
  if (a <= 0.25) c = 0;
  else if (a < 0.75) c = 1;
  else if (a <= 1.25) c = 2;
  else if (a < 1.75) c = 3;
  else if (a <= 2.5) c = 4;
  else if (a < 3.5) c = 5;
  else if (a <= 5.0) c = 6;
  else c = 7;
  return (t < 0.0 && c != 0) ? (c | 8) : c;
}

const float kE2m1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

// One MX block of n (<= 32) values: codes into `codes`, the exponent
// returned; `deq` (optional) receives code * 2^e.
int mx_block(const float* v, int n, int* codes, float* deq) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) amax = std::max(amax, std::fabs(v[i]));
  const int e = mx_exponent(amax);
  for (int i = 0; i < n; ++i) {
    const int c = e2m1_code(std::ldexp(static_cast<double>(v[i]), -e));
    codes[i] = c;
    if (deq) {
      const double mag = std::ldexp(static_cast<double>(kE2m1[c & 7]), e);
      deq[i] = static_cast<float>((c & 8) ? -mag : mag);
    }
  }
  return e;
}

void calibrate_mx_columns(const WeightView& W, int K, int r, const float* s, const int32_t* perm, int n0, int n1,
                          uint8_t* Wq, uint8_t* Wsc, uint8_t* Rq, uint8_t* Rsc) {
  const size_t Kb = static_cast<size_t>(K) / 2, Kblk = static_cast<size_t>(K) / 32;
  const size_t rb = static_cast<size_t>(r) / 2, rblk = static_cast<size_t>(r) / 32;
  std::vector<float> col(K), deq(K), R(r);
  std::vector<int> codes(K);
  for (int n = n0; n < n1; ++n) {
    for (int i = 0; i < K; ++i) {
      const int j = perm[i];
      col[i] = s[j] * W.at(j, n);                              // W^[i, n]
    }
    for (int b = 0; b < K / 32; ++b)
      Wsc[n * Kblk + b] = static_cast<uint8_t>(mx_block(&col[32 * b], 32, &codes[32 * b], &deq[32 * b]) + 127);
    for (int i = 0; i < K; i += 2) Wq[n * Kb + i / 2] = pack2(codes[i], codes[i + 1]);
    if (r == 0) continue;
    for (int i = 0; i < r; ++i) R[i] = col[i] - deq[i];        // R = W~_s - Q(W~_s)
    for (int b = 0; b < r / 32; ++b)
      Rsc[n * rblk + b] = static_cast<uint8_t>(mx_block(&R[32 * b], 32, &codes[32 * b], nullptr) + 127);
    for (int i = 0; i < r; i += 2) Rq[n * rb + i / 2] = pack2(codes[i], codes[i + 1]);
  }
}

}  // namespace

extern "C" int serq_calibrate_mx(const void* W, serq_dtype w_dtype, int K, int N, const float* act_absmax,
                                 float alpha, int r, int32_t* perm, float* s_hat_inv, uint8_t* Wq, uint8_t* Wsc,
                                 uint8_t* Rq, uint8_t* Rsc) {
  if (!W || !act_absmax || !perm || !s_hat_inv || !Wq || !Wsc) return SERQ_EINVAL;
  if (w_dtype != SERQ_F32 && w_dtype != SERQ_BF16) return SERQ_EINVAL;
  if (K <= 0 || N <= 0 || (K % 32) || (r % 32) || r < 0 || r > K) return SERQ_EINVAL;
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return SERQ_EINVAL;
  if (r > 0 && (!Rq || !Rsc)) return SERQ_EINVAL;
  const WeightView wv{W, w_dtype, N};
  std::vector<float> s(K), s_inv(K);
  smoothing_factors(wv, K, N, act_absmax, alpha, s.data(), s_inv.data());
  std::vector<int32_t> idx(K);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) { return s[x] > s[y]; });
  for (int i = 0; i < K; ++i) {
    perm[i] = idx[i];
    s_hat_inv[i] = s_inv[idx[i]];
  }
  const int T = worker_count(N);
  const int per = (N + T - 1) / T;
  std::vector<std::thread> pool;
  for (int t = 1; t < T; ++t) {
    const int n0 = t * per, n1 = std::min(N, n0 + per);
    if (n0 >= n1) break;
    pool.emplace_back(calibrate_mx_columns, std::cref(wv), K, r, s.data(), perm, n0, n1, Wq, Wsc, Rq, Rsc);
  }
  calibrate_mx_columns(wv, K, r, s.data(), perm, 0, std::min(N, per), Wq, Wsc, Rq, Rsc);
  for (auto& th : pool) th.join();
  return SERQ_OK;
}

// C ABI entry points of libserq: host-side argument validation and dispatch
// of the online calls onto the caller's HIP stream. The offline calls
// (serq_calibrate, serq_permute_outputs) live in calibrate.cpp.

#include <hip/hip_runtime.h>

#include "serq.h"
#include "serq_internal.h"

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool valid_sizes(int M, int K, int N, int r) {
  return M >= 0 && K > 0 && N > 0 && (K % 2) == 0 && r >= 0 && r <= K && (r % 2) == 0;
}

}  // namespace

extern "C" const char* serq_strerror(int status) {
  switch (status) {
    case SERQ_OK: return "SERQ_OK";
    case SERQ_EINVAL: return "SERQ_EINVAL: invalid argument";
    case SERQ_EALIGN: return "SERQ_EALIGN: device pointer not 16-byte aligned";
    case SERQ_EUNSUPPORTED: return "SERQ_EUNSUPPORTED: unsupported request";
    case SERQ_EHIP: return "SERQ_EHIP: HIP runtime error";
    default: return "SERQ: unknown status";
  }
}

extern "C" int serq_abi_version(void) { return 300; }

extern "C" int serq_rq_row_bytes(int r) { return r < 0 ? -1 : SERQ_RQ_ROW_BYTES(r); }

extern "C" int serq_quant_act(const void* X, serq_dtype x_dtype, int M, int K,
                              const float* s_hat_inv, int a_bits, void* Xq, float* sx,
                              void* stream) {
  if (x_dtype != SERQ_F32 && x_dtype != SERQ_BF16) return SERQ_EINVAL;
  if (a_bits != 4 && a_bits != 8) return SERQ_EINVAL;
  if (M < 0 || K <= 0 || (K % 2) != 0) return SERQ_EINVAL;
  if (!s_hat_inv) return SERQ_EINVAL;
  if (!aligned16(s_hat_inv)) return SERQ_EALIGN;
  if (M == 0) return SERQ_OK;  // the M-sized buffers may then be empty (NULL)
  if (!X || !Xq || !sx) return SERQ_EINVAL;
  if (!aligned16(X) || !aligned16(Xq) || !aligned16(sx)) return SERQ_EALIGN;
  hipError_t e = serq::launch_quant_act(X, x_dtype == SERQ_BF16, M, K, s_hat_inv, a_bits, Xq, sx,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SERQ_OK : SERQ_EHIP;
}

extern "C" int serq_silu_mul_quant_act(const void* G, const void* U, int ld, serq_dtype x_dtype, int M,
                                       int K, const float* s_hat_inv, int a_bits, void* Xq, float* sx,
                                       void* stream) {
  if (x_dtype != SERQ_F32 && x_dtype != SERQ_BF16) return SERQ_EINVAL;
  if (a_bits != 4 && a_bits != 8) return SERQ_EINVAL;
  if (M < 0 || K <= 0 || (K % 2) != 0 || ld < K) return SERQ_EINVAL;
  if (!s_hat_inv) return SERQ_EINVAL;
  if (!aligned16(s_hat_inv)) return SERQ_EALIGN;
  if (M == 0) return SERQ_OK;  // the M-sized buffers may then be empty (NULL)
  if (!G || !U || !Xq || !sx) return SERQ_EINVAL;
  const uintptr_t eb = x_dtype == SERQ_BF16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(G) % eb) != 0 || (reinterpret_cast<uintptr_t>(U) % eb) != 0 ||
      !aligned16(Xq) || !aligned16(sx))
    return SERQ_EALIGN;
  hipError_t e = serq::launch_silu_mul_quant_act(G, U, ld, x_dtype == SERQ_BF16, M, K, s_hat_inv, a_bits, Xq,
                                                 sx, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SERQ_OK : SERQ_EHIP;
}

extern "C" int serq_linear(const void* Xq, const float* sx, int a_bits, const uint8_t* Wq,
                           const float* sw, const uint8_t* Rq, const float* sr, int M, int K, int N,
                           int r, void* Y, serq_dtype y_dtype, int32_t* acc_main_dbg,
                           int32_t* acc_res_dbg, void* stream) {
  if (a_bits != 4 && a_bits != 8) return SERQ_EINVAL;
  if (y_dtype != SERQ_F32 && y_dtype != SERQ_BF16) return SERQ_EINVAL;
  if (!valid_sizes(M, K, N, r)) return SERQ_EINVAL;
  if (!Wq || !sw) return SERQ_EINVAL;
  if (r > 0 && (!Rq || !sr)) return SERQ_EINVAL;
  if ((acc_main_dbg == nullptr) != (acc_res_dbg == nullptr)) return SERQ_EINVAL;
  if (!aligned16(Wq) || !aligned16(sw)) return SERQ_EALIGN;
  if (r > 0 && (!aligned16(Rq) || !aligned16(sr))) return SERQ_EALIGN;
  if (M == 0) return SERQ_OK;  // the M-sized buffers may then be empty (NULL)
  if (!Xq || !sx || !Y) return SERQ_EINVAL;
  if (!aligned16(Xq) || !aligned16(sx) || !aligned16(Y)) return SERQ_EALIGN;
  if (acc_main_dbg && (!aligned16(acc_main_dbg) || !aligned16(acc_res_dbg))) return SERQ_EALIGN;
  serq::LinearArgs a{};
  a.Xq = static_cast<const uint8_t*>(Xq);
  a.sx = sx;
  a.Wq = Wq;
  a.sw = sw;
  a.Rq = r > 0 ? Rq : nullptr;
  a.sr = r > 0 ? sr : nullptr;
  a.Y = Y;
  a.dbg_main = acc_main_dbg;
  a.dbg_res = acc_res_dbg;
  a.M = M;
  a.K = K;
  a.N = N;
  a.r = r;
  a.a_bits = a_bits;
  a.y_bf16 = y_dtype == SERQ_BF16;
  const serq::LinearPlan plan = serq::plan_linear(M, K, N, r, a_bits);
  hipError_t e = serq::launch_linear(a, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SERQ_OK : SERQ_EHIP;
}

extern "C" const char* serq_linear_kernel_name(int M, int K, int N, int r, int a_bits) {
  if ((a_bits != 4 && a_bits != 8) || !valid_sizes(M, K, N, r)) return nullptr;
  return serq::plan_linear(M, K, N, r, a_bits).name;
}

namespace {
constexpr int kBf6MaxK = 1 << 18;       // |acc| <= 64 K stays an exact fp32 integer
constexpr int kBf6MaxResidual = 256;
}  // namespace

extern "C" int serq_act_bf6(const void* Xq, int M, int K, void* X6, void* stream) {
  if (M < 0 || K <= 0 || (K % 2) != 0 || K > kBf6MaxK) return SERQ_EINVAL;
  if (M == 0) return SERQ_OK;
  if (!Xq || !X6) return SERQ_EINVAL;
  if (!aligned16(Xq) || !aligned16(X6)) return SERQ_EALIGN;
  hipError_t e = serq::launch_act_bf6(Xq, M, K, X6, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SERQ_OK : SERQ_EHIP;
}

extern "C" int serq_linear_bf6(const void* X6, const float* sx, const uint8_t* W6, const float* sw,
                               const uint8_t* R6, const float* sr, int M, int K, int N, int r, void* Y,
                               serq_dtype y_dtype, int32_t* acc_main_dbg, int32_t* acc_res_dbg,
                               void* stream) {
  if (y_dtype != SERQ_F32 && y_dtype != SERQ_BF16) return SERQ_EINVAL;
  if (!valid_sizes(M, K, N, r) || K > kBf6MaxK || r > kBf6MaxResidual) return SERQ_EINVAL;
  if (!W6 || !sw) return SERQ_EINVAL;
  if (r > 0 && (!R6 || !sr)) return SERQ_EINVAL;
  if ((acc_main_dbg == nullptr) != (acc_res_dbg == nullptr)) return SERQ_EINVAL;
  if (!aligned16(W6) || !aligned16(sw)) return SERQ_EALIGN;
  if (r > 0 && (!aligned16(R6) || !aligned16(sr))) return SERQ_EALIGN;
  if (M == 0) return SERQ_OK;
  if (!X6 || !sx || !Y) return SERQ_EINVAL;
  if (!aligned16(X6) || !aligned16(sx) || !aligned16(Y)) return SERQ_EALIGN;
  if (acc_main_dbg && (!aligned16(acc_main_dbg) || !aligned16(acc_res_dbg))) return SERQ_EALIGN;
  serq::LinearArgs a{};
  a.Xq = static_cast<const uint8_t*>(X6);
  a.sx = sx;
  a.Wq = W6;
  a.sw = sw;
  a.Rq = r > 0 ? R6 : nullptr;
  a.sr = r > 0 ? sr : nullptr;
  a.Y = Y;
  a.dbg_main = acc_main_dbg;
  a.dbg_res = acc_res_dbg;
  a.M = M;
  a.K = K;
  a.N = N;
  a.r = r;
  a.a_bits = 4;
  a.y_bf16 = y_dtype == SERQ_BF16;
  hipError_t e = serq::launch_linear_bf6(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SERQ_OK : SERQ_EHIP;
}

extern "C" const char* serq_linear_bf6_kernel_name(int M, int N, int r) {
  if (M <= 0 || N <= 0 || r < 0) return nullptr;
  return serq::bf6_tile_kind(M, N, r) == 2 ? "bf6_tile256x256" : "bf6_tile128x128";
}

extern "C" int serq_quant_act_mx(const void* X, serq_dtype x_dtype, int M, int K, const float* s_hat_inv,
                                 uint8_t* Xq, uint8_t* Xsc, void* stream) {
  if (x_dtype != SERQ_F32 && x_dtype != SERQ_BF16) return SERQ_EINVAL;
  if (M < 0 || K <= 0 || (K % 32) != 0) return SERQ_EINVAL;
  if (!s_hat_inv) return SERQ_EINVAL;
  if (!aligned16(s_hat_inv)) return SERQ_EALIGN;
  if (M == 0) return SERQ_OK;
  if (!X || !Xq || !Xsc) return SERQ_EINVAL;
  if (!aligned16(X) || !aligned16(Xq)) return SERQ_EALIGN;
  hipError_t e = serq::launch_quant_act_mx(X, x_dtype == SERQ_BF16, M, K, s_hat_inv, Xq, Xsc,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SERQ_OK : SERQ_EHIP;
}

extern "C" int serq_linear_mx(const uint8_t* Xq, const uint8_t* Xsc, const uint8_t* Wq, const uint8_t* Wsc,
                              const uint8_t* Rq, const uint8_t* Rsc, int M, int K, int N, int r, void* Y,
                              serq_dtype y_dtype, float* acc_main_dbg, float* acc_res_dbg, void* stream) {
  if (y_dtype != SERQ_F32 && y_dtype != SERQ_BF16) return SERQ_EINVAL;
  if (M < 0 || K <= 0 || N <= 0 || (K % 32) || r < 0 || r > K || (r % 32)) return SERQ_EINVAL;
  if (!Wq || !Wsc) return SERQ_EINVAL;
  if (r > 0 && (!Rq || !Rsc)) return SERQ_EINVAL;
  if ((acc_main_dbg == nullptr) != (acc_res_dbg == nullptr)) return SERQ_EINVAL;
  if (!aligned16(Wq) || (r > 0 && !aligned16(Rq))) return SERQ_EALIGN;
  if (M == 0) return SERQ_OK;
  if (!Xq || !Xsc || !Y) return SERQ_EINVAL;
  if (!aligned16(Xq) || !aligned16(Y)) return SERQ_EALIGN;
  if (acc_main_dbg && (!aligned16(acc_main_dbg) || !aligned16(acc_res_dbg))) return SERQ_EALIGN;
  serq::MxArgs a{};
  a.Xq = Xq;
  a.Xsc = Xsc;
  a.Wq = Wq;
  a.Wsc = Wsc;
  a.Rq = r > 0 ? Rq : nullptr;
  a.Rsc = r > 0 ? Rsc : nullptr;
  a.Y = Y;
  a.dbg_main = acc_main_dbg;
  a.dbg_res = acc_res_dbg;
  a.M = M;
  a.K = K;
  a.N = N;
  a.r = r;
  a.y_bf16 = y_dtype == SERQ_BF16;
  hipError_t e = serq::launch_linear_mx(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SERQ_OK : SERQ_EHIP;
}

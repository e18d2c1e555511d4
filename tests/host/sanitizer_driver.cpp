// Host-side driver for the sanitizer build of libserq's host code.
//
// Built with g++ -fsanitize=address,undefined together with calibrate.cpp
// and serq_abi.cpp (no GPU code): the device launchers are replaced by stubs
// below that only count calls, so every host path runs -- the offline calls
// on random layers with every output buffer allocated at exactly its
// documented size (AddressSanitizer reports any byte written or read past
// it), and every argument validator of the online calls with valid and
// invalid arguments. Exits non-zero on a wrong status; the sanitizers abort
// on any memory or undefined-behaviour error.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <numeric>
#include <random>
#include <vector>

#include "serq.h"
#include "serq_internal.h"

namespace serq {
static int g_launches = 0;
LinearPlan plan_linear(int, int, int, int, int) { return {LinearKernel::kGeneric, 0, 0, 0, 1, "generic"}; }
hipError_t launch_quant_act(const void*, int, int, int, const float*, int, void*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_linear(const LinearArgs&, const LinearPlan&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_silu_mul_quant_act(const void*, const void*, int, int, int, int, const float*, int, void*, float*,
                                     hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_act_bf6(const void*, int, int, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_linear_bf6(const LinearArgs&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
int bf6_tile_kind(int, int, int) { return 0; }
hipError_t launch_quant_act_mx(const void*, int, int, int, const float*, uint8_t*, uint8_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_linear_mx(const MxArgs&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
int mx_kernel_kind(int, int, int) { return 0; }
}  // namespace serq

namespace {

int g_fail = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

std::mt19937 rng(7);

std::vector<float> randn(size_t n, float sd) {
  std::normal_distribution<float> d(0.0f, sd);
  std::vector<float> v(n);
  for (auto& x : v) x = d(rng);
  return v;
}

// exactly-sized heap buffers: ASan flags any access past the end
template <typename T>
std::unique_ptr<T[]> buf(size_t n) {
  return std::unique_ptr<T[]>(new T[n ? n : 1]);
}

void offline_calls() {
  const int shapes[][3] = {{2, 1, 0}, {2, 1, 2}, {64, 40, 8}, {130, 17, 6}, {256, 33, 256}, {512, 64, 64}};
  for (const auto& sh : shapes) {
    const int K = sh[0], N = sh[1], r = sh[2];
    auto W = randn(static_cast<size_t>(K) * N, 0.02f);
    auto a = randn(K, 3.0f);
    for (auto& x : a) x = std::fabs(x);
    a[0] = 0.0f;                                       // a dead channel
    std::vector<uint16_t> Wb(W.size());
    for (size_t i = 0; i < W.size(); ++i) {
      uint32_t u;
      std::memcpy(&u, &W[i], 4);
      Wb[i] = static_cast<uint16_t>(u >> 16);
    }
    auto perm = buf<int32_t>(K);
    auto shi = buf<float>(K);
    auto Wq = buf<uint8_t>(static_cast<size_t>(N) * K / 2);
    auto sw = buf<float>(N);
    auto Rq = buf<uint8_t>(static_cast<size_t>(N) * SERQ_RQ_ROW_BYTES(r));
    auto sr = buf<float>(N);
    for (int dt = 0; dt < 2; ++dt) {
      const void* Wp = dt ? static_cast<const void*>(Wb.data()) : static_cast<const void*>(W.data());
      EXPECT(serq_calibrate(Wp, static_cast<serq_dtype>(dt), K, N, a.data(), 0.5f, r, perm.get(), shi.get(), Wq.get(),
                            sw.get(), r ? Rq.get() : nullptr, r ? sr.get() : nullptr) == SERQ_OK);
      EXPECT(serq_calibrate(Wp, static_cast<serq_dtype>(dt), K, N, a.data(), 0.3f, r, perm.get(), shi.get(), Wq.get(),
                            sw.get(), r ? Rq.get() : nullptr, r ? sr.get() : nullptr) == SERQ_OK);
    }
    // GPTQ with T calibration tokens in each dtype
    const int T = 3 * K + 1;
    auto X = randn(static_cast<size_t>(T) * K, 1.0f);
    EXPECT(serq_calibrate_gptq(W.data(), SERQ_F32, K, N, a.data(), 0.5f, r, X.data(), SERQ_F32, T, 0.01f,
                               perm.get(), shi.get(), Wq.get(), sw.get(), r ? Rq.get() : nullptr,
                               r ? sr.get() : nullptr) == SERQ_OK);
    EXPECT(serq_calibrate_gptq(W.data(), SERQ_F32, K, N, a.data(), 0.5f, r, X.data(), SERQ_F32, 0, 0.01f,
                               perm.get(), shi.get(), Wq.get(), sw.get(), Rq.get(), sr.get()) == SERQ_EINVAL);
    // the next layer's order pushed into the outputs; a non-permutation is refused
    std::vector<int32_t> p(N);
    std::iota(p.begin(), p.end(), 0);
    std::shuffle(p.begin(), p.end(), rng);
    EXPECT(serq_permute_outputs(p.data(), K, N, r, Wq.get(), sw.get(), r ? Rq.get() : nullptr,
                                r ? sr.get() : nullptr) == SERQ_OK);
    if (N > 1) {
      p[0] = p[1];
      EXPECT(serq_permute_outputs(p.data(), K, N, r, Wq.get(), sw.get(), Rq.get(), sr.get()) == SERQ_EINVAL);
    }
    // bf6 prepack of Q(W^) and Q(R) into exactly SERQ_BF6_BYTES
    auto W6 = buf<uint8_t>(SERQ_BF6_BYTES(N, K));
    EXPECT(serq_prepack_bf6(Wq.get(), N, K, K / 2, W6.get()) == SERQ_OK);
    if (r) {
      auto R6 = buf<uint8_t>(SERQ_BF6_BYTES(N, r));
      EXPECT(serq_prepack_bf6(Rq.get(), N, r, SERQ_RQ_ROW_BYTES(r), R6.get()) == SERQ_OK);
    }
    // MXFP4 calibration (K and r multiples of 32)
    if (K % 32 == 0 && r % 32 == 0) {
      auto Wsc = buf<uint8_t>(static_cast<size_t>(N) * K / 32);
      auto Rq4 = buf<uint8_t>(static_cast<size_t>(N) * r / 2);
      auto Rsc = buf<uint8_t>(static_cast<size_t>(N) * r / 32);
      EXPECT(serq_calibrate_mx(W.data(), SERQ_F32, K, N, a.data(), 0.5f, r, perm.get(), shi.get(), Wq.get(), Wsc.get(),
                               r ? Rq4.get() : nullptr, r ? Rsc.get() : nullptr) == SERQ_OK);
    } else {
      auto Wsc = buf<uint8_t>(1);
      EXPECT(serq_calibrate_mx(W.data(), SERQ_F32, K, N, a.data(), 0.5f, r, perm.get(), shi.get(), Wq.get(), Wsc.get(),
                               Rq.get(), Wsc.get()) == SERQ_EINVAL);
    }
  }
}

// The online calls' validators: fake, aligned device addresses (never
// dereferenced: the launchers are stubs), then one bad argument at a time.
void online_validators() {
  uint8_t* const D = reinterpret_cast<uint8_t*>(uintptr_t{1} << 20);
  float* const F = reinterpret_cast<float*>(D);
  int32_t* const I = reinterpret_cast<int32_t*>(D);
  const int before = serq::g_launches;
  EXPECT(serq_quant_act(D, SERQ_BF16, 4, 64, F, 4, D, F, nullptr) == SERQ_OK);
  EXPECT(serq_quant_act(D, SERQ_BF16, 4, 63, F, 4, D, F, nullptr) == SERQ_EINVAL);
  EXPECT(serq_quant_act(D + 2, SERQ_BF16, 4, 64, F, 4, D, F, nullptr) == SERQ_EALIGN);
  EXPECT(serq_quant_act(nullptr, SERQ_BF16, 0, 64, F, 4, nullptr, nullptr, nullptr) == SERQ_OK);
  EXPECT(serq_quant_act(D, SERQ_BF16, 4, 64, F, 5, D, F, nullptr) == SERQ_EINVAL);
  EXPECT(serq_silu_mul_quant_act(D, D + 128, 64, SERQ_BF16, 4, 64, F, 4, D, F, nullptr) == SERQ_OK);
  EXPECT(serq_silu_mul_quant_act(D, D + 128, 32, SERQ_BF16, 4, 64, F, 4, D, F, nullptr) == SERQ_EINVAL);
  EXPECT(serq_silu_mul_quant_act(D + 1, D, 64, SERQ_BF16, 4, 64, F, 4, D, F, nullptr) == SERQ_EALIGN);
  EXPECT(serq_linear(D, F, 4, D, F, D, F, 4, 64, 32, 8, D, SERQ_BF16, nullptr, nullptr, nullptr) == SERQ_OK);
  EXPECT(serq_linear(D, F, 4, D, F, D, F, 4, 64, 32, 8, D, SERQ_BF16, I, I, nullptr) == SERQ_OK);
  EXPECT(serq_linear(D, F, 4, D, F, D, F, 4, 64, 32, 8, D, SERQ_BF16, I, nullptr, nullptr) == SERQ_EINVAL);
  EXPECT(serq_linear(D, F, 4, D, F, D, F, 4, 64, 32, 7, D, SERQ_BF16, nullptr, nullptr, nullptr) == SERQ_EINVAL);
  EXPECT(serq_linear(D, F, 4, D, F, D, F, 4, 64, 32, 66, D, SERQ_BF16, nullptr, nullptr, nullptr) == SERQ_EINVAL);
  EXPECT(serq_linear(D, F, 4, D + 8, F, D, F, 4, 64, 32, 8, D, SERQ_BF16, nullptr, nullptr, nullptr) == SERQ_EALIGN);
  EXPECT(serq_linear(nullptr, nullptr, 4, D, F, D, F, 0, 64, 32, 8, nullptr, SERQ_BF16, nullptr, nullptr, nullptr) ==
         SERQ_OK);
  EXPECT(serq_linear(D, F, 4, D, F, nullptr, nullptr, 4, 64, 32, 0, D, SERQ_F32, nullptr, nullptr, nullptr) == SERQ_OK);
  EXPECT(serq_act_bf6(D, 4, 64, D, nullptr) == SERQ_OK);
  EXPECT(serq_act_bf6(D, 4, (1 << 18) + 2, D, nullptr) == SERQ_EINVAL);
  EXPECT(serq_linear_bf6(D, F, D, F, D, F, 4, 256, 32, 8, D, SERQ_BF16, nullptr, nullptr, nullptr) == SERQ_OK);
  EXPECT(serq_linear_bf6(D, F, D, F, D, F, 4, 256, 32, 258, D, SERQ_BF16, nullptr, nullptr, nullptr) == SERQ_EINVAL);
  EXPECT(serq_quant_act_mx(D, SERQ_F32, 4, 64, F, D, D, nullptr) == SERQ_OK);
  EXPECT(serq_quant_act_mx(D, SERQ_F32, 4, 48, F, D, D, nullptr) == SERQ_EINVAL);
  EXPECT(serq_linear_mx(D, D, D, D, D, D, 4, 64, 32, 32, D, SERQ_BF16, nullptr, nullptr, nullptr) == SERQ_OK);
  EXPECT(serq_linear_mx(D, D, D, D, D, D, 4, 64, 32, 16, D, SERQ_BF16, nullptr, nullptr, nullptr) == SERQ_EINVAL);
  EXPECT(serq::g_launches - before == 9);   // one per accepted call with M > 0
  EXPECT(std::strlen(serq_strerror(-99)) > 0 && serq_rq_row_bytes(-1) == -1 && serq_bf6_bytes(-1, 2) == -1);
}

}  // namespace

int main() {
  offline_calls();
  online_validators();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host sanitizer driver: all checks passed\n");
  return 0;
}

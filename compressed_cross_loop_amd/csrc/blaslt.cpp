// Plain GEMMs on hipBLASLt, the vendor's matrix-core GEMM library, where its
// kernels beat the library's own tiled GEMM (gemm_nt.h): the bulk latent
// writer (16K tokens x 1024 x 6144 on the Ouro-1.4B shape: 155-187 against
// 290-365 us per call; 16K x 512 x 2048: 35 against 53 us).
//
//   C[m][n] = sum_k X[m][k] Y[n][k]      X, Y bf16 row-major; C fp32 or bf16
//
// hipBLASLt is column-major: with A = Y (K x N, leading dim ldy) transposed
// and B = X (K x M, leading dim ldx) as is, D = op(A) op(B) is N x M with
// leading dim ldc, i.e. C row-major.  K may come in segments that lie apart
// in memory (one per loop of the latent writer); each segment is one product
// added to the previous ones (beta = 1).
//
// The handle (one per device) and, per shape, the descriptors and the
// algorithm the library's heuristic picks (no workspace) are made on first
// use outside graph capture and kept until the process ends.  A call that
// would have to make them while its stream is being captured, or a shape the
// library declines, returns false and the caller runs its own GEMM.
#include <hipblaslt/hipblaslt.h>

#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>

#include "lla_internal.h"

namespace lla {

namespace {

constexpr int kMaxDevices = 64;

struct LtPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  bool ok = false;
};

// (device, M, N, K, ldx, ldy, ldc, C is fp32)
using LtKey = std::tuple<int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, bool>;

std::mutex g_mu;
hipblasLtHandle_t g_handle[kMaxDevices] = {};
bool g_handle_failed[kMaxDevices] = {};
std::map<LtKey, LtPlan> g_plans;

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) return true;   // unknown: do not set anything up
  return st != hipStreamCaptureStatusNone;
}

// the plan of a shape, made on first use (outside capture); nullptr if none
const LtPlan* plan_for(int dev, int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldy, int64_t ldc,
                       bool c_f32, hipStream_t s, hipblasLtHandle_t* handle) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (dev < 0 || dev >= kMaxDevices || g_handle_failed[dev]) return nullptr;
  const LtKey key{dev, M, N, K, ldx, ldy, ldc, c_f32};
  auto it = g_plans.find(key);
  if (it != g_plans.end()) {
    *handle = g_handle[dev];
    return it->second.ok ? &it->second : nullptr;
  }
  if (capturing(s)) return nullptr;
  if (!g_handle[dev] && hipblasLtCreate(&g_handle[dev]) != HIPBLAS_STATUS_SUCCESS) {
    g_handle[dev] = nullptr;
    g_handle_failed[dev] = true;
    return nullptr;
  }
  LtPlan& pl = g_plans[key];
  const hipDataType ct = c_f32 ? HIP_R_32F : HIP_R_16BF;
  bool ok = hipblasLtMatmulDescCreate(&pl.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  const int32_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  ok = ok && hipblasLtMatmulDescSetAttribute(pl.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)) ==
                 HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(pl.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)) ==
                 HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&pl.a, HIP_R_16BF, K, N, ldy) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&pl.b, HIP_R_16BF, K, M, ldx) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&pl.c, ct, N, M, ldc) == HIPBLAS_STATUS_SUCCESS;
  if (ok) {
    hipblasLtMatmulPreference_t pref = nullptr;
    ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
    const uint64_t ws = 0;
    ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws,
                                                     sizeof(ws)) == HIPBLAS_STATUS_SUCCESS;
    hipblasLtMatmulHeuristicResult_t res[1];
    int got = 0;
    ok = ok && hipblasLtMatmulAlgoGetHeuristic(g_handle[dev], pl.desc, pl.a, pl.b, pl.c, pl.c, pref, 1, res, &got) ==
                   HIPBLAS_STATUS_SUCCESS;
    ok = ok && got > 0 && res[0].state == HIPBLAS_STATUS_SUCCESS && res[0].workspaceSize == 0;
    if (ok) pl.algo = res[0].algo;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  }
  pl.ok = ok;
  *handle = g_handle[dev];
  return ok ? &pl : nullptr;
}

}  // namespace

bool lt_gemm_nt(const void* X, const void* Y, void* C, bool c_f32, int64_t M, int64_t N, int64_t kseg, int nseg,
                int64_t ldx, int64_t ldy, int64_t ldc, int64_t sxk, int64_t syk, hipStream_t s) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  hipblasLtHandle_t handle = nullptr;
  const LtPlan* pl = plan_for(dev, M, N, kseg, ldx, ldy, ldc, c_f32, s, &handle);
  if (!pl) return false;
  const float one = 1.f, zero = 0.f;
  for (int t = 0; t < nseg; ++t) {
    const void* A = static_cast<const char*>(Y) + 2 * t * syk;    // bf16 elements
    const void* Bm = static_cast<const char*>(X) + 2 * t * sxk;
    if (hipblasLtMatmul(handle, pl->desc, &one, A, pl->a, Bm, pl->b, t ? &one : &zero, C, pl->c, C, pl->c, &pl->algo,
                        nullptr, 0, s) != HIPBLAS_STATUS_SUCCESS)
      return false;   // the caller's GEMM then writes all of C
  }
  return true;
}

}  // namespace lla

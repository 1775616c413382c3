// bf16 linear y = bf16(x W^T + bias) through hipBLASLt, for the plain bf16
// layers of the DiT (the layers the model card leaves unquantised). This file
// launches no kernel of its own: it holds a per-device hipBLASLt handle and a
// per-shape plan (descriptors plus the heuristic's first algorithm), built on
// the first eager call of a shape and reused afterwards.
//
// Layout. hipBLASLt is column-major. Row-major y[M, N] is column-major
// y^T [N, M] (leading dimension N); row-major W[N, K] read column-major is
// W^T [K, N] (ld K), and row-major x[M, K] is x^T [K, M] (ld K). So
// y^T = op(A) B with A = W^T [K, N], op = transpose, B = x^T, m = N, n = M,
// k = K. The bias vector runs along m (one value per output channel), which is
// what hipBLASLt's bias epilogue broadcasts. Accumulation and the bias add are
// in fp32, one rounding to bf16 at the end, as in the hand-written kernel.
//
// Workspace: none (the heuristic is asked for algorithms that need none), so a
// call allocates nothing once its plan exists. A shape seen for the first time
// while the stream is capturing gets no plan and the caller takes the
// hand-written kernel instead (plan building queries the device).

#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>

#include "kernels.h"

namespace svdq {
namespace {

struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  hipblasLtMatmulAlgo_t algo{};
};

struct DeviceState {
  hipblasLtHandle_t handle = nullptr;
  bool failed = false;
  std::map<std::tuple<int64_t, int64_t, int64_t, bool>, Plan> plans;
};

std::mutex g_mu;
std::map<int, DeviceState> g_dev;

bool make_plan(hipblasLtHandle_t h, int64_t M, int64_t N, int64_t K, bool bias, Plan& p) {
  const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return false;
  bool ok = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)) ==
                HIPBLAS_STATUS_SUCCESS;
  if (ok && bias) {
    const hipblasLtEpilogue_t epi = HIPBLASLT_EPILOGUE_BIAS;
    const int32_t bias_type = HIP_R_16BF;
    ok = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bias_type,
                                         sizeof(bias_type)) == HIPBLAS_STATUS_SUCCESS;
  }
  ok = ok && hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, (uint64_t)K, (uint64_t)N, K) == HIPBLAS_STATUS_SUCCESS &&
       hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, (uint64_t)K, (uint64_t)M, K) == HIPBLAS_STATUS_SUCCESS &&
       hipblasLtMatrixLayoutCreate(&p.c, HIP_R_16BF, (uint64_t)N, (uint64_t)M, N) == HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulPreference_t pref = nullptr;
  ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
  uint64_t ws = 0;
  ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws,
                                                   sizeof(ws)) == HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulHeuristicResult_t res{};
  int found = 0;
  ok = ok && hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.a, p.b, p.c, p.c, pref, 1, &res, &found) ==
                 HIPBLAS_STATUS_SUCCESS &&
       found > 0 && res.state == HIPBLAS_STATUS_SUCCESS && res.workspaceSize == 0;
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ok) {
    p.algo = res.algo;
    return true;
  }
  if (p.a) hipblasLtMatrixLayoutDestroy(p.a);
  if (p.b) hipblasLtMatrixLayoutDestroy(p.b);
  if (p.c) hipblasLtMatrixLayoutDestroy(p.c);
  if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
  p = Plan{};
  return false;
}

}  // namespace

// Returns hipSuccess and sets *done when hipBLASLt ran the product; leaves
// *done false (nothing launched) when no plan exists or can be made now.
hipError_t blaslt_linear_bf16(const Bf16GemmArgs& a, hipStream_t stream, bool* done) {
  *done = false;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return e;
  const bool capturing = cs != hipStreamCaptureStatusNone;
  const auto key = std::make_tuple(a.M, a.N, a.K, a.bias != nullptr);
  Plan plan;
  hipblasLtHandle_t h = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    DeviceState& d = g_dev[dev];
    auto it = d.plans.find(key);
    if (it == d.plans.end()) {
      if (capturing || d.failed) return hipSuccess;
      if (!d.handle && hipblasLtCreate(&d.handle) != HIPBLAS_STATUS_SUCCESS) {
        d.handle = nullptr;
        d.failed = true;
        return hipSuccess;
      }
      Plan p;
      if (!make_plan(d.handle, a.M, a.N, a.K, a.bias != nullptr, p)) return hipSuccess;
      it = d.plans.emplace(key, p).first;
    }
    plan = it->second;
    h = d.handle;
  }
  if (a.bias != nullptr) {
    const void* bp = a.bias;
    if (hipblasLtMatmulDescSetAttribute(plan.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bp, sizeof(bp)) !=
        HIPBLAS_STATUS_SUCCESS)
      return hipErrorUnknown;
  }
  const float alpha = 1.0f, beta = 0.0f;
  if (hipblasLtMatmul(h, plan.desc, &alpha, a.w, plan.a, a.x, plan.b, &beta, a.y, plan.c, a.y, plan.c, &plan.algo,
                      nullptr, 0, stream) != HIPBLAS_STATUS_SUCCESS)
    return hipErrorUnknown;
  *done = true;
  return hipSuccess;
}

}  // namespace svdq

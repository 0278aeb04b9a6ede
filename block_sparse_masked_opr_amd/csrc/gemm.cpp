// Plain bf16 GEMMs of the attention block through hipBLASLt (gfx950 kernels,
// fp32 accumulation).  Row-major operands throughout: a row-major X[r][c] is
// the column-major matrix X^T, so C = op(A) op(B) in row-major terms is
// C^T = op(B)^T op(A)^T in hipBLASLt's column-major terms.
//
// One hipBLASLt handle per device, created on first use and kept for the life
// of the process; the descriptors of each problem shape and the heuristic's
// choice for it are made on its first call and kept likewise, so that a call
// costs the host little more than the matmul launch.
#include <hipblaslt/hipblaslt.h>

#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "opr_internal.h"

namespace opr {
namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
hipblasLtHandle_t g_handle[kMaxDevices] = {};
using Key = std::tuple<int, int, int, int, int64_t, int64_t, int64_t, int, size_t>;

bool handle_for(int dev, hipblasLtHandle_t *h) {
  if (dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_handle[dev] && hipblasLtCreate(&g_handle[dev]) != HIPBLAS_STATUS_SUCCESS) {
    g_handle[dev] = nullptr;
    return false;
  }
  *h = g_handle[dev];
  return true;
}

struct Plan {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  hipblasLtMatmulAlgo_t algo;
};
std::map<Key, Plan> g_plan;

}  // namespace

// Row-major C[M][N] = op(A) op(B), op(A) [M][K], op(B) [K][N]; A is stored
// [M][K] (trans_a = false) or [K][M] (true), B [K][N] or [N][K].  bf16 A, B;
// C bf16 or fp32 (c_f32).  ws: device scratch for hipBLASLt.
bool gemm_bf16(bool trans_a, bool trans_b, int64_t M, int64_t N, int64_t K, const void *A, const void *B, void *C,
               bool c_f32, void *ws, size_t ws_bytes, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  hipblasLtHandle_t h;
  if (!handle_for(dev, &h)) return false;
  const Key key{dev, (int)trans_a, (int)trans_b, (int)c_f32, M, N, K, 0, ws_bytes};
  Plan plan;
  bool have = false;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_plan.find(key);
    if (it != g_plan.end()) {
      plan = it->second;
      have = true;
    }
  }
  if (!have) {
    // column-major problem: C^T [N x M] = op'(B) [N x K] * op'(A) [K x M]
    const hipDataType ct = c_f32 ? HIP_R_32F : HIP_R_16BF;
    const int32_t ta = (int32_t)(trans_b ? HIPBLAS_OP_T : HIPBLAS_OP_N);  // applied to B's storage
    const int32_t tb = (int32_t)(trans_a ? HIPBLAS_OP_T : HIPBLAS_OP_N);
    hipblasLtMatmulPreference_t pref = nullptr;
    auto fail = [&]() {
      if (pref) hipblasLtMatmulPreferenceDestroy(pref);
      if (plan.c) hipblasLtMatrixLayoutDestroy(plan.c);
      if (plan.b) hipblasLtMatrixLayoutDestroy(plan.b);
      if (plan.a) hipblasLtMatrixLayoutDestroy(plan.a);
      if (plan.op) hipblasLtMatmulDescDestroy(plan.op);
      return false;
    };
    if (hipblasLtMatmulDescCreate(&plan.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return fail();
    hipblasLtMatmulDescSetAttribute(plan.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta));
    hipblasLtMatmulDescSetAttribute(plan.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb));
    // first operand: B's storage seen column-major: [N x K] with ld N (B [K][N]) or [K x N] with ld K (B [N][K])
    if (hipblasLtMatrixLayoutCreate(&plan.a, HIP_R_16BF, trans_b ? K : N, trans_b ? N : K, trans_b ? K : N) !=
        HIPBLAS_STATUS_SUCCESS)
      return fail();
    // second operand: A's storage: [K x M] with ld K (A [M][K]) or [M x K] with ld M (A [K][M])
    if (hipblasLtMatrixLayoutCreate(&plan.b, HIP_R_16BF, trans_a ? M : K, trans_a ? K : M, trans_a ? M : K) !=
        HIPBLAS_STATUS_SUCCESS)
      return fail();
    if (hipblasLtMatrixLayoutCreate(&plan.c, ct, N, M, N) != HIPBLAS_STATUS_SUCCESS) return fail();
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return fail();
    const uint64_t wsb = ws_bytes;
    hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb));
    hipblasLtMatmulHeuristicResult_t res[1];
    int n = 0;
    if (hipblasLtMatmulAlgoGetHeuristic(h, plan.op, plan.a, plan.b, plan.c, plan.c, pref, 1, res, &n) !=
            HIPBLAS_STATUS_SUCCESS ||
        n < 1)
      return fail();
    hipblasLtMatmulPreferenceDestroy(pref);
    plan.algo = res[0].algo;
    std::lock_guard<std::mutex> lock(g_mu);
    auto ins = g_plan.emplace(key, plan);
    if (!ins.second) {  // another thread made the same plan first: keep theirs
      hipblasLtMatrixLayoutDestroy(plan.c);
      hipblasLtMatrixLayoutDestroy(plan.b);
      hipblasLtMatrixLayoutDestroy(plan.a);
      hipblasLtMatmulDescDestroy(plan.op);
      plan = ins.first->second;
    }
  }
  const float alpha = 1.0f, beta = 0.0f;
  return hipblasLtMatmul(h, plan.op, &alpha, B, plan.a, A, plan.b, &beta, C, plan.c, C, plan.c, &plan.algo, ws,
                         ws_bytes, s) == HIPBLAS_STATUS_SUCCESS;
}

}  // namespace opr

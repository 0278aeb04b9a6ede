// Plain bf16 GEMMs of the attention block through hipBLASLt (gfx950 kernels,
// fp32 accumulation).  Row-major operands throughout: a row-major X[r][c] is
// the column-major matrix X^T, so C = op(A) op(B) in row-major terms is
// C^T = op(B)^T op(A)^T in hipBLASLt's column-major terms.
//
// One hipBLASLt handle per device, created on first use and kept for the life
// of the process; the heuristic's choice is cached per problem shape.
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
std::map<Key, hipblasLtMatmulAlgo_t> g_algo;

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

struct Descs {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  ~Descs() {
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (c) hipblasLtMatrixLayoutDestroy(c);
    if (b) hipblasLtMatrixLayoutDestroy(b);
    if (a) hipblasLtMatrixLayoutDestroy(a);
    if (op) hipblasLtMatmulDescDestroy(op);
  }
};

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
  // column-major problem: C^T [N x M] = op'(B) [N x K] * op'(A) [K x M]
  const hipblasOperation_t opb = trans_b ? HIPBLAS_OP_T : HIPBLAS_OP_N;  // applied to B^T storage
  const hipblasOperation_t opa = trans_a ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  Descs d;
  const hipDataType ct = c_f32 ? HIP_R_32F : HIP_R_16BF;
  if (hipblasLtMatmulDescCreate(&d.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return false;
  const int32_t ta = (int32_t)opb, tb = (int32_t)opa;
  hipblasLtMatmulDescSetAttribute(d.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta));
  hipblasLtMatmulDescSetAttribute(d.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb));
  // first operand: B's storage seen column-major: [N x K] with ld N (B [K][N]) or [K x N] with ld K (B [N][K])
  if (hipblasLtMatrixLayoutCreate(&d.a, HIP_R_16BF, trans_b ? K : N, trans_b ? N : K, trans_b ? K : N) !=
      HIPBLAS_STATUS_SUCCESS)
    return false;
  // second operand: A's storage: [K x M] with ld K (A [M][K]) or [M x K] with ld M (A [K][M])
  if (hipblasLtMatrixLayoutCreate(&d.b, HIP_R_16BF, trans_a ? M : K, trans_a ? K : M, trans_a ? M : K) !=
      HIPBLAS_STATUS_SUCCESS)
    return false;
  if (hipblasLtMatrixLayoutCreate(&d.c, ct, N, M, N) != HIPBLAS_STATUS_SUCCESS) return false;
  if (hipblasLtMatmulPreferenceCreate(&d.pref) != HIPBLAS_STATUS_SUCCESS) return false;
  const uint64_t wsb = ws_bytes;
  hipblasLtMatmulPreferenceSetAttribute(d.pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb));

  const Key key{dev, (int)trans_a, (int)trans_b, (int)c_f32, M, N, K, 0, ws_bytes};
  hipblasLtMatmulAlgo_t algo;
  bool have = false;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_algo.find(key);
    if (it != g_algo.end()) {
      algo = it->second;
      have = true;
    }
  }
  if (!have) {
    hipblasLtMatmulHeuristicResult_t res[1];
    int n = 0;
    if (hipblasLtMatmulAlgoGetHeuristic(h, d.op, d.a, d.b, d.c, d.c, d.pref, 1, res, &n) != HIPBLAS_STATUS_SUCCESS ||
        n < 1)
      return false;
    algo = res[0].algo;
    std::lock_guard<std::mutex> lock(g_mu);
    g_algo[key] = algo;
  }
  const float alpha = 1.0f, beta = 0.0f;
  return hipblasLtMatmul(h, d.op, &alpha, B, d.a, A, d.b, &beta, C, d.c, C, d.c, &algo, ws, ws_bytes, s) ==
         HIPBLAS_STATUS_SUCCESS;
}

}  // namespace opr

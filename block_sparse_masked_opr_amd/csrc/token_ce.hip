// Per-token cross entropy of a linear head on the attention output, and its
// gradient (gfx950): the loss step after the one-pass forward.
//
// The pages state that the one pass gives every token the same loss as the
// N separate passes (wiki summary, section "理论保证", Theorem 2.1); the loss
// is taken on the reasoning t_i and the generation copy r_out_i of each turn,
// while the context copy r_in_i and the human messages are context only
// (section "Token 复制").  This kernel scores exactly those rows:
//     z_p = W o_p,  loss_p = logsumexp(z_p) - z_p[y_p],
//     dout_p = grad_scale * (softmax(z_p) - onehot(y_p))^T W,
// with o_p the F = Hq * D outputs of token p and W the head's V x F weights.
//
// One workgroup of 4 waves per 32 rows.  Both products are bf16 MFMA with
// fp32 accumulation (v_mfma_f32_32x32x16_bf16):
//  1. z^T[v][row] = sum_f W[v][f] o[row][f]: wave w takes the 64-feature
//     groups w, w + 4, ...; lane (g, i) streams 64 contiguous bytes of W row
//     32 vb + i and of o row i per group (the 16 k values of each of the four
//     products of a group are assigned so that lane group g reads features
//     32 g .. 32 g + 31 of the group); the four partial sums meet in LDS.
//  2. per row: softmax statistics from the lane's 16 logits per 32-logit block
//     and its partner lane i + 32; loss and g = grad_scale * (p - onehot) in
//     the accumulator layout.
//  3. g is written to the workspace, bf16 [rows][V] (zero for rows that are
//     not scored or have an invalid label), and dout = g W is a plain GEMM
//     (hipBLASLt, bf16 operands, fp32 accumulation, bf16 out): with K = V it
//     streams dout at the rate of a copy.
// The kernel reads o once; the GEMM writes dout once.
#include "attn_common.h"
#include "opr_internal.h"

namespace opr {
namespace {

typedef __bf16 __attribute__((ext_vector_type(8))) bf16x8;

constexpr int kRows = 32;   // rows per workgroup
constexpr int kWaves = 4;   // feature groups are dealt to the waves round-robin
constexpr int kGroup = 64;  // features per group (four products of 16)

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }

template <int NVB>  // V = 32 * NVB
__global__ __launch_bounds__(256) void token_ce_kernel(const uint16_t *__restrict__ o, const uint16_t *__restrict__ w,
                                                       const int32_t *__restrict__ labels,
                                                       const uint8_t *__restrict__ tok_type, int64_t n_rows, int F,
                                                       float grad_scale, float *__restrict__ loss,
                                                       uint16_t *__restrict__ gout) {
  constexpr int V = 32 * NVB;
  __shared__ float red[kWaves][NVB][16][64];
  __shared__ int sh_any;

  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  const int64_t row = r0 + li;
  const bool in_range = row < n_rows;
  const uint8_t ty = in_range ? tok_type[row] : (uint8_t)OPR_TOK_PAD;
  const bool scored = ty == OPR_TOK_T || ty == OPR_TOK_ROUT;
  if (tid == 0) sh_any = 0;
  __syncthreads();
  if (wave == 0 && __ballot(scored) != 0 && lane == 0) sh_any = 1;
  __syncthreads();

  if (!sh_any) {  // no scored row: loss 0 and zero gradients
    if (wave == 0 && g == 0 && in_range) loss[row] = 0.0f;
    if (gout) {
      const int64_t nr = min((int64_t)kRows, n_rows - r0);
      const int64_t words = nr * V / 8;  // 16-byte words of the block's rows of g (V % 32 == 0)
      uint4 *d = reinterpret_cast<uint4 *>(gout + r0 * V);
      for (int64_t x = tid; x < words; x += 256) d[x] = make_uint4(0, 0, 0, 0);
    }
    return;
  }

  // 1. partial logits z^T[v][row] over this wave's feature groups
  const int64_t orow = in_range ? row : n_rows - 1;  // rows past the end read a valid row, then count as 0
  const uint4 *op = reinterpret_cast<const uint4 *>(o + orow * F + 32 * g);
  f32x16 acc[NVB];
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb) acc[vb] = zero_f32x16();
  const int ngroups = F / kGroup;
#pragma unroll 2
  for (int G = wave; G < ngroups; G += kWaves) {
    uint4 ov[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) ov[s] = op[G * (kGroup / 8) + s];
    if (!in_range) {
#pragma unroll
      for (int s = 0; s < 4; ++s) ov[s] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      const uint4 *wp = reinterpret_cast<const uint4 *>(w + (int64_t)(32 * vb + li) * F + G * kGroup + 32 * g);
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[vb] = mfma_bf16(as_bf16x8(wp[s]), as_bf16x8(ov[s]), acc[vb]);
    }
  }
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][vb][r][lane] = acc[vb][r];
  __syncthreads();
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      acc[vb][r] = (red[0][vb][r][lane] + red[1][vb][r][lane]) + (red[2][vb][r][lane] + red[3][vb][r][lane]);

  // 2. softmax statistics of row li (logits split between lanes li and li + 32):
  // register r of block vb in lane group g holds logit 32 vb + 8 (r / 4) + 4 g + r % 4
  float m = -INFINITY;
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[vb][r]);
  m = fmaxf(m, __shfl_xor(m, 32));
  float ssum = 0.0f;
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int r = 0; r < 16; ++r) ssum += __expf(acc[vb][r] - m);
  ssum += __shfl_xor(ssum, 32);
  const float lse = m + __logf(ssum);
  const int lab = scored ? labels[row] : -1;
  const bool valid = lab >= 0 && lab < V;
  float zl = 0.0f;
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * vb + 8 * (r >> 2) + 4 * g + (r & 3) == lab) zl = acc[vb][r];
  zl += __shfl_xor(zl, 32);  // exactly one of the two lanes holds the label's logit
  if (wave == 0 && g == 0 && in_range) loss[row] = !scored ? 0.0f : (valid ? lse - zl : __int_as_float(0x7fc00000));
  if (!gout) return;

  // g = grad_scale * (softmax - onehot) of row li, bf16: registers 4k .. 4k + 3
  // of logit block vb hold logits 32 vb + 8 k + 4 g + 0..3; every wave holds all
  // of them after the reduction, and wave k writes the register group k
  const bool grad = scored && valid;
  if (in_range) {
    uint16_t *grow = gout + row * V;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k != wave) continue;
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        uint16_t b4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * k + e, v = 32 * vb + 8 * k + 4 * g + e;
          const float pv = __expf(acc[vb][r] - lse) - (v == lab ? 1.0f : 0.0f);
          b4[e] = f32_to_bf16(grad ? grad_scale * pv : 0.0f);
        }
        *reinterpret_cast<uint2 *>(grow + 32 * vb + 8 * k + 4 * g) = *reinterpret_cast<const uint2 *>(b4);
      }
    }
  }
}

}  // namespace

constexpr size_t kCeGemmWs = (size_t)32 << 20;  // hipBLASLt scratch of the dout GEMM

size_t token_ce_ws_bytes(int64_t n_rows, int32_t V) { return align_up((size_t)n_rows * V * sizeof(uint16_t)) + kCeGemmWs; }

hipError_t launch_token_ce(int32_t B, int32_t L, int32_t F, int32_t V, const void *o, const void *w,
                           const int32_t *labels, const uint8_t *tok_type, float grad_scale, float *loss,
                           void *dout, void *workspace, hipStream_t s) {
  const int64_t n_rows = (int64_t)B * L;
  const uint16_t *w16 = static_cast<const uint16_t *>(w);
  uint16_t *gbuf = dout ? static_cast<uint16_t *>(workspace) : nullptr;
  const unsigned grid = (unsigned)((n_rows + kRows - 1) / kRows);
  const uint16_t *o16 = static_cast<const uint16_t *>(o);
  switch (V / 32) {
    case 1: token_ce_kernel<1><<<grid, 256, 0, s>>>(o16, w16, labels, tok_type, n_rows, F, grad_scale, loss, gbuf); break;
    case 2: token_ce_kernel<2><<<grid, 256, 0, s>>>(o16, w16, labels, tok_type, n_rows, F, grad_scale, loss, gbuf); break;
    default: token_ce_kernel<4><<<grid, 256, 0, s>>>(o16, w16, labels, tok_type, n_rows, F, grad_scale, loss, gbuf); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !dout) return e;
  // dout [rows][F] = g [rows][V] W [V][F]
  char *scratch = static_cast<char *>(workspace) + align_up((size_t)n_rows * V * sizeof(uint16_t));
  if (!gemm_bf16(false, false, n_rows, F, V, gbuf, w, dout, false, scratch, kCeGemmWs, s)) return hipErrorUnknown;
  return hipSuccess;
}

}  // namespace opr

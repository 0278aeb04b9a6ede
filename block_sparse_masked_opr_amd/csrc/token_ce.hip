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
//  3. dout^T[f][row] = sum_v W^T[f][v] g^T[v][row]: the accumulator registers
//     8j .. 8j + 7 of a logit block are directly the B operand of a product
//     whose 16 k values are logits 16 j + {0..3, 8..11} (lane group 0) and
//     16 j + {4..7, 12..15} (lane group 1); A comes from W^T (transposed once
//     into the workspace, the logits of each 16-block permuted so that each
//     lane group's eight are contiguous), one 16-byte read per lane.  Each 64-feature group
//     goes through LDS into row-major order, so dout is written in full
//     128-byte row pieces.
// The kernel is bound by HBM: it reads o once and writes dout once.
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

// W^T with the logits of each 16-logit block in the order the gradient
// product's lane groups take them: wt[f][16 b + p] = w[16 b + perm(p)][f] with
// perm = (0..3, 8..11, 4..7, 12..15), so that lane group g finds its eight
// logits 16 b + 4 g + {0..3, 8..11} in one 16-byte run.
__global__ void transpose_head_kernel(const uint16_t *__restrict__ w, uint16_t *__restrict__ wt, int F, int V) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)F * V) return;
  const int f = (int)(i % F), v = (int)(i / F);  // consecutive threads read consecutive f of one row
  const int q = v & 15;
  const int p = (q & 3) | ((q & 8) >> 1) | ((q & 4) << 1);  // position of logit v in its block
  wt[(int64_t)f * V + (v & ~15) + p] = w[i];
}

template <int NVB>  // V = 32 * NVB
__global__ __launch_bounds__(256) void token_ce_kernel(const uint16_t *__restrict__ o, const uint16_t *__restrict__ w,
                                                       const uint16_t *__restrict__ wt,
                                                       const int32_t *__restrict__ labels,
                                                       const uint8_t *__restrict__ tok_type, int64_t n_rows, int F,
                                                       float grad_scale, float *__restrict__ loss,
                                                       uint16_t *__restrict__ dout) {
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
    if (dout) {
      const int64_t nr = min((int64_t)kRows, n_rows - r0);
      const int64_t words = nr * F / 8;  // 16-byte words of the block's rows (F % 64 == 0)
      uint4 *d = reinterpret_cast<uint4 *>(dout + r0 * F);
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
  if (!dout) return;

  // g^T in the accumulator layout, as bf16 B operands
  const bool grad = scored && valid;
  bf16x8 gb[NVB][2];
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = 32 * vb + 8 * (r >> 2) + 4 * g + (r & 3);
      const float pv = __expf(acc[vb][r] - lse) - (v == lab ? 1.0f : 0.0f);
      gb[vb][r >> 3][r & 7] = (__bf16)(grad ? grad_scale * pv : 0.0f);
    }

  // 3. dout^T[f][row] over this wave's feature groups, 32 features at a time;
  // each 64-feature group is turned into row-major bf16 in LDS (the wave's
  // own 32 x 64 tile) and written as full 128-byte row pieces
  __syncthreads();  // the partial-sum buffer is reused for the tiles
  uint16_t *tile = reinterpret_cast<uint16_t *>(&red[0][0][0][0]) + wave * (kRows * kGroup);
  // W^T operands of a group: per half h, logit block vb and k half j, logits
  // 32 vb + 16 j + 4 g + {0..3, 8..11} of W^T row fb + li, one 16-byte run in
  // the permuted W^T.  The next group's are loaded while the current one is
  // computed and written.
  auto load_wt = [&](int G, uint4 (&a)[2][NVB][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint16_t *wr = wt + (int64_t)(G * kGroup + 32 * h + li) * V + 8 * g;
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int j = 0; j < 2; ++j) a[h][vb][j] = *reinterpret_cast<const uint4 *>(wr + 32 * vb + 16 * j);
    }
  };
  uint4 wa[2][NVB][2];
  if (wave < ngroups) load_wt(wave, wa);
  for (int G = wave; G < ngroups; G += kWaves) {
    uint4 cur[2][NVB][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int j = 0; j < 2; ++j) cur[h][vb][j] = wa[h][vb][j];
    if (G + kWaves < ngroups) load_wt(G + kWaves, wa);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int fb = G * kGroup + 32 * h;
      f32x16 c = zero_f32x16();
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int j = 0; j < 2; ++j) c = mfma_bf16(as_bf16x8(cur[h][vb][j]), gb[vb][j], c);
      // register r holds feature fb + 8 (r / 4) + 4 g + r % 4 of row li
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint16_t b4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) b4[e] = f32_to_bf16(c[4 * q4 + e]);
        *reinterpret_cast<uint2 *>(tile + li * kGroup + 32 * h + 8 * q4 + 4 * g) = *reinterpret_cast<const uint2 *>(b4);
      }
    }
    // the tile's 32 rows of 128 bytes: lane l writes 16 bytes of row 8 k + l / 8
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = 8 * k + (lane >> 3), c8 = (lane & 7) * 8;
      const uint4 val = *reinterpret_cast<const uint4 *>(tile + rr * kGroup + c8);
      if (r0 + rr < n_rows) *reinterpret_cast<uint4 *>(dout + (r0 + rr) * F + G * kGroup + c8) = val;
    }
  }
}

}  // namespace

size_t token_ce_ws_bytes(int32_t F, int32_t V) { return align_up((size_t)F * V * sizeof(uint16_t)); }

hipError_t launch_token_ce(int32_t B, int32_t L, int32_t F, int32_t V, const void *o, const void *w,
                           const int32_t *labels, const uint8_t *tok_type, float grad_scale, float *loss,
                           void *dout, void *workspace, hipStream_t s) {
  const uint16_t *w16 = static_cast<const uint16_t *>(w);
  uint16_t *wt = static_cast<uint16_t *>(workspace);
  if (dout) {
    const int64_t n = (int64_t)F * V;
    transpose_head_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(w16, wt, F, V);
  }
  const int64_t n_rows = (int64_t)B * L;
  const unsigned grid = (unsigned)((n_rows + kRows - 1) / kRows);
  const uint16_t *o16 = static_cast<const uint16_t *>(o);
  uint16_t *d16 = static_cast<uint16_t *>(dout);
  switch (V / 32) {
    case 1: token_ce_kernel<1><<<grid, 256, 0, s>>>(o16, w16, wt, labels, tok_type, n_rows, F, grad_scale, loss, d16); break;
    case 2: token_ce_kernel<2><<<grid, 256, 0, s>>>(o16, w16, wt, labels, tok_type, n_rows, F, grad_scale, loss, d16); break;
    default: token_ce_kernel<4><<<grid, 256, 0, s>>>(o16, w16, wt, labels, tok_type, n_rows, F, grad_scale, loss, d16); break;
  }
  return hipGetLastError();
}

}  // namespace opr

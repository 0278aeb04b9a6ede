// Elementwise kernels of the attention block around the masked attention
// (gfx950): the RMS normalisation of every q and k head before RoPE, as in
// Qwen-3 (the model family the pages train: wiki summary, "实验结果"), and its
// backward, with the deterministic reduction of the norm weights' gradients.
//
// Row layouts: qkv [T][Hq + 2 Hkv][D] bf16 (the projection's output, q heads,
// then k heads, then v heads, per token), qn [T][Hq][D], kn and v [T][Hkv][D].
// One item is one (token, head) vector of D values; D/8 consecutive lanes
// hold one item, 8 values (16 bytes of bf16) each, so a wave covers 8 or 4
// consecutive heads of one token in one coalesced run.
//
// RMSNorm of a head x with weight g: y = g * x * r, r = (mean(x^2) + eps)^-1/2.
// Backward: dx = r * g * dy - x * r^3 * mean(g * dy * x), dg = sum dy * x * r.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "opr_internal.h"

namespace opr {
namespace {

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ void load8_bf16(const uint16_t *p, float (&x)[8]) {
  const uint4 w = *reinterpret_cast<const uint4 *>(p);
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(a[i] << 16);
    x[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void store8_bf16(uint16_t *p, const float (&y)[8]) {
  uint4 w;
  w.x = (uint32_t)bf16_bits(y[0]) | ((uint32_t)bf16_bits(y[1]) << 16);
  w.y = (uint32_t)bf16_bits(y[2]) | ((uint32_t)bf16_bits(y[3]) << 16);
  w.z = (uint32_t)bf16_bits(y[4]) | ((uint32_t)bf16_bits(y[5]) << 16);
  w.w = (uint32_t)bf16_bits(y[6]) | ((uint32_t)bf16_bits(y[7]) << 16);
  *reinterpret_cast<uint4 *>(p) = w;
}

__device__ __forceinline__ void load8_f32(const float *p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// sum over the TPH lanes of an item (consecutive, aligned lanes)
template <int TPH>
__device__ __forceinline__ float item_sum(float v) {
#pragma unroll
  for (int m = 1; m < TPH; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void qk_norm_fwd_kernel(int64_t T, int Hq, int Hkv, float eps,
                                                          const uint16_t *__restrict__ qkv,
                                                          const float *__restrict__ gq,
                                                          const float *__restrict__ gk, uint16_t *__restrict__ qn,
                                                          uint16_t *__restrict__ kn, uint16_t *__restrict__ v) {
  constexpr int TPH = D / 8;
  constexpr int IPB = 256 / TPH;  // items per workgroup pass
  const int NH = Hq + 2 * Hkv;
  const int l = threadIdx.x % TPH, d0 = 8 * l;
  const int64_t items = T * NH;
  for (int64_t it = (int64_t)blockIdx.x * IPB + threadIdx.x / TPH; it < items; it += (int64_t)gridDim.x * IPB) {
    const int64_t t = it / NH;
    const int j = (int)(it - t * NH);
    float x[8];
    load8_bf16(qkv + it * D + d0, x);
    if (j >= Hq + Hkv) {  // v head: copied unchanged
      *reinterpret_cast<uint4 *>(v + (t * Hkv + (j - Hq - Hkv)) * D + d0) =
          *reinterpret_cast<const uint4 *>(qkv + it * D + d0);
      continue;
    }
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    const float r = rsqrtf(item_sum<TPH>(ss) * (1.0f / D) + eps);
    const bool isq = j < Hq;
    const float *g = isq ? gq : gk;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = g[d0 + e] * (x[e] * r);
    uint16_t *dst = isq ? qn + (t * Hq + j) * D : kn + (t * Hkv + (j - Hq)) * D;
    store8_bf16(dst + d0, y);
  }
}

template <int D>
__global__ __launch_bounds__(256) void qk_norm_bwd_kernel(int64_t T, int Hq, int Hkv, float eps,
                                                          const uint16_t *__restrict__ qkv,
                                                          const float *__restrict__ gq,
                                                          const float *__restrict__ gk,
                                                          const float *__restrict__ dqn,
                                                          const float *__restrict__ dkn,
                                                          const float *__restrict__ dv,
                                                          uint16_t *__restrict__ dqkv, float *__restrict__ part) {
  constexpr int TPH = D / 8;
  constexpr int IPB = 256 / TPH;
  const int NH = Hq + 2 * Hkv;
  const int l = threadIdx.x % TPH, d0 = 8 * l;
  const int64_t items = T * NH;
  float accq[8] = {}, acck[8] = {};
  for (int64_t it = (int64_t)blockIdx.x * IPB + threadIdx.x / TPH; it < items; it += (int64_t)gridDim.x * IPB) {
    const int64_t t = it / NH;
    const int j = (int)(it - t * NH);
    float dy[8];
    if (j >= Hq + Hkv) {  // v head: gradient passes through
      load8_f32(dv + (t * Hkv + (j - Hq - Hkv)) * D + d0, dy);
      store8_bf16(dqkv + it * D + d0, dy);
      continue;
    }
    const bool isq = j < Hq;
    load8_f32(isq ? dqn + (t * Hq + j) * D + d0 : dkn + (t * Hkv + (j - Hq)) * D + d0, dy);
    float x[8];
    load8_bf16(qkv + it * D + d0, x);
    const float *g = isq ? gq : gk;
    float ss = 0.0f, sg = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ss = fmaf(x[e], x[e], ss);
      sg = fmaf(g[d0 + e] * dy[e], x[e], sg);
    }
    const float r = rsqrtf(item_sum<TPH>(ss) * (1.0f / D) + eps);
    const float c = r * r * r * item_sum<TPH>(sg) * (1.0f / D);
    float dx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dx[e] = r * g[d0 + e] * dy[e] - x[e] * c;
      if (isq) accq[e] = fmaf(dy[e], x[e] * r, accq[e]);
      else acck[e] = fmaf(dy[e], x[e] * r, acck[e]);
    }
    store8_bf16(dqkv + it * D + d0, dx);
  }
  // per-workgroup partial sums of dg over its items: [2][D] (q, k)
  __shared__ float red[2][IPB][D];
  const int grp = threadIdx.x / TPH;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[0][grp][d0 + e] = accq[e];
    red[1][grp][d0 + e] = acck[e];
  }
  __syncthreads();
  for (int k = threadIdx.x; k < 2 * D; k += 256) {
    float s = 0.0f;
    for (int gi = 0; gi < IPB; ++gi) s += red[k / D][gi][k % D];
    part[(int64_t)blockIdx.x * 2 * D + k] = s;
  }
}

// dg[k] = sum over workgroups of part[w][k], k < 2D (q weights, then k
// weights): one workgroup per k, its threads striding over the partials, then
// a fixed-order tree over the workgroup (deterministic).
__global__ __launch_bounds__(256) void dg_reduce_kernel(int nparts, int D, const float *__restrict__ part,
                                                        float *__restrict__ dgq, float *__restrict__ dgk) {
  const int k = blockIdx.x;
  float s = 0.0f;
  for (int w = threadIdx.x; w < nparts; w += 256) s += part[(int64_t)w * 2 * D + k];
  __shared__ float red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int m = 128; m > 0; m >>= 1) {
    if (threadIdx.x < m) red[threadIdx.x] += red[threadIdx.x + m];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (k < D) dgq[k] = red[0];
    else dgk[k - D] = red[0];
  }
}

}  // namespace

int block_norm_grid(int D, int64_t T, int NH) {
  const int64_t ipb = 256 / (D / 8);
  const int64_t need = (T * NH + ipb - 1) / ipb;
  return (int)(need < 2048 ? (need < 1 ? 1 : need) : 2048);
}

hipError_t launch_qk_norm_fwd(int D, int64_t T, int Hq, int Hkv, float eps, const void *qkv, const float *gq,
                              const float *gk, void *qn, void *kn, void *v, hipStream_t s) {
  const int grid = block_norm_grid(D, T, Hq + 2 * Hkv);
  auto *src = static_cast<const uint16_t *>(qkv);
  auto *a = static_cast<uint16_t *>(qn), *b = static_cast<uint16_t *>(kn), *c = static_cast<uint16_t *>(v);
  if (D == 64) qk_norm_fwd_kernel<64><<<grid, 256, 0, s>>>(T, Hq, Hkv, eps, src, gq, gk, a, b, c);
  else qk_norm_fwd_kernel<128><<<grid, 256, 0, s>>>(T, Hq, Hkv, eps, src, gq, gk, a, b, c);
  return hipGetLastError();
}

hipError_t launch_qk_norm_bwd(int D, int64_t T, int Hq, int Hkv, float eps, const void *qkv, const float *gq,
                              const float *gk, const float *dqn, const float *dkn, const float *dv, void *dqkv,
                              float *part, float *dgq, float *dgk, hipStream_t s) {
  const int grid = block_norm_grid(D, T, Hq + 2 * Hkv);
  auto *src = static_cast<const uint16_t *>(qkv);
  auto *dst = static_cast<uint16_t *>(dqkv);
  if (D == 64) qk_norm_bwd_kernel<64><<<grid, 256, 0, s>>>(T, Hq, Hkv, eps, src, gq, gk, dqn, dkn, dv, dst, part);
  else qk_norm_bwd_kernel<128><<<grid, 256, 0, s>>>(T, Hq, Hkv, eps, src, gq, gk, dqn, dkn, dv, dst, part);
  dg_reduce_kernel<<<2 * D, 256, 0, s>>>(grid, D, part, dgq, dgk);
  return hipGetLastError();
}

}  // namespace opr

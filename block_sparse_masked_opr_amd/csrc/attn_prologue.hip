// Prologue kernels of the attention path: the RoPE table at the strategic
// position ids, head-major (optionally rotated) fp16 copies of q / k / v / dout
// with one power-of-two scale per 64-token block, padded to a whole number of
// 128-token tiles with zeros; the per-token mask records; and the backward
// preprocessing delta = rowsum(dout * o).
//
// RoPE (rotate-half): pair (j, j + D/2) of a head vector is rotated by
// pos * theta^(-2j/D).  The angle and its cosine and sine are computed in
// float64 (positions reach ~2.4e5, where a float32 angle would be off by
// ~1e-2 rad); the rotation itself runs in float32.
#include "attn_common.h"
#include "opr_internal.h"

namespace opr {
namespace {

// table[b][t][j] = (cos, sin) of pos(b, t) * theta^(-2j/D); PAD and t >= L use 0.
__global__ __launch_bounds__(256) void rope_table_kernel(int32_t B, int32_t L, int32_t Lp,
                                                         int32_t half, double log2_theta,
                                                         const int32_t *tok_pos, float2 *table) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)B * Lp * half;
  if (gid >= total) return;
  const int32_t j = (int32_t)(gid % half);
  const int64_t bt = gid / half;
  const int32_t t = (int32_t)(bt % Lp);
  const int32_t b = (int32_t)(bt / Lp);
  const int32_t pos = t < L ? tok_pos[(int64_t)b * L + t] : 0;
  const double inv_freq = exp2(-(2.0 * j / (2.0 * half)) * log2_theta);
  double s, c;
  sincos((double)pos * inv_freq, &s, &c);
  table[gid] = make_float2((float)c, (float)s);
}

// One workgroup per (64-token block, head, row).  x: [B][L][H][D] bf16.
// Writes the block as fp16(x' * 2^e), x' = RoPE(x) or x, with the block
// exponent e (largest |x'| of the block scaled into [2^14, 2^15)) stored in
// exps[b][h][block]; rows (optional): [B][H][Lp][D]; trans (optional):
// [B][H][D][Lp].  Tokens t >= L are zero.
template <int D, bool ROPE>
__global__ __launch_bounds__(256) void pack_kernel(int32_t L, int32_t Lp, int32_t H,
                                                   const uint16_t *x, const float2 *table,
                                                   uint16_t *rows, uint16_t *trans,
                                                   int32_t *exps) {
  constexpr int HALF = D / 2;
  constexpr int PER = HALF / 4;           // pairs per thread (4 threads per token)
  constexpr int TS = 64 + 8;              // LDS row stride of the transposed tile
  __shared__ __attribute__((aligned(16))) uint16_t tile[D * TS];
  __shared__ float wmax[4];
  const int t0 = blockIdx.x * 64;
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int tt = tid >> 2, part = tid & 3;
  const int t = t0 + tt;
  const int j0 = part * PER;
  float lo[PER], hi[PER];
  if (t < L) {
    const uint16_t *src = x + (((int64_t)b * L + t) * H + h) * D;
    uint16_t lb[PER], hb[PER];
#pragma unroll
    for (int c = 0; c < PER; c += 8) {
      *reinterpret_cast<uint4 *>(&lb[c]) = *reinterpret_cast<const uint4 *>(src + j0 + c);
      *reinterpret_cast<uint4 *>(&hb[c]) = *reinterpret_cast<const uint4 *>(src + HALF + j0 + c);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      lo[e] = bf16_to_f32(lb[e]);
      hi[e] = bf16_to_f32(hb[e]);
    }
    if (ROPE) {
      const float2 *cs = table + ((int64_t)b * Lp + t) * HALF + j0;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float2 r = cs[e];
        const float x1 = lo[e], x2 = hi[e];
        lo[e] = x1 * r.x - x2 * r.y;
        hi[e] = x2 * r.x + x1 * r.y;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) lo[e] = hi[e] = 0.0f;
  }
  // block max |x'|: lanes, then the four waves
  float m = 0.0f;
#pragma unroll
  for (int e = 0; e < PER; ++e) m = fmaxf(m, fmaxf(fabsf(lo[e]), fabsf(hi[e])));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int ex = block_exponent(m);
  if (tid == 0) exps[((int64_t)b * H + h) * (Lp / 64) + blockIdx.x] = ex;
  uint16_t lq[PER], hq[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    lq[e] = f32_to_f16_bits(ldexpf(lo[e], ex));
    hq[e] = f32_to_f16_bits(ldexpf(hi[e], ex));
  }
  if (rows) {
    uint16_t *dst = rows + (((int64_t)b * H + h) * Lp + t) * D;
#pragma unroll
    for (int c = 0; c < PER; c += 8) {
      *reinterpret_cast<uint4 *>(dst + j0 + c) = *reinterpret_cast<const uint4 *>(&lq[c]);
      *reinterpret_cast<uint4 *>(dst + HALF + j0 + c) = *reinterpret_cast<const uint4 *>(&hq[c]);
    }
  }
  if (trans) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      tile[(j0 + e) * TS + tt] = lq[e];
      tile[(HALF + j0 + e) * TS + tt] = hq[e];
    }
    __syncthreads();
    // D rows of 64 tokens (128 bytes = 8 chunks of 16 bytes)
    for (int c = tid; c < D * 8; c += 256) {
      const int d = c >> 3, ch = c & 7;
      uint16_t *dst = trans + (((int64_t)b * H + h) * D + d) * Lp + t0 + ch * 8;
      *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(&tile[d * TS + ch * 8]);
    }
  }
}

// meta[b][t] = (conv, turn * 8 + type) for t < L, (-1, PAD) past L.
__global__ __launch_bounds__(256) void meta_kernel(int32_t B, int32_t L, int32_t Lp, const int32_t *conv,
                                                   const int32_t *turn, const uint8_t *type, int2 *meta) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)B * Lp) return;
  const int32_t t = (int32_t)(gid % Lp);
  const int64_t b = gid / Lp;
  int2 m = make_int2(-1, 4);
  if (t < L) {
    const int64_t i = b * L + t;
    m = make_int2(conv[i], (turn[i] << 3) | type[i]);
  }
  meta[gid] = m;
}

// delta[b][h][t] = sum_d dout * o (float32 over bf16 inputs);
// lse2[b][h][t] = lse * log2(e), +inf where the row has no key (lse = -inf)
// or t >= L, so that recomputed probabilities are exactly 0 there.
// One wave per token: D/8 lanes read one head's 16-byte chunks, so a wave
// covers 64/(D/8) heads per step with fully coalesced row reads.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(int32_t B, int32_t L, int32_t Lp, int32_t Hq,
                                                    const uint16_t *o, const uint16_t *dout,
                                                    const float *lse, float *delta, float *lse2) {
  constexpr int LPH = D / 8;        // lanes per head
  constexpr int HPS = 64 / LPH;     // heads per step
  const int64_t bt = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bt >= (int64_t)B * Lp) return;
  const int lane = threadIdx.x & 63;
  const int32_t t = (int32_t)(bt % Lp);
  const int32_t b = (int32_t)(bt / Lp);
  const int hl = lane / LPH, part = lane % LPH;
  for (int h0 = 0; h0 < Hq; h0 += HPS) {
    const int h = h0 + hl;
    float acc = 0.0f;
    if (t < L && h < Hq) {
      const int64_t base = (((int64_t)b * L + t) * Hq + h) * D + part * 8;
      uint16_t ov[8], dv[8];
      *reinterpret_cast<uint4 *>(ov) = *reinterpret_cast<const uint4 *>(o + base);
      *reinterpret_cast<uint4 *>(dv) = *reinterpret_cast<const uint4 *>(dout + base);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += bf16_to_f32(ov[e]) * bf16_to_f32(dv[e]);
    }
#pragma unroll
    for (int off = LPH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (part == 0 && h < Hq) {
      float l2 = INFINITY;
      if (t < L) {
        const float l = lse[((int64_t)b * Hq + h) * L + t];
        l2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
      }
      const int64_t out = ((int64_t)b * Hq + h) * Lp + t;
      delta[out] = acc;
      lse2[out] = l2;
    }
  }
}

template <int D>
void launch_pack(bool rope, int32_t B, int32_t L, int32_t Lp, int32_t H, const void *x,
                 const float2 *table, uint16_t *rows, uint16_t *trans, int32_t *exps,
                 hipStream_t s) {
  const dim3 grid(Lp / 64, H, B);
  const uint16_t *src = static_cast<const uint16_t *>(x);
  if (rope)
    pack_kernel<D, true><<<grid, 256, 0, s>>>(L, Lp, H, src, table, rows, trans, exps);
  else
    pack_kernel<D, false><<<grid, 256, 0, s>>>(L, Lp, H, src, table, rows, trans, exps);
}

}  // namespace

void launch_meta(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  const int64_t total = (int64_t)in.B * ws.Lp;
  meta_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(in.B, in.L, ws.Lp, in.layout.tok_conv,
                                                              in.layout.tok_turn, in.layout.tok_type, ws.meta);
}

void launch_rope_table(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  const int32_t half = in.D / 2;
  const int64_t total = (int64_t)in.B * ws.Lp * half;
  rope_table_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
      in.B, in.L, ws.Lp, half, log2(in.rope_theta), in.layout.tok_pos, ws.rope);
}

void launch_pack_any(int D, bool rope, int32_t B, int32_t L, int32_t Lp, int32_t H, const void *x,
                     const float2 *table, uint16_t *rows, uint16_t *trans, int32_t *exps,
                     hipStream_t s) {
  if (D == 64) launch_pack<64>(rope, B, L, Lp, H, x, table, rows, trans, exps, s);
  else launch_pack<128>(rope, B, L, Lp, H, x, table, rows, trans, exps, s);
}

void launch_delta(const opr_attn_in &in, const void *o, const void *dout, const float *lse,
                  const AttnWs &ws, hipStream_t s) {
  const int64_t total = (int64_t)in.B * ws.Lp;   // one wave per token
  const unsigned blocks = (unsigned)((total + 3) / 4);
  const uint16_t *o16 = static_cast<const uint16_t *>(o);
  const uint16_t *d16 = static_cast<const uint16_t *>(dout);
  if (in.D == 64)
    delta_kernel<64><<<blocks, 256, 0, s>>>(in.B, in.L, ws.Lp, in.Hq, o16, d16, lse, ws.delta, ws.lse2);
  else
    delta_kernel<128><<<blocks, 256, 0, s>>>(in.B, in.L, ws.Lp, in.Hq, o16, d16, lse, ws.delta, ws.lse2);
}

}  // namespace opr

// Forward kernel of the one-pass masked attention (gfx950).
//
// One workgroup of 4 waves per (128-query tile m, q head h, row b); wave w
// owns queries m*128 + 32w .. +31, one query per lane column.  The kernel walks
// the ascending list of non-empty 128-key tiles of q-tile m, half a tile (64
// keys) at a time, skipping halves whose 32x32 sub-blocks are all empty.  Per
// half: K (after RoPE) and V^T are staged in LDS; each wave computes
// S^T = K Q^T on its non-empty 32x32 sub-blocks with fp16 MFMA (fp32
// accumulate), applies the mask predicate only on partial sub-blocks, updates
// the online softmax (base-2 exponent with log2(e) folded into the scale) and
// accumulates O^T += V^T P^T.  The epilogue normalises, writes O (bf16) and
// the natural-log LSE.  Operands are fp16 with per-64-token exponents: the q
// and k exponents are folded into the score scale, the v exponent into the
// units of the O accumulator (rescaled together with the softmax correction).
#include "attn_common.h"
#include "opr_internal.h"

namespace opr {
namespace {

template <int D>
__global__ __launch_bounds__(256, 1) void attn_fwd_kernel(AttnParams p, uint16_t *o, float *lse) {
  constexpr int KS = D + 8;    // LDS row stride (elements) of the K tile
  constexpr int VS = 64 + 8;   // LDS row stride of the V^T tile
  constexpr int NS = D / 16;   // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;  // 32-wide blocks of the head dim
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vts[D * VS];
  __shared__ TokMeta kmeta[64];

  const int m = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int kvh = h / p.group;
  const int q = m * 128 + 32 * w + li;
  const int64_t row_base = (int64_t)b * p.L;

  const int nblk = p.Lp / 64;
  f16x8 qb[NS];
  {
    const uint16_t *qrow = p.qr + (((int64_t)b * p.Hq + h) * p.Lp + q) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) qb[s] = ld_f16x8(qrow + 16 * s + 8 * g);
  }
  const int eq = p.eq[((int64_t)b * p.Hq + h) * nblk + (q >> 6)];
  const int32_t *ekp = p.ek + ((int64_t)b * p.Hkv + kvh) * nblk;
  const int32_t *evp = p.ev + ((int64_t)b * p.Hkv + kvh) * nblk;
  int ev_ref = 0;  // O accumulator holds O * sum(p) * 2^(kPExp + ev_ref)
  const TokMeta qm = load_meta(p.tok_conv, p.tok_turn, p.tok_type, row_base, q, p.L);

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = zero_f32x16();
  float mrow = -INFINITY, lrow = 0.0f;

  const int64_t trow = (int64_t)b * p.MT + m;
  const int nnz = p.q_nnz[trow];
  const uint16_t *kbase = p.kr + ((int64_t)b * p.Hkv + kvh) * p.Lp * D;
  const uint16_t *vbase = p.vt + ((int64_t)b * p.Hkv + kvh) * D * p.Lp;

  for (int it = 0; it < nnz; ++it) {
    const int n = p.q_list[trow * p.NT + it];
    const uint32_t sub = p.sub_class[trow * p.NT + n];
#pragma unroll 1
    for (int kh = 0; kh < 2; ++kh) {
      if ((sub & (kh ? 0xF0F0F0F0u : 0x0F0F0F0Fu)) == 0) continue;
      const int k0 = n * 128 + 64 * kh;
      __syncthreads();
      // K tile: 64 rows x D, 16-byte chunks
#pragma unroll
      for (int c = tid; c < 64 * D / 8; c += 256) {
        const int r = c / (D / 8), ch = c % (D / 8);
        *reinterpret_cast<uint4 *>(&Ks[r * KS + ch * 8]) =
            *reinterpret_cast<const uint4 *>(kbase + (int64_t)(k0 + r) * D + ch * 8);
      }
      // V^T tile: D rows x 64 keys
#pragma unroll
      for (int c = tid; c < D * 8; c += 256) {
        const int r = c >> 3, ch = c & 7;
        *reinterpret_cast<uint4 *>(&Vts[r * VS + ch * 8]) =
            *reinterpret_cast<const uint4 *>(vbase + (int64_t)r * p.Lp + k0 + ch * 8);
      }
      if (tid < 64) kmeta[tid] = load_meta(p.tok_conv, p.tok_turn, p.tok_type, row_base, k0 + tid, p.L);
      __syncthreads();

      const uint32_t c0 = (sub >> (2 * (4 * w + 2 * kh))) & 3u;
      const uint32_t c1 = (sub >> (2 * (4 * w + 2 * kh + 1))) & 3u;
      if ((c0 | c1) == 0) continue;
      const uint32_t cls[2] = {c0, c1};
      const int ek = ekp[k0 >> 6], ev = evp[k0 >> 6];
      const float fs = ldexpf(p.scale_log2, -(eq + ek));

      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = zero_f32x16();
        if (cls[kb] == 0) continue;
        const uint16_t *arow = &Ks[(32 * kb + kperm(li)) * KS + 8 * g];
#pragma unroll
        for (int st = 0; st < NS; ++st) s[kb] = mfma32x32x16(ld_f16x8(arow + 16 * st), qb[st], s[kb]);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kb][r] * fs;
          if (cls[kb] == 0) {
            x = -INFINITY;
          } else if (cls[kb] == 1) {
            const int kl = 32 * kb + acc_row(r, g);
            if (!mask_allows(q, qm, k0 + kl, kmeta[kl])) x = -INFINITY;
          }
          s[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrow, mx);
      const float msafe = (mnew == -INFINITY) ? 0.0f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(mrow - msafe);
      const float ofac = ldexpf(alpha, ev - ev_ref);  // softmax correction and new v units
      mrow = mnew;
      ev_ref = ev;
      lrow *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= ofac;
      }
      const float mshift = msafe - (float)kPExp;
      f16x8 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(s[kb][r] - mshift);  // p * 2^kPExp
          lrow += pv;
          pb[kb][r >> 3][r & 7] = (_Float16)pv;
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (cls[kb] == 0) continue;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t *arow = &Vts[(32 * db + li) * VS + 32 * kb + 8 * g];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) oacc[db] = mfma32x32x16(ld_f16x8(arow + 16 * hh), pb[kb][hh], oacc[db]);
        }
      }
    }
  }

  const float lsum = lrow + __shfl_xor(lrow, 32);
  if (q < p.L) {
    const float inv = lsum > 0.0f ? ldexpf(1.0f / lsum, -ev_ref) : 0.0f;
    uint16_t *orow = o + ((row_base + q) * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint16_t v4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v4[c] = f32_to_bf16(oacc[db][4 * a + c] * inv);
        *reinterpret_cast<uint2 *>(orow + acc_dim(db, 4 * a, g)) = *reinterpret_cast<const uint2 *>(v4);
      }
    }
    if (g == 0)
      lse[((int64_t)b * p.Hq + h) * p.L + q] =
          lsum > 0.0f ? (mrow + log2f(lsum) - (float)kPExp) * kLn2 : -INFINITY;
  }
}

}  // namespace

void fill_params(const opr_attn_in &in, float scale, const AttnWs &ws, AttnParams *p);

hipError_t launch_attn_fwd_kernel(const opr_attn_in &in, float scale, void *o, float *lse,
                                  const AttnWs &ws, hipStream_t s) {
  AttnParams p;
  fill_params(in, scale, ws, &p);
  const dim3 grid(p.MT, in.Hq, in.B);
  uint16_t *o16 = static_cast<uint16_t *>(o);
  if (in.D == 64) attn_fwd_kernel<64><<<grid, 256, 0, s>>>(p, o16, lse);
  else attn_fwd_kernel<128><<<grid, 256, 0, s>>>(p, o16, lse);
  return hipGetLastError();
}

}  // namespace opr

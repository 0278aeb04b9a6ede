// Forward kernel of the one-pass masked attention (gfx950).
//
// One workgroup of 4 waves per (128-query tile m, q head h, row b); wave w
// owns queries m*128 + 32w .. +31, one query per lane column.  Work items are
// remapped so each XCD walks a contiguous range of (row, kv head, q-tile,
// head-in-group): the heads of one kv group and neighbouring q-tiles run side
// by side and share K/V tiles in that XCD's L2.
//
// The non-empty 64-key halves of the q-tile's non-empty 128-key tiles are
// first compacted into a stage list in LDS (a ballot over the tile list and
// its 32x32 sub-block classes), so the main loop has no dependent global
// loads.  Stages are double buffered: while stage i is computed, K and V of
// stage i+1 stream from memory straight into LDS (global_load_lds); one
// barrier per stage.  Per stage each wave computes S^T = K Q^T on its
// non-empty 32x32 sub-blocks with fp16 MFMA (fp32 accumulate), applies the
// mask predicate only on partial sub-blocks, updates the online softmax
// (base-2 exponent, log2(e) folded into the scale) and accumulates
// O^T += V^T P^T, reading V^T from the row-major V tile with transposing LDS
// reads.  The epilogue normalises, writes O (bf16) and the natural-log LSE.
// Operands are fp16 with per-64-token exponents: the q and k exponents are
// folded into the score scale, the v exponent into the units of the O
// accumulator (rescaled together with the softmax correction).
#include "attn_common.h"
#include "attn_sched.h"
#include "opr_internal.h"

namespace opr {
namespace {

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnParams p, uint16_t *o, float *lse) {
  constexpr int NS = D / 16;   // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;  // 32-wide blocks of the head dim
  constexpr int TB = Tile<D>::BYTES;
  // per buffer: K tile, V tile, 64 key records
  constexpr int BUF = 2 * TB + 512;
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUF];
  __shared__ uint2 stages[kStageCap];
  __shared__ int sh_count, sh_next;

  const int64_t nitems = (int64_t)p.B * p.Hq * p.MT;
  const int64_t u = xcd_work_item(nitems);
  if (u >= nitems) return;
  const int j = (int)(u % p.group);
  int64_t rest = u / p.group;
  const int m = (int)(rest % p.MT);
  rest /= p.MT;
  const int kvh = (int)(rest % p.Hkv);
  const int b = (int)(rest / p.Hkv);
  const int h = kvh * p.group + j;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int q = m * 128 + 32 * w + li;
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
  const int2 qmi = p.meta[(int64_t)b * p.Lp + q];
  const TokMeta qm = {qmi.x, qmi.y};
  int ev_ref = 0;  // the O accumulator holds O * sum(p) * 2^(kPExp + ev_ref)

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = zero_f32x16();
  float mrow = -INFINITY, lrow = 0.0f;

  const int64_t trow = (int64_t)b * p.MT + m;
  const int nnz = p.q_nnz[trow];
  const int32_t *lst = p.q_list + trow * p.NT;
  const uint32_t *subs = p.sub_class + trow * p.NT;
  const int64_t kvoff = ((int64_t)b * p.Hkv + kvh) * p.Lp;
  const uint16_t *kbase = p.kr + kvoff * D;
  const uint16_t *vbase = p.vr + kvoff * D;
  const int2 *mbase = p.meta + (int64_t)b * p.Lp;

  int tnext = 0;
  while (tnext < nnz) {
    __syncthreads();  // previous chunk's stages and buffers are no longer read
    if (w == 0) {
      int t = tnext;
      const int c = build_q_stages(lst, subs, ekp, evp, nnz, &t, stages, lane);
      if (lane == 0) {
        sh_count = c;
        sh_next = t;
      }
    }
    __syncthreads();
    const int ns = sh_count;
    tnext = sh_next;
    if (ns == 0) continue;
    {
      const int k0 = (int)stages[0].x;
      tile_load_async<D>(kbase + (int64_t)k0 * D, smem, w, lane);
      tile_load_async<D>(vbase + (int64_t)k0 * D, smem + TB, w, lane);
      if (w == 0) rec8_load_async(mbase + k0, smem + 2 * TB, lane);
    }
    for (int i = 0; i < ns; ++i) {
      wait_all_and_barrier();
      const char *buf = smem + (i & 1) * BUF;
      if (i + 1 < ns) {
        char *nb = smem + ((i + 1) & 1) * BUF;
        const int k1 = (int)stages[i + 1].x;
        tile_load_async<D>(kbase + (int64_t)k1 * D, nb, w, lane);
        tile_load_async<D>(vbase + (int64_t)k1 * D, nb + TB, w, lane);
        if (w == 0) rec8_load_async(mbase + k1, nb + 2 * TB, lane);
      }
      const uint2 desc = stages[i];
      const uint32_t c0 = (desc.y >> (4 * w)) & 3u, c1 = (desc.y >> (4 * w + 2)) & 3u;
      if ((c0 | c1) == 0) continue;
      const uint32_t cls[2] = {c0, c1};
      const int k0 = (int)desc.x;
      const int ek = (int)((desc.y >> 16) & 255u) - 128, ev = (int)(desc.y >> 24) - 128;
      const float fs = ldexpf(p.scale_log2, -(eq + ek));
      const char *Kt = buf, *Vt = buf + TB;
      const int2 *kmeta = reinterpret_cast<const int2 *>(buf + 2 * TB);

      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = zero_f32x16();
        if (cls[kb] == 0) continue;
        const int r = 32 * kb + kperm(li);
#pragma unroll
        for (int st = 0; st < NS; ++st) s[kb] = mfma32x32x16(tile_row8<D>(Kt, r, 2 * st + g), qb[st], s[kb]);
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
            const int2 km = kmeta[kl];
            if (!mask_allows(q, qm, k0 + kl, TokMeta{km.x, km.y})) x = -INFINITY;
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
      for (int db = 0; db < NDB; ++db) oacc[db] *= ofac;
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
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            oacc[db] = mfma32x32x16(tile_col8<D>(Vt, 32 * kb + 16 * hh, 32 * db, lane), pb[kb][hh], oacc[db]);
        }
      }
    }
  }

  const float lsum = lrow + __shfl_xor(lrow, 32);
  if (q < p.L) {
    const float inv = lsum > 0.0f ? ldexpf(1.0f / lsum, -ev_ref) : 0.0f;
    uint16_t *orow = o + (((int64_t)b * p.L + q) * p.Hq + h) * D;
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
  const int64_t nitems = (int64_t)in.B * in.Hq * p.MT;
  const unsigned grid = (unsigned)(8 * ((nitems + 7) / 8));
  uint16_t *o16 = static_cast<uint16_t *>(o);
  if (in.D == 64) attn_fwd_kernel<64><<<grid, 256, 0, s>>>(p, o16, lse);
  else attn_fwd_kernel<128><<<grid, 256, 0, s>>>(p, o16, lse);
  return hipGetLastError();
}

}  // namespace opr

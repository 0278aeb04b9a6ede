// Backward kernels of the one-pass masked attention (gfx950).
//
// With P recomputed from the forward LSE (P = exp2(scale*log2(e)*S - lse2)),
//   dV  = sum over the group's q heads of P^T dO
//   dP  = dO V^T,  dS = P * (dP - delta),  delta = rowsum(dO * O)
//   dQ' = scale * dS K',  dK' = scale * sum over the group of dS^T Q'
// and dQ, dK are rotated back by the transposed RoPE rotation.
//
// attn_dkdv_kernel: one workgroup per (128-key tile n, kv head, row); wave w
//   owns keys n*128 + 32w .. +31, one key per lane column, K' and V of its
//   key in registers.  Its stages are (q-tile of k_list, head of the group,
//   64-query half) with a non-empty sub-block; each streams the Q' and dO rows
//   of the stage into LDS (double buffered, global_load_lds) and reads Q'^T
//   and dO^T from the same row-major tiles with transposing LDS reads.
//   dK^T and dV^T stay in accumulators; each key is owned by exactly one
//   workgroup: no atomics.
// attn_dq_kernel: one workgroup per (128-query tile, q head, row), pipelined
//   like the forward kernel over the K' / V tiles; S and dP^T are recomputed
//   per non-empty sub-block and dQ^T += K'^T dS^T (K'^T from the K' tile).
// Work items are remapped so each XCD walks a contiguous range (shared tiles
// stay in that XCD's L2).
//
// Operands are fp16 with per-64-token exponents (q, k, v, dout); P is stored
// as fp16(P * 2^kPExp) and dS in the units of dP (2^(e_v + e_dout)) shifted
// down by 2^kDsShift.  The accumulators carry power-of-two units that are
// rescaled whenever a block with other exponents arrives, and removed in the
// epilogue.
#include "attn_common.h"
#include "attn_sched.h"
#include "opr_internal.h"

namespace opr {
namespace {

template <int D>
__global__ __launch_bounds__(256, 1) void attn_dkdv_kernel(AttnParams p, float *dk, float *dv) {
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int HALF_DB = NDB / 2;
  constexpr int TB = Tile<D>::BYTES;
  // per buffer: Q' tile, dO tile, lse2[64], delta[64], 64 query records
  constexpr int BUF = 2 * TB + 1024;
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUF];
  __shared__ uint2 stages[kStageCap];
  __shared__ int sh_count;
  __shared__ int64_t sh_next;

  const int64_t nitems = (int64_t)p.B * p.Hkv * p.NT;
  const int64_t u = xcd_work_item(nitems);
  if (u >= nitems) return;
  const int n = (int)(u % p.NT);
  const int kvh = (int)((u / p.NT) % p.Hkv);
  const int b = (int)(u / ((int64_t)p.NT * p.Hkv));

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int key = n * 128 + 32 * w + li;
  const int nblk = p.Lp / 64;

  f16x8 kb_[NS], vb_[NS];
  {
    const int64_t off = (((int64_t)b * p.Hkv + kvh) * p.Lp + key) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kb_[s] = ld_f16x8(p.kr + off + 16 * s + 8 * g);
      vb_[s] = ld_f16x8(p.vr + off + 16 * s + 8 * g);
    }
  }
  const int ek = p.ek[((int64_t)b * p.Hkv + kvh) * nblk + (key >> 6)];
  const int ev = p.ev[((int64_t)b * p.Hkv + kvh) * nblk + (key >> 6)];
  // dV^T accumulator units 2^(kPExp + uv), dK^T units 2^(uk + ev - kDsShift)
  int uv = 0, uk = 0;
  const int2 kmi = p.meta[(int64_t)b * p.Lp + key];
  const TokMeta km = {kmi.x, kmi.y};

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dkacc[db] = zero_f32x16();
    dvacc[db] = zero_f32x16();
  }

  const int64_t tcol = (int64_t)b * p.NT + n;
  const int nnz = p.k_nnz[tcol];
  const int32_t *lst = p.k_list + tcol * p.MT;
  const uint32_t *subs_b = p.sub_class + (int64_t)b * p.MT * p.NT;
  const int64_t hbase = (int64_t)b * p.Hq + (int64_t)kvh * p.group;  // first head of the group
  const int32_t *eqp = p.eq + hbase * nblk;
  const int32_t *edop = p.edo + hbase * nblk;
  const int2 *mbase = p.meta + (int64_t)b * p.Lp;

  auto issue = [&](uint32_t x, char *nb) {
    const int q0 = (int)(x & 0xFFFFFFu), hj = (int)(x >> 24);
    const int64_t row = (hbase + hj) * p.Lp + q0;
    tile_load_async<D>(p.qr + row * D, nb, w, lane);
    tile_load_async<D>(p.dor + row * D, nb + TB, w, lane);
    if (w == 0) {
      f32x64_load_async(p.lse2 + row, nb + 2 * TB, lane);
    } else if (w == 1) {
      f32x64_load_async(p.delta + row, nb + 2 * TB + 256, lane);
    } else if (w == 2) {
      rec8_load_async(mbase + q0, nb + 2 * TB + 512, lane);
    }
  };

  int64_t fnext = 0;
  const int64_t ftotal = (int64_t)nnz * p.group * 2;
  while (fnext < ftotal) {
    __syncthreads();
    if (w == 0) {
      int64_t f = fnext;
      const int c = build_k_stages(lst, subs_b, p.NT, n, p.group, eqp, edop, nblk, nnz, &f, stages, lane);
      if (lane == 0) {
        sh_count = c;
        sh_next = f;
      }
    }
    __syncthreads();
    const int ns = sh_count;
    fnext = sh_next;
    if (ns == 0) continue;
    issue(stages[0].x, smem);
    for (int i = 0; i < ns; ++i) {
      wait_all_and_barrier();
      const char *buf = smem + (i & 1) * BUF;
      if (i + 1 < ns) issue(stages[i + 1].x, smem + ((i + 1) & 1) * BUF);
      const uint2 desc = stages[i];
      const uint32_t c0 = (desc.y >> (4 * w)) & 3u, c1 = (desc.y >> (4 * w + 2)) & 3u;
      if ((c0 | c1) == 0) continue;
      const uint32_t cls[2] = {c0, c1};
      const int q0 = (int)(desc.x & 0xFFFFFFu);
      const int eq = (int)((desc.y >> 16) & 255u) - 128, edo = (int)(desc.y >> 24) - 128;
      const float fs = ldexpf(p.scale_log2, -(eq + ek));
      const int udp = ev + edo;  // units of dP
      const char *Qt = buf, *dOt = buf + TB;
      const float *lse2s = reinterpret_cast<const float *>(buf + 2 * TB);
      const float *deltas = reinterpret_cast<const float *>(buf + 2 * TB + 256);
      const int2 *qmeta = reinterpret_cast<const int2 *>(buf + 2 * TB + 512);

      f16x8 pb[2][2], dsb[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (cls[qb] == 0) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) pb[qb][hh] = dsb[qb][hh] = zero_f16x8();
          continue;
        }
        f32x16 s = zero_f32x16(), dp = zero_f32x16();
        const int r = 32 * qb + kperm(li);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          s = mfma32x32x16(tile_row8<D>(Qt, r, 2 * st + g), kb_[st], s);
          dp = mfma32x32x16(tile_row8<D>(dOt, r, 2 * st + g), vb_[st], dp);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int ql = 32 * qb + acc_row(rr, g);
          const float x = s[rr] * fs - lse2s[ql];
          float pv = __builtin_amdgcn_exp2f(x);
          float ps = __builtin_amdgcn_exp2f(x + (float)kPExp);
          if (cls[qb] == 1) {
            const int2 qm = qmeta[ql];
            if (!mask_allows(q0 + ql, TokMeta{qm.x, qm.y}, key, km)) pv = ps = 0.0f;
          }
          const float ds = ldexpf(pv * (dp[rr] - ldexpf(deltas[ql], udp)), -kDsShift);
          pb[qb][rr >> 3][rr & 7] = (_Float16)ps;
          dsb[qb][rr >> 3][rr & 7] = (_Float16)ds;
        }
      }
      if (edo != uv) {
        const float f = ldexpf(1.0f, edo - uv);
#pragma unroll
        for (int db = 0; db < NDB; ++db) dvacc[db] *= f;
        uv = edo;
      }
      if (eq + edo != uk) {
        const float f = ldexpf(1.0f, eq + edo - uk);
#pragma unroll
        for (int db = 0; db < NDB; ++db) dkacc[db] *= f;
        uk = eq + edo;
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (cls[qb] == 0) continue;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            dvacc[db] = mfma32x32x16(tile_col8<D>(dOt, 32 * qb + 16 * hh, 32 * db, lane), pb[qb][hh], dvacc[db]);
            dkacc[db] = mfma32x32x16(tile_col8<D>(Qt, 32 * qb + 16 * hh, 32 * db, lane), dsb[qb][hh], dkacc[db]);
          }
        }
      }
    }
  }

  if (key < p.L) {
    const int64_t out = (((int64_t)b * p.L + key) * p.Hkv + kvh) * D;
    const float2 *cs = p.rope + ((int64_t)b * p.Lp + key) * (D / 2);
    const float kscale = ldexpf(p.scale, kDsShift - uk - ev);
    const float vscale = ldexpf(1.0f, -kPExp - uv);
#pragma unroll
    for (int db = 0; db < HALF_DB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float lo[4], hi[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = 4 * a + c;
          const float2 rc = cs[acc_dim(db, r, g)];
          const float g1 = kscale * dkacc[db][r], g2 = kscale * dkacc[db + HALF_DB][r];
          lo[c] = g1 * rc.x + g2 * rc.y;
          hi[c] = g2 * rc.x - g1 * rc.y;
        }
        *reinterpret_cast<float4 *>(dk + out + acc_dim(db, 4 * a, g)) = make_float4(lo[0], lo[1], lo[2], lo[3]);
        *reinterpret_cast<float4 *>(dk + out + acc_dim(db + HALF_DB, 4 * a, g)) = make_float4(hi[0], hi[1], hi[2], hi[3]);
      }
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4 *>(dv + out + acc_dim(db, 4 * a, g)) =
            make_float4(vscale * dvacc[db][4 * a], vscale * dvacc[db][4 * a + 1],
                        vscale * dvacc[db][4 * a + 2], vscale * dvacc[db][4 * a + 3]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256, 1) void attn_dq_kernel(AttnParams p, float *dq) {
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int HALF_DB = NDB / 2;
  constexpr int TB = Tile<D>::BYTES;
  constexpr int BUF = 2 * TB + 512;  // K' tile, V tile, 64 key records
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
  const int64_t hq_row = ((int64_t)b * p.Hq + h) * p.Lp + q;

  f16x8 qb[NS], dob[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qb[s] = ld_f16x8(p.qr + hq_row * D + 16 * s + 8 * g);
    dob[s] = ld_f16x8(p.dor + hq_row * D + 16 * s + 8 * g);
  }
  const float lse2_q = p.lse2[hq_row];
  const float delta_q = p.delta[hq_row];
  const int eq = p.eq[((int64_t)b * p.Hq + h) * nblk + (q >> 6)];
  const int edo = p.edo[((int64_t)b * p.Hq + h) * nblk + (q >> 6)];
  const int32_t *ekp = p.ek + ((int64_t)b * p.Hkv + kvh) * nblk;
  const int32_t *evp = p.ev + ((int64_t)b * p.Hkv + kvh) * nblk;
  const int2 qmi = p.meta[(int64_t)b * p.Lp + q];
  const TokMeta qm = {qmi.x, qmi.y};
  int uq = 0;  // dQ^T accumulator units 2^(uq + edo - kDsShift), uq = e_k + e_v of the block

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = zero_f32x16();

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
    __syncthreads();
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
      const float dd = ldexpf(delta_q, ev + edo);  // delta in the units of dP
      const char *Kt = buf, *Vt = buf + TB;
      const int2 *kmeta = reinterpret_cast<const int2 *>(buf + 2 * TB);

      f16x8 dsb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (cls[kb] == 0) {
          dsb[kb][0] = dsb[kb][1] = zero_f16x8();
          continue;
        }
        f32x16 s = zero_f32x16(), dpt = zero_f32x16();
        const int r = 32 * kb + kperm(li);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          s = mfma32x32x16(tile_row8<D>(Kt, r, 2 * st + g), qb[st], s);
          dpt = mfma32x32x16(tile_row8<D>(Vt, r, 2 * st + g), dob[st], dpt);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int kl = 32 * kb + acc_row(rr, g);
          float pv = __builtin_amdgcn_exp2f(s[rr] * fs - lse2_q);
          if (cls[kb] == 1) {
            const int2 kmv = kmeta[kl];
            if (!mask_allows(q, qm, k0 + kl, TokMeta{kmv.x, kmv.y})) pv = 0.0f;
          }
          dsb[kb][rr >> 3][rr & 7] = (_Float16)ldexpf(pv * (dpt[rr] - dd), -kDsShift);
        }
      }
      if (ek + ev != uq) {
        const float f = ldexpf(1.0f, ek + ev - uq);
#pragma unroll
        for (int db = 0; db < NDB; ++db) dqacc[db] *= f;
        uq = ek + ev;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (cls[kb] == 0) continue;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            dqacc[db] = mfma32x32x16(tile_col8<D>(Kt, 32 * kb + 16 * hh, 32 * db, lane), dsb[kb][hh], dqacc[db]);
        }
      }
    }
  }

  if (q < p.L) {
    float *out = dq + (((int64_t)b * p.L + q) * p.Hq + h) * D;
    const float2 *cs = p.rope + ((int64_t)b * p.Lp + q) * (D / 2);
    const float qscale = ldexpf(p.scale, kDsShift - uq - edo);
#pragma unroll
    for (int db = 0; db < HALF_DB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float lo[4], hi[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = 4 * a + c;
          const float2 rc = cs[acc_dim(db, r, g)];
          const float g1 = qscale * dqacc[db][r], g2 = qscale * dqacc[db + HALF_DB][r];
          lo[c] = g1 * rc.x + g2 * rc.y;
          hi[c] = g2 * rc.x - g1 * rc.y;
        }
        *reinterpret_cast<float4 *>(out + acc_dim(db, 4 * a, g)) = make_float4(lo[0], lo[1], lo[2], lo[3]);
        *reinterpret_cast<float4 *>(out + acc_dim(db + HALF_DB, 4 * a, g)) = make_float4(hi[0], hi[1], hi[2], hi[3]);
      }
    }
  }
}

}  // namespace

void fill_params(const opr_attn_in &in, float scale, const AttnWs &ws, AttnParams *p);

// ev (optional): events recorded before dK/dV, before dQ and after dQ.
hipError_t launch_attn_bwd_kernels(const opr_attn_in &in, float scale, float *dq, float *dk,
                                   float *dv, const AttnWs &ws, hipStream_t s, hipEvent_t *ev) {
  AttnParams p;
  fill_params(in, scale, ws, &p);
  const int64_t nk = (int64_t)in.B * in.Hkv * p.NT, nq = (int64_t)in.B * in.Hq * p.MT;
  const unsigned gk = (unsigned)(8 * ((nk + 7) / 8)), gq = (unsigned)(8 * ((nq + 7) / 8));
  if (ev) hipEventRecord(ev[0], s);
  if (in.D == 64) attn_dkdv_kernel<64><<<gk, 256, 0, s>>>(p, dk, dv);
  else attn_dkdv_kernel<128><<<gk, 256, 0, s>>>(p, dk, dv);
  if (ev) hipEventRecord(ev[1], s);
  if (in.D == 64) attn_dq_kernel<64><<<gq, 256, 0, s>>>(p, dq);
  else attn_dq_kernel<128><<<gq, 256, 0, s>>>(p, dq);
  if (ev) hipEventRecord(ev[2], s);
  return hipGetLastError();
}

}  // namespace opr

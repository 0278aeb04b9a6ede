// Backward kernels of the one-pass masked attention (gfx950).
//
// With P recomputed from the forward LSE (P = exp2(scale*log2(e)*S - lse2)),
//   dV  = sum over the group's q heads of P^T dO
//   dP  = dO V^T,  dS = P * (dP - delta),  delta = rowsum(dO * O)
//   dQ' = scale * dS K',  dK' = scale * sum over the group of dS^T Q'
// and dQ, dK are rotated back by the transposed RoPE rotation.
//
// attn_dkdv_kernel: one workgroup per (128-key tile n, kv head, row); wave w
//   owns keys n*128 + 32w .. +31, one key per lane column, K' and V of its key
//   in registers.  It walks the ascending list of non-empty q-tiles of k-tile
//   n, for every q head of the group, 64 queries at a time (Q', dO and their
//   transposes staged in LDS), and keeps dK^T, dV^T in accumulators.  Each key
//   is owned by exactly one workgroup: no atomics.
// attn_dq_kernel: one workgroup per (128-query tile, q head, row), like the
//   forward kernel; S and dP^T are recomputed per non-empty sub-block and
//   dQ^T += K'^T dS^T.
// Operands are fp16 with per-64-token exponents (q, k, v, dout); P is stored
// as fp16(P * 2^kPExp) and dS in the units of dP (2^(e_v + e_dout)) shifted
// down by 2^kDsShift.  The accumulators carry power-of-two units that are
// rescaled whenever a block with other exponents arrives, and removed in the
// epilogue.
#include "attn_common.h"
#include "opr_internal.h"

namespace opr {
namespace {

template <int D>
__global__ __launch_bounds__(256, 1) void attn_dkdv_kernel(AttnParams p, float *dk, float *dv) {
  constexpr int RS = D + 8;    // LDS row stride of row-major tiles
  constexpr int TS = 64 + 8;   // LDS row stride of transposed tiles
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int HALF_DB = NDB / 2;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[64 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[64 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Qts[D * TS];
  __shared__ __attribute__((aligned(16))) uint16_t dOts[D * TS];
  __shared__ __attribute__((aligned(16))) float lse2s[64];
  __shared__ __attribute__((aligned(16))) float deltas[64];
  __shared__ TokMeta qmeta[64];

  const int n = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int key = n * 128 + 32 * w + li;
  const int64_t row_base = (int64_t)b * p.L;

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
  const TokMeta km = load_meta(p.tok_conv, p.tok_turn, p.tok_type, row_base, key, p.L);

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dkacc[db] = zero_f32x16();
    dvacc[db] = zero_f32x16();
  }

  const int64_t tcol = (int64_t)b * p.NT + n;
  const int nnz = p.k_nnz[tcol];
  for (int it = 0; it < nnz; ++it) {
    const int m = p.k_list[tcol * p.MT + it];
    const uint32_t sub = p.sub_class[((int64_t)b * p.MT + m) * p.NT + n];
#pragma unroll 1
    for (int hq = 0; hq < p.group; ++hq) {
      const int h = kvh * p.group + hq;
      const int64_t hrow = ((int64_t)b * p.Hq + h) * p.Lp;   // row index base in [B][Hq][Lp]
#pragma unroll 1
      for (int qh = 0; qh < 2; ++qh) {
        if ((sub & (qh ? 0xFFFF0000u : 0x0000FFFFu)) == 0) continue;
        const int q0 = m * 128 + 64 * qh;
        __syncthreads();
#pragma unroll
        for (int c = tid; c < 64 * D / 8; c += 256) {
          const int r = c / (D / 8), ch = c % (D / 8);
          const int64_t src = (hrow + q0 + r) * D + ch * 8;
          *reinterpret_cast<uint4 *>(&Qs[r * RS + ch * 8]) = *reinterpret_cast<const uint4 *>(p.qr + src);
          *reinterpret_cast<uint4 *>(&dOs[r * RS + ch * 8]) = *reinterpret_cast<const uint4 *>(p.dor + src);
        }
#pragma unroll
        for (int c = tid; c < D * 8; c += 256) {
          const int r = c >> 3, ch = c & 7;
          const int64_t src = (hrow * D) + (int64_t)r * p.Lp + q0 + ch * 8;  // [B][Hq][D][Lp]
          *reinterpret_cast<uint4 *>(&Qts[r * TS + ch * 8]) = *reinterpret_cast<const uint4 *>(p.qt + src);
          *reinterpret_cast<uint4 *>(&dOts[r * TS + ch * 8]) = *reinterpret_cast<const uint4 *>(p.dot + src);
        }
        if (tid < 64) {
          lse2s[tid] = p.lse2[hrow + q0 + tid];
          deltas[tid] = p.delta[hrow + q0 + tid];
          qmeta[tid] = load_meta(p.tok_conv, p.tok_turn, p.tok_type, row_base, q0 + tid, p.L);
        }
        __syncthreads();

        const uint32_t c0 = (sub >> (2 * (4 * (2 * qh) + w))) & 3u;
        const uint32_t c1 = (sub >> (2 * (4 * (2 * qh + 1) + w))) & 3u;
        if ((c0 | c1) == 0) continue;
        const uint32_t cls[2] = {c0, c1};
        const int eq = p.eq[((int64_t)b * p.Hq + h) * nblk + (q0 >> 6)];
        const int edo = p.edo[((int64_t)b * p.Hq + h) * nblk + (q0 >> 6)];
        const float fs = ldexpf(p.scale_log2, -(eq + ek));
        const int udp = ev + edo;  // units of dP

        f16x8 pb[2][2], dsb[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (cls[qb] == 0) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) pb[qb][hh] = dsb[qb][hh] = zero_f16x8();
            continue;
          }
          f32x16 s = zero_f32x16(), dp = zero_f32x16();
          const int arow = (32 * qb + kperm(li)) * RS + 8 * g;
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            s = mfma32x32x16(ld_f16x8(&Qs[arow + 16 * st]), kb_[st], s);
            dp = mfma32x32x16(ld_f16x8(&dOs[arow + 16 * st]), vb_[st], dp);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = 32 * qb + acc_row(r, g);
            const float x = s[r] * fs - lse2s[ql];
            float pv = __builtin_amdgcn_exp2f(x);
            float ps = __builtin_amdgcn_exp2f(x + (float)kPExp);
            if (cls[qb] == 1 && !mask_allows(q0 + ql, qmeta[ql], key, km)) pv = ps = 0.0f;
            const float ds = ldexpf(pv * (dp[r] - ldexpf(deltas[ql], udp)), -kDsShift);
            pb[qb][r >> 3][r & 7] = (_Float16)ps;
            dsb[qb][r >> 3][r & 7] = (_Float16)ds;
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
          for (int db = 0; db < NDB; ++db) {
            const int arow = (32 * db + li) * TS + 32 * qb + 8 * g;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              dvacc[db] = mfma32x32x16(ld_f16x8(&dOts[arow + 16 * hh]), pb[qb][hh], dvacc[db]);
              dkacc[db] = mfma32x32x16(ld_f16x8(&Qts[arow + 16 * hh]), dsb[qb][hh], dkacc[db]);
            }
          }
        }
      }
    }
  }

  if (key < p.L) {
    const int64_t out = ((row_base + key) * p.Hkv + kvh) * D;
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
  constexpr int RS = D + 8;
  constexpr int TS = 64 + 8;
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int HALF_DB = NDB / 2;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Kts[D * TS];
  __shared__ TokMeta kmeta[64];

  const int m = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int kvh = h / p.group;
  const int q = m * 128 + 32 * w + li;
  const int64_t row_base = (int64_t)b * p.L;
  const int64_t hq_row = ((int64_t)b * p.Hq + h) * p.Lp + q;

  const int nblk = p.Lp / 64;
  f16x8 qb[NS], dob[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qb[s] = ld_f16x8(p.qr + hq_row * D + 16 * s + 8 * g);
    dob[s] = ld_f16x8(p.dor + hq_row * D + 16 * s + 8 * g);
  }
  const int eq = p.eq[((int64_t)b * p.Hq + h) * nblk + (q >> 6)];
  const int edo = p.edo[((int64_t)b * p.Hq + h) * nblk + (q >> 6)];
  const int32_t *ekp = p.ek + ((int64_t)b * p.Hkv + kvh) * nblk;
  const int32_t *evp = p.ev + ((int64_t)b * p.Hkv + kvh) * nblk;
  int uq = 0;  // dQ^T accumulator units 2^(uq + edo - kDsShift), uq = e_k + e_v of the block
  const float lse2_q = p.lse2[hq_row];
  const float delta_q = p.delta[hq_row];
  const TokMeta qm = load_meta(p.tok_conv, p.tok_turn, p.tok_type, row_base, q, p.L);

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = zero_f32x16();

  const int64_t trow = (int64_t)b * p.MT + m;
  const int nnz = p.q_nnz[trow];
  const int64_t kvrow = ((int64_t)b * p.Hkv + kvh) * p.Lp;
  for (int it = 0; it < nnz; ++it) {
    const int n = p.q_list[trow * p.NT + it];
    const uint32_t sub = p.sub_class[trow * p.NT + n];
#pragma unroll 1
    for (int kh = 0; kh < 2; ++kh) {
      if ((sub & (kh ? 0xF0F0F0F0u : 0x0F0F0F0Fu)) == 0) continue;
      const int k0 = n * 128 + 64 * kh;
      __syncthreads();
#pragma unroll
      for (int c = tid; c < 64 * D / 8; c += 256) {
        const int r = c / (D / 8), ch = c % (D / 8);
        const int64_t src = (kvrow + k0 + r) * D + ch * 8;
        *reinterpret_cast<uint4 *>(&Ks[r * RS + ch * 8]) = *reinterpret_cast<const uint4 *>(p.kr + src);
        *reinterpret_cast<uint4 *>(&Vs[r * RS + ch * 8]) = *reinterpret_cast<const uint4 *>(p.vr + src);
      }
#pragma unroll
      for (int c = tid; c < D * 8; c += 256) {
        const int r = c >> 3, ch = c & 7;
        *reinterpret_cast<uint4 *>(&Kts[r * TS + ch * 8]) =
            *reinterpret_cast<const uint4 *>(p.kt + kvrow * D + (int64_t)r * p.Lp + k0 + ch * 8);
      }
      if (tid < 64) kmeta[tid] = load_meta(p.tok_conv, p.tok_turn, p.tok_type, row_base, k0 + tid, p.L);
      __syncthreads();

      const uint32_t c0 = (sub >> (2 * (4 * w + 2 * kh))) & 3u;
      const uint32_t c1 = (sub >> (2 * (4 * w + 2 * kh + 1))) & 3u;
      if ((c0 | c1) == 0) continue;
      const uint32_t cls[2] = {c0, c1};
      const int ek = ekp[k0 >> 6], ev = evp[k0 >> 6];
      const float fs = ldexpf(p.scale_log2, -(eq + ek));
      const float dd = ldexpf(delta_q, ev + edo);  // delta in the units of dP

      f16x8 dsb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (cls[kb] == 0) {
          dsb[kb][0] = dsb[kb][1] = zero_f16x8();
          continue;
        }
        f32x16 s = zero_f32x16(), dpt = zero_f32x16();
        const int arow = (32 * kb + kperm(li)) * RS + 8 * g;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          s = mfma32x32x16(ld_f16x8(&Ks[arow + 16 * st]), qb[st], s);
          dpt = mfma32x32x16(ld_f16x8(&Vs[arow + 16 * st]), dob[st], dpt);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = 32 * kb + acc_row(r, g);
          float pv = __builtin_amdgcn_exp2f(s[r] * fs - lse2_q);
          if (cls[kb] == 1 && !mask_allows(q, qm, k0 + kl, kmeta[kl])) pv = 0.0f;
          dsb[kb][r >> 3][r & 7] = (_Float16)ldexpf(pv * (dpt[r] - dd), -kDsShift);
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
        for (int db = 0; db < NDB; ++db) {
          const int arow = (32 * db + li) * TS + 32 * kb + 8 * g;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) dqacc[db] = mfma32x32x16(ld_f16x8(&Kts[arow + 16 * hh]), dsb[kb][hh], dqacc[db]);
        }
      }
    }
  }

  if (q < p.L) {
    float *out = dq + ((row_base + q) * p.Hq + h) * D;
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
  const dim3 gk(p.NT, in.Hkv, in.B), gq(p.MT, in.Hq, in.B);
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

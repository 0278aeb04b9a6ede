// dQ kernel of the one-pass masked attention backward (gfx950).
//
// One workgroup per (128-query tile, q head, row), pipelined like the forward
// kernel: a stage list of the non-empty 64-key halves in LDS, K' and V tiles
// double buffered in LDS (buffer loads to LDS), one barrier per stage.  Per
// non-empty 32x32 sub-block each wave recomputes S^T = K' Q'^T and
// dP^T = V dO^T, masks partial sub-blocks with the query's key intervals,
// forms dS = P * (dP - delta) (P from the forward LSE) and accumulates
// dQ^T += K'^T dS^T, reading K'^T from the row-major K' tile with transposing
// LDS reads.  The epilogue removes the operand units, applies the softmax
// scale and rotates dQ back by the transposed RoPE rotation.
//
// Units: q' and dout carry one exponent per 16-slot tile and q head (one per
// lane's query), k' and v one per (row, kv head).  dP comes out in units
// 2^(e_dout + e_v); delta is brought into those units times 2^-kDsShift, and
// dS is formed as P * (dP * 2^-kDsShift - delta) before the fp16 conversion.
#include "attn_common.h"
#include "attn_sched.h"
#include "opr_internal.h"

namespace opr {
namespace {

constexpr int kReadsAhead = 4;  // S / dP products whose K' / V operand reads are in flight

template <int D>
__global__ __launch_bounds__(256, 2) void attn_dq_kernel(AttnParams p, float *dq) {
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int HALF_DB = NDB / 2;
  constexpr int TB = Tile<D>::BYTES, RB = Tile<D>::RB;
  constexpr int BUF = 2 * TB;  // K' tile, V tile
  // two separate LDS objects so the copy into one provably leaves the other alone
  __shared__ __attribute__((aligned(1024))) char buf0[BUF];
  __shared__ __attribute__((aligned(1024))) char buf1[BUF];
  __shared__ uint2 stages[kStageCap];
  __shared__ int sh_count, sh_next;

  const QItem it = q_work_item(p.q_order, p.MT, p.Hkv, p.group, (int64_t)p.B * p.MT);
  if (!it.valid) return;
  const int j = it.j, m = it.m, kvh = it.kvh, b = it.b;
  const int h = kvh * p.group + j;

  const int tid = threadIdx.x, w = uniform(tid >> 6), lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int q = m * 128 + 32 * w + li;
  const int64_t kvplane = (int64_t)b * p.Hkv + kvh;
  // q' and dout scales of the lane's tile (query slot q), and their kv-group minima
  const int64_t tix = ((int64_t)b * p.Hq + h) * p.MTS + q / kTile;
  const int eq = p.eqt[tix], edo = p.edot[tix];
  const int eqr = p.eref[2 * kvplane], edor = p.eref[2 * kvplane + 1];
  const int ek = plane_exponent(p.mk[kvplane]);
  const int ev = plane_exponent(p.mv[kvplane]);
  const float fs = ldexpf(p.scale_log2, -(eq + ek));
  const float dss = ldexpf(1.0f, -kDsShift);
  const int64_t hq_row = ((int64_t)b * p.Hq + h) * p.Lp + q;

  f16x8 qb[NS], dob[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qb[s] = ld_f16x8(p.qr + hq_row * D + 16 * s + 8 * g);
    dob[s] = ld_f16x8(p.dor + hq_row * D + 16 * s + 8 * g);
  }
  // the stored lse2 and delta are in the dK/dV kernel's units: undo them
  const float lse2_q = p.lse2[hq_row] + (float)(kPdvExp - (edo - edor));
  const float dsc_q = ldexpf(p.dsc[hq_row], kPdvExp + (eq - eqr));
  // key slots this query sees: [iv.x, iv.y) and [iv.z, iv.w)
  const int4 iv = q < p.L ? p.qiv[(int64_t)b * p.L + q] : make_int4(0, 0, 0, 0);
  OperandOffsets<D> of;
  of.init(lane);
  TileCopy<D> tc;
  tc.init(w, lane);
  const uint32_t plane_bytes = (uint32_t)p.Lp * D * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.kr + kvplane * p.Lp * D, plane_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.vr + kvplane * p.Lp * D, plane_bytes);

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = zero_f32x16();

  const int64_t trow = (int64_t)b * p.MT + m;
  const int nnz = p.q_nnz[trow];
  const int32_t *lst = p.q_list + trow * p.NT;
  const uint32_t *subs = p.sub_class + trow * p.NT;

  auto issue = [&](int k0, char *nb) {
    tc.issue(rk, k0, nb, w);
    tc.issue(rv, k0, nb + TB, w);
  };

  int tnext = 0;
  while (tnext < nnz) {
    __syncthreads();
    if (w == 0) {
      int t = tnext;
      const int c = build_q_stages(lst, subs, nnz, &t, stages, lane);
      if (lane == 0) {
        sh_count = c;
        sh_next = t;
      }
    }
    __syncthreads();
    const int ns = uniform(sh_count);
    tnext = uniform(sh_next);
    if (ns == 0) continue;
    issue(uniform((int)stages[0].x), buf0);
    auto stage = [&](int i, const char *buf, char *nxt) {
      wait_all_and_barrier();
      if (i + 1 < ns) issue(uniform((int)stages[i + 1].x), nxt);
      const uint2 desc = uniform(stages[i]);
      const uint32_t c0 = (desc.y >> (4 * w)) & 3u, c1 = (desc.y >> (4 * w + 2)) & 3u;
      if ((c0 | c1) == 0) return;
      const int k0 = (int)desc.x;
      const char *Kt = buf, *Vt = buf + TB;

      // Both 32-key sub-blocks always (straight-line code): the mask is exact,
      // so an empty one gives p = 0 and dS = 0.
      f32x16 s[2], dpt[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = zero_f32x16();
        dpt[kb] = zero_f32x16();
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb] = mfma32x32x16(lds_f16x8(Kt + kb * 32 * RB + of.row8[st]), qb[st], s[kb]);
          dpt[kb] = mfma32x32x16(lds_f16x8(Vt + kb * 32 * RB + of.row8[st]), dob[st], dpt[kb]);
        }
      }
      sched_lds_reads_ahead<4 * NS, kReadsAhead, 1>();
      __builtin_amdgcn_sched_barrier(0);
      if (c0 != 2 || c1 != 2) {
        const uint64_t mk = (range_bits(iv.x, iv.y, k0) | range_bits(iv.z, iv.w, k0)) >> (8 * g);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) s[kb][rr] = mask_select(mk, 32 * kb + 16 * (rr >> 3) + (rr & 7), s[kb][rr]);
        }
      }
      f16x8 dsb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][rr], fs, -lse2_q));
          dsb[kb][rr >> 3][rr & 7] = (_Float16)(pv * fmaf(dpt[kb][rr], dss, -dsc_q));
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            dqacc[db] = mfma32x32x16(tile_col8<D>(Kt, of, 32 * kb + 16 * hh, db), dsb[kb][hh], dqacc[db]);
        }
      }
    };
    for (int i = 0; i < ns; i += 2) {
      stage(i, buf0, buf1);
      if (i + 1 < ns) stage(i + 1, buf1, buf0);
    }
  }

  if (q < p.L) {
    const int tok = p.slot_tok[(int64_t)b * p.L + q];
    float *out = dq + (((int64_t)b * p.L + tok) * p.Hq + h) * D;
    const float2 *cs = p.rope + ((int64_t)b * p.Lp + q) * (D / 2);
    // dQ^T in units 2^(ek + ev + edo - kDsShift)
    const float qscale = ldexpf(p.scale, kDsShift - ek - ev - edo);
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

void launch_attn_dq_kernel(const AttnParams &p, int D, float *dq, hipStream_t s) {
  const unsigned gq = (unsigned)q_grid((int64_t)p.B * p.MT, p.Hkv, p.group);
  if (D == 64) attn_dq_kernel<64><<<gq, 256, 0, s>>>(p, dq);
  else attn_dq_kernel<128><<<gq, 256, 0, s>>>(p, dq);
}

}  // namespace opr

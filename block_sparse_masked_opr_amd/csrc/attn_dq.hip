// dQ kernel of the one-pass masked attention backward (gfx950).  It runs
// first in the backward and also prepares what the dK/dV kernel reads.
//
// One workgroup per (128-query tile, q head, row).  Each lane owns one query
// slot (and half of its head dims with its partner lane l ^ 32).  Prologue:
// the lane reads dout and o of its slot's token (bf16, token order), forms
// Delta = rowsum(dout * o) (fp32 over exact bf16 products), finds the
// largest |dout| of the row (its half and the partner lane's), converts dout
// to fp16 with that row's exponent into registers, and writes, for the dK/dV
// kernel, the fp16 dout plane, the row exponent (and its minimum over each
// 16-slot tile), and Delta, lse and the score factor in that kernel's
// per-slot units.
// Main loop, pipelined like the forward kernel: a stage list of the non-empty
// 32-key quarters in LDS, K' and V tiles in a ring of three LDS buffers
// (buffer loads to LDS, two stages in flight, each wave waiting only for its
// own copies of the current stage), one barrier per stage.  Per non-empty
// 32x32 sub-block each wave recomputes S^T = K' Q'^T and dP^T = V dO^T, masks
// partial sub-blocks with the query's key intervals, forms dS = P * (dP - Delta) (P from the forward
// LSE) and accumulates dQ^T += K'^T dS^T, reading K'^T from the row-major K'
// tile with transposing LDS reads.  The epilogue removes the operand units,
// applies the softmax scale and rotates dQ back by the transposed RoPE
// rotation.
//
// Units: q' and dout carry one exponent per row and q head (the lane's
// query: eq, edo), k' and v one per (row, kv head) plane (ek, ev).
// dP comes out in units 2^(edo + ev); Delta is brought into those units times
// 2^-kDsShift, and dS is formed as P * (dP * 2^-kDsShift - Delta) before the
// fp16 conversion.
#include "attn_common.h"
#include "attn_sched.h"
#include "opr_internal.h"

namespace opr {
namespace {

constexpr int kReadsAhead = 4;  // S / dP products whose K' / V operand reads are in flight
constexpr int kDqStageCap = 256;  // 32-key stages per list chunk (2 KB of LDS)

template <int D>
__global__ __launch_bounds__(256, 2) void attn_dq_kernel(AttnParams p, float *dq) {
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int HALF_DB = NDB / 2;
  constexpr int RB = Tile<D>::RB;
  constexpr int TB = 32 * RB;  // one 32-row tile
  constexpr int BUF = 2 * TB;  // K' tile, V tile
  // a ring of three separate LDS objects, so that the compiler sees that the
  // copies into two of them leave the third alone
  __shared__ __attribute__((aligned(1024))) char buf0[BUF];
  __shared__ __attribute__((aligned(1024))) char buf1[BUF];
  __shared__ __attribute__((aligned(1024))) char buf2[BUF];
  __shared__ uint2 stages[kDqStageCap];
  __shared__ int sh_count, sh_next;

  const QItem it = q_work_item(p.q_order, p.MT, p.Hkv, p.group, (int64_t)p.B * p.MT);
  if (!it.valid) return;
  const int j = it.j, m = it.m, kvh = it.kvh, b = it.b;
  const int h = kvh * p.group + j;

  const int tid = threadIdx.x, w = uniform(tid >> 6), lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int q = m * 128 + 32 * w + li;
  const int64_t kvplane = (int64_t)b * p.Hkv + kvh;
  const int64_t hq_row = ((int64_t)b * p.Hq + h) * p.Lp + q;
  const int eq = p.eqq[hq_row];
  const int ek = plane_exponent(p.mk[kvplane]);
  const int ev = plane_exponent(p.mv[kvplane]);
  const float fs = ldexpf(p.scale_log2, -(eq + ek));
  const float dss = ldexpf(1.0f, -kDsShift);

  f16x8 qb[NS], dob[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) qb[s] = ld_f16x8(p.qr + hq_row * D + 16 * s + 8 * g);

  // ---- prologue: Delta, the fp16 dout with its row exponent, the dK/dV
  // units.  The loads are issued here; the conversion (convert_dout) runs once
  // the stage list is built and the first K/V tiles stream in.
  int32_t tok = q < p.L ? p.slot_tok[(int64_t)b * p.L + q] : -1;
  if (tok >= 0 && !OPR_DCHECK(p.dbg, tok < p.L, kDbgToken)) tok = -1;
  uint4 dw[NS], ow[NS];  // bf16 dims 16 s + 8 g .. + 7 of dout and o
#pragma unroll
  for (int s = 0; s < NS; ++s) dw[s] = ow[s] = make_uint4(0u, 0u, 0u, 0u);
  float lse = -INFINITY;
  if (tok >= 0) {
    const int64_t base = (((int64_t)b * p.L + tok) * p.Hq + h) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      dw[s] = *reinterpret_cast<const uint4 *>(p.dout_in + base + 16 * s);
      ow[s] = *reinterpret_cast<const uint4 *>(p.o_in + base + 16 * s);
    }
    lse = p.lse_in[((int64_t)b * p.Hq + h) * p.L + tok];
  }
  float lse2_q, dsc_q;
  int edo_of_lane;
  auto convert_dout = [&]() {
    float delta = 0.0f;
    uint32_t mx = 0u;  // float bits of the largest |dout| (integer order)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      delta = dot2_bf16(ow[s].x, dw[s].x, delta);
      delta = dot2_bf16(ow[s].y, dw[s].y, delta);
      delta = dot2_bf16(ow[s].z, dw[s].z, delta);
      delta = dot2_bf16(ow[s].w, dw[s].w, delta);
      mx = max(mx, absmax8_bf16_bits(dw[s]));
    }
    delta += __shfl_xor(delta, 32);
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));  // the row's other half
    const int edo = mx > 0u ? plane_exponent(mx) : kExpMax;
    edo_of_lane = edo;
    uint16_t *drow = p.dor + hq_row * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint16_t *e16 = reinterpret_cast<const uint16_t *>(&dw[s]);
#pragma unroll
      for (int e = 0; e < 8; ++e) dob[s][e] = (_Float16)ldexpf(bf16_to_f32(e16[e]), edo);
      *reinterpret_cast<f16x8 *>(drow + 16 * s) = dob[s];
    }
    // the row exponent and its minimum over the kTile rows of the tile
    // (lanes 16 t .. 16 t + 15 of a half)
    int emin = edo;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) emin = min(emin, __shfl_xor(emin, off));
    if (g == 0) p.edoq[hq_row] = edo;
    if ((lane & 47) == 0) p.edot[((int64_t)b * p.Hq + h) * p.MTS + q / kTile] = emin;
    // this kernel's units: P = exp2(S * scale * log2 e - lse2_q) (+inf: no
    // key, P = 0), Delta in the units of dP times 2^-kDsShift
    const bool live = lse != -INFINITY;
    lse2_q = live ? lse * kLog2e : INFINITY;
    dsc_q = ldexpf(delta, edo + ev - kDsShift);
    // the dK/dV kernel's units (see attn_bwd.hip): the same quantities with
    // the slot's dout row exponent folded in and the 2^kPdvExp of its P
    if (g == 0) {
      p.lse2[hq_row] = live ? lse * kLog2e - (float)kPdvExp + (float)edo : INFINITY;
      p.dsc[hq_row] = ldexpf(delta, edo + ev - kDsShift - kPdvExp);
      p.fsq[hq_row] = fs;
    }
  };
  // key slots this query sees: [iv.x, iv.y) and [iv.z, iv.w)
  const int4 iv = q < p.L ? p.qiv[(int64_t)b * p.L + q] : make_int4(0, 0, 0, 0);
  OperandOffsets<D> of;
  of.init(lane);
  TileCopy<D, 4, 32> tc;
  tc.init(w, lane);
  constexpr int kCopies = 2 * TileCopy<D, 4, 32>::NI;  // copy instructions per wave and stage (K' and V)
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

  // the stage list (32-key quarters) is built in chunks of up to kDqStageCap stages
  int tnext = 0, ns = 0;
  auto build = [&]() {
    __syncthreads();  // the previous chunk's stages and buffers are no longer read
    if (w == 0) {
      int t = tnext;
      const int c = build_q_quarters<kDqStageCap>(lst, subs, nnz, p.NT, &t, stages, lane, p.dbg);
      if (lane == 0) {
        sh_count = c;
        sh_next = t;
      }
    }
    __syncthreads();
    ns = uniform(sh_count);
    tnext = uniform(sh_next);
    if (ns > 0) issue(uniform((int)stages[0].x), buf0);
    if (ns > 1) issue(uniform((int)stages[1].x), buf1);
  };
  build();
  convert_dout();  // while the first K/V tiles stream in
  for (;;) {
    // stage i reads `buf` (buf[i % 3]) while stages i+1 and i+2 stream in; at
    // its start it waits for its own tiles only (the copies of stage i+1, if
    // any, are the newest kCopies of the wave), then refills the buffer that
    // stage i-1 used with stage i+2.  The stage list is fixed for the chunk,
    // so both descriptors are read before the barrier, together (an entry
    // past the list is read but not used).
    auto stage = [&](int i, const char *buf, char *nxt2) {
      const uint2 d0 = stages[i];
      const uint32_t x2 = stages[min(i + 2, kDqStageCap - 1)].x;
      const uint2 desc = uniform(d0);
      const int k2 = uniform((int)x2);
      if (i + 1 < ns) wait_older_copies_and_barrier<kCopies>();
      else wait_older_copies_and_barrier<0>();
      if (i + 2 < ns) issue(k2, nxt2);
      const uint32_t c = (desc.y >> (2 * w)) & 3u;
      if (c == 0) return;
      const int k0 = (int)desc.x;
      const char *Kt = buf, *Vt = buf + TB;

      // S^T and dP^T of the stage's 32 keys (straight-line code: the mask is
      // exact, so masked scores give p = 0 and dS = 0)
      f32x16 sc = zero_f32x16(), dpt = zero_f32x16();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        sc = mfma32x32x16(lds_f16x8(Kt + of.row8[st]), qb[st], sc);
        dpt = mfma32x32x16(lds_f16x8(Vt + of.row8[st]), dob[st], dpt);
      }
      sched_lds_reads_ahead<2 * NS, kReadsAhead, 1>();
      __builtin_amdgcn_sched_barrier(0);
      if (c != 2) {
        // lane group g holds keys 16h + 8g + 0..7 of the 32
        const uint64_t mk = (range_bits(iv.x, iv.y, k0) | range_bits(iv.z, iv.w, k0)) >> (8 * g);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sc[rr] = mask_select(mk, 16 * (rr >> 3) + (rr & 7), sc[rr]);
      }
      f16x8 dsb[2];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sc[rr], fs, -lse2_q));
        dsb[rr >> 3][rr & 7] = (_Float16)(pv * fmaf(dpt[rr], dss, -dsc_q));
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          dqacc[db] = mfma32x32x16(tile_col8<D>(Kt, of, 16 * hh, db), dsb[hh], dqacc[db]);
      }
    };
    for (int i = 0; i < ns; i += 3) {
      stage(i, buf0, buf2);
      if (i + 1 < ns) stage(i + 1, buf1, buf0);
      if (i + 2 < ns) stage(i + 2, buf2, buf1);
    }
    if (tnext >= nnz) break;
    build();
  }

  // the slot's token, read again here rather than held through the loop
  const int etok = q < p.L ? p.slot_tok[(int64_t)b * p.L + q] : -1;
  if (etok >= 0 && OPR_DCHECK(p.dbg, etok < p.L, kDbgToken)) {
    float *out = dq + (((int64_t)b * p.L + etok) * p.Hq + h) * D;
    const float2 *cs = p.rope + ((int64_t)b * p.Lp + q) * (D / 2);
    // dQ^T in units 2^(ek + ev + edo - kDsShift); the unit exponent is
    // applied to the value (it can exceed fp32's range as a factor)
    const int uexp = kDsShift - ek - ev - edo_of_lane;
#pragma unroll
    for (int db = 0; db < HALF_DB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float lo[4], hi[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = 4 * a + c;
          const float2 rc = cs[acc_dim(db, r, g)];
          const float g1 = ldexpf(p.scale * dqacc[db][r], uexp), g2 = ldexpf(p.scale * dqacc[db + HALF_DB][r], uexp);
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

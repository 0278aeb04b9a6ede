// Backward kernels of the one-pass masked attention (gfx950).
//
// With P recomputed from the forward LSE (P = exp2(scale*log2(e)*S - lse2)),
//   dV  = sum over the group's q heads of P^T dO
//   dP  = dO V^T,  dS = P * (dP - delta),  delta = rowsum(dO * O)
//   dQ' = scale * dS K',  dK' = scale * sum over the group of dS^T Q'
// and dQ, dK are rotated back by the transposed RoPE rotation.
//
// Both kernels run in attention order (tiles of slots; results are written
// at the slot's token).
// attn_dkdv_kernel: one workgroup per (work item of 128-key tile n, kv head); wave w
//   owns key slots n*128 + 32w .. +31, one per lane column, K' and V of its
//   key in registers.  Its stages are (q-tile of k_list, head of the group,
//   64-query half) with a non-empty sub-block; each streams the Q' and dO rows
//   of the stage into LDS (double buffered, buffer loads to LDS) and reads
//   Q'^T and dO^T from the same row-major tiles with transposing LDS reads.
//   dK^T and dV^T stay in accumulators; each key is owned by exactly one
//   workgroup: no atomics.
// attn_dq_kernel (attn_dq.hip): one workgroup per (128-query tile, q head,
//   row), pipelined like the forward kernel over the K' / V tiles; S and dP^T
//   are recomputed per non-empty sub-block and dQ^T += K'^T dS^T.
// Work items start longest first, round-robin over the XCDs (q_order and
// k_items of the prologue).  A k-tile column whose stages exceed the cap of
// the work order runs as several items, each over a contiguous part of its
// stage range; parts after the first write partial dK/dV that
// dkdv_split_reduce_kernel adds in a fixed order (deterministic).  Partial
// sub-blocks are masked with 64-bit masks
// built from the two runs of slots of each query or key.
//
// Units: k' and v carry one exponent per (row, kv head), constant inside a
// workgroup; q' and dout one per 16-slot tile and q head, so they change
// inside a stage (eq, edo of the tile; eqr, edor their minima over the kv
// group; the stage descriptor carries the four tiles' eq and edo).  The products are brought to group-wide units like this:
//   S: the score scale is 2^-(eq + ek) per tile;
//   dV^T += dO'^T P'^T with P' = fp16(P * 2^(kPdvExp - (edo - edor))) (the
//       stored lse2 carries the shift), so dV is in units 2^(kPdvExp + edor);
//   dS' = P' (dP' dss - delta') with dP' = dO' V'^T in units 2^(edo + ev),
//       dss = 2^-(kDsShift + kPdvExp + eq - eqr) per tile and delta' stored
//       in the matching units, so dS' = dS 2^(eqr + edor + ev - kDsShift - eq)
//       and dK^T += Q'^T dS'^T is in units 2^(eqr + edor + ev - kDsShift).
#include "attn_common.h"
#include "attn_sched.h"
#include "opr_internal.h"

namespace opr {
namespace {

constexpr int kReadsAhead = 4;  // dV / dK products whose operand reads are in flight

template <int D>
__global__ __launch_bounds__(512, 1) void attn_dkdv_kernel(AttnParams p, float *dk, float *dv) {
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int HALF_DB = NDB / 2;
  constexpr int TB = Tile<D>::BYTES, RB = Tile<D>::RB;
  constexpr int PSTRIDE = 4096;  // P of one key block: [qb][hh][lane] x 16 bytes
  // per stage buffer: Q' tile, dO tile, lse2[64], scaled delta[64]
  constexpr int BUF = 2 * TB + 512;
  // Separate LDS objects, so that the compiler sees that a copy or a store
  // into one leaves the others alone: a ring of three stage buffers (the
  // P-waves read stage i, the dS-waves stage i-1, stage i+1 streams in) and
  // a ring of three P buffers of the 4 key blocks (written by the P-waves at
  // step i, read by the dS-waves at step i+1).
  __shared__ __attribute__((aligned(1024))) char buf0[BUF];
  __shared__ __attribute__((aligned(1024))) char buf1[BUF];
  __shared__ __attribute__((aligned(1024))) char buf2[BUF];
  __shared__ __attribute__((aligned(1024))) char pbf0[4 * PSTRIDE];
  __shared__ __attribute__((aligned(1024))) char pbf1[4 * PSTRIDE];
  __shared__ __attribute__((aligned(1024))) char pbf2[4 * PSTRIDE];
  __shared__ uint4 stages[kKStageCap];
  __shared__ int sh_count;
  __shared__ int64_t sh_next;

  const int64_t R = blockIdx.x;  // rank: longest items first, round-robin over the XCDs
  if (R / p.Hkv >= p.k_counts[0]) return;
  const int4 item = p.k_items[R / p.Hkv];  // (column, part, parts, partial slot or -1)
  const int32_t col = item.x;
  const int kvh = (int)(R % p.Hkv);
  const int b = col / p.NT;
  const int n = col - b * p.NT;

  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63, g = lane >> 5, li = lane & 31;
  const bool pwave = wave < 4;  // P-wave (S, P, dV) or dS-wave (dP, dS, dK) of key block w
  const int w = wave & 3;
  const int key = n * 128 + 32 * w + li;
  const int64_t kvplane = (int64_t)b * p.Hkv + kvh;
  const int64_t hbase = (int64_t)b * p.Hq + (int64_t)kvh * p.group;  // first q head of the group
  // q' and dout scales vary by stage (one per 64-slot tile, carried in the
  // stage descriptor); eqr, edor are their minima over the group
  const int eqr = p.eref[2 * kvplane], edor = p.eref[2 * kvplane + 1];
  const int ek = plane_exponent(p.mk[kvplane]);
  const int ev = plane_exponent(p.mv[kvplane]);

  // K' rows (P-waves) or V rows (dS-waves) of the lane's key, as B operands
  f16x8 frag[NS];
  {
    const uint16_t *src = (pwave ? p.kr : p.vr) + (kvplane * p.Lp + key) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) frag[s] = ld_f16x8(src + 16 * s + 8 * g);
  }
  // query slots that see this key: [iv.x, iv.y) and [iv.z, iv.w)
  const int4 iv = key < p.L ? p.kiv[(int64_t)b * p.L + key] : make_int4(0, 0, 0, 0);
  OperandOffsets<D> of;
  of.init(lane);
  TileCopy<D, 8> tc;
  tc.init(wave, lane);
  const uint32_t plane_bytes = (uint32_t)p.Lp * D * 2;

  f32x16 acc[NDB];  // dV^T (P-waves) or dK^T (dS-waves)
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero_f32x16();

  const int64_t tcol = (int64_t)b * p.NT + n;
  const int nnz = p.k_nnz[tcol];
  const int32_t *lst = p.k_list + tcol * p.MT;
  const uint32_t *subs_b = p.sub_class + (int64_t)b * p.MT * p.NT;

  auto issue = [&](uint32_t x, char *nb) {
    const int q0 = (int)(x & 0xFFFFFFu), hj = (int)(x >> 24);
    const int64_t plane = hbase + hj;
    tc.issue(make_rsrc(p.qr + plane * p.Lp * D, plane_bytes), q0, nb, wave);
    tc.issue(make_rsrc(p.dor + plane * p.Lp * D, plane_bytes), q0, nb + TB, wave);
    // lse2 (wave 0) and delta (wave 1) of the stage's 64 query slots
    if (wave < 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc((wave == 0 ? p.lse2 : p.dsc) + plane * p.Lp, (uint32_t)p.Lp * 4),
                                               (OPR_LDS void *)(nb + 2 * TB + 256 * wave), 4, 4 * lane, 4 * q0, 0, 0);
  };

  // P-wave element work of a stage: S^T = K' Q'^T (keys x queries) per
  // 32-query sub-block, P = exp2(S * scale * log2 e - lse2) masked by the
  // key's runs (unless both sub-blocks are full), as fp16(P * 2^kPdvExp) (lse2 carries the -kPdvExp) into op and
  // into LDS for the dS-wave.  The update that follows is dV^T += dO^T P^T.
  auto p_elem = [&](uint4 desc, const char *buf, char *pout, f16x8 (&op)[2][2]) {
    const int q0 = (int)(desc.x & 0xFFFFFFu);
    // raw score -> log2 units, per 16-query tile 2 qb + hh (its q' exponent)
    float fs[2][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) fs[k >> 1][k & 1] = ldexpf(p.scale_log2, -(stage_exponent(desc.z, k) + ek));
    const char *Qt = buf;
    const float *lse2s = reinterpret_cast<const float *>(buf + 2 * TB);
    char *Pw = pout + w * PSTRIDE;
    // both products first, then both element blocks
    f32x16 s[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f16x8 qf[NS];
#pragma unroll
      for (int st = 0; st < NS; ++st) qf[st] = lds_f16x8(Qt + qb * 32 * RB + of.row8[st]);
      s[qb] = zero_f32x16();
#pragma unroll
      for (int st = 0; st < NS; ++st) s[qb] = mfma32x32x16(qf[st], frag[st], s[qb]);
    }
    if (((desc.y >> (4 * w)) & 15u) != 10u) {  // a sub-block is not full: mask by the key's runs
      const uint64_t mq = (range_bits(iv.x, iv.y, q0) | range_bits(iv.z, iv.w, q0)) >> (8 * g);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][r] = mask_select(mq, 32 * qb + 16 * (r >> 3) + (r & 7), s[qb][r]);
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int qbase = 32 * qb + 16 * hh + 8 * g;  // query rows of registers 8hh .. 8hh+7
        const float4 l0 = *reinterpret_cast<const float4 *>(lse2s + qbase);
        const float4 l1 = *reinterpret_cast<const float4 *>(lse2s + qbase + 4);
        const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          op[qb][hh][e] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[qb][8 * hh + e], fs[qb][hh], -lv[e]));
        }
        *reinterpret_cast<f16x8 *>(Pw + (2 * qb + hh) * 1024 + lane * 16) = op[qb][hh];
      }
    }
  };

  // dS-wave element work of a stage (one stage behind): dP^T = V dO^T and
  // dS = P * (dP - delta) into op, with P read back from the P-wave of the same
  // key block (masked entries have P = 0 and so dS = 0).  The update that
  // follows is dK^T += Q'^T dS^T.
  auto ds_elem = [&](uint4 desc, const char *buf, const char *pin, f16x8 (&op)[2][2]) {
    // dP' -> dS' units, per 16-query tile 2 qb + hh (its q' exponent)
    float dss[2][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) dss[k >> 1][k & 1] = ldexpf(1.0f, -kDsShift - kPdvExp - (stage_exponent(desc.z, k) - eqr));
    const char *dOt = buf + TB;
    const float *dscs = reinterpret_cast<const float *>(buf + 2 * TB + 256);
    const char *Pw = pin + w * PSTRIDE;
    f32x16 dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f16x8 df[NS];
#pragma unroll
      for (int st = 0; st < NS; ++st) df[st] = lds_f16x8(dOt + qb * 32 * RB + of.row8[st]);
      dp[qb] = zero_f32x16();
#pragma unroll
      for (int st = 0; st < NS; ++st) dp[qb] = mfma32x32x16(df[st], frag[st], dp[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int qbase = 32 * qb + 16 * hh + 8 * g;
        const f16x8 pv = *reinterpret_cast<const f16x8 *>(Pw + (2 * qb + hh) * 1024 + lane * 16);
        const float4 d0 = *reinterpret_cast<const float4 *>(dscs + qbase);
        const float4 d1 = *reinterpret_cast<const float4 *>(dscs + qbase + 4);
        const float dvv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        // P * 2^kPdvExp times (dP * 2^-kDsShift - delta) * 2^-kPdvExp: the
        // second factor in fp32, then both multiplied as packed fp16 pairs
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f16x2 t = {(_Float16)fmaf(dp[qb][8 * hh + e], dss[qb][hh], -dvv[e]),
                           (_Float16)fmaf(dp[qb][8 * hh + e + 1], dss[qb][hh], -dvv[e + 1])};
          const f16x2 pp = {pv[e], pv[e + 1]};
          const f16x2 d = t * pp;
          op[qb][hh][e] = d[0];
          op[qb][hh][e + 1] = d[1];
        }
      }
    }
  };

  // Step i of a wave: the P-wave runs stage i (buf[i % 3] -> pbf[i % 3]) and
  // updates dV^T with dO^T; the dS-wave runs stage i - 1 (buf[(i - 1) % 3],
  // pbf[(i - 1) % 3]) and updates dK^T with Q'^T; a wave whose key block sees
  // no query of the stage skips it.  Both roles share the accumulator update
  // (one copy of the code, so the accumulators stay in place across the role
  // branch).
  auto wave_step = [&](int i, int ns, const char *ba, const char *bb, char *pa, const char *pr) {
    if (pwave ? i >= ns : i < 1) return;
    const uint4 desc = uniform(stages[pwave ? i : i - 1]);
    if (((desc.y >> (4 * w)) & 15u) == 0) return;
    f16x8 op[2][2];
    const char *T;
    if (pwave) {
      p_elem(desc, ba, pa, op);
      T = ba + TB;
    } else {
      ds_elem(desc, bb, pr, op);
      T = bb;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = mfma32x32x16(tile_col8<D>(T, of, 32 * qb + 16 * hh, db), op[qb][hh], acc[db]);
      }
    }
    sched_lds_reads_ahead<4 * NDB, kReadsAhead>();
    __builtin_amdgcn_sched_barrier(0);
  };

  // this item's part of the column's stage range
  const int64_t ftotal = (int64_t)nnz * p.group * 2;
  int64_t fnext = ftotal * item.y / item.z;
  const int64_t fend = ftotal * (item.y + 1) / item.z;
  while (fnext < fend) {
    __syncthreads();
    if (wave == 0) {
      int64_t f = fnext;
      const int c = build_k_stages(lst, subs_b, p.NT, n, p.group, fend, p.eqt + hbase * p.MTS,
                                   p.edot + hbase * p.MTS, p.MTS, &f, stages, lane);
      if (lane == 0) {
        sh_count = c;
        sh_next = f;
      }
    }
    __syncthreads();
    const int ns = uniform(sh_count);
    fnext = uniform(sh_next);
    if (ns == 0) continue;
    issue(uniform(stages[0].x), buf0);
    // step i: stage i + 1 streams into buf[(i + 1) % 3] while the waves run
    // their stages (wave_step)
    auto step = [&](int i, const char *ba, const char *bb, char *bl, char *pa, const char *pr) {
      wait_all_and_barrier();
      if (i + 1 < ns) issue(uniform((int)stages[i + 1].x), bl);
      wave_step(i, ns, ba, bb, pa, pr);
    };
    for (int i = 0; i <= ns; i += 3) {
      step(i, buf0, buf2, buf1, pbf0, pbf2);
      if (i + 1 <= ns) step(i + 1, buf1, buf0, buf2, pbf1, pbf0);
      if (i + 2 <= ns) step(i + 2, buf2, buf1, buf0, pbf2, pbf1);
    }
  }

  if (key < p.L) {
    // part 0 writes at the key's token, parts 1.. into their partial slot
    int64_t out;
    if (item.w < 0) {
      const int tok = p.slot_tok[(int64_t)b * p.L + key];
      out = (((int64_t)b * p.L + tok) * p.Hkv + kvh) * D;
    } else {
      out = (((int64_t)item.w * p.Hkv + kvh) * OPR_ATTN_BLOCK + (key - n * OPR_ATTN_BLOCK)) * D;
      dk = p.kpart;
      dv = p.kpart + (int64_t)kSplitSlots * OPR_ATTN_BLOCK * D;
    }
    if (!pwave) {
      // dK^T in units 2^(eqr + edor + ev - kDsShift), rotated back by RoPE
      const float2 *cs = p.rope + ((int64_t)b * p.Lp + key) * (D / 2);
      const float kscale = ldexpf(p.scale, kDsShift - eqr - edor - ev);
#pragma unroll
      for (int db = 0; db < HALF_DB; ++db) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          float lo[4], hi[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int r = 4 * a4 + c;
            const float2 rc = cs[acc_dim(db, r, g)];
            const float g1 = kscale * acc[db][r], g2 = kscale * acc[db + HALF_DB][r];
            lo[c] = g1 * rc.x + g2 * rc.y;
            hi[c] = g2 * rc.x - g1 * rc.y;
          }
          *reinterpret_cast<float4 *>(dk + out + acc_dim(db, 4 * a4, g)) = make_float4(lo[0], lo[1], lo[2], lo[3]);
          *reinterpret_cast<float4 *>(dk + out + acc_dim(db + HALF_DB, 4 * a4, g)) =
              make_float4(hi[0], hi[1], hi[2], hi[3]);
        }
      }
    } else {
      // dV^T in units 2^(kPdvExp + edor)
      const float vscale = ldexpf(1.0f, -kPdvExp - edor);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
          *reinterpret_cast<float4 *>(dv + out + acc_dim(db, 4 * a4, g)) =
              make_float4(vscale * acc[db][4 * a4], vscale * acc[db][4 * a4 + 1],
                          vscale * acc[db][4 * a4 + 2], vscale * acc[db][4 * a4 + 3]);
      }
    }
  }
}

// dK and dV of the columns cut into parts: part 0 wrote them at the tokens;
// add parts 1..s-1 from their partial slots, in order.  One workgroup per
// (cut column, kv head); grid.x covers the most cut columns there can be.
template <int D>
__global__ __launch_bounds__(256) void dkdv_split_reduce_kernel(AttnParams p, float *dk, float *dv) {
  if ((int)blockIdx.x >= p.k_counts[1]) return;
  const int4 e = p.k_split[blockIdx.x];  // (column, first partial slot, parts, 0)
  const int kvh = blockIdx.y;
  const int b = e.x / p.NT, n = e.x - b * p.NT;
  constexpr int C4 = D / 4;  // float4 per key row
  const float *pk = p.kpart, *pv = p.kpart + (int64_t)kSplitSlots * OPR_ATTN_BLOCK * D;
  for (int i = threadIdx.x; i < OPR_ATTN_BLOCK * C4; i += 256) {
    const int kl = i / C4, c4 = i - kl * C4;
    const int key = n * OPR_ATTN_BLOCK + kl;
    if (key >= p.L) continue;
    const int tok = p.slot_tok[(int64_t)b * p.L + key];
    const int64_t out = (((int64_t)b * p.L + tok) * p.Hkv + kvh) * D + 4 * c4;
    float4 ak = *reinterpret_cast<const float4 *>(dk + out);
    float4 av = *reinterpret_cast<const float4 *>(dv + out);
    for (int j = 0; j < e.z - 1; ++j) {
      const int64_t src = (((int64_t)(e.y + j) * p.Hkv + kvh) * OPR_ATTN_BLOCK + kl) * D + 4 * c4;
      const float4 xk = *reinterpret_cast<const float4 *>(pk + src);
      const float4 xv = *reinterpret_cast<const float4 *>(pv + src);
      ak.x += xk.x; ak.y += xk.y; ak.z += xk.z; ak.w += xk.w;
      av.x += xv.x; av.y += xv.y; av.z += xv.z; av.w += xv.w;
    }
    *reinterpret_cast<float4 *>(dk + out) = ak;
    *reinterpret_cast<float4 *>(dv + out) = av;
  }
}

}  // namespace

void fill_params(const opr_attn_in &in, float scale, const AttnWs &ws, AttnParams *p);

void launch_attn_dq_kernel(const AttnParams &p, int D, float *dq, hipStream_t s);

// ev (optional): events recorded before dK/dV, right after the dK/dV kernel
// (so that its span is that kernel alone) and after dQ.
hipError_t launch_attn_bwd_kernels(const opr_attn_in &in, float scale, float *dq, float *dk,
                                   float *dv, const AttnWs &ws, hipStream_t s, hipEvent_t *ev) {
  AttnParams p;
  fill_params(in, scale, ws, &p);
  // every column once, plus the most extra parts the work order can make
  const int32_t extra = kSplitSlots / in.Hkv + 1;
  const unsigned gk = (unsigned)(((int64_t)in.B * p.NT + extra) * in.Hkv);
  const dim3 gr((unsigned)extra, (unsigned)in.Hkv);
  if (ev) (void)hipEventRecord(ev[0], s);
  if (in.D == 64) attn_dkdv_kernel<64><<<gk, 512, 0, s>>>(p, dk, dv);
  else attn_dkdv_kernel<128><<<gk, 512, 0, s>>>(p, dk, dv);
  if (ev) (void)hipEventRecord(ev[1], s);
  if (in.D == 64) dkdv_split_reduce_kernel<64><<<gr, 256, 0, s>>>(p, dk, dv);
  else dkdv_split_reduce_kernel<128><<<gr, 256, 0, s>>>(p, dk, dv);
  launch_attn_dq_kernel(p, in.D, dq, s);
  if (ev) (void)hipEventRecord(ev[2], s);
  return hipGetLastError();
}

}  // namespace opr

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
// Units: k' and v carry one exponent per (row, kv head) plane (ek, ev),
// constant inside a workgroup; q' and dout one per query row and q head (eq,
// edo), so they change from query to query inside a stage.  Each key block w
// (the P-wave and the dS-wave of its 32 keys) accumulates in units fixed by
// eqr, edor: the smallest eq and edo over the queries of this work item's
// stages that see the block's keys (dkdv_units_kernel, before this kernel),
// so a key's units depend only on queries that see it, never on another
// conversation of the row.  The dQ kernel stores per slot
// lse2 = lse log2 e - kPdvExp + edo, delta' = delta 2^(edo + ev - kDsShift -
// kPdvExp) (delta in the units of dP' 2^-(kDsShift + kPdvExp)) and the score
// factor fsq = scale log2 e 2^-(eq + ek).  With the query's shift
// c = 2^-(eq - eqr):
//   S: raw scores times fsq are in log2 units;
//   dV^T += dO'^T P'^T with P' = fp16(P * 2^(kPdvExp - (edo - edor)))
//       = exp2(S fsq - lse2 + edor), so dV is in units 2^(kPdvExp + edor);
//   dS' = P' (dP' 2^-(kDsShift + kPdvExp) - delta') c 2^bs with dP' = dO' V'^T
//       in units 2^(edo + ev) and bs the dS-wave's shift of its keys' v' to
//       the top of fp16's range, so dS' = dS 2^(eqr + edor + ev + bs - kDsShift - eq)
//       and dK^T += Q'^T dS'^T is in units 2^(eqr + edor + ev + bs - kDsShift).
//   c is capped at 1: a query with eq below eqr does not see the block, its
//   P' is 0, and the cap keeps its factor finite.
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
  // per stage buffer: Q' tile, dO tile, lse2[64], scaled delta[64], score
  // factors[64]
  constexpr int BUF = 2 * TB + 768;
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
  __shared__ uint2 stages[kKStageCap];
  // per wave: two factors of each of the stage's 64 queries (see p_elem, ds_elem)
  __shared__ __attribute__((aligned(16))) float qfac[8][2][64];
  __shared__ int sh_count;
  __shared__ int64_t sh_next;

  const int64_t R = blockIdx.x;  // rank: longest items first, round-robin over the XCDs
  if (R / p.Hkv >= p.k_counts[0]) return;
  const int4 item = p.k_items[R / p.Hkv];  // (column, part, parts, partial slot or -1)
  if (!OPR_DCHECK(p.dbg, (unsigned)item.x < (unsigned)(p.B * p.NT) && (unsigned)item.y < (unsigned)item.z &&
                             item.w < kSplitSlots, kDbgItem))
    return;
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
  const int ek = plane_exponent(p.mk[kvplane]);
  const int ev = plane_exponent(p.mv[kvplane]);
  // K' rows (P-waves) or V rows (dS-waves) of the lane's key, as B operands
  f16x8 frag[NS];
  {
    const uint16_t *src = (pwave ? p.kr : p.vr) + (kvplane * p.Lp + key) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) frag[s] = ld_f16x8(src + 16 * s + 8 * g);
  }
  // dS-waves: the shift bs that brings the largest |v'| of the block's 32
  // keys to [2^14, 2^15).  v carries one scale per plane, so a block of small
  // v (another conversation of the row holding the plane's largest values)
  // would otherwise form its dP - delta bracket that much below fp16's normal
  // range; dK is accumulated per key, so each block may use its own units.
  int bs = 0;
  if (!pwave) {
    float mv = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) mv = fmaxf(mv, fabsf((float)frag[s][e]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mv = fmaxf(mv, __shfl_xor(mv, off));
    if (mv > 0.0f) {
      int x;
      frexpf(mv, &x);
      bs = max(0, 15 - x);
    }
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

  // this item's part of the column's stage range: flat stage index
  // f = (tile * G + head) * 2 + half over k_list
  const int64_t ftotal = (int64_t)nnz * p.group * 2;
  const int64_t fbegin = ftotal * item.y / item.z;
  const int64_t fend = ftotal * (item.y + 1) / item.z;

  // this key block's units, from dkdv_units_kernel
  const int eqr = uniform(p.kunits[R * 8 + 2 * w]), edor = uniform(p.kunits[R * 8 + 2 * w + 1]);
  const float edor_f = (float)edor;
  // a query's score factor fsq = scale log2(e) 2^-(eq + ek) times qsh is its
  // shift 2^-(eq - eqr) against this block's units, times 2^bs (capped at
  // qcap = 2^bs for a query the block is not seen by)
  const float qsh = ldexpf(1.0f / p.scale_log2, eqr + ek + bs);
  const float qcap = ldexpf(1.0f, bs);
  const float kDss = ldexpf(1.0f, -kDsShift - kPdvExp);

  auto issue = [&](uint32_t x, char *nb) {
    const int q0 = (int)(x & 0xFFFFFFu), hj = (int)(x >> 24);
    const int64_t plane = hbase + hj;
    tc.issue(make_rsrc(p.qr + plane * p.Lp * D, plane_bytes), q0, nb, wave);
    tc.issue(make_rsrc(p.dor + plane * p.Lp * D, plane_bytes), q0, nb + TB, wave);
    // lse2 (wave 0), delta (wave 1) and the score factors (wave 2) of the
    // stage's 64 query slots
    if (wave < 3)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          make_rsrc((wave == 0 ? p.lse2 : wave == 1 ? p.dsc : p.fsq) + plane * p.Lp, (uint32_t)p.Lp * 4),
          (OPR_LDS void *)(nb + 2 * TB + 256 * wave), 4, 4 * lane, 4 * q0, 0, 0);
  };

  // P-wave element work of a stage: S^T = K' Q'^T (keys x queries) per
  // 32-query sub-block, P = exp2(S * scale * log2 e - lse2) masked by the
  // key's runs (unless both sub-blocks are full), as
  // fp16(P * 2^(kPdvExp - (edo - edor))) (lse2 carries -kPdvExp + edo) into op
  // and into LDS for the dS-wave.  The update that follows is dV^T += dO^T P^T.
  auto p_elem = [&](uint2 desc, const char *buf, char *pout, f16x8 (&op)[2][2]) {
    const int q0 = (int)(desc.x & 0xFFFFFFu);
    const char *Qt = buf;
    // raw score -> log2 units, per query (its q' row exponent)
    const float *fss = reinterpret_cast<const float *>(buf + 2 * TB + 512);
    // lane i forms edor - lse2 of the stage's query i once, for all lanes
    float *bq = qfac[wave][0];
    bq[lane] = edor_f - reinterpret_cast<const float *>(buf + 2 * TB)[lane];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
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
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float4 l0 = *reinterpret_cast<const float4 *>(bq + qbase);
        const float4 l1 = *reinterpret_cast<const float4 *>(bq + qbase + 4);
        const float4 f0 = *reinterpret_cast<const float4 *>(fss + qbase);
        const float4 f1 = *reinterpret_cast<const float4 *>(fss + qbase + 4);
        const float bv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const float fv[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          op[qb][hh][e] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[qb][8 * hh + e], fv[e], bv[e]));
        }
        *reinterpret_cast<f16x8 *>(Pw + (2 * qb + hh) * 1024 + lane * 16) = op[qb][hh];
      }
    }
  };

  // dS-wave element work of a stage (one stage behind): dP^T = V dO^T and
  // dS = P * (dP - delta) into op, with P read back from the P-wave of the same
  // key block (masked entries have P = 0 and so dS = 0).  The update that
  // follows is dK^T += Q'^T dS^T.
  auto ds_elem = [&](uint2 desc, const char *buf, const char *pin, f16x8 (&op)[2][2]) {
    const char *dOt = buf + TB;
    // lane i forms, for the stage's query i, its shift 2^(bs - (eq - eqr))
    // from its score factor (clamped at 2^bs for a query the block is not
    // seen by) folded into the dP factor and into delta
    float *dsq = qfac[wave][0], *dvq = qfac[wave][1];
    {
      const float sh = fminf(qcap, reinterpret_cast<const float *>(buf + 2 * TB + 512)[lane] * qsh);
      dsq[lane] = kDss * sh;
      dvq[lane] = reinterpret_cast<const float *>(buf + 2 * TB + 256)[lane] * sh;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
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
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float4 s0 = *reinterpret_cast<const float4 *>(dsq + qbase);
        const float4 s1 = *reinterpret_cast<const float4 *>(dsq + qbase + 4);
        const float4 d0 = *reinterpret_cast<const float4 *>(dvq + qbase);
        const float4 d1 = *reinterpret_cast<const float4 *>(dvq + qbase + 4);
        const float dss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const float dvv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        // P * 2^kPdvExp times (dP * 2^-kDsShift - delta) * 2^-kPdvExp (with the
        // query's shift): the second factor in fp32, then both multiplied as
        // packed fp16 pairs
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f16x2 t = {(_Float16)fmaf(dp[qb][8 * hh + e], dss[e], -dvv[e]),
                           (_Float16)fmaf(dp[qb][8 * hh + e + 1], dss[e + 1], -dvv[e + 1])};
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
  auto wave_step = [&](int i, int ns, uint2 desc, const char *ba, const char *bb, char *pa, const char *pr) {
    if (pwave ? i >= ns : i < 1) return;
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

  int64_t fnext = fbegin;
  while (fnext < fend) {
    __syncthreads();
    if (wave == 0) {
      int64_t f = fnext;
      const int c = build_k_stages(lst, subs_b, p.NT, p.MT, n, p.group, fend, &f, stages, lane, p.dbg);
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
      // the stage list is fixed for the chunk: the wave's descriptor and the
      // next stage's are read before the barrier, together (entries outside
      // the list are read but not used)
      const uint2 d0 = stages[pwave ? min(i, kKStageCap - 1) : max(i - 1, 0)];
      const uint32_t x1 = stages[min(i + 1, kKStageCap - 1)].x;
      const uint2 desc = uniform(d0);
      const uint32_t k1 = uniform(x1);
      wait_all_and_barrier();
      if (i + 1 < ns) issue(k1, bl);
      wave_step(i, ns, desc, ba, bb, pa, pr);
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
      if (!OPR_DCHECK(p.dbg, (unsigned)tok < (unsigned)p.L, kDbgToken)) return;
      out = (((int64_t)b * p.L + tok) * p.Hkv + kvh) * D;
    } else {
      out = (((int64_t)item.w * p.Hkv + kvh) * OPR_ATTN_BLOCK + (key - n * OPR_ATTN_BLOCK)) * D;
      dk = p.kpart;
      dv = p.kpart + (int64_t)kSplitSlots * OPR_ATTN_BLOCK * D;
    }
    if (!pwave) {
      // dK^T in units 2^(eqr + edor + ev + bs - kDsShift), rotated back by
      // RoPE; the unit exponent is applied to the value (as a factor it can
      // leave fp32's range)
      const float2 *cs = p.rope + ((int64_t)b * p.Lp + key) * (D / 2);
      const int uexp = kDsShift - eqr - edor - ev - bs;
#pragma unroll
      for (int db = 0; db < HALF_DB; ++db) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          float lo[4], hi[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int r = 4 * a4 + c;
            const float2 rc = cs[acc_dim(db, r, g)];
            const float g1 = ldexpf(p.scale * acc[db][r], uexp), g2 = ldexpf(p.scale * acc[db + HALF_DB][r], uexp);
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
      const int uexp = -kPdvExp - edor;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
          *reinterpret_cast<float4 *>(dv + out + acc_dim(db, 4 * a4, g)) =
              make_float4(ldexpf(acc[db][4 * a4], uexp), ldexpf(acc[db][4 * a4 + 1], uexp),
                          ldexpf(acc[db][4 * a4 + 2], uexp), ldexpf(acc[db][4 * a4 + 3], uexp));
      }
    }
  }
}

// Units of the dK/dV work items: for rank R (item R / Hkv, kv head R % Hkv)
// and each of its 4 key blocks, the smallest q' and dout row exponents over
// the queries of the item's stages that see the block's keys, into
// kunits[R][block][q', dout].  The query slots that see a key form at most
// two runs; over the 32 keys of a block inside one conversation the first
// runs join into one interval and the second runs into another (consecutive
// history keys are seen by the history from their slot on and by the t /
// r_out tail from some turn on; consecutive t / r_out keys by overlapping
// runs from their own slot), so the block's two hulls are exact there and a
// superset across a conversation boundary.  A 16-query tile inside a hull
// contributes its precomputed minimum, a tile cut by a hull's end its rows
// inside the hull.  One workgroup of 4 waves per rank: wave w forms block w's
// hulls, then all threads share the stages.  (Its own launch of many small
// workgroups: inside the dK/dV kernel, with one workgroup per CU, these
// dependent loads would stall the matrix cores.)
__global__ __launch_bounds__(256) void dkdv_units_kernel(AttnParams p) {
  const int64_t R = blockIdx.x;
  if (R / p.Hkv >= p.k_counts[0]) return;
  const int4 item = p.k_items[R / p.Hkv];
  const int32_t col = item.x;
  const int kvh = (int)(R % p.Hkv);
  const int b = col / p.NT, n = col - b * p.NT;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  __shared__ int4 sh_hull[4];
  __shared__ int sh_emin[8];
  {
    constexpr int kNone = 0x7FFFFFFF;
    const int key = n * 128 + 32 * w + (lane & 31);
    const int4 iv = key < p.L ? p.kiv[(int64_t)b * p.L + key] : make_int4(0, 0, 0, 0);
    int h0 = iv.x < iv.y ? iv.x : kNone, h1 = iv.x < iv.y ? iv.y : -kNone;
    int h2 = iv.z < iv.w ? iv.z : kNone, h3 = iv.z < iv.w ? iv.w : -kNone;
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) {
      h0 = min(h0, __shfl_xor(h0, off));
      h1 = max(h1, __shfl_xor(h1, off));
      h2 = min(h2, __shfl_xor(h2, off));
      h3 = max(h3, __shfl_xor(h3, off));
    }
    if (lane == 0) sh_hull[w] = make_int4(h0, h1, h2, h3);
    if (tid < 8) sh_emin[tid] = kExpMax;
  }
  __syncthreads();
  int4 hull[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) hull[kb] = sh_hull[kb];
  int mn[8];  // [key block][q', dout]
#pragma unroll
  for (int e = 0; e < 8; ++e) mn[e] = kExpMax;
  const int64_t tcol = (int64_t)b * p.NT + n;
  const int32_t *lst = p.k_list + tcol * p.MT;
  const int64_t ftotal = (int64_t)p.k_nnz[tcol] * p.group * 2;
  const int64_t fbegin = ftotal * item.y / item.z, fend = ftotal * (item.y + 1) / item.z;
  const int64_t hbase = (int64_t)b * p.Hq + (int64_t)kvh * p.group;
  const int64_t gt = hbase * p.MTS, gr = hbase * p.Lp;  // the group's first head in the tile / row tables
  for (int64_t ff = fbegin + tid; ff < fend; ff += 256) {
    const int qh = (int)(ff & 1);
    const int64_t tj = ff >> 1;
    const int hj = (int)(tj % p.group);
    const int m = lst[tj / p.group];
    if (!OPR_DCHECK(p.dbg, (unsigned)m < (unsigned)p.MT, kDbgKList)) continue;
    const int q0 = m * 128 + 64 * qh;
    const int64_t tix = gt + (int64_t)hj * p.MTS + q0 / kTile;
    const int4 e4 = *reinterpret_cast<const int4 *>(p.eqt + tix);
    const int4 d4 = *reinterpret_cast<const int4 *>(p.edot + tix);
    const int eqk[4] = {e4.x, e4.y, e4.z, e4.w}, edk[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t0 = q0 + kTile * k, t1 = t0 + kTile;
      uint32_t cut = 0u;  // blocks whose hull ends inside this tile
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int4 hl = hull[kb];
        if ((hl.x <= t0 && t1 <= hl.y) || (hl.z <= t0 && t1 <= hl.w)) {
          mn[2 * kb] = min(mn[2 * kb], eqk[k]);
          mn[2 * kb + 1] = min(mn[2 * kb + 1], edk[k]);
        } else if ((hl.x < t1 && t0 < hl.y) || (hl.z < t1 && t0 < hl.w)) {
          cut |= 1u << kb;
        }
      }
      if (cut) {
        const int64_t rix = gr + (int64_t)hj * p.Lp + t0;
        for (int r = 0; r < kTile; ++r) {
          const int qs = t0 + r, eqv = p.eqq[rix + r], edv = p.edoq[rix + r];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const int4 hl = hull[kb];
            if (((cut >> kb) & 1u) && ((hl.x <= qs && qs < hl.y) || (hl.z <= qs && qs < hl.w))) {
              mn[2 * kb] = min(mn[2 * kb], eqv);
              mn[2 * kb + 1] = min(mn[2 * kb + 1], edv);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mn[e] = min(mn[e], __shfl_xor(mn[e], off));
  }
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) atomicMin(&sh_emin[e], mn[e]);
  }
  __syncthreads();
  if (tid < 8) p.kunits[R * 8 + tid] = sh_emin[tid];
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
    if (!OPR_DCHECK(p.dbg, (unsigned)tok < (unsigned)p.L, kDbgToken)) continue;
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

// The backward: the dQ kernel first (it also writes the dout plane, its tile
// exponents and the per-slot units that dK/dV reads), then dK/dV and the
// reduce of the cut columns.  ev (optional): events recorded before dQ, after
// it and the small kernel that picks the dK/dV units, and right after the
// dK/dV kernel (so that its span is that kernel alone).
hipError_t launch_attn_bwd_kernels(const opr_attn_in &in, float scale, const void *o, const float *lse,
                                   const void *dout, float *dq, float *dk, float *dv, const AttnWs &ws,
                                   hipStream_t s, hipEvent_t *ev) {
  AttnParams p;
  fill_params(in, scale, ws, &p);
  p.o_in = static_cast<const uint16_t *>(o);
  p.dout_in = static_cast<const uint16_t *>(dout);
  p.lse_in = lse;
  // every column once, plus the most extra parts the work order can make
  const int32_t extra = kSplitSlots / in.Hkv + 1;
  const unsigned gk = (unsigned)(((int64_t)in.B * p.NT + extra) * in.Hkv);
  const dim3 gr((unsigned)extra, (unsigned)in.Hkv);
  if (ev) (void)hipEventRecord(ev[0], s);
  launch_attn_dq_kernel(p, in.D, dq, s);
  dkdv_units_kernel<<<gk, 256, 0, s>>>(p);
  if (ev) (void)hipEventRecord(ev[1], s);
  if (in.D == 64) attn_dkdv_kernel<64><<<gk, 512, 0, s>>>(p, dk, dv);
  else attn_dkdv_kernel<128><<<gk, 512, 0, s>>>(p, dk, dv);
  if (ev) (void)hipEventRecord(ev[2], s);
  if (in.D == 64) dkdv_split_reduce_kernel<64><<<gr, 256, 0, s>>>(p, dk, dv);
  else dkdv_split_reduce_kernel<128><<<gr, 256, 0, s>>>(p, dk, dv);
  return hipGetLastError();
}

}  // namespace opr

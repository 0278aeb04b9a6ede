// Forward kernel of the one-pass masked attention (gfx950).
//
// The kernel runs in attention order: q-tile m is query slots m*128 .. +127
// and K/V rows are slots; results go to the slot's token.  Each lane first
// converts its own query row (RoPE, fp16 with the row's exponent) and writes
// it to the q' plane that the backward reads.  One workgroup of
// 4 waves per (128-slot query tile m, q head h, row b); wave w owns query
// slots m*128 + 32w .. +31, one per lane column.  Work items start longest
// first, spread over the XCDs, with the q heads of one kv group side by side
// on one XCD so that they share K/V tiles in its L2 (q_work_item).
//
// The non-empty 32-key quarters of the q-tile's non-empty 128-key tiles are
// first compacted into a stage list in LDS (a ballot over the tile list and
// its 32x32 sub-block classes), so the main loop has no dependent global
// loads.  K and V of a stage stream from memory straight into LDS (buffer
// loads to LDS with fixed per-lane offsets) through a ring of three buffers:
// while stage i is computed, stages i+1 and i+2 are in flight.  At the start
// of a stage each wave waits only for its own copies of that stage (the
// newer ones stay outstanding), then one barrier.  With D = 128 the short
// stages keep the LDS at 51 KB and the registers at 168 per lane, so three
// workgroups share a CU (three waves per SIMD hide each other's latencies).
// Per stage each wave computes S^T = K Q^T on its 32x32 sub-block, if not
// empty, with fp16 MFMA (fp32 accumulate); a partial sub-block is masked
// with a 64-bit mask built from the query's two runs of key slots; the
// online softmax keeps a running maximum that is only raised when a score
// exceeds it by more than kMaxSlack (so the O accumulator is rarely
// rescaled); O^T += V^T P^T reads V^T from the row-major V tile with
// transposing LDS reads.  The epilogue normalises, writes O (bf16) and the
// natural-log LSE.
#include "attn_common.h"
#include "attn_sched.h"
#include "opr_internal.h"

namespace opr {
namespace {

constexpr int kReadsAhead = 4;  // S products whose K' operand reads are in flight
constexpr int kFwdStageCap = 256;  // 32-key stages per list chunk (2 KB of LDS)

template <int D>
__global__ __launch_bounds__(256, 3) void attn_fwd_kernel(AttnParams p, uint16_t *o, float *lse) {
  constexpr int NS = D / 16;   // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;  // 32-wide blocks of the head dim
  constexpr int RB = Tile<D>::RB;
  constexpr int TB = 32 * RB;  // one 32-row tile
  constexpr int BUF = 2 * TB;  // K tile, V tile
  // A ring of three separate LDS objects (not one array indexed by the stage):
  // the compiler then knows that the asynchronous copies into two of them do
  // not write the third, and lets them run under the reads of the current
  // stage.  With the short stage list, three workgroups fit a CU.
  __shared__ __attribute__((aligned(1024))) char buf0[BUF];
  __shared__ __attribute__((aligned(1024))) char buf1[BUF];
  __shared__ __attribute__((aligned(1024))) char buf2[BUF];
  __shared__ uint2 stages[kFwdStageCap];
  __shared__ int sh_count, sh_next;

  const QItem it = q_work_item(p.q_order, p.MT, p.Hkv, p.group, (int64_t)p.B * p.MT);
  if (!it.valid) return;
  const int j = it.j, m = it.m, kvh = it.kvh, b = it.b;
  const int h = kvh * p.group + j;

  const int tid = threadIdx.x, w = uniform(tid >> 6), lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int q = m * 128 + 32 * w + li;
  const int64_t kvplane = (int64_t)b * p.Hkv + kvh;
  const int ek = plane_exponent(p.mk[kvplane]);
  const int ev = plane_exponent(p.mv[kvplane]);

  // Prologue: q of the lane's token (its half of the head dims, the partner
  // lane l ^ 32 holds the other half), rotated by RoPE at the slot's position
  // id, as fp16 with the row's own exponent eq; written to the q' plane with
  // eq (and eq's minimum over each 16-slot tile) for the backward.  Lane g
  // holds dims 16 s + 8 g + e, so each rotation pair (d, d + D/2) is the
  // lane's own (k-steps s and s + NS/2).  The loads of q are issued here; the
  // conversion (convert_q) runs once the stage list is built and the first
  // K/V tiles stream in, so that their latencies overlap.
  const int64_t hq_row = ((int64_t)b * p.Hq + h) * p.Lp + q;
  int32_t tok = q < p.L ? p.slot_tok[(int64_t)b * p.L + q] : -1;
  if (tok >= 0 && !OPR_DCHECK(p.dbg, tok < p.L, kDbgToken)) tok = -1;
  uint4 wv[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) wv[s] = make_uint4(0u, 0u, 0u, 0u);
  if (tok >= 0) {
    const uint16_t *src = p.q_in + (((int64_t)b * p.L + tok) * p.Hq + h) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) wv[s] = *reinterpret_cast<const uint4 *>(src + 16 * s);
  }
  // the (cos, sin) pairs of the lane's 8 rotation pairs of every k-step, 16
  // bytes (two pairs) per load; the table covers every slot below Lp, and a
  // PAD row's q is zero whatever its angle, so they need no condition
  float4 cs4[NS / 2][4];
  {
    const float4 *t4 = reinterpret_cast<const float4 *>(p.rope + ((int64_t)b * p.Lp + q) * (D / 2) + 8 * g);
#pragma unroll
    for (int s = 0; s < NS / 2; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) cs4[s][e] = t4[8 * s + e];  // pairs 16 s + 2e, 16 s + 2e + 1 of the lane's 8 g
  }
  f16x8 qb[NS];
  float fs;  // raw score -> log2 units: scale log2(e) 2^-(eq + ek)
  // Two passes over the rotation pairs (the row's largest |q'|, then the
  // conversion) from registers, so the rotated row is never held whole.
  auto rotate = [&](int s, float (&x1)[8], float (&x2)[8]) {
    const uint16_t *lo = reinterpret_cast<const uint16_t *>(&wv[s]);
    const uint16_t *hi = reinterpret_cast<const uint16_t *>(&wv[s + NS / 2]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float4 c4 = cs4[s][e >> 1];
      const float2 c = (e & 1) ? make_float2(c4.z, c4.w) : make_float2(c4.x, c4.y);
      rope_pair(bf16_to_f32(lo[e]), bf16_to_f32(hi[e]), c, x1[e], x2[e]);
    }
  };
  auto convert_q = [&]() {
    uint32_t mx = 0u;  // float bits of the row's largest |q'| (integer order)
#pragma unroll
    for (int s = 0; s < NS / 2; ++s) {
      float x1[8], x2[8];
      rotate(s, x1, x2);
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = max(mx, max(__float_as_uint(fabsf(x1[e])), __float_as_uint(fabsf(x2[e]))));
    }
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
    const int eq = mx > 0u ? plane_exponent(mx) : kExpMax;
    uint16_t *dst = p.qr + hq_row * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS / 2; ++s) {
      float x1[8], x2[8];
      rotate(s, x1, x2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qb[s][e] = (_Float16)ldexpf(x1[e], eq);
        qb[s + NS / 2][e] = (_Float16)ldexpf(x2[e], eq);
      }
      *reinterpret_cast<f16x8 *>(dst + 16 * s) = qb[s];
      *reinterpret_cast<f16x8 *>(dst + 16 * (s + NS / 2)) = qb[s + NS / 2];
    }
    int emin = eq;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) emin = min(emin, __shfl_xor(emin, off));
    if (g == 0) p.eqq[hq_row] = eq;
    if ((lane & 47) == 0) p.eqt[((int64_t)b * p.Hq + h) * p.MTS + q / kTile] = emin;
    fs = ldexpf(p.scale_log2, -(eq + ek));
  };
  // key slots this query sees: [iv.x, iv.y) and [iv.z, iv.w)
  const int4 iv = q < p.L ? p.qiv[(int64_t)b * p.L + q] : make_int4(0, 0, 0, 0);
  OperandOffsets<D> of;
  of.init(lane);
  TileCopy<D, 4, 32> tc;
  tc.init(w, lane);
  constexpr int kCopies = 2 * TileCopy<D, 4, 32>::NI;  // copy instructions per wave and stage (K and V)
  const uint32_t plane_bytes = (uint32_t)p.Lp * D * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.kr + kvplane * p.Lp * D, plane_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.vr + kvplane * p.Lp * D, plane_bytes);

  const int64_t trow = (int64_t)b * p.MT + m;
  const int nnz = p.q_nnz[trow];
  const int32_t *lst = p.q_list + trow * p.NT;
  const uint32_t *subs = p.sub_class + trow * p.NT;

  auto issue = [&](int k0, char *nb) {
    tc.issue(rk, k0, nb, w);
    tc.issue(rv, k0, nb + TB, w);
  };

  // the stage list (32-key quarters) is built in chunks of up to kFwdStageCap stages
  int tnext = 0, ns = 0;
  auto build = [&]() {
    __syncthreads();  // the previous chunk's stages and buffers are no longer read
    if (w == 0) {
      int t = tnext;
      const int c = build_q_quarters<kFwdStageCap>(lst, subs, nnz, p.NT, &t, stages, lane, p.dbg);
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
  convert_q();  // while the first K/V tiles stream in

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = zero_f32x16();
  float mrow = -INFINITY, lrow = 0.0f;
  for (;;) {
    // stage i reads `buf` (buf[i % 3]) while stages i+1 and i+2 stream in; at
    // its start it waits for its own tiles only (the copies of stage i+1, if
    // any, are the newest kCopies of the wave), then refills the buffer that
    // stage i-1 used with stage i+2.  The stage list is fixed for the chunk,
    // so both descriptors are read before the barrier, together.
    auto stage = [&](int i, const char *buf, char *nxt2) {
      // (an entry past the list is read but not used)
      const uint2 d0 = stages[i];
      const uint32_t x2 = stages[min(i + 2, kFwdStageCap - 1)].x;
      const uint2 desc = uniform(d0);
      const int k2 = uniform((int)x2);
      if (i + 1 < ns) wait_older_copies_and_barrier<kCopies>();
      else wait_older_copies_and_barrier<0>();
      if (i + 2 < ns) issue(k2, nxt2);
      const uint32_t c = (desc.y >> (2 * w)) & 3u;
      if (c == 0) return;
      const int k0 = (int)desc.x;
      const char *Kt = buf, *Vt = buf + TB;

      // S^T = K Q^T for the stage's 32 keys (straight-line code: the mask is
      // exact, so masked scores are -inf and their p = 0)
      f32x16 sc = zero_f32x16();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < NS; ++st) sc = mfma32x32x16(lds_f16x8(Kt + of.row8[st]), qb[st], sc);
      sched_lds_reads_ahead<NS, kReadsAhead, 1>();
      __builtin_amdgcn_sched_barrier(0);
      if (c != 2) {
        // lane group g holds keys 16h + 8g + 0..7 of the 32
        const uint64_t mk = (range_bits(iv.x, iv.y, k0) | range_bits(iv.z, iv.w, k0)) >> (8 * g);
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = mask_select(mk, 16 * (r >> 3) + (r & 7), sc[r]);
      }
      float mx = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
      mx = pair_max_xor32(mx) * fs;
      if (__ballot(mx > mrow + kMaxSlack) != 0) {  // raise the running maximum (wave-uniform)
        const float mnew = fmaxf(mrow, mx);
        const float alpha = (mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(mrow - mnew);
        lrow *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        mrow = mnew;
      }
      // p * 2^kPExp with p = 2^(score - running max) <= 2^kMaxSlack
      const float cexp = (float)kPExp - (mrow == -INFINITY ? 0.0f : mrow);
      f16x8 pb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) pb[r >> 3][r & 7] = (_Float16)__builtin_amdgcn_exp2f(fmaf(sc[r], fs, cexp));
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) lrow = sum_f16x8(pb[hh], lrow);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = mfma32x32x16(tile_col8<D>(Vt, of, 16 * hh, db), pb[hh], oacc[db]);
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

  const float lsum = lrow + __shfl_xor(lrow, 32);
  if (tok >= 0) {  // every slot below L holds a token
    // O = acc / sum, acc in units 2^ev (v) times 2^kPExp (shared with sum)
    const float inv = lsum > 0.0f ? ldexpf(1.0f / lsum, -ev) : 0.0f;
    uint16_t *orow = o + (((int64_t)b * p.L + tok) * p.Hq + h) * D;
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
      lse[((int64_t)b * p.Hq + h) * p.L + tok] =
          lsum > 0.0f ? (mrow + log2f(lsum) - (float)kPExp) * kLn2 : -INFINITY;
  }
}

}  // namespace

void fill_params(const opr_attn_in &in, float scale, const AttnWs &ws, AttnParams *p);

hipError_t launch_attn_fwd_kernel(const opr_attn_in &in, float scale, void *o, float *lse,
                                  const AttnWs &ws, hipStream_t s) {
  AttnParams p;
  fill_params(in, scale, ws, &p);
  p.q_in = static_cast<const uint16_t *>(in.q);
  const unsigned grid = (unsigned)q_grid((int64_t)in.B * p.MT, in.Hkv, p.group);
  uint16_t *o16 = static_cast<uint16_t *>(o);
  if (in.D == 64) attn_fwd_kernel<64><<<grid, 256, 0, s>>>(p, o16, lse);
  else attn_fwd_kernel<128><<<grid, 256, 0, s>>>(p, o16, lse);
  return hipGetLastError();
}

}  // namespace opr

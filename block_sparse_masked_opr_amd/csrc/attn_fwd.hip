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
// The non-empty 64-key halves of the q-tile's non-empty 128-key tiles are
// first compacted into a stage list in LDS (a ballot over the tile list and
// its 32x32 sub-block classes), so the main loop has no dependent global
// loads.  Stages are double buffered: while stage i is computed, K and V of
// stage i+1 stream from memory straight into LDS (buffer loads to LDS with
// fixed per-lane offsets); one barrier per stage.  Per stage each wave
// computes S^T = K Q^T on its non-empty 32x32 sub-blocks with fp16 MFMA
// (fp32 accumulate); partial sub-blocks are masked with a 64-bit mask built
// from the query's two runs of key slots; the online softmax keeps a running maximum
// that is only raised when a score exceeds it by more than kMaxSlack (so the
// O accumulator is rarely rescaled); O^T += V^T P^T reads V^T from the
// row-major V tile with transposing LDS reads.  The epilogue normalises,
// writes O (bf16) and the natural-log LSE.
#include "attn_common.h"
#include "attn_sched.h"
#include "opr_internal.h"

namespace opr {
namespace {

constexpr int kReadsAhead = 4;  // S products whose K' operand reads are in flight

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnParams p, uint16_t *o, float *lse) {
  constexpr int NS = D / 16;   // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;  // 32-wide blocks of the head dim
  constexpr int TB = Tile<D>::BYTES, RB = Tile<D>::RB;
  constexpr int BUF = 2 * TB;  // K tile, V tile
  // Two separate LDS objects (not one array indexed by stage parity): the
  // compiler then knows that the asynchronous copy into one buffer does not
  // write the other, and lets it run under the reads of the current stage.
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
  const int ek = plane_exponent(p.mk[kvplane]);
  const int ev = plane_exponent(p.mv[kvplane]);

  // Prologue: q of the lane's token (its half of the head dims, the partner
  // lane l ^ 32 holds the other half), rotated by RoPE at the slot's position
  // id, as fp16 with the row's own exponent eq; written to the q' plane with
  // eq (and eq's minimum over each 16-slot tile) for the backward.  Lane g
  // holds dims 16 s + 8 g + e, so each rotation pair (d, d + D/2) is the
  // lane's own (k-steps s and s + NS/2).  The loads are issued here; the
  // conversion (convert_q) runs once the stage list is built and the first
  // K/V tiles stream in, so that their latencies overlap.
  const int64_t hq_row = ((int64_t)b * p.Hq + h) * p.Lp + q;
  const int32_t tok = q < p.L ? p.slot_tok[(int64_t)b * p.L + q] : -1;
  uint4 wv[NS];
  float2 csv[NS / 2][8];
#pragma unroll
  for (int s = 0; s < NS; ++s) wv[s] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int s = 0; s < NS / 2; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) csv[s][e] = make_float2(1.0f, 0.0f);
  if (tok >= 0) {
    const uint16_t *src = p.q_in + (((int64_t)b * p.L + tok) * p.Hq + h) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) wv[s] = *reinterpret_cast<const uint4 *>(src + 16 * s);
    const float2 *cs = p.rope + ((int64_t)b * p.Lp + q) * (D / 2) + 8 * g;
#pragma unroll
    for (int s = 0; s < NS / 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) csv[s][e] = cs[16 * s + e];
  }
  f16x8 qb[NS];
  float fs;  // raw score -> log2 units: scale log2(e) 2^-(eq + ek)
  auto convert_q = [&]() {
    float x[NS][8];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint16_t *e16 = reinterpret_cast<const uint16_t *>(&wv[s]);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[s][e] = bf16_to_f32(e16[e]);
    }
#pragma unroll
    for (int s = 0; s < NS / 2; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x1 = x[s][e], x2 = x[s + NS / 2][e];
        rope_pair(x1, x2, csv[s][e], x[s][e], x[s + NS / 2][e]);
      }
    }
    uint32_t mx = 0u;  // float bits of the row's largest |q'| (integer order)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = max(mx, __float_as_uint(fabsf(x[s][e])));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
    const int eq = mx > 0u ? plane_exponent(mx) : kExpMax;
    uint16_t *dst = p.qr + hq_row * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[s][e] = (_Float16)ldexpf(x[s][e], eq);
      *reinterpret_cast<f16x8 *>(dst + 16 * s) = qb[s];
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
  TileCopy<D> tc;
  tc.init(w, lane);
  const uint32_t plane_bytes = (uint32_t)p.Lp * D * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.kr + kvplane * p.Lp * D, plane_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.vr + kvplane * p.Lp * D, plane_bytes);

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = zero_f32x16();
  float mrow = -INFINITY, lrow = 0.0f;

  const int64_t trow = (int64_t)b * p.MT + m;
  const int nnz = p.q_nnz[trow];
  const int32_t *lst = p.q_list + trow * p.NT;
  const uint32_t *subs = p.sub_class + trow * p.NT;

  auto issue = [&](int k0, char *nb) {
    tc.issue(rk, k0, nb, w);
    tc.issue(rv, k0, nb + TB, w);
  };

  // the stage list is built in chunks of up to kStageCap stages
  int tnext = 0, ns = 0;
  auto build = [&]() {
    __syncthreads();  // the previous chunk's stages and buffers are no longer read
    if (w == 0) {
      int t = tnext;
      const int c = build_q_stages(lst, subs, nnz, &t, stages, lane);
      if (lane == 0) {
        sh_count = c;
        sh_next = t;
      }
    }
    __syncthreads();
    ns = uniform(sh_count);
    tnext = uniform(sh_next);
    if (ns > 0) issue(uniform((int)stages[0].x), buf0);
  };
  build();
  convert_q();  // while the first K/V tiles stream in
  for (;;) {
    // stage i reads `buf` while stage i+1 streams into `nxt`
    auto stage = [&](int i, const char *buf, char *nxt) {
      wait_all_and_barrier();
      if (i + 1 < ns) issue(uniform((int)stages[i + 1].x), nxt);
      const uint2 desc = uniform(stages[i]);
      const uint32_t c0 = (desc.y >> (4 * w)) & 3u, c1 = (desc.y >> (4 * w + 2)) & 3u;
      if ((c0 | c1) == 0) return;
      const int k0 = (int)desc.x;
      const char *Kt = buf, *Vt = buf + TB;

      // Both 32-key sub-blocks always (straight-line code): the mask is exact,
      // so an empty one gives -inf scores and p = 0.
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = zero_f32x16();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s[kb] = mfma32x32x16(lds_f16x8(Kt + kb * 32 * RB + of.row8[st]), qb[st], s[kb]);
      }
      sched_lds_reads_ahead<2 * NS, kReadsAhead, 1>();
      __builtin_amdgcn_sched_barrier(0);
      if (c0 != 2 || c1 != 2) {
        uint64_t mk = range_bits(iv.x, iv.y, k0) | range_bits(iv.z, iv.w, k0);
        mk >>= 8 * g;  // lane group g holds keys 16h + 8g + 0..7 of each 32-key block
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = mask_select(mk, 32 * kb + 16 * (r >> 3) + (r & 7), s[kb][r]);
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * fs;
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
      f16x8 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pb[kb][r >> 3][r & 7] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[kb][r], fs, cexp));
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) lrow = sum_f16x8(pb[kb][hh], lrow);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            oacc[db] = mfma32x32x16(tile_col8<D>(Vt, of, 32 * kb + 16 * hh, db), pb[kb][hh], oacc[db]);
        }
      }
    };
    for (int i = 0; i < ns; i += 2) {
      stage(i, buf0, buf1);
      if (i + 1 < ns) stage(i + 1, buf1, buf0);
    }
    if (tnext >= nnz) break;
    build();
  }

  const float lsum = lrow + __shfl_xor(lrow, 32);
  if (q < p.L) {
    const int tok = p.slot_tok[(int64_t)b * p.L + q];
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

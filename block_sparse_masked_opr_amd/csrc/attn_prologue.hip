// Prologue kernels of the attention path.  Everything here is indexed by
// slot (attention order): slot s < L holds token slot_tok[s] of the layout,
// slots L .. Lp-1 are empty and padded with zeros.
//  - the RoPE table at the slots' strategic position ids (and the reset of
//    the plane maxima),
//  - the largest magnitude of every (row, kv head) plane of k and v,
//  - head-major fp16 copies of q, k (after RoPE), v and dout in slot order:
//    k and v with one power-of-two scale per plane, q and dout with one per
//    64-slot tile of each (row, head), found while the tile is converted,
//  - the backward preprocessing delta = rowsum(dout * o), fused with the dout
//    copy, and its scaling into the units of the backward kernels.
//
// RoPE (rotate-half): pair (j, j + D/2) of a head vector is rotated by
// pos * theta^(-2j/D).  The angle and its cosine and sine are computed in
// float64 (positions reach ~2.4e5, where a float32 angle would be off by
// ~1e-2 rad); the rotation itself runs in float32.
#include "attn_common.h"
#include "opr_internal.h"

namespace opr {
namespace {

// table[b][s][j] = (cos, sin) of pos(b, slot_tok[s]) * theta^(-2j/D); PAD
// and s >= L use position 0.  The first n_zero threads also clear zero_words
// (the plane maxima start at 0).
__global__ __launch_bounds__(256) void rope_table_kernel(int32_t B, int32_t L, int32_t Lp, int32_t half,
                                                         double log2_theta, const int32_t *tok_pos,
                                                         const int32_t *slot_tok, float2 *table,
                                                         uint32_t *zero_words, int32_t n_zero) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid < n_zero) zero_words[gid] = 0u;
  const int64_t total = (int64_t)B * Lp * half;
  if (gid >= total) return;
  const int32_t j = (int32_t)(gid % half);
  const int64_t bt = gid / half;
  const int32_t t = (int32_t)(bt % Lp);
  const int32_t b = (int32_t)(bt / Lp);
  const int32_t pos = t < L ? tok_pos[(int64_t)b * L + slot_tok[(int64_t)b * L + t]] : 0;
  const double inv_freq = exp2(-(2.0 * j / (2.0 * half)) * log2_theta);
  double s, c;
  sincos((double)pos * inv_freq, &s, &c);
  table[gid] = make_float2((float)c, (float)s);
}

// Largest |x| of each (row, head) plane of x [B][L][H][D] bf16, times
// `factor` (sqrt(2) bound of RoPE on a pair, rounded up), into pmax[b][h] as
// float bits.  A workgroup covers kAbsTokens tokens of up to HPB heads:
// thread (token row r, head hl, chunk j) reads 16-byte chunk j of head hl of
// every tpr-th token from r, so each D/8-lane group reads one head's whole row
// and a wave reads contiguous runs; with fewer heads than HPB the spare
// threads take further token rows.
constexpr int kAbsTokens = 64;

// One launch covers k and v: blockIdx.y runs over the head blocks of job 0,
// then job 1.
struct AbsmaxJob {
  const uint16_t *x;  // [B][L][H][D] bf16
  uint32_t *pmax;     // [B][H]
  int32_t H;
  int32_t hb_end;     // one past this job's last head block (cumulative)
  float factor;
};

template <int D>
__global__ __launch_bounds__(256) void absmax_kernel(int32_t L, AbsmaxJob j0, AbsmaxJob j1) {
  constexpr int CPH = D / 8, HPB = 256 / CPH;
  const int yb = blockIdx.y;
  const bool in0 = yb < j0.hb_end;
  const uint16_t *x = in0 ? j0.x : j1.x;
  uint32_t *pmax = in0 ? j0.pmax : j1.pmax;
  const int32_t H = in0 ? j0.H : j1.H;
  const float factor = in0 ? j0.factor : j1.factor;
  const int hb = yb - (in0 ? 0 : j0.hb_end);
  const int b = blockIdx.z, tid = threadIdx.x;
  // the block's heads [hb * HPB, hb * HPB + nh); threads beyond one token row
  // of them take further tokens (tpr token rows per pass)
  const int nh = min(HPB, H - hb * HPB);
  const int row = nh * CPH, tpr = 256 / row;
  const int r = tid / row, hl = (tid % row) / CPH, j = tid % CPH;
  const int h = hb * HPB + hl;
  const int t0 = blockIdx.x * kAbsTokens;
  uint32_t m = 0u;  // float bits of the largest |x| (non-negative: integer order)
  if (r < tpr) {
    const uint16_t *src = x + (((int64_t)b * L + t0) * H + h) * D + j * 8;
    const int nt = min(kAbsTokens, L - t0);
#pragma unroll 8
    for (int t = r; t < nt; t += tpr)
      m = max(m, absmax8_bf16_bits(*reinterpret_cast<const uint4 *>(src + (int64_t)t * H * D)));
  }
#pragma unroll
  for (int off = CPH / 2; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  // one atomic per head and workgroup: the token rows meet in LDS first
  __shared__ uint32_t hm[256 / CPH];
  if (tid < HPB) hm[tid] = 0u;
  __syncthreads();
  if (j == 0 && r < tpr && m > 0u) atomicMax(&hm[hl], m);
  __syncthreads();
  if (tid < nh && hm[tid] > 0u)
    atomicMax(pmax + (int64_t)b * H + hb * HPB + tid, __float_as_uint(__uint_as_float(hm[tid]) * factor));
}

// One workgroup per (64-slot block, group of kPackHeads heads, row): 4
// threads per slot, each owning D/8 rotation pairs (j, j + D/2), so that a
// wave covers exactly one kTile-slot tile.  The threads keep the slot's RoPE
// cosines and sines in registers and walk the heads.
// x: [B][L][H][D] bf16 -> rows [B][H][Lp][D] in slot order, fp16(x' * 2^e),
// x' = RoPE(x) or x.
// TILE = false: e is the exponent of the head's plane maximum pmax[b][h].
// TILE = true: e is the exponent of the largest |x'| of the wave's tile of the
// head (kExpMax for an all-zero tile), reduced inside the wave; it is stored
// in etile[b][h][tile] (group_min_kernel takes the minimum over each group).
// Slots s >= L are zero.
constexpr int kPackHeads = 8;
constexpr int kPackSlots = 64;

template <int D, bool ROPE, bool TILE>
__global__ __launch_bounds__(256) void pack_kernel(int32_t L, int32_t Lp, int32_t H, int32_t group,
                                                   const uint16_t *x, const int32_t *slot_tok,
                                                   const float2 *table, const uint32_t *pmax,
                                                   uint16_t *rows, int32_t *etile) {
  constexpr int HALF = D / 2;
  constexpr int PER = HALF / 4;  // pairs per thread (4 threads per slot)
  static_assert(kPackSlots == 4 * kTile, "a wave covers one tile");
  const int hgroups = (H + kPackHeads - 1) / kPackHeads;
  const int h0 = (int)(blockIdx.x % (unsigned)hgroups) * kPackHeads;
  const int blk = (int)(blockIdx.x / (unsigned)hgroups);
  const int t0 = blk * kPackSlots, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tt = tid >> 2, part = tid & 3;
  const int t = t0 + tt;
  const int j0 = part * PER;
  const int32_t tok = t < L ? slot_tok[(int64_t)b * L + t] : -1;
  float2 cs[PER];
  if (ROPE) {
    const float2 *row = table + ((int64_t)b * Lp + t) * HALF + j0;
#pragma unroll
    for (int e = 0; e < PER; ++e) cs[e] = row[e];
  }
  const int h1 = min(H, h0 + kPackHeads);
#pragma unroll 2
  for (int h = h0; h < h1; ++h) {
    float lo[PER], hi[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) lo[e] = hi[e] = 0.0f;
    if (tok >= 0) {
      const uint16_t *src = x + (((int64_t)b * L + tok) * H + h) * D;
      uint16_t lb[PER], hb[PER];
#pragma unroll
      for (int c = 0; c < PER; c += 8) {
        *reinterpret_cast<uint4 *>(&lb[c]) = *reinterpret_cast<const uint4 *>(src + j0 + c);
        *reinterpret_cast<uint4 *>(&hb[c]) = *reinterpret_cast<const uint4 *>(src + HALF + j0 + c);
      }
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        lo[e] = bf16_to_f32(lb[e]);
        hi[e] = bf16_to_f32(hb[e]);
        if (ROPE) {
          const float x1 = lo[e], x2 = hi[e];
          lo[e] = x1 * cs[e].x - x2 * cs[e].y;
          hi[e] = x2 * cs[e].x + x1 * cs[e].y;
        }
      }
    }
    int ex;
    if (TILE) {
      uint32_t m = 0u;  // float bits of the largest magnitude (integer order)
#pragma unroll
      for (int e = 0; e < PER; ++e) m = max(m, max(__float_as_uint(fabsf(lo[e])), __float_as_uint(fabsf(hi[e]))));
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
      ex = m > 0u ? plane_exponent(m) : kExpMax;
      if (lane == 0) etile[((int64_t)b * H + h) * (Lp / kTile) + t0 / kTile + wave] = ex;
    } else {
      ex = plane_exponent(pmax[(int64_t)b * H + h]);
    }
    uint16_t lq[PER], hq[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      lq[e] = f32_to_f16_bits(ldexpf(lo[e], ex));
      hq[e] = f32_to_f16_bits(ldexpf(hi[e], ex));
    }
    uint16_t *dst = rows + (((int64_t)b * H + h) * Lp + t) * D;
#pragma unroll
    for (int c = 0; c < PER; c += 8) {
      *reinterpret_cast<uint4 *>(dst + j0 + c) = *reinterpret_cast<const uint4 *>(&lq[c]);
      *reinterpret_cast<uint4 *>(dst + HALF + j0 + c) = *reinterpret_cast<const uint4 *>(&hq[c]);
    }
  }
}

// Backward preprocessing, one workgroup per (64-slot block, group of
// kPackHeads q heads, row) with the thread layout of pack_kernel (a wave per
// tile): per head and slot s, with t = slot_tok[s] the token there,
//   dsc[b][h][s] = sum_d dout * o of token t (float32 over bf16 inputs; the
//                  units are applied by scale_delta_kernel),
// and dout goes to its fp16 copy with the exponent of the tile's largest
// |dout| (kExpMax for an all-zero tile), stored in etile[b][h][tile].
template <int D>
__global__ __launch_bounds__(256) void delta_pack_kernel(int32_t L, int32_t Lp, int32_t H, int32_t group,
                                                         const uint16_t *o, const uint16_t *dout,
                                                         const int32_t *slot_tok, uint16_t *rows, float *dsc,
                                                         int32_t *etile) {
  constexpr int HALF = D / 2;
  constexpr int PER = HALF / 4;
  const int hgroups = (H + kPackHeads - 1) / kPackHeads;
  const int h0 = (int)(blockIdx.x % (unsigned)hgroups) * kPackHeads;
  const int blk = (int)(blockIdx.x / (unsigned)hgroups);
  const int t0 = blk * kPackSlots, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tt = tid >> 2, part = tid & 3;
  const int t = t0 + tt;
  const int j0 = part * PER;
  const int32_t tok = t < L ? slot_tok[(int64_t)b * L + t] : -1;
  const int h1 = min(H, h0 + kPackHeads);
#pragma unroll 2
  for (int h = h0; h < h1; ++h) {
    uint4 dw[PER / 4], ow[PER / 4];  // bf16 words, low halves then high halves
#pragma unroll
    for (int c = 0; c < PER / 4; ++c) dw[c] = ow[c] = make_uint4(0, 0, 0, 0);
    if (tok >= 0) {
      const int64_t base = (((int64_t)b * L + tok) * H + h) * D;
#pragma unroll
      for (int c = 0; c < PER / 8; ++c) {
        dw[c] = *reinterpret_cast<const uint4 *>(dout + base + j0 + 8 * c);
        dw[PER / 8 + c] = *reinterpret_cast<const uint4 *>(dout + base + HALF + j0 + 8 * c);
        ow[c] = *reinterpret_cast<const uint4 *>(o + base + j0 + 8 * c);
        ow[PER / 8 + c] = *reinterpret_cast<const uint4 *>(o + base + HALF + j0 + 8 * c);
      }
    }
    float acc = 0.0f;
    uint32_t m = 0u;
#pragma unroll
    for (int c = 0; c < PER / 4; ++c) {
      acc = dot2_bf16(ow[c].x, dw[c].x, acc);
      acc = dot2_bf16(ow[c].y, dw[c].y, acc);
      acc = dot2_bf16(ow[c].z, dw[c].z, acc);
      acc = dot2_bf16(ow[c].w, dw[c].w, acc);
      m = max(m, absmax8_bf16_bits(dw[c]));
    }
    acc += __shfl_xor(acc, 1);  // the 4 threads of a slot
    acc += __shfl_xor(acc, 2);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    const int ex = m > 0u ? plane_exponent(m) : kExpMax;
    if (lane == 0) etile[((int64_t)b * H + h) * (Lp / kTile) + t0 / kTile + wave] = ex;
    if (part == 0) dsc[((int64_t)b * H + h) * Lp + t] = acc;
    const uint16_t *dl = reinterpret_cast<const uint16_t *>(dw);
    uint16_t lq[PER], hq[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      lq[e] = f32_to_f16_bits(ldexpf(bf16_to_f32(dl[e]), ex));
      hq[e] = f32_to_f16_bits(ldexpf(bf16_to_f32(dl[PER + e]), ex));
    }
    uint16_t *dst = rows + (((int64_t)b * H + h) * Lp + t) * D;
#pragma unroll
    for (int c = 0; c < PER; c += 8) {
      *reinterpret_cast<uint4 *>(dst + j0 + c) = *reinterpret_cast<const uint4 *>(&lq[c]);
      *reinterpret_cast<uint4 *>(dst + HALF + j0 + c) = *reinterpret_cast<const uint4 *>(&hq[c]);
    }
  }
}

// emin[2 * (b * Hkv + kv)] = the smallest tile exponent of the kv group's
// heads, etile [B][Hq][MTS]: one workgroup per (row, kv group).
__global__ __launch_bounds__(256) void group_min_kernel(int32_t Hq, int32_t group, int32_t MTS,
                                                        const int32_t *etile, int32_t *emin) {
  __shared__ int32_t wmin[4];
  const int64_t gk = blockIdx.x;  // b * Hkv + kv
  const int64_t n = (int64_t)group * MTS;
  const int32_t *src = etile + gk * n;  // the group's heads are consecutive
  int32_t m = kExpMax;
  for (int64_t i = threadIdx.x; i < n; i += 256) m = min(m, src[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = min(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) wmin[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) emin[2 * gk] = min(min(wmin[0], wmin[1]), min(wmin[2], wmin[3]));
}

// Units of the backward, per slot s of q head h in kv group kv, with eq, edo
// the tile exponents of q and dout at s and eqr, edor their group minima:
//   lse2[b][h][s] = lse * log2(e) - kPdvExp + (edo - edor): the dK/dV kernel's
//       fp16(P * 2^(kPdvExp - (edo - edor))) then cancels the dout tile scale in
//       dV^T += dO'^T P^T; +inf where the row has no key or s >= L, so that
//       recomputed probabilities are exactly 0;
//   dsc[b][h][s] *= 2^(edo + ev - kDsShift - kPdvExp - (eq - eqr)): delta in
//       the units of dP = dO' V'^T of that slot, shifted so that
//       dS' = P' (dP dss - delta) comes out in units that Q' turns into the
//       group-wide units of dK.
// One thread per (b, h, s).
__global__ __launch_bounds__(256) void scale_delta_kernel(int32_t B, int32_t L, int32_t Lp, int32_t Hq, int32_t group,
                                                          const float *lse, const int32_t *slot_tok,
                                                          const int32_t *eqt, const int32_t *edot,
                                                          const int32_t *eref, const uint32_t *mv, float *dsc,
                                                          float *lse2) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)B * Hq * Lp) return;
  const int32_t sl = (int32_t)(gid % Lp);
  const int64_t bh = gid / Lp;
  const int h = (int)(bh % Hq);
  const int64_t b = bh / Hq;
  const int kv = h / group, Hkv = Hq / group;
  const int64_t tix = bh * (Lp / kTile) + sl / kTile;
  const int eq = eqt[tix], edo = edot[tix];
  const int eqr = eref[2 * (b * Hkv + kv)], edor = eref[2 * (b * Hkv + kv) + 1];
  const int ev = plane_exponent(mv[b * Hkv + kv]);
  float l2 = INFINITY;
  if (sl < L) {
    const float l = lse[bh * L + slot_tok[b * L + sl]];
    if (l != -INFINITY) l2 = l * kLog2e - (float)kPdvExp + (float)(edo - edor);
  }
  lse2[gid] = l2;
  dsc[gid] = ldexpf(dsc[gid], edo + ev - kDsShift - kPdvExp - (eq - eqr));
}

// Longest-first work order (see q_work_item): the q-tile rows (b*MT + m) by
// decreasing number of non-empty 64-key halves over their tile lists - the
// stages of a forward or dQ workgroup - and the dK/dV work items by
// decreasing number of non-empty 64-query halves.  A k-tile column is one
// item, or, when its halves exceed the cap, s = ceil(halves / cap) items
// that each take 1/s of its stage range (a column seen by every later turn
// of a long conversation would otherwise outlast all other workgroups).
// The cap is max(kMinSplit, ceil(total halves * Hkv / kSplitSlots)): one
// workgroup's share of the whole when one workgroup runs per CU on 256 CUs
// (a smaller cap cut columns of balanced workloads for no gain in a
// longest-first simulation of the schedule), and it keeps the extra items
// below kSplitSlots / Hkv.  Part 0 of a cut column writes dK/dV itself;
// parts 1..s-1 take partial slots, which dkdv_split_reduce_kernel adds in
// order.  One workgroup: per-item costs, then a counting sort (costs above
// kOrderBins - 1 share the last bin; ties in any order).
constexpr int kOrderThreads = 1024, kOrderBins = 4096;
constexpr int32_t kMinSplit = 16;

__device__ int64_t block_sum_i64(int64_t v, int64_t *red) {
  const int tid = threadIdx.x;
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  int64_t t = 0;
  for (int i = 0; i < kOrderThreads / 64; ++i) t += red[i];
  __syncthreads();
  return t;
}

// Exclusive scan of bins[] in place (bins[i] becomes the first rank of bin i).
__device__ void scan_bins(int32_t *bins, int32_t *wave_sum) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int PER = kOrderBins / kOrderThreads;
  int32_t v[PER], run = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    v[e] = bins[tid * PER + e];
    run += v[e];
  }
  int32_t incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_sum[wv] = incl;
  __syncthreads();
  int32_t base = 0;
  for (int i = 0; i < wv; ++i) base += wave_sum[i];
  int32_t start = base + incl - run;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    bins[tid * PER + e] = start;
    start += v[e];
  }
  __syncthreads();
}

__device__ __forceinline__ int32_t parts_of(int32_t c, int32_t cap) { return c > cap ? (c + cap - 1) / cap : 1; }

__global__ __launch_bounds__(kOrderThreads) void work_order_kernel(int32_t n_rows, int32_t n_cols, int32_t MT,
                                                                   int32_t NT, int32_t Hkv, const uint32_t *sub_class,
                                                                   const int32_t *q_nnz, const int32_t *q_list,
                                                                   const int32_t *k_nnz, const int32_t *k_list,
                                                                   int32_t *cost, int32_t *q_order, int4 *k_raw,
                                                                   int4 *k_items, int4 *k_split, int32_t *k_counts) {
  __shared__ int32_t bins[kOrderBins];
  __shared__ int32_t wave_sum[kOrderThreads / 64];
  __shared__ int64_t red[kOrderThreads / 64];
  __shared__ int32_t sh_items, sh_parts, sh_cut;
  const int tid = threadIdx.x;
  for (int pass = 0; pass < 2; ++pass) {
    const int32_t n = pass == 0 ? n_rows : n_cols;
    int32_t *c = cost + (pass == 0 ? 0 : n_rows);
    for (int i = tid; i < kOrderBins; i += kOrderThreads) bins[i] = 0;
    __syncthreads();
    // 8 lanes per item, each summing every 8th entry of its tile list
    const int sub = tid & 7;
    int64_t mine = 0;
    for (int32_t it = tid >> 3; it < n; it += kOrderThreads / 8) {
      int32_t k = 0;
      if (pass == 0) {  // row it: key halves are sub-block columns {0,1} and {2,3}
        const int32_t cnt = q_nnz[it];
        const int32_t *lst = q_list + (int64_t)it * NT;
        const uint32_t *subs = sub_class + (int64_t)it * NT;
        for (int32_t t = sub; t < cnt; t += 8) {
          const uint32_t w = subs[lst[t]];
          k += ((w & 0x0F0F0F0Fu) != 0) + ((w & 0xF0F0F0F0u) != 0);
        }
      } else {          // column it: query halves are sub-block rows {0,1} and {2,3}
        const int32_t b = it / NT, col = it - b * NT;
        const int32_t cnt = k_nnz[it];
        const int32_t *lst = k_list + (int64_t)it * MT;
        for (int32_t t = sub; t < cnt; t += 8) {
          const uint32_t w = sub_class[((int64_t)b * MT + lst[t]) * NT + col];
          k += ((w & 0x0000FFFFu) != 0) + ((w & 0xFFFF0000u) != 0);
        }
      }
      k += __shfl_xor(k, 1);
      k += __shfl_xor(k, 2);
      k += __shfl_xor(k, 4);
      if (sub == 0) {
        c[it] = k;
        mine += k;
        if (pass == 0) atomicAdd(&bins[kOrderBins - 1 - min(k, kOrderBins - 1)], 1);  // bin 0: largest
      }
    }
    if (pass == 0) {
      __syncthreads();
      scan_bins(bins, wave_sum);
      for (int32_t it = tid; it < n; it += kOrderThreads)
        q_order[atomicAdd(&bins[kOrderBins - 1 - min(c[it], kOrderBins - 1)], 1)] = it;
      __syncthreads();
      continue;
    }
    // columns: the cap, doubled until the extra parts fit (they do at once:
    // each cut column adds fewer than c / cap parts)
    const int64_t total = block_sum_i64(mine, red);
    int64_t cap64 = (total * Hkv + kSplitSlots - 1) / kSplitSlots;
    if (cap64 < kMinSplit) cap64 = kMinSplit;
    for (;;) {
      const int32_t cap = (int32_t)min(cap64, (int64_t)INT32_MAX);
      int64_t extra = 0;
      for (int32_t it = tid; it < n; it += kOrderThreads) extra += parts_of(c[it], cap) - 1;
      extra = block_sum_i64(extra, red);
      if (extra * Hkv < kSplitSlots || cap64 >= INT32_MAX) break;
      cap64 *= 2;
    }
    const int32_t cap = (int32_t)min(cap64, (int64_t)INT32_MAX);
    if (tid == 0) {
      sh_items = 0;
      sh_parts = 0;
      sh_cut = 0;
    }
    __syncthreads();
    for (int32_t it = tid; it < n; it += kOrderThreads) {
      const int32_t s = parts_of(c[it], cap);
      const int32_t first = atomicAdd(&sh_items, s);
      int32_t slot = -1;
      if (s > 1) {
        slot = atomicAdd(&sh_parts, s - 1);
        k_split[atomicAdd(&sh_cut, 1)] = make_int4(it, slot, s, 0);
      }
      const int32_t ic = (c[it] + s - 1) / s;
      for (int32_t j = 0; j < s; ++j) {
        k_raw[first + j] = make_int4(it, j, s, j == 0 ? -1 : slot + j - 1);
        atomicAdd(&bins[kOrderBins - 1 - min(ic, kOrderBins - 1)], 1);
      }
    }
    __syncthreads();
    const int32_t n_items = sh_items;
    scan_bins(bins, wave_sum);
    for (int32_t i = tid; i < n_items; i += kOrderThreads) {
      const int4 e = k_raw[i];
      const int32_t ic = (c[e.x] + e.z - 1) / e.z;
      k_items[atomicAdd(&bins[kOrderBins - 1 - min(ic, kOrderBins - 1)], 1)] = e;
    }
    if (tid == 0) {
      k_counts[0] = n_items;
      k_counts[1] = sh_cut;
    }
    __syncthreads();
  }
}


template <int D>
void launch_absmax_d(int32_t B, int32_t L, const AbsmaxJob *jobs, hipStream_t s) {
  absmax_kernel<D><<<dim3((L + kAbsTokens - 1) / kAbsTokens, jobs[1].hb_end, B), 256, 0, s>>>(L, jobs[0], jobs[1]);
}

template <int D, bool ROPE, bool TILE>
void launch_pack_d(int32_t B, int32_t L, int32_t Lp, int32_t H, int32_t group, const void *x,
                   const int32_t *slot_tok, const float2 *table, const uint32_t *pmax, uint16_t *rows,
                   int32_t *etile, hipStream_t s) {
  const unsigned hgroups = (unsigned)((H + kPackHeads - 1) / kPackHeads);
  const dim3 grid(hgroups * (unsigned)(Lp / kPackSlots), 1, B);
  pack_kernel<D, ROPE, TILE><<<grid, 256, 0, s>>>(L, Lp, H, group, static_cast<const uint16_t *>(x), slot_tok, table,
                                                 pmax, rows, etile);
}

}  // namespace

// RoPE table + clearing of the plane maxima (they start at zero).
void launch_rope_table(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  const int32_t half = in.D / 2;
  const int64_t total = (int64_t)in.B * ws.Lp * half;
  const int64_t n = total > ws.n_pmax ? total : (int64_t)ws.n_pmax;
  rope_table_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(in.B, in.L, ws.Lp, half, log2(in.rope_theta),
                                                                in.layout.tok_pos, in.layout.slot_tok, ws.rope,
                                                                ws.pmax, ws.n_pmax);
}

// Plane maxima of k (times sqrt(2), the RoPE bound) and of v.
void launch_absmax_kv(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  const int HPB = 256 / (in.D / 8);
  const int32_t hb = (in.Hkv + HPB - 1) / HPB;
  AbsmaxJob jobs[2] = {{static_cast<const uint16_t *>(in.k), ws.mk, in.Hkv, hb, 1.4142136f},
                       {static_cast<const uint16_t *>(in.v), ws.mv, in.Hkv, 2 * hb, 1.0f}};
  if (in.D == 64) launch_absmax_d<64>(in.B, in.L, jobs, s);
  else launch_absmax_d<128>(in.B, in.L, jobs, s);
}

// q after RoPE, one scale per 64-slot tile of each (row, head).
void launch_pack_q(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  const int32_t group = in.Hq / in.Hkv;
  if (in.D == 64)
    launch_pack_d<64, true, true>(in.B, in.L, ws.Lp, in.Hq, group, in.q, in.layout.slot_tok, ws.rope, nullptr,
                                  ws.qr, ws.eqt, s);
  else
    launch_pack_d<128, true, true>(in.B, in.L, ws.Lp, in.Hq, group, in.q, in.layout.slot_tok, ws.rope, nullptr,
                                   ws.qr, ws.eqt, s);
  group_min_kernel<<<(unsigned)(in.B * in.Hkv), 256, 0, s>>>(in.Hq, group, ws.Lp / kTile, ws.eqt, ws.eref);
}

// k (RoPE) or v, one scale per plane.
void launch_pack_any(int D, bool rope, int32_t B, int32_t L, int32_t Lp, int32_t H, int32_t group,
                     const void *x, const int32_t *slot_tok, const float2 *table, const uint32_t *pmax,
                     uint16_t *rows, hipStream_t s) {
  if (D == 64) {
    if (rope) launch_pack_d<64, true, false>(B, L, Lp, H, group, x, slot_tok, table, pmax, rows, nullptr, s);
    else launch_pack_d<64, false, false>(B, L, Lp, H, group, x, slot_tok, table, pmax, rows, nullptr, s);
  } else {
    if (rope) launch_pack_d<128, true, false>(B, L, Lp, H, group, x, slot_tok, table, pmax, rows, nullptr, s);
    else launch_pack_d<128, false, false>(B, L, Lp, H, group, x, slot_tok, table, pmax, rows, nullptr, s);
  }
}

void launch_work_order(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  const int32_t MT = ws.Lp / OPR_ATTN_BLOCK, NT = MT;
  work_order_kernel<<<1, kOrderThreads, 0, s>>>(in.B * MT, in.B * NT, MT, NT, in.Hkv, in.layout.sub_class,
                                               in.layout.q_nnz, in.layout.q_list, in.layout.k_nnz, in.layout.k_list,
                                               ws.order_cost, ws.q_order, ws.k_raw, ws.k_items, ws.k_split,
                                               ws.k_counts);
}

// delta and the fp16 dout copy with its tile exponents and their group minima.
void launch_delta_pack(const opr_attn_in &in, const void *o, const void *dout, const AttnWs &ws,
                       hipStream_t s) {
  const int32_t group = in.Hq / in.Hkv;
  const unsigned hgroups = (unsigned)((in.Hq + kPackHeads - 1) / kPackHeads);
  const dim3 grid(hgroups * (unsigned)(ws.Lp / kPackSlots), 1, in.B);
  const uint16_t *o16 = static_cast<const uint16_t *>(o);
  const uint16_t *d16 = static_cast<const uint16_t *>(dout);
  if (in.D == 64)
    delta_pack_kernel<64><<<grid, 256, 0, s>>>(in.L, ws.Lp, in.Hq, group, o16, d16, in.layout.slot_tok, ws.dor,
                                               ws.dsc, ws.edot);
  else
    delta_pack_kernel<128><<<grid, 256, 0, s>>>(in.L, ws.Lp, in.Hq, group, o16, d16, in.layout.slot_tok, ws.dor,
                                                ws.dsc, ws.edot);
  group_min_kernel<<<(unsigned)(in.B * in.Hkv), 256, 0, s>>>(in.Hq, group, ws.Lp / kTile, ws.edot, ws.eref + 1);
}

void launch_scale_delta(const opr_attn_in &in, const float *lse, const AttnWs &ws, hipStream_t s) {
  const int64_t total = (int64_t)in.B * in.Hq * ws.Lp;
  scale_delta_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(in.B, in.L, ws.Lp, in.Hq, in.Hq / in.Hkv, lse,
                                                                     in.layout.slot_tok, ws.eqt, ws.edot, ws.eref,
                                                                     ws.mv, ws.dsc, ws.lse2);
}

}  // namespace opr

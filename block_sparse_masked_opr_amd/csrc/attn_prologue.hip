// Prologue kernels of the attention path.  Everything here is indexed by
// slot (attention order): slot s < L holds token slot_tok[s] of the layout,
// slots L .. Lp-1 are empty and padded with zeros.  Two launches:
//  - rope_order_kernel: the longest-first work order of the attention kernels
//    (one workgroup), the partial maxima of every (row, kv head) plane of k
//    and v over 256-token blocks, and the RoPE table at the slots' strategic
//    position ids; all three need only the inputs and the layout,
//  - pack_kv_kernel: each workgroup reduces its planes' partial maxima, then
//    writes head-major fp16 copies of k (after RoPE) and v in slot order with
//    one power-of-two scale per plane.
// pack_kernel makes the same copy of q, one scale per row (token and head),
// for a backward that does not reuse the forward's state (the forward kernel
// converts q itself).
// (The backward's dout copy and delta = rowsum(dout * o) are formed by the
// dQ kernel, attn_dq.hip.)
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
// and s >= L use position 0.  Element gid < n_zero also clears zero_words[gid]
// (the plane maxima start at 0).
struct RopeArgs {
  int32_t B, L, Lp, half;
  double log2_theta;
  const int32_t *tok_pos, *slot_tok;
  float2 *table;
  uint32_t *zero_words;
  int32_t n_zero;
};

// 2 pi in two parts (the double nearest to it and the remainder) and 1 / (2 pi)
constexpr double k2PiHi = 6.283185307179586232, k2PiLo = 2.4492935982947064e-16;
constexpr double kInv2Pi = 0.15915494309189533577;

// One workgroup's entries (gid0 + threadIdx.x); the inverse frequencies of the
// D/2 <= 64 rotation pairs are formed once per workgroup.  The angle
// x = pos * inv_freq is reduced by the nearest multiple of 2 pi (two-part
// constant, each step one rounding) before sin and cos, so the library
// routines see |r| <= pi; the reduction adds about 1e-16 rad to x's own
// rounding.
__device__ __forceinline__ void rope_entries(const RopeArgs &a, int64_t gid0) {
  __shared__ double inv_freq[64];
  if ((int)threadIdx.x < a.half) inv_freq[threadIdx.x] = exp2(-(2.0 * threadIdx.x / (2.0 * a.half)) * a.log2_theta);
  __syncthreads();
  const int64_t gid = gid0 + threadIdx.x;
  if (gid < a.n_zero) a.zero_words[gid] = 0u;
  const int64_t total = (int64_t)a.B * a.Lp * a.half;
  if (gid >= total) return;
  const int32_t j = (int32_t)(gid % a.half);
  const int64_t bt = gid / a.half;
  const int32_t t = (int32_t)(bt % a.Lp);
  const int32_t b = (int32_t)(bt / a.Lp);
  const int32_t pos = t < a.L ? a.tok_pos[(int64_t)b * a.L + a.slot_tok[(int64_t)b * a.L + t]] : 0;
  const double x = (double)pos * inv_freq[j];
  const double nq = rint(x * kInv2Pi);
  const double r = fma(-nq, k2PiLo, fma(-nq, k2PiHi, x));
  double sn, cs;
  sincos(r, &sn, &cs);
  a.table[gid] = make_float2((float)cs, (float)sn);
}

// Largest |x| of each (row, head) plane of k and v [B][L][H][D] bf16 (k
// times sqrt(2), RoPE's bound on a pair, rounded up), as partial maxima over
// kAbsSlots-token blocks: part[job][b][h][x] (float bits; job 0 = k, 1 = v).
// No atomics into shared words, so nothing has to be cleared first and the
// workgroups run in the same launch as the work order and the RoPE table.  A
// workgroup of NT threads covers one token block of up to HPB heads: thread
// (token row r, head hl, chunk j) reads 16-byte chunk j of head hl of every
// tpr-th token from r, so each D/8-lane group reads one head's whole row and a
// wave reads contiguous runs; with fewer heads than HPB the spare threads take
// further token rows.
struct AbsArgs {
  const uint16_t *k, *v;    // [B][L][H][D] bf16
  uint32_t *part;           // [2][B][H][nx]
  int32_t B, L, H, nx, hb;  // nx token blocks, hb head blocks per (job, row)
};

template <int D, int NT>
__device__ void plane_max_part(const AbsArgs &a, int64_t blk) {
  constexpr int CPH = D / 8, HPB = NT / CPH;
  const int xb = (int)(blk % a.nx);
  int64_t rest = blk / a.nx;
  const int hb = (int)(rest % a.hb);
  rest /= a.hb;
  const int b = (int)(rest % a.B);
  const int job = (int)(rest / a.B);
  const uint16_t *x = job == 0 ? a.k : a.v;
  const float factor = job == 0 ? 1.4142136f : 1.0f;
  const int H = a.H, L = a.L, tid = threadIdx.x;
  // the block's heads [hb * HPB, hb * HPB + nh); threads beyond one token row
  // of them take further tokens (tpr token rows per pass)
  const int nh = min(HPB, H - hb * HPB);
  const int row = nh * CPH, tpr = NT / row;
  const int r = tid / row, hl = (tid % row) / CPH, j = tid % CPH;
  const int h = hb * HPB + hl;
  const int t0 = xb * kAbsSlots;
  uint32_t m = 0u;  // float bits of the largest |x| (non-negative: integer order)
  if (r < tpr) {
    const uint16_t *src = x + (((int64_t)b * L + t0) * H + h) * D + j * 8;
    const int nt = min(kAbsSlots, L - t0);
#pragma unroll 8
    for (int t = r; t < nt; t += tpr)
      m = max(m, absmax8_bf16_bits(*reinterpret_cast<const uint4 *>(src + (int64_t)t * H * D)));
  }
#pragma unroll
  for (int off = CPH / 2; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  // the token rows meet in LDS
  __shared__ uint32_t hm[HPB];
  if (tid < HPB) hm[tid] = 0u;
  __syncthreads();
  if (j == 0 && r < tpr && m > 0u) atomicMax(&hm[hl], m);
  __syncthreads();
  if (tid < nh)
    a.part[(((int64_t)job * a.B + b) * H + hb * HPB + tid) * a.nx + xb] =
        __float_as_uint(__uint_as_float(hm[tid]) * factor);
}

// One workgroup per (64-slot block, group of kPackHeads heads, row): 4
// threads per slot, each owning D/8 rotation pairs (j, j + D/2), so that a
// wave covers exactly one kTile-slot tile.  The threads keep the slot's RoPE
// cosines and sines in registers and walk the heads.
// x: [B][L][H][D] bf16 -> rows [B][H][Lp][D] in slot order, fp16(x' * 2^e),
// x' = RoPE(x) or x.
// ROWS = false: e is the exponent of the head's plane maximum hmax[h - h0]
// (the caller reduces it for the block's heads).
// ROWS = true: e is the exponent of the row's own largest |x'| (kExpMax for
// an all-zero row), reduced over the slot's 4 threads and stored in
// erow[b][h][s]; the smallest over the wave's kTile rows goes to
// etile[b][h][tile].
// Slots s >= L are zero.
constexpr int kPackHeads = 8;
constexpr int kPackSlots = 64;

template <int D, bool ROPE, bool ROWS>
__device__ __forceinline__ void pack_rows(unsigned bx, int b, int32_t L, int32_t Lp, int32_t H, const uint16_t *x,
                                          const int32_t *slot_tok, const float2 *table, const uint32_t *hmax,
                                          uint16_t *rows, int32_t *erow, int32_t *etile) {
  constexpr int HALF = D / 2;
  constexpr int PER = HALF / 4;  // pairs per thread (4 threads per slot)
  static_assert(kPackSlots == 4 * kTile, "a wave covers one tile");
  const int hgroups = (H + kPackHeads - 1) / kPackHeads;
  const int h0 = (int)(bx % (unsigned)hgroups) * kPackHeads;
  const int blk = (int)(bx / (unsigned)hgroups);
  const int t0 = blk * kPackSlots;
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
          rope_pair(x1, x2, cs[e], lo[e], hi[e]);
        }
      }
    }
    int ex;
    if (ROWS) {
      uint32_t m = 0u;  // float bits of the largest magnitude (integer order)
#pragma unroll
      for (int e = 0; e < PER; ++e) m = max(m, max(__float_as_uint(fabsf(lo[e])), __float_as_uint(fabsf(hi[e]))));
      m = max(m, (uint32_t)__shfl_xor((int)m, 1));  // the slot's 4 threads
      m = max(m, (uint32_t)__shfl_xor((int)m, 2));
      ex = m > 0u ? plane_exponent(m) : kExpMax;
      if (part == 0) erow[((int64_t)b * H + h) * Lp + t] = ex;
      int mn = ex;
#pragma unroll
      for (int off = 4; off < 64; off <<= 1) mn = min(mn, __shfl_xor(mn, off));
      if (lane == 0) etile[((int64_t)b * H + h) * (Lp / kTile) + t0 / kTile + wave] = mn;
    } else {
      ex = plane_exponent(hmax[h - h0]);
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

template <int D, bool ROPE, bool ROWS>
__global__ __launch_bounds__(256) void pack_kernel(int32_t L, int32_t Lp, int32_t H, const uint16_t *x,
                                                   const int32_t *slot_tok, const float2 *table, uint16_t *rows,
                                                   int32_t *erow, int32_t *etile) {
  pack_rows<D, ROPE, ROWS>(blockIdx.x, blockIdx.z, L, Lp, H, x, slot_tok, table, nullptr, rows, erow, etile);
}

// k (after RoPE; blockIdx.y = 0) and v (blockIdx.y = 1) in one launch, one
// scale per plane.  Each workgroup first reduces its heads' partial maxima;
// the first slot block of each (row, head group) also writes the plane maxima
// that the attention kernels read (mk, mv).
template <int D>
__global__ __launch_bounds__(256) void pack_kv_kernel(int32_t L, int32_t Lp, int32_t H, const uint16_t *k,
                                                      const uint16_t *v, const int32_t *slot_tok,
                                                      const float2 *table, const uint32_t *part, int32_t nx,
                                                      uint32_t *mk, uint32_t *mv, uint16_t *kr, uint16_t *vr) {
  const int job = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int hgroups = (H + kPackHeads - 1) / kPackHeads;
  const int h0 = (int)(blockIdx.x % (unsigned)hgroups) * kPackHeads;
  const int nh = min(kPackHeads, H - h0);
  __shared__ uint32_t hmax[kPackHeads];
  if (tid < kPackHeads) hmax[tid] = 0u;
  __syncthreads();
  const uint32_t *pp = part + (((int64_t)job * gridDim.z + b) * H + h0) * nx;
  for (int i = tid; i < nh * nx; i += 256) atomicMax(&hmax[i / nx], pp[i]);
  __syncthreads();
  if (blockIdx.x < (unsigned)hgroups && tid < nh) (job == 0 ? mk : mv)[(int64_t)b * H + h0 + tid] = hmax[tid];
  if (job == 0)
    pack_rows<D, true, false>(blockIdx.x, b, L, Lp, H, k, slot_tok, table, hmax, kr, nullptr, nullptr);
  else
    pack_rows<D, false, false>(blockIdx.x, b, L, Lp, H, v, slot_tok, table, hmax, vr, nullptr, nullptr);
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

struct OrderArgs {
  int32_t n_rows, n_cols, MT, NT, Hkv;
  const uint32_t *sub_class;
  const int32_t *q_nnz, *q_list, *k_nnz, *k_list;
  int32_t *cost, *q_order;
  int4 *k_raw, *k_items, *k_split;
  int32_t *k_counts;
  uint32_t *dbg;  // checked builds: the error word (attn_common.h)
};

__device__ void work_order(const OrderArgs &a) {
  const int32_t n_rows = a.n_rows, n_cols = a.n_cols, MT = a.MT, NT = a.NT, Hkv = a.Hkv;
  const uint32_t *sub_class = a.sub_class;
  const int32_t *q_nnz = a.q_nnz, *q_list = a.q_list, *k_nnz = a.k_nnz, *k_list = a.k_list;
  int32_t *cost = a.cost, *q_order = a.q_order, *k_counts = a.k_counts;
  int4 *k_raw = a.k_raw, *k_items = a.k_items, *k_split = a.k_split;
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
          const int32_t n = lst[t];
          const uint32_t w = OPR_DCHECK(a.dbg, (unsigned)n < (unsigned)NT, kDbgQList) ? subs[n] : 0u;
          k += ((w & 0x0F0F0F0Fu) != 0) + ((w & 0xF0F0F0F0u) != 0);
        }
      } else {          // column it: query halves are sub-block rows {0,1} and {2,3}
        const int32_t b = it / NT, col = it - b * NT;
        const int32_t cnt = k_nnz[it];
        const int32_t *lst = k_list + (int64_t)it * MT;
        for (int32_t t = sub; t < cnt; t += 8) {
          const int32_t m = lst[t];
          const uint32_t w =
              OPR_DCHECK(a.dbg, (unsigned)m < (unsigned)MT, kDbgKList) ? sub_class[((int64_t)b * MT + m) * NT + col] : 0u;
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


// The work order (workgroup 0), the k/v partial maxima (the next n_abs
// workgroups) and the RoPE table (the rest): all three depend on the inputs
// alone, so one launch runs them side by side, the single-workgroup order
// first so that it starts at once.
template <int D>
__global__ __launch_bounds__(kOrderThreads) void rope_order_kernel(RopeArgs ra, OrderArgs oa, AbsArgs aa,
                                                                   int32_t n_abs) {
  if (blockIdx.x == 0) {
    work_order(oa);
    return;
  }
  if ((int32_t)blockIdx.x <= n_abs) {
    plane_max_part<D, kOrderThreads>(aa, (int64_t)blockIdx.x - 1);
    return;
  }
  rope_entries(ra, (int64_t)(blockIdx.x - 1 - n_abs) * kOrderThreads);
}

template <int D, bool ROPE, bool ROWS>
void launch_pack_d(int32_t B, int32_t L, int32_t Lp, int32_t H, const void *x, const int32_t *slot_tok,
                   const float2 *table, uint16_t *rows, int32_t *erow, int32_t *etile, hipStream_t s) {
  const unsigned hgroups = (unsigned)((H + kPackHeads - 1) / kPackHeads);
  const dim3 grid(hgroups * (unsigned)(Lp / kPackSlots), 1, B);
  pack_kernel<D, ROPE, ROWS><<<grid, 256, 0, s>>>(L, Lp, H, static_cast<const uint16_t *>(x), slot_tok, table, rows,
                                                 erow, etile);
}

template <int D>
void launch_pack_kv_d(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  const unsigned hgroups = (unsigned)((in.Hkv + kPackHeads - 1) / kPackHeads);
  const dim3 grid(hgroups * (unsigned)(ws.Lp / kPackSlots), 2, in.B);
  pack_kv_kernel<D><<<grid, 256, 0, s>>>(in.L, ws.Lp, in.Hkv, static_cast<const uint16_t *>(in.k),
                                        static_cast<const uint16_t *>(in.v), in.layout.slot_tok, ws.rope,
                                        ws.pmax_part, ws.n_part, ws.mk, ws.mv, ws.kr, ws.vr);
}

template <int D>
void launch_rope_order_d(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  const int32_t half = in.D / 2;
  const int64_t n = (int64_t)in.B * ws.Lp * half;
  const RopeArgs ra = {in.B, in.L, ws.Lp, half, log2(in.rope_theta), in.layout.tok_pos, in.layout.slot_tok,
                       ws.rope, nullptr, 0};
  const int32_t MT = ws.Lp / OPR_ATTN_BLOCK, NT = MT;
  const OrderArgs oa = {in.B * MT, in.B * NT, MT, NT, in.Hkv, in.layout.sub_class, in.layout.q_nnz,
                        in.layout.q_list, in.layout.k_nnz, in.layout.k_list, ws.order_cost, ws.q_order,
                        ws.k_raw, ws.k_items, ws.k_split, ws.k_counts, debug_word()};
  constexpr int HPB = kOrderThreads / (D / 8);
  const int32_t hb = (in.Hkv + HPB - 1) / HPB;
  const AbsArgs aa = {static_cast<const uint16_t *>(in.k), static_cast<const uint16_t *>(in.v), ws.pmax_part,
                      in.B, in.L, in.Hkv, ws.n_part, hb};
  const int32_t n_abs = 2 * in.B * hb * ws.n_part;
  const unsigned grid = (unsigned)(1 + n_abs + (n + kOrderThreads - 1) / kOrderThreads);
  rope_order_kernel<D><<<grid, kOrderThreads, 0, s>>>(ra, oa, aa, n_abs);
}

}  // namespace

// The work order, the k/v partial maxima and the RoPE table, in one launch.
void launch_rope_order(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  if (in.D == 64) launch_rope_order_d<64>(in, ws, s);
  else launch_rope_order_d<128>(in, ws, s);
}

// q after RoPE, one scale per row of each (row, head).
void launch_pack_q(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  if (in.D == 64)
    launch_pack_d<64, true, true>(in.B, in.L, ws.Lp, in.Hq, in.q, in.layout.slot_tok, ws.rope, ws.qr, ws.eqq,
                                  ws.eqt, s);
  else
    launch_pack_d<128, true, true>(in.B, in.L, ws.Lp, in.Hq, in.q, in.layout.slot_tok, ws.rope, ws.qr, ws.eqq,
                                   ws.eqt, s);
}

// k (after RoPE) and v, one scale per plane.
void launch_pack_kv(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  if (in.D == 64) launch_pack_kv_d<64>(in, ws, s);
  else launch_pack_kv_d<128>(in, ws, s);
}

}  // namespace opr

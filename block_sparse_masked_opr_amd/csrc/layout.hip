// Layout kernels: token placement, strategic position ids and the tile
// schedule of the block-sparse mask (One-Pass to Reason; wiki summary of the
// paper, sections "Token 复制", "分块稀疏注意力掩码", "位置 ID 策略" and
// "实现细节": the mask is generated on the device, vectorised).
//
// Pipeline, all on one stream:
//   layout_prep      one workgroup: prefix sums over rows, conversations and
//                    turns (token starts, position starts, history counts)
//   layout_fill      one thread per token: binary search for its turn, then
//                    conversation, turn, type, position id, attention-order
//                    slot and the two runs of slots of its query and key
//   layout_classify  one workgroup per tile, one thread per query row: counts
//                    the allowed keys of each 32-key sub-block with interval
//                    arithmetic, then sums per 32x32 sub-block and per tile
//                    (layout_classify_attention: the same classes over
//                    attention order, one workgroup per q-tile row, from
//                    per-query-row masks of the 32-key blocks its two runs
//                    of slots touch and cover, reduced with OR and AND)
//   layout_compact   one wave per tile row; per 16 tile columns one
//                    workgroup that reads the classes row-wise and compacts
//                    the columns from LDS (one launch): ballot compaction of
//                    the non-empty tiles into ascending lists
//
// Visibility of a query q in turn i of a conversation, as key intervals of
// the packed row (segments of a turn are stored h, t, r_in, r_out):
//   history  H_<i : the h and r_in tokens in [conv_start, turn_start)
//   type h   : [turn_start, q]
//   type t   : [turn_start, q]                   (h_i, then t_i causally)
//   type r_in: [turn_start, turn_start + h) and [r_in_start, q]
//   type r_out:[turn_start, r_in_start)          (h_i and t_i)
//              and [r_out_start, q]
// The history part is counted with a prefix count of h/r_in tokens.
#include "opr_internal.h"

namespace opr {
namespace {

constexpr int kPrepThreads = 1024;

// Exclusive prefix sum of n values (produced by get(i)) into out[0..n], using
// the whole workgroup; out[n] is the total.  Per chunk of kPrepThreads
// values: an inclusive scan inside each wave (shuffles), the wave totals
// scanned by wave 0 through LDS (sh: kPrepThreads / 64 + 1 words), two
// barriers per chunk.
template <class Get>
__device__ void block_exclusive_scan(int n, Get get, int32_t *out, int32_t *sh) {
  constexpr int kWaves = kPrepThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t carry = 0;
  for (int base = 0; base < n; base += kPrepThreads) {
    const int i = base + tid;
    const int32_t v = (i < n) ? get(i) : 0;
    int32_t incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    if (lane == 63) sh[wv] = incl;
    __syncthreads();
    if (wv == 0) {
      int32_t t = lane < kWaves ? sh[lane] : 0;
#pragma unroll
      for (int d = 1; d < kWaves; d <<= 1) {
        const int32_t y = __shfl_up(t, d);
        if (lane >= d) t += y;
      }
      if (lane < kWaves) sh[lane] = t;  // inclusive totals of waves 0 .. lane
    }
    __syncthreads();
    const int32_t before = (wv > 0 ? sh[wv - 1] : 0) + incl - v;
    if (i < n) out[i] = carry + before;
    carry += sh[kWaves - 1];
    __syncthreads();  // sh is rewritten by the next chunk
  }
  if (tid == 0) out[n] = carry;
  __syncthreads();
}

// Two exclusive prefix sums in one pass (get(i) gives both values), as
// block_exclusive_scan; sh holds 2 * (kPrepThreads / 64) words.
template <class Get>
__device__ void block_exclusive_scan2(int n, Get get, int32_t *out0, int32_t *out1, int32_t *sh) {
  constexpr int kWaves = kPrepThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t carry0 = 0, carry1 = 0;
  for (int base = 0; base < n; base += kPrepThreads) {
    const int i = base + tid;
    const int2 v = (i < n) ? get(i) : make_int2(0, 0);
    int32_t inc0 = v.x, inc1 = v.y;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t y0 = __shfl_up(inc0, d), y1 = __shfl_up(inc1, d);
      if (lane >= d) {
        inc0 += y0;
        inc1 += y1;
      }
    }
    if (lane == 63) {
      sh[wv] = inc0;
      sh[kWaves + wv] = inc1;
    }
    __syncthreads();
    if (wv == 0) {
      int32_t t0 = lane < kWaves ? sh[lane] : 0, t1 = lane < kWaves ? sh[kWaves + lane] : 0;
#pragma unroll
      for (int d = 1; d < kWaves; d <<= 1) {
        const int32_t y0 = __shfl_up(t0, d), y1 = __shfl_up(t1, d);
        if (lane >= d) {
          t0 += y0;
          t1 += y1;
        }
      }
      if (lane < kWaves) {
        sh[lane] = t0;
        sh[kWaves + lane] = t1;
      }
    }
    __syncthreads();
    if (i < n) {
      out0[i] = carry0 + (wv > 0 ? sh[wv - 1] : 0) + inc0 - v.x;
      out1[i] = carry1 + (wv > 0 ? sh[kWaves + wv - 1] : 0) + inc1 - v.y;
    }
    carry0 += sh[kWaves - 1];
    carry1 += sh[2 * kWaves - 1];
    __syncthreads();  // sh is rewritten by the next chunk
  }
  if (tid == 0) {
    out0[n] = carry0;
    out1[n] = carry1;
  }
  __syncthreads();
}

// Index of the last entry of the non-decreasing a[lo..hi) that is <= x
// (a[lo] <= x is guaranteed by the callers).
__device__ inline int last_le(const int32_t *a, int lo, int hi, int32_t x) {
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// The three host lists (n0, n1, n2 words), read in place from host memory
// mapped for the device, into the workspace.  A read crosses the host link, so
// the words of all three lists are read as one flat range: each thread has
// kStageIn loads in flight before it stores, and one round trip covers
// kPrepThreads * kStageIn words (every list of a 64-row batch of 32768-token
// rows fits one).
constexpr int kStageIn = 16;
__device__ void stage_in3(const int32_t *s0, int32_t *d0, int n0, const int32_t *s1, int32_t *d1, int n1,
                          const int32_t *s2, int32_t *d2, int n2) {
  const int n = n0 + n1 + n2;
  for (int base = 0; base < n; base += kPrepThreads * kStageIn) {
    int32_t v[kStageIn];
#pragma unroll
    for (int u = 0; u < kStageIn; ++u) {  // unconditional loads (index clamped): no branch between them
      const int i = min(base + u * kPrepThreads + (int)threadIdx.x, n - 1);
      v[u] = i < n0 ? s0[i] : i < n0 + n1 ? s1[i - n0] : s2[i - n0 - n1];
    }
#pragma unroll
    for (int u = 0; u < kStageIn; ++u) {
      const int i = base + u * kPrepThreads + (int)threadIdx.x;
      if (i < n0) d0[i] = v[u];
      else if (i < n0 + n1) d1[i - n0] = v[u];
      else if (i < n) d2[i - n0 - n1] = v[u];
    }
  }
}

__global__ __launch_bounds__(kPrepThreads) void layout_prep(int32_t B, int32_t C, int32_t T,
                                                            LayoutWs ws) {
  __shared__ int32_t sh[kPrepThreads];
  if (ws.src_cpr) {
    // the host arrays, read in place (4-byte words: any opr_turn alignment)
    stage_in3(ws.src_cpr, ws.cpr, B, ws.src_tpc, ws.tpc, C, ws.src_turns, reinterpret_cast<int32_t *>(ws.turns), 4 * T);
    __syncthreads();  // the block's own copies are visible to all its threads
  }
  const int32_t *cpr = ws.cpr;
  const int32_t *tpc = ws.tpc;
  const int4 *turns = ws.turns;
  block_exclusive_scan(B, [&](int i) { return cpr[i]; }, ws.row_conv0, sh);
  block_exclusive_scan(C, [&](int i) { return tpc[i]; }, ws.conv_turn0, sh);
  // tokens of a turn: h + t + r_in + r_out; the next human message starts
  // after h_i and r_in_i: the position advance per turn is h + r_in, which is
  // also the number of history tokens
  block_exclusive_scan2(T, [&](int i) { const int4 u = turns[i]; return make_int2(u.x + u.y + u.z + u.w, u.x + u.z); },
                        ws.tok_g, ws.pos_g, sh);
  // the row of each conversation and the conversation of each turn, scattered
  // from the prefix sums (the scans end with a barrier)
  for (int b = threadIdx.x; b < B; b += kPrepThreads)
    for (int c = ws.row_conv0[b], ce = ws.row_conv0[b + 1]; c < ce; ++c) ws.conv_row[c] = b;
  for (int c = threadIdx.x; c < C; c += kPrepThreads)
    for (int t = ws.conv_turn0[c], te = ws.conv_turn0[c + 1]; t < te; ++t) ws.turn_conv[t] = c;
  for (int b = threadIdx.x; b <= B; b += kPrepThreads) ws.row_turn0[b] = ws.conv_turn0[ws.row_conv0[b]];
}

// Two runs [x0, x1) and [x2, x3) in the canonical form of the layout: the
// runs are disjoint and ascending (x1 <= x2); an empty first run is dropped,
// touching runs are merged and a missing run is written [x, x) with x the end
// of the run before it (0 if none).
__device__ inline int4 two_runs(int32_t x0, int32_t x1, int32_t x2, int32_t x3) {
  if (x0 >= x1) { x0 = x2; x1 = x3; x2 = x3; }  // first run empty
  if (x0 >= x1) return make_int4(0, 0, 0, 0);
  if (x2 >= x3) return make_int4(x0, x1, x1, x1);
  if (x1 == x2) return make_int4(x0, x3, x3, x3);
  return make_int4(x0, x1, x2, x3);
}

// Per-token fields of token x (row-local index) in row b, its attention-order
// slot and the mask of that slot as runs of slots.
//
// Attention order of a conversation at [a, e): the h and r_in tokens first -
// their position ids run 0 .. N1-1 without gaps, so a token of them sits at
// slot a + pos - then the t and r_out tokens, turn by turn: turn i's t_i and
// r_out_i occupy [p2(i), p2(i+1)) with p2(i) = a + N1 + (t and r_out tokens of
// the turns before i).  In slot order the rules become:
//   query h_i / r_in_i : keys [a, s]
//   query t_i / r_out_i: keys [a, a + s_t(i)) (H_<i and h_i) and [p2(i), s]
//   key h_j    : queries [s, a + N1) and [p2(j), e)      (later turns' t, r_out)
//   key r_in_j : queries [s, a + N1) and [p2(j+1), e)
//   key t_j / r_out_j: queries [s, p2(j+1))
__global__ __launch_bounds__(256) void layout_fill(int32_t B, int32_t L, LayoutWs ws,
                                                   opr_layout out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)B * L) return;
  const int32_t b = (int32_t)(gid / L);
  const int32_t x = (int32_t)(gid - (int64_t)b * L);
  const int32_t t0 = ws.row_turn0[b], t1 = ws.row_turn0[b + 1];
  const int32_t r0 = ws.tok_g[t0];
  int32_t conv = -1, turn = -1, pos = 0, gt = -1, slot = x;
  int4 qiv = make_int4(0, 0, 0, 0), kiv = make_int4(0, 0, 0, 0);
  uint8_t type = OPR_TOK_PAD;
  if (x < ws.tok_g[t1] - r0) {
    gt = last_le(ws.tok_g, t0, t1, r0 + x);
    const int32_t c = ws.turn_conv[gt];
    const int32_t c0 = ws.conv_turn0[c], c1 = ws.conv_turn0[c + 1];
    conv = c - ws.row_conv0[b];
    turn = gt - c0;
    const int4 u = ws.turns[gt];
    const int32_t o = r0 + x - ws.tok_g[gt];              // offset inside the turn
    const int32_t s_h = ws.pos_g[gt] - ws.pos_g[c0];      // first position of h_i
    if (o < u.x) {                                        // h_i
      type = OPR_TOK_H; pos = s_h + o;
    } else if (o < u.x + u.y) {                           // t_i: starts after h_i
      type = OPR_TOK_T; pos = s_h + o;
    } else if (o < u.x + u.y + u.z) {                     // r_in_i: starts after h_i
      type = OPR_TOK_RIN; pos = s_h + u.x + (o - u.x - u.y);
    } else {                                              // r_out_i: starts after t_i
      type = OPR_TOK_ROUT; pos = s_h + u.x + u.y + (o - u.x - u.y - u.z);
    }
    // attention order
    const int32_t a = ws.tok_g[c0] - r0, e = ws.tok_g[c1] - r0;
    const int32_t n1 = ws.pos_g[c1] - ws.pos_g[c0];                       // h and r_in tokens
    const int32_t p2 = a + n1 + (ws.tok_g[gt] - ws.tok_g[c0]) - (ws.pos_g[gt] - ws.pos_g[c0]);
    const int32_t p2n = p2 + u.y + u.w;                                   // p2(i+1)
    if (type == OPR_TOK_H || type == OPR_TOK_RIN) {
      slot = a + pos;
      qiv = two_runs(a, slot + 1, slot + 1, slot + 1);
      kiv = two_runs(slot, a + n1, type == OPR_TOK_H ? p2 : p2n, e);
    } else {
      slot = type == OPR_TOK_T ? p2 + (o - u.x) : p2 + u.y + (o - u.x - u.y - u.z);
      qiv = two_runs(a, a + s_h + u.x, p2, slot + 1);
      kiv = two_runs(slot, p2n, p2n, p2n);
    }
  }
  out.tok_conv[gid] = conv;
  out.tok_turn[gid] = turn;
  out.tok_pos[gid] = pos;
  out.tok_type[gid] = type;
  out.tok_slot[gid] = slot;
  const int64_t sg = (int64_t)b * L + slot;
  out.slot_tok[sg] = x;
  reinterpret_cast<int4 *>(out.slot_qiv)[sg] = qiv;
  reinterpret_cast<int4 *>(out.slot_kiv)[sg] = kiv;
  ws.gturn[gid] = gt;
}

// Number of h / r_in tokens in [0, x) of row b (x may be L or past the
// conversations; then the row total).
__device__ inline int32_t history_count(const LayoutWs &ws, int32_t b, int32_t L, int32_t x) {
  const int32_t t0 = ws.row_turn0[b], t1 = ws.row_turn0[b + 1];
  const int32_t gt = (x < L) ? ws.gturn[(int64_t)b * L + x] : -1;
  if (gt < 0) return ws.pos_g[t1] - ws.pos_g[t0];
  const int4 u = ws.turns[gt];
  const int32_t o = ws.tok_g[t0] + x - ws.tok_g[gt];
  int32_t in_turn;
  if (o < u.x) in_turn = o;
  else if (o < u.x + u.y) in_turn = u.x;
  else if (o < u.x + u.y + u.z) in_turn = u.x + (o - u.x - u.y);
  else in_turn = u.x + u.z;
  return ws.pos_g[gt] - ws.pos_g[t0] + in_turn;
}

__device__ inline int32_t overlap(int32_t a0, int32_t a1, int32_t b0, int32_t b1) {
  const int32_t lo = max(a0, b0), hi = min(a1, b1);
  return hi > lo ? hi - lo : 0;
}

// One workgroup of BQ threads per tile (b, m, n); thread r is query row m*BQ + r.
template <int BQ, int BK>
__global__ __launch_bounds__(BQ) void layout_classify(int32_t B, int32_t L, int32_t MT,
                                                      int32_t NT, LayoutWs ws, opr_layout out) {
  constexpr int SQ = BQ / OPR_SUB_BLOCK, SK = BK / OPR_SUB_BLOCK;
  __shared__ int32_t cnt[SQ * SK];
  const int64_t tile = blockIdx.x;
  const int32_t n = (int32_t)(tile % NT);
  const int32_t m = (int32_t)((tile / NT) % MT);
  const int32_t b = (int32_t)(tile / ((int64_t)NT * MT));
  const int tid = threadIdx.x;
  if (tid < SQ * SK) cnt[tid] = 0;
  __syncthreads();
  const int32_t q = m * BQ + tid;
  const int32_t k_begin = n * BK;
  // keys after every query of the tile are never visible
  const bool above = k_begin > m * BQ + BQ - 1;
  const int32_t gt = (!above && q < L) ? ws.gturn[(int64_t)b * L + q] : -1;
  if (gt >= 0) {
    const int32_t t0 = ws.row_turn0[b];
    const int32_t r0 = ws.tok_g[t0];
    const int4 u = ws.turns[gt];
    const int32_t c = ws.turn_conv[gt];
    const int32_t conv_start = ws.tok_g[ws.conv_turn0[c]] - r0;
    const int32_t turn_start = ws.tok_g[gt] - r0;
    const uint8_t type = out.tok_type[(int64_t)b * L + q];
    int32_t e1, s2;  // same-turn intervals [turn_start, e1) and [s2, q]
    if (type == OPR_TOK_RIN) {
      e1 = turn_start + u.x;
      s2 = turn_start + u.x + u.y;
    } else if (type == OPR_TOK_ROUT) {
      e1 = turn_start + u.x + u.y;
      s2 = turn_start + u.x + u.y + u.z;
    } else {
      e1 = q + 1;
      s2 = q + 1;
    }
    const int32_t hist_lo = history_count(ws, b, L, conv_start);
#pragma unroll
    for (int j = 0; j < SK; ++j) {
      const int32_t a = k_begin + j * OPR_SUB_BLOCK;
      const int32_t e = min(a + OPR_SUB_BLOCK, L);
      int32_t c_ = 0;
      if (a < e) {
        // history keys in [max(a, conv_start), min(e, turn_start))
        const int32_t h0 = max(a, conv_start), h1 = min(e, turn_start);
        if (h1 > h0) {
          const int32_t lo = (h0 == conv_start) ? hist_lo : history_count(ws, b, L, h0);
          c_ += history_count(ws, b, L, h1) - lo;
        }
        c_ += overlap(a, e, turn_start, e1);
        c_ += overlap(a, e, s2, q + 1);
      }
      if (c_) atomicAdd(&cnt[(tid / OPR_SUB_BLOCK) * SK + j], c_);
    }
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t word = 0;
    int32_t total = 0;
    for (int i = 0; i < SQ * SK; ++i) {
      const int32_t v = cnt[i];
      total += v;
      const uint32_t cls = v == 0 ? OPR_TILE_EMPTY
                         : (v == OPR_SUB_BLOCK * OPR_SUB_BLOCK ? OPR_TILE_FULL : OPR_TILE_PARTIAL);
      word |= cls << (2 * i);
    }
    const uint8_t tcls = total == 0 ? OPR_TILE_EMPTY : (total == BQ * BK ? OPR_TILE_FULL : OPR_TILE_PARTIAL);
    out.tile_class[tile] = tcls;
    out.sub_class[tile] = word;
  }
}

// Tile classes over attention order: one workgroup of kClsThreads threads
// per q-tile row (b, m).  The row's queries (slots m*BQ ..) put their two
// runs of slots in LDS, and their union gives the span of key slots any of
// them sees: key tiles outside it are empty and are written as such directly.
// Inside it only a 32x32 sub-block's class is needed, not its count: a query
// row's runs touch an interval of 32-key blocks and cover a (possibly empty)
// inner interval of them, so the lane of query row r forms two 64-bit masks
// over a window of 64 key blocks (blocks its runs touch, blocks they cover),
// and 32 lanes - the 32 query rows of a sub-row - OR the first and AND the
// second with shuffles: a block is empty if no row touches it, full if every
// row covers it (a row past L covers nothing), partial otherwise.  Adjacent
// runs are merged first, so that a block across their boundary counts as
// covered.  The masks go to LDS per (sub-row, window), and one thread per tile
// then assembles its 2-bit sub-block classes and the tile's class.  The span
// is taken in chunks of kClsWin windows.
constexpr int kClsThreads = 128;
constexpr int kClsWin = 32;  // 64-block windows per chunk (2048 key blocks)

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, off);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off);
  return ((uint64_t)hi << 32) | lo;
}

// Bits of the block indices [a, b) inside the 64-block window at base.
__device__ __forceinline__ uint64_t window_bits(int32_t a, int32_t b, int32_t base) {
  const int32_t lo = max(0, min(64, a - base)), hi = max(0, min(64, b - base));
  const uint64_t below_hi = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
  const uint64_t below_lo = lo >= 64 ? ~0ull : ((1ull << lo) - 1ull);
  return below_hi & ~below_lo;
}

// Blocks of 32 keys in the window at base that the slot run [x, y) touches
// and covers.
__device__ __forceinline__ void run_blocks(int32_t x, int32_t y, int32_t base, uint64_t &touch, uint64_t &cover) {
  if (x >= y) return;
  touch |= window_bits(x >> 5, ((y - 1) >> 5) + 1, base);
  cover |= window_bits((x + 31) >> 5, y >> 5, base);
}

template <int BQ, int BK>
__global__ __launch_bounds__(kClsThreads) void layout_classify_attention(int32_t B, int32_t L, int32_t MT,
                                                                         int32_t NT, opr_layout out) {
  constexpr int SQ = BQ / OPR_SUB_BLOCK, SK = BK / OPR_SUB_BLOCK;
  static_assert(OPR_SUB_BLOCK == 32, "32-key blocks: one bit per block in a 64-block window");
  static_assert(BQ <= kClsThreads, "one thread per query slot of the tile row");
  constexpr int kTilesPerChunk = kClsWin * 64 / SK;
  __shared__ int4 runs[BQ];
  __shared__ int32_t span[2];
  __shared__ uint64_t touch_w[SQ][kClsWin], cover_w[SQ][kClsWin];
  const int64_t row = blockIdx.x;  // b * MT + m
  const int32_t m = (int32_t)(row % MT);
  const int32_t b = (int32_t)(row / MT);
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid == 0) {
    span[0] = INT32_MAX;
    span[1] = INT32_MIN;
  }
  __syncthreads();
  {
    const int32_t q = m * BQ + tid;
    int4 iv = make_int4(0, 0, 0, 0);
    if (tid < BQ && q < L) iv = reinterpret_cast<const int4 *>(out.slot_qiv)[(int64_t)b * L + q];
    // merge two runs that touch or overlap, so that a block across their
    // boundary is covered
    if (iv.x < iv.y && iv.z < iv.w && max(iv.x, iv.z) <= min(iv.y, iv.w))
      iv = make_int4(min(iv.x, iv.z), max(iv.y, iv.w), 0, 0);
    if (tid < BQ) runs[tid] = iv;
    const bool any = iv.x < iv.y || iv.z < iv.w;
    int32_t lo = any ? (iv.x < iv.y ? iv.x : iv.z) : INT32_MAX;
    int32_t hi = any ? (iv.z < iv.w ? iv.w : iv.y) : INT32_MIN;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      lo = min(lo, __shfl_xor(lo, off));
      hi = max(hi, __shfl_xor(hi, off));
    }
    if (lane == 0 && lo <= hi) {  // one atomic pair per wave
      atomicMin(&span[0], lo);
      atomicMax(&span[1], hi);
    }
  }
  __syncthreads();
  uint8_t *tcls = out.tile_class + row * NT;
  uint32_t *scls = out.sub_class + row * NT;
  const int32_t n_lo = span[0] <= span[1] ? span[0] / BK : 0;
  const int32_t n_hi = span[0] <= span[1] ? (span[1] - 1) / BK : -1;  // empty range if no key is seen
  for (int32_t n = tid; n < NT; n += kClsThreads) {
    if (n < n_lo || n > n_hi) {
      tcls[n] = OPR_TILE_EMPTY;
      scls[n] = 0u;
    }
  }
  const int grp = tid >> 5, r = tid & 31;  // 32-lane groups: one (sub-row, window) each
  for (int32_t c0 = n_lo; c0 <= n_hi; c0 += kTilesPerChunk) {
    const int32_t c1 = min(n_hi, c0 + kTilesPerChunk - 1);
    const int32_t kb0 = c0 * SK;  // first key block of the chunk
    const int32_t nwin = ((c1 - c0 + 1) * SK + 63) / 64;
    for (int it = grp; it < SQ * nwin; it += kClsThreads / 32) {
      const int sq = it / nwin, win = it - sq * nwin;
      const int4 u = runs[sq * OPR_SUB_BLOCK + r];
      const int32_t base = kb0 + 64 * win;
      uint64_t touch = 0, cover = 0;
      run_blocks(u.x, u.y, base, touch, cover);
      run_blocks(u.z, u.w, base, touch, cover);
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) {
        touch |= shfl_xor_u64(touch, off);
        cover &= shfl_xor_u64(cover, off);
      }
      if (r == 0) {
        touch_w[sq][win] = touch;
        cover_w[sq][win] = cover;
      }
    }
    __syncthreads();
    for (int32_t n = c0 + tid; n <= c1; n += kClsThreads) {
      uint32_t word = 0;
      int touched = 0, covered = 0;
#pragma unroll
      for (int i = 0; i < SQ; ++i) {
#pragma unroll
        for (int j = 0; j < SK; ++j) {
          const int32_t k = n * SK + j - kb0;
          const uint32_t t = (uint32_t)(touch_w[i][k >> 6] >> (k & 63)) & 1u;
          const uint32_t f = (uint32_t)(cover_w[i][k >> 6] >> (k & 63)) & 1u;
          word |= (t ? (f ? OPR_TILE_FULL : OPR_TILE_PARTIAL) : OPR_TILE_EMPTY) << (2 * (i * SK + j));
          touched += (int)t;
          covered += (int)f;
        }
      }
      tcls[n] = touched == 0 ? OPR_TILE_EMPTY : (covered == SQ * SK ? OPR_TILE_FULL : OPR_TILE_PARTIAL);
      scls[n] = word;
    }
    __syncthreads();  // the masks are rewritten by the next chunk
  }
}

// The lists of non-empty tiles, ballot compaction, ascending; workgroups of
// kCmpThreads.  Workgroups [0, row_groups) take q-tile rows, one wave per row
// b*MT + m (its k-tile indices; the row's classes are contiguous).  The rest
// take kCmpCols k-tile columns of one row b each (their q-tile indices): a
// column's classes lie NT bytes apart, so the block's kCmpCols contiguous
// bytes of kCmpRows q-tile rows at a time are read row-wise (one load per
// row and thread where NT allows aligned loads), stored column-major in LDS,
// and each wave compacts its kCmpCols / 4 columns there.
constexpr int kCmpThreads = 256, kCmpCols = 16, kCmpRows = 256;

__device__ __forceinline__ void compact_ballot(bool nz, int32_t x, int32_t *lst, int32_t &count, int lane) {
  const uint64_t bal = __ballot(nz);
  const int32_t before = __popcll(bal & ((1ull << lane) - 1ull));
  if (nz) lst[count + before] = x;
  count += __popcll(bal);
}

__global__ __launch_bounds__(kCmpThreads) void layout_compact(int32_t B, int32_t MT, int32_t NT, int32_t row_groups,
                                                              opr_layout out) {
  __shared__ uint8_t tcol[kCmpCols][kCmpRows + 4];  // [column][row], padded
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if ((int32_t)blockIdx.x < row_groups) {
    const int64_t idx = (int64_t)blockIdx.x * (kCmpThreads / 64) + wv;  // row b*MT + m
    if (idx >= (int64_t)B * MT) return;
    const uint8_t *cls = out.tile_class + idx * NT;
    int32_t *lst = out.q_list + idx * NT;
    int32_t count = 0;
    for (int32_t base = 0; base < NT; base += 64) {
      const int32_t x = base + lane;
      compact_ballot(x < NT && cls[x] != OPR_TILE_EMPTY, x, lst, count, lane);
    }
    for (int32_t x = count + lane; x < NT; x += 64) lst[x] = -1;
    if (lane == 0) out.q_nnz[idx] = count;
    return;
  }
  // Workgroups go to the 8 XCDs round-robin by index, and the column groups
  // of one row b share the cache lines of its classes: the groups are numbered
  // so that consecutive ones (the same b) land on one XCD.  The column part of
  // the grid is padded to a multiple of 8 workgroups, Q per XCD.
  const int32_t cgroups = (NT + kCmpCols - 1) / kCmpCols;
  const int32_t Q = (B * cgroups + 7) / 8;
  const int32_t g = (int32_t)(blockIdx.x % 8) * Q + ((int32_t)blockIdx.x - row_groups) / 8;
  if (g >= B * cgroups) return;
  const int32_t b = g / cgroups, n0 = (g % cgroups) * kCmpCols;
  const uint8_t *cls = out.tile_class + (int64_t)b * MT * NT;
  // whole aligned 16-byte row pieces: every row of the block starts on a
  // 16-byte boundary and holds all kCmpCols columns
  const bool vec = (NT % kCmpCols) == 0 && (reinterpret_cast<uintptr_t>(out.tile_class) & 15u) == 0;
  constexpr int kWaveCols = kCmpCols / (kCmpThreads / 64);
  int32_t count[kWaveCols];
#pragma unroll
  for (int c = 0; c < kWaveCols; ++c) count[c] = 0;
  for (int32_t m0 = 0; m0 < MT; m0 += kCmpRows) {
    const int32_t rows = min(kCmpRows, MT - m0);
    __syncthreads();  // the previous chunk's columns have been read
    if (vec) {
      // thread r: the block's 16 bytes of row m0 + r
      if (tid < rows) {
        const uint4 w = *reinterpret_cast<const uint4 *>(cls + (int64_t)(m0 + tid) * NT + n0);
        const uint32_t ws4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < kCmpCols; ++e) tcol[e][tid] = (uint8_t)(ws4[e >> 2] >> (8 * (e & 3)));
      }
    } else {
      // thread: byte tid % kCmpCols of rows tid / kCmpCols + k * (kCmpThreads / kCmpCols)
      for (int32_t r = tid / kCmpCols; r < rows; r += kCmpThreads / kCmpCols) {
        const int32_t n = n0 + tid % kCmpCols;
        tcol[tid % kCmpCols][r] = n < NT ? cls[(int64_t)(m0 + r) * NT + n] : (uint8_t)OPR_TILE_EMPTY;
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kWaveCols; ++c) {
      const int32_t n = n0 + wv * kWaveCols + c;
      if (n >= NT) break;
      int32_t *lst = out.k_list + ((int64_t)b * NT + n) * MT;
      for (int32_t base = 0; base < rows; base += 64) {
        const int32_t x = base + lane;
        compact_ballot(x < rows && tcol[wv * kWaveCols + c][x] != OPR_TILE_EMPTY, m0 + x, lst, count[c], lane);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < kWaveCols; ++c) {
    const int32_t n = n0 + wv * kWaveCols + c;
    if (n >= NT) break;
    int32_t *lst = out.k_list + ((int64_t)b * NT + n) * MT;
    for (int32_t x = count[c] + lane; x < MT; x += 64) lst[x] = -1;
    if (lane == 0) out.k_nnz[(int64_t)b * NT + n] = count[c];
  }
}

template <int BQ, int BK>
void launch_classify(int64_t tiles, int32_t B, int32_t L, int32_t MT, int32_t NT,
                     const LayoutWs &ws, const opr_layout &out, hipStream_t s) {
  if (out.order == OPR_ORDER_ATTENTION)
    layout_classify_attention<BQ, BK><<<dim3((unsigned)((int64_t)B * MT)), dim3(kClsThreads), 0, s>>>(B, L, MT, NT, out);
  else
    layout_classify<BQ, BK><<<dim3((unsigned)tiles), dim3(BQ), 0, s>>>(B, L, MT, NT, ws, out);
}

}  // namespace

size_t carve_layout_ws(void *p, int32_t B, int32_t L, int32_t C, int32_t T, LayoutWs *o) {
  Carver cv(p);
  LayoutWs w;
  w.cpr = cv.take<int32_t>(B);
  w.tpc = cv.take<int32_t>(C > 0 ? C : 1);
  w.turns = cv.take<int4>(T > 0 ? T : 1);
  w.row_conv0 = cv.take<int32_t>(B + 1);
  w.conv_turn0 = cv.take<int32_t>(C + 1);
  w.tok_g = cv.take<int32_t>(T + 1);
  w.pos_g = cv.take<int32_t>(T + 1);
  w.conv_row = cv.take<int32_t>(C > 0 ? C : 1);
  w.turn_conv = cv.take<int32_t>(T > 0 ? T : 1);
  w.row_turn0 = cv.take<int32_t>(B + 1);
  w.gturn = cv.take<int32_t>((size_t)B * L);
  w.src_cpr = w.src_tpc = w.src_turns = nullptr;
  if (o) *o = w;
  return cv.off;
}

hipError_t launch_build_layout(int32_t B, int32_t L, int32_t bq, int32_t bk, int32_t C, int32_t T,
                               const LayoutWs &ws, const opr_layout &out, hipStream_t s) {
  const int32_t MT = (L + bq - 1) / bq, NT = (L + bk - 1) / bk;
  layout_prep<<<1, kPrepThreads, 0, s>>>(B, C, T, ws);
  const int64_t ntok = (int64_t)B * L;
  layout_fill<<<(unsigned)((ntok + 255) / 256), 256, 0, s>>>(B, L, ws, out);
  const int64_t tiles = (int64_t)B * MT * NT;
#define OPR_CLASSIFY_CASE(Q, K) \
  if (bq == Q && bk == K) launch_classify<Q, K>(tiles, B, L, MT, NT, ws, out, s);
  OPR_CLASSIFY_CASE(32, 32) OPR_CLASSIFY_CASE(32, 64) OPR_CLASSIFY_CASE(32, 128)
  OPR_CLASSIFY_CASE(64, 32) OPR_CLASSIFY_CASE(64, 64) OPR_CLASSIFY_CASE(64, 128)
  OPR_CLASSIFY_CASE(128, 32) OPR_CLASSIFY_CASE(128, 64) OPR_CLASSIFY_CASE(128, 128)
#undef OPR_CLASSIFY_CASE
  const int64_t row_groups = ((int64_t)B * MT + kCmpThreads / 64 - 1) / (kCmpThreads / 64);
  const int64_t col_groups = 8 * (((int64_t)B * ((NT + kCmpCols - 1) / kCmpCols) + 7) / 8);
  layout_compact<<<(unsigned)(row_groups + col_groups), kCmpThreads, 0, s>>>(B, MT, NT, (int32_t)row_groups, out);
  return hipGetLastError();
}

}  // namespace opr

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
//                    (layout_classify_attention: the same over attention
//                    order, from the query's two runs of slots, one
//                    workgroup per q-tile row)
//   layout_compact_q/k  one wave per tile row / column: ballot compaction of
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
// the whole workgroup; out[n] is the total.
template <class Get>
__device__ void block_exclusive_scan(int n, Get get, int32_t *out, int32_t *sh) {
  const int tid = threadIdx.x;
  int32_t carry = 0;
  for (int base = 0; base < n; base += kPrepThreads) {
    const int i = base + tid;
    const int32_t v = (i < n) ? get(i) : 0;
    sh[tid] = v;
    __syncthreads();
    for (int d = 1; d < kPrepThreads; d <<= 1) {
      const int32_t add = (tid >= d) ? sh[tid - d] : 0;
      __syncthreads();
      sh[tid] += add;
      __syncthreads();
    }
    if (i < n) out[i] = carry + sh[tid] - v;
    const int32_t total = sh[kPrepThreads - 1];
    __syncthreads();
    carry += total;
  }
  if (tid == 0) out[n] = carry;
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

__global__ __launch_bounds__(kPrepThreads) void layout_prep(int32_t B, int32_t C, int32_t T,
                                                            LayoutWs ws) {
  __shared__ int32_t sh[kPrepThreads];
  const int32_t *cpr = ws.cpr;
  const int32_t *tpc = ws.tpc;
  const int4 *turns = ws.turns;
  block_exclusive_scan(B, [&](int i) { return cpr[i]; }, ws.row_conv0, sh);
  block_exclusive_scan(C, [&](int i) { return tpc[i]; }, ws.conv_turn0, sh);
  // tokens of a turn: h + t + r_in + r_out
  block_exclusive_scan(T, [&](int i) { int4 u = turns[i]; return u.x + u.y + u.z + u.w; },
                       ws.tok_g, sh);
  // the next human message starts after h_i and r_in_i: the position advance
  // per turn is h + r_in, which is also the number of history tokens
  block_exclusive_scan(T, [&](int i) { int4 u = turns[i]; return u.x + u.z; }, ws.pos_g, sh);
  for (int c = threadIdx.x; c < C; c += kPrepThreads)
    ws.conv_row[c] = last_le(ws.row_conv0, 0, B + 1, c);
  for (int t = threadIdx.x; t < T; t += kPrepThreads)
    ws.turn_conv[t] = last_le(ws.conv_turn0, 0, C + 1, t);
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

// Tile classes over attention order: one workgroup of BQ threads per q-tile
// row (b, m).  The row's queries (slots m*BQ ..) put their two runs of slots
// in LDS, and their union gives the span of key slots any of them sees: key
// tiles outside it are empty and are written as such directly.  In the
// others each thread counts whole 32x32 sub-blocks, summing over the
// sub-block's 32 queries the part of their runs inside its 32 key slots.
// kClsBatch tiles at a time meet in LDS, and their class words are written
// together.
constexpr int kClsBatch = 64;

template <int BQ, int BK>
__global__ __launch_bounds__(BQ) void layout_classify_attention(int32_t B, int32_t L, int32_t MT,
                                                                int32_t NT, opr_layout out) {
  constexpr int SQ = BQ / OPR_SUB_BLOCK, SK = BK / OPR_SUB_BLOCK, NSB = SQ * SK;
  __shared__ int4 runs[BQ];
  __shared__ int32_t cnt[kClsBatch][NSB];
  __shared__ int32_t span[2];
  const int64_t row = blockIdx.x;  // b * MT + m
  const int32_t m = (int32_t)(row % MT);
  const int32_t b = (int32_t)(row / MT);
  const int tid = threadIdx.x;
  const int32_t q = m * BQ + tid;
  int4 iv = make_int4(0, 0, 0, 0);
  if (q < L) iv = reinterpret_cast<const int4 *>(out.slot_qiv)[(int64_t)b * L + q];
  runs[tid] = iv;
  if (tid == 0) {
    span[0] = INT32_MAX;
    span[1] = INT32_MIN;
  }
  __syncthreads();
  if (iv.x < iv.y || iv.z < iv.w) {
    atomicMin(&span[0], iv.x < iv.y ? iv.x : iv.z);
    atomicMax(&span[1], iv.z < iv.w ? iv.w : iv.y);
  }
  __syncthreads();
  uint8_t *tcls = out.tile_class + row * NT;
  uint32_t *scls = out.sub_class + row * NT;
  const int32_t n_lo = span[0] <= span[1] ? span[0] / BK : 0;
  const int32_t n_hi = span[0] <= span[1] ? (span[1] - 1) / BK : -1;  // empty range if no key is seen
  for (int32_t n = tid; n < NT; n += BQ) {
    if (n < n_lo || n > n_hi) {
      tcls[n] = OPR_TILE_EMPTY;
      scls[n] = 0u;
    }
  }
  for (int32_t nb = n_lo; nb <= n_hi; nb += kClsBatch) {
    const int nt = min(kClsBatch, n_hi + 1 - nb);
    for (int x = tid; x < nt * NSB; x += BQ) {
      const int t = x / NSB, i = x - t * NSB, sq = i / SK, j = i - sq * SK;
      const int32_t a = (nb + t) * BK + j * OPR_SUB_BLOCK;
      const int32_t e = min(a + OPR_SUB_BLOCK, L);
      int32_t c = 0;
#pragma unroll 8
      for (int r = 0; r < OPR_SUB_BLOCK; ++r) {
        const int4 u = runs[sq * OPR_SUB_BLOCK + r];
        c += overlap(a, e, u.x, u.y) + overlap(a, e, u.z, u.w);
      }
      cnt[t][i] = c;
    }
    __syncthreads();
    for (int t = tid; t < nt; t += BQ) {
      uint32_t word = 0;
      int32_t total = 0;
      for (int i = 0; i < NSB; ++i) {
        const int32_t v = cnt[t][i];
        total += v;
        const uint32_t cls = v == 0 ? OPR_TILE_EMPTY
                           : (v == OPR_SUB_BLOCK * OPR_SUB_BLOCK ? OPR_TILE_FULL : OPR_TILE_PARTIAL);
        word |= cls << (2 * i);
      }
      tcls[nb + t] = total == 0 ? OPR_TILE_EMPTY : (total == BQ * BK ? OPR_TILE_FULL : OPR_TILE_PARTIAL);
      scls[nb + t] = word;
    }
    __syncthreads();
  }
}

// One wave per (b, m): k-tile indices of the non-empty tiles of q-tile row m.
__global__ __launch_bounds__(64) void layout_compact_q(int32_t MT, int32_t NT, opr_layout out) {
  const int64_t row = blockIdx.x;  // b * MT + m
  const uint8_t *cls = out.tile_class + row * NT;
  int32_t *lst = out.q_list + row * NT;
  const int lane = threadIdx.x;
  int32_t count = 0;
  for (int32_t base = 0; base < NT; base += 64) {
    const int32_t n = base + lane;
    const bool nz = n < NT && cls[n] != OPR_TILE_EMPTY;
    const uint64_t bal = __ballot(nz);
    const int32_t before = __popcll(bal & ((1ull << lane) - 1ull));
    if (nz) lst[count + before] = n;
    count += __popcll(bal);
  }
  for (int32_t n = count + lane; n < NT; n += 64) lst[n] = -1;
  if (lane == 0) out.q_nnz[row] = count;
}

// One wave per (b, n): q-tile indices of the non-empty tiles of k-tile column n.
__global__ __launch_bounds__(64) void layout_compact_k(int32_t MT, int32_t NT, opr_layout out) {
  const int64_t col = blockIdx.x;  // b * NT + n
  const int64_t b = col / NT;
  const int32_t n = (int32_t)(col - b * NT);
  const uint8_t *cls = out.tile_class + b * MT * NT + n;
  int32_t *lst = out.k_list + col * MT;
  const int lane = threadIdx.x;
  int32_t count = 0;
  for (int32_t base = 0; base < MT; base += 64) {
    const int32_t m = base + lane;
    const bool nz = m < MT && cls[(int64_t)m * NT] != OPR_TILE_EMPTY;
    const uint64_t bal = __ballot(nz);
    const int32_t before = __popcll(bal & ((1ull << lane) - 1ull));
    if (nz) lst[count + before] = m;
    count += __popcll(bal);
  }
  for (int32_t m = count + lane; m < MT; m += 64) lst[m] = -1;
  if (lane == 0) out.k_nnz[col] = count;
}

template <int BQ, int BK>
void launch_classify(int64_t tiles, int32_t B, int32_t L, int32_t MT, int32_t NT,
                     const LayoutWs &ws, const opr_layout &out, hipStream_t s) {
  if (out.order == OPR_ORDER_ATTENTION)
    layout_classify_attention<BQ, BK><<<dim3((unsigned)((int64_t)B * MT)), dim3(BQ), 0, s>>>(B, L, MT, NT, out);
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
  layout_compact_q<<<(unsigned)((int64_t)B * MT), 64, 0, s>>>(MT, NT, out);
  layout_compact_k<<<(unsigned)((int64_t)B * NT), 64, 0, s>>>(MT, NT, out);
  return hipGetLastError();
}

}  // namespace opr

// K-pass chunk planner (host only): split one conversation into contiguous
// runs of turns, each trained in a sequence of its own after the context of
// the turns before it.
//
// The pages place the K-pass variant between one pass per conversation
// (fastest, most memory) and the N-pass formulation (least memory) and report
// how speed and memory move with K (wiki summary, section "实验结果", K-Pass;
// section "关键洞察", item 3).  How a conversation is cut into chunks is left
// open; this planner searches every contiguous split for the one of least
// modelled cost under a cap on a chunk's length.
//
// Cost model of a chunk sequence: pairs + weight * tokens, where pairs is the
// number of allowed (query, key) pairs, the quantity attention time follows,
// and tokens the packed length, which the per-token work (projections, the
// prologue passes) follows.  Under the strategic position ids (section
// "位置 ID 策略") every token sees exactly position id + 1 keys, so a segment
// of n tokens starting at position p holds n*p + n(n+1)/2 pairs, and the
// start of turn l is the same in every chunk sequence that contains it:
// S_l = sum over m < l of (h_m + r_in_m).  Chunk costs therefore come from
// prefix sums, and a dynamic program over turn boundaries finds the optimum in
// O(K * N^2) time and O(K * N) memory (exactly K chunks), or in O(N^2) time
// and O(N) memory (any number: one layer over (cost, chunks), compared in that
// order, so that ties go to fewer chunks).
//
// The context copy r_in of a chunk's last turn is seen by no query of its
// sequence (only later turns see a turn's r_in, and it carries no loss), so
// with elide_last_rin it is left out; no other token's position or output
// changes.
#include <cmath>
#include <cstdint>
#include <limits>
#include <new>
#include <vector>

#include "opr.h"

namespace {

// pairs of a segment of n tokens at positions p0 .. p0 + n - 1
inline int64_t seg_pairs(int64_t n, int64_t p0) { return n * p0 + n * (n + 1) / 2; }

struct Prefix {
  std::vector<int64_t> ctx_tok, full_tok;    // tokens of turns [0, l) as history / in full
  std::vector<int64_t> ctx_pair, full_pair;  // their pairs
  std::vector<int64_t> rin_tok, rin_pair;    // r_in of turn l alone
};

Prefix prefixes(const opr_turn *turns, int n) {
  Prefix P;
  P.ctx_tok.assign(n + 1, 0);
  P.full_tok.assign(n + 1, 0);
  P.ctx_pair.assign(n + 1, 0);
  P.full_pair.assign(n + 1, 0);
  P.rin_tok.assign(n, 0);
  P.rin_pair.assign(n, 0);
  int64_t s = 0;  // start position of turn l
  for (int l = 0; l < n; ++l) {
    const int64_t h = turns[l].h, t = turns[l].t, ri = turns[l].r_in, ro = turns[l].r_out;
    const int64_t ph = seg_pairs(h, s), pri = seg_pairs(ri, s + h);
    P.ctx_tok[l + 1] = P.ctx_tok[l] + h + ri;
    P.ctx_pair[l + 1] = P.ctx_pair[l] + ph + pri;
    P.full_tok[l + 1] = P.full_tok[l] + h + t + ri + ro;
    P.full_pair[l + 1] = P.full_pair[l] + ph + seg_pairs(t, s + h) + pri + seg_pairs(ro, s + h + t);
    P.rin_tok[l] = ri;
    P.rin_pair[l] = pri;
    s += h + ri;
  }
  return P;
}

struct Chunk {
  int64_t tokens, pairs;
};

// the sequence of turns [a, b): history [0, a) then turns a .. b-1 in full
inline Chunk chunk_of(const Prefix &P, int a, int b, bool elide) {
  Chunk c;
  c.tokens = P.ctx_tok[a] + P.full_tok[b] - P.full_tok[a];
  c.pairs = P.ctx_pair[a] + P.full_pair[b] - P.full_pair[a];
  if (elide) {
    c.tokens -= P.rin_tok[b - 1];
    c.pairs -= P.rin_pair[b - 1];
  }
  return c;
}

// Size limits: N <= kMaxTurns turns for any number of chunks (O(N^2)); for
// exactly K chunks K * N^2 <= kMaxWork (time) as well.
constexpr int32_t kMaxTurns = 1 << 16;
constexpr int64_t kMaxWork = (int64_t)1 << 33;

opr_status plan(const opr_turn *turns, int32_t n_turns, int32_t n_chunks, int32_t max_tokens, double tokens_weight,
                int32_t elide_last_rin, opr_chunk *chunks, int32_t *n_out, double *cost) {
  const int N = n_turns;
  const bool elide = elide_last_rin != 0;
  const Prefix P = prefixes(turns, N);
  const int64_t cap = max_tokens > 0 ? max_tokens : std::numeric_limits<int64_t>::max();
  const double inf = std::numeric_limits<double>::infinity();
  auto chunk_cost = [&](const Chunk &c) { return (double)c.pairs + tokens_weight * (double)c.tokens; };

  std::vector<int> ends;  // chunk boundaries 0 = ends[0] < ... < ends[K] = N
  double total = inf;
  if (n_chunks == 0) {
    // best[j]: least (cost, chunks) of turns [0, j), compared in that order
    std::vector<double> bc(N + 1, inf);
    std::vector<int32_t> bn(N + 1, std::numeric_limits<int32_t>::max()), from(N + 1, -1);
    bc[0] = 0.0;
    bn[0] = 0;
    for (int j = 1; j <= N; ++j) {
      for (int i = 0; i < j; ++i) {
        if (bc[i] == inf) continue;
        const Chunk c = chunk_of(P, i, j, elide);
        if (c.tokens > cap) continue;
        const double v = bc[i] + chunk_cost(c);
        const int32_t nv = bn[i] + 1;
        if (v < bc[j] || (v == bc[j] && nv < bn[j])) {
          bc[j] = v;
          bn[j] = nv;
          from[j] = i;
        }
      }
    }
    if (bc[N] == inf) return OPR_E_CAPACITY;
    total = bc[N];
    for (int j = N; j > 0; j = from[j]) ends.push_back(j);
    ends.push_back(0);
    std::vector<int>(ends.rbegin(), ends.rend()).swap(ends);
  } else {
    // best[k][j]: least cost of turns [0, j) in exactly k chunks
    const int K = n_chunks;
    std::vector<double> best((size_t)(K + 1) * (N + 1), inf);
    std::vector<int32_t> from((size_t)(K + 1) * (N + 1), -1);
    auto at = [&](int k, int j) { return (size_t)k * (N + 1) + j; };
    best[at(0, 0)] = 0.0;
    for (int k = 1; k <= K; ++k) {
      for (int j = k; j <= N; ++j) {
        double bj = inf;
        int arg = -1;
        for (int i = k - 1; i < j; ++i) {
          const double bi = best[at(k - 1, i)];
          if (bi == inf) continue;
          const Chunk c = chunk_of(P, i, j, elide);
          if (c.tokens > cap) continue;
          const double v = bi + chunk_cost(c);
          if (v < bj) {
            bj = v;
            arg = i;
          }
        }
        best[at(k, j)] = bj;
        from[at(k, j)] = arg;
      }
    }
    if (best[at(K, N)] == inf) return OPR_E_CAPACITY;
    total = best[at(K, N)];
    ends.assign(K + 1, 0);
    ends[K] = N;
    for (int k = K; k >= 1; --k) ends[k - 1] = from[at(k, ends[k])];
  }

  const int K = (int)ends.size() - 1;
  for (int k = 0; k < K; ++k) {
    const Chunk c = chunk_of(P, ends[k], ends[k + 1], elide);
    chunks[k].first_turn = ends[k];
    chunks[k].n_turns = ends[k + 1] - ends[k];
    chunks[k].tokens = (int32_t)c.tokens;
    chunks[k].rin_elided = elide ? 1 : 0;
    chunks[k].pairs = c.pairs;
  }
  *n_out = K;
  if (cost) *cost = total;
  return OPR_OK;
}

}  // namespace

extern "C" opr_status opr_kpass_plan(const opr_turn *turns, int32_t n_turns, int32_t n_chunks,
                                     int32_t max_tokens, double tokens_weight, int32_t elide_last_rin,
                                     opr_chunk *chunks, int32_t *n_out, double *cost) {
  if (!turns || !chunks || !n_out || n_turns < 1 || n_chunks < 0 || n_chunks > n_turns || max_tokens < 0 ||
      !std::isfinite(tokens_weight) || tokens_weight < 0.0)
    return OPR_E_INVALID;
  int64_t total = 0;
  for (int l = 0; l < n_turns; ++l) {
    const opr_turn &u = turns[l];
    if (u.h < 0 || u.t < 0 || u.r_in < 0 || u.r_out < 0) return OPR_E_INVALID;
    total += (int64_t)u.h + u.t + u.r_in + u.r_out;
  }
  // every chunk holds at most each turn's segments once
  if (total > std::numeric_limits<int32_t>::max()) return OPR_E_INVALID;
  if (n_turns > kMaxTurns) return OPR_E_UNSUPPORTED;
  if (n_chunks > 0 && (int64_t)n_chunks * n_turns * n_turns > kMaxWork) return OPR_E_UNSUPPORTED;
  try {
    return plan(turns, n_turns, n_chunks, max_tokens, tokens_weight, elide_last_rin, chunks, n_out, cost);
  } catch (const std::bad_alloc &) {
    return OPR_E_UNSUPPORTED;  // the tables do not fit in host memory; nothing was written
  }
}

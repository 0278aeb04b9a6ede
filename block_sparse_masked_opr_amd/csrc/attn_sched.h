// Stage lists of the attention kernels: the non-empty 32-key quarters
// (forward, dQ) or 64-query halves (dK/dV) of a workgroup's non-empty
// 128 x 128 tiles, compacted by one wave into LDS with a ballot, so that the
// pipelined main loops read their schedule from LDS.
#pragma once

#include "attn_common.h"

namespace opr {

// Forward: the stages are the 32-key quarters j of the tiles q_list[t ...]
// in which any wave's 32 x 32 sub-block (w, j) is non-empty, up to CAP per
// chunk.  Descriptor: x = first key slot, y bits 2w = class of wave w's
// sub-block.  Returns the count; advances *t.
template <int CAP>
__device__ inline int build_q_quarters(const int32_t *lst, const uint32_t *subs, int nnz, int NT, int *t,
                                       uint2 *stages, int lane, uint32_t *dbg) {
  int count = 0;
  while (*t < nnz && count + 64 <= CAP) {
    const int tile = *t + (lane >> 2), j = lane & 3;
    uint32_t cls = 0;
    int k0 = 0;
    const int n = tile < nnz ? lst[tile] : -1;
    if (tile < nnz && OPR_DCHECK(dbg, (unsigned)n < (unsigned)NT, kDbgQList)) {
      const uint32_t sub = subs[n];
      k0 = n * 128 + 32 * j;
#pragma unroll
      for (int w = 0; w < 4; ++w) cls |= ((sub >> (2 * (4 * w + j))) & 3u) << (2 * w);
    }
    const uint64_t bal = __ballot(cls != 0);
    if (cls != 0) stages[count + __popcll(bal & ((1ull << lane) - 1ull))] = make_uint2((uint32_t)k0, cls);
    count += __popcll(bal);
    *t += 16;
  }
  if (*t > nnz) *t = nnz;
  return count;
}

// Key-side kernel (dK/dV) of k-tile n: wave w owns key sub-column w; the
// stages run over the q-tiles k_list[...] x the G heads of the kv group x the
// two 64-query halves, flat index f = (tile * G + head) * 2 + half, from *f up
// to fend (a work item's part of the column's range).  Descriptor: x = first
// query slot, plus the head (in the kv group) at bits 24..31; y bits 4w + 2b
// = class (empty / partial / full) of the 32 x 32 sub-block that wave w
// meets in 32-query block b of the stage.
constexpr int kKStageCap = 1024;  // dK/dV descriptors per list chunk (8 KB of LDS)

__device__ inline int build_k_stages(const int32_t *lst, const uint32_t *subs_b, int NT, int MT, int n, int G,
                                     int64_t fend, int64_t *f, uint2 *stages, int lane, uint32_t *dbg) {
  int count = 0;
  while (*f < fend && count + 64 <= kKStageCap) {
    const int64_t ff = *f + lane;
    uint32_t cls = 0, x = 0;
    if (ff < fend) {
      const int qh = (int)(ff & 1);
      const int64_t tj = ff >> 1;
      const int hj = (int)(tj % G);
      const int m = lst[tj / G];
      const uint32_t sub =
          OPR_DCHECK(dbg, (unsigned)m < (unsigned)MT, kDbgKList) ? subs_b[(int64_t)m * NT + n] : 0u;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) cls |= ((sub >> (2 * (4 * (2 * qh + qb) + w))) & 3u) << (4 * w + 2 * qb);
      x = (uint32_t)(m * 128 + 64 * qh) | ((uint32_t)hj << 24);
    }
    const uint64_t bal = __ballot(cls != 0);
    if (cls != 0) stages[count + __popcll(bal & ((1ull << lane) - 1ull))] = make_uint2(x, cls);
    count += __popcll(bal);
    *f += 64;
  }
  if (*f > fend) *f = fend;
  return count;
}

}  // namespace opr

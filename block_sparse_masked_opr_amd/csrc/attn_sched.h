// Stage lists of the attention kernels: the non-empty 64-row halves of a
// workgroup's non-empty 128 x 128 tiles, compacted by one wave into LDS with
// a ballot, so that the pipelined main loops read their schedule from LDS.
//
// Descriptor (x, y):
//   y bits 4w + 2b : 2-bit class (empty / partial / full) of the 32 x 32
//                    sub-block that wave w meets in 32-row block b of the stage
//   x              : first streamed row; dK/dV stages add the head (in the
//                    kv group) at bits 24..31
#pragma once

#include "attn_common.h"

namespace opr {

constexpr int kStageCap = 1024;  // descriptors per list chunk (8 KB of LDS)

// Query-side kernels (forward, dQ): wave w owns query sub-row w; the stages
// are the 64-key halves kh of the tiles q_list[t ...].  Returns the count;
// advances *t.
__device__ inline int build_q_stages(const int32_t *lst, const uint32_t *subs, int nnz, int *t,
                                     uint2 *stages, int lane) {
  int count = 0;
  while (*t < nnz && count + 64 <= kStageCap) {
    const int tile = *t + (lane >> 1), kh = lane & 1;
    uint32_t cls = 0;
    int k0 = 0;
    if (tile < nnz) {
      const int n = lst[tile];
      const uint32_t sub = subs[n];
      k0 = n * 128 + 64 * kh;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) cls |= ((sub >> (2 * (4 * w + 2 * kh + kb))) & 3u) << (4 * w + 2 * kb);
    }
    const uint64_t bal = __ballot(cls != 0);
    if (cls != 0) stages[count + __popcll(bal & ((1ull << lane) - 1ull))] = make_uint2((uint32_t)k0, cls);
    count += __popcll(bal);
    *t += 32;
  }
  if (*t > nnz) *t = nnz;
  return count;
}

// Forward: the stages are the 32-key quarters j of the tiles q_list[t ...]
// in which any wave's 32 x 32 sub-block (w, j) is non-empty, up to CAP per
// chunk.  Descriptor: x = first key slot, y bits 2w = class of wave w's
// sub-block.  Returns the count; advances *t.
template <int CAP>
__device__ inline int build_q_quarters(const int32_t *lst, const uint32_t *subs, int nnz, int *t,
                                       uint2 *stages, int lane) {
  int count = 0;
  while (*t < nnz && count + 64 <= CAP) {
    const int tile = *t + (lane >> 2), j = lane & 3;
    uint32_t cls = 0;
    int k0 = 0;
    if (tile < nnz) {
      const int n = lst[tile];
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
// to fend (a work item's part of the column's range).  The descriptor is
// (x, y) as above.
constexpr int kKStageCap = 1024;  // dK/dV descriptors per list chunk (8 KB of LDS)

__device__ inline int build_k_stages(const int32_t *lst, const uint32_t *subs_b, int NT, int n, int G,
                                     int64_t fend, int64_t *f, uint2 *stages, int lane) {
  int count = 0;
  while (*f < fend && count + 64 <= kKStageCap) {
    const int64_t ff = *f + lane;
    uint32_t cls = 0, x = 0;
    if (ff < fend) {
      const int qh = (int)(ff & 1);
      const int64_t tj = ff >> 1;
      const int hj = (int)(tj % G);
      const int m = lst[tj / G];
      const uint32_t sub = subs_b[(int64_t)m * NT + n];
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

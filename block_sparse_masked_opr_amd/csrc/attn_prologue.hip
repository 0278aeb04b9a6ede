// Prologue kernels of the attention path.  Everything here is indexed by
// slot (attention order): slot s < L holds token slot_tok[s] of the layout,
// slots L .. Lp-1 are empty and padded with zeros.
//  - the RoPE table at the slots' strategic position ids (and zeroing of the
//    plane maxima),
//  - the largest magnitude of every (row, head) plane of q, k, v, dout,
//  - head-major fp16 copies of q, k (after RoPE), v and dout in slot order,
//    with one power-of-two scale per plane,
//  - the backward preprocessing delta = rowsum(dout * o), scaled, with the
//    dout plane maxima.
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
// and s >= L use position 0.  The first n_zero threads also clear zero_words.
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
// float bits.  A workgroup covers kAbsTokens tokens of HPB heads: thread
// (head hl, chunk j) reads 16-byte chunk j of head hl of every token, so each
// 16-lane group reads one head's whole row and a wave reads contiguous runs.
constexpr int kAbsTokens = 64;

// One launch covers q, k and v: blockIdx.y runs over the head blocks of
// job 0, then job 1, then job 2.
struct AbsmaxJob {
  const uint16_t *x;  // [B][L][H][D] bf16
  uint32_t *pmax;     // [B][H]
  int32_t H;
  int32_t hb_end;     // one past this job's last head block (cumulative)
  float factor;
};

template <int D>
__global__ __launch_bounds__(256) void absmax_kernel(int32_t L, AbsmaxJob j0, AbsmaxJob j1, AbsmaxJob j2) {
  constexpr int CPH = D / 8, HPB = 256 / CPH;
  const int yb = blockIdx.y;
  const bool in0 = yb < j0.hb_end, in1 = !in0 && yb < j1.hb_end;
  const uint16_t *x = in0 ? j0.x : (in1 ? j1.x : j2.x);
  uint32_t *pmax = in0 ? j0.pmax : (in1 ? j1.pmax : j2.pmax);
  const int32_t H = in0 ? j0.H : (in1 ? j1.H : j2.H);
  const float factor = in0 ? j0.factor : (in1 ? j1.factor : j2.factor);
  const int hb = yb - (in0 ? 0 : (in1 ? j0.hb_end : j1.hb_end));
  const int b = blockIdx.z, tid = threadIdx.x;
  const int hl = tid / CPH, j = tid % CPH;
  const int h = hb * HPB + hl;
  const int t0 = blockIdx.x * kAbsTokens;
  uint32_t m = 0u;  // float bits of the largest |x| (non-negative: integer order)
  if (h < H) {
    const uint16_t *src = x + (((int64_t)b * L + t0) * H + h) * D + j * 8;
    const int nt = min(kAbsTokens, L - t0);
#pragma unroll 8
    for (int t = 0; t < nt; ++t)
      m = max(m, absmax8_bf16_bits(*reinterpret_cast<const uint4 *>(src + (int64_t)t * H * D)));
  }
#pragma unroll
  for (int off = CPH / 2; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if (j == 0 && h < H && m > 0u) atomicMax(pmax + (int64_t)b * H + h, __float_as_uint(__uint_as_float(m) * factor));
}

// One workgroup per (64-slot block, group of kPackHeads heads, row): 4
// threads per slot, each owning D/8 rotation pairs, keep the slot's RoPE
// cosines and sines in registers and walk the heads.  x: [B][L][H][D] bf16 ->
// rows [B][H][Lp][D] in slot order, fp16(x' * 2^e), x' = RoPE(x) or x, e the
// exponent of the largest plane maximum of the head's group of `group`
// heads.  Slots s >= L are zero.
constexpr int kPackHeads = 8;

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void pack_kernel(int32_t L, int32_t Lp, int32_t H, int32_t group,
                                                   const uint16_t *x, const int32_t *slot_tok,
                                                   const float2 *table, const uint32_t *pmax,
                                                   uint16_t *rows) {
  constexpr int HALF = D / 2;
  constexpr int PER = HALF / 4;  // pairs per thread (4 threads per slot)
  const int hgroups = (H + kPackHeads - 1) / kPackHeads;
  const int h0 = (int)(blockIdx.x % (unsigned)hgroups) * kPackHeads;
  const int t0 = (int)(blockIdx.x / (unsigned)hgroups) * 64, b = blockIdx.z;
  const int tid = threadIdx.x;
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
    const int ex = group_exponent(pmax + (int64_t)b * H + (h / group) * group, group);
    uint16_t lq[PER], hq[PER];
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
        float lo = bf16_to_f32(lb[e]), hi = bf16_to_f32(hb[e]);
        if (ROPE) {
          const float x1 = lo, x2 = hi;
          lo = x1 * cs[e].x - x2 * cs[e].y;
          hi = x2 * cs[e].x + x1 * cs[e].y;
        }
        lq[e] = f32_to_f16_bits(ldexpf(lo, ex));
        hq[e] = f32_to_f16_bits(ldexpf(hi, ex));
      }
    } else {
#pragma unroll
      for (int e = 0; e < PER; ++e) lq[e] = hq[e] = 0;
    }
    uint16_t *dst = rows + (((int64_t)b * H + h) * Lp + t) * D;
#pragma unroll
    for (int c = 0; c < PER; c += 8) {
      *reinterpret_cast<uint4 *>(dst + j0 + c) = *reinterpret_cast<const uint4 *>(&lq[c]);
      *reinterpret_cast<uint4 *>(dst + HALF + j0 + c) = *reinterpret_cast<const uint4 *>(&hq[c]);
    }
  }
}

// Backward preprocessing, before dout is packed: per slot s and q head, with
// t = slot_tok[s] the token there,
//   dsc[b][h][s]  = sum_d dout * o of token t (float32 over bf16 inputs),
//   lse2[b][h][s] = lse * log2(e) - kPdvExp, +inf where the row has no key (lse = -inf)
//                   or s >= L, so that recomputed probabilities are exactly 0;
// and the largest |dout| of each (row, head) plane into mdo (float bits).
// One wave per slot: D/8 lanes read one head's 16-byte chunks, so a wave
// covers 64/(D/8) heads per step with fully coalesced row reads; the plane
// maxima are combined in LDS, then once per workgroup in memory.
constexpr int kMaxHeads = 1024;

template <int D>
__global__ __launch_bounds__(256) void delta_kernel(int32_t B, int32_t L, int32_t Lp, int32_t Hq,
                                                    const uint16_t *o, const uint16_t *dout, const float *lse,
                                                    const int32_t *slot_tok, uint32_t *mdo, float *dsc,
                                                    float *lse2) {
  constexpr int LPH = D / 8;        // lanes per head
  constexpr int HPS = 64 / LPH;     // heads per step
  constexpr int TPW = 4;            // tokens per wave
  __shared__ uint32_t hmax[kMaxHeads];
  for (int i = threadIdx.x; i < Hq; i += 256) hmax[i] = 0u;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int hl = lane / LPH, part = lane % LPH;
  const int64_t bt0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW;
  for (int k = 0; k < TPW; ++k) {
    const int64_t bt = bt0 + k;
    if (bt >= (int64_t)B * Lp) break;
    const int32_t sl = (int32_t)(bt % Lp);
    const int32_t b = (int32_t)(bt / Lp);
    if (b != (int32_t)(bt0 / Lp)) break;  // a workgroup's plane maxima stay within one row
    const int32_t t = sl < L ? slot_tok[(int64_t)b * L + sl] : L;  // token at the slot
#pragma unroll 4
    for (int h0 = 0; h0 < Hq; h0 += HPS) {
      const int h = h0 + hl;
      float acc = 0.0f;
      uint32_t mx = 0u;  // float bits of the largest |dout|
      if (t < L && h < Hq) {
        const int64_t base = (((int64_t)b * L + t) * Hq + h) * D + part * 8;
        const uint4 ov = *reinterpret_cast<const uint4 *>(o + base);
        const uint4 dv = *reinterpret_cast<const uint4 *>(dout + base);
        acc = dot2_bf16(ov.x, dv.x, acc);
        acc = dot2_bf16(ov.y, dv.y, acc);
        acc = dot2_bf16(ov.z, dv.z, acc);
        acc = dot2_bf16(ov.w, dv.w, acc);
        mx = absmax8_bf16_bits(dv);
      }
#pragma unroll
      for (int off = LPH / 2; off > 0; off >>= 1) {
        acc += __shfl_xor(acc, off);
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
      }
      if (part == 0 && h < Hq) {
        float l2 = INFINITY;
        if (t < L) {
          const float l = lse[((int64_t)b * Hq + h) * L + t];
          l2 = (l == -INFINITY) ? INFINITY : l * kLog2e - (float)kPdvExp;
        }
        const int64_t out = ((int64_t)b * Hq + h) * Lp + sl;
        dsc[out] = acc;
        lse2[out] = l2;
        if (mx > 0u) atomicMax(&hmax[h], mx);
      }
    }
  }
  __syncthreads();
  const int64_t b = ((int64_t)blockIdx.x * 4 * TPW) / Lp;
  if (b < B)
    for (int i = threadIdx.x; i < Hq; i += 256)
      if (hmax[i]) atomicMax(mdo + b * Hq + i, hmax[i]);
}

// dsc *= 2^(e_dout + e_v - kDsShift - kPdvExp): delta in the units of dP = dO V^T
// on the scaled operands, shifted like dS, times the 2^-kPdvExp that the
// fp16(P * 2^kPdvExp) of the dK/dV kernel cancels.  One thread per (b, h, t).
__global__ __launch_bounds__(256) void scale_delta_kernel(int32_t B, int32_t Lp, int32_t Hq, int32_t group,
                                                          const uint32_t *mdo, const uint32_t *mv, float *dsc) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)B * Hq * Lp) return;
  const int64_t bh = gid / Lp;
  const int h = (int)(bh % Hq);
  const int64_t b = bh / Hq;
  const int kv = h / group, Hkv = Hq / group;
  const int e = group_exponent(mdo + b * Hq + kv * group, group) + plane_exponent(mv[b * Hkv + kv]) - kDsShift - kPdvExp;
  dsc[gid] = ldexpf(dsc[gid], e);
}

// Longest-first work order (see q_work_item): the q-tile rows (b*MT + m) by
// decreasing number of non-empty 64-key halves over their tile lists - the
// stages of a forward or dQ workgroup - and the k-tile columns (b*NT + n) by
// decreasing number of non-empty 64-query halves - the stages of a dK/dV
// workgroup.  One workgroup: per-item costs, then a counting sort (costs
// above kOrderBins - 1 share the last bin; ties in any order).
constexpr int kOrderThreads = 1024, kOrderBins = 4096;

__global__ __launch_bounds__(kOrderThreads) void work_order_kernel(int32_t n_rows, int32_t n_cols, int32_t MT,
                                                                   int32_t NT, const uint32_t *sub_class,
                                                                   const int32_t *q_nnz, const int32_t *q_list,
                                                                   const int32_t *k_nnz, const int32_t *k_list,
                                                                   int32_t *cost, int32_t *q_order,
                                                                   int32_t *k_order) {
  __shared__ int32_t bins[kOrderBins];
  __shared__ int32_t wave_sum[kOrderThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int pass = 0; pass < 2; ++pass) {
    const int32_t n = pass == 0 ? n_rows : n_cols;
    int32_t *order = pass == 0 ? q_order : k_order;
    int32_t *c = cost + (pass == 0 ? 0 : n_rows);
    for (int i = tid; i < kOrderBins; i += kOrderThreads) bins[i] = 0;
    __syncthreads();
    // 8 lanes per item, each summing every 8th entry of its tile list
    const int sub = tid & 7;
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
        k = min(k, kOrderBins - 1);
        c[it] = k;
        atomicAdd(&bins[kOrderBins - 1 - k], 1);  // bin 0 holds the largest cost
      }
    }
    __syncthreads();
    // exclusive scan of the bins: 4 per thread, then over the threads
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
    for (int32_t it = tid; it < n; it += kOrderThreads) order[atomicAdd(&bins[kOrderBins - 1 - c[it]], 1)] = it;
    __syncthreads();
  }
}

__global__ void zero_words_kernel(uint32_t *p, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <int D>
void launch_absmax_d(int32_t B, int32_t L, const AbsmaxJob *jobs, hipStream_t s) {
  absmax_kernel<D><<<dim3((L + kAbsTokens - 1) / kAbsTokens, jobs[2].hb_end, B), 256, 0, s>>>(L, jobs[0], jobs[1],
                                                                                             jobs[2]);
}

template <int D>
void launch_pack_d(bool rope, int32_t B, int32_t L, int32_t Lp, int32_t H, int32_t group, const void *x,
                   const int32_t *slot_tok, const float2 *table, const uint32_t *pmax, uint16_t *rows,
                   hipStream_t s) {
  const unsigned hgroups = (unsigned)((H + kPackHeads - 1) / kPackHeads);
  const dim3 grid(hgroups * (unsigned)(Lp / 64), 1, B);
  const uint16_t *src = static_cast<const uint16_t *>(x);
  if (rope) pack_kernel<D, true><<<grid, 256, 0, s>>>(L, Lp, H, group, src, slot_tok, table, pmax, rows);
  else pack_kernel<D, false><<<grid, 256, 0, s>>>(L, Lp, H, group, src, slot_tok, table, pmax, rows);
}

}  // namespace

// RoPE table + clearing of the plane maxima (they must start at zero).
void launch_rope_table(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  const int32_t half = in.D / 2;
  const int64_t total = (int64_t)in.B * ws.Lp * half;
  const int64_t blocks = ((total > ws.n_pmax ? total : (int64_t)ws.n_pmax) + 255) / 256;
  rope_table_kernel<<<(unsigned)blocks, 256, 0, s>>>(in.B, in.L, ws.Lp, half, log2(in.rope_theta),
                                                     in.layout.tok_pos, in.layout.slot_tok, ws.rope, ws.pmax,
                                                     ws.n_pmax);
}

// Plane maxima of q and k (times sqrt(2), the RoPE bound) and of v.
void launch_absmax_qkv(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  const int HPB = 256 / (in.D / 8);
  AbsmaxJob jobs[3];
  const void *xs[3] = {in.q, in.k, in.v};
  uint32_t *ms[3] = {ws.mq, ws.mk, ws.mv};
  const int32_t hs[3] = {in.Hq, in.Hkv, in.Hkv};
  int32_t end = 0;
  for (int i = 0; i < 3; ++i) {
    end += (hs[i] + HPB - 1) / HPB;
    jobs[i] = AbsmaxJob{static_cast<const uint16_t *>(xs[i]), ms[i], hs[i], end, i < 2 ? 1.4142136f : 1.0f};
  }
  if (in.D == 64) launch_absmax_d<64>(in.B, in.L, jobs, s);
  else launch_absmax_d<128>(in.B, in.L, jobs, s);
}

void launch_pack_any(int D, bool rope, int32_t B, int32_t L, int32_t Lp, int32_t H, int32_t group,
                     const void *x, const int32_t *slot_tok, const float2 *table, const uint32_t *pmax,
                     uint16_t *rows, hipStream_t s) {
  if (D == 64) launch_pack_d<64>(rope, B, L, Lp, H, group, x, slot_tok, table, pmax, rows, s);
  else launch_pack_d<128>(rope, B, L, Lp, H, group, x, slot_tok, table, pmax, rows, s);
}

void launch_work_order(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  const int32_t MT = ws.Lp / OPR_ATTN_BLOCK, NT = MT;
  work_order_kernel<<<1, kOrderThreads, 0, s>>>(in.B * MT, in.B * NT, MT, NT, in.layout.sub_class, in.layout.q_nnz,
                                               in.layout.q_list, in.layout.k_nnz, in.layout.k_list, ws.order_cost,
                                               ws.q_order, ws.k_order);
}

// delta, lse2 and the dout plane maxima (mdo is cleared first), then dout
// packing and the delta scaling are done by the caller in that order.
void launch_delta(const opr_attn_in &in, const void *o, const void *dout, const float *lse,
                  const AttnWs &ws, hipStream_t s) {
  const int32_t nz = in.B * in.Hq;
  zero_words_kernel<<<(nz + 255) / 256, 256, 0, s>>>(ws.mdo, nz);
  const int64_t tokens = (int64_t)in.B * ws.Lp;  // 16 tokens per workgroup
  const unsigned blocks = (unsigned)((tokens + 15) / 16);
  const uint16_t *o16 = static_cast<const uint16_t *>(o);
  const uint16_t *d16 = static_cast<const uint16_t *>(dout);
  if (in.D == 64)
    delta_kernel<64><<<blocks, 256, 0, s>>>(in.B, in.L, ws.Lp, in.Hq, o16, d16, lse, in.layout.slot_tok,
                                            ws.mdo, ws.dsc, ws.lse2);
  else
    delta_kernel<128><<<blocks, 256, 0, s>>>(in.B, in.L, ws.Lp, in.Hq, o16, d16, lse, in.layout.slot_tok,
                                             ws.mdo, ws.dsc, ws.lse2);
}

void launch_scale_delta(const opr_attn_in &in, const AttnWs &ws, hipStream_t s) {
  const int64_t total = (int64_t)in.B * in.Hq * ws.Lp;
  scale_delta_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(in.B, ws.Lp, in.Hq, in.Hq / in.Hkv, ws.mdo,
                                                                     ws.mv, ws.dsc);
}

}  // namespace opr

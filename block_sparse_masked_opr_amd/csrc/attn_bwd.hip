// Backward kernels of the one-pass masked attention (gfx950).
//
// With P recomputed from the forward LSE (P = exp2(scale*log2(e)*S - lse2)),
//   dV  = sum over the group's q heads of P^T dO
//   dP  = dO V^T,  dS = P * (dP - delta),  delta = rowsum(dO * O)
//   dQ' = scale * dS K',  dK' = scale * sum over the group of dS^T Q'
// and dQ, dK are rotated back by the transposed RoPE rotation.
//
// Both kernels run in attention order (tiles of slots; results are written
// at the slot's token).
// attn_dkdv_kernel: one workgroup per (128-key tile n, kv head, row); wave w
//   owns key slots n*128 + 32w .. +31, one per lane column, K' and V of its
//   key in registers.  Its stages are (q-tile of k_list, head of the group,
//   64-query half) with a non-empty sub-block; each streams the Q' and dO rows
//   of the stage into LDS (double buffered, buffer loads to LDS) and reads
//   Q'^T and dO^T from the same row-major tiles with transposing LDS reads.
//   dK^T and dV^T stay in accumulators; each key is owned by exactly one
//   workgroup: no atomics.
// attn_dq_kernel (attn_dq.hip): one workgroup per (128-query tile, q head,
//   row), pipelined like the forward kernel over the K' / V tiles; S and dP^T
//   are recomputed per non-empty sub-block and dQ^T += K'^T dS^T.
// Work items start longest first, round-robin over the XCDs (q_order and
// k_order of the prologue).  Partial sub-blocks are masked with 64-bit masks
// built from the two runs of slots of each query or key.
//
// Units: q' and dout carry one exponent per (row, kv group), k' and v one per
// (row, kv head), all constant inside a workgroup.  dP = dO V^T comes out in
// units 2^(e_dout + e_v); delta arrives pre-scaled into those units times
// 2^-kDsShift, and dS is formed as P * 2^-kDsShift * (dP - delta) before the
// fp16 conversion; P for dV is stored as fp16(P * 2^15).
#include <type_traits>

#include "attn_common.h"
#include "attn_sched.h"
#include "opr_internal.h"

namespace opr {
namespace {

constexpr int kPdvExp = 15;  // P (<= 1) enters dV as fp16(P * 2^15)

template <int D>
__global__ __launch_bounds__(256, 1) void attn_dkdv_kernel(AttnParams p, float *dk, float *dv) {
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int HALF_DB = NDB / 2;
  constexpr int TB = Tile<D>::BYTES, RB = Tile<D>::RB;
  // per buffer: Q' tile, dO tile, lse2[64], scaled delta[64]
  constexpr int BUF = 2 * TB + 512;
  // two separate LDS objects so the copy into one provably leaves the other alone
  __shared__ __attribute__((aligned(1024))) char buf0[BUF];
  __shared__ __attribute__((aligned(1024))) char buf1[BUF];
  __shared__ uint2 stages[kStageCap];
  __shared__ int sh_count;
  __shared__ int64_t sh_next;

  const int64_t R = blockIdx.x;  // rank: longest columns first, round-robin over the XCDs
  if (R >= (int64_t)p.B * p.NT * p.Hkv) return;
  const int32_t col = p.k_order[R / p.Hkv];
  const int kvh = (int)(R % p.Hkv);
  const int b = col / p.NT;
  const int n = col - b * p.NT;

  const int tid = threadIdx.x, w = uniform(tid >> 6), lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int key = n * 128 + 32 * w + li;
  const int64_t kvplane = (int64_t)b * p.Hkv + kvh;
  const int64_t hbase = (int64_t)b * p.Hq + (int64_t)kvh * p.group;  // first q head of the group
  const int eq = group_exponent(p.mq + hbase, p.group);
  const int edo = group_exponent(p.mdo + hbase, p.group);
  const int ek = plane_exponent(p.mk[kvplane]);
  const int ev = plane_exponent(p.mv[kvplane]);
  const float fs = ldexpf(p.scale_log2, -(eq + ek));
  const float pdv = ldexpf(1.0f, kPdvExp);
  const float dss = ldexpf(1.0f, -kDsShift);

  f16x8 kb_[NS], vb_[NS];
  {
    const int64_t off = (kvplane * p.Lp + key) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kb_[s] = ld_f16x8(p.kr + off + 16 * s + 8 * g);
      vb_[s] = ld_f16x8(p.vr + off + 16 * s + 8 * g);
    }
  }
  // query slots that see this key: [iv.x, iv.y) and [iv.z, iv.w)
  const int4 iv = key < p.L ? p.kiv[(int64_t)b * p.L + key] : make_int4(0, 0, 0, 0);
  OperandOffsets<D> of;
  of.init(lane);
  TileCopy<D> tc;
  tc.init(w, lane);
  const uint32_t plane_bytes = (uint32_t)p.Lp * D * 2;

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dkacc[db] = zero_f32x16();
    dvacc[db] = zero_f32x16();
  }

  const int64_t tcol = (int64_t)b * p.NT + n;
  const int nnz = p.k_nnz[tcol];
  const int32_t *lst = p.k_list + tcol * p.MT;
  const uint32_t *subs_b = p.sub_class + (int64_t)b * p.MT * p.NT;

  auto issue = [&](uint32_t x, char *nb) {
    const int q0 = (int)(x & 0xFFFFFFu), hj = (int)(x >> 24);
    const int64_t plane = hbase + hj;
    tc.issue(make_rsrc(p.qr + plane * p.Lp * D, plane_bytes), q0, nb, w);
    tc.issue(make_rsrc(p.dor + plane * p.Lp * D, plane_bytes), q0, nb + TB, w);
    if (w == 0) words_load_async(p.lse2 + plane * p.Lp + q0, nb + 2 * TB, lane, 64);
    else if (w == 1) words_load_async(p.dsc + plane * p.Lp + q0, nb + 2 * TB + 256, lane, 64);
  };

  int64_t fnext = 0;
  const int64_t ftotal = (int64_t)nnz * p.group * 2;
  while (fnext < ftotal) {
    __syncthreads();
    if (w == 0) {
      int64_t f = fnext;
      const int c = build_k_stages(lst, subs_b, p.NT, n, p.group, nnz, &f, stages, lane);
      if (lane == 0) {
        sh_count = c;
        sh_next = f;
      }
    }
    __syncthreads();
    const int ns = uniform(sh_count);
    fnext = uniform(sh_next);
    if (ns == 0) continue;
    issue(uniform(stages[0].x), buf0);
    auto stage = [&](int i, const char *buf, char *nxt) {
      wait_all_and_barrier();
      if (i + 1 < ns) issue(uniform(stages[i + 1].x), nxt);
      const uint2 desc = uniform(stages[i]);
      const uint32_t c0 = (desc.y >> (4 * w)) & 3u, c1 = (desc.y >> (4 * w + 2)) & 3u;
      if ((c0 | c1) == 0) return;
      const int q0 = (int)(desc.x & 0xFFFFFFu);
      const char *Qt = buf, *dOt = buf + TB;
      const float *lse2s = reinterpret_cast<const float *>(buf + 2 * TB);
      const float *dscs = reinterpret_cast<const float *>(buf + 2 * TB + 256);
      const uint64_t mq = (range_bits(iv.x, iv.y, q0) | range_bits(iv.z, iv.w, q0)) >> (8 * g);

      // One straight-line body per case (both sub-blocks, masked or not; a
      // single sub-block), laid
      // out as a software pipeline over the present 32-query sub-blocks j:
      //   A(j): S^T = K' Q'^T and dP^T = V dO^T, operands read in the products
      //         before (16-byte reads of the row tiles);
      //   B(j): masking, P and dS (element work), overlapping A(j+1) / C(j-1);
      //   C(j): dV^T += dO^T P^T, dK^T += Q'^T dS^T (transposing reads).
      auto body = [&](auto both, auto msk, int QB0) {
        constexpr int NQ = decltype(both)::value ? 2 : 1;  // sub-blocks QB0 .. QB0 + NQ - 1
        constexpr bool M = decltype(msk)::value;
        f16x8 fa[NQ][2 * NS];
        f32x16 s[NQ], dp[NQ];
        f16x8 pb[NQ][2], dsb[NQ][2];
        auto read_a = [&](int j) {
          const int qb = QB0 + j;
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            fa[j][st] = lds_f16x8(Qt + qb * 32 * RB + of.row8[st]);
            fa[j][NS + st] = lds_f16x8(dOt + qb * 32 * RB + of.row8[st]);
          }
        };
        auto products_a = [&](int j) {
          s[j] = zero_f32x16();
          dp[j] = zero_f32x16();
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            s[j] = mfma32x32x16(fa[j][st], kb_[st], s[j]);
            dp[j] = mfma32x32x16(fa[j][NS + st], vb_[st], dp[j]);
          }
        };
        auto elementwise_b = [&](int j) {
          const int qb = QB0 + j;
          if (M) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) s[j][rr] = mask_select(mq, 32 * qb + 16 * (rr >> 3) + (rr & 7), s[j][rr]);
          }
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int qbase = 32 * qb + 16 * hh + 8 * g;  // rows of registers 8hh .. 8hh+7
            const float4 l0 = *reinterpret_cast<const float4 *>(lse2s + qbase);
            const float4 l1 = *reinterpret_cast<const float4 *>(lse2s + qbase + 4);
            const float4 d0 = *reinterpret_cast<const float4 *>(dscs + qbase);
            const float4 d1 = *reinterpret_cast<const float4 *>(dscs + qbase + 4);
            const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
            const float dvv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int rr = 8 * hh + e;
              const float pv = __builtin_amdgcn_exp2f(fmaf(s[j][rr], fs, -lv[e]));
              pb[j][hh][e] = (_Float16)(pv * pdv);
              dsb[j][hh][e] = (_Float16)(pv * fmaf(dp[j][rr], dss, -dvv[e]));
            }
          }
        };
        auto products_c = [&](int j) {
          const int qb = QB0 + j;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              dvacc[db] = mfma32x32x16(tile_col8<D>(dOt, of, 32 * qb + 16 * hh, db), pb[j][hh], dvacc[db]);
              dkacc[db] = mfma32x32x16(tile_col8<D>(Qt, of, 32 * qb + 16 * hh, db), dsb[j][hh], dkacc[db]);
            }
          }
        };
        read_a(0);
        products_a(0);
        if (NQ == 2) read_a(NQ - 1);
        if (NQ == 2) products_a(NQ - 1);
        elementwise_b(0);
        products_c(0);
        if (NQ == 2) elementwise_b(NQ - 1);
        if (NQ == 2) products_c(NQ - 1);
        // Interleave (one scheduling region): reads of the next phase between
        // the products of the current one, element work between products.
        constexpr int NA = 2 * NS;        // products (and 16-byte reads) of A(j)
        constexpr int NC = 4 * NDB;       // products of C(j); 2 transposing reads each
        constexpr unsigned kMfma = 0x008, kValu = 0x002, kDsRead = 0x100;
        __builtin_amdgcn_sched_group_barrier(kDsRead, NA, 0);
        if (NQ == 2) {
#pragma unroll
          for (int k = 0; k < NA; ++k) {  // A(0) products, A(1) reads
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
          }
#pragma unroll
          for (int k = 0; k < NA; ++k) {  // A(1) products, B(0)
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kValu, 7, 0);
          }
          __builtin_amdgcn_sched_group_barrier(kDsRead, 8, 0);
#pragma unroll
          for (int k = 0; k < NC; ++k) {  // C(0) products, B(1), C reads ahead
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kValu, 7, 0);
            __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
          }
#pragma unroll
          for (int k = 0; k < NC; ++k) {  // C(1) products, C(1) reads ahead
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
          }
        } else {
          __builtin_amdgcn_sched_group_barrier(kMfma, NA, 0);
          __builtin_amdgcn_sched_group_barrier(kDsRead, 8, 0);
#pragma unroll
          for (int k = 0; k < NA; ++k) {
            __builtin_amdgcn_sched_group_barrier(kValu, 6, 0);
            __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
          }
#pragma unroll
          for (int k = 0; k < NC; ++k) {
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
          }
        }
      };
      using T = std::true_type;
      using F = std::false_type;
      // Both sub-blocks always: the 64-bit mask is exact, so an empty one
      // (rare next to a non-empty one) contributes exact zeros.
      body(T{}, T{}, 0);
    };
    for (int i = 0; i < ns; i += 2) {
      stage(i, buf0, buf1);
      if (i + 1 < ns) stage(i + 1, buf1, buf0);
    }
  }

  if (key < p.L) {
    const int tok = p.slot_tok[(int64_t)b * p.L + key];
    const int64_t out = (((int64_t)b * p.L + tok) * p.Hkv + kvh) * D;
    const float2 *cs = p.rope + ((int64_t)b * p.Lp + key) * (D / 2);
    // dK^T in units 2^(eq + edo + ev - kDsShift), dV^T in 2^(kPdvExp + edo)
    const float kscale = ldexpf(p.scale, kDsShift - eq - edo - ev);
    const float vscale = ldexpf(1.0f, -kPdvExp - edo);
#pragma unroll
    for (int db = 0; db < HALF_DB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float lo[4], hi[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = 4 * a + c;
          const float2 rc = cs[acc_dim(db, r, g)];
          const float g1 = kscale * dkacc[db][r], g2 = kscale * dkacc[db + HALF_DB][r];
          lo[c] = g1 * rc.x + g2 * rc.y;
          hi[c] = g2 * rc.x - g1 * rc.y;
        }
        *reinterpret_cast<float4 *>(dk + out + acc_dim(db, 4 * a, g)) = make_float4(lo[0], lo[1], lo[2], lo[3]);
        *reinterpret_cast<float4 *>(dk + out + acc_dim(db + HALF_DB, 4 * a, g)) = make_float4(hi[0], hi[1], hi[2], hi[3]);
      }
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4 *>(dv + out + acc_dim(db, 4 * a, g)) =
            make_float4(vscale * dvacc[db][4 * a], vscale * dvacc[db][4 * a + 1],
                        vscale * dvacc[db][4 * a + 2], vscale * dvacc[db][4 * a + 3]);
    }
  }
}

}  // namespace

void fill_params(const opr_attn_in &in, float scale, const AttnWs &ws, AttnParams *p);

void launch_attn_dq_kernel(const AttnParams &p, int D, float *dq, hipStream_t s);

// ev (optional): events recorded before dK/dV, before dQ and after dQ.
hipError_t launch_attn_bwd_kernels(const opr_attn_in &in, float scale, float *dq, float *dk,
                                   float *dv, const AttnWs &ws, hipStream_t s, hipEvent_t *ev) {
  AttnParams p;
  fill_params(in, scale, ws, &p);
  const unsigned gk = (unsigned)((int64_t)in.B * in.Hkv * p.NT);
  if (ev) (void)hipEventRecord(ev[0], s);
  if (in.D == 64) attn_dkdv_kernel<64><<<gk, 256, 0, s>>>(p, dk, dv);
  else attn_dkdv_kernel<128><<<gk, 256, 0, s>>>(p, dk, dv);
  if (ev) (void)hipEventRecord(ev[1], s);
  launch_attn_dq_kernel(p, in.D, dq, s);
  if (ev) (void)hipEventRecord(ev[2], s);
  return hipGetLastError();
}

}  // namespace opr

// Device-side building blocks of the attention kernels (gfx950 / CDNA4).
//
// Number format.  Every matrix product runs on v_mfma_f32_32x32x16_f16 (fp16
// operands, fp32 accumulation; the same rate as bf16 on gfx950).  fp16 keeps
// 11 significant bits where bf16 keeps 8, which is what lets the summed
// gradients of a GQA group stay within 2e-2 of the exact result.  To keep
// bf16's range, each 64-token block of every staged operand (q and k after
// RoPE, v, dout) is stored as fp16(x * 2^e) with its own power-of-two exponent
// e chosen so that the block's largest magnitude lands in [2^14, 2^15).  The
// kernels fold the exponents back exactly: into the score scale (q, k), and
// into the running units of the fp32 accumulators (v, dout), which are
// rescaled by powers of two when a block with another exponent arrives.
// Probabilities are stored as fp16(p * 2^15) so that small ones keep full
// precision (p <= 1).
//
// MFMA v_mfma_f32_32x32x16_f16 computes C[32x32] += A[32x16] * B[16x32].
// Lane l (g = l / 32, i = l % 32) supplies 8 fp16 of A row i and 8 fp16 of
// B column i for k-group g; any assignment of the 16 k indices to (g, element)
// works as long as A and B use the same one.  The accumulator holds, in lane
// l and register r, C[8*(r/4) + 4*g + r%4][i].
//
// All kernels put the query (forward, dQ) or the key (dK/dV) of a lane on the
// accumulator column, so per-row softmax statistics live in the lane and its
// partner lane l ^ 32.  The row index of a score block runs over keys (or
// queries); the A operand rows are loaded in the permuted order kperm(i) (bits
// 2 and 3 of i swapped), which makes accumulator registers 8h..8h+7 of lane
// group g hold rows 16h + 8g + 0..7: exactly the 8 consecutive k values that
// the next MFMA needs in its B operand.  So probabilities go from the score
// accumulator straight into the next product without any lane exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace opr {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma32x32x16(const f16x8 &a, const f16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Exponent range of the per-block scales; keeps every folded product of up to
// three exponents inside fp32's normal range.
constexpr int kExpMin = -32, kExpMax = 32;
// Probabilities are stored scaled by 2^kPExp; dS by 2^-kDsShift on top of the
// units of v and dout (|v|, |dout| < 2^15 after scaling, so |dP| < 2^37).
constexpr int kPExp = 15;
constexpr int kDsShift = 22;

// A-operand row order of a 32-row block: swap bits 2 and 3.
__device__ __forceinline__ int kperm(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Row of a score block held by accumulator register r of lane group g when
// the A rows were loaded in kperm order.
__device__ __forceinline__ constexpr int acc_row(int r, int g) {
  return 16 * (r >> 3) + 8 * g + (r & 7);
}

// Head-dim index held by accumulator register r of lane group g in 32-row
// block db of an output accumulator (no permutation).
__device__ __forceinline__ constexpr int acc_dim(int db, int r, int g) {
  return 32 * db + 8 * (r >> 2) + 4 * g + (r & 3);
}

__device__ __forceinline__ f16x8 ld_f16x8(const uint16_t *p) {
  return *reinterpret_cast<const f16x8 *>(p);
}

__device__ __forceinline__ f16x8 zero_f16x8() {
  f16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (_Float16)0.0f;
  return z;
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return *reinterpret_cast<uint16_t *>(&h);
}

// Exponent e with max_abs * 2^e in [2^14, 2^15) (0 for an all-zero block),
// clamped to [kExpMin, kExpMax].
__device__ __forceinline__ int block_exponent(float max_abs) {
  if (!(max_abs > 0.0f)) return 0;
  int x;
  frexpf(max_abs, &x);
  return min(kExpMax, max(kExpMin, 15 - x));
}

__device__ __forceinline__ f32x16 zero_f32x16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.0f;
  return z;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return *reinterpret_cast<uint16_t *>(&h);
}

// Token metadata for the mask predicate: conv (-1 for PAD or past L) and
// turn * 8 + type.
struct TokMeta {
  int32_t conv;
  int32_t tt;
};

// Whether query qi may attend to key ki.  With segments stored h, t, r_in,
// r_out inside a turn, every allowed key precedes its query; across turns
// only h and r_in (the history H_<i) are visible; inside the turn the only
// excluded earlier keys are t_i for an r_in_i query and r_in_i for an
// r_out_i query.  (Derived from the four rules; the tile classes computed
// from the same rules tell the kernels where this test is needed.)
__device__ __forceinline__ bool mask_allows(int qi, TokMeta q, int ki, TokMeta k) {
  if (ki > qi || k.conv != q.conv || q.conv < 0) return false;
  const int tq = q.tt >> 3, tk = k.tt >> 3;
  const int yq = q.tt & 7, yk = k.tt & 7;
  if (tk < tq) return (yk & 1) == 0;               // h (0) or r_in (2)
  return !(yq >= 2 && yk == yq - 1);               // r_in vs t, r_out vs r_in
}

__device__ __forceinline__ TokMeta load_meta(const int32_t *conv, const int32_t *turn,
                                             const uint8_t *type, int64_t row_base, int idx,
                                             int L) {
  TokMeta m;
  if (idx < L) {
    m.conv = conv[row_base + idx];
    m.tt = (turn[row_base + idx] << 3) | type[row_base + idx];
  } else {
    m.conv = -1;
    m.tt = 4;
  }
  return m;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Parameters shared by the attention kernels.
struct AttnParams {
  int32_t B, L, Lp, Hq, Hkv, group, MT, NT;
  float scale, scale_log2;
  const int32_t *tok_conv, *tok_turn, *tok_pos;
  const uint8_t *tok_type;
  const uint8_t *tile_class;
  const uint32_t *sub_class;
  const int32_t *q_nnz, *q_list, *k_nnz, *k_list;
  const float2 *rope;                    // [B][Lp][D/2]
  // fp16 bits, scaled per 64-token block (see the number format above)
  const uint16_t *qr, *kr, *vt, *vr, *qt, *kt, *dor, *dot;
  // block exponents [B][H][Lp/64] of q, k, v, dout
  const int32_t *eq, *ek, *ev, *edo;
  const float *delta, *lse2;
};

}  // namespace opr

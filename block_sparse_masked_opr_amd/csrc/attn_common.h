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

// ---------------------------------------------------------------------------
// LDS tiles of 64 rows x D fp16.  A row is D/8 chunks of 16 bytes; chunk c of
// row r is stored in slot c ^ swz(r), so that 16 lanes reading the same chunk
// of 16 different rows (MFMA A operand) or 4 rows x 32 bytes (transposing
// reads) hit distinct banks without padding, and a 1 KB run of LDS is filled
// by one global_load_lds instruction (lane L writes bytes 16L..16L+15).
#define OPR_LDS __attribute__((address_space(3)))
typedef short __attribute__((ext_vector_type(4))) s16x4;

template <int D>
struct Tile {
  static constexpr int NC = D / 8;       // chunks per row
  static constexpr int RB = 2 * D;       // bytes per row
  static constexpr int BYTES = 64 * RB;
  __device__ static __forceinline__ int swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static __forceinline__ int off(int r, int c) { return r * RB + ((c ^ swz(r)) << 4); }
};

// Asynchronous copy of 64 consecutive rows (row stride D elements) into a
// swizzled LDS tile; the four waves of a workgroup share the D/8 instructions.
template <int D>
__device__ __forceinline__ void tile_load_async(const uint16_t *src, char *lds, int w, int lane) {
  constexpr int NC = Tile<D>::NC, RPI = 1024 / Tile<D>::RB;
#pragma unroll
  for (int t = w; t < NC; t += 4) {
    const int r = t * RPI + lane / NC;
    const int c = (lane % NC) ^ Tile<D>::swz(r);
    __builtin_amdgcn_global_load_lds(src + r * D + c * 8, (OPR_LDS void *)(lds + t * 1024), 16, 0, 0);
  }
}

// Asynchronous copy of 64 consecutive 8-byte records (256 B per instruction).
__device__ __forceinline__ void rec8_load_async(const void *src, char *lds, int lane) {
  const char *g = static_cast<const char *>(src);
  __builtin_amdgcn_global_load_lds(g + 4 * lane, (OPR_LDS void *)lds, 4, 0, 0);
  __builtin_amdgcn_global_load_lds(g + 256 + 4 * lane, (OPR_LDS void *)(lds + 256), 4, 0, 0);
}

// Asynchronous copy of 64 consecutive floats.
__device__ __forceinline__ void f32x64_load_async(const float *src, char *lds, int lane) {
  __builtin_amdgcn_global_load_lds(src + lane, (OPR_LDS void *)lds, 4, 0, 0);
}

// Wait for this thread's outstanding memory operations (including the
// asynchronous LDS fills), then for the whole workgroup.
__device__ __forceinline__ void wait_all_and_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

template <int D>
__device__ __forceinline__ f16x8 tile_row8(const char *lds, int r, int c) {
  return *reinterpret_cast<const f16x8 *>(lds + Tile<D>::off(r, c));
}

__device__ __forceinline__ s16x4 ds_read_tr16(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((OPR_LDS s16x4 *)p);
}

// Transposed MFMA operand from a row-major tile X[row][col]: lane l receives
// X[r0 + 0..7][col0 + l % 32] with r0 = rbase + 8 * (l / 32) and
// col0 = cbase; i.e. 8 consecutive rows of its own column.  Built from two
// ds_read_b64_tr_b16: inside each 16-lane group, the lane that points at
// row r0 + j / 4, columns c + 4 * (j % 4) .. +3 supplies column entries so
// that lane i receives rows r0 .. r0 + 3 of column c + i.
template <int D>
__device__ __forceinline__ f16x8 tile_col8(const char *lds, int rbase, int cbase, int lane) {
  const int G = lane >> 4, j = lane & 15;
  const int col = cbase + 16 * (G & 1) + 4 * (j & 3);
  const int r = rbase + 8 * (G >> 1) + (j >> 2);
  const int cb = (col & 7) * 2;
  const s16x4 lo = ds_read_tr16(lds + Tile<D>::off(r, col >> 3) + cb);
  const s16x4 hi = ds_read_tr16(lds + Tile<D>::off(r + 4, col >> 3) + cb);
  typedef short __attribute__((ext_vector_type(8))) s16x8;
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(f16x8, v);
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Remap the linear block id so that each XCD walks a contiguous range
// of work items: neighbouring items share K/V (or Q/dO) tiles in that L2.
__device__ __forceinline__ int64_t xcd_work_item(int64_t nitems) {
  const int64_t per = (nitems + 7) / 8;
  const int64_t bid = blockIdx.x;
  return (bid & 7) * per + (bid >> 3);
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
  const uint16_t *qr, *kr, *vr, *dor;
  // block exponents [B][H][Lp/64] of q, k, v, dout
  const int32_t *eq, *ek, *ev, *edo;
  const int2 *meta;                      // [B][Lp] (conv, turn * 8 + type); conv -1 for PAD / past L
  const float *delta, *lse2;
};

}  // namespace opr

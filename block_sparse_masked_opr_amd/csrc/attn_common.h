// Device-side building blocks of the attention kernels (gfx950 / CDNA4).
//
// Number format.  Every matrix product runs on v_mfma_f32_32x32x16_f16 (fp16
// operands, fp32 accumulation; the same rate as bf16 on gfx950).  fp16 keeps
// 11 significant bits where bf16 keeps 8, which is what lets the summed
// gradients of a GQA group stay within 2e-2 of the exact result.  To keep
// bf16's range, each staged operand (q and k after RoPE, v, dout) is stored
// as fp16(x * 2^e) with a power-of-two exponent e chosen from the largest
// magnitude it covers, so that this lands in [2^14, 2^15): for k and v one
// per (row, kv head) plane (an absmax pre-pass), for q and dout one per row
// of each q head, i.e. per query (found by the threads that convert the
// row), so that no two tokens - and no two conversations - share a scale.
// The kernels fold the exponents back exactly: into the score scale (q, k)
// and into the fixed units of their fp32 accumulators (v, dout), removed in
// the epilogues.
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
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma32x32x16(const f16x8 &a, const f16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Exponent range of the operand scales.  A factor folded from two exponents
// (the score scale 2^-(eq + ek)) stays inside fp32's normal range; sums of
// three (the epilogues' unit removal) are applied with ldexp to the
// accumulated value, never formed as a factor on their own.  A tile or plane
// whose largest magnitude lies in [2^(14 - kExpMax), 2^(15 - kExpMin)) keeps
// the full 11-bit fp16 significand: [2^-46, 2^75) here; below it the values
// keep an absolute precision of 2^-(kExpMax + 24), above it (and for the
// |x| >= 2^(16 - kExpMin) that overflow fp16) the results are not finite.
constexpr int kExpMin = -60, kExpMax = 60;
// dS is stored shifted down by 2^kDsShift on top of the units of dP
// (|v|, |dout| < 2^15 after scaling, so |dP| < 2^37 and |dS| < 2^15).
constexpr int kDsShift = 22;
// The backward kernels recompute P (<= 1) for dV as fp16(P * 2^kPdvExp); the
// stored lse2 and delta carry that factor (lse2 - kPdvExp, delta * 2^-kPdvExp)
// so that the per-element products need no extra scaling.
constexpr int kPdvExp = 15;
// Softmax: the running maximum is only raised when a new score exceeds it by
// more than kMaxSlack (log2 units); probabilities are stored as
// fp16(p * 2^kPExp) with p <= 2^kMaxSlack, i.e. at most 2^15.
constexpr float kMaxSlack = 8.0f;
constexpr int kPExp = 7;
// Slots per tile of the exponent minima of q' and dout (the dK/dV kernel's
// unit search reads these before looking at single rows).
constexpr int kTile = 16;

// A-operand row order of a 32-row block: swap bits 2 and 3.
// bf16 helpers on packed words.  dot2_bf16: a.lo*b.lo + a.hi*b.hi + c in
// float32 (the products of bf16 values are exact in float32).
// absmax8_bf16_bits: the largest |x| of 8 bf16 values as float bits - a bf16
// value is the top half of its float, and for finite values the magnitude
// bits order like the magnitudes, so a packed 16-bit integer max suffices.
typedef __bf16 __attribute__((ext_vector_type(2))) bf16x2;
typedef unsigned short __attribute__((ext_vector_type(2))) u16x2;
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ uint32_t absmax8_bf16_bits(uint4 v) {
  const u16x2 a = __builtin_elementwise_max(__builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu),
                                            __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu));
  const u16x2 b = __builtin_elementwise_max(__builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu),
                                            __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu));
  const u16x2 m = __builtin_elementwise_max(a, b);
  return (uint32_t)(m.x > m.y ? m.x : m.y) << 16;
}

// Wave-uniform values that the compiler cannot prove uniform (the wave index,
// words read from LDS): taking them from lane 0 puts them in scalar registers,
// so buffer offsets and branches on them need no per-lane loops.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ uint2 uniform(uint2 x) { return make_uint2(uniform(x.x), uniform(x.y)); }
__device__ __forceinline__ uint4 uniform(uint4 x) {
  return make_uint4(uniform(x.x), uniform(x.y), uniform(x.z), uniform(x.w));
}
__device__ __forceinline__ int64_t uniform(int64_t x) {
  const uint64_t u = (uint64_t)x;
  return (int64_t)(((uint64_t)uniform((uint32_t)(u >> 32)) << 32) | uniform((uint32_t)u));
}

// max(x[l], x[l ^ 32]) in every lane l: the two halves of the wave swapped
// with one v_permlane32_swap (VALU, no LDS round trip).  The builtin returns
// the lower halves of both operands in one register and the upper halves in
// the other, so each lane sees both values of its pair.
__device__ __forceinline__ float pair_max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

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

__device__ __forceinline__ f32x16 zero_f32x16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.0f;
  return z;
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return *reinterpret_cast<uint16_t *>(&h);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return *reinterpret_cast<uint16_t *>(&h);
}

// RoPE (rotate-half) of one rotation pair (x1, x2) = (x_j, x_{j+D/2}) by the
// angle's (cos, sin): (x1 cos - x2 sin, x2 cos + x1 sin), with explicit fused
// multiply-adds, so that every kernel that rotates q or k rounds the same way.
__device__ __forceinline__ void rope_pair(float x1, float x2, float2 cs, float &lo, float &hi) {
  lo = fmaf(x1, cs.x, -(x2 * cs.y));
  hi = fmaf(x2, cs.x, x1 * cs.y);
}

// Exponent e with max_abs * 2^e in [2^14, 2^15) (0 for an all-zero plane),
// clamped to [kExpMin, kExpMax].  max_abs is stored as the bits of a
// non-negative float (so that atomicMax on the bits orders them).
__device__ __forceinline__ int plane_exponent(uint32_t max_abs_bits) {
  const float m = __uint_as_float(max_abs_bits);
  if (!(m > 0.0f)) return 0;
  int x;
  frexpf(m, &x);
  return min(kExpMax, max(kExpMin, 15 - x));
}

// Sum of the 8 fp16 values of v (fp32 accumulation).
__device__ __forceinline__ float sum_f16x8(const f16x8 &v, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const f16x2 pr = {v[e], v[e + 1]};
    acc = __builtin_amdgcn_fdot2(pr, one, acc, false);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Mask bits.  For a query (or key) the allowed partners form a few intervals
// of the packed row; range_bits gives the bits of [a, b) inside the 64-row
// window starting at base.
__device__ __forceinline__ uint64_t low_bits(int n) {  // bits [0, n), n in [0, 64]
  return n >= 64 ? ~0ull : ((1ull << n) - 1ull);
}

__device__ __forceinline__ uint64_t range_bits(int a, int b, int base) {
  return low_bits(max(0, min(64, b - base))) & ~low_bits(max(0, min(64, a - base)));
}

// -inf where bit `pos` of the 64-bit mask m is clear, x otherwise.
__device__ __forceinline__ float mask_select(uint64_t m, int pos, float x) {
  const uint32_t w = pos < 32 ? (uint32_t)m : (uint32_t)(m >> 32);
  const int32_t full = __builtin_amdgcn_sbfe((int32_t)w, pos & 31, 1);  // 0 or -1
  return __uint_as_float((__float_as_uint(x) & (uint32_t)full) | (0xff800000u & ~(uint32_t)full));
}

// ---------------------------------------------------------------------------
// LDS tiles of 64 rows x D fp16.  A row is D/8 chunks of 16 bytes; chunk c of
// row r is stored in slot c ^ swz(r).  The LDS has 64 four-byte banks (256
// bytes per clock); a 16-byte read is served 16 lanes at a time and the
// transposing 8-byte read 32 lanes at a time, so conflict-free means:
//  - 16-byte reads: one chunk of the 16 rows kperm(0..15) (+16k) per group -
//    their 16 slots must fall in distinct 16-byte bank quads;
//  - transposing reads: 32 bytes of each of rows 4a..4a+3 (chunks 4q..4q+3
//    for D = 128) per group - the 4 rows must land in distinct 64-byte quarters.
// D = 128 (256-byte rows): swz(r) = 4(r mod 4) + (r div 4) mod 4.
// D = 64 (128-byte rows, two rows per bank cycle): swz(r) = 4((r div 2) mod 2)
// + (r div 4) mod 4.  Both were checked with the LDS bank-conflict counter.
// No padding is needed, and a 1 KB run of LDS is filled by one asynchronous
// copy instruction (lane L writes bytes 16L..16L+15).
#define OPR_LDS __attribute__((address_space(3)))
typedef short __attribute__((ext_vector_type(4))) s16x4;
typedef short __attribute__((ext_vector_type(8))) s16x8;

template <int D>
struct Tile {
  static constexpr int NC = D / 8;       // chunks per row
  static constexpr int RB = 2 * D;       // bytes per row
  static constexpr int BYTES = 64 * RB;
  __device__ static __forceinline__ int swz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  __device__ static __forceinline__ int off(int r, int c) { return r * RB + ((c ^ swz(r)) << 4); }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Asynchronous copies of ROWS-row tiles (64 or 32) from a plane [rows][D]
// fp16 (buffer resource over the plane) into swizzled LDS tiles.  Each of the
// NW waves issues NI of the tile's one-kilobyte instructions; the per-lane
// byte offsets inside the block are fixed, the first row goes in the scalar
// offset.
template <int D, int NW = 4, int ROWS = 64>
struct TileCopy {
  static constexpr int NI = ROWS * Tile<D>::RB / 1024 / NW;
  static_assert(NI >= 1 && NI * NW * 1024 == ROWS * Tile<D>::RB, "waves must split the tile's instructions evenly");
  int voff[NI];
  __device__ __forceinline__ void init(int w, int lane) {
    constexpr int NC = Tile<D>::NC, RPI = 1024 / Tile<D>::RB;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = w + NW * i;
      const int r = t * RPI + lane / NC;
      const int c = (lane % NC) ^ Tile<D>::swz(r);
      voff[i] = (r * D + c * 8) * 2;
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int row0, char *lds, int w) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (OPR_LDS void *)(lds + (w + NW * i) * 1024), 16, voff[i],
                                               row0 * D * 2, 0, 0);
  }
};

// Scheduling of a run of N matrix instructions that each take one operand
// from READS LDS reads (the scheduling region ends here): the reads of the
// first AHEAD products go first, then every product is followed by the reads
// of the product AHEAD places later, so that LDS latency hides behind the
// matrix core instead of one wait per product.
template <int N, int AHEAD, int READS = 2>
__device__ __forceinline__ void sched_lds_reads_ahead() {
  constexpr int kMfma = 0x008, kDsRead = 0x100;  // instruction classes of the scheduler
  __builtin_amdgcn_sched_group_barrier(kDsRead, READS * AHEAD, 0);
#pragma unroll
  for (int j = 0; j < N - AHEAD; ++j) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, READS, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, AHEAD, 0);
}

// Wait until at most N of this wave's vector memory operations (the newest:
// asynchronous LDS fills of later stages) are outstanding and all its LDS
// operations are done, then for the whole workgroup.  The barrier carries no
// fence (a fenced barrier would also wait for the fills still streaming into
// other buffers); the empty asm keeps the compiler from moving memory
// operations across it.
template <int N>
__device__ __forceinline__ void wait_older_copies_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));  // vmcnt(N) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for this thread's outstanding memory operations (including the
// asynchronous LDS fills), then for the whole workgroup.
__device__ __forceinline__ void wait_all_and_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

__device__ __forceinline__ f16x8 lds_f16x8(const char *p) {
  return *reinterpret_cast<const f16x8 *>(p);
}

__device__ __forceinline__ s16x4 ds_read_tr16(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((OPR_LDS s16x4 *)p);
}

// Per-lane LDS byte offsets of the two operand patterns, fixed for a kernel:
//  row8[st]: 8 elements (k-step st, lane group g) of row kperm(li) - the A
//            operand of a product whose k runs along the head dim; the rows
//            32b + kperm(li) of block b add 32 * RB.
//  col8[db][s]: the transposing reads for an A operand whose k runs along the
//            rows: inside each 16-lane group, the lane that points at row
//            rb + 8g + j/4 (+4 for s = 1), columns 32db + 16(G%2) + 4(j%4)..+3
//            supplies entries so that lane i receives rows rb + 8g + 0..3
//            (4..7) of column 32db + li; rb (a multiple of 16) adds rb * RB.
template <int D>
struct OperandOffsets {
  static constexpr int NS = D / 16, NDB = D / 32;
  int row8[NS];
  int col8[NDB][2];
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 5, li = lane & 31, G = lane >> 4, j = lane & 15;
#pragma unroll
    for (int st = 0; st < NS; ++st) row8[st] = Tile<D>::off(kperm(li), 2 * st + g);
    const int col = 16 * (G & 1) + 4 * (j & 3);
    const int r = 8 * (G >> 1) + (j >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        col8[db][s] = Tile<D>::off(r + 4 * s, (32 * db + col) >> 3) + ((col & 7) << 1);
  }
};

// The transposed operand X[rb + 8g + e][32db + li], e = 0..7, of a tile.
template <int D>
__device__ __forceinline__ f16x8 tile_col8(const char *lds, const OperandOffsets<D> &of, int rb, int db) {
  const s16x4 lo = ds_read_tr16(lds + rb * Tile<D>::RB + of.col8[db][0]);
  const s16x4 hi = ds_read_tr16(lds + rb * Tile<D>::RB + of.col8[db][1]);
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(f16x8, v);
}

// Work order.  Workgroups are dispatched round-robin over the 8 XCDs (block
// b goes to XCD b mod 8, each XCD with its own L2), and a kernel lasts as
// long as its slowest CU.  The work items are therefore handed out longest
// first: q_order lists the q-tile rows (b*MT + m) and k_items the dK/dV
// items (a k-tile column b*NT + n, or one part of a long column's stage
// range) by decreasing number of stages, and consecutive ranks go to
// consecutive XCDs.
//
// dK/dV: rank R = block id; item (k_items[R / Hkv], kv head R % Hkv).
// Forward and dQ: super-rank R = (i / group) * 8 + x for block 8i + x, head
// j = i % group of kv head R % Hkv of row k = q_order[R / Hkv]: the q heads
// of one kv group sit on one XCD back to back and share its K/V tiles in L2.
struct QItem {
  int b, m, kvh, j;
  bool valid;
};

__device__ __forceinline__ QItem q_work_item(const int32_t *q_order, int MT, int Hkv, int group, int64_t n_rows) {
  const int64_t bid = blockIdx.x, i = bid >> 3;
  const int64_t R = (i / group) * 8 + (bid & 7);
  QItem it;
  it.valid = R < n_rows * Hkv;
  if (!it.valid) return it;
  const int32_t row = q_order[R / Hkv];
  it.kvh = (int)(R % Hkv);
  it.j = (int)(i % group);
  it.b = row / MT;
  it.m = row - it.b * MT;
  return it;
}

// Blocks of the forward / dQ grid for n_rows q-tile rows.
inline int64_t q_grid(int64_t n_rows, int Hkv, int group) {
  return 8 * group * ((n_rows * Hkv + 7) / 8);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Checked builds (-DOPR_DEBUG): the attention kernels test the invariants
// their indexing relies on (tile-list entries inside the tile grid, the
// token of a live slot inside its row, dK/dV work items inside their
// tables); a violated one sets its bit in a device word (dbg) and the access
// it guards is skipped, so the kernel still ends normally.  Bits:
// 1 q-tile list entry, 2 k-tile list entry, 4 token of a slot, 8 dK/dV item.
// Release builds compile no test (OPR_DCHECK is true).
#ifdef OPR_DEBUG
#define OPR_DCHECK(dbg, cond, bit) ((cond) ? true : (atomicOr((dbg), (bit)), false))
#else
#define OPR_DCHECK(dbg, cond, bit) true
#endif
constexpr uint32_t kDbgQList = 1u, kDbgKList = 2u, kDbgToken = 4u, kDbgItem = 8u;

// Host: the current device's error word of a checked build (opr_api.cpp;
// opr_debug_errors reads it); null in release builds or if its address cannot
// be found.
uint32_t *debug_word();

// Parameters shared by the attention kernels.
struct AttnParams {
  int32_t B, L, Lp, Hq, Hkv, group, MT, NT;
  float scale, scale_log2;
  const uint8_t *tile_class;
  const uint32_t *sub_class;
  const int32_t *q_nnz, *q_list, *k_nnz, *k_list;
  // Everything is indexed by slot (attention order) except the outputs,
  // which are written at token slot_tok[s].
  const int32_t *q_order;      // [B*MT] q-tile rows, most stages first
  const int4 *k_items;         // dK/dV items (column, part, parts, partial slot), most stages first
  const int4 *k_split;         // columns cut into parts: (column, first partial slot, parts, 0)
  const int32_t *k_counts;     // [0] items, [1] cut columns
  float *kpart;                // partials of parts 1.. : [slot * Hkv + kv head][128][D], dK then dV
  int32_t *kunits;             // [rank][4 key blocks][q', dout]: the dK/dV units of each work item
  const int32_t *slot_tok;     // [B][L] token at each slot
  const int4 *qiv;             // [B][L] key slots a query slot sees: [x, y) and [z, w)
  const int4 *kiv;             // [B][L] query slots that see a key slot: [x, y) and [z, w)
  const float2 *rope;          // [B][Lp][D/2] (cos, sin)
  // fp16 bits [B][H][Lp][D]: k' and v with one power-of-two scale per
  // (row, kv head) plane, q' and dout with one per 16-slot tile of each
  // (row, q head).  The dQ kernel writes dor; the dK/dV kernel reads it.
  uint16_t *qr;                // written by the forward kernel (or the q pack)
  const uint16_t *kr, *vr;
  uint16_t *dor;
  // plane maxima (float bits) [B][Hkv] of k', v
  const uint32_t *mk, *mv;
  // row exponents [B][Hq][Lp] of q' and of dout (edoq, written by dQ), and
  // their minima over each kTile-slot tile [B][Hq][MTS]
  int32_t *eqq, *eqt;
  int32_t *edoq, *edot;
  int32_t MTS;                 // tiles per row: Lp / kTile
  // [B][Hq][Lp], written by the dQ kernel for dK/dV (units in attn_bwd.hip;
  // lse2 is +inf where no key)
  float *dsc, *lse2, *fsq;
  // inputs in token order: q (forward), o, dout bf16 [B][L][Hq][D], lse
  // [B][Hq][L] (backward)
  const uint16_t *q_in, *o_in, *dout_in;
  const float *lse_in;
  uint32_t *dbg;               // checked builds: the device's error word (else null)
};

}  // namespace opr

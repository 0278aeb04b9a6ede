// Internal declarations shared by the host entry points (opr_api.cpp) and the
// kernel launchers (*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "opr.h"

namespace opr {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Carves consecutive, 256-byte aligned pieces out of a workspace.
struct Carver {
  char *base;
  size_t off = 0;
  explicit Carver(void *p) : base(static_cast<char *>(p)) {}
  template <class T>
  T *take(size_t count) {
    T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
};

// ---------------------------------------------------------------- GEMM
// Row-major C[M][N] = op(A) op(B) with hipBLASLt, bf16 operands, fp32
// accumulation, C bf16 or fp32 (c_f32); A is stored [M][K] (trans_a = false)
// or [K][M], B [K][N] (trans_b = false) or [N][K].  ws: hipBLASLt scratch.
// Returns false if a hipBLASLt call fails.  (gemm.cpp)
bool gemm_bf16(bool trans_a, bool trans_b, int64_t M, int64_t N, int64_t K, const void *A, const void *B, void *C,
               bool c_f32, void *ws, size_t ws_bytes, hipStream_t s);

// ---------------------------------------------------------------- layout
// Tokens per workgroup of the k/v plane maxima (partial maxima per block).
constexpr int kAbsSlots = 256;

struct LayoutWs {
  int32_t *cpr;         // [B]   convs per row (copied from the host)
  int32_t *tpc;         // [C]   turns per conversation (copied)
  int4 *turns;          // [T]   (h, t, r_in, r_out) (copied)
  // The caller's host arrays at device addresses when they are page-locked
  // and mapped (layout_prep copies them into cpr, tpc, turns itself), else
  // null (they were copied with hipMemcpyAsync).
  const int32_t *src_cpr, *src_tpc, *src_turns;
  int32_t *row_conv0;   // [B+1] first conversation of each row
  int32_t *conv_turn0;  // [C+1] first turn of each conversation
  int32_t *tok_g;       // [T+1] tokens before each turn, counted over all rows
  int32_t *pos_g;       // [T+1] sum of (h + r_in) before each turn, over all rows
  int32_t *conv_row;    // [C]   row of each conversation
  int32_t *turn_conv;   // [T]   conversation of each turn
  int32_t *row_turn0;   // [B+1] first turn of each row
  int32_t *gturn;       // [B][L] turn of each token (-1 for PAD)
};

// Carves the layout workspace; with ws == nullptr only the size is computed.
size_t carve_layout_ws(void *ws, int32_t B, int32_t L, int32_t C, int32_t T, LayoutWs *out);

hipError_t launch_build_layout(int32_t B, int32_t L, int32_t block_q, int32_t block_k,
                               int32_t C, int32_t T, const LayoutWs &ws, const opr_layout &out,
                               hipStream_t stream);

// ---------------------------------------------------------------- attention
// Extra dK/dV work items from cutting long columns, summed over the kv heads:
// the cap on a part's stages is at least total * Hkv / kSplitSlots, so the
// parts beyond the first number fewer than kSplitSlots / Hkv.
constexpr int kSplitSlots = 256;

struct AttnWs {
  int32_t Lp;           // L rounded up to OPR_ATTN_BLOCK
  // everything below is in slot (attention) order
  float2 *rope;         // [B][Lp][D/2] (cos, sin) at each slot's position id
  // fp16 copies [B][H][Lp][D], zero past L: k and v with one power-of-two
  // scale per (row, kv head) plane, q and dout with one per row (slot and
  // q head)
  uint16_t *qr;         // q after RoPE
  uint16_t *kr;         // k after RoPE
  uint16_t *vr;         // v
  uint16_t *dor;        // dout, written by the dQ kernel             (bwd)
  // plane maxima (float bits): mk [B][Hkv], mv [B][Hkv], contiguous from pmax
  // (n_pmax words); their partial maxima over kAbsSlots-token blocks,
  // [2 (k, v)][B][Hkv][n_part] (the k/v packs reduce them)
  uint32_t *pmax, *mk, *mv;
  int32_t n_pmax;
  uint32_t *pmax_part;
  int32_t n_part;
  // row exponents [B][Hq][Lp] of q (eqq) and dout (edoq), and their minima
  // over each 16-slot tile [B][Hq][Lp/16] (eqt, edot)
  int32_t *eqq, *eqt;
  int32_t *edoq, *edot; //                                        (bwd)
  int32_t *q_order;     // [B*MT] q-tile rows, most stages first
  int32_t *order_cost;  // [B*MT + B*NT] stage counts of the rows and columns
  // dK/dV work items (column, part j, parts s, partial slot or -1), the
  // longest first; a column longer than the cap is cut into s parts of its
  // stage range (kSplitSlots bounds the extra parts, times Hkv)
  int4 *k_items;        // [B*NT + kSplitSlots] sorted
  int4 *k_raw;          // [B*NT + kSplitSlots] unsorted
  int4 *k_split;        // [kSplitSlots] cut columns: (column, first slot, s, 0)
  int32_t *k_counts;    // [4]: items, cut columns
  float *kpart;         // [kSplitSlots][128][D] dK then dV partials of parts 1..s-1 (bwd)
  float *dsc;           // [B][Hq][Lp] rowsum(dout * o) in dK/dV units (bwd)
  float *lse2;          // [B][Hq][Lp] log2-domain lse in dK/dV units, +inf where no key (bwd)
  float *fsq;           // [B][Hq][Lp] score factor of each query row in dK/dV (bwd)
  int32_t *kunits;      // [(B*NT + kSplitSlots/Hkv + 1) * Hkv][8] units of the dK/dV items (bwd)
};

size_t carve_attn_ws(void *ws, const opr_attn_in &in, int is_bwd, AttnWs *out);

hipError_t launch_attn_fwd(const opr_attn_in &in, float scale, void *o, float *lse,
                           const AttnWs &ws, hipStream_t stream);

hipError_t launch_attn_bwd(const opr_attn_in &in, float scale, const void *o, const float *lse,
                           const void *dout, float *dq, float *dk, float *dv, const AttnWs &ws,
                           hipStream_t stream);

}  // namespace opr

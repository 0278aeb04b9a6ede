// Host entry points of libopr: argument validation (before any HIP call),
// workspace carving and kernel launch order.  See include/opr.h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "attn_common.h"
#include "opr_internal.h"

namespace opr {

// launchers defined in the .hip files
void launch_rope_order(const opr_attn_in &in, const AttnWs &ws, hipStream_t s);
void launch_pack_q(const opr_attn_in &in, const AttnWs &ws, hipStream_t s);
void launch_pack_kv(const opr_attn_in &in, const AttnWs &ws, hipStream_t s);
hipError_t launch_attn_fwd_kernel(const opr_attn_in &in, float scale, void *o, float *lse,
                                  const AttnWs &ws, hipStream_t s);
hipError_t launch_attn_bwd_kernels(const opr_attn_in &in, float scale, const void *o, const float *lse,
                                   const void *dout, float *dq, float *dk, float *dv, const AttnWs &ws,
                                   hipStream_t s, hipEvent_t *ev);
size_t token_ce_ws_bytes(int64_t n_rows, int32_t V);
int block_norm_grid(int D, int64_t T, int NH);
hipError_t launch_qk_norm_fwd(int D, int64_t T, int Hq, int Hkv, float eps, const void *qkv, const float *gq,
                              const float *gk, void *qn, void *kn, void *v, hipStream_t s);
hipError_t launch_qk_norm_bwd(int D, int64_t T, int Hq, int Hkv, float eps, const void *qkv, const float *gq,
                              const float *gk, const float *dqn, const float *dkn, const float *dv, void *dqkv,
                              float *part, float *dgq, float *dgk, hipStream_t s);
hipError_t launch_token_ce(int32_t B, int32_t L, int32_t F, int32_t V, const void *o, const void *w,
                           const int32_t *labels, const uint8_t *tok_type, float grad_scale, float *loss,
                           void *dout, void *workspace, hipStream_t s);

static bool valid_block(int32_t b) { return b == 32 || b == 64 || b == 128; }

// The runs of slots, the attention tensors and the per-token rows are read
// and written as 16-byte vectors; workspaces are carved in 256-byte pieces
// that the kernels read with 16-byte (int4, float4) accesses.
static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool aligned256(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

size_t carve_attn_ws(void *p, const opr_attn_in &in, int is_bwd, AttnWs *o) {
  Carver cv(p);
  AttnWs w;
  memset(&w, 0, sizeof(w));
  const int64_t Lp = (int64_t)(in.L + OPR_ATTN_BLOCK - 1) / OPR_ATTN_BLOCK * OPR_ATTN_BLOCK;
  const size_t qn = (size_t)in.B * in.Hq * Lp * in.D;
  const size_t kn = (size_t)in.B * in.Hkv * Lp * in.D;
  w.Lp = (int32_t)Lp;
  w.rope = cv.take<float2>((size_t)in.B * Lp * (in.D / 2));
  w.qr = cv.take<uint16_t>(qn);
  w.kr = cv.take<uint16_t>(kn);
  w.vr = cv.take<uint16_t>(kn);
  w.n_pmax = 2 * in.B * in.Hkv;
  w.pmax = cv.take<uint32_t>((size_t)w.n_pmax);
  if (w.pmax) {
    w.mk = w.pmax;
    w.mv = w.mk + (size_t)in.B * in.Hkv;
  }
  w.n_part = (in.L + kAbsSlots - 1) / kAbsSlots;
  w.pmax_part = cv.take<uint32_t>((size_t)2 * in.B * in.Hkv * w.n_part);
  const size_t etiles = (size_t)in.B * in.Hq * (Lp / kTile);
  const size_t erows = (size_t)in.B * in.Hq * Lp;
  w.eqq = cv.take<int32_t>(erows);
  w.eqt = cv.take<int32_t>(etiles);
  const size_t tiles = (size_t)in.B * (Lp / OPR_ATTN_BLOCK);
  w.q_order = cv.take<int32_t>(tiles);
  w.order_cost = cv.take<int32_t>(2 * tiles);
  w.k_items = cv.take<int4>(tiles + kSplitSlots);
  w.k_raw = cv.take<int4>(tiles + kSplitSlots);
  w.k_split = cv.take<int4>(kSplitSlots);
  w.k_counts = cv.take<int32_t>(4);
  // everything above is the forward state; the backward part follows
  if (is_bwd) {
    w.dor = cv.take<uint16_t>(qn);
    w.edoq = cv.take<int32_t>(erows);
    w.edot = cv.take<int32_t>(etiles);
    w.dsc = cv.take<float>(erows);
    w.lse2 = cv.take<float>(erows);
    w.fsq = cv.take<float>(erows);
    w.kunits = cv.take<int32_t>(((size_t)in.B * (Lp / OPR_ATTN_BLOCK) + kSplitSlots / in.Hkv + 1) * in.Hkv * 8);
    w.kpart = cv.take<float>((size_t)kSplitSlots * OPR_ATTN_BLOCK * in.D * 2);
  }
  if (o) *o = w;
  return cv.off;
}

void fill_params(const opr_attn_in &in, float scale, const AttnWs &ws, AttnParams *p) {
  p->B = in.B;
  p->L = in.L;
  p->Lp = ws.Lp;
  p->Hq = in.Hq;
  p->Hkv = in.Hkv;
  p->group = in.Hq / in.Hkv;
  p->MT = ws.Lp / OPR_ATTN_BLOCK;
  p->NT = ws.Lp / OPR_ATTN_BLOCK;
  p->scale = scale;
  p->scale_log2 = scale * kLog2e;
  p->tile_class = in.layout.tile_class;
  p->sub_class = in.layout.sub_class;
  p->q_nnz = in.layout.q_nnz;
  p->q_list = in.layout.q_list;
  p->k_nnz = in.layout.k_nnz;
  p->k_list = in.layout.k_list;
  p->rope = ws.rope;
  p->qr = ws.qr;
  p->kr = ws.kr;
  p->vr = ws.vr;
  p->dor = ws.dor;
  p->mk = ws.mk;
  p->mv = ws.mv;
  p->eqq = ws.eqq;
  p->eqt = ws.eqt;
  p->edoq = ws.edoq;
  p->edot = ws.edot;
  p->MTS = ws.Lp / kTile;
  p->q_order = ws.q_order;
  p->k_items = ws.k_items;
  p->k_split = ws.k_split;
  p->k_counts = ws.k_counts;
  p->kpart = ws.kpart;
  p->slot_tok = in.layout.slot_tok;
  p->qiv = reinterpret_cast<const int4 *>(in.layout.slot_qiv);
  p->kiv = reinterpret_cast<const int4 *>(in.layout.slot_kiv);
  p->dsc = ws.dsc;
  p->lse2 = ws.lse2;
  p->fsq = ws.fsq;
  p->kunits = ws.kunits;
  p->q_in = nullptr;
  p->o_in = nullptr;
  p->dout_in = nullptr;
  p->lse_in = nullptr;
  p->dbg = debug_word();
}

// Shape checks shared by the attention entry points and the size query.
static opr_status check_attn_shape(int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D) {
  if (B < 1 || L < 1 || Hq < 1 || Hkv < 1 || D < 1) return OPR_E_INVALID;
  if (Hq % Hkv != 0) return OPR_E_INVALID;
  if (Hq / Hkv > 255) return OPR_E_UNSUPPORTED;  // head-in-group index of a dK/dV stage is 8 bits
  if (D != 64 && D != 128) return OPR_E_UNSUPPORTED;
  if (B > 65535 || Hq > 1024) return OPR_E_UNSUPPORTED;  // grid dimensions, per-head LDS tables
  const int64_t Lp = ((int64_t)L + OPR_ATTN_BLOCK - 1) / OPR_ATTN_BLOCK * OPR_ATTN_BLOCK;
  // every element index of the largest tensor must fit in int64 with room;
  // row indices (b*L + t) are kept in int32 by the layout
  if ((int64_t)B * Lp >= (int64_t)1 << 31) return OPR_E_UNSUPPORTED;
  if (Lp / OPR_ATTN_BLOCK > 65535) return OPR_E_UNSUPPORTED;
  return OPR_OK;
}

static opr_status check_attn_in(const opr_attn_in *in) {
  if (!in) return OPR_E_INVALID;
  const opr_status st = check_attn_shape(in->B, in->L, in->Hq, in->Hkv, in->D);
  if (st != OPR_OK) return st;
  if (!in->q || !in->k || !in->v) return OPR_E_INVALID;
  if (!aligned16(in->q) || !aligned16(in->k) || !aligned16(in->v)) return OPR_E_INVALID;
  const opr_layout &l = in->layout;
  if (!l.tok_pos || !l.slot_tok || !l.slot_qiv || !l.slot_kiv || !l.tile_class || !l.sub_class ||
      !l.q_nnz || !l.q_list || !l.k_nnz || !l.k_list)
    return OPR_E_INVALID;
  if (l.order != OPR_ORDER_ATTENTION) return OPR_E_INVALID;
  if (!aligned16(l.slot_qiv) || !aligned16(l.slot_kiv)) return OPR_E_INVALID;
  if (!(in->rope_theta > 0.0) || !isfinite(in->rope_theta)) return OPR_E_INVALID;
  if (!(in->softmax_scale >= 0.0f) || !isfinite(in->softmax_scale)) return OPR_E_INVALID;
  if (in->block_q != OPR_ATTN_BLOCK || in->block_k != OPR_ATTN_BLOCK) return OPR_E_UNSUPPORTED;
  return OPR_OK;
}

static float effective_scale(const opr_attn_in *in) {
  return in->softmax_scale > 0.0f ? in->softmax_scale : 1.0f / sqrtf((float)in->D);
}

static void mark(const opr_attn_in *in, int i, hipStream_t s) {
  if (in->timing_events) hipEventRecord(in->timing_events[i], s);
}

// RoPE table, plane maxima of k and v, fp16 copies of k and v in slot order
// and the work order: the forward state at the start of the workspace.  The
// forward kernel converts q itself (and leaves q' there); a backward that does
// not reuse the forward's workspace packs q here (pack_q).
static void forward_prologue(const opr_attn_in &in, const AttnWs &ws, hipStream_t stream, bool pack_q) {
  launch_rope_order(in, ws, stream);
  if (pack_q) launch_pack_q(in, ws, stream);
  launch_pack_kv(in, ws, stream);
}

static opr_status hip_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? OPR_OK : OPR_E_HIP;
}

// ---------------------------------------------------------------- attention block
constexpr size_t kGemmWs = (size_t)64 << 20;  // hipBLASLt scratch

// Block workspace: the hipBLASLt scratch, the attention's q, k, v and the
// attention's own workspace come first, at the same offsets for the forward
// and the backward sizes, so that a backward given the forward's workspace can
// reuse the normalised q, k, v and the attention's forward state.
struct BlockWs {
  void *gemm;                 // hipBLASLt scratch
  uint16_t *qn, *kn, *v;      // the attention's q, k, v: bf16 [T][H][D]
  void *attn;                 // the attention's own workspace (forward state first)
  size_t attn_bytes;
  uint16_t *dout;             // d(o), bf16 [T][Hq][D]              (bwd)
  float *dqn, *dkn, *dv;      // the attention's gradients, fp32    (bwd)
  uint16_t *dqkv;             // bf16 [T][Hq + 2 Hkv][D]            (bwd)
  float *part;                // [norm grid][2][D] partial dg sums  (bwd)
};

static size_t carve_block_ws(void *p, const opr_block_in &in, int is_bwd, BlockWs *o) {
  Carver cv(p);
  BlockWs w;
  memset(&w, 0, sizeof(w));
  const int64_t T = (int64_t)in.B * in.L;
  const int NH = in.Hq + 2 * in.Hkv;
  w.gemm = cv.take<char>(kGemmWs);
  w.qn = cv.take<uint16_t>((size_t)(T * in.Hq * in.D));
  w.kn = cv.take<uint16_t>((size_t)(T * in.Hkv * in.D));
  w.v = cv.take<uint16_t>((size_t)(T * in.Hkv * in.D));
  w.attn_bytes = opr_attn_workspace_size(in.B, in.L, in.Hq, in.Hkv, in.D, is_bwd);
  w.attn = cv.take<char>(w.attn_bytes);
  if (is_bwd) {
    w.dout = cv.take<uint16_t>((size_t)(T * in.Hq * in.D));
    w.dqn = cv.take<float>((size_t)(T * in.Hq * in.D));
    w.dkn = cv.take<float>((size_t)(T * in.Hkv * in.D));
    w.dv = cv.take<float>((size_t)(T * in.Hkv * in.D));
    w.dqkv = cv.take<uint16_t>((size_t)(T * NH * in.D));
    w.part = cv.take<float>((size_t)block_norm_grid(in.D, T, NH) * 2 * in.D);
  }
  if (o) *o = w;
  return cv.off;
}

static opr_attn_in attn_in_of(const opr_block_in &b, const void *q, const void *k, const void *v) {
  opr_attn_in a;
  memset(&a, 0, sizeof(a));
  a.B = b.B; a.L = b.L; a.Hq = b.Hq; a.Hkv = b.Hkv; a.D = b.D;
  a.softmax_scale = b.softmax_scale;
  a.rope_theta = b.rope_theta;
  a.q = q; a.k = k; a.v = v;
  a.layout = b.layout;
  a.block_q = b.block_q;
  a.block_k = b.block_k;
  return a;
}

static opr_status check_block_shape(int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t d_model) {
  const opr_status st = check_attn_shape(B, L, Hq, Hkv, D);
  if (st != OPR_OK) return st;
  if (d_model < 64 || d_model % 64 != 0) return OPR_E_INVALID;
  if (d_model > (1 << 16) || (Hq + 2 * Hkv) * D > (1 << 18)) return OPR_E_UNSUPPORTED;
  return OPR_OK;
}

static opr_status check_block_in(const opr_block_in *in) {
  if (!in) return OPR_E_INVALID;
  opr_status st = check_block_shape(in->B, in->L, in->Hq, in->Hkv, in->D, in->d_model);
  if (st != OPR_OK) return st;
  if (!in->x || !in->w_qkv || !in->w_o || !in->g_q || !in->g_k) return OPR_E_INVALID;
  if (!aligned16(in->x) || !aligned16(in->w_qkv) || !aligned16(in->w_o)) return OPR_E_INVALID;
  if (!(in->norm_eps > 0.0f) || !isfinite(in->norm_eps)) return OPR_E_INVALID;
  // the attention's own checks, with the block input standing in for q, k, v
  const opr_attn_in a = attn_in_of(*in, in->x, in->x, in->x);
  return check_attn_in(&a);
}

static void bmark(const opr_block_in *in, int i, hipStream_t s) {
  if (in->timing_events) hipEventRecord(in->timing_events[i], s);
}

// Arguments of the layout builders, validated on the host before any HIP
// call; on success *C and *T are the conversation and turn counts.
static opr_status check_layout_args(int32_t B, int32_t L, int32_t block_q, int32_t block_k,
                                    const int32_t *convs_per_row, const int32_t *turns_per_conv,
                                    const opr_turn *turns, const opr_layout *out, int64_t *C_out, int64_t *T_out) {
  if (B < 1 || L < 1) return OPR_E_INVALID;
  if ((int64_t)B * L >= (int64_t)1 << 31) return OPR_E_UNSUPPORTED;
  if (!valid_block(block_q) || !valid_block(block_k)) return OPR_E_UNSUPPORTED;
  if (!convs_per_row || !out) return OPR_E_INVALID;
  if (!out->tok_conv || !out->tok_turn || !out->tok_pos || !out->tok_type || !out->tok_slot ||
      !out->slot_tok || !out->slot_qiv || !out->slot_kiv || !out->tile_class || !out->sub_class ||
      !out->q_nnz || !out->q_list || !out->k_nnz || !out->k_list)
    return OPR_E_INVALID;
  if (out->order != OPR_ORDER_PACKED && out->order != OPR_ORDER_ATTENTION) return OPR_E_INVALID;
  if (!aligned16(out->slot_qiv) || !aligned16(out->slot_kiv)) return OPR_E_INVALID;
  const int64_t MT = ((int64_t)L + block_q - 1) / block_q, NT = ((int64_t)L + block_k - 1) / block_k;
  if ((int64_t)B * MT * NT >= (int64_t)1 << 31) return OPR_E_UNSUPPORTED;
  // count conversations and turns, check every length and each row's capacity
  int64_t C = 0, T = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (convs_per_row[b] < 0) return OPR_E_INVALID;
    C += convs_per_row[b];
    if (C >= (int64_t)1 << 30) return OPR_E_INVALID;
  }
  if (C > 0 && !turns_per_conv) return OPR_E_INVALID;
  int64_t c = 0;
  for (int32_t b = 0; b < B; ++b) {
    int64_t row_tokens = 0;
    for (int32_t i = 0; i < convs_per_row[b]; ++i, ++c) {
      const int32_t nt = turns_per_conv[c];
      if (nt < 0) return OPR_E_INVALID;
      if (nt > 0 && !turns) return OPR_E_INVALID;
      for (int32_t j = 0; j < nt; ++j) {
        const opr_turn &u = turns[T + j];
        if (u.h < 0 || u.t < 0 || u.r_in < 0 || u.r_out < 0) return OPR_E_INVALID;
        row_tokens += (int64_t)u.h + u.t + u.r_in + u.r_out;
        if (row_tokens > L) return OPR_E_CAPACITY;
      }
      T += nt;
      if (T >= (int64_t)1 << 30) return OPR_E_INVALID;
    }
  }
  *C_out = C;
  *T_out = T;
  return OPR_OK;
}

// Copies the host segment arrays into the workspace and launches the layout
// kernels (arguments already validated).
// The device address of a host array that the current GPU can read in place
// (page-locked and mapped into its address space), else null.  For pageable
// memory the query fails; that is not an error of the call, so the error it
// leaves is cleared.  Memory reported for another device takes the copy.
static const void *mapped_host(const void *p) {
  hipPointerAttribute_t a;
  int dev = -1;
  if (hipPointerGetAttributes(&a, p) != hipSuccess || hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (a.type != hipMemoryTypeHost || !a.devicePointer || a.device != dev) return nullptr;
  // the device address of p itself, also when p lies inside the allocation
  // and the query reports the allocation's own addresses
  const char *d = static_cast<const char *>(a.devicePointer);
  if (a.hostPointer && a.hostPointer != p) d += static_cast<const char *>(p) - static_cast<const char *>(a.hostPointer);
  return d;
}

static opr_status run_build_layout(int32_t B, int32_t L, int32_t block_q, int32_t block_k,
                                   const int32_t *convs_per_row, const int32_t *turns_per_conv,
                                   const opr_turn *turns, int64_t C, int64_t T, void *workspace,
                                   const opr_layout *out, hipStream_t stream) {
  LayoutWs ws;
  carve_layout_ws(workspace, B, L, (int32_t)C, (int32_t)T, &ws);
  // Page-locked, mapped host arrays are read in place by the first kernel:
  // no copy on the stream, so no wait between a copy engine and the compute
  // queue.  Any other host memory goes through hipMemcpyAsync.
  const void *dc = mapped_host(convs_per_row);
  const void *dt = C > 0 ? mapped_host(turns_per_conv) : dc;
  const void *du = T > 0 ? mapped_host(turns) : dc;
  if (dc && dt && du) {
    ws.src_cpr = static_cast<const int32_t *>(dc);
    ws.src_tpc = static_cast<const int32_t *>(dt);
    ws.src_turns = static_cast<const int32_t *>(du);
  } else {
    if (hipMemcpyAsync(ws.cpr, convs_per_row, sizeof(int32_t) * B, hipMemcpyHostToDevice, stream) != hipSuccess)
      return OPR_E_HIP;
    if (C > 0 &&
        hipMemcpyAsync(ws.tpc, turns_per_conv, sizeof(int32_t) * C, hipMemcpyHostToDevice, stream) != hipSuccess)
      return OPR_E_HIP;
    if (T > 0 && hipMemcpyAsync(ws.turns, turns, sizeof(opr_turn) * T, hipMemcpyHostToDevice, stream) != hipSuccess)
      return OPR_E_HIP;
  }
  if (launch_build_layout(B, L, block_q, block_k, (int32_t)C, (int32_t)T, ws, *out, stream) != hipSuccess)
    return OPR_E_HIP;
  return hip_status();
}

// The scratch of opr_build_layout_noalloc: a file-scope device array, one
// copy on every GPU the library runs on (held until the process ends).  In
// host code `scratch` names a host-side stand-in, not the device memory: the
// first call on a device looks up that device's copy with
// hipGetSymbolAddress (the device current) and keeps the address; every later
// use goes through that address.  All calls on one device share it.
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[OPR_LAYOUT_SCRATCH_BYTES];
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];

static opr_status layout_scratch(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return OPR_E_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return OPR_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return OPR_E_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return OPR_OK;
}

#ifdef OPR_DEBUG
// The error word of the checked kernels, one per device (found and kept like
// the layout scratch above).
static __device__ __align__(256) uint32_t dbg_word[64];
static void *g_dbg_ptr[kMaxDevices];
#endif

uint32_t *debug_word() {
#ifdef OPR_DEBUG
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_dbg_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(dbg_word)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_dbg_ptr[dev] = p;
  }
  return static_cast<uint32_t *>(g_dbg_ptr[dev]);
#else
  return nullptr;
#endif
}

}  // namespace opr

using namespace opr;

extern "C" {

opr_status opr_debug_errors(uint32_t *bits) {
  if (!bits) return OPR_E_INVALID;
  *bits = 0;
#ifdef OPR_DEBUG
  uint32_t *w = debug_word();
  if (!w) return OPR_E_HIP;
  uint32_t v = 0;
  if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(&v, w, sizeof v, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemset(w, 0, sizeof v) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipGetLastError();
    return OPR_E_HIP;
  }
  *bits = v;
  return OPR_OK;
#else
  return OPR_E_UNSUPPORTED;
#endif
}

size_t opr_build_layout_workspace_size(int32_t B, int32_t L, int32_t n_convs, int32_t n_turns) {
  if (B < 1 || L < 1 || n_convs < 0 || n_turns < 0) return 0;
  if ((int64_t)B * L >= (int64_t)1 << 31) return 0;
  return carve_layout_ws(nullptr, B, L, n_convs, n_turns, nullptr);
}

opr_status opr_build_layout(int32_t B, int32_t L, int32_t block_q, int32_t block_k,
                            const int32_t *convs_per_row, const int32_t *turns_per_conv,
                            const opr_turn *turns, void *workspace, size_t ws_bytes,
                            const opr_layout *out, hipStream_t stream) {
  int64_t C = 0, T = 0;
  const opr_status st = check_layout_args(B, L, block_q, block_k, convs_per_row, turns_per_conv, turns, out, &C, &T);
  if (st != OPR_OK) return st;
  if (!workspace) return OPR_E_INVALID;
  if (!aligned256(workspace)) return OPR_E_INVALID;
  if (ws_bytes < carve_layout_ws(nullptr, B, L, (int32_t)C, (int32_t)T, nullptr)) return OPR_E_CAPACITY;
  return run_build_layout(B, L, block_q, block_k, convs_per_row, turns_per_conv, turns, C, T, workspace, out, stream);
}

opr_status opr_build_layout_noalloc(int32_t B, int32_t L, int32_t block_q, int32_t block_k,
                                    const int32_t *convs_per_row, const int32_t *turns_per_conv,
                                    const opr_turn *turns, const opr_layout *out, hipStream_t stream) {
  int64_t C = 0, T = 0;
  const opr_status st = check_layout_args(B, L, block_q, block_k, convs_per_row, turns_per_conv, turns, out, &C, &T);
  if (st != OPR_OK) return st;
  if (carve_layout_ws(nullptr, B, L, (int32_t)C, (int32_t)T, nullptr) > OPR_LAYOUT_SCRATCH_BYTES)
    return OPR_E_CAPACITY;
  void *ws = nullptr;
  const opr_status ss = layout_scratch(&ws);
  if (ss != OPR_OK) return ss;
  return run_build_layout(B, L, block_q, block_k, convs_per_row, turns_per_conv, turns, C, T, ws, out, stream);
}

size_t opr_attn_workspace_size(int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int is_bwd) {
  if (check_attn_shape(B, L, Hq, Hkv, D) != OPR_OK) return 0;
  opr_attn_in in;
  memset(&in, 0, sizeof(in));
  in.B = B; in.L = L; in.Hq = Hq; in.Hkv = Hkv; in.D = D;
  return carve_attn_ws(nullptr, in, is_bwd ? 1 : 0, nullptr);
}

opr_status opr_attn_fwd(const opr_attn_in *in, void *o, float *lse, void *workspace, size_t ws_bytes,
                        hipStream_t stream) {
  const opr_status st = check_attn_in(in);
  if (st != OPR_OK) return st;
  if (!o || !lse || !workspace) return OPR_E_INVALID;
  if (!aligned16(o) || !aligned256(workspace)) return OPR_E_INVALID;
  if (ws_bytes < carve_attn_ws(nullptr, *in, 0, nullptr)) return OPR_E_CAPACITY;
  AttnWs ws;
  carve_attn_ws(workspace, *in, 0, &ws);
  mark(in, 0, stream);
  forward_prologue(*in, ws, stream, false);
  mark(in, 1, stream);
  if (launch_attn_fwd_kernel(*in, effective_scale(in), o, lse, ws, stream) != hipSuccess) return OPR_E_HIP;
  mark(in, 2, stream);
  return hip_status();
}

opr_status opr_attn_bwd(const opr_attn_in *in, const void *o, const float *lse, const void *dout,
                        float *dq, float *dk, float *dv, void *workspace, size_t ws_bytes,
                        hipStream_t stream) {
  const opr_status st = check_attn_in(in);
  if (st != OPR_OK) return st;
  if (!o || !lse || !dout || !dq || !dk || !dv || !workspace) return OPR_E_INVALID;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned256(workspace))
    return OPR_E_INVALID;
  if (ws_bytes < carve_attn_ws(nullptr, *in, 1, nullptr)) return OPR_E_CAPACITY;
  AttnWs ws;
  carve_attn_ws(workspace, *in, 1, &ws);
  mark(in, 0, stream);
  if (!in->reuse_fwd_workspace) forward_prologue(*in, ws, stream, true);
  if (launch_attn_bwd_kernels(*in, effective_scale(in), o, lse, dout, dq, dk, dv, ws, stream,
                              in->timing_events ? in->timing_events + 1 : nullptr) != hipSuccess)
    return OPR_E_HIP;
  return hip_status();
}

size_t opr_block_workspace_size(int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t d_model,
                                int is_bwd) {
  if (check_block_shape(B, L, Hq, Hkv, D, d_model) != OPR_OK) return 0;
  opr_block_in in;
  memset(&in, 0, sizeof(in));
  in.B = B; in.L = L; in.Hq = Hq; in.Hkv = Hkv; in.D = D; in.d_model = d_model;
  return carve_block_ws(nullptr, in, is_bwd ? 1 : 0, nullptr);
}

opr_status opr_block_fwd(const opr_block_in *in, void *y, void *qkv, void *o, float *lse, void *workspace,
                         size_t ws_bytes, hipStream_t stream) {
  const opr_status st = check_block_in(in);
  if (st != OPR_OK) return st;
  if (!y || !qkv || !o || !lse || !workspace) return OPR_E_INVALID;
  if (!aligned16(y) || !aligned16(qkv) || !aligned16(o) || !aligned256(workspace)) return OPR_E_INVALID;
  if (ws_bytes < carve_block_ws(nullptr, *in, 0, nullptr)) return OPR_E_CAPACITY;
  BlockWs w;
  carve_block_ws(workspace, *in, 0, &w);
  const int64_t T = (int64_t)in->B * in->L;
  const int64_t NHD = (int64_t)(in->Hq + 2 * in->Hkv) * in->D, HqD = (int64_t)in->Hq * in->D;
  bmark(in, 0, stream);
  if (!gemm_bf16(false, true, T, NHD, in->d_model, in->x, in->w_qkv, qkv, false, w.gemm, kGemmWs, stream))
    return OPR_E_HIP;
  bmark(in, 1, stream);
  if (launch_qk_norm_fwd(in->D, T, in->Hq, in->Hkv, in->norm_eps, qkv, in->g_q, in->g_k, w.qn, w.kn, w.v,
                         stream) != hipSuccess)
    return OPR_E_HIP;
  bmark(in, 2, stream);
  const opr_attn_in a = attn_in_of(*in, w.qn, w.kn, w.v);
  const opr_status sa = opr_attn_fwd(&a, o, lse, w.attn, w.attn_bytes, stream);
  if (sa != OPR_OK) return sa;
  bmark(in, 3, stream);
  if (!gemm_bf16(false, true, T, in->d_model, HqD, o, in->w_o, y, false, w.gemm, kGemmWs, stream))
    return OPR_E_HIP;
  bmark(in, 4, stream);
  return hip_status();
}

opr_status opr_block_bwd(const opr_block_in *in, const void *qkv, const void *o, const float *lse,
                         const void *dy, void *dx, float *dw_qkv, float *dw_o, float *dg_q, float *dg_k,
                         void *workspace, size_t ws_bytes, hipStream_t stream) {
  const opr_status st = check_block_in(in);
  if (st != OPR_OK) return st;
  if (!qkv || !o || !lse || !dy || !dx || !dw_qkv || !dw_o || !dg_q || !dg_k || !workspace) return OPR_E_INVALID;
  if (!aligned16(qkv) || !aligned16(o) || !aligned16(dy) || !aligned16(dx) || !aligned16(dw_qkv) ||
      !aligned16(dw_o) || !aligned256(workspace))
    return OPR_E_INVALID;
  if (ws_bytes < carve_block_ws(nullptr, *in, 1, nullptr)) return OPR_E_CAPACITY;
  BlockWs w;
  carve_block_ws(workspace, *in, 1, &w);
  const int64_t T = (int64_t)in->B * in->L;
  const int64_t NHD = (int64_t)(in->Hq + 2 * in->Hkv) * in->D, HqD = (int64_t)in->Hq * in->D;
  bmark(in, 0, stream);
  // y = o w_o^T:  d(o) = dy w_o,  dw_o = dy^T o
  if (!gemm_bf16(false, false, T, HqD, in->d_model, dy, in->w_o, w.dout, false, w.gemm, kGemmWs, stream) ||
      !gemm_bf16(true, false, in->d_model, HqD, T, dy, o, dw_o, true, w.gemm, kGemmWs, stream))
    return OPR_E_HIP;
  bmark(in, 1, stream);
  if (!in->reuse_fwd_workspace &&
      launch_qk_norm_fwd(in->D, T, in->Hq, in->Hkv, in->norm_eps, qkv, in->g_q, in->g_k, w.qn, w.kn, w.v,
                         stream) != hipSuccess)
    return OPR_E_HIP;
  bmark(in, 2, stream);
  opr_attn_in a = attn_in_of(*in, w.qn, w.kn, w.v);
  a.reuse_fwd_workspace = in->reuse_fwd_workspace ? 1 : 0;
  const opr_status sa = opr_attn_bwd(&a, o, lse, w.dout, w.dqn, w.dkn, w.dv, w.attn, w.attn_bytes, stream);
  if (sa != OPR_OK) return sa;
  bmark(in, 3, stream);
  if (launch_qk_norm_bwd(in->D, T, in->Hq, in->Hkv, in->norm_eps, qkv, in->g_q, in->g_k, w.dqn, w.dkn, w.dv,
                         w.dqkv, w.part, dg_q, dg_k, stream) != hipSuccess)
    return OPR_E_HIP;
  bmark(in, 4, stream);
  // qkv = x w_qkv^T:  dx = dqkv w_qkv,  dw_qkv = dqkv^T x
  if (!gemm_bf16(false, false, T, in->d_model, NHD, w.dqkv, in->w_qkv, dx, false, w.gemm, kGemmWs, stream) ||
      !gemm_bf16(true, false, NHD, in->d_model, T, w.dqkv, in->x, dw_qkv, true, w.gemm, kGemmWs, stream))
    return OPR_E_HIP;
  bmark(in, 5, stream);
  return hip_status();
}

size_t opr_token_ce_workspace_size(int32_t B, int32_t L, int32_t F, int32_t V) {
  if (B < 1 || L < 1 || (int64_t)B * L >= (int64_t)1 << 31) return 0;
  if (F < 64 || F % 64 != 0 || F > (1 << 20)) return 0;
  if (V != 32 && V != 64 && V != 128) return 0;
  return token_ce_ws_bytes((int64_t)B * L, V);
}

opr_status opr_token_ce(int32_t B, int32_t L, int32_t F, int32_t V, const void *o, const void *w,
                        const int32_t *labels, const uint8_t *tok_type, float grad_scale, float *loss,
                        void *dout, void *workspace, size_t ws_bytes, hipStream_t stream) {
  if (B < 1 || L < 1) return OPR_E_INVALID;
  if ((int64_t)B * L >= (int64_t)1 << 31) return OPR_E_UNSUPPORTED;
  if (F < 64 || F % 64 != 0 || F > (1 << 20)) return OPR_E_UNSUPPORTED;
  if (V != 32 && V != 64 && V != 128) return OPR_E_UNSUPPORTED;
  if (!o || !w || !labels || !tok_type || !loss) return OPR_E_INVALID;
  if (!aligned16(o) || !aligned16(w) || (dout && !aligned16(dout))) return OPR_E_INVALID;
  if (!isfinite(grad_scale)) return OPR_E_INVALID;
  if (dout && (!workspace || ws_bytes < token_ce_ws_bytes((int64_t)B * L, V))) {
    if (!workspace) return OPR_E_INVALID;
    return OPR_E_CAPACITY;
  }
  if (dout && !aligned16(workspace)) return OPR_E_INVALID;
  if (launch_token_ce(B, L, F, V, o, w, labels, tok_type, grad_scale, loss, dout, workspace, stream) !=
      hipSuccess)
    return OPR_E_HIP;
  return hip_status();
}

const char *opr_status_string(opr_status s) {
  // a C caller may pass any int: read the bytes, never an out-of-range enum value
  int32_t v;
  memcpy(&v, &s, sizeof(v));
  switch (v) {
    case OPR_OK: return "OPR_OK";
    case OPR_E_INVALID: return "OPR_E_INVALID: invalid argument";
    case OPR_E_CAPACITY: return "OPR_E_CAPACITY: row longer than L or workspace too small";
    case OPR_E_UNSUPPORTED: return "OPR_E_UNSUPPORTED: size or option not supported";
    case OPR_E_HIP: return "OPR_E_HIP: HIP launch or call failed";
  }
  return "unknown opr_status";
}

}  // extern "C"

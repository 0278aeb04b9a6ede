/*
 * opr.h - C ABI of libopr: one-pass block-sparse masked attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is One-Pass to Reason (Goru, Mehta, Jain; arXiv 2504.18246).
 * A multi-turn reasoning conversation is packed once: every turn i holds the
 * human message h_i, the reasoning t_i, and the response stored twice, as a
 * context copy r_in_i and a generation copy r_out_i (wiki summary of the
 * paper, section "Token 复制" / token duplication).  A block-sparse mask
 * (section "分块稀疏注意力掩码") lets
 *     h_i     see H_<i,
 *     t_i     see H_<i and h_i,
 *     r_in_i  see H_<i and h_i,
 *     r_out_i see H_<i, h_i and t_i,
 * where H_<i is the human messages and context copies of the earlier turns,
 * and every token sees its own segment causally.  Position ids (section
 * "位置 ID 策略") start t_i and r_in_i right after h_i, r_out_i right after
 * t_i, and h_{i+1} right after r_in_i, so that one pass gives the same
 * per-token results as the N separate causal passes (section "理论保证",
 * Theorem 2.1).  Packed conversations (section "实现细节") never see each
 * other and each starts at position 0.
 *
 * Conventions for every entry point
 *  - Pointers are device pointers unless the comment says "host".  The caller
 *    allocates and owns every buffer, including the workspace; the library
 *    never allocates or frees memory and never synchronises the stream
 *    (the one exception: the hipBLASLt handle of the entry points that run
 *    GEMMs, opr_token_ce with a gradient and opr_block_*).
 *  - All arguments are validated on the host before any HIP call.  On a
 *    validation failure the call returns an error status, writes nothing and
 *    enqueues nothing.
 *  - Work is enqueued on `stream` in order; outputs are ready when the stream
 *    reaches that point.  A failed launch returns OPR_E_HIP (the HIP error is
 *    read with hipGetLastError and cleared).
 *  - Concurrent calls on different streams must use different workspaces.
 *  - Row-major layouts are written [dim0][dim1]...; "bf16" is IEEE bfloat16.
 */
#ifndef OPR_H
#define OPR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  OPR_OK = 0,
  OPR_E_INVALID = -1,     /* null pointer, negative length, inconsistent sizes */
  OPR_E_CAPACITY = -2,    /* a row needs more than L tokens, or workspace too small */
  OPR_E_UNSUPPORTED = -3, /* well-formed but not implemented (head dim, tile size) */
  OPR_E_HIP = -4          /* a HIP call or kernel launch failed */
} opr_status;

/* Token types, in their order inside a turn. */
enum { OPR_TOK_H = 0, OPR_TOK_T = 1, OPR_TOK_RIN = 2, OPR_TOK_ROUT = 3, OPR_TOK_PAD = 4 };

/* Tile classes: no allowed pair / some / all (entries past L count as masked). */
enum { OPR_TILE_EMPTY = 0, OPR_TILE_PARTIAL = 1, OPR_TILE_FULL = 2 };

/* Sub-block edge of the sub-block classes, in tokens. */
#define OPR_SUB_BLOCK 32

/* Attention tile the kernels run on: opr_attn_* need a layout built with
 * block_q == block_k == OPR_ATTN_BLOCK and order OPR_ORDER_ATTENTION. */
#define OPR_ATTN_BLOCK 128

/* The token order a tile schedule covers.
 *  OPR_ORDER_PACKED     the packed rows as the pages draw the mask.
 *  OPR_ORDER_ATTENTION  attention order: inside each conversation's index
 *      range, first its h and r_in tokens (the ones later turns may see), in
 *      packed order, then its t and r_out tokens, in packed order; PAD tokens
 *      keep their index.  Attention commutes with reordering queries and keys
 *      alike, so this changes no result; it is the order the attention kernels
 *      run in, because there every query sees at most two runs of key slots,
 *      all at or before its own slot, and the non-empty tiles are fewer and
 *      denser.  (A choice of this library, not of the pages; the h and r_in
 *      slots are conversation start + position id.) */
enum { OPR_ORDER_PACKED = 0, OPR_ORDER_ATTENTION = 1 };

/* Segment lengths of one turn, each >= 0.  An ordinary turn has
 * r_in == r_out (the response stored twice); a history-only turn of a K-pass
 * chunk is (h, 0, r, 0) and the last turn of an N-pass sequence (h, t, 0, r). */
typedef struct {
  int32_t h, t, r_in, r_out;
} opr_turn;

/* Outputs of opr_build_layout for B rows of L tokens and block_q x block_k
 * tiles; MT = ceil(L / block_q), NT = ceil(L / block_k).  A "slot" is an
 * index in attention order.  Two runs [x0, x1) and [x2, x3) of slots are
 * stored as int32 [4] with x0 <= x1 <= x2 <= x3, maximal and ascending; a
 * missing run is written [x, x) with x the end of the run before it (0 if
 * there is none). */
typedef struct {
  int32_t *tok_conv;   /* [B][L] conversation index within the row; -1 for PAD */
  int32_t *tok_turn;   /* [B][L] turn index within the conversation; -1 for PAD */
  int32_t *tok_pos;    /* [B][L] strategic position id; 0 for PAD */
  uint8_t *tok_type;   /* [B][L] OPR_TOK_* */
  int32_t *tok_slot;   /* [B][L] slot of each token in attention order */
  int32_t *slot_tok;   /* [B][L] token at each slot (the inverse permutation) */
  int32_t *slot_qiv;   /* [B][L][4] key slots the query at slot s sees (two runs);
                          16-byte aligned */
  int32_t *slot_kiv;   /* [B][L][4] query slots that see the key at slot s (two
                          runs); 16-byte aligned */
  uint8_t *tile_class; /* [B][MT][NT] OPR_TILE_*, tiles over the order `order` */
  uint32_t *sub_class; /* [B][MT][NT] two bits per 32x32 sub-block (i, j) at bit
                          2*(i*(block_k/32) + j), same codes as tile_class */
  int32_t *q_nnz;      /* [B][MT] number of non-empty tiles in q-tile row m */
  int32_t *q_list;     /* [B][MT][NT] their k-tile indices ascending, then -1 */
  int32_t *k_nnz;      /* [B][NT] number of non-empty tiles in k-tile column n */
  int32_t *k_list;     /* [B][NT][MT] their q-tile indices ascending, then -1 */
  int32_t order;       /* set by the caller: OPR_ORDER_* of the tile fields */
} opr_layout;

/*
 * opr_build_layout - token layout, position ids and tile schedule.
 *
 * The sequence construction of the one pass: each response stored twice
 * (wiki summary, section "Token 复制"), the strategic position ids (section
 * "位置 ID 策略"), the block-sparse mask of the four visibility rules
 * (section "分块稀疏注意力掩码"), generated on the device (section "实现细节").
 * Packs each row's conversations back to back (segments of a turn in the
 * order h, t, r_in, r_out; the rest of the row is PAD), assigns the strategic
 * position ids above and the attention-order slots, writes the mask of every
 * slot as two runs of slots (for its query and for its key), and classifies
 * every block_q x block_k tile of the block-sparse mask, in the order
 * out->order, as empty / partial / full, with 32x32 sub-block classes and the
 * per-row and per-column lists of non-empty tiles.  Everything is computed on
 * the device from the segment lengths; no dense mask is formed.
 *
 *  B, L            rows and tokens per row; B >= 1, L >= 1, B*L < 2^31.
 *  block_q/block_k tile edges, each 32, 64 or 128.
 *  convs_per_row   host [B], >= 0.  turns_per_conv host [sum convs_per_row],
 *                  >= 0.  turns host [sum turns_per_conv].  Conversations are
 *                  listed row by row, turns conversation by conversation.
 *  workspace       device, at least opr_build_layout_workspace_size(...) bytes.
 *  out             host struct of device pointers, all non-NULL, and the
 *                  order (OPR_ORDER_*) of the tile schedule to build.
 * Errors: OPR_E_INVALID (null pointer, misaligned slot_qiv / slot_kiv,
 * negative count or length, bad B/L, unknown order),
 * OPR_E_UNSUPPORTED (block size), OPR_E_CAPACITY (a row longer than L, or
 * ws_bytes too small), OPR_E_HIP.
 * Host arrays: when all three are in page-locked host memory mapped for the
 * device (hipHostMalloc, or torch's pinned memory), the first kernel reads
 * them in place and no copy is enqueued; otherwise they are copied to the
 * workspace with hipMemcpyAsync (pageable memory is staged before the call
 * returns).  Either way, keep them unchanged until the stream has run the
 * call.
 */
opr_status opr_build_layout(int32_t B, int32_t L, int32_t block_q, int32_t block_k,
                            const int32_t *convs_per_row, const int32_t *turns_per_conv,
                            const opr_turn *turns, void *workspace, size_t ws_bytes,
                            const opr_layout *out, hipStream_t stream);

/* Workspace bytes for opr_build_layout with n_convs conversations and n_turns
 * turns in total (the sums of convs_per_row and turns_per_conv). */
size_t opr_build_layout_workspace_size(int32_t B, int32_t L, int32_t n_convs, int32_t n_turns);

/* Size of the fixed device scratch of opr_build_layout_noalloc: 32 MiB on
 * every GPU the library runs on. */
#define OPR_LAYOUT_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * opr_build_layout_noalloc - opr_build_layout for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes no workspace and allocates
 * nothing (no hipMalloc, hipFree or allocating library call): its scratch is
 * a fixed OPR_LAYOUT_SCRATCH_BYTES array in the library's device code, one
 * copy per GPU, held until the process ends.
 *
 * Arguments, results and errors are those of opr_build_layout without
 * workspace and ws_bytes, plus OPR_E_CAPACITY when
 * opr_build_layout_workspace_size(B, L, n_convs, n_turns) exceeds
 * OPR_LAYOUT_SCRATCH_BYTES (about 8 M packed tokens in total; checked
 * before any HIP call, nothing is enqueued).  The first call on a device
 * looks up that device's scratch with the device current; `stream` must
 * belong to the current device.  All calls on one GPU share its scratch:
 * calls that overlap on one GPU (other streams, other host threads) race
 * and must be serialised by the caller.  Every scratch word a call reads is
 * written earlier by the same call, so nothing needs clearing between calls.
 */
opr_status opr_build_layout_noalloc(int32_t B, int32_t L, int32_t block_q, int32_t block_k,
                                    const int32_t *convs_per_row, const int32_t *turns_per_conv,
                                    const opr_turn *turns, const opr_layout *out, hipStream_t stream);

/* Inputs shared by the forward and backward calls. */
typedef struct {
  int32_t B, L, Hq, Hkv, D; /* D in {64, 128}; Hq % Hkv == 0; q head h reads kv
                               head h / (Hq / Hkv) (grouped-query attention) */
  float softmax_scale;      /* 0 selects 1/sqrt(D) */
  double rope_theta;        /* RoPE base; > 0 */
  const void *q;            /* bf16 [B][L][Hq][D], before RoPE */
  const void *k;            /* bf16 [B][L][Hkv][D], before RoPE */
  const void *v;            /* bf16 [B][L][Hkv][D] */
  opr_layout layout;        /* from opr_build_layout(B, L, block_q, block_k, ...)
                               with order OPR_ORDER_ATTENTION */
  int32_t block_q, block_k; /* must both be OPR_ATTN_BLOCK */
  /* Optional instrumentation, may be NULL: host array of events created by
   * the caller (hipEventCreate).  opr_attn_fwd records [0] before its
   * prologue, [1] before the attention kernel and [2] after it;
   * opr_attn_bwd records [0] before its prologue (the forward state, only
   * without reuse_fwd_workspace), [1] before the dQ kernel (which also
   * forms delta = rowsum(dout * o) and the fp16 dout), [2] after it and
   * the small kernel that picks the dK/dV kernel's units, and [3] right
   * after the dK/dV kernel (the small kernel that sums the parts of
   * cut dK/dV columns runs after [3]). */
  hipEvent_t *timing_events;
  /* opr_attn_bwd only: nonzero when `workspace` is the one the matching
   * opr_attn_fwd call (same inputs, layout and stream, nothing written to the
   * workspace in between) just used.  The backward then reuses the fp16
   * copies of q, k, v, their scales and the mask intervals that the forward
   * left at the start of the workspace instead of recomputing them.  0 makes
   * opr_attn_bwd self-contained. */
  int32_t reuse_fwd_workspace;
} opr_attn_in;

/*
 * opr_attn_fwd - masked attention forward.
 *
 * The attention of the one pass: every token attends, with ordinary softmax
 * attention, to exactly the keys the four visibility rules allow (wiki
 * summary, section "分块稀疏注意力掩码"), with RoPE at the strategic position
 * ids (section "位置 ID 策略"), so that each token gets the result of its own
 * N-pass sequence (section "理论保证", Theorem 2.1).  RoPE (rotate-half pairs
 * (j, j + D/2), angle pos * theta^(-2j/D); the pages name no variant, this is
 * Qwen-3's, their model family) is applied to q and k at the layout's
 * position ids; then for every query token and q head, softmax(scale q k^T)
 * over the allowed keys, times v.  The kernels run in attention order: q, k,
 * v are gathered into slot order, empty tiles are skipped, and partial 32x32
 * sub-blocks test the mask per element from the two runs of slots of the
 * layout; results are written back at the tokens' own rows.
 *
 *  in->q, k, v  16-byte aligned.
 *  o    bf16 [B][L][Hq][D]   attention output; PAD rows get 0; 16-byte aligned.
 *  lse  fp32 [B][Hq][L]      natural-log sum of exp of the scaled scores of
 *                            the allowed keys; -inf for PAD rows.
 *  workspace  >= opr_attn_workspace_size(B, L, Hq, Hkv, D, 0) bytes, 256-byte
 *             aligned.
 * Input range: the matrix products run on fp16 operands with power-of-two
 * scales (one per query row and q head for q after RoPE, one per (row, kv
 * head) plane for k after RoPE and v).  Results are accurate for finite
 * inputs whose largest magnitude per row (q, dout) or per plane (k, v) lies
 * in [2^-46, 2^75); rows or planes of smaller values keep an absolute
 * precision of about 2^-84, and magnitudes of 2^76 and more overflow fp16
 * and give non-finite results.  (The data is not inspected on the host; no
 * status reports it.)
 * Errors: OPR_E_INVALID (null or misaligned pointer, a layout of another
 * order), OPR_E_UNSUPPORTED (D, block sizes), OPR_E_CAPACITY (ws_bytes),
 * OPR_E_HIP.
 */
opr_status opr_attn_fwd(const opr_attn_in *in, void *o, float *lse, void *workspace,
                        size_t ws_bytes, hipStream_t stream);

/*
 * opr_attn_bwd - gradients of sum(o * dout) with respect to q, k and v
 * (before RoPE: the RoPE rotation is transposed back onto dq and dk).
 *
 * The gradients of the one pass equal those of the N separate passes summed
 * onto the shared tokens (wiki summary, section "理论保证": the loss is the
 * same per token, so is its gradient).  With P the masked softmax,
 * dV = sum over the kv group's heads of P^T dout, dS = P (dout v^T - delta)
 * with delta = rowsum(dout * o) over the o given here, dQ = scale dS k',
 * dK = scale sum over the group of dS^T q'.
 *
 *  o, lse  the outputs of opr_attn_fwd for the same inputs; o 16-byte aligned.
 *  dout    bf16 [B][L][Hq][D]; 16-byte aligned.  The input range of
 *          opr_attn_fwd applies to it per row.
 *  dq      fp32 [B][L][Hq][D];  dk, dv  fp32 [B][L][Hkv][D]; 16-byte aligned.
 *          Every element is written (PAD rows get 0); nothing is accumulated
 *          into them.  The sums run in a fixed order: the same inputs give
 *          bit-identical gradients on every call.
 *  workspace  >= opr_attn_workspace_size(B, L, Hq, Hkv, D, 1) bytes, 256-byte
 *             aligned; the forward part of it is a prefix, so one
 *             backward-sized workspace serves both calls (see
 *             reuse_fwd_workspace).
 * Errors as for opr_attn_fwd.
 */
opr_status opr_attn_bwd(const opr_attn_in *in, const void *o, const float *lse,
                        const void *dout, float *dq, float *dk, float *dv,
                        void *workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for opr_attn_fwd (is_bwd = 0) or opr_attn_bwd (is_bwd = 1);
 * 0 if the sizes are invalid. */
size_t opr_attn_workspace_size(int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D,
                               int is_bwd);

/*
 * opr_token_ce - per-token cross entropy of a linear head on the attention
 * output, and its gradient: the loss step that follows opr_attn_fwd and
 * feeds opr_attn_bwd.
 *
 * The pages state that one pass gives every token the same loss as the N
 * separate passes (wiki summary, section "理论保证", Theorem 2.1).  The
 * scored rows are the tokens of type OPR_TOK_T and OPR_TOK_ROUT: the
 * reasoning and the generation copy of each response (section "Token 复制":
 * the generation copy is the one in the loss; the context copy r_in and the
 * human messages are context only).  For a scored row p, with o_p its
 * F = Hq * D attention outputs in the order o stores them and W the head:
 *     z_p       = W o_p                       (V logits, fp32)
 *     loss[p]   = logsumexp(z_p) - z_p[labels[p]]
 *     dout[p]   = grad_scale * (softmax(z_p) - onehot(labels[p]))^T W
 * Every other row gets loss 0 and dout 0.  Logits are bf16 products with
 * fp32 accumulation; the logit gradient g = grad_scale * (softmax - onehot) is
 * rounded to bf16 and dout = g W is a bf16 GEMM (hipBLASLt) with fp32
 * accumulation, rounded to bf16 once.
 *
 *  B, L        rows and tokens per row of the layout; B*L < 2^31.
 *  F, V        features per token (F % 64 == 0, 64 <= F <= 2^20) and logits
 *              (V in {32, 64, 128}).
 *  o           bf16 [B][L][F] (opr_attn_fwd's o with F = Hq * D); 16-byte aligned.
 *  w           bf16 [V][F], one row of weights per logit (the layout of a
 *              linear layer's weight); 16-byte aligned.
 *  labels      int32 [B][L]; read on scored rows only.  A label outside
 *              [0, V) gives that row loss NaN and dout 0.
 *  tok_type    uint8 [B][L], the layout's tok_type.
 *  grad_scale  factor on dout (1 for the gradient of the summed loss).
 *  loss        fp32 [B][L], every element written.
 *  dout        bf16 [B][L][F], every element written, or NULL to skip the
 *              gradient; 16-byte aligned.
 *  workspace   device, 16-byte aligned, >= opr_token_ce_workspace_size(B, L,
 *              F, V) bytes when dout is not NULL (it receives g and the GEMM's
 *              scratch); may be NULL otherwise.
 * Errors: OPR_E_INVALID (null or misaligned pointer, B/L, non-finite
 * grad_scale), OPR_E_UNSUPPORTED (F, V, B*L), OPR_E_CAPACITY (ws_bytes),
 * OPR_E_HIP (a launch or the hipBLASLt call failed).
 */
opr_status opr_token_ce(int32_t B, int32_t L, int32_t F, int32_t V, const void *o, const void *w,
                        const int32_t *labels, const uint8_t *tok_type, float grad_scale, float *loss,
                        void *dout, void *workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for opr_token_ce with a gradient on B x L rows; 0 if the
 * sizes are invalid. */
size_t opr_token_ce_workspace_size(int32_t B, int32_t L, int32_t F, int32_t V);

/* Inputs of the attention block (opr_block_fwd / opr_block_bwd). */
typedef struct {
  int32_t B, L, Hq, Hkv, D; /* as in opr_attn_in */
  int32_t d_model;          /* hidden size, a multiple of 64 */
  float softmax_scale;      /* 0 selects 1/sqrt(D) */
  double rope_theta;        /* RoPE base; > 0 */
  float norm_eps;           /* RMSNorm epsilon; > 0 */
  const void *x;            /* bf16 [B][L][d_model], the block's input rows */
  const void *w_qkv;        /* bf16 [(Hq + 2 Hkv) D][d_model]: the q heads', then the
                               k heads', then the v heads' output rows (a linear
                               layer's weight) */
  const void *w_o;          /* bf16 [d_model][Hq D] */
  const float *g_q, *g_k;   /* fp32 [D], RMSNorm weights shared by the q heads and
                               by the k heads */
  opr_layout layout;        /* as in opr_attn_in (order OPR_ORDER_ATTENTION) */
  int32_t block_q, block_k; /* must both be OPR_ATTN_BLOCK */
  /* Optional instrumentation, may be NULL: host array of caller-created
   * events.  opr_block_fwd records [0] at its start, [1] after the qkv
   * projection, [2] after the head norms, [3] after the attention and [4]
   * after the output projection; opr_block_bwd records [0] at its start, [1]
   * after the output projection's gradients, [2] after the head norms,
   * [3] after the attention backward, [4] after the norms' backward and [5]
   * after the qkv projection's gradients. */
  hipEvent_t *timing_events;
  /* opr_block_bwd only: nonzero when `workspace` is the one the matching
   * opr_block_fwd call (same inputs, layout and stream, nothing written to
   * the workspace in between) just used; the backward then reuses the
   * normalised q, k, v and the attention's forward state left at the start
   * of the workspace instead of recomputing them.  0 makes opr_block_bwd
   * self-contained. */
  int32_t reuse_fwd_workspace;
} opr_block_in;

/*
 * opr_block_fwd - one attention block around the masked attention, with the
 * per-head query/key normalisation of Qwen-3, the model family the pages
 * train (wiki summary, "实验结果").  Every op but the attention acts on each
 * token alone, so one pass over the packed rows still gives every token the
 * result of its own N-pass sequence (section "理论保证", Theorem 2.1).
 *
 *   qkv = x w_qkv^T                                  (bf16 out, fp32 accumulation)
 *   q_h = g_q * RMSNorm(qkv q head h), k_h = g_k * RMSNorm(qkv k head h)
 *         (per token and head over D: x / sqrt(mean(x^2) + norm_eps)),
 *   o   = opr_attn_fwd(q, k, v) with RoPE at the layout's position ids,
 *   y   = o w_o^T                                    (o seen as [B][L][Hq D])
 *
 *  y    bf16 [B][L][d_model]; PAD rows get 0.
 *  qkv  bf16 [B][L][(Hq + 2 Hkv) D], o bf16 [B][L][Hq][D] and lse fp32
 *       [B][Hq][L]: written, and kept by the caller for opr_block_bwd.
 *  workspace  >= opr_block_workspace_size(..., 0) bytes.
 * x, w_qkv, w_o, y, qkv and o must be 16-byte aligned.  Errors: as
 * opr_attn_fwd, plus OPR_E_INVALID (d_model, norm_eps, null or misaligned
 * pointers) and OPR_E_HIP when a hipBLASLt call fails.  The GEMMs run in
 * hipBLASLt; its handle is created on the device's first call and kept until
 * the process ends (the one allocation the library leaves to a dependency).
 */
opr_status opr_block_fwd(const opr_block_in *in, void *y, void *qkv, void *o, float *lse, void *workspace,
                         size_t ws_bytes, hipStream_t stream);

/*
 * opr_block_bwd - gradients of sum(y * dy) for opr_block_fwd.
 *
 *  qkv, o, lse  what opr_block_fwd wrote for the same inputs.
 *  dy      bf16 [B][L][d_model].
 *  dx      bf16 [B][L][d_model].
 *  dw_qkv  fp32 [(Hq + 2 Hkv) D][d_model], dw_o fp32 [d_model][Hq D],
 *  dg_q, dg_k  fp32 [D].  Every element is written, nothing accumulated.
 *  workspace  >= opr_block_workspace_size(..., 1) bytes.
 * The attention's q, k and v are recomputed from qkv unless the forward's
 * workspace is reused (reuse_fwd_workspace; the forward-sized workspace is a
 * prefix of the backward-sized one, so one backward-sized workspace serves
 * both calls).  dx, dw_qkv and dw_o must be 16-byte aligned.  Errors as for
 * opr_block_fwd.
 */
opr_status opr_block_bwd(const opr_block_in *in, const void *qkv, const void *o, const float *lse,
                         const void *dy, void *dx, float *dw_qkv, float *dw_o, float *dg_q, float *dg_k,
                         void *workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for opr_block_fwd (is_bwd = 0) or opr_block_bwd (is_bwd = 1);
 * 0 if the sizes are invalid. */
size_t opr_block_workspace_size(int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t d_model,
                                int is_bwd);

/* One chunk of a K-pass plan (see opr_kpass_plan). */
typedef struct {
  int32_t first_turn; /* the chunk trains turns [first_turn, first_turn + n_turns) */
  int32_t n_turns;
  int32_t tokens;     /* packed tokens of the chunk's sequence */
  int32_t rin_elided; /* 1 if r_in of its last turn is left out */
  int64_t pairs;      /* allowed (query, key) pairs of the sequence */
} opr_chunk;

/*
 * opr_kpass_plan - split one conversation into K-pass chunks (host only; no
 * HIP call).
 *
 * The K-pass variant trains a conversation in K sequences instead of one,
 * trading speed for memory between the one-pass and N-pass extremes (wiki
 * summary, section "实验结果", K-Pass; section "关键洞察", item 3).  The
 * sequence of a chunk of turns [a, b) is the history turns j < a written
 * (h_j, 0, r_in_j, 0), context only, followed by turns a .. b-1 unchanged;
 * with elide_last_rin, turn b-1 is written (h, t, 0, r_out): its context copy
 * is seen by no query of the sequence (only later turns see a turn's r_in,
 * and it is not scored), so dropping it changes no other token's position id
 * or result.  Passing these turn lists to opr_build_layout builds the rows.
 *
 * Among all splits into contiguous chunks, the call returns one that
 * minimises sum over chunks of (pairs + tokens_weight * tokens), where pairs
 * is the number of allowed (query, key) pairs of the chunk's sequence (every
 * token sees its position id + 1 keys) and tokens its length, subject to
 * tokens <= max_tokens for every chunk.  Ties go to fewer chunks.
 *
 *  turns          host [n_turns], n_turns >= 1, every length >= 0, and the
 *                 sum of all lengths < 2^31.
 *  n_chunks       exactly this many chunks (1 .. n_turns), or 0 for any number.
 *  max_tokens     cap on a chunk sequence's length; 0 for none.
 *  tokens_weight  >= 0, finite: the cost of a token in units of one pair.
 *  chunks         host [n_turns] (room for the most chunks a plan can have);
 *                 entries [0, *n_out) are written in turn order.
 *  n_out          host, the number of chunks.
 *  cost           host, may be NULL: the minimised objective.
 * Time and memory: O(n_turns^2) time and O(n_turns) memory for any number
 * of chunks, O(n_chunks * n_turns^2) time and O(n_chunks * n_turns) memory
 * for exactly n_chunks.
 * Errors: OPR_E_INVALID (null pointer, counts, lengths, weight),
 * OPR_E_CAPACITY (no split meets max_tokens: some turn's sequence alone is
 * longer, or n_chunks chunks cannot all fit), OPR_E_UNSUPPORTED (n_turns >
 * 65536, n_chunks * n_turns^2 > 2^33, or the tables do not fit in host
 * memory).  On error nothing is written.
 */
opr_status opr_kpass_plan(const opr_turn *turns, int32_t n_turns, int32_t n_chunks, int32_t max_tokens,
                          double tokens_weight, int32_t elide_last_rin, opr_chunk *chunks, int32_t *n_out,
                          double *cost);

/* Static, human-readable name of a status code. */
const char *opr_status_string(opr_status status);

/* ---------------------------------------------------------------------------
 * opr_debug_errors: the invariant tests of a checked build.
 *
 * A library built with -DOPR_DEBUG (libopr_debug.so; block_sparse_masked_opr_amd
 * build(debug=True)) runs the same kernels with tests of the invariants
 * their indexing relies on; a violated test sets a bit in a per-device word
 * and skips the access it guards, so no kernel leaves its buffers.  Bits:
 * 1 a q-tile list entry outside the tile grid, 2 a k-tile list entry outside
 * it, 4 the token of a live slot outside its row, 8 a dK/dV work item outside
 * its tables.  Any bit set means the layout given to the attention calls did
 * not come from opr_build_layout for the same B and L, or a library bug.
 *  bits   host; receives the current device's word, which is then cleared.
 * Synchronises the current device (checked builds only).
 * Errors: OPR_E_INVALID (bits NULL), OPR_E_UNSUPPORTED (a release build:
 * *bits = 0, nothing is tested), OPR_E_HIP.
 */
opr_status opr_debug_errors(uint32_t *bits);

#ifdef __cplusplus
}
#endif

#endif /* OPR_H */

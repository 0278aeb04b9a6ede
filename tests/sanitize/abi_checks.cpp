// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of opr_api.cpp and
// kpass_plan.cpp (tests/test_sanitize_host.py).  Every device pointer here is
// fake and every call is one that fails validation before any HIP call, except
// opr_kpass_plan, which is host-only and runs on real inputs.  The process
// exits nonzero on the first failed check; a sanitizer report aborts it.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <random>
#include <vector>

#include "opr.h"

static int g_checks = 0;

#define CHECK(cond)                                                              \
  do {                                                                           \
    ++g_checks;                                                                  \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);   \
      std::exit(1);                                                              \
    }                                                                            \
  } while (0)

static void *const FAKE = reinterpret_cast<void *>(0x100000);
static void *fake(size_t off) { return reinterpret_cast<char *>(FAKE) + off; }

static opr_layout fake_layout(int order = OPR_ORDER_ATTENTION) {
  opr_layout l;
  l.tok_conv = l.tok_turn = l.tok_pos = static_cast<int32_t *>(FAKE);
  l.tok_type = static_cast<uint8_t *>(FAKE);
  l.tok_slot = l.slot_tok = l.slot_qiv = l.slot_kiv = static_cast<int32_t *>(FAKE);
  l.tile_class = static_cast<uint8_t *>(FAKE);
  l.sub_class = static_cast<uint32_t *>(FAKE);
  l.q_nnz = l.q_list = l.k_nnz = l.k_list = static_cast<int32_t *>(FAKE);
  l.order = order;
  return l;
}

static void layout_checks() {
  const int32_t cpr[1] = {1}, tpc[1] = {1};
  const opr_turn turn[1] = {{8, 12, 6, 6}};
  opr_layout l = fake_layout();
  auto build = [&](int32_t B, int32_t L, int32_t bq, int32_t bk, const int32_t *c, const int32_t *t,
                   const opr_turn *u, void *ws, size_t wsb, const opr_layout *o) {
    return opr_build_layout(B, L, bq, bk, c, t, u, ws, wsb, o, nullptr);
  };
  CHECK(build(0, 64, 128, 128, cpr, tpc, turn, FAKE, 1 << 20, &l) == OPR_E_INVALID);
  CHECK(build(1, 0, 128, 128, cpr, tpc, turn, FAKE, 1 << 20, &l) == OPR_E_INVALID);
  CHECK(build(1, 64, 48, 128, cpr, tpc, turn, FAKE, 1 << 20, &l) == OPR_E_UNSUPPORTED);
  CHECK(build(1, 31, 128, 128, cpr, tpc, turn, FAKE, 1 << 20, &l) == OPR_E_CAPACITY);
  CHECK(build(1, 64, 128, 128, cpr, tpc, turn, FAKE, 16, &l) == OPR_E_CAPACITY);
  CHECK(build(1, 64, 128, 128, cpr, tpc, turn, nullptr, 1 << 20, &l) == OPR_E_INVALID);
  CHECK(build(1, 64, 128, 128, cpr, tpc, turn, fake(64), 1 << 20, &l) == OPR_E_INVALID);
  CHECK(build(1, 64, 128, 128, nullptr, tpc, turn, FAKE, 1 << 20, &l) == OPR_E_INVALID);
  CHECK(build(1 << 16, 1 << 15, 128, 128, cpr, tpc, turn, FAKE, 1 << 20, &l) == OPR_E_UNSUPPORTED);
  const opr_turn neg[1] = {{8, -1, 6, 6}};
  CHECK(build(1, 64, 128, 128, cpr, tpc, neg, FAKE, 1 << 20, &l) == OPR_E_INVALID);
  const int32_t cneg[1] = {-1};
  CHECK(build(1, 64, 128, 128, cneg, tpc, turn, FAKE, 1 << 20, &l) == OPR_E_INVALID);
  opr_layout odd = fake_layout();
  odd.slot_kiv = static_cast<int32_t *>(fake(8));
  CHECK(build(1, 64, 128, 128, cpr, tpc, turn, FAKE, 1 << 20, &odd) == OPR_E_INVALID);
  opr_layout bad = fake_layout(7);
  CHECK(build(1, 64, 128, 128, cpr, tpc, turn, FAKE, 1 << 20, &bad) == OPR_E_INVALID);
  for (int f = 0; f < 14; ++f) {  // every output field null in turn
    opr_layout z = fake_layout();
    void **fields[] = {(void **)&z.tok_conv, (void **)&z.tok_turn, (void **)&z.tok_pos, (void **)&z.tok_type,
                       (void **)&z.tok_slot, (void **)&z.slot_tok, (void **)&z.slot_qiv, (void **)&z.slot_kiv,
                       (void **)&z.tile_class, (void **)&z.sub_class, (void **)&z.q_nnz, (void **)&z.q_list,
                       (void **)&z.k_nnz, (void **)&z.k_list};
    *fields[f] = nullptr;
    CHECK(build(1, 64, 128, 128, cpr, tpc, turn, FAKE, 1 << 20, &z) == OPR_E_INVALID);
    CHECK(opr_build_layout_noalloc(1, 64, 128, 128, cpr, tpc, turn, &z, nullptr) == OPR_E_INVALID);
  }
  // the no-allocation variant: over its fixed scratch before any HIP call
  std::vector<int32_t> cpr64(64, 0);
  cpr64[0] = 1;
  CHECK(opr_build_layout_noalloc(64, 1 << 17, 128, 128, cpr64.data(), tpc, turn, &l, nullptr) == OPR_E_CAPACITY);
  CHECK(opr_build_layout_noalloc(1, 31, 128, 128, cpr, tpc, turn, &l, nullptr) == OPR_E_CAPACITY);
  // sizes: positive, zero for invalid, no overflow at the edges
  CHECK(opr_build_layout_workspace_size(1, 64, 1, 2) > 0);
  CHECK(opr_build_layout_workspace_size(0, 64, 1, 2) == 0);
  CHECK(opr_build_layout_workspace_size(1, 64, -1, 2) == 0);
  CHECK(opr_build_layout_workspace_size(1 << 15, 1 << 16, 0, 0) == 0);
  CHECK(opr_build_layout_workspace_size(65535, 32767, 1 << 29, 1 << 29) > (size_t)1 << 33);
}

static opr_attn_in attn_in() {
  opr_attn_in a{};
  a.B = 1; a.L = 256; a.Hq = 4; a.Hkv = 2; a.D = 128;
  a.softmax_scale = 0.0f;
  a.rope_theta = 1e6;
  a.q = a.k = a.v = FAKE;
  a.layout = fake_layout();
  a.block_q = a.block_k = 128;
  return a;
}

static void attn_checks() {
  const size_t big = (size_t)1 << 40;
  auto fwd = [&](const opr_attn_in &a, void *o, void *ws, size_t wsb) {
    return opr_attn_fwd(&a, o, static_cast<float *>(FAKE), ws, wsb, nullptr);
  };
  auto bwd = [&](const opr_attn_in &a, void *o, void *dout, void *dq, void *ws, size_t wsb) {
    return opr_attn_bwd(&a, o, static_cast<float *>(FAKE), dout, static_cast<float *>(dq),
                        static_cast<float *>(FAKE), static_cast<float *>(FAKE), ws, wsb, nullptr);
  };
  CHECK(opr_attn_fwd(nullptr, FAKE, static_cast<float *>(FAKE), FAKE, big, nullptr) == OPR_E_INVALID);
  opr_attn_in a = attn_in();
  CHECK(fwd(a, FAKE, FAKE, 1024) == OPR_E_CAPACITY);
  CHECK(bwd(a, FAKE, FAKE, FAKE, FAKE, 1024) == OPR_E_CAPACITY);
  a.D = 96;
  CHECK(fwd(a, FAKE, FAKE, big) == OPR_E_UNSUPPORTED);
  a = attn_in(); a.Hq = 6; a.Hkv = 4;
  CHECK(bwd(a, FAKE, FAKE, FAKE, FAKE, big) == OPR_E_INVALID);
  a = attn_in(); a.rope_theta = std::nan("");
  CHECK(fwd(a, FAKE, FAKE, big) == OPR_E_INVALID);
  a = attn_in(); a.softmax_scale = -1.0f;
  CHECK(fwd(a, FAKE, FAKE, big) == OPR_E_INVALID);
  a = attn_in(); a.layout.order = OPR_ORDER_PACKED;
  CHECK(fwd(a, FAKE, FAKE, big) == OPR_E_INVALID);
  a = attn_in(); a.block_q = 64;
  CHECK(fwd(a, FAKE, FAKE, big) == OPR_E_UNSUPPORTED);
  a = attn_in(); a.B = 70000;
  CHECK(fwd(a, FAKE, FAKE, big) == OPR_E_UNSUPPORTED);
  a = attn_in(); a.L = std::numeric_limits<int32_t>::max(); a.B = 2;
  CHECK(fwd(a, FAKE, FAKE, big) == OPR_E_UNSUPPORTED);
  a = attn_in(); a.Hq = 512; a.Hkv = 1;
  CHECK(fwd(a, FAKE, FAKE, big) == OPR_E_UNSUPPORTED);  // 512 q heads per kv head
  for (size_t off : {2, 4, 8}) {
    a = attn_in(); a.q = fake(off);
    CHECK(fwd(a, FAKE, FAKE, big) == OPR_E_INVALID);
    a = attn_in(); a.k = fake(off);
    CHECK(bwd(a, FAKE, FAKE, FAKE, FAKE, big) == OPR_E_INVALID);
    a = attn_in(); a.v = fake(off);
    CHECK(fwd(a, FAKE, FAKE, big) == OPR_E_INVALID);
  }
  a = attn_in();
  CHECK(fwd(a, fake(8), FAKE, big) == OPR_E_INVALID);
  CHECK(fwd(a, FAKE, fake(16), big) == OPR_E_INVALID);
  CHECK(bwd(a, FAKE, fake(4), FAKE, FAKE, big) == OPR_E_INVALID);
  CHECK(bwd(a, FAKE, FAKE, fake(4), FAKE, big) == OPR_E_INVALID);
  CHECK(bwd(a, FAKE, FAKE, nullptr, FAKE, big) == OPR_E_INVALID);
  CHECK(bwd(a, FAKE, FAKE, FAKE, fake(128), big) == OPR_E_INVALID);
  const size_t f = opr_attn_workspace_size(2, 16384, 32, 8, 128, 0), b = opr_attn_workspace_size(2, 16384, 32, 8, 128, 1);
  CHECK(f > 0 && b > f);
  CHECK(opr_attn_workspace_size(1, 100, 3, 2, 128, 0) == 0);
  CHECK(opr_attn_workspace_size(65535, 32767, 1024, 1, 128, 1) == 0);
  CHECK(opr_attn_workspace_size(8, 262144, 64, 8, 128, 1) > (size_t)1 << 36);
}

static void other_checks() {
  // loss step
  CHECK(opr_token_ce(1, 64, 100, 32, FAKE, FAKE, static_cast<int32_t *>(FAKE), static_cast<uint8_t *>(FAKE), 1.0f,
                     static_cast<float *>(FAKE), nullptr, nullptr, 0, nullptr) == OPR_E_UNSUPPORTED);
  CHECK(opr_token_ce(1, 64, 128, 33, FAKE, FAKE, static_cast<int32_t *>(FAKE), static_cast<uint8_t *>(FAKE), 1.0f,
                     static_cast<float *>(FAKE), nullptr, nullptr, 0, nullptr) == OPR_E_UNSUPPORTED);
  CHECK(opr_token_ce(1, 64, 128, 32, fake(8), FAKE, static_cast<int32_t *>(FAKE), static_cast<uint8_t *>(FAKE), 1.0f,
                     static_cast<float *>(FAKE), nullptr, nullptr, 0, nullptr) == OPR_E_INVALID);
  CHECK(opr_token_ce(1, 64, 128, 32, FAKE, FAKE, static_cast<int32_t *>(FAKE), static_cast<uint8_t *>(FAKE),
                     INFINITY, static_cast<float *>(FAKE), nullptr, nullptr, 0, nullptr) == OPR_E_INVALID);
  CHECK(opr_token_ce(1, 64, 128, 32, FAKE, FAKE, static_cast<int32_t *>(FAKE), static_cast<uint8_t *>(FAKE), 1.0f,
                     static_cast<float *>(FAKE), FAKE, FAKE, 16, nullptr) == OPR_E_CAPACITY);
  CHECK(opr_token_ce_workspace_size(2, 16384, 4096, 32) > 0);
  CHECK(opr_token_ce_workspace_size(2, 16384, 4000, 32) == 0);
  // attention block
  opr_block_in bi{};
  bi.B = 1; bi.L = 256; bi.Hq = 4; bi.Hkv = 2; bi.D = 128; bi.d_model = 256;
  bi.rope_theta = 1e6; bi.norm_eps = 1e-6f;
  bi.x = bi.w_qkv = bi.w_o = FAKE;
  bi.g_q = bi.g_k = static_cast<float *>(FAKE);
  bi.layout = fake_layout();
  bi.block_q = bi.block_k = 128;
  CHECK(opr_block_fwd(&bi, FAKE, FAKE, FAKE, static_cast<float *>(FAKE), FAKE, 1024, nullptr) == OPR_E_CAPACITY);
  CHECK(opr_block_fwd(&bi, FAKE, FAKE, FAKE, static_cast<float *>(FAKE), fake(16), (size_t)1 << 40, nullptr) ==
        OPR_E_INVALID);
  opr_block_in bx = bi;
  bx.d_model = 100;
  CHECK(opr_block_fwd(&bx, FAKE, FAKE, FAKE, static_cast<float *>(FAKE), FAKE, (size_t)1 << 40, nullptr) ==
        OPR_E_INVALID);
  bx = bi;
  bx.norm_eps = 0.0f;
  CHECK(opr_block_bwd(&bx, FAKE, FAKE, static_cast<float *>(FAKE), FAKE, FAKE, static_cast<float *>(FAKE),
                      static_cast<float *>(FAKE), static_cast<float *>(FAKE), static_cast<float *>(FAKE), FAKE,
                      (size_t)1 << 40, nullptr) == OPR_E_INVALID);
  CHECK(opr_block_workspace_size(2, 16384, 32, 8, 128, 4096, 1) > opr_block_workspace_size(2, 16384, 32, 8, 128, 4096, 0));
  CHECK(opr_block_workspace_size(2, 16384, 32, 8, 128, 100, 1) == 0);
  for (int s = -5; s <= 1; ++s) CHECK(opr_status_string(static_cast<opr_status>(s)) != nullptr);
}

static void plan_checks() {
  std::mt19937_64 rng(12345);
  auto U = [&](int lo, int hi) { return (int32_t)std::uniform_int_distribution<int>(lo, hi)(rng); };
  for (int it = 0; it < 300; ++it) {
    const int N = U(1, 40);
    std::vector<opr_turn> conv(N);
    int64_t total = 0;
    for (auto &t : conv) {
      t.h = U(0, 300); t.t = U(0, 2000); t.r_in = t.r_out = U(0, 500);
      total += t.h + t.t + t.r_in + t.r_out;
    }
    std::vector<opr_chunk> ch(N);
    int32_t n = 0;
    double cost = 0;
    const int32_t k = U(0, N);
    const int32_t cap = U(0, 2) == 0 ? 0 : (int32_t)(total / U(1, 4));
    const double w = U(0, 3) * 100.0;
    const opr_status st = opr_kpass_plan(conv.data(), N, k, cap, w, U(0, 1), ch.data(), &n, &cost);
    CHECK(st == OPR_OK || st == OPR_E_CAPACITY);
    if (st != OPR_OK) continue;
    CHECK(n >= 1 && n <= N && (k == 0 || n == k));
    int next = 0;
    double sum = 0;
    for (int i = 0; i < n; ++i) {
      CHECK(ch[i].first_turn == next && ch[i].n_turns >= 1);
      CHECK(cap == 0 || ch[i].tokens <= cap);
      next += ch[i].n_turns;
      sum += (double)ch[i].pairs + w * ch[i].tokens;
    }
    CHECK(next == N);
    CHECK(std::fabs(sum - cost) <= 1e-9 * std::max(1.0, cost));
  }
  // limits and invalid input
  std::vector<opr_turn> many(65537, opr_turn{1, 1, 1, 1});
  std::vector<opr_chunk> out(65537);
  int32_t n = 0;
  CHECK(opr_kpass_plan(many.data(), 65537, 0, 0, 0.0, 1, out.data(), &n, nullptr) == OPR_E_UNSUPPORTED);
  CHECK(opr_kpass_plan(many.data(), 3000, 2000, 0, 0.0, 1, out.data(), &n, nullptr) == OPR_E_UNSUPPORTED);
  CHECK(opr_kpass_plan(many.data(), 3000, 0, 0, 1.0, 1, out.data(), &n, nullptr) == OPR_OK);
  std::vector<opr_turn> huge(5, opr_turn{std::numeric_limits<int32_t>::max() / 4, 0, 0, 0});  // more than 2^31 tokens
  CHECK(opr_kpass_plan(huge.data(), 5, 0, 0, 0.0, 1, out.data(), &n, nullptr) == OPR_E_INVALID);
  CHECK(opr_kpass_plan(many.data(), 2, 0, 0, std::nan(""), 1, out.data(), &n, nullptr) == OPR_E_INVALID);
  CHECK(opr_kpass_plan(nullptr, 2, 0, 0, 0.0, 1, out.data(), &n, nullptr) == OPR_E_INVALID);
}

int main() {
  layout_checks();
  attn_checks();
  other_checks();
  plan_checks();
  std::printf("abi_checks: %d checks passed\n", g_checks);
  return 0;
}

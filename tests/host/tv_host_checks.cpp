// Host-side checks of libtreeverify's C ABI, built with AddressSanitizer:
// the argument checks of every entry point (each call below must return its
// error code before it touches a device), the workspace-size queries on bad
// shapes, the status strings, and the SpecPV host policy functions over many
// shapes and trees (their outputs checked against the definitions in
// treeverify.h).  No device is used: every pointer handed to a device call is
// null or the call is rejected first.
#include <stdio.h>
#include <string.h>

#include <random>
#include <vector>

#include "treeverify.h"

static int g_fail = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);      \
      ++g_fail;                                                             \
    }                                                                       \
  } while (0)

static void status_strings() {
  for (int s = -3; s < 64; ++s) {
    const char* m = tv_status_string((tv_status)s);
    EXPECT(m != nullptr && strlen(m) > 0);
  }
  EXPECT(tv_version() > 0);
}

static void attention_checks() {
  tv_attn_desc d;
  memset(&d, 0, sizeof(d));
  EXPECT(tv_tree_attention_workspace_size(nullptr) == 0);
  EXPECT(tv_tree_attention(nullptr, nullptr, nullptr, 0, nullptr, nullptr) == TV_ERR_NULL);
  d.batch = 1;
  d.n_nodes = 0;  // no nodes
  d.n_q_heads = 8;
  d.n_kv_heads = 2;
  d.head_dim = 128;
  EXPECT(tv_tree_attention_workspace_size(&d) == 0);
  EXPECT(tv_tree_attention(&d, nullptr, nullptr, 0, nullptr, nullptr) != TV_OK);
  d.n_nodes = TV_MAX_NODES + 1;
  EXPECT(tv_tree_attention_workspace_size(&d) == 0);
  d.n_nodes = 16;
  d.head_dim = 96;  // unsupported head size
  EXPECT(tv_tree_attention(&d, nullptr, nullptr, 0, nullptr, nullptr) != TV_OK);
  d.head_dim = 128;
  d.n_q_heads = 7;  // not a multiple of the kv heads
  EXPECT(tv_tree_attention_workspace_size(&d) == 0);
  d.n_q_heads = 8;
  d.cache_capacity = 64;
  d.max_prefix_len = 65;  // past the capacity
  EXPECT(tv_tree_attention_workspace_size(&d) == 0);
  d.max_prefix_len = 64;
  d.softmax_scale = -1.f;
  EXPECT(tv_tree_attention_workspace_size(&d) == 0);
  d.softmax_scale = 0.f;
  // a valid descriptor with no operands: rejected for the null pointers
  tv_attn_ptrs p;
  memset(&p, 0, sizeof(p));
  EXPECT(tv_tree_attention(&d, &p, nullptr, 0, nullptr, nullptr) == TV_ERR_NULL);
  // (the no-alloc call looks up its device array first: no device, no call)
  EXPECT(tv_tree_attention_noalloc(&d, &p, nullptr, nullptr) != TV_OK);
  EXPECT(tv_tree_attention_noalloc(nullptr, &p, nullptr, nullptr) != TV_OK);
}

static void mask_checks() {
  int32_t parents[4] = {-1, 0, 0, 1};
  uint32_t mask[4];
  EXPECT(tv_build_tree_mask(nullptr, 1, 4, mask, nullptr, nullptr, nullptr) == TV_ERR_NULL);
  EXPECT(tv_build_tree_mask(parents, 1, 4, nullptr, nullptr, nullptr, nullptr) == TV_ERR_NULL);
  EXPECT(tv_build_tree_mask(parents, -1, 4, mask, nullptr, nullptr, nullptr) == TV_ERR_SHAPE);
  EXPECT(tv_build_tree_mask(parents, 1, 0, mask, nullptr, nullptr, nullptr) == TV_ERR_SHAPE);
  EXPECT(tv_build_tree_mask(parents, 1, TV_MAX_NODES + 1, mask, nullptr, nullptr, nullptr) ==
         TV_ERR_SHAPE);
}

static void accept_checks() {
  const int32_t dummy[8] = {0};
  int32_t out[8];
  EXPECT(tv_greedy_accept_workspace_size(-1, 4, 100) == 0);
  EXPECT(tv_greedy_accept_workspace_size(1, 0, 100) == 0);
  EXPECT(tv_greedy_accept_workspace_size(1, 4, 0) == 0);
  EXPECT(tv_greedy_accept_workspace_size(1, 4, 1000) > 0);
  EXPECT(tv_stochastic_accept_workspace_size(1, TV_MAX_NODES + 1, 100) == 0);
  EXPECT(tv_stochastic_accept_workspace_size(2, 60, 128256) > 0);
  EXPECT(tv_greedy_accept(nullptr, TV_BF16, 100, 100, dummy, dummy, 1, 4, out, out, out, out,
                          nullptr, 0, nullptr, nullptr) == TV_ERR_NULL);
  // wrong dtype / shapes, with host addresses that no check lets through
  EXPECT(tv_greedy_accept(dummy, (tv_dtype)77, 100, 100, dummy, dummy, 1, 4, out, out, out, out,
                          out, 0, nullptr, nullptr) == TV_ERR_UNSUPPORTED);
  EXPECT(tv_greedy_accept(dummy, TV_BF16, 100, 99, dummy, dummy, 1, 4, out, out, out, out, out, 0,
                          nullptr, nullptr) == TV_ERR_SHAPE);
  EXPECT(tv_greedy_accept(dummy, TV_BF16, 100, 100, dummy, dummy, 1, 4, out, out, out, out, out, 0,
                          nullptr, nullptr) == TV_ERR_WORKSPACE);
  EXPECT(tv_stochastic_accept(dummy, TV_BF16, 100, 100, dummy, dummy, 1, 4, 0.f, 0, 0, 0, out, out,
                              out, out, 1 << 20, nullptr, nullptr) == TV_ERR_SHAPE);
  EXPECT(tv_stochastic_accept_filtered(dummy, TV_BF16, 100, 100, dummy, dummy, 1, 4, 1.f, -1, 1.f,
                                       0, 0, 0, out, out, out, out, 1 << 20, nullptr,
                                       nullptr) == TV_ERR_SHAPE);
  EXPECT(tv_stochastic_accept_filtered(dummy, TV_BF16, 100, 100, dummy, dummy, 1, 4, 1.f, 5, 1.5f,
                                       0, 0, 0, out, out, out, out, 1 << 20, nullptr,
                                       nullptr) == TV_ERR_SHAPE);
  EXPECT(tv_stochastic_accept_filtered(dummy, TV_BF16, 100, 100, dummy, dummy, 1, 4, 1.f, 5, 0.f,
                                       0, 0, 0, out, out, out, out, 1 << 20, nullptr,
                                       nullptr) == TV_ERR_SHAPE);
  EXPECT(tv_stochastic_accept_filtered(dummy, TV_BF16, 100, 100, dummy, dummy, 1, 4, 1.f, 5, 0.9f,
                                       0, 0, 0, out, out, out, out, 0, nullptr, nullptr) ==
         TV_ERR_WORKSPACE);
}

static void commit_checks() {
  const int32_t dummy[8] = {0};
  int32_t out[8];
  EXPECT(tv_commit_kv(nullptr, dummy, dummy, dummy, dummy, out, out, out, 1024, 8, 1, 4, 1, 128,
                      nullptr, nullptr) == TV_ERR_NULL);
  EXPECT(tv_commit_kv(dummy, dummy, dummy, dummy, dummy, out, out, out, 1024, 8, 1, 4, 1, 96,
                      nullptr, nullptr) == TV_ERR_UNSUPPORTED);
  EXPECT(tv_commit_kv(dummy, dummy, dummy, dummy, dummy, out, out, out, 100, 8, 1, 4, 1, 128,
                      nullptr, nullptr) == TV_ERR_SHAPE);  // row stride below cap * head_dim
  EXPECT(tv_block_summaries(nullptr, 1024, 8, 1, 1, 128, 16, dummy, nullptr, 0, out, nullptr,
                            nullptr) == TV_ERR_NULL);
  EXPECT(tv_select_blocks_workspace_size(nullptr) == 0);
}

// SpecPV: the rectifying tree against its definition, over random trees
static void specpv_checks() {
  EXPECT(tv_specpv_needs_rectification(-1, 20) == -1);
  EXPECT(tv_specpv_needs_rectification(20, 20) == 0);
  EXPECT(tv_specpv_needs_rectification(21, 20) == 1);
  std::mt19937 rng(7);
  for (int trial = 0; trial < 2000; ++trial) {
    const int nb = 1 + (int)(rng() % 40), nd = 1 + (int)(rng() % (TV_MAX_NODES - nb));
    std::vector<int32_t> buf(nb), par(nd), tok(nd);
    for (auto& x : buf) x = (int32_t)(rng() % 128256);
    par[0] = -1;
    for (int j = 1; j < nd; ++j) par[j] = (int32_t)(rng() % j);
    for (auto& x : tok) x = (int32_t)(rng() % 128256);
    // outputs sized exactly: ASan catches a write past them
    std::vector<int32_t> po(nb + nd), to(nb + nd);
    const int32_t root = 42;
    EXPECT(tv_specpv_rectify_tree(buf.data(), nb, root, par.data(), tok.data(), nd, po.data(),
                                  to.data()) == TV_OK);
    for (int i = 0; i < nb; ++i) {
      EXPECT(po[i] == i - 1);
      EXPECT(to[i] == buf[i]);
    }
    EXPECT(po[nb] == nb - 1 && to[nb] == root);
    for (int j = 1; j < nd; ++j) {
      EXPECT(po[nb + j] == nb + par[j]);
      EXPECT(to[nb + j] == tok[j]);
    }
  }
  int32_t b1[1] = {5}, p1[2] = {-1, 0}, t1[2] = {1, 2}, po[4], to[4];
  EXPECT(tv_specpv_rectify_tree(nullptr, 1, 0, p1, t1, 2, po, to) == TV_ERR_NULL);
  EXPECT(tv_specpv_rectify_tree(b1, 0, 0, p1, t1, 2, po, to) == TV_ERR_SHAPE);
  EXPECT(tv_specpv_rectify_tree(b1, 1, 0, p1, t1, 0, po, to) == TV_ERR_SHAPE);
  EXPECT(tv_specpv_rectify_tree(b1, TV_MAX_NODES, 0, p1, t1, 2, po, to) == TV_ERR_SHAPE);
  int32_t bad[2] = {-1, 1};  // a node its own parent
  EXPECT(tv_specpv_rectify_tree(b1, 1, 0, bad, t1, 2, po, to) == TV_ERR_SHAPE);
  int32_t noroot[2] = {0, 0};
  EXPECT(tv_specpv_rectify_tree(b1, 1, 0, noroot, t1, 2, po, to) == TV_ERR_SHAPE);
}

int main() {
  status_strings();
  attention_checks();
  mask_checks();
  accept_checks();
  commit_checks();
  specpv_checks();
  if (g_fail) {
    fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}

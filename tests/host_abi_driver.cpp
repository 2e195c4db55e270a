// Host-side exercise of the C ABI for the sanitizer build (tests/test_host_sanitizers.py): every
// pure host function over a grid of shapes, and every entry point on arguments that validation
// rejects, so that nothing reaches a kernel launch.  Exits 0 when every status is the expected one;
// the sanitizers abort on the first memory or undefined-behaviour error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "tsa.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

static tsa_shape shape(int64_t L, int Hq, int Hkv, int d, int q, float tau, int dtype) {
  tsa_shape s;
  s.L = L; s.Hq = Hq; s.Hkv = Hkv; s.d = d; s.q = q; s.tau = tau; s.dtype = dtype;
  return s;
}

int main() {
  // status strings, including unknown codes
  for (int c = -3; c < 12; ++c)
    if (tsa_status_string(c) == nullptr) { std::fprintf(stderr, "null status string %d\n", c); ++failures; }

  // argument checks and sizes over a grid of shapes, valid and not
  const int64_t Ls[] = {0, 1, 2, 37, 255, 256, 257, 1000, 32768, 32769, 131072, (int64_t)1 << 24,
                        ((int64_t)1 << 24) + 1, -5};
  const int Hs[][2] = {{1, 1}, {4, 2}, {32, 8}, {8, 3}, {1024, 1}, {1025, 1}, {0, 1}, {2, 4}};
  const int ds[] = {32, 64, 128, 256};
  const int qs[] = {0, 1, 16, 1024, 1025};
  const float taus[] = {0.f, 0.005f, 0.999f, 1.f, -0.1f, NAN};
  size_t checked = 0;
  for (int64_t L : Ls)
    for (auto& h : Hs)
      for (int d : ds)
        for (int q : qs)
          for (float tau : taus)
            for (int dt = -1; dt < 3; ++dt) {
              const tsa_shape s = shape(L, h[0], h[1], d, q, tau, dt);
              const int st = tsa_check_args(&s);
              const size_t a = tsa_stage_workspace_bytes(&s), b = tsa_layer_workspace_bytes(&s),
                           c = tsa_dense_workspace_bytes(&s), e = tsa_block_select_workspace_bytes(&s),
                           f = tsa_layer_block_sparse_workspace_bytes(&s);
              if (st != TSA_OK && (a | b | c)) { std::fprintf(stderr, "size for an invalid shape\n"); ++failures; }
              if (st == TSA_OK && (a == 0 || b == 0 || c == 0)) { std::fprintf(stderr, "zero size\n"); ++failures; }
              (void)e; (void)f;
              ++checked;
            }
  expect(tsa_check_args(nullptr), TSA_ERR_ARG, "check_args(NULL)");
  for (int64_t L : Ls)
    if (L >= 0) { (void)tsa_capacity(L); (void)tsa_block_count(L); }

  // varlen host rules: capacities and workspaces of well-formed and malformed batches, and a batch
  // of more samples than one attention launch takes
  std::vector<int64_t> cu = {0};
  for (int b = 0; b < 40; ++b) cu.push_back(cu.back() + 17 + 13 * b);
  const tsa_shape sv = shape(cu.back(), 8, 2, 128, 4, 0.05f, TSA_BF16);
  if (tsa_varlen_capacity(40, cu.data()) <= 0) { std::fprintf(stderr, "varlen capacity\n"); ++failures; }
  if (tsa_layer_varlen_workspace_bytes(&sv, 40, cu.data()) == 0) { std::fprintf(stderr, "varlen ws\n"); ++failures; }
  if (tsa_dense_varlen_workspace_bytes(&sv, 40, cu.data()) == 0) { std::fprintf(stderr, "dense varlen ws\n"); ++failures; }
  const int64_t bad1[] = {0, 5, 5}, bad2[] = {1, 5}, bad3[] = {0, 9, 3};
  if (tsa_varlen_capacity(2, bad1) != -1 || tsa_varlen_capacity(1, bad2) != -1 || tsa_varlen_capacity(2, bad3) != -1) {
    std::fprintf(stderr, "malformed cu accepted\n");
    ++failures;
  }
  expect((int)tsa_varlen_capacity(0, cu.data()), -1, "varlen_capacity(B = 0)");
  if (tsa_layer_varlen_workspace_bytes(&sv, 2, bad1) != 0) { std::fprintf(stderr, "ws for a bad batch\n"); ++failures; }

  // entry points on rejected arguments (none gets as far as a launch)
  const tsa_shape s = shape(4096, 32, 8, 128, 16, 0.005f, TSA_BF16);
  tsa_shape bad = s;
  bad.tau = 2.f;
  alignas(256) static unsigned char buf[1 << 12];
  void* p = buf;                       // aligned; never dereferenced on these paths
  void* mis = buf + 2;
  int32_t* ip = reinterpret_cast<int32_t*>(buf);
  int32_t* imis = reinterpret_cast<int32_t*>(buf + 2);
  float* fp = reinterpret_cast<float*>(buf);
  uint16_t* up16 = reinterpret_cast<uint16_t*>(buf);

  expect(tsa_score(&s, nullptr, p, fp, fp, p, 1 << 30, nullptr), TSA_ERR_ARG, "score: Q NULL");
  expect(tsa_score(&s, mis, p, fp, fp, p, 1 << 30, nullptr), TSA_ERR_ALIGN, "score: Q misaligned");
  expect(tsa_score(&s, p, p, fp, fp, nullptr, 0, nullptr), TSA_ERR_WORKSPACE, "score: no workspace");
  expect(tsa_score(&s, p, p, fp, fp, p, 16, nullptr), TSA_ERR_WORKSPACE, "score: small workspace");
  expect(tsa_score(&bad, p, p, fp, fp, p, 1 << 30, nullptr), TSA_ERR_ARG, "score: tau");
  expect(tsa_budget(&s, nullptr, ip, ip, p, 1 << 30, nullptr), TSA_ERR_ARG, "budget: s_l NULL");
  expect(tsa_budget(&s, fp, imis, ip, p, 1 << 30, nullptr), TSA_ERR_ALIGN, "budget: k misaligned");
  expect(tsa_budget(&s, fp, ip, ip, mis, 1 << 30, nullptr), TSA_ERR_WORKSPACE, "budget: workspace misaligned");
  expect(tsa_select(&s, fp, nullptr, ip, ip, p, 1 << 30, nullptr), TSA_ERR_ARG, "select: Lp NULL");
  expect(tsa_select(&s, fp, imis, ip, ip, p, 1 << 30, nullptr), TSA_ERR_ALIGN, "select: Lp misaligned");
  expect(tsa_select(&s, fp, ip, ip, ip, nullptr, 0, nullptr), TSA_ERR_WORKSPACE, "select: no workspace");
  expect(tsa_gather(&s, p, p, p, ip, nullptr, p, p, p, nullptr), TSA_ERR_ARG, "gather: Lp NULL");
  expect(tsa_gather(&s, p, p, p, ip, ip, mis, p, p, nullptr), TSA_ERR_ALIGN, "gather: Qh misaligned");
  expect(tsa_attn_causal(&bad, p, p, p, ip, p, nullptr), TSA_ERR_ARG, "attn: tau");
  expect(tsa_attn_causal(&s, p, p, nullptr, ip, p, nullptr), TSA_ERR_ARG, "attn: Vht NULL");
  expect(tsa_scatter_residual(&s, p, nullptr, nullptr, ip, nullptr, p, nullptr), TSA_ERR_ARG, "scatter: no idx, no inv");
  expect(tsa_scatter_residual(&s, p, ip, ip, ip, mis, p, nullptr), TSA_ERR_ALIGN, "scatter: X misaligned");
  expect(tsa_layer(&s, p, p, p, nullptr, nullptr, ip, p, 1 << 30, nullptr), TSA_ERR_ARG, "layer: Y NULL");
  expect(tsa_layer(&s, p, p, p, nullptr, p, imis, p, 1 << 30, nullptr), TSA_ERR_ALIGN, "layer: kLp misaligned");
  expect(tsa_layer(&s, p, p, p, nullptr, p, ip, p, 256, nullptr), TSA_ERR_WORKSPACE, "layer: small workspace");
  for (float sp : {-0.25f, 1.5f, NAN}) {
    expect(tsa_budget_ratio(&s, sp, ip, ip, nullptr), TSA_ERR_ARG, "budget_ratio: sparsity");
    expect(tsa_layer_ratio(&s, sp, p, p, p, nullptr, p, nullptr, p, 1 << 30, nullptr), TSA_ERR_ARG, "layer_ratio: sparsity");
  }
  expect(tsa_budget_ratio(&s, 0.3f, imis, ip, nullptr), TSA_ERR_ALIGN, "budget_ratio: k misaligned");
  expect(tsa_dense_attn_causal(&s, p, p, p, nullptr, p, nullptr, 0, nullptr), TSA_ERR_WORKSPACE, "dense: no workspace");
  expect(tsa_dense_attn_causal(&bad, p, p, p, nullptr, p, p, 1 << 30, nullptr), TSA_ERR_ARG, "dense: tau");
  for (float g : {-0.5f, NAN}) {
    expect(tsa_block_select(&s, g, p, p, ip, up16, ip, p, 1 << 30, nullptr), TSA_ERR_ARG, "block_select: gamma");
    expect(tsa_layer_block_sparse(&s, g, p, p, p, nullptr, p, nullptr, p, 1 << 30, nullptr), TSA_ERR_ARG,
           "layer_block_sparse: gamma");
  }
  const tsa_shape big = shape(524289, 8, 8, 128, 16, 0.005f, TSA_BF16);
  expect(tsa_attn_block_sparse(&big, p, p, p, ip, up16, ip, p, nullptr), TSA_ERR_UNSUPPORTED, "block sparse: too long");
  expect(tsa_block_select(&s, 0.9f, p, p, ip, up16, ip, nullptr, 0, nullptr), TSA_ERR_WORKSPACE, "block_select: no workspace");

  // varlen entry points on malformed batches and missing workspaces
  const int64_t short_q[] = {0, 3, 700, 1000};
  const tsa_shape s1000 = shape(1000, 4, 2, 128, 5, 0.05f, TSA_BF16);
  expect(tsa_layer_varlen(&s1000, 3, short_q, p, p, p, nullptr, p, nullptr, p, 1 << 30, nullptr), TSA_ERR_SHAPE,
         "layer_varlen: sample shorter than q");
  const int64_t wrong_total[] = {0, 37, 700, 999};
  expect(tsa_layer_varlen(&s1000, 3, wrong_total, p, p, p, nullptr, p, nullptr, p, 1 << 30, nullptr), TSA_ERR_ARG,
         "layer_varlen: total");
  expect(tsa_attn_causal_varlen(&s1000, 3, wrong_total, p, p, p, ip, p, nullptr), TSA_ERR_ARG, "attn_varlen: total");
  expect(tsa_layer_varlen(&sv, 40, cu.data(), p, p, p, nullptr, p, nullptr, nullptr, 0, nullptr), TSA_ERR_WORKSPACE,
         "layer_varlen: no workspace");
  expect(tsa_dense_attn_causal_varlen(&sv, 40, cu.data(), p, p, p, nullptr, p, nullptr, 0, nullptr), TSA_ERR_WORKSPACE,
         "dense_varlen: no workspace");
  expect(tsa_layer_varlen(&sv, 40, nullptr, p, p, p, nullptr, p, nullptr, p, 1 << 30, nullptr), TSA_ERR_ARG,
         "layer_varlen: cu NULL");

  std::printf("host ABI driver: %zu shapes checked, %d unexpected statuses\n", checked, failures);
  return failures ? 1 : 0;
}

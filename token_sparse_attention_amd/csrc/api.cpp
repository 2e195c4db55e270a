// C ABI of libtsa.so: argument validation (host only, before any launch), workspace carving and
// the stage-by-stage orchestration of the Token Sparse Attention prefill layer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "tsa.h"
#include "tsa_internal.h"

using namespace tsa;

namespace {

constexpr size_t kAlign = 256;

size_t up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
size_t elem_bytes(int dtype) { return dtype == TSA_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
hipStream_t stream_of(void* s) { return static_cast<hipStream_t>(s); }
int hip_status(hipError_t e) { return e == hipSuccess ? TSA_OK : TSA_ERR_HIP; }

// Offsets (bytes) of the stage workspace; each region 256-byte aligned.
struct StageWs {
  size_t partials, rowstat, S, tilesum, bhist, bctl, kLp, shist, sctl, tcnt, toff, total;
};

StageWs stage_layout(const tsa_shape* s) {
  StageWs w;
  size_t o = 0;
  auto take = [&](size_t n) { size_t at = o; o += up(n); return at; };
  w.partials = take(score_partial_bytes(s->L, s->Hq, s->Hkv, s->q));
  w.rowstat = take(score_rowstat_bytes(s->Hq, s->Hkv, s->q));
  w.S = take((size_t)s->L * sizeof(double));
  w.tilesum = take((size_t)layer_tiles(s->L) * sizeof(double));
  w.bhist = take((size_t)kRadixPasses * 2 * kRadixBins * sizeof(uint64_t));
  w.bctl = take((size_t)kRadixPasses * sizeof(RadixCtl));
  w.kLp = take(2 * sizeof(int32_t));
  w.shist = take((size_t)s->Hq * kRadixPasses * 2 * kRadixBins * sizeof(uint64_t));
  w.sctl = take((size_t)s->Hq * kRadixPasses * sizeof(RadixCtl));
  w.tcnt = take((size_t)s->Hq * select_tiles(s->L) * 2 * sizeof(uint32_t));
  w.toff = take((size_t)s->Hq * select_tiles(s->L) * 2 * sizeof(uint32_t));
  w.total = o;
  return w;
}

// Block sparsity: key blocks per head, pooled means and kept-block lists.
int64_t block_count(const tsa_shape* s) { return tsa_capacity(s->L) / kBlock; }
size_t pooled_bytes(const tsa_shape* s) { return (size_t)s->Hq * block_count(s) * s->d * sizeof(float); }
size_t list_bytes(const tsa_shape* s) { return (size_t)s->Hq * block_count(s) * block_count(s) * sizeof(uint16_t); }
size_t count_bytes(const tsa_shape* s) { return (size_t)s->Hq * block_count(s) * sizeof(int32_t); }
size_t logits_bytes(const tsa_shape* s) { return (size_t)s->Hq * block_count(s) * block_count(s) * sizeof(double); }

// The bf16 layer without block sparsity reads its query and key rows through idx inside the
// attention and writes Y from the attention's epilogue, so it never materialises Q_hat, K_hat or
// O_hat (only V_hat^T, which the matrix cores take transposed).
bool fused_layer(const tsa_shape* s, bool block_sparse) { return s->dtype == TSA_BF16 && !block_sparse; }

// The layer workspace = stage workspace + every intermediate tensor the layer materialises (+ the
// pooled means and block lists of the block-sparse variant).  Offsets of regions a variant does not
// use are 0 and never read.
struct LayerWs {
  StageWs st;
  size_t s_h, s_l, idx, inv, Qh, Kh, Vht, Oh;
  size_t qbar, kbar, zl, blist, bcnt, total;
};

LayerWs layer_layout(const tsa_shape* s, bool block_sparse) {
  LayerWs w{};
  w.st = stage_layout(s);
  size_t o = w.st.total;
  auto take = [&](size_t n) { size_t at = o; o += up(n); return at; };
  const size_t C = (size_t)tsa_capacity(s->L);
  const size_t hl = (size_t)s->Hq * s->L;
  const size_t comp = (size_t)s->Hq * C * s->d * elem_bytes(s->dtype);
  const bool fused = fused_layer(s, block_sparse);
  w.s_h = take(hl * sizeof(float));
  w.s_l = take((size_t)s->L * sizeof(float));
  w.idx = take(hl * sizeof(int32_t));
  w.inv = take(hl * sizeof(int32_t));
  if (!fused) w.Qh = take(comp);
  if (!fused) w.Kh = take(comp);
  w.Vht = take(comp);
  if (!fused) w.Oh = take(comp);
  if (block_sparse) {
    w.qbar = take(pooled_bytes(s));
    w.kbar = take(pooled_bytes(s));
    w.zl = take(logits_bytes(s));
    w.blist = take(list_bytes(s));
    w.bcnt = take(count_bytes(s));
  }
  w.total = o;
  return w;
}

template <typename T> T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }

int check_ws(void* ws, size_t have, size_t need) {
  if (ws == nullptr || ((uintptr_t)ws & (kAlign - 1)) != 0 || have < need) return TSA_ERR_WORKSPACE;
  return TSA_OK;
}

#define TSA_TRY(expr)                 \
  do {                                \
    const int st_ = (expr);           \
    if (st_ != TSA_OK) return st_;    \
  } while (0)

int need_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (p == nullptr) return TSA_ERR_ARG;
    if (!aligned16(p)) return TSA_ERR_ALIGN;
  }
  return TSA_OK;
}

int opt_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p != nullptr && !aligned16(p)) return TSA_ERR_ALIGN;
  return TSA_OK;
}

int need_int_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (p == nullptr) return TSA_ERR_ARG;
    if (((uintptr_t)p & 3u) != 0) return TSA_ERR_ALIGN;
  }
  return TSA_OK;
}

uint64_t budget_target(float tau) {
  // ceil(tau * 2^60): the integer fixed-point mass that "C(j) >= tau" must reach.
  return (uint64_t)std::ceil(std::ldexp((double)tau, 60));
}

// ---- varlen batches ------------------------------------------------------------------------------

int check_varlen(const tsa_shape* s, int32_t B, const int64_t* cu) {
  TSA_TRY(tsa_check_args(s));
  if (B < 1 || cu == nullptr || cu[0] != 0 || cu[B] != s->L) return TSA_ERR_ARG;
  for (int32_t b = 0; b < B; ++b) {
    if (cu[b + 1] <= cu[b]) return TSA_ERR_ARG;
    if (cu[b + 1] - cu[b] < s->q) return TSA_ERR_SHAPE;
  }
  return TSA_OK;
}

// One sequence of the batch viewed as a single-sequence problem.
tsa_shape sample_shape(const tsa_shape* s, const int64_t* cu, int32_t b) {
  tsa_shape t = *s;
  t.L = cu[b + 1] - cu[b];
  return t;
}

int64_t max_len(int32_t B, const int64_t* cu) {
  int64_t m = 0;
  for (int32_t b = 0; b < B; ++b) m = std::max(m, cu[b + 1] - cu[b]);
  return m;
}

int64_t varlen_capacity(int32_t B, const int64_t* cu) {
  int64_t P = 0;
  for (int32_t b = 0; b < B; ++b) P += tsa_capacity(cu[b + 1] - cu[b]);
  return P;
}

// Sequences in launch order: longest first (they hold the heaviest query blocks).
std::vector<int32_t> longest_first(int32_t B, const int64_t* cu) {
  std::vector<int32_t> order(B);
  for (int32_t b = 0; b < B; ++b) order[b] = b;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return cu[x + 1] - cu[x] > cu[y + 1] - cu[y]; });
  return order;
}

// Workspace of tsa_layer_varlen: one stage workspace for the longest sample (reused sample after
// sample on the stream) + per-sample {k, L'} pairs + the batch's intermediates.
struct VarlenWs {
  StageWs st;
  size_t kLp, s_h, s_l, idx, inv, Qh, Kh, Vht, Oh, total;
};

VarlenWs varlen_layout(const tsa_shape* s, int32_t B, const int64_t* cu) {
  VarlenWs w;
  tsa_shape big = *s;
  big.L = max_len(B, cu);
  w.st = stage_layout(&big);
  size_t o = w.st.total;
  auto take = [&](size_t n) { size_t at = o; o += up(n); return at; };
  // per-sample regions of the score and index arrays start at the capacity offsets P_b (multiples
  // of 256 rows) like the compressed tensors, so every region is aligned whatever the lengths
  const size_t P = (size_t)varlen_capacity(B, cu);
  const size_t comp = (size_t)s->Hq * P * s->d * elem_bytes(s->dtype);
  w.kLp = take((size_t)B * 2 * sizeof(int32_t));
  w.s_h = take((size_t)s->Hq * P * sizeof(float));
  w.s_l = take(P * sizeof(float));
  w.idx = take((size_t)s->Hq * P * sizeof(int32_t));
  w.inv = take((size_t)s->Hq * P * sizeof(int32_t));
  const bool fused = fused_layer(s, false);
  w.Qh = fused ? 0 : take(comp);
  w.Kh = fused ? 0 : take(comp);
  w.Vht = take(comp);
  w.Oh = fused ? 0 : take(comp);
  w.total = o;
  return w;
}

// Stages 1-5 of the layer on one stream.  fixed_ratio selects the ablation's fixed budget
// (k = round(sparsity * L)) in place of the coverage budget; s_l is then not needed.
int run_layer(const tsa_shape* s, bool fixed_ratio, float sparsity, const void* Q, const void* K,
              const void* V, const void* X, void* Y, int32_t* kLp_dev, void* ws, size_t ws_bytes,
              void* stream, bool block_sparse = false, float gamma = 1.f) {
  TSA_TRY(layer_args(s, Q, K, V, X, Y, kLp_dev));
  if (block_sparse && block_count(s) > kMaxKeyBlocks) return TSA_ERR_UNSUPPORTED;
  const LayerWs w = layer_layout(s, block_sparse);
  TSA_TRY(check_ws(ws, ws_bytes, w.total));
  hipStream_t st = stream_of(stream);
  const StageWs& g = w.st;
  const int64_t C = tsa_capacity(s->L);
  float* s_h = at<float>(ws, w.s_h);
  float* s_l = at<float>(ws, w.s_l);
  int32_t* kLp = at<int32_t>(ws, g.kLp);
  int32_t* idx = at<int32_t>(ws, w.idx);
  int32_t* inv = at<int32_t>(ws, w.inv);
  // one clear covers the budget's and the selection's histograms and control words (and the two
  // layer words between them, which the budget writes before anything reads them); the one-workgroup
  // selects of short rows use neither
  hipError_t e = radix_resident(s->L) ? hipSuccess : launch_fill_zero(at<char>(ws, g.bhist), g.tcnt - g.bhist, st);
  if (e == hipSuccess)
    e = launch_score(s->dtype, s->d, Q, K, s->L, s->Hq, s->Hkv, s->q, s_h, at<double2>(ws, g.partials),
                     at<double2>(ws, g.rowstat), st);
  // a short row under tau: budget and selection in one launch
  const bool merged = !fixed_ratio && radix_resident(s->L);
  if (fixed_ratio) {
    if (e == hipSuccess)
      e = launch_budget_ratio(sparsity, s->L, kLp, kLp_dev, kLp_dev ? kLp_dev + 1 : nullptr, st);
  } else if (merged) {
    if (e == hipSuccess)
      e = launch_layer_budget_select(s_h, s->L, s->Hq, at<double>(ws, g.S), at<double>(ws, g.tilesum), s_l,
                                     budget_target(s->tau), kLp, kLp_dev, kLp_dev ? kLp_dev + 1 : nullptr, idx, inv,
                                     st);
  } else {
    if (e == hipSuccess)
      e = launch_layer_score_budget(s_h, s->L, s->Hq, at<double>(ws, g.S), at<double>(ws, g.tilesum), s_l,
                                    budget_target(s->tau), at<uint64_t>(ws, g.bhist), at<RadixCtl>(ws, g.bctl),
                                    kLp, kLp_dev, kLp_dev ? kLp_dev + 1 : nullptr, st);
  }
  if (e == hipSuccess && !merged)
    e = launch_select(s_h, s->L, s->Hq, kLp + 1, at<uint64_t>(ws, g.shist), at<RadixCtl>(ws, g.sctl),
                      at<uint32_t>(ws, g.tcnt), at<uint32_t>(ws, g.toff), idx, inv, st);
  // bf16 without block sparsity: the attention reads the query and key rows through idx and writes Y
  // itself (the gather of Q and K and the decompression folded into it; only V_hat^T is gathered);
  // the result is bitwise the same as gather -> attention -> scatter
  // (fused: the rows no head kept are written by the gather's launch too)
  const bool fused = fused_layer(s, block_sparse);
  if (e == hipSuccess)
    e = launch_gather(s->dtype, s->d, Q, K, V, idx, kLp + 1, s->L, s->Hq, s->Hkv, C,
                      fused ? nullptr : at<void>(ws, w.Qh), fused ? nullptr : at<void>(ws, w.Kh), at<void>(ws, w.Vht),
                      st, fused ? inv : nullptr, fused ? X : nullptr, fused ? Y : nullptr);
  if (fused) {
    if (e == hipSuccess) {
      const AttnSeqDesc one{0, 0, s->L, C, kLp + 1, idx};
      e = launch_attention_varlen(s->dtype, s->d, false, Q, K, at<void>(ws, w.Vht), 1, &one, s->Hq, s->Hkv, X, Y, st,
                                  true);
    }
    return hip_status(e);
  }
  if (block_sparse) {
    if (e == hipSuccess)
      e = launch_block_select(s->dtype, s->d, at<void>(ws, w.Qh), at<void>(ws, w.Kh), kLp + 1, C, s->Hq, (double)gamma,
                              at<float>(ws, w.qbar), at<float>(ws, w.kbar), at<double>(ws, w.zl),
                              at<uint16_t>(ws, w.blist), at<int32_t>(ws, w.bcnt), st);
    if (e == hipSuccess)
      e = launch_attention_block_sparse(s->dtype, s->d, at<void>(ws, w.Qh), at<void>(ws, w.Kh), at<void>(ws, w.Vht),
                                        kLp + 1, s->L, s->Hq, s->Hkv, C, at<uint16_t>(ws, w.blist),
                                        at<int32_t>(ws, w.bcnt), at<void>(ws, w.Oh), st);
  } else if (e == hipSuccess) {
    e = launch_attention(s->dtype, s->d, false, at<void>(ws, w.Qh), at<void>(ws, w.Kh), at<void>(ws, w.Vht),
                         kLp + 1, s->L, s->Hq, s->Hkv, C, nullptr, at<void>(ws, w.Oh), st);
  }
  if (e == hipSuccess)
    e = launch_scatter(s->dtype, s->d, at<void>(ws, w.Oh), idx, inv, kLp + 1, X, Y, s->L, s->Hq, C, st);
  return hip_status(e);
}

}  // namespace

namespace tsa {

int layer_args(const tsa_shape* s, const void* Q, const void* K, const void* V, const void* X, const void* Y,
               const int32_t* kLp_dev) {
  TSA_TRY(tsa_check_args(s));
  TSA_TRY(need_ptrs({Q, K, V, Y}));
  TSA_TRY(opt_ptrs({X}));
  if (kLp_dev && ((uintptr_t)kLp_dev & 3u)) return TSA_ERR_ALIGN;
  return TSA_OK;
}

}  // namespace tsa

extern "C" {

const char* tsa_status_string(int status) {
  switch (status) {
    case TSA_OK: return "ok";
    case TSA_ERR_ARG: return "invalid argument";
    case TSA_ERR_SHAPE: return "unsupported shape";
    case TSA_ERR_DTYPE: return "unsupported dtype";
    case TSA_ERR_ALIGN: return "tensor not 16-byte aligned";
    case TSA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case TSA_ERR_HIP: return "HIP launch failed";
    case TSA_ERR_UNSUPPORTED: return "not implemented for these parameters";
    case TSA_ERR_TOO_LARGE: return "intermediates exceed the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

int tsa_check_args(const tsa_shape* s) {
  if (s == nullptr) return TSA_ERR_ARG;
  if (s->dtype != TSA_F32 && s->dtype != TSA_BF16) return TSA_ERR_DTYPE;
  if (!(s->tau >= 0.f && s->tau < 1.f)) return TSA_ERR_ARG;   // also rejects NaN
  // L <= 2^24: the attention kernels address a transposed value row of C tokens through 32-bit
  // buffer offsets ((d - 1) * 2C + 128 bytes must stay below 2^32)
  if (s->L < 1 || s->L > (int64_t(1) << 24)) return TSA_ERR_SHAPE;
  if (s->Hq < 1 || s->Hkv < 1 || s->Hq > 1024 || s->Hkv > s->Hq || s->Hq % s->Hkv != 0) return TSA_ERR_SHAPE;
  if (s->q < 1 || s->q > 1024 || (int64_t)s->q > s->L) return TSA_ERR_SHAPE;
  if (s->d != 64 && s->d != 128) return TSA_ERR_UNSUPPORTED;
  return TSA_OK;
}

int64_t tsa_capacity(int64_t L) { return (L + 255) / 256 * 256; }

size_t tsa_stage_workspace_bytes(const tsa_shape* s) {
  return tsa_check_args(s) == TSA_OK ? stage_layout(s).total : 0;
}

size_t tsa_layer_workspace_bytes(const tsa_shape* s) {
  return tsa_check_args(s) == TSA_OK ? layer_layout(s, false).total : 0;
}

size_t tsa_dense_workspace_bytes(const tsa_shape* s) {
  if (tsa_check_args(s) != TSA_OK) return 0;
  return up((size_t)s->Hkv * s->d * tsa_capacity(s->L) * elem_bytes(s->dtype));
}

int tsa_score(const tsa_shape* s, const void* Q, const void* K, float* s_h, float* s_l, void* ws,
              size_t ws_bytes, void* stream) {
  TSA_TRY(tsa_check_args(s));
  TSA_TRY(need_ptrs({Q, K, s_h}));
  TSA_TRY(opt_ptrs({s_l}));
  const StageWs w = stage_layout(s);
  TSA_TRY(check_ws(ws, ws_bytes, w.total));
  hipError_t e = launch_score(s->dtype, s->d, Q, K, s->L, s->Hq, s->Hkv, s->q, s_h,
                              at<double2>(ws, w.partials), at<double2>(ws, w.rowstat), stream_of(stream));
  if (e == hipSuccess && s_l)
    e = launch_layer_score(s_h, s->L, s->Hq, at<double>(ws, w.S), at<double>(ws, w.tilesum), s_l,
                           stream_of(stream));
  return hip_status(e);
}

int tsa_budget(const tsa_shape* s, const float* s_l, int32_t* k_dev, int32_t* Lp_dev, void* ws,
               size_t ws_bytes, void* stream) {
  TSA_TRY(tsa_check_args(s));
  TSA_TRY(need_ptrs({s_l}));
  if ((k_dev && ((uintptr_t)k_dev & 3u)) || (Lp_dev && ((uintptr_t)Lp_dev & 3u))) return TSA_ERR_ALIGN;
  const StageWs w = stage_layout(s);
  TSA_TRY(check_ws(ws, ws_bytes, w.total));
  hipStream_t st = stream_of(stream);
  hipError_t e = radix_resident(s->L) ? hipSuccess : launch_fill_zero(at<char>(ws, w.bhist), w.kLp - w.bhist, st);
  if (e == hipSuccess)
    e = launch_budget(s_l, s->L, budget_target(s->tau), at<uint64_t>(ws, w.bhist), at<RadixCtl>(ws, w.bctl),
                      at<int32_t>(ws, w.kLp), k_dev, Lp_dev, st);
  return hip_status(e);
}

int tsa_select(const tsa_shape* s, const float* s_h, const int32_t* Lp_dev, int32_t* idx, int32_t* inv,
               void* ws, size_t ws_bytes, void* stream) {
  TSA_TRY(tsa_check_args(s));
  TSA_TRY(need_ptrs({s_h, idx}));
  TSA_TRY(opt_ptrs({inv}));
  TSA_TRY(need_int_ptrs({Lp_dev}));
  const StageWs w = stage_layout(s);
  TSA_TRY(check_ws(ws, ws_bytes, w.total));
  hipStream_t st = stream_of(stream);
  hipError_t e = radix_resident(s->L) ? hipSuccess : launch_fill_zero(at<char>(ws, w.shist), w.tcnt - w.shist, st);
  if (e == hipSuccess)
    e = launch_select(s_h, s->L, s->Hq, Lp_dev, at<uint64_t>(ws, w.shist), at<RadixCtl>(ws, w.sctl),
                      at<uint32_t>(ws, w.tcnt), at<uint32_t>(ws, w.toff), idx, inv, st);
  return hip_status(e);
}

int tsa_gather(const tsa_shape* s, const void* Q, const void* K, const void* V, const int32_t* idx,
               const int32_t* Lp_dev, void* Qh, void* Kh, void* Vht, void* stream) {
  TSA_TRY(tsa_check_args(s));
  TSA_TRY(need_ptrs({Q, K, V, idx, Qh, Kh, Vht}));
  TSA_TRY(need_int_ptrs({Lp_dev}));
  return hip_status(launch_gather(s->dtype, s->d, Q, K, V, idx, Lp_dev, s->L, s->Hq, s->Hkv,
                                  tsa_capacity(s->L), Qh, Kh, Vht, stream_of(stream)));
}

int tsa_attn_causal(const tsa_shape* s, const void* Qh, const void* Kh, const void* Vht,
                    const int32_t* Lp_dev, void* Oh, void* stream) {
  TSA_TRY(tsa_check_args(s));
  TSA_TRY(need_ptrs({Qh, Kh, Vht, Oh}));
  TSA_TRY(need_int_ptrs({Lp_dev}));
  return hip_status(launch_attention(s->dtype, s->d, false, Qh, Kh, Vht, Lp_dev, s->L, s->Hq, s->Hkv,
                                     tsa_capacity(s->L), nullptr, Oh, stream_of(stream)));
}

int tsa_scatter_residual(const tsa_shape* s, const void* Oh, const int32_t* idx, const int32_t* inv,
                         const int32_t* Lp_dev, const void* X, void* Y, void* stream) {
  TSA_TRY(tsa_check_args(s));
  TSA_TRY(need_ptrs({Oh, Y}));
  TSA_TRY(opt_ptrs({X, inv}));
  if (inv == nullptr) {
    TSA_TRY(need_ptrs({idx}));
    TSA_TRY(need_int_ptrs({Lp_dev}));
  }
  return hip_status(launch_scatter(s->dtype, s->d, Oh, idx, inv, Lp_dev, X, Y, s->L, s->Hq,
                                   tsa_capacity(s->L), stream_of(stream)));
}

int tsa_layer(const tsa_shape* s, const void* Q, const void* K, const void* V, const void* X, void* Y,
              int32_t* kLp_dev, void* ws, size_t ws_bytes, void* stream) {
  return run_layer(s, false, 0.f, Q, K, V, X, Y, kLp_dev, ws, ws_bytes, stream);
}

int tsa_budget_ratio(const tsa_shape* s, float sparsity, int32_t* k_dev, int32_t* Lp_dev, void* stream) {
  TSA_TRY(tsa_check_args(s));
  if (!(sparsity >= 0.f && sparsity <= 1.f)) return TSA_ERR_ARG;   // also rejects NaN
  if ((k_dev && ((uintptr_t)k_dev & 3u)) || (Lp_dev && ((uintptr_t)Lp_dev & 3u))) return TSA_ERR_ALIGN;
  return hip_status(launch_budget_ratio(sparsity, s->L, nullptr, k_dev, Lp_dev, stream_of(stream)));
}

int tsa_layer_ratio(const tsa_shape* s, float sparsity, const void* Q, const void* K, const void* V,
                    const void* X, void* Y, int32_t* kLp_dev, void* ws, size_t ws_bytes, void* stream) {
  if (!(sparsity >= 0.f && sparsity <= 1.f)) return TSA_ERR_ARG;
  return run_layer(s, true, sparsity, Q, K, V, X, Y, kLp_dev, ws, ws_bytes, stream);
}

int tsa_dense_attn_causal(const tsa_shape* s, const void* Q, const void* K, const void* V, const void* X,
                          void* Y, void* ws, size_t ws_bytes, void* stream) {
  TSA_TRY(tsa_check_args(s));
  TSA_TRY(need_ptrs({Q, K, V, Y}));
  TSA_TRY(opt_ptrs({X}));
  TSA_TRY(check_ws(ws, ws_bytes, tsa_dense_workspace_bytes(s)));
  hipStream_t st = stream_of(stream);
  const int64_t C = tsa_capacity(s->L);
  hipError_t e = launch_transpose_v(s->dtype, s->d, V, s->L, s->Hkv, C, ws, st);
  if (e == hipSuccess)
    e = launch_attention(s->dtype, s->d, true, Q, K, ws, nullptr, s->L, s->Hq, s->Hkv, C, X, Y, st);
  return hip_status(e);
}

int64_t tsa_varlen_capacity(int32_t B, const int64_t* cu_seqlens) {
  if (B < 1 || cu_seqlens == nullptr || cu_seqlens[0] != 0) return -1;
  for (int32_t b = 0; b < B; ++b)
    if (cu_seqlens[b + 1] <= cu_seqlens[b]) return -1;
  return varlen_capacity(B, cu_seqlens);
}

size_t tsa_layer_varlen_workspace_bytes(const tsa_shape* s, int32_t B, const int64_t* cu_seqlens) {
  return check_varlen(s, B, cu_seqlens) == TSA_OK ? varlen_layout(s, B, cu_seqlens).total : 0;
}

size_t tsa_dense_varlen_workspace_bytes(const tsa_shape* s, int32_t B, const int64_t* cu_seqlens) {
  if (check_varlen(s, B, cu_seqlens) != TSA_OK) return 0;
  return up((size_t)s->Hkv * s->d * varlen_capacity(B, cu_seqlens) * elem_bytes(s->dtype));
}

int tsa_attn_causal_varlen(const tsa_shape* s, int32_t B, const int64_t* cu_seqlens, const void* Qh,
                           const void* Kh, const void* Vht, const int32_t* Lp_dev, void* Oh, void* stream) {
  TSA_TRY(check_varlen(s, B, cu_seqlens));
  TSA_TRY(need_ptrs({Qh, Kh, Vht, Oh}));
  TSA_TRY(need_int_ptrs({Lp_dev}));
  std::vector<AttnSeqDesc> seqs;
  std::vector<int64_t> P(B + 1, 0);
  for (int32_t b = 0; b < B; ++b) P[b + 1] = P[b] + tsa_capacity(cu_seqlens[b + 1] - cu_seqlens[b]);
  for (int32_t b : longest_first(B, cu_seqlens))
    seqs.push_back({cu_seqlens[b], P[b], cu_seqlens[b + 1] - cu_seqlens[b], P[b + 1] - P[b], Lp_dev + b, nullptr});
  return hip_status(launch_attention_varlen(s->dtype, s->d, false, Qh, Kh, Vht, B, seqs.data(), s->Hq, s->Hkv,
                                            nullptr, Oh, stream_of(stream)));
}

int tsa_dense_attn_causal_varlen(const tsa_shape* s, int32_t B, const int64_t* cu_seqlens, const void* Q,
                                 const void* K, const void* V, const void* X, void* Y, void* ws,
                                 size_t ws_bytes, void* stream) {
  TSA_TRY(check_varlen(s, B, cu_seqlens));
  TSA_TRY(need_ptrs({Q, K, V, Y}));
  TSA_TRY(opt_ptrs({X}));
  TSA_TRY(check_ws(ws, ws_bytes, tsa_dense_varlen_workspace_bytes(s, B, cu_seqlens)));
  hipStream_t st = stream_of(stream);
  const size_t eb = elem_bytes(s->dtype);
  std::vector<AttnSeqDesc> seqs;
  std::vector<int64_t> P(B + 1, 0);
  for (int32_t b = 0; b < B; ++b) P[b + 1] = P[b] + tsa_capacity(cu_seqlens[b + 1] - cu_seqlens[b]);
  hipError_t e = hipSuccess;
  for (int32_t b = 0; b < B && e == hipSuccess; ++b) {
    const int64_t Lb = cu_seqlens[b + 1] - cu_seqlens[b];
    e = launch_transpose_v(s->dtype, s->d, static_cast<const char*>(V) + (size_t)cu_seqlens[b] * s->Hkv * s->d * eb,
                           Lb, s->Hkv, P[b + 1] - P[b], static_cast<char*>(ws) + (size_t)P[b] * s->Hkv * s->d * eb, st);
  }
  for (int32_t b : longest_first(B, cu_seqlens))
    seqs.push_back({cu_seqlens[b], P[b], cu_seqlens[b + 1] - cu_seqlens[b], P[b + 1] - P[b], nullptr, nullptr});
  if (e == hipSuccess)
    e = launch_attention_varlen(s->dtype, s->d, true, Q, K, ws, B, seqs.data(), s->Hq, s->Hkv, X, Y, st);
  return hip_status(e);
}

int tsa_layer_varlen(const tsa_shape* s, int32_t B, const int64_t* cu_seqlens, const void* Q, const void* K,
                     const void* V, const void* X, void* Y, int32_t* kLp_dev, void* ws, size_t ws_bytes,
                     void* stream) {
  TSA_TRY(check_varlen(s, B, cu_seqlens));
  TSA_TRY(need_ptrs({Q, K, V, Y}));
  TSA_TRY(opt_ptrs({X}));
  if (kLp_dev && ((uintptr_t)kLp_dev & 3u)) return TSA_ERR_ALIGN;
  const VarlenWs w = varlen_layout(s, B, cu_seqlens);
  TSA_TRY(check_ws(ws, ws_bytes, w.total));
  hipStream_t st = stream_of(stream);
  const StageWs& g = w.st;
  const size_t eb = elem_bytes(s->dtype), Hq = s->Hq, Hkv = s->Hkv, d = s->d;
  int32_t* kLp = at<int32_t>(ws, w.kLp);
  const bool fused = fused_layer(s, false);
  std::vector<int64_t> P(B + 1, 0);
  for (int32_t b = 0; b < B; ++b) P[b + 1] = P[b] + tsa_capacity(cu_seqlens[b + 1] - cu_seqlens[b]);
  auto tok = [&](const void* base, size_t heads, int32_t b) {
    return static_cast<const char*>(base) + (size_t)cu_seqlens[b] * heads * d * eb;
  };
  auto comp = [&](size_t off, int32_t b) { return at<char>(ws, off) + (size_t)P[b] * Hq * d * eb; };
  hipError_t e = hipSuccess;
  // stages 1-4a sample by sample (each O(L_b)); the stage workspace is reused in stream order
  for (int32_t b = 0; b < B && e == hipSuccess; ++b) {
    const int64_t Lb = cu_seqlens[b + 1] - cu_seqlens[b], Cb = P[b + 1] - P[b];
    float* s_h = at<float>(ws, w.s_h) + Hq * (size_t)P[b];
    float* s_l = at<float>(ws, w.s_l) + (size_t)P[b];
    int32_t* idx = at<int32_t>(ws, w.idx) + Hq * (size_t)P[b];
    int32_t* inv = at<int32_t>(ws, w.inv) + Hq * (size_t)P[b];
    int32_t* kl = kLp + 2 * b;
    // histograms + control words (not used by the one-workgroup selects of short samples)
    if (!radix_resident(Lb)) e = launch_fill_zero(at<char>(ws, g.bhist), g.tcnt - g.bhist, st);
    if (e == hipSuccess)
      e = launch_score(s->dtype, s->d, tok(Q, Hq, b), tok(K, Hkv, b), Lb, s->Hq, s->Hkv, s->q, s_h,
                       at<double2>(ws, g.partials), at<double2>(ws, g.rowstat), st);
    if (e == hipSuccess && radix_resident(Lb))
      e = launch_layer_budget_select(s_h, Lb, s->Hq, at<double>(ws, g.S), at<double>(ws, g.tilesum), s_l,
                                     budget_target(s->tau), kl, kLp_dev ? kLp_dev + 2 * b : nullptr,
                                     kLp_dev ? kLp_dev + 2 * b + 1 : nullptr, idx, inv, st);
    if (e == hipSuccess && !radix_resident(Lb))
      e = launch_layer_score_budget(s_h, Lb, s->Hq, at<double>(ws, g.S), at<double>(ws, g.tilesum), s_l,
                                    budget_target(s->tau), at<uint64_t>(ws, g.bhist), at<RadixCtl>(ws, g.bctl), kl,
                                    kLp_dev ? kLp_dev + 2 * b : nullptr, kLp_dev ? kLp_dev + 2 * b + 1 : nullptr, st);
    if (e == hipSuccess && !radix_resident(Lb))
      e = launch_select(s_h, Lb, s->Hq, kl + 1, at<uint64_t>(ws, g.shist), at<RadixCtl>(ws, g.sctl),
                        at<uint32_t>(ws, g.tcnt), at<uint32_t>(ws, g.toff), idx, inv, st);
    if (e == hipSuccess)
      e = launch_gather(s->dtype, s->d, tok(Q, Hq, b), tok(K, Hkv, b), tok(V, Hkv, b), idx, kl + 1, Lb, s->Hq,
                        s->Hkv, Cb, fused ? nullptr : comp(w.Qh, b), fused ? nullptr : comp(w.Kh, b), comp(w.Vht, b),
                        st, fused ? inv : nullptr, fused && X ? tok(X, Hq, b) : nullptr,
                        fused ? static_cast<char*>(Y) + (size_t)cu_seqlens[b] * Hq * d * eb : nullptr);
  }
  // stage 4b: one launch over every sample's ragged L'_b (fused: stage 5 in its epilogue)
  if (e == hipSuccess) {
    std::vector<AttnSeqDesc> seqs;
    for (int32_t b : longest_first(B, cu_seqlens))
      seqs.push_back({cu_seqlens[b], P[b], cu_seqlens[b + 1] - cu_seqlens[b], P[b + 1] - P[b], kLp + 2 * b + 1,
                      at<int32_t>(ws, w.idx) + Hq * (size_t)P[b]});
    if (fused)
      e = launch_attention_varlen(s->dtype, s->d, false, Q, K, at<void>(ws, w.Vht), B, seqs.data(), s->Hq, s->Hkv, X,
                                  Y, st, true);
    else
      e = launch_attention_varlen(s->dtype, s->d, false, at<void>(ws, w.Qh), at<void>(ws, w.Kh), at<void>(ws, w.Vht),
                                  B, seqs.data(), s->Hq, s->Hkv, nullptr, at<void>(ws, w.Oh), st);
  }
  // stage 5 sample by sample
  for (int32_t b = 0; b < B && e == hipSuccess && !fused; ++b) {
    const int64_t Lb = cu_seqlens[b + 1] - cu_seqlens[b], Cb = P[b + 1] - P[b];
    const size_t row = (size_t)cu_seqlens[b] * Hq * d * eb;
    e = launch_scatter(s->dtype, s->d, comp(w.Oh, b), at<int32_t>(ws, w.idx) + Hq * (size_t)P[b],
                       at<int32_t>(ws, w.inv) + Hq * (size_t)P[b], kLp + 2 * b + 1,
                       X ? static_cast<const char*>(X) + row : nullptr, static_cast<char*>(Y) + row, Lb, s->Hq, Cb, st);
  }
  return hip_status(e);
}

int64_t tsa_block_count(int64_t L) { return tsa_capacity(L) / kBlock; }

size_t tsa_block_select_workspace_bytes(const tsa_shape* s) {
  return tsa_check_args(s) == TSA_OK ? 2 * up(pooled_bytes(s)) + up(logits_bytes(s)) : 0;
}

size_t tsa_layer_block_sparse_workspace_bytes(const tsa_shape* s) {
  return tsa_check_args(s) == TSA_OK ? layer_layout(s, true).total : 0;
}

int tsa_block_select(const tsa_shape* s, float gamma, const void* Qh, const void* Kh, const int32_t* Lp_dev,
                     uint16_t* list, int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  TSA_TRY(tsa_check_args(s));
  if (!(gamma >= 0.f)) return TSA_ERR_ARG;
  TSA_TRY(need_ptrs({Qh, Kh, list, count}));
  TSA_TRY(need_int_ptrs({Lp_dev}));
  if (block_count(s) > kMaxKeyBlocks) return TSA_ERR_UNSUPPORTED;
  TSA_TRY(check_ws(ws, ws_bytes, tsa_block_select_workspace_bytes(s)));
  float* qbar = at<float>(ws, 0);
  float* kbar = at<float>(ws, up(pooled_bytes(s)));
  double* zl = at<double>(ws, 2 * up(pooled_bytes(s)));
  return hip_status(launch_block_select(s->dtype, s->d, Qh, Kh, Lp_dev, tsa_capacity(s->L), s->Hq, (double)gamma,
                                        qbar, kbar, zl, list, count, stream_of(stream)));
}

int tsa_attn_block_sparse(const tsa_shape* s, const void* Qh, const void* Kh, const void* Vht, const int32_t* Lp_dev,
                          const uint16_t* list, const int32_t* count, void* Oh, void* stream) {
  TSA_TRY(tsa_check_args(s));
  TSA_TRY(need_ptrs({Qh, Kh, Vht, Oh, list, count}));
  TSA_TRY(need_int_ptrs({Lp_dev}));
  if (block_count(s) > kMaxKeyBlocks) return TSA_ERR_UNSUPPORTED;
  return hip_status(launch_attention_block_sparse(s->dtype, s->d, Qh, Kh, Vht, Lp_dev, s->L, s->Hq, s->Hkv,
                                                  tsa_capacity(s->L), list, count, Oh, stream_of(stream)));
}

int tsa_layer_block_sparse(const tsa_shape* s, float gamma, const void* Q, const void* K, const void* V,
                           const void* X, void* Y, int32_t* kLp_dev, void* ws, size_t ws_bytes, void* stream) {
  if (!(gamma >= 0.f)) return TSA_ERR_ARG;
  return run_layer(s, false, 0.f, Q, K, V, X, Y, kLp_dev, ws, ws_bytes, stream, true, gamma);
}

}  // extern "C"

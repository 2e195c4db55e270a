// Internal interface between the C ABI (api.cpp) and the kernel launchers (*.hip).
// Every launcher enqueues on `st` and returns hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsa.h"

namespace tsa {

// Host validation of tsa_layer's arguments other than the workspace (status codes of tsa.h).
int layer_args(const tsa_shape* s, const void* Q, const void* K, const void* V, const void* X, const void* Y,
               const int32_t* kLp_dev);

// Per-pass control word of a radix select over one segment (see select.hip).
struct RadixCtl {
  uint32_t prefix;      // key bits fixed so far (high bits first)
  uint32_t none;        // 1: the target exceeds the segment's total weight
  uint64_t cnt_below;   // elements whose key is below the current prefix range
  uint64_t w_below;     // their total weight
  uint64_t n_bin;       // elements in the chosen bucket of the last pass
};

constexpr int kRadixBins = 256;
constexpr int kRadixPasses = 4;

// ---- score.hip ----------------------------------------------------------------------------------
// Rows scored per KV group: R = (Hq/Hkv) * q; blocks of 256 keys; 4 waves per block.
int64_t score_blocks(int64_t L);
size_t score_partial_bytes(int64_t L, int Hq, int Hkv, int q);
size_t score_rowstat_bytes(int Hq, int Hkv, int q);
hipError_t launch_score(int dtype, int d, const void* Q, const void* K, int64_t L, int Hq, int Hkv,
                        int q, float* s_h, double2* partials, double2* rowstat, hipStream_t st);

// ---- select.hip ---------------------------------------------------------------------------------
int64_t layer_tiles(int64_t L);
hipError_t launch_layer_score(const float* s_h, int64_t L, int Hq, double* S, double* tile_sum,
                              float* s_l, hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
// Budget over s_l: writes k and L' (either may be null) and keeps them in kLp_ws[0..1].
hipError_t launch_budget(const float* s_l, int64_t L, uint64_t target, uint64_t* hist,
                         RadixCtl* ctl, int32_t* kLp_ws, int32_t* k_out, int32_t* Lp_out,
                         hipStream_t st);
// launch_layer_score followed by launch_budget (same s_l, k and L'), in fewer launches for short rows.
hipError_t launch_layer_score_budget(const float* s_h, int64_t L, int Hq, double* S, double* tile_sum, float* s_l,
                                     uint64_t target, uint64_t* hist, RadixCtl* ctl, int32_t* kLp_ws,
                                     int32_t* k_out, int32_t* Lp_out, hipStream_t st);
// Rows of at most this many keys are budgeted and selected by one workgroup per row, which needs
// neither the histograms nor the control words (nor their clearing).
bool radix_resident(int64_t L);
// Fixed-ratio budget: k = round(sparsity * L) (halves up); writes like launch_budget (kLp_ws may be null).
hipError_t launch_budget_ratio(float sparsity, int64_t L, int32_t* kLp_ws, int32_t* k_out, int32_t* Lp_out,
                               hipStream_t st);
int64_t select_tiles(int64_t L);
hipError_t launch_select(const float* s_h, int64_t L, int Hq, const int32_t* Lp_dev,
                         uint64_t* hist, RadixCtl* ctl, uint32_t* tile_cnt, uint32_t* tile_off,
                         int32_t* idx, int32_t* inv, hipStream_t st);
// For a resident row only (radix_resident(L)): launch_layer_score_budget followed by launch_select
// with L' from the budget (same s_l, k, L', idx and inv), budget and selection in one launch.
hipError_t launch_layer_budget_select(const float* s_h, int64_t L, int Hq, double* S, double* tile_sum, float* s_l,
                                      uint64_t target, int32_t* kLp_ws, int32_t* k_out, int32_t* Lp_out, int32_t* idx,
                                      int32_t* inv, hipStream_t st);

// ---- move.hip -----------------------------------------------------------------------------------
// With Y (bf16 only), the same launch also writes the rows outside every selection:
// Y[t][h] = X[t][h] (or +0.0 without X) where inv[h][t] < 0, nothing when Y aliases X.  (The fused
// layer writes the selected rows from the attention epilogue.)
hipError_t launch_gather(int dtype, int d, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const int32_t* Lp_dev, int64_t L, int Hq, int Hkv,
                         int64_t C, void* Qh, void* Kh, void* Vht, hipStream_t st, const int32_t* inv = nullptr,
                         const void* X = nullptr, void* Y = nullptr);
hipError_t launch_transpose_v(int dtype, int d, const void* V, int64_t L, int Hkv, int64_t C,
                              void* Vt, hipStream_t st);
hipError_t launch_scatter(int dtype, int d, const void* Oh, const int32_t* idx, const int32_t* inv,
                          const int32_t* Lp_dev, const void* X, void* Y, int64_t L, int Hq,
                          int64_t C, hipStream_t st);

// ---- blocksparse.hip ----------------------------------------------------------------------------
// Blocks of kBlock compressed rows (= the bf16 attention kernel's query rows per workgroup); at most
// kMaxKeyBlocks blocks per head (capacity <= kBlock * kMaxKeyBlocks rows).
constexpr int kBlock = 128;
constexpr int kMaxKeyBlocks = 4096;
// Pools Qh/Kh [Hq][C][d] into qbar/kbar [Hq][NB][d] (float32, NB = C/kBlock), forms the block
// logits zl [Hq][NB][NB] (float64, causal half) and writes the kept key blocks of every query
// block: list [Hq][NB][NB] ascending, count [Hq][NB] (0 past the last block).
hipError_t launch_block_select(int dtype, int d, const void* Qh, const void* Kh, const int32_t* Lp_dev, int64_t C,
                               int Hq, double gamma, float* qbar, float* kbar, double* zl, uint16_t* list,
                               int32_t* count, hipStream_t st);

// ---- attention.hip ------------------------------------------------------------------------------
// Compressed (dense == false): Qh/Kh [Hq][C][d], Vht [Hq][d][C], L' from Lp_dev, output Oh.
// Dense (dense == true): Q [L][Hq][d], K [L][Hkv][d], Vt [Hkv][d][C] (C >= L), output
// Y [L][Hq][d] = X + O (X may be null).
hipError_t launch_attention(int dtype, int d, bool dense, const void* Q, const void* K,
                            const void* Vt, const int32_t* Lp_dev, int64_t L, int Hq, int Hkv,
                            int64_t C, const void* X, void* O, hipStream_t st);

// One sequence of a varlen batch.  Compressed: its Qh/Kh/Oh region [Hq][C][d] and Vht region
// [Hq][d][C] start at element Hq*d*cap_off, L' is read from Lp_dev, and L bounds the grid (L' <= L).
// Dense: tokens [tok_off, tok_off + L) of Q/K/X/Y; its Vt region [Hkv][d][C] starts at element
// Hkv*d*cap_off.  Longer sequences listed first are scheduled first.
// Fused (compressed, bf16): Q and K are the uncompressed [tokens][Hq][d] and [tokens][Hkv][d] inputs,
// query and key row i of head h are token tok_off + idx[h][i] (idx [Hq][L] per sequence), and the
// output row is written to O (= Y) at that token, plus X when given, rounded as tsa_scatter_residual
// rounds; Vht as compressed.
struct AttnSeqDesc {
  int64_t tok_off, cap_off, L, C;
  const int32_t* Lp_dev;
  const int32_t* idx;
};
hipError_t launch_attention_varlen(int dtype, int d, bool dense, const void* Q, const void* K, const void* Vt,
                                   int nseq, const AttnSeqDesc* seqs, int Hq, int Hkv, const void* X, void* O,
                                   hipStream_t st, bool fused = false);
// Compressed attention restricted to the listed key blocks of every query block (launch_block_select's
// list and count, NB = C / kBlock).
hipError_t launch_attention_block_sparse(int dtype, int d, const void* Qh, const void* Kh, const void* Vht,
                                         const int32_t* Lp_dev, int64_t L, int Hq, int Hkv, int64_t C,
                                         const uint16_t* list, const int32_t* count, void* Oh, hipStream_t st);

}  // namespace tsa

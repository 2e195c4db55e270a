/*
 * tsa.h -- C ABI of libtsa.so, the Token Sparse Attention (TSA) prefill layer for MI355X (gfx950).
 *
 * The layer (papernotes.org reading notes, "Overall framework" and "Key design 1/2"; bxzpzcl.cn
 * article, sections 1.1 and 2.1; gist.science summary, "2. Methodology"):
 *
 *   1. score   -- the last q queries attend causally to all keys; the softmax weights summed over
 *                 those queries give a per-head token score s_h; s_l = normalize(sum_h s_h).
 *   2. budget  -- sort s_l ascending; k = the smallest count whose cumulative mass reaches tau;
 *                 keep L' = L - k tokens.
 *   3. select  -- each head keeps its own top-L' tokens by s_h, indices ascending.
 *   4. gather + causal attention on the compressed L' x L' problem.
 *   5. scatter the output into zeros of length L and add the residual: Y = X + Decompress(O_hat).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library allocates and frees
 *     nothing, keeps no pointer after returning and has no global mutable state.  Every call only
 *     enqueues work on `stream` (a hipStream_t passed as void*; NULL = the null stream) and returns;
 *     buffers must stay alive until the stream has finished that work.
 *   - Every argument is checked on the host BEFORE anything is launched: a call that returns an
 *     error has enqueued nothing.  TSA_ERR_HIP reports a failed launch.
 *   - Layouts (row-major, contiguous, 16-byte aligned):
 *       Q, X, Y      [L][Hq][d]     K, V  [L][Hkv][d]        (storage dtype)
 *       s_h          [Hq][L]        s_l   [L]                (float32)
 *       idx, inv     [Hq][L]                                  (int32)
 *       Qh, Kh, Oh   [Hq][C][d]     Vht   [Hq][d][C]          (storage dtype; C = tsa_capacity(L))
 *     Vht holds V_hat transposed (token index fastest) because the attention kernel feeds V_hat to
 *     the matrix cores along the token dimension.
 *   - Query head h reads KV head h / (Hq / Hkv) (grouped-query attention).
 *   - The keep count L' is data dependent and stays on the device: stages after the budget read it
 *     from `Lp_dev` (one int32), so no host synchronisation is needed anywhere on the path.
 *   - NaN or Inf inputs give undefined outputs.  Calls on distinct streams with distinct workspaces
 *     may run concurrently; Y may alias X; no other aliasing is allowed.
 *   - No call allocates, memsets or synchronises, so a call can be captured in a HIP graph on its
 *     stream and replayed (workspaces are cleared by kernels inside the captured work).
 */
#ifndef TSA_H
#define TSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TSA_OK = 0,
    TSA_ERR_ARG = 1,          /* NULL where a pointer is required, tau outside [0, 1), bad enum */
    TSA_ERR_SHAPE = 2,        /* L, Hq, Hkv, d or q outside the supported ranges (L <= 2^24) */
    TSA_ERR_DTYPE = 3,        /* dtype is neither TSA_F32 nor TSA_BF16 */
    TSA_ERR_ALIGN = 4,        /* a tensor pointer is not 16-byte aligned */
    TSA_ERR_WORKSPACE = 5,    /* workspace NULL, misaligned (256 B) or smaller than required */
    TSA_ERR_HIP = 6,          /* a kernel launch failed */
    TSA_ERR_UNSUPPORTED = 7,  /* valid but not implemented (e.g. d not in {64, 128}) */
    TSA_ERR_TOO_LARGE = 8     /* tsa_layer_noalloc: the layer's intermediates exceed its fixed scratch */
} tsa_status;

typedef enum { TSA_F32 = 0, TSA_BF16 = 1 } tsa_dtype;

/* Problem description.  Constraints: 1 <= q <= min(L, 1024); L <= 2^24; 1 <= Hkv <= Hq <= 1024;
 * Hq % Hkv == 0; d in {64, 128}; 0 <= tau < 1 (NaN rejected); dtype TSA_F32 or TSA_BF16. */
typedef struct {
    int64_t L;       /* tokens */
    int32_t Hq;      /* query heads */
    int32_t Hkv;     /* key/value heads */
    int32_t d;       /* head dimension */
    int32_t q;       /* recent queries used for scoring (the last q positions) */
    float   tau;     /* coverage threshold */
    int32_t dtype;   /* tsa_dtype of Q, K, V, X, Y and the compressed tensors */
} tsa_shape;

/* Human-readable name of a status code (static string, never NULL). */
const char* tsa_status_string(int status);

/* Validate a shape on the host.  No GPU needed. */
int tsa_check_args(const tsa_shape* s);

/* Row capacity C of the compressed tensors for length L (L rounded up to a multiple of 256). */
int64_t tsa_capacity(int64_t L);

/* Workspace (device memory, 256-byte aligned) needed by tsa_score, tsa_budget and tsa_select;
 * one buffer of this size serves any of them. */
size_t tsa_stage_workspace_bytes(const tsa_shape* s);
/* Workspace needed by tsa_layer and tsa_layer_ratio: the stage workspace plus every intermediate
 * the layer materialises: s_h, s_l, idx, inv and Vht; f32 also Qh, Kh and Oh (the bf16 layer reads
 * its query and key rows through idx and writes Y from the attention epilogue). */
size_t tsa_layer_workspace_bytes(const tsa_shape* s);
/* Workspace needed by tsa_dense_attn_causal. */
size_t tsa_dense_workspace_bytes(const tsa_shape* s);

/* Stage 1 -- Dynamic Token Coverage scoring (notes, "Key design 2"; article 2.1; summary, "Dynamic
 * Token Coverage").  For query head h (KV head g) and the recent positions p = L-q .. L-1:
 *   z[p][t] = <Q[p][h], K[t][g]> / sqrt(d) for t <= p,  a[p][.] = softmax(z[p][.]),
 *   s_h[h][t] = sum_p a[p][t].
 * If s_l != NULL also writes s_l[t] = sum_h s_h[h][t] / sum_t' sum_h s_h[h][t'].
 * The softmax statistics and the sums are accumulated in float64. */
int tsa_score(const tsa_shape* s, const void* Q, const void* K, float* s_h, float* s_l,
              void* ws, size_t ws_bytes, void* stream);

/* Stage 2 -- coverage budget (notes, "Key design 2"; article 2.1).  With v = s_l sorted ascending
 * and C(j) = v[0] + ... + v[j-1]: k = min { j in [0, L] : C(j) >= tau } (k = L if none), L' = L - k.
 * Writes k to k_dev[0] and L' to Lp_dev[0] (device int32; either may be NULL).  The cumulative mass
 * is summed exactly in 64-bit fixed point (2^-60 units) over the float32 s_l values. */
int tsa_budget(const tsa_shape* s, const float* s_l, int32_t* k_dev, int32_t* Lp_dev,
               void* ws, size_t ws_bytes, void* stream);

/* Stage 3 -- per-head selection (notes, "Key design 2"; summary, head-wise selection).  For every
 * head, idx[h][0..L'-1] = the L' tokens with the largest s_h[h][.] (ties: lower index first), in
 * ascending order; idx[h][L'..L-1] is left untouched.  If inv != NULL, inv[h][t] = position of t
 * in idx[h] or -1 when t is not selected.  L' is read from Lp_dev[0]. */
int tsa_select(const tsa_shape* s, const float* s_h, const int32_t* Lp_dev, int32_t* idx,
               int32_t* inv, void* ws, size_t ws_bytes, void* stream);

/* Stage 4a -- compress (notes, "Key design 1"; article 1.1 gather):
 *   Qh[h][i] = Q[idx[h][i]][h],  Kh[h][i] = K[idx[h][i]][g],  Vht[h][.][i] = V[idx[h][i]][g]
 * for i < L'.  Bit-exact copies.  Rows (Vht: columns) at and past L' hold unspecified values; no
 * entry point reads them. */
int tsa_gather(const tsa_shape* s, const void* Q, const void* K, const void* V, const int32_t* idx,
               const int32_t* Lp_dev, void* Qh, void* Kh, void* Vht, void* stream);

/* Stage 4b -- causal attention in the compressed space (article 1.1: softmax(QK^T/sqrt(d))V; the
 * mask is causal by original position, which for ascending idx is j <= i):
 *   Oh[h][i] = sum_{j<=i} softmax_j(<Qh[h][i], Kh[h][j]> / sqrt(d)) Vht[h][.][j]   for i < L'.
 * bf16: matrix-core products with float32 accumulation and a float32 online softmax; f32: float32
 * throughout.  Rows >= L' of Oh are not written. */
int tsa_attn_causal(const tsa_shape* s, const void* Qh, const void* Kh, const void* Vht,
                    const int32_t* Lp_dev, void* Oh, void* stream);

/* Stage 5 -- decompress and residual (notes, "Key design 1"; article 1.1 zeros + scatter):
 *   Y[t][h] = X[t][h] + Oh[h][inv[h][t]]  if t is selected,  X[t][h] otherwise.
 * X == NULL gives the pure decompress (unselected rows are +0.0).  The sum is formed in float32 and
 * rounded to nearest even once.  inv may be NULL; idx is then used and Y is pre-filled from X (or
 * zeros).  When Y aliases X only the selected rows are written. */
int tsa_scatter_residual(const tsa_shape* s, const void* Oh, const int32_t* idx, const int32_t* inv,
                         const int32_t* Lp_dev, const void* X, void* Y, void* stream);

/* The whole layer, stages 1-5 back to back on `stream` with no host synchronisation:
 * Y = X + Decompress(attention on the selected tokens).  X may be NULL (Y = Decompress only) and Y
 * may alias X.  If kLp_dev != NULL it receives {k, L'} (device int32[2]). */
int tsa_layer(const tsa_shape* s, const void* Q, const void* K, const void* V, const void* X,
              void* Y, int32_t* kLp_dev, void* ws, size_t ws_bytes, void* stream);

/* Allocation-free tsa_layer, for callers that cannot allocate device memory at call time (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation) and cannot hold a
 * workspace of their own.  Computes exactly what tsa_layer computes, with the same kernels, bit for
 * bit; its intermediates live in a fixed scratch array of TSA_NOALLOC_SCRATCH_BYTES that the library
 * holds in device memory on every GPU it runs on, from the first call on that GPU until the process
 * ends.  No call allocates or frees anything.
 *   - The layer's workspace (tsa_layer_workspace_bytes(s)) must fit the scratch; otherwise the call
 *     returns TSA_ERR_TOO_LARGE and enqueues nothing.  Arguments are validated as in tsa_layer.
 *   - Every call on one GPU uses that GPU's single scratch array: calls that overlap on one GPU
 *     (concurrent streams, or host threads sharing a device) race and give undefined results; calls
 *     on one stream, one after another, are safe (each clears what it needs).
 *   - The first call on a GPU looks up the array's device address with that GPU current (a host
 *     query, not an allocation); TSA_ERR_HIP if that fails. */
#define TSA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int tsa_layer_noalloc(const tsa_shape* s, const void* Q, const void* K, const void* V, const void* X, void* Y,
                      int32_t* kLp_dev, void* stream);

/* Fixed-ratio budget, the baseline the coverage budget is measured against in the ablations (notes,
 * "Ablations": tau = 0.005 against a fixed s = 0.3, tau = 0.010 against s = 0.5; "Key design 2"
 * describes the fixed keep ratio it replaces).  The pruned count ignores the scores:
 *   k = round(sparsity * L), halves rounded up, computed exactly from the float32 value;  L' = L - k.
 * Writes k to k_dev[0] and L' to Lp_dev[0] (device int32; either may be NULL).  sparsity must lie in
 * [0, 1] (TSA_ERR_ARG otherwise, NaN included); s->tau is not used.  Needs no workspace. */
int tsa_budget_ratio(const tsa_shape* s, float sparsity, int32_t* k_dev, int32_t* Lp_dev, void* stream);

/* tsa_layer with the fixed-ratio budget in place of the coverage budget: scoring (s_h only), then
 * L' from tsa_budget_ratio's rule, then selection, compression, attention, decompression and the
 * residual exactly as in tsa_layer.  Workspace: tsa_layer_workspace_bytes.  s->tau is not used. */
int tsa_layer_ratio(const tsa_shape* s, float sparsity, const void* Q, const void* K, const void* V,
                    const void* X, void* Y, int32_t* kLp_dev, void* ws, size_t ws_bytes, void* stream);

/* Dense causal attention over the full length with the same kernels (the dense layer that the
 * sparse layers replace; notes, "Overall framework"): Y[t][h] = X[t][h] + O[t][h] (X may be NULL;
 * Y may alias X).  The speedup baseline of the layer. */
int tsa_dense_attn_causal(const tsa_shape* s, const void* Q, const void* K, const void* V,
                          const void* X, void* Y, void* ws, size_t ws_bytes, void* stream);

/* ---- Block sparsity stacked on the token selection --------------------------------------------
 * The compressed Q_hat, K_hat, V_hat are dense and contiguous, so a block-sparse attention can run
 * on them after the token filter (notes, "Key findings"; article 3.2: token selection first, then
 * block-sparse computation).  The pages give no block rule; this library's rule mirrors the
 * coverage budget.  Blocks are 128 consecutive compressed rows; NB = tsa_block_count(L) blocks per
 * head (at most 4096, i.e. L <= 524288: TSA_ERR_UNSUPPORTED otherwise).
 *   pool   : qbar[h][b], kbar[h][b] = mean of block b's rows of Qh[h], Kh[h] (float64 sum in row
 *            order, rounded once to float32);
 *   select : for query block I, a_J = softmax over J <= I of <qbar_I, kbar_J> / sqrt(d) (float64);
 *            keep the fewest heaviest J (ties: lower J) whose weights sum to >= gamma (all J when
 *            gamma >= 1 or no prefix does), plus J = 0 and J = I;
 *   attend : query row i of block I sees the keys j <= i of its kept blocks only.
 * Lists: list [Hq][NB][NB] uint16, row (h, I) holds count[h][I] kept blocks ascending; count
 * [Hq][NB] int32 (0 for blocks at or past L'). */

/* Key blocks per head for length L (tsa_capacity(L) / 128). */
int64_t tsa_block_count(int64_t L);
/* Workspace of tsa_block_select and of tsa_layer_block_sparse.  tsa_block_select leaves the pooled
 * means in its workspace: qbar [Hq][NB][d] float32 at byte 0, kbar at the next multiple of 256
 * bytes after it (then the float64 block logits [Hq][NB][NB]). */
size_t tsa_block_select_workspace_bytes(const tsa_shape* s);
size_t tsa_layer_block_sparse_workspace_bytes(const tsa_shape* s);

/* Pool the compressed Qh, Kh (layout of tsa_gather, L' from Lp_dev) and write the kept key blocks
 * of every query block.  gamma >= 0 (NaN rejected). */
int tsa_block_select(const tsa_shape* s, float gamma, const void* Qh, const void* Kh, const int32_t* Lp_dev,
                     uint16_t* list, int32_t* count, void* ws, size_t ws_bytes, void* stream);

/* tsa_attn_causal restricted to the kept key blocks (list, count from tsa_block_select).  With every
 * block kept it computes exactly what tsa_attn_causal computes, bit for bit. */
int tsa_attn_block_sparse(const tsa_shape* s, const void* Qh, const void* Kh, const void* Vht, const int32_t* Lp_dev,
                          const uint16_t* list, const int32_t* count, void* Oh, void* stream);

/* tsa_layer with block-sparse compressed attention: scoring, budget, selection and compression as
 * in tsa_layer, then tsa_block_select and tsa_attn_block_sparse, then decompression and the
 * residual.  Workspace: tsa_layer_block_sparse_workspace_bytes. */
int tsa_layer_block_sparse(const tsa_shape* s, float gamma, const void* Q, const void* K, const void* V,
                           const void* X, void* Y, int32_t* kLp_dev, void* ws, size_t ws_bytes, void* stream);

/* ---- Batches of sequences of different lengths (varlen) -------------------------------------
 * The keep count L' is data dependent, so the samples of a batch compress to different lengths
 * (notes, "Limitations", names this raggedness as a practical cost of batching).  A batch packs B
 * independent sequences along the token dimension: sample b owns tokens [cu[b], cu[b+1]) of Q, K,
 * V, X and Y, where cu_seqlens is a HOST array of B+1 int64 with cu[0] = 0, cu[b] < cu[b+1] and
 * cu[B] = s->L (the total).  Every sample shares Hq, Hkv, d, q, tau and dtype, and needs
 * cu[b+1] - cu[b] >= q (TSA_ERR_SHAPE otherwise; a malformed cu gives TSA_ERR_ARG).  Each sample
 * gets its own scores, budget, keep count L'_b and selection, exactly as tsa_layer on that sample
 * alone.
 * Compressed tensors of a batch: sample b's region has the one-sequence layout for its length L_b
 * (Qh, Kh, Oh [Hq][C_b][d], Vht [Hq][d][C_b], C_b = tsa_capacity(L_b)) and starts at element
 * Hq*d*P_b, with P_b = C_0 + ... + C_{b-1}; the total row capacity is tsa_varlen_capacity(). */

/* P_B = sum of the per-sample capacities, or -1 if cu_seqlens is malformed.  Host only. */
int64_t tsa_varlen_capacity(int32_t B, const int64_t* cu_seqlens);
/* Workspace of tsa_layer_varlen / tsa_dense_attn_causal_varlen (0 for invalid arguments). */
size_t tsa_layer_varlen_workspace_bytes(const tsa_shape* s, int32_t B, const int64_t* cu_seqlens);
size_t tsa_dense_varlen_workspace_bytes(const tsa_shape* s, int32_t B, const int64_t* cu_seqlens);

/* Stage 4b over a batch in ONE launch: tsa_attn_causal for every sample, sample b reading its
 * keep count from Lp_dev[b] (device int32[B]).  Longer samples are scheduled first. */
int tsa_attn_causal_varlen(const tsa_shape* s, int32_t B, const int64_t* cu_seqlens, const void* Qh,
                           const void* Kh, const void* Vht, const int32_t* Lp_dev, void* Oh, void* stream);

/* tsa_layer for every sample of the batch.  Scoring, budget, selection, compression and
 * decompression run sample after sample on `stream` (each is O(L_b)); the attention runs as one
 * launch over all samples' ragged keep counts.  kLp_dev (optional) receives {k_b, L'_b} per sample
 * (device int32[B][2]).  Y may alias X.  Workspace: tsa_layer_varlen_workspace_bytes. */
int tsa_layer_varlen(const tsa_shape* s, int32_t B, const int64_t* cu_seqlens, const void* Q, const void* K,
                     const void* V, const void* X, void* Y, int32_t* kLp_dev, void* ws, size_t ws_bytes,
                     void* stream);

/* tsa_dense_attn_causal for every sample of the batch, the attention in one launch (the dense
 * baseline of tsa_layer_varlen).  Workspace: tsa_dense_varlen_workspace_bytes. */
int tsa_dense_attn_causal_varlen(const tsa_shape* s, int32_t B, const int64_t* cu_seqlens, const void* Q,
                                 const void* K, const void* V, const void* X, void* Y, void* ws,
                                 size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TSA_H */

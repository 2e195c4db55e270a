// Compress and decompress (papernotes.org reading notes, "Key design 1"; bxzpzcl.cn article,
// section 1.1 gather / zeros_like + scatter_): pure data movement in 16-byte vectors.
//
// gather : per query head, rows idx[h][0..L') of Q, K, V -> dense Qh, Kh [Hq][C][d] and the
//          transposed Vht [Hq][d][C] (bf16: Qh and Kh by a row-copy kernel, Vht by a second one
//          that transposes 8 x 8 blocks in registers; fp32: one kernel, a 64-row tile staged in
//          LDS and written column-major so the stores stay contiguous).
// scatter: Y[t][h] = X[t][h] + Oh[h][inv[h][t]] for selected t, X[t][h] otherwise (float32 sum,
//          one rounding); without X the selected rows are copied and the others are +0.0.
#include "kern_common.h"
#include "tsa_internal.h"

namespace tsa {

constexpr int kTileRows = 64;

template <typename T, int D>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                     const T* __restrict__ V, const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ Lp_dev, int64_t L, int Hq,
                                                     int Hkv, int64_t C, T* __restrict__ Qh,
                                                     T* __restrict__ Kh, T* __restrict__ Vht) {
  constexpr int VPR = D * (int)sizeof(T) / 16;     // 16-byte vectors per row
  constexpr int EPV = 16 / (int)sizeof(T);         // elements per vector
  __shared__ uint4 stage[kTileRows * VPR];
  const int h = blockIdx.y, g = h / (Hq / Hkv);
  const int64_t i0 = (int64_t)blockIdx.x * kTileRows;
  const int64_t Lp = Lp_dev[0];
  if (i0 >= Lp) return;
  const int n = (int)(Lp - i0 < kTileRows ? Lp - i0 : kTileRows);
  const uint4* Q4 = reinterpret_cast<const uint4*>(Q);
  const uint4* K4 = reinterpret_cast<const uint4*>(K);
  const uint4* V4 = reinterpret_cast<const uint4*>(V);
  uint4* Qh4 = reinterpret_cast<uint4*>(Qh);
  uint4* Kh4 = reinterpret_cast<uint4*>(Kh);
  for (int e = threadIdx.x; e < kTileRows * VPR; e += 256) {
    const int r = e / VPR, c = e % VPR;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < n) {
      const int64_t t = idx[(size_t)h * L + i0 + r];
      const size_t dst = ((size_t)h * C + i0 + r) * VPR + c;
      if (Qh4) st_stream(ld_stream(&Q4[((size_t)t * Hq + h) * VPR + c]), &Qh4[dst]);   // the fused layer reads Q
      if (Kh4) st_stream(K4[((size_t)t * Hkv + g) * VPR + c], &Kh4[dst]);               // and K in place
      v = V4[((size_t)t * Hkv + g) * VPR + c];
    }
    stage[e] = v;
  }
  __syncthreads();
  // Vht[h][dd][i0 + j .. i0 + j + EPV): gather EPV consecutive rows of column dd from the stage.
  const T* st = reinterpret_cast<const T*>(stage);
  for (int e = threadIdx.x; e < D * (kTileRows / EPV); e += 256) {
    const int dd = e / (kTileRows / EPV), j0 = (e % (kTileRows / EPV)) * EPV;
    T vals[EPV];
#pragma unroll
    for (int u = 0; u < EPV; ++u) vals[u] = st[(j0 + u) * D + dd];
    uint4 w;
    __builtin_memcpy(&w, vals, 16);
    *reinterpret_cast<uint4*>(Vht + ((size_t)h * D + dd) * C + i0 + j0) = w;
  }
}

// Compressed rows per block of the bf16 V^T gather (256 threads): 128 at d = 128, 256 at d = 64.
template <int D>
constexpr int vt_block_rows() { return 64 * (4 / (D / 64)); }

// The rows no head selected: Y = X (or +0.0).  The fused layer's attention epilogue writes the rest.
// A block of 256 threads takes 256 consecutive tokens of one head.  Their inverse-map entries are read with one
// coalesced load into LDS, and a block whose tokens are all selected stops there.  Then VPR
// consecutive lanes move one 16-byte chunk each of a row, so every store instruction writes whole
// rows: whole cache lines, which the streaming hint needs.  Rows written one 16-byte chunk per
// instruction lose the L2's merging, which cost 3.3 ms on a 131072-token layer keeping a quarter of
// its tokens.  Measured at L = 131072 (32 heads): a layer keeping nearly every row took 75.6 us when
// every lane read its row's inverse-map entry itself.
template <typename T, int D>
__device__ __forceinline__ void fill_unselected_block(const int32_t* __restrict__ inv, const T* __restrict__ X,
                                                      T* __restrict__ Y, int64_t L, int Hq, int h, int64_t bx,
                                                      int32_t* sinv) {   // LDS, 260 entries
  constexpr int VPR = D * (int)sizeof(T) / 16;
  constexpr int TPB = 256 / VPR;                  // rows per pass; VPR passes cover the 256 tokens
  const int c = threadIdx.x % VPR;
  const int64_t base = bx * 256;
  const int64_t tt = base + threadIdx.x;
  const int32_t mine = tt < L ? inv[(size_t)h * L + tt] : 0;
  sinv[threadIdx.x] = mine;
  if ((threadIdx.x & 63) == 0) sinv[256 + threadIdx.x / 64] = 0;
  const bool wave_any = __builtin_amdgcn_ballot_w64(mine < 0) != 0;
  if (wave_any && (threadIdx.x & 63) == 0) sinv[256 + threadIdx.x / 64] = 1;
  __syncthreads();
  if ((sinv[256] | sinv[257] | sinv[258] | sinv[259]) == 0) return;   // every token of the block is selected
  const uint4* X4 = reinterpret_cast<const uint4*>(X);
  // in batches of 8 rows, every load of a batch before its stores: with one branch per row, a load
  // placed after the previous row's store waited for it (one memory round trip per row)
  constexpr int NB = VPR < 8 ? VPR : 8;
#pragma unroll
  for (int p0 = 0; p0 < VPR; p0 += NB) {
    uint4 xv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int r = (p0 + b) * TPB + (int)threadIdx.x / VPR;
      const int64_t t = base + r;
      xv[b] = make_uint4(0, 0, 0, 0);
      if (X4 && t < L && sinv[r] < 0) xv[b] = ld_stream(&X4[((size_t)t * Hq + h) * VPR + c]);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int r = (p0 + b) * TPB + (int)threadIdx.x / VPR;
      const int64_t t = base + r;
      if (t >= L || sinv[r] >= 0) continue;
      st_stream(xv[b], reinterpret_cast<uint4*>(Y) + ((size_t)t * Hq + h) * VPR + c);
    }
  }
}

// bf16 V^T gather: Vht[h][c][i] = V[idx[h][i]][g][c] for rows i < L'.  No LDS: of a 256-thread
// block, wave w takes 64 consecutive compressed rows and 8 of a row's 16-byte chunks (64 columns);
// lane l loads chunk l % 8 of 8 consecutive rows (8 (l / 8) ..), so each load instruction reads 8
// half-rows of 128 bytes, transposes that 8 x 8 block of 16-bit values in registers with byte
// permutes, and stores one 16-byte piece (8 rows) per column.  A store instruction thus writes 8
// columns x 64 rows: 8 whole 128-byte lines.  Measured against staging the transpose through LDS
// behind a barrier (32/8 heads): 0.094 against 0.104 ms at L = 32768, 0.362 against 0.385 ms at
// L = 131072.  Loading the next 64-row group before storing the current one did not help: this
// kernel's reads and writes add up in HBM time (0.031 and 0.055 ms for each half alone at 32768),
// and a layout with each block's output contiguous ([C / 128][d][128]) was no faster than this one.
template <int D>
__device__ __forceinline__ void gather_vt_bf16_block(const uint16_t* __restrict__ V, const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ Lp_dev, int64_t L, int Hq, int Hkv,
                                                     int64_t C, uint16_t* __restrict__ Vht, unsigned bid) {
  constexpr int VPR = D / 8;            // 16-byte chunks per row
  constexpr int WPR = D / 64;           // waves across one row's chunks
  constexpr int TR = vt_block_rows<D>();
  static_assert(TR == 64 * (4 / WPR), "four waves of 64 rows per block");
  // block -> (KV group, row tile, head of the group): the G heads of one (group, tile) pair are
  // consecutive blocks of one XCD (block index % 8), so its L2 serves the V rows they share
  const int G = Hq / Hkv;
  const int64_t ntiles = (L + TR - 1) / TR;
  const int xcd = bid & 7, slot = bid >> 3;
  const int64_t pair = (int64_t)(slot / G) * 8 + xcd;
  if (pair >= ntiles * Hkv) return;
  const int g = (int)(pair % Hkv), h = g * G + slot % G;
  const int64_t Lp = Lp_dev[0];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int c = (w % WPR) * 8 + (l & 7);
  const int64_t r0 = (pair / Hkv) * TR + 64 * (w / WPR) + 8 * (l >> 3);
  if (r0 >= Lp) return;
  const uint4* V4 = reinterpret_cast<const uint4*>(V);
  const int32_t* hidx = idx + (size_t)h * L;
  // the 8 tokens first, then the 8 rows, with no per-row condition on a full group of 8: a load under
  // a per-row branch, or followed by a per-row select of its value, waited for every load before
  // it, so a thread's 8 token and 8 row loads ran one after another.  The group that crosses L'
  // reads row L' - 1 in place of the rows past it and zeroes them.
  int32_t tok[8];
  uint32_t v[8][4];
  if (r0 + 8 <= Lp) {
#pragma unroll
    for (int u = 0; u < 8; ++u) tok[u] = hidx[r0 + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint4 x = V4[((size_t)tok[u] * Hkv + g) * VPR + c];
      v[u][0] = x.x; v[u][1] = x.y; v[u][2] = x.z; v[u][3] = x.w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) tok[u] = hidx[r0 + u < Lp ? r0 + u : Lp - 1];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      uint4 x = V4[((size_t)tok[u] * Hkv + g) * VPR + c];
      if (r0 + u >= Lp) x = make_uint4(0, 0, 0, 0);   // columns of Vht past L' get zeros
      v[u][0] = x.x; v[u][1] = x.y; v[u][2] = x.z; v[u][3] = x.w;
    }
  }
  // column 2j of the chunk is the low half of word j of every row, column 2j+1 the high half; word
  // m of a column piece pairs rows 2m (low) and 2m+1 (high)
  uint16_t* dst = Vht + ((size_t)h * D + 8 * c) * C + r0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint4 lo, hi;
    lo.x = __builtin_amdgcn_perm(v[1][j], v[0][j], 0x05040100u);
    lo.y = __builtin_amdgcn_perm(v[3][j], v[2][j], 0x05040100u);
    lo.z = __builtin_amdgcn_perm(v[5][j], v[4][j], 0x05040100u);
    lo.w = __builtin_amdgcn_perm(v[7][j], v[6][j], 0x05040100u);
    hi.x = __builtin_amdgcn_perm(v[1][j], v[0][j], 0x07060302u);
    hi.y = __builtin_amdgcn_perm(v[3][j], v[2][j], 0x07060302u);
    hi.z = __builtin_amdgcn_perm(v[5][j], v[4][j], 0x07060302u);
    hi.w = __builtin_amdgcn_perm(v[7][j], v[6][j], 0x07060302u);
    st_stream(lo, reinterpret_cast<uint4*>(dst + (size_t)(2 * j) * C));
    st_stream(hi, reinterpret_cast<uint4*>(dst + (size_t)(2 * j + 1) * C));
  }
}

template <int D>
__global__ __launch_bounds__(256) void gather_vt_bf16_kernel(const uint16_t* __restrict__ V, const int32_t* __restrict__ idx,
                                                             const int32_t* __restrict__ Lp_dev, int64_t L, int Hq, int Hkv,
                                                             int64_t C, uint16_t* __restrict__ Vht) {
  gather_vt_bf16_block<D>(V, idx, Lp_dev, L, Hq, Hkv, C, Vht, blockIdx.x);
}

// The fused layer's V^T gather with its unselected-row fill in the same launch: blocks [0, ngather)
// gather, the Hq * ceil(L / 256) blocks after them fill (the two touch disjoint memory), token tile
// outermost.
template <int D>
__global__ __launch_bounds__(256) void gather_vt_fill_bf16_kernel(const uint16_t* __restrict__ V,
                                                                  const int32_t* __restrict__ idx,
                                                                  const int32_t* __restrict__ Lp_dev, int64_t L, int Hq,
                                                                  int Hkv, int64_t C, uint16_t* __restrict__ Vht,
                                                                  unsigned ngather, const int32_t* __restrict__ inv,
                                                                  const uint16_t* __restrict__ X, uint16_t* __restrict__ Y) {
  __shared__ int32_t sinv[260];          // the fill's inverse-map entries and wave flags
  if (blockIdx.x < ngather) {
    gather_vt_bf16_block<D>(V, idx, Lp_dev, L, Hq, Hkv, C, Vht, blockIdx.x);
  } else {
    // token-major, as the scatter: the Hq blocks of one 256-token tile are consecutive
    const int64_t f = blockIdx.x - ngather;
    fill_unselected_block<uint16_t, D>(inv, X, Y, L, Hq, (int)(f % Hq), f / Hq, sinv);
  }
}

// Row copies of the bf16 gather: Qh[h][i] = Q[idx[h][i]][h] and Kh[h][i] = K[idx[h][i]][g] for
// rows i < L'.  VPR consecutive lanes move one row, 16 bytes each, so a wave's load covers whole
// rows; a thread moves one chunk of Q and one of K.  No LDS, so 8 waves per SIMD stay resident.  One
// row per thread measured fastest at L = 131072 and 32768 (0.966 / 0.257 ms for the stage, against
// 0.988 / 0.263 with 2 rows, 1.025 / 0.287 with 4 and 1.061 / 0.306 with 8, all loads issued before
// the stores).  Block -> (KV group, row tile, head) as in the transposing kernel, so that one XCD's
// L2 serves the K rows the group's heads share.
template <int D>
constexpr int rows_block_rows() { return 256 / (D / 8); }

template <int D>
__device__ __forceinline__ void gather_rows_bf16_block(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                       const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ Lp_dev, int64_t L, int Hq, int Hkv,
                                                       int64_t C, uint16_t* __restrict__ Qh, uint16_t* __restrict__ Kh,
                                                       unsigned bid) {
  constexpr int VPR = D / 8, TRC = rows_block_rows<D>();   // rows per block
  const int G = Hq / Hkv;
  const int64_t ntiles = (L + TRC - 1) / TRC;
  const int xcd = bid & 7, slot = bid >> 3;
  const int64_t pair = (int64_t)(slot / G) * 8 + xcd;
  if (pair >= ntiles * Hkv) return;
  const int g = (int)(pair % Hkv), h = g * G + slot % G;
  const int64_t Lp = Lp_dev[0];
  const int64_t i = (pair / Hkv) * TRC + threadIdx.x / VPR;
  if (i >= Lp) return;
  const int c = threadIdx.x % VPR;
  const size_t t = (size_t)idx[(size_t)h * L + i];
  const size_t dst = ((size_t)h * C + i) * VPR + c;
  uint4 qv, kv;
  if (Qh) qv = ld_stream(reinterpret_cast<const uint4*>(Q) + (t * Hq + h) * VPR + c);
  if (Kh) kv = reinterpret_cast<const uint4*>(K)[(t * Hkv + g) * VPR + c];
  if (Qh) st_stream(qv, reinterpret_cast<uint4*>(Qh) + dst);
  if (Kh) st_stream(kv, reinterpret_cast<uint4*>(Kh) + dst);
}

template <int D>
__global__ __launch_bounds__(256) void gather_rows_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                               const int32_t* __restrict__ idx,
                                                               const int32_t* __restrict__ Lp_dev, int64_t L, int Hq,
                                                               int Hkv, int64_t C, uint16_t* __restrict__ Qh,
                                                               uint16_t* __restrict__ Kh) {
  gather_rows_bf16_block<D>(Q, K, idx, Lp_dev, L, Hq, Hkv, C, Qh, Kh, blockIdx.x);
}

// V [L][Hkv][d] -> Vt [Hkv][d][C], columns L .. C-1 zero (the dense path's value layout).
template <typename T, int D>
__global__ __launch_bounds__(256) void transpose_v_kernel(const T* __restrict__ V, int64_t L, int Hkv,
                                                          int64_t C, T* __restrict__ Vt) {
  constexpr int VPR = D * (int)sizeof(T) / 16;
  constexpr int EPV = 16 / (int)sizeof(T);
  __shared__ uint4 stage[kTileRows * VPR];
  const int g = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kTileRows;
  const uint4* V4 = reinterpret_cast<const uint4*>(V);
  for (int e = threadIdx.x; e < kTileRows * VPR; e += 256) {
    const int r = e / VPR, c = e % VPR;
    stage[e] = t0 + r < L ? V4[((size_t)(t0 + r) * Hkv + g) * VPR + c] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  const T* st = reinterpret_cast<const T*>(stage);
  for (int e = threadIdx.x; e < D * (kTileRows / EPV); e += 256) {
    const int dd = e / (kTileRows / EPV), j0 = (e % (kTileRows / EPV)) * EPV;
    T vals[EPV];
#pragma unroll
    for (int u = 0; u < EPV; ++u) vals[u] = st[(j0 + u) * D + dd];
    uint4 w;
    __builtin_memcpy(&w, vals, 16);
    *reinterpret_cast<uint4*>(Vt + ((size_t)g * D + dd) * C + t0 + j0) = w;
  }
}

// x + o on one 16-byte vector, float32 sum rounded once to the storage type.
template <typename T>
__device__ __forceinline__ uint4 add_vec(uint4 x, uint4 o) {
  uint4 y;
  if constexpr (sizeof(T) == 2) {
    const uint32_t xa[4] = {x.x, x.y, x.z, x.w}, oa[4] = {o.x, o.y, o.z, o.w};
    uint32_t ya[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_to_f32((uint16_t)xa[j]) + bf16_to_f32((uint16_t)oa[j]);
      const float hi = bf16_to_f32((uint16_t)(xa[j] >> 16)) + bf16_to_f32((uint16_t)(oa[j] >> 16));
      ya[j] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
    }
    y = make_uint4(ya[0], ya[1], ya[2], ya[3]);
  } else {
    y.x = __float_as_uint(__uint_as_float(x.x) + __uint_as_float(o.x));
    y.y = __float_as_uint(__uint_as_float(x.y) + __uint_as_float(o.y));
    y.z = __float_as_uint(__uint_as_float(x.z) + __uint_as_float(o.z));
    y.w = __float_as_uint(__uint_as_float(x.w) + __uint_as_float(o.w));
  }
  return y;
}

// Pass over Y using the inverse map: every (t, h) row is produced exactly once.  Grid (token tiles,
// heads); VPR threads cover one 16-byte-vector row, so no index division is needed.
template <typename T, int D>
__global__ __launch_bounds__(256) void scatter_inv_kernel(const T* __restrict__ Oh, const int32_t* __restrict__ inv,
                                                          const T* X, T* Y, int64_t L, int Hq, int64_t C) {
  constexpr int VPR = D * (int)sizeof(T) / 16;
  constexpr int TPB = 256 / VPR;                  // tokens per block
  // token-major: the Hq blocks of one token tile are consecutive, so the rows of a token (all heads,
  // Hq * d contiguous elements of X and Y) are read and written close together in time.  Head-major
  // order (each head's tokens first) touched 256-byte pieces 8 KB apart: 0.605 against 0.559 ms at
  // L = 131072, 0.181 against 0.148 ms at 32768.
  const int h = (int)(blockIdx.x % (unsigned)Hq), c = threadIdx.x % VPR;
  const int64_t t = (int64_t)(blockIdx.x / (unsigned)Hq) * TPB + threadIdx.x / VPR;
  if (t >= L) return;
  const uint4* O4 = reinterpret_cast<const uint4*>(Oh);
  const uint4* X4 = reinterpret_cast<const uint4*>(X);
  uint4* Y4 = reinterpret_cast<uint4*>(Y);
  const size_t e = ((size_t)t * Hq + h) * VPR + c;
  const int32_t j = inv[(size_t)h * L + t];
  if (j < 0) {
    if ((const void*)X == (const void*)Y) return;   // in place: the row already holds X
    st_stream(X4 ? ld_stream(&X4[e]) : make_uint4(0, 0, 0, 0), &Y4[e]);
  } else {
    const uint4 o = ld_stream(&O4[((size_t)h * C + j) * VPR + c]);
    st_stream(X4 ? add_vec<T>(ld_stream(&X4[e]), o) : o, &Y4[e]);
  }
}



// Index-driven variant (no inverse map): Y must already hold X (or zeros for a pure decompress).
template <typename T, int D>
__global__ __launch_bounds__(256) void scatter_idx_kernel(const T* __restrict__ Oh, const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ Lp_dev, bool add,
                                                          T* Y, int64_t L, int Hq, int64_t C) {
  constexpr int VPR = D * (int)sizeof(T) / 16;
  const int64_t Lp = Lp_dev[0];
  const uint4* O4 = reinterpret_cast<const uint4*>(Oh);
  uint4* Y4 = reinterpret_cast<uint4*>(Y);
  const size_t n = (size_t)Hq * Lp * VPR;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) {
    const int c = (int)(e % VPR);
    const size_t hi = e / VPR;
    const int h = (int)(hi / Lp);
    const int64_t i = (int64_t)(hi % Lp);
    const int64_t t = idx[(size_t)h * L + i];
    const size_t dst = ((size_t)t * Hq + h) * VPR + c;
    const uint4 o = O4[((size_t)h * C + i) * VPR + c];
    Y4[dst] = add ? add_vec<T>(Y4[dst], o) : o;
  }
}

__global__ void copy16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

static unsigned grid_for(size_t n) {
  const size_t b = (n + 255) / 256;
  return (unsigned)(b < 16384 ? (b ? b : 1) : 16384);
}

template <typename T, int D>
static hipError_t run_gather(const void* Q, const void* K, const void* V, const int32_t* idx,
                             const int32_t* Lp_dev, int64_t L, int Hq, int Hkv, int64_t C, void* Qh,
                             void* Kh, void* Vht, hipStream_t st, const int32_t* inv, const void* X, void* Y) {
  if constexpr (sizeof(T) == 2) {
    const auto Qt = static_cast<const uint16_t*>(Q), Kt = static_cast<const uint16_t*>(K);
    const auto Vt = static_cast<const uint16_t*>(V);
    // blocks of the transposing V^T gather and of the row copies (Q_hat, K_hat); both multiples of 8
    constexpr int TR = vt_block_rows<D>(), TRC = rows_block_rows<D>();
    const int64_t pairs = (L + TR - 1) / TR * Hkv, rpairs = (L + TRC - 1) / TRC * Hkv;
    const unsigned nblk = (unsigned)((pairs + 7) / 8 * 8 * (Hq / Hkv));
    const unsigned nrow = (unsigned)((rpairs + 7) / 8 * 8 * (Hq / Hkv));
    // the row copies, then the transposes: as fast as one launch interleaving the two (groups of 8
    // blocks in proportion) at 32768 and 131072 tokens, 1.7 us slower at 4096
    if (Qh || Kh)
      gather_rows_bf16_kernel<D><<<nrow, 256, 0, st>>>(Qt, Kt, idx, Lp_dev, L, Hq, Hkv, C, static_cast<uint16_t*>(Qh),
                                                       static_cast<uint16_t*>(Kh));
    if (Y) {
      const unsigned nfill = (unsigned)((L + 255) / 256 * Hq);
      gather_vt_fill_bf16_kernel<D><<<nblk + nfill, 256, 0, st>>>(Vt, idx, Lp_dev, L, Hq, Hkv, C,
                                                                  static_cast<uint16_t*>(Vht), nblk, inv,
                                                                  static_cast<const uint16_t*>(X), static_cast<uint16_t*>(Y));
    } else {
      gather_vt_bf16_kernel<D><<<nblk, 256, 0, st>>>(Vt, idx, Lp_dev, L, Hq, Hkv, C, static_cast<uint16_t*>(Vht));
    }
  } else {
    if (Y) return hipErrorInvalidValue;   // the fused fill is bf16 only
    const dim3 grid((unsigned)((L + kTileRows - 1) / kTileRows), (unsigned)Hq);
    gather_kernel<T, D><<<grid, 256, 0, st>>>(static_cast<const T*>(Q), static_cast<const T*>(K),
                                              static_cast<const T*>(V), idx, Lp_dev, L, Hq, Hkv, C,
                                              static_cast<T*>(Qh), static_cast<T*>(Kh), static_cast<T*>(Vht));
  }
  return hipGetLastError();
}

hipError_t launch_gather(int dtype, int d, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const int32_t* Lp_dev, int64_t L, int Hq, int Hkv,
                         int64_t C, void* Qh, void* Kh, void* Vht, hipStream_t st, const int32_t* inv,
                         const void* X, void* Y) {
  if (Y && X == Y) Y = nullptr;          // in place: the unselected rows already hold X
  if (dtype == 1)
    return d == 128 ? run_gather<uint16_t, 128>(Q, K, V, idx, Lp_dev, L, Hq, Hkv, C, Qh, Kh, Vht, st, inv, X, Y)
                    : run_gather<uint16_t, 64>(Q, K, V, idx, Lp_dev, L, Hq, Hkv, C, Qh, Kh, Vht, st, inv, X, Y);
  return d == 128 ? run_gather<float, 128>(Q, K, V, idx, Lp_dev, L, Hq, Hkv, C, Qh, Kh, Vht, st, inv, X, Y)
                  : run_gather<float, 64>(Q, K, V, idx, Lp_dev, L, Hq, Hkv, C, Qh, Kh, Vht, st, inv, X, Y);
}

template <typename T, int D>
static hipError_t run_transpose(const void* V, int64_t L, int Hkv, int64_t C, void* Vt, hipStream_t st) {
  const dim3 grid((unsigned)(C / kTileRows), (unsigned)Hkv);
  transpose_v_kernel<T, D><<<grid, 256, 0, st>>>(static_cast<const T*>(V), L, Hkv, C, static_cast<T*>(Vt));
  return hipGetLastError();
}

hipError_t launch_transpose_v(int dtype, int d, const void* V, int64_t L, int Hkv, int64_t C,
                              void* Vt, hipStream_t st) {
  if (dtype == 1)
    return d == 128 ? run_transpose<uint16_t, 128>(V, L, Hkv, C, Vt, st)
                    : run_transpose<uint16_t, 64>(V, L, Hkv, C, Vt, st);
  return d == 128 ? run_transpose<float, 128>(V, L, Hkv, C, Vt, st)
                  : run_transpose<float, 64>(V, L, Hkv, C, Vt, st);
}

template <typename T, int D>
static hipError_t run_scatter(const void* Oh, const int32_t* idx, const int32_t* inv,
                              const int32_t* Lp_dev, const void* X, void* Y, int64_t L, int Hq,
                              int64_t C, hipStream_t st) {
  constexpr int VPR = D * (int)sizeof(T) / 16;
  const size_t n = (size_t)L * Hq * VPR;
  if (inv) {
    constexpr int TPB = 256 / VPR;
    const dim3 grid((unsigned)((L + TPB - 1) / TPB * Hq));
    scatter_inv_kernel<T, D><<<grid, 256, 0, st>>>(static_cast<const T*>(Oh), inv, static_cast<const T*>(X),
                                                   static_cast<T*>(Y), L, Hq, C);
    return hipGetLastError();
  }
  if (X == nullptr) {
    hipError_t e = launch_fill_zero(Y, n * 16, st);
    if (e != hipSuccess) return e;
  } else if (X != Y) {
    copy16_kernel<<<grid_for(n), 256, 0, st>>>(static_cast<const uint4*>(X), static_cast<uint4*>(Y), n);
  }
  scatter_idx_kernel<T, D><<<grid_for(n), 256, 0, st>>>(static_cast<const T*>(Oh), idx, Lp_dev, X != nullptr,
                                                        static_cast<T*>(Y), L, Hq, C);
  return hipGetLastError();
}

hipError_t launch_scatter(int dtype, int d, const void* Oh, const int32_t* idx, const int32_t* inv,
                          const int32_t* Lp_dev, const void* X, void* Y, int64_t L, int Hq, int64_t C,
                          hipStream_t st) {
  if (dtype == 1)
    return d == 128 ? run_scatter<uint16_t, 128>(Oh, idx, inv, Lp_dev, X, Y, L, Hq, C, st)
                    : run_scatter<uint16_t, 64>(Oh, idx, inv, Lp_dev, X, Y, L, Hq, C, st);
  return d == 128 ? run_scatter<float, 128>(Oh, idx, inv, Lp_dev, X, Y, L, Hq, C, st)
                  : run_scatter<float, 64>(Oh, idx, inv, Lp_dev, X, Y, L, Hq, C, st);
}

}  // namespace tsa

// Compress and decompress (papernotes.org reading notes, "Key design 1"; bxzpzcl.cn article,
// section 1.1 gather / zeros_like + scatter_): pure data movement in 16-byte vectors.
//
// gather : per query head, rows idx[h][0..L') of Q, K, V -> dense Qh, Kh [Hq][C][d] and the
//          transposed Vht [Hq][d][C] (bf16: 8 x 8 blocks transposed in registers; fp32: a 64-row
//          tile staged in LDS and written column-major so the stores stay contiguous).
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
      if (Qh4) st_stream(ld_stream(&Q4[((size_t)t * Hq + h) * VPR + c]), &Qh4[dst]);   // the fused layer reads Q in place
      st_stream(K4[((size_t)t * Hkv + g) * VPR + c], &Kh4[dst]);
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

// bf16: a thread owns one 16-byte chunk (8 columns) of 8 consecutive compressed rows.  It loads that
// chunk of the 8 gathered rows (16 threads cover a 256-byte row, so the loads stay coalesced) and
// transposes the 8 x 8 block of 16-bit values in registers with byte permutes.  The resulting
// 16-byte pieces (8 rows of one column) are regrouped through LDS, [column][row] with a XOR swizzle
// of the piece slot, so that each column's run of TR rows leaves as contiguous 16-byte stores.
template <int D>
__global__ __launch_bounds__(256) void gather_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V, const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ Lp_dev, int64_t L, int Hq, int Hkv,
                                                          int64_t C, uint16_t* __restrict__ Qh, uint16_t* __restrict__ Kh,
                                                          uint16_t* __restrict__ Vht) {
  constexpr int VPR = D / 8;            // 16-byte chunks per row
  constexpr int NG = 256 / VPR;         // groups of 8 rows per block
  constexpr int TR = NG * 8;            // rows per block (128 for d = 128, 256 for d = 64)
  constexpr int PPC = TR / 8;           // 16-byte pieces per column in the block (= NG)
  __shared__ uint4 tile[D * PPC];       // [column][piece], piece slot swizzled
  // block -> (KV group, row tile, head of the group): the G heads of one (group, tile) pair are
  // consecutive blocks of one XCD (blockIdx % 8), so its L2 serves the K/V rows they share
  const int G = Hq / Hkv;
  const int64_t ntiles = (L + TR - 1) / TR;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int64_t pair = (int64_t)(slot / G) * 8 + xcd;
  if (pair >= ntiles * Hkv) return;
  const int g = (int)(pair % Hkv), h = g * G + slot % G;
  const int64_t Lp = Lp_dev[0];
  const int64_t b0 = (pair / Hkv) * TR;
  if (b0 >= Lp) return;
  const int c = threadIdx.x % VPR, grp = threadIdx.x / VPR;
  const int64_t r0 = b0 + grp * 8;
  const uint4* Q4 = reinterpret_cast<const uint4*>(Q);
  const uint4* K4 = reinterpret_cast<const uint4*>(K);
  const uint4* V4 = reinterpret_cast<const uint4*>(V);
  uint4* Qh4 = reinterpret_cast<uint4*>(Qh);
  uint4* Kh4 = reinterpret_cast<uint4*>(Kh);
  uint32_t v[8][4];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t i = r0 + u;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (i < Lp) {
      const int64_t t = idx[(size_t)h * L + i];
      const size_t dst = ((size_t)h * C + i) * VPR + c;
      if (Qh4) st_stream(ld_stream(&Q4[((size_t)t * Hq + h) * VPR + c]), &Qh4[dst]);   // the fused layer reads Q in place
      st_stream(K4[((size_t)t * Hkv + g) * VPR + c], &Kh4[dst]);
      x = V4[((size_t)t * Hkv + g) * VPR + c];
    }
    v[u][0] = x.x; v[u][1] = x.y; v[u][2] = x.z; v[u][3] = x.w;
  }
  // column 2j of the chunk is the low half of word j of every row, column 2j+1 the high half; word
  // m of a column piece pairs rows 2m (low) and 2m+1 (high).  Piece grp of column col sits in slot
  // grp ^ (col % PPC) of that column's LDS row.
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
    const int col = 8 * c + 2 * j;
    tile[col * PPC + (grp ^ (col % PPC))] = lo;
    tile[(col + 1) * PPC + (grp ^ ((col + 1) % PPC))] = hi;
  }
  __syncthreads();
  // each column's TR rows: PPC consecutive lanes store its PPC pieces contiguously
  const int64_t nrows = Lp - b0 < TR ? Lp - b0 : TR;
  for (int e = threadIdx.x; e < D * PPC; e += 256) {
    const int col = e / PPC, q = e % PPC;
    if ((int64_t)q * 8 >= nrows) continue;
    st_stream(tile[col * PPC + (q ^ (col % PPC))], reinterpret_cast<uint4*>(Vht + ((size_t)h * D + col) * C + b0 + 8 * q));
  }
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
  const int h = blockIdx.y, c = threadIdx.x % VPR;
  const int64_t t = (int64_t)blockIdx.x * TPB + threadIdx.x / VPR;
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

// The rows no head selected: Y = X (or +0.0).  The fused layer's attention epilogue writes the rest.
// A block takes 256 consecutive tokens of one head.  Their inverse-map entries are read with one
// coalesced load into LDS, and a block whose tokens are all selected stops there.  Then VPR
// consecutive lanes move one 16-byte chunk each of a row, so every store instruction writes whole
// rows: whole cache lines, which the streaming hint needs.  Rows written one 16-byte chunk per
// instruction lose the L2's merging, which cost 3.3 ms on a 131072-token layer keeping a quarter of
// its tokens.  Measured at L = 131072 (32 heads): a layer keeping nearly every row took 75.6 us when
// every lane read its row's inverse-map entry itself.
template <typename T, int D>
__global__ __launch_bounds__(256) void fill_unselected_kernel(const int32_t* __restrict__ inv, const T* __restrict__ X,
                                                              T* __restrict__ Y, int64_t L, int Hq) {
  constexpr int VPR = D * (int)sizeof(T) / 16;
  constexpr int TPB = 256 / VPR;                  // rows per pass; VPR passes cover the 256 tokens
  __shared__ int32_t sinv[256];
  const int h = blockIdx.y, c = threadIdx.x % VPR;
  const int64_t base = (int64_t)blockIdx.x * 256;
  const int64_t tt = base + threadIdx.x;
  const int32_t mine = tt < L ? inv[(size_t)h * L + tt] : 0;
  sinv[threadIdx.x] = mine;
  if (!__syncthreads_or(mine < 0)) return;        // every token of the block is selected
  const uint4* X4 = reinterpret_cast<const uint4*>(X);
#pragma unroll
  for (int p = 0; p < VPR; ++p) {
    const int r = p * TPB + (int)threadIdx.x / VPR;
    const int64_t t = base + r;
    if (t >= L || sinv[r] >= 0) continue;
    const size_t e = ((size_t)t * Hq + h) * VPR + c;
    st_stream(X4 ? ld_stream(&X4[e]) : make_uint4(0, 0, 0, 0), reinterpret_cast<uint4*>(Y) + e);
  }
}

template <typename T, int D>
static hipError_t run_fill_unselected(const int32_t* inv, const void* X, void* Y, int64_t L, int Hq, hipStream_t st) {
  const dim3 grid((unsigned)((L + 255) / 256), (unsigned)Hq);
  fill_unselected_kernel<T, D><<<grid, 256, 0, st>>>(inv, static_cast<const T*>(X), static_cast<T*>(Y), L, Hq);
  return hipGetLastError();
}

hipError_t launch_fill_unselected(int dtype, int d, const int32_t* inv, const void* X, void* Y, int64_t L, int Hq,
                                  hipStream_t st) {
  if (X == Y) return hipSuccess;             // in place: those rows already hold X
  if (dtype == 1)
    return d == 128 ? run_fill_unselected<uint16_t, 128>(inv, X, Y, L, Hq, st)
                    : run_fill_unselected<uint16_t, 64>(inv, X, Y, L, Hq, st);
  return d == 128 ? run_fill_unselected<float, 128>(inv, X, Y, L, Hq, st)
                  : run_fill_unselected<float, 64>(inv, X, Y, L, Hq, st);
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
                             void* Kh, void* Vht, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    constexpr int TR = 256 / (D / 8) * 8;
    const int64_t pairs = (L + TR - 1) / TR * Hkv;
    const unsigned nblk = (unsigned)((pairs + 7) / 8 * 8 * (Hq / Hkv));
    gather_bf16_kernel<D><<<nblk, 256, 0, st>>>(static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                                                static_cast<const uint16_t*>(V), idx, Lp_dev, L, Hq, Hkv, C,
                                                static_cast<uint16_t*>(Qh), static_cast<uint16_t*>(Kh),
                                                static_cast<uint16_t*>(Vht));
  } else {
    const dim3 grid((unsigned)((L + kTileRows - 1) / kTileRows), (unsigned)Hq);
    gather_kernel<T, D><<<grid, 256, 0, st>>>(static_cast<const T*>(Q), static_cast<const T*>(K),
                                              static_cast<const T*>(V), idx, Lp_dev, L, Hq, Hkv, C,
                                              static_cast<T*>(Qh), static_cast<T*>(Kh), static_cast<T*>(Vht));
  }
  return hipGetLastError();
}

hipError_t launch_gather(int dtype, int d, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const int32_t* Lp_dev, int64_t L, int Hq, int Hkv,
                         int64_t C, void* Qh, void* Kh, void* Vht, hipStream_t st) {
  if (dtype == 1)
    return d == 128 ? run_gather<uint16_t, 128>(Q, K, V, idx, Lp_dev, L, Hq, Hkv, C, Qh, Kh, Vht, st)
                    : run_gather<uint16_t, 64>(Q, K, V, idx, Lp_dev, L, Hq, Hkv, C, Qh, Kh, Vht, st);
  return d == 128 ? run_gather<float, 128>(Q, K, V, idx, Lp_dev, L, Hq, Hkv, C, Qh, Kh, Vht, st)
                  : run_gather<float, 64>(Q, K, V, idx, Lp_dev, L, Hq, Hkv, C, Qh, Kh, Vht, st);
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
    const dim3 grid((unsigned)((L + TPB - 1) / TPB), (unsigned)Hq);
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

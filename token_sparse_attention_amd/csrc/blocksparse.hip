// Block sparsity stacked on the token selection: inside the compressed space (Q_hat, K_hat, V_hat
// of one head are dense and contiguous) the causal attention is restricted to a per-query-block set
// of key blocks (papernotes.org reading notes, "Key findings": the token filter composes with a
// block-sparse kernel; bxzpzcl.cn article, section 3.2: token selection first, then block-sparse
// computation).  The pages give no block rule of their own; this one mirrors the coverage budget:
//
//   pool   : the rows of every block of kBlock compressed rows are averaged (float64 sum in row
//            order, one division, rounded once to float32) into qbar, kbar [Hq][NB][d];
//   logits : zl[h][I][J] = <qbar_I, kbar_J> / sqrt(d) for J <= I, a tiled float64 product;
//   select : query block I weighs its causal key blocks J <= I by a_J = softmax_J(zl[h][I][J])
//            (float64) and keeps the fewest heaviest (ties: lower J) whose weight reaches
//            gamma (all of them when gamma >= 1 or no prefix does), plus J = 0 and J = I.  The kept
//            blocks are listed ascending: list [Hq][NB][NB] (uint16), count [Hq][NB].
//
// The attention kernel then walks only the listed blocks' key tiles (attention.hip).
#include "kern_common.h"
#include "tsa_internal.h"

namespace tsa {

constexpr int kSortMax = kMaxKeyBlocks;       // candidates sorted in LDS per query block

template <typename T, int D>
__global__ __launch_bounds__(256) void block_pool_kernel(const T* __restrict__ Qh, const T* __restrict__ Kh,
                                                         const int32_t* __restrict__ Lp_dev, int64_t C, int nbmax,
                                                         float* __restrict__ qbar, float* __restrict__ kbar) {
  const int b = blockIdx.x, h = blockIdx.y;
  const int64_t Lp = Lp_dev[0];
  const int64_t r0 = (int64_t)b * kBlock;
  if (r0 >= Lp || threadIdx.x >= 2 * D) return;
  const int64_t r1 = r0 + kBlock < Lp ? r0 + kBlock : Lp;
  const bool isk = threadIdx.x >= D;
  const int c = threadIdx.x % D;
  const T* src = (isk ? Kh : Qh) + ((size_t)h * C) * D + c;
  double acc = 0.0;
  int64_t r = r0;
  for (; r + 8 <= r1; r += 8) {             // loads first, then the adds in row order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = to_f32(src[(size_t)(r + u) * D]);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += (double)v[u];
  }
  for (; r < r1; ++r) acc += (double)to_f32(src[(size_t)r * D]);
  (isk ? kbar : qbar)[((size_t)h * nbmax + b) * D + c] = (float)(acc / (double)(r1 - r0));
}

// zl[h][I][J] = <qbar[h][I], kbar[h][J]> / sqrt(d) for J <= I (float64 sums of exact float32
// products), one 64 x 64 tile of (I, J) per workgroup: the pooled rows are read once per tile
// instead of once per query block.  Each thread owns a 4 x 4 patch.
template <int D>
__global__ __launch_bounds__(256) void block_logits_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                           const int32_t* __restrict__ Lp_dev, int nbmax,
                                                           double* __restrict__ zl) {
  constexpr int T = 64, KC = 32;                 // tile edge, head-dim chunk staged at a time
  __shared__ float qs[T][KC + 1], ks[T][KC + 1];
  const int h = blockIdx.z, I0 = blockIdx.y * T, J0 = blockIdx.x * T;
  const int nb = (int)((Lp_dev[0] + kBlock - 1) / kBlock);
  if (J0 > I0 || I0 >= nb) return;               // causal tiles only
  const int tid = threadIdx.x, ti = tid / 16, tj = tid % 16;
  double acc[4][4] = {};
  for (int k0 = 0; k0 < D; k0 += KC) {
    for (int e = tid; e < T * KC; e += 256) {
      const int r = e / KC, cc = e % KC;
      qs[r][cc] = I0 + r < nb ? qbar[((size_t)h * nbmax + I0 + r) * D + k0 + cc] : 0.f;
      ks[r][cc] = J0 + r < nb ? kbar[((size_t)h * nbmax + J0 + r) * D + k0 + cc] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int cc = 0; cc < KC; ++cc) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = (double)qs[ti + 16 * u][cc];
        b[u] = (double)ks[tj + 16 * u][cc];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
  const double rsd = sqrt((double)D);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int I = I0 + ti + 16 * u, J = J0 + tj + 16 * v;
      if (I < nb && J <= I) zl[((size_t)h * nbmax + I) * nbmax + J] = acc[u][v] / rsd;
    }
}

// "x comes before y": heavier first, then lower block index
__device__ __forceinline__ bool before(double ax, int jx, double ay, int jy) {
  return ax > ay || (ax == ay && jx < jy);
}

__global__ __launch_bounds__(256) void block_select_kernel(const double* __restrict__ zl, const int32_t* __restrict__ Lp_dev,
                                                           int nbmax, double gamma, uint16_t* __restrict__ list,
                                                           int32_t* __restrict__ count) {
  __shared__ double av[kSortMax];
  __shared__ uint16_t jv[kSortMax];
  __shared__ double red[4];
  __shared__ uint32_t kept[kSortMax / 32];
  __shared__ uint32_t wbase[kSortMax / 32];
  __shared__ int cut;
  const int I = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t Lp = Lp_dev[0];
  const int nb = (int)((Lp + kBlock - 1) / kBlock);
  if (I >= nb) {
    if (tid == 0) count[(size_t)h * nbmax + I] = 0;
    return;
  }
  const int n = I + 1;
  int P2 = 1;
  while (P2 < n) P2 <<= 1;
  for (int i = tid; i < kSortMax / 32; i += 256) kept[i] = 0;
  if (tid == 0) cut = n - 1;
  __syncthreads();

  // logits (block_logits_kernel), max
  const double* zrow = zl + ((size_t)h * nbmax + I) * nbmax;
  double mx = -INFINITY;
  for (int J = tid; J < n; J += 256) {
    const double z = zrow[J];
    av[J] = z;
    mx = fmax(mx, z);
  }
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  mx = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  __syncthreads();
  // weights
  double sum = 0.0;
  for (int J = tid; J < n; J += 256) {
    const double e = exp(av[J] - mx);
    av[J] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  if (lane == 0) red[w] = sum;
  __syncthreads();
  sum = (red[0] + red[1]) + (red[2] + red[3]);
  for (int J = tid; J < P2; J += 256) {
    if (J < n) {
      av[J] = av[J] / sum;
      jv[J] = (uint16_t)J;
    } else {
      av[J] = -1.0;                          // padding sorts last
      jv[J] = 0xFFFF;
    }
  }
  __syncthreads();
  // bitonic sort of P2 (weight, block) pairs into "before" order; a stage of distance j = 2^s has
  // P2 / 2 pairs, and pair q is (i, i + j) with i = q with a zero bit inserted at bit s, so no
  // thread idles on the upper half of a pair
  for (int k = 2; k <= P2; k <<= 1) {
    for (int j = k >> 1, sj = __ffs(j) - 1; j > 0; j >>= 1, --sj) {
      for (int q = tid; q < P2 / 2; q += 256) {
        const int i = ((q >> sj) << (sj + 1)) | (q & (j - 1)), p = i + j;
        const bool up = (i & k) == 0;          // this run is sorted in "before" order
        const double a0 = av[i], a1 = av[p];
        const int j0 = jv[i], j1 = jv[p];
        const bool swap = up ? before(a1, j1, a0, j0) : before(a0, j0, a1, j1);
        if (swap) {
          av[i] = a1; av[p] = a0;
          jv[i] = (uint16_t)j1; jv[p] = (uint16_t)j0;
        }
      }
      __syncthreads();
    }
  }
  // cumulative weight in sorted order: contiguous chunks per thread, chunk totals scanned in
  // thread order, then each thread finds its first position reaching gamma
  if (gamma < 1.0) {
    const int per = (n + 255) / 256, lo = tid * per, hi = lo + per < n ? lo + per : n;
    double part = 0.0;
    for (int i = lo; i < hi; ++i) part += av[i];
    // exclusive scan of the 256 chunk totals in thread order: a shuffle scan within each wave,
    // then the wave totals in wave order (a fixed tree, so the result is deterministic)
    double incl = part;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double nb2 = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += nb2;
    }
    __syncthreads();                          // red[] is free again
    if (lane == 63) red[w] = incl;
    __syncthreads();
    double cum = incl - part;
    for (int v = 0; v < w; ++v) cum += red[v];
    for (int i = lo; i < hi; ++i) {
      cum += av[i];
      if (cum >= gamma) {
        atomicMin(&cut, i);
        break;
      }
    }
    __syncthreads();
  }
  const int p = cut;
  for (int i = tid; i <= p; i += 256) atomicOr(&kept[jv[i] >> 5], 1u << (jv[i] & 31));
  if (tid == 0) {
    atomicOr(&kept[0], 1u);
    atomicOr(&kept[I >> 5], 1u << (I & 31));
  }
  __syncthreads();
  // ascending list: exclusive popcount scan over the bitmap words
  const int nw = (n + 31) / 32;              // at most kSortMax / 32 = 128: two words per lane
  if (w == 0) {
    const uint32_t c0 = 2 * lane < nw ? (uint32_t)__popc(kept[2 * lane]) : 0u;
    const uint32_t c1 = 2 * lane + 1 < nw ? (uint32_t)__popc(kept[2 * lane + 1]) : 0u;
    const uint64_t incl = wave_incl_scan_u64((uint64_t)(c0 + c1));
    const uint32_t base = (uint32_t)incl - c0 - c1;
    if (2 * lane < nw) wbase[2 * lane] = base;
    if (2 * lane + 1 < nw) wbase[2 * lane + 1] = base + c0;
    if (lane == 63) count[(size_t)h * nbmax + I] = (int32_t)incl;
  }
  __syncthreads();
  uint16_t* out = list + ((size_t)h * nbmax + I) * nbmax;
  for (int i = tid; i < nw * 32 && i < n; i += 256) {
    const uint32_t word = kept[i >> 5];
    if ((word >> (i & 31)) & 1u) out[wbase[i >> 5] + __popc(word & ((1u << (i & 31)) - 1u))] = (uint16_t)i;
  }
}

hipError_t launch_block_select(int dtype, int d, const void* Qh, const void* Kh, const int32_t* Lp_dev, int64_t C,
                               int Hq, double gamma, float* qbar, float* kbar, double* zl, uint16_t* list,
                               int32_t* count, hipStream_t st) {
  const int nbmax = (int)(C / kBlock);
  const dim3 grid((unsigned)nbmax, (unsigned)Hq);
  if (dtype == 1) {
    if (d == 128)
      block_pool_kernel<uint16_t, 128><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(Qh),
                                                             static_cast<const uint16_t*>(Kh), Lp_dev, C, nbmax, qbar, kbar);
    else
      block_pool_kernel<uint16_t, 64><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(Qh),
                                                            static_cast<const uint16_t*>(Kh), Lp_dev, C, nbmax, qbar, kbar);
  } else {
    if (d == 128)
      block_pool_kernel<float, 128><<<grid, 256, 0, st>>>(static_cast<const float*>(Qh), static_cast<const float*>(Kh),
                                                          Lp_dev, C, nbmax, qbar, kbar);
    else
      block_pool_kernel<float, 64><<<grid, 256, 0, st>>>(static_cast<const float*>(Qh), static_cast<const float*>(Kh),
                                                         Lp_dev, C, nbmax, qbar, kbar);
  }
  const unsigned nt = (unsigned)((nbmax + 63) / 64);
  const dim3 lgrid(nt, nt, (unsigned)Hq);
  if (d == 128)
    block_logits_kernel<128><<<lgrid, 256, 0, st>>>(qbar, kbar, Lp_dev, nbmax, zl);
  else
    block_logits_kernel<64><<<lgrid, 256, 0, st>>>(qbar, kbar, Lp_dev, nbmax, zl);
  block_select_kernel<<<grid, 256, 0, st>>>(zl, Lp_dev, nbmax, gamma, list, count);
  return hipGetLastError();
}

}  // namespace tsa

// Layer score, coverage budget and per-head top-L' selection (papernotes.org reading notes, "Key
// design 2"; bxzpzcl.cn article, section 2.1; gist.science summary, "Dynamic Token Coverage").
//
// Neither stage sorts.  Both are radix selects over the float32 bit patterns of non-negative scores
// (whose unsigned order is their numeric order), four 8-bit digit passes from the top:
//   budget: weight of an element = its score in 64-bit fixed point (2^-60 units); the pass finds the
//           digit bucket where the ascending cumulative weight first reaches the target ceil(tau*2^60).
//           Integer weights make the histograms exact and independent of the summation order.
//   select: weight 1; the target is rank k+1 in ascending order, i.e. the L'-th largest score.
// Each histogram pass first re-derives the previous pass's bucket from its histogram (every block
// computes the same value; block 0 stores it), so a pass is one launch and no host sync is needed.
// Selection then keeps every score above the threshold plus the lowest-index ties at it, and
// compacts the indices in ascending order with wave ballots and a per-head scan over tiles.
// Rows of at most 32768 keys take a one-workgroup variant of both (below): the same integer
// counts and weights, one launch per stage.
#include "kern_common.h"
#include "tsa_internal.h"

namespace tsa {

constexpr int kLayerTile = 256;      // tokens per block in the layer-score kernels
constexpr int kSelTile = 2048;     // elements per block in the compaction kernels
constexpr int kHistTile = 4096;    // elements per block in the histogram kernels
constexpr double kTwo60 = 1152921504606846976.0;

// tile sums plus one slot for their total
int64_t layer_tiles(int64_t L) { return (L + kLayerTile - 1) / kLayerTile + 1; }
int64_t select_tiles(int64_t L) { return (L + kSelTile - 1) / kSelTile; }

// ---- layer score --------------------------------------------------------------------------------
// S[t] = sum over heads in head order (float64); s_l = S / total, the total summed in one fixed
// order (every block of the normalisation forms the same value).  One token per thread, so a launch
// has L/256 blocks.

__global__ __launch_bounds__(256) void layer_sum_kernel(const float* __restrict__ s_h, int64_t L, int Hq,
                                                        double* __restrict__ S, double* __restrict__ tile_sum) {
  __shared__ double red[4];
  const int64_t t = (int64_t)blockIdx.x * kLayerTile + threadIdx.x;
  double acc = 0.0;
  if (t < L) {
    int h = 0;
    for (; h + 8 <= Hq; h += 8) {       // loads first, then the adds in head order
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = s_h[(size_t)(h + u) * L + t];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += (double)v[u];
    }
    for (; h < Hq; ++h) acc += (double)s_h[(size_t)h * L + t];
    S[t] = acc;
  }
  const double local = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = local;
  __syncthreads();
  if (threadIdx.x == 0) tile_sum[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// total = sum of the tile sums (fixed order: strided per-thread partials, then a fixed tree),
// stored after them at tile_sum[ntiles].
// The first 256 threads form the partials; every thread of the block must call this (it holds a
// barrier) and every thread gets the total.
__device__ double tile_total(const double* __restrict__ tile_sum, int64_t ntiles, double* red) {
  double a = 0.0;
  if (threadIdx.x < 256)
    for (int64_t i = threadIdx.x; i < ntiles; i += 256) a += tile_sum[i];
  a = wave_sum(a);
  if (threadIdx.x < 256 && (threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// s_l = S / total; each block sums the tile sums itself (ntiles = L / 256 of them, a few KB read
// from L2), so the total needs no launch of its own
__global__ __launch_bounds__(256) void layer_norm_kernel(const double* __restrict__ S,
                                                         const double* __restrict__ tile_sum, int64_t ntiles,
                                                         int64_t L, float* __restrict__ s_l) {
  __shared__ double red[4];
  const int64_t t = (int64_t)blockIdx.x * kLayerTile + threadIdx.x;
  const double s = t < L ? S[t] : 0.0;        // loaded before the total's barrier
  const double total = tile_total(tile_sum, ntiles, red);
  if (t < L) s_l[t] = (float)(s / total);
}

hipError_t launch_layer_score(const float* s_h, int64_t L, int Hq, double* S, double* tile_sum,
                              float* s_l, hipStream_t st) {
  const unsigned n = (unsigned)(layer_tiles(L) - 1);
  layer_sum_kernel<<<n, 256, 0, st>>>(s_h, L, Hq, S, tile_sum);
  layer_norm_kernel<<<n, 256, 0, st>>>(S, tile_sum, n, L, s_l);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;   // callers pass multiples of 16
  if (n16 == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n16 + 255) / 256 < 4096 ? (n16 + 255) / 256 : 4096);
  fill_zero_kernel<<<blocks, 256, 0, st>>>(static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

// ---- radix machinery ----------------------------------------------------------------------------
// Histogram layout per segment and pass: 256 counts then 256 weights (uint64).

template <bool MASS>
__device__ __forceinline__ uint64_t weight_of(uint32_t key) {
  if constexpr (MASS) return (uint64_t)((double)__uint_as_float(key) * kTwo60);
  return 1;
}

// Run by one full wave.  Given the histogram of pass `pass` and the control word of the pass before,
// find the bucket where the ascending cumulative weight first reaches T.  All lanes return it.
__device__ RadixCtl radix_find(const uint64_t* __restrict__ hist, RadixCtl prev, uint64_t T) {
  const int lane = threadIdx.x & 63;
  uint64_t c4[4], w4[4], csum = 0, wsum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c4[j] = hist[4 * lane + j];
    w4[j] = hist[kRadixBins + 4 * lane + j];
    csum += c4[j];
    wsum += w4[j];
  }
  const uint64_t wincl = wave_incl_scan_u64(wsum);
  const uint64_t cincl = wave_incl_scan_u64(csum);
  const bool hit = prev.w_below + wincl >= T;
  const uint64_t mask = __ballot(hit);
  RadixCtl out = prev;
  if (mask == 0) { out.none = 1; return out; }
  const int first = __ffsll((long long)mask) - 1;
  uint32_t bin = 0;
  uint64_t cb = 0, wb = 0, nb = 0;
  if (lane == first) {
    uint64_t w = prev.w_below + (wincl - wsum), c = prev.cnt_below + (cincl - csum);
    int j = 0;
    for (; j < 3; ++j) {
      if (w + w4[j] >= T) break;
      w += w4[j];
      c += c4[j];
    }
    bin = 4 * lane + j; cb = c; wb = w; nb = c4[j];
  }
  out.prefix = (prev.prefix << 8) | (uint32_t)__shfl(bin, first, kWave);
  out.cnt_below = __shfl(cb, first, kWave);
  out.w_below = __shfl(wb, first, kWave);
  out.n_bin = __shfl(nb, first, kWave);
  out.none = 0;
  return out;
}

// Budget: a constant target weight.  Selection: rank k + 1 = L - L' + 1 from the device-side L'.
__device__ __forceinline__ uint64_t seg_target(uint64_t T_const, const int32_t* Lp_dev, int64_t L) {
  return Lp_dev ? (uint64_t)(L - (int64_t)Lp_dev[0] + 1) : T_const;
}

// The control word that a kernel of pass `pass` must match against (bucket of pass-1).
__device__ RadixCtl derive_ctl(const uint64_t* __restrict__ hist_seg, RadixCtl* __restrict__ ctl_seg,
                               int pass, uint64_t T) {
  __shared__ RadixCtl cur;
  if (threadIdx.x < 64) {
    RadixCtl prev = {0, 0, 0, 0, 0};
    if (pass >= 2) prev = ctl_seg[pass - 2];
    RadixCtl c = prev;
    if (!prev.none) c = radix_find(hist_seg + (size_t)(pass - 1) * 2 * kRadixBins, prev, T);
    if (threadIdx.x == 0) {
      cur = c;
      if (blockIdx.x == 0) ctl_seg[pass - 1] = c;
    }
  }
  __syncthreads();
  return cur;
}

template <bool MASS>
__global__ __launch_bounds__(256) void radix_hist_kernel(const float* __restrict__ keys, int64_t L,
                                                         int64_t seg_stride, int pass, uint64_t T_const,
                                                         const int32_t* __restrict__ Lp_dev,
                                                         uint64_t* __restrict__ hist,
                                                         RadixCtl* __restrict__ ctl) {
  __shared__ uint64_t hc[kRadixBins];
  __shared__ uint64_t hw[kRadixBins];
  const int seg = blockIdx.y;
  uint64_t* hseg = hist + (size_t)seg * kRadixPasses * 2 * kRadixBins;
  RadixCtl* cseg = ctl + (size_t)seg * kRadixPasses;
  const uint64_t T = seg_target(T_const, Lp_dev, L);
  RadixCtl cur = {0, 0, 0, 0, 0};
  if (pass > 0) cur = derive_ctl(hseg, cseg, pass, T);
  hc[threadIdx.x] = 0;
  hw[threadIdx.x] = 0;
  __syncthreads();
  if (cur.none) return;
  const int shift_digit = 24 - 8 * pass;
  const float* kseg = keys + (size_t)seg * seg_stride;
  const int64_t base = (int64_t)blockIdx.x * kHistTile;
  // every key of the thread first, then the counting: a load under a per-key branch waited for the
  // loads before it (one memory round trip per key)
  constexpr int KPT = kHistTile / 256;
  uint32_t kv[KPT];
  if (base + kHistTile <= L) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) kv[u] = __float_as_uint(kseg[base + u * 256 + threadIdx.x]);
  } else {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int64_t t = base + u * 256 + threadIdx.x;
      kv[u] = t < L ? __float_as_uint(kseg[t]) : 0u;
    }
  }
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int64_t t = base + u * 256 + threadIdx.x;
    if (t >= L) break;
    const uint32_t key = kv[u];
    if (pass > 0 && (key >> (32 - 8 * pass)) != cur.prefix) continue;
    const uint32_t dg = (key >> shift_digit) & 0xFFu;
    atomicAdd((unsigned long long*)&hc[dg], 1ull);
    if (MASS) atomicAdd((unsigned long long*)&hw[dg], (unsigned long long)weight_of<MASS>(key));
  }
  __syncthreads();
  const uint64_t c = hc[threadIdx.x];
  if (c) {
    uint64_t* hp = hseg + (size_t)pass * 2 * kRadixBins;
    atomicAdd((unsigned long long*)&hp[threadIdx.x], (unsigned long long)c);
    atomicAdd((unsigned long long*)&hp[kRadixBins + threadIdx.x],
              (unsigned long long)(MASS ? hw[threadIdx.x] : c));
  }
}

// k = (elements below the crossing value) + (copies of that value needed to reach the target).
__global__ void budget_final_kernel(const uint64_t* __restrict__ hist, RadixCtl* __restrict__ ctl,
                                    int64_t L, uint64_t T, int32_t* __restrict__ kLp_ws,
                                    int32_t* __restrict__ k_out, int32_t* __restrict__ Lp_out) {
  int64_t k;
  const RadixCtl fin = derive_ctl(hist, ctl, kRadixPasses, T);
  if (T == 0) {
    k = 0;
  } else if (fin.none) {
    k = L;
  } else {
    const uint64_t V = weight_of<true>(fin.prefix);
    const uint64_t need = T - fin.w_below;              // > 0 by construction
    k = (int64_t)fin.cnt_below + (int64_t)((need + V - 1) / V);
  }
  if (threadIdx.x == 0) {
    kLp_ws[0] = (int32_t)k;
    kLp_ws[1] = (int32_t)(L - k);
    if (k_out) k_out[0] = (int32_t)k;
    if (Lp_out) Lp_out[0] = (int32_t)(L - k);
  }
}

// ---- one-workgroup selects for rows of at most kResidentMax keys ---------------------------------
// A single 1024-thread workgroup per row holds the row in registers, NK consecutive keys per thread,
// and runs every digit pass itself: one launch where the multi-block select needs one per pass.
// Its digits start below the bits that every key of the row shares (the common leading bits of the
// smallest and the largest key), so a row of similar scores is spread over many bins from the first
// pass on, and they are 11 bits wide: at most three passes.  Counts and weights are integers, so the
// crossing key, the counts below it and the ties at it are the same as the multi-block select's.
constexpr int64_t kResidentMax = 32768;   // measured: at 65536 the multi-block budget is faster
constexpr int kResThreads = 1024, kResWaves = kResThreads / kWave;
constexpr int kResBits = 11, kResBins = 1 << kResBits;

bool radix_resident(int64_t L) { return L <= kResidentMax; }

// Once at most this many keys share the prefix fixed so far, one wave ranks them directly instead
// of running the remaining digit passes.
constexpr int kResFinish = 64;

// Two histograms: while wave 0 searches one pass's histogram, the other waves clear the next one's.
template <bool MASS>
struct ResShared {
  uint32_t hc[2][kResBins];                  // counts
  uint64_t hw[2][MASS ? kResBins : 1];       // weights (budget)
  uint32_t rmin[kResWaves], rmax[kResWaves], rcnt[kResWaves];
  uint64_t rw[kResWaves];
  uint32_t fkey[kResFinish];                 // the keys under the prefix, for the direct ranking
  uint64_t fw[MASS ? kResFinish : 1];        // and their weights (budget)
  uint32_t fcnt;
  RadixCtl ctl;
};

// Clears histogram `buf` using the threads from `first` on.
template <bool MASS>
__device__ __forceinline__ void res_clear(ResShared<MASS>& sh, int buf, int first) {
  for (int b = (int)threadIdx.x - first; b >= 0 && b < kResBins; b += kResThreads - first) {
    sh.hc[buf][b] = 0;
    if (MASS) sh.hw[buf][b] = 0;
  }
}

// Inclusive prefix sum over the 64 lanes of a wave (32-bit: counts of at most kResidentMax keys).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

// Exclusive prefix sum over the block (1024 threads); `total` receives the block sum.
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t* red, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t n = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += n;
  }
  if (lane == 63) red[w] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kResWaves; ++i) {
    const uint32_t r = red[i];
    before += i < w ? r : 0u;
    tot += r;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

// Run by wave 0 after a pass's histogram over nbins bins: the bin where the ascending cumulative
// weight (counts for a rank) first reaches T, given what lies below the current prefix.  Each lane
// sums a contiguous chunk of per bins; the first lane whose running total reaches T owns the bin,
// which a second scan over that chunk's bins (one per lane) then finds.
template <bool MASS>
__device__ void res_find(ResShared<MASS>& sh, int buf, int nbins, int width, uint32_t prefix, uint64_t cb,
                         uint64_t wb, uint64_t T) {
  const int lane = threadIdx.x & 63;
  const int per = nbins >= 64 ? nbins >> 6 : 1;          // 1 .. 32
  const int b0 = lane * per, n = b0 < nbins ? per : 0;
  // counts stay below 2^32 (at most kResidentMax keys); without masses the weight is the count
  uint32_t cs = 0;
  uint64_t ws = 0;
#pragma unroll
  for (int j = 0; j < kResBins / 64; ++j) {
    if (j < n) {
      const int b = b0 + ((j + lane) & (per - 1));      // rotated start: the lanes read distinct banks
      cs += sh.hc[buf][b];
      if (MASS) ws += sh.hw[buf][b];
    }
  }
  const uint64_t cincl = wave_incl_scan_u32(cs);
  if (!MASS) ws = cs;
  const uint64_t wincl = MASS ? wave_incl_scan_u64(ws) : cincl;
  const uint64_t mask = __ballot(wb + wincl >= T);
  if (mask == 0) {
    if (lane == 0) sh.ctl.none = 1;
    return;
  }
  const int f = __ffsll((long long)mask) - 1;
  const uint64_t wbase = wb + __shfl(wincl - ws, f, kWave), cbase = cb + __shfl(cincl - cs, f, kWave);
  const int bf = f * per;
  uint32_t c2 = 0;
  uint64_t w2 = 0;
  if (lane < per) {
    c2 = sh.hc[buf][bf + lane];
    w2 = MASS ? sh.hw[buf][bf + lane] : (uint64_t)c2;
  }
  const uint64_t ci2 = wave_incl_scan_u32(c2);
  const uint64_t wi2 = MASS ? wave_incl_scan_u64(w2) : ci2;
  // lane f's chunk reaches T, so some lane below per hits
  const uint64_t m2 = __ballot(lane < per && wbase + wi2 >= T);
  if (lane == __ffsll((long long)m2) - 1) {
    sh.ctl.prefix = (prefix << width) | (uint32_t)(bf + lane);
    sh.ctl.none = 0;
    sh.ctl.cnt_below = cbase + ci2 - c2;
    sh.ctl.w_below = wbase + wi2 - w2;
    sh.ctl.n_bin = c2;
  }
}

// The remaining digits at once, when n <= kResFinish keys share the prefix fixed so far: every thread
// puts its keys under the prefix into a list, then wave 0 ranks the n keys against each other.  The
// crossing key is the smallest one whose cumulative weight, counting every key equal to it,
// reaches T: the same key, counts and weights the remaining passes would find.  Ends with the
// result in sh.ctl, read after a barrier.
template <int NK, bool MASS>
__device__ void res_finish(const uint32_t (&key)[NK], int64_t L, int done, uint32_t prefix, uint64_t cb,
                           uint64_t wb, uint64_t T, ResShared<MASS>& sh) {
  const int64_t t0 = (int64_t)NK * threadIdx.x;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    uint32_t k = key[i];
    if (MASS) asm volatile("" : "+v"(k));             // weights computed here, not hoisted (registers)
    if (t0 + i < L && (k >> (32 - done)) == prefix) {
      const uint32_t pos = atomicAdd(&sh.fcnt, 1u);   // below kResFinish: n keys share the prefix
      sh.fkey[pos] = k;
      if (MASS) sh.fw[pos] = weight_of<true>(k);
    }
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x, n = (int)sh.fcnt;
    const uint32_t kk = lane < n ? sh.fkey[lane] : 0u;
    uint32_t ltc = 0, eqc = 0;
    uint64_t ltw = 0, eqw = 0;
#pragma unroll 1
    for (int j = 0; j < n; ++j) {
      const uint32_t kj = sh.fkey[j];
      const uint64_t wj = MASS ? sh.fw[j] : 1ull;
      if (kj < kk) { ++ltc; ltw += wj; }
      if (kj == kk) { ++eqc; eqw += wj; }
    }
    const bool ok = lane < n && wb + ltw + eqw >= T;
    uint32_t v = ok ? kk : 0xFFFFFFFFu;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor(v, o, kWave));
    const uint64_t hit = __ballot(ok && kk == v);
    if (hit == 0) {
      if (lane == 0) sh.ctl.none = 1;
    } else if (lane == __ffsll((long long)hit) - 1) {
      sh.ctl.prefix = v;
      sh.ctl.none = 0;
      sh.ctl.cnt_below = cb + ltc;
      sh.ctl.w_below = wb + ltw;
      sh.ctl.n_bin = eqc;
    }
  }
  __syncthreads();
}

// The key where the ascending cumulative weight of the row first reaches T (T >= 1), with the
// count and weight of the keys below it and the number of keys equal to it.  Thread j holds keys
// NK j .. NK j + NK - 1 (those at or past L are absent).  Every thread returns the same result.
struct ResResult {
  uint32_t key, none;
  uint64_t cnt_below, w_below, n_eq;
};

template <int NK, bool MASS>
__device__ ResResult resident_threshold(const uint32_t (&key)[NK], int64_t L, uint64_t T, ResShared<MASS>& sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t0 = (int64_t)NK * tid;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0;
  uint64_t wt = 0;
#pragma unroll
  for (int i = 0; i < NK; ++i)
    if (t0 + i < L) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
      if (MASS) wt += weight_of<true>(key[i]);
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor(kmin, o, kWave));
    kmax = max(kmax, (uint32_t)__shfl_xor(kmax, o, kWave));
  }
  if (MASS) wt = wave_sum_u64(wt);
  if (lane == 0) {
    sh.rmin[w] = kmin;
    sh.rmax[w] = kmax;
    sh.rw[w] = wt;
  }
  if (tid == 0) sh.fcnt = 0;
  res_clear<MASS>(sh, 0, 0);
  __syncthreads();
  uint64_t wtot = 0;
#pragma unroll
  for (int i = 0; i < kResWaves; ++i) {
    kmin = min(kmin, sh.rmin[i]);
    kmax = max(kmax, sh.rmax[i]);
    wtot += sh.rw[i];
  }
  ResResult r = {0u, 0u, 0, 0, 0};
  if (T > (MASS ? wtot : (uint64_t)L)) {
    r.none = 1;
    return r;
  }
  const uint32_t diff = kmin ^ kmax;
  int done = diff ? __clz((int)diff) : 32;                    // leading bits shared by every key
  uint32_t prefix = done == 0 ? 0u : kmin >> (32 - done);
  uint64_t cb = 0, wb = 0, n_eq = (uint64_t)L;
  int buf = 0;                         // histogram of this pass (cleared)
  while (done < 32) {
    const int width = 32 - done < kResBits ? 32 - done : kResBits;
    const int shift = 32 - done - width, nbins = 1 << width;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      uint32_t k = key[i];
      // the weights are recomputed in each pass: hoisted out of the pass loop, 64-bit weights of
      // every key would double the registers and spill
      if (MASS) asm volatile("" : "+v"(k));
      if (t0 + i < L && (done == 0 || (k >> (32 - done)) == prefix)) {
        const uint32_t d = (k >> shift) & (uint32_t)(nbins - 1);
        atomicAdd(&sh.hc[buf][d], 1u);
        if (MASS) atomicAdd((unsigned long long*)&sh.hw[buf][d], (unsigned long long)weight_of<true>(k));
      }
    }
    __syncthreads();
    if (w == 0) res_find<MASS>(sh, buf, nbins, width, prefix, cb, wb, T);
    else res_clear<MASS>(sh, buf ^ 1, kWave);
    __syncthreads();
    buf ^= 1;
    if (sh.ctl.none) {                 // not reached: T is within the row's total
      r.none = 1;
      return r;
    }
    prefix = sh.ctl.prefix;
    cb = sh.ctl.cnt_below;
    wb = sh.ctl.w_below;
    n_eq = sh.ctl.n_bin;
    done += width;
    if (done < 32 && n_eq <= (uint64_t)kResFinish) {   // block-uniform: read from LDS after a barrier
      res_finish<NK, MASS>(key, L, done, prefix, cb, wb, T, sh);
      if (sh.ctl.none) {
        r.none = 1;
        return r;
      }
      prefix = sh.ctl.prefix;
      cb = sh.ctl.cnt_below;
      wb = sh.ctl.w_below;
      n_eq = sh.ctl.n_bin;
      done = 32;
    }
  }
  r.key = prefix;
  r.cnt_below = cb;
  r.w_below = wb;
  r.n_eq = n_eq;
  return r;
}

// Thread j's NK consecutive values of a row of L floats (absent past L as 0).
template <int NK>
__device__ __forceinline__ void load_keys(const float* __restrict__ row, int64_t L, uint32_t (&key)[NK]) {
  const int64_t t0 = (int64_t)NK * threadIdx.x;
  if (t0 + NK <= L && ((reinterpret_cast<uintptr_t>(row + t0) & 15) == 0)) {
#pragma unroll
    for (int i = 0; i < NK; i += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + t0 + i);
      key[i] = v.x; key[i + 1] = v.y; key[i + 2] = v.z; key[i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NK; ++i) key[i] = t0 + i < L ? __float_as_uint(row[t0 + i]) : 0u;
  }
}

// The budget of one row by the whole workgroup: k (every thread returns it).  FROM_S: s_l is first
// formed from the head sums S and their tile sums (as launch_layer_score does) and, with write_sl,
// stored to s_l_out.
template <int NK, bool FROM_S>
__device__ __forceinline__ int64_t budget_resident_row(const float* __restrict__ s_l_in, const double* __restrict__ S,
                                       const double* __restrict__ tile_sum, int64_t ntiles, float* __restrict__ s_l_out,
                                       bool write_sl, int64_t L, uint64_t T, ResShared<true>& sh, double* red) {
  uint32_t key[NK];
  const int64_t t0 = (int64_t)NK * threadIdx.x;
  if constexpr (FROM_S) {
    // the head sums first (no per-element branch between the loads), then the divisions
    double sv[NK];
    if (t0 + NK <= L) {
#pragma unroll
      for (int i = 0; i < NK; ++i) sv[i] = S[t0 + i];
    } else {
#pragma unroll
      for (int i = 0; i < NK; ++i) sv[i] = t0 + i < L ? S[t0 + i] : 0.0;
    }
    const double total = tile_total(tile_sum, ntiles, red);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      key[i] = 0u;
      if (t0 + i < L) {
        const float v = (float)(sv[i] / total);
        if (write_sl) s_l_out[t0 + i] = v;
        key[i] = __float_as_uint(v);
      }
    }
  } else {
    load_keys<NK>(s_l_in, L, key);
  }
  int64_t k = 0;
  if (T != 0) {
    const ResResult r = resident_threshold<NK, true>(key, L, T, sh);
    if (r.none) {
      k = L;
    } else {
      const uint64_t V = weight_of<true>(r.key);
      k = (int64_t)r.cnt_below + (int64_t)((T - r.w_below + V - 1) / V);
    }
  }
  return k;
}

__device__ __forceinline__ void write_keep(int64_t k, int64_t L, int32_t* kLp_ws, int32_t* k_out, int32_t* Lp_out) {
  if (kLp_ws) { kLp_ws[0] = (int32_t)k; kLp_ws[1] = (int32_t)(L - k); }
  if (k_out) k_out[0] = (int32_t)k;
  if (Lp_out) Lp_out[0] = (int32_t)(L - k);
}

template <int NK, bool FROM_S>
__global__ __launch_bounds__(kResThreads) void budget_resident_kernel(const float* __restrict__ s_l_in,
                                                                      const double* __restrict__ S,
                                                                      const double* __restrict__ tile_sum,
                                                                      int64_t ntiles, float* __restrict__ s_l_out,
                                                                      int64_t L, uint64_t T,
                                                                      int32_t* __restrict__ kLp_ws,
                                                                      int32_t* __restrict__ k_out,
                                                                      int32_t* __restrict__ Lp_out) {
  __shared__ ResShared<true> sh;
  __shared__ double red[4];
  const int64_t k = budget_resident_row<NK, FROM_S>(s_l_in, S, tile_sum, ntiles, s_l_out, true, L, T, sh, red);
  if (threadIdx.x == 0) write_keep(k, L, kLp_ws, k_out, Lp_out);
}

template <bool FROM_S>
static hipError_t launch_budget_resident(const float* s_l_in, const double* S, const double* tile_sum,
                                         int64_t ntiles, float* s_l_out, int64_t L, uint64_t T, int32_t* kLp_ws,
                                         int32_t* k_out, int32_t* Lp_out, hipStream_t st) {
#define TSA_BUDGET_RES(NK) \
  budget_resident_kernel<NK, FROM_S><<<1, kResThreads, 0, st>>>(s_l_in, S, tile_sum, ntiles, s_l_out, L, T, kLp_ws, k_out, Lp_out)
  if (L <= 4 * kResThreads) TSA_BUDGET_RES(4);
  else if (L <= 8 * kResThreads) TSA_BUDGET_RES(8);
  else if (L <= 16 * kResThreads) TSA_BUDGET_RES(16);
  else TSA_BUDGET_RES(32);
#undef TSA_BUDGET_RES
  return hipGetLastError();
}

hipError_t launch_budget(const float* s_l, int64_t L, uint64_t target, uint64_t* hist,
                         RadixCtl* ctl, int32_t* kLp_ws, int32_t* k_out, int32_t* Lp_out,
                         hipStream_t st) {
  if (radix_resident(L))
    return launch_budget_resident<false>(s_l, nullptr, nullptr, 0, nullptr, L, target, kLp_ws, k_out, Lp_out, st);
  const dim3 grid((unsigned)((L + kHistTile - 1) / kHistTile), 1);
  for (int pass = 0; pass < kRadixPasses; ++pass)
    radix_hist_kernel<true><<<grid, 256, 0, st>>>(s_l, L, 0, pass, target, nullptr, hist, ctl);
  budget_final_kernel<<<1, 64, 0, st>>>(hist, ctl, L, target, kLp_ws, k_out, Lp_out);
  return hipGetLastError();
}

// Layer score and budget together.  For a row of at most 4096 tokens the budget's workgroup also
// forms s_l (from the head sums and their tile sums, as launch_layer_score does), which saves the
// layer score's total and normalisation launches.  Longer rows keep those launches: there each
// thread would read its run of head sums uncoalesced and divide it element by element (measured at
// 32768 tokens: 70 us against 41 us for the separate kernels).
hipError_t launch_layer_score_budget(const float* s_h, int64_t L, int Hq, double* S, double* tile_sum, float* s_l,
                                     uint64_t target, uint64_t* hist, RadixCtl* ctl, int32_t* kLp_ws,
                                     int32_t* k_out, int32_t* Lp_out, hipStream_t st) {
  if (L > 4 * kResThreads) {
    hipError_t e = launch_layer_score(s_h, L, Hq, S, tile_sum, s_l, st);
    return e == hipSuccess ? launch_budget(s_l, L, target, hist, ctl, kLp_ws, k_out, Lp_out, st) : e;
  }
  const unsigned n = (unsigned)(layer_tiles(L) - 1);
  layer_sum_kernel<<<n, 256, 0, st>>>(s_h, L, Hq, S, tile_sum);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_budget_resident<true>(nullptr, S, tile_sum, n, s_l, L, target, kLp_ws, k_out, Lp_out, st);
}

// Fixed-ratio budget: k = round(s * L), halves up, exact on the float32 value of s (s in [0, 1]).
// s = M * 2^-sh with an integer mantissa M < 2^24 and sh >= 23, so M * L < 2^55 and
// k = (M * L + 2^(sh-1)) >> sh fits 64-bit arithmetic; for sh >= 64, s * L < 1/2 and k = 0.
__global__ void budget_ratio_kernel(float s, int64_t L, int32_t* __restrict__ kLp_ws,
                                    int32_t* __restrict__ k_out, int32_t* __restrict__ Lp_out) {
  if (threadIdx.x != 0) return;
  const uint32_t bits = __float_as_uint(s);
  const uint32_t e = (bits >> 23) & 255u;
  const uint64_t M = e ? (uint64_t)((bits & 0x7FFFFFu) | 0x800000u) : (uint64_t)(bits & 0x7FFFFFu);
  const int sh = e ? 150 - (int)e : 149;
  int64_t k = 0;
  if (sh < 64) k = (int64_t)((M * (uint64_t)L + (1ull << (sh - 1))) >> sh);
  if (kLp_ws) { kLp_ws[0] = (int32_t)k; kLp_ws[1] = (int32_t)(L - k); }
  if (k_out) k_out[0] = (int32_t)k;
  if (Lp_out) Lp_out[0] = (int32_t)(L - k);
}

hipError_t launch_budget_ratio(float sparsity, int64_t L, int32_t* kLp_ws, int32_t* k_out, int32_t* Lp_out,
                               hipStream_t st) {
  budget_ratio_kernel<<<1, 64, 0, st>>>(sparsity, L, kLp_ws, k_out, Lp_out);
  return hipGetLastError();
}

// ---- per-head selection -------------------------------------------------------------------------

struct SelThr {
  uint32_t key;       // threshold bit pattern
  uint32_t take_eq;   // how many ties at the threshold are kept (lowest indices first)
};

__device__ SelThr sel_threshold(const RadixCtl& fin, int64_t L, int64_t Lp) {
  SelThr s;
  if (fin.none || Lp <= 0) {            // L' = 0: keep nothing
    s.key = 0xFFFFFFFFu;
    s.take_eq = 0;
    return s;
  }
  const int64_t gt = L - (int64_t)fin.cnt_below - (int64_t)fin.n_bin;
  s.key = fin.prefix;
  s.take_eq = (uint32_t)(Lp - gt);
  return s;
}

// Per tile: how many scores lie above the threshold and how many equal it.
__global__ __launch_bounds__(256) void select_count_kernel(const float* __restrict__ s_h, int64_t L,
                                                           const int32_t* __restrict__ Lp_dev,
                                                           uint64_t* __restrict__ hist,
                                                           RadixCtl* __restrict__ ctl,
                                                           uint32_t* __restrict__ tile_cnt) {
  __shared__ uint32_t red[2][4];
  const int h = blockIdx.y;
  const int64_t k = L - Lp_dev[0];
  const RadixCtl fin = derive_ctl(hist + (size_t)h * kRadixPasses * 2 * kRadixBins,
                                  ctl + (size_t)h * kRadixPasses, kRadixPasses, (uint64_t)k + 1);
  const SelThr thr = sel_threshold(fin, L, L - k);
  uint32_t gt = 0, eq = 0;
  const float* row = s_h + (size_t)h * L;
  for (int u = 0; u < kSelTile / 256; ++u) {
    const int64_t t = (int64_t)blockIdx.x * kSelTile + u * 256 + threadIdx.x;
    if (t < L) {
      const uint32_t key = __float_as_uint(row[t]);
      gt += key > thr.key;
      eq += key == thr.key;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    gt += __shfl_xor(gt, o, kWave);
    eq += __shfl_xor(eq, o, kWave);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = gt;
    red[1][threadIdx.x >> 6] = eq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const size_t o = ((size_t)h * gridDim.x + blockIdx.x) * 2;
    tile_cnt[o] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    tile_cnt[o + 1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
}

// Per head, exclusive scans over tiles: ties seen before the tile and selected entries before it.
__global__ __launch_bounds__(64) void select_scan_kernel(const uint32_t* __restrict__ tile_cnt,
                                                         int64_t ntiles, int64_t L,
                                                         const int32_t* __restrict__ Lp_dev,
                                                         const RadixCtl* __restrict__ ctl,
                                                         uint32_t* __restrict__ tile_off) {
  const int h = blockIdx.x, lane = threadIdx.x;
  const int64_t k = L - Lp_dev[0];
  const SelThr thr = sel_threshold(ctl[(size_t)h * kRadixPasses + kRadixPasses - 1], L, L - k);
  uint64_t eq_run = 0, sel_run = 0;
  for (int64_t base = 0; base < ntiles; base += 64) {
    const int64_t i = base + lane;
    uint64_t gt = 0, eq = 0;
    if (i < ntiles) {
      gt = tile_cnt[((size_t)h * ntiles + i) * 2];
      eq = tile_cnt[((size_t)h * ntiles + i) * 2 + 1];
    }
    const uint64_t eq_before = eq_run + wave_incl_scan_u64(eq) - eq;
    const uint64_t room = thr.take_eq > eq_before ? thr.take_eq - eq_before : 0;
    const uint64_t sel = gt + (eq < room ? eq : room);
    const uint64_t sel_incl = wave_incl_scan_u64(sel);
    if (i < ntiles) {
      tile_off[((size_t)h * ntiles + i) * 2] = (uint32_t)(sel_run + sel_incl - sel);
      tile_off[((size_t)h * ntiles + i) * 2 + 1] = (uint32_t)eq_before;
    }
    eq_run += __shfl(wave_incl_scan_u64(eq), 63, kWave);
    sel_run += __shfl(sel_incl, 63, kWave);
  }
}

__global__ __launch_bounds__(256) void select_write_kernel(const float* __restrict__ s_h, int64_t L,
                                                           const int32_t* __restrict__ Lp_dev,
                                                           const RadixCtl* __restrict__ ctl,
                                                           const uint32_t* __restrict__ tile_off,
                                                           int32_t* __restrict__ idx,
                                                           int32_t* __restrict__ inv) {
  __shared__ uint32_t weq[4], wsel[4];
  const int h = blockIdx.y, wave = threadIdx.x >> 6;
  const int64_t k = L - Lp_dev[0];
  const SelThr thr = sel_threshold(ctl[(size_t)h * kRadixPasses + kRadixPasses - 1], L, L - k);
  const size_t to = ((size_t)h * gridDim.x + blockIdx.x) * 2;
  uint32_t sel_base = tile_off[to], eq_base = tile_off[to + 1];
  const float* row = s_h + (size_t)h * L;
  for (int u = 0; u < kSelTile / 256; ++u) {
    const int64_t t = (int64_t)blockIdx.x * kSelTile + u * 256 + threadIdx.x;
    const bool in = t < L;
    const uint32_t key = in ? __float_as_uint(row[t]) : 0u;
    const bool is_eq = in && key == thr.key;
    const bool is_gt = in && key > thr.key;
    const uint64_t meq = __ballot(is_eq);
    if ((threadIdx.x & 63) == 0) weq[wave] = __popcll(meq);
    __syncthreads();
    uint32_t eq_rank = eq_base + lanes_below(meq);
    for (int w = 0; w < wave; ++w) eq_rank += weq[w];
    const bool flag = is_gt || (is_eq && eq_rank < thr.take_eq);
    const uint64_t msel = __ballot(flag);
    if ((threadIdx.x & 63) == 0) wsel[wave] = __popcll(msel);
    __syncthreads();
    uint32_t pos = sel_base + lanes_below(msel);
    for (int w = 0; w < wave; ++w) pos += wsel[w];
    if (flag) idx[(size_t)h * L + pos] = (int32_t)t;
    if (in && inv) inv[(size_t)h * L + t] = flag ? (int32_t)pos : -1;
    sel_base += wsel[0] + wsel[1] + wsel[2] + wsel[3];
    eq_base += weq[0] + weq[1] + weq[2] + weq[3];
    __syncthreads();
  }
}

// Selection over one head's row by the whole workgroup, for a keep count Lp known to every thread:
// the threshold key V = the (k+1)-th smallest score (k = L - L'), every key above it plus the
// lowest-index ties at it, compacted in ascending order.
template <int NK>
__device__ __forceinline__ void select_resident_row(const float* __restrict__ row, int64_t L, int64_t Lp, int32_t* __restrict__ irow,
                                    int32_t* __restrict__ vrow, ResShared<false>& sh, uint64_t* smask,
                                    uint32_t* sbase) {   // LDS, kResThreads entries each
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)NK * tid;
  uint32_t key[NK];
  load_keys<NK>(row, L, key);
  uint32_t V = 0xFFFFFFFFu;             // L' = 0: no key is above it or equal to it
  uint64_t take_eq = 0;
  if (Lp > 0) {
    const ResResult r = resident_threshold<NK, false>(key, L, (uint64_t)(L - Lp + 1), sh);
    if (!r.none) {
      V = r.key;
      take_eq = (uint64_t)Lp - ((uint64_t)L - r.cnt_below - r.n_eq);
    }
  }
  uint32_t ceq = 0, tot;
#pragma unroll
  for (int i = 0; i < NK; ++i) ceq += (t0 + i < L && key[i] == V) ? 1u : 0u;
  uint32_t er = block_excl_scan_u32(ceq, sh.rcnt, tot);    // ties at V before this thread's keys
  uint64_t m = 0;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    if (t0 + i >= L) continue;
    bool keep = key[i] > V;
    if (key[i] == V) keep = er++ < take_eq;
    if (keep) m |= 1ull << i;
  }
  const uint32_t base = block_excl_scan_u32((uint32_t)__popcll(m), sh.rcnt, tot);
  smask[tid] = m;
  sbase[tid] = base;
  __syncthreads();
  for (int64_t e = tid; e < L; e += kResThreads) {
    const int owner = (int)(e / NK), bit = (int)(e % NK);
    const uint64_t mo = smask[owner];
    const bool sel = (mo >> bit) & 1ull;
    const int32_t pos = (int32_t)(sbase[owner] + (uint32_t)__popcll(mo & ((1ull << bit) - 1ull)));
    if (sel) irow[pos] = (int32_t)e;
    if (vrow) vrow[e] = sel ? pos : -1;
  }
}

template <int NK>
__global__ __launch_bounds__(kResThreads) void select_resident_kernel(const float* __restrict__ s_h, int64_t L,
                                                                      const int32_t* __restrict__ Lp_dev,
                                                                      int32_t* __restrict__ idx,
                                                                      int32_t* __restrict__ inv) {
  __shared__ ResShared<false> sh;
  __shared__ uint64_t smask[kResThreads];
  __shared__ uint32_t sbase[kResThreads];
  const int h = blockIdx.x;
  select_resident_row<NK>(s_h + (size_t)h * L, L, Lp_dev[0], idx + (size_t)h * L, inv ? inv + (size_t)h * L : nullptr,
                          sh, smask, sbase);
}

struct SelectShared {
  ResShared<false> r;
  uint64_t smask[kResThreads];
  uint32_t sbase[kResThreads];
};
union BudgetSelectShared {   // budget first, then selection
  ResShared<true> b;
  SelectShared s;
};

// Budget and selection of a short layer in one launch of Hq workgroups: each forms s_l and runs the
// budget itself (the same arithmetic on the same values, so every workgroup finds the same k), then
// selects its head's L - k tokens; workgroup 0 also stores s_l, k and L'.  One launch and one
// dependency fewer than the budget's single workgroup followed by the selection.
template <int NK, bool FROM_S>
__global__ __launch_bounds__(kResThreads) void budget_select_resident_kernel(
    const float* __restrict__ s_h, const float* __restrict__ s_l_in, const double* __restrict__ S,
    const double* __restrict__ tile_sum, int64_t ntiles, float* __restrict__ s_l_out, int64_t L, uint64_t T,
    int32_t* __restrict__ kLp_ws, int32_t* __restrict__ k_out, int32_t* __restrict__ Lp_out,
    int32_t* __restrict__ idx, int32_t* __restrict__ inv) {
  __shared__ BudgetSelectShared sh;
  __shared__ double red[4];
  const int h = blockIdx.x;
  const int64_t k = budget_resident_row<NK, FROM_S>(s_l_in, S, tile_sum, ntiles, s_l_out, h == 0, L, T, sh.b, red);
  if (h == 0 && threadIdx.x == 0) write_keep(k, L, kLp_ws, k_out, Lp_out);
  __syncthreads();   // the selection reuses the budget's LDS
  select_resident_row<NK>(s_h + (size_t)h * L, L, L - k, idx + (size_t)h * L, inv ? inv + (size_t)h * L : nullptr,
                          sh.s.r, sh.s.smask, sh.s.sbase);
}

static hipError_t launch_select_resident(const float* s_h, int64_t L, int Hq, const int32_t* Lp_dev, int32_t* idx,
                                         int32_t* inv, hipStream_t st) {
#define TSA_SELECT_RES(NK) select_resident_kernel<NK><<<(unsigned)Hq, kResThreads, 0, st>>>(s_h, L, Lp_dev, idx, inv)
  if (L <= 4 * kResThreads) TSA_SELECT_RES(4);
  else if (L <= 8 * kResThreads) TSA_SELECT_RES(8);
  else if (L <= 16 * kResThreads) TSA_SELECT_RES(16);
  else TSA_SELECT_RES(32);
#undef TSA_SELECT_RES
  return hipGetLastError();
}

hipError_t launch_select(const float* s_h, int64_t L, int Hq, const int32_t* Lp_dev,
                         uint64_t* hist, RadixCtl* ctl, uint32_t* tile_cnt, uint32_t* tile_off,
                         int32_t* idx, int32_t* inv, hipStream_t st) {
  if (radix_resident(L)) return launch_select_resident(s_h, L, Hq, Lp_dev, idx, inv, st);
  const dim3 hgrid((unsigned)((L + kHistTile - 1) / kHistTile), (unsigned)Hq);
  for (int pass = 0; pass < kRadixPasses; ++pass)
    radix_hist_kernel<false><<<hgrid, 256, 0, st>>>(s_h, L, L, pass, 0, Lp_dev, hist, ctl);
  const int64_t nt = select_tiles(L);
  const dim3 sgrid((unsigned)nt, (unsigned)Hq);
  select_count_kernel<<<sgrid, 256, 0, st>>>(s_h, L, Lp_dev, hist, ctl, tile_cnt);
  select_scan_kernel<<<(unsigned)Hq, 64, 0, st>>>(tile_cnt, nt, L, Lp_dev, ctl, tile_off);
  select_write_kernel<<<sgrid, 256, 0, st>>>(s_h, L, Lp_dev, ctl, tile_off, idx, inv);
  return hipGetLastError();
}

// Layer score, budget and selection of a resident row (at most kResidentMax tokens).  The layer
// score's kernels run as in launch_layer_score_budget; budget and selection then take one launch.
hipError_t launch_layer_budget_select(const float* s_h, int64_t L, int Hq, double* S, double* tile_sum, float* s_l,
                                      uint64_t target, int32_t* kLp_ws, int32_t* k_out, int32_t* Lp_out, int32_t* idx,
                                      int32_t* inv, hipStream_t st) {
  int64_t ntiles = 0;
  if (L > 4 * kResThreads) {
    const hipError_t e = launch_layer_score(s_h, L, Hq, S, tile_sum, s_l, st);
    if (e != hipSuccess) return e;
  } else {
    ntiles = layer_tiles(L) - 1;
    layer_sum_kernel<<<(unsigned)ntiles, 256, 0, st>>>(s_h, L, Hq, S, tile_sum);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#define TSA_BUDGET_SELECT(NK, FS) \
  budget_select_resident_kernel<NK, FS><<<(unsigned)Hq, kResThreads, 0, st>>>(s_h, s_l, S, tile_sum, ntiles, s_l, L, \
                                                                              target, kLp_ws, k_out, Lp_out, idx, inv)
  if (L <= 4 * kResThreads) TSA_BUDGET_SELECT(4, true);
  else if (L <= 8 * kResThreads) TSA_BUDGET_SELECT(8, false);
  else if (L <= 16 * kResThreads) TSA_BUDGET_SELECT(16, false);
  else TSA_BUDGET_SELECT(32, false);
#undef TSA_BUDGET_SELECT
  return hipGetLastError();
}

}  // namespace tsa

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
// S[t] = sum over heads in head order (float64); s_l = S / total with the total summed once, in a
// fixed order, by a single block.  One token per thread, so a launch has L/256 blocks.

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
__global__ __launch_bounds__(256) void layer_total_kernel(double* __restrict__ tile_sum, int64_t ntiles) {
  __shared__ double red[4];
  double a = 0.0;
  for (int64_t i = threadIdx.x; i < ntiles; i += 256) a += tile_sum[i];
  a = wave_sum(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) tile_sum[ntiles] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void layer_norm_kernel(const double* __restrict__ S,
                                                         const double* __restrict__ total, int64_t L,
                                                         float* __restrict__ s_l) {
  const int64_t t = (int64_t)blockIdx.x * kLayerTile + threadIdx.x;
  if (t < L) s_l[t] = (float)(S[t] / total[0]);
}

hipError_t launch_layer_score(const float* s_h, int64_t L, int Hq, double* S, double* tile_sum,
                              float* s_l, hipStream_t st) {
  const unsigned n = (unsigned)(layer_tiles(L) - 1);
  layer_sum_kernel<<<n, 256, 0, st>>>(s_h, L, Hq, S, tile_sum);
  layer_total_kernel<<<1, 256, 0, st>>>(tile_sum, n);
  layer_norm_kernel<<<n, 256, 0, st>>>(S, tile_sum + n, L, s_l);
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
  for (int u = 0; u < kHistTile / 256; ++u) {
    const int64_t t = base + u * 256 + threadIdx.x;
    if (t >= L) break;
    const uint32_t key = __float_as_uint(kseg[t]);
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

hipError_t launch_budget(const float* s_l, int64_t L, uint64_t target, uint64_t* hist,
                         RadixCtl* ctl, int32_t* kLp_ws, int32_t* k_out, int32_t* Lp_out,
                         hipStream_t st) {
  const dim3 grid((unsigned)((L + kHistTile - 1) / kHistTile), 1);
  for (int pass = 0; pass < kRadixPasses; ++pass)
    radix_hist_kernel<true><<<grid, 256, 0, st>>>(s_l, L, 0, pass, target, nullptr, hist, ctl);
  budget_final_kernel<<<1, 64, 0, st>>>(hist, ctl, L, target, kLp_ws, k_out, Lp_out);
  return hipGetLastError();
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

hipError_t launch_select(const float* s_h, int64_t L, int Hq, const int32_t* Lp_dev,
                         uint64_t* hist, RadixCtl* ctl, uint32_t* tile_cnt, uint32_t* tile_off,
                         int32_t* idx, int32_t* inv, hipStream_t st) {
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

}  // namespace tsa

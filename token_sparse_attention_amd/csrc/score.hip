// Dynamic Token Coverage scoring (papernotes.org reading notes, "Key design 2"; bxzpzcl.cn article,
// section 2.1): the last q queries of every head attend causally to all keys, and the softmax
// weights are summed over those queries into a per-head token score s_h.
//
// Two passes over K, one block per (256 keys, KV group):
//   pass 1: logits for every recent query row of the group; per-wave (max, sum of exp) partials;
//   combine: per row, the global max m and 1 / sum_t exp(z - m), float64, fixed order;
//   pass 2: the same logits again; w = exp(z - m) / Z summed over each head's q rows -> s_h.
// The dot products, exponentials and sums are float64: the score decides a discrete selection, so
// it is kept far below the 1e-6 relative tie band of the selection (its only rounding is the final
// store to float32).  Both passes compute bit-identical logits.
#include "kern_common.h"
#include "tsa_internal.h"

namespace tsa {

constexpr int kScoreKeys = 256;   // keys per block = threads per block
constexpr int kQChunk = 32;       // recent-query rows staged in LDS at a time

int64_t score_blocks(int64_t L) { return (L + kScoreKeys - 1) / kScoreKeys; }

size_t score_partial_bytes(int64_t L, int Hq, int q) {
  // float64 path: a partial per row, 256-key block and wave; matrix-core path: a partial per padded
  // row and block of at least 256 keys (at most 16 * Hq * ceil(q/16) rows)
  const size_t vec = (size_t)Hq * q * score_blocks(L) * (kScoreKeys / kWave);
  const size_t mfma = (size_t)Hq * ((q + 15) / 16 * 16) * ((L + 255) / 256);
  return (vec > mfma ? vec : mfma) * sizeof(double2);
}

size_t score_rowstat_bytes(int Hq, int q) { return (size_t)Hq * ((q + 15) / 16 * 16) * sizeof(double2); }

template <typename T, int D>
__device__ __forceinline__ void load_row(const T* __restrict__ p, float (&r)[D]) {
  if constexpr (sizeof(T) == 2) {
    const uint4* v = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const uint4 w = v[i];
      const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r[8 * i + 2 * j] = __uint_as_float(a[j] << 16);
        r[8 * i + 2 * j + 1] = __uint_as_float(a[j] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* v = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      const float4 w = v[i];
      r[4 * i] = w.x; r[4 * i + 1] = w.y; r[4 * i + 2] = w.z; r[4 * i + 3] = w.w;
    }
  }
}

// Rows of group g are ordered head-major: row r -> query head g*G + r/q, position L - q + r%q.
template <typename T, int D, int PASS>
__global__ __launch_bounds__(kScoreKeys) void score_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, int64_t L, int Hq, int Hkv, int q,
    double scale, double2* __restrict__ part, const double2* __restrict__ rowstat,
    float* __restrict__ s_h) {
  __shared__ __attribute__((aligned(16))) float qs[kQChunk][D];
  __shared__ double zs[kQChunk][kScoreKeys];
  const int g = blockIdx.y;
  const int64_t blk = blockIdx.x, nblk = gridDim.x;
  const int tid = threadIdx.x;
  const int64_t t = blk * kScoreKeys + tid;
  const bool in = t < L;
  const int G = Hq / Hkv, R = G * q;

  float kr[D];
  if (in) {
    load_row<T, D>(K + ((size_t)t * Hkv + g) * D, kr);
  } else {
#pragma unroll
    for (int c = 0; c < D; ++c) kr[c] = 0.f;
  }

  double hsum = 0.0;
  for (int r0 = 0; r0 < R; r0 += kQChunk) {
    __syncthreads();
    for (int e = tid; e < kQChunk * D; e += kScoreKeys) {
      const int rr = e / D, c = e % D, r = r0 + rr;
      float v = 0.f;
      if (r < R) {
        const int h = g * G + r / q;
        const int64_t p = L - q + r % q;
        v = to_f32<T>(Q[((size_t)p * Hq + h) * D + c]);
      }
      qs[rr][c] = v;
    }
    __syncthreads();
    // acc[j] = <Q row r0+j, K row t>; each K element is widened once and used for all 32 rows.
    double acc[kQChunk];
#pragma unroll
    for (int j = 0; j < kQChunk; ++j) acc[j] = 0.0;
#pragma unroll
    for (int c4 = 0; c4 < D / 4; ++c4) {
      const double k0 = kr[4 * c4], k1 = kr[4 * c4 + 1], k2 = kr[4 * c4 + 2], k3 = kr[4 * c4 + 3];
#pragma unroll
      for (int j = 0; j < kQChunk; ++j) {
        const float4 qv = *reinterpret_cast<const float4*>(&qs[j][4 * c4]);
        acc[j] = fma((double)qv.x, k0, acc[j]);
        acc[j] = fma((double)qv.y, k1, acc[j]);
        acc[j] = fma((double)qv.z, k2, acc[j]);
        acc[j] = fma((double)qv.w, k3, acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < kQChunk; ++j) zs[j][tid] = acc[j];
    // (each thread reads back only its own column: no barrier needed)
#pragma unroll 1
    for (int j = 0; j < kQChunk; ++j) {
      const int r = r0 + j;
      if (r >= R) break;
      const int i = r % q;
      const bool vis = in && t <= L - q + i;       // causal: query at L-q+i sees t <= L-q+i
      const double z = zs[j][tid] * scale;
      if constexpr (PASS == 1) {
        const double m = wave_max(vis ? z : -INFINITY);
        const double e = vis ? exp(z - m) : 0.0;
        const double Z = wave_sum(e);
        if ((tid & 63) == 0)
          part[(((size_t)g * R + r) * nblk + blk) * (kScoreKeys / kWave) + (tid >> 6)] = make_double2(m, Z);
      } else {
        const double2 ms = rowstat[(size_t)g * R + r];
        hsum += vis ? exp(z - ms.x) * ms.y : 0.0;
        if (i == q - 1) {
          if (in) s_h[(size_t)(g * G + r / q) * L + t] = (float)hsum;
          hsum = 0.0;
        }
      }
    }
  }
}

// One wave per row: m = max of the partial maxima, Z = sum_p Z_p exp(m_p - m), fixed order.
// mul converts a difference of stored maxima into the natural-log units of the stored sums.
__global__ __launch_bounds__(256) void score_combine_kernel(const double2* __restrict__ part,
                                                            int64_t nrows, int64_t nparts, double mul,
                                                            double2* __restrict__ rowstat) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= nrows) return;
  const double2* p = part + row * nparts;
  double m = -INFINITY;
  for (int64_t i = lane; i < nparts; i += kWave) m = fmax(m, p[i].x);
  m = wave_max(m);
  double Z = 0.0;
  for (int64_t i = lane; i < nparts; i += kWave) {
    const double2 v = p[i];
    if (v.y > 0.0) Z += v.y * exp((v.x - m) * mul);
  }
  Z = wave_sum(Z);
  if (lane == 0) rowstat[row] = make_double2(m, 1.0 / Z);
}

template <typename T, int D>
static hipError_t run_score(const void* Q, const void* K, int64_t L, int Hq, int Hkv, int q,
                            float* s_h, double2* part, double2* rowstat, hipStream_t st) {
  const double scale = 1.0 / sqrt((double)D);
  const dim3 grid((unsigned)score_blocks(L), (unsigned)Hkv);
  const T* Qt = static_cast<const T*>(Q);
  const T* Kt = static_cast<const T*>(K);
  score_kernel<T, D, 1><<<grid, kScoreKeys, 0, st>>>(Qt, Kt, L, Hq, Hkv, q, scale, part, rowstat, s_h);
  const int64_t nrows = (int64_t)Hq * q;     // Hkv groups x (Hq/Hkv) * q rows
  const int64_t nparts = score_blocks(L) * (kScoreKeys / kWave);
  score_combine_kernel<<<(unsigned)((nrows + 3) / 4), 256, 0, st>>>(part, nrows, nparts, 1.0, rowstat);
  score_kernel<T, D, 2><<<grid, kScoreKeys, 0, st>>>(Qt, Kt, L, Hq, Hkv, q, scale, part, rowstat, s_h);
  return hipGetLastError();
}

// ---- bf16 path on the matrix cores ---------------------------------------------------------------
// Logits z = <Q[p][h], K[t][g]> come from v_mfma_f32_16x16x32_bf16 (bf16 products are exact in
// float32; only the accumulation rounds).  A = 16 recent-query rows of one head (each head's q rows
// padded to a multiple of 16 and staged in LDS), B = 16 keys; a wave owns 64 keys of a 256-key
// sub-chunk and a block walks four sub-chunks (1024 keys) of one KV group.
//   pass 1: per row, max and sum of exponentials over the wave's keys (cross-lane in the 16 lanes of
//           a row group), merged over waves and sub-chunks in LDS: one (max, sum) partial per
//           row and block;
//   pass 2: w = exp(z - m) / Z, summed over each M-tile's 16 rows and over the head's M-tiles.
// Every exponential is exp2 of (z - m) * log2(e) / sqrt(d) formed in float64 from the float32
// logits, evaluated as exp2f(hi) * (1 + lo * ln 2) with hi + lo that argument, and all sums are
// float64: about 1e-7 relative, far inside the selection's 1e-6 tie band.
constexpr int kMSub = 256, kMRows = 256;   // keys per sub-chunk (a block walks nsub of them); max rows

typedef __bf16 bf16x8s_t __attribute__((ext_vector_type(8)));
typedef float f32x4s_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double exp2_rel(float z, float m, double c) {
  const double y = ((double)z - (double)m) * c;
  const float hi = (float)y;
  const float lo = (float)(y - (double)hi);
  return (double)(__builtin_amdgcn_exp2f(hi) * fmaf(lo, 0.69314718055994531f, 1.0f));
}

__device__ __forceinline__ double shfl_sum16(double v) {     // over the 16 lanes of a row group
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float shfl_max16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

template <int D, int PASS>
__global__ __launch_bounds__(256) void score_mfma_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                         int64_t L, int Hq, int Hkv, int q, int qp, int nsub,
                                                         double c, double2* __restrict__ part,
                                                         const double2* __restrict__ rowstat, float* __restrict__ s_h) {
  constexpr int KST = D / 32;                  // K-steps of 32 over the head dim
  // LDS sized by the launch for Rp rows (score_mfma_smem): the recent queries, then per-wave partial
  // max / sum (pass 1) and the block's running max / sum, or the rows' max and 1 / Z (pass 2)
  extern __shared__ __attribute__((aligned(16))) char score_smem[];
  const int g = blockIdx.y, tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int G = Hq / Hkv, Rp = G * qp, MT = Rp / 16;
  uint16_t* qs = reinterpret_cast<uint16_t*>(score_smem);
  double* wz_ = reinterpret_cast<double*>(score_smem + (size_t)Rp * D * 2);
  double* bz = wz_ + 4 * Rp;
  float* wm_ = reinterpret_cast<float*>(bz + Rp);
  float* bm = wm_ + 4 * Rp;
  auto wm = [&](int v, int r) -> float& { return wm_[v * Rp + r]; };
  auto wz = [&](int v, int r) -> double& { return wz_[v * Rp + r]; };
  const int64_t nblk = gridDim.x;
  for (int e = tid; e < Rp * (D / 8); e += 256) {
    const int row = e / (D / 8), c8 = e % (D / 8), j = row / qp, i = row % qp;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (i < q) v = *reinterpret_cast<const uint4*>(Q + ((size_t)(L - q + i) * Hq + g * G + j) * D + 8 * c8);
    *reinterpret_cast<uint4*>(&qs[row * D + 8 * c8]) = v;
  }
  for (int r = tid; r < Rp; r += 256) {
    if (PASS == 1) {
      bm[r] = -INFINITY;
      bz[r] = 0.0;
    } else {
      const double2 ms = rowstat[(size_t)g * Rp + r];
      bm[r] = (float)ms.x;
      bz[r] = ms.y;
    }
  }
  __syncthreads();

  // Blocks whose keys all precede the recent window, with every padded row real (q % 16 == 0), see
  // every key from every row: no masks.
  const int64_t bkeys = (int64_t)nsub * kMSub;
  const bool open = (int64_t)(blockIdx.x + 1) * bkeys <= L - q + 1 && q == qp;
  for (int sub = 0; sub < nsub; ++sub) {
    const int64_t key0 = ((int64_t)blockIdx.x * bkeys + sub * kMSub) + 64 * w;
    bf16x8s_t kf[4][KST];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int64_t key = key0 + 16 * n + l16;
#pragma unroll
      for (int ks = 0; ks < KST; ++ks)
        kf[n][ks] = key < L ? *reinterpret_cast<const bf16x8s_t*>(K + ((size_t)key * Hkv + g) * D + 32 * ks + 8 * lg)
                            : bf16x8s_t{};
    }
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int mt = 0; mt < MT; ++mt) {
      f32x4s_t z[4] = {f32x4s_t{}, f32x4s_t{}, f32x4s_t{}, f32x4s_t{}};
#pragma unroll
      for (int ks = 0; ks < KST; ++ks) {
        const bf16x8s_t a = *reinterpret_cast<const bf16x8s_t*>(&qs[(16 * mt + l16) * D + 32 * ks + 8 * lg]);
#pragma unroll
        for (int n = 0; n < 4; ++n) z[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, kf[n][ks], z[n], 0, 0, 0);
      }
      // z[n][r]: row 16*mt + 4*lg + r, key key0 + 16*n + l16
      const int j = (16 * mt) / qp;
      if (PASS == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * lg + r, i = row % qp;
          const int64_t p = L - q + i;
          float zm = -INFINITY;
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const int64_t key = key0 + 16 * n + l16;
            if (open || (i < q && key <= p)) zm = fmaxf(zm, z[n][r]);
          }
          zm = shfl_max16(zm);
          double zs = 0.0;
          if (zm > -INFINITY) {
#pragma unroll
            for (int n = 0; n < 4; ++n) {
              const int64_t key = key0 + 16 * n + l16;
              if (open || (i < q && key <= p)) zs += exp2_rel(z[n][r], zm, c);
            }
          }
          zs = shfl_sum16(zs);
          if (l16 == 0) {
            wm(w, row) = zm;
            wz(w, row) = zs;
          }
        }
      } else {
        double cs[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * lg + r, i = row % qp;
          const int64_t p = L - q + i;
          const float m = bm[row];
          const double iz = bz[row];
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const int64_t key = key0 + 16 * n + l16;
            if (open || (i < q && key <= p)) cs[n] += exp2_rel(z[n][r], m, c) * iz;
          }
        }
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          cs[n] += __shfl_xor(cs[n], 16, kWave);
          cs[n] += __shfl_xor(cs[n], 32, kWave);
          acc[n] += cs[n];
        }
        if ((16 * (mt + 1)) % qp == 0) {       // last M-tile of head j: store its column sums
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const int64_t key = key0 + 16 * n + l16;
            if (lg == 0 && key < L) s_h[(size_t)(g * G + j) * L + key] = (float)acc[n];
            acc[n] = 0.0;
          }
        }
      }
    }
    if (PASS == 1) {                            // merge the four waves into the block's running state
      __syncthreads();
      for (int r = tid; r < Rp; r += 256) {
        float m = bm[r];
#pragma unroll
        for (int v = 0; v < 4; ++v) m = fmaxf(m, wm(v, r));
        double Z = 0.0;
        if (m > -INFINITY) {
          if (bz[r] > 0.0) Z += bz[r] * exp2(((double)bm[r] - (double)m) * c);
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (wz(v, r) > 0.0) Z += wz(v, r) * exp2(((double)wm(v, r) - (double)m) * c);
        }
        bm[r] = m;
        bz[r] = Z;
      }
      __syncthreads();
    }
  }
  if (PASS == 1)
    for (int r = tid; r < Rp; r += 256) part[((size_t)g * Rp + r) * nblk + blockIdx.x] = make_double2(bm[r], bz[r]);
}

int score_rows_padded(int Hq, int Hkv, int q) { return (Hq / Hkv) * ((q + 15) / 16 * 16); }

// dynamic LDS of score_mfma_kernel for Rp rows of head dimension D
static size_t score_mfma_smem(int Rp, int D) { return (size_t)Rp * D * 2 + (size_t)Rp * 5 * 8 + (size_t)Rp * 5 * 4; }

static bool use_mfma(int dtype, int Hq, int Hkv, int q) {
  return dtype == 1 && score_rows_padded(Hq, Hkv, q) <= kMRows;
}

template <int D>
static hipError_t run_score_mfma(const void* Q, const void* K, int64_t L, int Hq, int Hkv, int q, float* s_h,
                                 double2* part, double2* rowstat, hipStream_t st) {
  const int qp = (q + 15) / 16 * 16, Rp = score_rows_padded(Hq, Hkv, q);
  const double scale = 1.0 / sqrt((double)D), c = scale * 1.4426950408889634;
  // keys per block: 1024 when that still gives ~2 blocks per CU, down to 256 for short sequences
  int nsub = 4;
  while (nsub > 1 && ((L + nsub * kMSub - 1) / (nsub * kMSub)) * Hkv < 512) nsub >>= 1;
  const dim3 grid((unsigned)((L + nsub * kMSub - 1) / (nsub * kMSub)), (unsigned)Hkv);
  const uint16_t* Qt = static_cast<const uint16_t*>(Q);
  const uint16_t* Kt = static_cast<const uint16_t*>(K);
  const size_t smem = score_mfma_smem(Rp, D);
  if (smem > 48 * 1024) {                     // up to 79 KB for 256 rows: raise the dynamic-LDS limit
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&score_mfma_kernel<D, 1>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&score_mfma_kernel<D, 2>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  score_mfma_kernel<D, 1><<<grid, 256, smem, st>>>(Qt, Kt, L, Hq, Hkv, q, qp, nsub, c, part, rowstat, s_h);
  const int64_t nrows = (int64_t)Hkv * Rp;
  score_combine_kernel<<<(unsigned)((nrows + 3) / 4), 256, 0, st>>>(part, nrows, grid.x, scale, rowstat);
  score_mfma_kernel<D, 2><<<grid, 256, smem, st>>>(Qt, Kt, L, Hq, Hkv, q, qp, nsub, c, part, rowstat, s_h);
  return hipGetLastError();
}

hipError_t launch_score(int dtype, int d, const void* Q, const void* K, int64_t L, int Hq, int Hkv,
                        int q, float* s_h, double2* part, double2* rowstat, hipStream_t st) {
  if (use_mfma(dtype, Hq, Hkv, q))
    return d == 128 ? run_score_mfma<128>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st)
                    : run_score_mfma<64>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
  if (dtype == 1) {
    return d == 128 ? run_score<uint16_t, 128>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st)
                    : run_score<uint16_t, 64>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
  }
  return d == 128 ? run_score<float, 128>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st)
                  : run_score<float, 64>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
}

}  // namespace tsa

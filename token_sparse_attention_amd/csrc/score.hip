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
  return (size_t)Hq * q * score_blocks(L) * (kScoreKeys / kWave) * sizeof(double2);
}

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
__global__ __launch_bounds__(256) void score_combine_kernel(const double2* __restrict__ part,
                                                            int64_t nrows, int64_t nparts,
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
    if (v.y > 0.0) Z += v.y * exp(v.x - m);
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
  score_combine_kernel<<<(unsigned)((nrows + 3) / 4), 256, 0, st>>>(part, nrows, nparts, rowstat);
  score_kernel<T, D, 2><<<grid, kScoreKeys, 0, st>>>(Qt, Kt, L, Hq, Hkv, q, scale, part, rowstat, s_h);
  return hipGetLastError();
}

hipError_t launch_score(int dtype, int d, const void* Q, const void* K, int64_t L, int Hq, int Hkv,
                        int q, float* s_h, double2* part, double2* rowstat, hipStream_t st) {
  if (dtype == 1) {
    return d == 128 ? run_score<uint16_t, 128>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st)
                    : run_score<uint16_t, 64>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
  }
  return d == 128 ? run_score<float, 128>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st)
                  : run_score<float, 64>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
}

}  // namespace tsa

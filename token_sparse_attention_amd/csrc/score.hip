// Dynamic Token Coverage scoring (papernotes.org reading notes, "Key design 2"; bxzpzcl.cn article,
// section 2.1): the last q queries of every head attend causally to all keys, and the softmax
// weights are summed over those queries into a per-head token score s_h.
//
// Two passes over K, one block per (256 keys, KV group):
//   pass 1: logits for every recent query row of the group; per-wave (max, sum of exp) partials;
//   combine: per row, the global max m and 1 / sum_t exp(z - m), float64, fixed order;
//   pass 2: the same logits again; w = exp(z - m) / Z summed over each head's q rows -> s_h.
// The score decides a discrete selection, so its error is kept far below the selection's 1e-6
// relative tie band.  The vector-ALU kernel below (fp32 inputs, and bf16 groups of more than 256
// padded rows) forms dot products, exponentials and sums in float64, its only rounding the final
// store to float32; the matrix-core kernels further down keep within a few 1e-7 (described there).
// Both passes compute bit-identical logits.
#include "kern_common.h"
#include "tsa_internal.h"

namespace tsa {

constexpr int kScoreKeys = 256;   // keys per block = threads per block
constexpr int kQChunk = 32;       // recent-query rows staged in LDS at a time (16 when a group has no more)

int64_t score_blocks(int64_t L) { return (L + kScoreKeys - 1) / kScoreKeys; }

size_t score_partial_bytes(int64_t L, int Hq, int Hkv, int q) {
  // float64 path: a partial per row, 256-key block and wave; matrix-core path: a partial per padded
  // row (each group's rows padded to a multiple of 32, heads to 16 or a multiple of 32) and block of
  // at least 256 keys
  const size_t vec = (size_t)Hq * q * score_blocks(L) * (kScoreKeys / kWave);
  const size_t rows = (size_t)Hkv * (((Hq / Hkv) * (q <= 16 ? 16 : (q + 31) / 32 * 32) + 31) / 32 * 32);
  const size_t mfma = rows * ((L + 255) / 256);
  return (vec > mfma ? vec : mfma) * sizeof(double2);
}

size_t score_rowstat_bytes(int Hq, int Hkv, int q) {
  const size_t vec = (size_t)Hq * q;
  const size_t rows = (size_t)Hkv * (((Hq / Hkv) * (q <= 16 ? 16 : (q + 31) / 32 * 32) + 31) / 32 * 32);
  return (vec > rows ? vec : rows) * sizeof(double2);
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
// QC rows are formed at a time; every row's arithmetic is the same for either QC.
template <typename T, int D, int PASS, int QC>
__global__ __launch_bounds__(kScoreKeys) void score_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, int64_t L, int Hq, int Hkv, int q,
    double scale, double2* __restrict__ part, const double2* __restrict__ rowstat,
    float* __restrict__ s_h) {
  __shared__ __attribute__((aligned(16))) float qs[QC][D];
  __shared__ double zs[QC][kScoreKeys];
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
  for (int r0 = 0; r0 < R; r0 += QC) {
    __syncthreads();
    for (int e = tid; e < QC * D; e += kScoreKeys) {
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
    double acc[QC];
#pragma unroll
    for (int j = 0; j < QC; ++j) acc[j] = 0.0;
#pragma unroll
    for (int c4 = 0; c4 < D / 4; ++c4) {
      const double k0 = kr[4 * c4], k1 = kr[4 * c4 + 1], k2 = kr[4 * c4 + 2], k3 = kr[4 * c4 + 3];
#pragma unroll
      for (int j = 0; j < QC; ++j) {
        const float4 qv = *reinterpret_cast<const float4*>(&qs[j][4 * c4]);
        acc[j] = fma((double)qv.x, k0, acc[j]);
        acc[j] = fma((double)qv.y, k1, acc[j]);
        acc[j] = fma((double)qv.z, k2, acc[j]);
        acc[j] = fma((double)qv.w, k3, acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < QC; ++j) zs[j][tid] = acc[j];
    // (each thread reads back only its own column: no barrier needed)
#pragma unroll 1
    for (int j = 0; j < QC; ++j) {
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
  const bool small = (Hq / Hkv) * q <= kQChunk / 2;   // a group's rows fit one 16-row chunk
  if (small) score_kernel<T, D, 1, kQChunk / 2><<<grid, kScoreKeys, 0, st>>>(Qt, Kt, L, Hq, Hkv, q, scale, part, rowstat, s_h);
  else score_kernel<T, D, 1, kQChunk><<<grid, kScoreKeys, 0, st>>>(Qt, Kt, L, Hq, Hkv, q, scale, part, rowstat, s_h);
  const int64_t nrows = (int64_t)Hq * q;     // Hkv groups x (Hq/Hkv) * q rows
  const int64_t nparts = score_blocks(L) * (kScoreKeys / kWave);
  score_combine_kernel<<<(unsigned)((nrows + 3) / 4), 256, 0, st>>>(part, nrows, nparts, 1.0, rowstat);
  if (small) score_kernel<T, D, 2, kQChunk / 2><<<grid, kScoreKeys, 0, st>>>(Qt, Kt, L, Hq, Hkv, q, scale, part, rowstat, s_h);
  else score_kernel<T, D, 2, kQChunk><<<grid, kScoreKeys, 0, st>>>(Qt, Kt, L, Hq, Hkv, q, scale, part, rowstat, s_h);
  return hipGetLastError();
}

// ---- bf16 path on the matrix cores ---------------------------------------------------------------
// Logits z = <Q[p][h], K[t][g]> come from v_mfma_f32_32x32x16_bf16 (bf16 products are exact in
// float32; only the accumulation rounds).  The recent-query rows of a KV group are staged in LDS,
// each head's q rows padded to 16 (q <= 16) or to a multiple of 32, the group to a multiple of 32
// (MB blocks of 32 rows, a template parameter so the row loops unroll).  A wave owns 64 keys (two
// blocks of 32) of each 256-key sub-chunk; a workgroup walks nsub sub-chunks of one KV group.  The
// product is oriented so that every reduction is lane-local:
//   pass 1: D = K Q^T, a lane holds 16 keys of ONE row: it keeps that row's (reference R, sum of
//           exp2((z - R) c)) in registers over all of the workgroup's keys; the two lanes sharing a
//           row and the four waves are merged once at the end, one (R, Z) partial per row and
//           workgroup.  R is the first visible logit block's maximum and is raised only when a
//           logit exceeds it by more than kRaise / c (2^32 in weight), so every exponential stays
//           far from overflow and the (float64) rescale of the sum is rare;
//   pass 2: D = Q K^T, a lane holds 16 rows of ONE key: the weights exp2((z - m) c) / Z are summed
//           over the head's rows in the lane, plus one exchange with the lane holding the other
//           rows.
// Causal masks are applied only in workgroups that reach the recent window.  Every exponential is
// v_exp_f32 of a float32 argument (z - R) * c, with c split into a float32 pair (c_hi + c_lo) so
// the product rounds once; 16 weights are summed pairwise in float32 and those sums in float64.  The
// relative error of a score stays within a few 1e-7, inside the selection's 1e-6 tie band.
constexpr int kMSub = 256, kMRows = 256;   // keys per sub-chunk (a block walks nsub of them); max rows
constexpr float kRaise = 32.f;             // pass 1 raises its reference past this many log2 units
// Masked logits: finite, so (z - R) * c stays finite whatever the sign of c's low part (an infinite
// z would meet an infinity of the other sign in the split product), and its exponential is exactly 0
constexpr float kMasked = -1e30f;

typedef __bf16 bf16x8s_t __attribute__((ext_vector_type(8)));
typedef float f32x16s_t __attribute__((ext_vector_type(16)));

// The fragments of one key row (`key`, zeros past L) as the matrix-core operand wants them: lane
// half hf holds the 8 consecutive head-dim elements 16 ks + 8 hf of slice ks.
template <int D>
__device__ __forceinline__ void load_key_block(const uint16_t* __restrict__ K, int64_t L, int Hkv, int g,
                                               int64_t key, int hf, bf16x8s_t (&kf)[D / 16]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    kf[ks] = key < L ? *reinterpret_cast<const bf16x8s_t*>(K + ((size_t)key * Hkv + g) * D + 16 * ks + 8 * hf)
                     : bf16x8s_t{};
}

// LDS slot of 16-byte chunk c8 of staged query row r (XOR swizzle: 16 consecutive rows' reads of
// one chunk land on distinct banks)
template <int D>
__device__ __forceinline__ int qslot(int r, int c8) { return r * D + 8 * (c8 ^ (r & (D / 8 - 1))); }

// Stages the group's recent-query rows (row = j * qp + i for head j, recent query i; zero padding)
template <int D>
__device__ __forceinline__ void stage_queries(const uint16_t* __restrict__ Q, uint16_t* qs, int64_t L, int Hq, int g,
                                              int G, int q, int qp, int Rp) {
  for (int e = threadIdx.x; e < Rp * (D / 8); e += 256) {
    const int row = e / (D / 8), c8 = e % (D / 8), j = row / qp, i = row % qp;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < G && i < q) v = *reinterpret_cast<const uint4*>(Q + ((size_t)(L - q + i) * Hq + g * G + j) * D + 8 * c8);
    *reinterpret_cast<uint4*>(&qs[qslot<D>(row, c8)]) = v;
  }
}

// exp2((z - R) * c) for a logit z, c = c_hi + c_lo (kMasked gives exactly 0)
__device__ __forceinline__ float exp2_rel(float z, float R, float c_hi, float c_lo) {
  const float d = z - R;
  return __builtin_amdgcn_exp2f(fmaf(d, c_hi, d * c_lo));
}

// pairwise float32 sum of v[lo .. lo + n)
template <int N>
__device__ __forceinline__ float pair_sum(const float* v) {
  if constexpr (N == 1) return v[0];
  else return pair_sum<N / 2>(v) + pair_sum<N / 2>(v + N / 2);
}

template <int D, int MB>
__global__ __launch_bounds__(256, MB <= 2 ? 4 : 3) void score_p1_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                       int64_t L, int Hq, int Hkv, int q, int qp, int nsub, double c,
                                                       double2* __restrict__ part) {
  constexpr int KST = D / 16, Rp = 32 * MB;
  extern __shared__ __attribute__((aligned(16))) char score_smem[];
  const int g = blockIdx.y, tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int G = Hq / Hkv;
  uint16_t* qs = reinterpret_cast<uint16_t*>(score_smem);
  double* wz = reinterpret_cast<double*>(score_smem + (size_t)Rp * D * 2);   // [4][Rp]
  float* wm = reinterpret_cast<float*>(wz + 4 * Rp);                         // [4][Rp]
  stage_queries<D>(Q, qs, L, Hq, g, G, q, qp, Rp);
  __syncthreads();

  const float c_hi = (float)c, c_lo = (float)(c - (double)c_hi), raise = kRaise / c_hi;
  const int64_t bkeys = (int64_t)nsub * kMSub;
  // every key of the workgroup precedes every recent query: no causal mask
  const bool open = (int64_t)(blockIdx.x + 1) * bkeys <= L - q + 1;
  float R[MB];
  double S[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    R[mb] = -INFINITY;
    S[mb] = 0.0;
  }
  // the wave's key blocks of 32, jb = 2 sub + kb; the next block's fragments are loaded into the same
  // registers as soon as the current block's last product has been issued, so the loads run under
  // the exponentials (and the other waves of the SIMD)
  auto key_of = [&](int jb) { return (int64_t)blockIdx.x * bkeys + (jb >> 1) * kMSub + 64 * w + 32 * (jb & 1); };
  bf16x8s_t kf[KST];
  load_key_block<D>(K, L, Hkv, g, key_of(0) + l32, hf, kf);
#pragma unroll 1
  for (int jb = 0; jb < 2 * nsub; ++jb) {
    // z[r] below is key kbase + 8 (r / 4) + 4 hf + r % 4 of the lane's row
    const int64_t kbase = key_of(jb);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = 32 * mb + l32;
      f32x16s_t z = {};
#pragma unroll
      for (int ks = 0; ks < KST; ++ks)
        z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], *reinterpret_cast<const bf16x8s_t*>(&qs[qslot<D>(row, 2 * ks + hf)]),
                                                    z, 0, 0, 0);
      if (mb == MB - 1 && jb + 1 < 2 * nsub) load_key_block<D>(K, L, Hkv, g, key_of(jb + 1) + l32, hf, kf);
      if (!open) {
        // keys kbase + rel with rel <= lim are visible to this lane's row (none for padding rows)
        const int j = row / qp, i = row % qp;
        int lim = -1;
        if (j < G && i < q) {
          const int64_t last = L - q + i;                        // the row's last visible key
          lim = (int)(last - kbase < 63 ? (last - kbase < -1 ? -1 : last - kbase) : 63);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 8 * (r >> 2) + 4 * hf + (r & 3) <= lim ? z[r] : kMasked;
      }
      float zm = z[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) zm = fmaxf(zm, z[r]);
      if (zm > 0.1f * kMasked) {              // some key visible
        if (zm > R[mb] + raise) {             // first visible block, or a logit far above the reference
          if (R[mb] > -INFINITY) S[mb] *= exp2(((double)R[mb] - (double)zm) * c);
          R[mb] = zm;
        }
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = exp2_rel(z[r], R[mb], c_hi, c_lo);
        S[mb] += (double)pair_sum<16>(e);
      }
      // one row block at a time: keeps a single block's accumulators and fragments live
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the two lanes of a row, then the four waves
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const float m2 = __shfl_xor(R[mb], 32, kWave);
    const double s2 = __shfl_xor(S[mb], 32, kWave);
    const float mn = fmaxf(R[mb], m2);
    double Z = 0.0;
    if (mn > -INFINITY) {
      if (R[mb] > -INFINITY) Z += S[mb] * exp2(((double)R[mb] - (double)mn) * c);
      if (m2 > -INFINITY) Z += s2 * exp2(((double)m2 - (double)mn) * c);
    }
    if (hf == 0) {
      wm[w * Rp + 32 * mb + l32] = mn;
      wz[w * Rp + 32 * mb + l32] = Z;
    }
  }
  __syncthreads();
  const int64_t nblk = gridDim.x;
  for (int r = tid; r < Rp; r += 256) {
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) m = fmaxf(m, wm[v * Rp + r]);
    double Z = 0.0;
    if (m > -INFINITY) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (wz[v * Rp + r] > 0.0) Z += wz[v * Rp + r] * exp2(((double)wm[v * Rp + r] - (double)m) * c);
    }
    part[((size_t)g * Rp + r) * nblk + blockIdx.x] = make_double2(m, Z);
  }
}

template <int D, int MB>
__global__ __launch_bounds__(256, MB <= 2 ? 4 : 3) void score_p2_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                       int64_t L, int Hq, int Hkv, int q, int qp, int nsub, double c,
                                                       const double2* __restrict__ rowstat, float* __restrict__ s_h) {
  constexpr int KST = D / 16, Rp = 32 * MB;
  extern __shared__ __attribute__((aligned(16))) char score_smem[];
  const int g = blockIdx.y, tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int G = Hq / Hkv;
  uint16_t* qs = reinterpret_cast<uint16_t*>(score_smem);
  float2* rc = reinterpret_cast<float2*>(score_smem + (size_t)Rp * D * 2);   // per row: m, 1 / Z
  stage_queries<D>(Q, qs, L, Hq, g, G, q, qp, Rp);
  for (int r = tid; r < Rp; r += 256) {
    const double2 ms = rowstat[(size_t)g * Rp + r];
    const bool ok = r / qp < G && r % qp < q && ms.x > -INFINITY;
    rc[r] = ok ? make_float2((float)ms.x, (float)ms.y) : make_float2(0.f, 0.f);   // 1 / Z = 0: no such row
  }
  __syncthreads();

  const float c_hi = (float)c, c_lo = (float)(c - (double)c_hi);
  const int64_t bkeys = (int64_t)nsub * kMSub;
  // key chunks in reverse order: pass 1 streamed K front to back, so its tail is what the
  // last-level cache still holds
  const int64_t kblk = (int64_t)gridDim.x - 1 - blockIdx.x;
  const bool open = (kblk + 1) * bkeys <= L - q + 1;
  // this lane's key in block jb; as in pass 1, the next block's fragments load into the same
  // registers once the current block's last product has been issued
  auto key_of = [&](int jb) { return kblk * bkeys + (jb >> 1) * kMSub + 64 * w + 32 * (jb & 1) + l32; };
  bf16x8s_t kf[KST];
  load_key_block<D>(K, L, Hkv, g, key_of(0), hf, kf);
#pragma unroll 1
  for (int jb = 0; jb < 2 * nsub; ++jb) {
    const int64_t key = key_of(jb);
    // visible to recent query i iff key - (L - q) <= i (always in workgroups before the window)
    const int64_t kr64 = key - (L - q);
    const int kr = open ? -1 : (int)(kr64 < -1 ? -1 : (kr64 > 1 << 20 ? 1 << 20 : kr64));
    double hsA = 0.0, hsB = 0.0;            // the current head's rows (qp = 16: two heads)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x16s_t z = {};
#pragma unroll
      for (int ks = 0; ks < KST; ++ks)
        z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8s_t*>(&qs[qslot<D>(32 * mb + l32, 2 * ks + hf)]),
                                                    kf[ks], z, 0, 0, 0);
      if (mb == MB - 1 && jb + 1 < 2 * nsub) load_key_block<D>(K, L, Hkv, g, key_of(jb + 1), hf, kf);
      // z[r]: row 32 mb + 8 (r / 4) + 4 hf + r % 4 (its constants are LDS broadcasts: every lane
      // of a half reads the same row), recent-query index ibase + that offset (qp = 16: mod 16)
      const int ibase = qp == 16 ? 0 : (32 * mb) % qp;
      float wgt[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int off0 = 8 * r4 + 4 * hf;
        const float4 c01 = *reinterpret_cast<const float4*>(&rc[32 * mb + off0]);
        const float4 c23 = *reinterpret_cast<const float4*>(&rc[32 * mb + off0 + 2]);
        const float mr[4] = {c01.x, c01.z, c23.x, c23.z}, iz[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * r4 + u, off = off0 + u;
          const int i = qp == 16 ? off - 16 * (r >> 3) : ibase + off;
          const float zv = kr <= i ? z[r] : kMasked;                // masked: weight exactly 0
          wgt[r] = exp2_rel(zv, mr[u], c_hi, c_lo) * iz[u];
        }
      }
      if (qp == 16) {                       // rows 0-7 of the lane are head 2 mb, rows 8-15 head 2 mb + 1
        hsA += (double)pair_sum<8>(wgt);
        hsB += (double)pair_sum<8>(wgt + 8);
      } else {
        hsA += (double)pair_sum<16>(wgt);
      }
      if (qp == 16 || (32 * (mb + 1)) % qp == 0) {     // the block ends a head (qp = 16: two)
        const int jA = qp == 16 ? 2 * mb : (32 * mb) / qp;
        const double a = hsA + __shfl_xor(hsA, 32, kWave);
        if (hf == 0 && key < L && jA < G) s_h[(size_t)(g * G + jA) * L + key] = (float)a;
        if (qp == 16) {
          const double bsum = hsB + __shfl_xor(hsB, 32, kWave);
          if (hf == 0 && key < L && jA + 1 < G) s_h[(size_t)(g * G + jA + 1) * L + key] = (float)bsum;
        }
        hsA = 0.0;
        hsB = 0.0;
      }
      __builtin_amdgcn_sched_barrier(0);    // one row block at a time, as in pass 1
    }
  }
}

// recent-query rows per head in the matrix-core path: 16 when q <= 16, else q rounded up to 32
static int score_qp(int q) { return q <= 16 ? 16 : (q + 31) / 32 * 32; }

int score_rows_padded(int Hq, int Hkv, int q) { return ((Hq / Hkv) * score_qp(q) + 31) / 32 * 32; }

static bool use_mfma(int dtype, int Hq, int Hkv, int q) {
  return dtype == 1 && score_rows_padded(Hq, Hkv, q) <= kMRows;
}

// dynamic LDS of the two kernels for Rp rows of head dimension D (pass 1 is the larger)
static size_t score_mfma_smem(int Rp, int D) { return (size_t)Rp * D * 2 + (size_t)Rp * 4 * (8 + 4); }

template <int D, int MB>
static hipError_t run_score_mfma(const void* Q, const void* K, int64_t L, int Hq, int Hkv, int q, float* s_h,
                                 double2* part, double2* rowstat, hipStream_t st) {
  constexpr int Rp = 32 * MB;
  const int qp = score_qp(q);
  const double scale = 1.0 / sqrt((double)D), c = scale * 1.4426950408889634;
  // keys per block: 1024 when that still gives ~2 blocks per CU, down to 256 for short sequences
  int nsub = 4;
  while (nsub > 1 && ((L + nsub * kMSub - 1) / (nsub * kMSub)) * Hkv < 512) nsub >>= 1;
  const dim3 grid((unsigned)((L + nsub * kMSub - 1) / (nsub * kMSub)), (unsigned)Hkv);
  const uint16_t* Qt = static_cast<const uint16_t*>(Q);
  const uint16_t* Kt = static_cast<const uint16_t*>(K);
  const size_t smem = score_mfma_smem(Rp, D);
  if (smem > 48 * 1024) {                     // up to 76 KB for 256 rows: raise the dynamic-LDS limit
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&score_p1_kernel<D, MB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&score_p2_kernel<D, MB>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  score_p1_kernel<D, MB><<<grid, 256, smem, st>>>(Qt, Kt, L, Hq, Hkv, q, qp, nsub, c, part);
  const int64_t nrows = (int64_t)Hkv * Rp;
  score_combine_kernel<<<(unsigned)((nrows + 3) / 4), 256, 0, st>>>(part, nrows, grid.x, scale, rowstat);
  score_p2_kernel<D, MB><<<grid, 256, smem, st>>>(Qt, Kt, L, Hq, Hkv, q, qp, nsub, c, rowstat, s_h);
  return hipGetLastError();
}

template <int D>
static hipError_t run_score_mfma_rows(const void* Q, const void* K, int64_t L, int Hq, int Hkv, int q, float* s_h,
                                      double2* part, double2* rowstat, hipStream_t st) {
  switch (score_rows_padded(Hq, Hkv, q) / 32) {
    case 1: return run_score_mfma<D, 1>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
    case 2: return run_score_mfma<D, 2>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
    case 3: return run_score_mfma<D, 3>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
    case 4: return run_score_mfma<D, 4>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
    case 5: return run_score_mfma<D, 5>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
    case 6: return run_score_mfma<D, 6>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
    case 7: return run_score_mfma<D, 7>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
    default: return run_score_mfma<D, 8>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
  }
}

hipError_t launch_score(int dtype, int d, const void* Q, const void* K, int64_t L, int Hq, int Hkv,
                        int q, float* s_h, double2* part, double2* rowstat, hipStream_t st) {
  if (use_mfma(dtype, Hq, Hkv, q))
    return d == 128 ? run_score_mfma_rows<128>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st)
                    : run_score_mfma_rows<64>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
  if (dtype == 1) {
    return d == 128 ? run_score<uint16_t, 128>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st)
                    : run_score<uint16_t, 64>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
  }
  return d == 128 ? run_score<float, 128>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st)
                  : run_score<float, 64>(Q, K, L, Hq, Hkv, q, s_h, part, rowstat, st);
}

}  // namespace tsa

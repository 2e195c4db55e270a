// Causal softmax attention, O = softmax(Q K^T / sqrt(d)) V with key j visible to query i iff j <= i
// (bxzpzcl.cn article, section 1.1; papernotes.org reading notes, "Key design 1": dense attention on
// the compressed L' x L' problem; the mask by original position reduces to j <= i because the
// selected indices are ascending).  The same kernels run the dense full-length attention that the
// sparse layers are measured against.
//
// bf16 path (gfx950 matrix cores).  A block owns 128 query rows of one head, 4 waves x 32 rows, and
// walks 64-key tiles of K and V^T staged in LDS (double-buffered, one barrier per tile).  The scores
// are formed transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows, B = Q rows), so each
// lane holds 32 scores of ONE query row: the row max is a lane-local reduction plus one exchange
// with the partner lane (l ^ 32), and the exponentials feed O^T = V^T P^T directly as the B operand
// of the second product without any shuffle.  The accumulator O^T also keeps one query per lane, so
// the online-softmax rescale is lane-local.  Softmax statistics and accumulation are float32.
// Query rows are scheduled heaviest first, and on 8-XCD parts consecutive blocks of one XCD work on
// the same head so its L2 serves the shared K/V tiles.
//
// f32 path: a plain vector-ALU kernel (4 lanes per query row, 32-key tiles in LDS), float32 math.
#include "kern_common.h"
#include "tsa_internal.h"

namespace tsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const void* Q;        // compressed: Qh [Hq][C][d];  dense: Q [L][Hq][d]
  const void* K;        // compressed: Kh [Hq][C][d];  dense: K [L][Hkv][d]
  const void* Vt;       // compressed: Vht [Hq][d][C]; dense: Vt [Hkv][d][C]
  const int32_t* Lp_dev;
  const void* X;        // dense only: residual [L][Hq][d] or null
  void* O;              // compressed: Oh [Hq][C][d];  dense: Y [L][Hq][d]
  int64_t L, C;
  int Hq, Hkv;
  float scale;
};

// blockIdx -> (head, query block), heavy (late) query blocks first.
__device__ __forceinline__ void block_coords(int nmb, int Hq, int& h, int& mb) {
  const int b = blockIdx.x;
  if ((Hq & 7) == 0) {
    const int xcd = b & 7, slot = b >> 3;
    h = (slot / nmb) * 8 + xcd;
    mb = nmb - 1 - slot % nmb;
  } else {
    h = b / nmb;
    mb = nmb - 1 - b % nmb;
  }
}

// ------------------------------------------------------------------------------------------------
// bf16, matrix cores
// ------------------------------------------------------------------------------------------------
template <int D, bool DENSE>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
  constexpr int BM = 128, BN = 64;
  constexpr int KS = D / 16;          // K-steps of 16 over the head dim (score product)
  constexpr int DT = D / 32;          // 32-row tiles of O^T over the head dim
  constexpr int KLD = D + 8;          // LDS row pitch (elements) of the K tile
  constexpr int VLD = BN + 8;         // LDS row pitch of the V^T tile
  constexpr int KCH = BN * D / 8 / 256;   // 16-byte chunks per thread per K tile
  constexpr int VCH = D * BN / 8 / 256;   // ... per V^T tile
  __shared__ __attribute__((aligned(16))) uint16_t smK[2][BN * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t smV[2][D * VLD];

  const int nmb = (int)((a.L + BM - 1) / BM);
  int h, mb;
  block_coords(nmb, a.Hq, h, mb);
  const int64_t Lp = DENSE ? a.L : (int64_t)a.Lp_dev[0];
  const int64_t m0 = (int64_t)mb * BM;
  if (m0 >= Lp) return;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int g = h / (a.Hq / a.Hkv);
  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q);
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K);
  const uint16_t* Vp = static_cast<const uint16_t*>(a.Vt);
  // element offsets
  auto q_row = [&](int64_t i) -> size_t { return DENSE ? ((size_t)i * a.Hq + h) * D : ((size_t)h * a.C + i) * D; };
  auto k_row = [&](int64_t j) -> size_t { return DENSE ? ((size_t)j * a.Hkv + g) * D : ((size_t)h * a.C + j) * D; };
  const size_t v_base = (size_t)(DENSE ? g : h) * D * a.C;

  const int64_t qi = m0 + 32 * w + ln;      // this lane's query row
  bf16x8_t qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (qi < Lp) {
      qf[s] = *reinterpret_cast<const bf16x8_t*>(Qp + q_row(qi) + (D / 2) * hf + 8 * s);
    } else {
      qf[s] = bf16x8_t{};
    }
  }

  const int64_t kend = (m0 + BM < Lp ? m0 + BM : Lp);
  const int nkb = (int)((kend + BN - 1) / BN);

  uint4 pk[KCH], pv[VCH];
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int e = tid + 256 * u, row = e / (D / 8), c8 = e % (D / 8);
      const int64_t j = (int64_t)kb * BN + row;
      pk[u] = j < Lp ? *reinterpret_cast<const uint4*>(Kp + k_row(j) + 8 * c8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int e = tid + 256 * u, row = e / (BN / 8), c8 = e % (BN / 8);
      const int64_t j0 = (int64_t)kb * BN + 8 * c8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j0 < Lp) {
        v = *reinterpret_cast<const uint4*>(Vp + v_base + (size_t)row * a.C + j0);
        if (j0 + 8 > Lp) {             // zero the columns at and beyond L'
          uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int x = 0; x < 8; ++x)
            if (j0 + x >= Lp) wv[x >> 1] &= (x & 1) ? 0x0000FFFFu : 0xFFFF0000u;
          v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
      }
      pv[u] = v;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int e = tid + 256 * u, row = e / (D / 8), c8 = e % (D / 8);
      *reinterpret_cast<uint4*>(&smK[buf][row * KLD + 8 * c8]) = pk[u];
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int e = tid + 256 * u, row = e / (BN / 8), c8 = e % (BN / 8);
      *reinterpret_cast<uint4*>(&smV[buf][row * VLD + 8 * c8]) = pv[u];
    }
  };

  f32x16_t o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  const int64_t wrow0 = m0 + 32 * w;        // first query row of this wave

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load_tile(kb + 1);
    const int64_t key0 = (int64_t)kb * BN;
    if (key0 <= wrow0 + 31) {               // otherwise every key of the tile is masked for this wave
      f32x16_t s[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s[t] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(&smK[buf][(32 * t + ln) * KLD + (D / 2) * hf + 8 * ks]);
          s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[t], 0, 0, 0);
        }
      }
      if (key0 + BN - 1 > wrow0) {          // diagonal tile: mask keys after the query
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t key = key0 + 32 * t + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (key > qi) s[t][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      if (mx > m_run) {
        const float alpha = __builtin_amdgcn_exp2f((m_run - mx) * sl2);
#pragma unroll
        for (int t = 0; t < DT; ++t) o[t] *= alpha;
        l_run *= alpha;
        m_run = mx;
      }
      const float mb2 = m_run * sl2;
      bf16x8_t pb[4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[t][r], sl2, -mb2));
          l_run += p;
          pb[2 * t + (r >> 3)][r & 7] = (__bf16)p;
        }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const uint16_t* vrow = &smV[buf][(32 * dt + ln) * VLD + 16 * ks + 4 * hf];
          const bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(vrow);
          const bf16x4_t hi = *reinterpret_cast<const bf16x4_t*>(vrow + 8);
          const bf16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], o[dt], 0, 0, 0);
        }
    }
    if (kb + 1 < nkb) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (qi >= Lp) return;
  const float inv_l = 1.f / l_tot;
  uint16_t* Op = static_cast<uint16_t*>(a.O);
  const uint16_t* Xp = static_cast<const uint16_t*>(a.X);
  const size_t orow = q_row(qi);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * dt + 8 * rq + 4 * hf;
      float v[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) v[x] = o[dt][4 * rq + x] * inv_l;
      if (DENSE && Xp) {
        const uint2 xv = *reinterpret_cast<const uint2*>(Xp + orow + d0);
        v[0] += bf16_to_f32((uint16_t)xv.x);
        v[1] += bf16_to_f32((uint16_t)(xv.x >> 16));
        v[2] += bf16_to_f32((uint16_t)xv.y);
        v[3] += bf16_to_f32((uint16_t)(xv.y >> 16));
      }
      uint2 ov;
      ov.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
      ov.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
      *reinterpret_cast<uint2*>(Op + orow + d0) = ov;
    }
}

// ------------------------------------------------------------------------------------------------
// f32, vector ALU
// ------------------------------------------------------------------------------------------------
template <int D, bool DENSE>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  constexpr int TPR = 4, BM = 256 / TPR, BN = 32, DPT = D / TPR;
  __shared__ float smK[BN][D + 1];
  __shared__ float smV[BN][D + 1];
  const int nmb = (int)((a.L + BM - 1) / BM);
  int h, mb;
  block_coords(nmb, a.Hq, h, mb);
  const int64_t Lp = DENSE ? a.L : (int64_t)a.Lp_dev[0];
  const int64_t m0 = (int64_t)mb * BM;
  if (m0 >= Lp) return;
  const int tid = threadIdx.x, part = tid % TPR;
  const int64_t qi = m0 + tid / TPR;
  const int g = h / (a.Hq / a.Hkv);
  const float* Qp = static_cast<const float*>(a.Q);
  const float* Kp = static_cast<const float*>(a.K);
  const float* Vp = static_cast<const float*>(a.Vt);
  auto q_row = [&](int64_t i) -> size_t { return DENSE ? ((size_t)i * a.Hq + h) * D : ((size_t)h * a.C + i) * D; };
  auto k_row = [&](int64_t j) -> size_t { return DENSE ? ((size_t)j * a.Hkv + g) * D : ((size_t)h * a.C + j) * D; };
  const size_t v_base = (size_t)(DENSE ? g : h) * D * a.C;

  float qr[DPT], acc[DPT];
#pragma unroll
  for (int u = 0; u < DPT; ++u) {
    qr[u] = qi < Lp ? Qp[q_row(qi) + part + TPR * u] : 0.f;
    acc[u] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const int64_t kend = (m0 + BM < Lp ? m0 + BM : Lp);
  for (int64_t key0 = 0; key0 < kend; key0 += BN) {
    __syncthreads();
    for (int e = tid; e < BN * D; e += 256) {
      const int r = e / D, c = e % D;
      const int64_t j = key0 + r;
      smK[r][c] = j < Lp ? Kp[k_row(j) + c] : 0.f;
      const int cv = e / BN, rv = e % BN;           // V^T is token-fastest: coalesce along keys
      smV[rv][cv] = key0 + rv < Lp ? Vp[v_base + (size_t)cv * a.C + key0 + rv] : 0.f;
    }
    __syncthreads();
    float sc[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float pdot = 0.f;
#pragma unroll
      for (int u = 0; u < DPT; ++u) pdot = fmaf(qr[u], smK[j][part + TPR * u], pdot);
      pdot += __shfl_xor(pdot, 1, kWave);
      pdot += __shfl_xor(pdot, 2, kWave);
      sc[j] = key0 + j <= qi ? pdot * a.scale : -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    if (mx > m_run) {
      const float alpha = expf(m_run - mx);
#pragma unroll
      for (int u = 0; u < DPT; ++u) acc[u] *= alpha;
      l_run *= alpha;
      m_run = mx;
    }
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float p = expf(sc[j] - m_run);
      l_run += p;
#pragma unroll
      for (int u = 0; u < DPT; ++u) acc[u] = fmaf(p, smV[j][part + TPR * u], acc[u]);
    }
  }
  if (qi >= Lp) return;
  const float inv_l = 1.f / l_run;
  float* Op = static_cast<float*>(a.O);
  const float* Xp = static_cast<const float*>(a.X);
  const size_t orow = q_row(qi);
#pragma unroll
  for (int u = 0; u < DPT; ++u) {
    float v = acc[u] * inv_l;
    if (DENSE && Xp) v += Xp[orow + part + TPR * u];
    Op[orow + part + TPR * u] = v;
  }
}

template <int D, bool DENSE>
static hipError_t run_attn(int dtype, const AttnArgs& a, hipStream_t st) {
  if (dtype == 1) {
    const int nmb = (int)((a.L + 127) / 128);
    attn_bf16_kernel<D, DENSE><<<(unsigned)(nmb * a.Hq), 256, 0, st>>>(a);
  } else {
    const int nmb = (int)((a.L + 63) / 64);
    attn_f32_kernel<D, DENSE><<<(unsigned)(nmb * a.Hq), 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, int d, bool dense, const void* Q, const void* K,
                            const void* Vt, const int32_t* Lp_dev, int64_t L, int Hq, int Hkv,
                            int64_t C, const void* X, void* O, hipStream_t st) {
  AttnArgs a{Q, K, Vt, Lp_dev, X, O, L, C, Hq, Hkv, (float)(1.0 / sqrt((double)d))};
  if (d == 128) return dense ? run_attn<128, true>(dtype, a, st) : run_attn<128, false>(dtype, a, st);
  return dense ? run_attn<64, true>(dtype, a, st) : run_attn<64, false>(dtype, a, st);
}

}  // namespace tsa

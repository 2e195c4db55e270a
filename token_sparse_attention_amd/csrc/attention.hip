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
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Raw buffer descriptor over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int D, bool DENSE>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
  constexpr int BM = 128, BN = 64;
  constexpr int KS = D / 16;          // K-steps of 16 over the head dim (score product)
  constexpr int DT = D / 32;          // 32-row tiles of O^T over the head dim
  constexpr int KLD = D + 8;          // LDS row pitch (elements) of the K tile
  constexpr int VLD = BN + 8;         // LDS row pitch of the V^T tile
  constexpr int KCPR = D / 8;         // 16-byte chunks per K row
  constexpr int KCH = BN * KCPR / 256;    // chunks per thread per K tile
  constexpr int VCH = D * (BN / 8) / 256; // chunks per thread per V^T tile
  __shared__ __attribute__((aligned(16))) uint16_t smK[2][BN * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t smV[2][D * VLD];

  const int nmb = (int)((a.L + BM - 1) / BM);
  int h, mb;
  block_coords(nmb, a.Hq, h, mb);
  const int Lp = DENSE ? (int)a.L : a.Lp_dev[0];
  const int m0 = mb * BM;
  if (m0 >= Lp) return;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int g = h / (a.Hq / a.Hkv);
  // per-head bases (bytes) and row pitches
  const uint32_t q_rs = DENSE ? a.Hq * D * 2 : D * 2;
  const uint32_t k_rs = DENSE ? a.Hkv * D * 2 : D * 2;
  const uint32_t v_rs = (uint32_t)a.C * 2;
  const char* qbase = static_cast<const char*>(a.Q) + (DENSE ? (size_t)h * D * 2 : (size_t)h * a.C * D * 2);
  const char* kbase = static_cast<const char*>(a.K) + (DENSE ? (size_t)g * D * 2 : (size_t)h * a.C * D * 2);
  const char* vbase = static_cast<const char*>(a.Vt) + (size_t)(DENSE ? g : h) * D * a.C * 2;

  const int qi = m0 + 32 * w + ln;    // this lane's query row
  bf16x8_t qf[KS];
  {
    const char* qrow = qbase + (size_t)qi * q_rs + (D / 2) * hf * 2;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = qi < Lp ? *reinterpret_cast<const bf16x8_t*>(qrow + 16 * s) : bf16x8_t{};
  }

  const int kend = m0 + BM < Lp ? m0 + BM : Lp;
  const int nkb = (kend + BN - 1) / BN;

  uint32_t voff_k[KCH], voff_v[VCH];
#pragma unroll
  for (int u = 0; u < KCH; ++u) {
    const int e = tid + 256 * u;
    voff_k[u] = (uint32_t)(e / KCPR) * k_rs + (uint32_t)(e % KCPR) * 16u;
  }
#pragma unroll
  for (int u = 0; u < VCH; ++u) {
    const int e = tid + 256 * u;
    voff_v[u] = (uint32_t)(e / (BN / 8)) * v_rs + (uint32_t)(e % (BN / 8)) * 16u;
  }

  f32x16_t o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  const int wrow0 = m0 + 32 * w;      // first query row of this wave
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // S^T tile of key tile kb from the K slot it lives in (scores of this lane's query, unmasked)
  auto scores = [&](int slot, f32x16_t (&s)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(&smK[slot][(32 * t + ln) * KLD + (D / 2) * hf + 8 * ks]);
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[t], 0, 0, 0);
      }
    }
  };

  // Software pipeline: while the softmax of tile kb runs on the vector ALU, the matrix cores already
  // form the scores of tile kb+1.  K runs one tile ahead of V in LDS (both double-buffered):
  //   iteration kb reads K(kb+1) from slot (kb+1)&1 and V(kb) from slot kb&1, then stores the
  //   prefetched K(kb+2) into slot kb&1 and V(kb+1) into slot (kb+1)&1 before the barrier.
  u32x4_t pk[KCH], pv[VCH];
  auto load_k = [&](int kb) {
    const int key0 = kb * BN;
    const int nval = Lp - key0 < BN ? Lp - key0 : BN;
    // K rows at or beyond L' fall outside the descriptor and read as zero
    const auto rk = buffer_rsrc(kbase + (size_t)key0 * k_rs, (uint32_t)(nval - 1) * k_rs + D * 2);
#pragma unroll
    for (int u = 0; u < KCH; ++u) pk[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff_k[u], 0, 0);
  };
  auto load_v = [&](int kb) {
    const int key0 = kb * BN;
    const int nval = Lp - key0 < BN ? Lp - key0 : BN;
    const auto rv = buffer_rsrc(vbase + (size_t)key0 * 2, (uint32_t)(D - 1) * v_rs + BN * 2);
#pragma unroll
    for (int u = 0; u < VCH; ++u) pv[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v[u], 0, 0);
    if (nval < BN) {                   // last tile: zero the V^T columns at and beyond L'
#pragma unroll
      for (int u = 0; u < VCH; ++u) {
        const int c0 = ((tid + 256 * u) % (BN / 8)) * 8;
#pragma unroll
        for (int x = 0; x < 8; ++x)
          if (c0 + x >= nval) pv[u][x >> 1] &= (x & 1) ? 0x0000FFFFu : 0xFFFF0000u;
      }
    }
  };
  // Key j of a tile goes to LDS row perm(j), which swaps bits 2 and 3 of j.  The score product's
  // output row 8*(r/4) + 4*hf + r%4 then holds key 16*(r/8) + 8*hf + r%8 (within each 32-key half),
  // so the 8 probabilities a lane feeds to one value-product step are 8 consecutive keys and its
  // V^T operand is one contiguous 16-byte LDS read.
  auto perm = [](int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); };
  auto store_k = [&](int slot) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int e = tid + 256 * u;
      *reinterpret_cast<u32x4_t*>(&smK[slot][perm(e / KCPR) * KLD + 8 * (e % KCPR)]) = pk[u];
    }
  };
  auto store_v = [&](int slot) {
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int e = tid + 256 * u;
      *reinterpret_cast<u32x4_t*>(&smV[slot][(e / (BN / 8)) * VLD + 8 * (e % (BN / 8))]) = pv[u];
    }
  };

  load_k(0);
  load_v(0);
  store_k(0);
  store_v(0);
  if (nkb > 1) {
    load_k(1);
    store_k(1);
  }
  __syncthreads();
  f32x16_t sc[2];
  scores(0, sc);
  __syncthreads();                    // K slot 0 is refilled at the end of iteration 0
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 2 < nkb) load_k(kb + 2);
    if (kb + 1 < nkb) load_v(kb + 1);
    const int key0 = kb * BN;
    // Diagonal (or, for this wave, fully masked) tile: keys after the query get -inf.  Every
    // wave's first tile has a visible key, so the running max is finite from tile 0 on.
    if (key0 + BN - 1 > wrow0) {
      const int rel = qi - key0 - 8 * hf;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * t + 16 * (r >> 3) + (r & 7) > rel) sc[t][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    if (mx > m_run) {
      const float alpha = __builtin_amdgcn_exp2f((m_run - mx) * sl2);
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] *= alpha;
      l_run *= alpha;
      m_run = mx;
    }
    const float mb2 = m_run * sl2;
    // The next tile's score product (2*KS MFMAs) is issued in program order interleaved with this
    // tile's exponentials, EPC elements per MFMA, so the vector ALU works while the matrix cores
    // run; then the value product (4*DT MFMAs).  LDS fragments are read PF chunks ahead; the
    // sched_barrier fences keep the compiler from regrouping the chunks.  (On the last tile the
    // next-score product reads a stale slot and is discarded.)
    constexpr int NS = 2 * KS, EPC = 32 / NS, PF = 2, NV = 4 * DT;
    const uint16_t* kslot = smK[(kb + 1) & 1];
    const uint16_t* vslot = smV[kb & 1];
    auto kfrag = [&](int f) {          // f = 2*ks + t
      return *reinterpret_cast<const bf16x8_t*>(kslot + (32 * (f & 1) + ln) * KLD + (D / 2) * hf + 8 * (f >> 1));
    };
    auto vfrag = [&](int f) {          // f = DT*ks + dt: keys 16*ks + 8*hf .. +7 of head-dim row dt
      return *reinterpret_cast<const bf16x8_t*>(vslot + (32 * (f % DT) + ln) * VLD + 16 * (f / DT) + 8 * hf);
    };
    f32x16_t sn[2] = {f32x16_t{}, f32x16_t{}};
    bf16x8_t pb[4];
    bf16x8_t kf[PF + 1], vf[PF + 1];
#pragma unroll
    for (int f = 0; f < PF; ++f) kf[f] = kfrag(f);
#pragma unroll
    for (int f = 0; f < NS; ++f) {
      if (f + PF < NS) kf[(f + PF) % (PF + 1)] = kfrag(f + PF);
      else if (f + PF - NS < PF) vf[f + PF - NS] = vfrag(f + PF - NS);
      sn[f & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[f % (PF + 1)], qf[f >> 1], sn[f & 1], 0, 0, 0);
#pragma unroll
      for (int x = 0; x < EPC; x += 2) {
        const int e = f * EPC + x, t = e >> 4, r = e & 15;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[t][r], sl2, -mb2));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[t][r + 1], sl2, -mb2));
        const bf16x2_t pp = {(__bf16)p0, (__bf16)p1};
        pb[2 * t + (r >> 3)][r & 7] = pp[0];
        pb[2 * t + (r >> 3)][(r & 7) + 1] = pp[1];
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int f = 0; f < NV; ++f) {
      if (f + PF < NV) vf[(f + PF) % (PF + 1)] = vfrag(f + PF);
      o[f % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[f % (PF + 1)], pb[f / DT], o[f % DT], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kb + 2 < nkb) store_k(kb & 1);
    if (kb + 1 < nkb) store_v((kb + 1) & 1);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t) sc[t] = sn[t];
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (qi >= Lp) return;
  const float inv_l = 1.f / l_tot;
  char* obase = static_cast<char*>(a.O) + (DENSE ? (size_t)h * D * 2 : (size_t)h * a.C * D * 2);
  uint16_t* orow = reinterpret_cast<uint16_t*>(obase + (size_t)qi * q_rs);
  const uint16_t* xrow = DENSE && a.X
      ? reinterpret_cast<const uint16_t*>(static_cast<const char*>(a.X) + (size_t)h * D * 2 + (size_t)qi * q_rs)
      : nullptr;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * dt + 8 * rq + 4 * hf;
      float v[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) v[x] = o[dt][4 * rq + x] * inv_l;
      if (xrow) {
        const uint2 xv = *reinterpret_cast<const uint2*>(xrow + d0);
        v[0] += bf16_to_f32((uint16_t)xv.x);
        v[1] += bf16_to_f32((uint16_t)(xv.x >> 16));
        v[2] += bf16_to_f32((uint16_t)xv.y);
        v[3] += bf16_to_f32((uint16_t)(xv.y >> 16));
      }
      uint2 ov;
      ov.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
      ov.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
      *reinterpret_cast<uint2*>(orow + d0) = ov;
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

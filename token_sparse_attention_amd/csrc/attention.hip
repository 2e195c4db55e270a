// Causal softmax attention, O = softmax(Q K^T / sqrt(d)) V with key j visible to query i iff j <= i
// (bxzpzcl.cn article, section 1.1; papernotes.org reading notes, "Key design 1": dense attention on
// the compressed L' x L' problem; the mask by original position reduces to j <= i because the
// selected indices are ascending).  The same kernels run the dense full-length attention that the
// sparse layers are measured against.
//
// bf16 path (gfx950 matrix cores).  A block owns 256 query rows of one head, 8 waves x 32 rows (128
// rows, 4 waves, when every sequence of the launch is short), and walks 64-key tiles of K and V^T
// staged in LDS (double-buffered, one barrier per tile).  The scores
// are formed transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows, B = Q rows), so each
// lane holds 32 scores of ONE query row: the row max is a lane-local reduction plus one exchange
// with the partner lane (l ^ 32), and the exponentials feed O^T = V^T P^T directly as the B operand
// of the second product without any shuffle.  The accumulator O^T also keeps one query per lane, so
// the online-softmax rescale is lane-local.  Softmax statistics and accumulation are float32.
// Query rows are scheduled heaviest first, and on 8-XCD parts consecutive blocks of one XCD work on
// the same head so its L2 serves the shared K/V tiles (sequences of at most 16K rows instead spread
// each XCD's blocks over all its heads, heaviest first).  Normally the 8 XCDs hold 8 heads at once;
// compressed sequences of at least 163840 rows run 4 heads at once, each striped over 2 XCDs, so the
// per-head K_hat/V_hat that are live together stay nearer the last-level cache's size (measured:
// -0.4% at 160K, -1.3% at 192K, -2.0% at 256K, but +1% at 128K, and slower for the dense kernel,
// whose 8 heads share 2 KV heads).
//
// f32 path: a vector-ALU kernel (4 lanes per query row, each holding a quarter of the head dimension,
// 64 rows per block, or 16 lanes and 16 rows when the launch is small; 32-key tiles in LDS, the next
// tile loaded into registers while the current one is used), float32 math.
#include "kern_common.h"
#include "tsa_internal.h"

namespace tsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// bf16 attention weights exp2((s - m) * scale * log2 e) stay below 2^kLazyLog2 (lazy rescale)
constexpr float kLazyLog2 = 8.0f;
// waves (of 32 query rows each) per workgroup of the dense and compressed bf16 kernels: 8 (one
// 512-thread workgroup per CU, still two waves per SIMD) so that every K/V tile brought into LDS
// serves 256 query rows; the block-sparse variant keeps 4 (its key-block lists are per 128 rows).
// Launches whose longest sequence has at most kShortMaxLen rows also take 4: twice the workgroups
// (two per CU) fill the chip better there than the shared tiles save (measured layer times, 32/8
// heads: 4K -10%, 32K -1%, 48K -0.8%, but 64K +0.3%, 96K +2.5%, 128K +1.5%).
constexpr int kAttnWaves = 8;
// Lanes per query row of the f32 kernel (its 256-thread blocks hold 256 / lanes rows).  A launch
// that would have fewer than kF32SplitBelow blocks of 64 rows leaves CUs idle and is bound by the
// longest block's walk over its key tiles: it splits each row 16 ways over 16-row blocks instead
// (measured: tiny fp32 layer, L = 1024 and 4 heads, dense 0.228 -> 0.138 ms; L = 2500 and 8 heads
// 1.01 -> 0.79 ms; but at L = 4096 and 8 heads, 512 such blocks, 0.91 -> 1.11 ms, since the 16
// lanes of a row repeat its exponentials and shuffles).  Both give the same bits: the dot product
// is summed in the same order, and a row's keys are walked in the same tiles (the extra tiles a
// 64-row block walks are fully masked for the row, adding exact zeros).
constexpr int kF32Lanes = 4, kF32SplitLanes = 16;
constexpr int64_t kF32SplitBelow = 512;

static int f32_lanes(int64_t blocks64) { return blocks64 < kF32SplitBelow ? kF32SplitLanes : kF32Lanes; }
constexpr int64_t kShortMaxLen = 49152;

// One sequence of a launch.  A launch covers up to kMaxSeg sequences packed along the token
// dimension (a varlen batch; a single sequence is the one-segment case), each with its own length
// and, in the compressed case, its own keep count L' on the device.
constexpr int kMaxSeg = 32;
struct AttnSeg {
  int64_t tok_off;      // dense: first token of the sequence in Q, K, X and Y
  int64_t cap_off;      // first row of the sequence's region in the capacity-strided tensors
  int64_t L;            // dense: sequence length
  int64_t C;            // capacity of the sequence's region (multiple of 256, >= L)
  const int32_t* Lp;    // compressed: device keep count L'
  const int32_t* idx;   // fused compressed: the sequence's selection [Hq][L] (ascending tokens)
  int32_t blk0;         // first block of the sequence in the grid
  int32_t nmb;          // query blocks per head
  int32_t hp;           // heads in flight on 8-XCD parts: 8, 4 (nmb even), or 0 (all of them)
};

// compressed sequences at least this long run 4 heads in flight
constexpr int64_t kFourHeadsMinLen = 163840;
// Sequences at most this long run every head at once (hp = 0): each XCD takes the heaviest query
// block of all its Hq / 8 heads before the next lighter ones, so the few long causal blocks of a
// short sequence start first instead of waiting behind the light blocks of the heads before them
// (measured, 32/32 and 32/8 heads: layer -6.6% at 4K, -3.9% at 8K, -0.7% at 16K; but +1-7% at
// 32K and 48K, where one head per XCD keeps more of the shared K/V tiles in its L2).
constexpr int64_t kAllHeadsMaxLen = 16384;

// Compressed: the region of sequence s in Qh, Kh, Oh is [Hq][C][d] and in Vht [Hq][d][C], starting
// at element Hq * d * cap_off.  Dense: Q, X, Y [tokens][Hq][d], K [tokens][Hkv][d] from token
// tok_off on; Vt [Hkv][d][C] (V transposed) from element Hkv * d * cap_off on.  Fused compressed
// (the gather of Q and K and the decompression folded in): Q and K are the uncompressed [tokens][Hq][d]
// and [tokens][Hkv][d] inputs, query row i and key row j of head h are Q[tok_off + idx[h][i]][h] and
// K[tok_off + idx[h][j]][g]; Vht as compressed; the output of row i goes to Y at token idx[h][i],
// plus X when given, after rounding to the storage type as the separate decompression would.
struct AttnArgs {
  const void* Q;
  const void* K;
  const void* Vt;
  const void* X;        // dense only: residual or null
  void* O;
  int Hq, Hkv;
  float scale;
  int nseg;
  // block-sparse variant (one compressed sequence): ascending kept key blocks of every query block
  const uint16_t* blist;  // [Hq][nbmax][nbmax]
  const int32_t* bcnt;    // [Hq][nbmax]
  int nbmax;
  AttnSeg seg[kMaxSeg];
};

// blockIdx -> (segment, head, query block), heavy (late) query blocks first within a head.  Every
// segment starts at a multiple of 8 blocks when Hq % 8 == 0, so blockIdx % 8 is the XCD a block runs
// on.  With hp heads in flight, XCD x works on head x % hp of the current group of hp heads, and the
// 8 / hp XCDs of one head take its query blocks in turn (hp = 8: consecutive blocks of one XCD share
// a head and walk its query blocks in order).  With hp = 0, XCD x holds heads x, x + 8, ... and takes
// query block nmb - 1 of each of them, then block nmb - 2 of each, and so on.
__device__ __forceinline__ const AttnSeg& block_coords(const AttnArgs& a, int& h, int& mb) {
  int si = 0;
  while (si + 1 < a.nseg && (int)blockIdx.x >= a.seg[si + 1].blk0) ++si;
  const AttnSeg& sg = a.seg[si];
  const int b = (int)blockIdx.x - sg.blk0, nmb = sg.nmb;
  if ((a.Hq & 7) == 0) {
    const int xcd = b & 7, slot = b >> 3, hp = sg.hp;
    if (hp == 0) {
      const int nh = a.Hq >> 3;           // heads of this XCD
      h = xcd + 8 * (slot % nh);
      mb = nmb - 1 - slot / nh;
    } else {
      const int st = 8 / hp, per = nmb / st;   // per: blocks of one head on each of its XCDs
      h = (slot / per) * hp + xcd % hp;
      mb = nmb - 1 - ((slot % per) * st + xcd / hp);
    }
  } else {
    h = b / nmb;
    mb = nmb - 1 - b % nmb;
  }
  return sg;
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

typedef __attribute__((address_space(3))) void lds_void_t;

// 0x0F70: wait until every vector-memory load of this wave (including LDS-direct loads) is done.
#define TSA_WAIT_VMEM() __builtin_amdgcn_s_waitcnt(0x0F70)

// N direct loads of 1 KiB each (16 bytes per lane) from [base, base + bytes) at voff[i] into LDS
// at lds + 1024*i; bytes past the end arrive as zeros.  The kernel's lambdas are host+device, so
// the LDS address-space cast (not valid in host code) is compiled in the device pass only;
// otherwise the host pass silently drops the kernel's launch stub.
template <int N>
__host__ __device__ __forceinline__ void dma_1k(const void* base, uint32_t bytes, char* lds, const uint32_t (&voff)[N]) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds + 1024 * i), 16, voff[i], 0, 0, 0);
#endif
}

typedef __attribute__((address_space(1))) void glb_void_t;

// N direct loads of 1 KiB each into LDS at lds + 1024*i, lane l's 16 bytes coming from its own
// 64-bit address src[i] (rows gathered through an index, beyond the reach of 32-bit buffer
// offsets).  As dma_1k, compiled in the device pass only.
template <int N>
__host__ __device__ __forceinline__ void dma_1k_gather(char* lds, const char* const (&src)[N]) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_global_load_lds((glb_void_t*)src[i], (lds_void_t*)(lds + 1024 * i), 16, 0, 0);
#endif
}

template <int D, bool DENSE, bool SPARSE, bool FUSED, int NW, bool WIDE = false>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_bf16_kernel(AttnArgs a) {
  static_assert(!SPARSE || NW == 4, "block-sparse lists are per 128 query rows");
  static_assert(!WIDE || FUSED, "64-bit row addressing is for key rows gathered through idx");
  constexpr int NT = 64 * NW;           // threads
  constexpr int BM = 32 * NW, BN = 64;
  constexpr int KS = D / 16;            // K-steps of 16 over the head dim (score product)
  constexpr int DT = D / 32;            // 32-row tiles of O^T over the head dim
  constexpr int KROW = D * 2;           // bytes per K row in LDS (no padding; XOR-swizzled)
  constexpr int KTILE = BN * KROW;
  constexpr int VROW = BN * 2;          // bytes per V^T row in LDS
  constexpr int VTILE = D * VROW;
  constexpr int KDMA = KTILE / 1024 / NW;  // 1 KiB direct loads per wave per K tile
  constexpr int VDMA = VTILE / 1024 / NW;
  constexpr int NS = 2 * KS, NV = 4 * DT, PF = 3;
  // LDS: K slots 0,1 then V slots 0,1
  __shared__ __attribute__((aligned(1024))) char smem[2 * KTILE + 2 * VTILE];
  __shared__ uint16_t klist[SPARSE ? kMaxKeyBlocks : 1];

  int h, mb;
  const AttnSeg& sg = block_coords(a, h, mb);
  const int Lp = DENSE ? (int)sg.L : sg.Lp[0];
  const int m0 = mb * BM;
  if (m0 >= Lp) return;

  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = h / (a.Hq / a.Hkv);
  const int64_t C = sg.C;
  const uint32_t q_rs = (DENSE || FUSED) ? a.Hq * D * 2 : D * 2;
  const uint32_t k_rs = DENSE ? a.Hkv * D * 2 : D * 2;
  const uint32_t v_rs = (uint32_t)C * 2;
  // element offsets of this (sequence, head) in Q/O, K and V^T
  const size_t qo_off = (DENSE || FUSED) ? ((size_t)sg.tok_off * a.Hq + h) * D
                                         : ((size_t)sg.cap_off * a.Hq + (size_t)h * C) * D;
  const size_t k_off = (DENSE || FUSED) ? ((size_t)sg.tok_off * a.Hkv + g) * D
                                        : ((size_t)sg.cap_off * a.Hq + (size_t)h * C) * D;
  const size_t v_off = (size_t)sg.cap_off * (DENSE ? a.Hkv : a.Hq) * D + (size_t)(DENSE ? g : h) * D * C;
  const char* qbase = static_cast<const char*>(a.Q) + qo_off * 2;
  const char* kbase = static_cast<const char*>(a.K) + k_off * 2;
  const char* vbase = static_cast<const char*>(a.Vt) + v_off * 2;

  const int qi = m0 + 32 * w + ln;      // this lane's query row
  // its row in Q / X / Y: qi itself, or (fused) the token it stands for
  const int64_t qrow_i = FUSED ? (qi < Lp ? (int64_t)sg.idx[(size_t)h * sg.L + qi] : 0) : qi;
  bf16x8_t qf[KS];
  {
    const char* qrow = qbase + (size_t)qrow_i * q_rs + (D / 2) * hf * 2;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = qi < Lp ? *reinterpret_cast<const bf16x8_t*>(qrow + 16 * s) : bf16x8_t{};
  }
  const int kend = m0 + BM < Lp ? m0 + BM : Lp;
  // key tiles walked: all up to the diagonal, or (block sparse) the two tiles of every listed key
  // block, the last listed block being the diagonal one (query block mb = key block mb)
  int nkb = (kend + BN - 1) / BN;
  if constexpr (SPARSE) {
    const size_t row = (size_t)h * a.nbmax + mb;
    const int nlist = a.bcnt[row];
    for (int i = threadIdx.x; i < nlist; i += NT) klist[i] = a.blist[row * a.nbmax + i];
    nkb = 2 * (nlist - 1) + (kend - m0 + BN - 1) / BN;
    __syncthreads();
  }
  // tile t of the walk -> key tile index
  auto ktile = [&](int t) -> int {
    if constexpr (SPARSE) return 2 * __builtin_amdgcn_readfirstlane((int)klist[t >> 1]) + (t & 1);
    else return t;
  };

  // Tile layouts.  K: LDS row m holds key perm(m) (bits 2 and 3 of the key swapped), 16-byte chunk
  // c of a row sits in slot c ^ kswz(m).  V^T: row = head-dim index, chunk c (keys 8c..8c+7) in
  // slot c ^ vswz(row).  Both swizzles leave every 8 and every 16 consecutive rows' reads of one
  // chunk on distinct banks, and depend only on the row's low 4 bits.
  auto perm = [](int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); };
  auto kswz = [](int m) { return KROW == 256 ? (m & 15) : ((m ^ ((m >> 3) & 1)) & 7); };
  auto vswz = [](int r) { return (r ^ ((r >> 3) & 1)) & 7; };

  // direct-load sources: the tile row and the byte offset within that row of the chunk each lane
  // brings into its 16-byte LDS slot, and (V^T) the lane's offset within the tile
  int krow[KDMA];
  uint32_t kchunk[KDMA], voffV[VDMA];
#pragma unroll
  for (int i = 0; i < KDMA; ++i) {
    const int o = (w * KDMA + i) * 1024 + 16 * lane, m = o / KROW, c = ((o % KROW) / 16) ^ kswz(m);
    krow[i] = perm(m);
    kchunk[i] = (uint32_t)c * 16u;
  }
#pragma unroll
  for (int i = 0; i < VDMA; ++i) {
    const int o = (w * VDMA + i) * 1024 + 16 * lane, r = o / VROW, c = ((o % VROW) / 16) ^ vswz(r);
    voffV[i] = (uint32_t)r * v_rs + (uint32_t)c * 16u;
  }
  // Fused: the K rows come straight from K [tokens][Hkv][d] through idx, so K_hat is never written.
  // The tokens of a tile's rows are read from idx one tile ahead of their loads, through a buffer
  // over the tile's rows that ends at row L' (the tile starts below L'): rows at or past L' read
  // token 0, a valid row whose key follows every valid query, so the causal mask gives it weight
  // exactly 0.  Row offsets are 32-bit buffer offsets while K spans less than 4 GiB from the
  // sequence's first token, 64-bit addresses (WIDE) otherwise.
  const uint32_t tok_rs = (uint32_t)a.Hkv * D * 2;   // bytes between consecutive tokens' K rows
  const int32_t* hidx = FUSED ? sg.idx + (size_t)h * sg.L : nullptr;
  const uint32_t k_extent = FUSED && !WIDE ? (uint32_t)(sg.L - 1) * tok_rs + D * 2 : 0u;
  auto ktok = [&](int kb, int (&tk)[KDMA]) {
    const int key0 = kb * BN;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(hidx + key0, (uint32_t)(Lp - key0) * 4u);
#pragma unroll
    for (int i = 0; i < KDMA; ++i) tk[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)krow[i] * 4u, 0, 0);
  };
  int tk_next[KDMA];                    // fused: tokens of the next K tile to load
  auto dma_k = [&](int kb, int slot) {
    char* dst = smem + slot * KTILE + w * KDMA * 1024;
    if constexpr (FUSED && WIDE) {
      const char* src[KDMA];
#pragma unroll
      for (int i = 0; i < KDMA; ++i) src[i] = kbase + (size_t)(uint32_t)tk_next[i] * tok_rs + kchunk[i];
      dma_1k_gather<KDMA>(dst, src);
    } else if constexpr (FUSED) {
      uint32_t voff[KDMA];
#pragma unroll
      for (int i = 0; i < KDMA; ++i) voff[i] = __umul24((uint32_t)tk_next[i], tok_rs) + kchunk[i];
      dma_1k<KDMA>(kbase, k_extent, dst, voff);
    } else {
      const int key0 = kb * BN, nval = Lp - key0 < BN ? Lp - key0 : BN;
      uint32_t voff[KDMA];
#pragma unroll
      for (int i = 0; i < KDMA; ++i) voff[i] = (uint32_t)krow[i] * k_rs + kchunk[i];
      // K rows at or beyond L' fall outside the range and arrive as zeros
      dma_1k<KDMA>(kbase + (size_t)key0 * k_rs, (uint32_t)(nval - 1) * k_rs + D * 2, dst, voff);
    }
  };
  auto dma_v = [&](int kb, int slot) {
    dma_1k<VDMA>(vbase + (size_t)kb * BN * 2, (uint32_t)(D - 1) * v_rs + BN * 2, smem + 2 * KTILE + slot * VTILE + w * VDMA * 1024, voffV);
  };
  // LDS read offsets (bytes, within a slot) of this lane's fragments; the 32-row sub-tile is an
  // immediate offset on top
  uint32_t kaddr[KS], vaddr[4];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kaddr[ks] = ln * KROW + ((((D / 16) * hf) + ks) ^ kswz(ln)) * 16;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) vaddr[ks] = ln * VROW + ((2 * ks + hf) ^ vswz(ln)) * 16;

  f32x16_t o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  const int wrow0 = m0 + 32 * w;        // first query row of this wave
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  auto scores_into = [&](const char* kslot, f32x16_t (&s)[2]) {
#pragma unroll
    for (int f = 0; f < NS; ++f) {
      const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kslot + (f & 1) * 32 * KROW + kaddr[f >> 1]);
      s[f & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[f >> 1], s[f & 1], 0, 0, 0);
    }
  };

  if constexpr (FUSED) ktok(0, tk_next);
  dma_k(ktile(0), 0);
  dma_v(ktile(0), 0);
  if (nkb > 1) {
    if constexpr (FUSED) ktok(1, tk_next);
    dma_k(ktile(1), 1);
  }
  if constexpr (FUSED) {                // tokens of K(2), consumed by tile 0
    if (nkb > 2) ktok(2, tk_next);
  }
  TSA_WAIT_VMEM();
  __syncthreads();
  f32x16_t sc[2] = {f32x16_t{}, f32x16_t{}};
  scores_into(smem, sc);
  __syncthreads();                      // K slot 0 is refilled at the start of iteration 0

  // One tile.  K runs one tile ahead of V: iteration kb reads K(kb+1) from slot (kb+1)&1 and V(kb)
  // from slot kb&1; at its start it directs K(kb+2) into slot kb&1 and V(kb+1) into slot (kb+1)&1,
  // whose previous contents every wave finished with before the last barrier.
  auto tile = [&](int kb, int P) {     // P = kb & 1, a literal at both call sites
    const char* kslot = smem + (P ^ 1) * KTILE;
    const char* vslot = smem + 2 * KTILE + P * VTILE;
    if (kb + 2 < nkb) dma_k(ktile(kb + 2), P);
    if (kb + 1 < nkb) dma_v(ktile(kb + 1), P ^ 1);
    if constexpr (FUSED) {              // tokens of K(kb + 3), waited for with this tile's loads
      if (kb + 3 < nkb) ktok(kb + 3, tk_next);
    }
    const int key0 = ktile(kb) * BN, nval = Lp - key0;
    if (nval < BN) {                    // last tile: zero the V^T columns at and beyond L'
      for (int e = tid; e < D * (BN - nval); e += NT) {
        const int r = e / (BN - nval), col = nval + e % (BN - nval);
        *reinterpret_cast<uint16_t*>(const_cast<char*>(vslot) + r * VROW + (((col >> 3) ^ vswz(r)) << 4) + (col & 7) * 2) = 0;
      }
      __syncthreads();
    }
    // diagonal (or, for this wave, fully masked) tile: keys after the query get -inf; every
    // wave's first tile has a visible key, so the running max is finite from tile 0 on
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
    // Lazy rescale: a row's reference m_run (the exponent offset) moves only when the row maximum
    // passes it by more than kLazyLog2 in the exponent, so the weights stay below 2^kLazyLog2.  When
    // any row of the wave's 32 passes, every row moves to its own maximum (alpha is exactly 1 where
    // it did not grow); the branch is wave-uniform and, past the first tiles, almost never taken.
    const bool grow = (mx - m_run) * sl2 > kLazyLog2;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - mnew) * sl2);
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] *= alpha;
      l_run *= alpha;
      m_run = mnew;
    }
    const float mb2 = m_run * sl2;
    // next tile's score MFMAs issued in program order with this tile's exponentials (EPC per MFMA),
    // then the value MFMAs; LDS fragments read PF steps ahead; fences keep the order.  (On the last
    // tile the next-score product reads a stale slot and is discarded.)
    f32x16_t sn[2] = {f32x16_t{}, f32x16_t{}};
    bf16x8_t pb[4];
    // One issue stream of NS + NV MFMA slots: slots 0..NS-1 form the next tile's scores, the rest
    // the value product.  Probability pair q (elements 2q, 2q+1) is computed in slot
    // (q * SPAN) / 16, spreading the exponentials over the first SPAN slots while every block pb[k]
    // is complete before the value MFMAs that read it.  Operand fragments come from one LDS ring,
    // read PF slots ahead.
    constexpr int NSLOT = NS + NV, SPAN = NS + NV / 2;
    bf16x8_t fr[PF + 1];
    auto frag = [&](int j) {
      return j < NS ? *reinterpret_cast<const bf16x8_t*>(kslot + (j & 1) * 32 * KROW + kaddr[j >> 1])
                    : *reinterpret_cast<const bf16x8_t*>(vslot + ((j - NS) % DT) * 32 * VROW + vaddr[(j - NS) / DT]);
    };
#pragma unroll
    for (int j = 0; j < PF; ++j) fr[j] = frag(j);
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
      if (j + PF < NSLOT) fr[(j + PF) % (PF + 1)] = frag(j + PF);
      if (j < NS) {
        sn[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j % (PF + 1)], qf[j >> 1], sn[j & 1], 0, 0, 0);
      } else {
        const int f = j - NS;
        o[f % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j % (PF + 1)], pb[f / DT], o[f % DT], 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if ((q * SPAN) / 16 != j) continue;
        const int e = 2 * q, t = e >> 4, r = e & 15;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[t][r], sl2, -mb2));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[t][r + 1], sl2, -mb2));
        const bf16x2_t pp = {(__bf16)p0, (__bf16)p1};
        pb[2 * t + (r >> 3)][r & 7] = pp[0];
        pb[2 * t + (r >> 3)][(r & 7) + 1] = pp[1];
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    TSA_WAIT_VMEM();
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t) sc[t] = sn[t];
  };
  int kb = 0;
  for (; kb + 1 < nkb; kb += 2) {
    tile(kb, 0);
    tile(kb + 1, 1);
  }
  if (kb < nkb) tile(kb, 0);

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (qi >= Lp) return;
  const float inv_l = 1.f / l_tot;
  uint16_t* orow = reinterpret_cast<uint16_t*>(static_cast<char*>(a.O) + qo_off * 2 + (size_t)qrow_i * q_rs);
  const uint16_t* xrow = (DENSE || FUSED) && a.X
      ? reinterpret_cast<const uint16_t*>(static_cast<const char*>(a.X) + qo_off * 2 + (size_t)qrow_i * q_rs)
      : nullptr;
  // the residual row first, every load before any store: Y may alias X (in place), which would
  // otherwise make each load wait for the store before it (16 round trips per wave)
  uint2 xr[DT][4];
  if (xrow) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) xr[dt][rq] = *reinterpret_cast<const uint2*>(xrow + 32 * dt + 8 * rq + 4 * hf);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * dt + 8 * rq + 4 * hf;
      float v[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) v[x] = o[dt][4 * rq + x] * inv_l;
      if (FUSED) {                      // the stored O_hat value, as decompression would read it
#pragma unroll
        for (int x = 0; x < 4; ++x) v[x] = bf16_to_f32(f32_to_bf16(v[x]));
      }
      if (xrow) {
        const uint2 xv = xr[dt][rq];
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
template <int D, bool DENSE, bool SPARSE, int TPR>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  // TPR threads per query row, each owning DPT consecutive head-dim elements (16-byte LDS reads);
  // 32-key tiles of K and V (rows, padded to a 16-byte multiple) in LDS, the next tile's elements
  // loaded into registers while the current one is used
  constexpr int BM = 256 / TPR, BN = 32, DPT = D / TPR, ROW = D + 4;
  constexpr int CH = D / kF32SplitLanes, NCH = DPT / CH;   // dot-product partials: length, per lane
  constexpr int NV4 = BN * D / 4 / 256;     // 16-byte pieces of a K (or V) tile per thread
  __shared__ __attribute__((aligned(16))) float smK[BN][ROW];
  __shared__ __attribute__((aligned(16))) float smV[BN][ROW];
  __shared__ uint16_t klist[SPARSE ? kMaxKeyBlocks : 1];
  int h, mb;
  const AttnSeg& sg = block_coords(a, h, mb);
  const int64_t Lp = DENSE ? sg.L : (int64_t)sg.Lp[0];
  const int64_t m0 = (int64_t)mb * BM;
  if (m0 >= Lp) return;
  const int tid = threadIdx.x, part = tid % TPR, d0 = part * DPT;
  const int64_t qi = m0 + tid / TPR;
  const int g = h / (a.Hq / a.Hkv);
  const int64_t C = sg.C;
  const float* Qp = static_cast<const float*>(a.Q);
  const float* Kp = static_cast<const float*>(a.K);
  const float* Vp = static_cast<const float*>(a.Vt);
  auto q_row = [&](int64_t i) -> size_t {
    return DENSE ? ((size_t)(sg.tok_off + i) * a.Hq + h) * D : ((size_t)sg.cap_off * a.Hq + (size_t)h * C + i) * D;
  };
  auto k_row = [&](int64_t j) -> size_t {
    return DENSE ? ((size_t)(sg.tok_off + j) * a.Hkv + g) * D : ((size_t)sg.cap_off * a.Hq + (size_t)h * C + j) * D;
  };
  const size_t v_base = (size_t)sg.cap_off * (DENSE ? a.Hkv : a.Hq) * D + (size_t)(DENSE ? g : h) * D * C;

  float qr[DPT], acc[DPT];
  {
    const float4* q4 = reinterpret_cast<const float4*>(Qp + q_row(qi < Lp ? qi : m0) + d0);
#pragma unroll
    for (int u = 0; u < DPT / 4; ++u) {
      const float4 v = qi < Lp ? q4[u] : make_float4(0.f, 0.f, 0.f, 0.f);
      qr[4 * u] = v.x; qr[4 * u + 1] = v.y; qr[4 * u + 2] = v.z; qr[4 * u + 3] = v.w;
    }
  }
#pragma unroll
  for (int u = 0; u < DPT; ++u) acc[u] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;     // scores kept in log2 units
  const int64_t kend = (m0 + BM < Lp ? m0 + BM : Lp);
  // key ranges walked: [0, kend), or (block sparse) every listed key block of this rows' query block
  int nrange = 1;
  if constexpr (SPARSE) {
    const size_t row = (size_t)h * a.nbmax + m0 / kBlock;
    nrange = a.bcnt[row];
    for (int i = threadIdx.x; i < nrange; i += 256) klist[i] = a.blist[row * a.nbmax + i];
    __syncthreads();
  }
  auto range_begin = [&](int rg) -> int64_t { return SPARSE ? (int64_t)klist[rg] * kBlock : 0; };
  auto range_end = [&](int rg) -> int64_t {
    const int64_t b = range_begin(rg);
    return SPARSE ? (b + kBlock < kend ? b + kBlock : kend) : kend;
  };
  // this thread's pieces of the tile at key0: K piece e -> key row e / (D/4), columns 4 (e % (D/4));
  // V^T piece e -> head-dim row e / (BN/4), keys 4 (e % (BN/4)).  Keys at or past L' read as zeros.
  float4 kv[NV4], vv[NV4];
  auto load_tile = [&](int64_t key0) {
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int e = tid + 256 * i;
      const int r = e / (D / 4), c4 = e % (D / 4);
      kv[i] = key0 + r < Lp ? *reinterpret_cast<const float4*>(Kp + k_row(key0 + r) + 4 * c4)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
      const int cv = e / (BN / 4), k4 = e % (BN / 4);
      const int64_t j = key0 + 4 * k4;   // V^T rows have capacity C >= key0 + BN: the load stays inside
      float4 v = *reinterpret_cast<const float4*>(Vp + v_base + (size_t)cv * C + j);
      if (j + 3 >= Lp) {
        v.x = j < Lp ? v.x : 0.f;
        v.y = j + 1 < Lp ? v.y : 0.f;
        v.z = j + 2 < Lp ? v.z : 0.f;
        v.w = j + 3 < Lp ? v.w : 0.f;
      }
      vv[i] = v;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int e = tid + 256 * i;
      const int r = e / (D / 4), c4 = e % (D / 4);
      *reinterpret_cast<float4*>(&smK[r][4 * c4]) = kv[i];
      const int cv = e / (BN / 4), k4 = e % (BN / 4);
      smV[4 * k4][cv] = vv[i].x;
      smV[4 * k4 + 1][cv] = vv[i].y;
      smV[4 * k4 + 2][cv] = vv[i].z;
      smV[4 * k4 + 3][cv] = vv[i].w;
    }
  };
  int rg = 0;
  int64_t key0 = range_begin(0);
  load_tile(key0);
  while (true) {
    __syncthreads();                    // every thread is done with the previous tile
    store_tile();
    __syncthreads();
    // the next tile of the walk, loaded while this one is used
    int rn = rg;
    int64_t kn = key0 + BN;
    if (kn >= range_end(rg)) {
      rn = rg + 1;
      kn = rn < nrange ? range_begin(rn) : -1;
    }
    if (kn >= 0) load_tile(kn);
    float sc[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      // the dot product in one fixed order for either lane count: D / 16 consecutive products per
      // partial sum, then a pairwise tree over the 16 partials (inside the lane, then across lanes)
      float part[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        part[c] = 0.f;
#pragma unroll
        for (int u = 0; u < CH / 4; ++u) {
          const int e = c * CH + 4 * u;
          const float4 k4 = *reinterpret_cast<const float4*>(&smK[j][d0 + e]);
          part[c] = fmaf(qr[e], k4.x, part[c]);
          part[c] = fmaf(qr[e + 1], k4.y, part[c]);
          part[c] = fmaf(qr[e + 2], k4.z, part[c]);
          part[c] = fmaf(qr[e + 3], k4.w, part[c]);
        }
      }
#pragma unroll
      for (int w = 1; w < NCH; w <<= 1)
#pragma unroll
        for (int c = 0; c < NCH; c += 2 * w) part[c] += part[c + w];
      float pdot = part[0];
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) pdot += __shfl_xor(pdot, o, kWave);
      sc[j] = key0 + j <= qi ? pdot * sl2 : -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    if (mx > m_run) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mx);
#pragma unroll
      for (int u = 0; u < DPT; ++u) acc[u] *= alpha;
      l_run *= alpha;
      m_run = mx;
    }
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float p = __builtin_amdgcn_exp2f(sc[j] - m_run);
      l_run += p;
#pragma unroll
      for (int u = 0; u < DPT / 4; ++u) {
        const float4 v4 = *reinterpret_cast<const float4*>(&smV[j][d0 + 4 * u]);
        acc[4 * u] = fmaf(p, v4.x, acc[4 * u]);
        acc[4 * u + 1] = fmaf(p, v4.y, acc[4 * u + 1]);
        acc[4 * u + 2] = fmaf(p, v4.z, acc[4 * u + 2]);
        acc[4 * u + 3] = fmaf(p, v4.w, acc[4 * u + 3]);
      }
    }
    if (kn < 0) break;
    rg = rn;
    key0 = kn;
  }
  if (qi >= Lp) return;
  const float inv_l = 1.f / l_run;
  float* Op = static_cast<float*>(a.O);
  const float* Xp = static_cast<const float*>(a.X);
  const size_t orow = q_row(qi) + d0;
  float4 xr[DPT / 4];                   // residual loads before any store (Y may alias X)
#pragma unroll
  for (int u = 0; u < DPT / 4; ++u)
    xr[u] = DENSE && Xp ? *reinterpret_cast<const float4*>(Xp + orow + 4 * u) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < DPT / 4; ++u) {
    float4 v = make_float4(acc[4 * u] * inv_l, acc[4 * u + 1] * inv_l, acc[4 * u + 2] * inv_l, acc[4 * u + 3] * inv_l);
    if (DENSE && Xp) { v.x += xr[u].x; v.y += xr[u].y; v.z += xr[u].z; v.w += xr[u].w; }
    *reinterpret_cast<float4*>(Op + orow + 4 * u) = v;
  }
}

template <int D, bool DENSE, bool SPARSE = false, bool FUSED = false>
static hipError_t run_attn(int dtype, const AttnArgs& a, int nblocks, hipStream_t st, int nw = kAttnWaves,
                           bool wide = false, int f32lanes = kF32Lanes) {
  if (dtype == 1) {
    if constexpr (SPARSE) {
      attn_bf16_kernel<D, DENSE, SPARSE, FUSED, 4><<<(unsigned)nblocks, 256, 0, st>>>(a);
    } else if constexpr (FUSED) {
      // key rows gathered through idx: 32-bit buffer offsets while K spans less than 4 GiB
      if (wide) {
        if (nw == 4) attn_bf16_kernel<D, false, false, true, 4, true><<<(unsigned)nblocks, 256, 0, st>>>(a);
        else attn_bf16_kernel<D, false, false, true, kAttnWaves, true><<<(unsigned)nblocks, 64 * kAttnWaves, 0, st>>>(a);
      } else {
        if (nw == 4) attn_bf16_kernel<D, false, false, true, 4><<<(unsigned)nblocks, 256, 0, st>>>(a);
        else attn_bf16_kernel<D, false, false, true, kAttnWaves><<<(unsigned)nblocks, 64 * kAttnWaves, 0, st>>>(a);
      }
    } else {
      if (nw == 4) attn_bf16_kernel<D, DENSE, SPARSE, FUSED, 4><<<(unsigned)nblocks, 256, 0, st>>>(a);
      else attn_bf16_kernel<D, DENSE, SPARSE, FUSED, kAttnWaves><<<(unsigned)nblocks, 64 * kAttnWaves, 0, st>>>(a);
    }
  } else if (!FUSED) {
    if (f32lanes == kF32SplitLanes) attn_f32_kernel<D, DENSE, SPARSE, kF32SplitLanes><<<(unsigned)nblocks, 256, 0, st>>>(a);
    else attn_f32_kernel<D, DENSE, SPARSE, kF32Lanes><<<(unsigned)nblocks, 256, 0, st>>>(a);
  }
  else
    return hipErrorInvalidValue;         // the fused layer is bf16 only
  return hipGetLastError();
}

hipError_t launch_attention_varlen(int dtype, int d, bool dense, const void* Q, const void* K, const void* Vt,
                                   int nseq, const AttnSeqDesc* seqs, int Hq, int Hkv, const void* X, void* O,
                                   hipStream_t st, bool fused) {
  AttnArgs a{};
  a.Q = Q; a.K = K; a.Vt = Vt; a.X = X; a.O = O;
  a.Hq = Hq; a.Hkv = Hkv; a.scale = (float)(1.0 / sqrt((double)d));
  for (int first = 0; first < nseq; first += kMaxSeg) {
    a.nseg = nseq - first < kMaxSeg ? nseq - first : kMaxSeg;
    int64_t longest = 0;
    for (int i = 0; i < a.nseg; ++i) longest = seqs[first + i].L > longest ? seqs[first + i].L : longest;
    const int nw = longest <= kShortMaxLen ? 4 : kAttnWaves;
    // a sequence's K rows span L * Hkv * d * 2 bytes from its first token
    const bool wide = (uint64_t)longest * (uint64_t)Hkv * (uint64_t)d * 2u >= (uint64_t(1) << 32);
    int64_t blocks64 = 0;                          // f32: blocks of 64 rows over the launch
    for (int i = 0; i < a.nseg; ++i) blocks64 += (seqs[first + i].L + 63) / 64 * Hq;
    const int lanes = f32_lanes(blocks64);
    const int bm = dtype == 1 ? 32 * nw : 256 / lanes;      // query rows per block
    int nblocks = 0;
    for (int i = 0; i < a.nseg; ++i) {
      const AttnSeqDesc& q = seqs[first + i];
      AttnSeg& g = a.seg[i];
      g.tok_off = q.tok_off; g.cap_off = q.cap_off; g.L = q.L; g.C = q.C; g.Lp = q.Lp_dev; g.idx = q.idx;
      g.blk0 = nblocks;
      g.nmb = (int)((q.L + bm - 1) / bm);
      g.hp = q.L <= kAllHeadsMaxLen ? 0 : !dense && dtype == 1 && q.L >= kFourHeadsMinLen && g.nmb % 2 == 0 ? 4 : 8;
      nblocks += g.nmb * Hq;
    }
    hipError_t e;
    if (fused)
      e = d == 128 ? run_attn<128, false, false, true>(dtype, a, nblocks, st, nw, wide)
                   : run_attn<64, false, false, true>(dtype, a, nblocks, st, nw, wide);
    else if (d == 128)
      e = dense ? run_attn<128, true>(dtype, a, nblocks, st, nw, false, lanes)
                : run_attn<128, false>(dtype, a, nblocks, st, nw, false, lanes);
    else
      e = dense ? run_attn<64, true>(dtype, a, nblocks, st, nw, false, lanes)
                : run_attn<64, false>(dtype, a, nblocks, st, nw, false, lanes);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attention_block_sparse(int dtype, int d, const void* Qh, const void* Kh, const void* Vht,
                                         const int32_t* Lp_dev, int64_t L, int Hq, int Hkv, int64_t C,
                                         const uint16_t* list, const int32_t* count, void* Oh, hipStream_t st) {
  const int lanes = f32_lanes((L + 63) / 64 * Hq);
  const int bm = dtype == 1 ? 128 : 256 / lanes;
  AttnArgs a{};
  a.Q = Qh; a.K = Kh; a.Vt = Vht; a.X = nullptr; a.O = Oh;
  a.Hq = Hq; a.Hkv = Hkv; a.scale = (float)(1.0 / sqrt((double)d));
  a.blist = list; a.bcnt = count; a.nbmax = (int)(C / kBlock);
  a.nseg = 1;
  a.seg[0] = AttnSeg{0, 0, L, C, Lp_dev, nullptr, 0, (int)((L + bm - 1) / bm), 8};
  const int nblocks = a.seg[0].nmb * Hq;
  return d == 128 ? run_attn<128, false, true>(dtype, a, nblocks, st, kAttnWaves, false, lanes)
                  : run_attn<64, false, true>(dtype, a, nblocks, st, kAttnWaves, false, lanes);
}

hipError_t launch_attention(int dtype, int d, bool dense, const void* Q, const void* K,
                            const void* Vt, const int32_t* Lp_dev, int64_t L, int Hq, int Hkv,
                            int64_t C, const void* X, void* O, hipStream_t st) {
  const AttnSeqDesc one{0, 0, L, C, Lp_dev, nullptr};
  return launch_attention_varlen(dtype, d, dense, Q, K, Vt, 1, &one, Hq, Hkv, X, O, st, false);
}

}  // namespace tsa

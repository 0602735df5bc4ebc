// Fine branch of VSA-H3: block-sparse flash attention on bf16 MFMA, with the
// gate-and-combine epilogue and the scatter back to packed order fused in.
//
// What is computed (FastH3 4-step Preview (VSA, data-free), section "Video
// Sparse Attention is not optional here"; FastH3 NVFP4 on RTX PRO 6000,
// "Block-sparse FP4 attention for VSA tiles"): a video query tile attends to
// every prefix key tile plus its selected video key tiles; a prefix query
// tile attends to all tiles; pad keys of partial tiles are masked.  Then
//     out[r] = o[r] + gate[r] * c[tile(r)]
// written at the token's packed row ("Model integration": the output is
// gathered back to packed order; the per-token gate multiplies the small
// per-tile compression output, "What was tried and not shipped").
//
// Design (gfx950, wave64):
//   - one block of 2 waves per (head, query tile); wave w owns query rows
//     32w..32w+31 of the 64-row tile, gathered straight from the packed
//     [L][H][D] input through the tile's slot table into MFMA operand
//     registers;
//   - the visit list is ascending (prefix tiles 0..P-1, then the selected
//     video tiles), so every row starts from a finite running max;
//   - K [64][D] and V^T [D][64] of the current key tile sit in two LDS
//     regions filled by direct global->LDS loads (global_load_lds_dwordx4,
//     no register staging).  K(t+1) is requested as soon as S(t) is computed
//     and V(t+1) as soon as P(t).V(t) is done, so each load overlaps about
//     half an iteration, and four blocks per CU cover the rest;
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys are the M dimension, so
//     each lane holds one query column), online softmax in fp32 via exp2 with
//     the 1/sqrt(D) scale folded into log2 units; the running max is raised
//     only when a tile exceeds it by more than 2^8 (probabilities stay below
//     256, exact enough for bf16 P and fp32 sums), so the O rescale is rare;
//   - O^T += V^T P^T on the same MFMA: P^T is consumed straight from the S^T
//     accumulator layout; V^T is stored with the keys of each 16-key group
//     permuted (0-3, 8-11, 4-7, 12-15) so that each lane's 8 keys are one
//     16-byte LDS read;
//   - LDS rows use XOR-swizzled 16-byte chunks, bank-conflict free for the
//     MFMA operand reads;
//   - partial key tiles skip their empty 16-key chunks entirely;
//   - blocks are mapped to the 8 XCDs so that each XCD works through its own
//     heads, head by head: the 32 CUs of an XCD sweep the same head's K/V;
//   - long key lists are cut into key chunks, one launch each: every query
//     tile of a head visits its tiles of the current chunk at about the same
//     time, so those reads mostly hit the L2 (and the Infinity Cache) instead
//     of HBM.  Each wave's running state (O^T, running max, its lanes' row
//     sums) is stored in fp32 at the end of a launch and loaded at the start
//     of the next; visit order and arithmetic are those of a single launch,
//     so the result is the same bit for bit.
#include "device.hpp"
#include "kernels.hpp"

namespace vsa {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

template <typename T>
struct IoOps;

template <>
struct IoOps<uint16_t> {  // bf16 I/O
  static __device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
  }
  static __device__ __forceinline__ void load4(const uint16_t* p, float v[4]) {
    const u32x2 u = *reinterpret_cast<const u32x2*>(p);
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xffff0000u);
  }
  static __device__ __forceinline__ void store4(uint16_t* p, const float v[4]) {
    u32x2 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2*>(p) = u;
  }
};

template <>
struct IoOps<float> {  // fp32 I/O; the MFMA operands are rounded to bf16
  static __device__ __forceinline__ bf16x8 load8(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    u32x4 u;
    u.x = pack_bf16x2(a.x, a.y);
    u.y = pack_bf16x2(a.z, a.w);
    u.z = pack_bf16x2(b.x, b.y);
    u.w = pack_bf16x2(b.z, b.w);
    return __builtin_bit_cast(bf16x8, u);
  }
  static __device__ __forceinline__ void load4(const float* p, float v[4]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
  static __device__ __forceinline__ void store4(float* p, const float v[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// (head, query tile) of block b in a single-launch forward.  With heads
// divisible by 8, XCD x (blocks b = x mod 8) owns heads x, x+8, ...; inside
// an XCD, the prefix items of its heads come first, then the video items
// head by head.
__device__ __forceinline__ void decode_item(int b, int H, int P, int NV, int& h, int& i) {
  if ((H & 7) == 0) {
    const int x = b & 7;
    int s = b >> 3;
    const int nh = H >> 3;
    int k;
    if (s < nh * P) {
      k = s / P;
      i = s - k * P;
    } else {
      s -= nh * P;
      k = s / NV;
      i = P + (s - k * NV);
    }
    h = x + 8 * k;
  } else {
    if (b < H * P) {
      h = b / P;
      i = b - h * P;
    } else {
      const int s = b - H * P;
      h = s / NV;
      i = P + (s - h * NV);
    }
  }
}

// (head, query tile) of block b in one key-chunk launch: XCD x works through
// its heads x, x+8, ... one at a time, every query tile of a head in turn, so
// the XCD's L2 only has to hold the current head's chunk of K and V.
__device__ __forceinline__ void decode_item_chunked(int b, int H, int Nt, int& h, int& i) {
  if ((H & 7) == 0) {
    const int s = b >> 3;
    const int k = s / Nt;
    i = s - k * Nt;
    h = (b & 7) + 8 * k;
  } else {
    h = b / Nt;
    i = b - h * Nt;
  }
}

// s_waitcnt immediate that waits for vmcnt <= N (N < 16, OR-ed in) and leaves
// expcnt and lgkmcnt unconstrained.  The builtin, unlike inline asm, is seen
// by the compiler's own wait-count pass, which then does not add a
// conservative vmcnt(0) in front of the LDS reads.
constexpr int kWaitVm = 0x0F70;

// XOR swizzle of the 16-byte chunk index inside an LDS row, conflict free
// for the operand reads of 8 (32 banks) or 16 (64 banks) consecutive rows.
__device__ __forceinline__ int swz128(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz256(int row) { return row & 15; }

// Swizzle of the 16-byte chunks of one key row in LDS (physical chunk =
// logical chunk ^ kswz(row)): conflict-free MFMA operand reads for 256-byte
// (bf16, D 128), 128-byte (bf16 D 64, or FP8 D 128) and 64-byte rows.
template <int ROW_BYTES, bool FP8ROWS>
__device__ __forceinline__ int kswz(int row) {
  if (FP8ROWS) return ROW_BYTES == 128 ? (row >> 1) & 7 : (row >> 2) & 3;
  return ROW_BYTES == 256 ? swz256(row) : swz128(row);
}

// Eight input values as fp32.
template <typename TIO>
__device__ __forceinline__ void load_f32x8(const TIO* p, float v[8]) {
  IoOps<TIO>::load4(p, v);
  IoOps<TIO>::load4(p + 4, v + 4);
}

template <typename TIO, int D, bool QK8>
__global__ __launch_bounds__(128, 2) void fine_attn_kernel(FineArgs a,
                                                          const int32_t* __restrict__ valid,
                                                          const int32_t* __restrict__ sel,
                                                          const int32_t* __restrict__ choff,
                                                          float* __restrict__ state, int chunk) {
  constexpr int TILE_BYTES = 64 * D * 2;       // one bf16 K (or V^T) tile
  constexpr int LOADS = TILE_BYTES / 1024 / 2; // 1 KB DMA loads per wave per V^T tile
  // K rows: bf16 (2D bytes), or OCP FP8 E4M3 codes (D bytes) with QK8.
  constexpr int KROWB = QK8 ? D : 2 * D;
  constexpr int KROW = KROWB / 16;             // 16-byte chunks per K row
  constexpr int K_TILE = 64 * KROWB;
  constexpr int KLOADS = K_TILE / 1024 / 2;    // 1 KB DMA loads per wave per K tile
  constexpr int NK64 = D / 64;                 // FP8 MFMA steps of 64 channels
  constexpr int NCK = D / 16;                  // QK contraction steps
  constexpr int NB = D / 32;                   // O^T blocks of 32 channels
  // With QK8 the K tile is followed by 1 KB per wave for the per-key scales
  // (the first 128 bytes of each hold the wave's 32 scales).
  __shared__ __attribute__((aligned(1024))) char lds_k[QK8 ? K_TILE + 2048 : K_TILE];
  __shared__ __attribute__((aligned(1024))) char lds_v[TILE_BYTES];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int lane = tid & 63;
  const int hl = lane >> 5;      // lane half: k-slots 8*hl..8*hl+7 of each MFMA
  const int l32 = lane & 31;
  const int H = a.H, Nt = a.Nt, P = a.P, NV = a.NV, topk = a.topk;

  int hd, i;
  if (a.nchunks > 1)
    decode_item_chunked(blockIdx.x, H, Nt, hd, i);
  else
    decode_item(blockIdx.x, H, P, NV, hd, i);

  // Visit list: prefix tiles 0..P-1 then the selected video tiles (all
  // tiles for a prefix query tile), ascending.  This launch covers the part
  // of it with ids in [chunk * chunk_tiles, (chunk + 1) * chunk_tiles).
  const bool dense = i < P;
  int beg = 0, end = dense ? Nt : P + topk;
  if (a.nchunks > 1) {
    const int lo = chunk * a.chunk_tiles;
    const int hi = min(lo + a.chunk_tiles, Nt);
    if (dense) {
      beg = lo;
      end = hi;
    } else {
      const int32_t* co = choff + (static_cast<size_t>(hd) * NV + (i - P)) * (a.nchunks + 1) + chunk;
      beg = min(lo, P) + co[0];
      end = min(hi, P) + co[1];
    }
  }
  const bool first = chunk == 0;
  const bool last = chunk == a.nchunks - 1;
  // Nothing to add, and the running state stays where it is.
  if (beg >= end && !first && !last) return;

  // Query fragment: B operand of S^T = K Q^T (column = query, k = channel).
  const TIO* q = static_cast<const TIO*>(a.q);
  const int pr = a.perm[static_cast<size_t>(i) * 64 + 32 * w + l32];
  // A wave whose 32 query rows are all pad slots (the second half of a tile
  // with at most 32 valid tokens) only takes part in the loads and barriers.
  const bool active = 32 * w < valid[i];
  // Rows come from the packed input, or from the tile-ordered copy that the
  // gather wrote after QK-norm and RoPE (pad rows are zero there).
  bf16x8 qf[QK8 ? 1 : NCK];
  // QK8: this lane's 64 channels 64m + 32hl + 0..31 (m < NK64) of its query
  // row as E4M3 codes of x * (448 / amax) (amax over the whole row), and the
  // row's dequantisation scale amax / 448 (zero rows: zero codes and scale).
  i32x8 qf8[QK8 ? NK64 : 1];
  float qsc = 1.0f;
  if constexpr (QK8) {
    float x[NK64][32];
#pragma unroll
    for (int m = 0; m < NK64; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 64 * m + 32 * hl + 8 * g;
        if (a.qt) {
          load_f32x8(a.qt + ((static_cast<size_t>(hd) * Nt + i) * 64 + 32 * w + l32) * D + d0,
                     &x[m][8 * g]);
        } else if (pr >= 0) {
          load_f32x8(q + (static_cast<size_t>(pr) * H + hd) * D + d0, &x[m][8 * g]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[m][8 * g + e] = 0.0f;
        }
      }
    float amax = 0.0f;
#pragma unroll
    for (int m = 0; m < NK64; ++m)
#pragma unroll
      for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(x[m][e]));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float inv = amax > 0.0f ? __fdiv_rn(448.0f, amax) : 0.0f;
    qsc = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 0.0f;
#pragma unroll
    for (int m = 0; m < NK64; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t u = __builtin_amdgcn_cvt_pk_fp8_f32(x[m][4 * j] * inv, x[m][4 * j + 1] * inv, 0,
                                                     false);
        u = __builtin_amdgcn_cvt_pk_fp8_f32(x[m][4 * j + 2] * inv, x[m][4 * j + 3] * inv, u,
                                            true);
        qf8[m][j] = static_cast<int>(u);
      }
  } else if (a.qt) {
    const uint16_t* qrow = a.qt + ((static_cast<size_t>(hd) * Nt + i) * 64 + 32 * w + l32) * D;
#pragma unroll
    for (int c = 0; c < NCK; ++c) qf[c] = IoOps<uint16_t>::load8(qrow + 16 * c + 8 * hl);
  } else {
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
      if (pr >= 0)
        qf[c] = IoOps<TIO>::load8(q + (static_cast<size_t>(pr) * H + hd) * D + 16 * c + 8 * hl);
      else
        qf[c] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  const int32_t* sl = sel + (dense ? 0 : (static_cast<size_t>(hd) * NV + (i - P)) * topk);
  const char* kth = (QK8 ? reinterpret_cast<const char*>(a.kt8) : reinterpret_cast<const char*>(a.kt)) +
                    static_cast<size_t>(hd) * Nt * K_TILE;
  const char* ksh =
      QK8 ? reinterpret_cast<const char*>(a.kscale) + static_cast<size_t>(hd) * Nt * 256 : nullptr;
  const char* vth = reinterpret_cast<const char*>(a.vt) + static_cast<size_t>(hd) * Nt * TILE_BYTES;
  // Listed ids are clamped into [0, Nt): a corrupt list can give a wrong
  // result but never an out-of-bounds read.
  auto tile_at = [&](int it) -> int {
    const int t = (dense || it < P) ? it : sl[it - P];
    return min(max(t, 0), Nt - 1);
  };

  // Per-lane source offsets of the DMA loads: the lane that fills LDS chunk p
  // fetches the global chunk that the swizzle places there.  The swizzle term
  // repeats every KREP (VREP) loads, so a few base offsets plus a constant
  // stride cover all of them.  Wave w fills K rows 32w..32w+31.
  constexpr int KROWS_PER_LOAD = 1024 / KROWB;
  constexpr int KREP = 16 / KROWS_PER_LOAD;                // the K swizzle repeats every 16 rows
  constexpr int KSTEP = 16 * KROWB;
  constexpr int VREP = 2;
  constexpr int VSTEP = 16 * 128;
  int kbase[KREP], vbase[VREP], vmin[VREP];
#pragma unroll
  for (int e = 0; e < KREP; ++e) {
    const int p = (w * KLOADS + e) * 64 + lane;
    const int key = p / KROW, pc = p % KROW;
    kbase[e] = key * KROWB + ((pc ^ kswz<KROWB, QK8>(key)) << 4);
  }
#pragma unroll
  for (int e = 0; e < VREP; ++e) {
    const int p = (w * LOADS + e) * 64 + lane;
    const int d = p >> 3, pv = p & 7;
    const int lc = pv ^ swz128(d);               // logical chunk: positions 8lc..8lc+7
    vbase[e] = d * 128 + (lc << 4);
    // The P.V step reads whole 16-key groups (pad slots included, which are
    // zero in memory): a chunk is needed iff its group holds a valid key.
    vmin[e] = 16 * (lc >> 1);
  }
// Block barrier without the workgroup fence of __syncthreads(): the fence
// would also wait for every outstanding global->LDS load, which this loop
// keeps in flight on purpose.  LDS reads are drained first (so no wave's
// pending read can race the next DMA into that region) and DMA completion is
// awaited explicitly (kWaitVm) before the barriers that publish a tile.  The
// memory clobber keeps the compiler from moving memory accesses across it.
#define VSA_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")
// K: only the loads whose rows hold valid keys (a count uniform per wave).
// Scores of rows not loaded are never used: empty 16-key chunks are skipped
// and pad keys inside a chunk are overwritten with -inf.
// V^T: every load is issued, so that its count stays fixed, but lanes whose
// chunk lies in a 16-key group without valid keys stay idle; P.V never reads
// those groups, so their stale contents (possibly non-finite) cannot leak.
// With QK8 every wave also requests its 32 per-key scales (one load, lanes
// 8..63 repeating lanes 0..7), so a K group is NKL + 1 loads.
#define VSA_LOAD_K(J, NKL)                                                                    \
  {                                                                                            \
    const char* src_ = kth + static_cast<size_t>(J) * K_TILE;                                  \
    _Pragma("unroll") for (int e = 0; e < KLOADS; ++e) {                                       \
      if (e < (NKL))                                                                           \
        __builtin_amdgcn_global_load_lds(                                                      \
            (gbl_void*)(src_ + (e / KREP) * KSTEP + kbase[e % KREP]),                          \
            (lds_void*)(lds_k + (w * KLOADS + e) * 1024), 16, 0, 0);                           \
    }                                                                                          \
    if (QK8)                                                                                   \
      __builtin_amdgcn_global_load_lds(                                                        \
          (gbl_void*)(ksh + static_cast<size_t>(J) * 256 + 128 * w + 16 * (lane & 7)),         \
          (lds_void*)(lds_k + K_TILE + 1024 * w), 16, 0, 0);                                   \
  }
#define VSA_LOAD_V(SRC, NJ)                                                                   \
  _Pragma("unroll") for (int e = 0; e < LOADS; ++e) {                                          \
    if (vmin[e % VREP] < (NJ))                                                                 \
      __builtin_amdgcn_global_load_lds(                                                        \
          (gbl_void*)((SRC) + (e / VREP) * VSTEP + vbase[e % VREP]),                           \
          (lds_void*)(lds_v + (w * LOADS + e) * 1024), 16, 0, 0);                              \
  }
  // K tile loads this wave issues for a tile with n valid keys.
  auto k_loads = [&](int n) -> int {
    const int rows = n - 32 * w;
    return rows <= 0 ? 0 : min(KLOADS, (rows + KROWS_PER_LOAD - 1) / KROWS_PER_LOAD);
  };

  // Per-lane LDS read offsets of the MFMA operands.
  const int kswz_r = kswz<KROWB, QK8>(l32);
  const int vswz_r = swz128(l32);

  // Logit scale in log2 units; with QK8 it also carries the query row's
  // dequantisation scale (the key scales are applied to S below).
  const float scale_log2 = (1.4426950408889634f / sqrtf(static_cast<float>(D))) * qsc;
  // Running state of this wave's 32 rows: O^T accumulators, running max (in
  // log2 units) and this lane's partial row sum.  Between key-chunk launches
  // it lives in `state`, one 16-byte quad per lane per 4 words, coalesced:
  // quads 0..4NB-1 hold oacc, quad 4NB holds (m_run, l_run, 0, 0).
  f32x16 oacc[NB];
  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x4* wstate = reinterpret_cast<f32x4*>(state) +
                  ((static_cast<size_t>(hd) * Nt + i) * 2 + w) * (4 * NB + 1) * 64 + lane;
  if (!first && active) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const f32x4 t = __builtin_nontemporal_load(wstate + (4 * n + k4) * 64);
        oacc[n][4 * k4 + 0] = t.x;
        oacc[n][4 * k4 + 1] = t.y;
        oacc[n][4 * k4 + 2] = t.z;
        oacc[n][4 * k4 + 3] = t.w;
      }
    const f32x4 ml = __builtin_nontemporal_load(wstate + 4 * NB * 64);
    m_run = ml.x;
    l_run = ml.y;
  } else {
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[n][r] = 0.0f;
  }

  int j = 0, nj = 0;
  if (beg < end) {
    j = tile_at(beg);
    nj = valid[j];
    VSA_LOAD_K(j, k_loads(nj));
    VSA_LOAD_V(vth + static_cast<size_t>(j) * TILE_BYTES, nj);
  }
  // Query and state registers (and the first tile) have landed.
  __builtin_amdgcn_s_waitcnt(kWaitVm);

  for (int it = beg; it < end; ++it) {
    const int nchunk = active ? (nj + 15) >> 4 : 0;   // 16-key chunks to process
    // K(t) landed (V(t) may still be in flight).
    __builtin_amdgcn_s_waitcnt(kWaitVm | LOADS);
    VSA_BARRIER();

    // Block 1 (keys 32..63) is computed only if it holds valid keys; its
    // registers are read only for chunks below nchunk.
    f32x16 sacc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (active && (b == 0 || nj > 32)) {
        const char* krow = lds_k + (32 * b + l32) * KROWB;
        if constexpr (QK8) {
          // Scale bytes 127 (2^0): plain E4M3 x E4M3 products, fp32 sums.
#pragma unroll
          for (int m = 0; m < NK64; ++m) {
            const int lc = 4 * m + 2 * hl;
            const u32x4 k0 = *reinterpret_cast<const u32x4*>(krow + ((lc ^ kswz_r) << 4));
            const u32x4 k1 = *reinterpret_cast<const u32x4*>(krow + (((lc + 1) ^ kswz_r) << 4));
            const i32x8 kf = __builtin_bit_cast(
                i32x8, u32x8{k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w});
            sacc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                kf, qf8[m], m == 0 ? f32x16{} : sacc[b], 0, 0, 0, 127, 0, 127);
          }
          // Key dequantisation scales (before the pad mask: pad scales are 0).
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 ks = *reinterpret_cast<const f32x4*>(lds_k + K_TILE + 1024 * b +
                                                             4 * (8 * r4 + 4 * hl));
            sacc[b][4 * r4 + 0] *= ks.x;
            sacc[b][4 * r4 + 1] *= ks.y;
            sacc[b][4 * r4 + 2] *= ks.z;
            sacc[b][4 * r4 + 3] *= ks.w;
          }
        } else {
#pragma unroll
          for (int c = 0; c < NCK; ++c) {
            const bf16x8 kf =
                *reinterpret_cast<const bf16x8*>(krow + (((2 * c + hl) ^ kswz_r) << 4));
            sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c],
                                                              c == 0 ? f32x16{} : sacc[b], 0, 0, 0);
          }
        }
      }
    }
    VSA_BARRIER();  // every wave is done with K(t)
    // The last iteration re-requests its own tile, so that every iteration
    // issues the same loads and the wait counts below stay exact.
    const int jn = it + 1 < end ? tile_at(it + 1) : j;
    const int njn = valid[jn];
    const int kl_next = k_loads(njn);
    VSA_LOAD_K(jn, kl_next);

    // Lane holds keys 32b + 8(r/4) + 4hl + r%4 of query column l32; 16-key
    // chunk e is registers 8(e%2)..8(e%2)+7 of block e/2.
    if (active && (nj & 15)) {
      // Key 32b + 8(r/4) + 4hl + r%4 is a pad key iff its constant part
      // reaches nj - 4hl (one per-lane limit, not one index per register).
      const int lim = nj - 4 * hl;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * b + 8 * (r >> 2) + (r & 3) >= lim) sacc[b][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (e < nchunk) {
#pragma unroll
        for (int r = 0; r < 8; ++r) mx = fmaxf(mx, sacc[e >> 1][8 * (e & 1) + r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_tile = mx * scale_log2;
    if (__builtin_amdgcn_ballot_w64(m_tile > m_run + 8.0f) != 0) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < NB; ++n) oacc[n] *= alpha;
    }

    bf16x8 pf[4];
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (e < nchunk) {
        float pv[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          pv[r] = __builtin_amdgcn_exp2f(fmaf(sacc[e >> 1][8 * (e & 1) + r], scale_log2, -m_run));
          psum += pv[r];
        }
        u32x4 pu;
        pu.x = pack_bf16x2(pv[0], pv[1]);
        pu.y = pack_bf16x2(pv[2], pv[3]);
        pu.z = pack_bf16x2(pv[4], pv[5]);
        pu.w = pack_bf16x2(pv[6], pv[7]);
        pf[e] = __builtin_bit_cast(bf16x8, pu);
      }
    }
    l_run += psum;

    // V(t) landed (the K(t+1) group may still be in flight).
    switch (kl_next + (QK8 ? 1 : 0)) {
      case 0: __builtin_amdgcn_s_waitcnt(kWaitVm | 0); break;
      case 1: __builtin_amdgcn_s_waitcnt(kWaitVm | 1); break;
      case 2: __builtin_amdgcn_s_waitcnt(kWaitVm | 2); break;
      case 3: __builtin_amdgcn_s_waitcnt(kWaitVm | 3); break;
      case 4: __builtin_amdgcn_s_waitcnt(kWaitVm | 4); break;
      case 5: __builtin_amdgcn_s_waitcnt(kWaitVm | 5); break;
      case 6: __builtin_amdgcn_s_waitcnt(kWaitVm | 6); break;
      case 7: __builtin_amdgcn_s_waitcnt(kWaitVm | 7); break;
      default: __builtin_amdgcn_s_waitcnt(kWaitVm | 8); break;
    }
    VSA_BARRIER();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (e < nchunk) {
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const char* vrow = lds_v + (32 * n + l32) * 128;
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vrow + (((2 * e + hl) ^ vswz_r) << 4));
          oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[e], oacc[n], 0, 0, 0);
        }
      }
    }
    VSA_BARRIER();  // every wave is done with V(t)
    VSA_LOAD_V(vth + static_cast<size_t>(jn) * TILE_BYTES, njn);
    j = jn;
    nj = njn;
  }
  // No global->LDS load may still be in flight when the block's LDS is released.
  __builtin_amdgcn_s_waitcnt(kWaitVm);
#undef VSA_LOAD_K
#undef VSA_LOAD_V
#undef VSA_BARRIER

  if (!last) {
    if (active) {
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const f32x4 t = {oacc[n][4 * k4 + 0], oacc[n][4 * k4 + 1], oacc[n][4 * k4 + 2],
                           oacc[n][4 * k4 + 3]};
          __builtin_nontemporal_store(t, wstate + (4 * n + k4) * 64);
        }
      const f32x4 ml = {m_run, l_run, 0.0f, 0.0f};
      __builtin_nontemporal_store(ml, wstate + 4 * NB * 64);
    }
    return;
  }

  // Epilogue: normalise, add gate * coarse, store at the packed row.
  l_run += __shfl_xor(l_run, 32);
  if (pr >= 0) {
    const float inv = 1.0f / l_run;
    const float* cg = a.coarse + (static_cast<size_t>(hd) * Nt + i) * D;
    const size_t rowoff = (static_cast<size_t>(pr) * H + hd) * D;
    const TIO* gate = static_cast<const TIO*>(a.gate) + rowoff;
    TIO* out = static_cast<TIO*>(a.out) + rowoff;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * n + 8 * g4 + 4 * hl;
        const float4 cc = *reinterpret_cast<const float4*>(cg + d0);
        float gv[4];
        IoOps<TIO>::load4(gate + d0, gv);
        float res[4];
        res[0] = fmaf(gv[0], cc.x, oacc[n][4 * g4 + 0] * inv);
        res[1] = fmaf(gv[1], cc.y, oacc[n][4 * g4 + 1] * inv);
        res[2] = fmaf(gv[2], cc.z, oacc[n][4 * g4 + 2] * inv);
        res[3] = fmaf(gv[3], cc.w, oacc[n][4 * g4 + 3] * inv);
        IoOps<TIO>::store4(out + d0, res);
      }
    }
  }
}

template <typename TIO, int D, bool QK8>
hipError_t launch_q(const FineArgs& a, hipStream_t stream) {
  const int blocks = a.H * a.Nt;
  const int nchunks = a.nchunks > 1 ? a.nchunks : 1;
  for (int c = 0; c < nchunks; ++c) {
    hipLaunchKernelGGL((fine_attn_kernel<TIO, D, QK8>), dim3(blocks), dim3(128), 0, stream, a,
                       a.valid, a.sel, a.choff, a.state, c);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <typename TIO, int D>
hipError_t launch(const FineArgs& a, hipStream_t stream) {
  return a.kt8 ? launch_q<TIO, D, true>(a, stream) : launch_q<TIO, D, false>(a, stream);
}

}  // namespace

hipError_t launch_fine(const FineArgs& a, hipStream_t stream) {
  if (a.io_f32) return a.D == 64 ? launch<float, 64>(a, stream) : launch<float, 128>(a, stream);
  return a.D == 64 ? launch<uint16_t, 64>(a, stream) : launch<uint16_t, 128>(a, stream);
}

}  // namespace vsa

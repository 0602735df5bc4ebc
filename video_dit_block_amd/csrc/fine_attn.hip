// Fine branch of VSA-H3: block-sparse flash attention on bf16 MFMA, with the
// gate-and-combine epilogue and the scatter back to packed order fused in.
//
// What is computed (FastH3 4-step Preview (VSA, data-free), section "Video
// Sparse Attention is not optional here"; FastH3 NVFP4 on RTX PRO 6000,
// "Block-sparse FP4 attention for VSA tiles"): a video query tile attends to
// every prefix key tile plus its selected video key tiles; a prefix query
// tile attends to all tiles; pad keys of partial tiles are masked.  With a
// reference keep ratio (the OmniRef page, "Device profiles") a video query
// tile visits only its selected reference (cond) tiles among the prefix
// tiles, and its whole key list comes from the coarse stage.  Then
//     out[r] = o[r] + gate[r] * c[tile(r)]
// written at the token's packed row ("Model integration": the output is
// gathered back to packed order; the per-token gate multiplies the small
// per-tile compression output, "What was tried and not shipped").
//
// Design (gfx950, wave64):
//   - tiles hold 64 or 128 tokens and are handled as 64-slot blocks (a
//     128-token tile is two consecutive blocks);
//   - one workgroup of 2 waves per (head, query block), or with 128-token
//     tiles one of 4 waves per (head, query tile), so that the tile's two
//     query blocks share every K/V load (FP8 keys at head_dim 64 keep two-wave
//     blocks); wave w owns query rows 32w..32w+31, gathered straight from the
//     packed [L][H][D] input through the slot table into MFMA operand
//     registers;
//   - the visit list is ascending (prefix tiles 0..P-1, or the listed ones,
//     then the selected video tiles) and visits each tile's blocks in order,
//     stepping over a block without valid keys (the second block of a
//     128-token tile with at most 64 tokens); a tile's first block always
//     holds a token, so every row starts from a finite running max;
//   - a key tile is staged in LDS as four half tiles (K keys 0-31, K keys
//     32-63, V^T keys 0-31, V^T keys 32-63), one slot each, filled by direct
//     global->LDS loads (global_load_lds_dwordx4, no register staging).  A
//     slot is refilled with the next tile's half as soon as all waves have
//     read it, so each load has about three quarters of an iteration to land
//     (32 KB of LDS per workgroup: four two-wave or two four-wave
//     workgroups per CU);
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys are the M dimension, so
//     each lane holds one query column), online softmax in fp32 via exp2 with
//     the 1/sqrt(D) scale folded into log2 units; the running max is raised
//     only when a tile exceeds it by more than 2^8 (probabilities stay below
//     256, exact enough for bf16 P and fp32 sums), so the O rescale is rare;
//   - O^T += V^T P^T on the same MFMA: P^T is consumed straight from the S^T
//     accumulator layout; V^T is stored with the keys of each 16-key group
//     permuted (0-3, 8-11, 4-7, 12-15) so that each lane's 8 keys are one
//     16-byte LDS read;
//   - LDS slots are made of 64-byte rows with XOR-swizzled 16-byte chunks,
//     bank-conflict free for the MFMA operand reads; one per-lane offset
//     serves every DMA load of a slot;
//   - each key tile is taken in two 32-key halves, and the exp of one half
//     is issued between the MFMAs of the other (Q.K of the second half, then
//     P.V of the first), so softmax arithmetic and matrix work can overlap
//     inside each wave; a half without valid keys is skipped, and the
//     running max is tested per lane, with the row's two lanes combined only
//     when it has to rise;
//   - blocks are mapped to the 8 XCDs so that each XCD works through its own
//     heads, head by head: the 32 CUs of an XCD sweep the same head's K/V;
//   - long key lists are cut into key chunks, one launch each: every query
//     tile of a head visits its tiles of the current chunk at about the same
//     time, so many of those reads hit the L2 (and the Infinity Cache)
//     instead of HBM.  Each wave's running state (O^T, running max, its lanes' row
//     sums) is stored in fp32 at the end of a launch and loaded at the start
//     of the next; visit order and arithmetic are those of a single launch,
//     so the result is the same bit for bit.
#include <type_traits>

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

// (head, query item) of block b in a single-launch forward, for P prefix and
// NV video items per head.  With heads divisible by 8, XCD x (blocks b = x
// mod 8) owns heads x, x+8, ...; inside an XCD, the prefix items of its heads
// come first, then the video items head by head.
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

// (head, query item) of block b in one key-chunk launch, for n items per
// head: XCD x works through its heads x, x+8, ... one at a time, every query
// item of a head in turn, so the XCD's L2 only has to hold the current head's
// chunk of K and V.
__device__ __forceinline__ void decode_item_chunked(int b, int H, int n, int& h, int& i) {
  if ((H & 7) == 0) {
    const int s = b >> 3;
    const int k = s / n;
    i = s - k * n;
    h = (b & 7) + 8 * k;
  } else {
    h = b / n;
    i = b - h * n;
  }
}

// s_waitcnt immediate that waits for vmcnt <= N (N < 16, OR-ed in) and leaves
// expcnt and lgkmcnt unconstrained.  The builtin, unlike inline asm, is seen
// by the compiler's own wait-count pass, which then does not add a
// conservative vmcnt(0) in front of the LDS reads.
constexpr int kWaitVm = 0x0F70;

// XOR swizzle of the 16-byte chunk index inside a 64-byte LDS row: rows
// r, r + 4, r + 8, r + 12 differ, so the 16 lanes of one pass of a 16-byte
// operand read (rows r0..r0+15, one chunk each) hit all 64 banks once.
__device__ __forceinline__ int swz64(int row) { return (row >> 2) & 3; }

// An opaque copy of x: no instruction is emitted, but code that uses the
// result cannot be moved above this point (for instance out of a branch).
__device__ __forceinline__ float pinned(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Eight input values as fp32.
template <typename TIO>
__device__ __forceinline__ void load_f32x8(const TIO* p, float v[8]) {
  IoOps<TIO>::load4(p, v);
  IoOps<TIO>::load4(p + 4, v + 4);
}

// NW waves per block own NW * 32 query rows: 2 (a 64-slot block) or 4 (a
// whole 128-token tile, whose two blocks share every K/V load).  A tile is
// 1 << BSH blocks (BSH 0: 64-token tiles, 1: 128-token tiles).
template <typename TIO, int D, bool QK8, int NW, int BSH>
__global__ __launch_bounds__(64 * NW, 2) void fine_attn_kernel(FineArgs a,
                                                          const int32_t* __restrict__ valid,
                                                          const int32_t* __restrict__ list,
                                                          const int32_t* __restrict__ choff,
                                                          float* __restrict__ state, int chunk) {
  // K rows: bf16 (2D bytes), or OCP FP8 E4M3 codes (D bytes) with QK8.
  constexpr int KROWB = QK8 ? D : 2 * D;
  constexpr int K_TILE = 64 * KROWB;
  constexpr int KH_BYTES = 32 * KROWB;           // one 32-key half of a K tile
  constexpr int VH_BYTES = 64 * D;               // one 32-key half of a V^T tile: D rows of 64 B
  constexpr int V_TILE = 2 * VH_BYTES;
  static_assert(NW == 2 || (NW == 4 && BSH == 1), "four waves only for 128-token tiles");
  constexpr int KH_LOADS = KH_BYTES / 1024 / NW;  // 1 KB DMA loads per wave per K half
  constexpr int VH_LOADS = VH_BYTES / 1024 / NW;  // the same per V^T half
  static_assert(KH_LOADS * NW * 1024 == KH_BYTES && VH_LOADS * NW * 1024 == VH_BYTES,
                "a half splits evenly over the waves");
  constexpr int NK64 = D / 64;                   // FP8 MFMA steps of 64 channels
  constexpr int NCK = D / 16;                    // QK contraction steps
  constexpr int NB = D / 32;                     // O^T blocks of 32 channels
  // Four LDS slots, one per half tile: K keys 0-31, K keys 32-63, V^T keys
  // 0-31 and V^T keys 32-63.  With QK8 a K slot is followed by 1 KB per wave
  // for per-key scales (the first 64 bytes hold the wave's 16 scales).
  constexpr int KSLOT = QK8 ? KH_BYTES + 2048 : KH_BYTES;
  __shared__ __attribute__((aligned(1024))) char lds_ka[KSLOT];
  __shared__ __attribute__((aligned(1024))) char lds_kb[KSLOT];
  __shared__ __attribute__((aligned(1024))) char lds_va[VH_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds_vb[VH_BYTES];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int lane = tid & 63;
  const int hl = lane >> 5;      // lane half: k-slots 8*hl..8*hl+7 of each MFMA
  const int l32 = lane & 31;
  const int H = a.H, Nt = a.Nt, P = a.P, NV = a.NV;
  // Tiles are 1 << bsh blocks of 64 slots; the block is the unit of work.
  constexpr int bsh = BSH;
  const int Nb = Nt << bsh, Pvis = a.Pvis;

  // A query item is 1 << ish blocks: one block with two waves, a whole
  // 128-token tile with four.
  constexpr int ish = NW == 4 ? 1 : 0;
  int hd, ib;  // head, first query block of the item
  if (a.nchunks > 1) {
    // The items of a head run in the chunk's order of its query tiles, the
    // tiles with the most visits first (an item is a tile or one of its
    // blocks).
    int s;
    decode_item_chunked(blockIdx.x, H, Nb >> ish, hd, s);
    constexpr int sub = bsh - ish;
    const int t = min(max(a.order[(static_cast<size_t>(hd) * a.nchunks + chunk) * Nt + (s >> sub)],
                          0), Nt - 1);
    ib = (t << sub) | (s & ((1 << sub) - 1));
  } else {
    decode_item(blockIdx.x, H, (P << bsh) >> ish, (NV << bsh) >> ish, hd, ib);
  }
  ib <<= ish;
  const int i = ib >> bsh;  // query tile
  const int nrows = NW == 4 ? valid[ib] + valid[ib + 1] : valid[ib];
  // The second block of a 128-token tile with at most 64 tokens has no rows.
  if (nrows == 0) return;

  // Visit list of tiles: prefix tiles 0..Pvis-1 then the query tile's row of
  // the list (all tiles for a prefix query tile), ascending; every tile is
  // visited block by block.  This launch covers the part of it with ids in
  // [chunk * chunk_tiles, (chunk + 1) * chunk_tiles).
  const bool dense = i < P;
  int beg = 0, end = dense ? Nt : Pvis + a.listlen;
  if (a.nchunks > 1) {
    const int lo = chunk * a.chunk_tiles;
    const int hi = min(lo + a.chunk_tiles, Nt);
    if (dense) {
      beg = lo;
      end = hi;
    } else {
      const int32_t* co = choff + (static_cast<size_t>(hd) * NV + (i - P)) * (a.nchunks + 1) + chunk;
      beg = min(lo, Pvis) + co[0];
      end = min(hi, Pvis) + co[1];
    }
  }
  beg <<= bsh;
  end <<= bsh;
  const bool first = chunk == 0;
  const bool last = chunk == a.nchunks - 1;
  // Nothing to add, and the running state stays where it is.
  if (beg >= end && !first && !last) return;

  // Query fragment: B operand of S^T = K Q^T (column = query, k = channel).
  const TIO* q = static_cast<const TIO*>(a.q);
  const int pr = a.perm[static_cast<size_t>(ib) * 64 + 32 * w + l32];
  // A wave whose 32 query rows are all pad slots (the end of an item with
  // fewer valid tokens) only takes part in the loads and barriers.
  const bool active = 32 * w < nrows;
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
          load_f32x8(a.qt + ((static_cast<size_t>(hd) * Nb + ib) * 64 + 32 * w + l32) * D + d0,
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
    const uint16_t* qrow = a.qt + ((static_cast<size_t>(hd) * Nb + ib) * 64 + 32 * w + l32) * D;
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

  const int32_t* sl = list + (dense ? 0 : (static_cast<size_t>(hd) * NV + (i - P)) * a.listlen);
  const char* kth = (QK8 ? reinterpret_cast<const char*>(a.kt8) : reinterpret_cast<const char*>(a.kt)) +
                    static_cast<size_t>(hd) * Nb * K_TILE;
  const char* ksh =
      QK8 ? reinterpret_cast<const char*>(a.kscale) + static_cast<size_t>(hd) * Nb * 256 : nullptr;
  const char* vth = reinterpret_cast<const char*>(a.vt) + static_cast<size_t>(hd) * Nb * V_TILE;
  // Block of visit it.  Listed ids are clamped into [0, Nt): a corrupt list
  // can give a wrong result but never an out-of-bounds read.
  const int bmask = (1 << bsh) - 1;
  auto tile_at = [&](int it) -> int {
    const int v = it >> bsh;
    if (dense || v < Pvis) return it;
    const int t = min(max(sl[v - Pvis], 0), Nt - 1);
    return (t << bsh) | (it & bmask);
  };

  // LDS slot layouts (16-byte chunks, XOR-swizzled inside 64-byte rows so
  // that the MFMA operand reads are free of bank conflicts):
  //   K half:   [KROWB/64 groups][32 keys][64 B]: chunks 4G..4G+3 of a key
  //             row; logical chunk c sits at (c ^ swz64(key)) in its group;
  //   V^T half: [D rows][64 B] (the 32 keys of the half), the same swizzle.
  // DMA load number x (0..NW*KH_LOADS-1, or 0..NW*VH_LOADS-1, over all waves;
  // 64 lanes x 16 B each)
  // fills LDS chunks 64x..64x+63: K rows 16(x % 2) + lane/4 of group x/2,
  // V^T rows 16x + lane/4.  The lane part of the source offset is the same
  // for every load, the rest is uniform.
  const int lane_sw = ((lane & 3) ^ ((lane >> 4) & 3)) << 4;
  const int kbase = (lane >> 2) * KROWB + lane_sw;
  const int vbase = (lane >> 2) * 64 + lane_sw;
// Block barrier without the workgroup fence of __syncthreads(): the fence
// would also wait for every outstanding global->LDS load, which this loop
// keeps in flight on purpose.  LDS reads are drained first (so no wave's
// pending read can race the next DMA into that region) and DMA completion is
// awaited explicitly (kWaitVm) before the barriers that publish a slot.  The
// memory clobber keeps the compiler from moving memory accesses across it.
#define VSA_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")
// Half B of K tile J into slot SLOT: KH_LOADS loads per wave and, with QK8,
// one load of 16 per-key scales by each of waves 0 and 1 (lanes 4..63 repeat
// lanes 0..3).
// Pad rows are zero in memory, so a loaded half holds no stale data; a half
// without valid keys is neither loaded nor read.
#define VSA_LOAD_KH(SLOT, J, B)                                                               \
  {                                                                                            \
    const char* src_ = kth + static_cast<size_t>(J) * K_TILE + (B) * KH_BYTES;                 \
    _Pragma("unroll") for (int e = 0; e < KH_LOADS; ++e) {                                     \
      const int x_ = w * KH_LOADS + e;                                                         \
      __builtin_amdgcn_global_load_lds(                                                        \
          (gbl_void*)(src_ + kbase + (x_ & 1) * 16 * KROWB + (x_ >> 1) * 64),                  \
          (lds_void*)((SLOT) + x_ * 1024), 16, 0, 0);                                          \
    }                                                                                          \
    if (QK8 && w < 2)                                                                          \
      __builtin_amdgcn_global_load_lds(                                                        \
          (gbl_void*)(ksh + static_cast<size_t>(J) * 256 + 128 * (B) + 64 * w + 16 * (lane & 3)), \
          (lds_void*)((SLOT) + KH_BYTES + 1024 * w), 16, 0, 0);                                \
  }
// Half B of V^T tile J into slot SLOT: VH_LOADS loads per wave.
#define VSA_LOAD_VH(SLOT, J, B)                                                               \
  {                                                                                            \
    const char* src_ = vth + static_cast<size_t>(J) * V_TILE + (B) * VH_BYTES;                 \
    _Pragma("unroll") for (int e = 0; e < VH_LOADS; ++e) {                                     \
      const int x_ = w * VH_LOADS + e;                                                         \
      __builtin_amdgcn_global_load_lds((gbl_void*)(src_ + vbase + x_ * 1024),                  \
                                       (lds_void*)((SLOT) + x_ * 1024), 16, 0, 0);             \
    }                                                                                          \
  }
  // Loads this wave issues for half b of a tile with n valid keys.
  constexpr int CKMAX = KH_LOADS + (QK8 ? 1 : 0);
  const int CK = KH_LOADS + (QK8 && w < 2 ? 1 : 0);
  constexpr int CV = VH_LOADS;
  static_assert(2 * (CKMAX > CV ? CKMAX : CV) <= 8, "wait counts above 8");
  auto ck = [CK](int n, int b) -> int { return n > 32 * b ? CK : 0; };
  auto cv = [](int n, int b) -> int { return n > 32 * b ? CV : 0; };
  // Wait until at most n of this wave's loads are in flight.
  auto wait_vm = [](int n) {
    switch (n) {
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
  };

  // Swizzle of this lane's operand rows (key l32 of a K half, V^T row
  // 32n + l32; the latter does not depend on n).
  const int rswz = swz64(l32);

  // Logit scale in log2 units; with QK8 it also carries the query row's
  // dequantisation scale (the key scales are applied to S below).
  // A query row of zeros has qsc 0 and all-zero logits; the scale then stays
  // at its positive bf16 value so that masked keys (-inf) give exp2 = 0
  // rather than -inf * 0.
  const float scale_log2 = (1.4426950408889634f / sqrtf(static_cast<float>(D))) *
                           (qsc > 0.0f ? qsc : 1.0f);
  // Running state of this wave's 32 rows: O^T accumulators, running max (in
  // log2 units) and this lane's partial row sum.  Between key-chunk launches
  // it lives in `state`, one 16-byte quad per lane per 4 words, coalesced:
  // quads 0..4NB-1 hold oacc, quad 4NB holds (m_run, l_run, 0, 0).
  f32x16 oacc[NB];
  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x4* wstate = reinterpret_cast<f32x4*>(state) +
                  ((static_cast<size_t>(hd) * Nb + ib) * 2 + w) * (4 * NB + 1) * 64 + lane;
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

  // A key tile is taken in two halves of 32 keys; each half is 8 Q.K MFMA
  // steps (bf16; 2 with FP8 q/k) and 8 P.V steps (D 128).  The work of one
  // tile runs as four phases, each a fixed sequence of steps fenced with
  // sched_barrier so that the compiler keeps the order:
  //   1. Q.K of half 0;
  //   2. Q.K of half 1, with the exp of half 0 spread over its steps;
  //   3. P.V of half 0, with the exp of half 1 spread over its steps;
  //   4. P.V of half 1.
  // The MFMA operands are read from LDS kAhead steps ahead of their use.
  constexpr int kQkSteps = QK8 ? NK64 : NCK;
  constexpr int kPvSteps = 2 * NB;
  constexpr int kAhead = 3;
  typedef typename std::conditional<QK8, i32x8, bf16x8>::type QkOp;

  // LDS operand of Q.K step k of half b (lane row l32 of the half's keys).
  auto qk_read = [&](int b, int k) -> QkOp {
    const char* krow = (b ? lds_kb : lds_ka) + l32 * 64;
    if constexpr (QK8) {
      // Chunks 4k + 2hl and 4k + 2hl + 1 (channels 64k + 32hl + 0..31).
      const char* g = krow + k * 2048;
      const u32x4 k0 = *reinterpret_cast<const u32x4*>(g + (((2 * hl) ^ rswz) << 4));
      const u32x4 k1 = *reinterpret_cast<const u32x4*>(g + (((2 * hl + 1) ^ rswz) << 4));
      return __builtin_bit_cast(i32x8, u32x8{k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w});
    } else {
      // Chunk 2k + hl (channels 16k + 8hl + 0..7).
      return *reinterpret_cast<const bf16x8*>(krow + (k >> 1) * 2048 +
                                              (((2 * (k & 1) + hl) ^ rswz) << 4));
    }
  };
  // Q.K step k: S^T (keys x queries) of the half accumulates channels of step k.
  auto qk_step = [&](int k, const QkOp& kf, f32x16& acc) {
    if constexpr (QK8) {
      // Scale bytes 127 (2^0): plain E4M3 x E4M3 products, fp32 sums.
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf8[k], k == 0 ? f32x16{} : acc,
                                                            0, 0, 0, 127, 0, 127);
    } else {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[k], k == 0 ? f32x16{} : acc, 0, 0, 0);
    }
  };
  // FP8 keys: multiply S by the per-key dequantisation scales (pad keys have
  // scale 0 and are masked afterwards).  Keys 16v..16v+15 of the half were
  // staged by wave v.
  auto key_scales = [&](int b, f32x16& acc) {
    if constexpr (QK8) {
      const char* sc = (b ? lds_kb : lds_ka) + KH_BYTES;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 ks = *reinterpret_cast<const f32x4*>(sc + 1024 * (r4 >> 1) +
                                                         4 * (8 * (r4 & 1) + 4 * hl));
        acc[4 * r4 + 0] *= ks.x;
        acc[4 * r4 + 1] *= ks.y;
        acc[4 * r4 + 2] *= ks.z;
        acc[4 * r4 + 3] *= ks.w;
      }
    }
  };
  // LDS operand of P.V step k of half b: V^T rows 32n.., 16-key group g of the half.
  auto pv_read = [&](int b, int k) -> bf16x8 {
    const int g = k / NB, n = k % NB;
    const char* vrow = (b ? lds_vb : lds_va) + (32 * n + l32) * 64;
    return *reinterpret_cast<const bf16x8*>(vrow + (((2 * g + hl) ^ rswz) << 4));
  };
  auto pv_step = [&](int k, const bf16x8& vf, const bf16x8& pa, const bf16x8& pb) {
    const int g = k / NB, n = k % NB;
    oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, g == 0 ? pa : pb, oacc[n], 0, 0, 0);
  };
  // Softmax pairs [8k/NS, 8(k+1)/NS) of one half: p = exp2(s*scale - mref),
  // packed to bf16 pair by pair (word r/2 of the two 16-key operands).
  auto sm_part = [&](int k, int ns, const f32x16& sacc, float mref, uint32_t pw[8], float& ps) {
#pragma unroll
    for (int q = 8 * k / ns; q < 8 * (k + 1) / ns; ++q) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[2 * q], scale_log2, -mref));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[2 * q + 1], scale_log2, -mref));
      ps += p0;
      ps += p1;
      pw[q] = pack_bf16x2(p0, p1);
    }
  };
  // p <- bf16(p * f) for the 8 probabilities of one operand.
  auto rescale_bf16 = [](bf16x8& p, float f) {
    u32x4 u = __builtin_bit_cast(u32x4, p);
    u.x = pack_bf16x2(__uint_as_float(u.x << 16) * f, __uint_as_float(u.x & 0xffff0000u) * f);
    u.y = pack_bf16x2(__uint_as_float(u.y << 16) * f, __uint_as_float(u.y & 0xffff0000u) * f);
    u.z = pack_bf16x2(__uint_as_float(u.z << 16) * f, __uint_as_float(u.z & 0xffff0000u) * f);
    u.w = pack_bf16x2(__uint_as_float(u.w << 16) * f, __uint_as_float(u.w & 0xffff0000u) * f);
    p = __builtin_bit_cast(bf16x8, u);
  };
  auto pack16 = [](const uint32_t pw[8], bf16x8& pa, bf16x8& pb) {
    pa = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
    pb = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
  };
  // Q.K of half b; if SM, the softmax of the other half (s_other, reference
  // mref) is spread over the steps.  Returns that softmax's lane sum.
  auto qk_phase = [&](int b, f32x16& acc, bool sm, const f32x16& s_other, float mref,
                      bf16x8& pa, bf16x8& pb) -> float {
    QkOp kf[kQkSteps];
    uint32_t pv[8];
    float ps = 0.0f;
#pragma unroll
    for (int k = 0; k < kAhead && k < kQkSteps; ++k) kf[k] = qk_read(b, k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kQkSteps; ++k) {
      if (k + kAhead < kQkSteps) kf[k + kAhead] = qk_read(b, k + kAhead);
      qk_step(k, kf[k], acc);
      if (sm) sm_part(k, kQkSteps, s_other, mref, pv, ps);
      __builtin_amdgcn_sched_barrier(0);
    }
    key_scales(b, acc);
    if (sm) pack16(pv, pa, pb);
    return ps;
  };
  // P.V of half b (probabilities pa, pb); if SM, the softmax of s_other is
  // spread over the steps.  Returns that softmax's lane sum.
  auto pv_phase = [&](int b, const bf16x8& pa, const bf16x8& pb, bool sm, const f32x16& s_other,
                      float mref, bf16x8& qa, bf16x8& qb) -> float {
    bf16x8 vf[kPvSteps];
    uint32_t pv[8];
    float ps = 0.0f;
#pragma unroll
    for (int k = 0; k < kAhead; ++k) vf[k] = pv_read(b, k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kPvSteps; ++k) {
      if (k + kAhead < kPvSteps) vf[k + kAhead] = pv_read(b, k + kAhead);
      pv_step(k, vf[k], pa, pb);
      if (sm) sm_part(k, kPvSteps, s_other, mref, pv, ps);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (sm) pack16(pv, qa, qb);
    return ps;
  };
  // Pad keys (index >= nj) of half b to -inf: key 32b + 8(r/4) + 4hl + r%4
  // is a pad key iff its constant part reaches nj - 32b - 4hl.
  auto mask_half = [&](f32x16& acc, int b, int n) {
    const int lim = n - 32 * b - 4 * hl;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) >= lim) acc[r] = -INFINITY;
  };
  auto max16 = [](const f32x16& acc) -> float {
    float m = acc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) m = fmaxf(m, acc[r]);
    return m;
  };
  // New running max (log2 units) when some row of the wave has a score more
  // than 2^8 above it, else m_run itself.  Each lane tests its own 16 keys
  // of a row; only then are the two halves of each row (lanes l, l ^ 32)
  // combined, so the common case needs no cross-lane exchange.
  auto raised_max = [&](float mx_lane) -> float {
    if (__builtin_amdgcn_ballot_w64(mx_lane * scale_log2 > m_run + 8.0f) == 0) return m_run;
    const float mx = fmaxf(mx_lane, __shfl_xor(mx_lane, 32));
    return fmaxf(m_run, mx * scale_log2);
  };

  int j = 0, nj = 0;
  if (beg < end) {
    j = tile_at(beg);
    nj = valid[j];
    VSA_LOAD_KH(lds_ka, j, 0);
    if (nj > 32) VSA_LOAD_KH(lds_kb, j, 1);
    VSA_LOAD_VH(lds_va, j, 0);
  }
  // Query and state registers (and the first tile's halves) have landed.
  __builtin_amdgcn_s_waitcnt(kWaitVm);

  // Slot ring: each half tile is requested as soon as its slot has been read
  // by all waves, about three quarters of an iteration before it is needed.
  // Issue order, in iteration t: V^T half 1 of t, then K half 0, K half 1 and
  // V^T half 0 of t + 1; each wait below counts the loads issued after the
  // half it needs.
  const f32x16 kNone = {};
  for (int it = beg; it < end;) {
    const bool has1 = nj > 32;   // the second half holds a valid key
    // The last iteration re-requests its own tile, so that every iteration
    // issues the same loads and the wait counts stay exact.  A block without
    // valid keys (only ever the second block of a short 128-token tile) is
    // stepped over.
    int itn = it + 1;
    int jn = itn < end ? tile_at(itn) : j;
    int njn = valid[jn];
    if (bsh > 0 && njn == 0) {
      ++itn;
      jn = itn < end ? tile_at(itn) : j;
      njn = valid[jn];
    }

    // K half 0 of t landed; every wave is done with V^T half 1 of t - 1.
    wait_vm(ck(nj, 1) + cv(nj, 0));
    VSA_BARRIER();
    if (has1) VSA_LOAD_VH(lds_vb, j, 1);

    f32x16 s0, s1;
    bf16x8 pf[4];
    if (active) {
      // Phase 1.
      qk_phase(0, s0, false, kNone, 0.0f, pf[0], pf[1]);
      if (nj < 32) mask_half(s0, 0, nj);
      const float m0 = raised_max(max16(s0));
      if (m0 != m_run) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m0);
        m_run = m0;
        l_run *= alpha;
#pragma unroll
        for (int n = 0; n < NB; ++n) oacc[n] *= alpha;
      }
    }
    // K half 1 of t landed; every wave is done with K half 0 of t.
    wait_vm(cv(nj, 0) + cv(nj, 1));
    VSA_BARRIER();
    VSA_LOAD_KH(lds_ka, jn, 0);

    float alpha1 = 1.0f;
    if (active) {
      // Phase 2 (the pinned copy keeps the softmax inside the branch).
      if (has1) {
        l_run += qk_phase(1, s1, true, s0, pinned(m_run), pf[0], pf[1]);
      } else {
        uint32_t pv[8];
        float ps = 0.0f;
        sm_part(0, 1, s0, m_run, pv, ps);
        pack16(pv, pf[0], pf[1]);
        l_run += ps;
      }
      // The second half's max is settled before P.V of the first half starts.
      if (has1) {
        if (nj < 64) mask_half(s1, 1, nj);
        const float m1 = raised_max(max16(s1));
        alpha1 = __builtin_amdgcn_exp2f(m_run - m1);
        m_run = m1;
      }
    }
    const bool resc1 = __builtin_amdgcn_ballot_w64(alpha1 != 1.0f) != 0;

    // V^T half 0 of t landed; every wave is done with K half 1 of t.
    wait_vm(cv(nj, 1) + ck(njn, 0));
    VSA_BARRIER();
    if (njn > 32) VSA_LOAD_KH(lds_kb, jn, 1);

    if (active) {
      if (has1) {
        if (resc1) {
          // Rare: the second half raised the max.  O, the row sum and the
          // first half's probabilities (already bf16) move to the new max
          // before they are combined, so O is only ever updated in place.
          l_run *= alpha1;
#pragma unroll
          for (int n = 0; n < NB; ++n) oacc[n] *= alpha1;
          rescale_bf16(pf[0], alpha1);
          rescale_bf16(pf[1], alpha1);
        }
        // Phase 3.
        l_run += pv_phase(0, pf[0], pf[1], true, s1, pinned(m_run), pf[2], pf[3]);
      } else {
        pv_phase(0, pf[0], pf[1], false, kNone, 0.0f, pf[2], pf[3]);
      }
    }
    // V^T half 1 of t landed; every wave is done with V^T half 0 of t.
    wait_vm(ck(njn, 0) + ck(njn, 1));
    VSA_BARRIER();
    VSA_LOAD_VH(lds_va, jn, 0);

    if (active && has1) {
      // Phase 4.
      pv_phase(1, pf[2], pf[3], false, kNone, 0.0f, pf[2], pf[3]);
    }
    j = jn;
    nj = njn;
    it = itn;
  }
  // No global->LDS load may still be in flight when the block's LDS is released.
  __builtin_amdgcn_s_waitcnt(kWaitVm);
#undef VSA_LOAD_KH
#undef VSA_LOAD_VH
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

template <typename TIO, int D, bool QK8, int NW, int BSH>
hipError_t launch_w(const FineArgs& a, hipStream_t stream) {
  // One block per query item: a 64-slot block (NW 2) or a 128-token tile (NW 4).
  const int blocks = a.H * ((a.Nt << BSH) >> (NW == 4 ? 1 : 0));
  const int nchunks = a.nchunks > 1 ? a.nchunks : 1;
  for (int c = 0; c < nchunks; ++c) {
    hipLaunchKernelGGL((fine_attn_kernel<TIO, D, QK8, NW, BSH>), dim3(blocks), dim3(64 * NW), 0,
                       stream, a, a.valid, a.list, a.choff, a.state, c);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <typename TIO, int D, bool QK8>
hipError_t launch_q(const FineArgs& a, hipStream_t stream) {
  if (a.bsh == 0) return launch_w<TIO, D, QK8, 2, 0>(a, stream);
  // 128-token tiles: the tile's two query blocks share one block of four
  // waves, and so every K/V load -- unless a K half (FP8 codes at head_dim
  // 64: 2 KB) does not split into 1 KB loads for four waves.
  if constexpr (QK8 && D == 64)
    return launch_w<TIO, D, true, 2, 1>(a, stream);
  else
    return launch_w<TIO, D, QK8, 4, 1>(a, stream);
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

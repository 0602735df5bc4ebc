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
//     holds a token, so every row starts from a finite running max; with
//     64-token tiles, two consecutive visited tiles of at most 32 tokens (a
//     short tile holds one half) are taken as the two halves of one
//     iteration, in the same order;
//   - a key tile is staged in LDS as four half tiles (K keys 0-31, K keys
//     32-63, V^T keys 0-31, V^T keys 32-63), one slot each, filled by direct
//     global->LDS loads (buffer_load_dwordx4 ... lds, no register staging).
//     A tile runs as four matrix phases (Q.K of half 0, P.V of the previous
//     tile's half 1, Q.K of half 1, P.V of half 0), and the waves sync twice
//     per tile, after the second and the fourth phase; at each sync the two
//     slots the waves have just finished with take the next halves.  Each
//     load has two of the four phases to land, and every wait is for all of
//     the wave's loads (32 KB of LDS per workgroup: four two-wave or two
//     four-wave workgroups per CU);
//   - S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys are the M dimension, so
//     each lane holds one query column), online softmax in fp32 via exp2 with
//     the 1/sqrt(D) scale folded into log2 units.  The exps of a half tile
//     are taken against the running max as it stands, with no max pass: the
//     max is raised, O and the row sum rescaled and the half redone only when
//     a lane's sum of the half's probabilities is not in [0, 2^20] (always at
//     a row's first block, whose running max is still -inf).  Probabilities
//     then stay below 2^20, far inside fp32 and bf16 range, and the result
//     differs from a max-subtracted softmax only by rounding;
//   - O^T += V^T P^T on the same MFMA: P^T is consumed straight from the S^T
//     accumulator layout; V^T is stored with the keys of each 16-key group
//     permuted (0-3, 8-11, 4-7, 12-15) so that each lane's 8 keys are one
//     16-byte LDS read;
//   - LDS slots are made of 64-byte rows with XOR-swizzled 16-byte chunks,
//     bank-conflict free for the MFMA operand reads; one per-lane offset
//     serves every DMA load of a slot;
//   - each key tile is taken in two 32-key halves, and a half's softmax is
//     issued in two parts between the MFMAs of the neighbouring phases, so
//     softmax arithmetic and matrix work overlap inside each wave; a half
//     without valid keys is skipped, and the row's two lanes are combined
//     only when its running max has to rise;
//   - blocks are mapped to the 8 XCDs so that each XCD works through its own
//     heads, head by head: the 32 CUs of an XCD sweep the same head's K/V;
//   - fp32 I/O keeps fp32-level accuracy on the bf16 matrix cores: every
//     operand x is split into bf16 parts hi = bf16(x), lo = bf16(x - hi), and
//     each product a*b is formed as a_hi*b_hi + a_hi*b_lo + a_lo*b_hi with
//     fp32 sums (three MFMAs per step of Q.K and of P.V; the dropped a_lo*b_lo
//     and the split residues are about 2^-16 of |a*b|); K and V^T arrive with
//     their low parts in the same slot, so the LDS ring doubles;
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
struct IoOps<float> {  // fp32 I/O; load8 gives the high bf16 parts, load8_lo the low parts
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
  static __device__ __forceinline__ bf16x8 load8_lo(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    u32x4 u;
    u.x = pack_bf16x2_lo(a.x, a.y);
    u.y = pack_bf16x2_lo(a.z, a.w);
    u.z = pack_bf16x2_lo(b.x, b.y);
    u.w = pack_bf16x2_lo(b.z, b.w);
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

// The key halves of one iteration of the fine kernel's loop.
struct Visit {
  int j, n0;        // block of the first half and its valid keys (1..32)
  int j1, b1, n1;   // block and half of the second half, its valid keys (0..32)
  int step;         // visits taken
};

// s_waitcnt immediate that waits for vmcnt 0 and leaves expcnt and lgkmcnt
// unconstrained.  The builtin, unlike inline asm, is seen by the compiler's
// own wait-count pass, which then does not add a conservative vmcnt(0) in
// front of the LDS reads.
constexpr int kWaitVm = 0x0F70;
// The same, waiting until at most n vector-memory loads are outstanding
// (vmcnt in bits 3:0 and 15:14).
constexpr int wait_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

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

// High and low bf16 parts of eight operand values (fp32 I/O).
struct Bf16Pair {
  bf16x8 h, l;
};

// Eight input values as fp32.
template <typename TIO>
__device__ __forceinline__ void load_f32x8(const TIO* p, float v[8]) {
  IoOps<TIO>::load4(p, v);
  IoOps<TIO>::load4(p + 4, v + 4);
}

// NW waves per block own NW * 32 query rows: 2 (a 64-slot block) or 4 (a
// whole 128-token tile, whose two blocks share every K/V load).  A tile is
// 1 << BSH blocks (BSH 0: 64-token tiles, 1: 128-token tiles).
// fp32 I/O (TIO float) carries low parts of every operand: more registers,
// so one wave per SIMD is allowed there.
template <typename TIO>
constexpr int kFineMinWaves = sizeof(TIO) == 4 ? 1 : 2;

template <typename TIO, int D, bool QK8, int NW, int BSH>
__global__ __launch_bounds__(64 * NW, kFineMinWaves<TIO>) void fine_attn_kernel(FineArgs a,
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
  // fp32 I/O: K (unless FP8) and V^T come with low bf16 parts, stored right
  // after the high parts in each slot.
  constexpr bool SPLIT = std::is_same<TIO, float>::value;
  constexpr bool KSPLIT = SPLIT && !QK8;
  constexpr int KPARTS = KSPLIT ? 2 : 1;
  constexpr int VPARTS = SPLIT ? 2 : 1;
  constexpr int NK64 = D / 64;                   // FP8 MFMA steps of 64 channels
  constexpr int NCK = D / 16;                    // QK contraction steps
  constexpr int NB = D / 32;                     // O^T blocks of 32 channels
  constexpr int kWaitVmO = wait_vm(4 * NB);      // all but the 4 NB loads of O
  // Four LDS slots, one per half tile: K keys 0-31, K keys 32-63, V^T keys
  // 0-31 and V^T keys 32-63.  With QK8 a K slot is followed by 1 KB per wave
  // for per-key scales (the first 64 bytes hold the wave's 16 scales).
  constexpr int KSLOT = QK8 ? KH_BYTES + 2048 : KPARTS * KH_BYTES;
  constexpr int VSLOT = VPARTS * VH_BYTES;
  __shared__ __attribute__((aligned(1024))) char lds_ka[KSLOT];
  __shared__ __attribute__((aligned(1024))) char lds_kb[KSLOT];
  __shared__ __attribute__((aligned(1024))) char lds_va[VSLOT];
  __shared__ __attribute__((aligned(1024))) char lds_vb[VSLOT];

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
  bf16x8 qfl[KSPLIT ? NCK : 1];   // fp32 I/O: low parts
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
          const size_t at = ((static_cast<size_t>(hd) * Nb + ib) * 64 + 32 * w + l32) * D + d0;
          load_f32x8(a.qt + at, &x[m][8 * g]);
          if constexpr (SPLIT) {
            float lo[8];
            load_f32x8(a.qt_lo + at, lo);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[m][8 * g + e] += lo[e];
          }
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
    const size_t at = ((static_cast<size_t>(hd) * Nb + ib) * 64 + 32 * w + l32) * D;
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
      qf[c] = IoOps<uint16_t>::load8(a.qt + at + 16 * c + 8 * hl);
      if constexpr (KSPLIT) qfl[c] = IoOps<uint16_t>::load8(a.qt_lo + at + 16 * c + 8 * hl);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
      if (pr >= 0) {
        const TIO* src = q + (static_cast<size_t>(pr) * H + hd) * D + 16 * c + 8 * hl;
        qf[c] = IoOps<TIO>::load8(src);
        if constexpr (KSPLIT) qfl[c] = IoOps<float>::load8_lo(src);
      } else {
        qf[c] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        if constexpr (KSPLIT) qfl[c] = qf[c];
      }
    }
  }

  const int32_t* sl = list + (dense ? 0 : (static_cast<size_t>(hd) * NV + (i - P)) * a.listlen);
  const char* kth = (QK8 ? reinterpret_cast<const char*>(a.kt8) : reinterpret_cast<const char*>(a.kt)) +
                    static_cast<size_t>(hd) * Nb * K_TILE;
  const char* ksh =
      QK8 ? reinterpret_cast<const char*>(a.kscale) + static_cast<size_t>(hd) * Nb * 256 : nullptr;
  const char* vth = reinterpret_cast<const char*>(a.vt) + static_cast<size_t>(hd) * Nb * V_TILE;
  // Low parts (fp32 I/O): same layouts as Kt and Vt.
  const char* ktl =
      KSPLIT ? reinterpret_cast<const char*>(a.kt_lo) + static_cast<size_t>(hd) * Nb * K_TILE
             : nullptr;
  const char* vtl =
      SPLIT ? reinterpret_cast<const char*>(a.vt_lo) + static_cast<size_t>(hd) * Nb * V_TILE
            : nullptr;
  // Buffer descriptors of this head's K, V^T (and low parts, key scales) for
  // the DMA loads below: the MUBUF form takes a uniform byte offset in an
  // SGPR and the lane's offset in one 32-bit VGPR, so no 64-bit address
  // arithmetic runs per load, and the compiler's wait-count pass keeps exact
  // LDS counts for the operand reads (it treats a global-segment load to LDS
  // like a flat access and then waits for every outstanding LDS read).
  // Word 3 selects 32-bit raw access (data format 32); reads past num_records
  // return zero.
  constexpr int kRawDword = 0x00020000;
  const int kbytes = Nb * K_TILE, vbytes = Nb * V_TILE;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kth), 0, kbytes, kRawDword);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vth), 0, vbytes, kRawDword);
  const __amdgpu_buffer_rsrc_t rkl =
      KSPLIT ? __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(ktl), 0, kbytes, kRawDword) : rk;
  const __amdgpu_buffer_rsrc_t rvl =
      SPLIT ? __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vtl), 0, vbytes, kRawDword) : rv;
  const __amdgpu_buffer_rsrc_t rks =
      QK8 ? __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(ksh), 0, Nb * 256, kRawDword) : rk;
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
  // Both halves are stored in memory in this order (the gather writes K
  // halves group by group), so DMA load number x (0..NW*KH_LOADS-1, or
  // 0..NW*VH_LOADS-1, over all waves; 64 lanes x 16 B each) reads bytes
  // 1024x..1024x+1023 of the half and fills LDS chunks 64x..64x+63: K rows
  // 16(x % 2) + lane/4 of group x/2, V^T rows 16x + lane/4.  The lane part of
  // the source offset (the row and its swizzled chunk) is the same for every
  // load, the rest is uniform.
  const int lane_sw = ((lane & 3) ^ ((lane >> 4) & 3)) << 4;
  const int lbase = (lane >> 2) * 64 + lane_sw;
// Block barrier without the workgroup fence of __syncthreads() and its cache
// maintenance.  LDS reads are drained first (so no wave's pending read can
// race the next DMA into that region); DMA completion is awaited explicitly
// (kWaitVm) right before each barrier, which then publishes the slots.  The
// memory clobber keeps the compiler from moving memory accesses across it.
#define VSA_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")
// Half B of K tile J into slot SLOT: KH_LOADS loads per wave (per part: the
// low parts of fp32 I/O follow the high parts at KH_BYTES) and, with QK8,
// one load of 16 per-key scales by each of waves 0 and 1 (lanes 4..63 repeat
// lanes 0..3).
// Pad rows are zero in memory, so a loaded half holds no stale data; a half
// without valid keys is neither loaded nor read.
// This wave's loads cover consecutive 1 KB of both memory and LDS: one LDS
// base (M0) and one SGPR offset serve them all, and the instruction's
// immediate offset, which the hardware adds to the global and to the LDS
// address alike, steps through them.
#define VSA_LOAD_KH(SLOT, J, B)                                                               \
  {                                                                                            \
    _Pragma("unroll") for (int p_ = 0; p_ < KPARTS; ++p_) {                                    \
      char* const l_ = (SLOT) + p_ * KH_BYTES + w * KH_LOADS * 1024;                           \
      const int s_ = (J) * K_TILE + (B) * KH_BYTES + w * KH_LOADS * 1024;                     \
      VSA_KLOAD(0);                                                                            \
      if (KH_LOADS > 1) VSA_KLOAD(1024);                                                       \
      if (KH_LOADS > 2) VSA_KLOAD(2048);                                                       \
      if (KH_LOADS > 3) VSA_KLOAD(3072);                                                       \
    }                                                                                          \
    if (QK8 && w < 2)                                                                          \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rks, (lds_void*)((SLOT) + KH_BYTES + 1024 * w),  \
                                               16, 16 * (lane & 3),                            \
                                               (J) * 256 + 128 * (B) + 64 * w, 0, 0);          \
  }
// (the immediate offset must be a literal)
#define VSA_KLOAD(OFF)                                                                         \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(p_ ? rkl : rk, (lds_void*)l_, 16, lbase, s_, OFF, 0)
  static_assert(KH_LOADS * 1024 <= 4096, "immediate offsets of a K half fit in 12 bits");
// Half B of V^T tile J into slot SLOT: VH_LOADS loads per wave and part.  A
// V^T half is stored in LDS order, so this wave's loads cover consecutive
// 1 KB of both memory and LDS: one LDS base (M0) and one SGPR offset serve
// them all, and the instruction's immediate offset, which the hardware adds
// to the global and to the LDS address alike, steps through them.
#define VSA_LOAD_VH(SLOT, J, B)                                                               \
  {                                                                                            \
    _Pragma("unroll") for (int p_ = 0; p_ < VPARTS; ++p_) {                                    \
      char* const l_ = (SLOT) + p_ * VH_BYTES + w * VH_LOADS * 1024;                           \
      const int s_ = (J) * V_TILE + (B) * VH_BYTES + w * VH_LOADS * 1024;                     \
      VSA_VLOAD(0);                                                                            \
      if (VH_LOADS > 1) VSA_VLOAD(1024);                                                       \
      if (VH_LOADS > 2) VSA_VLOAD(2048);                                                       \
      if (VH_LOADS > 3) VSA_VLOAD(3072);                                                       \
    }                                                                                          \
  }
// (the immediate offset must be a literal)
#define VSA_VLOAD(OFF)                                                                         \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(p_ ? rvl : rv, (lds_void*)l_, 16, lbase, s_, OFF, 0)
  static_assert(VH_LOADS * 1024 <= 4096, "immediate offsets of a V^T half fit in 12 bits");
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
  // The running max and sums come first; O follows the first tile's loads
  // (below), since the first iteration needs it only from its last phase.
  const bool load_state = !first && active;
  if (load_state) {
    const f32x4 ml = __builtin_nontemporal_load(wstate + 4 * NB * 64);
    m_run = ml.x;
    l_run = ml.y;
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
  typedef typename std::conditional<QK8, i32x8,
                                    typename std::conditional<KSPLIT, Bf16Pair, bf16x8>::type>::type
      QkOp;
  typedef typename std::conditional<SPLIT, Bf16Pair, bf16x8>::type PvOp;

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
      // Chunk 2k + hl (channels 16k + 8hl + 0..7); with fp32 I/O the low
      // parts sit KH_BYTES further.
      const char* c = krow + (k >> 1) * 2048 + (((2 * (k & 1) + hl) ^ rswz) << 4);
      if constexpr (KSPLIT)
        return Bf16Pair{*reinterpret_cast<const bf16x8*>(c),
                        *reinterpret_cast<const bf16x8*>(c + KH_BYTES)};
      else
        return *reinterpret_cast<const bf16x8*>(c);
    }
  };
  // Q.K step k: S^T (keys x queries) of the half accumulates channels of step k.
  auto qk_step = [&](int k, const QkOp& kf, f32x16& acc) {
    if constexpr (QK8) {
      // Scale bytes 127 (2^0): plain E4M3 x E4M3 products, fp32 sums.
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf8[k], k == 0 ? f32x16{} : acc,
                                                            0, 0, 0, 127, 0, 127);
    } else if constexpr (KSPLIT) {
      // k.q = k_hi.q_hi + k_lo.q_hi + k_hi.q_lo (fp32 sums).
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.h, qf[k], k == 0 ? f32x16{} : acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.l, qf[k], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.h, qfl[k], acc, 0, 0, 0);
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
  auto pv_read = [&](int b, int k) -> PvOp {
    const int g = k / NB, n = k % NB;
    const char* c = (b ? lds_vb : lds_va) + (32 * n + l32) * 64 + (((2 * g + hl) ^ rswz) << 4);
    if constexpr (SPLIT)
      return Bf16Pair{*reinterpret_cast<const bf16x8*>(c),
                      *reinterpret_cast<const bf16x8*>(c + VH_BYTES)};
    else
      return *reinterpret_cast<const bf16x8*>(c);
  };
  // P.V step k; pa/pb the probabilities of the half's two 16-key groups,
  // pal/pbl their low parts (fp32 I/O).
  auto pv_step = [&](int k, const PvOp& vf, const bf16x8& pa, const bf16x8& pb,
                     const bf16x8& pal, const bf16x8& pbl) {
    const int g = k / NB, n = k % NB;
    if constexpr (SPLIT) {
      // v.p = v_hi.p_hi + v_lo.p_hi + v_hi.p_lo (fp32 sums).
      oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.h, g == 0 ? pa : pb, oacc[n], 0, 0, 0);
      oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.l, g == 0 ? pa : pb, oacc[n], 0, 0, 0);
      oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf.h, g == 0 ? pal : pbl, oacc[n], 0, 0, 0);
    } else {
      oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, g == 0 ? pa : pb, oacc[n], 0, 0, 0);
    }
  };
  // Softmax of elements [e0, e1) of one half's S^T accumulator (16 per lane):
  // p = exp2(s*scale - mref), added to the lane sum ps in element order and
  // packed to bf16 pairs (word e/2 of pw; low parts in pwl with fp32 I/O).
  // Element 0 starts the sum; an even element waits in `odd` for its pair
  // (ranges start at even elements).
  auto sm_elems = [&](int e0, int e1, const f32x16& sacc, float mref, uint32_t pw[8],
                      uint32_t pwl[8], float& ps, float& odd) {
#pragma unroll
    for (int e = e0; e < e1; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[e], scale_log2, -mref));
      ps = e == 0 ? p : ps + p;
      if (e & 1) {
        pw[e >> 1] = pack_bf16x2(odd, p);
        if constexpr (SPLIT) pwl[e >> 1] = pack_bf16x2_lo(odd, p);
      } else {
        odd = p;
      }
    }
  };
  // The two 16-key P^T operands of a half from its packed words.
  auto pack16 = [](const uint32_t pw[8], bf16x8& pa, bf16x8& pb) {
    pa = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
    pb = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
  };
  // Q.K of half b into acc; if SM, softmax elements [e0, e0 + 8) of s_other
  // (reference mref) are spread over the steps.
  auto qk_phase = [&](int b, f32x16& acc, bool sm, const f32x16& s_other, float mref, int e0,
                      uint32_t pw[8], uint32_t pwl[8], float& ps) {
    QkOp kf[kQkSteps];
    float odd = 0.0f;
#pragma unroll
    for (int k = 0; k < kAhead && k < kQkSteps; ++k) kf[k] = qk_read(b, k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kQkSteps; ++k) {
      if (k + kAhead < kQkSteps) kf[k + kAhead] = qk_read(b, k + kAhead);
      qk_step(k, kf[k], acc);
      if (sm)
        sm_elems(e0 + 8 * k / kQkSteps, e0 + 8 * (k + 1) / kQkSteps, s_other, mref, pw, pwl, ps,
                 odd);
      __builtin_amdgcn_sched_barrier(0);
    }
    key_scales(b, acc);
  };
  // P.V of half b with the half's packed probabilities pw (low parts pwl);
  // if SM, softmax elements [e0, e0 + 8) of s_other are spread over the steps
  // into qw (qwl).
  auto pv_phase = [&](int b, const uint32_t pw[8], const uint32_t pwl[8], bool sm,
                      const f32x16& s_other, float mref, int e0, uint32_t qw[8], uint32_t qwl[8],
                      float& ps) {
    bf16x8 pa, pb, pal, pbl;
    float odd = 0.0f;
    pack16(pw, pa, pb);
    if constexpr (SPLIT) pack16(pwl, pal, pbl);
    PvOp vf[kPvSteps];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) vf[k] = pv_read(b, k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kPvSteps; ++k) {
      if (k + kAhead < kPvSteps) vf[k + kAhead] = pv_read(b, k + kAhead);
      pv_step(k, vf[k], pa, pb, pal, pbl);
      if (sm)
        sm_elems(e0 + 8 * k / kPvSteps, e0 + 8 * (k + 1) / kPvSteps, s_other, mref, qw, qwl, ps,
                 odd);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Softmax elements [e0, e0 + 8) of s alone (a phase without matrix work).
  auto sm_phase = [&](const f32x16& sacc, float mref, int e0, uint32_t pw[8], uint32_t pwl[8],
                      float& ps) {
    float odd = 0.0f;
    sm_elems(e0, e0 + 8, sacc, mref, pw, pwl, ps, odd);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Pad keys (index >= n) of half b to -inf: key 32b + 8(r/4) + 4hl + r%4
  // is a pad key iff its constant part reaches n - 32b - 4hl.
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
  // The exps of a half are taken against the running max as it stands; it
  // is raised only when some lane's sum of the half's 16 probabilities
  // leaves [0, 2^20] (a score far above it, or the row's first block, whose
  // running max is still -inf: then the sum is inf or NaN).
  auto overflowed = [&](float ps) -> bool {
    return __builtin_amdgcn_ballot_w64(!(ps <= 1048576.0f)) != 0;
  };
  // Rare: raise the running max of each row to the half's maximum (the row's
  // two lanes combined), move O and the row sum to it, and redo the half's
  // probabilities and their sum.
  auto redo_half = [&](const f32x16& s, float& ps, uint32_t pw[8], uint32_t pwl[8]) {
    const float mx = max16(s);
    const float mnew = fmaxf(m_run, fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
    m_run = mnew;
    l_run *= alpha;
#pragma unroll
    for (int n = 0; n < NB; ++n) oacc[n] *= alpha;
    float odd = 0.0f;
    sm_elems(0, 16, s, m_run, pw, pwl, ps, odd);
  };

  // An iteration takes one key block as two 32-key halves, or two
  // consecutive visited blocks of at most 32 keys each (a short tile holds
  // one half) as the two halves of one: the first half is always block j's
  // keys 0-31, the second is block j's keys 32-63 or block j2's keys 0-31.
  // The visit order, and so every operation on the running state, is the
  // same either way.  `step` is the number of visits the iteration takes.
  // With 128-token tiles no blocks are paired.
  auto visit_at = [&](int at) -> Visit {
    Visit v;
    v.j = tile_at(at);
    const int n = valid[v.j];
    v.n0 = min(n, 32);
    v.j1 = v.j;
    v.b1 = 1;
    v.n1 = max(n - 32, 0);
    v.step = 1;
    if (bsh == 0 && n <= 32 && at + 1 < end) {
      const int j2 = tile_at(at + 1);
      const int n2 = valid[j2];
      if (n2 <= 32) {
        v.j1 = j2;
        v.b1 = 0;
        v.n1 = n2;
        v.step = 2;
      }
    }
    return v;
  };
  Visit cv{};
  if (beg < end) {
    cv = visit_at(beg);
    VSA_LOAD_KH(lds_ka, cv.j, 0);
    if (cv.n1 > 0) VSA_LOAD_KH(lds_kb, cv.j1, cv.b1);
    VSA_LOAD_VH(lds_va, cv.j, 0);
  }

  // The softmax of each half tile is split in two parts of 8 elements, and
  // the work of tile t runs as four phases of matrix steps, each with one
  // softmax part spread over its steps:
  //   1. Q.K of half 0 of t        | second part of half 1 of t - 1;
  //   2. P.V of half 1 of t - 1    | first part of half 0 of t;
  //   3. Q.K of half 1 of t        | second part of half 0 of t;
  //   4. P.V of half 0 of t        | first part of half 1 of t.
  // A half's running-max check follows its second part, before its P.V, so
  // the softmax, the P.V order and every rounding are those of a tile taken
  // whole.  An extra iteration after the last tile finishes the last half 1.
  // Slots, two syncs per tile: after phase 2 (A) every wave is done with
  // K half 0 of t and V^T half 1 of t - 1, whose slots take K half 0 of t + 1
  // and V^T half 1 of t; after phase 4 (B) every wave is done with K half 1
  // and V^T half 0 of t, whose slots take those of t + 1.  At each sync the
  // loads issued at the previous one have landed (two or three phases to
  // land), and nothing else is in flight.
  uint32_t w0[8], w0l[8], w1[8], w1l[8];   // packed probabilities of halves 0 and 1
  float ps0 = 0.0f, ps1 = 0.0f;
  // S^T of the halves.  The phases take a softmax part whether or not its
  // half exists, so that the common path has no branches; a part taken of
  // a half that does not exist (s1 of a tile whose second half holds no key)
  // is never used.
  f32x16 s0 = {}, s1 = {};
  bool prev1 = false;   // half 1 of the previous tile awaits its second part and P.V
  if (load_state) {
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
  } else {
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[n][r] = 0.0f;
  }
  // K half 0 and 1 and V^T half 0 of the first tile landed (and the query
  // and the running max and sums); the 4 NB loads of O may still be in
  // flight across the barrier (the compiler waits for them before the loop,
  // which uses O).
  if (load_state)
    __builtin_amdgcn_s_waitcnt(kWaitVmO);
  else
    __builtin_amdgcn_s_waitcnt(kWaitVm);
  VSA_BARRIER();
  for (int it = beg;;) {
    const bool cur = it < end;
    const bool has1 = cur && cv.n1 > 0;   // the second half holds a valid key
    // The next iteration (none after the last).  A block without valid keys
    // (only ever the second block of a short 128-token tile) is stepped over.
    int itn = it + cv.step;
    Visit nv = cv;
    nv.n1 = 0;
    if (itn < end) {
      nv = visit_at(itn);
      if (bsh > 0 && nv.n0 == 0) {
        ++itn;
        if (itn < end) {
          nv = visit_at(itn);
        } else {
          nv = cv;
          nv.n1 = 0;
        }
      }
    }
    if (active) {
      // Phase 1.
      if (cur)
        qk_phase(0, s0, true, s1, pinned(m_run), 8, w1, w1l, ps1);
      else
        sm_phase(s1, m_run, 8, w1, w1l, ps1);
      if (prev1) {
        if (overflowed(ps1)) redo_half(s1, ps1, w1, w1l);
        l_run += ps1;
      }
      if (cur && cv.n0 < 32) mask_half(s0, 0, cv.n0);
      // Phase 2.
      if (prev1)
        pv_phase(1, w1, w1l, true, s0, pinned(m_run), 0, w0, w0l, ps0);
      else
        sm_phase(s0, m_run, 0, w0, w0l, ps0);
    }
    if (!cur) break;

    // Sync A: K half 1 and V^T half 0 of t landed.
    __builtin_amdgcn_s_waitcnt(kWaitVm);
    VSA_BARRIER();
    if (itn < end) VSA_LOAD_KH(lds_ka, nv.j, 0);
    if (has1) VSA_LOAD_VH(lds_vb, cv.j1, cv.b1);

    if (active) {
      // Phase 3.
      if (has1)
        qk_phase(1, s1, true, s0, pinned(m_run), 8, w0, w0l, ps0);
      else
        sm_phase(s0, m_run, 8, w0, w0l, ps0);
      if (overflowed(ps0)) redo_half(s0, ps0, w0, w0l);
      l_run += ps0;
      if (has1 && cv.n1 < 32) mask_half(s1, 1, 32 + cv.n1);
      // Phase 4.
      pv_phase(0, w0, w0l, true, s1, pinned(m_run), 0, w1, w1l, ps1);
    }
    prev1 = has1;

    // Sync B: K half 0 of t + 1 and V^T half 1 of t landed.
    __builtin_amdgcn_s_waitcnt(kWaitVm);
    VSA_BARRIER();
    if (itn < end) {
      if (nv.n1 > 0) VSA_LOAD_KH(lds_kb, nv.j1, nv.b1);
      VSA_LOAD_VH(lds_va, nv.j, 0);
    }
    cv = nv;
    it = itn;
  }
  // No global->LDS load may still be in flight when the block's LDS is released.
  __builtin_amdgcn_s_waitcnt(kWaitVm);
#undef VSA_LOAD_KH
#undef VSA_LOAD_VH
#undef VSA_BARRIER
#undef VSA_VLOAD
#undef VSA_KLOAD

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

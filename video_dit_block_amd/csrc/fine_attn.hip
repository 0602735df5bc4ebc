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
//   - one block of 4 waves per (head, query tile); wave w owns query rows
//     16w..16w+15 of the 64-row tile; query rows are gathered straight from
//     the packed [L][H][D] input through the tile's slot table;
//   - the visit list is ascending (prefix tiles 0..P-1, then the selected
//     video tiles), so every row starts from a finite running max;
//   - per key tile: K [64][D] and V^T [D][64] (bf16) are staged in LDS with
//     XOR-swizzled 16-byte chunks (conflict-free MFMA operand reads), the next
//     tile is prefetched into registers meanwhile;
//   - S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys are the M dimension, so
//     each lane holds one query column), online softmax in fp32 via exp2 with
//     the 1/sqrt(D) scale folded into log2 units, P rounded to bf16;
//   - O^T += V^T P^T on the same MFMA; the key order inside each 32-key chunk
//     is permuted identically in both operands so that P^T is consumed
//     straight from the S^T accumulator layout, without a shuffle.
//   - blocks are mapped to the 8 XCDs so that each XCD works through its own
//     heads, head by head, prefix (long) items first: the 32 CUs of an XCD
//     sweep the same head's K/V, which keeps it hot in that XCD's L2.
#include "device.hpp"
#include "kernels.hpp"

namespace vsa {

namespace {

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

// (head, query tile) of block b.  With heads divisible by 8, XCD x (blocks
// b = x mod 8) owns heads x, x+8, ...; inside an XCD, the prefix items of its
// heads come first, then the video items head by head.
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

template <typename TIO, int D>
__global__ __launch_bounds__(256, 2) void fine_attn_kernel(FineArgs a) {
  constexpr int KCH = D / 32;        // 16-byte chunks per thread per K (or V) tile
  constexpr int KROW = D / 8;        // 16-byte chunks per K row
  constexpr int NB = D / 16;         // O^T blocks of 16 channels
  __shared__ __attribute__((aligned(16))) uint16_t ks[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs[D * 64];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int ln = lane & 15;
  const int H = a.H, Nt = a.Nt, P = a.P, NV = a.NV, topk = a.topk;

  int h, i;
  decode_item(blockIdx.x, H, P, NV, h, i);

  const TIO* q = static_cast<const TIO*>(a.q);
  const int slot_q = 16 * w + ln;
  const int pr = a.perm[static_cast<size_t>(i) * 64 + slot_q];

  // Query fragment: B operand of S^T = K Q^T (column = query, k = channel).
  bf16x8 qf[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    if (pr >= 0) {
      qf[c] = IoOps<TIO>::load8(q + (static_cast<size_t>(pr) * H + h) * D + 32 * c + 8 * g);
    } else {
      qf[c] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  const int nlist = i < P ? Nt : P + topk;
  const int32_t* sl = i < P ? nullptr : a.sel + (static_cast<size_t>(h) * NV + (i - P)) * topk;
  const uint16_t* kth = a.kt + static_cast<size_t>(h) * Nt * 64 * D;
  const uint16_t* vth = a.vt + static_cast<size_t>(h) * Nt * 64 * D;

  // Listed ids are clamped into [0, Nt): a corrupt list can give a wrong
  // result but never an out-of-bounds read.
  auto tile_at = [&](int it) -> int {
    const int t = (sl == nullptr || it < P) ? it : sl[it - P];
    return min(max(t, 0), Nt - 1);
  };

  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  f32x4 oacc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) oacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.0f;

  // Register prefetch of the next K / V^T tile (16-byte chunks, coalesced).
  u32x4 kr[KCH], vr[KCH];
  int j = tile_at(0);
  {
    const u32x4* kg = reinterpret_cast<const u32x4*>(kth + static_cast<size_t>(j) * 64 * D);
    const u32x4* vg = reinterpret_cast<const u32x4*>(vth + static_cast<size_t>(j) * 64 * D);
#pragma unroll
    for (int e = 0; e < KCH; ++e) {
      kr[e] = kg[e * 256 + tid];
      vr[e] = vg[e * 256 + tid];
    }
  }
  for (int it = 0; it < nlist; ++it) {
    const int nj = a.valid[j];
#pragma unroll
    for (int e = 0; e < KCH; ++e) {
      const int id = e * 256 + tid;
      const int key = id / KROW, ch = id % KROW;
      reinterpret_cast<u32x4*>(ks)[key * KROW + (ch ^ (key & (KROW - 1)))] = kr[e];
      const int d = id >> 3, cv = id & 7;
      reinterpret_cast<u32x4*>(vs)[d * 8 + (cv ^ ((d >> 1) & 7))] = vr[e];
    }
    __syncthreads();
    // Next tile (the last iteration re-reads the current one instead of branching).
    const int jn = it + 1 < nlist ? tile_at(it + 1) : j;
    {
      const u32x4* kg = reinterpret_cast<const u32x4*>(kth + static_cast<size_t>(jn) * 64 * D);
      const u32x4* vg = reinterpret_cast<const u32x4*>(vth + static_cast<size_t>(jn) * 64 * D);
#pragma unroll
      for (int e = 0; e < KCH; ++e) {
        kr[e] = kg[e * 256 + tid];
        vr[e] = vg[e * 256 + tid];
      }
    }

    // S^T block b: keys 16b..16b+15 (rows) x this wave's 16 queries (columns).
    f32x4 sacc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      sacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = 16 * b + ln;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const int ch = (4 * c + g) ^ (key & (KROW - 1));
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + key * D + ch * 8);
        sacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], sacc[b], 0, 0, 0);
      }
    }
    // Lane holds keys 16b + 4g + r of query column ln.
    if (nj < 64) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * b + 4 * g + r >= nj) sacc[b][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[b][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float p[4][4];
    float psum = 0.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[b][r] = __builtin_amdgcn_exp2f(fmaf(sacc[b][r], scale_log2, -m_new));
        psum += p[b][r];
      }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int n = 0; n < NB; ++n) oacc[n] *= alpha;

    // O^T += V^T P^T over two 32-key chunks.  k-slot 8g+e <-> key
    // 32*c2 + 16*(e/4) + 4g + e%4, in both operands.
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      u32x4 pu;
      pu.x = pack_bf16x2(p[2 * c2][0], p[2 * c2][1]);
      pu.y = pack_bf16x2(p[2 * c2][2], p[2 * c2][3]);
      pu.z = pack_bf16x2(p[2 * c2 + 1][0], p[2 * c2 + 1][1]);
      pu.w = pack_bf16x2(p[2 * c2 + 1][2], p[2 * c2 + 1][3]);
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pu);
      const int c8a = 8 * c2 + g, c8b = 8 * c2 + 4 + g;
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const int d = 16 * n + ln;
        const uint16_t* row = vs + d * 64;
        const int sw = (d >> 1) & 7;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(row + (((c8a >> 1) ^ sw) * 8 + (c8a & 1) * 4));
        const u32x2 hi = *reinterpret_cast<const u32x2*>(row + (((c8b >> 1) ^ sw) * 8 + (c8b & 1) * 4));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[n], 0, 0, 0);
      }
    }
    __syncthreads();
    j = jn;
  }

  // Epilogue: normalise, add gate * coarse, store at the packed row.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (pr >= 0) {
    const float inv = 1.0f / l_run;
    const float* cg = a.coarse + (static_cast<size_t>(h) * Nt + i) * D;
    const size_t rowoff = (static_cast<size_t>(pr) * H + h) * D;
    const TIO* gate = static_cast<const TIO*>(a.gate) + rowoff;
    TIO* out = static_cast<TIO*>(a.out) + rowoff;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int d0 = 16 * n + 4 * g;
      const float4 cc = *reinterpret_cast<const float4*>(cg + d0);
      float gv[4];
      IoOps<TIO>::load4(gate + d0, gv);
      float res[4];
      res[0] = fmaf(gv[0], cc.x, oacc[n][0] * inv);
      res[1] = fmaf(gv[1], cc.y, oacc[n][1] * inv);
      res[2] = fmaf(gv[2], cc.z, oacc[n][2] * inv);
      res[3] = fmaf(gv[3], cc.w, oacc[n][3] * inv);
      IoOps<TIO>::store4(out + d0, res);
    }
  }
}

template <typename TIO, int D>
hipError_t launch(const FineArgs& a, hipStream_t stream) {
  const int blocks = a.H * a.Nt;
  hipLaunchKernelGGL((fine_attn_kernel<TIO, D>), dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fine(const FineArgs& a, hipStream_t stream) {
  if (a.io_f32) return a.D == 64 ? launch<float, 64>(a, stream) : launch<float, 128>(a, stream);
  return a.D == 64 ? launch<uint16_t, 64>(a, stream) : launch<uint16_t, 128>(a, stream);
}

}  // namespace vsa

// Tile-permute gather with fused tile mean-pooling.
//
// FastH3 NVFP4 on RTX PRO 6000, "Model integration": the attention input is
// gathered into tile order once, with pad rows left at zero.  FastH3 4-step
// Preview, "Video Sparse Attention is not optional here": tile scores come
// from pooled q and k in fp32, and the compression branch uses pool(v).
//
// One block per (head, tile).  A tile is one or two 64-slot blocks (64- or
// 128-token tiles; block b holds slots 64b..64b+63).  For each block in turn
// its 64 slots of q, k and v are staged in LDS (pad slots zero), then
//   - k is written to Kt (bf16): per 64-slot block, each 32-slot half is
//     stored in the order the fine kernel stages it in LDS, [group][32
//     slots][64 bytes] with a group being 64 bytes of a key row (32 channels;
//     64 channels of FP8 codes), so that every 1 KB DMA load of the fine
//     kernel reads 1 KB of contiguous memory,
//   - v is written transposed to Vt[h][tile][half][d][pos] (bf16, positions
//     0-31 and 32-63 in two halves, so that the fine kernel can fetch a half
//     tile as one block), the layout its P.V operand wants: inside each group of 16 slots the
//     storage order is slots 0-3, 8-11, 4-7, 12-15 (bits 2 and 3 of the slot
//     swapped), so that the 8 keys one MFMA lane contracts over are adjacent;
//   - q, k, v are mean-pooled per channel: a sequential fp32 sum over the
//     tile's valid slots in slot order (carried from block to block), then
//     one correctly rounded division by the count.  That fixed order makes
//     the pooled values, and therefore the top-k selection, reproducible bit
//     for bit.
// q itself is not permuted: the fine kernel gathers query rows directly.
//
// Optionally (PREP) q and k are first put through QK-norm and RoPE on the
// staged rows (FastH3 NVFP4 on RTX PRO 6000, "Model integration": both are
// applied to tile-ordered q and k with per-step cos/sin tables; pad rows stay
// zero), in a fixed fp32 order so that the pooled values stay reproducible:
//   ss = sum_d x_d * x_d (sequential, separately rounded), inv = 1 /
//   sqrt(ss / D + eps) (each step correctly rounded), y_d = (x_d * inv) * w_d,
//   then each interleaved pair (a, b) = (y_2i, y_2i+1) becomes
//   (a*c - b*s, a*s + b*c) with the token's cos/sin;
// the results replace the staged rows (rounded to the I/O type), so pooling,
// Kt and the tile-ordered copy of q (Qt, for the fine kernel) all use them.
//
// With fp32 I/O the tile-ordered operands are also written as low parts
// lo = bf16(x - bf16(x)) next to the bf16 high parts (Kt_lo, Vt_lo, Qt_lo,
// same layouts), so that the fine kernel can form fp32-accurate products from
// bf16 matrix-core terms.
#include "device.hpp"
#include "kernels.hpp"

namespace vsa {

namespace {

__device__ __forceinline__ void store_pair(uint16_t* p, float a, float b) {
  *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
}
__device__ __forceinline__ void store_pair(float* p, float a, float b) {
  p[0] = a;
  p[1] = b;
}

template <typename T, int D, bool PREP>
__global__ __launch_bounds__(384) void permute_pool_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ valid, int H, int Nt, int bsh,
    uint16_t* __restrict__ kt, uint16_t* __restrict__ vt, float* __restrict__ qp,
    float* __restrict__ kp, float* __restrict__ vp, QkPrepArgs prep, uint8_t* __restrict__ kt8,
    float* __restrict__ kscale, uint16_t* __restrict__ kt_lo, uint16_t* __restrict__ vt_lo) {
  // Low parts exist only for fp32 inputs.
  constexpr bool kLo = sizeof(T) == 4;
  constexpr int kRowBytes = D * static_cast<int>(sizeof(T));
  constexpr int kChunksPerRow = kRowBytes / 16;
  constexpr int kChunksPerTensor = 64 * kChunksPerRow;
  // Rows padded by 16 bytes: the per-row norm pass reads one column of 64
  // rows at a time, which would otherwise fall into a single LDS bank.
  constexpr int kPad = 16 / static_cast<int>(sizeof(T));
  __shared__ __attribute__((aligned(16))) T lds[3][64][D + kPad];

  const int h = blockIdx.x;
  const int tile = blockIdx.y;
  const int tid = threadIdx.x;
  const int Nb = Nt << bsh;
  __shared__ int sperm[64];
  // Pooling: one thread per (tensor, channel), fp32 sum over the tile's slots.
  float pacc = 0.0f;
  int ntile = 0;

  for (int blk = 0; blk < (1 << bsh); ++blk) {
    const int j = (tile << bsh) + blk;   // block
    const int n = valid[j];
    ntile += n;
    const int32_t* tperm = perm + static_cast<size_t>(j) * 64;

    // Stage q, k, v rows of this block (16-byte chunks, a whole row contiguous
    // in memory): the slot table first, then every load of this thread before
    // any LDS store, so that the loads are in flight together.
    if (tid < 64) sperm[tid] = tid < n ? tperm[tid] : -1;
    __syncthreads();
    static_assert((3 * kChunksPerTensor) % 384 == 0, "staging split");
    constexpr int PER = 3 * kChunksPerTensor / 384;
    uint4 val[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int c = tid + 384 * r;
      const int x = c / kChunksPerTensor;
      const int rem = c - x * kChunksPerTensor;
      const int slot = rem / kChunksPerRow;
      const int part = rem - slot * kChunksPerRow;
      const T* src = x == 0 ? q : (x == 1 ? k : v);
      const int row = sperm[slot];
      val[r] = make_uint4(0, 0, 0, 0);
      if (row >= 0)
        val[r] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(src) +
                                                 (static_cast<size_t>(row) * H + h) * kRowBytes +
                                                 part * 16);
    }
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int c = tid + 384 * r;
      const int x = c / kChunksPerTensor;
      const int rem = c - x * kChunksPerTensor;
      const int slot = rem / kChunksPerRow;
      const int part = rem - slot * kChunksPerRow;
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(&lds[x][slot][0]) + part * 16) = val[r];
    }
    __syncthreads();

    if constexpr (PREP) {
      __shared__ float rinv[2][64];
      // Each thread's cos/sin entries for the rotation below, requested up
      // front so that they arrive while the norms are computed (q and k of one
      // (slot, pair) share them).
      constexpr int PAIRS = D / 2;
      constexpr int ITER = (64 * PAIRS + 383) / 384;
      float cs[ITER], sn[ITER];
#pragma unroll
      for (int r = 0; r < ITER; ++r) {
        const int c = tid + 384 * r;
        const int s = c / PAIRS;
        cs[r] = 1.0f;
        sn[r] = 0.0f;
        if (c < 64 * PAIRS && s < n) {
          const size_t t = static_cast<size_t>(sperm[s]) * PAIRS + (c - s * PAIRS);
          cs[r] = prep.cos[t];
          sn[r] = prep.sin[t];
        }
      }
      // Inverse RMS of every valid q and k row, one thread per row.
      if (tid < 128) {
        const int x = tid >> 6, s = tid & 63;
        float inv = 0.0f;
        if (s < n) {
#pragma clang fp contract(off)
          float ss = 0.0f;
          for (int d = 0; d < D; ++d) {
            const float e = to_f32(lds[x][s][d]);
            ss = ss + e * e;
          }
          const float ms = __fdiv_rn(ss, static_cast<float>(D));
          inv = __fdiv_rn(1.0f, __builtin_sqrtf(ms + prep.eps));   // IEEE (correctly rounded)
        }
        rinv[x][s] = inv;
      }
      __syncthreads();
      // Scale, weight and rotate every interleaved pair of the valid rows.
#pragma unroll
      for (int r = 0; r < ITER; ++r) {
        const int c = tid + 384 * r;
        const int s = c / PAIRS;
        const int i = c - s * PAIRS;
        if (c < 64 * PAIRS && s < n) {
#pragma unroll
          for (int x = 0; x < 2; ++x) {
#pragma clang fp contract(off)
            const float inv = rinv[x][s];
            const float* w = x == 0 ? prep.q_weight : prep.k_weight;
            const float a = (to_f32(lds[x][s][2 * i]) * inv) * w[2 * i];
            const float b = (to_f32(lds[x][s][2 * i + 1]) * inv) * w[2 * i + 1];
            store_pair(&lds[x][s][2 * i], a * cs[r] - b * sn[r], a * sn[r] + b * cs[r]);
          }
        }
      }
      __syncthreads();
    }

    const size_t tile_base = static_cast<size_t>(h) * Nb + j;   // block row of Kt, Vt, ...

    // Pool: continue the sequential fp32 sum in slot order.
    if (tid < 3 * D) {
#pragma clang fp contract(off)
      const int x = tid / D;
      const int d = tid - x * D;
      for (int s = 0; s < n; ++s) pacc = pacc + to_f32(lds[x][s][d]);
    }

    // Keys as per-token FP8 (OCP E4M3) codes instead of bf16: amax of each
    // valid row, codes of x * (448 / amax) (the division correctly rounded, the
    // product rounded to fp32, the conversion to nearest even), and the
    // dequantisation scale amax / 448; pad rows get zero codes and scale.
    if (kt8) {
      __shared__ float kinv[64];
      if (tid < 64) {
        float amax = 0.0f;
        if (tid < n)
          for (int d = 0; d < D; ++d) amax = fmaxf(amax, fabsf(to_f32(lds[1][tid][d])));
        kinv[tid] = amax > 0.0f ? __fdiv_rn(448.0f, amax) : 0.0f;
        kscale[tile_base * 64 + tid] = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 0.0f;
      }
      __syncthreads();
      // Codes in the Kt order: chunk c of 16 bytes is chunk c % 4 of slot
      // 32 * half + (c / 4) % 32 in group (c / 128) % (D / 64) of 64 codes.
      uint8_t* dst = kt8 + tile_base * 64 * D;
      for (int c = tid; c < 64 * (D / 16); c += blockDim.x) {
        const int g = (c >> 7) % (D / 64);
        const int slot = 32 * ((c >> 7) / (D / 64)) + ((c >> 2) & 31);
        const int d0 = 64 * g + 16 * (c & 3);
        const float inv = kinv[slot];
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const T* e = &lds[1][slot][d0 + 4 * j];
          uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(to_f32(e[0]) * inv, to_f32(e[1]) * inv, 0,
                                                       false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(to_f32(e[2]) * inv, to_f32(e[3]) * inv, w, true);
          o[j] = w;
        }
        *reinterpret_cast<u32x4*>(dst + static_cast<size_t>(c) * 16) = o;
      }
    }

    // Qt (with PREP): [slot][d] bf16; Kt: 16-byte chunk c (8 channels) is
    // chunk c % 4 of slot 32 * half + (c / 4) % 32 in group (c / 128) % (D / 32)
    // of 32 channels.  Consecutive threads write consecutive chunks.
    for (int x = PREP ? 0 : 1; x < (kt8 ? 1 : 2); ++x) {
      uint16_t* dst = (x == 0 ? prep.qt : kt) + tile_base * 64 * D;
      uint16_t* dlo = (x == 0 ? prep.qt_lo : kt_lo) + tile_base * 64 * D;
      for (int c = tid; c < 64 * (D / 8); c += blockDim.x) {
        int slot, d0;
        if (x == 0) {
          slot = c / (D / 8);
          d0 = (c - slot * (D / 8)) * 8;
        } else {
          slot = 32 * ((c >> 7) / (D / 32)) + ((c >> 2) & 31);
          d0 = 32 * ((c >> 7) % (D / 32)) + 8 * (c & 3);
        }
        const T* e = &lds[x][slot][d0];
        uint4 o;
        o.x = pack_bf16x2(to_f32(e[0]), to_f32(e[1]));
        o.y = pack_bf16x2(to_f32(e[2]), to_f32(e[3]));
        o.z = pack_bf16x2(to_f32(e[4]), to_f32(e[5]));
        o.w = pack_bf16x2(to_f32(e[6]), to_f32(e[7]));
        const size_t at = x == 0 ? static_cast<size_t>(slot) * D + d0 : static_cast<size_t>(c) * 8;
        *reinterpret_cast<uint4*>(dst + at) = o;
        if constexpr (kLo) {
          o.x = pack_bf16x2_lo(e[0], e[1]);
          o.y = pack_bf16x2_lo(e[2], e[3]);
          o.z = pack_bf16x2_lo(e[4], e[5]);
          o.w = pack_bf16x2_lo(e[6], e[7]);
          *reinterpret_cast<uint4*>(dlo + at) = o;
        }
      }
    }
    // Vt: two halves of positions (0-31, 32-63), each [d][32] bf16 with
    // 16-byte chunks of 8 positions.  Positions p0..p0+7 (p0 = 8m) hold slots
    // 16(m/2) + 4(m%2) + {0..3} and the same + 8.  Consecutive threads write
    // consecutive 16-byte chunks (the four chunks of a row d, then row d+1).
    {
      uint16_t* dst = vt + tile_base * 64 * D;
      for (int c = tid; c < D * 8; c += blockDim.x) {
        const int d = (c >> 2) % D;
        const int m = 4 * ((c >> 2) / D) + (c & 3);
        const int sa = 16 * (m >> 1) + 4 * (m & 1);
        const int sb = sa + 8;
        const size_t at = static_cast<size_t>(m >> 2) * 32 * D + d * 32 + 8 * (m & 3);
        uint4 o;
        o.x = pack_bf16x2(to_f32(lds[2][sa + 0][d]), to_f32(lds[2][sa + 1][d]));
        o.y = pack_bf16x2(to_f32(lds[2][sa + 2][d]), to_f32(lds[2][sa + 3][d]));
        o.z = pack_bf16x2(to_f32(lds[2][sb + 0][d]), to_f32(lds[2][sb + 1][d]));
        o.w = pack_bf16x2(to_f32(lds[2][sb + 2][d]), to_f32(lds[2][sb + 3][d]));
        *reinterpret_cast<uint4*>(dst + at) = o;
        if constexpr (kLo) {
          o.x = pack_bf16x2_lo(lds[2][sa + 0][d], lds[2][sa + 1][d]);
          o.y = pack_bf16x2_lo(lds[2][sa + 2][d], lds[2][sa + 3][d]);
          o.z = pack_bf16x2_lo(lds[2][sb + 0][d], lds[2][sb + 1][d]);
          o.w = pack_bf16x2_lo(lds[2][sb + 2][d], lds[2][sb + 3][d]);
          *reinterpret_cast<uint4*>(vt_lo + tile_base * 64 * D + at) = o;
        }
      }
    }
    // Every read of this block's LDS rows is done before the next block's staging.
    __syncthreads();
  }

  if (tid < 3 * D) {
    const int x = tid / D;
    const int d = tid - x * D;
    float* dst = x == 0 ? qp : (x == 1 ? kp : vp);
    dst[(static_cast<size_t>(h) * Nt + tile) * D + d] = __fdiv_rn(pacc, static_cast<float>(ntile));
  }
}

template <typename T, int D>
hipError_t launch(const PermutePoolArgs& a, hipStream_t stream) {
  dim3 grid(a.H, a.Nt);   // one block per (head, tile)
  if (a.prep.qt)
    hipLaunchKernelGGL((permute_pool_kernel<T, D, true>), grid, dim3(384), 0, stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.perm, a.valid, a.H, a.Nt, a.bsh, a.kt, a.vt,
                       a.qp, a.kp, a.vp, a.prep, a.kt8, a.kscale, a.kt_lo, a.vt_lo);
  else
    hipLaunchKernelGGL((permute_pool_kernel<T, D, false>), grid, dim3(384), 0, stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.perm, a.valid, a.H, a.Nt, a.bsh, a.kt, a.vt,
                       a.qp, a.kp, a.vp, a.prep, a.kt8, a.kscale, a.kt_lo, a.vt_lo);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute_pool(const PermutePoolArgs& a, hipStream_t stream) {
  if (a.io_f32) return a.D == 64 ? launch<float, 64>(a, stream) : launch<float, 128>(a, stream);
  return a.D == 64 ? launch<uint16_t, 64>(a, stream) : launch<uint16_t, 128>(a, stream);
}

}  // namespace vsa

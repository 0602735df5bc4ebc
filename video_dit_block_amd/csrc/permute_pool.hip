// Tile-permute gather with fused tile mean-pooling.
//
// FastH3 NVFP4 on RTX PRO 6000, "Model integration": the attention input is
// gathered into tile order once, with pad rows left at zero.  FastH3 4-step
// Preview, "Video Sparse Attention is not optional here": tile scores come
// from pooled q and k in fp32, and the compression branch uses pool(v).
//
// One block per (head, tile).  The tile's 64 slots of q, k and v are staged
// in LDS (pad slots zero), then
//   - k is written to Kt[h][tile][slot][d] (bf16),
//   - v is written transposed to Vt[h][tile][d][pos] (bf16), the layout the
//     fine kernel's P.V operand wants: inside each group of 16 slots the
//     storage order is slots 0-3, 8-11, 4-7, 12-15 (bits 2 and 3 of the slot
//     swapped), so that the 8 keys one MFMA lane contracts over are adjacent;
//   - q, k, v are mean-pooled per channel: a sequential fp32 sum over the
//     valid slots in slot order, then one correctly rounded division by the
//     count.  That fixed order makes the pooled values, and therefore the
//     top-k selection, reproducible bit for bit.
// q itself is not permuted: the fine kernel gathers query rows directly.
#include "device.hpp"
#include "kernels.hpp"

namespace vsa {

namespace {

template <typename T, int D>
__global__ __launch_bounds__(384) void permute_pool_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ valid, int H, int Nt,
    uint16_t* __restrict__ kt, uint16_t* __restrict__ vt, float* __restrict__ qp,
    float* __restrict__ kp, float* __restrict__ vp) {
  constexpr int kRowBytes = D * static_cast<int>(sizeof(T));
  constexpr int kChunksPerRow = kRowBytes / 16;
  constexpr int kChunksPerTensor = 64 * kChunksPerRow;
  __shared__ __attribute__((aligned(16))) T lds[3][64][D];

  const int h = blockIdx.x;
  const int j = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = valid[j];
  const int32_t* tperm = perm + static_cast<size_t>(j) * 64;

  // Stage q, k, v rows of this tile (16-byte chunks, 256 B contiguous per row).
  for (int c = tid; c < 3 * kChunksPerTensor; c += blockDim.x) {
    const int x = c / kChunksPerTensor;
    const int rem = c - x * kChunksPerTensor;
    const int slot = rem / kChunksPerRow;
    const int part = rem - slot * kChunksPerRow;
    const T* src = x == 0 ? q : (x == 1 ? k : v);
    uint4 val = make_uint4(0, 0, 0, 0);
    const int r = slot < n ? tperm[slot] : -1;
    if (r >= 0) {
      const char* p = reinterpret_cast<const char*>(src) +
                      (static_cast<size_t>(r) * H + h) * kRowBytes + part * 16;
      val = *reinterpret_cast<const uint4*>(p);
    }
    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(&lds[x][slot][0]) + part * 16) = val;
  }
  __syncthreads();

  const size_t tile_base = static_cast<size_t>(h) * Nt + j;

  // Pool: one thread per (tensor, channel), sequential fp32 sum in slot order.
  if (tid < 3 * D) {
    const int x = tid / D;
    const int d = tid - x * D;
    float acc = 0.0f;
    {
#pragma clang fp contract(off)
      for (int s = 0; s < n; ++s) acc = acc + to_f32(lds[x][s][d]);
    }
    const float mean = __fdiv_rn(acc, static_cast<float>(n));
    float* dst = x == 0 ? qp : (x == 1 ? kp : vp);
    dst[tile_base * D + d] = mean;
  }

  // Kt: [slot][d] bf16, 16-byte chunks of 8 channels.
  {
    uint16_t* dst = kt + tile_base * 64 * D;
    for (int c = tid; c < 64 * (D / 8); c += blockDim.x) {
      const int slot = c / (D / 8);
      const int d0 = (c - slot * (D / 8)) * 8;
      uint4 o;
      o.x = pack_bf16x2(to_f32(lds[1][slot][d0 + 0]), to_f32(lds[1][slot][d0 + 1]));
      o.y = pack_bf16x2(to_f32(lds[1][slot][d0 + 2]), to_f32(lds[1][slot][d0 + 3]));
      o.z = pack_bf16x2(to_f32(lds[1][slot][d0 + 4]), to_f32(lds[1][slot][d0 + 5]));
      o.w = pack_bf16x2(to_f32(lds[1][slot][d0 + 6]), to_f32(lds[1][slot][d0 + 7]));
      *reinterpret_cast<uint4*>(dst + static_cast<size_t>(slot) * D + d0) = o;
    }
  }
  // Vt: [d][pos] bf16, 16-byte chunks of 8 positions.  Positions p0..p0+7
  // (p0 = 8m) hold slots 16(m/2) + 4(m%2) + {0..3} and the same + 8.
  {
    uint16_t* dst = vt + tile_base * 64 * D;
    for (int c = tid; c < D * 8; c += blockDim.x) {
      const int d = c % D;
      const int m = c / D;
      const int sa = 16 * (m >> 1) + 4 * (m & 1);
      const int sb = sa + 8;
      uint4 o;
      o.x = pack_bf16x2(to_f32(lds[2][sa + 0][d]), to_f32(lds[2][sa + 1][d]));
      o.y = pack_bf16x2(to_f32(lds[2][sa + 2][d]), to_f32(lds[2][sa + 3][d]));
      o.z = pack_bf16x2(to_f32(lds[2][sb + 0][d]), to_f32(lds[2][sb + 1][d]));
      o.w = pack_bf16x2(to_f32(lds[2][sb + 2][d]), to_f32(lds[2][sb + 3][d]));
      *reinterpret_cast<uint4*>(dst + static_cast<size_t>(d) * 64 + 8 * m) = o;
    }
  }
}

template <typename T, int D>
hipError_t launch(const PermutePoolArgs& a, hipStream_t stream) {
  dim3 grid(a.H, a.Nt);
  hipLaunchKernelGGL((permute_pool_kernel<T, D>), grid, dim3(384), 0, stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), a.perm, a.valid, a.H, a.Nt, a.kt, a.vt, a.qp,
                     a.kp, a.vp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute_pool(const PermutePoolArgs& a, hipStream_t stream) {
  if (a.io_f32) return a.D == 64 ? launch<float, 64>(a, stream) : launch<float, 128>(a, stream);
  return a.D == 64 ? launch<uint16_t, 64>(a, stream) : launch<uint16_t, 128>(a, stream);
}

}  // namespace vsa

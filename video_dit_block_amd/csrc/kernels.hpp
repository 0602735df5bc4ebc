// Launch interfaces of the gfx950 kernels of the VSA-H3 forward (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {

// Optional QK-norm + RoPE applied while gathering (all null: not applied).
struct QkPrepArgs {
  const float *q_weight, *k_weight;  // [D]
  const float *cos, *sin;            // [L][D/2], packed token order
  float eps;
  uint16_t* qt;                      // [H][Nt][64][D] bf16: normalised, rotated q
};

struct PermutePoolArgs {
  const void *q, *k, *v;        // [L][H][D], bf16 or fp32
  bool io_f32;
  const int32_t* perm;          // [Nt][64]
  const int32_t* valid;         // [Nt]
  int H, Nt, D;
  uint16_t *kt, *vt;            // [H][Nt][64][D], [H][Nt][D][64] bf16
  float *qp, *kp, *vp;          // [H][Nt][D]
  QkPrepArgs prep;
  uint8_t* kt8;                 // [H][Nt][64][D] E4M3 keys instead of kt, or null
  float* kscale;                // [H][Nt][64] per-key scale (with kt8)
};
hipError_t launch_permute_pool(const PermutePoolArgs& a, hipStream_t stream);

struct CoarseArgs {
  const float *qp, *kp, *vp;    // [H][Nt][D]
  float* scores;                // [H][Nt][Ns]
  float* coarse;                // [H][Nt][D]
  int32_t* sel;                 // [H][NV][topk]
  int32_t* choff;               // [H][NV][nchunks + 1], written if nchunks > 1
  int H, Nt, Ns, P, NV, topk, D;
  int nchunks, chunk_tiles;
};
hipError_t launch_coarse(const CoarseArgs& a, hipStream_t stream);

struct FineArgs {
  const void* q;                // [L][H][D] io dtype (unused if qt is set)
  const uint16_t* qt;           // [H][Nt][64][D] bf16 tile-ordered q, or null
  const void* gate;             // [L][H][D] io dtype
  void* out;                    // [L][H][D] io dtype
  bool io_f32;
  const uint16_t* kt;           // [H][Nt][64][D] bf16
  const uint16_t* vt;           // [H][Nt][D][64] bf16
  const float* coarse;          // [H][Nt][D]
  const int32_t* perm;          // [Nt][64]
  const int32_t* valid;         // [Nt]
  const int32_t* sel;           // [H][NV][topk]
  const int32_t* choff;         // [H][NV][nchunks + 1] (nchunks > 1)
  float* state;                 // running softmax state between chunks (nchunks > 1)
  int H, Nt, P, NV, topk, D;
  int nchunks, chunk_tiles;
  const uint8_t* kt8;           // [H][Nt][64][D] E4M3 keys: FP8 Q/K logits, or null
  const float* kscale;          // [H][Nt][64]
};
hipError_t launch_fine(const FineArgs& a, hipStream_t stream);

}  // namespace vsa

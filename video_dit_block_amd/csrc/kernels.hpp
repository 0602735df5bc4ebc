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
  uint16_t* qt;                      // [H][Nb][64][D] bf16: normalised, rotated q
  uint16_t* qt_lo;                   // fp32 I/O: low bf16 parts of qt, or null
};

// Nt counts tiles; a tile is 1 << bsh blocks of 64 slots (bsh 0: 64-token
// tiles, 1: 128-token tiles), Nb = Nt << bsh blocks.
struct PermutePoolArgs {
  const void *q, *k, *v;        // [L][H][D], bf16 or fp32
  bool io_f32;
  const int32_t* perm;          // [Nb][64]
  const int32_t* valid;         // [Nb] valid slots per block
  int H, Nt, D, bsh;
  uint16_t *kt, *vt;            // [H][Nb][2][D/32][32][32], [H][Nb][2][D][32] bf16
  float *qp, *kp, *vp;          // [H][Nt][D]
  QkPrepArgs prep;
  uint8_t* kt8;                 // [H][Nb][2][D/64][32][64] E4M3 keys instead of kt, or null
  float* kscale;                // [H][Nb][64] per-key scale (with kt8)
  // fp32 I/O: low parts lo = bf16(x - bf16(x)) of the keys (layout of kt; not
  // with kt8) and values (layout of vt); null for bf16 I/O.
  uint16_t *kt_lo, *vt_lo;
};
hipError_t launch_permute_pool(const PermutePoolArgs& a, hipStream_t stream);

constexpr int32_t kKindRefTile = 1;
struct CoarseArgs {
  const float *qp, *kp, *vp;    // [H][Nt][D]
  float* scores;                // [H][Nt][Ns]
  float* coarse;                // [H][Nt][D]
  int32_t* sel;                 // [H][NV][topk_ref + topk]: selected reference, then video tiles
  int32_t* choff;               // [H][NV][nchunks + 1], written if nchunks > 1
  int H, Nt, Ns, P, NV, topk, D;
  int nchunks, chunk_tiles;
  // Reference selection (topk_ref > 0): kind [Nt] marks the reference tiles
  // (value kKindRefTile);
  // visit [H][NV][visit_len] receives every key tile a video query visits
  // (fixed prefix, selected reference and video tiles, ascending), and choff
  // then counts entries of visit instead of sel.
  const int32_t* kind;
  int topk_ref;
  int32_t* visit;
  int visit_len;
  // With nchunks > 1: order [H][nchunks][Nt] receives each head's query
  // tiles sorted by their visits in the chunk, most first (the fine branch
  // dispatches them in that order); the fine list holds tiles 0..Pvis-1
  // implicitly.
  int32_t* order;
  int Pvis;
};
hipError_t launch_coarse(const CoarseArgs& a, hipStream_t stream);

// Key tiles visited by a video query tile: tiles 0..Pvis-1, then its row of
// `list` (listlen tile ids, ascending); a prefix query tile visits every tile.
struct FineArgs {
  const void* q;                // [L][H][D] io dtype (unused if qt is set)
  const uint16_t* qt;           // [H][Nb][64][D] bf16 tile-ordered q, or null
  const void* gate;             // [L][H][D] io dtype
  void* out;                    // [L][H][D] io dtype
  bool io_f32;
  const uint16_t* kt;           // [H][Nb][2][D/32][32][32] bf16: per 32-key half, 32-channel groups
  const uint16_t* vt;           // [H][Nb][2][D][32] bf16
  const float* coarse;          // [H][Nt][D]
  const int32_t* perm;          // [Nb][64]
  const int32_t* valid;         // [Nb]
  const int32_t* list;          // [H][NV][listlen]
  const int32_t* choff;         // [H][NV][nchunks + 1] (nchunks > 1): list entries below
                                // each chunk boundary
  float* state;                 // running softmax state between chunks (nchunks > 1)
  int H, Nt, P, NV, listlen, D;
  int nchunks, chunk_tiles;
  const uint8_t* kt8;           // [H][Nb][2][D/64][32][64] E4M3 keys: FP8 Q/K logits, or null
  const float* kscale;          // [H][Nb][64]
  int bsh, Pvis;
  const int32_t* order;         // [H][nchunks][Nt] dispatch order of query tiles (nchunks > 1)
  // fp32 I/O: low bf16 parts of kt, vt and qt (each null where its high part
  // is unused); every product is then formed from hi and lo terms.
  const uint16_t *kt_lo, *vt_lo, *qt_lo;
};
hipError_t launch_fine(const FineArgs& a, hipStream_t stream);

}  // namespace vsa

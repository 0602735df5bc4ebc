// Host-side plan of the VSA-H3 forward: tile geometry, device tables and the
// workspace layout.  Pure C++ (no HIP calls), so it can be built and tested
// on a machine without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "vsa_h3.h"

namespace vsa {

constexpr int kTile = 64;          // tokens per block: the unit of the gather and fine kernels
                                   // (a 64-token tile is one block, a 128-token tile two)
constexpr int kMaxTilesCoarse = 4096;  // key tiles one wave can hold in the coarse/top-k kernel
constexpr int kMaxKeyChunks = 63;      // chunk boundaries one wave writes per query tile
// K+V bytes of one head's key chunk in the fine branch.  All query tiles of a
// head sweep a chunk together, so the eight XCDs' current chunks (8 x 10 MiB)
// stay in the 256 MiB Infinity Cache and much of the reuse among the blocks
// of one XCD hits its 4 MiB L2.  Smaller chunks raise the L2 hit rate but pass
// the running state through memory more often; at the 73,600-token layouts,
// 128- to 320-tile chunks measured alike on random selections and larger
// chunks did better on spatially smooth ones.
constexpr uint64_t kChunkBytes = uint64_t(10) << 20;
// The same budget for 128-token tiles.  Their four-wave workgroups stream
// every K/V block once for 128 query rows, so the L2 hit rate matters less
// than the running-state round trips between launches.  Chunks are sized so
// that the eight XCDs' current chunks together fill the 256 MiB Infinity
// Cache.  On the 77,696-token OmniRef layout, chunks of 335 tiles (2
// launches) measured 4 % faster than chunks within 10 MiB (5 launches).
constexpr uint64_t kChunkBytesWide = uint64_t(32) << 20;

struct Layout {
  uint64_t perm, valid, kt, vt, qp, kp, vp, scores, coarse, sel, choff, state, qt, kt8, kscale,
      kind, visit, order, kt_lo, vt_lo, qt_lo, total;
  int64_t ns;  // scores row stride
};

// Key-tile kinds for the selection (device table `kind`).
enum TileKind : int32_t { kKindPrefix = 0, kKindRef = 1, kKindVideo = 2 };

// fp32 words of fine-branch state per wave lane (O accumulators + running
// max + running sum, padded to 4): head_dim / 2 + 4.
inline int state_words_per_lane(int head_dim) { return head_dim / 2 + 4; }

}  // namespace vsa

struct vsa_h3_plan {
  int64_t L = 0, P = 0, NV = 0, Nt = 0, topk = 0;
  int32_t heads = 0, head_dim = 0;
  vsa_dims3 grid{0, 0, 0};
  vsa_dims3 tile{4, 4, 4};
  int32_t tile_tokens = 64;        // 64 or 128
  int32_t bsh = 0;                 // log2 of the 64-token blocks per tile
  int64_t Nb = 0;                  // blocks, Nt << bsh
  double sparsity = 0.0;
  std::vector<int32_t> perm;       // [Nt*tile_tokens] == [Nb*64]
  std::vector<int32_t> valid;      // [Nt]
  std::vector<int32_t> bvalid;     // [Nb] valid tokens per block
  std::vector<int32_t> kind;       // [Nt] TileKind of each key tile
  std::vector<int32_t> tile_slot;  // [L]
  int64_t num_ref = 0;             // tiles tagged cond
  int64_t num_fixed = 0;           // prefix tiles every video query visits (with ref keep)
  double ref_keep = 1.0;           // reference keep ratio; 1 visits every reference tile
  int64_t topk_ref = 0;            // reference tiles selected per video query (0 if keep is 1)
  int32_t chunk_tiles = 0;         // key tiles per fine-branch chunk
  int32_t chunk_request = 0;       // as last requested (0 = automatic)
  int32_t num_chunks = 0;          // ceil(Nt / chunk_tiles); 0 when Nt == 0
  bool qk_prep = false;            // workspace holds Qt for the QK-norm + RoPE forward
  bool qk_fp8 = false;             // fine branch uses per-token FP8 q and k
  bool io_f32 = false;             // laid out for fp32 I/O: low bf16 parts of K, V^T (and Qt)
  vsa::Layout layout{};
};

namespace vsa {

// Thread-local error message shared by every entry point.
void set_error(const std::string& msg);
const char* get_error();

int64_t topk_rule(int64_t num_video_tiles, double sparsity);

// Builds the plan; returns VSA_OK or an error status (message set).
// Sets the key-chunk size of the fine branch (0 = automatic) and lays out
// the workspace again.
vsa_status set_chunk_tiles(vsa_h3_plan* plan, int32_t chunk_tiles);

// Adds (or drops) the workspace region of the tile-ordered, normalised and
// rotated q used by the QK-norm + RoPE forward.
void set_qk_prep(vsa_h3_plan* plan, bool enable);

// Switches the fine branch to per-token FP8 (E4M3) q and k and adds the
// regions of the quantised key tiles and their scales (or drops them).
void set_qk_fp8(vsa_h3_plan* plan, bool enable);

// Lays the workspace out for fp32 (true) or bf16 (false) I/O.  fp32 I/O
// adds the low bf16 parts (x - bf16(x), rounded to bf16) of the tile-ordered
// keys, values and, with QK-norm + RoPE, queries, so that the fine branch can
// form fp32-accurate products from two bf16 terms.
void set_io_f32(vsa_h3_plan* plan, bool f32);

// Reference keep ratio in (0, 1]: below 1 each video query tile keeps only
// its best-scoring reference (cond) key tiles; lays out the workspace again.
vsa_status set_ref_keep(vsa_h3_plan* plan, double keep);

// Reference tiles kept per video query tile for keep ratio r, in IEEE double
// as written: max(1, min(ceil(r * n), n)); 0 when n == 0.
int64_t ref_keep_rule(int64_t num_ref_tiles, double keep);

// Selected key tiles per video query row of sel_idx: topk_ref + topk.
inline int64_t sel_width(const vsa_h3_plan* plan) { return plan->topk_ref + plan->topk; }

// Explicit visit-list length per video query tile when reference tiles are
// selected (fixed prefix tiles + selected reference tiles + top-k video tiles).
inline int64_t visit_len(const vsa_h3_plan* plan) {
  return plan->num_fixed + plan->topk_ref + plan->topk;
}

vsa_status build_plan(const int64_t* token_tags, const int64_t* position_ids, int64_t L,
                      vsa_dims3 grid, vsa_dims3 tile, int32_t heads, int32_t head_dim,
                      double sparsity, vsa_h3_plan* plan);

}  // namespace vsa

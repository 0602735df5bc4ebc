// Host-side plan of the VSA-H3 forward: tile geometry, device tables and the
// workspace layout.  Pure C++ (no HIP calls), so it can be built and tested
// on a machine without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "vsa_h3.h"

namespace vsa {

constexpr int kTile = 64;          // tokens per tile (video (4,4,4) and prefix)
constexpr int kMaxTilesCoarse = 4096;  // key tiles one wave can hold in the coarse/top-k kernel

struct Layout {
  uint64_t perm, valid, kt, vt, qp, kp, vp, scores, coarse, sel, total;
  int64_t ns;  // scores row stride
};

}  // namespace vsa

struct vsa_h3_plan {
  int64_t L = 0, P = 0, NV = 0, Nt = 0, topk = 0;
  int32_t heads = 0, head_dim = 0;
  vsa_dims3 grid{0, 0, 0};
  double sparsity = 0.0;
  std::vector<int32_t> perm;       // [Nt*64]
  std::vector<int32_t> valid;      // [Nt]
  std::vector<int32_t> tile_slot;  // [L]
  vsa::Layout layout{};
};

namespace vsa {

// Thread-local error message shared by every entry point.
void set_error(const std::string& msg);
const char* get_error();

int64_t topk_rule(int64_t num_video_tiles, double sparsity);

// Builds the plan; returns VSA_OK or an error status (message set).
vsa_status build_plan(const int64_t* token_tags, const int64_t* position_ids, int64_t L,
                      vsa_dims3 grid, vsa_dims3 tile, int32_t heads, int32_t head_dim,
                      double sparsity, vsa_h3_plan* plan);

}  // namespace vsa

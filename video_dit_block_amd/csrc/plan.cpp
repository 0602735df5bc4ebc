// Tile geometry of VSA-H3 (FastH3 4-step Preview (VSA, data-free), section
// "Video Sparse Attention is not optional here"): segment-pure prefix tiles
// and (4,4,4) video tiles over the post-patchify grid, derived from the
// packed stream's tags and positions; the top-k rule of the same passage.
// The OmniRef page ("Device profiles") also runs 128-token tiles with a
// reference keep ratio: here a video tile is any box of 64 or 128 grid cells,
// prefix tiles hold as many tokens, and with keep r < 1 a video query tile
// keeps only max(1, min(ceil(r * n_ref), n_ref)) of the n_ref cond tiles.
// Kernels work on 64-token blocks: a 128-token tile is blocks 2j (slots
// 0-63) and 2j + 1 (slots 64-127).
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <limits>

namespace vsa {

namespace {
thread_local std::string g_error;

uint64_t align256(uint64_t x) { return (x + 255u) & ~uint64_t(255u); }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

void set_error(const std::string& msg) { g_error = msg; }
const char* get_error() { return g_error.c_str(); }

int64_t ref_keep_rule(int64_t n, double r) {
  if (n <= 0) return 0;
  double want = std::ceil(r * static_cast<double>(n));
  int64_t k = want >= static_cast<double>(n) ? n : static_cast<int64_t>(want);
  return k < 1 ? 1 : k;
}

int64_t topk_rule(int64_t nv, double s) {
  if (!(s >= 0.0 && s <= 1.0)) return -1;  // also rejects NaN
  if (nv <= 0) return 0;
  // Evaluated in IEEE double exactly as the rule is written.
  double want = std::ceil((1.0 - s) * static_cast<double>(nv));
  int64_t k = want >= static_cast<double>(nv) ? nv : static_cast<int64_t>(want);
  return k < 1 ? 1 : k;
}

namespace {

// Workspace layout; every region 256-byte aligned, sizes in 64-bit.
void lay_out(vsa_h3_plan* plan) {
  const uint64_t h64 = static_cast<uint64_t>(plan->heads);
  const uint64_t d64 = static_cast<uint64_t>(plan->head_dim);
  const uint64_t nt64 = static_cast<uint64_t>(plan->Nt);
  const uint64_t nb64 = static_cast<uint64_t>(plan->Nb);
  const uint64_t nv64 = static_cast<uint64_t>(plan->NV);
  const int64_t ns = (plan->Nt + 3) / 4 * 4;
  Layout& lo = plan->layout;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    uint64_t at = off;
    off = align256(off + bytes);
    return at;
  };
  lo.perm = take(nb64 * kTile * 4);
  lo.valid = take(nb64 * 4);
  lo.kind = take(nt64 * 4);
  lo.kt = take(h64 * nb64 * kTile * d64 * 2);
  lo.vt = take(h64 * nb64 * kTile * d64 * 2);
  lo.qp = take(h64 * nt64 * d64 * 4);
  lo.kp = take(h64 * nt64 * d64 * 4);
  lo.vp = take(h64 * nt64 * d64 * 4);
  lo.scores = take(h64 * nt64 * static_cast<uint64_t>(ns) * 4);
  lo.coarse = take(h64 * nt64 * d64 * 4);
  lo.sel = take(h64 * nv64 * static_cast<uint64_t>(sel_width(plan)) * 4);
  lo.visit = take(plan->topk_ref > 0 ? h64 * nv64 * static_cast<uint64_t>(visit_len(plan)) * 4 : 0);
  const bool chunked = plan->num_chunks > 1;
  lo.choff = take(chunked ? h64 * nv64 * static_cast<uint64_t>(plan->num_chunks + 1) * 4 : 0);
  lo.order = take(chunked ? h64 * static_cast<uint64_t>(plan->num_chunks) * nt64 * 4 : 0);
  // Two waves of 64 lanes per query block.
  lo.state = take(chunked ? h64 * nb64 * 2 * 64 *
                                static_cast<uint64_t>(state_words_per_lane(plan->head_dim)) * 4
                          : 0);
  lo.qt = take(plan->qk_prep ? h64 * nb64 * kTile * d64 * 2 : 0);
  lo.kt8 = take(plan->qk_fp8 ? h64 * nb64 * kTile * d64 : 0);
  lo.kscale = take(plan->qk_fp8 ? h64 * nb64 * kTile * 4 : 0);
  // fp32 I/O: low bf16 parts of Kt (not with FP8 keys), Vt and Qt.
  const uint64_t tok_bytes = h64 * nb64 * kTile * d64 * 2;
  lo.kt_lo = take(plan->io_f32 && !plan->qk_fp8 ? tok_bytes : 0);
  lo.vt_lo = take(plan->io_f32 ? tok_bytes : 0);
  lo.qt_lo = take(plan->io_f32 && plan->qk_prep ? tok_bytes : 0);
  lo.total = off < 256 ? 256 : off;
  lo.ns = ns;
}

}  // namespace

vsa_status set_chunk_tiles(vsa_h3_plan* plan, int32_t chunk_tiles) {
  if (chunk_tiles < 0) {
    set_error("chunk_tiles must be >= 0 (0 = automatic)");
    return VSA_E_ARG;
  }
  const int64_t Nt = plan->Nt;
  int64_t ch;
  if (chunk_tiles == 0) {
    // Largest chunk within kChunkBytes of K and V (tile_tokens keys x D: K
    // in bf16, or FP8 codes, plus bf16 V^T), then balanced over the chunks.
    const uint64_t tile_bytes =
        uint64_t(plan->tile_tokens) * plan->head_dim * (plan->qk_fp8 ? 3 : 4);
    const uint64_t budget = plan->tile_tokens == 128 ? kChunkBytesWide : kChunkBytes;
    const int64_t cap = static_cast<int64_t>(budget / tile_bytes);
    const int64_t nc = std::max<int64_t>(1, ceil_div(Nt, cap));
    ch = std::max<int64_t>(1, ceil_div(Nt, nc));
  } else {
    ch = chunk_tiles;
  }
  const int64_t nc = Nt == 0 ? 0 : ceil_div(Nt, ch);
  if (nc > kMaxKeyChunks) {
    set_error("chunk_tiles " + std::to_string(ch) + " gives " + std::to_string(nc) +
              " key chunks; at most " + std::to_string(kMaxKeyChunks) + " are supported");
    return VSA_E_ARG;
  }
  plan->chunk_request = chunk_tiles;
  plan->chunk_tiles = static_cast<int32_t>(std::min<int64_t>(ch, std::max<int64_t>(Nt, 1)));
  plan->num_chunks = static_cast<int32_t>(nc);
  lay_out(plan);
  return VSA_OK;
}

void set_qk_prep(vsa_h3_plan* plan, bool enable) {
  plan->qk_prep = enable;
  lay_out(plan);
}

void set_io_f32(vsa_h3_plan* plan, bool f32) {
  plan->io_f32 = f32;
  lay_out(plan);
}

void set_qk_fp8(vsa_h3_plan* plan, bool enable) {
  plan->qk_fp8 = enable;
  // An automatic chunk length depends on the key bytes per tile.
  if (plan->chunk_request != 0 || set_chunk_tiles(plan, 0) != VSA_OK) lay_out(plan);
}

vsa_status set_ref_keep(vsa_h3_plan* plan, double keep) {
  if (!(keep > 0.0 && keep <= 1.0)) {  // also rejects NaN
    set_error("the reference keep ratio must lie in (0, 1]");
    return VSA_E_ARG;
  }
  plan->ref_keep = keep;
  plan->topk_ref = keep < 1.0 ? ref_keep_rule(plan->num_ref, keep) : 0;
  lay_out(plan);
  return VSA_OK;
}

vsa_status build_plan(const int64_t* tags, const int64_t* pos, int64_t L, vsa_dims3 grid,
                      vsa_dims3 tile, int32_t heads, int32_t head_dim, double sparsity,
                      vsa_h3_plan* plan) {
  if (L < 0 || L >= (int64_t(1) << 31) - kTile) {
    set_error("L must be in [0, 2^31 - 64)");
    return VSA_E_ARG;
  }
  if (L > 0 && (!tags || !pos)) {
    set_error("token_tags and position_ids must be non-NULL host arrays");
    return VSA_E_ARG;
  }
  if (heads < 1) {
    set_error("heads must be >= 1");
    return VSA_E_ARG;
  }
  if (!(sparsity >= 0.0 && sparsity <= 1.0)) {
    set_error("sparsity must lie in [0, 1]");
    return VSA_E_ARG;
  }
  if (grid.t < 0 || grid.h < 0 || grid.w < 0) {
    set_error("grid dimensions must be >= 0");
    return VSA_E_ARG;
  }
  if (tile.t < 1 || tile.h < 1 || tile.w < 1 ||
      (int64_t(tile.t) * tile.h * tile.w != 64 && int64_t(tile.t) * tile.h * tile.w != 128)) {
    set_error("a video tile must be a box of 64 or 128 grid cells");
    return VSA_E_UNSUPPORTED;
  }
  const int64_t tt = tile.t, th = tile.h, tw = tile.w;
  const int64_t ntok = tt * th * tw;
  if (head_dim != 64 && head_dim != 128) {
    set_error("head_dim must be 64 or 128");
    return VSA_E_UNSUPPORTED;
  }

  // Packing: every non-video token precedes every video token.
  int64_t n_pre = 0;
  while (n_pre < L && tags[n_pre] != VSA_TAG_VIDEO) {
    if (tags[n_pre] < 0 || tags[n_pre] > VSA_TAG_VIDEO) {
      set_error("unknown token tag at index " + std::to_string(n_pre));
      return VSA_E_LAYOUT;
    }
    ++n_pre;
  }
  for (int64_t r = n_pre; r < L; ++r) {
    if (tags[r] != VSA_TAG_VIDEO) {
      set_error(tags[r] < 0 || tags[r] > VSA_TAG_VIDEO
                    ? "unknown token tag at index " + std::to_string(r)
                    : "prefix token after the first video token at index " + std::to_string(r));
      return VSA_E_LAYOUT;
    }
  }
  const int64_t n_vid = L - n_pre;
  const int64_t T = grid.t, H = grid.h, W = grid.w;
  if (T * H * W != n_vid) {
    set_error("video token count " + std::to_string(n_vid) + " != grid volume " +
              std::to_string(T * H * W));
    return VSA_E_POSITIONS;
  }

  // Prefix tiles: each maximal run of one tag is cut into tile-sized chunks.
  std::vector<int64_t> pre_start, pre_len, pre_tag;
  for (int64_t s = 0; s < n_pre;) {
    int64_t e = s;
    while (e < n_pre && tags[e] == tags[s]) ++e;
    for (int64_t c = s; c < e; c += ntok) {
      pre_start.push_back(c);
      pre_len.push_back(std::min<int64_t>(ntok, e - c));
      pre_tag.push_back(tags[s]);
    }
    s = e;
  }
  const int64_t P = static_cast<int64_t>(pre_start.size());
  const int64_t nt = ceil_div(T, tt), nh = ceil_div(H, th), nw = ceil_div(W, tw);
  const int64_t NV = n_vid ? nt * nh * nw : 0;
  const int64_t Nt = P + NV;
  if (Nt * ntok >= (int64_t(1) << 31)) {
    set_error("too many tiles for 32-bit slot indices");
    return VSA_E_UNSUPPORTED;
  }
  if (Nt > kMaxTilesCoarse) {
    set_error("more than " + std::to_string(kMaxTilesCoarse) + " tiles per head is not supported");
    return VSA_E_UNSUPPORTED;
  }

  plan->L = L;
  plan->P = P;
  plan->NV = NV;
  plan->Nt = Nt;
  plan->topk = topk_rule(NV, sparsity);
  plan->heads = heads;
  plan->head_dim = head_dim;
  plan->grid = grid;
  plan->tile = tile;
  plan->tile_tokens = static_cast<int32_t>(ntok);
  plan->bsh = ntok == 128 ? 1 : 0;
  plan->Nb = Nt << plan->bsh;
  plan->sparsity = sparsity;
  plan->perm.assign(static_cast<size_t>(Nt * ntok), -1);
  plan->valid.assign(static_cast<size_t>(Nt), 0);
  plan->kind.assign(static_cast<size_t>(Nt), vsa::kKindVideo);
  plan->tile_slot.assign(static_cast<size_t>(L), -1);
  plan->num_ref = 0;
  for (int64_t j = 0; j < P; ++j) {
    const bool ref = pre_tag[j] == VSA_TAG_COND;
    plan->kind[j] = ref ? vsa::kKindRef : vsa::kKindPrefix;
    plan->num_ref += ref;
  }
  plan->num_fixed = P - plan->num_ref;

  for (int64_t j = 0; j < P; ++j) {
    plan->valid[j] = static_cast<int32_t>(pre_len[j]);
    for (int64_t s = 0; s < pre_len[j]; ++s) {
      plan->perm[j * ntok + s] = static_cast<int32_t>(pre_start[j] + s);
      plan->tile_slot[pre_start[j] + s] = static_cast<int32_t>(j * ntok + s);
    }
  }

  // Video tiles: tile id from the (t/tt, y/th, x/tw) raster; the slot is the
  // compact (t, y, x) raster inside the tile's valid extent.
  std::vector<uint8_t> seen(static_cast<size_t>(n_vid), 0);
  for (int64_t r = n_pre; r < L; ++r) {
    const int64_t t = pos[3 * r], y = pos[3 * r + 1], x = pos[3 * r + 2];
    if (t < 0 || t >= T || y < 0 || y >= H || x < 0 || x >= W) {
      set_error("video position outside the grid at index " + std::to_string(r));
      return VSA_E_POSITIONS;
    }
    const int64_t cell = (t * H + y) * W + x;
    if (seen[cell]) {
      set_error("duplicate video position at index " + std::to_string(r));
      return VSA_E_POSITIONS;
    }
    seen[cell] = 1;
    const int64_t bt = t / tt, by = y / th, bx = x / tw;
    const int64_t et = std::min<int64_t>(tt, T - tt * bt);
    const int64_t eh = std::min<int64_t>(th, H - th * by);
    const int64_t ew = std::min<int64_t>(tw, W - tw * bx);
    const int64_t j = P + (bt * nh + by) * nw + bx;
    const int64_t slot = ((t % tt) * eh + (y % th)) * ew + (x % tw);
    plan->valid[j] = static_cast<int32_t>(et * eh * ew);
    plan->perm[j * ntok + slot] = static_cast<int32_t>(r);
    plan->tile_slot[r] = static_cast<int32_t>(j * ntok + slot);
  }

  // Valid tokens of each 64-token block (slots fill a tile from the front).
  plan->bvalid.assign(static_cast<size_t>(plan->Nb), 0);
  for (int64_t j = 0; j < Nt; ++j)
    for (int64_t b = 0; b < (int64_t(1) << plan->bsh); ++b)
      plan->bvalid[(j << plan->bsh) + b] = static_cast<int32_t>(
          std::max<int64_t>(0, std::min<int64_t>(kTile, plan->valid[j] - kTile * b)));

  plan->ref_keep = 1.0;
  plan->topk_ref = 0;
  return set_chunk_tiles(plan, 0);
}

}  // namespace vsa

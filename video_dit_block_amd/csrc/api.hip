// C ABI of the VSA-H3 forward: argument checks, workspace carving and the
// launch sequence  permute+pool -> coarse scores -> softmax+top-k -> P.pool(v)
// -> fine attention (one launch per key chunk) with the fused gate-combine
// epilogue in the last.
#include <cstring>
#include <list>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "plan.hpp"
#include "vsa_h3.h"

using vsa::set_error;

static_assert(vsa::kKindRef == vsa::kKindRefTile, "reference tiles carry one kind value");

namespace {

vsa_status hip_fail(const char* what, hipError_t err) {
  set_error(std::string(what) + ": " + hipGetErrorString(err));
  return VSA_E_HIP;
}

vsa_status check_workspace(const vsa_h3_plan* plan, const void* ws, uint64_t bytes) {
  if (!ws) {
    set_error("workspace is NULL");
    return VSA_E_WORKSPACE;
  }
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) {
    set_error("workspace must be 256-byte aligned");
    return VSA_E_WORKSPACE;
  }
  if (bytes < plan->layout.total) {
    set_error("workspace holds " + std::to_string(bytes) + " bytes, plan needs " +
              std::to_string(plan->layout.total));
    return VSA_E_WORKSPACE;
  }
  return VSA_OK;
}

// Plans built by the one-call form, keyed by everything that defines them.
struct CacheEntry {
  std::vector<int64_t> tags, pos;
  vsa_dims3 grid, tile;
  int32_t heads, head_dim;
  double sparsity;
  bool io_f32;
  std::shared_ptr<const vsa_h3_plan> plan;
};
std::mutex g_cache_mu;
std::list<CacheEntry> g_cache;  // most recently used first
constexpr size_t kCacheMax = 8;

vsa_status cached_plan(const int64_t* tags, const int64_t* pos, int64_t L, vsa_dims3 grid,
                       vsa_dims3 tile, int32_t heads, int32_t head_dim, double sparsity,
                       vsa_dtype io_dtype, std::shared_ptr<const vsa_h3_plan>* out) {
  if (L < 0 || (L > 0 && (!tags || !pos))) {
    set_error("token_tags / position_ids must be non-NULL for L > 0");
    return VSA_E_ARG;
  }
  if (io_dtype != VSA_BF16 && io_dtype != VSA_F32) {
    set_error("io_dtype must be VSA_BF16 or VSA_F32");
    return VSA_E_ARG;
  }
  const bool f32 = io_dtype == VSA_F32;
  std::lock_guard<std::mutex> lock(g_cache_mu);
  for (auto it = g_cache.begin(); it != g_cache.end(); ++it) {
    if (it->heads == heads && it->head_dim == head_dim && it->sparsity == sparsity &&
        it->io_f32 == f32 &&
        it->grid.t == grid.t && it->grid.h == grid.h && it->grid.w == grid.w &&
        it->tile.t == tile.t && it->tile.h == tile.h && it->tile.w == tile.w &&
        static_cast<int64_t>(it->tags.size()) == L &&
        (L == 0 || (std::memcmp(it->tags.data(), tags, L * sizeof(int64_t)) == 0 &&
                    std::memcmp(it->pos.data(), pos, 3 * L * sizeof(int64_t)) == 0))) {
      g_cache.splice(g_cache.begin(), g_cache, it);
      *out = g_cache.front().plan;
      return VSA_OK;
    }
  }
  auto plan = std::make_shared<vsa_h3_plan>();
  vsa_status st = vsa::build_plan(tags, pos, L, grid, tile, heads, head_dim, sparsity, plan.get());
  if (st != VSA_OK) return st;
  if (f32) vsa::set_io_f32(plan.get(), true);
  CacheEntry e;
  e.tags.assign(tags, tags + L);
  e.pos.assign(pos, pos + 3 * L);
  e.grid = grid;
  e.tile = tile;
  e.heads = heads;
  e.head_dim = head_dim;
  e.sparsity = sparsity;
  e.io_f32 = f32;
  e.plan = std::move(plan);
  g_cache.push_front(std::move(e));
  if (g_cache.size() > kCacheMax) g_cache.pop_back();
  *out = g_cache.front().plan;
  return VSA_OK;
}

}  // namespace

extern "C" {

int64_t vsa_h3_topk(int64_t num_video_tiles, double sparsity) {
  return vsa::topk_rule(num_video_tiles, sparsity);
}

vsa_status vsa_h3_plan_create(const int64_t* token_tags, const int64_t* position_ids, int64_t L,
                              vsa_dims3 grid, vsa_dims3 tile, int32_t heads, int32_t head_dim,
                              double sparsity, vsa_h3_plan** plan_out) {
  if (!plan_out) {
    set_error("plan_out is NULL");
    return VSA_E_ARG;
  }
  *plan_out = nullptr;
  auto plan = std::make_unique<vsa_h3_plan>();
  vsa_status st = vsa::build_plan(token_tags, position_ids, L, grid, tile, heads, head_dim,
                                  sparsity, plan.get());
  if (st != VSA_OK) return st;
  *plan_out = plan.release();
  return VSA_OK;
}

vsa_status vsa_h3_plan_info(const vsa_h3_plan* plan, vsa_h3_info* out) {
  if (!plan || !out) {
    set_error("plan and out must be non-NULL");
    return VSA_E_ARG;
  }
  out->L = plan->L;
  out->num_prefix_tiles = plan->P;
  out->num_video_tiles = plan->NV;
  out->num_tiles = plan->Nt;
  out->topk = plan->topk;
  out->heads = plan->heads;
  out->head_dim = plan->head_dim;
  out->workspace_bytes = plan->layout.total;
  out->chunk_tiles = plan->chunk_tiles;
  out->num_chunks = plan->num_chunks;
  out->num_ref_tiles = plan->num_ref;
  out->topk_ref = plan->topk_ref;
  out->ref_keep = plan->ref_keep;
  out->tile_tokens = plan->tile_tokens;
  out->num_blocks = static_cast<int32_t>(plan->Nb);
  return VSA_OK;
}

vsa_status vsa_h3_plan_set_chunk_tiles(vsa_h3_plan* plan, int32_t chunk_tiles) {
  if (!plan) {
    set_error("plan is NULL");
    return VSA_E_ARG;
  }
  return vsa::set_chunk_tiles(plan, chunk_tiles);
}

vsa_status vsa_h3_plan_layout(const vsa_h3_plan* plan, vsa_h3_ws_layout* out) {
  if (!plan || !out) {
    set_error("plan and out must be non-NULL");
    return VSA_E_ARG;
  }
  const vsa::Layout& lo = plan->layout;
  out->perm = lo.perm;
  out->valid = lo.valid;
  out->kt = lo.kt;
  out->vt = lo.vt;
  out->qp = lo.qp;
  out->kp = lo.kp;
  out->vp = lo.vp;
  out->scores = lo.scores;
  out->coarse = lo.coarse;
  out->sel = lo.sel;
  out->total = lo.total;
  out->scores_row_stride = lo.ns;
  out->chunk_offsets = lo.choff;
  out->state = lo.state;
  out->qt = lo.qt;
  out->kt8 = lo.kt8;
  out->kscale = lo.kscale;
  out->kind = lo.kind;
  out->visit = lo.visit;
  out->order = lo.order;
  out->kt_lo = lo.kt_lo;
  out->vt_lo = lo.vt_lo;
  out->qt_lo = lo.qt_lo;
  return VSA_OK;
}

vsa_status vsa_h3_plan_set_io_dtype(vsa_h3_plan* plan, vsa_dtype io_dtype) {
  if (!plan) {
    set_error("plan is NULL");
    return VSA_E_ARG;
  }
  if (io_dtype != VSA_BF16 && io_dtype != VSA_F32) {
    set_error("io_dtype must be VSA_BF16 or VSA_F32");
    return VSA_E_ARG;
  }
  vsa::set_io_f32(plan, io_dtype == VSA_F32);
  return VSA_OK;
}

vsa_status vsa_h3_plan_tables(const vsa_h3_plan* plan, int32_t* perm, int32_t* valid,
                              int32_t* tile_slot) {
  if (!plan) {
    set_error("plan is NULL");
    return VSA_E_ARG;
  }
  if (perm) std::memcpy(perm, plan->perm.data(), plan->perm.size() * sizeof(int32_t));
  if (valid) std::memcpy(valid, plan->valid.data(), plan->valid.size() * sizeof(int32_t));
  if (tile_slot)
    std::memcpy(tile_slot, plan->tile_slot.data(), plan->tile_slot.size() * sizeof(int32_t));
  return VSA_OK;
}

vsa_status vsa_h3_plan_upload(const vsa_h3_plan* plan, void* workspace, uint64_t workspace_bytes,
                              void* stream) {
  if (!plan) {
    set_error("plan is NULL");
    return VSA_E_ARG;
  }
  vsa_status st = check_workspace(plan, workspace, workspace_bytes);
  if (st != VSA_OK) return st;
  if (plan->Nt == 0) return VSA_OK;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipMemcpyAsync(ws + plan->layout.perm, plan->perm.data(),
                                  plan->perm.size() * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (err != hipSuccess) return hip_fail("hipMemcpyAsync(perm)", err);
  err = hipMemcpyAsync(ws + plan->layout.valid, plan->bvalid.data(),
                       plan->bvalid.size() * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (err != hipSuccess) return hip_fail("hipMemcpyAsync(valid)", err);
  err = hipMemcpyAsync(ws + plan->layout.kind, plan->kind.data(),
                       plan->kind.size() * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (err != hipSuccess) return hip_fail("hipMemcpyAsync(kind)", err);
  return VSA_OK;
}

vsa_status vsa_h3_forward(const vsa_h3_plan* plan, const void* q, const void* k, const void* v,
                          const void* gate, vsa_dtype io_dtype, void* out, int32_t* sel_idx,
                          void* workspace, uint64_t workspace_bytes, void* stream) {
  return vsa_h3_forward_timed(plan, q, k, v, gate, io_dtype, out, sel_idx, workspace,
                              workspace_bytes, stream, nullptr);
}

}  // extern "C"

namespace {

// The whole forward; `prep` is null, or the QK-norm + RoPE inputs.
vsa_status run_forward(const vsa_h3_plan* plan, const void* q, const void* k, const void* v,
                       const void* gate, const vsa::QkPrepArgs* prep, vsa_dtype io_dtype,
                       void* out, int32_t* sel_idx, void* workspace, uint64_t workspace_bytes,
                       void* stream, void* const* events) {
  if (!plan) {
    set_error("plan is NULL");
    return VSA_E_ARG;
  }
  if (io_dtype != VSA_BF16 && io_dtype != VSA_F32) {
    set_error("io_dtype must be VSA_BF16 or VSA_F32");
    return VSA_E_ARG;
  }
  if (io_dtype == VSA_F32 && !plan->io_f32) {
    set_error("fp32 I/O needs a plan laid out for it: call vsa_h3_plan_set_io_dtype(plan, "
              "VSA_F32) before sizing the workspace");
    return VSA_E_ARG;
  }
  vsa_status st = check_workspace(plan, workspace, workspace_bytes);
  if (st != VSA_OK) return st;
  if (plan->L == 0) return VSA_OK;
  if (!q || !k || !v || !gate || !out) {
    set_error("q, k, v, gate and out must be non-NULL device pointers");
    return VSA_E_ARG;
  }
  const bool f32 = io_dtype == VSA_F32;
  const size_t elt = f32 ? 4 : 2;
  const size_t bytes = static_cast<size_t>(plan->L) * plan->heads * plan->head_dim * elt;
  const char* ob = static_cast<const char*>(out);
  for (const void* in : {q, k, v, gate}) {
    const char* ib = static_cast<const char*>(in);
    if (ib < ob + bytes && ob < ib + bytes) {
      set_error("out must not overlap q, k, v or gate");
      return VSA_E_ARG;
    }
  }
  for (const void* p : {q, k, v, gate, static_cast<const void*>(out)}) {
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) {
      set_error("tensors must be 16-byte aligned");
      return VSA_E_ARG;
    }
  }

  char* ws = static_cast<char*>(workspace);
  const vsa::Layout& lo = plan->layout;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = plan->heads, D = plan->head_dim;
  const int Nt = static_cast<int>(plan->Nt), P = static_cast<int>(plan->P);
  const int NV = static_cast<int>(plan->NV), topk = static_cast<int>(plan->topk);
  const int topk_ref = static_cast<int>(plan->topk_ref), bsh = plan->bsh;
  const int visit_len = static_cast<int>(vsa::visit_len(plan));
  const int32_t* perm = reinterpret_cast<const int32_t*>(ws + lo.perm);
  const int32_t* valid = reinterpret_cast<const int32_t*>(ws + lo.valid);
  uint16_t* kt = reinterpret_cast<uint16_t*>(ws + lo.kt);
  uint16_t* vt = reinterpret_cast<uint16_t*>(ws + lo.vt);
  float* qp = reinterpret_cast<float*>(ws + lo.qp);
  float* kp = reinterpret_cast<float*>(ws + lo.kp);
  float* vp = reinterpret_cast<float*>(ws + lo.vp);
  float* scores = reinterpret_cast<float*>(ws + lo.scores);
  float* coarse = reinterpret_cast<float*>(ws + lo.coarse);
  int32_t* sel = sel_idx ? sel_idx : reinterpret_cast<int32_t*>(ws + lo.sel);
  const int nchunks = plan->num_chunks, chunk_tiles = plan->chunk_tiles;
  int32_t* choff = reinterpret_cast<int32_t*>(ws + lo.choff);
  float* state = reinterpret_cast<float*>(ws + lo.state);

  auto mark = [&](int idx) -> hipError_t {
    return events ? hipEventRecord(static_cast<hipEvent_t>(events[idx]), s) : hipSuccess;
  };
  hipError_t err = mark(0);
  if (err != hipSuccess) return hip_fail("hipEventRecord", err);
  // fp32 I/O: the low bf16 parts of the tile-ordered operands.
  uint16_t* kt_lo = f32 && !plan->qk_fp8 ? reinterpret_cast<uint16_t*>(ws + lo.kt_lo) : nullptr;
  uint16_t* vt_lo = f32 ? reinterpret_cast<uint16_t*>(ws + lo.vt_lo) : nullptr;
  vsa::QkPrepArgs pp{};
  if (prep) {
    pp = *prep;
    pp.qt = reinterpret_cast<uint16_t*>(ws + lo.qt);
    pp.qt_lo = f32 ? reinterpret_cast<uint16_t*>(ws + lo.qt_lo) : nullptr;
  }
  uint8_t* kt8 = plan->qk_fp8 ? reinterpret_cast<uint8_t*>(ws + lo.kt8) : nullptr;
  float* kscale = plan->qk_fp8 ? reinterpret_cast<float*>(ws + lo.kscale) : nullptr;
  vsa::PermutePoolArgs pa{q, k, v, f32, perm, valid, H, Nt, D, bsh, kt, vt, qp, kp, vp, pp, kt8,
                          kscale, kt_lo, vt_lo};
  err = vsa::launch_permute_pool(pa, s);
  if (err != hipSuccess) return hip_fail("permute_pool launch", err);
  if ((err = mark(1)) != hipSuccess) return hip_fail("hipEventRecord", err);

  int32_t* visit = topk_ref > 0 ? reinterpret_cast<int32_t*>(ws + lo.visit) : nullptr;
  const int32_t* kind = reinterpret_cast<const int32_t*>(ws + lo.kind);
  // With a reference selection every key tile of a video query comes from
  // its visit list; otherwise the prefix tiles are implicit and sel follows.
  const int pvis = topk_ref > 0 ? 0 : P;
  int32_t* order = nchunks > 1 ? reinterpret_cast<int32_t*>(ws + lo.order) : nullptr;
  vsa::CoarseArgs ca{qp, kp, vp, scores, coarse, sel, choff, H, Nt, static_cast<int>(lo.ns),
                     P, NV, topk, D, nchunks, chunk_tiles, kind, topk_ref, visit, visit_len,
                     order, pvis};
  err = vsa::launch_coarse(ca, s);
  if (err != hipSuccess) return hip_fail("coarse launch", err);
  if ((err = mark(2)) != hipSuccess) return hip_fail("hipEventRecord", err);

  const int32_t* list = topk_ref > 0 ? visit : sel;
  const int listlen = topk_ref > 0 ? visit_len : topk;
  vsa::FineArgs fa{q, pp.qt, gate, out, f32, kt, vt, coarse, perm, valid, list, choff, state,
                   H, Nt, P, NV, listlen, D, nchunks, chunk_tiles, kt8, kscale, bsh, pvis, order,
                   kt_lo, vt_lo, pp.qt_lo};
  err = vsa::launch_fine(fa, s);
  if (err != hipSuccess) return hip_fail("fine_attn launch", err);
  if ((err = mark(3)) != hipSuccess) return hip_fail("hipEventRecord", err);
  return VSA_OK;
}

}  // namespace

extern "C" {

vsa_status vsa_h3_forward_timed(const vsa_h3_plan* plan, const void* q, const void* k,
                                const void* v, const void* gate, vsa_dtype io_dtype, void* out,
                                int32_t* sel_idx, void* workspace, uint64_t workspace_bytes,
                                void* stream, void* const* events) {
  return run_forward(plan, q, k, v, gate, nullptr, io_dtype, out, sel_idx, workspace,
                     workspace_bytes, stream, events);
}

vsa_status vsa_h3_plan_set_qk_prep(vsa_h3_plan* plan, int32_t enable) {
  if (!plan) {
    set_error("plan is NULL");
    return VSA_E_ARG;
  }
  vsa::set_qk_prep(plan, enable != 0);
  return VSA_OK;
}

vsa_status vsa_h3_plan_set_qk_fp8(vsa_h3_plan* plan, int32_t enable) {
  if (!plan) {
    set_error("plan is NULL");
    return VSA_E_ARG;
  }
  vsa::set_qk_fp8(plan, enable != 0);
  return VSA_OK;
}

vsa_status vsa_h3_plan_set_ref_keep(vsa_h3_plan* plan, double keep) {
  if (!plan) {
    set_error("plan is NULL");
    return VSA_E_ARG;
  }
  return vsa::set_ref_keep(plan, keep);
}

vsa_status vsa_h3_forward_qk_prep(const vsa_h3_plan* plan, const void* q, const void* k,
                                  const void* v, const void* gate, const float* q_norm_weight,
                                  const float* k_norm_weight, float eps, const float* rope_cos,
                                  const float* rope_sin, vsa_dtype io_dtype, void* out,
                                  int32_t* sel_idx, void* workspace, uint64_t workspace_bytes,
                                  void* stream, void* const* events) {
  if (!plan) {
    set_error("plan is NULL");
    return VSA_E_ARG;
  }
  if (!plan->qk_prep) {
    set_error("the plan has no QK-norm + RoPE workspace: call vsa_h3_plan_set_qk_prep first");
    return VSA_E_ARG;
  }
  if (plan->L > 0 && (!q_norm_weight || !k_norm_weight || !rope_cos || !rope_sin)) {
    set_error("norm weights and RoPE tables must be non-NULL device pointers");
    return VSA_E_ARG;
  }
  if (!(eps >= 0.0f) || eps > 3.0e38f) {
    set_error("eps must be finite and >= 0");
    return VSA_E_ARG;
  }
  for (const void* p : {static_cast<const void*>(q_norm_weight),
                        static_cast<const void*>(k_norm_weight),
                        static_cast<const void*>(rope_cos), static_cast<const void*>(rope_sin)}) {
    if (reinterpret_cast<uintptr_t>(p) % 4 != 0) {
      set_error("norm weights and RoPE tables must be 4-byte aligned");
      return VSA_E_ARG;
    }
  }
  vsa::QkPrepArgs prep{q_norm_weight, k_norm_weight, rope_cos, rope_sin, eps, nullptr, nullptr};
  return run_forward(plan, q, k, v, gate, &prep, io_dtype, out, sel_idx, workspace,
                     workspace_bytes, stream, events);
}

vsa_status vsa_h3_oneshot_workspace_bytes(const int64_t* token_tags, const int64_t* position_ids,
                                          int64_t L, vsa_dims3 grid, vsa_dims3 tile,
                                          int32_t heads, int32_t head_dim, double sparsity,
                                          vsa_dtype io_dtype, uint64_t* bytes_out) {
  if (!bytes_out) {
    set_error("bytes_out is NULL");
    return VSA_E_ARG;
  }
  std::shared_ptr<const vsa_h3_plan> plan;
  vsa_status st = cached_plan(token_tags, position_ids, L, grid, tile, heads, head_dim, sparsity,
                              io_dtype, &plan);
  if (st != VSA_OK) return st;
  *bytes_out = plan->layout.total;
  return VSA_OK;
}

vsa_status vsa_h3_forward_oneshot(const void* q, const void* k, const void* v, const void* gate,
                                  const int64_t* token_tags, const int64_t* position_ids,
                                  int64_t L, int32_t heads, int32_t head_dim, vsa_dims3 grid,
                                  double sparsity, vsa_dims3 tile, vsa_dtype io_dtype, void* out,
                                  int32_t* sel_idx, void* workspace, uint64_t workspace_bytes,
                                  void* stream) {
  std::shared_ptr<const vsa_h3_plan> plan;
  vsa_status st = cached_plan(token_tags, position_ids, L, grid, tile, heads, head_dim, sparsity,
                              io_dtype, &plan);
  if (st != VSA_OK) return st;
  st = vsa_h3_plan_upload(plan.get(), workspace, workspace_bytes, stream);
  if (st != VSA_OK) return st;
  return vsa_h3_forward(plan.get(), q, k, v, gate, io_dtype, out, sel_idx, workspace, workspace_bytes,
                        stream);
}

}  // extern "C"

namespace {

// Workspace of the forward that allocates nothing: one file-scope device
// array, which each GPU the library runs on holds until the process ends.
// Host code never passes the array's name to a kernel or a copy (on the host
// it is only a stand-in symbol); it uses the device address that
// hipGetSymbolAddress reports for the current device, looked up once per
// device on the first call there.
constexpr uint64_t kScratchBytes = uint64_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

vsa_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_fail("hipGetDevice", err);
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device index " + std::to_string(dev) + " is beyond the " +
              std::to_string(kMaxDevices) + " devices the no-allocation forward tracks");
    return VSA_E_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", err);
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256 != 0) {
      set_error("hipGetSymbolAddress(scratch) gave an unusable address");
      return VSA_E_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return VSA_OK;
}

}  // namespace

extern "C" {

vsa_status vsa_h3_forward_noalloc(const vsa_h3_plan* plan, const void* q, const void* k,
                                  const void* v, const void* gate, vsa_dtype io_dtype, void* out,
                                  int32_t* sel_idx, void* stream) {
  if (!plan) {
    set_error("plan is NULL");
    return VSA_E_ARG;
  }
  if (plan->layout.total > kScratchBytes) {
    set_error("the plan needs a workspace of " + std::to_string(plan->layout.total) +
              " bytes; the no-allocation forward holds at most " + std::to_string(kScratchBytes) +
              " (use vsa_h3_forward with a caller-provided workspace)");
    return VSA_E_WORKSPACE;
  }
  void* ws = nullptr;
  vsa_status st = scratch_for_current_device(&ws);
  if (st != VSA_OK) return st;
  // The array keeps whatever the last call on this GPU left, so this call's
  // plan tables go in first; nothing else in it has to start at zero (every
  // other region is written before it is read within one forward).
  st = vsa_h3_plan_upload(plan, ws, kScratchBytes, stream);
  if (st != VSA_OK) return st;
  return vsa_h3_forward(plan, q, k, v, gate, io_dtype, out, sel_idx, ws, kScratchBytes, stream);
}

void vsa_h3_plan_destroy(vsa_h3_plan* plan) { delete plan; }

const char* vsa_h3_last_error(void) { return vsa::get_error(); }

const char* vsa_h3_version(void) { return "vsa_h3 0.1.0 gfx950"; }

}  // extern "C"

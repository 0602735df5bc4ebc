// Coarse branch and top-k selection of VSA-H3 (FastH3 4-step Preview (VSA,
// data-free), section "Video Sparse Attention is not optional here"):
//   S[h][i][j]  = pooled q_i . pooled k_j in fp32           (tile scores)
//   sel[h][i]   = top-k video key tiles of video query tile i by S (and,
//                 with a reference keep ratio -- the OmniRef page, "Device
//                 profiles" -- its best reference (cond) tiles before them)
//   c[h][i][:]  = softmax_j(S[h][i][j] / sqrt(D)) @ pooled v  (compression)
//
// Scores are evaluated in a fixed order -- start at +0, add the separately
// rounded products d = 0..D-1, no fused multiply-add -- so the selection is
// reproducible bit for bit.  That is why the score contraction runs on the
// VALU rather than on the matrix cores, whose internal accumulation order is
// not specified.  The selection breaks ties toward the lower tile index.
//
// Three kernels:
//   scores        64x64 output tile per block, 4x4 per thread, pooled rows
//                 staged transposed (and swizzled) in LDS in chunks of 32
//                 channels;
//   softmax_topk  one wave per (head, query tile): the row lives in
//                 registers; an MSB-first bitwise search finds the k-th
//                 largest key of each group (video tiles; reference tiles),
//                 ties are admitted in ascending index order, the kept
//                 indices are compacted in ascending order (with their counts
//                 below each key-chunk boundary of the fine branch); the row
//                 is then overwritten with its softmax probabilities;
//   pv            c = probabilities @ pooled v, 64 rows x D per block.
#include "device.hpp"
#include "kernels.hpp"

namespace vsa {

namespace {

constexpr int kScoreTile = 64;
constexpr int kMaxTiles = 4096;   // tiles per head the plan accepts
constexpr int kDChunk = 32;
constexpr int kPad = 4;
static_assert(kDChunk == 32, "the staging swizzle pairs channel rows 16-31 with c4 >= 4");

template <int D>
__global__ __launch_bounds__(256) void coarse_scores_kernel(const float* __restrict__ qp,
                                                            const float* __restrict__ kp,
                                                            int Nt, int Ns,
                                                            float* __restrict__ S) {
  __shared__ __attribute__((aligned(16))) float qs[kDChunk][kScoreTile + kPad];
  __shared__ __attribute__((aligned(16))) float ks[kDChunk][kScoreTile + kPad];
  const int h = blockIdx.z;
  const int i0 = blockIdx.y * kScoreTile;
  const int j0 = blockIdx.x * kScoreTile;
  const int tid = threadIdx.x;
  const int ti = tid / 16, tj = tid % 16;
  const float* qh = qp + static_cast<size_t>(h) * Nt * D;
  const float* kh = kp + static_cast<size_t>(h) * Nt * D;

  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;

  for (int dc = 0; dc < D; dc += kDChunk) {
    // 64 rows x 32 channels = 512 float4 per operand; 2 per thread.
    // Channel rows 16-31 of the staging hold their 64 entries with the
    // column index XOR-ed with 8 (whole groups of 4 change places): a wave's
    // transposing stores then meet each LDS bank at most twice (once with
    // 64 banks) instead of four (two) times.
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int id = tid + e * 256;
      const int r = id / 8, c4 = id % 8;
      const int rs = r ^ ((c4 >> 2) << 3);
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (i0 + r < Nt) a = *reinterpret_cast<const float4*>(qh + static_cast<size_t>(i0 + r) * D + dc + 4 * c4);
      if (j0 + r < Nt) b = *reinterpret_cast<const float4*>(kh + static_cast<size_t>(j0 + r) * D + dc + 4 * c4);
      qs[4 * c4 + 0][rs] = a.x; qs[4 * c4 + 1][rs] = a.y; qs[4 * c4 + 2][rs] = a.z; qs[4 * c4 + 3][rs] = a.w;
      ks[4 * c4 + 0][rs] = b.x; ks[4 * c4 + 1][rs] = b.y; ks[4 * c4 + 2][rs] = b.z; ks[4 * c4 + 3][rs] = b.w;
    }
    __syncthreads();
    {
#pragma clang fp contract(off)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int ci = (4 * ti) ^ (8 * hh), cj = (4 * tj) ^ (8 * hh);
#pragma unroll 8
        for (int d16 = 0; d16 < kDChunk / 2; ++d16) {
          const int dd = 16 * hh + d16;
          const float4 a = *reinterpret_cast<const float4*>(&qs[dd][ci]);
          const float4 b = *reinterpret_cast<const float4*>(&ks[dd][cj]);
          const float av[4] = {a.x, a.y, a.z, a.w};
          const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
          for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y) acc[x][y] = acc[x][y] + av[x] * bv[y];
        }
      }
    }
    __syncthreads();
  }
  const int jc = j0 + 4 * tj;
  if (jc < Ns) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int i = i0 + 4 * ti + x;
      if (i < Nt) {
        *reinterpret_cast<float4*>(S + (static_cast<size_t>(h) * Nt + i) * Ns + jc) =
            make_float4(acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
      }
    }
  }
}

// Order-preserving map of fp32 to uint32 (-0 folded onto +0; inputs finite).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Largest T with #{key >= T} >= k (the k-th largest key of a group), and how
// many keys equal to T are still to be admitted.  Slots outside the group
// hold key 0, which no candidate (>= 1) reaches: every real key is nonzero
// (finite scores map above 2^23).  Counts are ballots and popcounts (scalar
// unit), not lane sums.  The search fixes one bit of T per step, from the
// top; once exactly k keys reach the candidate, T is the least of them, and
// a wave minimum ends the search (typically half way for distinct scores).
template <int MAXM>
__device__ __forceinline__ void kth_key(const uint32_t (&key)[MAXM], int k, uint32_t& thr,
                                        int& need) {
  thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int c = 0;
#pragma unroll
    for (int m = 0; m < MAXM; ++m) c += __popcll(__builtin_amdgcn_ballot_w64(key[m] >= cand));
    if (c >= k) {
      thr = cand;
      if (c == k) {   // wave-uniform
        uint32_t mn = 0xffffffffu;
#pragma unroll
        for (int m = 0; m < MAXM; ++m)
          if (key[m] >= cand) mn = min(mn, key[m]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mn = min(mn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mn), o)));
        thr = mn;
        break;
      }
    }
  }
  int gt = 0;
#pragma unroll
  for (int m = 0; m < MAXM; ++m) gt += __popcll(__builtin_amdgcn_ballot_w64(key[m] > thr));
  need = k - gt;
}

// REFSEL: a reference selection (topk_ref > 0) runs as its own instance, so
// that the registers of its second key group do not weigh on the common case.
template <int MAXM, bool REFSEL>
__global__ __launch_bounds__(256) void coarse_softmax_topk_kernel(
    float* __restrict__ S, int H, int Nt, int Ns, int P, int NV, int topk, float scale_log2,
    int32_t* __restrict__ sel, int nchunks, int chunk_tiles, int32_t* __restrict__ choff,
    const int32_t* __restrict__ kind, int topk_ref, int32_t* __restrict__ visit, int visit_len) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= H * Nt) return;  // wave-uniform
  const int h = row / Nt;
  const int i = row - h * Nt;
  float* srow = S + static_cast<size_t>(row) * Ns;

  float s[MAXM];
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    const int j = lane + 64 * m;
    s[m] = j < Nt ? srow[j] : -INFINITY;
  }

  if (i >= P && topk > 0) {
    // Keys of the two groups: the video key tiles j in [P, Nt) and, with a
    // reference selection, the reference tiles among 0..P-1 (0 elsewhere).
    constexpr int MR = REFSEL ? MAXM : 1;
    uint32_t keyv[MAXM], keyr[MR];
    bool okv[MAXM], okr[MR];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      const int j = lane + 64 * m;
      okv[m] = j >= P && j < Nt;
      keyv[m] = okv[m] ? order_key(s[m]) : 0u;
      if constexpr (REFSEL) {
        okr[m] = j < P && kind[j] == kKindRefTile;
        keyr[m] = okr[m] ? order_key(s[m]) : 0u;
      }
    }
    uint32_t thr_v, thr_r = 0;
    int need_v, need_r = 0;  // ties to admit, lowest index first
    kth_key<MAXM>(keyv, topk, thr_v, need_v);
    if constexpr (REFSEL) kth_key<MAXM>(keyr, topk_ref, thr_r, need_r);
    const uint64_t below = (uint64_t(1) << lane) - 1;
    // Lane c <= nchunks also counts the entries of the fine branch's list
    // (visit with a reference selection, else sel) below c * chunk_tiles (the
    // key-chunk boundaries): the count before block xm plus the listed
    // lanes of block xm below xr.
    const int xb = min(lane * chunk_tiles, Nt);
    const int xm = xb >> 6, xr = xb & 63;
    int below_x = REFSEL ? visit_len : topk;
    int tie_v = 0, tie_r = 0, out_s = 0, out_l = 0;
    const size_t row = static_cast<size_t>(h) * NV + (i - P);
    int32_t* dst = sel + row * (topk_ref + topk);
    int32_t* vdst = REFSEL ? visit + row * visit_len : nullptr;
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      const bool tv = okv[m] && keyv[m] == thr_v;
      const uint64_t tvmask = __ballot(tv);
      const int rank_v = tie_v + __popcll(tvmask & below);
      tie_v += __popcll(tvmask);
      bool take = okv[m] && (keyv[m] > thr_v || (tv && rank_v < need_v));
      uint64_t lmask;
      if constexpr (REFSEL) {
        const bool tr = okr[m] && keyr[m] == thr_r;
        const uint64_t trmask = __ballot(tr);
        const int rank_r = tie_r + __popcll(trmask & below);
        tie_r += __popcll(trmask);
        take = take || (okr[m] && (keyr[m] > thr_r || (tr && rank_r < need_r)));
        // Listed: the selected tiles and the prefix tiles outside the reference group.
        const bool listed = take || (lane + 64 * m < P && !okr[m]);
        lmask = __ballot(listed);
        if (listed) vdst[out_l + __popcll(lmask & below)] = lane + 64 * m;
      }
      const uint64_t omask = __ballot(take);
      if (take) dst[out_s + __popcll(omask & below)] = lane + 64 * m;
      out_s += __popcll(omask);
      if constexpr (!REFSEL) lmask = omask;
      if (m == xm) below_x = out_l + __popcll(lmask & ((uint64_t(1) << xr) - 1));
      out_l += __popcll(lmask);
    }
    if (nchunks > 1 && lane <= nchunks)
      choff[row * (nchunks + 1) + lane] = below_x;
  }

  // Softmax over all key tiles with the 1/sqrt(D) scale (log2 domain).
  float mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < MAXM; ++m) mx = fmaxf(mx, s[m]);
  mx = wave_max(mx);
  float e[MAXM];
  float sum = 0.0f;
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    const int j = lane + 64 * m;
    e[m] = j < Nt ? __builtin_amdgcn_exp2f((s[m] - mx) * scale_log2) : 0.0f;
    sum += e[m];
  }
  sum = wave_sum(sum);
  const float inv = 1.0f / sum;
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    const int j = lane + 64 * m;
    if (j < Nt) srow[j] = e[m] * inv;
  }
}

// Dispatch order of one head's query tiles in one key-chunk launch: the
// tiles sorted by their visits in the chunk, most first, so that the long
// blocks start first and the launch does not end on one of them (a counting
// sort; the order among equal counts is whatever the LDS atomics give, which
// changes no block's arithmetic).  One workgroup per (chunk, head).
__global__ __launch_bounds__(1024) void chunk_order_kernel(const int32_t* __restrict__ choff,
                                                           int Nt, int P, int NV, int nchunks,
                                                           int chunk_tiles, int Pvis,
                                                           int32_t* __restrict__ order) {
  __shared__ int cnt[kMaxTiles + 2];
  __shared__ int part[1024];
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int lo = c * chunk_tiles, hi = min(lo + chunk_tiles, Nt);
  const int wmax = hi - lo;  // a prefix (dense) query tile visits every tile of the chunk
  auto work = [&](int i) -> int {
    if (i < P) return wmax;
    const int32_t* co = choff + (static_cast<size_t>(h) * NV + (i - P)) * (nchunks + 1) + c;
    return min(max(min(hi, Pvis) - min(lo, Pvis) + co[1] - co[0], 0), wmax);
  };
  for (int w = tid; w <= wmax; w += 1024) cnt[w] = 0;
  __syncthreads();
  for (int i = tid; i < Nt; i += 1024) atomicAdd(&cnt[wmax - work(i)], 1);
  __syncthreads();
  // Exclusive prefix sum of cnt over d = wmax - work (most work first):
  // each thread sums a run of R entries, then the 1024 run sums are scanned.
  const int R = (wmax + 1 + 1023) / 1024;
  int run = 0;
  for (int d = tid * R; d < min((tid + 1) * R, wmax + 1); ++d) run += cnt[d];
  part[tid] = run;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int base = part[tid] - run;
  for (int d = tid * R; d < min((tid + 1) * R, wmax + 1); ++d) {
    const int n = cnt[d];
    cnt[d] = base;
    base += n;
  }
  __syncthreads();
  int32_t* dst = order + (static_cast<size_t>(h) * nchunks + c) * Nt;
  for (int i = tid; i < Nt; i += 1024) dst[atomicAdd(&cnt[wmax - work(i)], 1)] = i;
}

// c[h] = Pr[h] @ vp[h] on the fp32 matrix cores (v_mfma_f32_32x32x2_f32): a
// block of 4 waves owns 64 query tiles x D channels, wave w the 32 rows
// 32(w/2).. and the D/2 channels (D/2)(w%2)..; the K loop stages 32 key
// tiles at a time in LDS (P transposed, [key][row], and vp, [key][channel]),
// with row strides chosen so that the two lane halves of an operand read
// (keys k and k+1) fall into (nearly) disjoint banks.  The order of the
// fp32 sums is the matrix cores' own; c is compared with tolerance.
template <int D>
__global__ __launch_bounds__(256) void coarse_pv_kernel(const float* __restrict__ Pr,
                                                        const float* __restrict__ vp, int Nt,
                                                        int Ns, float* __restrict__ c) {
  constexpr int KB = 32;
  constexpr int NTW = D / 64;          // 32x32 output tiles per wave
  constexpr int PS = 64 + 33;          // 33 (mod 64): reads of keys k, k+1 and the
  constexpr int VS = D + 32;           // transposing stores are at most 2-way conflicted
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  __shared__ __attribute__((aligned(16))) float ps[KB][PS];
  __shared__ __attribute__((aligned(16))) float vs[KB][VS];
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int r0 = 32 * (w >> 1);
  const int c0 = (D / 2) * (w & 1);
  const float* ph = Pr + static_cast<size_t>(h) * Nt * Ns;
  const float* vh = vp + static_cast<size_t>(h) * Nt * D;
  f32x16 acc[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) acc[t] = f32x16{};

  // The next 32 key tiles are loaded into registers while the matrix cores
  // work on the current ones in LDS.
  constexpr int NV4 = KB * D / 4 / 256;  // float4 of vp per thread
  float4 pa[2], vb[NV4];
  auto load = [&](int j0) {
    // probabilities: 64 rows x 32 keys = 512 float4, 2 per thread
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int id = tid + e * 256;
      const int r = id / 8, j = j0 + 4 * (id % 8);
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i0 + r < Nt) {
        const float* src = ph + static_cast<size_t>(i0 + r) * Ns + j;
        if (j + 3 < Nt) {
          x = *reinterpret_cast<const float4*>(src);
        } else {
          if (j + 0 < Nt) x.x = src[0];
          if (j + 1 < Nt) x.y = src[1];
          if (j + 2 < Nt) x.z = src[2];
        }
      }
      pa[e] = x;
    }
    // pooled values: 32 rows x D (zero past the last key tile)
#pragma unroll
    for (int e = 0; e < NV4; ++e) {
      const int id = tid + e * 256;
      const int r = id / (D / 4), c4 = id % (D / 4);
      vb[e] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j0 + r < Nt) vb[e] = *reinterpret_cast<const float4*>(vh + static_cast<size_t>(j0 + r) * D + 4 * c4);
    }
  };
  load(0);
  for (int j0 = 0; j0 < Nt; j0 += KB) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int id = tid + e * 256;
      const int r = id / 8, c4 = id % 8;
      ps[4 * c4 + 0][r] = pa[e].x; ps[4 * c4 + 1][r] = pa[e].y;
      ps[4 * c4 + 2][r] = pa[e].z; ps[4 * c4 + 3][r] = pa[e].w;
    }
#pragma unroll
    for (int e = 0; e < NV4; ++e) {
      const int id = tid + e * 256;
      *reinterpret_cast<float4*>(&vs[id / (D / 4)][4 * (id % (D / 4))]) = vb[e];
    }
    __syncthreads();
    if (j0 + KB < Nt) load(j0 + KB);
    // A: lane l holds P[row r0 + l%32][key k + l/32]; B: vp[key k + l/32][channel + l%32].
#pragma unroll 4
    for (int k = 0; k < KB; k += 2) {
      const float av = ps[k + (lane >> 5)][r0 + (lane & 31)];
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const float bv = vs[k + (lane >> 5)][c0 + 32 * t + (lane & 31)];
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // Accumulator register r of lane l holds row 8(r/4) + 4(l/32) + r%4, column l%32.
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + r0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (i < Nt)
        c[(static_cast<size_t>(h) * Nt + i) * D + c0 + 32 * t + (lane & 31)] = acc[t][r];
    }
}

template <int D>
hipError_t launch_d(const CoarseArgs& a, hipStream_t stream) {
  const int nb = (a.Nt + kScoreTile - 1) / kScoreTile;
  hipLaunchKernelGGL((coarse_scores_kernel<D>), dim3(nb, nb, a.H), dim3(256), 0, stream, a.qp,
                     a.kp, a.Nt, a.Ns, a.scores);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  const int rows = a.H * a.Nt;
  dim3 g2((rows + 3) / 4);
  // Row registers per lane: the smallest instantiated multiple of 4 (up to
  // 32, then of 8) covering ceil(Nt / 64).
  const int maxm = (a.Nt + 63) / 64;
#define VSA_TOPK(M)                                                                           \
  do {                                                                                       \
    if (a.topk_ref > 0)                                                                      \
      hipLaunchKernelGGL((coarse_softmax_topk_kernel<M, true>), g2, dim3(256), 0, stream,      \
                         a.scores, a.H, a.Nt, a.Ns, a.P, a.NV, a.topk, scale_log2, a.sel,      \
                         a.nchunks, a.chunk_tiles, a.choff, a.kind, a.topk_ref, a.visit,       \
                         a.visit_len);                                                       \
    else                                                                                     \
      hipLaunchKernelGGL((coarse_softmax_topk_kernel<M, false>), g2, dim3(256), 0, stream,     \
                         a.scores, a.H, a.Nt, a.Ns, a.P, a.NV, a.topk, scale_log2, a.sel,      \
                         a.nchunks, a.chunk_tiles, a.choff, a.kind, a.topk_ref, a.visit,       \
                         a.visit_len);                                                       \
  } while (0)
  if (maxm <= 4) VSA_TOPK(4);
  else if (maxm <= 8) VSA_TOPK(8);
  else if (maxm <= 12) VSA_TOPK(12);
  else if (maxm <= 16) VSA_TOPK(16);
  else if (maxm <= 20) VSA_TOPK(20);
  else if (maxm <= 24) VSA_TOPK(24);
  else if (maxm <= 28) VSA_TOPK(28);
  else if (maxm <= 32) VSA_TOPK(32);
  else if (maxm <= 40) VSA_TOPK(40);
  else if (maxm <= 48) VSA_TOPK(48);
  else if (maxm <= 56) VSA_TOPK(56);
  else VSA_TOPK(64);
#undef VSA_TOPK
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  if (a.order) {
    hipLaunchKernelGGL(chunk_order_kernel, dim3(a.nchunks, a.H), dim3(1024), 0, stream, a.choff,
                       a.Nt, a.P, a.NV, a.nchunks, a.chunk_tiles, a.Pvis, a.order);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL((coarse_pv_kernel<D>), dim3(nb, a.H), dim3(256), 0, stream, a.scores, a.vp,
                     a.Nt, a.Ns, a.coarse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_coarse(const CoarseArgs& a, hipStream_t stream) {
  return a.D == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace vsa

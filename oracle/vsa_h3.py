"""Plain, slow CPU definition of the VSA-H3 attention forward (NumPy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never called by the
product path.

What is computed, and where the pages state it
----------------------------------------------
The normative description is the VSA-H3 paragraph of "FastH3 4-step Preview
(VSA, data-free)", section "Video Sparse Attention is not optional here":
video tokens are cut into 64-token (4, 4, 4) tiles over the post-patchify
grid; the conditioning prefix is cut into tiles that never mix segments;
per-head fp32 tile scores come from pooled q and k; every video query tile
keeps the top ``topk = max(1, min(ceil((1 - sparsity) * n_video_tiles),
n_video_tiles))`` video key tiles; prefix key tiles are always kept and prefix
query tiles attend to everything; a compression branch ``softmax(scores) @
pool(v)`` is broadcast over each query tile's rows and scaled by a gate with
no activation; the tile geometry is derived from token tags and positions.
Supporting passages: "FastH3 NVFP4 on RTX PRO 6000 (sm_120)", section
"Block-sparse FP4 attention for VSA tiles" (per-query-block lists of key
blocks, partially filled tiles, every query visits prefix block 0) and
section "Model integration" (gather into tile order with zero pad rows,
gather back to packed order; the gate is applied per token after the small
per-tile compression output, section "What was tried and not shipped").
The sparsity-0 case equals plain scaled-dot-product attention (FastH3 4-step
Preview, same section, the self-test against SDPA).

Readings taken where the pages are silent (each one is also listed in the
design notes of the repository):
  R1 pooling is the arithmetic mean over a tile's valid tokens;
  R2 the fine-branch scale is 1/sqrt(D) (the SDPA default); the coarse
     softmax uses the same scale; top-k works on the unscaled scores;
  R3 the coarse softmax runs over every key tile, prefix and video, each
     weighted once;
  R4 every query tile, prefix included, receives the gated coarse term;
  R5 out = o_fine + gate * c_tile, with gate shaped like q: [L, H, D];
  R6 topk is evaluated in IEEE double exactly as written; with no video
     tiles there is nothing to select (topk 0);
  R7 ties in the top-k go to the lower tile index; -0 equals +0;
  R8 fp32 order of pool and scores is fixed so that the integer selection
     is reproducible: element -> fp32 exactly; pool = sequential fp32 sum over
     a tile's slots in slot order, then one correctly rounded division by the
     count; score = sequential fp32 sum over d of separately rounded
     products (no fused multiply-add), starting from +0;
  R9 slot order inside a video tile is the (t, y, x) raster of its valid
     positions, compacted; inside a prefix tile it is packed order;
  R10 tile order: prefix tiles first in packed order, then video tiles in
     (t/4, y/4, x/4) raster order;
  R11 partial tiles hold only their valid tokens: pad keys are masked, pad
     query rows produce no output, pooling divides by the valid count;
  R12 prefix tiles hold 64 tokens (the video tile volume); each maximal run
     of one tag is one segment;
  R13 all non-video tokens precede all video tokens; video positions are
     zero-based and cover the grid exactly once.

Variant with 128-token tiles and a reference keep ratio (the OmniRef page,
section "Device profiles": its Blackwell stack runs VSA at sparsity 0.9 with
128-token tiles and reference keep 0.1; neither the tile shape nor the keep
rule is spelled out there):
  R22 a video tile is a (tt, ty, tx) box of 64 or 128 grid cells, given by
     the caller; tiles cover the grid in (t/tt, y/ty, x/tx) raster order and
     prefix tiles hold as many tokens as a video tile (R12 with that count).
     The 128-token shape used by the workloads is (4, 8, 4), which divides the
     height and width of the 480p and 768p grids;
  R23 reference keep r in (0, 1]: a video query tile keeps only the
     kr = max(1, min(ceil(r * NR), NR)) reference key tiles (tag cond, NR of
     them) with the highest unscaled scores, ties to the lower tile index,
     next to the top-k video tiles; text and audio key tiles stay always
     visited, prefix query tiles stay dense, and the compression branch still
     covers every key tile.  r = 1 keeps every reference tile, which is the
     method without the keep ratio.

Optional upstream step, fused into the tile gather ("FastH3 NVFP4 on RTX PRO
6000", section "Model integration": QK-norm and RoPE are applied to the
tile-ordered q and k with cos/sin tables computed once per step, and pad rows
stay zero through them).  The pages give neither the H3 norm weights nor the
RoPE frequencies, so both arrive as inputs:
  R14 QK-norm is an RMS norm over head_dim for every (token, head), with one
     fp32 weight vector [D] for q and one for k, shared by all heads; eps is
     added to the mean square;
  R15 canonical fp32 order (so that pooled values and the selection stay
     reproducible bit for bit): ss = +0, then ss = ss + x_d * x_d for
     d = 0..D-1 (separately rounded, no fused multiply-add);
     inv = 1 / sqrt(ss / D + eps), each of the division, addition, square
     root and reciprocal correctly rounded; y_d = (x_d * inv) * w_d;
  R16 RoPE rotates the interleaved pairs (y_2i, y_2i+1), i = 0..D/2-1, by the
     caller's per-token cos/sin [L, D/2] as the complex product
     (a + ib)(c + is): a' = a*c - b*s, b' = a*s + b*c, products and sums
     separately rounded in fp32;
  R17 the normalised, rotated q and k are rounded to the I/O dtype (bf16
     nearest-even, or kept fp32) and are then the attention inputs: the
     pooling, scores, selection and fine branch all use them; v is unchanged.

Optional 8-bit Q/K for the fine branch (the OmniRef page, section
"Fallbacks": per-token FP8 Q/K with bf16 P.V, which its Blackwell profiles
use for prefix rows):
  R19 the format is OCP FP8 E4M3 (bias 7, 3 mantissa bits, subnormals, max
     448, no infinities); encoding rounds to nearest with ties to the even
     code and saturates at +-448;
  R20 per-token scales: for every (token, head) row x of q and of k,
     amax = max_d |x_d| (fp32); inv = fl32(448 / amax); code_d =
     E4M3(fl32(x_d * inv)); the dequantisation scale is s = fl32(amax / 448);
     a zero row has s = 0 and zero codes;
  R21 only the fine branch uses the quantised values s * decode(code) for
     its logits; pooling, scores, selection, the coarse branch and P.V
     (bf16 V) are unchanged, and so is the 1/sqrt(D) scale.

Pins (tests/test_oracle_pins.py) -- each function is checked against
something other than itself:
  topk_count         closed-form values and the double-evaluation case
  geometry           per-dimension closed-form tile counts on odd grids;
                     permutation of the packed video order
  pool_canonical     constant tiles (exact), float64 mean within rounding
  scores_canonical   float64 dot product within the fp32 error bound;
                     constructed exact cases
  select_topk        exhaustive Python sort on (-score, index); forced ties
  select_ref         exhaustive Python sort over the reference tiles only;
                     r = 1 reproduces the unrestricted key lists
  geometry (128)     closed-form tile counts and extents for (4, 8, 4) and
                     (8, 4, 4) boxes; raster slot order; 128-token prefix cuts
  fine / fine_item   sparsity 0 == torch SDPA (float64) on the packed
                     sequence; prefix rows == dense rows at any sparsity;
                     token-level masked dense attention on tiny grids
  coarse             closed form on tile-constant inputs (== dense attention);
                     all-equal pooled keys -> mean of pooled values
  combine            gate 0 -> out == o; tile-constant inputs, gate 1 ->
                     out == 2 * dense; per-channel gates
  e4m3_encode/decode codes printed in the OCP definition (0, smallest
                     subnormal, 1, 448, NaN...); every finite code round
                     trips; every midpoint rounds to the even code (exact
                     rationals); torch's float8_e4m3fn cast in range;
                     saturation
  quantize_rows      the largest element maps to +-448 exactly; relative
                     error at most 2^-4 for normal codes; zero rows
  qk_norm_rope       a hand-computed 2-channel row; exact invariance under
                     power-of-two scaling (eps 0); unit RMS with unit
                     weights; identity and quarter-turn tables; one pair
                     against Python complex multiplication; rotation keeps
                     pair norms; dot products depend only on the position
                     difference
No function here is marked "parity unpinned"; the numeric values of a real
FastH3 forward are not printed anywhere on the pages, so parity rests on the
pins above.
"""
from __future__ import annotations

import math
import time
from dataclasses import dataclass

import numpy as np

TEXT, COND, AUDIO, VIDEO = 0, 1, 2, 3
TILE_TOKENS = 64
TILE_DIMS = (4, 4, 4)
TILE_TOKEN_COUNTS = (64, 128)      # video tile volumes that are defined (R22)


class GeometryError(ValueError):
    pass


@dataclass
class Geometry:
    L: int
    P: int                  # prefix tiles
    NV: int                 # video tiles
    tiles: list             # per tile: int64 array of packed indices in slot order
    tile_tag: np.ndarray    # [Nt] segment tag of each tile
    grid: tuple
    tile_dims: tuple = TILE_DIMS

    @property
    def Nt(self) -> int:
        return self.P + self.NV

    @property
    def tile_tokens(self) -> int:
        return int(np.prod(self.tile_dims))

    @property
    def valid(self) -> np.ndarray:
        return np.array([len(t) for t in self.tiles], dtype=np.int64)

    def tile_of_token(self) -> np.ndarray:
        out = np.full(self.L, -1, dtype=np.int64)
        for j, idx in enumerate(self.tiles):
            out[idx] = j
        return out

    def slot_of_token(self) -> np.ndarray:
        out = np.full(self.L, -1, dtype=np.int64)
        for idx in self.tiles:
            out[idx] = np.arange(len(idx))
        return out

    def perm(self) -> np.ndarray:
        """[Nt, tile_tokens] packed index of each slot, -1 for pad slots."""
        p = np.full((self.Nt, self.tile_tokens), -1, dtype=np.int64)
        for j, idx in enumerate(self.tiles):
            p[j, :len(idx)] = idx
        return p


def topk_count(n_video_tiles: int, sparsity: float) -> int:
    """The VSA-H3 top-k rule (FastH3 4-step Preview, "Video Sparse Attention is
    not optional here"), in IEEE double as written (reading R6)."""
    if n_video_tiles <= 0:
        return 0
    s = float(sparsity)
    return max(1, min(math.ceil((1.0 - s) * n_video_tiles), n_video_tiles))


def ref_keep_count(n_ref_tiles: int, keep: float) -> int:
    """Reference tiles kept per video query tile under keep ratio r (R23), in
    IEEE double like the top-k rule."""
    if n_ref_tiles <= 0:
        return 0
    return max(1, min(math.ceil(float(keep) * n_ref_tiles), n_ref_tiles))


def geometry(token_tags, position_ids, grid, tile=TILE_DIMS) -> Geometry:
    """Tile geometry from tags and positions (readings R9-R13, R22)."""
    tile = tuple(int(d) for d in tile)
    if len(tile) != 3 or min(tile) < 1 or int(np.prod(tile)) not in TILE_TOKEN_COUNTS:
        raise GeometryError("a video tile is a box of 64 or 128 grid cells")
    tt, ty, tx = tile
    n_tile = tt * ty * tx
    tags = np.asarray(token_tags, dtype=np.int64).reshape(-1)
    pos = np.asarray(position_ids, dtype=np.int64).reshape(-1, 3)
    L = tags.shape[0]
    if pos.shape[0] != L:
        raise GeometryError("position_ids length differs from token_tags")
    if np.any((tags < 0) | (tags > 3)):
        raise GeometryError("unknown segment tag")
    is_video = tags == VIDEO
    nvid = int(is_video.sum())
    n_pre = L - nvid
    if np.any(is_video[:n_pre]):
        raise GeometryError("video tokens must follow every prefix token")
    T, H, W = (int(g) for g in grid)
    if min(T, H, W) < 0 or T * H * W != nvid:
        raise GeometryError("video token count does not match the grid")

    tiles, tile_tag = [], []
    # Prefix: maximal runs of one tag, cut into tile-sized chunks in packed order.
    start = 0
    while start < n_pre:
        end = start
        while end < n_pre and tags[end] == tags[start]:
            end += 1
        for c in range(start, end, n_tile):
            tiles.append(np.arange(c, min(c + n_tile, end), dtype=np.int64))
            tile_tag.append(int(tags[start]))
        start = end
    P = len(tiles)

    NV = 0
    if nvid:
        vidx = np.nonzero(is_video)[0]
        vp = pos[vidx]
        t, y, x = vp[:, 0], vp[:, 1], vp[:, 2]
        if np.any((t < 0) | (t >= T) | (y < 0) | (y >= H) | (x < 0) | (x >= W)):
            raise GeometryError("video position outside the grid")
        cell = (t * H + y) * W + x
        if np.unique(cell).shape[0] != nvid:
            raise GeometryError("duplicate video position")
        nt, nh, nw = -(-T // tt), -(-H // ty), -(-W // tx)
        NV = nt * nh * nw
        vtile = ((t // tt) * nh + (y // ty)) * nw + (x // tx)
        # order: by video tile, then (t, y, x) raster inside it
        order = np.lexsort((x, y, t, vtile))
        sorted_tile = vtile[order]
        bounds = np.searchsorted(sorted_tile, np.arange(NV + 1))
        for j in range(NV):
            tiles.append(vidx[order[bounds[j]:bounds[j + 1]]])
            tile_tag.append(VIDEO)
    return Geometry(L=L, P=P, NV=NV, tiles=tiles, tile_tag=np.array(tile_tag, np.int64),
                    grid=(T, H, W), tile_dims=tile)


def to_f32(x) -> np.ndarray:
    """Exact conversion of an input tensor (bf16 or fp32, torch or numpy) to fp32."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    if a.dtype != np.float32:
        raise TypeError("expected fp32 values")
    return a


def pool_canonical(x32: np.ndarray, geom: Geometry) -> np.ndarray:
    """Per-tile mean of one head's rows, [L, D] fp32 -> [Nt, D] fp32 (R1, R8).

    acc starts at +0 and adds the tile's rows one by one in slot order, each
    addition rounded to fp32; the mean is one correctly rounded fp32 division.
    """
    D = x32.shape[1]
    perm = geom.perm()
    n = geom.valid
    acc = np.zeros((geom.Nt, D), dtype=np.float32)
    for s in range(geom.tile_tokens):
        live = np.nonzero(s < n)[0]
        if live.size == 0:
            break
        acc[live] = np.add(acc[live], x32[perm[live, s]], dtype=np.float32)
    return np.divide(acc, n.astype(np.float32)[:, None], dtype=np.float32)


def scores_canonical(qp: np.ndarray, kp: np.ndarray) -> np.ndarray:
    """S[i, j] = sum_d qp[i, d] * kp[j, d] in the fixed fp32 order of R8."""
    nq, D = qp.shape
    S = np.zeros((nq, kp.shape[0]), dtype=np.float32)
    prod = np.empty_like(S)
    for d in range(D):
        np.multiply.outer(qp[:, d], kp[:, d], out=prod)
        np.add(S, prod, out=S)
    return S


def select_topk(S: np.ndarray, geom: Geometry, topk: int) -> np.ndarray:
    """Top-k video key tiles of each video query tile (R7), ascending.

    Returns int32 [NV, topk] of global tile indices (P..Nt-1).
    """
    P, NV = geom.P, geom.NV
    if NV == 0:
        return np.zeros((0, topk), dtype=np.int32)
    rows = S[P:, P:]
    order = np.argsort(-rows, axis=1, kind="stable")[:, :topk]
    return (np.sort(order, axis=1) + P).astype(np.int32)


def select_ref(S: np.ndarray, geom: Geometry, kr: int) -> np.ndarray:
    """The kr reference key tiles (tag cond) of each video query tile with the
    highest scores, ties to the lower index (R23), ascending.

    Returns int32 [NV, kr] of global tile indices."""
    ref = np.nonzero(geom.tile_tag == COND)[0]
    if geom.NV == 0 or kr == 0:
        return np.zeros((geom.NV, 0), dtype=np.int32)
    rows = S[geom.P:][:, ref]
    order = np.argsort(-rows, axis=1, kind="stable")[:, :kr]
    return np.sort(ref[order], axis=1).astype(np.int32)


def key_tiles(geom: Geometry, sel: np.ndarray, i: int, ref_sel=None) -> np.ndarray:
    """Key tiles visited by query tile i: all tiles for a prefix query tile;
    for a video query tile the prefix tiles (only the selected ones among the
    reference tiles when ``ref_sel`` is given) plus the selected video tiles."""
    if i < geom.P:
        return np.arange(geom.Nt)
    prefix = np.arange(geom.P)
    if ref_sel is not None:
        prefix = np.concatenate([prefix[geom.tile_tag[:geom.P] != COND],
                                 ref_sel[i - geom.P].astype(np.int64)])
    return np.concatenate([prefix, sel[i - geom.P].astype(np.int64)])


def fine_item(q64: np.ndarray, k64: np.ndarray, v64: np.ndarray, geom: Geometry,
              sel: np.ndarray, i: int, scale: float, ref_sel=None) -> np.ndarray:
    """Softmax attention of query tile i's valid rows over the valid tokens of
    its key tiles (float64, one head).  Returns [n_i, D]."""
    rows = geom.tiles[i]
    keys = np.concatenate([geom.tiles[j] for j in key_tiles(geom, sel, i, ref_sel)])
    logits = (q64[rows] @ k64[keys].T) * scale
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v64[keys]


def fine(q64, k64, v64, geom: Geometry, sel: np.ndarray, scale: float,
         items=None, ref_sel=None) -> np.ndarray:
    """Fine branch of one head for all query tiles (or ``items``): [L, D] float64,
    rows of tiles not computed are NaN."""
    out = np.full((geom.L, q64.shape[1]), np.nan)
    for i in (range(geom.Nt) if items is None else items):
        out[geom.tiles[i]] = fine_item(q64, k64, v64, geom, sel, i, scale, ref_sel)
    return out


def coarse(S: np.ndarray, vp: np.ndarray, scale: float) -> np.ndarray:
    """c[i] = sum_j softmax_j(S[i, j] * scale) * vp[j] over all key tiles (R2, R3),
    float64.  Returns [Nt, D]."""
    C = S.astype(np.float64) * scale
    C -= C.max(axis=1, keepdims=True)
    p = np.exp(C)
    p /= p.sum(axis=1, keepdims=True)
    return p @ vp.astype(np.float64)


def combine(o: np.ndarray, g: np.ndarray, c: np.ndarray, geom: Geometry) -> np.ndarray:
    """out[r] = o[r] + gate[r] * c[tile(r)] (R4, R5), float64, one head."""
    tile = geom.tile_of_token()
    return o + g.astype(np.float64) * c[tile]


def qk_norm_rope(x32: np.ndarray, weight: np.ndarray, eps: float, cos: np.ndarray,
                 sin: np.ndarray) -> np.ndarray:
    """RMS norm over the last axis, then RoPE on interleaved pairs, in the
    canonical fp32 order of R14-R16.  x32 [L, D] fp32 (one head), weight [D],
    cos / sin [L, D/2] fp32.  Returns [L, D] fp32 (before the R17 rounding)."""
    x = np.asarray(x32, dtype=np.float32)
    L, D = x.shape
    f32 = np.float32
    ss = np.zeros(L, dtype=f32)
    for d in range(D):
        ss = np.add(ss, np.multiply(x[:, d], x[:, d], dtype=f32), dtype=f32)
    ms = np.divide(ss, f32(D), dtype=f32)
    r = np.sqrt(np.add(ms, f32(eps), dtype=f32), dtype=f32)
    inv = np.divide(f32(1.0), r, dtype=f32)
    y = np.multiply(np.multiply(x, inv[:, None], dtype=f32),
                    np.asarray(weight, dtype=f32)[None, :], dtype=f32)
    a, b = y[:, 0::2], y[:, 1::2]
    c = np.asarray(cos, dtype=f32)
    s = np.asarray(sin, dtype=f32)
    out = np.empty_like(y)
    out[:, 0::2] = np.subtract(np.multiply(a, c, dtype=f32), np.multiply(b, s, dtype=f32),
                               dtype=f32)
    out[:, 1::2] = np.add(np.multiply(a, s, dtype=f32), np.multiply(b, c, dtype=f32), dtype=f32)
    return out


E4M3_MAX = 448.0


def e4m3_decode(code) -> np.ndarray:
    """OCP FP8 E4M3 code (uint8) -> float64 (R19): sign, 4-bit exponent with
    bias 7, 3-bit mantissa; exponent 0 is subnormal; S.1111.111 is NaN."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


_E4M3_POS = e4m3_decode(np.arange(127))        # the 127 finite non-negative values, ascending


def e4m3_encode(x) -> np.ndarray:
    """float64 -> OCP FP8 E4M3 code, nearest with ties to the even code,
    saturating at +-448 (R19).  NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a == _E4M3_POS[hi], hi, np.where(pick_hi, hi, lo)).astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    return np.where(np.isnan(x), 0x7F, code).astype(np.uint8)


def quantize_rows(x32: np.ndarray):
    """Per-row FP8 quantisation of R20.  x32 [N, D] fp32 -> (codes uint8
    [N, D], scale fp32 [N])."""
    x = np.asarray(x32, dtype=np.float32)
    f32 = np.float32
    amax = np.abs(x).max(axis=1)
    nz = amax > 0
    inv = np.where(nz, np.divide(f32(E4M3_MAX), np.where(nz, amax, f32(1)), dtype=f32), f32(0))
    y = np.multiply(x, inv[:, None], dtype=f32)
    codes = e4m3_encode(y.astype(np.float64))
    scale = np.where(nz, np.divide(amax, f32(E4M3_MAX), dtype=f32), f32(0)).astype(np.float32)
    return codes, scale


def dequantize_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """s * decode(code), float64 [N, D] (R20, R21)."""
    return scale.astype(np.float64)[:, None] * e4m3_decode(codes)


def round_bf16_from_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as
    float64.  One rounding step, straight from float64."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        _, e = np.frexp(x)
        e = np.maximum(e, -125)                 # below 2^-126: fixed 2^-133 quantum
        q = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
        big = (2.0 - 2.0 ** -7) * 2.0 ** 127
        q = np.where(np.abs(q) > big, np.copysign(np.inf, x), q)
    return np.where(np.isfinite(x), q, x)


@dataclass
class HeadResult:
    qp: np.ndarray
    kp: np.ndarray
    vp: np.ndarray
    S: np.ndarray
    sel: np.ndarray
    c: np.ndarray
    o: np.ndarray | None        # [L, D] float64 (NaN rows where not computed)
    out: np.ndarray | None      # [L, D] float64 before I/O rounding
    ref_sel: np.ndarray | None = None   # [NV, kr] with a reference keep ratio below 1


def forward_head(q, k, v, gate, geom: Geometry, topk: int, h: int, items=None,
                 with_fine: bool = True, qk_fp8: bool = False,
                 ref_keep: float = 1.0, timings: dict | None = None) -> HeadResult:
    """The whole forward for head h.  q, k, v, gate: [L, H, D] (torch or numpy).
    qk_fp8: the fine branch uses per-token FP8 q and k (R19-R21).
    ref_keep: reference keep ratio r of R23 (1 keeps every reference tile).
    timings: if a dict is given, the wall seconds of each step are added to
    it under "pool", "scores", "topk", "coarse", "fine" and "combine"."""
    clock = [time.perf_counter()]

    def lap(name):
        if timings is not None:
            t = time.perf_counter()
            timings[name] = timings.get(name, 0.0) + t - clock[0]
            clock[0] = t

    qh = to_f32(q[:, h, :])
    kh = to_f32(k[:, h, :])
    vh = to_f32(v[:, h, :])
    D = qh.shape[1]
    scale = 1.0 / math.sqrt(D)
    qp = pool_canonical(qh, geom)
    kp = pool_canonical(kh, geom)
    vp = pool_canonical(vh, geom)
    lap("pool")
    S = scores_canonical(qp, kp)
    lap("scores")
    sel = select_topk(S, geom, topk)
    ref_sel = None
    if not 0.0 < ref_keep <= 1.0:
        raise ValueError("the reference keep ratio must lie in (0, 1]")
    if ref_keep < 1.0:
        ref_sel = select_ref(S, geom, ref_keep_count(int(np.sum(geom.tile_tag == COND)),
                                                     ref_keep))
    lap("topk")
    c = coarse(S, vp, scale)
    lap("coarse")
    o = out = None
    if with_fine:
        if qk_fp8:
            q64 = dequantize_rows(*quantize_rows(qh))
            k64 = dequantize_rows(*quantize_rows(kh))
        else:
            q64, k64 = qh.astype(np.float64), kh.astype(np.float64)
        o = fine(q64, k64, vh.astype(np.float64), geom, sel, scale, items, ref_sel)
        lap("fine")
        out = combine(o, to_f32(gate[:, h, :]), c, geom)
        lap("combine")
    return HeadResult(qp, kp, vp, S, sel, c, o, out, ref_sel)


def prep_qk(q, k, q_weight, k_weight, eps, cos, sin):
    """R14-R17 on every head: returns the attention inputs (q', k') as float32
    arrays [L, H, D] holding bf16 values when q is bf16 (else fp32 values)."""
    qa = to_f32(q)
    ka = to_f32(k)
    is_bf16 = str(getattr(q, "dtype", "")).endswith("bfloat16")
    outs = []
    for x, wgt in ((qa, q_weight), (ka, k_weight)):
        y = np.empty_like(x)
        for h in range(x.shape[1]):
            r = qk_norm_rope(x[:, h, :], wgt, eps, cos, sin)
            y[:, h, :] = (round_bf16_from_f64(r.astype(np.float64)).astype(np.float32)
                          if is_bf16 else r)
        outs.append(y)
    return outs[0], outs[1]


def forward(q, k, v, gate, token_tags, position_ids, grid, sparsity, tile=TILE_DIMS,
            heads=None, ref_keep: float = 1.0):
    """Whole VSA-H3 forward on all (or the listed) heads.

    Returns a dict with
      out   [L, H, D] float64, already rounded to the I/O dtype's values
            (bf16 or fp32 inputs decide), NaN for heads not computed;
      o, c, qp, kp, vp, S, sel per head (lists indexed by head);
      geom, topk.
    """
    geom = geometry(token_tags, position_ids, grid, tile)
    topk = topk_count(geom.NV, sparsity)
    L, H, D = q.shape
    hs = range(H) if heads is None else heads
    is_bf16 = str(getattr(q, "dtype", "")).endswith("bfloat16")
    out = np.full((L, H, D), np.nan)
    res = {"geom": geom, "topk": topk, "heads": {}}
    for h in hs:
        r = forward_head(q, k, v, gate, geom, topk, h, ref_keep=ref_keep)
        out[:, h, :] = (round_bf16_from_f64(r.out) if is_bf16
                        else r.out.astype(np.float32).astype(np.float64))
        res["heads"][h] = r
    res["out"] = out
    return res

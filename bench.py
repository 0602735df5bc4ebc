"""Benchmark of the VSA-H3 attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 768p10s]

One step is one whole forward (permute+pool, coarse branch + top-k, fine
block-sparse attention with the fused gate-combine epilogue) over the
768p 10-s layout: 73,600 tokens (1,024 prefix + 18x48x84 video), 56 heads,
head_dim 128, bf16, sparsity 0.8 (topk 252), on seeded synthetic inputs that
are resident in HBM before the timed region starts.

Prints one JSON line.  ``value`` is the effective throughput in TFLOP/s: the
algorithmic FLOPs of the selected blocks (valid tokens only, from this run's
own selection) plus the coarse branch, divided by the measured time per
forward.  ``roofline`` covers the dominant kernel (fine attention) from HIP
events recorded on the kernels' stream around each launch; ``cpu_baseline``
times the CPU oracle on one head of the same workload (a bounded sample) and
also checks the GPU output of that head against it.  ``configs`` repeats the
measurement on the other workloads (480p 5 s, the structured 768p 10-s and
15-s clips at sparsity 0.9, the OmniRef profile), each with its head-0 parity
against the oracle.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 flop/clk (MI355X dense bf16 MFMA)
PEAK_FP8_TFLOPS = 5033.2      # dense FP8 MFMA, twice the bf16 rate
PEAK_HBM_GBS = 8000.0
METRIC = "VSA-H3 fwd ms and effective TFLOP/s (% bf16 MFMA peak) at 73.6k tokens"
FINE_SOURCES = ["video_dit_block_amd/csrc/fine_attn.hip", "video_dit_block_amd/csrc/device.hpp",
                "video_dit_block_amd/csrc/kernels.hpp", "video_dit_block_amd/csrc/plan.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fine_attn_{workload}_traffic.json")
# Timed after the headline workload and reported in the configs array: the
# 480p 5-s clip, the 768p 10-s and 15-s clips with structured q/k at sparsity
# 0.9, and the OmniRef profile (128-token tiles, reference keep 0.1).
EXTRA_WORKLOADS = ("480p5s", "768p10s_smooth", "768p15s_smooth", "omniref768p10s")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles from the HIP runtime (the stage events are recorded
    by the library on the stream its kernels run on)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def _blocks(valid: np.ndarray, tile_tokens: int) -> np.ndarray:
    """Valid tokens of each 64-slot block of every tile: [Nt, tile_tokens / 64]."""
    b = np.arange(tile_tokens // 64)
    return np.clip(valid.astype(np.int64)[:, None] - 64 * b[None, :], 0, 64)


def fine_flops(sel: np.ndarray, valid: np.ndarray, P: int, L: int, D: int, fixed=None,
               tile_tokens: int = 64) -> tuple[float, float]:
    """Algorithmic fine-branch FLOPs (valid tokens only) and the padded-block
    FLOPs the MFMA executes, for one forward.  sel: [H, NV, n] selected key
    tiles (global ids) of each video query tile; fixed: the prefix tiles every
    video query tile visits besides them (default: all P prefix tiles).  The
    kernel works on 64-slot blocks: each query block that holds a token meets
    every block that holds a key in each listed key tile."""
    H, NV, nsel = sel.shape
    fixed = np.arange(P) if fixed is None else np.asarray(fixed, np.int64)
    n = valid.astype(np.float64)
    per_row = float(n[fixed].sum()) + n[sel].sum(axis=2)      # [H, NV] keys per video query
    video = float((per_row * n[P:][None, :]).sum())
    prefix = float(n[:P].sum()) * L * H
    alg = 4.0 * D * (video + prefix)
    nb = (_blocks(valid, tile_tokens) > 0).sum(axis=1).astype(np.float64)   # blocks with a token
    keys_video = float(nb[fixed].sum()) + nb[sel].sum(axis=2)               # [H, NV]
    pairs = float((keys_video * nb[P:][None, :]).sum()) + H * float(nb[:P].sum()) * float(nb.sum())
    padded = 4.0 * D * 64 * 64 * pairs
    return alg, padded


def kv_stream_bytes(sel: np.ndarray, valid: np.ndarray, P: int, D: int, qk_fp8: bool,
                    fixed=None, tile_tokens: int = 64) -> float:
    """Bytes of K and V^T the fine kernel streams from L2 into LDS in one
    forward: each query item visits every 64-slot block that holds a key in
    its key tiles (sel and fixed as for fine_flops), and a block visit brings
    the block's 32-key halves that hold a valid key, each a K half (32 keys x
    D, bf16 or E4M3 codes plus 32 fp32 scales) and a V^T half (D x 32 keys,
    bf16).  A query item is a whole 128-token tile (its two query blocks
    share one workgroup), except with FP8 keys at head_dim 64, and with
    64-token tiles a query block."""
    H, NV, nsel = sel.shape
    fixed = np.arange(P) if fixed is None else np.asarray(fixed, np.int64)
    bv = _blocks(valid, tile_tokens)
    halves = (bv > 0) * (1.0 + (bv > 32))
    kh = 32 * D * (1 if qk_fp8 else 2) + (32 * 4 if qk_fp8 else 0)
    vh = 32 * D * 2
    per_tile = (halves * (kh + vh)).sum(axis=1)                 # [Nt]
    if tile_tokens == 128 and not (qk_fp8 and D == 64):
        qb = np.ones(bv.shape[0])                               # one item per query tile
    else:
        qb = (bv > 0).sum(axis=1).astype(np.float64)           # query blocks with a token
    prefix_rows = float(qb[:P].sum()) * float(per_tile.sum()) * H
    per_row = float(per_tile[fixed].sum()) + per_tile[sel].sum(axis=2)   # [H, NV]
    video_rows = float((per_row * qb[P:][None, :]).sum())
    return prefix_rows + video_rows


def fixed_prefix_tiles(plan, token_tags) -> np.ndarray:
    """Prefix tiles every video query tile visits besides its selection: all
    of them, or with a reference selection those whose tag is not cond."""
    P = plan.num_prefix_tiles
    if plan.topk_ref == 0:
        return np.arange(P)
    perm, _, _ = plan.tables()
    tags = np.asarray(token_tags).reshape(-1)
    return np.array([j for j in range(P) if tags[perm[j, 0]] != 1], np.int64)


def sources_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(launches: int, workload: str, chunk_tiles: int):
    """HBM bytes per fine-attention launch (the forward's fine-branch bytes over
    its key-chunk launches) from the committed counter summary, or None if it
    is missing or was taken on a different workload, kernel source or key-chunk
    schedule."""
    try:
        with open(TRAFFIC_FILE.format(workload=workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload:
        return None
    if t.get("kernel_sources_sha256") != sources_digest(FINE_SOURCES):
        return None
    if t.get("launches_per_forward") != launches or t.get("key_chunk_tiles") != chunk_tiles:
        return None
    return t.get("bytes_per_launch")


def host_cpu() -> dict:
    """The host's logical CPU count, CPU model and the thread counts of the
    BLAS and OpenMP pools the oracle's NumPy calls run on."""
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    pools = []
    try:
        from threadpoolctl import threadpool_info
        pools = [{"api": i.get("user_api"), "library": i.get("internal_api"),
                  "threads": int(i.get("num_threads", 1))} for i in threadpool_info()]
    except Exception:  # pragma: no cover
        pass
    blas = [p["threads"] for p in pools if p["api"] == "blas"]
    return {"host_cpus": os.cpu_count(), "cpu_model": model,
            "blas_threads": max(blas) if blas else None, "thread_pools": pools}


def oracle_head(x, w, head=0):
    """The oracle's whole forward of one head, with the seconds of each step."""
    import oracle
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid, w.tile)
    topk = oracle.topk_count(g.NV, w.sparsity)
    stages = {}
    t0 = time.perf_counter()
    r = oracle.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, head,
                            ref_keep=w.ref_keep, timings=stages)
    return g, r, time.perf_counter() - t0, stages


def head_parity(g, r, gpu_out, gpu_sel, head=0):
    """Selection (bit-exact) and output error of one head against the oracle."""
    import oracle
    sel_o = r.sel if r.ref_sel is None else np.concatenate([r.ref_sel, r.sel], axis=1)
    ref = oracle.round_bf16_from_f64(r.out)
    got = gpu_out[:, head, :].to("cpu").double().numpy()
    d = got - ref
    return sel_o, {"head": head, "sel_bit_exact": bool(np.array_equal(gpu_sel[head], sel_o)),
                   "max_abs": float(np.abs(d).max()),
                   "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref)),
                   "bar": {"max_abs": 2e-2, "rel_l2": 5e-3}}


def oracle_flops(g, sel_o, w, head_dim):
    import oracle
    fixed = None
    if sel_o.shape[1] != oracle.topk_count(g.NV, w.sparsity):
        fixed = np.nonzero(g.tile_tag[:g.P] != oracle.COND)[0]
    alg, _ = fine_flops(sel_o[None].astype(np.int64), g.valid, g.P, g.L, head_dim, fixed,
                        g.tile_tokens)
    return alg + 4.0 * head_dim * g.Nt ** 2


def cpu_baseline(x, w, gpu_out, gpu_sel, head=0):
    """Time the oracle (as it stands) on one head of the workload and check the
    GPU's output and selection for that head against it."""
    hc = host_cpu()
    g, r, secs, stages = oracle_head(x, w, head)
    sel_o, parity = head_parity(g, r, gpu_out, gpu_sel, head)
    flops = oracle_flops(g, sel_o, w, w.head_dim)
    cb = {"value": flops / secs / 1e12, "unit": "TFLOP/s",
          # the float64 fine branch (all but a few % of the time) is BLAS
          # matrix products; the other steps run on one thread
          "cores": hc["blas_threads"] or 1,
          "kind": "oracle", "seconds": secs, "heads_timed": 1, "heads_total": w.heads,
          "sample": f"head {head} of {w.heads} of the {w.name} workload (whole per-head forward: "
                    "pool, scores, top-k, coarse, float64 fine branch, combine); value = that "
                    "head's effective flops over its wall time",
          "host_cpus": hc["host_cpus"], "cpu_model": hc["cpu_model"],
          "blas_threads": hc["blas_threads"], "thread_pools": hc["thread_pools"],
          "stage_s": {k: round(v, 4) for k, v in stages.items()}}
    return cb, parity


def run_forward(w, args, torch, vsa, dev, qk_prep=False, qk_fp8=False, chunk_tiles=0,
                calibrate=False):
    """Seeded inputs of workload w in HBM, one plan, W untimed and K timed
    forwards with HIP events around each stage.  Returns the pieces the
    reports need."""
    from workloads import make_inputs, make_qk_prep_inputs
    t = time.perf_counter()
    x = make_inputs(w, seed=0)
    log(f"bench: {w.name}: inputs generated in {time.perf_counter() - t:.1f}s")
    xd = {n: x[n].to(dev) for n in ("q", "k", "v", "gate")}
    plan = vsa.Plan(x["token_tags"], x["position_ids"], w.grid, w.heads, w.head_dim, w.sparsity,
                    w.tile, chunk_tiles=chunk_tiles, qk_prep=qk_prep, qk_fp8=qk_fp8,
                    ref_keep=w.ref_keep)
    stream = torch.cuda.current_stream(dev)
    ws = plan.workspace(dev, stream.cuda_stream)
    out = torch.empty_like(xd["q"])
    sel = torch.empty((w.heads, plan.num_video_tiles, plan.sel_width), dtype=torch.int32,
                      device=dev)
    io = vsa.VSA_BF16 if w.io_dtype == "bf16" else vsa.VSA_F32
    ptrs = [xd[n].data_ptr() for n in ("q", "k", "v", "gate")]

    if calibrate:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)                      # calibration copy: 1 GiB read + 1 GiB written
        torch.cuda.synchronize()
        del src, dst

    hip = HipEvents()
    evs = [hip.create(4) for _ in range(args.steps)]
    if qk_prep:
        prep = make_qk_prep_inputs(w, x["position_ids"])
        pd = {n: prep[n].to(dev) for n in ("q_weight", "k_weight", "cos", "sin")}

    def step(events=None):
        if qk_prep:
            vsa.vsa_h3_forward_qk_prep(plan.handle, *ptrs, pd["q_weight"].data_ptr(),
                                       pd["k_weight"].data_ptr(), prep["eps"],
                                       pd["cos"].data_ptr(), pd["sin"].data_ptr(), io,
                                       out.data_ptr(), sel.data_ptr(), ws.data_ptr(),
                                       plan.workspace_bytes, stream.cuda_stream, events)
        else:
            vsa.vsa_h3_forward_timed(plan.handle, *ptrs, io, out.data_ptr(), sel.data_ptr(),
                                     ws.data_ptr(), plan.workspace_bytes, stream.cuda_stream,
                                     events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    stage = np.array([[hip.elapsed_ms(e[a], e[a + 1]) for a in range(3)] for e in evs])
    event_ms = np.array([hip.elapsed_ms(e[0], e[3]) for e in evs])
    for e in evs:
        hip.destroy(e)
    log(f"bench: {w.name}: {args.steps} timed steps, {ms_per_step:.3f} ms/step (wall), "
        f"{event_ms.mean():.3f} ms/step (events)")

    perm, valid, _ = plan.tables()
    sel_h = sel.cpu().numpy()
    fixed = fixed_prefix_tiles(plan, x["token_tags"])
    alg_fine, padded_fine = fine_flops(sel_h.astype(np.int64), valid, plan.num_prefix_tiles,
                                       plan.L, w.head_dim, fixed, plan.tile_tokens)
    kv_bytes = kv_stream_bytes(sel_h.astype(np.int64), valid, plan.num_prefix_tiles, w.head_dim,
                               bool(qk_fp8), fixed, plan.tile_tokens)
    coarse_flops = 4.0 * w.head_dim * plan.num_tiles ** 2 * w.heads
    total = alg_fine + coarse_flops
    fine_ms = float(stage[:, 2].mean())
    # With FP8 q/k half of the fine flops (Q.K) run at the dense FP8 rate and
    # half (P.V) at the bf16 rate: the peak of that mix is their harmonic mean.
    fine_peak = (2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS) if qk_fp8
                 else PEAK_BF16_TFLOPS)
    out_host = out.cpu()
    r = {"x": x, "plan": plan, "out": out_host, "sel": sel_h, "ms": ms_per_step,
         "event_ms": float(event_ms.mean()), "stage_ms": stage.mean(axis=0),
         "alg_fine": alg_fine, "padded_fine": padded_fine, "kv_bytes": kv_bytes, "total": total,
         "tflops": total / (ms_per_step * 1e-3) / 1e12, "fine_ms": fine_ms,
         "fine_tflops": alg_fine / (fine_ms * 1e-3) / 1e12, "fine_peak": fine_peak,
         "launches": max(plan.num_chunks, 1)}
    del xd, ws, out, sel
    plan.release_workspaces()
    torch.cuda.empty_cache()
    return r


def copy_tbps(torch, dev, reps=5) -> float:
    """Read + write bandwidth of a 1 GiB device-to-device copy on this GPU,
    in TB/s of bytes moved: the practical ceiling of a kernel whose traffic
    mixes reads and writes, as the gather's does."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * n / (ms * 1e-3) / 1e12


def gather_bytes(plan, w, qk_prep=False, qk_fp8=False) -> float:
    """Algorithmic HBM bytes of the tile-permute gather with pooling: q, k, v
    read once; K (bf16, or E4M3 codes and per-key scales) and V^T written per
    64-slot block (pad slots included, they are stored zero), low parts with
    fp32 I/O, Qt with QK-norm + RoPE; the pooled q, k, v tiles in fp32."""
    es = 2 if w.io_dtype == "bf16" else 4
    L, H, D, Nb, Nt = plan.L, w.heads, w.head_dim, plan.num_blocks, plan.num_tiles
    parts = 1 if es == 2 else 2
    blk = H * Nb * 64 * D
    wr = blk * 2 * parts                                   # V^T
    wr += blk * 1 + H * Nb * 64 * 4 if qk_fp8 else blk * 2 * parts   # K
    if qk_prep:
        wr += blk * 2 * parts                              # Qt
    return 3.0 * L * H * D * es + wr + 3.0 * H * Nt * D * 4


def stage_dict(st) -> dict:
    return {"permute_pool": round(float(st[0]), 4), "coarse_topk": round(float(st[1]), 4),
            "fine_attn": round(float(st[2]), 4)}


def config_entry(w, r, with_parity=True) -> dict:
    """One line of the ``configs`` array: time, throughput, fine-kernel
    fraction of peak and head-0 parity for workload w."""
    plan = r["plan"]
    e = {"workload": w.name, "tokens": plan.L, "heads": w.heads, "head_dim": w.head_dim,
         "prefix_tokens": w.n_prefix_tokens, "grid": list(w.grid), "sparsity": w.sparsity,
         "topk": plan.topk, "tiles": plan.num_tiles, "tile": list(w.tile),
         "ref_keep": w.ref_keep, "topk_ref": plan.topk_ref,
         "ms_per_step": round(r["ms"], 4), "tflops_effective": round(r["tflops"], 2),
         "pct_bf16_peak": round(100.0 * r["tflops"] / PEAK_BF16_TFLOPS, 2),
         "stage_ms": stage_dict(r["stage_ms"]),
         "fine": {"achieved": round(r["fine_tflops"], 2), "peak": r["fine_peak"],
                  "unit": "TFLOP/s", "frac": round(r["fine_tflops"] / r["fine_peak"], 4),
                  "launches_per_forward": r["launches"], "key_chunk_tiles": plan.chunk_tiles}}
    if with_parity:
        g, hr, secs, _ = oracle_head(r["x"], w, 0)
        _, parity = head_parity(g, hr, r["out"], r["sel"], 0)
        e["parity"] = parity
        e["oracle_head0_s"] = round(secs, 2)
        log(f"bench: {w.name}: oracle head 0 {secs:.1f}s, parity {parity}")
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="768p10s",
                    help="a workload name from workloads.WORKLOADS, e.g. omniref768p10s "
                         "(128-token tiles, reference keep 0.1)")
    ap.add_argument("--configs", default=",".join(EXTRA_WORKLOADS),
                    help="comma-separated workloads also timed (with head-0 parity against "
                         "the oracle) and reported in the configs array; '' for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chunk-tiles", type=int, default=0,
                    help="key tiles per fine-branch key chunk (0: the library's default)")
    ap.add_argument("--qk-fp8", action="store_true",
                    help="time the forward with per-token FP8 (E4M3) q and k in the fine branch")
    ap.add_argument("--qk-prep", action="store_true",
                    help="time the forward with QK RMS norm + RoPE fused into the gather "
                         "(synthetic weights and cos/sin tables)")
    ap.add_argument("--profile-pass", action="store_true",
                    help="counter runs: one 1 GiB device copy (traffic calibration), then the "
                         "warmup and timed forwards; no CPU baseline, no other configs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the forward is single-GPU; multi-GPU sharding is a design note only)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    sys.path.insert(0, ROOT)
    import video_dit_block_amd as vsa
    from workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    log(f"bench: workload {w.name}: {w.description}")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    r = run_forward(w, args, torch, vsa, dev, args.qk_prep, args.qk_fp8, args.chunk_tiles,
                    calibrate=args.profile_pass)
    plan = r["plan"]
    launches = r["launches"]
    tflops = r["tflops"]
    fine_ms = r["fine_ms"]

    metric = METRIC if w.name == "768p10s" else (
        f"VSA-H3 fwd ms and effective TFLOP/s (% bf16 MFMA peak) at {plan.L / 1000:.1f}k tokens")
    # The gather's HBM traffic against a device copy's read + write rate.
    gb = gather_bytes(plan, w, args.qk_prep, args.qk_fp8)
    cp = copy_tbps(torch, dev)
    g_tbps = gb / (float(r["stage_ms"][0]) * 1e-3) / 1e12
    rec = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8e4m3 QK + bf16 PV" if args.qk_fp8 else "bf16") if w.io_dtype == "bf16"
                 else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "tokens": plan.L, "heads": w.heads, "head_dim": w.head_dim,
            "prefix_tokens": w.n_prefix_tokens, "grid": list(w.grid),
            "sparsity": w.sparsity, "topk": plan.topk, "tiles": plan.num_tiles,
            "tile": list(w.tile), "ref_keep": w.ref_keep, "topk_ref": plan.topk_ref,
            "qk_prep": bool(args.qk_prep), "qk_fp8": bool(args.qk_fp8),
            "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
            "flops_effective": r["total"], "flops_fine_padded_tiles": r["padded_fine"],
            "stage_ms": stage_dict(r["stage_ms"]),
            "event_ms_per_step": round(r["event_ms"], 4),
            "permute_pool_hbm": {"bytes": gb, "achieved_tbps": round(g_tbps, 3),
                                 "copy_tbps": round(cp, 3), "frac_of_copy": round(g_tbps / cp, 4),
                                 "peak_tbps": PEAK_HBM_GBS / 1000.0,
                                 "frac_of_peak": round(g_tbps / (PEAK_HBM_GBS / 1000.0), 4)},
        },
        "roofline": {
            "bound": "mfma", "kernel": "fine_attn_kernel",
            "achieved": round(r["fine_tflops"], 2), "peak": r["fine_peak"], "unit": "TFLOP/s",
            "frac": round(r["fine_tflops"] / r["fine_peak"], 4),
            "traffic": load_traffic(launches, w.name, plan.chunk_tiles),
            "launches_per_forward": launches,
            "key_chunk_tiles": plan.chunk_tiles,
            "algorithmic_flops_per_launch": r["alg_fine"] / launches,
            "avg_launch_ms": round(fine_ms / launches, 4),
            # The kernel's other ceiling: K/V bytes moved from L2 into LDS.
            "kv_stream": {"bytes_per_launch": r["kv_bytes"] / launches,
                          "achieved": round(r["kv_bytes"] / (fine_ms * 1e-3) / 1e12, 2),
                          "unit": "TB/s"},
        },
    }
    if not args.no_cpu_baseline and not args.profile_pass and not args.qk_prep and not args.qk_fp8:
        log("bench: timing the CPU oracle on one head (bounded sample)")
        cb, parity = cpu_baseline(r["x"], w, r["out"], r["sel"])
        rec["cpu_baseline"] = cb
        rec["parity"] = parity
        log(f"bench: oracle head 0: {cb['seconds']:.1f}s, parity {parity}")
    else:
        rec["cpu_baseline"] = None
    del r
    extras = [n for n in args.configs.split(",") if n and n != w.name]
    if args.profile_pass or args.qk_prep or args.qk_fp8:
        extras = []
    rec["configs"] = []
    for name in extras:
        we = WORKLOADS[name]
        log(f"bench: config {we.name}: {we.description}")
        re_ = run_forward(we, args, torch, vsa, dev)
        rec["configs"].append(config_entry(we, re_, with_parity=not args.no_cpu_baseline))
        del re_
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

"""Host-side accounting of bench.py (no GPU): the algorithmic fine-branch
flops and the K/V bytes the fine kernel streams, each against a brute-force
count over every (head, query tile, key tile) visit."""
import numpy as np

import bench
import oracle
from workloads import AUDIO, COND, TEXT, Workload, make_layout


def _geometry():
    # 100 text tokens (one full and one partial prefix tile), a 6x10x10 grid:
    # tiles of 4x4x4 with partial tiles along every axis
    w = Workload("acct", 3, 64, "f32", ((TEXT, 100), (AUDIO, 40)), (6, 10, 10), 0.7)
    tags, pos = make_layout(w)
    g = oracle.geometry(tags, pos, w.grid)
    return w, g


def _random_selection(g, H, topk, seed=0):
    rng = np.random.default_rng(seed)
    return np.stack([np.stack([np.sort(rng.choice(np.arange(g.P, g.Nt), topk, replace=False))
                               for _ in range(g.NV)]) for _ in range(H)])


def _visits(g, sel, h, i):
    return list(range(g.Nt)) if i < g.P else list(range(g.P)) + [int(t) for t in sel[h, i - g.P]]


def test_fine_flops_brute_force():
    w, g = _geometry()
    topk = oracle.topk_count(g.NV, w.sparsity)
    sel = _random_selection(g, w.heads, topk)
    alg, padded = bench.fine_flops(sel, g.valid, g.P, g.L, w.head_dim)
    a = p = 0.0
    for h in range(w.heads):
        for i in range(g.Nt):
            for j in _visits(g, sel, h, i):
                a += 4.0 * w.head_dim * g.valid[i] * g.valid[j]
                p += 4.0 * w.head_dim * 64 * 64
    assert alg == a and padded == p


def test_kv_stream_bytes_brute_force():
    w, g = _geometry()
    topk = oracle.topk_count(g.NV, w.sparsity)
    sel = _random_selection(g, w.heads, topk, seed=1)
    D = w.head_dim
    for fp8 in (False, True):
        got = bench.kv_stream_bytes(sel, g.valid, g.P, D, fp8)
        want = 0
        for h in range(w.heads):
            for i in range(g.Nt):
                for j in _visits(g, sel, h, i):
                    halves = 2 if g.valid[j] > 32 else 1
                    k_half = 32 * D * (1 if fp8 else 2) + (32 * 4 if fp8 else 0)
                    want += halves * (k_half + 32 * D * 2)
        assert got == want, (fp8, got, want)


def test_kv_stream_counts_one_half_for_short_tiles():
    w, g = _geometry()
    assert (g.valid <= 32).any() and (g.valid > 32).any()
    sel = _random_selection(g, w.heads, 1, seed=2)
    full = bench.kv_stream_bytes(sel, np.full_like(g.valid, 64), g.P, w.head_dim, False)
    part = bench.kv_stream_bytes(sel, g.valid, g.P, w.head_dim, False)
    assert part < full


def _wide_geometry():
    # 128-token (4,8,4) tiles: prefix tiles of 128, 72 (one empty second
    # block), 128 + 40 reference tokens and 30 audio tokens; a 6x10x10 grid
    # gives video tiles of 128, 64 (empty second block) and fewer tokens.
    w = Workload("acct128", 2, 64, "f32", ((TEXT, 200), (COND, 168), (AUDIO, 30)), (6, 10, 10),
                 0.6, tile=(4, 8, 4), ref_keep=0.5)
    tags, pos = make_layout(w)
    g = oracle.geometry(tags, pos, w.grid, w.tile)
    assert g.tile_tokens == 128 and (g.valid <= 64).any() and (g.valid <= 32).any()
    return w, g


def _wide_lists(g, H, topk, kr, seed):
    rng = np.random.default_rng(seed)
    ref = np.nonzero(g.tile_tag == COND)[0]
    fixed = np.nonzero((g.tile_tag != COND) & (np.arange(g.Nt) < g.P))[0]
    sel = np.stack([np.stack([np.sort(np.concatenate([
        rng.choice(ref, kr, replace=False), rng.choice(np.arange(g.P, g.Nt), topk, replace=False)]))
        for _ in range(g.NV)]) for _ in range(H)])
    return sel, fixed


def _block_visits(g, sel, fixed, h, i):
    keys = list(range(g.Nt)) if i < g.P else [int(t) for t in fixed] + [int(t) for t in sel[h, i - g.P]]
    for j in keys:
        for b in range(2):
            yield j, b


def test_wide_fine_flops_and_kv_bytes_brute_force_over_blocks():
    """A query block without rows does no work and a key block without keys
    is stepped over.  Both query blocks of a 128-token tile share one
    workgroup and so one K/V stream, except with FP8 keys at head_dim 64,
    where each query block that holds a row streams its own."""
    w, g = _wide_geometry()
    assert (g.valid[g.P:] <= 64).any()
    topk = oracle.topk_count(g.NV, w.sparsity)
    sel, fixed = _wide_lists(g, w.heads, topk, 1, seed=3)
    D = w.head_dim
    alg, padded = bench.fine_flops(sel, g.valid, g.P, g.L, D, fixed, 128)
    bvalid = lambda j, b: int(min(max(g.valid[j] - 64 * b, 0), 64))
    a = p = 0.0
    kv = {False: 0, True: 0}
    kv_half = {fp8: 32 * D * (1 if fp8 else 2) + (128 if fp8 else 0) + 32 * D * 2
               for fp8 in (False, True)}
    for h in range(w.heads):
        for i in range(g.Nt):
            visits = [(j, b) for j, b in _block_visits(g, sel, fixed, h, i) if bvalid(j, b) > 0]
            tile_bytes = sum(2 if bvalid(j, b) > 32 else 1 for j, b in visits)
            kv[False] += tile_bytes * kv_half[False]            # once per query tile
            for qb in range(2):
                if bvalid(i, qb) == 0:
                    continue
                kv[True] += tile_bytes * kv_half[True]          # once per query block
                for j, b in visits:
                    a += 4.0 * D * bvalid(i, qb) * bvalid(j, b)
                    p += 4.0 * D * 64 * 64
    assert alg == a and padded == p
    for fp8 in (False, True):
        assert bench.kv_stream_bytes(sel, g.valid, g.P, D, fp8, fixed, 128) == kv[fp8]
    # at head_dim 128 FP8 keys split over four waves too: once per query tile
    kv128 = kv[False] // kv_half[False] * (32 * 128 + 128 + 32 * 128 * 2)
    assert bench.kv_stream_bytes(sel, g.valid, g.P, 128, True, fixed, 128) == kv128


def test_cpu_baseline_pieces_report_host_and_stage_split():
    # host details: the logical CPU count as the OS reports it, a BLAS pool
    hc = bench.host_cpu()
    import os
    assert hc["host_cpus"] == os.cpu_count()
    assert hc["blas_threads"] is None or hc["blas_threads"] >= 1
    # the oracle's stage split covers every step and adds up to the head's time
    w, g = _geometry()
    from workloads import make_inputs
    x = make_inputs(w, seed=2)
    g2, r, secs, stages = bench.oracle_head(x, w, 1)
    assert set(stages) == {"pool", "scores", "topk", "coarse", "fine", "combine"}
    assert 0.0 < sum(stages.values()) <= secs
    ref = oracle.forward_head(x["q"], x["k"], x["v"], x["gate"], g2,
                              oracle.topk_count(g2.NV, w.sparsity), 1)
    assert np.array_equal(r.out, ref.out) and np.array_equal(r.sel, ref.sel)


def test_traffic_record_is_used_only_for_its_kernel_sources_and_schedule(tmp_path, monkeypatch):
    """roofline.traffic comes from a committed counter record, and only while
    the record matches the fine kernel's current sources (SHA-256), the
    workload and the key-chunk schedule; anything else reports null."""
    import json
    rec = {"workload": "w", "bytes_per_launch": 123, "launches_per_forward": 4,
           "key_chunk_tiles": 319,
           "kernel_sources_sha256": bench.sources_digest(bench.FINE_SOURCES)}
    path = tmp_path / "fine_attn_{workload}_traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    (tmp_path / "fine_attn_w_traffic.json").write_text(json.dumps(rec))
    assert bench.load_traffic(4, "w", 319) == 123
    assert bench.load_traffic(3, "w", 319) is None           # other launch count
    assert bench.load_traffic(4, "w", 426) is None           # other chunk length
    assert bench.load_traffic(4, "other", 319) is None       # no record for the workload
    stale = dict(rec, kernel_sources_sha256="0" * 64)        # kernel changed since
    (tmp_path / "fine_attn_w_traffic.json").write_text(json.dumps(stale))
    assert bench.load_traffic(4, "w", 319) is None
    (tmp_path / "fine_attn_w_traffic.json").write_text("not json")
    assert bench.load_traffic(4, "w", 319) is None


"""Benchmark: selected-token attention queries/s on one MI355X.

A step is one sa_select_attend call over the whole batch: indexer score -> per-row top-k
-> sparse gather attention, inputs resident in HBM.  The headline workload is the largest
one that fits one GPU: the latent (MLA-style) causal prefill with n = 32768 query rows,
128 query heads sharing one 576-wide latent key/value head, 64 index heads of width 128
(e4m3 index keys) and k = 2048.  The bf16 multi-head prefill (B = 2, n = 4096), the
64-request latent decode over a 65536-long cache and the planted-needle decode are timed
under "workloads".

Prints ONE JSON line.  Besides the headline value it reports per-stage times, the
indexer TFLOP/s, a roofline object for the dominant kernel, timed live with HIP events on
the stream the library launches on, and the CPU oracle's rate on a stratified row sample of
the headline workload.  It also reports the p10 / median / p90 of single-step times and
each stage timed with cold caches (a 512 MiB write between calls evicts L2 and the MALL),
the numbers to use for claims against the HBM roofline.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "selected-token attn queries/sec + indexer TFLOP/s & gather GB/s (% roofline)"


def kv_cache_bytes(kv_heads, head_dim, positions, bytes_per):
    """Bytes of one layer's K and V cache for one request: 2 (K and V) x heads x width x positions x bytes."""
    return 2 * kv_heads * head_dim * positions * bytes_per


def visible_counts(W):
    """Visible history length of every query row (0 for padded rows)."""
    import numpy as np

    B, nq = W["B"], W["n_q"]
    i = np.arange(nq)[None, :]
    qp = W["q_pos0"][:, None].astype(np.int64) + i
    kl = W["kv_len"][:, None].astype(np.int64)
    valid = qp < kl
    L = np.minimum(qp + 1, kl) if W["causal"] else np.broadcast_to(kl, (B, nq))
    return np.where(valid, L, 0)


def algorithmic(W):
    """Algorithmic work of one step (visible pairs, selected pairs, FLOPs, gather bytes)."""
    import numpy as np

    L = visible_counts(W)
    pairs = int(L.sum())
    sel = int(np.minimum(L, W["k"]).sum())
    rows = int((L > 0).sum())
    esz = 4 if W["main_dtype"] == 0 else 2
    idx_flops = 2 * W["d_idx"] * W["Hidx"] * pairs
    attn_flops = 2 * W["Hq"] * (W["d_qk"] + W["d_v"]) * sel
    # one gathered history row feeds every head of its key/value group; latent rows carry V inside K
    row_bytes = W["Hkv"] * (W["d_qk"] + (0 if W["mla"] else W["d_v"])) * esz
    q_bytes = W["B"] * W["Hq"] * W["n_q"] * W["d_qk"] * esz
    o_bytes = W["B"] * W["Hq"] * W["n_q"] * W["d_v"] * esz
    idx_bytes = W["B"] * W["n_q"] * W["k"] * 4
    gather = sel * row_bytes + q_bytes + o_bytes + idx_bytes
    # indexer: every visible index key once per query row (decode: the full-history scan), the
    # index queries and weights once, one fp32 score per visible pair written
    kb = {0: 4, 1: 2, 2: 1}[W["kidx_dtype"]]
    qb = {0: 4, 1: 2}[W["qidx_dtype"]]
    idx_scan_bytes = pairs * W["d_idx"] * kb + W["B"] * W["n_q"] * W["Hidx"] * (W["d_idx"] * qb + 4) + pairs * 4
    # top-k: every visible score read once, the selection written once
    topk_bytes = pairs * 4 + idx_bytes
    return dict(pairs=pairs, selected=sel, rows=rows, idx_flops=idx_flops, attn_flops=attn_flops,
                gather_bytes=gather, row_bytes=row_bytes, idx_scan_bytes=idx_scan_bytes, topk_bytes=topk_bytes,
                decode=bool(W.get("decode")) or W["n_q"] <= 8)


def stage_rooflines(W, alg, t):
    """Roofline position of each stage from its algorithmic work and measured time (ms)."""
    def hbm(nbytes, ms):
        a = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "bytes_per_launch": int(nbytes), "ms_per_launch": round(ms, 4)}

    def mfma(flops, ms):
        a = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(a / BF16_PEAK_TFLOPS, 4), "flops_per_launch": int(flops), "ms_per_launch": round(ms, 4)}

    out = {}
    out["indexer_score"] = hbm(alg["idx_scan_bytes"], t["indexer_score"]) if alg["decode"] else \
        mfma(alg["idx_flops"], t["indexer_score"])
    out["topk"] = hbm(alg["topk_bytes"], t["topk"])
    if "select" in t:  # score + select in one call: the indexer's work, no score matrix
        out["select"] = hbm(alg["idx_scan_bytes"] - alg["pairs"] * 4, t["select"]) if alg["decode"] else \
            mfma(alg["idx_flops"], t["select"])
    if not alg["decode"]:
        # prefill attention runs on the matrix cores (latent rows, or the tile kernel for
        # multi-head rows); the logical gather rate is reported beside it
        out["sparse_attn"] = mfma(alg["attn_flops"], t["sparse_attn"])
        out["sparse_attn"]["gather_gbs_logical"] = round(alg["gather_bytes"] / (t["sparse_attn"] * 1e-3) / 1e9, 1)
    else:
        out["sparse_attn"] = hbm(alg["gather_bytes"], t["sparse_attn"])
        # the same launch against the matrix cores: with many query heads per gathered latent
        # row, decode attention does hundreds of FLOPs per gathered byte
        out["sparse_attn"]["mfma_view"] = {k: v for k, v in mfma(alg["attn_flops"], t["sparse_attn"]).items()
                                           if k in ("achieved", "peak", "unit", "frac", "flops_per_launch")}
    for k in out:
        out[k]["kernel"] = k
    return out


def counted_traffic(workload, stage):
    """HBM bytes per launch measured by rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, scaled by a
    plain-copy calibration) as recorded under profiles/, or None when no record exists for this
    workload and stage or the kernel source has changed since the counters were taken."""
    import glob
    import hashlib

    for path in glob.glob(os.path.join(ROOT, "profiles", "*_counters.md")):
        rec = {}
        for line in open(path):
            if ":" in line and not line.startswith((" ", "|", "#")):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
        if rec.get("workload") != workload or rec.get("stage") != stage:
            continue
        src = os.path.join(ROOT, rec.get("source", ""))
        if not os.path.isfile(src):
            return None
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec.get("source_sha256"):
            return None
        return int(float(rec["traffic_bytes_per_launch"]))
    return None


def hisa_stage(W, P, d, stream, timed, reps, flat_idx, t_flat):
    """Hierarchical selection (block representatives, k_b blocks, token top-k inside them)
    timed beside the flat score + select, with the overlap of the two selections.  Block size
    64 and k_b = ceil(2k / 64) kept blocks (candidates about twice the budget).  The
    representatives are index state built once per completed block; their build is timed
    separately and is not part of the selection."""
    import numpy as np
    import torch

    import token_selector_gather_amd as sa

    blk = 64
    kb = -(-2 * W["k"] // blk)
    nb = W["n_kv"] // blk
    if nb < 1 or (kb + 1) * blk > 32768:
        return None
    kbar = torch.empty((W["B"], nb, W["d_idx"]), dtype=torch.bfloat16, device="cuda")
    t_bm = timed(lambda: sa.sa_block_means(P, d["k_idx"], blk, kbar, stream), reps)
    ws_h = sa.hisa_workspace(P, blk, kb)
    idx_h = torch.empty((W["B"], W["n_q"], W["k"]), dtype=torch.int32, device="cuda")
    t_h = timed(lambda: sa.sa_hisa_select(P, d["q_idx"], d["k_idx"], d["w"], kbar, blk, kb, idx_h, ws_h,
                                          stream=stream), reps)
    st = sa.sa_device_status(ws_h)
    if st != sa.SA_OK:
        raise RuntimeError("hierarchical selection: device status " + sa.sa_status_str(st))
    a = idx_h.reshape(-1, W["k"]).cpu().numpy()
    f = flat_idx.reshape(-1, W["k"]).cpu().numpy()
    L = visible_counts(W).reshape(-1)
    iou = [np.intersect1d(x[x >= 0], y[y >= 0]).size / max(1, np.union1d(x[x >= 0], y[y >= 0]).size)
           for x, y, n in zip(a, f, L) if n > 0]
    # algorithmic bytes: every visible complete block's representative (bf16) and every
    # candidate's index key once per row, the selection written once
    kbytes = {0: 4, 1: 2, 2: 1}[W["kidx_dtype"]]
    Pb = L // blk
    ncand = np.minimum(kb, Pb) * blk + (L - Pb * blk)
    nbytes = int((Pb * W["d_idx"] * 2 + ncand * W["d_idx"] * kbytes).sum() + W["B"] * W["n_q"] * W["k"] * 4)
    return {"blk": blk, "k_blocks": kb, "select_ms": round(t_h, 4), "flat_score_select_ms": round(t_flat, 4),
            "speedup_vs_flat": round(t_flat / t_h, 3), "block_means_ms": round(t_bm, 4),
            "iou_vs_flat": round(float(np.mean(iou)), 4) if iou else None,
            "bytes_per_call": nbytes, "achieved_gbs": round(nbytes / (t_h * 1e-3) / 1e9, 1)}


def misa_stage(W, P, d, stream, timed, reps, flat_idx, t_flat, residual=False):
    """Active index heads (g = Hidx / 4 of the heads per query, routed by the block
    representatives, b = 128) timed beside the flat fused score + select, with the overlap
    of the two selections; the representatives are prebuilt index state.  With `residual`,
    the shared linear term plus g = Hidx / 4 - 6 residual heads: the same Hidx / 4 scored
    heads per query (the shared query takes six)."""
    import numpy as np
    import torch

    import token_selector_gather_amd as sa

    blk = 128
    g = W["Hidx"] // 4 - (6 if residual else 0)
    ws_bytes = sa.sa_resmisa_workspace_bytes if residual else sa.sa_misa_workspace_bytes
    nb = W["n_kv"] // blk
    if nb < 1 or g < 1 or ws_bytes(P, blk, g) == 0:
        return None
    kbar = torch.empty((W["B"], nb, W["d_idx"]), dtype=torch.bfloat16, device="cuda")
    sa.sa_block_means(P, d["k_idx"], blk, kbar, stream)
    ws_m = (sa.resmisa_workspace if residual else sa.misa_workspace)(P, blk, g)
    idx_m = torch.empty((W["B"], W["n_q"], W["k"]), dtype=torch.int32, device="cuda")
    call = sa.sa_resmisa_select if residual else sa.sa_misa_select
    t_m = timed(lambda: call(P, d["q_idx"], d["k_idx"], d["w"], kbar, blk, g, idx_m, ws_m, stream=stream), reps)
    st = sa.sa_device_status(ws_m)
    if st != sa.SA_OK:
        raise RuntimeError("active-head selection: device status " + sa.sa_status_str(st))
    a = idx_m.reshape(-1, W["k"]).cpu().numpy()
    f = flat_idx.reshape(-1, W["k"]).cpu().numpy()
    L = visible_counts(W).reshape(-1)
    rng = np.random.default_rng(0)
    rows = rng.choice(np.where(L > 0)[0], size=min(2048, int((L > 0).sum())), replace=False)
    iou = [np.intersect1d(a[r][a[r] >= 0], f[r][f[r] >= 0]).size /
           max(1, np.union1d(a[r][a[r] >= 0], f[r][f[r] >= 0]).size) for r in rows]
    pairs = int(L.sum())
    hs = W["Hidx"] // 4  # scored heads per query
    flops = 2 * W["d_idx"] * hs * pairs + 2 * W["d_idx"] * W["Hidx"] * int((L // blk).sum())
    return {"blk": blk, "g": g, "scored_heads": hs, "select_ms": round(t_m, 4), "flat_score_select_ms": round(t_flat, 4),
            "speedup_vs_flat": round(t_flat / t_m, 3), "iou_vs_flat": round(float(np.mean(iou)), 4),
            "iou_rows": int(len(rows)), "flops_per_call": flops, "tflops": round(flops / (t_m * 1e-3) / 1e12, 2)}


def paged_stage(W, P, d, stream, timed, cold, reps, idx, t_attn, t_attn_cold, O_ref, lse_ref):
    """The sparse attention over paged K/V (pages of 64 rows at seeded random places in one
    pool, block-table translation in the gather) timed beside the contiguous call on the same
    candidates, warm and with cold caches; the two outputs must agree bit for bit."""
    import numpy as np
    import torch

    import sa_synth
    import token_selector_gather_amd as sa
    from tests.device_inputs import device_pool, empty_outputs

    ps = 64
    bt, pool_rows = sa_synth.paged_layout(W["seed"] + 7, W["B"], W["n_kv"], ps, 3)
    Kp = device_pool(d["K"], bt, ps, pool_rows)
    Vp = Kp[..., : W["d_v"]] if W.get("V") is None else device_pool(d["V"], bt, ps, pool_rows)
    btd = torch.from_numpy(bt).cuda()
    O, lse, _ = empty_outputs(W, O_ref.dtype)
    ws = sa.workspace(P, sa.SA_OP_SPARSE_ATTN_PAGED)

    def call():
        sa.sa_sparse_attn_paged(P, d["Q"], Kp, Vp, btd, ps, idx, O, lse, ws, stream)

    try:
        call()
    except sa.SaError as e:  # layouts the paged kernels do not take (f32, grouped heads)
        if e.status != sa.SA_ERR_UNSUPPORTED:
            raise
        return None
    t = timed(call, reps)
    tc = cold(call)
    same = bool(torch.equal(O, O_ref) and torch.equal(lse, lse_ref))
    del Kp, Vp
    return {"page_size": ps, "pool_pages": pool_rows // ps, "sparse_attn_paged_ms": round(t, 4),
            "sparse_attn_ms": round(t_attn, 4), "paged_over_contiguous": round(t / t_attn, 4),
            "sparse_attn_paged_ms_cold": round(tc, 4), "sparse_attn_ms_cold": round(t_attn_cold, 4),
            "bit_identical_to_contiguous": same}


def grouped_stage(W, P, d, stream, timed, reps, G, t_step):
    """Grouped candidate sets (G groups of query heads, each selecting with its own Hidx / G
    index heads) timed as one call, beside the shared fused step; the overlap (IoU) of the
    first two groups' sets says how far the groups' selections differ."""
    import numpy as np
    import torch

    import token_selector_gather_amd as sa
    from tests.device_inputs import empty_outputs

    if sa.sa_grouped_workspace_bytes(P, G) == 0:
        return None
    O, lse, _ = empty_outputs(W, torch.bfloat16 if W["main_dtype"] != 0 else torch.float32)
    idx = torch.empty((G, W["B"], W["n_q"], W["k"]), dtype=torch.int32, device="cuda")
    ws = sa.grouped_workspace(P, G)
    t = timed(lambda: sa.sa_select_attend_grouped(P, G, d["q_idx"], d["k_idx"], d["w"], d["Q"], d["K"], d["V"], idx,
                                                   O, lse, ws, stream), reps)
    st = sa.sa_device_status(ws)
    if st != sa.SA_OK:
        raise RuntimeError("grouped selection: device status " + sa.sa_status_str(st))
    a = idx[0].reshape(-1, W["k"])[:4096].cpu().numpy()
    b = idx[1].reshape(-1, W["k"])[:4096].cpu().numpy()
    iou = [np.intersect1d(x[x >= 0], y[y >= 0]).size / max(1, np.union1d(x[x >= 0], y[y >= 0]).size)
           for x, y in zip(a, b) if (x >= 0).any()]
    return {"groups": G, "step_ms": round(t, 4), "shared_step_ms": round(t_step, 4),
            "over_shared": round(t / t_step, 3), "iou_group0_group1": round(float(np.mean(iou)), 4) if iou else None}


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stratified_rows(W, n_first=64, n_last=64, n_rand=384, seed=0):
    """The first n_first and last n_last valid query rows of the flattened batch plus n_rand
    other valid rows drawn at random (seed 0): the stratified sample of the oracle's CPU runs."""
    import numpy as np

    L = visible_counts(W).reshape(-1)
    valid = np.where(L > 0)[0]
    if valid.size <= n_first + n_last + n_rand:
        return valid.astype(np.int32), "all %d valid query rows" % valid.size
    ends = np.concatenate([valid[:n_first], valid[-n_last:]])
    rest = np.setdiff1d(valid, ends)
    rng = np.random.default_rng(seed)
    pick = rng.choice(rest, size=n_rand, replace=False)
    rows = np.sort(np.concatenate([ends, pick])).astype(np.int32)
    return rows, ("first %d, last %d and %d random (seed %d) of %d valid query rows"
                  % (n_first, n_last, n_rand, seed, valid.size))


def cpu_baseline(W, rows, what):
    """The oracle (unchanged) on the given query rows: fp64 score, select and attend."""
    from oracle import oracle as orc

    threads = orc.threads()
    t0 = time.perf_counter()
    orc.select_attend(W, rows)
    dt = time.perf_counter() - t0
    return {"value": rows.size / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": "%s; fp64 score + select + attend on %d threads, %.1f s" % (what, threads, dt),
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def measure(W, args, stream, full):
    """Times one workload: the fused step, each stage (warm and cold), single-step spread;
    with `full`, also the optional selectors and layouts beside it."""
    import numpy as np
    import torch

    import token_selector_gather_amd as sa
    from token_selector_gather_amd.inputs import device_workload
    from tests.device_inputs import empty_outputs

    alg = algorithmic(W)
    P, d = device_workload(W)
    dt = torch.float32 if W["main_dtype"] == 0 else torch.bfloat16
    O, lse, idx = empty_outputs(W, dt)
    ws = sa.workspace(P, sa.SA_OP_SELECT_ATTEND)

    def step():
        sa.sa_select_attend(P, d["q_idx"], d["k_idx"], d["w"], d["Q"], d["K"], d["V"], idx, O, lse, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st = sa.sa_device_status(ws)
    if st != sa.SA_OK:
        raise RuntimeError("device status " + sa.sa_status_str(st))
    ms_step = 1e3 * elapsed / args.steps

    # per-stage timing with HIP events recorded on the stream the library launches on
    def timed(fn, reps):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(reps):
            fn()
        ev1.record(stream)
        ev1.synchronize()
        return ev0.elapsed_time(ev1) / reps

    reps = max(3, args.steps)
    scores = torch.empty((W["B"], W["n_q"], W["n_kv"]), dtype=torch.float32, device="cuda")
    ws_t = sa.workspace(P, sa.SA_OP_TOPK)
    ws_s = sa.workspace(P, sa.SA_OP_SELECT)
    ws_a = sa.workspace(P, sa.SA_OP_SPARSE_ATTN)
    idx2, idx3 = idx.clone(), idx.clone()
    O2, lse2 = O.clone(), lse.clone()
    stage_fns = {
        "indexer_score": lambda: sa.sa_indexer_score(P, d["q_idx"], d["k_idx"], d["w"], scores, stream),
        "topk": lambda: sa.sa_topk(P, scores, W["n_kv"], idx2, None, ws_t, stream),
        "select": lambda: sa.sa_select(P, d["q_idx"], d["k_idx"], d["w"], idx3, ws_s, stream),
        "sparse_attn": lambda: sa.sa_sparse_attn(P, d["Q"], d["K"], d["V"], idx, O2, lse2, ws_a, stream),
    }
    times = {k: timed(f, reps) for k, f in stage_fns.items()}

    # distribution of single-step times (HIP events around each step, after the timed region)
    nrep = max(20, args.steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nrep)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([e0.elapsed_time(e1) for e0, e1 in evs])

    # cold caches: a 512 MiB write between calls evicts L2 and the MALL, so HBM-bound stages
    # are measured without reuse from an earlier call
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def cold(fn, reps=5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for r in range(reps):
            flush.fill_(r & 1)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    cold_times = {k: cold(f) for k, f in stage_fns.items()}
    if sa.sa_device_status(ws_s) != sa.SA_OK:
        raise RuntimeError("select: device status")
    roofs = stage_rooflines(W, alg, times)
    out = {
        "workload": W["name"],
        "value": round(alg["rows"] / (elapsed / args.steps), 2),
        "ms_per_step": round(ms_step, 4),
        "dtype": "bf16" if dt == torch.bfloat16 else "f32",
        "config": {"workload": W["name"], "B": W["B"], "n_q": W["n_q"], "n_kv": W["n_kv"], "Hq": W["Hq"],
                   "Hkv": W["Hkv"], "d_qk": W["d_qk"], "d_v": W["d_v"], "Hidx": W["Hidx"], "d_idx": W["d_idx"],
                   "k": W["k"], "causal": W["causal"], "valid_rows": alg["rows"]},
        "stages_ms": {k: round(v, 4) for k, v in times.items()},
        "step_ms_dist": {"p10": round(float(np.percentile(step_ms, 10)), 4), "p50": round(float(np.median(step_ms)), 4),
                         "p90": round(float(np.percentile(step_ms, 90)), 4), "reps": nrep},
        "stages_ms_cold": {k: round(v, 4) for k, v in cold_times.items()},
        "indexer": {"tflops": round(alg["idx_flops"] / (times["indexer_score"] * 1e-3) / 1e12, 3),
                    "frac_bf16_peak": round(alg["idx_flops"] / (times["indexer_score"] * 1e-3) / 1e12 /
                                            BF16_PEAK_TFLOPS, 5),
                    "flops_per_call": alg["idx_flops"]},
        "stage_rooflines": roofs,
        "stage_rooflines_cold": stage_rooflines(W, alg, cold_times),
        "_times": times,
        "_alg": alg,
    }
    if args.hisa == 1 or (args.hisa == -1 and alg["decode"]):
        out["hisa"] = hisa_stage(W, P, d, stream, timed, reps, idx, times["indexer_score"] + times["topk"])
    if full:
        if args.misa == 1 or (args.misa == -1 and not alg["decode"] and W["Hidx"] == 64):
            out["misa"] = misa_stage(W, P, d, stream, timed, reps, idx, times["select"])
            out["resmisa"] = misa_stage(W, P, d, stream, timed, reps, idx, times["select"], residual=True)
        if args.groups > 1:
            out["grouped"] = grouped_stage(W, P, d, stream, timed, reps, args.groups, float(np.median(step_ms)))
        if args.paged == 1:
            out["paged"] = paged_stage(W, P, d, stream, timed, cold, reps, idx, times["sparse_attn"],
                                       cold_times["sparse_attn"], O2, lse2)
    del P, d, O, lse, idx, ws, scores, ws_t, ws_s, ws_a, idx2, idx3, O2, lse2, flush
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2,
                    help="headline workload id (2 = latent prefill n=32768, the largest single-GPU workload)")
    ap.add_argument("--others", type=str, default="0,1,3,4",
                    help="other workload ids timed under 'workloads' (empty = none)")
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="rows in the oracle's stratified CPU-baseline sample (first 64, last 64, the rest random; "
                         "0 = skip)")
    ap.add_argument("--hisa", type=int, default=-1,
                    help="time the hierarchical selection beside the flat one (default: decode workloads only)")
    ap.add_argument("--misa", type=int, default=-1,
                    help="time the active-head selection beside the flat one (default: prefill workloads with 64 index heads)")
    ap.add_argument("--paged", type=int, default=1,
                    help="time the sparse attention over paged K/V beside the contiguous call")
    ap.add_argument("--groups", type=int, default=2,
                    help="time grouped candidate sets with this many groups beside the shared step (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (HBM counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (--gpus 1); multi-GPU runs are not supported",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sa_synth

    os.environ.setdefault("OMP_NUM_THREADS", "16")
    stream = torch.cuda.current_stream()
    print("bench: workload %d" % args.config, file=sys.stderr, flush=True)
    W = sa_synth.make_config(args.config)
    head = measure(W, args, stream, full=True)
    times, alg = head.pop("_times"), head.pop("_alg")
    roofs = head["stage_rooflines"]
    step_stages = {k: v for k, v in times.items() if k in ("select", "sparse_attn")}
    dominant = max(step_stages, key=step_stages.get)
    roof = dict(roofs[dominant])
    roof["traffic"] = counted_traffic(W["name"], dominant)
    out = {
        "metric": METRIC,
        "value": head.pop("value"),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.pop("dtype"),
        "data": "synthetic (seeded generator, seed = workload id)",
        "config": head.pop("config"),
        "roofline": roof,
    }
    head.pop("workload")
    out.update(head)
    others = {}
    for cid in [int(c) for c in args.others.split(",") if c.strip()]:
        if cid == args.config:
            continue
        print("bench: workload %d" % cid, file=sys.stderr, flush=True)
        Wo = sa_synth.make_config(cid)
        r = measure(Wo, args, stream, full=False)
        r.pop("_times"), r.pop("_alg")
        r["queries_per_s"] = r.pop("value")
        others[r.pop("workload")] = r
        del Wo
    if others:
        out["workloads"] = others
    if args.cpu_rows > 0:
        print("bench: oracle on the host", file=sys.stderr, flush=True)
        n_rand = max(0, args.cpu_rows - 128)
        rows, what = stratified_rows(W, 64, 64, n_rand)
        out["cpu_baseline"] = cpu_baseline(W, rows, what)
        # single-core rates of the two small workloads (all of c0, a stratified 256-row
        # sample of c1), as context for the per-core cost of the oracle
        one = {}
        saved = os.environ.get("OMP_NUM_THREADS")
        os.environ["OMP_NUM_THREADS"] = "1"
        try:
            for cid, n_rand in ((0, 1 << 30), (1, 128)):
                Wc = sa_synth.make_config(cid)
                rows_c, what_c = stratified_rows(Wc, 64, 64, n_rand)
                r = cpu_baseline(Wc, rows_c, what_c)
                one[Wc["name"]] = {"value": r["value"], "unit": r["unit"], "cores": r["cores"], "sample": r["sample"]}
                del Wc
        finally:
            if saved is None:
                os.environ.pop("OMP_NUM_THREADS", None)
            else:
                os.environ["OMP_NUM_THREADS"] = saved
        out["cpu_baseline"]["one_core"] = one
    print(json.dumps(out))


if __name__ == "__main__":
    main()

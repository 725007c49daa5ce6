"""Throughput of the DSA hot path (lightning indexer + causal top-k + sparse MQA attention) on one MI355X.

python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1] [--no-cpu-baseline] [--cpu-seconds S]

One step = the three libdsa calls over one batch of the workload, inputs resident in HBM. Prints one JSON line:
query tokens/s over K steps timed back to back, the dominant kernel's roofline fraction (algorithmic bytes or
flops over its launch duration, from HIP events between the stages on the kernels' stream during K further
steps), and the CPU oracle timed on a bounded row sample of the same workload.

Profiling helpers (same file, so every profile is made by committed code):
  python bench.py --copy-calibration        a plain device copy of known size, for scaling the HBM counters
  python bench.py --profile-commands DIR    the rocprofv3 passes behind the profiles/ summaries (output under DIR)
  python bench.py --ingest-profiles DIR     turn the rocprofv3 output under DIR into summaries in profiles/
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s (datasheet)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s (datasheet)
DEFAULT_WORKLOAD = "prefill_64k"
COPY_MIB = 2048                # size of the calibration / measured-peak copy
CSRC = os.path.join(ROOT, "dsa_lightning_indexer_02_amd", "csrc")
# kernel source behind each stage (its hash marks which build a set of counters belongs to)
STAGE_SOURCES = {"indexer": ["indexer.hip", "common.h"], "topk": ["topk.hip", "common.h"],
                 "attention": ["sparse_attn.hip", "common.h"]}
# kernel names (substrings) of each stage in rocprofv3 output
STAGE_KERNELS = {"indexer": ["indexer_"], "topk": ["topk_"], "attention": ["sparse_attn_kernel", "attn_combine"]}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true", help="skip the cache-append and IndexCache measurements")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="time budget of the oracle sample")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="per-kernel HBM bytes from rocprofv3 counters (JSON), if present")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--ingest-profiles", metavar="DIR")
    ap.add_argument("--profile-commands", metavar="DIR",
                    help="print the rocprofv3 commands of the workload's profile passes (output under DIR), one a line")
    return ap.parse_args()


def source_hash(stage: str) -> str:
    h = hashlib.sha256()
    for f in STAGE_SOURCES[stage]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic(wl, q_pos: np.ndarray):
    """Algorithmic work of one step per stage (DSA's own work: causal candidates, selected rows)."""
    n_q, k = wl.n_q, wl.k
    cand = q_pos.astype(np.int64) + 1
    sel = np.minimum(cand, k)
    key_bytes = wl.d_I * (1 if wl.k_dtype == "fp8" else 2) + (4 if wl.k_dtype == "fp8" else 0)
    # indexer: flops per causal pair; bytes = q_idx + w + each sequence's keys once + the scores written
    idx_flops = float(cand.sum()) * wl.H_I * wl.d_I * 2
    seq_keys = np.zeros(wl.num_seqs, dtype=np.int64)
    for b, p in zip(wl.q_seq.numpy(), q_pos):
        seq_keys[b] = max(seq_keys[b], p + 1)
    idx_bytes = n_q * (wl.H_I * wl.d_I * 2 + wl.H_I * 4) + float(seq_keys.sum()) * key_bytes + float(cand.sum()) * 4
    # top-k: every candidate score of rows that must select, plus the index rows written
    topk_bytes = float(cand[cand > k].sum()) * 4 + n_q * k * 4
    # attention: one latent row per selected entry, plus q, out, idx and lse per row
    attn_bytes = float(sel.sum()) * wl.D_qk * 2 + n_q * (wl.H * wl.D_qk * 2 + wl.H * wl.D_v * 2 + k * 4 + wl.H * 4)
    attn_flops = float(sel.sum()) * wl.H * (wl.D_qk + wl.D_v) * 2
    return dict(indexer=(idx_flops, idx_bytes), topk=(0.0, topk_bytes), attention=(attn_flops, attn_bytes))


def _cpu_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    return model, blas, usable


def _spread_order(n: int) -> list:
    """Row order whose every prefix is spread evenly over 0..n-1 (bit-reversed stride order)."""
    bits = max(1, (n - 1).bit_length())
    order = [int(format(i, f"0{bits}b")[::-1], 2) for i in range(1 << bits)]
    return [r for r in order if r < n]


def cpu_baseline(wl, seconds: float):
    """The oracle, as it stands, on a bounded row sample of the same workload (query tokens/s over the sample).

    Batches of more than 4096 rows (the 64K prefill) use a fixed stratified sample of 512 rows: 256 evenly spaced
    and 256 seeded-random (workloads.stratified_rows, the rows its sampled parity test checks), all of them, and
    report the measured time per row and the whole-batch time extrapolated from it. Smaller batches take rows in
    an order whose every prefix spreads evenly over the batch until the time budget is spent. All three steps run
    for each row (indexer row, its top-k, attention over that top-k)."""
    import oracle
    from workloads import bits_u16, bits_u8, stratified_rows

    model, blas, usable = _cpu_info()
    fp8 = wl.k_dtype == "fp8"
    kw = dict(q_seq=wl.q_seq.numpy(), seq_stride=wl.seq_stride,
              page_table=None if wl.page_table is None else wl.page_table.numpy(), page_size=wl.page_size)
    qidx, kidx = bits_u16(wl.q_idx), (bits_u8(wl.k_idx) if fp8 else bits_u16(wl.k_idx))
    q, lat = bits_u16(wl.q), bits_u16(wl.latent)
    fixed = wl.n_q > 4096
    order = [int(r) for r in stratified_rows(wl.n_q)] if fixed else _spread_order(wl.n_q)
    done, dt, chunk = 0, 0.0, 8
    while done < len(order) and (fixed or dt < seconds):
        rows = sorted(order[done: done + chunk])
        t0 = time.perf_counter()
        sc = oracle.indexer_scores_rows(rows, q_idx=qidx, w=wl.w.numpy(), k_idx=kidx,
                                        k_scale=wl.k_scale.numpy() if fp8 else None, q_pos=wl.q_pos.numpy(), **kw)
        idx = {r: oracle.topk_select(v.astype(np.float32), wl.k) for r, v in sc.items()}
        oracle.sparse_attn_rows(rows, q=q, latent=lat, idx=idx, sm_scale=wl.sm_scale, D_v=wl.D_v, **kw)
        dt += time.perf_counter() - t0
        done += len(rows)
    how = ("fixed stratified sample: 256 evenly spaced + 256 seeded-random rows" if fixed
           else "rows spread evenly over the batch, until the time budget was spent")
    rec = {"value": done / dt, "unit": "query tokens/s", "cores": int(blas), "kind": "oracle",
           "sample": f"{done} of {wl.n_q} query rows ({how}), all three steps, {dt:.1f} s; "
                     f"numpy fp64, {blas} BLAS threads of {usable} usable cores, {model}",
           "per_row_ms": round(1e3 * dt / done, 3)}
    if done < wl.n_q:
        rec["extrapolated_full_batch_s"] = round(dt / done * wl.n_q, 1)   # an estimate, not a measurement
    return rec


def copy_calibration(reps: int = 5):
    """A plain device-to-device copy of COPY_MIB MiB: reads and writes exactly that many bytes per launch."""
    import torch

    n = COPY_MIB << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"bytes_read": n, "bytes_written": n, "ms": ms, "copy_GBs": 2 * n / (ms * 1e-3) / 1e9}


def main():
    args = parse()
    if args.ingest_profiles:
        ingest_profiles(args.ingest_profiles, args.workload)
        return
    if args.profile_commands:
        for c in profile_commands(args.workload).values():
            print(c.replace("DIR", os.path.abspath(args.profile_commands)).replace("$R", ROOT))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no multi-GPU path; "
              "the DSA path would shard by query rows and sequences.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        print(json.dumps({"copy_calibration": copy_calibration()}), flush=True)
        return

    import torch

    import dsa_lightning_indexer_02_amd as dsa
    from workloads import make

    dsa.lib()  # fail loudly if the HIP library is not built
    wl_host = make(args.workload)
    wl = wl_host.to("cuda")
    b = dsa.Batch.from_workload(wl)
    ld = (wl.max_kv_len + 3) // 4 * 4
    scores = torch.zeros((wl.n_q, ld), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.n_q, wl.k), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.n_q, wl.H, wl.D_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((wl.n_q, wl.H), dtype=torch.float32, device="cuda")
    tk_ws_n = dsa.topk_workspace_size(b, wl.k)
    at_ws_n = dsa.sparse_attn_workspace_size(b, wl.k, wl.H, wl.D_v)
    tk_ws = torch.empty(max(tk_ws_n, 16), dtype=torch.uint8, device="cuda") if tk_ws_n else None
    at_ws = torch.empty(max(at_ws_n, 16), dtype=torch.uint8, device="cuda") if at_ws_n else None

    stages = (("indexer", lambda: dsa.indexer_scores(b, wl.q_idx, wl.w, wl.k_idx, wl.k_scale, scores)),
              ("topk", lambda: dsa.topk(b, scores, wl.k, idx, tk_ws)),
              ("attention", lambda: dsa.sparse_attn(b, wl.q, wl.latent, idx, wl.sm_scale, wl.D_v, out, lse, at_ws)))

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()
    # timed region: K steps back to back, events only around the whole region
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        for _, fn in stages:
            fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # then K more steps with events between the stages (same stream): each stage's launch durations, kept out of
    # the timed region above (an event between two short kernels adds its own gap)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        for j, (_, fn) in enumerate(stages):
            fn()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = {name: float(np.median([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, (name, _) in enumerate(stages)}

    cal = copy_calibration()        # measured HBM peak on this machine (plain copy), beside the datasheet figure
    work = algorithmic(wl_host, wl_host.q_pos.numpy())
    prefill = wl_host.n_q / wl_host.num_seqs >= 8
    st = {}
    for name, t in stage_ms.items():
        flops, nbytes = work[name]
        gbs = nbytes / (t * 1e-3) / 1e9
        tfl = flops / (t * 1e-3) / 1e12
        if name == "indexer" and prefill:
            st[name] = dict(ms=t, bound="mfma", achieved=tfl, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                            frac=tfl / BF16_PEAK_TFLOPS, algorithmic=flops)
        else:
            st[name] = dict(ms=t, bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=gbs / HBM_PEAK_GBS,
                            frac_of_measured_copy=gbs / cal["copy_GBs"], algorithmic=nbytes)
        if name == "attention":
            st[name]["mfma_frac"] = tfl / BF16_PEAK_TFLOPS
    dom = max(stage_ms, key=stage_ms.get)
    traffic = None
    try:
        with open(args.traffic) as f:
            tr = json.load(f).get(args.workload, {}).get(dom)
        if tr is not None and tr.get("source_sha") == source_hash(dom):
            traffic = tr.get("bytes_per_launch")
            st[dom]["traffic_fetch_bytes"] = tr.get("fetch_bytes")
            st[dom]["traffic_write_bytes"] = tr.get("write_bytes")
    except (OSError, ValueError):
        traffic = None
    d = st[dom]
    roofline = {"bound": d["bound"], "achieved": round(d["achieved"], 3), "peak": d["peak"], "unit": d["unit"],
                "frac": round(d["frac"], 4), "traffic": traffic, "kernel": dom,
                "launch_ms": round(stage_ms[dom], 4), "algorithmic": work[dom][1] if d["bound"] == "hbm" else work[dom][0]}
    if traffic:
        # the rate of the bytes that really crossed the L2/MALL boundary (rocprofv3 FETCH_SIZE + WRITE_SIZE), beside
        # the algorithmic rate above: the two differ by the cache reuse of the gathered rows
        roofline["measured_traffic_GBs"] = round(traffic / (stage_ms[dom] * 1e-3) / 1e9, 1)
        roofline["measured_traffic_frac"] = round(traffic / (stage_ms[dom] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    if dom == "attention":
        roofline["mfma_frac"] = round(st[dom]["mfma_frac"], 4)

    nxt = None if args.no_next_rows else next_rows(args, dsa, torch, wl, b, scores, idx, out, lse, tk_ws, at_ws,
                                                   stage_ms, stream)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl_host, args.cpu_seconds)

    value = wl.n_q / (ms * 1e-3)
    rec = {
        "metric": "query tokens/s (indexer+top-k+sparse attn) at k=2048; % of HBM/MFMA peak",
        "value": round(value, 1),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, shaped like the workload; no trained weights)",
        "config": {"workload": args.workload, "n_q": wl.n_q, "max_kv_len": wl.max_kv_len, "k": wl.k,
                   "H_I": wl.H_I, "d_I": wl.d_I, "H": wl.H, "D_qk": wl.D_qk, "D_v": wl.D_v,
                   "k_dtype": wl.k_dtype, "paged": wl.page_table is not None},
        "roofline": roofline,
        "stages": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                   for k, v in st.items()},
        "measured_copy_GBs": round(cal["copy_GBs"], 1),
        "next_rows": nxt,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def _median_ms(torch, stream, fn, reps: int) -> float:
    ts = []
    for _ in range(reps):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        z.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(z))
    return float(np.median(ts))


def next_rows(args, dsa, torch, wl, b, scores, idx, out, lse, tk_ws, at_ws, stage_ms, stream) -> dict:
    """Measurements of the steps around the three-call path, after the timed region (not part of `value`).

    cache_append: the batch's tokens written into FP8-key / latent caches of the workload's size (the step that
    precedes a decode step), algorithmic bytes = what each token reads and writes, against the HBM peak.
    indexcache_4_layers: one indexer + top-k shared by the attention of 4 layers (each layer its own latent
    cache), amortised per layer, beside the per-layer path of the main measurement.
    fused_indexer_topk: the indexer and the top-k in one call (scores never written), against the two calls.
    block_vs_token_64: block selection with the same token budget (32 blocks of 64) and attention over it,
    against the token path; how many of the token top-k positions the blocks contain; and what reading whole
    blocks of the token selection would cost (tokens read per useful token).
    """
    res = {}
    reps = max(3, min(args.steps, 20))
    slots = int(wl.latent.shape[0])
    g = torch.Generator(device="cuda").manual_seed(17)
    k_new = torch.randn((wl.n_q, wl.d_I), device="cuda", generator=g)
    lat_new = (torch.randn((wl.n_q, wl.D_qk), device="cuda", generator=g) / 24).to(torch.bfloat16)
    k_pool = torch.empty((slots, wl.d_I), dtype=torch.uint8, device="cuda")
    k_sc = torch.empty(slots, dtype=torch.float32, device="cuda")
    l_pool = torch.empty((slots, wl.D_qk), dtype=torch.bfloat16, device="cuda")
    fn = lambda: dsa.cache_append(b, k_new, lat_new, k_pool, k_sc, l_pool)  # noqa: E731
    fn()
    t = _median_ms(torch, stream, fn, reps)
    per_tok = wl.d_I * 4 + wl.D_qk * 2 + wl.d_I + 4 + wl.D_qk * 2
    gbs = wl.n_q * per_tok / (t * 1e-3) / 1e9
    res["cache_append"] = {"tokens": wl.n_q, "ms": round(t, 5), "bytes_per_token": per_tok, "achieved_GBs": round(gbs, 2),
                           "frac": round(gbs / HBM_PEAK_GBS, 4)}
    del k_new, lat_new, k_pool, k_sc, l_pool

    layers = 4
    lats = [wl.latent] + [wl.latent.clone() for _ in range(layers - 1)]

    def group():
        dsa.indexer_scores(b, wl.q_idx, wl.w, wl.k_idx, wl.k_scale, scores)
        dsa.topk(b, scores, wl.k, idx, tk_ws)
        for lat in lats:
            dsa.sparse_attn(b, wl.q, lat, idx, wl.sm_scale, wl.D_v, out, lse, at_ws)

    group()
    t = _median_ms(torch, stream, group, max(3, min(args.steps, 10)))
    per_layer = sum(stage_ms.values())
    res["indexcache_4_layers"] = {"ms_per_group": round(t, 4), "ms_per_layer": round(t / layers, 4),
                                  "layer_tokens_per_s": round(layers * wl.n_q / (t * 1e-3), 1),
                                  "speedup_vs_indexer_per_layer": round(per_layer * layers / t, 3)}
    del lats

    # fused indexer -> top-k (scores stay on chip), against the two calls of the main measurement
    try:
        fws = torch.empty(max(dsa.indexer_topk_workspace_size(b, wl.H_I, wl.d_I, wl.k), 16), dtype=torch.uint8,
                          device="cuda")
        fidx = torch.empty_like(idx)
        ffn = lambda: dsa.indexer_topk(b, wl.q_idx, wl.w, wl.k_idx, wl.k_scale, wl.k, fidx, fws)  # noqa: E731
        ffn()
        t = _median_ms(torch, stream, ffn, max(3, min(args.steps, 10)))
        res["fused_indexer_topk"] = {"ms": round(t, 5), "unfused_ms": round(stage_ms["indexer"] + stage_ms["topk"], 5),
                                     "speedup": round((stage_ms["indexer"] + stage_ms["topk"]) / t, 3)}
        del fws, fidx
    except dsa.DSAError as e:   # shapes the fused kernel is not built for
        res["fused_indexer_topk"] = {"unsupported": str(e)}

    # block-versus-token comparator: the same 2048-token budget spent on 32 whole 64-token blocks
    block = 64
    kb = max(1, wl.k // block)
    bidx = torch.empty((wl.n_q, kb * block), dtype=torch.int32, device="cuda")
    bws_n = dsa.block_topk_workspace_size(b, block, kb)
    bws = torch.empty(max(bws_n, 256), dtype=torch.uint8, device="cuda")
    dsa.indexer_scores(b, wl.q_idx, wl.w, wl.k_idx, wl.k_scale, scores)
    dsa.topk(b, scores, wl.k, idx, tk_ws)

    def block_path():
        dsa.block_topk(b, scores, block, kb, bidx, bws)
        dsa.sparse_attn(b, wl.q, wl.latent, bidx, wl.sm_scale, wl.D_v, out, lse, at_ws)

    block_path()
    reps2 = max(3, min(args.steps, 10))
    t_sel = _median_ms(torch, stream, lambda: dsa.block_topk(b, scores, block, kb, bidx, bws), reps2)
    t_blk = _median_ms(torch, stream, block_path, reps2)
    cnt = dsa.block_cover(b, idx, block).cpu().numpy().astype(np.float64)
    tok, blk = idx.cpu().numpy(), bidx.cpu().numpy()
    rows = np.unique(np.linspace(0, wl.n_q - 1, num=min(wl.n_q, 512)).astype(int))
    rec = [np.isin(tok[r][tok[r] >= 0], blk[r]).mean() for r in rows]
    res["block_vs_token_64"] = {
        "block_select_ms": round(t_sel, 5), "block_path_ms": round(t_blk, 5),
        "token_path_ms": round(stage_ms["topk"] + stage_ms["attention"], 5),
        "token_topk_recall_of_blocks": round(float(np.mean(rec)), 4),
        "token_selection_read_as_blocks": {"useful": round(float(cnt[:, 0].mean()), 1),
                                           "blocks": round(float(cnt[:, 1].mean()), 1),
                                           "tokens_read": round(float(cnt[:, 2].mean()), 1),
                                           "extra_work_x": round(float(cnt[:, 2].sum() / max(cnt[:, 0].sum(), 1)), 2)}}
    return res


# ---------------------------------------------------------------------------------------------------------------
# rocprofv3 output -> profiles/ summaries (run on any machine; reads CSV files only)

# Counter passes (rocprofv3 collects at most 8 SQ_ and 2 GRBM_ counters in one pass; each pass is its own run).
# MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCC * 4 SIMDs * 256 CUs), the expression of
# rocprofv3's own MfmaUtil metric, which the third pass collects for comparison together with LDSBankConflict.
COUNTER_PASSES = {
    "sq_issue": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD",
                 "SQ_INSTS_SALU", "SQ_WAVES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "GRBM_COUNT"],
    "sq_lds": ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
               "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
               "GRBM_GUI_ACTIVE"],
    "derived": ["MfmaUtil", "LDSBankConflict"],
}
N_XCC, N_CU, N_SIMD = 8, 256, 1024


def profile_commands(workload: str) -> dict:
    """The rocprofv3 commands whose output --ingest-profiles reads, run from the repository root on the MI355X machine
    (after `cd /tmp && export TMPDIR=/tmp`, with R the repository root; each pass is its own process)."""
    b = f"python3 $R/bench.py --workload {workload} --steps 5 --warmup 2 --no-cpu-baseline --no-next-rows"
    c = "python3 $R/bench.py --copy-calibration"
    cmds = {
        "ktrace": f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR/ktrace -o run -- {b}",
        "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch -o run -- {b}",
        "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/write -o run -- {b}",
        "cal_fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/cal_fetch -o run -- {c}",
        "cal_write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/cal_write -o run -- {c}",
    }
    for name, ctrs in COUNTER_PASSES.items():
        cmds[name] = f"rocprofv3 --pmc {' '.join(ctrs)} --output-format csv -d DIR/{name} -o run -- {b}"
    return cmds


def _read_csv(pattern):
    files = sorted(glob.glob(pattern, recursive=True))
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _stage_of(kernel_name: str):
    for stage, subs in STAGE_KERNELS.items():
        if any(s in kernel_name for s in subs):
            return stage
    return None


def _counter_per_dispatch(rows, counter):
    """{kernel name: mean counter value per dispatch} for one counter."""
    acc = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        acc.setdefault(r["Kernel_Name"], {})
        d = acc[r["Kernel_Name"]]
        d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {k: float(np.mean(list(v.values()))) for k, v in acc.items()}


def ingest_profiles(d: str, workload: str):
    cmds = profile_commands(workload)
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    lines_cmd = "\n".join(f"    {v.replace('DIR', d.rstrip('/'))}" for v in cmds.values())

    # kernel trace: per-kernel average duration
    stats = _read_csv(os.path.join(d, "ktrace", "**", "*kernel_stats.csv"))
    per_stage = {}
    for r in stats:
        s = _stage_of(r["Name"])
        if s is not None:
            per_stage.setdefault(s, []).append(r)
    for stage, rows in per_stage.items():
        txt = [f"# {stage} kernels, workload {workload}: rocprofv3 kernel-trace statistics", "",
               "Command (from the repository root, R = its path; `cd /tmp && export TMPDIR=/tmp` first):", "",
               f"    {cmds['ktrace'].replace('DIR', d.rstrip('/'))}", "",
               f"Kernel source hash (sha256 of {', '.join(STAGE_SOURCES[stage])}, first 16 hex): {source_hash(stage)}",
               "", "| kernel | calls | average µs | min µs | max µs | share of GPU time |", "|---|---|---|---|---|---|"]
        for r in rows:
            name = r["Name"].split("(")[0][:80]
            txt.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} "
                       f"| {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} % |")
        with open(os.path.join(out_dir, f"{stage}_{workload}_kernel_trace.md"), "w") as f:
            f.write("\n".join(txt) + "\n")

    # HBM counters, scaled by what the same counters read for a copy of known size
    fetch = _counter_per_dispatch(_read_csv(os.path.join(d, "fetch", "**", "*counter_collection.csv")), "FETCH_SIZE")
    write = _counter_per_dispatch(_read_csv(os.path.join(d, "write", "**", "*counter_collection.csv")), "WRITE_SIZE")
    cf = _counter_per_dispatch(_read_csv(os.path.join(d, "cal_fetch", "**", "*counter_collection.csv")), "FETCH_SIZE")
    cw = _counter_per_dispatch(_read_csv(os.path.join(d, "cal_write", "**", "*counter_collection.csv")), "WRITE_SIZE")
    if not (fetch and write and cf and cw):
        print("no FETCH_SIZE / WRITE_SIZE files found; no traffic summary", file=sys.stderr)
        ingest_counters(d, workload, cmds, stats)
        return
    copy_bytes = COPY_MIB << 20
    # the copy kernel is the one whose counters are largest in the calibration runs
    f_scale = copy_bytes / (max(cf.values()) * 1024.0)
    w_scale = copy_bytes / (max(cw.values()) * 1024.0)
    path = os.path.join(out_dir, "traffic.json")
    try:
        with open(path) as f:
            traffic = json.load(f)
    except (OSError, ValueError):
        traffic = {}
    txt = [f"# HBM traffic per launch, workload {workload}: rocprofv3 FETCH_SIZE and WRITE_SIZE", "",
           "Commands (from the repository root, R = its path; `cd /tmp && export TMPDIR=/tmp` first; one pass each):",
           "", lines_cmd, "",
           f"Calibration: a device copy of {COPY_MIB} MiB reads FETCH_SIZE {max(cf.values()):.0f} KiB and WRITE_SIZE "
           f"{max(cw.values()):.0f} KiB per dispatch, so the counters are scaled by {f_scale:.4f} (fetch) and "
           f"{w_scale:.4f} (write) to bytes.", "",
           "| stage | kernel | FETCH bytes / launch | WRITE bytes / launch | source hash |", "|---|---|---|---|---|"]
    traffic.setdefault(workload, {})
    for stage in STAGE_KERNELS:
        fb = sum(v for k, v in fetch.items() if _stage_of(k) == stage) * 1024.0 * f_scale
        wb = sum(v for k, v in write.items() if _stage_of(k) == stage) * 1024.0 * w_scale
        names = sorted({k.split("(")[0][:60] for k in fetch if _stage_of(k) == stage})
        if not names:
            continue
        traffic[workload][stage] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
                                    "source_sha": source_hash(stage)}
        txt.append(f"| {stage} | {', '.join('`' + n + '`' for n in names)} | {fb:.4g} | {wb:.4g} | {source_hash(stage)} |")
    with open(path, "w") as f:
        json.dump(traffic, f, indent=1, sort_keys=True)
    with open(os.path.join(out_dir, f"hbm_traffic_{workload}.md"), "w") as f:
        f.write("\n".join(txt) + "\n")
    print(f"wrote {path} and summaries in {out_dir}")
    ingest_counters(d, workload, cmds, stats)


def _per_dispatch(rows):
    """{kernel: {counter: mean per dispatch}} and {kernel: mean duration ns under counter collection}."""
    acc, dur = {}, {}
    for r in rows:
        k = r["Kernel_Name"]
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], {})
        d = acc[k][r["Counter_Name"]]
        d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        dur.setdefault(k, {})[r["Dispatch_Id"]] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return ({k: {c: float(np.mean(list(v.values()))) for c, v in cs.items()} for k, cs in acc.items()},
            {k: float(np.mean(list(v.values()))) for k, v in dur.items()})


def ingest_counters(d: str, workload: str, cmds: dict, stats):
    """profiles/counters_<workload>.md: per-kernel SQ counters of the indexer, top-k and attention kernels."""
    per, dur = {}, {}
    for name in COUNTER_PASSES:
        rows = _read_csv(os.path.join(d, name, "**", "*counter_collection.csv"))
        p, t = _per_dispatch(rows)
        for k, cs in p.items():
            per.setdefault(k, {}).update(cs)
        for k, v in t.items():
            dur.setdefault(k, []).append(v)
    if not per:
        print("no SQ counter files found", file=sys.stderr)
        return
    trace_ns = {r["Name"]: float(r["AverageNs"]) for r in stats}
    txt = [f"# SQ counters per launch, workload {workload}: MFMA utilisation, instruction mix, LDS bank conflicts", "",
           "Commands (from the repository root, R = its path; `cd /tmp && export TMPDIR=/tmp` first; one pass each):", ""]
    txt += [f"    {cmds[n].replace('DIR', d.rstrip('/'))}" for n in COUNTER_PASSES]
    txt += ["", "Derived here, per launch (counter values are summed over the chip by rocprofv3):",
            f"- clock = GRBM_GUI_ACTIVE / {N_XCC} XCDs / the kernel-trace average duration (meaningful for launches of "
            "a millisecond or more: for short ones GRBM_GUI_ACTIVE also counts the dispatch around the kernel, so the "
            "figure, and the MFMA busy share derived from the same count, are off);",
            f"- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {N_XCC} x {N_SIMD} SIMDs), rocprofv3's MfmaUtil "
            "expression (its own MfmaUtil value is listed beside it);",
            "- MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512;",
            "- LDS bank-conflict cycles per LDS-active cycle = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE;",
            "- instructions per wave = SQ_INSTS_* / SQ_WAVES.", ""]
    hdr = ("| kernel | trace µs | clock GHz | MFMA busy (MfmaUtil) | MFMA TFLOP/s | MFMA / VALU / LDS / VMEM-rd / SALU "
           "instr per wave | LDS conflict cycles / LDS-active cycles (LDSBankConflict) | wait-any / active-any |")
    txt += [hdr, "|---|---|---|---|---|---|---|---|"]
    for k in sorted(per, key=lambda x: -trace_ns.get(x, 0.0)):
        stage = _stage_of(k)
        if stage is None:
            continue
        c = per[k]
        t_ns = trace_ns.get(k) or float(np.mean(dur.get(k, [0.0])))
        gui = c.get("GRBM_GUI_ACTIVE", 0.0) / N_XCC
        clk = gui / t_ns if t_ns else 0.0
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * N_SIMD) if gui else 0.0
        flops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        waves = max(c.get("SQ_WAVES", 1.0), 1.0)
        mix = " / ".join(f"{c.get(x, 0.0) / waves:.0f}" for x in
                         ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU"))
        lds = c.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(c.get("SQ_LDS_IDX_ACTIVE", 0.0), 1.0)
        wait = c.get("SQ_WAIT_INST_ANY", 0.0) / max(c.get("SQ_ACTIVE_INST_ANY", 0.0), 1.0)
        txt.append(f"| `{k.split('(')[0][:70]}` | {t_ns / 1e3:.2f} | {clk:.2f} | {100 * busy:.1f} % "
                   f"({c.get('MfmaUtil', float('nan')):.1f} %) | {flops / (t_ns * 1e-9) / 1e12 if t_ns else 0:.0f} "
                   f"| {mix} | {lds:.4f} ({c.get('LDSBankConflict', float('nan')):.2f} %) | {wait:.2f} |")
    txt += ["", "Raw counter means per launch:", "", "| kernel | counter | value |", "|---|---|---|"]
    for k in sorted(per):
        if _stage_of(k) is None:
            continue
        for cn, v in sorted(per[k].items()):
            txt.append(f"| `{k.split('(')[0][:50]}` | {cn} | {v:.6g} |")
    with open(os.path.join(ROOT, "profiles", f"counters_{workload}.md"), "w") as f:
        f.write("\n".join(txt) + "\n")
    print(f"wrote profiles/counters_{workload}.md")


if __name__ == "__main__":
    main()

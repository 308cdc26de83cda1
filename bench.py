"""Benchmark of the CSA2 hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  encoder64k / tiny : Full scoring -> Top-512 -> sparse attention;
  decoder256k / decode1m : Full scoring (+ 8-position block maxima) -> Top-512
      and Top-2048 blocks -> attention; 3 x (Reindex over the 16384-entry pool
      -> Top-512 -> attention); 1 Reuse attention;
  prefill128k : Full scoring of 4096 queries with causal visibility -> Top-512
      -> attention with per-query windows;
  encoder_group64k : the 64K shapes as a layer group sharing one cache: Full
      -> Top-512 -> 6 attention layers (the Full layer's and 5 Reuse layers');
  decoder_group256k : the 256K shapes as a decoder group: Reindex over a pool
      built once beforehand (untimed) -> Top-512 -> 4 attention layers (the
      Reindex layer's and 3 Reuse layers');
  encoder64k_fp4k / decode1m_fp4k : the 64K and 1M steps reading the indexer
      K as FP4 entries (68 B) packed from the same kind of bf16 keys before
      timing;
  encoder64k_fp4k_fp8w / decode1m_fp4k_fp8w : the same with the window KV
      as FP8 rows (528 B) as well: both of the pages' cache precisions;
  prefill128k_fp4k : the prefill step over FP4 indexer-K entries;
  prefill128k_fp4qk : the same with the indexer Q in MXFP4 too (the step
      packs the bf16 query into one entry per head, then scores on the
      scaled FP4 matrix instruction);
  encoder64k_fp4qk_fp8w / decode1m_fp4qk_fp8w : the 64K and 1M steps with
      MXFP4 indexer Q and K and FP8 window KV (each scoring layer's query
      packed inside the step).
In every decode step (one query per sequence) the Full layer's scoring and
Top-512 run fused (csa2_index_topk: scoring with a per-chunk Top-512 in one
launch, the chunks' merge in a second; no score row is written); the prefill
chunk scores and selects in one launch (csa2_index_prefill_topk: a workgroup
scores 8 queries' whole rows and keeps their Top-512). The prefill extra also
times csa2_index_full alone (the same scoring with the 1 GiB score row
written, no selection).
The headline is decode queries/s on encoder64k (64 queries, 64K-token context
at m=2 = 32768 FP4 entries per sequence). Inputs live in HBM before timing and
four independent input sets rotate between decode steps (together well above
1 GiB), so the 256 MB last-level cache cannot hold the data a step reads. Per-call times come from HIP events on
the stream the kernels run on.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workloads a,b,...]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
FP4_PEAK_TFLOPS = 10100.0   # MI355X dense fp4 MFMA
METRIC = "CSA2 decode queries/s + HBM GB/s at 64K/1M ctx; prefill indexer TFLOP/s"
HEADLINE = "encoder64k"


def query_bytes(wl):
    """One query's indexer Q: 32 x 128 bf16, or 32 MXFP4 entries of 68 B."""
    return 32 * 68 if wl.qfmt == "fp4" else 32 * 128 * 2


def alg_bytes_index_full(wl):
    """K_idx rows read once per query (256 B bf16 or 68 B FP4 entries; prefill:
    once per sequence), scores written (4 B per entry per query), queries and
    weights read."""
    n_vis = wl.N * wl.nq if wl.n_visible is None else int(wl.n_visible.sum().item())
    row = 68 if wl.kfmt == "fp4" else 256
    kbytes = (wl.N * row * wl.nseq) if wl.q_per_seq > 1 else n_vis * row
    out = wl.nq * wl.N * 4 + (wl.nq * ((wl.N + 7) // 8) * 4 if wl.hier else 0)
    return kbytes + out + wl.nq * (query_bytes(wl) + 32 * 4)


def fused_chunks(nq, N):
    """Chunks per query of csa2_index_topk: 8192 entries, or 4096 when 8192
    would leave fewer than 512 workgroups (the rule in the fused kernel's
    launcher)."""
    c = 4096 if nq * ((N + 8191) // 8192) < 512 else 8192
    return (N + c - 1) // c


def alg_bytes_index_topk(wl, k=512):
    """Fused scoring + per-chunk Top-k (the select launch): K_idx rows read
    once per query (prefill: once per sequence), queries and weights read,
    each chunk's k candidates written (4 B key + 4 B id; the final ids when a
    row is one chunk), block maxima written for the hierarchical pool."""
    n_vis = wl.N * wl.nq if wl.n_visible is None else int(wl.n_visible.sum().item())
    row = 68 if wl.kfmt == "fp4" else 256
    if wl.q_per_seq > 1:  # prefill: one chunk per row at the benchmark's shapes
        return wl.N * row * wl.nseq + wl.nq * k * 4 + wl.nq * (query_bytes(wl) + 32 * 4)
    c = fused_chunks(wl.nq, wl.N)
    out = wl.nq * k * (8 * c if c > 1 else 4) + (wl.nq * ((wl.N + 7) // 8) * 4 if wl.hier else 0)
    return n_vis * row + out + wl.nq * (query_bytes(wl) + 32 * 4)


def alg_flops_index_full(wl):
    n_vis = wl.N * wl.nq if wl.n_visible is None else int(wl.n_visible.sum().item())
    return 2 * 32 * 128 * n_vis


def alg_bytes_attn(nq, k=512, window=128, window_row=1024):
    """Per query-layer: k FP4 records (288 B), the window rows (1 KiB bf16 or
    528 B FP8 each), the query (64 KiB), the output (64 KiB) and k indices."""
    return nq * (k * 288 + window * window_row + 64 * 1024 + 64 * 1024 + k * 4)


def alg_bytes_step_unfused(wl, k=512, pool_blocks=2048):
    """Algorithmic bytes of one decode step counted as the unfused calls move
    them (the accounting the step targets are stated in): Full scoring with its
    score row (and block maxima) written, both read back by the Top-K, each
    Reindex layer's pool keys read and its pool scores and ids written, and
    every attention layer."""
    blk = ((wl.N + 7) // 8) * 4 if wl.hier else 0
    index = alg_bytes_index_full(wl)
    topk = wl.nq * (wl.N * 4 + blk)
    n_re = wl.n_index_layers - 1
    pool = pool_blocks * 8
    reindex = n_re * wl.nq * pool * (256 + 4 + 4)
    return index + topk + reindex + wl.n_attn_layers * alg_bytes_attn(wl.nq)


def alg_flops_attn(nq, k=512, window=128):
    return nq * 2 * 2 * 64 * (k + window) * 512


class Timer:
    """Records HIP events around named calls on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.rec = []

    def span(self, name):
        t = self

        class _S:
            def __enter__(s):
                s.a = t.torch.cuda.Event(enable_timing=True)
                s.b = t.torch.cuda.Event(enable_timing=True)
                s.a.record()

            def __exit__(s, *exc):
                s.b.record()
                t.rec.append((name, s.a, s.b))
        return _S()

    def summary(self):
        """{name: (mean ms, count, median ms)} over the recorded calls."""
        out = {}
        for name, a, b in self.rec:
            out.setdefault(name, []).append(a.elapsed_time(b))
        return {k: (sum(v) / len(v), len(v), sorted(v)[len(v) // 2]) for k, v in out.items()}


def run_step(step, k_idx, kv, timer=None):
    """One pass of the hot path, with optional per-call event spans."""
    step.run(k_idx, kv, timer.span if timer else None)


def bench_workload(name, steps, warmup, nsets, torch):
    from kv_cache_compression_csa2_amd.pipeline import Step, pack_workload_kv, workload_kidx
    from kv_cache_compression_csa2_amd.workloads import CONFIGS, make_workload
    dev = "cuda"
    sets = []
    for s in range(nsets):
        wl = make_workload(name, device=dev, seed=CONFIGS[name]["seed"] + 100 * s)
        kv = pack_workload_kv(wl, dev)
        kk = workload_kidx(wl)
        if kk is not wl.k_idx:
            wl.k_idx = None  # the step reads the FP4 entries only
        st = Step(wl, dev)
        st.prepare(kk)
        sets.append((st, wl, kv, kk))
    torch.cuda.synchronize()
    for i in range(warmup):
        st, wl, kv, kk = sets[i % nsets]
        run_step(st, kk, kv)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        st, wl, kv, kk = sets[i % nsets]
        run_step(st, kk, kv)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # second timed pass with per-call events (same work, separate from the wall clock)
    timer = Timer(torch)
    for i in range(steps):
        st, wl, kv, kk = sets[i % nsets]
        run_step(st, kk, kv, timer)
    torch.cuda.synchronize()
    calls = timer.summary()
    wl = sets[0][1]
    ms_step = wall * 1e3 / steps
    res = {"workload": name, "nq": wl.nq, "N": wl.N, "ms_per_step": ms_step,
           "queries_per_s": wl.nq / (ms_step * 1e-3),
           # per-call medians (a host-side stall can inflate a single span)
           "calls_ms": {k: round(v[2], 5) for k, v in calls.items()},
           "_calls_mean_ms": {k: v[0] for k, v in calls.items()}}
    if "index_full" in calls:
        t_idx = calls["index_full"][2] * 1e-3
        res["index_full_GBps"] = alg_bytes_index_full(wl) / t_idx / 1e9
        res["index_full_TFLOPs"] = alg_flops_index_full(wl) / t_idx / 1e12
    if "index_topk" in calls:
        t_idx = calls["index_topk"][0] * 1e-3
        res["index_topk_GBps"] = alg_bytes_index_topk(wl) / t_idx / 1e9
        res["index_topk_TFLOPs"] = alg_flops_index_full(wl) / t_idx / 1e12
        res["_alg_bytes_index_topk"] = alg_bytes_index_topk(wl)
    t_att = calls["attn"][2] * 1e-3
    res["attn_GBps"] = alg_bytes_attn(wl.nq, window_row=528 if wl.swa_fmt == "fp8" else 1024) / t_att / 1e9
    res["attn_TFLOPs"] = alg_flops_attn(wl.nq) / t_att / 1e12
    res["_alg_bytes_index_full"] = alg_bytes_index_full(wl)
    res["_alg_bytes_step"] = alg_bytes_step_unfused(wl)
    res["_alg_flops_index_full"] = alg_flops_index_full(wl)
    if wl.q_per_seq > 1:
        # the same scoring alone, score row written (csa2_index_full), outside the step
        from kv_cache_compression_csa2_amd import _lib as L
        st, wl0, kv, kk = sets[0]
        kb, kf = st._k(kk)
        t = Timer(torch)
        for i in range(warmup + steps):
            with t.span("index_full" if i >= warmup else "warm"):
                if st.qf is not None:  # the MXFP4 query the step packed
                    L.csa2_index_full(None, wl0.w[0], kb, wl0.N, wl0.q_per_seq, wl0.n_visible, 0, st.scores,
                                      k_fp4=kf, q_fp4=st.qf)
                else:
                    L.csa2_index_full(wl0.q_idx[0], wl0.w[0], kb, wl0.N, wl0.q_per_seq, wl0.n_visible, 0, st.scores,
                                      k_fp4=kf)
        torch.cuda.synchronize()
        t_sc = t.summary()["index_full"][2] * 1e-3
        res["scoring_only_ms"] = t_sc * 1e3
        res["scoring_only_TFLOPs"] = alg_flops_index_full(wl) / t_sc / 1e12
        res["_mfma_dtype"] = "fp4" if wl.qfmt == "fp4" else "bf16"
    del sets
    torch.cuda.empty_cache()
    return res


def bench_attn_gather(nq, torch, steps=20, warmup=3, nsets=4):
    """The FP4 main-KV gather path alone: nq decode queries (one sequence each,
    4096 entries), 512 random distinct entries + 128 window rows each;
    `nsets` independent KV caches and index sets rotate between calls."""
    from kv_cache_compression_csa2_amd import _lib as L
    from kv_cache_compression_csa2_amd.workloads import bf16_normal, generator, random_records
    dev = "cuda"
    N = 4096
    sets = []
    for s in range(nsets):
        g = generator(dev, 77 + s, 1)
        kv = random_records(nq * N, g, dev).view(nq, N, 288)
        idx = torch.sort(torch.rand((nq, N), generator=generator(dev, 77 + s, 2), device=dev).argsort(1)[:, :512],
                         1)[0].to(torch.int32).contiguous()
        q = bf16_normal((nq, 64, 512), generator(dev, 77 + s, 3), dev)
        swa = bf16_normal((nq, 128, 512), generator(dev, 77 + s, 4), dev)
        st = torch.zeros((nq,), dtype=torch.int32, device=dev)
        sl = torch.full((nq,), 128, dtype=torch.int32, device=dev)
        out = torch.empty((nq, 64, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((nq, 64), dtype=torch.float32, device=dev)
        ws = torch.empty((max(L.csa2_sparse_attn_workspace_bytes(nq, 512), 1),), dtype=torch.uint8, device=dev)
        sets.append((q, kv, idx, swa, st, sl, out, lse, ws))
    torch.cuda.synchronize()

    def call(i):
        q, kv, idx, swa, st, sl, out, lse, ws = sets[i % nsets]
        L.csa2_sparse_attn(q, kv, N, 1, idx, swa, st, sl, out=out, lse=lse, workspace=ws)

    for i in range(warmup):
        call(i)
    timer = Timer(torch)
    for i in range(steps):
        with timer.span("attn"):
            call(i)
    torch.cuda.synchronize()
    t = timer.summary()["attn"][0] * 1e-3
    del sets
    torch.cuda.empty_cache()
    return {"nq": nq, "ms": t * 1e3, "GBps": alg_bytes_attn(nq) / t / 1e9, "TFLOPs": alg_flops_attn(nq) / t / 1e12}


def cpu_baseline(torch, target_s=15.0):
    """The CPU oracle, as it stands, on a bounded sample of the headline
    workload: the first n queries (scoring over all 32768 entries, Top-512,
    attention), n chosen from a 4-query trial so the run takes ~target_s."""
    import numpy as np
    from kv_cache_compression_csa2_amd.workloads import make_workload
    from oracle import oracle as O
    O.build(force=False)
    wl = make_workload(HEADLINE, device="cuda")

    def u16(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    qi_all, w_all, k_all = u16(wl.q_idx[0]), wl.w[0].cpu().numpy(), u16(wl.k_idx)
    kv_all = wl.kv.cpu().numpy()
    flat = wl.kv_prepack_rows.cpu().numpy()
    pre = u16(wl.kv_prepack)
    q_all, swa_all = u16(wl.q[0]), u16(wl.swa[0])
    st_all, sl_all = wl.swa_start.cpu().numpy(), wl.swa_len.cpu().numpy()

    def run(n):
        kv = kv_all[:n].copy()
        t0 = time.perf_counter()
        recs = O.fp4_pack(pre)  # the oracle packs the planted entries itself
        for j, fid in enumerate(flat):
            if fid // wl.N < n:
                kv[fid // wl.N, fid % wl.N] = recs[j]
        s = O.index_full(qi_all[:n], w_all[:n], k_all[:n], wl.N, 1)
        top = O.topk(s, 512)
        O.sparse_attn(q_all[:n], kv, wl.N, 1, top, swa_all[:n], wl.swa_T, st_all[:n], sl_all[:n],
                      1.0 / math.sqrt(512.0))
        return time.perf_counter() - t0

    t4 = run(4)
    n = int(min(wl.nq, max(4, round(4 * target_s / max(t4, 1e-3)))))
    reps, total, done = 0, 0.0, 0
    while total < target_s * 0.66 and reps < 64:
        total += run(n)
        done += n
        reps += 1
    return {"value": round(done / total, 3), "unit": "queries/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": "%d x %d of the 64 encoder64k queries (whole path: score 32768 entries, Top-512, attention), "
                      "%.1f s of CPU time" % (reps, n, total)}


# sources the scoring kernels (fused decode scoring + Top-K, prefill scoring) are compiled from
KERNEL_SOURCES = ["index.hip", "topk_select.h", "device_common.h"]
# sources of the sparse attention kernels
ATTN_SOURCES = ["attn.hip", "device_common.h"]


def kernel_source_hash(files=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "kv_cache_compression_csa2_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def profile_fields(name, files):
    """The machine-read 'key: value' lines of a committed rocprofv3 summary
    under profiles/, if it was taken on the current sources of its kernel
    (its kernel_source_sha256_16 line); else {}."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return {}
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "`", "rocprof")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    return fields if fields.get("kernel_source_sha256_16") == kernel_source_hash(files) else {}


def traffic_from_profiles():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE, calibrated on a 1 GiB copy), if it
    was taken on the current kernel sources; else None."""
    f = profile_fields("index_topk_encoder64k_traffic.md", KERNEL_SOURCES)
    return int(f["hbm_bytes_per_launch"]) if "hbm_bytes_per_launch" in f else None


def target_rooflines(res, sweep):
    """The three step targets, each against its roofline: the FP4 main-KV
    gather at 1024 query-layers (>= 60% of HBM), the prefill indexer (>= 50%
    of bf16 MFMA) and the 1M decode step (>= 60% of HBM, step bytes counted as
    the unfused calls move them). Counter figures come from the committed
    summaries while they match the current kernel sources (else null)."""
    t = {}
    if "1024" in sweep:
        g = sweep["1024"]
        f = profile_fields("sparse_attn_gather_traffic.md", ATTN_SOURCES)
        t["fp4_gather_1024_queries"] = {
            "bound": "hbm", "achieved": round(g["GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(g["GBps"] / HBM_PEAK_GBS, 4), "target_frac": 0.60,
            "alg_bytes_per_launch": alg_bytes_attn(1024),
            "traffic": int(f["hbm_bytes_per_launch_1024q"]) if "hbm_bytes_per_launch_1024q" in f else None}
    if "prefill128k" in res:
        p = res["prefill128k"]
        f = profile_fields("index_prefill_prefill128k_mfma.md", KERNEL_SOURCES)
        t["prefill_indexer"] = {
            "bound": "mfma", "achieved": round(p["scoring_only_TFLOPs"], 1), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(p["scoring_only_TFLOPs"] / BF16_PEAK_TFLOPS, 4), "target_frac": 0.50,
            "call": "csa2_index_full", "ms": round(p["scoring_only_ms"], 4),
            "mfma_busy": float(f["mfma_busy_scoring_only"]) if "mfma_busy_scoring_only" in f else None,
            "clock_ghz": float(f["clock_ghz_scoring_only"]) if "clock_ghz_scoring_only" in f else None}
    for pn, dt in [("prefill128k_fp4k", "bf16"), ("prefill128k_fp4qk", "fp4")]:
        # the same indexer figure at the pages' FP4 indexer-K precision (bf16
        # products), and with the indexer Q in MXFP4 too (fp4 products)
        if pn in res:
            p = res[pn]
            peak = FP4_PEAK_TFLOPS if dt == "fp4" else BF16_PEAK_TFLOPS
            t["prefill_indexer_" + pn.split("_", 1)[1]] = {
                "bound": "mfma", "achieved": round(p["scoring_only_TFLOPs"], 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(p["scoring_only_TFLOPs"] / peak, 4), "target_frac": 0.50, "mfma_dtype": dt,
                "call": "csa2_index_full" + ("_fp4qk" if dt == "fp4" else "_fp4k"),
                "ms": round(p["scoring_only_ms"], 4)}
            if dt == "fp4":
                f = profile_fields("index_prefill_prefill128k_mfma.md", KERNEL_SOURCES)
                e = t["prefill_indexer_" + pn.split("_", 1)[1]]
                e["mfma_busy"] = float(f["mfma_busy_fp4qk_scoring_only"]) if "mfma_busy_fp4qk_scoring_only" in f else None
                e["clock_ghz"] = float(f["clock_ghz_fp4qk_scoring_only"]) if "clock_ghz_fp4qk_scoring_only" in f else None
    if "decode1m" in res:
        d = res["decode1m"]
        gbs = d["_alg_bytes_step"] / (d["ms_per_step"] * 1e-3) / 1e9
        t["decode1m_step"] = {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "target_frac": 0.60, "alg_bytes_per_step": d["_alg_bytes_step"],
            "queries_per_s": round(d["queries_per_s"], 1)}
    return t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workloads",
                    default="encoder64k,decoder256k,decode1m,prefill128k,encoder_group64k,decoder_group256k,"
                            "encoder64k_fp4k,decode1m_fp4k,encoder64k_fp4k_fp8w,decode1m_fp4k_fp8w,"
                            "prefill128k_fp4k,prefill128k_fp4qk,encoder64k_fp4qk_fp8w,decode1m_fp4qk_fp8w")
    ap.add_argument("--attn-sweep", default="64,256,1024")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the benchmark runs on one GPU only; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import kv_cache_compression_csa2_amd as K
    K.load()
    if args.calibrate_copy:
        a = torch.empty((1 << 30,), dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": 1 << 30}))
        return
    names = [n for n in args.workloads.split(",") if n]
    if HEADLINE not in names:
        names.insert(0, HEADLINE)
    res = {}
    for n in names:
        print("bench: %s ..." % n, file=sys.stderr, flush=True)
        res[n] = bench_workload(n, args.steps, args.warmup, 1 if n.startswith("prefill") or n == "tiny" else 4, torch)
        print("bench: %s %.4f ms/step" % (n, res[n]["ms_per_step"]), file=sys.stderr, flush=True)
    sweep = {}
    for nq in [int(x) for x in args.attn_sweep.split(",") if x]:
        print("bench: attention gather nq=%d ..." % nq, file=sys.stderr, flush=True)
        sweep[str(nq)] = bench_attn_gather(nq, torch)
    h = res[HEADLINE]
    # dominant kernel: the fused Full-layer scoring + per-chunk Top-512
    # (index_topk_kernel, the select launch of csa2_index_topk; one launch per
    # "index_topk" span)
    t_idx_s = h["_calls_mean_ms"]["index_topk"] * 1e-3  # mean launch duration
    achieved = h["_alg_bytes_index_topk"] / t_idx_s / 1e9
    roofline = {"kernel": "index_topk_kernel (csa2_index_topk_select: Full scoring + per-chunk Top-512)",
                "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profiles(),
                "alg_bytes_per_launch": h["_alg_bytes_index_topk"]}
    cpu = None
    if not args.no_cpu:
        print("bench: cpu oracle baseline ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(torch)
    extra = {}
    for n, r in res.items():
        e = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items() if not k.startswith("_")}
        extra[n] = e
    for pn in [n for n in res if n.startswith("prefill")]:
        # the prefill indexer figure: the chunk's scoring flops over the time of
        # csa2_index_full (scoring alone, score row written); the step runs the
        # fused scoring + Top-512 call, reported beside it. The peak is that of
        # the matrix instruction's own operand type (bf16, or fp4 for MXFP4 Q x K).
        p = res[pn]
        e = extra[pn]
        dt = p["_mfma_dtype"]
        peak = FP4_PEAK_TFLOPS if dt == "fp4" else BF16_PEAK_TFLOPS
        tf = p["scoring_only_TFLOPs"]
        e["indexer_TFLOPs"] = round(tf, 2)
        e["indexer_mfma_dtype"] = dt
        e["indexer_frac_of_%s_peak" % dt] = round(tf / peak, 4)
        if "index_topk_TFLOPs" in p:
            e["fused_indexer_TFLOPs"] = round(p["index_topk_TFLOPs"], 2)
            e["fused_indexer_frac_of_%s_peak" % dt] = round(p["index_topk_TFLOPs"] / peak, 4)
    extra["attn_gather_sweep"] = {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in sweep.items()}
    extra["targets"] = target_rooflines(res, sweep)
    line = {
        "metric": METRIC, "value": round(h["queries_per_s"], 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(h["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16/fp16",
        "data": "synthetic (seeded; shapes and distributions of the pages' 64K encoder decode)",
        "config": {"workload": "encoder64k: 64 decode queries, 64K-token context at m=2 = 32768 FP4 entries "
                               "per sequence, Full mode, Top-512, 64x512 MQA + 128 SWA",
                   "global_batch": 64, "seq_len": 65536, "entries": 32768, "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

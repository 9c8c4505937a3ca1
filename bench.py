"""Decode-attention benchmark: one step = score_pages + select_pages + sparse_decode_attn for the
whole batch (every head, one query token per sequence, one layer), inputs resident in HBM.

Prints ONE JSON line (rank 0): steps/s, ms/step, achieved HBM GB/s on the step's algorithmic
bytes, a roofline record for the dominant kernel (timed live with HIP events on the stream it
runs on) and the float64 oracle timed on a bounded sample on the host cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload token128k] [--no-cpu]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_kv_cache_build_amd as skv  # noqa: E402
import workloads as W  # noqa: E402

METRIC = "decode attn steps/sec and achieved HBM GB/s (% of peak) at 128K ctx, 1 GPU"
PEAK_GBPS = 8000.0          # MI355X HBM3E
MALL_BYTES = 256 << 20      # Infinity Cache: rotate buffer sets so a round touches > 2x this


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Step:
    """Preallocated buffers of one decode step on one buffer set."""

    def __init__(self, w: W.Workload, alpha: float, split: int = 0, full: bool = False):
        cfg = w.cfg
        self.w, self.alpha, self.full = w, alpha, full
        self.kind = cfg["score"]
        self.cache = skv.PagedCache(w.k, w.v, w.block_table, w.seq_lens, w.Hq)
        self.events = None   # timing events for the dominant kernel (skv.event_pair())
        meta_kinds = ("gauss" if self.kind == "gauss_q" else self.kind,)
        self.meta = skv.build_page_meta(self.cache, meta_kinds, proj=w.proj, pool_block=cfg.get("pool_block", 0),
                                        lsh_planes=w.lsh_planes)
        # the build timed on its second run (the first also loads the kernels' code)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        skv._binding._check(skv.lib().skv_build_page_meta(self.cache.ref, self.meta.ref, skv._binding._stream(None)),
                            "skv_build_page_meta")
        e1.record()
        torch.cuda.synchronize()
        self.meta_s = e0.elapsed_time(e1) * 1e-3
        # token top-k: keep only the candidate set of the selection (fused scoring, no dense keys)
        self.fused = cfg["policy"] == "token_topk" and cfg["score"] == "proj" and not full
        self.scores = skv.ScoreBuffers(self.cache, self.kind, cfg.get("k", 0) if self.fused else 0)
        if full:   # full-cache comparator: every page, the same attention kernels
            p = skv.select_params("all", tokens=0)
        else:
            p = skv.select_params(cfg["policy"], k=cfg.get("k", 0), budget_pct=cfg.get("pct", 0),
                                  alpha=cfg.get("sel_alpha", 1.5), delta=cfg.get("delta", 0.0),
                                  tokens=1 if self.kind in ("proj", "lsh") else 0)
        self.sel = skv.Selection(self.cache, p)
        self.attn = skv.AttnBuffers(self.cache, skv.attn_params(self.cache, alpha, None, self.sel.granularity, split),
                                    self.sel.cap)

    def pre(self):
        """Work before the dominant kernel: the sampled bound of the fused token scoring, or the
        selection of every page for the full-cache comparator."""
        if self.full:
            skv.select_pages(self.cache, self.scores, None, out=self.sel)
        elif self.fused:
            skv.score_pages(self.cache, self.meta, self.w.q, self.kind, out=self.scores, phase=skv.TOKEN_PHASE_BOUND)

    def score(self):
        """The dominant kernel: the filtered token scoring, the page scorer, or (full-cache
        comparator) the attention over every page."""
        if self.full:
            skv.sparse_decode_attn(self.cache, self.w.q, self.sel, out=self.attn, events=self.events)
        else:
            skv.score_pages(self.cache, self.meta, self.w.q, self.kind, out=self.scores,
                            phase=skv.TOKEN_PHASE_FILTER if self.fused else skv.TOKEN_PHASE_ALL,
                            temperature=self.w.cfg.get("lsh_tau"), events=self.events)

    def rest(self):
        if not self.full:
            skv.select_pages(self.cache, self.scores, None, out=self.sel)
            skv.sparse_decode_attn(self.cache, self.w.q, self.sel, out=self.attn)

    def run(self):
        self.pre()
        self.score()
        self.rest()

    def capture(self):
        """Record the three stages as HIP graphs (no allocation happens inside run())."""
        self.g_pre, self.g_score, self.g_rest = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(self.g_pre):
            self.pre()
        with torch.cuda.graph(self.g_score):
            self.score()
        with torch.cuda.graph(self.g_rest):
            self.rest()
        torch.cuda.synchronize()


def step_bytes(st: Step):
    """Algorithmic bytes of one step: metadata read + K of the selected rows + V of the rows that
    carry weight + q + out. Returns (total, score_kernel_bytes, details)."""
    w = st.w
    e = 2 if w.dtype == torch.bfloat16 else 4
    d, S, G = w.d, w.S, w.G
    lens = np.array(w.lens)
    P = (lens + S - 1) // S
    cnt = st.sel.count.cpu().numpy().astype(np.int64)
    bt = int(P.sum()) * w.Hkv * 4        # block-table entries, read once per unit
    if st.full:
        meta, keys_out = 0, 0
    elif st.kind == "box":
        meta = int(P.sum()) * w.Hkv * 2 * d * e
        keys_out = w.B * w.Hkv * w.maxP * 4
    elif st.kind in ("gauss", "gauss_q"):
        meta = int(P.sum()) * w.Hkv * 2 * d * 4
        keys_out = 3 * w.B * w.Hq * w.maxP * 4
    elif st.kind == "pool":              # float32 means of the sub-blocks holding a token
        pb = w.cfg["pool_block"]
        n_sb = int(sum(-(-min(S, int(L) - p * S) // pb) for L in lens for p in range(-(-int(L) // S))))
        meta = n_sb * w.Hkv * d * 4
        keys_out = w.B * w.Hkv * w.maxP * 4
    elif st.kind == "lsh":               # bucket ids (one byte per table) and the value norm of every token
        meta = int(lens.sum()) * w.Hkv * (w.cfg["lsh_tables"] + 4)
        keys_out = w.B * w.Hkv * w.maxP * S * 4
    else:
        r = w.proj.shape[0]
        meta = int(lens.sum()) * w.Hkv * r * 2
        # fused: only the candidate pairs are written (about k per unit, 8 bytes each), not counted
        keys_out = 0 if st.fused else w.B * w.Hkv * w.maxP * S * 4
    if st.sel.granularity:
        k_rows = int(cnt.sum())
    else:
        idx = st.sel.idx.cpu().numpy()
        k_rows = 0
        for b in range(w.B):
            for g in range(w.Hkv):
                pg = idx[b, g, :cnt[b, g]].astype(np.int64)
                k_rows += int(np.minimum(S, lens[b] - pg * S).sum())
    kv_row = d * e
    # softmax weights every selected row; entmax reads V only for its (small) support, which is not
    # counted, so entmax figures are conservative
    v_rows = k_rows if st.alpha == 1.0 else 0
    q_out = w.B * w.Hq * d * (e + 4)
    total = meta + bt + k_rows * kv_row + v_rows * kv_row + q_out
    dom = (k_rows + v_rows) * kv_row + q_out if st.full else meta + keys_out + bt
    det = dict(meta=meta, block_table=bt, k=k_rows * kv_row, v=v_rows * kv_row, q_out=q_out)
    assert sum(det.values()) == total
    return total, dom, det, dict(selected_rows=k_rows, weighted_rows=v_rows, keys_written_bytes=keys_out)


def meta_read_bytes(w: W.Workload) -> int:
    """Bytes of the cache the metadata build reads: K of every valid token (and V for the soft-LSH
    value norms)."""
    e = 2 if w.dtype == torch.bfloat16 else 4
    n = int(np.array(w.lens).sum()) * w.Hkv * w.d * e
    return 2 * n if w.cfg["score"] == "lsh" else n


def dominant_kernel(st: Step) -> str:
    """The kernel the roofline record covers: the scoring kernel proper (after any query
    preparation), or the first attention kernel for the full-cache comparator."""
    if st.full:
        if st.alpha == 1.0:
            return "attn_softmax_kernel"
        return "attn_entmax_logits_mfma_kernel" if st.w.dtype == torch.bfloat16 else "attn_entmax_logits_kernel"
    if st.fused:
        return "score_proj_cand_kernel"
    return {"box": "score_box_kernel", "gauss": "score_gauss_kernel", "gauss_q": "score_gauss_kernel",
            "proj": "score_proj_kernel", "pool": "score_pool_kernel", "lsh": "score_lsh_kernel"}[st.kind]


def kernel_sources_sha256(sources) -> str:
    """One hash over the listed source files (repository-relative paths), in order."""
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    return h.hexdigest()


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the dominant kernel from the committed PMC record (profiles/), or None
    when there is no record or a source the kernel is built from changed since the counters were
    taken (the record lists the files and their joint hash)."""
    path = os.path.join(ROOT, "profiles", f"{workload}_score_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    srcs = rec.get("sources")
    if rec.get("kernel") != kernel or not srcs or not all(os.path.exists(os.path.join(ROOT, f)) for f in srcs):
        return None
    if kernel_sources_sha256(srcs) != rec.get("sources_sha256"):
        return None
    return int(rec["traffic_bytes"])


def cpu_baseline(name: str, alpha: float, max_threads: int = 16):
    """The float64 oracle (unchanged) on a bounded sample of the workload: units (sequence, KV head)
    of sequences drawn on the CPU with the workload's shapes at full context. Metadata is built
    first (prefill work, not timed). Timed: score + select + attention of each sampled unit, one
    unit per task on a pool of threads (the oracle releases the GIL), then scaled to whole steps;
    and one unit alone on one thread. The pool uses every core the process may run on, up to
    max_threads (the CPU share of one GPU's host)."""
    import oracle
    from oracle import pipeline

    host_cores = len(os.sched_getaffinity(0))
    threads = max(1, min(host_cores, max_threads))
    cfg = W.CONFIGS[name]
    n_seq = max(1, -(-threads // cfg["Hkv"]))          # enough sequences for one unit per thread
    w = W.make(name, device="cpu", B=n_seq)
    spec = pipeline.Spec(score="gauss" if w.cfg["score"] == "gauss_q" else w.cfg["score"], policy=w.cfg["policy"],
                         k=w.cfg.get("k", 0), pct=w.cfg.get("pct", 0),
                         sel_alpha=w.cfg.get("sel_alpha", 1.5), delta=w.cfg.get("delta", 0.0), alphas=(alpha,),
                         proj=w.proj.numpy() if w.proj is not None else None,
                         gauss_max="quantile" if w.cfg["score"] == "gauss_q" else "sqrt2log",
                         pool_block=w.cfg.get("pool_block", 4),
                         lsh_planes=w.lsh_planes.numpy() if w.lsh_planes is not None else None,
                         lsh_tau=w.cfg.get("lsh_tau", 1.0))
    caches = []
    G = w.G
    for b in range(n_seq):     # one unit per sub-cache (exact bytes of that sequence and KV head)
        h = W.host_arrays(w, [b])
        for g in range(w.Hkv):
            caches.append(oracle.Cache(q=np.ascontiguousarray(h["q"][:, g * G:(g + 1) * G]),
                                       k=np.ascontiguousarray(h["k"][:, g:g + 1]),
                                       v=np.ascontiguousarray(h["v"][:, g:g + 1]),
                                       block_table=h["block_table"], seq_lens=h["seq_lens"]))
    n_units = len(caches)
    with cf.ThreadPoolExecutor(threads) as ex:
        mds = list(ex.map(lambda c: pipeline.build_metadata(c, spec), caches))

    def one(i):
        c, md = caches[i], mds[i]
        sc = pipeline.compute_scores(c, spec, md)
        r = pipeline.run_unit(c, spec, sc, 0, 0)
        return len(r.sel)

    t0 = time.perf_counter()
    one(0)
    single = time.perf_counter() - t0
    reps, t = 0, 0.0
    with cf.ThreadPoolExecutor(threads) as ex:
        while t < 5.0 and reps < 50:
            t0 = time.perf_counter()
            list(ex.map(one, range(n_units)))
            t += time.perf_counter() - t0
            reps += 1
    per_round = t / reps
    units_total = sum(1 for _ in range(cfg["B"])) * cfg["Hkv"]
    steps_per_s = (n_units / units_total) / per_round
    return dict(value=steps_per_s, unit="steps/s", cores=threads, host_cores=host_cores, kind="oracle",
                single_thread_unit_s=round(single, 4),
                single_thread_steps_per_s=1.0 / (single * units_total),
                sample=f"{n_units} units ({n_seq} sequence(s) x {w.Hkv} KV heads, {G} query heads each) of {name} at "
                       f"full context ({w.lens[0]} tokens), metadata prebuilt; score+select+attention on {threads} "
                       f"threads over {reps} round(s), {per_round:.3f} s per round, scaled by {units_total} units "
                       f"per step; one unit alone on one thread took {single:.3f} s")


def w0_row_bytes(w: W.Workload) -> int:
    return w.d * (2 if w.dtype == torch.bfloat16 else 4)


def reference_ceilings(dev, n_rows: int, row_bytes: int, reps: int = 5):
    """Bandwidth ceilings on this GPU from the reference kernels of libskv_ref.so (context for the
    roofline fractions): a plain streaming read of 1 GiB; a gather of n_rows random rows of
    row_bytes, twice (K and V rows, as the attention reads them), from a 4 GiB table, each row read
    by a group of row_bytes / 16 lanes; and torch's 1 GiB copy (read + write). The reads are timed
    at several grid sizes, with plain and with non-temporal loads; the best of each is reported,
    with every configuration's figure."""
    import ctypes as C
    ref = C.CDLL(os.path.join(ROOT, "sparse_kv_cache_build_amd", "libskv_ref.so"))
    ref.skv_ref_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_int, C.c_void_p]
    ref.skv_ref_gather_rows.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_int, C.c_int,
                                        C.c_void_p]
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    grids = (512, 1024, 2048, 4096, 8192)
    sink = torch.empty(max(grids), dtype=torch.int32, device=dev)

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    def ok(rc):
        assert rc == 0, rc

    def sweep(nbytes, launch):
        res = {f"{'nt' if nt else 'plain'}_{bl}": round(nbytes / timed(lambda: ok(launch(bl, nt))) / 1e9, 1)
               for nt in (0, 1) for bl in grids}
        best = max(res, key=res.get)
        return res[best], best, res

    out = {}
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    best, how, res = sweep(1 << 30, lambda bl, nt: ref.skv_ref_stream_read(src.data_ptr(), (1 << 30) // 16,
                                                                            sink.data_ptr(), bl, nt, stream))
    out["stream_read_1GiB_GBps"] = best
    out["stream_read_best"] = how
    out["stream_read_sweep"] = res
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src))
    out["copy_1GiB_GBps"] = round(2 * (1 << 30) / t / 1e9, 1)
    del src, dst
    n_rows = max(1, int(n_rows))
    words = row_bytes // 16
    table = torch.ones(4 << 30, dtype=torch.uint8, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    rows_in_table = (4 << 30) // row_bytes
    off = (torch.randint(0, rows_in_table, (2 * n_rows,), generator=g, device=dev) * words).to(torch.int64)
    best, how, res = sweep(2 * n_rows * row_bytes, lambda bl, nt: ref.skv_ref_gather_rows(
        table.data_ptr(), off.data_ptr(), 2 * n_rows, words, sink.data_ptr(), bl, nt, stream))
    out["gather_rows"] = 2 * n_rows
    out["gather_row_bytes"] = row_bytes
    out["gather_GBps"] = best
    out["gather_best"] = how
    out["gather_sweep"] = res
    del table, off
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="token128k", choices=list(W.CONFIGS))
    ap.add_argument("--alpha", type=float, default=None)
    ap.add_argument("--split", type=int, default=0)
    ap.add_argument("--sets", type=int, default=0, help="buffer sets rotated per step (0: enough to exceed 2x MALL)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--graph", action="store_true", help="replay the stages as HIP graphs instead of launching them")
    ap.add_argument("--full", action="store_true",
                    help="full-cache comparator: attention over every page with the same kernels, no scoring")
    ap.add_argument("--calibrate", action="store_true",
                    help="after timing, copy a 1 GiB buffer 3 times (reference kernel for HBM byte counters)")
    ap.add_argument("--ceilings", action="store_true",
                    help="also time reference kernels: a 1 GiB copy, a 1 GiB read-only reduction and a gather of "
                         "the step's number of random 256-byte rows")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the decode path has no multi-GPU mode "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    name = args.workload
    cfg = W.CONFIGS[name]
    alpha = args.alpha if args.alpha is not None else cfg["alphas"][0]

    log(f"[bench] drawing {name} on {dev}")
    sets = [Step(W.make(name, device=dev), alpha, args.split, args.full)]
    sets[0].run()
    torch.cuda.synchronize()
    total, score_bytes, det, rows = step_bytes(sets[0])
    n_sets = args.sets or max(1, math.ceil(2 * MALL_BYTES / max(total, 1)))
    for i in range(1, n_sets):
        log(f"[bench] buffer set {i + 1}/{n_sets}")
        sets.append(Step(W.make(name, device=dev, seed=cfg["seed"] + 100 * i), alpha, args.split, args.full))
    meta_s = sets[0].meta_s
    graphs = args.graph
    if graphs:
        for st in sets:
            st.capture()
        pre_fn = [st.g_pre.replay for st in sets]
        score_fn = [st.g_score.replay for st in sets]
        rest_fn = [st.g_rest.replay for st in sets]
    else:
        pre_fn = [st.pre for st in sets]
        score_fn = [st.score for st in sets]
        rest_fn = [st.rest for st in sets]

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        pre_fn[i % n_sets]()
        score_fn[i % n_sets]()
        rest_fn[i % n_sets]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    if graphs:
        # graph replays: events on the stream around the scoring graph (which holds the query
        # preparation too, where the scorer has one)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        start.record(stream)
        for i in range(args.steps):
            pre_fn[i % n_sets]()
            ev[i][0].record(stream)
            score_fn[i % n_sets]()
            ev[i][1].record(stream)
            rest_fn[i % n_sets]()
        end.record(stream)
        torch.cuda.synchronize()
        score_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
        timed_by = "HIP events around the scoring graph's replay"
    else:
        # caller-owned event pairs, one per step, that the library records on the launch stream right
        # around the dominant kernel
        pairs = [skv.event_pair() for _ in range(args.steps)]
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            sets[i % n_sets].events = pairs[i]
            pre_fn[i % n_sets]()
            score_fn[i % n_sets]()
            rest_fn[i % n_sets]()
        end.record(stream)
        torch.cuda.synchronize()
        for st in sets:
            st.events = None
        score_ms = sum(a.elapsed_time(b) for a, b in pairs) / args.steps
        timed_by = "HIP events the library records around each launch of the kernel"
    ms = start.elapsed_time(end) / args.steps
    sps = 1000.0 / ms
    gbps = total / (ms * 1e-3) / 1e9
    score_gbps = score_bytes / (score_ms * 1e-3) / 1e9
    log(f"[bench] {ms * 1e3:.1f} us/step, score stage {score_ms * 1e3:.1f} us")

    # metadata upkeep per decode step, outside the step: one new token per sequence (its page's box or
    # moments recomputed, or its projected key written)
    st0 = sets[0]
    for _ in range(3):
        skv.append_page_meta(st0.cache, st0.meta, 1)
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(20):
        skv.append_page_meta(st0.cache, st0.meta, 1)
    a1.record(stream)
    torch.cuda.synchronize()
    append_us = a0.elapsed_time(a1) / 20 * 1e3

    if args.calibrate:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ceil = reference_ceilings(dev, rows["selected_rows"], w0_row_bytes(sets[0].w)) if args.ceilings else None

    cpu = None
    if not args.no_cpu and not args.full:   # the comparator is context: no oracle baseline
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(name, alpha)

    key_desc = {"box": "box bound", "pool": f"pooled key (sub-blocks of {cfg.get('pool_block')})",
                "gauss": "Gaussian estimated maximum", "gauss_q": "Gaussian quantile maximum"}.get(cfg["score"], cfg["score"])
    sel_desc = {"topk": f"top-{cfg.get('k')} pages by {key_desc}", "budget": f"{cfg.get('pct')}% page budget by {key_desc}",
                "thresh": f"Gaussian entmax threshold (alpha {cfg.get('sel_alpha')}, Delta {cfg.get('delta')})",
                "token_topk": (f"top-{cfg.get('k')} tokens per KV head, " + (
                    f"soft-LSH scores ({cfg.get('lsh_tables')} tables x {cfg.get('lsh_bits')} bits, "
                    f"temperature {cfg.get('lsh_tau')})" if cfg["score"] == "lsh"
                    else f"rank-{cfg.get('proj_rank')} projection"))}
    w0 = sets[0].w
    line = {
        "metric": METRIC,
        "value": round(sps, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w0.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": name, "batch": w0.B, "ctx": int(max(w0.lens)), "mean_ctx": float(np.mean(w0.lens)),
                   "q_heads": w0.Hq, "kv_heads": w0.Hkv, "head_dim": w0.d, "page": w0.S, "kv_dtype": "bf16"
                   if w0.dtype == torch.bfloat16 else "f32",
                   "select": "every page (full-cache comparator)" if args.full else sel_desc[cfg["policy"]],
                   "attn": "softmax" if alpha == 1.0 else f"{alpha}-entmax", "bytes_per_step": int(total),
                   "achieved_GBps": round(gbps, 1), "pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
                   "accumulation": ("fp32 (Gaussian page scores, attention)" if cfg["score"] in ("gauss", "gauss_q")
                                    else "fp32 (attention), fp64 (ranking keys)"),
                   "buffer_sets": n_sets, "hip_graphs": graphs, "meta_build_s": round(meta_s, 6),
                   "meta_build_GBps": round(meta_read_bytes(w0) / meta_s / 1e9, 1),
                   "meta_append_us": round(append_us, 2),
                   "bytes_detail": det, **rows},
        "roofline": {"bound": "hbm", "kernel": dominant_kernel(sets[0]), "achieved": round(score_gbps, 1),
                     "peak": PEAK_GBPS, "unit": "GB/s", "frac": round(score_gbps / PEAK_GBPS, 4),
                     "traffic": recorded_traffic(name, dominant_kernel(sets[0])),
                     "avg_us": round(score_ms * 1e3, 2), "bytes_per_launch": int(score_bytes),
                     "timed_by": timed_by},
        "cpu_baseline": cpu,
    }
    if ceil is not None:
        line["ceilings"] = ceil
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Runs one decode step of a workload through libskv (GPU) and the same step through the float64
oracle (CPU, raw inputs only) and compares them. Used by the GPU parity tests."""
from __future__ import annotations

import concurrent.futures as cf
import json
import math
import os
import sys
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
from oracle import pipeline
import sparse_kv_cache_build_amd as skv
import workloads as W

# Output tolerance (bf16 inputs, fp32 accumulation): |gpu - ref| <= ATOL + RTOL |ref|
RTOL, ATOL = 2e-3, 1e-3
# tau_hat: the GPU solves in float32 from float32 (m, s); decisions closer than this to the
# threshold may go either way (certified near-ties)
TAU_TOL = 1e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def record(entry: dict):
    """Appends one JSON line to the file named by the environment variable SKV_PARITY_RECORD, if
    set: the per-test parity summary (units compared, certified near-ties with their margins,
    largest error as a fraction of the tolerance)."""
    path = os.environ.get("SKV_PARITY_RECORD")
    if not path:
        return
    entry = dict(entry, test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0])
    with open(path, "a") as f:
        f.write(json.dumps(entry) + "\n")


def spec_of(w: W.Workload, alphas=None) -> pipeline.Spec:
    cfg = w.cfg
    score = "gauss" if cfg["score"] == "gauss_q" else cfg["score"]
    return pipeline.Spec(score=score, policy=cfg["policy"], k=cfg.get("k", 0), pct=cfg.get("pct", 0),
                         sel_alpha=cfg.get("sel_alpha", 1.5), delta=cfg.get("delta", 0.0),
                         alphas=tuple(alphas or cfg["alphas"]),
                         proj=w.proj.cpu().numpy() if w.proj is not None else None,
                         gauss_max="quantile" if cfg["score"] == "gauss_q" else "sqrt2log",
                         pool_block=cfg.get("pool_block", 4),
                         lsh_planes=w.lsh_planes.cpu().numpy() if w.lsh_planes is not None else None,
                         lsh_tau=cfg.get("lsh_tau", 1.0))


@dataclass
class GpuStep:
    cache: skv.PagedCache
    meta: skv.PageMeta
    scores: skv.ScoreBuffers
    sel: skv.Selection
    outs: dict = field(default_factory=dict)


def gpu_step(w: W.Workload, alphas=None, split=0, policy=None, cap=None, fused=False) -> GpuStep:
    """fused: projected token scores kept only as the candidate set of the top-k (no dense keys)."""
    cfg = w.cfg
    cache = skv.PagedCache(w.k, w.v, w.block_table, w.seq_lens, w.Hq)
    kind = cfg["score"]
    pol = policy or cfg["policy"]
    meta_kinds = ("gauss" if kind == "gauss_q" else kind,) + (("box",) if pol == "thresh_box" else ())
    meta = skv.build_page_meta(cache, meta_kinds, proj=w.proj, pool_block=cfg.get("pool_block", 0),
                               lsh_planes=w.lsh_planes)
    token_k = cfg.get("k", 0) if (fused and kind == "proj" and pol == "token_topk") else 0
    scores = skv.score_pages(cache, meta, w.q, kind, token_k=token_k, temperature=cfg.get("lsh_tau"))
    if pol == "thresh_box":   # the box key beside the Gaussian m, s in one skv_scores
        scores = skv.CombinedScores(skv.score_pages(cache, meta, w.q, "box"), scores)
    sel = skv.select_pages(cache, scores, pol, k=cfg.get("k", 0), budget_pct=cfg.get("pct", 0),
                           alpha=cfg.get("sel_alpha", 1.5), delta=cfg.get("delta", 0.0),
                           tokens=1 if kind in ("proj", "lsh") else 0, cap=cap)
    st = GpuStep(cache, meta, scores, sel)
    for a in (alphas or cfg["alphas"]):
        st.outs[a] = skv.sparse_decode_attn(cache, w.q, sel, alpha=a, split=split).clone()
    torch.cuda.synchronize()
    return st


def oracle_cache(h) -> oracle.Cache:
    return oracle.Cache(q=h["q"], k=h["k"], v=h["v"], block_table=h["block_table"], seq_lens=h["seq_lens"])


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


@dataclass
class Report:
    units: int = 0
    near_ties: int = 0
    max_err: float = 0.0
    notes: list = field(default_factory=list)
    ties: list = field(default_factory=list)        # certified near-ties: (seq, kv head, indices, margins)
    tie_units_checked: int = 0                      # near-tie units whose outputs were checked on the GPU's set

    def merge(self, o: "Report"):
        self.units += o.units
        self.near_ties += o.near_ties
        self.max_err = max(self.max_err, o.max_err)
        self.notes += o.notes
        self.ties += o.ties
        self.tie_units_checked += o.tie_units_checked

    def entry(self, w: W.Workload, seqs, **extra) -> dict:
        return dict(workload=w.name, B=w.B, Hq=w.Hq, Hkv=w.Hkv, d=w.d, S=w.S, max_len=w.max_len,
                    seqs=None if seqs is None else [int(x) for x in seqs], units=self.units,
                    near_ties=self.near_ties, tie_units_checked=self.tie_units_checked,
                    max_err_over_tol=round(self.max_err, 4), ties=self.ties[:50], **extra)


def compare(w: W.Workload, st: GpuStep, seqs=None, alphas=None, check_meta=True) -> Report:
    """Oracle on sequences `seqs` (all if None) from raw inputs; asserts parity. Returns a report."""
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    h = W.host_arrays(w, None if seqs == list(range(w.B)) else seqs)
    c = oracle_cache(h)
    spec = spec_of(w, alphas)
    md = pipeline.build_metadata(c, spec)
    sc = pipeline.compute_scores(c, spec, md)
    rep = Report()
    pm = h["phys_map"]
    G = w.G
    if check_meta and spec.policy != "thresh_box":
        _compare_meta(w, st, c, md, pm, spec)
    if spec.score == "gauss" or spec.policy == "thresh_box":
        _compare_gauss_scores(w, st, c, pm, spec, seqs)
    idx = st.sel.idx.cpu().numpy()
    cnt = st.sel.count.cpu().numpy()
    outs = {a: o.cpu().numpy() for a, o in st.outs.items()}
    gkey = st.scores.key.cpu().numpy() if (st.scores.key is not None and spec.policy != "thresh_box") else None
    lsh_slack = _lsh_tables(w, st, sc, seqs, spec) if spec.score == "lsh" else {}
    if spec.policy == "thresh_box":   # the box key of the combined scores: bit-exact as well
        bk = st.scores.key.cpu().numpy()
        for i, b in enumerate(seqs):
            assert np.array_equal(bk[b, :, :c.maxP], sc.key[i, :, :c.maxP]), f"box key mismatch in sequence {b}"
    for i, b in enumerate(seqs):
        for g in range(w.Hkv):
            rep.units += 1
            slack = lsh_slack.get(b, 0.0)
            if gkey is not None and slack > 0.0:     # certified rounding of a bucket mass: keys within slack
                n = c.maxP * c.S
                vn = pipeline_vnorm(c, md, i, g)
                dk = np.abs(gkey[b, g, :n].astype(np.float64) - sc.key[i, g, :n].astype(np.float64))
                fin = np.isfinite(sc.key[i, g, :n])
                assert np.array_equal(np.isfinite(gkey[b, g, :n]), fin)
                assert np.all(dk[fin] <= vn[fin] * slack * 2.0 ** -24 * (1 + 2 ** -20)
                              + np.spacing(np.abs(sc.key[i, g, :n][fin]))), f"lsh key beyond slack ({b},{g})"
            elif gkey is not None:
                n = c.maxP if spec.score in ("box", "pool") else c.maxP * c.S
                ok = np.array_equal(gkey[b, g, :n], sc.key[i, g, :n])
                if not ok:
                    bad = np.nonzero(gkey[b, g, :n] != sc.key[i, g, :n])[0]
                    raise AssertionError(f"key mismatch unit ({b},{g}) at {bad[:8]}: gpu {gkey[b, g, bad[:4]]} "
                                         f"oracle {sc.key[i, g, bad[:4]]}")
            r = pipeline.select_unit(c, spec, sc, i, g)
            got = idx[b, g, :cnt[b, g]]
            same = len(got) == len(r.sel) and np.array_equal(got, r.sel)
            if spec.policy in ("thresh", "thresh_box"):
                tau_g = st.sel.tau_hat[b, g * G:(g + 1) * G].cpu().numpy().astype(np.float64)
                if np.all(np.isnan(r.tau_hat)):          # empty sequence: no threshold
                    assert np.all(np.isnan(tau_g)) and len(got) == 0, (b, g, tau_g, got)
                    continue
                assert np.all(np.abs(tau_g - r.tau_hat) <= TAU_TOL * np.maximum(1.0, np.abs(r.tau_hat))), \
                    (b, g, tau_g, r.tau_hat)
                if not same:
                    diff = np.setxor1d(got, r.sel)
                    if spec.policy == "thresh":
                        shat = sc.shat[i, g * G:(g + 1) * G, :]
                        margin = np.max((spec.sel_alpha - 1.0) * shat[:, diff] - (r.tau_hat[:, None] - spec.delta),
                                        axis=0)
                    else:
                        margin = ((spec.sel_alpha - 1.0) * pipeline.scale_of(spec, c.d) * sc.key[i, g, diff]
                                  - (r.tau_hat.min() - spec.delta))
                    assert np.all(np.abs(margin) <= TAU_TOL * max(1.0, np.abs(r.tau_hat).max())), (b, g, diff, margin)
                    rep.near_ties += len(diff)
                    rep.ties.append(dict(seq=int(b), kv_head=int(g), indices=[int(x) for x in diff],
                                         margins=[float(x) for x in np.atleast_1d(margin)]))
            elif not same and slack > 0.0:   # differences only among keys within the slack of the cut
                kk = np.sort(sc.key[i, g, :c.length(b)].astype(np.float64))[::-1]
                cut = kk[min(spec.k, len(kk)) - 1]
                diff = np.setxor1d(got, r.sel)
                vn = pipeline_vnorm(c, md, i, g)
                gaps = np.abs(sc.key[i, g, diff] - cut)
                assert np.all(gaps <= 2 * vn[diff] * slack * 2.0 ** -24 + 1e-6 * abs(cut)), (b, g, diff)
                rep.near_ties += len(diff)
                rep.ties.append(dict(seq=int(b), kv_head=int(g), indices=[int(x) for x in diff],
                                     margins=[float(x) for x in gaps]))
            else:
                assert same, f"selection mismatch unit ({b},{g}): gpu {got[:10]}.. ({len(got)}) oracle " \
                             f"{r.sel[:10]}.. ({len(r.sel)})"
            # values: against the oracle's attention over the GPU's own selection (the same set where
            # the selections agree; where certified near-ties changed it, the GPU's set)
            if not same:
                rep.tie_units_checked += 1
            for a in spec.alphas:
                ref = pipeline.attend_unit(c, spec, i, g, r.sel if same else got, a)
                gpu = outs[a][b, g * G:(g + 1) * G]
                err = np.abs(gpu - ref)
                rep.max_err = max(rep.max_err, float((err / (ATOL + RTOL * np.abs(ref))).max()))
                assert np.all(err <= ATOL + RTOL * np.abs(ref)), \
                    f"output mismatch unit ({b},{g}) alpha {a}: max abs err {err.max():.3g}"
    return rep


def check(w: W.Workload, st: GpuStep, seqs=None, alphas=None, check_meta=True, **extra) -> Report:
    """compare() (one sequence per thread when several are given), then the parity record of the
    test (record())."""
    if seqs is not None and len(seqs) > 1:
        rep = compare_seqs(w, st, seqs, alphas=alphas, check_meta=check_meta)
    else:
        rep = compare(w, st, seqs=seqs, alphas=alphas, check_meta=check_meta)
    record(rep.entry(w, seqs, **extra))
    return rep


def compare_seqs(w: W.Workload, st: GpuStep, seqs, alphas=None, check_meta=True, threads=16) -> Report:
    """compare() of each sequence in `seqs` on its own, in parallel threads (the oracle releases
    the GIL), merged into one report."""
    rep = Report()
    with cf.ThreadPoolExecutor(min(threads, max(1, len(seqs)))) as ex:
        for r in ex.map(lambda b: compare(w, st, seqs=[b], alphas=alphas, check_meta=check_meta), list(seqs)):
            rep.merge(r)
    return rep


def _compare_gauss_scores(w, st, c, pm, spec, seqs):
    """Stage parity of the Gaussian scores: the oracle's m, s and estimated maximum computed from
    the GPU's own float32 moments of the same pages, element by element. The tolerance is what a
    float32 accumulation of the d terms could add (d 2^-24 of the sum of absolute terms, with a
    margin), plus the final rounding to float32."""
    ga = st.meta.gauss[torch.from_numpy(pm).to(w.k.device)].cpu().numpy().astype(np.float64)
    n_, h_ = ga.shape[:2]   # [n, Hkv, d / 16, 2, 16]: mean and variance blocks alternate
    mean = np.ascontiguousarray(ga[:, :, :, 0].reshape(n_, h_, -1))
    var = np.ascontiguousarray(ga[:, :, :, 1].reshape(n_, h_, -1))
    scale = pipeline.scale_of(spec, c.d)
    m, s, shat = oracle.score_gauss(c, mean, var, scale, spec.gauss_max == "quantile")
    sc = st.scores
    gm, gs, gh = (t[list(seqs)].cpu().numpy().astype(np.float64) for t in (sc.m, sc.s, sc.shat))
    q = bf16_to_f64(w.q[list(seqs)])
    eps = 2.0 * c.d * 2.0 ** -24
    for i in range(c.B):
        P = c.pages(i)
        if P == 0:
            continue
        phys = c.block_table[i, :P]
        n = np.array([c.page_tokens(i, p) for p in range(P)])
        fac = np.where(n > 1, (shat[i, :, :P] - m[i, :, :P]) / np.where(s[i, :, :P] > 0, s[i, :, :P], 1.0), 0.0)
        for h in range(c.Hq):
            g = h // c.G
            am = scale * (np.abs(mean[phys, g]) @ np.abs(q[i, h]))
            tol_m = eps * am + 2.0 ** -23 * np.abs(m[i, h, :P]) + 1e-30
            tol_s = eps * s[i, h, :P] + 1e-30
            tol_h = tol_m + tol_s * np.abs(fac[h]) + 2.0 ** -23 * np.abs(shat[i, h, :P])
            for name, got, ref, tol in (("m", gm, m, tol_m), ("s", gs, s, tol_s), ("shat", gh, shat, tol_h)):
                err = np.abs(got[i, h, :P] - ref[i, h, :P])
                assert np.all(err <= tol), \
                    f"gaussian {name} mismatch seq {seqs[i]} head {h}: max err {err.max():.3g} at page {err.argmax()}"
            assert np.all(np.isnan(gm[i, h, P:c.maxP])), f"gaussian m past the sequence must be NaN ({seqs[i]}, {h})"


def stage_parity_box_budget(w: W.Workload, st: GpuStep, seqs, pct: int, threads=16) -> int:
    """Stage parity of the page scoring and selection on every sequence in `seqs`: the oracle's box
    keys computed from the GPU's own box metadata (bit-identical bytes) must equal the GPU's keys
    bit for bit, and the oracle's budget selection over those keys must equal the GPU's selection.
    Needs no K or V on the host. Returns the number of units compared."""
    bt = w.block_table.cpu().numpy()
    key = st.scores.key.cpu().numpy()
    idx, cnt = st.sel.idx.cpu().numpy(), st.sel.count.cpu().numpy()
    qb = W.host_arrays_q(w)

    def one(b):
        P = w.pages(b)
        if P == 0:
            assert np.all(cnt[b] == 0), b
            return w.Hkv
        box = bf16_to_f64(st.meta.box[torch.from_numpy(bt[b, :P].astype(np.int64)).to(w.k.device)])
        n_, h_ = box.shape[:2]
        kmin = np.ascontiguousarray(box[:, :, :, 0].reshape(n_, h_, -1))
        kmax = np.ascontiguousarray(box[:, :, :, 1].reshape(n_, h_, -1))
        kdt = np.uint16 if w.dtype == torch.bfloat16 else np.float32
        dummy = np.zeros((P, w.Hkv, w.S, w.d), dtype=kdt)    # never read by the scoring (zero pages, untouched)
        c = oracle.Cache(q=qb[b:b + 1], k=dummy, v=dummy, block_table=np.arange(P, dtype=np.int32)[None, :],
                         seq_lens=np.array([w.lens[b]], dtype=np.int32))
        ok = oracle.score_box(c, kmin, kmax)
        for g in range(w.Hkv):
            assert np.array_equal(ok[0, g, :P], key[b, g, :P]), f"box key mismatch ({b},{g})"
            ref = oracle.select_topk(ok[0, g, :P], oracle.budget_k(P, pct))
            got = idx[b, g, :cnt[b, g]]
            assert len(got) == len(ref) and np.array_equal(got, ref), f"selection mismatch ({b},{g})"
        return w.Hkv

    with cf.ThreadPoolExecutor(threads) as ex:
        return sum(ex.map(one, list(seqs)))


def full_cache_invariants(w: W.Workload, st: GpuStep, seqs, threads=16) -> dict:
    """The error bound of the sparse output against the full-cache output ("EntmaxKV" s3): with
    delta the full-cache weight of the tokens left out of the selection and B the largest value
    norm of the sequence, |o_full - o_sparse|_2 <= 2 B delta. Checked on the GPU's outputs, with the
    output tolerance added for the GPU's own rounding; also reports the recall of the full-cache
    support (tokens with weight > 0) by the selection."""
    spec = spec_of(w)
    idx, cnt = st.sel.idx.cpu().numpy(), st.sel.count.cpu().numpy()
    outs = {a: o.cpu().numpy() for a, o in st.outs.items()}
    gran = 1 if spec.score in ("proj", "lsh") else 0
    stats = dict(units=0, max_delta=0.0, min_recall=1.0, max_ratio=0.0)

    def one(b):
        h = W.host_arrays(w, [b])
        c = oracle_cache(h)
        res = []
        L = c.length(0)
        t = np.arange(L)
        for g in range(w.Hkv):
            sel = idx[b, g, :cnt[b, g]]
            keep = np.zeros(max(L, c.pages(0) * c.S), dtype=bool)
            if gran:
                keep[sel] = True
            else:
                for p in sel:
                    keep[p * c.S:(p + 1) * c.S] = True
            keep = keep[:L]
            vb = h["v"][c.block_table[0, t // c.S], g, t % c.S]     # [L, d] raw bytes of the valid rows
            rows = ((vb.astype(np.uint32) << 16).view(np.float32) if vb.dtype == np.uint16 else vb).astype(np.float64)
            Bv = float(np.sqrt((rows * rows).sum(1)).max()) if L else 0.0
            for a in spec.alphas:
                full, ps = pipeline.full_reference(c, spec, 0, g, a)
                sparse = pipeline.attend_unit(c, spec, 0, g, sel, a)
                for hh in range(w.G):
                    p = ps[hh]
                    delta = float(p[~keep].sum())
                    supp = p > 0
                    recall = float(keep[supp].mean()) if supp.any() else 1.0
                    tol = np.linalg.norm(ATOL + RTOL * np.abs(sparse[hh]))
                    gap = float(np.linalg.norm(full[hh] - outs[a][b, g * w.G + hh]))
                    bound = 2.0 * Bv * delta + tol
                    assert gap <= bound, (b, g, hh, a, gap, 2.0 * Bv * delta, tol)
                    res.append((delta, recall, gap / bound if bound > 0 else 0.0))
        return res

    with cf.ThreadPoolExecutor(min(threads, max(1, len(seqs)))) as ex:
        for res in ex.map(one, list(seqs)):
            for delta, recall, ratio in res:
                stats["units"] += 1
                stats["max_delta"] = max(stats["max_delta"], delta)
                stats["min_recall"] = min(stats["min_recall"], recall)
                stats["max_ratio"] = max(stats["max_ratio"], ratio)
    return stats


def pipeline_vnorm(c, md, i, g):
    """Value norms [maxP * S] of sequence i (oracle cache numbering), KV head g, by token position."""
    t = np.arange(c.maxP * c.S)
    out = np.zeros(c.maxP * c.S)
    L = c.length(i)
    phys = c.block_table[i, t[:L] // c.S]
    out[:L] = md.vnorm[phys, g, t[:L] % c.S]
    return out


def _lsh_tables(w, st, sc, seqs, spec):
    """GPU bucket masses (the scoring workspace, [B, Hkv, L, 2^P, G] uint32) against the oracle's.
    Both round p * 2^24 of a float64 p; their exp implementations differ in the last bit at most,
    so an entry may differ by one only where p * 2^24 lies within about 1e-9 of a half-integer.
    Such entries are certified with an independent float64 evaluation of p and reported as the
    largest key slack (in units of 2^-24 times the value norm) per sequence."""
    import scipy.special
    Lt, nb = sc.lsh_tab.shape[2], sc.lsh_tab.shape[3]
    P = nb.bit_length() - 1
    n = w.B * w.Hq * Lt * nb
    raw = st.scores.ws[:4 * n].view(torch.int32).cpu().numpy().view(np.uint32)
    gt = raw.reshape(w.B, w.Hkv, Lt, nb, w.G).transpose(0, 1, 4, 2, 3).reshape(w.B, w.Hq, Lt, nb)
    planes = spec.lsh_planes.astype(np.float64)
    sgn = np.where((np.arange(nb)[:, None] >> np.arange(P)[None, :]) & 1, 1.0, -1.0)
    slack = {}
    for i, b in enumerate(seqs):
        d = gt[b].astype(np.int64) - sc.lsh_tab[i].astype(np.int64)
        assert np.all(np.abs(d) <= 1), f"bucket masses differ by more than one in sequence {b}"
        bad = np.argwhere(d != 0)
        for h, l, beta in bad:
            q = bf16_to_f64(w.q[b, h])
            z = planes[l] @ q / np.linalg.norm(q)
            x = scipy.special.softmax(sgn @ z / float(np.float32(spec.lsh_tau)))[beta] * 2.0 ** 24
            assert abs(x - np.floor(x) - 0.5) < 1e-6, (b, h, l, beta, x)
        if len(bad):
            slack[b] = float(Lt)
    return slack


def _compare_meta(w, st, c, md, pm, spec):
    """Metadata of every page the sampled sequences use: box and kproj bit-exact; Gaussian mean and
    variance equal the float32 rounding of the float64 values."""
    used = set()
    for i in range(c.B):
        used.update(int(x) for x in c.block_table[i, :c.pages(i)])
    used = np.array(sorted(used), dtype=np.int64)
    if len(used) == 0:
        return
    gp = torch.from_numpy(pm[used]).to(w.k.device)
    if spec.score == "box":
        box = bf16_to_f64(st.meta.box[gp])          # [n, Hkv, d / C, 2, C]: min and max blocks alternate
        n_, h_ = box.shape[:2]
        assert np.array_equal(box[:, :, :, 0].reshape(n_, h_, -1), md.kmin[used]), "kmin mismatch"
        assert np.array_equal(box[:, :, :, 1].reshape(n_, h_, -1), md.kmax[used]), "kmax mismatch"
    elif spec.score == "gauss":
        ga = st.meta.gauss[gp].cpu().numpy()           # [n, Hkv, d / 16, 2, 16]: mean and variance blocks alternate
        n_, h_ = ga.shape[:2]
        assert np.array_equal(ga[:, :, :, 0].reshape(n_, h_, -1), md.mean[used].astype(np.float32)), "mean mismatch"
        assert np.array_equal(ga[:, :, :, 1].reshape(n_, h_, -1), md.var[used].astype(np.float32)), "var mismatch"
    elif spec.score == "pool":
        po = st.meta.pool[gp].cpu().numpy()            # [n, Hkv, S/pb, d]; sub-blocks with a token only
        owner = {}
        for i in range(c.B):
            for p in range(c.pages(i)):
                owner[int(c.block_table[i, p])] = c.page_tokens(i, p)
        for n, pg in enumerate(used):
            nsb = -(-owner[int(pg)] // spec.pool_block)
            assert np.array_equal(po[n, :, :nsb], md.pool[pg, :, :nsb]), f"pool mismatch page {pg}"
    elif spec.score == "lsh":                          # bucket ids and value norms of valid tokens
        bk = st.meta.lsh_bucket[gp].cpu().numpy()
        vn = st.meta.vnorm[gp].cpu().numpy()
        owner = {}
        for i in range(c.B):
            for p in range(c.pages(i)):
                owner[int(c.block_table[i, p])] = c.page_tokens(i, p)
        for n, pg in enumerate(used):
            nt = owner[int(pg)]
            assert np.array_equal(bk[n, :, :nt], md.lsh_bucket[pg, :, :nt]), f"bucket mismatch page {pg}"
            assert np.array_equal(vn[n, :, :nt].view(np.uint32), md.vnorm[pg, :, :nt].view(np.uint32)), \
                f"value norm mismatch page {pg}"
    elif spec.score == "proj":
        kp = st.meta.kproj[gp].cpu().numpy().view(np.uint16)
        owner = {}
        for i in range(c.B):
            for p in range(c.pages(i)):
                owner[int(c.block_table[i, p])] = c.page_tokens(i, p)
        for n, pg in enumerate(used):
            nt = owner[int(pg)]          # only rows of valid tokens are defined
            assert np.array_equal(kp[n, :, :nt], md.kproj[pg, :, :nt]), f"kproj mismatch page {pg}"

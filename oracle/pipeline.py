"""One decode-attention step computed by the float64 oracle from raw inputs only.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``). The step is the pages' pipeline
([EKV] "EntmaxKV" summary s2: page metadata -> query-aware page scores -> candidate
selection -> attention over the selected KV only; [JSSA] abstract for the token-level variant):

  metadata  box (kmin, kmax) | gauss (mean, var) | proj (k~ = RN_bf16(P k)) | pool (sub-block mean keys)
            | lsh (bucket ids per table, value norms)
  scores    box / pool key per (b, g, page) | gauss (m, s, shat) per (b, h, page)
            | proj / lsh key per (b, g, token)
  select    topk(k) | budget(pct) | thresh(alpha, delta) | thresh_box(alpha, delta) | token_topk(k) | all
  attend    alpha = 1 (softmax) or alpha in (1, 2] (entmax) per query head over the selection
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import (Cache, attend_full_head, attend_head, budget_k, lsh_tables, meta_box, meta_gauss, meta_lsh, meta_pool,
               meta_proj, score_box, score_gauss, score_lsh, score_pool, score_proj, select_thresh, select_thresh_box,
               select_topk, tau_hat)


@dataclass
class Spec:
    score: str                 # 'box' | 'gauss' | 'proj' | 'pool' | 'lsh'
    policy: str                # 'topk' | 'budget' | 'thresh' | 'thresh_box' | 'token_topk' | 'all'
    k: int = 0
    pct: int = 0
    sel_alpha: float = 1.5     # alpha of the Gaussian threshold
    delta: float = 0.0
    alphas: tuple = (1.0,)     # attention alphas to evaluate
    scale: float = 0.0         # logit scale; 0 means 1/sqrt(d)
    proj: np.ndarray | None = None
    gauss_max: str = "sqrt2log"  # estimated page maximum: m + s sqrt(2 ln n) | 'quantile': m + s Phi^-1(1 - 1/n)
    pool_block: int = 4          # tokens per sub-block of the pooled page key
    lsh_planes: np.ndarray | None = None   # soft-LSH hyperplanes [L, P, d] float32
    lsh_tau: float = 1.0                   # soft-LSH temperature


@dataclass
class Metadata:
    kmin: np.ndarray | None = None
    kmax: np.ndarray | None = None
    mean: np.ndarray | None = None
    var: np.ndarray | None = None
    kproj: np.ndarray | None = None
    pool: np.ndarray | None = None
    lsh_bucket: np.ndarray | None = None
    vnorm: np.ndarray | None = None


@dataclass
class Scores:
    key: np.ndarray | None = None      # box [B,Hkv,maxP] or proj [B,Hkv,maxP*S], float32
    m: np.ndarray | None = None        # gauss [B,Hq,maxP]
    s: np.ndarray | None = None
    shat: np.ndarray | None = None
    lsh_tab: np.ndarray | None = None  # lsh [B,Hq,L,2^P] uint32 fixed-point bucket masses


@dataclass
class UnitResult:
    sel: np.ndarray                            # ascending page or token indices
    tau_hat: np.ndarray | None = None          # [G] (thresh only)
    out: dict = field(default_factory=dict)    # alpha -> [G, d] float64


def scale_of(spec: Spec, d: int) -> float:
    return spec.scale if spec.scale else 1.0 / math.sqrt(d)


def _needs(spec: Spec):
    """Score kinds a step needs: the threshold with the box key uses both box and Gaussian."""
    return {spec.score} | ({"box", "gauss"} if spec.policy == "thresh_box" else set())


def build_metadata(c: Cache, spec: Spec) -> Metadata:
    md = Metadata()
    kinds = _needs(spec)
    if "box" in kinds:
        md.kmin, md.kmax = meta_box(c)
    if "gauss" in kinds:
        md.mean, md.var = meta_gauss(c)
    if "proj" in kinds:
        md.kproj = meta_proj(c, spec.proj)
    if "pool" in kinds:
        md.pool = meta_pool(c, spec.pool_block)
    if "lsh" in kinds:
        md.lsh_bucket, md.vnorm = meta_lsh(c, spec.lsh_planes)
    return md


def compute_scores(c: Cache, spec: Spec, md: Metadata) -> Scores:
    sc = Scores()
    kinds = _needs(spec)
    if "box" in kinds:
        sc.key = score_box(c, md.kmin, md.kmax)
    if "gauss" in kinds:
        sc.m, sc.s, sc.shat = score_gauss(c, md.mean, md.var, scale_of(spec, c.d), spec.gauss_max == "quantile")
    if "proj" in kinds:
        sc.key = score_proj(c, spec.proj, md.kproj)
    if "pool" in kinds:
        sc.key = score_pool(c, spec.pool_block, md.pool)
    if "lsh" in kinds:
        sc.lsh_tab = lsh_tables(c, spec.lsh_planes, spec.lsh_tau)
        sc.key = score_lsh(c, md.lsh_bucket, md.vnorm, sc.lsh_tab)
    return sc


def page_counts(c: Cache, b: int) -> np.ndarray:
    return np.array([c.page_tokens(b, p) for p in range(c.pages(b))], dtype=np.int32)


def select_unit(c: Cache, spec: Spec, sc: Scores, b: int, g: int) -> UnitResult:
    P_b, L_b = c.pages(b), c.length(b)
    if spec.policy == "all":
        n = L_b if spec.score in ("proj", "lsh") else P_b
        return UnitResult(sel=np.arange(n, dtype=np.int32))
    if spec.policy == "topk":
        return UnitResult(sel=select_topk(sc.key[b, g, :P_b], spec.k))
    if spec.policy == "budget":
        return UnitResult(sel=select_topk(sc.key[b, g, :P_b], budget_k(P_b, spec.pct)))
    if spec.policy == "token_topk":
        return UnitResult(sel=select_topk(sc.key[b, g, :L_b], spec.k))
    if spec.policy in ("thresh", "thresh_box"):
        heads = range(g * c.G, g * c.G + c.G)
        if P_b == 0:
            return UnitResult(sel=np.zeros(0, np.int32), tau_hat=np.full(c.G, np.nan))
        n = page_counts(c, b)
        taus = np.array([tau_hat(sc.m[b, h, :P_b], sc.s[b, h, :P_b], n, spec.sel_alpha) for h in heads])
        if spec.policy == "thresh":
            sel = select_thresh(sc.shat[b, g * c.G:(g + 1) * c.G, :P_b], taus, spec.sel_alpha, spec.delta)
        else:
            sel = select_thresh_box(sc.key[b, g, :P_b], taus, scale_of(spec, c.d), spec.sel_alpha, spec.delta)
        return UnitResult(sel=sel, tau_hat=taus)
    raise ValueError(spec.policy)


def attend_unit(c: Cache, spec: Spec, b: int, g: int, sel: np.ndarray, alpha: float) -> np.ndarray:
    gran = 1 if spec.score in ("proj", "lsh") else 0
    sc = scale_of(spec, c.d)
    return np.stack([attend_head(c, b, h, sel, gran, alpha, sc)[0] for h in range(g * c.G, (g + 1) * c.G)])


def run_unit(c: Cache, spec: Spec, sc: Scores, b: int, g: int) -> UnitResult:
    r = select_unit(c, spec, sc, b, g)
    for a in spec.alphas:
        r.out[a] = attend_unit(c, spec, b, g, r.sel, a)
    return r


def run(c: Cache, spec: Spec, units=None):
    """Full step from raw inputs. Returns (metadata, scores, {(b, g): UnitResult})."""
    md = build_metadata(c, spec)
    sc = compute_scores(c, spec, md)
    if units is None:
        units = [(b, g) for b in range(c.B) for g in range(c.Hkv)]
    return md, sc, {u: run_unit(c, spec, sc, *u) for u in units}


def full_reference(c: Cache, spec: Spec, b: int, g: int, alpha: float):
    """Full-cache outputs [G, d] and weights (list of [L] arrays) of unit (b, g)."""
    outs, ps = [], []
    for h in range(g * c.G, (g + 1) * c.G):
        o, p = attend_full_head(c, b, h, alpha, scale_of(spec, c.d))
        outs.append(o)
        ps.append(p)
    return np.stack(outs), ps

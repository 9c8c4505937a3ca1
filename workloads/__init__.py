"""Seeded synthetic inputs for sparse decode attention over a paged GQA KV cache.

This module only draws inputs. It holds none of the method's arithmetic (no metadata, scores,
selection or attention) and imports neither the GPU binding nor the oracle. Both sides receive
the same bytes: GPU tests use the tensors directly, the oracle gets host copies (``host_cache``).

Seven workloads, shaped like the pages' long-context decode settings (GQA 32/8 x 128 as in
Llama-3.1-8B, 32K to 256K contexts, bf16):

  tiny        B=1, 1/1 heads, d=64, L=4096, page 16, float32 N(0,1); top-32 pages by box bound;
              entmax alpha=1.5 and softmax
  gqa32k      B=8, 32/8 heads, d=128, L=32768, page 16, bf16 N(0,1) with 4 planted
              high-dot-product tokens per KV head (one per query head, q.k/sqrt(d) ~ 16);
              top-64 pages by box bound; softmax and alpha=1.5
  long_gauss  B=4, 32/8, d=128, L=131072, page 32; q, V ~ N(0,1); keys (x + mu_p) * c with
              x ~ N(0,1), mu_p an AR(1) drift over pages (rho 0.99, stationary sd 0.5, per KV head),
              c = 10 on 8 seeded channels per KV head; Gaussian threshold alpha=1.5, Delta=0.5
  token128k   B=16, 32/8, d=128, L=131072, page 16, bf16 N(0,1); shared rank-32 projection with
              orthonormal rows (QR of a seeded Gaussian); top-2048 tokens per KV head; softmax
  ragged      64 sequences, L ~ U{8192..262144}, 64/8 heads, d=128, page 64, bf16 N(0,1);
              5% page budget by box bound; sparsemax (alpha=2)
  pool32k     the gqa32k draw (seed 1006) with the pooled page key instead of the box bound: means
              of 4-token sub-blocks, the page key the largest q.mean over sub-blocks and query
              heads; top-64 pages; softmax and alpha=1.5
  socket128k  B=4, 32/8, d=128, L=131072, page 16, bf16 N(0,1); 32 soft-LSH tables of 6 random
              N(0,1) hyperplanes each (float32), temperature 0.5; top-4096 tokens per KV head
              (32x sparsity); softmax

Physical pages are a seeded permutation (block_table), so every kernel goes through the
indirection. Any field can be overridden (smaller B or L for parity cases, ragged tails).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

CONFIGS = {
    "tiny": dict(B=1, Hq=1, Hkv=1, d=64, L=4096, S=16, dtype="f32", seed=1001,
                 score="box", policy="topk", k=32, alphas=(1.5, 1.0)),
    "gqa32k": dict(B=8, Hq=32, Hkv=8, d=128, L=32768, S=16, dtype="bf16", seed=1002,
                   planted=4, zstar=16.0, score="box", policy="topk", k=64, alphas=(1.0, 1.5)),
    "long_gauss": dict(B=4, Hq=32, Hkv=8, d=128, L=131072, S=32, dtype="bf16", seed=1003,
                       outlier_channels=8, outlier_scale=10.0, drift_rho=0.99, drift_sd=0.5,
                       score="gauss", policy="thresh", sel_alpha=1.5, delta=0.5, alphas=(1.5,)),
    "token128k": dict(B=16, Hq=32, Hkv=8, d=128, L=131072, S=16, dtype="bf16", seed=1004,
                      proj_rank=32, score="proj", policy="token_topk", k=2048, alphas=(1.0,)),
    "ragged": dict(B=64, Hq=64, Hkv=8, d=128, Lmin=8192, Lmax=262144, S=64, dtype="bf16", seed=1005,
                   score="box", policy="budget", pct=5, alphas=(2.0,)),
    "pool32k": dict(B=8, Hq=32, Hkv=8, d=128, L=32768, S=16, dtype="bf16", seed=1006,
                    planted=4, zstar=16.0, score="pool", pool_block=4, policy="topk", k=64, alphas=(1.0, 1.5)),
    "socket128k": dict(B=4, Hq=32, Hkv=8, d=128, L=131072, S=16, dtype="bf16", seed=1007, score="lsh",
                       lsh_tables=32, lsh_bits=6, lsh_tau=0.5, policy="token_topk", k=4096, alphas=(1.0,)),
}


@dataclass
class Workload:
    name: str
    cfg: dict
    B: int
    Hq: int
    Hkv: int
    d: int
    S: int
    maxP: int
    Nphys: int
    dtype: torch.dtype
    q: torch.Tensor            # [B, Hq, d]
    k: torch.Tensor            # [Nphys, Hkv, S, d]
    v: torch.Tensor            # [Nphys, Hkv, S, d]
    block_table: torch.Tensor  # [B, maxP] int32
    seq_lens: torch.Tensor     # [B] int32
    lens: list                 # host copy of seq_lens
    proj: torch.Tensor | None = None     # [r, d] float32 (token128k)
    lsh_planes: torch.Tensor | None = None   # [tables, bits, d] float32 (socket128k)
    planted: np.ndarray | None = None    # [B, Hkv, n] token positions (gqa32k)
    extra: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def pages(self, b: int) -> int:
        return (self.lens[b] + self.S - 1) // self.S

    @property
    def max_len(self) -> int:
        return max(self.lens) if self.lens else 0


def _randn(shape, gen, device, dtype, chunk_rows=None):
    """N(0,1) draws in float32, converted to dtype, filled chunk by chunk along dim 0."""
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    per_row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    chunk_rows = chunk_rows or max(1, (1 << 26) // max(per_row, 1))
    for i in range(0, rows, chunk_rows):
        n = min(chunk_rows, rows - i)
        out[i:i + n] = torch.randn((n,) + tuple(shape[1:]), generator=gen, device=device,
                                   dtype=torch.float32).to(dtype)
    return out


def make(name: str, device="cpu", **over) -> Workload:
    """Draw workload `name` (see CONFIGS) on `device`, with optional field overrides."""
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(cfg["seed"]))
    dtype = torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16
    B, Hq, Hkv, d, S = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["S"]

    if "lens" in cfg:
        lens = [int(x) for x in cfg["lens"]]
    elif "Lmin" in cfg:
        lens = torch.randint(cfg["Lmin"], cfg["Lmax"] + 1, (B,), generator=gen, device=dev).tolist()
    else:
        lens = [int(cfg["L"])] * B
    assert len(lens) == B
    pages = [(L + S - 1) // S for L in lens]
    maxP = max(1, max(pages) if pages else 1)
    maxP = max(maxP, int(cfg.get("maxP", 0)))
    Nphys = max(1, sum(pages))
    perm = torch.randperm(Nphys, generator=gen, device=dev).to(torch.int32)
    bt = torch.zeros((B, maxP), dtype=torch.int32, device=dev)
    owner = torch.zeros((Nphys, 2), dtype=torch.int64, device=dev)   # physical page -> (b, p)
    off = 0
    for b, P in enumerate(pages):
        if P:
            bt[b, :P] = perm[off:off + P]
            owner[perm[off:off + P].long(), 0] = b
            owner[perm[off:off + P].long(), 1] = torch.arange(P, device=dev)
        off += P
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)

    q = _randn((B, Hq, d), gen, dev, dtype)
    k = _randn((Nphys, Hkv, S, d), gen, dev, dtype)
    v = _randn((Nphys, Hkv, S, d), gen, dev, dtype)
    w = Workload(name=name, cfg=cfg, B=B, Hq=Hq, Hkv=Hkv, d=d, S=S, maxP=maxP, Nphys=Nphys,
                 dtype=dtype, q=q, k=k, v=v, block_table=bt, seq_lens=seq_lens, lens=lens)

    if cfg.get("outlier_channels"):
        _outliers_and_drift(w, cfg, gen, dev, owner, pages)
    if cfg.get("planted"):
        _plant(w, cfg, gen, dev)
    if cfg.get("proj_rank"):
        r = int(cfg["proj_rank"])
        a = torch.randn((d, r), generator=gen, device=dev, dtype=torch.float32).double().cpu()
        qm, _ = torch.linalg.qr(a)           # [d, r], orthonormal columns
        w.proj = qm.t().contiguous().float().to(dev)   # [r, d], orthonormal rows
    if cfg.get("lsh_tables"):
        w.lsh_planes = torch.randn((int(cfg["lsh_tables"]), int(cfg["lsh_bits"]), d), generator=gen, device=dev,
                                   dtype=torch.float32)
    return w


def _outliers_and_drift(w: Workload, cfg, gen, dev, owner, pages):
    """Keys become RN((x + mu_p) * c): AR(1) drift mu over logical pages per (b, KV head),
    stationary sd `drift_sd`, coefficient `drift_rho`; c = `outlier_scale` on
    `outlier_channels` seeded channels per (b, KV head), 1 elsewhere."""
    B, Hkv, d = w.B, w.Hkv, w.d
    rho, sd = float(cfg["drift_rho"]), float(cfg["drift_sd"])
    maxP = w.maxP
    cur = (sd * torch.randn((B, Hkv, d), generator=gen, device=dev)).cpu().numpy()
    innov = sd * math.sqrt(1.0 - rho * rho)
    eps = torch.randn((maxP, B, Hkv, d), generator=gen, device=dev).cpu().numpy()
    # The recursion runs on the host in float32 with the same operations as elementwise device
    # arithmetic would (rho * cur and innov * eps rounded to float32, then their float32 sum),
    # and the whole drift goes to the device in one copy: a per-page loop of device operations
    # would issue several thousand tiny dispatches.
    rho32, innov32 = np.float32(rho), np.float32(innov)
    mu_h = np.empty((B, Hkv, maxP, d), dtype=np.float32)
    for p in range(maxP):
        if p:
            cur = rho32 * cur + innov32 * eps[p]
        mu_h[:, :, p] = cur
    mu = torch.from_numpy(mu_h).to(dev)
    nch = int(cfg["outlier_channels"])
    # one permutation of the channels per (b, KV head), drawn in order, applied in one scatter
    chans = torch.stack([torch.randperm(d, generator=gen, device=dev)[:nch] for _ in range(B * Hkv)])
    scale = torch.ones((B * Hkv, d), dtype=torch.float32, device=dev)
    scale.scatter_(1, chans, float(cfg["outlier_scale"]))
    scale = scale.view(B, Hkv, d)
    # physical page -> its (b, p): add the drift and scale, chunk by chunk
    chunk = max(1, (1 << 24) // (Hkv * w.S * d))
    for i in range(0, w.Nphys, chunk):
        n = min(chunk, w.Nphys - i)
        b_idx, p_idx = owner[i:i + n, 0], owner[i:i + n, 1]
        mu_pg = mu[b_idx, :, p_idx]           # [n, Hkv, d]
        sc_pg = scale[b_idx]                  # [n, Hkv, d]
        x = w.k[i:i + n].float()
        w.k[i:i + n] = ((x + mu_pg[:, :, None, :]) * sc_pg[:, :, None, :]).to(w.dtype)
    w.extra["outlier_scale"] = scale


def _plant(w: Workload, cfg, gen, dev):
    """Per (b, KV head): `planted` distinct uniform token positions; token j gets the key
    RN(zstar * sqrt(d) * q_h / |q_h|^2) for query head h = g*G + (j mod G), so that
    q_h . k / sqrt(d) ~= zstar."""
    n, zstar = int(cfg["planted"]), float(cfg["zstar"])
    pos = np.zeros((w.B, w.Hkv, n), dtype=np.int64)
    for b in range(w.B):
        for g in range(w.Hkv):
            pp = torch.randperm(w.lens[b], generator=gen, device=dev)[:n].cpu().numpy()
            pos[b, g, :len(pp)] = pp
            for j, t in enumerate(pp):
                h = g * w.G + (j % w.G)
                qh = w.q[b, h].float()
                krow = zstar * math.sqrt(w.d) * qh / (qh * qh).sum()
                phys = int(w.block_table[b, int(t) // w.S])
                w.k[phys, g, int(t) % w.S] = krow.to(w.dtype)
    w.planted = pos


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().astype(np.float32, copy=False)


def host_arrays_q(w: Workload) -> np.ndarray:
    """Exact host bytes of the queries alone, [B, Hq, d]."""
    return _bits(w.q)


def host_arrays(w: Workload, seqs=None):
    """Exact host bytes for the oracle: dict(q, k, v, block_table, seq_lens, phys_map).

    With `seqs`, only those sequences are copied: their pages are packed into a new physical
    array in (sequence, logical page) order, and phys_map[i] gives the original physical page of
    packed page i. Without it the whole cache is copied and phys_map is the identity."""
    if seqs is None:
        return dict(q=_bits(w.q), k=_bits(w.k), v=_bits(w.v),
                    block_table=w.block_table.cpu().numpy().astype(np.int32),
                    seq_lens=np.array(w.lens, dtype=np.int32),
                    phys_map=np.arange(w.Nphys, dtype=np.int64))
    seqs = list(seqs)
    bt = w.block_table.cpu().numpy()
    rows, new_bt, off = [], np.zeros((len(seqs), w.maxP), dtype=np.int32), 0
    for i, b in enumerate(seqs):
        P = w.pages(b)
        rows.extend(int(x) for x in bt[b, :P])
        new_bt[i, :P] = np.arange(off, off + P, dtype=np.int32)
        off += P
    idx = torch.tensor(rows if rows else [0], dtype=torch.long, device=w.k.device)
    return dict(q=_bits(w.q[seqs]), k=_bits(w.k[idx]), v=_bits(w.v[idx]), block_table=new_bt,
                seq_lens=np.array([w.lens[b] for b in seqs], dtype=np.int32),
                phys_map=np.array(rows if rows else [0], dtype=np.int64))

"""GPU parity of skv_append_page_meta: after new tokens, the metadata of the pages holding them must
equal a full build at the new lengths (GPU and oracle), and every other page and row must be left
as it was."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import gpu_harness as H
import sparse_kv_cache_build_amd as skv
import workloads as W
from oracle import pipeline

pytestmark = pytest.mark.gpu

CASES = [
    # (workload, overrides, n_new): one token inside a page, one token opening a page, several tokens
    # across page boundaries, a sequence shorter than n_new, an empty sequence, page size 64
    ("gqa32k", dict(B=3, lens=[3000, 3009, 4096]), 1),
    ("gqa32k", dict(B=3, lens=[3001, 16, 1]), 1),
    ("long_gauss", dict(B=3, lens=[6000, 6033, 5]), 37),
    ("token128k", dict(B=3, lens=[5000, 4097, 0], k=512), 3),
    ("token128k", dict(B=2, lens=[5000, 20], k=512), 40),
    ("ragged", dict(B=3, lens=[4500, 129, 64]), 2),
    ("pool32k", dict(B=3, lens=[3000, 3003, 5]), 3),   # pooled key: sub-blocks of 4 in pages of 16
    ("socket128k", dict(B=3, lens=[5000, 4113, 2], k=256), 19),   # soft-LSH buckets and value norms
    # more than 128 new tokens per sequence: the projected keys and soft-LSH buckets take the tiled
    # row-dot kernel (fewer take one thread per token and output)
    ("token128k", dict(B=2, lens=[5000, 900], k=512), 700),
    ("socket128k", dict(B=2, lens=[5000, 300], k=256), 300),
]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _used_pages(w, lens):
    bt = w.block_table.cpu().numpy()
    return {int(bt[b, p]): (b, p) for b in range(w.B) for p in range((lens[b] + w.S - 1) // w.S)}


def _snapshot(meta):
    keys = ("box", "gauss", "kproj", "pool", "lsh_bucket", "vnorm")
    return {k: getattr(meta, k).clone() for k in keys if getattr(meta, k) is not None}


def _page_meta(meta, kind, phys):
    """The page's metadata for kinds defined on the whole page (box, gauss) or on its sub-blocks."""
    return getattr(meta, "gauss" if kind == "gauss_q" else kind)[phys]


@pytest.mark.parametrize("name,over,n_new", CASES)
def test_append_equals_rebuild(dev, name, over, n_new):
    H.log(f"[append] {name} {over} n_new={n_new}")
    w = W.make(name, device=dev, **over)
    kind = w.cfg["score"]
    new = [int(x) for x in w.lens]
    old = [max(0, L - n_new) for L in new]
    cache = skv.PagedCache(w.k, w.v, w.block_table, w.seq_lens, w.Hq)
    w.seq_lens.copy_(torch.tensor(old, dtype=torch.int32))
    pb = w.cfg.get("pool_block", 0)
    meta = skv.build_page_meta(cache, (kind,), proj=w.proj, pool_block=pb, lsh_planes=w.lsh_planes)
    torch.cuda.synchronize()
    before = _snapshot(meta)
    w.seq_lens.copy_(torch.tensor(new, dtype=torch.int32))
    skv.append_page_meta(cache, meta, n_new)
    ref = skv.build_page_meta(cache, (kind,), proj=w.proj, pool_block=pb, lsh_planes=w.lsh_planes)
    torch.cuda.synchronize()

    # 1. equal to a fresh build of every page in use, bit for bit
    for phys, (b, p) in _used_pages(w, new).items():
        n = min(w.S, new[b] - p * w.S)
        if kind == "proj":
            assert torch.equal(meta.kproj[phys, :, :n], ref.kproj[phys, :, :n]), (b, p)
        elif kind == "lsh":
            assert torch.equal(meta.lsh_bucket[phys, :, :n], ref.lsh_bucket[phys, :, :n]), (b, p)
            assert torch.equal(meta.vnorm[phys, :, :n], ref.vnorm[phys, :, :n]), (b, p)
        elif kind == "pool":                    # sub-blocks holding a token
            nsb = -(-n // pb)
            assert torch.equal(meta.pool[phys, :, :nsb], ref.pool[phys, :, :nsb]), (b, p)
        else:
            assert torch.equal(_page_meta(meta, kind, phys), _page_meta(ref, kind, phys)), (b, p)

    # 2. untouched: pages and kproj rows that hold no new token
    for phys, (b, p) in _used_pages(w, old).items():
        first_new = old[b]                     # tokens >= old[b] are new
        if kind in ("proj", "lsh"):                 # per-token rows: the old ones stay as they were
            n_old = min(w.S, old[b] - p * w.S)
            for key in (("kproj",) if kind == "proj" else ("lsh_bucket", "vnorm")):
                assert torch.equal(getattr(meta, key)[phys, :, :n_old], before[key][phys, :, :n_old]), (b, p)
        elif (p + 1) * w.S <= first_new:       # the page ended before the new tokens
            key = "gauss" if kind == "gauss_q" else kind
            assert torch.equal(getattr(meta, key)[phys], before[key][phys]), (b, p)

    # 3. equal to the oracle's build at the new lengths
    h = W.host_arrays(w)
    c = H.oracle_cache(h)
    spec = H.spec_of(w)
    md = pipeline.build_metadata(c, spec)
    H._compare_meta(w, SimpleNamespace(meta=meta), c, md, h["phys_map"], spec)


def test_append_sequence_of_single_tokens_matches_one_build(dev):
    """Twenty decode steps of one token each, from lengths that cross page boundaries."""
    H.log("[append] 20 single-token steps")
    w = W.make("gqa32k", device=dev, B=2, lens=[1000, 45])
    final = [int(x) for x in w.lens]
    cache = skv.PagedCache(w.k, w.v, w.block_table, w.seq_lens, w.Hq)
    lens = [L - 20 for L in final]
    w.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    meta = skv.build_page_meta(cache, ("box", "gauss"))
    for _ in range(20):
        lens = [L + 1 for L in lens]
        w.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        skv.append_page_meta(cache, meta, 1)
    ref = skv.build_page_meta(cache, ("box", "gauss"))
    torch.cuda.synchronize()
    for phys in _used_pages(w, final):
        assert torch.equal(meta.box[phys], ref.box[phys]) and torch.equal(meta.gauss[phys], ref.gauss[phys]), phys

"""skv_sparse_decode_attn_noalloc (the attention for callers that cannot allocate: its workspace is
the library's fixed device scratch) against skv_sparse_decode_attn with a caller workspace, through
the C ABI: bit-identical outputs on calls in a row, the later ones with a smaller input and another
plan, so that the scratch's previous contents cannot leak into a result."""
import ctypes
import types

import pytest
import torch

import gpu_harness as H
import sparse_kv_cache_build_amd as skv
import workloads as W

pytestmark = pytest.mark.gpu

CALLS = [
    ("token128k", dict(B=2, L=5000, k=512), 1.0),      # tokens, softmax split partials
    ("gqa32k", dict(B=2, L=3000), 1.5),                # smaller: pages, entmax candidate lists
    ("gqa32k", dict(B=1, lens=[700]), 1.0),            # smaller still: softmax over pages
    ("token128k", dict(B=2, L=5000, k=512), 1.0),      # the first call again, after the others
]


def test_noalloc_attention_equals_the_workspace_entry_point():
    dev = torch.device("cuda:0")
    for name, over, alpha in CALLS:
        H.log(f"[noalloc] {name} {over} alpha={alpha}")
        w = W.make(name, device=dev, **over)
        st = H.gpu_step(w, alphas=(alpha,), fused=True)
        need = skv.workspace_bytes(st.cache, skv._binding.OP_ATTN,
                                   skv.attn_params(st.cache, alpha, None, st.sel.granularity), st.sel.cap)
        assert 0 < need <= skv._binding.NOALLOC_SCRATCH_BYTES, need
        ref = st.outs[alpha]
        out = torch.full_like(ref, float("nan"))
        skv.sparse_decode_attn_noalloc(st.cache, w.q, st.sel, out, alpha=alpha)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (name, over, alpha, float((out - ref).abs().max()))


def test_noalloc_attention_refuses_a_workspace_beyond_its_scratch():
    """An entmax selection whose candidate lists exceed the scratch: SKV_ERR_WORKSPACE, nothing run."""
    w = W.make("long_gauss", device=torch.device("cuda:0"), B=4, L=131072)
    cache = skv.PagedCache(w.k, w.v, w.block_table, w.seq_lens, w.Hq)
    p = skv.select_params("all", tokens=0)
    sel = skv.Selection(cache, p)
    no_scores = types.SimpleNamespace(ref=ctypes.byref(skv._binding.Scores()))   # the all-pages policy reads none
    skv.select_pages(cache, no_scores, None, out=sel)
    need = skv.workspace_bytes(cache, skv._binding.OP_ATTN, skv.attn_params(cache, 1.5), sel.cap)
    assert need > skv._binding.NOALLOC_SCRATCH_BYTES
    out = torch.zeros((w.B, w.Hq, w.d), dtype=torch.float32, device=w.k.device)
    with pytest.raises(skv.SkvError) as e:
        skv.sparse_decode_attn_noalloc(cache, w.q, sel, out, alpha=1.5)
    assert e.value.code == skv._binding.SKV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0

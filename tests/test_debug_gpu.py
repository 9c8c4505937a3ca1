"""SKV_DEBUG=1: host-side checks of the device-side inputs before any launch. Valid inputs give the
same results as without the checks; an out-of-range block-table entry, selection entry or count
returns SKV_ERR_INVALID_ARG from the call that would have used it, with nothing launched. Every
invalid input here still points inside allocated memory, so the kernels would not fault even if a
check let it through."""
import os

import numpy as np
import pytest
import torch

import gpu_harness as H
import sparse_kv_cache_build_amd as skv
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_env():
    old = os.environ.get("SKV_DEBUG")
    os.environ["SKV_DEBUG"] = "1"
    yield
    if old is None:
        del os.environ["SKV_DEBUG"]
    else:
        os.environ["SKV_DEBUG"] = old


def test_debug_checks_accept_valid_inputs(debug_env):
    H.log("[debug] valid inputs")
    for name, over in [("gqa32k", dict(B=2, L=3000)), ("token128k", dict(B=2, L=5000, k=512)),
                       ("long_gauss", dict(B=2, L=6000))]:
        w = W.make(name, device="cuda:0", **over)
        st = H.gpu_step(w, fused=True)
        os.environ["SKV_DEBUG"] = "0"
        ref = H.gpu_step(w, fused=True)
        os.environ["SKV_DEBUG"] = "1"
        assert torch.equal(st.sel.count, ref.sel.count), name
        for a in st.outs:
            assert torch.equal(st.outs[a], ref.outs[a]), (name, a)


def test_debug_checks_refuse_out_of_range_inputs(debug_env):
    H.log("[debug] out-of-range inputs")
    w = W.make("gqa32k", device="cuda:0", B=2, L=3000)
    st = H.gpu_step(w)
    cache, sel = st.cache, st.sel
    # a block-table entry at the last physical page while the cache declares one page fewer
    last = w.Nphys - 1
    p = int(np.nonzero(w.block_table[0, :w.pages(0)].cpu().numpy() != last)[0][0])
    saved = int(w.block_table[0, p])
    w.block_table[0, p] = last
    cache.c.num_phys_pages = w.Nphys - 1
    with pytest.raises(skv.SkvError) as e:
        skv.score_pages(cache, st.meta, w.q, "box", out=st.scores)
    assert e.value.code == skv._binding.SKV_ERR_INVALID_ARG
    with pytest.raises(skv.SkvError) as e:
        skv.build_page_meta(cache, ("box",))
    assert e.value.code == skv._binding.SKV_ERR_INVALID_ARG
    w.block_table[0, p] = saved
    cache.c.num_phys_pages = w.Nphys
    skv.score_pages(cache, st.meta, w.q, "box", out=st.scores)   # valid again
    # a selected page past the sequence, a descending pair, a count above the capacity
    cnt = sel.count.clone()
    idx = sel.idx.clone()
    for mutate in ("past", "order", "count"):
        sel.idx.copy_(idx)
        sel.count.copy_(cnt)
        if mutate == "past":
            sel.idx[1, 0, 0] = w.pages(1)
            sel.idx[1, 0, :int(cnt[1, 0])] = torch.sort(sel.idx[1, 0, :int(cnt[1, 0])]).values
        elif mutate == "order":
            sel.idx[0, 1, 0], sel.idx[0, 1, 1] = idx[0, 1, 1], idx[0, 1, 0]
        else:
            sel.count[1, 1] = sel.cap + 1
        with pytest.raises(skv.SkvError) as e:
            skv.sparse_decode_attn(cache, w.q, sel, alpha=1.0)
        assert e.value.code == skv._binding.SKV_ERR_INVALID_ARG, mutate
    sel.idx.copy_(idx)
    sel.count.copy_(cnt)
    out = skv.sparse_decode_attn(cache, w.q, sel, alpha=1.0)
    torch.cuda.synchronize()
    assert torch.equal(out, st.outs[1.0])

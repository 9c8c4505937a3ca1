"""Timing events of the C ABI, a measurement aid: a caller-owned HIP event pair given to
skv_score_pages (skv_scores.ev_begin / ev_end) or skv_sparse_decode_attn (skv_attn_params) is
recorded on the launch stream right around the scoring kernel proper or the first attention
kernel. The pair must time that one launch, stay within the time of the whole call, and leave the
results bit-identical; calls without events record nothing."""
import numpy as np
import pytest
import torch

import gpu_harness as H
import sparse_kv_cache_build_amd as skv
import workloads as W

pytestmark = pytest.mark.gpu

CASES = {
    "token128k": dict(B=2, L=5000, k=512),
    "gqa32k": dict(B=2, L=3000),
    "long_gauss": dict(B=2, L=6000),
    "pool32k": dict(B=2, lens=[3003, 2998]),
    "socket128k": dict(B=2, lens=[5000, 3001], k=512),
}


def _outputs(sc: skv.ScoreBuffers):
    return [t.cpu().numpy() for t in (sc.key, sc.m, sc.s, sc.shat, sc.cand) if t is not None]


@pytest.mark.parametrize("name", list(CASES))
def test_events_time_each_scorer_launch(name):
    H.log(f"[kernel events score] {name} {CASES[name]}")
    w = W.make(name, device=torch.device("cuda:0"), **CASES[name])
    st = H.gpu_step(w)
    kind, tau = w.cfg["score"], w.cfg.get("lsh_tau")
    before = _outputs(st.scores)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pairs = [skv.event_pair() for _ in range(5)]
    torch.cuda.synchronize()
    a.record()
    for ev in pairs:
        skv.score_pages(st.cache, st.meta, w.q, kind, out=st.scores, temperature=tau, events=ev)
    b.record()
    torch.cuda.synchronize()
    times = [x.elapsed_time(y) for x, y in pairs]
    assert all(t > 0.0 for t in times), times
    assert sum(times) <= a.elapsed_time(b)
    for x, y in zip(before, _outputs(st.scores)):
        assert np.array_equal(x, y, equal_nan=True)


def test_events_of_attention_and_calls_without_events():
    """The attention pair times the first attention kernel; a later call without events leaves a
    pair as it was; results are unchanged."""
    H.log("[kernel events attn] token128k")
    w = W.make("token128k", device=torch.device("cuda:0"), **CASES["token128k"])
    st = H.gpu_step(w)
    ref = st.outs[1.0].clone()
    ev = skv.event_pair()
    torch.cuda.synchronize()
    out = skv.sparse_decode_attn(st.cache, w.q, st.sel, alpha=1.0, events=ev)
    torch.cuda.synchronize()
    t0 = ev[0].elapsed_time(ev[1])
    assert t0 > 0.0 and torch.equal(out, ref)
    for _ in range(3):
        out = skv.sparse_decode_attn(st.cache, w.q, st.sel, alpha=1.0)
        skv.score_pages(st.cache, st.meta, w.q, "proj", out=st.scores)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) == t0
    assert torch.equal(out, ref)

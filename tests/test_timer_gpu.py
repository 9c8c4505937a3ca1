"""The kernel timer of the C ABI (skv_kernel_timer_start/stop), a measurement aid: HIP events the
library records on the launch stream right around each launch of the scoring kernel or the first
attention kernel. It must time every call up to its capacity, stay within the time of the whole
calls, and leave results bit-identical."""
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
def test_kernel_timer_times_each_scorer_launch(name):
    H.log(f"[kernel timer score] {name} {CASES[name]}")
    w = W.make(name, device=torch.device("cuda:0"), **CASES[name])
    st = H.gpu_step(w)
    kind, tau = w.cfg["score"], w.cfg.get("lsh_tau")
    before = _outputs(st.scores)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 5
    with skv.KernelTimer("score", capacity=16) as kt:
        a.record()
        for _ in range(n):
            skv.score_pages(st.cache, st.meta, w.q, kind, out=st.scores, temperature=tau)
        b.record()
        torch.cuda.synchronize()
    assert kt.count == n
    assert 0.0 < kt.total_ms <= a.elapsed_time(b)
    for x, y in zip(before, _outputs(st.scores)):
        assert np.array_equal(x, y, equal_nan=True)


def test_kernel_timer_capacity_and_classes():
    """Launches past the capacity are not timed; the attention class ignores scoring calls and
    times the attention kernel; a second start while running is refused."""
    H.log("[kernel timer attn] token128k")
    w = W.make("token128k", device=torch.device("cuda:0"), **CASES["token128k"])
    st = H.gpu_step(w)
    with skv.KernelTimer("score", capacity=2) as kt:
        for _ in range(4):
            skv.score_pages(st.cache, st.meta, w.q, "proj", out=st.scores)
        with pytest.raises(skv.SkvError):
            skv.KernelTimer("attn").__enter__()
    assert kt.count == 2 and kt.total_ms > 0.0
    ref = st.outs[1.0].clone()
    with skv.KernelTimer("attn", capacity=8) as kt:
        skv.score_pages(st.cache, st.meta, w.q, "proj", out=st.scores)
        for _ in range(3):
            out = skv.sparse_decode_attn(st.cache, w.q, st.sel, alpha=1.0)
        torch.cuda.synchronize()
    assert kt.count == 3 and kt.total_ms > 0.0
    assert torch.equal(out, ref)

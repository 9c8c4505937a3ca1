"""The decode step captured as a HIP graph replays to the same bits as eager launches, replay after
replay, with eager work and synchronisations in between (no memset nodes are recorded)."""
import numpy as np
import pytest
import torch

import bench
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,over", [("gqa32k", dict(B=2, L=3000)), ("token128k", dict(B=2, L=5000, k=512)),
                                       ("ragged", dict(B=4, lens=[100, 4500, 20000, 12345])),
                                       ("long_gauss", dict(B=2, L=6000))])
def test_graph_replays_match_eager(name, over):
    print(f"[graph] {name} {over}", flush=True)
    w = W.make(name, device="cuda:0", **over)
    st = bench.Step(w, W.CONFIGS[name]["alphas"][0])
    st.run()
    torch.cuda.synchronize()
    ref_out = st.attn.out.clone()
    ref_cnt = st.sel.count.clone()
    cnt = ref_cnt.cpu().numpy()
    ref_idx = st.sel.idx.cpu().numpy()
    st.capture()
    for rep in range(3):
        st.attn.out.zero_()
        st.sel.count.zero_()
        st.g_pre.replay()             # the sampled bound of a fused token top-k (empty otherwise)
        st.g_score.replay()
        st.g_rest.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.sel.count, ref_cnt), rep
        idx = st.sel.idx.cpu().numpy()
        for u, n in np.ndenumerate(cnt):
            assert np.array_equal(idx[u][:n], ref_idx[u][:n]), (rep, u)
        assert torch.equal(st.attn.out, ref_out), rep
        st.run()                      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(st.attn.out, ref_out)


def test_kernel_events_are_not_recorded_under_capture():
    """Timing events passed to a call on a capturing stream are not recorded (an event record would
    become part of the graph): the capture succeeds, the events keep their eager timing, and the
    replays match the eager result."""
    print("[graph] kernel events under capture", flush=True)
    import sparse_kv_cache_build_amd as skv
    w = W.make("token128k", device="cuda:0", B=2, L=5000, k=512)
    st = bench.Step(w, 1.0)
    st.run()
    torch.cuda.synchronize()
    ref = st.attn.out.clone()
    ev = skv.event_pair()
    st.events = ev
    st.score()                        # eager: recorded
    torch.cuda.synchronize()
    eager_ms = ev[0].elapsed_time(ev[1])
    assert eager_ms > 0.0
    st.capture()                      # the capture holds the scoring launch, not the records
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) == eager_ms
    for _ in range(2):
        st.attn.out.zero_()
        st.g_pre.replay()
        st.g_score.replay()
        st.g_rest.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.attn.out, ref)
    assert ev[0].elapsed_time(ev[1]) == eager_ms

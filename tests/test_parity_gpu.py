"""GPU parity: libskv (HIP, through the C ABI) against the float64 oracle on the same seeded inputs.

Indices (selected pages / tokens) and box / projected keys and metadata must be bit-exact;
outputs within 2e-3 relative / 1e-3 absolute; the Gaussian threshold within 1e-4 relative,
with decisions that close to the threshold counted as certified near-ties.
Small cases cover every unit and span several tiles with ragged tails; full-size cases run the
launch configuration the benchmark times and check sampled sequences."""
import numpy as np
import pytest
import torch

import gpu_harness as H
import sparse_kv_cache_build_amd as skv
import workloads as W

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny": dict(),
    "gqa32k": dict(B=2, L=3000),
    "long_gauss": dict(B=2, L=6000),
    "token128k": dict(B=2, L=5000, k=512),
    "ragged": dict(B=5, lens=[0, 100, 4500, 20000, 12345]),
    "pool32k": dict(B=2, lens=[3003, 2998]),
    "socket128k": dict(B=2, lens=[5000, 3001], k=512),
}

# Sequences the oracle checks end to end at full size (None: every sequence). ragged: eight seeded
# sequences, the shortest and the longest among them; its selection is checked on all 64 by stage
# parity (test_ragged_full_stage_parity_all_sequences).
FULL_SAMPLE = {"tiny": None, "gqa32k": None, "long_gauss": None, "token128k": [0, 5, 10, 15], "ragged": "seeded8",
               "pool32k": None, "socket128k": [2]}


def ragged_sample(w) -> list:
    order = np.argsort(w.lens)
    rest = [int(x) for x in order[1:-1]]
    pick = np.random.default_rng(1005).choice(len(rest), 6, replace=False)
    return sorted([int(order[0]), int(order[-1])] + [rest[i] for i in pick])


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("name", list(SMALL))
def test_small_parity(dev, name):
    H.log(f"[parity small] {name} {SMALL[name]}")
    w = W.make(name, device=dev, **SMALL[name])
    st = H.gpu_step(w)
    rep = H.check(w, st)
    H.log(f"  units={rep.units} near_ties={rep.near_ties} max_err/tol={rep.max_err:.3f}")


@pytest.mark.parametrize("over", [dict(pool_block=1), dict(pool_block=16), dict(pool_block=2, S=64, k=20),
                                  dict(pool_block=8, dtype="f32", Hq=8, Hkv=2, d=64, k=30)])
def test_pooled_key_block_sizes(dev, over):
    """Sub-blocks of one token (the largest q.k on the page), of the whole page, and in pages of 64
    and a float32 cache with d=64."""
    H.log(f"[parity pool] {over}")
    w = W.make("pool32k", device=dev, **{**SMALL["pool32k"], **over})
    st = H.gpu_step(w)
    H.check(w, st)


@pytest.mark.parametrize("over", [
    dict(lsh_tables=16, lsh_bits=1, lsh_tau=0.2),
    dict(lsh_tables=48, lsh_bits=4, lsh_tau=3.0),
    dict(lsh_tables=32, lsh_bits=8, Hq=8, Hkv=4, lsh_tau=1.0),                # G = 2, 256 buckets
    dict(lsh_tables=64, lsh_bits=6, lsh_tau=0.5),                             # G = 4, 64 tables
    dict(lsh_tables=16, lsh_bits=7, Hq=64, Hkv=8, lsh_tau=0.5),               # G = 8, 16384 masses
    dict(lsh_tables=32, lsh_bits=5, dtype="f32", d=64, Hq=4, Hkv=4, S=64),    # G = 1, float32, page 64
    dict(B=4, lens=[0, 1, 17, 4097], k=100),                                  # empty, single-token, k >= L_b
    dict(lsh_tables=48, lsh_bits=3, S=48, lsh_tau=1.0),                       # pages of 48: cut by the 4096-token blocks
    dict(lsh_tables=16, lsh_bits=4, S=8, Hq=64, Hkv=8, lsh_tau=0.5),          # pages of 8 (513 per block), G = 8
])
def test_soft_lsh_variants(dev, over):
    """Soft-LSH token scores with 16 to 64 tables of 1 to 8 bits, every group size, a float32 cache,
    pages of 8, 48 and 64 tokens and ragged / empty sequences: buckets, norms and keys bit-exact,
    selections exact."""
    H.log(f"[parity lsh] {over}")
    w = W.make("socket128k", device=dev, **{**SMALL["socket128k"], **over})
    st = H.gpu_step(w)
    H.check(w, st)


@pytest.mark.parametrize("name,split", [("gqa32k", 1), ("gqa32k", 3), ("token128k", 7), ("ragged", 1),
                                        ("ragged", 2), ("tiny", 5), ("long_gauss", 1)])
def test_explicit_splits_match_oracle(dev, name, split):
    H.log(f"[parity split] {name} split={split}")
    w = W.make(name, device=dev, **SMALL[name])
    st = H.gpu_step(w, split=split)
    H.check(w, st, check_meta=False)


@pytest.mark.parametrize("name,alphas", [("gqa32k", (1.0, 1.5, 2.0, 1.25)), ("tiny", (1.0, 1.5, 2.0)),
                                         ("ragged", (1.0, 2.0)), ("token128k", (1.0, 1.5))])
def test_alphas_over_selection(dev, name, alphas):
    H.log(f"[parity alphas] {name} {alphas}")
    w = W.make(name, device=dev, **SMALL[name])
    st = H.gpu_step(w, alphas=alphas)
    H.check(w, st, alphas=alphas, check_meta=False)


@pytest.mark.parametrize("name", ["gqa32k", "ragged", "token128k"])
@pytest.mark.parametrize("alpha", [1.0, 1.5, 2.0])
def test_full_cache_comparator(dev, name, alpha):
    """policy 'all' = full-cache decode with the same kernels (the pages' comparator)."""
    H.log(f"[parity full-cache] {name} alpha={alpha}")
    w = W.make(name, device=dev, **SMALL[name])
    w.cfg = dict(w.cfg, policy="all")
    st = H.gpu_step(w, alphas=(alpha,))
    H.check(w, st, alphas=(alpha,), check_meta=False)


@pytest.mark.parametrize("name,over", [("gqa32k", dict(Hq=16, Hkv=8)), ("gqa32k", dict(Hq=64, Hkv=8, d=64)),
                                       ("gqa32k", dict(Hq=8, Hkv=8, d=64, dtype="f32")),
                                       ("gqa32k", dict(Hq=16, Hkv=4, dtype="f32")),
                                       ("gqa32k", dict(Hq=32, Hkv=4, dtype="f32")),
                                       ("long_gauss", dict(Hq=16, Hkv=8)), ("long_gauss", dict(Hq=64, Hkv=8)),
                                       ("long_gauss", dict(Hq=8, Hkv=4, d=64, dtype="f32")),
                                       ("ragged", dict(Hq=16, Hkv=8, alphas=(1.0, 1.5)))])
def test_page_keys_over_groups(dev, name, over):
    """Box and Gaussian page keys, their selections and attention at GQA groups of 1, 2, 4 and 8,
    d = 64 and 128, bf16 and float32 caches."""
    H.log(f"[parity groups] {name} {over}")
    w = W.make(name, device=dev, **{**SMALL[name], **over})
    st = H.gpu_step(w)
    H.check(w, st)


@pytest.mark.parametrize("over", [dict(proj_rank=16, Hq=8, Hkv=8), dict(proj_rank=64, Hq=16, Hkv=8),
                                  dict(proj_rank=32, Hq=64, Hkv=8), dict(proj_rank=64, Hq=64, Hkv=8),
                                  dict(proj_rank=16, Hq=8, Hkv=4, d=64)])
@pytest.mark.parametrize("fused", [True, False])
def test_projected_ranks_and_groups(dev, over, fused):
    """Projected token keys at ranks 16, 32 and 64 and GQA groups of 1, 2 and 8 (d = 128 and 64),
    kept as the fused candidate set or as dense keys."""
    H.log(f"[parity projected] {over} fused={fused}")
    w = W.make("token128k", device=dev, B=2, lens=[9000, 4100], k=512, **over)
    st = H.gpu_step(w, fused=fused)
    if fused:
        assert st.scores.key is None
    H.check(w, st)


@pytest.mark.parametrize("lens", [[600, 700], [2000, 3100]])
@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25])
def test_entmax_many_survivors(dev, lens, alpha):
    """Keys scaled down so that every logit lies within 1 of the maximum (in z' units): the solve
    keeps hundreds (LDS-staged) or thousands (the pair lists walked in global memory) of survivors,
    beyond the ones held in registers."""
    H.log(f"[parity entmax survivors] lens={lens} alpha={alpha}")
    w = W.make("gqa32k", device=dev, B=2, lens=lens)
    w.k.mul_(1e-3)
    w.cfg = dict(w.cfg, policy="all")
    st = H.gpu_step(w, alphas=(alpha,))
    H.check(w, st, alphas=(alpha,), check_meta=False)


@pytest.mark.parametrize("over", [dict(B=2, L=20000, k=512), dict(B=2, L=5000, k=512),
                                  dict(B=3, lens=[0, 9000, 40000], k=2048), dict(B=2, lens=[1500, 30000], k=1000),
                                  dict(B=2, lens=[3000, 7001], k=300, S=8), dict(B=2, lens=[2500, 6000], k=400, S=48),
                                  dict(B=2, lens=[5000, 2100], k=256, S=64)])
def test_fused_token_topk_matches_oracle(dev, over):
    """Projected scoring kept as the candidate set of the top-k (no dense keys) selects the same tokens,
    also for pages of 8 and 48 tokens (block-table entries loaded per row) and 64 (one per lane)."""
    H.log(f"[parity fused token top-k] {over}")
    w = W.make("token128k", device=dev, **over)
    st = H.gpu_step(w, fused=True)
    assert st.scores.key is None
    H.check(w, st)


def test_fused_token_topk_falls_back_when_the_sample_misleads(dev):
    """Keys of every sampled position are zeroed, so the sampled bound admits about half of all
    tokens (more than the candidate buffer holds): the selection must re-score every token and still
    match the oracle."""
    H.log("[parity fused token top-k fallback]")
    L = 20000
    w = W.make("token128k", device=dev, B=2, L=L, k=512)
    run, stride = 2048 // 64, L // 64
    pos = [(s // run) * stride + s % run for s in range(2048)]
    for b in range(w.B):
        for t in pos:
            w.k[int(w.block_table[b, t // w.S]), :, t % w.S, :] = 0
    st = H.gpu_step(w, fused=True)
    H.check(w, st)


def test_fused_token_topk_keeps_tokens_the_estimate_undercounts(dev):
    """The scorer filters with a bf16 estimate of each key plus an error bound. Here the estimate of
    'trap' rows is 0 while their exact key is X/32: P = diag(1 + 2^-10 on channels 0-15,
    1 - 2^-10 on 16-31) and q = 1 on those channels give q~ entries that both round to bf16 1.0,
    and a trap row k = (X x16, -X x16) cancels under the rounded q~ but not under q~ itself.
    Trap keys 8 .. 16 straddle the top-512 threshold (about 11 for the N(0, 1) rows), so a filter
    without its error bound would drop the selected traps."""
    H.log("[parity fused token top-k, cancelling rows]")
    L, R = 20000, 32
    w = W.make("token128k", device=dev, B=2, L=L, k=512)
    P = torch.zeros((R, w.d), dtype=torch.float32)
    P[torch.arange(16), torch.arange(16)] = 1.0 + 2.0 ** -10
    P[torch.arange(16, 32), torch.arange(16, 32)] = 1.0 - 2.0 ** -10
    w.proj = P.to(dev)
    w.q[:, :, :R] = 1.0
    gen = torch.Generator().manual_seed(77)
    xs = torch.tensor([256.0, 320.0, 384.0, 448.0, 512.0])
    traps = {}
    for b in range(w.B):
        pos = torch.randperm(L, generator=gen)[:400]
        xv = xs[torch.randint(0, len(xs), (400,), generator=gen)]
        traps[b] = (pos.numpy(), xv.numpy())
        for t, x in zip(pos.tolist(), xv.tolist()):
            row = w.k[int(w.block_table[b, t // w.S]), :, t % w.S, :]
            row[:, :16] = x
            row[:, 16:R] = -x
    st = H.gpu_step(w, fused=True)
    H.check(w, st)
    idx, cnt = st.sel.idx.cpu().numpy(), st.sel.count.cpu().numpy()
    for b in range(w.B):
        pos, xv = traps[b]
        for g in range(w.Hkv):
            chosen = np.isin(pos, idx[b, g, :cnt[b, g]])
            assert chosen.any() and not chosen.all(), (b, g, int(chosen.sum()))


@pytest.mark.parametrize("over,shrink", [
    (dict(sel_alpha=1.25, delta=0.0, drift_sd=2.0), False),        # tau_hat by quadrature
    (dict(sel_alpha=1.75), False),
    (dict(policy="thresh_box", delta=0.0), True),                  # box bound as the page maximum
    (dict(policy="thresh_box", sel_alpha=1.25, delta=0.0, drift_sd=2.0), True),
    (dict(score="gauss_q", delta=1.5), False),                     # estimated maximum m + s Phi^-1(1 - 1/n)
])
def test_threshold_variants_match_oracle(dev, over, shrink):
    """Variants of the Gaussian-aware threshold: any alpha in (1, 2], the box key in the test,
    the quantile estimate of the page maximum. tau_hat within 1e-4 relative; decisions that close
    to the threshold are certified near-ties; everything else bit-exact. With `shrink` the keys of
    every third page are scaled by 0.05 (bf16), so that the loose box bound still drops pages."""
    H.log(f"[parity threshold variant] {over} shrink={shrink}")
    w = W.make("long_gauss", device=dev, **dict(B=2, L=2500, Hq=8, Hkv=2, **over))
    if shrink:
        for b in range(w.B):
            for p in range(0, w.pages(b), 3):
                ph = int(w.block_table[b, p])
                w.k[ph] = (w.k[ph].float() * 0.05).to(w.k.dtype)
    st = H.gpu_step(w)
    rep = H.check(w, st)
    cnt = st.sel.count.cpu().numpy()
    assert cnt.min() > 0 and cnt.max() < w.pages(0), cnt   # the case selects a proper subset
    H.log(f"  units={rep.units} near_ties={rep.near_ties} max_err/tol={rep.max_err:.3f} counts={cnt.ravel()}")


def test_k_at_least_pages_and_tokens_selects_all(dev):
    H.log("[edge] k >= P_b, k >= L_b")
    w = W.make("gqa32k", device=dev, B=2, lens=[700, 33], k=400)
    st = H.gpu_step(w)
    cnt = st.sel.count.cpu().numpy()
    assert np.array_equal(cnt, np.array([[44] * 8, [3] * 8]))
    H.check(w, st)
    w2 = W.make("token128k", device=dev, B=2, lens=[600, 1500], k=1000)
    st2 = H.gpu_step(w2)
    assert np.array_equal(st2.sel.count.cpu().numpy(), np.array([[600] * 8, [1000] * 8]))
    H.check(w2, st2)


def test_empty_sequence_gives_zero_output_and_no_selection(dev):
    H.log("[edge] empty sequences")
    for name in ("gqa32k", "long_gauss", "token128k", "ragged"):
        w = W.make(name, device=dev, B=2, lens=[0, 37 if name != "ragged" else 130])
        st = H.gpu_step(w)
        assert np.all(st.sel.count.cpu().numpy()[0] == 0), name
        for o in st.outs.values():
            assert torch.all(o[0] == 0).item(), name
        H.check(w, st)


def test_determinism(dev):
    H.log("[determinism] gqa32k, ragged")
    for name in ("gqa32k", "ragged", "long_gauss"):
        w = W.make(name, device=dev, **SMALL[name])
        a, b = H.gpu_step(w), H.gpu_step(w)
        assert torch.equal(a.sel.count, b.sel.count)
        cnt = a.sel.count.cpu().numpy()
        ia, ib = a.sel.idx.cpu().numpy(), b.sel.idx.cpu().numpy()
        for u, n in np.ndenumerate(cnt):        # entries past the count are unwritten by contract
            assert np.array_equal(ia[u][:n], ib[u][:n]), (name, u)
        for al in a.outs:
            assert torch.equal(a.outs[al], b.outs[al]), (name, al)


@pytest.mark.parametrize("name", list(FULL_SAMPLE))
def test_full_size_sampled(dev, name):
    H.log(f"[parity full size] {name}")
    w = W.make(name, device=dev)
    st = H.gpu_step(w, fused=True)   # the benchmark's configuration (fused for token top-k)
    seqs = FULL_SAMPLE[name]
    if seqs == "seeded8":
        seqs = ragged_sample(w)
    rep = H.check(w, st, seqs=seqs)
    H.log(f"  sampled seqs={seqs} units={rep.units} near_ties={rep.near_ties} max_err/tol={rep.max_err:.3f}")
    del st, w
    torch.cuda.empty_cache()


def test_ragged_full_stage_parity_all_sequences(dev):
    """All 64 sequences of the ragged workload at full size: the oracle's box keys from the GPU's own
    box metadata equal the GPU keys bit for bit, and the oracle's 5 % budget selection over them
    equals the GPU's selection (the end-to-end check from raw inputs covers eight sequences)."""
    H.log("[stage parity] ragged, all 64 sequences")
    w = W.make("ragged", device=dev)
    st = H.gpu_step(w)
    n = H.stage_parity_box_budget(w, st, range(w.B), w.cfg["pct"])
    assert n == w.B * w.Hkv
    H.record(dict(workload="ragged", kind="stage parity: box keys and budget selection", seqs=w.B, units=n))
    H.log(f"  units={n}")
    del st, w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,seqs", [("ragged", "seeded8"), ("long_gauss", None), ("gqa32k", None)])
def test_full_size_error_bound(dev, name, seqs):
    """At full size, the GPU's sparse outputs against the oracle's full-cache outputs: within 2 B delta
    ("EntmaxKV" s3), delta the full-cache weight of the tokens the selection leaves out, B the largest
    value norm, plus the output tolerance. Reports the support recall and the largest delta."""
    H.log(f"[error bound full size] {name}")
    w = W.make(name, device=dev)
    st = H.gpu_step(w)
    seqs = ragged_sample(w) if seqs == "seeded8" else list(range(w.B))
    stats = H.full_cache_invariants(w, st, seqs)
    H.record(dict(workload=name, kind="full-cache error bound", seqs=seqs, **stats))
    H.log(f"  {stats}")
    del st, w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,over,k", [
    ("socket128k", dict(B=2, lens=[40000, 9000]), 700),
    ("socket128k", dict(B=3, lens=[40000, 100, 0]), 10000),       # more than LDS holds: the exact fallback
    ("token128k", dict(B=2, lens=[30000, 20001]), 512),
])
def test_dense_token_topk_many_workgroups_equals_one(dev, name, over, k):
    """The token top-k over dense keys with a selection workspace (bound, filtered pass on many
    workgroups, selection among candidates) against the one-workgroup path without it."""
    H.log(f"[dense token top-k] {name} {over} k={k}")
    w = W.make(name, device=dev, **over)
    st = H.gpu_step(w)
    p = skv.select_params("token_topk", k=k, tokens=1)
    many = skv.Selection(st.cache, p)
    assert many.ws.numel() >= skv.workspace_bytes(st.cache, skv._binding.OP_SELECT, p, many.cap) > 256
    one = skv.Selection(st.cache, p)
    one.ws = torch.empty(256, dtype=torch.uint8, device=dev)
    skv.select_pages(st.cache, st.scores, None, out=many)
    skv.select_pages(st.cache, st.scores, None, out=one)
    torch.cuda.synchronize()
    cm, co = many.count.cpu().numpy(), one.count.cpu().numpy()
    assert np.array_equal(cm, co)
    im, io = many.idx.cpu().numpy(), one.idx.cpu().numpy()
    for b in range(w.B):
        for g in range(w.Hkv):
            assert np.array_equal(im[b, g, :cm[b, g]], io[b, g, :co[b, g]]), (b, g)

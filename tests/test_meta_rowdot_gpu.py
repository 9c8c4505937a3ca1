"""GPU parity of the projected keys at the edges of bf16 rounding.

Every key row is 2^e times the unit vector e_0 (a power of two is exact in bf16 from 2^-133 up), so
the float64 dot with a row of P is exactly P[i][0] * 2^e, and kproj[t][i] must equal the oracle's
round-to-nearest-even of that value. The rows of P are chosen to land on ties (1 + 2^-8 lies
halfway between bf16 1 and 1 + 2^-7), one float32 step on either side of a tie, on the carry into
the next binade (2 - 2^-8), and on random values; the exponents e = -133 .. 127 take the products
through bf16's subnormal range, its normal range and past its largest value (infinity).
The whole build (more than 128 tokens: the tiled row-dot kernel) and an append of 100 tokens (one
thread per token and output) are checked against the oracle (``orc_meta_proj``), bit for bit."""
import numpy as np
import pytest
import torch

import gpu_harness as H
import oracle
import sparse_kv_cache_build_amd as skv
import workloads as W

pytestmark = pytest.mark.gpu


def _rows_of_p(r: int, d: int) -> np.ndarray:
    f = np.float32
    u = float(np.finfo(np.float32).eps)   # 2^-23
    base = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + u, 1.0 + 2.0 ** -8 - u,
            2.0 - 2.0 ** -8, 2.0 - 2.0 ** -8 - 2 * u, 1.5 + 2.0 ** -9, 1.0, 0.0,
            1.0 + 5 * 2.0 ** -9, 1.0 + 2.0 ** -9 + u]
    vals = base + [-v for v in base]
    rng = np.random.default_rng(2024)
    vals += list(rng.standard_normal(r - len(vals)) * 3.0)
    P = np.zeros((r, d), dtype=f)
    P[:, 0] = np.array(vals[:r], dtype=f)
    P[:, 1:] = rng.standard_normal((r, d - 1)).astype(f)   # multiplied by zero keys: no effect
    return P


def test_projected_keys_round_like_the_oracle(dev):
    H.log("[parity projected keys, bf16 rounding edges]")
    L = 600
    w = W.make("token128k", device=dev, B=1, L=L, k=64)
    r = w.cfg["proj_rank"]
    P = _rows_of_p(r, w.d)
    w.proj = torch.from_numpy(P).to(dev)
    exps = -133 + (np.arange(L) % 261)   # -133 .. 127
    for t in range(L):
        row = w.k[int(w.block_table[0, t // w.S]), :, t % w.S, :]
        row.zero_()
        row[:, 0] = float(2.0 ** int(exps[t]))
    cache = skv.PagedCache(w.k, w.v, w.block_table, w.seq_lens, w.Hq)

    def oracle_kproj():
        c = H.oracle_cache(W.host_arrays(w))
        return oracle.meta_proj(c, P)

    ref = oracle_kproj()
    used = sorted({int(w.block_table[0, p]) for p in range((L + w.S - 1) // w.S)})
    meta = skv.build_page_meta(cache, ("proj",), proj=w.proj)
    got = meta.kproj.cpu().numpy().view(np.uint16)
    for ph in used:
        assert np.array_equal(got[ph], ref[ph]), f"build: page {ph}"
    # an append of 100 tokens with new key values (e shifted by 7) must agree again
    n_new = 100
    w.seq_lens.fill_(L - n_new)
    for t in range(L - n_new, L):
        row = w.k[int(w.block_table[0, t // w.S]), :, t % w.S, :]
        row[:, 0] = float(2.0 ** int(-133 + (exps[t] + 133 + 7) % 261))
    w.seq_lens.fill_(L)
    skv.append_page_meta(cache, meta, n_new)
    ref = oracle_kproj()
    got = meta.kproj.cpu().numpy().view(np.uint16)
    for ph in used:
        assert np.array_equal(got[ph], ref[ph]), f"append: page {ph}"


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")

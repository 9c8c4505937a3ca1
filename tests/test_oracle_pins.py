"""Pins of the float64 oracle against what the pages and mathematics fix (no GPU needed).

Each pin checks the oracle against something other than itself: worked examples
(tests/golden), independent library routines the oracle does not use (numpy sorting and
reductions, scipy quadrature and optimisation, torch's bf16 cast), closed forms, invariants the
pages state (EntmaxKV summary s2.A box upper bound, s2.C / s3 support recovery and the
2 B delta error bound), special cases that reduce to a textbook result, and brute force.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.special
import torch

import oracle
from oracle import pipeline
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _f32_cache(rng, B=2, Hq=4, Hkv=2, d=16, S=8, lens=(37, 64), bf16=False):
    """A small random cache with a permuted block table (host arrays only)."""
    maxP = max((L + S - 1) // S for L in lens)
    pages = [(L + S - 1) // S for L in lens]
    Nphys = sum(pages)
    perm = rng.permutation(Nphys).astype(np.int32)
    bt = np.zeros((B, maxP), np.int32)
    off = 0
    for b, P in enumerate(pages):
        bt[b, :P] = perm[off:off + P]
        off += P
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    k = rng.standard_normal((Nphys, Hkv, S, d)).astype(np.float32)
    v = rng.standard_normal((Nphys, Hkv, S, d)).astype(np.float32)
    if bf16:
        q, k, v = (torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                   for a in (q, k, v))
    return oracle.Cache(q=q, k=k, v=v, block_table=bt, seq_lens=np.array(lens, np.int32))


def _dec(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _rows(c, b, g, arr):
    """[L, d] float64 rows of sequence b, KV head g, gathered with numpy (independent of the oracle)."""
    L = c.length(b)
    t = np.arange(L)
    phys = c.block_table[b, t // c.S]
    return _dec(arr)[phys, g, t % c.S]


# ---------------------------------------------------------------- bf16 rounding

def test_round_bf16_golden(orc):
    cases = json.load(open(os.path.join(GOLD, "bf16_rounding.json")))["cases"]
    for cse in cases:
        assert orc.round_bf16(cse["x"]) == int(cse["bits"], 16), cse


def test_round_bf16_matches_torch_cast_on_float32_inputs(orc):
    # float32 inputs are exact doubles, so torch's single rounding f32 -> bf16 is the reference
    rng = _rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(2000) * 1e-39]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.round_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- metadata

def test_meta_box_bounds_every_key_and_is_attained(orc):
    c = _f32_cache(_rng(2), bf16=True)
    kmin, kmax = orc.meta_box(c)
    for b in range(c.B):
        for p in range(c.pages(b)):
            phys, n = c.block_table[b, p], c.page_tokens(b, p)
            for g in range(c.Hkv):
                keys = _dec(c.k)[phys, g, :n]
                assert np.array_equal(kmin[phys, g], keys.min(0))
                assert np.array_equal(kmax[phys, g], keys.max(0))


def test_meta_gauss_matches_numpy_moments(orc):
    c = _f32_cache(_rng(3))
    mean, var = orc.meta_gauss(c)
    for b in range(c.B):
        for p in range(c.pages(b)):
            phys, n = c.block_table[b, p], c.page_tokens(b, p)
            keys = _dec(c.k)[phys, :, :n]            # [Hkv, n, d]
            np.testing.assert_allclose(mean[phys], keys.mean(1), rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(var[phys], keys.var(1), rtol=1e-12, atol=1e-14)


def test_meta_proj_identity_and_permutation_are_exact(orc):
    # P = I (r = d) keeps bf16 keys exactly; P = rows of a permutation picks coordinates exactly
    c = _f32_cache(_rng(4), bf16=True)
    kp = orc.meta_proj(c, np.eye(c.d, dtype=np.float32))
    perm = _rng(5).permutation(c.d)[:6]
    kq = orc.meta_proj(c, np.eye(c.d, dtype=np.float32)[perm])
    for b in range(c.B):
        for p in range(c.pages(b)):
            phys, n = c.block_table[b, p], c.page_tokens(b, p)
            assert np.array_equal(kp[phys, :, :n], c.k[phys, :, :n])
            assert np.array_equal(kq[phys, :, :n], c.k[phys, :, :n][..., perm])


def test_meta_proj_rounds_float64_sum_to_nearest_bf16(orc):
    # one token, P with two rows: [1, 2^-9] picks k0 + k1 / 512, rounded once (no f32 detour)
    q = np.zeros((1, 1, 2), np.float32)
    k = np.array([1.0, 1.0 + 2 ** -7], np.float32).reshape(1, 1, 1, 2)
    c = oracle.Cache(q=q, k=k, v=k.copy(), block_table=np.zeros((1, 1), np.int32),
                     seq_lens=np.array([1], np.int32))
    P = np.array([[1.0, 2.0 ** -9], [2.0 ** -9, 1.0]], np.float32)
    got = orc.meta_proj(c, P)[0, 0, 0]
    # row 0: 1 + (1 + 2^-7) 2^-9 = 1 + 2^-9 + 2^-16 -> below the midpoint 1 + 2^-8 -> 1.0
    # row 1: 2^-9 + 1 + 2^-7 -> between 1+2^-7 and 1+2^-6, above 1+2^-7 by 2^-9 -> 1+2^-7
    assert got[0] == 0x3f80 and got[1] == 0x3f81


def test_meta_proj_rounds_once_not_through_float32(orc):
    # P row [1, 2^-8] on k = (1, 1 + 2^-22): the float64 sum 1 + 2^-8 + 2^-30 lies just above the
    # midpoint between bf16 1.0 and 1 + 2^-7, so one rounding gives 1 + 2^-7 (0x3f81); through
    # float32 first it would become the tie 1 + 2^-8 and then 1.0 (0x3f80)
    q = np.zeros((1, 1, 2), np.float32)
    k = np.array([1.0, 1.0 + 2 ** -22], np.float32).reshape(1, 1, 1, 2)
    c = oracle.Cache(q=q, k=k, v=k.copy(), block_table=np.zeros((1, 1), np.int32),
                     seq_lens=np.array([1], np.int32))
    P = np.array([[1.0, 2.0 ** -8], [-1.0, -(2.0 ** -8)]], np.float32)
    got = orc.meta_proj(c, P)[0, 0, 0]
    assert got[0] == 0x3f81 and got[1] == 0xbf81


# ---------------------------------------------------------------- scores

def test_score_box_is_upper_bound_of_true_max_and_tight_for_single_tokens(orc):
    c = _f32_cache(_rng(6), S=4, lens=(33, 20))       # ragged tails: pages with 1 token exist
    kmin, kmax = orc.meta_box(c)
    key = orc.score_box(c, kmin, kmax)
    q = _dec(c.q)
    for b in range(c.B):
        for g in range(c.Hkv):
            rows = _rows(c, b, g, c.k)
            for p in range(c.maxP):
                if p >= c.pages(b):
                    assert key[b, g, p] == -np.inf
                    continue
                toks = rows[p * c.S: p * c.S + c.page_tokens(b, p)]
                true_max = max((q[b, h] @ toks.T).max() for h in range(g * c.G, (g + 1) * c.G))
                assert key[b, g, p] >= np.float32(true_max) - 1e-5 * max(1, abs(true_max))
                if len(toks) == 1:
                    assert abs(key[b, g, p] - true_max) <= 1e-6 * max(1, abs(true_max))


def test_score_box_one_hot_query_is_exact(orc):
    # q = +2 e_j (head 0) and -3 e_j' (head 1): U = 2 kmax_j and -3 kmin_j'; the key is their max
    rng = _rng(7)
    c0 = _f32_cache(rng, B=1, Hq=2, Hkv=1, lens=(40,))
    q = np.zeros_like(c0.q)
    q[0, 0, 3], q[0, 1, 5] = 2.0, -3.0
    c = oracle.Cache(q=q, k=c0.k, v=c0.v, block_table=c0.block_table, seq_lens=c0.seq_lens)
    kmin, kmax = orc.meta_box(c)
    key = orc.score_box(c, kmin, kmax)
    for p in range(c.pages(0)):
        phys = c.block_table[0, p]
        want = max(2.0 * kmax[phys, 0, 3], -3.0 * kmin[phys, 0, 5])
        assert key[0, 0, p] == np.float32(want)


def test_score_gauss_mean_is_mean_of_true_scores(orc):
    # linearity: the page mean of scale * q.k_t equals scale * q.mu exactly (up to rounding)
    c = _f32_cache(_rng(8))
    mean, var = orc.meta_gauss(c)
    scale = 1 / math.sqrt(c.d)
    m, s, shat = orc.score_gauss(c, mean, var, scale)
    q = _dec(c.q)
    for b in range(c.B):
        for h in range(c.Hq):
            rows = _rows(c, b, h // c.G, c.k)
            for p in range(c.pages(b)):
                z = scale * rows[p * c.S: p * c.S + c.page_tokens(b, p)] @ q[b, h]
                assert abs(m[b, h, p] - z.mean()) <= 1e-12 * (1 + abs(z).max())
                n = c.page_tokens(b, p)
                assert shat[b, h, p] == pytest.approx(m[b, h, p] + s[b, h, p] * math.sqrt(2 * math.log(n)),
                                                       rel=1e-14, abs=1e-14)


def test_score_gauss_sd_is_sd_of_true_scores_for_uncorrelated_coordinates(orc):
    # With pages whose coordinates are empirically uncorrelated (columns of a Hadamard matrix),
    # the diagonal model is exact: s^2 = var_t(scale * q.k_t).
    S, d = 16, 8
    H = np.array([[1]])
    while H.shape[0] < S:
        H = np.block([[H, H], [H, -H]])
    rng = _rng(9)
    amp = rng.uniform(0.5, 2.0, d)
    mu = rng.standard_normal(d)
    k = (mu + H[:, 1:d + 1] * amp).astype(np.float32).reshape(1, 1, S, d)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    c = oracle.Cache(q=q, k=k, v=k.copy(), block_table=np.zeros((1, 1), np.int32),
                     seq_lens=np.array([S], np.int32))
    mean, var = orc.meta_gauss(c)
    m, s, _ = orc.score_gauss(c, mean, var, 0.5)
    z = 0.5 * (k[0, 0].astype(np.float64) @ q[0, 0].astype(np.float64))
    assert m[0, 0, 0] == pytest.approx(z.mean(), rel=1e-12, abs=1e-12)
    assert s[0, 0, 0] == pytest.approx(z.std(), rel=1e-12)


def test_gauss_max_estimate_bounds_expected_page_max(orc):
    # reading of the "estimated maximum": shat = m + s sqrt(2 ln n) >= E[max of n Gaussians]
    rng = _rng(10)
    for n in (2, 16, 32, 64):
        draws = rng.standard_normal((20000, n)).max(1).mean()
        assert draws <= math.sqrt(2 * math.log(n))


def test_gauss_max_factor_of_the_oracle_is_the_chernoff_bound_on_the_expected_maximum(orc):
    """The oracle's estimated page maximum, read back as the factor f = (shat - m) / s of pages
    holding n = 1 .. 64 valid tokens, against what fixes it without its formula:
      - the moment-generating-function bound on the expected maximum of n standard normals,
        E[max] <= min over lam > 0 of (ln n) / lam + lam / 2, minimised numerically by scipy;
      - Monte Carlo: f lies above the mean maximum of n draws (it bounds it) and by less than
        0.65 (the bound's slack for n <= 64; sqrt(ln n) falls below the mean, sqrt(2 log2 n)
        and 2 ln n above the slack);
      - n = 1: shat = m.
    A page's valid-token count, not the page size, is n (partial last pages)."""
    import scipy.optimize
    rng = _rng(31)
    S, d = 64, 16
    lens = (64 * 3 + 1, 64 * 2 + 2, 64 + 3, 5, 16, 33, 64 + 17)
    c = _f32_cache(rng, B=len(lens), Hq=2, Hkv=1, d=d, S=S, lens=lens)
    mean, var = orc.meta_gauss(c)
    m, s, shat = orc.score_gauss(c, mean, var, 0.3)
    seen = {}
    for b in range(c.B):
        for p in range(c.pages(b)):
            n = c.page_tokens(b, p)
            for h in range(c.Hq):
                if n == 1:
                    assert shat[b, h, p] == m[b, h, p]
                else:
                    assert s[b, h, p] > 0
                    seen.setdefault(n, []).append((shat[b, h, p] - m[b, h, p]) / s[b, h, p])
    assert {2, 3, 5, 16, 17, 33, 64} <= set(seen)
    for n, fs in seen.items():
        f = fs[0]
        assert np.allclose(fs, f, rtol=1e-12, atol=0)
        res = scipy.optimize.minimize_scalar(lambda lam: math.log(n) / lam + lam / 2, bounds=(1e-3, 50.0),
                                             method="bounded", options=dict(xatol=1e-12))
        assert f == pytest.approx(res.fun, rel=1e-6), (n, f, res.fun)
        mc = rng.standard_normal((200000, n)).max(1).mean()
        assert mc - 0.01 <= f <= mc + 0.65, (n, f, mc)


def _seq_dot(a, b):
    """float64 dot product summed in index order (the oracle's order)."""
    return np.cumsum(a * b, axis=-1)[..., -1]


@pytest.mark.parametrize("bf16", [True, False])
def test_pool_single_token_blocks_give_exact_page_max(orc, bf16):
    # sub-blocks of one token: the pooled key is the exact maximum score of the page's tokens
    c = _f32_cache(_rng(41), B=2, Hq=4, Hkv=2, d=16, S=8, lens=(37, 21), bf16=bf16)
    pool = orc.meta_pool(c, 1)
    key = orc.score_pool(c, 1, pool)
    q = _dec(c.q)
    for b, L in enumerate((37, 21)):
        for g in range(2):
            rows = _rows(c, b, g, c.k)                       # [L, d] in token order
            for p in range(c.pages(b)):
                t = np.arange(p * c.S, min(L, (p + 1) * c.S))
                u = _seq_dot(rows[t][:, None, :], q[b, 2 * g:2 * g + 2][None, :, :])
                assert key[b, g, p] == np.float32(u.max()), (b, g, p)
            assert np.all(key[b, g, c.pages(b):] == -np.inf)


def test_pool_means_are_float32_of_float64_means_and_partial_blocks_count_valid_tokens(orc):
    c = _f32_cache(_rng(42), B=1, Hq=2, Hkv=1, d=16, S=8, lens=(29,), bf16=True)
    pb = 4
    pool = orc.meta_pool(c, pb)
    rows = _rows(c, 0, 0, c.k)
    for p in range(c.pages(0)):
        ph = c.block_table[0, p]
        for sb in range(c.S // pb):
            t = np.arange(p * c.S + sb * pb, min(29, p * c.S + sb * pb + pb))
            if len(t) == 0:
                assert np.all(np.isnan(pool[ph, 0, sb])), (p, sb)   # no valid token: not written
                continue
            want = (np.cumsum(rows[t], axis=0)[-1] / len(t)).astype(np.float32)
            assert np.array_equal(pool[ph, 0, sb], want), (p, sb)


def test_pool_key_is_max_over_blocks_of_mean_scores(orc):
    # pooling keys = pooling scores (linearity), up to the float32 rounding of the means
    c = _f32_cache(_rng(43), B=1, Hq=4, Hkv=1, d=16, S=8, lens=(40,), bf16=True)
    pb = 2
    key = orc.score_pool(c, pb, orc.meta_pool(c, pb))
    q, rows = _dec(c.q)[0], _rows(c, 0, 0, c.k)
    z = rows @ q.T                                           # [40, 4] exact scores
    for p in range(c.pages(0)):
        blocks = z[p * 8:(p + 1) * 8].reshape(4, 2, 4).mean(axis=1)
        assert key[0, 0, p] == pytest.approx(blocks.max(), rel=1e-6, abs=1e-6)
    whole = orc.score_pool(c, 8, orc.meta_pool(c, 8))       # one block per page: q . mean key
    for p in range(c.pages(0)):
        assert whole[0, 0, p] == pytest.approx(z[p * 8:(p + 1) * 8].mean(axis=0).max(), rel=1e-6, abs=1e-6)


def test_score_proj_identity_projection_ranks_exact_scores(orc):
    c = _f32_cache(_rng(11), B=1, Hq=4, Hkv=1, d=16, S=8, lens=(61,), bf16=True)
    P = np.eye(c.d, dtype=np.float32)
    key = orc.score_proj(c, P, orc.meta_proj(c, P))
    q = _dec(c.q)
    rows = _rows(c, 0, 0, c.k)
    exact = np.max(rows @ q[0].T, axis=1)          # bf16 x bf16 products: exact in float64
    assert np.array_equal(key[0, 0, :61], exact.astype(np.float32))
    assert np.all(key[0, 0, 61:] == -np.inf)
    top = orc.select_topk(key[0, 0, :61], 10)
    assert np.array_equal(top, np.sort(np.lexsort((np.arange(61), -exact))[:10]))


def test_score_proj_permutation_projection_scores_partial_dot(orc):
    c = _f32_cache(_rng(12), B=1, Hq=2, Hkv=1, d=16, S=8, lens=(30,), bf16=True)
    sel = np.array([3, 7, 1, 12])
    P = np.eye(c.d, dtype=np.float32)[sel]
    key = orc.score_proj(c, P, orc.meta_proj(c, P))
    q = _dec(c.q)
    rows = _rows(c, 0, 0, c.k)
    want = np.max(rows[:, sel] @ q[0][:, sel].T, axis=1)
    assert np.array_equal(key[0, 0, :30], want.astype(np.float32))


# ---------------------------------------------------------------- selection

def test_select_topk_matches_lexsort_with_ties_to_lower_index(orc):
    rng = _rng(13)
    for trial in range(50):
        n = int(rng.integers(1, 400))
        key = rng.integers(-5, 5, n).astype(np.float32) * 0.5     # many exact ties
        k = int(rng.integers(1, n + 5))
        want = np.sort(np.lexsort((np.arange(n), -key))[:min(k, n)])
        assert np.array_equal(orc.select_topk(key, k), want)


def test_select_topk_k_at_least_n_takes_all_and_handles_signed_zero(orc):
    key = np.array([0.0, -0.0, 1.0, -np.inf], np.float32)
    assert np.array_equal(orc.select_topk(key, 10), [0, 1, 2, 3])
    assert np.array_equal(orc.select_topk(key, 2), [0, 2])   # -0 == +0: the lower index wins


def test_budget_rounds_up_percent_of_pages(orc):
    assert [orc.budget_k(P, 5) for P in (0, 1, 19, 20, 21, 128, 4096)] == [0, 1, 1, 1, 2, 7, 205]


# ---------------------------------------------------------------- Gaussian threshold

@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_gauss_partial_moment_closed_form_matches_quadrature(orc, alpha):
    rng = _rng(14)
    for _ in range(40):
        mu, sd, tau = rng.normal(0, 2), rng.uniform(0.05, 3), rng.normal(0, 2)
        f = lambda x: (x - tau) ** (1 / (alpha - 1)) * math.exp(-0.5 * ((x - mu) / sd) ** 2) / (sd * math.sqrt(2 * math.pi))
        ref, err = scipy.integrate.quad(f, tau, mu + 40 * sd, epsabs=1e-14, epsrel=1e-13)
        got = orc.gauss_partial_moment(mu, sd, tau, alpha)
        assert got == pytest.approx(ref, rel=1e-9, abs=1e-12)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_tau_hat_degenerate_pages_equal_exact_entmax_threshold(orc, alpha):
    # pages of identical tokens have s = 0: the normalization equation becomes the exact
    # entmax normalization over n_p copies of m_p, so tau_hat must equal the exact threshold
    rng = _rng(15)
    for _ in range(10):
        P = int(rng.integers(1, 60))
        m = rng.normal(0, 2, P)
        n = rng.integers(1, 33, P).astype(np.int32)
        tau = orc.tau_hat(m, np.zeros(P), n, alpha)
        z = np.repeat(m, n)
        _, tau_exact = orc.entmax(z, alpha)
        assert tau == pytest.approx(tau_exact, abs=1e-9)


def test_tau_hat_brackets_root_of_monotone_equation(orc):
    rng = _rng(16)
    alpha = 1.5
    for _ in range(10):
        P = 200
        m, s = rng.normal(0, 1, P), rng.uniform(0.1, 2, P)
        n = np.full(P, 32, np.int32)
        tau = orc.tau_hat(m, s, n, alpha)
        F = lambda t: sum(nn * orc.gauss_partial_moment(0.5 * mm, 0.5 * ss, t, alpha)
                          for mm, ss, nn in zip(m, s, n)) - 1
        assert abs(F(tau)) < 1e-8
        assert F(tau - 1e-3) > 0 > F(tau + 1e-3)
        assert tau >= 0.5 * m.max() - 1


def _phi(a):
    return math.exp(-0.5 * a * a) / math.sqrt(2 * math.pi)


def _Phi(a):
    return 0.5 * scipy.special.erfc(-a / math.sqrt(2))


@pytest.mark.parametrize("a", [-6.0, -3.5, -0.7, 0.0, 0.4, 2.0, 9.0, 35.0])
def test_truncated_power_moment_matches_closed_forms_at_integer_powers(orc, a):
    # E[(Z + a)_+^k] for integer k: k = 1, 2, 3 reduce to Phi and phi (scipy's erfc here); below
    # a = -6 the closed forms cancel catastrophically, and the quadrature is pinned by scipy instead
    closed = {1: a * _Phi(a) + _phi(a),
              2: (a * a + 1) * _Phi(a) + a * _phi(a),
              3: (a ** 3 + 3 * a) * _Phi(a) + (a * a + 2) * _phi(a)}
    for k, want in closed.items():
        assert orc.trunc_power_moment(a, k) == pytest.approx(want, rel=1e-10, abs=1e-300)


@pytest.mark.parametrize("k", [1.25, 1.6, 2.5, 4.0, 10.0])
def test_truncated_power_moment_matches_scipy_quad(orc, k):
    for a in (-12.0, -6.0, -1.3, 0.0, 0.8, 3.0, 12.0):
        f = lambda u: u ** k * _phi(u - a)
        ref, _ = scipy.integrate.quad(f, 0.0, max(a, 0.0) + 40.0, epsabs=1e-300, epsrel=1e-12, limit=400,
                                      points=[max(a, 0.0)])
        assert orc.trunc_power_moment(a, k) == pytest.approx(ref, rel=1e-9, abs=1e-300)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_general_alpha_moment_reproduces_closed_forms(orc, alpha):
    rng = _rng(31)
    for _ in range(30):
        mu, sd, tau = rng.normal(0, 2), rng.uniform(0.05, 3), rng.normal(0, 2)
        assert orc.gauss_partial_moment_quad(mu, sd, tau, alpha) == pytest.approx(
            orc.gauss_partial_moment(mu, sd, tau, alpha), rel=1e-10, abs=1e-14)
    assert orc.gauss_partial_moment_quad(2.0, 0.0, 0.5, 1.25) == pytest.approx(1.5 ** 4, rel=1e-15)   # point mass
    assert orc.gauss_partial_moment_quad(0.2, 0.0, 0.5, 1.25) == 0.0


@pytest.mark.parametrize("alpha", [1.25, 1.75])
def test_tau_hat_general_alpha_degenerate_pages_equal_exact_entmax_threshold(orc, alpha):
    # s = 0 turns the normalization equation into the exact entmax normalization over n_p copies
    # of m_p; the oracle's entmax for these alpha is its own bisection on the logits
    rng = _rng(32)
    for _ in range(6):
        P = int(rng.integers(1, 30))
        m = rng.normal(0, 2, P)
        n = rng.integers(1, 17, P).astype(np.int32)
        tau = orc.tau_hat(m, np.zeros(P), n, alpha)
        _, tau_exact = orc.entmax(np.repeat(m, n), alpha)
        assert tau == pytest.approx(tau_exact, abs=1e-9)


@pytest.mark.parametrize("alpha", [1.25, 1.8])
def test_tau_hat_general_alpha_is_root_of_equation_by_scipy(orc, alpha):
    rng = _rng(33)
    P = 12
    m, s = rng.normal(0, 1, P), rng.uniform(0.1, 1.5, P)
    n = np.full(P, 16, np.int32)
    tau = orc.tau_hat(m, s, n, alpha)
    k = 1.0 / (alpha - 1.0)

    def F(t):
        tot = -1.0
        for mm, ss, nn in zip(m, s, n):
            mu, sd = (alpha - 1) * mm, (alpha - 1) * ss
            f = lambda x: (x - t) ** k * _phi((x - mu) / sd) / sd
            v, _ = scipy.integrate.quad(f, t, max(t, mu) + 40 * sd, epsabs=1e-300, epsrel=1e-11, limit=200)
            tot += nn * v
        return tot
    assert abs(F(tau)) < 1e-7
    assert F(tau - 1e-3) > 0 > F(tau + 1e-3)


def test_phi_inverse_matches_scipy_ppf_and_isf(orc):
    import scipy.stats
    for p in (1e-12, 0.01, 0.25, 0.5, 0.75, 15 / 16, 31 / 32, 63 / 64):
        assert orc.Phi_inv(p) == pytest.approx(scipy.stats.norm.ppf(p), rel=1e-12, abs=1e-12)
    for n in (2, 3, 16, 64, 1024, 10 ** 9):
        assert orc.Phi_inv_upper(1 / n) == pytest.approx(scipy.stats.norm.isf(1 / n), rel=1e-12, abs=1e-12)


def test_score_gauss_quantile_max_uses_phi_inverse(orc):
    c = _f32_cache(_rng(34), B=1, Hq=2, Hkv=1, d=16, S=8, lens=(29,))
    mean, var = orc.meta_gauss(c)
    m, s, shat = orc.score_gauss(c, mean, var, 0.25)
    mq, sq, shatq = orc.score_gauss(c, mean, var, 0.25, quantile=True)
    assert np.array_equal(m, mq) and np.array_equal(s, sq)
    import scipy.stats
    for p in range(c.pages(0)):
        n = c.page_tokens(0, p)
        fac = scipy.stats.norm.isf(1 / n) if n > 1 else 0.0
        assert shatq[0, :, p] == pytest.approx(m[0, :, p] + s[0, :, p] * fac, rel=1e-12, abs=1e-12)
        assert shat[0, :, p] == pytest.approx(m[0, :, p] + s[0, :, p] * math.sqrt(2 * math.log(n)), rel=1e-12,
                                              abs=1e-12)


def test_select_thresh_box_is_the_box_test_and_covers_the_per_head_test(orc):
    # brute force: keep iff (alpha-1) scale key > min tau - delta, key = max over the group's heads of
    # the unscaled box bound; every page that some head's own bound would keep is kept
    c = _f32_cache(_rng(35), B=1, Hq=4, Hkv=1, d=16, S=8, lens=(200,))
    kmin, kmax = orc.meta_box(c)
    key = orc.score_box(c, kmin, kmax)[0, 0, :c.pages(0)].astype(np.float64)
    q = _dec(c.q)[0]
    U = np.zeros((4, c.pages(0)))
    for p in range(c.pages(0)):
        lo, hi = kmin[c.block_table[0, p], 0].astype(np.float64), kmax[c.block_table[0, p], 0].astype(np.float64)
        U[:, p] = np.maximum(q * lo, q * hi).sum(1)
    scale, alpha, delta = 0.25, 1.5, 0.1
    v = (alpha - 1) * scale * key
    lo_v, hi_v = np.quantile(v, [0.2, 0.8])
    taus = np.array([lo_v, hi_v, 0.5 * (lo_v + hi_v), hi_v + 0.1]) + delta   # cuts inside the keys' spread
    got = orc.select_thresh_box(key, taus, scale, alpha, delta)
    want = np.nonzero(v > taus.min() - delta)[0]
    assert np.array_equal(got, want)
    assert 0 < len(got) < c.pages(0)
    assert len(got) > len(np.nonzero(v > taus.max() - delta)[0])   # the lowest threshold decides
    per_head = np.nonzero(((alpha - 1) * scale * U > (taus - delta)[:, None]).any(0))[0]
    assert set(per_head) <= set(got)
    assert np.allclose(key, U.max(0), rtol=1e-6)


def test_select_thresh_keeps_iff_some_head_clears_threshold(orc):
    shat = np.array([[0.0, 3.0, 1.0, 2.0], [2.5, 0.0, 0.0, 0.5]])
    tau = np.array([1.2, 1.0])
    # keep iff 0.5 * shat > tau - 0.5: head0 needs shat > 1.4 (pages 1, 3); head1 needs > 1.0 (page 0)
    assert np.array_equal(orc.select_thresh(shat, tau, 1.5, 0.5), [0, 1, 3])
    # equality is not enough (strict >): head0 page 3 has 0.5 * 2.0 = 1.0 = 1.5 - 0.5
    assert np.array_equal(orc.select_thresh(shat[:1], np.array([1.5]), 1.5, 0.5), [1])


# ---------------------------------------------------------------- entmax

def test_entmax_golden_examples(orc):
    for cse in json.load(open(os.path.join(GOLD, "entmax_worked.json")))["cases"]:
        p, tau = orc.entmax(np.array(cse["z"]), cse["alpha"])
        np.testing.assert_allclose(p, cse["p"], rtol=0, atol=1e-15)
        assert tau == pytest.approx(cse["tau"], abs=1e-15)


def test_sparsemax_is_euclidean_projection_onto_simplex(orc):
    # sparsemax(z) = argmin_{p in simplex} |p - z|^2 ; checked by its KKT conditions and by
    # scipy's SLSQP on small inputs
    import scipy.optimize
    rng = _rng(17)
    for _ in range(20):
        n = int(rng.integers(2, 12))
        z = rng.normal(0, 1.5, n)
        p, tau = orc.sparsemax(z)
        res = scipy.optimize.minimize(lambda x: ((x - z) ** 2).sum(), np.full(n, 1 / n), method="SLSQP",
                                      bounds=[(0, 1)] * n,
                                      constraints=[{"type": "eq", "fun": lambda x: x.sum() - 1}],
                                      options=dict(ftol=1e-14, maxiter=500))
        np.testing.assert_allclose(p, res.x, atol=1e-6)
        on = p > 0
        np.testing.assert_allclose(p[on], z[on] - tau, atol=1e-14)
        assert np.all(z[~on] <= tau + 1e-14)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_sort_based_entmax_equals_bisection(orc, alpha):
    rng = _rng(18)
    for n in (1, 2, 7, 100, 5000):
        z = rng.normal(0, 3, n)
        p_sort, t_sort = orc.entmax(z, alpha)
        p_bis, t_bis = orc.entmax_bisect(z, alpha)
        np.testing.assert_allclose(p_sort, p_bis, atol=1e-12)
        assert t_sort == pytest.approx(t_bis, abs=1e-12)


def test_entmax15_is_tsallis_regularised_argmax(orc):
    # 1.5-entmax = argmax_p <p, z> + H(p), H(p) = (1 - sum p^1.5) / (alpha (alpha - 1)) = 4/3 (1 - sum p^1.5)
    import scipy.optimize
    rng = _rng(19)
    for _ in range(10):
        n = int(rng.integers(2, 8))
        z = rng.normal(0, 1.5, n)
        p, _ = orc.entmax15(z)
        obj = lambda x: -(x @ z + 4.0 / 3.0 * (1 - (np.clip(x, 0, None) ** 1.5).sum()))
        res = scipy.optimize.minimize(obj, np.full(n, 1 / n), method="SLSQP", bounds=[(0, 1)] * n,
                                      constraints=[{"type": "eq", "fun": lambda x: x.sum() - 1}],
                                      options=dict(ftol=1e-15, maxiter=1000))
        np.testing.assert_allclose(p, res.x, atol=2e-5)


def test_entmax_sums_to_one_with_exact_zeros_below_threshold(orc):
    rng = _rng(20)
    for alpha in (1.5, 2.0, 1.25, 1.75):
        z = rng.normal(0, 2, 3000)
        p, tau = orc.entmax(z, alpha)
        assert abs(p.sum() - 1) <= 1e-10
        zero = (alpha - 1) * z <= tau
        assert np.all(p[zero] == 0.0) and np.all(p[~zero] > 0.0)


def test_entmax_alpha_to_one_is_softmax(orc):
    rng = _rng(21)
    z = rng.normal(0, 1, 50)
    sm = scipy.special.softmax(z)
    errs = [np.abs(orc.entmax_bisect(z, 1 + eps)[0] - sm).max() for eps in (1e-2, 1e-3, 1e-4)]
    assert errs[0] > errs[1] > errs[2] and errs[2] < 1e-3
    assert errs[1] / errs[2] == pytest.approx(10, rel=0.3)       # first-order in (alpha - 1)
    np.testing.assert_allclose(orc.softmax(z), sm, rtol=1e-13)


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("alpha", [1.0, 1.5, 2.0])
@pytest.mark.parametrize("gran", [0, 1])
def test_attend_head_equals_dense_attention_on_gathered_copy(orc, alpha, gran):
    c = _f32_cache(_rng(22), bf16=True, lens=(37, 61))
    scale = 1 / math.sqrt(c.d)
    q = _dec(c.q)
    rng = _rng(23)
    for b in range(c.B):
        for h in range(c.Hq):
            g = h // c.G
            if gran == 0:
                sel = np.sort(rng.choice(c.pages(b), size=3, replace=False))
                toks = np.concatenate([np.arange(p * c.S, p * c.S + c.page_tokens(b, p)) for p in sel])
            else:
                sel = np.sort(rng.choice(c.length(b), size=11, replace=False))
                toks = sel
            K, V = _rows(c, b, g, c.k)[toks], _rows(c, b, g, c.v)[toks]
            z = scale * (K @ q[b, h])
            if alpha == 1.0:
                p = scipy.special.softmax(z)
            else:   # weights from the (separately pinned) entmax; this pins gather, scale and sum
                p, _ = orc.entmax(z, alpha)
            out, pw, tok = orc.attend_head(c, b, h, sel, gran, alpha, scale)
            assert np.array_equal(tok, toks)
            np.testing.assert_allclose(pw, p, atol=1e-13)
            np.testing.assert_allclose(out, p @ V, atol=1e-12)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_support_recovery_gives_full_cache_output(orc, alpha):
    # EntmaxKV s2 / s2.C / s3: if the kept pages contain the entmax support, the sparse output
    # equals the full-cache output
    c = _f32_cache(_rng(24), bf16=True, lens=(200, 97), d=32, S=8)
    scale = 1.0   # larger logits: small supports
    rng = _rng(25)
    for b in range(c.B):
        for h in range(c.Hq):
            full, p = orc.attend_full_head(c, b, h, alpha, scale)
            supp_pages = np.unique(np.nonzero(p > 0)[0] // c.S)
            extra = rng.choice(c.pages(b), size=2, replace=False)
            sel = np.unique(np.concatenate([supp_pages, extra]))
            out, _, _ = orc.attend_head(c, b, h, sel, 0, alpha, scale)
            np.testing.assert_allclose(out, full, atol=1e-12)


@pytest.mark.parametrize("alpha", [1.0, 1.5, 2.0])
def test_error_bound_two_B_delta(orc, alpha):
    # EntmaxKV s3: |o - o~| <= 2 B delta, B = max |v_t|, delta = full-cache mass dropped.
    # For softmax any dropped token gives delta > 0 (dense tail, s1).
    c = _f32_cache(_rng(26), bf16=True, lens=(150,), B=1, d=32, S=8)
    scale = 1 / math.sqrt(c.d)
    rng = _rng(27)
    V = _rows(c, 0, 0, c.v)
    Bn = np.linalg.norm(V, axis=1).max()
    for h in range(c.Hq):
        full, p = orc.attend_full_head(c, 0, h, alpha, scale)
        for _ in range(5):
            sel = np.sort(rng.choice(c.pages(0), size=int(rng.integers(1, c.pages(0))), replace=False))
            out, _, tok = orc.attend_head(c, 0, h, sel, 0, alpha, scale)
            delta = p.sum() - p[tok].sum()
            assert np.linalg.norm(out - full) <= 2 * Bn * delta + 1e-12
            if alpha == 1.0:
                assert delta > 0


def test_empty_selection_and_empty_sequence_give_zero_output(orc):
    c = _f32_cache(_rng(28), lens=(0, 9))
    out, p, tok = orc.attend_head(c, 0, 0, np.zeros(0, np.int32), 0, 1.5, 1.0)
    assert np.all(out == 0) and len(p) == 0
    out, _, _ = orc.attend_head(c, 1, 0, np.zeros(0, np.int32), 0, 1.0, 1.0)
    assert np.all(out == 0)
    kmin, kmax = orc.meta_box(c)
    assert np.all(orc.score_box(c, kmin, kmax)[0] == -np.inf)


# ---------------------------------------------------------------- the step on the workloads

def test_tiny_step_support_recovery_and_bound(orc):
    w = W.make("tiny")
    h = W.host_arrays(w)
    c = oracle.Cache(q=h["q"], k=h["k"], v=h["v"], block_table=h["block_table"], seq_lens=h["seq_lens"])
    spec = pipeline.Spec(score="box", policy="topk", k=32, alphas=(1.5, 1.0))
    md, sc, res = pipeline.run(c, spec)
    r = res[(0, 0)]
    assert len(r.sel) == 32 and np.all(np.diff(r.sel) > 0)
    q = _dec(c.q)[0, 0]
    rows = _rows(c, 0, 0, c.k)
    true_page_max = (rows @ q).reshape(-1, c.S).max(1)
    assert np.all(sc.key[0, 0] >= true_page_max.astype(np.float32) - 1e-4)
    for a in (1.5, 1.0):
        full, p = pipeline.full_reference(c, spec, 0, 0, a)
        kept = np.zeros(c.pages(0), bool)
        kept[r.sel] = True
        delta = p[0].reshape(-1, c.S)[~kept].sum()
        Bn = np.linalg.norm(_rows(c, 0, 0, c.v), axis=1).max()
        assert np.linalg.norm(r.out[a][0] - full[0]) <= 2 * Bn * delta + 1e-12


# ---------------------------------------------------------------- soft-LSH token scores (SOCKET)

def _planes(rng, L, P, d):
    return rng.standard_normal((L, P, d)).astype(np.float32)


def _sign_matrix(P):
    """[2^P, P]: row beta holds +1 where bit i of beta is set, else -1."""
    beta = np.arange(1 << P)[:, None]
    return np.where((beta >> np.arange(P)[None, :]) & 1, 1.0, -1.0)


@pytest.mark.parametrize("bf16", [False, True])
def test_lsh_buckets_are_sign_patterns_of_numpy_projections(orc, bf16):
    rng = _rng(301)
    c = _f32_cache(rng, bf16=bf16)
    W_ = _planes(rng, 5, 6, c.d)
    bucket, vnorm = orc.meta_lsh(c, W_)
    for b in range(c.B):
        for g in range(c.Hkv):
            K = _rows(c, b, g, c.k)                                   # [L, d]
            dots = np.einsum("lpd,td->tlp", W_.astype(np.float64), K)  # [L_b, tables, bits]
            assert np.abs(dots).min() > 1e-9                           # no sign is decided by rounding
            ids = ((dots > 0) << np.arange(6)[None, None, :]).sum(-1)
            t = np.arange(c.length(b))
            got = bucket[c.block_table[b, t // c.S], g, t % c.S]
            assert np.array_equal(got, ids)
            vn = np.sqrt(np.sum(_rows(c, b, g, c.v) ** 2, axis=1)).astype(np.float32)
            gv = vnorm[c.block_table[b, t // c.S], g, t % c.S]
            assert np.all(np.abs(gv.view(np.int32) - vn.view(np.int32)) <= 1)   # rounding order only


@pytest.mark.parametrize("tau", [0.3, 1.0, 4.0])
def test_lsh_tables_equal_softmax_over_all_buckets(orc, tau):
    """The soft assignment, by its definition: a softmax over all 2^P sign vectors of <s, z>/tau."""
    rng = _rng(302)
    c = _f32_cache(rng, bf16=True)
    P = 5
    W_ = _planes(rng, 4, P, c.d)
    tab = orc.lsh_tables(c, W_, tau)
    S_ = _sign_matrix(P)
    t32 = float(np.float32(tau))
    for b in range(c.B):
        for h in range(c.Hq):
            q = _dec(c.q[b, h])
            z = W_.astype(np.float64) @ q / np.linalg.norm(q)          # [L, P]
            p = scipy.special.softmax(z @ S_.T / t32, axis=1)          # [L, 2^P]
            x = p * 2.0 ** 24
            ref = np.rint(x)
            diff = tab[b, h].astype(np.int64) - ref.astype(np.int64)
            near = np.abs(x - np.floor(x) - 0.5) < 1e-6
            assert np.all(np.abs(diff) <= 1) and np.all((diff == 0) | near), (b, h)


def test_lsh_tables_limits_and_zero_query(orc):
    rng = _rng(303)
    c = _f32_cache(rng)
    P = 4
    W_ = _planes(rng, 3, P, c.d)
    # probabilities sum to one (up to the rounding of each of the 2^P masses)
    tab = orc.lsh_tables(c, W_, 1.0).astype(np.int64)
    assert np.all(np.abs(tab.sum(-1) - 2 ** 24) <= 2 ** P // 2)
    # tau -> 0: all mass on the query's own (hard) bucket: plain sign-random-projection hashing
    hard = orc.lsh_tables(c, W_, 1e-6)
    for b in range(c.B):
        for h in range(c.Hq):
            z = W_.astype(np.float64) @ c.q[b, h].astype(np.float64)
            ids = ((z > 0) << np.arange(P)[None, :]).sum(-1)
            for l in range(3):
                expect = np.zeros(1 << P, np.uint32)
                expect[ids[l]] = 2 ** 24
                assert np.array_equal(hard[b, h, l], expect)
    # tau -> infinity: uniform
    flat = orc.lsh_tables(c, W_, 1e12)
    assert np.all(flat == 2 ** (24 - P))
    # a zero query puts equal mass on every bucket
    c.q[0, 1] = 0
    c2 = oracle.Cache(q=c.q, k=c.k, v=c.v, block_table=c.block_table, seq_lens=c.seq_lens)
    assert np.all(orc.lsh_tables(c2, W_, 1.0)[0, 1] == 2 ** (24 - P))


def test_lsh_token_scores_match_brute_force_soft_collision(orc):
    """End to end against the definition evaluated with numpy and scipy (no fixed point): the key
    of token t is ||v_t|| times the largest over the group's heads of sum_l p_l(bucket_l(t))."""
    rng = _rng(304)
    c = _f32_cache(rng, bf16=True, lens=(45, 80))
    P, L, tau = 6, 8, 0.7
    W_ = _planes(rng, L, P, c.d)
    spec = pipeline.Spec(score="lsh", policy="token_topk", k=10, lsh_planes=W_, lsh_tau=tau)
    md = pipeline.build_metadata(c, spec)
    sc = pipeline.compute_scores(c, spec, md)
    S_ = _sign_matrix(P)
    for b in range(c.B):
        Lb = c.length(b)
        for g in range(c.Hkv):
            K, V = _rows(c, b, g, c.k), _rows(c, b, g, c.v)
            ids = (((np.einsum("lpd,td->tlp", W_.astype(np.float64), K) > 0) << np.arange(P)).sum(-1))  # [Lb, L]
            best = np.zeros(Lb)
            for h in range(g * c.G, (g + 1) * c.G):
                q = _dec(c.q[b, h])
                p = scipy.special.softmax((W_.astype(np.float64) @ q / np.linalg.norm(q)) @ S_.T
                                          / float(np.float32(tau)), axis=1)
                best = np.maximum(best, p[np.arange(L)[None, :], ids].sum(1))
            ref = np.linalg.norm(V, axis=1) * best
            got = sc.key[b, g, :Lb].astype(np.float64)
            # fixed point (2^-24 per table) and two float32 roundings
            assert np.all(np.abs(got - ref) <= np.linalg.norm(V, axis=1) * L * 2.0 ** -24 + 2e-7 * ref)
            assert np.all(np.isneginf(sc.key[b, g, Lb:]))
            r = pipeline.select_unit(c, spec, sc, b, g)
            order = np.lexsort((np.arange(Lb), -ref))[:spec.k]
            gap = np.sort(ref)[::-1]
            if gap[spec.k - 1] - gap[spec.k] > 1e-5 * gap[0]:                  # no near-tie at the cut
                assert np.array_equal(r.sel, np.sort(order))


def test_lsh_single_table_at_zero_temperature_is_hard_collision_times_value_norm(orc):
    """One table and tau -> 0: the score is ||v|| where the key's bucket equals the query's own
    bucket for some head of the group, and 0 elsewhere (plain LSH collision)."""
    rng = _rng(305)
    c = _f32_cache(rng, lens=(64, 30))
    P = 2
    W_ = _planes(rng, 1, P, c.d)
    spec = pipeline.Spec(score="lsh", policy="token_topk", k=5, lsh_planes=W_, lsh_tau=1e-6)
    md = pipeline.build_metadata(c, spec)
    sc = pipeline.compute_scores(c, spec, md)
    for b in range(c.B):
        Lb = c.length(b)
        for g in range(c.Hkv):
            K, V = _rows(c, b, g, c.k), _rows(c, b, g, c.v)
            kid = ((K @ W_[0].T.astype(np.float64) > 0) << np.arange(P)).sum(-1)
            qid = [int(((W_[0].astype(np.float64) @ c.q[b, h].astype(np.float64) > 0) << np.arange(P)).sum())
                   for h in range(g * c.G, (g + 1) * c.G)]
            hit = np.isin(kid, qid)
            ref = np.where(hit, np.linalg.norm(V, axis=1), 0.0).astype(np.float32)
            assert np.array_equal(sc.key[b, g, :Lb], ref)

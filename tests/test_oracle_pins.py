"""Pins of the fp64 CPU oracle against what the Locks paper and plain
mathematics fix, independently of the oracle's own code.

Each test names the passage of "Locks: Page-Local Compact Key Summaries for
Efficient Long-Context Decoding" (arXiv 2607.24555) it checks. Independent
references used here: numpy/LAPACK SVD and eigh, scipy logsumexp, torch's
scaled_dot_product_attention on the CPU, torch's bfloat16 cast, closed forms
printed in the paper, and brute-force enumeration of page sets.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page(rng, P, d, rank, noise=0.05, cstd=0.5, var=None):
    var = var if var is not None else [4.0 / 2 ** i for i in range(rank)]
    B, _ = np.linalg.qr(rng.standard_normal((d, rank)))
    a = rng.standard_normal((P, rank)) * np.sqrt(var)
    return cstd * rng.standard_normal(d) + a @ B.T + noise * rng.standard_normal((P, d))


def _svd(k):
    D = k - k.mean(0)
    _, s, vh = np.linalg.svd(D)
    return D, s, vh


# --------------------------------------------------------------------------
# O1 summary fit: [Locks] §3 (mu_j, H_j), §4 (D_j, V_j, C_j), App. A.2 Cor. 1
# --------------------------------------------------------------------------
@pytest.mark.parametrize("P,d,r", [(8, 6, 2), (16, 12, 4), (12, 16, 3), (16, 64, 4)])
def test_build_matches_lapack_svd(P, d, r):
    rng = np.random.default_rng(P * 100 + d)
    keys = np.stack([_page(rng, P, d, r) for _ in range(5)])
    mu, vt, coef, ev, _ = oracle.build_pages(keys, r)
    for j in range(keys.shape[0]):
        D, s, vh = _svd(keys[j])
        np.testing.assert_allclose(mu[j], keys[j].mean(0), rtol=0, atol=1e-14)
        # eigenvalues of H = D^T D are the squared singular values of D
        lam = np.zeros(d)
        lam[: len(s)] = s ** 2
        np.testing.assert_allclose(ev[j], lam, rtol=1e-10, atol=1e-10 * lam[0])
        # same top-r subspace (the gap sigma_r > sigma_r+1 holds for these draws)
        assert s[r - 1] > 1.05 * (s[r] if r < len(s) else 0.0)
        Pl = vh[:r].T @ vh[:r]
        Po = vt[j].T @ vt[j]
        assert np.linalg.norm(Pl - Po) < 1e-9
        # Eckart-Young residual, [Locks] App. A.2 Cor. 1
        resid = np.linalg.norm(D - D @ vt[j].T @ vt[j]) ** 2
        assert abs(resid - np.sum(s[r:] ** 2)) <= 1e-9 * max(1.0, np.sum(s ** 2))


def test_build_invariants():
    rng = np.random.default_rng(3)
    P, d, r = 16, 32, 5
    keys = np.stack([_page(rng, P, d, 6) for _ in range(4)])
    mu, vt, coef, _, _ = oracle.build_pages(keys, r)
    for j in range(4):
        D = keys[j] - mu[j]
        np.testing.assert_allclose(vt[j] @ vt[j].T, np.eye(r), atol=1e-12)   # V^T V = I
        np.testing.assert_allclose(coef[j].sum(0), 0.0, atol=1e-11)          # centred keys
        np.testing.assert_allclose(coef[j], D @ vt[j].T, atol=1e-12)         # C = D V
        # sign convention: the largest-magnitude entry of each basis vector is positive
        for rho in range(r):
            assert vt[j, rho, np.argmax(np.abs(vt[j, rho]))] > 0


def test_full_rank_reconstructs_keys():
    """r >= rank(D_j): mu + V c_i = k_i ([Locks] §4 Thm. 1(i), eta = 0)."""
    rng = np.random.default_rng(4)
    P, d = 8, 16
    keys = np.stack([_page(rng, P, d, 3) for _ in range(3)])
    mu, vt, coef, _, _ = oracle.build_pages(keys, P - 1)   # rank(D) <= P-1
    rec = mu[:, None, :] + np.einsum("jpr,jrd->jpd", coef, vt)
    np.testing.assert_allclose(rec, keys, atol=1e-12)


# --------------------------------------------------------------------------
# O2 scores: [Locks] §2 Eq. (1), §4 Eq. (2), App. A.2-A.3
# --------------------------------------------------------------------------
def test_exact_lse_bruteforce():
    rng = np.random.default_rng(5)
    G, n, P, d = 3, 7, 16, 24
    q = rng.standard_normal((G, d))
    keys = rng.standard_normal((n, P, d))
    nv = rng.integers(1, P + 1, n)
    scale = 1 / math.sqrt(d)
    s = oracle.exact_page_lse(q, keys, scale, n_valid=nv)
    for g in range(G):
        for j in range(n):
            ref = logsumexp(keys[j, : nv[j]] @ q[g] * scale)
            assert abs(s[g, j] - ref) < 1e-12


@pytest.mark.parametrize("P,d", [(16, 64), (8, 12)])
def test_full_rank_scores_equal_exact(P, d):
    """At r >= rank(D_j) the reconstructed LSE equals the exact one (Thm. 1(i))."""
    rng = np.random.default_rng(6)
    keys = np.stack([_page(rng, P, d, 5, noise=0.3) for _ in range(6)])
    q = rng.standard_normal((4, d))
    r = min(d, P - 1)
    mu, vt, coef, _, _ = oracle.build_pages(keys, r)
    scale = 1 / math.sqrt(d)
    sh = oracle.page_scores(q, mu, vt, coef, scale)
    s = oracle.exact_page_lse(q, keys, scale)
    np.testing.assert_allclose(sh, s, rtol=0, atol=1e-11)


def test_score_error_bound():
    """|shat - s| <= ||q_perp|| sigma_{r+1} / sqrt(d)  ([Locks] Thm. 1(i), A.3 Step 1)."""
    rng = np.random.default_rng(7)
    P, d, r = 16, 32, 3
    keys = np.stack([_page(rng, P, d, 6, noise=0.2) for _ in range(8)])
    q = 2.0 * rng.standard_normal((5, d))
    mu, vt, coef, _, _ = oracle.build_pages(keys, r)
    scale = 1 / math.sqrt(d)
    sh = oracle.page_scores(q, mu, vt, coef, scale)
    s = oracle.exact_page_lse(q, keys, scale)
    worst_ratio = 0.0
    for j in range(8):
        _, sv, _ = _svd(keys[j])
        for g in range(5):
            qp = q[g] - vt[j].T @ (vt[j] @ q[g])
            bound = np.linalg.norm(qp) * sv[r] * scale
            assert abs(sh[g, j] - s[g, j]) <= bound + 1e-12
            worst_ratio = max(worst_ratio, abs(sh[g, j] - s[g, j]) / bound)
    assert worst_ratio > 0.01  # the bound is not vacuous on these pages


def test_score_rotation_invariance():
    """Any orthonormal basis of the same subspace gives the same score ([Locks] A.2 Cor. 1)."""
    rng = np.random.default_rng(8)
    P, d, r = 16, 20, 4
    keys = np.stack([_page(rng, P, d, 5) for _ in range(3)])
    mu, vt, coef, _, _ = oracle.build_pages(keys, r)
    R, _ = np.linalg.qr(rng.standard_normal((r, r)))
    vt2 = np.einsum("ab,jbd->jad", R.T, vt)       # V -> V R
    coef2 = coef @ R                              # C -> C R
    q = rng.standard_normal((3, d))
    a = oracle.page_scores(q, mu, vt, coef, 0.3)
    b = oracle.page_scores(q, mu, vt2, coef2, 0.3)
    np.testing.assert_allclose(a, b, atol=1e-12)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden("closed_forms.json")["prop1"])
def test_prop1_closed_form(case):
    """[Locks] App. A.2, proof of Prop. 1: B zero keys give s_P(u) = log B; replacing two
    by +-c u gives log(B - 2 + 2 cosh(c/sqrt(d))); a page-local rank-1 fit is exact."""
    B, d, c = case["B"], case["d"], case["c"]
    rng = np.random.default_rng(9)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    P0 = np.zeros((B, d))
    Pc = np.zeros((B, d))
    Pc[0] = c * u
    Pc[1] = -c * u
    scale = 1 / math.sqrt(d)
    s = oracle.exact_page_lse(u[None], np.stack([P0, Pc]), scale)
    assert abs(s[0, 0] - math.log(B)) < 1e-12
    assert abs(s[0, 1] - math.log(B - 2 + 2 * math.cosh(c / math.sqrt(d)))) < 1e-10
    mu, vt, coef, _, _ = oracle.build_pages(np.stack([P0, Pc]), 1)
    sh = oracle.page_scores(u[None], mu, vt, coef, scale)
    np.testing.assert_allclose(sh, s, atol=1e-10)
    np.testing.assert_allclose(np.abs(vt[1, 0]), np.abs(u), atol=1e-12)


@pytest.mark.parametrize("case", _golden("closed_forms.json")["lemma2"])
def test_lemma2_pair(case):
    """[Locks] App. A.2, proof of Lemma 2: pages with equal per-dimension extremes whose
    exact log-masses differ; for q = (e1+e2)/sqrt(2), s_P = log B and
    s_P' = log(B - 2 + 2 cosh(t sqrt(2)/sqrt(d))). Both have rank-1 centred keys, so the
    rank-1 local summary is exact for both."""
    B, d, t = case["B"], case["d"], case["t"]
    Pp = np.zeros((B, d)); Pp[0, :2] = [t, t]; Pp[1, :2] = [-t, -t]
    Pn = np.zeros((B, d)); Pn[0, :2] = [t, -t]; Pn[1, :2] = [-t, t]
    assert np.array_equal(Pp.max(0), Pn.max(0)) and np.array_equal(Pp.min(0), Pn.min(0))
    q = np.zeros(d); q[:2] = 1 / math.sqrt(2)
    scale = 1 / math.sqrt(d)
    s = oracle.exact_page_lse(q[None], np.stack([Pn, Pp]), scale)
    assert abs(s[0, 0] - math.log(B)) < 1e-12
    x = t * math.sqrt(2) / math.sqrt(d)
    assert abs(s[0, 1] - math.log(B - 2 + 2 * math.cosh(x))) < 1e-10
    assert s[0, 1] - s[0, 0] >= x - math.log(B) - 1e-12
    mu, vt, coef, _, _ = oracle.build_pages(np.stack([Pn, Pp]), 1)
    sh = oracle.page_scores(q[None], mu, vt, coef, scale)
    np.testing.assert_allclose(sh, s, atol=1e-10)


# --------------------------------------------------------------------------
# O3/O4 combine + select: [Locks] §2 (mandatory pages, k slots), §4 (shares,
# share average), App. A.1 Lemma 1(ii), App. A.3 Steps 2-3, App. A.4
# --------------------------------------------------------------------------
def _token_masses(q, keys, scale):
    """Softmax weight of every token of every page, per head (independent of the oracle)."""
    G = q.shape[0]
    n, P, d = keys.shape
    z = np.einsum("gd,npd->gnp", q, keys) * scale
    z = z.reshape(G, -1)
    w = np.exp(z - z.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    return w.reshape(G, n, P)


def _coverage(masses, S):
    """Group-average coverage: mean over heads of the attention mass inside pages S."""
    return float(np.mean([masses[g, list(S)].sum() for g in range(masses.shape[0])]))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_selection_maximises_group_coverage_bruteforce(seed):
    """With exact scores, {0, J-1} + top-(k-2) by the share average maximises the
    group-average coverage over all shared sets containing the two mandatory pages
    ([Locks] App. A.4, Lemma 1(ii)). Coverage is measured from token-level softmax
    weights, not from the oracle's combine."""
    rng = np.random.default_rng(100 + seed)
    J, P, d, G, k = 11, 4, 8, 3, 5
    # heads of very different norms so that un-normalised pooling would rank differently
    q = rng.standard_normal((G, d)) * np.array([[0.3], [1.0], [3.0]])
    keys = rng.standard_normal((J, P, d)) * 1.5
    scale = 1 / math.sqrt(d)
    s = oracle.exact_page_lse(q, keys, scale)
    _, sigma = oracle.combine(s)
    sel = oracle.select(sigma, J, J, k)
    S = set(int(x) for x in sel if x >= 0)
    assert len(S) == k and {0, J - 1} <= S
    masses = _token_masses(q, keys, scale).sum(-1)   # [G][J] page masses
    best = max(_coverage(masses, {0, J - 1} | set(c))
               for c in itertools.combinations(range(1, J - 1), k - 2))
    assert abs(_coverage(masses, S) - best) < 1e-12
    # the share average equals the group-mean page mass computed from tokens
    np.testing.assert_allclose(np.exp(sigma), masses.mean(0), rtol=1e-12)


def test_selection_single_head_is_exact_topk():
    """G = 1: the free slots take the top pages by exact LSE ([Locks] Lemma 1(ii))."""
    rng = np.random.default_rng(11)
    J, P, d, k = 12, 4, 6, 6
    q = rng.standard_normal((1, d))
    keys = rng.standard_normal((J, P, d))
    s = oracle.exact_page_lse(q, keys, 0.4)
    _, sigma = oracle.combine(s)
    sel = oracle.select(sigma, J, J, k)
    free = sorted(range(1, J - 1), key=lambda j: -s[0, j])[: k - 2]
    assert sorted(sel.tolist()) == sorted([0, J - 1] + free)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_theorem1_retention_and_sandwich(seed):
    """Low-rank summaries: |log mhat_j - log m_j| <= 2 eta (A.3 Step 2) and
    gamma(S) >= exp(-4 eta) gamma* (Thm. 1(ii)), gamma* by brute force."""
    rng = np.random.default_rng(200 + seed)
    J, P, d, G, k, r = 10, 8, 12, 4, 4, 2
    keys = np.stack([_page(rng, P, d, 4, noise=0.3, var=[2.0, 1.0, 0.7, 0.5])
                     for _ in range(J)])
    q = 2.0 * rng.standard_normal((G, d))
    scale = 1 / math.sqrt(d)
    mu, vt, coef, _, _ = oracle.build_pages(keys, r)
    sh = oracle.page_scores(q, mu, vt, coef, scale)
    s = oracle.exact_page_lse(q, keys, scale)
    eta = np.max(np.abs(sh - s))
    assert eta > 0.01
    _, sig_hat = oracle.combine(sh)
    _, sig = oracle.combine(s)
    assert np.max(np.abs(sig_hat - sig)) <= 2 * eta + 1e-12
    sel = oracle.select(sig_hat, J, J, k)
    masses = _token_masses(q, keys, scale).sum(-1)
    S = set(int(x) for x in sel)
    best = max(_coverage(masses, {0, J - 1} | set(c))
               for c in itertools.combinations(range(1, J - 1), k - 2))
    assert _coverage(masses, S) >= math.exp(-4 * eta) * best - 1e-12


def test_select_rules():
    """[Locks] §2/§4 with readings: J <= k keeps all pages; the partial page J-1 is kept
    but never ranked; equal keys go to the lower page id; output ascending, -1 padded."""
    assert oracle.select(np.zeros(3), 3, 4, 6).tolist() == [0, 1, 2, 3, -1, -1]
    assert oracle.select(np.zeros(0), 0, 1, 2).tolist() == [0, -1]
    sig = np.array([5.0, 1.0, 3.0, 3.0, 0.5, 3.0, 9.0])      # 7 complete pages
    # J = 8: page 7 is the partial current page
    assert oracle.select(sig, 7, 8, 4).tolist() == [0, 2, 6, 7]   # 6 ranks first; 2 wins the tie
    # J = 7, all complete: page 6 (current) is mandatory though top-scored
    assert oracle.select(sig, 7, 7, 5).tolist() == [0, 2, 3, 5, 6]
    assert oracle.select(sig, 7, 7, 2).tolist() == [0, 6]


# --------------------------------------------------------------------------
# O5 attention: [Locks] §2, App. A.1 Lemma 1(i)
# --------------------------------------------------------------------------
def test_attend_matches_torch_sdpa():
    rng = np.random.default_rng(12)
    G, n, d = 4, 37, 16
    q = rng.standard_normal((G, d)); k = rng.standard_normal((n, d)); v = rng.standard_normal((n, d))
    o, lse = oracle.attend(q, k, v, 1 / math.sqrt(d))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[:, None, None, :], torch.tensor(k)[None, None].expand(G, 1, n, d),
        torch.tensor(v)[None, None].expand(G, 1, n, d))[:, 0, 0]
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    np.testing.assert_allclose(lse, logsumexp(q @ k.T / math.sqrt(d), axis=1), atol=1e-12)


def test_lemma1_identity_and_bound():
    """o - o_S = eps (vbar_Sc - vbar_S), eps = 1 - gamma_S; ||o - o_S|| <= 2R(1 - gamma_S)."""
    rng = np.random.default_rng(13)
    J, P, d = 9, 4, 10
    q = rng.standard_normal((1, d)); keys = rng.standard_normal((J, P, d))
    vals = rng.standard_normal((J, P, d))
    scale = 1 / math.sqrt(d)
    S = [0, 3, 4, 8]; Sc = [j for j in range(J) if j not in S]
    o, _ = oracle.attend(q, keys.reshape(-1, d), vals.reshape(-1, d), scale)
    oS, _ = oracle.attend(q, keys[S].reshape(-1, d), vals[S].reshape(-1, d), scale)
    oSc, _ = oracle.attend(q, keys[Sc].reshape(-1, d), vals[Sc].reshape(-1, d), scale)
    gamma = _token_masses(q, keys, scale)[0, S].sum()
    eps = 1 - gamma
    np.testing.assert_allclose(o - oS, eps * (oSc - oS), atol=1e-12)
    R = np.linalg.norm(vals.reshape(-1, d), axis=1).max()
    assert np.linalg.norm(o - oS) <= 2 * R * eps + 1e-12


def test_lse_merge_of_splits_equals_one_pass():
    """Splitting the token set and merging (o, lse) by LSE weights reproduces one pass
    (the split-K combination rule; exact algebra of the softmax normaliser)."""
    rng = np.random.default_rng(14)
    G, n, d = 3, 50, 8
    q = rng.standard_normal((G, d)); k = rng.standard_normal((n, d)); v = rng.standard_normal((n, d))
    o, lse = oracle.attend(q, k, v, 0.5)
    parts = [oracle.attend(q, k[a:b], v[a:b], 0.5) for a, b in ((0, 13), (13, 40), (40, 50))]
    L = logsumexp(np.stack([p[1] for p in parts]), axis=0)
    om = sum(np.exp(p[1] - L)[:, None] * p[0] for p in parts)
    np.testing.assert_allclose(om, o, atol=1e-12)
    np.testing.assert_allclose(L, lse, atol=1e-12)


def test_decode_step_full_budget_is_dense():
    """Budget >= pages: the whole pipeline attends every valid token (dense decode)."""
    rng = np.random.default_rng(15)
    P, d, Hkv, G = 4, 8, 2, 2
    T = 4 * 5 + 3
    J = 6
    blocks = 9
    kp = rng.standard_normal((blocks, Hkv, P, d)); vp = rng.standard_normal((blocks, Hkv, P, d))
    bt = np.array([[3, 0, 7, 1, 8, 5]])
    q = rng.standard_normal((1, Hkv * G, d))
    res = oracle.decode_step(q, None, None, None, kp, vp, bt, [T], P, J, 0.3, threads=1)
    for h in range(Hkv):
        keys = np.concatenate([kp[bt[0, j], h] for j in range(J)])[:T]
        vals = np.concatenate([vp[bt[0, j], h] for j in range(J)])[:T]
        o, lse = oracle.attend(q[0, h * G:(h + 1) * G], keys, vals, 0.3)
        np.testing.assert_allclose(res[(0, h)]["out"], o, atol=1e-13)
        assert res[(0, h)]["sel"].tolist() == list(range(J))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_step_over_budget_selects_exact_set_at_full_rank(seed):
    """The J > k branch of the whole step ([Locks] §2 budget and mandatory
    pages, §4 share-average selection, Thm. 1 (i)): summaries gathered through
    a shuffled block table, scored, combined, selected and attended with a
    partial current page. With full-rank summaries (r = P - 1 spans every
    centred page) the selection must be the exact-LSE page set and the output
    softmax attention over those pages' valid tokens, both computed here from
    the keys with numpy and scipy."""
    rng = np.random.default_rng(100 + seed)
    B, Hkv, G, d, P, k, scale = 3, 2, 3, 16, 8, 6, 0.3
    lens = [P * 20 + 3, P * 14, P * 9 + 7]  # partial, complete and partial current pages
    maxp = max(-(-T // P) for T in lens)
    nblk = B * maxp + 4
    bt = rng.permutation(nblk)[:B * maxp].reshape(B, maxp)
    keys = rng.standard_normal((nblk, Hkv, P, d)) * 0.7
    vals = rng.standard_normal((nblk, Hkv, P, d))
    q = rng.standard_normal((B, Hkv * G, d))
    for b, T in enumerate(lens):  # slots past T hold a poison value
        if T % P:
            keys[bt[b, T // P], :, T % P:] = 100.0
            vals[bt[b, T // P], :, T % P:] = 100.0
    mu, vt, cf, _, _ = oracle.build_pages(keys.reshape(-1, P, d), P - 1)
    res = oracle.decode_step(q, mu.reshape(nblk, Hkv, d), vt.reshape(nblk, Hkv, P - 1, d),
                             cf.reshape(nblk, Hkv, P, P - 1), keys, vals, bt, lens, P, k, scale,
                             threads=2)
    for b, T in enumerate(lens):
        J, Jc = -(-T // P), T // P
        for h in range(Hkv):
            qg = q[b, h * G:(h + 1) * G]
            s = logsumexp(np.einsum("gd,jpd->gjp", qg, keys[bt[b, :Jc], h]) * scale, axis=2)
            sigma = logsumexp(s - logsumexp(s, axis=1)[:, None], axis=0) - math.log(G)
            cand = sorted((j for j in range(1, Jc) if j != J - 1), key=lambda j: (-sigma[j], j))
            assert sigma[cand[k - 3]] - sigma[cand[k - 2]] > 1e-6  # no near-tie at the cut
            want = sorted([0, J - 1] + cand[:k - 2])
            assert res[(b, h)]["sel"].tolist() == want
            kk = np.concatenate([keys[bt[b, j], h, :min(P, T - j * P)] for j in want])
            vv = np.concatenate([vals[bt[b, j], h, :min(P, T - j * P)] for j in want])
            z = qg @ kk.T * scale
            lse = logsumexp(z, axis=1)
            o = np.exp(z - lse[:, None]) @ vv
            np.testing.assert_allclose(res[(b, h)]["out"], o, atol=1e-12)
            np.testing.assert_allclose(res[(b, h)]["lse"], lse, atol=1e-12)


# --------------------------------------------------------------------------
# bf16 storage rounding (summaries are stored in bf16, [Locks] §4 storage)
# --------------------------------------------------------------------------
def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(16)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -130, 3.3e38,
                  -3.4e38, 0.0, 1e-45], dtype=np.float32)])
    x = x.astype(np.float32)
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


# --------------------------------------------------------------------------
# Quantized summary storage ([Locks] §4 "i4" variants, App. C.7)
# --------------------------------------------------------------------------
def _quantize_one_group(x, L):
    """Quantize a single group through the oracle by placing it where that
    group width lives: L = 7 -> one basis vector, L = 127 -> the centroid."""
    x = np.asarray(x, dtype=np.float64)
    n = x.size
    if L == 7:
        qs = oracle.quantize_summaries(np.zeros((1, n)), x[None, None, :], np.zeros((1, 1, 1)))
        return qs["vt_scale"][0, 0], qs["vt_code"][0, 0]
    qs = oracle.quantize_summaries(x[None, :], np.zeros((1, 1, n)), np.zeros((1, 1, 1)))
    return qs["mu_scale"][0], qs["mu_code"][0]


@pytest.mark.parametrize("case", _golden("quantize_worked.json")["groups"], ids=lambda c: c["name"])
def test_quantize_worked_examples(case):
    scale, codes = _quantize_one_group(case["x"], case["L"])
    assert scale == case["scale"]
    assert codes.tolist() == case["codes"]


def test_quantize_coefficient_rows_use_their_own_scale():
    # the coefficient group is a token's row of r values: the hand-worked row
    # as token 1 of a page, next to a token whose row is 64x smaller
    row = [-2.54, 0.01, 1.0]
    coef = np.array([[[x / 64 for x in row], row]])
    qs = oracle.quantize_summaries(np.zeros((1, 4)), np.zeros((1, 3, 4)), coef)
    assert qs["coef_scale"][0, 1] == 0.02001953125
    assert qs["coef_code"][0, 1].tolist() == [-127, 0, 50]
    assert qs["coef_scale"][0, 0] == 0.02001953125 / 64  # a power of two apart: same codes
    assert qs["coef_code"][0, 0].tolist() == [-127, 0, 50]


@pytest.mark.parametrize("case", _golden("byte_model.json")["summaries_with_scales"],
                         ids=lambda c: f"r{c['r']}")
def test_quantized_byte_model(case):
    """Bits of the stored codes and scales equal the pages' byte counts."""
    rng = np.random.default_rng(case["r"])
    B, d, r = case["B"], case["d"], case["r"]
    keys = _page(rng, B, d, 6)[None]
    mu, vt, cf, _, _ = oracle.build_pages(keys, r)
    qs = oracle.quantize_summaries(mu, vt, cf)
    assert np.abs(qs["vt_code"]).max() <= 7        # fits a signed 4-bit field
    assert np.abs(qs["mu_code"]).max() <= 127      # fits a signed 8-bit field
    assert np.abs(qs["coef_code"]).max() <= 127
    n_scales = qs["mu_scale"].size + qs["vt_scale"].size + qs["coef_scale"].size
    bits = 4 * qs["vt_code"].size + 8 * (qs["mu_code"].size + qs["coef_code"].size) + 16 * n_scales
    assert bits % 8 == 0
    assert bits // 8 == case["bytes"]
    kv = _golden("byte_model.json")["kv_page_bytes"]["bytes"]
    assert round(case["bytes"] / kv, 3) == case["alpha"]


def _fitted(seed, n=6, P=16, d=64, r=4):
    rng = np.random.default_rng(seed)
    keys = np.stack([_page(rng, P, d, 6) for _ in range(n)])
    return oracle.build_pages(keys, r)[:3]


@pytest.mark.parametrize("seed", [0, 1])
def test_quantize_roundtrip_bound(seed):
    """No code is ever clamped (bf16(amax/L) is within 2^-9 of amax/L), so every
    stored value is within half a step of the fitted one, and the group's
    largest entry maps to +-L."""
    mu, vt, cf = _fitted(seed)
    qs = oracle.quantize_summaries(mu, vt, cf)
    dmu, dvt, dcf = oracle.dequantize_summaries(qs)
    for x, y, s, L, code in ((mu, dmu, qs["mu_scale"][:, None], 127, qs["mu_code"]),
                             (vt, dvt, qs["vt_scale"][:, :, None], 7, qs["vt_code"]),
                             (cf, dcf, qs["coef_scale"][:, :, None], 127, qs["coef_code"])):
        assert np.all(np.abs(x - y) <= 0.5 * s * (1 + 1e-6) + 1e-7 * np.abs(x))
        assert np.all(np.abs(code).max(axis=-1) == L)


def test_quantize_grid_values_roundtrip_exactly():
    """Values already on the grid (integer codes times a bf16 scale, largest
    code +-L, a different scale per group) come back exactly, so the quantized
    page score equals the unquantized one."""
    rng = np.random.default_rng(7)
    n, P, d, r = 3, 16, 64, 4

    def grid(shape, L):
        c = rng.integers(-L, L + 1, size=shape)
        c[..., 0] = L * rng.choice([-1, 1], size=shape[:-1])
        s = oracle.round_bf16(2.0 ** rng.uniform(-9, 2, size=shape[:-1]))
        return c, s

    mc, ms = grid((n, d), 127)
    vc, vs = grid((n, r, d), 7)
    cc, cs = grid((n, P, r), 127)
    mu, vt, cf = mc * ms[:, None], vc * vs[:, :, None], cc * cs[:, :, None]
    qs = oracle.quantize_summaries(mu, vt, cf)
    assert np.array_equal(qs["mu_code"], mc) and np.array_equal(qs["mu_scale"], ms)
    assert np.array_equal(qs["vt_code"], vc) and np.array_equal(qs["vt_scale"], vs)
    assert np.array_equal(qs["coef_code"], cc) and np.array_equal(qs["coef_scale"], cs)
    dmu, dvt, dcf = oracle.dequantize_summaries(qs)
    q = rng.standard_normal((4, d))
    np.testing.assert_array_equal(oracle.page_scores(q, dmu, dvt, dcf, d ** -0.5),
                                  oracle.page_scores(q, mu, vt, cf, d ** -0.5))


def test_quantized_score_within_lipschitz_bound():
    """Log-sum-exp moves by at most the largest logit change, so the quantized
    page score differs from the fitted one by at most
    scale * (|q.(mu'-mu)| + max_i |q.(V'c'_i - V c_i)|), evaluated here on the
    reconstructed keys rather than through V^T q."""
    mu, vt, cf = _fitted(3)
    dmu, dvt, dcf = oracle.dequantize_summaries(oracle.quantize_summaries(mu, vt, cf))
    d = mu.shape[1]
    sc = d ** -0.5
    q = np.random.default_rng(4).standard_normal((4, d))
    s0 = oracle.page_scores(q, mu, vt, cf, sc)
    s1 = oracle.page_scores(q, dmu, dvt, dcf, sc)
    rec0 = np.einsum("nrd,npr->npd", vt, cf)    # V c_i, per page and token
    rec1 = np.einsum("nrd,npr->npd", dvt, dcf)
    for g in range(q.shape[0]):
        bound = sc * (np.abs((dmu - mu) @ q[g]) + np.abs((rec1 - rec0) @ q[g]).max(axis=1))
        assert np.all(np.abs(s1[g] - s0[g]) <= bound * (1 + 1e-9) + 1e-12)
        assert np.any(s1[g] != s0[g])

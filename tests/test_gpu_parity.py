"""GPU parity of the HIP path against the fp64 oracle, stage by stage and end to
end, through the C ABI (liblocks.so). Inputs come from the seeded generator;
stage inputs of the GPU (summaries, page scores, selections) come from the
oracle or the generator, never from an earlier GPU stage.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_kv_page_amd import locks as L
from sparse_kv_page_amd import synth
from tests import gpu_glue as gg

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
TINY = W["tiny_f32"]
W32K = W["llama8b_32k"]
# small bf16 workload for end-to-end checks: ragged batch, partial pages, J > k
E2E = synth.Workload("e2e_bf16", 3, 2, 4, 128, 64, (64 * 40 + 37, 64 * 24, 64 * 9 + 1), 4, 8,
                     "bf16", "bf16", n_needles=3, extra_blocks=5)
# the 128K batch-8 generator (AR(1) centroids, six signal directions, noise,
# needles) at r = 8 on a batch small enough for the oracle to fit every page
HEAD_E2E = synth.Workload("e2e_headline_r8", 2, 8, 4, 128, 64, (64 * 40 + 37, 64 * 33), 8, 8, "bf16", "bf16",
                          centroid_std=0.5, ar_rho=0.99, n_needles=4)
# a common offset of +20 on every key coordinate (large centroid norm)
OFFSET = E2E.with_(name="e2e_offset20_r8", rank=8, key_offset=20.0)
# a slowly decaying spectrum: 16 signal directions with variances 4 * 0.8^i
SLOW = E2E.with_(name="e2e_slow_spectrum_r8", rank=8, basis_var=tuple(4.0 * 0.8 ** i for i in range(16)))


def _cfg(wl):
    return L.config_for(wl)


# --------------------------------------------------------------------------
# (a2) scorer on identical summary bytes
# --------------------------------------------------------------------------
@pytest.mark.parametrize("wl,source", [(TINY, "oracle"), (E2E, "oracle"), (W32K, "synthetic")],
                         ids=["tiny_f32", "e2e_bf16", "llama8b_32k"])
def test_page_score_parity(wl, source):
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=0)
    if source == "oracle":
        summ, _, _ = gg.oracle_summaries(wl, data)
        pool = gg.pool_from_summaries(wl, cfg, summ)
    else:
        pool = gg.synthetic_pool(wl, cfg, seed=0)
    hs = gg.gpu_scores(wl, cfg, g, pool)
    torch.cuda.synchronize()
    hs_c = hs.cpu()
    pool_c = pool.cpu()
    worst = 0.0
    for b in range(wl.batch):
        _, J, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            mu, vt, cf = gg.unit_records(wl, cfg, pool_c, data["block_table"], b, h, Jc)
            ref = gg.oracle_unit_scores(wl, data, b, h, mu, vt, cf)
            got = gg.f64(hs_c[b, h * wl.group:(h + 1) * wl.group, :Jc])
            worst = max(worst, gg.mixed_violation(got, ref))
            # entries past the complete pages are left untouched
            assert torch.isnan(hs_c[b, h * wl.group:(h + 1) * wl.group, Jc:]).all()
    assert worst <= 1.0, f"score violation {worst:.3f} x tolerance"


# --------------------------------------------------------------------------
# (a3+a4) selector on identical page scores
# --------------------------------------------------------------------------
@pytest.mark.parametrize("wl", [TINY, E2E, W32K], ids=["tiny_f32", "e2e_bf16", "llama8b_32k"])
def test_select_parity(wl):
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=1)
    pool = gg.synthetic_pool(wl, cfg, seed=1, device="cpu")
    hs = torch.full((wl.batch, wl.num_q_heads, wl.max_pages), float("nan"), dtype=torch.float32)
    refs = {}
    for b in range(wl.batch):
        _, J, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            mu, vt, cf = gg.unit_records(wl, cfg, pool, data["block_table"], b, h, Jc)
            s = gg.oracle_unit_scores(wl, data, b, h, mu, vt, cf)
            hs[b, h * wl.group:(h + 1) * wl.group, :Jc] = torch.from_numpy(s).float()
            s32 = hs[b, h * wl.group:(h + 1) * wl.group, :Jc].double().numpy()
            refs[(b, h)] = gg.oracle_unit_select(wl, b, s32)
    sel, sig = gg.gpu_select(wl, cfg, g, hs.to(gg.DEV))
    torch.cuda.synchronize()
    sel, sig = sel.cpu(), sig.cpu()
    ndiff = 0
    for (b, h), (sel_o, sigma_o) in refs.items():
        ndiff += gg.check_selection(wl, b, sel[b, h].tolist(), sel_o.tolist(), sigma_o)
        if sigma_o is not None:
            _, J, Jc = gg.lens(wl, b)
            assert gg.mixed_violation(gg.f64(sig[b, h, :Jc]), sigma_o) <= 1.0
    assert ndiff <= 2 * len(refs)


@pytest.mark.parametrize("G,lens", [(4, (64 * 10000 + 5, 64 * 6000)), (8, (64 * 3000 + 17, 64 * 2100)),
                                     (1, (64 * 9000,)), (4, (64 * 5000 + 1, 64 * 40))],
                         ids=["g4_10000_pages", "g8_3000_pages", "g1_9000_pages", "g4_5000_pages"])
def test_select_long_context_paths(G, lens):
    """The selector's long-context kernels (1024 threads with 8 register pages
    up to 8192 pages, 1024 threads re-reading the scores beyond that) for
    G in {1, 4, 8}, on seeded random page scores, against the oracle."""
    wl = synth.Workload("sel_long", len(lens), 2, G, 128, 64, lens, 4, 32, "bf16", "bf16")
    cfg = _cfg(wl)
    gen = torch.Generator().manual_seed(31 + G)
    hs = (torch.randn((wl.batch, wl.num_q_heads, wl.max_pages), generator=gen) * 2.5).float()
    g = {"seq_lens": torch.tensor(list(lens), dtype=torch.int32, device=gg.DEV)}
    sel, sig = gg.gpu_select(wl, cfg, g, hs.to(gg.DEV))
    torch.cuda.synchronize()
    sel, sig = sel.cpu(), sig.cpu()
    ndiff = 0
    for b in range(wl.batch):
        _, J, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            s32 = hs[b, h * G:(h + 1) * G, :Jc].double().numpy()
            sel_o, sigma_o = gg.oracle_unit_select(wl, b, s32)
            ndiff += gg.check_selection(wl, b, sel[b, h].tolist(), sel_o.tolist(), sigma_o)
            if sigma_o is not None:
                assert gg.mixed_violation(gg.f64(sig[b, h, :Jc]), sigma_o) <= 1.0
    assert ndiff <= 2 * wl.batch * wl.num_kv_heads


@pytest.mark.parametrize("G,lens", [(4, (64 * 2000 + 9, 64 * 1500)), (8, (64 * 1800, 64 * 900 + 3)),
                                     (4, (64 * 7000 + 5, 64 * 5000))],
                         ids=["g4_2000_pages", "g8_1800_pages", "g4_7000_pages"])
def test_select_wide_score_spread(G, lens):
    """Pages whose scores sit 100-250 below the head maxima in every head: the
    register paths form sigma from exponentials kept against each wave's
    maximum, and take the per-page-max form where those underflow. Sequence 0
    has a third of its pages that far down (their sigma only is checked);
    sequence 1 keeps 10 pages near the top, so most of its k - 2 slots go to
    pages ranked by the per-page-max form. Sigma and selections against the
    oracle."""
    wl = synth.Workload("sel_spread", len(lens), 2, G, 128, 64, lens, 4, 32, "bf16", "bf16")
    cfg = _cfg(wl)
    gen = torch.Generator().manual_seed(71 + G)
    hs = (torch.randn((wl.batch, wl.num_q_heads, wl.max_pages), generator=gen) * 2.5).float()
    low = torch.rand((wl.batch, wl.max_pages), generator=gen)
    drop = 100.0 + 150.0 * torch.rand((wl.batch, wl.max_pages), generator=gen)
    down0 = low[0] < 1.0 / 3.0
    down1 = torch.ones(wl.max_pages, dtype=torch.bool)
    down1[torch.randperm(wl.max_pages, generator=gen)[:10]] = False
    for b, down in ((0, down0), (1, down1)):
        hs[b, :, down] -= drop[b, down]
    g = {"seq_lens": torch.tensor(list(lens), dtype=torch.int32, device=gg.DEV)}
    sel, sig = gg.gpu_select(wl, cfg, g, hs.to(gg.DEV))
    torch.cuda.synchronize()
    sel, sig = sel.cpu(), sig.cpu()
    ndiff = 0
    for b in range(wl.batch):
        _, J, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            s32 = hs[b, h * G:(h + 1) * G, :Jc].double().numpy()
            sel_o, sigma_o = gg.oracle_unit_select(wl, b, s32)
            ndiff += gg.check_selection(wl, b, sel[b, h].tolist(), sel_o.tolist(), sigma_o)
            assert sigma_o is not None
            assert gg.mixed_violation(gg.f64(sig[b, h, :Jc]), sigma_o) <= 1.0
            assert np.isfinite(gg.f64(sig[b, h, :Jc])).all()
    assert ndiff <= 2 * wl.batch * wl.num_kv_heads


def test_select_ties_go_to_lower_page():
    """Equal keys: the lower page id wins (radix select resolves full 64-bit keys)."""
    wl = E2E.with_(batch=1, seq_lens=(64 * 40,), budget_pages=6)
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=2)
    hs = torch.zeros((1, wl.num_q_heads, wl.max_pages), dtype=torch.float32)
    hs[0, :, [3, 7, 11, 20, 30]] = 1.0    # 5 tied winners for 4 free slots
    hs[0, :, 38] = 5.0                    # page J-1 = 39 is mandatory; 38 wins outright
    sel, _ = gg.gpu_select(wl, cfg, g, hs.to(gg.DEV))
    for h in range(wl.num_kv_heads):
        assert sel[0, h].tolist() == [0, 3, 7, 11, 38, 39]
    # all-equal scores: lowest ids
    hs2 = torch.full((1, wl.num_q_heads, wl.max_pages), -3.25)
    sel2, _ = gg.gpu_select(wl, cfg, g, hs2.to(gg.DEV))
    assert sel2[0, 0].tolist() == [0, 1, 2, 3, 4, 39]


@pytest.mark.parametrize("lens", [(64 * 40 + 7, 64 * 3, 64 * 2, 17), (64 * 2000, 64 * 1 + 1, 64 * 300, 0)],
                         ids=["short", "long"])
def test_select_budget_of_two_pages(lens):
    """k = 2 leaves no free slot: only the sink and the current page are kept
    (and J <= 2 keeps every page), whatever the scores."""
    wl = E2E.with_(batch=len(lens), seq_lens=lens, budget_pages=2, extra_blocks=0)
    cfg = _cfg(wl)
    gen = torch.Generator().manual_seed(57)
    hs = (torch.randn((wl.batch, wl.num_q_heads, wl.max_pages), generator=gen) * 3).float()
    g = {"seq_lens": torch.tensor(list(lens), dtype=torch.int32, device=gg.DEV)}
    sel, _ = gg.gpu_select(wl, cfg, g, hs.to(gg.DEV))
    torch.cuda.synchronize()
    for b in range(wl.batch):
        _, J, Jc = gg.lens(wl, b)
        sel_o, sigma_o = gg.oracle_unit_select(wl, b, hs[b, :, :Jc].double().numpy())
        assert sel_o.tolist() == ([0, J - 1] if J > 2 else [j if j < J else -1 for j in range(2)])
        for h in range(wl.num_kv_heads):
            assert sel[b, h].tolist() == sel_o.tolist()


def _record_pool(wl, cfg, g, page_mu_weight):
    """bf16 summary pool whose record of logical page j has V = 0, C = 0 and
    mu = page_mu_weight[j] * (mean query of the group), so a page's score is
    w_j * (q_g . mean q) * scale + log P: equal weights give bit-equal scores."""
    d, r, P, G = wl.head_dim, wl.rank, wl.page_size, wl.group
    rec_elems = d * (1 + r) + P * r
    pool = torch.zeros((wl.num_blocks, wl.num_kv_heads, rec_elems), dtype=torch.bfloat16)
    q = g["q"].float().cpu()
    bt = g["block_table"].cpu()
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            qbar = q[b, h * G:(h + 1) * G].mean(0)
            for j, w in enumerate(page_mu_weight):
                pool[int(bt[b, j]), h, :d] = (w * qbar).to(torch.bfloat16)
    assert L.locks_summary_record_bytes(cfg) == rec_elems * 2
    return pool.view(torch.uint8).reshape(-1).to(gg.DEV)


def test_score_select_ties_go_to_lower_page():
    """Summary records that score exactly alike: through locks_score_select the
    tied pages go to the lower page ids, as through the separate calls."""
    wl = E2E.with_(batch=1, seq_lens=(64 * 40,), budget_pages=6)
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=2)
    w = [0.0] * wl.max_pages
    for j in (3, 7, 11, 20, 30):
        w[j] = 0.5      # 5 tied winners for 4 free slots
    w[38] = 1.0         # page J-1 = 39 is mandatory; 38 wins outright
    pool = _record_pool(wl, cfg, g, w)
    sel = gg.gpu_score_select(wl, cfg, g, pool)
    hs = gg.gpu_scores(wl, cfg, g, pool)
    sel_s, _ = gg.gpu_select(wl, cfg, g, hs)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel_s)
    for h in range(wl.num_kv_heads):
        assert sel[0, h].tolist() == [0, 3, 7, 11, 38, 39]
    # all pages equal: lowest ids
    pool2 = _record_pool(wl, cfg, g, [0.25] * wl.max_pages)
    sel2 = gg.gpu_score_select(wl, cfg, g, pool2)
    torch.cuda.synchronize()
    for h in range(wl.num_kv_heads):
        assert sel2[0, h].tolist() == [0, 1, 2, 3, 4, 39]


# --------------------------------------------------------------------------
# (a5) sparse decode on the oracle's page selection
# --------------------------------------------------------------------------
@pytest.mark.parametrize("wl", [TINY, E2E, W32K], ids=["tiny_f32", "e2e_bf16", "llama8b_32k"])
def test_sparse_decode_parity(wl):
    _decode_parity(wl)


def _decode_parity(wl):
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=3, gen_device=gg.DEV if wl.batch * wl.num_kv_heads > 64 else "cpu")
    rng = np.random.default_rng(3)
    k = wl.budget_pages
    sel = np.full((wl.batch, wl.num_kv_heads, k), -1, dtype=np.int32)
    for b in range(wl.batch):
        _, J, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            if J <= k:
                sel[b, h, :J] = np.arange(J)
            else:   # a valid selection: sink, current page, k-2 random others
                others = rng.choice(np.arange(1, J - 1), size=k - 2, replace=False)
                sel[b, h] = np.sort(np.concatenate([[0, J - 1], others]))
    out, lse = gg.gpu_decode(wl, cfg, g, torch.from_numpy(sel).to(gg.DEV))
    torch.cuda.synchronize()
    out, lse = gg.f64(out.cpu()), gg.f64(lse.cpu())
    worst_o, worst_l = 0.0, 0.0
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            o_ref, l_ref = gg.oracle_unit_attend(wl, data, b, h, sel[b, h])
            sl = slice(h * wl.group, (h + 1) * wl.group)
            worst_o = max(worst_o, float(np.max(np.abs(out[b, sl] - o_ref))))
            worst_l = max(worst_l, gg.mixed_violation(lse[b, sl], l_ref))
    assert worst_o <= gg.out_tol(wl), worst_o
    assert worst_l <= 1.0, worst_l


@pytest.mark.parametrize("d,G,P", [(128, 4, 64), (64, 4, 16), (128, 8, 32), (64, 1, 64), (128, 2, 16)],
                         ids=["d128-g4-p64", "d64-g4-p16", "d128-g8-p32", "d64-g1-p64", "d128-g2-p16"])
@pytest.mark.parametrize("tiles", [8, 4], ids=["eight-tile", "four-tile"])
def test_sparse_decode_large_workgroups(d, G, P, tiles):
    """Grids of at least 256 workgroups take eight or four 16-token tiles per
    wave (K staged through LDS): 256 units at k = 8 pages give eight, 128
    units at k = 1024 / P pages four. Ragged lengths, partial current pages
    and J <= k units, against the oracle."""
    Hkv = 8
    B, k = (32, 8) if tiles == 8 else (16, 1024 // P)
    lens = tuple(P * (3 + (7 * b) % 37) + (b * 5) % P for b in range(B))
    wl = synth.Workload(f"large_wg_d{d}_g{G}_p{P}_t{tiles}", B, Hkv, G, d, P, lens, 2, k, "bf16", "bf16")
    _decode_parity(wl)


@pytest.mark.parametrize("k", [8, 32, 40, 136, 264],
                         ids=["2-splits", "4-splits", "5-splits", "9-splits", "17-splits"])
def test_sparse_decode_split_merge_runs(k):
    """The last workgroup of a unit folds the split partials in runs of 4
    loads when a unit has at most 4 splits, else in runs of 16. At batch 8
    with 8 KV heads and 64-token pages the budgets give 2 splits (two tiles
    per wave), 4 and 5 splits (four tiles per wave), 9 splits (eight tiles
    per wave: one run of 16, 7 loads past the end) and 17 splits (two runs,
    the second mostly past the end). One short sequence has J <= k."""
    B, Hkv, G, d, P = 8, 8, 4, 128, 64
    lens = tuple(P * (k + 3 + (7 * b) % 29) + (b * 5) % P for b in range(B - 1)) + (P * 3 + 17,)
    wl = synth.Workload(f"split_runs_k{k}", B, Hkv, G, d, P, lens, 2, k, "bf16", "bf16")
    _decode_parity(wl)


def test_full_budget_decode_is_dense():
    """k >= J: every page is selected and the result is dense decode attention."""
    wl = E2E.with_(budget_pages=64)
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=4)
    pool = gg.synthetic_pool(wl, cfg, seed=4)
    sel = gg.gpu_score_select(wl, cfg, g, pool)
    out, _ = gg.gpu_decode(wl, cfg, g, sel)
    torch.cuda.synchronize()
    out = gg.f64(out.cpu())
    for b in range(wl.batch):
        T, J, _ = gg.lens(wl, b)
        assert sel[b, 0].tolist() == list(range(J)) + [-1] * (64 - J)
        for h in range(wl.num_kv_heads):
            G = wl.group
            bt = data["block_table"][b, :J].long()
            keys = gg.f64(data["k_pool"][bt, h].reshape(-1, wl.head_dim)[:T])
            vals = gg.f64(data["v_pool"][bt, h].reshape(-1, wl.head_dim)[:T])
            o_ref, _ = oracle.attend(gg.f64(data["q"][b, h * G:(h + 1) * G]), keys, vals,
                                     wl.softmax_scale)
            assert np.max(np.abs(out[b, h * G:(h + 1) * G] - o_ref)) <= gg.out_tol(wl)


# --------------------------------------------------------------------------
# (a1) summary build
# --------------------------------------------------------------------------
@pytest.mark.parametrize("wl,npages", [(TINY, None), (E2E, 48), (W32K, 48), (HEAD_E2E, 64), (OFFSET, 48),
                                       (SLOW, 48)],
                         ids=["tiny_f32", "e2e_bf16", "llama8b_32k", "headline_gen_r8", "offset20_r8",
                              "slow_spectrum_r8"])
def test_build_parity(wl, npages):
    """The GPU fit against the oracle's on every (or a sample of) complete
    page: the stored centroid is the rounded mean, the stored basis is
    orthonormal, C = D V for the stored V, the span attains the Eckart-Young
    residual, and every leading subspace the spectrum separates is the
    oracle's ([Locks] §4, App. A.2 Cor. 1; any basis of a subspace is valid)."""
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=5)
    pool = gg.gpu_build(wl, cfg, g)
    torch.cuda.synchronize()
    pool_c = pool.cpu()
    mu_g, vt_g, cf_g = L.split_records(cfg, pool_c)
    pages = []
    for b in range(wl.batch):
        _, _, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            pages += [(int(data["block_table"][b, j]), h) for j in range(Jc)]
    if npages is not None:
        rng = np.random.default_rng(5)
        pages = [pages[i] for i in sorted(rng.choice(len(pages), npages, replace=False))]
    summ, raw, keys = gg.oracle_summaries(wl, data, pages)
    bf = wl.summary_dtype == "bf16"
    r = wl.rank
    checked = 0
    for i, (blk, h) in enumerate(pages):
        mu_o, vt_o, cf_o, ev = raw[(blk, h)]
        K = keys[i]
        D = K - mu_o
        mu = gg.f64(mu_g[blk, h]); vt = gg.f64(vt_g[blk, h]); cf = gg.f64(cf_g[blk, h])
        # centroid: the rounded mean (one storage ulp)
        ulp = 2.0 ** -7 if bf else 1e-6
        assert np.all(np.abs(mu - mu_o) <= ulp * np.maximum(np.abs(mu_o), 1e-3) + 1e-7)
        # orthonormal basis (up to storage rounding)
        assert np.max(np.abs(vt @ vt.T - np.eye(r))) <= (2e-2 if bf else 1e-5)
        # C = D V for the stored V (up to storage rounding)
        scale_c = max(1.0, np.max(np.abs(cf_o)))
        assert np.max(np.abs(cf - D @ vt.T)) <= (3e-2 if bf else 1e-4) * scale_c
        checked += gg.check_fit(K, vt, ev, vt_o, r, *(() if bf else (1e-6, 1e-4)))
    # the signal directions are well separated on most pages
    assert checked >= len(pages) * min(r, 3)


@pytest.mark.parametrize("wl", [TINY, E2E, HEAD_E2E, OFFSET, SLOW, E2E.with_(page_size=32, rank=4),
                                E2E.with_(page_size=16, rank=8, budget_pages=24), E2E.with_(head_dim=64, rank=15)],
                         ids=["tiny_f32", "e2e_bf16", "headline_gen_r8", "offset20_r8", "slow_spectrum_r8",
                              "p32_r4", "p16_r8", "d64_r15"])
def test_build_fit_report(wl):
    """Every fit meets the Ritz residual bound (locks_build_summaries_ex
    reports a positive product count), P = 16 pages in one step, and the
    report-free entry point writes the same records byte for byte."""
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=8)
    fits = []
    pool = gg.gpu_build(wl, cfg, g, fits=fits)
    ids = torch.cat([g["block_table"][b, :gg.lens(wl, b)[2]] for b in range(wl.batch)]).contiguous()
    pool2 = torch.zeros_like(pool)
    L.locks_build_summaries(cfg, g["k_pool"], wl.num_blocks, ids, ids.numel(), pool2)
    torch.cuda.synchronize()
    assert torch.equal(pool.view(torch.uint8), pool2.view(torch.uint8))
    counts = np.bincount(np.asarray(fits))
    print(f"[fit report] {wl.name}: products per tile {dict((i, int(c)) for i, c in enumerate(counts) if c)}")
    if wl.page_size == 16:
        assert set(fits) == {1}
    else:
        assert max(fits) < 32


@pytest.mark.parametrize("rank,noise", [(15, 0.2), (5, 0.0)], ids=["r15_noisy", "r5_noise_free"])
def test_full_rank_reconstruction_equals_exact_lse(rank, noise):
    """r >= rank(D): the GPU-built summaries reproduce the exact page LSE
    ([Locks] Thm. 1(i), eta = 0) and the selection equals the exact-LSE set.
    r = P - 1 covers any page; r = 5 covers the noise-free keys of the tiny
    workload, whose centred pages have rank 4."""
    wl = TINY.with_(rank=rank, noise=noise)
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=6)
    pool = gg.gpu_build(wl, cfg, g)
    hs = gg.gpu_scores(wl, cfg, g, pool)
    sel, _ = gg.gpu_select(wl, cfg, g, hs)
    torch.cuda.synchronize()
    T, J, Jc = gg.lens(wl, 0)
    bt = data["block_table"][0, :Jc].long()
    keys = gg.f64(data["k_pool"][bt, 0])
    q = gg.f64(data["q"][0])
    s_exact = oracle.exact_page_lse(q, keys, wl.softmax_scale)
    assert gg.mixed_violation(gg.f64(hs[0, :, :Jc].cpu()), s_exact) <= 1.0
    sel_o, sigma_o = gg.oracle_unit_select(wl, 0, s_exact)
    gg.check_selection(wl, 0, sel[0, 0].tolist(), sel_o.tolist(), sigma_o)


# --------------------------------------------------------------------------
# end to end: build -> score -> select -> decode on the GPU vs the oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("wl", [TINY, E2E, HEAD_E2E], ids=["tiny_f32", "e2e_bf16", "headline_gen_r8"])
def test_end_to_end(wl):
    """GPU build -> GPU score -> GPU select -> GPU decode against oracle build
    -> oracle score -> oracle select -> oracle attend, every unit: scores of
    the two chains within the score bar, selections equal under the window
    rule, outputs on equal selections within the output bar. (Two valid fits
    round their coefficients to bf16 independently; with a large common key
    offset a needle token's coefficient is in the hundreds, where one bf16
    step moves its logit past the score bar, so the offset pages are checked
    on the fit itself in test_build_parity instead.)"""
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=7)
    pool = gg.gpu_build(wl, cfg, g)
    hs = gg.gpu_scores(wl, cfg, g, pool)
    sel, _ = gg.gpu_select(wl, cfg, g, hs)
    sel_c = gg.gpu_score_select(wl, cfg, g, pool)
    out, _ = gg.gpu_decode(wl, cfg, g, sel)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel_c)  # the fused entry point matches the two stages
    summ, _, _ = gg.oracle_summaries(wl, data)
    hs, sel, out = hs.cpu(), sel.cpu(), gg.f64(out.cpu())
    same = 0
    units = 0
    for b in range(wl.batch):
        _, J, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            units += 1
            blocks = [int(x) for x in data["block_table"][b, :Jc]]
            mu = np.stack([summ[(x, h)][0] for x in blocks])
            vt = np.stack([summ[(x, h)][1] for x in blocks])
            cf = np.stack([summ[(x, h)][2] for x in blocks])
            s_o = gg.oracle_unit_scores(wl, data, b, h, mu, vt, cf)
            assert gg.mixed_violation(gg.f64(hs[b, h * wl.group:(h + 1) * wl.group, :Jc]), s_o) <= 1.0
            sel_o, sigma_o = gg.oracle_unit_select(wl, b, s_o)
            nd = gg.check_selection(wl, b, sel[b, h].tolist(), sel_o.tolist(), sigma_o)
            if nd == 0:
                same += 1
                o_ref, _ = gg.oracle_unit_attend(wl, data, b, h, sel_o)
                sl = slice(h * wl.group, (h + 1) * wl.group)
                assert np.max(np.abs(out[b, sl] - o_ref)) <= gg.out_tol(wl)
    assert same >= units - 1


# --------------------------------------------------------------------------
# shapes: group sizes, head dims, page sizes, ranks (generic-rank kernels too)
# --------------------------------------------------------------------------
VARIANTS = [
    dict(group=1, head_dim=128, page_size=64, rank=8),
    dict(group=2, head_dim=64, page_size=32, rank=3),
    dict(group=8, head_dim=128, page_size=16, rank=5),
    dict(group=4, head_dim=64, page_size=16, rank=1),
    dict(group=4, head_dim=128, page_size=32, rank=2, kv_dtype="f32", summary_dtype="f32"),
]


@pytest.mark.parametrize("kw", VARIANTS, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
def test_shape_variants(kw):
    P = kw["page_size"]
    wl = synth.Workload("variant", 2, 2, kw["group"], kw["head_dim"], P, (P * 21 + 3, P * 12),
                        kw["rank"], 6, kw.get("kv_dtype", "bf16"), kw.get("summary_dtype", "bf16"),
                        n_needles=2)
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=8)
    summ, _, _ = gg.oracle_summaries(wl, data)
    pool = gg.pool_from_summaries(wl, cfg, summ)
    hs = gg.gpu_scores(wl, cfg, g, pool)
    # selector on the oracle's scores rounded to fp32; decode on the oracle's selection
    hs_o = torch.full_like(hs.cpu(), float("nan"))
    sel_o_all = torch.full((wl.batch, wl.num_kv_heads, wl.budget_pages), -1, dtype=torch.int32)
    refs = {}
    for b in range(wl.batch):
        _, J, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            blocks = [int(x) for x in data["block_table"][b, :Jc]]
            mu = np.stack([summ[(x, h)][0] for x in blocks])
            vt = np.stack([summ[(x, h)][1] for x in blocks])
            cf = np.stack([summ[(x, h)][2] for x in blocks])
            s_o = gg.oracle_unit_scores(wl, data, b, h, mu, vt, cf)
            sl = slice(h * wl.group, (h + 1) * wl.group)
            assert gg.mixed_violation(gg.f64(hs[b, sl, :Jc].cpu()), s_o) <= 1.0
            hs_o[b, sl, :Jc] = torch.from_numpy(s_o).float()
            s32 = hs_o[b, sl, :Jc].double().numpy()
            sel_o, sigma_o = gg.oracle_unit_select(wl, b, s32)
            refs[(b, h)] = (sel_o, sigma_o)
            sel_o_all[b, h] = torch.from_numpy(sel_o)
    sel, _ = gg.gpu_select(wl, cfg, g, hs_o.to(gg.DEV))
    out, _ = gg.gpu_decode(wl, cfg, g, sel_o_all.to(gg.DEV))
    torch.cuda.synchronize()
    sel, out = sel.cpu(), gg.f64(out.cpu())
    for (b, h), (sel_o, sigma_o) in refs.items():
        gg.check_selection(wl, b, sel[b, h].tolist(), sel_o.tolist(), sigma_o)
        o_ref, _ = gg.oracle_unit_attend(wl, data, b, h, sel_o)
        sl = slice(h * wl.group, (h + 1) * wl.group)
        assert np.max(np.abs(out[b, sl] - o_ref)) <= gg.out_tol(wl)


# --------------------------------------------------------------------------
# edge cases and robustness
# --------------------------------------------------------------------------
def test_edge_lengths():
    """Empty, one-token, exactly-k, k+1 pages, partial pages; max_pages > needed."""
    P, k = 64, 4
    lens_ = (0, 1, 63, 64, 65, P * k, P * k + 1, P * (k + 1), P * 9 + 17)
    wl = synth.Workload("edges", len(lens_), 2, 4, 128, P, lens_, 4, k, "bf16", "bf16",
                        extra_blocks=3)
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=9)
    pool = gg.synthetic_pool(wl, cfg, seed=9)
    sel = gg.gpu_score_select(wl, cfg, g, pool)
    out, lse = gg.gpu_decode(wl, cfg, g, sel)
    torch.cuda.synchronize()
    sel, out, lse = sel.cpu(), gg.f64(out.cpu()), gg.f64(lse.cpu())
    pool_c = pool.cpu()
    for b, T in enumerate(lens_):
        _, J, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            if J > k:
                mu, vt, cf = gg.unit_records(wl, cfg, pool_c, data["block_table"], b, h, Jc)
                s_o = gg.oracle_unit_scores(wl, data, b, h, mu, vt, cf)
            else:
                s_o = None
            sel_o, sigma_o = gg.oracle_unit_select(wl, b, s_o)
            gg.check_selection(wl, b, sel[b, h].tolist(), sel_o.tolist(), sigma_o)
            sl = slice(h * wl.group, (h + 1) * wl.group)
            if T == 0:
                assert np.all(out[b, sl] == 0) and np.all(np.isneginf(lse[b, sl]))
                continue
            if sel[b, h].tolist() == sel_o.tolist():
                o_ref, _ = gg.oracle_unit_attend(wl, data, b, h, sel_o)
                assert np.max(np.abs(out[b, sl] - o_ref)) <= gg.out_tol(wl)


def test_invalid_block_ids_are_skipped():
    """A block id outside the pool scores -inf and is never chosen; decode skips it."""
    wl = E2E.with_(batch=1, seq_lens=(64 * 30,))
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=10)
    g["block_table"][0, 5] = -1
    g["block_table"][0, 6] = wl.num_blocks + 100
    pool = gg.synthetic_pool(wl, cfg, seed=10)
    hs = gg.gpu_scores(wl, cfg, g, pool)
    sel, _ = gg.gpu_select(wl, cfg, g, hs)
    torch.cuda.synchronize()
    assert torch.isneginf(hs[0, :, 5]).all() and torch.isneginf(hs[0, :, 6]).all()
    assert torch.isfinite(hs[0, :, :30][:, [j for j in range(30) if j not in (5, 6)]]).all()
    for h in range(wl.num_kv_heads):
        assert 5 not in sel[0, h].tolist() and 6 not in sel[0, h].tolist()
    # a selection naming the bad pages attends the remaining ones only
    bad = torch.tensor([[[0, 5, 6, 9, 12, 15, 20, 29]] * wl.num_kv_heads], dtype=torch.int32)
    good = torch.tensor([[[0, -1, -1, 9, 12, 15, 20, 29]] * wl.num_kv_heads], dtype=torch.int32)
    o1, _ = gg.gpu_decode(wl, cfg, g, bad.to(gg.DEV))
    o2, _ = gg.gpu_decode(wl, cfg, g, good.to(gg.DEV))
    assert torch.equal(o1, o2)


def test_deterministic_repeats():
    wl = E2E
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=11)
    res = []
    for _ in range(3):
        pool = gg.gpu_build(wl, cfg, g)
        hs = gg.gpu_scores(wl, cfg, g, pool)
        sel, sig = gg.gpu_select(wl, cfg, g, hs)
        out, lse = gg.gpu_decode(wl, cfg, g, sel)
        torch.cuda.synchronize()
        res.append([t.cpu() for t in (pool, hs, sel, out, lse)])
    for other in res[1:]:
        for a, b in zip(res[0], other):
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


# --------------------------------------------------------------------------
# 128K context, batch 8, r = 8: every unit at full size
# --------------------------------------------------------------------------
def _fit_sample(wl, cfg, d, pool, sample):
    """check_fit on sampled (block, head) tiles of a GPU-built pool; returns the
    number of separated leading subspaces checked."""
    keys = np.stack([gg.f64(d["k_pool"][blk, h].cpu()) for blk, h in sample])
    _, vt_o, _, ev, _ = oracle.build_pages(keys, wl.rank)
    recs = pool[torch.tensor([x for x, _ in sample], device=gg.DEV),
                torch.tensor([y for _, y in sample], device=gg.DEV)].cpu()
    _, vt_g, _ = L.split_records(cfg, recs)
    return sum(gg.check_fit(keys[i], gg.f64(vt_g[i]), ev[i], vt_o[i], wl.rank) for i in range(len(sample)))


def test_128k_b8_all_units():
    """Every (sequence, KV head) unit of the 128K-context batch of 8 at r = 8,
    in the launch configuration bench.py times: page scores element by element
    and the selection (window rule) against the oracle on identical records,
    the attention output of every unit on the oracle's selection, and the
    full-size build on sampled tiles (Eckart-Young residual, separated
    leading subspaces)."""
    wl = W["llama8b_128k_b8"]
    cfg = _cfg(wl)
    d = synth.generate(wl, 0, gg.DEV)
    pool = gg.synthetic_pool(wl, cfg, seed=0)
    hs = gg.gpu_scores(wl, cfg, d, pool)
    sel = gg.gpu_score_select(wl, cfg, d, pool)
    torch.cuda.synchronize()
    data_c = {"q": d["q"].cpu(), "block_table": d["block_table"].cpu()}
    pool_c = pool.cpu()
    mu_c, vt_c, cf_c = L.split_records(cfg, pool_c)
    bt_c = data_c["block_table"]

    def unit_summaries(b, h, Jc):
        idx = bt_c[b, :Jc].long()
        return gg.f64(mu_c[idx, h]), gg.f64(vt_c[idx, h]), gg.f64(cf_c[idx, h])

    sel_o, ndiff = gg.check_all_units(wl, data_c, hs.cpu(), sel.cpu(), unit_summaries)
    assert ndiff <= wl.batch * wl.num_kv_heads
    del pool_c, mu_c, vt_c, cf_c
    out, _ = gg.gpu_decode(wl, cfg, d, sel_o.to(gg.DEV))
    torch.cuda.synchronize()
    gg.check_all_outputs(wl, d, out.cpu(), sel_o)
    # build at full size: every page of every unit, sampled tiles against the oracle
    ids = d["block_table"].reshape(-1).contiguous()
    pool2 = L.summary_pool_for(cfg, wl.num_blocks, gg.DEV)
    L.locks_build_summaries(cfg, d["k_pool"], wl.num_blocks, ids, ids.numel(), pool2)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    sample = [(int(bt_c[b, j]), int(h)) for b, j, h in zip(rng.integers(0, 8, 16),
                                                            rng.integers(0, 2048, 16),
                                                            rng.integers(0, 8, 16))]
    assert _fit_sample(wl, cfg, d, pool2, sample) >= len(sample) * 4


# --------------------------------------------------------------------------
# long-context stress (one 512K-token sequence, J = 8192, r in {2, 4, 8}):
# the whole step on GPU-built summaries, sampled units against the oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("rank", [2, 4, 8])
def test_stress_512k_sampled(rank):
    wl = W["llama8b_512k"].with_(rank=rank)
    cfg = _cfg(wl)
    d = synth.generate(wl, 0, gg.DEV)
    ids = d["block_table"].reshape(-1).contiguous()
    pool = L.summary_pool_for(cfg, wl.num_blocks, gg.DEV)
    L.locks_build_summaries(cfg, d["k_pool"], wl.num_blocks, ids, ids.numel(), pool)
    hs = gg.gpu_scores(wl, cfg, d, pool)
    sel, out, lse = gg.gpu_decode_step(wl, cfg, d, pool)
    torch.cuda.synchronize()
    T, J, Jc = gg.lens(wl, 0)
    bt_c = d["block_table"].cpu()
    q_c = d["q"].cpu()
    out_c, sel_c = gg.f64(out.cpu()), sel.cpu()
    G = wl.group
    idx = bt_c[0, :Jc].long().to(gg.DEV)
    for h in (1, 6):
        rec = pool[idx, h].cpu()
        mu, vt, cf = (gg.f64(x) for x in L.split_records(cfg, rec))
        s_o = oracle.page_scores(gg.f64(q_c[0, h * G:(h + 1) * G]), mu, vt, cf, wl.softmax_scale)
        assert gg.mixed_violation(gg.f64(hs[0, h * G:(h + 1) * G, :Jc].cpu()), s_o) <= 1.0
        sel_o, sigma_o = gg.oracle_unit_select(wl, 0, s_o)
        gg.check_selection(wl, 0, sel_c[0, h].tolist(), sel_o.tolist(), sigma_o)
        # attention over the GPU's own selection
        ks, vs = [], []
        for j in sel_c[0, h].tolist():
            if j < 0:
                continue
            nv = min(wl.page_size, T - j * wl.page_size)
            blk = int(bt_c[0, j])
            ks.append(gg.f64(d["k_pool"][blk, h, :nv].cpu()))
            vs.append(gg.f64(d["v_pool"][blk, h, :nv].cpu()))
        o_ref, _ = oracle.attend(gg.f64(q_c[0, h * G:(h + 1) * G]), np.concatenate(ks), np.concatenate(vs),
                                 wl.softmax_scale)
        assert np.max(np.abs(out_c[0, h * G:(h + 1) * G] - o_ref)) <= gg.out_tol(wl)
    # build: sampled tiles against the oracle's fit (Eckart-Young residual,
    # separated leading subspaces)
    rng = np.random.default_rng(rank)
    sample = [(int(bt_c[0, j]), int(h)) for j, h in zip(rng.integers(0, Jc, 8), rng.integers(0, 8, 8))]
    assert _fit_sample(wl, cfg, d, pool, sample) >= len(sample) * min(rank, 4)


# --------------------------------------------------------------------------
# 128K context, batch 8 with 16-token pages (k = 128 pages), r in {1, 2, 4, 8}:
# the whole step on GPU-built summaries, sampled units against the oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("rank", [1, 2, 4, 8])
def test_p16_rank_sweep_sampled(rank):
    wl = W["llama8b_128k_b8_p16"].with_(rank=rank)
    cfg = _cfg(wl)
    d = synth.generate(wl, 0, gg.DEV)
    ids = d["block_table"].reshape(-1).contiguous()
    pool = L.summary_pool_for(cfg, wl.num_blocks, gg.DEV)
    L.locks_build_summaries(cfg, d["k_pool"], wl.num_blocks, ids, ids.numel(), pool)
    hs = gg.gpu_scores(wl, cfg, d, pool)
    sel, out, lse = gg.gpu_decode_step(wl, cfg, d, pool)
    torch.cuda.synchronize()
    bt_c = d["block_table"].cpu()
    q_c = d["q"].cpu()
    out_c, sel_c = gg.f64(out.cpu()), sel.cpu()
    G, P = wl.group, wl.page_size
    for (b, h) in ((0, 2), (5, 7)):
        T, J, Jc = gg.lens(wl, b)
        idx = bt_c[b, :Jc].long().to(gg.DEV)
        rec = pool[idx, h].cpu()
        mu, vt, cf = (gg.f64(x) for x in L.split_records(cfg, rec))
        qg = gg.f64(q_c[b, h * G:(h + 1) * G])
        s_o = oracle.page_scores(qg, mu, vt, cf, wl.softmax_scale)
        assert gg.mixed_violation(gg.f64(hs[b, h * G:(h + 1) * G, :Jc].cpu()), s_o) <= 1.0
        sel_o, sigma_o = gg.oracle_unit_select(wl, b, s_o)
        gg.check_selection(wl, b, sel_c[b, h].tolist(), sel_o.tolist(), sigma_o)
        ks, vs = [], []
        for j in sel_c[b, h].tolist():
            if j < 0:
                continue
            nv = min(P, T - j * P)
            blk = int(bt_c[b, j])
            ks.append(gg.f64(d["k_pool"][blk, h, :nv].cpu()))
            vs.append(gg.f64(d["v_pool"][blk, h, :nv].cpu()))
        o_ref, _ = oracle.attend(qg, np.concatenate(ks), np.concatenate(vs), wl.softmax_scale)
        assert np.max(np.abs(out_c[b, h * G:(h + 1) * G] - o_ref)) <= gg.out_tol(wl)
    # build: sampled tiles against the oracle's fit (Eckart-Young residual,
    # separated leading subspaces)
    rng = np.random.default_rng(10 + rank)
    sample = [(int(bt_c[b, j]), int(h)) for b, j, h in zip(rng.integers(0, 8, 8), rng.integers(0, 8192, 8),
                                                            rng.integers(0, 8, 8))]
    assert _fit_sample(wl, cfg, d, pool, sample) >= len(sample) * min(rank, 3) * 3 // 4


# --------------------------------------------------------------------------
# whole decode step (score/select then decode on one workspace) vs the oracle
# and the stages
# --------------------------------------------------------------------------
# a ragged batch: partial current pages, a sequence with J <= k and one with a
# single page
RAGGED = synth.Workload("ragged_bf16", 5, 2, 4, 128, 64,
                       (64 * 40 + 37, 64 * 24, 64 * 9 + 1, 64 * 5, 17), 8, 8, "bf16", "bf16",
                       n_needles=3, extra_blocks=4)


def test_decode_step_end_to_end():
    wl = RAGGED
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=21)
    summ, _, _ = gg.oracle_summaries(wl, data)
    pool = gg.pool_from_summaries(wl, cfg, summ)
    sel, out, lse = gg.gpu_decode_step(wl, cfg, g, pool)
    torch.cuda.synchronize()
    sel, out, lse = sel.cpu(), gg.f64(out.cpu()), gg.f64(lse.cpu())
    same = units = 0
    for b in range(wl.batch):
        _, J, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            units += 1
            if J > wl.budget_pages:
                blocks = [int(x) for x in data["block_table"][b, :Jc]]
                mu = np.stack([summ[(x, h)][0] for x in blocks])
                vt = np.stack([summ[(x, h)][1] for x in blocks])
                cf = np.stack([summ[(x, h)][2] for x in blocks])
                s_o = gg.oracle_unit_scores(wl, data, b, h, mu, vt, cf)
            else:
                s_o = None
            sel_o, sigma_o = gg.oracle_unit_select(wl, b, s_o)
            if gg.check_selection(wl, b, sel[b, h].tolist(), sel_o.tolist(), sigma_o) == 0:
                same += 1
                o_ref, lse_ref = gg.oracle_unit_attend(wl, data, b, h, sel_o)
                sl = slice(h * wl.group, (h + 1) * wl.group)
                assert np.max(np.abs(out[b, sl] - o_ref)) <= gg.out_tol(wl)
                assert np.max(np.abs(lse[b, sl] - lse_ref)) <= 1e-3 * max(1.0, float(np.max(np.abs(lse_ref))))
    assert same >= units - 1


@pytest.mark.parametrize("wl", [RAGGED, W["llama8b_128k_b8"], W["llama8b_512k"].with_(rank=8)],
                         ids=["ragged_bf16", "llama8b_128k_b8", "llama8b_512k_r8"])
def test_decode_step_matches_stages(wl):
    """The step equals locks_score_select then locks_sparse_decode, bit for bit."""
    cfg = _cfg(wl)
    d = synth.generate(wl, 4, gg.DEV)
    pool = gg.synthetic_pool(wl, cfg, seed=4)
    sel_f, out_f, lse_f = gg.gpu_decode_step(wl, cfg, d, pool)
    sel_s = gg.gpu_score_select(wl, cfg, d, pool)
    out_s, lse_s = gg.gpu_decode(wl, cfg, d, sel_s)
    torch.cuda.synchronize()
    assert torch.equal(sel_f, sel_s)
    assert torch.equal(out_f.view(torch.uint8), out_s.view(torch.uint8))
    assert torch.equal(lse_f, lse_s)


def test_decode_step_repeats_and_resets():
    """Counters and flags return to zero: repeated calls on one workspace give
    bitwise identical results, also after a call with a different batch."""
    wl = RAGGED
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=22)
    pool = gg.synthetic_pool(wl, cfg, seed=22)
    nbytes = L.locks_workspace_size(cfg, wl.batch, wl.max_pages)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=gg.DEV)
    ref = gg.gpu_decode_step(wl, cfg, g, pool, ws)
    # same pool (num_blocks) for the smaller batch
    small = wl.with_(batch=2, seq_lens=wl.seq_lens[:2], extra_blocks=wl.num_blocks - 2 * wl.max_pages)
    g2 = dict(g, block_table=g["block_table"][:2].contiguous(), seq_lens=g["seq_lens"][:2].contiguous(),
              q=g["q"][:2].contiguous())
    for it in range(3):
        got = gg.gpu_decode_step(wl, cfg, g, pool, ws)
        got_small = gg.gpu_decode_step(small, cfg, g2, pool, ws)
        torch.cuda.synchronize()
        for a_, b_ in zip(ref, got):
            assert torch.equal(a_.contiguous().view(torch.uint8), b_.contiguous().view(torch.uint8))
        assert torch.equal(got_small[0], ref[0][:2])
        assert torch.equal(got_small[1], ref[1][:2])
    # control words are back to zero (first bytes of the workspace)
    assert int(ws[:256].count_nonzero()) == 0


def test_decode_step_shares_workspace_with_stages():
    """The staged entry points write only scratch: staged calls and fused
    steps interleaved on one workspace give the results of each alone, and
    the control words stay zero between calls."""
    wl = RAGGED
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=24)
    pool = gg.synthetic_pool(wl, cfg, seed=24)
    ref_f = gg.gpu_decode_step(wl, cfg, g, pool)
    ref_sel = gg.gpu_score_select(wl, cfg, g, pool)
    ref_out, ref_lse = gg.gpu_decode(wl, cfg, g, ref_sel)
    torch.cuda.synchronize()
    nbytes = L.locks_workspace_size(cfg, wl.batch, wl.max_pages)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=gg.DEV)
    ctl = wl.batch * wl.num_kv_heads * 4
    for it in range(2):
        sel = gg.gpu_score_select(wl, cfg, g, pool, ws)
        out, lse = gg.gpu_decode(wl, cfg, g, sel, ws)
        got_f = gg.gpu_decode_step(wl, cfg, g, pool, ws)
        torch.cuda.synchronize()
        assert torch.equal(sel, ref_sel)
        assert torch.equal(out.view(torch.uint8), ref_out.view(torch.uint8))
        assert torch.equal(lse, ref_lse)
        for a_, b_ in zip(ref_f, got_f):
            assert torch.equal(a_.contiguous().view(torch.uint8), b_.contiguous().view(torch.uint8))
        assert int(ws[:ctl].count_nonzero()) == 0


@pytest.mark.parametrize("wl", [RAGGED, W["llama8b_128k_b8"]], ids=["ragged_bf16", "llama8b_128k_b8"])
def test_decode_step_graph_replay(wl):
    """The step only enqueues kernels (no allocation, memset or sync), so it
    can be captured into a HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager step bit for bit."""
    cfg = _cfg(wl)
    d = synth.generate(wl, 5, gg.DEV)
    pool = gg.synthetic_pool(wl, cfg, seed=5)
    ref = gg.gpu_decode_step(wl, cfg, d, pool)
    torch.cuda.synchronize()
    nbytes = L.locks_workspace_size(cfg, wl.batch, wl.max_pages)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=gg.DEV)
    sel = torch.empty_like(ref[0])
    out = torch.empty_like(ref[1])
    lse = torch.empty_like(ref[2])

    def step():
        L.locks_decode_step(cfg, d["q"], pool, d["k_pool"], d["v_pool"], wl.num_blocks, d["block_table"],
                            d["seq_lens"], wl.batch, wl.max_pages, sel, out, lse, ws, nbytes)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(4):
        sel.fill_(-7)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, ref[0])
        assert torch.equal(out.view(torch.uint8), ref[1].view(torch.uint8))
        assert torch.equal(lse, ref[2])
    # the control words are back to zero after the replays
    assert int(ws[:4 * wl.batch * wl.num_kv_heads].count_nonzero()) == 0


def test_decode_step_large_budget():
    """A large budget (260 pages of 16, over 33 decode splits) gives exactly
    the staged results."""
    wl = synth.Workload("budget_260", 2, 1, 4, 64, 16, (16 * 300 + 5, 16 * 280), 4, 260, "bf16", "bf16",
                        n_needles=2)
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=23)
    pool = gg.synthetic_pool(wl, cfg, seed=23)
    sel_f, out_f, _ = gg.gpu_decode_step(wl, cfg, g, pool)
    sel_s = gg.gpu_score_select(wl, cfg, g, pool)
    out_s, _ = gg.gpu_decode(wl, cfg, g, sel_s)
    torch.cuda.synchronize()
    assert torch.equal(sel_f, sel_s)
    assert torch.equal(out_f, out_s)


# --------------------------------------------------------------------------
# K/V held in pinned host memory (the capacity use of [Locks] §5: only the
# selected pages cross the host link); the decode reads them in place
# --------------------------------------------------------------------------
def test_decode_with_host_resident_kv():
    wl = E2E
    cfg = _cfg(wl)
    data, g = gg.make_inputs(wl, seed=13)
    pool = gg.gpu_build(wl, cfg, g)
    ref_sel, ref_out, ref_lse = gg.gpu_decode_step(wl, cfg, g, pool)
    kh, kdev = gg.host_pool(data["k_pool"])
    vh, vdev = gg.host_pool(data["v_pool"])
    gh = dict(g, k_pool=kdev, v_pool=vdev)
    sel, out, lse = gg.gpu_decode_step(wl, cfg, gh, pool)
    out2, lse2 = gg.gpu_decode(wl, cfg, gh, ref_sel)
    torch.cuda.synchronize()
    assert torch.equal(sel, ref_sel)
    assert torch.equal(out.view(torch.uint16), ref_out.view(torch.uint16))
    assert torch.equal(lse, ref_lse)
    assert torch.equal(out2.view(torch.uint16), ref_out.view(torch.uint16))
    del kh, vh


# --------------------------------------------------------------------------
# the whole-model step at its full size: 32 layers x 16 sequences of ~64K
# tokens (all layers' K/V in one ~138 GB pool, block offsets past 4 GiB),
# r = 4, k = 32, keys from the low-rank generator. One step (every layer's
# decode step, the build of the pages the step's token completes, the length
# increment) is captured into one HIP graph and replayed step after step;
# after every replay sampled (layer, sequence, KV head) units are checked
# against the oracle, and the pages built inside the graph against the
# oracle's fit.
# --------------------------------------------------------------------------
FULL_STEPS = 16


def full_step_graph(cfg, inp, spool, seq, sel, out, lse, ws, ws_bytes, step_idx, ids_buf):
    """The step function that is captured: every layer's locks_decode_step,
    the build of the page this step's token completes (block ids gathered from
    the step table by a step counter kept on the device, -1 = none), then the
    lengths and the counter advance."""
    nl = inp["q"].shape[0]
    B = inp["q"].shape[1]
    NB, maxp = inp["num_blocks"], inp["max_pages"]

    def step():
        for layer in range(nl):
            L.locks_decode_step(cfg, inp["q"][layer], spool, inp["k_pool"], inp["v_pool"], NB,
                                inp["block_table"][layer], seq, B, maxp, sel[layer], out[layer], lse[layer], ws,
                                ws_bytes)
        torch.index_select(inp["build_ids"], 0, step_idx, out=ids_buf)
        L.locks_build_summaries(cfg, inp["k_pool"], NB, ids_buf, ids_buf.numel(), spool)
        seq.add_(1)
        step_idx.add_(1)
    return step


def _full_step_check():
    sh = synth.FULL_STEP
    nl, B, Hkv, G, d, P, r, k = (sh["layers"], sh["batch"], sh["kv_heads"], sh["group"], sh["head_dim"],
                                 sh["page_size"], sh["rank"], sh["budget_pages"])
    Hq = Hkv * G
    dev = gg.DEV
    inp = synth.full_step_inputs(FULL_STEPS + 1, seed=5, device=dev,
                                 log=lambda m: print(f"[full step] {m}", flush=True))
    NB, maxp, lens0 = inp["num_blocks"], inp["max_pages"], inp["lens0"]
    cfg = L.make_config(d, P, r, Hq, Hkv, k, "bf16", "bf16", 1.0 / np.sqrt(d))
    kp, vp, bt = inp["k_pool"], inp["v_pool"], inp["block_table"]
    spool = L.summary_pool_for(cfg, NB, dev)
    full_ids = torch.cat([bt[layer, s, :lens0[s] // P] for layer in range(nl) for s in range(B)]).contiguous()
    L.locks_build_summaries(cfg, kp, NB, full_ids, full_ids.numel(), spool)
    torch.cuda.synchronize()
    print(f"[full step] {NB} blocks filled, {full_ids.numel() * Hkv} tiles built", flush=True)
    ws_bytes = L.locks_workspace_size(cfg, B, maxp)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    sel = torch.full((nl, B, Hkv, k), -7, dtype=torch.int32, device=dev)
    out = torch.empty((nl, B, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((nl, B, Hq), dtype=torch.float32, device=dev)
    seq = torch.tensor(lens0, dtype=torch.int32, device=dev)
    step_idx = torch.zeros(1, dtype=torch.int64, device=dev)
    ids_buf = torch.full((1, nl), -1, dtype=torch.int32, device=dev)
    step = full_step_graph(cfg, inp, spool, seq, sel, out, lse, ws, ws_bytes, step_idx, ids_buf)
    # warm-up on the capture stream, then back to the initial lengths and step
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    seq.copy_(torch.tensor(lens0, dtype=torch.int32))
    step_idx.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    assert int(step_idx.item()) == 0 and seq.cpu().tolist() == lens0  # capture records, runs nothing
    bt_c = bt.cpu()
    q_c = inp["q"].cpu()
    ids_c = inp["build_ids"].cpu()
    rng = np.random.default_rng(5)
    built = []  # (sequence, logical page) built inside the graph
    checked = 0
    for t in range(FULL_STEPS):
        assert t < ids_c.shape[0]  # the step table covers every replay
        graph.replay()
        torch.cuda.synchronize()
        lens_t = [x + t for x in lens0]  # lengths this step's decode saw
        sel_c = sel.cpu()
        out_c = gg.f64(out.cpu())
        # units: the sequence whose page the previous replay built (its summary
        # is now a candidate), and random others
        units = [(int(rng.integers(nl)), int(rng.integers(B)), int(rng.integers(Hkv))) for _ in range(3)]
        if built:
            units.append((int(rng.integers(nl)), built[-1][0], int(rng.integers(Hkv))))
        for layer, s, h in units:
            T = lens_t[s]
            J, Jc = -(-T // P), T // P
            idx = bt_c[layer, s, :Jc].long().to(dev)
            mu, vt, cf = (gg.f64(x) for x in L.split_records(cfg, spool[idx, h].cpu()))
            qu = gg.f64(q_c[layer, s, h * G:(h + 1) * G])
            s_o = oracle.page_scores(qu, mu, vt, cf, cfg.softmax_scale)
            if J <= k:
                sel_o, sigma_o = oracle.select(np.zeros(0), Jc, J, k), None
            else:
                _, sigma_o = oracle.combine(s_o)
                sel_o = oracle.select(sigma_o, Jc, J, k)
            wl_u = synth.Workload("full_unit", 1, Hkv, G, d, P, (T,), r, k, "bf16", "bf16")
            gg.check_selection(wl_u, 0, sel_c[layer, s, h].tolist(), sel_o.tolist(), sigma_o)
            ks, vs = [], []
            for j in sel_c[layer, s, h].tolist():
                if j < 0:
                    continue
                blk = int(bt_c[layer, s, j])
                nt = min(P, T - j * P)
                ks.append(gg.f64(kp[blk, h, :nt].cpu()))
                vs.append(gg.f64(vp[blk, h, :nt].cpu()))
            o_ref, _ = oracle.attend(qu, np.concatenate(ks), np.concatenate(vs), cfg.softmax_scale)
            err = float(np.max(np.abs(out_c[layer, s, h * G:(h + 1) * G] - o_ref)))
            assert err <= 2e-2, f"step {t} unit {(layer, s, h)}: output error {err}"
            checked += 1
        # the page this replay's token completed, built inside the graph
        if int(ids_c[t, 0]) >= 0:
            s_done = [s for s in range(B) if (lens0[s] + t + 1) % P == 0][0]
            built.append((s_done, (lens0[s_done] + t + 1) // P - 1))
        print(f"[full step] replay {t}: {len(units)} units match the oracle; pages built so far {built}",
              flush=True)
    assert int(step_idx.item()) == FULL_STEPS and seq.cpu().tolist() == [x + FULL_STEPS for x in lens0]
    assert built, "a page completes during the steps"
    # the pages built inside the graph: rank-4 fits checked against the oracle's
    for s, j in built:
        for layer in (0, nl - 1):
            blk = int(bt_c[layer, s, j])
            keys = np.stack([gg.f64(kp[blk, h].cpu()) for h in range(Hkv)])
            _, vt_o, _, ev, _ = oracle.build_pages(keys, r)
            _, vt_g, _ = L.split_records(cfg, spool[blk].cpu())
            for h in range(Hkv):
                gg.check_fit(keys[h], gg.f64(vt_g[h]), ev[h], vt_o[h], r)
    assert checked >= 3 * FULL_STEPS


def test_full_step_graph_against_oracle():
    try:
        _full_step_check()  # its ~150 GB of device buffers are released on return
    finally:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

"""GPU parity of the quantized ("i4") summary path — [Locks] §4 and App. C.7:
4-bit basis, 8-bit centroid and coefficients, bf16 scales — against the fp64
oracle, through the C ABI.

* Scorer: on identical record bytes (codes and scales from the seeded
  generator, or oracle fits quantized by the oracle, packed by the test-side
  packer), every page score within 1e-3 (mixed) of Eq. (2) evaluated by the
  oracle on the dequantized values.
* Build: the GPU's fp32 fit differs from the oracle's fp64 fit by rounding,
  so its codes are checked for being a valid quantization of the oracle's
  fit: each scale a bf16 rounding of the group's max over L, each code within
  half a step of the oracle's value (plus the fit tolerance), on groups whose
  basis vectors are well separated (several bases are correct otherwise).
* Whole step: selection and output against the oracle on oracle-quantized
  summaries.
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

# d, P, r, G across the supported set; ragged lengths with partial current
# pages; G * P < 64 leaves lanes without a token (G = 1 / P = 16, G = 2 / P = 16)
SHAPES = [
    synth.Workload("i4_d128_p64_r8_g4", 3, 2, 4, 128, 64, (64 * 40 + 37, 64 * 24, 64 * 9 + 1), 8, 8,
                   "bf16", "i4", extra_blocks=5),
    synth.Workload("i4_d128_p16_r1_g4", 2, 2, 4, 128, 16, (16 * 150 + 5, 16 * 70), 1, 16, "bf16", "i4",
                   extra_blocks=3),
    synth.Workload("i4_d128_p16_r2_g8", 2, 2, 8, 128, 16, (16 * 130, 16 * 33 + 15), 2, 16, "bf16", "i4"),
    synth.Workload("i4_d128_p32_r4_g4", 2, 3, 4, 128, 32, (32 * 90 + 31, 32 * 41), 4, 12, "bf16", "i4"),
    synth.Workload("i4_d64_p16_r4_g1", 2, 4, 1, 64, 16, (16 * 100 + 3, 16 * 60), 4, 10, "bf16", "i4"),
    synth.Workload("i4_d64_p16_r8_g2", 2, 2, 2, 64, 16, (16 * 77, 16 * 20 + 9), 8, 10, "bf16", "i4"),
    synth.Workload("i4_d64_p32_r2_g2", 1, 2, 2, 64, 32, (32 * 64 + 1,), 2, 8, "bf16", "i4"),
    synth.Workload("i4_d64_p64_r1_g8", 2, 1, 8, 64, 64, (64 * 50, 64 * 3), 1, 8, "bf16", "i4"),
    # ranks 8 and 4 with 4 query heads per KV head score their tokens on the
    # matrix cores (up to 4 pages per product): page counts that leave 1-3
    # pages over
    synth.Workload("i4_d128_p16_r8_g4", 2, 2, 4, 128, 16, (16 * 139 + 7, 16 * 66), 8, 16, "bf16", "i4",
                   extra_blocks=2),
    synth.Workload("i4_d128_p32_r8_g4", 3, 1, 4, 128, 32, (32 * 71, 32 * 5 + 3, 32 * 2), 8, 8, "bf16", "i4"),
    synth.Workload("i4_d64_p64_r8_g4", 2, 2, 4, 64, 64, (64 * 45 + 1, 64 * 7), 8, 8, "bf16", "i4"),
    synth.Workload("i4_d128_p16_r4_g4", 2, 2, 4, 128, 16, (16 * 101 + 9, 16 * 18), 4, 16, "bf16", "i4"),
    synth.Workload("i4_d64_p64_r4_g4", 1, 3, 4, 64, 64, (64 * 37 + 50,), 4, 8, "bf16", "i4"),
]


def _scores_vs_oracle(wl, data, hs, qs, units=None):
    G = wl.group
    bt = data["block_table"]
    units = units or [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]
    for b, h in units:
        _, _, Jc = gg.lens(wl, b)
        if Jc == 0:
            continue
        mu, vt, cf = gg.i4_unit_summaries(wl, qs, bt, b, h, Jc)
        s_o = gg.oracle_unit_scores(wl, data, b, h, mu, vt, cf)
        got = gg.f64(hs[b, h * G:(h + 1) * G, :Jc])
        v = gg.mixed_violation(got, s_o)
        assert v <= 1.0, (wl.name, b, h, v)


@pytest.mark.parametrize("wl", SHAPES, ids=lambda w: w.name)
def test_i4_scores_on_identical_bytes(wl):
    cfg = L.config_for(wl)
    data, g = gg.make_inputs(wl, seed=3)
    qs = synth.random_i4_codes(wl, seed=3)
    pool = gg.i4_pool_from_codes(wl, cfg, qs)
    hs = gg.gpu_scores(wl, cfg, g, pool)
    torch.cuda.synchronize()
    hs = hs.cpu()
    _scores_vs_oracle(wl, data, hs, qs)
    # entries past the complete pages are left untouched
    G = wl.group
    for b in range(wl.batch):
        _, _, Jc = gg.lens(wl, b)
        assert torch.isnan(hs[b, :, Jc:]).all()


def test_i4_invalid_block_ids_score_minus_inf():
    wl = SHAPES[0]
    cfg = L.config_for(wl)
    data, g = gg.make_inputs(wl, seed=4)
    bad = {(0, 3): -1, (0, 5): wl.num_blocks + 10}
    for (b, j), v in bad.items():
        data["block_table"][b, j] = v
        g["block_table"][b, j] = v
    qs = synth.random_i4_codes(wl, seed=4)
    pool = gg.i4_pool_from_codes(wl, cfg, qs)
    hs = gg.gpu_scores(wl, cfg, g, pool)
    torch.cuda.synchronize()
    hs = hs.cpu()
    for (b, j) in bad:
        assert torch.isinf(hs[b, :, j]).all() and (hs[b, :, j] < 0).all()
    ok = [(b, h) for b in range(1, wl.batch) for h in range(wl.num_kv_heads)]
    _scores_vs_oracle(wl, data, hs, qs, ok)


# --------------------------------------------------------------------------
# build: valid quantization of the oracle's fit
# --------------------------------------------------------------------------
def _check_group(x_o, codes, s, L_, tol, what):
    """codes/s must be a nearest rounding of values within tol of x_o."""
    amax = float(np.max(np.abs(x_o)))
    if amax <= tol:
        return
    lo, hi = (amax - tol) / L_, (amax + tol) / L_
    assert lo * (1 - 2.0 ** -8) <= s <= hi * (1 + 2.0 ** -8), (what, s, amax / L_)
    err = np.abs(codes * s - x_o)
    assert np.all(err <= 0.5 * s + tol + 1e-12), (what, float(np.max(err / s)))
    assert int(np.max(np.abs(codes))) == L_, what


def _separated(ev, rho, rel=0.2):
    lam = ev[rho]
    if lam <= 0:
        return False
    gaps = [ev[rho] - ev[rho + 1]]
    if rho > 0:
        gaps.append(ev[rho - 1] - ev[rho])
    return min(gaps) / lam > rel


def _check_build(wl, rec, data, pages):
    d, r, P = wl.head_dim, wl.rank, wl.page_size
    _, raw, keys = gg.oracle_summaries(wl, data, pages)
    n_basis = n_coef = 0
    for blk, h in pages:
        mu_o, vt_o, cf_o, ev = raw[(blk, h)]
        u = {k: v[blk, h] for k, v in rec.items()}
        assert np.all(u["padding"] == 0)
        _check_group(mu_o, u["mu_code"], u["mu_scale"], 127, 1e-5 * np.max(np.abs(mu_o)) + 1e-6, "mu")
        sep = [_separated(ev, rho) for rho in range(r)]
        signs = np.ones(r)
        for rho in range(r):
            if not sep[rho]:
                continue
            signs[rho] = 1.0 if np.dot(u["vt_code"][rho], vt_o[rho]) >= 0 else -1.0
            _check_group(signs[rho] * vt_o[rho], u["vt_code"][rho], u["vt_scale"][rho], 7, 1e-3, f"V{rho}")
            n_basis += 1
        if all(sep):
            cf_a = cf_o * signs
            tol = 1e-3 * float(np.max(np.abs(cf_a)))
            for i in range(P):
                _check_group(cf_a[i], u["coef_code"][i], u["coef_scale"][i], 127, tol, f"C{i}")
            n_coef += 1
    return n_basis, n_coef


@pytest.mark.parametrize("rank", [4, 8])
def test_i4_build_is_valid_quantization(rank):
    wl = synth.Workload(f"i4_build_r{rank}", 3, 2, 4, 128, 64, (64 * 40 + 37, 64 * 24, 64 * 9 + 1), rank, 8,
                        "bf16", "i4", extra_blocks=5)
    cfg = L.config_for(wl)
    data, g = gg.make_inputs(wl, seed=5)
    pool = gg.gpu_build(wl, cfg, g)
    torch.cuda.synchronize()
    rec = gg.unpack_i4(pool.cpu().numpy(), wl.head_dim, wl.rank, wl.page_size)
    pages = []
    for b in range(wl.batch):
        _, _, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            pages += [(int(data["block_table"][b, j]), h) for j in range(Jc)]
    rng = np.random.default_rng(5)
    pages = [pages[i] for i in sorted(rng.choice(len(pages), 40, replace=False))]
    n_basis, n_coef = _check_build(wl, rec, data, pages)
    # the generator's six signal directions are well separated: most basis
    # vectors (and at rank 4 most coefficient rows) are checked
    assert n_basis >= len(pages) * min(rank, 6) // 2
    if rank == 4:
        assert n_coef >= len(pages) // 2


# --------------------------------------------------------------------------
# whole decode step on oracle-quantized summaries
# --------------------------------------------------------------------------
def _oracle_i4_codes(wl, data):
    """Oracle fit of every complete page, quantized by the oracle; codes and
    scales over the whole pool (zero for blocks without a complete page)."""
    d, r, P, H = wl.head_dim, wl.rank, wl.page_size, wl.num_kv_heads
    n = wl.num_blocks
    qs = dict(mu_code=np.zeros((n, H, d), np.int64), vt_code=np.zeros((n, H, r, d), np.int64),
              coef_code=np.zeros((n, H, P, r), np.int64), mu_scale=np.zeros((n, H)),
              vt_scale=np.zeros((n, H, r)), coef_scale=np.zeros((n, H, P)))
    _, raw, _ = gg.oracle_summaries(wl, data)
    pages = list(raw.keys())
    mu = np.stack([raw[p][0] for p in pages]); vt = np.stack([raw[p][1] for p in pages])
    cf = np.stack([raw[p][2] for p in pages])
    q = oracle.quantize_summaries(mu, vt, cf)
    for i, (blk, h) in enumerate(pages):
        for k in qs:
            qs[k][blk, h] = q[k][i]
    return qs


def test_i4_decode_step_end_to_end():
    wl = synth.Workload("ragged_i4", 5, 2, 4, 128, 64, (64 * 40 + 37, 64 * 24, 64 * 9 + 1, 64 * 5, 17), 8, 8,
                        "bf16", "i4", n_needles=3, extra_blocks=4)
    cfg = L.config_for(wl)
    data, g = gg.make_inputs(wl, seed=21)
    qs = _oracle_i4_codes(wl, data)
    pool = gg.i4_pool_from_codes(wl, cfg, qs)
    sel, out, lse = gg.gpu_decode_step(wl, cfg, g, pool)
    torch.cuda.synchronize()
    sel, out, lse = sel.cpu(), gg.f64(out.cpu()), gg.f64(lse.cpu())
    same = units = 0
    for b in range(wl.batch):
        _, J, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            units += 1
            s_o = None
            if J > wl.budget_pages:
                mu, vt, cf = gg.i4_unit_summaries(wl, qs, data["block_table"], b, h, Jc)
                s_o = gg.oracle_unit_scores(wl, data, b, h, mu, vt, cf)
            sel_o, sigma_o = gg.oracle_unit_select(wl, b, s_o)
            if gg.check_selection(wl, b, sel[b, h].tolist(), sel_o.tolist(), sigma_o) == 0:
                same += 1
                o_ref, lse_ref = gg.oracle_unit_attend(wl, data, b, h, sel_o)
                sl = slice(h * wl.group, (h + 1) * wl.group)
                assert np.max(np.abs(out[b, sl] - o_ref)) <= gg.out_tol(wl)
                assert np.max(np.abs(lse[b, sl] - lse_ref)) <= 1e-3 * max(1.0, float(np.max(np.abs(lse_ref))))
    assert same >= units - 1


def test_i4_gpu_build_end_to_end():
    """GPU build (fit and quantization) -> GPU score -> GPU select -> GPU
    decode against oracle fit -> oracle quantization -> oracle score ->
    oracle select -> oracle attend, every unit. The two chains quantize two
    valid fits independently, so a page's two scores may differ by as much as
    their reconstructed keys do: the page LSE is 1-Lipschitz in the max norm,
    so |s_gpu - s_oracle| <= max_i |q . (k_gpu,i - k_oracle,i)| * scale (keys
    rebuilt from each chain's stored codes and scales) plus the score bar;
    selections agree except for pages within twice the unit's largest such
    difference of the (k-2)-th key; outputs on equal selections within the
    output bar."""
    wl = synth.Workload("e2e_i4_gpu_build", 3, 2, 4, 128, 64, (64 * 40 + 37, 64 * 24, 64 * 9 + 1), 8, 8,
                        "bf16", "i4", n_needles=3, extra_blocks=3)
    cfg = L.config_for(wl)
    data, g = gg.make_inputs(wl, seed=9)
    pool = gg.gpu_build(wl, cfg, g)
    hs = gg.gpu_scores(wl, cfg, g, pool)
    sel, out, _ = gg.gpu_decode_step(wl, cfg, g, pool)
    torch.cuda.synchronize()
    hs, sel, out = hs.cpu(), sel.cpu(), gg.f64(out.cpu())
    rec_g = gg.unpack_i4(pool.cpu().numpy(), wl.head_dim, wl.rank, wl.page_size)
    qs_o = _oracle_i4_codes(wl, data)
    bt = data["block_table"]
    G, scale = wl.group, wl.softmax_scale
    same = units = 0
    worst = 0.0
    for b in range(wl.batch):
        _, J, Jc = gg.lens(wl, b)
        for h in range(wl.num_kv_heads):
            units += 1
            s_o, tol = None, gg.SCORE_TOL
            if Jc > 0:
                mu_g, vt_g, cf_g = gg.i4_unit_summaries(wl, rec_g, bt, b, h, Jc)
                mu_o, vt_o, cf_o = gg.i4_unit_summaries(wl, qs_o, bt, b, h, Jc)
                q = gg.f64(data["q"][b, h * G:(h + 1) * G])
                dk = (mu_g - mu_o)[:, None, :] + cf_g @ vt_g - cf_o @ vt_o  # [Jc][P][d]
                dz = np.abs(np.einsum("gd,jpd->gjp", q, dk)).max(axis=2) * scale  # [G][Jc]
                s_o = gg.oracle_unit_scores(wl, data, b, h, mu_o, vt_o, cf_o)
                s_g = gg.f64(hs[b, h * G:(h + 1) * G, :Jc])
                bar = dz + gg.SCORE_TOL * np.maximum(1.0, np.abs(s_o))
                assert np.all(np.abs(s_g - s_o) <= bar), f"unit {(b, h)}: scores beyond the quantization bound"
                worst = max(worst, float(dz.max()))
                tol = gg.SCORE_TOL + 2.0 * float(dz.max())
            sel_o, sigma_o = gg.oracle_unit_select(wl, b, s_o if J > wl.budget_pages else None)
            if gg.check_selection(wl, b, sel[b, h].tolist(), sel_o.tolist(), sigma_o, tol=tol) == 0:
                same += 1
                o_ref, _ = gg.oracle_unit_attend(wl, data, b, h, sel_o)
                sl = slice(h * G, (h + 1) * G)
                assert np.max(np.abs(out[b, sl] - o_ref)) <= gg.out_tol(wl)
    print(f"[i4 e2e] largest score bound {worst:.4g}; {same}/{units} selections equal")
    assert same >= units - 1


# --------------------------------------------------------------------------
# full-size shapes: every unit scored and selected on the GPU, sampled units
# against the oracle; the full-size i4 build sampled for validity
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name,rank", [("llama8b_128k_b8", 8), ("llama8b_128k_b8_p16", 8),
                                       ("llama8b_128k_b8_p16", 4)],
                         ids=["p64_r8", "p16_r8", "p16_r4"])
def test_i4_full_size_all_units(name, rank):
    wl = W[name].with_(summary_dtype="i4", rank=rank)
    cfg = L.config_for(wl)
    G = wl.group
    d = synth.generate(wl, 0, gg.DEV)
    qs = {k: v.cpu().numpy() for k, v in synth.random_i4_codes(wl, 0, gg.DEV).items()}
    pool = gg.i4_pool_from_codes(wl, cfg, qs)
    hs = gg.gpu_scores(wl, cfg, d, pool)
    sel = gg.gpu_score_select(wl, cfg, d, pool)
    torch.cuda.synchronize()
    data_c = {"q": d["q"].cpu(), "block_table": d["block_table"].cpu()}
    # every unit: scores element by element and selections against the oracle
    # on the dequantized records, outputs on the oracle's selections
    sel_o, ndiff = gg.check_all_units(
        wl, data_c, hs.cpu(), sel.cpu(),
        lambda b, h, Jc: gg.i4_unit_summaries(wl, qs, data_c["block_table"], b, h, Jc))
    assert ndiff <= wl.batch * wl.num_kv_heads
    out, _ = gg.gpu_decode(wl, cfg, d, sel_o.to(gg.DEV))
    torch.cuda.synchronize()
    gg.check_all_outputs(wl, d, out.cpu(), sel_o)
    # full-size build, every page of every unit; a sample checked for validity
    del pool, hs
    ids = d["block_table"].reshape(-1).contiguous()
    pool2 = L.summary_pool_for(cfg, wl.num_blocks, gg.DEV)
    L.locks_build_summaries(cfg, d["k_pool"], wl.num_blocks, ids, ids.numel(), pool2)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    bt = data_c["block_table"]
    sample = sorted({(int(bt[b, j]), int(h)) for b, j, h in zip(rng.integers(0, wl.batch, 12),
                                                                 rng.integers(0, wl.max_pages, 12),
                                                                 rng.integers(0, wl.num_kv_heads, 12))})
    blocks = sorted({blk for blk, _ in sample})
    pos = {blk: i for i, blk in enumerate(blocks)}
    un = gg.unpack_i4(pool2[torch.tensor(blocks, device=gg.DEV)].cpu().numpy(), wl.head_dim, wl.rank,
                      wl.page_size)
    # (blk, h)-keyed views of the sampled records and keys
    rec = {k: {(blk, h): v[pos[blk], h] for blk, h in sample} for k, v in un.items()}
    keys = {"k_pool": {(blk, h): d["k_pool"][blk, h].cpu() for blk, h in sample}, "block_table": None}
    n_basis, _ = _check_build(wl, rec, keys, sample)
    assert n_basis >= len(sample)

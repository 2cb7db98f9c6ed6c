"""GPU tests of the decode step through the hot-page cache (K/V pools in
pinned host memory, tiles kept in device memory; [Locks] §5.3 Table 3 and
App. B.4.2), called through the C ABI:

- every step's selection and attention output against the oracle (the
  selection on the GPU-built records under the window rule, the output on the
  original K/V of the selected pages), over decode steps whose lengths grow
  (pages complete inside the run and are built, tiles copied while their page
  was incomplete are copied again), with a capacity that forces evictions;
- the same step without the cache on device-resident pools gives the same
  bits;
- the cache state after every step (clock hand, maps, stamps, flags,
  counters) equals the host model of the policy fed the same selections.
"""
import numpy as np
import pytest
import torch

from sparse_kv_page_amd import locks as L
from sparse_kv_page_amd import synth
from tests import gpu_glue as gg
from tests.hot_cache_model import ClockModel, accesses_of

pytestmark = pytest.mark.gpu


def _cfg(wl):
    return L.make_config(wl.head_dim, wl.page_size, wl.rank, wl.num_q_heads, wl.num_kv_heads, wl.budget_pages,
                         wl.kv_dtype, wl.summary_dtype, wl.softmax_scale)


def _check_state(cache, model):
    st = cache.state()
    assert st["hand"] == model.hand and st["step"] == model.step_no
    assert torch.equal(st["slot_of"], torch.from_numpy(model.slot_of).to(torch.int32))
    assert torch.equal(st["tile_of"], torch.from_numpy(model.tile_of).to(torch.int32))
    assert torch.equal(st["stamp"], torch.from_numpy(model.stamp).to(torch.int32))
    assert torch.equal(st["flags"], torch.from_numpy(model.flags).to(torch.int32))
    assert cache.stats() == model.stats


def _run_cached_steps(wl, steps, capacity, rho, seed, check_units, log=print, share_prefix=0):
    """Decode steps 0..steps-1 at lengths lens_end - (steps - 1) + t through
    the cache (pages that complete get their summaries before the next step);
    after each: bitwise equality with the uncached step on device pools, the
    policy model, and check_units(t, wl_t, g_t, pool, sel, out).
    share_prefix > 0: sequence 1's first share_prefix pages use sequence 0's
    blocks (a shared prompt), so page slots of one step name the same tiles."""
    cfg = _cfg(wl)
    g = synth.generate(wl, seed, gg.DEV)
    if share_prefix:
        g["block_table"][1, :share_prefix] = g["block_table"][0, :share_prefix]
    lens_end = [int(x) for x in wl.seq_lens]
    lens0 = [x - (steps - 1) for x in lens_end]
    P, NB, Hkv = wl.page_size, wl.num_blocks, wl.num_kv_heads
    bt_c = g["block_table"].cpu()
    # summaries of the pages complete at the first step
    ids = torch.cat([g["block_table"][b, :lens0[b] // P] for b in range(wl.batch)]).contiguous()
    pool = gg.gpu_build(wl, cfg, g, block_ids=ids)
    kh, kdev = gg.host_pool(g["k_pool"])
    vh, vdev = gg.host_pool(g["v_pool"])
    cache = L.HotCache(cfg, NB, capacity, gg.DEV)
    model = ClockModel(capacity, NB * Hkv)
    qs = synth.query_sequence(g["q"], steps, rho, seed)
    nbytes = L.locks_workspace_size(cfg, wl.batch, wl.max_pages)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=gg.DEV)
    ws2 = torch.zeros(nbytes, dtype=torch.uint8, device=gg.DEV)
    dt = synth.torch_dtype(wl.kv_dtype)
    sel = torch.empty((wl.batch, Hkv, wl.budget_pages), dtype=torch.int32, device=gg.DEV)
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=dt, device=gg.DEV)
    lse = torch.empty((wl.batch, wl.num_q_heads), device=gg.DEV)
    for t in range(steps):
        lens_t = [x + t for x in lens0]
        seq = torch.tensor(lens_t, dtype=torch.int32, device=gg.DEV)
        L.locks_decode_step_cached(cfg, qs[t], pool, kdev, vdev, NB, g["block_table"], seq, wl.batch,
                                   wl.max_pages, sel, out, lse, cache.buf, capacity, ws, nbytes)
        g_t = dict(g, q=qs[t], seq_lens=seq)
        sel_d, out_d, lse_d = gg.gpu_decode_step(wl, cfg, g_t, pool, ws=ws2)
        torch.cuda.synchronize()
        assert torch.equal(sel, sel_d), f"step {t}: selection differs from the uncached step"
        assert torch.equal(out.view(torch.int16), out_d.view(torch.int16)), f"step {t}: output differs"
        assert torch.equal(lse, lse_d), f"step {t}: lse differs"
        sel_c = sel.cpu()
        model.step(accesses_of(sel_c.numpy(), bt_c.numpy(), lens_t, P, NB, Hkv))
        _check_state(cache, model)
        check_units(t, wl.with_(seq_lens=tuple(lens_t)), g_t, pool, sel_c, out.cpu())
        log(f"[cache] step {t}: {cache.stats()}")
        # pages the next token completes get their summaries (gpu_build fills
        # a fresh pool; the new records are copied into the running one)
        done = [int(bt_c[b, (x + 1) // P - 1]) for b, x in enumerate(lens_t) if (x + 1) % P == 0]
        if done and t + 1 < steps:
            fresh = gg.gpu_build(wl, cfg, g, block_ids=torch.tensor(done, dtype=torch.int32, device=gg.DEV))
            idx = torch.tensor(done, device=gg.DEV).long()
            pool[idx] = fresh[idx]
    del kh, vh
    return cache, model


GROW = synth.Workload("cache_grow", 3, 4, 2, 128, 64, (64 * 30 + 4, 64 * 25 + 40, 64 * 18 + 9), 8, 8,
                      "bf16", "bf16", centroid_std=0.5, ar_rho=0.99, n_needles=4)


GROW_F32 = synth.Workload("cache_grow_f32", 2, 2, 2, 64, 16, (16 * 40 + 3, 16 * 23 + 9), 4, 6, "f32", "f32")


@pytest.mark.parametrize("wl,capacity_mult,rho", [(GROW, 1.25, 0.7), (GROW, 3.0, 0.9), (GROW, 1.0, 0.0),
                                                   (GROW_F32, 1.5, 0.8)],
                         ids=["bf16-x1.25", "bf16-x3", "bf16-x1-indep", "f32-p16-x1.5"])
def test_cached_step_against_oracle(wl, capacity_mult, rho):
    """Growing lengths over 14 steps (every sequence's current page is
    incomplete at first, pages complete during the run): every unit of every
    step against the oracle, bits against the uncached step, state against the
    policy model; bf16 at 64-token pages and fp32 at 16-token pages."""
    steps = 14
    n = wl.batch * wl.num_kv_heads * wl.budget_pages
    capacity = int(n * capacity_mult)
    cfg = _cfg(wl)

    def check_units(t, wl_t, g_t, pool, sel_c, out_c):
        data_c = {"q": g_t["q"].cpu(), "block_table": g_t["block_table"].cpu()}
        hs = gg.gpu_scores(wl, cfg, g_t, pool).cpu()  # launched at the table's max_pages
        pool_c = pool.cpu()
        mu_c, vt_c, cf_c = L.split_records(cfg, pool_c)
        bt = data_c["block_table"]

        def unit_summaries(b, h, Jc):
            idx = bt[b, :Jc].long()
            return gg.f64(mu_c[idx, h]), gg.f64(vt_c[idx, h]), gg.f64(cf_c[idx, h])

        gg.check_all_units(wl_t, data_c, hs, sel_c, unit_summaries)
        gg.check_all_outputs(wl_t, dict(g_t, q=data_c["q"]), out_c, sel_c)

    cache, model = _run_cached_steps(wl, steps, capacity, rho, seed=3, check_units=check_units)
    s = cache.stats()
    assert s["failed"] == 0 and s["steps"] == steps
    assert s["misses"] > 0 and s["refreshes"] > 0
    if capacity_mult > 1.0:
        assert s["hits"] > 0


def test_cached_step_shared_prefix():
    """Two sequences share their first 12 pages' blocks (a common prompt):
    the sink page and any shared page both select name one tile, which takes
    one slot (the later page slot is served as shared); every unit against the
    oracle, bits against the uncached step, state against the policy model."""
    wl = GROW
    cfg = _cfg(wl)
    n = wl.batch * wl.num_kv_heads * wl.budget_pages

    def check_units(t, wl_t, g_t, pool, sel_c, out_c):
        data_c = {"q": g_t["q"].cpu(), "block_table": g_t["block_table"].cpu()}
        hs = gg.gpu_scores(wl, cfg, g_t, pool).cpu()
        mu_c, vt_c, cf_c = L.split_records(cfg, pool.cpu())
        bt = data_c["block_table"]

        def unit_summaries(b, h, Jc):
            idx = bt[b, :Jc].long()
            return gg.f64(mu_c[idx, h]), gg.f64(vt_c[idx, h]), gg.f64(cf_c[idx, h])

        gg.check_all_units(wl_t, data_c, hs, sel_c, unit_summaries)
        gg.check_all_outputs(wl_t, dict(g_t, q=data_c["q"]), out_c, sel_c)

    cache, model = _run_cached_steps(wl, 10, n + n // 2, 0.8, seed=4, check_units=check_units, share_prefix=12)
    s = cache.stats()
    assert s["shared"] > 0 and s["failed"] == 0


def test_cached_step_128k_batch8():
    """The 128K-context batch of 8 (r = 8, k = 32) through a cache of 4 steps'
    tiles, 16 steps of AR(1) queries (rho 0.9) ending at 128K tokens: bits
    against the uncached step, state against the policy model every step, and
    sampled units against the oracle."""
    wl = synth.WORKLOADS["llama8b_128k_b8"]
    cfg = _cfg(wl)
    n = wl.batch * wl.num_kv_heads * wl.budget_pages
    rng = np.random.default_rng(1)

    def check_units(t, wl_t, g_t, pool, sel_c, out_c):
        G = wl.group
        q_c = g_t["q"].cpu()
        bt = g_t["block_table"].cpu()
        for _ in range(2):
            b, h = int(rng.integers(wl.batch)), int(rng.integers(wl.num_kv_heads))
            T, J, Jc = gg.lens(wl_t, b)
            idx = bt[b, :Jc].long().to(gg.DEV)
            mu, vt, cf = (gg.f64(x) for x in L.split_records(cfg, pool[idx, h].cpu()))
            data_u = {"q": q_c, "block_table": bt, "k_pool": g_t["k_pool"], "v_pool": g_t["v_pool"]}
            s_o = gg.oracle_unit_scores(wl_t, data_u, b, h, mu, vt, cf)
            sel_o, sigma_o = gg.oracle_unit_select(wl_t, b, s_o)
            gg.check_selection(wl_t, b, sel_c[b, h].tolist(), sel_o.tolist(), sigma_o)
            o_ref, _ = gg.oracle_unit_attend(wl_t, data_u, b, h, sel_c[b, h].tolist())
            err = float(np.max(np.abs(gg.f64(out_c[b, h * G:(h + 1) * G]) - o_ref)))
            assert err <= gg.out_tol(wl), f"step {t} unit {(b, h)}: output error {err}"

    cache, model = _run_cached_steps(wl, 16, 4 * n, 0.9, seed=0, check_units=check_units)
    s = cache.stats()
    total = s["hits"] + s["misses"] + s["refreshes"] + s["shared"]
    print(f"[cache] 128K batch 8: hit share {s['hits'] / total:.3f} over {s['steps']} steps: {s}")
    assert s["failed"] == 0 and s["shared"] == 0


def test_cached_step_in_a_graph():
    """The cached step captured into a HIP graph (queries and lengths read
    from buffers the program refills between replays) and replayed over 8
    steps, with eager work in between: every replay's selection, output and
    the cache's whole state equal those of the same steps run eagerly on a
    second cache."""
    wl = GROW
    cfg = _cfg(wl)
    steps = 8
    n = wl.batch * wl.num_kv_heads * wl.budget_pages
    capacity = n + n // 4
    g = synth.generate(wl, 11, gg.DEV)
    P, NB, Hkv = wl.page_size, wl.num_blocks, wl.num_kv_heads
    lens0 = [int(x) - (steps - 1) for x in wl.seq_lens]
    pool = gg.gpu_build(wl, cfg, g)  # every page complete at the end; earlier steps see only their own
    kh, kdev = gg.host_pool(g["k_pool"])
    vh, vdev = gg.host_pool(g["v_pool"])
    qs = synth.query_sequence(g["q"], steps, 0.8, 11)
    nbytes = L.locks_workspace_size(cfg, wl.batch, wl.max_pages)
    dt = synth.torch_dtype(wl.kv_dtype)

    def buffers():
        return (torch.zeros(nbytes, dtype=torch.uint8, device=gg.DEV),
                torch.empty((wl.batch, Hkv, wl.budget_pages), dtype=torch.int32, device=gg.DEV),
                torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=dt, device=gg.DEV),
                torch.empty((wl.batch, wl.num_q_heads), device=gg.DEV))

    # eager reference on cache A
    cache_a = L.HotCache(cfg, NB, capacity, gg.DEV)
    ws_a, sel_a, out_a, lse_a = buffers()
    ref = []
    for t in range(steps):
        seq = torch.tensor([x + t for x in lens0], dtype=torch.int32, device=gg.DEV)
        L.locks_decode_step_cached(cfg, qs[t], pool, kdev, vdev, NB, g["block_table"], seq, wl.batch, wl.max_pages,
                                   sel_a, out_a, lse_a, cache_a.buf, capacity, ws_a, nbytes)
        torch.cuda.synchronize()
        ref.append((sel_a.clone(), out_a.clone(), lse_a.clone(), cache_a.state(), cache_a.stats()))
    # the same steps replayed from one graph on cache B
    cache_b = L.HotCache(cfg, NB, capacity, gg.DEV)
    ws_b, sel_b, out_b, lse_b = buffers()
    q_buf = qs[0].clone()
    seq_buf = torch.tensor(lens0, dtype=torch.int32, device=gg.DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            L.locks_decode_step_cached(cfg, q_buf, pool, kdev, vdev, NB, g["block_table"], seq_buf, wl.batch,
                                       wl.max_pages, sel_b, out_b, lse_b, cache_b.buf, capacity, ws_b, nbytes)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    st0 = cache_b.stats()
    assert st0["steps"] == 0, "capturing must not run the step"
    for t in range(steps):
        q_buf.copy_(qs[t])
        seq_buf.copy_(torch.tensor([x + t for x in lens0], dtype=torch.int32))
        graph.replay()
        torch.cuda.synchronize()
        _ = torch.randn(1024, device=gg.DEV).sum().item()  # eager work between replays
        s_ref, o_ref, l_ref, state_ref, stats_ref = ref[t]
        assert torch.equal(sel_b, s_ref), f"replay {t}: selection"
        assert torch.equal(out_b.view(torch.int16), o_ref.view(torch.int16)), f"replay {t}: output"
        assert torch.equal(lse_b, l_ref), f"replay {t}: lse"
        st = cache_b.state()
        for key in ("hand", "step"):
            assert st[key] == state_ref[key], f"replay {t}: {key}"
        for key in ("slot_of", "tile_of", "stamp", "flags"):
            assert torch.equal(st[key], state_ref[key]), f"replay {t}: {key}"
        assert cache_b.stats() == stats_ref, f"replay {t}: counters"
    del kh, vh

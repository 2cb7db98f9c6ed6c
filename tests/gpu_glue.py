"""Glue shared by the GPU parity tests: run the HIP path through the C ABI and
the fp64 oracle on the same seeded inputs, and compare to the stated bars.

Tolerances (from the spec bar):
  page scores / page keys : |gpu - oracle| <= 1e-3 * max(1, |oracle|)
  selected pages          : identical except pages whose oracle key lies within
                            that same tolerance of the (k-2)-th ranked key
  attention output        : 2e-2 absolute (bf16 storage), 1e-4 absolute (fp32)
No oracle input is ever taken from the HIP path: stage inputs (summaries,
page scores, page selections) are produced by the oracle or the generator.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from sparse_kv_page_amd import locks as L
from sparse_kv_page_amd import synth

DEV = "cuda"
SCORE_TOL = 1e-3


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def mixed_violation(gpu, ref, tol=SCORE_TOL) -> float:
    """max |gpu - ref| / (tol * max(1, |ref|)); <= 1 passes."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isinf(gpu) & np.isinf(ref) & (np.sign(gpu) == np.sign(ref))
    err = np.where(both_inf, 0.0, np.abs(gpu - ref)) / (tol * np.maximum(1.0, np.abs(ref)))
    return float(np.max(err)) if err.size else 0.0


def out_tol(wl) -> float:
    return 2e-2 if wl.kv_dtype == "bf16" else 1e-4


def lens(wl, b):
    T = int(wl.seq_lens[b])
    P = wl.page_size
    return T, -(-T // P), T // P


# --------------------------------------------------------------------------
# inputs
# --------------------------------------------------------------------------
def make_inputs(wl, seed=0, gen_device="cpu"):
    d = synth.generate(wl, seed, gen_device)
    gpu = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in d.items()}
    return d, gpu


def oracle_summaries(wl, data, pages=None, threads=None):
    """Oracle fits (fp64 and rounded to the summary dtype) for the given
    (block, head) pairs (default: every complete page of every unit).
    Returns dict (block, head) -> (mu, vt, coef, evals) rounded, and raw."""
    kp = data["k_pool"]
    bt = data["block_table"]
    if pages is None:
        pages = []
        for b in range(wl.batch):
            _, _, Jc = lens(wl, b)
            for h in range(wl.num_kv_heads):
                pages += [(int(bt[b, j]), h) for j in range(Jc)]
    keys = np.stack([f64(kp[blk, h]) for blk, h in pages]) if pages else np.zeros((0, wl.page_size, wl.head_dim))
    mu, vt, cf, ev, _ = oracle.build_pages(keys, wl.rank, threads=threads)
    raw = {p: (mu[i], vt[i], cf[i], ev[i]) for i, p in enumerate(pages)}
    if wl.summary_dtype == "bf16":
        mu, vt, cf = oracle.round_bf16(mu), oracle.round_bf16(vt), oracle.round_bf16(cf)
    rounded = {p: (mu[i], vt[i], cf[i], ev[i]) for i, p in enumerate(pages)}
    return rounded, raw, keys


def pool_from_summaries(wl, cfg, summ):
    """Summary pool on the device holding the given records (others zero)."""
    pool = torch.zeros_like(L.summary_pool_for(cfg, wl.num_blocks, "cpu"))
    for (blk, h), (mu, vt, cf, _) in summ.items():
        rec = np.concatenate([mu, vt.ravel(), cf.ravel()])
        pool[blk, h] = torch.from_numpy(rec).to(pool.dtype)
    return pool.to(DEV)


def synthetic_pool(wl, cfg, seed=0, device=DEV):
    mu, vt, cf = synth.random_summaries(wl, seed, device)
    pool = L.summary_pool_for(cfg, wl.num_blocks, device)
    d, r, P = wl.head_dim, wl.rank, wl.page_size
    pool[..., :d] = mu
    pool[..., d:d + r * d] = vt.flatten(-2)
    pool[..., d + r * d:] = cf.flatten(-2)
    return pool


def unit_records(wl, cfg, pool_cpu, bt, b, h, n):
    mu, vt, cf = L.split_records(cfg, pool_cpu)
    idx = bt[b, :n].long()
    return f64(mu[idx, h]), f64(vt[idx, h]), f64(cf[idx, h])


# --------------------------------------------------------------------------
# GPU stages
# --------------------------------------------------------------------------
def gpu_build(wl, cfg, g, block_ids=None, fits=None):
    """GPU fit of the given block ids (default: every complete page). The fit
    report of every tile must say converged; `fits` (a list) receives the
    per-tile product counts."""
    pool = L.summary_pool_for(cfg, wl.num_blocks, DEV)
    pool.zero_()
    if block_ids is None:
        ids = []
        for b in range(wl.batch):
            _, _, Jc = lens(wl, b)
            ids += g["block_table"][b, :Jc].tolist()
        block_ids = torch.tensor(ids, dtype=torch.int32, device=DEV)
    info = torch.zeros((max(1, block_ids.numel()), wl.num_kv_heads), dtype=torch.int32, device=DEV)
    L.locks_build_summaries_ex(cfg, g["k_pool"], wl.num_blocks, block_ids, block_ids.numel(), pool, info)
    if block_ids.numel():
        info = info[:block_ids.numel()].cpu()
        valid = ((block_ids >= 0) & (block_ids < wl.num_blocks)).cpu()
        got = info[valid]
        assert bool((got > 0).all()), f"{int((got <= 0).sum())} fits did not meet the Ritz residual bound"
        if fits is not None:
            fits.extend(got.reshape(-1).tolist())
    return pool


def gpu_scores(wl, cfg, g, pool):
    hs = torch.full((wl.batch, wl.num_q_heads, wl.max_pages), float("nan"), device=DEV)
    L.locks_page_score(cfg, g["q"], pool, wl.num_blocks, g["block_table"], g["seq_lens"], wl.batch,
                       wl.max_pages, hs)
    return hs


def gpu_select(wl, cfg, g, head_scores):
    sel = torch.full((wl.batch, wl.num_kv_heads, wl.budget_pages), -7, dtype=torch.int32, device=DEV)
    sig = torch.full((wl.batch, wl.num_kv_heads, wl.max_pages), float("nan"), device=DEV)
    L.locks_select_pages(cfg, head_scores, g["seq_lens"], wl.batch, wl.max_pages, sel, sig)
    return sel, sig


def gpu_decode(wl, cfg, g, sel, ws=None):
    dt = synth.torch_dtype(wl.kv_dtype)
    out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"), dtype=dt, device=DEV)
    lse = torch.full((wl.batch, wl.num_q_heads), float("nan"), device=DEV)
    nbytes = L.locks_workspace_size(cfg, wl.batch, wl.max_pages)
    if ws is None:
        ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    L.locks_sparse_decode(cfg, g["q"], g["k_pool"], g["v_pool"], wl.num_blocks, g["block_table"],
                          g["seq_lens"], sel, wl.batch, wl.max_pages, out, lse, ws, nbytes)
    return out, lse


def gpu_score_select(wl, cfg, g, pool, ws=None):
    sel = torch.full((wl.batch, wl.num_kv_heads, wl.budget_pages), -7, dtype=torch.int32, device=DEV)
    nbytes = L.locks_workspace_size(cfg, wl.batch, wl.max_pages)
    if ws is None:
        ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    L.locks_score_select(cfg, g["q"], pool, wl.num_blocks, g["block_table"], g["seq_lens"], wl.batch,
                         wl.max_pages, sel, ws, nbytes)
    return sel


# --------------------------------------------------------------------------
# oracle stages per unit
# --------------------------------------------------------------------------
def oracle_unit_scores(wl, data, b, h, mu, vt, cf):
    G = wl.group
    q = f64(data["q"][b, h * G:(h + 1) * G])
    return oracle.page_scores(q, mu, vt, cf, wl.softmax_scale)


def oracle_unit_select(wl, b, shat):
    _, J, Jc = lens(wl, b)
    if J <= wl.budget_pages:
        return oracle.select(np.zeros(0), Jc, J, wl.budget_pages), None
    _, sigma = oracle.combine(shat[:, :Jc])
    return oracle.select(sigma, Jc, J, wl.budget_pages), sigma


def oracle_unit_attend(wl, data, b, h, sel):
    T, _, _ = lens(wl, b)
    G, P = wl.group, wl.page_size
    bt = data["block_table"]
    ks, vs = [], []
    for j in sel:
        if j < 0:
            continue
        nv = min(P, T - j * P)
        blk = int(bt[b, j])
        ks.append(f64(data["k_pool"][blk, h, :nv]))
        vs.append(f64(data["v_pool"][blk, h, :nv]))
    q = f64(data["q"][b, h * G:(h + 1) * G])
    if not ks:
        return np.zeros((G, wl.head_dim)), np.full(G, -np.inf)
    return oracle.attend(q, np.concatenate(ks), np.concatenate(vs), wl.softmax_scale)


def check_selection(wl, b, sel_gpu, sel_ora, sigma_ora, tol=SCORE_TOL):
    """Sets equal except pages inside the window around the (k-2)-th key."""
    k = wl.budget_pages
    sg = [int(x) for x in sel_gpu]
    so = [int(x) for x in sel_ora]
    nvalid = sum(1 for x in so if x >= 0)
    assert sg[:nvalid] == sorted(sg[:nvalid]), f"not ascending: {sg}"
    assert all(x == -1 for x in sg[nvalid:]), f"bad padding: {sg}"
    assert sum(1 for x in sg if x >= 0) == nvalid
    if sg == so:
        return 0
    assert sigma_ora is not None, f"sets differ with J <= k: {sg} vs {so}"
    _, J, Jc = lens(wl, b)
    cand = [j for j in range(1, Jc) if j != J - 1]
    ranked = sorted(cand, key=lambda j: (-sigma_ora[j], j))
    kth = sigma_ora[ranked[k - 3]]
    win = tol * max(1.0, abs(kth))
    diff = set(sg) ^ set(so)
    for j in diff:
        assert j in cand and abs(sigma_ora[j] - kth) <= win, \
            f"page {j} (sigma {sigma_ora[j]}) outside window around {kth}"
    return len(diff)


def gpu_decode_step(wl, cfg, g, pool, ws=None):
    """One fused decode step (locks_decode_step); returns (selected, out, lse)."""
    dt = synth.torch_dtype(wl.kv_dtype)
    sel = torch.full((wl.batch, wl.num_kv_heads, wl.budget_pages), -7, dtype=torch.int32, device=DEV)
    out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"), dtype=dt, device=DEV)
    lse = torch.full((wl.batch, wl.num_q_heads), float("nan"), device=DEV)
    nbytes = L.locks_workspace_size(cfg, wl.batch, wl.max_pages)
    if ws is None:
        ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    L.locks_decode_step(cfg, g["q"], pool, g["k_pool"], g["v_pool"], wl.num_blocks, g["block_table"],
                        g["seq_lens"], wl.batch, wl.max_pages, sel, out, lse, ws, nbytes)
    return sel, out, lse


# --------------------------------------------------------------------------
# every unit of a full-size batch against the oracle (host threads)
# --------------------------------------------------------------------------
HOST_THREADS = 8


def check_all_units(wl, data_c, hs_c, sel_c, unit_summaries, threads=HOST_THREADS):
    """For every (sequence, KV head) unit: the GPU page scores hs_c element by
    element against Eq. (2) evaluated by the oracle on the unit's stored
    records (unit_summaries(b, h, Jc) -> (mu, vt, coef) as float64), and the
    GPU selection sel_c against the oracle's under the window rule. data_c
    holds CPU copies of q and block_table. Returns the oracle selections
    [B][H_kv][k] (int32) and the number of pages inside the window."""
    G = wl.group
    units = [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]

    def one(u):
        b, h = u
        _, J, Jc = lens(wl, b)
        s_o = None
        if Jc > 0:
            mu, vt, cf = unit_summaries(b, h, Jc)
            s_o = oracle_unit_scores(wl, data_c, b, h, mu, vt, cf)
            v = mixed_violation(f64(hs_c[b, h * G:(h + 1) * G, :Jc]), s_o)
            assert v <= 1.0, f"unit {u}: score violation {v:.3f} x tolerance"
        sel_o, sigma_o = oracle_unit_select(wl, b, s_o if J > wl.budget_pages else None)
        nd = check_selection(wl, b, sel_c[b, h].tolist(), sel_o.tolist(), sigma_o)
        return u, sel_o, nd

    sel_o_all = torch.full((wl.batch, wl.num_kv_heads, wl.budget_pages), -1, dtype=torch.int32)
    ndiff = 0
    with ThreadPoolExecutor(threads) as ex:
        for (b, h), sel_o, nd in ex.map(one, units):
            sel_o_all[b, h] = torch.from_numpy(sel_o)
            ndiff += nd
    return sel_o_all, ndiff


def check_all_outputs(wl, data, out_c, sel_c, threads=HOST_THREADS):
    """Attention output of every unit against the oracle over the pages listed
    in sel_c (the partial current page's valid tokens only)."""
    G = wl.group
    kp, vp = data["k_pool"], data["v_pool"]
    bt = data["block_table"].cpu()
    q_c = data["q"].cpu()
    units = [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]
    gathered = {}
    for b, h in units:  # device gathers stay on this thread
        T, _, _ = lens(wl, b)
        pages = [j for j in sel_c[b, h].tolist() if j >= 0]
        if not pages:
            continue
        idx = torch.tensor([int(bt[b, j]) for j in pages], device=kp.device)
        nv = [min(wl.page_size, T - j * wl.page_size) for j in pages]
        gathered[(b, h)] = (kp[idx, h].cpu(), vp[idx, h].cpu(), nv)

    def one(u):
        b, h = u
        sl = slice(h * G, (h + 1) * G)
        if u not in gathered:
            assert not np.any(f64(out_c[b, sl])), f"unit {u}: empty selection must give zeros"
            return
        k_, v_, nv = gathered[u]
        ks = np.concatenate([f64(k_[i, :n]) for i, n in enumerate(nv)])
        vs = np.concatenate([f64(v_[i, :n]) for i, n in enumerate(nv)])
        o_ref, _ = oracle.attend(f64(q_c[b, sl]), ks, vs, wl.softmax_scale)
        err = float(np.max(np.abs(f64(out_c[b, sl]) - o_ref)))
        assert err <= out_tol(wl), f"unit {u}: output error {err}"

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, units))


# --------------------------------------------------------------------------
# summary fits: basis-invariant checks against the oracle ([Locks] §4,
# App. A.2 Cor. 1: the top-r right singular subspace of the centred page)
# --------------------------------------------------------------------------
FIT_ENERGY_SLACK = 1e-3   # of the page's total centred energy
FIT_SUBSPACE_TOL = 3e-2   # sine of the angles (Frobenius) to the oracle's leading subspace
FIT_GAP = 0.2             # relative eigen-gap that makes a leading subspace well defined ...
FIT_GAP_ABS = 2.0 ** -6   # ... and its gap against the largest eigenvalue (the stored keys' own
                          # bf16 rounding moves the Gram by ~2^-8 of it, so smaller gaps leave the
                          # subspace undetermined by the data)


def check_fit(keys, vt_stored, ev_o, vt_o, r, energy_slack=FIT_ENERGY_SLACK, subspace_tol=FIT_SUBSPACE_TOL):
    """keys [P][d] as stored; vt_stored [r][d] the GPU basis as stored;
    ev_o [d] the oracle's eigenvalues of D^T D (descending) and vt_o [r][d]
    its basis. With Q an orthonormal basis of the stored span (QR):
      * Eckart-Young: ||D - D Q Q^T||_F^2 <= sum_{l > r} ev_l + slack * sum ev;
      * every leading oracle subspace of size m <= r that is separated from
        the next eigenvalue by a gap both relative to its own eigenvalue and
        against the largest one lies in span(Q) up to the tolerance
        (||(I - Q Q^T) V_o[:m]||_F).
    Returns the number of leading subspaces checked."""
    keys = np.asarray(keys, dtype=np.float64)
    D = keys - keys.mean(0)
    Q, _ = np.linalg.qr(np.asarray(vt_stored, dtype=np.float64).T)  # d x r
    ev = np.clip(np.asarray(ev_o, dtype=np.float64), 0.0, None)
    total = float(np.sum(ev))
    opt = float(np.sum(ev[r:]))
    resid = float(np.linalg.norm(D - D @ Q @ Q.T) ** 2)
    assert resid <= opt + energy_slack * total, \
        f"residual {resid:.6g} > optimum {opt:.6g} + {energy_slack} x {total:.6g}"
    checked = 0
    for m in range(1, r + 1):
        gap = ev[m - 1] - ev[m]
        if ev[m - 1] <= 0 or gap <= FIT_GAP * ev[m - 1] or gap <= FIT_GAP_ABS * ev[0]:
            continue
        Vm = np.asarray(vt_o[:m], dtype=np.float64).T
        off = float(np.linalg.norm(Vm - Q @ (Q.T @ Vm)))
        assert off <= subspace_tol, f"leading {m}-subspace off by {off:.4g}"
        checked += 1
    return checked


# --------------------------------------------------------------------------
# quantized (LOCKS_I4) records: packing from codes and scales, written from
# the record layout that include/locks.h states (test side; no arithmetic of
# the method, only bit placement)
# --------------------------------------------------------------------------
def i4_record_bytes(d, r, P):
    raw = (r + 2) * d // 2 + P * r + 2 * (1 + r + P)
    return (raw + 15) // 16 * 16


def _nibble_slots(d):
    """(word index, bit offset) of element a of a row of d 4-bit fields."""
    a = np.arange(d)
    e = a % 8
    word = (a % 32) // 8 * (d // 32) + a // 32
    m = np.where(e % 2 == 0, e // 2, 4 + (e - 1) // 2)
    return word, 4 * m


def _bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    assert torch.equal(t.float(), torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))), \
        "scales must be bf16 values"
    return t.view(torch.int16).numpy().view(np.uint16)


def pack_i4(qs, d, r, P):
    """Codes/scales (leading dims [...]) -> uint8 records [...][record bytes]."""
    lead = qs["mu_code"].shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    mu_c = np.asarray(qs["mu_code"]).reshape(n, d)
    vt_c = np.asarray(qs["vt_code"]).reshape(n, r, d)
    cf_c = np.asarray(qs["coef_code"]).reshape(n, P, r)
    assert np.abs(vt_c).max(initial=0) <= 7 and np.abs(mu_c).max(initial=0) <= 127
    assert np.abs(cf_c).max(initial=0) <= 127
    word, shift = _nibble_slots(d)
    mu_b = (mu_c + 128).astype(np.uint32)
    fields = np.concatenate([(vt_c + 8).astype(np.uint32), (mu_b >> 4)[:, None], (mu_b & 15)[:, None]], axis=1)
    words = np.zeros((n, r + 2, d // 8), np.uint32)
    for a in range(d):
        words[:, :, word[a]] |= fields[:, :, a] << np.uint32(shift[a])
    out = np.zeros((n, i4_record_bytes(d, r, P)), np.uint8)
    hb = (r + 2) * d // 2
    out[:, :hb] = words.astype("<u4").view(np.uint8).reshape(n, hb)
    out[:, hb:hb + P * r] = (cf_c + 128).astype(np.uint8).reshape(n, P * r)
    sc = np.concatenate([np.asarray(qs["vt_scale"]).reshape(n, r), np.asarray(qs["mu_scale"]).reshape(n, 1),
                         np.asarray(qs["coef_scale"]).reshape(n, P)], axis=1)
    out[:, hb + P * r:hb + P * r + 2 * (1 + r + P)] = _bf16_bits(sc).astype("<u2").view(np.uint8).reshape(n, -1)
    return out.reshape(tuple(lead) + (out.shape[-1],))


def unpack_i4(rec, d, r, P):
    """uint8 records [...][bytes] -> codes (int) and scales (float64) as in
    oracle.quantize_summaries, plus the padding bytes."""
    rec = np.asarray(rec, dtype=np.uint8)
    lead = rec.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    rec = rec.reshape(n, -1)
    hb = (r + 2) * d // 2
    words = np.ascontiguousarray(rec[:, :hb]).view("<u4").reshape(n, r + 2, d // 8)
    word, shift = _nibble_slots(d)
    fields = np.stack([(words[:, :, word[a]] >> np.uint32(shift[a])) & np.uint32(15) for a in range(d)], axis=-1)
    fields = fields.astype(np.int64)
    mu_b = fields[:, r] * 16 + fields[:, r + 1]
    coef_b = rec[:, hb:hb + P * r].astype(np.int64).reshape(n, P, r)
    sb = np.ascontiguousarray(rec[:, hb + P * r:hb + P * r + 2 * (1 + r + P)]).view("<u2").reshape(n, 1 + r + P)
    sc = torch.from_numpy(sb.astype(np.int16)).view(torch.bfloat16).double().numpy()
    res = dict(mu_code=mu_b - 128, vt_code=fields[:, :r] - 8, coef_code=coef_b - 128,
               mu_scale=sc[:, r], vt_scale=sc[:, :r], coef_scale=sc[:, r + 1:],
               padding=rec[:, hb + P * r + 2 * (1 + r + P):])
    return {k: v.reshape(tuple(lead) + v.shape[1:]) for k, v in res.items()}


def i4_pool_from_codes(wl, cfg, qs, device=DEV):
    """Device pool [blocks][Hkv][record bytes] from codes/scales over every (block, head)."""
    qs = {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in qs.items()}
    rec = pack_i4(qs, wl.head_dim, wl.rank, wl.page_size)
    assert rec.shape[-1] == L.locks_summary_record_bytes(cfg)
    return torch.from_numpy(rec).to(device)


def i4_unit_summaries(wl, qs, bt, b, h, n):
    """Dequantized (mu, vt, coef) of the first n pages of unit (b, h), by the oracle."""
    idx = np.asarray(bt[b, :n], dtype=np.int64)
    sub = {k: (v.cpu().numpy() if torch.is_tensor(v) else np.asarray(v))[idx, h] for k, v in qs.items()
           if k != "padding"}
    return oracle.dequantize_summaries(sub)


# --------------------------------------------------------------------------
# host-resident K/V: pinned host memory that the GPU reads over the host link
# --------------------------------------------------------------------------
_hip = None


def _hip_runtime():
    global _hip
    if _hip is None:
        import ctypes
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                 ctypes.c_uint]
        _hip.hipHostGetDevicePointer.restype = ctypes.c_int
    return _hip


def host_pool(t: torch.Tensor):
    """A pinned host copy of the pool `t` and the address the GPU reads it at
    (hipHostGetDevicePointer; raises when the memory is not mapped for the
    device, so no kernel is launched on an unmapped address)."""
    import ctypes
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    dptr = ctypes.c_void_p()
    st = _hip_runtime().hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(h.data_ptr()), 0)
    if st != 0 or not dptr.value:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({st})")
    return h, int(dptr.value)

"""Seeded synthetic workloads for the Locks decode-step path.

This module only draws random inputs (queries, paged K/V, block tables). It
holds none of the method's arithmetic, so both the HIP path and the CPU oracle
can be fed from it.

Key generator, per (sequence, KV head, page p) and token i:
    k_i = c_p + B_p a_i + noise * eps_i
    B_p : orthonormal d x R basis (Gram-Schmidt of a Gaussian d x R matrix)
    a_i ~ N(0, diag(basis_var)),  eps_i ~ N(0, I_d)
    c_p ~ N(0, centroid_std^2 I), or with ar_rho > 0 an AR(1) drift along the
          sequence: c_0 ~ N(0, s^2 I), c_p = rho c_{p-1} + sqrt(1 - rho^2) eta_p,
          eta_p ~ N(0, s^2 I) (stationary variance s^2)
A constant `key_offset` may be added to every coordinate of every key (a
common offset, as in models whose keys share a large mean). Values ~ N(0, I_d);
queries q_g ~ N(0, I_d) (drawn first). In `n_needles`
pages per (sequence, KV head), chosen uniformly without replacement among the
complete pages other than the sink page 0 and the current page J-1, one
uniformly chosen token key is replaced by needle_scale * qhat, qhat the unit
mean of that KV head's query group. Everything is drawn in float32 and cast
(round-to-nearest-even) to the storage dtype. Token slots past the context
length in the last page hold the poison value 100.

Paged layout: K and V pools are [num_blocks][H_kv][P][d]; block_table[b][j]
is the physical block of logical page j of sequence b, a seeded random
permutation so consecutive pages are scattered like a real paged allocator.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_kv_heads: int
    group: int
    head_dim: int
    page_size: int
    seq_lens: tuple          # one context length (tokens) per sequence
    rank: int
    budget_pages: int
    kv_dtype: str            # "bf16" or "f32"
    summary_dtype: str       # "bf16", "f32" or "i4" (quantized records)
    centroid_std: float = 0.5
    ar_rho: float = 0.0
    basis_var: tuple = (4.0, 2.0, 1.0, 0.5, 0.25, 0.125)
    noise: float = 0.05
    n_needles: int = 0
    needle_scale: float = 6.0
    extra_blocks: int = 0    # unused physical blocks appended to the pools
    key_offset: float = 0.0  # added to every coordinate of every key (a common offset)

    @property
    def num_q_heads(self) -> int:
        return self.num_kv_heads * self.group

    @property
    def max_pages(self) -> int:
        return max(-(-int(t) // self.page_size) for t in self.seq_lens)

    @property
    def num_blocks(self) -> int:
        return self.batch * self.max_pages + self.extra_blocks

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _uniform(batch, t):
    return tuple([int(t)] * batch)


# The workload shapes the path is measured and checked on.
WORKLOADS = {
    # tiny fp32 case: 64 full pages of 16 + an 8-token partial page
    "tiny_f32": Workload("tiny_f32", 1, 1, 4, 64, 16, _uniform(1, 1032), 4, 8, "f32", "f32",
                         centroid_std=0.5, basis_var=(4.0, 2.0, 1.0, 0.5), n_needles=3),
    # Llama-3.1-8B-shaped layer at 32K, batch 1
    "llama8b_32k": Workload("llama8b_32k", 1, 8, 4, 128, 64, _uniform(1, 32768), 4, 32,
                            "bf16", "bf16", centroid_std=0.5, n_needles=8),
    # 128K context, batch 8, AR(1) centroids
    "llama8b_128k_b8": Workload("llama8b_128k_b8", 8, 8, 4, 128, 64, _uniform(8, 131072), 8, 32,
                                "bf16", "bf16", centroid_std=0.5, ar_rho=0.99, n_needles=16),
    # the 128K-context batch-8 shape with the pages' default 16-token pages (the same
    # 2048-token budget is k = 128 pages; rank swept by the caller)
    "llama8b_128k_b8_p16": Workload("llama8b_128k_b8_p16", 8, 8, 4, 128, 16, _uniform(8, 131072), 8, 128,
                                    "bf16", "bf16", centroid_std=0.5, ar_rho=0.99, n_needles=16),
    # long-context stress: 512K, batch 1 (rank swept by the caller)
    "llama8b_512k": Workload("llama8b_512k", 1, 8, 4, 128, 64, _uniform(1, 524288), 4, 32,
                             "bf16", "bf16", centroid_std=0.5, n_needles=8),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _orthonormal(x: torch.Tensor) -> torch.Tensor:
    """Modified Gram-Schmidt over the last dim's columns: x [..., d, R]."""
    cols = []
    for j in range(x.shape[-1]):
        v = x[..., j]
        for u in cols:
            v = v - (u * v).sum(-1, keepdim=True) * u
        v = v / v.norm(dim=-1, keepdim=True)
        cols.append(v)
    return torch.stack(cols, dim=-1)


def generate(wl: Workload, seed: int = 0, device="cpu"):
    """Draw one batch. Returns a dict of tensors on `device`:
    q [B][Hq][d], k_pool/v_pool [blocks][Hkv][P][d], block_table [B][max_pages]
    int32, seq_lens [B] int32, needles (list of (b, h, page, token))."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    B, Hkv, G, d, P = wl.batch, wl.num_kv_heads, wl.group, wl.head_dim, wl.page_size
    Hq = Hkv * G
    maxp = wl.max_pages
    dt = torch_dtype(wl.kv_dtype)
    f32 = torch.float32

    q = torch.randn((B, Hq, d), generator=g, device=dev, dtype=f32)
    perm = torch.randperm(wl.num_blocks, generator=g, device=dev)
    bt = perm[: B * maxp].reshape(B, maxp).to(torch.int32)
    k_pool = torch.zeros((wl.num_blocks, Hkv, P, d), device=dev, dtype=dt)
    v_pool = torch.zeros((wl.num_blocks, Hkv, P, d), device=dev, dtype=dt)
    R = len(wl.basis_var)
    sd = torch.tensor([math.sqrt(v) for v in wl.basis_var], device=dev, dtype=f32)
    needles = []
    for b in range(B):
        T = int(wl.seq_lens[b])
        J = -(-T // P)
        Jc = T // P
        if J == 0:
            continue
        # centroids [Hkv][J][d]
        if wl.ar_rho > 0.0:
            eta = torch.randn((Hkv, J, d), generator=g, device=dev, dtype=f32) * wl.centroid_std
            c = torch.empty_like(eta)
            c[:, 0] = eta[:, 0]
            a = wl.ar_rho
            s = math.sqrt(1.0 - a * a)
            for p in range(1, J):
                c[:, p] = a * c[:, p - 1] + s * eta[:, p]
        else:
            c = torch.randn((Hkv, J, d), generator=g, device=dev, dtype=f32) * wl.centroid_std
        basis = _orthonormal(torch.randn((Hkv, J, d, R), generator=g, device=dev, dtype=f32))
        coef = torch.randn((Hkv, J, P, R), generator=g, device=dev, dtype=f32) * sd
        keys = c[:, :, None, :] + torch.einsum("hjdr,hjpr->hjpd", basis, coef)
        keys = keys + wl.noise * torch.randn((Hkv, J, P, d), generator=g, device=dev, dtype=f32)
        if wl.key_offset:
            keys = keys + wl.key_offset
        vals = torch.randn((Hkv, J, P, d), generator=g, device=dev, dtype=f32)
        # needles
        if wl.n_needles > 0:
            qh = q[b].reshape(Hkv, G, d).mean(1)
            qh = qh / qh.norm(dim=-1, keepdim=True)
            cand = [j for j in range(1, Jc) if j != J - 1]
            for h in range(Hkv):
                n = min(wl.n_needles, len(cand))
                if n == 0:
                    continue
                pick = torch.randperm(len(cand), generator=g, device=dev)[:n].tolist()
                toks = torch.randint(0, P, (n,), generator=g, device=dev).tolist()
                for pi, ti in zip(pick, toks):
                    pg = cand[pi]
                    keys[h, pg, ti] = wl.needle_scale * qh[h]
                    needles.append((b, h, pg, ti))
        # slots beyond T in the last page hold a large poison value, so a
        # reader that forgets the token count shows up at once
        if T % P:
            keys[:, J - 1, T % P:] = 100.0
            vals[:, J - 1, T % P:] = 100.0
        blocks = bt[b, :J].long()
        k_pool[blocks] = keys.permute(1, 0, 2, 3).to(dt)
        v_pool[blocks] = vals.permute(1, 0, 2, 3).to(dt)
    seq_lens = torch.tensor([int(t) for t in wl.seq_lens], dtype=torch.int32, device=dev)
    return dict(q=q.to(dt), k_pool=k_pool, v_pool=v_pool, block_table=bt, seq_lens=seq_lens,
                needles=needles)


def random_summaries(wl: Workload, seed: int = 0, device="cpu"):
    """Random summary records (not fits): mu ~ N(0, 0.25 I), V orthonormal,
    C ~ N(0, diag(basis_var[:r]) * P)-scaled, cast to the summary dtype.
    Returns (mu [blocks][Hkv][d], vt [blocks][Hkv][r][d], coef [blocks][Hkv][P][r])."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed) + 7919)
    n, H, d, P, r = wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.rank
    f32 = torch.float32
    mu = torch.randn((n, H, d), generator=g, device=dev, dtype=f32) * 0.5
    v = _orthonormal(torch.randn((n, H, d, r), generator=g, device=dev, dtype=f32))
    var = list(wl.basis_var) + [wl.noise ** 2 * d] * max(0, r - len(wl.basis_var))
    sd = torch.tensor([math.sqrt(x) for x in var[:r]], device=dev, dtype=f32)
    coef = torch.randn((n, H, P, r), generator=g, device=dev, dtype=f32) * sd
    dt = torch_dtype(wl.summary_dtype)
    return mu.to(dt), v.transpose(-1, -2).contiguous().to(dt), coef.to(dt)


def random_i4_codes(wl: Workload, seed: int = 0, device="cpu"):
    """Random quantized summary records (codes and scales, not fits) for every
    (block, KV head): 4-bit basis codes uniform in [-7, 7], 8-bit centroid and
    coefficient codes uniform in [-127, 127], scales log-uniform and cast to
    bf16 (basis 0.02-0.07, centroid 0.004-0.016, coefficients 0.004-0.05).
    Returns a dict of tensors: mu_code [blocks][Hkv][d], vt_code [..][r][d],
    coef_code [..][P][r] (int32) and mu_scale [blocks][Hkv], vt_scale [..][r],
    coef_scale [..][P] (float32 holding bf16 values)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed) + 104729)
    n, H, d, P, r = wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.rank
    i32 = torch.int32

    def codes(shape, L):
        return torch.randint(-L, L + 1, shape, generator=g, device=dev, dtype=i32)

    def scales(shape, lo, hi):
        u = torch.rand(shape, generator=g, device=dev, dtype=torch.float32)
        return torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))).to(torch.bfloat16).float()

    return dict(mu_code=codes((n, H, d), 127), vt_code=codes((n, H, r, d), 7),
                coef_code=codes((n, H, P, r), 127), mu_scale=scales((n, H), 0.004, 0.016),
                vt_scale=scales((n, H, r), 0.02, 0.07), coef_scale=scales((n, H, P), 0.004, 0.05))


# The whole-model decode step: `layers` attention layers of a batch whose
# sequence s holds base_len + stagger * s tokens, each step appending one token
# to every sequence (so with stagger 4 and 16 sequences at most one sequence
# completes a page per step).
def query_sequence(q0: torch.Tensor, steps: int, rho: float, seed: int = 0) -> torch.Tensor:
    """Queries of `steps` consecutive decode steps, [steps][*q0.shape] in
    q0's dtype on q0's device: an AR(1) sequence per element,
    q_0 = q0, q_{t+1} = rho q_t + sqrt(1 - rho^2) eps_t, eps_t iid standard
    normal, so each step's queries keep the N(0, 1) marginal of generate()'s q
    while consecutive steps stay correlated (rho = 0: independent queries)."""
    g = torch.Generator(device=q0.device)
    g.manual_seed(int(seed) + 77)
    out = torch.empty((steps,) + tuple(q0.shape), dtype=q0.dtype, device=q0.device)
    cur = q0.float()
    s = math.sqrt(max(0.0, 1.0 - rho * rho))
    for t in range(steps):
        out[t] = cur.to(q0.dtype)
        eps = torch.randn(cur.shape, generator=g, device=q0.device, dtype=torch.float32)
        cur = rho * cur + s * eps
    return out


FULL_STEP = dict(layers=32, batch=16, kv_heads=8, group=4, head_dim=128, page_size=64, rank=4,
                 budget_pages=32, base_len=65536, stagger=4)


def full_step_inputs(steps: int, seed: int = 0, device="cuda", slabs: int = 2, log=None, **over):
    """Inputs of `steps` whole-model decode steps (FULL_STEP shape unless
    overridden). Keys and values of each layer come from generate() with the
    128K batch-8 generator (six signal directions plus noise, AR(1) centroids,
    needle tokens): `slabs` independently drawn slabs of the whole batch, layer
    l holding slab l % slabs under its own random block permutation inside
    the layer's block range [l nb, (l + 1) nb), so every layer's pages sit at
    different physical blocks. Queries are drawn per layer.

    Returns dict: k_pool, v_pool [layers * nb][H_kv][P][d] bf16; block_table
    [layers][B][max_pages] int32; q [layers][B][H_q][d] bf16; lens0 (list of
    initial lengths); build_ids [steps][layers] int32 (device): the block of
    every layer of the page that the token of step t completes, -1 when no
    page completes; num_blocks, max_pages."""
    c = dict(FULL_STEP, **over)
    nl, B, Hkv, G, d, P = c["layers"], c["batch"], c["kv_heads"], c["group"], c["head_dim"], c["page_size"]
    lens0 = [c["base_len"] + c["stagger"] * s for s in range(B)]
    lens_end = tuple(x + steps for x in lens0)
    wl = Workload("full_step_slab", B, Hkv, G, d, P, lens_end, c["rank"], c["budget_pages"], "bf16", "bf16",
                  centroid_std=0.5, ar_rho=0.99, n_needles=8)
    maxp, nb = wl.max_pages, wl.num_blocks
    NB = nl * nb
    dev = torch.device(device)
    k_pool = torch.empty((NB, Hkv, P, d), dtype=torch.bfloat16, device=dev)
    v_pool = torch.empty((NB, Hkv, P, d), dtype=torch.bfloat16, device=dev)
    bt = torch.empty((nl, B, maxp), dtype=torch.int32, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed) + 31)
    for si in range(slabs):
        slab = generate(wl, int(seed) * 1000 + si, dev)
        for layer in range(si, nl, slabs):
            # physical block of slab block x in this layer
            perm = torch.randperm(nb, generator=g, device=dev)
            k_pool[layer * nb + perm] = slab["k_pool"]
            v_pool[layer * nb + perm] = slab["v_pool"]
            bt[layer] = (layer * nb + perm[slab["block_table"].long()]).to(torch.int32)
        del slab
        if log:
            log(f"slab {si + 1}/{slabs} placed")
    q = torch.randn((nl, B, Hkv * G, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    bt_c = bt.cpu()
    ids = torch.full((max(1, steps), nl), -1, dtype=torch.int32)
    for t in range(steps):
        for s in range(B):
            T = lens0[s] + t + 1  # length once the token of step t is in
            if T % P == 0:
                ids[t] = bt_c[:, s, T // P - 1]
    return dict(k_pool=k_pool, v_pool=v_pool, block_table=bt, q=q, lens0=lens0, build_ids=ids.to(dev),
                num_blocks=NB, max_pages=maxp, shape=c)

"""Plain fp64 CPU oracle for the Locks decode-step path (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product library never does, and the
two share no code: this wrapper marshals numpy arrays into the plain C++ in
``locks_oracle.cpp`` and contains no arithmetic of the method beyond what is
listed per function below (a gather by block table, widening to float64).

Formulas follow "Locks: Page-Local Compact Key Summaries for Efficient
Long-Context Decoding" (arXiv 2607.24555): §2 Eq. (1) exact page LSE, §3-§4
summary fit, §4 Eq. (2) reconstructed page LSE, §4 share-average combine and
selection, §2 restricted attention, §4 / App. C.7 quantized ("i4") summary
storage.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "locks_oracle.cpp")
_LIB_DEFAULT = os.path.join(_HERE, "liblocks_oracle.so")
# LOCKS_ORACLE_LIB names another build of the same source to load instead
# (the sanitizer test uses one); it is taken as it is, never rebuilt
_LIB = os.environ.get("LOCKS_ORACLE_LIB") or _LIB_DEFAULT
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def build(force: bool = False) -> str:
    """Compile the oracle with g++ (plain -O2, no fast-math)."""
    if _LIB != _LIB_DEFAULT:
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
             "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.lo_build_pages.argtypes = [ctypes.c_int] * 4 + [_dp] * 5 + [_ip, ctypes.c_int]
        L.lo_round_bf16.argtypes = [_dp, ctypes.c_long, _dp]
        L.lo_round_bf16.restype = None
        L.lo_page_scores.argtypes = [ctypes.c_int] * 5 + [_dp] * 4 + [ctypes.c_double, _dp]
        L.lo_exact_page_lse.argtypes = [ctypes.c_int] * 4 + [_ip, _dp, _dp, ctypes.c_double, _dp]
        L.lo_combine.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        L.lo_select.argtypes = [ctypes.c_int] * 3 + [_dp, _ip]
        L.lo_attend.argtypes = [ctypes.c_int] * 3 + [_dp] * 3 + [ctypes.c_double, _dp, _dp]
        L.lo_quantize_summaries.argtypes = [ctypes.c_int] * 4 + [_dp] * 3 + [_ip] * 3 + [_dp] * 3
        _lib = L
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _check(rc: int, what: str) -> None:
    if rc < 0:
        raise ValueError(f"oracle {what}: bad arguments (rc={rc})")


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


# --------------------------------------------------------------------------
# O1: summary fit ([Locks] §3-§4)
# --------------------------------------------------------------------------
def build_pages(keys, r: int, threads: int | None = None):
    """keys [n][P][d] -> (mu [n][d], vt [n][r][d], coef [n][P][r], evals [n][d], sweeps [n]).

    V is the top-r eigenvectors of H_j = D_j^T D_j by cyclic Jacobi in fp64,
    sign-fixed so the largest-magnitude entry of each is positive."""
    k = _f64(keys)
    n, P, d = k.shape
    mu = np.zeros((n, d)); vt = np.zeros((n, r, d)); coef = np.zeros((n, P, r))
    ev = np.zeros((n, d)); sw = np.zeros(n, dtype=np.int32)
    rc = lib().lo_build_pages(n, P, d, r, _p(k), _p(mu), _p(vt), _p(coef), _p(ev),
                              sw.ctypes.data_as(_ip), threads or default_threads())
    _check(rc, "build_pages")
    return mu, vt, coef, ev, sw


def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even), returned as float64."""
    a = _f64(x)
    out = np.empty_like(a)
    lib().lo_round_bf16(_p(a), a.size, _p(out))
    return out


# --------------------------------------------------------------------------
# Quantized summary storage ([Locks] §4 "i4" variants, App. C.7)
# --------------------------------------------------------------------------
def quantize_summaries(mu, vt, coef):
    """Full-precision (mu [n][d], vt [n][r][d], coef [n][P][r]) -> int4/int8 codes and
    bf16 scales: dict(mu_code [n][d], vt_code [n][r][d], coef_code [n][P][r] (int32),
    mu_scale [n], vt_scale [n][r], coef_scale [n][P] (float64 holding bf16 values)).

    One symmetric scale per basis vector (4-bit codes in [-7, 7]), per token's
    coefficient row and for the centroid (8-bit codes in [-127, 127]); scale =
    bf16(max|x| / L), code = round-half-even(x / scale), in double precision."""
    mu = _f64(mu); vt = _f64(vt); coef = _f64(coef)
    n, r, d = vt.shape
    P = coef.shape[1]
    out = dict(mu_code=np.zeros((n, d), np.int32), vt_code=np.zeros((n, r, d), np.int32),
               coef_code=np.zeros((n, P, r), np.int32), mu_scale=np.zeros(n),
               vt_scale=np.zeros((n, r)), coef_scale=np.zeros((n, P)))
    ip = lambda a: a.ctypes.data_as(_ip)
    _check(lib().lo_quantize_summaries(n, d, P, r, _p(mu), _p(vt), _p(coef), ip(out["mu_code"]),
                                       ip(out["vt_code"]), ip(out["coef_code"]),
                                       _p(out["mu_scale"]), _p(out["vt_scale"]),
                                       _p(out["coef_scale"])), "quantize_summaries")
    return out


def dequantize_summaries(qs):
    """Stored values of quantized summaries: code * scale of its group, in float64.
    Returns (mu [n][d], vt [n][r][d], coef [n][P][r])."""
    mu = qs["mu_code"] * qs["mu_scale"][:, None]
    vt = qs["vt_code"] * qs["vt_scale"][:, :, None]
    coef = qs["coef_code"] * qs["coef_scale"][:, :, None]
    return mu.astype(np.float64), vt.astype(np.float64), coef.astype(np.float64)


# --------------------------------------------------------------------------
# O2: page scores ([Locks] §4 Eq. (2)) and exact page LSE (§2 Eq. (1))
# --------------------------------------------------------------------------
def page_scores(q, mu, vt, coef, scale: float) -> np.ndarray:
    """q [G][d]; mu [n][d]; vt [n][r][d]; coef [n][P][r] -> shat [G][n]."""
    q = _f64(q); mu = _f64(mu); vt = _f64(vt); coef = _f64(coef)
    G, d = q.shape
    n, r, _ = vt.shape
    P = coef.shape[1]
    out = np.zeros((G, n))
    _check(lib().lo_page_scores(G, d, r, P, n, _p(q), _p(mu), _p(vt), _p(coef), float(scale),
                                _p(out)), "page_scores")
    return out


def exact_page_lse(q, keys, scale: float, n_valid=None) -> np.ndarray:
    """q [G][d]; keys [n][P][d] -> s [G][n]; n_valid [n] limits each page's tokens."""
    q = _f64(q); k = _f64(keys)
    G, d = q.shape
    n, P, _ = k.shape
    out = np.zeros((G, n))
    nv = None
    if n_valid is not None:
        nv = np.ascontiguousarray(np.asarray(n_valid, dtype=np.int32))
    _check(lib().lo_exact_page_lse(G, d, P, n, nv.ctypes.data_as(_ip) if nv is not None else None,
                                   _p(q), _p(k), float(scale), _p(out)), "exact_page_lse")
    return out


# --------------------------------------------------------------------------
# O3/O4: combine and select ([Locks] §4)
# --------------------------------------------------------------------------
def combine(s):
    """s [G][n] -> (logz [G], sigma [n]) with sigma = log of the share average."""
    s = _f64(s)
    G, n = s.shape
    logz = np.zeros(G); sigma = np.zeros(n)
    _check(lib().lo_combine(G, n, _p(s), _p(logz), _p(sigma)), "combine")
    return logz, sigma


def select(sigma, n_complete: int, J: int, k: int) -> np.ndarray:
    """Ascending page ids [k] (-1 padded): sink 0, current J-1, top-(k-2) by sigma."""
    sg = _f64(sigma) if n_complete > 0 else np.zeros(1)
    sel = np.full(k, -1, dtype=np.int32)
    rc = lib().lo_select(n_complete, J, k, _p(sg), sel.ctypes.data_as(_ip))
    _check(rc, "select")
    return sel


# --------------------------------------------------------------------------
# O5: attention over a token set ([Locks] §2)
# --------------------------------------------------------------------------
def attend(q, keys, vals, scale: float):
    """q [G][d]; keys/vals [n][d] -> (o [G][d], lse [G])."""
    q = _f64(q); k = _f64(keys); v = _f64(vals)
    G, d = q.shape
    n = k.shape[0]
    out = np.zeros((G, d)); lse = np.zeros(G)
    _check(lib().lo_attend(G, d, n, _p(q), _p(k), _p(v), float(scale), _p(out), _p(lse)),
           "attend")
    return out, lse


# --------------------------------------------------------------------------
# Whole decode step over a paged batch (glue: gathers by block table, then
# calls the functions above per (sequence, KV head) unit on a thread pool).
# --------------------------------------------------------------------------
def unit_pages(pool, block_table_row, n_pages: int, head: int) -> np.ndarray:
    """Gather [n_pages][...] for one KV head from a paged pool [blocks][H_kv][...]."""
    return pool[np.asarray(block_table_row[:n_pages], dtype=np.int64), head]


def decode_step(q, sum_mu, sum_vt, sum_coef, k_pool, v_pool, block_table, seq_lens,
                page_size: int, budget: int, scale: float, units=None, threads=None,
                want_scores=False):
    """Score -> combine -> select -> attend for each (sequence, KV head) unit.

    q [B][Hq][d]; sum_* [blocks][Hkv][...] (widened summaries); *_pool
    [blocks][Hkv][P][d]; block_table [B][max_pages]; seq_lens [B].
    Returns dict with per-unit results keyed by (b, h)."""
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    if units is None:
        units = [(b, h) for b in range(B) for h in range(Hkv)]

    def one(u):
        b, h = u
        T = int(seq_lens[b])
        J = -(-T // page_size)
        Jc = T // page_size
        qg = q[b, h * G:(h + 1) * G]
        res = {}
        if J > budget:
            mu = unit_pages(sum_mu, block_table[b], Jc, h)
            vt = unit_pages(sum_vt, block_table[b], Jc, h)
            cf = unit_pages(sum_coef, block_table[b], Jc, h)
            s = page_scores(qg, mu, vt, cf, scale)
            logz, sigma = combine(s)
            if want_scores:
                res["shat"] = s; res["sigma"] = sigma; res["logz"] = logz
        else:
            sigma = np.zeros(0)
        sel = select(sigma, Jc, J, budget)
        ks, vs = [], []
        for j in sel:
            if j < 0:
                continue
            nv = min(page_size, T - j * page_size)
            blk = int(block_table[b][j])
            ks.append(k_pool[blk, h, :nv]); vs.append(v_pool[blk, h, :nv])
        o, lse = attend(qg, np.concatenate(ks), np.concatenate(vs), scale)
        res.update(sel=sel, out=o, lse=lse)
        return u, res

    nt = threads or default_threads()
    if nt == 1:
        return dict(one(u) for u in units)
    with ThreadPoolExecutor(nt) as ex:
        return dict(ex.map(one, units))

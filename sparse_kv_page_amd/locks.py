"""ctypes binding of liblocks.so (include/locks.h), same names as the C ABI.

Argument marshalling only: tensors are passed as device pointers and the
stream is torch's current HIP stream. Every call raises LocksError on a
non-OK status. The binding loads the in-tree liblocks.so and raises if it is
missing; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LOCKS_LIB names another build of the same sources to load instead (the
# sanitizer test loads a build whose host code carries ASan and UBSan)
LIB_PATH = os.environ.get("LOCKS_LIB") or os.path.join(_HERE, "liblocks.so")

LOCKS_OK = 0
LOCKS_E_INVALID_ARG = -1
LOCKS_E_UNSUPPORTED = -2
LOCKS_E_WORKSPACE = -3
LOCKS_E_HIP = -4
LOCKS_BF16 = 0
LOCKS_F32 = 1
LOCKS_I4 = 2  # summary dtype only: 4-bit basis, 8-bit centroid and coefficients, bf16 scales

# every exported entry point declared in include/locks.h
EXPORTED = ("locks_status_string", "locks_version", "locks_summary_record_bytes",
            "locks_workspace_size", "locks_build_summaries", "locks_build_summaries_ex",
            "locks_page_score",
            "locks_select_pages", "locks_score_select", "locks_sparse_decode",
            "locks_decode_step", "locks_hot_cache_layout", "locks_hot_cache_init",
            "locks_decode_step_cached")

# fields of the hot-page cache buffer, in order (locks_hot_cache_layout)
HOT_CACHE_FIELDS = ("stats", "meta", "clock", "slot_of", "tile_of", "stamp", "flags", "k", "v")
HOT_CACHE_STATS = ("hits", "misses", "refreshes", "shared", "failed", "steps")


class LocksError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("budget_pages", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("summary_dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


def make_config(head_dim, page_size, rank, num_q_heads, num_kv_heads, budget_pages,
                kv_dtype="bf16", summary_dtype=None, softmax_scale=None) -> Config:
    dt = {"bf16": LOCKS_BF16, "f32": LOCKS_F32, "i4": LOCKS_I4}
    sd = summary_dtype or kv_dtype
    scale = softmax_scale if softmax_scale is not None else head_dim ** -0.5
    return Config(head_dim, page_size, rank, num_q_heads, num_kv_heads, budget_pages,
                  dt[kv_dtype] if isinstance(kv_dtype, str) else kv_dtype,
                  dt[sd] if isinstance(sd, str) else sd, scale)


def config_for(wl) -> Config:
    """Config of a synth.Workload."""
    return make_config(wl.head_dim, wl.page_size, wl.rank, wl.num_q_heads, wl.num_kv_heads,
                       wl.budget_pages, wl.kv_dtype, wl.summary_dtype, wl.softmax_scale)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_kv_page_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cp = ctypes.POINTER(Config)
        L.locks_status_string.argtypes = [ctypes.c_int]
        L.locks_status_string.restype = ctypes.c_char_p
        L.locks_version.restype = ctypes.c_int
        L.locks_summary_record_bytes.argtypes = [cp]
        L.locks_summary_record_bytes.restype = sz
        L.locks_workspace_size.argtypes = [cp, i32, i32, ctypes.POINTER(sz)]
        L.locks_build_summaries.argtypes = [cp, vp, i64, vp, i32, vp, vp]
        L.locks_build_summaries_ex.argtypes = [cp, vp, i64, vp, i32, vp, vp, vp]
        L.locks_page_score.argtypes = [cp, vp, vp, i64, vp, vp, i32, i32, vp, vp]
        L.locks_select_pages.argtypes = [cp, vp, vp, i32, i32, vp, vp, vp]
        L.locks_score_select.argtypes = [cp, vp, vp, i64, vp, vp, i32, i32, vp, vp, sz, vp]
        L.locks_sparse_decode.argtypes = [cp, vp, vp, vp, i64, vp, vp, vp, i32, i32, vp, vp, vp,
                                          sz, vp]
        L.locks_decode_step.argtypes = [cp, vp, vp, vp, vp, i64, vp, vp, i32, i32, vp, vp, vp, vp,
                                        sz, vp]
        L.locks_hot_cache_layout.argtypes = [cp, i64, i32, ctypes.POINTER(i64), ctypes.POINTER(sz)]
        L.locks_hot_cache_init.argtypes = [cp, vp, i64, i32, vp]
        L.locks_decode_step_cached.argtypes = [cp, vp, vp, vp, vp, i64, vp, vp, i32, i32, vp, vp, vp, vp,
                                               i32, vp, sz, vp]
        for name in ("locks_workspace_size", "locks_build_summaries", "locks_build_summaries_ex",
                     "locks_page_score",
                     "locks_select_pages", "locks_score_select", "locks_sparse_decode",
                     "locks_decode_step", "locks_hot_cache_layout", "locks_hot_cache_init",
                     "locks_decode_step_cached"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(st: int) -> str:
    return lib().locks_status_string(st).decode()


def _check(fn: str, st: int) -> None:
    if st != LOCKS_OK:
        raise LocksError(fn, st, status_string(st))


def _ptr(t):
    """Device address of a tensor (ints pass through as raw device addresses).

    The kernels index every buffer as dense row-major memory on the GPU, so a
    tensor in host memory or a strided view is refused here rather than read
    as the wrong bytes (or as an address the GPU cannot reach)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"expected a GPU tensor, got one on {t.device}; pass host-resident "
                         "buffers as their mapped device address (an int)")
    if not t.is_contiguous():
        raise ValueError(f"expected a contiguous tensor, got strides {t.stride()} "
                         f"for shape {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def locks_version() -> int:
    return lib().locks_version()


def locks_summary_record_bytes(cfg: Config) -> int:
    return lib().locks_summary_record_bytes(ctypes.byref(cfg))


def locks_workspace_size(cfg: Config, batch: int, max_pages: int) -> int:
    out = ctypes.c_size_t(0)
    _check("locks_workspace_size", lib().locks_workspace_size(ctypes.byref(cfg), batch, max_pages,
                                                              ctypes.byref(out)))
    return out.value


def locks_build_summaries(cfg, k_pool, num_blocks, block_ids, n_ids, summary_pool, stream=None):
    _check("locks_build_summaries",
           lib().locks_build_summaries(ctypes.byref(cfg), _ptr(k_pool), int(num_blocks),
                                       _ptr(block_ids), int(n_ids), _ptr(summary_pool),
                                       _stream(stream)))


def locks_build_summaries_ex(cfg, k_pool, num_blocks, block_ids, n_ids, summary_pool, fit_info,
                             stream=None):
    _check("locks_build_summaries_ex",
           lib().locks_build_summaries_ex(ctypes.byref(cfg), _ptr(k_pool), int(num_blocks),
                                          _ptr(block_ids), int(n_ids), _ptr(summary_pool),
                                          _ptr(fit_info), _stream(stream)))


def locks_page_score(cfg, q, summary_pool, num_blocks, block_table, seq_lens, batch, max_pages,
                     head_scores, stream=None):
    _check("locks_page_score",
           lib().locks_page_score(ctypes.byref(cfg), _ptr(q), _ptr(summary_pool), int(num_blocks),
                                  _ptr(block_table), _ptr(seq_lens), int(batch), int(max_pages),
                                  _ptr(head_scores), _stream(stream)))


def locks_select_pages(cfg, head_scores, seq_lens, batch, max_pages, selected, page_sigma,
                       stream=None):
    _check("locks_select_pages",
           lib().locks_select_pages(ctypes.byref(cfg), _ptr(head_scores), _ptr(seq_lens),
                                    int(batch), int(max_pages), _ptr(selected), _ptr(page_sigma),
                                    _stream(stream)))


def locks_score_select(cfg, q, summary_pool, num_blocks, block_table, seq_lens, batch, max_pages,
                       selected, ws, ws_bytes, stream=None):
    _check("locks_score_select",
           lib().locks_score_select(ctypes.byref(cfg), _ptr(q), _ptr(summary_pool),
                                    int(num_blocks), _ptr(block_table), _ptr(seq_lens), int(batch),
                                    int(max_pages), _ptr(selected), _ptr(ws), int(ws_bytes),
                                    _stream(stream)))


def locks_sparse_decode(cfg, q, k_pool, v_pool, num_blocks, block_table, seq_lens, selected,
                        batch, max_pages, out, lse, ws, ws_bytes, stream=None):
    _check("locks_sparse_decode",
           lib().locks_sparse_decode(ctypes.byref(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                     int(num_blocks), _ptr(block_table), _ptr(seq_lens),
                                     _ptr(selected), int(batch), int(max_pages), _ptr(out),
                                     _ptr(lse), _ptr(ws), int(ws_bytes), _stream(stream)))


def locks_decode_step(cfg, q, summary_pool, k_pool, v_pool, num_blocks, block_table, seq_lens, batch,
                      max_pages, selected, out, lse, ws, ws_bytes, stream=None):
    _check("locks_decode_step",
           lib().locks_decode_step(ctypes.byref(cfg), _ptr(q), _ptr(summary_pool), _ptr(k_pool),
                                   _ptr(v_pool), int(num_blocks), _ptr(block_table), _ptr(seq_lens),
                                   int(batch), int(max_pages), _ptr(selected), _ptr(out), _ptr(lse),
                                   _ptr(ws), int(ws_bytes), _stream(stream)))


def locks_hot_cache_layout(cfg: Config, num_blocks: int, capacity: int):
    """(offsets dict by HOT_CACHE_FIELDS name, total bytes) of a hot-page cache buffer."""
    offs = (ctypes.c_int64 * len(HOT_CACHE_FIELDS))()
    nb = ctypes.c_size_t(0)
    _check("locks_hot_cache_layout",
           lib().locks_hot_cache_layout(ctypes.byref(cfg), int(num_blocks), int(capacity), offs, ctypes.byref(nb)))
    return dict(zip(HOT_CACHE_FIELDS, list(offs))), nb.value


def locks_hot_cache_init(cfg, cache, num_blocks, capacity, stream=None):
    _check("locks_hot_cache_init",
           lib().locks_hot_cache_init(ctypes.byref(cfg), _ptr(cache), int(num_blocks), int(capacity),
                                      _stream(stream)))


def locks_decode_step_cached(cfg, q, summary_pool, k_pool, v_pool, num_blocks, block_table, seq_lens, batch,
                             max_pages, selected, out, lse, cache, capacity, ws, ws_bytes, stream=None):
    _check("locks_decode_step_cached",
           lib().locks_decode_step_cached(ctypes.byref(cfg), _ptr(q), _ptr(summary_pool), _ptr(k_pool),
                                          _ptr(v_pool), int(num_blocks), _ptr(block_table), _ptr(seq_lens),
                                          int(batch), int(max_pages), _ptr(selected), _ptr(out), _ptr(lse),
                                          _ptr(cache), int(capacity), _ptr(ws), int(ws_bytes), _stream(stream)))


# --------------------------------------------------------------------------
# Convenience layer over torch tensors (allocation of outputs / workspace)
# --------------------------------------------------------------------------
def summary_pool_for(cfg: Config, num_blocks: int, device) -> torch.Tensor:
    """Empty summary pool [blocks][H_kv][record elements] in the summary dtype
    (uint8 bytes for LOCKS_I4 records)."""
    rb = locks_summary_record_bytes(cfg)
    if rb == 0:
        raise LocksError("locks_summary_record_bytes", LOCKS_E_UNSUPPORTED, "bad config")
    if cfg.summary_dtype == LOCKS_I4:
        return torch.empty((num_blocks, cfg.num_kv_heads, rb), dtype=torch.uint8, device=device)
    dt = torch.bfloat16 if cfg.summary_dtype == LOCKS_BF16 else torch.float32
    el = rb // (2 if dt == torch.bfloat16 else 4)
    return torch.empty((num_blocks, cfg.num_kv_heads, el), dtype=dt, device=device)


class HotCache:
    """A hot-page cache buffer on `device` for a pool of num_blocks blocks with
    `capacity` tile slots, emptied on creation; views of its state."""

    def __init__(self, cfg: Config, num_blocks: int, capacity: int, device, stream=None):
        self.cfg, self.num_blocks, self.capacity = cfg, int(num_blocks), int(capacity)
        self.offsets, self.bytes = locks_hot_cache_layout(cfg, num_blocks, capacity)
        self.buf = torch.empty(self.bytes, dtype=torch.uint8, device=device)
        locks_hot_cache_init(cfg, self.buf, num_blocks, capacity, stream)

    def reset(self, stream=None):
        locks_hot_cache_init(self.cfg, self.buf, self.num_blocks, self.capacity, stream)

    def field(self, name: str, dtype, count: int) -> torch.Tensor:
        o = self.offsets[name]
        return self.buf[o:o + count * torch.tensor([], dtype=dtype).element_size()].view(dtype)

    def stats(self) -> dict:
        """Counters (host ints): hits, misses, refreshes, shared, failed, steps."""
        v = self.field("stats", torch.int64, len(HOT_CACHE_STATS)).cpu().tolist()
        return dict(zip(HOT_CACHE_STATS, v))

    def state(self) -> dict:
        """Host copies of the clock state and maps (int32 tensors; hand and step as ints)."""
        tiles = self.num_blocks * self.cfg.num_kv_heads
        hand, step = self.field("clock", torch.int32, 2).cpu().tolist()
        return dict(hand=hand, step=step, slot_of=self.field("slot_of", torch.int32, tiles).cpu(),
                    tile_of=self.field("tile_of", torch.int32, self.capacity).cpu(),
                    stamp=self.field("stamp", torch.int32, self.capacity).cpu(),
                    flags=self.field("flags", torch.int32, self.capacity).cpu())


def split_records(cfg: Config, pool: torch.Tensor):
    """Views (mu [..][d], vt [..][r][d], coef [..][P][r]) of a bf16 / fp32 summary pool."""
    if cfg.summary_dtype == LOCKS_I4:
        raise ValueError("LOCKS_I4 records hold packed codes, not element views")
    d, r, P = cfg.head_dim, cfg.rank, cfg.page_size
    mu = pool[..., :d]
    vt = pool[..., d:d + r * d].unflatten(-1, (r, d))
    coef = pool[..., d + r * d:d + r * d + P * r].unflatten(-1, (P, r))
    return mu, vt, coef

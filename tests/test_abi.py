"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/locks.h declares, and every argument error is reported from the host
before anything is enqueued (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from sparse_kv_page_amd import locks as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "locks.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(locks_[a-z_]+)\s*\(", src)))


def test_header_matches_binding_list():
    assert _declared() == sorted(L.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def _cfg(**kw):
    base = dict(head_dim=128, page_size=64, rank=8, num_q_heads=32, num_kv_heads=8,
                budget_pages=32, kv_dtype="bf16")
    base.update(kw)
    return L.make_config(**base)


def test_version_and_status_strings():
    assert L.locks_version() == 1
    assert L.status_string(0) == "ok"
    for st in (-1, -2, -3, -4):
        assert L.status_string(st) not in ("ok", "unknown status")
    assert L.status_string(-99) == "unknown status"


@pytest.mark.parametrize("d,P,r,dt,expect", [
    (128, 64, 8, "bf16", 2 * (128 + 8 * 128 + 64 * 8)),   # 3328 B
    (128, 64, 4, "bf16", 2 * (128 + 4 * 128 + 64 * 4)),   # 1792 B
    (128, 64, 2, "bf16", 2 * (128 + 2 * 128 + 64 * 2)),   # 1024 B
    (64, 16, 4, "f32", 4 * (64 + 4 * 64 + 16 * 4)),
    (128, 16, 15, "bf16", 2 * (128 + 15 * 128 + 16 * 15)),
])
def test_record_bytes(d, P, r, dt, expect):
    cfg = _cfg(head_dim=d, page_size=P, rank=r, kv_dtype=dt)
    assert L.locks_summary_record_bytes(cfg) == expect
    assert expect % 16 == 0  # every record stays 16-byte aligned


@pytest.mark.parametrize("r,pages_bytes", [(8, 818), (4, 490), (2, 326)])
def test_i4_record_bytes_follow_the_byte_model(r, pages_bytes):
    """[Locks] App. C.7: 818 / 490 / 326 B per page at B = 16, d = 128 with scales;
    records are that payload padded to 16 bytes."""
    cfg = _cfg(head_dim=128, page_size=16, rank=r, summary_dtype="i4")
    assert L.locks_summary_record_bytes(cfg) == (pages_bytes + 15) // 16 * 16


@pytest.mark.parametrize("d,P,r", [(128, 64, 8), (128, 64, 1), (64, 32, 2), (64, 16, 4)])
def test_i4_record_bytes_layout(d, P, r):
    cfg = _cfg(head_dim=d, page_size=P, rank=r, summary_dtype="i4")
    payload = d * r // 2 + P * r + d + 2 * (r + P + 1)
    assert L.locks_summary_record_bytes(cfg) == (payload + 15) // 16 * 16


def test_i4_packer_places_fields_as_the_header_states():
    """The test-side packer against hand-placed words: d = 64, so a row is 8
    words and element a sits in word ((a % 32) // 8) * 2 + a // 32 at nibble
    a % 8 // 2 (even) or 4 + (a % 8 - 1) // 2 (odd)."""
    import numpy as np
    from tests import gpu_glue as gg
    d, r, P = 64, 1, 16
    vt = np.zeros((1, r, d), np.int64)
    # field = code + 8; choose codes so fields are 1 .. 7 at a few elements, 8 (code 0) elsewhere
    for a, f in [(0, 1), (1, 2), (7, 3), (8, 4), (32, 5), (63, 6), (33, 7)]:
        vt[0, 0, a] = f - 8
    qs = dict(mu_code=np.zeros((1, d), np.int64), vt_code=vt, coef_code=np.zeros((1, P, r), np.int64),
              mu_scale=np.ones(1), vt_scale=np.ones((1, r)), coef_scale=np.ones((1, P)))
    rec = gg.pack_i4(qs, d, r, P)[0]
    words = rec[:d // 2].view("<u4")
    base = 0x88888888
    expect = [base] * 8
    def put(w, m, f):
        expect[w] = (expect[w] & ~(0xF << (4 * m))) | (f << (4 * m))
    put(0, 0, 1)   # a = 0: word 0, nibble 0
    put(0, 4, 2)   # a = 1: word 0, nibble 4
    put(0, 7, 3)   # a = 7: word 0, nibble 7
    put(2, 0, 4)   # a = 8: word 2, nibble 0
    put(1, 0, 5)   # a = 32: word 1, nibble 0
    put(1, 4, 7)   # a = 33: word 1, nibble 4
    put(7, 7, 6)   # a = 63: word 7, nibble 7
    assert [int(x) for x in words] == expect
    # centroid code 0 is byte 128: high nibble 8, low nibble 0
    assert all(int(x) == 0x88888888 for x in rec[d // 2:d].view("<u4"))
    assert all(int(x) == 0 for x in rec[d:3 * d // 2].view("<u4"))
    # coefficient code 0 is byte 128; scales 1.0 are bf16 0x3F80
    assert all(int(x) == 128 for x in rec[3 * d // 2:3 * d // 2 + P * r])
    assert all(int(x) == 0x3F80 for x in rec[3 * d // 2 + P * r:3 * d // 2 + P * r + 2 * (1 + r + P)].view("<u2"))


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), L.LOCKS_E_UNSUPPORTED),
    (dict(page_size=48), L.LOCKS_E_UNSUPPORTED),
    (dict(rank=16), L.LOCKS_E_UNSUPPORTED),
    (dict(page_size=16, rank=16), L.LOCKS_E_UNSUPPORTED),     # r > P - 1
    (dict(rank=0), L.LOCKS_E_INVALID_ARG),
    (dict(budget_pages=1), L.LOCKS_E_INVALID_ARG),
    (dict(budget_pages=1025), L.LOCKS_E_UNSUPPORTED),
    (dict(num_q_heads=30), L.LOCKS_E_INVALID_ARG),            # H_q % H_kv != 0
    (dict(num_q_heads=24), L.LOCKS_E_UNSUPPORTED),            # G = 3
    (dict(num_q_heads=128), L.LOCKS_E_UNSUPPORTED),           # G = 16
    (dict(softmax_scale=0.0), L.LOCKS_E_INVALID_ARG),
    (dict(softmax_scale=float("nan")), L.LOCKS_E_INVALID_ARG),
    (dict(kv_dtype=7), L.LOCKS_E_INVALID_ARG),
    (dict(kv_dtype="bf16", summary_dtype="f32"), L.LOCKS_E_UNSUPPORTED),
    (dict(kv_dtype="f32", summary_dtype="i4"), L.LOCKS_E_UNSUPPORTED),     # i4 needs bf16 queries
    (dict(summary_dtype="i4", rank=3), L.LOCKS_E_UNSUPPORTED),             # i4 ranks: 1, 2, 4, 8
    (dict(summary_dtype="i4", rank=16), L.LOCKS_E_UNSUPPORTED),
    (dict(summary_dtype=3), L.LOCKS_E_INVALID_ARG),
])
def test_config_errors(kw, status):
    cfg = _cfg(**kw)
    assert L.locks_summary_record_bytes(cfg) == 0
    with pytest.raises(L.LocksError) as ei:
        L.locks_workspace_size(cfg, 8, 2048)
    assert ei.value.status == status
    # every entry point rejects the same config before touching the device
    fake = 1 << 20
    calls = [
        lambda: L.locks_build_summaries(cfg, fake, 10, fake, 4, fake, stream=0),
        lambda: L.locks_page_score(cfg, fake, fake, 10, fake, fake, 1, 4, fake, stream=0),
        lambda: L.locks_select_pages(cfg, fake, fake, 1, 4, fake, fake, stream=0),
        lambda: L.locks_score_select(cfg, fake, fake, 10, fake, fake, 1, 4, fake, fake, 1 << 30,
                                     stream=0),
        lambda: L.locks_sparse_decode(cfg, fake, fake, fake, 10, fake, fake, fake, 1, 4, fake,
                                      None, fake, 1 << 30, stream=0),
        lambda: L.locks_decode_step(cfg, fake, fake, fake, fake, 10, fake, fake, 1, 4, fake, fake,
                                    None, fake, 1 << 30, stream=0),
        lambda: L.locks_hot_cache_layout(cfg, 10, 1000),
        lambda: L.locks_hot_cache_init(cfg, fake, 10, 1000, stream=0),
        lambda: L.locks_decode_step_cached(cfg, fake, fake, fake, fake, 10, fake, fake, 1, 4, fake, fake,
                                           None, fake, 1000, fake, 1 << 30, stream=0),
    ]
    for c in calls:
        with pytest.raises(L.LocksError) as ei:
            c()
        assert ei.value.status == status


def test_null_pointers_and_sizes():
    cfg = _cfg()
    fake = 1 << 20
    E = L.LOCKS_E_INVALID_ARG
    cases = [
        lambda: L.locks_build_summaries(cfg, None, 10, fake, 4, fake, stream=0),
        lambda: L.locks_build_summaries(cfg, fake, 10, None, 4, fake, stream=0),
        lambda: L.locks_build_summaries(cfg, fake, 10, fake, 4, None, stream=0),
        lambda: L.locks_build_summaries(cfg, fake, 10, fake, -1, fake, stream=0),
        lambda: L.locks_build_summaries(cfg, fake, -5, fake, 4, fake, stream=0),
        lambda: L.locks_page_score(cfg, None, fake, 10, fake, fake, 1, 4, fake, stream=0),
        lambda: L.locks_page_score(cfg, fake, fake, 10, fake, fake, 1, 4, None, stream=0),
        lambda: L.locks_page_score(cfg, fake, fake, 10, fake, fake, -1, 4, fake, stream=0),
        lambda: L.locks_page_score(cfg, fake, fake, 10, fake, fake, 2, 0, fake, stream=0),
        lambda: L.locks_select_pages(cfg, fake, fake, 1, 4, None, fake, stream=0),
        lambda: L.locks_select_pages(cfg, fake, fake, 1, 4, fake, None, stream=0),
        lambda: L.locks_sparse_decode(cfg, fake, fake, None, 10, fake, fake, fake, 1, 4, fake,
                                      None, fake, 1 << 30, stream=0),
        lambda: L.locks_sparse_decode(cfg, fake, fake, fake, 10, fake, fake, fake, 1, 4, None,
                                      None, fake, 1 << 30, stream=0),
        lambda: L.locks_decode_step(cfg, fake, None, fake, fake, 10, fake, fake, 1, 4, fake, fake,
                                    None, fake, 1 << 30, stream=0),
        lambda: L.locks_decode_step(cfg, fake, fake, fake, fake, 10, fake, fake, 1, 4, None, fake,
                                    None, fake, 1 << 30, stream=0),
        lambda: L.locks_decode_step(cfg, fake, fake, fake, fake, -1, fake, fake, 1, 4, fake, fake,
                                    None, fake, 1 << 30, stream=0),
        # an empty pool cannot be read: every call that reads one wants num_blocks >= 1
        lambda: L.locks_page_score(cfg, fake, fake, 0, fake, fake, 1, 4, fake, stream=0),
        lambda: L.locks_score_select(cfg, fake, fake, 0, fake, fake, 1, 4, fake, fake, 1 << 30, stream=0),
        lambda: L.locks_sparse_decode(cfg, fake, fake, fake, 0, fake, fake, fake, 1, 4, fake,
                                      None, fake, 1 << 30, stream=0),
        lambda: L.locks_decode_step(cfg, fake, fake, fake, fake, 0, fake, fake, 1, 4, fake, fake,
                                    None, fake, 1 << 30, stream=0),
    ]
    for c in cases:
        with pytest.raises(L.LocksError) as ei:
            c()
        assert ei.value.status == E


def test_workspace_checks():
    cfg = _cfg()
    need = L.locks_workspace_size(cfg, 8, 2048)
    # scores (8*32*2048) + sigma (8*8*2048) floats for 128K context at batch 8
    assert need >= 4 * (8 * 32 * 2048 + 8 * 8 * 2048)
    fake = 1 << 20
    for ws, nbytes in ((None, need), (fake, 16)):
        with pytest.raises(L.LocksError) as ei:
            L.locks_score_select(cfg, fake, fake, 10, fake, fake, 8, 2048, fake, ws, nbytes, stream=0)
        assert ei.value.status == L.LOCKS_E_WORKSPACE
        with pytest.raises(L.LocksError) as ei:
            L.locks_sparse_decode(cfg, fake, fake, fake, 10, fake, fake, fake, 8, 2048, fake, None,
                                  ws, nbytes, stream=0)
        assert ei.value.status == L.LOCKS_E_WORKSPACE
        with pytest.raises(L.LocksError) as ei:
            L.locks_decode_step(cfg, fake, fake, fake, fake, 10, fake, fake, 8, 2048, fake, fake, None,
                                ws, nbytes, stream=0)
        assert ei.value.status == L.LOCKS_E_WORKSPACE



def test_workspace_monotone_and_empty_calls():
    cfg = _cfg()
    sizes = [L.locks_workspace_size(cfg, b, m) for b, m in ((1, 1), (1, 512), (8, 512), (8, 2048))]
    assert sizes == sorted(sizes)
    assert L.locks_workspace_size(cfg, 0, 0) == 0
    # empty work is OK and enqueues nothing (null pointers accepted)
    L.locks_build_summaries(cfg, None, 0, None, 0, None, stream=0)
    L.locks_page_score(cfg, None, None, 0, None, None, 0, 0, None, stream=0)
    L.locks_select_pages(cfg, None, None, 0, 0, None, None, stream=0)
    L.locks_score_select(cfg, None, None, 0, None, None, 0, 0, None, None, 0, stream=0)
    L.locks_sparse_decode(cfg, None, None, None, 0, None, None, None, 0, 0, None, None, None, 0,
                          stream=0)
    L.locks_decode_step(cfg, None, None, None, None, 0, None, None, 0, 0, None, None, None, None, 0,
                        stream=0)
    L.locks_decode_step_cached(cfg, None, None, None, None, 0, None, None, 0, 0, None, None, None, None, 0,
                               None, 0, stream=0)


def test_hot_cache_layout():
    """Fields in the header's order, 256-byte aligned, each as large as the
    header states: 8 + 2 int64, 2 int32, one int32 per (block, KV head) tile,
    three int32 per slot, and a P x d K and V tile per slot."""
    cfg = _cfg()
    nb, cap = 1000, 300
    offs, nbytes = L.locks_hot_cache_layout(cfg, nb, cap)
    o = [offs[f] for f in L.HOT_CACHE_FIELDS]
    assert o[0] == 0 and all(x % 256 == 0 for x in o) and o == sorted(o)
    tile = 64 * 128 * 2
    sizes = [64, 16, 8, nb * 8 * 4, cap * 4, cap * 4, cap * 4, cap * tile, cap * tile]
    for i, sz in enumerate(sizes):
        end = o[i + 1] if i + 1 < len(o) else nbytes
        assert sz <= end - o[i] < sz + 256, L.HOT_CACHE_FIELDS[i]
    f32 = _cfg(kv_dtype="f32")
    _, nb32 = L.locks_hot_cache_layout(f32, nb, cap)
    assert nb32 - nbytes == 2 * cap * tile


def test_hot_cache_argument_errors():
    """Reported on the host before anything is enqueued."""
    cfg = _cfg()
    fake = 1 << 20
    need = L.locks_workspace_size(cfg, 2, 64)
    n = 2 * 8 * 32  # batch * H_kv * k tiles in one step
    cases = [
        (lambda: L.locks_hot_cache_layout(cfg, 0, 10), L.LOCKS_E_INVALID_ARG),
        (lambda: L.locks_hot_cache_layout(cfg, 10, 0), L.LOCKS_E_INVALID_ARG),
        (lambda: L.locks_hot_cache_layout(cfg, 1 << 28, 10), L.LOCKS_E_UNSUPPORTED),
        (lambda: L.locks_hot_cache_init(cfg, None, 10, 10, stream=0), L.LOCKS_E_INVALID_ARG),
        (lambda: L.locks_hot_cache_init(cfg, fake, 10, -1, stream=0), L.LOCKS_E_INVALID_ARG),
        # capacity below one step's tiles
        (lambda: L.locks_decode_step_cached(cfg, fake, fake, fake, fake, 10, fake, fake, 2, 64, fake, fake,
                                            None, fake, n - 1, fake, need, stream=0), L.LOCKS_E_INVALID_ARG),
        (lambda: L.locks_decode_step_cached(cfg, fake, fake, fake, fake, 10, fake, fake, 2, 64, fake, fake,
                                            None, None, n, fake, need, stream=0), L.LOCKS_E_INVALID_ARG),
        (lambda: L.locks_decode_step_cached(cfg, fake, fake, None, fake, 10, fake, fake, 2, 64, fake, fake,
                                            None, fake, n, fake, need, stream=0), L.LOCKS_E_INVALID_ARG),
        (lambda: L.locks_decode_step_cached(cfg, fake, fake, fake, fake, 10, fake, fake, 2, 64, fake, fake,
                                            None, fake, n, fake, need - 1, stream=0), L.LOCKS_E_WORKSPACE),
        (lambda: L.locks_decode_step_cached(cfg, fake, fake, fake, fake, 10, fake, fake, 2, 64, fake, fake,
                                            None, fake, n, None, need, stream=0), L.LOCKS_E_WORKSPACE),
    ]
    for c, status in cases:
        with pytest.raises(L.LocksError) as ei:
            c()
        assert ei.value.status == status


def test_binding_refuses_host_tensors():
    """A tensor in host memory is refused before the call: its address would
    reach a kernel as a device pointer."""
    import torch
    cfg = _cfg()
    fake = 1 << 20
    with pytest.raises(ValueError, match="GPU tensor"):
        L.locks_select_pages(cfg, torch.zeros(4), fake, 1, 4, fake, fake, stream=0)

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
    ]
    for c in cases:
        with pytest.raises(L.LocksError) as ei:
            c()
        assert ei.value.status == E


def test_workspace_checks():
    cfg = _cfg()
    need = L.locks_workspace_size(cfg, 8, 2048)
    # scores (8*32*2048) + sigma (8*8*2048) floats for the headline shape
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

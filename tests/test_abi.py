"""C-ABI checks that need no GPU: the library loads, exports every entry point that
include/sfx.h declares, and rejects bad configurations and arguments before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_entry_points():
    text = open(os.path.join(ROOT, "include", "sfx.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sfx_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def sfx():
    import suffix_match_drafter_amd as S

    if not os.path.exists(S.LIB_PATH):
        from suffix_match_drafter_amd import build

        build.build()
    return S


def test_exports_match_header(sfx):
    L = sfx.load()
    names = declared_entry_points()
    assert len(names) >= 14
    assert set(names) == set(sfx.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def _cfg(sfx, **kw):
    base = dict(k=8, max_tree_depth=24, num_backoff=1, max_occurrences=128, mode=0,
                max_batch=4, max_seq=64, max_sampled=1)
    base.update(kw)
    return sfx.Config(**base)


@pytest.mark.parametrize("bad", [
    dict(k=0), dict(k=33), dict(max_tree_depth=0), dict(max_tree_depth=65),
    dict(num_backoff=0), dict(num_backoff=9), dict(num_backoff=2, mode=0),
    dict(max_occurrences=0), dict(max_occurrences=129), dict(mode=2), dict(min_self_match=0),
    dict(max_seq=70000), dict(max_seq=32769), dict(max_sampled=17), dict(max_batch=-1),
    dict(mode=1, num_backoff=2, spec_factor_ppm=-1), dict(mode=1, min_token_prob_ppm=1_000_001),
    dict(mode=1, min_token_prob_ppm=-5), dict(corpus_capacity=-1),
    dict(corpus_capacity=(1 << 30) + 1), dict(corpus_capacity=100, max_tree_depth=1),
    dict(corpus_capacity=100, min_corpus_match=1), dict(corpus_capacity=100, min_corpus_match=25),
    dict(flags=8), dict(flags=16), dict(reserved=1),
])
def test_create_rejects_bad_config(sfx, bad):
    L = sfx.load()
    h = ctypes.c_void_p()
    rc = L.sfx_create(ctypes.byref(_cfg(sfx, **bad)._c()), ctypes.byref(h))
    assert rc == sfx.EINVAL
    assert h.value is None
    assert len(L.sfx_last_error()) > 0


def test_null_arguments_rejected(sfx):
    L = sfx.load()
    assert L.sfx_create(None, ctypes.byref(ctypes.c_void_p())) == sfx.EINVAL
    assert L.sfx_propose(None, 1, 4, 1, None, None, None, None, None, None) == sfx.EINVAL
    assert L.sfx_update_state(1, 4, 1, None, None, None, None, None) == sfx.EINVAL
    assert L.sfx_update_state(-1, 4, 1, None, None, None, None, None) == sfx.EINVAL
    assert L.sfx_build_suffix_array(None, 10, None, None, 0, None) == sfx.EINVAL
    assert L.sfx_build_suffix_array(None, -1, None, None, 0, None) == sfx.EINVAL
    assert L.sfx_build_suffix_array(None, 0, None, None, 0, None) == sfx.OK
    assert L.sfx_save(None, b"/nonexistent", None) == sfx.EINVAL
    assert L.sfx_ingest_inflight(None, 1, None, None, None, None, 1, 1, 1, None) == sfx.EINVAL
    assert L.sfx_accept_estimate(None, 1, None, None) == sfx.EINVAL
    assert L.sfx_propose_masked(None, 1, 4, None, None, None, None, None, None) == sfx.EINVAL
    assert L.sfx_propose_counts(None, 1, 1, 4, 1, None, None, None, None, None, None,
                                None) == sfx.EINVAL
    assert L.sfx_accept_feedback(None, 1, None, None) == sfx.EINVAL
    assert L.sfx_accept_reset(None, None) == sfx.EINVAL
    assert L.sfx_accept_counts(None, None, None) == sfx.EINVAL
    assert L.sfx_load(None, b"/nonexistent", None) == sfx.EINVAL
    assert L.sfx_debug_errors(None, None, None) == sfx.EINVAL
    assert L.sfx_debug_fail_next_rebuild(None) == sfx.EINVAL
    # an empty update is a no-op that touches nothing
    assert L.sfx_update_state(0, 4, 1, None, None, None, None, None) == sfx.OK


def test_workspace_size_monotone(sfx):
    L = sfx.load()
    sizes = [L.sfx_suffix_array_workspace_bytes(n) for n in (0, 1, 1000, 1 << 20, 1 << 22)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    assert sizes[-1] >= 16 * (1 << 22)

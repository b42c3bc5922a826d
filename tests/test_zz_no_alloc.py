"""The allocation-free suffix-array entry point (sfx_build_suffix_array_noalloc) against the
workspace one (sfx_build_suffix_array), bit for bit, through the C-ABI: two calls in a row on
one stream, the second with a smaller text, plus the largest accepted size and the rejection of
a larger one."""
import ctypes

import numpy as np
import pytest

import workloads as W


def _texts():
    rng = np.random.default_rng(11)
    # template-like text: shared spans with noise, documents ended by -1 (many doubling rounds)
    spans = [rng.integers(0, 900, size=int(rng.integers(16, 128))).astype(np.int32)
             for _ in range(40)]
    docs = []
    for _ in range(2500):
        parts = [spans[int(i)] for i in rng.integers(0, len(spans), size=4)]
        d = np.concatenate(parts)
        noise = rng.random(d.shape[0]) < 0.2
        d[noise] = rng.integers(0, 900, size=int(noise.sum()))
        docs.append(d)
    big = W.join_docs(docs)
    small = rng.integers(-1, 7, size=70001).astype(np.int32)  # few symbols: long repeats
    return big, small


def test_noalloc_rejects_beyond_maximum():
    import suffix_match_drafter_amd as sfx

    L = sfx.load()
    rc = L.sfx_build_suffix_array_noalloc(None, sfx.NOALLOC_MAX_TOKENS + 1, None, None)
    assert rc == sfx.ECAPACITY
    assert b"allocation-free maximum" in L.sfx_last_error()
    assert L.sfx_build_suffix_array_noalloc(None, -1, None, None) == sfx.ECAPACITY
    assert L.sfx_build_suffix_array_noalloc(None, 0, None, None) == sfx.OK


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point():
    import torch

    import suffix_match_drafter_amd as sfx

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    big, small = _texts()
    assert small.shape[0] < big.shape[0] <= sfx.NOALLOC_MAX_TOKENS
    stream = torch.cuda.current_stream()
    outs = []
    for text in (big, small):
        t = torch.from_numpy(text).cuda()
        sa = torch.full_like(t, -7)
        sfx.build_suffix_array_noalloc(t, sa, stream)
        outs.append((t, sa))
    torch.cuda.synchronize()
    for t, sa in outs:
        ref = sfx.build_suffix_array(t, stream)
        torch.cuda.synchronize()
        assert torch.equal(sa, ref), f"n={t.shape[0]}"


@pytest.mark.gpu
def test_noalloc_largest_size():
    import torch

    import suffix_match_drafter_amd as sfx

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    rng = np.random.default_rng(5)
    text = rng.integers(-1, 40, size=sfx.NOALLOC_MAX_TOKENS).astype(np.int32)
    t = torch.from_numpy(text).cuda()
    sa = torch.empty_like(t)
    sfx.build_suffix_array_noalloc(t, sa)
    ref = sfx.build_suffix_array(t)
    torch.cuda.synchronize()
    assert torch.equal(sa, ref)
    # the same array again after a smaller call
    sfx.build_suffix_array_noalloc(t[:1000], sa[:1000])
    sfx.build_suffix_array_noalloc(t, sa)
    torch.cuda.synchronize()
    assert torch.equal(sa, ref)

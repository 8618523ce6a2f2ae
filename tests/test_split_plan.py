"""Host logic of the split prefill: attn_prefill_split_plan (pure host
arithmetic in libattn.so, no GPU).  Checks the plan's invariants on the
shapes the split exists for (one head, short chunks against a long cache)
and that ordinary shapes are left whole."""

import ctypes

import pytest

from io_aware_softmax_amd import binding

ROWS, KT = 256, 64  # query rows per tile, keys per key tile


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def _nkv(Lq, Lk, causal):
    """Key tiles of each 256-row query tile (bottom-right causal alignment)."""
    out = []
    for qt in range((Lq + ROWS - 1) // ROWS):
        last = min((qt + 1) * ROWS, Lq) - 1
        keys = min(Lk, last + (Lk - Lq) + 1) if causal else Lk
        out.append((keys + KT - 1) // KT)
    return out


def _check_plan(B, H, Lq, Lk, causal, cus, forced=0):
    ranges, items = binding.attn_prefill_split_plan(B, H, Lq, Lk, causal, cus, forced)
    nkv = _nkv(Lq, Lk, causal)
    assert len(ranges) == len(nkv)
    assert items == sum(ranges)
    for r, n in zip(ranges, nkv):
        assert r >= 1
        if r > 1:
            assert r <= n  # no empty range
            assert r <= 32
    return ranges, items, nkv


@pytest.mark.parametrize("Lq,Lk", [(16384, 16384), (4096, 4096), (32768, 32768), (8192, 65536)])
def test_one_head_causal_is_balanced(Lq, Lk):
    cus = 256
    ranges, items, nkv = _check_plan(1, 1, Lq, Lk, True, cus)
    assert items <= cus  # one range per workgroup
    assert max(ranges) > 1
    # Largest range within 1.35x of an even share of the job per CU (at
    # least 8 key tiles); the rounding of range counts to whole numbers
    # costs the rest (32k: 128 tiles for 256 items, 172 vs 129).  Unsplit,
    # the largest item would be the whole last tile.
    share = max(8, -(-sum(nkv) // cus))
    largest = max(-(-n // r) for n, r in zip(nkv, ranges))
    assert largest <= 1.35 * share
    assert largest <= max(nkv) / 2
    # Heavier tiles never get fewer ranges.
    assert all(a <= b for a, b in zip(ranges, ranges[1:]))


def test_chunk_against_long_cache():
    ranges, items, _ = _check_plan(1, 32, 512, 8192, True, 256)
    assert ranges == [4, 4] and items == 8


@pytest.mark.parametrize("B,H,L", [(1, 32, 8192), (1, 8, 16384), (1, 1, 65536), (16, 32, 1024)])
def test_wide_shapes_stay_whole(B, H, L):
    ranges, items, nkv = _check_plan(B, H, L, L, True, 256)
    assert ranges == [1] * len(nkv) and items == len(nkv)


def test_smaller_part_splits_less():
    r256, _, _ = _check_plan(1, 1, 16384, 16384, True, 256)
    r64, _, _ = _check_plan(1, 1, 16384, 16384, True, 64)
    assert sum(r64) <= 64 < sum(r256) + 1
    assert sum(r64) < sum(r256)


def test_forced_counts_are_capped():
    assert _check_plan(1, 2, 700, 700, True, 256, 3)[0] == [3, 3, 3]
    # first causal tile has 4 key tiles: at most 4 ranges
    assert _check_plan(1, 2, 700, 700, True, 256, 100)[0] == [4, 4, 4]
    assert _check_plan(1, 2, 64, 640, True, 256, 9)[0] == [9]
    # at most 16 when forced
    assert _check_plan(1, 1, 300, 4096, False, 256, 40)[0] == [16, 16]
    # 1 (or a tile without keys) never splits
    assert _check_plan(1, 1, 4096, 4096, True, 256, 1)[0] == [1] * 16
    assert _check_plan(1, 1, 1000, 500, True, 256, 4)[0] == [1] * 4


def test_rows_without_keys_are_not_split():
    # causal with Lq > Lk: the first query tiles see no key at all
    ranges, items, nkv = _check_plan(1, 1, 2000, 300, True, 256)
    assert nkv[0] <= 0 and ranges == [1] * len(nkv)


def test_invalid_arguments(lib):
    r = (ctypes.c_int * 4)()
    n = ctypes.c_int()
    assert lib.attn_prefill_split_plan(0, 1, 256, 256, 1, 256, 0, r, ctypes.byref(n)) < 0
    assert lib.attn_prefill_split_plan(1, 1, 256, 256, 1, 0, 0, r, ctypes.byref(n)) < 0
    assert lib.attn_prefill_split_plan(1, 1, 256, 256, 1, 256, -1, r, ctypes.byref(n)) < 0
    assert lib.attn_prefill_split_plan(1, 1, 256, 256, 1, 256, 0, None, ctypes.byref(n)) < 0
    assert lib.attn_prefill_split_plan(1, 1, 256, 256, 1, 256, 0, r, None) < 0

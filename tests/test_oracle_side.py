"""Pins of the oracle's side cache and cache-write step (CPU).

The side cache holds the pooled key of every micro-block of every request (reading R11 of
the oracle); a decode step appends its token and refreshes one side-cache entry (R12).
Pinned by: a brute-force element sum; equality of the scores read from the side cache with
the scores computed from the indexer keys; and re-appending each request's last token
through the oracle, which must reproduce, bit for bit, the caches the input generator made
at full length.
"""
import numpy as np
import pytest

import oracle
from sparse_attention_decode_qsa_amd.inputs import Workload, make_inputs
from tests.helpers import oracle_arrays

LENS = (0, 1, 2, 3, 4, 5, 63, 64, 65, 127, 130, 257)


def _inputs(lens=LENS, seed=21, paging="shuffled"):
    w = Workload("side", len(lens), ("list",) + tuple(lens), 16, 2, 2, paging=paging)
    return make_inputs(w, seed, "cpu")


def test_side_cache_brute_force(lens=LENS):
    x = _inputs(lens)
    a = oracle_arrays(x)
    side = oracle.side_cache(a["idx_cache"], a["page_table"], a["lengths"])
    idx, pt = a["idx_cache"], a["page_table"]
    assert side.shape == (idx.shape[0], 16, 4, 64)
    used = np.zeros(side.shape[:2], dtype=bool)
    for b, L in enumerate(a["lengths"]):
        for j in range((L + 3) // 4):
            page, slot = int(pt[b][j // 16]), j % 16
            used[page, slot] = True
            for h in range(4):
                for d in range(0, 64, 7):          # every 7th dim, summed element by element
                    want = 0
                    for t in range(4 * j, min(4 * j + 4, L)):
                        want += int(idx[int(pt[b][t // 64]), t % 64, h, d])
                    assert side[page, slot, h, d] == want, (b, j, h, d)
    assert np.all(side[~used] == 0)
    assert np.abs(side).max() <= 4 * 127


def test_side_scores_equal_index_scores():
    x = _inputs()
    a = oracle_arrays(x)
    side = oracle.side_cache(a["idx_cache"], a["page_table"], a["lengths"])
    for b, L in enumerate(a["lengths"]):
        want = oracle.index_scores(a["q_idx"][b], a["idx_cache"], a["page_table"][b], L)
        got = oracle.side_scores(a["q_idx"][b], side, a["page_table"][b], L)
        assert np.array_equal(got, want), b


def _strip_last_token(a, seed=5):
    """Caches with each request's last row overwritten by noise, and the side cache of the
    shorter requests, plus the rows that were removed."""
    rng = np.random.default_rng(seed)
    k, v, idx = (np.array(a[n], copy=True) for n in ("k_cache", "v_cache", "idx_cache"))
    pt, lens = a["page_table"], a["lengths"]
    B, Hkv, D = len(lens), k.shape[2], k.shape[3]
    k_new = np.zeros((B, Hkv, D), np.uint16)
    v_new = np.zeros((B, Hkv, D), np.uint16)
    i_new = np.zeros((B,) + idx.shape[2:], np.int8)
    for b, L in enumerate(lens):
        if L == 0:
            continue
        page, row = int(pt[b][(L - 1) // 64]), (L - 1) % 64
        k_new[b], v_new[b], i_new[b] = k[page, row], v[page, row], idx[page, row]
        k[page, row] = rng.integers(0, 1 << 16, (Hkv, D), dtype=np.uint16)
        v[page, row] = rng.integers(0, 1 << 16, (Hkv, D), dtype=np.uint16)
        idx[page, row] = rng.integers(-127, 128, idx.shape[2:], dtype=np.int8)
    side = oracle.side_cache(idx, pt, [max(L - 1, 0) for L in lens])
    return k, v, idx, side, k_new, v_new, i_new


def test_append_reproduces_full_caches(lens=LENS, paging="shuffled"):
    x = _inputs(lens, paging=paging)
    a = oracle_arrays(x)
    k, v, idx, side, k_new, v_new, i_new = _strip_last_token(a)
    k2, v2, i2, s2 = oracle.append_token(k, v, idx, side, a["page_table"], a["lengths"], k_new, v_new, i_new)
    assert np.array_equal(k2, a["k_cache"]) and np.array_equal(v2, a["v_cache"])
    assert np.array_equal(i2, a["idx_cache"])
    assert np.array_equal(s2, oracle.side_cache(a["idx_cache"], a["page_table"], a["lengths"]))


def test_append_write_flag_and_empty_requests():
    x = _inputs()
    a = oracle_arrays(x)
    k, v, idx, side, k_new, v_new, i_new = _strip_last_token(a)
    write = [b % 2 for b in range(len(a["lengths"]))]
    k2, v2, i2, s2 = oracle.append_token(k, v, idx, side, a["page_table"], a["lengths"], k_new, v_new, i_new,
                                         write)
    full = oracle.side_cache(a["idx_cache"], a["page_table"], a["lengths"])
    for b, L in enumerate(a["lengths"]):
        if L == 0:
            continue
        page, row = int(a["page_table"][b][(L - 1) // 64]), (L - 1) % 64
        j = (L - 1) // 4
        sp, ss = int(a["page_table"][b][j // 16]), j % 16
        if write[b]:
            assert np.array_equal(k2[page, row], a["k_cache"][page, row])
            assert np.array_equal(s2[sp, ss], full[sp, ss])
        else:   # nothing of this request changes
            assert np.array_equal(k2[page, row], k[page, row]) and np.array_equal(i2[page, row], idx[page, row])
            assert np.array_equal(s2[sp, ss], side[sp, ss])


@pytest.mark.parametrize("lens", [(1,), (4,), (5,), (64,), (65,), (2048, 7)])
def test_append_block_boundaries(lens):
    """A new block (L % 4 == 1), a completed block (L % 4 == 0), page edges."""
    test_append_reproduces_full_caches(lens, paging="identity")

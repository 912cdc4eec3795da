"""bench.py's bookkeeping that needs no GPU: the rotation rule and the algorithmic byte counts."""
import importlib.util
import os

import pytest

from sparse_attention_decode_qsa_amd.inputs import WORKLOADS, draw_lengths

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_rules_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", ["w2", "w3", "w4", "w4_fixed"])
@pytest.mark.parametrize("draft", [1, 2, 4])
def test_rotation_defeats_the_mall(name, draft):
    # one rotation streams >= 1 GiB of indexer keys and gathers >= 512 MiB of distinct kept
    # K/V rows, unless the set or byte cap binds first
    b = _bench()
    w = WORKLOADS[name]
    L = draw_lengths(w, 0)
    n = b.default_sets(L, w.hkv, draft)
    idx = 256 * sum(L)
    kept = draft * sum(min(2048, x) for x in L) * w.hkv * 512
    per_set = idx + sum(L) * w.hkv * 512
    capped = n == 64 or (n + 1) * per_set > (96 << 30)
    assert capped or (n * idx >= 1 << 30 and n * kept >= 512 << 20)
    assert n * per_set <= 96 << 30


def test_rotation_at_the_headline_batch():
    b = _bench()
    w = WORKLOADS["w4"]
    L = draw_lengths(w, 0)
    assert b.default_sets(L, w.hkv) == 32          # 16.8 MB of kept rows per call -> 32 sets


def test_algorithmic_bytes_by_hand():
    # one request of 10 tokens (3 blocks, all kept, 10 kept tokens), Hq/Hkv = 8/2
    b = _bench()
    L, hq, hkv = 10, 8, 2
    expect = 256 * L + 256 + 4 * 1 + 10 * hkv * 512 + 256 * hq + 512 * hq
    assert b.algorithmic_bytes([L], hq, hkv) == expect
    # a long request keeps 512 blocks = 2048 tokens
    L = 100_000
    expect = 256 * L + 256 + 4 * ((L + 63) // 64) + 2048 * hkv * 512 + 256 * hq + 512 * hq
    assert b.algorithmic_bytes([L], hq, hkv) == expect
    assert b.index_bytes([L]) == 256 * L + 256 + 4 * ((L + 63) // 64) + 4 * ((L + 3) // 4)

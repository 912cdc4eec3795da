"""Pins of the oracle's multi-token (draft) decode, reading R13 (CPU).

Draft token t of T is a single-token decode at length L - T + 1 + t. Pinned by: T = 1 is the
single-token decode; the last draft token is the single-token decode at full length; and
causality - rewriting every cache row a draft token must not see leaves its result
unchanged, while the same rewrite changes the last token's result.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_decode_qsa_amd.inputs import Workload, bf16_bits, draft_queries, make_inputs
from tests.helpers import oracle_arrays

LENS = (3, 4, 5, 64, 65, 66, 67, 130, 2049, 5000)


def _case(T, lens=LENS, seed=41):
    x = make_inputs(Workload("draft", len(lens), ("list",) + tuple(lens), 16, 2, 2), seed, "cpu")
    q, qi = draft_queries(x, T, seed)
    return x, bf16_bits(q), qi.numpy(), oracle_arrays(x)


def _multi(a, q, qi, T, P=2, idx=None, k=None, v=None):
    return oracle.decode_multi(q, qi, a["idx_cache"] if idx is None else idx, a["k_cache"] if k is None else k,
                               a["v_cache"] if v is None else v, a["page_table"], a["lengths"], T, P, 128 ** -0.5)


def test_one_draft_token_is_single_decode():
    x, q, qi, a = _case(1)
    multi = _multi(a, q, qi, 1)
    single = oracle.decode(q[:, 0], qi[:, 0], a["idx_cache"], a["k_cache"], a["v_cache"], a["page_table"],
                           a["lengths"], 2, 128 ** -0.5)
    for m, s in zip(multi, single):
        assert np.array_equal(m["kept"], s["kept"]) and np.array_equal(m["out"], s["out"])


@pytest.mark.parametrize("T", [2, 3, 4])
def test_last_draft_token_sees_the_whole_context(T):
    x, q, qi, a = _case(T)
    multi = _multi(a, q, qi, T)
    single = oracle.decode(q[:, T - 1], qi[:, T - 1], a["idx_cache"], a["k_cache"], a["v_cache"], a["page_table"],
                           a["lengths"], 2, 128 ** -0.5)
    for b in range(len(LENS)):
        r = multi[b * T + T - 1]
        assert np.array_equal(r["scores"], single[b]["scores"]) and np.array_equal(r["out"], single[b]["out"])


@pytest.mark.parametrize("T", [2, 4])
def test_draft_tokens_are_causal(T):
    x, q, qi, a = _case(T)
    base = _multi(a, q, qi, T)
    rng = np.random.default_rng(3)
    for t in range(T - 1):
        idx, k, v = (np.array(a[n], copy=True) for n in ("idx_cache", "k_cache", "v_cache"))
        for b, L in enumerate(a["lengths"]):       # rewrite the rows draft token t must not see
            for u in range(oracle.draft_length(L, T, t), L):
                page, row = int(a["page_table"][b][u // 64]), u % 64
                idx[page, row] = rng.integers(-127, 128, idx.shape[2:], dtype=np.int8)
                k[page, row] = bf16_bits(torch.randn(k.shape[2:]).to(torch.bfloat16))
                v[page, row] = bf16_bits(torch.randn(v.shape[2:]).to(torch.bfloat16))
        moved = _multi(a, q, qi, T, idx=idx, k=k, v=v)
        for b in range(len(LENS)):
            r0, r1 = base[b * T + t], moved[b * T + t]
            assert np.array_equal(r0["scores"], r1["scores"]) and np.array_equal(r0["out"], r1["out"]), (b, t)
            last0, last1 = base[b * T + T - 1], moved[b * T + T - 1]
            assert not np.array_equal(last0["scores"], last1["scores"]), (b, t)

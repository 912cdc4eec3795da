"""Property-style parity of the whole chain on the GPU, over many small random shapes.

Hypothesis draws the shape of each case (derandomised, so every run checks the same cases).
Single-token decode:
1 to 4 requests with lengths in [0, 5000] (not rounded to blocks or pages), GQA shapes 8/1,
16/2 and 32/4, P in [1, 8], and the three value alphabets (full int8, {-2..2} with many
score ties, and an all-zero indexer query where every block ties). Every request's block
scores, kept blocks and outputs are compared with the CPU oracle through the C ABI, the
four separate calls and qsa_decode must agree bit for bit, and the unused rows of each
request's last page hold poison (NaN K/V, indexer keys 127) that must not reach a result.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from sparse_attention_decode_qsa_amd import qsa
from sparse_attention_decode_qsa_amd.inputs import Workload, bf16_bits, draft_queries, make_inputs
from tests.helpers import oracle_arrays, oracle_decode
from tests.test_gpu_multi import _run as run_multi
from tests.test_gpu_parity import check_request, run_chain, say

pytestmark = pytest.mark.gpu

GQA = [(8, 1), (16, 2), (32, 4)]
ALPHABETS = ["u127", "u2", "zero_q"]


@settings(max_examples=60, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(lens=st.lists(st.integers(0, 5000), min_size=1, max_size=4),
       gqa=st.sampled_from(GQA), P=st.integers(1, 8), alphabet=st.sampled_from(ALPHABETS),
       seed=st.integers(0, 2**16))
def test_chain_matches_oracle_on_random_shapes(lens, gqa, P, alphabet, seed):
    hq, hkv = gqa
    w = Workload("prop", len(lens), ("list",) + tuple(lens), hq, hkv, P, alphabet=alphabet)
    x = make_inputs(w, seed, "cuda")
    say(f"[prop] lens={lens} Hq/Hkv={hq}/{hkv} P={P} alphabet={alphabet} seed={seed}")
    g = run_chain(x, P)
    refs = oracle_decode(oracle, x, P=P)
    for b, r in enumerate(refs):
        check_request(g, b, r, x.lengths[b], what="prop")
    plan = qsa.decode(x.q, x.q_idx, x.idx_cache, x.k_cache, x.v_cache, x.page_table, x.context_lens, P=P)
    torch.cuda.synchronize()
    assert np.array_equal(plan.sel.cpu().numpy(), g["sel"])
    assert np.array_equal(plan.out.cpu().numpy().view(np.int32), g["out"].view(np.int32))
    assert np.array_equal(plan.out_lse.cpu().numpy().view(np.int32), g["lse"].view(np.int32))


@settings(max_examples=30, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(lens=st.lists(st.integers(0, 3000), min_size=1, max_size=3),
       T=st.one_of(st.integers(1, 8), st.just(20)), gqa=st.sampled_from(GQA), P=st.integers(1, 4),
       alphabet=st.sampled_from(ALPHABETS), seed=st.integers(0, 2**16))
def test_multi_token_matches_oracle_on_random_shapes(lens, T, gqa, P, alphabet, seed):
    """Several new tokens per request (T <= 4 on the per-query scan, 5..8 and 20 on the
    matrix-core scan): every (request, token) against the oracle's causal reading."""
    hq, hkv = gqa
    w = Workload("propm", len(lens), ("list",) + tuple(lens), hq, hkv, P, alphabet=alphabet)
    x = make_inputs(w, seed, "cuda")
    q, qi = draft_queries(x, T, seed)
    say(f"[prop multi] lens={lens} T={T} Hq/Hkv={hq}/{hkv} P={P} alphabet={alphabet} seed={seed}")
    _, g = run_multi(x, q, qi, P)
    a = oracle_arrays(x)
    refs = oracle.decode_multi(bf16_bits(q), qi.cpu().numpy(), a["idx_cache"], a["k_cache"], a["v_cache"],
                               a["page_table"], a["lengths"], T, P, x.scale)
    for b, L in enumerate(lens):
        for t in range(T):
            r = b * T + t
            check_request(g, r, refs[r], oracle.draft_length(L, T, t), what=f"prop T{T} b{b} t{t}")

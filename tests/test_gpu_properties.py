"""Property-style parity of the whole chain on the GPU, over many small random shapes.

Hypothesis draws the shape of each case (derandomised, so every run checks the same cases).
Single-token decode:
1 to 4 requests with lengths in [0, 5000] (not rounded to blocks or pages), GQA shapes 8/1,
16/2 and 32/4, P in [1, 8], and the three value alphabets (full int8, {-2..2} with many
score ties, and an all-zero indexer query where every block ties). Every request's block
scores, kept blocks and outputs are compared with the CPU oracle through the C ABI, the
four separate calls and qsa_decode must agree bit for bit, and the unused rows of each
request's last page hold poison (NaN K/V, indexer keys 127) that must not reach a result.
Multi-token decode: up to 3 requests, T from 1 to 8 or 16 to 40 new tokens, independent or
correlated indexer queries. Wider shapes: up to 6
requests of up to 80,000 tokens, group sizes 16, 3 and 1, up to 64 slices, k below 512 and
page tables with spare capacity. Side cache: the fused decode step (cache writes in the
scan) and draft tokens scored from the side cache, up to 4 requests of up to 20,000 tokens.
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
from tests.test_gpu_side_cache import _stripped as stripped_caches
from tests.test_gpu_side_cache import _valid_entries as side_entries
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
       T=st.one_of(st.integers(1, 8), st.integers(16, 40)), gqa=st.sampled_from(GQA), P=st.integers(1, 4),
       alphabet=st.sampled_from(ALPHABETS), spread=st.sampled_from([None, None, 0, 3, 20]),
       seed=st.integers(0, 2**16))
def test_multi_token_matches_oracle_on_random_shapes(lens, T, gqa, P, alphabet, spread, seed):
    """Several new tokens per request (T <= 4 on the per-query scan, 5..8 and 16..40 on the
    matrix-core scan, 16..40 with neighbouring tokens paired in the attention), with
    independent or correlated indexer queries: every (request, token) against the oracle's
    causal reading."""
    hq, hkv = gqa
    w = Workload("propm", len(lens), ("list",) + tuple(lens), hq, hkv, P, alphabet=alphabet)
    x = make_inputs(w, seed, "cuda")
    q, qi = draft_queries(x, T, seed, spread=spread)
    say(f"[prop multi] lens={lens} T={T} Hq/Hkv={hq}/{hkv} P={P} alphabet={alphabet} spread={spread} seed={seed}")
    _, g = run_multi(x, q, qi, P)
    a = oracle_arrays(x)
    refs = oracle.decode_multi(bf16_bits(q), qi.cpu().numpy(), a["idx_cache"], a["k_cache"], a["v_cache"],
                               a["page_table"], a["lengths"], T, P, x.scale)
    for b, L in enumerate(lens):
        for t in range(T):
            r = b * T + t
            check_request(g, r, refs[r], oracle.draft_length(L, T, t), what=f"prop T{T} b{b} t{t}")


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(lens=st.lists(st.one_of(st.integers(0, 3000), st.integers(2000, 80000)), min_size=1, max_size=6),
       gqa=st.sampled_from(GQA + [(64, 4), (12, 4), (16, 16)]), P=st.sampled_from([1, 2, 3, 5, 8, 16, 64]),
       k=st.sampled_from([1, 100, 511, 512]), alphabet=st.sampled_from(ALPHABETS),
       extra_pages=st.sampled_from([0, 1, 80]), seed=st.integers(0, 2**16))
def test_chain_matches_oracle_on_wider_shapes(lens, gqa, P, k, alphabet, extra_pages, seed):
    """Longer contexts (up to 80,000 tokens, several slices and shares per request), group
    sizes 16, 3 and 1, up to 64 slices, k below 512, and page tables with spare capacity: the
    four separate calls against the oracle, every request."""
    hq, hkv = gqa
    cap = max(lens) + 64 * extra_pages
    w = Workload("propw", len(lens), ("list",) + tuple(lens), hq, hkv, P, alphabet=alphabet, max_context=cap, k=k)
    x = make_inputs(w, seed, "cuda")
    say(f"[prop wide] lens={lens} Hq/Hkv={hq}/{hkv} P={P} k={k} alphabet={alphabet} cap={cap} seed={seed}")
    g = run_chain(x, P, k)
    refs = oracle_decode(oracle, x, P=P, k=k)
    for b, r in enumerate(refs):
        check_request(g, b, r, x.lengths[b], k, what="prop wide")


@settings(max_examples=30, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(lens=st.lists(st.one_of(st.integers(0, 300), st.integers(0, 20000)), min_size=1, max_size=4),
       gqa=st.sampled_from(GQA), P=st.integers(1, 8), alphabet=st.sampled_from(ALPHABETS),
       seed=st.integers(0, 2**16))
def test_side_cache_step_matches_oracle_on_random_shapes(lens, gqa, P, alphabet, seed):
    """The decode step over the side cache (qsa_decode_step_pooled: the new token's K, V and
    indexer rows and its block's side-cache entry written inside the scan, then selection,
    attention and merge) on caches one token short of the generator's: the caches it leaves are
    the generator's bit for bit, every side-cache entry is the oracle's pooled key, and every
    request's results are the oracle's decode at full length."""
    hq, hkv = gqa
    w = Workload("props", len(lens), ("list",) + tuple(lens), hq, hkv, P, alphabet=alphabet)
    x = make_inputs(w, seed, "cuda")
    say(f"[prop side step] lens={lens} Hq/Hkv={hq}/{hkv} P={P} alphabet={alphabet} seed={seed}")
    k, v, idx, side, k_new, v_new, i_new = stripped_caches(x, seed)
    plan = qsa.StepPlan(k_new, v_new, i_new, x.q, x.q_idx, idx, k, v, x.page_table, x.context_lens, side, P)
    plan.run()
    torch.cuda.synchronize()
    assert torch.equal(k.view(torch.int16), x.k_cache.view(torch.int16))
    assert torch.equal(v.view(torch.int16), x.v_cache.view(torch.int16))
    assert torch.equal(idx, x.idx_cache)
    a = oracle_arrays(x)
    got, want = side_entries(side.cpu().numpy(), a)
    assert np.array_equal(got, want)
    g = dict(scores=plan.scores.cpu().numpy(), sel=plan.sel.cpu().numpy(), cnt=plan.sel_count.cpu().numpy(),
             po=plan.partial_out.cpu().numpy(), pl=plan.partial_lse.cpu().numpy(), out=plan.out.cpu().numpy(),
             lse=plan.out_lse.cpu().numpy())
    refs = oracle_decode(oracle, x, P=P)
    for b, r in enumerate(refs):
        check_request(g, b, r, x.lengths[b], what="prop side step")


@settings(max_examples=20, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(lens=st.lists(st.one_of(st.integers(0, 300), st.integers(0, 20000)), min_size=1, max_size=4),
       T=st.integers(2, 4), gqa=st.sampled_from(GQA), P=st.integers(1, 4), alphabet=st.sampled_from(ALPHABETS),
       seed=st.integers(0, 2**16))
def test_side_cache_drafts_match_oracle_on_random_shapes(lens, T, gqa, P, alphabet, seed):
    """Draft tokens scored from the side cache (qsa_decode_multi_pooled; the pages holding
    draft positions from the int8 rows): every (request, draft token) against the oracle."""
    hq, hkv = gqa
    w = Workload("propd", len(lens), ("list",) + tuple(lens), hq, hkv, P, alphabet=alphabet)
    x = make_inputs(w, seed, "cuda")
    q, qi = draft_queries(x, T, seed)
    say(f"[prop side drafts] lens={lens} T={T} Hq/Hkv={hq}/{hkv} P={P} alphabet={alphabet} seed={seed}")
    side = qsa.pool_build(x.idx_cache, x.page_table, x.context_lens)
    plan = qsa.MultiDecodePlan(q, qi, x.idx_cache, x.k_cache, x.v_cache, x.page_table, x.context_lens, P,
                               pooled=side)
    plan.run()
    torch.cuda.synchronize()
    g = dict(scores=plan.scores.cpu().numpy(), sel=plan.sel.cpu().numpy(), cnt=plan.sel_count.cpu().numpy(),
             po=plan.partial_out.cpu().numpy(), pl=plan.partial_lse.cpu().numpy(), out=plan.out.cpu().numpy(),
             lse=plan.out_lse.cpu().numpy())
    a = oracle_arrays(x)
    refs = oracle.decode_multi(bf16_bits(q), qi.cpu().numpy(), a["idx_cache"], a["k_cache"], a["v_cache"],
                               a["page_table"], a["lengths"], T, P, x.scale)
    for b, L in enumerate(lens):
        for t in range(T):
            r = b * T + t
            check_request(g, r, refs[r], oracle.draft_length(L, T, t), what=f"prop side T{T} b{b} t{t}")

"""Caches above 2^31 elements.

The requests' pages are placed at the top of indexer and K/V caches of more than 2^31
elements each (the K and V caches hold 4.5 GB of bf16 apiece), so every K/V address the
kernels form lies past element 2^31 and every page id is at least 65,600. The pages below are
filled with NaN (K/V) and the largest indexer value, so a read of a page the request does not
own would show in the scores, the selection or the outputs. The results are compared with the
oracle run on the same requests held in a compact cache.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_decode_qsa_amd import qsa
from sparse_attention_decode_qsa_amd.inputs import PAGE_SIZE, Workload, bf16_bits, draft_queries, make_inputs
from tests.helpers import oracle_arrays, oracle_decode
from tests.test_gpu_parity import check_properties, check_request, run_chain, say

pytestmark = pytest.mark.gpu

LENS = (70000, 2049, 9000, 300, 4, 131072)
HKV, HEAD_DIM = 4, 128


def _lifted(c):
    """Copy of the compact inputs c with every page moved to the top of caches whose K/V element
    count exceeds 2^31; returns (inputs on the GPU, page offset)."""
    np_small = c.k_cache.shape[0]
    np_big = (1 << 31) // (PAGE_SIZE * HKV * HEAD_DIM) + 64 + np_small
    off = np_big - np_small
    assert np_big * PAGE_SIZE * HKV * HEAD_DIM > (1 << 31) and off * PAGE_SIZE * HKV * HEAD_DIM >= (1 << 31)

    def big(t, fill):
        out = torch.empty((np_big,) + tuple(t.shape[1:]), dtype=t.dtype, device="cuda")
        out[:off].fill_(fill)
        out[off:].copy_(t.cuda())
        return out

    pt = c.page_table.clone()
    pt[pt >= 0] += off
    x = dataclasses.replace(c, q=c.q.cuda(), q_idx=c.q_idx.cuda(), idx_cache=big(c.idx_cache, 127),
                            k_cache=big(c.k_cache, float("nan")), v_cache=big(c.v_cache, float("nan")),
                            page_table=pt.cuda(), context_lens=c.context_lens.cuda())
    torch.cuda.synchronize()
    return x, off


@pytest.fixture(scope="module")
def lifted():
    c = make_inputs(Workload("big", len(LENS), ("list",) + LENS, 32, HKV, 4), 71, "cpu")
    x, off = _lifted(c)
    say(f"[large cache] {x.k_cache.numel():,} K elements per cache, pages from {off} up, lens={LENS}")
    yield c, x
    del x
    torch.cuda.empty_cache()


def test_decode_on_caches_above_2g_elements(lifted):
    c, x = lifted
    plan = qsa.DecodePlan(x.q, x.q_idx, x.idx_cache, x.k_cache, x.v_cache, x.page_table, x.context_lens, 4)
    plan.run()
    torch.cuda.synchronize()
    g = dict(scores=plan.scores.cpu().numpy(), sel=plan.sel.cpu().numpy(), cnt=plan.sel_count.cpu().numpy(),
             po=plan.partial_out.cpu().numpy(), pl=plan.partial_lse.cpu().numpy(), out=plan.out.cpu().numpy(),
             lse=plan.out_lse.cpu().numpy())
    check_properties(x, g)
    refs = oracle_decode(oracle, c)
    for b, r in enumerate(refs):
        check_request(g, b, r, LENS[b], what="large cache")
    s = run_chain(x)                    # the four entry points one by one: the same bits
    for key in ("scores", "sel", "cnt", "po", "pl", "out", "lse"):
        assert np.array_equal(s[key].view(np.int32), g[key].view(np.int32)), key
    say(f"[large cache] qsa_decode and the four calls match the oracle on all {len(LENS)} requests")


@pytest.mark.parametrize("T", [4, 16, 65])
def test_multi_token_on_caches_above_2g_elements(lifted, T):
    """Draft tokens (T = 4, dot-product or MFMA scan) and prefill chunks (T = 16: the MFMA scan
    and the pair attention kernel; T = 65: the scan's form for more than 64 queries) on the
    lifted caches."""
    c, x = lifted
    q, qi = draft_queries(c, T, 71 + T)
    plan = qsa.MultiDecodePlan(q.cuda(), qi.cuda(), x.idx_cache, x.k_cache, x.v_cache, x.page_table,
                               x.context_lens, 2)
    plan.run()
    torch.cuda.synchronize()
    g = dict(scores=plan.scores.cpu().numpy(), sel=plan.sel.cpu().numpy(), cnt=plan.sel_count.cpu().numpy(),
             po=plan.partial_out.cpu().numpy(), pl=plan.partial_lse.cpu().numpy(), out=plan.out.cpu().numpy(),
             lse=plan.out_lse.cpu().numpy())
    a = oracle_arrays(c)
    refs = oracle.decode_multi(bf16_bits(q), qi.numpy(), a["idx_cache"], a["k_cache"], a["v_cache"],
                               a["page_table"], a["lengths"], T, 2, c.scale)
    for b, L in enumerate(LENS):
        for t in range(T):
            r = b * T + t
            check_request(g, r, refs[r], oracle.draft_length(L, T, t), what=f"large cache T{T} b{b} t{t}")
    say(f"[large cache T={T}] every (request, token) matches the oracle")


def test_side_cache_step_on_caches_above_2g_elements(lifted):
    """The side-cache decode step (qsa_decode_step_pooled) on the lifted caches: each request's
    last row removed and the side cache built one token short, then the step writes the row
    back (main and side cache, past element 2^31) and decodes over the pooled keys. The caches
    must come back bit for bit and every request must match the oracle."""
    from tests.test_gpu_side_cache import _stripped
    c, x = lifted
    k, v, idx, side, k_new, v_new, i_new = _stripped(x, seed=7)
    step = qsa.StepPlan(k_new, v_new, i_new, x.q, x.q_idx, idx, k, v, x.page_table, x.context_lens, side, 4)
    step.run()
    full_side = qsa.pool_build(x.idx_cache, x.page_table, x.context_lens)
    torch.cuda.synchronize()
    for name, u, w in (("k", k, x.k_cache), ("v", v, x.v_cache), ("idx", idx, x.idx_cache)):
        assert torch.equal(u.view(torch.int8), w.view(torch.int8)), name
    pt = x.page_table.cpu().numpy()
    for b, L in enumerate(LENS):                 # the side cache of every page of every request
        for p in range((L + PAGE_SIZE - 1) // PAGE_SIZE):
            nb = min(PAGE_SIZE, L - p * PAGE_SIZE + 3) // 4
            pg = int(pt[b][p])
            assert torch.equal(side[pg, :nb], full_side[pg, :nb]), (b, p)
    g = dict(scores=step.scores.cpu().numpy(), sel=step.sel.cpu().numpy(), cnt=step.sel_count.cpu().numpy(),
             po=step.partial_out.cpu().numpy(), pl=step.partial_lse.cpu().numpy(), out=step.out.cpu().numpy(),
             lse=step.out_lse.cpu().numpy())
    refs = oracle_decode(oracle, c)
    for b, r in enumerate(refs):
        check_request(g, b, r, LENS[b], what="large cache side-cache step")
    say("[large cache] side-cache step: caches restored, every request matches the oracle")

"""The indexer's side cache on the GPU (through the C ABI) against the CPU oracle.

Side-cache entries, block scores and page maxima must match bit for bit; the decode chain
reading the side cache must give the same bits as the chain reading the int8 keys; the
decode step's cache writes must reproduce, bit for bit, the caches the input generator made
at full length.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_decode_qsa_amd import qsa
from sparse_attention_decode_qsa_amd.inputs import WORKLOADS, Workload, bf16_bits, draft_queries, make_inputs
from tests.helpers import oracle_arrays, oracle_decode
from tests.test_gpu_parity import check_request, say

pytestmark = pytest.mark.gpu

LENS = (0, 1, 2, 3, 4, 5, 63, 64, 65, 130, 2049, 9000, 70001)


def W(lens, hq=32, hkv=4, P=3, **kw):
    return Workload("side", len(lens), ("list",) + tuple(lens), hq, hkv, P, **kw)


def _valid_entries(side_gpu, a):
    """(gpu entries, oracle entries) of every block of every request, as int64 arrays."""
    ref = oracle.side_cache(a["idx_cache"], a["page_table"], a["lengths"])
    got, want = [], []
    for b, L in enumerate(a["lengths"]):
        for j in range((L + 3) // 4):
            page, slot = int(a["page_table"][b][j // 16]), j % 16
            got.append(side_gpu[page, slot])
            want.append(ref[page, slot])
    return np.array(got, dtype=np.int64), np.array(want, dtype=np.int64)


def test_pool_build_matches_oracle():
    x = make_inputs(W(LENS), 31, "cuda")
    side = qsa.pool_build(x.idx_cache, x.page_table, x.context_lens)
    torch.cuda.synchronize()
    got, want = _valid_entries(side.cpu().numpy(), oracle_arrays(x))
    say(f"[pool_build] {len(got)} block entries")
    assert np.array_equal(got, want)


def test_pooled_scores_equal_int8_scan_and_oracle():
    x = make_inputs(W(LENS), 32, "cuda")
    side = qsa.pool_build(x.idx_cache, x.page_table, x.context_lens)
    B, mp = x.page_table.shape
    pm_a = torch.full((B, mp), 7, dtype=torch.int32, device="cuda")
    pm_b = torch.full((B, mp), 7, dtype=torch.int32, device="cuda")
    s_int8 = qsa.index_score(x.q_idx, x.idx_cache, x.page_table, x.context_lens, page_max=pm_a)
    s_side = qsa.index_score_pooled(x.q_idx, side, x.page_table, x.context_lens, page_max=pm_b)
    torch.cuda.synchronize()
    a = oracle_arrays(x)
    for b, L in enumerate(x.lengths):
        nblk, npg = (L + 3) // 4, (L + 63) // 64
        ref = oracle.index_scores(a["q_idx"][b], a["idx_cache"], a["page_table"][b], L)
        assert np.array_equal(s_side[b, :nblk].cpu().numpy(), ref), b
        assert np.array_equal(s_int8[b, :nblk].cpu().numpy(), ref), b
        assert torch.equal(pm_a[b, :npg], pm_b[b, :npg]), b


@pytest.mark.parametrize("P", [1, 4])
def test_decode_pooled_equals_decode(P):
    x = make_inputs(W((70000, 3000, 20000, 2049, 0, 130), P=P), 33, "cuda")
    side = qsa.pool_build(x.idx_cache, x.page_table, x.context_lens)
    plain = qsa.DecodePlan(x.q, x.q_idx, x.idx_cache, x.k_cache, x.v_cache, x.page_table, x.context_lens, P)
    fast = qsa.DecodePlan(x.q, x.q_idx, x.idx_cache, x.k_cache, x.v_cache, x.page_table, x.context_lens, P,
                          pooled=side)
    plain.run()
    fast.run()
    torch.cuda.synchronize()
    for name in ("sel", "sel_count", "partial_out", "partial_lse", "out", "out_lse"):
        u, v = getattr(plain, name), getattr(fast, name)
        assert torch.equal(u.view(torch.int32), v.view(torch.int32)), name
    refs = oracle_decode(oracle, x, P=P)
    g = dict(scores=fast.scores.cpu().numpy(), sel=fast.sel.cpu().numpy(), cnt=fast.sel_count.cpu().numpy(),
             po=fast.partial_out.cpu().numpy(), pl=fast.partial_lse.cpu().numpy(), out=fast.out.cpu().numpy(),
             lse=fast.out_lse.cpu().numpy())
    for b, r in enumerate(refs):
        check_request(g, b, r, x.lengths[b], what="pooled")


def _stripped(x, seed=3):
    """Device copies of the caches with each request's last row overwritten by noise, the side
    cache of the requests one token shorter, and the removed rows."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    k, v, idx = x.k_cache.clone(), x.v_cache.clone(), x.idx_cache.clone()
    B, Hkv, D = len(x.lengths), k.shape[2], k.shape[3]
    k_new = torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v_new = torch.zeros_like(k_new)
    i_new = torch.zeros((B,) + tuple(idx.shape[2:]), dtype=torch.int8, device="cuda")
    pt = x.page_table.cpu().numpy()
    for b, L in enumerate(x.lengths):
        if L == 0:
            continue
        page, row = int(pt[b][(L - 1) // 64]), (L - 1) % 64
        k_new[b], v_new[b], i_new[b] = k[page, row], v[page, row], idx[page, row]
        k[page, row] = torch.randn((Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
        v[page, row] = torch.randn((Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)
        idx[page, row] = torch.randint(-127, 128, tuple(idx.shape[2:]), generator=gen, device="cuda",
                                       dtype=torch.int8)
    shorter = torch.clamp(x.context_lens - 1, min=0)
    side = qsa.pool_build(idx, x.page_table, shorter)
    return k, v, idx, side, k_new, v_new, i_new


def test_cache_append_reproduces_full_caches():
    x = make_inputs(W(LENS), 34, "cuda")
    k, v, idx, side, k_new, v_new, i_new = _stripped(x)
    qsa.cache_append(k_new, v_new, i_new, k, v, idx, x.page_table, x.context_lens, pooled=side)
    full_side = qsa.pool_build(x.idx_cache, x.page_table, x.context_lens)
    torch.cuda.synchronize()
    assert torch.equal(k.view(torch.int16), x.k_cache.view(torch.int16))
    assert torch.equal(v.view(torch.int16), x.v_cache.view(torch.int16))
    assert torch.equal(idx, x.idx_cache)
    a = oracle_arrays(x)
    got, want = _valid_entries(side.cpu().numpy(), a)
    assert np.array_equal(got, want)
    g2, _ = _valid_entries(full_side.cpu().numpy(), a)
    assert np.array_equal(got, g2)


def test_cache_append_write_flags():
    """Requests whose write flag is 0 leave every cache, main and side, untouched."""
    x = make_inputs(W(LENS), 35, "cuda")
    k, v, idx, side, k_new, v_new, i_new = _stripped(x)
    write = torch.tensor([b % 2 for b in range(len(x.lengths))], dtype=torch.int32, device="cuda")
    k0, v0, i0, s0 = k.clone(), v.clone(), idx.clone(), side.clone()
    qsa.cache_append(k_new, v_new, i_new, k, v, idx, x.page_table, x.context_lens, pooled=side, write=write)
    torch.cuda.synchronize()
    pt = x.page_table.cpu().numpy()
    for b, L in enumerate(x.lengths):
        if L == 0:
            continue
        page, row = int(pt[b][(L - 1) // 64]), (L - 1) % 64
        sp, ss = int(pt[b][(L - 1) // 64]), ((L - 1) // 4) % 16
        if b % 2:
            assert torch.equal(k[page, row].view(torch.int16), x.k_cache[page, row].view(torch.int16))
            assert torch.equal(idx[page, row], x.idx_cache[page, row])
        else:
            for new, old in ((k, k0), (v, v0)):
                assert torch.equal(new[page, row].view(torch.int16), old[page, row].view(torch.int16))
            assert torch.equal(idx[page, row], i0[page, row]) and torch.equal(side[sp, ss], s0[sp, ss])
    # nothing outside the written rows changed
    written = torch.zeros(k.shape[:2], dtype=torch.bool)
    for b, L in enumerate(x.lengths):
        if L and b % 2:
            written[int(pt[b][(L - 1) // 64]), (L - 1) % 64] = True
    assert torch.equal(k[~written].view(torch.int16), k0[~written].view(torch.int16))


def test_full_w4_pooled_chain():
    x = make_inputs(WORKLOADS["w4"], 0, "cuda")
    side = qsa.pool_build(x.idx_cache, x.page_table, x.context_lens)
    plain = qsa.DecodePlan(x.q, x.q_idx, x.idx_cache, x.k_cache, x.v_cache, x.page_table, x.context_lens, 4)
    fast = qsa.DecodePlan(x.q, x.q_idx, x.idx_cache, x.k_cache, x.v_cache, x.page_table, x.context_lens, 4,
                          pooled=side)
    plain.run()
    fast.run()
    torch.cuda.synchronize()
    for name in ("sel", "sel_count", "out", "out_lse"):
        assert torch.equal(getattr(plain, name).view(torch.int32), getattr(fast, name).view(torch.int32)), name
    for b, L in enumerate(x.lengths):
        nblk = (L + 3) // 4
        assert torch.equal(plain.scores[b, :nblk], fast.scores[b, :nblk])


@pytest.mark.parametrize("masked", [False, True])
def test_fused_step_equals_append_then_decode(masked):
    """qsa_decode_step_pooled (cache writes made by the scan) against qsa_cache_append followed
    by qsa_decode_pooled: every result and every cache, main and side, bit for bit."""
    lens = (1, 4, 5, 64, 65, 130, 2049, 9000, 70001)
    x = make_inputs(W(lens, P=4), 36, "cuda")
    write = (torch.tensor([b % 2 for b in range(len(lens))], dtype=torch.int32, device="cuda") if masked else None)
    k, v, idx, side, k_new, v_new, i_new = _stripped(x)
    k2, v2, idx2, side2 = k.clone(), v.clone(), idx.clone(), side.clone()
    # A: the two calls
    qsa.cache_append(k_new, v_new, i_new, k, v, idx, x.page_table, x.context_lens, pooled=side, write=write)
    a = qsa.DecodePlan(x.q, x.q_idx, idx, k, v, x.page_table, x.context_lens, 4, pooled=side)
    a.run()
    # B: the fused step
    bplan = qsa.StepPlan(k_new, v_new, i_new, x.q, x.q_idx, idx2, k2, v2, x.page_table, x.context_lens, side2, 4,
                         write=write)
    bplan.run()
    torch.cuda.synchronize()
    for name, u, w in (("k", k, k2), ("v", v, v2), ("idx", idx, idx2), ("side", side, side2)):
        assert torch.equal(u.view(torch.int8), w.view(torch.int8)), name
    for name in ("sel", "sel_count", "partial_out", "partial_lse", "out", "out_lse"):
        assert torch.equal(getattr(a, name).view(torch.int32), getattr(bplan, name).view(torch.int32)), name
    for b, L in enumerate(lens):
        n = (L + 3) // 4
        assert torch.equal(a.scores[b, :n], bplan.scores[b, :n]), b


def _multi(x, q, qi, P, pooled=None):
    plan = qsa.MultiDecodePlan(q, qi, x.idx_cache, x.k_cache, x.v_cache, x.page_table, x.context_lens, P,
                               pooled=pooled)
    plan.run()
    return plan


@pytest.mark.parametrize("T", [2, 3, 4])
def test_multi_pooled_equals_multi(T):
    """qsa_decode_multi_pooled (draft tokens scored from the side cache, the pages holding
    draft positions from the int8 rows) against qsa_decode_multi: scores of every draft token,
    selections, partials and outputs bit for bit, at lengths whose draft positions cross a
    block or a page boundary or cover a whole short request; the side cache pools every row
    below L_b, the draft tokens' included. Every (request, draft token) against the oracle."""
    lens = (1, 2, 3, 4, 5, 6, 63, 64, 65, 66, 67, 129, 130, 2049, 9000, 40001)
    x = make_inputs(W(lens), 40 + T, "cuda")
    q, qi = draft_queries(x, T, 40 + T)
    side = qsa.pool_build(x.idx_cache, x.page_table, x.context_lens)
    say(f"[multi pooled T={T}] lens={lens}")
    plain, fast = _multi(x, q, qi, 3), _multi(x, q, qi, 3, pooled=side)
    torch.cuda.synchronize()
    for name in ("sel", "sel_count", "partial_out", "partial_lse", "out", "out_lse"):
        u, v = getattr(plain, name), getattr(fast, name)
        assert torch.equal(u.view(torch.int32), v.view(torch.int32)), name
    a = oracle_arrays(x)
    refs = oracle.decode_multi(bf16_bits(q), qi.cpu().numpy(), a["idx_cache"], a["k_cache"], a["v_cache"],
                               a["page_table"], a["lengths"], T, 3, x.scale)
    g = dict(scores=fast.scores.cpu().numpy(), sel=fast.sel.cpu().numpy(), cnt=fast.sel_count.cpu().numpy(),
             po=fast.partial_out.cpu().numpy(), pl=fast.partial_lse.cpu().numpy(), out=fast.out.cpu().numpy(),
             lse=fast.out_lse.cpu().numpy())
    for b, L in enumerate(lens):
        for t in range(T):
            r = b * T + t
            Lt = oracle.draft_length(L, T, t)
            n = (Lt + 3) // 4
            assert torch.equal(plain.scores[r, :n], fast.scores[r, :n]), (b, t)
            check_request(g, r, refs[r], Lt, what=f"multi pooled T{T} b{b} t{t}")


def test_multi_pooled_full_w4():
    """Four draft tokens on the 256K batch: the side-cache path against the int8 path."""
    x = make_inputs(WORKLOADS["w4"], 0, "cuda")
    q, qi = draft_queries(x, 4, 0)
    side = qsa.pool_build(x.idx_cache, x.page_table, x.context_lens)
    plain, fast = _multi(x, q, qi, 4), _multi(x, q, qi, 4, pooled=side)
    torch.cuda.synchronize()
    for name in ("sel", "sel_count", "out", "out_lse"):
        assert torch.equal(getattr(plain, name).view(torch.int32), getattr(fast, name).view(torch.int32)), name

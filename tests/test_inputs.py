"""The seeded input generator: determinism, shapes, the length laws and the poison rows."""
import torch

from sparse_attention_decode_qsa_amd.inputs import (PAGE_SIZE, WORKLOADS, Workload, draft_queries, draw_lengths,
                                                    make_inputs, request_subset)


def test_same_seed_same_bits_other_seed_other_bits():
    w = Workload("t", 3, ("list", 100, 1, 700), 16, 2, 2)
    a, b, c = make_inputs(w, 7), make_inputs(w, 7), make_inputs(w, 8)
    for name in ("q", "q_idx", "idx_cache", "k_cache", "v_cache", "page_table"):
        ta, tb, tc = getattr(a, name), getattr(b, name), getattr(c, name)
        assert torch.equal(ta.view(torch.uint8) if ta.dtype == torch.bfloat16 else ta,
                           tb.view(torch.uint8) if tb.dtype == torch.bfloat16 else tb)
    assert not torch.equal(a.q.float(), c.q.float())


def test_length_laws():
    assert draw_lengths(WORKLOADS["w1"], 0) == [4096]
    assert draw_lengths(WORKLOADS["w3"], 0) == [131072] * 8
    l4 = draw_lengths(WORKLOADS["w4"], 0)
    assert len(l4) == 4 and all(65536 <= x <= 262144 for x in l4)
    l5 = draw_lengths(WORKLOADS["w5"], 0)
    assert len(l5) == 128 and all(512 <= x <= 262144 for x in l5)
    assert sum(x <= 2048 for x in l5) >= 1        # some requests must reduce to dense attention
    assert 512 in l5 and 262144 in l5             # both clips are exercised at seed 0


def test_paging_poison_and_table():
    w = Workload("t", 3, ("list", 65, 64, 130), 16, 2, 2, alphabet="u2")
    x = make_inputs(w, 3)
    pt = x.page_table
    used = sorted(int(v) for v in pt.flatten() if v >= 0)
    assert used == list(range(2 + 1 + 3))          # a permutation of all pages
    assert pt.shape == (3, 3) and int(pt[1, 1]) == -1
    assert int(x.idx_cache.abs().max()) == 127      # only the poison reaches 127
    for b, L in enumerate(x.lengths):
        last = int(pt[b, (L - 1) // PAGE_SIZE])
        r = L % PAGE_SIZE
        if r:
            assert torch.all(x.idx_cache[last, r:] == 127)
            assert torch.isnan(x.k_cache[last, r:].float()).all()
            assert torch.isnan(x.v_cache[last, r:].float()).all()
            assert int(x.idx_cache[last, :r].abs().max()) <= 2
        assert not torch.isnan(x.k_cache[last, :r or PAGE_SIZE].float()).any()


def test_planted_blocks_copy_the_query_key():
    w = Workload("t", 2, ("fixed", 4096), 16, 2, 2, paging="identity", planted=512)
    x = make_inputs(w, 1)
    for b in range(2):
        assert len(set(x.planted[b])) == 512
        j = x.planted[b][7]
        t = 4 * j
        page = int(x.page_table[b, t // PAGE_SIZE])
        assert torch.equal(x.idx_cache[page, t % PAGE_SIZE], x.q_idx[b])


def test_request_subset_keeps_request_content():
    w = Workload("t", 3, ("list", 200, 70, 129), 16, 2, 2)
    x = make_inputs(w, 4)
    s = request_subset(x, [2, 0])
    assert s.lengths == [129, 200]
    for i, b in enumerate([2, 0]):
        for t in (0, 64, 128):
            p_old = int(x.page_table[b, t // PAGE_SIZE])
            p_new = int(s.page_table[i, t // PAGE_SIZE])
            assert torch.equal(x.idx_cache[p_old, t % PAGE_SIZE], s.idx_cache[p_new, t % PAGE_SIZE])
            assert torch.equal(x.k_cache[p_old, t % PAGE_SIZE].view(torch.int16),
                               s.k_cache[p_new, t % PAGE_SIZE].view(torch.int16))


def test_correlated_chunk_queries():
    """spread = d: every new token's indexer query is the request's own query plus an offset
    in {-d..d}, clipped to the alphabet; d = 0 repeats the request's query; the attention
    queries are the independent ones either way."""
    for alphabet, lim in (("u127", 127), ("u2", 2)):
        x = make_inputs(Workload("cq", 2, ("list", 300, 70), 16, 2, 1, alphabet=alphabet), 3, "cpu")
        q_ind, qi_ind = draft_queries(x, 5, 9)
        q0, qi0 = draft_queries(x, 5, 9, spread=0)
        assert torch.equal(qi0, x.q_idx[:, None].expand(-1, 5, -1, -1))
        assert torch.equal(q0, q_ind)
        _, qi3 = draft_queries(x, 5, 9, spread=3)
        _, qi3b = draft_queries(x, 5, 9, spread=3)
        assert torch.equal(qi3, qi3b)
        d = qi3.to(torch.int16) - x.q_idx[:, None].to(torch.int16)
        assert int(d.abs().max()) <= 3 and int(qi3.abs().max()) <= lim
        assert bool((d != 0).any()) and not torch.equal(qi3, qi_ind)

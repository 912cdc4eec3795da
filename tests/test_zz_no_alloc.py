"""qsa_decode_noalloc through the C ABI against qsa_decode: two calls in a row on one device,
the second with a smaller batch (fewer requests, shorter contexts, fewer slices), each equal
to qsa_decode's results bit for bit (the same kernels; only where the workspace lives differs)."""
import sys

import pytest
import torch

from sparse_attention_decode_qsa_amd import qsa
from sparse_attention_decode_qsa_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _results(plan):
    return [t.clone() for t in (plan.scores, plan.sel, plan.sel_count, plan.partial_out, plan.partial_lse,
                                plan.out, plan.out_lse)]


def _case(lens, P, seed):
    w = Workload("noalloc", len(lens), ("list",) + tuple(lens), 32, 4, P)
    x = make_inputs(w, seed, "cuda")
    args = (x.q, x.q_idx, x.idx_cache, x.k_cache, x.v_cache, x.page_table, x.context_lens, P)
    return x, qsa.DecodePlan(*args), qsa.DecodePlan(*args, noalloc=True)


def test_noalloc_equals_decode_twice_second_smaller():
    big = _case((70000, 3000, 20000, 2049, 131072), 4, 21)
    small = _case((5000, 777), 2, 22)
    assert small[0].batch < big[0].batch and max(small[0].lengths) < max(big[0].lengths)
    for name, (x, ref, na) in (("first (5 requests)", big), ("second (2 requests)", small)):
        print(f"[noalloc] {name}: lengths {x.lengths}", flush=True)
        sys.stdout.flush()
        for t in (na.sel, na.partial_out, na.out, na.out_lse):
            t.fill_(-7)                                  # stale values must not survive
        ref.run()
        na.run()
        torch.cuda.synchronize()
        for key, u, v in zip(("scores", "sel", "count", "partial_out", "partial_lse", "out", "lse"),
                             _results(ref), _results(na)):
            if key == "scores":
                u = torch.cat([u[b, :(L + 3) // 4] for b, L in enumerate(x.lengths)])
                v = torch.cat([v[b, :(L + 3) // 4] for b, L in enumerate(x.lengths)])
            assert torch.equal(u.view(torch.int32), v.view(torch.int32)), f"{name}: {key} differs"


def test_noalloc_replays_from_a_hip_graph():
    """The allocation-free call captured in a HIP graph (its workspace address is fixed, so the
    graph holds no allocation): every replay, with eager work in between, gives qsa_decode's bits."""
    x, ref, na = _case((9000, 70000, 2049), 4, 23)
    ref.run()
    torch.cuda.synchronize()
    want = _results(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        na.run()                                         # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        na.run()
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for t in (na.sel, na.partial_out, na.out, na.out_lse):
            t.fill_(-7)
        junk.mul_(1.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key, u, v in zip(("scores", "sel", "count", "partial_out", "partial_lse", "out", "lse"), want,
                             _results(na)):
            if key == "scores":
                u = torch.cat([u[b, :(L + 3) // 4] for b, L in enumerate(x.lengths)])
                v = torch.cat([v[b, :(L + 3) // 4] for b, L in enumerate(x.lengths)])
            assert torch.equal(u.view(torch.int32), v.view(torch.int32)), f"replay {rep}: {key} differs"

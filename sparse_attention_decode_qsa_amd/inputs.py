"""Seeded synthetic inputs for the QSA decode path.

This module only draws numbers and lays them out in paged caches. It holds no step of
the method itself: no pooling, scoring, selection, softmax or merge. Both the CPU
oracle (through the tests) and the HIP library consume what it produces.

Workloads follow the article "Qwen 4 QSA gets decode context parallelism: inside
vLLM's draft PR for Qwen3.8-Flash-Next", section "What the pull request actually
changes" (micro-blocks of 4 tokens, 512 kept blocks, softmax and value aggregation on
the full K/V rows, each context read as slices whose partials are then joined), at the
shapes of the five decode workloads this library is measured on:

  w1  B=1,   L=4096,                       Hq/Hkv=16/2, identity pages, P=1
  w2  B=32,  L=32768,                      Hq/Hkv=16/2, identity pages, P=2, 512 planted blocks
  w3  B=8,   L=131072,                     Hq/Hkv=32/4, shuffled pages, P=4
  w4  B=4,   L uniform in [65536, 262144], Hq/Hkv=32/4, shuffled pages, P=4  (256K context)
  w5  B=128, L lognormal(median 16384, sigma 1.5) clipped to [512, 262144],
             Hq/Hkv=32/4, shuffled pages, P=4, indexer values in {-2..2}

Layouts (all row-major):
  q           [B, Hq, 128]          bf16, N(0,1) rounded to nearest even
  q_idx       [B, 4, 64]            int8
  idx_cache   [NP, 64, 4, 64]       int8  (one page = 64 tokens = 16 KiB)
  k_cache     [NP, 64, Hkv, 128]    bf16
  v_cache     [NP, 64, Hkv, 128]    bf16
  page_table  [B, max_pages]        int32 (unused entries are -1)
  context_lens[B]                   int32

Rows of a request's last page beyond its length are poisoned (K/V = NaN, indexer keys
= 127) so that a read past the context shows up in the results.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

PAGE_SIZE = 64
HEAD_DIM = 128
IDX_HEADS = 4
IDX_DIM = 64
TOP_BLOCKS = 512
MAX_CONTEXT = 262144


@dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic decode batch."""

    name: str
    batch: int
    lengths: tuple          # ("fixed", L) | ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi) | ("list", L0, L1, ...)
    hq: int
    hkv: int
    slices: int
    alphabet: str = "u127"  # "u127": uniform integers in [-127, 127]; "u2": uniform in [-2, 2]; "zero_q": keys u127, q_idx = 0
    paging: str = "shuffled"  # "identity" | "shuffled"
    planted: int = 0        # blocks per request whose indexer keys equal q_idx
    max_context: int = 0    # page-table capacity in tokens (0: the largest drawn length)
    k: int = TOP_BLOCKS

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "w1": Workload("w1", 1, ("fixed", 4096), 16, 2, 1, paging="identity"),
    "w2": Workload("w2", 32, ("fixed", 32768), 16, 2, 2, paging="identity", planted=512),
    "w3": Workload("w3", 8, ("fixed", 131072), 32, 4, 4),
    "w4": Workload("w4", 4, ("uniform", 65536, 262144), 32, 4, 4, max_context=MAX_CONTEXT),
    "w4_fixed": Workload("w4_fixed", 4, ("fixed", 262144), 32, 4, 4, max_context=MAX_CONTEXT),
    "w5": Workload("w5", 128, ("lognormal", 16384, 1.5, 512, 262144), 32, 4, 4,
                   alphabet="u2", max_context=MAX_CONTEXT),
}


@dataclass
class DecodeInputs:
    workload: Workload
    seed: int
    q: torch.Tensor
    q_idx: torch.Tensor
    idx_cache: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    page_table: torch.Tensor
    context_lens: torch.Tensor
    lengths: list            # host copy of context_lens
    planted: list = field(default_factory=list)  # per request: sorted planted block ids (or [])

    @property
    def batch(self) -> int:
        return len(self.lengths)

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def max_blocks(self) -> int:
        return self.max_pages * PAGE_SIZE // 4

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_DIM)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _request_seed(seed: int, b: int) -> int:
    return (seed << 24) + 0x9E37 + b


def draw_lengths(w: Workload, seed: int) -> list:
    g = _gen("cpu", seed)
    kind = w.lengths[0]
    if kind == "fixed":
        return [int(w.lengths[1])] * w.batch
    if kind == "list":
        lens = [int(x) for x in w.lengths[1:]]
        assert len(lens) == w.batch
        return lens
    if kind == "uniform":
        lo, hi = int(w.lengths[1]), int(w.lengths[2])
        return [int(x) for x in torch.randint(lo, hi + 1, (w.batch,), generator=g)]
    if kind == "lognormal":
        median, sigma, lo, hi = w.lengths[1:]
        z = torch.randn(w.batch, generator=g, dtype=torch.float64)
        raw = torch.floor(median * torch.exp(sigma * z))
        return [int(x) for x in torch.clamp(raw, lo, hi)]
    raise ValueError(f"unknown length law {kind}")


def _int_values(shape, alphabet: str, g, device) -> torch.Tensor:
    lo, hi = (-2, 2) if alphabet == "u2" else (-127, 127)
    return torch.randint(lo, hi + 1, shape, generator=g, device=device, dtype=torch.int8)


def make_inputs(w: Workload, seed: int = 0, device="cpu") -> DecodeInputs:
    """Draw one batch. The same (workload, seed, device type) always gives the same bits."""
    device = torch.device(device)
    lens = draw_lengths(w, seed)
    B = w.batch
    npages = [(L + PAGE_SIZE - 1) // PAGE_SIZE for L in lens]
    cap_tokens = max(w.max_context, max(lens) if lens else 0, 1)
    max_pages = (cap_tokens + PAGE_SIZE - 1) // PAGE_SIZE
    total_pages = sum(npages)

    g0 = _gen("cpu", seed ^ 0x51A5)
    planted = []
    for b in range(B):
        if w.planted:
            nblk = (lens[b] + 3) // 4
            assert nblk >= w.planted
            ids = torch.randperm(nblk, generator=g0)[: w.planted]
            planted.append(sorted(int(x) for x in ids))
        else:
            planted.append([])
    if w.paging == "identity":
        phys = torch.arange(total_pages, dtype=torch.int32)
    else:
        phys = torch.randperm(total_pages, generator=g0).to(torch.int32)

    page_table = torch.full((B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        page_table[b, : npages[b]] = phys[off: off + npages[b]]
        off += npages[b]

    NP = max(total_pages, 1)
    q = torch.empty((B, w.hq, HEAD_DIM), dtype=torch.bfloat16, device=device)
    q_idx = torch.empty((B, IDX_HEADS, IDX_DIM), dtype=torch.int8, device=device)
    idx_cache = torch.zeros((NP, PAGE_SIZE, IDX_HEADS, IDX_DIM), dtype=torch.int8, device=device)
    k_cache = torch.zeros((NP, PAGE_SIZE, w.hkv, HEAD_DIM), dtype=torch.bfloat16, device=device)
    v_cache = torch.zeros((NP, PAGE_SIZE, w.hkv, HEAD_DIM), dtype=torch.bfloat16, device=device)

    key_alphabet = "u127" if w.alphabet == "zero_q" else w.alphabet
    off = 0
    for b in range(B):
        g = _gen(device, _request_seed(seed, b))
        L, n = lens[b], npages[b]
        q[b] = torch.randn((w.hq, HEAD_DIM), generator=g, device=device).to(torch.bfloat16)
        qi = _int_values((IDX_HEADS, IDX_DIM), key_alphabet, g, device)
        if w.alphabet == "zero_q":
            qi.zero_()
        q_idx[b] = qi
        if n == 0:
            continue
        pages = phys[off: off + n].to(device=device, dtype=torch.long)
        off += n
        rows = n * PAGE_SIZE
        keys = _int_values((rows, IDX_HEADS, IDX_DIM), key_alphabet, g, device)
        for j in planted[b]:
            keys[4 * j: 4 * j + 4] = q_idx[b]
        kk = torch.randn((rows, w.hkv, HEAD_DIM), generator=g, device=device).to(torch.bfloat16)
        vv = torch.randn((rows, w.hkv, HEAD_DIM), generator=g, device=device).to(torch.bfloat16)
        if L < rows:  # poison the unused rows of the last page
            keys[L:] = 127
            kk[L:] = float("nan")
            vv[L:] = float("nan")
        idx_cache.index_copy_(0, pages, keys.view(n, PAGE_SIZE, IDX_HEADS, IDX_DIM))
        k_cache.index_copy_(0, pages, kk.view(n, PAGE_SIZE, w.hkv, HEAD_DIM))
        v_cache.index_copy_(0, pages, vv.view(n, PAGE_SIZE, w.hkv, HEAD_DIM))
        del keys, kk, vv

    return DecodeInputs(
        workload=w, seed=seed, q=q, q_idx=q_idx, idx_cache=idx_cache, k_cache=k_cache,
        v_cache=v_cache, page_table=page_table.to(device),
        context_lens=torch.tensor(lens, dtype=torch.int32, device=device),
        lengths=lens, planted=planted)


def draft_queries(x: DecodeInputs, T: int, seed: int = 0, spread: int | None = None):
    """Queries of T draft tokens per request: (q [B, T, Hq, 128] bf16, q_idx [B, T, 4, 64] int8),
    drawn like the single query (bf16 of N(0,1); indexer values from the workload's alphabet)
    from one generator per request, independently for every token.

    spread = d (correlated chunk queries): token t's indexer query is instead the request's own
    query x.q_idx[b] plus an offset drawn uniformly from {-d..d} per element, clipped to the
    alphabet's range, so the tokens of a chunk select overlapping block sets (d = 0: all the
    same query). The attention queries stay independent."""
    w = x.workload
    device = x.q.device
    B = x.batch
    q = torch.empty((B, T, w.hq, HEAD_DIM), dtype=torch.bfloat16, device=device)
    q_idx = torch.empty((B, T, IDX_HEADS, IDX_DIM), dtype=torch.int8, device=device)
    alphabet = "u127" if w.alphabet == "zero_q" else w.alphabet
    lo, hi = (-2, 2) if alphabet == "u2" else (-127, 127)
    for b in range(B):
        g = _gen(device, _request_seed(seed ^ 0x7D1F, b))
        q[b] = torch.randn((T, w.hq, HEAD_DIM), generator=g, device=device).to(torch.bfloat16)
        if spread is None:
            qi = _int_values((T, IDX_HEADS, IDX_DIM), alphabet, g, device)
        else:
            off = torch.randint(-spread, spread + 1, (T, IDX_HEADS, IDX_DIM), generator=g, device=device,
                                dtype=torch.int16)
            qi = (x.q_idx[b].to(torch.int16)[None] + off).clamp_(lo, hi).to(torch.int8)
        if w.alphabet == "zero_q":
            qi.zero_()
        q_idx[b] = qi
    return q, q_idx


def bf16_bits(t: torch.Tensor):
    """Raw bf16 bit patterns as a host numpy uint16 array (exact, no rounding)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")


def request_subset(x: DecodeInputs, rows: list) -> DecodeInputs:
    """The requests `rows` of a batch as a batch of their own: only their pages, renumbered.

    Used to hand a few sampled requests of a large batch to the CPU oracle.
    """
    B = len(rows)
    lens = [x.lengths[b] for b in rows]
    npages = [(L + PAGE_SIZE - 1) // PAGE_SIZE for L in lens]
    max_pages = max(max(npages), 1)
    pt = torch.full((B, max_pages), -1, dtype=torch.int32)
    chunks_i, chunks_k, chunks_v = [], [], []
    off = 0
    for i, b in enumerate(rows):
        ids = x.page_table[b, : npages[i]].to(torch.long)
        chunks_i.append(x.idx_cache.index_select(0, ids.to(x.idx_cache.device)))
        chunks_k.append(x.k_cache.index_select(0, ids.to(x.k_cache.device)))
        chunks_v.append(x.v_cache.index_select(0, ids.to(x.v_cache.device)))
        pt[i, : npages[i]] = torch.arange(off, off + npages[i], dtype=torch.int32)
        off += npages[i]
    sel = torch.tensor(rows, dtype=torch.long, device=x.q.device)
    return DecodeInputs(
        workload=x.workload.with_(batch=B), seed=x.seed,
        q=x.q.index_select(0, sel), q_idx=x.q_idx.index_select(0, sel),
        idx_cache=torch.cat(chunks_i), k_cache=torch.cat(chunks_k), v_cache=torch.cat(chunks_v),
        page_table=pt.to(x.page_table.device),
        context_lens=torch.tensor(lens, dtype=torch.int32, device=x.context_lens.device),
        lengths=lens, planted=[x.planted[b] for b in rows])

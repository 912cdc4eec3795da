"""CPU oracle for the QSA decode path: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this module;
only the tests, the smoke check and the benchmark's CPU-baseline leg use it. It shares no
code with the HIP library and does not import it.

Integers are exact (numpy int64, with an explicit check that every block score fits in
int32). Floating point is float64 throughout, starting from the exact values of the bf16
inputs.

What it follows. The article "Qwen 4 QSA gets decode context parallelism: inside vLLM's
draft PR for Qwen3.8-Flash-Next" (orcarouter.ai blog):

  [QSA]   section "What the pull request actually changes", second paragraph: a light
          indexer pools the keys of every 4 consecutive tokens into a micro-block, scores them,
          keeps the 512 best (about 2,048 token positions), and the final softmax and the
          value aggregation use the full K and V rows of the kept tokens, not pooled ones.
  [SPLIT] same section, first paragraph and first bullets: with decode context
          parallelism the main KV cache is sharded by context position, a rank attends
          over its own contiguous piece, and a second step joins the pieces.
  [MERGE] section "Questions worth answering directly", answer on how DCP differs from
          tensor parallelism: the shards are pieces of the sequence rather than of the
          heads, so the per-piece attention partials have to be joined at the end.
  [GROUP] section "What the pull request actually changes", bullets: the selector's cache and
          the main K/V cache belong to a single cache group (here: one page table and one length per
          request serve both the indexer keys and K/V).

Readings where the pages leave a step open (each is repeated in the design notes):

  R1 pooling      the pooled key of a micro-block is the integer sum of the int8 indexer
                  keys of its (up to) 4 consecutive tokens.
  R2 score        score = sum over the 4 indexer heads of dot(q_idx[h], pooled[h]); one
                  q_idx per request; no weights, scaling or nonlinearity.
  R3 blocks       block j holds logical positions 4j .. 4j+3; a request of length L has
                  ceil(L/4) blocks and the last one pools only the tokens that exist.
  R4 fewer blocks K = min(512, number of blocks); all blocks are kept when there are
                  at most 512.
  R5 ties         order by higher score, then lower block index; the kept ids are
                  reported in ascending order.
  R6 sharing      one selection per request, shared by every query head and every slice.
  R7 attention    one decode query per request; scale 1/sqrt(head_dim); query head h
                  reads KV head h // (Hq/Hkv).
  R8 slices       the request's pages are cut into P contiguous runs of
                  ceil(ceil(L/page)/P) pages; slice p covers tokens
                  [p*S*page, min((p+1)*S*page, L)); a slice may hold no kept token.
  R9 partials     a slice's partial is (slice-normalised output, lse = max + ln sum);
                  an empty slice is (0, -inf). The merge skips -inf partials.
  R10 empty       a request of length 0 keeps nothing; its output is 0 and its lse -inf.
  R11 side cache  the side cache the indexer maintains ([QSA] paragraph: besides the main
                  cache the indexer keeps a selector cache and side caches of its own) holds the
                  pooled key (R1) of every micro-block, page-aligned like the main cache:
                  block j of a request sits in page page_table[j // (page/4)], slot
                  j % (page/4). Scores read from it are R2 on the stored keys.
  R12 append      a decode step writes its token at position L-1 (L counts the new token):
                  the K, V and indexer rows go there, and the side-cache entry of block
                  (L-1)//4 becomes the sum of that block's indexer rows at positions < L.
                  A request whose write flag is 0 writes nothing (section "What the pull
                  request actually changes", bullets: synthetic batches must not write the
                  side caches); neither does a request of length 0.
  R13 draft       multi-token decode (T new tokens: speculative drafts, or a prefill chunk):
                  the T new tokens are the last T positions of the cache (L counts them all); token t
                  sits at position L-T+t and is decoded exactly as a single token at length
                  L-T+1+t - its own indexer query and selection, attention over its own kept
                  tokens, slices of that length - so it sees itself and the tokens before it.
"""
from __future__ import annotations

import numpy as np

TOKENS_PER_BLOCK = 4
TOP_BLOCKS = 512
INT32_MAX = 2**31 - 1


# ---------------------------------------------------------------------------- inputs

def bf16_to_f64(x) -> np.ndarray:
    """bf16 values as float64. Accepts raw bf16 bits (uint16) or any float array."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def request_rows(cache: np.ndarray, page_table_row: np.ndarray, length: int) -> np.ndarray:
    """Rows 0 .. length-1 of one request, in logical order, read through its page table.

    Logical position t lives in physical page page_table_row[t // page_size], row
    t % page_size. [GROUP]: indexer keys and K/V use the same table.
    """
    page_size = cache.shape[1]
    out = []
    for p in range(-(-length // page_size)):
        take = min(page_size, length - p * page_size)
        out.append(cache[int(page_table_row[p]), :take])
    if not out:
        return np.zeros((0,) + cache.shape[2:], dtype=cache.dtype)
    return np.concatenate(out, axis=0)


# ------------------------------------------------------------------------ indexer [QSA]

def pooled_keys(idx_rows: np.ndarray) -> np.ndarray:
    """Micro-block pooling, R1 and R3: pooled[j] = sum of the keys of tokens 4j..4j+3 < L."""
    L = idx_rows.shape[0]
    nblk = -(-L // TOKENS_PER_BLOCK)
    pooled = np.zeros((nblk,) + idx_rows.shape[1:], dtype=np.int64)
    for i in range(TOKENS_PER_BLOCK):
        tok = idx_rows[i::TOKENS_PER_BLOCK].astype(np.int64)   # tokens 4j + i
        pooled[: tok.shape[0]] += tok
    return pooled


def block_scores(q_idx: np.ndarray, pooled: np.ndarray) -> np.ndarray:
    """Block score, R2: S[j] = sum_h sum_d q_idx[h, d] * pooled[j, h, d] (exact int64)."""
    s = (pooled * q_idx.astype(np.int64)[None]).sum(axis=(1, 2))
    assert np.all(np.abs(s) <= INT32_MAX), "block score outside int32"
    return s


def index_scores(q_idx, idx_cache, page_table_row, length) -> np.ndarray:
    """All block scores of one request."""
    return block_scores(np.asarray(q_idx), pooled_keys(request_rows(idx_cache, page_table_row, length)))


def select_blocks(scores: np.ndarray, k: int = TOP_BLOCKS) -> np.ndarray:
    """Keep the best min(k, n) blocks, R4 and R5: higher score first, then lower index.

    Returns the kept block ids in ascending order.
    """
    n = scores.shape[0]
    K = min(k, n)
    j = np.arange(n)
    order = np.lexsort((j, -np.asarray(scores, dtype=np.int64)))   # primary: -score, then j
    return np.sort(order[:K])


def kept_tokens(kept_blocks: np.ndarray, length: int) -> np.ndarray:
    """Token positions of the kept blocks (the tail block only up to length-1)."""
    toks = (np.asarray(kept_blocks, dtype=np.int64)[:, None] * TOKENS_PER_BLOCK
            + np.arange(TOKENS_PER_BLOCK)[None]).reshape(-1)
    return toks[toks < length]


# ------------------------------------------------------ side cache and cache writes [QSA]

def side_cache(idx_cache: np.ndarray, page_table: np.ndarray, lengths) -> np.ndarray:
    """R11: side cache [pages, page_size/4, heads, dim] (int64) holding the pooled key of
    every block of every request; entries that belong to no block are 0."""
    pages, page_size = idx_cache.shape[:2]
    bpp = page_size // TOKENS_PER_BLOCK
    out = np.zeros((pages, bpp) + idx_cache.shape[2:], dtype=np.int64)
    for b, L in enumerate(lengths):
        pooled = pooled_keys(request_rows(idx_cache, page_table[b], int(L)))
        for j in range(pooled.shape[0]):
            out[int(page_table[b][j // bpp]), j % bpp] = pooled[j]
    return out


def side_scores(q_idx, side: np.ndarray, page_table_row, length: int) -> np.ndarray:
    """Block scores of one request read from the side cache (R2 on the stored keys)."""
    bpp = side.shape[1]
    nblk = -(-int(length) // TOKENS_PER_BLOCK)
    pooled = np.zeros((nblk,) + side.shape[2:], dtype=np.int64)
    for j in range(nblk):
        pooled[j] = side[int(page_table_row[j // bpp]), j % bpp]
    return block_scores(np.asarray(q_idx), pooled)


def append_token(k_cache, v_cache, idx_cache, side, page_table, lengths, k_new, v_new, idx_new,
                 write=None):
    """R12 on copies of the caches; returns the new (k_cache, v_cache, idx_cache, side).

    k_new, v_new [B, Hkv, D] (bf16 bits), idx_new [B, heads, dim] int8; write [B] or None.
    """
    k2, v2, i2, s2 = (np.array(a, copy=True) for a in (k_cache, v_cache, idx_cache, side))
    page_size = idx_cache.shape[1]
    bpp = page_size // TOKENS_PER_BLOCK
    for b, L in enumerate(lengths):
        L = int(L)
        if L == 0 or (write is not None and not write[b]):
            continue
        t = L - 1
        page, row = int(page_table[b][t // page_size]), t % page_size
        k2[page, row] = k_new[b]
        v2[page, row] = v_new[b]
        i2[page, row] = idx_new[b]
        j = t // TOKENS_PER_BLOCK
        total = np.zeros(idx_cache.shape[2:], dtype=np.int64)
        for u in range(TOKENS_PER_BLOCK * j, L):
            total += i2[int(page_table[b][u // page_size]), u % page_size].astype(np.int64)
        s2[int(page_table[b][j // bpp]), j % bpp] = total
    return k2, v2, i2, s2


# ---------------------------------------------------------------------- attention [QSA]

def attend(q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float):
    """Softmax attention of one decode query over the given rows, R7.

    q [Hq, D]; k_rows, v_rows [T, Hkv, D] (float64). Returns o [Hq, D] and lse [Hq]
    (natural log). With T = 0 the result is (0, -inf), R9.
    """
    Hq, D = q.shape
    T, Hkv = k_rows.shape[0], k_rows.shape[1]
    group = Hq // Hkv
    o = np.zeros((Hq, D))
    lse = np.full(Hq, -np.inf)
    if T == 0:
        return o, lse
    for h in range(Hq):
        g = h // group
        s = (k_rows[:, g, :] @ q[h]) * scale
        m = s.max()
        w = np.exp(s - m)
        l = w.sum()
        o[h] = (w @ v_rows[:, g, :]) / l
        lse[h] = m + np.log(l)
    return o, lse


# ------------------------------------------------------------------ split read [SPLIT]

def slice_ranges(length: int, P: int, page_size: int):
    """Token range of each of the P contiguous page-aligned slices, R8."""
    npages = -(-length // page_size)
    per = -(-npages // P) if npages else 0
    out = []
    for p in range(P):
        lo = min(p * per * page_size, length)
        hi = min((p + 1) * per * page_size, length)
        out.append((lo, hi))
    return out


def partial_attention(q, k_rows, v_rows, tokens, ranges, scale):
    """Per-slice partials over the kept tokens that fall in each slice, R8 and R9.

    k_rows[i], v_rows[i] are the K/V rows of token position tokens[i].
    """
    Hq, D = q.shape
    P = len(ranges)
    o_part = np.zeros((P, Hq, D))
    lse_part = np.full((P, Hq), -np.inf)
    for p, (lo, hi) in enumerate(ranges):
        inside = (tokens >= lo) & (tokens < hi)
        o_part[p], lse_part[p] = attend(q, k_rows[inside], v_rows[inside], scale)
    return o_part, lse_part


# ------------------------------------------------------------------------ merge [MERGE]

def lse_merge(o_part: np.ndarray, lse_part: np.ndarray):
    """Log-sum-exp merge of slice partials: M = max finite lse_p, w_p = exp(lse_p - M),
    O = sum w_p o_p / sum w_p, lse = M + ln sum w_p. Partials with lse = -inf carry no
    weight; if every partial is -inf the result is (0, -inf), R10.
    """
    P, Hq, D = o_part.shape
    o = np.zeros((Hq, D))
    lse = np.full(Hq, -np.inf)
    for h in range(Hq):
        finite = np.isfinite(lse_part[:, h])
        if not finite.any():
            continue
        M = lse_part[finite, h].max()
        w = np.where(finite, np.exp(np.where(finite, lse_part[:, h], 0.0) - M), 0.0)
        o[h] = (w[:, None] * np.where(finite[:, None], o_part[:, h, :], 0.0)).sum(axis=0) / w.sum()
        lse[h] = M + np.log(w.sum())
    return o, lse


# -------------------------------------------------------------------------- whole path

def decode_request(q, q_idx, idx_cache, k_cache, v_cache, page_table_row, length,
                   P: int, scale: float, k: int = TOP_BLOCKS) -> dict:
    """The whole decode path for one request: index -> select -> per-slice attention -> merge.

    q [Hq, D] (bf16 bits or float), q_idx [4, 64] int, caches paged as
    [pages, page_size, heads, dim]. Returns every intermediate.
    """
    page_size = idx_cache.shape[1]
    scores = index_scores(q_idx, idx_cache, page_table_row, length)
    kept = select_blocks(scores, k)
    tokens = kept_tokens(kept, length)
    k_rows = bf16_to_f64(request_rows(k_cache, page_table_row, length)[tokens])
    v_rows = bf16_to_f64(request_rows(v_cache, page_table_row, length)[tokens])
    qf = bf16_to_f64(q)
    ranges = slice_ranges(length, P, page_size)
    o_part, lse_part = partial_attention(qf, k_rows, v_rows, tokens, ranges, scale)
    out, lse = lse_merge(o_part, lse_part)
    return dict(scores=scores, kept=kept, tokens=tokens, ranges=ranges, o_part=o_part,
                lse_part=lse_part, out=out, lse=lse)


def decode(q, q_idx, idx_cache, k_cache, v_cache, page_table, lengths, P: int,
           scale: float, k: int = TOP_BLOCKS) -> list:
    """decode_request for every request of a batch."""
    return [decode_request(q[b], q_idx[b], idx_cache, k_cache, v_cache, page_table[b],
                           int(lengths[b]), P, scale, k) for b in range(len(lengths))]


def draft_length(length: int, T: int, t: int) -> int:
    """R13: the context seen by draft token t of T (itself included)."""
    return max(0, int(length) - (T - 1 - t))


def decode_multi(q, q_idx, idx_cache, k_cache, v_cache, page_table, lengths, T: int, P: int,
                 scale: float, k: int = TOP_BLOCKS) -> list:
    """R13: q [B, T, Hq, D], q_idx [B, T, 4, 64]; one result per (request, draft token), in
    the order b*T + t, each a single-token decode at length L_b - T + 1 + t."""
    out = []
    for b in range(len(lengths)):
        for t in range(T):
            out.append(decode_request(q[b][t], q_idx[b][t], idx_cache, k_cache, v_cache, page_table[b],
                                      draft_length(lengths[b], T, t), P, scale, k))
    return out

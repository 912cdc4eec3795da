"""Plant plausible mistakes in the CPU oracle and check that a pin catches each one.

The mistakes are planted in the oracle only, on the CPU, by swapping one of its
functions for a wrong variant for the duration of one test.
"""
import numpy as np
import pytest

import oracle
import oracle.qsa_oracle as Q
from tests import test_oracle as pins
from tests import test_oracle_multi as multi_pins
from tests import test_oracle_side as side_pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(Q, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _pooled_floor(idx_rows):            # drops the partial tail block
    L = idx_rows.shape[0] // 4 * 4
    return Q.__dict__["_orig_pooled"](idx_rows[:L])


def _pooled_shifted(idx_rows):          # pools tokens 4j+1 .. 4j+4
    return Q.__dict__["_orig_pooled"](idx_rows[1:])


def _scores_sign(q_idx, pooled):        # wrong sign on the last indexer head
    q = q_idx.astype(np.int64).copy()
    q[-1] = -q[-1]
    return (pooled * q[None]).sum(axis=(1, 2))


def _select_tie_high(scores, k=512):    # ties go to the higher index
    n = len(scores)
    order = np.lexsort((-np.arange(n), -np.asarray(scores)))
    return np.sort(order[: min(k, n)])


def _select_lowest(scores, k=512):      # keeps the lowest scores
    n = len(scores)
    order = np.lexsort((np.arange(n), np.asarray(scores)))
    return np.sort(order[: min(k, n)])


def _attend_head_mod(q, k_rows, v_rows, scale):   # query head h reads KV head h % Hkv
    Hq, Hkv = q.shape[0], k_rows.shape[1]
    perm = np.array([(h % Hkv) * (Hq // Hkv) + h // Hkv for h in range(Hq)])
    o, lse = Q.__dict__["_orig_attend"](q[perm], k_rows, v_rows, scale)
    inv = np.argsort(perm)
    return o[inv], lse[inv]


def _attend_no_scale(q, k_rows, v_rows, scale):
    return Q.__dict__["_orig_attend"](q, k_rows, v_rows, 1.0)


def _slices_token_split(length, P, page_size):     # not page aligned
    per = -(-length // P) if length else 0
    return [(min(p * per, length), min((p + 1) * per, length)) for p in range(P)]


def _merge_unnormalised(o_part, lse_part):          # forgets to divide by sum w
    P, Hq, D = o_part.shape
    o, lse = np.zeros((Hq, D)), np.full(Hq, -np.inf)
    for h in range(Hq):
        fin = np.isfinite(lse_part[:, h])
        if fin.any():
            M = lse_part[fin, h].max()
            w = np.where(fin, np.exp(np.where(fin, lse_part[:, h], 0.0) - M), 0.0)
            o[h] = (w[:, None] * o_part[:, h]).sum(axis=0)
            lse[h] = M + np.log(w.sum())
    return o, lse


def _rows_ignore_table(cache, page_table_row, length):
    return Q.__dict__["_orig_rows"](cache, np.arange(len(page_table_row)), length)


def _side_slot_shift(idx_cache, page_table, lengths):   # block j stored one slot late
    s = Q.__dict__["_orig_side"](idx_cache, page_table, lengths)
    return np.roll(s, 1, axis=1)


def _append_whole_block(k_cache, v_cache, idx_cache, side, page_table, lengths, k_new, v_new, idx_new,
                        write=None):                      # pools all 4 rows of the block, even past L
    k2, v2, i2, s2 = Q.__dict__["_orig_append"](k_cache, v_cache, idx_cache, side, page_table, lengths,
                                                k_new, v_new, idx_new, write)
    for b, L in enumerate(lengths):
        if L == 0:
            continue
        j = (L - 1) // 4
        total = sum(i2[int(page_table[b][u // 64]), u % 64].astype(np.int64) for u in range(4 * j, 4 * j + 4))
        s2[int(page_table[b][j // 16]), j % 16] = total
    return k2, v2, i2, s2


def _append_new_row_only(k_cache, v_cache, idx_cache, side, page_table, lengths, k_new, v_new, idx_new,
                         write=None):                     # forgets the block's earlier tokens
    k2, v2, i2, s2 = Q.__dict__["_orig_append"](k_cache, v_cache, idx_cache, side, page_table, lengths,
                                                k_new, v_new, idx_new, write)
    for b, L in enumerate(lengths):
        if L:
            j = (L - 1) // 4
            s2[int(page_table[b][j // 16]), j % 16] = idx_new[b].astype(np.int64)
    return k2, v2, i2, s2


def _bf16_as_fp16(x):                    # reads the bits as IEEE half precision
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return a.view(np.float16).astype(np.float64)
    return a.astype(np.float64)


def _bf16_shift8(x):                     # places the 16 bits 8 positions too low in the float32
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 8).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _draft_one_short(length, T, t):              # draft token t misses itself
    return max(0, int(length) - (T - t))


def _draft_sees_all(length, T, t):               # no causality inside the draft
    return int(length)


Q._orig_side = Q.side_cache
Q._orig_append = Q.append_token
Q._orig_pooled = Q.pooled_keys
Q._orig_attend = Q.attend
Q._orig_rows = Q.request_rows

MUTATIONS = [
    ("pooled_keys", _pooled_floor, lambda: pins.test_scores_brute_force((1, 3))),
    ("pooled_keys", _pooled_shifted, lambda: pins.test_scores_brute_force((5, 64))),
    ("block_scores", _scores_sign, lambda: pins.test_scores_brute_force((65, 130))),
    ("select_blocks", _select_tie_high, pins.test_select_all_ties_keeps_lowest_indices),
    ("select_blocks", _select_lowest, pins.test_select_monotone_scores_pin_direction),
    ("attend", _attend_head_mod, lambda: pins.test_short_context_equals_dense_attention(100)),
    ("attend", _attend_no_scale, lambda: pins.test_short_context_equals_dense_attention(5)),
    ("slice_ranges", _slices_token_split, pins.test_slice_ranges_table),
    ("lse_merge", _merge_unnormalised, pins.test_merge_independent_of_slice_count),
    ("request_rows", _rows_ignore_table, lambda: pins.test_scores_brute_force((257, 200))),
    ("side_cache", _side_slot_shift, lambda: side_pins.test_side_cache_brute_force((5, 70))),
    ("append_token", _append_whole_block, lambda: side_pins.test_append_reproduces_full_caches((6, 130))),
    ("append_token", _append_new_row_only, lambda: side_pins.test_append_reproduces_full_caches((7, 64))),
    ("bf16_to_f64", _bf16_as_fp16, pins.test_bf16_decoding_every_bit_pattern),
    ("bf16_to_f64", _bf16_shift8, pins.test_bf16_decoding_every_bit_pattern),
    ("bf16_to_f64", _bf16_as_fp16, pins.test_bf16_decoding_hand_values),
    ("bf16_to_f64", _bf16_shift8, pins.test_bf16_decoding_hand_values),
    ("bf16_to_f64", _bf16_as_fp16, lambda: pins.test_short_context_equals_dense_attention(100)),
    ("bf16_to_f64", _bf16_shift8, lambda: pins.test_short_context_equals_dense_attention(5)),
    ("draft_length", _draft_one_short, lambda: multi_pins.test_last_draft_token_sees_the_whole_context(2)),
    ("draft_length", _draft_sees_all, lambda: multi_pins.test_draft_tokens_are_causal(2)),
]


@pytest.mark.parametrize("name,bad,pin", MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_pin_catches_planted_mistake(monkeypatch, name, bad, pin):
    pin()                                   # passes on the real oracle
    _patch(monkeypatch, name, bad)
    with pytest.raises(AssertionError):
        pin()

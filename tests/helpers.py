"""Glue between the input generator and the CPU oracle (no arithmetic of the method)."""
import numpy as np

from sparse_attention_decode_qsa_amd.inputs import bf16_bits


def oracle_arrays(x):
    """Host numpy views of a DecodeInputs batch, bf16 tensors as raw bits."""
    return dict(
        q=bf16_bits(x.q),
        q_idx=x.q_idx.cpu().numpy(),
        idx_cache=x.idx_cache.cpu().numpy(),
        k_cache=bf16_bits(x.k_cache),
        v_cache=bf16_bits(x.v_cache),
        page_table=x.page_table.cpu().numpy(),
        lengths=list(x.lengths),
    )


def oracle_decode(oracle, x, P=None, k=512):
    a = oracle_arrays(x)
    P = x.workload.slices if P is None else P
    return oracle.decode(a["q"], a["q_idx"], a["idx_cache"], a["k_cache"], a["v_cache"],
                         a["page_table"], a["lengths"], P, x.scale, k)


# The parity bar for floating-point results against the float64 oracle: a maximum absolute
# error of 2e-3 and, separately, a maximum relative error of 1e-2. The relative error is taken
# over elements with |oracle| >= REL_FLOOR: below that an fp32 result's relative error is set
# by absolute rounding (~1e-7 here) and says nothing about the method.
ATOL, RTOL, REL_FLOOR = 2e-3, 1e-2, 1e-3


def tolerance_report(got, ref, atol=ATOL, rtol=RTOL, floor=REL_FLOOR):
    """Two separate bounds: max |g - r| <= atol over every element, and max |g - r| / |r| <= rtol
    over the elements with |r| >= floor; every result must be finite.

    Returns (ok, max_abs, max_rel)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return True, 0.0, 0.0
    err = np.abs(got - ref)
    big = np.abs(ref) >= floor
    max_abs = float(err.max())
    max_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    ok = bool(np.all(np.isfinite(got)) and max_abs <= atol and max_rel <= rtol)
    return ok, max_abs, max_rel

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


def tolerance_report(got, ref, atol=2e-3, rtol=1e-2):
    """Element-wise |g - r| <= atol + rtol*|r|; returns (ok, max_abs, max_rel_over_big)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    ok = bool(np.all(err <= atol + rtol * np.abs(ref)) and np.all(np.isfinite(got)))
    big = np.abs(ref) >= atol / rtol
    max_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    return ok, float(err.max()) if err.size else 0.0, max_rel

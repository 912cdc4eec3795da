#!/usr/bin/env python3
"""Throughput of the QSA decode path on one MI355X.

One step = one call of the whole path (indexer scan + pooling + scores -> top-512
selection -> paged gather + attention per slice -> LSE merge) for one decode token of
every request of the batch, launched as qsa_decode on one stream. Inputs are resident
in HBM before timing starts. Default workload: w4, the 256K-context batch (B=4, lengths
uniform in [65536, 262144] drawn with seed 0, Hq/Hkv=32/4, head_dim 128, shuffled 64-token
pages, P=4 slices).

Prints one JSON line. `value` is decode calls/s; it also reports per-call latency
percentiles, the algorithmic GB/s of the whole call, measured device copy and read ceilings, a
roofline entry for the dominant kernel (the indexer scan, timed on its own with HIP events on
the stream it runs on) and the CPU oracle's rate on the same workload.

    python bench.py [--steps K] [--warmup W] [--workload w4] [--sets R] [--no-cpu-baseline]
                    [--graph] [--copy-calibration MIB]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QSA decode attn calls/s and achieved HBM GB/s (% peak) at 256K ctx, 1 GPU"
HBM_PEAK_GBS = 8000.0
IDX_TOKEN_BYTES = 256


def algorithmic_bytes(lengths, hq, hkv, k=512):
    """Bytes the method must move per call (intermediates excluded).

    per request: 256*L (indexer keys) + 256 (q_idx) + 4*ceil(L/64) (page table)
                 + |T|*Hkv*512 (kept K and V rows) + 256*Hq (q, bf16) + 512*Hq (out, fp32)
    with |T| = number of kept token positions.
    """
    total = 0
    for L in lengths:
        nblk = (L + 3) // 4
        K = min(k, nblk)
        T = min(4 * K, L)                 # exact when the tail block is kept; <= 3 high otherwise
        total += IDX_TOKEN_BYTES * L + 256 + 4 * ((L + 63) // 64) + T * hkv * 512 + 256 * hq + 512 * hq
    return total


def index_bytes(lengths):
    """Algorithmic bytes of the indexer scan: keys + q_idx + page table + block scores written."""
    return sum(IDX_TOKEN_BYTES * L + 256 + 4 * ((L + 63) // 64) + 4 * ((L + 3) // 4) for L in lengths)


def default_sets(lengths, hkv, draft=1, k=512, max_sets=64, max_bytes=96 << 30):
    """Rotated input sets for a timed window that no cache can shorten.

    The scan's nontemporal loads do not displace what sits in the 256 MB MALL, so a set's
    kept K/V rows (16.8 MB per call at the 256K batch) would still be there when the rotation
    comes back to it after a few sets; in a model with many layers nothing of one layer's K/V
    survives until its next step. So one rotation must both stream >= 1 GiB of indexer keys and
    gather >= 512 MiB of distinct K/V rows. Capped at max_sets and at max_bytes of inputs.
    """
    idx = IDX_TOKEN_BYTES * sum(lengths)
    kept = draft * sum(min(4 * k, L) for L in lengths) * hkv * 512
    per_set = idx + sum(lengths) * hkv * 512           # indexer keys + K and V caches
    n = max(math.ceil((1 << 30) / max(idx, 1)), math.ceil((512 << 20) / max(kept, 1)))
    return max(1, min(n, max_sets, max(1, max_bytes // max(per_set, 1))))


def kept_tokens_exact(sel, lengths):
    """|T_b| from the kept block ids (tail block counted with its valid tokens only)."""
    import numpy as np
    total = 0
    for b, L in enumerate(lengths):
        s = sel[b][sel[b] >= 0]
        toks = (s[:, None] * 4 + np.arange(4)[None]).reshape(-1)
        total += int((toks < L).sum())
    return total


def mq_roofline(scan_ops, k1_bytes, ms_k1, D):
    """Roofline of the many-query scan: an int8 contraction (2*256 operations per query and
    visible token, against 5.0 POP/s dense int8) that also reads the keys and writes every
    query's block scores (bytes against HBM). The bound is the side with the longer time at
    peak; achieved, peak, unit and frac are given for it, the other side as extra fields."""
    t = ms_k1 * 1e-3
    tops, gbs = scan_ops / t / 1e12, k1_bytes / t / 1e9
    mfma = {"achieved": round(tops, 1), "peak": 5000.0, "unit": "TOP/s (int8 dense)", "frac": round(tops / 5000.0, 4)}
    hbm = {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
    bound = "mfma" if scan_ops / 5.0e15 > k1_bytes / (HBM_PEAK_GBS * 1e9) else "hbm"
    main, other = (mfma, hbm) if bound == "mfma" else (hbm, mfma)
    r = {"kernel": f"index_score_mq_kernel (T={D} queries per request: int8 MFMA 16x16x64 scan)", "bound": bound}
    r.update(main)
    r.update({"traffic": None, "avg_launch_us": round(ms_k1 * 1000, 3), "ops_per_launch": scan_ops,
              "bytes_per_launch": k1_bytes,
              ("hbm" if bound == "mfma" else "mfma") + "_side": other})
    return r


_CPU_BATCH = {}


def _host_cpu():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def _oracle_calls(budget_s):
    """Whole-batch oracle calls on one host thread for about budget_s seconds: (calls, seconds)."""
    from threadpoolctl import threadpool_limits
    import oracle
    a = _CPU_BATCH
    calls, t_total = 0, 0.0
    with threadpool_limits(limits=1):
        while t_total < budget_s:
            t0 = time.perf_counter()
            oracle.decode(a["q"], a["q_idx"], a["idx"], a["k"], a["v"], a["pt"], a["lengths"], a["P"], a["scale"])
            t_total += time.perf_counter() - t0
            calls += 1
    return calls, t_total


def cpu_baseline(wl, seed, budget_s=12.0):
    """The CPU oracle, as it stands, on a batch of the benchmarked workload drawn on the host
    (the same lengths, shapes and value laws as the GPU's input sets), run before anything
    touches the GPU: first on one host thread, then in one forked worker process per host core
    available to this process, each on one thread, all calling the oracle on the whole batch."""
    import multiprocessing as mp
    import torch
    from sparse_attention_decode_qsa_amd.inputs import bf16_bits, make_inputs

    x = make_inputs(wl, seed, "cpu")
    _CPU_BATCH.update(q=bf16_bits(x.q), q_idx=x.q_idx.numpy(), idx=x.idx_cache.numpy(), k=bf16_bits(x.k_cache),
                      v=bf16_bits(x.v_cache), pt=x.page_table.numpy(), lengths=list(x.lengths),
                      P=x.workload.slices, scale=x.scale)
    del x
    torch.set_num_threads(1)
    calls1, t1 = _oracle_calls(budget_s)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as pool:
        per = pool.map(_oracle_calls, [budget_s] * cores)
    wall = time.perf_counter() - t0
    rate_all = sum(c / t for c, t in per)
    model = _host_cpu()
    return {"value": rate_all, "unit": "calls/s", "cores": cores, "kind": "oracle",
            "sample": f"the benchmarked workload's batch drawn on the host (same lengths and shapes as the GPU "
                      f"sets; all {len(_CPU_BATCH['lengths'])} requests per call), numpy float64/int64: "
                      f"{cores} worker processes of one thread each on {model}, "
                      f"{sum(c for c, _ in per)} whole calls in {wall:.1f} s",
            "one_core": {"value": calls1 / t1, "unit": "calls/s", "cores": 1,
                         "sample": f"{calls1} whole calls on one thread in {t1:.1f} s"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="w4")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sets", type=int, default=0,
                    help="rotated input sets (0: enough that one rotation streams >= 1 GiB of indexer keys "
                         "and gathers >= 512 MiB of distinct K/V rows, so the 256 MB MALL serves no repeat)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each call from a HIP graph captured once per input set")
    ap.add_argument("--pooled", action="store_true",
                    help="the side-cache variant: each call writes the step's token into the caches (side "
                         "cache included) and decodes with a scan that reads the pooled int16 keys instead "
                         "of the int8 keys (qsa_decode_step_pooled)")
    ap.add_argument("--separate-append", action="store_true",
                    help="with --pooled: make the step's cache writes with qsa_cache_append before "
                         "qsa_decode_pooled instead of inside the scan (qsa_decode_step_pooled)")
    ap.add_argument("--draft", type=int, default=1, metavar="T",
                    help="multi-token decode: T new tokens per request (qsa_decode_multi; drafts for T <= 4, "
                         "a prefill chunk beyond); a call then decodes B*T tokens")
    ap.add_argument("--spread", type=int, default=None, metavar="D",
                    help="with --draft T: correlated chunk queries, each new token's indexer query = the "
                         "request's query + a uniform offset in {-D..D} per element (default: independent "
                         "queries), so that neighbouring tokens keep overlapping blocks")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run 3 copies of MIB MiB each with qsa_calib_copy (the scan's "
                         "kind of loads and stores), so that hardware byte counters can be scaled "
                         "against a kernel of known traffic")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_decode_qsa_amd import qsa
    from sparse_attention_decode_qsa_amd.inputs import WORKLOADS, draft_queries, draw_lengths, make_inputs

    w = WORKLOADS[args.workload]
    lengths = draw_lengths(w, args.seed)
    wl = w.with_(lengths=("list",) + tuple(lengths))   # every rotated set keeps seed-0 lengths
    sets = args.sets or default_sets(lengths, w.hkv, args.draft)

    cpu = None
    if not args.no_cpu_baseline and args.draft == 1:
        # before anything touches the GPU, so that the forked workers carry no GPU state
        print("# timing the CPU oracle on the same workload", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.seed)
    elif not args.no_cpu_baseline:
        print("# no CPU baseline with several new tokens per request (the oracle would take minutes per call)",
              file=sys.stderr, flush=True)

    torch.cuda.init()
    dev = torch.device("cuda:0")
    plans, inputs, appends, pooled = [], [], [], []
    for r in range(sets):
        x = make_inputs(wl, args.seed + 1000 * r, dev)
        inputs.append(x)
        side = None
        if args.pooled and args.draft > 1:
            if args.draft > 4:
                raise SystemExit("--pooled takes at most 4 draft tokens (--draft 1..4)")
            side = qsa.pool_build(x.idx_cache, x.page_table, x.context_lens)   # pools the draft rows too
            pooled.append(side)
        elif args.pooled:
            # the side cache as prefill leaves it, and the step's new rows = the rows at L-1 (so
            # every call rewrites the same values and the inputs stay fixed)
            side = qsa.pool_build(x.idx_cache, x.page_table, x.context_lens)
            pt = x.page_table.cpu()
            pages = torch.tensor([int(pt[b, (L - 1) // 64]) for b, L in enumerate(lengths)], device=dev)
            rows = torch.tensor([(L - 1) % 64 for L in lengths], device=dev)
            k_new, v_new = x.k_cache[pages, rows].contiguous(), x.v_cache[pages, rows].contiguous()
            i_new = x.idx_cache[pages, rows].contiguous()
            if args.separate_append:
                appends.append(qsa.AppendPlan(k_new, v_new, i_new, x.k_cache, x.v_cache, x.idx_cache,
                                              x.page_table, x.context_lens, pooled=side))
            pooled.append(side)
        if args.pooled and args.draft == 1 and not args.separate_append:
            plans.append(qsa.StepPlan(k_new, v_new, i_new, x.q, x.q_idx, x.idx_cache, x.k_cache, x.v_cache,
                                      x.page_table, x.context_lens, side, w.slices))
        elif args.draft > 1:
            dq, dqi = draft_queries(x, args.draft, args.seed + 1000 * r, spread=args.spread)
            plans.append(qsa.MultiDecodePlan(dq, dqi, x.idx_cache, x.k_cache, x.v_cache, x.page_table,
                                             x.context_lens, w.slices, pooled=side))
        else:
            plans.append(qsa.DecodePlan(x.q, x.q_idx, x.idx_cache, x.k_cache, x.v_cache, x.page_table,
                                        x.context_lens, w.slices, pooled=side))
    torch.cuda.synchronize()
    print(f"# workload {args.workload}: B={len(lengths)} lengths={lengths[:8]}{'...' if len(lengths) > 8 else ''} "
          f"sets={sets}", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    # ---- whole path
    def step(i):
        if appends:
            appends[i % sets].run()
        plans[i % sets].run()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.graph:
        for r in range(sets):              # every set run eagerly once (the warm-up may cover fewer)
            step(r)
        torch.cuda.synchronize()
        ref = [(p.sel.clone(), p.out.clone()) for p in plans]
        graphs = []
        for r in range(sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r)
            graphs.append(g)
        for r, g in enumerate(graphs):     # a replay must reproduce the eager call bit for bit
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(plans[r].sel, ref[r][0]) and torch.equal(plans[r].out.view(torch.int32),
                                                                        ref[r][1].view(torch.int32))
        step = lambda i: graphs[i % sets].replay()
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # ---- per-call latency (event pair around each call; a separate pass so the events do not
    # touch the headline timing)
    n_lat = min(args.steps, 200)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_lat)]
    for i, (a, b) in enumerate(pairs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    lat = sorted(a.elapsed_time(b) * 1000.0 for a, b in pairs)
    pct = lambda q: round(lat[min(len(lat) - 1, int(q * len(lat)))], 2)

    # ---- the dominant kernel (indexer scan), timed inside the chain: qsa_time_next_scan makes
    # the scan launched by the next qsa_decode call record a pair of events at the kernel's own
    # start and end (kernel timestamps, as a kernel trace takes them; no marker packets in the
    # chain), on the stream it runs on. Every call of this pass is a whole qsa_decode call.
    k_iters = max(args.steps, 100)
    # int8 or side-cache scan inside whole calls (draft tokens on the side cache too: that scan has
    # no entry point of its own)
    in_call_timing = (args.draft == 1 or args.pooled) and not args.graph
    if in_call_timing:
        marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k_iters)]
        for a, b in marks:               # torch creates an event at its first record
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        for i in range(10):
            step(i)
        for i, (a, b) in enumerate(marks):
            qsa.time_next_scan(a, b)
            step(i)
        torch.cuda.synchronize()
        ms_k1 = sum(a.elapsed_time(b) for a, b in marks) / k_iters

    def scan(i):
        x = inputs[i % sets]
        if args.draft > 1:
            qsa.index_score_multi(plans[i % sets].inputs[1], x.idx_cache, x.page_table, x.context_lens,
                                  out=plans[i % sets].scores)
        elif args.pooled:
            qsa.index_score_pooled(x.q_idx, pooled[i % sets], x.page_table, x.context_lens, out=plans[i % sets].scores)
        else:
            qsa.index_score(x.q_idx, x.idx_cache, x.page_table, x.context_lens, out=plans[i % sets].scores)

    if not in_call_timing:   # other modes: the scan alone, back to back, same stream and inputs
        for i in range(10):
            scan(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(k_iters):
            scan(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_k1 = e0.elapsed_time(e1) / k_iters

    # ---- measured device ceilings, same stream: qsa_calib_copy of 1 GiB (read + write) and
    # qsa_calib_read of 1 GiB (the scan's kind of loads, read only)
    from sparse_attention_decode_qsa_amd import calib
    csrc_t = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    cdst_t = torch.empty_like(csrc_t)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def _rate(fn, nbytes, reps=5):
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9

    copy_gbs = _rate(lambda: calib.copy(cdst_t, csrc_t), 2 << 30)
    read_gbs = _rate(lambda: calib.read(csrc_t, sink), 1 << 30)
    del csrc_t, cdst_t

    sel = plans[0].sel.cpu().numpy()
    D = args.draft
    # per (request, draft token) the context length it sees
    vlens = [max(0, L - (D - 1 - t)) for L in lengths for t in range(D)]
    T_exact = kept_tokens_exact(sel, vlens)
    algo = algorithmic_bytes(lengths, w.hq, w.hkv)
    # the indexer keys are read once for all draft tokens; kept K/V rows, q and the output
    # count per (request, draft token): replace the single-token |T| bound by the exact count
    algo += (D - 1) * sum(256 * (w.hq + 1) + 512 * w.hq for _ in lengths)
    algo += T_exact * w.hkv * 512 - sum(min(4 * min(512, (L + 3) // 4), L) for L in lengths) * w.hkv * 512
    k1_bytes = index_bytes(lengths) + (D - 1) * sum(256 + 4 * ((L + 3) // 4) for L in lengths)
    if args.pooled:
        # the scan reads 512 B per block instead of 256 B per token (with draft tokens, the one or
        # two pages holding draft positions are read as int8 rows instead: traffic, not counted
        # here); the single-token step's append writes the K/V rows (2*Hkv*256 B), the indexer
        # row (256 B) and one side-cache entry (512 B) per request and reads up to 3 earlier
        # indexer rows
        pooled_keys = sum(512 * ((L + 3) // 4) for L in lengths)
        algo += pooled_keys - IDX_TOKEN_BYTES * sum(lengths)
        if D == 1:
            algo += sum(2 * w.hkv * 256 + 256 + 512 + 256 * ((L - 1) % 4) for L in lengths if L)
        k1_bytes += pooled_keys - IDX_TOKEN_BYTES * sum(lengths)
    gbs = algo / (ms_step * 1e-3) / 1e9
    # With more than 4 new tokens per request the scan is an int8 matrix product on the matrix
    # cores: 2*256 operations per (query, visible token); it also writes every query's block
    # scores. Its roofline is the larger of the two times at peak.
    scan_ops = 2 * 256 * sum(vlens) if D > 4 else 0
    k1_gbs = k1_bytes / (ms_k1 * 1e-3) / 1e9

    # HBM bytes per launch of the scan from the committed counter runs, while the scan's
    # sources are the ones those runs measured (same workload); otherwise unknown.
    from sparse_attention_decode_qsa_amd import profiling
    tr = profiling.read_traffic(os.path.join(ROOT, "profiles", f"index_score_{args.workload}_traffic.md"))
    traffic = (tr["traffic_bytes"] if tr and tr.get("source_hash") == profiling.scan_source_hash() and not args.pooled
               and args.draft == 1 else None)

    result = {
        "metric": METRIC,
        "value": round(1000.0 / ms_step, 2),
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: B={len(lengths)}, L={lengths}, Hq/Hkv={w.hq}/{w.hkv}, head_dim=128, "
                        f"indexer 4x64 int8, page=64 shuffled, top-512 blocks of 4, P={w.slices}, seed {args.seed}",
            "global_batch": len(lengths),
            "seq_len": max(lengths),
            "parallelism": f"1 GPU, P={w.slices} slices merged by LSE",
            "rotated_input_sets": sets,
            "launch": ("hip graph replay" if args.graph else "stream launches") +
                      (f" (qsa_decode_multi_pooled, T={D}, per call)" if args.pooled and D > 1 else
                       (" (qsa_cache_append + qsa_decode_pooled per call)" if args.separate_append else
                        " (qsa_decode_step_pooled: cache writes in the scan, per call)") if args.pooled else
                       f" (qsa_decode_multi, T={D}, per call)" if D > 1 else " (qsa_decode per call)"),
            "indexer_keys": "pooled int16 side cache" if args.pooled else "int8 per token, pooled in the scan",
            "draft_tokens_per_request": D,
            "chunk_query_spread": args.spread if D > 1 else None,
            "tokens_per_s": round(1000.0 / ms_step * len(lengths) * D, 1),
        },
        "call_us": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9), "calls": n_lat},
        "achieved_GBps": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "copy_ceiling_GBps": round(copy_gbs, 1),
        "read_ceiling_GBps": round(read_gbs, 1),
        "algorithmic_bytes_per_call": algo,
        "roofline": (mq_roofline(scan_ops, k1_bytes, ms_k1, D) if D > 4 else {
            "kernel": (f"index_score_pooled_multi_kernel<T={D}> (side-cache scan + scores of {D} draft tokens)"
                       if args.pooled and D > 1
                       else "index_score_pooled_kernel (side-cache scan + scores)" if args.pooled
                       else f"index_score_kernel<T={D}> (indexer scan + pooling + scores of {D} draft tokens)"
                       if D > 1 else "index_score_kernel (indexer scan + pooling + scores)"),
            "bound": "hbm",
            "achieved": round(k1_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "frac_of_read_ceiling": round(k1_gbs / read_gbs, 4),
            "avg_launch_us": round(ms_k1 * 1000, 3),
            "bytes_per_launch": k1_bytes,
            "timing": (("inside whole qsa_decode_multi_pooled calls" if args.pooled and D > 1
                        else "inside whole qsa_decode_step_pooled calls" if args.pooled else "inside whole qsa_decode calls")
                       + ": events recorded at the scan kernel's own start and end (qsa_time_next_scan)"
                       if in_call_timing else "the scan alone, back to back"),
        }),
    }
    if args.copy_calibration:
        from sparse_attention_decode_qsa_amd import calib
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            calib.copy(dst, src)
        torch.cuda.synchronize()
        assert torch.equal(dst, src)
        print(f"# copy calibration: 3 copies of {n} bytes (read {n}, write {n} each)", file=sys.stderr, flush=True)
    if cpu is not None:
        # the oracle's effective rate over the same algorithmic bytes per call
        cpu["GBps"] = round(cpu["value"] * algo / 1e9, 3)
        cpu["one_core"]["GBps"] = round(cpu["one_core"]["value"] * algo / 1e9, 4)
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

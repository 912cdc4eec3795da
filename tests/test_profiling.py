"""The counter arithmetic behind the bench's traffic figure, on synthetic rocprofv3 CSV rows."""
import csv

from sparse_attention_decode_qsa_amd import profiling

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow(dict(Dispatch_Id=i, Kernel_Name=k, Counter_Name=c, Counter_Value=v))


def test_traffic_scaling(tmp_path):
    scan = "void qsa::index_score_kernel<16>(signed char const*, ...)"
    cal = "qsa_calib::calib_copy_kernel(int __vector(4)*, int __vector(4) const*, unsigned long)"
    other = "void at::native::vectorized_elementwise_kernel<4, ...>"
    mib = 1 << 20
    # the copy moves 1 MiB each way; its counters read half the reads and all the writes
    _csv(tmp_path / "f.csv", [(cal, "FETCH_SIZE", 512.0), (cal, "FETCH_SIZE", 512.0), (scan, "FETCH_SIZE", 100.0),
                              (scan, "FETCH_SIZE", 300.0), (other, "FETCH_SIZE", 9e9)])
    _csv(tmp_path / "w.csv", [(cal, "WRITE_SIZE", 1024.0), (scan, "WRITE_SIZE", 10.0), (other, "WRITE_SIZE", 7.0)])
    r = profiling.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), mib)
    assert r["read_factor"] == 0.5 and r["write_factor"] == 1.0
    assert r["read_bytes"] == 200 * 1024 * 2          # mean 200 KiB counted, 2 bytes per counted byte
    assert r["write_bytes"] == 10 * 1024
    assert r["traffic_bytes"] == r["read_bytes"] + r["write_bytes"]
    out = tmp_path / "t.md"
    profiling.write_traffic(r, "cmd f", "cmd w", str(out), "title", algorithmic_bytes=409600)
    back = profiling.read_traffic(str(out))
    assert back == r and back["source_hash"] == profiling.scan_source_hash()
    assert profiling.read_traffic(str(tmp_path / "missing.md")) is None


def test_chain_timeline_medians(tmp_path):
    """The per-call timeline: calls are found as scan, selection, attention, merge in a row;
    other kernels in between break a call; offsets are from each call's scan start."""
    names = ["void qsa::index_score_kernel<16, 1>(...)", "void qsa::topk_select_kernel<1>(...)",
             "qsa::sparse_attn_kernel(...)", "qsa::slice_merge_kernel(...)"]
    rows, t = [], 1000
    for call in range(5):
        durs = [30 + call, 9, 10, 4]                      # us
        for n, d in zip(names, durs):
            rows.append((n, t, t + d * 1000))
            t += d * 1000 + 100                           # 0.1 us gap after each kernel
        t += 5000
    scan1_end = rows[4][2]                                # call 1's scan
    rows.append(("qsa::lse_merge_kernel(...)", scan1_end + 10, scan1_end + 20))   # breaks call 1
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for n, a, b in sorted(rows, key=lambda r: r[1]):
            w.writerow(dict(Kernel_Name=n, Start_Timestamp=a, End_Timestamp=b))
    tl = profiling.chain_timeline(str(path), skip=0)
    assert [r["kernel"] for r in tl] == ["qsa::index_score_kernel<16, 1>", "qsa::topk_select_kernel<1>",
                                         "qsa::sparse_attn_kernel", "qsa::slice_merge_kernel"]
    assert tl[0]["calls"] == 4
    assert tl[0]["start_us"] == 0.0 and tl[1]["dur_us"] == 9.0 and tl[3]["dur_us"] == 4.0
    assert abs(tl[1]["start_us"] - (tl[0]["dur_us"] + 0.1)) < 1e-9

"""A C program, not Python, drives the library: tests/c/decode_from_c.c allocates with the HIP
runtime, fills a small paged batch on the host, calls qsa_decode and qsa_decode_multi and
dumps inputs and results. The CPU test checks that it compiles and links with gcc against include/qsa.h; the
GPU test runs it and compares every result with the oracle on the inputs it wrote."""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import oracle
from tests.helpers import ATOL, RTOL, tolerance_report

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_decode_qsa_amd")
SRC = os.path.join(ROOT, "tests", "c", "decode_from_c.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    if not os.path.exists(os.path.join(PKG, "libqsa.so")):
        pytest.skip("libqsa.so not built")
    if not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("no HIP runtime headers")
    exe = tmp_path / "decode_from_c"
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-O2", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
                        "-o", str(exe), "-L", PKG, "-lqsa", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                        "-lm", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program_builds(tmp_path):
    _build(tmp_path)


def _load(d, name, dtype, shape):
    return np.fromfile(os.path.join(d, name), dtype=dtype).reshape(shape)


@pytest.mark.gpu
def test_c_program_decode_matches_oracle(tmp_path):
    exe = _build(tmp_path)
    out_dir = tmp_path / "out"
    out_dir.mkdir()
    print("running the C program", flush=True)
    r = subprocess.run([str(exe), str(out_dir)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok ok"
    meta = [int(v) for v in (out_dir / "meta.txt").read_text().split()]
    B, Hq, Hkv, P, NP, max_pages, max_blocks, k, TD = meta[:9]
    lens = meta[9:9 + B]
    D, page = 128, 64
    d = str(out_dir)
    q = _load(d, "q.bin", np.uint16, (B, Hq, D))
    qi = _load(d, "q_idx.bin", np.int8, (B, 4, 64))
    idx = _load(d, "idx_cache.bin", np.int8, (NP, page, 4, 64))
    kc = _load(d, "k_cache.bin", np.uint16, (NP, page, Hkv, D))
    vc = _load(d, "v_cache.bin", np.uint16, (NP, page, Hkv, D))
    pt = _load(d, "page_table.bin", np.int32, (B, max_pages))
    g = dict(scores=_load(d, "scores.bin", np.int32, (B, max_blocks)),
             sel=_load(d, "sel.bin", np.int32, (B, k)),
             cnt=_load(d, "sel_count.bin", np.int32, (B,)),
             po=_load(d, "partial_out.bin", np.float32, (B, P, Hq, D)),
             pl=_load(d, "partial_lse.bin", np.float32, (B, P, Hq)),
             out=_load(d, "out.bin", np.float32, (B, Hq, D)),
             lse=_load(d, "out_lse.bin", np.float32, (B, Hq)))
    scale = 1.0 / np.sqrt(np.float32(D))
    for b, L in enumerate(lens):
        ref = oracle.decode_request(q[b], qi[b], idx, kc, vc, pt[b], L, P, float(scale), k)
        nblk = (L + 3) // 4
        assert np.array_equal(g["scores"][b, :nblk], ref["scores"]), f"scores differ (b={b})"
        K = len(ref["kept"])
        assert g["cnt"][b] == K
        assert np.array_equal(g["sel"][b, :K], ref["kept"]), f"kept blocks differ (b={b})"
        assert np.all(g["sel"][b, K:] == -1)
        for name, got, want in (("partial_out", g["po"][b], ref["o_part"]), ("out", g["out"][b], ref["out"])):
            ok, ma, mr = tolerance_report(got, want, ATOL, RTOL)
            assert ok, f"{name} outside tolerance (b={b}, max abs {ma:.3g}, max rel {mr:.3g})"
        for name, got, want in (("partial_lse", g["pl"][b], ref["lse_part"]), ("lse", g["lse"][b], ref["lse"])):
            fin = np.isfinite(want)
            assert np.array_equal(np.isfinite(got), fin), f"{name}: -inf pattern differs (b={b})"
            ok, ma, mr = tolerance_report(got[fin], want[fin], ATOL, RTOL)
            assert ok, f"{name} outside tolerance (b={b}, max abs {ma:.3g}, max rel {mr:.3g})"
        print(f"request {b} L={L}: kept {K} blocks, parity ok", flush=True)
    # the multi-token call: TD new tokens per request, each decoded at its own length
    mq = _load(d, "m_q.bin", np.uint16, (B, TD, Hq, D))
    mqi = _load(d, "m_q_idx.bin", np.int8, (B, TD, 4, 64))
    ms = _load(d, "m_scores.bin", np.int32, (B * TD, max_blocks))
    msel = _load(d, "m_sel.bin", np.int32, (B * TD, k))
    mcnt = _load(d, "m_sel_count.bin", np.int32, (B * TD,))
    mout = _load(d, "m_out.bin", np.float32, (B * TD, Hq, D))
    refs = oracle.decode_multi(mq, mqi, idx, kc, vc, pt, lens, TD, P, float(scale), k)
    for b, L in enumerate(lens):
        for t in range(TD):
            r, ref = b * TD + t, refs[b * TD + t]
            Lt = oracle.draft_length(L, TD, t)
            assert np.array_equal(ms[r, :(Lt + 3) // 4], ref["scores"]), f"multi scores (b={b}, t={t})"
            K = len(ref["kept"])
            assert mcnt[r] == K and np.array_equal(msel[r, :K], ref["kept"]) and np.all(msel[r, K:] == -1)
            ok, ma, mr = tolerance_report(mout[r], ref["out"], ATOL, RTOL)
            assert ok, f"multi out outside tolerance (b={b}, t={t}, max abs {ma:.3g}, max rel {mr:.3g})"
    print(f"multi-token call ({TD} tokens per request): parity ok", flush=True)
    sys.stdout.flush()

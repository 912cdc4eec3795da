"""The C ABI on the CPU: the library loads, exports what include/qsa.h declares, and its
host-side argument checks return their documented codes before anything is enqueued."""
import ctypes
import os
import re

import pytest

from sparse_attention_decode_qsa_amd import qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")
OK, NULL, SHAPE, UNSUP, WS = 0, 1, 2, 3, 4
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails a host check


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(qsa.SIGNATURES)


def test_library_exports_every_declared_symbol():
    L = qsa.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name


def test_status_strings_and_version():
    L = qsa.lib()
    for s in range(7):
        assert L.qsa_status_string(s) and L.qsa_status_string(s) != b"unknown status"
    assert L.qsa_status_string(99) == b"unknown status"
    assert L.qsa_version() >= 100
    assert L.qsa_last_hip_error() == 0


def _index(L, **kw):
    a = dict(q_idx=FAKE, idx=FAKE, pt=FAKE, lens=FAKE, B=2, nh=4, dim=64, ps=64, mp=16, mb=256, out=FAKE)
    a.update(kw)
    return L.qsa_index_score(a["q_idx"], a["idx"], a["pt"], a["lens"], a["B"], a["nh"], a["dim"], a["ps"],
                             a["mp"], a["mb"], a["out"], None, None)


def test_index_score_checks():
    L = qsa.lib()
    assert _index(L, B=0) == OK
    assert _index(L, q_idx=None) == NULL
    assert _index(L, out=None) == NULL
    assert _index(L, B=-1) == SHAPE
    assert _index(L, mb=255) == SHAPE            # rows must hold every block of a full table
    assert _index(L, nh=8) == UNSUP
    assert _index(L, dim=128) == UNSUP
    assert _index(L, ps=32) == UNSUP
    assert _index(L, idx=ctypes.c_void_p(0x1001)) == SHAPE   # 16-byte alignment
    assert _index(L, B=65536) == UNSUP


def test_topk_checks():
    L = qsa.lib()

    def f(scores=FAKE, lens=FAKE, pm=None, B=2, mb=100, mp=7, k=512, sel=FAKE, cnt=FAKE):
        return L.qsa_topk_select(scores, lens, pm, B, mb, mp, k, sel, cnt, None, 0, None)

    assert f(B=0) == OK
    assert f(scores=None) == NULL
    assert f(sel=None) == NULL
    assert f(k=0) == SHAPE
    assert f(B=-1) == SHAPE
    assert f(k=513) == UNSUP
    assert f(mb=262148) == UNSUP                         # > 1M-token contexts
    assert f(mb=102) == SHAPE                            # rows of 4-block vectors
    assert f(scores=ctypes.c_void_p(0x1004)) == SHAPE    # 16-byte alignment
    assert f(pm=FAKE, mp=0) == SHAPE                     # page maxima need their row stride
    assert f(pm=FAKE, mp=5) == SHAPE                     # 16*5 < 100 - 15: rows not covered
    assert L.qsa_topk_workspace_size(2, 100, 512) == 0   # one workgroup per request, no scratch


def _attn(L, **kw):
    a = dict(B=2, Hq=32, Hkv=4, D=128, ps=64, mp=16, k=512, P=4, ws=FAKE, nbytes=1 << 30, q=FAKE, po=FAKE)
    a.update(kw)
    return L.qsa_sparse_attn_decode(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["B"], a["Hq"], a["Hkv"],
                                    a["D"], a["ps"], a["mp"], a["k"], a["P"], 0.1, a["po"], FAKE, a["ws"],
                                    a["nbytes"], None)


def test_attention_checks():
    L = qsa.lib()
    assert _attn(L, B=0) == OK
    assert _attn(L, q=None) == NULL
    assert _attn(L, po=None) == NULL
    assert _attn(L, Hq=30) == SHAPE               # Hq % Hkv
    assert _attn(L, P=0) == SHAPE
    assert _attn(L, P=65) == UNSUP
    assert _attn(L, Hq=68, Hkv=4) == UNSUP         # group of 17 > 16 MFMA rows
    assert _attn(L, D=64) == UNSUP
    assert _attn(L, k=600) == UNSUP
    assert _attn(L, ws=None, nbytes=0) == WS       # the share partials need a workspace
    assert _attn(L, nbytes=attn_ws(2, 32, 4, 4) - 1) == WS
    # share partials of C shares per slice
    assert [attn_split(B, 4, 4) for B in (1, 2, 3, 5, 8, 16, 32, 128)] == [32, 16, 8, 4, 4, 2, 1, 1]
    assert attn_split(1, 2, 1) == 32 and attn_split(4, 4, 4) == 8     # one small request; w4
    assert L.qsa_attn_workspace_size(2, 32, 4, 512, 4) == attn_ws(2, 32, 4, 4)
    assert L.qsa_attn_workspace_size(128, 32, 4, 512, 4) == attn_ws(128, 32, 4, 4) == 0   # C = 1
    assert L.qsa_attn_workspace_size(0, 32, 4, 512, 4) == 0


def align256(n):
    return (n + 255) // 256 * 256


def attn_split(B, Hkv, P):
    """Shares per slice: largest power of two <= min(32, ceil(512 / (B*Hkv*P))), at least 1."""
    want = min(32, -(-512 // (B * Hkv * P)))
    c = 1
    while 2 * c <= want:
        c *= 2
    return c


def attn_ws(B, Hq, Hkv, P):
    C = attn_split(B, Hkv, P)
    if C == 1:
        return 0              # one share per slice: the slice partials are written directly
    return align256(B * P * C * Hq * 128 * 4) + align256(B * P * C * Hq * 4)


def test_merge_and_decode_checks():
    L = qsa.lib()
    m = L.qsa_lse_merge
    assert m(FAKE, FAKE, 0, 4, 32, 128, FAKE, None, None) == OK
    assert m(FAKE, None, 2, 4, 32, 128, FAKE, None, None) == NULL
    assert m(FAKE, FAKE, 2, 0, 32, 128, FAKE, None, None) == SHAPE
    assert m(FAKE, FAKE, 2, 4, 32, 64, FAKE, None, None) == UNSUP
    d = L.qsa_decode
    args = [FAKE] * 7 + [2, 32, 4, 128, 4, 64, 64, 16, 256, 512, 4, 0.1] + [FAKE] * 7 + [FAKE, 1 << 24, None]
    bad = list(args)
    bad[1] = None                  # q_idx
    assert d(*bad) == NULL
    bad = list(args)
    bad[24] = None                 # out
    assert d(*bad) == NULL
    bad = list(args)
    bad[8] = 33                    # Hq % Hkv
    assert d(*bad) == SHAPE
    bad = list(args)
    bad[15] = 255                  # max_blocks below max_pages * 16
    assert d(*bad) == SHAPE
    bad = list(args)
    bad[17] = 0                    # P
    assert d(*bad) == SHAPE
    bad = list(args)
    bad[26], bad[27] = None, 0     # the per-page maxima need a workspace
    assert d(*bad) == WS
    bad = list(args)
    bad[27] = 100                  # too small
    assert d(*bad) == WS
    assert L.qsa_workspace_clear(None, 0, None) == OK
    assert L.qsa_workspace_clear(None, 64, None) == NULL
    assert L.qsa_workspace_clear(FAKE, 63, None) == SHAPE
    # the decode workspace: per-page maxima (B * max_blocks/16 int32, 256-byte aligned), then
    # the attention workspace
    assert L.qsa_decode_workspace_size(4, 32, 4, 65536, 512, 4) == 4 * 4096 * 4 + attn_ws(4, 32, 4, 4)
    assert L.qsa_decode_workspace_size(0, 32, 4, 65536, 512, 4) == 0


def test_calibration_library():
    """libqsa_calib exports what include/qsa_calib.h declares; its host checks need no GPU."""
    from sparse_attention_decode_qsa_amd import calib
    text = open(os.path.join(ROOT, "include", "qsa_calib.h")).read()
    names = sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", text)))
    assert names == ["qsa_calib_copy", "qsa_calib_read"]
    C = calib.lib()
    assert C.qsa_calib_copy(None, None, 0, None) == 0
    assert C.qsa_calib_copy(None, FAKE.value, 16, None) == 1
    assert C.qsa_calib_copy(FAKE.value, FAKE.value, 15, None) == 2
    assert C.qsa_calib_copy(FAKE.value + 4, FAKE.value, 16, None) == 2
    assert C.qsa_calib_read(None, 0, None, None) == 0
    assert C.qsa_calib_read(FAKE.value, 16, None, None) == 1
    assert C.qsa_calib_read(FAKE.value, 24, FAKE.value, None) == 2


def test_check_pages_host_checks():
    L = qsa.lib()
    c = L.qsa_check_pages
    assert c(None, None, 0, 16, 64, 100, None, None) == OK
    assert c(FAKE, None, 2, 16, 64, 100, FAKE, None) == NULL
    assert c(FAKE, FAKE, 2, 16, 64, 100, None, None) == NULL
    assert c(FAKE, FAKE, -1, 16, 64, 100, FAKE, None) == SHAPE
    assert c(FAKE, FAKE, 2, 0, 64, 100, FAKE, None) == SHAPE
    assert c(FAKE, FAKE, 2, 16, 0, 100, FAKE, None) == SHAPE
    assert c(FAKE, FAKE, 2, 16, 64, -1, FAKE, None) == SHAPE
    assert c(FAKE, FAKE, 70000, 16, 64, 100, FAKE, None) == UNSUP


def test_side_cache_host_checks():
    L = qsa.lib()
    assert L.qsa_pool_build(None, None, None, 0, 4, 64, 64, 16, None, None) == OK
    assert L.qsa_pool_build(FAKE, FAKE, FAKE, 2, 4, 64, 64, 16, None, None) == NULL
    assert L.qsa_pool_build(FAKE, FAKE, FAKE, 2, 4, 32, 64, 16, FAKE, None) == UNSUP
    assert L.qsa_pool_build(FAKE, FAKE, FAKE, 2, 4, 64, 64, 0, FAKE, None) == SHAPE
    ap = L.qsa_cache_append
    args = [FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, 2, 4, 128, 4, 64, 64, 16, None]
    assert ap(*args[:10], 0, *args[11:]) == OK
    bad = list(args); bad[0] = None
    assert ap(*bad) == NULL
    bad = list(args); bad[12] = 64
    assert ap(*bad) == UNSUP
    bad = list(args); bad[11] = 0
    assert ap(*bad) == SHAPE
    bad = list(args); bad[7] = FAKE.value + 8
    assert ap(*bad) == SHAPE                       # misaligned side cache
    sp = L.qsa_index_score_pooled
    assert sp(FAKE, None, FAKE, FAKE, 2, 4, 64, 64, 16, 256, FAKE, None, None) == NULL
    assert sp(FAKE, FAKE, FAKE, FAKE, 2, 4, 64, 64, 16, 255, FAKE, None, None) == SHAPE
    d = L.qsa_decode_pooled
    dargs = [FAKE] * 7 + [2, 32, 4, 128, 4, 64, 64, 16, 256, 512, 4, 0.1] + [FAKE] * 7 + [FAKE, 1 << 24, None]
    bad = list(dargs); bad[2] = None
    assert d(*bad) == NULL
    bad = list(dargs); bad[8] = 33
    assert d(*bad) == SHAPE


def test_decode_multi_host_checks():
    L = qsa.lib()
    assert L.qsa_decode_multi_workspace_size(4, 3, 32, 4, 65536, 512, 4) == L.qsa_decode_workspace_size(
        12, 32, 4, 65536, 512, 4)
    assert L.qsa_decode_multi_workspace_size(4, 0, 32, 4, 65536, 512, 4) == 0
    d = L.qsa_decode_multi
    args = [FAKE] * 7 + [2, 2, 32, 4, 128, 4, 64, 64, 16, 256, 512, 4, 0.1] + [FAKE] * 7 + [FAKE, 1 << 26, None]
    bad = list(args); bad[8] = 0
    assert d(*bad) == SHAPE                        # T = 0
    bad = list(args); bad[8] = 4097
    assert d(*bad) == UNSUP                        # more than 4096 new tokens
    bad = list(args); bad[7], bad[8] = 20000, 4
    assert d(*bad) == UNSUP                        # B*T > 65535
    bad = list(args); bad[1] = None
    assert d(*bad) == NULL
    bad = list(args); bad[28] = 100
    assert d(*bad) == WS


def test_decode_multi_pooled_host_checks():
    """qsa_decode_multi_pooled: qsa_decode_multi's checks, both key caches required, T <= 4."""
    d = qsa.lib().qsa_decode_multi_pooled
    args = [FAKE] * 8 + [2, 2, 32, 4, 128, 4, 64, 64, 16, 256, 512, 4, 0.1] + [FAKE] * 7 + [FAKE, 1 << 26, None]
    assert len(args) == len(qsa.SIGNATURES["qsa_decode_multi_pooled"][1])
    assert d(*args[:8], 0, *args[9:]) == OK        # B = 0
    bad = list(args); bad[3] = None
    assert d(*bad) == NULL                         # no side cache
    bad = list(args); bad[2] = None
    assert d(*bad) == NULL                         # no int8 keys for the pages with draft positions
    bad = list(args); bad[9] = 0
    assert d(*bad) == SHAPE                        # T = 0
    bad = list(args); bad[9] = 5
    assert d(*bad) == UNSUP                        # more than 4 draft tokens
    bad = list(args); bad[29] = 100
    assert d(*bad) == WS


def test_index_score_multi_host_checks():
    L = qsa.lib()
    f = L.qsa_index_score_multi
    assert f(None, None, None, None, 0, 2, 4, 64, 64, 16, 256, None, None, None) == OK
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 0, 4, 64, 64, 16, 256, FAKE, None, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 4097, 4, 64, 64, 16, 256, FAKE, None, None) == UNSUP
    assert f(FAKE, FAKE, FAKE, FAKE, 2, 2, 4, 64, 64, 16, 255, FAKE, None, None) == SHAPE
    assert f(FAKE, None, FAKE, FAKE, 2, 2, 4, 64, 64, 16, 256, FAKE, None, None) == NULL


def test_decode_step_pooled_host_checks():
    L = qsa.lib()
    f = L.qsa_decode_step_pooled
    args = [FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 32, 4, 128, 4, 64, 64, 16,
            256, 512, 4, 0.1] + [FAKE] * 7 + [FAKE, 1 << 26, None]
    bad = list(args); bad[0] = None
    assert f(*bad) == NULL
    bad = list(args); bad[7] = None
    assert f(*bad) == NULL
    bad = list(args); bad[7] = FAKE.value + 4
    assert f(*bad) == SHAPE
    bad = list(args); bad[13] = 33
    assert f(*bad) == SHAPE                        # Hq % Hkv
    bad = list(args); bad[32] = 100
    assert f(*bad) == WS


def test_decode_noalloc_host_checks():
    """qsa_decode_noalloc: qsa_decode's argument checks, then the static scratch's limit; a
    call that fails either returns its code before any device call (none runs here)."""
    L = qsa.lib()
    f = L.qsa_decode_noalloc
    args = [FAKE] * 7 + [2, 32, 4, 128, 4, 64, 64, 16, 256, 512, 4, 0.1] + [FAKE] * 7 + [None]
    assert len(args) == len(qsa.SIGNATURES["qsa_decode_noalloc"][1])
    assert f(*args[:7], 0, *args[8:]) == OK
    bad = list(args); bad[7] = -1
    assert f(*bad) == SHAPE
    bad = list(args); bad[0] = None
    assert f(*bad) == NULL
    bad = list(args); bad[8] = 33
    assert f(*bad) == SHAPE                        # Hq % Hkv
    bad = list(args); bad[10] = 64
    assert f(*bad) == UNSUP                        # head_dim
    # more workspace than the scratch holds: 4096 requests of up to 262,144 tokens
    big = list(args); big[7], big[14], big[15] = 4096, 4096, 65536
    need = L.qsa_decode_workspace_size(4096, 32, 4, 65536, 512, 4)
    assert need > qsa.NOALLOC_SCRATCH_BYTES
    assert f(*big) == 6                            # QSA_ERR_SCRATCH
    # the w4 and 128-request shapes fit
    assert L.qsa_decode_workspace_size(4, 32, 4, 65536, 512, 4) <= qsa.NOALLOC_SCRATCH_BYTES
    assert L.qsa_decode_workspace_size(128, 32, 4, 65536, 512, 4) <= qsa.NOALLOC_SCRATCH_BYTES


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every entry point raises: there is no fallback path."""
    from sparse_attention_decode_qsa_amd import qsa
    monkeypatch.setattr(qsa, "LIB_PATH", str(tmp_path / "libqsa.so"))
    monkeypatch.setattr(qsa, "_lib", None)
    with pytest.raises(ImportError, match="missing"):
        qsa.lib()
    with pytest.raises(ImportError):
        qsa.decode_workspace_size(4, 32, 4, 65536, 512, 4)

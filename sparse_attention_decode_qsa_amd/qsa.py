"""Python binding of libqsa: the C ABI entry points with the same names, on torch tensors.

Argument marshalling only. Every step of the decode path runs in the HIP kernels of
libqsa.so; there is no fallback. Loading fails with an error if the library has not
been built (python -m sparse_attention_decode_qsa_amd.build).

Tensors must be contiguous and on the current GPU; calls enqueue on torch's current
stream and return without synchronizing.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqsa.so")

PAGE_SIZE = 64
IDX_HEADS = 4
IDX_DIM = 64
HEAD_DIM = 128
MAX_K = 512

STATUS = {0: "QSA_OK", 1: "QSA_ERR_NULL", 2: "QSA_ERR_SHAPE", 3: "QSA_ERR_UNSUPPORTED",
          4: "QSA_ERR_WORKSPACE", 5: "QSA_ERR_HIP", 6: "QSA_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 32 << 20   # QSA_NOALLOC_SCRATCH_BYTES of include/qsa.h

# (name, restype, argtypes) of every symbol declared in include/qsa.h
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "qsa_status_string": (ctypes.c_char_p, [_I]),
    "qsa_last_hip_error": (_I, []),
    "qsa_version": (_I, []),
    "qsa_index_score": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "qsa_topk_workspace_size": (_Z, [_I, _I, _I]),
    "qsa_topk_select": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _Z, _P]),
    "qsa_attn_workspace_size": (_Z, [_I, _I, _I, _I, _I]),
    "qsa_sparse_attn_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                                    _P, _P, _P, _Z, _P]),
    "qsa_lse_merge": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "qsa_decode_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I]),
    "qsa_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                        _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "qsa_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                                _P, _P, _P, _P, _P, _P, _P, _P]),
    "qsa_workspace_clear": (_I, [_P, _Z, _P]),
    "qsa_time_next_scan": (_I, [_P, _P]),
    "qsa_check_pages": (_I, [_P, _P, _I, _I, _I, _I, _P, _P]),
    "qsa_decode_multi_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "qsa_index_score_multi": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "qsa_decode_multi": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                              _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "qsa_decode_multi_pooled": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                     _I, _F, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "qsa_decode_step_pooled": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                    _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "qsa_pool_build": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "qsa_cache_append": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "qsa_index_score_pooled": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "qsa_decode_pooled": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                               _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
}


class QsaError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libqsa.so (raises if it is missing: there is no other implementation)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m sparse_attention_decode_qsa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        L = lib()
        msg = L.qsa_status_string(status).decode()
        extra = f" (hipError {L.qsa_last_hip_error()})" if status == 5 else ""
        raise QsaError(f"{STATUS.get(status, status)}: {msg}{extra}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name}: expected {dim} dims, got {tuple(t.shape)}")


class Workspace:
    """A device workspace of the size a libqsa *_workspace_size query returned."""

    def __init__(self, nbytes: int, device=None):
        self.nbytes = int(nbytes)
        self.tensor = torch.zeros(max(self.nbytes, 16), dtype=torch.uint8, device=device or "cuda")

    def ptr(self):
        return ctypes.c_void_p(self.tensor.data_ptr())


def topk_workspace_size(B, max_blocks, k=MAX_K) -> int:
    return int(lib().qsa_topk_workspace_size(B, max_blocks, k))


def attn_workspace_size(B, Hq, Hkv, k=MAX_K, P=1) -> int:
    return int(lib().qsa_attn_workspace_size(B, Hq, Hkv, k, P))


def decode_workspace_size(B, Hq, Hkv, max_blocks, k=MAX_K, P=1) -> int:
    return int(lib().qsa_decode_workspace_size(B, Hq, Hkv, max_blocks, k, P))


def index_score(q_idx, idx_cache, page_table, context_lens, max_blocks=None, out=None, page_max=None):
    """Block scores [B, max_blocks] int32 (entries past ceil(L_b/4) are left as they are).

    page_max: optional [B, max_pages] int32 output of the largest block score per page.
    """
    _need(q_idx, torch.int8, "q_idx", 3)
    _need(idx_cache, torch.int8, "idx_cache", 4)
    _need(page_table, torch.int32, "page_table", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, max_pages = page_table.shape
    max_blocks = max_pages * PAGE_SIZE // 4 if max_blocks is None else max_blocks
    if out is None:
        out = torch.empty((B, max_blocks), dtype=torch.int32, device=q_idx.device)
    _need(out, torch.int32, "out", 2)
    if page_max is not None:
        _need(page_max, torch.int32, "page_max", 2)
        if tuple(page_max.shape) != (B, max_pages):
            raise ValueError(f"page_max: expected {(B, max_pages)}, got {tuple(page_max.shape)}")
    _check(lib().qsa_index_score(_ptr(q_idx), _ptr(idx_cache), _ptr(page_table), _ptr(context_lens),
                                 B, q_idx.shape[1], q_idx.shape[2], idx_cache.shape[1], max_pages,
                                 out.shape[1], _ptr(out), _ptr(page_max), _stream()))
    return out


def topk_select(block_scores, context_lens, k=MAX_K, workspace=None, sel=None, count=None, page_max=None):
    """(sel_blocks [B, k] int32 ascending, -1 padded; sel_count [B] int32).

    page_max: optional [B, max_pages] int32 as written by index_score (same result, fewer reads).
    """
    _need(block_scores, torch.int32, "block_scores", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, max_blocks = block_scores.shape
    max_pages = 0
    if page_max is not None:
        _need(page_max, torch.int32, "page_max", 2)
        max_pages = page_max.shape[1]
    dev = block_scores.device
    sel = torch.empty((B, k), dtype=torch.int32, device=dev) if sel is None else sel
    count = torch.empty((B,), dtype=torch.int32, device=dev) if count is None else count
    ws = workspace or Workspace(topk_workspace_size(B, max_blocks, k), dev)
    _check(lib().qsa_topk_select(_ptr(block_scores), _ptr(context_lens), _ptr(page_max), B, max_blocks,
                                 max_pages, k, _ptr(sel), _ptr(count), ws.ptr(), ws.nbytes, _stream()))
    return sel, count


def sparse_attn_decode(q, k_cache, v_cache, page_table, context_lens, sel_blocks, sel_count, P=1,
                       softmax_scale=None, workspace=None, out=None, lse=None):
    """Per-slice partials: (partial_out [B, P, Hq, 128] f32, partial_lse [B, P, Hq] f32)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(k_cache, torch.bfloat16, "k_cache", 4)
    _need(v_cache, torch.bfloat16, "v_cache", 4)
    _need(page_table, torch.int32, "page_table", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    _need(sel_blocks, torch.int32, "sel_blocks", 2)
    _need(sel_count, torch.int32, "sel_count", 1)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    k = sel_blocks.shape[1]
    scale = D ** -0.5 if softmax_scale is None else softmax_scale
    dev = q.device
    out = torch.empty((B, P, Hq, D), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, P, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    ws = workspace or Workspace(attn_workspace_size(B, Hq, Hkv, k, P), dev)
    _check(lib().qsa_sparse_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(context_lens), _ptr(sel_blocks),
        _ptr(sel_count), B, Hq, Hkv, D, k_cache.shape[1], page_table.shape[1], k, P, scale, _ptr(out),
        _ptr(lse), ws.ptr(), ws.nbytes, _stream()))
    return out, lse


def lse_merge(partial_out, partial_lse, out=None, out_lse=None, want_lse=True):
    """(out [B, Hq, 128] f32, out_lse [B, Hq] f32 or None)."""
    _need(partial_out, torch.float32, "partial_out", 4)
    _need(partial_lse, torch.float32, "partial_lse", 3)
    B, P, Hq, D = partial_out.shape
    dev = partial_out.device
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev) if out is None else out
    if want_lse and out_lse is None:
        out_lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _check(lib().qsa_lse_merge(_ptr(partial_out), _ptr(partial_lse), B, P, Hq, D, _ptr(out),
                               _ptr(out_lse), _stream()))
    return out, out_lse


def time_next_scan(start, stop):
    """The next indexer-scan launch of this thread records torch.cuda.Event `start` at the
    kernel's start and `stop` at its end (events created with enable_timing=True and recorded
    once before, so that torch has created them)."""
    if not start.cuda_event or not stop.cuda_event:
        raise ValueError("time_next_scan: the events must have been recorded once (torch creates them lazily)")
    _check(lib().qsa_time_next_scan(ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event)))


class DecodePlan:
    """Preallocated buffers and one qsa_decode call per run(): the whole chain on one stream.

    Holds every intermediate (scores, sel, sel_count, partials) and the outputs.
    """

    def __init__(self, q, q_idx, idx_cache, k_cache, v_cache, page_table, context_lens, P, k=MAX_K,
                 softmax_scale=None, max_blocks=None, pooled=None, noalloc=False):
        """pooled: optional side cache of pooled keys (int16); the scan then reads it
        (qsa_decode_pooled) instead of idx_cache, for the same results.
        noalloc: run qsa_decode_noalloc, whose workspace is the library's static scratch (no
        workspace is allocated here; calls that overlap on one device race on that scratch)."""
        for t, dt, n in ((q, torch.bfloat16, "q"), (q_idx, torch.int8, "q_idx"),
                         (idx_cache, torch.int8, "idx_cache"), (k_cache, torch.bfloat16, "k_cache"),
                         (v_cache, torch.bfloat16, "v_cache"), (page_table, torch.int32, "page_table"),
                         (context_lens, torch.int32, "context_lens")):
            _need(t, dt, n)
        self.inputs = (q, q_idx, idx_cache, k_cache, v_cache, page_table, context_lens)
        B, Hq, D = q.shape
        Hkv = k_cache.shape[2]
        max_pages = page_table.shape[1]
        self.max_blocks = max_pages * PAGE_SIZE // 4 if max_blocks is None else max_blocks
        dev = q.device
        self.scores = torch.empty((B, self.max_blocks), dtype=torch.int32, device=dev)
        self.sel = torch.empty((B, k), dtype=torch.int32, device=dev)
        self.sel_count = torch.empty((B,), dtype=torch.int32, device=dev)
        self.partial_out = torch.empty((B, P, Hq, D), dtype=torch.float32, device=dev)
        self.partial_lse = torch.empty((B, P, Hq), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        self.out_lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        if noalloc and pooled is not None:
            raise ValueError("noalloc runs qsa_decode_noalloc, which reads the int8 indexer keys")
        self.workspace = None if noalloc else Workspace(decode_workspace_size(B, Hq, Hkv, self.max_blocks, k, P),
                                                        dev)
        scale = D ** -0.5 if softmax_scale is None else softmax_scale
        if pooled is not None:
            _need(pooled, torch.int16, "pooled", 4)
        self._fn = (lib().qsa_decode_noalloc if noalloc else
                    lib().qsa_decode if pooled is None else lib().qsa_decode_pooled)
        self._args = [
            _ptr(q), _ptr(q_idx), _ptr(idx_cache if pooled is None else pooled), _ptr(k_cache), _ptr(v_cache),
            _ptr(page_table),
            _ptr(context_lens), B, Hq, Hkv, D, q_idx.shape[1], q_idx.shape[2], k_cache.shape[1],
            max_pages, self.max_blocks, k, P, ctypes.c_float(scale), _ptr(self.scores), _ptr(self.sel),
            _ptr(self.sel_count), _ptr(self.partial_out), _ptr(self.partial_lse), _ptr(self.out),
            _ptr(self.out_lse)]
        if not noalloc:
            self._args += [self.workspace.ptr(), self.workspace.nbytes]

    def run(self, stream=None):
        s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream()
        _check(self._fn(*self._args, s))
        return self.out, self.out_lse


def new_pooled_cache(idx_cache):
    """A zeroed side cache [num_pages, 16, 4, 64] int16 matching the int8 indexer cache."""
    _need(idx_cache, torch.int8, "idx_cache", 4)
    n, ps, h, d = idx_cache.shape
    return torch.zeros((n, ps // 4, h, d), dtype=torch.int16, device=idx_cache.device)


def pool_build(idx_cache, page_table, context_lens, pooled=None):
    """Side-cache entries of every block of every request (entries of no block untouched)."""
    _need(idx_cache, torch.int8, "idx_cache", 4)
    _need(page_table, torch.int32, "page_table", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    pooled = new_pooled_cache(idx_cache) if pooled is None else pooled
    _need(pooled, torch.int16, "pooled", 4)
    B, max_pages = page_table.shape
    _check(lib().qsa_pool_build(_ptr(idx_cache), _ptr(page_table), _ptr(context_lens), B, idx_cache.shape[2],
                                idx_cache.shape[3], idx_cache.shape[1], max_pages, _ptr(pooled), _stream()))
    return pooled


def cache_append(k_new, v_new, idx_new, k_cache, v_cache, idx_cache, page_table, context_lens, pooled=None,
                 write=None):
    """Write each request's new token (at L_b - 1) into the caches and refresh its block's
    side-cache entry; requests with write[b] == 0 write nothing."""
    for t, dt, n in ((k_new, torch.bfloat16, "k_new"), (v_new, torch.bfloat16, "v_new"), (idx_new, torch.int8, "idx_new"),
                     (k_cache, torch.bfloat16, "k_cache"), (v_cache, torch.bfloat16, "v_cache"),
                     (idx_cache, torch.int8, "idx_cache"), (page_table, torch.int32, "page_table"),
                     (context_lens, torch.int32, "context_lens")):
        _need(t, dt, n)
    if pooled is not None:
        _need(pooled, torch.int16, "pooled", 4)
    if write is not None:
        _need(write, torch.int32, "write", 1)
    B, max_pages = page_table.shape
    Hkv = k_cache.shape[2]
    _check(lib().qsa_cache_append(_ptr(k_new), _ptr(v_new), _ptr(idx_new), _ptr(write), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(idx_cache), _ptr(pooled), _ptr(page_table), _ptr(context_lens), B, Hkv,
                                  k_cache.shape[3], idx_cache.shape[2], idx_cache.shape[3], k_cache.shape[1],
                                  max_pages, _stream()))


def index_score_pooled(q_idx, pooled, page_table, context_lens, max_blocks=None, out=None, page_max=None):
    """index_score reading the side cache: the same block scores [B, max_blocks] int32."""
    _need(q_idx, torch.int8, "q_idx", 3)
    _need(pooled, torch.int16, "pooled", 4)
    _need(page_table, torch.int32, "page_table", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, max_pages = page_table.shape
    max_blocks = max_pages * PAGE_SIZE // 4 if max_blocks is None else max_blocks
    if out is None:
        out = torch.empty((B, max_blocks), dtype=torch.int32, device=q_idx.device)
    _need(out, torch.int32, "out", 2)
    if page_max is not None:
        _need(page_max, torch.int32, "page_max", 2)
    _check(lib().qsa_index_score_pooled(_ptr(q_idx), _ptr(pooled), _ptr(page_table), _ptr(context_lens), B,
                                        q_idx.shape[1], q_idx.shape[2], PAGE_SIZE, max_pages, out.shape[1], _ptr(out),
                                        _ptr(page_max), _stream()))
    return out


def check_pages(page_table, context_lens, num_pages, verdict=None):
    """Per-request verdict [B] int32: -1 valid, -2 length out of range, p = first bad page slot."""
    _need(page_table, torch.int32, "page_table", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, max_pages = page_table.shape
    if verdict is None:
        verdict = torch.empty((B,), dtype=torch.int32, device=page_table.device)
    _need(verdict, torch.int32, "verdict", 1)
    _check(lib().qsa_check_pages(_ptr(page_table), _ptr(context_lens), B, max_pages, PAGE_SIZE, int(num_pages),
                                 _ptr(verdict), _stream()))
    return verdict


def index_score_multi(q_idx, idx_cache, page_table, context_lens, max_blocks=None, out=None, page_max=None):
    """Scores of T draft tokens per request from one read of the keys: q_idx [B, T, 4, 64];
    returns [B*T, max_blocks] int32 (row b*T + t)."""
    _need(q_idx, torch.int8, "q_idx", 4)
    _need(idx_cache, torch.int8, "idx_cache", 4)
    _need(page_table, torch.int32, "page_table", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, T = q_idx.shape[:2]
    max_pages = page_table.shape[1]
    max_blocks = max_pages * PAGE_SIZE // 4 if max_blocks is None else max_blocks
    if out is None:
        out = torch.empty((B * T, max_blocks), dtype=torch.int32, device=q_idx.device)
    _need(out, torch.int32, "out", 2)
    if page_max is not None:
        _need(page_max, torch.int32, "page_max", 2)
    _check(lib().qsa_index_score_multi(_ptr(q_idx), _ptr(idx_cache), _ptr(page_table), _ptr(context_lens), B, T,
                                       q_idx.shape[2], q_idx.shape[3], idx_cache.shape[1], max_pages, out.shape[1],
                                       _ptr(out), _ptr(page_max), _stream()))
    return out


class MultiDecodePlan:
    """Multi-token decode: T draft tokens per request, one qsa_decode_multi call per run().

    q [B, T, Hq, 128] bf16, q_idx [B, T, 4, 64] int8; the results hold one row per
    (request, draft token) in the order b*T + t (e.g. out [B*T, Hq, 128]). With pooled (the
    side cache, T <= 4) each run() is one qsa_decode_multi_pooled call instead: the same
    results from the side cache."""

    def __init__(self, q, q_idx, idx_cache, k_cache, v_cache, page_table, context_lens, P, k=MAX_K,
                 softmax_scale=None, max_blocks=None, pooled=None):
        _need(q, torch.bfloat16, "q", 4)
        _need(q_idx, torch.int8, "q_idx", 4)
        for t, dt, n in ((idx_cache, torch.int8, "idx_cache"), (k_cache, torch.bfloat16, "k_cache"),
                         (v_cache, torch.bfloat16, "v_cache"), (page_table, torch.int32, "page_table"),
                         (context_lens, torch.int32, "context_lens")):
            _need(t, dt, n)
        self.inputs = (q, q_idx, idx_cache, k_cache, v_cache, page_table, context_lens)
        B, T, Hq, D = q.shape
        Hkv = k_cache.shape[2]
        max_pages = page_table.shape[1]
        self.T = T
        self.max_blocks = max_pages * PAGE_SIZE // 4 if max_blocks is None else max_blocks
        dev = q.device
        BT = B * T
        self.scores = torch.empty((BT, self.max_blocks), dtype=torch.int32, device=dev)
        self.sel = torch.empty((BT, k), dtype=torch.int32, device=dev)
        self.sel_count = torch.empty((BT,), dtype=torch.int32, device=dev)
        self.partial_out = torch.empty((BT, P, Hq, D), dtype=torch.float32, device=dev)
        self.partial_lse = torch.empty((BT, P, Hq), dtype=torch.float32, device=dev)
        self.out = torch.empty((BT, Hq, D), dtype=torch.float32, device=dev)
        self.out_lse = torch.empty((BT, Hq), dtype=torch.float32, device=dev)
        self.workspace = Workspace(lib().qsa_decode_multi_workspace_size(B, T, Hq, Hkv, self.max_blocks, k, P), dev)
        scale = D ** -0.5 if softmax_scale is None else softmax_scale
        if pooled is not None:
            _need(pooled, torch.int16, "pooled", 4)
        self._fn = lib().qsa_decode_multi if pooled is None else lib().qsa_decode_multi_pooled
        keys = [_ptr(idx_cache)] if pooled is None else [_ptr(idx_cache), _ptr(pooled)]
        self._args = [
            _ptr(q), _ptr(q_idx), *keys, _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
            _ptr(context_lens), B, T, Hq, Hkv, D, q_idx.shape[2], q_idx.shape[3], k_cache.shape[1],
            max_pages, self.max_blocks, k, P, ctypes.c_float(scale), _ptr(self.scores), _ptr(self.sel),
            _ptr(self.sel_count), _ptr(self.partial_out), _ptr(self.partial_lse), _ptr(self.out),
            _ptr(self.out_lse), self.workspace.ptr(), self.workspace.nbytes]

    def run(self, stream=None):
        s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream()
        _check(self._fn(*self._args, s))
        return self.out, self.out_lse


class StepPlan:
    """One decode step on the side cache per run(): the new token's cache writes and the decode
    (qsa_decode_step_pooled; the same results as AppendPlan.run() then DecodePlan(pooled).run())."""

    def __init__(self, k_new, v_new, idx_new, q, q_idx, idx_cache, k_cache, v_cache, page_table, context_lens,
                 pooled, P, k=MAX_K, softmax_scale=None, write=None):
        for t, dt, n in ((k_new, torch.bfloat16, "k_new"), (v_new, torch.bfloat16, "v_new"),
                         (idx_new, torch.int8, "idx_new"), (q, torch.bfloat16, "q"), (q_idx, torch.int8, "q_idx"),
                         (idx_cache, torch.int8, "idx_cache"), (k_cache, torch.bfloat16, "k_cache"),
                         (v_cache, torch.bfloat16, "v_cache"), (page_table, torch.int32, "page_table"),
                         (context_lens, torch.int32, "context_lens")):
            _need(t, dt, n)
        _need(pooled, torch.int16, "pooled", 4)
        if write is not None:
            _need(write, torch.int32, "write", 1)
        self.inputs = (k_new, v_new, idx_new, q, q_idx, idx_cache, k_cache, v_cache, page_table, context_lens,
                       pooled, write)
        B, Hq, D = q.shape
        Hkv = k_cache.shape[2]
        max_pages = page_table.shape[1]
        self.max_blocks = max_pages * PAGE_SIZE // 4
        dev = q.device
        self.scores = torch.empty((B, self.max_blocks), dtype=torch.int32, device=dev)
        self.sel = torch.empty((B, k), dtype=torch.int32, device=dev)
        self.sel_count = torch.empty((B,), dtype=torch.int32, device=dev)
        self.partial_out = torch.empty((B, P, Hq, D), dtype=torch.float32, device=dev)
        self.partial_lse = torch.empty((B, P, Hq), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        self.out_lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        self.workspace = Workspace(decode_workspace_size(B, Hq, Hkv, self.max_blocks, k, P), dev)
        scale = D ** -0.5 if softmax_scale is None else softmax_scale
        self._fn = lib().qsa_decode_step_pooled
        self._args = [
            _ptr(k_new), _ptr(v_new), _ptr(idx_new), _ptr(write), _ptr(k_cache), _ptr(v_cache), _ptr(idx_cache),
            _ptr(pooled), _ptr(q), _ptr(q_idx), _ptr(page_table), _ptr(context_lens), B, Hq, Hkv, D,
            q_idx.shape[1], q_idx.shape[2], k_cache.shape[1], max_pages, self.max_blocks, k, P, ctypes.c_float(scale),
            _ptr(self.scores), _ptr(self.sel), _ptr(self.sel_count), _ptr(self.partial_out), _ptr(self.partial_lse),
            _ptr(self.out), _ptr(self.out_lse), self.workspace.ptr(), self.workspace.nbytes]

    def run(self, stream=None):
        s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream()
        _check(self._fn(*self._args, s))
        return self.out, self.out_lse


class AppendPlan:
    """One qsa_cache_append call per run() with fixed buffers (the decode step's cache writes)."""

    def __init__(self, k_new, v_new, idx_new, k_cache, v_cache, idx_cache, page_table, context_lens, pooled=None,
                 write=None):
        for t, dt, n in ((k_new, torch.bfloat16, "k_new"), (v_new, torch.bfloat16, "v_new"),
                         (idx_new, torch.int8, "idx_new"), (k_cache, torch.bfloat16, "k_cache"),
                         (v_cache, torch.bfloat16, "v_cache"), (idx_cache, torch.int8, "idx_cache"),
                         (page_table, torch.int32, "page_table"), (context_lens, torch.int32, "context_lens")):
            _need(t, dt, n)
        if pooled is not None:
            _need(pooled, torch.int16, "pooled", 4)
        if write is not None:
            _need(write, torch.int32, "write", 1)
        self.keep = (k_new, v_new, idx_new, k_cache, v_cache, idx_cache, page_table, context_lens, pooled, write)
        B, max_pages = page_table.shape
        self._fn = lib().qsa_cache_append
        self._args = [_ptr(k_new), _ptr(v_new), _ptr(idx_new), _ptr(write), _ptr(k_cache), _ptr(v_cache),
                      _ptr(idx_cache), _ptr(pooled), _ptr(page_table), _ptr(context_lens), B, k_cache.shape[2],
                      k_cache.shape[3], idx_cache.shape[2], idx_cache.shape[3], k_cache.shape[1], max_pages]

    def run(self, stream=None):
        s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream()
        _check(self._fn(*self._args, s))


def decode(q, q_idx, idx_cache, k_cache, v_cache, page_table, context_lens, P=1, k=MAX_K,
           softmax_scale=None):
    """The whole path; returns the DecodePlan holding the outputs and intermediates."""
    plan = DecodePlan(q, q_idx, idx_cache, k_cache, v_cache, page_table, context_lens, P, k, softmax_scale)
    plan.run()
    return plan

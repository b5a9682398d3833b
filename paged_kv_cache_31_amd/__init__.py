"""Python binding of libpa.so, the MI355X paged decode-attention library (see include/pa.h).

Argument marshalling only: shapes and dtypes are read from torch tensors, the stream is torch's
current stream, and every step of the computation runs in the library's HIP kernels.  There is
no fallback: if libpa.so is missing or a call fails, a RuntimeError is raised.

Cache layout:  k_cache [num_blocks][num_kv_heads][16][head_dim],
               v_cache [num_blocks][num_kv_heads][head_dim][16];
fp8 caches are uint8 (or float8_e4m3fn) tensors of OCP e4m3fn codes with fp32 scales
[num_blocks][num_kv_heads] for K and for V.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

from . import contract

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_OUT_OF_BLOCKS = range(6)
PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
PA_SCALE_KEEP, PA_SCALE_FIRST_TOKEN = 0, 1
BLOCK_SIZE = 16


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("cache", CacheDesc), ("batch", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("max_context_len", ctypes.c_int32), ("partition_tokens", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("shared_prefixes", ctypes.c_int32)]


class MultiDesc(ctypes.Structure):
    _fields_ = [("cache", CacheDesc), ("batch", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("max_context_len", ctypes.c_int32), ("total_queries", ctypes.c_int32),
                ("max_query_len", ctypes.c_int32), ("partition_tokens", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32)]


class PaError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{fn} failed: {status_string(status)} (status {status})"
        if status == PA_ERR_HIP:
            msg += f", hipError {hip_error}"
        super().__init__(msg)


_lib = None
_lock = threading.Lock()

EXPORTS = ("pa_kv_append", "pa_kv_append_quant", "pa_decode", "pa_decode_append",
           "pa_decode_noalloc",
           "pa_decode_workspace_size", "pa_decode_multi", "pa_decode_multi_workspace_size",
           "pa_graph_begin", "pa_graph_end", "pa_graph_launch", "pa_graph_destroy",
           "pa_pool_create", "pa_pool_destroy", "pa_pool_free_blocks", "pa_pool_refcount",
           "pa_pool_alloc", "pa_pool_share", "pa_pool_release", "pa_pool_write",
           "pa_pool_slot_for", "pa_copy_blocks",
           "pa_status_string", "pa_last_hip_error")


def lib() -> ctypes.CDLL:
    """Load libpa.so (built in-tree by __graft_entry__.build()); raises if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
            L = ctypes.CDLL(LIB_PATH)
            vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
            L.pa_kv_append.argtypes = [ctypes.POINTER(CacheDesc), i32, vp, vp, vp, vp, vp, vp]
            L.pa_kv_append.restype = i32
            L.pa_kv_append_quant.argtypes = [ctypes.POINTER(CacheDesc), i32, i32, vp, vp, vp, vp,
                                             vp, vp, vp, i32, vp]
            L.pa_kv_append_quant.restype = i32
            L.pa_decode.argtypes = [ctypes.POINTER(DecodeDesc), vp, vp, vp, vp, vp, vp, vp,
                                    ctypes.c_float, vp, vp, sz, vp]
            L.pa_decode.restype = i32
            L.pa_decode_append.argtypes = [ctypes.POINTER(DecodeDesc), vp, vp, vp, vp, vp, vp,
                                           vp, vp, vp, ctypes.c_float, vp, vp, sz, vp]
            L.pa_decode_append.restype = i32
            L.pa_decode_noalloc.argtypes = [ctypes.POINTER(DecodeDesc), vp, vp, vp, vp, vp, vp,
                                            vp, ctypes.c_float, vp, vp]
            L.pa_decode_noalloc.restype = i32
            L.pa_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeDesc)]
            L.pa_decode_workspace_size.restype = sz
            L.pa_decode_multi.argtypes = [ctypes.POINTER(MultiDesc), vp, vp, vp, vp, vp, vp, vp,
                                          vp, ctypes.c_float, vp, vp, sz, vp]
            L.pa_decode_multi.restype = i32
            L.pa_decode_multi_workspace_size.argtypes = [ctypes.POINTER(MultiDesc)]
            L.pa_decode_multi_workspace_size.restype = sz
            L.pa_graph_begin.argtypes = [vp]
            L.pa_graph_begin.restype = i32
            L.pa_graph_end.argtypes = [vp, ctypes.POINTER(vp)]
            L.pa_graph_end.restype = i32
            L.pa_graph_launch.argtypes = [vp, vp]
            L.pa_graph_launch.restype = i32
            L.pa_graph_destroy.argtypes = [vp]
            L.pa_graph_destroy.restype = i32
            ip = ctypes.POINTER(i32)
            L.pa_pool_create.argtypes = [i32, ctypes.POINTER(vp)]
            L.pa_pool_destroy.argtypes = [vp]
            L.pa_pool_free_blocks.argtypes = [vp]
            L.pa_pool_refcount.argtypes = [vp, i32]
            L.pa_pool_alloc.argtypes = [vp, i32, ip]
            L.pa_pool_share.argtypes = [vp, i32, ip]
            L.pa_pool_release.argtypes = [vp, i32, ip]
            L.pa_pool_write.argtypes = [vp, i32, ip, ip]
            L.pa_pool_slot_for.argtypes = [vp, ip, ip, i32, i32, ctypes.POINTER(ctypes.c_int64),
                                           ip, ip]
            for f in ("pa_pool_create", "pa_pool_destroy", "pa_pool_free_blocks",
                      "pa_pool_refcount", "pa_pool_alloc", "pa_pool_share", "pa_pool_release",
                      "pa_pool_write", "pa_pool_slot_for"):
                getattr(L, f).restype = i32
            L.pa_copy_blocks.argtypes = [ctypes.POINTER(CacheDesc), i32, vp, vp, vp, vp, vp, vp]
            L.pa_copy_blocks.restype = i32
            L.pa_status_string.argtypes = [i32]
            L.pa_status_string.restype = ctypes.c_char_p
            L.pa_last_hip_error.argtypes = []
            L.pa_last_hip_error.restype = i32
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().pa_status_string(status).decode()


def _dtype_code(t: torch.Tensor, allow_fp8: bool) -> int:
    if t.dtype == torch.float16:
        return PA_F16
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if allow_fp8 and t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int):
    if status != PA_OK:
        raise PaError(fn, status, lib().pa_last_hip_error() if status == PA_ERR_HIP else 0)


def cache_desc(k_cache: torch.Tensor) -> CacheDesc:
    NB, Hkv, bs, D = k_cache.shape
    return CacheDesc(NB, Hkv, D, bs, _dtype_code(k_cache, True))


class AppendCall:
    """pa_kv_append with its arguments marshalled once; calling it only enqueues the kernel."""

    def __init__(self, k_new, v_new, slot_mapping, k_cache, v_cache, stream=None):
        assert k_cache.is_cuda and k_cache.is_contiguous() and v_cache.is_contiguous()
        assert k_new.is_contiguous() and v_new.is_contiguous() and slot_mapping.is_contiguous()
        assert slot_mapping.dtype == torch.int64
        NB, Hkv, bs, D = k_cache.shape
        assert tuple(v_cache.shape) == (NB, Hkv, D, bs), "v_cache must be [NB][Hkv][D][16]"
        T = slot_mapping.shape[0]
        assert tuple(k_new.shape) == (T, Hkv, D) and tuple(v_new.shape) == (T, Hkv, D)
        assert k_new.element_size() == k_cache.element_size()
        self._keep = (k_new, v_new, slot_mapping, k_cache, v_cache)
        self._desc = cache_desc(k_cache)
        self._fn = lib().pa_kv_append
        self._args = (ctypes.byref(self._desc), T, _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                      _ptr(k_cache), _ptr(v_cache), _stream(stream))

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != PA_OK:
            _check("pa_kv_append", st)


def _host(t):
    return t.detach().cpu().numpy()


def pa_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, stream=None,
                 check=False) -> None:
    """Scatter k_new/v_new [T][Hkv][D] into their slots (int64 [T], <0 skips).

    check=True (tests): first copy slot_mapping to the host and validate it (contract.py)."""
    if check:
        contract.check_slots(_host(slot_mapping), k_cache.shape[0])
    AppendCall(k_new, v_new, slot_mapping, k_cache, v_cache, stream)()


def pa_kv_append_quant(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                       first_token_scale=False, stream=None) -> None:
    """Quantise 16-bit k_new/v_new [T][Hkv][D] into the fp8 pools at their slots with the
    per-(block, KV head) scales; first_token_scale: a token at offset 0 of its block first sets
    that block's scales (amax / 448)."""
    for t in (k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale):
        assert t.is_cuda and t.is_contiguous()
    assert slot_mapping.dtype == torch.int64 and k_scale.dtype == torch.float32
    NB, Hkv, bs, D = k_cache.shape
    assert tuple(v_cache.shape) == (NB, Hkv, D, bs) and tuple(k_scale.shape) == (NB, Hkv)
    T = slot_mapping.shape[0]
    assert tuple(k_new.shape) == (T, Hkv, D) and tuple(v_new.shape) == (T, Hkv, D)
    st = lib().pa_kv_append_quant(ctypes.byref(cache_desc(k_cache)), T, _dtype_code(k_new, False),
                                  _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                  PA_SCALE_FIRST_TOKEN if first_token_scale else PA_SCALE_KEEP,
                                  _stream(stream))
    _check("pa_kv_append_quant", st)


def decode_desc(q, k_cache, block_tables, max_context_len=0, partition_tokens=0,
                shared_prefixes=False) -> DecodeDesc:
    # shared_prefixes: False/0 off, True/1 plan the groups, 2 reuse the plan of the last
    # planning call on the same workspace (unchanged tables and lengths)
    B, Hq, D = q.shape
    return DecodeDesc(cache_desc(k_cache), B, Hq, block_tables.shape[1], int(max_context_len),
                      int(partition_tokens), _dtype_code(q, False), int(shared_prefixes))


def pa_decode_workspace_size(desc: DecodeDesc) -> int:
    return int(lib().pa_decode_workspace_size(ctypes.byref(desc)))


_workspaces: dict = {}

# Which call last left a shared-prefix plan in a workspace (keyed by its device address): the
# key of a planning call with the same descriptor, tables and lengths lets a later call reuse
# the plan (shared_prefixes 2); any other call on the workspace overwrites its scratch, so it
# forgets the entry and the next reusing call plans again.
_plan_owner: dict = {}


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A pa_decode / pa_decode_multi workspace: zero-filled once (the kernels leave their arrival
    counters at zero)."""
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def _workspace(nbytes: int, device, stream_handle: int):
    key = (device, stream_handle)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = new_workspace(nbytes, device)
        _workspaces[key] = ws
    return ws


class DecodeCall:
    """pa_decode (or, with k_new/v_new, pa_decode_append) with its arguments marshalled once;
    calling it only enqueues the kernels."""

    def __init__(self, q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale=None,
                 v_scale=None, max_context_len=0, partition_tokens=0, workspace=None,
                 stream=None, shared_prefixes=False, k_new=None, v_new=None):
        for t in (q, k_cache, v_cache, block_tables, context_lens, out):
            assert t.is_cuda and t.is_contiguous()
        assert block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32
        assert out.shape == q.shape and out.dtype == q.dtype
        NB, Hkv, bs, D = k_cache.shape
        assert tuple(v_cache.shape) == (NB, Hkv, D, bs), "v_cache must be [NB][Hkv][D][16]"
        assert q.shape[2] == D and context_lens.shape[0] == q.shape[0] == block_tables.shape[0]
        fused = k_new is not None
        if fused:
            B = q.shape[0]
            for t in (k_new, v_new):
                assert t.is_contiguous() and tuple(t.shape) == (B, Hkv, D)
                assert t.element_size() == k_cache.element_size()
        self._desc = decode_desc(q, k_cache, block_tables, max_context_len, partition_tokens,
                                 shared_prefixes)
        need = pa_decode_workspace_size(self._desc)
        st = _stream(stream)
        if workspace is None:
            workspace = _workspace(need, q.device, st.value or 0)
        wbytes = workspace.numel() * workspace.element_size()
        self._keep = (q, k_cache, v_cache, block_tables, context_lens, out, k_scale, v_scale,
                      workspace, k_new, v_new)
        tail = (_ptr(k_scale), _ptr(v_scale), _ptr(block_tables), _ptr(context_lens),
                ctypes.c_float(scale), _ptr(out), _ptr(workspace), ctypes.c_size_t(wbytes), st)
        if fused:
            self._name, self._fn = "pa_decode_append", lib().pa_decode_append
            head = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache))
        else:
            self._name, self._fn = "pa_decode", lib().pa_decode
            head = (_ptr(q), _ptr(k_cache), _ptr(v_cache))
        self._args = (ctypes.byref(self._desc),) + head + tail
        # shared-prefix plan bookkeeping (see _plan_owner)
        self._ws = workspace.data_ptr()
        self._mode = int(shared_prefixes)
        d = self._desc
        self._plan_key = (d.cache.num_blocks, d.cache.num_kv_heads, d.cache.head_dim,
                          d.cache.kv_dtype, d.batch, d.num_q_heads, d.max_blocks_per_seq,
                          d.max_context_len, d.partition_tokens, d.q_dtype,
                          block_tables.data_ptr(), context_lens.data_ptr(), wbytes)
        if self._mode == 2:                  # the planning form, for when the plan is gone
            self._plan_desc = decode_desc(q, k_cache, block_tables, max_context_len,
                                          partition_tokens, 1)
            self._plan_args = (ctypes.byref(self._plan_desc),) + head + tail

    def __call__(self) -> None:
        args = self._args
        self.reused = False           # whether this call took a saved plan (shared_prefixes 2)
        if self._mode == 0:
            _plan_owner.pop(self._ws, None)
        else:
            if self._mode == 2:
                if _plan_owner.get(self._ws) == self._plan_key:
                    self.reused = True
                else:
                    args = self._plan_args
            _plan_owner[self._ws] = self._plan_key
        st = self._fn(*args)
        if st != PA_OK:
            _check(self._name, st)


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale=None,
              v_scale=None, max_context_len=0, partition_tokens=0, workspace=None,
              stream=None, shared_prefixes=False, check=False) -> torch.Tensor:
    """out[b][h] = softmax(scale * q[b][h] . K_b^T) . V_b through the block tables; returns out.

    shared_prefixes: read blocks that several sequences' tables start with once per group of
    sequences; 2 reuses the grouping planned by the previous call on the same workspace (the
    layers of one step, and later steps while the batch keeps its sequences: the kernel drops
    members whose tables or lengths no longer fit the saved grouping), see
    pa_decode_desc.shared_prefixes.  The binding tracks which call last used each workspace and
    plans again when another call has used it since the planning call.
    check=True (tests): first copy the tables and lengths to the host and validate them."""
    if check:
        contract.check_tables(_host(block_tables), _host(context_lens), k_cache.shape[0],
                              max_context_len)
    DecodeCall(q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale, v_scale,
               max_context_len, partition_tokens, workspace, stream, shared_prefixes)()
    return out


def pa_decode_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out,
                     k_scale=None, v_scale=None, max_context_len=0, partition_tokens=0,
                     workspace=None, stream=None, shared_prefixes=False,
                     check=False) -> torch.Tensor:
    """Store k_new/v_new [B][Hkv][D] as token context_lens[b]-1 of every sequence, then decode
    (pa_kv_append + pa_decode in one launch); returns out.
    check=True (tests): first validate the tables, lengths and appended blocks on the host."""
    if check:
        contract.check_decode_append(_host(block_tables), _host(context_lens), k_cache.shape[0],
                                     max_context_len)
    DecodeCall(q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale, v_scale,
               max_context_len, partition_tokens, workspace, stream, shared_prefixes, k_new,
               v_new)()
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def pa_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale=None,
                      v_scale=None, max_context_len=0, partition_tokens=0, stream=None,
                      shared_prefixes=False) -> torch.Tensor:
    """pa_decode with the library's own static scratch (no workspace, no allocation anywhere):
    for code that must not allocate, e.g. under graph capture.  Calls on one GPU share that
    scratch, so they must not overlap.  Returns out."""
    for t in (q, k_cache, v_cache, block_tables, context_lens, out):
        assert t.is_cuda and t.is_contiguous()
    assert block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32
    assert out.shape == q.shape and out.dtype == q.dtype
    desc = decode_desc(q, k_cache, block_tables, max_context_len, partition_tokens,
                       shared_prefixes)
    st = lib().pa_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                                 _ptr(context_lens), ctypes.c_float(scale), _ptr(out),
                                 _stream(stream))
    _check("pa_decode_noalloc", st)
    return out


def multi_desc(q, k_cache, block_tables, max_query_len, max_context_len=0,
               partition_tokens=0) -> MultiDesc:
    N, Hq, D = q.shape
    return MultiDesc(cache_desc(k_cache), block_tables.shape[0], Hq, block_tables.shape[1],
                     int(max_context_len), N, int(max_query_len), int(partition_tokens),
                     _dtype_code(q, False))


def pa_decode_multi_workspace_size(desc: MultiDesc) -> int:
    return int(lib().pa_decode_multi_workspace_size(ctypes.byref(desc)))


class MultiCall:
    """pa_decode_multi with its arguments marshalled once; calling it only enqueues the kernels.

    q, out [N][Hq][D]; query_start int32 [B + 1] (rows of sequence b: query_start[b] ..
    query_start[b+1]-1, the last tokens of its context_lens[b] cached tokens)."""

    def __init__(self, q, query_start, k_cache, v_cache, block_tables, context_lens, scale, out,
                 max_query_len, k_scale=None, v_scale=None, max_context_len=0,
                 partition_tokens=0, workspace=None, stream=None):
        for t in (q, query_start, k_cache, v_cache, block_tables, context_lens, out):
            assert t.is_cuda and t.is_contiguous()
        assert query_start.dtype == torch.int32 and block_tables.dtype == torch.int32
        assert context_lens.dtype == torch.int32
        assert out.shape == q.shape and out.dtype == q.dtype
        NB, Hkv, bs, D = k_cache.shape
        assert tuple(v_cache.shape) == (NB, Hkv, D, bs), "v_cache must be [NB][Hkv][D][16]"
        B = block_tables.shape[0]
        assert q.shape[2] == D and context_lens.shape[0] == B and query_start.shape[0] == B + 1
        self._desc = multi_desc(q, k_cache, block_tables, max_query_len, max_context_len,
                                partition_tokens)
        need = pa_decode_multi_workspace_size(self._desc)
        st = _stream(stream)
        if workspace is None and need > 0:
            workspace = _workspace(need, q.device, st.value or 0)
        wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self._keep = (q, query_start, k_cache, v_cache, block_tables, context_lens, out, k_scale,
                      v_scale, workspace)
        self._ws = None if workspace is None else workspace.data_ptr()
        self._fn = lib().pa_decode_multi
        self._args = (ctypes.byref(self._desc), _ptr(q), _ptr(query_start), _ptr(k_cache),
                      _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                      _ptr(context_lens), ctypes.c_float(scale), _ptr(out), _ptr(workspace),
                      ctypes.c_size_t(wbytes), st)

    def __call__(self) -> None:
        if self._ws is not None:
            _plan_owner.pop(self._ws, None)          # its scratch overwrites a saved plan
        st = self._fn(*self._args)
        if st != PA_OK:
            _check("pa_decode_multi", st)


def pa_decode_multi(q, query_start, k_cache, v_cache, block_tables, context_lens, scale, out,
                    max_query_len, k_scale=None, v_scale=None, max_context_len=0,
                    partition_tokens=0, workspace=None, stream=None,
                    check=False) -> torch.Tensor:
    """Causal attention of several query tokens per sequence (speculative verification, prefill
    chunks) over the paged cache; returns out.
    check=True (tests): first validate query_start, tables and lengths on the host."""
    if check:
        contract.check_multi(_host(query_start), _host(block_tables), _host(context_lens),
                             k_cache.shape[0], q.shape[0], max_query_len, max_context_len)
    MultiCall(q, query_start, k_cache, v_cache, block_tables, context_lens, scale, out,
              max_query_len, k_scale, v_scale, max_context_len, partition_tokens, workspace,
              stream)()
    return out


class StepGraph:
    """A step made of prepared calls (AppendCall, DecodeCall, MultiCall, ...), captured once into
    a HIP graph (pa_graph_begin / pa_graph_end) and replayed with one launch per call of the
    object.  Every call must have been made with `stream` (a non-default torch stream) and run
    once outside the capture first.  Replays read and write the same buffers: update their data
    in place between replays."""

    def __init__(self, calls, stream):
        assert stream is not None and stream.cuda_stream != 0, "capture needs its own stream"
        L = lib()
        self._lib, self._calls = L, list(calls)
        self._stream = ctypes.c_void_p(stream.cuda_stream)
        _check("pa_graph_begin", L.pa_graph_begin(self._stream))
        graph = ctypes.c_void_p()
        try:
            for c in self._calls:
                c()
        finally:
            st = L.pa_graph_end(self._stream, ctypes.byref(graph))
        _check("pa_graph_end", st)
        self._graph = graph

    def __call__(self) -> None:
        st = self._lib.pa_graph_launch(self._graph, self._stream)
        if st != PA_OK:
            _check("pa_graph_launch", st)

    def __del__(self):
        g = getattr(self, "_graph", None)
        if g is not None and g.value:
            self._lib.pa_graph_destroy(g)
            self._graph = None


class BlockPool:
    """The library's host-side block pool (pa_pool_*): reference counts and copy-on-write for
    num_blocks physical blocks.  Refusals raise PaError and leave the pool unchanged."""

    def __init__(self, num_blocks: int):
        self._lib = lib()
        p = ctypes.c_void_p()
        _check("pa_pool_create", self._lib.pa_pool_create(int(num_blocks), ctypes.byref(p)))
        self._p = p

    def __del__(self):
        p = getattr(self, "_p", None)
        if p is not None and p.value:
            self._lib.pa_pool_destroy(p)
            self._p = None

    @staticmethod
    def _ids(blocks):
        arr = (ctypes.c_int32 * max(1, len(blocks)))(*[int(b) for b in blocks])
        return len(blocks), arr

    def free_blocks(self) -> int:
        return int(self._lib.pa_pool_free_blocks(self._p))

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_pool_refcount(self._p, int(block)))

    def alloc(self, n: int) -> list:
        arr = (ctypes.c_int32 * max(1, n))()
        _check("pa_pool_alloc", self._lib.pa_pool_alloc(self._p, int(n), arr))
        return list(arr[:n])

    def share(self, blocks) -> None:
        n, arr = self._ids(blocks)
        _check("pa_pool_share", self._lib.pa_pool_share(self._p, n, arr))

    def release(self, blocks) -> None:
        n, arr = self._ids(blocks)
        _check("pa_pool_release", self._lib.pa_pool_release(self._p, n, arr))

    def write(self, block: int):
        """(target block, whether block's content must first be copied into it)."""
        t, c = ctypes.c_int32(), ctypes.c_int32()
        _check("pa_pool_write", self._lib.pa_pool_write(self._p, int(block), ctypes.byref(t),
                                                        ctypes.byref(c)))
        return int(t.value), bool(c.value)

    def slot_for(self, table: list, pos: int, max_blocks: int):
        """Slot of token pos for a sequence with block list `table` (updated in place): returns
        (slot, (source, target) of the copy to make, or None)."""
        arr = (ctypes.c_int32 * max(1, max_blocks))(*[int(b) for b in table])
        nb = ctypes.c_int32(len(table))
        slot = ctypes.c_int64()
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        _check("pa_pool_slot_for", self._lib.pa_pool_slot_for(
            self._p, arr, ctypes.byref(nb), int(max_blocks), int(pos), ctypes.byref(slot),
            ctypes.byref(src), ctypes.byref(dst)))
        table[:] = list(arr[:nb.value])
        return int(slot.value), (None if src.value < 0 else (int(src.value), int(dst.value)))


def pa_copy_blocks(pairs, k_cache, v_cache, k_scale=None, v_scale=None, stream=None,
                   check=False) -> None:
    """Copy whole blocks (every KV head, K and V, fp8 scales) for int32 pairs [n][2] on the
    device: (source, target).  check=True (tests): first validate the pairs on the host."""
    for t in (pairs, k_cache, v_cache):
        assert t.is_cuda and t.is_contiguous()
    assert pairs.dtype == torch.int32 and pairs.dim() == 2 and pairs.shape[1] == 2
    if check:
        contract.check_copy_pairs(_host(pairs), k_cache.shape[0])
    st = lib().pa_copy_blocks(ctypes.byref(cache_desc(k_cache)), pairs.shape[0], _ptr(pairs),
                              _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                              _stream(stream))
    _check("pa_copy_blocks", st)

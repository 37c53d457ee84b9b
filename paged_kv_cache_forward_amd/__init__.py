"""Python binding for libpagedattn (argument marshalling only).

Every computation runs in the HIP library; this module turns torch tensors
into device pointers and shapes, passes the current HIP stream, and raises on
a non-OK status.  It never computes attention, slots or block tables itself,
and there is no fallback: if ``libpagedattn.so`` is missing, the first call
into the library raises ImportError (the module itself imports without it so
that ``paged_kv_cache_forward_amd.build`` can create it).

Functions carry the C names: ``pa_write_kv``, ``pa_copy_blocks``,
``pa_forward_workspace_size``, ``pa_forward``, ``pa_write_kv_forward``, ...; ``BlockAllocator`` wraps the
``pa_alloc_*`` / ``pa_seq_*`` calls.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

PA_OK, PA_ERR_ARG, PA_ERR_UNSUPPORTED, PA_ERR_OOM, PA_ERR_RANGE, PA_ERR_HIP = range(6)
PA_F32, PA_BF16, PA_FP8 = 0, 1, 2
_STATUS = {1: "PA_ERR_ARG", 2: "PA_ERR_UNSUPPORTED", 3: "PA_ERR_OOM", 4: "PA_ERR_RANGE", 5: "PA_ERR_HIP"}


class PagedAttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class OutOfBlocks(PagedAttnError):
    pass


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class TraceRecord(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char_p), ("ms", ctypes.c_float)]


class AllocStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("blocks_total", "blocks_free", "blocks_used", "blocks_shared",
                 "tokens_logical", "slots_logical", "slots_physical")]


class PrefixStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("blocks_registered", "registered_free", "lookups", "hit_blocks", "evictions")]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_pi32, _pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
_pdesc = ctypes.POINTER(CacheDesc)

_SIGS = {
    "pa_version": (ctypes.c_char_p, []),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_write_kv": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _pdesc, _vp]),
    "pa_copy_blocks": (_i32, [_vp, _vp, _vp, _i32, _pdesc, _vp]),
    "pa_forward_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _pdesc]),
    "pa_forward": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                          _pdesc, ctypes.c_float, _i32, _vp, _sz, _vp]),
    "pa_write_kv_forward": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32,
                                   _i32, _i32, _pdesc, ctypes.c_float, _i32, _vp, _sz, _vp]),
    "pa_write_kv_forward_shared": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32,
                                          _i32, _i32, _i32, _i32, _pdesc, ctypes.c_float, _i32, _vp, _sz, _vp]),
    "pa_forward_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                  _pdesc, ctypes.c_float, _i32, _vp]),
    "pa_forward_shared_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _pdesc]),
    "pa_forward_shared": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                 _pdesc, ctypes.c_float, _i32, _vp, _sz, _vp]),
    "pa_trace_enable": (_i32, [_i32]),
    "pa_trace_read": (_i32, [ctypes.POINTER(TraceRecord), _i32, _pi32]),
    "pa_trace_clock": (_i32, [_vp, ctypes.POINTER(ctypes.c_float)]),
    "pa_alloc_create": (_i32, [_i32, _i32, _pi32, ctypes.POINTER(_vp)]),
    "pa_alloc_destroy": (None, [_vp]),
    "pa_seq_create": (_i32, [_vp, _pi32]),
    "pa_seq_fork": (_i32, [_vp, _i32, _i32, _pi32]),
    "pa_seq_append": (_i32, [_vp, _i32, _i32, _pi64, _pi32, _i32, _pi32]),
    "pa_seq_free": (_i32, [_vp, _i32]),
    "pa_seq_block_table": (_i32, [_vp, _i32, _pi32, _i32, _pi32, _pi32]),
    "pa_alloc_stats": (_i32, [_vp, ctypes.POINTER(AllocStats)]),
    "pa_block_refcount": (_i32, [_vp, _i32]),
    "pa_alloc_shared_blocks": (_i32, [_vp, _pi32, _i32, _pi32]),
    "pa_alloc_free_list": (_i32, [_vp, _pi32, _i32, _pi32]),
    "pa_prefix_register": (_i32, [_vp, _i32, _pi32, _i32]),
    "pa_prefix_lookup": (_i32, [_vp, _pi32, _i32, _pi32, _pi32]),
    "pa_prefix_stats": (_i32, [_vp, ctypes.POINTER(PrefixStats)]),
}

_LIB = None


def _load():
    """Load libpagedattn.so (once).  There is no fallback: a missing library is an error."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run paged_kv_cache_forward_amd.build.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def __getattr__(name):
    # `paged_kv_cache_forward_amd.lib` is the loaded library; loading happens on
    # first use so that the `build` submodule can be imported before it exists.
    if name == "lib":
        return _load()
    raise AttributeError(name)


EXPORTED = tuple(_SIGS)


def _check(status):
    if status != PA_OK:
        msg = _load().pa_last_error().decode()
        if status == PA_ERR_OOM:
            raise OutOfBlocks(status, msg)
        raise PagedAttnError(status, msg)


def version():
    return _load().pa_version().decode()


# -- device calls (torch tensors) ---------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def cache_desc(k_cache):
    """Descriptor of a pool tensor: [num_blocks][num_kv_heads][16][head_dim] (fp32 / bf16), or a
    quantised pool, uint8 of shape [num_blocks][num_kv_heads][16 * head_dim + 16]: a size only; its
    bytes are the plane of E4M3 code tiles, then the plane of row exponents (pagedattn.h)."""
    torch = _torch()
    if k_cache.dtype == torch.uint8:
        if k_cache.dim() != 3 or (k_cache.shape[2] - 16) % 16:
            raise ValueError("an fp8 pool is uint8 [num_blocks][num_kv_heads][16 * head_dim + 16]")
        nb, hkv, tile = k_cache.shape
        return CacheDesc(nb, hkv, (tile - 16) // 16, 16, PA_FP8)
    nb, hkv, bs, d = k_cache.shape
    return CacheDesc(nb, hkv, d, bs, _dtype_code(k_cache))


def fp8_pool_shape(num_blocks, num_kv_heads, head_dim):
    """Shape of a quantised (fp8) pool tensor (uint8)."""
    return (num_blocks, num_kv_heads, 16 * head_dim + 16)


def _row_dtype(k_cache):
    """Element type of k/v/q/out rows for this cache (bf16 for an fp8 pool)."""
    torch = _torch()
    return torch.bfloat16 if k_cache.dtype == torch.uint8 else k_cache.dtype


def pa_write_kv(k, v, k_cache, v_cache, slot_mapping, stream=None, bind=False):
    torch = _torch()
    desc = cache_desc(k_cache)
    if k.dtype != _row_dtype(k_cache) or v.dtype != k.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("k, v and the caches must share one dtype (bf16 rows for an fp8 cache)")
    if v_cache.shape != k_cache.shape or v.shape != k.shape:
        raise ValueError("K and V shapes differ")
    T = k.shape[0]
    if k.dim() != 3 or k.shape[1:] != (desc.num_kv_heads, desc.head_dim) or slot_mapping.shape != (T,):
        raise ValueError("k/v must be [T][num_kv_heads][head_dim] and slot_mapping [T]")
    return _call("pa_write_kv", (_dev(k, "k"), _dev(v, "v"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dev(slot_mapping, "slot_mapping", torch.int64), T, ctypes.byref(desc),
                           _stream(stream)), (desc,), bind)


def pa_copy_blocks(k_cache, v_cache, pairs, stream=None, bind=False):
    torch = _torch()
    desc = cache_desc(k_cache)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n][2]")
    return _call("pa_copy_blocks", (_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                              _dev(pairs, "pairs", torch.int32), pairs.shape[0], ctypes.byref(desc),
                              _stream(stream)), (desc,), bind)


def pa_forward_workspace_size(num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, k_cache):
    desc = cache_desc(k_cache)
    return int(_load().pa_forward_workspace_size(num_seqs, num_tokens, num_q_heads, max_seq_len,
                                             max_query_len, ctypes.byref(desc)))


def new_workspace(nbytes, device):
    """A uint8 device tensor of ``nbytes`` for ``pa_forward``'s split-KV partials."""
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def pa_forward(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, cached_lens,
               max_seq_len, max_query_len, scale, causal=True, workspace=None, stream=None, bind=False):
    """Attention for the super-batch; ``out`` is written in place.

    ``workspace`` is a uint8 device tensor of at least
    ``pa_forward_workspace_size(...)`` bytes (contents need no initialisation);
    when omitted, one is allocated here from torch's caching allocator.
    """
    torch = _torch()
    desc = cache_desc(k_cache)
    T, Hq, D = q.shape
    if out.shape != q.shape or out.dtype != q.dtype or q.dtype != _row_dtype(k_cache):
        raise ValueError("out must match q, and q the cache dtype (bf16 for an fp8 cache)")
    S = seq_lens.shape[0]
    if query_start_loc.shape != (S + 1,) or cached_lens.shape != (S,) or block_tables.shape[0] != S:
        raise ValueError("metadata shapes do not match num_seqs")
    need = pa_forward_workspace_size(S, T, Hq, max_seq_len, max_query_len, k_cache)
    if workspace is None and need > 0:
        workspace = new_workspace(need, q.device)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return _call("pa_forward", (_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                          _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
                          _dev(seq_lens, "seq_lens", torch.int32),
                          _dev(query_start_loc, "query_start_loc", torch.int32),
                          _dev(cached_lens, "cached_lens", torch.int32), S, T, Hq, int(max_seq_len),
                          int(max_query_len), ctypes.byref(desc), float(scale), int(bool(causal)),
                          ws_ptr, ws_bytes, _stream(stream)), (desc, workspace), bind)


def _write_kv_forward_args(k, v, slot_mapping, out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                           cached_lens, max_seq_len, max_query_len, scale, causal, workspace, stream, need=None):
    torch = _torch()
    desc = cache_desc(k_cache)
    T, Hq, D = q.shape
    if k.dtype != _row_dtype(k_cache) or v.dtype != k.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("k, v and the caches must share one dtype (bf16 rows for an fp8 cache)")
    if v_cache.shape != k_cache.shape or v.shape != k.shape or k.dim() != 3 or k.shape[0] != T:
        raise ValueError("k/v must be [T][num_kv_heads][head_dim] with q's T")
    if k.shape[1:] != (desc.num_kv_heads, desc.head_dim) or slot_mapping.shape != (T,):
        raise ValueError("k/v must be [T][num_kv_heads][head_dim] and slot_mapping [T]")
    if out.shape != q.shape or out.dtype != q.dtype or q.dtype != _row_dtype(k_cache):
        raise ValueError("out must match q, and q the cache dtype (bf16 for an fp8 cache)")
    S = seq_lens.shape[0]
    if query_start_loc.shape != (S + 1,) or cached_lens.shape != (S,) or block_tables.shape[0] != S:
        raise ValueError("metadata shapes do not match num_seqs")
    if need is None:
        need = pa_forward_workspace_size(S, T, Hq, max_seq_len, max_query_len, k_cache)
    if workspace is None and need > 0:
        workspace = new_workspace(need, q.device)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    # the descriptor and the workspace stay referenced by the tuple for as long as it is used
    return (_dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping", torch.int64), _dev(out, "out"),
            _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
            _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
            _dev(seq_lens, "seq_lens", torch.int32), _dev(query_start_loc, "query_start_loc", torch.int32),
            _dev(cached_lens, "cached_lens", torch.int32), S, T, Hq, int(max_seq_len), int(max_query_len),
            ctypes.byref(desc), float(scale), int(bool(causal)), ws_ptr, ws_bytes, _stream(stream)), (desc, workspace)


def pa_write_kv_forward(k, v, slot_mapping, out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                        cached_lens, max_seq_len, max_query_len, scale, causal=True, workspace=None, stream=None,
                        bind=False):
    """``pa_write_kv`` then ``pa_forward`` in one call (a single-token batch fuses the write into the
    decode); the workspace is ``pa_forward``'s."""
    args, keep = _write_kv_forward_args(k, v, slot_mapping, out, q, k_cache, v_cache, block_tables, seq_lens,
                                        query_start_loc, cached_lens, max_seq_len, max_query_len, scale, causal,
                                        workspace, stream)
    return _call("pa_write_kv_forward", args, keep, bind)


def _call(name, args, keep, bind):
    """Issue library call `name` with marshalled `args`, or with ``bind`` return it as a BoundCall."""
    if bind:
        return BoundCall(name, args, keep)
    _check(getattr(_load(), name)(*args))
    return None


class BoundCall:
    """One library call with its arguments marshalled once: calling it issues the same call again.

    The device calls take ``bind=True`` to return one instead of issuing the call.

    For a serving loop whose tensors stay where they are between steps (their
    contents may change): the per-call cost is the C call alone.  The tensors
    and the stream must outlive the object; it keeps the workspace and the
    cache descriptor alive itself."""

    def __init__(self, name, args, keep):
        self._fn = getattr(_load(), name)
        self._args = args
        self._keep = keep

    def __call__(self):
        _check(self._fn(*self._args))


def pa_forward_shared_workspace_size(num_seqs, num_tokens, num_q_heads, max_seq_len, max_query_len, k_cache):
    desc = cache_desc(k_cache)
    return int(_load().pa_forward_shared_workspace_size(num_seqs, num_tokens, num_q_heads, max_seq_len,
                                                        max_query_len, ctypes.byref(desc)))


def pa_forward_shared(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, cached_lens,
                      shared_blocks, max_seq_len, max_query_len, scale, causal=True, workspace=None, stream=None, bind=False):
    """pa_forward for a batch whose sequences share prefix blocks: ``shared_blocks`` (int32 device
    tensor [num_seqs]) gives the leading blocks each sequence has in common with the previous one
    (``BlockAllocator.shared_blocks``)."""
    torch = _torch()
    desc = cache_desc(k_cache)
    T, Hq, D = q.shape
    if out.shape != q.shape or out.dtype != q.dtype or q.dtype != _row_dtype(k_cache):
        raise ValueError("out must match q, and q the cache dtype (bf16 for an fp8 cache)")
    S = seq_lens.shape[0]
    if (query_start_loc.shape != (S + 1,) or cached_lens.shape != (S,) or block_tables.shape[0] != S
            or shared_blocks.shape != (S,)):
        raise ValueError("metadata shapes do not match num_seqs")
    need = pa_forward_shared_workspace_size(S, T, Hq, max_seq_len, max_query_len, k_cache)
    if workspace is None and need > 0:
        workspace = new_workspace(need, q.device)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return _call("pa_forward_shared", (_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"),
                                     _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables", torch.int32),
                                     block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32),
                                     _dev(query_start_loc, "query_start_loc", torch.int32),
                                     _dev(cached_lens, "cached_lens", torch.int32),
                                     _dev(shared_blocks, "shared_blocks", torch.int32), S, T, Hq, int(max_seq_len),
                                     int(max_query_len), ctypes.byref(desc), float(scale), int(bool(causal)),
                                     ws_ptr, ws_bytes, _stream(stream)), (desc, workspace), bind)


def pa_write_kv_forward_shared(k, v, slot_mapping, out, q, k_cache, v_cache, block_tables, seq_lens,
                               query_start_loc, cached_lens, shared_blocks, max_seq_len, max_query_len, scale,
                               causal=True, workspace=None, stream=None, bind=False):
    """``pa_write_kv`` then ``pa_forward_shared`` in one call (fused when the shared-prefix decode
    takes the batch); the workspace is ``pa_forward_shared``'s."""
    torch = _torch()
    S = seq_lens.shape[0]
    if shared_blocks.shape != (S,):
        raise ValueError("shared_blocks must be [num_seqs]")
    T, Hq, _ = q.shape
    if workspace is None:
        need = pa_forward_shared_workspace_size(S, T, Hq, max_seq_len, max_query_len, k_cache)
        workspace = new_workspace(need, q.device) if need > 0 else None
    args, keep = _write_kv_forward_args(k, v, slot_mapping, out, q, k_cache, v_cache, block_tables, seq_lens,
                                        query_start_loc, cached_lens, max_seq_len, max_query_len, scale, causal,
                                        workspace, stream, need=0)
    # pa_write_kv_forward's arguments with shared_blocks after cached_lens
    args = args[:12] + (_dev(shared_blocks, "shared_blocks", torch.int32),) + args[12:]
    return _call("pa_write_kv_forward_shared", args, keep, bind)


NOALLOC_MAX_SCRATCH = 64 << 20      # PA_FORWARD_NOALLOC_MAX_SCRATCH


def pa_forward_noalloc(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, cached_lens,
                       max_seq_len, max_query_len, scale, causal=True, stream=None):
    """pa_forward without a workspace: the library's own per-GPU scratch array is used, and nothing
    is allocated (here or in the library).  Batches needing more than NOALLOC_MAX_SCRATCH bytes of
    scratch raise PA_ERR_UNSUPPORTED."""
    torch = _torch()
    desc = cache_desc(k_cache)
    T, Hq, D = q.shape
    if out.shape != q.shape or out.dtype != q.dtype or q.dtype != _row_dtype(k_cache):
        raise ValueError("out must match q, and q the cache dtype (bf16 for an fp8 cache)")
    S = seq_lens.shape[0]
    if query_start_loc.shape != (S + 1,) or cached_lens.shape != (S,) or block_tables.shape[0] != S:
        raise ValueError("metadata shapes do not match num_seqs")
    _check(_load().pa_forward_noalloc(_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"),
                                      _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables", torch.int32),
                                      block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32),
                                      _dev(query_start_loc, "query_start_loc", torch.int32),
                                      _dev(cached_lens, "cached_lens", torch.int32), S, T, Hq, int(max_seq_len),
                                      int(max_query_len), ctypes.byref(desc), float(scale), int(bool(causal)),
                                      _stream(stream)))


# -- tracing ---------------------------------------------------------------------

def pa_trace_enable(on=True):
    """Per-kernel HIP-event timing of every later device call (see pa_trace_read)."""
    _check(_load().pa_trace_enable(1 if on else 0))


def pa_trace_read(cap=4096):
    """Waits for the recorded events; returns [(kernel name, ms), ...] in launch order and clears them."""
    buf = (TraceRecord * cap)()
    n = ctypes.c_int32()
    _check(_load().pa_trace_read(buf, cap, ctypes.byref(n)))
    return [(buf[k].kernel.decode(), float(buf[k].ms)) for k in range(n.value)]


def pa_trace_clock(stream=None):
    """The shader clock (MHz) a short probe kernel runs at now (waits for the stream)."""
    mhz = ctypes.c_float()
    _check(_load().pa_trace_clock(_stream(stream), ctypes.byref(mhz)))
    return float(mhz.value)


# -- host allocator -------------------------------------------------------------

class BlockAllocator:
    """The library's host block allocator (refcounts, sharing, copy-on-write)."""

    def __init__(self, num_blocks, block_size=16, free_order=None):
        self._h = ctypes.c_void_p()
        order = None
        if free_order is not None:
            self._order = np.ascontiguousarray(free_order, dtype=np.int32)
            order = self._order.ctypes.data_as(_pi32)
        _check(_load().pa_alloc_create(num_blocks, block_size, order, ctypes.byref(self._h)))
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and h.value and _LIB is not None:   # at interpreter exit the module may be torn down first
            _LIB.pa_alloc_destroy(h)
            self._h = ctypes.c_void_p()

    def create(self):
        sid = ctypes.c_int32()
        _check(_load().pa_seq_create(self._h, ctypes.byref(sid)))
        return sid.value

    def fork(self, parent, share_tokens):
        sid = ctypes.c_int32()
        _check(_load().pa_seq_fork(self._h, parent, share_tokens, ctypes.byref(sid)))
        return sid.value

    def append(self, seq, n_tokens, cow_cap=4):
        """Returns (slots int64 array, list of (src, dst) copy-on-write pairs)."""
        slots = np.empty(max(n_tokens, 1), dtype=np.int64)
        pairs = np.empty(2 * cow_cap, dtype=np.int32)
        n_cow = ctypes.c_int32()
        _check(_load().pa_seq_append(self._h, seq, n_tokens, slots.ctypes.data_as(_pi64),
                                 pairs.ctypes.data_as(_pi32), cow_cap, ctypes.byref(n_cow)))
        return slots[:n_tokens], [(int(pairs[2 * k]), int(pairs[2 * k + 1])) for k in range(n_cow.value)]

    def free_seq(self, seq):
        _check(_load().pa_seq_free(self._h, seq))

    def block_table(self, seq):
        nb, ln = ctypes.c_int32(), ctypes.c_int32()
        _check(_load().pa_seq_block_table(self._h, seq, None, 0, ctypes.byref(nb), ctypes.byref(ln)))
        out = np.empty(max(nb.value, 1), dtype=np.int32)
        _check(_load().pa_seq_block_table(self._h, seq, out.ctypes.data_as(_pi32), nb.value,
                                      ctypes.byref(nb), ctypes.byref(ln)))
        return out[:nb.value].tolist()

    def length(self, seq):
        nb, ln = ctypes.c_int32(), ctypes.c_int32()
        _check(_load().pa_seq_block_table(self._h, seq, None, 0, ctypes.byref(nb), ctypes.byref(ln)))
        return ln.value

    def stats(self):
        st = AllocStats()
        _check(_load().pa_alloc_stats(self._h, ctypes.byref(st)))
        return {name: getattr(st, name) for name, _ in AllocStats._fields_}

    def shared_blocks(self, seq_ids):
        """Leading blocks each of ``seq_ids`` (batch order) shares with the one before it (int32 array)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        out = np.zeros(max(len(ids), 1), dtype=np.int32)
        _check(_load().pa_alloc_shared_blocks(self._h, ids.ctypes.data_as(_pi32), len(ids), out.ctypes.data_as(_pi32)))
        return out[:len(ids)]

    def refcount(self, block):
        return int(_load().pa_block_refcount(self._h, block))

    def free_list(self):
        n = ctypes.c_int32()
        _check(_load().pa_alloc_free_list(self._h, None, 0, ctypes.byref(n)))
        out = np.empty(max(n.value, 1), dtype=np.int32)
        _check(_load().pa_alloc_free_list(self._h, out.ctypes.data_as(_pi32), n.value, ctypes.byref(n)))
        return out[:n.value].tolist()

    # prefix caching
    def prefix_register(self, seq, tokens, n_tokens=None):
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        n = len(tok) if n_tokens is None else n_tokens
        _check(_load().pa_prefix_register(self._h, seq, tok.ctypes.data_as(_pi32), n))

    def prefix_lookup(self, tokens, n_tokens=None):
        """Returns (new sequence id, tokens already cached)."""
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        n = len(tok) if n_tokens is None else n_tokens
        sid, cached = ctypes.c_int32(), ctypes.c_int32()
        _check(_load().pa_prefix_lookup(self._h, tok.ctypes.data_as(_pi32), n, ctypes.byref(sid),
                                        ctypes.byref(cached)))
        return sid.value, cached.value

    def prefix_stats(self):
        st = PrefixStats()
        _check(_load().pa_prefix_stats(self._h, ctypes.byref(st)))
        return {name: getattr(st, name) for name, _ in PrefixStats._fields_}

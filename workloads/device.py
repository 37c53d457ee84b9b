"""GPU-side harness: run one engine step of a workload through the library.

Test and benchmark infrastructure (tests, smoke and bench.py use it; the
library never imports it).  Replays the workload's allocator trace on the
library's host allocator (``workloads.drive``), puts the pools, queries and
metadata in device memory (torch tensors), stores the cached tokens with
``pa_write_kv``, and then performs the step itself: ``pa_copy_blocks`` for
copy-on-write pairs, then ``pa_write_kv_forward`` (the new tokens' K/V and
attention; or ``pa_write_kv`` and ``pa_forward`` separately).  Every step of the path runs in the HIP library; this module
only marshals.
"""

import numpy as np

import paged_kv_cache_forward_amd as pa

from . import drive

BF16_NAN_BITS = 0x7FC0


class DeviceRun:
    """One workload's device state; ``copies`` > 1 keeps that many identical K/V pools.

    Steps can rotate through the copies (``use``) so that consecutive steps
    read different HBM and nothing is served from the 256 MB last-level cache
    (the way successive layers of a model read different caches).
    """

    def __init__(self, wl, device="cuda:0", fill="nan", free_order=None, table_stride=None, copies=1,
                 max_seq_len=None, shared=False, fused=True):
        import torch
        self.torch = torch
        self.wl = wl
        self.dev = torch.device(device)
        self.tdtype = torch.float32 if wl.dtype == "f32" else torch.bfloat16
        order = wl.free_order if free_order is None else free_order
        self.alloc = pa.BlockAllocator(wl.num_blocks, wl.block_size, order)
        self.ids, self.ctx_slots, self.new_slots, self.cow = drive(wl, self.alloc)

        if wl.cache == "fp8":
            shape = pa.fp8_pool_shape(wl.pool_blocks, wl.num_kv_heads, wl.head_dim)
        else:
            shape = (wl.pool_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
        self.k_cache = self._pool(shape, fill)
        self.v_cache = self._pool(shape, fill)
        self.q = self.upload(wl.q)
        self.k_new = self.upload(wl.k_new)
        self.v_new = self.upload(wl.v_new)
        self.new_slots_d = torch.from_numpy(self.new_slots).to(self.dev)
        pairs = np.asarray(self.cow, dtype=np.int32).reshape(-1, 2)
        self.pairs_d = torch.from_numpy(pairs).to(self.dev)

        tables = [self.alloc.block_table(self.ids[h]) for h in wl.batch]
        width = max([len(t) for t in tables] + [1]) if table_stride is None else table_stride
        bt = np.full((len(tables), width), wl.guard_block, dtype=np.int32)
        for i, t in enumerate(tables):
            bt[i, :len(t)] = t
        self.tables = tables
        self.block_tables = torch.from_numpy(bt).to(self.dev)
        self.seq_lens = torch.from_numpy(wl.seq_lens.astype(np.int32)).to(self.dev)
        self.cached_lens = torch.from_numpy(wl.cached_lens.astype(np.int32)).to(self.dev)
        self.qsl = torch.from_numpy(wl.query_start_loc.astype(np.int32)).to(self.dev)
        self.out = torch.full_like(self.q, float("nan"))
        # host bound on the lengths passed to pa_forward (may exceed the workload's, e.g. to let
        # a captured step be replayed after the sequences grow)
        self.max_seq_len = wl.max_seq_len if max_seq_len is None else max_seq_len
        # shared: attention through pa_forward_shared, with the blocks each batch sequence shares
        # with the one before it as the host allocator reports them
        self.shared = shared
        self.fused = fused
        self._bound_calls = {}
        self.shared_blocks = self.alloc.shared_blocks([self.ids[h] for h in wl.batch])
        self.shared_blocks_d = torch.from_numpy(self.shared_blocks).to(self.dev)
        self.workspace = None
        self.ensure_workspace()
        self.fill_context()
        self.pools = [(self.k_cache, self.v_cache)]
        for _ in range(1, copies):
            self.pools.append((self.k_cache.clone(), self.v_cache.clone()))

    def ensure_workspace(self):
        """Size the workspace for the call as the library would make it now.

        The size depends on the routing knobs in the environment (PA_VERIFY,
        PA_DECODE, ...): call this again after changing them.  A larger
        workspace replaces the old one (and the calls bound to it).
        """
        wl = self.wl
        size = pa.pa_forward_shared_workspace_size if self.shared else pa.pa_forward_workspace_size
        ws = size(wl.num_seqs, wl.num_tokens, wl.num_q_heads, self.max_seq_len, wl.max_query_len, self.k_cache)
        if ws and (self.workspace is None or self.workspace.numel() < ws):
            self.workspace = pa.new_workspace(ws, self.dev)
            self._bound_calls = {}

    def use(self, copy):
        """Make pool copy ``copy`` the one later calls read and write."""
        self.k_cache, self.v_cache = self.pools[copy % len(self.pools)]

    def _pool(self, shape, fill):
        torch = self.torch
        if self.wl.cache == "fp8":   # 0xff: a NaN code and a NaN scale in every byte
            return torch.full(shape, 0 if fill == "zero" else 0xFF, dtype=torch.uint8, device=self.dev)
        if fill == "zero":
            return torch.zeros(shape, dtype=self.tdtype, device=self.dev)
        if self.tdtype == torch.float32:
            return torch.full(shape, float("nan"), dtype=torch.float32, device=self.dev)
        return torch.full(shape, BF16_NAN_BITS, dtype=torch.int16, device=self.dev).view(torch.bfloat16)

    def upload(self, arr):
        torch = self.torch
        if self.wl.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(arr)).to(self.dev)
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(self.dev).view(torch.bfloat16)

    def fill_context(self, chunk_tokens=1 << 18):
        """Store every cached token (the state before this step) with pa_write_kv."""
        torch = self.torch
        wl = self.wl
        n = len(wl.ctx_k)
        for a in range(0, n, chunk_tokens):
            b = min(n, a + chunk_tokens)
            k = self.upload(wl.ctx_k[a:b])
            v = self.upload(wl.ctx_v[a:b])
            s = torch.from_numpy(self.ctx_slots[a:b]).to(self.dev)
            pa.pa_write_kv(k, v, self.k_cache, self.v_cache, s)
            del k, v, s

    # Each library call's arguments are marshalled once per (call, pool copy, stream) and the
    # bound call re-issued (pa.BoundCall): the tensors stay where they are between steps.
    def _bound(self, what, stream, make):
        s = self.torch.cuda.current_stream() if stream is None else stream
        key = (what, self.k_cache.data_ptr(), s.cuda_stream)
        call = self._bound_calls.get(key)
        if call is None:
            call = make(s)
            self._bound_calls[key] = call
        return call

    def step_writes(self, stream=None):
        """This step's cache updates: copy-on-write copies, then the new tokens' K/V."""
        if self.pairs_d.shape[0]:
            self._bound("copy", stream, lambda s: pa.pa_copy_blocks(self.k_cache, self.v_cache, self.pairs_d,
                                                                    stream=s, bind=True))()
        self._bound("write", stream, lambda s: pa.pa_write_kv(self.k_new, self.v_new, self.k_cache, self.v_cache,
                                                              self.new_slots_d, stream=s, bind=True))()

    def forward(self, stream=None):
        wl = self.wl
        if self.shared:
            self._bound("shared", stream, lambda s: pa.pa_forward_shared(
                self.out, self.q, self.k_cache, self.v_cache, self.block_tables, self.seq_lens, self.qsl,
                self.cached_lens, self.shared_blocks_d, self.max_seq_len, wl.max_query_len, wl.scale, wl.causal,
                workspace=self.workspace, stream=s, bind=True))()
            return
        self._bound("forward", stream, lambda s: pa.pa_forward(
            self.out, self.q, self.k_cache, self.v_cache, self.block_tables, self.seq_lens, self.qsl,
            self.cached_lens, self.max_seq_len, wl.max_query_len, wl.scale, wl.causal, workspace=self.workspace,
            stream=s, bind=True))()

    def step(self, stream=None):
        """One engine step.  With ``fused`` (the default) the new tokens' write and attention are one
        ``pa_write_kv_forward`` (``pa_write_kv_forward_shared``) call: the library fuses the write into
        a single-token batch's decode; otherwise ``pa_write_kv`` then ``pa_forward``
        (``pa_forward_shared``)."""
        if not self.fused:
            self.step_writes(stream)
            self.forward(stream)
            return
        wl = self.wl
        if self.pairs_d.shape[0]:
            self._bound("copy", stream, lambda s: pa.pa_copy_blocks(self.k_cache, self.v_cache, self.pairs_d,
                                                                    stream=s, bind=True))()
        if self.shared:
            self._bound("fused_shared", stream, lambda s: pa.pa_write_kv_forward_shared(
                self.k_new, self.v_new, self.new_slots_d, self.out, self.q, self.k_cache, self.v_cache,
                self.block_tables, self.seq_lens, self.qsl, self.cached_lens, self.shared_blocks_d,
                self.max_seq_len, wl.max_query_len, wl.scale, wl.causal, workspace=self.workspace, stream=s,
                bind=True))()
            return
        self._bound("fused", stream, lambda s: pa.pa_write_kv_forward(
            self.k_new, self.v_new, self.new_slots_d, self.out, self.q, self.k_cache, self.v_cache,
            self.block_tables, self.seq_lens, self.qsl, self.cached_lens, self.max_seq_len, wl.max_query_len,
            wl.scale, wl.causal, workspace=self.workspace, stream=s, bind=True))()

    # -- host copies for checking -------------------------------------------
    def host(self, t):
        torch = self.torch
        t = t.detach()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    def out_f64(self):
        torch = self.torch
        return self.out.detach().to(torch.float64).cpu().numpy()

"""The C-ABI library loads on a machine without a GPU and exports every call its header declares."""

import os
import re

from helpers import ensure_library

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pagedattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(pa_[a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("pa_write_kv", "pa_copy_blocks", "pa_forward", "pa_forward_workspace_size",
                     "pa_alloc_create", "pa_seq_append", "pa_seq_fork", "pa_seq_free", "pa_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    pa = ensure_library()
    for name in declared_functions():
        assert hasattr(pa.lib, name), f"{name} declared in the header but not exported"
    assert set(declared_functions()) == set(pa.EXPORTED)


def test_version_and_error_strings():
    pa = ensure_library()
    assert "gfx950" in pa.version()
    assert isinstance(pa.lib.pa_last_error().decode(), str)


def test_host_argument_errors_without_a_gpu():
    # Argument checks run before any HIP call, so they work with no device present.
    import ctypes
    pa = ensure_library()
    desc = pa.CacheDesc(32, 2, 64, 8, pa.PA_F32)          # block_size 8: not built
    st = pa.lib.pa_write_kv(None, None, None, None, None, 4, ctypes.byref(desc), None)
    assert st == pa.PA_ERR_UNSUPPORTED and "block_size" in pa.lib.pa_last_error().decode()
    desc = pa.CacheDesc(32, 2, 96, 16, pa.PA_BF16)        # head_dim 96: not built for attention
    assert pa.lib.pa_forward_workspace_size(4, 4, 4, 100, 1, ctypes.byref(desc)) == 0
    st = pa.lib.pa_forward(None, None, None, None, None, 1, None, None, None, 4, 4, 4, 100, 1,
                           ctypes.byref(desc), 0.1, 1, None, 0, None)
    assert st == pa.PA_ERR_UNSUPPORTED
    desc = pa.CacheDesc(32, 2, 64, 16, pa.PA_BF16)
    st = pa.lib.pa_forward(None, None, None, None, None, 1, None, None, None, 4, 4, 6, 100, 1,
                           ctypes.byref(desc), 0.1, 1, None, 0, None)   # 6 q heads / 2 kv heads = 3
    assert st == pa.PA_ERR_UNSUPPORTED
    st = pa.lib.pa_forward(None, None, None, None, None, 1, None, None, None, 4, 4, 5, 100, 1,
                           ctypes.byref(desc), 0.1, 1, None, 0, None)   # not a multiple
    assert st == pa.PA_ERR_ARG
    st = pa.lib.pa_forward(None, None, None, None, None, 1, None, None, None, 4, 4, 4, 100, 1,
                           ctypes.byref(desc), 0.1, 1, None, 0, None)   # NULL device pointers
    assert st == pa.PA_ERR_ARG
    # empty batch is a no-op
    st = pa.lib.pa_forward(None, None, None, None, None, 1, None, None, None, 0, 0, 4, 0, 0,
                           ctypes.byref(desc), 0.1, 1, None, 0, None)
    assert st == pa.PA_OK


def _r256(n):
    return (n + 255) // 256 * 256


def test_workspace_size_follows_the_split(monkeypatch):
    """Partitioned decode: partial accumulators [S][Hq][P][D] fp32, then (max, sum) [S][Hq][P][2]."""
    import ctypes
    monkeypatch.setenv("PA_DECODE", "partition")
    pa = ensure_library()
    desc = pa.CacheDesc(20000, 8, 128, 16, pa.PA_BF16)
    small = pa.lib.pa_forward_workspace_size(64, 64, 32, 200, 1, ctypes.byref(desc))
    big = pa.lib.pa_forward_workspace_size(64, 64, 32, 4096, 1, ctypes.byref(desc))
    assert small == 0 and big > 0
    parts = [p for p in range(1, 4097) if big == _r256(64 * 32 * p * 128 * 4) + _r256(64 * 32 * p * 8)]
    assert len(parts) == 1 and parts[0] > 1


def test_workspace_size_of_the_balanced_decode(monkeypatch):
    """Balanced decode: part table [S][2] int32, then partials for S + Wg slots per KV head
    ([Hkv][S+Wg][G][D] fp32 and [Hkv][S+Wg][G][2] fp32), Wg = min(total waves / Hkv, S * tiles)."""
    import ctypes
    monkeypatch.delenv("PA_DECODE", raising=False)
    pa = ensure_library()
    desc = pa.CacheDesc(20000, 8, 128, 16, pa.PA_BF16)

    def expect(S, Hq, wg):
        return _r256(S * 8) + _r256((S + wg) * Hq * 128 * 4) + _r256((S + wg) * Hq * 8)

    for total, S, L, wg in [(None, 64, 4096, 128), (None, 3, 20, 6), ("64", 64, 4096, 8), ("1", 5, 100, 1)]:
        if total is None:
            monkeypatch.delenv("PA_DECODE_TOTAL_WAVES", raising=False)
        else:
            monkeypatch.setenv("PA_DECODE_TOTAL_WAVES", total)
        got = pa.lib.pa_forward_workspace_size(S, S, 32, L, 1, ctypes.byref(desc))
        assert got == expect(S, 32, wg), (total, S, L, got)
    # over 1024 sequences the partitioned kernel takes over
    monkeypatch.delenv("PA_DECODE_TOTAL_WAVES", raising=False)
    got = pa.lib.pa_forward_workspace_size(2000, 2000, 32, 200, 1, ctypes.byref(desc))
    assert got == 0


def test_noalloc_host_checks_without_a_gpu():
    """pa_forward_noalloc checks its host arguments, and refuses a batch whose scratch exceeds the
    library's per-GPU array, before any HIP call."""
    import ctypes
    pa = ensure_library()
    desc = pa.CacheDesc(100, 8, 128, 16, pa.PA_BF16)
    st = pa.lib.pa_forward_noalloc(None, None, None, None, None, 1, None, None, None, 4, 4, 32, 100, 1,
                                   ctypes.byref(desc), 0.1, 1, None)
    assert st == pa.PA_ERR_ARG and "NULL" in pa.lib.pa_last_error().decode()
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: the call returns before launching
    S = 65536
    assert pa.lib.pa_forward_workspace_size(S, S, 32, 8192, 1, ctypes.byref(desc)) > pa.NOALLOC_MAX_SCRATCH
    st = pa.lib.pa_forward_noalloc(fake, fake, fake, fake, fake, 1, fake, fake, fake, S, S, 32, 8192, 1,
                                   ctypes.byref(desc), 0.1, 1, None)
    assert st == pa.PA_ERR_UNSUPPORTED and "scratch" in pa.lib.pa_last_error().decode()
    # empty batches are a no-op, as for pa_forward
    assert pa.lib.pa_forward_noalloc(None, None, None, None, None, 1, None, None, None, 0, 0, 32, 0, 0,
                                     ctypes.byref(desc), 0.1, 1, None) == pa.PA_OK


def test_write_kv_forward_host_checks_without_a_gpu():
    """pa_write_kv_forward checks its host arguments (NULL pointers, a short workspace) before any HIP
    call, and an empty batch is a no-op."""
    import ctypes
    pa = ensure_library()
    desc = pa.CacheDesc(100, 8, 128, 16, pa.PA_BF16)
    fn = pa.lib.pa_write_kv_forward
    st = fn(None, None, None, None, None, None, None, None, 1, None, None, None, 4, 4, 32, 100, 1,
            ctypes.byref(desc), 0.1, 1, None, 0, None)
    assert st == pa.PA_ERR_ARG and "NULL" in pa.lib.pa_last_error().decode()
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: the call returns before launching
    S = 64
    assert pa.lib.pa_forward_workspace_size(S, S, 32, 8192, 1, ctypes.byref(desc)) > 0
    st = fn(fake, fake, fake, fake, fake, fake, fake, fake, 1, fake, fake, fake, S, S, 32, 8192, 1,
            ctypes.byref(desc), 0.1, 1, fake, 16, None)
    assert st == pa.PA_ERR_ARG and "workspace" in pa.lib.pa_last_error().decode()
    st = fn(None, fake, fake, fake, fake, fake, fake, fake, 1, fake, fake, fake, S, S, 32, 8192, 1,
            ctypes.byref(desc), 0.1, 1, None, 0, None)
    assert st == pa.PA_ERR_ARG and "NULL" in pa.lib.pa_last_error().decode()
    assert fn(None, None, None, None, None, None, None, None, 1, None, None, None, 0, 0, 32, 0, 0,
              ctypes.byref(desc), 0.1, 1, None, 0, None) == pa.PA_OK


def test_write_kv_forward_shared_host_checks_without_a_gpu():
    """pa_write_kv_forward_shared refuses NULL pointers before any HIP call; an empty batch is a no-op."""
    import ctypes
    pa = ensure_library()
    desc = pa.CacheDesc(100, 8, 128, 16, pa.PA_BF16)
    fn = pa.lib.pa_write_kv_forward_shared
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: the calls return before launching
    st = fn(None, fake, fake, fake, fake, fake, fake, fake, 1, fake, fake, fake, fake, 64, 64, 32, 4096, 1,
            ctypes.byref(desc), 0.1, 1, fake, 1 << 30, None)
    assert st == pa.PA_ERR_ARG and "NULL" in pa.lib.pa_last_error().decode()
    st = fn(fake, fake, fake, fake, fake, fake, fake, fake, 1, fake, fake, fake, None, 64, 64, 32, 4096, 1,
            ctypes.byref(desc), 0.1, 1, fake, 1 << 30, None)
    assert st == pa.PA_ERR_ARG and "shared_blocks" in pa.lib.pa_last_error().decode()
    assert fn(None, None, None, None, None, None, None, None, 1, None, None, None, None, 0, 0, 32, 0, 0,
              ctypes.byref(desc), 0.1, 1, None, 0, None) == pa.PA_OK


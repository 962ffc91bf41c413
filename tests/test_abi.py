"""The C ABI without a GPU: libep.so loads, exports every entry point that
include/ep.h declares, and rejects bad arguments on the host before making any
HIP call (so these run on machines with no device)."""

import ctypes
import os
import re

import pytest

import bulk_async_tensor_amd as ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")

# fake device addresses: only their alignment matters, none is dereferenced
A16 = 0x7F0000000000
A4 = A16 + 4
ODD = A16 + 1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ep.LIB_PATH):
        pytest.fail("libep.so is not built (run __graft_entry__.build())")
    return ep.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 23
    for n in names:
        assert hasattr(lib, n), n
        assert n in ep._SIGNATURES, f"binding lacks {n}"


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(ep, "LIB_PATH", "/nonexistent/libep.so")
    monkeypatch.setattr(ep, "_lib", None)
    with pytest.raises(ep.EpLibraryMissing):
        ep.lib()


def test_num_cus_and_variant_settings(lib):
    assert lib.ep_set_num_cus(-1) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_set_num_cus(4097) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_set_num_cus(24) == 0 and lib.ep_get_num_cus() == 24
    assert lib.ep_set_num_cus(0) == 0 and lib.ep_get_num_cus() == 0
    assert lib.ep_set_variant(b"bogus") == ep.EP_ERR_UNSUPPORTED
    assert "bogus" in lib.ep_last_error().decode()
    for v in ep.VARIANTS:
        assert lib.ep_set_variant(v.encode()) == 0
        assert lib.ep_get_variant().decode() == v
    assert lib.ep_set_variant(b"auto") == 0


def test_slab_setting(lib):
    for v in (0, 1, 2, 4, 7, 8, 14, 16):
        assert lib.ep_set_slab(v) == 0 and lib.ep_get_slab() == v
    for v in (-1, 3, 5, 32):
        assert lib.ep_set_slab(v) == ep.EP_ERR_UNSUPPORTED
    assert lib.ep_set_slab(0) == 0


def test_workspace_bytes(lib):
    # the one-launch path needs no workspace: a few 1024-entry chunks, or up to 64 chunks with E > 64
    # and at most 12288 tokens
    assert lib.ep_layout_workspace_bytes(128, 8, 256) == 0
    assert lib.ep_layout_workspace_bytes(128, 2, 8) == 0
    assert lib.ep_layout_workspace_bytes(4096, 8, 256) == 0
    assert lib.ep_layout_workspace_bytes(8192, 8, 256) == 0
    assert lib.ep_layout_workspace_bytes(512, 8, 64) == 0
    assert lib.ep_layout_workspace_bytes(12288, 4, 128) == 0  # 48 chunks, at the token cap
    # past 12288 tokens two launches even within 64 chunks: 12289 x 4 -> 49 chunks of 256 tokens,
    # 49 * 256 * 4 = 50,176 (256-aligned); 20000 x 2 -> 40 chunks of 512 tokens
    assert lib.ep_layout_workspace_bytes(12289, 4, 256) == 49 * 256 * 4 + 49 * 4
    assert lib.ep_layout_workspace_bytes(20000, 2, 128) == 40 * 128 * 4 + 40 * 4
    # the two-launch path counts per chunk of 1024 // k tokens into a (chunk, expert) table,
    # 256-aligned, followed by one status word per chunk.  E <= 64 past four chunks:
    # 16384 x 6 -> 97 chunks of 170 tokens; 97 * 64 * 4 = 24,832 is already 256-aligned
    assert lib.ep_layout_workspace_bytes(16384, 6, 64) == 97 * 64 * 4 + 97 * 4
    # 513 x 8 = 4104 entries with E = 64: five chunks of 128 tokens
    assert lib.ep_layout_workspace_bytes(513, 8, 64) == 5 * 64 * 4 + 5 * 4
    # more than 64 chunks: 8193 x 8 -> 65 chunks of 128 tokens
    assert lib.ep_layout_workspace_bytes(8193, 8, 256) == 65 * 256 * 4 + 65 * 4
    # T=131072, k=8 -> 1024 chunks; 1024*256*4 = 1 MiB
    assert lib.ep_layout_workspace_bytes(131072, 8, 256) == 1024 * 256 * 4 + 1024 * 4
    # T=40000, k=32, E=1024 -> 32 tokens per chunk -> 1250 chunks; 1250*1024*4 = 5,120,000 (256-aligned)
    assert lib.ep_layout_workspace_bytes(40000, 32, 1024) == 1250 * 1024 * 4 + 1250 * 4
    assert lib.ep_layout_workspace_bytes(0, 8, 256) == 0
    assert lib.ep_layout_workspace_bytes(10, 0, 256) == 0


def layout(lib, idx=A4, T=16, k=2, E=8, counts=A4, offsets=A4, dest=A4, src=A4, status=A4, ws=A16, wsb=1 << 20):
    return lib.ep_layout(idx, T, k, E, counts, offsets, dest, src, status, ws, wsb, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(T=-1), ep.EP_ERR_INVALID_ARG),
        (dict(k=0), ep.EP_ERR_INVALID_ARG),
        (dict(k=33, E=64), ep.EP_ERR_INVALID_ARG),
        (dict(E=0), ep.EP_ERR_INVALID_ARG),
        (dict(E=1025), ep.EP_ERR_INVALID_ARG),
        (dict(k=9, E=8), ep.EP_ERR_INVALID_ARG),
        (dict(T=2**30, k=4), ep.EP_ERR_INVALID_ARG),
        (dict(counts=None), ep.EP_ERR_INVALID_ARG),
        (dict(offsets=None), ep.EP_ERR_INVALID_ARG),
        (dict(idx=None), ep.EP_ERR_INVALID_ARG),
        (dict(dest=None), ep.EP_ERR_INVALID_ARG),
        (dict(dest=ODD), ep.EP_ERR_ALIGNMENT),
        (dict(idx=ODD), ep.EP_ERR_ALIGNMENT),
        (dict(status=A4 + 2), ep.EP_ERR_ALIGNMENT),
        # shapes beyond the one-launch path need a workspace
        (dict(T=131072, k=8, E=256, ws=None), ep.EP_ERR_WORKSPACE),
        (dict(T=16384, k=6, E=64, ws=None), ep.EP_ERR_WORKSPACE),
        (dict(T=16384, k=6, E=64, wsb=97 * 64 * 4), ep.EP_ERR_WORKSPACE),
        (dict(T=131072, k=8, E=256, wsb=16), ep.EP_ERR_WORKSPACE),
        (dict(T=131072, k=8, E=256, ws=A4, wsb=1 << 24), ep.EP_ERR_ALIGNMENT),
    ],
)
def test_layout_rejects(lib, kw, code):
    assert layout(lib, **kw) == code
    assert lib.ep_last_error().decode() != ""


def layout_noalloc(lib, idx=A4, T=16, k=2, E=8, counts=A4, offsets=A4, dest=A4, src=A4, status=A4):
    return lib.ep_layout_noalloc(idx, T, k, E, counts, offsets, dest, src, status, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(T=-1), ep.EP_ERR_INVALID_ARG),
        (dict(k=0), ep.EP_ERR_INVALID_ARG),
        (dict(E=1025), ep.EP_ERR_INVALID_ARG),
        (dict(k=9, E=8), ep.EP_ERR_INVALID_ARG),
        (dict(counts=None), ep.EP_ERR_INVALID_ARG),
        (dict(dest=None), ep.EP_ERR_INVALID_ARG),
        (dict(idx=ODD), ep.EP_ERR_ALIGNMENT),
        # scratch above the static 4 MiB: 40000 x 32 with E = 1024 needs 5,125,000 bytes
        (dict(T=40000, k=32, E=1024), ep.EP_ERR_WORKSPACE),
        (dict(T=200000, k=8, E=1024), ep.EP_ERR_WORKSPACE),
    ],
)
def test_layout_noalloc_rejects(lib, kw, code):
    """Host-side errors of the no-allocation layout, before any HIP call; the
    size limit is the static scratch (the same workspace sizes as ep_layout)."""
    assert layout_noalloc(lib, **kw) == code
    msg = lib.ep_last_error().decode()
    assert msg.startswith("ep_layout_noalloc")
    if code == ep.EP_ERR_WORKSPACE:
        assert "scratch" in msg


def test_layout_noalloc_scratch_limit(lib):
    """The largest batches the static scratch covers at a few expert counts:
    the limit equals ep_layout_workspace_bytes against the stated maximum."""
    limit = ep.EP_LAYOUT_NOALLOC_MAX_SCRATCH
    assert limit == 4 << 20
    assert lib.ep_layout_workspace_bytes(16384, 6, 64) <= limit  # the prefill shape
    assert lib.ep_layout_workspace_bytes(131072, 8, 256) <= limit
    assert lib.ep_layout_workspace_bytes(40000, 32, 1024) > limit


def dispatch(lib, x=A16, T=16, H=1024, dest=A4, k=2, recv=A16, rows=32):
    return lib.ep_dispatch(x, T, H, dest, k, recv, rows, None)


def test_max_entries_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define EP_MAX_ENTRIES (\d+)", text)
    assert m and int(m.group(1)) == ep.EP_MAX_ENTRIES == 2**31 - 1 - 2**22


# Counts at EP_MAX_ENTRIES pass the size checks; one more is refused before
# anything is launched.  A count that passes reaches the null-pointer check
# (x = None here), so the two codes tell which check stopped the call.
@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(T=ep.EP_MAX_ENTRIES, k=1, H=8, rows=0), ep.EP_ERR_INVALID_ARG),
        (dict(T=ep.EP_MAX_ENTRIES // 2, k=2, H=8, rows=0), ep.EP_ERR_INVALID_ARG),
        (dict(T=ep.EP_MAX_ENTRIES + 1, k=1, H=8, rows=0), ep.EP_ERR_INVALID_ARG),
        (dict(T=ep.EP_MAX_ENTRIES // 2 + 1, k=2, H=8, rows=0), ep.EP_ERR_INVALID_ARG),
        (dict(T=1, k=1, H=8, rows=ep.EP_MAX_ENTRIES + 1), ep.EP_ERR_INVALID_ARG),
        (dict(T=1, k=1, H=1024, rows=ep.EP_MAX_ENTRIES // 2 + 1), ep.EP_ERR_INVALID_ARG),
        (dict(T=ep.EP_MAX_ENTRIES // 2 + 1, k=1, H=1024, rows=0), ep.EP_ERR_INVALID_ARG),
    ],
)
def test_dispatch_size_limits(lib, kw, code):
    assert dispatch(lib, x=None, **kw) == code
    msg = lib.ep_last_error().decode()
    over = kw["T"] * kw["k"] > ep.EP_MAX_ENTRIES or kw["rows"] > ep.EP_MAX_ENTRIES or \
        max(kw["T"], kw["rows"]) * -(-kw["H"] // 512) > ep.EP_MAX_ENTRIES
    assert ("EP_MAX_ENTRIES" in msg) == over, msg
    if not over:
        assert "null" in msg


def test_combine_and_rows_size_limits(lib):
    big = ep.EP_MAX_ENTRIES // 2 + 1  # two slabs per row at H = 1024
    assert lib.ep_combine(A16, 32, 1024, A4, A4, big, 1, A16, None) == ep.EP_ERR_INVALID_ARG
    assert "EP_MAX_ENTRIES" in lib.ep_last_error().decode()
    assert lib.ep_dispatch_rows(A16, 16, 1024, A4, A16, big, None) == ep.EP_ERR_INVALID_ARG
    assert "EP_MAX_ENTRIES" in lib.ep_last_error().decode()
    assert lib.ep_dispatch_rows(A16, big, 1024, A4, A16, 32, None) == ep.EP_ERR_INVALID_ARG
    assert "EP_MAX_ENTRIES" in lib.ep_last_error().decode()


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(T=-1), ep.EP_ERR_INVALID_ARG),
        (dict(H=0), ep.EP_ERR_INVALID_ARG),
        (dict(H=1020), ep.EP_ERR_INVALID_ARG),
        (dict(k=0), ep.EP_ERR_INVALID_ARG),
        (dict(k=33), ep.EP_ERR_INVALID_ARG),
        (dict(rows=-1), ep.EP_ERR_INVALID_ARG),
        (dict(rows=2**31), ep.EP_ERR_INVALID_ARG),
        (dict(T=2**30, k=4), ep.EP_ERR_INVALID_ARG),
        (dict(x=None), ep.EP_ERR_INVALID_ARG),
        (dict(dest=None), ep.EP_ERR_INVALID_ARG),
        (dict(recv=None), ep.EP_ERR_INVALID_ARG),
        (dict(x=A16 + 8), ep.EP_ERR_ALIGNMENT),
        (dict(recv=A4), ep.EP_ERR_ALIGNMENT),
        (dict(dest=ODD), ep.EP_ERR_ALIGNMENT),
    ],
)
def test_dispatch_rejects(lib, kw, code):
    assert dispatch(lib, **kw) == code


def combine(lib, y=A16, rows=32, H=1024, dest=A4, w=A4, T=16, k=2, out=A16):
    return lib.ep_combine(y, rows, H, dest, w, T, k, out, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(T=-1), ep.EP_ERR_INVALID_ARG),
        (dict(H=12), ep.EP_ERR_INVALID_ARG),
        (dict(k=0), ep.EP_ERR_INVALID_ARG),
        (dict(rows=-5), ep.EP_ERR_INVALID_ARG),
        (dict(w=None), ep.EP_ERR_INVALID_ARG),
        (dict(out=None), ep.EP_ERR_INVALID_ARG),
        (dict(y=None), ep.EP_ERR_INVALID_ARG),
        (dict(out=A16 + 4), ep.EP_ERR_ALIGNMENT),
        (dict(y=A16 + 2), ep.EP_ERR_ALIGNMENT),
        (dict(w=ODD), ep.EP_ERR_ALIGNMENT),
    ],
)
def test_combine_rejects(lib, kw, code):
    assert combine(lib, **kw) == code


def combine_reduce(lib, y=A16, rows=32, H=1024, src=A4, dest=A4, w=A4, T=16, k=2, out=A16, ws=A16,
                   wsb=16 * 1024 * 4):
    return lib.ep_combine_reduce(y, rows, H, src, dest, w, T, k, out, ws, wsb, None)


def test_combine_reduce_workspace_bytes(lib):
    # the fp32 accumulator [T, H]
    assert lib.ep_combine_reduce_workspace_bytes(4096, 7168) == 4096 * 7168 * 4
    assert lib.ep_combine_reduce_workspace_bytes(1, 8) == 32
    assert lib.ep_combine_reduce_workspace_bytes(0, 1024) == 0
    assert lib.ep_combine_reduce_workspace_bytes(16, 12) == 0


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(T=-1), ep.EP_ERR_INVALID_ARG),
        (dict(H=12), ep.EP_ERR_INVALID_ARG),
        (dict(k=0), ep.EP_ERR_INVALID_ARG),
        (dict(k=33), ep.EP_ERR_INVALID_ARG),
        (dict(rows=-5), ep.EP_ERR_INVALID_ARG),
        (dict(y=None), ep.EP_ERR_INVALID_ARG),
        (dict(src=None), ep.EP_ERR_INVALID_ARG),
        (dict(dest=None), ep.EP_ERR_INVALID_ARG),
        (dict(w=None), ep.EP_ERR_INVALID_ARG),
        (dict(out=None), ep.EP_ERR_INVALID_ARG),
        (dict(out=A16 + 4), ep.EP_ERR_ALIGNMENT),
        (dict(y=A16 + 2), ep.EP_ERR_ALIGNMENT),
        (dict(src=ODD), ep.EP_ERR_ALIGNMENT),
        (dict(w=ODD), ep.EP_ERR_ALIGNMENT),
        (dict(ws=None), ep.EP_ERR_WORKSPACE),
        (dict(wsb=16 * 1024 * 4 - 1), ep.EP_ERR_WORKSPACE),
        (dict(ws=A4), ep.EP_ERR_ALIGNMENT),
    ],
)
def test_combine_reduce_rejects(lib, kw, code):
    assert combine_reduce(lib, **kw) == code
    assert lib.ep_last_error().decode() != ""


def test_combine_reduce_empty_batch_is_a_host_no_op(lib):
    assert combine_reduce(lib, T=0, y=None, src=None, dest=None, w=None, out=None, ws=None) == 0


def test_layout_dispatch_rejects(lib):
    def f(idx=A4, T=16, k=2, E=8, x=A16, H=1024, recv=A16, rows=32, ws=A16, wsb=1 << 20):
        return lib.ep_layout_dispatch(idx, T, k, E, x, H, A4, A4, A4, A4, A4, ws, wsb, recv, rows, None)

    assert f(T=-1) == ep.EP_ERR_INVALID_ARG
    assert f(k=9) == ep.EP_ERR_INVALID_ARG
    assert f(H=12) == ep.EP_ERR_INVALID_ARG
    assert f(x=None) == ep.EP_ERR_INVALID_ARG
    assert f(recv=None) == ep.EP_ERR_INVALID_ARG
    assert f(x=A16 + 8) == ep.EP_ERR_ALIGNMENT
    assert f(idx=ODD) == ep.EP_ERR_ALIGNMENT
    assert f(T=131072, k=8, E=256, ws=None) == ep.EP_ERR_WORKSPACE


def test_dispatch_rows_rejects(lib):
    f = lib.ep_dispatch_rows
    assert f(A16, -1, 1024, A4, A16, 32, None) == ep.EP_ERR_INVALID_ARG
    assert f(A16, 16, 1020, A4, A16, 32, None) == ep.EP_ERR_INVALID_ARG
    assert f(A16, 16, 1024, A4, A16, -1, None) == ep.EP_ERR_INVALID_ARG
    assert f(None, 16, 1024, A4, A16, 32, None) == ep.EP_ERR_INVALID_ARG
    assert f(A16, 16, 1024, None, A16, 32, None) == ep.EP_ERR_INVALID_ARG
    assert f(A16 + 4, 16, 1024, A4, A16, 32, None) == ep.EP_ERR_ALIGNMENT
    assert f(A16, 16, 1024, ODD, A16, 32, None) == ep.EP_ERR_ALIGNMENT
    assert f(A16, 0, 1024, A4, A16, 32, None) == 0
    assert f(None, 16, 1024, None, None, 0, None) == 0


def test_empty_batches_are_host_no_ops(lib):
    # T == 0 returns before touching the device
    assert dispatch(lib, T=0, x=None, dest=None, recv=None) == 0
    assert combine(lib, T=0, y=None, dest=None, w=None, out=None) == 0
    # so does an empty receive buffer
    assert dispatch(lib, rows=0, recv=None) == 0


def test_probe_rejects(lib):
    assert lib.ep_bw_probe(-1, A16, A16, 1024, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_bw_probe(0x30, A16, A16, 1024, None) == ep.EP_ERR_INVALID_ARG  # depth code 3
    assert lib.ep_bw_probe(0x601, A16, A16, 1024, None) == ep.EP_ERR_INVALID_ARG  # policy 6
    assert lib.ep_bw_probe(0x1000, A16, A16, 1024, None) == ep.EP_ERR_INVALID_ARG  # unknown bit
    assert lib.ep_bw_probe(7, A16, A16, 65536, None) == ep.EP_ERR_INVALID_ARG  # phases need 128 KiB multiples
    assert lib.ep_bw_probe(6, A16, A16, 8192, None) == ep.EP_ERR_INVALID_ARG  # bursts need 64 KiB multiples
    assert lib.ep_bw_probe(4, A16, A16, 4096, None) == ep.EP_ERR_INVALID_ARG  # mixed needs 8 KiB multiples
    assert lib.ep_bw_probe(0, A16, A16, 1000 + 4, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_bw_probe(0, None, A16, 1024, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_bw_probe(0, A16 + 4, A16, 1024, None) == ep.EP_ERR_ALIGNMENT
    assert lib.ep_bw_probe(0, A16, A16, 0, None) == 0
    assert lib.ep_probe_placement(None, 4, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_probe_placement(A4, 0, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_mfma_probe(4, 10, None, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_mfma_probe(0, 10, A4, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_mfma_probe(4, -1, A4, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_mfma_probe(4, 10, ODD, None) == ep.EP_ERR_ALIGNMENT


def test_masked_stream_rejects(lib):
    out = ctypes.c_void_p()
    mask = (ctypes.c_uint32 * 8)(*([0] * 8))
    assert lib.ep_stream_create_cu_masked(None, 8, ctypes.byref(out)) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_stream_create_cu_masked(mask, 8, None) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_stream_create_cu_masked(mask, 0, ctypes.byref(out)) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_stream_create_cu_masked(mask, 65, ctypes.byref(out)) == ep.EP_ERR_INVALID_ARG
    assert lib.ep_stream_create_cu_masked(mask, 8, ctypes.byref(out)) == ep.EP_ERR_INVALID_ARG  # empty
    assert lib.ep_stream_destroy(None) == ep.EP_ERR_INVALID_ARG
    assert ep.cu_mask_words([0, 33, 255]) == [1, 2, 0, 0, 0, 0, 0, 1 << 31]


def test_inflight_probe_rejects(lib):
    f = lib.ep_inflight_probe
    assert f(0, 8, 0, A16, 1024, A16, None, 0, 0, None, None) == ep.EP_ERR_INVALID_ARG
    assert f(17, 8, 0, A16, 1024, A16, None, 0, 0, None, None) == ep.EP_ERR_INVALID_ARG
    assert f(4, 3, 0, A16, 1024, A16, None, 0, 0, None, None) == ep.EP_ERR_INVALID_ARG
    assert f(16, 16, 0, A16, 1024, A16, None, 0, 0, None, None) == ep.EP_ERR_INVALID_ARG
    assert f(4, 8, 0, A16, 1000, A16, None, 0, 0, None, None) == ep.EP_ERR_INVALID_ARG
    assert f(4, 8, 0, None, 1024, A16, None, 0, 0, None, None) == ep.EP_ERR_INVALID_ARG
    assert f(4, 8, 0, A16, 1024, A16, None, 0, 10, A16, None) == ep.EP_ERR_INVALID_ARG  # a chase needs a chain
    assert f(4, 8, 0, A16, 1024, A16, A16, 0, 10, A16, None) == ep.EP_ERR_INVALID_ARG  # of at least one element
    assert f(4, 8, 0, A16, 1024, A16, A4, 8, 10, A16, None) == ep.EP_ERR_ALIGNMENT
    assert f(4, 8, 0, A4, 1024, A16, None, 0, 0, None, None) == ep.EP_ERR_ALIGNMENT
    assert f(4, 8, 2, A16, 1024, A16, None, 0, 0, None, None) == ep.EP_ERR_INVALID_ARG


def test_status_strings(lib):
    seen = set()
    for code in [0, -1, -2, -3, -4, -5]:
        s = lib.ep_status_string(code).decode()
        assert s and s not in seen
        seen.add(s)
    assert lib.ep_status_string(-99).decode() == "unknown code"


def test_binding_checks_tensors_before_the_library():
    import torch

    cpu = torch.zeros((4, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ep.ep_dispatch(cpu, torch.zeros((4, 2), dtype=torch.int32), cpu)
    with pytest.raises(TypeError):
        ep.ep_combine(None, None, None, cpu)


class _ReachedLibrary(Exception):
    pass


@pytest.fixture
def host_binding(monkeypatch):
    """The binding with host tensors standing in for device ones (only the
    device test is lifted) and a library stub that raises as soon as it is
    reached: a size error must be raised before any call into libep.so."""
    import torch

    def host_tensor(t, name, dtype=None):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        return t

    class Stub:
        def __getattr__(self, name):
            if name == "ep_layout_workspace_bytes":
                return lambda T, k, E: 64
            raise _ReachedLibrary(name)

    monkeypatch.setattr(ep, "_device_tensor", host_tensor)
    monkeypatch.setattr(ep, "lib", lambda: Stub())
    monkeypatch.setattr(ep, "_stream", lambda stream, t=None: 0)
    return torch


@pytest.mark.parametrize("which", ["counts", "offsets", "dest_row_short", "dest_row_shape", "src_token", "status"])
@pytest.mark.parametrize("entry", ["ep_layout", "ep_layout_dispatch"])
def test_layout_binding_rejects_short_outputs(host_binding, entry, which):
    torch = host_binding
    T, k, E, H = 16, 4, 8, 64
    i32 = torch.int32
    good = {"counts": torch.zeros(E, dtype=i32), "offsets": torch.zeros(E + 1, dtype=i32),
            "dest_row": torch.zeros((T, k), dtype=i32), "src_token": torch.zeros(T * k, dtype=i32),
            "status": torch.zeros(1, dtype=i32), "workspace": torch.zeros(64, dtype=torch.uint8)}
    bad = dict(good)
    if which == "counts":
        bad["counts"] = torch.zeros(E - 1, dtype=i32)
    elif which == "offsets":
        bad["offsets"] = torch.zeros(E, dtype=i32)
    elif which == "dest_row_short":
        bad["dest_row"] = torch.zeros((T, k - 1), dtype=i32)
    elif which == "dest_row_shape":
        bad["dest_row"] = torch.zeros((T * k,), dtype=i32)
    elif which == "src_token":
        bad["src_token"] = torch.zeros(T * k - 1, dtype=i32)
    else:
        bad["status"] = torch.zeros(0, dtype=i32)
    idx = torch.zeros((T, k), dtype=i32)
    fn = getattr(ep, entry)
    extra = () if entry == "ep_layout" else (torch.zeros((T, H), dtype=torch.bfloat16),
                                            torch.zeros((T * k, H), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fn(idx, E, *extra, **bad)
    # the same call with every output large enough gets through to the library
    with pytest.raises(_ReachedLibrary):
        fn(idx, E, *extra, **good)

"""Python binding of libep.so, the MI355X (gfx950) MoE row-movement library.

Argument marshalling only: every step of layout, dispatch and combine runs in
the library's HIP kernels.  torch provides device memory and the stream
(``torch.cuda.current_stream()`` unless one is given).  The functions carry
the names of the C entry points declared in ``include/ep.h``.

There is no fallback: if ``libep.so`` is missing or cannot be loaded, every
call raises ``EpLibraryMissing``.  Build it with
``python -m bulk_async_tensor_amd.build``.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep.so")

EP_OK = 0
EP_ERR_INVALID_ARG = -1
EP_ERR_ALIGNMENT = -2
EP_ERR_UNSUPPORTED = -3
EP_ERR_WORKSPACE = -4
EP_ERR_HIP = -5
EP_STATUS_EXPERT_OUT_OF_RANGE = 1
EP_STATUS_DUPLICATE_EXPERT = 2
EP_MAX_TOPK = 32
EP_MAX_EXPERTS = 1024
EP_MAX_ENTRIES = (1 << 31) - 1 - (1 << 22)

VARIANTS = ("auto", "vgpr", "vgpr2", "lds1", "lds2", "vgpr_cached", "phase", "lds3", "pc", "vgpr_wg")

_c_int, _c_i64, _c_sz, _p = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes), mirroring include/ep.h
_SIGNATURES = {
    "ep_set_num_cus": (_c_int, [_c_int]),
    "ep_get_num_cus": (_c_int, []),
    "ep_set_variant": (_c_int, [ctypes.c_char_p]),
    "ep_get_variant": (ctypes.c_char_p, []),
    "ep_set_slab": (_c_int, [_c_int]),
    "ep_get_slab": (_c_int, []),
    "ep_layout_workspace_bytes": (_c_sz, [_c_int, _c_int, _c_int]),
    "ep_layout": (_c_int, [_p, _c_int, _c_int, _c_int, _p, _p, _p, _p, _p, _p, _c_sz, _p]),
    "ep_layout_noalloc": (_c_int, [_p, _c_int, _c_int, _c_int, _p, _p, _p, _p, _p, _p]),
    "ep_dispatch": (_c_int, [_p, _c_int, _c_int, _p, _c_int, _p, _c_i64, _p]),
    "ep_dispatch_rows": (_c_int, [_p, _c_int, _c_int, _p, _p, _c_i64, _p]),
    "ep_layout_dispatch": (_c_int, [_p, _c_int, _c_int, _c_int, _p, _c_int, _p, _p, _p, _p, _p, _p, _c_sz, _p,
                                    _c_i64, _p]),
    "ep_combine": (_c_int, [_p, _c_i64, _c_int, _p, _p, _c_int, _c_int, _p, _p]),
    "ep_combine_reduce_workspace_bytes": (_c_sz, [_c_int, _c_int]),
    "ep_combine_reduce": (_c_int, [_p, _c_i64, _c_int, _p, _p, _p, _c_int, _c_int, _p, _p, _c_sz, _p]),
    "ep_status_string": (ctypes.c_char_p, [_c_int]),
    "ep_last_error": (ctypes.c_char_p, []),
    "ep_bw_probe": (_c_int, [_c_int, _p, _p, _c_i64, _p]),
    "ep_probe_placement": (_c_int, [_p, _c_int, _p]),
    "ep_inflight_probe": (_c_int, [_c_int, _c_int, _c_int, _p, _c_i64, _p, _p, _c_i64, _c_i64, _p, _p]),
    "ep_mfma_probe": (_c_int, [_c_int, _c_int, _p, _p]),
    "ep_stream_create_cu_masked": (_c_int, [ctypes.POINTER(ctypes.c_uint32), _c_int, ctypes.POINTER(_p)]),
    "ep_stream_destroy": (_c_int, [_p]),
}


class EpLibraryMissing(RuntimeError):
    pass


class EpError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{message} (code {code})")
        self.code = code


_lib = None


def lib():
    """The loaded libep.so (raises EpLibraryMissing when it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise EpLibraryMissing(
                f"{LIB_PATH} is not built; run `python -m bulk_async_tensor_amd.build` (hipcc, gfx950)"
            )
        try:
            handle = ctypes.CDLL(LIB_PATH)
        except OSError as exc:  # pragma: no cover - depends on the machine
            raise EpLibraryMissing(f"cannot load {LIB_PATH}: {exc}") from exc
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(rc, what):
    if rc < 0:
        detail = lib().ep_last_error().decode()
        raise EpError(rc, f"{what}: {detail or lib().ep_status_string(rc).decode()}")
    return rc


def _ptr(t):
    # a plain int: the c_void_p argtypes convert it (NULL for None)
    return None if t is None else t.data_ptr()


def _stream(stream, t=None):
    """The raw HIP stream: the given torch stream, else the current stream of
    t's device (of the current device when t is None).  The raw accessor
    skips building a torch.cuda.Stream object per call."""
    if stream is not None:
        return stream.cuda_stream
    import torch

    dev = t.get_device() if t is not None else torch.cuda.current_device()
    return torch._C._cuda_getCurrentRawStream(dev)


def _device_tensor(t, name, dtype=None):
    # fast path for a valid argument (torch dtypes are singletons); the checks
    # below give the error for anything else
    try:
        if t.is_cuda and t.is_contiguous() and (dtype is None or t.dtype is dtype):
            return t
    except (AttributeError, TypeError):
        pass
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _layout_outputs(T, k, E, dev, counts, offsets, dest_row, src_token, status):
    """The layout's output tensors: the caller's, checked for dtype and for
    room (the C ABI takes bare pointers and cannot), or new ones."""
    import torch

    i32 = dict(dtype=torch.int32, device=dev)

    def given(t, name, need):
        _device_tensor(t, name, torch.int32)
        if t.numel() < need:
            raise ValueError(f"{name} holds {t.numel()} int32, needs at least {need}")
        return t

    counts = torch.empty(E, **i32) if counts is None else given(counts, "counts", E)
    offsets = torch.empty(E + 1, **i32) if offsets is None else given(offsets, "offsets", E + 1)
    if dest_row is None:
        dest_row = torch.empty((T, k), **i32)
    else:
        given(dest_row, "dest_row", T * k)
        if tuple(dest_row.shape) != (T, k):
            raise ValueError(f"dest_row must be [T, k] = [{T}, {k}], got {list(dest_row.shape)}")
    src_token = torch.empty(T * k, **i32) if src_token is None else given(src_token, "src_token", T * k)
    status = torch.empty(1, **i32) if status is None else given(status, "status", 1)
    return counts, offsets, dest_row, src_token, status


# ------------------------------------------------------------------ settings
def ep_set_num_cus(n):
    return _check(lib().ep_set_num_cus(int(n)), "ep_set_num_cus")


def ep_get_num_cus():
    return lib().ep_get_num_cus()


def ep_set_variant(name):
    return _check(lib().ep_set_variant(name.encode()), "ep_set_variant")


def ep_get_variant():
    return lib().ep_get_variant().decode()


def ep_set_slab(vectors_per_lane):
    return _check(lib().ep_set_slab(int(vectors_per_lane)), "ep_set_slab")


def ep_get_slab():
    return lib().ep_get_slab()


def ep_layout_workspace_bytes(T, k, E):
    return lib().ep_layout_workspace_bytes(int(T), int(k), int(E))


def ep_status_string(code):
    return lib().ep_status_string(int(code)).decode()


def ep_last_error():
    return lib().ep_last_error().decode()


# ------------------------------------------------------------------ hot path
def ep_layout(topk_idx, num_experts, counts=None, offsets=None, dest_row=None, src_token=None, status=None,
              workspace=None, stream=None):
    """Per-expert counts, offsets and stable destination rows of topk_idx [T, k] (int32).

    Missing outputs are allocated with torch on the input's device.  Returns a
    dict of the output tensors (``status`` is a 1-element int32 tensor).
    """
    import torch

    _device_tensor(topk_idx, "topk_idx", torch.int32)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, k]")
    T, k = topk_idx.shape
    E = int(num_experts)
    dev = topk_idx.device
    counts, offsets, dest_row, src_token, status = _layout_outputs(T, k, E, dev, counts, offsets, dest_row,
                                                                   src_token, status)
    if workspace is None:
        need = ep_layout_workspace_bytes(T, k, E) if 1 <= k <= EP_MAX_TOPK and 1 <= E <= EP_MAX_EXPERTS else 0
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    else:
        _device_tensor(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(
        lib().ep_layout(_ptr(topk_idx), T, k, E, _ptr(counts), _ptr(offsets), _ptr(dest_row), _ptr(src_token),
                        _ptr(status), _ptr(workspace), ws_bytes, _stream(stream, topk_idx)),
        "ep_layout",
    )
    return {"counts": counts, "offsets": offsets, "dest_row": dest_row, "src_token": src_token, "status": status}


EP_LAYOUT_NOALLOC_MAX_SCRATCH = 4 << 20


def ep_layout_noalloc(topk_idx, num_experts, counts, offsets, dest_row, src_token=None, status=None, stream=None):
    """ep_layout with the library's static scratch instead of a workspace
    (the C call allocates nothing).  Every output except src_token and
    status must be given; returns the same dict as ep_layout."""
    import torch

    _device_tensor(topk_idx, "topk_idx", torch.int32)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, k]")
    if counts is None or offsets is None or dest_row is None:
        raise ValueError("ep_layout_noalloc needs counts, offsets and dest_row")
    T, k = topk_idx.shape
    E = int(num_experts)
    counts, offsets, dest_row, src_token, status = _layout_outputs(T, k, E, topk_idx.device, counts, offsets,
                                                                   dest_row, src_token, status)
    _check(lib().ep_layout_noalloc(_ptr(topk_idx), T, k, E, _ptr(counts), _ptr(offsets), _ptr(dest_row),
                                   _ptr(src_token), _ptr(status), _stream(stream, topk_idx)), "ep_layout_noalloc")
    return {"counts": counts, "offsets": offsets, "dest_row": dest_row, "src_token": src_token, "status": status}


def ep_layout_dispatch(topk_idx, num_experts, x, recv, counts=None, offsets=None, dest_row=None, src_token=None,
                       status=None, workspace=None, stream=None):
    """ep_layout then ep_dispatch, in one launch where the library can (see include/ep.h).  Returns the
    layout dict."""
    import torch

    _device_tensor(topk_idx, "topk_idx", torch.int32)
    _device_tensor(x, "x", torch.bfloat16)
    _device_tensor(recv, "recv", torch.bfloat16)
    if topk_idx.dim() != 2 or x.dim() != 2:
        raise ValueError("topk_idx must be [T, k] and x [T, H]")
    T, k = topk_idx.shape
    E = int(num_experts)
    H = x.shape[1]
    if x.shape[0] != T or recv.dim() != 2 or recv.shape[1] != H:
        raise ValueError("x must be [T, H] and recv [R, H]")
    dev = topk_idx.device
    counts, offsets, dest_row, src_token, status = _layout_outputs(T, k, E, dev, counts, offsets, dest_row,
                                                                   src_token, status)
    if workspace is None:
        need = ep_layout_workspace_bytes(T, k, E) if 1 <= k <= EP_MAX_TOPK and 1 <= E <= EP_MAX_EXPERTS else 0
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    else:
        _device_tensor(workspace, "workspace")
    _check(lib().ep_layout_dispatch(_ptr(topk_idx), T, k, E, _ptr(x), H, _ptr(counts), _ptr(offsets),
                                    _ptr(dest_row), _ptr(src_token), _ptr(status), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _ptr(recv), recv.shape[0],
                                    _stream(stream, x)), "ep_layout_dispatch")
    return {"counts": counts, "offsets": offsets, "dest_row": dest_row, "src_token": src_token, "status": status}


def ep_dispatch(x, dest_row, recv, stream=None):
    """recv[dest_row[t, j]] = x[t] for x [T, H] bf16, dest_row [T, k] int32, recv [R, H] bf16."""
    import torch

    _device_tensor(x, "x", torch.bfloat16)
    _device_tensor(dest_row, "dest_row", torch.int32)
    _device_tensor(recv, "recv", torch.bfloat16)
    T, H = x.shape
    if dest_row.dim() != 2 or dest_row.shape[0] != T:
        raise ValueError("dest_row must be [T, k]")
    if recv.dim() != 2 or recv.shape[1] != H:
        raise ValueError("recv must be [R, H]")
    k = dest_row.shape[1]
    _check(lib().ep_dispatch(_ptr(x), T, H, _ptr(dest_row), k, _ptr(recv), recv.shape[0], _stream(stream, x)),
           "ep_dispatch")
    return recv


def ep_dispatch_rows(x, src_token, recv, stream=None):
    """recv[r] = x[src_token[r]] for x [T, H] bf16, src_token [R] int32, recv [R, H] bf16."""
    import torch

    _device_tensor(x, "x", torch.bfloat16)
    _device_tensor(src_token, "src_token", torch.int32)
    _device_tensor(recv, "recv", torch.bfloat16)
    T, H = x.shape
    if recv.dim() != 2 or recv.shape[1] != H or src_token.numel() < recv.shape[0]:
        raise ValueError("recv must be [R, H] and src_token hold at least R entries")
    _check(lib().ep_dispatch_rows(_ptr(x), T, H, _ptr(src_token), _ptr(recv), recv.shape[0], _stream(stream, x)),
           "ep_dispatch_rows")
    return recv


def ep_combine(y, dest_row, topk_w, out, stream=None):
    """out[t] = bf16(sum_j w[t, j] * y[dest_row[t, j]]) for y [R, H] bf16, out [T, H] bf16."""
    import torch

    _device_tensor(y, "y", torch.bfloat16)
    _device_tensor(dest_row, "dest_row", torch.int32)
    _device_tensor(topk_w, "topk_w", torch.float32)
    _device_tensor(out, "out", torch.bfloat16)
    T, H = out.shape
    if dest_row.dim() != 2 or dest_row.shape[0] != T or tuple(topk_w.shape) != tuple(dest_row.shape):
        raise ValueError("dest_row and topk_w must both be [T, k]")
    if y.dim() != 2 or y.shape[1] != H:
        raise ValueError("y must be [R, H]")
    k = dest_row.shape[1]
    _check(lib().ep_combine(_ptr(y), y.shape[0], H, _ptr(dest_row), _ptr(topk_w), T, k, _ptr(out),
                            _stream(stream, out)), "ep_combine")
    return out


def ep_combine_reduce_workspace_bytes(T, H):
    return lib().ep_combine_reduce_workspace_bytes(int(T), int(H))


def ep_combine_reduce(y, src_token, dest_row, topk_w, out, workspace=None, stream=None):
    """Reduce-on-store combine: out[t] = bf16(sum of w[t, j] * y[r] over the rows r
    that src_token assigns to t and dest_row[t, j] lists), fp32 atomics into
    ``workspace`` (float32 [T, H] worth of bytes; allocated when None)."""
    import torch

    _device_tensor(y, "y", torch.bfloat16)
    _device_tensor(src_token, "src_token", torch.int32)
    _device_tensor(dest_row, "dest_row", torch.int32)
    _device_tensor(topk_w, "topk_w", torch.float32)
    _device_tensor(out, "out", torch.bfloat16)
    T, H = out.shape
    if dest_row.dim() != 2 or dest_row.shape[0] != T or tuple(topk_w.shape) != tuple(dest_row.shape):
        raise ValueError("dest_row and topk_w must both be [T, k]")
    if y.dim() != 2 or y.shape[1] != H or src_token.numel() < y.shape[0]:
        raise ValueError("y must be [R, H] and src_token hold at least R entries")
    k = dest_row.shape[1]
    if workspace is None:
        workspace = torch.empty(max(ep_combine_reduce_workspace_bytes(T, H), 16), dtype=torch.uint8,
                                device=out.device)
    else:
        _device_tensor(workspace, "workspace")
    _check(lib().ep_combine_reduce(_ptr(y), y.shape[0], H, _ptr(src_token), _ptr(dest_row), _ptr(topk_w), T, k,
                                   _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream, out)), "ep_combine_reduce")
    return out


# ------------------------------------------------------------------ probes
def ep_bw_probe(mode, src, dst, nbytes, stream=None):
    """Streaming probe under the current CU budget (0 copy, 1 read, 2 write)."""
    return _check(lib().ep_bw_probe(int(mode), _ptr(src), _ptr(dst), int(nbytes), _stream(stream)), "ep_bw_probe")


def ep_inflight_probe(waves_per_cu, vectors_per_lane, src, nbytes, sink, chain=None, hops=0, out=None, cached=False,
                      stream=None):
    """Streaming nt reads with a chosen depth per CU, beside one pointer-chasing
    wave (see include/ep.h).  chain: int64 device tensor of next indices;
    out: int64 device tensor of at least 4 elements."""
    import torch

    if chain is not None:
        _device_tensor(chain, "chain", torch.int64)
    if out is not None:
        _device_tensor(out, "out", torch.int64)
        if out.numel() < 4:
            raise ValueError("out must hold 4 int64")
    clen = 0 if chain is None else chain.numel()
    return _check(lib().ep_inflight_probe(int(waves_per_cu), int(vectors_per_lane), int(bool(cached)), _ptr(src),
                                          int(nbytes),
                                          _ptr(sink), _ptr(chain), clen, int(hops), _ptr(out), _stream(stream)),
                  "ep_inflight_probe")


def ep_probe_placement(out, n_groups, stream=None):
    """Writes {XCC, SE, (SH<<4)|CU, raw HW_ID} per workgroup into out (int32 [n_groups, 4])."""
    import torch

    _device_tensor(out, "out", torch.int32)
    if out.numel() < 4 * n_groups:
        raise ValueError("out must hold 4 * n_groups int32")
    return _check(lib().ep_probe_placement(_ptr(out), int(n_groups), _stream(stream)), "ep_probe_placement")


def ep_mfma_probe(n_groups, iters, out, stream=None):
    """Compute-bound matrix-core loop: n_groups workgroups of 4 waves, iters
    rounds of 4 x 16384 flop per wave; out: float32 tensor of 256 * n_groups."""
    import torch

    _device_tensor(out, "out", torch.float32)
    if out.numel() < 256 * int(n_groups):
        raise ValueError("out must hold 256 * n_groups floats")
    return _check(lib().ep_mfma_probe(int(n_groups), int(iters), _ptr(out), _stream(stream)), "ep_mfma_probe")


# ------------------------------------------------------------------ CU-masked streams
def cu_mask_words(cus, n_words=8):
    """Mask words with the bits of the given CU indices set."""
    words = [0] * n_words
    for c in cus:
        words[c // 32] |= 1 << (c % 32)
    return words


def ep_stream_create_cu_masked(mask_words):
    """A torch ExternalStream over a new HIP stream restricted to the CUs whose
    bits are set in mask_words (a list of uint32)."""
    import torch

    arr = (ctypes.c_uint32 * len(mask_words))(*[int(w) & 0xFFFFFFFF for w in mask_words])
    out = ctypes.c_void_p()
    _check(lib().ep_stream_create_cu_masked(arr, len(mask_words), ctypes.byref(out)), "ep_stream_create_cu_masked")
    return torch.cuda.ExternalStream(out.value)


def ep_stream_destroy(stream):
    """Destroys a stream made by ep_stream_create_cu_masked (after use)."""
    return _check(lib().ep_stream_destroy(ctypes.c_void_p(stream.cuda_stream)), "ep_stream_destroy")


__all__ = [n for n in list(globals()) if n.startswith("ep_") or n.startswith("EP_")] + [
    "lib", "LIB_PATH", "VARIANTS", "EpError", "EpLibraryMissing", "cu_mask_words",
]

"""ctypes binding of libfa.so (the C ABI declared in include/fa.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no CPU or PyTorch fallback -- if libfa.so is missing or the
device is unsupported, the call raises.
"""

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfa.so"

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_HIP = 3
FA_ERR_NO_MEMORY = 4
FA_ERR_TOO_LARGE = 5

# name -> (restype, argtypes); the exported symbols of include/fa.h
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "fa_strerror": (ctypes.c_char_p, [_i]),
    "fa_version": (_i, []),
    "fa_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp]),
    "fa_prefill_f32": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp]),
    "fa_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp]),
    "fa_decode_ws": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "fa_decode_f32": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp]),
    "fa_decode_f32_ws": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "fa_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "fa_prefill_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _f,
                               _vp]),
    "fa_prefill_backward": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _sz,
                                 _vp]),
    "fa_prefill_backward_workspace_bytes": (_sz, [_i, _i, _i]),
    "fa_decode_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "fa_decode_paged_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "fa_decode_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp]),
}

_lib = None
_lock = threading.Lock()


class FaError(RuntimeError):
    """A libfa call returned a non-zero fa_status."""

    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} (status {status})")


def library_path():
    return os.environ.get("FA_LIBRARY", os.path.join(PKG, _LIB_NAME))


def load_library():
    """Load libfa.so once and declare every exported signature."""
    global _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise FaError(-1, f"{path} not found; build it with "
                                  "`python -m exact_tiled_attention_prefill_amd.build`")
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def strerror(status):
    if status == -1:
        return "library not built"
    try:
        return load_library().fa_strerror(int(status)).decode()
    except Exception:  # library unavailable: plain code
        return f"fa_status {status}"


def _check(status, what):
    if status != FA_OK:
        raise FaError(status, what)


def _torch():
    import torch

    return torch


def _stream_ptr(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _require(t, name, dtype, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def prefill(q, k, v, causal=False, scale=None, out=None, lse=None, return_lse=True, stream=None):
    """Exact attention softmax(scale*QK^T + mask)V on the GPU.

    q [B,Hq,N,d], k/v [B,Hkv,N,d]: contiguous device tensors, all bf16 or
    all float32.  Returns (o, lse) with o like q and lse float32 [B,Hq,N]
    (lse is None when return_lse=False and no lse buffer is given).
    """
    torch = _torch()
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q/k/v must be bfloat16 or float32")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, dtype, 4)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ValueError("k and v must be [B, Hkv, N, d] matching q")
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", dtype, 4)
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must match q")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, Hq, N):
            raise ValueError("lse must be [B, Hq, N]")
    lib = load_library()
    fn = lib.fa_prefill if dtype == torch.bfloat16 else lib.fa_prefill_f32
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse) if lse is not None else None,
            B, Hq, Hkv, N, d, 1 if causal else 0, float(scale), _stream_ptr(stream))
    _check(st, "fa_prefill" if dtype == torch.bfloat16 else "fa_prefill_f32")
    return out, lse


def decode_workspace_bytes(B, Hq, Hkv, maxlen, d):
    return int(load_library().fa_decode_workspace_bytes(B, Hq, Hkv, maxlen, d))


def decode(q, kcache, vcache, seqlens, scale=None, out=None, workspace=None, stream=None):
    """One query token per sequence against a contiguous KV cache.

    q [B,Hq,d]; kcache/vcache [B,Hkv,maxlen,d] (bf16 or float32, matching q);
    seqlens int32 [B] on the device.  `workspace` (uint8 device tensor of at
    least decode_workspace_bytes(...) bytes) avoids the library's
    stream-ordered allocation.  Returns o [B,Hq,d].
    """
    torch = _torch()
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q/kcache/vcache must be bfloat16 or float32")
    _require(q, "q", dtype, 3)
    _require(kcache, "kcache", dtype, 4)
    _require(vcache, "vcache", dtype, 4)
    _require(seqlens, "seqlens", torch.int32, 1)
    B, Hq, d = q.shape
    _, Hkv, maxlen, _ = kcache.shape
    if tuple(kcache.shape) != (B, Hkv, maxlen, d) or tuple(vcache.shape) != (B, Hkv, maxlen, d):
        raise ValueError("kcache/vcache must be [B, Hkv, maxlen, d] matching q")
    if seqlens.shape[0] != B:
        raise ValueError("seqlens must be [B]")
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", dtype, 3)
    lib = load_library()
    args = (_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(seqlens), _ptr(out), B, Hq, Hkv, maxlen, d,
            float(scale))
    bf16 = dtype == torch.bfloat16
    if workspace is None:
        fn = lib.fa_decode if bf16 else lib.fa_decode_f32
        st = fn(*args, _stream_ptr(stream))
    else:
        if workspace.dtype != torch.uint8 or not workspace.is_cuda:
            raise TypeError("workspace must be a uint8 device tensor")
        fn = lib.fa_decode_ws if bf16 else lib.fa_decode_f32_ws
        st = fn(*args, _ptr(workspace), workspace.numel(), _stream_ptr(stream))
    _check(st, fn.__name__)
    return out


def decode_noalloc(q, kcache, vcache, seqlens, scale=None, out=None, stream=None):
    """decode() through fa_decode_noalloc (bf16): the library allocates no
    device memory; its partials go to a fixed per-GPU array (calls that can
    overlap on one GPU race on it).  Raises FaError(FA_ERR_TOO_LARGE) when the
    sizes exceed that array.  Returns o [B,Hq,d]."""
    torch = _torch()
    _require(q, "q", torch.bfloat16, 3)
    _require(kcache, "kcache", torch.bfloat16, 4)
    _require(vcache, "vcache", torch.bfloat16, 4)
    _require(seqlens, "seqlens", torch.int32, 1)
    B, Hq, d = q.shape
    _, Hkv, maxlen, _ = kcache.shape
    if tuple(kcache.shape) != (B, Hkv, maxlen, d) or tuple(vcache.shape) != (B, Hkv, maxlen, d):
        raise ValueError("kcache/vcache must be [B, Hkv, maxlen, d] matching q")
    if seqlens.shape[0] != B:
        raise ValueError("seqlens must be [B]")
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", torch.bfloat16, 3)
    st = load_library().fa_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(seqlens), _ptr(out), B, Hq,
                                          Hkv, maxlen, d, float(scale), _stream_ptr(stream))
    _check(st, "fa_decode_noalloc")
    return out


def decode_paged_workspace_bytes(B, Hq, Hkv, page_size, max_pages, d):
    return int(load_library().fa_decode_paged_workspace_bytes(B, Hq, Hkv, page_size, max_pages, d))


def decode_paged(q, kpages, vpages, block_table, seqlens, scale=None, out=None, workspace=None, stream=None):
    """One query token per sequence against a paged KV cache (bf16).

    q [B,Hq,d]; kpages/vpages [num_pages,Hkv,page_size,d]; block_table int32
    [B,max_pages] and seqlens int32 [B], both on the device.  `workspace`
    (uint8 device tensor of at least decode_paged_workspace_bytes(...)
    bytes) avoids the library's stream-ordered allocation.  Returns o [B,Hq,d].
    """
    torch = _torch()
    _require(q, "q", torch.bfloat16, 3)
    _require(kpages, "kpages", torch.bfloat16, 4)
    _require(vpages, "vpages", torch.bfloat16, 4)
    _require(block_table, "block_table", torch.int32, 2)
    _require(seqlens, "seqlens", torch.int32, 1)
    B, Hq, d = q.shape
    num_pages, Hkv, page_size, _ = kpages.shape
    if tuple(kpages.shape) != (num_pages, Hkv, page_size, d) or tuple(vpages.shape) != tuple(kpages.shape):
        raise ValueError("kpages/vpages must be [num_pages, Hkv, page_size, d] matching q")
    if block_table.shape[0] != B or seqlens.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages] and seqlens [B]")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", torch.bfloat16, 3)
    ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_cuda:
            raise TypeError("workspace must be a uint8 device tensor")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    lib = load_library()
    st = lib.fa_decode_paged(_ptr(q), _ptr(kpages), _ptr(vpages), _ptr(block_table), _ptr(seqlens), _ptr(out),
                             B, Hq, Hkv, num_pages, page_size, max_pages, d, float(scale), ws_ptr, ws_bytes,
                             _stream_ptr(stream))
    _check(st, "fa_decode_paged")
    return out


def prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal=False, window_left=-1,
                   scale=None, out=None, lse=None, return_lse=True, stream=None):
    """Packed variable-length attention (bf16): chunked prefill, sliding window.

    q [total_q,Hq,d]; k/v [total_k,Hkv,d]; cu_seqlens_q/k int32 [B+1] on the
    device; a sequence's queries are its last n_q positions (causal row i
    sees keys <= i + n_k - n_q, and >= that minus window_left when
    window_left >= 0).  Returns o [total_q,Hq,d] and, if return_lse, lse
    [Hq,total_q] (fp32).
    """
    torch = _torch()
    _require(q, "q", torch.bfloat16, 3)
    _require(k, "k", torch.bfloat16, 3)
    _require(v, "v", torch.bfloat16, 3)
    _require(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _require(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    total_q, Hq, d = q.shape
    total_k, Hkv, _ = k.shape
    if tuple(k.shape) != (total_k, Hkv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k/v must be [total_k, Hkv, d] matching q")
    B = cu_seqlens_q.shape[0] - 1
    if B < 1 or cu_seqlens_k.shape[0] != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B+1]")
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", torch.bfloat16, 3)
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require(lse, "lse", torch.float32, 2)
    st = load_library().fa_prefill_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse) if lse is not None else None, _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), B, Hq, Hkv, total_q, total_k, int(max_seqlen_q), d, int(bool(causal)),
        int(window_left), float(scale), _stream_ptr(stream))
    _check(st, "fa_prefill_varlen")
    return (out, lse) if return_lse else out


def prefill_backward_workspace_bytes(B, Hq, N):
    return int(load_library().fa_prefill_backward_workspace_bytes(B, Hq, N))


def prefill_backward(q, k, v, o, dout, lse, causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None,
                     stream=None):
    """Gradients of sum(o * dout) for o = prefill(q, k, v) (bf16).

    q, o, dout [B,Hq,N,d]; k, v [B,Hkv,N,d]; lse [B,Hq,N] fp32 as returned by
    prefill() with the same causal and scale.  Returns (dq, dk, dv).
    """
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _require(t, n, torch.bfloat16, 4)
    _require(lse, "lse", torch.float32, 3)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k/v must be [B, Hkv, N, d] matching q")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("o/dout must match q and lse must be [B, Hq, N]")
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _require(t, n, torch.bfloat16, 4)
        if t.shape != ref.shape:
            raise ValueError(f"{n} must have the shape of its input")
    ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_cuda:
            raise TypeError("workspace must be a uint8 device tensor")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    st = load_library().fa_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                            _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                                            ws_ptr, ws_bytes, _stream_ptr(stream))
    _check(st, "fa_prefill_backward")
    return dq, dk, dv

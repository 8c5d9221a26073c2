"""Exact blockwise attention forward and (O, lse) merge on MI355X: Python binding of libattn.so.

The binding only marshals arguments: it turns torch tensors into device pointers and the current HIP
stream, calls the C ABI declared in ``include/attn.h``, and raises ``AttnError`` on a non-zero status.
Every step of the computation runs in the library's HIP kernels; torch only provides device memory and
streams.  If the library has not been built, every call raises (there is no fallback).

    o, lse = fwd(q, k, v, causal=True)                # q, k, v: [B, H, N, d] cuda tensors, bf16 or fp32
    o, lse = fwd_chunked(q, k, v, chunks=8, causal=True)
    o, lse = fwd_chunked_noalloc(q, k, v, chunks=8, causal=True)  # partial in a fixed scratch, no allocation
    o, lse = merge(o_a, lse_a, o_b, lse_b)
    o, lse = fwd_acc(q, k, v, o_acc, lse_acc, causal_offset=..., key_range=(lo, hi))   # fold a key range in
    o, lse = fwd_streamed(q, k_host, v_host, chunks=8, causal=True)  # k, v in pinned host memory
"""
from __future__ import annotations

import ctypes
import math
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_F32, ATTN_BF16 = 0, 1
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL_PTR", 2: "ATTN_ERR_BAD_SHAPE", 3: "ATTN_ERR_UNSUPPORTED_D",
          4: "ATTN_ERR_BAD_DTYPE", 5: "ATTN_ERR_BAD_SCALE", 6: "ATTN_ERR_WORKSPACE_TOO_SMALL",
          7: "ATTN_ERR_BAD_ALIAS", 8: "ATTN_ERR_HIP", 9: "ATTN_ERR_MISALIGNED"}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {STATUS.get(status, status)} ({detail})")


def lib() -> ctypes.CDLL:
    """Load libattn.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m exact_blockwise_attention_fwd_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, ll, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_longlong, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    L.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, ll, ll, i, i, vp]
    L.attn_fwd_acc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, ll, ll, i, i, vp]
    L.attn_merge.argtypes = [vp, vp, vp, vp, vp, vp, ll, i, i, i, vp]
    L.attn_fwd_chunked_workspace_bytes.argtypes = [i, i, i, i, i]
    L.attn_fwd_chunked_workspace_bytes.restype = sz
    L.attn_fwd_chunked.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    L.attn_fwd_chunked_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    L.attn_fwd_streamed_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.attn_fwd_streamed_workspace_bytes.restype = sz
    L.attn_fwd_streamed.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, sz, vp, vp]
    L.attn_ffn_workspace_bytes.argtypes = [ll, i, ll]
    L.attn_ffn_workspace_bytes.restype = sz
    L.attn_ffn_blockwise.argtypes = [vp, vp, vp, vp, vp, vp, ll, i, i, ll, i, vp, sz, vp]
    L.attn_strerror.argtypes = [i]
    L.attn_strerror.restype = ctypes.c_char_p
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_timing_enable.argtypes = [i]
    L.attn_timing_read.argtypes = [ctypes.POINTER(ll), ctypes.POINTER(ctypes.c_double)]
    for name in ("attn_fwd", "attn_fwd_ex", "attn_fwd_acc", "attn_merge", "attn_fwd_chunked",
                 "attn_fwd_chunked_noalloc", "attn_fwd_streamed",
                 "attn_ffn_blockwise", "attn_timing_enable", "attn_timing_read"):
        getattr(L, name).restype = i
    _lib = L
    return L


def _check(status: int, func: str):
    if status != 0:
        raise AttnError(status, func, lib().attn_last_error().decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _torch_dtype(code: int):
    import torch
    return torch.bfloat16 if code == ATTN_BF16 else torch.float32


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _on(t):
    """The library launches on the current HIP device: make it the tensors' device for the call."""
    import torch
    return torch.cuda.device(t.device)


def _same_device(t, device, name):
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _need(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _qkv(q, k, v):
    """q [B,H,N_q,d]; k and v [B,H,N_kv,d] of q's dtype and device."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, N_q, d], got shape {tuple(q.shape)}")
    B, H, _, d = q.shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError(f"k must be [B, H, N_kv, d] matching q {tuple(q.shape)}, got {tuple(k.shape)}")
    _same_shape(v, k.shape, "v")
    for t, n in ((k, "k"), (v, "v")):
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{n} must have q's dtype and device")
    return _dtype_code(q)


def _out(out, shape, code, device, name):
    """A new output tensor, or the caller's after checking that it is exactly what the call writes."""
    import torch
    if out is None:
        return torch.empty(tuple(shape), dtype=_torch_dtype(code), device=device)
    _need(out, name)
    _same_shape(out, shape, name)
    if out.dtype != _torch_dtype(code) or out.device != device:
        raise ValueError(f"{name} must be {_torch_dtype(code)} on {device}, got {out.dtype} on {out.device}")
    return out


def _out_code(out, out_dtype, default: int) -> int:
    """Output dtype code: the given output tensor's, else out_dtype, else the input's."""
    import torch
    if out is not None:
        if out_dtype is not None and out.dtype != out_dtype:
            raise ValueError(f"out is {out.dtype} but out_dtype is {out_dtype}")
        return _dtype_code(out)
    return default if out_dtype is None else _dtype_code(torch.empty(0, dtype=out_dtype))


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """Exact attention over all keys.  q [B,H,N_q,d], k and v [B,H,N_kv,d] -> (o [B,H,N_q,d], lse fp32)."""
    dt = _qkv(q, k, v)
    B, H, N_q, d = q.shape
    N_kv = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = _out(out, q.shape, dt, q.device, "out")
    lse = _out(lse, (B, H, N_q), ATTN_F32, q.device, "lse")
    with _on(q):
        _check(lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                              B, H, N_q, N_kv, d, int(causal), scale, dt, _stream(q)), "attn_fwd")
    return out, lse


def fwd_ex(q, k, v, causal: bool = False, scale: float | None = None, causal_offset: int | None = None,
           key_range: tuple[int, int] | None = None, out_dtype=None, out=None, lse=None):
    """Attention of q against keys [lo, hi) of k and v with an explicit causal offset and output dtype."""
    dt = _qkv(q, k, v)
    B, H, N_q, d = q.shape
    n_total = k.shape[2]
    lo, hi = key_range if key_range is not None else (0, n_total)
    if not (0 <= lo <= hi <= n_total):
        raise ValueError(f"key_range {key_range} outside [0, {n_total}]")
    odt = _out_code(out, out_dtype, dt)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    offset = (hi - lo) - N_q if causal_offset is None else int(causal_offset)
    out = _out(out, q.shape, odt, q.device, "out")
    lse = _out(lse, (B, H, N_q), ATTN_F32, q.device, "lse")
    es = q.element_size()
    with _on(q):
        _check(lib().attn_fwd_ex(q.data_ptr(), k.data_ptr() + lo * d * es, v.data_ptr() + lo * d * es,
                                 out.data_ptr(), lse.data_ptr(), B, H, N_q, hi - lo, d, int(causal), scale,
                                 offset, n_total * d, dt, odt, _stream(q)), "attn_fwd_ex")
    return out, lse


def fwd_acc(q, k, v, o_acc, lse_acc, causal: bool = False, scale: float | None = None,
            causal_offset: int | None = None, key_range: tuple[int, int] | None = None, out_dtype=None,
            out=None, lse=None):
    """fwd_ex over keys [lo, hi) merged, in the kernel's epilogue, into the running fp32 partial
    (o_acc, lse_acc).  With out=o_acc and lse=lse_acc (and an fp32 out_dtype) the fold is in place."""
    import torch
    dt = _qkv(q, k, v)
    for t, n in ((o_acc, "o_acc"), (lse_acc, "lse_acc")):
        _need(t, n)
    B, H, N_q, d = q.shape
    if o_acc.dtype != torch.float32 or lse_acc.dtype != torch.float32:
        raise TypeError("o_acc and lse_acc must be float32")
    if tuple(o_acc.shape) != (B, H, N_q, d) or tuple(lse_acc.shape) != (B, H, N_q):
        raise ValueError("o_acc must be [B, H, N_q, d] and lse_acc [B, H, N_q]")
    if o_acc.device != q.device or lse_acc.device != q.device:
        raise ValueError("o_acc and lse_acc must be on q's device")
    n_total = k.shape[2]
    lo, hi = key_range if key_range is not None else (0, n_total)
    if not (0 <= lo <= hi <= n_total):
        raise ValueError(f"key_range {key_range} outside [0, {n_total}]")
    odt = _out_code(out, out_dtype, dt)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    offset = (hi - lo) - N_q if causal_offset is None else int(causal_offset)
    out = _out(out, q.shape, odt, q.device, "out")
    lse = _out(lse, (B, H, N_q), ATTN_F32, q.device, "lse")
    es = q.element_size()
    with _on(q):
        _check(lib().attn_fwd_acc(q.data_ptr(), k.data_ptr() + lo * d * es, v.data_ptr() + lo * d * es,
                                  o_acc.data_ptr(), lse_acc.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N_q,
                                  hi - lo, d, int(causal), scale, offset, n_total * d, dt, odt, _stream(q)),
               "attn_fwd_acc")
    return out, lse


def merge(o_a, lse_a, o_b, lse_b, out=None, lse=None, out_dtype=None):
    """Combine two partial results (o [..., d], lse [...]) over disjoint key sets."""
    import torch
    for t, n in ((o_a, "o_a"), (lse_a, "lse_a"), (o_b, "o_b"), (lse_b, "lse_b")):
        _need(t, n)
    if o_a.dim() < 1 or tuple(o_a.shape[:-1]) != tuple(lse_a.shape):
        raise ValueError(f"o_a must be lse_a's shape plus d, got {tuple(o_a.shape)} and {tuple(lse_a.shape)}")
    _same_shape(o_b, o_a.shape, "o_b")
    _same_shape(lse_b, lse_a.shape, "lse_b")
    if o_b.dtype != o_a.dtype:
        raise ValueError("o_a and o_b must have the same dtype")
    for t, n in ((lse_a, "lse_a"), (lse_b, "lse_b")):
        if t.dtype != torch.float32:
            raise TypeError(f"{n} must be float32")
    for t, n in ((lse_a, "lse_a"), (o_b, "o_b"), (lse_b, "lse_b")):
        if t.device != o_a.device:
            raise ValueError(f"{n} must be on o_a's device")
    d = o_a.shape[-1]
    rows = lse_a.numel()
    dt = _dtype_code(o_a)
    odt = _out_code(out, out_dtype, dt)
    out = _out(out, o_a.shape, odt, o_a.device, "out")
    lse = _out(lse, lse_a.shape, ATTN_F32, o_a.device, "lse")
    with _on(o_a):
        _check(lib().attn_merge(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(), lse_b.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), rows, d, dt, odt, _stream(o_a)), "attn_merge")
    return out, lse


def workspace_bytes(B: int, H: int, N_q: int, d: int, chunks: int) -> int:
    return int(lib().attn_fwd_chunked_workspace_bytes(B, H, N_q, d, chunks))


def fwd_chunked(q, k, v, chunks: int, causal: bool = False, scale: float | None = None, out=None, lse=None,
                workspace=None):
    """Keys cut into `chunks` contiguous chunks, each attended separately and folded through the merge."""
    import torch
    dt = _qkv(q, k, v)
    B, H, N_q, d = q.shape
    N_kv = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = _out(out, q.shape, dt, q.device, "out")
    lse = _out(lse, (B, H, N_q), ATTN_F32, q.device, "lse")
    need = workspace_bytes(B, H, N_q, d, chunks)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace is not None:
        _need(workspace, "workspace")
        _same_device(workspace, q.device, "workspace")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with _on(q):
        _check(lib().attn_fwd_chunked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                      B, H, N_q, N_kv, d, int(causal), scale, int(chunks), dt, ws_ptr, ws_n,
                                      _stream(q)), "attn_fwd_chunked")
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20   # ATTN_NOALLOC_SCRATCH_BYTES of include/attn.h


def fwd_chunked_noalloc(q, k, v, chunks: int, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """fwd_chunked with the running partial in the library's fixed per-device scratch instead of a workspace
    (attn_fwd_chunked_noalloc): for callers that cannot allocate; with `out` and `lse` given, nothing is
    allocated.  Calls that overlap in time on one device share that scratch and race."""
    dt = _qkv(q, k, v)
    B, H, N_q, d = q.shape
    N_kv = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = _out(out, q.shape, dt, q.device, "out")
    lse = _out(lse, (B, H, N_q), ATTN_F32, q.device, "lse")
    with _on(q):
        _check(lib().attn_fwd_chunked_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                              lse.data_ptr(), B, H, N_q, N_kv, d, int(causal), scale, int(chunks), dt,
                                              _stream(q)), "attn_fwd_chunked_noalloc")
    return out, lse


def streamed_workspace_bytes(B: int, H: int, N_q: int, N_kv: int, d: int, chunks: int, dtype) -> int:
    return int(lib().attn_fwd_streamed_workspace_bytes(B, H, N_q, N_kv, d, chunks, _dtype_code(
        __import__("torch").empty(0, dtype=dtype))))


def fwd_streamed(q, k_host, v_host, chunks: int, causal: bool = False, scale: float | None = None, out=None,
                 lse=None, workspace=None, copy_stream=None):
    """fwd_chunked with k and v in host memory ([B,H,N_kv,d] CPU tensors, pinned for overlap): chunk p+1 is
    copied to the device on `copy_stream` (a torch stream other than the current one) while chunk p computes."""
    import torch
    _need(q, "q")
    for t, n in ((k_host, "k_host"), (v_host, "v_host")):
        if t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous host tensor")
        if t.dtype != q.dtype:
            raise TypeError(f"{n} must have q's dtype")
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, N_q, d], got shape {tuple(q.shape)}")
    B, H, N_q, d = q.shape
    if k_host.dim() != 4 or k_host.shape[0] != B or k_host.shape[1] != H or k_host.shape[3] != d:
        raise ValueError(f"k_host must be [B, H, N_kv, d] matching q {tuple(q.shape)}, got {tuple(k_host.shape)}")
    _same_shape(v_host, k_host.shape, "v_host")
    N_kv = k_host.shape[2]
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = _out(out, q.shape, dt, q.device, "out")
    lse = _out(lse, (B, H, N_q), ATTN_F32, q.device, "lse")
    need = streamed_workspace_bytes(B, H, N_q, N_kv, d, chunks, q.dtype)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace")
    _same_device(workspace, q.device, "workspace")
    if copy_stream is None:
        copy_stream = torch.cuda.Stream(device=q.device)
    elif copy_stream.device != q.device:
        raise ValueError(f"copy_stream must be on {q.device}, got {copy_stream.device}")
    with _on(q):
        _check(lib().attn_fwd_streamed(q.data_ptr(), k_host.data_ptr(), v_host.data_ptr(), out.data_ptr(),
                                       lse.data_ptr(), B, H, N_q, N_kv, d, int(causal), scale, int(chunks), dt,
                                       workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q),
                                       ctypes.c_void_p(copy_stream.cuda_stream)), "attn_fwd_streamed")
    return out, lse


ATTN_ACT = {"none": 0, "relu": 1, "gelu": 2}


def ffn_workspace_bytes(M: int, d_ff: int, block: int) -> int:
    return int(lib().attn_ffn_workspace_bytes(int(M), int(d_ff), int(block)))


def ffn_blockwise(x, w1, b1, w2, b2, block: int | None = None, act: str = "gelu", out=None, workspace=None):
    """Blockwise feed-forward: act(x W1^T + b1) W2^T + b2 for every row of x [..., d_model] (bf16), the rows
    taken in contiguous blocks of `block` (default 4096); w1 [d_ff, d_model], w2 [d_model, d_ff] bf16;
    b1 [d_ff], b2 [d_model] fp32 or None."""
    import torch
    for t, n in ((x, "x"), (w1, "w1"), (w2, "w2")):
        _need(t, n)
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16")
    d_model = x.shape[-1]
    d_ff = w1.shape[0]
    _same_shape(w1, (d_ff, d_model), "w1")
    _same_shape(w2, (d_model, d_ff), "w2")
    for t, n, size in ((b1, "b1", d_ff), (b2, "b2", d_model)):
        if t is not None:
            _need(t, n)
            _same_shape(t, (size,), n)
            if t.dtype != torch.float32:
                raise TypeError(f"{n} must be float32")
    for t, n in ((w1, "w1"), (w2, "w2"), (b1, "b1"), (b2, "b2")):
        if t is not None and t.device != x.device:
            raise ValueError(f"{n} must be on x's device")
    if act not in ATTN_ACT:
        raise ValueError(f"act must be one of {sorted(ATTN_ACT)}")
    M = x.numel() // d_model
    block = 4096 if block is None else int(block)
    out = _out(out, x.shape, ATTN_BF16, x.device, "out")
    need = ffn_workspace_bytes(M, d_ff, block)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace")
    _same_device(workspace, x.device, "workspace")
    with _on(x):
        _check(lib().attn_ffn_blockwise(x.data_ptr(), w1.data_ptr(), None if b1 is None else b1.data_ptr(),
                                        w2.data_ptr(), None if b2 is None else b2.data_ptr(), out.data_ptr(), M,
                                        d_model, d_ff, block, ATTN_ACT[act], workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), _stream(x)),
               "attn_ffn_blockwise")
    return out


def timing_enable(on: bool = True):
    _check(lib().attn_timing_enable(int(on)), "attn_timing_enable")


def timing_read():
    """{'fwd': (launches, total_ms), 'merge': (...), 'copy': (chunk copies, total_ms), 'ffn': (GEMM launches,
    total_ms)} since the last read."""
    counts = (ctypes.c_longlong * 4)()
    ms = (ctypes.c_double * 4)()
    _check(lib().attn_timing_read(counts, ms), "attn_timing_read")
    return {"fwd": (counts[0], ms[0]), "merge": (counts[1], ms[1]), "copy": (counts[2], ms[2]),
            "ffn": (counts[3], ms[3])}

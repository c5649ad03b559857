"""MI355X (gfx950) IO-aware exact attention: Python binding of libfa.so.

The functions named like the C ABI (``fa_fwd``, ``fa_bwd``, ``fa_fwd_ex``,
``fa_bwd_ex``, ``fa_bwd_workspace_size``, ``fa_strerror``) only marshal
arguments: they read shapes, dtype, device pointers and the current HIP
stream from torch tensors and call the library, which does every step of the
computation in its own kernels. ``forward``/``backward`` additionally
allocate the outputs (and the backward workspace) with torch. There is no
fallback: if libfa.so is missing, or a tensor is not on the GPU, these raise.

Grouped K/V heads are expressed by the shape of k and v ([B, Hkv, N, d] with
Hkv dividing H); a local window by ``window=(left, right)`` where a negative
(or None) bound is unbounded on that side. ``fa_fwd_fp8``/``forward_fp8``
take Q, K, V as OCP FP8 E4M3 codes with one dequantization factor each.
``fa_fwd_sparse``/``fa_bwd_sparse`` (and ``block_mask=`` of ``forward`` and
``backward``) take a [ceil(N/64)]^2 byte map of the (64-row query block,
64-key block) pairs whose scores are kept.
"""

from __future__ import annotations

import contextlib
import ctypes
import math

import torch

from . import _lib

__all__ = ["FaError", "fa_fwd", "fa_bwd", "fa_fwd_ex", "fa_fwd_keysplit", "fa_bwd_ex",
           "fa_bwd_workspace_size",
           "fa_fwd_num_splits", "fa_fwd_splitkv_workspace_size", "fa_fwd_splitkv",
           "fa_fwd_fp8", "fa_fwd_sparse", "fa_bwd_sparse", "fa_bwd_noalloc", "fa_strerror",
           "forward",
           "forward_fp8", "backward", "DTYPES", "FP8_DTYPES", "MASK_BLOCK"]

DTYPES = {torch.float32: _lib.FA_F32, torch.float16: _lib.FA_F16,
          torch.bfloat16: _lib.FA_BF16}
# Tensor types accepted as E4M3 codes by fa_fwd_fp8 (the bytes are used as is).
FP8_DTYPES = (torch.float8_e4m3fn, torch.uint8)


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_strerror(status)} (status {status})")


def fa_strerror(status: int) -> str:
    return _lib.load().fa_strerror(status).decode()


def fa_bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(_lib.load().fa_bwd_workspace_size(B, H, N, d))


def _check(tensors: dict, shape, dtype) -> None:
    shape = tuple(shape)
    for name, t in tensors.items():
        if t.dtype is dtype and t.shape == shape and t.is_cuda and t.is_contiguous():
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        raise ValueError(f"{name}: expected contiguous {shape} {dtype}, got "
                         f"{tuple(t.shape)} {t.dtype} contiguous={t.is_contiguous()}")


# The raw current-stream handle of a device, without building a torch Stream
# object per call (a few microseconds saved on every call of a short kernel).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(t.get_device())
        return torch.cuda.current_stream(t.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _on_device(t: torch.Tensor):
    """Context that makes t's GPU current (a no-op when it already is)."""
    idx = t.get_device()
    if idx == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(idx)


def _shape(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    if q.dtype not in DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    return tuple(q.shape)


def fa_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None) -> None:
    """Enqueue the forward kernel: o, lse <- attention(q, k, v)."""
    B, H, N, d = _shape(q)
    _check({"q": q, "k": k, "v": v, "o": o}, (B, H, N, d), q.dtype)
    _check({"lse": lse}, (B, H, N), torch.float32)
    with _on_device(q):
        st = _lib.load().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                                DTYPES[q.dtype], _stream(q, stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd")


def fa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool, workspace,
           stream=None) -> None:
    """Enqueue the backward kernels: dq, dk, dv <- gradients of sum(do * o)."""
    B, H, N, d = _shape(q)
    _check({"q": q, "k": k, "v": v, "o": o, "do": do, "dq": dq, "dk": dk, "dv": dv},
           (B, H, N, d), q.dtype)
    _check({"lse": lse}, (B, H, N), torch.float32)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    with _on_device(q):
        st = _lib.load().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                                DTYPES[q.dtype], workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), _stream(q, stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_bwd")


def fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool,
                   stream=None) -> None:
    """fa_bwd without a workspace: the library's static per-GPU scratch is
    used instead (no allocation at all; calls overlapping in time on one GPU
    race). Raises FaError (FA_ERR_SCRATCH) for problems too large for it."""
    B, H, N, d = _shape(q)
    _check({"q": q, "k": k, "v": v, "o": o, "do": do, "dq": dq, "dk": dk, "dv": dv},
           (B, H, N, d), q.dtype)
    _check({"lse": lse}, (B, H, N), torch.float32)
    with _on_device(q):
        st = _lib.load().fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                                        dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale),
                                        int(bool(causal)), DTYPES[q.dtype], _stream(q, stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_bwd_noalloc")


def _kv_shape(q, k):
    B, H, N, d = _shape(q)
    if k.dim() != 4:
        raise ValueError("k must be [B, Hkv, N, d]")
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or Hkv < 1 or H % Hkv:
        raise ValueError(f"k: expected [B, Hkv, N, d] with Hkv dividing H={H}, got "
                         f"{tuple(k.shape)}")
    return B, H, Hkv, N, d


_INT32_MAX = 2 ** 31 - 1


def _options(Hkv: int, window):
    """fa_options for Hkv K/V heads and window (left, right); None or a
    negative bound is unbounded. Bounds must fit the C int: a larger one
    would wrap in ctypes, so it is rejected here."""
    wl, wr = (None, None) if window is None else window
    bounds = []
    for name, b in (("left", wl), ("right", wr)):
        if b is not None and int(b) > _INT32_MAX:
            raise ValueError(f"window {name} bound {b} does not fit a 32-bit int "
                             "(any bound >= N - 1 is unbounded; pass None or -1)")
        bounds.append(-1 if b is None or b < 0 else int(b))
    return _lib.FaOptions(Hkv, bounds[0], bounds[1])


def fa_fwd_ex(q, k, v, o, lse, scale: float, causal: bool, window=None, stream=None) -> None:
    """fa_fwd with grouped K/V heads (from k's shape) and a local window."""
    B, H, Hkv, N, d = _kv_shape(q, k)
    _check({"q": q, "o": o}, (B, H, N, d), q.dtype)
    _check({"k": k, "v": v}, (B, Hkv, N, d), q.dtype)
    _check({"lse": lse}, (B, H, N), torch.float32)
    opts = _options(Hkv, window)
    with _on_device(q):
        st = _lib.load().fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                                   DTYPES[q.dtype], ctypes.byref(opts), _stream(q, stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_ex")


def fa_fwd_keysplit(q, k, v, o, lse, scale: float, causal: bool, window=None,
                    stream=None) -> None:
    """fa_fwd_ex computed by the key-split kernel (bf16/fp16), whatever the
    shape."""
    B, H, Hkv, N, d = _kv_shape(q, k)
    _check({"q": q, "o": o}, (B, H, N, d), q.dtype)
    _check({"k": k, "v": v}, (B, Hkv, N, d), q.dtype)
    _check({"lse": lse}, (B, H, N), torch.float32)
    opts = _options(Hkv, window)
    with _on_device(q):
        st = _lib.load().fa_fwd_keysplit(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                         lse.data_ptr(), B, H, N, d, float(scale),
                                         int(bool(causal)), DTYPES[q.dtype], ctypes.byref(opts),
                                         _stream(q, stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_keysplit")


def fa_bwd_ex(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool, workspace,
              window=None, stream=None) -> None:
    """fa_bwd with grouped K/V heads (from k's shape) and a local window."""
    B, H, Hkv, N, d = _kv_shape(q, k)
    _check({"q": q, "o": o, "do": do, "dq": dq}, (B, H, N, d), q.dtype)
    _check({"k": k, "v": v, "dk": dk, "dv": dv}, (B, Hkv, N, d), q.dtype)
    _check({"lse": lse}, (B, H, N), torch.float32)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    opts = _options(Hkv, window)
    with _on_device(q):
        st = _lib.load().fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                                   DTYPES[q.dtype], ctypes.byref(opts), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(),
                                   _stream(q, stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_bwd_ex")


def fa_fwd_num_splits(B: int, H: int, N: int, d: int, dtype) -> int:
    """Split count fa_fwd_splitkv picks for num_splits=0 (dtype: torch dtype)."""
    return int(_lib.load().fa_fwd_num_splits(B, H, N, d, DTYPES[dtype]))


def fa_fwd_splitkv_workspace_size(B: int, H: int, N: int, d: int, dtype,
                                  num_splits: int = 0) -> int:
    return int(_lib.load().fa_fwd_splitkv_workspace_size(B, H, N, d, DTYPES[dtype],
                                                         num_splits))


def fa_fwd_splitkv(q, k, v, o, lse, scale: float, causal: bool, num_splits: int, workspace,
                   window=None, stream=None) -> None:
    """fa_fwd_ex computed with split-KV: the key tiles of every query tile in
    ``num_splits`` slices (0 = the library's choice), merged afterwards.
    ``workspace`` may be None when fa_fwd_splitkv_workspace_size is 0."""
    B, H, Hkv, N, d = _kv_shape(q, k)
    _check({"q": q, "o": o}, (B, H, N, d), q.dtype)
    _check({"k": k, "v": v}, (B, Hkv, N, d), q.dtype)
    _check({"lse": lse}, (B, H, N), torch.float32)
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    opts = _options(Hkv, window)
    with _on_device(q):
        st = _lib.load().fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        lse.data_ptr(), B, H, N, d, float(scale),
                                        int(bool(causal)), DTYPES[q.dtype], ctypes.byref(opts),
                                        int(num_splits), ws_ptr, ws_bytes, _stream(q, stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_splitkv")


def fa_fwd_fp8(q8, k8, v8, o, lse, scale: float, causal: bool, q_descale: float,
               k_descale: float, v_descale: float, window=None, stream=None) -> None:
    """Enqueue the 8-bit forward: q8, k8, v8 hold E4M3 codes (float8_e4m3fn or
    uint8 tensors; k8, v8 [B, Hkv, N, d]); o (bf16 or fp16) and lse receive
    the attention of the dequantized values descale * code."""
    if q8.dim() != 4:
        raise ValueError("q8 must be [B, H, N, d]")
    B, H, N, d = tuple(q8.shape)
    if k8.dim() != 4 or k8.shape[1] < 1 or H % k8.shape[1]:
        raise ValueError(f"k8: expected [B, Hkv, N, d] with Hkv dividing H={H}")
    Hkv = k8.shape[1]
    for name, t, shape in (("q8", q8, (B, H, N, d)), ("k8", k8, (B, Hkv, N, d)),
                           ("v8", v8, (B, Hkv, N, d))):
        if not t.is_cuda or t.dtype not in FP8_DTYPES or tuple(t.shape) != shape \
                or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous {shape} float8_e4m3fn/uint8 GPU tensor,"
                             f" got {tuple(t.shape)} {t.dtype}")
    if o.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("o must be bfloat16 or float16")
    _check({"o": o}, (B, H, N, d), o.dtype)
    _check({"lse": lse}, (B, H, N), torch.float32)
    opts = _options(Hkv, window)
    with _on_device(q8):
        st = _lib.load().fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                                    float(q_descale), float(k_descale), float(v_descale),
                                    DTYPES[o.dtype], ctypes.byref(opts), _stream(q8, stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_fp8")


MASK_BLOCK = _lib.FA_MASK_BLOCK


def _check_mask(mask, N: int, device) -> None:
    nmb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    if not mask.is_cuda or mask.device != device or mask.dtype not in (torch.uint8, torch.bool) \
            or tuple(mask.shape) != (nmb, nmb) or not mask.is_contiguous():
        raise ValueError(f"block_mask: expected a contiguous ({nmb}, {nmb}) uint8/bool tensor on "
                         f"{device}, got {tuple(mask.shape)} {mask.dtype} on {mask.device}")


def fa_fwd_sparse(q, k, v, o, lse, scale: float, causal: bool, block_mask, window=None,
                  stream=None) -> None:
    """fa_fwd_ex under a block mask: ``block_mask`` is a [ceil(N/64)]^2 uint8
    (or bool) GPU tensor; query block i sees key block j where it is nonzero."""
    B, H, Hkv, N, d = _kv_shape(q, k)
    _check({"q": q, "o": o}, (B, H, N, d), q.dtype)
    _check({"k": k, "v": v}, (B, Hkv, N, d), q.dtype)
    _check({"lse": lse}, (B, H, N), torch.float32)
    _check_mask(block_mask, N, q.device)
    opts = _options(Hkv, window)
    with _on_device(q):
        st = _lib.load().fa_fwd_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), B, H, N, d, float(scale),
                                       int(bool(causal)), DTYPES[q.dtype], ctypes.byref(opts),
                                       block_mask.data_ptr(), _stream(q, stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_sparse")


def fa_bwd_sparse(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool, block_mask,
                  workspace, window=None, stream=None) -> None:
    """fa_bwd_ex under the forward's block mask."""
    B, H, Hkv, N, d = _kv_shape(q, k)
    _check({"q": q, "o": o, "do": do, "dq": dq}, (B, H, N, d), q.dtype)
    _check({"k": k, "v": v, "dk": dk, "dv": dv}, (B, Hkv, N, d), q.dtype)
    _check({"lse": lse}, (B, H, N), torch.float32)
    _check_mask(block_mask, N, q.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    opts = _options(Hkv, window)
    with _on_device(q):
        st = _lib.load().fa_bwd_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                                       dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale),
                                       int(bool(causal)), DTYPES[q.dtype], ctypes.byref(opts),
                                       block_mask.data_ptr(), workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(q, stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_bwd_sparse")


def forward_fp8(q8, k8, v8, descale=(1.0, 1.0, 1.0), causal: bool = False,
                scale: float | None = None, out_dtype=torch.bfloat16, window=None, stream=None):
    """Allocate O (``out_dtype``) and LSE with torch and run fa_fwd_fp8;
    ``descale`` = (q_descale, k_descale, v_descale). Returns (o, lse)."""
    B, H, N, d = tuple(q8.shape)
    o = torch.empty((B, H, N, d), dtype=out_dtype, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    fa_fwd_fp8(q8, k8, v8, o, lse, _default_scale(d, scale), causal, *descale, window=window,
               stream=stream)
    return o, lse


def _plain(q, k, window) -> bool:
    return window is None and k.dim() == 4 and k.shape[1] == q.shape[1]


def _default_scale(d: int, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def forward(q, k, v, causal: bool = False, scale: float | None = None, stream=None,
            window=None, num_splits: int | None = None, block_mask=None,
            key_split: bool = False):
    """Allocate O and LSE with torch and run fa_fwd (fa_fwd_ex when k, v have
    fewer heads than q or a window is given; fa_fwd_splitkv, with a workspace
    allocated here, when ``num_splits`` is given; fa_fwd_sparse when
    ``block_mask`` is given; fa_fwd_keysplit when ``key_split``); returns
    (o, lse)."""
    B, H, N, d = _shape(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if key_split and (block_mask is not None or num_splits is not None):
        raise ValueError("key_split cannot be combined with block_mask or num_splits")
    if key_split:
        fa_fwd_keysplit(q, k, v, o, lse, _default_scale(d, scale), causal, window, stream)
    elif block_mask is not None:
        if num_splits is not None:
            raise ValueError("block_mask and num_splits cannot be combined")
        fa_fwd_sparse(q, k, v, o, lse, _default_scale(d, scale), causal, block_mask, window,
                      stream)
    elif num_splits is not None:
        nbytes = fa_fwd_splitkv_workspace_size(B, H, N, d, q.dtype, num_splits)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
        fa_fwd_splitkv(q, k, v, o, lse, _default_scale(d, scale), causal, num_splits, ws,
                       window, stream)
    elif _plain(q, k, window):
        fa_fwd(q, k, v, o, lse, _default_scale(d, scale), causal, stream)
    else:
        fa_fwd_ex(q, k, v, o, lse, _default_scale(d, scale), causal, window, stream)
    return o, lse


def backward(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None,
             stream=None, workspace=None, window=None, block_mask=None):
    """Allocate dQ, dK, dV (and the workspace unless given) and run fa_bwd
    (fa_bwd_ex when k, v have fewer heads than q or a window is given,
    fa_bwd_sparse when ``block_mask`` is given)."""
    B, H, N, d = _shape(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        workspace = torch.empty(fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8,
                                device=q.device)
    if block_mask is not None:
        fa_bwd_sparse(q, k, v, o, do, lse, dq, dk, dv, _default_scale(d, scale), causal,
                      block_mask, workspace, window, stream)
    elif _plain(q, k, window):
        fa_bwd(q, k, v, o, do, lse, dq, dk, dv, _default_scale(d, scale), causal, workspace,
               stream)
    else:
        fa_bwd_ex(q, k, v, o, do, lse, dq, dk, dv, _default_scale(d, scale), causal, workspace,
                  window, stream)
    return dq, dk, dv

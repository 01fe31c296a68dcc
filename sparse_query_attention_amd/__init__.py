"""Sparse Query Attention (SQA) forward pass on AMD MI355X (gfx950).

SQA ("Sparse Query Attention (SQA): A Computationally Efficient Attention
Mechanism with Query Heads Reduction", arXiv 2510.01817, abstract) is
grouped-query attention with only H_q < H query heads, so its score FLOPs
scale with H_q. Query head i reads key/value head floor(i / (H_q/H_kv)), and
the query and output projections are narrowed to the H_q used heads
(ReactiveAI/xSMQAT-m model card, description).

This package is a thin binding of ``libsqa.so`` (C ABI in include/sqa.h).
Tensors are torch device tensors, used only for memory and streams. Every
arithmetic step runs in the library's HIP kernels. There is no CPU fallback:
if the library is missing, importing the functions still works but calling
them raises.
"""
from __future__ import annotations

from typing import Optional, Tuple

from . import _lib
from ._lib import SQAError

__all__ = ["forward_varlen", "forward_train", "backward", "prefill", "decode_step", "forward",
           "forward_noalloc", "qkv_projection", "attention", "output_projection", "padded_length",
           "SQAError", "library_path"]

library_path = _lib.LIB_PATH


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return _lib.SQA_DTYPE_FP32
    if t.dtype == torch.bfloat16:
        return _lib.SQA_DTYPE_BF16
    raise NotImplementedError(f"dtype {t.dtype} is not supported (float32 or bfloat16)")


def _check_tensor(name: str, t, shape, dtype, device) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def padded_length(N: int) -> int:
    """Sequence length Np of the q/k/vt layouts (N rounded up to 256)."""
    return int(_lib.load().sqa_padded_length(N))


def forward(x, Wq, Wk, Wv, Wo, *, H: int, H_q: int, H_kv: int, causal: bool = False, out=None):
    """Y = SQA(x) for x [B, N, d_model]; weights stored [in, out] (y = x W):
    Wq [d_model, H_q*d], Wk/Wv [d_model, H_kv*d], Wo [H_q*d, d_model], with
    d = d_model / H. Runs on the current stream of x's device."""
    lib = _lib.load()
    if x.dim() != 3:
        raise ValueError("x must be [B, N, d_model]")
    B, N, D = x.shape
    if H <= 0 or D % H:
        raise ValueError("d_model must be a multiple of H")
    d = D // H
    if out is None:
        out = _torch().empty_like(x)
    for name, t, shp in (("x", x, (B, N, D)), ("Wq", Wq, (D, H_q * d)), ("Wk", Wk, (D, H_kv * d)),
                         ("Wv", Wv, (D, H_kv * d)), ("Wo", Wo, (H_q * d, D)), ("out", out, (B, N, D))):
        _check_tensor(name, t, shp, x.dtype, x.device)
    _lib.check(lib.sqa_forward(x.data_ptr(), Wq.data_ptr(), Wk.data_ptr(), Wv.data_ptr(),
                               Wo.data_ptr(), out.data_ptr(), B, N, D, H, H_q, H_kv, d,
                               int(bool(causal)), _dtype_code(x), _stream(x.device)))
    return out


def forward_noalloc(x, Wq, Wk, Wv, Wo, *, H: int, H_q: int, H_kv: int, causal: bool = False,
                    out):
    """forward() through sqa_forward_noalloc: the library allocates nothing and
    takes its workspace from its fixed device array (SQA_NOALLOC_SCRATCH_BYTES,
    128 MiB); `out` must be given. Calls that may overlap in time on one device
    share that array and race."""
    lib = _lib.load()
    if x.dim() != 3:
        raise ValueError("x must be [B, N, d_model]")
    B, N, D = x.shape
    if H <= 0 or D % H:
        raise ValueError("d_model must be a multiple of H")
    d = D // H
    for name, t, shp in (("x", x, (B, N, D)), ("Wq", Wq, (D, H_q * d)), ("Wk", Wk, (D, H_kv * d)),
                         ("Wv", Wv, (D, H_kv * d)), ("Wo", Wo, (H_q * d, D)), ("out", out, (B, N, D))):
        _check_tensor(name, t, shp, x.dtype, x.device)
    _lib.check(lib.sqa_forward_noalloc(x.data_ptr(), Wq.data_ptr(), Wk.data_ptr(), Wv.data_ptr(),
                                       Wo.data_ptr(), out.data_ptr(), B, N, D, H, H_q, H_kv, d,
                                       int(bool(causal)), _dtype_code(x), _stream(x.device)))
    return out


def forward_train(x, Wq, Wk, Wv, Wo, *, H: int, H_q: int, H_kv: int, causal: bool = False,
                  out=None):
    """forward() that also keeps the activations backward() needs
    (sqa_forward_train). Returns (out, saved); saved is an opaque uint8 device
    tensor to pass to backward() with the same inputs."""
    lib = _lib.load()
    if x.dim() != 3:
        raise ValueError("x must be [B, N, d_model]")
    B, N, D = x.shape
    if H <= 0 or D % H:
        raise ValueError("d_model must be a multiple of H")
    d = D // H
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    for name, t, shp in (("x", x, (B, N, D)), ("Wq", Wq, (D, H_q * d)), ("Wk", Wk, (D, H_kv * d)),
                         ("Wv", Wv, (D, H_kv * d)), ("Wo", Wo, (H_q * d, D)), ("out", out, (B, N, D))):
        _check_tensor(name, t, shp, x.dtype, x.device)
    nbytes = int(lib.sqa_training_saved_bytes(B, N, H_q, H_kv, d, _dtype_code(x)))
    if nbytes == 0 and B * N > 0:
        raise ValueError("invalid shape for sqa_forward_train")
    saved = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    _lib.check(lib.sqa_forward_train(x.data_ptr(), Wq.data_ptr(), Wk.data_ptr(), Wv.data_ptr(),
                                     Wo.data_ptr(), out.data_ptr(), saved.data_ptr(), saved.numel(),
                                     B, N, D, H, H_q, H_kv, d, int(bool(causal)), _dtype_code(x),
                                     _stream(x.device)))
    return out, saved


def backward(x, Wq, Wk, Wv, Wo, dy, *, H: int, H_q: int, H_kv: int, causal: bool = False,
             saved=None, out=None):
    """Gradients of the SQA layer (sqa_backward): for Y = forward(x, ...) and
    dy = dL/dY, returns (dx, dWq, dWk, dWv, dWo) with the shapes of x and the
    weights. `saved` is forward_train()'s buffer for the same inputs (None:
    the activations are recomputed). `out` may pass the five tensors to write."""
    lib = _lib.load()
    if x.dim() != 3:
        raise ValueError("x must be [B, N, d_model]")
    B, N, D = x.shape
    if H <= 0 or D % H:
        raise ValueError("d_model must be a multiple of H")
    d = D // H
    torch = _torch()
    if out is None:
        out = (torch.empty_like(x), torch.empty_like(Wq), torch.empty_like(Wk),
               torch.empty_like(Wv), torch.empty_like(Wo))
    dx, dWq, dWk, dWv, dWo = out
    for name, t, shp in (("x", x, (B, N, D)), ("Wq", Wq, (D, H_q * d)), ("Wk", Wk, (D, H_kv * d)),
                         ("Wv", Wv, (D, H_kv * d)), ("Wo", Wo, (H_q * d, D)), ("dy", dy, (B, N, D)),
                         ("dx", dx, (B, N, D)), ("dWq", dWq, (D, H_q * d)),
                         ("dWk", dWk, (D, H_kv * d)), ("dWv", dWv, (D, H_kv * d)),
                         ("dWo", dWo, (H_q * d, D))):
        _check_tensor(name, t, shp, x.dtype, x.device)
    if saved is not None and (saved.device != x.device or not saved.is_contiguous()):
        raise ValueError("saved must be a contiguous tensor on x's device")
    sp, sn = (saved.data_ptr(), saved.numel() * saved.element_size()) if saved is not None else (0, 0)
    _lib.check(lib.sqa_backward(x.data_ptr(), Wq.data_ptr(), Wk.data_ptr(), Wv.data_ptr(),
                                Wo.data_ptr(), dy.data_ptr(), sp or None, sn, dx.data_ptr(),
                                dWq.data_ptr(), dWk.data_ptr(), dWv.data_ptr(), dWo.data_ptr(), B, N,
                                D, H, H_q, H_kv, d, int(bool(causal)), _dtype_code(x),
                                _stream(x.device)))
    return dx, dWq, dWk, dWv, dWo


def forward_varlen(x, Wq, Wk, Wv, Wo, lens, *, H: int, H_q: int, H_kv: int, causal: bool = False,
                   out=None):
    """forward() over sequences padded to N: lens is an int32 tensor [B] on x's
    device, sequence b being rows 0 .. lens[b]-1 of x[b]. Rows past a sequence's
    length come back as zeros."""
    lib = _lib.load()
    if x.dim() != 3:
        raise ValueError("x must be [B, N, d_model]")
    B, N, D = x.shape
    if H <= 0 or D % H:
        raise ValueError("d_model must be a multiple of H")
    d = D // H
    torch = _torch()
    if lens.dtype != torch.int32 or tuple(lens.shape) != (B,) or lens.device != x.device \
            or not lens.is_contiguous():
        raise ValueError("lens must be a contiguous int32 tensor [B] on x's device")
    if out is None:
        out = torch.empty_like(x)
    for name, t, shp in (("x", x, (B, N, D)), ("Wq", Wq, (D, H_q * d)), ("Wk", Wk, (D, H_kv * d)),
                         ("Wv", Wv, (D, H_kv * d)), ("Wo", Wo, (H_q * d, D)), ("out", out, (B, N, D))):
        _check_tensor(name, t, shp, x.dtype, x.device)
    _lib.check(lib.sqa_forward_varlen(x.data_ptr(), Wq.data_ptr(), Wk.data_ptr(), Wv.data_ptr(),
                                      Wo.data_ptr(), out.data_ptr(), lens.data_ptr(), B, N, D, H,
                                      H_q, H_kv, d, int(bool(causal)), _dtype_code(x),
                                      _stream(x.device)))
    return out


def _check_caches(k_cache, v_cache, B, H_kv, d, x):
    if k_cache.dim() != 4 or tuple(k_cache.shape[:2]) != (B, H_kv) or k_cache.shape[3] != d:
        raise ValueError("k_cache must be [B, H_kv, N_max, d_head]")
    shp = tuple(k_cache.shape)
    _check_tensor("k_cache", k_cache, shp, x.dtype, x.device)
    _check_tensor("v_cache", v_cache, shp, x.dtype, x.device)
    return shp[2]


def prefill(x, Wq, Wk, Wv, Wo, k_cache, v_cache, *, H: int, H_q: int, H_kv: int, out=None):
    """Causal forward over x [B, N, d_model] that also writes the keys and values
    of tokens 0..N-1 to rows 0..N-1 of k_cache / v_cache [B, H_kv, N_max, d]."""
    lib = _lib.load()
    B, N, D = x.shape
    d = D // H
    N_max = _check_caches(k_cache, v_cache, B, H_kv, d, x)
    out = _torch().empty_like(x) if out is None else out
    for name, t, shp in (("x", x, (B, N, D)), ("Wq", Wq, (D, H_q * d)), ("Wk", Wk, (D, H_kv * d)),
                         ("Wv", Wv, (D, H_kv * d)), ("Wo", Wo, (H_q * d, D)), ("out", out, (B, N, D))):
        _check_tensor(name, t, shp, x.dtype, x.device)
    _lib.check(lib.sqa_prefill(x.data_ptr(), Wq.data_ptr(), Wk.data_ptr(), Wv.data_ptr(),
                               Wo.data_ptr(), out.data_ptr(), k_cache.data_ptr(),
                               v_cache.data_ptr(), B, N, N_max, D, H, H_q, H_kv, d, _dtype_code(x),
                               _stream(x.device)))
    return out


def decode_step(x_new, Wq, Wk, Wv, Wo, k_cache, v_cache, pos, *, H: int, H_q: int, H_kv: int,
                out=None):
    """One token per sequence: x_new [B, d_model], pos int32 [B] (tokens already
    cached). Writes the tokens' keys/values to cache row pos[b] and returns
    out [B, d_model], row pos[b] of the causal forward."""
    lib = _lib.load()
    torch = _torch()
    if x_new.dim() != 2:
        raise ValueError("x_new must be [B, d_model]")
    B, D = x_new.shape
    d = D // H
    N_max = _check_caches(k_cache, v_cache, B, H_kv, d, x_new)
    if pos.dtype != torch.int32 or tuple(pos.shape) != (B,) or pos.device != x_new.device \
            or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int32 tensor [B] on x_new's device")
    out = torch.empty_like(x_new) if out is None else out
    for name, t, shp in (("x_new", x_new, (B, D)), ("Wq", Wq, (D, H_q * d)), ("Wk", Wk, (D, H_kv * d)),
                         ("Wv", Wv, (D, H_kv * d)), ("Wo", Wo, (H_q * d, D)), ("out", out, (B, D))):
        _check_tensor(name, t, shp, x_new.dtype, x_new.device)
    _lib.check(lib.sqa_decode_step(x_new.data_ptr(), Wq.data_ptr(), Wk.data_ptr(), Wv.data_ptr(),
                                   Wo.data_ptr(), out.data_ptr(), k_cache.data_ptr(),
                                   v_cache.data_ptr(), pos.data_ptr(), B, N_max, D, H, H_q, H_kv,
                                   d, _dtype_code(x_new), _stream(x_new.device)))
    return out


def qkv_projection(x, Wq, Wk, Wv, *, H: int, H_q: int, H_kv: int, q=None, k=None, vt=None
                   ) -> Tuple[object, object, object]:
    """Step 1: returns q [B,H_q,Np,d], k [B,H_kv,Np,d], vt [B,H_kv,d,Np]
    (Np = padded_length(N); padded rows are zero)."""
    lib = _lib.load()
    torch = _torch()
    B, N, D = x.shape
    d = D // H
    Np = padded_length(N)
    q = torch.empty((B, H_q, Np, d), dtype=x.dtype, device=x.device) if q is None else q
    k = torch.empty((B, H_kv, Np, d), dtype=x.dtype, device=x.device) if k is None else k
    vt = torch.empty((B, H_kv, d, Np), dtype=x.dtype, device=x.device) if vt is None else vt
    for name, t, shp in (("x", x, (B, N, D)), ("Wq", Wq, (D, H_q * d)), ("Wk", Wk, (D, H_kv * d)),
                         ("Wv", Wv, (D, H_kv * d)), ("q", q, (B, H_q, Np, d)),
                         ("k", k, (B, H_kv, Np, d)), ("vt", vt, (B, H_kv, d, Np))):
        _check_tensor(name, t, shp, x.dtype, x.device)
    _lib.check(lib.sqa_qkv_projection(x.data_ptr(), Wq.data_ptr(), Wk.data_ptr(), Wv.data_ptr(),
                                      q.data_ptr(), k.data_ptr(), vt.data_ptr(), B, N, D, H, H_q,
                                      H_kv, d, _dtype_code(x), _stream(x.device)))
    return q, k, vt


def attention(q, k, vt, *, N: int, causal: bool = False, a=None):
    """Step 2: a [B*N, H_q*d] from the step-1 layouts."""
    lib = _lib.load()
    torch = _torch()
    B, H_q, Np, d = q.shape
    H_kv = k.shape[1]
    if Np != padded_length(N):
        raise ValueError(f"q has {Np} rows per head, expected padded_length(N)={padded_length(N)}")
    a = torch.empty((B * N, H_q * d), dtype=q.dtype, device=q.device) if a is None else a
    for name, t, shp in (("k", k, (B, H_kv, Np, d)), ("vt", vt, (B, H_kv, d, Np)),
                         ("a", a, (B * N, H_q * d)), ("q", q, (B, H_q, Np, d))):
        _check_tensor(name, t, shp, q.dtype, q.device)
    _lib.check(lib.sqa_attention(q.data_ptr(), k.data_ptr(), vt.data_ptr(), a.data_ptr(), B, N,
                                 H_q, H_kv, d, int(bool(causal)), _dtype_code(q),
                                 _stream(q.device)))
    return a


def output_projection(a, Wo, out=None):
    """Step 3: out [M, d_model] = a [M, K] @ Wo [K, d_model]."""
    lib = _lib.load()
    M, K = a.shape
    D = Wo.shape[1]
    out = _torch().empty((M, D), dtype=a.dtype, device=a.device) if out is None else out
    for name, t, shp in (("a", a, (M, K)), ("Wo", Wo, (K, D)), ("out", out, (M, D))):
        _check_tensor(name, t, shp, a.dtype, a.device)
    _lib.check(lib.sqa_output_projection(a.data_ptr(), Wo.data_ptr(), out.data_ptr(), M, K, D,
                                         _dtype_code(a), _stream(a.device)))
    return out

"""exact_tiled_attention_amd -- Python binding of libattn (gfx950 HIP kernels).

Argument marshalling only: every step of attention runs in the library's kernels.
torch supplies device memory and the current stream.  Importing this package does
not touch the GPU; the first call loads libattn.so and raises if it is missing.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import AttnError, LibraryMissing, lib

__all__ = ["attn_fwd", "attn_fwd_exp_emulated", "exp2_soft", "attn_fwd_varlen", "attn_decode_paged", "attn_fwd_dropout", "fp8_quantize", "attn_fwd_fp8", "attn_bwd_fp8", "attn_bwd", "attn_decode_splitkv", "attn_decode_splitkv_noalloc",
           "bwd_workspace_size", "decode_workspace_size", "fp8_kv_tile",
           "AttnError", "LibraryMissing", "lib"]

_CODES = {torch.float16: _lib.ATTN_F16, torch.bfloat16: _lib.ATTN_BF16, torch.float32: _lib.ATTN_F32}


def _code(dtype):
    if dtype not in _CODES:
        raise TypeError(f"unsupported dtype {dtype}")
    return _CODES[dtype]


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _require(t, name, ndim):
    if t.dim() != ndim or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous {ndim}-d CUDA tensor")


def _expect(t, name, shape, dtype, device):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def attn_fwd(q, k, v, scale=None, causal=False, o=None, lse=None, stream=None):
    """O, LSE = attention(q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d]); fp16/bf16; LSE float32."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, 4)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    _expect(k, "k", (B, Hkv, Sk, d), q.dtype, q.device)
    _expect(v, "v", (B, Hkv, Sk, d), q.dtype, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, Hq, Sq), torch.float32, q.device)
    st = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Sq, Sk, d,
                        scale, int(bool(causal)), _code(q.dtype), _stream(stream))
    _lib.check("attn_fwd", st)
    return o, lse


def attn_fwd_exp_emulated(q, k, v, emulated_per_8, scale=None, causal=False, o=None, lse=None,
                          stream=None):
    """attn_fwd with emulated_per_8 (0, 2 or 4) of every 8 softmax exponentials evaluated by
    the software exp2 on the FMA pipe instead of the exponential unit."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, 4)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    _expect(k, "k", (B, Hkv, Sk, d), q.dtype, q.device)
    _expect(v, "v", (B, Hkv, Sk, d), q.dtype, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, Hq, Sq), torch.float32, q.device)
    st = lib().attn_fwd_exp_emulated(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                     Sq, Sk, d, scale, int(bool(causal)), _code(q.dtype),
                                     int(emulated_per_8), _stream(stream))
    _lib.check("attn_fwd_exp_emulated", st)
    return o, lse


def exp2_soft(x, y=None, stream=None):
    """y = software exp2 of a float32 tensor x (the forward's emulated exponential)."""
    _require(x, "x", x.dim())
    if x.dtype != torch.float32:
        raise TypeError("x must be float32")
    y = torch.empty_like(x) if y is None else y
    _expect(y, "y", x.shape, torch.float32, x.device)
    st = lib().attn_exp2_soft(_ptr(x), _ptr(y), x.numel(), _stream(stream))
    _lib.check("attn_exp2_soft", st)
    return y


def attn_fwd_dropout(q, k, v, dropout_p, seed, offset=0, scale=None, causal=False, o=None, lse=None,
                     stream=None):
    """attn_fwd with attention dropout (keep decisions from Philox4x32-10 by element
    coordinates; LSE of the undropped softmax)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, 4)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    _expect(k, "k", (B, Hkv, Sk, d), q.dtype, q.device)
    _expect(v, "v", (B, Hkv, Sk, d), q.dtype, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, Hq, Sq), torch.float32, q.device)
    st = lib().attn_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Sq, Sk, d, scale,
                                int(bool(causal)), float(dropout_p), int(seed) & (2 ** 64 - 1),
                                int(offset) & 0xFFFFFFFF, _code(q.dtype), _stream(stream))
    _lib.check("attn_fwd_dropout", st)
    return o, lse


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale=None,
                    causal=False, o=None, lse=None, stream=None):
    """O [total_q, Hq, d], LSE [Hq, total_q] of packed token-major sequences
    (q [total_q, Hq, d], k/v [total_k, Hkv, d]; cu_seqlens_* int32 [B+1] on the device)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, n, 3)
    for t, n in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
        _require(t, n, 1)
        if t.dtype != torch.int32:
            raise TypeError(f"{n} must be int32")
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.numel() - 1
    _expect(k, "k", (total_k, Hkv, d), q.dtype, q.device)
    _expect(v, "v", (total_k, Hkv, d), q.dtype, q.device)
    _expect(cu_seqlens_q, "cu_seqlens_q", (B + 1,), torch.int32, q.device)
    _expect(cu_seqlens_k, "cu_seqlens_k", (B + 1,), torch.int32, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (Hq, total_q), torch.float32, q.device)
    st = lib().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                               _ptr(cu_seqlens_k), B, Hq, Hkv, int(max_seqlen_q), int(max_seqlen_k),
                               total_q, total_k, d, scale, int(bool(causal)), _code(q.dtype), _stream(stream))
    _lib.check("attn_fwd_varlen", st)
    return o, lse


def fp8_quantize(x, signs=None, per_tensor=False, codes=None, descale=None, stream=None):
    """E4M3 codes [B,H,S,d] (uint8) and float32 descales [B,H,ceil(S/128)] of x (fp16/bf16),
    optionally after the incoherent transform x diag(signs) H / sqrt(d) (signs: float32 [d])."""
    _require(x, "x", 4)
    B, H, S, d = x.shape
    nb = (S + 127) // 128
    codes = torch.empty((B, H, S, d), dtype=torch.uint8, device=x.device) if codes is None else codes
    descale = torch.empty((B, H, nb), dtype=torch.float32, device=x.device) if descale is None else descale
    _expect(codes, "codes", (B, H, S, d), torch.uint8, x.device)
    _expect(descale, "descale", (B, H, nb), torch.float32, x.device)
    if signs is not None:
        _expect(signs, "signs", (d,), torch.float32, x.device)
    st = lib().attn_fp8_quantize(_ptr(x), _code(x.dtype), B, H, S, d, _ptr(signs), int(bool(per_tensor)),
                                 _ptr(codes), _ptr(descale), _stream(stream))
    _lib.check("attn_fp8_quantize", st)
    return codes, descale


def fp8_kv_tile() -> int:
    return lib().attn_fp8_kv_tile()


_FP8_CODE_DTYPES = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))


def attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, scale=None, o_dtype=torch.bfloat16,
                 o=None, lse=None, stream=None, causal=False):
    """Forward on E4M3FN codes (uint8 or float8_e4m3fn tensors) with 128-row-block descales."""
    # types first (TypeError), then shapes, layout and device (ValueError): nothing
    # reaches the library unless every tensor is what the kernel will read or write
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        if t.dtype not in _FP8_CODE_DTYPES:
            raise TypeError(f"{n} must hold E4M3FN codes (uint8 or float8_e4m3fn), got {t.dtype}")
    for t, n in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        if t.dtype != torch.float32:
            raise TypeError(f"{n} must be float32, got {t.dtype}")
    if o is not None and o.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"o must be bfloat16 or float32, got {o.dtype}")
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        _require(t, n, 4)
    B, Hq, Sq, d = q8.shape
    Hkv, Sk = k8.shape[1], k8.shape[2]
    dev = q8.device
    _expect(k8, "k8", (B, Hkv, Sk, d), k8.dtype, dev)
    _expect(v8, "v8", (B, Hkv, Sk, d), v8.dtype, dev)
    _expect(q_scale, "q_scale", (B, Hq, (Sq + 127) // 128), torch.float32, dev)
    _expect(k_scale, "k_scale", (B, Hkv, (Sk + 127) // 128), torch.float32, dev)
    _expect(v_scale, "v_scale", (B, Hkv, (Sk + 127) // 128), torch.float32, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty((B, Hq, Sq, d), dtype=o_dtype, device=dev) if o is None else o
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev) if lse is None else lse
    _expect(o, "o", (B, Hq, Sq, d), o.dtype, dev)
    _expect(lse, "lse", (B, Hq, Sq), torch.float32, dev)
    st = lib().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                            _ptr(o), _ptr(lse), B, Hq, Hkv, Sq, Sk, d, scale, int(bool(causal)), _code(o.dtype),
                            _stream(stream))
    _lib.check("attn_fwd_fp8", st)
    return o, lse


def attn_bwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, do, scale=None, causal=False,
                 grad_dtype=torch.float32, workspace=None, dq=None, dk=None, dv=None, stream=None):
    """dQ, dK, dV with respect to the dequantised operands of attention on E4M3 codes
    (as attn_fwd_fp8 takes them); o and do bf16, lse float32."""
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        if t.dtype not in _FP8_CODE_DTYPES:
            raise TypeError(f"{n} must hold E4M3FN codes (uint8 or float8_e4m3fn), got {t.dtype}")
    for t, n in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale"), (lse, "lse")):
        if t.dtype != torch.float32:
            raise TypeError(f"{n} must be float32, got {t.dtype}")
    for t, n in ((o, "o"), (do, "do")):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{n} must be bfloat16, got {t.dtype}")
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8"), (o, "o"), (do, "do")):
        _require(t, n, 4)
    B, Hq, Sq, d = q8.shape
    Hkv, Sk = k8.shape[1], k8.shape[2]
    dev = q8.device
    _expect(k8, "k8", (B, Hkv, Sk, d), k8.dtype, dev)
    _expect(v8, "v8", (B, Hkv, Sk, d), v8.dtype, dev)
    _expect(q_scale, "q_scale", (B, Hq, (Sq + 127) // 128), torch.float32, dev)
    _expect(k_scale, "k_scale", (B, Hkv, (Sk + 127) // 128), torch.float32, dev)
    _expect(v_scale, "v_scale", (B, Hkv, (Sk + 127) // 128), torch.float32, dev)
    _expect(o, "o", (B, Hq, Sq, d), torch.bfloat16, dev)
    _expect(do, "do", (B, Hq, Sq, d), torch.bfloat16, dev)
    _expect(lse, "lse", (B, Hq, Sq), torch.float32, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty((B, Hq, Sq, d), dtype=grad_dtype, device=dev) if dq is None else dq
    dk = torch.empty((B, Hkv, Sk, d), dtype=grad_dtype, device=dev) if dk is None else dk
    dv = torch.empty((B, Hkv, Sk, d), dtype=grad_dtype, device=dev) if dv is None else dv
    _expect(dq, "dq", (B, Hq, Sq, d), grad_dtype, dev)
    _expect(dk, "dk", (B, Hkv, Sk, d), grad_dtype, dev)
    _expect(dv, "dv", (B, Hkv, Sk, d), grad_dtype, dev)
    need = bwd_workspace_size(B, Hq, Hkv, Sq, Sk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib().attn_bwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(o),
                            _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, Sq, Sk, d, scale,
                            int(bool(causal)), _code(grad_dtype), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("attn_bwd_fp8", st)
    return dq, dk, dv


def bwd_workspace_size(B, Hq, Hkv, Sq, Sk, d) -> int:
    return lib().attn_bwd_workspace_size(B, Hq, Hkv, Sq, Sk, d)


def attn_bwd(q, k, v, o, lse, do, scale=None, causal=False, grad_dtype=torch.float32,
             workspace=None, dq=None, dk=None, dv=None, stream=None, deterministic=False, dq_splits=1,
             dropout_p=None, seed=0, offset=0, atomic=False):
    """dQ, dK, dV of attn_fwd (dK/dV already summed over each K/V head's query group).
    Default: dQ in the library's form for the key length (atomic adds below 1024 keys,
    the query-row owner from there on).  atomic=True: the column owner's atomic dQ at
    every length.  deterministic=True: no atomics, bitwise-repeatable results; dQ from a
    query-row owner over dq_splits (1, 2, 4, 8, 16) key ranges whose partials are summed
    in a fixed tree.  dropout_p (with seed, offset): the backward of attn_fwd_dropout with
    the same values."""
    if atomic and (deterministic or dropout_p is not None):
        raise ValueError("atomic=True excludes deterministic and dropout_p")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _require(t, n, 4)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    _expect(k, "k", (B, Hkv, Sk, d), q.dtype, q.device)
    _expect(v, "v", (B, Hkv, Sk, d), q.dtype, q.device)
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(do, "do", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, Hq, Sq), torch.float32, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=grad_dtype, device=q.device) if dv is None else dv
    _expect(dq, "dq", q.shape, grad_dtype, q.device)
    _expect(dk, "dk", k.shape, grad_dtype, q.device)
    _expect(dv, "dv", v.shape, grad_dtype, q.device)
    if deterministic:
        need = lib().attn_bwd_deterministic_workspace_size(B, Hq, Hkv, Sq, Sk, d, int(dq_splits))
    else:
        need = bwd_workspace_size(B, Hq, Hkv, Sq, Sk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if dropout_p is not None:
        st = lib().attn_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                    _ptr(dv), B, Hq, Hkv, Sq, Sk, d, scale, int(bool(causal)), float(dropout_p),
                                    int(seed) & (2 ** 64 - 1), int(offset) & 0xFFFFFFFF, _code(q.dtype),
                                    _code(grad_dtype), int(bool(deterministic)), int(dq_splits), _ptr(workspace),
                                    ws_bytes, _stream(stream))
        _lib.check("attn_bwd_dropout", st)
    elif deterministic:
        st = lib().attn_bwd_deterministic(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                                          _ptr(dk), _ptr(dv), B, Hq, Hkv, Sq, Sk, d, scale, int(bool(causal)),
                                          _code(q.dtype), _code(grad_dtype), int(dq_splits), _ptr(workspace),
                                          ws_bytes, _stream(stream))
        _lib.check("attn_bwd_deterministic", st)
    else:
        name = "attn_bwd_atomic" if atomic else "attn_bwd"
        st = getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                  _ptr(dv), B, Hq, Hkv, Sq, Sk, d, scale, int(bool(causal)), _code(q.dtype),
                                  _code(grad_dtype), _ptr(workspace), ws_bytes, _stream(stream))
        _lib.check(name, st)
    return dq, dk, dv


def decode_pick_chunk(B, Hq, Smax) -> int:
    """The library's default split size for this shape (attn_decode_pick_chunk)."""
    return lib().attn_decode_pick_chunk(B, Hq, Smax)


def decode_workspace_size(B, Hq, Smax, d, chunk=None) -> int:
    if chunk is None:
        chunk = decode_pick_chunk(B, Hq, Smax)
    return lib().attn_decode_workspace_size(B, Hq, Smax, d, chunk)


def attn_decode_splitkv(q, k_cache, v_cache, seqlens, scale=None, chunk=None, workspace=None,
                        o=None, lse=None, stream=None):
    """Split-KV decode: q [B,Hq,1,d], caches [B,Hkv,Smax,d], seqlens int32 [B] on device.
    chunk=None takes the library's choice (decode_pick_chunk)."""
    _code(q.dtype)
    if seqlens.dtype != torch.int32:
        raise TypeError(f"seqlens must be int32, got {seqlens.dtype}")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dtype != q.dtype:
            raise TypeError(f"{n} must have q's dtype {q.dtype}, got {t.dtype}")
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _require(t, n, 4)
    B, Hq, _, d = q.shape
    Hkv, Smax = k_cache.shape[1], k_cache.shape[2]
    _expect(q, "q", (B, Hq, 1, d), q.dtype, q.device)
    _expect(k_cache, "k_cache", (B, Hkv, Smax, d), q.dtype, q.device)
    _expect(v_cache, "v_cache", (B, Hkv, Smax, d), q.dtype, q.device)
    _expect(seqlens, "seqlens", (B,), torch.int32, q.device)
    if chunk is None:
        chunk = decode_pick_chunk(B, Hq, Smax)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, Hq, 1), torch.float32, q.device)
    need = decode_workspace_size(B, Hq, Smax, d, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", workspace.dim())
    if workspace.device != q.device:
        raise ValueError(f"workspace must be on {q.device}")
    st = lib().attn_decode_splitkv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(lse),
                                   B, Hq, Hkv, Smax, d, scale, chunk, _code(q.dtype), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("attn_decode_splitkv", st)
    return o, lse


DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20


def attn_decode_splitkv_noalloc(q, k_cache, v_cache, seqlens, scale=None, chunk=None, o=None, lse=None,
                                stream=None):
    """attn_decode_splitkv with the partial states in the library's own per-GPU device
    scratch (no workspace; the library call allocates nothing).  o and lse must be
    given by callers that cannot allocate; chunk=None takes the library's choice."""
    _code(q.dtype)
    if seqlens.dtype != torch.int32:
        raise TypeError(f"seqlens must be int32, got {seqlens.dtype}")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dtype != q.dtype:
            raise TypeError(f"{n} must have q's dtype {q.dtype}, got {t.dtype}")
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _require(t, n, 4)
    B, Hq, _, d = q.shape
    Hkv, Smax = k_cache.shape[1], k_cache.shape[2]
    _expect(q, "q", (B, Hq, 1, d), q.dtype, q.device)
    _expect(k_cache, "k_cache", (B, Hkv, Smax, d), q.dtype, q.device)
    _expect(v_cache, "v_cache", (B, Hkv, Smax, d), q.dtype, q.device)
    _expect(seqlens, "seqlens", (B,), torch.int32, q.device)
    if chunk is None:
        chunk = decode_pick_chunk(B, Hq, Smax)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, Hq, 1), torch.float32, q.device)
    st = lib().attn_decode_splitkv_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o),
                                           _ptr(lse), B, Hq, Hkv, Smax, d, scale, chunk, _code(q.dtype),
                                           _stream(stream))
    _lib.check("attn_decode_splitkv_noalloc", st)
    return o, lse


def attn_decode_paged(q, k_pages, v_pages, block_table, seqlens, scale=None, chunk=None, workspace=None,
                      o=None, lse=None, stream=None):
    """Split-KV decode over a paged pool: q [B,Hq,1,d], pools [num_pages,Hkv,P,d],
    block_table int32 [B, max_pages], seqlens int32 [B], all on the device.
    chunk=None takes the library's choice (decode_pick_chunk over max_pages * P keys)."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _require(t, n, 4)
    _require(block_table, "block_table", 2)
    B, Hq, _, d = q.shape
    num_pages, Hkv, P = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    max_pages = block_table.shape[1]
    _expect(q, "q", (B, Hq, 1, d), q.dtype, q.device)
    _expect(k_pages, "k_pages", (num_pages, Hkv, P, d), q.dtype, q.device)
    _expect(v_pages, "v_pages", (num_pages, Hkv, P, d), q.dtype, q.device)
    _expect(block_table, "block_table", (B, max_pages), torch.int32, q.device)
    _expect(seqlens, "seqlens", (B,), torch.int32, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, Hq, 1), torch.float32, q.device)
    if chunk is None:
        chunk = decode_pick_chunk(B, Hq, max_pages * P)
    need = decode_workspace_size(B, Hq, max_pages * P, d, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib().attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seqlens), _ptr(o),
                                 _ptr(lse), B, Hq, Hkv, num_pages, P, max_pages, d, scale, chunk, _code(q.dtype),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("attn_decode_paged", st)
    return o, lse

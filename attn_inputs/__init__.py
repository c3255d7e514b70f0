"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and bench.py.

This module only draws and stores numbers.  It holds none of the attention
arithmetic: no scores, no softmax, no merge.  The GPU path and the oracle both
consume exactly the tensors produced here (the GPU gets a device copy, the oracle
widens the same stored values to float64), so they share data, never code.

Recipe (every draw is reproducible from its seed):
  * numpy ``default_rng(seed)`` (PCG64); each tensor of a workload gets its own
    sub-stream ``default_rng([seed, tensor_index])``.
  * entries are drawn as float32 N(0, 1) and cast to the storage dtype by torch
    (round-to-nearest-even for fp16 / bf16).
  * split-KV decode lengths are integers drawn uniformly from [lo, hi] inclusive.
  * the fp8 workload draws float32 N(0, 1), multiplies each element independently
    by 20 with probability 0.01 (outliers), then stores e4m3fn codes with one
    float32 descale per (batch, head, 128-row block): scale = amax / 448 (1 if the
    block is all zero) and code = e4m3fn(x / scale) by torch's cast.  The
    quantisation is input preparation: the attention path receives codes + scales.
  * packed variable-length prefill: token-major q [total_q, H_q, d] and k/v
    [total_k, H_kv, d] with int32 cumulative offsets cu_q, cu_k [B+1].
  * paged decode: K/V pools [num_pages, H_kv, P, d] with a seeded random permutation
    of the pages as the int32 block table [B, max_pages]; unused pages hold draws too.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "f32": torch.float32,
}

E4M3_MAX = 448.0
FP8_BLOCK_ROWS = 128


def _rng(seed: int, index: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(index)])


def normal(shape, seed: int, index: int, dtype: str = "f32") -> torch.Tensor:
    """float32 N(0,1) draws cast to ``dtype`` (CPU tensor)."""
    x = _rng(seed, index).standard_normal(size=tuple(shape), dtype=np.float32)
    return torch.from_numpy(x).to(DTYPES[dtype])


def decode_lengths(seed: int, batch: int, lo: int = 1024, hi: int = 32768) -> np.ndarray:
    """Per-sequence K/V lengths, uniform integers in [lo, hi] (int32)."""
    return _rng(seed, 99).integers(lo, hi + 1, size=batch).astype(np.int32)


def outlier_normal(shape, seed: int, index: int, p: float = 0.01, factor: float = 20.0) -> torch.Tensor:
    """float32 N(0,1) with each element independently scaled by ``factor`` w.p. ``p``."""
    g = _rng(seed, index)
    x = g.standard_normal(size=tuple(shape), dtype=np.float32)
    hit = g.random(size=tuple(shape)) < p
    x = np.where(hit, x * np.float32(factor), x).astype(np.float32)
    return torch.from_numpy(x)


def fp8_block_quantize(x: torch.Tensor, block: int = FP8_BLOCK_ROWS):
    """Store float32 ``x`` [B,H,S,d] as e4m3fn codes with one descale per 128-row block.

    Returns (codes: torch.uint8 [B,H,S,d], scales: float32 [B,H,ceil(S/block)]).
    ``x ~= decode(codes) * scale`` row-block-wise.
    """
    B, H, S, d = x.shape
    nblk = (S + block - 1) // block
    pad = nblk * block - S
    xp = torch.nn.functional.pad(x, (0, 0, 0, pad)) if pad else x
    xb = xp.reshape(B, H, nblk, block, d)
    amax = xb.abs().amax(dim=(3, 4))
    scales = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).to(torch.float32)
    q = (xb / scales[..., None, None]).clamp(-E4M3_MAX, E4M3_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(B, H, nblk * block, d)[:, :, :S]
    return codes.contiguous(), scales.contiguous()


@dataclass
class Workload:
    """One named synthetic workload (CPU tensors)."""
    name: str
    tensors: dict = field(default_factory=dict)
    params: dict = field(default_factory=dict)


def prefill(B, Hq, Hkv, Sq, Sk, d, dtype, seed, causal=False, with_grad=False, scale=None) -> Workload:
    """Q [B,Hq,Sq,d], K/V [B,Hkv,Sk,d] (and dO like Q when ``with_grad``)."""
    t = {
        "q": normal((B, Hq, Sq, d), seed, 0, dtype),
        "k": normal((B, Hkv, Sk, d), seed, 1, dtype),
        "v": normal((B, Hkv, Sk, d), seed, 2, dtype),
    }
    if with_grad:
        t["do"] = normal((B, Hq, Sq, d), seed, 3, dtype)
    p = dict(B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, d=d, dtype=dtype, causal=bool(causal),
             scale=float(np.float32(1.0 / math.sqrt(d))) if scale is None else float(np.float32(scale)))
    return Workload(f"prefill_{dtype}_{B}x{Hq}x{Hkv}x{Sq}x{Sk}x{d}", t, p)


def decode(B, Hq, Hkv, d, dtype, seed, lo=1024, hi=32768, chunk=256, lengths=None) -> Workload:
    """q [B,Hq,1,d]; padded caches [B,Hkv,Smax,d] with Smax = max length rounded up to ``chunk``."""
    lens = decode_lengths(seed, B, lo, hi) if lengths is None else np.asarray(lengths, dtype=np.int32)
    smax = int(max(1, -(-int(lens.max()) // chunk) * chunk)) if len(lens) else chunk
    t = {
        "q": normal((B, Hq, 1, d), seed, 0, dtype),
        "k": normal((B, Hkv, smax, d), seed, 1, dtype),
        "v": normal((B, Hkv, smax, d), seed, 2, dtype),
        "seqlens": torch.from_numpy(lens.copy()),
    }
    p = dict(B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, Smax=smax, chunk=chunk,
             scale=float(np.float32(1.0 / math.sqrt(d))))
    return Workload(f"decode_{dtype}_{B}x{Hq}x{Hkv}x{smax}x{d}", t, p)


def fp8_prefill(B, Hq, Hkv, Sq, Sk, d, seed, block=FP8_BLOCK_ROWS) -> Workload:
    """e4m3fn Q/K/V codes + per-128-row-block float32 descales (outlier recipe)."""
    t = {}
    for name, idx, shape in (("q", 0, (B, Hq, Sq, d)), ("k", 1, (B, Hkv, Sk, d)), ("v", 2, (B, Hkv, Sk, d))):
        codes, scales = fp8_block_quantize(outlier_normal(shape, seed, idx), block)
        t[name + "8"] = codes
        t[name + "_scale"] = scales
    p = dict(B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, d=d, dtype="fp8_e4m3", causal=False,
             scale=float(np.float32(1.0 / math.sqrt(d))), block=block)
    return Workload(f"fp8_{B}x{Hq}x{Hkv}x{Sq}x{Sk}x{d}", t, p)


def varlen_prefill(seqlens_q, seqlens_k, Hq, Hkv, d, dtype, seed, causal=False, scale=None) -> Workload:
    """Packed token-major q [sum Sq, Hq, d], k/v [sum Sk, Hkv, d] + cu_q, cu_k [B+1] int32."""
    sq = np.asarray(seqlens_q, dtype=np.int64)
    sk = np.asarray(seqlens_k, dtype=np.int64)
    cq = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(sk)]).astype(np.int32)
    t = {
        "q": normal((int(cq[-1]), Hq, d), seed, 0, dtype),
        "k": normal((int(ck[-1]), Hkv, d), seed, 1, dtype),
        "v": normal((int(ck[-1]), Hkv, d), seed, 2, dtype),
        "cu_q": torch.from_numpy(cq.copy()),
        "cu_k": torch.from_numpy(ck.copy()),
    }
    p = dict(B=len(sq), Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, causal=bool(causal),
             seqlens_q=sq.tolist(), seqlens_k=sk.tolist(), max_seqlen_q=int(sq.max()) if len(sq) else 0, max_seqlen_k=int(sk.max()) if len(sk) else 0,
             scale=float(np.float32(1.0 / math.sqrt(d))) if scale is None else float(np.float32(scale)))
    return Workload(f"varlen_{dtype}_B{len(sq)}x{Hq}x{Hkv}x{d}", t, p)


def paged_decode(B, Hq, Hkv, d, dtype, seed, page_size, lo=1024, hi=32768, chunk=256, lengths=None,
                 spare_pages=3) -> Workload:
    """q [B,Hq,1,d]; K/V pools [num_pages, Hkv, P, d]; block table [B, max_pages] int32
    (a seeded random permutation of all pages); seqlens int32 [B]."""
    lens = decode_lengths(seed, B, lo, hi) if lengths is None else np.asarray(lengths, dtype=np.int32)
    maxp = max(1, -(-int(lens.max()) // page_size)) if len(lens) else 1
    npages = B * maxp + spare_pages
    perm = _rng(seed, 5).permutation(npages)[:B * maxp].astype(np.int32)
    t = {
        "q": normal((B, Hq, 1, d), seed, 0, dtype),
        "k_pages": normal((npages, Hkv, page_size, d), seed, 1, dtype),
        "v_pages": normal((npages, Hkv, page_size, d), seed, 2, dtype),
        "block_table": torch.from_numpy(perm.reshape(B, maxp).copy()),
        "seqlens": torch.from_numpy(lens.copy()),
    }
    p = dict(B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, page_size=page_size, max_pages=maxp, num_pages=npages,
             chunk=chunk, scale=float(np.float32(1.0 / math.sqrt(d))))
    return Workload(f"paged_decode_{dtype}_{B}x{Hq}x{Hkv}x{d}_P{page_size}", t, p)


# The five workloads the library is measured on, with their sizes.
CONFIGS = {
    "fwd_f16_1x4x128_d64": lambda: prefill(1, 4, 4, 128, 128, 64, "f16", seed=1),
    "fwd_f16_1x8x4096_d64": lambda: prefill(1, 8, 8, 4096, 4096, 64, "f16", seed=2),
    "causal_gqa_bf16_2x32x8192_kv8_d128": lambda: prefill(2, 32, 8, 8192, 8192, 128, "bf16", seed=3, causal=True, with_grad=True),
    "decode_bf16_b64_hq32_kv8_d128": lambda: decode(64, 32, 8, 128, "bf16", seed=4),
    "fwd_fp8_4x16x8192_d128": lambda: fp8_prefill(4, 16, 16, 8192, 8192, 128, seed=5),
}

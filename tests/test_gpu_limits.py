"""GPU parity at the library's size limits: S_q = S_k = 2^20 (the longest sequence the
forward and the decode accept) and B * H_q = 2^16 (the most (batch, head) pairs), on
rows, heads or batches the oracle computes one by one."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import dense
from gpu_common import TOL_OUT, assert_close_lse, assert_close_out, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

S_MAX = 1 << 20
BH_MAX = 1 << 16


def _fwd(w, rows=None, heads=None):
    import exact_tiled_attention_amd as eta
    t, p = w.tensors, w.params
    q, k, v = (to_dev(t[n]) for n in ("q", "k", "v"))
    say(f"[limits fwd] {w.name} causal={p['causal']}")
    o, lse = eta.attn_fwd(q, k, v, scale=p["scale"], causal=p["causal"])
    torch.cuda.synchronize()
    oo, ll = o.cpu(), lse.cpu()
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    O, L = dense.forward(t["q"], t["k"], t["v"], p["scale"], p["causal"], rows=rows, heads=heads)
    if rows is not None:
        oo, ll = oo[:, :, rows], ll[:, :, rows]
    if heads is not None:
        sel = tuple(np.array(heads).T)
        oo, ll, O, L = oo[sel], ll[sel], O[sel], L[sel]
    e1 = assert_close_out(oo, O, TOL_OUT[t["q"].dtype], w.name)
    e2 = assert_close_lse(ll, L, w.name)
    say(f"    max|dO|={e1:.2e} max|dLSE|={e2:.2e}")


def test_fwd_longest_sequence_f16_d64():
    need_gpu()
    w = attn_inputs.prefill(1, 1, 1, S_MAX, S_MAX, 64, "f16", seed=900)
    _fwd(w, rows=np.array([0, 1, 77_777, 524_287, 524_288, S_MAX - 2, S_MAX - 1]))


def test_fwd_longest_sequence_causal_gqa_bf16_d128():
    need_gpu()
    # rows at the start (few visible keys), across tile edges and at the end (all keys)
    w = attn_inputs.prefill(1, 2, 1, S_MAX, S_MAX, 128, "bf16", seed=901, causal=True)
    _fwd(w, rows=np.array([0, 1, 255, 256, 300_001, S_MAX - 257, S_MAX - 1]))


def test_fwd_most_batch_heads():
    need_gpu()
    B, Hq, Hkv = 4, BH_MAX // 4, BH_MAX // 16
    w = attn_inputs.prefill(B, Hq, Hkv, 70, 45, 64, "bf16", seed=902)
    heads = [(0, 0), (0, 1), (1, 5000), (2, 8191), (3, Hq - 4), (3, Hq - 1)]
    _fwd(w, heads=heads)


def test_decode_longest_cache():
    need_gpu()
    import exact_tiled_attention_amd as eta
    lens = [S_MAX, 1, S_MAX - 1000]
    w = attn_inputs.decode(3, 8, 1, 128, "bf16", seed=903, chunk=256, lengths=lens)
    t, p = w.tensors, w.params
    assert p["Smax"] == S_MAX
    q, kc, vc = (to_dev(t[n]) for n in ("q", "k", "v"))
    say(f"[limits decode] {w.name} lens={lens}")
    o, lse = eta.attn_decode_splitkv(q, kc, vc, to_dev(t["seqlens"]), scale=p["scale"])
    torch.cuda.synchronize()
    O, L = dense.decode(t["q"], t["k"], t["v"], t["seqlens"], p["scale"])
    e1 = assert_close_out(o.cpu(), O, TOL_OUT[t["q"].dtype], w.name)
    e2 = assert_close_lse(lse.cpu(), L, w.name)
    say(f"    max|dO|={e1:.2e} max|dLSE|={e2:.2e}")


def test_sizes_past_the_limits_are_rejected():
    need_gpu()
    import exact_tiled_attention_amd as eta
    q = torch.zeros((1, 1, S_MAX + 1, 64), dtype=torch.float16, device="cuda")
    k = torch.zeros((1, 1, 8, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(eta.AttnError):
        eta.attn_fwd(q, k, k)
    q = torch.zeros((1, BH_MAX + 1, 8, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(eta.AttnError):
        eta.attn_fwd(q, k.expand(1, BH_MAX + 1, 8, 64).contiguous(), k.expand(1, BH_MAX + 1, 8, 64).contiguous())

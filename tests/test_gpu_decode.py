"""GPU parity of attn_decode_splitkv against the float64 oracle."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import dense
from gpu_common import TOL_OUT, assert_close_lse, assert_close_out, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _run(w, chunk, batches=None):
    import exact_tiled_attention_amd as eta
    t, p = w.tensors, w.params
    q, kc, vc = (to_dev(t[n]) for n in ("q", "k", "v"))
    lens = to_dev(t["seqlens"])
    say(f"[decode] {w.name} chunk={chunk} lens={t['seqlens'].tolist()[:8]}")
    o, lse = eta.attn_decode_splitkv(q, kc, vc, lens, scale=p["scale"], chunk=chunk)
    torch.cuda.synchronize()
    O, L = dense.decode(t["q"], t["k"], t["v"], t["seqlens"], p["scale"], batches=batches)
    oo, ll = o.cpu(), lse.cpu()
    if batches is not None:
        oo, ll, O, L = oo[batches], ll[batches], O[batches], L[batches]
    e1 = assert_close_out(oo, O, TOL_OUT[t["q"].dtype], w.name)
    e2 = assert_close_lse(ll, L, w.name)
    say(f"    max|dO|={e1:.2e} max|dLSE|={e2:.2e}")
    return o, lse


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (6, 1), (16, 2)])
@pytest.mark.parametrize("chunk", [64, 256])
def test_decode_small_elementwise(dtype, d, Hq, Hkv, chunk):
    need_gpu()
    lens = [1, 63, 64, 65, 256, 257, 700, 0]
    w = attn_inputs.decode(len(lens), Hq, Hkv, d, dtype, seed=40 + d + Hq, chunk=chunk, lengths=lens)
    _run(w, chunk)


@pytest.mark.parametrize("chunk", [512, 768, 1536])
def test_decode_long_chunk_and_uneven_lengths(chunk):
    # several 64-key passes per wave; a cache length (5120) that is not a multiple of
    # the chunk leaves a short last chunk
    need_gpu()
    lens = [5000, 1, 1300, 4097]
    w = attn_inputs.decode(len(lens), 8, 2, 128, "bf16", seed=77, chunk=256, lengths=lens)
    _run(w, chunk)


@pytest.mark.parametrize("chunk", [256, None])
def test_decode_b64_full_size_sampled(chunk):
    """The full-size workload in both benchmarked launches: 256-token chunks as the
    workload is written, and the library's own pick (1536 keys)."""
    need_gpu()
    w = attn_inputs.CONFIGS["decode_bf16_b64_hq32_kv8_d128"]()
    lens = w.tensors["seqlens"].numpy()
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 17, 42, 63})
    import exact_tiled_attention_amd as eta
    p = w.params
    if chunk is None:
        chunk = eta.decode_pick_chunk(p["B"], p["Hq"], p["Smax"])
        assert chunk == 1536
    _run(w, chunk, batches=pick)


def test_decode_bitwise_repeatable():
    need_gpu()
    import exact_tiled_attention_amd as eta
    w = attn_inputs.decode(8, 32, 8, 128, "bf16", seed=5, lo=100, hi=3000)
    t, p = w.tensors, w.params
    q, kc, vc, lens = (to_dev(t[n]) for n in ("q", "k", "v", "seqlens"))
    o1, l1 = eta.attn_decode_splitkv(q, kc, vc, lens)
    o2, l2 = eta.attn_decode_splitkv(q, kc, vc, lens)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)

"""attn_decode_splitkv_noalloc (partial states in the library's per-GPU device scratch)
against attn_decode_splitkv with a caller workspace, through the C ABI: two calls in a
row, the second with a smaller input, and a size past the scratch rejected."""
import pytest
import torch

import attn_inputs
from oracle import dense
from gpu_common import TOL_OUT, assert_close_lse, assert_close_out, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _both(w, chunk):
    import exact_tiled_attention_amd as eta
    t, p = w.tensors, w.params
    q, kc, vc, lens = (to_dev(t[n]) for n in ("q", "k", "v", "seqlens"))
    say(f"[noalloc] {w.name} chunk={chunk}")
    o1, l1 = eta.attn_decode_splitkv_noalloc(q, kc, vc, lens, scale=p["scale"], chunk=chunk)
    o2, l2 = eta.attn_decode_splitkv(q, kc, vc, lens, scale=p["scale"], chunk=chunk)
    torch.cuda.synchronize()
    # same kernels, same chunking: identical results; and both within the oracle's bar
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    O, L = dense.decode(t["q"], t["k"], t["v"], t["seqlens"], p["scale"])
    assert_close_out(o1.cpu(), O, TOL_OUT[t["q"].dtype], w.name)
    assert_close_lse(l1.cpu(), L, w.name)


def test_noalloc_decode_matches_workspace_decode_twice():
    need_gpu()
    big = attn_inputs.decode(16, 32, 8, 128, "bf16", seed=501, lo=1000, hi=9000)
    small = attn_inputs.decode(3, 8, 2, 64, "f16", seed=502, lengths=[1, 700, 65])
    _both(big, 256)
    _both(small, 64)          # the scratch still holds the first call's partials


def test_noalloc_decode_rejects_sizes_past_the_scratch():
    need_gpu()
    import exact_tiled_attention_amd as eta
    B, Hq, Smax, d = 64, 32, 32768, 128
    assert eta.decode_workspace_size(B, Hq, Smax, d, 256) > eta.DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, Hq, 1, d, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(B, 8, Smax, d, dtype=torch.bfloat16, device="cuda")
    lens = torch.full((B,), Smax, dtype=torch.int32, device="cuda")
    with pytest.raises(eta.AttnError) as e:
        eta.attn_decode_splitkv_noalloc(q, kc, kc, lens, chunk=256)
    assert e.value.status == -6

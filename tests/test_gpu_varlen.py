"""GPU parity of attn_fwd_varlen (packed token-major sequences) against the float64
oracle, elementwise, plus bitwise agreement with attn_fwd on equal lengths."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import dense
from gpu_common import TOL_OUT, assert_close_lse, assert_close_out, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

LENGTH_SETS = {
    "printed_fixture": ([512, 257, 0], [512, 193, 256]),   # FA2 page, section 0x04B
    "empty_keys_and_tails": ([1, 70, 300, 129], [0, 64, 301, 1]),
    "mixed": ([900, 33, 1500, 256, 7, 1100], [1000, 500, 1500, 255, 300, 1100]),
}


def _run(w):
    import exact_tiled_attention_amd as eta
    t, p = w.tensors, w.params
    q, k, v, cq, ck = (to_dev(t[n]) for n in ("q", "k", "v", "cu_q", "cu_k"))
    o, lse = eta.attn_fwd_varlen(q, k, v, cq, ck, p["max_seqlen_q"], p["max_seqlen_k"], scale=p["scale"],
                                 causal=p["causal"])
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lengths", list(LENGTH_SETS))
def test_varlen_elementwise(dtype, d, causal, lengths):
    need_gpu()
    sq, sk = LENGTH_SETS[lengths]
    Hq, Hkv = (8, 2) if lengths != "mixed" else (8, 8)
    w = attn_inputs.varlen_prefill(sq, sk, Hq, Hkv, d, dtype, seed=500 + d + len(sq), causal=causal)
    say(f"[varlen] {w.name} {lengths} causal={causal}")
    o, lse = _run(w)
    t, p = w.tensors, w.params
    O, L = dense.forward_varlen(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], p["scale"], causal)
    e1 = assert_close_out(o.cpu(), O, TOL_OUT[t["q"].dtype], w.name)
    e2 = assert_close_lse(lse.cpu(), L, w.name)
    say(f"    max|dO|={e1:.2e} max|dLSE|={e2:.2e}")


@pytest.mark.parametrize("d", [64, 128])
def test_varlen_equal_lengths_bitwise_equal_to_padded(d):
    need_gpu()
    import exact_tiled_attention_amd as eta
    B, H, S = 3, 4, 333
    w = attn_inputs.varlen_prefill([S] * B, [S] * B, H, H, d, "bf16", seed=77, causal=True)
    o, lse = _run(w)
    t = w.tensors
    qp, kp, vp = (to_dev(t[n]).reshape(B, S, H, d).permute(0, 2, 1, 3).contiguous() for n in ("q", "k", "v"))
    o2, l2 = eta.attn_fwd(qp, kp, vp, scale=w.params["scale"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2.permute(0, 2, 1, 3).reshape(B * S, H, d))
    assert torch.equal(lse, l2.permute(1, 0, 2).reshape(H, B * S))

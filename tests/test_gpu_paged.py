"""GPU parity of attn_decode_paged (split-KV decode over a paged K/V pool) against the
float64 oracle, and bitwise agreement with attn_decode_splitkv on the gathered cache."""
import numpy as np
import pytest
import torch

import attn_inputs
from oracle import dense
from gpu_common import TOL_OUT, assert_close_lse, assert_close_out, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _paged(w, chunk, block_table=None):
    import exact_tiled_attention_amd as eta
    t, p = w.tensors, w.params
    bt = t["block_table"] if block_table is None else block_table
    say(f"[paged] {w.name} chunk={chunk} lens={t['seqlens'].tolist()[:8]}")
    o, lse = eta.attn_decode_paged(to_dev(t["q"]), to_dev(t["k_pages"]), to_dev(t["v_pages"]), to_dev(bt),
                                   to_dev(t["seqlens"]), scale=p["scale"], chunk=chunk)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check(w, o, lse, batches=None, block_table=None):
    t, p = w.tensors, w.params
    bt = t["block_table"] if block_table is None else block_table
    q, lens = t["q"], t["seqlens"]
    if batches is not None:
        q, bt, lens, o, lse = q[batches], bt[batches], lens[batches], o[batches], lse[batches]
    O, L = dense.decode_paged(q, t["k_pages"], t["v_pages"], bt, lens, p["scale"])
    e1 = assert_close_out(o, O, TOL_OUT[t["q"].dtype], w.name)
    e2 = assert_close_lse(lse, L, w.name)
    say(f"    max|dO|={e1:.2e} max|dLSE|={e2:.2e}")


def _poison_tails(w):
    """Rows of each sequence's last page past its length (and unused pages) hold NaN:
    they must never be read."""
    t, p = w.tensors, w.params
    P = p["page_size"]
    used = np.zeros(p["num_pages"], dtype=bool)
    for b, n in enumerate(t["seqlens"].tolist()):
        npg = -(-n // P)
        for i in range(npg):
            used[int(t["block_table"][b, i])] = True
        if n % P:
            pg = int(t["block_table"][b, npg - 1])
            t["k_pages"][pg, :, n % P:] = float("nan")
            t["v_pages"][pg, :, n % P:] = float("nan")
    t["k_pages"][torch.from_numpy(~used)] = float("nan")
    t["v_pages"][torch.from_numpy(~used)] = float("nan")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (32, 8)])
@pytest.mark.parametrize("page_size", [64, 128, 256])
def test_paged_elementwise(dtype, d, Hq, Hkv, page_size):
    need_gpu()
    lens = [1, 63, 64, 65, page_size - 1, page_size, page_size + 1, 700, 0, 1500]
    w = attn_inputs.paged_decode(len(lens), Hq, Hkv, d, dtype, seed=60 + d + Hq + page_size,
                                 page_size=page_size, lengths=lens)
    _poison_tails(w)
    o, lse = _paged(w, 256)
    _check(w, o, lse)


@pytest.mark.parametrize("chunk", [64, 512, 1536])
def test_paged_chunks_and_several_passes(chunk):
    need_gpu()
    lens = [5000, 1, 1300, 4097, 128, 2049]
    w = attn_inputs.paged_decode(len(lens), 8, 2, 128, "bf16", seed=91, page_size=64, lengths=lens)
    _poison_tails(w)
    o, lse = _paged(w, chunk)
    _check(w, o, lse)


def test_paged_bitwise_equal_to_contiguous():
    need_gpu()
    import exact_tiled_attention_amd as eta
    lens = [3000, 17, 1024, 2500, 0, 777]
    w = attn_inputs.paged_decode(len(lens), 32, 8, 128, "bf16", seed=92, page_size=128, lengths=lens)
    t, p = w.tensors, w.params
    P, maxp = p["page_size"], p["max_pages"]
    # contiguous cache holding the same logical rows (pages gathered in table order)
    bt = t["block_table"].long()
    kc = t["k_pages"][bt].permute(0, 2, 1, 3, 4).reshape(len(lens), p["Hkv"], maxp * P, p["d"])
    vc = t["v_pages"][bt].permute(0, 2, 1, 3, 4).reshape(len(lens), p["Hkv"], maxp * P, p["d"])
    o1, l1 = _paged(w, 256)
    o2, l2 = eta.attn_decode_splitkv(to_dev(t["q"]), to_dev(kc), to_dev(vc), to_dev(t["seqlens"]),
                                     scale=p["scale"], chunk=256)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2.cpu())
    assert torch.equal(l1, l2.cpu())


def test_paged_out_of_range_entries_are_clamped():
    """Table entries outside the pool read the nearest pool page (never outside it)."""
    need_gpu()
    lens = [300, 200]
    w = attn_inputs.paged_decode(len(lens), 8, 2, 64, "f16", seed=93, page_size=64, lengths=lens)
    bt = w.tensors["block_table"].clone()
    bt[0, 1] = -7
    bt[1, 2] = w.params["num_pages"] + 1000
    o, lse = _paged(w, 256, block_table=bt)
    _check(w, o, lse, block_table=bt.clamp(0, w.params["num_pages"] - 1))


def test_paged_large_sampled():
    need_gpu()
    w = attn_inputs.paged_decode(16, 32, 8, 128, "bf16", seed=94, page_size=128, lo=1024, hi=20000)
    lens = w.tensors["seqlens"].numpy()
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 7, 15})
    o, lse = _paged(w, None)   # the library's chunk choice
    _check(w, o, lse, batches=pick)

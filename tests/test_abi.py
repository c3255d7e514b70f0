"""The C ABI: libattn.so loads without a GPU, exports every function include/attn.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from conftest import golden, ROOT

HEADER = os.path.join(ROOT, "include", "attn.h")


def _lib():
    from exact_tiled_attention_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libattn.so not built (run __graft_entry__.build())")
    return _lib.lib(), _lib


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib, mod = _lib()
    names = _declared()
    assert "attn_fwd" in names and "attn_bwd" in names and "attn_decode_splitkv" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(mod.PROTOTYPES), "binding prototypes and header differ"


def test_status_strings():
    lib, _ = _lib()
    for code in range(0, -9, -1):
        assert lib.attn_status_string(code)
    assert lib.attn_status_string(5) == b"unknown status"


P = ctypes.c_void_p(16)   # a non-NULL placeholder: never dereferenced on rejected calls


def test_fwd_argument_checks():
    lib, _ = _lib()
    f = lib.attn_fwd
    ok = dict(B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=64)
    def call(q=P, k=P, v=P, o=P, dtype=0, scale=0.125, **kw):
        a = dict(ok, **kw)
        return f(q, k, v, o, None, a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"], scale, 0, dtype, None)
    assert call(q=None) == -1 and call(o=None) == -1 and call(k=None) == -1
    assert call(B=0) == -2 and call(Sq=0) == -2 and call(Sk=-1) == -2 and call(Sq=1 << 21) == -2
    assert call(Hq=3) == -3
    assert call(d=96) == -4 and call(d=256) == -4
    assert call(dtype=2) == -5 and call(dtype=3) == -5
    assert call(scale=float("inf")) == -8 and call(scale=float("nan")) == -8


def test_fwd_exp_emulated_and_exp2_soft_checks():
    lib, _ = _lib()
    f = lib.attn_fwd_exp_emulated
    def call(emu, q=P, B=1, d=64):
        return f(q, P, P, P, None, B, 4, 2, 8, 8, d, 0.125, 0, 0, emu, None)
    for emu in (1, 3, 5, 8, -2):
        assert call(emu) == -8
    assert call(2, q=None) == -1 and call(4, B=0) == -2 and call(2, d=96) == -4
    g = lib.attn_exp2_soft
    assert g(P, P, -1, None) == -2 and g(P, P, (1 << 31) + 1, None) == -2
    assert g(None, P, 5, None) == -1 and g(P, None, 5, None) == -1
    assert g(None, None, 0, None) == 0          # nothing to compute, no launch


def test_fwd_varlen_argument_checks():
    lib, _ = _lib()
    f = lib.attn_fwd_varlen
    def call(q=P, k=P, o=P, cuq=P, cuk=P, dtype=1, scale=0.125, **kw):
        a = dict(B=2, Hq=4, Hkv=2, mq=16, mk=16, tq=20, tk=24, d=128)
        a.update(kw)
        return f(q, k, k, o, None, cuq, cuk, a["B"], a["Hq"], a["Hkv"], a["mq"], a["mk"], a["tq"], a["tk"],
                 a["d"], scale, 1, dtype, None)
    assert call(cuq=None) == -1 and call(cuk=None) == -1 and call(q=None) == -1 and call(k=None) == -1
    assert call(B=0) == -2 and call(mq=-1) == -2 and call(tk=-1) == -2 and call(mq=1 << 21) == -2
    assert call(Hq=64, mq=1 << 20) == -2                       # one sequence spans >= 2 GiB
    assert call(Hq=3) == -3 and call(d=80) == -4 and call(dtype=2) == -5
    assert call(scale=float("nan")) == -8
    # nothing to compute: no launch, no dereference of the placeholders
    assert call(tq=0, q=None, o=None) == 0 and call(mq=0) == 0


def test_bwd_and_workspace_checks():
    lib, _ = _lib()
    ws = lib.attn_bwd_workspace_size(1, 4, 2, 8, 8, 64)
    assert ws >= 1 * 4 * 8 * 64 * 4 + 1 * 4 * 8 * 4
    assert lib.attn_bwd_workspace_size(1, 3, 2, 8, 8, 64) == 0
    def call(ws_ptr=P, ws_bytes=ws, grad=2, **kw):
        a = dict(B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=64, dtype=1)
        a.update(kw)
        return lib.attn_bwd(P, P, P, P, P, P, P, P, P, a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"],
                            0.125, 1, a["dtype"], grad, ws_ptr, ws_bytes, None)
    assert call(ws_ptr=None) == -6 and call(ws_bytes=ws - 1) == -6
    assert call(grad=3) == -5 and call(dtype=2) == -5
    assert call(Sk=0) == -2 and call(Hkv=3) == -3 and call(d=32) == -4
    assert lib.attn_bwd(None, P, P, P, P, P, P, P, P, 1, 4, 2, 8, 8, 64, 0.125, 0, 1, 2, P, ws, None) == -1
    # the atomic form takes the same arguments and workspace
    assert lib.attn_bwd_atomic(P, P, P, P, P, P, P, P, P, 1, 4, 2, 8, 8, 64, 0.125, 1, 1, 2, None, ws, None) == -6
    assert lib.attn_bwd_atomic(P, P, P, P, P, P, P, P, P, 1, 4, 3, 8, 8, 64, 0.125, 1, 1, 2, P, ws, None) == -3
    # enough for either form: at 1024 keys and more attn_bwd runs the deterministic form
    for sk in (8, 1024):
        assert lib.attn_bwd_workspace_size(1, 4, 2, 8, sk, 64) >= lib.attn_bwd_deterministic_workspace_size(
            1, 4, 2, 8, sk, 64, 1)


def test_decode_and_fp8_checks():
    lib, _ = _lib()
    ws = lib.attn_decode_workspace_size(2, 8, 512, 128, 256)
    assert ws >= 2 * 8 * 2 * (128 + 2) * 4
    assert lib.attn_decode_workspace_size(2, 8, 512, 128, 100) == 0
    def dec(chunk=256, ws_bytes=ws, **kw):
        a = dict(B=2, Hq=8, Hkv=2, Smax=512, d=128)
        a.update(kw)
        return lib.attn_decode_splitkv(P, P, P, P, P, None, a["B"], a["Hq"], a["Hkv"], a["Smax"], a["d"],
                                       0.088, chunk, 1, P, ws_bytes, None)
    assert dec(chunk=100) == -8 and dec(chunk=0) == -8 and dec(ws_bytes=ws - 1) == -6
    assert dec(Hkv=3) == -3 and dec(d=80) == -4 and dec(Smax=0) == -2
    assert lib.attn_fp8_kv_tile() in (32, 64, 128)
    def f8(d=128, causal=0, odt=1, **kw):
        a = dict(B=1, Hq=2, Hkv=2, Sq=8, Sk=8)
        a.update(kw)
        return lib.attn_fwd_fp8(P, P, P, P, P, P, P, None, a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], d,
                                0.088, causal, odt, None)
    assert f8(d=32) == -4 and f8(odt=0) == -5 and f8(Sk=0) == -2 and f8(Hkv=3) == -3


def test_decode_pick_chunk():
    # pure host arithmetic: the largest of 1536, 768 keys that keeps >= 16384 (query
    # head, chunk) pairs at full length, else 256
    lib, _ = _lib()
    assert lib.attn_decode_pick_chunk(64, 32, 32768) == 1536     # 2048 rows x 22 chunks
    assert lib.attn_decode_pick_chunk(8, 32, 32768) == 256       # 256 x 43 < 16384 at 768
    assert lib.attn_decode_pick_chunk(16, 32, 32768) == 768      # 512 x 22 < 16384 <= 512 x 43
    assert lib.attn_decode_pick_chunk(1, 1, 100) == 256
    assert lib.attn_decode_pick_chunk(0, 32, 32768) == 256 and lib.attn_decode_pick_chunk(4, 8, -1) == 256
    for args in ((64, 32, 32768), (16, 32, 32768), (3, 5, 7000)):
        c = lib.attn_decode_pick_chunk(*args)
        assert c % 64 == 0 and lib.attn_decode_workspace_size(args[0], args[1], args[2], 128, c) > 0


def test_decode_paged_argument_checks():
    lib, _ = _lib()
    ws = lib.attn_decode_workspace_size(2, 8, 4 * 128, 128, 256)
    def call(q=P, bt=P, lens=P, P_=128, maxp=4, npages=9, chunk=256, ws_bytes=ws, **kw):
        a = dict(B=2, Hq=8, Hkv=2, d=128, dtype=1)
        a.update(kw)
        return lib.attn_decode_paged(q, P, P, bt, lens, P, None, a["B"], a["Hq"], a["Hkv"], npages, P_, maxp,
                                     a["d"], 0.088, chunk, a["dtype"], P, ws_bytes, None)
    assert call(q=None) == -1 and call(bt=None) == -1 and call(lens=None) == -1
    assert call(P_=32) == -8 and call(P_=96) == -8 and call(P_=8192) == -8     # power of two, 64 .. 4096
    assert call(npages=0) == -2 and call(maxp=0) == -2 and call(maxp=1 << 14, P_=128) == -2
    assert call(Hkv=3) == -3 and call(d=80) == -4 and call(dtype=2) == -5
    assert call(chunk=100) == -8 and call(ws_bytes=ws - 1) == -6
    # the workspace is sized for max_pages * P keys
    assert call(maxp=8, ws_bytes=ws) == -6


def test_tile_plan_matches_printed_causal_ledger():
    """The kernels' tile iterator (exported host function) reproduces the printed
    causal tile counts: visits and masked tiles per query tile."""
    lib, _ = _lib()
    n, fm = ctypes.c_int(), ctypes.c_int()
    for c in golden("causal_tiles.json")["cases"]:
        Sq, Sk, Br, Bc = c["Sq"], c["Sk"], c["Br"], c["Bc"]
        visits, full = [], 0
        for q0 in range(0, Sq, Br):
            assert lib.attn_tile_plan(q0, min(Sq, q0 + Br), Sq, Sk, Bc, 1, ctypes.byref(n), ctypes.byref(fm)) == 0
            visits.append(n.value)
            full += fm.value
        if "visited" in c:
            assert sum(visits) == c["visited"]
        if "visits_per_query_tile_first" in c:
            assert visits[0] == c["visits_per_query_tile_first"] and visits[-1] == c["visits_per_query_tile_last"]
        # tiles before first_masked are exactly the fully visible ones that need no tail mask
        if Sk % Bc == 0:
            assert full == c["full"]
    assert lib.attn_tile_plan(0, 0, 8, 8, 64, 1, ctypes.byref(n), ctypes.byref(fm)) == -8
    assert lib.attn_tile_plan(0, 8, 8, 8, 64, 1, None, ctypes.byref(fm)) == -1


def test_bwd_deterministic_argument_checks():
    lib, _ = _lib()
    ws1 = lib.attn_bwd_deterministic_workspace_size(1, 4, 2, 8, 8, 64, 1)
    ws4 = lib.attn_bwd_deterministic_workspace_size(1, 4, 2, 8, 8, 64, 4)
    assert ws1 >= 1 * 4 * 8 * 4 and ws4 >= ws1 + 4 * 1 * 4 * 8 * 64 * 4
    # room for the fp16 copies of q, dO (4 x 8 rows) and k, v (2 x 8 rows) of bf16 operands
    assert ws1 >= 1 * 4 * 8 * 4 + 2 * (4 * 8 * 64 * 2) + 2 * (2 * 8 * 64 * 2)
    assert lib.attn_bwd_deterministic_workspace_size(1, 4, 2, 8, 8, 64, 3) == 0
    def call(splits=1, ws_bytes=ws1, **kw):
        a = dict(B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=64)
        a.update(kw)
        return lib.attn_bwd_deterministic(P, P, P, P, P, P, P, P, P, a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"],
                                          a["d"], 0.125, 1, 1, 2, splits, P, ws_bytes, None)
    assert call(splits=3) == -8 and call(splits=32) == -8 and call(splits=0) == -8
    assert call(splits=4, ws_bytes=ws4 - 1) == -6 and call(ws_bytes=ws1 - 1) == -6
    assert call(Sk=0) == -2 and call(Hkv=3) == -3 and call(d=32) == -4


def test_dropout_argument_checks():
    lib, _ = _lib()
    f = lib.attn_fwd_dropout
    def fwd(p=0.1, **kw):
        a = dict(B=1, Hq=2, Hkv=2, Sq=8, Sk=8, d=64)
        a.update(kw)
        return f(P, P, P, P, None, a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"], 0.125, 0, p, 1, 0, 1, None)
    assert fwd(p=1.0) == -8 and fwd(p=-0.1) == -8 and fwd(p=float("nan")) == -8 and fwd(d=80) == -4
    ws = lib.attn_bwd_workspace_size(1, 2, 2, 8, 8, 64)
    def bwd(p=0.1, det=0, splits=1, ws_bytes=ws):
        return lib.attn_bwd_dropout(P, P, P, P, P, P, P, P, P, 1, 2, 2, 8, 8, 64, 0.125, 0, p, 1, 0, 1, 2, det,
                                    splits, P, ws_bytes, None)
    assert bwd(p=1.0) == -8 and bwd(ws_bytes=ws - 1) == -6 and bwd(det=1, splits=3) == -8


def test_missing_library_raises_instead_of_falling_back(monkeypatch, tmp_path):
    from exact_tiled_attention_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libattn.so"))
    with pytest.raises(_lib.LibraryMissing):
        _lib.lib()


def test_fp8_and_decode_bindings_check_types_first():
    """The Python bindings reject a wrong dtype (TypeError) and then a wrong shape,
    layout or device (ValueError) before the library is called."""
    import torch
    import exact_tiled_attention_amd as eta
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32)
    q8, k8 = u8(1, 2, 8, 128), u8(1, 2, 8, 128)
    sc = f32(1, 2, 1)
    with pytest.raises(TypeError):
        eta.attn_fwd_fp8(q8.float(), k8, k8, sc, sc, sc)
    with pytest.raises(TypeError):
        eta.attn_fwd_fp8(q8, k8, k8, sc.double(), sc, sc)
    with pytest.raises(TypeError):
        eta.attn_fwd_fp8(q8, k8, k8, sc, sc, sc, o=torch.zeros(1, 2, 8, 128, dtype=torch.float16))
    with pytest.raises(ValueError):                       # CPU tensors: not on a GPU
        eta.attn_fwd_fp8(q8, k8, k8, sc, sc, sc)
    q = torch.zeros(2, 8, 1, 128, dtype=torch.bfloat16)
    kc = torch.zeros(2, 2, 512, 128, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        eta.attn_decode_splitkv(q, kc, kc, torch.zeros(2, dtype=torch.int64))
    with pytest.raises(TypeError):
        eta.attn_decode_splitkv(q, kc.half(), kc, torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError):
        eta.attn_decode_splitkv(q, kc, kc, torch.zeros(2, dtype=torch.int32))


def test_decode_noalloc_checks_run_before_any_hip_call():
    lib, _ = _lib()
    def call(chunk=256, **kw):
        a = dict(B=2, Hq=8, Hkv=2, Smax=512, d=128)
        a.update(kw)
        return lib.attn_decode_splitkv_noalloc(P, P, P, P, P, None, a["B"], a["Hq"], a["Hkv"], a["Smax"], a["d"],
                                               0.088, chunk, 1, None)
    assert call(chunk=100) == -8 and call(Hkv=3) == -3 and call(d=80) == -4 and call(Smax=0) == -2
    # partial states past the 64 MiB device scratch: rejected on the host
    assert lib.attn_decode_workspace_size(64, 32, 32768, 128, 256) > (64 << 20)
    assert call(B=64, Hq=32, Hkv=8, Smax=32768, chunk=256) == -6
    assert lib.attn_decode_splitkv_noalloc(None, P, P, P, P, None, 2, 8, 2, 512, 128, 0.088, 256, 1, None) == -1


def test_bwd_fp8_argument_checks():
    lib, _ = _lib()
    ws = lib.attn_bwd_workspace_size(1, 4, 2, 64, 64, 128)
    def call(d=128, grad=2, ws_bytes=ws, **kw):
        a = dict(B=1, Hq=4, Hkv=2, Sq=64, Sk=64)
        a.update(kw)
        return lib.attn_bwd_fp8(P, P, P, P, P, P, P, P, P, P, P, P, a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], d,
                                0.088, 1, grad, P, ws_bytes, None)
    assert call(d=96) == -4 and call(grad=3) == -5 and call(Hkv=3) == -3 and call(Sk=0) == -2
    assert call(ws_bytes=ws - 1) == -6
    assert lib.attn_bwd_fp8(None, P, P, P, P, P, P, P, P, P, P, P, 1, 4, 2, 64, 64, 128, 0.088, 1, 2, P, ws,
                            None) == -1

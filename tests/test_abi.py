"""CPU tests of the C-ABI boundary: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host before any launch.
No compute call is made here (there is no GPU in this suite)."""
import ctypes
import os
import re

import pytest

import linear_hybrid_attention_amd as ttr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = 1 << 20  # a 16-byte-aligned fake device address; never dereferenced on these paths
OK, NULL, SHAPE, DTYPE, UNSUP, WS, ALIGN, HIP, ALIAS = range(9)


@pytest.fixture(scope="module")
def lib():
    return ttr.load_library()


def test_header_declarations_are_exported(lib):
    names = ttr.exported_symbols()
    assert {"ttr_feature_map", "ttr_kv_reduce", "ttr_apply", "ttr_landmark_attn", "ttr_blend",
            "ttr_causal_scan", "ttr_hybrid_forward", "ttr_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_dynamic_symbol_table_matches_header():
    # every extern "C" function in the header is a dynamic symbol of the .so
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", ttr.library_path()], capture_output=True, text=True).stdout
    syms = set(re.findall(r"\bT (ttr_\w+)", out))
    assert set(ttr.exported_symbols()) <= syms


def test_status_strings(lib):
    for st in range(9):
        s = ttr.status_string(st)
        assert isinstance(s, str) and s
    assert ttr.status_string(0) == "ok"
    assert lib.ttr_last_hip_error() == 0
    assert ttr.version().startswith("ttr ")


def D(B=1, H=2, N=256, Dm=64, F=256, dt=0):
    return ttr.Dims(B, H, N, Dm, F, dt)


def hyb(lib, d, Q=P, K=2 * P, V=3 * P, W=4 * P, b=None, g=5 * P, L=16, causal=0, out=6 * P, ws=7 * P,
        wsb=1 << 30):
    return lib.ttr_hybrid_forward(d, Q, K, V, W, b, g, 1e-6, L, causal, out, ws, wsb, None)


def test_hybrid_forward_validation(lib):
    big = 1 << 40
    kw = dict(Q=big, K=2 * big, V=3 * big, W=4 * big, g=5 * big, out=6 * big, ws=7 * big)
    assert hyb(lib, D(dt=5), **kw) == DTYPE
    assert hyb(lib, D(B=0), **kw) == SHAPE
    assert hyb(lib, D(N=0), **kw) == SHAPE
    assert hyb(lib, D(Dm=96), **kw) == SHAPE
    assert hyb(lib, D(F=200), **kw) == SHAPE          # feature_dim must be a multiple of 256
    assert hyb(lib, D(F=384), **kw) == SHAPE          # not a multiple of 256
    assert hyb(lib, D(F=512), **kw) == UNSUP          # fp32 IO: F == 256 only
    assert hyb(lib, D(F=768, dt=1), wsb=16, **kw) == WS  # bf16: 256, 512, 768 and 1024 are implemented
    assert hyb(lib, D(F=512, dt=1), wsb=16, **kw) == WS  # bf16 F = 512: valid, reaches the workspace check
    assert hyb(lib, D(F=1024, dt=1), wsb=16, **kw) == WS
    assert hyb(lib, D(F=1280, dt=1), **kw) == UNSUP
    assert hyb(lib, D(Dm=128, F=256, dt=0), wsb=16, **kw) == WS  # fp32 IO with D = 128: valid
    kw2 = dict(kw)
    kw2["W"] = None
    assert hyb(lib, D(Dm=128, F=128, dt=0), causal=128, L=0, **kw2) == UNSUP  # fp32, D = 128: chunk 64 only
    assert hyb(lib, D(Dm=128, F=128, dt=0), causal=64, L=0, wsb=16, **kw2) == WS
    assert hyb(lib, D(), L=257, **kw) == SHAPE
    assert hyb(lib, D(), L=-1, **kw) == SHAPE
    kw2 = dict(kw)
    kw2["Q"] = None
    assert hyb(lib, D(), **kw2) == NULL
    kw2 = dict(kw)
    kw2["g"] = None
    assert hyb(lib, D(), **kw2) == NULL
    assert hyb(lib, D(), L=0, **kw2) != NULL          # g unused without landmarks
    kw2 = dict(kw)
    kw2["V"] = 3 * big + 4
    assert hyb(lib, D(), **kw2) == ALIGN
    kw2 = dict(kw)
    kw2["ws"] = None
    assert hyb(lib, D(), **kw2) == WS
    assert hyb(lib, D(), wsb=16, **kw) == WS
    kw2 = dict(kw)
    kw2["out"] = kw["Q"]
    assert hyb(lib, D(), **kw2) == ALIAS
    kw2 = dict(kw)
    kw2["out"] = kw["Q"] + 64                          # partial overlap
    assert hyb(lib, D(), **kw2) == ALIAS
    # identity map: F must equal D
    kw2 = dict(kw)
    kw2["W"] = None
    assert hyb(lib, D(F=256), **kw2) == SHAPE
    # causal: landmarks and projections are not defined for it
    assert hyb(lib, D(F=64, dt=1), causal=1, L=16, **kw2) == UNSUP
    assert hyb(lib, D(F=256, dt=1), causal=1, L=0, **kw) == UNSUP


def test_feature_map_kind_validation(lib):
    big = 1 << 40
    kw = dict(Q=big, K=2 * big, V=3 * big, W=4 * big, g=5 * big, out=6 * big, ws=7 * big)
    nw = dict(kw)
    nw["W"] = None

    def Dm(fmap, F=256, dt=0):
        d = D(F=F, dt=dt)
        d.fmap = fmap
        return d

    assert hyb(lib, Dm(3), **kw) == SHAPE
    assert hyb(lib, Dm(-1), **kw) == SHAPE
    # relu / softmax are the NNT layer's maps on projected features: no W, no landmarks
    assert hyb(lib, Dm(1), **kw) == UNSUP
    assert hyb(lib, Dm(2, F=64), L=16, **nw) == UNSUP
    assert hyb(lib, Dm(2, F=64), L=0, wsb=16, **nw) == WS      # otherwise valid: reaches the workspace check
    assert lib.ttr_feature_map(Dm(1), big, 2 * big, None, 3 * big, None) == UNSUP
    assert lib.ttr_workspace_bytes(Dm(2, F=64, dt=1), 0, 0, 0) > 0
    assert lib.ttr_workspace_bytes(Dm(2, F=256, dt=1), 0, 0, 0) == 0


def test_nnt_layer_validation(lib):
    big = 1 << 40

    def LD(B=2, N=100, E=512, H=8, dt=1, fmap=0):
        return ttr.LayerDims(B, N, E, H, dt, fmap)

    def layer(d, x=big, Wq=2 * big, Wk=3 * big, Wv=4 * big, Wo=5 * big, bq=None, out=6 * big, ws=7 * big,
              wsb=1 << 34, causal=0):
        return lib.ttr_nnt_layer_forward(d, x, Wq, bq, Wk, None, Wv, None, Wo, None, 1e-6, causal, out, ws, wsb,
                                         None)

    assert layer(LD(dt=5)) == DTYPE
    assert layer(LD(fmap=3)) == SHAPE
    assert layer(LD(B=0)) == SHAPE
    assert layer(LD(E=512, H=3)) == SHAPE          # embed_dim must divide by num_heads
    assert layer(LD(E=192, H=3)) == UNSUP          # E not a multiple of 128
    assert layer(LD(E=512, H=16)) == UNSUP         # D = 32
    assert layer(LD(E=512, H=4, dt=0), wsb=16) == WS  # fp32 with D = 128: valid, reaches the workspace check
    assert layer(LD(E=512, H=4, dt=0), causal=1, wsb=16) == WS  # fp32 causal with D = 128: chunk 64
    assert layer(LD(), x=None) == NULL
    assert layer(LD(), Wo=None) == NULL
    assert layer(LD(), Wq=big + 8) == ALIGN
    assert layer(LD(), bq=big + 4) == ALIGN
    assert layer(LD(), wsb=16) == WS
    assert layer(LD(), ws=None) == WS
    assert layer(LD(), out=big + 64) == ALIAS        # out overlaps x
    assert lib.ttr_nnt_layer_workspace_bytes(LD(), 0) > lib.ttr_nnt_layer_workspace_bytes(LD(N=10), 0)
    assert lib.ttr_nnt_layer_workspace_bytes(LD(H=3), 0) == 0
    # the layer's workspace holds the transposed weights, Q, K, V and the attention output
    ws = lib.ttr_nnt_layer_workspace_bytes(LD(B=1, N=256, E=512, H=8), 1)
    assert ws >= 4 * 512 * 512 * 2 + 4 * 256 * 512 * 2


def test_causal_scan_validation(lib):
    big = 1 << 40
    d = D(B=8, H=8, N=32768, Dm=64, F=64, dt=1)
    need = lib.ttr_workspace_bytes(d, 0, 1, 256)
    assert need > 0

    def cs(dd, chunk=256, W=None, ws=7 * big, wsb=need):
        return lib.ttr_causal_scan(dd, big, 2 * big, 3 * big, W, None, 1e-6, chunk, 6 * big, ws, wsb, None)

    assert cs(d, chunk=100) == SHAPE
    assert cs(d, chunk=512) == SHAPE
    assert cs(d, W=4 * big) == UNSUP
    assert cs(D(Dm=128, F=128, dt=1), chunk=256) == UNSUP   # LDS budget of the D=128 chunk walk
    assert cs(D(Dm=64, F=64, dt=0), chunk=256) == UNSUP     # fp32 walks chunks of at most 128
    assert cs(d, wsb=need - 1) == WS
    assert cs(d, ws=None) == WS


def test_staged_validation(lib):
    big = 1 << 40
    d = D()
    assert lib.ttr_feature_map(d, None, big, None, 2 * big, None) == NULL
    assert lib.ttr_feature_map(d, big, big + 8, None, 2 * big, None) == ALIGN
    assert lib.ttr_feature_map(d, big, 2 * big, None, big, None) == ALIAS
    assert lib.ttr_landmark_attn(d, big, 2 * big, 3 * big, 0, 4 * big, None) == SHAPE
    assert lib.ttr_landmark_attn(d, big, 2 * big, 3 * big, 257, 4 * big, None) == SHAPE
    assert lib.ttr_apply(d, big, 2 * big, None, None, 3 * big, 1e-6, 4 * big, None) == NULL
    assert lib.ttr_blend(D(F=64), big, 2 * big, None, 3 * big, None) == NULL
    assert lib.ttr_kv_reduce(D(N=4096), big, 2 * big, 3 * big, None, 4 * big, 5 * big, None, 0, None) == WS


def test_distillation_validation(lib):
    # host-side checks of the distillation steps (no launch: every call fails before enqueueing)
    big = 1 << 40
    d = D(B=1, H=2, N=256, Dm=64, F=256, dt=0)
    P9 = [big * (i + 1) for i in range(9)]
    Q, K, V, T, W, b, g, s_, m = P9
    loss, ws = 10 * big, 11 * big

    def rows(nq, step=1, lr=1e-3, L=16, wsb=1 << 40, teacher=T):
        return lib.ttr_distill_step_rows(d, nq, Q, K, V, teacher, W, b, g, s_, m, step, lr, 1e-6, L, loss, ws, wsb,
                                         None)

    assert rows(0) == SHAPE and rows(257) == SHAPE         # 1 <= Nq <= N
    assert rows(64, step=0) == SHAPE and rows(64, lr=0.0) == SHAPE
    assert rows(64, L=257) == SHAPE
    assert rows(64, wsb=16) == WS
    assert lib.ttr_distill_rows_workspace_bytes(d, 0, 16, 0) == 0
    assert lib.ttr_distill_rows_workspace_bytes(d, 257, 16, 0) == 0
    full = lib.ttr_distill_rows_workspace_bytes(d, 256, 16, 1)
    assert full == lib.ttr_distill_workspace_bytes(d, 16, 1) > 0
    assert 0 < lib.ttr_distill_rows_workspace_bytes(d, 64, 16, 1) < full
    assert lib.ttr_distill_step(d, Q, K, V, T, W, b, g, s_, m, 1, 1e-3, 1e-6, 16, loss, ws, 16, None) == WS


def test_workspace_bytes(lib):
    assert lib.ttr_workspace_bytes(D(Dm=96), 0, 0, 0) == 0
    assert lib.ttr_workspace_bytes(D(), 300, 0, 0) == 0
    c2 = lib.ttr_workspace_bytes(ttr.Dims(1, 24, 4608, 128, 256, 1), 128, 0, 0)
    # at least KV and ksum in fp32
    assert c2 >= 24 * (256 * 128 + 256) * 4
    assert lib.ttr_workspace_bytes(ttr.Dims(8, 8, 32768, 64, 64, 1), 0, 1, 256) > 0
    # feature dimension: bf16 F = 512, 768, 1024 have growing workspaces, F = 384 (not a multiple
    # of 256) and 1280 (beyond the implemented) none
    c4 = lib.ttr_workspace_bytes(ttr.Dims(1, 24, 4608, 128, 512, 1), 128, 0, 0)
    c6 = lib.ttr_workspace_bytes(ttr.Dims(1, 24, 4608, 128, 768, 1), 128, 0, 0)
    c8 = lib.ttr_workspace_bytes(ttr.Dims(1, 24, 4608, 128, 1024, 1), 128, 0, 0)
    assert c8 > c6 > c4 > c2
    assert lib.ttr_workspace_bytes(ttr.Dims(1, 24, 4608, 128, 384, 1), 128, 0, 0) == 0
    assert lib.ttr_workspace_bytes(ttr.Dims(1, 24, 4608, 128, 1280, 1), 128, 0, 0) == 0
    assert lib.ttr_workspace_bytes(ttr.Dims(1, 2, 256, 64, 512, 0), 16, 0, 0) == 0  # fp32: 256 only


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(ttr, "_lib", None)
    monkeypatch.setattr(ttr, "library_path", lambda: str(tmp_path / "libttr.so"))
    with pytest.raises(ImportError):
        ttr.load_library()


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "linear_hybrid_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("oracle-free", ""), f

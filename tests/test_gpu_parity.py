"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Metric: per (batch, head) slice, max|gpu - oracle| / max|oracle|; bars 1e-4
for fp32 IO and 2e-2 for bf16 IO. Inputs are the seeded workloads of
workloads.py; the bf16 bit patterns are shared exactly by both sides.
"""
import numpy as np
import pytest
import torch

import linear_hybrid_attention_amd as ttr
import oracle.ttr_oracle as O
import workloads
from _util import TOL, dev_f32, host, normwise, small, to_device

pytestmark = pytest.mark.gpu


def oracle_hybrid(w, x):
    return O.hybrid_forward(x["Q"], x["K"], x["V"], x["W"], x["b"], x["g"], x["eps"], w.L)


def run_hybrid(w, d):
    return ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], d["g"], float(np.float32(w.eps)), w.L)


# ------------------------------------------------------------------ whole forward, all workloads

@pytest.mark.parametrize("name", ["tiny_fp32", "flux_512", "flux_1024", "flux_2048", "flux_1024_h3"])
def test_hybrid_forward_full_workloads(name):
    w = workloads.WORKLOADS[name]
    x = workloads.make_inputs(w)
    print(f"[hybrid] {name} B={w.B} H={w.H} N={w.N} D={w.D} F={w.F} L={w.L}", flush=True)
    out = run_hybrid(w, to_device(w, x))
    torch.cuda.synchronize()
    ref = oracle_hybrid(w, x)
    err = normwise(host(out), ref)
    print(f"[hybrid] {name} normwise err {err:.3e}", flush=True)
    assert np.isfinite(host(out)).all()
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("shape", [dict(), dict(B=2, H=2, N=777, L=33), dict(H=2, N=1500, D=64, L=48),
                                   dict(H=2, N=1000, L=0)])
def test_hybrid_forward_feature_dim_512(shape):
    # feature_dim 512 ("Flux2TTRTrainer", "Inputs worth setting": a multiple of
    # 256): the flux_1024 shape at F = 512, every element, and ragged shapes
    w = small("flux_1024", F=512, seed=40 + len(shape), **shape)
    x = workloads.make_inputs(w)
    print(f"[hybrid-f512] B={w.B} H={w.H} N={w.N} D={w.D} F={w.F} L={w.L}", flush=True)
    out = run_hybrid(w, to_device(w, x))
    torch.cuda.synchronize()
    ref = oracle_hybrid(w, x)
    err = normwise(host(out), ref)
    print(f"[hybrid-f512] normwise err {err:.3e}", flush=True)
    assert np.isfinite(host(out)).all()
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("F,shape", [(768, dict()), (1024, dict()), (768, dict(B=2, H=2, N=777, L=33)),
                                     (1024, dict(H=2, N=1500, D=64, L=48)), (1024, dict(H=2, N=300, L=0)),
                                     (768, dict(H=3, N=999, D=64, L=20)), (256, dict(B=2))])
def test_hybrid_forward_feature_dim_768_1024(F, shape):
    # feature_dim 768 and 1024 (a multiple of 256, "Flux2TTRTrainer", "Inputs
    # worth setting"): the flux_1024 shape, every element, and ragged shapes;
    # last, the flux_1024 shape with two batches (F = 256)
    w = small("flux_1024", F=F, seed=70 + F // 256 + len(shape), **shape)
    x = workloads.make_inputs(w)
    print(f"[hybrid-f{F}] B={w.B} H={w.H} N={w.N} D={w.D} F={w.F} L={w.L}", flush=True)
    out = run_hybrid(w, to_device(w, x))
    torch.cuda.synchronize()
    err = normwise(host(out), oracle_hybrid(w, x))
    print(f"[hybrid-f{F}] normwise err {err:.3e}", flush=True)
    assert np.isfinite(host(out)).all()
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("shape", [dict(N=256, D=128, L=16), dict(B=2, H=3, N=333, D=128, L=7),
                                   dict(N=200, D=128, L=0), dict(N=100, D=128, F=128, proj=False, L=5)])
def test_hybrid_forward_fp32_d128(shape):
    # fp32 IO with D = 128: W^T and KV^T are staged 64 features at a time
    # (together they would fill 256 KB of LDS); identity map: F = D = 128
    w = small("tiny_fp32", seed=60 + len(shape) + shape["N"], **shape)
    x = workloads.make_inputs(w)
    print(f"[hybrid-fp32-d128] B={w.B} H={w.H} N={w.N} D={w.D} F={w.F} L={w.L}", flush=True)
    out = run_hybrid(w, to_device(w, x))
    torch.cuda.synchronize()
    err = normwise(host(out), oracle_hybrid(w, x))
    print(f"[hybrid-fp32-d128] normwise err {err:.3e}", flush=True)
    assert np.isfinite(host(out)).all()
    assert err <= TOL["fp32"], err


@pytest.mark.timeout(600)
def test_causal_full_size_whole_output():
    # the causal configuration as stated (chunk 256) through the metric entry
    # point, every element of all 64 (batch, head) slices against the oracle's
    # per-token prefix recurrence; chunks 128 and 64 of the scan on the same inputs
    w = workloads.WORKLOADS["causal"]
    x = workloads.make_inputs(w)
    d = to_device(w, x)
    eps = float(np.float32(w.eps))
    print(f"[causal] B={w.B} H={w.H} N={w.N} D={w.D} chunk={w.chunk} (hybrid entry point)", flush=True)
    assert w.chunk == 256
    outs = {256: host(ttr.hybrid_forward(d["Q"], d["K"], d["V"], None, None, None, eps, 0, causal=True,
                                         chunk=w.chunk))}
    for c in (128, 64):
        print(f"[causal] chunk {c} (scan entry point)", flush=True)
        outs[c] = host(ttr.causal_scan(d["Q"], d["K"], d["V"], eps=eps, chunk=c))
    torch.cuda.synchronize()
    print("[causal] oracle (per-token recurrence over 32768 tokens)", flush=True)
    ref = O.causal_forward(x["Q"], x["K"], x["V"], None, None, x["eps"])
    for c, out in outs.items():
        assert np.isfinite(out).all()
        err = normwise(out, ref)
        # per-row normwise error, a diagnostic: |gpu - ref| / max|ref| within each row
        row = float((np.abs(out - ref).max(axis=-1) / np.abs(ref).max(axis=-1)).max())
        print(f"[causal] chunk {c}: slice normwise err {err:.3e}, worst row {row:.3e}", flush=True)
        assert err <= TOL["bf16"], (c, err)


@pytest.mark.parametrize("dtype,D,chunk", [("bf16", 64, 256), ("bf16", 64, 128), ("bf16", 64, 64),
                                           ("bf16", 128, 128), ("bf16", 128, 64), ("fp32", 64, 128),
                                           ("fp32", 64, 64), ("fp32", 128, 64)])
def test_causal_small_full(dtype, D, chunk):
    w = small("causal", B=2, H=3, N=1000, D=D, F=D, dtype=dtype, seed=11)
    x = workloads.make_inputs(w)
    print(f"[causal-small] {dtype} D={D} chunk={chunk} N={w.N}", flush=True)
    d = to_device(w, x)
    out = ttr.causal_scan(d["Q"], d["K"], d["V"], eps=float(np.float32(w.eps)), chunk=chunk)
    torch.cuda.synchronize()
    ref = O.causal_forward(x["Q"], x["K"], x["V"], None, None, x["eps"])
    err = normwise(host(out), ref)
    print(f"[causal-small] err {err:.3e}", flush=True)
    assert err <= TOL[dtype], err


def test_causal_chunk_invariance_and_bias():
    w = small("causal", B=1, H=2, N=777, seed=12)
    x = workloads.make_inputs(w)
    d = to_device(w, x)
    b = np.random.default_rng(3).standard_normal((w.H, w.D)).astype(np.float32) * 0.1
    outs = [host(ttr.causal_scan(d["Q"], d["K"], d["V"], b=dev_f32(b), chunk=c)) for c in (64, 128, 256)]
    ref = O.causal_forward(x["Q"], x["K"], x["V"], None, b, x["eps"])
    for o in outs:
        assert normwise(o, ref) <= TOL["bf16"]
    assert normwise(outs[0], outs[2]) <= TOL["bf16"]


@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("B,H,N", [(4, 256, 333), (2, 260, 1100)])
def test_causal_segments_of_several_chunks(B, H, N, chunk):
    # Enough (batch, head) slices that each segment walks several chunks
    # (one segment per slice for B*H >= 1024, two for B*H = 520): every slice
    # is independent, so a few of them are checked against the oracle.
    w = small("causal", B=B, H=H, N=N, seed=15)
    x = workloads.make_inputs(w)
    d = to_device(w, x)
    b = np.random.default_rng(4).standard_normal((w.H, w.D)).astype(np.float32) * 0.1
    print(f"[causal-segments] B={B} H={H} N={N} chunk={chunk}", flush=True)
    out = ttr.causal_scan(d["Q"], d["K"], d["V"], b=dev_f32(b), chunk=chunk)
    torch.cuda.synchronize()
    for bi, hi in [(0, 0), (0, 1), (B - 1, H - 1), (B // 2, H // 2)]:
        sl = (slice(bi, bi + 1), slice(hi, hi + 1))
        ref = O.causal_forward(x["Q"][sl], x["K"][sl], x["V"][sl], None, b[hi:hi + 1], x["eps"])
        err = normwise(host(out[sl]), ref)
        assert err <= TOL["bf16"], (bi, hi, err)


def test_causal_last_token_equals_noncausal():
    # identity feature map on both sides; the last causal row sees every token
    w = small("causal", B=1, H=2, N=500, seed=13)
    x = workloads.make_inputs(w)
    d = to_device(w, x)
    c = host(ttr.causal_scan(d["Q"], d["K"], d["V"], chunk=128))
    nc = host(ttr.hybrid_forward(d["Q"], d["K"], d["V"], None, None, None, 1e-6, 0))
    last = np.abs(c[:, :, -1] - nc[:, :, -1]).max() / np.abs(nc[:, :, -1]).max()
    assert last <= TOL["bf16"], last


def test_hybrid_causal_route():
    w = small("causal", B=1, H=2, N=300, seed=14)
    x = workloads.make_inputs(w)
    d = to_device(w, x)
    out = ttr.hybrid_forward(d["Q"], d["K"], d["V"], None, None, None, 1e-6, 0, causal=True)
    ref = O.causal_forward(x["Q"], x["K"], x["V"], None, None, x["eps"])
    assert normwise(host(out), ref) <= TOL["bf16"]


# ------------------------------------------------------------------ staged calls

STAGED = [("tiny_fp32", {}), ("flux_512", dict(H=3, N=1000, L=7, seed=21)),
          ("flux_512", dict(H=2, N=333, D=64, L=33, seed=22)),
          ("tiny_fp32", dict(N=257, L=5, seed=23)),
          ("tiny_fp32", dict(H=3, N=300, D=128, L=9, seed=26)),  # fp32 with D = 128
          ("flux_1024", {})]  # the staged calls at the size their bench line times


@pytest.mark.parametrize("name,kw", STAGED)
def test_staged_stages(name, kw):
    w = small(name, **kw)
    x = workloads.make_inputs(w)
    d = to_device(w, x)
    tol = TOL[w.dtype]
    print(f"[staged] {w}", flush=True)
    phi = ttr.feature_map(d["Q"], d["W"], d["b"])
    assert normwise(host(phi), O.feature_map(x["Q"], x["W"], x["b"])) <= tol
    assert (host(phi) > 0).all()  # phi > 0 on the workload's pre-activations

    KV, ksum = ttr.kv_reduce(d["K"], d["V"], d["W"], d["b"])
    KVr, ksr = O.kv_reduce(x["K"], x["V"], x["W"], x["b"])
    assert normwise(host(KV), KVr) <= tol
    assert normwise(host(ksum)[..., None], ksr[..., None]) <= tol

    lin = ttr.apply(d["Q"], d["W"], d["b"], dev_f32(KVr), dev_f32(ksr), float(x["eps"]))
    lin_ref = O.apply(x["Q"], x["W"], x["b"], KVr, ksr, x["eps"])
    assert normwise(host(lin), lin_ref) <= tol

    lm = ttr.landmark_attn(d["Q"], d["K"], d["V"], w.L)
    lm_ref = O.landmark_attn(x["Q"], x["K"], x["V"], w.L)
    assert normwise(host(lm), lm_ref) <= tol

    tdt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    out = ttr.blend(dev_f32(lin_ref), dev_f32(lm_ref), d["g"], dtype=tdt)
    assert normwise(host(out), O.blend(lin_ref, lm_ref, x["g"])) <= tol


def test_feature_map_identity_and_bias():
    w = small("tiny_fp32", H=3, N=100, F=64, proj=False, seed=24)
    x = workloads.make_inputs(w)
    d = to_device(w, x)
    b = np.random.default_rng(5).standard_normal((w.H, w.D)).astype(np.float32)
    phi = ttr.feature_map(d["Q"], None, dev_f32(b))
    assert normwise(host(phi), O.feature_map(x["Q"], None, b)) <= TOL["fp32"]


# ------------------------------------------------------------------ invariants and edge cases

def _bf16_case(**kw):
    w = small("flux_512", **kw)
    x = workloads.make_inputs(w)
    return w, x, to_device(w, x)


def test_alpha_limits():
    w, x, d = _bf16_case(H=2, N=640, L=20, seed=31)
    for gval, ref in ((-np.inf, O.landmark_attn(x["Q"], x["K"], x["V"], w.L)),
                      (np.inf, O.apply(x["Q"], x["W"], x["b"], *O.kv_reduce(x["K"], x["V"], x["W"], x["b"]),
                                       x["eps"]))):
        g = torch.full((w.H,), float(gval), device="cuda")
        out = ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], g, 1e-6, w.L)
        assert normwise(host(out), ref) <= TOL["bf16"]


def test_all_landmarks_alpha_zero_is_full_softmax():
    w, x, d = _bf16_case(H=2, N=256, L=256, seed=32)
    g = torch.full((w.H,), float("-inf"), device="cuda")
    out = ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], g, 1e-6, 256)
    q, k, v = (torch.from_numpy(x[n]).double() for n in ("Q", "K", "V"))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()
    assert normwise(host(out), ref) <= TOL["bf16"]


def test_single_landmark_and_no_landmarks():
    w, x, d = _bf16_case(H=2, N=300, L=1, seed=33)
    lm = host(ttr.landmark_attn(d["Q"], d["K"], d["V"], 1))
    assert np.array_equal(lm, np.broadcast_to(x["V"][:, :, :1, :].astype(np.float64), lm.shape))
    out = ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], d["g"], 1e-6, 0)
    ref = O.hybrid_forward(x["Q"], x["K"], x["V"], x["W"], x["b"], x["g"], x["eps"], 0)
    assert normwise(host(out), ref) <= TOL["bf16"]


@pytest.mark.parametrize("N", [1, 2, 31, 33, 129, 257, 1000])
def test_ragged_lengths(N):
    w, x, d = _bf16_case(B=2, H=2, N=N, L=min(N, 9), seed=40 + N)
    out = run_hybrid(w, d)
    assert normwise(host(out), oracle_hybrid(w, x)) <= TOL["bf16"]
    wf = small("tiny_fp32", N=N, L=min(N, 3), seed=50 + N)
    xf = workloads.make_inputs(wf)
    outf = run_hybrid(wf, to_device(wf, xf))
    assert normwise(host(outf), oracle_hybrid(wf, xf)) <= TOL["fp32"]


def test_identity_map_noncausal_hybrid():
    w = small("flux_512", H=2, N=400, D=128, F=128, proj=False, L=10, seed=34)
    x = workloads.make_inputs(w)
    d = to_device(w, x)
    out = run_hybrid(w, d)
    assert normwise(host(out), oracle_hybrid(w, x)) <= TOL["bf16"]


def test_deterministic_bitwise():
    w, x, d = _bf16_case(H=4, N=2000, L=40, seed=35)
    a = run_hybrid(w, d)
    b = run_hybrid(w, d)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    wc = small("causal", B=1, H=4, N=3000, seed=36)
    dc = to_device(wc, workloads.make_inputs(wc))
    c1 = ttr.causal_scan(dc["Q"], dc["K"], dc["V"])
    c2 = ttr.causal_scan(dc["Q"], dc["K"], dc["V"])
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_output_guard_bands_untouched():
    w, x, d = _bf16_case(H=3, N=999, L=11, seed=37)
    n = w.B * w.H * w.N * w.D
    pad = 4096
    flat = torch.full((n + 2 * pad,), 1234.0, dtype=torch.bfloat16, device="cuda")
    out = flat[pad:pad + n].view(w.B, w.H, w.N, w.D)
    ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], d["g"], 1e-6, w.L, out=out)
    torch.cuda.synchronize()
    assert (flat[:pad] == 1234.0).all() and (flat[pad + n:] == 1234.0).all()
    assert normwise(host(out), oracle_hybrid(w, x)) <= TOL["bf16"]
    # causal writes stay inside too
    wc = small("causal", B=1, H=2, N=513, seed=38)
    dc = to_device(wc, workloads.make_inputs(wc))
    nc = wc.H * wc.N * wc.D
    flat = torch.full((nc + 2 * pad,), 1234.0, dtype=torch.bfloat16, device="cuda")
    ttr.causal_scan(dc["Q"], dc["K"], dc["V"], out=flat[pad:pad + nc].view(1, wc.H, wc.N, wc.D))
    torch.cuda.synchronize()
    assert (flat[:pad] == 1234.0).all() and (flat[pad + nc:] == 1234.0).all()


def test_errors_raise_on_gpu():
    w, x, d = _bf16_case(H=2, N=64, L=4, seed=39)
    with pytest.raises(ttr.TTRError) as e:
        ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], d["g"], 1e-6, 65)
    assert e.value.status == 2
    with pytest.raises(ttr.TTRError):
        ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], d["g"], 1e-6, 4, out=d["Q"])

"""GPU parity of the hybrid backward (ttr_hybrid_backward: dW, db, dg) against
the fp64 oracle's chain rule, which finite differences and torch autograd pin.

Bar: normwise error per gradient tensor (max |gpu - ref| / max |ref|) at most
1e-4 for fp32 IO and 2e-2 for bf16 IO (the bf16 path runs its products on bf16
operands with fp32 accumulation and fp32 intermediates)."""
import numpy as np
import pytest
import torch

import linear_hybrid_attention_amd as ttr
import oracle.ttr_oracle as O
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def _dev_io(x, name, w):
    if x[name] is None:
        return None
    if w.dtype == "bf16":
        return torch.from_numpy(x[name + "_bits"].view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(x[name]).to(DEV)


def _check(w, seed=7, no_bias=False):
    print(f"[backward] {w.name} B={w.B} H={w.H} N={w.N} D={w.D} F={w.F} L={w.L} {w.dtype} bias={not no_bias}",
          flush=True)
    x = workloads.make_inputs(w)
    dout = workloads.make_grad_output(w, seed)
    b = None if no_bias else x["b"]
    Q, K, V, W = (_dev_io(x, k, w) for k in ("Q", "K", "V", "W"))
    bt = None if b is None else torch.from_numpy(b).to(DEV)
    g = torch.from_numpy(x["g"]).to(DEV)
    dW, db, dg = ttr.hybrid_backward(Q, K, V, W, bt, g, float(x["eps"]), w.L, torch.from_numpy(dout).to(DEV))
    torch.cuda.synchronize()
    rW, rb, rg = O.hybrid_backward(x["Q"], x["K"], x["V"], x["W"], b, x["g"], float(x["eps"]), w.L, dout)
    errs = []
    for got, ref in ((dW, rW), (db, rb), (dg, rg)):
        got = got.cpu().numpy()
        assert np.isfinite(got).all()
        scale = np.abs(ref).max()
        errs.append(0.0 if scale == 0 else float(np.abs(got - ref).max() / scale))
        if scale == 0:
            assert not got.any()
    print(f"[backward] normwise errors dW {errs[0]:.2e} db {errs[1]:.2e} dg {errs[2]:.2e}", flush=True)
    assert max(errs) <= TOL[w.dtype]
    return dW, db, dg


BASE = workloads.WORKLOADS


@pytest.mark.parametrize("w", [
    BASE["tiny_fp32"].with_(name="bw_fp32", N=100, L=10),
    BASE["tiny_fp32"].with_(name="bw_fp32_l0", N=130, L=0),
    BASE["flux_512"].with_(name="bw_bf16", B=2, H=3, N=300, L=20),
    BASE["flux_512"].with_(name="bw_bf16_d64", B=1, H=2, N=257, D=64, L=7, w_std=0.125),
    BASE["flux_512"].with_(name="bw_bf16_l0", B=1, H=2, N=190, L=0),
    # whole row groups and K-steps (the products' unconditional-load variant) with a partial last tile
    BASE["flux_512"].with_(name="bw_bf16_rows16", B=1, H=2, N=272, L=16),
    BASE["tiny_fp32"].with_(name="bw_fp32_rows32", N=160, L=8),
    BASE["tiny_fp32"].with_(name="bw_fp32_d128", N=120, D=128, L=6, w_std=1 / np.sqrt(128.0)),
], ids=lambda w: w.name)
def test_backward_matches_oracle(w):
    _check(w)


def test_backward_without_bias():
    _check(BASE["flux_512"].with_(name="bw_nobias", B=1, H=2, N=140, L=12), no_bias=True)


def test_backward_full_size_flux_1024():
    _check(BASE["flux_1024"])


def test_backward_is_bitwise_deterministic():
    w = BASE["flux_512"].with_(name="bw_det", B=1, H=2, N=200, L=8)
    a = _check(w)
    b = _check(w)
    for x, y in zip(a, b):
        assert torch.equal(x, y)

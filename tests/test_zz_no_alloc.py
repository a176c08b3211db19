"""ttr_hybrid_forward_noalloc (the library's fixed per-GPU workspace) against
ttr_hybrid_forward with a caller's workspace, through the C ABI: the same
kernels on the same inputs, so the outputs must agree bit for bit (which is
within the oracle bar the forward's own parity tests hold it to). Two calls in
a row, the second with a smaller input (the array keeps the first call's
contents), a causal call, and a request beyond the array's size."""
import numpy as np
import pytest
import torch

import linear_hybrid_attention_amd as ttr
import workloads
from _util import host, small, to_device

pytestmark = pytest.mark.gpu


def _pair(w, causal=False, chunk=0):
    x = workloads.make_inputs(w)
    d = to_device(w, x)
    eps = float(np.float32(w.eps))
    print(f"[noalloc] B={w.B} H={w.H} N={w.N} D={w.D} F={w.F} L={w.L} causal={causal}", flush=True)
    W, b, g = (None, None, None) if causal else (d["W"], d["b"], d["g"])
    ref = ttr.hybrid_forward(d["Q"], d["K"], d["V"], W, b, g, eps, w.L, causal=causal, chunk=chunk)
    got = ttr.hybrid_forward_noalloc(d["Q"], d["K"], d["V"], W, b, g, eps, w.L, causal=causal, chunk=chunk)
    torch.cuda.synchronize()
    return host(got), host(ref)


def test_noalloc_matches_workspace_entry_point_twice():
    # a flux-shaped call, then a smaller one on the same array
    first = small("flux_1024", H=4, N=2000, L=64, seed=31)
    second = small("flux_1024", H=2, N=700, L=16, seed=32)
    for w in (first, second):
        need = ttr.workspace_bytes(w.B, w.H, w.N, w.D, w.F, 1, w.L, False, 0)
        assert 0 < need <= ttr.NOALLOC_SCRATCH_BYTES
        got, ref = _pair(w)
        assert np.isfinite(got).all()
        assert np.array_equal(got, ref)


def test_noalloc_full_size_flux_1024():
    w = workloads.WORKLOADS["flux_1024"]
    got, ref = _pair(w)
    assert np.array_equal(got, ref)


def test_noalloc_causal():
    w = small("causal", B=2, H=3, N=5000, D=64, F=64, seed=33)
    got, ref = _pair(w, causal=True, chunk=128)
    assert np.array_equal(got, ref)


def test_noalloc_full_size_causal():
    # the causal configuration at its stated chunk: the largest workspace of the workloads
    w = workloads.WORKLOADS["causal"]
    need = ttr.workspace_bytes(w.B, w.H, w.N, w.D, w.F, 1, 0, True, w.chunk)
    assert need <= ttr.NOALLOC_SCRATCH_BYTES
    got, ref = _pair(w, causal=True, chunk=w.chunk)
    assert np.array_equal(got, ref)


def test_noalloc_rejects_beyond_the_array():
    # host-side check: the call needs more than the array holds, nothing runs
    w = small("flux_1024", B=8, H=64, N=4096, L=0, seed=34)
    need = ttr.workspace_bytes(w.B, w.H, w.N, w.D, w.F, 1, w.L, False, 0)
    assert need > ttr.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda:0")
    Q = torch.zeros(w.B, w.H, w.N, w.D, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(w.H, w.D, w.F, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ttr.TTRError) as e:
        ttr.hybrid_forward_noalloc(Q, Q, Q, W, None, None, 1e-6, 0)
    assert e.value.status == 5  # TTR_ERR_WORKSPACE

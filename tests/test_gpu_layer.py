"""GPU parity of the NNT linear-attention layer (ttr_nnt_layer_forward)
against the fp64 oracle: projections, heads, attention (causal or not, every
feature map) and the out projection, on ragged token counts that span several
128-row tiles, and on sampled batches of the full-size workload.

Bar: the normwise error per batch (max |gpu - ref| / max |ref| over [N, E]) is
at most 1e-4 for fp32 IO and 2e-2 for bf16 IO (Q, K, V and the attention
output are rounded to bf16 between the stages)."""
import numpy as np
import pytest
import torch

import linear_hybrid_attention_amd as ttr
import oracle.ttr_oracle as O
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def _to_dev(x, bits, dtype):
    if dtype == "bf16":
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(x).to(DEV)


def _run(w, x):
    t = {k: _to_dev(x[k], x.get(k + "_bits"), w.dtype) for k in ("x", "Wq", "Wk", "Wv", "Wo")}
    b = {k: None if x[k] is None else torch.from_numpy(x[k]).to(DEV) for k in ("bq", "bk", "bv", "bo")}
    out = ttr.nnt_layer_forward(t["x"], t["Wq"], b["bq"], t["Wk"], b["bk"], t["Wv"], b["bv"], t["Wo"], b["bo"],
                                w.H, float(x["eps"]), w.causal, w.fmap)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _ref(w, x, batches=None):
    sel = slice(None) if batches is None else batches
    return O.nnt_layer_forward(x["x"][sel], x["Wq"], x["bq"], x["Wk"], x["bk"], x["Wv"], x["bv"], x["Wo"], x["bo"],
                               w.H, float(x["eps"]), w.causal, w.fmap)


def _err(got, ref):
    return max(float(np.abs(got[i] - ref[i]).max() / np.abs(ref[i]).max()) for i in range(ref.shape[0]))


CASES = [
    ("bf16", 2, 200, 256, 4, False, "elu1"),
    ("bf16", 2, 200, 256, 4, True, "elu1"),
    ("bf16", 1, 300, 256, 2, False, "elu1"),      # D = 128
    ("bf16", 1, 300, 256, 2, True, "elu1"),       # D = 128, causal
    ("bf16", 1, 130, 512, 8, True, "relu"),
    ("bf16", 2, 77, 512, 8, False, "softmax"),
    ("bf16", 3, 1, 128, 2, False, "elu1"),        # one token per sequence
    ("fp32", 1, 150, 128, 2, False, "elu1"),
    ("fp32", 1, 150, 128, 2, True, "elu1"),
    ("fp32", 2, 64, 256, 4, False, "relu"),
    ("fp32", 1, 129, 256, 4, True, "softmax"),
    ("fp32", 2, 100, 256, 2, False, "elu1"),      # D = 128
    ("fp32", 1, 150, 256, 2, True, "elu1"),       # D = 128, causal (chunk 64)
]


@pytest.mark.parametrize("dtype,B,N,E,H,causal,fmap", CASES)
def test_layer_matches_oracle(dtype, B, N, E, H, causal, fmap):
    w = workloads.LayerWorkload("t", B, N, E, H, dtype, causal, fmap, 2000 + N + E)
    print(f"[layer] {dtype} B={B} N={N} E={E} H={H} causal={causal} {fmap}", flush=True)
    x = workloads.make_layer_inputs(w)
    got, ref = _run(w, x), _ref(w, x)
    assert np.isfinite(got).all()
    e = _err(got, ref)
    print(f"[layer] normwise error {e:.3e}", flush=True)
    assert e <= TOL[dtype]


def test_layer_without_biases():
    w = workloads.LayerWorkload("t", 2, 140, 256, 4, "bf16", False, "elu1", 2100)
    x = workloads.make_layer_inputs(w, bias=False)
    assert _err(_run(w, x), _ref(w, x)) <= TOL["bf16"]


def test_layer_repeated_calls_are_bitwise_equal():
    w = workloads.LayerWorkload("t", 1, 257, 512, 8, "bf16", True, "elu1", 2101)
    x = workloads.make_layer_inputs(w)
    assert np.array_equal(_run(w, x), _run(w, x))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["nnt_layer", "nnt_layer_causal"])
def test_layer_full_size_all_sequences(name):
    # the full workload on the GPU, every element of all B sequences against the oracle
    w = workloads.LAYER_WORKLOADS[name]
    print(f"[layer] full size {name}", flush=True)
    x = workloads.make_layer_inputs(w)
    got = _run(w, x)
    ref = _ref(w, x, list(range(w.B)))
    e = _err(got, ref)
    print(f"[layer] {name} normwise error {e:.3e}", flush=True)
    assert e <= TOL[w.dtype]

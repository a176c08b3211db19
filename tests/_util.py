"""Shared test helpers: device copies of the seeded inputs and the parity metric."""
import numpy as np
import torch

import workloads

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def dev_io(arr_f32, bits, dtype, device="cuda"):
    """Canonical input -> device tensor in the IO dtype (bit-exact for bf16)."""
    if arr_f32 is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr_f32, dtype=np.float32)).to(device)


def dev_f32(arr, device="cuda"):
    if arr is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_device(w, x, device="cuda"):
    """Device tensors Q, K, V, W (IO dtype) and b, g (fp32) for workload w."""
    d = {}
    for k in ("Q", "K", "V", "W"):
        d[k] = dev_io(x[k], x.get(k + "_bits"), w.dtype, device)
    d["b"] = dev_f32(x["b"], device)
    d["g"] = dev_f32(x["g"], device)
    return d


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise(got, ref):
    """max over leading slices of max|got-ref| / max|ref| over the last two axes."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(got - ref).max(axis=(-2, -1))
    den = np.abs(ref).max(axis=(-2, -1))
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def small(name, **kw):
    return workloads.WORKLOADS[name].with_(**kw)

"""GPU parity of the cosine distance (ttr_cosine_distance) against the
oracle's definition, on the IO values both sides read; and the gate driven by
it over a short distillation run. Bar: relative error 1e-4 (fp32
accumulation over rows of D values, two fixed-order reduction levels)."""
import numpy as np
import pytest
import torch

import linear_hybrid_attention_amd as ttr
import oracle.ttr_oracle as O
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("dtype,B,H,N,D", [("fp32", 1, 2, 300, 64), ("bf16", 2, 3, 1000, 128),
                                           ("bf16", 1, 24, 4608, 128), ("bf16", 1, 1, 1, 64)])
def test_cosine_distance_matches_oracle(dtype, B, H, N, D):
    r = np.random.default_rng(N + D)
    t = r.standard_normal((B, H, N, D), dtype=np.float32)
    o = (t + 0.7 * r.standard_normal((B, H, N, D), dtype=np.float32)).astype(np.float32)
    if dtype == "bf16":
        ob, tb = workloads.bf16_round_bits(o), workloads.bf16_round_bits(t)
        o, t = workloads.bf16_bits_to_f32(ob), workloads.bf16_bits_to_f32(tb)
        od = torch.from_numpy(ob.view(np.int16)).view(torch.bfloat16).to(DEV)
        td = torch.from_numpy(tb.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        od, td = torch.from_numpy(o).to(DEV), torch.from_numpy(t).to(DEV)
    got = float(ttr.cosine_distance(od, td).cpu())
    ref = O.cosine_distance(o, t)
    print(f"[gate] cosine distance {dtype} {B}x{H}x{N}x{D}: {got:.7f} vs {ref:.7f}", flush=True)
    assert abs(got - ref) <= 1e-4 * max(abs(ref), 1e-3)
    assert float(ttr.cosine_distance(td, td).cpu()) < 1e-5


def test_gate_follows_a_distillation_run():
    # the student approaches the teacher; the gate opens only after min_updates and a low EMA distance
    w = workloads.WORKLOADS["flux_512"].with_(name="gate_run", B=1, H=2, N=256, L=16)
    x = workloads.make_inputs(w)
    io = lambda k: torch.from_numpy(x[k + "_bits"].view(np.int16)).view(torch.bfloat16).to(DEV)
    Q, K, V = io("Q"), io("K"), io("V")
    st = ttr.DistillState(torch.from_numpy(x["W"]).to(DEV), torch.from_numpy(x["b"]).to(DEV),
                          torch.from_numpy(x["g"]).to(DEV))
    losses = [ttr.distill_step(st, Q, K, V, w.L, 3e-3, float(x["eps"])).cpu().numpy() for _ in range(40)]
    cos = [float(l[2]) for l in losses]
    gate, ref = ttr.ReadinessGate(0.8, cos[-1] * 1.05, cos[-1] * 1.2, 10), O.ReadinessGate(0.8, cos[-1] * 1.05,
                                                                                          cos[-1] * 1.2, 10)
    states = [gate.update(c) for c in cos]
    assert states == [ref.update(c) for c in cos]
    assert not any(states[:9]) and states[-1]

"""The readiness gate and the landmark-count rule of the library (host code,
no GPU) against the oracle's: identical decisions on long random distance
sequences (both sides in fp64), the hand-worked cases, fail-closed behaviour
and argument validation."""
import numpy as np
import pytest

import linear_hybrid_attention_amd as ttr
import oracle.ttr_oracle as O


@pytest.mark.parametrize("seed", range(6))
def test_gate_matches_oracle_on_random_sequences(seed):
    r = np.random.default_rng(seed)
    rate, on = float(r.uniform(0, 0.95)), float(r.uniform(0.02, 0.2))
    off, mins = on + float(r.uniform(0, 0.1)), int(r.integers(0, 20))
    lib_gate, ref = ttr.ReadinessGate(rate, on, off, mins), O.ReadinessGate(rate, on, off, mins)
    walk = np.clip(0.15 + np.cumsum(r.normal(0, 0.02, 400)), 0, 2)
    for d in walk:
        a, b = lib_gate.update(float(d)), ref.update(float(d))
        assert a == b and lib_gate.updates == ref.updates and lib_gate.ema == ref.ema
    assert lib_gate.ready == ref.ready


def test_gate_hand_worked():
    g = ttr.ReadinessGate(0.5, 0.1, 0.2, 1)
    seq = [(0.4, 0.4, False), (0.0, 0.2, False), (0.0, 0.1, True), (0.3, 0.2, True), (0.3, 0.25, False),
           (0.05, 0.15, False)]
    for d, ema, ready in seq:
        assert g.update(d) == ready and abs(g.ema - ema) < 1e-15


def test_gate_fails_closed():
    g = ttr.ReadinessGate(0.9, 0.1, 0.2, 5)
    assert [g.update(0.0) for _ in range(5)] == [False] * 4 + [True]
    assert g.update(float("nan")) is False and g.updates == 5 and not g.ready


def test_gate_config_validation():
    lib = ttr.load_library()
    import ctypes
    st = ttr.GateState(0.0, 0, 0)
    for cfg in (ttr.GateConfig(1.0, 0.1, 0.2, 1), ttr.GateConfig(0.5, 0.3, 0.2, 1), ttr.GateConfig(0.5, -0.1, 0.2, 1),
                ttr.GateConfig(0.5, 0.1, 0.2, -1)):
        assert lib.ttr_gate_update(ctypes.byref(cfg), ctypes.byref(st), 0.0) == 2
        assert st.updates == 0 and st.ready == 0
    assert lib.ttr_gate_update(None, ctypes.byref(st), 0.0) == 1


@pytest.mark.parametrize("N,frac,lmin,lmax", [(4608, 1 / 36, 16, 512), (1536, 1 / 24, 16, 512), (100, 0.005, 16, 512),
                                              (100000, 0.1, 16, 512), (10, 0.5, 16, 512), (30, 0.05, 0, 512),
                                              (0, 0.5, 0, 4), (257, 0.0625, 1, 64)])
def test_landmark_count_matches_oracle(N, frac, lmin, lmax):
    assert ttr.landmark_count(N, frac, lmin, lmax) == O.landmark_count(N, frac, lmin, lmax)


def test_landmark_count_validation():
    with pytest.raises(ValueError):
        ttr.landmark_count(10, -0.1, 0, 4)
    with pytest.raises(ValueError):
        ttr.landmark_count(10, 0.1, 5, 4)

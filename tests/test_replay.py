"""CPU tests of the replay buffer's host side: the library's sample footprint
equals the oracle's rule, and invalid arguments are rejected before any HIP
call. (Pushes and fetches need a GPU: tests/test_gpu_replay.py.)"""
import ctypes

import numpy as np
import pytest
import torch

import linear_hybrid_attention_amd as ttr
import oracle.ttr_oracle as O

NULL, SHAPE, DTYPE, UNSUP, BUDGET, NOT_FOUND, DEVICE = 1, 2, 3, 4, 9, 10, 11


@pytest.fixture(scope="module")
def lib():
    return ttr.load_library()


def test_sample_bytes_match_oracle():
    r = np.random.default_rng(8)
    for _ in range(200):
        dt = [torch.float32, torch.bfloat16][int(r.integers(0, 2))]
        D = 64 if dt == torch.float32 else int(r.choice([64, 128]))
        B, H, N = int(r.integers(1, 4)), int(r.integers(1, 30)), int(r.integers(1, 5000))
        Nq = int(r.integers(1, N + 1))
        teacher = bool(r.integers(0, 2))
        io = 4 if dt == torch.float32 else 2
        assert ttr.replay_sample_bytes(B, H, N, D, dt, Nq, teacher) == O.replay_sample_bytes(B, H, N, D, io, Nq,
                                                                                             teacher)


def test_sample_bytes_invalid_shape(lib):
    assert ttr.replay_sample_bytes(1, 2, 10, 64, torch.bfloat16, 0, True) == 0
    assert ttr.replay_sample_bytes(1, 2, 10, 64, torch.bfloat16, 11, True) == 0
    assert ttr.replay_sample_bytes(1, 2, 10, 96, torch.bfloat16, 3, True) == 0
    # fp32 with D = 128 is a valid sample shape (the fp32 forward, backward and
    # distillation step take D = 128)
    assert ttr.replay_sample_bytes(1, 2, 10, 128, torch.float32, 3, True) == \
        O.replay_sample_bytes(1, 2, 10, 128, 4, 3, True)
    assert lib.ttr_replay_sample_bytes(ttr.Dims(1, 2, 10, 64, 64, 7, 0), 3, 0) == 0


def test_create_rejects_bad_sizes(lib):
    h = ctypes.c_void_p(12345)
    assert lib.ttr_replay_create(1 << 20, 1 << 20, None) == NULL
    assert lib.ttr_replay_create(100, 100, ctypes.byref(h)) == SHAPE and h.value is None
    assert lib.ttr_replay_create(1 << 20, 0, ctypes.byref(h)) == SHAPE
    assert lib.ttr_replay_create(1 << 20, (1 << 20) + 1, ctypes.byref(h)) == SHAPE


def test_calls_on_null_object(lib):
    idx = np.arange(4, dtype=np.int32)
    sid = ctypes.c_int64()
    d = ttr.Dims(1, 2, 16, 64, 64, 1, 0)
    P = 1 << 20
    assert lib.ttr_replay_push(None, d, 4, P, 2 * P, 3 * P, None, idx.ctypes.data, None, ctypes.byref(sid)) == NULL
    assert lib.ttr_replay_fetch(None, 0, P, 2 * P, 3 * P, None, None, None) == NULL
    assert lib.ttr_replay_wait_pushed(None, None) == NULL
    assert lib.ttr_replay_synchronize(None) == NULL
    assert lib.ttr_replay_info(None, 0, None, None, None) == NULL
    st = ttr.ReplayStats()
    assert lib.ttr_replay_get_stats(None, ctypes.byref(st)) == NULL
    lib.ttr_replay_destroy(None)


def test_status_strings_for_replay(lib):
    assert "budget" in ttr.status_string(BUDGET)
    assert "not held" in ttr.status_string(NOT_FOUND)
    assert "device" in ttr.status_string(DEVICE)

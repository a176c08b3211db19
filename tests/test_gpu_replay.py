"""GPU tests of the replay buffer (ttr_replay_*) against the oracle's model:
the samples held after every push (ids, bytes used, evictions) are identical,
and every fetched sample is bit-identical to the oracle's stored arrays (K, V
whole, the query and teacher rows at the index subset, the indices). Byte
work, so the bar is exact equality."""
import ctypes

import numpy as np
import pytest
import torch

import linear_hybrid_attention_amd as ttr
import oracle.ttr_oracle as O
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _sample(seed, B, H, N, D, dtype, Nq, teacher):
    """Host arrays (bf16 as uint16 bit patterns) for the oracle and device tensors for the library."""
    r = np.random.default_rng(seed)
    host = {k: r.standard_normal((B, H, N, D), dtype=np.float32) for k in ("Q", "K", "V")}
    dev = {}
    for k in ("Q", "K", "V"):
        if dtype == "bf16":
            host[k] = workloads.bf16_round_bits(host[k])
            dev[k] = torch.from_numpy(host[k].view(np.int16)).view(torch.bfloat16).to(DEV)
        else:
            dev[k] = torch.from_numpy(host[k]).to(DEV)
    host["T"] = r.standard_normal((B, H, N, D), dtype=np.float32) if teacher else None
    dev["T"] = None if host["T"] is None else torch.from_numpy(host["T"]).to(DEV)
    host["idx"] = workloads.query_subsample(N, Nq, seed + 1)
    return host, dev


def _bits(t):
    a = t.cpu()
    return a.view(torch.int16).numpy().view(np.uint16) if a.dtype == torch.bfloat16 else a.numpy().view(np.uint32)


def _same(got, want):
    want = np.asarray(want)
    return got.shape == want.shape and np.array_equal(got, want.view(got.dtype))


def _check_fetch(rb, ref, sid):
    smp = ref.fetch(sid)
    Qs, K, V, T, idx = rb.fetch(sid)
    assert _same(_bits(K), smp["K"]) and _same(_bits(V), smp["V"]), f"K/V of sample {sid}"
    assert _same(_bits(Qs), smp["Q"]), f"query rows of sample {sid}"
    assert np.array_equal(idx, smp["idx"])
    if smp["T"] is None:
        assert T is None
    else:
        assert _same(_bits(T), smp["T"]), f"teacher rows of sample {sid}"


def _push_both(rb, ref, host, dev):
    sid = rb.push(dev["Q"], dev["K"], dev["V"], host["idx"], dev["T"])
    assert ref.push(host["Q"], host["K"], host["V"], host["idx"], host["T"]) == sid
    return sid


@pytest.mark.parametrize("dtype,B,H,N,D,Nq,teacher", [
    ("fp32", 1, 2, 300, 64, 77, True),
    ("bf16", 2, 3, 1000, 128, 130, False),
    ("bf16", 1, 1, 1, 64, 1, True),
    ("bf16", 1, 24, 4608, 128, 1152, True),      # one flux_1024 layer call, a quarter of the queries
])
def test_replay_round_trip_is_bit_exact(dtype, B, H, N, D, Nq, teacher):
    print(f"[replay] round trip {dtype} {B}x{H}x{N}x{D} Nq={Nq} teacher={teacher}", flush=True)
    host, dev = _sample(N + Nq, B, H, N, D, dtype, Nq, teacher)
    ref = O.ReplayBuffer(256 << 20)
    with ttr.ReplayBuffer(256 << 20, 128 << 20) as rb:
        sid = _push_both(rb, ref, host, dev)
        _check_fetch(rb, ref, sid)                # no host synchronisation between push and fetch
        d, nq, ht = rb.info(sid)
        assert (d.B, d.H, d.N, d.D, nq, ht) == (B, H, N, D, Nq, teacher)
        st = rb.stats()
        assert st.count == 1 and st.bytes_used == ref.used == O.replay_sample_bytes(
            B, H, N, D, 2 if dtype == "bf16" else 4, Nq, teacher)


def test_replay_sequence_matches_oracle():
    # random shapes, a budget of a few samples: the ring wraps many times
    r = np.random.default_rng(77)
    budget = 3 << 20
    ref = O.ReplayBuffer(budget)
    with ttr.ReplayBuffer(budget, budget) as rb:
        for step in range(60):
            dtype = ["fp32", "bf16"][int(r.integers(0, 2))]
            D = 64 if dtype == "fp32" else int(r.choice([64, 128]))
            B, H, N = int(r.integers(1, 3)), int(r.integers(1, 5)), int(r.integers(1, 1200))
            Nq, teacher = int(r.integers(1, N + 1)), bool(r.integers(0, 2))
            host, dev = _sample(1000 + step, B, H, N, D, dtype, Nq, teacher)
            foot = O.replay_sample_bytes(B, H, N, D, 2 if dtype == "bf16" else 4, Nq, teacher)
            if foot > budget:
                with pytest.raises(ttr.TTRError) as ei:
                    rb.push(dev["Q"], dev["K"], dev["V"], host["idx"], dev["T"])
                assert ei.value.status == 9
                assert ref.push(host["Q"], host["K"], host["V"], host["idx"], host["T"]) is None
            else:
                _push_both(rb, ref, host, dev)
            st = rb.stats()
            assert rb.ids() == ref.ids(), f"step {step}"
            assert (st.bytes_used, st.evicted, st.pushed) == (ref.used, ref.evicted, ref.next_id)
            if step % 7 == 3:
                _check_fetch(rb, ref, ref.ids()[int(r.integers(0, len(ref.ids())))])
        assert ref.evicted > 30
        for sid in ref.ids():
            _check_fetch(rb, ref, sid)


def test_replay_inputs_reusable_after_wait_pushed():
    host, dev = _sample(5, 1, 4, 700, 128, "bf16", 200, True)
    ref = O.ReplayBuffer(64 << 20)
    with ttr.ReplayBuffer(64 << 20, 64 << 20) as rb:
        sid = _push_both(rb, ref, host, dev)
        rb.wait_pushed()
        for t in dev.values():                    # overwritten on the current stream after the copies
            t.zero_()
        _check_fetch(rb, ref, sid)


def test_replay_refusals_and_evicted_ids():
    host, dev = _sample(9, 1, 2, 256, 64, "bf16", 64, True)
    foot = O.replay_sample_bytes(1, 2, 256, 64, 2, 64, True)
    lib = ttr.load_library()
    with ttr.ReplayBuffer(2 * foot, foot) as rb:
        ids = [rb.push(dev["Q"], dev["K"], dev["V"], host["idx"], dev["T"]) for _ in range(3)]
        assert ids == [0, 1, 2] and rb.ids() == [1, 2] and rb.stats().evicted == 1
        with pytest.raises(ttr.TTRError) as ei:
            rb.fetch(0)
        assert ei.value.status == 10
        with pytest.raises(ttr.TTRError) as ei:  # bigger than max_sample_bytes: nothing changes
            big = workloads.query_subsample(256, 200, 1)
            rb.push(dev["Q"], dev["K"], dev["V"], big, dev["T"])
        assert ei.value.status == 9 and rb.ids() == [1, 2]
        for bad in ([3, 3], [5, 2], [-1, 4], [0, 256]):
            with pytest.raises(ttr.TTRError) as ei:
                rb.push(dev["Q"], dev["K"], dev["V"], np.array(bad), dev["T"])
            assert ei.value.status == 2
        assert rb.ids() == [1, 2]
        # teacher rows asked of a sample pushed without them
        sid = rb.push(dev["Q"], dev["K"], dev["V"], host["idx"][:10], None)
        Qs = torch.empty(1, 2, 10, 64, dtype=torch.bfloat16, device=DEV)
        K = torch.empty(1, 2, 256, 64, dtype=torch.bfloat16, device=DEV)
        V, T = torch.empty_like(K), torch.empty(1, 2, 10, 64, device=DEV)
        st = lib.ttr_replay_fetch(rb._h, sid, Qs.data_ptr(), K.data_ptr(), V.data_ptr(), T.data_ptr(), None,
                                  torch.cuda.current_stream().cuda_stream)
        assert st == 2
        rb.synchronize()


def test_replay_fetch_on_two_streams_then_evict():
    # a sample fetched on two streams, then evicted at once by the next pushes:
    # the ring bytes are reused only after both fetches' copies have read them
    host, dev = _sample(21, 1, 8, 4096, 128, "bf16", 512, True)
    foot = O.replay_sample_bytes(1, 8, 4096, 128, 2, 512, True)
    ref = O.ReplayBuffer(2 * foot)
    with ttr.ReplayBuffer(2 * foot, foot) as rb:
        sid = _push_both(rb, ref, host, dev)
        smp = ref.fetch(sid)
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
        with torch.cuda.stream(sa):
            got_a = rb.fetch(sid)
        with torch.cuda.stream(sb):
            got_b = rb.fetch(sid)
        other, odev = _sample(22, 1, 8, 4096, 128, "bf16", 512, True)
        for _ in range(2):                        # the second push evicts the fetched sample
            _push_both(rb, ref, other, odev)
        assert sid not in rb.ids()
        torch.cuda.synchronize()
        for Qs, K, V, T, idx in (got_a, got_b):
            assert _same(_bits(K), smp["K"]) and _same(_bits(V), smp["V"])
            assert _same(_bits(Qs), smp["Q"]) and _same(_bits(T), smp["T"])
            assert np.array_equal(idx, smp["idx"])

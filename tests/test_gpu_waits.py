"""The kernels' inter-workgroup waits, forced from the host through the
library's test hooks (environment variables read at every launch):

* TTR_KVS_CROSS_XCD_ROUND=1: the key/value stage takes its cross-XCD round
  (each split writes its L2 back, counts in again, then drops stale lines)
  although all splits of a group share an XCD here. The result must be bit
  for bit that of the usual path.
* TTR_SPIN_LIMIT=1: every bounded wait gives up after one poll. The kernels
  must still finish, and a result is either the usual one bit for bit or
  visibly poisoned (NaN), never silently different; the causal scan also sets
  its error word. Without the hook the next call is clean again (the causal
  scan's reset launch clears its flags and error word; the key/value stage's
  meeting words carry the launch's number and are cleared by the group's last
  workgroup).
* The key/value stage needs no reset: a workspace full of arbitrary bytes
  gives the usual result bit for bit, and so do replays of a captured forward
  (each replay carries the same launch number).

Every kernel exits normally in all of these runs: only the waits are cut short."""
import numpy as np
import pytest
import torch

import linear_hybrid_attention_amd as ttr
import workloads
from _util import host, small, to_device

pytestmark = pytest.mark.gpu


def _forward(w, d):
    out = ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], d["g"], float(np.float32(w.eps)), w.L)
    torch.cuda.synchronize()
    return host(out)


def test_kv_stage_cross_xcd_round_is_bitwise_equal(monkeypatch):
    w = small("flux_1024", H=4, N=2000, L=64, seed=51)
    d = to_device(w, workloads.make_inputs(w))
    ref = _forward(w, d)
    kv_ref, ks_ref = ttr.kv_reduce(d["K"], d["V"], d["W"], d["b"])
    monkeypatch.setenv("TTR_KVS_CROSS_XCD_ROUND", "1")
    got = _forward(w, d)
    kv, ks = ttr.kv_reduce(d["K"], d["V"], d["W"], d["b"])
    torch.cuda.synchronize()
    assert np.array_equal(got, ref)
    assert torch.equal(kv, kv_ref) and torch.equal(ks, ks_ref)


def test_kv_stage_wait_timeout_is_visible(monkeypatch):
    w = small("flux_1024", H=4, N=3000, L=32, seed=52)
    d = to_device(w, workloads.make_inputs(w))
    ref = _forward(w, d)
    monkeypatch.setenv("TTR_SPIN_LIMIT", "1")
    for i in range(3):
        got = _forward(w, d)
        print(f"[waits] key/value stage, one poll per wait, run {i}: "
              f"{'NaN (gave up)' if np.isnan(got).any() else 'the usual result'}", flush=True)
        assert np.array_equal(got, ref) or np.isnan(got).any()
    monkeypatch.delenv("TTR_SPIN_LIMIT")
    assert np.array_equal(_forward(w, d), ref)


@pytest.mark.parametrize("fill", ["ones", "random"])
def test_kv_stage_any_workspace_contents(fill):
    w = small("flux_1024", H=5, N=3000, L=64, seed=54)
    d = to_device(w, workloads.make_inputs(w))
    eps = float(np.float32(w.eps))
    need = ttr.workspace_bytes(w.B, w.H, w.N, w.D, w.F, 1, w.L, False, 0)
    ref = host(ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], d["g"], eps, w.L))
    gen = torch.Generator(device="cpu").manual_seed(7)
    for i in range(3):
        if fill == "ones":
            ws = torch.full((need,), 255, dtype=torch.uint8, device=d["Q"].device)
        else:
            ws = torch.randint(0, 256, (need,), generator=gen, dtype=torch.uint8).to(d["Q"].device)
        got = host(ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], d["g"], eps, w.L, ws=ws))
        torch.cuda.synchronize()
        print(f"[waits] workspace filled with {fill} bytes, call {i}", flush=True)
        assert np.array_equal(got, ref)


def test_kv_stage_graph_replays():
    w = small("flux_1024", H=4, N=2500, L=64, seed=55)
    d = to_device(w, workloads.make_inputs(w))
    eps = float(np.float32(w.eps))
    need = ttr.workspace_bytes(w.B, w.H, w.N, w.D, w.F, 1, w.L, False, 0)
    ws = torch.empty(need, dtype=torch.uint8, device=d["Q"].device)
    out = torch.empty_like(d["Q"])
    ref = host(ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], d["g"], eps, w.L, ws=ws))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # (a warm-up on the capture stream)
        ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], d["g"], eps, w.L, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], d["g"], eps, w.L, out=out, ws=ws)
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[waits] graph replay {i}", flush=True)
        assert np.array_equal(host(out), ref)
        # eager calls between replays use new launch numbers on the same workspace
        again = host(ttr.hybrid_forward(d["Q"], d["K"], d["V"], d["W"], d["b"], d["g"], eps, w.L, ws=ws))
        assert np.array_equal(again, ref)


def _causal_plan(B, H, N, chunk):
    # segments as the library plans them: about 1024 tokens each, shorter when
    # that gives fewer than 512 workgroups; returns (segments, chunks per segment)
    nchunks = -(-N // chunk)
    want = max(-(-N // 1024), -(-512 // (B * H)))
    want = max(min(want, nchunks), 1)
    cps = -(-nchunks // want)
    return -(-nchunks // cps), cps


def _causal_err_word(ws, B, H, N, chunk):
    # the causal workspace's layout: inclusive prefixes [B H][nseg][64 64 + 64]
    # fp32, then flags [B H][nseg], the ticket and the error word
    nseg, _ = _causal_plan(B, H, N, chunk)
    off = B * H * nseg * (64 * 64 + 64) * 4 + B * H * nseg * 4 + 4
    return int(ws[off:off + 4].cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("chunk", [128, 256])
def test_causal_wait_timeout_sets_error(monkeypatch, chunk):
    w = small("causal", B=2, H=2, N=8192, D=64, F=64, seed=53)
    d = to_device(w, workloads.make_inputs(w))
    eps = float(np.float32(w.eps))
    need = ttr.workspace_bytes(w.B, w.H, w.N, w.D, w.F, 1, 0, True, chunk)
    ws = torch.empty(need, dtype=torch.uint8, device=d["Q"].device)
    ref = host(ttr.causal_scan(d["Q"], d["K"], d["V"], eps=eps, chunk=chunk, ws=ws))
    torch.cuda.synchronize()
    assert _causal_err_word(ws, w.B, w.H, w.N, chunk) == 0
    monkeypatch.setenv("TTR_SPIN_LIMIT", "1")
    got = host(ttr.causal_scan(d["Q"], d["K"], d["V"], eps=eps, chunk=chunk, ws=ws))
    torch.cuda.synchronize()
    err = _causal_err_word(ws, w.B, w.H, w.N, chunk)
    print(f"[waits] causal chunk {chunk}, one poll per wait: error word {err}, "
          f"{int(np.isnan(got).any(axis=-1).sum())} rows NaN", flush=True)
    if np.isnan(got).any():
        assert err == 1
    else:
        assert err == 0 and np.array_equal(got, ref)
    # the first segment of every sequence waits for nothing
    seg0 = min(w.N, _causal_plan(w.B, w.H, w.N, chunk)[1] * chunk)
    assert np.array_equal(got[:, :, :seg0], ref[:, :, :seg0])
    monkeypatch.delenv("TTR_SPIN_LIMIT")
    again = host(ttr.causal_scan(d["Q"], d["K"], d["V"], eps=eps, chunk=chunk, ws=ws))
    torch.cuda.synchronize()
    assert _causal_err_word(ws, w.B, w.H, w.N, chunk) == 0 and np.array_equal(again, ref)

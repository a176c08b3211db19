"""Pins for the fp64 oracle: checks against facts other than the oracle itself.

Each check is something the pages or the mathematics fix independently of
the oracle's own formulas: hand-worked values (tests/golden), brute-force
N x N attention, torch library routines in fp64, closed forms and
invariants. The mutation tests at the end plant plausible mistakes into the
oracle (on the CPU) and confirm some pin fails.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle.ttr_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = float(np.float32(1e-6))


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _small(seed=0, B=1, H=2, N=40, D=8, F=16, proj=True, bscale=0.1):
    r = np.random.default_rng(seed)
    Q = r.standard_normal((B, H, N, D))
    K = r.standard_normal((B, H, N, D))
    V = r.standard_normal((B, H, N, D))
    W = r.standard_normal((H, D, F)) / math.sqrt(D) if proj else None
    b = r.standard_normal((H, F if proj else D)) * bscale
    g = r.standard_normal(H)
    return Q, K, V, W, b, g


def _eval(expr):
    return float(eval(expr, {"e": math.e, "__builtins__": {}}))


def _golden_hand():
    rows = {}
    with open(os.path.join(GOLDEN, "hand_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, n, num, den = line.split()
            rows.setdefault(name, {})[int(n)] = _eval(num) / _eval(den)
    return {k: np.array([v[i] for i in sorted(v)]) for k, v in rows.items()}


HAND_X = np.array([0.0, 1.0, 3.0]).reshape(1, 1, 3, 1)
HAND_V = np.array([3.0, 6.0, -3.0]).reshape(1, 1, 3, 1)


TORCH_MAPS = {"elu1": lambda z: torch.nn.functional.elu(z, alpha=1.0) + 1.0,
              "relu": torch.relu,
              "softmax": lambda z: torch.softmax(z, dim=-1)}


def brute_linear(Q, K, V, W, b, eps, causal=False, kind="elu1"):
    """Row-normalised N x N form: A = phi(Q) phi(K)^T, out = A V / (A 1 + eps),
    with the feature maps taken from torch (fp64)."""
    B, H, N, D = Q.shape
    out = np.empty((B, H, N, V.shape[3]))
    for bi in range(B):
        for h in range(H):
            Wh = None if W is None else torch.from_numpy(W[h])
            def phi(x):
                t = torch.from_numpy(x)
                z = t @ Wh if Wh is not None else t
                if b is not None:
                    z = z + torch.from_numpy(b[h])
                return TORCH_MAPS[kind](z).numpy()
            A = phi(Q[bi, h]) @ phi(K[bi, h]).T
            if causal:
                A = A * np.tril(np.ones((N, N)))
            out[bi, h] = (A @ V[bi, h]) / (A.sum(axis=1, keepdims=True) + eps)
    return out


def sdpa(q, k, v):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()


# ---------------------------------------------------------------- feature map

def test_elu_plus_one_matches_torch_elu():
    z = np.linspace(-40.0, 40.0, 20001)
    ref = (torch.nn.functional.elu(torch.from_numpy(z), alpha=1.0) + 1.0).numpy()
    np.testing.assert_allclose(O.elu_plus_one(z), ref, rtol=1e-14, atol=2e-16)


def test_elu_plus_one_special_values():
    assert O.elu_plus_one(np.array([0.0]))[0] == 1.0
    z = np.linspace(-700, 700, 10001)
    p = O.elu_plus_one(z)
    assert (p > 0).all()
    assert (p[z >= 0] >= 1.0).all()
    assert (p[z < 0] < 1.0).all()
    np.testing.assert_allclose(p[z > 0], z[z > 0] + 1.0, rtol=0, atol=0)


def test_feature_map_hand_worked():
    xs, want = [], []
    with open(os.path.join(GOLDEN, "feature_map_hand.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, c = line.split("|")
            xs.append([float(t) for t in a.split()])
            want.append([_eval(t) for t in c.split()])
    X = np.array(xs).reshape(1, 1, -1, 2)
    W = np.array([[[1.0, 0.0], [0.0, -1.0]]])
    b = np.array([[0.0, 1.0]])
    np.testing.assert_allclose(O.feature_map(X, W, b)[0, 0], np.array(want), rtol=1e-15)


def test_feature_map_zero_projection_is_constant():
    Q, _, _, W, b, _ = _small(1)
    phi = O.feature_map(Q, np.zeros_like(W), b)
    want = (torch.nn.functional.elu(torch.from_numpy(b), alpha=1.0) + 1.0).numpy()
    np.testing.assert_allclose(phi[0], np.broadcast_to(want[:, None, :], phi[0].shape), rtol=1e-15)


def test_feature_map_identity_projection_equals_no_projection():
    Q, _, _, _, b, _ = _small(2, proj=False)
    D = Q.shape[3]
    eye = np.broadcast_to(np.eye(D), (Q.shape[1], D, D)).copy()
    np.testing.assert_allclose(O.feature_map(Q, eye, b), O.feature_map(Q, None, b), rtol=1e-15)


def test_feature_map_positive_on_config_scale():
    Q, _, _, W, b, _ = _small(3, N=512, D=64, F=256)
    assert (O.feature_map(Q, W, b) > 0).all()


# ---------------------------------------------------------------- linear branch

def test_linear_branch_matches_bruteforce_nxn():
    for seed, proj in ((4, True), (5, False)):
        Q, K, V, W, b, _ = _small(seed, proj=proj)
        KV, ksum = O.kv_reduce(K, V, W, b)
        got = O.apply(Q, W, b, KV, ksum, EPS)
        ref = brute_linear(Q, K, V, W, b, EPS)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_linear_branch_hand_worked():
    want = _golden_hand()
    KV, ksum = O.kv_reduce(HAND_X, HAND_V, None, None)
    assert KV.shape == (1, 1, 1, 1) and KV[0, 0, 0, 0] == 3.0 and ksum[0, 0, 0] == 7.0
    got = O.apply(HAND_X, None, None, KV, ksum, 1e-6)[0, 0, :, 0]
    np.testing.assert_allclose(got, want["lin"], rtol=1e-14)


def test_linear_branch_closed_form_constant_phi():
    # W = 0, b = 0 -> phi == 1 on all F features: out_n = F sum(V) / (F N + eps)
    Q, K, V, W, _, _ = _small(6)
    F = W.shape[2]
    N = Q.shape[2]
    KV, ksum = O.kv_reduce(K, V, np.zeros_like(W), None)
    got = O.apply(Q, np.zeros_like(W), None, KV, ksum, EPS)
    want = F * V.sum(axis=2, keepdims=True) / (F * N + EPS)
    np.testing.assert_allclose(got, np.broadcast_to(want, got.shape), rtol=1e-13)


def test_linear_branch_constant_values():
    # V == c -> out = c * den / (den + eps) with den = phi(q) . ksum
    Q, K, V, W, b, _ = _small(7)
    c = 1.75
    Vc = np.full_like(V, c)
    KV, ksum = O.kv_reduce(K, Vc, W, b)
    got = O.apply(Q, W, b, KV, ksum, 0.5)
    den = np.einsum("bhnf,bhf->bhn", O.feature_map(Q, W, b), ksum)
    np.testing.assert_allclose(got, np.broadcast_to((c * den / (den + 0.5))[..., None], got.shape), rtol=1e-13)


def test_linear_branch_invariants():
    Q, K, V, W, b, _ = _small(8)
    KV, ksum = O.kv_reduce(K, V, W, b)
    base = O.apply(Q, W, b, KV, ksum, EPS)
    perm = np.random.default_rng(0).permutation(K.shape[2])
    KV2, ks2 = O.kv_reduce(K[:, :, perm], V[:, :, perm], W, b)
    np.testing.assert_allclose(O.apply(Q, W, b, KV2, ks2, EPS), base, rtol=1e-12)
    # linear in V
    V2 = _rand(V.shape, 9)
    KVa, _ = O.kv_reduce(K, 2.0 * V - 3.0 * V2, W, b)
    KVb, _ = O.kv_reduce(K, V2, W, b)
    lhs = O.apply(Q, W, b, KVa, ksum, EPS)
    rhs = 2.0 * base - 3.0 * O.apply(Q, W, b, KVb, ksum, EPS)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-10, atol=1e-12)
    # convex hull of {0} and the values (weights are positive and sum below 1)
    lo = np.minimum(0.0, V.min(axis=2, keepdims=True))
    hi = np.maximum(0.0, V.max(axis=2, keepdims=True))
    assert (base >= lo - 1e-12).all() and (base <= hi + 1e-12).all()


def test_kv_reduce_shapes_and_ksum():
    Q, K, V, W, b, _ = _small(10, F=32)
    KV, ksum = O.kv_reduce(K, V, W, b)
    assert KV.shape == (1, 2, 32, 8) and ksum.shape == (1, 2, 32)
    # ksum equals KV against an all-ones value column
    ones = np.ones(V.shape[:3] + (1,))
    KV1, _ = O.kv_reduce(K, ones, W, b)
    np.testing.assert_allclose(KV1[..., 0], ksum, rtol=1e-14)


# ---------------------------------------------------------------- landmarks

def test_landmark_indices_golden():
    with open(os.path.join(GOLDEN, "landmarks_tiny.txt")) as f:
        lines = [l for l in f.read().splitlines() if l and not l.startswith("#")]
    N, L = map(int, lines[0].split())
    want = [int(t) for t in lines[1].split()]
    assert O.landmark_indices(N, L).tolist() == want


@pytest.mark.parametrize("N,L", [(1536, 64), (4608, 128), (16896, 256), (257, 16), (1000, 7), (5, 5), (9, 1)])
def test_landmark_indices_properties(N, L):
    idx = O.landmark_indices(N, L)
    assert idx[0] == 0 and len(idx) == L
    assert (np.diff(idx) > 0).all() and idx[-1] < N
    if N % L == 0:
        assert (np.diff(idx) == N // L).all()
    if L == N:
        assert idx.tolist() == list(range(N))


def test_landmark_single_landmark_returns_first_value():
    Q, K, V, _, _, _ = _small(11)
    got = O.landmark_attn(Q, K, V, 1)
    np.testing.assert_allclose(got, np.broadcast_to(V[:, :, :1, :], got.shape), rtol=1e-15)


def test_landmark_zero_query_is_mean():
    Q, K, V, _, _, _ = _small(12)
    L = 8
    idx = O.landmark_indices(Q.shape[2], L)
    got = O.landmark_attn(np.zeros_like(Q), K, V, L)
    want = V[:, :, idx, :].mean(axis=2, keepdims=True)
    np.testing.assert_allclose(got, np.broadcast_to(want, got.shape), rtol=1e-13)


def test_landmark_matches_torch_sdpa_on_gathered():
    Q, K, V, _, _, _ = _small(13, D=16)
    Q = Q * 3.0  # spread the scores so the softmax is far from uniform
    L = 10
    idx = O.landmark_indices(Q.shape[2], L)
    ref = sdpa(Q, K[:, :, idx], V[:, :, idx])
    np.testing.assert_allclose(O.landmark_attn(Q, K, V, L), ref, rtol=1e-12, atol=1e-14)


def test_landmark_hand_worked():
    want = _golden_hand()
    np.testing.assert_allclose(O.landmark_attn(HAND_X, HAND_X, HAND_V, 1)[0, 0, :, 0], want["lm1"], rtol=1e-15)
    np.testing.assert_allclose(O.landmark_attn(HAND_X, HAND_X, HAND_V, 3)[0, 0, :, 0], want["lm3"], rtol=1e-13)


def test_landmark_shift_invariance():
    Q, K, V, _, _, _ = _small(14)
    base = O.landmark_attn(Q, K, V, 8)
    # adding a vector orthogonal... use a per-query constant: scores shift by q . c for all landmarks
    # when every landmark key moves by the same c, the softmax is unchanged
    c = _rand((1, 1, 1, Q.shape[3]), 15)
    np.testing.assert_allclose(O.landmark_attn(Q, K + c, V, 8), base, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- blend and hybrid

def test_blend_limits_and_direction():
    Q, K, V, W, b, _ = _small(16)
    KV, ksum = O.kv_reduce(K, V, W, b)
    lin = O.apply(Q, W, b, KV, ksum, EPS)
    lm = O.landmark_attn(Q, K, V, 8)
    H = Q.shape[1]
    np.testing.assert_array_equal(O.blend(lin, lm, np.full(H, np.inf)), lin)
    np.testing.assert_array_equal(O.blend(lin, lm, np.full(H, -np.inf)), lm)
    np.testing.assert_allclose(O.blend(lin, lm, np.zeros(H)), 0.5 * (lin + lm), rtol=1e-15)
    # g = ln 3 -> alpha = 3/4 on the linear branch
    np.testing.assert_allclose(O.blend(lin, lm, np.full(H, math.log(3.0))), 0.75 * lin + 0.25 * lm, rtol=1e-14)


def test_hybrid_hand_worked():
    want = _golden_hand()
    g = np.array([math.log(3.0)])
    got = O.hybrid_forward(HAND_X, HAND_X, HAND_V, None, None, g, 1e-6, 3)[0, 0, :, 0]
    np.testing.assert_allclose(got, 0.75 * want["lin"] + 0.25 * want["lm3"], rtol=1e-13)


def test_hybrid_alpha_zero_all_landmarks_is_full_softmax():
    Q, K, V, W, b, _ = _small(17, N=48, D=16)
    H = Q.shape[1]
    got = O.hybrid_forward(Q, K, V, W, b, np.full(H, -np.inf), EPS, Q.shape[2])
    np.testing.assert_allclose(got, sdpa(Q, K, V), rtol=1e-12, atol=1e-14)


def test_hybrid_alpha_zero_is_landmark_softmax():
    Q, K, V, W, b, _ = _small(18, N=64, D=16)
    H = Q.shape[1]
    idx = O.landmark_indices(64, 16)
    got = O.hybrid_forward(Q, K, V, W, b, np.full(H, -np.inf), EPS, 16)
    np.testing.assert_allclose(got, sdpa(Q, K[:, :, idx], V[:, :, idx]), rtol=1e-12, atol=1e-14)


def test_hybrid_no_landmarks_is_linear():
    Q, K, V, W, b, g = _small(19)
    got = O.hybrid_forward(Q, K, V, W, b, g, EPS, 0)
    np.testing.assert_allclose(got, brute_linear(Q, K, V, W, b, EPS), rtol=1e-11, atol=1e-13)


def test_hybrid_rows_match_full():
    Q, K, V, W, b, g = _small(20, B=2, N=50)
    full = O.hybrid_forward(Q, K, V, W, b, g, EPS, 5)
    rows = [(0, 0, 0), (1, 1, 49), (0, 1, 17), (1, 0, 33)]
    got = O.hybrid_rows(Q, K, V, W, b, g, EPS, 5, rows)
    np.testing.assert_allclose(got, np.stack([full[r] for r in rows]), rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- causal

def test_causal_hand_worked():
    want = _golden_hand()
    got = O.causal_forward(HAND_X, HAND_X, HAND_V, None, None, 1e-6)[0, 0, :, 0]
    np.testing.assert_allclose(got, want["causal"], rtol=1e-14)


def test_causal_matches_masked_bruteforce():
    for seed, proj in ((21, False), (22, True)):
        Q, K, V, W, b, _ = _small(seed, B=2, N=33, proj=proj)
        got = O.causal_forward(Q, K, V, W, b, EPS)
        ref = brute_linear(Q, K, V, W, b, EPS, causal=True)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_causal_first_token_closed_form():
    Q, K, V, _, b, _ = _small(23, proj=False)
    got = O.causal_forward(Q, K, V, None, b, EPS)[:, :, 0, :]
    phiq = O.elu_plus_one(Q[:, :, 0, :] + b[None])
    phik = O.elu_plus_one(K[:, :, 0, :] + b[None])
    a = (phiq * phik).sum(-1, keepdims=True)
    np.testing.assert_allclose(got, V[:, :, 0, :] * a / (a + EPS), rtol=1e-13)


def test_causal_last_token_equals_noncausal():
    Q, K, V, _, b, _ = _small(24, N=70, proj=False)
    c = O.causal_forward(Q, K, V, None, b, EPS)
    KV, ksum = O.kv_reduce(K, V, None, b)
    nc = O.apply(Q, None, b, KV, ksum, EPS)
    np.testing.assert_allclose(c[:, :, -1], nc[:, :, -1], rtol=1e-12)


def test_causal_rows_match_full():
    Q, K, V, _, _, _ = _small(25, B=2, N=40, proj=False)
    full = O.causal_forward(Q, K, V, None, None, EPS)
    rows = [(0, 0, 0), (1, 1, 39), (0, 1, 20)]
    np.testing.assert_allclose(O.causal_rows(Q, K, V, None, None, EPS, rows),
                               np.stack([full[r] for r in rows]), rtol=1e-11)


def test_normwise_err():
    ref = np.zeros((2, 3, 4, 5))
    ref[0, 0] = 2.0
    ref[1, 2] = 4.0
    got = ref.copy()
    got[1, 2, 0, 0] += 0.4
    assert O.normwise_err(got, ref) == pytest.approx(0.1)


# ---------------------------------------------------------------- relu and softmax feature maps

def test_relu_map_values():
    z = np.array([-2.0, -0.0, 0.0, 1e-300, 3.5])
    np.testing.assert_array_equal(O.relu_map(z), [0.0, 0.0, 0.0, 1e-300, 3.5])
    Q, _, _, W, b, _ = _small(40)
    assert (O.feature_map(Q, W, b, "relu") >= 0.0).all()


def test_softmax_map_hand_worked_and_invariants():
    # softmax([0, ln 3]) = [1/4, 3/4]; rows sum to 1; adding a constant to a
    # token's features changes nothing
    np.testing.assert_allclose(O.softmax_map(np.array([[0.0, math.log(3.0)]])), [[0.25, 0.75]], rtol=1e-15)
    Q, _, _, _, b, _ = _small(41, proj=False)
    phi = O.feature_map(Q, None, b, "softmax")
    np.testing.assert_allclose(phi.sum(-1), 1.0, rtol=1e-14)
    shifted = O.feature_map(Q + 7.25, None, b, "softmax")
    np.testing.assert_allclose(shifted, phi, rtol=1e-12)
    assert (phi > 0).all()


def test_softmax_map_matches_torch():
    Q, _, _, W, b, _ = _small(42)
    got = O.feature_map(Q, W, b, "softmax")
    z = torch.from_numpy(Q) @ torch.from_numpy(W)[None] + torch.from_numpy(b)[None, :, None, :]
    np.testing.assert_allclose(got, torch.softmax(z, dim=-1).numpy(), rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("kind", ["relu", "softmax"])
def test_other_maps_linear_and_causal_match_bruteforce(kind):
    for seed, proj in ((43, False), (44, True)):
        Q, K, V, W, b, _ = _small(seed, B=2, N=33, proj=proj)
        KV, ksum = O.kv_reduce(K, V, W, b, kind)
        got = O.apply(Q, W, b, KV, ksum, EPS, kind)
        np.testing.assert_allclose(got, brute_linear(Q, K, V, W, b, EPS, kind=kind), rtol=1e-10, atol=1e-12)
        got = O.causal_forward(Q, K, V, W, b, EPS, kind)
        np.testing.assert_allclose(got, brute_linear(Q, K, V, W, b, EPS, causal=True, kind=kind),
                                   rtol=1e-10, atol=1e-12)
        assert np.allclose(O.hybrid_forward(Q, K, V, W, b, None, EPS, 0, kind), O.apply(Q, W, b, KV, ksum, EPS, kind))


@pytest.mark.parametrize("kind", ["relu", "softmax"])
def test_other_maps_last_causal_token_and_rows(kind):
    Q, K, V, _, b, _ = _small(45, N=50, proj=False)
    c = O.causal_forward(Q, K, V, None, b, EPS, kind)
    KV, ksum = O.kv_reduce(K, V, None, b, kind)
    nc = O.apply(Q, None, b, KV, ksum, EPS, kind)
    np.testing.assert_allclose(c[:, :, -1], nc[:, :, -1], rtol=1e-11)
    rows = [(0, 0, 0), (0, 1, 17), (0, 1, 49)]
    np.testing.assert_allclose(O.causal_rows(Q, K, V, None, b, EPS, rows, kind),
                               np.stack([c[r] for r in rows]), rtol=1e-11)
    np.testing.assert_allclose(O.hybrid_rows(Q, K, V, None, b, None, EPS, 0, rows, kind),
                               np.stack([nc[r] for r in rows]), rtol=1e-11)


def test_relu_map_all_negative_keys_give_zero():
    # every key feature negative -> phi(K) = 0 -> KV = 0, ksum = 0 -> out = 0 / (0 + eps) = 0
    Q, K, V, _, _, _ = _small(46, proj=False)
    KV, ksum = O.kv_reduce(-np.abs(K) - 0.1, V, None, None, "relu")
    assert not KV.any() and not ksum.any()
    assert not O.apply(Q, None, None, KV, ksum, EPS, "relu").any()


# ---------------------------------------------------------------- NNT layer (in/out projections)

def _layer_params(seed, B=2, N=24, E=32, H=4, bias=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, N, E))
    Ws = [r.standard_normal((E, E)) / math.sqrt(E) for _ in range(4)]
    bs = [r.standard_normal(E) * 0.1 if bias else None for _ in range(4)]
    return x, Ws, bs


def brute_layer(x, Ws, bs, H, eps, causal=False, kind="elu1"):
    """The layer restated in torch (fp64): heads as column slices of the
    projections, attention in the N x N row-normalised form."""
    X = torch.from_numpy(x)

    def lin(inp, W, b):
        y = inp @ torch.from_numpy(W)
        return y if b is None else y + torch.from_numpy(b)

    q, k, v = (lin(X, W, b) for W, b in zip(Ws[:3], bs[:3]))
    B, N, E = x.shape
    D = E // H
    heads = torch.empty(B, N, E, dtype=torch.float64)
    for h in range(H):
        sl = slice(h * D, (h + 1) * D)
        A = TORCH_MAPS[kind](q[..., sl]) @ TORCH_MAPS[kind](k[..., sl]).transpose(-1, -2)
        if causal:
            A = A * torch.tril(torch.ones(N, N, dtype=torch.float64))
        heads[..., sl] = (A @ v[..., sl]) / (A.sum(-1, keepdim=True) + eps)
    return lin(heads, Ws[3], bs[3]).numpy()


def _layer(x, Ws, bs, H, causal=False, kind="elu1"):
    return O.nnt_layer_forward(x, Ws[0], bs[0], Ws[1], bs[1], Ws[2], bs[2], Ws[3], bs[3], H, EPS, causal, kind)


@pytest.mark.parametrize("kind", ["elu1", "relu", "softmax"])
@pytest.mark.parametrize("causal", [False, True])
def test_nnt_layer_matches_bruteforce(kind, causal):
    x, Ws, bs = _layer_params(70)
    got = _layer(x, Ws, bs, 4, causal, kind)
    ref = brute_layer(x, Ws, bs, 4, EPS, causal, kind)
    assert got.shape == x.shape
    assert np.abs(got - ref).max() < 1e-11 * max(1.0, np.abs(ref).max())


def test_nnt_layer_no_bias_matches_bruteforce():
    x, Ws, bs = _layer_params(71, B=1, N=17, E=48, H=3, bias=False)
    assert np.abs(_layer(x, Ws, bs, 3) - brute_layer(x, Ws, bs, 3, EPS)).max() < 1e-11


@pytest.mark.parametrize("causal", [False, True])
def test_nnt_layer_zero_query_key_projection_closed_form(causal):
    # phi(0) = 1 for elu + 1, so every score is D: each head returns
    # D * sum(v) / (D * count + eps) over the visible keys.
    x, Ws, bs = _layer_params(72, B=1, N=9, E=16, H=2)
    Ws[0] = np.zeros_like(Ws[0])
    Ws[1] = np.zeros_like(Ws[1])
    bs[0] = np.zeros_like(bs[0])
    bs[1] = np.zeros_like(bs[1])
    D = 8
    v = x[0] @ Ws[2] + bs[2]
    cnt = np.arange(1, 10)[:, None] if causal else np.full((9, 1), 9.0)
    sums = np.cumsum(v, axis=0) if causal else np.repeat(v.sum(axis=0, keepdims=True), 9, axis=0)
    heads = D * sums / (D * cnt + EPS)
    want = heads @ Ws[3] + bs[3]
    assert np.abs(_layer(x, Ws, bs, 2, causal)[0] - want).max() < 1e-12


def test_nnt_layer_head_permutation_invariance():
    x, Ws, bs = _layer_params(73, E=32, H=4)
    perm = [2, 0, 3, 1]
    D = 8
    cols = np.concatenate([np.arange(h * D, (h + 1) * D) for h in perm])
    Wp = [W[:, cols] for W in Ws[:3]] + [Ws[3][cols, :]]
    bp = [b[cols] for b in bs[:3]] + [bs[3]]
    assert np.abs(_layer(x, Ws, bs, 4) - _layer(x, Wp, bp, 4)).max() < 1e-12


# ---------------------------------------------------------------- backward and distillation

def _bw_small(seed=80, B=2, H=2, N=24, D=4, F=8, L=6):
    Q, K, V, W, b, g = _small(seed, B=B, H=H, N=N, D=D, F=F)
    dout = np.random.default_rng(seed + 1).standard_normal(Q.shape)
    return Q, K, V, W, b, g, L, dout


def _fd(f, x, idx, h=1e-6):
    xp, xm = x.copy(), x.copy()
    xp[idx] += h
    xm[idx] -= h
    return (f(xp) - f(xm)) / (2 * h)


def test_backward_matches_finite_differences():
    Q, K, V, W, b, g, L, dout = _bw_small()
    dW, db, dg = O.hybrid_backward(Q, K, V, W, b, g, EPS, L, dout)
    obj = lambda W_, b_, g_: float((dout * O.hybrid_forward(Q, K, V, W_, b_, g_, EPS, L)).sum())
    r = np.random.default_rng(3)
    for _ in range(12):
        idx = tuple(int(r.integers(n)) for n in W.shape)
        assert abs(_fd(lambda x: obj(x, b, g), W, idx) - dW[idx]) < 1e-6 * max(1.0, abs(dW[idx]))
    for h in range(b.shape[0]):
        for f in (0, 3, 7):
            assert abs(_fd(lambda x: obj(W, x, g), b, (h, f)) - db[h, f]) < 1e-6 * max(1.0, abs(db[h, f]))
    for h in range(g.shape[0]):
        assert abs(_fd(lambda x: obj(W, b, x), g, (h,)) - dg[h]) < 1e-6 * max(1.0, abs(dg[h]))


def _torch_hybrid(Q, K, V, W, b, g, eps, L):
    """The forward restated in torch (fp64, differentiable): N x N linear form,
    softmax over the gathered landmarks, sigmoid blend."""
    Qt, Kt, Vt = (torch.from_numpy(a) for a in (Q, K, V))
    B, H, N, D = Q.shape
    idx = torch.tensor([(j * N) // L for j in range(L)])
    outs = []
    for h in range(H):
        pq = torch.nn.functional.elu(Qt[:, h] @ W[h] + b[h]) + 1
        pk = torch.nn.functional.elu(Kt[:, h] @ W[h] + b[h]) + 1
        A = pq @ pk.transpose(-1, -2)
        lin = (A @ Vt[:, h]) / (A.sum(-1, keepdim=True) + eps)
        S = (Qt[:, h] @ Kt[:, h, idx].transpose(-1, -2)) / math.sqrt(D)
        lm = torch.softmax(S, dim=-1) @ Vt[:, h, idx]
        a = torch.sigmoid(g[h])
        outs.append(a * lin + (1 - a) * lm)
    return torch.stack(outs, dim=1)


def test_backward_matches_torch_autograd():
    Q, K, V, W, b, g, L, dout = _bw_small(81, B=2, H=3, N=30, D=5, F=7, L=5)
    Wt, bt, gt = (torch.tensor(a, requires_grad=True) for a in (W, b, g))
    (torch.from_numpy(dout) * _torch_hybrid(Q, K, V, Wt, bt, gt, EPS, L)).sum().backward()
    dW, db, dg = O.hybrid_backward(Q, K, V, W, b, g, EPS, L, dout)
    for mine, ref in ((dW, Wt.grad), (db, bt.grad), (dg, gt.grad)):
        assert np.abs(mine - ref.numpy()).max() < 1e-10 * max(1.0, np.abs(ref.numpy()).max())


def test_backward_without_landmarks_has_no_g_gradient():
    Q, K, V, W, b, g, _, dout = _bw_small(82)
    dW, db, dg = O.hybrid_backward(Q, K, V, W, b, g, EPS, 0, dout)
    assert not dg.any()
    obj = lambda W_: float((dout * O.hybrid_forward(Q, K, V, W_, b, g, EPS, 0)).sum())
    assert abs(_fd(obj, W, (1, 2, 3)) - dW[1, 2, 3]) < 1e-6 * max(1.0, abs(dW[1, 2, 3]))


def test_elu_plus_one_grad():
    z = np.array([-3.0, -1e-3, 0.0, 1e-3, 2.0])
    want = np.array([math.exp(-3.0), math.exp(-1e-3), 1.0, 1.0, 1.0])
    assert np.abs(O.elu_plus_one_grad(z) - want).max() < 1e-15


def test_full_softmax_attention_matches_sdpa():
    Q, K, V, _, _, _ = _small(83, B=2, H=2, N=33, D=8)
    assert np.abs(O.full_softmax_attention(Q, K, V) - sdpa(Q, K, V)).max() < 1e-12


def test_distill_loss_matches_torch():
    r = np.random.default_rng(84)
    o = r.standard_normal((2, 3, 10, 6)) * 1.5
    t = r.standard_normal((2, 3, 10, 6))
    o[0, 0, 0] = 0.0  # a zero row: cos is 0 there and its gradient is t / 1e-8 . 0
    s = np.array([0.3, -0.2])
    loss, dout, ds, H, C = O.distill_loss(o, t, s)
    ot = torch.tensor(o, requires_grad=True)
    st = torch.tensor(s, requires_grad=True)
    Ht = torch.nn.functional.huber_loss(ot, torch.from_numpy(t), delta=1.0)
    Ct = (1 - torch.nn.functional.cosine_similarity(ot, torch.from_numpy(t), dim=-1, eps=1e-8)).mean()
    Lt = torch.exp(-st[0]) * Ht + st[0] + torch.exp(-st[1]) * Ct + st[1]
    Lt.backward()
    assert abs(H - Ht.item()) < 1e-12 and abs(C - Ct.item()) < 1e-12 and abs(loss - Lt.item()) < 1e-12
    assert np.abs(dout[:, :, 1:] - ot.grad.numpy()[:, :, 1:]).max() < 1e-12
    assert np.abs(ds - st.grad.numpy()).max() < 1e-12


def test_adam_matches_torch_optim():
    r = np.random.default_rng(85)
    p0 = r.standard_normal(7)
    grads = [r.standard_normal(7) for _ in range(5)]
    pt = torch.tensor(p0, requires_grad=True)
    opt = torch.optim.Adam([pt], lr=3e-3, betas=(0.9, 0.999), eps=1e-8)
    p, m, v = p0.copy(), np.zeros(7), np.zeros(7)
    for k, gr in enumerate(grads, start=1):
        opt.zero_grad()
        pt.grad = torch.from_numpy(gr.copy())
        opt.step()
        p, m, v = O.adam_update(p, gr, m, v, k, 3e-3)
    assert np.abs(p - pt.detach().numpy()).max() < 1e-14


def _adam_state(W, b, g, s):
    z = np.zeros_like
    return {"mW": z(W), "vW": z(W), "mb": z(b), "vb": z(b), "mg": z(g), "vg": z(g), "ms": z(s), "vs": z(s)}


def test_distill_step_self_teacher_moves_only_log_variances():
    Q, K, V, W, b, g, L, _ = _bw_small(86)
    s = np.zeros(2)
    T = O.hybrid_forward(Q, K, V, W, b, g, EPS, L)
    W2, b2, g2, s2, _, loss = O.distill_step(Q, K, V, W, b, g, s, _adam_state(W, b, g, s), 1, 1e-2, EPS, L, T)
    assert abs(loss) < 1e-12  # huber 0, cos 1 everywhere, s = 0
    # the gradient is zero up to rounding (cos = 1 - ulp), which Adam's eps turns into < 1e-9 steps
    assert np.abs(W2 - W).max() < 1e-9 and np.abs(b2 - b).max() < 1e-9 and np.abs(g2 - g).max() < 1e-9
    assert np.all(s2 < 0)  # d loss / d s = 1 - exp(-s) * 0 = 1 > 0 pushes s down


def test_distill_step_matches_torch_autograd_and_adam():
    # three whole steps against an independent composition: the forward restated
    # in torch, the teacher from SDPA, huber and cosine from torch, gradients by
    # autograd and the update by torch.optim.Adam (one optimiser over W, b, g, s)
    Q, K, V, W, b, g, L, _ = _bw_small(88, B=1, H=2, N=24, D=6, F=8, L=6)
    s = np.array([0.1, -0.2])
    lr = 5e-3
    Wt, bt, gt, stt = (torch.tensor(a.copy(), requires_grad=True) for a in (W, b, g, s))
    opt = torch.optim.Adam([Wt, bt, gt, stt], lr=lr, betas=(0.9, 0.999), eps=1e-8)
    T = torch.nn.functional.scaled_dot_product_attention(*(torch.from_numpy(a) for a in (Q, K, V)))
    st = _adam_state(W, b, g, s)
    for k in range(1, 4):
        W, b, g, s, st, loss = O.distill_step(Q, K, V, W, b, g, s, st, k, lr, EPS, L)
        opt.zero_grad()
        out = _torch_hybrid(Q, K, V, Wt, bt, gt, EPS, L)
        Ht = torch.nn.functional.huber_loss(out, T, delta=1.0)
        Ct = (1 - torch.nn.functional.cosine_similarity(out, T, dim=-1, eps=1e-8)).mean()
        Lt = torch.exp(-stt[0]) * Ht + stt[0] + torch.exp(-stt[1]) * Ct + stt[1]
        Lt.backward()
        opt.step()
        assert abs(loss - Lt.item()) < 1e-10 * max(1.0, abs(Lt.item()))
        for mine, ref in ((W, Wt), (b, bt), (g, gt), (s, stt)):
            assert np.abs(mine - ref.detach().numpy()).max() < 1e-10


def test_distill_steps_reduce_the_loss():
    Q, K, V, W, b, g, L, _ = _bw_small(87, B=1, H=2, N=32, D=8, F=16, L=8)
    s = np.zeros(2)
    st = _adam_state(W, b, g, s)
    T = O.full_softmax_attention(Q, K, V)
    losses = []
    for k in range(1, 31):
        W, b, g, s, st, loss = O.distill_step(Q, K, V, W, b, g, s, st, k, 1e-2, EPS, L, T)
        losses.append(loss)
    assert losses[-1] < losses[0] - 0.05


# ---------------------------------------------------------------- readiness gating

def test_cosine_distance_matches_torch():
    r = np.random.default_rng(90)
    o, t = r.standard_normal((2, 3, 11, 8)), r.standard_normal((2, 3, 11, 8))
    ref = (1 - torch.nn.functional.cosine_similarity(torch.from_numpy(o), torch.from_numpy(t), dim=-1,
                                                     eps=1e-8)).mean().item()
    assert abs(O.cosine_distance(o, t) - ref) < 1e-14
    assert abs(O.cosine_distance(t, t)) < 1e-14 and abs(O.cosine_distance(-t, t) - 2.0) < 1e-14
    assert abs(O.cosine_distance(3.0 * t, t)) < 1e-14  # scale invariant


def test_landmark_count_hand_worked():
    assert O.landmark_count(4608, 1 / 36, 16, 512) == 128
    assert O.landmark_count(1536, 1 / 24, 16, 512) == 64
    assert O.landmark_count(100, 0.005, 16, 512) == 16      # min clamp (0.5 rounds up to 1, then 16)
    assert O.landmark_count(100000, 0.1, 16, 512) == 512    # max clamp
    assert O.landmark_count(10, 0.5, 16, 512) == 10         # never more than N
    assert O.landmark_count(30, 0.05, 0, 512) == 2          # 1.5 rounds half up


def test_gate_fails_closed_until_min_updates():
    g = O.ReadinessGate(0.9, 0.1, 0.2, 5)
    assert [g.update(0.0) for _ in range(5)] == [False, False, False, False, True]


def test_gate_ema_hand_worked():
    g = O.ReadinessGate(0.5, 0.1, 0.2, 1)
    g.update(0.4)
    assert g.ema == 0.4 and not g.ready
    g.update(0.0)                         # 0.5 * 0.4 + 0.5 * 0 = 0.2
    assert abs(g.ema - 0.2) < 1e-15 and not g.ready
    g.update(0.0)                         # 0.1 <= on: ready
    assert abs(g.ema - 0.1) < 1e-15 and g.ready
    g.update(0.3)                         # 0.2: inside the band, stays ready
    assert abs(g.ema - 0.2) < 1e-15 and g.ready
    g.update(0.3)                         # 0.25 > off: drops
    assert abs(g.ema - 0.25) < 1e-15 and not g.ready
    g.update(0.05)                        # 0.15: inside the band, stays down
    assert not g.ready


def test_gate_hysteresis_does_not_flap():
    g = O.ReadinessGate(0.0, 0.1, 0.2, 1)  # rate 0: ema = the last distance
    states = [g.update(d) for d in (0.05, 0.15, 0.12, 0.18, 0.21, 0.15, 0.11, 0.09)]
    assert states == [True, True, True, True, False, False, False, True]


def test_gate_non_finite_distance_fails_closed():
    g = O.ReadinessGate(0.9, 0.1, 0.2, 1)
    assert g.update(0.0) and not g.update(float("nan")) and g.updates == 1


# ---------------------------------------------------------------- replay buffer

def test_replay_footprint_hand_worked():
    # bf16 [1,2,10,64]: K and V 2560 B each; 3 query rows 768 B; fp32 teacher
    # rows 1536 B; 3 int32 indices 12 B -> one 256-byte unit
    assert O.replay_sample_bytes(1, 2, 10, 64, 2, 3, True) == 2560 + 2560 + 768 + 1536 + 256
    # fp32 [2,3,5,64], every token kept, no teacher: 3 x 7680 + 256
    assert O.replay_sample_bytes(2, 3, 5, 64, 4, 5, False) == 23296
    assert O.replay_part_bytes(0) == 0 and O.replay_part_bytes(1) == 256 and O.replay_part_bytes(257) == 512


def _replay_sample(rng, N, Nq, D=64, B=1, H=2, teacher=True):
    Q, K, V = (rng.standard_normal((B, H, N, D)).astype(np.float32) for _ in range(3))
    T = rng.standard_normal((B, H, N, D)).astype(np.float32) if teacher else None
    idx = np.sort(rng.choice(N, size=Nq, replace=False)).astype(np.int32)
    return Q, K, V, idx, T


def _longest_fitting_suffix(history, budget):
    """Brute force: the most recent pushes whose footprints fit, longest first."""
    for k in range(len(history), -1, -1):
        tail = history[len(history) - k:]
        if sum(f for _, f in tail) <= budget:
            return [i for i, _ in tail]
    return []


def test_replay_holds_longest_fitting_suffix():
    rng = np.random.default_rng(31)
    budget = 200_000
    rb = O.ReplayBuffer(budget)
    history = []
    for _ in range(40):
        N = int(rng.integers(8, 120))
        Nq = int(rng.integers(1, N + 1))
        Q, K, V, idx, T = _replay_sample(rng, N, Nq, teacher=bool(rng.integers(0, 2)))
        foot = O.replay_sample_bytes(1, 2, N, 64, 4, Nq, T is not None)
        sid = rb.push(Q, K, V, idx, T)
        if foot > budget:
            assert sid is None
            continue
        history.append((sid, foot))
        assert rb.ids() == _longest_fitting_suffix(history, budget)
        assert rb.used <= budget and rb.ids()[-1] == sid
    assert rb.evicted > 0 and len(history) > len(rb.ids())


def test_replay_stores_gathered_query_rows():
    rng = np.random.default_rng(5)
    Q, K, V, idx, T = _replay_sample(rng, 37, 9)
    rb = O.ReplayBuffer(1 << 20)
    sid = rb.push(Q, K, V, idx, T)
    Q0, K0 = Q.copy(), K.copy()
    Q[...] = 0.0                                 # the sample is a copy taken at push time
    K[...] = 0.0
    smp = rb.fetch(sid)
    for b in range(Q.shape[0]):
        for h in range(Q.shape[1]):
            for j, n in enumerate(idx):
                assert np.array_equal(smp["Q"][b, h, j], Q0[b, h, n])
                assert np.array_equal(smp["T"][b, h, j], T[b, h, n])
    assert np.array_equal(smp["K"], K0) and np.array_equal(smp["V"], V) and np.array_equal(smp["idx"], idx)


def test_replay_refuses_sample_above_budget():
    rng = np.random.default_rng(2)
    Q, K, V, idx, T = _replay_sample(rng, 16, 4)
    foot = O.replay_sample_bytes(1, 2, 16, 64, 4, 4, True)
    rb = O.ReplayBuffer(foot)                    # exactly one sample fits
    assert rb.push(Q, K, V, idx, T) == 0
    assert rb.push(Q, K, V, idx, T) == 1 and rb.ids() == [1] and rb.evicted == 1
    small = O.ReplayBuffer(foot - 1)
    assert small.push(Q, K, V, idx, T) is None and small.ids() == [] and small.next_id == 0
    with pytest.raises(KeyError):
        small.fetch(0)


@pytest.mark.parametrize("bad", [[3, 3], [5, 2], [-1, 4], [0, 16]])
def test_replay_rejects_bad_indices(bad):
    rng = np.random.default_rng(3)
    Q, K, V, _, T = _replay_sample(rng, 16, 4)
    with pytest.raises(ValueError):
        O.ReplayBuffer(1 << 20).push(Q, K, V, np.array(bad), T)


# ---------------------------------------------------------------- sampled query rows

def _sampled_case(seed=91, B=2, H=2, N=40, D=6, F=9, L=7, Nq=13):
    r = np.random.default_rng(seed)
    Q, K, V = (r.standard_normal((B, H, N, D)) for _ in range(3))
    W = r.standard_normal((H, D, F)) / math.sqrt(D)
    b = r.standard_normal((H, F)) * 0.1
    g = r.standard_normal(H)
    idx = np.sort(r.choice(N, size=Nq, replace=False))
    return Q, K, V, W, b, g, L, idx


def test_sampled_rows_forward_equals_rows_of_full_forward():
    Q, K, V, W, b, g, L, idx = _sampled_case()
    full = O.hybrid_forward(Q, K, V, W, b, g, EPS, L)
    rows = O.hybrid_forward(Q[:, :, idx], K, V, W, b, g, EPS, L)
    assert np.abs(rows - full[:, :, idx]).max() < 1e-12
    assert np.abs(O.full_softmax_attention(Q[:, :, idx], K, V) - O.full_softmax_attention(Q, K, V)[:, :, idx]).max() < 1e-12


def test_sampled_rows_backward_equals_full_backward_with_zero_rows():
    # rows outside the sample get a zero upstream gradient: nothing of theirs reaches W, b or g
    Q, K, V, W, b, g, L, idx = _sampled_case(92)
    r = np.random.default_rng(5)
    dout_s = r.standard_normal((Q.shape[0], Q.shape[1], idx.size, Q.shape[3]))
    dout = np.zeros_like(Q)
    dout[:, :, idx] = dout_s
    for LL in (L, 0):
        got = O.hybrid_backward(Q[:, :, idx], K, V, W, b, g, EPS, LL, dout_s)
        ref = O.hybrid_backward(Q, K, V, W, b, g, EPS, LL, dout)
        for a, c in zip(got, ref):
            assert np.abs(a - c).max() < 1e-10 * max(1.0, np.abs(c).max())


# ---------------------------------------------------------------- planted mistakes

def _pins_linear():
    test_linear_branch_hand_worked()
    test_linear_branch_matches_bruteforce_nxn()
    test_linear_branch_closed_form_constant_phi()


def _pins_landmark():
    test_landmark_hand_worked()
    test_landmark_matches_torch_sdpa_on_gathered()
    test_hybrid_alpha_zero_all_landmarks_is_full_softmax()


def _pins_causal():
    test_causal_hand_worked()
    test_causal_matches_masked_bruteforce()


def _mut_apply_no_eps(Q, W, b, KV, ksum, eps):
    phiq = O.feature_map(Q, W, b)
    return np.einsum("bhnf,bhfd->bhnd", phiq, KV) / np.einsum("bhnf,bhf->bhn", phiq, ksum)[..., None]


def _mut_apply_eps_outside(Q, W, b, KV, ksum, eps):
    phiq = O.feature_map(Q, W, b)
    return np.einsum("bhnf,bhfd->bhnd", phiq, KV) / np.einsum("bhnf,bhf->bhn", phiq, ksum)[..., None] + eps


def _mut_elu_no_plus_one(z):
    z = np.asarray(z, dtype=np.float64)
    return np.where(z > 0.0, z, np.expm1(np.minimum(z, 0.0)))


def _mut_elu_relu(z):
    return np.maximum(np.asarray(z, dtype=np.float64), 0.0) + 1.0


def _mut_landmark_no_scale(Q, K, V, L):
    Q = np.asarray(Q, dtype=np.float64)
    return _orig_landmark(Q * math.sqrt(Q.shape[3]), K, V, L)


def _mut_landmark_idx_offset(N, L):
    return np.array([min(N - 1, (j * N) // L + 1) for j in range(L)], dtype=np.int64)


def _mut_blend_swapped(out_lin, out_lm, g):
    return _orig_blend(out_lm, out_lin, g)


def _mut_causal_exclusive(Q, K, V, W, b, eps):
    phiq = O.feature_map(Q, W, b)
    phik = O.feature_map(K, W, b)
    V = np.asarray(V, dtype=np.float64)
    B, H, N, F = phiq.shape
    S = np.zeros((B, H, F, V.shape[3]))
    z = np.zeros((B, H, F))
    out = np.empty((B, H, N, V.shape[3]))
    for n in range(N):
        qn = phiq[:, :, n, :]
        out[:, :, n, :] = np.einsum("bhf,bhfd->bhd", qn, S) / (np.einsum("bhf,bhf->bh", qn, z) + eps)[..., None]
        S += phik[:, :, n, :, None] * V[:, :, n, None, :]
        z += phik[:, :, n, :]
    return out


def _mut_softmax_token_axis(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=-2, keepdims=True))
    return e / e.sum(axis=-2, keepdims=True)


def _mut_relu_plus_one(z):
    return np.maximum(np.asarray(z, dtype=np.float64), 0.0) + 1.0


def _pins_softmax():
    test_softmax_map_hand_worked_and_invariants()
    test_softmax_map_matches_torch()
    test_other_maps_linear_and_causal_match_bruteforce("softmax")


def _pins_relu():
    test_relu_map_values()
    test_other_maps_linear_and_causal_match_bruteforce("relu")


def _mut_split_heads_interleaved(y, H):
    B, N, E = y.shape
    return y.reshape(B, N, E // H, H).transpose(0, 3, 1, 2)


def _mut_merge_heads_interleaved(a):
    B, H, N, D = a.shape
    return a.transpose(0, 2, 3, 1).reshape(B, N, H * D)


def _mut_layer_no_value_bias(x, Wq, bq, Wk, bk, Wv, bv, Wo, bo, H, eps, causal=False, kind="elu1"):
    return _orig_layer(x, Wq, bq, Wk, bk, Wv, None, Wo, bo, H, eps, causal, kind)


def _pins_layer():
    test_nnt_layer_matches_bruteforce("elu1", False)
    test_nnt_layer_matches_bruteforce("elu1", True)


def _mut_elu_grad_one(z):
    return np.ones_like(np.asarray(z, dtype=np.float64))


def _mut_backward_no_den_term(Q, K, V, W, b, g, eps, L, dout):
    # the chain rule without the normaliser's path (dden = 0): a plausible slip
    Q, K, V, W, b, g, dout = (np.asarray(a, dtype=np.float64) for a in (Q, K, V, W, b, g, dout))
    B, H, N, D = Q.shape
    dW, db, dg = np.zeros_like(W), np.zeros_like(b), np.zeros_like(g)
    alpha = 1 / (1 + np.exp(-g))
    lm = O.landmark_attn(Q, K, V, L)
    for bi in range(B):
        for h in range(H):
            zq, zk = Q[bi, h] @ W[h] + b[h], K[bi, h] @ W[h] + b[h]
            pq, pk = O.elu_plus_one(zq), O.elu_plus_one(zk)
            KV, ks = pk.T @ V[bi, h], pk.sum(axis=0)
            den = pq @ ks + eps
            lin = (pq @ KV) / den[:, None]
            G = dout[bi, h]
            dg[h] += (G * (lin - lm[bi, h])).sum() * alpha[h] * (1 - alpha[h])
            dnum = alpha[h] * G / den[:, None]
            dKV = pq.T @ dnum
            dzq = (dnum @ KV.T) * O.elu_plus_one_grad(zq)
            dzk = (V[bi, h] @ dKV.T) * O.elu_plus_one_grad(zk)
            dW[h] += Q[bi, h].T @ dzq + K[bi, h].T @ dzk
            db[h] += dzq.sum(axis=0) + dzk.sum(axis=0)
    return dW, db, dg


def _mut_loss_unweighted(out, teacher, s, delta=1.0):
    loss, dout, ds, H, C = _orig_loss(out, teacher, np.zeros(2), delta)
    return H + C + s[0] + s[1], dout, ds, H, C


def _mut_adam_no_bias_correction(p, grad, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8):
    p, grad, m, v = (np.asarray(a, dtype=np.float64) for a in (p, grad, m, v))
    m = beta1 * m + (1 - beta1) * grad
    v = beta2 * v + (1 - beta2) * grad * grad
    return p - lr * m / (np.sqrt(v) + eps), m, v


def _mut_gate_no_hysteresis_update(self, d):
    self.ema = d if self.updates == 0 else self.rate * self.ema + (1.0 - self.rate) * d
    self.updates += 1
    self.ready = self.updates >= self.min_updates and self.ema <= self.on
    return self.ready


def _pins_gate():
    test_gate_ema_hand_worked()
    test_gate_hysteresis_does_not_flap()


def _pins_backward():
    test_backward_matches_finite_differences()
    test_backward_matches_torch_autograd()


_orig_landmark = O.landmark_attn
_orig_blend = O.blend
_orig_layer = O.nnt_layer_forward
_orig_backward = O.hybrid_backward
_orig_loss = O.distill_loss


@pytest.mark.parametrize("attr,mutant,pins", [
    ("apply", _mut_apply_no_eps, _pins_linear),
    ("apply", _mut_apply_eps_outside, _pins_linear),
    ("elu_plus_one", _mut_elu_no_plus_one, _pins_linear),
    ("elu_plus_one", _mut_elu_relu, _pins_linear),
    ("landmark_attn", _mut_landmark_no_scale, _pins_landmark),
    ("landmark_indices", _mut_landmark_idx_offset, _pins_landmark),
    ("blend", _mut_blend_swapped, test_hybrid_hand_worked),
    ("causal_forward", _mut_causal_exclusive, _pins_causal),
    ("softmax_map", _mut_softmax_token_axis, _pins_softmax),
    ("relu_map", _mut_relu_plus_one, _pins_relu),
    ("split_heads", _mut_split_heads_interleaved, _pins_layer),
    ("merge_heads", _mut_merge_heads_interleaved, _pins_layer),
    ("nnt_layer_forward", _mut_layer_no_value_bias, _pins_layer),
    ("elu_plus_one_grad", _mut_elu_grad_one, _pins_backward),
    ("hybrid_backward", _mut_backward_no_den_term, _pins_backward),
    ("distill_loss", _mut_loss_unweighted, test_distill_loss_matches_torch),
    ("adam_update", _mut_adam_no_bias_correction, test_adam_matches_torch_optim),
])
def test_planted_mistake_is_caught(monkeypatch, attr, mutant, pins):
    monkeypatch.setattr(O, attr, mutant)
    with pytest.raises(AssertionError):
        pins()


def test_planted_gate_without_hysteresis_is_caught(monkeypatch):
    monkeypatch.setattr(O.ReadinessGate, "update", _mut_gate_no_hysteresis_update)
    with pytest.raises(AssertionError):
        _pins_gate()


def _mut_replay_lifo_push(self, Q, K, V, idx, teacher=None):
    """Planted mistake: evicts the newest sample instead of the oldest."""
    idx = np.asarray(idx, dtype=np.int32)
    B, H, N, D = np.asarray(K).shape
    foot = O.replay_sample_bytes(B, H, N, D, np.asarray(K).dtype.itemsize, idx.size, teacher is not None)
    if foot > self.budget:
        return None
    while self.samples and self.used + foot > self.budget:
        self.samples.pop()
        self.evicted += 1
    sid = self.next_id
    self.next_id += 1
    self.samples.append((sid, foot, {"K": K, "V": V, "Q": np.asarray(Q)[:, :, idx], "idx": idx, "T": teacher}))
    return sid


def test_planted_replay_lifo_eviction_is_caught(monkeypatch):
    monkeypatch.setattr(O.ReplayBuffer, "push", _mut_replay_lifo_push)
    with pytest.raises(AssertionError):
        test_replay_holds_longest_fitting_suffix()


def _mut_landmarks_over_queries(Q, K, V, L):
    """Planted mistake: the landmark stride taken from the query rows."""
    Q, K, V = np.asarray(Q, float), np.asarray(K, float), np.asarray(V, float)
    B, H, N, D = Q.shape
    idx = O.landmark_indices(N, L)
    out = np.empty((B, H, N, D))
    for bi in range(B):
        for h in range(H):
            s_ = (Q[bi, h] @ K[bi, h][idx].T) / math.sqrt(D)
            p_ = np.exp(s_ - s_.max(axis=1, keepdims=True))
            out[bi, h] = (p_ @ V[bi, h][idx]) / p_.sum(axis=1, keepdims=True)
    return out


def test_planted_landmarks_over_queries_is_caught(monkeypatch):
    monkeypatch.setattr(O, "landmark_attn", _mut_landmarks_over_queries)
    with pytest.raises(AssertionError):
        test_sampled_rows_forward_equals_rows_of_full_forward()

"""fp64 CPU oracle for the TTR hybrid-attention forward and the causal elu+1 variant.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it. It shares no code with the HIP library and imports
nothing from it.

Sources (page titles and sections of the method's web pages):

* "Flux2TTRTrainer", section "How the distillation works": the TTR layer
  combines a kernel branch whose cost grows linearly with the tokens and an
  exact softmax over a few landmark tokens, mixed by a weight kept in (0, 1). Section "Why this exists":
  the branch stands in for a layer's attention as a kernel regression. Section
  "Inputs worth setting": feature_dim defaults to 256 and is a multiple of 256.
* "NNT Define Linear Attention", section "The inputs": the elu feature map is
  elu(x) + 1; eps (default 1e-6) sits in the denominator; causal masks so a
  token attends only to earlier tokens. Section "How it works": compute
  K'^T V first, normalise with 1 / (Q' . sum(K') + eps), never form the
  N x N map.

Every function computes the plain definition in float64 with numpy, one
(batch, head) slice at a time. Readings taken where the pages are silent:

* elu uses alpha = 1 (the standard elu).
* The same W_h, b_h map both Q and K; W is [H, D, F], b is [H, F], g is [H].
* Landmarks are idx_j = floor(j * N / L), j = 0..L-1 (strided from token 0;
  with N = 256, L = 16 this is every 16th token).
* The landmark branch is softmax(Q K_L^T / sqrt(D)) V_L on the raw Q, K, V.
* alpha_h = sigmoid(g_h) weights the linear branch:
  out = alpha * out_lin + (1 - alpha) * out_lm.
* L = 0 means no landmark branch: out = out_lin.
* The causal mask includes the diagonal (key index <= query index).
* Without W the feature map is the identity projection: phi(x) = elu(x + b) + 1
  with F = D (b optional).
* The relu and softmax feature maps ("NNT Define Linear Attention", section
  "The inputs") are max(z, 0) and the softmax over each token's features,
  applied to z = x (+ b) like elu + 1.

The NNT linear-attention layer ("NNT Define Linear Attention", sections "The
inputs" and "How it works": project Q/K/V, apply the feature map, K'^T V
first, normalise, project back out; embed_dim divides by num_heads;
batch_first) is read as: x [B, N, E]; each projection is x @ W + b with W
[E, E] (input rows, output columns, the same row-vector convention as W_h)
and b [E]; heads are consecutive D = E / H column blocks; dropout is the
identity (an inference forward).

The distillation step ("Flux2TTRTrainer", section "How the distillation
works": the teacher is native softmax attention, the student is the TTR
layer, the huber and cosine terms of the loss are weighed by learned
uncertainties after Kendall, optimizer state persists per layer) is read as: teacher =
softmax(Q K^T / sqrt(D)) V on the same inputs; loss = exp(-s1) huber + s1 +
exp(-s2) (1 - cos) + s2 with learnable log-variances s = (s1, s2) (Kendall,
Gal and Cipolla's homoscedastic weighting), huber with delta = 1 averaged over
every element, cos per (batch, head, token) row over D averaged over rows
(cos = o.t / max(|o| |t|, 1e-8)); Adam (beta1 0.9, beta2 0.999, eps 1e-8,
bias-corrected, no weight decay) updates W, b, g and s. The backward gives
the gradients of the trainable parameters W, b, g (Q, K, V are the frozen
model's activations).

A replay sample (below) keeps every key and value but only some query rows,
and the student is trained on it ("Flux2TTRTrainer", section "How the
distillation works"). Every function here therefore takes Q with Nq rows and
K, V with N rows: the linear branch and the landmarks (strided over the N
keys) come from K and V, and each query row's output depends on that row
only. Trained on a sample, the loss averages over the sample's rows, and its
teacher is the teacher's output at those rows.

Readiness gating and the landmark count ("Flux2TTRTrainer", section "How the
distillation works": a layer serves the student only after enough updates and
once the moving average of its cosine distance to the teacher has dropped far
enough, with separate on and off thresholds, and serves the teacher otherwise; section "Inputs worth setting": landmark
fraction/min/max and a readiness threshold) are read as: distance = mean over
(batch, head, token) rows of 1 - cos(student_row, teacher_row); ema = d on
the first update, then rate * ema + (1 - rate) * d; a gate that is not ready
becomes ready when updates >= min_updates and ema <= threshold_on, a ready
gate drops when ema > threshold_off (threshold_off >= threshold_on); a
non-finite distance drops it; L = clamp(round-half-up(fraction * N), lmin,
lmax), at most N.

The replay buffer ("Flux2TTRTrainer", section "How the distillation works":
samples keep full keys and values but subsampled queries, offloaded to CPU
memory with a 768 MB budget by default; section "The honest gotchas": replay
offloads to the CPU by default) is read as: a sample of one layer call holds
K and V [B, H, N, D] whole, the query rows Q[:, :, idx] [B, H, Nq, D] at a
caller-given strictly increasing subset idx of the N tokens, optionally the
teacher's fp32 output rows at the same idx, and idx itself (int32); each
stored array counts toward the budget rounded up to 256 bytes; when a new
sample would exceed the budget the oldest samples are evicted first (FIFO)
until it fits, and a sample larger than the whole budget is refused without
changing anything. Under FIFO the samples held are exactly the longest run of
most recent pushes whose sizes fit the budget.

Pins (tests/test_oracle.py): brute-force N x N row-normalised attention,
torch's elu and scaled_dot_product_attention in fp64, closed forms
(W = 0, L = 1, Q = 0, first causal token), invariants (phi > 0, permutation,
linearity, convex hull, alpha limits, last causal token equals the non-causal
result), and a hand-worked example under tests/golden/. The NNT layer is pinned by
the layer restated in torch with heads as column slices and the N x N form,
the zero query/key projection closed form, and head-permutation invariance.
Sampled query rows are pinned by the forward on a subset of rows equal to
those rows of the full forward, and the backward on them equal to the full
backward with a zero upstream gradient on every other row.
The replay buffer is pinned by the brute-force longest-fitting-suffix rule over
a random push sequence, hand-worked footprints, row-by-row gathering and the
refusal of a sample larger than the budget.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "elu_plus_one", "relu_map", "softmax_map", "MAPS", "feature_map", "kv_reduce", "apply", "landmark_indices",
    "landmark_attn", "blend", "hybrid_forward", "causal_forward",
    "hybrid_rows", "causal_rows", "normwise_err", "split_heads", "merge_heads", "nnt_layer_forward",
    "elu_plus_one_grad", "hybrid_backward", "full_softmax_attention", "distill_loss", "adam_update", "distill_step",
    "cosine_distance", "landmark_count", "ReadinessGate", "replay_part_bytes", "replay_sample_bytes",
    "ReplayBuffer",
]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def elu_plus_one(z: np.ndarray) -> np.ndarray:
    """elu(z) + 1 with alpha = 1: z + 1 for z > 0, exp(z) otherwise.

    "NNT Define Linear Attention", section "The inputs" (elu mapped as elu(x)+1).
    """
    z = np.asarray(z, dtype=np.float64)
    # elu(z) = z for z > 0 and exp(z) - 1 otherwise; adding 1 gives the two
    # branches below exactly (written this way so that exp(z) is not lost to
    # cancellation against 1 for very negative z).
    return np.where(z > 0.0, z + 1.0, np.exp(np.minimum(z, 0.0)))


def relu_map(z: np.ndarray) -> np.ndarray:
    """max(z, 0): the relu feature map of "NNT Define Linear Attention", section
    "The inputs" (named there beside elu as cheap and non-negative)."""
    return np.maximum(np.asarray(z, dtype=np.float64), 0.0)


def softmax_map(z: np.ndarray) -> np.ndarray:
    """Softmax over the feature axis (the last one) of every token: the softmax
    feature map of "NNT Define Linear Attention", section "The inputs". The
    page names the option only; normalising each token's features (not the
    tokens) is the reading taken, since the map replaces the similarity score
    by a dot product of mapped features."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# map kind -> function name (looked up when called)
MAPS = {"elu1": "elu_plus_one", "relu": "relu_map", "softmax": "softmax_map"}


def _phi_slice(x: np.ndarray, W: Optional[np.ndarray], b: Optional[np.ndarray], kind: str = "elu1") -> np.ndarray:
    # x [N, D] -> phi [N, F]; one head's map.
    z = x @ W if W is not None else x.copy()
    if b is not None:
        z = z + b[None, :]
    return globals()[MAPS[kind]](z)


def feature_map(X, W=None, b=None, kind: str = "elu1") -> np.ndarray:
    """phi(X) = map(X W_h + b_h) per (batch, head).  X [B,H,N,D] -> [B,H,N,F].

    map is elu(z) + 1 by default (the hybrid forward's map; "Flux2TTRTrainer"
    section "Inputs worth setting" for feature_dim F; "NNT Define Linear
    Attention" section "The inputs" for elu + 1), or relu / softmax over the
    features (the other options of that section).
    """
    X, W, b = _f64(X), _f64(W), _f64(b)
    B, H, N, D = X.shape
    F = W.shape[2] if W is not None else D
    out = np.empty((B, H, N, F))
    for bi in range(B):
        for h in range(H):
            out[bi, h] = _phi_slice(X[bi, h], None if W is None else W[h], None if b is None else b[h], kind)
    return out


def kv_reduce(K, V, W=None, b=None, kind: str = "elu1"):
    """KV_h = phi(K)^T V  [B,H,F,D] and ksum_h = sum_n phi(K)_n  [B,H,F].

    "NNT Define Linear Attention", section "How it works" (accumulate kv = K^T V,
    the sum of K' for the normaliser).
    """
    K, V = _f64(K), _f64(V)
    phik = feature_map(K, W, b, kind)
    B, H, N, F = phik.shape
    D = V.shape[3]
    KV = np.empty((B, H, F, D))
    ksum = np.empty((B, H, F))
    for bi in range(B):
        for h in range(H):
            KV[bi, h] = phik[bi, h].T @ V[bi, h]
            ksum[bi, h] = phik[bi, h].sum(axis=0)
    return KV, ksum


def apply(Q, W, b, KV, ksum, eps, kind: str = "elu1") -> np.ndarray:
    """out_lin = (phi(Q) KV) / (phi(Q) . ksum + eps)  [B,H,N,D].

    "NNT Define Linear Attention", section "How it works" (Q'(K'^T V), normalised by
    1 / (Q' . sum(K') + eps)); eps from section "The inputs".
    """
    phiq = feature_map(Q, W, b, kind)
    KV, ksum = _f64(KV), _f64(ksum)
    eps = float(eps)
    B, H, N, F = phiq.shape
    D = KV.shape[3]
    out = np.empty((B, H, N, D))
    for bi in range(B):
        for h in range(H):
            num = phiq[bi, h] @ KV[bi, h]
            den = phiq[bi, h] @ ksum[bi, h] + eps
            out[bi, h] = num / den[:, None]
    return out


def landmark_indices(N: int, L: int) -> np.ndarray:
    """Strided landmark tokens idx_j = floor(j N / L), integer arithmetic.

    "Flux2TTRTrainer", section "How the distillation works" (landmark tokens);
    strided placement from token 0 is the reading taken (with N = 256, L = 16 it
    gives every 16th token).
    """
    if not (0 < L <= N):
        raise ValueError("need 0 < L <= N")
    return np.array([(j * N) // L for j in range(L)], dtype=np.int64)


def landmark_attn(Q, K, V, L: int) -> np.ndarray:
    """Exact softmax attention of every query over the L landmark tokens.

    S = Q K_L^T / sqrt(D); P = softmax over landmarks (max-subtracted);
    out_lm = P V_L.  "Flux2TTRTrainer", section "How the distillation works"
    (small exact-softmax branch over landmark tokens).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, N, D = Q.shape
    idx = landmark_indices(K.shape[2], L)  # landmarks stride over the keys (N keys may differ from Q's rows)
    out = np.empty((B, H, N, D))
    scale = 1.0 / math.sqrt(D)
    for bi in range(B):
        for h in range(H):
            kl = K[bi, h][idx]
            vl = V[bi, h][idx]
            s = (Q[bi, h] @ kl.T) * scale
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[bi, h] = (p @ vl) / p.sum(axis=1, keepdims=True)
    return out


def _sigmoid(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def blend(out_lin, out_lm, g) -> np.ndarray:
    """out = alpha_h out_lin + (1 - alpha_h) out_lm with alpha_h = sigmoid(g_h).

    "Flux2TTRTrainer", section "How the distillation works" (blended by a
    bounded weight).
    """
    out_lin, out_lm = _f64(out_lin), _f64(out_lm)
    a = _sigmoid(g)[None, :, None, None]
    return a * out_lin + (1.0 - a) * out_lm


def hybrid_forward(Q, K, V, W, b, g, eps, L: int, kind: str = "elu1") -> np.ndarray:
    """The TTR hybrid forward: linear kernel branch, landmark softmax branch, blend.

    With L = 0 the landmark branch is absent and the result is out_lin (the
    plain linear attention of "NNT Define Linear Attention", with any of its
    feature maps).
    """
    KV, ksum = kv_reduce(K, V, W, b, kind)
    lin = apply(Q, W, b, KV, ksum, eps, kind)
    if L == 0:
        return lin
    lm = landmark_attn(Q, K, V, L)
    return blend(lin, lm, g)


def causal_forward(Q, K, V, W, b, eps, kind: str = "elu1") -> np.ndarray:
    """Causal linear attention (elu+1 by default) as the running prefix over tokens.

    For n = 0..N-1:  S += phi(k_n) v_n^T,  z += phi(k_n),
    out_n = phi(q_n) S / (phi(q_n) . z + eps).
    "NNT Define Linear Attention", section "The inputs" (causal: tokens attend
    only to earlier tokens, here including themselves) and section "How it works".
    Vectorised over the (batch, head) slices; the loop runs over tokens.
    """
    phiq = feature_map(Q, W, b, kind)
    phik = feature_map(K, W, b, kind)
    V = _f64(V)
    eps = float(eps)
    B, H, N, F = phiq.shape
    D = V.shape[3]
    S = np.zeros((B, H, F, D))
    z = np.zeros((B, H, F))
    out = np.empty((B, H, N, D))
    for n in range(N):
        kn = phik[:, :, n, :]
        S += kn[..., :, None] * V[:, :, n, None, :]
        z += kn
        qn = phiq[:, :, n, :]
        num = np.einsum("bhf,bhfd->bhd", qn, S)
        den = np.einsum("bhf,bhf->bh", qn, z) + eps
        out[:, :, n, :] = num / den[..., None]
    return out


def hybrid_rows(Q, K, V, W, b, g, eps, L: int, rows: Sequence[tuple], kind: str = "elu1") -> np.ndarray:
    """hybrid_forward evaluated only at the listed (batch, head, token) rows.

    The linear branch uses the kernel-regression form of the same definition
    (weights phi(q_n) . phi(k_m), normalised by their sum plus eps), which needs
    one pass over the slice per row; the landmark branch and blend are as in
    ``landmark_attn`` and ``blend``.  Returns [len(rows), D].
    """
    Q, K, V, W, b = _f64(Q), _f64(K), _f64(V), _f64(W), _f64(b)
    _, _, N, D = Q.shape
    res = np.empty((len(rows), D))
    cache = {}
    for i, (bi, h, n) in enumerate(rows):
        key = (bi, h)
        if key not in cache:
            Wh = None if W is None else W[h]
            bh = None if b is None else b[h]
            cache[key] = _phi_slice(K[bi, h], Wh, bh, kind)
        phik = cache[key]
        Wh = None if W is None else W[h]
        bh = None if b is None else b[h]
        phiq = _phi_slice(Q[bi, h][n:n + 1], Wh, bh, kind)[0]
        wts = phik @ phiq
        lin = (wts @ V[bi, h]) / (wts.sum() + float(eps))
        if L == 0:
            res[i] = lin
            continue
        idx = landmark_indices(N, L)
        s = (K[bi, h][idx] @ Q[bi, h][n]) / math.sqrt(D)
        p = np.exp(s - s.max())
        lm = (p @ V[bi, h][idx]) / p.sum()
        a = float(_sigmoid(np.asarray(g, dtype=np.float64)[h]))
        res[i] = a * lin + (1.0 - a) * lm
    return res


def causal_rows(Q, K, V, W, b, eps, rows: Sequence[tuple], kind: str = "elu1") -> np.ndarray:
    """causal_forward evaluated only at the listed (batch, head, token) rows.

    Direct masked sum for row n: weights phi(q_n) . phi(k_m) for m <= n,
    out_n = sum_m w_m v_m / (sum_m w_m + eps).  Returns [len(rows), D].
    """
    Q, K, V, W, b = _f64(Q), _f64(K), _f64(V), _f64(W), _f64(b)
    D = V.shape[3]
    res = np.empty((len(rows), D))
    for i, (bi, h, n) in enumerate(rows):
        Wh = None if W is None else W[h]
        bh = None if b is None else b[h]
        phik = _phi_slice(K[bi, h][: n + 1], Wh, bh, kind)
        phiq = _phi_slice(Q[bi, h][n:n + 1], Wh, bh, kind)[0]
        wts = phik @ phiq
        res[i] = (wts @ V[bi, h][: n + 1]) / (wts.sum() + float(eps))
    return res


def split_heads(y: np.ndarray, H: int) -> np.ndarray:
    """[B, N, E] -> [B, H, N, D]: head h takes columns h*D .. h*D + D - 1."""
    B, N, E = y.shape
    return y.reshape(B, N, H, E // H).transpose(0, 2, 1, 3)


def merge_heads(a: np.ndarray) -> np.ndarray:
    """[B, H, N, D] -> [B, N, H*D], the inverse of split_heads."""
    B, H, N, D = a.shape
    return a.transpose(0, 2, 1, 3).reshape(B, N, H * D)


def nnt_layer_forward(x, Wq, bq, Wk, bk, Wv, bv, Wo, bo, H: int, eps, causal: bool = False,
                      kind: str = "elu1") -> np.ndarray:
    """NNT linear-attention layer, inference forward.

    "NNT Define Linear Attention", section "How it works": Q, K, V are
    projections of x; the feature map applies to Q and K; the attention is
    phi(Q) (phi(K)^T V) / (phi(Q) . sum phi(K) + eps) per head (prefix sums
    when causal, section "The inputs"); the heads are merged and projected
    out. x [B, N, E]; W* [E, E] used as x @ W; b* [E] or None. Returns
    [B, N, E] float64.
    """
    x = _f64(x)
    B, N, E = x.shape
    assert E % H == 0, "embed_dim must divide by num_heads"

    def proj(inp, W, b):
        y = inp @ _f64(W)
        return y if b is None else y + _f64(b)

    Q, K, V = (split_heads(proj(x, W, b), H) for W, b in ((Wq, bq), (Wk, bk), (Wv, bv)))
    if causal:
        A = causal_forward(Q, K, V, None, None, eps, kind)
    else:
        KV, ksum = kv_reduce(K, V, None, None, kind)
        A = apply(Q, None, None, KV, ksum, eps, kind)
    return proj(merge_heads(A), Wo, bo)


def elu_plus_one_grad(z: np.ndarray) -> np.ndarray:
    """d(elu(z) + 1)/dz: 1 for z > 0, exp(z) otherwise (equal to the map itself there)."""
    z = np.asarray(z, dtype=np.float64)
    return np.where(z > 0.0, 1.0, np.exp(np.minimum(z, 0.0)))


def hybrid_backward(Q, K, V, W, b, g, eps, L: int, dout):
    """Gradients of sum(dout * hybrid_forward(...)) with respect to W [H,D,F],
    b [H,F] and g [H] (elu + 1 map with a projection), by the chain rule through
    the forward's definition:

      z_q = Q W + b, z_k = K W + b, phi = elu(z) + 1
      KV = phi_k^T V, ks = sum_n phi_k, num = phi_q KV, den = phi_q . ks + eps
      lin = num / den, alpha = sigmoid(g), out = alpha lin + (1 - alpha) lm

      dlin   = alpha dout;       dalpha = sum(dout * (lin - lm));  dg = dalpha alpha (1 - alpha)
      dnum   = dlin / den;       dden = -sum_d(dlin * lin) / den
      dphi_q = dnum KV^T + dden ks^T
      dKV    = phi_q^T dnum;     dks = phi_q^T dden
      dphi_k = V dKV^T + 1 dks^T
      dz     = dphi * phi'(z);   dW = Q^T dz_q + K^T dz_k;   db = sum_n (dz_q + dz_k)

    The landmark branch (raw Q, K, V) holds no parameter: it enters through
    alpha only. Sums run over the batch for the per-head parameters.
    """
    Q, K, V, W, b, g, dout = (_f64(a) for a in (Q, K, V, W, b, g, dout))
    B, H, N, D = Q.shape
    F = W.shape[2]
    dW = np.zeros((H, D, F))
    db = np.zeros((H, F))
    dg = np.zeros(H)
    alpha = _sigmoid(g)
    lm = landmark_attn(Q, K, V, L) if L > 0 else np.zeros_like(Q)
    for bi in range(B):
        for h in range(H):
            bh = np.zeros(F) if b is None else b[h]
            zq = Q[bi, h] @ W[h] + bh
            zk = K[bi, h] @ W[h] + bh
            pq, pk = elu_plus_one(zq), elu_plus_one(zk)
            KV = pk.T @ V[bi, h]
            ks = pk.sum(axis=0)
            num = pq @ KV
            den = pq @ ks + eps
            lin = num / den[:, None]
            G = dout[bi, h]
            a = alpha[h] if L > 0 else 1.0
            if L > 0:
                dg[h] += (G * (lin - lm[bi, h])).sum() * alpha[h] * (1.0 - alpha[h])
            dlin = a * G
            dnum = dlin / den[:, None]
            dden = -(dlin * lin).sum(axis=1) / den
            dpq = dnum @ KV.T + np.outer(dden, ks)
            dKV = pq.T @ dnum
            dks = pq.T @ dden
            dpk = V[bi, h] @ dKV.T + dks[None, :]
            dzq = dpq * elu_plus_one_grad(zq)
            dzk = dpk * elu_plus_one_grad(zk)
            dW[h] += Q[bi, h].T @ dzq + K[bi, h].T @ dzk
            db[h] += dzq.sum(axis=0) + dzk.sum(axis=0)
    return dW, db, dg


def full_softmax_attention(Q, K, V) -> np.ndarray:
    """softmax(Q K^T / sqrt(D)) V per (batch, head): native attention, the teacher.
    One (batch, head) slice at a time, with matrix products (queries may be
    fewer than keys: Q [B,H,Nq,D], K and V [B,H,N,D])."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, Nq, D = Q.shape
    out = np.empty((B, H, Nq, V.shape[3]))
    for bi in range(B):
        for h in range(H):
            S = (Q[bi, h] @ K[bi, h].T) / math.sqrt(D)
            S -= S.max(axis=-1, keepdims=True)
            P = np.exp(S)
            out[bi, h] = (P @ V[bi, h]) / P.sum(axis=-1)[:, None]
    return out


def distill_loss(out, teacher, s, delta: float = 1.0):
    """Uncertainty-weighted huber + cosine distillation loss and its gradients.

    loss = exp(-s1) H + s1 + exp(-s2) C + s2, H = mean over elements of
    huber_delta(out - teacher), C = mean over rows of 1 - cos(out_row,
    teacher_row). Returns (loss, dloss/dout, dloss/ds, H, C)."""
    o, t, s = _f64(out), _f64(teacher), _f64(s)
    r = o - t
    ar = np.abs(r)
    H = np.where(ar <= delta, 0.5 * r * r, delta * (ar - 0.5 * delta)).mean()
    dH = np.clip(r, -delta, delta) / r.size
    no = np.linalg.norm(o, axis=-1)
    nt = np.linalg.norm(t, axis=-1)
    dot = (o * t).sum(axis=-1)
    den = np.maximum(no * nt, 1e-8)
    cos = dot / den
    rows = cos.size
    C = (1.0 - cos).mean()
    # d cos / d o = t / den - dot * o * nt / (no den^2) where no * nt > 1e-8 (else t / 1e-8)
    live = (no * nt) > 1e-8
    safe_no = np.where(no > 0, no, 1.0)
    dcos = t / den[..., None] - np.where(live, dot * nt / (safe_no * den * den), 0.0)[..., None] * o
    dC = -dcos / rows
    w1, w2 = math.exp(-s[0]), math.exp(-s[1])
    loss = w1 * H + s[0] + w2 * C + s[1]
    dout = w1 * dH + w2 * dC
    ds = np.array([1.0 - w1 * H, 1.0 - w2 * C])
    return loss, dout, ds, H, C


def adam_update(p, grad, m, v, step: int, lr: float, beta1=0.9, beta2=0.999, eps=1e-8):
    """One Adam step (bias-corrected moments, step counted from 1). Returns (p, m, v)."""
    p, grad, m, v = _f64(p), _f64(grad), _f64(m), _f64(v)
    m = beta1 * m + (1.0 - beta1) * grad
    v = beta2 * v + (1.0 - beta2) * grad * grad
    mh = m / (1.0 - beta1 ** step)
    vh = v / (1.0 - beta2 ** step)
    return p - lr * mh / (np.sqrt(vh) + eps), m, v


def distill_step(Q, K, V, W, b, g, s, state, step: int, lr: float, eps, L: int, teacher=None):
    """One Phase-1 distillation step: teacher (full softmax attention unless
    given), student forward, loss, backward, Adam on W, b, g, s.

    state: dict of Adam moments {"mW","vW","mb","vb","mg","vg","ms","vs"}.
    Returns (W, b, g, s, state, loss)."""
    T = full_softmax_attention(Q, K, V) if teacher is None else _f64(teacher)
    out = hybrid_forward(Q, K, V, W, b, g, eps, L)
    loss, dout, ds, _, _ = distill_loss(out, T, s)
    dW, db, dg = hybrid_backward(Q, K, V, W, b, g, eps, L, dout)
    new = {}
    W2, new["mW"], new["vW"] = adam_update(W, dW, state["mW"], state["vW"], step, lr)
    b2, new["mb"], new["vb"] = adam_update(b, db, state["mb"], state["vb"], step, lr)
    g2, new["mg"], new["vg"] = adam_update(g, dg, state["mg"], state["vg"], step, lr)
    s2, new["ms"], new["vs"] = adam_update(s, ds, state["ms"], state["vs"], step, lr)
    return W2, b2, g2, s2, new, loss


def cosine_distance(student, teacher) -> float:
    """Mean over rows of 1 - o.t / max(|o| |t|, 1e-8), rows over the last axis."""
    o, t = _f64(student), _f64(teacher)
    cos = (o * t).sum(axis=-1) / np.maximum(np.linalg.norm(o, axis=-1) * np.linalg.norm(t, axis=-1), 1e-8)
    return float((1.0 - cos).mean())


def landmark_count(N: int, fraction: float, lmin: int, lmax: int) -> int:
    """round-half-up(fraction * N) clamped to [lmin, lmax] and to N."""
    L = int(math.floor(fraction * N + 0.5))
    return min(N, max(lmin, min(lmax, L)))


class ReadinessGate:
    """Per-layer fail-closed readiness gate with an EMA of the cosine distance and hysteresis."""

    def __init__(self, rate: float, threshold_on: float, threshold_off: float, min_updates: int):
        self.rate, self.on, self.off, self.min_updates = rate, threshold_on, threshold_off, min_updates
        self.ema, self.updates, self.ready = 0.0, 0, False

    def update(self, d: float) -> bool:
        if not math.isfinite(d):
            self.ready = False
            return self.ready
        self.ema = d if self.updates == 0 else self.rate * self.ema + (1.0 - self.rate) * d
        self.updates += 1
        if self.ready:
            if self.ema > self.off:
                self.ready = False
        elif self.updates >= self.min_updates and self.ema <= self.on:
            self.ready = True
        return self.ready


REPLAY_ALIGN = 256  # each stored array is counted (and placed) in whole 256-byte units


def replay_part_bytes(nbytes: int) -> int:
    """Bytes an array of ``nbytes`` takes from the replay budget."""
    return -(-int(nbytes) // REPLAY_ALIGN) * REPLAY_ALIGN


def replay_sample_bytes(B: int, H: int, N: int, D: int, io_bytes: int, Nq: int, teacher: bool) -> int:
    """Budget footprint of one sample: K, V (IO dtype), the Nq query rows (IO
    dtype), the teacher rows (fp32, when kept) and the int32 indices."""
    kv = replay_part_bytes(B * H * N * D * io_bytes)
    q = replay_part_bytes(B * H * Nq * D * io_bytes)
    t = replay_part_bytes(B * H * Nq * D * 4) if teacher else 0
    return 2 * kv + q + t + replay_part_bytes(Nq * 4)


class ReplayBuffer:
    """FIFO replay buffer of (K, V, subsampled Q, teacher rows, indices) under a byte budget.

    Arrays are kept as given (IO-dtype values or bf16 bit patterns, fp32
    teacher rows), copied at push time; ids count pushes from 0."""

    def __init__(self, budget: int):
        self.budget = int(budget)
        self.samples = []  # (id, footprint, dict) oldest first
        self.next_id = 0
        self.evicted = 0

    @property
    def used(self) -> int:
        return sum(f for _, f, _ in self.samples)

    def ids(self):
        return [i for i, _, _ in self.samples]

    def push(self, Q, K, V, idx, teacher=None):
        """Store one sample; return its id, or None (nothing changed) if it exceeds the budget."""
        Q, K, V = np.asarray(Q), np.asarray(K), np.asarray(V)
        idx = np.asarray(idx, dtype=np.int32)
        B, H, N, D = K.shape
        if Q.shape != K.shape or V.shape != K.shape or idx.ndim != 1 or idx.size < 1:
            raise ValueError("Q, K, V must share [B, H, N, D]; idx must be a non-empty vector")
        if idx[0] < 0 or idx[-1] >= N or np.any(np.diff(idx) <= 0):
            raise ValueError("idx must be strictly increasing in [0, N)")
        sample = {"K": K.copy(), "V": V.copy(), "Q": Q[:, :, idx, :].copy(), "idx": idx.copy(),
                  "T": None if teacher is None else np.asarray(teacher, dtype=np.float32)[:, :, idx, :].copy()}
        foot = replay_sample_bytes(B, H, N, D, K.dtype.itemsize, idx.size, teacher is not None)
        if foot > self.budget:
            return None
        while self.samples and self.used + foot > self.budget:
            self.samples.pop(0)
            self.evicted += 1
        sid = self.next_id
        self.next_id += 1
        self.samples.append((sid, foot, sample))
        return sid

    def fetch(self, sid: int):
        for i, _, smp in self.samples:
            if i == sid:
                return smp
        raise KeyError(sid)


def normwise_err(got, ref, axes=(-2, -1)) -> float:
    """max over slices of max|got - ref| / max|ref| (slices reduce over ``axes``)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(got - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    den = np.where(den == 0.0, 1.0, den)
    return float((num / den).max())

/*
 * ttr.h -- C ABI of the MI355X (gfx950) TTR hybrid-attention library (libttr.so).
 *
 * The method (web pages it is described on, by title and section):
 *   "Flux2TTRTrainer", "How the distillation works": a TTR layer combines a
 *     kernel branch whose cost grows linearly with the tokens and an exact
 *     softmax over a few landmark tokens, mixed by a weight kept in (0, 1); "Inputs worth setting":
 *     feature_dim F defaults to 256 and must be a multiple of 256.
 *   "NNT Define Linear Attention", "The inputs": feature map elu(x) + 1
 *     (also relu or softmax), eps = 1e-6 in the denominator, causal flag;
 *     "How it works": Q'(K'^T V) normalised by 1 / (Q' . sum(K') + eps).
 *
 * Computed per (batch b, head h), with x a row of Q or K and z = x W_h + b_h
 * (W == NULL: z = x + b_h, F = D):
 *   phi(x)  = elu(z) + 1                     (dims.fmap == TTR_FMAP_ELU1, the default)
 *           = max(z, 0)                      (TTR_FMAP_RELU)
 *           = exp(z) / sum_f exp(z_f)        (TTR_FMAP_SOFTMAX, over the F features)
 *   KV      = phi(K)^T V           [F, D]    ksum = sum_n phi(K)_n   [F]
 *   out_lin = phi(Q) KV / (phi(Q) . ksum + eps)
 *   idx_j   = floor(j N / L), j = 0..L-1     (strided landmarks from token 0)
 *   out_lm  = softmax(Q K[idx]^T / sqrt(D)) V[idx]
 *   out     = alpha_h out_lin + (1 - alpha_h) out_lm,  alpha_h = sigmoid(g_h)
 *   causal:  out_n = phi(q_n) S_n / (phi(q_n) . z_n + eps),
 *            S_n = sum_{m<=n} phi(k_m) v_m^T,  z_n = sum_{m<=n} phi(k_m)
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers to contiguous row-major arrays:
 *     Q, K, V, out_* [B,H,N,D]; W [H,D,F]; b [H,F] (or [H,D] when W is NULL);
 *     g [H]; KV [B,H,F,D]; ksum [B,H,F]; phi [B,H,N,F].
 *   - Q, K, V, W, phi and `out` of ttr_blend / ttr_hybrid_forward /
 *     ttr_causal_scan use the IO dtype (dims.dtype). b, g, KV, ksum, out_lin
 *     and out_lm are always fp32.
 *   - Every pointer must be 16-byte aligned. Outputs must not overlap inputs.
 *   - The caller owns all memory, including the workspace; the library never
 *     allocates, frees, synchronises or keeps a pointer after returning (the
 *     replay buffer object and the fixed workspace array of
 *     ttr_hybrid_forward_noalloc are the library's own, see there).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream). Calls are stateless and thread-safe.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     validation failure the call returns a non-zero status and enqueues
 *     nothing. A failed launch returns TTR_ERR_HIP; ttr_last_hip_error()
 *     gives the hipError_t (per calling thread).
 *   - Results are bitwise deterministic run to run (no floating-point atomics).
 *   - Kernels that wait for one another's results (the key/value stage's
 *     splits, the causal scan's segments) poll a bounded number of times
 *     (about 2^20). A wait that gives up makes the outputs it feeds NaN, and
 *     the causal scan also sets the error word of its workspace. Two
 *     environment variables, read at every launch, exist for tests:
 *     TTR_SPIN_LIMIT=n sets the poll limit (n >= 1), and
 *     TTR_KVS_CROSS_XCD_ROUND=1 makes the key/value stage take the coherent
 *     round it otherwise takes only when a group's workgroups span XCDs.
 *   - The key/value stage's meeting counters live in the workspace and need
 *     no reset launch: each launch carries a number (a process-wide count)
 *     that tags them, so their contents on entry do not matter, and the last
 *     workgroup of a group to leave clears them, so a launch captured in a
 *     graph can be replayed. Concurrent calls must not share a workspace.
 *   - Shape rules: B, H, N >= 1; D in {64, 128}; with W, F a multiple of 256
 *     (else TTR_ERR_SHAPE), of which F == 256 is implemented by every entry
 *     point and F == 512, 768 and 1024 by the bf16 ttr_hybrid_forward (and its
 *     _noalloc form); other multiples return TTR_ERR_UNSUPPORTED. Without W, F == D.
 *     The causal scan with fp32 IO and D == 128 takes chunk 64 only (others:
 *     TTR_ERR_UNSUPPORTED); its default chunk is then 64.
 *     0 <= L <= N. Ragged N (not a multiple of any tile size) is supported.
 *   - The relu and softmax feature maps are those of the NNT linear attention,
 *     applied to already projected features: they need W == NULL and no
 *     landmark branch (L == 0); otherwise TTR_ERR_UNSUPPORTED.
 */
#ifndef TTR_H
#define TTR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TTR_OK = 0,
  TTR_ERR_NULL = 1,        /* a required pointer is NULL                        */
  TTR_ERR_SHAPE = 2,       /* B/H/N/D/F/L/chunk outside the rules above          */
  TTR_ERR_DTYPE = 3,       /* unknown dims.dtype                                 */
  TTR_ERR_UNSUPPORTED = 4, /* a valid request this library does not implement    */
  TTR_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than ttr_workspace_bytes */
  TTR_ERR_ALIGN = 6,       /* a pointer is not 16-byte aligned                   */
  TTR_ERR_HIP = 7,         /* a HIP launch failed, see ttr_last_hip_error()      */
  TTR_ERR_ALIAS = 8,       /* an output overlaps an input                        */
  TTR_ERR_BUDGET = 9,      /* a replay sample larger than the budget or max size */
  TTR_ERR_NOT_FOUND = 10,  /* a replay sample id that is not (or no longer) held */
  TTR_ERR_DEVICE = 11      /* called with another device current than at create  */
} ttr_status;

typedef enum { TTR_FP32 = 0, TTR_BF16 = 1 } ttr_dtype;

typedef enum { TTR_FMAP_ELU1 = 0, TTR_FMAP_RELU = 1, TTR_FMAP_SOFTMAX = 2 } ttr_fmap;

/* Problem sizes. F is the feature dimension (a multiple of 256 with a projection W, D without). */
typedef struct {
  int32_t B, H, N, D, F;
  int32_t dtype; /* ttr_dtype of the IO tensors */
  int32_t fmap;  /* ttr_fmap; 0 (elu + 1) when zero-initialised */
} ttr_dims;

/* Feature map: phi = map(X W_h + b_h) (map per dims.fmap) written as [B,H,N,F] in the IO dtype.
 * "Flux2TTRTrainer", "Inputs worth setting" (feature_dim);
 * "NNT Define Linear Attention", "The inputs" (elu(x) + 1).
 * X [B,H,N,D]; W [H,D,F] or NULL (identity, F == D); b [H,F] fp32 or NULL. */
ttr_status ttr_feature_map(ttr_dims d, const void* X, const void* W, const float* b,
                           void* phi, void* stream);

/* Key/value reduction with the feature map fused: KV = phi(K)^T V (fp32
 * [B,H,F,D]) and ksum = sum_n phi(K)_n (fp32 [B,H,F]).
 * "NNT Define Linear Attention", "How it works" (kv = K^T V, sum(K)).
 * ws: device workspace of at least ttr_workspace_bytes(d, 0, 0, 0) bytes
 * (split-N partial sums; its contents on entry do not matter). */
ttr_status ttr_kv_reduce(ttr_dims d, const void* K, const void* V, const void* W,
                         const float* b, float* KV, float* ksum, void* ws, size_t ws_bytes,
                         void* stream);

/* Apply and normalise with the feature map of Q fused:
 * out_lin = phi(Q) KV / (phi(Q) . ksum + eps), fp32 [B,H,N,D].
 * "NNT Define Linear Attention", "How it works" and "The inputs" (eps). */
ttr_status ttr_apply(ttr_dims d, const void* Q, const void* W, const float* b,
                     const float* KV, const float* ksum, float eps, float* out_lin,
                     void* stream);

/* Exact softmax over L strided landmarks (1 <= L <= N):
 * out_lm = softmax(Q K[idx]^T / sqrt(D)) V[idx], idx_j = floor(j N / L); fp32 [B,H,N,D].
 * "Flux2TTRTrainer", "How the distillation works" (exact-softmax branch). */
ttr_status ttr_landmark_attn(ttr_dims d, const void* Q, const void* K, const void* V,
                             int32_t L, float* out_lm, void* stream);

/* Bounded blend: out = sigmoid(g_h) out_lin + (1 - sigmoid(g_h)) out_lm, out in
 * the IO dtype (round to nearest even for bf16). g [H] fp32 (+-inf allowed).
 * "Flux2TTRTrainer", "How the distillation works" (bounded weight). */
ttr_status ttr_blend(ttr_dims d, const float* out_lin, const float* out_lm, const float* g,
                     void* out, void* stream);

/* Causal linear attention as a chunked prefix scan (chunk in {64,128,256};
 * the chunk changes the schedule, not the result). Identity feature map only
 * (W must be NULL, F == D); b [H,D] fp32 or NULL.
 * out [B,H,N,D] in the IO dtype. ws: at least ttr_workspace_bytes(d, 0, 1, chunk) bytes.
 * "NNT Define Linear Attention", "The inputs" (causal) and "How it works". */
ttr_status ttr_causal_scan(ttr_dims d, const void* Q, const void* K, const void* V,
                           const void* W, const float* b, float eps, int32_t chunk,
                           void* out, void* ws, size_t ws_bytes, void* stream);

/* The whole hybrid forward (kv_reduce, then apply + landmark + blend in one
 * fused kernel), out [B,H,N,D] in the IO dtype. L == 0: out = out_lin.
 * causal != 0 routes to ttr_causal_scan and needs L == 0 and W == NULL (the
 * pages define no causal landmark branch: TTR_ERR_UNSUPPORTED otherwise).
 * The value names the chunk: 64, 128 or 256 runs that chunk; 1 runs the
 * default one (128, or the largest supported chunk below it for the dtype and
 * D); any other value is TTR_ERR_SHAPE.
 * ws: at least ttr_workspace_bytes(d, L, causal, 0) bytes. */
ttr_status ttr_hybrid_forward(ttr_dims d, const void* Q, const void* K, const void* V,
                              const void* W, const float* b, const float* g, float eps,
                              int32_t L, int32_t causal, void* out, void* ws,
                              size_t ws_bytes, void* stream);

/* ttr_hybrid_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation). The workspace is a fixed array of
 * TTR_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU it runs
 * on until the process ends; the call itself allocates nothing. Arguments,
 * layouts and results are those of ttr_hybrid_forward. TTR_ERR_WORKSPACE when
 * ttr_workspace_bytes(d, L, causal, 0) exceeds TTR_NOALLOC_SCRATCH_BYTES.
 * Every call on one GPU uses that GPU's one array (the kernels clear what must
 * start at zero): calls that overlap on one GPU (other streams, other host
 * threads) race and give undefined results; calls in one stream are safe. */
#define TTR_NOALLOC_SCRATCH_BYTES (64u << 20)
ttr_status ttr_hybrid_forward_noalloc(ttr_dims d, const void* Q, const void* K, const void* V,
                                      const void* W, const float* b, const float* g, float eps,
                                      int32_t L, int32_t causal, void* out, void* stream);

/* Gradients of the hybrid forward (non-causal, elu + 1 map, projection W
 * required, 0 <= L <= N) for its trainable parameters, given
 * dout = dLoss/dout fp32 [B,H,N,D]:
 *   dW [H,D,F], db [H,F], dg [H], all fp32, summed over the batch (overwritten).
 * Chain rule through out = alpha lin + (1 - alpha) lm, alpha = sigmoid(g),
 * lin = phi(Q) KV / (phi(Q) . ksum + eps), phi = elu(x W + b) + 1; the landmark
 * branch holds no parameter and contributes through alpha only (dg = 0 when
 * L == 0). Gradients for Q, K, V are not computed.
 * "Flux2TTRTrainer", "How the distillation works" (the student layer that
 * Phase 1 trains); "NNT Define Linear Attention", "How it works" (the linear branch).
 * b may be NULL (zero bias; db is still written). g is needed when L > 0.
 * ws: at least ttr_backward_workspace_bytes(d, L) bytes (the intermediates: fp32,
 * with phi(z), dz and dnum in bf16 on the bf16 path). */
ttr_status ttr_hybrid_backward(ttr_dims d, const void* Q, const void* K, const void* V, const void* W,
                               const float* b, const float* g, float eps, int32_t L, const float* dout,
                               float* dW, float* db, float* dg, void* ws, size_t ws_bytes, void* stream);

/* Workspace size in bytes of ttr_hybrid_backward (0 if the shape is invalid). */
size_t ttr_backward_workspace_bytes(ttr_dims d, int32_t L);

/* One Phase-1 distillation step of a TTR layer on one batch of Q, K, V
 * ("Flux2TTRTrainer", "How the distillation works": the student TTR layer
 * regresses native softmax attention; huber and cosine terms weighed by
 * learned uncertainties after Kendall; optimizer state persists):
 *   teacher = softmax(Q K^T / sqrt(D)) V per (b, h) (computed when teacher is NULL)
 *   out     = the hybrid forward with W, b, g (W rounded to the IO dtype for it)
 *   loss    = exp(-s1) huber + s1 + exp(-s2) (1 - cos) + s2
 *             (huber with delta 1 averaged over every element; cos per (b, h, n)
 *             row over D, o.t / max(|o| |t|, 1e-8), averaged over rows)
 *   then Adam (beta1 0.9, beta2 0.999, eps 1e-8, bias-corrected at `step`,
 *   counted from 1, no weight decay) on W, b, g, s with the gradients of
 *   ttr_hybrid_backward and dloss/ds.
 * W [H,D,F], b [H,F], g [H], s [2]: fp32 master parameters, updated in place.
 * moments: fp32 Adam moments, 2 (H D F + H F + H + 2) values laid out
 * [mW vW mb vb mg vg ms vs], zero before step 1, updated in place.
 * teacher: fp32 [B,H,N,D] or NULL. loss: fp32 [3] device output (loss,
 * huber, 1 - cos) of the parameters before the update.
 * Shape rules as ttr_hybrid_backward (F == 256 with the projection).
 * ws: at least ttr_distill_workspace_bytes(d, L, teacher == NULL) bytes. */
ttr_status ttr_distill_step(ttr_dims d, const void* Q, const void* K, const void* V, const float* teacher,
                            float* W, float* b, float* g, float* s, float* moments, int32_t step, float lr,
                            float eps, int32_t L, float* loss, void* ws, size_t ws_bytes, void* stream);

/* Workspace size in bytes of ttr_distill_step (0 if the shape is invalid). */
size_t ttr_distill_workspace_bytes(ttr_dims d, int32_t L, int32_t compute_teacher);

/* The distillation step on a replay sample ("Flux2TTRTrainer", "How the
 * distillation works": the student is trained on replay samples, which keep
 * every key and value but only some query rows): as ttr_distill_step, with
 * Q [B,H,Nq,D] the sample's query rows (1 <= Nq <= d.N) over K, V [B,H,N,D]
 * (N = d.N keys; the landmarks stride over the keys), teacher [B,H,Nq,D] fp32
 * the teacher's output at those rows or NULL (then computed: softmax attention
 * of the Nq queries over all N keys). The loss averages over the B*H*Nq rows.
 * With Nq == d.N this is ttr_distill_step. */
ttr_status ttr_distill_step_rows(ttr_dims d, int32_t Nq, const void* Q, const void* K, const void* V,
                                 const float* teacher, float* W, float* b, float* g, float* s, float* moments,
                                 int32_t step, float lr, float eps, int32_t L, float* loss, void* ws, size_t ws_bytes,
                                 void* stream);

/* Workspace size in bytes of ttr_distill_step_rows (0 if the shape is invalid). */
size_t ttr_distill_rows_workspace_bytes(ttr_dims d, int32_t Nq, int32_t L, int32_t compute_teacher);

/* Cosine distance of a student's attention output to a teacher's: the mean
 * over the B*H*N rows of 1 - o.t / max(|o| |t|, 1e-8) (rows of D values),
 * written to out (one fp32 device value). student, teacher [B,H,N,D] in the
 * IO dtype. The quantity the readiness gate tracks ("Flux2TTRTrainer", "How
 * the distillation works": a moving average of the cosine distance to the teacher).
 * ws: at least ttr_cosine_workspace_bytes(d) bytes. */
ttr_status ttr_cosine_distance(ttr_dims d, const void* student, const void* teacher, float* out, void* ws,
                               size_t ws_bytes, void* stream);
size_t ttr_cosine_workspace_bytes(ttr_dims d);

/* Per-layer readiness gate, host only ("Flux2TTRTrainer", "How the
 * distillation works": fail-closed until enough updates and a low EMA cosine
 * distance, with hysteresis). A layer serves the student only while ready;
 * otherwise it keeps the teacher's attention.
 *   ema  = distance on the first update, then ema_rate ema + (1 - ema_rate) distance
 *   not ready -> ready  when updates >= min_updates and ema <= threshold_on
 *   ready -> not ready  when ema > threshold_off (threshold_off >= threshold_on)
 * A zero-initialised state is a fresh, not-ready gate. A non-finite distance
 * makes the gate not ready, leaves ema and updates unchanged and returns
 * TTR_ERR_SHAPE; an invalid config (0 <= ema_rate < 1, 0 <= threshold_on <=
 * threshold_off, min_updates >= 0) returns TTR_ERR_SHAPE and changes nothing. */
typedef struct {
  double ema_rate, threshold_on, threshold_off;
  int32_t min_updates;
} ttr_gate_config;
typedef struct {
  double ema;
  int32_t updates;
  int32_t ready;
} ttr_gate_state;
ttr_status ttr_gate_update(const ttr_gate_config* cfg, ttr_gate_state* st, double distance);

/* Landmark count from the trainer's fraction/min/max knobs ("Flux2TTRTrainer",
 * "Inputs worth setting"): round-half-up(fraction * N) clamped to [lmin, lmax]
 * and to N. Returns -1 for N < 0, fraction < 0 or lmax < lmin (or lmin < 0). */
int32_t ttr_landmark_count(int32_t N, double fraction, int32_t lmin, int32_t lmax);

/* Sizes of the NNT linear-attention layer: x [B,N,E] (batch first), H heads of D = E / H. */
typedef struct {
  int32_t B, N, E, H;
  int32_t dtype; /* ttr_dtype of x, the weights and out */
  int32_t fmap;  /* ttr_fmap of the attention; 0 (elu + 1) when zero-initialised */
} ttr_layer_dims;

/* NNT linear-attention layer, inference forward (dropout is the identity):
 *   Q = x Wq + bq, K = x Wk + bk, V = x Wv + bv    (W* [E,E] in the IO dtype,
 *                                                   input rows, output columns; b* [E] fp32 or NULL)
 *   head h takes columns h*D .. h*D + D - 1; per head the linear attention of
 *   ttr_hybrid_forward with W == NULL, b == NULL, L == 0 (causal: that of
 *   ttr_causal_scan), feature map d.fmap;
 *   out = merged heads . Wo + bo                  ([B,N,E], IO dtype).
 * "NNT Define Linear Attention", "The inputs" (embed_dim, num_heads,
 * feature_map, eps, causal, batch_first) and "How it works" (project Q/K/V,
 * feature map, K'^T V first, normalise, project back out).
 * Shape rules: B, N, H >= 1; E % 128 == 0; E % H == 0; D = E / H in {64, 128}
 * B*N*E < 2^31; B*H <= 65535.
 * ws: at least ttr_nnt_layer_workspace_bytes(d, causal) bytes (transposed
 * weights, Q/K/V and the attention output in [B,H,N,D], and the attention's
 * own workspace); its contents on entry do not matter. */
ttr_status ttr_nnt_layer_forward(ttr_layer_dims d, const void* x, const void* Wq, const float* bq,
                                 const void* Wk, const float* bk, const void* Wv, const float* bv,
                                 const void* Wo, const float* bo, float eps, int32_t causal, void* out,
                                 void* ws, size_t ws_bytes, void* stream);

/* Workspace size in bytes of ttr_nnt_layer_forward (0 if the shape is invalid). */
size_t ttr_nnt_layer_workspace_bytes(ttr_layer_dims d, int32_t causal);

/* Workspace size in bytes for the given call shape (0 if the shape is invalid).
 * causal takes the values ttr_hybrid_forward accepts; chunk, when non-zero,
 * names the causal chunk instead (ttr_causal_scan's argument). */
size_t ttr_workspace_bytes(ttr_dims d, int32_t L, int32_t causal, int32_t chunk);

/* Static, never-NULL description of a status code. */
const char* ttr_status_string(ttr_status st);

/* ------------------------------------------------------------------------
 * Replay buffer ("Flux2TTRTrainer", "How the distillation works": samples keep
 * full keys and values but subsampled queries, offloaded to CPU memory within
 * a budget, 768 MB by default; "The honest gotchas": replay offloads to the CPU
 * by default).
 *
 * Unlike the stateless calls above, a ttr_replay object owns memory: a ring of
 * pinned host memory (hipHostMalloc) of budget_bytes + max_sample_bytes, a
 * device staging area of max_sample_bytes, and one side stream of the device current at ttr_replay_create (default
 * priority, non-blocking). Every later call must be made with that device
 * current (else TTR_ERR_DEVICE). Calls on one object are serialised by a
 * lock; calls on different objects are independent.
 *
 * A sample of one layer call holds K, V [B,H,N,D] whole, the query rows
 * Q[:, :, q_index] [B,H,Nq,D] (IO dtype), optionally the teacher's fp32
 * output rows at the same q_index [B,H,Nq,D], and q_index itself (int32 [Nq],
 * strictly increasing in [0, N)). Each of these arrays takes its size rounded
 * up to 256 bytes from the budget (ttr_replay_sample_bytes). A push that would
 * exceed the budget first evicts the oldest samples (FIFO) until the new one
 * fits, so the samples held are always the longest run of most recent pushes
 * that fits the budget; the extra max_sample_bytes of the ring are slack that
 * lets a contiguous placement always be found, so placement never evicts
 * more. Sample ids count accepted pushes from 0.
 * ------------------------------------------------------------------------ */
typedef struct ttr_replay ttr_replay;

typedef struct {
  int32_t count;      /* samples held */
  int64_t first_id;   /* id of the oldest sample held (-1 when empty) */
  int64_t pushed;     /* accepted pushes so far */
  int64_t evicted;    /* samples evicted so far */
  size_t bytes_used;  /* sum of the held samples' footprints (<= budget_bytes) */
  size_t budget_bytes, max_sample_bytes, ring_bytes;
} ttr_replay_stats;

/* Budget footprint in bytes of one sample (0 if the shape is invalid): dims
 * d (F ignored, taken as D), Nq query rows, with or without teacher rows. */
size_t ttr_replay_sample_bytes(ttr_dims d, int32_t Nq, int32_t with_teacher);

/* Create a replay buffer on the current device. budget_bytes >= 256;
 * 256 <= max_sample_bytes <= budget_bytes bounds every later push. *out
 * receives the object (NULL on failure). TTR_ERR_HIP when the pinned ring or
 * the stream cannot be created. */
ttr_status ttr_replay_create(size_t budget_bytes, size_t max_sample_bytes, ttr_replay** out);

/* Wait for every copy the object enqueued, then free its ring, events and
 * stream. NULL is a no-op. */
void ttr_replay_destroy(ttr_replay* rb);

/* Push one sample. Q, K, V: device [B,H,N,D] in the IO dtype; teacher: device
 * fp32 [B,H,N,D] or NULL; q_index: HOST int32 [Nq] (copied before returning).
 * The copies run on the object's side stream after the work already enqueued
 * on `stream`: a kernel gathers the Q and teacher rows into the object's
 * device staging area, then DMA copies move them, K and V into the ring. The
 * caller must
 * not modify Q, K, V or teacher until ttr_replay_wait_pushed (or
 * ttr_replay_synchronize) has ordered its later work after the copies.
 * *id_out receives the sample's id. TTR_ERR_BUDGET when the footprint exceeds
 * budget_bytes or max_sample_bytes (nothing changes); TTR_ERR_SHAPE for Nq
 * outside [1, N] or an index list that is not strictly increasing in [0, N). */
ttr_status ttr_replay_push(ttr_replay* rb, ttr_dims d, int32_t Nq, const void* Q, const void* K, const void* V,
                           const float* teacher, const int32_t* q_index, void* stream, int64_t* id_out);

/* Make `stream` wait for the copies of every push enqueued so far (after
 * which the pushed inputs may be reused by work on that stream). */
ttr_status ttr_replay_wait_pushed(ttr_replay* rb, void* stream);

/* Block the host until every push's copies have finished. */
ttr_status ttr_replay_synchronize(ttr_replay* rb);

/* Copy sample `id` back to device memory on `stream` (which first waits for
 * the sample's own push): Qs [B,H,Nq,D] and K, V [B,H,N,D] in the IO dtype,
 * teacher rows fp32 [B,H,Nq,D] (NULL to skip; a non-NULL pointer for a sample
 * without teacher rows is TTR_ERR_SHAPE), q_index host int32 [Nq] (NULL to
 * skip; filled before returning). The sample's ring space is not reused
 * until these copies have finished. TTR_ERR_NOT_FOUND for an id not held. */
ttr_status ttr_replay_fetch(ttr_replay* rb, int64_t id, void* Qs, void* K, void* V, float* teacher_rows,
                            int32_t* q_index, void* stream);

/* Shape of sample `id`: *d (F = D), *Nq, *has_teacher (each pointer may be NULL). */
ttr_status ttr_replay_info(ttr_replay* rb, int64_t id, ttr_dims* d, int32_t* Nq, int32_t* has_teacher);

/* Counters of the object (see ttr_replay_stats). */
ttr_status ttr_replay_get_stats(ttr_replay* rb, ttr_replay_stats* out);

/* hipError_t of the last TTR_ERR_HIP returned on the calling thread (0 if none). */
int ttr_last_hip_error(void);

/* Per-kernel timing for profilers and benchmarks. After this call, the
 * calling thread's next ttr_hybrid_forward, ttr_causal_scan,
 * ttr_nnt_layer_forward, ttr_hybrid_backward, ttr_distill_step (or _rows),
 * ttr_cosine_distance or ttr_replay_push records
 * events[0] on its stream before its first kernel and events[1], events[2],
 * ... after each kernel (or stage) it launches, as long as events remain:
 *   bf16 hybrid: the key/value stage (partials, split reduction and operand
 *     pack in one launch), the fused query kernel;
 *   fp32 hybrid: key/value reduction, query kernel;
 *   causal, bf16 with D = 64: the reset of its segment flags, the single-pass scan;
 *   other causal: segment totals (when the sequence has several segments), chunk walk;
 *   layer: the weight transposes, Q/K/V projection, the attention's stages
 *     as above, out projection;
 *   backward: Q projection, K projection (one stage each, whatever the batch),
 *     KV and ksum (bf16: one stage, from K and V; fp32: ksum, then KV), num,
 *     normaliser, landmark branch (L > 0), then dnum/dden,
 *     dz_q (its product with the phi' factor in the epilogue), dKV, dks, dz_k
 *     (likewise), dW from Q, dW from K, db/dg;
 *   distillation step: W to bf16 (bf16 IO), teacher (when computed), the
 *     backward's forward stages, loss rows with dnum/dden, loss total, the
 *     backward's gradient stages after dnum/dden, Adam;
 *   cosine distance: per-workgroup partial sums, total;
 *   replay push (on the replay object's side stream): the row gather, the
 *     rows' copy, K's copy, V's copy.
 * Events left over are recorded after the last kernel. The registration is
 * consumed by that one call. events holds n hipEvent_t handles created by the
 * caller; NULL clears the registration. The events only observe: the enqueued
 * kernels and results are the same with or without them. */
void ttr_set_stage_events(void* const* events, int32_t n);

/* Library version string, e.g. "ttr 0.1.0 gfx950". */
const char* ttr_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TTR_H */

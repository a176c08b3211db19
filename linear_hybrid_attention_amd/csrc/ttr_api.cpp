// C ABI of libttr.so: validation on the host, then kernel launches on the
// caller's stream. Declarations and conventions: include/ttr.h.
#include <hip/hip_runtime.h>

#include "../../include/ttr.h"
#include "launch.hpp"
#include "validate.hpp"

using namespace ttr;

namespace {

thread_local int g_last_hip_error = 0;
thread_local void* const* g_stage_events = nullptr;
thread_local int g_stage_n = 0;

}  // namespace

// Take (and clear) the calling thread's registered stage events; record the first.
StageTimer ttr::take_stage_timer(hipStream_t s) {
  StageTimer t;
  t.ev = g_stage_events;
  t.n = g_stage_n;
  t.s = s;
  g_stage_events = nullptr;
  g_stage_n = 0;
  t.mark();
  return t;
}

namespace {

ttr_status hip_status(hipError_t e) {
  if (e == hipSuccess) return TTR_OK;
  g_last_hip_error = (int)e;
  return TTR_ERR_HIP;
}

Problem make_problem(const ttr_dims& d, bool proj) {
  Problem p;
  p.B = d.B;
  p.H = d.H;
  p.N = d.N;
  p.D = d.D;
  p.F = d.F;
  p.dtype = d.dtype;
  p.proj = proj;
  p.fmap = d.fmap;
  p.Nq = d.N;
  return p;
}

size_t io(const ttr_dims& d) { return dtype_bytes(d.dtype); }
size_t qkv_bytes(const ttr_dims& d) { return (size_t)d.B * d.H * d.N * d.D * io(d); }
size_t w_bytes(const ttr_dims& d) { return (size_t)d.H * d.D * d.F * io(d); }
size_t b_bytes(const ttr_dims& d) { return (size_t)d.H * d.F * sizeof(float); }
size_t kv_bytes(const ttr_dims& d) { return (size_t)d.B * d.H * d.F * d.D * sizeof(float); }
size_t ks_bytes(const ttr_dims& d) { return (size_t)d.B * d.H * d.F * sizeof(float); }
size_t f32_out_bytes(const ttr_dims& d) { return (size_t)d.B * d.H * d.N * d.D * sizeof(float); }

#define TTR_TRY(expr)                    \
  do {                                   \
    const ttr_status st_ = (expr);       \
    if (st_ != TTR_OK) return st_;       \
  } while (0)

// Bytes the hybrid forward needs. bf16: split partials + operand pack of the
// fused query kernel; fp32: KV/ksum (fp32) plus the split partials.
size_t hybrid_ws(const ttr_dims& d, bool proj, int32_t L) {
  const Problem p = make_problem(d, proj);
  if (d.dtype == TTR_BF16) return fused_workspace_bytes(p, L);
  return kv_bytes(d) + ks_bytes(d) + kv_workspace_bytes(p);
}

}  // namespace

ttr_status ttr::report_hip(hipError_t e) { return hip_status(e); }

extern "C" {

const char* ttr_status_string(ttr_status st) {
  switch (st) {
    case TTR_OK: return "ok";
    case TTR_ERR_NULL: return "a required pointer is NULL";
    case TTR_ERR_SHAPE: return "invalid shape (B, H, N, D, F, L or chunk)";
    case TTR_ERR_DTYPE: return "unknown dtype";
    case TTR_ERR_UNSUPPORTED: return "valid request not supported by this library";
    case TTR_ERR_WORKSPACE: return "workspace missing or too small";
    case TTR_ERR_ALIGN: return "pointer not 16-byte aligned";
    case TTR_ERR_HIP: return "HIP launch failed";
    case TTR_ERR_ALIAS: return "an output overlaps an input";
    case TTR_ERR_BUDGET: return "replay sample larger than the budget or the maximum sample size";
    case TTR_ERR_NOT_FOUND: return "replay sample id not held";
    case TTR_ERR_DEVICE: return "called with another device current than at create";
  }
  return "unknown status";
}

int ttr_last_hip_error(void) { return g_last_hip_error; }

const char* ttr_version(void) { return "ttr 0.1.0 gfx950"; }

void ttr_set_stage_events(void* const* events, int32_t n) {
  g_stage_events = (events != nullptr && n >= 1) ? events : nullptr;
  g_stage_n = g_stage_events ? n : 0;
}

// The causal chunk a `causal` argument of ttr_hybrid_forward names: 1 is the
// default chunk, 64 / 128 / 256 that chunk; 0 for any other value.
static int32_t causal_chunk_of(const ttr_dims& d, int32_t causal) {
  if (causal == 1) return causal_default_chunk(d.dtype, d.D);
  if (causal == 64 || causal == 128 || causal == 256) return causal;
  return 0;
}

size_t ttr_workspace_bytes(ttr_dims d, int32_t L, int32_t causal, int32_t chunk) {
  if (causal) {
    if (d.F != d.D || check_dims(d, false) != TTR_OK) return 0;
    if (chunk == 0) chunk = causal_chunk_of(d, causal);
    if (!causal_chunk_ok(d.dtype, d.D, chunk)) return 0;
    return causal_workspace_bytes(make_problem(d, false), chunk);
  }
  const bool proj = d.F != d.D;
  if (check_dims(d, proj, forward_max_f(d)) != TTR_OK || L < 0 || L > d.N) return 0;
  return hybrid_ws(d, proj, L);
}

ttr_status ttr_feature_map(ttr_dims d, const void* X, const void* W, const float* b, void* phi,
                           void* stream) {
  const bool proj = W != nullptr;
  TTR_TRY(check_dims(d, proj));
  TTR_TRY(check_ptr(X));
  TTR_TRY(check_ptr(phi));
  TTR_TRY(check_opt_ptr(W));
  TTR_TRY(check_opt_ptr(b));
  const Range outs[] = {{phi, (size_t)d.B * d.H * d.N * d.F * io(d)}};
  const Range ins[] = {{X, qkv_bytes(d)}, {W, proj ? w_bytes(d) : 0}, {b, b ? b_bytes(d) : 0}};
  TTR_TRY(check_no_alias(outs, 1, ins, 3));
  HybridArgs a = {};
  a.Q = X;
  a.W = W;
  a.bias = b;
  a.H = d.H;
  a.N = d.N;
  a.out = phi;
  return hip_status(launch_hybrid(make_problem(d, proj), M_PHI, true, a, (hipStream_t)stream));
}

ttr_status ttr_kv_reduce(ttr_dims d, const void* K, const void* V, const void* W, const float* b, float* KV,
                         float* ksum, void* ws, size_t ws_bytes, void* stream) {
  const bool proj = W != nullptr;
  TTR_TRY(check_dims(d, proj));
  TTR_TRY(check_ptr(K));
  TTR_TRY(check_ptr(V));
  TTR_TRY(check_ptr(KV));
  TTR_TRY(check_ptr(ksum));
  TTR_TRY(check_opt_ptr(W));
  TTR_TRY(check_opt_ptr(b));
  const Problem p = make_problem(d, proj);
  // bf16: the fused path's partial kernel, then a fixed-order sum; fp32: the generic kernels
  const bool fast = d.dtype == TTR_BF16;
  const size_t need = fast ? kv2_reduce_workspace_bytes(p) : kv_workspace_bytes(p);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return TTR_ERR_WORKSPACE;
    TTR_TRY(check_ptr(ws));
  }
  const Range outs[] = {{KV, kv_bytes(d)}, {ksum, ks_bytes(d)}, {ws, need}};
  const Range ins[] = {{K, qkv_bytes(d)}, {V, qkv_bytes(d)}, {W, proj ? w_bytes(d) : 0}, {b, b ? b_bytes(d) : 0}};
  TTR_TRY(check_no_alias(outs, 3, ins, 4));
  if (fast) return hip_status(launch_kv2_reduce(p, K, V, W, b, KV, ksum, ws, (hipStream_t)stream));
  return hip_status(launch_kv_reduce(p, K, V, W, b, KV, ksum, ws, (hipStream_t)stream));
}

ttr_status ttr_apply(ttr_dims d, const void* Q, const void* W, const float* b, const float* KV,
                     const float* ksum, float eps, float* out_lin, void* stream) {
  const bool proj = W != nullptr;
  TTR_TRY(check_dims(d, proj));
  TTR_TRY(check_ptr(Q));
  TTR_TRY(check_ptr(KV));
  TTR_TRY(check_ptr(ksum));
  TTR_TRY(check_ptr(out_lin));
  TTR_TRY(check_opt_ptr(W));
  TTR_TRY(check_opt_ptr(b));
  const Range outs[] = {{out_lin, f32_out_bytes(d)}};
  const Range ins[] = {{Q, qkv_bytes(d)}, {W, proj ? w_bytes(d) : 0}, {b, b ? b_bytes(d) : 0},
                       {KV, kv_bytes(d)}, {ksum, ks_bytes(d)}};
  TTR_TRY(check_no_alias(outs, 1, ins, 5));
  HybridArgs a = {};
  a.Q = Q;
  a.W = W;
  a.bias = b;
  a.KV = KV;
  a.ksum = ksum;
  a.eps = eps;
  a.H = d.H;
  a.N = d.N;
  a.out = out_lin;
  return hip_status(launch_hybrid(make_problem(d, proj), M_LIN, false, a, (hipStream_t)stream));
}

ttr_status ttr_landmark_attn(ttr_dims d, const void* Q, const void* K, const void* V, int32_t L, float* out_lm,
                             void* stream) {
  TTR_TRY(check_dims(d, d.F != d.D));
  if (L < 1 || L > d.N) return TTR_ERR_SHAPE;
  TTR_TRY(check_ptr(Q));
  TTR_TRY(check_ptr(K));
  TTR_TRY(check_ptr(V));
  TTR_TRY(check_ptr(out_lm));
  const Range outs[] = {{out_lm, f32_out_bytes(d)}};
  const Range ins[] = {{Q, qkv_bytes(d)}, {K, qkv_bytes(d)}, {V, qkv_bytes(d)}};
  TTR_TRY(check_no_alias(outs, 1, ins, 3));
  HybridArgs a = {};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.H = d.H;
  a.N = d.N;
  a.L = L;
  a.out = out_lm;
  return hip_status(launch_hybrid(make_problem(d, false), M_LM, false, a, (hipStream_t)stream));
}

ttr_status ttr_blend(ttr_dims d, const float* out_lin, const float* out_lm, const float* g, void* out,
                     void* stream) {
  TTR_TRY(check_dims(d, d.F != d.D));
  TTR_TRY(check_ptr(out_lin));
  TTR_TRY(check_ptr(out_lm));
  TTR_TRY(check_ptr(g));
  TTR_TRY(check_ptr(out));
  const Range outs[] = {{out, qkv_bytes(d)}};
  const Range ins[] = {{out_lin, f32_out_bytes(d)}, {out_lm, f32_out_bytes(d)}, {g, (size_t)d.H * sizeof(float)}};
  TTR_TRY(check_no_alias(outs, 1, ins, 3));
  return hip_status(launch_blend(make_problem(d, false), out_lin, out_lm, g, out, (hipStream_t)stream));
}

// The bodies of ttr_causal_scan and ttr_hybrid_forward. `outer` is the
// stage timer of an enclosing entry point (the layer), or NULL: then the call
// takes the thread's registration itself, after validation, and finishes it.
static ttr_status causal_scan_impl(ttr_dims d, const void* Q, const void* K, const void* V, const void* W,
                                   const float* b, float eps, int32_t chunk, void* out, void* ws, size_t ws_bytes,
                                   hipStream_t s, StageTimer* outer) {
  if (dtype_bytes(d.dtype) == 0) return TTR_ERR_DTYPE;
  if (W != nullptr) return TTR_ERR_UNSUPPORTED;  // the causal variant has no projection
  TTR_TRY(check_dims(d, false));
  TTR_TRY(check_causal(d, W, 0, chunk));
  TTR_TRY(check_ptr(Q));
  TTR_TRY(check_ptr(K));
  TTR_TRY(check_ptr(V));
  TTR_TRY(check_ptr(out));
  TTR_TRY(check_opt_ptr(b));
  const Problem p = make_problem(d, false);
  const size_t need = causal_workspace_bytes(p, chunk);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return TTR_ERR_WORKSPACE;
    TTR_TRY(check_ptr(ws));
  }
  const Range outs[] = {{out, qkv_bytes(d)}, {ws, need}};
  const Range ins[] = {{Q, qkv_bytes(d)}, {K, qkv_bytes(d)}, {V, qkv_bytes(d)}, {b, b ? b_bytes(d) : 0}};
  TTR_TRY(check_no_alias(outs, 2, ins, 4));
  StageTimer own;
  StageTimer* t = outer;
  if (t == nullptr) {
    own = take_stage_timer(s);
    t = &own;
  }
  const ttr_status st = hip_status(causal2_supported(p, chunk)
                                       ? launch_causal2(p, Q, K, V, b, eps, chunk, out, ws, s, t)
                                       : launch_causal(p, Q, K, V, b, eps, chunk, out, ws, s, t));
  if (outer == nullptr) t->finish();
  return st;
}

static ttr_status hybrid_forward_impl(ttr_dims d, const void* Q, const void* K, const void* V, const void* W,
                                      const float* b, const float* g, float eps, int32_t L, int32_t causal,
                                      void* out, void* ws, size_t ws_bytes, hipStream_t s, StageTimer* outer) {
  if (causal) {
    if (dtype_bytes(d.dtype) == 0) return TTR_ERR_DTYPE;
    if (W != nullptr || L != 0) return TTR_ERR_UNSUPPORTED;
    TTR_TRY(check_dims(d, false));
    if (causal != 1 && causal != 64 && causal != 128 && causal != 256) return TTR_ERR_SHAPE;
    const int32_t chunk = causal_chunk_of(d, causal);
    if (chunk == 0) return TTR_ERR_UNSUPPORTED;
    return causal_scan_impl(d, Q, K, V, W, b, eps, chunk, out, ws, ws_bytes, s, outer);
  }
  const bool proj = W != nullptr;
  TTR_TRY(check_dims(d, proj, forward_max_f(d)));
  if (L < 0 || L > d.N) return TTR_ERR_SHAPE;
  if (d.fmap != TTR_FMAP_ELU1 && L > 0) return TTR_ERR_UNSUPPORTED;  // landmarks belong to the elu+1 TTR layer
  TTR_TRY(check_ptr(Q));
  TTR_TRY(check_ptr(K));
  TTR_TRY(check_ptr(V));
  TTR_TRY(check_ptr(out));
  TTR_TRY(check_opt_ptr(W));
  TTR_TRY(check_opt_ptr(b));
  if (L > 0) TTR_TRY(check_ptr(g));
  const Problem p = make_problem(d, proj);
  const size_t need = hybrid_ws(d, proj, L);
  if (ws == nullptr || ws_bytes < need) return TTR_ERR_WORKSPACE;
  TTR_TRY(check_ptr(ws));
  const Range outs[] = {{out, qkv_bytes(d)}, {ws, need}};
  const Range ins[] = {{Q, qkv_bytes(d)}, {K, qkv_bytes(d)}, {V, qkv_bytes(d)}, {W, proj ? w_bytes(d) : 0},
                       {b, b ? b_bytes(d) : 0}, {g, (L > 0) ? (size_t)d.H * sizeof(float) : 0}};
  TTR_TRY(check_no_alias(outs, 2, ins, 6));

  StageTimer own;
  StageTimer* t = outer;
  if (t == nullptr) {
    own = take_stage_timer(s);
    t = &own;
  }
  if (d.dtype == TTR_BF16) {
    // split-N key/value reduction + operand pack, then the fused query kernel
    FusedPack pk;
    TTR_TRY(hip_status(launch_kv2(p, K, V, W, b, L, ws, &pk, s, t)));
    const ttr_status st = hip_status(launch_fused_query(p, Q, pk, g, eps, L, out, s));
    t->mark();
    if (outer == nullptr) t->finish();
    return st;
  }
  // fp32: KV [B,H,F,D] fp32 | ksum [B,H,F] fp32 | split partials, then the generic query kernel
  float* KV = static_cast<float*>(ws);
  float* ksum = KV + (size_t)d.B * d.H * d.F * d.D;
  void* part = ksum + (size_t)d.B * d.H * d.F;
  TTR_TRY(hip_status(launch_kv_reduce(p, K, V, W, b, KV, ksum, part, s)));
  t->mark();
  HybridArgs a = {};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.W = W;
  a.bias = b;
  a.KV = KV;
  a.ksum = ksum;
  a.g = g;
  a.eps = eps;
  a.H = d.H;
  a.N = d.N;
  a.L = L;
  a.out = out;
  const ttr_status st = hip_status(launch_hybrid(p, L > 0 ? (M_LIN | M_LM) : M_LIN, true, a, s));
  t->mark();
  if (outer == nullptr) t->finish();
  return st;
}

ttr_status ttr_causal_scan(ttr_dims d, const void* Q, const void* K, const void* V, const void* W, const float* b,
                           float eps, int32_t chunk, void* out, void* ws, size_t ws_bytes, void* stream) {
  return causal_scan_impl(d, Q, K, V, W, b, eps, chunk, out, ws, ws_bytes, (hipStream_t)stream, nullptr);
}

ttr_status ttr_hybrid_forward(ttr_dims d, const void* Q, const void* K, const void* V, const void* W,
                              const float* b, const float* g, float eps, int32_t L, int32_t causal, void* out,
                              void* ws, size_t ws_bytes, void* stream) {
  return hybrid_forward_impl(d, Q, K, V, W, b, g, eps, L, causal, out, ws, ws_bytes, (hipStream_t)stream, nullptr);
}

// ---------------------------------------------------------------- NNT layer
// Workspace: Wqkv^T [3E][E] | Wo^T [E][E] | Q | K | V | attention out (each
// [B,H,N,D]) | the attention's workspace; regions 256-byte aligned.
static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t ttr_nnt_layer_workspace_bytes(ttr_layer_dims d, int32_t causal) {
  ttr_dims c;
  if (check_layer(d, &c) != TTR_OK) return 0;
  const size_t es = dtype_bytes(d.dtype), E = (size_t)d.E, act = (size_t)d.B * d.N * E * es;
  return align256(3 * E * E * es) + align256(E * E * es) + 4 * align256(act) +
         ttr_workspace_bytes(c, 0, causal ? 1 : 0, 0);
}

ttr_status ttr_nnt_layer_forward(ttr_layer_dims d, const void* x, const void* Wq, const float* bq, const void* Wk,
                                 const float* bk, const void* Wv, const float* bv, const void* Wo, const float* bo,
                                 float eps, int32_t causal, void* out, void* ws, size_t ws_bytes, void* stream) {
  ttr_dims c;
  TTR_TRY(check_layer(d, &c));
  if (causal && causal_default_chunk(c.dtype, c.D) == 0) return TTR_ERR_UNSUPPORTED;
  TTR_TRY(check_ptr(x));
  TTR_TRY(check_ptr(Wq));
  TTR_TRY(check_ptr(Wk));
  TTR_TRY(check_ptr(Wv));
  TTR_TRY(check_ptr(Wo));
  TTR_TRY(check_ptr(out));
  TTR_TRY(check_opt_ptr(bq));
  TTR_TRY(check_opt_ptr(bk));
  TTR_TRY(check_opt_ptr(bv));
  TTR_TRY(check_opt_ptr(bo));
  const size_t need = ttr_nnt_layer_workspace_bytes(d, causal);
  if (ws == nullptr || ws_bytes < need) return TTR_ERR_WORKSPACE;
  TTR_TRY(check_ptr(ws));
  const size_t es = dtype_bytes(d.dtype), E = (size_t)d.E, act = (size_t)d.B * d.N * E * es;
  const size_t wb = E * E * es, bb = E * sizeof(float);
  const Range outs[] = {{out, act}, {ws, need}};
  const Range ins[] = {{x, act}, {Wq, wb}, {Wk, wb}, {Wv, wb}, {Wo, wb},
                       {bq, bq ? bb : 0}, {bk, bk ? bb : 0}, {bv, bv ? bb : 0}, {bo, bo ? bb : 0}};
  TTR_TRY(check_no_alias(outs, 2, ins, 9));

  unsigned char* w8 = static_cast<unsigned char*>(ws);
  void* wqkv_t = w8;
  w8 += align256(3 * wb);
  void* wo_t = w8;
  w8 += align256(wb);
  void* qkv[3];
  for (int i = 0; i < 3; ++i) {
    qkv[i] = w8;
    w8 += align256(act);
  }
  void* attn = w8;
  w8 += align256(act);
  void* core_ws = w8;
  const size_t core_bytes = need - (size_t)(w8 - static_cast<unsigned char*>(ws));

  hipStream_t s = (hipStream_t)stream;
  StageTimer t = take_stage_timer(s);  // stages: transposes, QKV projection, attention kernels, out projection
  const int M = d.B * d.N, D = c.D;
  const void* wsrc[4] = {Wq, Wk, Wv, Wo};
  void* wdst[4] = {wqkv_t, static_cast<unsigned char*>(wqkv_t) + wb, static_cast<unsigned char*>(wqkv_t) + 2 * wb,
                   wo_t};
  TTR_TRY(hip_status(launch_wt_transpose(d.dtype, wsrc, wdst, 4, d.E, s)));
  t.mark();
  const float* bqkv[3] = {bq, bk, bv};
  TTR_TRY(hip_status(launch_proj_gemm(d.dtype, false, true, x, wqkv_t, bqkv, qkv, M, d.E, 3 * d.E, d.N, d.H, D,
                                      d.E, s)));
  t.mark();
  TTR_TRY(hybrid_forward_impl(c, qkv[0], qkv[1], qkv[2], nullptr, nullptr, nullptr, eps, 0, causal ? 1 : 0, attn,
                              core_ws, core_bytes, s, &t));
  const float* bo3[3] = {bo, nullptr, nullptr};
  void* out3[3] = {out, nullptr, nullptr};
  const ttr_status st = hip_status(
      launch_proj_gemm(d.dtype, true, false, attn, wo_t, bo3, out3, M, d.E, d.E, d.N, d.H, D, d.E, s));
  t.finish();
  return st;
}

// ---------------------------------------------------------------- backward
static ttr_status check_backward(const ttr_dims& d, int32_t L) {
  TTR_TRY(check_dims(d, true));
  if (d.fmap != TTR_FMAP_ELU1) return TTR_ERR_UNSUPPORTED;
  if (L < 0 || L > d.N) return TTR_ERR_SHAPE;
  return TTR_OK;
}

size_t ttr_backward_workspace_bytes(ttr_dims d, int32_t L) {
  if (check_backward(d, L) != TTR_OK) return 0;
  return backward_layout(make_problem(d, true)).bytes;
}

ttr_status ttr_hybrid_backward(ttr_dims d, const void* Q, const void* K, const void* V, const void* W, const float* b,
                               const float* g, float eps, int32_t L, const float* dout, float* dW, float* db,
                               float* dg, void* ws, size_t ws_bytes, void* stream) {
  TTR_TRY(check_backward(d, L));
  TTR_TRY(check_ptr(Q));
  TTR_TRY(check_ptr(K));
  TTR_TRY(check_ptr(V));
  TTR_TRY(check_ptr(W));
  TTR_TRY(check_ptr(dout));
  TTR_TRY(check_ptr(dW));
  TTR_TRY(check_ptr(db));
  TTR_TRY(check_ptr(dg));
  TTR_TRY(check_opt_ptr(b));
  if (L > 0) TTR_TRY(check_ptr(g));
  const Problem p = make_problem(d, true);
  const size_t need = backward_layout(p).bytes;
  if (ws == nullptr || ws_bytes < need) return TTR_ERR_WORKSPACE;
  TTR_TRY(check_ptr(ws));
  const Range outs[] = {{dW, (size_t)d.H * d.D * d.F * 4}, {db, (size_t)d.H * d.F * 4}, {dg, (size_t)d.H * 4},
                        {ws, need}};
  const Range ins[] = {{Q, qkv_bytes(d)}, {K, qkv_bytes(d)}, {V, qkv_bytes(d)}, {W, w_bytes(d)},
                       {b, b ? b_bytes(d) : 0}, {g, g ? (size_t)d.H * 4 : 0}, {dout, f32_out_bytes(d)}};
  TTR_TRY(check_no_alias(outs, 4, ins, 7));
  hipStream_t st = (hipStream_t)stream;
  StageTimer t = take_stage_timer(st);
  const ttr_status r = hip_status(launch_hybrid_backward(p, Q, K, V, W, b, g, eps, L, dout, dW, db, dg, ws, st, &t));
  t.finish();
  return r;
}

size_t ttr_distill_workspace_bytes(ttr_dims d, int32_t L, int32_t compute_teacher) {
  return ttr_distill_rows_workspace_bytes(d, d.N, L, compute_teacher);
}

size_t ttr_distill_rows_workspace_bytes(ttr_dims d, int32_t Nq, int32_t L, int32_t compute_teacher) {
  if (check_backward(d, L) != TTR_OK || Nq < 1 || Nq > d.N) return 0;
  Problem p = make_problem(d, true);
  p.Nq = Nq;
  return distill_layout(p, compute_teacher != 0).bytes;
}

ttr_status ttr_distill_step_rows(ttr_dims d, int32_t Nq, const void* Q, const void* K, const void* V,
                                 const float* teacher, float* W, float* b, float* g, float* s, float* moments,
                                 int32_t step, float lr, float eps, int32_t L, float* loss, void* ws, size_t ws_bytes,
                                 void* stream) {
  TTR_TRY(check_backward(d, L));
  if (Nq < 1 || Nq > d.N) return TTR_ERR_SHAPE;
  if (step < 1 || !(lr > 0.f) || !(lr < 1e30f)) return TTR_ERR_SHAPE;
  TTR_TRY(check_ptr(Q));
  TTR_TRY(check_ptr(K));
  TTR_TRY(check_ptr(V));
  TTR_TRY(check_opt_ptr(teacher));
  for (const void* ptr : {(const void*)W, (const void*)b, (const void*)g, (const void*)s, (const void*)moments,
                          (const void*)loss})
    TTR_TRY(check_ptr(ptr));
  Problem p = make_problem(d, true);
  p.Nq = Nq;
  const size_t need = distill_layout(p, teacher == nullptr).bytes;
  if (ws == nullptr || ws_bytes < need) return TTR_ERR_WORKSPACE;
  TTR_TRY(check_ptr(ws));
  const size_t nW = (size_t)d.H * d.D * d.F * 4, nb = (size_t)d.H * d.F * 4, ng = (size_t)d.H * 4;
  const size_t nm = 2 * (nW + nb + ng + 8);
  const size_t q_bytes = (size_t)d.B * d.H * Nq * d.D * io(d), rows_f32 = (size_t)d.B * d.H * Nq * d.D * 4;
  const Range outs[] = {{W, nW}, {b, nb}, {g, ng}, {s, 8}, {moments, nm}, {loss, 12}, {ws, need}};
  const Range ins[] = {{Q, q_bytes}, {K, qkv_bytes(d)}, {V, qkv_bytes(d)}, {teacher, teacher ? rows_f32 : 0}};
  TTR_TRY(check_no_alias(outs, 7, ins, 4));
  hipStream_t st = (hipStream_t)stream;
  StageTimer t = take_stage_timer(st);
  const ttr_status r = hip_status(
      launch_distill_step(p, Q, K, V, teacher, W, b, g, s, moments, step, lr, eps, L, loss, ws, st, &t));
  t.finish();
  return r;
}

ttr_status ttr_distill_step(ttr_dims d, const void* Q, const void* K, const void* V, const float* teacher, float* W,
                            float* b, float* g, float* s, float* moments, int32_t step, float lr, float eps, int32_t L,
                            float* loss, void* ws, size_t ws_bytes, void* stream) {
  return ttr_distill_step_rows(d, d.N, Q, K, V, teacher, W, b, g, s, moments, step, lr, eps, L, loss, ws, ws_bytes,
                               stream);
}

size_t ttr_cosine_workspace_bytes(ttr_dims d) {
  if (check_dims(d, false) != TTR_OK && check_dims(d, true) != TTR_OK) return 0;
  return cosine_workspace_bytes(make_problem(d, d.F != d.D));
}

ttr_status ttr_cosine_distance(ttr_dims d, const void* student, const void* teacher, float* out, void* ws,
                               size_t ws_bytes, void* stream) {
  if (dtype_bytes(d.dtype) == 0) return TTR_ERR_DTYPE;
  if (check_dims(d, false) != TTR_OK && check_dims(d, true) != TTR_OK) return TTR_ERR_SHAPE;
  TTR_TRY(check_ptr(student));
  TTR_TRY(check_ptr(teacher));
  TTR_TRY(check_ptr(out));
  const Problem p = make_problem(d, d.F != d.D);
  const size_t need = cosine_workspace_bytes(p);
  if (ws == nullptr || ws_bytes < need) return TTR_ERR_WORKSPACE;
  TTR_TRY(check_ptr(ws));
  const Range outs[] = {{out, 4}, {ws, need}};
  const Range ins[] = {{student, qkv_bytes(d)}, {teacher, qkv_bytes(d)}};
  TTR_TRY(check_no_alias(outs, 2, ins, 2));
  hipStream_t st = (hipStream_t)stream;
  StageTimer t = take_stage_timer(st);
  const ttr_status r = hip_status(launch_cosine_distance(p, student, teacher, out, ws, st, &t));
  t.finish();
  return r;
}

}  // extern "C"

// Internal launch interface between the C-ABI layer (ttr_api.cpp) and the
// kernel translation units. Shapes reaching these functions are validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ttr.h"

namespace ttr {

struct Problem {
  int B, H, N, D, F;
  int dtype;  // 0 = fp32, 1 = bf16
  bool proj;  // W present (F == 256) or identity map (F == D)
  int fmap;   // feature map: kElu1, kRelu or kSoftmax (the last two only without W)
  int Nq;     // query rows (a replay sample keeps fewer queries than keys); 0 means N
};

// Query rows of a problem: N unless the queries are a subsample of the N keys.
inline int query_rows(const Problem& p) { return p.Nq > 0 ? p.Nq : p.N; }

enum { M_PHI = 1, M_LIN = 2, M_LM = 4 };

// Optional per-kernel timing: records the next caller-provided event on the
// stream after each kernel launch (no-op without events).
struct StageTimer {
  void* const* ev = nullptr;
  int n = 0, i = 0;
  hipStream_t s = nullptr;
  void mark() {
    if (ev != nullptr && i < n) (void)hipEventRecord(static_cast<hipEvent_t>(ev[i++]), s);
  }
  void finish() {  // events not used by a kernel are recorded at the end
    while (ev != nullptr && i < n) mark();
  }
};

struct HybridArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* W;
  const float* bias;
  const float* KV;    // fp32 [B,H,F,D]
  const float* ksum;  // fp32 [B,H,F]
  const float* g;     // fp32 [H]
  float eps;
  int H, N, L;  // N keys (and queries unless Nq is set)
  void* out;
  int Nq;       // query rows when they differ from the keys' N (0: N)
};

// k_hybrid.hip: feature map / apply / landmark / fused apply+landmark+blend.
// out_io selects the IO dtype (instead of fp32) for the M_LIN output.
hipError_t launch_hybrid(const Problem& p, int mode, bool out_io, const HybridArgs& a, hipStream_t s);

// k_kv.hip: KV = phi(K)^T V and ksum over split token ranges, then a
// fixed-order sum of the partials.
int kv_nsplit(const Problem& p);
size_t kv_workspace_bytes(const Problem& p);
hipError_t launch_kv_reduce(const Problem& p, const void* K, const void* V, const void* W,
                            const float* bias, float* KV, float* ksum, void* ws, hipStream_t s);
// Fixed-order sum of split partials [B*H][nsplit][F*D + F] into KV and ksum.
hipError_t launch_kv_finalize(const Problem& p, const float* part, int nsplit, float* KV, float* ksum,
                              hipStream_t s);

// k_kv2.hip + k_fused.hip: the bf16 hot path. launch_kv2 runs the split-N
// key/value reduction and writes the per-head operand pack into ws; then
// launch_fused_query runs apply + landmark softmax + blend over Q.
struct FusedPack {
  const unsigned char* pack_bh;  // [B*H][bh_bytes]
  const unsigned char* pack_w;   // [H][w_bytes]
  size_t bh_bytes, w_bytes;
};
size_t fused_workspace_bytes(const Problem& p, int L);
hipError_t launch_kv2(const Problem& p, const void* K, const void* V, const void* W, const float* bias, int L,
                      void* ws, FusedPack* pk, hipStream_t s, StageTimer* t);
// Softmax attention of the query rows over landmarks j < L alone (keys at
// (j N) / L): a pack of landmark chunks (lm_pack_bytes of workspace), then the
// fused query kernel without its linear branch; bf16, D = 64 or 128.
size_t lm_pack_bytes(const Problem& p, int L);
hipError_t launch_lm_pack(const Problem& p, const void* K, const void* V, int L, void* ws, FusedPack* pk,
                          hipStream_t s);
hipError_t launch_softmax_query(const Problem& p, const void* Q, const FusedPack& pk, int L, void* out,
                                hipStream_t s);
// The same with an fp32 output (N D 4 bytes per slice must fit 32 bits).
hipError_t launch_softmax_query_f32(const Problem& p, const void* Q, const FusedPack& pk, int L, float* out,
                                    hipStream_t s);
hipError_t launch_fused_query(const Problem& p, const void* Q, const FusedPack& pk, const float* g, float eps,
                              int L, void* out, hipStream_t s);
// The key/value reduction alone on the bf16 path (ttr_kv_reduce): the partial
// kernel of the fused path, then the fixed-order sum into fp32 KV and ksum.
size_t kv2_reduce_workspace_bytes(const Problem& p);
hipError_t launch_kv2_reduce(const Problem& p, const void* K, const void* V, const void* W, const float* bias,
                             float* KV, float* ksum, void* ws, hipStream_t s);

// k_blend.hip
hipError_t launch_blend(const Problem& p, const float* lin, const float* lm, const float* g, void* out,
                        hipStream_t s);

// k_causal.hip: chunked prefix scan (segment totals, then an in-order chunk walk).
void causal_plan(const Problem& p, int chunk, int* nseg, int* chunks_per_seg);
size_t causal_workspace_bytes(const Problem& p, int chunk);
size_t causal_seg_bytes(const Problem& p, int chunk);  // the segment-totals part of the workspace
size_t causal1_workspace_bytes(const Problem& p, int chunk);  // the single-pass bf16 D = 64 kernel's
// k_causal2.hip: the bf16, D = 64 scan with streamed chunk tiles (same plan; the
// workspace adds a sink for the stores of rows past N after the segment totals).
constexpr size_t CAUSAL2_SINK_BYTES = 8192;
bool causal2_supported(const Problem& p, int chunk);
hipError_t launch_causal2(const Problem& p, const void* Q, const void* K, const void* V, const float* bias,
                          float eps, int chunk, void* out, void* ws, hipStream_t s, StageTimer* t);
hipError_t launch_causal(const Problem& p, const void* Q, const void* K, const void* V, const float* bias,
                         float eps, int chunk, void* out, void* ws, hipStream_t s, StageTimer* t);

// NNT layer projections (k_proj.hip)
hipError_t launch_wt_transpose(int dtype, const void* const* W, void* const* Wt, int nmat, int E, hipStream_t s);
hipError_t launch_proj_gemm(int dtype, bool a_heads, bool c_qkv, const void* A, const void* Wt,
                            const float* const* bias, void* const* out, int M, int K, int Nc, int Ntok, int H,
                            int D, int E, hipStream_t s);

// k_backward.hip: gradients of the hybrid forward for W, b, g (fp32
// intermediates in the workspace, byte offsets below).
struct BackwardLayout {
  size_t zq, zk, dzq, dzk, lin, lm, dnum, kv, dkv, ks, dks, den, dden, rpart, cs1, cs2, cs3, splitk, bytes;
};
BackwardLayout backward_layout(const Problem& p);
hipError_t launch_hybrid_backward(const Problem& p, const void* Q, const void* K, const void* V, const void* W,
                                  const float* bias, const float* g, float eps, int L, const float* dout, float* dW,
                                  float* db, float* dg, void* ws, hipStream_t s, StageTimer* t);

// Phase-1 distillation step (k_backward.hip): workspace after the backward's
struct DistillLayout {
  size_t w_io, teacher, tws, hrow, crow, grads, lpart, bytes;
};
DistillLayout distill_layout(const Problem& p, bool need_teacher);
hipError_t launch_distill_step(const Problem& p, const void* Q, const void* K, const void* V, const float* teacher,
                               float* W, float* bias, float* g, float* sv, float* moments, int step, float lr,
                               float eps, int L, float* loss_out, void* ws, hipStream_t s, StageTimer* t);

// k_gate.hip: cosine distance of two attention outputs
size_t cosine_workspace_bytes(const Problem& p);
hipError_t launch_cosine_distance(const Problem& p, const void* student, const void* teacher, float* out, void* ws,
                                  hipStream_t s, StageTimer* t);

// k_replay.hip: rows q_index[0..Nq) (device-readable, e.g. mapped pinned
// memory) of every (batch, head) slice of Q, and of T when non-NULL, copied
// to [slices, Nq, row] (device).
hipError_t launch_replay_gather(const void* Q, void* q_dst, int q_row_bytes, const float* T, void* t_dst,
                                int t_row_bytes, const int32_t* q_index, int slices, int N, int Nq, hipStream_t s);

// The calling thread's registered stage events (ttr_set_stage_events), taken
// and cleared; the first is recorded on s at once.
StageTimer take_stage_timer(hipStream_t s);

// Records a failed HIP call's error for ttr_last_hip_error (calling thread)
// and maps it to a status.
ttr_status report_hip(hipError_t e);

}  // namespace ttr

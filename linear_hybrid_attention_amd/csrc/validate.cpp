// Host-only argument validation for the C ABI. Shape rules follow the
// method's pages: "Flux2TTRTrainer", section "Inputs worth setting"
// (feature_dim is a multiple of 256; this library implements 256, and 512,
// 768 and 1024 on the bf16 hybrid forward), and
// "NNT Define Linear Attention", section "The inputs" (causal flag, eps).
#include "validate.hpp"

#include <cstdlib>

namespace ttr {

unsigned env_spin_limit(unsigned deflt) {
  const char* v = std::getenv("TTR_SPIN_LIMIT");
  if (v == nullptr || *v == 0) return deflt;
  const unsigned long n = std::strtoul(v, nullptr, 10);
  return n >= 1 && n <= 0xFFFFFFFFul ? (unsigned)n : deflt;
}

bool env_flag(const char* name) {
  const char* v = std::getenv(name);
  return v != nullptr && v[0] == '1' && v[1] == 0;
}

size_t dtype_bytes(int32_t dtype) {
  switch (dtype) {
    case TTR_FP32: return 4;
    case TTR_BF16: return 2;
    default: return 0;
  }
}

ttr_status check_dims(const ttr_dims& d, bool has_w, int32_t max_f) {
  if (dtype_bytes(d.dtype) == 0) return TTR_ERR_DTYPE;
  if (d.fmap < TTR_FMAP_ELU1 || d.fmap > TTR_FMAP_SOFTMAX) return TTR_ERR_SHAPE;
  // relu / softmax: the NNT linear attention's maps on projected features
  if (d.fmap != TTR_FMAP_ELU1 && has_w) return TTR_ERR_UNSUPPORTED;
  if (d.B < 1 || d.H < 1 || d.N < 1) return TTR_ERR_SHAPE;
  if (d.D != 64 && d.D != 128) return TTR_ERR_SHAPE;
  if (has_w) {
    if (d.F < 256 || d.F % 256 != 0) return TTR_ERR_SHAPE;
    if (d.F > max_f) return TTR_ERR_UNSUPPORTED;
  } else if (d.F != d.D) {
    return TTR_ERR_SHAPE;
  }
  // grid limits: (batch, head) pairs run on grid.y
  if ((int64_t)d.B * d.H > 65535) return TTR_ERR_UNSUPPORTED;
  if ((int64_t)d.N * d.D >= ((int64_t)1 << 31)) return TTR_ERR_UNSUPPORTED;
  return TTR_OK;
}

ttr_status check_ptr(const void* p) {
  if (p == nullptr) return TTR_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return TTR_ERR_ALIGN;
  return TTR_OK;
}

ttr_status check_opt_ptr(const void* p) {
  if (p == nullptr) return TTR_OK;
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return TTR_ERR_ALIGN;
  return TTR_OK;
}

bool overlaps(Range a, Range b) {
  if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

ttr_status check_no_alias(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(outs[i], ins[j])) return TTR_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i], outs[j])) return TTR_ERR_ALIAS;
  }
  return TTR_OK;
}

bool causal_chunk_ok(int32_t dtype, int32_t D, int32_t chunk) {
  if (chunk != 64 && chunk != 128 && chunk != 256) return false;
  if (dtype == TTR_BF16 && D == 64) return true;
  if (dtype == TTR_BF16 && D == 128) return chunk <= 128;
  if (dtype == TTR_FP32 && D == 64) return chunk <= 128;
  if (dtype == TTR_FP32 && D == 128) return chunk == 64;
  return false;
}

int32_t causal_default_chunk(int32_t dtype, int32_t D) {
  // 128 where it fits: two workgroups of the streamed bf16 kernel share a CU
  for (int32_t c = 128; c >= 64; c /= 2)
    if (causal_chunk_ok(dtype, D, c)) return c;
  return 0;
}

ttr_status check_causal(const ttr_dims& d, const void* W, int32_t L, int32_t chunk) {
  if (chunk != 64 && chunk != 128 && chunk != 256) return TTR_ERR_SHAPE;
  if (W != nullptr) return TTR_ERR_UNSUPPORTED;  // the causal variant has no projection
  if (L != 0) return TTR_ERR_UNSUPPORTED;        // no causal landmark branch is defined
  if (!causal_chunk_ok(d.dtype, d.D, chunk)) return TTR_ERR_UNSUPPORTED;
  return TTR_OK;
}

ttr_status check_layer(const ttr_layer_dims& d, ttr_dims* core) {
  if (dtype_bytes(d.dtype) == 0) return TTR_ERR_DTYPE;
  if (d.fmap < TTR_FMAP_ELU1 || d.fmap > TTR_FMAP_SOFTMAX) return TTR_ERR_SHAPE;
  if (d.B < 1 || d.N < 1 || d.H < 1 || d.E < 1) return TTR_ERR_SHAPE;
  if (d.E % d.H != 0) return TTR_ERR_SHAPE;  // embed_dim divides by num_heads
  // projection tiles are 128 columns wide
  if (d.E % 128 != 0) return TTR_ERR_UNSUPPORTED;
  if ((int64_t)d.B * d.N * d.E >= ((int64_t)1 << 31)) return TTR_ERR_UNSUPPORTED;
  ttr_dims c;
  c.B = d.B;
  c.H = d.H;
  c.N = d.N;
  c.D = d.E / d.H;
  c.F = c.D;
  c.dtype = d.dtype;
  c.fmap = d.fmap;
  const ttr_status st = check_dims(c, false);
  if (st != TTR_OK) return st == TTR_ERR_SHAPE ? TTR_ERR_UNSUPPORTED : st;  // D outside {64, 128}: a valid layer not implemented
  *core = c;
  return TTR_OK;
}

}  // namespace ttr

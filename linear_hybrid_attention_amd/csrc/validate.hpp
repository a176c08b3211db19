// Host-only argument validation for the C ABI (no HIP calls; compiles with
// any C++17 compiler). Each check returns the ttr_status the entry point
// reports before anything is enqueued.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/ttr.h"

namespace ttr {

// Size in bytes of one IO element, 0 for an unknown dtype.
size_t dtype_bytes(int32_t dtype);

// Rules on B, H, N, D, F, dtype shared by every entry point.
// has_w: a projection W is given (F must be 256) or not (F must equal D).
// Test hooks read at every launch (no effect unless set): TTR_SPIN_LIMIT
// replaces the poll limit of the kernels' bounded waits (a tiny value makes
// them give up, so a test can check that they fail visibly and finish);
// TTR_KVS_CROSS_XCD_ROUND=1 makes the key/value stage take its cross-XCD round
// (write-back, second count, invalidate) even when a group's splits share an
// XCD, so the round is exercised on hardware that never needs it.
unsigned env_spin_limit(unsigned deflt);
bool env_flag(const char* name);

// max_f: the largest projected feature dimension the calling entry point
// implements (a multiple of 256 above it is TTR_ERR_UNSUPPORTED).
ttr_status check_dims(const ttr_dims& d, bool has_w, int32_t max_f = 256);

// Projected feature dimensions of the bf16 hybrid forward: 256, 512, 768 and 1024.
constexpr int32_t kMaxFeatureDimBf16Forward = 1024;
inline int32_t forward_max_f(const ttr_dims& d) { return d.dtype == TTR_BF16 ? kMaxFeatureDimBf16Forward : 256; }

// NULL and 16-byte alignment of a required pointer (NULL -> TTR_ERR_NULL).
ttr_status check_ptr(const void* p);
// Optional pointer: NULL allowed, else 16-byte aligned.
ttr_status check_opt_ptr(const void* p);

// Byte range [p, p + n) of an argument, used for the overlap rule.
struct Range {
  const void* p;
  size_t n;
};
bool overlaps(Range a, Range b);
// TTR_ERR_ALIAS if any output overlaps any input.
ttr_status check_no_alias(const Range* outs, int nout, const Range* ins, int nin);

// Causal rules: identity map only, no landmarks, a supported chunk size.
ttr_status check_causal(const ttr_dims& d, const void* W, int32_t L, int32_t chunk);

// NNT layer shape rules (see ttr_nnt_layer_forward); on success *core holds
// the per-head attention's dims (F = D, no projection).
ttr_status check_layer(const ttr_layer_dims& d, ttr_dims* core);

// Largest supported causal chunk <= 256 for this dtype and head dim (0 if none).
int32_t causal_default_chunk(int32_t dtype, int32_t D);

// Whether the causal kernels support this (dtype, D, chunk); mirrors the
// kernels' LDS budget.
bool causal_chunk_ok(int32_t dtype, int32_t D, int32_t chunk);

}  // namespace ttr

// Bounded per-head blend of the two TTR branches:
//   out = alpha_h out_lin + (1 - alpha_h) out_lm,  alpha_h = sigmoid(g_h)
// "Flux2TTRTrainer", section "How the distillation works" (the branches are
// blended by a bounded weight). Elementwise and HBM-bound: each thread moves
// four consecutive elements (one head, since D is a multiple of 4).
#include "common.hpp"
#include "launch.hpp"

namespace ttr {

template <typename T>
__global__ __launch_bounds__(256) void blend_kernel(const float* lin, const float* lm, const float* g, T* out,
                                                    int H, long long nd, long long n4) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) {
    const long long e = i * 4;
    const int h = (int)((e / nd) % H);
    const float alpha = 1.f / (1.f + expf(-g[h]));  // g = +inf -> 1, g = -inf -> 0
    const float beta = 1.f - alpha;
    const f32x4 a = *reinterpret_cast<const f32x4*>(lin + e);
    const f32x4 b = *reinterpret_cast<const f32x4*>(lm + e);
    st4(out + e, alpha * a[0] + beta * b[0], alpha * a[1] + beta * b[1], alpha * a[2] + beta * b[2],
        alpha * a[3] + beta * b[3]);
  }
}

hipError_t launch_blend(const Problem& p, const float* lin, const float* lm, const float* g, void* out,
                        hipStream_t s) {
  const long long nd = (long long)p.N * p.D;
  const long long n4 = (long long)p.B * p.H * nd / 4;
  long long blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (p.dtype == 1)
    hipLaunchKernelGGL(blend_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, lin, lm, g,
                       static_cast<uint16_t*>(out), p.H, nd, n4);
  else
    hipLaunchKernelGGL(blend_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, lin, lm, g,
                       static_cast<float*>(out), p.H, nd, n4);
  return hipGetLastError();
}

}  // namespace ttr

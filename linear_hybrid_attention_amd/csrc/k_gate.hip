// Cosine distance between a student's and a teacher's attention outputs, the
// quantity the per-layer readiness gate tracks ("Flux2TTRTrainer", section
// "How the distillation works": a layer serves the student once its EMA cosine
// distance to the teacher is low). distance = mean over (batch, head, token)
// rows of 1 - o.t / max(|o| |t|, 1e-8), rows of D values in the IO dtype.
// One wave per row, then two fixed-order reduction levels (bitwise
// reproducible).
#include "common.hpp"
#include "launch.hpp"

namespace ttr {

constexpr int kCosRows = 4096;  // rows per first-level partial

template <typename T>
__global__ void cos_rows_kernel(const T* o, const T* t, int rows, int D, float* crow) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const T* orow = o + (size_t)row * D;
  const T* trow = t + (size_t)row * D;
  float dot = 0.f, oo = 0.f, tt = 0.f;
  for (int d = lane; d < D; d += 64) {
    const float a = to_f32<T>(orow[d]), b = to_f32<T>(trow[d]);
    dot += a * b;
    oo += a * a;
    tt += b * b;
  }
  for (int off = 32; off > 0; off >>= 1) {
    dot += __shfl_xor(dot, off);
    oo += __shfl_xor(oo, off);
    tt += __shfl_xor(tt, off);
  }
  if (lane == 0) crow[row] = 1.f - dot / fmaxf(sqrtf(oo) * sqrtf(tt), 1e-8f);
}

__global__ void cos_part_kernel(const float* crow, int rows, float* part) {
  __shared__ float sh[256];
  const int t = threadIdx.x, r0 = blockIdx.x * kCosRows, r1 = min(rows, r0 + kCosRows);
  float c = 0.f;
  for (int i = r0 + t; i < r1; i += 256) c += crow[i];
  sh[t] = c;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (t < o) sh[t] += sh[t + o];
    __syncthreads();
  }
  if (t == 0) part[blockIdx.x] = sh[0];
}

__global__ void cos_total_kernel(const float* part, int nparts, int rows, float* out) {
  if (threadIdx.x != 0) return;
  float s = 0.f;
  for (int k = 0; k < nparts; ++k) s += part[k];
  out[0] = s / (float)rows;
}

size_t cosine_workspace_bytes(const Problem& p) {
  const size_t rows = (size_t)p.B * p.H * p.N;
  return ((rows * 4 + 255) & ~(size_t)255) + ((rows + kCosRows - 1) / kCosRows) * 4;
}

hipError_t launch_cosine_distance(const Problem& p, const void* student, const void* teacher, float* out, void* ws,
                                  hipStream_t s) {
  const int rows = p.B * p.H * p.N;
  float* crow = static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + (((size_t)rows * 4 + 255) & ~(size_t)255));
  const dim3 grid((rows + 3) / 4);
  if (p.dtype == 1)
    hipLaunchKernelGGL(cos_rows_kernel<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(student),
                       static_cast<const uint16_t*>(teacher), rows, p.D, crow);
  else
    hipLaunchKernelGGL(cos_rows_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(student),
                       static_cast<const float*>(teacher), rows, p.D, crow);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nparts = (rows + kCosRows - 1) / kCosRows;
  hipLaunchKernelGGL(cos_part_kernel, dim3(nparts), dim3(256), 0, s, crow, rows, part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cos_total_kernel, dim3(1), dim3(64), 0, s, part, nparts, rows, out);
  return hipGetLastError();
}

}  // namespace ttr

// Cosine distance between a student's and a teacher's attention outputs, the
// quantity the per-layer readiness gate tracks ("Flux2TTRTrainer", section
// "How the distillation works": a layer serves the student once its EMA cosine
// distance to the teacher is low). distance = mean over (batch, head, token)
// rows of 1 - o.t / max(|o| |t|, 1e-8), rows of D values in the IO dtype.
// Rows are read with 16-byte loads by small lane groups; two fixed-order
// reduction levels (bitwise reproducible).
#include "common.hpp"
#include "launch.hpp"

namespace ttr {

constexpr int kCosRows = 64;  // rows per workgroup (first-level partial)

// Workgroup k: rows [k * 64, (k + 1) * 64). A row is read with 16-byte loads
// by G = D * sizeof(T) / 16 consecutive lanes (8, 16 or 32), 256 / G rows per
// pass; every pass's loads are issued before any arithmetic. A row's dot
// product and norms are reduced across its G lanes, its 1 - cos is kept by
// its first lane, and the workgroup's sum (fixed order) goes to part[k].
template <typename T, int D>
__global__ __launch_bounds__(256) void cos_part_kernel(const T* o, const T* t, int rows, float* part) {
  constexpr int P = 16 / sizeof(T), G = D / P, RPP = 256 / G, NP = kCosRows / RPP;
  static_assert(G >= 8 && G <= 64 && (G & (G - 1)) == 0 && NP >= 1, "row group");
  __shared__ float sh[256];
  const int tid = threadIdx.x, gl = tid % G, rr = tid / G;
  u32x4 ov[NP], tv[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int row = blockIdx.x * kCosRows + q * RPP + rr;
    if (row < rows) {
      ov[q] = *reinterpret_cast<const u32x4*>(o + (size_t)row * D + gl * P);
      tv[q] = *reinterpret_cast<const u32x4*>(t + (size_t)row * D + gl * P);
    } else {
      ov[q] = u32x4{0u, 0u, 0u, 0u};
      tv[q] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int row = blockIdx.x * kCosRows + q * RPP + rr;
    const T* oe = reinterpret_cast<const T*>(&ov[q]);
    const T* te = reinterpret_cast<const T*>(&tv[q]);
    float dot = 0.f, oo = 0.f, tt = 0.f;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const float a = to_f32<T>(oe[j]), b = to_f32<T>(te[j]);
      dot += a * b;
      oo += a * a;
      tt += b * b;
    }
#pragma unroll
    for (int off = 1; off < G; off <<= 1) {
      dot += __shfl_xor(dot, off);
      oo += __shfl_xor(oo, off);
      tt += __shfl_xor(tt, off);
    }
    if (gl == 0 && row < rows) acc += 1.f - dot / fmaxf(sqrtf(oo) * sqrtf(tt), 1e-8f);
  }
  sh[tid] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) sh[tid] += sh[tid + off];
    __syncthreads();
  }
  if (tid == 0) part[blockIdx.x] = sh[0];
}

// One workgroup: thread j sums parts j, j + 256, ... in order, then a fixed
// tree over the 256 sums.
__global__ __launch_bounds__(256) void cos_total_kernel(const float* part, int nparts, int rows, float* out) {
  __shared__ float sh[256];
  const int tid = threadIdx.x;
  float s = 0.f;
  for (int k = tid; k < nparts; k += 256) s += part[k];
  sh[tid] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) sh[tid] += sh[tid + off];
    __syncthreads();
  }
  if (tid == 0) out[0] = sh[0] / (float)rows;
}

size_t cosine_workspace_bytes(const Problem& p) {
  const size_t rows = (size_t)p.B * p.H * p.N;
  return ((rows + kCosRows - 1) / kCosRows) * 4;
}

template <typename T, int D>
static hipError_t launch_cos_t(const void* o, const void* t, int rows, float* part, hipStream_t s) {
  hipLaunchKernelGGL((cos_part_kernel<T, D>), dim3((rows + kCosRows - 1) / kCosRows), dim3(256), 0, s,
                     static_cast<const T*>(o), static_cast<const T*>(t), rows, part);
  return hipGetLastError();
}

hipError_t launch_cosine_distance(const Problem& p, const void* student, const void* teacher, float* out, void* ws,
                                  hipStream_t s, StageTimer* t) {
  const int rows = p.B * p.H * p.N;
  float* part = static_cast<float*>(ws);
  hipError_t e;
  if (p.dtype == 1) e = p.D == 128 ? launch_cos_t<uint16_t, 128>(student, teacher, rows, part, s)
                                   : launch_cos_t<uint16_t, 64>(student, teacher, rows, part, s);
  else e = p.D == 128 ? launch_cos_t<float, 128>(student, teacher, rows, part, s)
                      : launch_cos_t<float, 64>(student, teacher, rows, part, s);
  if (e != hipSuccess) return e;
  t->mark();
  const int nparts = (rows + kCosRows - 1) / kCosRows;
  hipLaunchKernelGGL(cos_total_kernel, dim3(1), dim3(256), 0, s, part, nparts, rows, out);
  e = hipGetLastError();
  t->mark();
  return e;
}

}  // namespace ttr

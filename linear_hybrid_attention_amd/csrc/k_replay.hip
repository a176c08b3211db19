// Replay-buffer row gather ("Flux2TTRTrainer", section "How the distillation
// works": samples keep full keys and values but only a subsample of the
// queries, offloaded to CPU memory). Copies the rows q_index[0..Nq) of every
// (batch, head) slice of Q (and of the fp32 teacher output) from [S, N, row]
// into a contiguous [S, Nq, row] device staging area, HBM to HBM; the staged
// rows then cross PCIe by DMA together with K and V. (Kernel stores straight
// into pinned host memory were measured to stall the memory traffic of the
// kernels running beside them for as long as they last; DMA copies do not.)
#include "common.hpp"
#include "launch.hpp"

namespace ttr {

constexpr int kGatherRows = 64;  // query rows per workgroup

struct GatherJob {
  const uint8_t* src;  // [S, N, row_bytes]
  uint8_t* dst;        // [S, Nq, row_bytes]
  int row_bytes;       // multiple of 16
};

// grid (ceil(Nq / 64), S, jobs): workgroup (x, s, z) copies query rows
// [64 x, 64 x + 64) of slice s for job z; the 64 indices are read once into
// LDS, then each thread moves 16-byte pieces, four loads ahead of the stores.
__global__ __launch_bounds__(256) void gather_rows_kernel(GatherJob j0, GatherJob j1, const int32_t* q_index,
                                                          int Nq, int N) {
  __shared__ int32_t rows_s[kGatherRows];
  const GatherJob j = blockIdx.z == 0 ? j0 : j1;
  const int q0 = blockIdx.x * kGatherRows, nq = min(kGatherRows, Nq - q0);
  const size_t slice = blockIdx.y;
  if (threadIdx.x < nq) rows_s[threadIdx.x] = q_index[q0 + threadIdx.x];
  __syncthreads();
  const int per_row = j.row_bytes / 16, n = nq * per_row;
  const uint8_t* src = j.src + slice * (size_t)N * j.row_bytes;
  u32x4* dst = reinterpret_cast<u32x4*>(j.dst + (slice * (size_t)Nq + q0) * j.row_bytes);
  int p = threadIdx.x;
  for (; p + 3 * 256 < n; p += 4 * 256) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (p + i * 256) / per_row, k = (p + i * 256) - r * per_row;
      v[i] = *reinterpret_cast<const u32x4*>(src + (size_t)rows_s[r] * j.row_bytes + k * 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[p + i * 256] = v[i];
  }
  for (; p < n; p += 256) {
    const int r = p / per_row, k = p - r * per_row;
    dst[p] = *reinterpret_cast<const u32x4*>(src + (size_t)rows_s[r] * j.row_bytes + k * 16);
  }
}

hipError_t launch_replay_gather(const void* Q, void* q_dst, int q_row_bytes, const float* T, void* t_dst,
                                int t_row_bytes, const int32_t* q_index, int slices, int N, int Nq, hipStream_t s) {
  GatherJob a{static_cast<const uint8_t*>(Q), static_cast<uint8_t*>(q_dst), q_row_bytes};
  GatherJob b = a;
  int jobs = 1;
  if (T != nullptr) {
    b = GatherJob{reinterpret_cast<const uint8_t*>(T), static_cast<uint8_t*>(t_dst), t_row_bytes};
    jobs = 2;
  }
  hipLaunchKernelGGL(gather_rows_kernel, dim3((Nq + kGatherRows - 1) / kGatherRows, slices, jobs), dim3(256), 0, s,
                     a, b, q_index, Nq, N);
  return hipGetLastError();
}

}  // namespace ttr

// Key/value reduction of the TTR kernel branch with the feature map fused:
//   KV_h = phi(K)^T V  [F x D],   ksum_h = sum_n phi(K)_n  [F]
// "NNT Define Linear Attention", section "How it works" (accumulate K'^T V
// first so the sequence dimension collapses; sum(K') for the normaliser).
//
// The contraction runs over N, far longer than the [F x D] output, so the
// token range of each (batch, head) is split over several workgroups
// (kv_partial_kernel) and the partial sums are added in a fixed split order
// by kv_finalize_kernel: no atomics, bitwise reproducible.
//
// In a workgroup each wave owns a 64-wide feature slice f0..f0+63:
//   phi [tok x 64] = K [tok x D] . W[:, slice]        (A = K rows from global, B = W in registers)
//   KV  [64 x D]  += phi^T [64 x tok] . V [tok x D]   (A = previous C tile, B = V^T from LDS)
// The C tile of the first product (lane = feature, registers = tokens) is the
// A operand of the second one, with the tokens of V^T stored in kperm order.
#include "common.hpp"
#include "launch.hpp"

namespace ttr {

struct KvArgs {
  const void* K;
  const void* V;
  const void* W;
  const float* bias;
  int H, N, chunk, nsplit;
  float* kv_out;  // nsplit > 1: partials [BH][nsplit][F*D + F]; else KV [BH][F*D]
  float* ks_out;  // nsplit == 1: ksum [BH][F]; unused otherwise
};

template <typename T, int D, int F>
struct KvShape {
  static constexpr int NFS = F / 64;        // feature slices per workgroup
  static constexpr int NTW = 4 / NFS;       // waves sharing one slice (split tokens)
  static constexpr int STEP = 32 * NTW;     // tokens per workgroup step
  using WR = LdsRow<T, D>;                  // W^T [F][D] (prologue only)
  using VR = LdsRow<T, STEP>;               // V^T [D][STEP] (tokens in kperm order)
  static constexpr int RED_FLOATS = 2 * (D / 32) * 16 * 64 + 2 * 64;  // one wave's KV + ksum
  static constexpr int w_bytes = F * WR::bytes_per_row;
  static constexpr int v_bytes = D * VR::bytes_per_row;
  static constexpr int r_bytes = (NTW - 1) * NFS * RED_FLOATS * 4;
  static constexpr int m1 = w_bytes > v_bytes ? w_bytes : v_bytes;
  static constexpr int bytes = m1 > r_bytes ? m1 : r_bytes;
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

template <typename T, int D, int F, bool PROJ, int MAP>
__global__ __launch_bounds__(256, 1) void kv_partial_kernel(KvArgs a) {
  using S = KvShape<T, D, F>;
  constexpr int NFS = S::NFS, NTW = S::NTW, STEP = S::STEP;
  using WR = typename S::WR;
  using VR = typename S::VR;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::bytes];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int bh = blockIdx.y, h = bh % a.H, split = blockIdx.x;
  const int fs = w % NFS, tw = w / NFS, f0 = 64 * fs;
  const int N = a.N;
  const int t_begin = split * a.chunk;
  const int t_end = min(N, t_begin + a.chunk);

  // W[:, slice] as B operand (lane = feature column, k = D) kept in registers.
  Frag<T> wf[2][D / 16];
  {
    T* Wt = reinterpret_cast<T*>(smem);
    if constexpr (PROJ) {
      const T* W = static_cast<const T*>(a.W) + (size_t)h * D * F;
      for (int u = tid; u < (D / 2) * (F / 8); u += 256) {
        const int d = 2 * (u % (D / 2));
        const int fo = (u / (D / 2)) * 8;
        const Vec8<T> w0 = ld8(W + (size_t)d * F + fo);
        const Vec8<T> w1 = ld8(W + (size_t)(d + 1) * F + fo);
#pragma unroll
        for (int j = 0; j < 8; ++j) st_pair(Wt + (fo + j) * WR::stride + d, w0.v[j], w1.v[j]);
      }
    } else {
      for (int u = tid; u < F * D; u += 256) {
        const int f = u / D, d = u % D;
        Wt[f * WR::stride + d] = from_f32<T>(f == d ? 1.f : 0.f);
      }
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb)
        wf[cb][kb] = ld_frag<T>(Wt + (f0 + cb * 32 + c) * WR::stride + kb * 16 + 8 * g);
    __syncthreads();  // the region is reused for V tiles
  }
  float bcol[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) bcol[cb] = a.bias ? a.bias[(size_t)h * F + f0 + cb * 32 + c] : 0.f;
  // softmax map (identity projection, F == D): the bias of this lane's half
  // of a key row's features
  float brow[MAP == kSoftmax ? D / 2 : 1];
  if constexpr (MAP == kSoftmax) {
    static_assert(!PROJ, "the softmax map takes already projected features");
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) brow[8 * kb + j] = a.bias ? a.bias[(size_t)h * F + kb * 16 + 8 * g + j] : 0.f;
  }

  const T* K = static_cast<const T*>(a.K) + (size_t)bh * N * D;
  const T* V = static_cast<const T*>(a.V) + (size_t)bh * N * D;
  T* Vt = reinterpret_cast<T*>(smem);

  f32x16 kv[2][D / 32];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) kv[cb][db] = f32x16{};
  float ks[2] = {0.f, 0.f};

  for (int t_step = t_begin; t_step < t_end; t_step += STEP) {
    // V^T tile: Vt[d][kperm(tl)] = V[t_step + tl][d]; tokens past the range are zero.
    for (int u = tid; u < (STEP / 2) * (D / 8); u += 256) {
      const int tl = 2 * (u % (STEP / 2)), d0 = (u / (STEP / 2)) * 8, t = t_step + tl;
      const Vec8<T> v0 = t < t_end ? ld8(V + (size_t)t * D + d0) : zero8<T>();
      const Vec8<T> v1 = t + 1 < t_end ? ld8(V + (size_t)(t + 1) * D + d0) : zero8<T>();
      const int pos = kperm(tl);
#pragma unroll
      for (int j = 0; j < 8; ++j) st_pair(Vt + (d0 + j) * VR::stride + pos, v0.v[j], v1.v[j]);
    }
    __syncthreads();

    const int t0 = t_step + 32 * tw;
    Frag<T> kf[D / 16];
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
      kf[kb] = t0 + c < t_end ? ld_frag<T>(K + (size_t)(t0 + c) * D + kb * 16 + 8 * g) : zero_frag<T>();

    // softmax: the feature maximum and inverse sum of this lane's key row
    // (token t0 + c; half its features here, half in lane ^ 32)
    float km = 0.f, kinv = 1.f;
    if constexpr (MAP == kSoftmax) {
      float z[D / 2];
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        frag_to_f32(kf[kb], z + 8 * kb);
#pragma unroll
        for (int j = 0; j < 8; ++j) z[8 * kb + j] += brow[8 * kb + j];
      }
      softmax_stats<D / 2, 32>(z, km, kinv);
    }
    Frag<T> pa[2][2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = bcol[cb];
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) mma(acc, kf[kb], wf[cb][kb]);
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // row r of the C tile is token t0 + crow(lane, r), whose statistics
        // lane crow(lane, r) holds
        const float mr = MAP == kSoftmax ? __shfl(km, crow(lane, r)) : 0.f;
        const float ir = MAP == kSoftmax ? __shfl(kinv, crow(lane, r)) : 1.f;
        p[r] = t0 + crow(lane, r) < t_end ? phi_of<MAP>(acc[r], mr, ir) : 0.f;
        ks[cb] += p[r];
      }
      pa[cb][0] = to_frag<T>(p);
      pa[cb][1] = to_frag<T>(p + 8);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const Frag<T> vb = ld_frag<T>(Vt + (db * 32 + c) * VR::stride + 32 * tw + 16 * kk + 8 * g);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) mma(kv[cb][db], pa[cb][kk], vb);
      }
    __syncthreads();
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) ks[cb] += shfl_xor32(ks[cb]);

  if constexpr (NTW > 1) {
    // Waves that share a feature slice add their token partials in wave order.
    float* red = reinterpret_cast<float*>(smem);
    if (tw > 0) {
      float* rb = red + ((tw - 1) * NFS + fs) * S::RED_FLOATS;
      int i = 0;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) rb[(i++) * 64 + lane] = kv[cb][db][r];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) rb[(i++) * 64 + lane] = ks[cb];
    }
    __syncthreads();
    if (tw == 0) {
      for (int t2 = 1; t2 < NTW; ++t2) {
        const float* rb = red + ((t2 - 1) * NFS + fs) * S::RED_FLOATS;
        int i = 0;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) kv[cb][db][r] += rb[(i++) * 64 + lane];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) ks[cb] += rb[(i++) * 64 + lane];
      }
    }
  }

  if (tw == 0) {
    float* kvo;
    float* kso;
    if (a.nsplit > 1) {
      kvo = a.kv_out + ((size_t)bh * a.nsplit + split) * (size_t)(F * D + F);
      kso = kvo + F * D;
    } else {
      kvo = a.kv_out + (size_t)bh * F * D;
      kso = a.ks_out + (size_t)bh * F;
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          kvo[(size_t)(f0 + cb * 32 + crow(lane, r)) * D + db * 32 + c] = kv[cb][db][r];
    if (g == 0) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) kso[f0 + cb * 32 + c] = ks[cb];
    }
  }
}

// KV[bh] = sum over splits s = 0, 1, ... of the partials, in that order.
__global__ __launch_bounds__(256) void kv_finalize_kernel(const float* part, int nsplit, int FD, int F,
                                                          float* KV, float* ksum) {
  const int bh = blockIdx.y;
  const int total = FD + F;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= total) return;
  const float* p = part + (size_t)bh * nsplit * total + e;
  f32x4 acc = *reinterpret_cast<const f32x4*>(p);
  for (int s = 1; s < nsplit; ++s) acc += *reinterpret_cast<const f32x4*>(p + (size_t)s * total);
  if (e < FD)
    *reinterpret_cast<f32x4*>(KV + (size_t)bh * FD + e) = acc;
  else
    *reinterpret_cast<f32x4*>(ksum + (size_t)bh * F + (e - FD)) = acc;
}

static int kv_step(const Problem& p) { return 32 * (4 / (p.F / 64)); }

// Split plan: about one workgroup per compute unit over all (batch, head)
// pairs, each split at least two steps long; the chunk is a multiple of the step.
static void kv_plan(const Problem& p, int* nsplit, int* chunk) {
  const int step = kv_step(p);
  const int bh = p.B * p.H;
  const int nsteps = (p.N + step - 1) / step;
  int want = 256 / bh;
  if (want < 1) want = 1;
  int maxs = nsteps / 2;
  if (maxs < 1) maxs = 1;
  if (want > maxs) want = maxs;
  const int steps_per = (nsteps + want - 1) / want;
  *chunk = steps_per * step;
  *nsplit = (p.N + *chunk - 1) / *chunk;
}

int kv_nsplit(const Problem& p) {
  int ns, ch;
  kv_plan(p, &ns, &ch);
  return ns;
}

size_t kv_workspace_bytes(const Problem& p) {
  const int ns = kv_nsplit(p);
  if (ns <= 1) return 0;
  return (size_t)p.B * p.H * ns * (size_t)(p.F * p.D + p.F) * sizeof(float);
}

template <typename T, int D, int F, bool PROJ, int MAP>
static void launch_kv_t(const KvArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL((kv_partial_kernel<T, D, F, PROJ, MAP>), dim3(a.nsplit, B * a.H), dim3(256), 0, s, a);
}

template <typename T, int D>
static void launch_kv_d(const Problem& p, const KvArgs& a, hipStream_t s) {
  if (p.proj) launch_kv_t<T, D, 256, true, kElu1>(a, p.B, s);
  else if (p.fmap == kRelu) launch_kv_t<T, D, D, false, kRelu>(a, p.B, s);
  else if (p.fmap == kSoftmax) launch_kv_t<T, D, D, false, kSoftmax>(a, p.B, s);
  else launch_kv_t<T, D, D, false, kElu1>(a, p.B, s);
}

hipError_t launch_kv_reduce(const Problem& p, const void* K, const void* V, const void* W,
                            const float* bias, float* KV, float* ksum, void* ws, hipStream_t s) {
  int nsplit, chunk;
  kv_plan(p, &nsplit, &chunk);
  KvArgs a;
  a.K = K;
  a.V = V;
  a.W = W;
  a.bias = bias;
  a.H = p.H;
  a.N = p.N;
  a.chunk = chunk;
  a.nsplit = nsplit;
  a.kv_out = nsplit > 1 ? static_cast<float*>(ws) : KV;
  a.ks_out = ksum;
  if (p.dtype == 1 && p.D == 128) {
    launch_kv_d<uint16_t, 128>(p, a, s);
  } else if (p.dtype == 1 && p.D == 64) {
    launch_kv_d<uint16_t, 64>(p, a, s);
  } else if (p.dtype == 0 && p.D == 64) {
    launch_kv_d<float, 64>(p, a, s);
  } else if (p.dtype == 0 && p.D == 128) {
    launch_kv_d<float, 128>(p, a, s);
  } else {
    return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit <= 1) return e;
  const int FD = p.F * p.D;
  const int blocks = (FD + p.F + 1023) / 1024;
  hipLaunchKernelGGL(kv_finalize_kernel, dim3(blocks, p.B * p.H), dim3(256), 0, s,
                     static_cast<const float*>(ws), nsplit, FD, p.F, KV, ksum);
  return hipGetLastError();
}

hipError_t launch_kv_finalize(const Problem& p, const float* part, int nsplit, float* KV, float* ksum,
                              hipStream_t s) {
  const int FD = p.F * p.D;
  const int blocks = (FD + p.F + 1023) / 1024;
  hipLaunchKernelGGL(kv_finalize_kernel, dim3(blocks, p.B * p.H), dim3(256), 0, s, part, nsplit, FD, p.F, KV, ksum);
  return hipGetLastError();
}

}  // namespace ttr

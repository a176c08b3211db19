// Causal linear attention (elu + 1, relu or softmax feature map) as a chunked prefix scan.
// "NNT Define Linear Attention", section "The inputs" (causal: a token attends
// only to earlier tokens; elu(x) + 1 map; eps) and section "How it works".
//
//   out_n = phi(q_n) S_n / (phi(q_n) . z_n + eps),
//   S_n = sum_{m <= n} phi(k_m) v_m^T,  z_n = sum_{m <= n} phi(k_m)
//
// Tokens are cut into chunks of C. For chunk c starting at c0, with the state
// P = S_{c0-1}, z = z_{c0-1} of everything before it:
//   num = tril(phi(Q_c) phi(K_c)^T) V_c + phi(Q_c) P
//   den = rowsum(tril(phi(Q_c) phi(K_c)^T)) + phi(Q_c) . z
//   P += phi(K_c)^T V_c,  z += colsum(phi(K_c))
// The chunks of one (batch, head) are grouped into segments. Pass 1
// (causal_segsum_kernel) sums each segment's chunk states; pass 2
// (causal_scan_kernel) starts each segment from the fixed-order sum of the
// totals before it and walks its chunks in order. No atomics and no
// inter-workgroup waits: the result is deterministic and every wave exits.
//
// The state is kept transposed (P^T, rows = value dim d, columns = feature f),
// fp32 in registers (each wave owns 32x32 tiles) and as a bf16/fp32 MFMA
// operand in LDS. Products, in the transposed MFMA form used everywhere:
//   S^T  [key x q] = phi(K) [key x f] . phi(Q)^T [f x q]
//   num^T[d x q]  += V^T [d x key] . S^T (masked)   and   += P^T [d x f] . phi(Q)^T
//   P^T  [d x f]  += V^T [d x key] . phi(K) [key x f]
#include "common.hpp"
#include "launch.hpp"

namespace ttr {

struct CausalArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* bias;  // [H][D] or NULL
  float eps;
  int H, N, cps, nseg;
  float* seg;  // [BH][nseg][D*D + D]: segment totals P^T (row d, column f), then z
  void* out;
};

template <typename T, int D, int C>
struct CausalShape {
  using KR = LdsRow<T, D>;  // phi(K) [C][D]
  using TR = LdsRow<T, C>;  // phi(K)^T and V^T [D][C], tokens in kperm order
  using PR = LdsRow<T, D>;  // P^T [D][D]
  static constexpr int NTPW = (D / 32) * (D / 32) / 4;  // state tiles per wave
  static constexpr int t_bytes = D * TR::bytes_per_row;
  static constexpr int p_bytes = D * PR::bytes_per_row;
  // phi(K) also as rows (the score product's operand) when it fits; else
  // (fp32 with D = 128) the score operand is gathered from phi(K)^T
  static constexpr bool ROWS = C * KR::bytes_per_row + 2 * t_bytes + p_bytes + D * 4 <= 160 * 1024;
  static constexpr int phik_bytes = ROWS ? C * KR::bytes_per_row : 0;
  static constexpr int off_phikt = phik_bytes;
  static constexpr int off_vt = off_phikt + t_bytes;
  static constexpr int off_pt = off_vt + t_bytes;
  static constexpr int off_z = off_pt + p_bytes;
  static constexpr int scan_bytes = off_z + D * 4;
  static constexpr int seg_bytes = 2 * t_bytes;
  static_assert(scan_bytes <= 160 * 1024, "LDS budget");
};

// Stage one chunk: phi(K) rows (if ROWS), phi(K)^T and V^T (tokens in kperm
// order). Tokens at or past N are zero. Consecutive threads read consecutive
// 16-byte pieces of one row.
template <typename T, int D, int C, bool ROWS, int MAP>
__device__ __forceinline__ void stage_chunk(const T* K, const T* V, const float* bias, int c0, int N, T* phiK,
                                            T* phiKt, T* Vt, int tid) {
  using S = CausalShape<T, D, C>;
  using KR = typename S::KR;
  using TR = typename S::TR;
  static_assert(MAP != kSoftmax || (C / 2) * (D / 8) % 256 == 0, "every lane runs every round (row shuffles)");
  for (int u = tid; u < (C / 2) * (D / 8); u += 256) {
    const int d0 = (u % (D / 8)) * 8, tl = 2 * (u / (D / 8)), t = c0 + tl;
    const bool ok0 = t < N, ok1 = t + 1 < N;
    const Vec8<T> k0 = ok0 ? ld8(K + (size_t)t * D + d0) : zero8<T>();
    const Vec8<T> k1 = ok1 ? ld8(K + (size_t)(t + 1) * D + d0) : zero8<T>();
    const Vec8<T> v0 = ok0 ? ld8(V + (size_t)t * D + d0) : zero8<T>();
    const Vec8<T> v1 = ok1 ? ld8(V + (size_t)(t + 1) * D + d0) : zero8<T>();
    Vec8<T> p0, p1;
    float z0[8], z1[8], m0 = 0.f, i0 = 1.f, m1 = 0.f, i1 = 1.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float bj = bias ? bias[d0 + j] : 0.f;
      z0[j] = to_f32<T>(k0.v[j]) + bj;
      z1[j] = to_f32<T>(k1.v[j]) + bj;
    }
    if constexpr (MAP == kSoftmax) {  // a row's D / 8 pieces sit in D / 8 consecutive lanes
      softmax_stats<8, D / 8 - 1>(z0, m0, i0);
      softmax_stats<8, D / 8 - 1>(z1, m1, i1);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p0.v[j] = from_f32<T>(ok0 ? phi_of<MAP>(z0[j], m0, i0) : 0.f);
      p1.v[j] = from_f32<T>(ok1 ? phi_of<MAP>(z1[j], m1, i1) : 0.f);
    }
    if constexpr (ROWS) {
      st8(phiK + tl * KR::stride + d0, p0);
      st8(phiK + (tl + 1) * KR::stride + d0, p1);
    }
    const int pos = kperm(tl);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      st_pair(phiKt + (d0 + j) * TR::stride + pos, p0.v[j], p1.v[j]);
      st_pair(Vt + (d0 + j) * TR::stride + pos, v0.v[j], v1.v[j]);
    }
  }
}

// P^T tile (dt, ft) += V^T[dt rows] . phi(K)[:, ft cols] over the chunk; waves
// owning a dt == 0 tile also add the chunk's column sums of phi(K) to z.
template <typename T, int D, int C>
__device__ __forceinline__ void state_update(f32x16* P, float* zr, const T* phiKt, const T* Vt, int w,
                                             int lane) {
  using S = CausalShape<T, D, C>;
  using TR = typename S::TR;
  const int g = lane >> 5, c = lane & 31;
#pragma unroll
  for (int i = 0; i < S::NTPW; ++i) {
    const int ti = w * S::NTPW + i, dt = ti / (D / 32), ft = ti % (D / 32);
    float zp = 0.f;
#pragma unroll 4
    for (int kk = 0; kk < C / 16; ++kk) {
      const Frag<T> av = ld_frag<T>(Vt + (dt * 32 + c) * TR::stride + 16 * kk + 8 * g);
      const Frag<T> bk = ld_frag<T>(phiKt + (ft * 32 + c) * TR::stride + 16 * kk + 8 * g);
      mma(P[i], av, bk);
      if (dt == 0) {
        float bv[8];
        frag_to_f32(bk, bv);
#pragma unroll
        for (int j = 0; j < 8; ++j) zp += bv[j];
      }
    }
    if (dt == 0) zr[i] += zp + shfl_xor32(zp);
  }
}

template <typename T, int D, int C>
__device__ __forceinline__ void write_state(const f32x16* P, const float* zr, T* Pt, float* zS, int w,
                                            int lane) {
  using S = CausalShape<T, D, C>;
  using PR = typename S::PR;
  const int g = lane >> 5, c = lane & 31;
#pragma unroll
  for (int i = 0; i < S::NTPW; ++i) {
    const int ti = w * S::NTPW + i, dt = ti / (D / 32), ft = ti % (D / 32);
#pragma unroll
    for (int r = 0; r < 16; ++r) Pt[(dt * 32 + crow(lane, r)) * PR::stride + ft * 32 + c] = from_f32<T>(P[i][r]);
    if (dt == 0 && g == 0) zS[ft * 32 + c] = zr[i];
  }
}

template <typename T, int D, int C, int MAP>
__global__ __launch_bounds__(256, 1) void causal_segsum_kernel(CausalArgs a) {
  using S = CausalShape<T, D, C>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::seg_bytes];
  const int s = blockIdx.x, bh = blockIdx.y, h = bh % a.H;
  if (s >= a.nseg - 1) return;  // the last segment's total is never read
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31;
  const int N = a.N;
  const T* K = static_cast<const T*>(a.K) + (size_t)bh * N * D;
  const T* V = static_cast<const T*>(a.V) + (size_t)bh * N * D;
  const float* bias = a.bias ? a.bias + (size_t)h * D : nullptr;
  T* phiKt = reinterpret_cast<T*>(smem);
  T* Vt = reinterpret_cast<T*>(smem + S::t_bytes);
  const int nchunks = (N + C - 1) / C;
  const int cbeg = s * a.cps, cend = min(nchunks, cbeg + a.cps);

  f32x16 P[S::NTPW];
  float zr[S::NTPW];
#pragma unroll
  for (int i = 0; i < S::NTPW; ++i) { P[i] = f32x16{}; zr[i] = 0.f; }
  for (int ch = cbeg; ch < cend; ++ch) {
    __syncthreads();
    stage_chunk<T, D, C, false, MAP>(K, V, bias, ch * C, N, nullptr, phiKt, Vt, tid);
    __syncthreads();
    state_update<T, D, C>(P, zr, phiKt, Vt, w, lane);
  }
  float* out = a.seg + ((size_t)bh * a.nseg + s) * (size_t)(D * D + D);
#pragma unroll
  for (int i = 0; i < S::NTPW; ++i) {
    const int ti = w * S::NTPW + i, dt = ti / (D / 32), ft = ti % (D / 32);
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(dt * 32 + crow(lane, r)) * D + ft * 32 + c] = P[i][r];
    if (dt == 0 && lane < 32) out[D * D + ft * 32 + c] = zr[i];
  }
}

template <typename T, int D, int C, int MAP>
__global__ __launch_bounds__(256, 1) void causal_scan_kernel(CausalArgs a) {
  using S = CausalShape<T, D, C>;
  using KR = typename S::KR;
  using TR = typename S::TR;
  using PR = typename S::PR;
  constexpr int NB = C / 32;  // 32-token query/key blocks per chunk
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::scan_bytes];
  T* phiK = reinterpret_cast<T*>(smem);
  T* phiKt = reinterpret_cast<T*>(smem + S::off_phikt);
  T* Vt = reinterpret_cast<T*>(smem + S::off_vt);
  T* Pt = reinterpret_cast<T*>(smem + S::off_pt);
  float* zS = reinterpret_cast<float*>(smem + S::off_z);

  const int s = blockIdx.x, bh = blockIdx.y, h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, c = lane & 31;
  const int N = a.N;
  const size_t base = (size_t)bh * N * D;
  const T* Q = static_cast<const T*>(a.Q) + base;
  const T* K = static_cast<const T*>(a.K) + base;
  const T* V = static_cast<const T*>(a.V) + base;
  T* O = static_cast<T*>(a.out) + base;
  const float* bias = a.bias ? a.bias + (size_t)h * D : nullptr;
  const int nchunks = (N + C - 1) / C;
  const int cbeg = s * a.cps, cend = min(nchunks, cbeg + a.cps);

  // Exclusive prefix over earlier segments, summed in segment order.
  f32x16 P[S::NTPW];
  float zr[S::NTPW];
#pragma unroll
  for (int i = 0; i < S::NTPW; ++i) { P[i] = f32x16{}; zr[i] = 0.f; }
  for (int s2 = 0; s2 < s; ++s2) {
    const float* sp = a.seg + ((size_t)bh * a.nseg + s2) * (size_t)(D * D + D);
#pragma unroll
    for (int i = 0; i < S::NTPW; ++i) {
      const int ti = w * S::NTPW + i, dt = ti / (D / 32), ft = ti % (D / 32);
#pragma unroll
      for (int r = 0; r < 16; ++r) P[i][r] += sp[(dt * 32 + crow(lane, r)) * D + ft * 32 + c];
      if (dt == 0) zr[i] += sp[D * D + ft * 32 + c];
    }
  }
  write_state<T, D, C>(P, zr, Pt, zS, w, lane);

  for (int ch = cbeg; ch < cend; ++ch) {
    const int c0 = ch * C;
    __syncthreads();  // state written; previous chunk fully consumed
    stage_chunk<T, D, C, S::ROWS, MAP>(K, V, bias, c0, N, phiK, phiKt, Vt, tid);
    __syncthreads();

    for (int i = 0; i < (NB + 3) / 4; ++i) {
      const int qb = (i & 1) ? (4 * i + 3 - w) : (4 * i + w);  // balanced triangle split
      if (qb >= NB) continue;
      const int q = c0 + qb * 32 + c;
      const bool ok = q < N;
      Frag<T> qf[D / 16];
      float den = 0.f;
      float zq[D / 16][8], m = 0.f, inv = 1.f;
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        const Vec8<T> raw = ok ? ld8(Q + (size_t)q * D + kb * 16 + 8 * g) : zero8<T>();
#pragma unroll
        for (int j = 0; j < 8; ++j) zq[kb][j] = to_f32<T>(raw.v[j]) + (bias ? bias[kb * 16 + 8 * g + j] : 0.f);
      }
      // the query's features: half in this lane, half in lane ^ 32
      if constexpr (MAP == kSoftmax) softmax_stats<D / 2, 32>(&zq[0][0], m, inv);
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = ok ? phi_of<MAP>(zq[kb][j], m, inv) : 0.f;
        qf[kb] = to_frag<T>(v);
        float vr[8];
        frag_to_f32(qf[kb], vr);  // the operand values the products see
#pragma unroll
        for (int j = 0; j < 8; ++j) den += vr[j] * zS[kb * 16 + 8 * g + j];
      }
      f32x16 num[D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        num[db] = f32x16{};
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb)
          mma(num[db], ld_frag<T>(Pt + (db * 32 + c) * PR::stride + kb * 16 + 8 * g), qf[kb]);
      }
      for (int kb2 = 0; kb2 <= qb; ++kb2) {
        f32x16 sc = f32x16{};
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) {
          if constexpr (S::ROWS) {
            mma(sc, ld_frag<T>(phiK + (kb2 * 32 + c) * KR::stride + kb * 16 + 8 * g), qf[kb]);
          } else {  // key kb2 * 32 + c, features kb * 16 + 8 g + j: column kperm(key) of phi(K)^T
            Frag<T> kf;
            const T* col = phiKt + kperm(kb2 * 32 + c);
#pragma unroll
            for (int j = 0; j < 8; ++j) kf[j] = col[(kb * 16 + 8 * g + j) * TR::stride];
            mma(sc, kf, qf[kb]);
          }
        }
        float sv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sv[r] = (kb2 == qb && crow(lane, r) > c) ? 0.f : sc[r];
        }
        const Frag<T> sb0 = to_frag<T>(sv), sb1 = to_frag<T>(sv + 8);
        float sr[16];
        frag_to_f32(sb0, sr);
        frag_to_f32(sb1, sr + 8);
#pragma unroll
        for (int r = 0; r < 16; ++r) den += sr[r];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const T* ap = Vt + (db * 32 + c) * TR::stride + kb2 * 32 + 8 * g;
          mma(num[db], ld_frag<T>(ap), sb0);
          mma(num[db], ld_frag<T>(ap + 16), sb1);
        }
      }
      den += shfl_xor32(den);
      if (ok) {
        const float inv = 1.f / (den + a.eps);
        T* o = O + (size_t)q * D + 4 * g;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            st4(o + db * 32 + 8 * qq, num[db][4 * qq] * inv, num[db][4 * qq + 1] * inv,
                num[db][4 * qq + 2] * inv, num[db][4 * qq + 3] * inv);
      }
    }
    __syncthreads();  // every wave is done reading P^T, z and this chunk's tiles
    if (ch + 1 < cend) {
      state_update<T, D, C>(P, zr, phiKt, Vt, w, lane);
      write_state<T, D, C>(P, zr, Pt, zS, w, lane);
    }
  }
}

void causal_plan(const Problem& p, int chunk, int* nseg, int* cps) {
  const int nchunks = (p.N + chunk - 1) / chunk;
  const int bh = p.B * p.H;
  int want = (1024 + bh - 1) / bh;
  if (want < 1) want = 1;
  if (want > nchunks) want = nchunks;
  *cps = (nchunks + want - 1) / want;
  *nseg = (nchunks + *cps - 1) / *cps;
}

size_t causal_seg_bytes(const Problem& p, int chunk) {
  int nseg, cps;
  causal_plan(p, chunk, &nseg, &cps);
  if (nseg <= 1) return 0;
  return (size_t)p.B * p.H * nseg * (size_t)(p.D * p.D + p.D) * sizeof(float);
}

size_t causal_workspace_bytes(const Problem& p, int chunk) {
  // the streamed single-pass kernel's prefixes, flags and store sink; else segment totals
  return causal2_supported(p, chunk) ? causal1_workspace_bytes(p, chunk) : causal_seg_bytes(p, chunk);
}

template <typename T, int D, int C, int MAP>
static hipError_t launch_causal_t(const CausalArgs& a, int B, hipStream_t s, StageTimer* t) {
  const dim3 grid(a.nseg, B * a.H), block(256);
  if (a.nseg > 1) {
    hipLaunchKernelGGL((causal_segsum_kernel<T, D, C, MAP>), grid, block, 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    t->mark();
  }
  hipLaunchKernelGGL((causal_scan_kernel<T, D, C, MAP>), grid, block, 0, s, a);
  const hipError_t e = hipGetLastError();
  t->mark();
  return e;
}

// bf16 with D = 64 runs the streamed kernels of k_causal2.hip; these cover
// fp32 (D = 64, and D = 128 at chunk 64) and bf16 with D = 128.
template <int MAP>
static hipError_t launch_causal_m(const Problem& p, const CausalArgs& a, int chunk, hipStream_t s, StageTimer* t) {
  if (p.dtype == 1 && p.D == 128) {
    if (chunk == 64) return launch_causal_t<uint16_t, 128, 64, MAP>(a, p.B, s, t);
    if (chunk == 128) return launch_causal_t<uint16_t, 128, 128, MAP>(a, p.B, s, t);
  } else if (p.dtype == 0 && p.D == 64) {
    if (chunk == 64) return launch_causal_t<float, 64, 64, MAP>(a, p.B, s, t);
    if (chunk == 128) return launch_causal_t<float, 64, 128, MAP>(a, p.B, s, t);
  } else if (p.dtype == 0 && p.D == 128) {
    if (chunk == 64) return launch_causal_t<float, 128, 64, MAP>(a, p.B, s, t);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_causal(const Problem& p, const void* Q, const void* K, const void* V, const float* bias,
                         float eps, int chunk, void* out, void* ws, hipStream_t s, StageTimer* t) {
  CausalArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.bias = bias;
  a.eps = eps;
  a.H = p.H;
  a.N = p.N;
  causal_plan(p, chunk, &a.nseg, &a.cps);
  a.seg = static_cast<float*>(ws);
  a.out = out;
  if (p.fmap == kRelu) return launch_causal_m<kRelu>(p, a, chunk, s, t);
  if (p.fmap == kSoftmax) return launch_causal_m<kSoftmax>(p, a, chunk, s, t);
  return launch_causal_m<kElu1>(p, a, chunk, s, t);
}

}  // namespace ttr

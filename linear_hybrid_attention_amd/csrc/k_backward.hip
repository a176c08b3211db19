// Backward of the hybrid forward for the trainable parameters W_h, b_h, g_h,
// and the Phase-1 distillation step around it ("Flux2TTRTrainer", section "How
// the distillation works": the TTR student regresses native softmax attention;
// the loss is an uncertainty-weighted blend of huber and cosine; per-layer
// optimizer state). The chain rule (dout -> dW, db, dg):
//   dlin   = alpha dout,   dalpha = sum dout (lin - lm),   dg = dalpha alpha (1 - alpha)
//   dnum   = dlin / den,   dden = -sum_d dlin lin / den
//   dphi_q = dnum KV^T + dden ks^T,   dKV = phi_q^T dnum,   dks = phi_q^T dden
//   dphi_k = V dKV^T + 1 dks^T,       dz = dphi phi'(z)
//   dW = sum_b Q^T dz_q + K^T dz_k,   db = sum_{b,n} dz_q + dz_k
// The products run on one generic batched GEMM (bgemm_kernel) with per-operand
// strides, so transposed operands need no copies, and with elu + 1 applied to
// the A operand while it is loaded, so phi is never stored. Everything else is
// small elementwise or reduction kernels with a fixed summation order
// (results are bitwise reproducible).
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace ttr {

// ---------------------------------------------------------------- generic GEMM
// C[z](m, n) (+)= sum_{kb < KB} sum_{k < K} A[z](kb, m, k) B[z](kb, k, n)
//   A[z](kb, m, k) = A[z*sAz + kb*sAkb + m*sAm + k*sAk]   (elu + 1 applied when A_ELU)
//   B[z](kb, k, n) = B[z*sBz + kb*sBkb + k*sBk + n*sBn]
//   C[z](m, n)     = C[z*sCz + m*sCm + n*sCn], fp32; accumulate when beta != 0
struct BgemmArgs {
  const void* A;
  const void* B;
  float* C;
  int M, N, K, KB;
  long long sAz, sAkb, sAm, sAk;
  long long sBz, sBkb, sBk, sBn;
  long long sCz, sCm, sCn;
  int beta;
};

template <typename CT> struct BgTile {
  static constexpr int KT = 32;                  // K per step
  static constexpr int LD = KT + 16 / (int)sizeof(CT);  // padded row (16-byte multiple)
};

template <typename T> __device__ __forceinline__ float ld_elem(const T* p, long long i);
template <> __device__ __forceinline__ float ld_elem<float>(const float* p, long long i) { return p[i]; }
template <> __device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p, long long i) { return bf2f(p[i]); }

template <typename CT> __device__ __forceinline__ CT to_ct(float x);
template <> __device__ __forceinline__ float to_ct<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t to_ct<uint16_t>(float x) { return f2bf(x); }

// Loads one operand tile [64 rows][KT] of step (kb, k0) into registers: 8
// elements per thread. Along k when the k stride is 1 (8 consecutive k per
// thread), else along the rows (consecutive threads, consecutive rows).
template <typename T, bool ELU>
__device__ __forceinline__ void bg_load(float (&v)[8], const T* base, long long s_row, long long s_k, int row0,
                                        int nrows, int k0, int K, bool k_contig, int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r, k;
    if (k_contig) {
      r = tid / 4;
      k = (tid % 4) * 8 + i;
    } else {
      r = tid % 64;
      k = (tid / 64) * 8 + i;
    }
    const int gr = row0 + r, gk = k0 + k;
    float x = 0.f;
    if (gr < nrows && gk < K) {
      x = ld_elem<T>(base, (long long)gr * s_row + (long long)gk * s_k);
      if (ELU) x = elu1(x);
    }
    v[i] = x;
  }
}
template <typename CT>
__device__ __forceinline__ void bg_store(CT* tile, const float (&v)[8], bool k_contig, int tid) {
  constexpr int LD = BgTile<CT>::LD;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r, k;
    if (k_contig) {
      r = tid / 4;
      k = (tid % 4) * 8 + i;
    } else {
      r = tid % 64;
      k = (tid / 64) * 8 + i;
    }
    tile[r * LD + k] = to_ct<CT>(v[i]);
  }
}

template <typename CT, typename TA, typename TB, bool A_ELU>
__global__ __launch_bounds__(256) void bgemm_kernel(BgemmArgs a) {
  constexpr int KT = BgTile<CT>::KT, LD = BgTile<CT>::LD;
  __shared__ __attribute__((aligned(16))) CT As[64 * LD];
  __shared__ __attribute__((aligned(16))) CT Bs[64 * LD];  // B^T: [64 n][KT]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int wm = w & 1, wn = w >> 1;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64, z = blockIdx.z;
  const TA* A = static_cast<const TA*>(a.A) + z * a.sAz;
  const TB* B = static_cast<const TB*>(a.B) + z * a.sBz;
  const bool a_kc = a.sAk == 1, b_kc = a.sBk == 1;

  f32x16 acc = f32x16{};
  float va[8], vb[8];
  const int nks = (a.K + KT - 1) / KT, total = a.KB * nks;
  auto load = [&](int s) {
    const int kb = s / nks, k0 = (s % nks) * KT;
    bg_load<TA, A_ELU>(va, A + kb * a.sAkb, a.sAm, a.sAk, m0, a.M, k0, a.K, a_kc, tid);
    bg_load<TB, false>(vb, B + kb * a.sBkb, a.sBn, a.sBk, n0, a.N, k0, a.K, b_kc, tid);
  };
  load(0);
  for (int s = 0; s < total; ++s) {
    __syncthreads();  // every wave is done with the previous tile
    bg_store<CT>(As, va, a_kc, tid);
    bg_store<CT>(Bs, vb, b_kc, tid);
    __syncthreads();
    if (s + 1 < total) load(s + 1);  // in flight during the products
#pragma unroll
    for (int kb = 0; kb < KT / 16; ++kb) {
      const Frag<CT> fa = ld_frag<CT>(As + (wm * 32 + c) * LD + kb * 16 + 8 * g);
      const Frag<CT> fb = ld_frag<CT>(Bs + (wn * 32 + c) * LD + kb * 16 + 8 * g);
      mma(acc, fa, fb);
    }
  }
  // lane (c, g) holds column n0 + wn*32 + c and rows crow(lane, r)
  const int n = n0 + wn * 32 + c;
  if (n < a.N) {
    float* C = a.C + z * a.sCz + n * a.sCn;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * 32 + crow(lane, r);
      if (m < a.M) {
        float* p = C + m * a.sCm;
        *p = a.beta ? *p + acc[r] : acc[r];
      }
    }
  }
}

template <typename CT, typename TA, typename TB, bool ELU>
static hipError_t launch_bgemm_t(const BgemmArgs& a, int Z, hipStream_t s) {
  const dim3 grid((a.M + 63) / 64, (a.N + 63) / 64, Z);
  hipLaunchKernelGGL((bgemm_kernel<CT, TA, TB, ELU>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// dtype: 1 = bf16 IO (bf16 MFMA), 0 = fp32 IO (fp32 MFMA). a_io / b_io: the
// operand is in the IO dtype (else fp32).
static hipError_t launch_bgemm(int dtype, bool a_io, bool b_io, bool a_elu, const BgemmArgs& a, int Z, hipStream_t s) {
  if (dtype == 1) {
    if (a_io && b_io) return launch_bgemm_t<uint16_t, uint16_t, uint16_t, false>(a, Z, s);
    if (a_io && !b_io) return launch_bgemm_t<uint16_t, uint16_t, float, false>(a, Z, s);
    if (!a_io && b_io) {
      return a_elu ? launch_bgemm_t<uint16_t, float, uint16_t, true>(a, Z, s)
                   : launch_bgemm_t<uint16_t, float, uint16_t, false>(a, Z, s);
    }
    return a_elu ? launch_bgemm_t<uint16_t, float, float, true>(a, Z, s)
                 : launch_bgemm_t<uint16_t, float, float, false>(a, Z, s);
  }
  return a_elu ? launch_bgemm_t<float, float, float, true>(a, Z, s) : launch_bgemm_t<float, float, float, false>(a, Z, s);
}

// ---------------------------------------------------------------- small kernels
// ks[z][f] = sum_n phi(z_k[z][n][f])
__global__ void colsum_phi_kernel(const float* zk, float* ks, int Z, int N, int F) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Z * F) return;
  const int z = i / F, f = i % F;
  const float* p = zk + (size_t)z * N * F + f;
  float s = 0.f;
  for (int n = 0; n < N; ++n) s += elu1(p[(size_t)n * F]);
  ks[i] = s;
}

// Per row (z, n), one wave: den = phi(z_q) . ks + eps; lin = num / den (in place).
__global__ void den_lin_kernel(const float* zq, const float* ks, float* num, float* den, int Z, int N, int F, int D,
                               float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= Z * N) return;
  const int z = row / N;
  const float* zr = zq + (size_t)row * F;
  const float* k = ks + (size_t)z * F;
  float s = 0.f;
  for (int f = lane; f < F; f += 64) s += elu1(zr[f]) * k[f];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  const float dn = s + eps;
  if (lane == 0) den[row] = dn;
  float* nr = num + (size_t)row * D;
  for (int d = lane; d < D; d += 64) nr[d] = nr[d] / dn;
}

// Per row: dlin = alpha dout; dnum = dlin / den; dden = -sum_d dlin lin / den;
// and the row's share of dalpha: sum_d dout (lin - lm) (into rpart[row]).
__global__ void dlin_kernel(const float* dout, const float* lin, const float* lm, const float* den, const float* g,
                            int H, int N, int D, int Z, int has_lm, float* dnum, float* dden, float* rpart) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= Z * N) return;
  const int h = (row / N) % H;
  const float alpha = has_lm ? 1.f / (1.f + expf(-g[h])) : 1.f;
  const float inv = 1.f / den[row];
  const float* G = dout + (size_t)row * D;
  const float* li = lin + (size_t)row * D;
  float sd = 0.f, sa = 0.f;
  for (int d = lane; d < D; d += 64) {
    const float dl = alpha * G[d];
    dnum[(size_t)row * D + d] = dl * inv;
    sd += dl * li[d];
    if (has_lm) sa += G[d] * (li[d] - lm[(size_t)row * D + d]);
  }
  for (int o = 32; o > 0; o >>= 1) {
    sd += __shfl_xor(sd, o);
    sa += __shfl_xor(sa, o);
  }
  if (lane == 0) {
    dden[row] = -sd * inv;
    rpart[row] = sa;
  }
}

// dz[z][n][f] = (dphi[z][n][f] + r[z][n] s[z][f]) phi'(zv[z][n][f]), in place on dphi;
// r == NULL means r = 1.
__global__ void dz_kernel(float* dphi, const float* zv, const float* r, const float* sv, int Z, int N, int F) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)Z * N * F) return;
  const int f = (int)(i % F);
  const size_t row = i / F;
  const int z = (int)(row / N);
  const float x = zv[i];
  const float dp = dphi[i] + (r ? r[row] : 1.f) * sv[(size_t)z * F + f];
  dphi[i] = x > 0.f ? dp : dp * __expf(x);
}

// dks[z][f] = sum_n phi(z_q[z][n][f]) dden[z][n]
__global__ void dks_kernel(const float* zq, const float* dden, float* dks, int Z, int N, int F) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Z * F) return;
  const int z = i / F, f = i % F;
  const float* p = zq + (size_t)z * N * F + f;
  const float* dd = dden + (size_t)z * N;
  float s = 0.f;
  for (int n = 0; n < N; ++n) s += elu1(p[(size_t)n * F]) * dd[n];
  dks[i] = s;
}

// db[h][f] = sum_b sum_n dzq + dzk; dg[h] = alpha (1 - alpha) sum_b sum_n rpart
__global__ void db_dg_kernel(const float* dzq, const float* dzk, const float* rpart, const float* g, int B, int H, int N,
                             int F, int has_lm, float* db, float* dg) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < H * F) {
    const int h = i / F, f = i % F;
    float s = 0.f;
    for (int b = 0; b < B; ++b) {
      const size_t base = ((size_t)(b * H + h) * N) * F + f;
      for (int n = 0; n < N; ++n) s += dzq[base + (size_t)n * F] + dzk[base + (size_t)n * F];
    }
    db[i] = s;
  }
  if (i < H) {
    float s = 0.f;
    if (has_lm) {
      for (int b = 0; b < B; ++b) {
        const float* rp = rpart + (size_t)(b * H + i) * N;
        for (int n = 0; n < N; ++n) s += rp[n];
      }
      const float al = 1.f / (1.f + expf(-g[i]));
      s *= al * (1.f - al);
    }
    dg[i] = s;
  }
}

// z[b,h][n][f] += bias[h][f] for both projections
__global__ void add_bias_kernel(float* zq, float* zk, const float* bias, int H, int N, int F, size_t total) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int f = (int)(i % F);
  const int h = (int)((i / ((size_t)N * F)) % H);
  const float bv = bias[(size_t)h * F + f];
  zq[i] += bv;
  zk[i] += bv;
}

// ---------------------------------------------------------------- launches
static unsigned blocks(size_t n, unsigned t) { return (unsigned)((n + t - 1) / t); }

static hipError_t launch_add_bias(float* zq, float* zk, const float* bias, int B, int H, int N, int F, hipStream_t s) {
  const size_t total = (size_t)B * H * N * F;
  hipLaunchKernelGGL(add_bias_kernel, dim3(blocks(total, 256)), dim3(256), 0, s, zq, zk, bias, H, N, F, total);
  return hipGetLastError();
}
static hipError_t launch_colsum_phi(const float* zk, float* ks, int Z, int N, int F, hipStream_t s) {
  hipLaunchKernelGGL(colsum_phi_kernel, dim3(blocks((size_t)Z * F, 256)), dim3(256), 0, s, zk, ks, Z, N, F);
  return hipGetLastError();
}
static hipError_t launch_den_lin(const float* zq, const float* ks, float* num, float* den, int Z, int N, int F, int D,
                                 float eps, hipStream_t s) {
  hipLaunchKernelGGL(den_lin_kernel, dim3(blocks((size_t)Z * N, 4)), dim3(256), 0, s, zq, ks, num, den, Z, N, F, D,
                     eps);
  return hipGetLastError();
}
static hipError_t launch_dlin(const float* dout, const float* lin, const float* lm, const float* den, const float* g,
                              int H, int N, int D, int Z, bool has_lm, float* dnum, float* dden, float* rpart,
                              hipStream_t s) {
  hipLaunchKernelGGL(dlin_kernel, dim3(blocks((size_t)Z * N, 4)), dim3(256), 0, s, dout, lin, lm, den, g, H, N, D, Z,
                     has_lm ? 1 : 0, dnum, dden, rpart);
  return hipGetLastError();
}
static hipError_t launch_dks(const float* zq, const float* dden, float* dks, int Z, int N, int F, hipStream_t s) {
  hipLaunchKernelGGL(dks_kernel, dim3(blocks((size_t)Z * F, 256)), dim3(256), 0, s, zq, dden, dks, Z, N, F);
  return hipGetLastError();
}
static hipError_t launch_dz(float* dphi, const float* zv, const float* r, const float* sv, int Z, int N, int F,
                            hipStream_t s) {
  hipLaunchKernelGGL(dz_kernel, dim3(blocks((size_t)Z * N * F, 256)), dim3(256), 0, s, dphi, zv, r, sv, Z, N, F);
  return hipGetLastError();
}
static hipError_t launch_db_dg(const float* dzq, const float* dzk, const float* rpart, const float* g, int B, int H,
                               int N, int F, bool has_lm, float* db, float* dg, hipStream_t s) {
  hipLaunchKernelGGL(db_dg_kernel, dim3(blocks((size_t)H * F, 256)), dim3(256), 0, s, dzq, dzk, rpart, g, B, H, N, F,
                     has_lm ? 1 : 0, db, dg);
  return hipGetLastError();
}

// ---------------------------------------------------------------- host side
BackwardLayout backward_layout(const Problem& p) {
  BackwardLayout l;
  const size_t Z = (size_t)p.B * p.H, N = p.N, F = p.F, D = p.D;
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t at = o;
    o += (n * 4 + 255) & ~(size_t)255;
    return at;
  };
  l.zq = take(Z * N * F);
  l.zk = take(Z * N * F);
  l.dzq = take(Z * N * F);
  l.dzk = take(Z * N * F);
  l.lin = take(Z * N * D);
  l.lm = take(Z * N * D);
  l.dnum = take(Z * N * D);
  l.kv = take(Z * F * D);
  l.dkv = take(Z * F * D);
  l.ks = take(Z * F);
  l.dks = take(Z * F);
  l.den = take(Z * N);
  l.dden = take(Z * N);
  l.rpart = take(Z * N);
  l.bytes = o;
  return l;
}

#define TTR_HIP(x)                 \
  do {                             \
    const hipError_t e_ = (x);     \
    if (e_ != hipSuccess) return e_; \
  } while (0)

// Workspace views of the backward's fp32 intermediates.
struct BwBufs {
  float *zq, *zk, *dzq, *dzk, *lin, *lm, *dnum, *kv, *dkv, *ks, *dks, *den, *dden, *rpart;
};
static BwBufs bw_bufs(const Problem& p, void* ws) {
  const BackwardLayout l = backward_layout(p);
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  auto F32 = [&](size_t off) { return reinterpret_cast<float*>(w8 + off); };
  return BwBufs{F32(l.zq),  F32(l.zk), F32(l.dzq), F32(l.dzk), F32(l.lin), F32(l.lm),  F32(l.dnum),
                F32(l.kv),  F32(l.dkv), F32(l.ks), F32(l.dks), F32(l.den), F32(l.dden), F32(l.rpart)};
}

// Forward pass with the intermediates the gradients need: z_q, z_k (biased),
// ks, KV, den, lin = num / den and (L > 0) the landmark output lm.
static hipError_t backward_forward_pass(const Problem& p, const void* Q, const void* K, const void* V, const void* W,
                                        const float* bias, float eps, int L, const BwBufs& t, hipStream_t s) {
  float *zq = t.zq, *zk = t.zk, *lin = t.lin, *lm = t.lm, *kv = t.kv, *ks = t.ks, *den = t.den;
  const int B = p.B, H = p.H, N = p.N, D = p.D, F = p.F, Z = B * H, dt = p.dtype;
  const long long NF = (long long)N * F, ND = (long long)N * D, FD = (long long)F * D;
  // z_q = Q W + b, z_k = K W + b: per (b, h), [N x D] . [D x F]; the bias in a second pass
  auto proj = [&](const void* X, float* Zout) {
    BgemmArgs a{};
    a.A = X;
    a.B = W;
    a.C = Zout;
    a.M = N;
    a.N = F;
    a.K = D;
    a.KB = 1;
    a.sAz = ND;
    a.sAm = D;
    a.sAk = 1;
    // W[h] for z = b*H + h: z-stride cannot express "z % H", so launch per batch
    a.sBk = F;
    a.sBn = 1;
    a.sCm = F;
    a.sCn = 1;
    a.beta = 0;
    for (int b = 0; b < B; ++b) {
      BgemmArgs ab = a;
      ab.A = static_cast<const unsigned char*>(X) + (size_t)b * H * ND * (dt == 1 ? 2 : 4);
      ab.C = Zout + (size_t)b * H * NF;
      ab.sBz = (long long)D * F;
      ab.sCz = NF;
      TTR_HIP(launch_bgemm(dt, true, true, false, ab, H, s));
    }
    return hipSuccess;
  };
  TTR_HIP(proj(Q, zq));
  TTR_HIP(proj(K, zk));
  if (bias != nullptr) TTR_HIP(launch_add_bias(zq, zk, bias, B, H, N, F, s));

  // ks = sum_n phi(z_k); KV = phi(z_k)^T V
  TTR_HIP(launch_colsum_phi(zk, ks, Z, N, F, s));
  {
    BgemmArgs a{};
    a.A = zk;  // A(m = f, k = n) = phi(z_k[n][f])
    a.B = V;
    a.C = kv;
    a.M = F;
    a.N = D;
    a.K = N;
    a.KB = 1;
    a.sAz = NF;
    a.sAm = 1;
    a.sAk = F;
    a.sBz = ND;
    a.sBk = D;
    a.sBn = 1;
    a.sCz = FD;
    a.sCm = D;
    a.sCn = 1;
    TTR_HIP(launch_bgemm(dt, false, true, true, a, Z, s));
  }
  // num = phi(z_q) KV -> lin (in place after den)
  {
    BgemmArgs a{};
    a.A = zq;
    a.B = kv;
    a.C = lin;
    a.M = N;
    a.N = D;
    a.K = F;
    a.KB = 1;
    a.sAz = NF;
    a.sAm = F;
    a.sAk = 1;
    a.sBz = FD;
    a.sBk = D;
    a.sBn = 1;
    a.sCz = ND;
    a.sCm = D;
    a.sCn = 1;
    TTR_HIP(launch_bgemm(dt, false, false, true, a, Z, s));
  }
  TTR_HIP(launch_den_lin(zq, ks, lin, den, Z, N, F, D, eps, s));
  // landmark branch output (fp32), for dalpha
  if (L > 0) {
    HybridArgs ha = {};
    ha.Q = Q;
    ha.K = K;
    ha.V = V;
    ha.H = H;
    ha.N = N;
    ha.L = L;
    ha.out = lm;
    Problem pl = p;
    pl.proj = false;
    pl.F = p.D;
    TTR_HIP(launch_hybrid(pl, M_LM, false, ha, s));
  }
  return hipSuccess;
}

// Gradients from dout, after backward_forward_pass filled t.
static hipError_t backward_grad_pass(const Problem& p, const void* Q, const void* K, const void* V, const float* g,
                                     int L, const float* dout, float* dW, float* db, float* dg, const BwBufs& t,
                                     hipStream_t s) {
  float *zq = t.zq, *zk = t.zk, *dzq = t.dzq, *dzk = t.dzk, *lin = t.lin, *lm = t.lm, *dnum = t.dnum, *kv = t.kv;
  float *dkv = t.dkv, *ks = t.ks, *dks = t.dks, *den = t.den, *dden = t.dden, *rpart = t.rpart;
  const int B = p.B, H = p.H, N = p.N, D = p.D, F = p.F, Z = B * H, dt = p.dtype;
  const long long NF = (long long)N * F, ND = (long long)N * D, FD = (long long)F * D;
  // dnum, dden, dalpha row shares
  TTR_HIP(launch_dlin(dout, lin, lm, den, g, H, N, D, Z, L > 0, dnum, dden, rpart, s));
  // dphi_q = dnum KV^T (+ dden ks^T in dz): [N x D] . [D x F]
  {
    BgemmArgs a{};
    a.A = dnum;
    a.B = kv;  // B(k = d, n = f) = KV[f][d]
    a.C = dzq;
    a.M = N;
    a.N = F;
    a.K = D;
    a.KB = 1;
    a.sAz = ND;
    a.sAm = D;
    a.sAk = 1;
    a.sBz = FD;
    a.sBk = 1;
    a.sBn = D;
    a.sCz = NF;
    a.sCm = F;
    a.sCn = 1;
    TTR_HIP(launch_bgemm(dt, false, false, false, a, Z, s));
  }
  // dKV = phi(z_q)^T dnum: [F x N] . [N x D]; dks = phi(z_q)^T dden
  {
    BgemmArgs a{};
    a.A = zq;
    a.B = dnum;
    a.C = dkv;
    a.M = F;
    a.N = D;
    a.K = N;
    a.KB = 1;
    a.sAz = NF;
    a.sAm = 1;
    a.sAk = F;
    a.sBz = ND;
    a.sBk = D;
    a.sBn = 1;
    a.sCz = FD;
    a.sCm = D;
    a.sCn = 1;
    TTR_HIP(launch_bgemm(dt, false, false, true, a, Z, s));
  }
  TTR_HIP(launch_dks(zq, dden, dks, Z, N, F, s));
  // dz_q = (dphi_q + dden ks^T) phi'(z_q)
  TTR_HIP(launch_dz(dzq, zq, dden, ks, Z, N, F, s));
  // dphi_k = V dKV^T (+ dks in dz): [N x D] . [D x F]
  {
    BgemmArgs a{};
    a.A = V;
    a.B = dkv;  // B(k = d, n = f) = dKV[f][d]
    a.C = dzk;
    a.M = N;
    a.N = F;
    a.K = D;
    a.KB = 1;
    a.sAz = ND;
    a.sAm = D;
    a.sAk = 1;
    a.sBz = FD;
    a.sBk = 1;
    a.sBn = D;
    a.sCz = NF;
    a.sCm = F;
    a.sCn = 1;
    TTR_HIP(launch_bgemm(dt, true, false, false, a, Z, s));
  }
  TTR_HIP(launch_dz(dzk, zk, nullptr, dks, Z, N, F, s));
  // dW[h] = sum_b Q[b,h]^T dz_q[b,h] + K[b,h]^T dz_k[b,h]: the batch is the outer K loop
  auto dw = [&](const void* X, const float* dzv, int beta) {
    BgemmArgs a{};
    a.A = X;  // A(m = d, k = n) = X[n][d]
    a.B = dzv;
    a.C = dW;
    a.M = D;
    a.N = F;
    a.K = N;
    a.KB = B;
    a.sAz = ND;
    a.sAkb = (long long)H * ND;
    a.sAm = 1;
    a.sAk = D;
    a.sBz = NF;
    a.sBkb = (long long)H * NF;
    a.sBk = F;
    a.sBn = 1;
    a.sCz = (long long)D * F;
    a.sCm = F;
    a.sCn = 1;
    a.beta = beta;
    return launch_bgemm(dt, true, false, false, a, H, s);
  };
  TTR_HIP(dw(Q, dzq, 0));
  TTR_HIP(dw(K, dzk, 1));
  TTR_HIP(launch_db_dg(dzq, dzk, rpart, g, B, H, N, F, L > 0, db, dg, s));
  return hipSuccess;
}

hipError_t launch_hybrid_backward(const Problem& p, const void* Q, const void* K, const void* V, const void* W,
                                  const float* bias, const float* g, float eps, int L, const float* dout, float* dW,
                                  float* db, float* dg, void* ws, hipStream_t s) {
  const BwBufs t = bw_bufs(p, ws);
  TTR_HIP(backward_forward_pass(p, Q, K, V, W, bias, eps, L, t, s));
  return backward_grad_pass(p, Q, K, V, g, L, dout, dW, db, dg, t, s);
}

// ---------------------------------------------------------------- distillation step
// Per row (z, n), one wave: o = alpha lin + (1 - alpha) lm (lin alone when L == 0),
// t = the teacher row; writes dout = w1 clip(o - t, -1, 1) / numel - w2 dcos / rows,
// the row's huber sum and 1 - cos. w = exp(-s).
__global__ void distill_loss_rows_kernel(const float* lin, const float* lm, const float* teacher, const float* g,
                                         const float* sv, int H, int N, int D, int Z, int has_lm, float* dout,
                                         float* hrow, float* crow_) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= Z * N) return;
  const int h = (row / N) % H;
  const float alpha = has_lm ? 1.f / (1.f + expf(-g[h])) : 1.f;
  const float w1 = expf(-sv[0]), w2 = expf(-sv[1]);
  const float inv_numel = 1.f / ((float)Z * N * D), inv_rows = 1.f / ((float)Z * N);
  const float* li = lin + (size_t)row * D;
  const float* lr = lm + (size_t)row * D;
  const float* tr = teacher + (size_t)row * D;
  float ov[4], tv[4];  // D <= 256: up to 4 elements per lane
  float hs = 0.f, dot = 0.f, oo = 0.f, tt = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = lane + 64 * j;
    float o = 0.f, t = 0.f;
    if (d < D) {
      o = has_lm ? alpha * li[d] + (1.f - alpha) * lr[d] : li[d];
      t = tr[d];
      const float r = o - t, ar = fabsf(r);
      hs += ar <= 1.f ? 0.5f * r * r : ar - 0.5f;
    }
    ov[j] = o;
    tv[j] = t;
    dot += o * t;
    oo += o * o;
    tt += t * t;
  }
  for (int off = 32; off > 0; off >>= 1) {
    hs += __shfl_xor(hs, off);
    dot += __shfl_xor(dot, off);
    oo += __shfl_xor(oo, off);
    tt += __shfl_xor(tt, off);
  }
  const float no = sqrtf(oo), nt = sqrtf(tt);
  const float den = fmaxf(no * nt, 1e-8f);
  const float cosv = dot / den;
  const bool live = no * nt > 1e-8f;
  const float co = live ? dot * nt / (no * den * den) : 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = lane + 64 * j;
    if (d < D) {
      const float r = ov[j] - tv[j];
      const float dcos = tv[j] / den - co * ov[j];
      dout[(size_t)row * D + d] = w1 * fminf(fmaxf(r, -1.f), 1.f) * inv_numel - w2 * dcos * inv_rows;
    }
  }
  if (lane == 0) {
    hrow[row] = hs;
    crow_[row] = 1.f - cosv;
  }
}

// One workgroup: H = sum hrow / numel, C = sum crow / rows (fixed order);
// loss = w1 H + s1 + w2 C + s2; ds = (1 - w1 H, 1 - w2 C). out: loss, H, C.
__global__ void distill_loss_total_kernel(const float* hrow, const float* crow_, int rows, int D, const float* sv,
                                          float* loss_out, float* ds) {
  __shared__ float sh[256], sc[256];
  const int t = threadIdx.x;
  float h = 0.f, c = 0.f;
  for (int i = t; i < rows; i += 256) {
    h += hrow[i];
    c += crow_[i];
  }
  sh[t] = h;
  sc[t] = c;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (t < o) {
      sh[t] += sh[t + o];
      sc[t] += sc[t + o];
    }
    __syncthreads();
  }
  if (t == 0) {
    const float H = sh[0] / ((float)rows * D), C = sc[0] / (float)rows;
    const float w1 = expf(-sv[0]), w2 = expf(-sv[1]);
    loss_out[0] = w1 * H + sv[0] + w2 * C + sv[1];
    loss_out[1] = H;
    loss_out[2] = C;
    ds[0] = 1.f - w1 * H;
    ds[1] = 1.f - w2 * C;
  }
}

// Adam over the parameter blocks (W, b, g, s) with their gradients; moments
// [mW vW mb vb mg vg ms vs], bias-corrected at step `step` (from 1).
struct AdamArgs {
  float* p[4];
  const float* grad[4];
  float* moments;
  long long n[4];
  float lr, c1, c2;  // c1 = 1 - beta1^step, c2 = 1 - beta2^step
};
__global__ void adam_kernel(AdamArgs a) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  long long off = 0;
  for (int k = 0; k < 4; ++k) {
    if (i < a.n[k]) {
      float* m = a.moments + 2 * off;
      float* v = m + a.n[k];
      const float gr = a.grad[k][i];
      const float mi = 0.9f * m[i] + 0.1f * gr;
      const float vi = 0.999f * v[i] + 0.001f * gr * gr;
      m[i] = mi;
      v[i] = vi;
      a.p[k][i] -= a.lr * (mi / a.c1) / (sqrtf(vi / a.c2) + 1e-8f);
      return;
    }
    i -= a.n[k];
    off += a.n[k];
  }
}

// fp32 -> bf16 (round to nearest even)
__global__ void to_bf16_kernel(const float* x, uint16_t* y, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = f2bf(x[i]);
}

DistillLayout distill_layout(const Problem& p, bool need_teacher) {
  DistillLayout l;
  const size_t Z = (size_t)p.B * p.H, N = p.N, D = p.D, F = p.F, H = p.H;
  auto al = [](size_t n) { return (n + 255) & ~(size_t)255; };
  size_t o = al(backward_layout(p).bytes);
  l.w_io = o;
  o += al(p.dtype == 1 ? H * D * F * 2 : 0);
  l.teacher = o;
  o += al(need_teacher ? Z * N * D * 4 : 0);
  l.dout = o;
  o += al(Z * N * D * 4);
  l.hrow = o;
  o += al(Z * N * 4);
  l.crow = o;
  o += al(Z * N * 4);
  l.grads = o;  // dW | db | dg | ds
  o += al((H * D * F + H * F + H + 2) * 4);
  l.bytes = o;
  return l;
}

hipError_t launch_distill_step(const Problem& p, const void* Q, const void* K, const void* V, const float* teacher,
                               float* W, float* bias, float* g, float* sv, float* moments, int step, float lr,
                               float eps, int L, float* loss_out, void* ws, hipStream_t s) {
  const DistillLayout l = distill_layout(p, teacher == nullptr);
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  const int B = p.B, H = p.H, N = p.N, D = p.D, F = p.F, Z = B * H;
  const size_t nW = (size_t)H * D * F, nb = (size_t)H * F;
  // weights in the IO dtype for the forward and backward
  const void* Wio = W;
  if (p.dtype == 1) {
    uint16_t* wb = reinterpret_cast<uint16_t*>(w8 + l.w_io);
    hipLaunchKernelGGL(to_bf16_kernel, dim3(blocks(nW, 256)), dim3(256), 0, s, W, wb, nW);
    TTR_HIP(hipGetLastError());
    Wio = wb;
  }
  // teacher: softmax over every token (the landmark branch with L = N)
  const float* T = teacher;
  if (T == nullptr) {
    float* tw = reinterpret_cast<float*>(w8 + l.teacher);
    HybridArgs ha = {};
    ha.Q = Q;
    ha.K = K;
    ha.V = V;
    ha.H = H;
    ha.N = N;
    ha.L = N;
    ha.out = tw;
    Problem pl = p;
    pl.proj = false;
    pl.F = p.D;
    TTR_HIP(launch_hybrid(pl, M_LM, false, ha, s));
    T = tw;
  }
  const BwBufs t = bw_bufs(p, ws);
  TTR_HIP(backward_forward_pass(p, Q, K, V, Wio, bias, eps, L, t, s));
  float* dout = reinterpret_cast<float*>(w8 + l.dout);
  float* hrow = reinterpret_cast<float*>(w8 + l.hrow);
  float* crw = reinterpret_cast<float*>(w8 + l.crow);
  float* gr = reinterpret_cast<float*>(w8 + l.grads);
  float *dW = gr, *db = gr + nW, *dg = db + nb, *ds = dg + H;
  hipLaunchKernelGGL(distill_loss_rows_kernel, dim3(blocks((size_t)Z * N, 4)), dim3(256), 0, s, t.lin, t.lm, T, g,
                     sv, H, N, D, Z, L > 0 ? 1 : 0, dout, hrow, crw);
  TTR_HIP(hipGetLastError());
  hipLaunchKernelGGL(distill_loss_total_kernel, dim3(1), dim3(256), 0, s, hrow, crw, Z * N, D, sv, loss_out, ds);
  TTR_HIP(hipGetLastError());
  TTR_HIP(backward_grad_pass(p, Q, K, V, g, L, dout, dW, db, dg, t, s));
  AdamArgs a;
  a.p[0] = W;
  a.p[1] = bias;
  a.p[2] = g;
  a.p[3] = sv;
  a.grad[0] = dW;
  a.grad[1] = db;
  a.grad[2] = dg;
  a.grad[3] = ds;
  a.moments = moments;
  a.n[0] = (long long)nW;
  a.n[1] = (long long)nb;
  a.n[2] = H;
  a.n[3] = 2;
  a.lr = lr;
  a.c1 = 1.f - powf(0.9f, (float)step);
  a.c2 = 1.f - powf(0.999f, (float)step);
  hipLaunchKernelGGL(adam_kernel, dim3(blocks(nW + nb + H + 2, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttr

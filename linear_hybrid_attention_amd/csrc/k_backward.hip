// Backward of the hybrid forward for the trainable parameters W_h, b_h, g_h,
// and the Phase-1 distillation step around it ("Flux2TTRTrainer", section "How
// the distillation works": the TTR student regresses native softmax attention;
// huber and cosine terms weighed by learned uncertainties; per-layer
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
  const float* bias_n;  // optional: C(m, n) += bias_n[z * sbz + n]
  long long sbz;
  int ksplit;           // > 1: item z * ksplit + split per tile; partial sums go to part
  float* part;          // [Z][ksplit][M][N]
  // optional dz epilogue (no split-K): C(m, n) = (acc + r(m) s(n)) phi'(x(m, n)), phi = elu + 1,
  // x = dz_x laid out like C, r = dz_r[z * dz_srz + m] (1 when NULL), s = dz_s[z * dz_ssz + n]
  const float* dz_x;
  const uint16_t* dz_phi;  // (EPI 5, 6) instead of dz_x: phi(x) in bf16; phi'(x) = min(phi(x), 1)
  const float* dz_r;
  const float* dz_s;
  long long dz_srz, dz_ssz;
  // optional column sums of the epilogue (no split-K), as partials per (z, 64-row half
  // tile): [z][2 ceil(M / 128)][N], of the written values (cs_val), of elu1(dz_x) dz_r
  // (cs_phir) or of elu1 of the written values (cs_phi)
  float* cs_val;
  float* cs_phir;
  float* cs_phi;
  // optional (epilogue variants, beta = 0): the output rounded to bf16 here instead of C
  uint16_t* C16;
  int phi_out;  // (epilogue variant 4) the output is phi(acc + bias) in bf16, into C16
  // optional normaliser (no split-K; A = phi(x) rows, k contiguous): den(m) = sum_k A(m, k)
  // den_ks[z * den_ksz + k] + den_eps, written to den_out[z * den_oz + m] by the first N
  // tile, and C(m, n) = acc / den(m)
  const float* den_ks;
  long long den_ksz, den_oz;
  float* den_out;
  float den_eps;
};

template <typename CT> struct BgTile {
  static constexpr int TM = 128;                          // output rows per workgroup (operand A tile rows)
  static constexpr int TN = 64;                           // output columns per workgroup (operand B tile rows)
  static constexpr int KT = 32;                           // K per step
  static constexpr int LD = KT + 16 / (int)sizeof(CT);    // padded row (16-byte multiple)
};

template <typename T> __device__ __forceinline__ float ld_elem(const T* p, long long i);
template <> __device__ __forceinline__ float ld_elem<float>(const float* p, long long i) { return p[i]; }
template <> __device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p, long long i) { return bf2f(p[i]); }

template <typename CT> __device__ __forceinline__ CT to_ct(float x);
template <> __device__ __forceinline__ float to_ct<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t to_ct<uint16_t>(float x) { return f2bf(x); }

// NE consecutive elements at p (16-byte aligned) as floats
template <typename T, int NE> __device__ __forceinline__ void ld_run(const T* p, float (&v)[NE]) {
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int q = 0; q < NE / 4; ++q) {
      const f32x4 x = reinterpret_cast<const f32x4*>(p)[q];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * q + j] = x[j];
    }
  } else {
#pragma unroll
    for (int q = 0; q < NE / 8; ++q) {
      const u32x4 x = reinterpret_cast<const u32x4*>(p)[q];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * q + 2 * j] = __uint_as_float(x[j] << 16);
        v[8 * q + 2 * j + 1] = __uint_as_float(x[j] & 0xffff0000u);
      }
    }
  }
}

// Operand tile geometry: ROWS rows x KT k of one K-step, NE = ROWS / 8
// elements per thread (256 threads) along the operand's contiguous dimension.
// k_contig: thread t takes row t / TPR and k (t % TPR) NE .. + NE - 1 (TPR =
// KT / NE threads per row); else k t / 8 and rows (t % 8) NE .. + NE - 1.
// Whole runs inside the matrix and 16-byte aligned use vector loads; others
// load element by element with bounds (zeros outside). phi = elu + 1 applies
// to loaded elements only (outside stays 0).
template <int ROWS> struct BgGeo {
  static constexpr int NE = ROWS / 8, TPR = 32 / NE;
  __device__ static int kc_row(int t) { return t / TPR; }
  __device__ static int kc_k(int t) { return (t % TPR) * NE; }
  __device__ static int nk_k(int t) { return t / 8; }
  __device__ static int nk_row(int t) { return (t % 8) * NE; }
};

template <typename T, bool ELU, int ROWS>
__device__ __forceinline__ void bg_load(float (&v)[ROWS / 8], const T* base, long long s_row, long long s_k, int row0,
                                        int nrows, int k0, int K, bool k_contig, bool vec, int tid) {
  using G = BgGeo<ROWS>;
  constexpr int NE = G::NE;
  if (k_contig) {
    const int gr = row0 + G::kc_row(tid), gk = k0 + G::kc_k(tid);
    if (vec && gr < nrows && gk + NE <= K) {
      ld_run<T, NE>(base + (long long)gr * s_row + gk, v);  // s_k == 1 here
      if (ELU)
#pragma unroll
        for (int i = 0; i < NE; ++i) v[i] = elu1(v[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        float x = 0.f;
        if (gr < nrows && gk + i < K) {
          x = ld_elem<T>(base, (long long)gr * s_row + (long long)(gk + i) * s_k);
          if (ELU) x = elu1(x);
        }
        v[i] = x;
      }
    }
  } else {
    const int gk = k0 + G::nk_k(tid), gr = row0 + G::nk_row(tid);
    if (vec && gk < K && gr + NE <= nrows) {
      ld_run<T, NE>(base + (long long)gk * s_k + gr, v);  // s_row == 1 here
      if (ELU)
#pragma unroll
        for (int i = 0; i < NE; ++i) v[i] = elu1(v[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        float x = 0.f;
        if (gr + i < nrows && gk < K) {
          x = ld_elem<T>(base, (long long)(gr + i) * s_row + (long long)gk * s_k);
          if (ELU) x = elu1(x);
        }
        v[i] = x;
      }
    }
  }
}
template <typename CT, int ROWS>
__device__ __forceinline__ void bg_store(CT* tile, const float (&v)[ROWS / 8], bool k_contig, int tid) {
  using G = BgGeo<ROWS>;
  constexpr int LD = BgTile<CT>::LD, NE = G::NE;
  if (k_contig) {
    CT* p = tile + G::kc_row(tid) * LD + G::kc_k(tid);
#pragma unroll
    for (int i = 0; i < NE; ++i) p[i] = to_ct<CT>(v[i]);
  } else {
    CT* p = tile + G::nk_row(tid) * LD + G::nk_k(tid);
#pragma unroll
    for (int i = 0; i < NE; ++i) p[i * LD] = to_ct<CT>(v[i]);
  }
}

// The same tile move for a 16-bit operand going to a 16-bit tile unchanged:
// the elements stay packed (NE / 2 registers) and are stored as they came.
template <int ROWS>
__device__ __forceinline__ void bg_load_raw(u32x4 (&v)[ROWS / 64], const uint16_t* base, long long s_row,
                                            long long s_k, int row0, int nrows, int k0, int K, bool k_contig,
                                            bool vec, int tid) {
  using G = BgGeo<ROWS>;
  constexpr int NE = G::NE;
  uint16_t e[NE];
  if (k_contig) {
    const int gr = row0 + G::kc_row(tid), gk = k0 + G::kc_k(tid);
    if (vec && gr < nrows && gk + NE <= K) {
      const u32x4* q = reinterpret_cast<const u32x4*>(base + (long long)gr * s_row + gk);
#pragma unroll
      for (int u = 0; u < NE / 8; ++u) v[u] = q[u];
      return;
    }
#pragma unroll
    for (int i = 0; i < NE; ++i)
      e[i] = (gr < nrows && gk + i < K) ? base[(long long)gr * s_row + (long long)(gk + i) * s_k] : (uint16_t)0;
  } else {
    const int gk = k0 + G::nk_k(tid), gr = row0 + G::nk_row(tid);
    if (vec && gk < K && gr + NE <= nrows) {
      const u32x4* q = reinterpret_cast<const u32x4*>(base + (long long)gk * s_k + gr);
#pragma unroll
      for (int u = 0; u < NE / 8; ++u) v[u] = q[u];
      return;
    }
#pragma unroll
    for (int i = 0; i < NE; ++i)
      e[i] = (gr + i < nrows && gk < K) ? base[(long long)(gr + i) * s_row + (long long)gk * s_k] : (uint16_t)0;
  }
#pragma unroll
  for (int u = 0; u < NE / 8; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) v[u][j] = (uint32_t)e[8 * u + 2 * j] | ((uint32_t)e[8 * u + 2 * j + 1] << 16);
}
template <int ROWS>
__device__ __forceinline__ void bg_store_raw(uint16_t* tile, const u32x4 (&v)[ROWS / 64], bool k_contig, int tid) {
  using G = BgGeo<ROWS>;
  constexpr int LD = BgTile<uint16_t>::LD, NE = G::NE;
  if (k_contig) {
    u32x4* p = reinterpret_cast<u32x4*>(tile + G::kc_row(tid) * LD + G::kc_k(tid));
#pragma unroll
    for (int u = 0; u < NE / 8; ++u) p[u] = v[u];
  } else {
    uint16_t* p = tile + G::nk_row(tid) * LD + G::nk_k(tid);
#pragma unroll
    for (int i = 0; i < NE; ++i) p[i * LD] = (uint16_t)(v[i >> 3][(i & 7) >> 1] >> (16 * (i & 1)));
  }
}

// The thread's run for unconditional vector loads (the host has checked the
// alignment, K % KT == 0 and, for row-strided operands, whole row groups): a
// row past nrows reads a valid row instead; it only feeds output rows or
// columns that are never stored.
template <typename T, int ROWS>
__device__ __forceinline__ const T* bg_fast_ptr(const T* base, long long s_row, long long s_k, int row0, int nrows,
                                                int k0, bool k_contig, int tid) {
  using G = BgGeo<ROWS>;
  if (k_contig) return base + (long long)min(row0 + G::kc_row(tid), nrows - 1) * s_row + (k0 + G::kc_k(tid));
  return base + (long long)(k0 + G::nk_k(tid)) * s_k + min(row0 + G::nk_row(tid), nrows - G::NE);
}

// One operand's staging registers for a K-step: packed 16-bit elements when
// they go to the tile unchanged, else floats (converted or mapped on the way).
template <typename CT, typename T, bool ELU, int ROWS>
struct BgStage {
  float v[ROWS / 8];
  __device__ __forceinline__ float val(int i) const { return v[i]; }
  __device__ __forceinline__ void load(const T* base, long long s_row, long long s_k, int row0, int nrows, int k0,
                                       int K, bool kc, bool vec, int tid) {
    bg_load<T, ELU, ROWS>(v, base, s_row, s_k, row0, nrows, k0, K, kc, vec, tid);
  }
  __device__ __forceinline__ void load_fast(const T* base, long long s_row, long long s_k, int row0, int nrows,
                                            int k0, bool kc, int tid) {
    ld_run<T, ROWS / 8>(bg_fast_ptr<T, ROWS>(base, s_row, s_k, row0, nrows, k0, kc, tid), v);
    if (ELU)
#pragma unroll
      for (int i = 0; i < ROWS / 8; ++i) v[i] = elu1(v[i]);
  }
  __device__ __forceinline__ void store(CT* tile, bool kc, int tid) const { bg_store<CT, ROWS>(tile, v, kc, tid); }
  // (a row-strided operand into a bf16 tile stored [k][row], kTrRead layout:
  // the thread's NE consecutive rows at its k are whole 16-byte pieces)
  __device__ __forceinline__ void store_tr(uint16_t* tile, int tid) const {
    using G = BgGeo<ROWS>;
#pragma unroll
    for (int u = 0; u < G::NE / 8; ++u) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(v[8 * u + 2 * j], v[8 * u + 2 * j + 1]);
      *reinterpret_cast<u32x4*>(tile + toff<ROWS, kTrRead>(G::nk_k(tid), G::nk_row(tid) + 8 * u)) = w;
    }
  }
};
template <int ROWS>
struct BgStage<uint16_t, uint16_t, false, ROWS> {
  u32x4 v[ROWS / 64];
  __device__ __forceinline__ float val(int i) const {
    const uint32_t w = v[i >> 3][(i & 7) >> 1];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ __forceinline__ void load(const uint16_t* base, long long s_row, long long s_k, int row0, int nrows,
                                       int k0, int K, bool kc, bool vec, int tid) {
    bg_load_raw<ROWS>(v, base, s_row, s_k, row0, nrows, k0, K, kc, vec, tid);
  }
  __device__ __forceinline__ void load_fast(const uint16_t* base, long long s_row, long long s_k, int row0,
                                            int nrows, int k0, bool kc, int tid) {
    const u32x4* q = reinterpret_cast<const u32x4*>(bg_fast_ptr<uint16_t, ROWS>(base, s_row, s_k, row0, nrows, k0, kc, tid));
#pragma unroll
    for (int u = 0; u < ROWS / 64; ++u) v[u] = q[u];
  }
  __device__ __forceinline__ void store(uint16_t* tile, bool kc, int tid) const {
    bg_store_raw<ROWS>(tile, v, kc, tid);
  }
  __device__ __forceinline__ void store_tr(uint16_t* tile, int tid) const {
    using G = BgGeo<ROWS>;
#pragma unroll
    for (int u = 0; u < G::NE / 8; ++u)
      *reinterpret_cast<u32x4*>(tile + toff<ROWS, kTrRead>(G::nk_k(tid), G::nk_row(tid) + 8 * u)) = v[u];
  }
};

// Work item of workgroup i in a one-dimensional grid of n: the hardware places
// workgroup i on XCD i % 8, so items are renumbered such that consecutive ones
// run on one XCD (the N tiles of one M tile share that XCD's L2 copy of A).
__device__ __forceinline__ int bg_item(int i, int n) {
  const int per = n / 8;
  return i < per * 8 ? (i % 8) * per + i / 8 : i;
}

// 128 x 64 output tile per workgroup, 4 waves of 32 x 64 (1 x 2 MFMA tiles):
// a small accumulator, so that four workgroups share a compute unit and their
// memory phases overlap. Workgroup items run N tile fastest, then M tile, then
// z * ksplit + split. EPI: the epilogue's dz and column-sum terms (0: none;
// never with split-K); O16: that epilogue's output in bf16. DEN: the normaliser
// of each row is formed from the staged A rows (thread pair t, t + 1 holds one
// row's k run of a step) and divides the row (never with split-K).
constexpr int kDenMaxK = 512;  // the normaliser's K (the feature count) at most
template <typename CT, typename TA, typename TB, bool A_ELU, int EPI, bool DEN = false, bool O16 = false,
          bool FAST = false, bool TT = false, bool BT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DEN ? 3 : 4))) void bgemm_kernel(BgemmArgs a) {
  constexpr int TM = BgTile<CT>::TM, TN = BgTile<CT>::TN, KT = BgTile<CT>::KT, LD = BgTile<CT>::LD;
  __shared__ __attribute__((aligned(16))) CT As[TM * LD];
  __shared__ __attribute__((aligned(16))) CT Bs[TN * LD];  // B^T: [64 n][KT]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int mtiles = (a.M + TM - 1) / TM, ntiles = (a.N + TN - 1) / TN;
  const int item = bg_item(blockIdx.x, gridDim.x), rest = item / ntiles;
  const int ntile = item % ntiles, mtile = rest % mtiles, zs = rest / mtiles;
  const int m0 = mtile * TM, n0 = ntile * TN, z = zs / a.ksplit, split = zs % a.ksplit;
  const TA* A = static_cast<const TA*>(a.A) + z * a.sAz;
  const TB* B = static_cast<const TB*>(a.B) + z * a.sBz;
  const bool a_kc = a.sAk == 1, b_kc = a.sBk == 1;
  // vector loads need 16-byte aligned runs: every stride of the operand a multiple of 16 bytes
  constexpr int PA = 16 / sizeof(TA), PB = 16 / sizeof(TB);
  // (the run's own stride must be 1: k for k_contig, else the rows)
  const bool a_vec = (a_kc || a.sAm == 1) && ((a_kc ? a.sAm : a.sAk) % PA == 0) && (a.sAz % PA == 0) &&
                     (a.sAkb % PA == 0) && ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0);
  const bool b_vec = (b_kc || a.sBn == 1) && ((b_kc ? a.sBn : a.sBk) % PB == 0) && (a.sBz % PB == 0) &&
                     (a.sBkb % PB == 0) && ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0);

  f32x16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[j] = f32x16{};
  BgStage<CT, TA, A_ELU, TM> va;
  BgStage<CT, TB, false, TN> vb;
  const int nks = (a.K + KT - 1) / KT, steps = a.KB * nks;
  const int per = (steps + a.ksplit - 1) / a.ksplit, s_begin = split * per, total = min(steps, s_begin + per);
  auto load = [&](int s) {
    const int kb = s / nks, k0 = (s % nks) * KT;
    if constexpr (FAST) {
      va.load_fast(A + kb * a.sAkb, a.sAm, a.sAk, m0, a.M, k0, a_kc, tid);
      vb.load_fast(B + kb * a.sBkb, a.sBn, a.sBk, n0, a.N, k0, b_kc, tid);
    } else {
      va.load(A + kb * a.sAkb, a.sAm, a.sAk, m0, a.M, k0, a.K, a_kc, a_vec, tid);
      vb.load(B + kb * a.sBkb, a.sBn, a.sBk, n0, a.N, k0, a.K, b_kc, b_vec, tid);
    }
  };
  float dpart = 0.f;  // DEN: this thread's share of its row's phi(A) . ks
  __shared__ __attribute__((aligned(16))) float ksh[DEN ? kDenMaxK : 1];  // DEN: ks, zero past K
  if constexpr (DEN)
    for (int k = tid; k < kDenMaxK; k += 256) ksh[k] = k < a.K ? a.den_ks[z * a.den_ksz + k] : 0.f;
  if (s_begin < total) load(s_begin);
  for (int s = s_begin; s < total; ++s) {
    __syncthreads();  // every wave is done with the previous tile (and, DEN, ksh is written)
    if constexpr (DEN) {  // (A is k-contiguous: the thread's 16 values are k0 + (tid % 2) 16 ..)
      const f32x4* kp = reinterpret_cast<const f32x4*>(ksh + (s % nks) * KT + (tid % 2) * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 kv = kp[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) dpart += va.val(4 * q + i) * kv[i];
      }
    }
    if constexpr (TT) {  // both operands row-strided: [k][row] tiles
      va.store_tr(As, tid);
      vb.store_tr(Bs, tid);
    } else if constexpr (BT) {  // B row-strided: its tile [k][row]; A's as usual
      va.store(As, true, tid);
      vb.store_tr(Bs, tid);
    } else {
      va.store(As, a_kc, tid);
      vb.store(Bs, b_kc, tid);
    }
    __syncthreads();
    if (s + 1 < total) load(s + 1);  // in flight during the products
#pragma unroll
    for (int kb = 0; kb < KT / 16; ++kb) {
      Frag<CT> fa, fb[2];
      if constexpr (TT) {  // transposed reads: both fragments hold k in the same (C-row) order
        fa = tr_frag<TM>(As, kb * 16, w * 32, lane);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = tr_frag<TN>(Bs, kb * 16, j * 32, lane);
      } else if constexpr (BT) {  // A's k values in that order: k0 + 4g .. + 3, then k0 + 8 + 4g .. + 3
        const uint16_t* ap = As + (w * 32 + c) * LD + kb * 16 + 4 * g;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(ap), hi = *reinterpret_cast<const u32x2*>(ap + 8);
        fa = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = tr_frag<TN>(Bs, kb * 16, j * 32, lane);
      } else {
        fa = ld_frag<CT>(As + (w * 32 + c) * LD + kb * 16 + 8 * g);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = ld_frag<CT>(Bs + (j * 32 + c) * LD + kb * 16 + 8 * g);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) mma(acc[j], fa, fb[j]);
    }
  }
  // lane (c, g) holds, per tile j, column n0 + j*32 + c and rows m0 + w*32 + crow(lane, r)
  const int mb = m0 + w * 32;
  if constexpr (DEN) {
    __shared__ float dsh[TM];
    dpart += __shfl_xor(dpart, 1);
    if ((tid & 1) == 0) dsh[tid >> 1] = dpart + a.den_eps;
    __syncthreads();
    if (ntile == 0 && tid < TM && m0 + tid < a.M) a.den_out[z * a.den_oz + m0 + tid] = dsh[tid];
    float* __restrict__ Cz = a.C + z * a.sCz;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + j * 32 + c;
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ml = w * 32 + crow(lane, r), m = m0 + ml;
        if (m < a.M) Cz[(long long)m * a.sCm + (long long)n * a.sCn] = acc[j][r] / dsh[ml];
      }
    }
    return;
  }
  if constexpr (EPI == 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + j * 32 + c;
      if (n >= a.N) continue;  // (lanes c and c + 32 share n: both skip or both go on)
      if (a.ksplit > 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mb + crow(lane, r);
          if (m < a.M) a.part[((size_t)zs * a.M + m) * a.N + n] = acc[j][r];
        }
        continue;
      }
      const float bn = a.bias_n ? a.bias_n[z * a.sbz + n] : 0.f;
      float* __restrict__ Cz = a.C + z * a.sCz + (long long)n * a.sCn;
      if (m0 + TM <= a.M && !a.beta) {  // a full tile, written over: no row checks
#pragma unroll
        for (int r = 0; r < 16; ++r) Cz[(long long)(mb + crow(lane, r)) * a.sCm] = acc[j][r] + bn;
        continue;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + crow(lane, r);
        if (m >= a.M) continue;
        float* p = Cz + (long long)m * a.sCm;
        *p = (a.beta ? *p + acc[j][r] : acc[j][r]) + bn;
      }
    }
    return;
  }
  // Epilogue with the dz products and column sums (no split-K, beta = 0), its
  // terms fixed by EPI: 1: dz with the row factor r = dz_r, the column sums of
  // dz (cs_val) and of phi(x) r (cs_phir); 2: dz with r = 1 and the column sums
  // of dz; 3: the column sums of phi of the output (cs_phi); 4: phi of the
  // output (with O16); 5, 6: as 1, 2 with the dz operand given as phi(x) in
  // bf16 (dz_phi). O16: the output rounded to bf16 into C16. Offsets within a z slice are 32-bit (the host
  // checks the slice's extent); full tiles store without row checks.
  constexpr bool XP = EPI == 5 || EPI == 6;  // the dz operand is phi(x) in bf16
  constexpr bool DZ = EPI == 1 || EPI == 2 || XP, HAS_R = EPI == 1 || EPI == 5, CSV = DZ,
                 CSR = HAS_R, CSQ = EPI == 3, PHI_OUT = EPI == 4;
  const long long zo = (long long)z * a.sCz;
  const float* __restrict__ dzx = DZ && !XP ? a.dz_x + zo : nullptr;
  const uint16_t* __restrict__ dzp = XP ? a.dz_phi + zo : nullptr;
  float* __restrict__ Cz = O16 ? nullptr : a.C + zo;
  uint16_t* __restrict__ Cz16 = O16 ? a.C16 + zo : nullptr;
  const int sCm = (int)a.sCm, sCn = (int)a.sCn;
  const bool full = m0 + TM <= a.M;  // every row of the tile exists (workgroup-uniform)
  __shared__ float csw[3][4][64];  // per wave: its 32 rows' column sums
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + j * 32 + c;
    float cv = 0.f, cp = 0.f, cq = 0.f;  // this lane's column sums over its rows
    if (n < a.N) {  // (lanes c and c + 32 share n: both skip or both go on)
      const float bn = a.bias_n ? a.bias_n[z * a.sbz + n] : 0.f;
      const float sn = DZ ? a.dz_s[z * a.dz_ssz + n] : 0.f;
      // the dz operands of the 16 rows are loaded before any store
      float xv[16], rv[16];
      if constexpr (DZ) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = min(mb + crow(lane, r), a.M - 1);
          xv[r] = XP ? bf2f(dzp[m * sCm + n * sCn]) : dzx[m * sCm + n * sCn];
          rv[r] = HAS_R ? a.dz_r[z * a.dz_srz + m] : 1.f;
        }
      }
      auto emit = [&](int r, int m) __attribute__((always_inline)) {
        const int off = m * sCm + n * sCn;
        float v = acc[j][r] + bn;
        if constexpr (DZ) {  // dz = (dphi + r s) phi'(x), phi'(x) = 1 for x > 0, exp(x) otherwise
          const float dp = v + rv[r] * sn;
          if constexpr (XP) v = dp * fminf(xv[r], 1.f);  // (phi(x) = exp(x) <= 1 for x <= 0, x + 1 > 1 else)
          else v = xv[r] > 0.f ? dp : dp * __expf(xv[r]);
          if constexpr (CSR) cp += (XP ? xv[r] : elu1(xv[r])) * rv[r];
        }
        if constexpr (PHI_OUT) v = elu1(v);
        if constexpr (CSV) cv += v;
        if constexpr (CSQ) cq += elu1(v);
        if constexpr (O16) Cz16[off] = f2bf(v);  // (the column sums above use the fp32 value)
        else Cz[off] = v;
      };
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) emit(r, mb + crow(lane, r));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mb + crow(lane, r);
          if (m < a.M) emit(r, m);
        }
      }
    }
    // the column's two lanes (rows 4g..) combine; the wave's sums go to LDS
    cv += __shfl_xor(cv, 32);
    cp += __shfl_xor(cp, 32);
    cq += __shfl_xor(cq, 32);
    if (g == 0) {
      csw[0][w][j * 32 + c] = cv;
      csw[1][w][j * 32 + c] = cp;
      csw[2][w][j * 32 + c] = cq;
    }
  }
  __syncthreads();
  // one partial per (z, 64-row half tile): waves 2h and 2h + 1, added in that order
  if (tid < 128) {
    const int h = tid >> 6, col = tid & 63, n = n0 + col;
    if (n < a.N) {
      const size_t at = ((size_t)z * (2 * mtiles) + 2 * mtile + h) * a.N + n;
      if constexpr (CSV) a.cs_val[at] = csw[0][2 * h][col] + csw[0][2 * h + 1][col];
      if constexpr (CSR) a.cs_phir[at] = csw[1][2 * h][col] + csw[1][2 * h + 1][col];
      if constexpr (CSQ) a.cs_phi[at] = csw[2][2 * h][col] + csw[2][2 * h + 1][col];
    }
  }
}

// C[z](m, n) = (beta ? C : 0) + bias + sum_split part[z][split](m, n), splits in order
__global__ void bgemm_reduce_kernel(BgemmArgs a, int Z) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t mn = (size_t)a.M * a.N;
  if (i >= (size_t)Z * mn) return;
  const int z = (int)(i / mn), m = (int)((i % mn) / a.N), n = (int)(i % a.N);
  float* p = a.C + z * a.sCz + (long long)m * a.sCm + (long long)n * a.sCn;
  float v = a.beta ? *p : 0.f;
  const float* P = a.part + (size_t)z * a.ksplit * mn + (size_t)m * a.N + n;
  // every split's load issued before the first add (ksplit <= 16), added in order
  float x[16];
#pragma unroll
  for (int sp = 0; sp < 16; ++sp) x[sp] = sp < a.ksplit ? P[(size_t)sp * mn] : 0.f;
#pragma unroll
  for (int sp = 0; sp < 16; ++sp)
    if (sp < a.ksplit) v += x[sp];
  if (a.bias_n) v += a.bias_n[z * a.sbz + n];
  *p = v;
}

// The unconditional-load variant's conditions: both operands 16-byte aligned
// with whole runs (as the kernel's vector path requires), K a multiple of the
// K-step, and whole row groups for an operand whose rows are contiguous.
template <typename TA, typename TB>
static bool bg_fast(const BgemmArgs& a) {
  const long long PA = 16 / sizeof(TA), PB = 16 / sizeof(TB);
  const bool a_kc = a.sAk == 1, b_kc = a.sBk == 1;
  const bool a_vec = (a_kc || a.sAm == 1) && ((a_kc ? a.sAm : a.sAk) % PA == 0) && (a.sAz % PA == 0) &&
                     (a.sAkb % PA == 0) && ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0);
  const bool b_vec = (b_kc || a.sBn == 1) && ((b_kc ? a.sBn : a.sBk) % PB == 0) && (a.sBz % PB == 0) &&
                     (a.sBkb % PB == 0) && ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0);
  return a_vec && b_vec && a.K % 32 == 0 && (a_kc || (a.M >= 16 && a.M % 16 == 0)) &&
         (b_kc || (a.N >= 8 && a.N % 8 == 0));
}

template <typename CT, typename TA, typename TB, bool ELU, int EPI = 0, bool DEN = false, bool O16 = false,
          bool TT = false, bool BT = false>
static hipError_t launch_bgemm_t(const BgemmArgs& a, int Z, hipStream_t s) {
  const dim3 grid((unsigned)(((a.M + 127) / 128) * ((a.N + 63) / 64) * Z * a.ksplit));
  if (bg_fast<TA, TB>(a))
    hipLaunchKernelGGL((bgemm_kernel<CT, TA, TB, ELU, EPI, DEN, O16, true, TT, BT>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bgemm_kernel<CT, TA, TB, ELU, EPI, DEN, O16, false, TT, BT>), grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ksplit == 1) return e;
  const size_t n = (size_t)Z * a.M * a.N;
  hipLaunchKernelGGL(bgemm_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, Z);
  return hipGetLastError();
}

// dtype: 1 = bf16 IO (bf16 MFMA), 0 = fp32 IO (fp32 MFMA). a_io / b_io: the
// operand is in the IO dtype (else fp32).
// Split-K scratch of the backward: enough for 16 partial products of F x D per slice.
static size_t splitk_elems(const Problem& p) { return (size_t)16 * p.B * p.H * p.F * p.D; }

// A grid of few tiles with a long reduction splits K (at most 16 ways, at
// least 8 steps each, aiming at about 1024 workgroups), when `scratch` holds
// the partial products.
static hipError_t launch_bgemm(int dtype, bool a_io, bool b_io, bool a_elu, const BgemmArgs& a0, int Z, hipStream_t s,
                               float* scratch = nullptr, size_t scratch_elems = 0) {
  BgemmArgs a = a0;
  a.ksplit = 1;
  a.part = nullptr;
  if (a.dz_s != nullptr || a.cs_val || a.cs_phir || a.cs_phi || a.den_ks) scratch = nullptr;  // epilogue work: no split-K
  const int tiles = ((a.M + 127) / 128) * ((a.N + 63) / 64) * Z;
  const int steps = a.KB * ((a.K + 31) / 32);
  if (scratch != nullptr && tiles < 512 && steps >= 32) {
    int ks = min(16, max(1, 1024 / tiles));
    ks = min(ks, steps / 8);
    while (ks > 1 && (size_t)ks * Z * a.M * a.N > scratch_elems) --ks;
    if (ks > 1) {
      a.ksplit = ks;
      a.part = scratch;
    }
  }
  // The epilogue's terms select its variant (EPI 1: dz with a row factor, with
  // the column sums of dz and of phi(x) r; 2: dz, with the column sums of dz; 3:
  // the column sums of phi of the output); the variants exist for the operand
  // kinds the products use, other combinations are refused.
  // (4: phi of the output in bf16; 5, 6: as 1, 2 with the dz operand given as
  // phi(x) in bf16)
  int epi = 0;
  if (a.dz_s != nullptr) {
    if (!a.cs_val || a.cs_phi || a.phi_out || (a.dz_r != nullptr) != (a.cs_phir != nullptr)) return hipErrorInvalidValue;
    if ((a.dz_x != nullptr) == (a.dz_phi != nullptr)) return hipErrorInvalidValue;
    epi = a.dz_phi ? (a.dz_r ? 5 : 6) : (a.dz_r ? 1 : 2);
  } else if (a.cs_val || a.cs_phir) {
    return hipErrorInvalidValue;
  } else if (a.cs_phi) {
    if (a.phi_out) return hipErrorInvalidValue;
    epi = 3;
  } else if (a.phi_out) {
    epi = 4;
  }
  if (epi != 0) {
    if (a_elu || a.beta) return hipErrorInvalidValue;
    // offsets within a slice are 32-bit
    const long long ext = (long long)(a.M - 1) * a.sCm + (long long)(a.N - 1) * a.sCn;
    if (ext > 0x7fffffffLL || a.sCm > 0x7fffffffLL || a.sCn > 0x7fffffffLL) return hipErrorInvalidValue;
  }
  const bool o16 = a.C16 != nullptr;
  if (o16 && (epi == 0 || epi == 3 || dtype != 1)) return hipErrorInvalidValue;
  if (epi >= 4 && (!o16 || dtype != 1)) return hipErrorInvalidValue;  // (bf16 outputs of the bf16 path)
  if (a.den_ks != nullptr) {  // phi rows as A (fp32 mapped on staging, or bf16 phi), k contiguous, fp32 B
    if (epi != 0 || b_io || a.sAk != 1 || a.K > kDenMaxK || a.KB != 1) return hipErrorInvalidValue;
    if (dtype == 1 && a_io && !a_elu && a.sBk != 1)
      return launch_bgemm_t<uint16_t, uint16_t, float, false, 0, true, false, false, true>(a, Z, s);
    if (!a_elu || a_io) return hipErrorInvalidValue;
    if (dtype == 1 && a.sBk != 1)  // B row-strided (lin: KV)
      return launch_bgemm_t<uint16_t, float, float, true, 0, true, false, false, true>(a, Z, s);
    return dtype == 1 ? launch_bgemm_t<uint16_t, float, float, true, 0, true>(a, Z, s)
                      : launch_bgemm_t<float, float, float, true, 0, true>(a, Z, s);
  }
  if (epi != 0) {
    if (dtype == 1) {
      if (epi == 1 && o16 && !a_io && !b_io) return launch_bgemm_t<uint16_t, float, float, false, 1, false, true>(a, Z, s);
      if (epi == 1 && o16 && a_io && !b_io) return launch_bgemm_t<uint16_t, uint16_t, float, false, 1, false, true>(a, Z, s);
      if (epi == 5 && o16 && a_io && !b_io) return launch_bgemm_t<uint16_t, uint16_t, float, false, 5, false, true>(a, Z, s);
      if (epi == 6 && o16 && a_io && !b_io) return launch_bgemm_t<uint16_t, uint16_t, float, false, 6, false, true>(a, Z, s);
      if (epi == 4 && o16 && a_io && b_io && a.sAk == 1 && a.sBk != 1)
        return launch_bgemm_t<uint16_t, uint16_t, uint16_t, false, 4, false, true, false, true>(a, Z, s);
      if (epi == 2 && o16 && a_io && !b_io) return launch_bgemm_t<uint16_t, uint16_t, float, false, 2, false, true>(a, Z, s);
      if (epi == 3 && a_io && b_io) return launch_bgemm_t<uint16_t, uint16_t, uint16_t, false, 3>(a, Z, s);
      return hipErrorInvalidValue;
    }
    if (epi == 1) return launch_bgemm_t<float, float, float, false, 1>(a, Z, s);
    if (epi == 2) return launch_bgemm_t<float, float, float, false, 2>(a, Z, s);
    return launch_bgemm_t<float, float, float, false, 3>(a, Z, s);
  }
  // bf16 products whose operands are both row-strided (dW, dKV) stage them as
  // [k][row] tiles read by transposing LDS reads: whole 16-byte stores instead
  // of scattered 2-byte ones
  const bool tt = a.sAk != 1 && a.sBk != 1;
  if (dtype == 1 && tt && a_io && b_io && !a_elu) return launch_bgemm_t<uint16_t, uint16_t, uint16_t, false, 0, false, false, true>(a, Z, s);
  if (dtype == 1 && tt && !a_io && !b_io && a_elu) return launch_bgemm_t<uint16_t, float, float, true, 0, false, false, true>(a, Z, s);
  if (dtype == 1 && tt && !a_io && b_io && a_elu) return launch_bgemm_t<uint16_t, float, uint16_t, true, 0, false, false, true>(a, Z, s);
  // B alone row-strided (z = X W + b): its tile [k][row], A's fragments read in the same k order
  if (dtype == 1 && epi == 0 && a.sAk == 1 && a.sBk != 1 && a_io && b_io && !a_elu)
    return launch_bgemm_t<uint16_t, uint16_t, uint16_t, false, 0, false, false, false, true>(a, Z, s);
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
// Column sums from the GEMM epilogues' half-tile partials, in a fixed order:
// out[o][n] = sum_{b < nb} (sum_{t < t1} p1[(b zs + o)][t][n] + sum_{t < t2} p2[(b zs + o)][t][n])
// (p2 may be NULL). Workgroup (x, o): columns 64 x .. 64 x + 63 of output row o;
// thread group q (0..3) adds the partials t = q, q + 4, ... in order, and the
// four group sums are added in order.
__global__ __launch_bounds__(256) void tile_colsum_kernel(const float* p1, int t1, const float* p2, int t2, int nb,
                                                          int zs, int ncol, float* out) {
  __shared__ float sh[4][64];
  const int n = blockIdx.x * 64 + (threadIdx.x & 63), q = threadIdx.x >> 6, o = blockIdx.y;
  float s = 0.f;
  if (n < ncol) {
    for (int b = 0; b < nb; ++b) {
      const size_t zz = (size_t)b * zs + o;
#pragma unroll 8
      for (int t = q; t < t1; t += 4) s += p1[(zz * t1 + t) * ncol + n];
      if (p2 != nullptr)
#pragma unroll 8
        for (int t = q; t < t2; t += 4) s += p2[(zz * t2 + t) * ncol + n];
    }
  }
  sh[q][threadIdx.x & 63] = s;
  __syncthreads();
  if (q == 0 && n < ncol) out[(size_t)o * ncol + n] = ((sh[0][threadIdx.x] + sh[1][threadIdx.x]) + sh[2][threadIdx.x]) +
                                                      sh[3][threadIdx.x];
}

// Per row: dlin = alpha dout; dnum = dlin / den; dden = -sum_d dlin lin / den;
// and the row's share of dalpha: sum_d dout (lin - lm) (into rpart[row]).
__global__ void dlin_kernel(const float* dout, const float* lin, const float* lm, const float* den, const float* g,
                            int H, int N, int D, int Z, int has_lm, float* dnum, uint16_t* dnum16, float* dden,
                            float* rpart) {
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
    if (dnum16) dnum16[(size_t)row * D + d] = f2bf(dl * inv);
    else dnum[(size_t)row * D + d] = dl * inv;
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

// dg[h] = alpha (1 - alpha) sum_{b, n} rpart[(b H + h) NQ + n] (0 without
// landmarks): one workgroup per head, each thread adds a strided run of the
// rows in order, then a fixed-order tree over the threads.
__global__ __launch_bounds__(256) void dg_kernel(const float* rpart, const float* g, int B, int H, int NQ,
                                                 int has_lm, float* dg) {
  __shared__ float sh[256];
  const int h = blockIdx.x, t = threadIdx.x;
  float s = 0.f;
  for (int b = 0; b < B; ++b) {
    const float* r = rpart + ((size_t)b * H + h) * NQ;
#pragma unroll 8
    for (int n = t; n < NQ; n += 256) s += r[n];
  }
  sh[t] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (t < o) sh[t] += sh[t + o];
    __syncthreads();
  }
  if (t == 0) {
    const float al = has_lm ? 1.f / (1.f + expf(-g[h])) : 0.f;
    dg[h] = has_lm ? sh[0] * al * (1.f - al) : 0.f;
  }
}

// ---------------------------------------------------------------- launches
static unsigned blocks(size_t n, unsigned t) { return (unsigned)((n + t - 1) / t); }
static int half_tiles(int rows) { return 2 * ((rows + 127) / 128); }
static hipError_t launch_tile_colsum(const float* p1, int t1, const float* p2, int t2, int nb, int zs, int ncol,
                                     int nout, float* out, hipStream_t s) {
  hipLaunchKernelGGL(tile_colsum_kernel, dim3((ncol + 63) / 64, nout), dim3(256), 0, s, p1, t1, p2, t2, nb, zs, ncol,
                     out);
  return hipGetLastError();
}

static hipError_t launch_dlin(const float* dout, const float* lin, const float* lm, const float* den, const float* g,
                              int H, int N, int D, int Z, bool has_lm, float* dnum, uint16_t* dnum16, float* dden,
                              float* rpart,
                              hipStream_t s) {
  hipLaunchKernelGGL(dlin_kernel, dim3(blocks((size_t)Z * N, 4)), dim3(256), 0, s, dout, lin, lm, den, g, H, N, D, Z,
                     has_lm ? 1 : 0, dnum, dnum16, dden, rpart);
  return hipGetLastError();
}
// ---------------------------------------------------------------- host side
// bf16 at D = 64 or 128 with L <= N: the student's landmark branch runs the
// fused query kernel's landmark loop (fp32 output; the store resource covers a
// slice; the workspace holds a pack of up to N landmarks).
static bool lm_fused(const Problem& p, int L) {
  return p.dtype == 1 && (p.D == 64 || p.D == 128) && L >= 1 && L <= p.N &&
         (size_t)query_rows(p) * p.D * 4 < ((size_t)1 << 32);
}

// bf16 with the elu + 1 projection at D = 64 or 128: KV and ksum come from the
// forward's key/value kernel (split partials over the keys, a fixed-order sum).
static bool kv_from_keys(const Problem& p) {
  return p.dtype == 1 && p.proj && p.fmap == kElu1 && (p.D == 64 || p.D == 128) && p.F == 256;
}

BackwardLayout backward_layout(const Problem& p) {
  BackwardLayout l;
  const size_t Z = (size_t)p.B * p.H, N = p.N, NQ = query_rows(p), F = p.F, D = p.D;
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t at = o;
    o += (n * 4 + 255) & ~(size_t)255;
    return at;
  };
  // z_q, z_k: fp32 pre-activations, or on the bf16 path phi(z) in bf16 (every
  // reader takes phi; phi'(z) = min(phi(z), 1))
  const size_t z_el = p.dtype == 1 ? 2 : 4;
  l.zq = take((Z * NQ * F * z_el + 3) / 4);
  l.zk = take((Z * N * F * z_el + 3) / 4);
  // dz_q, dz_k: bf16 on the bf16 path (their only reader, the dW products,
  // stages them as bf16 operands), else fp32
  const size_t dz_el = p.dtype == 1 ? 2 : 4;
  l.dzq = take((Z * NQ * F * dz_el + 3) / 4);
  l.dzk = take((Z * N * F * dz_el + 3) / 4);
  l.lin = take(Z * NQ * D);
  l.lm = take(Z * NQ * D);
  // dnum: bf16 on the bf16 path (its readers, the dz_q and dKV products, stage
  // it as a bf16 operand), else fp32
  l.dnum = take((Z * NQ * D * (p.dtype == 1 ? 2 : 4) + 3) / 4);
  l.kv = take(Z * F * D);
  l.dkv = take(Z * F * D);
  l.ks = take(Z * F);
  l.dks = take(Z * F);
  l.den = take(Z * NQ);
  l.dden = take(Z * NQ);
  l.rpart = take(Z * NQ);
  // half-tile column partials of the GEMM epilogues: ksum then db (query rows), dks, db (key rows)
  const size_t cs = Z * (size_t)half_tiles((int)(N > NQ ? N : NQ)) * F;
  l.cs1 = take(cs);
  l.cs2 = take(cs);
  l.cs3 = take(cs);
  // split-K partials, or (bf16 with the projection) the key/value kernel's split partials and W^T chunks
  size_t sk = splitk_elems(p);
  if (kv_from_keys(p)) sk = std::max(sk, (kv2_reduce_workspace_bytes(p) + 3) / 4);
  // (and the landmark pack of the student's landmark branch; the largest L is N)
  if (lm_fused(p, p.N)) sk = std::max(sk, (lm_pack_bytes(p, p.N) + 3) / 4);
  l.splitk = take(sk);
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
  float *zq, *zk, *dzq, *dzk, *lin, *lm, *dnum, *kv, *dkv, *ks, *dks, *den, *dden, *rpart, *cs1, *cs2, *cs3,
      *splitk;
  size_t splitk_n;
};
static BwBufs bw_bufs(const Problem& p, void* ws) {
  const BackwardLayout l = backward_layout(p);
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  auto F32 = [&](size_t off) { return reinterpret_cast<float*>(w8 + off); };
  return BwBufs{F32(l.zq),  F32(l.zk),  F32(l.dzq),  F32(l.dzk),   F32(l.lin),     F32(l.lm),
                F32(l.dnum), F32(l.kv),  F32(l.dkv),  F32(l.ks),    F32(l.dks),     F32(l.den),
                F32(l.dden), F32(l.rpart), F32(l.cs1), F32(l.cs2), F32(l.cs3),
                F32(l.splitk), splitk_elems(p)};
}

// Forward pass with the intermediates the gradients need: z_q, z_k (biased),
// ks, KV, den, lin = num / den and (L > 0) the landmark output lm.
static hipError_t backward_forward_pass(const Problem& p, const void* Q, const void* K, const void* V, const void* W,
                                        const float* bias, float eps, int L, const BwBufs& t, hipStream_t s,
                                        StageTimer* tm) {
  float *zq = t.zq, *zk = t.zk, *lin = t.lin, *lm = t.lm, *kv = t.kv, *ks = t.ks, *den = t.den;
  const int B = p.B, H = p.H, N = p.N, NQ = query_rows(p), D = p.D, F = p.F, Z = B * H, dt = p.dtype;
  const long long NF = (long long)N * F, ND = (long long)N * D, FD = (long long)F * D;
  const long long QF = (long long)NQ * F, QD = (long long)NQ * D;
  // z_q = Q W + b, z_k = K W + b: per (b, h), [rows x D] . [D x F], the bias in the epilogue
  auto proj = [&](const void* X, float* Zout, int rows, float* phi_part) {
    const long long RD = (long long)rows * D, RF = (long long)rows * F;
    BgemmArgs a{};
    a.A = X;
    a.B = W;
    a.C = Zout;
    a.M = rows;
    a.N = F;
    a.K = D;
    a.KB = 1;
    a.sAz = RD;
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
      ab.A = static_cast<const unsigned char*>(X) + (size_t)b * H * RD * (dt == 1 ? 2 : 4);
      if (dt == 1) {  // bf16: phi(z) in bf16, what every later reader takes
        ab.C16 = reinterpret_cast<uint16_t*>(Zout) + (size_t)b * H * RF;
        ab.phi_out = 1;
      } else {
        ab.C = Zout + (size_t)b * H * RF;
      }
      ab.sBz = (long long)D * F;
      ab.sCz = RF;
      ab.bias_n = bias;  // z = h within one batch row
      ab.sbz = F;
      if (phi_part) ab.cs_phi = phi_part + (size_t)b * H * half_tiles(rows) * F;  // sum of phi(z) per half tile
      TTR_HIP(launch_bgemm(dt, true, true, false, ab, H, s));
    }
    return hipSuccess;
  };
  // bf16: KV = phi(z_k)^T V and ks = sum_n phi(z_k) straight from K and V by the
  // forward's key/value kernel (it forms z_k = K W + b in registers), which
  // reads K and V instead of the fp32 z_k
  const bool kv_direct = kv_from_keys(p);
  TTR_HIP(proj(Q, zq, NQ, nullptr));
  tm->mark();
  TTR_HIP(proj(K, zk, N, kv_direct ? nullptr : t.cs1));
  tm->mark();
  if (kv_direct) {
    TTR_HIP(launch_kv2_reduce(p, K, V, W, bias, kv, ks, t.splitk, s));
    tm->mark();
  } else {
    // ks = sum_n phi(z_k) from the z_k products' half-tile sums; KV = phi(z_k)^T V
    TTR_HIP(launch_tile_colsum(t.cs1, half_tiles(N), nullptr, 0, 1, 0, F, Z, ks, s));
    tm->mark();
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
      TTR_HIP(launch_bgemm(dt, false, true, true, a, Z, s, t.splitk, t.splitk_n));
      tm->mark();
    }
  }
  // lin = phi(z_q) KV / den, den = phi(z_q) . ks + eps
  {
    BgemmArgs a{};
    a.A = zq;
    a.B = kv;
    a.C = lin;
    a.M = NQ;
    a.N = D;
    a.K = F;
    a.KB = 1;
    a.sAz = QF;
    a.sAm = F;
    a.sAk = 1;
    a.sBz = FD;
    a.sBk = D;
    a.sBn = 1;
    a.sCz = QD;
    a.sCm = D;
    a.sCn = 1;
    a.den_ks = ks;  // den = phi(z_q) . ks + eps, and lin = num / den, in the same pass
    a.den_ksz = F;
    a.den_out = den;
    a.den_oz = NQ;
    a.den_eps = eps;
    TTR_HIP(launch_bgemm(dt, dt == 1, false, dt != 1, a, Z, s));  // bf16: A is phi(z_q) in bf16
    tm->mark();
  }
  // landmark branch output (fp32), for dalpha. bf16: a pack of the L landmarks
  // (strided over the N keys) in the split-K scratch, free at this point, and
  // the fused query kernel's landmark loop alone with an fp32 output.
  if (L > 0 && lm_fused(p, L)) {
    FusedPack pk;
    TTR_HIP(launch_lm_pack(p, K, V, L, t.splitk, &pk, s));
    Problem pq = p;
    pq.N = NQ;
    TTR_HIP(launch_softmax_query_f32(pq, Q, pk, L, lm, s));
    tm->mark();
  } else if (L > 0) {
    HybridArgs ha = {};
    ha.Q = Q;
    ha.K = K;
    ha.V = V;
    ha.H = H;
    ha.N = N;
    ha.Nq = NQ;
    ha.L = L;
    ha.out = lm;
    Problem pl = p;
    pl.proj = false;
    pl.F = p.D;
    TTR_HIP(launch_hybrid(pl, M_LM, false, ha, s));
    tm->mark();
  }
  return hipSuccess;
}

// Gradients from dout, after backward_forward_pass filled t (dout NULL: dnum,
// dden and rpart are already in t).
static hipError_t backward_grad_pass(const Problem& p, const void* Q, const void* K, const void* V, const float* g,
                                     int L, const float* dout, float* dW, float* db, float* dg, const BwBufs& t,
                                     hipStream_t s, StageTimer* tm) {
  float *zq = t.zq, *zk = t.zk, *dzq = t.dzq, *dzk = t.dzk, *lin = t.lin, *lm = t.lm, *dnum = t.dnum, *kv = t.kv;
  float *dkv = t.dkv, *ks = t.ks, *dks = t.dks, *den = t.den, *dden = t.dden, *rpart = t.rpart;
  const int B = p.B, H = p.H, N = p.N, NQ = query_rows(p), D = p.D, F = p.F, Z = B * H, dt = p.dtype;
  const long long NF = (long long)N * F, ND = (long long)N * D, FD = (long long)F * D;
  const long long QF = (long long)NQ * F, QD = (long long)NQ * D;
  // dnum, dden, dalpha row shares (one per query row)
  if (dout != nullptr) {  // (NULL: the caller has formed them)
    TTR_HIP(launch_dlin(dout, lin, lm, den, g, H, NQ, D, Z, L > 0, dt == 1 ? nullptr : dnum,
                        dt == 1 ? reinterpret_cast<uint16_t*>(dnum) : nullptr, dden, rpart, s));
    tm->mark();
  }
  // dz_q = (dnum KV^T + dden ks^T) phi'(z_q): [Nq x D] . [D x F], the rest in the epilogue
  {
    BgemmArgs a{};
    a.A = dnum;
    a.B = kv;  // B(k = d, n = f) = KV[f][d]
    if (dt == 1) a.C16 = reinterpret_cast<uint16_t*>(dzq);
    else a.C = dzq;
    if (dt == 1) a.dz_phi = reinterpret_cast<const uint16_t*>(zq);  // phi(z_q), bf16
    else a.dz_x = zq;
    a.dz_r = dden;
    a.dz_s = ks;
    a.dz_srz = NQ;
    a.dz_ssz = F;
    a.cs_val = t.cs1;   // db, query rows
    a.cs_phir = t.cs2;  // dks = sum_n phi(z_q) dden
    a.M = NQ;
    a.N = F;
    a.K = D;
    a.KB = 1;
    a.sAz = QD;
    a.sAm = D;
    a.sAk = 1;
    a.sBz = FD;
    a.sBk = 1;
    a.sBn = D;
    a.sCz = QF;
    a.sCm = F;
    a.sCn = 1;
    TTR_HIP(launch_bgemm(dt, dt == 1, false, false, a, Z, s));  // dnum in the IO dtype
    tm->mark();
  }
  // dKV = phi(z_q)^T dnum: [F x N] . [N x D]; dks = phi(z_q)^T dden
  {
    BgemmArgs a{};
    a.A = zq;
    a.B = dnum;
    a.C = dkv;
    a.M = F;
    a.N = D;
    a.K = NQ;
    a.KB = 1;
    a.sAz = QF;
    a.sAm = 1;
    a.sAk = F;
    a.sBz = QD;
    a.sBk = D;
    a.sBn = 1;
    a.sCz = FD;
    a.sCm = D;
    a.sCn = 1;
    // dnum in the IO dtype; bf16: A is phi(z_q) in bf16 already
    TTR_HIP(launch_bgemm(dt, dt == 1, dt == 1, dt != 1, a, Z, s, t.splitk, t.splitk_n));
    tm->mark();
  }
  TTR_HIP(launch_tile_colsum(t.cs2, half_tiles(NQ), nullptr, 0, 1, 0, F, Z, dks, s));
  tm->mark();
  // dz_k = (V dKV^T + 1 dks^T) phi'(z_k): [N x D] . [D x F], the rest in the epilogue
  {
    BgemmArgs a{};
    a.A = V;
    a.B = dkv;  // B(k = d, n = f) = dKV[f][d]
    if (dt == 1) a.C16 = reinterpret_cast<uint16_t*>(dzk);
    else a.C = dzk;
    if (dt == 1) a.dz_phi = reinterpret_cast<const uint16_t*>(zk);  // phi(z_k), bf16
    else a.dz_x = zk;
    a.dz_s = dks;
    a.dz_ssz = F;
    a.cs_val = t.cs3;  // db, key rows
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
    tm->mark();
  }
  // dW[h] = sum_b Q[b,h]^T dz_q[b,h] + K[b,h]^T dz_k[b,h]: the batch is the outer K loop
  auto dw = [&](const void* X, const void* dzv, int rows, int beta) {  // dz in the IO dtype
    const long long RD = (long long)rows * D, RF = (long long)rows * F;
    BgemmArgs a{};
    a.A = X;  // A(m = d, k = n) = X[n][d]
    a.B = dzv;
    a.C = dW;
    a.M = D;
    a.N = F;
    a.K = rows;
    a.KB = B;
    a.sAz = RD;
    a.sAkb = (long long)H * RD;
    a.sAm = 1;
    a.sAk = D;
    a.sBz = RF;
    a.sBkb = (long long)H * RF;
    a.sBk = F;
    a.sBn = 1;
    a.sCz = (long long)D * F;
    a.sCm = F;
    a.sCn = 1;
    a.beta = beta;
    return launch_bgemm(dt, true, dt == 1, false, a, H, s, t.splitk, t.splitk_n);
  };
  TTR_HIP(dw(Q, dzq, NQ, 0));
  tm->mark();
  TTR_HIP(dw(K, dzk, N, 1));
  tm->mark();
  // db[h] over rows (b, n) of slice h; dg[h] from the row shares of dalpha
  TTR_HIP(launch_tile_colsum(t.cs1, half_tiles(NQ), t.cs3, half_tiles(N), B, H, F, H, db, s));
  hipLaunchKernelGGL(dg_kernel, dim3(H), dim3(256), 0, s, rpart, g, B, H, NQ, L > 0 ? 1 : 0, dg);
  TTR_HIP(hipGetLastError());
  tm->mark();
  return hipSuccess;
}

hipError_t launch_hybrid_backward(const Problem& p, const void* Q, const void* K, const void* V, const void* W,
                                  const float* bias, const float* g, float eps, int L, const float* dout, float* dW,
                                  float* db, float* dg, void* ws, hipStream_t s, StageTimer* tm) {
  const BwBufs t = bw_bufs(p, ws);
  TTR_HIP(backward_forward_pass(p, Q, K, V, W, bias, eps, L, t, s, tm));
  return backward_grad_pass(p, Q, K, V, g, L, dout, dW, db, dg, t, s, tm);
}

// ---------------------------------------------------------------- distillation step
// Per row (z, n), D / 4 lanes: o = alpha lin + (1 - alpha) lm (lin alone when L == 0),
// t = the teacher row; dout = w1 clip(o - t, -1, 1) / numel - w2 dcos / rows (the
// loss's gradient with respect to o, kept in registers), the row's huber sum
// and 1 - cos; then the linear branch's row gradients from dout: dlin = alpha
// dout, dnum = dlin / den, dden = -sum_d dlin lin / den, and the row's share of
// dalpha, sum_d dout (lin - lm). w = exp(-s).
template <int D, bool DN16>
__global__ __launch_bounds__(256) void distill_loss_dlin_kernel(const float* lin, const float* lm, const float* teacher,
                                                                const uint16_t* teacher_bf16, const float* g,
                                                                const float* sv, const float* den_row, int H, int N,
                                                                int Z, int has_lm, float* hrow, float* crow_,
                                                                float* dnum, float* dden, float* rpart) {
  // A row is LPR lanes of 4 consecutive elements (16-byte loads and stores);
  // a wave holds 64 / LPR rows, and the row sums stay within a row's lanes.
  constexpr int LPR = D / 4, RPW = 64 / LPR;
  static_assert(D % 4 == 0 && 64 % LPR == 0, "row layout");
  const int lane = threadIdx.x & 63, l4 = lane % LPR;
  const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int rows = Z * N;
  const bool ok = row0 < rows;
  const int row = ok ? row0 : rows - 1;  // (every lane takes part in the shuffles)
  const int h = (row / N) % H;
  const float alpha = has_lm ? 1.f / (1.f + expf(-g[h])) : 1.f;
  const float w1 = expf(-sv[0]), w2 = expf(-sv[1]);
  const float inv_numel = 1.f / ((float)rows * D), inv_rows = 1.f / (float)rows;
  const size_t at = (size_t)row * D + 4 * l4;
  const f32x4 lv = *reinterpret_cast<const f32x4*>(lin + at);
  const f32x4 mv = has_lm ? *reinterpret_cast<const f32x4*>(lm + at) : f32x4{};
  f32x4 tv;
  if (teacher_bf16) {
    const uint2 b = *reinterpret_cast<const uint2*>(teacher_bf16 + at);
    tv[0] = __uint_as_float(b.x << 16);
    tv[1] = __uint_as_float(b.x & 0xffff0000u);
    tv[2] = __uint_as_float(b.y << 16);
    tv[3] = __uint_as_float(b.y & 0xffff0000u);
  } else {
    tv = *reinterpret_cast<const f32x4*>(teacher + at);
  }
  float ov[4];
  float hs = 0.f, dot = 0.f, oo = 0.f, tt = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float o = has_lm ? alpha * lv[e] + (1.f - alpha) * mv[e] : lv[e];
    const float r = o - tv[e], ar = fabsf(r);
    hs += ar <= 1.f ? 0.5f * r * r : ar - 0.5f;
    ov[e] = o;
    dot += o * tv[e];
    oo += o * o;
    tt += tv[e] * tv[e];
  }
  for (int off = LPR / 2; off > 0; off >>= 1) {
    hs += __shfl_xor(hs, off);
    dot += __shfl_xor(dot, off);
    oo += __shfl_xor(oo, off);
    tt += __shfl_xor(tt, off);
  }
  const float no = sqrtf(oo), nt = sqrtf(tt);
  const float cden = fmaxf(no * nt, 1e-8f);
  const float cosv = dot / cden;
  const bool live = no * nt > 1e-8f;
  const float co = live ? dot * nt / (no * cden * cden) : 0.f;
  const float inv = 1.f / den_row[row];
  float sd = 0.f, sa = 0.f;
  f32x4 dn;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float r = ov[e] - tv[e];
    const float dcos = tv[e] / cden - co * ov[e];
    const float G = w1 * fminf(fmaxf(r, -1.f), 1.f) * inv_numel - w2 * dcos * inv_rows;
    const float dl = alpha * G;
    dn[e] = dl * inv;
    sd += dl * lv[e];
    if (has_lm) sa += G * (lv[e] - mv[e]);
  }
  if (ok) {
    if constexpr (DN16) {  // the bf16 path keeps dnum in bf16
      uint2 b;
      b.x = pack_bf16x2(dn[0], dn[1]);
      b.y = pack_bf16x2(dn[2], dn[3]);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(dnum) + at) = b;
    } else {
      *reinterpret_cast<f32x4*>(dnum + at) = dn;
    }
  }
  for (int off = LPR / 2; off > 0; off >>= 1) {
    sd += __shfl_xor(sd, off);
    sa += __shfl_xor(sa, off);
  }
  if (ok && l4 == 0) {
    hrow[row] = hs;
    crow_[row] = 1.f - cosv;
    dden[row] = -sd * inv;
    rpart[row] = sa;
  }
}

// Loss totals in two fixed-order levels: workgroup k sums rows
// [k * kLossRows, (k + 1) * kLossRows) into part[2k], part[2k + 1]; one
// workgroup then adds the parts in order and forms
// loss = w1 H + s1 + w2 C + s2, H = sum hrow / numel, C = sum crow / rows,
// ds = (1 - w1 H, 1 - w2 C). out: loss, H, C.
constexpr int kLossRows = 4096;
__global__ void distill_loss_part_kernel(const float* hrow, const float* crow_, int rows, float* part) {
  __shared__ float sh[256], sc[256];
  const int t = threadIdx.x, r0 = blockIdx.x * kLossRows, r1 = min(rows, r0 + kLossRows);
  float h = 0.f, c = 0.f;
  for (int i = r0 + t; i < r1; i += 256) {
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
    part[2 * blockIdx.x] = sh[0];
    part[2 * blockIdx.x + 1] = sc[0];
  }
}
__global__ void distill_loss_total_kernel(const float* part, int nparts, int rows, int D, const float* sv,
                                          float* loss_out, float* ds) {
  if (threadIdx.x != 0) return;
  float hs = 0.f, cs = 0.f;
  for (int k = 0; k < nparts; ++k) {
    hs += part[2 * k];
    cs += part[2 * k + 1];
  }
  const float H = hs / ((float)rows * D), C = cs / (float)rows;
  const float w1 = expf(-sv[0]), w2 = expf(-sv[1]);
  loss_out[0] = w1 * H + sv[0] + w2 * C + sv[1];
  loss_out[1] = H;
  loss_out[2] = C;
  ds[0] = 1.f - w1 * H;
  ds[1] = 1.f - w2 * C;
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
  const size_t Z = (size_t)p.B * p.H, N = query_rows(p), D = p.D, F = p.F, H = p.H;  // N: query rows here
  auto al = [](size_t n) { return (n + 255) & ~(size_t)255; };
  size_t o = al(backward_layout(p).bytes);
  l.w_io = o;
  o += al(p.dtype == 1 ? H * D * F * 2 : 0);
  l.teacher = o;  // fp32 teacher (fp32 IO), or bf16 teacher and its landmark pack (bf16 IO)
  if (need_teacher) {
    if (p.dtype == 1) {
      l.tws = o + al(Z * N * D * 2);
      o = l.tws + al(lm_pack_bytes(p, p.N));
    } else {
      o += al(Z * N * D * 4);
    }
  }
  l.hrow = o;
  o += al(Z * N * 4);
  l.crow = o;
  o += al(Z * N * 4);
  l.grads = o;  // dW | db | dg | ds
  o += al((H * D * F + H * F + H + 2) * 4);
  l.lpart = o;
  o += al(2 * ((Z * N + kLossRows - 1) / kLossRows) * 4);
  l.bytes = o;
  return l;
}

hipError_t launch_distill_step(const Problem& p, const void* Q, const void* K, const void* V, const float* teacher,
                               float* W, float* bias, float* g, float* sv, float* moments, int step, float lr,
                               float eps, int L, float* loss_out, void* ws, hipStream_t s, StageTimer* tm) {
  const DistillLayout l = distill_layout(p, teacher == nullptr);
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  const int B = p.B, H = p.H, N = p.N, NQ = query_rows(p), D = p.D, F = p.F, Z = B * H;
  const size_t nW = (size_t)H * D * F, nb = (size_t)H * F;
  // weights in the IO dtype for the forward and backward
  const void* Wio = W;
  if (p.dtype == 1) {
    uint16_t* wb = reinterpret_cast<uint16_t*>(w8 + l.w_io);
    hipLaunchKernelGGL(to_bf16_kernel, dim3(blocks(nW, 256)), dim3(256), 0, s, W, wb, nW);
    TTR_HIP(hipGetLastError());
    tm->mark();
    Wio = wb;
  }
  // Teacher: softmax over every token. bf16: the fused query kernel without its
  // linear branch over a pack in which every key is a landmark, output in
  // bf16; fp32: the landmark branch with L = N.
  const float* T = teacher;
  const uint16_t* Tb = nullptr;
  if (teacher == nullptr) {
    if (p.dtype == 1) {
      uint16_t* tb = reinterpret_cast<uint16_t*>(w8 + l.teacher);
      FusedPack pk;
      TTR_HIP(launch_lm_pack(p, K, V, N, w8 + l.tws, &pk, s));  // every one of the N keys
      Problem pq = p;  // the query kernel tiles the query rows
      pq.N = NQ;
      TTR_HIP(launch_softmax_query(pq, Q, pk, N, tb, s));
      Tb = tb;
    } else {
      float* tw = reinterpret_cast<float*>(w8 + l.teacher);
      HybridArgs ha = {};
      ha.Q = Q;
      ha.K = K;
      ha.V = V;
      ha.H = H;
      ha.N = N;
      ha.Nq = NQ;
      ha.L = N;
      ha.out = tw;
      Problem pl = p;
      pl.proj = false;
      pl.F = p.D;
      TTR_HIP(launch_hybrid(pl, M_LM, false, ha, s));
      T = tw;
    }
    tm->mark();
  }
  const BwBufs t = bw_bufs(p, ws);
  TTR_HIP(backward_forward_pass(p, Q, K, V, Wio, bias, eps, L, t, s, tm));
  float* hrow = reinterpret_cast<float*>(w8 + l.hrow);
  float* crw = reinterpret_cast<float*>(w8 + l.crow);
  float* gr = reinterpret_cast<float*>(w8 + l.grads);
  float *dW = gr, *db = gr + nW, *dg = db + nb, *ds = dg + H;
  {
    const size_t waves = ((size_t)Z * NQ + (256 / D) - 1) / (256 / D);  // 256 / D rows per wave
    // (dnum in the IO dtype: bf16 on the bf16 path)
    auto launch = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(blocks(waves, 4)), dim3(256), 0, s, t.lin, t.lm, T, Tb, g, sv, t.den, H, NQ, Z,
                         L > 0 ? 1 : 0, hrow, crw, t.dnum, t.dden, t.rpart);
    };
    const bool b16 = p.dtype == 1;
    if (D == 128) b16 ? launch(distill_loss_dlin_kernel<128, true>) : launch(distill_loss_dlin_kernel<128, false>);
    else if (D == 64) b16 ? launch(distill_loss_dlin_kernel<64, true>) : launch(distill_loss_dlin_kernel<64, false>);
    else return hipErrorInvalidValue;
  }
  TTR_HIP(hipGetLastError());
  tm->mark();
  float* lpart = reinterpret_cast<float*>(w8 + l.lpart);
  const int nparts = (Z * NQ + kLossRows - 1) / kLossRows;
  hipLaunchKernelGGL(distill_loss_part_kernel, dim3(nparts), dim3(256), 0, s, hrow, crw, Z * NQ, lpart);
  TTR_HIP(hipGetLastError());
  hipLaunchKernelGGL(distill_loss_total_kernel, dim3(1), dim3(64), 0, s, lpart, nparts, Z * NQ, D, sv, loss_out, ds);
  TTR_HIP(hipGetLastError());
  tm->mark();
  TTR_HIP(backward_grad_pass(p, Q, K, V, g, L, nullptr, dW, db, dg, t, s, tm));  // dnum, dden, rpart are in place
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
  TTR_HIP(hipGetLastError());
  tm->mark();
  return hipSuccess;
}

}  // namespace ttr

// Query-side kernel of the TTR forward: one templated kernel computes, for a
// 128-token tile of one (batch, head),
//   M_PHI  phi(Q) = elu(Q W_h + b_h) + 1                      (ttr_feature_map)
//   M_LIN  out_lin = phi(Q) KV / (phi(Q) . ksum + eps)        (ttr_apply)
//   M_LM   out_lm = softmax(Q K_L^T / sqrt(D)) V_L            (ttr_landmark_attn)
//   M_LIN|M_LM  out = sigmoid(g_h) out_lin + (1 - sigmoid(g_h)) out_lm
// Method: "Flux2TTRTrainer", section "How the distillation works" (kernel
// branch + landmark exact-softmax branch + bounded blend);
// "NNT Define Linear Attention", sections "The inputs" (elu + 1, eps) and
// "How it works" (Q'(K'^T V) with the 1 / (Q' . sum(K') + eps) normaliser).
//
// Each of the 4 waves owns 32 query tokens. Every product runs on MFMA in
// "transposed" form so that a C tile (lane = token, registers = feature) can
// be fed straight back as the B operand of the next product:
//   phi^T [F x tok]  = W^T [F x D]   . Q^T [D x tok]       (A from LDS, B in registers)
//   num^T [D x tok] += KV^T [D x F]  . phi^T [F x tok]     (A from LDS, B = previous C)
//   S^T  [L x tok]   = K_L [L x D]   . Q^T                 (A from LDS)
//   out^T[D x tok]  += V_L^T [D x L] . P^T [L x tok]       (online softmax over L)
// The normaliser phi(Q) . ksum and the softmax statistics are per-lane fp32
// sums finished with one cross-half lane exchange.
#include "common.hpp"
#include "launch.hpp"

namespace ttr {

template <typename T, int D, int F, int MODE>
struct HybridSmem {
  // Features staged at a time: all F when W^T and KV^T fit in LDS together,
  // else blocks of 64 (fp32 with D = 128: 128 KB each in full)
  static constexpr int full_bytes = F * LdsRow<T, D>::bytes_per_row +
                                    ((MODE & M_LIN) ? D * LdsRow<T, F>::bytes_per_row : 0) + 2 * F * 4;
  static constexpr int FB = full_bytes <= 160 * 1024 ? F : 64;
  static_assert(F % FB == 0, "whole feature blocks");
  using WR = LdsRow<T, D>;   // W^T   [FB][D]
  using KR = LdsRow<T, FB>;  // KV^T  [D][FB]  (columns in kperm order)
  static constexpr int LB = 64;  // landmarks per LDS block
  using LR = LdsRow<T, D>;   // K_L   [LB][D]
  using VR = LdsRow<T, LB>;  // V_L^T [D][LB] (columns in kperm order)
  static constexpr int w_bytes = FB * WR::bytes_per_row;
  static constexpr int kv_bytes = (MODE & M_LIN) ? D * KR::bytes_per_row : 0;
  static constexpr int lin_bytes = (MODE & (M_PHI | M_LIN)) ? w_bytes + kv_bytes + 2 * F * 4 : 0;
  static constexpr int lm_bytes = (MODE & M_LM) ? LB * LR::bytes_per_row + D * VR::bytes_per_row : 0;
  static constexpr int bytes = lin_bytes > lm_bytes ? lin_bytes : lm_bytes;
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int landmark_index(int j, int N, int L) {
  return (int)(((long long)j * (long long)N) / (long long)L);
}

// Stage rows f0 .. f0 + FB - 1 of W^T (or of the identity when there is no
// projection) into LDS; W is [D][F].
template <typename T, int D, int F, int FB, bool PROJ>
__device__ __forceinline__ void stage_wt(T* Wt, const T* W, int f0, int tid) {
  using WR = LdsRow<T, D>;
  if constexpr (PROJ) {
    // consecutive threads take consecutive d pairs: conflict-free LDS writes
    for (int u = tid; u < (D / 2) * (FB / 8); u += 256) {
      const int d = 2 * (u % (D / 2));
      const int fo = (u / (D / 2)) * 8;
      const Vec8<T> w0 = ld8(W + (size_t)d * F + f0 + fo);
      const Vec8<T> w1 = ld8(W + (size_t)(d + 1) * F + f0 + fo);
#pragma unroll
      for (int j = 0; j < 8; ++j) st_pair(Wt + (fo + j) * WR::stride + d, w0.v[j], w1.v[j]);
    }
  } else {
    for (int u = tid; u < FB * D; u += 256) {
      const int f = u / D, d = u % D;
      Wt[f * WR::stride + d] = from_f32<T>(f0 + f == d ? 1.f : 0.f);
    }
  }
}

template <typename T, int D, int F, bool PROJ, int MODE, typename OutT, int MAP>
__global__ __launch_bounds__(256, 1) void hybrid_kernel(HybridArgs a) {
  using S = HybridSmem<T, D, F, MODE>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::bytes];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int bh = blockIdx.y, h = bh % a.H;
  const int N = a.N, NQ = a.Nq > 0 ? a.Nq : a.N;  // keys, query rows
  const int tok = blockIdx.x * 128 + 32 * w + c;
  const bool tok_ok = tok < NQ;
  const T* Q = static_cast<const T*>(a.Q) + (size_t)bh * NQ * D;

  // Q^T as B operand: lane = token, k-slots = 8 consecutive features of Q.
  Frag<T> qf[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb)
    qf[kb] = tok_ok ? ld_frag<T>(Q + (size_t)tok * D + kb * 16 + 8 * g) : zero_frag<T>();

  // Per-lane results: row d = db*32 + crow(lane, r) of the output column `tok`.
  float res[D / 32][16];

  if constexpr ((MODE & (M_PHI | M_LIN)) != 0) {
    using WR = typename S::WR;
    using KR = typename S::KR;
    T* Wt = reinterpret_cast<T*>(smem);
    T* KVt = reinterpret_cast<T*>(smem + S::w_bytes);
    float* biasP = reinterpret_cast<float*>(smem + S::w_bytes + S::kv_bytes);
    float* ksumP = biasP + F;

    constexpr int FB = S::FB;
    // W^T rows and KV^T columns of features f0 .. f0 + FB - 1 (kperm order
    // within each aligned 16: the same in the block as in the whole)
    auto stage_block = [&](int f0) {
      stage_wt<T, D, F, FB, PROJ>(Wt, static_cast<const T*>(a.W) + (size_t)h * D * F, f0, tid);
      if constexpr ((MODE & M_LIN) != 0) {
        const float* KV = a.KV + (size_t)bh * F * D;
        for (int u = tid; u < (FB / 2) * (D / 4); u += 256) {
          const int f = 2 * (u % (FB / 2));
          const int d0 = (u / (FB / 2)) * 4;
          const f32x4 k0 = *reinterpret_cast<const f32x4*>(KV + (size_t)(f0 + f) * D + d0);
          const f32x4 k1 = *reinterpret_cast<const f32x4*>(KV + (size_t)(f0 + f + 1) * D + d0);
          const int pos = kperm(f);  // f even: kperm(f + 1) == pos + 1
#pragma unroll
          for (int j = 0; j < 4; ++j)
            st_pair(KVt + (d0 + j) * KR::stride + pos, from_f32<T>(k0[j]), from_f32<T>(k1[j]));
        }
      }
    };
    stage_block(0);
    for (int f = tid; f < F; f += 256) biasP[kperm(f)] = a.bias ? a.bias[(size_t)h * F + f] : 0.f;
    if constexpr ((MODE & M_LIN) != 0)
      for (int f = tid; f < F; f += 256) ksumP[kperm(f)] = a.ksum[(size_t)bh * F + f];
    __syncthreads();

    // softmax map (identity projection, F == D): the token's feature maximum
    // and inverse sum, from its Q row (half in this lane, half in lane ^ 32)
    float qm = 0.f, qinv = 1.f;
    if constexpr (MAP == kSoftmax) {
      static_assert(!PROJ, "the softmax map takes already projected features");
      float z[D / 2];
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        frag_to_f32(qf[kb], z + 8 * kb);
#pragma unroll
        for (int j = 0; j < 8; ++j) z[8 * kb + j] += biasP[kperm(kb * 16 + 8 * g + j)];
      }
      softmax_stats<D / 2, 32>(z, qm, qinv);
    }

    f32x16 num[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) num[db] = f32x16{};
    float den = 0.f;

    for (int fc = 0; fc < F / 32; ++fc) {
      if (FB < F && fc > 0 && fc % (FB / 32) == 0) {  // next feature block (workgroup-uniform)
        __syncthreads();
        stage_block(fc * 32);
        __syncthreads();
      }
      const int fl = fc % (FB / 32);  // chunk within the staged block
      // phi^T chunk [32 features x 32 tokens]; the bias is preloaded into the accumulator.
      f32x16 acc;
      {
        const float* bp = biasP + fc * 32 + 8 * g;
#pragma unroll
        for (int r = 0; r < 8; ++r) { acc[r] = bp[r]; acc[8 + r] = bp[16 + r]; }
      }
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb)
        mma(acc, ld_frag<T>(Wt + (fl * 32 + c) * WR::stride + kb * 16 + 8 * g), qf[kb]);
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = phi_of<MAP>(acc[r], qm, qinv);

      if constexpr ((MODE & M_PHI) != 0) {
        if (tok_ok) {
          OutT* o = static_cast<OutT*>(a.out) + ((size_t)bh * NQ + tok) * F + fc * 32 + 4 * g;
#pragma unroll
          for (int q = 0; q < 4; ++q) st4(o + 8 * q, p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]);
        }
      }
      if constexpr ((MODE & M_LIN) != 0) {
        const float* kp = ksumP + fc * 32 + 8 * g;
#pragma unroll
        for (int r = 0; r < 8; ++r) den += p[r] * kp[r] + p[8 + r] * kp[16 + r];
        const Frag<T> pb0 = to_frag<T>(p), pb1 = to_frag<T>(p + 8);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const T* ap = KVt + (db * 32 + c) * KR::stride + fl * 32 + 8 * g;
          mma(num[db], ld_frag<T>(ap), pb0);
          mma(num[db], ld_frag<T>(ap + 16), pb1);
        }
      }
    }
    if constexpr ((MODE & M_LIN) != 0) {
      den += shfl_xor32(den);
      const float inv = 1.f / (den + a.eps);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) res[db][r] = num[db][r] * inv;
    }
  }

  if constexpr ((MODE & M_LM) != 0) {
    constexpr int LB = S::LB;
    using LR = typename S::LR;
    using VR = typename S::VR;
    T* KL = reinterpret_cast<T*>(smem);
    T* VLt = reinterpret_cast<T*>(smem + LB * LR::bytes_per_row);
    const T* K = static_cast<const T*>(a.K) + (size_t)bh * N * D;
    const T* V = static_cast<const T*>(a.V) + (size_t)bh * N * D;
    const int L = a.L;
    // scores in base 2: exp(s / sqrt(D)) = 2^(s log2(e) / sqrt(D))
    const float sl2 = kLog2e * rsqrtf((float)D);

    float m = -INFINITY, l = 0.f;
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};

    for (int j0 = 0; j0 < L; j0 += LB) {
      __syncthreads();  // previous users of this LDS region are done
      for (int u = tid; u < LB * (D / 8); u += 256) {
        const int jl = u / (D / 8), d0 = (u % (D / 8)) * 8, j = j0 + jl;
        const Vec8<T> v = j < L ? ld8(K + (size_t)landmark_index(j, N, L) * D + d0) : zero8<T>();
        st8(KL + jl * LR::stride + d0, v);
      }
      for (int u = tid; u < (LB / 2) * (D / 8); u += 256) {
        const int jl = 2 * (u % (LB / 2)), d0 = (u / (LB / 2)) * 8, j = j0 + jl;
        const Vec8<T> v0 = j < L ? ld8(V + (size_t)landmark_index(j, N, L) * D + d0) : zero8<T>();
        const Vec8<T> v1 = j + 1 < L ? ld8(V + (size_t)landmark_index(j + 1, N, L) * D + d0) : zero8<T>();
        const int pos = kperm(jl);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) st_pair(VLt + (d0 + jj) * VR::stride + pos, v0.v[jj], v1.v[jj]);
      }
      __syncthreads();

      for (int jc = 0; jc < LB / 32; ++jc) {
        if (j0 + jc * 32 >= L) break;  // uniform across the workgroup
        f32x16 s = f32x16{};
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb)
          mma(s, ld_frag<T>(KL + (jc * 32 + c) * LR::stride + kb * 16 + 8 * g), qf[kb]);
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool valid = j0 + jc * 32 + crow(lane, r) < L;
          const float v = valid ? s[r] * sl2 : -INFINITY;
          s[r] = v;
          mx = fmaxf(mx, v);
        }
        mx = fmaxf(mx, shfl_xor32(mx));
        const float mn = fmaxf(m, mx);  // finite: every visited chunk holds a valid landmark
        const float corr = fast_exp2(m - mn);
        float p[16], ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) { p[r] = fast_exp2(s[r] - mn); ls += p[r]; }
        ls += shfl_xor32(ls);
        l = l * corr + ls;
        m = mn;
        const Frag<T> pb0 = to_frag<T>(p), pb1 = to_frag<T>(p + 8);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= corr;
          const T* ap = VLt + (db * 32 + c) * VR::stride + jc * 32 + 8 * g;
          mma(o[db], ld_frag<T>(ap), pb0);
          mma(o[db], ld_frag<T>(ap + 16), pb1);
        }
      }
    }
    const float invl = 1.f / l;
    if constexpr ((MODE & M_LIN) != 0) {
      const float gh = a.g[h];
      const float alpha = 1.f / (1.f + expf(-gh));  // g = +inf -> 1, g = -inf -> 0
      const float beta = 1.f - alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) res[db][r] = alpha * res[db][r] + beta * (o[db][r] * invl);
    } else {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) res[db][r] = o[db][r] * invl;
    }
  }

  if constexpr (MODE != M_PHI) {
    if (tok_ok) {
      OutT* o = static_cast<OutT*>(a.out) + ((size_t)bh * NQ + tok) * D + 4 * g;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          st4(o + db * 32 + 8 * q, res[db][4 * q], res[db][4 * q + 1], res[db][4 * q + 2], res[db][4 * q + 3]);
    }
  }
}

template <typename T, int D, bool PROJ, int MAP>
static hipError_t launch_hybrid_t(int mode, bool out_io, const HybridArgs& a, int B, hipStream_t s) {
  constexpr int F = PROJ ? 256 : D;
  const dim3 grid(((a.Nq > 0 ? a.Nq : a.N) + 127) / 128, B * a.H), block(256);
  switch (mode) {
    case M_PHI:
      hipLaunchKernelGGL((hybrid_kernel<T, D, F, PROJ, M_PHI, T, MAP>), grid, block, 0, s, a);
      break;
    case M_LIN:
      if (out_io)
        hipLaunchKernelGGL((hybrid_kernel<T, D, F, PROJ, M_LIN, T, MAP>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((hybrid_kernel<T, D, F, PROJ, M_LIN, float, MAP>), grid, block, 0, s, a);
      break;
    case M_LM:
      if constexpr (MAP != kElu1) return hipErrorInvalidValue;  // the landmark branch has no feature map
      hipLaunchKernelGGL((hybrid_kernel<T, D, D, false, M_LM, float, kElu1>), grid, block, 0, s, a);
      break;
    case M_LIN | M_LM:
      if constexpr (MAP != kElu1) return hipErrorInvalidValue;  // landmarks belong to the elu+1 layer
      hipLaunchKernelGGL((hybrid_kernel<T, D, F, PROJ, M_LIN | M_LM, T, kElu1>), grid, block, 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_hybrid_d(const Problem& p, int mode, bool out_io, const HybridArgs& a, hipStream_t s) {
  if (p.proj || mode == M_LM) return launch_hybrid_t<T, D, true, kElu1>(mode, out_io, a, p.B, s);
  if (p.fmap == kRelu) return launch_hybrid_t<T, D, false, kRelu>(mode, out_io, a, p.B, s);
  if (p.fmap == kSoftmax) return launch_hybrid_t<T, D, false, kSoftmax>(mode, out_io, a, p.B, s);
  return launch_hybrid_t<T, D, false, kElu1>(mode, out_io, a, p.B, s);
}

hipError_t launch_hybrid(const Problem& p, int mode, bool out_io, const HybridArgs& a, hipStream_t s) {
  if (p.dtype == 1) {
    if (p.D == 64) return launch_hybrid_d<uint16_t, 64>(p, mode, out_io, a, s);
    if (p.D == 128) return launch_hybrid_d<uint16_t, 128>(p, mode, out_io, a, s);
  } else if (p.dtype == 0) {
    if (p.D == 64) return launch_hybrid_d<float, 64>(p, mode, out_io, a, s);
    if (p.D == 128) return launch_hybrid_d<float, 128>(p, mode, out_io, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ttr

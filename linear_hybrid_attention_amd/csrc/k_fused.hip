// bf16 hot path, stage 2: apply + landmark softmax + blend over Q in one pass.
//   out = alpha_h . phi(Q) KV / (phi(Q) . ksum + eps)
//       + (1 - alpha_h) . softmax(Q K_L^T / sqrt(D)) V_L,      alpha_h = sigmoid(g_h)
// ("Flux2TTRTrainer", section "How the distillation works": linear kernel
// branch + exact softmax over landmark tokens + bounded blend; "NNT Define
// Linear Attention", sections "The inputs" and "How it works".)
//
// Workgroup: 4 waves x 32 query tokens, two workgroups per compute unit (two
// waves per SIMD). The per-head operands come from the pack written by the
// key/value stage as a sequence of equal-size chunks (W^T, KV^T alternately
// per 64 features, then one K_L + V_L^T chunk per 32 landmarks), copied
// global -> LDS asynchronously into a ring of four slots, one step ahead.
// Q stays in registers as the B operand of every product, and every LDS
// operand read is a plain 16-byte row read:
//   W^T chunk:   phi^T [64 f x tok]  = W^T . Q^T (+ bias, then the map; phi . ksum)
//   KV^T chunk:  num^T [D x tok]    += KV^T . phi^T
//   landmark chunk (32 landmarks: K_L then V_L^T):
//                S^T  [32 j x tok]   = K_L . Q^T  (scaled to base 2, online max)
//                o^T  [D x tok]     += V_L^T . P^T
// Both branches are software-pipelined so that each step issues two
// independent MFMA products and overlaps the elementwise work (feature map,
// softmax) of one with the execution of the other.
// The online softmax keeps a running row max m and only rescales o and the
// row sum when a new score exceeds m by more than 8 (base 2), so the exp
// arguments stay below 2^8 and most chunks skip the rescale.
// Workgroups are numbered so that consecutive tiles of one (batch, head) run
// on one XCD and share its L2 copy of the pack.
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace ttr {

struct FusedArgs {
  const uint16_t* Q;
  const unsigned char* pack_bh;
  const unsigned char* pack_w;
  unsigned long long bh_bytes, w_bytes;
  const float* g;
  float eps;
  int H, N, L, ntiles, nwg;
  uint16_t* out;
  float* out32;  // OUT32: the output in fp32 instead
};

// LIN = false: softmax attention over the landmarks alone, out = o / l (the
// pack then holds only the landmark chunks; no linear branch, no blend).
// OUT32: the output in fp32 (out32).
// The map of the linear branch on a product that already holds the pack's
// bias: for elu + 1 the pack stores b + 1, so x = z + b + 1 and
// elu(z + b) + 1 = max(x, min(exp(x - 1), 1)) (an fma, the exponential with
// its clamp, a max); relu and softmax take x = z + b.
template <int MAP>
__device__ __forceinline__ float phi_q(float x, float m, float inv_s) {
  if constexpr (MAP == kElu1) return fmaxf(x, fminf(fmaxf(__builtin_amdgcn_exp2f(fmaf(x, kLog2e, -kLog2e)), 0.f), 1.f));
  else return phi_of<MAP>(x, m, inv_s);
}

template <int D, int F, int MAP, bool LIN = true, bool OUT32 = false>
__global__ __launch_bounds__(256, 2) void fused_query_kernel(FusedArgs a) {
  constexpr int CH = 64 * D;  // elements per chunk (every chunk kind)
  constexpr int NFC = F / 64;
  constexpr int PER_T = CH * 2 / 16 / 256;  // 16-byte copies per thread per chunk
  static_assert(PER_T * 256 * 16 == CH * 2, "whole pieces");
  constexpr int NSLOT = 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * F * 4 + NSLOT * CH * 2];
  float* vecS = reinterpret_cast<float*>(smem);  // biasP [F] | ksumP [F]
  uint16_t* const slots = reinterpret_cast<uint16_t*>(smem + 2 * F * 4);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, c = lane & 31;

  // XCD-aware numbering: hardware places workgroup i on XCD i % 8.
  int wg = blockIdx.x;
  const int per = a.nwg / 8;
  if (wg < per * 8) wg = (wg % 8) * per + wg / 8;
  const int bh = wg / a.ntiles, tile = wg % a.ntiles, h = bh % a.H;
  const int N = a.N, L = a.L;
  const int tok = tile * 128 + 32 * w + c;
  const bool tok_ok = tok < N;

  const unsigned char* pbh = a.pack_bh + (size_t)bh * a.bh_bytes;
  const uint16_t* wpk = reinterpret_cast<const uint16_t*>(a.pack_w + (size_t)h * a.w_bytes);
  constexpr int VEC = LIN ? 2 * F * 4 : 0;  // bias and ksum ahead of the chunks
  constexpr int LB = LIN ? 2 * NFC : 0;     // index of the first landmark chunk
  const uint16_t* kvpk = reinterpret_cast<const uint16_t*>(pbh + VEC);
  const int nlc = (L + 31) / 32;  // landmark chunks
  const int nch = LB + nlc;

  // Chunk ci is copied global -> LDS slot ci % 4 asynchronously at the start
  // of the step before the one that first reads it; every step ends by
  // waiting for its copies and a barrier. A step reads at most two chunks
  // (consecutive), so the two it reads and the two in flight never share a slot.
  const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(wpk, (uint32_t)a.w_bytes);                     // W^T chunks
  const __amdgpu_buffer_rsrc_t rkv = buffer_rsrc(kvpk, (uint32_t)(a.bh_bytes - VEC));   // KV^T, then landmark chunks
  auto issue = [&](int ci) {
    if (ci >= nch) return;  // workgroup-uniform
    const bool wchunk = LIN && ci < 2 * NFC && !(ci & 1);
    const uint32_t soff = (uint32_t)(!LIN ? ci : ci < 2 * NFC ? (ci >> 1) : NFC + ci - 2 * NFC) * (CH * 2);
    uint16_t* dst = slots + (ci % NSLOT) * CH;
#pragma unroll
    for (int i = 0; i < PER_T; ++i)
      copy16_async(wchunk ? rw : rkv, (uint32_t)(tid + 256 * i) * 16, soff, dst + (256 * i + 64 * w) * 8);
  };
  auto end_step = [&]() {
    wait_vmcnt<0>();
    barrier_lds();
  };
  auto slot_of = [&](int ci) -> const uint16_t* { return slots + (ci % NSLOT) * CH; };

  // Prologue: the copies of chunks 0..2 (read from L2 by every tile of the
  // head) and of the bias/ksum vectors start first, then the query loads
  // (from HBM), so that one wait covers all their latencies.
  issue(0);
  issue(1);
  if constexpr (LIN) {  // (landmarks alone: step lc starts chunk lc + 2)
    issue(2);
    const __amdgpu_buffer_rsrc_t rvec = buffer_rsrc(pbh, 2 * F * 4);
    constexpr int NVP = 2 * F * 4 / 16;  // 16-byte pieces of the two vectors (a multiple of 64)
#pragma unroll
    for (int r = 0; r < (NVP + 255) / 256; ++r)
      if (tid + 256 * r < NVP)  // wave-uniform
        copy16_async(rvec, (uint32_t)(tid + 256 * r) * 16, 0, smem + (256 * r + w * 64) * 16);
  }
  Frag<uint16_t> qf[D / 16];
  const uint16_t* Qp = a.Q + ((size_t)bh * N + (tok_ok ? tok : 0)) * D + 8 * g;
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) qf[kb] = ld_frag<uint16_t>(Qp + kb * 16);  // rows past N: row 0, not stored
  const float gh = LIN && L > 0 ? a.g[h] : 0.f;
  end_step();  // chunks 0..2, bias and ksum in LDS (landmarks alone: chunks 0, 1); Q in registers

  // softmax map (identity projection, F == D): the token's feature maximum
  // and inverse sum, from its Q row (half in this lane, half in lane ^ 32)
  // plus the bias (stored in MFMA row order: feature f at kperm(f))
  float qm = 0.f, qinv = 1.f;
  if constexpr (LIN && MAP == kSoftmax) {
    float z[D / 2];
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      frag_to_f32(qf[kb], z + 8 * kb);
#pragma unroll
      for (int j = 0; j < 8; ++j) z[8 * kb + j] += vecS[kperm(kb * 16 + 8 * g + j)];
    }
    softmax_stats<D / 2, 32>(z, qm, qinv);
  }

  f32x16 num[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) num[db] = f32x16{};
  float den = 0.f;

  // ---- the products, one chunk each
  // phi^T of features fc*64.. (two 32-row blocks) = W^T chunk . Q^T + bias
  auto gemm1 = [&](int fc, f32x16 (&acc)[2]) {
    const uint16_t* wt = slot_of(2 * fc);
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) {
      const float* bp = vecS + fc * 64 + fb * 32 + 8 * g;
#pragma unroll
      for (int r = 0; r < 8; ++r) { acc[fb][r] = bp[r]; acc[fb][8 + r] = bp[16 + r]; }
    }
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
        mma(acc[fb], ld_frag<uint16_t>(wt + toff<D, kRowRead>(fb * 32 + c, kb * 16 + 8 * g)), qf[kb]);
  };
  // phi = map(acc) as bf16 operands, and phi . ksum into den
  auto map_den = [&](int fc, const f32x16 (&acc)[2], Frag<uint16_t> (&pb)[4]) {
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) {
      const float* kp = vecS + F + fc * 64 + fb * 32 + 8 * g;
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = phi_q<MAP>(acc[fb][r], qm, qinv);
#pragma unroll
      for (int r = 0; r < 8; ++r) den += p[r] * kp[r] + p[8 + r] * kp[16 + r];
      pb[2 * fb] = to_frag<uint16_t>(p);
      pb[2 * fb + 1] = to_frag<uint16_t>(p + 8);
    }
  };
  // num^T += KV^T chunk . phi^T
  auto gemm2 = [&](int fc, const Frag<uint16_t> (&pb)[4]) {
    const uint16_t* kvt = slot_of(2 * fc + 1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        mma(num[db], ld_frag<uint16_t>(kvt + toff<64, kRowRead>(db * 32 + c, kk * 16 + 8 * g)), pb[kk]);
  };

  // ---- linear branch, software-pipelined: step k issues GEMM1 of feature
  // chunk k and GEMM2 of chunk k - 1 (independent products), then maps the
  // GEMM1 result while the GEMM2 MFMAs are still executing. Step k reads
  // chunks 2k - 1 (KV^T) and 2k (W^T).
  Frag<uint16_t> pb[4];
  if constexpr (LIN) {  // (chunks 1 and 2 are already in flight)
    f32x16 acc[2];
    gemm1(0, acc);
    map_den(0, acc, pb);
    end_step();
  }
  // Steady linear step k (1 <= k < NFC): GEMM1 of feature chunk k (N1 MFMAs,
  // two accumulator chains) then GEMM2 of chunk k - 1 (N2 MFMAs, four chains),
  // one MFMA per slot in a fixed order. Each slot also issues the LDS reads of
  // slot j + LEAD (operand, and for the map the matching ksum pair), and each
  // GEMM2 slot maps PPS pairs of GEMM1's results, so the map's VALU work and
  // the LDS latency both overlap the matrix core's execution.
  constexpr int N1 = 2 * (D / 16), N2 = 4 * (D / 32), NJ = N1 + N2, LEAD = 4, PPS = 16 / N2;
  static_assert(N1 >= LEAD && 16 % N2 == 0, "slot plan");
  auto load_bias = [&](int fc, f32x16 (&acc)[2]) {
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) {
      const float* bp = vecS + fc * 64 + fb * 32 + 8 * g;
#pragma unroll
      for (int r = 0; r < 8; ++r) { acc[fb][r] = bp[r]; acc[fb][8 + r] = bp[16 + r]; }
    }
  };
  f32x16 accb[2];  // the next step's accumulators, holding its bias
  if constexpr (LIN) {
    if (NFC > 1) load_bias(1, accb);
    pin_before(accb[0]);
    pin_before(accb[1]);
  }
  // Step k reads KV^T chunk 2k - 1 and W^T chunk 2k: slots 1 and 2 for odd
  // k, 3 and 0 for even k. Both call sites pass the parity as a literal and
  // the step is inlined, so every operand address folds to a lane base plus
  // an immediate offset.
  auto lin_step = [&](int k, bool ODD) __attribute__((always_inline)) {
    issue(2 * k + 1);
    issue(2 * k + 2);
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* wt = slots + (ODD ? 2 : 0) * CH;
    const uint16_t* kvt = slots + (ODD ? 1 : 3) * CH;
    const float* kbase = vecS + F + k * 64 + 8 * g;
    auto a_ptr = [&](int j) -> const uint16_t* {
      if (j < N1) return wt + toff<D, kRowRead>((j & 1) * 32 + c, (j >> 1) * 16 + 8 * g);
      const int jj = j - N1;
      return kvt + toff<64, kRowRead>((jj % (D / 32)) * 32 + c, (jj / (D / 32)) * 16 + 8 * g);
    };
    // pair t (0..15) of the map: accumulator fb = t / 8, elements 2q, 2q + 1
    // (q = t % 8), features fb * 32 + 8 g + {2q, 2q + 1} (+ 8 from q = 4 on)
    auto k_quad = [&](int t) -> u32x4 {  // pairs t, t + 1 (t even)
      const int fb = t >> 3, q = t & 7;
      return *reinterpret_cast<const u32x4*>(kbase + fb * 32 + (q < 4 ? 2 * q : 16 + 2 * (q - 4)));
    };
    // (The slots run at raised wave priority: of the SIMD's two waves, the
    // one in its slots issues first, the other fills in with its map,
    // softmax or step end.)
    f32x16 acc[2] = {accb[0], accb[1]};
    Frag<uint16_t> fa[NJ];
    u32x4 kq[8];
    u32x4 pw[4];
#pragma unroll
    for (int j = 0; j < LEAD; ++j) fa[j] = ld_frag<uint16_t>(a_ptr(j));
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + LEAD < NJ) fa[j + LEAD] = ld_frag<uint16_t>(a_ptr(j + LEAD));
      if (j + LEAD >= N1 && j + LEAD < NJ)
#pragma unroll
        for (int u = 0; u < PPS; ++u) {
          const int t = (j + LEAD - N1) * PPS + u;
          if ((t & 1) == 0) kq[t >> 1] = k_quad(t);
        }
      if (j < N1) mma(acc[j & 1], fa[j], qf[j >> 1]);
      else mma(num[(j - N1) % (D / 32)], fa[j], pb[(j - N1) / (D / 32)]);
      if (j >= N1) {
#pragma unroll
        for (int u = 0; u < PPS; ++u) {
          const int t = (j - N1) * PPS + u, fb = t >> 3, q = t & 7;
          const float p0 = phi_q<MAP>(acc[fb][2 * q], qm, qinv);
          const float p1 = phi_q<MAP>(acc[fb][2 * q + 1], qm, qinv);
          den = fmaf(p0, __uint_as_float(kq[t >> 1][2 * (t & 1)]), den);
          den = fmaf(p1, __uint_as_float(kq[t >> 1][2 * (t & 1) + 1]), den);
          pw[2 * fb + (q >> 2)][q & 3] = pack_bf16x2(p0, p1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = __builtin_bit_cast(bf16x8, pw[i]);
    load_bias(min(k + 1, NFC - 1), accb);  // unconditional: a branch here would let the map sink past the slots
#pragma unroll
    for (int i = 0; i < 4; ++i) pin_before(pb[i]);
    pin_before(den);
    pin_before(accb[0]);
    pin_before(accb[1]);
    end_step();
  };
  if constexpr (LIN) {
#pragma clang loop unroll(disable)
    for (int k = 1; k < NFC; k += 2) {
      lin_step(k, true);
      if (k + 1 < NFC) lin_step(k + 1, false);  // workgroup-uniform
    }
  }
  // landmark branch state
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const float sl2 = kLog2e * rsqrtf((float)D);
  // S^T of landmark chunk lc = K_L . Q^T
  auto scores = [&](int lc, f32x16& s) {
    const uint16_t* kl = slot_of(LB + lc);
    s = f32x16{};
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) mma(s, ld_frag<uint16_t>(kl + toff<D, kRowRead>(c, kb * 16 + 8 * g)), qf[kb]);
  };
  // online softmax of chunk lc's scores: new running max (rescaling o and l
  // only when it grows by more than 8 in base 2), probabilities as operands
  auto softmax = [&](int lc, f32x16& s, Frag<uint16_t> (&pf)[2]) {
    const int j0 = lc * 32;
    float mx = -INFINITY;
    if (j0 + 32 <= L) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    } else {  // only the last chunk can hold landmarks past L
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (j0 + crow(lane, r) >= L) s[r] = -INFINITY;
        mx = fmaxf(mx, s[r]);
      }
    }
    mx = fmaxf(mx, shfl_xor32(mx)) * sl2;  // base-2 scaled; finite: landmark j0 is valid
    if (__builtin_expect(__any(mx > m + 8.f), 0)) {
      const float mn = fmaxf(m, mx);
      const float corr = fast_exp2(m - mn);
      l *= corr;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= corr;
      m = mn;
    }
    const float nm = -m;
    float p[16], ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) { p[r] = fast_exp2(fmaf(s[r], sl2, nm)); ls += p[r]; }
    l += ls + shfl_xor32(ls);
    pf[0] = to_frag<uint16_t>(p);
    pf[1] = to_frag<uint16_t>(p + 8);
  };
  // o^T += V_L^T . P^T of chunk lc
  auto pv = [&](int lc, const Frag<uint16_t> (&pf)[2]) {
    const uint16_t* vlt = slot_of(LB + lc) + 32 * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      mma(o[db], ld_frag<uint16_t>(vlt + toff32(db * 32 + c, 8 * g)), pf[0]);
      mma(o[db], ld_frag<uint16_t>(vlt + toff32(db * 32 + c, 16 + 8 * g)), pf[1]);
    }
  };

  // last linear step: GEMM2 of the last feature chunk, with the scores of
  // landmark chunk 0 (chunk 2 NFC) beside it (landmarks alone: the scores and
  // softmax of chunk 0, already in LDS with chunk 1)
  f32x16 s;
  Frag<uint16_t> pf[2];
  if constexpr (!LIN) {
    scores(0, s);  // (the launch has L >= 1)
    softmax(0, s, pf);
  } else {
    issue(2 * NFC + 1);
    if (nlc > 0) scores(0, s);  // workgroup-uniform
    gemm2(NFC - 1, pb);
    __builtin_amdgcn_sched_barrier(0);
    den += shfl_xor32(den);
    const float alpha = L > 0 ? 1.f / (1.f + expf(-gh)) : 1.f;  // g = +inf -> 1, g = -inf -> 0
    const float ca = alpha / (den + a.eps);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) num[db][r] *= ca;  // alpha * out_lin
    if (nlc > 0) softmax(0, s, pf);
    end_step();
  }

  // ---- landmark branch, software-pipelined: step lc issues the scores of
  // chunk lc + 1 and the PV product of chunk lc, then runs the softmax of
  // chunk lc + 1 while the PV MFMAs execute. Step lc reads chunks LB + lc
  // (V_L^T) and LB + lc + 1 (K_L), LB = 2 NFC (0 for landmarks alone).
  // The two products alternate one MFMA per slot (the scores are a single
  // accumulation chain; a PV MFMA between two of its links covers the
  // chain's latency), and every operand is read from LDS LEAD slots ahead.
  constexpr int NPV = 2 * (D / 32), NSC = D / 16, NL = NPV + NSC;
  static_assert(NPV == NSC, "one scores MFMA after each PV MFMA");
  auto lm_step = [&](int lc) __attribute__((always_inline)) {
    const uint16_t* kl = slot_of(LB + lc + 1);
    const uint16_t* vlt = slot_of(LB + lc) + 32 * D;
    auto a_ptr = [&](int j) -> const uint16_t* {
      const int i = j >> 1;
      if (j & 1) return kl + toff<D, kRowRead>(c, i * 16 + 8 * g);
      return vlt + toff32((i >> 1) * 32 + c, (i & 1) * 16 + 8 * g);
    };
    Frag<uint16_t> fa[NL];
#pragma unroll
    for (int j = 0; j < LEAD; ++j) fa[j] = ld_frag<uint16_t>(a_ptr(j));
    s = f32x16{};
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      if (j + LEAD < NL) fa[j + LEAD] = ld_frag<uint16_t>(a_ptr(j + LEAD));
      const int i = j >> 1;
      if (j & 1) mma(s, fa[j], qf[i]);
      else mma(o[i >> 1], fa[j], pf[i & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
#pragma clang loop unroll(disable)
  for (int lc = 0; lc + 1 < nlc; ++lc) {
    issue(LB + lc + 2);
    lm_step(lc);
    softmax(lc + 1, s, pf);
    end_step();
  }
  if (nlc > 0) {  // the last chunk: its PV product alone
    pv(nlc - 1, pf);
    end_step();
  }

  // Epilogue: the wave's 32 x D output tile goes through LDS (the slots are
  // free after the last barrier) so that the global stores are whole 16-byte
  // pieces, four full rows per store instruction.
  const float cb = !LIN ? 1.f / l : L > 0 ? (1.f - 1.f / (1.f + expf(-gh))) / l : 0.f;
  if constexpr (OUT32) {
    // the wave's [32 tokens][D] fp32 tile: rows of 4 D bytes swizzled as bf16
    // rows of 2 D columns (a 16-byte piece is 4 floats), 16-byte stores
    uint16_t* ot = slots + w * 32 * 2 * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (LIN ? num[db][4 * q + j] : 0.f) + cb * o[db][4 * q + j];
        *reinterpret_cast<f32x4*>(ot + toff<2 * D, kRowRead>(c, 2 * (db * 32 + 8 * q + 4 * g))) = v;
      }
    wave_lds_order();
    constexpr int PPR = D / 4, NP32 = 32 * PPR / 64;  // pieces per row, per lane
    const uint32_t bytes32 = (uint32_t)((size_t)N * D * 4);  // (the launch checks it fits 32 bits)
    const __amdgpu_buffer_rsrc_t r32 = buffer_rsrc(a.out32 + (size_t)bh * N * D, bytes32);
    u32x4 v32[NP32];
#pragma unroll
    for (int i = 0; i < NP32; ++i) {
      const int P = 64 * i + lane, row = P / PPR, pc = P % PPR;
      v32[i] = *reinterpret_cast<const u32x4*>(ot + toff<2 * D, kRowRead>(row, pc * 8));
    }
#pragma unroll
    for (int i = 0; i < NP32; ++i) {
      const int P = 64 * i + lane, row = P / PPR, pc = P % PPR;
      const int n = tile * 128 + 32 * w + row;
      store16(r32, n < N ? (uint32_t)(n * D + pc * 4) * 4 : bytes32, v32[i]);
    }
    return;
  }
  uint16_t* ot = slots + w * 32 * D;  // [32 tokens][D], kRowRead swizzle
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (LIN ? num[db][4 * q + j] : 0.f) + cb * o[db][4 * q + j];
      st4(ot + toff<D, kRowRead>(c, db * 32 + 8 * q + 4 * g), v[0], v[1], v[2], v[3]);
    }
  wave_lds_order();
  // The stores go through a buffer resource over this (batch, head)'s output
  // rows: a row past N gets offset N D 2 bytes, the resource's size, which
  // the hardware drops. They write through the L2 (the output is not read
  // again by this forward), so the L2 holds no dirty output lines when the
  // kernel ends and its end-of-kernel write-back is short. No branch, so all the LDS reads are in flight at once.
  // (The validated N D < 2^31 keeps every offset within 32 bits.)
  constexpr int PIECES_PER_ROW = D / 8, NP = 32 * PIECES_PER_ROW / 64;
  const uint32_t out_bytes = (uint32_t)((size_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t rout = buffer_rsrc(a.out + (size_t)bh * N * D, out_bytes);
  u32x4 v[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int P = 64 * i + lane, row = P / PIECES_PER_ROW, pc = P % PIECES_PER_ROW;
    v[i] = *reinterpret_cast<const u32x4*>(ot + toff<D, kRowRead>(row, pc * 8));
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int P = 64 * i + lane, row = P / PIECES_PER_ROW, pc = P % PIECES_PER_ROW;
    const int n = tile * 128 + 32 * w + row;
    store16_wt(rout, n < N ? (uint32_t)(n * D + pc * 8) * 2 : out_bytes, v[i]);
  }
}

template <int D, int F, int MAP, bool LIN = true, bool OUT32 = false>
static hipError_t launch_fused_t(const FusedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((fused_query_kernel<D, F, MAP, LIN, OUT32>), dim3(a.nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_softmax_query(const Problem& p, const void* Q, const FusedPack& pk, int L, void* out,
                                hipStream_t s) {
  if (p.dtype != 1 || L < 1 || (p.D != 64 && p.D != 128)) return hipErrorInvalidValue;
  FusedArgs a{};
  a.Q = static_cast<const uint16_t*>(Q);
  a.pack_bh = pk.pack_bh;
  a.bh_bytes = pk.bh_bytes;
  a.H = p.H;
  a.N = p.N;
  a.L = L;
  a.ntiles = (p.N + 127) / 128;
  a.nwg = a.ntiles * p.B * p.H;
  a.out = static_cast<uint16_t*>(out);
  // (F and the map do not enter the landmark-only variant)
  return p.D == 128 ? launch_fused_t<128, 64, kElu1, false>(a, s) : launch_fused_t<64, 64, kElu1, false>(a, s);
}

hipError_t launch_softmax_query_f32(const Problem& p, const void* Q, const FusedPack& pk, int L, float* out,
                                    hipStream_t s) {
  if (p.dtype != 1 || L < 1 || (p.D != 64 && p.D != 128)) return hipErrorInvalidValue;
  if ((size_t)p.N * p.D * 4 >= ((size_t)1 << 32)) return hipErrorInvalidValue;  // the store resource's size
  FusedArgs a{};
  a.Q = static_cast<const uint16_t*>(Q);
  a.pack_bh = pk.pack_bh;
  a.bh_bytes = pk.bh_bytes;
  a.H = p.H;
  a.N = p.N;
  a.L = L;
  a.ntiles = (p.N + 127) / 128;
  a.nwg = a.ntiles * p.B * p.H;
  a.out32 = out;
  return p.D == 128 ? launch_fused_t<128, 64, kElu1, false, true>(a, s) : launch_fused_t<64, 64, kElu1, false, true>(a, s);
}

hipError_t launch_fused_query(const Problem& p, const void* Q, const FusedPack& pk, const float* g, float eps,
                              int L, void* out, hipStream_t s) {
  FusedArgs a;
  a.Q = static_cast<const uint16_t*>(Q);
  a.pack_bh = pk.pack_bh;
  a.pack_w = pk.pack_w;
  a.bh_bytes = pk.bh_bytes;
  a.w_bytes = pk.w_bytes;
  a.g = g;
  a.eps = eps;
  a.H = p.H;
  a.N = p.N;
  a.L = L;
  a.ntiles = (p.N + 127) / 128;
  a.nwg = a.ntiles * p.B * p.H;
  a.out = static_cast<uint16_t*>(out);
  if (p.dtype != 1) return hipErrorInvalidValue;
  if (p.proj && p.F != 256 && p.F != 512 && p.F != 768 && p.F != 1024) return hipErrorInvalidValue;
  if (p.D == 128) {
    if (p.proj) {
      if (p.F == 1024) return launch_fused_t<128, 1024, kElu1>(a, s);
      if (p.F == 768) return launch_fused_t<128, 768, kElu1>(a, s);
      return p.F == 512 ? launch_fused_t<128, 512, kElu1>(a, s) : launch_fused_t<128, 256, kElu1>(a, s);
    }
    if (p.fmap == kRelu) return launch_fused_t<128, 128, kRelu>(a, s);
    if (p.fmap == kSoftmax) return launch_fused_t<128, 128, kSoftmax>(a, s);
    return launch_fused_t<128, 128, kElu1>(a, s);
  }
  if (p.D == 64) {
    if (p.proj) {
      if (p.F == 1024) return launch_fused_t<64, 1024, kElu1>(a, s);
      if (p.F == 768) return launch_fused_t<64, 768, kElu1>(a, s);
      return p.F == 512 ? launch_fused_t<64, 512, kElu1>(a, s) : launch_fused_t<64, 256, kElu1>(a, s);
    }
    if (p.fmap == kRelu) return launch_fused_t<64, 64, kRelu>(a, s);
    if (p.fmap == kSoftmax) return launch_fused_t<64, 64, kSoftmax>(a, s);
    return launch_fused_t<64, 64, kElu1>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ttr

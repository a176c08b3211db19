// bf16 hot path, stage 2: apply + landmark softmax + blend over Q in one pass.
//   out = alpha_h . phi(Q) KV / (phi(Q) . ksum + eps)
//       + (1 - alpha_h) . softmax(Q K_L^T / sqrt(D)) V_L,      alpha_h = sigmoid(g_h)
// ("Flux2TTRTrainer", section "How the distillation works": linear kernel
// branch + exact softmax over landmark tokens + bounded blend; "NNT Define
// Linear Attention", sections "The inputs" and "How it works".)
//
// Workgroup: 4 waves x 32 query tokens, two workgroups per compute unit (two
// waves per SIMD, so one wave's exp/elu work overlaps the other's MFMAs).
// The per-head operands come from the pack written by the key/value stage as
// a sequence of equal-size chunks (W^T, KV^T alternately per 64 features,
// then one K_L + V_L^T chunk per 32 landmarks). They stream global ->
// registers -> three LDS slots, two chunks ahead of the one being consumed in
// the linear branch and one ahead in the landmark branch (whose accumulators
// leave room for one register set only), one barrier per chunk. Q stays in registers as the B operand of every
// product, and every operand read from LDS is a plain 16-byte row read:
//   W^T chunk:   phi^T [64 f x tok]  = W^T . Q^T (+ bias, then elu + 1; phi . ksum)
//   KV^T chunk:  num^T [D x tok]    += KV^T . phi^T
//   landmark chunk (32 landmarks: K_L then V_L^T):
//                S^T  [32 j x tok]   = K_L . Q^T  (scaled to base 2, online max)
//                o^T  [D x tok]     += V_L^T . P^T
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
};

template <int D, int F, int MAP>
__global__ __launch_bounds__(256, 2) void fused_query_kernel(FusedArgs a) {
  constexpr int CH = 64 * D;  // elements per chunk (every chunk kind)
  constexpr int NFC = F / 64;
  constexpr int PER_T = CH * 2 / 16 / 256;  // 16-byte pieces per thread per chunk
  static_assert(PER_T * 256 * 16 == CH * 2, "whole pieces");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * F * 4 + 3 * CH * 2];
  float* vecS = reinterpret_cast<float*>(smem);  // biasP [F] | ksumP [F]
  uint16_t* const slots = reinterpret_cast<uint16_t*>(smem + 2 * F * 4);  // 3 chunk slots

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
  const uint16_t* kvpk = reinterpret_cast<const uint16_t*>(pbh + 2 * F * 4);
  const uint16_t* lmpk = kvpk + F * D;
  const int nlc = (L + 31) / 32;  // landmark chunks
  const int nch = 2 * NFC + nlc;

  // Chunk ci streams global -> registers -> LDS slot ci % 3. Its loads are
  // issued two chunks ahead (at the start of step ci - 2, into register set
  // ci & 1) and it is written to LDS at the end of step ci - 1, so each load
  // has two steps of compute to land. The sets are named statically (the
  // loops below take chunks in pairs of even and odd index), and loads are
  // issued on every step (indexes clamped) so the compiler's count of loads
  // in flight, and with it every wait, is exact.
  auto chunk_src = [&](int ci) {
    ci = min(ci, nch - 1);
    return reinterpret_cast<const u32x4*>(ci < 2 * NFC ? ((ci & 1) ? kvpk : wpk) + (ci >> 1) * CH
                                                       : lmpk + (ci - 2 * NFC) * CH);
  };
  u32x4 sa[PER_T], sb[PER_T];  // register sets for even / odd chunks
  auto load_to = [&](u32x4 (&st)[PER_T], int ci) {
    const u32x4* s4 = chunk_src(ci);
#pragma unroll
    for (int i = 0; i < PER_T; ++i) st[i] = s4[tid + 256 * i];
  };
  auto store_from = [&](const u32x4 (&st)[PER_T], int ci) {
    u32x4* d4 = reinterpret_cast<u32x4*>(slots + (ci % 3) * CH);
#pragma unroll
    for (int i = 0; i < PER_T; ++i) d4[tid + 256 * i] = st[i];
  };
  auto slot_of = [&](int ci) -> const uint16_t* { return slots + (ci % 3) * CH; };

  // prologue: query fragments, then chunks 0 and 1; chunk 0 to LDS
  Frag<uint16_t> qf[D / 16];
  const uint16_t* Qp = a.Q + ((size_t)bh * N + (tok_ok ? tok : 0)) * D + 8 * g;
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) qf[kb] = ld_frag<uint16_t>(Qp + kb * 16);  // rows past N: row 0, not stored
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(pbh);
    u32x4* dst = reinterpret_cast<u32x4*>(smem);
    for (int i = tid; i < 2 * F * 4 / 16; i += 256) dst[i] = src[i];
  }
  const float gh = L > 0 ? a.g[h] : 0.f;
  load_to(sa, 0);
  load_to(sb, 1);
  store_from(sa, 0);

  f32x16 num[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) num[db] = f32x16{};
  float den = 0.f;

  // softmax map (identity projection, F == D): the token's feature maximum
  // and inverse sum, from its Q row (half in this lane, half in lane ^ 32)
  // plus the bias (stored in MFMA row order: feature f at kperm(f))
  float qm = 0.f, qinv = 1.f;
  if constexpr (MAP == kSoftmax) {
    barrier_lds();  // bias in LDS
    float z[D / 2];
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      frag_to_f32(qf[kb], z + 8 * kb);
#pragma unroll
      for (int j = 0; j < 8; ++j) z[8 * kb + j] += vecS[kperm(kb * 16 + 8 * g + j)];
    }
    softmax_stats<D / 2, 32>(z, qm, qinv);
  }

  // ---- linear branch: per 64 features, a W^T chunk (even) then a KV^T chunk (odd)
#pragma clang loop unroll(disable)
  for (int fc = 0; fc < NFC; ++fc) {
    const int ci = 2 * fc;
    barrier_lds();  // chunk ci in LDS; every wave is done with step ci - 1
    load_to(sa, ci + 2);
    Frag<uint16_t> pb[4];  // phi^T of these 64 features, 4 k-blocks of 16
    {
      const uint16_t* wt = slot_of(ci);
      // two independent accumulation chains (feature blocks 0 and 1), interleaved
      f32x16 acc[2];
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
#pragma unroll
      for (int fb = 0; fb < 2; ++fb) {
        const float* kp = vecS + F + fc * 64 + fb * 32 + 8 * g;
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = phi_of<MAP>(acc[fb][r], qm, qinv);
#pragma unroll
        for (int r = 0; r < 8; ++r) den += p[r] * kp[r] + p[8 + r] * kp[16 + r];
        pb[2 * fb] = to_frag<uint16_t>(p);
        pb[2 * fb + 1] = to_frag<uint16_t>(p + 8);
      }
    }
    store_from(sb, ci + 1);
    barrier_lds();  // chunk ci + 1 in LDS
    load_to(sb, ci + 3);
    {
      const uint16_t* kvt = slot_of(ci + 1);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          mma(num[db], ld_frag<uint16_t>(kvt + toff<64, kRowRead>(db * 32 + c, kk * 16 + 8 * g)), pb[kk]);
    }
    if (ci + 2 < nch) store_from(sa, ci + 2);
  }
  den += shfl_xor32(den);
  {
    const float inv = 1.f / (den + a.eps);
    const float alpha = L > 0 ? 1.f / (1.f + expf(-gh)) : 1.f;  // g = +inf -> 1, g = -inf -> 0
    const float ca = alpha * inv;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) num[db][r] *= ca;  // alpha * out_lin
  }

  // ---- landmark branch: one chunk per 32 landmarks, K_L [32 j][D] then V_L^T [D][32 j]
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const float sl2 = kLog2e * rsqrtf((float)D);
  auto lm_step = [&](int lc) {
    const uint16_t* kl = slot_of(2 * NFC + lc);
    const uint16_t* vlt = kl + 32 * D;
    const int j0 = lc * 32;
    f32x16 s = f32x16{};
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) mma(s, ld_frag<uint16_t>(kl + toff<D, kRowRead>(c, kb * 16 + 8 * g)), qf[kb]);
    // row max of the raw scores (landmarks past L masked to -inf; only the last
    // chunk can hold such landmarks)
    float mx = -INFINITY;
    if (j0 + 32 <= L) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    } else {
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
    const Frag<uint16_t> p0 = to_frag<uint16_t>(p), p1 = to_frag<uint16_t>(p + 8);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      mma(o[db], ld_frag<uint16_t>(vlt + toff32(db * 32 + c, 8 * g)), p0);
      mma(o[db], ld_frag<uint16_t>(vlt + toff32(db * 32 + c, 16 + 8 * g)), p1);
    }
  };
  // The first landmark chunk's successor is already in set b (loaded by the
  // last linear step); after it, one register set suffices: each step loads
  // its successor and writes it to LDS at its end.
  if (nlc > 0) {  // workgroup-uniform
    barrier_lds();
    lm_step(0);
    if (2 * NFC + 1 < nch) store_from(sb, 2 * NFC + 1);
  }
#pragma clang loop unroll(disable)
  for (int lc = 1; lc < nlc; ++lc) {
    const int ci = 2 * NFC + lc;
    barrier_lds();
    load_to(sa, ci + 1);
    lm_step(lc);
    if (ci + 1 < nch) store_from(sa, ci + 1);
  }
  barrier_lds();  // the slots are free for the output staging

  // Epilogue: the wave's 32 x D output tile goes through LDS so that the
  // global stores are whole 16-byte pieces, four full rows per store instruction.
  const float cb = L > 0 ? (1.f - 1.f / (1.f + expf(-gh))) / l : 0.f;
  uint16_t* ot = slots + w * 32 * D;  // [32 tokens][D], kRowRead swizzle
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = num[db][4 * q + j] + cb * o[db][4 * q + j];
      st4(ot + toff<D, kRowRead>(c, db * 32 + 8 * q + 4 * g), v[0], v[1], v[2], v[3]);
    }
  wave_lds_order();
  constexpr int PIECES_PER_ROW = D / 8;
  uint16_t* obase = a.out + ((size_t)bh * N + tile * 128 + 32 * w) * D;
#pragma unroll
  for (int i = 0; i < 32 * PIECES_PER_ROW / 64; ++i) {
    const int P = 64 * i + lane;
    const int row = P / PIECES_PER_ROW, pc = P % PIECES_PER_ROW;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ot + toff<D, kRowRead>(row, pc * 8));
    if (tile * 128 + 32 * w + row < N) *reinterpret_cast<u32x4*>(obase + (size_t)row * D + pc * 8) = v;
  }
}

template <int D, int F, int MAP>
static hipError_t launch_fused_t(const FusedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((fused_query_kernel<D, F, MAP>), dim3(a.nwg), dim3(256), 0, s, a);
  return hipGetLastError();
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
  if (p.D == 128) {
    if (p.proj) return launch_fused_t<128, 256, kElu1>(a, s);
    if (p.fmap == kRelu) return launch_fused_t<128, 128, kRelu>(a, s);
    if (p.fmap == kSoftmax) return launch_fused_t<128, 128, kSoftmax>(a, s);
    return launch_fused_t<128, 128, kElu1>(a, s);
  }
  if (p.D == 64) {
    if (p.proj) return launch_fused_t<64, 256, kElu1>(a, s);
    if (p.fmap == kRelu) return launch_fused_t<64, 64, kRelu>(a, s);
    if (p.fmap == kSoftmax) return launch_fused_t<64, 64, kSoftmax>(a, s);
    return launch_fused_t<64, 64, kElu1>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ttr

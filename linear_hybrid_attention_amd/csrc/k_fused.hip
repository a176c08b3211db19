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
// then one K_L + V_L chunk per 32 landmarks). They stream through two LDS
// slots: the global loads of the next chunk are issued into registers before
// the current chunk is consumed and written to the free slot after it, one
// barrier per chunk. (Direct global -> LDS copies are avoided here: while one
// is in flight the compiler drains every LDS read with lgkmcnt(0), which
// stalls each MFMA on the prefetch.) Q stays in registers as the B operand of every product:
//   W^T chunk:   phi^T [64 f x tok]  = W^T . Q^T (+ bias, then elu + 1; phi . ksum)
//   KV^T chunk:  num^T [D x tok]    += KV^T . phi^T
//   landmark chunk (32 landmarks: K_L then V_L):
//                S^T  [32 j x tok]   = K_L . Q^T  (scaled to base 2, online max)
//                o^T  [D x tok]     += V_L^T . P^T  (V_L read transposed)
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

template <int D, int F>
__global__ __launch_bounds__(256, 2) void fused_query_kernel(FusedArgs a) {
  constexpr int CH = 64 * D;  // elements per chunk (every chunk kind)
  constexpr int NFC = F / 64;
  constexpr int PER_T = CH * 2 / 16 / 256;  // 16-byte pieces per thread per chunk
  static_assert(PER_T * 256 * 16 == CH * 2, "whole pieces");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * F * 4 + 2 * CH * 2];
  float* vecS = reinterpret_cast<float*>(smem);  // biasP [F] | ksumP [F]
  uint16_t* slot0 = reinterpret_cast<uint16_t*>(smem + 2 * F * 4);
  uint16_t* slot1 = slot0 + CH;

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

  // Register-staged chunk copies: the global loads of chunk ci + 1 are issued
  // before chunk ci is consumed and written to the other LDS slot after it.
  u32x4 stg[PER_T];
  auto load_chunk = [&](int ci) {
    const uint16_t* src = ci < 2 * NFC ? ((ci & 1) ? kvpk : wpk) + (ci >> 1) * CH : lmpk + (ci - 2 * NFC) * CH;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
#pragma unroll
    for (int i = 0; i < PER_T; ++i) stg[i] = s4[tid + 256 * i];
  };
  auto store_chunk = [&](uint16_t* slot) {
    u32x4* d4 = reinterpret_cast<u32x4*>(slot);
#pragma unroll
    for (int i = 0; i < PER_T; ++i) d4[tid + 256 * i] = stg[i];
  };

  // prologue: bias/ksum vectors, chunk 0, Q fragments
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(pbh);
    u32x4* dst = reinterpret_cast<u32x4*>(smem);
    for (int i = tid; i < 2 * F * 4 / 16; i += 256) dst[i] = src[i];
  }
  load_chunk(0);
  store_chunk(slot0);
  Frag<uint16_t> qf[D / 16];
  const uint16_t* Qp = a.Q + ((size_t)bh * N + (tok_ok ? tok : 0)) * D + 8 * g;
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) qf[kb] = tok_ok ? ld_frag<uint16_t>(Qp + kb * 16) : zero_frag<uint16_t>();
  barrier_lds();

  f32x16 num[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) num[db] = f32x16{};
  float den = 0.f;

  // ---- linear branch: per 64 features, a W^T chunk (slot 0) then a KV^T chunk (slot 1)
#pragma clang loop unroll(disable)
  for (int fc = 0; fc < NFC; ++fc) {
    load_chunk(2 * fc + 1);
    Frag<uint16_t> pb[4];  // phi^T of these 64 features, 4 k-blocks of 16
    {
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
          mma(acc[fb], ld_frag<uint16_t>(slot0 + toff<D, kRowRead>(fb * 32 + c, kb * 16 + 8 * g)), qf[kb]);
#pragma unroll
      for (int fb = 0; fb < 2; ++fb) {
        const float* kp = vecS + F + fc * 64 + fb * 32 + 8 * g;
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = elu1(acc[fb][r]);
#pragma unroll
        for (int r = 0; r < 8; ++r) den += p[r] * kp[r] + p[8 + r] * kp[16 + r];
        pb[2 * fb] = to_frag<uint16_t>(p);
        pb[2 * fb + 1] = to_frag<uint16_t>(p + 8);
      }
    }
    store_chunk(slot1);
    barrier_lds();
    if (2 * fc + 2 < nch) load_chunk(2 * fc + 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        mma(num[db], ld_frag<uint16_t>(slot1 + toff<64, kRowRead>(db * 32 + c, kk * 16 + 8 * g)), pb[kk]);
    if (2 * fc + 2 < nch) store_chunk(slot0);
    barrier_lds();
  }
  den += shfl_xor32(den);
  {
    const float inv = 1.f / (den + a.eps);
    const float alpha = L > 0 ? 1.f / (1.f + expf(-a.g[h])) : 1.f;  // g = +inf -> 1, g = -inf -> 0
    const float ca = alpha * inv;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) num[db][r] *= ca;  // alpha * out_lin
  }

  // ---- landmark branch: one chunk per 32 landmarks, K_L [32 j][D] then V_L [32 j][D];
  // chunk lc sits in slot lc % 2 (the linear branch used an even number of chunks)
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const float sl2 = kLog2e * rsqrtf((float)D);
#pragma clang loop unroll(disable)
  for (int lc = 0; lc < nlc; ++lc) {
    const int ci = 2 * NFC + lc;
    if (ci + 1 < nch) load_chunk(ci + 1);
    const uint16_t* sl = (lc & 1) ? slot1 : slot0;
    const uint16_t* vl = sl + 32 * D;
    const int j0 = lc * 32;
    // scores: two independent half-depth chains, added at the end
    f32x16 s = f32x16{}, s2 = f32x16{};
#pragma unroll
    for (int kb = 0; kb < D / 16; kb += 2) {
      mma(s, ld_frag<uint16_t>(sl + toff<D, kRowRead>(c, kb * 16 + 8 * g)), qf[kb]);
      mma(s2, ld_frag<uint16_t>(sl + toff<D, kRowRead>(c, kb * 16 + 16 + 8 * g)), qf[kb + 1]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] += s2[r];
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
      mma(o[db], tr_frag<D>(vl, 0, 32 * db, lane), p0);
      mma(o[db], tr_frag<D>(vl, 16, 32 * db, lane), p1);
    }
    if (ci + 1 < nch) store_chunk((lc & 1) ? slot0 : slot1);
    barrier_lds();
  }

  // Epilogue: the wave's 32 x D output tile goes through LDS (the ring is free
  // after the last barrier) so that the global stores are whole 16-byte pieces,
  // four full rows per store instruction.
  const float cb = L > 0 ? (1.f - 1.f / (1.f + expf(-a.g[h]))) / l : 0.f;
  uint16_t* ot = slot0 + w * 32 * D;  // [32 tokens][D], kRowRead swizzle
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

template <int D, int F>
static hipError_t launch_fused_t(const FusedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((fused_query_kernel<D, F>), dim3(a.nwg), dim3(256), 0, s, a);
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
  if (p.D == 128) return p.proj ? launch_fused_t<128, 256>(a, s) : launch_fused_t<128, 128>(a, s);
  if (p.D == 64) return p.proj ? launch_fused_t<64, 256>(a, s) : launch_fused_t<64, 64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace ttr

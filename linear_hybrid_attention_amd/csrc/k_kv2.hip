// bf16 hot path, stage 1: key/value reduction and the per-head operand pack.
//
// kv2_partial_kernel: KV = phi(K)^T V and ksum over one token range of one
// (batch, head) ("NNT Define Linear Attention", section "How it works":
// K'^T V first, sum(K') for the normaliser; phi(x) = elu(x W_h + b_h) + 1 per
// "Flux2TTRTrainer", section "Inputs worth setting", and the elu(x) + 1 map of
// the linear-attention page, section "The inputs").
//   8 waves, two per SIMD. Wave w owns features f0 = 32 (w % NFS) ..
//   f0 + 31 and keeps that slice of W in registers. Per step of 32 tokens:
//     phi[tok x 32]  = K[tok x D] . W[:, slice]     (A = K rows from LDS)
//     KV[32 x D]    += phi^T . V                    (B = V read transposed
//                                                    from LDS, ds_read_b64_tr_b16)
//   K and V rows of 128-token super-steps are loaded into registers one
//   super-step ahead and written to a double LDS buffer; one barrier per
//   super-step.
//
// kv2_pack_kernel: adds the split partials in split order (deterministic) and
// writes the operands of the fused query kernel as bf16 "chunks" that are
// exact images of its LDS tiles (swizzled, feature order matched to the MFMA
// register layout), so that kernel stages them with straight 16-byte copies:
//   per head h:         W^T chunks  [64 f][D]        (F / 64 of them)
//   per (batch, head):  bias, ksum  [F] fp32 each, in kperm order
//                       KV^T chunks [D][64 f]        (F / 64)
//                       per 32 landmarks: K_L [32 j][D], V_L^T [D][32 j]
//   with landmarks idx_j = floor(j N / L) ("Flux2TTRTrainer", section "How the
//   distillation works": exact softmax over strided landmark tokens).
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace ttr {

// ---------------------------------------------------------------- pack layout
// Every chunk holds 64 * D bf16 elements:
//   W^T chunk   [64 f][D]   kRowRead      KV^T chunk [D][64 f]   kRowRead
//   landmark chunk: K_L [32 j][D] kRowRead, then V_L^T [D][32 j] (toff32),
//   landmark j in column kperm(j)
// Feature columns of a KV^T chunk are in MFMA C-row order: column
// (f & 32) + kperm(f & 31) holds feature f of the chunk.
struct PackLayout {
  int D, F, L, nlb;  // nlb: landmark chunks of 32
  __host__ __device__ size_t vec_bytes() const { return (size_t)2 * F * 4; }
  __host__ __device__ size_t chunk_elems() const { return (size_t)64 * D; }
  __host__ __device__ size_t kv_bytes() const { return (size_t)F * D * 2; }
  __host__ __device__ size_t lm_bytes() const { return (size_t)nlb * chunk_elems() * 2; }
  __host__ __device__ size_t bh_bytes() const { return vec_bytes() + kv_bytes() + lm_bytes(); }
  __host__ __device__ size_t w_bytes() const { return (size_t)F * D * 2; }
};

// ---------------------------------------------------------------- kv2 partial kernel
struct Kv2Args {
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* W;  // [H][D][F] or NULL (identity)
  const float* bias;  // [H][F] or NULL
  int H, N, chunk, nsplit;
  float* part;             // [BH][nsplit][F*D + F]
  unsigned char* pack_w;   // [H][F*D bf16]: W^T chunks, written by split 0 of batch 0
};

template <int D, int F>
struct Kv2Shape {
  static constexpr int NW = 8;
  static constexpr int NFS = F / 32;
  static constexpr int NTW = NW / NFS;
  static constexpr int STEP = 32 * NTW;           // tokens all waves consume per MFMA step
  static constexpr int SS = 128;                  // tokens per staged super-step
  static_assert(SS % STEP == 0, "whole steps per super-step");
  static constexpr int TILE = SS * D;             // elements of the K (or V) tile of a super-step
  static constexpr int BUF = 2 * TILE;            // K tile, then V tile
  static constexpr int PER_T = BUF / 8 / 512;     // 16-byte pieces per thread per super-step
  static_assert(PER_T * 512 * 8 == BUF && (TILE / 8) % 512 == 0, "whole pieces, K/V split per piece index");
  using WR = LdsRow<uint16_t, D>;                 // W^T [F][D] staging (prologue)
  static constexpr int w_bytes = F * WR::bytes_per_row;
  static constexpr int ring_bytes = 2 * BUF * 2 + 2 * SS * 8;  // K/V double buffer, then per-token softmax stats
  static constexpr int red_floats = (D / 32) * 16 * 64 + 64;  // one wave's KV slice + ksum
  static constexpr int r_bytes = (NTW - 1) * NFS * red_floats * 4;
  static constexpr int m1 = w_bytes > ring_bytes ? w_bytes : ring_bytes;
  static constexpr int bytes = m1 > r_bytes ? m1 : r_bytes;
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Work item of workgroup i in a one-dimensional grid of n: the hardware places
// workgroup i on XCD i % 8, so items are renumbered such that consecutive ones
// (the splits or jobs of one (batch, head)) run on one XCD and share its L2
// copy of that head's W and partials.
__device__ __forceinline__ int xcd_item(int i, int n) {
  const int per = n / 8;
  return i < per * 8 ? (i % 8) * per + i / 8 : i;
}

template <int D, int F, bool PROJ, int MAP>
__global__ __launch_bounds__(512, 1) void kv2_partial_kernel(Kv2Args a) {
  using S = Kv2Shape<D, F>;
  constexpr int NFS = S::NFS, NTW = S::NTW, STEP = S::STEP, SS = S::SS, PER_T = S::PER_T;
  using WR = typename S::WR;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::bytes];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int split = item % a.nsplit, bh = item / a.nsplit, h = bh % a.H;
  const int fs = w % NFS, tw = w / NFS, f0 = 32 * fs;
  const int N = a.N;
  const int t_begin = split * a.chunk;
  const int t_end = min(N, t_begin + a.chunk);
  const int nss = (t_end - t_begin + SS - 1) / SS;
  const uint16_t* K = a.K + (size_t)bh * N * D;
  const uint16_t* V = a.V + (size_t)bh * N * D;

  // K/V staging through registers: piece i of thread tid is piece tid + 512 i
  // of the super-step (K pieces first). Rows past the range repeat the last
  // valid token; their phi is masked to zero below, so they add nothing.
  // (Direct global -> LDS copies are not used: the compiler waits for every
  // such copy in flight before a transposed LDS read, which would serialise
  // the prefetch.)
  u32x4 stg[PER_T];
  auto load_stg = [&](int ss) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const bool isv = i >= PER_T / 2;
      const int Pl = tid + 512 * (isv ? i - PER_T / 2 : i);
      const int row = Pl / (D / 8), p = Pl % (D / 8);
      const int t = min(t_begin + ss * SS + row, t_end - 1);
      stg[i] = *reinterpret_cast<const u32x4*>((isv ? V : K) + (size_t)t * D + p * 8);
    }
  };
  uint16_t* const ring = reinterpret_cast<uint16_t*>(smem);
  float2* const stats = reinterpret_cast<float2*>(smem + 2 * S::BUF * 2);  // [2][SS] (max, 1 / sum)
  // softmax map (identity projection, F == D): a thread's K pieces are all
  // logical piece tid % (D / 8) of their rows, so its 8 bias values are fixed
  float kbias[8];
  if constexpr (MAP == kSoftmax) {
#pragma unroll
    for (int j = 0; j < 8; ++j) kbias[j] = a.bias ? a.bias[(size_t)h * F + (tid % (D / 8)) * 8 + j] : 0.f;
  }
  auto store_stg = [&](int buf) {
    uint16_t* kt = ring + buf * S::BUF;
    uint16_t* vt = kt + S::TILE;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const bool isv = i >= PER_T / 2;
      const int Pl = tid + 512 * (isv ? i - PER_T / 2 : i);
      const int row = Pl / (D / 8), p = Pl % (D / 8);
      if (isv) {
        *reinterpret_cast<u32x4*>(vt + toff<D, kTrRead>(row, p * 8)) = stg[i];
      } else {
        *reinterpret_cast<u32x4*>(kt + toff<D, kRowRead>(row, p * 8)) = stg[i];
        if constexpr (MAP == kSoftmax) {  // the row's D / 8 pieces: D / 8 consecutive lanes
          const Vec8<uint16_t> kv8 = __builtin_bit_cast(Vec8<uint16_t>, stg[i]);
          float z[8], m, inv;
#pragma unroll
          for (int j = 0; j < 8; ++j) z[j] = bf2f(kv8.v[j]) + kbias[j];
          softmax_stats<8, D / 8 - 1>(z, m, inv);
          if (p == 0) stats[buf * SS + row] = float2{m, inv};
        }
      }
    }
  };
  load_stg(0);  // in flight during the W staging below

  // W slice as B operand (lane = feature column f0 + c, k = D), via a transposed LDS image.
  Frag<uint16_t> wf[D / 16];
  {
    uint16_t* Wt = reinterpret_cast<uint16_t*>(smem);
    if constexpr (PROJ) {
      const uint16_t* W = a.W + (size_t)h * D * F;
      static_assert((D / 2) * (F / 8) % 512 == 0, "whole rounds");
#pragma unroll
      for (int u = tid; u < (D / 2) * (F / 8); u += 512) {
        const int d = 2 * (u % (D / 2)), fo = (u / (D / 2)) * 8;
        const Vec8<uint16_t> w0 = ld8(W + (size_t)d * F + fo);
        const Vec8<uint16_t> w1 = ld8(W + (size_t)(d + 1) * F + fo);
#pragma unroll
        for (int j = 0; j < 8; ++j) st_pair(Wt + (fo + j) * WR::stride + d, w0.v[j], w1.v[j]);
      }
    } else {
      for (int u = tid; u < F * D; u += 512) {
        const int f = u / D, d = u % D;
        Wt[f * WR::stride + d] = f == d ? (uint16_t)0x3f80 : (uint16_t)0;  // bf16 1.0 / 0.0
      }
    }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) wf[kb] = ld_frag<uint16_t>(Wt + (f0 + c) * WR::stride + kb * 16 + 8 * g);
    __syncthreads();  // the region becomes the K/V double buffer
    // The fused query kernel's W^T chunks [64 f][D] (kRowRead) are per head:
    // one workgroup per head writes them, each lane its row f0 + c in 16-byte pieces.
    if (split == 0 && bh < a.H && tw == 0) {
      uint16_t* wc = reinterpret_cast<uint16_t*>(a.pack_w + (size_t)h * F * D * 2) + (size_t)((f0 + c) / 64) * 64 * D;
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb)
        *reinterpret_cast<u32x4*>(wc + toff<D, kRowRead>((f0 + c) & 63, kb * 16 + 8 * g)) = __builtin_bit_cast(u32x4, wf[kb]);
    }
  }
  const float bcol = a.bias ? a.bias[(size_t)h * F + f0 + c] : 0.f;
  f32x16 bias16;  // GEMM1 starts from the bias (MFMA C operand, only read)
#pragma unroll
  for (int r = 0; r < 16; ++r) bias16[r] = bcol;

  f32x16 kv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) kv[db] = f32x16{};
  float ks = 0.f;

  store_stg(0);
  if (nss > 1) load_stg(1);
  for (int ss = 0; ss < nss; ++ss) {
    barrier_lds();  // super-step ss is in buffer ss & 1; every wave is done with the other buffer
    const uint16_t* kt = ring + (ss & 1) * S::BUF;
    const uint16_t* vt = kt + S::TILE;
#pragma unroll
    for (int j = 0; j < SS / STEP; ++j) {
      const int r0 = j * STEP + 32 * tw;  // this wave's 32 rows of the super-step
      const int t0 = t_begin + ss * SS + r0;
      if (t0 >= t_end) break;  // wave-uniform
      // two independent chains over alternate k-blocks, added at the end
      f32x16 acc = mma_from(bias16, ld_frag<uint16_t>(kt + toff<D, kRowRead>(r0 + c, 8 * g)), wf[0]);
      f32x16 acc2 = mma_from(f32x16{}, ld_frag<uint16_t>(kt + toff<D, kRowRead>(r0 + c, 16 + 8 * g)), wf[1]);
#pragma unroll
      for (int kb = 2; kb < D / 16; kb += 2) {
        mma(acc, ld_frag<uint16_t>(kt + toff<D, kRowRead>(r0 + c, kb * 16 + 8 * g)), wf[kb]);
        mma(acc2, ld_frag<uint16_t>(kt + toff<D, kRowRead>(r0 + c, kb * 16 + 16 + 8 * g)), wf[kb + 1]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += acc2[r];
      float p[16];
      // softmax: (max, 1 / sum) of the row's token, from the staging pass
      auto st = [&](int r) {
        if constexpr (MAP == kSoftmax) return stats[(ss & 1) * SS + r0 + crow(lane, r)];
        else return float2{0.f, 1.f};
      };
      if (t0 + 32 <= t_end) {  // wave-uniform: only the range's last step has rows past it
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float2 sr = st(r);
          p[r] = phi_of<MAP>(acc[r], sr.x, sr.y);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float2 sr = st(r);
          p[r] = t0 + crow(lane, r) < t_end ? phi_of<MAP>(acc[r], sr.x, sr.y) : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) ks += p[r];
      const Frag<uint16_t> pa0 = to_frag<uint16_t>(p), pa1 = to_frag<uint16_t>(p + 8);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        mma(kv[db], pa0, tr_frag<D>(vt, r0, 32 * db, lane));
        mma(kv[db], pa1, tr_frag<D>(vt, r0 + 16, 32 * db, lane));
      }
    }
    // The only global loads in flight are the staged super-step's, so this
    // wait (issued one super-step ago) is the full count.
    if (ss + 1 < nss) {
      store_stg((ss + 1) & 1);
      if (ss + 2 < nss) load_stg(ss + 2);
    }
  }
  ks += shfl_xor32(ks);
  __syncthreads();  // K/V buffers no longer read

  if constexpr (NTW > 1) {
    float* red = reinterpret_cast<float*>(smem);
    if (tw > 0) {
      float* rb = red + ((tw - 1) * NFS + fs) * S::red_floats;
      int i = 0;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) rb[(i++) * 64 + lane] = kv[db][r];
      rb[i * 64 + lane] = ks;
    }
    __syncthreads();
    if (tw == 0) {
      for (int t2 = 1; t2 < NTW; ++t2) {
        const float* rb = red + ((t2 - 1) * NFS + fs) * S::red_floats;
        int i = 0;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) kv[db][r] += rb[(i++) * 64 + lane];
        ks += rb[i * 64 + lane];
      }
    }
  }
  if (tw == 0) {
    float* kvo = a.part + ((size_t)bh * a.nsplit + split) * (size_t)(F * D + F);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) kvo[(size_t)(f0 + crow(lane, r)) * D + db * 32 + c] = kv[db][r];
    if (g == 0) kvo[F * D + f0 + c] = ks;
  }
}

// ---------------------------------------------------------------- pack kernel
struct PackArgs {
  const float* part;  // [BH][nsplit][F*D + F]
  int nsplit;
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* W;
  const float* bias;
  int H, N, L;
  unsigned char* pack_bh;  // [BH][bh_bytes]
  unsigned char* pack_w;   // [H][w_bytes]
  int lm_only;             // 1: the landmark jobs alone, into a pack of landmark chunks only
};

// Jobs of one (batch, head), by job index:
//   [0, KVJ)            KV^T rows: FJ features x D (sum of partials), ksum, bias
//   then one per 32-landmark chunk (K_L and V_L^T)
// (The W^T chunks are written by the partial kernel, which holds W in registers.)
template <int D, int F, bool PROJ>
__global__ __launch_bounds__(256) void kv2_pack_kernel(PackArgs a) {
  constexpr int FJ = 2048 / D > F ? F : 2048 / D;  // features per KV job: (FJ/2)*(D/4) = 256 threads
  constexpr int KVJ = F / FJ;
  const int tid = threadIdx.x;
  const int nlb = (a.L + 31) / 32;
  const int item = xcd_item(blockIdx.x, gridDim.x), njobs = a.lm_only ? nlb : KVJ + nlb;
  const int bh = item / njobs, h = bh % a.H;
  PackLayout pl{D, a.lm_only ? 0 : F, a.L, nlb};
  unsigned char* base = a.pack_bh + (size_t)bh * pl.bh_bytes();
  float* biasP = reinterpret_cast<float*>(base);
  float* ksumP = biasP + F;
  uint16_t* kvc = reinterpret_cast<uint16_t*>(base + pl.vec_bytes());
  uint16_t* lmc = reinterpret_cast<uint16_t*>(base + pl.vec_bytes() + pl.kv_bytes());
  const int job = item % njobs + (a.lm_only ? KVJ : 0);

  if (job < KVJ) {
    // FJ features f0.. x D values: thread -> (feature pair, 4 consecutive d).
    // Partials are loaded 8 splits at a time and added in split order.
    const int f0 = job * FJ;
    const size_t stride = (size_t)F * D + F;
    const float* p0 = a.part + (size_t)bh * a.nsplit * stride;
    for (int u = tid; u < (FJ / 2) * (D / 4); u += 256) {
      const int fp = u / (D / 4), d0 = (u % (D / 4)) * 4, f = f0 + 2 * fp;
      f32x4 s0 = f32x4{}, s1 = f32x4{};
      for (int s = 0; s < a.nsplit; s += 8) {
        f32x4 v0[8], v1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int sk = min(s + k, a.nsplit - 1);
          v0[k] = *reinterpret_cast<const f32x4*>(p0 + sk * stride + (size_t)f * D + d0);
          v1[k] = *reinterpret_cast<const f32x4*>(p0 + sk * stride + (size_t)(f + 1) * D + d0);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (s + k < a.nsplit) {
            s0 += v0[k];
            s1 += v1[k];
          }
      }
      // KV^T chunk f / 64, column q = (f & 32) + kperm(f & 31); f even so q + 1 holds f + 1
      uint16_t* ch = kvc + (size_t)(f / 64) * 64 * D;
      const int q = (f & 32) + kperm(f & 31);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = d0 + j;
        *reinterpret_cast<uint32_t*>(ch + toff<64, kRowRead>(d, q)) = pack_bf16x2(s0[j], s1[j]);
      }
    }
    if (tid < FJ) {
      const int f = f0 + tid;
      float s = 0.f;
      for (int sp = 0; sp < a.nsplit; sp += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = p0[min(sp + k, a.nsplit - 1) * stride + (size_t)F * D + f];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (sp + k < a.nsplit) s += v[k];
      }
      ksumP[kperm(f)] = s;
      biasP[kperm(f)] = a.bias ? a.bias[(size_t)h * F + f] : 0.f;
    }
    return;
  }
  const int jb = job - KVJ;  // landmark chunk of 32
  if (jb >= nlb) return;
  const uint16_t* K = a.K + (size_t)bh * a.N * D;
  const uint16_t* V = a.V + (size_t)bh * a.N * D;
  uint16_t* kl = lmc + (size_t)jb * pl.chunk_elems();
  uint16_t* vl = kl + 32 * D;
  // K_L [32 j][D] straight to the chunk; V_L rows through LDS so that V_L^T
  // [D][32 j] (landmark jl in column kperm(jl)) is written in 16-byte pieces.
  // Landmarks past L are zero.
  __shared__ uint16_t vrows[32][D + 8];
  for (int u = tid; u < 2 * 32 * (D / 8); u += 256) {
    const int isv = u >= 32 * (D / 8);
    const int uu = u - isv * 32 * (D / 8);
    const int jl = uu / (D / 8), d0 = (uu % (D / 8)) * 8, j = jb * 32 + jl;
    const uint16_t* src = isv ? V : K;
    const Vec8<uint16_t> v =
        j < a.L ? ld8(src + (size_t)(((long long)j * a.N) / a.L) * D + d0) : zero8<uint16_t>();
    if (isv) *reinterpret_cast<Vec8<uint16_t>*>(&vrows[jl][d0]) = v;
    else st8(kl + toff<D, kRowRead>(jl, d0), v);
  }
  __syncthreads();
  for (int u = tid; u < D * 4; u += 256) {  // piece (row d, columns 8q .. 8q + 7)
    const int d = u / 4, q = u % 4;
    Vec8<uint16_t> v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v.v[e] = vrows[kperm(8 * q + e)][d];  // kperm is its own inverse
    st8(vl + toff32(d, 8 * q), v);
  }
}

// ---------------------------------------------------------------- host side
static void kv2_plan(const Problem& p, int* nsplit, int* chunk) {
  const int step = 32 * (8 / (p.F / 32));
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

static PackLayout pack_layout(const Problem& p, int L) {
  PackLayout pl{p.D, p.F, L, (L + 31) / 32};
  return pl;
}

size_t fused_workspace_bytes(const Problem& p, int L) {
  int ns, ch;
  kv2_plan(p, &ns, &ch);
  const PackLayout pl = pack_layout(p, L);
  return (size_t)p.B * p.H * ns * (size_t)(p.F * p.D + p.F) * 4 + (size_t)p.B * p.H * pl.bh_bytes() +
         (size_t)p.H * pl.w_bytes();
}

template <int D, int F, bool PROJ, int MAP>
static hipError_t launch_kv2_t(const Problem& p, const Kv2Args& ka, const PackArgs& pa, hipStream_t s,
                               StageTimer* t) {
  hipLaunchKernelGGL((kv2_partial_kernel<D, F, PROJ, MAP>), dim3(ka.nsplit * p.B * p.H), dim3(512), 0, s, ka);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  t->mark();
  constexpr int FJ = 2048 / D > F ? F : 2048 / D;
  const int jobs = F / FJ + (pa.L + 31) / 32;
  hipLaunchKernelGGL((kv2_pack_kernel<D, F, PROJ>), dim3(jobs * p.B * p.H), dim3(256), 0, s, pa);
  e = hipGetLastError();
  t->mark();
  return e;
}

hipError_t launch_kv2(const Problem& p, const void* K, const void* V, const void* W, const float* bias, int L,
                      void* ws, FusedPack* pk, hipStream_t s, StageTimer* t) {
  int nsplit, chunk;
  kv2_plan(p, &nsplit, &chunk);
  const PackLayout pl = pack_layout(p, L);
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  float* part = reinterpret_cast<float*>(w8);
  unsigned char* pbh = w8 + (size_t)p.B * p.H * nsplit * (size_t)(p.F * p.D + p.F) * 4;
  unsigned char* pw = pbh + (size_t)p.B * p.H * pl.bh_bytes();
  pk->pack_bh = pbh;
  pk->pack_w = pw;
  pk->bh_bytes = pl.bh_bytes();
  pk->w_bytes = pl.w_bytes();

  Kv2Args ka;
  ka.K = static_cast<const uint16_t*>(K);
  ka.V = static_cast<const uint16_t*>(V);
  ka.W = static_cast<const uint16_t*>(W);
  ka.bias = bias;
  ka.H = p.H;
  ka.N = p.N;
  ka.chunk = chunk;
  ka.nsplit = nsplit;
  ka.part = part;
  ka.pack_w = pw;
  PackArgs pa;
  pa.part = part;
  pa.nsplit = nsplit;
  pa.K = ka.K;
  pa.V = ka.V;
  pa.W = ka.W;
  pa.bias = bias;
  pa.H = p.H;
  pa.N = p.N;
  pa.L = L;
  pa.pack_bh = pbh;
  pa.pack_w = pw;
  pa.lm_only = 0;
  if (p.dtype != 1) return hipErrorInvalidValue;
  if (p.D == 128) {
    if (p.proj) return launch_kv2_t<128, 256, true, kElu1>(p, ka, pa, s, t);
    if (p.fmap == kRelu) return launch_kv2_t<128, 128, false, kRelu>(p, ka, pa, s, t);
    if (p.fmap == kSoftmax) return launch_kv2_t<128, 128, false, kSoftmax>(p, ka, pa, s, t);
    return launch_kv2_t<128, 128, false, kElu1>(p, ka, pa, s, t);
  }
  if (p.D == 64) {
    if (p.proj) return launch_kv2_t<64, 256, true, kElu1>(p, ka, pa, s, t);
    if (p.fmap == kRelu) return launch_kv2_t<64, 64, false, kRelu>(p, ka, pa, s, t);
    if (p.fmap == kSoftmax) return launch_kv2_t<64, 64, false, kSoftmax>(p, ka, pa, s, t);
    return launch_kv2_t<64, 64, false, kElu1>(p, ka, pa, s, t);
  }
  return hipErrorInvalidValue;
}

// The key/value reduction on its own (ttr_kv_reduce, bf16 IO): the partial
// kernel into the workspace, then the fixed-order sum of the split partials into
// fp32 KV [F][D] and ksum [F] (the partials' own layout). Workspace: the
// partials, then room for the W^T chunks the partial kernel also writes.
size_t kv2_reduce_workspace_bytes(const Problem& p) {
  int ns, ch;
  kv2_plan(p, &ns, &ch);
  return (size_t)p.B * p.H * ns * (size_t)(p.F * p.D + p.F) * 4 + (size_t)p.H * p.F * p.D * 2;
}

template <int D, int F, bool PROJ, int MAP>
static void launch_kv2_partial_t(const Problem& p, const Kv2Args& ka, hipStream_t s) {
  hipLaunchKernelGGL((kv2_partial_kernel<D, F, PROJ, MAP>), dim3(ka.nsplit * p.B * p.H), dim3(512), 0, s, ka);
}

hipError_t launch_kv2_reduce(const Problem& p, const void* K, const void* V, const void* W, const float* bias,
                             float* KV, float* ksum, void* ws, hipStream_t s) {
  if (p.dtype != 1 || (p.D != 64 && p.D != 128)) return hipErrorInvalidValue;
  int nsplit, chunk;
  kv2_plan(p, &nsplit, &chunk);
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  Kv2Args ka;
  ka.K = static_cast<const uint16_t*>(K);
  ka.V = static_cast<const uint16_t*>(V);
  ka.W = static_cast<const uint16_t*>(W);
  ka.bias = bias;
  ka.H = p.H;
  ka.N = p.N;
  ka.chunk = chunk;
  ka.nsplit = nsplit;
  ka.part = reinterpret_cast<float*>(w8);
  ka.pack_w = w8 + (size_t)p.B * p.H * nsplit * (size_t)(p.F * p.D + p.F) * 4;
  if (p.D == 128) {
    if (p.proj) launch_kv2_partial_t<128, 256, true, kElu1>(p, ka, s);
    else if (p.fmap == kRelu) launch_kv2_partial_t<128, 128, false, kRelu>(p, ka, s);
    else if (p.fmap == kSoftmax) launch_kv2_partial_t<128, 128, false, kSoftmax>(p, ka, s);
    else launch_kv2_partial_t<128, 128, false, kElu1>(p, ka, s);
  } else {
    if (p.proj) launch_kv2_partial_t<64, 256, true, kElu1>(p, ka, s);
    else if (p.fmap == kRelu) launch_kv2_partial_t<64, 64, false, kRelu>(p, ka, s);
    else if (p.fmap == kSoftmax) launch_kv2_partial_t<64, 64, false, kSoftmax>(p, ka, s);
    else launch_kv2_partial_t<64, 64, false, kElu1>(p, ka, s);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_kv_finalize(p, ka.part, nsplit, KV, ksum, s);
}

// Every key j < L of a landmark pack alone (the chunks of the softmax-only query
// kernel): K_L and V_L^T chunks per (batch, head), nothing else.
size_t lm_pack_bytes(const Problem& p, int L) {
  const PackLayout pl{p.D, 0, L, (L + 31) / 32};
  return (size_t)p.B * p.H * pl.bh_bytes();
}

hipError_t launch_lm_pack(const Problem& p, const void* K, const void* V, int L, void* ws, FusedPack* pk,
                          hipStream_t s) {
  if (p.dtype != 1 || L < 1 || (p.D != 64 && p.D != 128)) return hipErrorInvalidValue;
  const PackLayout pl{p.D, 0, L, (L + 31) / 32};
  PackArgs pa{};
  pa.K = static_cast<const uint16_t*>(K);
  pa.V = static_cast<const uint16_t*>(V);
  pa.H = p.H;
  pa.N = p.N;
  pa.L = L;
  pa.pack_bh = static_cast<unsigned char*>(ws);
  pa.lm_only = 1;
  pk->pack_bh = pa.pack_bh;
  pk->pack_w = nullptr;
  pk->bh_bytes = pl.bh_bytes();
  pk->w_bytes = 0;
  const dim3 grid((unsigned)(pl.nlb * p.B * p.H));
  // (the landmark jobs do not depend on the feature count: any instantiation serves)
  if (p.D == 128) hipLaunchKernelGGL((kv2_pack_kernel<128, 256, true>), grid, dim3(256), 0, s, pa);
  else hipLaunchKernelGGL((kv2_pack_kernel<64, 256, true>), grid, dim3(256), 0, s, pa);
  return hipGetLastError();
}

}  // namespace ttr

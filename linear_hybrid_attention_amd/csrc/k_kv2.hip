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
//   K and V tiles are copied global -> LDS asynchronously into a 4-step
//   ring: three steps are in flight while one is consumed; one barrier per
//   step.
//
// kv2_pack_kernel: adds the split partials in split order (deterministic) and
// writes the operands of the fused query kernel as bf16 "chunks" that are
// exact images of its LDS tiles (swizzled, feature order matched to the MFMA
// register layout), so that kernel stages them with straight 16-byte copies:
//   per head h:         W^T chunks  [64 f][D]        (F / 64 of them)
//   per (batch, head):  bias, ksum  [F] fp32 each, in kperm order
//                       KV^T chunks [D][64 f]        (F / 64)
//                       per 32 landmarks: K_L [32 j][D], V_L [32 j][D]
//   with landmarks idx_j = floor(j N / L) ("Flux2TTRTrainer", section "How the
//   distillation works": exact softmax over strided landmark tokens).
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace ttr {

// ---------------------------------------------------------------- pack layout
// Every chunk holds 64 * D bf16 elements:
//   W^T chunk   [64 f][D]   kRowRead      KV^T chunk [D][64 f]   kRowRead
//   landmark chunk: K_L [32 j][D] kRowRead, then V_L [32 j][D] kTrRead
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
  float* part;  // [BH][nsplit][F*D + F]
};

template <int D, int F>
struct Kv2Shape {
  static constexpr int NW = 8;
  static constexpr int NFS = F / 32;
  static constexpr int NTW = NW / NFS;
  static constexpr int STEP = 32 * NTW;
  static constexpr int NS = 4;                   // ring depth (steps)
  static constexpr int TILE = STEP * D;          // elements of the K (or V) tile of one step
  static constexpr int SLOT = 2 * TILE;          // K tile, then V tile
  static constexpr int PER_T = SLOT * 2 / 16 / 512;  // 16-byte pieces per thread per step
  static_assert(PER_T * 512 * 16 == SLOT * 2, "whole pieces");
  using WR = LdsRow<uint16_t, D>;                // W^T [F][D] staging (prologue)
  static constexpr int w_bytes = F * WR::bytes_per_row;
  static constexpr int ring_bytes = NS * SLOT * 2;
  static constexpr int red_floats = (D / 32) * 16 * 64 + 64;  // one wave's KV slice + ksum
  static constexpr int r_bytes = (NTW - 1) * NFS * red_floats * 4;
  static constexpr int m1 = w_bytes > ring_bytes ? w_bytes : ring_bytes;
  static constexpr int bytes = m1 > r_bytes ? m1 : r_bytes;
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

template <int D, int F, bool PROJ>
__global__ __launch_bounds__(512, 1) void kv2_partial_kernel(Kv2Args a) {
  using S = Kv2Shape<D, F>;
  constexpr int NFS = S::NFS, NTW = S::NTW, STEP = S::STEP, NS = S::NS, PER_T = S::PER_T;
  using WR = typename S::WR;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::bytes];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int split = blockIdx.x, bh = blockIdx.y, h = bh % a.H;
  const int fs = w % NFS, tw = w / NFS, f0 = 32 * fs;
  const int N = a.N;
  const int t_begin = split * a.chunk;
  const int t_end = min(N, t_begin + a.chunk);

  // W slice as B operand (lane = feature column f0 + c, k = D), via a transposed LDS image.
  Frag<uint16_t> wf[D / 16];
  {
    uint16_t* Wt = reinterpret_cast<uint16_t*>(smem);
    if constexpr (PROJ) {
      const uint16_t* W = a.W + (size_t)h * D * F;
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
    __syncthreads();  // the region becomes the step ring
  }
  const float bcol = a.bias ? a.bias[(size_t)h * F + f0 + c] : 0.f;
  wait_vmcnt<0>();  // bias is in a register before the asynchronous copies start

  const uint16_t* K = a.K + (size_t)bh * N * D;
  const uint16_t* V = a.V + (size_t)bh * N * D;
  uint16_t* const ring = reinterpret_cast<uint16_t*>(smem);

  // Async copy of step st into its ring slot. Piece P of the slot (16 bytes)
  // is row (P % TILE8) / (D/8) of the K (P < TILE8) or V tile at physical
  // piece p = P % (D/8), i.e. logical piece p ^ swizzle(row). Rows past the
  // range repeat the last valid token: their phi is masked to zero below, so
  // they add nothing.
  constexpr int TILE8 = S::TILE / 8;
  auto issue_step = [&](int st) {
    const int t_step = t_begin + st * STEP;
    uint16_t* slot = ring + (st % NS) * S::SLOT;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int P = tid + 512 * i;
      const int isv = P >= TILE8;
      const int Pl = P - isv * TILE8;
      const int row = Pl / (D / 8), p = Pl % (D / 8);
      const int lp = isv ? (p ^ tswz<D, kTrRead>(row)) : (p ^ tswz<D, kRowRead>(row));
      const int t = min(t_step + row, t_end - 1);
      const uint16_t* src = (isv ? V : K) + (size_t)t * D + lp * 8;
      copy16_async(src, slot + (512 * i + 64 * w) * 8);
    }
  };

  f32x16 kv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) kv[db] = f32x16{};
  float ks = 0.f;

  const int nsteps = (t_end - t_begin + STEP - 1) / STEP;
  for (int st = 0; st < NS - 1 && st < nsteps; ++st) issue_step(st);
  for (int st = 0; st < nsteps; ++st) {
    // this wave's pieces of step st have landed once at most (later issued steps) x PER_T remain
    const int later = min(NS - 2, nsteps - 1 - st);
    if (later >= 2) wait_vmcnt<2 * PER_T>();
    else if (later == 1) wait_vmcnt<PER_T>();
    else wait_vmcnt<0>();
    barrier_lds();  // step st visible to all waves; all waves are done with step st - 1
    if (st + NS - 1 < nsteps) issue_step(st + NS - 1);

    const uint16_t* kt = ring + (st % NS) * S::SLOT;
    const uint16_t* vt = kt + S::TILE;
    const int t0 = t_begin + st * STEP + 32 * tw;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = bcol;
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
      mma(acc, ld_frag<uint16_t>(kt + toff<D, kRowRead>(32 * tw + c, kb * 16 + 8 * g)), wf[kb]);
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = t0 + crow(lane, r) < t_end ? elu1(acc[r]) : 0.f;
      ks += p[r];
    }
    const Frag<uint16_t> pa0 = to_frag<uint16_t>(p), pa1 = to_frag<uint16_t>(p + 8);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      mma(kv[db], pa0, tr_frag<D>(vt, 32 * tw, 32 * db, lane));
      mma(kv[db], pa1, tr_frag<D>(vt, 32 * tw + 16, 32 * db, lane));
    }
  }
  ks += shfl_xor32(ks);
  __syncthreads();  // ring no longer read

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
};

// Jobs of one (batch, head), by blockIdx.x:
//   [0, F/8)            KV^T rows: 8 features x D (sum of partials), ksum, bias
//   [F/8, F/8 + F/8)    W^T rows for 8 features (batch 0 only)
//   then one per 32-landmark chunk (K_L and V_L^T)
template <int D, int F, bool PROJ>
__global__ __launch_bounds__(256) void kv2_pack_kernel(PackArgs a) {
  const int tid = threadIdx.x;
  const int bh = blockIdx.y, h = bh % a.H, b = bh / a.H;
  const int nlb = (a.L + 31) / 32;
  PackLayout pl{D, F, a.L, nlb};
  unsigned char* base = a.pack_bh + (size_t)bh * pl.bh_bytes();
  float* biasP = reinterpret_cast<float*>(base);
  float* ksumP = biasP + F;
  uint16_t* kvc = reinterpret_cast<uint16_t*>(base + pl.vec_bytes());
  uint16_t* lmc = reinterpret_cast<uint16_t*>(base + pl.vec_bytes() + pl.kv_bytes());
  const int job = blockIdx.x;

  if (job < F / 8) {
    // 8 features f0..f0+7 x D values: thread -> (feature pair, 4 consecutive d)
    const int f0 = job * 8;
    const size_t stride = (size_t)F * D + F;
    const float* p0 = a.part + (size_t)bh * a.nsplit * stride;
    for (int u = tid; u < 4 * (D / 4); u += 256) {
      const int fp = u / (D / 4), d0 = (u % (D / 4)) * 4, f = f0 + 2 * fp;
      f32x4 s0 = *reinterpret_cast<const f32x4*>(p0 + (size_t)f * D + d0);
      f32x4 s1 = *reinterpret_cast<const f32x4*>(p0 + (size_t)(f + 1) * D + d0);
      for (int s = 1; s < a.nsplit; ++s) {
        s0 += *reinterpret_cast<const f32x4*>(p0 + s * stride + (size_t)f * D + d0);
        s1 += *reinterpret_cast<const f32x4*>(p0 + s * stride + (size_t)(f + 1) * D + d0);
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
    if (tid < 8) {
      const int f = f0 + tid;
      float s = p0[(size_t)F * D + f];
      for (int sp = 1; sp < a.nsplit; ++sp) s += p0[sp * stride + (size_t)F * D + f];
      ksumP[kperm(f)] = s;
      biasP[kperm(f)] = a.bias ? a.bias[(size_t)h * F + f] : 0.f;
    }
    return;
  }
  if (job < F / 4) {
    if (b != 0) return;  // W^T is per head
    const int f0 = (job - F / 8) * 8;
    uint16_t* wc = reinterpret_cast<uint16_t*>(a.pack_w + (size_t)h * pl.w_bytes());
    for (int u = tid; u < 8 * (D / 8); u += 256) {
      const int f = f0 + u / (D / 8), d0 = (u % (D / 8)) * 8;
      Vec8<uint16_t> v;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (PROJ) v.v[j] = a.W[((size_t)h * D + d0 + j) * F + f];
        else v.v[j] = (d0 + j == f) ? (uint16_t)0x3f80 : (uint16_t)0;
      }
      uint16_t* ch = wc + (size_t)(f / 64) * 64 * D;
      st8(ch + toff<D, kRowRead>(f & 63, d0), v);
    }
    return;
  }
  const int jb = job - F / 4;  // landmark chunk of 32
  if (jb >= nlb) return;
  const uint16_t* K = a.K + (size_t)bh * a.N * D;
  const uint16_t* V = a.V + (size_t)bh * a.N * D;
  uint16_t* kl = lmc + (size_t)jb * pl.chunk_elems();
  uint16_t* vl = kl + 32 * D;
  // K_L [32 j][D] (row reads) and V_L [32 j][D] (transposed reads); rows past L are zero
  for (int u = tid; u < 2 * 32 * (D / 8); u += 256) {
    const int isv = u >= 32 * (D / 8);
    const int uu = u - isv * 32 * (D / 8);
    const int jl = uu / (D / 8), d0 = (uu % (D / 8)) * 8, j = jb * 32 + jl;
    const uint16_t* src = isv ? V : K;
    const Vec8<uint16_t> v =
        j < a.L ? ld8(src + (size_t)(((long long)j * a.N) / a.L) * D + d0) : zero8<uint16_t>();
    if (isv) st8(vl + toff<D, kTrRead>(jl, d0), v);
    else st8(kl + toff<D, kRowRead>(jl, d0), v);
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

template <int D, int F, bool PROJ>
static hipError_t launch_kv2_t(const Problem& p, const Kv2Args& ka, const PackArgs& pa, hipStream_t s,
                               StageTimer* t) {
  hipLaunchKernelGGL((kv2_partial_kernel<D, F, PROJ>), dim3(ka.nsplit, p.B * p.H), dim3(512), 0, s, ka);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  t->mark();
  const int jobs = F / 4 + (pa.L + 31) / 32;
  hipLaunchKernelGGL((kv2_pack_kernel<D, F, PROJ>), dim3(jobs, p.B * p.H), dim3(256), 0, s, pa);
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
  if (p.dtype != 1) return hipErrorInvalidValue;
  if (p.D == 128) {
    if (p.proj) return launch_kv2_t<128, 256, true>(p, ka, pa, s, t);
    return launch_kv2_t<128, 128, false>(p, ka, pa, s, t);
  }
  if (p.D == 64) {
    if (p.proj) return launch_kv2_t<64, 256, true>(p, ka, pa, s, t);
    return launch_kv2_t<64, 64, false>(p, ka, pa, s, t);
  }
  return hipErrorInvalidValue;
}

}  // namespace ttr

// Projections of the NNT linear-attention layer ("NNT Define Linear
// Attention", section "How it works": project Q/K/V, run the linear attention,
// project back out; section "The inputs": embed_dim divides by num_heads,
// batch_first).
//
// proj_gemm_kernel: C = A . W + bias with fp32 accumulation, W given
// transposed (Wt [Nc][K], made by wt_transpose_kernel) so that both MFMA
// operands are row reads of LDS tiles:
//   C^T tile [128 n][128 m] = Wt tile . A^T tile  (A operand: Wt rows,
//                                                 B operand: A rows)
//   4 waves in a 2 x 2 grid, each 64 n x 64 m = 2 x 2 MFMA tiles.
//   Tiles of 128 rows x 128 bytes (64 bf16 or 32 fp32 of K) stream into a
//   two-slot LDS ring by buffer-resource LDS DMA, one K-step ahead.
// Row modes of A: kRows (x [M][K]) or kHeads (the attention output
// [B][H][N][D], row m = (b, t), column k = (h, d)). Column modes of C:
// kRows (out [M][Nc]) or kQkvHeads (Nc = 3E: columns (which, h, d) go to
// Q, K or V [B][H][N][D]).
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace ttr {

enum ProjAMode { kARows = 0, kAHeads = 1 };
enum ProjCMode { kCRows = 0, kCQkvHeads = 1 };

struct ProjArgs {
  const void* A;      // kARows: [M][K]; kAHeads: [B][H][Ntok][D]
  const void* Wt;     // [Nc][K]
  const float* bias[3];  // per output block of E columns (kCQkvHeads: q, k, v); [0] only for kCRows; each nullable
  void* out[3];       // kCRows: out[0] [M][Nc]; kCQkvHeads: Q, K, V [B][H][Ntok][D]
  int M, K, Nc, Ntok, H, D, E;
  int ntn, nwg;       // n-tiles, workgroups
  uint32_t a_bytes, w_bytes;
};

// 16-byte pieces per 128-byte tile row: 8; elements per piece
template <typename T> struct ProjTile {
  static constexpr int P = 16 / sizeof(T);  // elements per piece
  static constexpr int KT = 8 * P;          // K per step
  static constexpr int ELEMS = 128 * KT;    // per operand tile
  // element offset of (row, k) in a tile: kRowRead swizzle of 128-byte rows
  __device__ static int off(int row, int k) { return row * KT + ((((k / P) ^ ((row >> 1) & 7))) * P) + k % P; }
};

template <typename T>
__device__ __forceinline__ Frag<T> ld_tile_frag(const T* tile, int row, int k0);
template <>
__device__ __forceinline__ bf16x8 ld_tile_frag<uint16_t>(const uint16_t* tile, int row, int k0) {
  return ld_frag<uint16_t>(tile + ProjTile<uint16_t>::off(row, k0));
}
template <>
__device__ __forceinline__ f32x8 ld_tile_frag<float>(const float* tile, int row, int k0) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(tile + ProjTile<float>::off(row, k0));
  const f32x4 hi = *reinterpret_cast<const f32x4*>(tile + ProjTile<float>::off(row, k0 + 4));
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) { r[i] = lo[i]; r[4 + i] = hi[i]; }
  return r;
}

template <typename T, int AMODE, int CMODE>
__global__ __launch_bounds__(256, 2) void proj_gemm_kernel(ProjArgs a) {
  using TL = ProjTile<T>;
  constexpr int P = TL::P, KT = TL::KT, ELEMS = TL::ELEMS;
  // ring: 2 slots x (Wt tile, A tile); reused for the output tile [128 m][128 n]
  constexpr int RING = 2 * 2 * ELEMS * (int)sizeof(T);
  constexpr int OUTB = 128 * 128 * (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) unsigned char smem[RING > OUTB ? RING : OUTB];
  T* const ring = reinterpret_cast<T*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, c = lane & 31;
  const int wn = w & 1, wm = w >> 1;

  // XCD-aware numbering: consecutive tiles (one m band, every n tile) share an XCD's L2
  int wg = blockIdx.x;
  const int per = a.nwg / 8;
  if (wg < per * 8) wg = (wg % 8) * per + wg / 8;
  const int mt = wg / a.ntn, nt = wg % a.ntn;
  const int m0 = mt * 128, n0 = nt * 128;
  const int M = a.M, K = a.K;

  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a.A, a.a_bytes);
  const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.Wt, a.w_bytes);

  // Lane tid copies, for every K-step, the pieces at LDS positions tid + 256 i
  // of both tiles (i < 4): tile row r = pos / 8, stored piece s = pos % 8,
  // logical piece s ^ ((r >> 1) & 7). The byte offsets of the K-step-0 pieces
  // are computed once; a K-step adds KT elements.
  uint32_t offw[4], offa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pos = tid + 256 * i, r = pos / 8, kc = ((pos % 8) ^ ((r >> 1) & 7)) * P;
    offw[i] = (uint32_t)((size_t)(n0 + r) * K + kc) * sizeof(T);
    const int m = min(m0 + r, M - 1);  // rows past M repeat the last row; their results are not stored
    if constexpr (AMODE == kARows) {
      offa[i] = (uint32_t)((size_t)m * K + kc) * sizeof(T);
    } else {
      const int b = m / a.Ntok, t = m % a.Ntok;
      // column kc of K-step 0 lies in head 0; a K-step moves KT columns, which
      // stays inside one head (D is a multiple of KT)
      offa[i] = (uint32_t)(((size_t)b * a.H * a.Ntok + t) * a.D + kc) * sizeof(T);
    }
  }
  auto issue = [&](int ks) {
    T* wt_s = ring + (ks & 1) * 2 * ELEMS;
    T* a_s = wt_s + ELEMS;
    const int k0 = ks * KT;
    uint32_t adv;
    if constexpr (AMODE == kARows) {
      adv = (uint32_t)k0 * sizeof(T);
    } else {  // head h = k0 / D, column k0 % D of that head
      adv = (uint32_t)(((size_t)(k0 / a.D) * a.Ntok * a.D + k0 % a.D) * sizeof(T));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      copy16_async(rw, offw[i], (uint32_t)k0 * sizeof(T), wt_s + (256 * i + 64 * w) * P);
      copy16_async(ra, offa[i], adv, a_s + (256 * i + 64 * w) * P);
    }
  };

  // C^T accumulators: [n tile j][m tile i], started from the bias of each n row
  const int ob = CMODE == kCQkvHeads ? n0 / a.E : 0;
  const float* bias = a.bias[ob];
  const int nb_in = n0 - ob * a.E;  // bias index of the tile's first column
  f32x16 acc[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    f32x16 bj;
#pragma unroll
    for (int r = 0; r < 16; ++r) bj[r] = bias ? bias[nb_in + wn * 64 + j * 32 + crow(lane, r)] : 0.f;
    acc[j][0] = bj;
    acc[j][1] = bj;
  }

  const int nks = K / KT;
  issue(0);
  for (int ks = 0; ks < nks; ++ks) {
    wait_vmcnt<0>();
    barrier_lds();  // step ks is in LDS; every wave is done with the other slot
    if (ks + 1 < nks) issue(ks + 1);  // workgroup-uniform
    const T* wt_s = ring + (ks & 1) * 2 * ELEMS;
    const T* a_s = wt_s + ELEMS;
    // Fixed order: four MFMA slots per k-block (Wt tile j, A tile i); each
    // slot also reads one of the next k-block's four operands, so the LDS
    // latency overlaps the matrix core.
    constexpr int NKB = KT / 16;
    auto ld = [&](int kb, int q) {  // q 0, 1: Wt tiles; 2, 3: A tiles
      return q < 2 ? ld_tile_frag<T>(wt_s, wn * 64 + q * 32 + c, kb * 16 + 8 * g)
                   : ld_tile_frag<T>(a_s, wm * 64 + (q - 2) * 32 + c, kb * 16 + 8 * g);
    };
    Frag<T> f[NKB][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) f[0][q] = ld(0, q);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        if (kb + 1 < NKB) f[kb + 1][sl] = ld(kb + 1, sl);
        mma(acc[sl >> 1][sl & 1], f[kb][sl >> 1], f[kb][2 + (sl & 1)]);
        __builtin_amdgcn_sched_barrier(0);
      }
  }
  barrier_lds();  // the ring becomes the output tile

  // Output tile [128 m][128 n] in T, 256-byte rows (bf16) or 512-byte rows
  // (fp32), 16-byte pieces swizzled by (row & 15). Lane (c, g) holds, per MFMA
  // tile, token m = c and columns crow(lane, r): four consecutive per group.
  T* ot = reinterpret_cast<T*>(smem);
  constexpr int OP = 128 / P;  // pieces per output row
  auto ooff = [&](int m, int n) { return m * 128 + (((n / P) ^ (m & 15)) * P) + n % P; };
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = wm * 64 + i * 32 + c, n = wn * 64 + j * 32 + 8 * q + 4 * g;
        T* p = ot + ooff(m, n);
        if constexpr (sizeof(T) == 2) {
          uint2 v;
          v.x = pack_bf16x2(acc[j][i][4 * q], acc[j][i][4 * q + 1]);
          v.y = pack_bf16x2(acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]);
          *reinterpret_cast<uint2*>(p) = v;
        } else {
          *reinterpret_cast<f32x4*>(p) =
              f32x4{acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]};
        }
      }
  barrier_lds();
  // 128 rows x OP pieces; rows past M are not stored
  for (int u = tid; u < 128 * OP; u += 256) {
    const int mr = u / OP, pc = u % OP, m = m0 + mr;
    if (m >= M) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ot + ooff(mr, pc * P));
    const int n = n0 + pc * P;
    T* dst;
    if constexpr (CMODE == kCRows) {
      dst = static_cast<T*>(a.out[0]) + (size_t)m * a.Nc + n;
    } else {
      const int which = n / a.E, e = n % a.E, h = e / a.D, d = e % a.D;
      const int b = m / a.Ntok, t = m % a.Ntok;
      dst = static_cast<T*>(a.out[which]) + (((size_t)b * a.H + h) * a.Ntok + t) * a.D + d;
    }
    *reinterpret_cast<u32x4*>(dst) = v;
  }
}

// Wt[n][k] = W[k][n] for up to four [E x E] matrices (blockIdx.z), 64 x 64
// tiles through LDS, 16-byte loads and stores.
struct TransposeArgs {
  const void* W[4];
  void* Wt[4];
  int E;
};

template <typename T>
__global__ __launch_bounds__(256) void wt_transpose_kernel(TransposeArgs a) {
  constexpr int P = 16 / sizeof(T);  // elements per 16-byte piece
  __shared__ T tile[64][64 + 1];
  const int z = blockIdx.z, E = a.E;
  const T* W = static_cast<const T*>(a.W[z]);
  T* Wt = static_cast<T*>(a.Wt[z]);
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int u = threadIdx.x; u < 64 * (64 / P); u += 256) {
    const int r = u / (64 / P), pc = (u % (64 / P)) * P;
    const u32x4 v = *reinterpret_cast<const u32x4*>(W + (size_t)(r0 + r) * E + c0 + pc);
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int j = 0; j < P; ++j) tile[r][pc + j] = e[j];
  }
  __syncthreads();
  for (int u = threadIdx.x; u < 64 * (64 / P); u += 256) {
    const int cc = u / (64 / P), pr = (u % (64 / P)) * P;  // output row c0 + cc, columns r0 + pr ..
    u32x4 v;
    T* e = reinterpret_cast<T*>(&v);
#pragma unroll
    for (int j = 0; j < P; ++j) e[j] = tile[pr + j][cc];
    *reinterpret_cast<u32x4*>(Wt + (size_t)(c0 + cc) * E + r0 + pr) = v;
  }
}

// ---------------------------------------------------------------- host side
template <typename T, int AMODE, int CMODE>
static hipError_t launch_proj_t(ProjArgs a, hipStream_t s) {
  hipLaunchKernelGGL((proj_gemm_kernel<T, AMODE, CMODE>), dim3(a.nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_wt_transpose(int dtype, const void* const* W, void* const* Wt, int nmat, int E, hipStream_t s) {
  TransposeArgs a;
  for (int i = 0; i < 4; ++i) {
    a.W[i] = i < nmat ? W[i] : nullptr;
    a.Wt[i] = i < nmat ? Wt[i] : nullptr;
  }
  a.E = E;
  const dim3 grid(E / 64, E / 64, nmat);
  if (dtype == 1) hipLaunchKernelGGL((wt_transpose_kernel<uint16_t>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((wt_transpose_kernel<float>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// out = A . W + bias for the layer's shapes (E % 128 == 0, D % 64 == 0). See ProjArgs.
hipError_t launch_proj_gemm(int dtype, bool a_heads, bool c_qkv, const void* A, const void* Wt,
                            const float* const* bias, void* const* out, int M, int K, int Nc, int Ntok, int H,
                            int D, int E, hipStream_t s) {
  ProjArgs a;
  a.A = A;
  a.Wt = Wt;
  for (int i = 0; i < 3; ++i) {
    a.bias[i] = bias[i];
    a.out[i] = out[i];
  }
  a.M = M;
  a.K = K;
  a.Nc = Nc;
  a.Ntok = Ntok;
  a.H = H;
  a.D = D;
  a.E = E;
  a.ntn = Nc / 128;
  a.nwg = ((M + 127) / 128) * a.ntn;
  const size_t es = dtype == 1 ? 2 : 4;
  a.a_bytes = (uint32_t)((size_t)M * K * es);
  a.w_bytes = (uint32_t)((size_t)Nc * K * es);
  if (dtype == 1) {
    if (a_heads) return launch_proj_t<uint16_t, kAHeads, kCRows>(a, s);
    return c_qkv ? launch_proj_t<uint16_t, kARows, kCQkvHeads>(a, s) : launch_proj_t<uint16_t, kARows, kCRows>(a, s);
  }
  if (a_heads) return launch_proj_t<float, kAHeads, kCRows>(a, s);
  return c_qkv ? launch_proj_t<float, kARows, kCQkvHeads>(a, s) : launch_proj_t<float, kARows, kCRows>(a, s);
}

}  // namespace ttr

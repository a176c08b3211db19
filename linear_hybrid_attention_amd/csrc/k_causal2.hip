// Causal elu+1 linear attention, bf16 with D = 64: chunked prefix scan with
// register-staged chunk prefetch. Same computation and segment structure as
// the generic kernels in k_causal.hip ("NNT Define Linear Attention", sections
// "The inputs" (causal, elu(x) + 1, eps) and "How it works"):
//   chunk c:  num = tril(phi(Q_c) phi(K_c)^T) V_c + phi(Q_c) P,
//             den = rowsum(tril(.)) + phi(Q_c) . z,  out = num / (den + eps),
//             P += phi(K_c)^T V_c,  z += colsum(phi(K_c))
// What differs from the generic kernels (all about keeping HBM busy):
//  * the K and V rows of chunk c + 2 are loaded into registers while chunk c
//    is processed; chunk c + 1 is written to LDS at the end of chunk c, with
//    phi applied to K on the way, so one K/V buffer and two barriers per
//    chunk suffice and two workgroups fit on a CU at C = 128;
//  * phi(K) and V are read as transposed MFMA operands with
//    ds_read_b64_tr_b16 (no transposed copies). These reads are not mixed
//    with asynchronous global->LDS copies: the compiler waits for every such
//    copy in flight before a transposed read, which would serialise the
//    prefetch;
//  * the next chunk's query rows are loaded during the current chunk;
//  * each wave's 32 x 64 output block goes through LDS so the global stores
//    are whole 16-byte pieces.
// One launch (after a one-workgroup reset of its flags): each workgroup sums
// its segment's state, takes the inclusive prefix of the segment before from
// the workgroup that had it (a chained scan over segments, waits bounded),
// publishes its own, then walks the segment (causal1_kernel below).
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"
#include "validate.hpp"

namespace ttr {

struct Causal2Args {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const float* bias;  // [H][64] or NULL
  float eps;
  int H, N, cps, nseg, nbh;
  float* seg;        // [BH][nseg][64*64 + 64]: inclusive prefixes P^T (row d, column f), then z
  unsigned* flags;   // [BH][nseg]: prefix published (zero on entry, causal1_reset_kernel)
  unsigned* ticket;  // next segment to take (zero on entry)
  unsigned* err;     // set when a wait gave up (zero on entry)
  unsigned spin_limit;
  uint16_t* sink;  // CAUSAL2_SINK_BYTES of workspace that absorb the stores of rows past N
  uint16_t* out;
};

template <int C, bool WALK>
struct Causal2Shape {
  static constexpr int D = 64;
  // waves: four own the 32 x 32 tiles of the state P^T; at C = 256 four more
  // take query blocks, so that every wave holds one block (two waves per SIMD)
  static constexpr int NW = C == 256 ? 8 : 4;
  static constexpr int NT = 64 * NW;
  static constexpr int TILE = C * D;               // elements of the K (or V) tile
  static constexpr int PER_T = 2 * TILE / 8 / NT;  // 16-byte pieces per thread per chunk (K then V)
  static_assert(PER_T * NT * 8 == 2 * TILE && (TILE / 8) % NT == 0, "whole pieces, K/V split per piece index");
  // phi(K) is read transposed by the state update and, in the walk, also as
  // rows by the score product: the walk keeps it twice, once per swizzle.
  static constexpr int nk = WALK ? 2 : 1;
  static constexpr int kv_bytes = (nk + 1) * TILE * 2;
  static constexpr int pt_bytes = WALK ? D * D * 2 : 0;  // P^T as MFMA operand, [d][f] kRowRead
  static constexpr int zb_bytes = 2 * D * 4;             // z, then the bias (zeros without one)
  static constexpr int NB = C / 32;                // 32-token blocks per chunk
  static constexpr int QB = (NB + NW - 1) / NW;    // query blocks per wave
  static constexpr int o_bytes = WALK ? NW * QB * 32 * D * 2 : 0;  // per-wave output staging
  static constexpr int bytes = kv_bytes + pt_bytes + zb_bytes + o_bytes;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static constexpr int WG_PER_CU = (160 * 1024) / bytes >= 2 ? 2 : 1;
};

// Chunks [cbeg, cend) of (batch, head) bh. WALK = false: the segment's
// state only (P and zr summed from the values they hold on entry); WALK = true:
// the outputs, starting from the state P, zr of the tokens before the
// segment. smem is laid out for the walk (the state pass uses its first two tiles).
template <int C, bool WALK, int MAP>
__device__ __forceinline__ void causal_segment(const Causal2Args& a, unsigned char* smem, int bh, int cbeg, int cend,
                                               f32x16& P, float& zr) {
  using S = Causal2Shape<C, true>;
  constexpr int D = 64, NB = S::NB, QB = S::QB, PER_T = S::PER_T, NW = S::NW, NT = S::NT;
  uint16_t* ktt = reinterpret_cast<uint16_t*>(smem);  // phi(K) rows, kTrRead (state update)
  uint16_t* vt = ktt + S::TILE;                        // V rows, kTrRead
  uint16_t* kt = vt + S::TILE;                         // phi(K) rows, kRowRead (walk: scores)
  float* zS = reinterpret_cast<float*>(smem + S::kv_bytes + S::pt_bytes);
  float* bS = zS + D;
  uint16_t* Pt = reinterpret_cast<uint16_t*>(smem + S::kv_bytes);
  uint16_t* ostage = reinterpret_cast<uint16_t*>(smem + S::kv_bytes + S::pt_bytes + S::zb_bytes);

  const int h = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);  // wave-uniform, kept in a scalar register
  const bool owner = w < 4;  // owns a tile of the state
  const int N = a.N;
  const size_t base = (size_t)bh * N * D;
  const uint16_t* Qg = a.Q + base;
  const uint16_t* Kg = a.K + base;
  const uint16_t* Vg = a.V + base;

  const Frag<uint16_t> ones = __builtin_bit_cast(Frag<uint16_t>, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  // P^T tile owned by waves 0-3: rows dt*32.., columns ft*32.. (dt = w >> 1, ft = w & 1).
  const int dt = (w >> 1) & 1, ft = w & 1;
  // (zr: z[ft*32 + c]; the waves with dt == 0 write it to LDS)
  // A thread's K pieces are all logical piece tid % 8 of their rows: 8 fixed columns.
  const int kcol = (tid & 7) * 8;
  float kb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kb[j] = a.bias ? a.bias[(size_t)h * D + kcol + j] : 0.f;
  if (tid < D) bS[tid] = a.bias ? a.bias[(size_t)h * D + tid] : 0.f;

  // K/V staging: piece i of thread tid is piece tid + NT i of the chunk
  // (K pieces first); rows past N repeat row N - 1 and are zeroed (K) when
  // stored, so they contribute nothing.
  u32x4 stg[PER_T];
  auto load_stg = [&](int ch) {
    [[maybe_unused]] const int c0 = ch * C;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const bool isv = i >= PER_T / 2;
      const int Pl = tid + NT * (isv ? i - PER_T / 2 : i);
      const int row = Pl / (D / 8), p = Pl % (D / 8);
      const int t = min(c0 + row, N - 1);
      stg[i] = *reinterpret_cast<const u32x4*>((isv ? Vg : Kg) + (size_t)t * D + p * 8);
    }
  };
  auto store_stg = [&](int ch) {
    [[maybe_unused]] const int c0 = ch * C;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const bool isv = i >= PER_T / 2;
      const int Pl = tid + NT * (isv ? i - PER_T / 2 : i);
      const int row = Pl / (D / 8), p = Pl % (D / 8);
      if (isv) {
        *reinterpret_cast<u32x4*>(vt + toff<D, kTrRead>(row, p * 8)) = stg[i];
      } else {
        const float keep = c0 + row < N ? 1.f : 0.f;
        Vec8<uint16_t> v = __builtin_bit_cast(Vec8<uint16_t>, stg[i]);
        float z[8], m = 0.f, inv = 1.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = bf2f(v.v[j]) + kb[j];
        if constexpr (MAP == kSoftmax) softmax_stats<8, 7>(z, m, inv);  // a row's 8 pieces: 8 consecutive lanes
#pragma unroll
        for (int j = 0; j < 8; ++j) v.v[j] = f2bf(phi_of<MAP>(z[j], m, inv) * keep);
        *reinterpret_cast<u32x4*>(ktt + toff<D, kTrRead>(row, p * 8)) = __builtin_bit_cast(u32x4, v);
        if constexpr (WALK) *reinterpret_cast<u32x4*>(kt + toff<D, kRowRead>(row, p * 8)) = __builtin_bit_cast(u32x4, v);
      }
    }
  };
  auto write_state = [&]() {
    if (!owner) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) Pt[toff<D, kRowRead>(dt * 32 + crow(lane, r), ft * 32 + c)] = f2bf(P[r]);
    if (dt == 0 && g == 0) zS[ft * 32 + c] = zr;
  };

  // Raw query fragments (B operand: column = token, k = feature) of this
  // wave's query blocks of chunk ch.
  Frag<uint16_t> qraw[QB][D / 16];
  auto load_q = [&](int ch) {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      const int qb = (i & 1) ? (NW * i + NW - 1 - w) : (NW * i + w);
      // Rows past N repeat row N - 1 and blocks past the chunk (waves without
      // a block when C = 64) load the last block: their outputs are not stored.
      const int q = min(ch * C + min(qb, NB - 1) * 32 + c, N - 1);
#pragma unroll
      for (int kb2 = 0; kb2 < D / 16; ++kb2) qraw[i][kb2] = ld_frag<uint16_t>(Qg + (size_t)q * D + kb2 * 16 + 8 * g);
    }
  };

  // Every iteration issues the same global loads and stores whatever the
  // chunk (indexes are clamped, rows past N are stored to the sink): with no
  // data-dependent branch around them the compiler's count of memory
  // operations in flight is exact, and each wait below covers only what it
  // needs (the prologue issues the same sequence as an iteration).
  auto store_out = [&](int ch) {
    wave_lds_order();
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      const int qb = (i & 1) ? (NW * i + NW - 1 - w) : (NW * i + w);
      const uint16_t* ot = ostage + (w * QB + i) * 32 * D;
      const int t0 = max(ch, 0) * C + qb * 32;
      uint16_t* og = a.out + base + (size_t)t0 * D;
#pragma unroll
      for (int k = 0; k < 32 * D / 8 / 64; ++k) {
        const int P8 = 64 * k + lane;
        const int row = P8 / (D / 8), pc = P8 % (D / 8);
        const u32x4 v = *reinterpret_cast<const u32x4*>(ot + toff<D, kRowRead>(row, pc * 8));
        const bool ok = qb < NB && ch >= 0 && t0 + row < N;
        // one sink slot per store, so that none of them is merged away
        uint16_t* sk = a.sink + ((i * (32 * D / 8 / 64) + k) * 64 + lane) * 8;
        // nontemporal: the output streams past the caches (it is not read
        // again here), leaving the L2 and the last-level cache to the K and
        // V rows that the walk reads a second time
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(ok ? og + (size_t)row * D + pc * 8 : sk));
      }
    }
  };

  load_stg(cbeg);
  if constexpr (WALK) {
    write_state();
    load_q(cbeg);
  }
  store_stg(cbeg);
  load_stg(min(cbeg + 1, cend - 1));
  if constexpr (WALK) store_out(-1);  // sink only (stands in for the previous chunk's stores)

  for (int ch = cbeg; ch < cend; ++ch) {
    [[maybe_unused]] const int c0 = ch * C;
    barrier_lds();  // chunk ch (phi(K), V), P^T and z are in LDS

    // phi(Q) fragments of this wave's query blocks and their inter-chunk
    // normaliser phi(q) . z; the raw rows are then free for the next chunk's
    // (no register copy, which would have to wait for the loads).
    Frag<uint16_t> qf[QB][D / 16];
    float den0[QB];
    if constexpr (WALK) {
#pragma unroll
      for (int i = 0; i < QB; ++i) {
        den0[i] = 0.f;
        float zq[D / 16][8], m = 0.f, inv = 1.f;
#pragma unroll
        for (int kb2 = 0; kb2 < D / 16; ++kb2) {
          frag_to_f32(qraw[i][kb2], zq[kb2]);
#pragma unroll
          for (int j = 0; j < 8; ++j) zq[kb2][j] += bS[kb2 * 16 + 8 * g + j];
        }
        // the query's features: half in this lane, half in lane ^ 32
        if constexpr (MAP == kSoftmax) softmax_stats<D / 2, 32>(&zq[0][0], m, inv);
#pragma unroll
        for (int kb2 = 0; kb2 < D / 16; ++kb2) {
          float v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = phi_of<MAP>(zq[kb2][j], m, inv);
          qf[i][kb2] = to_frag<uint16_t>(v);
#pragma unroll
          for (int j = 0; j < 8; ++j) den0[i] += v[j] * zS[kb2 * 16 + 8 * g + j];
        }
      }
      load_q(min(ch + 1, cend - 1));
    }

    // Next state: P^T[dt block][ft block] += V^T phi(K) over the chunk and
    // z += column sums of phi(K) (here an MFMA against an all-ones operand:
    // every row of Z holds the sums), in registers (the LDS copy is updated after
    // every wave has read the current one).
    // (The walk, short of registers, sums z on the VALU instead.)
    if (!owner) {
      // (no state tile: waves 4-7 at C = 256)
    } else if constexpr (!WALK) {
      f32x16 Z = f32x16{};
#pragma unroll
      for (int kk = 0; kk < C / 16; ++kk) {
        const Frag<uint16_t> av = tr_frag<D>(vt, kk * 16, dt * 32, lane);
        const Frag<uint16_t> bk = tr_frag<D>(ktt, kk * 16, ft * 32, lane);
        mma(P, av, bk);
        mma(Z, ones, bk);
      }
      zr += Z[0];
    } else {
      float zp = 0.f;
#pragma unroll
      for (int kk = 0; kk < C / 16; ++kk) {
        const Frag<uint16_t> av = tr_frag<D>(vt, kk * 16, dt * 32, lane);
        const Frag<uint16_t> bk = tr_frag<D>(ktt, kk * 16, ft * 32, lane);
        float bv[8];
        frag_to_f32(bk, bv);
#pragma unroll
        for (int j = 0; j < 8; ++j) zp += bv[j];
        mma(P, av, bk);
      }
      zr += zp + shfl_xor32(zp);
    }

    if constexpr (WALK) {
#pragma unroll
      for (int i = 0; i < QB; ++i) {
        const int qb = (i & 1) ? (NW * i + NW - 1 - w) : (NW * i + w);
        if (qb >= NB) continue;  // wave-uniform (C = 64 only)
        float den = den0[i];
        f32x16 num[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          num[db] = f32x16{};
#pragma unroll
          for (int kb2 = 0; kb2 < D / 16; ++kb2)
            mma(num[db], ld_frag<uint16_t>(Pt + toff<D, kRowRead>(db * 32 + c, kb2 * 16 + 8 * g)), qf[i][kb2]);
        }
        // score blocks: kb < qb whole, then the diagonal block kb == qb with
        // the keys after the query masked. The normaliser sums the fp32
        // scores (the products use their bf16 rounding).
        auto score_block = [&](int kb, bool diag) {
          f32x16 sc = f32x16{};
#pragma unroll
          for (int kb2 = 0; kb2 < D / 16; ++kb2)
            mma(sc, ld_frag<uint16_t>(kt + toff<D, kRowRead>(kb * 32 + c, kb2 * 16 + 8 * g)), qf[i][kb2]);
          if (diag) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[r] = crow(lane, r) > c ? 0.f : sc[r];
          }
          float sv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            sv[r] = sc[r];
            den += sv[r];
          }
          const Frag<uint16_t> sb0 = to_frag<uint16_t>(sv), sb1 = to_frag<uint16_t>(sv + 8);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            mma(num[db], tr_frag<D>(vt, kb * 32, db * 32, lane), sb0);
            mma(num[db], tr_frag<D>(vt, kb * 32 + 16, db * 32, lane), sb1);
          }
        };
#pragma unroll
        for (int kb = 0; kb < NB - 1; ++kb) {
          if (kb >= qb) break;  // wave-uniform
          score_block(kb, false);
        }
        score_block(qb, true);
        den += shfl_xor32(den);
        const float inv = 1.f / (den + a.eps);
        // 32 x 64 output block -> this wave's LDS staging (swizzled rows)
        uint16_t* ot = ostage + (w * QB + i) * 32 * D;
        wave_lds_order();  // the previous chunk's reads of ot are done
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            st4(ot + toff<D, kRowRead>(c, db * 32 + 8 * qq + 4 * g), num[db][4 * qq] * inv,
                num[db][4 * qq + 1] * inv, num[db][4 * qq + 2] * inv, num[db][4 * qq + 3] * inv);
      }
    }
    barrier_lds();  // every wave is done reading chunk ch, P^T and z
    if constexpr (WALK) write_state();
    store_stg(min(ch + 1, cend - 1));
    load_stg(min(ch + 2, cend - 1));
    // Global stores after the staging loads are issued: the wait for the
    // staged chunk in the next iteration never covers these stores.
    if constexpr (WALK) store_out(ch);
  }

}


// Single pass: workgroups take segments in the order of an atomic ticket
// (ticket t: segment t / BH of (batch, head) t % BH), sum the segment's
// state, wait for the inclusive prefix of the segment before (published by a
// workgroup with a smaller ticket, so one that is already running), publish
// their own inclusive prefix (the one before plus this segment's, in that
// order: the result is the same whatever the timing), then walk the segment.
// Prefixes are written and read with agent-coherent accesses; a wait that
// exceeds spin_limit polls sets *err and makes the outputs NaN.
template <int C, int MAP>
__global__ __launch_bounds__((Causal2Shape<C, true>::NT), (Causal2Shape<C, true>::WG_PER_CU)) void causal1_kernel(Causal2Args a) {
  constexpr int D = 64, E = D * D + D;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Causal2Shape<C, true>::bytes];
  __shared__ unsigned tk_s, ok_s;
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), dt = (w >> 1) & 1, ft = w & 1;
  const bool owner = w < 4;  // the waves that hold a tile of the state
  if (tid == 0) tk_s = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int t = (int)tk_s;
  const int s = t / a.nbh, bh = t % a.nbh;
  const int nchunks = (a.N + C - 1) / C;
  const int cbeg = s * a.cps, cend = min(nchunks, cbeg + a.cps);  // non-empty by the plan
  const bool last = s == a.nseg - 1;  // no segment reads its prefix

  f32x16 PA = f32x16{};
  float zA = 0.f;
  if (!last) {
    causal_segment<C, false, MAP>(a, smem, bh, cbeg, cend, PA, zA);
    __syncthreads();  // LDS free for the walk
  }
  f32x16 P = f32x16{};
  float zr = 0.f;
  if (s > 0) {
    if (tid == 0) {
      const unsigned* fl = a.flags + (size_t)bh * a.nseg + (s - 1);
      unsigned n = 0;
      while (__hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u && ++n < a.spin_limit)
        __builtin_amdgcn_s_sleep(2);
      ok_s = n < a.spin_limit;
      if (!ok_s) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const float* ip = a.seg + ((size_t)bh * a.nseg + (s - 1)) * E;
    const bool ok = ok_s != 0;
    if (owner) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      P[r] = ok ? __hip_atomic_load(ip + (dt * 32 + crow(lane, r)) * D + ft * 32 + c, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT)
                : __uint_as_float(0x7fc00000u);
    zr = ok ? __hip_atomic_load(ip + D * D + ft * 32 + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
            : __uint_as_float(0x7fc00000u);
    }
  }
  if (!last) {
    float* op = a.seg + ((size_t)bh * a.nseg + s) * E;
    if (owner) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      __hip_atomic_store(op + (dt * 32 + crow(lane, r)) * D + ft * 32 + c, P[r] + PA[r], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    if (dt == 0 && lane < 32)
      __hip_atomic_store(op + D * D + ft * 32 + c, zr + zA, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vmcnt<0>();  // the prefix is at the agent's coherence point before its flag
    __syncthreads();
    if (tid == 0) __hip_atomic_store(a.flags + (size_t)bh * a.nseg + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  causal_segment<C, true, MAP>(a, smem, bh, cbeg, cend, P, zr);
}

__global__ void causal1_reset_kernel(unsigned* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) __hip_atomic_store(p + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int C, int MAP>
static hipError_t launch_causal2_t(const Causal2Args& a, int B, hipStream_t s, StageTimer* t) {
  hipLaunchKernelGGL(causal1_reset_kernel, dim3(1), dim3(256), 0, s, a.flags, a.nbh * a.nseg + 2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  t->mark();
  hipLaunchKernelGGL((causal1_kernel<C, MAP>), dim3(a.nseg * a.nbh), dim3(Causal2Shape<C, true>::NT), 0, s, a);
  e = hipGetLastError();
  t->mark();
  return e;
}

// Segments of the single pass: about 1024 tokens each (so the K and V rows a
// segment reads twice are still in the last-level cache the second time),
// shorter when that gives fewer than 512 workgroups; every segment non-empty.
void causal1_plan(const Problem& p, int chunk, int* nseg, int* cps) {
  const int nchunks = (p.N + chunk - 1) / chunk;
  const int bh = p.B * p.H;
  int want = (p.N + 1023) / 1024;
  const int fill = (512 + bh - 1) / bh;
  if (want < fill) want = fill;
  if (want > nchunks) want = nchunks;
  if (want < 1) want = 1;
  *cps = (nchunks + want - 1) / want;
  *nseg = (nchunks + *cps - 1) / *cps;
}

// Workspace: prefixes [BH][nseg][D D + D] fp32 | flags [BH][nseg], ticket, err
// (256-byte aligned) | the store sink.
static size_t causal1_prefix_bytes(const Problem& p, int nseg) {
  return (size_t)p.B * p.H * nseg * (size_t)(64 * 64 + 64) * sizeof(float);
}
static size_t causal1_flag_bytes(const Problem& p, int nseg) {
  return ((size_t)p.B * p.H * nseg * 4 + 8 + 255) / 256 * 256;
}
size_t causal1_workspace_bytes(const Problem& p, int chunk) {
  int nseg, cps;
  causal1_plan(p, chunk, &nseg, &cps);
  return causal1_prefix_bytes(p, nseg) + causal1_flag_bytes(p, nseg) + CAUSAL2_SINK_BYTES;
}

bool causal2_supported(const Problem& p, int chunk) {
  return p.dtype == 1 && p.D == 64 && (chunk == 64 || chunk == 128 || chunk == 256);
}

template <int MAP>
static hipError_t launch_causal2_m(const Causal2Args& a, int B, int chunk, hipStream_t s, StageTimer* t) {
  if (chunk == 64) return launch_causal2_t<64, MAP>(a, B, s, t);
  if (chunk == 128) return launch_causal2_t<128, MAP>(a, B, s, t);
  if (chunk == 256) return launch_causal2_t<256, MAP>(a, B, s, t);
  return hipErrorInvalidValue;
}

hipError_t launch_causal2(const Problem& p, const void* Q, const void* K, const void* V, const float* bias,
                          float eps, int chunk, void* out, void* ws, hipStream_t s, StageTimer* t) {
  Causal2Args a;
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.bias = bias;
  a.eps = eps;
  a.H = p.H;
  a.N = p.N;
  causal1_plan(p, chunk, &a.nseg, &a.cps);
  a.nbh = p.B * p.H;
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  a.seg = reinterpret_cast<float*>(w8);
  a.flags = reinterpret_cast<unsigned*>(w8 + causal1_prefix_bytes(p, a.nseg));
  a.ticket = a.flags + (size_t)a.nbh * a.nseg;
  a.err = a.ticket + 1;
  a.spin_limit = env_spin_limit(1u << 20);  // a tenth of a second or so of polling
  a.sink = reinterpret_cast<uint16_t*>(w8 + causal1_prefix_bytes(p, a.nseg) + causal1_flag_bytes(p, a.nseg));
  static_assert(CAUSAL2_SINK_BYTES >= 2 * 4 * 64 * 16, "one 16-byte slot per store of a wave (QB <= 2)");
  a.out = static_cast<uint16_t*>(out);
  if (p.fmap == kRelu) return launch_causal2_m<kRelu>(a, p.B, chunk, s, t);
  if (p.fmap == kSoftmax) return launch_causal2_m<kSoftmax>(a, p.B, chunk, s, t);
  return launch_causal2_m<kElu1>(a, p.B, chunk, s, t);
}

}  // namespace ttr

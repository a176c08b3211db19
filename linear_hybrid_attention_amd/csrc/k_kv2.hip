// bf16 hot path, stage 1: the key/value reduction and the per-head operand
// pack of the fused query kernel, in one launch.
//
// KV = phi(K)^T V and ksum = sum over tokens of phi(K), per (batch, head)
// ("NNT Define Linear Attention", section "How it works": K'^T V first,
// sum(K') for the normaliser; phi(x) = elu(x W_h + b_h) + 1 per
// "Flux2TTRTrainer", section "Inputs worth setting", and the elu(x) + 1 map of
// the linear-attention page, section "The inputs").
//
// kv_stage_kernel. A workgroup owns FG = min(F, 128) features of one (batch,
// head) and one token range ("split"); its four waves (one per SIMD, up to
// 512 registers each) own 64 features each, the group's features covered by
// NFW = FG / 64 waves and the tokens of a step by the NTG = 4 / NFW token
// groups of 32. Per step a wave computes, for its 32 tokens:
//   phi[tok x 64]  = map(K[tok x D] . W[:, 64 features] + b)   (A = K rows read from
//                     LDS, B = W held in registers)
//   KV[64 x D]    += phi^T . V                                  (A = phi^T from LDS,
//                     B = V read transposed from LDS)
// The K and V rows of a step reach LDS by asynchronous copies (global -> LDS,
// whole 128-byte lines per 16 lanes, pieces placed in the swizzled layout the
// operand reads want), issued two steps ahead by the waves that map, into
// three-slot rings. The waves of the second product issue no copies: the
// compiler makes transposing LDS reads wait for every copy the reading wave
// has in flight.
//
// The splits of a (batch, head, feature group) then meet: each writes its
// fp32 partial (its waves' token groups added through LDS first), counts
// itself in at the group's counter and waits for the others (a bounded spin;
// every workgroup of the launch is resident, the grid is at most one
// workgroup per compute unit), and each reduces a share of the group's
// outputs over the splits in split order -- deterministic -- straight into
// the fused query kernel's pack (bf16 KV^T chunks, ksum and bias) or into
// fp32 KV and ksum. The grid is numbered so that the splits of a group run on
// one XCD: their partials then stay in that XCD's L2 (plain stores and loads,
// no trip to memory before the reduction). Each workgroup counts itself in
// under its XCD's id; a group found spread over several XCDs takes a second
// round in which every split first writes its L2 back to memory and then
// drops stale lines, so the result never depends on where the hardware put
// the workgroups.
//
// The pack, per (batch, head): bias (b + 1 for the elu + 1 map, which then
// takes x = z + b + 1 straight from the products), ksum [F] fp32 in kperm order; F / 64
// KV^T chunks [D][64 f]; one K_L + V_L^T chunk per 32 landmarks
// idx_j = floor(j N / L) ("Flux2TTRTrainer", section "How the distillation
// works": exact softmax over strided landmark tokens); per head the W^T
// chunks [64 f][D]. Every chunk is an exact image of the query kernel's LDS
// tile (swizzled, features in MFMA C-row order).
//
// lm_pack_kernel: the landmark chunks alone (every key a landmark for the
// distillation's teacher, or the student's landmark branch).
#include <atomic>
#include <chrono>
#include <random>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"
#include "validate.hpp"

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

// Work item of workgroup i in a one-dimensional grid of n: the hardware places
// workgroup i on XCD i % 8, so items are renumbered such that consecutive ones
// (the splits or jobs of one (batch, head)) run on one XCD.
__device__ __forceinline__ int xcd_item(int i, int n) {
  const int per = n / 8;
  return i < per * 8 ? (i % 8) * per + i / 8 : i;
}

// Landmark chunk jb of one (batch, head): K_L [32 j][D] straight to the chunk,
// V_L rows through LDS (vrows, 32 x (D + 8) bf16) so that V_L^T [D][32 j]
// (landmark jl in column kperm(jl)) is written in 16-byte pieces. Landmarks
// past L are zero. All 256 threads of the workgroup take part.
template <int D, int NT>
__device__ __forceinline__ void landmark_chunk(const uint16_t* K, const uint16_t* V, int N, int L, int jb,
                                               uint16_t* kl, uint16_t (*vrows)[D + 8], int tid) {
  uint16_t* vl = kl + 32 * D;
  for (int u = tid; u < 2 * 32 * (D / 8); u += NT) {
    const int isv = u >= 32 * (D / 8);
    const int uu = u - isv * 32 * (D / 8);
    const int jl = uu / (D / 8), d0 = (uu % (D / 8)) * 8, j = jb * 32 + jl;
    const uint16_t* src = isv ? V : K;
    const Vec8<uint16_t> v = j < L ? ld8(src + (size_t)(((long long)j * N) / L) * D + d0) : zero8<uint16_t>();
    if (isv) *reinterpret_cast<Vec8<uint16_t>*>(&vrows[jl][d0]) = v;
    else st8(kl + toff<D, kRowRead>(jl, d0), v);
  }
  barrier_lds();
  for (int u = tid; u < D * 4; u += NT) {  // piece (row d, columns 8q .. 8q + 7)
    const int d = u / 4, q = u % 4;
    Vec8<uint16_t> v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v.v[e] = vrows[kperm(8 * q + e)][d];  // kperm is its own inverse
    st8(vl + toff32(d, 8 * q), v);
  }
  barrier_lds();
}

// ---------------------------------------------------------------- key/value stage
struct KvsArgs {
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* W;  // [H][D][F] or NULL (identity)
  const float* bias;  // [H][F] or NULL
  int H, N, L;
  int nsplit, chunk;     // token splits of a group and the tokens of each (a multiple of the step)
  int groups, per_xcd;   // (batch, head, feature group) groups; grid slots per XCD (grid = 8 per_xcd)
  float* part;           // [groups][nsplit][FG * D + FG] fp32 partials
  unsigned long long* counters;  // [groups][4] meeting words: arrivals, second round, departures, unused
  unsigned long long call;        // this launch's number (45 bits, never 0), which tags the meeting words
  unsigned spin_limit;   // polls of a waiting workgroup before it gives up
  unsigned force_round2;  // take the cross-XCD round whatever the placement (a test hook)
  unsigned char* pack_bh;  // pack mode: [BH][bh_bytes]
  unsigned long long bh_bytes;
  unsigned char* pack_w;   // pack mode: [H][F D bf16] W^T chunks (written by batch 0)
  float* kv_out;           // fp32 mode: KV [BH][F][D]
  float* ks_out;           // fp32 mode: ksum [BH][F]
};

template <int D, int F>
struct KvsShape {
  static constexpr int FG = F < 128 ? F : 128;  // features of a workgroup
  static constexpr int NG = F / FG;             // feature groups of a head
  static constexpr int NPW = FG / 64;           // producer (and consumer) waves across the group's features
  static constexpr int NTG = 4 / NPW;           // token groups of 32 per step
  static constexpr int STEP = 32 * NTG;         // tokens of a workgroup step
  static constexpr int NKB = D / 16;            // k-blocks of a K row
  static constexpr int NDB = D / 32;            // 32-column blocks of V
  static constexpr int NI = STEP * D / 8 / 64 / 4;  // copies (16 bytes per lane) per producer wave per tile
  static constexpr int PART = FG * D + FG;       // floats of one split's partial
  static_assert(F == 64 || F % 128 == 0, "feature count");
  static_assert(NI * 4 * 64 * 8 == STEP * D && NI >= 1, "whole copies");
  // consumer wave: features fs, CW_DB of the NDB 32-column blocks of V (part
  // dp of NDP), CW_TG of the NTG token groups (part tp of NTP)
  static constexpr int CW_DB = FG == 128 ? NDB / 2 : 1;
  static constexpr int NDP = NDB / CW_DB;
  static constexpr int NTP = 4 / NPW / NDP;
  static constexpr int CW_TG = NTG / NTP;
  static_assert(NPW * NDP * NTP == 4 && CW_TG * NTP == NTG && CW_DB * NDP == NDB, "consumer split");
  static_assert(NTG > 1, "both roles take the same barriers after the loop");
  static constexpr int tile_elems = STEP * D;                // one step of K (or V) rows, one ring slot
  static constexpr int pbuf_bytes = 3 * 4 * 64 * 32 * 2;     // phi^T ring [3][4 producers][64 f][32 tok]
  static constexpr int wtile_bytes = D * FG * 2;             // W tile (prologue)
  static constexpr int stats_bytes = 4 * 3 * 32 * 8;         // softmax (max, 1 / sum) per producer and ring slot
  static constexpr int lm_bytes = 32 * (D + 8) * 2;          // landmark V rows (prologue)
  static constexpr int CIMG = 2 * CW_DB * 16 * 64;           // floats of a consumer wave's accumulators
  static constexpr int KSOFF = (NTP - 1) * NPW * NDP * CIMG;  // producer ksum sums after the consumer images
  static constexpr int red_bytes = (KSOFF + (NTG - 1) * NPW * 64) * 4;
  static constexpr int max2(int x, int y) { return x > y ? x : y; }
  static constexpr int bytes = max2(max2(pbuf_bytes + stats_bytes, wtile_bytes), max2(lm_bytes, red_bytes));
  static_assert(bytes + 6 * tile_elems * 2 <= 160 * 1024, "LDS budget");
};

// (a quiet NaN by its bits: the file is built without NaN semantics)
#define kQNaN __uint_as_float(0x7fc00000u)

// Partial loads and stores through the XCD's L2 (see the meeting of the
// splits for when that is coherent). The stores are system-scope (sc0 sc1):
// the L2 writes them through to memory while the kernel runs, so no partial
// is still dirty in L2 when the kernel ends and the end-of-kernel write-back
// covers only the pack (about 1 us less between this kernel and the query
// kernel at flux_1024, where the partials are 15.7 MB).
__device__ __forceinline__ u32x4 ld16_part(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ void st16_part(__amdgpu_buffer_rsrc_t r, uint32_t off, const u32x4& v) {
  constexpr int kSc0Sc1 = 1 | 16;  // cache-policy bits: sc0 (1), sc1 (16)
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kSc0Sc1);
}

// Id of the XCD the calling wave runs on (hardware register XCC_ID, bits 0-3;
// gfx950 parts have at most eight XCDs).
__device__ __forceinline__ unsigned xcd_id() { return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 7u; }

// Meeting words of a group (arrivals, second round, departures): bits 0-7
// count the splits, bits 8-15 (arrivals) count those that run on another XCD
// than split 0, bits 16-18 (arrivals) hold split 0's XCD, bits 19-63 the
// number of the launch the word belongs to. Split 0 writes the three words
// afresh when it starts; the others add themselves to a word only once they
// have seen it carry this launch's number (a load and an atomic add on one
// location, so the add lands after split 0's write), so the words' contents
// on entry do not matter and no reset launch is needed. The last split to
// leave clears them, so a replay of a captured launch (the same number
// again) waits for split 0 as well.
constexpr int kMeetTag = 19;
__device__ __forceinline__ unsigned long long meet_load(const unsigned long long* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Polls w until it carries this launch's number (true) or the limit runs out;
// n counts the polls, v receives the word.
__device__ __forceinline__ bool meet_tagged(const unsigned long long* w, unsigned long long call, unsigned limit,
                                            unsigned& n, unsigned long long& v) {
  while (((v = meet_load(w)) >> kMeetTag) != call)
    if (++n >= limit) return false;
    else __builtin_amdgcn_s_sleep(2);
  return true;
}
// Polls w until its count reaches ns (true) or the limit runs out.
__device__ __forceinline__ bool meet_all(const unsigned long long* w, unsigned ns, unsigned limit, unsigned& n,
                                         unsigned long long& v) {
  while (((v = meet_load(w)) & 255u) < ns)
    if (++n >= limit) return false;
    else __builtin_amdgcn_s_sleep(2);
  return true;
}

// Eight waves, two per SIMD: waves 0-3 are producers, 4-7 consumers (wave w
// and w + 4 share a SIMD, so one's vector work runs beside the other's
// matrix products). Producer (fp, tg) computes, for the 32 tokens of token
// group tg of a step and its 64 features fp:
//   phi[tok x 64] = map(K[tok x D] . W[:, 64 features] + b)     (A = K rows straight
//                    from global memory into registers, B = W in registers)
// and writes phi^T [64 f][32 tok] to LDS; consumer (fc = fp, tg) accumulates
//   KV[64 x D] += phi^T . V                                       (A = phi^T from LDS,
//                    B = V read transposed from LDS)
// Iteration t: producers form the products of step t and map step t - 1,
// consumers take step t - 2; one barrier.
template <int D, int F, bool PROJ, int MAP, bool PACK>
__global__ __launch_bounds__(512, 1) void kv_stage_kernel(KvsArgs a) {
  using S = KvsShape<D, F>;
  constexpr int FG = S::FG, NG = S::NG, NPW = S::NPW, NTG = S::NTG, STEP = S::STEP, NKB = S::NKB,
                NDB = S::NDB, NI = S::NI;
  // Ring slots of K ([STEP][D] kRowRead) and V ([STEP][D] kTrRead), each its
  // own LDS object: the compiler then keeps a wave's LDS reads from waiting
  // on copies into other slots. smem: the phi^T ring and the softmax stats;
  // before the loop the W tile and landmark rows, after it the reductions.
  __shared__ __attribute__((aligned(16))) uint16_t kr0[S::tile_elems], kr1[S::tile_elems], kr2[S::tile_elems];
  __shared__ __attribute__((aligned(16))) uint16_t vr0[S::tile_elems], vr1[S::tile_elems], vr2[S::tile_elems];
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::bytes];
  uint16_t* const pbuf = reinterpret_cast<uint16_t*>(smem);                      // [3][4][64][32] toff32
  float2* const stats = reinterpret_cast<float2*>(smem + S::pbuf_bytes);
  uint16_t* const wt = reinterpret_cast<uint16_t*>(smem);                        // [D][FG], rows kperm'd
  auto lmrows = reinterpret_cast<uint16_t(*)[D + 8]>(smem);
  auto kslot = [&](auto sl) -> uint16_t* {
    if constexpr (decltype(sl)::value == 0) return kr0;
    else if constexpr (decltype(sl)::value == 1) return kr1;
    else return kr2;
  };
  auto vslot = [&](auto sl) -> uint16_t* {
    if constexpr (decltype(sl)::value == 0) return vr0;
    else if constexpr (decltype(sl)::value == 1) return vr1;
    else return vr2;
  };

  // (the wave index is read into a scalar register, so LDS copy destinations
  // derived from it are computed with scalar instructions)
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  const bool producer = w < 4;
  const int pw = w & 3;                   // index among the producers (or the consumers)
  const int fs = pw % NPW, tg = pw / NPW;  // feature slice, token group
  // Workgroup i runs on XCD i % 8 and takes slot i / 8 of that XCD's per_xcd
  // slots; the slots of one XCD hold whole groups (per_xcd is a multiple of
  // nsplit), so all splits of a group share an L2. Slots past the last group
  // have no work.
  const int item = (blockIdx.x & 7) * a.per_xcd + (blockIdx.x >> 3);
  if (item >= a.groups * a.nsplit) return;
  const int split = item % a.nsplit, group = item / a.nsplit;
  unsigned long long* const mw = a.counters + 4 * group;  // the group's meeting words
  if (split == 0 && tid == 0) {
    const unsigned long long t = a.call << kMeetTag;
    __hip_atomic_store(mw, t | ((unsigned long long)xcd_id() << 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(mw + 1, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(mw + 2, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int bh = group / NG, fgi = group % NG, h = bh % a.H;
  const int fg0 = fgi * FG;         // first feature of the group
  const int fs0 = fg0 + 64 * fs;    // first of this wave's 64 features
  const int N = a.N;
  const int t_begin = split * a.chunk;
  const int t_end = min(N, t_begin + a.chunk);
  const int nsteps = (t_end - t_begin + STEP - 1) / STEP;
  const uint16_t* Kp = a.K + (size_t)bh * N * D;
  const uint16_t* Vp = a.V + (size_t)bh * N * D;

  // ---- operand streams, through buffer resources that end at the range's
  // last token: a row past it reads as zeros (so it adds nothing to KV, and
  // a fixed phi(0 W + b) to ksum, taken out after the loop). Producer wave pw
  // copies pieces 64 (NI pw + i) + lane of a step's tile: row r = piece / (D / 8),
  // physical piece q' = piece % (D / 8), which holds the row's piece q' ^ tswz(r).
  const uint32_t range_bytes = (uint32_t)((size_t)t_end * D * 2);
  uint32_t koff[NI], voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int P = 64 * (NI * pw + i) + lane, r = P / (D / 8), qp = P % (D / 8);
    koff[i] = (uint32_t)(t_begin + r) * (D * 2) + (uint32_t)(qp ^ tswz<D, kRowRead>(r)) * 16;
    voff[i] = (uint32_t)(t_begin + r) * (D * 2) + (uint32_t)(qp ^ tswz<D, kTrRead>(r)) * 16;
  }
  // Step j goes to ring slot j % 3, given as a constant: LDS offsets the
  // compiler can see apart keep it from making the wave's LDS reads wait for
  // copies into other slots. Step j's copies go through a resource whose base
  // is moved j steps on and whose size shrinks by as much (never below zero),
  // built with scalar instructions: the lane offsets stay as they are, and
  // the bounds check still ends at the range's last token.
  auto step_rsrc = [&](const uint16_t* base, int j) {
    const uint32_t off = (uint32_t)__builtin_amdgcn_readfirstlane(j * STEP * D * 2);
    const uint32_t left = range_bytes > off ? range_bytes - off : 0u;
    return buffer_rsrc(reinterpret_cast<const unsigned char*>(base) + off, __builtin_amdgcn_readfirstlane(left));
  };
  auto copy_k = [&](int j, auto slot) {
    uint16_t* dst = kslot(slot);
    const __amdgpu_buffer_rsrc_t r = step_rsrc(Kp, j);
#pragma unroll
    for (int i = 0; i < NI; ++i) copy16_async(r, koff[i], 0, dst + (NI * pw + i) * 512);
  };
  auto copy_v = [&](int j, auto slot) {
    uint16_t* dst = vslot(slot);
    const __amdgpu_buffer_rsrc_t r = step_rsrc(Vp, j);
#pragma unroll
    for (int i = 0; i < NI; ++i) copy16_async(r, voff[i], 0, dst + (NI * pw + i) * 512);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  // K(0) and K(1) first: they land while the prologue runs
  if (producer) {
    copy_k(0, C0{});
    copy_k(1, C1{});
  }
  // ---- landmark chunks of this (batch, head), spread over its workgroups
  // (they need no partial: done first, beside the W loads)
  if constexpr (PACK) {
    const int nlb = (a.L + 31) / 32;
    if (nlb > 0) {
      const PackLayout pl{D, F, a.L, nlb};
      uint16_t* lmc = reinterpret_cast<uint16_t*>(a.pack_bh + (size_t)bh * a.bh_bytes + pl.vec_bytes() + pl.kv_bytes());
      const int nwg = NG * a.nsplit, me = fgi * a.nsplit + split;
      for (int jb = me; jb < nlb; jb += nwg)
        landmark_chunk<D, 512>(Kp, Vp, N, a.L, jb, lmc + (size_t)jb * pl.chunk_elems(), lmrows, tid);
    }
  }
  // ---- the group's W columns as a [D][FG] tile whose rows are permuted by
  // kperm within each block of 16, so that the transposing read (which hands
  // a lane its k-rows in C-row order) returns them in natural order, the
  // order of the K fragments
  if constexpr (PROJ) {
    const uint16_t* W = a.W + (size_t)h * D * F + fg0;
    constexpr int WP = D * FG / 8 / 512;
    static_assert(WP * 512 * 8 == D * FG, "whole W pieces");
    u32x4 wv[WP];
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int P = tid + 512 * i, d = P / (FG / 8), p = P % (FG / 8);
      wv[i] = *reinterpret_cast<const u32x4*>(W + (size_t)d * F + p * 8);
    }
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int P = tid + 512 * i, d = P / (FG / 8), p = P % (FG / 8);
      *reinterpret_cast<u32x4*>(wt + toff<FG, kTrRead>((d & ~15) | kperm(d & 15), p * 8)) = wv[i];
    }
    barrier_lds();
  }
  const size_t pstride = (size_t)S::PART * 4;
  const __amdgpu_buffer_rsrc_t rpart = buffer_rsrc(a.part + (size_t)group * a.nsplit * S::PART,
                                                   (uint32_t)(a.nsplit * pstride));
  float* red = reinterpret_cast<float*>(smem);
  // phi^T of a producer: [64 f][32 tok] in the toff32 layout, tokens of each
  // half in kperm column order, so that a consumer's plain 16-byte row read
  // hands it the tokens in the C-row order of the transposed V fragments
  auto ptile = [&](int slot, int p) -> uint16_t* { return pbuf + (slot * 4 + p) * 64 * 32; };
  // Both roles take nsteps + 2 loop barriers (the producers' iteration t
  // forms the products of step t and maps step t - 1, the consumers take
  // step t - 2), then the same barriers after the loop: their s_barrier
  // counts match. Each role's state lives in its own branch.
  unsigned long long pre = 0;  // (tid 0) the arrivals word, read early: split 0 wrote it at its start
  if (producer) {
    // ---- producer: W slice as the B operand (lane = feature fs0 + 32 fb + c,
    // k-slots = rows 16 kb + 8 g ..)
    Frag<uint16_t> wf[2][NKB];
    if constexpr (PROJ) {
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) wf[fb][kb] = tr_frag<FG>(wt, 16 * kb, 64 * fs + 32 * fb, lane);
    } else {
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int f = fs0 + 32 * fb + c;
          u32x4 u;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int d0 = 16 * kb + 8 * g + 2 * q;
            u[q] = (d0 == f ? 0x3f80u : 0u) | (d0 + 1 == f ? 0x3f800000u : 0u);  // bf16 1.0 on the diagonal
          }
          wf[fb][kb] = __builtin_bit_cast(bf16x8, u);
        }
    }
    // The fused query kernel's W^T chunks [64 f][D] (kRowRead) are per head:
    // batch 0's first split writes them, each producer lane the 16-byte row
    // pieces of the W slice it holds (the identity map too: the query kernel
    // multiplies by it to transpose Q).
    if constexpr (PACK) {
      if (split == 0 && bh < a.H && tg == 0) {
        uint16_t* wc = reinterpret_cast<uint16_t*>(a.pack_w + (size_t)h * F * D * 2) + (size_t)(fs0 / 64) * 64 * D;
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            *reinterpret_cast<u32x4*>(wc + toff<D, kRowRead>(32 * fb + c, 16 * kb + 8 * g)) =
                __builtin_bit_cast(u32x4, wf[fb][kb]);
      }
    }
    // The bias enters the product: the first MFMA of a step takes as its C
    // input a tile holding each lane's bias (lane = feature column), b + 1
    // for elu + 1, so the products come out as x = z + b + 1 and the map is
    // phi = max(x, min(exp2(x log2e - log2e), 1)) (three instructions: an
    // fma, the exponential with its clamp, a max; the relu and softmax maps
    // take x = z + b as it is).
    f32x16 bsplat[2];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) {
      const float bc = a.bias ? a.bias[(size_t)h * F + fs0 + 32 * fb + c] : 0.f;
      const float b1 = MAP == kElu1 ? bc + 1.f : bc;
#pragma unroll
      for (int r = 0; r < 16; ++r) bsplat[fb][r] = b1;
    }
    auto phi_b = [&](float x, float2 st) -> float {
      if constexpr (MAP == kElu1) {
        const float e = __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -kLog2e));
        return fmaxf(x, fminf(fmaxf(e, 0.f), 1.f));
      } else {
        return phi_of<MAP>(x, st.x, st.y);
      }
    };
    // softmax map (identity projection, F == D): each lane's bias values for
    // the columns its K fragments hold, for the token statistics
    float kbias[MAP == kSoftmax ? NKB * 8 : 1];
    if constexpr (MAP == kSoftmax) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) kbias[8 * kb + i] = a.bias ? a.bias[(size_t)h * F + 16 * kb + 8 * g + i] : 0.f;
    }
    float2* const wstats = stats + pw * 96;  // [3 slots][32 tokens]
    auto token_stats = [&](const Frag<uint16_t> (&kf)[NKB], int par) {
      if constexpr (MAP == kSoftmax) {
        float z[NKB * 8], m, inv;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          frag_to_f32(kf[kb], z + 8 * kb);
#pragma unroll
          for (int i = 0; i < 8; ++i) z[8 * kb + i] += kbias[8 * kb + i];
        }
        softmax_stats<NKB * 8, 32>(z, m, inv);
        if (g == 0) wstats[par * 32 + c] = float2{m, inv};
      }
    };
    float ks[2] = {0.f, 0.f};
    const uint32_t ones2 = 0x3f803f80u;  // bf16 (1, 1)
    // a step's first product: acc = K rows . W slice
    auto products = [&](const Frag<uint16_t> (&kf)[NKB], f32x16 (&acc)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int fb = 0; fb < 2; ++fb) acc[fb] = mma_from(bsplat[fb], kf[0], wf[fb][0]);
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb)
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) mma(acc[fb], kf[kb], wf[fb][kb]);
    };
    // the map of a step's products, phi^T into LDS slot `slot`, ksum from the
    // rounded pairs (two per v_dot2)
    auto map_store = [&](int slot, const f32x16 (&acc)[2]) __attribute__((always_inline)) {
      uint16_t* pt = ptile(slot, pw);
#pragma unroll
      for (int fb = 0; fb < 2; ++fb) {
        uint32_t u[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float2 s0 = float2{0.f, 1.f}, s1 = float2{0.f, 1.f};
          if constexpr (MAP == kSoftmax) {
            s0 = wstats[slot * 32 + crow(lane, 2 * i)];
            s1 = wstats[slot * 32 + crow(lane, 2 * i + 1)];
          }
          const bf16x2 pr = {(__bf16)phi_b(acc[fb][2 * i], s0), (__bf16)phi_b(acc[fb][2 * i + 1], s1)};
          ks[fb] = __builtin_amdgcn_fdot2_f32_bf16(pr, __builtin_bit_cast(bf16x2, ones2), ks[fb], false);
          u[i] = __builtin_bit_cast(uint32_t, pr);
        }
        // registers 0-7 are tokens kperm(8 g .. 8 g + 7), 8-15 kperm(16 + 8 g ..)
        const u32x4 lo = {u[0], u[1], u[2], u[3]}, hi = {u[4], u[5], u[6], u[7]};
        *reinterpret_cast<u32x4*>(pt + toff32(32 * fb + c, 8 * g)) = lo;
        *reinterpret_cast<u32x4*>(pt + toff32(32 * fb + c, 16 + 8 * g)) = hi;
      }
    };
    // Iteration t (0 .. nsteps) forms the products of step t (t < nsteps)
    // and, beside them, maps step t - 1 (t >= 1) from the products the
    // previous iteration left in acc, so the map no longer waits for its own
    // step's products. Copies: K(t + 2) into ring slot (t + 2) % 3 and V(t)
    // into slot t % 3 (the consumers take V(t - 2) from slot (t + 1) % 3).
    // At the start of iteration t this wave's copies of K(t) and V(t - 2)
    // have landed once at most the 2 NI copies of iteration t - 1 are in
    // flight (iteration 0: at most NI, K(1)); after the barrier everyone's
    // have, and phi^T slot (t - 1) % 3 is free (the consumers read step t - 4
    // there last, in iteration t - 2). Copies past the range read zeros.
    // (t % 3 == slot; kind 0: products only, 1: both, 2: the last map only)
    f32x16 acc[2];
    auto iteration = [&](int t, auto slot, auto waitn, auto kind) __attribute__((always_inline)) {
      constexpr int sl = decltype(slot)::value, KIND = decltype(kind)::value;
      wait_vmcnt<decltype(waitn)::value>();
      barrier_lds();
      // this wave's work first on the SIMD (the consumer wave beside it
      // fills the matrix core's gaps)
      __builtin_amdgcn_s_setprio(1);
      copy_k(t + 2, std::integral_constant<int, (sl + 2) % 3>{});
      copy_v(t, std::integral_constant<int, sl>{});
      f32x16 nacc[2];
      if constexpr (KIND != 2) {
        const uint16_t* kt = kslot(slot);
        Frag<uint16_t> kf[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) kf[kb] = ld_frag<uint16_t>(kt + toff<D, kRowRead>(32 * tg + c, 16 * kb + 8 * g));
        if constexpr (MAP == kSoftmax) {
          token_stats(kf, sl);
          wave_lds_order();
        }
        products(kf, nacc);
      }
      if constexpr (KIND != 0) map_store((sl + 2) % 3, acc);
      __builtin_amdgcn_s_setprio(0);
      if constexpr (KIND != 2) {
        acc[0] = nacc[0];
        acc[1] = nacc[1];
      }
    };
    using W1 = std::integral_constant<int, NI>;
    using W2 = std::integral_constant<int, 2 * NI>;
    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    using K2 = std::integral_constant<int, 2>;
    iteration(0, C0{}, W1{}, K0{});  // (every split has at least one step)
    int t3 = 1;
    for (; t3 + 3 <= nsteps; t3 += 3) {
      iteration(t3, C1{}, W2{}, K1{});
      iteration(t3 + 1, C2{}, W2{}, K1{});
      iteration(t3 + 2, C0{}, W2{}, K1{});
    }
    if (t3 < nsteps) iteration(t3, C1{}, W2{}, K1{});
    if (t3 + 1 < nsteps) iteration(t3 + 1, C2{}, W2{}, K1{});
    // iteration nsteps: the map of the last step, then one more barrier while
    // the consumers take it (no products of a step nobody reads)
    const int rl = nsteps % 3;
    if (rl == 0) iteration(nsteps, C0{}, W2{}, K2{});
    else if (rl == 1) iteration(nsteps, C1{}, W2{}, K2{});
    else iteration(nsteps, C2{}, W2{}, K2{});
    wait_vmcnt<0>();  // the last (zero) copies have landed before LDS is reused
    barrier_lds();
    if (tid == 0) pre = meet_load(mw);  // (its latency hides behind the partial stores)
    // Rows past the range: the maps of steps nfull .. nsteps - 1 saw K = 0 there,
    // i.e. phi(0 W + b), the same bits each time; take them out of ksum.
    {
      const int nfull = (t_end - t_begin) / STEP;
      float2 st0 = float2{0.f, 1.f};
      if constexpr (MAP == kSoftmax) {
        float z[NKB * 8], m, inv;
#pragma unroll
        for (int i = 0; i < NKB * 8; ++i) z[i] = kbias[i];
        softmax_stats<NKB * 8, 32>(z, m, inv);
        st0 = float2{m, inv};
      }
      int nzero = 0;  // rows past the range among this lane's 16 rows of each map
      for (int jj = nfull; jj < nsteps; ++jj) {
        const int lim = t_end - (t_begin + jj * STEP + 32 * tg);
#pragma unroll
        for (int r = 0; r < 16; ++r) nzero += crow(lane, r) >= lim;
      }
#pragma unroll
      for (int fb = 0; fb < 2; ++fb) {
        const float z0 = bf2f(f2bf(phi_b(bsplat[fb][0], st0)));  // a zero row's products are the bias tile
        ks[fb] -= (float)nzero * z0;
        ks[fb] += shfl_xor32(ks[fb]);
      }
    }
    __syncthreads();  // LDS free
    if constexpr (NTG > 1) {  // the token groups' ksum, added in order into token group 0
      if (tg > 0 && g == 0) {
        float* rb = red + S::KSOFF + ((tg - 1) * NPW + fs) * 64;
        rb[c] = ks[0];
        rb[32 + c] = ks[1];
      }
      __syncthreads();
      if (tg == 0)
        for (int u = 1; u < NTG; ++u) {
          const float* rb = red + S::KSOFF + ((u - 1) * NPW + fs) * 64;
          ks[0] += rb[c];
          ks[1] += rb[32 + c];
        }
    }
    if (tg == 0) {  // this split's ksum [FG] after its KV, in 16-byte pieces (lane c % 4 == 0: lanes c .. c + 3)
      float k4[2][4];
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int e = 0; e < 4; ++e) k4[fb][e] = __shfl(ks[fb], (lane & ~3) + e, 64);
      if (g == 0 && (c & 3) == 0) {
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) {
          f32x4 v = {k4[fb][0], k4[fb][1], k4[fb][2], k4[fb][3]};
          st16_part(rpart, (uint32_t)(split * pstride) + (uint32_t)(FG * D + 64 * fs + 32 * fb + c) * 4,
                     __builtin_bit_cast(u32x4, v));
        }
      }
    }
  } else {
    // ---- consumer: KV[64 features x the wave's CW_DB column blocks] += phi^T . V
    // over the tokens of its CW_TG token groups, per step
    constexpr int CW_DB = S::CW_DB, CW_TG = S::CW_TG, NDP = S::NDP, NTP = S::NTP;
    const int dp = (pw / NPW) % NDP, tp = pw / NPW / NDP;
    f32x16 kv[2][CW_DB];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
      for (int i = 0; i < CW_DB; ++i) kv[fb][i] = f32x16{};
    auto consume = [&](int j) __attribute__((always_inline)) {
      const int sl = j % 3;
      const uint16_t* vt = sl == 0 ? vr0 : sl == 1 ? vr1 : vr2;
#pragma unroll
      for (int u = 0; u < CW_TG; ++u) {
        const int tgx = tp * CW_TG + u;
        const uint16_t* pt = ptile(sl, tgx * NPW + fs);  // the producer (fs, tgx)
        Frag<uint16_t> pa[2][2], vf[CW_DB][2];
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) pa[fb][hh] = ld_frag<uint16_t>(pt + toff32(32 * fb + c, 16 * hh + 8 * g));
#pragma unroll
        for (int i = 0; i < CW_DB; ++i)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) vf[i][hh] = tr_frag<D>(vt, 32 * tgx + 16 * hh, 32 * (dp * CW_DB + i), lane);
#pragma unroll
        for (int i = 0; i < CW_DB; ++i)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int fb = 0; fb < 2; ++fb) mma(kv[fb][i], pa[fb][hh], vf[i][hh]);
      }
    };
    for (int t = 0; t <= nsteps + 1; ++t) {
      barrier_lds();  // phi^T and V of step t - 2 are in LDS
      if (t > 1) consume(t - 2);
    }
    __syncthreads();  // LDS free
    // the token parts' KV (more than one only when a feature group is one
    // wave wide), added in order into part 0; the same barriers as the
    // producers' ksum sums
    float* const img = red + (((tp > 0 ? tp : 1) - 1) * NPW + fs) * NDP * S::CIMG + dp * S::CIMG;
    if constexpr (NTP > 1) {
      if (tp > 0) {
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
          for (int i = 0; i < CW_DB; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              f32x4 v = {kv[fb][i][4 * q], kv[fb][i][4 * q + 1], kv[fb][i][4 * q + 2], kv[fb][i][4 * q + 3]};
              *reinterpret_cast<f32x4*>(img + (((fb * CW_DB + i) * 4 + q) * 64 + lane) * 4) = v;
            }
      }
    }
    __syncthreads();
    if constexpr (NTP > 1) {
      if (tp == 0)
        for (int u = 1; u < NTP; ++u) {
          const float* rb = red + ((u - 1) * NPW + fs) * NDP * S::CIMG + dp * S::CIMG;
#pragma unroll
          for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int i = 0; i < CW_DB; ++i)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(rb + (((fb * CW_DB + i) * 4 + q) * 64 + lane) * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) kv[fb][i][4 * q + e] += v[e];
              }
        }
    }
    // this split's partial: [fs][fb][db][q][lane][4] (the accumulators'
    // register image: element e of piece q of lane l is KV[f][d] with
    // f = fg0 + 64 fs + 32 fb + crow(l, 4 q + e), d = 32 db + (l & 31)), then ksum [FG]
    if (tp == 0) {
      const uint32_t base = (uint32_t)(split * pstride);
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int i = 0; i < CW_DB; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int db = dp * CW_DB + i;
            f32x4 v = {kv[fb][i][4 * q], kv[fb][i][4 * q + 1], kv[fb][i][4 * q + 2], kv[fb][i][4 * q + 3]};
            st16_part(rpart, base + (uint32_t)((((fs * 2 + fb) * NDB + db) * 4 + q) * 64 + lane) * 16,
                      __builtin_bit_cast(u32x4, v));
          }
    }
  }

  // ---- meet the group's other splits. The partial stores are complete (in
  // this XCD's L2) before the count. If every split of the group runs on one
  // XCD, that L2 is the one place all of them read the partials from. If not,
  // each split writes its L2 back (an agent-scope release) and counts itself
  // in again, and after the second count drops stale lines (an agent-scope
  // acquire), so its loads see memory.
  wait_vmcnt<0>();
  __syncthreads();
  __shared__ unsigned ok_s;
  if (tid == 0) {
    const unsigned ns = (unsigned)a.nsplit;
    unsigned n = 0;
    unsigned long long v = 0;
    bool ok = (pre >> kMeetTag) == a.call ? (v = pre, true) : meet_tagged(mw, a.call, a.spin_limit, n, v);
    if (ok) {
      const bool away = (unsigned)((v >> 16) & 7u) != xcd_id();
      __hip_atomic_fetch_add(mw, away ? 257ull : 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = meet_all(mw, ns, a.spin_limit, n, v);
    }
    // (every split that got here saw the same, final, arrivals word)
    if (ok && (((v >> 8) & 255u) != 0 || a.force_round2 != 0)) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      unsigned long long v2;
      ok = meet_tagged(mw + 1, a.call, a.spin_limit, n, v2);
      if (ok) {
        __hip_atomic_fetch_add(mw + 1, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = meet_all(mw + 1, ns, a.spin_limit, n, v2);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    ok_s = ok;
    // leave: after the last split's departure nobody reads the group's words
    // again in this launch, and that split clears them
    unsigned m = 0;
    unsigned long long d;
    if (meet_tagged(mw + 2, a.call, a.spin_limit, m, d) &&
        (__hip_atomic_fetch_add(mw + 2, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 255u) + 1 == ns) {
      __hip_atomic_store(mw, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(mw + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(mw + 2, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  // A workgroup that gave up writes NaN into its share of the outputs (the
  // call's result is then undefined, and visibly so).
  const bool ok = ok_s != 0;

  // ksum of feature fg0 + f summed over the splits in split order (loads
  // issued eight at a time, ahead of their adds)
  auto ksum_over_splits = [&](int f) -> float {
    float s = 0.f;
    for (int sp = 0; sp < a.nsplit; sp += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             rpart, (int)((uint32_t)(min(sp + u, a.nsplit - 1) * pstride) + (FG * D + f) * 4),
                                             0, 0));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (sp + u < a.nsplit) s += v[u];
    }
    return s;
  };

  // ---- this split's share of the reduction, summed over the splits in order
  // (each thread's loads for up to eight splits issued before its adds)
  if constexpr (PACK) {
    const PackLayout pl{D, F, a.L, (a.L + 31) / 32};
    unsigned char* base = a.pack_bh + (size_t)bh * a.bh_bytes;
    float* biasP = reinterpret_cast<float*>(base);
    float* ksumP = biasP + F;
    uint16_t* kvc = reinterpret_cast<uint16_t*>(base + pl.vec_bytes());
    // task: (fs, fb, db, k, lane) -> the bf16 piece of KV^T chunk fs at row
    // d = 32 db + (lane & 31), columns 32 fb + 16 k + 8 (lane >> 5) .. + 7,
    // from pieces q = 2 k and 2 k + 1 of the partials
    constexpr int TASKS = NPW * 2 * NDB * 2 * 64;
    const int per = (TASKS + a.nsplit - 1) / a.nsplit;
    for (int t = split * per + tid; t < min(TASKS, (split + 1) * per); t += 512) {
      const int ln = t & 63, k = (t >> 6) & 1, db = (t >> 7) % NDB, fb = (t / (128 * NDB)) & 1,
                fst = t / (256 * NDB);
      const uint32_t o0 = (uint32_t)((((fst * 2 + fb) * NDB + db) * 4 + 2 * k) * 64 + ln) * 16;
      const uint32_t o1 = o0 + 64 * 16;
      f32x4 s0 = f32x4{}, s1 = f32x4{};
      for (int sp = 0; sp < a.nsplit; sp += 8) {
        u32x4 v0[8], v1[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t so = (uint32_t)(min(sp + u, a.nsplit - 1) * pstride);
          v0[u] = ld16_part(rpart, so + o0);
          v1[u] = ld16_part(rpart, so + o1);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (sp + u < a.nsplit) {
            s0 += __builtin_bit_cast(f32x4, v0[u]);
            s1 += __builtin_bit_cast(f32x4, v1[u]);
          }
      }
      if (!ok) s0 = s1 = f32x4{kQNaN, kQNaN, kQNaN, kQNaN};
      u32x4 o;
      o[0] = pack_bf16x2(s0[0], s0[1]);
      o[1] = pack_bf16x2(s0[2], s0[3]);
      o[2] = pack_bf16x2(s1[0], s1[1]);
      o[3] = pack_bf16x2(s1[2], s1[3]);
      uint16_t* ch = kvc + (size_t)((fg0 + 64 * fst) / 64) * 64 * D;
      *reinterpret_cast<u32x4*>(ch + toff<64, kRowRead>(32 * db + (ln & 31), 32 * fb + 16 * k + 8 * (ln >> 5))) = o;
    }
    if (split == 0 && tid < FG) {  // ksum and bias of the group's features, in kperm order
      const float s = ksum_over_splits(tid);
      const int f = fg0 + tid;
      ksumP[kperm(f)] = ok ? s : kQNaN;
      biasP[kperm(f)] = (a.bias ? a.bias[(size_t)h * F + f] : 0.f) + (MAP == kElu1 ? 1.f : 0.f);
    }
  } else {
    // task: (fs, fb, db, q, g, lane quad) -> KV rows f = .. crow(l, 4 q + e) (e = 0..3),
    // columns d = 32 db + 4 cq .. + 3: four lanes' pieces, transposed
    constexpr int TASKS = NPW * 2 * NDB * 4 * 2 * 8;
    const int per = (TASKS + a.nsplit - 1) / a.nsplit;
    for (int t = split * per + tid; t < min(TASKS, (split + 1) * per); t += 512) {
      const int cq = t & 7, gg = (t >> 3) & 1, q = (t >> 4) & 3, db = (t >> 6) % NDB, fb = (t / (64 * NDB)) & 1,
                fst = t / (128 * NDB);
      f32x4 sum[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};  // [lane i][element e]
      for (int sp = 0; sp < a.nsplit; ++sp) {
        u32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ln = 32 * gg + 4 * cq + i;
          v[i] = ld16_part(rpart, (uint32_t)(sp * pstride) +
                                       (uint32_t)((((fst * 2 + fb) * NDB + db) * 4 + q) * 64 + ln) * 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[i] += __builtin_bit_cast(f32x4, v[i]);
      }
      float* kvo = a.kv_out + (size_t)bh * F * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = fg0 + 64 * fst + 32 * fb + 8 * q + 4 * gg + e;  // crow(lane of half gg, 4 q + e)
        f32x4 o = {sum[0][e], sum[1][e], sum[2][e], sum[3][e]};
        if (!ok) o = f32x4{kQNaN, kQNaN, kQNaN, kQNaN};
        *reinterpret_cast<f32x4*>(kvo + (size_t)f * D + 32 * db + 4 * cq) = o;
      }
    }
    if (split == 0 && tid < FG) {
      const float s = ksum_over_splits(tid);
      a.ks_out[(size_t)bh * F + fg0 + tid] = ok ? s : kQNaN;
    }
  }
}

// ---------------------------------------------------------------- landmark-only pack
struct LmPackArgs {
  const uint16_t* K;
  const uint16_t* V;
  int N, L;
  unsigned char* pack_bh;  // [BH][nlb chunks]
};

template <int D>
__global__ __launch_bounds__(256) void lm_pack_kernel(LmPackArgs a) {
  __shared__ uint16_t vrows[32][D + 8];
  const int nlb = (a.L + 31) / 32;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int bh = item / nlb, jb = item % nlb;
  const PackLayout pl{D, 0, a.L, nlb};
  uint16_t* kl = reinterpret_cast<uint16_t*>(a.pack_bh + (size_t)bh * pl.bh_bytes()) + (size_t)jb * pl.chunk_elems();
  landmark_chunk<D, 256>(a.K + (size_t)bh * a.N * D, a.V + (size_t)bh * a.N * D, a.N, a.L, jb, kl, vrows, threadIdx.x);
}

// ---------------------------------------------------------------- host side
// Compute units the grid may fill (one workgroup each), for the device that is
// current: the workspace is sized for at most 256, the MI355X count.
static int kvs_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    v = n < 256 ? n : 256;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

struct KvsPlan {
  int FG, NG, groups, nsplit, chunk, per_xcd;
  size_t part_bytes, cnt_bytes;  // fp32 partials; counters (256-byte aligned)
};

static KvsPlan kvs_plan(const Problem& p, int cus) {
  KvsPlan k;
  k.FG = p.F < 128 ? p.F : 128;
  k.NG = p.F / k.FG;
  const int step = 32 * (4 / (k.FG / 64));
  k.groups = p.B * p.H * k.NG;
  // Groups are spread over the 8 XCDs, gx per XCD, each with its splits on
  // that XCD's compute units (one workgroup per unit).
  const int gx = (k.groups + 7) / 8;
  int ns = (cus / 8) / gx;
  const int maxs = (p.N + 2 * step - 1) / (2 * step);  // at least two steps per split
  if (ns > maxs) ns = maxs;
  // At most 16 splits: with fewer groups than XCDs (the 3-head share shape)
  // more splits only add meeting and reduction work (16: 27.7 against 28.7 us
  // with 24 at [1,3,4608,128]; 8 and 12 gave no gain). (The count of a
  // meeting word is a byte: at most 255 splits in any case.)
  if (ns > 16) ns = 16;
  if (ns < 1) ns = 1;
  const int per = (p.N + ns - 1) / ns;
  k.chunk = (per + step - 1) / step * step;
  k.nsplit = (p.N + k.chunk - 1) / k.chunk;  // every split non-empty
  k.per_xcd = gx * k.nsplit;
  k.part_bytes = (size_t)k.groups * k.nsplit * (size_t)(k.FG * p.D + k.FG) * 4;
  k.cnt_bytes = ((size_t)k.groups * 32 + 255) / 256 * 256;
  return k;
}

static PackLayout pack_layout(const Problem& p, int L) {
  PackLayout pl{p.D, p.F, L, (L + 31) / 32};
  return pl;
}

static bool kvs_supported(const Problem& p) {
  if (p.dtype != 1 || (p.D != 64 && p.D != 128)) return false;
  if (p.proj) return p.fmap == kElu1 && p.F % 128 == 0;
  return p.F == p.D;
}

size_t fused_workspace_bytes(const Problem& p, int L) {
  const KvsPlan k = kvs_plan(p, 256);
  const PackLayout pl = pack_layout(p, L);
  return k.part_bytes + k.cnt_bytes + (size_t)p.B * p.H * pl.bh_bytes() + (size_t)p.H * pl.w_bytes();
}

size_t kv2_reduce_workspace_bytes(const Problem& p) {
  const KvsPlan k = kvs_plan(p, 256);
  return k.part_bytes + k.cnt_bytes;
}

// Launch numbers tag the meeting words (45 bits; 0, the number of a cleared
// word, is skipped). Each process starts the count at a random point, so
// words another process left in reused memory (only a launch whose splits
// never all left does so) are not taken for this process's.
static unsigned long long first_launch_number() {
  std::random_device rd;
  return ((unsigned long long)rd() << 32) ^ (unsigned long long)rd() ^
         (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
}
static unsigned long long next_launch_number() {
  static std::atomic<unsigned long long> counter{first_launch_number()};
  unsigned long long v;
  do v = (counter.fetch_add(1, std::memory_order_relaxed) + 1) & ((1ull << (64 - kMeetTag)) - 1);
  while (v == 0);
  return v;
}

template <int D, int F, bool PROJ, int MAP, bool PACK>
static hipError_t launch_kvs_t(const KvsArgs& a0, int groups, hipStream_t s, StageTimer* t) {
  (void)groups;
  KvsArgs a = a0;
  a.call = next_launch_number();
  hipLaunchKernelGGL((kv_stage_kernel<D, F, PROJ, MAP, PACK>), dim3(8 * a.per_xcd), dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (t) t->mark();
  return e;
}

template <bool PACK>
static hipError_t launch_kvs(const Problem& p, const KvsArgs& a, int groups, hipStream_t s, StageTimer* t) {
  if (p.D == 128) {
    if (p.proj) {
      if (p.F == 256) return launch_kvs_t<128, 256, true, kElu1, PACK>(a, groups, s, t);
      if (p.F == 512) return launch_kvs_t<128, 512, true, kElu1, PACK>(a, groups, s, t);
      if (p.F == 768) return launch_kvs_t<128, 768, true, kElu1, PACK>(a, groups, s, t);
      if (p.F == 1024) return launch_kvs_t<128, 1024, true, kElu1, PACK>(a, groups, s, t);
      return hipErrorInvalidValue;
    }
    if (p.fmap == kRelu) return launch_kvs_t<128, 128, false, kRelu, PACK>(a, groups, s, t);
    if (p.fmap == kSoftmax) return launch_kvs_t<128, 128, false, kSoftmax, PACK>(a, groups, s, t);
    return launch_kvs_t<128, 128, false, kElu1, PACK>(a, groups, s, t);
  }
  if (p.proj) {
    if (p.F == 256) return launch_kvs_t<64, 256, true, kElu1, PACK>(a, groups, s, t);
    if (p.F == 512) return launch_kvs_t<64, 512, true, kElu1, PACK>(a, groups, s, t);
    if (p.F == 768) return launch_kvs_t<64, 768, true, kElu1, PACK>(a, groups, s, t);
    if (p.F == 1024) return launch_kvs_t<64, 1024, true, kElu1, PACK>(a, groups, s, t);
    return hipErrorInvalidValue;
  }
  if (p.fmap == kRelu) return launch_kvs_t<64, 64, false, kRelu, PACK>(a, groups, s, t);
  if (p.fmap == kSoftmax) return launch_kvs_t<64, 64, false, kSoftmax, PACK>(a, groups, s, t);
  return launch_kvs_t<64, 64, false, kElu1, PACK>(a, groups, s, t);
}

static KvsArgs kvs_args(const Problem& p, const KvsPlan& k, const void* K, const void* V, const void* W,
                        const float* bias, int L, unsigned char* ws) {
  KvsArgs a{};
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.W = static_cast<const uint16_t*>(W);
  a.bias = bias;
  a.H = p.H;
  a.N = p.N;
  a.L = L;
  a.nsplit = k.nsplit;
  a.chunk = k.chunk;
  a.groups = k.groups;
  a.per_xcd = k.per_xcd;
  a.part = reinterpret_cast<float*>(ws);
  a.counters = reinterpret_cast<unsigned long long*>(ws + k.part_bytes);
  a.spin_limit = env_spin_limit(1u << 20);  // about a second of polling
  a.force_round2 = env_flag("TTR_KVS_CROSS_XCD_ROUND") ? 1u : 0u;
  return a;
}

hipError_t launch_kv2(const Problem& p, const void* K, const void* V, const void* W, const float* bias, int L,
                      void* ws, FusedPack* pk, hipStream_t s, StageTimer* t) {
  if (!kvs_supported(p)) return hipErrorInvalidValue;
  const KvsPlan k = kvs_plan(p, kvs_cus());
  const KvsPlan kw = kvs_plan(p, 256);  // the workspace's layout
  const PackLayout pl = pack_layout(p, L);
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  unsigned char* pbh = w8 + kw.part_bytes + kw.cnt_bytes;
  unsigned char* pw = pbh + (size_t)p.B * p.H * pl.bh_bytes();
  pk->pack_bh = pbh;
  pk->pack_w = pw;
  pk->bh_bytes = pl.bh_bytes();
  pk->w_bytes = pl.w_bytes();
  KvsArgs a = kvs_args(p, k, K, V, W, bias, L, w8);
  a.counters = reinterpret_cast<unsigned long long*>(w8 + kw.part_bytes);
  a.pack_bh = pbh;
  a.bh_bytes = pl.bh_bytes();
  a.pack_w = pw;
  return launch_kvs<true>(p, a, k.groups, s, t);
}

hipError_t launch_kv2_reduce(const Problem& p, const void* K, const void* V, const void* W, const float* bias,
                             float* KV, float* ksum, void* ws, hipStream_t s) {
  if (!kvs_supported(p)) return hipErrorInvalidValue;
  const KvsPlan k = kvs_plan(p, kvs_cus());
  const KvsPlan kw = kvs_plan(p, 256);
  unsigned char* w8 = static_cast<unsigned char*>(ws);
  KvsArgs a = kvs_args(p, k, K, V, W, bias, 0, w8);
  a.counters = reinterpret_cast<unsigned long long*>(w8 + kw.part_bytes);
  a.kv_out = KV;
  a.ks_out = ksum;
  return launch_kvs<false>(p, a, k.groups, s, nullptr);
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
  LmPackArgs a{};
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.N = p.N;
  a.L = L;
  a.pack_bh = static_cast<unsigned char*>(ws);
  pk->pack_bh = a.pack_bh;
  pk->pack_w = nullptr;
  pk->bh_bytes = pl.bh_bytes();
  pk->w_bytes = 0;
  const dim3 grid((unsigned)(pl.nlb * p.B * p.H));
  if (p.D == 128) hipLaunchKernelGGL((lm_pack_kernel<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((lm_pack_kernel<64>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttr

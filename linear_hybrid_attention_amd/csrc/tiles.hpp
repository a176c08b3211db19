// LDS tile layouts shared by the bf16 hot-path kernels (the key/value stage
// writes operand packs in exactly these layouts; the query kernel copies them
// into LDS verbatim), plus the asynchronous-copy and wait helpers.
//
// All tiles are row-major bf16 with 16-byte pieces permuted within a row
// (XOR swizzle) so that the MFMA operand reads hit disjoint LDS banks:
//   kRowRead:  rows read as MFMA A/B fragments with ds_read_b128 by 32
//              consecutive rows at one column (phys = piece ^ (row & 15) for
//              rows of >= 256 bytes, piece ^ ((row >> 1) & 7) for 128 bytes).
//   kTrRead:   rows read column-wise with ds_read_b64_tr_b16 (the tile holds
//              [k][n]; the read yields a fragment with k in registers). Half a
//              wave reads 4 consecutive rows x 64 bytes; rows whose addresses
//              are a multiple of 256 bytes apart share banks, so their 64-byte
//              windows are moved apart: phys = piece ^ ((row & 3) << 2) for
//              >= 256-byte rows, piece ^ (((row >> 1) & 1) << 2) for 128-byte
//              rows (rows r and r + 2 of a group of 4).
#pragma once
#include "common.hpp"

namespace ttr {

enum TileKind { kRowRead = 0, kTrRead = 1 };

template <int COLS, int KIND>
__host__ __device__ __forceinline__ constexpr int tswz(int row) {
  static_assert(COLS * 2 == 128 || COLS * 2 >= 256, "row size");
  if constexpr (KIND == kRowRead) return (COLS * 2 == 128) ? ((row >> 1) & 7) : (row & 15);
  else return (COLS * 2 == 128) ? (((row >> 1) & 1) << 2) : ((row & 3) << 2);
}
// element offset of (row, col) in a bf16 tile with COLS columns
template <int COLS, int KIND>
__host__ __device__ __forceinline__ constexpr int toff(int row, int col) {
  return row * COLS + (((col >> 3) ^ tswz<COLS, KIND>(row)) << 3) + (col & 7);
}

// Element offset of (row r, column j) in a bf16 tile with 32 columns (64-byte
// rows), stored as rows of 128 bytes holding rows 2 i and 2 i + 1 with the
// kRowRead swizzle, so that 16-byte row reads by 32 consecutive rows are
// spread over the banks.
__host__ __device__ __forceinline__ constexpr int toff32(int r, int j) {
  return toff<64, kRowRead>(r >> 1, ((r & 1) << 5) + j);
}

// Fragment (8 k-values of one lane) of a tile stored [k rows][n cols] (kTrRead
// layout), for the 16 k-rows starting at k0 and the 32 n-columns starting at
// n0. Slot 8g + i of lane l (g = l / 32) holds k = k0 + crow(l, i): the same
// k order as a 32x32 MFMA C tile reused as an operand (see common.hpp).
// Within each 16-lane group the hardware hands lane l element (l % 4) of the
// 8 bytes addressed by lane 4 e + (l % 16) / 4 of the group as its element e.
template <int COLS, int KIND = kTrRead>
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tile, int k0, int n0, int lane) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const int G = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
  const int row = k0 + 4 * (G >> 1) + e;
  const int col = n0 + 16 * (G & 1) + 4 * q;
  const uint16_t* p0 = tile + toff<COLS, KIND>(row, col);
  const uint16_t* p1 = tile + toff<COLS, KIND>(row + 8, col);
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p0);
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p1);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Asynchronous global -> LDS copy of one 16-byte piece per lane: lane l of
// the wave writes lds_wave_base + 16 l (the LDS address must be wave-uniform).
__device__ __forceinline__ void copy16_async(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// Raw buffer resource over [base, base + bytes): 32-bit data format, no
// stride or swizzle; an access at or past `bytes` reads zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The same asynchronous copy through a buffer resource: lane l copies the 16
// bytes at soff + voff of r to lds_wave_base + 16 l. Unlike the global form,
// this one is not a flat-segment access, so the compiler can still count the
// wave's outstanding LDS reads in order while copies are in flight.
__device__ __forceinline__ void copy16_async(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, (int)voff,
                                           (int)soff, 0, 0);
}

// 16-byte store through a buffer resource at byte offset off (dropped by the
// hardware when off is at or past the resource's size).
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t off, const u32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

// The same store at system scope (cache-policy bits sc0 and sc1): the L2
// writes it through to memory at once instead of holding a dirty line until
// the end-of-kernel write-back.
__device__ __forceinline__ void store16_wt(__amdgpu_buffer_rsrc_t r, uint32_t off, const u32x4& v) {
  constexpr int kSc0Sc1 = 1 | 16;
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kSc0Sc1);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the release/acquire fence of __syncthreads (which
// would wait for every outstanding global load, including prefetches). The
// memory clobber keeps the compiler from moving LDS accesses across it; the
// callers wait for the asynchronous copies they need before calling it.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads/writes are done
  asm volatile("s_barrier" ::: "memory");
}

// Instruction classes of the compiler's scheduling groups: sched_group<kind,
// n>() asks the scheduler to place the next n instructions of that kind at
// this point of the region's order (a hint; data dependences still hold).
enum SchedKind : int { kSchedValu = 0x002, kSchedTrans = 0x400, kSchedAnyValu = 0x402, kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100, kSchedDsWrite = 0x200 };
template <int KIND, int N>
__device__ __forceinline__ void sched_group() { __builtin_amdgcn_sched_group_barrier(KIND, N, 0); }

// Makes v count as used at this point of the instruction stream: the
// computation of v cannot then be moved past a later barrier or other
// volatile asm (the compiler otherwise sinks pure register work towards its
// first use).
// (Device pass only: the host compiler has no "v" register class, and a
// constraint it rejects inside a kernel template makes it drop that kernel's
// launch stubs.)
template <typename T>
__device__ __forceinline__ void pin_before(const T& v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(v));
#else
  (void)v;
#endif
}

// Orders this wave's LDS accesses across lanes (lane i writes what lane j
// then reads). The hardware executes one wave's LDS instructions in order, so
// this emits no instruction; it only keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

}  // namespace ttr

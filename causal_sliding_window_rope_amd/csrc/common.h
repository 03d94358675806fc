// Device-side helpers shared by the gfx950 kernels of libswa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};
template <> struct Elem<bf16> {
  static __device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
  static __device__ __forceinline__ bf16 from_f(float x) { return (bf16)x; }  // RNE
};

// bf16 <-> float on packed 32-bit words (two bf16 per word, low half = lower index).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// A 128-bit word as float values: 4 float or 8 bf16 elements (overloaded on the array size).
__device__ __forceinline__ void unpack16(uint4 w, float (&o)[4]) {
  o[0] = __uint_as_float(w.x); o[1] = __uint_as_float(w.y);
  o[2] = __uint_as_float(w.z); o[3] = __uint_as_float(w.w);
}
__device__ __forceinline__ void unpack16(uint4 w, float (&o)[8]) {
  o[0] = bf_lo(w.x); o[1] = bf_hi(w.x); o[2] = bf_lo(w.y); o[3] = bf_hi(w.y);
  o[4] = bf_lo(w.z); o[5] = bf_hi(w.z); o[6] = bf_lo(w.w); o[7] = bf_hi(w.w);
}
__device__ __forceinline__ uint4 pack16(const float (&v)[4]) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3]));
}
__device__ __forceinline__ uint4 pack16(const float (&v)[8]) {
  return make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                    pack_bf2(v[6], v[7]));
}

// Wave64 cross-lane helpers.
__device__ __forceinline__ float xor_shfl(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Lane exchange inside a DPP row of 16 lanes (no trip through the LDS crossbar that
// xor_shfl takes). CTRL: 0xB1 quad_perm [1,0,3,2] (lane ^ 1), 0x4E quad_perm [2,3,0,1]
// (lane ^ 2), 0x141 row_half_mirror (i <-> 7 - i), 0x140 row_mirror (i <-> 15 - i), 0x128
// row_ror:8 (lane ^ 8 within the row).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N a power of two <= 64): DPP adds up to a 16-lane row
// (quad swaps, then the half-row and row mirrors), shuffles beyond.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);
  if constexpr (N >= 16) x += dpp_mov<0x140>(x);
#pragma unroll
  for (int m = 16; m < N; m <<= 1) x += xor_shfl(x, m);
  return x;
}

// max / sum over the two 32-lane halves of a wave (lane l and lane l^32).
__device__ __forceinline__ float half_swap(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // lanes < 32 receive the partner's value in r[1], lanes >= 32 in r[0]
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

// LDS-qualified pointers (address space 3).
template <typename T> using lds_t = __attribute__((address_space(3))) T;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// One query row of an O^T accumulator tile (32 dims x 32 queries, lane = query l32, half hi
// holding dims 8a + 4hi .. + 3 of each group of 8, a < 4), scaled by `inv` and stored as bf16
// at row + 32 db in 16-byte pieces: the lane stores dims 16j + 8hi .. + 7 of each 16 (a = 2j + hi)
// and takes the other four from its partner lane (same query) by a half-wave swap. Every lane
// of the wave takes part in the swap; `store` gates the memory write.
template <typename V16>
__device__ __forceinline__ void store_orow16(bf16* row, int db, const V16& acc, float inv,
                                             int hi, bool store) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    unsigned c[2][2];   // this lane's 4 dims of a = 2j and of a = 2j + 1, as bf16 pairs
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int a = 2 * j + e;
      c[e][0] = pack_bf2(acc[4 * a + 0] * inv, acc[4 * a + 1] * inv);
      c[e][1] = pack_bf2(acc[4 * a + 2] * inv, acc[4 * a + 3] * inv);
    }
    unsigned r[2];   // the partner's 4 dims of this lane's a
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const unsigned sv = hi ? c[0][x] : c[1][x];
      const auto pr = __builtin_amdgcn_permlane32_swap(sv, sv, false, false);
      r[x] = hi ? pr[0] : pr[1];
    }
    const u32x4 w = hi ? (u32x4){r[0], r[1], c[1][0], c[1][1]}
                       : (u32x4){c[0][0], c[0][1], r[0], r[1]};
    if (store) *reinterpret_cast<u32x4*>(row + 32 * db + 16 * j + 8 * hi) = w;
  }
}

// Asynchronous 16-byte global -> LDS copy in its buffer form (buffer_load_dwordx4 ... lds):
// lane l of the wave reads resource + voff bytes and writes lds_base + 16*l bytes (lds_base
// must be the same for the whole wave). The resource is a uniform base address with a range of
// 2^31 - 1 bytes (every offset from a tile's first row stays below it: the entry points cap a
// tensor at 2^30 elements) and the raw-buffer configuration word of gfx9-family targets. The compiler
// counts these copies on vmcnt alone; the global form (global_load_lds) it also treats as a
// possible LDS access, which makes every LDS read issued while a copy is in flight wait for
// lgkmcnt(0) instead of for its own place in the queue (3-5 % of the dK/dV kernel's time).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void b2lds16(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                        lds_t<void>* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voff, 0, 0, 0);
}

// Per-lane 32-bit offset made opaque to the optimiser at its use, so that base + offset is
// formed at the load (uniform base + 32-bit lane offset) instead of being hoisted out of
// the tile loop as a per-lane 64-bit address: the hoisted addresses cost two VGPRs each and
// pushed the forward and dQ kernels into spilling (7-9 % of their time).
__device__ __forceinline__ unsigned opaque(unsigned x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Wait until this wave's outstanding vector-memory operations (incl. LDS DMA) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Wait until at most N vector-memory operations of this wave are outstanding (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Transposing LDS read: each 16-lane group reads a 4 x 16 block of b16 (lane j gives the
// address of row j/4, columns 4(j%4)..+3) and lane i receives column i, rows 0..3.
__device__ __forceinline__ bf16x4 ds_read_tr16(const lds_t<bf16>* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_t<s16x4>*)p);
  return __builtin_bit_cast(bf16x4, r);
}

// Bank swizzle of 16-byte chunk positions within a tile row of D bf16 (XOR with a function of
// the row). gfx950 LDS has 64 four-byte banks; a 128-bit read serves 16 lanes per cycle and a
// transposing 64-bit read 32 lanes per cycle. With these functions the row reads of 16
// consecutive rows at one chunk, and the transposing reads of 4 consecutive rows x 4 chunks,
// each touch all 64 banks once (measured: zero SQ_LDS_BANK_CONFLICT).
template <int D> __device__ __forceinline__ int swz(int r);
template <> __device__ __forceinline__ int swz<128>(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
template <> __device__ __forceinline__ int swz<64>(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// Block (bh, r) of a grid of nper blocks per head in longest-first order (lpt_order in
// internal.h): workgroup ids go to the eight XCDs in turn; XCD x holds heads x * hpx .. + hpx - 1
// and issues rank r = 0 (a head's largest block) of each of them before rank 1.
// snake > 0 (kernels whose whole grid is resident at once, so that the order fixes which blocks
// share a CU): every other round of `snake` workgroups of an XCD (one per CU) is issued in
// reverse, so that the CUs that took the largest blocks of one round take the smallest of the
// next.
__device__ __forceinline__ int2 lpt_block(int nper, int snake = 0) {
  const int hpx = (int)(gridDim.x >> 3) / nper;
  int j = (int)(blockIdx.x >> 3);
  if (snake > 0) {
    const int rd = j / snake, c = j - rd * snake;
    if ((rd & 1) && (rd + 1) * snake <= hpx * nper) j = rd * snake + (snake - 1 - c);
  }
  const int r = j / hpx;
  return make_int2((int)(blockIdx.x & 7) * hpx + (j - r * hpx), r);
}

// CUs per XCD of gfx950 (256 CUs in 8 XCDs).
constexpr int kCusPerXcd = 32;

// Scheduling fence: the compiler may not move instructions across it. Used to bound how far
// ahead LDS loads are hoisted (each hoisted load keeps its result registers live).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Placed first in the body of a rarely taken, wave-uniform branch: an empty volatile asm may not
// be speculated, so the compiler keeps the branch instead of executing the body unconditionally
// under a select.
__device__ __forceinline__ void branch_keep() { asm volatile("" ::: "memory"); }

// Workgroup barrier for LDS data produced by ds_* stores only: waits for this wave's LDS
// operations (lgkmcnt(0)) but not for outstanding global loads, async global->LDS copies or
// atomics, then s_barrier; empty volatile asm on both sides keeps the compiler from moving
// memory accesses across it. (__syncthreads() also drains vmcnt, which would expose the latency
// of in-flight prefetches and atomics.) Data written by async copies needs wait_vmem* first.
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt left at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 8-byte LDS store issued as a plain ds_write_b64. The compiler conservatively drains all
// outstanding vector-memory operations before a normal LDS store while async global->LDS
// copies are in flight; the stores that use this helper go to an LDS array those copies never
// write, and lds_sync() waits for them (lgkmcnt(0)) before any other wave reads them.
__device__ __forceinline__ void ds_store_b64(lds_t<bf16>* p, unsigned long long v) {
  asm volatile("ds_write_b64 %0, %1" : : "v"((unsigned)(size_t)p), "v"(v) : "memory");
}

// Value-embedding row (D bf16 of head h) of token t of sequence b: either in the (B, T, H*D)
// tensor, or, with token ids, row ids[b*T + t] of a (rows, H*D) table; nullptr for an id outside
// the table (such a token gets a zero value embedding and no table gradient).
template <int D, typename E>
__device__ __forceinline__ const E* ve_row(const E* ve, const int* ids, int rows, int b, int T,
                                           int H, int h, int t) {
  if (ids) {
    const int id = ids[(size_t)b * T + t];
    return (unsigned)id < (unsigned)rows ? ve + ((size_t)id * H + h) * D : nullptr;
  }
  return ve + (((size_t)b * T + t) * H + h) * D;
}

// Keys visible to this lane's query row: [lo, lo + n) (causal window, sequence end and, with
// document masking, the start of the row's document); wlo0 / wlo1: lo of the wave's first and
// last query (lo never decreases along a row, so these bound the whole wave).
struct RowRange {
  int lo;
  unsigned n;
  int wlo0, wlo1;
};

template <bool DOC>
__device__ __forceinline__ RowRange row_range(const int* bounds, int b, int T, int W, int myq) {
  const int qc = min(myq, T - 1);
  int start = 0;
  if constexpr (DOC) start = bounds[2 * ((size_t)b * T + qc)];
  RowRange r;
  r.lo = max(qc - W + 1, start);
  r.n = (unsigned)(qc - r.lo + 1);
  r.wlo0 = __builtin_amdgcn_readlane(r.lo, 0);
  r.wlo1 = __builtin_amdgcn_readlane(r.lo, 31);
  return r;
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace swa

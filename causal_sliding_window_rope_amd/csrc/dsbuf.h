// Layout of the stored dS^T of the bf16 backward: the key-block-major dK/dV kernel writes the
// bf16 dS^T it has already formed for dK, and the query-block-major dQ kernel reads it back
// (dQ = scale dS K) instead of recomputing S, P and dP ("GPT-2 124M 复现" §19: the backward
// recomputes what it needs from the saved row statistics; dS is formed once, by that
// recomputation, and kept for the second product that needs it).
//
// Unit of storage: a chunk = one 32-key x 32-query block of dS^T (the work of one wave of the
// dK/dV kernel on one 32-query unit), 2 KiB of bf16, in the order that wave holds it: lane
// (key kappa = l % 32, h = l / 32) owns queries 8a + 4h + r (a, r < 4) and stores them as four
// 8-byte runs, run a at byte 64 kappa + 32 h + 8 a. A transposing LDS read (ds_read_b64_tr_b16)
// of a chunk then yields the B operand of dQ^T += K^T dS^T (lane = query, 4 keys per read)
// with every 32-lane half touching all 64 banks once.
//
// Chunks of a (b, h) head: key block kb (128 keys = 4 key groups w of 32), query tile qt
// (128 queries = 4 units mb of 32), slot = qt - kb in [0, nslot): chunk index
// ((((b*H + h) * nqt + qt) * nslot + slot) * 4 + w) * 4 + mb, query-tile major, so that the dQ
// kernel (one workgroup per query tile) reads one contiguous run. A chunk is written iff the
// dK/dV kernel computes that unit (chunk_live); no other chunk is ever read.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace swa {
namespace dsb {

constexpr int KEYS = 128;          // keys per key block (one dK/dV workgroup)
constexpr int QUERIES = 128;       // queries per query tile
constexpr int CHUNK_BYTES = 2048;  // 32 x 32 bf16
constexpr int CHUNKS = 16;         // chunks per (key block, query tile)

// Query tiles a key block can see: kb .. kb + nslot - 1 (window W already clamped to T).
__host__ __device__ inline int nslot(int T, int W) {
  const int nqt = (T + QUERIES - 1) / QUERIES;
  const int s = (W + KEYS - 2) / QUERIES + 1;
  return s < nqt ? s : nqt;
}

__host__ __device__ inline int nkb(int T) { return (T + KEYS - 1) / KEYS; }

__host__ inline size_t buffer_bytes(int B, int T, int H, int W) {
  return (size_t)B * H * nkb(T) * nslot(T, W) * CHUNKS * CHUNK_BYTES;
}

// Byte offset of the first chunk of (head bh, key block kb, slot): query tile kb + slot of
// the nkb_ (= number of query tiles) of the head.
__device__ __forceinline__ size_t block_offset(int bh, int kb, int slot, int nkb_, int nslot_) {
  return (((size_t)bh * nkb_ + kb + slot) * nslot_ + slot) * (size_t)(CHUNKS * CHUNK_BYTES);
}

// Whether the dK/dV kernel computes (and stores) the unit of key group [kw, kw + 32) and
// queries [qm, qm + 32): the same test as its skip of a 32-query unit. The last query that sees
// key kw + 31 is min(kc + W - 1, end - 1) with kc = min(kw + 31, T - 1) and end the end of
// kc's document (T without document masking).
template <bool DOC>
__device__ __forceinline__ bool chunk_live(const int* bounds, int b, int T, int W, int kw, int qm) {
  if (kw >= T) return false;
  const int kc = min(kw + 31, T - 1);
  int kend = T;
  if constexpr (DOC) kend = bounds[2 * ((size_t)b * T + kc) + 1];
  const int whi1 = min(kc + W - 1, kend - 1);
  return !(qm + 31 < kw || qm > whi1);
}

}  // namespace dsb
}  // namespace swa

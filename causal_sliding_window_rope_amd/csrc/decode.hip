// Sliding-window decoding from a ring K/V cache for gfx950: one new token per sequence.
//
// "GPT-2 124M 复现" §7: generation that keeps the past keys and values instead of recomputing
// every prefix position. A decoding step at position p is row p of the training forward: the
// new q and k are rotated by the angle p * theta_i and QK-normalised, k and v go to the cache
// (position j lives in slot j mod C of a C-slot ring per sequence, native (B, C, H, D) layout),
// and the query attends to positions max(0, p-W+1) .. p.
//
// The attention of one query is HBM-bound (each cached K/V row is read once per step), so it
// runs on the vector ALUs, not on MFMA: a row group of D*size/16 lanes reads one K or V row
// with one 16-byte load per lane (the whole row in one coalesced access), keeps an online
// softmax in exp2 units, and the window is split over several workgroups per (b, h) so that a
// step launches ~768 workgroups of eight waves (flash-decoding); a second kernel merges the
// splits. On the d24 decoding step (32 sequences, 12 heads, windows 1024 / 2048) eight-wave
// workgroups at ~768 per step measured best among 4, 8 and 16 waves at 384 to 1024 workgroups
// (spread ~8 %), and nontemporal cache loads another ~8 % over ordinary ones.
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "rope_row.h"

namespace swa {
namespace dec {

// ---------------------------------------------------------------------------------------------
// Prologue: RoPE at position pos[b], then the RMS QK-norm, of each new q and k row, in the row
// layout of rope_row.h (TPR = D*size/16 lanes per row, 64/TPR rows per 64-lane workgroup), so
// that the rows are bitwise what rope_qknorm_fwd computes for the same position; k and v go to
// the cache.
// ---------------------------------------------------------------------------------------------
template <typename E, int D>
__global__ void __launch_bounds__(64) prologue_kernel(const E* __restrict__ q,
                                                      const E* __restrict__ k,
                                                      const E* __restrict__ v,
                                                      const float* __restrict__ cs, int rows,
                                                      const int* __restrict__ pos,
                                                      E* __restrict__ qn, E* __restrict__ kc,
                                                      E* __restrict__ vc, int H, int cap,
                                                      float eps, int nbh) {
  using RW = RowWord<E>;
  constexpr int VPT = RW::VPT, TPR = D / VPT, RPW = 64 / TPR;
  const int lane = threadIdx.x, li = lane % TPR;
  const int bh = blockIdx.x * RPW + lane / TPR;
  if (bh >= nbh) return;   // whole row groups leave together
  const int b = bh / H, h = bh - b * H;
  const int p = pos[b];
  const bool ok = p >= 0 && p < rows;   // the angle table must cover the position
  const size_t in = (size_t)bh * D + li * VPT;
  float c[VPT], sn[VPT];
  load_cs<VPT>(cs, ok ? p : 0, D / 2, (li % (TPR / 2)) * VPT, c, sn);
  const bool second = li >= TPR / 2;
  RW x, y;
  x.load(q + in);
  rope_norm_row<VPT, TPR, D>(x.v, c, sn, second, eps, y.v);
  if (!ok) {
#pragma unroll
    for (int e = 0; e < VPT; ++e) y.v[e] = NAN;
  }
  y.store(qn + in);
  if (!ok) return;   // the cache is left untouched for an invalid position
  const size_t cr = (((size_t)b * cap + p % cap) * H + h) * D + li * VPT;
  x.load(k + in);
  rope_norm_row<VPT, TPR, D>(x.v, c, sn, second, eps, y.v);
  y.store(kc + cr);
  *reinterpret_cast<uint4*>(vc + cr) = *reinterpret_cast<const uint4*>(v + in);
}

// ---------------------------------------------------------------------------------------------
// Attention of the new query over its window.
// ---------------------------------------------------------------------------------------------
struct Params {
  const void* qn; const void* kc; const void* vc; const int* pos;
  void* o; float* lse; float* part;   // part: (B*H, nsplit, D + 2) floats when nsplit > 1
  int H, cap, window, nsplit;
  float c;   // scale * log2(e)
};

template <typename E, int D> struct Cfg {
  static constexpr int VPL = 16 / sizeof(E);   // elements per 16-byte load
  static constexpr int LPR = D / VPL;          // lanes per row
  static constexpr int RPW = 64 / LPR;         // rows per wave per load
  static constexpr int U = 4;                  // rows per row group in flight
};

__device__ __forceinline__ void merge(float& m, float& l, float* acc, float m2, float l2,
                                      const float* acc2, int n) {
  const float mn = fmaxf(m, m2);
  const float a = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
  const float b = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
  l = l * a + l2 * b;
  for (int i = 0; i < n; ++i) acc[i] = acc[i] * a + acc2[i] * b;
  m = mn;
}

template <typename E>
__device__ __forceinline__ void unpack16(const uint4 w, float* dst) {
  if constexpr (sizeof(E) == 2) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { dst[2 * i] = bf_lo(ws[i]); dst[2 * i + 1] = bf_hi(ws[i]); }
  } else {
    dst[0] = __uint_as_float(w.x); dst[1] = __uint_as_float(w.y);
    dst[2] = __uint_as_float(w.z); dst[3] = __uint_as_float(w.w);
  }
}

// Cached K / V rows are read once per step and not again before the other layers have swept
// the caches through: loaded with the nontemporal hint.
__device__ __forceinline__ uint4 ld16_stream(const void* src) {
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <typename E, int D>
__device__ __forceinline__ void load16(const E* src, float* dst) {
  unpack16<E>(*reinterpret_cast<const uint4*>(src), dst);
}

#ifndef SWA_DECODE_WAVES
#define SWA_DECODE_WAVES 8   // waves per workgroup (4, 8 or 16)
#endif
#ifndef SWA_DECODE_WG
#define SWA_DECODE_WG 768    // workgroups per step the split count aims for
#endif
constexpr int NWV = SWA_DECODE_WAVES;   // waves per workgroup

// one workgroup of NWV waves per (b, h, split); row group g of a wave handles every
// (NWV * RPW)-th position of the split, U positions per trip: all their loads first, then the U
// scores, then one online-softmax update for the U rows (rows past the split end, re-reading
// the last one, get score -inf and weight 0, without a branch)
template <typename E, int D>
__global__ void __launch_bounds__(64 * NWV) decode_kernel(Params p) {
  using C = Cfg<E, D>;
  constexpr int VPL = C::VPL, LPR = C::LPR, RPW = C::RPW, U = C::U;
  __shared__ float sm[NWV][LPR][VPL + 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x % p.nsplit, bh = blockIdx.x / p.nsplit;
  const int b = bh / p.H, h = bh - b * p.H;
  const int g = lane / LPR, li = lane % LPR;
  const int pp = p.pos[b];
  const int lo = max(0, pp - p.window + 1);
  const int n = pp >= 0 ? pp - lo + 1 : 0;
  const int per = (n + p.nsplit - 1) / p.nsplit;
  const int s0 = lo + split * per, s1 = min(lo + n, s0 + per);

  const E* qn = reinterpret_cast<const E*>(p.qn);
  const E* kc = reinterpret_cast<const E*>(p.kc);
  const E* vc = reinterpret_cast<const E*>(p.vc);
  float qv[VPL];
  load16<E, D>(qn + (size_t)bh * D + li * VPL, qv);
#pragma unroll
  for (int i = 0; i < VPL; ++i) qv[i] *= p.c;

  float m = -INFINITY, l = 0.f, acc[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) acc[i] = 0.f;
  const size_t rs = (size_t)p.H * D;
  const size_t base = ((size_t)b * p.cap * p.H + h) * D + li * VPL;
  constexpr int STRIDE = NWV * RPW;   // positions between a group's consecutive rows
  // trip bound uniform over the wave (the groups' last trips may hold only invalid rows)
  for (int w0 = s0 + wave * RPW; w0 < s1; w0 += STRIDE * U) {
    const int j0 = w0 + g;
    float kv[U][VPL], vv[U][VPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = min(j0 + u * STRIDE, s1 - 1);   // past-the-end rows re-read the last one
      const size_t off = base + (size_t)(j % p.cap) * rs;
      unpack16<E>(ld16_stream(kc + off), kv[u]);
      unpack16<E>(ld16_stream(vc + off), vv[u]);
    }
    float d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i) x = fmaf(qv[i], kv[u][i], x);
      x = group_sum<LPR>(x);   // DPP adds within a 16-lane row
      d[u] = (j0 + u * STRIDE < s1) ? x : -INFINITY;
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mn = fmaxf(mn, d[u]);
    const float ms = (mn == -INFINITY) ? 0.f : mn;   // all -inf so far: every weight is 0
    const float a = __builtin_amdgcn_exp2f(m - ms);
    l *= a;
#pragma unroll
    for (int i = 0; i < VPL; ++i) acc[i] *= a;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float e = __builtin_amdgcn_exp2f(d[u] - ms);
      l += e;
#pragma unroll
      for (int i = 0; i < VPL; ++i) acc[i] = fmaf(e, vv[u][i], acc[i]);
    }
    m = mn;
  }
  // merge the row groups of the wave (lanes li, li + LPR, ...), then the waves via LDS
#pragma unroll
  for (int msk = LPR; msk < 64; msk <<= 1) {
    float a2[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) a2[i] = xor_shfl(acc[i], msk);
    const float m2 = xor_shfl(m, msk), l2 = xor_shfl(l, msk);
    merge(m, l, acc, m2, l2, a2, VPL);
  }
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) sm[wave][li][i] = acc[i];
    sm[wave][li][VPL] = m;
    sm[wave][li][VPL + 1] = l;
  }
  __syncthreads();
  if (wave != 0 || g != 0) return;
  for (int w = 1; w < NWV; ++w) merge(m, l, acc, sm[w][li][VPL], sm[w][li][VPL + 1], sm[w][li], VPL);
  if (p.nsplit == 1) {
    const float inv = 1.f / l;
    E* o = reinterpret_cast<E*>(p.o) + (size_t)bh * D + li * VPL;
#pragma unroll
    for (int i = 0; i < VPL; ++i) o[i] = Elem<E>::from_f(acc[i] * inv);
    if (li == 0) p.lse[bh] = (m + __log2f(l)) * kLn2;
  } else {
    float* pr = p.part + ((size_t)bh * p.nsplit + split) * (D + 2);
#pragma unroll
    for (int i = 0; i < VPL; ++i) pr[li * VPL + i] = acc[i];
    if (li == 0) { pr[D] = m; pr[D + 1] = l; }
  }
}

// merge the splits of each (b, h): one wave per (b, h). Lane s holds split s's running max and
// sum (at most 64 splits), the wave reduces them, and each lane then accumulates dims lane,
// lane + 64 over the splits with the split weights read from their lanes; the loads of the
// splits do not depend on one another, so several are in flight at once.
template <typename E, int D>
__global__ void __launch_bounds__(64) combine_kernel(Params p) {
  const int bh = blockIdx.x, lane = threadIdx.x, ns = p.nsplit;
  const float* pr = p.part + (size_t)bh * ns * (D + 2);
  float ms = -INFINITY, ls = 0.f;
  if (lane < ns) {
    ms = pr[lane * (D + 2) + D];
    ls = pr[lane * (D + 2) + D + 1];
  }
  float M = ms;
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) M = fmaxf(M, xor_shfl(M, k));
  const float w = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
  float L = w * ls;
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) L += xor_shfl(L, k);
  float acc[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) acc[i] = 0.f;
#pragma unroll 8
  for (int s = 0; s < ns; ++s) {
    const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s));
#pragma unroll
    for (int i = 0; i < D / 64; ++i) acc[i] = fmaf(ws, pr[s * (D + 2) + lane + 64 * i], acc[i]);
  }
  E* o = reinterpret_cast<E*>(p.o) + (size_t)bh * D;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) o[lane + 64 * i] = Elem<E>::from_f(acc[i] / L);
  if (lane == 0) p.lse[bh] = (M + __log2f(L)) * kLn2;
}

}  // namespace dec

// Splits per (b, h): about SWA_DECODE_WG workgroups per step, at least 64 window positions per
// split.
int decode_splits(int B, int H, int window) {
  const long bh = (long)B * H;
  int ns = (int)std::min<long>(32, std::max<long>(1, (SWA_DECODE_WG + bh - 1) / bh));
  ns = std::min(ns, std::max(1, window / 64));
  return ns;
}

size_t decode_workspace_bytes(int B, int H, int D, int window) {
  const int ns = decode_splits(B, H, window);
  return ns > 1 ? (size_t)B * H * ns * (D + 2) * sizeof(float) : 256;
}

hipError_t launch_decode_prologue(const void* q, const void* k, const void* v, const float* cs,
                                  int rows, const int* pos, void* qn, void* kc, void* vc, int B,
                                  int H, int D, int cap, float eps, bool is_bf16, hipStream_t s) {
  const int tpr = D * (is_bf16 ? 2 : 4) / 16, rpw = 64 / tpr;   // lanes per row, rows per wave
  const dim3 grid((B * H + rpw - 1) / rpw), blk(64);
#define SWA_DEC_PRO(E, DD)                                                                      \
  hipLaunchKernelGGL((dec::prologue_kernel<E, DD>), grid, blk, 0, s, (const E*)q, (const E*)k, \
                     (const E*)v, cs, rows, pos, (E*)qn, (E*)kc, (E*)vc, H, cap, eps, B * H)
  if (is_bf16) { if (D == 64) SWA_DEC_PRO(bf16, 64); else SWA_DEC_PRO(bf16, 128); }
  else { if (D == 64) SWA_DEC_PRO(float, 64); else SWA_DEC_PRO(float, 128); }
#undef SWA_DEC_PRO
  return hipGetLastError();
}

hipError_t launch_decode(const void* qn, const void* kc, const void* vc, const int* pos, void* o,
                         float* lse, void* ws, int B, int H, int D, int cap, int window,
                         float scale, bool is_bf16, hipStream_t s) {
  dec::Params p;
  p.qn = qn; p.kc = kc; p.vc = vc; p.pos = pos; p.o = o; p.lse = lse;
  p.part = reinterpret_cast<float*>(ws);
  p.H = H; p.cap = cap; p.window = window;
  p.nsplit = decode_splits(B, H, window);
  p.c = scale * kLog2e;
  const dim3 grid(B * H * p.nsplit), blk(64 * dec::NWV), cgrid(B * H), cblk(64);
#define SWA_DEC(E, DD)                                                               \
  do {                                                                               \
    hipLaunchKernelGGL((dec::decode_kernel<E, DD>), grid, blk, 0, s, p);             \
    if (p.nsplit > 1) hipLaunchKernelGGL((dec::combine_kernel<E, DD>), cgrid, cblk, 0, s, p); \
  } while (0)
  if (is_bf16) { if (D == 64) SWA_DEC(bf16, 64); else SWA_DEC(bf16, 128); }
  else { if (D == 64) SWA_DEC(float, 64); else SWA_DEC(float, 128); }
#undef SWA_DEC
  return hipGetLastError();
}

}  // namespace swa

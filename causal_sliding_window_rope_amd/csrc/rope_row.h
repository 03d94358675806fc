// Per-row arithmetic of the RoPE -> RMS QK-norm prologue, shared by the prologue kernels and by
// the attention kernels that run the query half of it in their own prologue / epilogue
// ("从4万美元到73美元：GPT-2复现的成本革命" §2.2: q, k = norm(rope(q)), norm(rope(k)); §2.1: the
// RMSNorm has no learnable parameters).
//
// A row of D elements is held by TPR = D / VPT consecutive lanes, one 128-bit word (VPT
// elements) each; lane j of the group holds elements VPT j .. VPT j + VPT - 1, so the first half
// of the group holds pair indices i < D/2 and the rotation partner of lane j is lane
// j ^ (TPR/2). Every caller that uses these helpers in this layout gets the same bits for a row.
#pragma once
#include "common.h"

namespace swa {

// One 128-bit word of a row: VPT elements as floats.
template <typename E> struct RowWord {
  static constexpr int VPT = 16 / sizeof(E);
  float v[VPT];
  __device__ __forceinline__ void load(const E* p) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    if constexpr (sizeof(E) == 4) {
      v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
      v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
    } else {
      v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
      v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
    }
  }
  // the same with the nontemporal hint (rows read once where they are read)
  __device__ __forceinline__ void load_stream(const E* p) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    if constexpr (sizeof(E) == 4) {
      v[0] = __uint_as_float(w[0]); v[1] = __uint_as_float(w[1]);
      v[2] = __uint_as_float(w[2]); v[3] = __uint_as_float(w[3]);
    } else {
      v[0] = bf_lo(w[0]); v[1] = bf_hi(w[0]); v[2] = bf_lo(w[1]); v[3] = bf_hi(w[1]);
      v[4] = bf_lo(w[2]); v[5] = bf_hi(w[2]); v[6] = bf_lo(w[3]); v[7] = bf_hi(w[3]);
    }
  }
  __device__ __forceinline__ void store(E* p) const {
    uint4 w;
    if constexpr (sizeof(E) == 4) {
      w.x = __float_as_uint(v[0]); w.y = __float_as_uint(v[1]);
      w.z = __float_as_uint(v[2]); w.w = __float_as_uint(v[3]);
    } else {
      w.x = pack_bf2(v[0], v[1]); w.y = pack_bf2(v[2], v[3]);
      w.z = pack_bf2(v[4], v[5]); w.w = pack_bf2(v[6], v[7]);
    }
    *reinterpret_cast<uint4*>(p) = w;
  }
};

// Sum over the TPR lanes that hold one row (TPR is a power of two <= 64, groups aligned).
template <int TPR>
__device__ __forceinline__ float row_sum(float x) {
  return group_sum<TPR>(x);
}

// The rotation partner's value: lane j ^ (TPR/2) of the row group (a DPP row rotation for
// 16-lane groups, a shuffle otherwise).
template <int TPR>
__device__ __forceinline__ float partner(float x) {
  if constexpr (TPR == 16) return dpp_mov<0x128>(x);
  else return xor_shfl(x, TPR / 2);
}

// cos/sin of the VPT angle slots starting at pair index i0 for position t.
template <int VPT>
__device__ __forceinline__ void load_cs(const float* __restrict__ cs, int t, int half, int i0,
                                        float* c, float* s) {
  const float4* p = reinterpret_cast<const float4*>(cs + 2 * ((size_t)t * half + i0));
#pragma unroll
  for (int e = 0; e < VPT / 2; ++e) {
    const float4 w = p[e];
    c[2 * e] = w.x; s[2 * e] = w.y; c[2 * e + 1] = w.z; s[2 * e + 1] = w.w;
  }
}

// Rotate one word: lanes in the first half of the row hold x1 (pair index i < D/2), lanes in
// the second half hold x2; `other` is the partner lane's word. sign = +1 forward, -1 transpose.
template <int VPT>
__device__ __forceinline__ void rotate(float* y, const float* x, const float* other, const float* c,
                                       const float* s, bool second_half, float sign) {
#pragma unroll
  for (int e = 0; e < VPT; ++e) {
    const float ss = sign * s[e];
    // first half: y1 = x1 c - x2 s ; second half: y2 = x1 s + x2 c
    y[e] = second_half ? fmaf(other[e], ss, x[e] * c[e]) : fmaf(-other[e], ss, x[e] * c[e]);
  }
}

// Forward of one row word: y = RoPE_t(x) (x as floats, c/s the word's angles), then
// out = y / sqrt(mean y^2 + eps) over the TPR lanes of the row.
template <int VPT, int TPR, int D>
__device__ __forceinline__ void rope_norm_row(const float* x, const float* c, const float* s,
                                              bool second, float eps, float* out) {
  float other[VPT], y[VPT];
#pragma unroll
  for (int e = 0; e < VPT; ++e) other[e] = partner<TPR>(x[e]);
  rotate<VPT>(y, x, other, c, s, second, 1.0f);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < VPT; ++e) ss = fmaf(y[e], y[e], ss);
  ss = row_sum<TPR>(ss);
  const float rinv = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int e = 0; e < VPT; ++e) out[e] = y[e] * rinv;
}

// Backward of one row word: from the raw row x and the gradient g of the normalised row,
//   du = r (g - x_hat (x_hat . g) / D),  dx = RoPE_t^T(du),  r = (mean u^2 + eps)^(-1/2).
template <int VPT, int TPR, int D>
__device__ __forceinline__ void rope_norm_row_bwd(const float* x, const float* g, const float* c,
                                                  const float* s, bool second, float eps,
                                                  float* dx) {
  float other[VPT], u[VPT];
#pragma unroll
  for (int e = 0; e < VPT; ++e) other[e] = partner<TPR>(x[e]);
  rotate<VPT>(u, x, other, c, s, second, 1.0f);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < VPT; ++e) ss = fmaf(u[e], u[e], ss);
  ss = row_sum<TPR>(ss);
  const float rinv = 1.0f / sqrtf(ss / (float)D + eps);
  float dot = 0.f;
#pragma unroll
  for (int e = 0; e < VPT; ++e) dot = fmaf(u[e] * rinv, g[e], dot);
  dot = row_sum<TPR>(dot);
  const float dd = dot / (float)D;
  float du[VPT];
#pragma unroll
  for (int e = 0; e < VPT; ++e) du[e] = rinv * (g[e] - u[e] * rinv * dd);
#pragma unroll
  for (int e = 0; e < VPT; ++e) other[e] = partner<TPR>(du[e]);
  rotate<VPT>(dx, du, other, c, s, second, -1.0f);
}

}  // namespace swa

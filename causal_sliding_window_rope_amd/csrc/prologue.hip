// RoPE table and the fused RoPE -> RMS QK-norm prologue (forward and backward) for gfx950.
//
// "从4万美元到73美元：GPT-2复现的成本革命" (intelliparadigm.com) §2.2: q, k = norm(rope(q)),
// norm(rope(k)); §2.1: the RMSNorm has no learnable parameters. The rotation is rotate-half:
// pair (i, i + D/2) turns by t * theta_i, theta_i = base^(-2i/D).
//
// These kernels are HBM-bound: one row of D elements per (tensor, b, t, h) is read once and
// written once. A row is spread over D*sizeof(E)/16 lanes so that every lane moves exactly one
// 128-bit word; the rotation partner of lane j is lane j ^ (lanes/2) (a DPP/permute within
// the row's lane group) and the row sum of squares is a butterfly over the same group. In the
// forward a wave walks the H heads of one token, which share the rotation angles; the backward
// (two row reads per row) keeps one row per lane group, which measured faster for it.
#include "common.h"
#include "internal.h"
#include "rope_row.h"

namespace swa {

__global__ void __launch_bounds__(256) rope_table_kernel(float* __restrict__ cs, int T, int D,
                                                         double base) {
  const int half = D / 2;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * half) return;
  const int t = idx / half, i = idx - t * half;
  const double theta = pow(base, -2.0 * (double)i / (double)D);
  const double ang = (double)t * theta;
  cs[2 * idx + 0] = (float)cos(ang);
  cs[2 * idx + 1] = (float)sin(ang);
}

hipError_t launch_rope_table(float* cos_sin, int T, int D, double base, hipStream_t s) {
  const int n = T * (D / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cos_sin, T, D,
                     base);
  return hipGetLastError();
}

// Forward: one wave per (tensor, token). Its 64 / TPR row groups (TPR lanes, one 128-bit word
// each) take consecutive heads, so each load instruction covers a contiguous run of rows, and
// walk the H heads with stride 64 / TPR, U rows per group with their loads issued together.
// The cos/sin of the token's position are loaded once per group for all its heads (a group per
// row re-reads them for every head: four times as many L2 bytes as row bytes).
constexpr int kRowsInFlight = 4;

// OUT8: the normalised rows are written as e4m3 codes (scale 1; every entry of a normalised
// row is below sqrt(D) <= 11.4 in magnitude, far inside e4m3's range, so no saturation) for
// the fp8 forward; qn / kn then point to bytes.
template <typename E, int D, bool OUT8>
__global__ void __launch_bounds__(256) rope_qknorm_fwd_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const float* __restrict__ cs,
    void* __restrict__ qn, void* __restrict__ kn, int tokens, int T, int H, float eps, int wv0) {
  using W = RowWord<E>;
  constexpr int VPT = W::VPT, TPR = D / VPT, HALF_T = TPR / 2, U = kRowsInFlight;
  constexpr int GPW = 64 / TPR;   // row groups per wave = head stride
  const int lane_in_row = threadIdx.x % TPR;
  const int gw = (threadIdx.x % 64) / TPR;
  const int wv = wv0 + blockIdx.x * 4 + threadIdx.x / 64;   // wv0 = tokens: k only
  if (wv >= 2 * tokens) return;  // whole waves exit together
  const bool is_k = wv >= tokens;
  const int bt = is_k ? wv - tokens : wv;
  const int t = bt % T;
  const E* src = is_k ? k : q;
  const bool second = lane_in_row >= HALF_T;
  float c[VPT], s[VPT];
  load_cs<VPT>(cs, t, D / 2, (lane_in_row % HALF_T) * VPT, c, s);
  for (int h0 = gw; h0 < H; h0 += GPW * U) {
    W x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int h = min(h0 + GPW * u, H - 1);   // past the last head: re-read it, store nothing
      x[u].load(src + ((size_t)bt * H + h) * D + lane_in_row * VPT);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (h0 + GPW * u >= H) break;
      const size_t off = ((size_t)bt * H + h0 + GPW * u) * D + lane_in_row * VPT;
      W out;
      rope_norm_row<VPT, TPR, D>(x[u].v, c, s, second, eps, out.v);
      if constexpr (OUT8) {
        unsigned w[VPT / 4];
#pragma unroll
        for (int j = 0; j < VPT / 4; ++j) {
          const unsigned lo =
              __builtin_amdgcn_cvt_pk_fp8_f32(out.v[4 * j], out.v[4 * j + 1], 0u, false);
          w[j] = __builtin_amdgcn_cvt_pk_fp8_f32(out.v[4 * j + 2], out.v[4 * j + 3], lo, true);
        }
        unsigned char* dst = static_cast<unsigned char*>(is_k ? kn : qn) + off;
        if constexpr (VPT == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
        else *reinterpret_cast<unsigned*>(dst) = w[0];
      } else {
        out.store(static_cast<E*>(is_k ? kn : qn) + off);
      }
    }
  }
}

template <typename E, int D>
__global__ void __launch_bounds__(256) rope_qknorm_bwd_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const float* __restrict__ cs,
    const E* __restrict__ dqn, const E* __restrict__ dkn, E* __restrict__ dq, E* __restrict__ dk,
    int rows_per_tensor, int T, int H, float eps, int row0) {
  using W = RowWord<E>;
  constexpr int VPT = W::VPT, TPR = D / VPT, HALF_T = TPR / 2;
  const int lane_in_row = threadIdx.x % TPR;
  const int row = row0 + blockIdx.x * (256 / TPR) + threadIdx.x / TPR;   // row0 > 0: k only
  if (row >= 2 * rows_per_tensor) return;
  const bool is_k = row >= rows_per_tensor;
  const int r = is_k ? row - rows_per_tensor : row;
  const int t = (r / H) % T;
  const size_t off = (size_t)r * D + lane_in_row * VPT;
  W x, g;
  x.load((is_k ? k : q) + off);
  g.load((is_k ? dkn : dqn) + off);
  const bool second = lane_in_row >= HALF_T;
  float c[VPT], s[VPT];
  load_cs<VPT>(cs, t, D / 2, (lane_in_row % HALF_T) * VPT, c, s);
  W out;
  rope_norm_row_bwd<VPT, TPR, D>(x.v, g.v, c, s, second, eps, out.v);
  // dq, dk are the step's final outputs: written with the nontemporal hint, so that they do
  // not displace what the next layer's backward kernels re-read (its row-term pass ~13 %
  // faster on the d24 sweep)
  if constexpr (sizeof(E) == 2) {
    const u32x4 w = {pack_bf2(out.v[0], out.v[1]), pack_bf2(out.v[2], out.v[3]),
                     pack_bf2(out.v[4], out.v[5]), pack_bf2(out.v[6], out.v[7])};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>((is_k ? dk : dq) + off));
  } else {
    out.store((is_k ? dk : dq) + off);
  }
}

template <typename E, int D, bool OUT8 = false>
static hipError_t launch_fwd_t(const void* q, const void* k, const float* cs, void* qn, void* kn,
                               int B, int T, int H, float eps, hipStream_t s) {
  const int tokens = B * T;
  const int wv0 = q ? 0 : tokens;   // no q: the k rows only
  const int blocks = (2 * tokens - wv0 + 3) / 4;   // one wave per (tensor, token)
  hipLaunchKernelGGL((rope_qknorm_fwd_kernel<E, D, OUT8>), dim3(blocks), dim3(256), 0, s,
                     (const E*)q, (const E*)k, cs, qn, kn, tokens, T, H, eps, wv0);
  return hipGetLastError();
}

hipError_t launch_rope_qknorm_fwd_fp8(const void* q, const void* k, const float* cs, void* q8,
                                      void* k8, int B, int T, int H, int D, float eps, bool bf16,
                                      hipStream_t s) {
  if (bf16) {
    return D == 64 ? launch_fwd_t<swa::bf16, 64, true>(q, k, cs, q8, k8, B, T, H, eps, s)
                   : launch_fwd_t<swa::bf16, 128, true>(q, k, cs, q8, k8, B, T, H, eps, s);
  }
  return D == 64 ? launch_fwd_t<float, 64, true>(q, k, cs, q8, k8, B, T, H, eps, s)
                 : launch_fwd_t<float, 128, true>(q, k, cs, q8, k8, B, T, H, eps, s);
}

template <typename E, int D>
static hipError_t launch_bwd_t(const void* q, const void* k, const float* cs, const void* dqn,
                               const void* dkn, void* dq, void* dk, int B, int T, int H, float eps,
                               hipStream_t s) {
  constexpr int TPR = D / (16 / sizeof(E));
  const int rows = B * T * H;
  const int rpb = 256 / TPR;
  const int row0 = q ? 0 : rows;   // no q: the k rows only
  const int blocks = (2 * rows - row0 + rpb - 1) / rpb;
  hipLaunchKernelGGL((rope_qknorm_bwd_kernel<E, D>), dim3(blocks), dim3(256), 0, s,
                     (const E*)q, (const E*)k, cs, (const E*)dqn, (const E*)dkn, (E*)dq, (E*)dk,
                     rows, T, H, eps, row0);
  return hipGetLastError();
}

hipError_t launch_rope_qknorm_fwd(const void* q, const void* k, const float* cs, void* qn, void* kn,
                                  int B, int T, int H, int D, float eps, bool bf16, hipStream_t s) {
  if (bf16) {
    return D == 64 ? launch_fwd_t<swa::bf16, 64>(q, k, cs, qn, kn, B, T, H, eps, s)
                   : launch_fwd_t<swa::bf16, 128>(q, k, cs, qn, kn, B, T, H, eps, s);
  }
  return D == 64 ? launch_fwd_t<float, 64>(q, k, cs, qn, kn, B, T, H, eps, s)
                 : launch_fwd_t<float, 128>(q, k, cs, qn, kn, B, T, H, eps, s);
}

hipError_t launch_rope_qknorm_bwd(const void* q, const void* k, const float* cs, const void* dqn,
                                  const void* dkn, void* dq, void* dk, int B, int T, int H, int D,
                                  float eps, bool bf16, hipStream_t s) {
  if (bf16) {
    return D == 64 ? launch_bwd_t<swa::bf16, 64>(q, k, cs, dqn, dkn, dq, dk, B, T, H, eps, s)
                   : launch_bwd_t<swa::bf16, 128>(q, k, cs, dqn, dkn, dq, dk, B, T, H, eps, s);
  }
  return D == 64 ? launch_bwd_t<float, 64>(q, k, cs, dqn, dkn, dq, dk, B, T, H, eps, s)
                 : launch_bwd_t<float, 128>(q, k, cs, dqn, dkn, dq, dk, B, T, H, eps, s);
}

}  // namespace swa

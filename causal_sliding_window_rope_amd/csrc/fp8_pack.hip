// Packing of q, k, v into the e4m3 operands of the fp8 forward (fp8.hip).
//
// Format and calibration ("NanoGPT Speedrun：大模型训练效率的极限竞速指南", kongchang.com,
// section "工程与硬件优化", its paragraph on bf16 and fp8: fp8 needs finer calibration to stay
// accurate): OCP e4m3, one float32 scale per tensor,
// code = e4m3(x * (1/scale)) with one float32 multiply and one nearest-even rounding,
// saturating finite values beyond 448 (the conversion instruction itself would give NaN there)
// and keeping NaN. This file is compiled with NaN semantics honoured (the rest of the library
// is not), so the NaN test below is not folded away.
//
// v is written transposed per (b, h) (a D x Tp byte matrix, Tp = T rounded up to 64) with the
// keys of every 64-key block permuted into the order in which the forward kernel's
// probabilities leave its score accumulators: byte 32g + 16kb + 4a + c of a block holds key
// 32kb + 8a + 4g + c. Keys >= T are 0.
#include "common.h"
#include "internal.h"

namespace swa {

namespace f8p {

constexpr float kE4m3Max = 448.0f;

// Saturating conversion of two floats to e4m3 codes in half `hi` of `old` (NaN stays NaN; the
// instruction itself turns values beyond the largest finite code into NaN).
__device__ __forceinline__ unsigned cvt2(float a, float b, unsigned old, bool hi) {
  a = __builtin_isnan(a) ? a : fminf(fmaxf(a, -kE4m3Max), kE4m3Max);
  b = __builtin_isnan(b) ? b : fminf(fmaxf(b, -kE4m3Max), kE4m3Max);
  return hi ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true)
            : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}

// Four floats -> one dword of e4m3 codes (lowest index in the lowest byte).
__device__ __forceinline__ unsigned pack4(float a, float b, float c, float d) {
  return cvt2(c, d, cvt2(a, b, 0u, false), true);
}

// x8 = e4m3(x * inv), 16 elements per thread.
template <typename E>
__global__ void __launch_bounds__(256) quant_kernel(const E* __restrict__ x,
                                                    uint4* __restrict__ x8, float inv,
                                                    size_t n16) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  constexpr int VPT = 16 / sizeof(E);
  float v[16];
#pragma unroll
  for (int w = 0; w < 16 / VPT; ++w) {
    float t[VPT];
    unpack16(reinterpret_cast<const uint4*>(x)[i * (16 / VPT) + w], t);
#pragma unroll
    for (int j = 0; j < VPT; ++j) v[w * VPT + j] = t[j] * inv;
  }
  x8[i] = make_uint4(pack4(v[0], v[1], v[2], v[3]), pack4(v[4], v[5], v[6], v[7]),
                     pack4(v[8], v[9], v[10], v[11]), pack4(v[12], v[13], v[14], v[15]));
}

// v (B, T, H, D) -> v8t: one workgroup per (64-key block, b, h). Phase 1 reads the block's rows
// coalesced, quantises them and stores the codes key-major in LDS (rows padded to D + 4 bytes);
// phase 2 assembles each 16-byte chunk of a v8t row (one dimension d, 16 stored positions) from
// the 16 keys it holds. With the padding the byte reads of one wave fall in distinct banks.
template <typename E, int D>
__global__ void __launch_bounds__(256) vpack_kernel(const E* __restrict__ v,
                                                    uint4* __restrict__ v8t, float inv, int T,
                                                    int H, int Tp) {
  constexpr int RS = D + 4;    // LDS row stride in bytes
  __shared__ unsigned tile32[64 * RS / 4];
  unsigned char* tile = reinterpret_cast<unsigned char*>(tile32);
  const int kt = blockIdx.y, bh = blockIdx.x, b = bh / H, h = bh - b * H;
  constexpr int CPR = D / 8;   // 8-element chunks per key row
  for (int i = threadIdx.x; i < 64 * CPR; i += 256) {
    const int key = i / CPR, c = i - key * CPR;
    const int t = kt * 64 + key;
    float f[8];
    if (t < T) {
      const E* src = v + (((size_t)b * T + t) * H + h) * D + 8 * c;
      if constexpr (sizeof(E) == 2) {
        unpack16(*reinterpret_cast<const uint4*>(src), f);
      } else {
        float a[4], bq[4];
        unpack16(reinterpret_cast<const uint4*>(src)[0], a);
        unpack16(reinterpret_cast<const uint4*>(src)[1], bq);
#pragma unroll
        for (int j = 0; j < 4; ++j) { f[j] = a[j]; f[4 + j] = bq[j]; }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = 0.f;
    }
    unsigned* dst = reinterpret_cast<unsigned*>(tile + key * RS + 8 * c);
    dst[0] = pack4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
    dst[1] = pack4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < D * 4; i += 256) {
    const int d = i >> 2, cc = i & 3;
    // stored position 16 cc + j holds key 32 (cc & 1) + 8 (j >> 2) + 4 (cc >> 1) + (j & 3)
    const int kbase = 32 * (cc & 1) + 4 * (cc >> 1);
    unsigned w[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      unsigned x = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) x |= (unsigned)tile[(kbase + 8 * a + c) * RS + d] << (8 * c);
      w[a] = x;
    }
    v8t[((((size_t)b * H + h) * D + d) * Tp + (size_t)kt * 64) / 16 + cc] =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace f8p

size_t fp8_v_bytes(int B, int T, int H, int D) {
  const size_t Tp = ((size_t)T + 63) / 64 * 64;
  return (size_t)B * H * D * Tp;
}

template <typename E>
static void quant_t(const void* x, void* x8, float inv, size_t n, hipStream_t s) {
  const size_t n16 = n / 16;
  hipLaunchKernelGGL(f8p::quant_kernel<E>, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                     (const E*)x, (uint4*)x8, inv, n16);
}

template <typename E>
static void vpack_t(const void* v, void* v8t, float inv, int B, int T, int H, int D,
                    hipStream_t s) {
  const int Tp = (T + 63) / 64 * 64;
  const dim3 grid(B * H, Tp / 64);   // the heads of one key block in neighbouring workgroups
  if (D == 64)
    hipLaunchKernelGGL((f8p::vpack_kernel<E, 64>), grid, dim3(256), 0, s, (const E*)v,
                       (uint4*)v8t, inv, T, H, Tp);
  else
    hipLaunchKernelGGL((f8p::vpack_kernel<E, 128>), grid, dim3(256), 0, s, (const E*)v,
                       (uint4*)v8t, inv, T, H, Tp);
}

hipError_t launch_fp8_pack(const void* q, const void* k, const void* v, float q_inv, float k_inv,
                           float v_inv, void* q8, void* k8, void* v8t, int B, int T, int H,
                           int D, bool bf16, hipStream_t s) {
  const size_t n = (size_t)B * T * H * D;
  if (bf16) {
    if (q) quant_t<swa::bf16>(q, q8, q_inv, n, s);
    if (k) quant_t<swa::bf16>(k, k8, k_inv, n, s);
    if (v) vpack_t<swa::bf16>(v, v8t, v_inv, B, T, H, D, s);
  } else {
    if (q) quant_t<float>(q, q8, q_inv, n, s);
    if (k) quant_t<float>(k, k8, k_inv, n, s);
    if (v) vpack_t<float>(v, v8t, v_inv, B, T, H, D, s);
  }
  return hipGetLastError();
}

}  // namespace swa

// Value-embedding gate for gfx950 (lanjinlin.com.cn repost of the nanochat d24 write-up,
// "3. Value Embeddings"): gate = 2 * sigmoid(ve_gate(x[:, :, :32])), v = v + gate * ve,
// with ve_gate a bias-free 32 -> H projection, one gate per head broadcast over D.
//
// The gate itself is tiny (32 MACs per (b, t, h)); the optional v_eff materialisation is a
// 128-bit streaming kernel. The backward reduces dWg over all B*T rows in a fixed order: one
// workgroup per (c, h) entry, strided per-thread partial sums, then a tree over the block.
#include "common.h"
#include "internal.h"

namespace swa {

template <typename E>
__global__ void __launch_bounds__(256) gate_kernel(const E* __restrict__ x, int ldx,
                                                   const float* __restrict__ Wg,
                                                   float* __restrict__ gate, int rows, int H) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * H) return;
  const int n = idx / H, h = idx - n * H;
  const E* xr = x + (size_t)n * ldx;
  float z = 0.f;
#pragma unroll 8
  for (int c = 0; c < 32; ++c) z = fmaf(Elem<E>::to_f(xr[c]), Wg[c * H + h], z);
  gate[idx] = 2.0f / (1.0f + expf(-z));
}

// v_eff = v + gate * ve; one lane per 128-bit word, D/VPT words per (b, t, h) row.
template <typename E>
__global__ void __launch_bounds__(256) apply_gate_kernel(const E* __restrict__ v,
                                                         const E* __restrict__ ve,
                                                         const float* __restrict__ gate,
                                                         E* __restrict__ v_eff, size_t words,
                                                         int words_per_row) {
  constexpr int VPT = 16 / sizeof(E);
  const size_t w = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= words) return;
  const float g = gate[w / words_per_row];
  const uint4 a = reinterpret_cast<const uint4*>(v)[w];
  const uint4 b = reinterpret_cast<const uint4*>(ve)[w];
  uint4 o;
  if constexpr (VPT == 4) {
    o.x = __float_as_uint(fmaf(g, __uint_as_float(b.x), __uint_as_float(a.x)));
    o.y = __float_as_uint(fmaf(g, __uint_as_float(b.y), __uint_as_float(a.y)));
    o.z = __float_as_uint(fmaf(g, __uint_as_float(b.z), __uint_as_float(a.z)));
    o.w = __float_as_uint(fmaf(g, __uint_as_float(b.w), __uint_as_float(a.w)));
  } else {
    o.x = pack_bf2(fmaf(g, bf_lo(b.x), bf_lo(a.x)), fmaf(g, bf_hi(b.x), bf_hi(a.x)));
    o.y = pack_bf2(fmaf(g, bf_lo(b.y), bf_lo(a.y)), fmaf(g, bf_hi(b.y), bf_hi(a.y)));
    o.z = pack_bf2(fmaf(g, bf_lo(b.z), bf_lo(a.z)), fmaf(g, bf_hi(b.z), bf_hi(a.z)));
    o.w = pack_bf2(fmaf(g, bf_lo(b.w), bf_lo(a.w)), fmaf(g, bf_hi(b.w), bf_hi(a.w)));
  }
  reinterpret_cast<uint4*>(v_eff)[w] = o;
}

// dWg[c, h] = sum_n x[n, c] * dz[n, h], dz = dgate * g * (1 - g/2). One block per (c, h).
template <typename E>
__global__ void __launch_bounds__(256) gate_dw_kernel(const E* __restrict__ x, int ldx,
                                                      const float* __restrict__ gate,
                                                      const float* __restrict__ dgate,
                                                      float* __restrict__ dWg, int rows, int H) {
  const int c = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  float acc = 0.f;
  for (int n = threadIdx.x; n < rows; n += 256) {
    const float g = gate[(size_t)n * H + h];
    const float dz = dgate[(size_t)n * H + h] * g * (1.0f - 0.5f * g);
    acc = fmaf(Elem<E>::to_f(x[(size_t)n * ldx + c]), dz, acc);
  }
  __shared__ float red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
#pragma unroll
  for (int m = 128; m > 0; m >>= 1) {
    if ((int)threadIdx.x < m) red[threadIdx.x] += red[threadIdx.x + m];
    __syncthreads();
  }
  if (threadIdx.x == 0) dWg[c * H + h] = red[0];
}

// dx32[n, c] = sum_h dz[n, h] * Wg[c, h].
template <typename E>
__global__ void __launch_bounds__(256) gate_dx_kernel(const float* __restrict__ Wg,
                                                      const float* __restrict__ gate,
                                                      const float* __restrict__ dgate,
                                                      E* __restrict__ dx32, int rows, int H) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * 32) return;
  const int n = idx / 32, c = idx % 32;
  float acc = 0.f;
  for (int h = 0; h < H; ++h) {
    const float g = gate[(size_t)n * H + h];
    const float dz = dgate[(size_t)n * H + h] * g * (1.0f - 0.5f * g);
    acc = fmaf(dz, Wg[c * H + h], acc);
  }
  dx32[idx] = Elem<E>::from_f(acc);
}

template <typename E>
static hipError_t gate_t(const void* x, int ldx, const float* Wg, float* gate, const void* v,
                         const void* ve, void* v_eff, int B, int T, int H, int D, hipStream_t s) {
  const int rows = B * T;
  hipLaunchKernelGGL(gate_kernel<E>, dim3((rows * H + 255) / 256), dim3(256), 0, s, (const E*)x,
                     ldx, Wg, gate, rows, H);
  if (v_eff) {
    constexpr int VPT = 16 / sizeof(E);
    const size_t words = (size_t)rows * H * D / VPT;
    hipLaunchKernelGGL(apply_gate_kernel<E>, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                       s, (const E*)v, (const E*)ve, gate, (E*)v_eff, words, D / VPT);
  }
  return hipGetLastError();
}

template <typename E>
static hipError_t gate_bwd_t(const void* x, int ldx, const float* Wg, const float* gate,
                             const float* dgate, float* dWg, void* dx32, int B, int T, int H,
                             hipStream_t s) {
  const int rows = B * T;
  hipLaunchKernelGGL(gate_dw_kernel<E>, dim3(32 * H), dim3(256), 0, s, (const E*)x, ldx, gate,
                     dgate, dWg, rows, H);
  if (dx32) {
    hipLaunchKernelGGL(gate_dx_kernel<E>, dim3((rows * 32 + 255) / 256), dim3(256), 0, s, Wg, gate,
                       dgate, (E*)dx32, rows, H);
  }
  return hipGetLastError();
}

hipError_t launch_ve_gate(const void* x, int ldx, const float* Wg, float* gate, const void* v,
                          const void* ve, void* v_eff, int B, int T, int H, int D, bool bf16,
                          hipStream_t s) {
  return bf16 ? gate_t<swa::bf16>(x, ldx, Wg, gate, v, ve, v_eff, B, T, H, D, s)
              : gate_t<float>(x, ldx, Wg, gate, v, ve, v_eff, B, T, H, D, s);
}

hipError_t launch_ve_gate_bwd(const void* x, int ldx, const float* Wg, const float* gate,
                              const float* dgate, float* dWg, void* dx32, int B, int T, int H,
                              bool bf16, hipStream_t s) {
  return bf16 ? gate_bwd_t<swa::bf16>(x, ldx, Wg, gate, dgate, dWg, dx32, B, T, H, s)
              : gate_bwd_t<float>(x, ldx, Wg, gate, dgate, dWg, dx32, B, T, H, s);
}

}  // namespace swa

// Value-embedding gate for gfx950 (lanjinlin.com.cn repost of the nanochat d24 write-up,
// "3. Value Embeddings"): gate = 2 * sigmoid(ve_gate(x[:, :, :32])), v = v + gate * ve,
// with ve_gate a bias-free 32 -> H projection, one gate per head broadcast over D.
//
// The gate itself is tiny (32 MACs per (b, t, h)); the optional v_eff materialisation and its
// backward (dve = gate * dv_eff, dgate = sum_d dv_eff * ve) are 128-bit streaming kernels. In
// the table mode the per-layer embedding is a lookup of the token ids: ve rows are gathered from
// a (rows, H*D) table and dve is added into the table's float gradient. The gate's backward
// reduces dWg over all B*T rows in a fixed order (bitwise repeatable).
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

// The ve word c of (b, t, h) row r = (b*T + t)*H + h: from the per-token (B, T, H*D) tensor, or
// from table row ids[r / H] (nullptr for an id outside the table: a zero row).
template <typename E, int WPR>
__device__ __forceinline__ const uint4* ve_word(const E* ve, const int* ids, int rows, size_t r,
                                                int c, int H) {
  if (!ids) return reinterpret_cast<const uint4*>(ve) + r * WPR + c;
  const size_t n = r / H;
  const int id = ids[n];
  if ((unsigned)id >= (unsigned)rows) return nullptr;
  return reinterpret_cast<const uint4*>(ve) + ((size_t)id * H + (r - n * H)) * WPR + c;
}

// v_eff = v + gate * ve; one lane per 128-bit word, WPR words per (b, t, h) row.
template <typename E, int WPR>
__global__ void __launch_bounds__(256) apply_gate_kernel(const E* __restrict__ v,
                                                         const E* __restrict__ ve,
                                                         const int* __restrict__ ids, int rows,
                                                         const float* __restrict__ gate,
                                                         E* __restrict__ v_eff, size_t words,
                                                         int H) {
  constexpr int VPT = 16 / sizeof(E);
  const size_t w = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= words) return;
  const size_t r = w / WPR;
  const float g = gate[r];
  const uint4 a = reinterpret_cast<const uint4*>(v)[w];
  const uint4* pe = ve_word<E, WPR>(ve, ids, rows, r, (int)(w - r * WPR), H);
  const uint4 b = pe ? *pe : make_uint4(0, 0, 0, 0);
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

// Backward of v_eff = v + gate * ve through ve and gate: dve = gate * dv_eff (per token, or
// added into the float table gradient at the token's id) and dgate = sum_d dv_eff * ve. One lane
// per 128-bit word; the WPR lanes of a row (aligned groups inside a wave) reduce dgate.
template <typename E, int WPR>
__global__ void __launch_bounds__(256) gate_dv_kernel(const E* __restrict__ dv,
                                                      const E* __restrict__ ve,
                                                      const int* __restrict__ ids, int rows,
                                                      const float* __restrict__ gate,
                                                      E* __restrict__ dve, float* __restrict__ dtab,
                                                      float* __restrict__ dgate, size_t words,
                                                      int H) {
  constexpr int VPT = 16 / sizeof(E);
  const size_t w = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool ok = w < words;   // no early exit: every lane of a row group joins the reduction
  const size_t r = w / WPR;
  const int c = (int)(w - r * WPR);
  float a[VPT], e[VPT];
  const uint4* pe = nullptr;
  float g = 0.f;
  if (ok) {
    g = gate[r];
    const uint4 av = reinterpret_cast<const uint4*>(dv)[w];
    pe = ve_word<E, WPR>(ve, ids, rows, r, c, H);
    const uint4 ev = pe ? *pe : make_uint4(0, 0, 0, 0);
    unpack16(av, a);
    unpack16(ev, e);
  } else {
#pragma unroll
    for (int i = 0; i < VPT; ++i) a[i] = e[i] = 0.f;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) s = fmaf(a[i], e[i], s);
  s = group_sum<WPR>(s);   // DPP adds within a 16-lane row
  if (!ok) return;
  if (c == 0) dgate[r] = s;
  if (!ids) {
    float o[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) o[i] = g * a[i];
    reinterpret_cast<uint4*>(dve)[w] = pack16(o);
  } else if (pe) {
    float* dst = dtab + (reinterpret_cast<const E*>(pe) - ve);
#pragma unroll
    for (int i = 0; i < VPT; ++i) atomicAdd(dst + i, g * a[i]);
  }
}

// Table mode of the same backward: one wave per (b, t, h) row, lane l owning elements l + 64 e,
// so each float atomic instruction adds into 64 consecutive floats of the table row (two cache
// lines) instead of 64 scattered words.
template <typename E, int D>
__global__ void __launch_bounds__(256) gate_dv_table_kernel(const E* __restrict__ dv,
                                                            const E* __restrict__ ve,
                                                            const int* __restrict__ ids, int rows,
                                                            const float* __restrict__ gate,
                                                            float* __restrict__ dtab,
                                                            float* __restrict__ dgate,
                                                            size_t nrows, int H) {
  constexpr int PER = D / 64;
  const size_t r = (size_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (r >= nrows) return;   // r is uniform across the wave
  const size_t n = r / H;
  const int id = ids[n];
  const bool valid = (unsigned)id < (unsigned)rows;
  const float g = gate[r];
  const size_t eoff = ((size_t)(valid ? id : 0) * H + (r - n * H)) * D;
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int d = lane + 64 * e;
    const float a = Elem<E>::to_f(dv[r * D + d]);
    if (valid) {
      s = fmaf(a, Elem<E>::to_f(ve[eoff + d]), s);
      atomicAdd(dtab + eoff + d, g * a);
    }
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) s += xor_shfl(s, m);
  if (lane == 0) dgate[r] = s;
}

// dWg[c, h] = sum_n x[n, c] * dz[n, h], dz = dgate * g * (1 - g/2), in two passes with a fixed
// summation order (bitwise repeatable). Pass 1: block k stages rows [128k, 128k + 128) of x's 32
// gate channels and of dz in LDS and writes the chunk's 32 x H partial sums to the workspace.
// Pass 2: one wave per (c, h): lane l adds chunks l, l + 64, ... in order, then a fixed shuffle
// tree combines the lanes.
constexpr int kDwRows = 128;

template <typename E, bool VEC>
__global__ void __launch_bounds__(256) gate_dw_partial_kernel(const E* __restrict__ x, int ldx,
                                                              const float* __restrict__ gate,
                                                              const float* __restrict__ dgate,
                                                              float* __restrict__ part, int rows,
                                                              int H) {
  extern __shared__ float sm[];
  float* xs = sm;                       // [kDwRows][33] (padded: column reads hit distinct banks)
  float* dz = sm + kDwRows * 33;        // [kDwRows][H]
  const int n0 = blockIdx.x * kDwRows;
  const int nr = min(kDwRows, rows - n0);
  if constexpr (VEC) {
    constexpr int VPT = 16 / sizeof(E), WPR = 32 / VPT;   // 128-bit words per row
#pragma unroll
    for (int j = 0; j < kDwRows * WPR / 256; ++j) {
      const int i = threadIdx.x + 256 * j;
      const int r = i / WPR, w = i % WPR;
      float v[VPT];
      if (r < nr) {
        unpack16(reinterpret_cast<const uint4*>(x + (size_t)(n0 + r) * ldx)[w], v);
      } else {
#pragma unroll
        for (int k = 0; k < VPT; ++k) v[k] = 0.f;
      }
#pragma unroll
      for (int k = 0; k < VPT; ++k) xs[r * 33 + w * VPT + k] = v[k];
    }
  } else {
    for (int i = threadIdx.x; i < kDwRows * 32; i += 256) {
      const int r = i / 32, c = i % 32;
      xs[r * 33 + c] = r < nr ? Elem<E>::to_f(x[(size_t)(n0 + r) * ldx + c]) : 0.f;
    }
  }
  for (int i = threadIdx.x; i < kDwRows * H; i += 256) {
    const int r = i / H;
    float v = 0.f;
    if (r < nr) {
      const float g = gate[(size_t)n0 * H + i];
      v = dgate[(size_t)n0 * H + i] * g * (1.0f - 0.5f * g);
    }
    dz[i] = v;
  }
  __syncthreads();
  for (int pidx = threadIdx.x; pidx < 32 * H; pidx += 256) {
    const int c = pidx / H, h = pidx - c * H;
    float acc = 0.f;
#pragma unroll 8
    for (int r = 0; r < kDwRows; ++r) acc = fmaf(xs[r * 33 + c], dz[r * H + h], acc);
    part[(size_t)blockIdx.x * 32 * H + pidx] = acc;
  }
}

__global__ void __launch_bounds__(256) gate_dw_reduce_kernel(const float* __restrict__ part,
                                                             float* __restrict__ dWg, int chunks,
                                                             int n) {
  const int pidx = blockIdx.x * 4 + threadIdx.x / 64;   // uniform across the wave
  const int lane = threadIdx.x & 63;
  if (pidx >= n) return;
  float acc = 0.f;
  for (int k = lane; k < chunks; k += 64) acc += part[(size_t)k * n + pidx];
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) acc += xor_shfl(acc, m);
  if (lane == 0) dWg[pidx] = acc;
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
                         const void* ve, const int* ids, int ve_rows, void* v_eff, int B, int T,
                         int H, int D, hipStream_t s) {
  const int rows = B * T;
  hipLaunchKernelGGL(gate_kernel<E>, dim3((rows * H + 255) / 256), dim3(256), 0, s, (const E*)x,
                     ldx, Wg, gate, rows, H);
  if (v_eff) {
    constexpr int VPT = 16 / sizeof(E);
    const size_t words = (size_t)rows * H * D / VPT;
    const dim3 grid((unsigned)((words + 255) / 256));
    if (D == 64)
      hipLaunchKernelGGL((apply_gate_kernel<E, 64 / VPT>), grid, dim3(256), 0, s, (const E*)v,
                         (const E*)ve, ids, ve_rows, gate, (E*)v_eff, words, H);
    else
      hipLaunchKernelGGL((apply_gate_kernel<E, 128 / VPT>), grid, dim3(256), 0, s, (const E*)v,
                         (const E*)ve, ids, ve_rows, gate, (E*)v_eff, words, H);
  }
  return hipGetLastError();
}

template <typename E>
static hipError_t gate_dv_t(const void* dv, const void* ve, const int* ids, int ve_rows,
                            const float* gate, void* dve, float* dgate, int B, int T, int H, int D,
                            hipStream_t s) {
  constexpr int VPT = 16 / sizeof(E);
  if (ids) {
    const size_t nrows = (size_t)B * T * H;
    const dim3 tgrid((unsigned)((nrows + 3) / 4));
    if (D == 64)
      hipLaunchKernelGGL((gate_dv_table_kernel<E, 64>), tgrid, dim3(256), 0, s, (const E*)dv,
                         (const E*)ve, ids, ve_rows, gate, (float*)dve, dgate, nrows, H);
    else
      hipLaunchKernelGGL((gate_dv_table_kernel<E, 128>), tgrid, dim3(256), 0, s, (const E*)dv,
                         (const E*)ve, ids, ve_rows, gate, (float*)dve, dgate, nrows, H);
    return hipGetLastError();
  }
  const size_t words = (size_t)B * T * H * D / VPT;
  const dim3 grid((unsigned)((words + 255) / 256));
  E* dve_e = (E*)dve;
  float* dtab = nullptr;
  if (D == 64)
    hipLaunchKernelGGL((gate_dv_kernel<E, 64 / VPT>), grid, dim3(256), 0, s, (const E*)dv,
                       (const E*)ve, ids, ve_rows, gate, dve_e, dtab, dgate, words, H);
  else
    hipLaunchKernelGGL((gate_dv_kernel<E, 128 / VPT>), grid, dim3(256), 0, s, (const E*)dv,
                       (const E*)ve, ids, ve_rows, gate, dve_e, dtab, dgate, words, H);
  return hipGetLastError();
}

size_t gate_bwd_workspace_bytes(int B, int T, int H) {
  const size_t chunks = ((size_t)B * T + kDwRows - 1) / kDwRows;
  return chunks * 32 * H * sizeof(float);
}

template <typename E>
static hipError_t gate_bwd_t(const void* x, int ldx, const float* Wg, const float* gate,
                             const float* dgate, float* dWg, void* dx32, void* ws, int B, int T,
                             int H, hipStream_t s) {
  const int rows = B * T;
  const int chunks = (rows + kDwRows - 1) / kDwRows;
  const size_t lds = (size_t)kDwRows * (33 + H) * sizeof(float);
  const bool vec =
      reinterpret_cast<uintptr_t>(x) % 16 == 0 && ((size_t)ldx * sizeof(E)) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((gate_dw_partial_kernel<E, true>), dim3(chunks), dim3(256), lds, s,
                       (const E*)x, ldx, gate, dgate, (float*)ws, rows, H);
  else
    hipLaunchKernelGGL((gate_dw_partial_kernel<E, false>), dim3(chunks), dim3(256), lds, s,
                       (const E*)x, ldx, gate, dgate, (float*)ws, rows, H);
  hipLaunchKernelGGL(gate_dw_reduce_kernel, dim3((32 * H + 3) / 4), dim3(256), 0, s,
                     (const float*)ws, dWg, chunks, 32 * H);
  if (dx32) {
    hipLaunchKernelGGL(gate_dx_kernel<E>, dim3((rows * 32 + 255) / 256), dim3(256), 0, s, Wg, gate,
                       dgate, (E*)dx32, rows, H);
  }
  return hipGetLastError();
}

hipError_t launch_ve_gate(const void* x, int ldx, const float* Wg, float* gate, const void* v,
                          const void* ve, const int* ids, int ve_rows, void* v_eff, int B, int T,
                          int H, int D, bool bf16, hipStream_t s) {
  return bf16 ? gate_t<swa::bf16>(x, ldx, Wg, gate, v, ve, ids, ve_rows, v_eff, B, T, H, D, s)
              : gate_t<float>(x, ldx, Wg, gate, v, ve, ids, ve_rows, v_eff, B, T, H, D, s);
}

hipError_t launch_ve_gate_dv(const void* dv, const void* ve, const int* ids, int ve_rows,
                             const float* gate, void* dve, float* dgate, int B, int T, int H,
                             int D, bool bf16, hipStream_t s) {
  return bf16 ? gate_dv_t<swa::bf16>(dv, ve, ids, ve_rows, gate, dve, dgate, B, T, H, D, s)
              : gate_dv_t<float>(dv, ve, ids, ve_rows, gate, dve, dgate, B, T, H, D, s);
}

hipError_t launch_ve_gate_bwd(const void* x, int ldx, const float* Wg, const float* gate,
                              const float* dgate, float* dWg, void* dx32, void* ws, int B, int T,
                              int H, bool bf16, hipStream_t s) {
  return bf16 ? gate_bwd_t<swa::bf16>(x, ldx, Wg, gate, dgate, dWg, dx32, ws, B, T, H, s)
              : gate_bwd_t<float>(x, ldx, Wg, gate, dgate, dWg, dx32, ws, B, T, H, s);
}

}  // namespace swa

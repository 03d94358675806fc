// Causal sliding-window attention forward for gfx950.
//
// Method: "GPT-2 124M 复现" (notes.cassieliang.com) §3 (scaled scores, causal mask including
// the diagonal, softmax over keys, P V) and §19 (tiles of Q/K/V on chip, online softmax with a
// running max m and normaliser l, no T x T matrix in HBM). Windows: "从4万美元到73美元" §3.2.
//
// bf16 kernel design (one workgroup = 4 waves = 128 query rows of one (b, h)):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K tile rows read from LDS (128-bit), B = the
//    wave's 32 query rows held in VGPRs for the whole kernel. In the 32x32 accumulator layout
//    lane l owns query column l%32 and 16 keys, so the row max / row sum are in-lane, plus one
//    v_permlane32_swap between the two half-waves that share a query.
//  * O^T += V^T P^T on the same MFMA: B = P^T comes straight from the S^T accumulators
//    (converted to bf16) because the keys of one k-step sit in one lane in a fixed permuted
//    order; the V^T tile is written to LDS in that same permuted key order, so A is one
//    128-bit LDS read per lane.
//  * K and V^T tiles of 64 keys are double-buffered in LDS; the next tile's global loads are
//    issued before the current tile's MFMAs and written to the other buffer after them.
//  * Tiles wholly outside a wave's causal window are skipped; only tiles that straddle the
//    diagonal, the window's lower edge or the sequence end evaluate the mask.
//  * Workgroup order: all query blocks of one (b, h) run on one XCD (K/V reuse in that XCD's
//    L2), longest blocks first.
//  * Optional value-embedding gate: v_eff = v + gate * ve is formed in fp32 while the V tile is
//    staged into LDS, so v_eff never touches HBM.
#include "common.h"
#include "internal.h"

namespace swa {

namespace fwdk {

constexpr int NW = 4;          // waves per workgroup
constexpr int BM = 32 * NW;    // query rows per workgroup
constexpr int BN = 64;         // keys per tile

template <int D> struct Cfg {
  static constexpr int KP = D + 8;          // K tile row pitch (bf16 elements)
  static constexpr int VP = BN + 8;         // V^T tile row pitch
  static constexpr int K_ELEMS = BN * KP;
  static constexpr int V_ELEMS = D * VP;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int KG = (D == 128) ? 4 : 2;      // keys per V staging unit
  static constexpr int KGROUPS = BN / KG;             // 16 or 32
  static constexpr int K_CHUNKS = BN * D / 8 / 256;   // 16-byte K chunks per thread
};

// Position of key `k` (0..63) of a tile inside a V^T row: bits 2 and 3 swapped, which puts the
// 8 keys one lane feeds to a PV k-step next to each other.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

struct Params {
  const bf16* q; const bf16* k; const bf16* v; const bf16* ve; const float* gate;
  bf16* o; float* lse;
  int B, T, H, window, nqb;
  float c;      // scale * log2(e)
};

template <int D, bool GATE>
struct Stage {
  using C = Cfg<D>;
  uint4 kw[C::K_CHUNKS];
  uint4 vw[C::KG];
  float g[C::KG];
  uint4 ew[GATE ? C::KG : 1];

  __device__ __forceinline__ void load(const Params& p, int b, int h, int kt, int tid) {
    const int T = p.T, H = p.H;
    // K rows, 16-byte chunks, row-major
#pragma unroll
    for (int r = 0; r < C::K_CHUNKS; ++r) {
      const int c = tid + 256 * r;
      const int key = c / (D / 8), dc = c % (D / 8);
      const int kg = kt * BN + key;
      if (kg < T) kw[r] = *reinterpret_cast<const uint4*>(p.k + (((size_t)b * T + kg) * H + h) * D + dc * 8);
      else kw[r] = make_uint4(0, 0, 0, 0);
    }
    // V: KG consecutive keys x 8 dims
    const int kgrp = tid % C::KGROUPS, dgrp = tid / C::KGROUPS;
#pragma unroll
    for (int j = 0; j < C::KG; ++j) {
      const int kg = kt * BN + kgrp * C::KG + j;
      if (kg < T) {
        const size_t row = ((size_t)b * T + kg) * H + h;
        vw[j] = *reinterpret_cast<const uint4*>(p.v + row * D + dgrp * 8);
        if constexpr (GATE) {
          ew[j] = *reinterpret_cast<const uint4*>(p.ve + row * D + dgrp * 8);
          g[j] = p.gate[row];
        }
      } else {
        vw[j] = make_uint4(0, 0, 0, 0);
        if constexpr (GATE) { ew[j] = make_uint4(0, 0, 0, 0); g[j] = 0.f; }
      }
    }
  }

  __device__ __forceinline__ void store(bf16* buf, int tid) {
    bf16* ks = buf;
    bf16* vs = buf + C::K_ELEMS;
#pragma unroll
    for (int r = 0; r < C::K_CHUNKS; ++r) {
      const int c = tid + 256 * r;
      const int key = c / (D / 8), dc = c % (D / 8);
      *reinterpret_cast<uint4*>(ks + key * C::KP + dc * 8) = kw[r];
    }
    const int kgrp = tid % C::KGROUPS, dgrp = tid / C::KGROUPS;
    // unpack to floats: f[j][e] = V[key j][d = dgrp*8 + e]
    float f[C::KG][8];
#pragma unroll
    for (int j = 0; j < C::KG; ++j) {
      const uint32_t w[4] = {vw[j].x, vw[j].y, vw[j].z, vw[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) { f[j][2 * e] = bf_lo(w[e]); f[j][2 * e + 1] = bf_hi(w[e]); }
      if constexpr (GATE) {
        const uint32_t u[4] = {ew[j].x, ew[j].y, ew[j].z, ew[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[j][2 * e] = fmaf(g[j], bf_lo(u[e]), f[j][2 * e]);
          f[j][2 * e + 1] = fmaf(g[j], bf_hi(u[e]), f[j][2 * e + 1]);
        }
      }
    }
    const int pos = vt_pos(kgrp * C::KG);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16* dst = vs + (dgrp * 8 + e) * C::VP + pos;
      if constexpr (C::KG == 4) {
        uint2 w;
        w.x = pack_bf2(f[0][e], f[1][e]);
        w.y = pack_bf2(f[2][e], f[3][e]);
        *reinterpret_cast<uint2*>(dst) = w;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = pack_bf2(f[0][e], f[1][e]);
      }
    }
  }
};

template <int D, bool GATE>
__global__ void __launch_bounds__(256) fwd_bf16_kernel(Params p) {
  using C = Cfg<D>;
  constexpr int NDB = D / 32;  // 32-wide d blocks of O^T
  constexpr int NKS = D / 16;  // k-steps of S^T
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16* smem = reinterpret_cast<bf16*>(smem_raw);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int T = p.T, H = p.H, W = p.window;

  // XCD-aware, longest-first block order.
  const int nblk = gridDim.x;
  int L = blockIdx.x;
  if ((nblk & 7) == 0) L = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int bh = L / p.nqb;
  const int qb = p.nqb - 1 - (L - bh * p.nqb);
  const int b = bh / H, h = bh - b * H;

  const int q0 = qb * BM;
  const int qw = q0 + wave * 32;      // first query of this wave
  const int myq = qw + l32;           // this lane's query row

  // Q^T operand: 8 bf16 of row myq per k-step, held for the whole kernel.
  bf16x8 qreg[NKS];
  {
    const bf16* qp = p.q + (((size_t)b * T + min(myq, T - 1)) * H + h) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 w = *reinterpret_cast<const uint4*>(qp + 16 * ks);
      if (myq >= T) w = make_uint4(0, 0, 0, 0);
      qreg[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int kt_lo = max(0, q0 - W + 1) / BN;
  const int kt_hi = min(T - 1, q0 + BM - 1) / BN;

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;

  Stage<D, GATE> st;
  st.load(p, b, h, kt_lo, tid);
  st.store(smem, tid);
  __syncthreads();

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int cur = (kt - kt_lo) & 1;
    const bool has_next = kt < kt_hi;
    if (has_next) st.load(p, b, h, kt + 1, tid);

    const bf16* ks = smem + cur * C::BUF_ELEMS;
    const bf16* vs = ks + C::K_ELEMS;
    const int k0 = kt * BN;
    // wave-uniform skip / mask decisions
    const bool skip = (k0 > qw + 31) || (k0 + BN - 1 < qw - W + 1);
    if (!skip) {
      const bool need_mask = (k0 + BN - 1 > qw) || (k0 < qw + 31 - W + 1) || (k0 + BN > T);
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = (f32x16){};
        const bf16* arow = ks + (kb * 32 + l32) * C::KP + 8 * hi;
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + 16 * kk);
          s[kb] = mfma32(a, qreg[kk], s[kb]);
        }
      }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kg = k0 + kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
            const bool ok = (kg <= myq) && (kg > myq - W) && (kg < T);
            s[kb][i] = ok ? s[kb][i] : -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = fmaxf(mx, half_swap(mx));
      const float m_new = fmaxf(m_run, mx * p.c);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float lsum = 0.f;
      bf16x8 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          float e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            e[j] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * sp + j], p.c, -m_use));
            lsum += e[j];
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[kb][sp][j] = (bf16)e[j];
        }
      l_run = fmaf(l_run, alpha, lsum);
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16* vrow = vs + (db * 32 + l32) * C::VP + 8 * hi;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int sp = 0; sp < 2; ++sp) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + kb * 32 + sp * 16);
            oacc[db] = mfma32(a, pb[kb][sp], oacc[db]);
          }
      }
    }
    if (has_next) st.store(smem + (cur ^ 1) * C::BUF_ELEMS, tid);
    __syncthreads();
  }

  // Epilogue: combine the two half-wave partial sums, normalise, store O and lse.
  const float l_tot = l_run + half_swap(l_run);
  const float inv = 1.0f / l_tot;
  if (myq < T) {
    bf16* op = p.o + (((size_t)b * T + myq) * H + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint2 w;
        w.x = pack_bf2(oacc[db][4 * a + 0] * inv, oacc[db][4 * a + 1] * inv);
        w.y = pack_bf2(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv);
        *reinterpret_cast<uint2*>(op + db * 32 + 8 * a + 4 * hi) = w;
      }
    if (hi == 0) p.lse[((size_t)b * H + h) * T + myq] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace fwdk

// ------------------------------------------------------------------------------------------
// float32 path: one wave per query row; exact expf softmax. Used for the fp32 parity bar.
// ------------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(64) fwd_f32_kernel(const float* __restrict__ q,
                                                     const float* __restrict__ k,
                                                     const float* __restrict__ v,
                                                     const float* __restrict__ ve,
                                                     const float* __restrict__ gate,
                                                     float* __restrict__ o, float* __restrict__ lse,
                                                     int T, int H, int W, float scale) {
  constexpr int PER = D / 64;
  const int i = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H, lane = threadIdx.x;
  const size_t qrow = ((size_t)b * T + i) * H + h;
  float qv[PER], acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) { qv[e] = q[qrow * D + lane + 64 * e]; acc[e] = 0.f; }
  float m = -INFINITY, l = 0.f;
  for (int j = max(0, i - W + 1); j <= i; ++j) {
    const size_t krow = ((size_t)b * T + j) * H + h;
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) d = fmaf(qv[e], k[krow * D + lane + 64 * e], d);
#pragma unroll
    for (int msk = 32; msk > 0; msk >>= 1) d += xor_shfl(d, msk);
    const float s = d * scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float pj = expf(s - m_new);
    l = l * alpha + pj;
    const float g = gate ? gate[krow] : 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      float vv = v[krow * D + lane + 64 * e];
      if (gate) vv = fmaf(g, ve[krow * D + lane + 64 * e], vv);
      acc[e] = fmaf(acc[e], alpha, pj * vv);
    }
    m = m_new;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) o[qrow * D + lane + 64 * e] = acc[e] / l;
  if (lane == 0) lse[(size_t)bh * T + i] = m + logf(l);
}

template <int D, bool GATE>
static hipError_t launch_fwd_bf16_t(const AttnShape& a, const void* q, const void* k, const void* v,
                                    const void* ve, const float* gate, void* o, float* lse,
                                    hipStream_t s) {
  using C = fwdk::Cfg<D>;
  fwdk::Params p;
  p.q = (const bf16*)q; p.k = (const bf16*)k; p.v = (const bf16*)v; p.ve = (const bf16*)ve;
  p.gate = gate; p.o = (bf16*)o; p.lse = lse;
  p.B = a.B; p.T = a.T; p.H = a.H; p.window = a.window;
  p.nqb = (a.T + fwdk::BM - 1) / fwdk::BM;
  p.c = a.scale * kLog2e;
  const size_t smem = 2 * C::BUF_ELEMS * sizeof(bf16);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fwdk::fwd_bf16_kernel<D, GATE>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (attr != hipSuccess) return attr;
  const unsigned blocks = (unsigned)p.nqb * a.B * a.H;
  hipLaunchKernelGGL((fwdk::fwd_bf16_kernel<D, GATE>), dim3(blocks), dim3(256), smem, s, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const AttnShape& a, const void* q, const void* k, const void* v,
                      const void* ve, const float* gate, void* o, float* lse, bool is_bf16,
                      hipStream_t s) {
  if (is_bf16) {
    const bool g = gate != nullptr;
    if (a.D == 64)
      return g ? launch_fwd_bf16_t<64, true>(a, q, k, v, ve, gate, o, lse, s)
               : launch_fwd_bf16_t<64, false>(a, q, k, v, ve, gate, o, lse, s);
    return g ? launch_fwd_bf16_t<128, true>(a, q, k, v, ve, gate, o, lse, s)
             : launch_fwd_bf16_t<128, false>(a, q, k, v, ve, gate, o, lse, s);
  }
  dim3 grid(a.T, a.B * a.H);
  if (a.D == 64)
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(64), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)ve, gate, (float*)o, lse, a.T, a.H, a.window,
                       a.scale);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(64), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)ve, gate, (float*)o, lse, a.T, a.H, a.window,
                       a.scale);
  return hipGetLastError();
}

}  // namespace swa

// fp8 (OCP e4m3) forward variant of the causal sliding-window attention for gfx950.
//
// Method: as the bf16 forward ("GPT-2 124M 复现" §3 and §19: scaled scores, causal window,
// online softmax, P V), with both contractions on v_mfma_f32_32x32x64_f8f6f4. fp8 follows
// "NanoGPT Speedrun：大模型训练效率的极限竞速指南" (kongchang.com), section "工程与硬件优化",
// its paragraph on bf16 and fp8: an 8-bit floating-point format that can double matrix
// throughput over bf16 and needs finer calibration (scales). Each of q_hat, k_hat, v carries one float32 scale; scores and probabilities
// stay in float32, P is rounded to e4m3 as the PV operand (as the bf16 kernels round it to
// bf16), and O is written in bf16.
//
// Layouts (written by the packing kernels of fp8_pack.hip):
//  * q8, k8: (B, T, H, D) e4m3 codes.
//  * v8t: per (b, h) a D x Tp matrix (Tp = T rounded up to 64) of e4m3 codes, V transposed so
//    that the PV operand (keys along the contraction) is a row read. Inside every block of 64
//    keys the keys are stored in the order in which one lane's probabilities come out of the
//    S^T accumulators: byte 32g + 16kb + 4a + c holds key 32kb + 8a + 4g + c. Keys >= T are 0.
//
// Kernel (one workgroup = 4 waves = 128 query rows of one (b, h), 64-key tiles):
//  * S^T = K Q^T: A = 32 K rows x 64 dims (32 bytes per lane from LDS), B = the wave's 32 query
//    rows (32 bytes per lane and k-step, held in VGPRs). Accumulator layout and online softmax
//    are the bf16 kernel's: lane l owns query l%32 and 16 keys of each 32-key half.
//  * O^T += V^T P^T: B = the lane's 32 probabilities (both halves of the tile) packed into 32
//    e4m3 bytes in accumulator order; A = 32 bytes of a V^T row read from LDS, whose key order
//    was made to match when v8t was packed. One MFMA per 32 dims per tile.
//  * P needs no saturation: the running reference keeps every probability <= 2^8 < 448.
//  * K and V^T tiles double-buffered in LDS through asynchronous 16-byte global->LDS copies,
//    XOR-swizzled 16-byte chunks (conflict-free 128-bit reads of 16 consecutive rows).
#include "common.h"
#include "internal.h"

namespace swa {

namespace f8k {

constexpr int NW = 4;
constexpr int BM = 32 * NW;
constexpr int BN = 64;
constexpr float kRescaleSlack = 8.0f;   // probabilities stay <= 2^8 < 448

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Chunk swizzles: rows of 128 bytes (K at D = 128) and of 64 bytes (K at D = 64, V^T rows).
template <int ROWBYTES> __device__ __forceinline__ int swz8(int r);
template <> __device__ __forceinline__ int swz8<128>(int r) { return (r >> 1) & 7; }
template <> __device__ __forceinline__ int swz8<64>(int r) { return (r >> 2) & 3; }

// ---- forward -------------------------------------------------------------------------------

struct Params {
  const unsigned char* q8; const unsigned char* k8; const unsigned char* v8t;
  const int* bounds;
  bf16* o; float* lse;
  int B, T, H, window, nqb, Tp;
  float c;        // scale * q_scale * k_scale * log2(e)
  float vscale;
};

template <int D>
struct Cfg {
  static constexpr int KCH = D / 16;             // 16-byte chunks per K row
  static constexpr int KRPI = 64 / KCH;          // K rows per wave-wide 1 KiB copy
  static constexpr int KNIW = BN / KRPI / NW;    // ... copies per wave per tile
  static constexpr int VNIW = D / 16 / NW;       // V^T: 16 rows of 64 bytes per copy
  static constexpr int NKS = D / 64;             // k-steps of S^T = K Q^T
  static constexpr int NDB = D / 32;             // 32-dim blocks of O^T
};

template <int D>
struct Tiles {
  using C = Cfg<D>;
  int krow[C::KNIW];
  unsigned koff[C::KNIW];
  int kdst[C::KNIW];
  unsigned voff[C::VNIW];
  int vdst[C::VNIW];
  __device__ __forceinline__ void init(int H, int Tp, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < C::KNIW; ++i) {
      const int I = wave * C::KNIW + i;
      krow[i] = I * C::KRPI + lane / C::KCH;
      koff[i] = (unsigned)(krow[i] * H * D + 16 * ((lane % C::KCH) ^ swz8<D>(krow[i])));
      kdst[i] = I * C::KRPI * D;
    }
#pragma unroll
    for (int i = 0; i < C::VNIW; ++i) {
      const int I = wave * C::VNIW + i;
      const int r = I * 16 + lane / 4;
      voff[i] = (unsigned)(r * Tp + 16 * ((lane % 4) ^ swz8<64>(r)));
      vdst[i] = I * 16 * 64;
    }
  }
  __device__ __forceinline__ void load(const Params& p, const unsigned char* kbase,
                                       const unsigned char* vbase, lds_t<unsigned char>* ks,
                                       lds_t<unsigned char>* vs, int kt) const {
    const size_t rs = (size_t)p.H * D;
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kbase + (size_t)kt * BN * rs);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vbase + (size_t)kt * BN);
    if (kt * BN + BN <= p.T) {
#pragma unroll
      for (int i = 0; i < C::KNIW; ++i)
        b2lds16(rk, opaque(koff[i]), (lds_t<void>*)(ks + kdst[i]));
    } else {
      // rows past the sequence end re-read row T-1 (their scores are masked)
#pragma unroll
      for (int i = 0; i < C::KNIW; ++i) {
        const int over = max(kt * BN + krow[i] - (p.T - 1), 0);
        b2lds16(rk, koff[i] - (unsigned)over * (unsigned)rs, (lds_t<void>*)(ks + kdst[i]));
      }
    }
#pragma unroll
    for (int i = 0; i < C::VNIW; ++i)
      b2lds16(rv, opaque(voff[i]), (lds_t<void>*)(vs + vdst[i]));
  }
};

template <int D>
struct WaveState {
  f32x16 oacc[D / 32];
  float m_ref, l_run;
};

template <int D>
__device__ __forceinline__ void tile_step(WaveState<D>& ws, const i32x8* qreg,
                                          const lds_t<unsigned char>* ks,
                                          const lds_t<unsigned char>* vs, const int* kofs,
                                          const int* vofs, int k0, int qw, int T,
                                          const RowRange& rr, float c, int lane) {
  using C = Cfg<D>;
  const int hi = lane >> 5;
  const bool skip = (k0 > qw + 31) || (k0 + BN - 1 < rr.wlo0);
  if (skip) return;
  const bool need_mask = (k0 + BN - 1 > qw) || (k0 < rr.wlo1) || (k0 + BN > T);
  auto read32 = [](const lds_t<unsigned char>* base, int o0, int o1) {
    const u32x4 a = *reinterpret_cast<const lds_t<u32x4>*>(base + o0);
    const u32x4 b = *reinterpret_cast<const lds_t<u32x4>*>(base + o1);
    return (i32x8){(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                   (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  };
  i32x8 ka[2][C::NKS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int kk = 0; kk < C::NKS; ++kk)
      ka[kb][kk] = read32(ks + kb * 32 * D, kofs[2 * kk], kofs[2 * kk + 1]);
  sched_fence();
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = (f32x16){};
#pragma unroll
    for (int kk = 0; kk < C::NKS; ++kk) s[kb] = mfma8(ka[kb][kk], qreg[kk], s[kb]);
  }
  i32x8 va[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) va[db] = read32(vs + db * 32 * 64, vofs[0], vofs[1]);
  sched_fence();
  if (need_mask) {
    branch_keep();
    const int lo = rr.lo - k0 - 4 * hi;
    const unsigned n = rr.n;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = kb * 32 + 8 * (i >> 2) + (i & 3);
        s[kb][i] = ((unsigned)(t - lo) < n) ? s[kb][i] : -INFINITY;
      }
  }
  float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = (kb == 0 ? 2 : 0); i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[kb][i], s[kb][i + 1]));
  mx = fmaxf(mx, half_swap(mx));
  const float mt = mx * c;
  if (__builtin_amdgcn_ballot_w64(mt > ws.m_ref + kRescaleSlack) != 0) {
    branch_keep();
    const float m_new = fmaxf(ws.m_ref, mt);
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(ws.m_ref - m_new);
    ws.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) ws.oacc[db] *= alpha;
    ws.m_ref = m_new;
  }
  const float m_use = (ws.m_ref == -INFINITY) ? 0.f : ws.m_ref;
  float lsum = 0.f;
  unsigned pw[8];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[j] = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * w + j], c, -m_use));
        lsum += e[j];
      }
      const unsigned lo2 = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0u, false);
      pw[4 * kb + w] = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], lo2, true);
    }
  ws.l_run += lsum;
  const i32x8 pb = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3],
                    (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) ws.oacc[db] = mfma8(va[db], pb, ws.oacc[db]);
}

// Three workgroups per CU (32 KiB of LDS each, at most 168 VGPRs: the partial last tile's
// address arithmetic spills a few values): 7-8 % faster than two.
template <int D, bool DOC>
__global__ void __launch_bounds__(64 * NW, 3) fwd_fp8_kernel(Params p) {
  using C = Cfg<D>;
  constexpr int KT = BN * D, VT = D * 64;
  __shared__ __attribute__((aligned(16))) unsigned char k0s[KT], v0s[VT], k1s[KT], v1s[VT];
  auto* K0 = (lds_t<unsigned char>*)k0s;
  auto* V0 = (lds_t<unsigned char>*)v0s;
  auto* K1 = (lds_t<unsigned char>*)k1s;
  auto* V1 = (lds_t<unsigned char>*)v1s;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T, H = p.H, W = p.window;

  const int nblk = gridDim.x;
  int L = blockIdx.x;
  if ((nblk & 7) == 0) L = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int bh = L / p.nqb;
  const int qb = p.nqb - 1 - (L - bh * p.nqb);
  const int b = bh / H, h = bh - b * H;
  const size_t head0 = ((size_t)b * T * H + h) * D;
  const unsigned char* kbase = p.k8 + head0;
  const unsigned char* vbase = p.v8t + (size_t)bh * D * p.Tp;

  const int q0 = qb * BM;
  const int qw = q0 + wave * 32;
  const int myq = qw + l32;

  // Q^T operand: dims 64 kk + 32 hi .. +31 of row myq.
  i32x8 qreg[C::NKS];
  {
    const unsigned char* qp = p.q8 + head0 + (size_t)min(myq, T - 1) * H * D + 32 * hi;
#pragma unroll
    for (int kk = 0; kk < C::NKS; ++kk) {
      uint4 a = reinterpret_cast<const uint4*>(qp + 64 * kk)[0];
      uint4 bq = reinterpret_cast<const uint4*>(qp + 64 * kk)[1];
      if (myq >= T) a = bq = make_uint4(0, 0, 0, 0);
      qreg[kk] = (i32x8){(int)a.x, (int)a.y, (int)a.z, (int)a.w,
                         (int)bq.x, (int)bq.y, (int)bq.z, (int)bq.w};
    }
  }

  const RowRange rr = row_range<DOC>(p.bounds, b, T, W, myq);
  int lo_q0 = max(q0 - W + 1, 0);
  if constexpr (DOC) lo_q0 = max(lo_q0, p.bounds[2 * ((size_t)b * T + q0)]);
  const int kt_lo = lo_q0 / BN;
  const int kt_hi = min(T - 1, q0 + BM - 1) / BN;

  WaveState<D> ws;
#pragma unroll
  for (int i = 0; i < C::NDB; ++i) ws.oacc[i] = (f32x16){};
  ws.m_ref = -INFINITY;
  ws.l_run = 0.f;

  // LDS byte offsets: K row l32 (+32 kb at use), logical chunks 4 kk + 2 hi and + 1; V^T row
  // l32 (+32 db at use), logical chunks 2 hi and 2 hi + 1. Both swizzles depend on the row
  // modulo 16 only, so the +32 row offsets keep them.
  int kofs[2 * C::NKS], vofs[2];
#pragma unroll
  for (int kk = 0; kk < C::NKS; ++kk)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      kofs[2 * kk + j] = l32 * D + 16 * ((4 * kk + 2 * hi + j) ^ swz8<D>(l32));
#pragma unroll
  for (int j = 0; j < 2; ++j) vofs[j] = l32 * 64 + 16 * ((2 * hi + j) ^ swz8<64>(l32));

  Tiles<D> tl;
  tl.init(H, p.Tp, wave, lane);
  tl.load(p, kbase, vbase, K0, V0, kt_lo);
  wait_vmem();
  __syncthreads();
  for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
    if (kt + 1 <= kt_hi) tl.load(p, kbase, vbase, K1, V1, kt + 1);
    tile_step<D>(ws, qreg, K0, V0, kofs, vofs, kt * BN, qw, T, rr, p.c, lane);
    wait_vmem();
    __syncthreads();
    if (kt + 1 > kt_hi) break;
    if (kt + 2 <= kt_hi) tl.load(p, kbase, vbase, K0, V0, kt + 2);
    tile_step<D>(ws, qreg, K1, V1, kofs, vofs, (kt + 1) * BN, qw, T, rr, p.c, lane);
    wait_vmem();
    __syncthreads();
  }

  const float l_tot = ws.l_run + half_swap(ws.l_run);
  const float inv = p.vscale / l_tot;
  bf16* op = p.o + head0 + (size_t)min(myq, T - 1) * H * D;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) store_orow16(op, db, ws.oacc[db], inv, hi, myq < T);
  if (myq < T && hi == 0)
    p.lse[((size_t)b * H + h) * T + myq] = (ws.m_ref + __log2f(l_tot)) * kLn2;
}

}  // namespace f8k

hipError_t launch_fwd_fp8(const AttnShape& a, const void* q8, const void* k8, const void* v8t,
                          float qk_scale, float v_scale, void* o, float* lse, hipStream_t s) {
  f8k::Params p;
  p.q8 = (const unsigned char*)q8; p.k8 = (const unsigned char*)k8;
  p.v8t = (const unsigned char*)v8t;
  p.bounds = a.bounds; p.o = (bf16*)o; p.lse = lse;
  p.B = a.B; p.T = a.T; p.H = a.H; p.window = a.window;
  p.nqb = (a.T + f8k::BM - 1) / f8k::BM;
  p.Tp = (a.T + 63) / 64 * 64;
  p.c = a.scale * qk_scale * kLog2e;
  p.vscale = v_scale;
  const unsigned blocks = (unsigned)p.nqb * a.B * a.H;
  const dim3 blk(64 * f8k::NW);
  if (a.D == 64) {
    if (a.bounds) hipLaunchKernelGGL((f8k::fwd_fp8_kernel<64, true>), dim3(blocks), blk, 0, s, p);
    else hipLaunchKernelGGL((f8k::fwd_fp8_kernel<64, false>), dim3(blocks), blk, 0, s, p);
  } else {
    if (a.bounds) hipLaunchKernelGGL((f8k::fwd_fp8_kernel<128, true>), dim3(blocks), blk, 0, s, p);
    else hipLaunchKernelGGL((f8k::fwd_fp8_kernel<128, false>), dim3(blocks), blk, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace swa

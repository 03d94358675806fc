// dQ of causal sliding-window attention for gfx950: a query-block-major kernel that recomputes
// the scores ("GPT-2 124M 复现" §19: the backward recomputes intermediates) and writes dq
// directly, so the key-block-major dK/dV kernel needs no dQ accumulator and no atomics.
//
//   S^T = K Q^T, P^T = exp(S^T - lse), dP^T = V dO^T, dS^T = P^T (dP^T - delta),
//   dQ^T = scale K^T dS^T.
//
// Layout is that of the forward kernel (fwd.hip): one workgroup = 4 waves = 128 query rows of
// one (b, h); each lane owns one query column of the 32x32 MFMA accumulators, so lse and delta
// are per-lane scalars; the K^T operand of dQ^T comes from the row-major K tile by transposing
// reads, and dS^T feeds the MFMA straight from registers in the permuted key order. K and V tiles
// of 64 keys are double-buffered in LDS with asynchronous global->LDS copies.
#include "common.h"
#include "internal.h"

namespace swa {
namespace dqk {

constexpr int NW = 4;
constexpr int BM = 32 * NW;
constexpr int BN = 64;

template <int D> struct Cfg {
  static constexpr int CH = D / 8;
  static constexpr int RPI = 64 / CH;
  static constexpr int NI = BN / RPI;
  static constexpr int NIW = NI / NW;
  static constexpr int TILE = BN * D;
  static constexpr int CPT = BN * CH / (64 * NW);
};

struct Params {
  const bf16* q; const bf16* k; const bf16* v; const bf16* ve; const float* gate;
  const int* bounds;   // per-token document [start, end) (document masking only)
  const int* ve_ids;   // value-embedding table rows per token (table mode only)
  int ve_rows;
  const bf16* dO;
  float* nlse2; float* ndelta;   // row terms, negated (read; written when o is set)
  const bf16* o; const float* lse;   // set: compute the row terms here and store them
  bf16* dq;
  int B, T, H, window, nqb;
  float c;       // scale * log2(e)
  float scale;
};

template <int D, bool GATE>
struct Tiles {
  using C = Cfg<D>;
  unsigned loff[C::NIW];
  int wave, lane;
  __device__ __forceinline__ int row(int i) const { return (wave * C::NIW + i) * C::RPI + lane / C::CH; }
  __device__ __forceinline__ int ldst(int i) const { return (wave * C::NIW + i) * C::RPI * D; }
  __device__ __forceinline__ void init(int H, int wave_, int lane_) {
    wave = wave_;
    lane = lane_;
#pragma unroll
    for (int i = 0; i < C::NIW; ++i)
      loff[i] = 2u * (unsigned)(row(i) * H * D + 8 * ((lane % C::CH) ^ swz<D>(row(i))));
  }
  __device__ __forceinline__ void load_rows(const bf16* base, lds_t<bf16>* dst, int kt, int T,
                                            size_t rs) const {
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(base + (size_t)kt * BN * rs);
    if (kt * BN + BN <= T) {
#pragma unroll
      for (int i = 0; i < C::NIW; ++i) b2lds16(r, opaque(loff[i]), (lds_t<void>*)(dst + ldst(i)));
    } else {
#pragma unroll
      for (int i = 0; i < C::NIW; ++i) {
        const int over = max(kt * BN + row(i) - (T - 1), 0);
        b2lds16(r, opaque(loff[i]) - 2u * (unsigned)over * (unsigned)rs,
                (lds_t<void>*)(dst + ldst(i)));
      }
    }
  }
  // K and v_eff tile kt into LDS (row-major, swizzled); rows past the end re-read row T-1.
  __device__ __forceinline__ void load(const Params& p, const bf16* kbase, const bf16* vbase,
                                       lds_t<bf16>* ks, lds_t<bf16>* vs, int kt, int tid) const {
    const size_t rs = (size_t)p.H * D;
    load_rows(kbase, ks, kt, p.T, rs);
    if constexpr (!GATE) {
      load_rows(vbase, vs, kt, p.T, rs);
    } else {
#pragma unroll
      for (int j = 0; j < C::CPT; ++j) {
        const int id = tid + 64 * NW * j;
        const int r = id / C::CH, pos = id % C::CH;
        const int c = pos ^ swz<D>(r);
        const int grow = min(kt * BN + r, p.T - 1);
        const size_t goff = (size_t)grow * rs + 8 * c;
        const uint4 a = *reinterpret_cast<const uint4*>(vbase + goff);
        const size_t hb = (size_t)(vbase - p.v) / D;   // b * T * H + h
        const int bb = (int)(hb / ((size_t)p.T * p.H)), hh = (int)(hb - (size_t)bb * p.T * p.H);
        const bf16* er = ve_row<D>(p.ve, p.ve_ids, p.ve_rows, bb, p.T, p.H, hh, grow);
        const uint4 e = er ? *reinterpret_cast<const uint4*>(er + 8 * c) : make_uint4(0, 0, 0, 0);
        const float g = p.gate[hb + (size_t)grow * p.H];
        u32x4 o;
        o.x = pack_bf2(fmaf(g, bf_lo(e.x), bf_lo(a.x)), fmaf(g, bf_hi(e.x), bf_hi(a.x)));
        o.y = pack_bf2(fmaf(g, bf_lo(e.y), bf_lo(a.y)), fmaf(g, bf_hi(e.y), bf_hi(a.y)));
        o.z = pack_bf2(fmaf(g, bf_lo(e.z), bf_lo(a.z)), fmaf(g, bf_hi(e.z), bf_hi(a.z)));
        o.w = pack_bf2(fmaf(g, bf_lo(e.w), bf_lo(a.w)), fmaf(g, bf_hi(e.w), bf_hi(a.w)));
        *reinterpret_cast<lds_t<u32x4>*>(vs + r * D + 8 * pos) = o;
      }
    }
  }
};

// One 64-key tile for one wave (32 query rows).
template <int D>
__device__ __forceinline__ void dq_tile(f32x16* dqacc, const bf16x8* qreg, const bf16x8* oreg,
                                        const lds_t<bf16>* ks, const lds_t<bf16>* vs,
                                        const int* krow, const int* ktr1, const int* ktr2, int k0,
                                        int qw, int T, int lo_row, unsigned n, int wlo0, int wlo1,
                                        float c, float nl2, float ndl, int hi) {
  constexpr int NKS = D / 16, NDB = D / 32;
  // visible keys of this lane's query row: [lo_row, lo_row + n); wlo0 / wlo1: lo_row of the
  // wave's first and last query (lo_row never decreases along a row)
  const bool skip = (k0 > qw + 31) || (k0 + BN - 1 < wlo0);
  if (skip) return;
  const bool need_mask = (k0 + BN - 1 > qw) || (k0 < wlo1) || (k0 + BN > T);
  const int lo = lo_row - k0 - 4 * hi;
  // the two 32-key halves of the tile one after the other (halves the live registers)
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
      const bf16x8 a = *reinterpret_cast<const lds_t<bf16x8>*>(
          (const lds_t<char>*)ks + 2 * kb * 32 * D + krow[kk]);
      const bf16x8 b = *reinterpret_cast<const lds_t<bf16x8>*>(
          (const lds_t<char>*)vs + 2 * kb * 32 * D + krow[kk]);
      s = mfma32(a, qreg[kk], s);
      dp = mfma32(b, oreg[kk], dp);
    }
    sched_fence();
    float pv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, nl2));
    if (need_mask) {
      branch_keep();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = kb * 32 + 8 * (i >> 2) + (i & 3);
        pv[i] = ((unsigned)(t - lo) < n) ? pv[i] : 0.f;
      }
    }
    bf16x8 dsb[2];
#pragma unroll
    for (int sp = 0; sp < 2; ++sp)
#pragma unroll
      for (int jj = 0; jj < 8; jj += 2) {
        const int i = 8 * sp + jj;
        const bf16x2 t = __builtin_convertvector(
            (f32x2){pv[i] * (dp[i] + ndl), pv[i + 1] * (dp[i + 1] + ndl)}, bf16x2);
        dsb[sp][jj] = t[0];
        dsb[sp][jj + 1] = t[1];
      }
    // dQ^T += K^T dS^T for these 32 keys; K^T by transposing reads of the row-major K tile.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const int ro = 2 * (kb * 32 + sp * 16) * D;
        const lds_t<char>* kc = (const lds_t<char>*)ks + ro;
        const bf16x8 a = __builtin_shufflevector(
            ds_read_tr16((const lds_t<bf16>*)(kc + ktr1[db])),
            ds_read_tr16((const lds_t<bf16>*)(kc + ktr2[db])), 0, 1, 2, 3, 4, 5, 6, 7);
        dqacc[db] = mfma32(a, dsb[sp], dqacc[db]);
      }
    }
    sched_fence();
  }
}

template <int D, bool GATE, bool DOC>
__global__ void __launch_bounds__(64 * NW, 8 / NW) dq_bf16_kernel(Params p) {
  using C = Cfg<D>;
  constexpr int NDB = D / 32, NKS = D / 16;
  __shared__ __attribute__((aligned(16))) bf16 k0s[C::TILE], v0s[C::TILE], k1s[C::TILE], v1s[C::TILE];
  lds_t<bf16>* K0 = (lds_t<bf16>*)k0s;
  lds_t<bf16>* V0 = (lds_t<bf16>*)v0s;
  lds_t<bf16>* K1 = (lds_t<bf16>*)k1s;
  lds_t<bf16>* V1 = (lds_t<bf16>*)v1s;

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
  const bf16* kbase = p.k + head0;
  const bf16* vbase = p.v + head0;

  const int q0 = qb * BM;
  const int qw = q0 + wave * 32;
  const int myq = qw + l32;

  // B operands (lane = query column): 8 dims of this lane's Q and dO rows per k-step.
  bf16x8 qreg[NKS], oreg[NKS];
  {
    const size_t off = head0 + (size_t)min(myq, T - 1) * H * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 wq = *reinterpret_cast<const uint4*>(p.q + off + 16 * ks);
      uint4 wo = *reinterpret_cast<const uint4*>(p.dO + off + 16 * ks);
      if (myq >= T) { wq = make_uint4(0, 0, 0, 0); wo = make_uint4(0, 0, 0, 0); }
      qreg[ks] = __builtin_bit_cast(bf16x8, wq);
      oreg[ks] = __builtin_bit_cast(bf16x8, wo);
    }
  }
  const size_t rrow = (size_t)bh * T + min(myq, T - 1);
  float nl2, ndl;
  if (p.o) {
    // Row terms of this lane's query from O, dO and lse (the other half-wave holds the other
    // dims of the row), stored for the key-major kernel that runs after this one.
    const size_t off = head0 + (size_t)min(myq, T - 1) * H * D + 8 * hi;
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float ov[8], gv[8];
      unpack16(*reinterpret_cast<const uint4*>(p.o + off + 16 * ks), ov);
      unpack16(__builtin_bit_cast(uint4, oreg[ks]), gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(ov[e], gv[e], acc);
    }
    acc += half_swap(acc);
    nl2 = -p.lse[rrow] * kLog2e;
    ndl = -acc;
    if (hi == 0 && myq < T) {
      p.nlse2[rrow] = nl2;
      p.ndelta[rrow] = ndl;
    } else if (hi == 0 && bh == p.B * H - 1) {
      // past the end of the last head: the slack rows the dK/dV kernel's last query tile
      // reads (masked queries) are zeroed, so no bit pattern left in the workspace reaches dS
      const size_t tail = (size_t)bh * T + myq;
      p.nlse2[tail] = 0.f;
      p.ndelta[tail] = 0.f;
    }
  } else {
    nl2 = p.nlse2[rrow];
    ndl = p.ndelta[rrow];
  }

  const int qc = min(myq, T - 1);
  int start = 0;
  if constexpr (DOC) start = p.bounds[2 * ((size_t)b * T + qc)];
  const int lo_row = max(qc - W + 1, start);
  const unsigned n_row = (unsigned)(qc - lo_row + 1);
  const int wlo0 = __builtin_amdgcn_readlane(lo_row, 0);
  const int wlo1 = __builtin_amdgcn_readlane(lo_row, 31);
  int lo_q0 = max(q0 - W + 1, 0);   // first key any query of the workgroup sees
  if constexpr (DOC) lo_q0 = max(lo_q0, p.bounds[2 * ((size_t)b * T + q0)]);
  const int kt_lo = lo_q0 / BN;
  const int kt_hi = min(T - 1, q0 + BM - 1) / BN;

  int krow[NKS];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) krow[kk] = 2 * (l32 * D + 8 * ((2 * kk + hi) ^ swz<D>(l32)));
  int ktr1[NDB], ktr2[NDB];
  {
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 32 * db + 16 * (g & 1) + 4 * (j & 3);
      const int r1 = 4 * hi + (j >> 2), r2 = r1 + 8;
      ktr1[db] = 2 * (r1 * D + 8 * ((d >> 3) ^ swz<D>(r1)) + 4 * ((d >> 2) & 1));
      ktr2[db] = 2 * (r2 * D + 8 * ((d >> 3) ^ swz<D>(r2)) + 4 * ((d >> 2) & 1));
    }
  }

  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = (f32x16){};

  Tiles<D, GATE> tl;
  tl.init(H, wave, lane);
  tl.load(p, kbase, vbase, K0, V0, kt_lo, tid);
  wait_vmem();
  __syncthreads();
  // The lane offsets (bytes) are redefined at every tile so that tile buffer + offset is formed
  // at each LDS read, folded into its immediate offset, instead of being held once per buffer
  // (which the register budget does not allow: the sums were recomputed at every read).
  auto launder = [&]() {
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) asm volatile("" : "+v"(krow[kk]));
#pragma unroll
    for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(ktr1[db]), "+v"(ktr2[db]));
  };
  for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
    if (kt + 1 <= kt_hi) tl.load(p, kbase, vbase, K1, V1, kt + 1, tid);
    launder();
    dq_tile<D>(dqacc, qreg, oreg, K0, V0, krow, ktr1, ktr2, kt * BN, qw, T, lo_row, n_row, wlo0, wlo1, p.c, nl2, ndl, hi);
    wait_vmem();
    __syncthreads();
    if (kt + 1 > kt_hi) break;
    if (kt + 2 <= kt_hi) tl.load(p, kbase, vbase, K0, V0, kt + 2, tid);
    launder();
    dq_tile<D>(dqacc, qreg, oreg, K1, V1, krow, ktr1, ktr2, (kt + 1) * BN, qw, T, lo_row, n_row, wlo0, wlo1, p.c, nl2, ndl, hi);
    wait_vmem();
    __syncthreads();
  }

  // dq row myq: lane holds d = 32 db + 8 a + 4 hi + (0..3)
  if (myq < T) {
    bf16* op = p.dq + head0 + (size_t)myq * H * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint2 w;
        w.x = pack_bf2(dqacc[db][4 * a + 0] * p.scale, dqacc[db][4 * a + 1] * p.scale);
        w.y = pack_bf2(dqacc[db][4 * a + 2] * p.scale, dqacc[db][4 * a + 3] * p.scale);
        *reinterpret_cast<uint2*>(op + db * 32 + 8 * a + 4 * hi) = w;
      }
  }
}

template <int D, bool GATE>
static hipError_t launch_t(const AttnShape& a, const Params& p, hipStream_t s) {
  const unsigned blocks = (unsigned)p.nqb * a.B * a.H;
  if (a.bounds)
    hipLaunchKernelGGL((dq_bf16_kernel<D, GATE, true>), dim3(blocks), dim3(64 * dqk::NW), 0, s, p);
  else
    hipLaunchKernelGGL((dq_bf16_kernel<D, GATE, false>), dim3(blocks), dim3(64 * dqk::NW), 0, s, p);
  return hipGetLastError();
}

}  // namespace dqk

hipError_t launch_dq_bf16(const AttnShape& a, const void* q, const void* k, const void* v,
                          const void* ve, const float* gate, const void* dO, float* nlse2,
                          float* ndelta, const void* o, const float* lse, void* dq,
                          hipStream_t s) {
  dqk::Params p;
  p.q = (const bf16*)q; p.k = (const bf16*)k; p.v = (const bf16*)v; p.ve = (const bf16*)ve;
  p.ve_ids = a.ve_ids; p.ve_rows = a.ve_rows;
  p.gate = gate; p.bounds = a.bounds; p.dO = (const bf16*)dO; p.nlse2 = nlse2; p.ndelta = ndelta;
  p.o = (const bf16*)o; p.lse = lse; p.dq = (bf16*)dq;
  p.B = a.B; p.T = a.T; p.H = a.H; p.window = a.window;
  p.nqb = (a.T + dqk::BM - 1) / dqk::BM;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  const bool g = gate != nullptr;
  if (a.D == 64) return g ? dqk::launch_t<64, true>(a, p, s) : dqk::launch_t<64, false>(a, p, s);
  return g ? dqk::launch_t<128, true>(a, p, s) : dqk::launch_t<128, false>(a, p, s);
}

}  // namespace swa

// Causal sliding-window attention backward for gfx950, by recomputation of the scores
// ("GPT-2 124M 复现" §19: the backward recomputes intermediates, trading FLOPs for HBM traffic).
//
//   delta_i = dO_i . O_i                                 (preprocess kernel)
//   P = exp(s - lse), dV = P^T dO, dP = dO V^T, dS = P (dP - delta),
//   dQ = scale dS K, dK = scale dS^T Q                   (main kernel, key-block major)
//   dq = bf16(dQ accumulator)                            (finalize kernel)
//
// bf16 main kernel (one workgroup = 4 waves = 128 keys of one (b, h); query tiles of 64):
//  * S = Q K^T and dP = dO V^T on v_mfma_f32_32x32x16_bf16 with B = the wave's 32 key rows of
//    K and V held in VGPRs for the whole kernel and A = the query tile's rows from LDS. In the
//    32x32 accumulator layout each lane then owns one key and 16 queries, so P^T and dS^T are
//    already in the A-operand layout of dV += P^T dO and dK += dS^T Q (fixed permutation of the
//    query order, matched by the transposed dO^T / Q^T tiles the workgroup writes to LDS).
//  * dQ needs dS with queries on lanes: dS is written to LDS (bf16), then every wave contracts
//    its 32-wide slice of D over all 128 keys of the block (A = dS rows, B = K^T from LDS) and
//    adds the result to a float32 dQ accumulator with hardware float atomics (the accumulator
//    is zeroed by the preprocess kernel, so the path needs no memset).
//  * Query tiles that lie wholly outside a wave's keys' windows are skipped by that wave.
//  * Workgroup order: all key blocks of one (b, h) on one XCD, longest (earliest) blocks first.
//  * Value-embedding gate: v_eff = v + gate * ve is formed in fp32 when the V rows are loaded;
//    the epilogue writes dv = dv_eff, dve = gate * dv_eff and dgate = sum_d dv_eff * ve.
#include "common.h"
#include "internal.h"

namespace swa {

// ------------------------------------------------------------------------------------------
// delta_i = sum_d dO[i, d] * O[i, d]; also zeroes the float32 dQ accumulator row.
// ------------------------------------------------------------------------------------------
template <typename E, int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const E* __restrict__ o,
                                                      const E* __restrict__ dO,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ dq_acc, int rows, int T,
                                                      int H) {
  constexpr int VPT = 16 / sizeof(E), TPR = D / VPT;
  const int lr = threadIdx.x % TPR;
  const int row = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (row >= rows) return;
  const size_t off = (size_t)row * D + lr * VPT;
  const uint4 a = *reinterpret_cast<const uint4*>(o + off);
  const uint4 g = *reinterpret_cast<const uint4*>(dO + off);
  float acc;
  if constexpr (VPT == 4) {
    acc = __uint_as_float(a.x) * __uint_as_float(g.x);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(g.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(g.z), acc);
    acc = fmaf(__uint_as_float(a.w), __uint_as_float(g.w), acc);
  } else {
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, gw[4] = {g.x, g.y, g.z, g.w};
    acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf_lo(aw[e]), bf_lo(gw[e]), acc);
      acc = fmaf(bf_hi(aw[e]), bf_hi(gw[e]), acc);
    }
  }
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) acc += xor_shfl(acc, m);
  if (dq_acc) {
    float4* z = reinterpret_cast<float4*>(dq_acc + (size_t)row * D + lr * VPT);
#pragma unroll
    for (int e = 0; e < VPT / 4; ++e) z[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (lr == 0) {
    const int h = row % H, t = (row / H) % T, b = row / (H * T);
    delta[((size_t)b * H + h) * T + t] = acc;
  }
}

// dq (bf16) = dQ accumulator (float32, already scaled); 8 elements per lane.
__global__ void __launch_bounds__(256) bwd_dq_final_kernel(const float* __restrict__ acc,
                                                           bf16* __restrict__ dq, size_t n8) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(acc)[2 * i];
  const float4 b = reinterpret_cast<const float4*>(acc)[2 * i + 1];
  uint4 w;
  w.x = pack_bf2(a.x, a.y); w.y = pack_bf2(a.z, a.w);
  w.z = pack_bf2(b.x, b.y); w.w = pack_bf2(b.z, b.w);
  reinterpret_cast<uint4*>(dq)[i] = w;
}

namespace bwdk {

constexpr int NW = 4;
constexpr int BNK = 32 * NW;  // keys per workgroup
constexpr int BMQ = 64;       // queries per tile

template <int D> struct Cfg {
  static constexpr int QP = D + 8;       // Q / dO tile pitch (row-major)
  static constexpr int TP = BMQ + 8;     // Q^T / dO^T tile pitch
  static constexpr int SP = BNK + 8;     // dS tile pitch
  static constexpr int KTP = BNK + 8;    // K^T pitch
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = OFF_Q + BMQ * QP;
  static constexpr int OFF_QT = OFF_DO + BMQ * QP;
  static constexpr int OFF_DOT = OFF_QT + D * TP;
  static constexpr int OFF_DS = OFF_DOT + D * TP;
  static constexpr int OFF_KT = OFF_DS + BMQ * SP;
  static constexpr int BF_ELEMS = OFF_KT + D * KTP;
  static constexpr size_t SMEM = BF_ELEMS * 2 + 2 * BMQ * 4;
  static constexpr int KG = (D == 128) ? 4 : 2;   // queries per staging unit
  static constexpr int QGROUPS = BMQ / KG;         // 16 or 32 (x D/8 dgroups = 256 units)
};

__device__ __forceinline__ int tpos(int q) {  // bits 2 and 3 swapped (see fwd.hip)
  return (q & ~12) | ((q & 4) << 1) | ((q & 8) >> 1);
}

struct Params {
  const bf16* q; const bf16* k; const bf16* v; const bf16* ve; const float* gate;
  const float* lse; const float* delta; const bf16* dO;
  float* dq_acc; bf16* dk; bf16* dv; bf16* dve; float* dgate;
  int B, T, H, window, nkb;
  float c;       // scale * log2(e)
  float scale;
};

template <int D>
struct QStage {
  using C = Cfg<D>;
  uint4 qw[C::KG], ow[C::KG];
  float l2, dl;
  __device__ __forceinline__ void load(const Params& p, int b, int h, int qt, int tid) {
    const int qgrp = tid % C::QGROUPS, dgrp = tid / C::QGROUPS;
#pragma unroll
    for (int j = 0; j < C::KG; ++j) {
      const int qg = qt * BMQ + qgrp * C::KG + j;
      if (qg < p.T) {
        const size_t off = (((size_t)b * p.T + qg) * p.H + h) * D + dgrp * 8;
        qw[j] = *reinterpret_cast<const uint4*>(p.q + off);
        ow[j] = *reinterpret_cast<const uint4*>(p.dO + off);
      } else {
        qw[j] = make_uint4(0, 0, 0, 0);
        ow[j] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < BMQ) {
      const int qg = qt * BMQ + tid;
      const size_t r = ((size_t)b * p.H + h) * p.T + qg;
      l2 = qg < p.T ? p.lse[r] * kLog2e : 0.f;
      dl = qg < p.T ? p.delta[r] : 0.f;
    }
  }
  __device__ __forceinline__ void store(unsigned char* smem, int tid) const {
    bf16* sb = reinterpret_cast<bf16*>(smem);
    float* sf = reinterpret_cast<float*>(smem + C::BF_ELEMS * 2);
    const int qgrp = tid % C::QGROUPS, dgrp = tid / C::QGROUPS;
#pragma unroll
    for (int j = 0; j < C::KG; ++j) {
      const int ql = qgrp * C::KG + j;
      *reinterpret_cast<uint4*>(sb + C::OFF_Q + ql * C::QP + dgrp * 8) = qw[j];
      *reinterpret_cast<uint4*>(sb + C::OFF_DO + ql * C::QP + dgrp * 8) = ow[j];
    }
    const int pos = tpos(qgrp * C::KG);
    transpose_store(sb + C::OFF_QT, qw, dgrp, pos);
    transpose_store(sb + C::OFF_DOT, ow, dgrp, pos);
    if (tid < BMQ) { sf[tid] = l2; sf[BMQ + tid] = dl; }
  }
  __device__ __forceinline__ static void transpose_store(bf16* base, const uint4* w, int dgrp,
                                                         int pos) {
    uint32_t u[C::KG][4];
#pragma unroll
    for (int j = 0; j < C::KG; ++j) { u[j][0] = w[j].x; u[j][1] = w[j].y; u[j][2] = w[j].z; u[j][3] = w[j].w; }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16* dst = base + (dgrp * 8 + e) * C::TP + pos;
      // 16-bit element e of each row j
      auto el = [&](int j) -> uint32_t { return (e & 1) ? (u[j][e >> 1] >> 16) : (u[j][e >> 1] & 0xffffu); };
      if constexpr (C::KG == 4) {
        uint2 o;
        o.x = el(0) | (el(1) << 16);
        o.y = el(2) | (el(3) << 16);
        *reinterpret_cast<uint2*>(dst) = o;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = el(0) | (el(1) << 16);
      }
    }
  }
};

template <int D, bool GATE>
__global__ void __launch_bounds__(256) bwd_bf16_kernel(Params p) {
  using C = Cfg<D>;
  constexpr int NDB = D / 32, NKS = D / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* sb = reinterpret_cast<bf16*>(smem);
  const float* sf = reinterpret_cast<const float*>(smem + C::BF_ELEMS * 2);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int T = p.T, H = p.H, W = p.window;

  const int nblk = gridDim.x;
  int L = blockIdx.x;
  if ((nblk & 7) == 0) L = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int bh = L / p.nkb;
  const int kbk = L - bh * p.nkb;
  const int b = bh / H, h = bh - b * H;
  const int kb0 = kbk * BNK;
  const int kw = kb0 + 32 * wave;
  const int mykey = kw + l32;

  // B operands: this lane's key row of K and of v_eff, 8 dims per k-step.
  bf16x8 kreg[NKS], vreg[NKS];
  float gk = 0.f;
  {
    const size_t row = ((size_t)b * T + min(mykey, T - 1)) * H + h;
    const bool ok = mykey < T;
    if constexpr (GATE) gk = ok ? p.gate[row] : 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const size_t off = row * D + 16 * ks + 8 * hi;
      uint4 kk = *reinterpret_cast<const uint4*>(p.k + off);
      uint4 vv = *reinterpret_cast<const uint4*>(p.v + off);
      if constexpr (GATE) {
        const uint4 ee = *reinterpret_cast<const uint4*>(p.ve + off);
        vv.x = pack_bf2(fmaf(gk, bf_lo(ee.x), bf_lo(vv.x)), fmaf(gk, bf_hi(ee.x), bf_hi(vv.x)));
        vv.y = pack_bf2(fmaf(gk, bf_lo(ee.y), bf_lo(vv.y)), fmaf(gk, bf_hi(ee.y), bf_hi(vv.y)));
        vv.z = pack_bf2(fmaf(gk, bf_lo(ee.z), bf_lo(vv.z)), fmaf(gk, bf_hi(ee.z), bf_hi(vv.z)));
        vv.w = pack_bf2(fmaf(gk, bf_lo(ee.w), bf_lo(vv.w)), fmaf(gk, bf_hi(ee.w), bf_hi(vv.w)));
      }
      if (!ok) { kk = make_uint4(0, 0, 0, 0); vv = make_uint4(0, 0, 0, 0); }
      kreg[ks] = __builtin_bit_cast(bf16x8, kk);
      vreg[ks] = __builtin_bit_cast(bf16x8, vv);
    }
  }
  // K^T of the whole key block into LDS (B operand of dQ = dS K): KT[d][key].
  for (int u = tid; u < (BNK / 4) * (D / 8); u += 256) {
    const int kg4 = u % (BNK / 4), dgrp = u / (BNK / 4);
    uint32_t w[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = kb0 + kg4 * 4 + j;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (key < T) x = *reinterpret_cast<const uint4*>(p.k + (((size_t)b * T + key) * H + h) * D + dgrp * 8);
      w[j][0] = x.x; w[j][1] = x.y; w[j][2] = x.z; w[j][3] = x.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      auto el = [&](int j) -> uint32_t { return (e & 1) ? (w[j][e >> 1] >> 16) : (w[j][e >> 1] & 0xffffu); };
      uint2 o;
      o.x = el(0) | (el(1) << 16);
      o.y = el(2) | (el(3) << 16);
      *reinterpret_cast<uint2*>(sb + C::OFF_KT + (dgrp * 8 + e) * C::KTP + kg4 * 4) = o;
    }
  }

  f32x16 dv[NDB], dk[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) { dv[i] = (f32x16){}; dk[i] = (f32x16){}; }

  const int qt_lo = kb0 / BMQ;
  const int qt_hi = min(T - 1, kb0 + BNK - 1 + W - 1) / BMQ;

  QStage<D> st;
  st.load(p, b, h, qt_lo, tid);
  st.store(smem, tid);
  __syncthreads();

  for (int qt = qt_lo; qt <= qt_hi; ++qt) {
    const bool has_next = qt < qt_hi;
    if (has_next) st.load(p, b, h, qt + 1, tid);
    const int q0 = qt * BMQ;
    const bool skip = (q0 + BMQ - 1 < kw) || (q0 > kw + 31 + W - 1) || (kw >= T);
    if (!skip) {
      const bool need_mask = (q0 < kw + 31) || (q0 + BMQ - 1 > kw + W - 1) || (q0 + BMQ > T) ||
                             (kw + 32 > T);
      f32x16 s[2], dp[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = (f32x16){};
        dp[mb] = (f32x16){};
        const bf16* qrow = sb + C::OFF_Q + (mb * 32 + l32) * C::QP + 8 * hi;
        const bf16* orow = sb + C::OFF_DO + (mb * 32 + l32) * C::QP + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          s[mb] = mfma32(*reinterpret_cast<const bf16x8*>(qrow + 16 * ks), kreg[ks], s[mb]);
          dp[mb] = mfma32(*reinterpret_cast<const bf16x8*>(orow + 16 * ks), vreg[ks], dp[mb]);
        }
      }
      bf16x8 pb[2][2], sbf[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int ql = mb * 32 + 8 * a + 4 * hi;  // first of 4 consecutive queries
          const float4 l2 = *reinterpret_cast<const float4*>(sf + ql);
          const float4 dl = *reinterpret_cast<const float4*>(sf + BMQ + ql);
          const float l2v[4] = {l2.x, l2.y, l2.z, l2.w};
          const float dlv[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * a + r;
            float pv = __builtin_amdgcn_exp2f(fmaf(s[mb][i], p.c, -l2v[r]));
            if (need_mask) {
              const int qg = q0 + ql + r;
              const bool ok = (mykey <= qg) && (mykey > qg - W) && (qg < T) && (mykey < T);
              pv = ok ? pv : 0.f;
            }
            const float ds = pv * (dp[mb][i] - dlv[r]);
            pb[mb][i >> 3][i & 7] = (bf16)pv;
            sbf[mb][i >> 3][i & 7] = (bf16)ds;
          }
        }
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16* otr = sb + C::OFF_DOT + (db * 32 + l32) * C::TP + 8 * hi;
        const bf16* qtr = sb + C::OFF_QT + (db * 32 + l32) * C::TP + 8 * hi;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int sp = 0; sp < 2; ++sp) {
            dv[db] = mfma32(pb[mb][sp], *reinterpret_cast<const bf16x8*>(otr + mb * 32 + sp * 16), dv[db]);
            dk[db] = mfma32(sbf[mb][sp], *reinterpret_cast<const bf16x8*>(qtr + mb * 32 + sp * 16), dk[db]);
          }
      }
      // dS (queries x keys) into LDS for the dQ contraction
      bf16* dsw = sb + C::OFF_DS + 32 * wave + l32;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ql = mb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
          dsw[ql * C::SP] = sbf[mb][i >> 3][i & 7];
        }
    } else {
      // this wave's keys see none of the tile: zero its dS columns
      for (int r = lane; r < BMQ * 4; r += 64) {
        const int ql = r >> 2, c = r & 3;
        *reinterpret_cast<uint4*>(sb + C::OFF_DS + ql * C::SP + 32 * wave + 8 * c) = make_uint4(0, 0, 0, 0);
      }
    }
    __syncthreads();
    // dQ slice: D=128 -> wave owns d-block `wave`, both 32-query halves; D=64 -> d-block
    // (wave & 1), query half (wave >> 1).
    {
      constexpr int NMB = (D == 128) ? 2 : 1;
      const int db = (D == 128) ? wave : (wave & 1);
#pragma unroll
      for (int j = 0; j < NMB; ++j) {
        const int mb = (D == 128) ? j : (wave >> 1);
        f32x16 acc = (f32x16){};
        const bf16* arow = sb + C::OFF_DS + (mb * 32 + l32) * C::SP + 8 * hi;
        const bf16* brow = sb + C::OFF_KT + (db * 32 + l32) * C::KTP + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < BNK / 16; ++ks)
          acc = mfma32(*reinterpret_cast<const bf16x8*>(arow + 16 * ks),
                       *reinterpret_cast<const bf16x8*>(brow + 16 * ks), acc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qg = q0 + mb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
          if (qg < T)
            unsafeAtomicAdd(p.dq_acc + (((size_t)b * T + qg) * H + h) * D + db * 32 + l32,
                            acc[i] * p.scale);
        }
      }
    }
    __syncthreads();
    if (has_next) {
      st.store(smem, tid);
      __syncthreads();
    }
  }

  // Epilogue: lane owns d = 32 db + l32 of keys kw + 8(i/4) + 4 hi + (i%4).
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = kw + 8 * (i >> 2) + 4 * hi + (i & 3);
    if (key >= T) continue;
    const size_t row = ((size_t)b * T + key) * H + h;
    float gsum = 0.f;
    float gkey = 0.f;
    if constexpr (GATE) gkey = p.gate[row];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const size_t off = row * D + db * 32 + l32;
      p.dk[off] = (bf16)(dk[db][i] * p.scale);
      p.dv[off] = (bf16)dv[db][i];
      if constexpr (GATE) {
        p.dve[off] = (bf16)(gkey * dv[db][i]);
        gsum = fmaf(dv[db][i], (float)p.ve[off], gsum);
      }
    }
    if constexpr (GATE) {
#pragma unroll
      for (int m = 1; m < 32; m <<= 1) gsum += xor_shfl(gsum, m);
      if (l32 == 0) p.dgate[row] = gsum;
    }
  }
}

}  // namespace bwdk

// ------------------------------------------------------------------------------------------
// float32 path: one wave per key row (dK, dV) and one wave per query row (dQ); no atomics.
// ------------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ float wave_dot(const float* a, const float* __restrict__ g, int lane) {
  constexpr int PER = D / 64;
  float d = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) d = fmaf(a[e], g[lane + 64 * e], d);
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) d += xor_shfl(d, m);
  return d;
}

template <int D>
__global__ void __launch_bounds__(64) bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ ve, const float* __restrict__ gate, const float* __restrict__ lse,
    const float* __restrict__ delta, const float* __restrict__ dO, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dve, float* __restrict__ dgate, int T, int H,
    int W, float scale) {
  constexpr int PER = D / 64;
  const int j = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H, lane = threadIdx.x;
  const size_t krow = ((size_t)b * T + j) * H + h;
  const float g = gate ? gate[krow] : 0.f;
  float kv[PER], vv[PER], ak[PER], av[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    kv[e] = k[krow * D + lane + 64 * e];
    vv[e] = v[krow * D + lane + 64 * e];
    if (gate) vv[e] = fmaf(g, ve[krow * D + lane + 64 * e], vv[e]);
    ak[e] = 0.f; av[e] = 0.f;
  }
  for (int i = j; i <= min(T - 1, j + W - 1); ++i) {
    const size_t qrow = ((size_t)b * T + i) * H + h;
    const float s = wave_dot<D>(kv, q + qrow * D, lane) * scale;
    const float pij = expf(s - lse[(size_t)bh * T + i]);
    const float dp = wave_dot<D>(vv, dO + qrow * D, lane);
    const float ds = pij * (dp - delta[(size_t)bh * T + i]);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      av[e] = fmaf(pij, dO[qrow * D + lane + 64 * e], av[e]);
      ak[e] = fmaf(ds, q[qrow * D + lane + 64 * e], ak[e]);
    }
  }
  float gs = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    dk[krow * D + lane + 64 * e] = ak[e] * scale;
    dv[krow * D + lane + 64 * e] = av[e];
    if (gate) {
      dve[krow * D + lane + 64 * e] = g * av[e];
      gs = fmaf(av[e], ve[krow * D + lane + 64 * e], gs);
    }
  }
  if (gate) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) gs += xor_shfl(gs, m);
    if (lane == 0) dgate[krow] = gs;
  }
}

template <int D>
__global__ void __launch_bounds__(64) bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ ve, const float* __restrict__ gate, const float* __restrict__ lse,
    const float* __restrict__ delta, const float* __restrict__ dO, float* __restrict__ dq, int T,
    int H, int W, float scale) {
  constexpr int PER = D / 64;
  const int i = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H, lane = threadIdx.x;
  const size_t qrow = ((size_t)b * T + i) * H + h;
  float qv[PER], ov[PER], aq[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    qv[e] = q[qrow * D + lane + 64 * e];
    ov[e] = dO[qrow * D + lane + 64 * e];
    aq[e] = 0.f;
  }
  const float L = lse[(size_t)bh * T + i], dl = delta[(size_t)bh * T + i];
  for (int j = max(0, i - W + 1); j <= i; ++j) {
    const size_t krow = ((size_t)b * T + j) * H + h;
    const float s = wave_dot<D>(qv, k + krow * D, lane) * scale;
    const float pij = expf(s - L);
    float dp = 0.f;
    const float g = gate ? gate[krow] : 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      float vv = v[krow * D + lane + 64 * e];
      if (gate) vv = fmaf(g, ve[krow * D + lane + 64 * e], vv);
      dp = fmaf(ov[e], vv, dp);
    }
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) dp += xor_shfl(dp, m);
    const float ds = pij * (dp - dl);
#pragma unroll
    for (int e = 0; e < PER; ++e) aq[e] = fmaf(ds, k[krow * D + lane + 64 * e], aq[e]);
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) dq[qrow * D + lane + 64 * e] = aq[e] * scale;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t bwd_workspace_bytes(int B, int T, int H, int D, bool bf16) {
  const size_t delta = align256((size_t)B * H * T * sizeof(float));
  const size_t acc = bf16 ? align256((size_t)B * T * H * D * sizeof(float)) : 0;
  return delta + acc;
}

template <typename E, int D>
static void launch_pre(const void* o, const void* dO, float* delta, float* dq_acc, int B, int T,
                       int H, hipStream_t s) {
  constexpr int TPR = D / (16 / sizeof(E));
  const int rows = B * T * H;
  const int rpb = 256 / TPR;
  hipLaunchKernelGGL((bwd_pre_kernel<E, D>), dim3((rows + rpb - 1) / rpb), dim3(256), 0, s,
                     (const E*)o, (const E*)dO, delta, dq_acc, rows, T, H);
}

template <int D, bool GATE>
static hipError_t launch_bwd_bf16_t(const AttnShape& a, const bwdk::Params& p, hipStream_t s) {
  using C = bwdk::Cfg<D>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&bwdk::bwd_bf16_kernel<D, GATE>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::SMEM);
  if (attr != hipSuccess) return attr;
  const unsigned blocks = (unsigned)p.nkb * a.B * a.H;
  hipLaunchKernelGGL((bwdk::bwd_bf16_kernel<D, GATE>), dim3(blocks), dim3(256), C::SMEM, s, p);
  return hipGetLastError();
}

namespace {
struct WsView {
  float* delta;
  float* dq_acc;  // bf16 path only
};
WsView ws_view(void* ws, int B, int T, int H, bool is_bf16) {
  WsView w;
  w.delta = reinterpret_cast<float*>(ws);
  w.dq_acc = is_bf16 ? reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                                align256((size_t)B * H * T * sizeof(float)))
                     : nullptr;
  return w;
}
}  // namespace

hipError_t launch_bwd_pre(const AttnShape& a, const void* o, const void* dO, void* ws,
                          bool is_bf16, hipStream_t s) {
  const WsView w = ws_view(ws, a.B, a.T, a.H, is_bf16);
  if (is_bf16) {
    if (a.D == 64) launch_pre<swa::bf16, 64>(o, dO, w.delta, w.dq_acc, a.B, a.T, a.H, s);
    else launch_pre<swa::bf16, 128>(o, dO, w.delta, w.dq_acc, a.B, a.T, a.H, s);
  } else {
    if (a.D == 64) launch_pre<float, 64>(o, dO, w.delta, nullptr, a.B, a.T, a.H, s);
    else launch_pre<float, 128>(o, dO, w.delta, nullptr, a.B, a.T, a.H, s);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_main(const AttnShape& a, const void* q, const void* k, const void* v,
                           const void* ve, const float* gate, const float* lse, const void* dO,
                           void* dq, void* dk, void* dv, void* dve, float* dgate, void* ws,
                           bool is_bf16, hipStream_t s) {
  const int B = a.B, T = a.T, H = a.H, D = a.D;
  const WsView w = ws_view(ws, B, T, H, is_bf16);
  if (is_bf16) {
    bwdk::Params p;
    p.q = (const bf16*)q; p.k = (const bf16*)k; p.v = (const bf16*)v; p.ve = (const bf16*)ve;
    p.gate = gate; p.lse = lse; p.delta = w.delta; p.dO = (const bf16*)dO; p.dq_acc = w.dq_acc;
    p.dk = (bf16*)dk; p.dv = (bf16*)dv; p.dve = (bf16*)dve; p.dgate = dgate;
    p.B = B; p.T = T; p.H = H; p.window = a.window;
    p.nkb = (T + bwdk::BNK - 1) / bwdk::BNK;
    p.c = a.scale * kLog2e;
    p.scale = a.scale;
    const bool g = gate != nullptr;
    if (D == 64) return g ? launch_bwd_bf16_t<64, true>(a, p, s) : launch_bwd_bf16_t<64, false>(a, p, s);
    return g ? launch_bwd_bf16_t<128, true>(a, p, s) : launch_bwd_bf16_t<128, false>(a, p, s);
  }
  dim3 grid(T, B * H);
  if (D == 64) {
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<64>, grid, dim3(64), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)ve, gate, lse, w.delta, (const float*)dO,
                       (float*)dk, (float*)dv, (float*)dve, dgate, T, H, a.window, a.scale);
    hipLaunchKernelGGL(bwd_dq_f32_kernel<64>, grid, dim3(64), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)ve, gate, lse, w.delta, (const float*)dO,
                       (float*)dq, T, H, a.window, a.scale);
  } else {
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<128>, grid, dim3(64), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)ve, gate, lse, w.delta, (const float*)dO,
                       (float*)dk, (float*)dv, (float*)dve, dgate, T, H, a.window, a.scale);
    hipLaunchKernelGGL(bwd_dq_f32_kernel<128>, grid, dim3(64), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)ve, gate, lse, w.delta, (const float*)dO,
                       (float*)dq, T, H, a.window, a.scale);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_final(const AttnShape& a, void* dq, void* ws, bool is_bf16, hipStream_t s) {
  if (!is_bf16) return hipSuccess;  // the fp32 path writes dq directly
  const WsView w = ws_view(ws, a.B, a.T, a.H, is_bf16);
  const size_t n8 = (size_t)a.B * a.T * a.H * a.D / 8;
  hipLaunchKernelGGL(bwd_dq_final_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                     w.dq_acc, (bf16*)dq, n8);
  return hipGetLastError();
}

}  // namespace swa

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
//    L2), longest blocks first; small full-causal grids longest first across heads (lpt_block).
//  * Optional value-embedding gate: v_eff = v + gate * ve is formed in fp32 while the V tile is
//    staged into LDS, so v_eff never touches HBM.
#include "common.h"
#include "internal.h"
#include "rope_row.h"

namespace swa {

namespace fwdk {

constexpr int NW = 4;          // waves per workgroup
constexpr int BM = 32 * NW;    // query rows per workgroup
constexpr int BN = 64;         // keys per tile

template <int D> struct Cfg {
  static constexpr int CH = D / 8;          // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;       // rows per wave-wide 1 KiB load
  static constexpr int NI = BN / RPI;       // 1 KiB loads per tile
  static constexpr int NIW = NI / NW;       // ... per wave
  static constexpr int TILE = BN * D;       // elements per K or V tile
  static constexpr int CPT = BN * CH / (64 * NW);   // chunks per thread (register-staged gate path)
};

struct Params {
  const bf16* q; const bf16* k; const bf16* v; const bf16* ve; const float* gate;
  const int* bounds;   // per-token document [start, end) (document masking only)
  const int* ve_ids;   // value-embedding table rows per token (table mode only)
  int ve_rows;
  bf16* o; float* lse;
  const bf16* qraw; const float* cs; float eps; bf16* qn;   // QN kernels: the query prologue
  int B, T, H, window, nqb;
  int lpt;      // longest-first order across heads (lpt_order)
  float c;      // scale * log2(e)
};

// Online-softmax reference updates only when a row max grows by more than 2^8 (see kernel).
constexpr float kRescaleSlack = 8.0f;

template <int D, bool GATE>
struct Tiles {
  using C = Cfg<D>;
  // Lane-constant part of the asynchronous tile loads: lane l of wave load I lands at row
  // I*RPI + l/CH, position l%CH, and fetches source chunk (l%CH) ^ swz(row).
  int row[C::NIW];         // tile row of each of this wave's loads
  unsigned loff[C::NIW];   // byte offset of the fetched chunk within a tile that starts at row 0
  int ldst[C::NIW];        // LDS element offset of the wave load inside a tile buffer
  __device__ __forceinline__ void init(int H, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < C::NIW; ++i) {
      const int I = wave * C::NIW + i;
      row[i] = I * C::RPI + lane / C::CH;
      loff[i] = 2u * (unsigned)(row[i] * H * D + 8 * ((lane % C::CH) ^ swz<D>(row[i])));
      ldst[i] = I * C::RPI * D;
    }
  }
  // Issue the loads of key tile kt into (ks, vs): buffer resource at the tile base + 32-bit lane offset.
  // In the last tile, rows past the sequence end re-read row T-1 (their scores are masked).
  __device__ __forceinline__ void load(const Params& p, const bf16* kbase, const bf16* vbase,
                                       lds_t<bf16>* ks, lds_t<bf16>* vs, int kt, int tid) const {
    const int T = p.T;
    const size_t rs = (size_t)p.H * D;
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kbase + (size_t)kt * BN * rs);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vbase + (size_t)kt * BN * rs);
    if (kt * BN + BN <= T) {
#pragma unroll
      for (int i = 0; i < C::NIW; ++i) {
        const unsigned o = opaque(loff[i]);
        b2lds16(rk, o, (lds_t<void>*)(ks + ldst[i]));
        if constexpr (!GATE) b2lds16(rv, o, (lds_t<void>*)(vs + ldst[i]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::NIW; ++i) {
        const int over = max(kt * BN + row[i] - (T - 1), 0);
        const unsigned off = opaque(loff[i]) - 2u * (unsigned)over * (unsigned)rs;
        b2lds16(rk, off, (lds_t<void>*)(ks + ldst[i]));
        if constexpr (!GATE) b2lds16(rv, off, (lds_t<void>*)(vs + ldst[i]));
      }
    }
    if constexpr (GATE) {
      // v_eff = v + gate * ve is formed in fp32 on the way into LDS
#pragma unroll
      for (int j = 0; j < C::CPT; ++j) {
        const int id = tid + 64 * NW * j;
        const int r = id / C::CH, pos = id % C::CH;
        const int c = pos ^ swz<D>(r);
        const int grow = min(kt * BN + r, T - 1);
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

template <int D>
struct WaveState {
  static constexpr int NDB = D / 32;
  f32x16 oacc[NDB];
  float m_ref, l_run;
};

// One 64-key tile for one wave (32 query rows): S^T = K Q^T, mask, online softmax, O^T += V^T P^T.
template <int D>
__device__ __forceinline__ void tile_step(WaveState<D>& ws, const bf16x8* qreg,
                                          const lds_t<bf16>* ks, const lds_t<bf16>* vs,
                                          const int* krow, const int* vtr1, const int* vtr2,
                                          int k0, int qw, int T, const RowRange& rr, float c,
                                          int lane) {
  constexpr int NKS = D / 16, NDB = D / 32;
  const int l32 = lane & 31, hi = lane >> 5;
  const bool skip = (k0 > qw + 31) || (k0 + BN - 1 < rr.wlo0);
  if (skip) return;
  const bool need_mask = (k0 + BN - 1 > qw) || (k0 < rr.wlo1) || (k0 + BN > T);
  // All K operands of the tile are requested before the S MFMAs and all V^T operands right
  // after them, so the LDS reads overlap one another (and the softmax arithmetic) instead of
  // each MFMA waiting for its own read.
  bf16x8 ka0[NKS], ka1[NKS];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) ka0[kk] = *reinterpret_cast<const lds_t<bf16x8>*>(ks + krow[kk]);
  sched_fence();
  f32x16 s[2];
  s[0] = (f32x16){};
  s[1] = (f32x16){};
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) s[0] = mfma32(ka0[kk], qreg[kk], s[0]);
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk)
    ka1[kk] = *reinterpret_cast<const lds_t<bf16x8>*>(ks + 32 * D + krow[kk]);
  sched_fence();
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) s[1] = mfma32(ka1[kk], qreg[kk], s[1]);
  auto read_v = [&](bf16x8 (&dst)[NDB][2], int kb) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const int ro = (kb * 32 + sp * 16) * D;
        dst[db][sp] = __builtin_shufflevector(ds_read_tr16(vs + ro + vtr1[db]),
                                              ds_read_tr16(vs + ro + vtr2[db]),
                                              0, 1, 2, 3, 4, 5, 6, 7);
      }
  };
  bf16x8 va0[NDB][2];
  read_v(va0, 0);
  sched_fence();
  if (need_mask) {
    branch_keep();
    // key k0 + t is visible iff t - lo lies in [0, n): the row's keys are [rr.lo, rr.lo + rr.n)
    const int lo = rr.lo - k0 - 4 * hi;
    const unsigned n = rr.n;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = kb * 32 + 8 * (i >> 2) + (i & 3);   // key offset minus 4*hi
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
  // Lazy rescale: the reference m_ref only moves when some row's max exceeds it by more than
  // kRescaleSlack (in log2 units), so exp2(s*c - m_ref) <= 2^8 and the O rescale is rare.
  // Every term of a row is weighted against the same reference, so the result is exact.
  if (__builtin_amdgcn_ballot_w64(mt > ws.m_ref + kRescaleSlack) != 0) {
    branch_keep();
    const float m_new = fmaxf(ws.m_ref, mt);
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(ws.m_ref - m_new);
    ws.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) ws.oacc[db] *= alpha;
    ws.m_ref = m_new;
  }
  const float m_use = (ws.m_ref == -INFINITY) ? 0.f : ws.m_ref;
  float lsum = 0.f;
  bf16x8 pb[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        e[j] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * sp + j], c, -m_use));
        lsum += e[j];
      }
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const bf16x2 t = __builtin_convertvector((f32x2){e[j], e[j + 1]}, bf16x2);
        pb[kb][sp][j] = t[0];
        pb[kb][sp][j + 1] = t[1];
      }
    }
  ws.l_run += lsum;
  sched_fence();
  // O^T += V^T P^T
  bf16x8 va1[NDB][2];
  read_v(va1, 1);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) ws.oacc[db] = mfma32(va0[db][sp], pb[0][sp], ws.oacc[db]);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) ws.oacc[db] = mfma32(va1[db][sp], pb[1][sp], ws.oacc[db]);
}

template <int D, bool GATE, bool DOC, bool QN>
__global__ void __launch_bounds__(64 * NW, 8 / NW) fwd_bf16_kernel(Params p) {
  using C = Cfg<D>;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  __shared__ __attribute__((aligned(16))) bf16 k0s[C::TILE], v0s[C::TILE], k1s[C::TILE], v1s[C::TILE];
  lds_t<bf16>* K0 = (lds_t<bf16>*)k0s;
  lds_t<bf16>* V0 = (lds_t<bf16>*)v0s;
  lds_t<bf16>* K1 = (lds_t<bf16>*)k1s;
  lds_t<bf16>* V1 = (lds_t<bf16>*)v1s;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int T = p.T, H = p.H, W = p.window;

  // XCD-aware, longest-first block order.
  int bh, qb;
  if (p.lpt) {
    const int2 br = lpt_block(p.nqb, kCusPerXcd);
    bh = br.x;
    qb = p.nqb - 1 - br.y;
  } else {
    const int nblk = gridDim.x;
    int L = blockIdx.x;
    if ((nblk & 7) == 0) L = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    bh = L / p.nqb;
    qb = p.nqb - 1 - (L - bh * p.nqb);
  }
  const int b = bh / H, h = bh - b * H;
  const size_t head0 = ((size_t)b * T * H + h) * D;   // element (b, 0, h, 0)
  const bf16* kbase = p.k + head0;
  const bf16* vbase = p.v + head0;

  const int q0 = qb * BM;
  const int qw = q0 + wave * 32;      // first query of this wave
  const int myq = qw + l32;           // this lane's query row

  const RowRange rr = row_range<DOC>(p.bounds, b, T, W, myq);
  int lo_q0 = max(q0 - W + 1, 0);   // first key any query of the workgroup sees
  if constexpr (DOC) lo_q0 = max(lo_q0, p.bounds[2 * ((size_t)b * T + q0)]);
  const int kt_lo = lo_q0 / BN;
  const int kt_hi = min(T - 1, q0 + BM - 1) / BN;

  Tiles<D, GATE> tl;
  tl.init(H, wave, lane);
  if constexpr (QN) tl.load(p, kbase, vbase, K0, V0, kt_lo, tid);   // overlaps the query prologue

  // Q^T operand: 8 bf16 of row myq per k-step, held for the whole kernel.
  bf16x8 qreg[NKS];
  if constexpr (QN) {
    // The query rows' prologue (RoPE, then RMS norm) in the row layout of rope_row.h, so that
    // each normalised row is bitwise what rope_qknorm_fwd writes: TPR lanes per row, RPP rows
    // per pass. Each row goes to qn and, 16-byte chunks XOR-swizzled as in the K tiles, to the
    // second K/V buffers (rows 0-63 in K1, 64-127 in V1; unused until the second key tile),
    // from which every wave then reads its 32 rows as the Q^T operand.
    using RW = RowWord<bf16>;
    constexpr int VPT = RW::VPT, TPR = D / VPT, RPP = 64 * NW / TPR, NP = BM / RPP;
    const int lr = tid % TPR;
    const bool second = lr >= TPR / 2;
    // every pass's row and angle loads first (rows past the end re-read the last row and
    // store nothing), then the arithmetic
    RW x[NP];
    float c[NP][VPT], s[NP][VPT];
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
      const int t = min(q0 + pass * RPP + tid / TPR, T - 1);
      x[pass].load_stream(p.qraw + head0 + (size_t)t * H * D + lr * VPT);
      load_cs<VPT>(p.cs, t, D / 2, (lr % (TPR / 2)) * VPT, c[pass], s[pass]);
    }
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
      const int r = pass * RPP + tid / TPR;
      const int t = q0 + r;
      RW out;
      rope_norm_row<VPT, TPR, D>(x[pass].v, c[pass], s[pass], second, p.eps, out.v);
      u32x4 w = {0u, 0u, 0u, 0u};   // rows past the end: zero operands
      if (t < T) {
        out.store(p.qn + head0 + (size_t)t * H * D + lr * VPT);
        w = (u32x4){pack_bf2(out.v[0], out.v[1]), pack_bf2(out.v[2], out.v[3]),
                    pack_bf2(out.v[4], out.v[5]), pack_bf2(out.v[6], out.v[7])};
      }
      const int rl = r & 63;
      *reinterpret_cast<lds_t<u32x4>*>((r < 64 ? K1 : V1) + rl * D + 8 * (lr ^ swz<D>(rl))) = w;
    }
    __syncthreads();
    const lds_t<bf16>* qs = (wave < 2 ? K1 : V1);
    const int rl = 32 * (wave & 1) + l32;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qreg[ks] = *reinterpret_cast<const lds_t<bf16x8>*>(qs + rl * D +
                                                          8 * ((2 * ks + hi) ^ swz<D>(rl)));
  } else {
    const bf16* qp = p.q + head0 + (size_t)min(myq, T - 1) * H * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 w = *reinterpret_cast<const uint4*>(qp + 16 * ks);
      if (myq >= T) w = make_uint4(0, 0, 0, 0);
      qreg[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }


  WaveState<D> ws;
#pragma unroll
  for (int i = 0; i < NDB; ++i) ws.oacc[i] = (f32x16){};
  ws.m_ref = -INFINITY;
  ws.l_run = 0.f;

  // Lane-constant LDS element offsets (plus compile-time row offsets at each use): K rows for
  // the S^T MFMA A operand (row l32, chunk 2 kk + hi) and the two transposing reads of V^T
  // (rows 4 hi + (j / 4) and + 8, 4 dims of d-block db), all through the chunk swizzle, which
  // depends only on the row modulo 16.
  int krow[NKS], vtr1[NDB], vtr2[NDB];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) krow[kk] = l32 * D + 8 * ((2 * kk + hi) ^ swz<D>(l32));
  {
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 32 * db + 16 * (g & 1) + 4 * (j & 3);
      const int r1 = 4 * hi + (j >> 2), r2 = r1 + 8;
      vtr1[db] = r1 * D + 8 * ((d >> 3) ^ swz<D>(r1)) + 4 * ((d >> 2) & 1);
      vtr2[db] = r2 * D + 8 * ((d >> 3) ^ swz<D>(r2)) + 4 * ((d >> 2) & 1);
    }
  }

  if constexpr (!QN) tl.load(p, kbase, vbase, K0, V0, kt_lo, tid);
  wait_vmem();
  __syncthreads();
  // Two tiles per trip so that each LDS buffer is named statically.
  for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
    if (kt + 1 <= kt_hi) tl.load(p, kbase, vbase, K1, V1, kt + 1, tid);
    tile_step<D>(ws, qreg, K0, V0, krow, vtr1, vtr2, kt * BN, qw, T, rr, p.c, lane);
    wait_vmem();
    __syncthreads();
    if (kt + 1 > kt_hi) break;
    if (kt + 2 <= kt_hi) tl.load(p, kbase, vbase, K0, V0, kt + 2, tid);
    tile_step<D>(ws, qreg, K1, V1, krow, vtr1, vtr2, (kt + 1) * BN, qw, T, rr, p.c, lane);
    wait_vmem();
    __syncthreads();
  }

  // Epilogue: combine the two half-wave partial sums, normalise, store O and lse.
  const float l_tot = ws.l_run + half_swap(ws.l_run);
  const float inv = 1.0f / l_tot;
  // O in 16-byte pieces (store_orow16): half the store instructions of 8-byte pieces;
  // measured 2.5-3.5 % off the forward.
  bf16* op = p.o + head0 + (size_t)min(myq, T - 1) * H * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_orow16(op, db, ws.oacc[db], inv, hi, myq < T);
  if (myq < T && hi == 0)
    p.lse[((size_t)b * H + h) * T + myq] = (ws.m_ref + __log2f(l_tot)) * kLn2;
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
                                                     const int* __restrict__ bounds,
                                                     const int* __restrict__ ve_ids, int ve_rows,
                                                     float* __restrict__ o, float* __restrict__ lse,
                                                     int T, int H, int W, float scale) {
  constexpr int PER = D / 64;
  const int i = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H, lane = threadIdx.x;
  const size_t qrow = ((size_t)b * T + i) * H + h;
  float qv[PER], acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) { qv[e] = q[qrow * D + lane + 64 * e]; acc[e] = 0.f; }
  float m = -INFINITY, l = 0.f;
  const int j0 = max(max(0, i - W + 1), bounds ? bounds[2 * ((size_t)b * T + i)] : 0);
  for (int j = j0; j <= i; ++j) {
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
    const float* er = gate ? ve_row<D>(ve, ve_ids, ve_rows, b, T, H, h, j) : nullptr;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      float vv = v[krow * D + lane + 64 * e];
      if (er) vv = fmaf(g, er[lane + 64 * e], vv);
      acc[e] = fmaf(acc[e], alpha, pj * vv);
    }
    m = m_new;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) o[qrow * D + lane + 64 * e] = acc[e] / l;
  if (lane == 0) lse[(size_t)bh * T + i] = m + logf(l);
}

template <int D, bool GATE, bool QN>
static hipError_t launch_fwd_bf16_t(const AttnShape& a, const void* q, const void* k, const void* v,
                                    const void* ve, const float* gate, void* o, float* lse,
                                    hipStream_t s, const QNorm* qnorm) {
  fwdk::Params p;
  p.q = (const bf16*)q; p.k = (const bf16*)k; p.v = (const bf16*)v; p.ve = (const bf16*)ve;
  p.ve_ids = a.ve_ids; p.ve_rows = a.ve_rows;
  p.gate = gate; p.bounds = a.bounds; p.o = (bf16*)o; p.lse = lse;
  p.B = a.B; p.T = a.T; p.H = a.H; p.window = a.window;
  p.nqb = (a.T + fwdk::BM - 1) / fwdk::BM;
  p.lpt = lpt_order(a) ? 1 : 0;
  p.c = a.scale * kLog2e;
  p.qraw = nullptr; p.cs = nullptr; p.eps = 0.f; p.qn = nullptr;
  if (QN) {
    p.qraw = (const bf16*)qnorm->q; p.cs = qnorm->cs; p.eps = qnorm->eps;
    p.qn = (bf16*)qnorm->qn;
  }
  const unsigned blocks = (unsigned)p.nqb * a.B * a.H;
  if (a.bounds)
    hipLaunchKernelGGL((fwdk::fwd_bf16_kernel<D, GATE, true, QN>), dim3(blocks),
                       dim3(64 * fwdk::NW), 0, s, p);
  else
    hipLaunchKernelGGL((fwdk::fwd_bf16_kernel<D, GATE, false, QN>), dim3(blocks),
                       dim3(64 * fwdk::NW), 0, s, p);
  return hipGetLastError();
}

template <int D, bool GATE>
static hipError_t launch_fwd_bf16_q(const AttnShape& a, const void* q, const void* k,
                                    const void* v, const void* ve, const float* gate, void* o,
                                    float* lse, hipStream_t s, const QNorm* qnorm) {
  return qnorm ? launch_fwd_bf16_t<D, GATE, true>(a, q, k, v, ve, gate, o, lse, s, qnorm)
               : launch_fwd_bf16_t<D, GATE, false>(a, q, k, v, ve, gate, o, lse, s, qnorm);
}

hipError_t launch_fwd(const AttnShape& a, const void* q, const void* k, const void* v,
                      const void* ve, const float* gate, void* o, float* lse, bool is_bf16,
                      hipStream_t s, const QNorm* qnorm) {
  if (is_bf16) {
    const bool g = gate != nullptr;
    if (a.D == 64)
      return g ? launch_fwd_bf16_q<64, true>(a, q, k, v, ve, gate, o, lse, s, qnorm)
               : launch_fwd_bf16_q<64, false>(a, q, k, v, ve, gate, o, lse, s, qnorm);
    return g ? launch_fwd_bf16_q<128, true>(a, q, k, v, ve, gate, o, lse, s, qnorm)
             : launch_fwd_bf16_q<128, false>(a, q, k, v, ve, gate, o, lse, s, qnorm);
  }
  if (qnorm) return hipErrorInvalidValue;   // the fused query prologue is bf16 only
  dim3 grid(a.T, a.B * a.H);
  if (a.D == 64)
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(64), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)ve, gate, a.bounds, a.ve_ids, a.ve_rows, (float*)o, lse, a.T, a.H, a.window,
                       a.scale);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(64), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)ve, gate, a.bounds, a.ve_ids, a.ve_rows, (float*)o, lse, a.T, a.H, a.window,
                       a.scale);
  return hipGetLastError();
}

}  // namespace swa

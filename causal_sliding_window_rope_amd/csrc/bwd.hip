// Causal sliding-window attention backward for gfx950, by recomputation of the scores
// ("GPT-2 124M 复现" §19: the backward recomputes intermediates, trading FLOPs for HBM traffic).
//
//   delta_i = dO_i . O_i                                 (preprocess kernel)
//   P = exp(s - lse), dV = P^T dO, dP = dO V^T, dS = P (dP - delta),
//   dK = scale dS^T Q                                    (this file, key-block major)
//   dQ = scale dS K                                      (dq.hip, query-block major)
//
// Splitting dK/dV from dQ costs one more recomputation of S and dP (6 D instead of 4 D extra
// FLOPs per visible pair) but removes the float atomics, the dQ accumulator with its zeroing
// and its bf16 conversion pass, and makes every gradient bitwise repeatable.
//
// bf16 dK/dV kernel (one workgroup = 4 waves = 128 keys of one (b, h); query tiles of 128):
//  * S = Q K^T and dP = dO V^T on v_mfma_f32_32x32x16_bf16 with B = the wave's 32 key rows of
//    K and V held in VGPRs for the whole kernel and A = the query tile's rows from LDS. In the
//    32x32 accumulator layout each lane then owns one key and 16 queries, so P^T and dS^T are
//    already in the A-operand layout of dV += P^T dO and dK += dS^T Q (fixed permutation of the
//    query order, matched by the transposing LDS reads of the dO and Q tiles).
//  * Query tiles are double-buffered in LDS by asynchronous global->LDS copies; 32-query
//    halves that lie wholly outside a wave's keys' windows are skipped by that wave.
//  * Workgroup order: all key blocks of one (b, h) on one XCD; small full-causal grids longest
//    first across heads (lpt_block).
//  * Value-embedding gate: v_eff = v + gate * ve is formed in fp32 when the V rows are loaded;
//    the epilogue writes dv = dv_eff, dve = gate * dv_eff and dgate = sum_d dv_eff * ve.
//  * STORE_DS: the bf16 dS^T each wave forms for dK is also written, one 2 KiB chunk per
//    32-query unit (dsbuf.h), for dq_ds_kernel (dqds.hip), which then needs only dQ = scale dS K
//    instead of recomputing S, P and dP.
//  * Scores in exp2 units: the wave's K rows are multiplied by scale * log2(e) once, when they
//    are loaded, and rounded back to bf16 as the MFMA operand. This rounding (relative 2^-9 per
//    element) is not in the forward; on the CPU, with everything else exact, it moves dq, dk, dv
//    by 1.7e-3 relative L2 (T = 512, W = 256, D = 128), a sixth of the 1e-2 bar.
#include "common.h"
#include "dsbuf.h"
#include "internal.h"

namespace swa {

// ------------------------------------------------------------------------------------------
// ndelta_i = -sum_d dO[i, d] * O[i, d] and nlse2_i = -lse_i * log2(e), both (B, H, T).
// One workgroup = 64 consecutive positions t of one (b, h): D / (16 / sizeof(E)) lanes per row
// (one 16-byte load of O and of dO each), all the rows' loads issued before any arithmetic, and
// the row terms written as contiguous runs of the (B, H, T) arrays.
// ------------------------------------------------------------------------------------------
// Rows of slack zeroed behind each row-term array (a query tile is 128 rows).
constexpr int kRowTermSlackRows = 128;
constexpr int kPreRows = 64;   // positions per workgroup

template <typename E, int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const E* __restrict__ o,
                                                      const E* __restrict__ dO,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ ndelta,
                                                      float* __restrict__ nlse2, int T, int H,
                                                      int nbh) {
  constexpr int VPT = 16 / sizeof(E), TPR = D / VPT, RPP = 256 / TPR, PASSES = kPreRows / RPP;
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int t0 = blockIdx.x * kPreRows;
  // The 128-query tiles of the bf16 dK/dV kernel read the row terms of the last head up to 127
  // rows past its end, in the slack behind each array: positions T .. T + 127 of the last head
  // are written as zeros, so that a workspace holding NaN or Inf bit patterns cannot reach
  // dS = P (dP - delta) of a masked query.
  auto zero_slack = [&](int t) {
    if (bh == nbh - 1 && t >= T && t - T < kRowTermSlackRows) {
      ndelta[(size_t)nbh * T + (t - T)] = 0.f;
      nlse2[(size_t)nbh * T + (t - T)] = 0.f;
    }
  };
  if (t0 >= T) {
    if (threadIdx.x < kPreRows) zero_slack(t0 + (int)threadIdx.x);
    return;
  }
  const int lr = threadIdx.x % TPR, rr = threadIdx.x / TPR;
  uint4 a[PASSES], g[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int t = min(t0 + i * RPP + rr, T - 1);
    const size_t off = (((size_t)b * T + t) * H + h) * D + lr * VPT;
    // O is read by no later kernel of the backward: nontemporal. dO is, by dK/dV right after.
    {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o + off));
      a[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    g[i] = *reinterpret_cast<const uint4*>(dO + off);
  }
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    float acc;
    if constexpr (VPT == 4) {
      acc = __uint_as_float(a[i].x) * __uint_as_float(g[i].x);
      acc = fmaf(__uint_as_float(a[i].y), __uint_as_float(g[i].y), acc);
      acc = fmaf(__uint_as_float(a[i].z), __uint_as_float(g[i].z), acc);
      acc = fmaf(__uint_as_float(a[i].w), __uint_as_float(g[i].w), acc);
    } else {
      const uint32_t aw[4] = {a[i].x, a[i].y, a[i].z, a[i].w};
      const uint32_t gw[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
      acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(bf_lo(aw[e]), bf_lo(gw[e]), acc);
        acc = fmaf(bf_hi(aw[e]), bf_hi(gw[e]), acc);
      }
    }
    acc = group_sum<TPR>(acc);
    const int t = t0 + i * RPP + rr;
    if (lr == 0 && t < T) {
      const size_t r = (size_t)bh * T + t;
      // stored negated: the bf16 kernels seed their S and dP accumulators with these
      ndelta[r] = -acc;
      nlse2[r] = -lse[r] * kLog2e;   // log2-domain row term of the exp2
    } else if (lr == 0) {
      zero_slack(t);
    }
  }
}

namespace bwdk {

constexpr int NW = 4;
constexpr int BNK = 32 * NW;  // keys per workgroup
constexpr int BMQ = 128;      // queries per tile (4 halves of 32, processed one after another)

template <int D> struct Cfg {
  static constexpr int CH = D / 8;            // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;         // rows per 1 KiB wave load
  static constexpr int QTILE = BMQ * D;       // elements of a Q or dO tile
  static constexpr int NIQ = BMQ / RPI / NW;  // wave loads per tile per wave
};

struct Params {
  const bf16* q; const bf16* k; const bf16* v; const bf16* ve; const float* gate;
  const float* nlse2; const float* ndelta; const bf16* dO;   // row terms, negated
  const int* bounds;   // per-token document [start, end) (document masking only)
  bf16* dk; bf16* dv; bf16* dve; float* dgate;
  const int* ve_ids;   // table mode: ve is (ve_rows, H*D), dve_tab the float table gradient
  int ve_rows;
  float* dve_tab;
  bf16* ds;      // stored dS^T (dsbuf.h), written by the STORE_DS instantiation
  int nslot;     // query-tile slots per key block in ds
  int B, T, H, window, nkb;
  int lpt;       // longest-first order across heads (lpt_order)
  float c;       // scale * log2(e)
  float scale;
};

// Asynchronous loads of query tile qt (Q, dO rows and the negated row terms) into LDS, part
// `part` of NPART: the tile's copies are issued in NPART portions spread over the previous
// tile's units, because a burst of them stalls the wave at issue until the copy path has
// drained enough of them (it moves far fewer bytes per clock than the matrix cores consume).
template <int D, int NPART = 1>
__device__ __forceinline__ void load_qtile(const Params& p, const bf16* qbase, const bf16* obase,
                                           const float* l2base, const float* dlbase,
                                           lds_t<bf16>* Qs, lds_t<bf16>* Os, lds_t<float>* Ls,
                                           lds_t<float>* Dls, int qt, int wave, int lane,
                                           int part = 0) {
  using C = Cfg<D>;
  static_assert(C::NIQ % NPART == 0, "copies split evenly");
  constexpr int PER = C::NIQ / NPART;
  const size_t rs = (size_t)p.H * D;
  // buffer copies relative to the tile's first row (32-bit lane offsets within one tile)
  const size_t t0 = (size_t)qt * BMQ * rs;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(qbase + t0), ro = buf_rsrc(obase + t0);
#pragma unroll
  for (int i = part * PER; i < part * PER + PER; ++i) {
    const int I = wave * C::NIQ + i;
    const int r = I * C::RPI + lane / C::CH;
    const int c = (lane % C::CH) ^ swz<D>(r);
    const unsigned vo = 2u * ((unsigned)(min(qt * BMQ + r, p.T - 1) - qt * BMQ) * (unsigned)rs +
                              8u * c);
    b2lds16(rq, vo, (lds_t<void>*)(Qs + I * C::RPI * D));
    b2lds16(ro, vo, (lds_t<void>*)(Os + I * C::RPI * D));
  }
  if (part == 0 && lane < BMQ / 4 && wave < 2) {
    // a tile that runs past the sequence end reads into the next head's row or the workspace
    // slack (see bwd_workspace_bytes); those queries are masked
    const __amdgpu_buffer_rsrc_t rl = buf_rsrc((wave == 0 ? l2base : dlbase) + qt * BMQ);
    b2lds16(rl, 16u * lane, (lds_t<void>*)(wave == 0 ? Ls : Dls));
  }
}

// Scheduling of N MFMAs with the LDS reads written after them (a row term and the operand rows
// of one 32-query unit, 4 + N reads when N = D / 16): each MFMA is followed by two reads for the
// first four, then by one.
template <int N, int I = 0>
__device__ __forceinline__ void mfma_ds_interleave() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, I < 4 ? 2 : 1, 0);      // LDS reads
    mfma_ds_interleave<N, I + 1>();
  }
}

template <int D, bool GATE, bool DOC, bool STORE_DS>
__global__ void __launch_bounds__(256, D == 64 ? 2 : 1) dkdv_bf16_kernel(Params p) {
  using C = Cfg<D>;
  constexpr int NDB = D / 32, NKS = D / 16;
  __shared__ __attribute__((aligned(16))) bf16 q0_[C::QTILE], q1_[C::QTILE], o0_[C::QTILE],
      o1_[C::QTILE];
  __shared__ __attribute__((aligned(16))) float l0_[BMQ], l1_[BMQ], d0_[BMQ], d1_[BMQ];
  lds_t<bf16>* Q0 = (lds_t<bf16>*)q0_;
  lds_t<bf16>* Q1 = (lds_t<bf16>*)q1_;
  lds_t<bf16>* O0 = (lds_t<bf16>*)o0_;
  lds_t<bf16>* O1 = (lds_t<bf16>*)o1_;
  lds_t<float>* L0 = (lds_t<float>*)l0_;
  lds_t<float>* L1 = (lds_t<float>*)l1_;
  lds_t<float>* D0 = (lds_t<float>*)d0_;
  lds_t<float>* D1 = (lds_t<float>*)d1_;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int g = lane >> 4, j = lane & 15;
  const int T = p.T, H = p.H, W = p.window;

  int bh, kbk;   // key block kbk of (b, h); the first key blocks see the most queries
  if (p.lpt) {
    const int2 br = lpt_block(p.nkb);
    bh = br.x;
    kbk = br.y;
  } else {
    const int nblk = gridDim.x;
    int L = blockIdx.x;
    if ((nblk & 7) == 0) L = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    bh = L / p.nkb;
    kbk = L - bh * p.nkb;
  }
  const int b = bh / H, h = bh - b * H;
  const size_t head0 = ((size_t)b * T * H + h) * D;
  const size_t rs = (size_t)H * D;
  const int kb0 = kbk * BNK;
  const int kw = kb0 + 32 * wave;
  const int mykey = kw + l32;
  const bf16* qbase = p.q + head0;
  const bf16* obase = p.dO + head0;
  const float* l2base = p.nlse2 + (size_t)bh * T;
  const float* dlbase = p.ndelta + (size_t)bh * T;

  // B operands of S = Q K^T and dP = dO V^T: this lane's key row of K and of v_eff.
  bf16x8 kreg[NKS], vreg[NKS];
  {
    const size_t row = head0 + (size_t)min(mykey, T - 1) * rs;
    const bool ok = mykey < T;
    float gk = 0.f;
    if constexpr (GATE) gk = p.gate[(size_t)(b * T + min(mykey, T - 1)) * H + h];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const size_t off = row + 16 * ks + 8 * hi;
      uint4 kk = *reinterpret_cast<const uint4*>(p.k + off);
      uint4 vv = *reinterpret_cast<const uint4*>(p.v + off);
      if constexpr (GATE) {
        const bf16* er = ve_row<D>(p.ve, p.ve_ids, p.ve_rows, b, T, H, h, min(mykey, T - 1));
        const uint4 ee = er ? *reinterpret_cast<const uint4*>(er + 16 * ks + 8 * hi)
                            : make_uint4(0, 0, 0, 0);
        vv.x = pack_bf2(fmaf(gk, bf_lo(ee.x), bf_lo(vv.x)), fmaf(gk, bf_hi(ee.x), bf_hi(vv.x)));
        vv.y = pack_bf2(fmaf(gk, bf_lo(ee.y), bf_lo(vv.y)), fmaf(gk, bf_hi(ee.y), bf_hi(vv.y)));
        vv.z = pack_bf2(fmaf(gk, bf_lo(ee.z), bf_lo(vv.z)), fmaf(gk, bf_hi(ee.z), bf_hi(vv.z)));
        vv.w = pack_bf2(fmaf(gk, bf_lo(ee.w), bf_lo(vv.w)), fmaf(gk, bf_hi(ee.w), bf_hi(vv.w)));
      }
      // K pre-scaled by scale * log2(e), so S comes out of the MFMA in exp2 units
      kk.x = pack_bf2(p.c * bf_lo(kk.x), p.c * bf_hi(kk.x));
      kk.y = pack_bf2(p.c * bf_lo(kk.y), p.c * bf_hi(kk.y));
      kk.z = pack_bf2(p.c * bf_lo(kk.z), p.c * bf_hi(kk.z));
      kk.w = pack_bf2(p.c * bf_lo(kk.w), p.c * bf_hi(kk.w));
      if (!ok) { kk = make_uint4(0, 0, 0, 0); vv = make_uint4(0, 0, 0, 0); }
      kreg[ks] = __builtin_bit_cast(bf16x8, kk);
      vreg[ks] = __builtin_bit_cast(bf16x8, vv);
    }
  }

  f32x16 dv[NDB], dk[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) { dv[i] = (f32x16){}; dk[i] = (f32x16){}; }

  // Queries that see this lane's key: [key, hi_key] (window, sequence end and, with document
  // masking, the end of the key's document); whi0 / whi1: hi_key of the wave's first and last
  // key (hi_key never decreases along a row).
  const int kc = min(mykey, T - 1);
  int kend = T;
  if constexpr (DOC) kend = p.bounds[2 * ((size_t)b * T + kc) + 1];
  const int hi_key = min(kc + W - 1, kend - 1);
  const int whi0 = __builtin_amdgcn_readlane(hi_key, 0);
  const int whi1 = __builtin_amdgcn_readlane(hi_key, 31);
  int hi_wg = min(T - 1, kb0 + BNK - 1 + W - 1);   // last query any key of the workgroup sees
  if constexpr (DOC) {
    const int kl = min(kb0 + BNK - 1, T - 1);
    hi_wg = min(kl + W - 1, p.bounds[2 * ((size_t)b * T + kl) + 1] - 1);
  }
  const int qt_lo = kb0 / BMQ;
  const int qt_hi = hi_wg / BMQ;

  // Lane-constant LDS element offsets: every swizzled address below is one of these plus a
  // compile-time row offset, so the LDS loads use immediate offsets off a few registers.
  const int jr = j >> 2, jc = j & 3;
  int rowb[NKS];   // 128-bit row reads, row (32 mb + l32), chunk 2 ks + hi
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) rowb[ks] = l32 * D + 8 * ((2 * ks + hi) ^ swz<D>(l32));
  int trb1[NDB], trb2[NDB];  // transposing reads: rows 4 hi + jr (+8) (+32 mb + 16 sp), d-block db
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d = 32 * db + 16 * (g & 1) + 4 * jc;
    const int r1 = 4 * hi + jr, r2 = r1 + 8;
    trb1[db] = r1 * D + 8 * ((d >> 3) ^ swz<D>(r1)) + 4 * ((d >> 2) & 1);
    trb2[db] = r2 * D + 8 * ((d >> 3) ^ swz<D>(r2)) + 4 * ((d >> 2) & 1);
  }
  // number of queries (from the key itself on) that see this lane's key
  const unsigned mask_n = mykey < T ? (unsigned)(hi_key - mykey + 1) : 0u;

  // Stored dS^T: resource at this head's chunks; each lane writes its 32 bytes of a chunk at
  // 64 * key + 32 * hi (the chunk layout of dsbuf.h).
  const __amdgpu_buffer_rsrc_t ds_rsrc =
      buf_rsrc(STORE_DS ? reinterpret_cast<char*>(p.ds) + dsb::block_offset(bh, 0, 0, p.nkb, p.nslot)
                        : nullptr);
  const unsigned ds_voff = 64u * l32 + 32u * hi;
  // A unit's dS^T is stored at the start of the next computed unit (the last one after the
  // loop). The wait for a tile's copies at its end is a wait for every vector-memory operation
  // of the wave, stores included (one counter; loads and stores may complete out of order), so
  // stores issued in a tile's last unit would expose their write latency at every tile end;
  // issued a unit later, they have completed by then.
  u32x4 pend0 = {}, pend1 = {};
  int pend_off = -1;   // chunk offset of the pending store, -1: none
  auto store_pending = [&]() __attribute__((always_inline)) {
    if constexpr (STORE_DS) {
      if (pend_off >= 0) {
        __builtin_amdgcn_raw_buffer_store_b128(pend0, ds_rsrc, ds_voff, pend_off, 2);
        __builtin_amdgcn_raw_buffer_store_b128(pend1, ds_rsrc, ds_voff + 16u, pend_off, 2);
      }
    }
  };

  // One query tile: recompute S, P, dP, dS in 32-query halves; accumulate dV and dK.
  // The next tile's copies (into Qn, On, Ln, Dn, if qt + 1 <= qt_hi) are issued a quarter at
  // the start of each unit, whether or not this wave computes the unit.
  auto tile = [&](const lds_t<bf16>* Qs, const lds_t<bf16>* Os, const lds_t<float>* Ls,
                  const lds_t<float>* Dls, int qt, lds_t<bf16>* Qn, lds_t<bf16>* On,
                  lds_t<float>* Ln, lds_t<float>* Dn) {
    const int q0 = qt * BMQ;
    // S operands of a unit (row term, Q rows): read for unit 0 here and for unit mb + 1 during
    // the dK MFMAs of unit mb
    f32x4 l2v[4];
    bf16x8 aq[NKS];
    auto read_s_ops = [&](int mb) __attribute__((always_inline)) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        l2v[a] = *reinterpret_cast<const lds_t<f32x4>*>(Ls + mb * 32 + 8 * a + 4 * hi);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        aq[ks] = *reinterpret_cast<const lds_t<bf16x8>*>(Qs + mb * 32 * D + rowb[ks]);
    };
    read_s_ops(0);
#pragma unroll
    for (int mb = 0; mb < BMQ / 32; ++mb) {
      if (qt + 1 <= qt_hi)
        load_qtile<D, BMQ / 32>(p, qbase, obase, l2base, dlbase, Qn, On, Ln, Dn, qt + 1, wave,
                                lane, mb);
      const int qm = q0 + 32 * mb;
      const bool skip = (qm + 31 < kw) || (qm > whi1) || (kw >= T);
      if (skip) {
        if (mb + 1 < BMQ / 32) read_s_ops(mb + 1);
        continue;
      }
      const bool need_mask = (qm < kw + 31) || (qm + 31 > whi0) || (qm + 32 > T) ||
                             (kw + 32 > T);
      store_pending();
      // The LDS operands of each phase are requested one phase ahead, so the reads overlap one
      // another and the MFMAs of the previous phase: the S operands (row term, Q) during the
      // previous unit's dK MFMAs, the dP operands (row term, dO) between the S MFMAs, the dV
      // operands during the dP MFMAs, the dK operands during the dV MFMAs. LDS reads complete
      // in order, so each MFMA waits only for its own operand.
      // S' = -lse2 + c Q K^T and dP' = -delta + dO V^T (lane = key, 16 queries per lane): the
      // accumulators start from the negated row terms of their 16 queries.
      f32x4 dlv[4];
      bf16x8 ao[NKS];
      sched_fence();
      f32x16 s = __builtin_shufflevector(__builtin_shufflevector(l2v[0], l2v[1], 0, 1, 2, 3, 4, 5, 6, 7),
                                         __builtin_shufflevector(l2v[2], l2v[3], 0, 1, 2, 3, 4, 5, 6, 7),
                                         0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) s = mfma32(aq[ks], kreg[ks], s);
#pragma unroll
      for (int a = 0; a < 4; ++a)
        dlv[a] = *reinterpret_cast<const lds_t<f32x4>*>(Dls + mb * 32 + 8 * a + 4 * hi);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        ao[ks] = *reinterpret_cast<const lds_t<bf16x8>*>(Os + mb * 32 * D + rowb[ks]);
      mfma_ds_interleave<NKS>();
      // The MFMA builtins carry no order: without this use of S here, instruction selection
      // may place the last S MFMA behind the dP chain, and the exp2 of S then waits for dP.
      // At D = 128 (one wave per SIMD, more than 256 registers) every MFMA accumulates in
      // AGPRs anyway. At D = 64 (two waves per SIMD) a use in AGPRs would make the compiler put
      // every accumulator there; in VGPRs, the S and dP results feed the exp2 and dS
      // arithmetic with no AGPR reads (about 60 fewer vector instructions per 32-query unit,
      // dK/dV 46.5 -> 44.3 us on the GPT-2 layer).
      if constexpr (D == 128) asm volatile("" : "+a"(s));
      else asm volatile("" : "+v"(s));
      sched_fence();
      f32x16 dp = __builtin_shufflevector(__builtin_shufflevector(dlv[0], dlv[1], 0, 1, 2, 3, 4, 5, 6, 7),
                                          __builtin_shufflevector(dlv[2], dlv[3], 0, 1, 2, 3, 4, 5, 6, 7),
                                          0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) dp = mfma32(ao[ks], vreg[ks], dp);
      // B operands of dV += P^T dO by transposing reads of the row-major dO tile
      bf16x8 bo[NDB][2];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          const int ro = (mb * 32 + sp * 16) * D;
          bo[db][sp] = __builtin_shufflevector(ds_read_tr16(Os + ro + trb1[db]),
                                               ds_read_tr16(Os + ro + trb2[db]),
                                               0, 1, 2, 3, 4, 5, 6, 7);
        }
      sched_fence();
      float pv[16];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          pv[4 * a + r] = __builtin_amdgcn_exp2f(s[4 * a + r]);
      if (need_mask) {
        branch_keep();
        // query qm + 8a + 4hi + r is visible to key `mykey` iff (q - mykey) in [0, mask_n)
        const int base = qm + 4 * hi - mykey;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = 8 * (i >> 2) + (i & 3);
          pv[i] = ((unsigned)(base + t) < mask_n) ? pv[i] : 0.f;
        }
      }
      bf16x8 pb[2];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const bf16x2 p01 = __builtin_convertvector((f32x2){pv[4 * a], pv[4 * a + 1]}, bf16x2);
        const bf16x2 p23 = __builtin_convertvector((f32x2){pv[4 * a + 2], pv[4 * a + 3]}, bf16x2);
        const int e0 = 4 * (a & 1);
        pb[a >> 1][e0] = p01[0]; pb[a >> 1][e0 + 1] = p01[1];
        pb[a >> 1][e0 + 2] = p23[0]; pb[a >> 1][e0 + 3] = p23[1];
      }
      sched_fence();
      // dV += P^T dO, with the Q^T reads for dK and the dS arithmetic issued alongside
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) dv[db] = mfma32(pb[sp], bo[db][sp], dv[db]);
      bf16x8 bq[NDB][2];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          const int ro = (mb * 32 + sp * 16) * D;
          bq[db][sp] = __builtin_shufflevector(ds_read_tr16(Qs + ro + trb1[db]),
                                               ds_read_tr16(Qs + ro + trb2[db]),
                                               0, 1, 2, 3, 4, 5, 6, 7);
        }
      bf16x8 sbf[2];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float dsv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) dsv[r] = pv[4 * a + r] * dp[4 * a + r];
        const bf16x2 d01 = __builtin_convertvector((f32x2){dsv[0], dsv[1]}, bf16x2);
        const bf16x2 d23 = __builtin_convertvector((f32x2){dsv[2], dsv[3]}, bf16x2);
        const int e0 = 4 * (a & 1);
        sbf[a >> 1][e0] = d01[0]; sbf[a >> 1][e0 + 1] = d01[1];
        sbf[a >> 1][e0 + 2] = d23[0]; sbf[a >> 1][e0 + 3] = d23[1];
      }
      if constexpr (STORE_DS) {
        pend0 = __builtin_bit_cast(u32x4, sbf[0]);
        pend1 = __builtin_bit_cast(u32x4, sbf[1]);
        pend_off = (int)(dsb::block_offset(0, kbk, qt - kbk, p.nkb, p.nslot) +
                         (size_t)((wave * 4 + mb) * dsb::CHUNK_BYTES));
      }
      sched_fence();
      // dK += dS^T Q, with the next unit's S operands read between the MFMAs
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) dk[db] = mfma32(sbf[sp], bq[db][sp], dk[db]);
      if (mb + 1 < BMQ / 32) {
        read_s_ops(mb + 1);
        mfma_ds_interleave<2 * NDB>();
      }
      sched_fence();
    }
  };

  load_qtile<D>(p, qbase, obase, l2base, dlbase, Q0, O0, L0, D0, qt_lo, wave, lane);
  wait_vmem();
  __syncthreads();
  for (int qt = qt_lo; qt <= qt_hi; qt += 2) {
    tile(Q0, O0, L0, D0, qt, Q1, O1, L1, D1);
    if (qt + 1 > qt_hi) break;
    wait_vmem();
    lds_sync();
    tile(Q1, O1, L1, D1, qt + 1, Q0, O0, L0, D0);
    if (qt + 2 > qt_hi) break;
    wait_vmem();
    lds_sync();
  }
  store_pending();

  // Epilogue: lane owns d = 32 db + l32 of keys kw + 8(i/4) + 4 hi + (i%4).
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = kw + 8 * (i >> 2) + 4 * hi + (i & 3);
    if (key >= T) continue;
    const size_t row = head0 + (size_t)key * rs;
    float gsum = 0.f, gkey = 0.f;
    const bf16* er = nullptr;
    if constexpr (GATE) {
      gkey = p.gate[(size_t)(b * T + key) * H + h];
      er = ve_row<D>(p.ve, p.ve_ids, p.ve_rows, b, T, H, h, key);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const size_t off = row + db * 32 + l32;
      // written with the nontemporal hint: the dS chunks this kernel stored stay cached for the
      // dQ kernel that reads them next (dQ ~2 % faster on the d24 sweep)
      __builtin_nontemporal_store(__builtin_bit_cast(unsigned short, (bf16)(dk[db][i] * p.scale)),
                                  reinterpret_cast<unsigned short*>(p.dk + off));
      __builtin_nontemporal_store(__builtin_bit_cast(unsigned short, (bf16)dv[db][i]),
                                  reinterpret_cast<unsigned short*>(p.dv + off));
      if constexpr (GATE) {
        if (p.ve_ids) {
          // table mode: tokens sharing an id add into one row (float atomics)
          if (er) atomicAdd(p.dve_tab + (er - p.ve) + db * 32 + l32, gkey * dv[db][i]);
        } else {
          p.dve[off] = (bf16)(gkey * dv[db][i]);
        }
        if (er) gsum = fmaf(dv[db][i], (float)er[db * 32 + l32], gsum);
      }
    }
    if constexpr (GATE) {
#pragma unroll
      for (int m = 1; m < 32; m <<= 1) gsum += xor_shfl(gsum, m);
      if (l32 == 0) p.dgate[(size_t)(b * T + key) * H + h] = gsum;
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
    const float* __restrict__ ndelta, const float* __restrict__ dO, const int* __restrict__ bounds,
    const int* __restrict__ ve_ids, int ve_rows,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dve,
    float* __restrict__ dgate, int T, int H, int W, float scale) {
  constexpr int PER = D / 64;
  const int j = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H, lane = threadIdx.x;
  const size_t krow = ((size_t)b * T + j) * H + h;
  const float g = gate ? gate[krow] : 0.f;
  const float* er = gate ? ve_row<D>(ve, ve_ids, ve_rows, b, T, H, h, j) : nullptr;
  float kv[PER], vv[PER], ak[PER], av[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    kv[e] = k[krow * D + lane + 64 * e];
    vv[e] = v[krow * D + lane + 64 * e];
    if (er) vv[e] = fmaf(g, er[lane + 64 * e], vv[e]);
    ak[e] = 0.f; av[e] = 0.f;
  }
  const int i1 = min(min(T - 1, j + W - 1), bounds ? bounds[2 * ((size_t)b * T + j) + 1] - 1 : T - 1);
  for (int i = j; i <= i1; ++i) {
    const size_t qrow = ((size_t)b * T + i) * H + h;
    const float s = wave_dot<D>(kv, q + qrow * D, lane) * scale;
    const float pij = expf(s - lse[(size_t)bh * T + i]);
    const float dp = wave_dot<D>(vv, dO + qrow * D, lane);
    const float ds = pij * (dp + ndelta[(size_t)bh * T + i]);
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
      if (!ve_ids) dve[krow * D + lane + 64 * e] = g * av[e];
      else if (er) atomicAdd(dve + (er - ve) + lane + 64 * e, g * av[e]);
      if (er) gs = fmaf(av[e], er[lane + 64 * e], gs);
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
    const float* __restrict__ ndelta, const float* __restrict__ dO, const int* __restrict__ bounds,
    const int* __restrict__ ve_ids, int ve_rows, float* __restrict__ dq, int T, int H, int W,
    float scale) {
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
  const float L = lse[(size_t)bh * T + i], ndl = ndelta[(size_t)bh * T + i];
  const int j0 = max(max(0, i - W + 1), bounds ? bounds[2 * ((size_t)b * T + i)] : 0);
  for (int j = j0; j <= i; ++j) {
    const size_t krow = ((size_t)b * T + j) * H + h;
    const float s = wave_dot<D>(qv, k + krow * D, lane) * scale;
    const float pij = expf(s - L);
    float dp = 0.f;
    const float g = gate ? gate[krow] : 0.f;
    const float* er = gate ? ve_row<D>(ve, ve_ids, ve_rows, b, T, H, h, j) : nullptr;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      float vv = v[krow * D + lane + 64 * e];
      if (er) vv = fmaf(g, er[lane + 64 * e], vv);
      dp = fmaf(ov[e], vv, dp);
    }
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) dp += xor_shfl(dp, m);
    const float ds = pij * (dp + ndl);
#pragma unroll
    for (int e = 0; e < PER; ++e) aq[e] = fmaf(ds, k[krow * D + lane + 64 * e], aq[e]);
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) dq[qrow * D + lane + 64 * e] = aq[e] * scale;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace: -delta (B,H,T) | -lse*log2(e) (B,H,T), float32. Each block is 256-byte aligned and followed
// by 512 bytes of slack, so the 16-byte row-term loads of a query tile that runs past the
// sequence end stay inside the allocation; the kernels that write the row terms also write
// zeros to the first 128 slack rows (the only ones such a tile reads).
static size_t rowterm_block(int B, int T, int H) {
  return align256((size_t)B * H * T * sizeof(float)) + 512;
}

size_t bwd_workspace_bytes(int B, int T, int H, int D, bool bf16) {
  (void)D;
  (void)bf16;
  return 2 * rowterm_block(B, T, H);
}

template <typename E, int D>
static void launch_pre(const void* o, const void* dO, const float* lse, float* ndelta, float* nlse2,
                       int B, int T, int H, hipStream_t s) {
  // the positions of each head, then (last head only) the zeroed slack
  const dim3 grid((T + kPreRows - 1) / kPreRows + kRowTermSlackRows / kPreRows, B * H);
  hipLaunchKernelGGL((bwd_pre_kernel<E, D>), grid, dim3(256), 0, s, (const E*)o, (const E*)dO,
                     lse, ndelta, nlse2, T, H, B * H);
}

template <int D, bool GATE, bool STORE_DS>
static hipError_t launch_dkdv_bf16_t(const AttnShape& a, const bwdk::Params& p, hipStream_t s) {
  const unsigned blocks = (unsigned)p.nkb * a.B * a.H;
  if (a.bounds)
    hipLaunchKernelGGL((bwdk::dkdv_bf16_kernel<D, GATE, true, STORE_DS>), dim3(blocks), dim3(256),
                       0, s, p);
  else
    hipLaunchKernelGGL((bwdk::dkdv_bf16_kernel<D, GATE, false, STORE_DS>), dim3(blocks),
                       dim3(256), 0, s, p);
  return hipGetLastError();
}

namespace {
struct WsView {
  float* ndelta;
  float* nlse2;
};
WsView ws_view(void* ws, int B, int T, int H) {
  WsView w;
  char* base = reinterpret_cast<char*>(ws);
  w.ndelta = reinterpret_cast<float*>(base);
  w.nlse2 = reinterpret_cast<float*>(base + rowterm_block(B, T, H));
  return w;
}
}  // namespace

hipError_t launch_bwd_pre(const AttnShape& a, const void* o, const void* dO, const float* lse,
                          void* ws, bool is_bf16, hipStream_t s) {
  const WsView w = ws_view(ws, a.B, a.T, a.H);
  if (is_bf16) {
    if (a.D == 64) launch_pre<swa::bf16, 64>(o, dO, lse, w.ndelta, w.nlse2, a.B, a.T, a.H, s);
    else launch_pre<swa::bf16, 128>(o, dO, lse, w.ndelta, w.nlse2, a.B, a.T, a.H, s);
  } else {
    if (a.D == 64) launch_pre<float, 64>(o, dO, lse, w.ndelta, w.nlse2, a.B, a.T, a.H, s);
    else launch_pre<float, 128>(o, dO, lse, w.ndelta, w.nlse2, a.B, a.T, a.H, s);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const AttnShape& a, const void* q, const void* k, const void* v,
                           const void* ve, const float* gate, const float* lse, const void* dO,
                           void* dk, void* dv, void* dve, float* dgate, void* ws, bool is_bf16,
                           hipStream_t s, void* ds) {
  const int B = a.B, T = a.T, H = a.H, D = a.D;
  const WsView w = ws_view(ws, B, T, H);
  if (is_bf16) {
    bwdk::Params p;
    p.q = (const bf16*)q; p.k = (const bf16*)k; p.v = (const bf16*)v; p.ve = (const bf16*)ve;
    p.gate = gate; p.nlse2 = w.nlse2; p.ndelta = w.ndelta; p.dO = (const bf16*)dO;
    p.bounds = a.bounds;
    p.dk = (bf16*)dk; p.dv = (bf16*)dv; p.dve = (bf16*)dve; p.dgate = dgate;
    p.ve_ids = a.ve_ids; p.ve_rows = a.ve_rows; p.dve_tab = (float*)dve;
    p.B = B; p.T = T; p.H = H; p.window = a.window;
    p.nkb = (T + bwdk::BNK - 1) / bwdk::BNK;
    p.lpt = lpt_order(a) ? 1 : 0;
    p.c = a.scale * kLog2e;
    p.scale = a.scale;
    p.ds = (bf16*)ds;
    p.nslot = dsb::nslot(T, a.window);
    const bool g = gate != nullptr;
    if (ds) {
      if (D == 64)
        return g ? launch_dkdv_bf16_t<64, true, true>(a, p, s) : launch_dkdv_bf16_t<64, false, true>(a, p, s);
      return g ? launch_dkdv_bf16_t<128, true, true>(a, p, s) : launch_dkdv_bf16_t<128, false, true>(a, p, s);
    }
    if (D == 64)
      return g ? launch_dkdv_bf16_t<64, true, false>(a, p, s) : launch_dkdv_bf16_t<64, false, false>(a, p, s);
    return g ? launch_dkdv_bf16_t<128, true, false>(a, p, s) : launch_dkdv_bf16_t<128, false, false>(a, p, s);
  }
  dim3 grid(T, B * H);
  if (D == 64)
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<64>, grid, dim3(64), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)ve, gate, lse, w.ndelta, (const float*)dO,
                       a.bounds, a.ve_ids, a.ve_rows, (float*)dk, (float*)dv, (float*)dve, dgate, T, H,
                       a.window, a.scale);
  else
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<128>, grid, dim3(64), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)ve, gate, lse, w.ndelta, (const float*)dO,
                       a.bounds, a.ve_ids, a.ve_rows, (float*)dk, (float*)dv, (float*)dve, dgate, T, H,
                       a.window, a.scale);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const AttnShape& a, const void* q, const void* k, const void* v,
                         const void* ve, const float* gate, const float* lse, const void* dO,
                         void* dq, void* ws, bool is_bf16, hipStream_t s) {
  const int B = a.B, T = a.T, H = a.H, D = a.D;
  const WsView w = ws_view(ws, B, T, H);
  if (is_bf16)
    return launch_dq_bf16(a, q, k, v, ve, gate, dO, w.nlse2, w.ndelta, nullptr, nullptr, dq, s);
  dim3 grid(T, B * H);
  if (D == 64)
    hipLaunchKernelGGL(bwd_dq_f32_kernel<64>, grid, dim3(64), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)ve, gate, lse, w.ndelta, (const float*)dO,
                       a.bounds, a.ve_ids, a.ve_rows, (float*)dq, T, H, a.window, a.scale);
  else
    hipLaunchKernelGGL(bwd_dq_f32_kernel<128>, grid, dim3(64), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (const float*)ve, gate, lse, w.ndelta, (const float*)dO,
                       a.bounds, a.ve_ids, a.ve_rows, (float*)dq, T, H, a.window, a.scale);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_rowterms(const AttnShape& a, const void* q, const void* k,
                                  const void* v, const void* ve, const float* gate,
                                  const void* o, const float* lse, const void* dO, void* dq,
                                  void* ws, bool is_bf16, hipStream_t s) {
  if (!is_bf16) {
    const hipError_t e = launch_bwd_pre(a, o, dO, lse, ws, false, s);
    return e != hipSuccess ? e : launch_bwd_dq(a, q, k, v, ve, gate, lse, dO, dq, ws, false, s);
  }
  const WsView w = ws_view(ws, a.B, a.T, a.H);
  return launch_dq_bf16(a, q, k, v, ve, gate, dO, w.nlse2, w.ndelta, o, lse, dq, s);
}

}  // namespace swa

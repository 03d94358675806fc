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
// delta_i = sum_d dO[i, d] * O[i, d] and lse2_i = lse_i * log2(e); also zeroes the float32
// dQ accumulator row.
// ------------------------------------------------------------------------------------------
template <typename E, int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const E* __restrict__ o,
                                                      const E* __restrict__ dO,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ lse2,
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
    const size_t r = ((size_t)b * H + h) * T + t;
    delta[r] = acc;
    lse2[r] = lse[r] * kLog2e;   // log2-domain row terms for the exp2 in the main kernel
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
  static constexpr int CH = D / 8;            // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;         // rows per 1 KiB wave load
  static constexpr int QTILE = BMQ * D;       // elements of a Q or dO tile
  static constexpr int NIQ = BMQ / RPI / NW;  // wave loads per tile per wave
  static constexpr int NIK = BNK / RPI / NW;  // wave loads of the K block per wave
  static constexpr int ST = BNK * BMQ;        // dS^T tile elements ([key][query], 128-byte rows)
};

struct Params {
  const bf16* q; const bf16* k; const bf16* v; const bf16* ve; const float* gate;
  const float* lse2; const float* delta; const bf16* dO;
  float* dq_acc; bf16* dk; bf16* dv; bf16* dve; float* dgate;
  int B, T, H, window, nkb;
  float c;       // scale * log2(e)
  float scale;
};

// Asynchronous loads of query tile qt (Q, dO rows and the lse2 / delta row terms) into LDS.
template <int D>
__device__ __forceinline__ void load_qtile(const Params& p, const bf16* qbase, const bf16* obase,
                                           const float* l2base, const float* dlbase,
                                           lds_t<bf16>* Qs, lds_t<bf16>* Os, lds_t<float>* Ls,
                                           lds_t<float>* Dls, int qt, int wave, int lane) {
  using C = Cfg<D>;
  const size_t rs = (size_t)p.H * D;
#pragma unroll
  for (int i = 0; i < C::NIQ; ++i) {
    const int I = wave * C::NIQ + i;
    const int r = I * C::RPI + lane / C::CH;
    const int c = (lane % C::CH) ^ swz<D>(r);
    const size_t goff = (size_t)min(qt * BMQ + r, p.T - 1) * rs + 8 * c;
    g2lds16(qbase + goff, Qs + I * C::RPI * D);
    g2lds16(obase + goff, Os + I * C::RPI * D);
  }
  if (lane < BMQ / 4) {
    // a tile that runs past the sequence end reads into the next head's row or the workspace
    // slack (see bwd_workspace_bytes); those queries are masked
    if (wave == 0) g2lds16(l2base + qt * BMQ + 4 * lane, (lds_t<bf16>*)Ls);
    if (wave == 1) g2lds16(dlbase + qt * BMQ + 4 * lane, (lds_t<bf16>*)Dls);
  }
}

template <int D, bool GATE>
__global__ void __launch_bounds__(256, 1) bwd_bf16_kernel(Params p) {
  using C = Cfg<D>;
  constexpr int NDB = D / 32, NKS = D / 16;
  __shared__ __attribute__((aligned(16))) bf16 ks_[BNK * D], vs_[BNK * D], q0_[C::QTILE],
      q1_[C::QTILE], o0_[C::QTILE], o1_[C::QTILE], st_[C::ST];
  __shared__ __attribute__((aligned(16))) float l0_[BMQ], l1_[BMQ], d0_[BMQ], d1_[BMQ];
  lds_t<bf16>* Ks = (lds_t<bf16>*)ks_;
  lds_t<bf16>* Vs = (lds_t<bf16>*)vs_;
  lds_t<bf16>* Q0 = (lds_t<bf16>*)q0_;
  lds_t<bf16>* Q1 = (lds_t<bf16>*)q1_;
  lds_t<bf16>* O0 = (lds_t<bf16>*)o0_;
  lds_t<bf16>* O1 = (lds_t<bf16>*)o1_;
  lds_t<bf16>* ST = (lds_t<bf16>*)st_;
  lds_t<float>* L0 = (lds_t<float>*)l0_;
  lds_t<float>* L1 = (lds_t<float>*)l1_;
  lds_t<float>* D0 = (lds_t<float>*)d0_;
  lds_t<float>* D1 = (lds_t<float>*)d1_;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int g = lane >> 4, j = lane & 15;
  const int T = p.T, H = p.H, W = p.window;

  const int nblk = gridDim.x;
  int L = blockIdx.x;
  if ((nblk & 7) == 0) L = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int bh = L / p.nkb;
  const int kbk = L - bh * p.nkb;
  const int b = bh / H, h = bh - b * H;
  const size_t head0 = ((size_t)b * T * H + h) * D;
  const size_t rs = (size_t)H * D;
  const int kb0 = kbk * BNK;
  const int kw = kb0 + 32 * wave;
  const int mykey = kw + l32;
  const bf16* qbase = p.q + head0;
  const bf16* obase = p.dO + head0;
  const float* l2base = p.lse2 + (size_t)bh * T;
  const float* dlbase = p.delta + (size_t)bh * T;

  // K and v_eff rows of the workgroup's key block into LDS (row-major, swizzled). K is the B
  // operand of S = Q K^T (128-bit row reads) and of dQ = dS K (transposing reads); v_eff is the
  // B operand of dP = dO V^T.
#pragma unroll
  for (int i = 0; i < C::NIK; ++i) {
    const int I = wave * C::NIK + i;
    const int r = I * C::RPI + lane / C::CH;
    const int c = (lane % C::CH) ^ swz<D>(r);
    const size_t goff = head0 + (size_t)min(kb0 + r, T - 1) * rs + 8 * c;
    g2lds16(p.k + goff, Ks + I * C::RPI * D);
    if constexpr (!GATE) g2lds16(p.v + goff, Vs + I * C::RPI * D);
  }
  if constexpr (GATE) {
    for (int id = tid; id < BNK * C::CH; id += 256) {
      const int r = id / C::CH, pos = id % C::CH;
      const int c = pos ^ swz<D>(r);
      const int row = min(kb0 + r, T - 1);
      const size_t goff = head0 + (size_t)row * rs + 8 * c;
      const uint4 a = *reinterpret_cast<const uint4*>(p.v + goff);
      const uint4 e = *reinterpret_cast<const uint4*>(p.ve + goff);
      const float gk = p.gate[(size_t)(b * T + row) * H + h];
      u32x4 o;
      o.x = pack_bf2(fmaf(gk, bf_lo(e.x), bf_lo(a.x)), fmaf(gk, bf_hi(e.x), bf_hi(a.x)));
      o.y = pack_bf2(fmaf(gk, bf_lo(e.y), bf_lo(a.y)), fmaf(gk, bf_hi(e.y), bf_hi(a.y)));
      o.z = pack_bf2(fmaf(gk, bf_lo(e.z), bf_lo(a.z)), fmaf(gk, bf_hi(e.z), bf_hi(a.z)));
      o.w = pack_bf2(fmaf(gk, bf_lo(e.w), bf_lo(a.w)), fmaf(gk, bf_hi(e.w), bf_hi(a.w)));
      *reinterpret_cast<lds_t<u32x4>*>(Vs + r * D + 8 * pos) = o;
    }
  }

  f32x16 dv[NDB], dk[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) { dv[i] = (f32x16){}; dk[i] = (f32x16){}; }

  const int qt_lo = kb0 / BMQ;
  const int qt_hi = min(T - 1, kb0 + BNK - 1 + W - 1) / BMQ;

  // Lane-constant LDS element offsets. Every swizzled address below is one of these plus a
  // compile-time row offset, so the LDS loads use immediate offsets off a few registers.
  const int jr = j >> 2, jc = j & 3;
  // (a) 128-bit row reads, row (32 mb + l32) of a [rows][D] tile, chunk 2 ks + hi
  int rowb[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) rowb[ks] = l32 * D + 8 * ((2 * ks + hi) ^ swz<D>(l32));
  const int kvrow = 32 * wave * D;  // this wave's key rows in the K / V blocks
  // (b) transposing reads of a [rows][D] tile: rows 4 hi + jr (+8) (+ 32 mb + 16 sp), d-block db
  int trb1[NDB], trb2[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d = 32 * db + 16 * (g & 1) + 4 * jc;
    const int r1 = 4 * hi + jr, r2 = r1 + 8;
    trb1[db] = r1 * D + 8 * ((d >> 3) ^ swz<D>(r1)) + 4 * ((d >> 2) & 1);
    trb2[db] = r2 * D + 8 * ((d >> 3) ^ swz<D>(r2)) + 4 * ((d >> 2) & 1);
  }
  // (c) dQ: transposing reads of dS^T ([key][query], 128-byte rows) and of the K block
  constexpr int NMB = (D == 128) ? 2 : 1;
  const int dq_db = (D == 128) ? wave : (wave & 1);
  int stb1[NMB], stb2[NMB];
#pragma unroll
  for (int jm = 0; jm < NMB; ++jm) {
    const int mb = (D == 128) ? jm : (wave >> 1);
    const int qc = 32 * mb + 16 * (g & 1) + 4 * jc;
    const int k1 = 8 * hi + jr, k2 = k1 + 4;
    stb1[jm] = k1 * BMQ + 8 * ((qc >> 3) ^ swz<64>(k1)) + 4 * ((qc >> 2) & 1);
    stb2[jm] = k2 * BMQ + 8 * ((qc >> 3) ^ swz<64>(k2)) + 4 * ((qc >> 2) & 1);
  }
  int kqb1, kqb2;
  {
    const int dc = 32 * dq_db + 16 * (g & 1) + 4 * jc;
    const int k1 = 8 * hi + jr, k2 = k1 + 4;
    kqb1 = k1 * D + 8 * ((dc >> 3) ^ swz<D>(k1)) + 4 * ((dc >> 2) & 1);
    kqb2 = k2 * D + 8 * ((dc >> 3) ^ swz<D>(k2)) + 4 * ((dc >> 2) & 1);
  }
  // (d) this lane's dS^T row and its 8-byte slot
  const int kl = 32 * wave + l32;
  const int stw = kl * BMQ + 4 * hi;
  const int stsw = swz<64>(kl);
  // dQ accumulator: this lane's column for query row (q0 + 4 hi) of the tile
  float* const dqcol = p.dq_acc + head0 + (size_t)(4 * hi) * rs + dq_db * 32 + l32;

  // number of queries (from the key itself on) that see this lane's key: min(W, T - key)
  const unsigned mask_n = mykey < T ? (unsigned)min(W, T - mykey) : 0u;

  // One query tile: recompute S, P, dP, dS; accumulate dV, dK; dS^T to LDS; dQ slice -> atomics.
  auto tile = [&](const lds_t<bf16>* Qs, const lds_t<bf16>* Os, const lds_t<float>* Ls,
                  const lds_t<float>* Dls, int qt) {
    const int q0 = qt * BMQ;
    const bool skip = (q0 + BMQ - 1 < kw) || (q0 > kw + 31 + W - 1) || (kw >= T);
    if (!skip) {
      const bool need_mask = (q0 < kw + 31) || (q0 + BMQ - 1 > kw + W - 1) || (q0 + BMQ > T) ||
                             (kw + 32 > T);
      // the two 32-query halves of the tile one after the other (halves the live registers)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int off = mb * 32 * D + rowb[ks];
          const bf16x8 aq = *reinterpret_cast<const lds_t<bf16x8>*>(Qs + off);
          const bf16x8 bk = *reinterpret_cast<const lds_t<bf16x8>*>(Ks + kvrow + rowb[ks]);
          const bf16x8 ao = *reinterpret_cast<const lds_t<bf16x8>*>(Os + off);
          const bf16x8 bv = *reinterpret_cast<const lds_t<bf16x8>*>(Vs + kvrow + rowb[ks]);
          s = mfma32(aq, bk, s);
          dp = mfma32(ao, bv, dp);
        }
        sched_fence();
        float pv[16];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 l2 = *reinterpret_cast<const lds_t<f32x4>*>(Ls + mb * 32 + 8 * a + 4 * hi);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            pv[4 * a + r] = __builtin_amdgcn_exp2f(fmaf(s[4 * a + r], p.c, -l2[r]));
        }
        if (need_mask) {
          branch_keep();
          // query q0 + mb*32 + 8a + 4hi + r is visible to key `mykey` iff (q - mykey) in [0, n)
          const int base = q0 + mb * 32 + 4 * hi - mykey;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int t = 8 * (i >> 2) + (i & 3);
            pv[i] = ((unsigned)(base + t) < mask_n) ? pv[i] : 0.f;
          }
        }
        bf16x8 pb[2], sbf[2];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int ql = mb * 32 + 8 * a + 4 * hi;  // first of 4 consecutive queries
          const f32x4 dl = *reinterpret_cast<const lds_t<f32x4>*>(Dls + ql);
          float dsv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) dsv[r] = pv[4 * a + r] * (dp[4 * a + r] - dl[r]);
          const bf16x2 p01 = __builtin_convertvector((f32x2){pv[4 * a], pv[4 * a + 1]}, bf16x2);
          const bf16x2 p23 = __builtin_convertvector((f32x2){pv[4 * a + 2], pv[4 * a + 3]}, bf16x2);
          const bf16x2 d01 = __builtin_convertvector((f32x2){dsv[0], dsv[1]}, bf16x2);
          const bf16x2 d23 = __builtin_convertvector((f32x2){dsv[2], dsv[3]}, bf16x2);
          const int e0 = 4 * (a & 1);
          pb[a >> 1][e0] = p01[0]; pb[a >> 1][e0 + 1] = p01[1];
          pb[a >> 1][e0 + 2] = p23[0]; pb[a >> 1][e0 + 3] = p23[1];
          sbf[a >> 1][e0] = d01[0]; sbf[a >> 1][e0 + 1] = d01[1];
          sbf[a >> 1][e0 + 2] = d23[0]; sbf[a >> 1][e0 + 3] = d23[1];
          // dS^T row kl, queries ql..ql+3 (8 bytes); chunk (4 mb + a) of the row
          const unsigned long long w4 = (unsigned long long)__builtin_bit_cast(unsigned, d01) |
                                        ((unsigned long long)__builtin_bit_cast(unsigned, d23) << 32);
          ds_store_b64(ST + stw + 8 * ((4 * mb + a) ^ stsw), w4);
        }
        // dV += P^T dO and dK += dS^T Q; B operands by transposing reads of the row-major tiles.
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int sp = 0; sp < 2; ++sp) {
            const int ro = (mb * 32 + sp * 16) * D;
            const bf16x8 bo = __builtin_shufflevector(ds_read_tr16(Os + ro + trb1[db]),
                                                      ds_read_tr16(Os + ro + trb2[db]),
                                                      0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 bq = __builtin_shufflevector(ds_read_tr16(Qs + ro + trb1[db]),
                                                      ds_read_tr16(Qs + ro + trb2[db]),
                                                      0, 1, 2, 3, 4, 5, 6, 7);
            dv[db] = mfma32(pb[sp], bo, dv[db]);
            dk[db] = mfma32(sbf[sp], bq, dk[db]);
          }
          sched_fence();
        }
      }
    } else {
      // this wave's keys see none of the tile: zero its dS^T rows
      for (int r = lane; r < 32 * (BMQ / 4); r += 64)
        ds_store_b64(ST + (32 * wave + (r >> 4)) * BMQ + 4 * (r & 15), 0ull);
    }
    lds_sync();
    // dQ slice: D=128 -> wave owns d-block `wave` for both 32-query halves; D=64 -> d-block
    // (wave & 1) for query half (wave >> 1). A = dS (from dS^T), B = K, both transposing reads.
#pragma unroll
    for (int jm = 0; jm < NMB; ++jm) {
      const int mb = (D == 128) ? jm : (wave >> 1);
      f32x16 acc = (f32x16){};
#pragma unroll
      for (int ks = 0; ks < BNK / 16; ++ks) {
        const bf16x8 a = __builtin_shufflevector(ds_read_tr16(ST + 16 * ks * BMQ + stb1[jm]),
                                                 ds_read_tr16(ST + 16 * ks * BMQ + stb2[jm]),
                                                 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 bk = __builtin_shufflevector(ds_read_tr16(Ks + 16 * ks * D + kqb1),
                                                  ds_read_tr16(Ks + 16 * ks * D + kqb2),
                                                  0, 1, 2, 3, 4, 5, 6, 7);
        acc = mfma32(a, bk, acc);
        if (ks & 1) sched_fence();
      }
      // lane owns d = 32 dq_db + l32 of queries q0 + 32 mb + 8(i/4) + 4 hi + (i%4)
      // Every lane issues all 16 atomics (a fixed count per tile, which the wait at the top of
      // the next tile relies on); rows past the sequence end carry dS = 0, so they add exactly
      // zero, to row T-1.
      float* const col = dqcol + (size_t)(q0 + 32 * mb) * rs;
      const int rlast = T - 1 - (q0 + 32 * mb + 4 * hi);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qr = min(8 * (i >> 2) + (i & 3), rlast);
        unsafeAtomicAdd(col + (size_t)qr * rs, acc[i] * p.scale);
      }
    }
  };

  // Tile loop. Each tile issues NMB*16 dQ atomics after the prefetch of the next tile, and
  // vector-memory counts retire in issue order, so waiting for vmcnt <= NMB*16 at the top of
  // the next tile waits for that prefetch without waiting for the atomics.
  load_qtile<D>(p, qbase, obase, l2base, dlbase, Q0, O0, L0, D0, qt_lo, wave, lane);
  wait_vmem();
  __syncthreads();
  for (int qt = qt_lo; qt <= qt_hi; qt += 2) {
    if (qt + 1 <= qt_hi) load_qtile<D>(p, qbase, obase, l2base, dlbase, Q1, O1, L1, D1, qt + 1, wave, lane);
    tile(Q0, O0, L0, D0, qt);
    if (qt + 1 > qt_hi) break;
    wait_vmem_but<NMB * 16>();
    lds_sync();
    if (qt + 2 <= qt_hi) load_qtile<D>(p, qbase, obase, l2base, dlbase, Q0, O0, L0, D0, qt + 2, wave, lane);
    tile(Q1, O1, L1, D1, qt + 1);
    if (qt + 2 > qt_hi) break;
    wait_vmem_but<NMB * 16>();
    lds_sync();
  }

  // Epilogue: lane owns d = 32 db + l32 of keys kw + 8(i/4) + 4 hi + (i%4).
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = kw + 8 * (i >> 2) + 4 * hi + (i & 3);
    if (key >= T) continue;
    const size_t row = head0 + (size_t)key * rs;
    float gsum = 0.f, gkey = 0.f;
    if constexpr (GATE) gkey = p.gate[(size_t)(b * T + key) * H + h];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const size_t off = row + db * 32 + l32;
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

// Workspace: delta (B,H,T) | lse2 (B,H,T) | [bf16 path] dq accumulator (B,T,H,D) float32. Each
// block is 256-byte aligned and followed by 512 bytes of slack, so the 16-byte row-term loads of
// a query tile that runs past the sequence end stay inside the allocation.
static size_t rowterm_block(int B, int T, int H) {
  return align256((size_t)B * H * T * sizeof(float)) + 512;
}

size_t bwd_workspace_bytes(int B, int T, int H, int D, bool bf16) {
  const size_t acc = bf16 ? align256((size_t)B * T * H * D * sizeof(float)) : 0;
  return 2 * rowterm_block(B, T, H) + acc;
}

template <typename E, int D>
static void launch_pre(const void* o, const void* dO, const float* lse, float* delta, float* lse2,
                       float* dq_acc, int B, int T, int H, hipStream_t s) {
  constexpr int TPR = D / (16 / sizeof(E));
  const int rows = B * T * H;
  const int rpb = 256 / TPR;
  hipLaunchKernelGGL((bwd_pre_kernel<E, D>), dim3((rows + rpb - 1) / rpb), dim3(256), 0, s,
                     (const E*)o, (const E*)dO, lse, delta, lse2, dq_acc, rows, T, H);
}

template <int D, bool GATE>
static hipError_t launch_bwd_bf16_t(const AttnShape& a, const bwdk::Params& p, hipStream_t s) {
  const unsigned blocks = (unsigned)p.nkb * a.B * a.H;
  hipLaunchKernelGGL((bwdk::bwd_bf16_kernel<D, GATE>), dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

namespace {
struct WsView {
  float* delta;
  float* lse2;
  float* dq_acc;  // bf16 path only
};
WsView ws_view(void* ws, int B, int T, int H, bool is_bf16) {
  WsView w;
  char* base = reinterpret_cast<char*>(ws);
  const size_t blk = rowterm_block(B, T, H);
  w.delta = reinterpret_cast<float*>(base);
  w.lse2 = reinterpret_cast<float*>(base + blk);
  w.dq_acc = is_bf16 ? reinterpret_cast<float*>(base + 2 * blk) : nullptr;
  return w;
}
}  // namespace

hipError_t launch_bwd_pre(const AttnShape& a, const void* o, const void* dO, const float* lse,
                          void* ws, bool is_bf16, hipStream_t s) {
  const WsView w = ws_view(ws, a.B, a.T, a.H, is_bf16);
  if (is_bf16) {
    if (a.D == 64) launch_pre<swa::bf16, 64>(o, dO, lse, w.delta, w.lse2, w.dq_acc, a.B, a.T, a.H, s);
    else launch_pre<swa::bf16, 128>(o, dO, lse, w.delta, w.lse2, w.dq_acc, a.B, a.T, a.H, s);
  } else {
    if (a.D == 64) launch_pre<float, 64>(o, dO, lse, w.delta, w.lse2, nullptr, a.B, a.T, a.H, s);
    else launch_pre<float, 128>(o, dO, lse, w.delta, w.lse2, nullptr, a.B, a.T, a.H, s);
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
    p.gate = gate; p.lse2 = w.lse2; p.delta = w.delta; p.dO = (const bf16*)dO; p.dq_acc = w.dq_acc;
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

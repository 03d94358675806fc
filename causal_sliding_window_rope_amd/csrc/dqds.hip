// dQ of causal sliding-window attention from the stored dS^T, for gfx950.
//
//   dQ = scale dS K    ("GPT-2 124M 复现" §19: the backward's products of the recomputed
//                       score gradient with the saved inputs)
//
// The key-block-major dK/dV kernel (bwd.hip) has already formed dS^T = P^T (dP^T - delta) in
// bf16 for dK and stored it chunk by chunk (dsbuf.h). This kernel only contracts it with K:
// 2 D FLOP per visible pair, against 6 D for recomputing S, P and dP here, and it streams the
// stored chunks from HBM once.
//
// One workgroup = 4 waves = one 128-query tile of one (b, h); wave w owns queries 32 w .. +31,
// which is unit w of every chunk, so a wave reads only its own chunks. Steps of 64 keys (half a
// key block: key groups 2h, 2h + 1). The wave's two chunks of a step go straight into registers
// (one 16-byte load per lane per half chunk), PF steps ahead of the one computed, and its share
// of the step's K rows (row-major, 16-byte chunks XOR-swizzled) into registers KPF steps ahead,
// written into one of two LDS buffers at the step (Pipe below). Streaming dS from HBM is what
// bounds this kernel: with two-stage LDS buffering of both it reached about 3.4 TB/s, too few
// bytes in flight per CU; registers hold several steps of dS per wave without taking LDS, or,
// with three workgroups per CU, more waves hold one step each. At its step, a wave writes its
// chunks into a private LDS buffer and reads them back transposed. dQ^T += K^T dS^T on
// v_mfma_f32_32x32x16_bf16: A = K^T by transposing LDS reads of the K rows, B = dS^T by
// transposing reads of the chunk (lane = query, 4 keys per read), both in natural key order.
// Chunks the dK/dV kernel did not compute (outside the window, past the sequence end) are read
// as zeros through an empty buffer range (no memory access) and skipped.
#include "common.h"
#include "dsbuf.h"
#include "internal.h"
#include "rope_row.h"

namespace swa {
namespace dqs {

constexpr int NW = 4;
constexpr int BM = dsb::QUERIES;   // queries per workgroup
constexpr int BN = 64;             // keys per step
// Load pipeline. Without document masking: two workgroups per CU, dS issued PF = 3 and K KPF = 2
// steps ahead. With document masking the workgroups' lengths follow the documents, and three
// workgroups per CU (<= 168 VGPRs: dS and K one step ahead, the epilogue's row loads in two
// batches) measured 15 % faster on the masked d24 layer (193 -> 164 us); without masking the
// same configuration was level on the d24 sweep and slower on the GPT-2 layer.
template <bool DOC> struct Pipe {
  static constexpr int PF = DOC ? 1 : 3;         // dS: steps issued ahead of the one computed
  static constexpr int RING = PF + 1;            // dS register sets
  static constexpr int KPF = DOC ? 1 : 2;        // K: steps issued ahead
  static constexpr int UNROLL = 2 * RING;        // steps per loop trip (a multiple of RING and KPF)
  static constexpr int WG_PER_CU = DOC ? 3 : 2;
  static constexpr int NBATCH = DOC ? 2 : 1;     // batches of the query-prologue epilogue's loads
};

template <int D> struct Cfg {
  static constexpr int CH = D / 8;            // 16-byte chunks per K row
  static constexpr int RPI = 64 / CH;         // K rows per 1 KiB wave load
  static constexpr int KLW = BN / RPI / NW;   // K wave loads per wave per step
  static constexpr int KTILE = BN * D;        // elements of a K tile
  static constexpr int DS_LOADS = 4;           // dS loads per wave per step
};

struct Params {
  const bf16* k;
  const char* ds;
  const int* bounds;   // per-token document [start, end) (document masking only)
  bf16* dq;
  const bf16* qraw; const float* cs; float eps;   // QN kernels: the query prologue's backward
  int B, T, H, window, nkb, nslot, nqt;
  int lpt;   // longest-first order across heads (lpt_order)
  float scale;
};

// 16-byte LDS store issued as a plain ds_write_b128 (see ds_store_b64 in common.h: the compiler
// would otherwise drain the in-flight global->LDS copies before it). The buffer it writes is
// private to the wave and never a copy target.
__device__ __forceinline__ void ds_store_b128(lds_t<char>* p, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"((unsigned)(size_t)p), "v"(v) : "memory");
}

template <int D, bool DOC, bool QN>
__global__ void __launch_bounds__(64 * NW, Pipe<DOC>::WG_PER_CU) dq_ds_kernel(Params p) {
  using C = Cfg<D>;
  constexpr int PF = Pipe<DOC>::PF, RING = Pipe<DOC>::RING, KPF = Pipe<DOC>::KPF,
                UNROLL = Pipe<DOC>::UNROLL, NBATCH = Pipe<DOC>::NBATCH;
  constexpr int NDB = D / 32;
  // K tiles: double-buffered, written from registers at their step. Transpose buffers: each
  // wave's two stored chunks of the current step (written from registers).
  __shared__ __attribute__((aligned(16))) bf16 kb0[C::KTILE], kb1[C::KTILE];
  __shared__ __attribute__((aligned(16))) char tbuf[NW * 2 * dsb::CHUNK_BYTES];
  auto kslot = [&](int slot) __attribute__((always_inline)) {
    return (lds_t<bf16>*)(slot == 0 ? kb0 : kb1);
  };

  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5;
  const int l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int T = p.T, H = p.H, W = p.window;

  // XCD-aware order (the query tiles of one (b, h) share that XCD's L2 for K), most key blocks
  // first, heads in the reverse of the order the dK/dV kernel wrote them, so that the chunks
  // written last (still in the memory-side cache) are read first.
  int bh, qt;
  if (p.lpt) {   // small full-causal grids: longest first across heads
    const int2 br = lpt_block(p.nqt, kCusPerXcd);
    bh = br.x;
    qt = p.nqt - 1 - br.y;
  } else {
    const int nblk = gridDim.x;
    int L = blockIdx.x;
    if ((nblk & 7) == 0) L = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    L = nblk - 1 - L;
    L = (L / p.nqt) * p.nqt + (p.nqt - 1 - L % p.nqt);   // keep the longest tiles first
    bh = L / p.nqt;
    qt = p.nqt - 1 - (L - bh * p.nqt);
  }
  const int b = bh / H, h = bh - b * H;
  const size_t head0 = ((size_t)b * T * H + h) * D;
  const size_t rs = (size_t)H * D;
  const bf16* kbase = p.k + head0;
  const int q0 = qt * BM;
  const int myq = q0 + 32 * wave + l32;

  // Key blocks the tile's queries can see: the window's, and with document masking none before
  // the block holding the document start of the tile's first query (later queries start their
  // documents no earlier).
  int kb_lo = max(0, qt - p.nslot + 1);
  if constexpr (DOC) kb_lo = max(kb_lo, p.bounds[2 * ((size_t)b * T + q0)] / dsb::KEYS);
  const int kb_hi = min(qt, p.nkb - 1);
  const int nsteps = 2 * (kb_hi - kb_lo + 1);

  // Lane-constant LDS offsets (bytes). K^T reads: key rows 8 hi + 4 t + (j / 4) (+ 32 cc + 16 ks
  // at each use, multiples of 16 rows, which keep the swizzle), dims 32 db + 16 (g % 2) + 4 (j % 4).
  // dS^T reads: key 8 hi + 4 t + (j / 4) (+ 16 ks), queries 16 (g % 2) + 4 (j % 4) .. + 3, stored
  // as run a = that / 8 of half (j % 4) % 2 at 64 key + 32 half + 8 a.
  int ktr[2][NDB], dtr[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 8 * hi + 4 * t + (j >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 32 * db + 16 * (g & 1) + 4 * (j & 3);
      ktr[t][db] = 2 * (r * D + 8 * ((d >> 3) ^ swz<D>(r)) + 4 * ((d >> 2) & 1));
    }
    const int c = j & 3;
    dtr[t] = 64 * r + 32 * (c & 1) + 16 * (g & 1) + 8 * (c >> 1);
  }

  // K tile loads: lane l of wave load I lands at row I*RPI + l/CH, position l%CH, and fetches
  // source chunk (l%CH) ^ swz(row).
  unsigned kloff[C::KLW];
  int krow[C::KLW];
#pragma unroll
  for (int i = 0; i < C::KLW; ++i) {
    const int I = wave * C::KLW + i;
    krow[i] = I * C::RPI + lane / C::CH;
    kloff[i] = 2u * (unsigned)(krow[i] * (int)rs + 8 * ((lane % C::CH) ^ swz<D>(krow[i])));
  }

  // With document masking a chunk's liveness depends on the end of its key group's document.
  // Lane i holds that end for key group i of the tile's key range, loaded once here, so that
  // the issue of each step's loads does not wait on a load of the bounds (ranges of more than
  // 64 key groups read them at the step).
  const int nkg = 4 * (kb_hi - kb_lo + 1);
  int kend_l = T;
  if constexpr (DOC) {
    const int kc = min(kb_lo * dsb::KEYS + 32 * lane + 31, T - 1);
    if (lane < nkg) kend_l = p.bounds[2 * ((size_t)b * T + kc) + 1];
  }
  auto live = [&](int st, int w) {
    const int kw = (kb_lo + (st >> 1)) * dsb::KEYS + 32 * w;
    if constexpr (DOC) {
      if (nkg <= 64) {
        if (kw >= T) return false;
        const int kc = min(kw + 31, T - 1);
        const int kend = __builtin_amdgcn_readlane(kend_l, 4 * (st >> 1) + w);
        const int whi1 = min(kc + W - 1, kend - 1);
        const int qm = q0 + 32 * wave;
        return !(qm + 31 < kw || qm > whi1);
      }
    }
    return dsb::chunk_live<DOC>(p.bounds, b, T, W, kw, q0 + 32 * wave);
  };

  // Loads of step st, clamped to the last step (the surplus issues at the end keep the count of
  // vector-memory operations per step fixed). issue_ds: the wave's two stored chunks into
  // registers (a chunk the dK/dV kernel did not write is read through an empty buffer range,
  // which returns zeros without a memory access). issue_k: this wave's share of the K tile into
  // LDS buffer `slot`.
  u32x4 dsr[RING][4];
  auto issue_ds = [&](int st_raw, u32x4 (&dst)[4]) __attribute__((always_inline)) {
    const int st = min(st_raw, nsteps - 1);
    const int kb = kb_lo + (st >> 1), hh = st & 1;
    const char* blk = p.ds + dsb::block_offset(bh, kb, qt - kb, p.nkb, p.nslot);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const char* chunk = blk + (size_t)((2 * hh + cc) * 4 + wave) * dsb::CHUNK_BYTES;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(chunk), 0, live(st, 2 * hh + cc) ? dsb::CHUNK_BYTES : 0, 0x00020000);
      dst[2 * cc + 0] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16u * lane, 0, 2));
      dst[2 * cc + 1] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16u * lane + 1024u, 0, 2));
    }
  };
  // issue_k: this wave's share of the K tile of step st into registers (lane l of wave load I
  // holds row I*RPI + l/CH, source chunk (l%CH) ^ swz(row), for LDS position l%CH).
  u32x4 kreg[KPF][C::KLW];
  auto issue_k = [&](int st_raw, u32x4 (&dst)[C::KLW]) __attribute__((always_inline)) {
    const int st = min(st_raw, nsteps - 1);
    const int kb = kb_lo + (st >> 1), hh = st & 1;
    const int k0 = kb * dsb::KEYS + BN * hh;
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kbase + (size_t)k0 * rs);
#pragma unroll
    for (int i = 0; i < C::KLW; ++i) {
      const int over = max(k0 + krow[i] - (T - 1), 0);   // rows past the end re-read row T-1
      dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
          rk, opaque(kloff[i]) - 2u * (unsigned)over * (unsigned)rs, 0, 0));
    }
  };
  auto put_k = [&](const u32x4 (&src)[C::KLW], int slot) __attribute__((always_inline)) {
    lds_t<bf16>* ks = kslot(slot);
#pragma unroll
    for (int i = 0; i < C::KLW; ++i)
      *reinterpret_cast<lds_t<u32x4>*>(ks + (wave * C::KLW + i) * C::RPI * D + 8 * lane) = src[i];
  };

  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = (f32x16){};

  lds_t<char>* tb = (lds_t<char>*)tbuf + wave * 2 * dsb::CHUNK_BYTES;
  // this wave's stored chunks of a step into its transpose buffer, in their stored layout
  auto stage = [&](const u32x4 (&src)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ds_store_b128(tb + (i >> 1) * dsb::CHUNK_BYTES + 16 * lane + 1024 * (i & 1), src[i]);
  };
  auto compute = [&](int st, int slot) __attribute__((always_inline)) {
    const lds_t<char>* ks = (const lds_t<char>*)kslot(slot);
    const int hh = st & 1;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      if (!live(st, 2 * hh + cc)) continue;
      const lds_t<char>* sc = tb + cc * dsb::CHUNK_BYTES;
      const lds_t<char>* kc = ks + 2 * (32 * cc) * D;
#pragma unroll
      for (int kst = 0; kst < 2; ++kst) {
        const bf16x8 bs = __builtin_shufflevector(
            ds_read_tr16((const lds_t<bf16>*)(sc + 1024 * kst + dtr[0])),
            ds_read_tr16((const lds_t<bf16>*)(sc + 1024 * kst + dtr[1])), 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const lds_t<char>* kr = kc + 2 * (16 * kst) * D;
          const bf16x8 ak = __builtin_shufflevector(
              ds_read_tr16((const lds_t<bf16>*)(kr + ktr[0][db])),
              ds_read_tr16((const lds_t<bf16>*)(kr + ktr[1][db])), 0, 1, 2, 3, 4, 5, 6, 7);
          dqacc[db] = mfma32(ak, bs, dqacc[db]);
        }
      }
    }
  };

  // Step st: write its K rows and its dS chunks into LDS (every wave is past the previous
  // step's barrier, so no wave still reads the K buffer of step st - 2), workgroup barrier,
  // load the K rows of step st + KPF and the dS chunks of step st + PF into the registers just
  // freed, compute step st. The compiler waits for the K rows and dS chunks of step st; the
  // counter being in order, that also waits for the loads issued before them, which still leaves
  // the dS loads of steps st + 1 .. st + PF - 1 and the K rows of steps st + 1 .. st + KPF - 1 in
  // flight.
  auto step = [&](int st, int R) __attribute__((always_inline)) {
    put_k(kreg[R % KPF], R & 1);
    stage(dsr[R]);
    lds_sync();
    sched_fence();
    issue_k(st + KPF, kreg[R % KPF]);
    issue_ds(st + PF, dsr[(R + PF) % RING]);
    sched_fence();
    compute(st, R & 1);
  };

  // prologue: the loads of steps 0 .. PF - 1 in the order the steps keep (K rows KPF steps and
  // dS chunks PF steps ahead of the step that issues them)
#pragma unroll
  for (int s0 = 0; s0 < PF; ++s0) {
    if (s0 < KPF) issue_k(s0, kreg[s0]);
    issue_ds(s0, dsr[s0]);
  }
  sched_fence();
  // Unrolled by two turns of the register ring: the compiler's wait analysis does not carry
  // the ages of the ring's loads across the loop's back edge and waits for all of them at its
  // head, so the head comes once per UNROLL steps. Each step waits for its own K rows and dS
  // chunks (issued KPF and PF steps earlier) and, the counter being in order, for every load
  // issued before them: with PF = 3 the dS loads of the next step stay in flight; with PF = 1
  // (three workgroups per CU) none of the wave's loads do, and the CU's other workgroups cover
  // the wait.
  for (int st = 0; st < nsteps; st += UNROLL) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if (st + u >= nsteps) break;
      step(st + u, u % RING);
    }
  }

  wait_vmem();   // the surplus loads of the last steps land before the wave ends

  if constexpr (QN) {
    // The backward of the query prologue (RMS norm, then RoPE) in the row layout of
    // rope_row.h, so that dq is bitwise what rope_qknorm_bwd computes from this kernel's bf16
    // dq_hat: each wave puts its dq_hat rows, rounded to bf16 and 16-byte chunks XOR-swizzled,
    // into the K buffers (rows 0-63 in kb0, 64-127 in kb1) once every wave is done with them;
    // then TPR lanes per row read a row back with the raw q row and the angles of its position
    // and write dq.
    using RW = RowWord<bf16>;
    constexpr int VPT = RW::VPT, TPR = D / VPT, RPP = 64 * NW / TPR, NP = BM / RPP;
    const int lr = tid % TPR;
    const bool second = lr >= TPR / 2;
    // The raw rows and angles of the passes are loaded in NBATCH batches (rows past the end
    // re-read the last row and store nothing); the first batch's latency overlaps the staging
    // below.
    constexpr int PB = NP / NBATCH;
    static_assert(NP % NBATCH == 0, "whole batches");
    RW x[PB];
    float c[PB][VPT], s[PB][VPT];
    auto load_batch = [&](int bt) __attribute__((always_inline)) {
#pragma unroll
      for (int pp = 0; pp < PB; ++pp) {
        const int t = min(q0 + (bt * PB + pp) * RPP + tid / TPR, T - 1);
        x[pp].load_stream(p.qraw + head0 + (size_t)t * rs + lr * VPT);
        load_cs<VPT>(p.cs, t, D / 2, (lr % (TPR / 2)) * VPT, c[pp], s[pp]);
      }
    };
    load_batch(0);
    __syncthreads();
    if (myq < T) {
      const int rl = (32 * wave + l32) & 63;
      lds_t<bf16>* rowp = kslot(wave >> 1) + rl * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const u32x2 w = {pack_bf2(dqacc[db][4 * a + 0] * p.scale, dqacc[db][4 * a + 1] * p.scale),
                           pack_bf2(dqacc[db][4 * a + 2] * p.scale, dqacc[db][4 * a + 3] * p.scale)};
          const int ch = 4 * db + a;   // 16-byte chunk of d = 32 db + 8 a
          *reinterpret_cast<lds_t<u32x2>*>(rowp + 8 * (ch ^ swz<D>(rl)) + 4 * hi) = w;
        }
    }
    __syncthreads();
#pragma unroll
    for (int bt = 0; bt < NBATCH; ++bt) {
      if (bt > 0) load_batch(bt);
#pragma unroll
      for (int pp = 0; pp < PB; ++pp) {
        const int r = (bt * PB + pp) * RPP + tid / TPR;
        const int t = q0 + r;
        const int rl = r & 63;
        const u32x4 gw = *reinterpret_cast<const lds_t<u32x4>*>(kslot(r >> 6) + rl * D +
                                                                 8 * (lr ^ swz<D>(rl)));
        RW g, out;
        g.v[0] = bf_lo(gw[0]); g.v[1] = bf_hi(gw[0]); g.v[2] = bf_lo(gw[1]); g.v[3] = bf_hi(gw[1]);
        g.v[4] = bf_lo(gw[2]); g.v[5] = bf_hi(gw[2]); g.v[6] = bf_lo(gw[3]); g.v[7] = bf_hi(gw[3]);
        rope_norm_row_bwd<VPT, TPR, D>(x[pp].v, g.v, c[pp], s[pp], second, p.eps, out.v);
        // dq is the layer's final output: written with the nontemporal hint, so that it does
        // not displace cached data (~3 % of this kernel's time on the d24 sweep)
        if (t < T) {
          const u32x4 w = {pack_bf2(out.v[0], out.v[1]), pack_bf2(out.v[2], out.v[3]),
                           pack_bf2(out.v[4], out.v[5]), pack_bf2(out.v[6], out.v[7])};
          __builtin_nontemporal_store(
              w, reinterpret_cast<u32x4*>(p.dq + head0 + (size_t)t * rs + lr * VPT));
        }
      }
    }
    return;
  }
  // dq row myq: lane holds d = 32 db + 8 a + 4 hi + (0..3)
  if (myq < T) {
    bf16* op = p.dq + head0 + (size_t)myq * rs;
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

template <int D, bool QN>
static hipError_t launch_t(const AttnShape& a, const Params& p, hipStream_t s) {
  const unsigned blocks = (unsigned)p.nqt * a.B * a.H;
  if (a.bounds)
    hipLaunchKernelGGL((dq_ds_kernel<D, true, QN>), dim3(blocks), dim3(64 * NW), 0, s, p);
  else
    hipLaunchKernelGGL((dq_ds_kernel<D, false, QN>), dim3(blocks), dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

}  // namespace dqs

size_t ds_buffer_bytes(int B, int T, int H, int window) {
  return dsb::buffer_bytes(B, T, H, window);
}

hipError_t launch_dq_from_ds(const AttnShape& a, const void* k, const void* ds, void* dq,
                             hipStream_t s, const QNorm* qnorm) {
  dqs::Params p;
  p.k = (const bf16*)k;
  p.ds = (const char*)ds;
  p.bounds = a.bounds;
  p.dq = (bf16*)dq;
  p.B = a.B; p.T = a.T; p.H = a.H; p.window = a.window;
  p.nkb = dsb::nkb(a.T);
  p.nslot = dsb::nslot(a.T, a.window);
  p.nqt = (a.T + dqs::BM - 1) / dqs::BM;
  p.lpt = lpt_order(a) ? 1 : 0;
  p.scale = a.scale;
  p.qraw = qnorm ? (const bf16*)qnorm->q : nullptr;
  p.cs = qnorm ? qnorm->cs : nullptr;
  p.eps = qnorm ? qnorm->eps : 0.f;
  if (qnorm)
    return a.D == 64 ? dqs::launch_t<64, true>(a, p, s) : dqs::launch_t<128, true>(a, p, s);
  return a.D == 64 ? dqs::launch_t<64, false>(a, p, s) : dqs::launch_t<128, false>(a, p, s);
}

}  // namespace swa

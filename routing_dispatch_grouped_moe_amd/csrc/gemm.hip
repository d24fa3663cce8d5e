// Grouped GEMMs of the expert FFN and its backward (SwiGLU row of the T4
// tuning page's "RMSNorm, RoPE, SwiGLU" table: three matrix products per
// expert; MoonEP page, weights step: one contiguous tensor per projection,
// the grouped GEMM reaching expert e's weights from e alone; MoonEP page,
// gradient step: an fp32 gradient buffer shaped like the weights).
//
// Two grouping kinds over the expert row offsets cu[E+1]:
//   M-grouped  C[rows of e, N] = A[rows of e, K] * B_e[K, N]      (fwd, dA, dxd)
//   K-grouped  C_e[M, N] = A[rows of e, M]^T * B[rows of e, N]    (dW1, dW3, dW2)
//
// gfx950 design.  Every bf16 product computes 256 x 256 output tiles
// (256 x (128 + 128) for the two-operand gate/up and dW1/dW3 cases) on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators, K advancing 64 per step.
// Operand tiles live in LDS in one of two layouts, both XOR-swizzled on
// 16-byte chunks for the 64-bank LDS (measured conflict-free):
//   - K-contiguous rows ([rows][64], 128 B a row) for operands stored
//     K-major in HBM (activations in the forward, weights in dA/dxd);
//     fragments are read with ds_read_b128;
//   - K-major rows ([64][cols]) for operands stored with M or N contiguous
//     (weights [H, H'] in the forward, activations in the weight gradients);
//     fragments are read with the gfx950 LDS transpose load
//     ds_read_b64_tr_b16, which hands each lane four consecutive-k values of
//     one column, so no operand is ever transposed in registers.
// Two tile forms:
//   - one wavefront per SIMD (gemm_bf16_w4_kernel): the forward, dA, dxd and
//     the weight gradients of experts with many rows.  256 accumulators per
//     lane, operands reach LDS by direct loads, and every epilogue is staged
//     through LDS and leaves as whole rows;
//   - eight wavefronts, two per SIMD (gemm_bf16_kernel): the weight
//     gradients of experts with few rows and the accumulating weight
//     gradients, with register-staged loads one K step ahead.
// Global reads are bounded by buffer descriptors to the expert's rows (reads
// past the end return zero, which pads ragged M tiles and the ragged K tail
// of the weight gradients).  M tiles come from a device-built table (expert,
// first row), so nothing syncs with the host; their block ids are renumbered
// so that each XCD (own L2) runs a contiguous patch of tiles, and the tiles
// of a partial last wave of the plain-store products are split along K.
//
// The fp32 storage type (the tiny fp32 workload) uses a plain FMA kernel
// with the same tile table and epilogues.
#include <type_traits>

#include "dev_common.h"
#include "launch.h"
#include "tile.h"

namespace moe {

// f(integral_constant<int, I>) for I = B .. E-1, unrolled by construction (a
// loop the optimiser leaves rolled would index the accumulator array at run
// time and move it to scratch memory)
template <int B, int E>
struct StaticFor {
  template <class F>
  __device__ __forceinline__ static void run(F&& f) {
    if constexpr (B < E) {
      f(std::integral_constant<int, B>{});
      StaticFor<B + 1, E>::run(f);
    }
  }
};

constexpr int kThreads = 512;  // eight wavefronts: 2 along M x 4 along N

// EPI_F32 overwrites the fp32 weight gradient, EPI_F32_ACC adds to it (two
// kinds, so the overwrite form carries no loads of the old values)
enum { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2, EPI_F32 = 3, EPI_F32_ACC = 4 };
constexpr bool epi_f32(int epi) { return epi == EPI_F32 || epi == EPI_F32_ACC; }

struct GemmArgs {
  const int32_t* cu;      // [E+1] row offsets of the experts
  const int2* tiles;      // M-grouped: (expert, first row inside the expert) of each M tile
  const int32_t* ntiles;  // M-grouped: number of valid M tiles
  const int32_t* eorder;  // K-grouped: experts in dealing order (nullptr: index order)
  int E, M, N, K;         // M-grouped: N and K (K per segment); K-grouped: M and N
  int mtn, ntn;           // tiles along M (K-grouped) / along N
  const void* A0;         // row-indexed operand (second K segment in A1)
  const void* A1;
  int64_t lda;
  const void* B0;         // second B operand in B1 (dual) or second K segment (two-segment)
  const void* B1;
  int64_t ldb;
  int64_t sBe;            // per-expert stride of B (weights); 0 when B is row-indexed
  void* C0;
  void* C1;
  void* C2;
  int64_t ldc;
  int64_t sCe;            // per-expert stride of C (weight gradients)
  const void* X0;         // h1, h3 for the SwiGLU backward epilogue
  const void* X1;
  int accum;
  float* part;            // K-split partial tiles of the last wave (store epilogue)
  int tail_cap;           // capacity of part in tiles
  int ncu;                // compute units of the device (tiles in flight per wave)
  int deal_whole;         // K-grouped with eorder: light experts go whole to one XCD
};

// ------------------------------------------------------------- epilogue --
template <int EPI, bool BF16, bool DUAL>
__device__ __forceinline__ void epilogue(const GemmArgs& p, int e, int64_t row, int col, float v0,
                                         float v1) {
  const int64_t o = row * p.ldc + col;
  if constexpr (EPI == EPI_STORE) {
    store1<BF16>(p.C0, o, v0);
  } else if constexpr (EPI == EPI_SWIGLU_FWD) {
    // h1 (C0), h3 (C1) and a (C2); a null output is not written
    if (p.C0) store1<BF16>(p.C0, o, v0);
    if (p.C1) store1<BF16>(p.C1, o, v1);
    if (p.C2) store1<BF16>(p.C2, o, silu_f(v0) * v1);
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    const float z = load1<BF16>(p.X0, o), u = load1<BF16>(p.X1, o);
    const float sg = sigmoid_f(z);
    store1<BF16>(p.C0, o, v0 * u * sg * (1.0f + z * (1.0f - sg)));
    store1<BF16>(p.C1, o, v0 * z * sg);
  } else {
    // weight gradients are written once and not read again in the layer:
    // non-temporal stores keep them from displacing operand tiles in L2
    float* c0 = reinterpret_cast<float*>(p.C0) + (int64_t)e * p.sCe + o;
    __builtin_nontemporal_store(EPI == EPI_F32_ACC ? *c0 + v0 : v0, c0);
    if constexpr (DUAL) {
      float* c1 = reinterpret_cast<float*>(p.C1) + (int64_t)e * p.sCe + o;
      __builtin_nontemporal_store(EPI == EPI_F32_ACC ? *c1 + v1 : v1, c1);
    }
  }
}

// Tile coordinates of a block.  Returns false when the block has no tile.
// valid: rows of the tile inside the expert (M-grouped) or the expert's row
// count, i.e. the reduction length (K-grouped).
//
// M tile groups (2^gms M tiles x all N tiles) in the order the XCDs take
// them; the tile table picks gms.  Groups of four M tiles share each weight
// panel in L2 while experts have several tiles; when none has more than
// one, groups of one put all N tiles of an expert on one XCD at once, and
// its activation rows are fetched into that L2 once (measured at 384
// experts: ffn_up 28.3 -> 25.1 GB fetched, bwd_dxd 25.6 -> 24.3 GB; groups
// of one with hot experts of many tiles: +0.7 ms per step at maxvio 20).
// When most experts have one tile and a few hot ones many (skewed routing),
// groups of two do best: -0.3 to -0.9 ms per step at maxvio 20 and -1.2% on
// 64 Zipf-skewed experts, where balanced multi-tile routing (8 experts of
// 2048 rows, 16 of 512) runs 1-2% slower with them than with four.
// The tile table lists the M tiles longest expert first, so groups come in
// falling cost: under skew the first are the heavy experts' full
// tiles (MFMA-bound), the last the light experts' short ones (bound by the
// weight stream).  XCD a walks a contiguous range of positions pg = a Q + b
// (Q = G / 8 groups each).  Its i-th costliest share is group 8 i + a for
// even i and 8 i + 7 - a for odd i (snake order: like work per XCD), and it
// takes its shares alternately from the costly and the cheap end, the even
// XCDs starting at the costly end and the odd ones at the cheap end, so
// that at any time about half the XCDs run MFMA-bound tiles while the rest
// stream weights.  The last G mod 8 groups keep their place.
__device__ __forceinline__ int group_dealt(int pg, int G) {
  const int Q = G >> 3;
  if (pg >= 8 * Q) return pg;
  const int a = pg / Q, b = pg - a * Q, h = b >> 1;
  const int i = (((b ^ a) & 1) == 0) ? h : Q - 1 - h;
  return 8 * i + ((i & 1) ? 7 - a : a);
}

// M-grouped tile t of T = ntiles * ntn: groups of 2^gms M tiles (fewer in
// the last group) walked with the M tile fastest, full groups dealt to the
// XCDs by group_dealt.
__device__ __forceinline__ void mtile_of(int t, int ntiles, int ntn, int gms, int& mt, int& nt) {
  const int gm = 1 << gms, per_group = ntn << gms, nfull = ntiles >> gms;
  const int g4 = nfull * per_group;
  if (t < g4) {
    const int pg = t / per_group, r = t - pg * per_group;
    const int g = group_dealt(pg, nfull);
    mt = (g << gms) + (r & (gm - 1));
    nt = r >> gms;
  } else {
    const int r = t - g4, gl = ntiles & (gm - 1);
    mt = (nfull << gms) + r % gl;
    nt = r / gl;
  }
}

// Last-wave K split.  With T tiles on ncu compute units, a last wave of
// rem = T mod ncu tiles (at most half a wave) leaves most units idle for a
// whole tile time; those tiles are split along K into s parts (s rem blocks
// after the T - rem whole tiles), each part writes an fp32 partial tile and
// a second kernel sums the parts in order.  Both kernels derive the plan
// from the same inputs.
struct SplitPlan {
  int full;  // whole tiles (block ids 0 .. full-1)
  int rem;   // tiles of the last wave that are split
  int s;     // parts per split tile (1: no split)
};
constexpr int kMaxSplit = 8, kMinSplitSteps = 16;
__device__ __forceinline__ SplitPlan split_plan(const GemmArgs& p, int nk2) {
  const int T = *p.ntiles * p.ntn;
  SplitPlan sp{T, 0, 1};
  const int rem = p.ncu > 0 ? T % p.ncu : 0;
  if (rem > 0 && 2 * rem <= p.ncu) {
    const int s = min(min(p.ncu / rem, kMaxSplit), min(p.tail_cap / rem, nk2 / kMinSplitSteps));
    if (s >= 2) sp = SplitPlan{T - rem, rem, s};
  }
  return sp;
}

// Tile of block bid of an M-grouped launch that may split its last wave;
// part = -1 for a whole tile, else the K part (item = its partial tile).
template <int BM, int BN, bool SPLIT>
__device__ __forceinline__ bool mtile_split(const GemmArgs& p, int bid, int nk2, int& e,
                                            int64_t& row0, int& valid, int& n0, int& part,
                                            int& item, int& nparts) {
  SplitPlan sp{*p.ntiles * p.ntn, 0, 1};
  if constexpr (SPLIT) sp = split_plan(p, nk2);
  part = -1; item = 0; nparts = sp.s;
  int t;
  if (bid < sp.full) {
    t = xcd_remap(bid, sp.full);
  } else {
    const int j = bid - sp.full;
    if (j >= sp.rem * sp.s) return false;
    t = sp.full + j / sp.s;
    part = j % sp.s;
    item = j;
  }
  int mt, nt;
  mtile_of(t, p.ntiles[0], p.ntn, p.ntiles[1], mt, nt);
  n0 = nt * BN;
  const int2 tt = p.tiles[mt];
  e = tt.x;
  row0 = (int64_t)p.cu[e] + tt.y;
  valid = min(BM, p.cu[e + 1] - (int)row0);
  return true;
}

// K-grouped blocks go expert by expert, the experts in the tile table's
// longest-first order when one is given.  With deal_whole, that order, and
// tiles per expert a multiple of 8, the heavy experts' tiles are shared by
// all XCDs (balanced load) and every other expert's tiles stay on one XCD
// (one L2 fetch of its operand rows); otherwise every XCD shares every
// expert.  Measured at 384 experts: whole dealing speeds dW2 up by 7-10% and
// slows dW1/dW3 by 6-12%, so only dW2 asks for it.
// Inside an expert's range the tiles run N fastest, or with PATCH in groups
// of 1024 / BM M tiles (1024 rows of the M side) x all N tiles (M fastest),
// so the tiles an XCD holds at once form a compact patch whose operand rows
// its L2 shares.  Measured: PATCH speeds up the few-row dW1/dW3 product (-9%
// at 384 experts) and slows the others (dW2 there, the many-row products),
// whose N-fastest order keeps each block's fp32 output rows contiguous; with
// 128-row tiles, patches of 8 M tiles beat 4, 6 and 12 (dW1/dW3 9.2 against
// 9.7-10.1, 9.5 and 9.3 ms at 384 experts).
template <bool KGROUP, int BM, int BN, bool PATCH = false, bool PATCH_SKEW = false>
__device__ __forceinline__ bool tile_of(const GemmArgs& p, int bid, int& e, int64_t& row0,
                                        int& valid, int& m0, int& n0) {
  if constexpr (KGROUP) {
    const int per_e = p.mtn * p.ntn;
    int slot, rp;
    // PATCH_SKEW: patches only under skewed routing, i.e. when the hottest
    // expert has more than twice the mean rows (measured with the one-
    // wavefront-per-SIMD dW1/dW3: -9% on 64 Zipf-skewed experts, +6% on 16
    // balanced ones, the same on 8 balanced ones)
    bool patch = PATCH;
    if constexpr (PATCH_SKEW) {
      if (p.eorder != nullptr) {
        const int eh = p.eorder[0];
        const int64_t rows = (int64_t)p.cu[p.E] - p.cu[0];
        patch = (int64_t)(p.cu[eh + 1] - p.cu[eh]) * p.E > 2 * rows;
      }
    }
    if (p.deal_whole && p.eorder != nullptr && (per_e & 7) == 0) {
      // Block bid runs on XCD bid % 8 as that XCD's block bid / 8.  The first
      // T experts of the dealing order (the heavy ones) are split eight ways,
      // one contiguous eighth of each per XCD; every other expert goes whole
      // to one XCD, dealt in snake order (0..7, 7..0, ...), so its operand
      // rows are fetched into one L2 instead of eight.
      const int x = bid & 7, j = bid >> 3, P = per_e >> 3;
      int T = p.eorder[p.E];
      if (T < 0 || T > p.E || ((p.E - T) & 7)) T = p.E;
      if (j < T * P) {
        slot = j / P;
        rp = x * P + (j - slot * P);
      } else {
        const int jc = j - T * P, wv = jc / per_e;
        rp = jc - wv * per_e;
        slot = T + 8 * wv + ((wv & 1) ? 7 - x : x);
      }
    } else {
      slot = bid / per_e;
      const int rem = bid - slot * per_e;
      rp = patch ? xcd_remap(rem, per_e) : rem;
    }
    e = p.eorder ? p.eorder[slot] : slot;
    if (patch) {
      constexpr int kPatchM = 1024 / BM;
      const int per_group = kPatchM * p.ntn;
      const int g = rp / per_group, r = rp - g * per_group;
      const int gm = min(kPatchM, p.mtn - g * kPatchM);  // the last group may be short
      m0 = (g * kPatchM + r % gm) * BM;
      n0 = (r / gm) * BN;
    } else {
      m0 = (rp / p.ntn) * BM;
      n0 = (rp % p.ntn) * BN;
    }
    row0 = p.cu[e];
    valid = max(0, p.cu[e + 1] - p.cu[e]);
    return true;
  } else {
    // The grid is sized for the most M tiles the routing could produce; only
    // the first nvalid block ids carry tiles, and only they are renumbered
    // (so every XCD gets its share of the real work).
    const int gms = p.ntiles[1], gm = 1 << gms, per_group = p.ntn << gms;
    const int nvalid = ((*p.ntiles + gm - 1) >> gms) * per_group;
    if (bid >= nvalid) return false;
    bid = xcd_remap(bid, nvalid);
    const int pg = bid / per_group, r = bid - pg * per_group;
    const int mt = (group_dealt(pg, nvalid / per_group) << gms) + (r & (gm - 1));
    n0 = (r >> gms) * BN;
    if (mt >= *p.ntiles) return false;
    const int2 t = p.tiles[mt];
    e = t.x;
    row0 = (int64_t)p.cu[e] + t.y;
    valid = min(BM, p.cu[e + 1] - (int)row0);
    m0 = 0;
    return true;
  }
}

// One operand tile of one K step, staged global -> registers -> LDS.
//   KC:  stored [rows][K] in HBM, tile rows [0, ROWS), k [k0, k0+64)
//   !KC: stored [K][cols] in HBM, tile k rows [k0, k0+64), cols [c0, c0+ROWS)
template <bool KC, int ROWS, int NOPS, int THREADS = kThreads>
struct Stager {
  static constexpr int kChunks = ROWS * (kBK / 8);          // 16-byte chunks per operand
  static constexpr int kPer = NOPS * kChunks / THREADS;     // per thread
  static_assert(kChunks % THREADS == 0, "operand tile not a multiple of the block");
  u32x4 r[kPer];

  __device__ __forceinline__ void load(const __amdgpu_buffer_rsrc_t (&rs)[NOPS], int64_t ld,
                                       int base, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      // operand index from the unrolled step alone (uniform), chunk from the thread
      const int op = (THREADS * i) / kChunks, lq = (THREADS * i) % kChunks + tid;
      int64_t el;
      if constexpr (KC) {
        el = (int64_t)(base + (lq >> 3)) * ld + k0 + (lq & 7) * 8;
      } else {
        constexpr int cpr = ROWS / 8;  // chunks per k row
        el = (int64_t)(k0 + lq / cpr) * ld + base + (lq % cpr) * 8;
      }
      r[i] = buf_load16(rs[op], (uint32_t)(el * 2));
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int op = (THREADS * i) / kChunks, lq = (THREADS * i) % kChunks + tid;
      char* t = lds + op * (ROWS * kBK * 2);
      uint32_t off;
      if constexpr (KC) {
        off = kc_off(lq >> 3, lq & 7);
      } else {
        constexpr int cpr = ROWS / 8;
        off = km_off<ROWS>(lq / cpr, lq % cpr);
      }
      *reinterpret_cast<u32x4*>(t + off) = r[i];
    }
  }
};

// Wait for this wave's LDS accesses, then a workgroup barrier.  Global loads
// stay in flight (no vmcnt wait) and the compiler may not move memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Largest row count r (BM / 2^j, at least 32) whose r rows of rf bytes fit
// in lds bytes: the fp32 epilogue's staging rounds.
constexpr int f32_stage_rows(int lds, int rf, int bm) {
  return (bm > 32 && bm * rf > lds) ? f32_stage_rows(lds, rf, bm / 2) : bm;
}

// NS: LDS operand stages.  NS == 2 double-buffers the K loop (one block per
// CU); NS == 1 keeps one stage, which the next K step's staged registers
// overwrite after a barrier, so that two blocks share a CU (four wavefronts
// per SIMD, at most 128 registers each) and one block's fp32 stores can
// overlap the other's loads and MFMAs.  For that the two must not run in
// step: the first-round blocks that take the second slot of each CU (block
// ids ncu .. 2 ncu - 1, as blocks are handed to every CU once before any
// gets a second) start about 8 us late, roughly half a few-row tile's life,
// and the blocks that replace them inherit the offset.  Measured at 384
// experts: dW1/dW3 10.2 ms with both in step, 9.6-9.7 ms with the offset.
template <int BM, int BN, bool A_KC, bool B_KC, bool DUAL, bool TWOSEG, bool KGROUP, int EPI,
          int NS = 2>
__global__ __launch_bounds__(kThreads, NS == 1 ? 4 : 1) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int kWaves = kThreads / 64;
  constexpr int WM = BM / 2, WN = BN / 4;      // wavefront tile (per B operand)
  constexpr int MI = WM / 32, NJ = WN / 32;    // 32x32 MFMA blocks per wavefront
  constexpr int kTileA = BM * kBK * 2, kTileB = BN * kBK * 2;
  constexpr int kStage = kTileA + NB * kTileB;
  // This form serves the fp32 weight gradients and, with 64-row M tiles,
  // the M-grouped products of few-row experts.  The overwriting weight
  // gradient takes the transposed MFMA result (four consecutive columns per
  // lane), staged through LDS and stored as whole rows; the others keep the
  // direct result (each 4-byte load/store instruction of the accumulating
  // kind covers two whole 128-byte rows of the gradient it adds to; the
  // few-row outputs are small).
  static_assert(epi_f32(EPI) || (!KGROUP && BM == kGemmBMFew),
                "the eight-wavefront form: fp32 weight gradients, few-row M-grouped products");
  constexpr bool kSwapAB = EPI == EPI_F32;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  int e, valid, m0, n0;
  int64_t row0;
  if (!tile_of<KGROUP, BM, BN, KGROUP && DUAL>(p, blockIdx.x, e, row0, valid, m0, n0)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;

  __amdgpu_buffer_rsrc_t ra[TWOSEG ? 2 : 1];
  __amdgpu_buffer_rsrc_t rb[(DUAL || TWOSEG) ? 2 : 1];
  int a_base, b_base, nk;
  const int nk_seg = KGROUP ? 0 : p.K / kBK;
  if constexpr (KGROUP) {
    // A: [rows][M] of expert e (A^T read), B: [rows][N]; the reduction runs over the rows.
    if (valid == 0) {
      if (EPI != EPI_F32_ACC) {
        for (int i = tid; i < BM * BN; i += kThreads) {
          const int r = i / BN, c = i % BN;
          if (m0 + r < p.M && n0 + c < p.N) epilogue<EPI, true, DUAL>(p, e, m0 + r, n0 + c, 0.f, 0.f);
        }
      }
      return;
    }
    ra[0] = make_rsrc(reinterpret_cast<const uint16_t*>(p.A0) + row0 * p.lda,
                      (uint32_t)((int64_t)valid * p.lda * 2));
    rb[0] = make_rsrc(reinterpret_cast<const uint16_t*>(p.B0) + row0 * p.ldb,
                      (uint32_t)((int64_t)valid * p.ldb * 2));
    if constexpr (DUAL)
      rb[1] = make_rsrc(reinterpret_cast<const uint16_t*>(p.B1) + row0 * p.ldb,
                        (uint32_t)((int64_t)valid * p.ldb * 2));
    a_base = m0;
    b_base = n0;
    nk = (valid + kBK - 1) / kBK;
  } else {
    ra[0] = make_rsrc(reinterpret_cast<const uint16_t*>(p.A0) + row0 * p.lda,
                      (uint32_t)((int64_t)valid * p.lda * 2));
    if constexpr (TWOSEG)
      ra[1] = make_rsrc(reinterpret_cast<const uint16_t*>(p.A1) + row0 * p.lda,
                        (uint32_t)((int64_t)valid * p.lda * 2));
    const uint32_t wbytes = (uint32_t)((int64_t)p.N * p.K * 2);
    rb[0] = make_rsrc(reinterpret_cast<const uint16_t*>(p.B0) + (int64_t)e * p.sBe, wbytes);
    if constexpr (DUAL || TWOSEG)
      rb[1] = make_rsrc(reinterpret_cast<const uint16_t*>(p.B1) + (int64_t)e * p.sBe, wbytes);
    a_base = 0;
    b_base = n0;
    nk = TWOSEG ? 2 * nk_seg : nk_seg;
  }

  Stager<A_KC, BM, 1> sa;
  Stager<B_KC, BN, NB> sb;
  auto load = [&](int kt) {
    int seg = 0, k0 = kt * kBK;
    if constexpr (TWOSEG) {
      seg = kt >= nk_seg ? 1 : 0;
      k0 = (kt - seg * nk_seg) * kBK;
      const __amdgpu_buffer_rsrc_t rA[1] = {seg ? ra[1] : ra[0]};
      const __amdgpu_buffer_rsrc_t rB[1] = {seg ? rb[1] : rb[0]};
      sa.load(rA, p.lda, a_base, k0, tid);
      sb.load(rB, p.ldb, b_base, k0, tid);
    } else {
      sa.load(ra, p.lda, a_base, k0, tid);
      if constexpr (DUAL) {
        sb.load(rb, p.ldb, b_base, k0, tid);
      } else {
        const __amdgpu_buffer_rsrc_t rB[1] = {rb[0]};
        sb.load(rB, p.ldb, b_base, k0, tid);
      }
    }
  };

  f32x16 acc[NB][MI][NJ];
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][i][j][v] = 0.f;

  auto compute = [&](const char* st) {
    const char* tA = st;
    const char* tB = st + kTileA;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      u32x4 af[MI], bfr[NB][NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        if constexpr (A_KC) af[i] = frag_kc(tA, wm * WM + i * 32, kk, lane);
        else af[i] = frag_km<BM>(tA, wm * WM + i * 32, kk, lane);
      }
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const char* t = tB + q * kTileB;
          if constexpr (B_KC) bfr[q][j] = frag_kc(t, wn * WN + j * 32, kk, lane);
          else bfr[q][j] = frag_km<BN>(t, wn * WN + j * 32, kk, lane);
        }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[q][i][j] = kSwapAB
                ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bfr[q][j]),
                                                          __builtin_bit_cast(bf16x8, af[i]),
                                                          acc[q][i][j], 0, 0, 0)
                : __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                          __builtin_bit_cast(bf16x8, bfr[q][j]),
                                                          acc[q][i][j], 0, 0, 0);
      // keep one K16 slice of fragments live at a time (register budget of
      // two wavefronts per SIMD)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  load(0);
  sa.store(smem, tid);
  sb.store(smem + kTileA, tid);
  lds_barrier();
  if constexpr (NS == 1) {
    if ((int)blockIdx.x >= p.ncu && (int)blockIdx.x < 2 * p.ncu) {
      __builtin_amdgcn_s_sleep(127);  // 64 x 127 clocks each
      __builtin_amdgcn_s_sleep(127);
    }
  }
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = NS == 2 ? smem + (kt & 1) * kStage : smem;
    char* nxt = NS == 2 ? smem + ((kt + 1) & 1) * kStage : smem;
    if (kt + 1 < nk) load(kt + 1);
    compute(cur);
    if (kt + 1 < nk) {
      if constexpr (NS == 1) lds_barrier();  // every wavefront is done reading the stage
      sa.store(nxt, tid);
      sb.store(nxt + kTileA, tid);
    }
    lds_barrier();
  }

  if constexpr (EPI == EPI_F32) {
    // fp32 weight gradient of expert e: the NS x kStage bytes of LDS (free
    // after the loop's last barrier) hold kRows rows of BN floats (RF bytes,
    // 16-byte chunk c of row q at c ^ (q & 15)); non-temporal whole-row
    // stores.  Each operand's BM rows go in BM / kRows rounds; a wavefront
    // stages the 32-row blocks of its rows that fall in the round.
    constexpr int RF = BN * 4, LPRF = BN / 4, RPIF = 64 / LPRF;
    constexpr int kRows = f32_stage_rows(NS * kStage, RF, BM);
    constexpr int kRoundsPerOp = BM / kRows;
    static_assert(kRows % 32 == 0 && BM % kRows == 0 && kRows % (kWaves * RPIF) == 0,
                  "fp32 staging rounds");
    auto put_f4 = [&](int q, int c, const float (&v)[4]) {
      *reinterpret_cast<f32x4*>(smem + (uint32_t)q * RF + ((uint32_t)((c >> 2) ^ (q & 15)) << 4)) =
          f32x4{v[0], v[1], v[2], v[3]};
    };
    auto store_round = [&](float* C, int rbase) __attribute__((always_inline)) {
      // lane (c, q0) stores chunk c of rows q0, q0 + kPass, ...: one row
      // pointer per lane advanced by a fixed stride, one row-count compare
      constexpr int kPass = kWaves * RPIF;
      const int c = lane % LPRF, col = n0 + 4 * c, q0 = w * RPIF + lane / LPRF;
      if (col >= p.N) return;
      const int left = p.M - (m0 + rbase + q0);
      float* dst = C + (int64_t)(m0 + rbase + q0) * p.ldc + col;
      const int64_t step = (int64_t)kPass * p.ldc;
      const char* src = smem + (uint32_t)q0 * RF;
#pragma unroll
      for (int it = 0; it < kRows / kPass; ++it) {
        const int q = q0 + it * kPass;
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + it * kPass * RF + ((uint32_t)(c ^ (q & 15)) << 4));
        if (it * kPass < left) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
        dst += step;
      }
    };
    StaticFor<0, NB * kRoundsPerOp>::run([&](auto r_tag) {
      constexpr int x0 = decltype(r_tag)::value, b = x0 / kRoundsPerOp, rd = x0 % kRoundsPerOp;
      if constexpr (x0 > 0) lds_barrier();
      StaticFor<0, MI>::run([&](auto i_tag) {
        constexpr int i = decltype(i_tag)::value;
        const int row = wm * WM + i * 32;  // first tile row of the 32-row block
        if (row / kRows == rd) {
          StaticFor<0, NJ * 4>::run([&](auto tag) {
            constexpr int j = decltype(tag)::value / 4, g = decltype(tag)::value % 4;
            const float v[4] = {acc[b][i][j][4 * g], acc[b][i][j][4 * g + 1], acc[b][i][j][4 * g + 2],
                                acc[b][i][j][4 * g + 3]};
            put_f4(row - rd * kRows + (lane & 31), wn * WN + j * 32 + 8 * g + 4 * (lane >> 5), v);
          });
        }
      });
      lds_barrier();
      float* C = reinterpret_cast<float*>(b ? p.C1 : p.C0) + (int64_t)e * p.sCe;
      store_round(C, rd * kRows);
    });
  } else {
    // direct 32x32 result: lane holds column (lane % 32), rows 8 (v/4) + 4 (lane/32) + v%4
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = n0 + wn * WN + j * 32 + (lane & 31);
        if (c >= p.N) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const float v1 = DUAL ? acc[NB - 1][i][j][v] : 0.f;
          if constexpr (KGROUP) {
            if (m0 + r < p.M) epilogue<EPI, true, DUAL>(p, e, m0 + r, c, acc[0][i][j][v], v1);
          } else {
            if (r < valid) epilogue<EPI, true, DUAL>(p, e, row0 + r, c, acc[0][i][j][v], v1);
          }
        }
      }
  }
}

// ------------------------------------------------ one wavefront per SIMD --
// Four wavefronts (2 x 2) over the same 256 x 256 tile, each owning 128 x 128
// (4 x 4 MFMA blocks, or 4 x 2 per operand for the dual-B products): 256
// fp32 accumulators per lane in the accumulation registers, which takes the
// whole register file of a SIMD (one wavefront per SIMD) and does twice the
// MFMA work per LDS byte of the eight-wavefront form.  Operand tiles arrive
// in LDS by direct loads (no staging registers, no LDS store instructions)
// into two 64-KB stages, one LDS object each.  A K step is four K16 slices,
// each in a pinned issue order (MFMA, then the next slice's fragment read,
// then possibly one direct load); the second half of the next step's loads
// goes out in slice 0, the barrier follows slice 2 once this wavefront's
// loads of the next step have landed, and slice 3 sends the first half of
// the loads of the step after next into the stage just finished.  The MFMA
// takes the B fragment as its first operand, so each lane ends with four
// consecutive output columns per register group and the epilogue writes
// 8- or 16-byte pieces.
constexpr int kThreads4 = 256;

template <int BM, int BN, bool A_KC, bool B_KC, bool DUAL, bool TWOSEG, bool KGROUP, int EPI>
__global__ __launch_bounds__(kThreads4) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_w4_kernel(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int WM = BM / 2, WN = BN / 2;      // wavefront tile (per B operand)
  constexpr int MI = WM / 32, NJ = WN / 32;    // 32x32 MFMA blocks per wavefront
  constexpr int kTileA = BM * kBK * 2, kTileB = BN * kBK * 2;
  constexpr int kStage = kTileA + NB * kTileB;
  // every output kind here leaves through the LDS-staged epilogue, which
  // takes the transposed MFMA result (four consecutive columns per lane)
  static_assert(EPI != EPI_F32_ACC, "accumulating weight gradients use the eight-wavefront form");
  constexpr bool kSwapAB = true;
  // one LDS object per stage: the compiler can then tell that direct loads
  // into one stage never alias fragment reads of the other, and does not make
  // those reads wait for the loads
  __shared__ __attribute__((aligned(1024))) char stage0[kStage];
  __shared__ __attribute__((aligned(1024))) char stage1[kStage];
  // the third buffer of the B operand (the first two follow the A tiles in
  // stage0 and stage1): 160 KB in all, the whole LDS of a compute unit
  __shared__ __attribute__((aligned(1024))) char stage2[NB * kTileB];
  static_assert(2 * kStage + NB * kTileB <= 160 * 1024, "LDS of one compute unit");

  // products with a plain store epilogue split the tiles of a partial last
  // wave along K (fp32 partial tiles, summed by tail_reduce_kernel)
  constexpr bool kSplit = !KGROUP && EPI == EPI_STORE;
  int e, valid, m0 = 0, n0, part = -1, item = 0, nparts = 1;
  int64_t row0;
  if constexpr (KGROUP) {
    if (!tile_of<KGROUP, BM, BN, false, KGROUP && DUAL>(p, blockIdx.x, e, row0, valid, m0, n0))
      return;
  } else {
    const int nks = p.K / kBK, nkt = TWOSEG ? 2 * nks : nks;
    if (!mtile_split<BM, BN, kSplit>(p, blockIdx.x, (nkt + 1) & ~1, e, row0, valid, n0, part, item,
                                     nparts))
      return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  // 32-row block of the tile that the wavefront's row block i is.  M-grouped
  // tiles interleave the two wavefront rows (blocks wm, wm + 2, ...), and an
  // expert's last, partial tile runs MFMAs only over the blocks that hold
  // valid rows (mi_act per wavefront): with 171 rows both wavefront rows
  // take 3 blocks where contiguous halves would give one of them 4.  The
  // K-grouped tiles (M is not rows there) keep contiguous halves, all active.
  auto blk = [&](int i) { return KGROUP ? wm * MI + i : 2 * i + wm; };
  int mi_act = MI;
  if constexpr (!KGROUP)
    mi_act = __builtin_amdgcn_readfirstlane(min(MI, max(0, ((valid + 31) / 32 - wm + 1) / 2)));

  // operand bases (A segments, B operands) and their byte ranges
  const uint16_t* a_ptr[TWOSEG ? 2 : 1];
  const uint16_t* b_ptr[(DUAL || TWOSEG) ? 2 : 1];
  uint32_t a_bytes, b_bytes;
  int a_base, b_base, nk;
  const int nk_seg = KGROUP ? 0 : p.K / kBK;
  if constexpr (KGROUP) {
    if (valid == 0) {
      if (EPI != EPI_F32_ACC) {
        for (int i = tid; i < BM * BN; i += kThreads4) {
          const int r = i / BN, c = i % BN;
          if (m0 + r < p.M && n0 + c < p.N) epilogue<EPI, true, DUAL>(p, e, m0 + r, n0 + c, 0.f, 0.f);
        }
      }
      return;
    }
    a_ptr[0] = reinterpret_cast<const uint16_t*>(p.A0) + row0 * p.lda;
    b_ptr[0] = reinterpret_cast<const uint16_t*>(p.B0) + row0 * p.ldb;
    if constexpr (DUAL) b_ptr[1] = reinterpret_cast<const uint16_t*>(p.B1) + row0 * p.ldb;
    a_bytes = (uint32_t)((int64_t)valid * p.lda * 2);
    b_bytes = (uint32_t)((int64_t)valid * p.ldb * 2);
    a_base = m0;
    b_base = n0;
    nk = (valid + kBK - 1) / kBK;
  } else {
    a_ptr[0] = reinterpret_cast<const uint16_t*>(p.A0) + row0 * p.lda;
    if constexpr (TWOSEG) a_ptr[1] = reinterpret_cast<const uint16_t*>(p.A1) + row0 * p.lda;
    b_ptr[0] = reinterpret_cast<const uint16_t*>(p.B0) + (int64_t)e * p.sBe;
    if constexpr (DUAL || TWOSEG) b_ptr[1] = reinterpret_cast<const uint16_t*>(p.B1) + (int64_t)e * p.sBe;
    a_bytes = (uint32_t)((int64_t)valid * p.lda * 2);
    b_bytes = (uint32_t)((int64_t)p.N * p.K * 2);
    a_base = 0;
    b_base = n0;
    nk = TWOSEG ? 2 * nk_seg : nk_seg;
  }

  DmaOperand<A_KC, BM, 1, 4> da;
  DmaOperand<B_KC, BN, NB, 4> db;
  da.init(p.lda, a_base, w, lane);
  db.init(p.ldb, b_base, w, lane);
  // descriptors of K step kt (scalar work)
  auto step_rsrc = [&](int kt, u32x4 (&ra)[1], u32x4 (&rb)[NB]) {
    int seg = 0, k0 = kt * kBK;
    if constexpr (TWOSEG) {
      seg = kt >= nk_seg ? 1 : 0;
      k0 = (kt - seg * nk_seg) * kBK;
    }
    const uint16_t* const pa[1] = {seg ? a_ptr[TWOSEG ? 1 : 0] : a_ptr[0]};
    da.rsrc_for(pa, a_bytes, p.lda, k0, ra);
    if constexpr (DUAL) {
      db.rsrc_for(b_ptr, b_bytes, p.ldb, k0, rb);
    } else {
      const uint16_t* const pb[1] = {seg ? b_ptr[(DUAL || TWOSEG) ? 1 : 0] : b_ptr[0]};
      db.rsrc_for(pb, b_bytes, p.ldb, k0, rb);
    }
  };
  constexpr int kDmaA = DmaOperand<A_KC, BM, 1, 4>::kPer;
  constexpr int kDmaB = DmaOperand<B_KC, BN, NB, 4>::kPer;
  f32x16 acc[NB][MI][NJ];
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][i][j][v] = 0.f;

  u32x4 af0[MI], bf0[NB][NJ], af1[MI], bf1[NB][NJ];
  // fragment f of slice kk: f < MI an A fragment, else B fragment (q, j)
  // per-lane LDS bases of the transposed fragments (loop invariant)
  uint32_t abase[MI], bbase[NJ];
#pragma unroll
  for (int f = 0; f < MI; ++f) abase[f] = frag_km_base<BM>(blk(f) * 32, lane);
#pragma unroll
  for (int f = 0; f < NJ; ++f) bbase[f] = frag_km_base<BN>(wn * WN + f * 32, lane);
  // sa: the A tile of the step, sb: its B buffer; act: the row blocks with
  // MFMA work (fragments of the others are not read)
  auto read_frag = [&](const char* sa, const char* sb, int kk, int f, u32x4 (&af)[MI],
                       u32x4 (&bfr)[NB][NJ], int act) {
    if (f < MI) {
      if (KGROUP || f < act) {
        if constexpr (A_KC) af[f] = frag_kc(sa, blk(f) * 32, kk, lane);
        else af[f] = frag_km_at<BM>(sa, abase[f], kk);
      }
    } else {
      const int q = (f - MI) / NJ, j = (f - MI) % NJ;
      const char* t = sb + q * kTileB;
      if constexpr (B_KC) bfr[q][j] = frag_kc(t, wn * WN + j * 32, kk, lane);
      else bfr[q][j] = frag_km_at<BN>(t, bbase[j], kk);
    }
  };
  constexpr int kMfma = MI * NB * NJ;
  constexpr int kFrag = MI + NB * NJ;
  // B loads of a step spread over slices 0-2 (kB0, kB1, the rest), A loads
  // over slice 3
  constexpr int kB0 = (kDmaB + 2) / 3, kB1 = (kDmaB + 1) / 3, kB2 = kDmaB - kB0 - kB1;
  static_assert(kFrag <= kMfma && kDmaA <= kMfma && kB0 <= kMfma, "slice interleave");

  // The SwiGLU backward epilogue's first 128 rows of h1 and h3 (256 columns,
  // 512-byte rows) as four 64-row halves of 32 KB: instruction i of this
  // wavefront fills 1-KB slot 8 w + i of a half, staged rows 2 j and 2 j + 1
  // with 16-byte chunk c of row q at c ^ (q & 15) (the staged-tile layout).
  const int hl = lane >> 5, slot = lane & 31;
  auto epi_issue = [&](int i, const u32x4& rs, char* ds) {
    const int j = w * 8 + i, q = 2 * j + hl;
    const uint32_t voff = ((uint32_t)q * (uint32_t)p.ldc + 8u * (uint32_t)(slot ^ (q & 15))) * 2u;
    dma16(rs, voff, ds + j * 1024);
  };
  // One K16 slice in a pinned issue order: MFMA t on the current fragments,
  // then fragment t of the next slice (from A tile ra_t and B buffer rb_t),
  // then, spread evenly over the slice's MFMAs, its n direct loads:
  // instructions d0 .. d0+n-1 of operand OP (0: A, 1: B) of the step whose
  // descriptors are rs, into LDS at ds.  The address unit accepts one such
  // 1-KB load about every 16 cycles, so a step's loads are not bunched.
  auto slice = [&](const u32x4 (&afc)[MI], const u32x4 (&bfc)[NB][NJ], const char* ra_t,
                   const char* rb_t, int rd_kk, u32x4 (&afn)[MI], u32x4 (&bfn)[NB][NJ],
                   const u32x4* rs, char* ds, int d0, auto act_tag, auto op_tag, auto n_tag) {
    constexpr int OP = decltype(op_tag)::value, N = decltype(n_tag)::value;
    constexpr int act = decltype(act_tag)::value;
#pragma unroll
    for (int t = 0; t < kMfma; ++t) {
      const int i = t / (NB * NJ), q = (t / NJ) % NB, j = t % NJ;
      if (i < act)
        acc[q][i][j] = kSwapAB
            ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bfc[q][j]),
                                                      __builtin_bit_cast(bf16x8, afc[i]),
                                                      acc[q][i][j], 0, 0, 0)
            : __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, afc[i]),
                                                      __builtin_bit_cast(bf16x8, bfc[q][j]),
                                                      acc[q][i][j], 0, 0, 0);
      // (no null test on the tile pointers: LDS address 0 is a valid
      // address, so the compiler would keep it as a branch between MFMAs)
      if (t < kFrag) read_frag(ra_t, rb_t, rd_kk, t, afn, bfn, act);
#pragma unroll
      for (int n = 0; n < N; ++n)
        if (t == n * kMfma / N) {
          if constexpr (OP == 0) {
            const u32x4 r1[1] = {rs[0]};
            da.issue_one(d0 + n, r1, ds, w);
          } else if constexpr (OP == 2) {
            epi_issue(d0 + n, rs[0], ds);
          } else {
            u32x4 rn[NB];
#pragma unroll
            for (int o = 0; o < NB; ++o) rn[o] = rs[o];
            db.issue_one(d0 + n, rn, ds, w);
          }
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using IA = std::integral_constant<int, 0>;
  using IB = std::integral_constant<int, 1>;
  using NA = std::integral_constant<int, kDmaA>;
  using N0 = std::integral_constant<int, kB0>;
  using N1 = std::integral_constant<int, kB1>;
  using N2 = std::integral_constant<int, kB2>;

  // The A tiles (activation rows, mostly L2 hits) take two stages, the B
  // tiles (the expert weights, streamed from HBM when an expert has few rows)
  // three buffers, so B is fetched two steps ahead.  Step kt (local index i,
  // A tile in stage CUR, B in buffer i % 3; A(kt+1) and B(kt+1) in flight):
  //   slices 0-2  B(kt+2) into buffer (i+2) % 3, last read in step kt-1
  //   barrier     after everything but those loads landed (vmcnt(kDmaB):
  //               loads complete in issue order), i.e. A(kt+1), B(kt+1)
  //   slice 3     A(kt+2) into stage CUR, which every wavefront finished
  //               reading before the barrier
  // Loads past the last step stay inside the descriptors' ranges and go to
  // tiles that are not read again, so the loop has no tail copy; the step
  // count is rounded up to even for the two-stage unroll (K-grouped products
  // then run one step of zero rows when their row count needs an odd number).
  char* const bbuf0 = stage0 + kTileA;
  char* const bbuf1 = stage1 + kTileA;
  auto bsel = [&](int i) -> char* { return i == 0 ? bbuf0 : (i == 1 ? bbuf1 : stage2); };
  auto step = [&](int kt, int i3, auto cur_tag, auto act) {
    constexpr int CUR = decltype(cur_tag)::value;
    char* cur = CUR ? stage1 : stage0;
    char* nxt = CUR ? stage0 : stage1;
    char* bc = bsel(i3);
    char* bn = bsel(i3 == 2 ? 0 : i3 + 1);
    char* bnn = bsel(i3 == 0 ? 2 : i3 - 1);
    u32x4 ra2[1], rb2[NB];
    step_rsrc(kt + 2, ra2, rb2);
    slice(af0, bf0, cur, bc, 1, af1, bf1, rb2, bnn, 0, act, IB{}, N0{});
    slice(af1, bf1, cur, bc, 2, af0, bf0, rb2, bnn, kB0, act, IB{}, N1{});
    slice(af0, bf0, cur, bc, 3, af1, bf1, rb2, bnn, kB0 + kB1, act, IB{}, N2{});
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kDmaB) : "memory");
    slice(af1, bf1, nxt, bn, 0, af0, bf0, ra2, cur, 0, act, IA{}, NA{});
  };
  // The last two steps of a tile would load operand tiles for steps past
  // the end, never read; in the SwiGLU backward product they load the
  // epilogue's first h1 rows (into the B buffer each step frees, in the
  // B loads' slots) and h3 rows (into its A stage), the same count of
  // 1-KB loads at the same points, so the waits and the buffer protocol
  // are those of any other step.  The epilogue's first phase then finds its
  // inputs in LDS instead of waiting for them after the K loop (measured:
  // dA 1885 -> 1836 us at 8 experts x 2048 rows, H 4096, H' 14336; within
  // noise at 384 experts, where the product is bound by HBM).
  constexpr bool kEpiFetch = EPI == EPI_SWIGLU_BWD;
  static_assert(!kEpiFetch || (kDmaA == 8 && kDmaB == 8 && BN == 256), "h1/h3 halves in the load slots");
  using IE = std::integral_constant<int, 2>;
  auto step_epi = [&](int i3, auto cur_tag, auto act, const u32x4 (&rz)[1], const u32x4 (&ru)[1]) {
    constexpr int CUR = decltype(cur_tag)::value;
    char* cur = CUR ? stage1 : stage0;
    char* nxt = CUR ? stage0 : stage1;
    char* bc = bsel(i3);
    char* bn = bsel(i3 == 2 ? 0 : i3 + 1);
    char* bnn = bsel(i3 == 0 ? 2 : i3 - 1);
    slice(af0, bf0, cur, bc, 1, af1, bf1, rz, bnn, 0, act, IE{}, N0{});
    slice(af1, bf1, cur, bc, 2, af0, bf0, rz, bnn, kB0, act, IE{}, N1{});
    slice(af0, bf0, cur, bc, 3, af1, bf1, rz, bnn, kB0 + kB1, act, IE{}, N2{});
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kDmaB) : "memory");
    slice(af1, bf1, nxt, bn, 0, af0, bf0, ru, cur, 0, act, IE{}, NA{});
  };

  // K steps [k_lo, k_end) of this block: all of them, or one part of a split
  // tile (even boundaries, so the two-stage unroll holds)
  const int nk2 = (nk + 1) & ~1;
  int k_lo = 0, k_end = nk2;
  if constexpr (kSplit) {
    if (part >= 0) {
      const int pairs = nk2 >> 1;
      k_lo = 2 * (part * pairs / nparts);
      k_end = 2 * ((part + 1) * pairs / nparts);
    }
  }
  {
    // A(k_lo), B(k_lo), then B(k_lo+1), A(k_lo+1) (left in flight)
    u32x4 ra[1], rb[NB];
    step_rsrc(k_lo, ra, rb);
#pragma unroll
    for (int t = 0; t < kDmaA; ++t) da.issue_one(t, ra, stage0, w);
#pragma unroll
    for (int t = 0; t < kDmaB; ++t) db.issue_one(t, rb, bbuf0, w);
    step_rsrc(k_lo + 1, ra, rb);
#pragma unroll
    for (int t = 0; t < kDmaB; ++t) db.issue_one(t, rb, bbuf1, w);
#pragma unroll
    for (int t = 0; t < kDmaA; ++t) da.issue_one(t, ra, stage1, w);
  }
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kDmaA + kDmaB) : "memory");
#pragma unroll
  for (int f = 0; f < kFrag; ++f) read_frag(stage0, bbuf0, 0, f, af0, bf0, mi_act);
  // one copy of the K loop per active row-block count, without branches
  // between its MFMAs (a wavefront takes the copy of its own count; every
  // copy runs the same loads and barriers)
  // descriptors of the epilogue's h1 (rz) and h3 (ru) rows 0-63 and 64-127
  // (rows past the tile's valid ones and columns past N read zeros), and the
  // B buffers that the two h1 halves land in
  u32x4 rz[2][1], ru[2][1];
  char* ez[2] = {stage2, stage2};
  if constexpr (kEpiFetch) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t rows_left = (int64_t)valid - 64 * h;
      const int64_t lim = rows_left > 0 ? ((rows_left - 1) * p.ldc + (p.N - n0)) * 2 : 0;
      const int64_t off = ((row0 + 64 * h) * p.ldc + n0) * 2;
      rz[h][0] = rsrc_words(reinterpret_cast<const char*>(p.X0) + off, (uint32_t)lim);
      ru[h][0] = rsrc_words(reinterpret_cast<const char*>(p.X1) + off, (uint32_t)lim);
    }
    const int i3a = (k_end - 2 - k_lo) % 3, i3b = i3a == 2 ? 0 : i3a + 1;
    ez[0] = bsel(i3a == 0 ? 2 : i3a - 1);
    ez[1] = bsel(i3b == 0 ? 2 : i3b - 1);
  }
  auto kloop = [&](auto act) {
    int i3 = 0;
    const int k_main = kEpiFetch ? k_end - 2 : k_end;
    for (int kt = k_lo; kt < k_main; kt += 2) {
      step(kt, i3, I0{}, act);
      i3 = i3 == 2 ? 0 : i3 + 1;
      step(kt + 1, i3, I1{}, act);
      i3 = i3 == 2 ? 0 : i3 + 1;
    }
    if constexpr (kEpiFetch) {
      step_epi(i3, I0{}, act, rz[0], ru[0]);
      i3 = i3 == 2 ? 0 : i3 + 1;
      step_epi(i3, I1{}, act, rz[1], ru[1]);
    }
  };
  if (KGROUP || mi_act == MI) {
    kloop(std::integral_constant<int, MI>{});
  } else if constexpr (!KGROUP && MI == 4) {
    if (mi_act == 3) kloop(std::integral_constant<int, 3>{});
    else if (mi_act == 2) kloop(std::integral_constant<int, 2>{});
    else if (mi_act == 1) kloop(std::integral_constant<int, 1>{});
    else kloop(std::integral_constant<int, 0>{});
  }
  // no direct load may still be writing LDS when the block exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // With the B fragment as the MFMA's first operand the 32x32 result is
  // transposed: lane l holds row (l % 32) of the block and, for v = 4g + t,
  // column 8 g + 4 (l / 32) + t, i.e. four consecutive columns per g.
  // Written straight to memory, one such store instruction touches 32 rows
  // with 16 bytes each; the bf16 outputs are instead staged through the two
  // (now free) 64-KB LDS stages and leave as whole rows, 16 bytes a lane.
  if constexpr (kSplit) {
    if (part >= 0) {
      // one K part of a split tile: the fp32 accumulators in fragment order
      // (each store instruction writes 1 KB contiguous)
      f32x4* dst = reinterpret_cast<f32x4*>(p.part) + (size_t)item * (BM * BN / 4);
      StaticFor<0, MI * NJ * 4>::run([&](auto tag) {
        constexpr int x = decltype(tag)::value, i = x / (NJ * 4), j = (x / 4) % NJ, g = x % 4;
        dst[(((w * MI + i) * NJ + j) * 4 + g) * 64 + lane] =
            f32x4{acc[0][i][j][4 * g], acc[0][i][j][4 * g + 1], acc[0][i][j][4 * g + 2],
                  acc[0][i][j][4 * g + 3]};
      });
      return;
    }
  }
  if constexpr (kSwapAB) {
    static_assert(!KGROUP || EPI == EPI_F32, "staged epilogue kinds");
    // every direct load has landed and every wavefront is done with the stages
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // A staged tile: rows of BN bf16 (RS bytes), 16-byte chunk c of row r at
    // c ^ (r & 15).  A transposed piece write (32 rows, same chunk) then hits
    // every bank group twice, and a row read hits each once per 16 chunks.
    constexpr int RS = BN * 2, LPR = BN / 8, RPI = 64 / LPR;
    auto put4 = [&](char* st, int r, int c, const float (&v)[4]) {
      const uint32_t o = (uint32_t)r * RS + ((uint32_t)((c >> 3) ^ (r & 15)) << 4) + ((c >> 2) & 1) * 8;
      u32x2 w2;
      w2[0] = pack_bf16x2(v[0], v[1]);
      w2[1] = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<u32x2*>(st + o) = w2;
    };
    auto get4 = [&](const char* st, int r, int c, float (&v)[4]) {
      const uint32_t o = (uint32_t)r * RS + ((uint32_t)((c >> 3) ^ (r & 15)) << 4) + ((c >> 2) & 1) * 8;
      const u32x2 w2 = *reinterpret_cast<const u32x2*>(st + o);
      v[0] = bf16_lo(w2[0]); v[1] = bf16_hi(w2[0]); v[2] = bf16_lo(w2[1]); v[3] = bf16_hi(w2[1]);
    };
    // NR staged rows -> memory; staged row q is tile row
    // rbase + q + (q / SEG) * GAP (runs of SEG rows, GAP rows apart).  Each
    // instruction of the block covers RPI whole rows (kPass rows a pass of
    // the four wavefronts); lane (c, q0) stores chunk c of staged rows
    // q0, q0 + kPass, ... through one row pointer, the row offsets being
    // compile-time multiples of ldc.
    auto store_rows = [&](const char* st, auto nr_tag, void* C, int rbase, auto seg_tag, auto gap_tag) {
      constexpr int NR = decltype(nr_tag)::value, SEG = decltype(seg_tag)::value,
                    GAP = decltype(gap_tag)::value, kPass = 4 * RPI;
      static_assert(NR % kPass == 0 && SEG % kPass == 0, "staged row passes");
      const int c = lane % LPR, col = n0 + 8 * c, q0 = w * RPI + lane / LPR;
      if (col >= p.N) return;
      const int left = valid - (rbase + q0);
      uint16_t* dst = reinterpret_cast<uint16_t*>(C) + (row0 + rbase + q0) * p.ldc + col;
      const char* src = st + (uint32_t)q0 * RS;
#pragma unroll
      for (int it = 0; it < NR / kPass; ++it) {
        const int qd = it * kPass, rd = qd + (qd / SEG) * GAP;
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + qd * RS + ((uint32_t)(c ^ ((q0 + qd) & 15)) << 4));
        if (rd < left) {
          // non-temporal, except the forward SwiGLU outputs, which the next
          // product reads at once (measured: down, dA -5%; up +2.5% if NT)
          u32x4* d = reinterpret_cast<u32x4*>(dst + (int64_t)rd * p.ldc);
          if constexpr (EPI == EPI_SWIGLU_FWD) *d = v;
          else __builtin_nontemporal_store(v, d);
        }
      }
    };
    using R128 = std::integral_constant<int, 128>;
    using R256 = std::integral_constant<int, 256>;
    using R0 = std::integral_constant<int, 0>;

    if constexpr (EPI == EPI_F32) {
      // fp32 weight gradient of expert e (K-grouped): rows of BN floats
      // (RF bytes, 16-byte chunk c of row r at c ^ (r & 15)), non-temporal
      // whole-row stores.  One output of 256 rows x 128 columns fills both
      // stages (rows 0-127 and 128-255); a 256-column output goes in two
      // halves, one per wavefront row.
      constexpr int RF = BN * 4, LPRF = BN / 4, RPIF = 64 / LPRF;
      constexpr int kHalfRows = 64 * 1024 / RF;        // staged rows per stage
      constexpr int kRound = 2 * kHalfRows;            // staged rows per round
      static_assert(kRound == 128 || kRound == 256, "fp32 staging");
      float* gbase = reinterpret_cast<float*>(p.C0) + (int64_t)e * p.sCe;
      auto put_f4 = [&](int q, int c, const float (&v)[4]) {
        char* st = q < kHalfRows ? stage0 : stage1;
        const int ql = q < kHalfRows ? q : q - kHalfRows;
        const uint32_t o = (uint32_t)ql * RF + ((uint32_t)((c >> 2) ^ (ql & 15)) << 4);
        *reinterpret_cast<f32x4*>(st + o) = f32x4{v[0], v[1], v[2], v[3]};
      };
      auto store_round = [&](float* C, int rbase) __attribute__((always_inline)) {
        // lane (c, q0) stores chunk c of staged rows q0, q0 + kPass, ...
        // through one row pointer advanced by kPass rows
        constexpr int kPass = 4 * RPIF;
        static_assert(kHalfRows % kPass == 0, "staged row passes");
        const int c = lane % LPRF, col = n0 + 4 * c, q0 = w * RPIF + lane / LPRF;
        if (col >= p.N) return;
        const int left = p.M - (m0 + rbase + q0);
        float* dst = C + (int64_t)(m0 + rbase + q0) * p.ldc + col;
        const int64_t step = (int64_t)kPass * p.ldc;
#pragma unroll
        for (int it = 0; it < kRound / kPass; ++it) {
          const int qd = it * kPass;
          const char* st = qd < kHalfRows ? stage0 : stage1;
          const int ql = q0 + (qd < kHalfRows ? qd : qd - kHalfRows);
          const f32x4 v = *reinterpret_cast<const f32x4*>(st + (uint32_t)ql * RF + ((uint32_t)(c ^ (ql & 15)) << 4));
          if (qd < left) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
          dst += step;
        }
      };
      if constexpr (kRound == 256) {
        // dual: each output tile is one round written by all four wavefronts
        static_assert(DUAL, "256-row rounds hold a 128-column output");
        StaticFor<0, NB>::run([&](auto b_tag) {
          constexpr int b = decltype(b_tag)::value;
          if constexpr (b > 0) __syncthreads();
          StaticFor<0, MI * NJ * 4>::run([&](auto tag) {
            constexpr int x = decltype(tag)::value, i = x / (NJ * 4), j = (x / 4) % NJ, g = x % 4;
            const float v[4] = {acc[b][i][j][4 * g], acc[b][i][j][4 * g + 1], acc[b][i][j][4 * g + 2],
                                acc[b][i][j][4 * g + 3]};
            put_f4(wm * WM + i * 32 + (lane & 31), wn * WN + j * 32 + 8 * g + 4 * (lane >> 5), v);
          });
          __syncthreads();
          store_round((b ? reinterpret_cast<float*>(p.C1) + (int64_t)e * p.sCe : gbase), 0);
        });
      } else {
        // one output of 256 columns: wavefront row hh stages its 128 rows
        static_assert(!DUAL && BM == 256, "128-row rounds hold half a 256-column output");
        StaticFor<0, 2>::run([&](auto h_tag) {
          constexpr int hh = decltype(h_tag)::value;
          if constexpr (hh > 0) __syncthreads();
          if (wm == hh) {
            StaticFor<0, MI * NJ * 4>::run([&](auto tag) {
              constexpr int x = decltype(tag)::value, i = x / (NJ * 4), j = (x / 4) % NJ, g = x % 4;
              const float v[4] = {acc[0][i][j][4 * g], acc[0][i][j][4 * g + 1], acc[0][i][j][4 * g + 2],
                                  acc[0][i][j][4 * g + 3]};
              put_f4(i * 32 + (lane & 31), wn * WN + j * 32 + 8 * g + 4 * (lane >> 5), v);
            });
          }
          __syncthreads();
          store_round(gbase, hh * 128);
        });
      }
    } else if constexpr (EPI == EPI_STORE) {
      // tile rows 0-127 in stage 0, 128-255 in stage 1: row block 2i + wm of
      // the tile goes to stage i / 2
      static_assert(NB == 1 && BM == 256 && MI == 4, "store epilogue tile");
      StaticFor<0, MI * NJ * 4>::run([&](auto tag) {
        constexpr int x = decltype(tag)::value, i = x / (NJ * 4), j = (x / 4) % NJ, g = x % 4;
        if (i < mi_act) {
          const float v[4] = {acc[0][i][j][4 * g], acc[0][i][j][4 * g + 1], acc[0][i][j][4 * g + 2],
                              acc[0][i][j][4 * g + 3]};
          put4(i >= 2 ? stage1 : stage0, (2 * (i & 1) + wm) * 32 + (lane & 31),
               wn * WN + j * 32 + 8 * g + 4 * (lane >> 5), v);
        }
      });
      __syncthreads();
      store_rows(stage0, R128{}, p.C0, 0, R128{}, R0{});
      store_rows(stage1, R128{}, p.C0, 128, R128{}, R0{});
    } else if constexpr (EPI == EPI_SWIGLU_FWD) {
      // h1 in stage 0 and a = silu(h1) h3 in stage 1 (256 rows x 128 columns
      // each; a from the fp32 accumulators), then h3 in stage 0
      static_assert(NB == 2 && BM == 256 && BN == 128, "SwiGLU epilogue tile");
      StaticFor<0, MI * NJ * 4>::run([&](auto tag) {
        constexpr int x = decltype(tag)::value, i = x / (NJ * 4), j = (x / 4) % NJ, g = x % 4;
        if (i < mi_act) {
          const int r = blk(i) * 32 + (lane & 31), c = wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);
          float v0[4], a[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            v0[t] = acc[0][i][j][4 * g + t];
            a[t] = silu_f(v0[t]) * acc[1][i][j][4 * g + t];
          }
          put4(stage0, r, c, v0);
          put4(stage1, r, c, a);
        }
      });
      __syncthreads();
      // a null output (h1, h3 under recompute, or a when recomputing) is skipped
      if (p.C0) store_rows(stage0, R256{}, p.C0, 0, R256{}, R0{});
      if (p.C2) store_rows(stage1, R256{}, p.C2, 0, R256{}, R0{});
      if (p.C1) {
        __syncthreads();
        StaticFor<0, MI * NJ * 4>::run([&](auto tag) {
          constexpr int x = decltype(tag)::value, i = x / (NJ * 4), j = (x / 4) % NJ, g = x % 4;
          if (i < mi_act) {
            const int r = blk(i) * 32 + (lane & 31), c = wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);
            const float v1[4] = {acc[1][i][j][4 * g], acc[1][i][j][4 * g + 1],
                                 acc[1][i][j][4 * g + 2], acc[1][i][j][4 * g + 3]};
            put4(stage0, r, c, v1);
          }
        });
        __syncthreads();
        store_rows(stage0, R256{}, p.C1, 0, R256{}, R0{});
      }
    } else {
      // SwiGLU backward: two phases of 128 tile rows, phase ph the tile rows
      // 128 ph .. 128 ph + 127 (row blocks 2 ph and 2 ph + 1 of both
      // wavefront rows, interleaved).  The first phase's h1 and h3 rows
      // arrived during the K loop's last two steps, in 64-row halves (h1 in
      // the B buffers ez[], h3 in the A parts of stages 0 and 1); the second
      // phase's come into stage 0 (h1) and stage 1 (h3) by direct loads (no
      // staging registers).  dh1 and dh3 overwrite them in place and leave
      // as whole rows.  A tile of at most 128 valid rows has no second phase.
      static_assert(EPI == EPI_SWIGLU_BWD && NB == 1 && BM == 256 && BN == 256, "dA epilogue tile");
      static_assert(MI == 4 && RS == 512, "two 128-row phases of 256 columns");
      // staged row q of phase 1 is tile row 128 + q; wavefront w loads
      // 32 KB of one matrix: instruction u covers staged rows
      // 2 (32 (w & 1) + u) and the next one
      const int mat = w >> 1;
      const char* xbase = reinterpret_cast<const char*>(mat ? p.X1 : p.X0) +
                          ((int64_t)row0 * p.ldc + n0) * 2;
      char* dstage = mat ? stage1 : stage0;
      auto dma_phase = [&](int ph) {
        // rows past the tile's valid ones and columns past N read zeros
        const int64_t rows_left = (int64_t)valid - 128 * ph;
        const int64_t lim = rows_left > 0 ? ((rows_left - 1) * p.ldc + (p.N - n0)) * 2 : 0;
        const u32x4 rs = rsrc_words(xbase + (int64_t)128 * ph * p.ldc * 2, (uint32_t)lim);
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          const int j = 32 * (w & 1) + u, q = 2 * j + hl;  // q: tile row minus 128 ph
          const uint32_t voff = ((uint32_t)q * (uint32_t)p.ldc + 8u * (uint32_t)(slot ^ (q & 15))) * 2u;
          dma16(rs, voff, dstage + j * 1024);
        }
      };
      using R64 = std::integral_constant<int, 64>;
      StaticFor<0, 2>::run([&](auto ph_tag) {
        constexpr int ph = decltype(ph_tag)::value;
        if (ph == 1 && valid <= 128) return;  // uniform over the block
        // this wavefront's loads (and, from the second phase on, its stores
        // of the previous one) are done; after the barrier everyone's are
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        StaticFor<0, 2 * NJ * 4>::run([&](auto x_tag) {
          constexpr int x = decltype(x_tag)::value, ib = x / (NJ * 4), j = (x / 4) % NJ, g = x % 4;
          constexpr int i = 2 * ph + ib;
          if (i < mi_act) {
            // tile row block 2 i + wm = 4 ph + 2 ib + wm; in the first phase
            // half ib, row wm * 32 + lane % 32 of it
            const int q = ph == 0 ? wm * 32 + (lane & 31) : (2 * ib + wm) * 32 + (lane & 31);
            char* const sz = ph == 0 ? ez[ib] : stage0;
            char* const su = ph == 0 ? (ib ? stage1 : stage0) : stage1;
            const int c = wn * WN + j * 32 + 8 * g + 4 * (lane >> 5);
            float z[4], u[4], d1[4], d3[4];
            get4(sz, q, c, z);
            get4(su, q, c, u);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const float v = acc[0][i][j][4 * g + t];
              const float sg = sigmoid_f(z[t]);
              const float vs = v * sg;
              d3[t] = vs * z[t];
              d1[t] = vs * u[t] * (1.0f + z[t] - z[t] * sg);
            }
            put4(sz, q, c, d1);
            put4(su, q, c, d3);
          }
        });
        __syncthreads();
        if constexpr (ph == 0) {
          store_rows(ez[0], R64{}, p.C0, 0, R64{}, R0{});
          store_rows(ez[1], R64{}, p.C0, 64, R64{}, R0{});
          store_rows(stage0, R64{}, p.C1, 0, R64{}, R0{});
          store_rows(stage1, R64{}, p.C1, 64, R64{}, R0{});
        } else {
          store_rows(stage0, R128{}, p.C0, 128, R128{}, R0{});
          store_rows(stage1, R128{}, p.C1, 128, R128{}, R0{});
        }
        if constexpr (ph == 0) {
          if (valid > 128) {
            // every wavefront has read the stages for its stores
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            dma_phase(1);
          }
        }
      });
    }
  } else {
    // direct 32x32 result: lane holds column (lane % 32), rows 8 (v/4) + 4 (lane/32) + v%4
    StaticFor<0, MI * NJ>::run([&](auto ij_tag) {
      constexpr int i = decltype(ij_tag)::value / NJ, j = decltype(ij_tag)::value % NJ;
      const int c = n0 + wn * WN + j * 32 + (lane & 31);
      if (c < p.N) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = blk(i) * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const float v1 = DUAL ? acc[NB - 1][i][j][v] : 0.f;
          if constexpr (KGROUP) {
            if (m0 + r < p.M) epilogue<EPI, true, DUAL>(p, e, m0 + r, c, acc[0][i][j][v], v1);
          } else {
            if (r < valid) epilogue<EPI, true, DUAL>(p, e, row0 + r, c, acc[0][i][j][v], v1);
          }
        }
      }
    });
  }
#endif
}

// Sums the K parts of each split tile (in part order) and stores the bf16
// result.  Block (tile tt, 32-row group i); thread (w, lane) takes the
// accumulators that wavefront w, lane held in the GEMM: row
// 32 (2 i + w / 2) + lane % 32, columns (w % 2) * WN + 32 j + 8 g + 4 (lane / 32) + t.
template <int BM, int BN, bool TWOSEG>
__global__ __launch_bounds__(256) void tail_reduce_kernel(GemmArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NJ = WN / 32;
  const int nks = p.K / kBK, nkt = TWOSEG ? 2 * nks : nks;
  const SplitPlan sp = split_plan(p, (nkt + 1) & ~1);
  const int tt = blockIdx.x / MI, i = blockIdx.x % MI;
  if (sp.s < 2 || tt >= sp.rem) return;
  int mt, nt;
  mtile_of(sp.full + tt, p.ntiles[0], p.ntn, p.ntiles[1], mt, nt);
  const int2 tl = p.tiles[mt];
  const int64_t row0 = (int64_t)p.cu[tl.x] + tl.y;
  const int valid = min(BM, p.cu[tl.x + 1] - (int)row0);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  // row block 2 i + (w / 2) of the tile (the GEMM interleaves its wavefront rows)
  const int r = (2 * i + (w >> 1)) * 32 + (lane & 31);
  if (r >= valid) return;
  constexpr size_t kTile = BM * BN / 4;
  const f32x4* src = reinterpret_cast<const f32x4*>(p.part) + (size_t)tt * sp.s * kTile +
                     (size_t)((w * MI + i) * NJ * 4) * 64 + lane;
  // part by part, all NJ * 4 pieces of a part in flight together
  f32x4 a[NJ * 4];
#pragma unroll
  for (int x = 0; x < NJ * 4; ++x) a[x] = src[x * 64];
  for (int k = 1; k < sp.s; ++k) {
#pragma unroll
    for (int x = 0; x < NJ * 4; ++x) a[x] += src[k * kTile + x * 64];
  }
#pragma unroll
  for (int x = 0; x < NJ * 4; ++x) {
    const int j = x / 4, g = x % 4;
    const int col = nt * BN + (w & 1) * WN + j * 32 + 8 * g + 4 * (lane >> 5);
    const float v[4] = {a[x][0], a[x][1], a[x][2], a[x][3]};
    if (col < p.N) store4_bf16(p.C0, (row0 + r) * p.ldc + col, v);
  }
}

// ---------------------------------------------------------- fp32 kernel --
// M tile of kGemmBM rows x 32 columns; thread (tid % 32) owns a column,
// rows tid/32 + 8 i.  The K-grouped products (weight gradients) take 64-row
// tiles: their grid is E x (M / 64) x (N / 32), four times the blocks of
// 256-row tiles for the same work.
constexpr int kBMf = kGemmBM, kBNf = 32, kBMfK = 64;

template <bool A_KC, bool B_KC, bool DUAL, bool TWOSEG, bool KGROUP, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p) {
  constexpr int kBM = KGROUP ? kBMfK : kBMf;
  int e, valid, m0, n0;
  int64_t row0;
  if (!tile_of<KGROUP, kBM, kBNf>(p, blockIdx.x, e, row0, valid, m0, n0)) return;
  const int tid = threadIdx.x;
  const int col = n0 + (tid & 31);
  if (col >= p.N) return;
  const float* A0 = reinterpret_cast<const float*>(p.A0);
  const float* A1 = reinterpret_cast<const float*>(p.A1);
  const float* B0 = reinterpret_cast<const float*>(p.B0);
  const float* B1 = reinterpret_cast<const float*>(p.B1);
  // Every output is one fmaf chain in ascending k.  The loads do not depend
  // on the chain, so they are issued ahead of it: four k per 16-byte load
  // along a contiguous K (K, lda, ldb multiples of 128, pointers 16-byte
  // aligned), and in the K-grouped form four output rows per pass.
  if constexpr (KGROUP) {
    constexpr int kRows = 4;
    for (int i0 = 0; i0 < kBM / 8; i0 += kRows) {
      int rr[kRows];
      float acc0[kRows], acc1[kRows];
#pragma unroll
      for (int j = 0; j < kRows; ++j) {
        rr[j] = m0 + (tid >> 5) + 8 * (i0 + j);
        acc0[j] = acc1[j] = 0.f;
      }
      if (rr[0] >= p.M) break;  // rows ascend with i0 and j
      // C_e[rr, col] = sum over the expert's rows k of A[k, rr] * B[k, col];
      // rows past M read row M - 1 and are not stored
      for (int k = 0; k < valid; ++k) {
        const int64_t gr = row0 + k;
        const float b0 = B0[gr * p.ldb + col];
        const float b1 = DUAL ? B1[gr * p.ldb + col] : 0.f;
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
          const float a = A0[gr * p.lda + min(rr[j], p.M - 1)];
          acc0[j] = fmaf(a, b0, acc0[j]);
          if constexpr (DUAL) acc1[j] = fmaf(a, b1, acc1[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < kRows; ++j)
        if (rr[j] < p.M && (valid > 0 || EPI != EPI_F32_ACC))
          epilogue<EPI, false, DUAL>(p, e, rr[j], col, acc0[j], acc1[j]);
    }
  } else {
    static_assert(!(DUAL && B_KC), "the dual product reads row-major weights");
    for (int i = 0; i < kBM / 8; ++i) {
      const int r = (tid >> 5) + 8 * i;
      if (r >= valid) break;  // rows ascend with i
      const int64_t gr = row0 + r;
      float acc0 = 0.f, acc1 = 0.f;
      for (int seg = 0; seg < (TWOSEG ? 2 : 1); ++seg) {
        const float* arow = (seg ? A1 : A0) + gr * p.lda;
        const float* Bw = (seg ? B1 : B0) + (int64_t)e * p.sBe;
        const float* Bw1 = B1 + (int64_t)e * p.sBe;
        if constexpr (B_KC) {
          const float* brow = Bw + (int64_t)col * p.ldb;
#pragma unroll 4
          for (int k = 0; k < p.K; k += 4) {
            const float4 a4 = *reinterpret_cast<const float4*>(arow + k);
            const float4 b4 = *reinterpret_cast<const float4*>(brow + k);
            acc0 = fmaf(a4.x, b4.x, acc0);
            acc0 = fmaf(a4.y, b4.y, acc0);
            acc0 = fmaf(a4.z, b4.z, acc0);
            acc0 = fmaf(a4.w, b4.w, acc0);
          }
        } else {
#pragma unroll 4
          for (int k = 0; k < p.K; k += 4) {
            const float4 a4 = *reinterpret_cast<const float4*>(arow + k);
            const float* bk = Bw + (int64_t)k * p.ldb + col;
            acc0 = fmaf(a4.x, bk[0], acc0);
            acc0 = fmaf(a4.y, bk[p.ldb], acc0);
            acc0 = fmaf(a4.z, bk[2 * (int64_t)p.ldb], acc0);
            acc0 = fmaf(a4.w, bk[3 * (int64_t)p.ldb], acc0);
            if constexpr (DUAL) {
              const float* bk1 = Bw1 + (int64_t)k * p.ldb + col;
              acc1 = fmaf(a4.x, bk1[0], acc1);
              acc1 = fmaf(a4.y, bk1[p.ldb], acc1);
              acc1 = fmaf(a4.z, bk1[2 * (int64_t)p.ldb], acc1);
              acc1 = fmaf(a4.w, bk1[3 * (int64_t)p.ldb], acc1);
            }
          }
        }
      }
      epilogue<EPI, false, DUAL>(p, e, gr, col, acc0, acc1);
    }
  }
}

// ------------------------------------------------------------ tile table --
__device__ int block_exclusive_scan_1024_g(int v, int* sh, int* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int incl = sh[tid];
  *total = sh[1023];
  __syncthreads();
  return incl - v;
}

// The experts by descending row count (ties to the lower index): the M
// tiles of the M-grouped products are listed expert by expert in that
// order, and when eorder is given it is also the order in which the
// K-grouped products deal out experts.  Under skew the hot experts' tiles
// are the costly ones (full M tiles; long K loops); taken first, they
// overlap the many short tiles instead of trailing after them.
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ cu, int E,
                                                          int bm, int max_tiles,
                                                          int2* __restrict__ tiles,
                                                          int32_t* __restrict__ ntiles,
                                                          int32_t* __restrict__ eorder) {
  __shared__ int sh[1024];
  // order key of each expert: row count, then the lower index first (past
  // E: 0, below every expert); one unsigned compare orders two experts
  typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
  __shared__ __attribute__((aligned(16))) unsigned long long okey[1024];
  __shared__ int nt_at[1024];     // M tiles of the expert at each rank
  __shared__ int start_at[1024];  // its first slot in the table
  const int e = threadIdx.x;
  // A malformed cu (not monotone) yields no tiles for that expert rather than
  // a table overflow.
  const int c = e < E ? max(0, cu[e + 1] - cu[e]) : 0;
  const unsigned long long key =
      e < E ? ((unsigned long long)(uint32_t)c << 32) | (0xffffffffu - (uint32_t)e) : 0ull;
  okey[e] = key;
  const int nt = (c + bm - 1) / bm;
  if (e >= E) nt_at[e] = 0;  // the ranks of the experts are exactly 0 .. E-1
  __syncthreads();
  // rank = experts ahead of e (larger key); keys read two per 16-byte load
  // (every thread reads the same words: broadcast), eight loads in flight
  // per iteration.  Measured at 384 experts: the whole table 21 -> 15 us
  // against comparing counts and indices separately from 4-byte reads.
  int rank = 0;
  if (e < E) {
    const u64x2* k2 = reinterpret_cast<const u64x2*>(okey);
    for (int j2 = 0; j2 < (E + 15) / 16 * 8; j2 += 8) {
      u64x2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = k2[j2 + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) rank += (v[u].x > key ? 1 : 0) + (v[u].y > key ? 1 : 0);
    }
    nt_at[rank] = nt;
    if (eorder != nullptr) eorder[rank] = e;
  }
  __syncthreads();
  // M tiles listed expert by expert in that order (thread r scans rank r)
  int total;
  start_at[e] = block_exclusive_scan_1024_g(nt_at[e], sh, &total);
  __syncthreads();
  if (e < E) {
    const int start = start_at[rank];
    for (int t = 0; t < nt && start + t < max_tiles; ++t) tiles[start + t] = make_int2(e, t * bm);
  }
  // M tiles per group of the M-grouped products: 1 when no expert has more
  // than one tile; 2 when most experts with rows have one (a few hot ones
  // hold the rest); else 4
  const int multi = __syncthreads_count(e < E && nt > 1);
  const int single = __syncthreads_count(e < E && nt == 1);
  if (e == 0) {
    ntiles[0] = min(total, max_tiles);
    ntiles[1] = multi == 0 ? 0 : (single > multi ? 1 : 2);
  }
  if (eorder != nullptr) {
    // T: experts with more than twice the mean row count, rounded up so that
    // E - T is a multiple of 8 (the weight-gradient products split these
    // eight ways across the XCDs and deal the rest whole)
    const int64_t rows = E > 0 ? (int64_t)cu[E] - cu[0] : 0;
    const int hot = __syncthreads_count(e < E && (int64_t)c * E > 2 * rows);
    if (e == 0) eorder[E] = hot + ((E - hot) & 7);
  }
}

void launch_tile_table(const int32_t* cu, int E, const WsLayout& L, char* ws, bool expert_order,
                       hipStream_t s) {
  TimedLaunch tl("gemm_tile_table", s);
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, s, cu, E, L.bm, L.max_tiles,
                     reinterpret_cast<int2*>(ws + L.tiles), reinterpret_cast<int32_t*>(ws + L.ntiles),
                     expert_order ? reinterpret_cast<int32_t*>(ws + L.eorder) : nullptr);
}

// -------------------------------------------------------------- launches --
template <int BM, int BN, bool A_KC, bool B_KC, bool DUAL, bool TWOSEG, bool KGROUP, int EPI,
          bool W4 = true, int NS = 2>
static void gemm_launch(const char* name, GemmArgs p, int max_mtiles, bool bf16, hipStream_t s) {
  static_assert(KGROUP || BM == kGemmBM || (BM == kGemmBMFew && !W4),
                "M-grouped tiles follow the tile table");
  const int bm = bf16 ? BM : (KGROUP ? kBMfK : kBMf), bn = bf16 ? BN : kBNf;
  p.ntn = (p.N + bn - 1) / bn;
  int blocks;
  if (KGROUP) {
    p.mtn = (p.M + bm - 1) / bm;
    blocks = p.E * p.mtn * p.ntn;
  } else {
    // groups of four M tiles: enough blocks for either group size
    const int groups = (max_mtiles + 3) >> 2;
    blocks = (groups << 2) * p.ntn;
  }
  // a split last wave adds at most tail_cap blocks (its rem tiles become
  // s * rem parts, s * rem <= tail_cap)
  constexpr bool kSplit = !KGROUP && EPI == EPI_STORE;
  const bool split = kSplit && bf16 && W4 && p.part != nullptr && p.tail_cap > 0 && p.ncu > 0;
  if (kSplit && !split) p.ncu = 0;
  if (split) blocks += p.tail_cap;
  if (blocks <= 0) return;
  TimedLaunch tl(name, s);
  if (bf16) {
    constexpr int lds = NS * (BM * kBK * 2 + (DUAL ? 2 : 1) * BN * kBK * 2);
    static bool attr = false;
    if constexpr (W4 && EPI != EPI_F32_ACC) {
      // the one-wavefront-per-SIMD form; accumulating weight gradients keep
      // the eight-wavefront form (the old values they load do not fit one
      // SIMD's register file next to 256 accumulators)
      auto kern = gemm_bf16_w4_kernel<BM, BN, A_KC, B_KC, DUAL, TWOSEG, KGROUP, EPI>;
      hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads4), 0, s, p);
      if constexpr (kSplit) {
        // at most tail_cap / 2 split tiles (each has at least two parts)
        if (split)
          hipLaunchKernelGGL((tail_reduce_kernel<BM, BN, TWOSEG>), dim3(p.tail_cap / 2 * (BM / 64)),
                             dim3(256), 0, s, p);
      }
    } else {
      auto kern = gemm_bf16_kernel<BM, BN, A_KC, B_KC, DUAL, TWOSEG, KGROUP, EPI, NS>;
      // a failure stays the thread's last HIP error (so the entry point
      // reports it) and the next call tries again
      if (!attr)
        attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess;
      hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), lds, s, p);
    }
  } else {
    hipLaunchKernelGGL((gemm_f32_kernel<A_KC, B_KC, DUAL, TWOSEG, KGROUP, EPI>), dim3(blocks),
                       dim3(256), 0, s, p);
  }
}

// The weight-gradient products reduce over each expert's rows.  With many
// rows per expert (mean at least 512) they run long K loops and take the
// one-wavefront-per-SIMD form; with few, the K loop is a handful of steps
// and the eight-wavefront form (no even-step rounding, shorter per-tile
// set-up) is faster.  The host knows the mean without reading the counts.
// Measured at a mean of 512 rows: the MoD block's 16 experts 1.27 -> 1.14 ms
// (dW1/dW3) and 0.63 -> 0.58 ms (dW2) in the one-wavefront form; 64
// Zipf-skewed experts +4% and -4.5%.
static bool many_rows(int64_t R, int E) { return R >= (int64_t)512 * E; }

// Compute units of the current device (cached per device; 0 if unknown,
// which turns the last-wave split off).
static int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cache[dev] = n;
  }
  return cache[dev];
}

static void split_args(GemmArgs& p, const WsLayout& L, char* ws) {
  p.part = reinterpret_cast<float*>(ws + L.gemm_part);
  p.tail_cap = L.tail_items;
  p.ncu = device_cus();
}

static GemmArgs base_args(const int32_t* cu, const WsLayout& L, char* ws, int E) {
  GemmArgs p{};
  p.cu = cu;
  p.tiles = reinterpret_cast<const int2*>(ws + L.tiles);
  p.ntiles = reinterpret_cast<const int32_t*>(ws + L.ntiles);
  p.E = E;
  return p;
}

void launch_ffn_up(const void* xd, const int32_t* cu, const void* W1, const void* W3, void* h1,
                   void* h3, void* a, int64_t R, int H, int Hf, int E, const WsLayout& L, char* ws,
                   bool bf16, hipStream_t s) {
  (void)R;
  // [h1 | h3][rows, Hf] = xd[rows, H] * [W1[e] | W3[e]]; W is [H][Hf] = [K][N].
  GemmArgs p = base_args(cu, L, ws, E);
  p.N = Hf; p.K = H;
  p.A0 = xd; p.lda = H;
  p.B0 = W1; p.B1 = W3; p.ldb = Hf; p.sBe = (int64_t)H * Hf;
  p.C0 = h1; p.C1 = h3; p.C2 = a; p.ldc = Hf;
  if (L.bm == kGemmBMFew)
    gemm_launch<kGemmBMFew, 128, true, false, true, false, false, EPI_SWIGLU_FWD, false>(
        "ffn_up", p, L.max_tiles, bf16, s);
  else
    gemm_launch<256, 128, true, false, true, false, false, EPI_SWIGLU_FWD>("ffn_up", p,
                                                                           L.max_tiles, bf16, s);
}

void launch_ffn_down(const void* a, const int32_t* cu, const void* W2, void* y, int64_t R, int H,
                     int Hf, int E, const WsLayout& L, char* ws, bool bf16, hipStream_t s) {
  (void)R;
  // y[rows, H] = a[rows, Hf] * W2[e]; W2[e] is [Hf][H] = [K][N].
  GemmArgs p = base_args(cu, L, ws, E);
  p.N = H; p.K = Hf;
  p.A0 = a; p.lda = Hf;
  p.B0 = W2; p.ldb = H; p.sBe = (int64_t)Hf * H;
  p.C0 = y; p.ldc = H;
  split_args(p, L, ws);
  if (L.bm == kGemmBMFew)
    gemm_launch<kGemmBMFew, 256, true, false, false, false, false, EPI_STORE, false>(
        "ffn_down", p, L.max_tiles, bf16, s);
  else
    gemm_launch<256, 256, true, false, false, false, false, EPI_STORE>("ffn_down", p, L.max_tiles,
                                                                       bf16, s);
}

void launch_bwd_da(const void* dy, const int32_t* cu, const void* W2, const void* h1,
                   const void* h3, void* dh1, void* dh3, int64_t R, int H, int Hf, int E,
                   const WsLayout& L, char* ws, bool bf16, hipStream_t s) {
  (void)R;
  // da[rows, Hf] = dy[rows, H] * W2[e]^T; W2[e] is [Hf][H] = [N][K], K contiguous.
  GemmArgs p = base_args(cu, L, ws, E);
  p.N = Hf; p.K = H;
  p.A0 = dy; p.lda = H;
  p.B0 = W2; p.ldb = H; p.sBe = (int64_t)Hf * H;
  p.C0 = dh1; p.C1 = dh3; p.ldc = Hf;
  p.X0 = h1; p.X1 = h3;
  if (L.bm == kGemmBMFew)
    gemm_launch<kGemmBMFew, 256, true, true, false, false, false, EPI_SWIGLU_BWD, false>(
        "bwd_dA", p, L.max_tiles, bf16, s);
  else
    gemm_launch<256, 256, true, true, false, false, false, EPI_SWIGLU_BWD>("bwd_dA", p,
                                                                           L.max_tiles, bf16, s);
}

void launch_bwd_dxd(const void* dh1, const void* dh3, const int32_t* cu, const void* W1,
                    const void* W3, void* dxd, int64_t R, int H, int Hf, int E, const WsLayout& L,
                    char* ws, bool bf16, hipStream_t s) {
  (void)R;
  // dxd[rows, H] = dh1 * W1[e]^T + dh3 * W3[e]^T; W1[e] is [H][Hf] = [N][K].
  GemmArgs p = base_args(cu, L, ws, E);
  p.N = H; p.K = Hf;
  p.A0 = dh1; p.A1 = dh3; p.lda = Hf;
  p.B0 = W1; p.B1 = W3; p.ldb = Hf; p.sBe = (int64_t)H * Hf;
  p.C0 = dxd; p.ldc = H;
  split_args(p, L, ws);
  if (L.bm == kGemmBMFew)
    gemm_launch<kGemmBMFew, 256, true, true, false, true, false, EPI_STORE, false>(
        "bwd_dxd", p, L.max_tiles, bf16, s);
  else
    gemm_launch<256, 256, true, true, false, true, false, EPI_STORE>("bwd_dxd", p, L.max_tiles,
                                                                     bf16, s);
}

void launch_bwd_dw2(const void* a, const void* dy, const int32_t* cu, const int32_t* eorder,
                    float* dW2, int64_t R, int H, int Hf, int E, bool accum, bool bf16,
                    hipStream_t s) {
  // dW2[e][Hf, H] = a[rows, Hf]^T * dy[rows, H]
  GemmArgs p{};
  p.cu = cu; p.eorder = eorder; p.E = E; p.M = Hf; p.N = H;
  p.deal_whole = 1;  // light experts whole per XCD (-7..10% at 384 experts)
  p.A0 = a; p.lda = Hf;
  p.B0 = dy; p.ldb = H;
  p.C0 = dW2; p.ldc = H; p.sCe = (int64_t)Hf * H;
  p.accum = accum;
  if (accum)
    gemm_launch<256, 256, false, false, false, false, true, EPI_F32_ACC, false>("bwd_dW2", p, 0,
                                                                                bf16, s);
  else if (many_rows(R, E))
    gemm_launch<256, 256, false, false, false, false, true, EPI_F32, true>("bwd_dW2", p, 0, bf16, s);
  else
    gemm_launch<256, 256, false, false, false, false, true, EPI_F32, false>("bwd_dW2", p, 0, bf16, s);
}

void launch_bwd_dw13(const void* xd, const void* dh1, const void* dh3, const int32_t* cu,
                     const int32_t* eorder, float* dW1, float* dW3, int64_t R, int H, int Hf,
                     int E, bool accum, bool bf16, hipStream_t s) {
  // dW1[e][H, Hf] = xd[rows, H]^T * dh1[rows, Hf]; dW3 likewise with dh3.
  GemmArgs p{};
  p.cu = cu; p.eorder = eorder; p.E = E; p.M = H; p.N = Hf;
  p.deal_whole = 0;  // all XCDs share each expert (whole per XCD: +6..12% at 384 experts)
  p.A0 = xd; p.lda = H;
  p.B0 = dh1; p.B1 = dh3; p.ldb = Hf;
  p.C0 = dW1; p.C1 = dW3; p.ldc = Hf; p.sCe = (int64_t)H * Hf;
  p.accum = accum;
  if (accum)
    gemm_launch<256, 128, false, false, true, false, true, EPI_F32_ACC, false>("bwd_dW13", p, 0,
                                                                               bf16, s);
  else if (many_rows(R, E))
    gemm_launch<256, 128, false, false, true, false, true, EPI_F32, true>("bwd_dW13", p, 0, bf16, s);
  else if (bf16) {
    // few rows: 128 x 128 tiles, two blocks per CU (measured at 384 experts:
    // 10.2-11.0 -> 9.6-10.0 ms against 256 x 128 tiles, one block per CU)
    p.ncu = device_cus();
    gemm_launch<128, 128, false, false, true, false, true, EPI_F32, false, 1>("bwd_dW13", p, 0,
                                                                            bf16, s);
  } else {
    gemm_launch<256, 128, false, false, true, false, true, EPI_F32, false>("bwd_dW13", p, 0, bf16, s);
  }
}

}  // namespace moe

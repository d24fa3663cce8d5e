// Router: logits = x*Wg + bias, softmax, top-K and per-expert counts in one
// kernel ("What's in the box" routing/gating item of the MoE/MoD framework
// page: softmax over the experts and the top-k pick in a single launch; the
// T4 tuning page's router section: fuse softmax with top-k and keep the
// routing sparse).
//
// gfx950 design: a block owns 32 tokens.  The router GEMM runs on MFMA
// (v_mfma_f32_16x16x32_bf16) against a transposed copy of the router weight
// made once per call, K-blocked as [H / 32][Epad][32] so that each direct
// load of 16 experts' K32 slices is 1 KB of whole cache lines (a row-major
// [Epad][H] copy would give 64 bytes of each of 16 lines); both operands
// stream through a ring of LDS stages filled by direct global->LDS loads,
// several K slices ahead of the MFMAs.  Four wavefronts issue those loads and four others read the
// stages and run the MFMAs, so a stall of the address unit never holds up
// the matrix core.  The MFMA wavefronts split the 16-expert column blocks,
// or the H reduction when there are fewer than four column blocks (partial
// sums meet in LDS in a fixed order).  Top-K then runs one token per
// wavefront on all eight: each lane holds
// E/64 64-bit order keys (ordered logit bits : ~expert), and K rounds of a
// butterfly max pick the winners.  Counts come from an LDS histogram flushed
// with one atomic per (block, expert).  With few token blocks (small
// batches, up to 1024 tokens) the H reduction is split over several blocks
// per 32 tokens: each writes its fp32 partial logits, and the block that
// finishes last (a per-group ticket) sums the parts in part order and runs
// the top-K.
#include <algorithm>

#include "dev_common.h"
#include "launch.h"
#include "moe.h"
#include "tile.h"

namespace moe {

constexpr int kRouteBT = 32;
constexpr int kRouteWaves = 8;  // bf16 router: 4 load wavefronts + 4 MFMA wavefronts
constexpr int kRouteMaxParts = 16;  // K parts per token group of the split router

__global__ void fill_i32_kernel(int32_t* p, int32_t v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}
__global__ void fill_f32_kernel(float* p, float v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

void launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  TimedLaunch tl("fill", s);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks), dim3(256), 0, s, p, v, n);
}
void launch_fill_f32(float* p, float v, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  TimedLaunch tl("fill", s);
  hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks), dim3(256), 0, s, p, v, n);
}

// WgT[e][h] = Wg[h][e] for e < E, zero rows for E <= e < epad.  Row-major
// [epad][H] (one contiguous row per expert, for the fp32 router and the
// dispatch backward), or K-blocked [H / 32][epad][32] for the bf16 router:
// there one K32 slice of every expert row is 64 contiguous bytes and the
// slices of consecutive experts are adjacent, so a direct load of 16
// experts' slices reads 1 KB of whole cache lines.
template <bool BF16, bool BLOCKED>
__global__ __launch_bounds__(256) void transpose_wg_kernel(const void* Wg, void* wgT, int H, int E,
                                                           int epad, int32_t* tickets,
                                                           int ntickets) {
  // the router's per-group tickets start every call at zero
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < ntickets; i += 256) tickets[i] = 0;
  __shared__ float tile[32][33];
  const int h0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int h = h0 + i, e = e0 + tx;
    tile[i][tx] = (h < H && e < E) ? load1<BF16>(Wg, (int64_t)h * E + e) : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int e = e0 + i, h = h0 + tx;
    if (e < epad && h < H) {
      const int64_t o = BLOCKED ? ((int64_t)(h >> 5) * epad + e) * 32 + (h & 31) : (int64_t)e * H + h;
      store1<BF16>(wgT, o, tile[tx][i]);
    }
  }
}

void launch_transpose_wg(const void* Wg, void* wgT, int H, int E, int epad, bool bf16,
                         bool blocked, int32_t* tickets, int ntickets, hipStream_t s) {
  dim3 grid((H + 31) / 32, (epad + 31) / 32);
  TimedLaunch tl("route_wg_transpose", s);
  if (bf16 && blocked)
    hipLaunchKernelGGL((transpose_wg_kernel<true, true>), grid, dim3(256), 0, s, Wg, wgT, H, E,
                       epad, tickets, ntickets);
  else if (bf16)
    hipLaunchKernelGGL((transpose_wg_kernel<true, false>), grid, dim3(256), 0, s, Wg, wgT, H, E,
                       epad, tickets, ntickets);
  else
    hipLaunchKernelGGL((transpose_wg_kernel<false, false>), grid, dim3(256), 0, s, Wg, wgT, H, E,
                       epad, tickets, ntickets);
}

// ------------------------------------------------------------ router GEMM --
// Waves split the 16-expert column blocks (nwn of them side by side, NCB
// blocks each) and, when there are fewer than four column blocks, the K
// range (KS waves along K); U K32 sub-slices per wave per stage keep the
// stages of small routers from being tiny.
struct RouteSplit {
  int nwn, ks, ncb, u;
};
inline RouteSplit route_split(int epad) {
  const int nb = epad / 16;
  RouteSplit r;
  r.nwn = nb >= 4 ? 4 : (nb >= 2 ? 2 : 1);
  r.ks = 4 / r.nwn;
  r.ncb = (nb + r.nwn - 1) / r.nwn;
  r.u = (r.ks == 1 && r.ncb <= 2) ? 2 : 1;
  return r;
}

// LDS pipeline of the bf16 router GEMM.  A stage holds one K slice of BK
// elements: the x tile [32 tokens][BK] (shared by all wavefronts) and, per
// wavefront, its NCB column blocks x U sub-slices of router-weight rows
// ([16][32] each, 1 KB).  Every wavefront issues the same kNI direct loads per
// stage (kXI 256-byte loads of x, NCB U 1-KB loads of its own weight rows),
// so each one can wait for its own loads of a stage with one vmcnt.
template <int NCB, int KS, int U>
struct RouteTile {
  static constexpr int BK = 32 * KS * U;
  static constexpr int kXB = kRouteBT * BK * 2;
  static constexpr int kWB = NCB * U * 1024;
  static constexpr int kStage = kXB + 4 * kWB;
  static constexpr int kXI = kXB / 1024;
  static constexpr int kNI = kXI + NCB * U;
  static constexpr int NS0 = (104 * 1024) / kStage;
  static constexpr int NS1 = NS0 < 2 ? 2 : (NS0 > 8 ? 8 : NS0);
  // a wavefront waits with vmcnt((NS - 2) kNI), and vmcnt counts to 63
  static constexpr int NS = (NS1 - 2) * kNI <= 63 ? NS1 : 2 + 63 / kNI;
  static constexpr int CPR = BK / 8;  // 16-byte chunks per x row
};
// x rows: 16-byte chunk c of row r stored at c ^ xswz(r), which keeps a
// 16x16x32 fragment read (16 rows x 4 chunks) on all 16 bank groups per
// 16 lanes.  Weight rows are 64 bytes (four chunks): c ^ ((r >> 2) & 3).
template <int CPR>
__device__ __forceinline__ int xswz(int r) {
  return CPR == 4 ? (r >> 2) & 3 : CPR == 8 ? (r >> 1) & 7 : r & 15;
}

// Logits, softmax, top-K and counts of the block's tokens from the partial
// logits part[ks][32][epad] (the bias already in slice 0; slices summed in
// slice order).  Wavefront w of NW owns tokens w, w + NW, ...: it finishes their
// logit rows (coalesced row stores, no index division) and then picks
// their top K.  NJ bounds the keys per lane (E <= 64 NJ).
template <int NJ, int NW>
__device__ __forceinline__ void route_tail(float* part, int* hist, int ks, float* logits,
                                           int32_t* idx, float* gates, int32_t* counts,
                                           uint32_t* status, int t0, int nt, int E, int epad,
                                           int K, int renorm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t bad = 0;
  for (int t = w; t < nt; t += NW) {
    float* lrow = part + t * epad;
    for (int e = lane; e < E; e += 64) {
      float v = lrow[e];
      for (int k2 = 1; k2 < ks; ++k2) v += part[((size_t)k2 * kRouteBT + t) * epad + e];
      if (ks > 1) lrow[e] = v;
      if (!isfinite(v)) bad = 1;
      if (logits) logits[(int64_t)(t0 + t) * E + e] = v;
    }
  }
  if (bad) atomicOr(status, (uint32_t)MOE_DEV_NONFINITE_LOGIT);

  // Top-K: one token per wavefront at a time (the rows this wavefront just
  // finished, so no barrier is needed).
  const int nj = (E + 63) / 64;
  for (int t = w; t < nt; t += NW) {
    const float* lrow = part + t * epad;
    uint64_t keys[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      keys[j] = (j < nj && e < E) ? topk_key(lrow[e], e) : 0ull;
    }
    float m = 0.f, my_l = 0.f;
    int my_e = -1;
    for (int k = 0; k < K; ++k) {
      uint64_t best = 0ull;
#pragma unroll
      for (int j = 0; j < NJ; ++j) best = keys[j] > best ? keys[j] : best;
      best = wave_max_u64(best);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (keys[j] == best) keys[j] = 0ull;
      const int e = key_expert(best);
      const float l = lrow[e];
      if (k == 0) m = l;
      if (lane == k) { my_e = e; my_l = l; }
    }
    const float wk = lane < K ? expf(my_l - m) : 0.f;
    float denom;
    if (renorm) {
      denom = wave_sum(wk);
    } else {
      float z = 0.f;
      for (int j = 0; j < nj; ++j) {
        const int e = lane + 64 * j;
        if (e < E) z += expf(lrow[e] - m);
      }
      denom = wave_sum(z);
    }
    if (lane < K) {
      const int64_t o = (int64_t)(t0 + t) * K + lane;
      idx[o] = my_e;
      gates[o] = wk / denom;
      atomicAdd(&hist[my_e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 64 * NW)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

// bf16 router: x [S, H] times the K-blocked transposed weight on
// v_mfma_f32_16x16x32_bf16, both operands streamed through an NS-stage LDS
// ring by direct loads; NS - 1 stages are in flight while one is computed.
template <int NCB, int KS, int U>
__global__ __launch_bounds__(64 * kRouteWaves) void route_mfma_kernel(const void* __restrict__ x,
                                                         const void* __restrict__ wgT,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits,
                                                         int32_t* __restrict__ idx,
                                                         float* __restrict__ gates,
                                                         int32_t* __restrict__ counts,
                                                         uint32_t* __restrict__ status, int S,
                                                         int H, int E, int epad, int K,
                                                         int renorm, int nparts,
                                                         float* __restrict__ rpart,
                                                         int32_t* __restrict__ tickets) {
  using T = RouteTile<NCB, KS, U>;
  constexpr int NWN = 4 / KS;
  extern __shared__ __attribute__((aligned(1024))) char smem[];  // stages, then partial logits
  __shared__ int hist[1024];
  __shared__ int last_part;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wavefronts 0-3 compute, 4-7 load on behalf of compute wavefront w
  const bool loader = wv >= 4;
  const int w = wv & 3;
  const int wn = w % NWN, ksi = w / NWN;
  // token group g, K part `part` of nparts (steps [s_lo, s_lo + nsteps))
  const int g = blockIdx.x / nparts, part_id = blockIdx.x - g * nparts;
  const int t0 = g * kRouteBT;
  const int nt = min(kRouteBT, S - t0);
  const int ns_all = H / T::BK;
  const int s_lo = part_id * ns_all / nparts;
  const int nsteps = (part_id + 1) * ns_all / nparts - s_lo;
  for (int e = tid; e < E; e += 64 * kRouteWaves) hist[e] = 0;

  // per-lane byte offsets of this wavefront's direct loads (relative to the
  // stage's K origin)
  uint32_t vx[T::kXI], vw[NCB * U];
#pragma unroll
  for (int i = 0; i < T::kXI; ++i) {
    const int P = (w * T::kXI + i) * 64 + lane;  // physical dword of the x tile
    const int row = P / (T::BK / 2), pdw = P % (T::BK / 2);
    const int c = (pdw >> 2) ^ xswz<T::CPR>(row);
    vx[i] = ((uint32_t)row * H + c * 8 + (pdw & 3) * 2) * 2u;
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = lane >> 2, c = (lane & 3) ^ ((row >> 2) & 3);
      const int n = (wn + cb * NWN) * 16 + row;
      // K-blocked WgT: K32 slice ksi U + u of the stage, expert row n
      vw[cb * U + u] = (((uint32_t)(ksi * U + u) * epad + n) * 32 + c * 8) * 2u;
    }
  const char* xb = reinterpret_cast<const char*>(x) + (int64_t)t0 * H * 2;
  const char* wb = reinterpret_cast<const char*>(wgT);
  const uint32_t xbytes = (uint32_t)nt * H * 2u, wbytes = (uint32_t)epad * H * 2u;
  // loads of K slice kt into stage st (past the end of K they read zeros or
  // rows of this block's own range, into a stage that is not read again)
  auto issue = [&](int kt, int st) {
    const uint32_t k2 = (uint32_t)(s_lo + kt) * T::BK * 2u;                  // along a row of x
    const uint32_t w2 = (uint32_t)(s_lo + kt) * (T::BK / 32) * epad * 64u;  // K32 blocks of WgT
    const u32x4 rx = rsrc_words(xb + k2, xbytes - min(k2, xbytes));
    const u32x4 rw = rsrc_words(wb + w2, wbytes - min(w2, wbytes));
    char* sb = smem + st * T::kStage;
#pragma unroll
    for (int i = 0; i < T::kXI; ++i) dma4(rx, vx[i], sb + (w * T::kXI + i) * 256);
#pragma unroll
    for (int j = 0; j < NCB * U; ++j) dma16(rw, vw[j], sb + T::kXB + w * T::kWB + j * 1024);
  };

  f32x4 acc[2][NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[0][cb] = acc[1][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (loader) {
#pragma unroll
    for (int st = 0; st < T::NS - 1; ++st) issue(st, st);
  }
  const int r16 = lane & 15, q = lane >> 4;
  for (int kt = 0; kt < nsteps; ++kt) {
    // a loader's loads of slice kt landed (compute wavefronts have none in
    // flight); after the barrier so have everyone's, and every compute
    // wavefront is done with slice kt - 1's stage, which the loads of slice
    // kt + NS - 1 now refill
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((T::NS - 2) * T::kNI) : "memory");
    if (loader) {
      issue(kt + T::NS - 1, (kt + T::NS - 1) % T::NS);
      continue;
    }
    const char* sb = smem + (kt % T::NS) * T::kStage;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = ksi * U + u;  // K32 sub-slice of the stage
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(
          sb + r16 * (T::BK * 2) + (((kk * 4 + q) ^ xswz<T::CPR>(r16)) << 4));
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(
          sb + (r16 + 16) * (T::BK * 2) + (((kk * 4 + q) ^ xswz<T::CPR>(r16 + 16)) << 4));
      // column blocks past epad hold zeros (their weight rows lie outside
      // the descriptor's range): no branch, so all fragment reads go out
      // before the MFMAs
      u32x4 b[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        b[cb] = *reinterpret_cast<const u32x4*>(sb + T::kXB + w * T::kWB + (cb * U + u) * 1024 +
                                                r16 * 64 + ((q ^ ((r16 >> 2) & 3)) << 4));
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        acc[0][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a0), __builtin_bit_cast(bf16x8, b[cb]), acc[0][cb], 0, 0, 0);
        acc[1][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a1), __builtin_bit_cast(bf16x8, b[cb]), acc[1][cb], 0, 0, 0);
      }
    }
  }
  // every direct load has landed and every wavefront is done with the stages
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

  // 16x16 MFMA result: lane holds column (lane % 16), rows 4 (lane / 16) + i;
  // slice 0 carries the bias
  float* part = reinterpret_cast<float*>(smem);
  if constexpr (KS == 1) {
    if (nparts > 1) {
      // this part's logits (no bias) -> rpart[group][part][32][epad]
      float* gp = rpart + (size_t)blockIdx.x * kRouteBT * epad;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int nbk = wn + cb * NWN;
        if (!loader && nbk * 16 < epad) {
          const int col = nbk * 16 + r16;
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) gp[(size_t)(rb * 16 + q * 4 + i) * epad + col] = acc[rb][cb][i];
        }
      }
      // publish the part; the group's last block to take a ticket sums them
      __threadfence();
      __syncthreads();
      if (tid == 0) last_part = atomicAdd(&tickets[g], 1) == nparts - 1;
      __syncthreads();
      if (!last_part) return;
      __threadfence();
      // sum the parts in part order, four logits a lane, all parts' loads
      // in flight together (epad is a multiple of 16, so a 4-float piece
      // never crosses a row)
      const f32x4* g0 = reinterpret_cast<const f32x4*>(rpart + (size_t)g * nparts * kRouteBT * epad);
      const int n4 = kRouteBT * epad / 4, pstride = kRouteBT * epad / 4;
      for (int i = tid; i < n4; i += 64 * kRouteWaves) {
        f32x4 pv[kRouteMaxParts];
#pragma unroll
        for (int pp = 0; pp < kRouteMaxParts; ++pp)
          if (pp < nparts) pv[pp] = g0[(size_t)pp * pstride + i];
        f32x4 v = pv[0];
#pragma unroll
        for (int pp = 1; pp < kRouteMaxParts; ++pp)
          if (pp < nparts) v += pv[pp];
        const int col = (4 * i) % epad;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (bias != nullptr && col + c < E) v[c] += bias[col + c];
        reinterpret_cast<f32x4*>(part)[i] = v;
      }
      __syncthreads();
      route_tail<NCB, kRouteWaves>(part, hist, 1, logits, idx, gates, counts, status, t0, nt, E,
                                   epad, K, renorm);
      return;
    }
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int nbk = wn + cb * NWN;
    if (!loader && nbk * 16 < epad) {
      const int col = nbk * 16 + r16;
      const float bv = (bias != nullptr && ksi == 0 && col < E) ? bias[col] : 0.f;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          part[((size_t)ksi * kRouteBT + rb * 16 + q * 4 + i) * epad + col] = acc[rb][cb][i] + bv;
    }
  }
  __syncthreads();
  // keys per lane: at most NCB (one wavefront row of K) or one (E < 64)
  route_tail<KS == 1 ? NCB : 1, kRouteWaves>(part, hist, KS, logits, idx, gates, counts, status,
                                             t0, nt, E, epad, K, renorm);
}

// ------------------------------------------------- tiled router (many E) --
// With many experts and many tokens the fused router above streams the whole
// router weight once per 32 tokens (at 384 experts and 8192 tokens, 256
// blocks each reading 5.5 MB of weight through L2 into LDS: the L2 -> CU feed
// bounds it).  Here the projection is a tiled GEMM instead: a block owns 128
// tokens x 128 experts, so each weight byte is fed once per 128 tokens and
// each activation byte once per 128 experts, and the logits go to memory
// (fp32, bias added); a second launch then does the softmax, the top-K, the
// gates and the counts per token from those logits.  The weight is read in
// its [H][E] layout as a K-major tile (transposing LDS reads), so no
// transposed copy is made.  Taken for bf16 with E >= 256 experts (a multiple
// of 8: 16-byte rows) at any token count (few tokens split H into parts,
// below); the fused router keeps the rest (few experts, fp32, ragged E).
constexpr int kRgBM = 128, kRgBN = 128, kRgNS = 4;  // tile, LDS stages (3 in flight)

bool route_tiled(int64_t, int E, bool bf16) { return bf16 && E >= 256 && E % 8 == 0; }

// K parts of the tiled router: while the tiles alone fill less than half
// the chip, the H extent is cut into up to 16 parts (each at least 4 K
// steps) whose fp32 partial logits a second launch sums in part order.
// Measured at 128 tokens x 384 experts x H 7168 (3 tiles -> 16 parts, 48
// blocks): the route call (projection, sum, top-K) takes 27 us against 63 us
// for the fused router split over H with tickets; 32 parts take 30 us and
// 64 parts 40 us (the partial logits' traffic grows with the parts).
int route_tiled_parts(int64_t S, int H, int E) {
  constexpr int kMaxParts = 16, kMinSteps = 4;
  const int64_t tiles = (S + kRgBM - 1) / kRgBM * ((E + kRgBN - 1) / kRgBN);
  const int nk = H / kBK;
  int P = 1;
  while (P < kMaxParts && tiles * P * 2 <= 256 && nk >= kMinSteps * P * 2) P *= 2;
  return P;
}

// logits [S, E] = x [S, H] * Wg [H, E] + bias; kRgWaves wavefronts (2 along
// the tokens), each 64 tokens x 128 / (kRgWaves / 2) experts on
// v_mfma_f32_32x32x16_bf16 with the weight fragment as the first operand
// (each lane ends with four consecutive experts of one token).
constexpr int kRgWaves = 8;
__global__ __launch_bounds__(64 * kRgWaves) void route_gemm_kernel(const void* __restrict__ x,
                                                         const void* __restrict__ Wg,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ out,
                                                         int32_t* __restrict__ counts, int S,
                                                         int H, int E, int ntn) {
  // blockIdx.y: K part; with several parts each block writes its part's
  // partial logits (no bias) to out + part * S * E
  constexpr int kTileA = kRgBM * kBK * 2, kTileB = kRgBN * kBK * 2, kStage = kTileA + kTileB;
  __shared__ __attribute__((aligned(1024))) char smem[kRgNS * kStage];
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = bid / ntn, nt = bid - mt * ntn;
  const int t0 = mt * kRgBM, e0 = nt * kRgBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the top-K launch that follows adds each block's expert counts
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = tid; i < E; i += 64 * kRgWaves) counts[i] = 0;
  const int nparts = gridDim.y, part = blockIdx.y;
  if (nparts > 1) {
    out += (int64_t)part * S * E;
    bias = nullptr;  // added once, when the parts are summed
  }
  constexpr int kWN = kRgWaves / 2, kWNT = kRgBN / kWN, NJ = kWNT / 32;
  const int wm = w / kWN, wn = w % kWN;
  const int rows = min(kRgBM, S - t0);

  // x rows of the tile (rows past S read zeros) and the weight columns
  // e0 .. e0 + 127 (columns past E read other columns or zeros; they are
  // never stored)
  DmaOperand<true, kRgBM, 1, kRgWaves> da;
  DmaOperand<false, kRgBN, 1, kRgWaves> db;
  da.init(H, 0, w, lane);
  db.init(E, 0, w, lane);
  const uint16_t* const pa[1] = {reinterpret_cast<const uint16_t*>(x) + (int64_t)t0 * H};
  const uint16_t* const pb[1] = {reinterpret_cast<const uint16_t*>(Wg) + e0};
  const uint32_t a_bytes = (uint32_t)rows * (uint32_t)H * 2u;
  const uint32_t b_bytes = ((uint32_t)H * (uint32_t)E - (uint32_t)e0) * 2u;
  constexpr int kPA = DmaOperand<true, kRgBM, 1, kRgWaves>::kPer;
  constexpr int kPB = DmaOperand<false, kRgBN, 1, kRgWaves>::kPer;
  auto issue = [&](int kt, int st) {
    u32x4 ra[1], rb[1];
    da.rsrc_for(pa, a_bytes, H, kt * kBK, ra);
    db.rsrc_for(pb, b_bytes, E, kt * kBK, rb);
    char* sb = smem + st * kStage;
#pragma unroll
    for (int i = 0; i < kPA; ++i) da.issue_one(i, ra, sb, w);
#pragma unroll
    for (int i = 0; i < kPB; ++i) db.issue_one(i, rb, sb + kTileA, w);
  };
  // K steps [kb, ke) of this block's part
  const int nkall = H / kBK, kb = part * nkall / nparts, ke = (part + 1) * nkall / nparts;
#pragma unroll
  for (int st = 0; st < kRgNS - 1; ++st) issue(kb + st, st);  // past ke: in-range or zero reads, never used

  f32x16 acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  uint32_t bbase[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) bbase[j] = frag_km_base<kRgBN>(wn * kWNT + j * 32, lane);

  for (int kt = kb; kt < ke; ++kt) {
    // this wavefront's loads of step kt landed (those of the next NS - 2
    // steps may still be in flight); after the barrier everyone's have, and
    // every wavefront is done with step kt - 1's stage, which step
    // kt + NS - 1 now refills
    const int li = kt - kb;
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((kRgNS - 2) * (kPA + kPB)) : "memory");
    issue(kt + kRgNS - 1, (li + kRgNS - 1) % kRgNS);
    const char* sa = smem + (li % kRgNS) * kStage;
    const char* sbt = sa + kTileA;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      u32x4 af[2], bf[NJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = frag_kc(sa, wm * 64 + i * 32, kk, lane);
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[j] = frag_km_at<kRgBN>(sbt, bbase[j], kk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, bf[j]), __builtin_bit_cast(bf16x8, af[i]), acc[i][j], 0,
              0, 0);
    }
  }
  // no direct load may still be writing LDS when the block exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // lane l holds token row (l % 32) of each 32 x 32 block and experts
  // 8 g + 4 (l / 32) + 0..3 (E is a multiple of 8, so a piece is all in or
  // all out)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wm * 64 + i * 32 + (lane & 31);
    if (r >= rows) continue;
    float* orow = out + (int64_t)(t0 + r) * E;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = e0 + wn * kWNT + j * 32 + 8 * g + 4 * (lane >> 5);
        if (c >= E) continue;
        f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                   acc[i][j][4 * g + 3]};
        if (bias != nullptr) {
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(bias + c);
          v += b4;
        }
        *reinterpret_cast<f32x4*>(orow + c) = v;
      }
  }
}

// Softmax, top-K, gates and counts from the logit rows (the router GEMM's
// output): 16 tokens per block, one per wavefront, their rows staged in LDS
// and their (token, k) pairs counted in an LDS histogram.
constexpr int kTopkTB = 16;

template <int NJ>
__global__ __launch_bounds__(64 * kTopkTB) void route_topk_kernel(
    const float* __restrict__ logits, int32_t* __restrict__ idx, float* __restrict__ gates,
    int32_t* __restrict__ counts, uint32_t* __restrict__ status, int S, int E, int epad, int K,
    int renorm) {
  extern __shared__ __attribute__((aligned(16))) float rows_l[];  // [kTopkTB][epad]
  __shared__ int hist[1024];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTopkTB;
  const int nt = min(kTopkTB, S - t0);
  for (int e = tid; e < E; e += 64 * kTopkTB) hist[e] = 0;
  const int n4 = E / 4;
  for (int i = tid; i < nt * n4; i += 64 * kTopkTB) {
    const int t = i / n4, c = i - t * n4;
    reinterpret_cast<f32x4*>(rows_l + t * epad)[c] =
        reinterpret_cast<const f32x4*>(logits + (int64_t)(t0 + t) * E)[c];
  }
  __syncthreads();
  route_tail<NJ, kTopkTB>(rows_l, hist, 1, nullptr, idx, gates, counts, status, t0, nt, E, epad,
                          K, renorm);
}

// logits [S, E] = bias + the sum of the K parts' partial logits, in part order
__global__ __launch_bounds__(256) void route_part_sum_kernel(const float* __restrict__ part,
                                                            int nparts,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int S,
                                                            int E) {
  const int64_t n4 = (int64_t)S * E / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4 v = reinterpret_cast<const f32x4*>(part)[i];
  for (int pp = 1; pp < nparts; ++pp) v += reinterpret_cast<const f32x4*>(part)[(int64_t)pp * n4 + i];
  if (bias != nullptr) v += *reinterpret_cast<const f32x4*>(bias + (4 * i) % E);
  reinterpret_cast<f32x4*>(logits)[i] = v;
}

void launch_route_tiled(const void* x, const void* Wg, const float* bias, float* logits,
                        int32_t* idx, float* gates, int32_t* counts, uint32_t* status, int64_t S,
                        int H, int E, int epad, int K, bool renorm, float* part, hipStream_t s) {
  const int ntn = (E + kRgBN - 1) / kRgBN;
  const int blocks = (int)((S + kRgBM - 1) / kRgBM) * ntn;
  const int P = part != nullptr ? route_tiled_parts(S, H, E) : 1;
  {
    TimedLaunch tl("route", s);
    hipLaunchKernelGGL(route_gemm_kernel, dim3(blocks, P), dim3(64 * kRgWaves), 0, s, x, Wg, bias,
                       P > 1 ? part : logits, counts, (int)S, H, E, ntn);
  }
  if (P > 1) {
    TimedLaunch tl("route_part_sum", s);
    const int64_t n4 = S * (int64_t)E / 4;
    hipLaunchKernelGGL(route_part_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       part, P, bias, logits, (int)S, E);
  }
  const size_t lds = (size_t)kTopkTB * epad * sizeof(float);
  const int tb = (int)((S + kTopkTB - 1) / kTopkTB);
  TimedLaunch tl("route_topk", s);
#define TOPK_CASE(NJ)                                                                          \
  if ((E + 63) / 64 <= NJ) {                                                                   \
    static bool attr = false;                                                                  \
    if (!attr)                                                                                 \
      attr = hipFuncSetAttribute(reinterpret_cast<const void*>(route_topk_kernel<NJ>),         \
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024) ==    \
             hipSuccess;                                                                       \
    hipLaunchKernelGGL(route_topk_kernel<NJ>, dim3(tb), dim3(64 * kTopkTB), lds, s, logits, idx, \
                       gates, counts, status, (int)S, E, epad, K, renorm ? 1 : 0);            \
    return;                                                                                    \
  }
  TOPK_CASE(4) TOPK_CASE(8) TOPK_CASE(16)
#undef TOPK_CASE
}

// fp32 router: plain dot products, one (token, expert) pair per thread.
__global__ __launch_bounds__(256) void route_f32_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ wgT,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ logits,
                                                        int32_t* __restrict__ idx,
                                                        float* __restrict__ gates,
                                                        int32_t* __restrict__ counts,
                                                        uint32_t* __restrict__ status, int S,
                                                        int H, int E, int epad, int K, int renorm) {
  extern __shared__ float fpart[];  // [32][epad]
  __shared__ int hist[1024];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRouteBT;
  const int nt = min(kRouteBT, S - t0);
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  for (int i = tid; i < kRouteBT * E; i += 256) {
    const int t = i / E, e = i % E;
    float acc = 0.f;
    if (t < nt) {
      const float* xr = x + (int64_t)(t0 + t) * H;
      const float* wr = wgT + (int64_t)e * H;
      for (int h = 0; h < H; ++h) acc = fmaf(xr[h], wr[h], acc);
    }
    fpart[t * epad + e] = acc + (bias ? bias[e] : 0.f);
  }
  __syncthreads();
  route_tail<16, 4>(fpart, hist, 1, logits, idx, gates, counts, status, t0, nt, E, epad, K, renorm);
}

template <int NCB, int KS, int U>
static void route_launch_t(const void* x, const void* wgT, const float* bias, float* logits,
                           int32_t* idx, float* gates, int32_t* counts, uint32_t* status, int64_t S,
                           int H, int E, int epad, int K, bool renorm, int nparts, float* rpart,
                           int32_t* tickets, hipStream_t s) {
  using T = RouteTile<NCB, KS, U>;
  const size_t lds = std::max((size_t)T::NS * T::kStage, (size_t)KS * kRouteBT * epad * sizeof(float));
  auto kern = route_mfma_kernel<NCB, KS, U>;
  // a failure stays the thread's last HIP error (the entry point reports it)
  static bool attr = false;
  if (!attr)
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024) == hipSuccess;
  const int blocks = (int)((S + kRouteBT - 1) / kRouteBT) * nparts;
  TimedLaunch tl("route", s);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * kRouteWaves), lds, s, x, wgT, bias, logits, idx,
                     gates, counts, status, (int)S, H, E, epad, K, renorm ? 1 : 0, nparts, rpart,
                     tickets);
}

// Up to kRouteMaxParts parts while the grid stays within a quarter of the
// compute units and every part keeps at least four K steps.  The split costs
// each part an agent-scope release and the last one an acquire, which on
// gfx950 write back and invalidate the L2 of its XCD; every other block of
// that XCD then fetches its router-weight slices again.  That is cheap next
// to the work of a few groups but not once the groups alone fill the chip:
// measured at 8192 tokens (256 groups), two parts took the router from 146
// to 359 us at 384 experts and from 26 to 210 us at 64 experts, while at 128
// tokens (4 groups, 384 experts) four parts took it from 130 to 60 us.
int route_parts(int64_t S, int H, int epad) {
  const RouteSplit sp = route_split(epad);
  if (sp.ks != 1) return 1;
  const int64_t groups = (S + kRouteBT - 1) / kRouteBT;
  const int steps = H / (32 * sp.u);
  int P = 1;
  while (P < kRouteMaxParts && groups * P * 2 <= 64 && steps >= 4 * P * 2) P *= 2;
  return P;
}

void launch_route(const void* x, const void* wgT, const float* bias, float* logits, int32_t* idx,
                  float* gates, int32_t* counts, uint32_t* status, int64_t S, int H, int E,
                  int epad, int K, bool renorm, bool bf16, int nparts, float* rpart,
                  int32_t* tickets, hipStream_t s) {
  if (S <= 0) return;
  if (!bf16) {
    const size_t lds = (size_t)kRouteBT * epad * sizeof(float);
    static bool attr = false;
    if (!attr)
      attr = hipFuncSetAttribute(reinterpret_cast<const void*>(route_f32_kernel),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024) == hipSuccess;
    const int blocks = (int)((S + kRouteBT - 1) / kRouteBT);
    TimedLaunch tl("route", s);
    hipLaunchKernelGGL(route_f32_kernel, dim3(blocks), dim3(256), lds, s,
                       reinterpret_cast<const float*>(x), reinterpret_cast<const float*>(wgT), bias,
                       logits, idx, gates, counts, status, (int)S, H, E, epad, K, renorm ? 1 : 0);
    return;
  }
  const RouteSplit sp = route_split(epad);
#define ROUTE_CASE(N, KS_, U_)                                                                  \
  if (sp.ks == KS_ && sp.u == U_ && sp.ncb <= N) {                                             \
    route_launch_t<N, KS_, U_>(x, wgT, bias, logits, idx, gates, counts, status, S, H, E, epad, \
                               K, renorm, nparts, rpart, tickets, s);                          \
    return;                                                                                    \
  }
  ROUTE_CASE(1, 4, 1) ROUTE_CASE(1, 2, 1) ROUTE_CASE(2, 2, 1) ROUTE_CASE(1, 1, 2)
  ROUTE_CASE(2, 1, 2) ROUTE_CASE(3, 1, 1) ROUTE_CASE(4, 1, 1) ROUTE_CASE(6, 1, 1)
  ROUTE_CASE(8, 1, 1) ROUTE_CASE(12, 1, 1) ROUTE_CASE(16, 1, 1)
#undef ROUTE_CASE
}

// Load statistics of the routing histogram (the MoonEP page's load measure
// maxvio = max load / mean load - 1, and the entropy of the load shares):
// one block of 1024 threads, one expert each; the sums and the maximum meet
// through the wavefront reductions and LDS in a fixed order (deterministic).
__global__ __launch_bounds__(1024) void load_stats_kernel(const int32_t* __restrict__ counts,
                                                          int E, float* __restrict__ stats) {
  __shared__ float part[3][16];
  const int e = threadIdx.x, lane = e & 63, w = e >> 6;
  const float c = e < E ? (float)max(counts[e], 0) : 0.f;
  const float tot = wave_sum(c), mx = wave_max_f32(c);
  if (lane == 0) { part[0][w] = tot; part[1][w] = mx; }
  __syncthreads();
  float total = 0.f, cmax = 0.f;
  for (int i = 0; i < 16; ++i) { total += part[0][i]; cmax = fmaxf(cmax, part[1][i]); }
  const float f = total > 0.f ? c / total : 0.f;
  const float h = wave_sum(f > 0.f ? -f * logf(f) : 0.f);
  if (lane == 0) part[2][w] = h;
  __syncthreads();
  if (e == 0) {
    float ent = 0.f;
    for (int i = 0; i < 16; ++i) ent += part[2][i];
    stats[0] = total > 0.f ? cmax * (float)E / total - 1.0f : 0.f;
    stats[1] = ent;
  }
}

void launch_load_stats(const int32_t* counts, int E, float* stats, hipStream_t s) {
  TimedLaunch tl("load_stats", s);
  hipLaunchKernelGGL(load_stats_kernel, dim3(1), dim3(1024), 0, s, counts, E, stats);
}

}  // namespace moe

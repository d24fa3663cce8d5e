// Combine and the gating/dispatch backward.
//
// combine      out[s] = sum_k g[s,k] y[row_of[s*K+k]]   (MoE/MoD framework
//              page, "What's in the box", dispatch/combine item)
// combine_bwd  one pass over each token's K rows computes dy = g*dout, the
//              gate gradient <dout, y[row]>, and the logit gradient through
//              the renormalised softmax, without storing anything else
//              (same page, sparse-backward item: gating and dispatch
//              gradients in one kernel, no saved intermediates)
// dx           dx[s] = sum_k dxd[row] + sum_k dl[s,idx_k] Wg[:, idx_k]
// dwg          dWg[:, e] = sum over expert e's rows of dl_row[r] * xd[r]
//
// gfx950 design: each lane streams 16-byte pieces (8 bf16) of a token's
// rows, accumulates in fp32 and writes 16-byte pieces, so every row read and
// write is a full coalesced 1-KB wave access.  combine and dx give each
// wavefront one 128-piece column chunk of one token (a 7168-wide row is
// seven wavefronts, so the launch ends evenly across the compute units);
// combine_bwd does the same inside one block per token, whose wavefronts
// then add up the gate gradient's partial dot products in LDS.
// The router-weight gradient reduces over each expert's contiguous rows in
// row order (deterministic), cut into row items of bounded size so a hot
// expert spreads over many blocks; a second kernel adds the items in order.
#include "dev_common.h"
#include "launch.h"
#include "moe.h"

namespace moe {

// Rows are read as 16-byte pieces (8 bf16 or 4 fp32 values) through one
// buffer descriptor per (token, k) held in scalar registers; a pair with no
// row (k >= K, or an invalid row index) gets an empty range and reads zero,
// and pieces past the row end read zero too, so the loads carry no branches
// and all K of them (for two or four column chunks) are in flight at once.
template <bool BF16>
struct Piece {
  static constexpr int kEl = BF16 ? 8 : 4;   // values per 16-byte piece
  static constexpr int kEb = BF16 ? 2 : 4;   // bytes per value
  __device__ __forceinline__ static void unpack(const u32x4 w, float (&v)[8]) {
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(w[i]); v[2 * i + 1] = bf16_hi(w[i]); }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
    }
  }
  __device__ __forceinline__ static u32x4 pack(const float (&v)[8]) {
    u32x4 w;
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(v[i]);
    }
    return w;
  }
};

// Descriptor of row `row` (wave-uniform) of a [rows, H] tensor; empty when !ok.
template <bool BF16>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int row, int H,
                                                           bool ok) {
  const int r = __builtin_amdgcn_readfirstlane(ok ? row : 0);
  const uint32_t bytes = __builtin_amdgcn_readfirstlane(ok ? (uint32_t)H * Piece<BF16>::kEb : 0u);
  return make_rsrc(reinterpret_cast<const char*>(base) + (int64_t)r * H * Piece<BF16>::kEb, bytes);
}

// column chunks (of 64 pieces) per iteration; one chunk measured 10-12 us
// faster than two for dx at 384 experts, top-8 (252 against 263 us), and the
// same at 8 experts
constexpr int kCombU = 1;
// combine and dx: one wavefront per (token, chunk of kCombChunk pieces), so
// a wide row spreads over several wavefronts and the last wave of a launch
// is short
constexpr int kCombChunk = 64 * kCombU;

template <bool BF16, int KT>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ gates,
                                                      void* __restrict__ out, int S, int H, int K,
                                                      int64_t R) {
  using PC = Piece<BF16>;
  const int lane = threadIdx.x & 63;
  const int pieces = H / PC::kEl;
  const int nch = (pieces + kCombChunk - 1) / kCombChunk;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)S * nch) return;
  const int s = (int)(item / nch);
  int rk = -1;
  float gk = 0.f;
  if (lane < K) {
    rk = row_of[(int64_t)s * K + lane];
    if (rk < 0 || rk >= R) rk = -1;
    gk = gates[(int64_t)s * K + lane];
  }
  __amdgpu_buffer_rsrc_t rs[KT];
  float g[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const int r = __shfl(rk, k < K ? k : 0, kWave);
    g[k] = k < K ? __shfl(gk, k, kWave) : 0.f;
    rs[k] = row_rsrc<BF16>(y, r, H, k < K && r >= 0);
  }
  {
    const int p0 = (int)(item - (int64_t)s * nch) * kCombChunk + lane;
    u32x4 w[kCombU][KT];
#pragma unroll
    for (int u = 0; u < kCombU; ++u)
#pragma unroll
      for (int k = 0; k < KT; ++k) w[u][k] = buf_load16(rs[k], (uint32_t)(p0 + 64 * u) * 16u);
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {
      const int p = p0 + 64 * u;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KT; ++k) {  // k order: the gates' order
        float v[8];
        PC::unpack(w[u][k], v);
#pragma unroll
        for (int i = 0; i < PC::kEl; ++i) acc[i] += g[k] * v[i];
      }
      if (p < pieces)
        __builtin_nontemporal_store(  // non-temporal: -7% at 384 experts
            PC::pack(acc), reinterpret_cast<u32x4*>(reinterpret_cast<char*>(out) +
                                                    ((int64_t)s * H + (int64_t)p * PC::kEl) * PC::kEb));
    }
  }
}

// K rounded up to a power of two (1..16) as a compile-time bound
template <template <bool, int> class Launch, bool BF16, typename... A>
static void with_kt(int K, A... args) {
  if (K <= 1) Launch<BF16, 1>::run(args...);
  else if (K <= 2) Launch<BF16, 2>::run(args...);
  else if (K <= 4) Launch<BF16, 4>::run(args...);
  else if (K <= 8) Launch<BF16, 8>::run(args...);
  else Launch<BF16, 16>::run(args...);
}

template <bool BF16, int KT>
struct CombineLaunch {
  static void run(const void* y, const int32_t* row_of, const float* gates, void* out, int64_t S,
                  int H, int K, int64_t R, hipStream_t s) {
    const int64_t items = S * ((H / Piece<BF16>::kEl + kCombChunk - 1) / kCombChunk);
    hipLaunchKernelGGL((combine_kernel<BF16, KT>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0,
                       s, y, row_of, gates, out, (int)S, H, K, R);
  }
};

void launch_combine(const void* y, const int32_t* row_of, const float* gates, void* out, int64_t S,
                    int H, int K, int64_t R, bool bf16, hipStream_t s) {
  if (S <= 0) return;
  TimedLaunch tl("combine", s);
  if (bf16) with_kt<CombineLaunch, true>(K, y, row_of, gates, out, S, H, K, R, s);
  else with_kt<CombineLaunch, false>(K, y, row_of, gates, out, S, H, K, R, s);
}

// combine_bwd: one block per token, one wavefront per 128-piece column chunk
// (up to kCbWaves; wider rows give a wavefront several chunks).  Each
// wavefront writes its chunk of dy and sums its part of every <dout, y[row]>;
// the parts meet in LDS and wavefront 0 adds them in wavefront order, then
// finishes the gate and logit gradients.
constexpr int kCbWaves = 8;

static int combine_bwd_waves(int H, int piece_el) {
  const int nch = (H / piece_el + kCombChunk - 1) / kCombChunk;
  return nch < 1 ? 1 : (nch > kCbWaves ? kCbWaves : nch);
}

template <bool BF16, int KT, bool RAW>
__global__ __launch_bounds__(64 * kCbWaves) void combine_bwd_kernel(
    const void* __restrict__ dout, const void* __restrict__ y, const int32_t* __restrict__ row_of,
    const int32_t* __restrict__ idx, const float* __restrict__ gates,
    const float* __restrict__ logits, void* __restrict__ dy, float* __restrict__ dgates,
    float* __restrict__ dlogits, float* __restrict__ dl_row, int S, int H, int E, int K,
    int64_t R) {
  using PC = Piece<BF16>;
  __shared__ float part[kCbWaves][KT];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int s = blockIdx.x;
  int rk = -1, ek = -1;
  float gk = 0.f;
  if (lane < K) {
    rk = row_of[(int64_t)s * K + lane];
    if (rk < 0 || rk >= R) rk = -1;
    ek = idx[(int64_t)s * K + lane];
    gk = gates[(int64_t)s * K + lane];
  }
  __amdgpu_buffer_rsrc_t rs[KT];
  int rows[KT];
  float g[KT], dot[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    rows[k] = k < K ? __shfl(rk, k, kWave) : -1;
    g[k] = k < K ? __shfl(gk, k, kWave) : 0.f;
    dot[k] = 0.f;
    rs[k] = row_rsrc<BF16>(y, rows[k], H, rows[k] >= 0);
  }
  const __amdgpu_buffer_rsrc_t rd = row_rsrc<BF16>(dout, s, H, true);
  const int pieces = H / PC::kEl;
  for (int p0 = w * kCombChunk + lane; p0 < pieces; p0 += nw * kCombChunk) {
    u32x4 wd[kCombU], wv[kCombU][KT];
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {
      wd[u] = buf_load16(rd, (uint32_t)(p0 + 64 * u) * 16u);
#pragma unroll
      for (int k = 0; k < KT; ++k) wv[u][k] = buf_load16(rs[k], (uint32_t)(p0 + 64 * u) * 16u);
    }
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {
      const int p = p0 + 64 * u;
      float d[8];
      PC::unpack(wd[u], d);
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        float v[8], o[8];
        PC::unpack(wv[u][k], v);
#pragma unroll
        for (int i = 0; i < PC::kEl; ++i) {
          dot[k] += d[i] * v[i];
          o[i] = g[k] * d[i];
        }
        if (rows[k] >= 0 && p < pieces)
          *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dy) +
                                    ((int64_t)rows[k] * H + (int64_t)p * PC::kEl) * PC::kEb) =
              PC::pack(o);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    if (k < K) {
      const float t = wave_sum(dot[k]);
      if (lane == 0) part[w][k] = t;
    }
  }
  __syncthreads();
  if (w != 0) return;
  float my_dg = 0.f;
  if (lane < K)
    for (int ww = 0; ww < nw; ++ww) my_dg += part[ww][lane];
  const float inner = wave_sum(lane < K ? gk * my_dg : 0.f);  // sum_j g_j dg_j
  int ee[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) ee[k] = k < K ? __shfl(ek, k, kWave) : -1;
  if constexpr (!RAW) {
    // Renormalised softmax over the chosen experts: dl_k = g_k (dg_k - sum_j g_j dg_j),
    // zero off the chosen experts.
    const float my_dl = gk * (my_dg - inner);
    if (lane < K) {
      dgates[(int64_t)s * K + lane] = my_dg;
      if (rk >= 0) dl_row[rk] = my_dl;
    }
    float dd[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) dd[k] = __shfl(my_dl, k < K ? k : 0, kWave);
    for (int e = lane; e < E; e += 64) {
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < KT; ++k)
        if (ee[k] == e) v = dd[k];
      dlogits[(int64_t)s * E + e] = v;
    }
  } else {
    // Softmax over all E experts, the chosen probabilities used as gates:
    // dl_e = p_e (dp_e - sum_j g_j dg_j) with dp_e = dg_k where e = idx_k,
    // else 0; p from the token's logits row (max-shifted, as the router).
    const float* lrow = logits + (int64_t)s * E;
    float m = -INFINITY;
    for (int e = lane; e < E; e += 64) m = fmaxf(m, lrow[e]);
    m = wave_max_f32(m);
    float z = 0.f;
    for (int e = lane; e < E; e += 64) z += expf(lrow[e] - m);
    const float rz = 1.0f / wave_sum(z);
    float dgk[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) dgk[k] = __shfl(my_dg, k < K ? k : 0, kWave);
    if (lane < K) dgates[(int64_t)s * K + lane] = my_dg;
    for (int e = lane; e < E; e += 64) {
      float dp = 0.f;
#pragma unroll
      for (int k = 0; k < KT; ++k)
        if (ee[k] == e) dp = dgk[k];
      dlogits[(int64_t)s * E + e] = expf(lrow[e] - m) * rz * (dp - inner);
    }
  }
}

template <bool BF16, int KT>
struct CombineBwdLaunch {
  static void run(const void* dout, const void* y, const int32_t* row_of, const int32_t* idx,
                  const float* gates, const float* logits, void* dy, float* dgates,
                  float* dlogits, float* dl_row, int64_t S, int H, int E, int K, int64_t R,
                  hipStream_t s) {
    const int nw = combine_bwd_waves(H, Piece<BF16>::kEl);
    if (logits)
      hipLaunchKernelGGL((combine_bwd_kernel<BF16, KT, true>), dim3((unsigned)S), dim3(64 * nw),
                         0, s, dout, y, row_of, idx, gates, logits, dy, dgates, dlogits, dl_row,
                         (int)S, H, E, K, R);
    else
      hipLaunchKernelGGL((combine_bwd_kernel<BF16, KT, false>), dim3((unsigned)S), dim3(64 * nw),
                         0, s, dout, y, row_of, idx, gates, logits, dy, dgates, dlogits, dl_row,
                         (int)S, H, E, K, R);
  }
};

void launch_combine_bwd(const void* dout, const void* y, const int32_t* row_of,
                        const int32_t* idx, const float* gates, const float* logits, void* dy,
                        float* dgates, float* dlogits, float* dl_row, int64_t S, int H, int E,
                        int K, int64_t R, bool bf16, hipStream_t s) {
  if (S <= 0) return;
  TimedLaunch tl("combine_bwd", s);
  if (bf16)
    with_kt<CombineBwdLaunch, true>(K, dout, y, row_of, idx, gates, logits, dy, dgates, dlogits,
                                    dl_row, S, H, E, K, R, s);
  else
    with_kt<CombineBwdLaunch, false>(K, dout, y, row_of, idx, gates, logits, dy, dgates, dlogits,
                                     dl_row, S, H, E, K, R, s);
}

template <bool BF16, int KT>
__global__ __launch_bounds__(256) void dx_kernel(const void* __restrict__ dxd,
                                                 const int32_t* __restrict__ row_of,
                                                 const int32_t* __restrict__ idx,
                                                 const float* __restrict__ dlogits,
                                                 const void* __restrict__ wgT,
                                                 void* __restrict__ dx, int S, int H, int E, int K,
                                                 int64_t R) {
  using PC = Piece<BF16>;
  const int lane = threadIdx.x & 63;
  const int pieces = H / PC::kEl;
  const int nch = (pieces + kCombChunk - 1) / kCombChunk;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)S * nch) return;
  const int s = (int)(item / nch);
  int rk = -1, ek = -1;
  float dk = 0.f;
  if (lane < K) {
    rk = row_of[(int64_t)s * K + lane];
    if (rk < 0 || rk >= R) rk = -1;
    ek = idx[(int64_t)s * K + lane];
    if (ek < 0 || ek >= E) ek = -1;
    else dk = dlogits[(int64_t)s * E + ek];
  }
  __amdgpu_buffer_rsrc_t rr[KT], re[KT];
  float dl[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const int r = k < K ? __shfl(rk, k, kWave) : -1;
    const int ex = k < K ? __shfl(ek, k, kWave) : -1;
    dl[k] = k < K ? __shfl(dk, k, kWave) : 0.f;
    rr[k] = row_rsrc<BF16>(dxd, r, H, r >= 0);
    re[k] = row_rsrc<BF16>(wgT, ex, H, ex >= 0);
  }
  {
    const int p0 = (int)(item - (int64_t)s * nch) * kCombChunk + lane;
    u32x4 wr[kCombU][KT], we[kCombU][KT];
#pragma unroll
    for (int u = 0; u < kCombU; ++u)
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        wr[u][k] = buf_load16(rr[k], (uint32_t)(p0 + 64 * u) * 16u);
        we[u][k] = buf_load16(re[k], (uint32_t)(p0 + 64 * u) * 16u);
      }
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {
      const int p = p0 + 64 * u;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KT; ++k) {  // the K dispatched rows, in k order
        float v[8];
        PC::unpack(wr[u][k], v);
#pragma unroll
        for (int i = 0; i < PC::kEl; ++i) acc[i] += v[i];
      }
#pragma unroll
      for (int k = 0; k < KT; ++k) {  // then the router term, in k order
        float v[8];
        PC::unpack(we[u][k], v);
#pragma unroll
        for (int i = 0; i < PC::kEl; ++i) acc[i] += dl[k] * v[i];
      }
      if (p < pieces)
        *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dx) +
                                  ((int64_t)s * H + (int64_t)p * PC::kEl) * PC::kEb) = PC::pack(acc);
    }
  }
}

template <bool BF16, int KT>
struct DxLaunch {
  static void run(const void* dxd, const int32_t* row_of, const int32_t* idx, const float* dlogits,
                  const void* wgT, void* dx, int64_t S, int H, int E, int K, int64_t R,
                  hipStream_t s) {
    const int64_t items = S * ((H / Piece<BF16>::kEl + kCombChunk - 1) / kCombChunk);
    hipLaunchKernelGGL((dx_kernel<BF16, KT>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s,
                       dxd, row_of, idx, dlogits, wgT, dx, (int)S, H, E, K, R);
  }
};

void launch_dx(const void* dxd, const int32_t* row_of, const int32_t* idx, const float* dlogits,
               const void* wgT, void* dx, int64_t S, int H, int E, int K, int64_t R, bool bf16,
               hipStream_t s) {
  if (S <= 0) return;
  TimedLaunch tl("dispatch_bwd_dx", s);
  if (bf16) with_kt<DxLaunch, true>(K, dxd, row_of, idx, dlogits, wgT, dx, S, H, E, K, R, s);
  else with_kt<DxLaunch, false>(K, dxd, row_of, idx, dlogits, wgT, dx, S, H, E, K, R, s);
}

// Router-weight gradient, balanced over skewed experts.  Each expert's rows
// are cut into items of about rb rows, at most 64 per expert (a hot
// expert's items grow instead), with one table entry per item built on the
// device from cu_seqlens, so no host sync.  Block (item, 2048-column chunk)
// sums dl_row[r] * xd[r, h..h+8) over the item's rows in row order into an
// fp32 partial; the reduce adds each expert's items in item order
// (deterministic) and writes dWg [H, E] through an LDS transpose so both the
// partial reads and the dWg writes are contiguous.
constexpr int kDwgMaxItems = 64;

__global__ __launch_bounds__(1024) void dwg_items_kernel(const int32_t* __restrict__ cu, int E,
                                                         int R, int rb, int max_items,
                                                         int4* __restrict__ items,
                                                         int32_t* __restrict__ estart) {
  __shared__ int sh[1024];
  const int e = threadIdx.x;
  // rows outside [0, R) of a malformed cu_seqlens are never visited
  const int r0 = e < E ? min(max(cu[e], 0), R) : 0;
  const int c = e < E ? max(0, min(cu[e + 1], R) - r0) : 0;
  // at most kDwgMaxItems items per expert (a hot expert's items grow
  // instead), so the reduce never walks more than that many partials
  const int nt = min((c + rb - 1) / rb, kDwgMaxItems);
  const int rpi = nt > 0 ? (c + nt - 1) / nt : 0;  // rows per item
  sh[e] = nt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = e >= o ? sh[e - o] : 0;
    __syncthreads();
    sh[e] += add;
    __syncthreads();
  }
  const int start = sh[e] - nt, total = sh[1023];
  for (int t = 0; t < nt && start + t < max_items; ++t)
    items[start + t] = make_int4(e, r0 + t * rpi, min(rpi, c - t * rpi), 0);
  if (e < E) estart[e] = min(start, max_items);
  if (e == 0) estart[E] = min(total, max_items);
}

template <bool BF16>
__global__ __launch_bounds__(256) void dwg_partial_kernel(const void* __restrict__ x,
                                                          const int32_t* __restrict__ tok_of,
                                                          const int4* __restrict__ items,
                                                          const int32_t* __restrict__ estart,
                                                          const float* __restrict__ dl_row,
                                                          float* __restrict__ part, int H, int E,
                                                          int S) {
  // row r of the expert's rows is token tok_of[r] of x (the same bits as
  // the dispatched row): x is 1/K of the dispatched rows' bytes, so the K
  // reads of each token mostly hit the last-level cache (measured at 384
  // experts, top-8: 195 -> 115 us against reading the dispatched rows).  A
  // token index outside [0, S) (a corrupted tok_of) reads nothing and adds
  // zero.
  const int it = blockIdx.x;
  if (it >= estart[E]) return;
  const int h = blockIdx.y * 2048 + threadIdx.x * 8;
  if (h >= H) return;
  const int4 item = items[it];
  const int r0 = item.y, n = item.z;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int r = 0;
  for (; r + 4 <= n; r += 4) {  // four rows in flight per step; sums stay in row order
    float v[4][8], d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tok_of[r0 + r + j];
      const bool ok = (unsigned)t < (unsigned)S;
      d[j] = ok ? dl_row[r0 + r + j] : 0.f;
      load8<BF16>(x, (int64_t)(ok ? t : 0) * H + h, v[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += d[j] * v[j][i];
  }
  for (; r < n; ++r) {
    float v[8];
    const int t = tok_of[r0 + r];
    const bool ok = (unsigned)t < (unsigned)S;
    const float d = ok ? dl_row[r0 + r] : 0.f;
    load8<BF16>(x, (int64_t)(ok ? t : 0) * H + h, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += d * v[i];
  }
  float* o = part + (size_t)it * H + h;
  *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// Block (64 columns h, 16 experts): 256 threads each sum 4 columns of one
// expert over its items, then write 4 experts of one column.
__global__ __launch_bounds__(256) void dwg_reduce_kernel(const float* __restrict__ part,
                                                         const int32_t* __restrict__ estart,
                                                         float* __restrict__ dWg, int H, int E,
                                                         int accum) {
  __shared__ float tile[16][65];
  const int h0 = blockIdx.x * 64, e0 = blockIdx.y * 16;
  const int t = threadIdx.x;
  {
    const int el = t >> 4, hs = (t & 15) * 4, e = e0 + el, h = h0 + hs;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (e < E && h < H) {
      const int i0 = estart[e], i1 = estart[e + 1];
      for (int i = i0; i < i1; ++i) {
        const float4 p = *reinterpret_cast<const float4*>(part + (size_t)i * H + h);
        v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
      }
    }
    tile[el][hs] = v.x; tile[el][hs + 1] = v.y; tile[el][hs + 2] = v.z; tile[el][hs + 3] = v.w;
  }
  __syncthreads();
  const int hl = t >> 2, es = (t & 3) * 4, h = h0 + hl;
  if (h >= H) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + es + j;
    if (e >= E) break;
    float* o = dWg + (int64_t)h * E + e;
    *o = accum ? *o + tile[es + j][hl] : tile[es + j][hl];
  }
}

void launch_dwg(const void* x, const int32_t* tok_of, int64_t S, const int32_t* cu,
                const float* dl_row, float* dWg,
                const WsLayout& L, char* ws, int64_t R, int H, int E, bool accum, bool bf16,
                hipStream_t s) {
  int4* items = reinterpret_cast<int4*>(ws + L.dwg_items);
  int32_t* estart = reinterpret_cast<int32_t*>(ws + L.dwg_estart);
  float* part = reinterpret_cast<float*>(ws + L.dwg_part);
  {
    TimedLaunch tl("router_dWg_items", s);
    hipLaunchKernelGGL(dwg_items_kernel, dim3(1), dim3(1024), 0, s, cu, E, (int)R, L.dwg_rb,
                       L.dwg_max_items, items, estart);
  }
  if (L.dwg_max_items > 0) {
    TimedLaunch tl("router_dWg_partial", s);
    dim3 grid(L.dwg_max_items, (H + 2047) / 2048);
    if (bf16)
      hipLaunchKernelGGL(dwg_partial_kernel<true>, grid, dim3(256), 0, s, x, tok_of, items, estart,
                         dl_row, part, H, E, (int)S);
    else
      hipLaunchKernelGGL(dwg_partial_kernel<false>, grid, dim3(256), 0, s, x, tok_of, items,
                         estart, dl_row, part, H, E, (int)S);
  }
  {
    TimedLaunch tl("router_dWg_reduce", s);
    hipLaunchKernelGGL(dwg_reduce_kernel, dim3((H + 63) / 64, (E + 15) / 16), dim3(256), 0, s, part,
                       estart, dWg, H, E, accum ? 1 : 0);
  }
}

// ------------------------------------------- router backward, raw softmax --
// Raw softmax gates (the MoE/MoD framework page's routing/gating item read
// literally: a softmax over the experts, the chosen probabilities used as
// gates without renormalisation).  Every expert's logit then has a gradient,
// so the router terms are dense products over all E experts:
//   dx[s]  = sum_k dxd[row_of[s*K+k]] + sum_e dl[s,e] Wg[:, e]
//   dWg    = x^T dl
// Both are fp32 FMA tiles through LDS (E is small next to H: the products
// are 2 S H E flops, a few percent of the expert GEMMs).

// Block: 64 tokens x 256 columns; thread (ty, tx) holds tokens 8 ty .. 8 ty + 7
// and columns 8 tx .. 8 tx + 7 (64 fp32 FMAs per four LDS reads); experts in
// chunks of 16 through LDS (dl as [e][token], the row-major transposed router
// weight as [e][column]).
template <bool BF16, int KT>
__global__ __launch_bounds__(256) void dx_dense_kernel(const void* __restrict__ dxd,
                                                       const int32_t* __restrict__ row_of,
                                                       const float* __restrict__ dlogits,
                                                       const void* __restrict__ wgT,
                                                       void* __restrict__ dx, int S, int H, int E,
                                                       int K, int64_t R) {
  constexpr int TS = 64, TH = 256, TE = 16;
  __shared__ __attribute__((aligned(16))) float sd[TE][TS];
  __shared__ __attribute__((aligned(16))) float sw[TE][TH];
  const int s0 = blockIdx.x * TS, h0 = blockIdx.y * TH;
  const int tid = threadIdx.x, tx = tid & 31, ty = tid >> 5;
  float acc[8][8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = 0.f;
  for (int e0 = 0; e0 < E; e0 += TE) {
    for (int i = tid; i < TS * TE; i += 256) {
      const int t = i / TE, e = i % TE;
      sd[e][t] = (s0 + t < S && e0 + e < E) ? dlogits[(int64_t)(s0 + t) * E + e0 + e] : 0.f;
    }
    for (int i = tid; i < TE * TH / 8; i += 256) {
      const int e = i / (TH / 8), c = (i % (TH / 8)) * 8;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (e0 + e < E && h0 + c < H) load8<BF16>(wgT, (int64_t)(e0 + e) * H + h0 + c, v);
      *reinterpret_cast<float4*>(&sw[e][c]) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(&sw[e][c + 4]) = make_float4(v[4], v[5], v[6], v[7]);
    }
    __syncthreads();
#pragma unroll 2
    for (int e = 0; e < TE; ++e) {
      const float4 w0 = *reinterpret_cast<const float4*>(&sw[e][8 * tx]);
      const float4 w1 = *reinterpret_cast<const float4*>(&sw[e][8 * tx + 4]);
      const float4 d0 = *reinterpret_cast<const float4*>(&sd[e][8 * ty]);
      const float4 d1 = *reinterpret_cast<const float4*>(&sd[e][8 * ty + 4]);
      const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      const float d[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = fmaf(d[j], w[i], acc[j][i]);
    }
    __syncthreads();
  }
  const int h = h0 + 8 * tx;
  if (h >= H) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = s0 + 8 * ty + j;
    if (t >= S) continue;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KT; ++k) {  // the K dispatched rows, in k order
      if (k >= K) break;
      const int r = row_of[(int64_t)t * K + k];
      if (r < 0 || r >= R) continue;
      float u[8];
      load8<BF16>(dxd, (int64_t)r * H + h, u);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += u[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] += acc[j][i];  // then the router term
    store8<BF16>(dx, (int64_t)t * H + h, v);
  }
}

template <bool BF16, int KT>
struct DxDenseLaunch {
  static void run(const void* dxd, const int32_t* row_of, const float* dlogits, const void* wgT,
                  void* dx, int64_t S, int H, int E, int K, int64_t R, hipStream_t s) {
    hipLaunchKernelGGL((dx_dense_kernel<BF16, KT>), dim3((unsigned)((S + 63) / 64), (H + 255) / 256),
                       dim3(256), 0, s, dxd, row_of, dlogits, wgT, dx, (int)S, H, E, K, R);
  }
};

void launch_dx_dense(const void* dxd, const int32_t* row_of, const float* dlogits,
                     const void* wgT, void* dx, int64_t S, int H, int E, int K, int64_t R,
                     bool bf16, hipStream_t s) {
  if (S <= 0) return;
  TimedLaunch tl("dispatch_bwd_dx", s);
  if (bf16) with_kt<DxDenseLaunch, true>(K, dxd, row_of, dlogits, wgT, dx, S, H, E, K, R, s);
  else with_kt<DxDenseLaunch, false>(K, dxd, row_of, dlogits, wgT, dx, S, H, E, K, R, s);
}

// dWg partials: block (256 columns h, 32 experts, token slice z); thread
// (ty, tx) holds experts 4 ty .. 4 ty + 3 of columns 8 tx .. 8 tx + 7 (32 fp32
// FMAs per three LDS reads), summing the slice's tokens in order;
// part[z][h][e] (e over epad).
template <bool BF16>
__global__ __launch_bounds__(256) void dwg_dense_kernel(const void* __restrict__ x,
                                                        const float* __restrict__ dlogits,
                                                        float* __restrict__ part, int S, int H,
                                                        int E, int epad, int per_split) {
  constexpr int TS = 32, TH = 256, TE = 32;
  __shared__ __attribute__((aligned(16))) float sx[TS][TH];
  __shared__ __attribute__((aligned(16))) float sd[TS][TE];
  const int h0 = blockIdx.x * TH, e0 = blockIdx.y * TE, z = blockIdx.z;
  const int s_lo = z * per_split, s_hi = min(S, s_lo + per_split);
  const int tid = threadIdx.x, tx = tid & 31, ty = tid >> 5;
  float acc[4][8];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[q][i] = 0.f;
  for (int t0 = s_lo; t0 < s_hi; t0 += TS) {
    for (int i = tid; i < TS * TH / 8; i += 256) {
      const int t = i / (TH / 8), c = (i % (TH / 8)) * 8;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (t0 + t < s_hi && h0 + c < H) load8<BF16>(x, (int64_t)(t0 + t) * H + h0 + c, v);
      *reinterpret_cast<float4*>(&sx[t][c]) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(&sx[t][c + 4]) = make_float4(v[4], v[5], v[6], v[7]);
    }
    for (int i = tid; i < TS * TE; i += 256) {
      const int t = i / TE, e = i % TE;
      sd[t][e] = (t0 + t < s_hi && e0 + e < E) ? dlogits[(int64_t)(t0 + t) * E + e0 + e] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int t = 0; t < TS; ++t) {
      const float4 w0 = *reinterpret_cast<const float4*>(&sx[t][8 * tx]);
      const float4 w1 = *reinterpret_cast<const float4*>(&sx[t][8 * tx + 4]);
      const float4 dq = *reinterpret_cast<const float4*>(&sd[t][4 * ty]);
      const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      const float d[4] = {dq.x, dq.y, dq.z, dq.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[q][i] = fmaf(d[q], w[i], acc[q][i]);
    }
    __syncthreads();
  }
  const int h = h0 + 8 * tx;
  if (h >= H) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = e0 + 4 * ty + q;
    if (e >= epad) continue;
    float* o = part + ((size_t)z * H + h) * epad + e;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[(size_t)i * epad] = acc[q][i];
  }
}

// dWg[h][e] = (old value under accumulate) + sum over token slices, in order.
__global__ __launch_bounds__(256) void dwg_dense_reduce_kernel(const float* __restrict__ part,
                                                               float* __restrict__ dWg, int H,
                                                               int E, int epad, int nsplit,
                                                               int accum) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)H * E) return;
  const int h = (int)(i / E), e = (int)(i % E);
  float v = 0.f;
  for (int z = 0; z < nsplit; ++z) v += part[((size_t)z * H + h) * epad + e];
  dWg[i] = accum ? dWg[i] + v : v;
}

// token slices of the dense dWg: about 1024 blocks in all (several waves,
// so the last one is short), at least 32 tokens per slice, at most 64 slices
int dwg_dense_splits(int64_t S, int H, int epad) {
  const int64_t blocks = (int64_t)((H + 255) / 256) * ((epad + 31) / 32);
  int64_t n = (1024 + blocks - 1) / blocks;
  const int64_t chunks = (S + 31) / 32;
  if (n > chunks) n = chunks;
  return (int)(n < 1 ? 1 : (n > 64 ? 64 : n));
}

void launch_dwg_dense(const void* x, const float* dlogits, float* dWg, const WsLayout& L,
                      char* ws, int64_t S, int H, int E, bool accum, bool bf16, hipStream_t s) {
  float* part = reinterpret_cast<float*>(ws + L.dwg_dense_part);
  const int ns = dwg_dense_splits(S, H, L.epad);
  const int per = (int)(((S + ns - 1) / ns + 31) / 32 * 32);
  {
    TimedLaunch tl("router_dWg_partial", s);
    dim3 grid((H + 255) / 256, (L.epad + 31) / 32, ns);
    if (bf16)
      hipLaunchKernelGGL(dwg_dense_kernel<true>, grid, dim3(256), 0, s, x, dlogits, part, (int)S, H,
                         E, L.epad, per);
    else
      hipLaunchKernelGGL(dwg_dense_kernel<false>, grid, dim3(256), 0, s, x, dlogits, part, (int)S,
                         H, E, L.epad, per);
  }
  {
    TimedLaunch tl("router_dWg_reduce", s);
    const int64_t n = (int64_t)H * E;
    hipLaunchKernelGGL(dwg_dense_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       part, dWg, H, E, L.epad, ns, accum ? 1 : 0);
  }
}

}  // namespace moe

// Mixture-of-Depths step around the MoE layer (MoE/MoD framework page,
// "Comparison with alternatives": a share of the tokens skips the layer
// entirely, custom kernels at 50% sparsity; "Who the framework saves": the
// MoE + MoD combination).  Reading used (no formula on the page): a linear
// score r = <x, w_r>; per sequence the C best tokens (ties to the lower
// position) go through the MoE and come back as x + r*m; the rest are copied.
//
// gfx950 design: scores and every row copy run one wavefront per token with
// 16-byte pieces; the per-sequence selection runs in one 1024-thread block
// per sequence: 64-bit order keys (score bits : ~position) in LDS, a radix
// select of the C-th largest key (eight 8-bit digit passes), then a block
// scan of per-thread counts of the keys at or above it writes the kept
// positions out in ascending order.  The merge and the backward find a token's kept
// slot by binary search in its sequence's ascending keep list.
#include "dev_common.h"
#include "launch.h"
#include "moe.h"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void mod_score_kernel(const void* __restrict__ x,
                                                        const void* __restrict__ w_r,
                                                        float* __restrict__ r, int S, int H) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= S) return;
  float acc = 0.f;
  for (int c = lane * 8; c < H; c += 512) {
    float a[8], b[8];
    load8<BF16>(x, (int64_t)s * H + c, a);
    load8<BF16>(w_r, c, b);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += a[i] * b[i];
  }
  acc = wave_sum(acc);
  if (lane == 0) r[s] = acc;
}

// One block (1024 threads) per sequence; T <= 8192.  The (score, position)
// keys are unique (ties broken toward the earlier position), so the kept set
// is the keys at or above the C-th largest.  That key is found digit by digit
// from the top: eight passes of 8 bits, each an LDS histogram of the keys
// that still match the digits fixed so far, in which one wavefront finds the
// bin holding the C-th key from the top.  Every thread then counts the kept
// keys of its own run of positions, and a block scan writes them out in
// position order.  Measured at 4 sequences x 2048 tokens: 13 us against 38
// us for a bitonic sort of the keys (66 barrier rounds).
__global__ __launch_bounds__(1024) void mod_select_kernel(const float* __restrict__ r,
                                                          int32_t* __restrict__ keep, int T,
                                                          int C) {
  __shared__ uint64_t keys[8192];
  __shared__ int hist[256];
  __shared__ int scan[1024];
  __shared__ int pick[2];  // the digit of the C-th key, and the keys above its bin
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  for (int t = tid; t < T; t += 1024) keys[t] = topk_key(r[(int64_t)b * T + t], t);
  uint64_t prefix = 0, mask = 0;  // the digits fixed so far
  int need = C;                   // rank of the wanted key among the matching ones
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();  // (the first time also publishes the keys)
    for (int t = tid; t < T; t += 1024) {
      const uint64_t k = keys[t];
      if ((k & mask) == prefix) atomicAdd(&hist[(int)(k >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 4l .. 4l + 3; above = the matching keys in higher
      // bins, from a scan of the lane sums in reverse lane order
      int h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = hist[4 * lane + i];
      const int sum4 = h[0] + h[1] + h[2] + h[3];
      int v = __shfl(sum4, 63 - lane, 64);  // lane l: the sum of lane 63 - l
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
      }
      // v at lane l: the sum of lanes 63 - l .. 63; lanes above L: lane 62 - L
      const int up = __shfl(v, lane < 63 ? 62 - lane : 0, 64);
      int above = lane < 63 ? up : 0;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (above < need && above + h[i] >= need) {
          pick[0] = 4 * lane + i;
          pick[1] = above;
        }
        above += h[i];
      }
    }
    __syncthreads();
    need -= pick[1];
    prefix |= (uint64_t)pick[0] << shift;
    mask |= 255ull << shift;
  }
  // prefix is now the C-th largest key.  Each thread owns a run of
  // consecutive positions.
  const int per = (T + 1023) / 1024;
  const int t0 = tid * per;
  int cnt = 0;
  for (int i = 0; i < per; ++i) {
    const int t = t0 + i;
    if (t < T && keys[t] >= prefix) ++cnt;
  }
  scan[tid] = cnt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = tid >= o ? scan[tid - o] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  int j = scan[tid] - cnt;
  for (int i = 0; i < per; ++i) {
    const int t = t0 + i;
    if (t < T && keys[t] >= prefix) keep[(int64_t)b * C + j++] = b * T + t;
  }
}

// Copy rows: dst[j] = src[idx[j]] (one wavefront per row).
template <bool BF16>
__global__ __launch_bounds__(256) void gather_rows_kernel(const void* __restrict__ src,
                                                          const int32_t* __restrict__ idx,
                                                          void* __restrict__ dst, int n, int H) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= n) return;
  const int64_t s = idx[j];
  constexpr int kEl = BF16 ? 8 : 4;
  const u32x4* a = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(src) +
                                                  s * H * (BF16 ? 2 : 4));
  u32x4* d = reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dst) + (int64_t)j * H * (BF16 ? 2 : 4));
  for (int c = lane; c < H / kEl; c += 64) d[c] = a[c];
}

// Kept slot of token s, or -1 (binary search in its sequence's ascending list).
__device__ __forceinline__ int kept_slot(const int32_t* keep, int s, int T, int C) {
  const int b = s / T;
  int lo = 0, hi = C;
  const int32_t* kb = keep + (int64_t)b * C;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (kb[mid] < s) lo = mid + 1;
    else hi = mid;
  }
  return (lo < C && kb[lo] == s) ? b * C + lo : -1;
}

template <bool BF16>
__global__ __launch_bounds__(256) void mod_merge_kernel(const void* __restrict__ x,
                                                        const float* __restrict__ r,
                                                        const int32_t* __restrict__ keep,
                                                        const void* __restrict__ m,
                                                        void* __restrict__ out, int S, int T, int C,
                                                        int H) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= S) return;
  int j = lane == 0 ? kept_slot(keep, s, T, C) : 0;
  j = __shfl(j, 0, kWave);
  const float rs = r[s];
  for (int c = lane * 8; c < H; c += 512) {
    float v[8];
    load8<BF16>(x, (int64_t)s * H + c, v);
    if (j >= 0) {
      float mv[8];
      load8<BF16>(m, (int64_t)j * H + c, mv);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += rs * mv[i];
    }
    store8<BF16>(out, (int64_t)s * H + c, v);
  }
}

// Phase 1: dm[j] = r[s] dout[s]; dr[j] = <dout[s], m[j]> (one wavefront per kept slot).
template <bool BF16>
__global__ __launch_bounds__(256) void mod_bwd_slots_kernel(const float* __restrict__ r,
                                                            const int32_t* __restrict__ keep,
                                                            const void* __restrict__ m,
                                                            const void* __restrict__ dout,
                                                            void* __restrict__ dm,
                                                            float* __restrict__ dr, int n, int H) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= n) return;
  const int s = keep[j];
  const float rs = r[s];
  float acc = 0.f;
  for (int c = lane * 8; c < H; c += 512) {
    float d[8], mv[8], o[8];
    load8<BF16>(dout, (int64_t)s * H + c, d);
    load8<BF16>(m, (int64_t)j * H + c, mv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc += d[i] * mv[i];
      o[i] = rs * d[i];
    }
    store8<BF16>(dm, (int64_t)j * H + c, o);
  }
  acc = wave_sum(acc);
  if (lane == 0) dr[j] = acc;
}

// Phase 2: dx[s] = dout[s] + [kept](dxk[j] + dr[j] w_r).
template <bool BF16>
__global__ __launch_bounds__(256) void mod_bwd_dx_kernel(const void* __restrict__ dout,
                                                         const int32_t* __restrict__ keep,
                                                         const void* __restrict__ dxk,
                                                         const float* __restrict__ dr,
                                                         const void* __restrict__ w_r,
                                                         void* __restrict__ dx, int S, int T, int C,
                                                         int H) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= S) return;
  int j = lane == 0 ? kept_slot(keep, s, T, C) : 0;
  j = __shfl(j, 0, kWave);
  const float d = j >= 0 ? dr[j] : 0.f;
  for (int c = lane * 8; c < H; c += 512) {
    float v[8];
    load8<BF16>(dout, (int64_t)s * H + c, v);
    if (j >= 0) {
      float g[8], w[8];
      load8<BF16>(dxk, (int64_t)j * H + c, g);
      load8<BF16>(w_r, c, w);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += g[i] + d * w[i];
    }
    store8<BF16>(dx, (int64_t)s * H + c, v);
  }
}

// dw_r partials over slot ranges, then a fixed-order reduction.  128 row
// ranges (a block per range and 2048 columns: 256 blocks at H = 4096) and
// four rows in flight per thread: at the MoD block's 4096 kept tokens
// (H = 4096) the partial sums and their reduce take 21 us against 42 us with
// 64 ranges and one row in flight (that loop was bound by load latency).  A
// kept position outside [0, S) adds zero.
constexpr int kModSplits = kModSplitsHost;

template <bool BF16>
__global__ __launch_bounds__(256) void mod_dwr_partial_kernel(const void* __restrict__ x,
                                                              const int32_t* __restrict__ keep,
                                                              const float* __restrict__ dr,
                                                              float* __restrict__ part, int n,
                                                              int H, int S) {
  const int h = blockIdx.x * 2048 + threadIdx.x * 8;
  if (h >= H) return;
  const int sp = blockIdx.y;
  const int a = (int)((int64_t)n * sp / kModSplits), b = (int)((int64_t)n * (sp + 1) / kModSplits);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int j = a;
  for (; j + 4 <= b; j += 4) {  // sums stay in row order
    float v[4][8], d[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = keep[j + u];
      const bool ok = (unsigned)t < (unsigned)S;
      d[u] = ok ? dr[j + u] : 0.f;
      load8<BF16>(x, (int64_t)(ok ? t : 0) * H + h, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += d[u] * v[u][i];
  }
  for (; j < b; ++j) {
    const int t = keep[j];
    const bool ok = (unsigned)t < (unsigned)S;
    const float d = ok ? dr[j] : 0.f;
    float v[8];
    load8<BF16>(x, (int64_t)(ok ? t : 0) * H + h, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += d * v[i];
  }
  float* o = part + (size_t)sp * H + h;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = acc[i];
}

__global__ __launch_bounds__(256) void mod_dwr_reduce_kernel(const float* __restrict__ part,
                                                             float* __restrict__ dw_r, int H,
                                                             int accum) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= H) return;
  float v = 0.f;
  for (int sp = 0; sp < kModSplits; ++sp) v += part[(size_t)sp * H + h];
  dw_r[h] = accum ? dw_r[h] + v : v;
}

void launch_mod_select(int B, int T, int C, int H, bool bf16, const void* x, const void* w_r,
                       float* r, int32_t* keep, void* xk, hipStream_t s) {
  const int S = B * T;
  if (S <= 0) return;
  {
    TimedLaunch tl("mod_score", s);
    if (bf16)
      hipLaunchKernelGGL(mod_score_kernel<true>, dim3((S + 3) / 4), dim3(256), 0, s, x, w_r, r, S, H);
    else
      hipLaunchKernelGGL(mod_score_kernel<false>, dim3((S + 3) / 4), dim3(256), 0, s, x, w_r, r, S, H);
  }
  if (C <= 0) return;
  {
    TimedLaunch tl("mod_select", s);
    hipLaunchKernelGGL(mod_select_kernel, dim3(B), dim3(1024), 0, s, r, keep, T, C);
  }
  {
    TimedLaunch tl("mod_gather", s);
    const int n = B * C;
    if (bf16)
      hipLaunchKernelGGL(gather_rows_kernel<true>, dim3((n + 3) / 4), dim3(256), 0, s, x, keep, xk, n, H);
    else
      hipLaunchKernelGGL(gather_rows_kernel<false>, dim3((n + 3) / 4), dim3(256), 0, s, x, keep, xk, n, H);
  }
}

void launch_mod_merge(int B, int T, int C, int H, bool bf16, const void* x, const float* r,
                      const int32_t* keep, const void* m, void* out, hipStream_t s) {
  const int S = B * T;
  if (S <= 0) return;
  TimedLaunch tl("mod_merge", s);
  if (bf16)
    hipLaunchKernelGGL(mod_merge_kernel<true>, dim3((S + 3) / 4), dim3(256), 0, s, x, r, keep, m, out,
                       S, T, C, H);
  else
    hipLaunchKernelGGL(mod_merge_kernel<false>, dim3((S + 3) / 4), dim3(256), 0, s, x, r, keep, m,
                       out, S, T, C, H);
}

void launch_mod_backward(int B, int T, int C, int H, bool bf16, bool accum, const void* x,
                         const void* w_r, const float* r, const int32_t* keep, const void* m,
                         const void* dout, const void* dxk, void* dm, float* dr, void* dx,
                         float* dw_r, float* part, hipStream_t s) {
  const int S = B * T, n = B * C;
  if (!dxk) {
    if (n <= 0) return;
    TimedLaunch tl("mod_bwd_slots", s);
    if (bf16)
      hipLaunchKernelGGL(mod_bwd_slots_kernel<true>, dim3((n + 3) / 4), dim3(256), 0, s, r, keep, m,
                         dout, dm, dr, n, H);
    else
      hipLaunchKernelGGL(mod_bwd_slots_kernel<false>, dim3((n + 3) / 4), dim3(256), 0, s, r, keep, m,
                         dout, dm, dr, n, H);
    return;
  }
  if (S > 0) {
    TimedLaunch tl("mod_bwd_dx", s);
    if (bf16)
      hipLaunchKernelGGL(mod_bwd_dx_kernel<true>, dim3((S + 3) / 4), dim3(256), 0, s, dout, keep, dxk,
                         dr, w_r, dx, S, T, C, H);
    else
      hipLaunchKernelGGL(mod_bwd_dx_kernel<false>, dim3((S + 3) / 4), dim3(256), 0, s, dout, keep,
                         dxk, dr, w_r, dx, S, T, C, H);
  }
  {
    TimedLaunch tl("mod_bwd_dwr", s);
    dim3 grid((H + 2047) / 2048, kModSplits);
    if (bf16)
      hipLaunchKernelGGL(mod_dwr_partial_kernel<true>, grid, dim3(256), 0, s, x, keep, dr, part, n, H,
                         S);
    else
      hipLaunchKernelGGL(mod_dwr_partial_kernel<false>, grid, dim3(256), 0, s, x, keep, dr, part, n,
                         H, S);
    hipLaunchKernelGGL(mod_dwr_reduce_kernel, dim3((H + 255) / 256), dim3(256), 0, s, part, dw_r, H,
                       accum ? 1 : 0);
  }
}

}  // namespace moe

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
// gfx950 design: one wavefront per token; each lane streams 16-byte pieces
// (8 bf16) of the token's rows, accumulates in fp32 and writes 16-byte
// pieces, so every row read and write is a full coalesced 1-KB wave access.
// The router-weight gradient reduces over each expert's contiguous rows in
// row order (deterministic), split over row ranges into fp32 partials that a
// second kernel adds in split order.
#include "dev_common.h"
#include "launch.h"
#include "moe.h"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ gates,
                                                      void* __restrict__ out, int S, int H, int K,
                                                      int64_t R) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= S) return;
  int rk = -1;
  float gk = 0.f;
  if (lane < K) {
    rk = row_of[(int64_t)s * K + lane];
    if (rk < 0 || rk >= R) rk = -1;
    gk = gates[(int64_t)s * K + lane];
  }
  int rows[16];
  float g[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    rows[k] = __shfl(rk, k < K ? k : 0, kWave);
    g[k] = __shfl(gk, k < K ? k : 0, kWave);
  }
  for (int c = lane * 8; c < H; c += 64 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < K && rows[k] >= 0) {
        float v[8];
        load8<BF16>(y, (int64_t)rows[k] * H + c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += g[k] * v[i];
      }
    }
    store8<BF16>(out, (int64_t)s * H + c, acc);
  }
}

void launch_combine(const void* y, const int32_t* row_of, const float* gates, void* out, int64_t S,
                    int H, int K, int64_t R, bool bf16, hipStream_t s) {
  if (S <= 0) return;
  TimedLaunch tl("combine", s);
  const int blocks = (int)((S + 3) / 4);
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(blocks), dim3(256), 0, s, y, row_of, gates, out,
                       (int)S, H, K, R);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(blocks), dim3(256), 0, s, y, row_of, gates, out,
                       (int)S, H, K, R);
}

template <bool BF16>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const void* __restrict__ dout, const void* __restrict__ y, const int32_t* __restrict__ row_of,
    const int32_t* __restrict__ idx, const float* __restrict__ gates, void* __restrict__ dy,
    float* __restrict__ dgates, float* __restrict__ dlogits, float* __restrict__ dl_row, int S,
    int H, int E, int K, int64_t R) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= S) return;
  int rk = -1, ek = -1;
  float gk = 0.f;
  if (lane < K) {
    rk = row_of[(int64_t)s * K + lane];
    if (rk < 0 || rk >= R) rk = -1;
    ek = idx[(int64_t)s * K + lane];
    gk = gates[(int64_t)s * K + lane];
  }
  int rows[16];
  float g[16], dot[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    rows[k] = __shfl(rk, k < K ? k : 0, kWave);
    g[k] = __shfl(gk, k < K ? k : 0, kWave);
    dot[k] = 0.f;
  }
  for (int c = lane * 8; c < H; c += 64 * 8) {
    float d[8];
    load8<BF16>(dout, (int64_t)s * H + c, d);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < K && rows[k] >= 0) {
        float v[8], o[8];
        load8<BF16>(y, (int64_t)rows[k] * H + c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dot[k] += d[i] * v[i];
          o[i] = g[k] * d[i];
        }
        store8<BF16>(dy, (int64_t)rows[k] * H + c, o);
      }
    }
  }
  float my_dg = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if (k < K) {
      const float t = wave_sum(dot[k]);
      if (lane == k) my_dg = t;
    }
  }
  // Renormalised softmax over the chosen experts: dl_k = g_k (dg_k - sum_j g_j dg_j).
  const float inner = wave_sum(lane < K ? gk * my_dg : 0.f);
  const float my_dl = gk * (my_dg - inner);
  if (lane < K) {
    dgates[(int64_t)s * K + lane] = my_dg;
    if (rk >= 0) dl_row[rk] = my_dl;
  }
  // Dense logit-gradient row: zero off the chosen experts.
  int ee[16];
  float dd[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    ee[k] = __shfl(ek, k < K ? k : 0, kWave);
    dd[k] = __shfl(my_dl, k < K ? k : 0, kWave);
  }
  for (int e = lane; e < E; e += 64) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k < K && ee[k] == e) v = dd[k];
    dlogits[(int64_t)s * E + e] = v;
  }
}

void launch_combine_bwd(const void* dout, const void* y, const int32_t* row_of,
                        const int32_t* idx, const float* gates, void* dy, float* dgates,
                        float* dlogits, float* dl_row, int64_t S, int H, int E, int K, int64_t R,
                        bool bf16, hipStream_t s) {
  if (S <= 0) return;
  TimedLaunch tl("combine_bwd", s);
  const int blocks = (int)((S + 3) / 4);
  if (bf16)
    hipLaunchKernelGGL(combine_bwd_kernel<true>, dim3(blocks), dim3(256), 0, s, dout, y, row_of,
                       idx, gates, dy, dgates, dlogits, dl_row, (int)S, H, E, K, R);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<false>, dim3(blocks), dim3(256), 0, s, dout, y, row_of,
                       idx, gates, dy, dgates, dlogits, dl_row, (int)S, H, E, K, R);
}

template <bool BF16>
__global__ __launch_bounds__(256) void dx_kernel(const void* __restrict__ dxd,
                                                 const int32_t* __restrict__ row_of,
                                                 const int32_t* __restrict__ idx,
                                                 const float* __restrict__ dlogits,
                                                 const void* __restrict__ wgT,
                                                 void* __restrict__ dx, int S, int H, int E, int K,
                                                 int64_t R) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= S) return;
  int rk = -1, ek = -1;
  float dk = 0.f;
  if (lane < K) {
    rk = row_of[(int64_t)s * K + lane];
    if (rk < 0 || rk >= R) rk = -1;
    ek = idx[(int64_t)s * K + lane];
    if (ek < 0 || ek >= E) ek = -1;
    else dk = dlogits[(int64_t)s * E + ek];
  }
  int rows[16], ex[16];
  float dl[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    rows[k] = __shfl(rk, k < K ? k : 0, kWave);
    ex[k] = __shfl(ek, k < K ? k : 0, kWave);
    dl[k] = __shfl(dk, k < K ? k : 0, kWave);
  }
  for (int c = lane * 8; c < H; c += 64 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < K && rows[k] >= 0) {
        float v[8];
        load8<BF16>(dxd, (int64_t)rows[k] * H + c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
      }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < K && ex[k] >= 0) {
        float v[8];
        load8<BF16>(wgT, (int64_t)ex[k] * H + c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += dl[k] * v[i];
      }
    }
    store8<BF16>(dx, (int64_t)s * H + c, acc);
  }
}

void launch_dx(const void* dxd, const int32_t* row_of, const int32_t* idx, const float* dlogits,
               const void* wgT, void* dx, int64_t S, int H, int E, int K, int64_t R, bool bf16,
               hipStream_t s) {
  if (S <= 0) return;
  TimedLaunch tl("dispatch_bwd_dx", s);
  const int blocks = (int)((S + 3) / 4);
  if (bf16)
    hipLaunchKernelGGL(dx_kernel<true>, dim3(blocks), dim3(256), 0, s, dxd, row_of, idx, dlogits,
                       wgT, dx, (int)S, H, E, K, R);
  else
    hipLaunchKernelGGL(dx_kernel<false>, dim3(blocks), dim3(256), 0, s, dxd, row_of, idx, dlogits,
                       wgT, dx, (int)S, H, E, K, R);
}

// Partial router-weight gradient: block (e, h-chunk of 2048, split) sums
// dl_row[r] * xd[r, h..h+8) over its share of expert e's rows, in row order.
template <bool BF16>
__global__ __launch_bounds__(256) void dwg_partial_kernel(const void* __restrict__ xd,
                                                          const int32_t* __restrict__ cu,
                                                          const float* __restrict__ dl_row,
                                                          float* __restrict__ part, int H, int E,
                                                          int splits) {
  const int e = blockIdx.x, sp = blockIdx.z;
  const int h = blockIdx.y * 2048 + threadIdx.x * 8;
  if (h >= H) return;
  const int r0 = cu[e], n = cu[e + 1] - r0;
  const int a = r0 + (int)((int64_t)n * sp / splits), b = r0 + (int)((int64_t)n * (sp + 1) / splits);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = a; r < b; ++r) {
    const float d = dl_row[r];
    float v[8];
    load8<BF16>(xd, (int64_t)r * H + h, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += d * v[i];
  }
  float* o = part + ((size_t)sp * E + e) * H + h;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = acc[i];
}

__global__ __launch_bounds__(256) void dwg_reduce_kernel(const float* __restrict__ part,
                                                         float* __restrict__ dWg, int H, int E,
                                                         int splits, int accum) {
  const int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x;  // over [H, E], e fastest
  if (i >= (int64_t)H * E) return;
  const int h = (int)(i / E), e = (int)(i % E);
  float v = 0.f;
  for (int sp = 0; sp < splits; ++sp) v += part[((size_t)sp * E + e) * H + h];
  dWg[i] = accum ? dWg[i] + v : v;
}

void launch_dwg(const void* xd, const int32_t* cu, const float* dl_row, float* dWg,
                const WsLayout& L, char* ws, int64_t R, int H, int E, bool accum, bool bf16,
                hipStream_t s) {
  (void)R;
  float* part = reinterpret_cast<float*>(ws + L.dwg_part);
  dim3 grid(E, (H + 2047) / 2048, L.dwg_splits);
  {
    TimedLaunch tl("router_dWg_partial", s);
    if (bf16)
      hipLaunchKernelGGL(dwg_partial_kernel<true>, grid, dim3(256), 0, s, xd, cu, dl_row, part, H, E,
                         L.dwg_splits);
    else
      hipLaunchKernelGGL(dwg_partial_kernel<false>, grid, dim3(256), 0, s, xd, cu, dl_row, part, H,
                         E, L.dwg_splits);
  }
  {
    TimedLaunch tl("router_dWg_reduce", s);
    const int64_t n = (int64_t)H * E;
    hipLaunchKernelGGL(dwg_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part,
                       dWg, H, E, L.dwg_splits, accum ? 1 : 0);
  }
}

}  // namespace moe

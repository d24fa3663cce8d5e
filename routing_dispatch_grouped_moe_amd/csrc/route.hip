// Router: logits = x*Wg + bias, softmax, top-K and per-expert counts in one
// kernel ("What's in the box" routing/gating item of the MoE/MoD framework
// page: softmax over the experts and the top-k pick in a single launch; the
// T4 tuning page's router section: fuse softmax with top-k and keep the
// routing sparse).
//
// gfx950 design: a block owns 32 tokens.  The router GEMM runs on MFMA
// (v_mfma_f32_16x16x32_bf16) with both operands read straight from global
// memory in K-contiguous 16-byte fragments: x rows as they are, and the
// router weight through a transposed copy WgT [Epad, H] made once per call.
// Waves split the expert columns, or the H reduction when there are fewer
// than four 16-wide column blocks; partial sums meet in LDS in a fixed order.
// Top-K then runs one token per wavefront: each lane holds E/64 64-bit order
// keys (ordered logit bits : ~expert), and K rounds of a butterfly max pick
// the winners.  Counts come from an LDS histogram flushed with one atomic
// per (block, expert).
#include "dev_common.h"
#include "launch.h"
#include "moe.h"

namespace moe {

constexpr int kRouteBT = 32;

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

// WgT[e][h] = Wg[h][e] for e < E, zero rows for E <= e < epad.
template <bool BF16>
__global__ __launch_bounds__(256) void transpose_wg_kernel(const void* Wg, void* wgT, int H, int E,
                                                           int epad) {
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
    if (e < epad && h < H) store1<BF16>(wgT, (int64_t)e * H + h, tile[tx][i]);
  }
}

void launch_transpose_wg(const void* Wg, void* wgT, int H, int E, int epad, bool bf16,
                         hipStream_t s) {
  dim3 grid((H + 31) / 32, (epad + 31) / 32);
  TimedLaunch tl("route_wg_transpose", s);
  if (bf16)
    hipLaunchKernelGGL(transpose_wg_kernel<true>, grid, dim3(256), 0, s, Wg, wgT, H, E, epad);
  else
    hipLaunchKernelGGL(transpose_wg_kernel<false>, grid, dim3(256), 0, s, Wg, wgT, H, E, epad);
}

// Column blocks of 16 experts per wave and H slices per wave for a given Epad.
struct RouteSplit {
  int nwn, ks, ncb;
};
__host__ __device__ inline RouteSplit route_split(int epad, bool bf16) {
  RouteSplit r;
  const int nb = epad / 16;
  if (!bf16) { r.nwn = 4; r.ks = 1; r.ncb = 0; return r; }
  r.nwn = nb < 4 ? nb : 4;
  r.ks = 4 / r.nwn;
  r.ncb = (nb + r.nwn - 1) / r.nwn;
  return r;
}

template <bool BF16, int NCB>
__global__ __launch_bounds__(256) void route_kernel(const void* __restrict__ x,
                                                    const void* __restrict__ wgT,
                                                    const float* __restrict__ bias,
                                                    float* __restrict__ logits,
                                                    int32_t* __restrict__ idx,
                                                    float* __restrict__ gates,
                                                    int32_t* __restrict__ counts,
                                                    uint32_t* __restrict__ status, int S, int H,
                                                    int E, int epad, int K, int renorm) {
  extern __shared__ float part[];  // [ks][BT][epad] partial logits; slice 0 ends up holding logits
  __shared__ int hist[1024];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t0 = blockIdx.x * kRouteBT;
  const int nt = min(kRouteBT, S - t0);
  const RouteSplit sp = route_split(epad, BF16);

  for (int e = tid; e < E; e += 256) hist[e] = 0;

  if constexpr (BF16) {
    const int wn = w % sp.nwn, ks = w / sp.nwn;
    if (ks < sp.ks) {
      const int kslice = H / sp.ks, kbeg = ks * kslice;
      const uint16_t* xb = reinterpret_cast<const uint16_t*>(x) + (int64_t)t0 * H;
      const __amdgpu_buffer_rsrc_t rx = make_rsrc(xb, (uint32_t)nt * (uint32_t)H * 2u);
      const uint16_t* wb = reinterpret_cast<const uint16_t*>(wgT);
      f32x4 acc[2][NCB];
#pragma unroll
      for (int c = 0; c < NCB; ++c) acc[0][c] = acc[1][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r16 = lane & 15, kq = (lane >> 4) * 8;
      const uint32_t aoff0 = ((uint32_t)r16 * H + kq) * 2u;
      const uint32_t aoff1 = ((uint32_t)(r16 + 16) * H + kq) * 2u;
      for (int k = kbeg; k < kbeg + kslice; k += 32) {
        const u32x4 a0 = buf_load16(rx, aoff0 + k * 2u);
        const u32x4 a1 = buf_load16(rx, aoff1 + k * 2u);
#pragma unroll
        for (int c = 0; c < NCB; ++c) {
          const int nbk = wn + c * sp.nwn;
          if (nbk * 16 < epad) {
            const int n = nbk * 16 + r16;
            const u32x4 b = *reinterpret_cast<const u32x4*>(wb + (int64_t)n * H + k + kq);
            acc[0][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a0), __builtin_bit_cast(bf16x8, b), acc[0][c], 0, 0, 0);
            acc[1][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a1), __builtin_bit_cast(bf16x8, b), acc[1][c], 0, 0, 0);
          }
        }
      }
      // 16x16 MFMA result: lane holds column (lane % 16), rows 4*(lane/16) + i.
      float* pk = part + (size_t)ks * kRouteBT * epad;
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const int nbk = wn + c * sp.nwn;
        if (nbk * 16 < epad) {
          const int col = nbk * 16 + r16;
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) pk[(rb * 16 + (lane >> 4) * 4 + i) * epad + col] = acc[rb][c][i];
        }
      }
    }
  } else {
    // fp32 storage: plain dot products, one (token, expert) pair per thread.
    const float* xf = reinterpret_cast<const float*>(x);
    const float* wf = reinterpret_cast<const float*>(wgT);
    for (int i = tid; i < kRouteBT * E; i += 256) {
      const int t = i / E, e = i % E;
      float acc = 0.f;
      if (t < nt) {
        const float* xr = xf + (int64_t)(t0 + t) * H;
        const float* wr = wf + (int64_t)e * H;
        for (int h = 0; h < H; ++h) acc = fmaf(xr[h], wr[h], acc);
      }
      part[t * epad + e] = acc;
    }
  }
  __syncthreads();

  // Sum the H slices in slice order, add the bias, store the logits.
  uint32_t bad = 0;
  for (int i = tid; i < nt * E; i += 256) {
    const int t = i / E, e = i % E;
    float v = part[t * epad + e];
    for (int k2 = 1; k2 < sp.ks; ++k2) v += part[((size_t)k2 * kRouteBT + t) * epad + e];
    if (bias) v += bias[e];
    part[t * epad + e] = v;
    if (!isfinite(v)) bad = 1;
    if (logits) logits[(int64_t)(t0 + t) * E + e] = v;
  }
  if (bad) atomicOr(status, (uint32_t)MOE_DEV_NONFINITE_LOGIT);
  __syncthreads();

  // Top-K: one token per wavefront.
  const int nj = (E + 63) / 64;
  for (int t = w; t < nt; t += 4) {
    const float* lrow = part + t * epad;
    uint64_t keys[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = lane + 64 * j;
      keys[j] = (j < nj && e < E) ? topk_key(lrow[e], e) : 0ull;
    }
    float m = 0.f, my_l = 0.f;
    int my_e = -1;
    for (int k = 0; k < K; ++k) {
      uint64_t best = 0ull;
#pragma unroll
      for (int j = 0; j < 16; ++j) best = keys[j] > best ? keys[j] : best;
      best = wave_max_u64(best);
#pragma unroll
      for (int j = 0; j < 16; ++j)
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
  for (int e = tid; e < E; e += 256)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

template <bool BF16, int NCB>
static void route_launch_t(const void* x, const void* wgT, const float* bias, float* logits,
                           int32_t* idx, float* gates, int32_t* counts, uint32_t* status, int64_t S,
                           int H, int E, int epad, int K, bool renorm, hipStream_t s) {
  const RouteSplit sp = route_split(epad, BF16);
  const size_t lds = (size_t)sp.ks * kRouteBT * epad * sizeof(float);
  auto kern = route_kernel<BF16, NCB>;
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                        hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
    attr_set = true;
  }
  const int blocks = (int)((S + kRouteBT - 1) / kRouteBT);
  TimedLaunch tl("route", s);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), lds, s, x, wgT, bias, logits, idx, gates,
                     counts, status, (int)S, H, E, epad, K, renorm ? 1 : 0);
}

void launch_route(const void* x, const void* wgT, const float* bias, float* logits, int32_t* idx,
                  float* gates, int32_t* counts, uint32_t* status, int64_t S, int H, int E,
                  int epad, int K, bool renorm, bool bf16, hipStream_t s) {
  if (S <= 0) return;
  if (!bf16) {
    route_launch_t<false, 1>(x, wgT, bias, logits, idx, gates, counts, status, S, H, E, epad, K,
                             renorm, s);
    return;
  }
  const int ncb = route_split(epad, true).ncb;
#define ROUTE_CASE(N)                                                                          \
  if (ncb <= N) {                                                                              \
    route_launch_t<true, N>(x, wgT, bias, logits, idx, gates, counts, status, S, H, E, epad, K, \
                            renorm, s);                                                        \
    return;                                                                                    \
  }
  ROUTE_CASE(1) ROUTE_CASE(2) ROUTE_CASE(4) ROUTE_CASE(8) ROUTE_CASE(16)
#undef ROUTE_CASE
}

}  // namespace moe

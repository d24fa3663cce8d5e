// Dispatch: a stable counting sort of the (token, k) pairs by expert, and the
// copy of every token into its K expert rows (MoonEP page, step-by-step guide:
// the S*K-rows contract and dispatch returning cu_seqlens with each token
// written straight to its final row; MoE/MoD framework page, "What's in the
// box", dispatch/combine item).
//
// gfx950 design, three launches, no atomics on the row order:
//   1. bits:    one block per 256 tokens sets bit t of word [expert][t/32]
//               in an LDS bitmap for every pair (order-free ds_or), then
//               stores the bitmap and the per-expert popcounts.
//   2. scan:    one block turns the [block, expert] counts into cu_seqlens
//               and the first row of every (block, expert) run (the count
//               table staged in LDS by one round of coalesced loads).
//   3. scatter: one wavefront per token.  The rank of token s inside its
//               expert's run is the popcount of the bitmap bits below s, so
//               rows come out in ascending token order (bit-exact, unique).
//               The wavefront then streams x[s] once in 16-byte pieces and
//               writes each piece to the token's K rows (coalesced rows).
#include "dev_common.h"
#include "launch.h"
#include "moe.h"

namespace moe {

constexpr int kDispTok = kDispatchTokens;  // tokens per bitmap block (8 words of 32 bits)

__global__ __launch_bounds__(256) void dispatch_bits_kernel(const int32_t* __restrict__ idx,
                                                            uint32_t* __restrict__ bits_g,
                                                            int32_t* __restrict__ hist_g,
                                                            uint32_t* __restrict__ status, int S,
                                                            int E, int K) {
  extern __shared__ uint32_t bits[];  // [E][8]
  const int tid = threadIdx.x, b = blockIdx.x;
  for (int i = tid; i < E * 8; i += 256) bits[i] = 0u;
  __syncthreads();
  const int s = b * kDispTok + tid;
  uint32_t st = 0;
  if (s < S) {
    const uint32_t bit = 1u << (tid & 31);
    for (int k = 0; k < K; ++k) {
      const int e = idx[(int64_t)s * K + k];
      if (e < 0 || e >= E) { st |= MOE_DEV_BAD_EXPERT; continue; }
      const uint32_t old = atomicOr(&bits[e * 8 + (tid >> 5)], bit);
      if (old & bit) st |= MOE_DEV_DUP_EXPERT;
    }
  }
  if (st) atomicOr(status, st);
  __syncthreads();
  uint32_t* bo = bits_g + (size_t)b * E * 8;
  for (int i = tid; i < E * 8; i += 256) bo[i] = bits[i];
  for (int e = tid; e < E; e += 256) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) c += __popc(bits[e * 8 + w]);
    hist_g[(size_t)b * E + e] = c;
  }
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// Counts of every (block, expert) -> cu_seqlens and the first row of every
// (block, expert) run.  The [nb][E] count table is staged in LDS with its
// loads all in flight at once (up to sixteen per thread); thread e then
// scans its expert's column there, the expert totals are scanned with lane
// shuffles (per wavefront, then across the sixteen wavefront sums), and the
// bases leave as coalesced rows.  Tables larger than the LDS budget take the
// per-thread column walk through global memory.
constexpr int kScanLdsInts = 32768;  // 128 KB of dynamic LDS
constexpr int kScanLoads = 16;       // table loads in flight per thread

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ hist,
                                                             int32_t* __restrict__ base,
                                                             int32_t* __restrict__ cu, int nb,
                                                             int E) {
  extern __shared__ int tab[];  // [nb][E] when it fits
  __shared__ int start_e[1024];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool in_lds = (int64_t)nb * E <= kScanLdsInts;
  const int n = in_lds ? nb * E : 0;
  int tot = 0;
  if (in_lds) {
    for (int i0 = 0; i0 < n; i0 += kScanLoads * 1024) {
      int v[kScanLoads];
#pragma unroll
      for (int u = 0; u < kScanLoads; ++u) {
        const int i = i0 + u * 1024 + tid;
        v[u] = i < n ? hist[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < kScanLoads; ++u) {
        const int i = i0 + u * 1024 + tid;
        if (i < n) tab[i] = v[u];
      }
    }
    __syncthreads();
    if (tid < E) {
      // exclusive prefix of the column, in place
      for (int b = 0; b < nb; ++b) {
        const int c = tab[b * E + tid];
        tab[b * E + tid] = tot;
        tot += c;
      }
    }
  } else if (tid < E) {
    for (int b = 0; b < nb; ++b) {
      const int c = hist[(size_t)b * E + tid];
      base[(size_t)b * E + tid] = tot;
      tot += c;
    }
  }
  // exclusive prefix of the expert totals: per wavefront, then across them
  const int incl = wave_incl_scan(tid < E ? tot : 0);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();  // also publishes the scanned columns
  if (w == 0) {
    const int s16 = lane < 16 ? wsum[lane] : 0;
    const int i16 = wave_incl_scan(s16);
    if (lane < 16) wsum[lane] = i16 - s16;
  }
  __syncthreads();
  const int start = wsum[w] + incl - (tid < E ? tot : 0);
  if (tid < E) {
    cu[tid] = start;
    start_e[tid] = start;
  }
  if (tid == E - 1) cu[E] = start + tot;
  __syncthreads();
  if (in_lds) {
    for (int i = tid; i < n; i += 1024) base[i] = tab[i] + start_e[i % E];
  } else if (tid < E) {
    for (int b = 0; b < nb; ++b) base[(size_t)b * E + tid] += start;
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const void* __restrict__ x, const int32_t* __restrict__ idx,
    const uint32_t* __restrict__ bits, const int32_t* __restrict__ base,
    int32_t* __restrict__ row_of, int32_t* __restrict__ tok_of, void* __restrict__ xd, int S,
    int H, int E, int K) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= S) return;
  const int b = s / kDispTok, t = s % kDispTok, wi = t >> 5;
  int row = -1;
  if (lane < K) {
    const int e = idx[(int64_t)s * K + lane];
    if (e >= 0 && e < E) {
      const uint32_t* bw = bits + ((size_t)b * E + e) * 8;
      int r = base[(size_t)b * E + e];
      for (int w = 0; w < wi; ++w) r += __popc(bw[w]);
      r += __popc(bw[wi] & ((1u << (t & 31)) - 1u));
      row = r;
      tok_of[row] = s;
    }
    row_of[(int64_t)s * K + lane] = row;
  }
  int rows[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) rows[k] = __shfl(row, k < K ? k : 0, kWave);
  // four 16-byte pieces per lane in flight per iteration (the token's row is
  // read once, through a descriptor so pieces past the row end read zero)
  constexpr int kEl = BF16 ? 8 : 4;  // elements per 16-byte piece
  constexpr int kU = 4;
  const int pieces = H / kEl;
  const uint32_t row_bytes = (uint32_t)H * (BF16 ? 2u : 4u);
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(reinterpret_cast<const char*>(x) + (int64_t)s * row_bytes, row_bytes);
  for (int c0 = lane; c0 < pieces; c0 += 64 * kU) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = buf_load16(rx, (uint32_t)(c0 + 64 * u) * 16u);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < K && rows[k] >= 0) {
        u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<char*>(xd) +
                                              (int64_t)rows[k] * row_bytes);
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (c0 + 64 * u < pieces) dst[c0 + 64 * u] = v[u];
      }
    }
  }
}

void launch_dispatch(const void* x, const int32_t* idx, int32_t* cu, int32_t* row_of,
                     int32_t* tok_of, void* xd, const WsLayout& L, char* ws, uint32_t* status,
                     int64_t S, int H, int E, int K, bool bf16, hipStream_t s) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + L.bits);
  int32_t* hist = reinterpret_cast<int32_t*>(ws + L.hist);
  int32_t* base = reinterpret_cast<int32_t*>(ws + L.base);
  const int nb = L.nb;
  if (nb > 0) {
    TimedLaunch tl("dispatch_bits", s);
    hipLaunchKernelGGL(dispatch_bits_kernel, dim3(nb), dim3(256), (size_t)E * 8 * 4, s, idx, bits,
                       hist, status, (int)S, E, K);
  }
  {
    const size_t lds = (size_t)nb * E <= (size_t)kScanLdsInts ? (size_t)nb * E * 4 : 0;
    // a failure stays the thread's last HIP error (the entry point reports it)
    static bool attr = false;
    if (!attr)
      attr = hipFuncSetAttribute(reinterpret_cast<const void*>(dispatch_scan_kernel),
                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                 kScanLdsInts * 4) == hipSuccess;
    TimedLaunch tl("dispatch_scan", s);
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), lds, s, hist, base, cu, nb, E);
  }
  if (S > 0) {
    TimedLaunch tl("dispatch_scatter", s);
    const int blocks = (int)((S + 3) / 4);
    if (bf16)
      hipLaunchKernelGGL(dispatch_scatter_kernel<true>, dim3(blocks), dim3(256), 0, s, x, idx, bits,
                         base, row_of, tok_of, xd, (int)S, H, E, K);
    else
      hipLaunchKernelGGL(dispatch_scatter_kernel<false>, dim3(blocks), dim3(256), 0, s, x, idx,
                         bits, base, row_of, tok_of, xd, (int)S, H, E, K);
  }
}

}  // namespace moe

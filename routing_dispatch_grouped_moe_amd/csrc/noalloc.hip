// moe_dispatch_noalloc: moe_dispatch for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  It launches the same three dispatch kernels; their
// per-block bitmaps, counts and bases live in this file's scratch array
// instead of a caller workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "moe.h"

namespace moe {

// One copy per GPU, held until the process ends; every call on a GPU reuses
// its copy, so calls that overlap on one GPU race.  No region has to start at
// zero: the bitmap kernel clears its LDS table and writes every bitmap word and
// count of the call's blocks, the scan writes every base it later reads.
static __device__ __align__(256) unsigned char scratch[MOE_DISPATCH_NOALLOC_SCRATCH_BYTES];

// Bitmap / count / base regions from offset 0 of the scratch (L.total bytes).
static WsLayout scratch_layout(int64_t S, int E) {
  WsLayout L{};
  auto a256 = [](size_t v) { return (v + 255) & ~size_t(255); };
  L.nb = (int)((S + kDispatchTokens - 1) / kDispatchTokens);
  const size_t cells = (size_t)L.nb * E;
  size_t off = 0;
  L.status = off; off = a256(off + 4);
  L.bits = off; off = a256(off + cells * 8 * 4);
  L.hist = off; off = a256(off + cells * 4);
  L.base = off; off = a256(off + cells * 4);
  L.total = off;
  return L;
}

// In host code `scratch` names a host-side stand-in, not device memory: the
// array's address on the current device comes from the runtime, fetched once
// per device with that device current, and only that address is handed to
// kernels.  nullptr if the runtime cannot give it.
static char* scratch_ptr() {
  static std::mutex mu;
  static char* ptr[64] = {nullptr};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptr[dev] = reinterpret_cast<char*>(p);
  }
  return ptr[dev];
}

}  // namespace moe

using namespace moe;

extern "C" moe_status_t moe_dispatch_noalloc(const moe_dims_t* d, const void* x,
                                             const int32_t* topk_idx, int32_t* cu_seqlens,
                                             int32_t* row_of, int32_t* tok_of, void* xd,
                                             uint32_t* status, void* stream) {
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->S == 0) st = check_ptrs({cu_seqlens});  // only cu_seqlens (all zeros) is written
  else st = check_ptrs({x, topk_idx, cu_seqlens, row_of, tok_of, xd});
  if (st != MOE_OK) return st;
  if (status && (reinterpret_cast<uintptr_t>(status) & 3u)) return MOE_ERR_ALIGN;
  const WsLayout L = scratch_layout(d->S, d->E);
  if (L.total > (size_t)MOE_DISPATCH_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  char* w = scratch_ptr();
  if (!w) return MOE_ERR_HIP;
  // without a caller status word the kernels report into the scratch's own
  uint32_t* sw = status ? status : reinterpret_cast<uint32_t*>(w + L.status);
  launch_dispatch(x, topk_idx, cu_seqlens, row_of, tok_of, xd, L, w, sw, d->S, d->H, d->E, d->K,
                  d->dtype == MOE_BF16, reinterpret_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// C ABI of the MoE hot path: host-side validation, workspace layout, launch
// sequencing and the optional per-kernel timer.  Declarations and the
// contract of every entry point are in include/moe.h.
#include <hip/hip_runtime.h>

#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"
#include "moe.h"

namespace moe {

// ------------------------------------------------------------------ timer --
namespace {
struct TimerRec {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timer_on = false;
std::vector<TimerRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t pool_get() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

TimedLaunch::TimedLaunch(const char* name, hipStream_t s) : name_(name), stream_(s), slot_(nullptr) {
  if (!g_timer_on) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  TimerRec r{name, pool_get(), pool_get()};
  if (!r.a || !r.b) return;
  hipEventRecord(r.a, s);
  g_recs.push_back(r);
  slot_ = reinterpret_cast<void*>(g_recs.size());
}
TimedLaunch::~TimedLaunch() {
  if (!slot_) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  hipEventRecord(g_recs[reinterpret_cast<size_t>(slot_) - 1].b, stream_);
}

// ------------------------------------------------------------- workspace --
static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

WsLayout ws_layout(int64_t S, int H, int Hf, int E, int K, int dtype, uint32_t flags) {
  (void)Hf;
  WsLayout L{};
  const size_t esz = dtype == MOE_BF16 ? 2 : 4;
  const int64_t R = S * K;
  L.nb = (int)((S + 255) / 256);
  L.epad = (E + 15) / 16 * 16;
  // few rows per expert (small batches: the grouped GEMMs stream weights)
  // take 64-row M tiles, so that a tile is not mostly padding
  L.bm = (dtype == MOE_BF16 && R <= (int64_t)kFewRows * E) ? kGemmBMFew : kGemmBM;
  L.max_tiles = (int)((R + (int64_t)E * (L.bm - 1)) / L.bm);
  // dWg row items: about 2048 (item, 2048-column chunk) blocks whatever the skew
  const int hblocks = (H + 2047) / 2048;
  int rb = 16;
  while (rb < 256 && (int64_t)rb * 2 * 2048 <= R * hblocks) rb *= 2;
  L.dwg_rb = rb;
  L.dwg_max_items = (int)((R + (int64_t)E * (rb - 1)) / rb);
  size_t off = 0;
  L.status = off; off = align256(off + 4);
  L.wgT = off; off = align256(off + (size_t)L.epad * H * esz);
  L.bits = off; off = align256(off + (size_t)L.nb * E * 8 * 4);
  L.hist = off; off = align256(off + (size_t)L.nb * E * 4);
  L.base = off; off = align256(off + (size_t)L.nb * E * 4);
  L.tiles = off; off = align256(off + (size_t)std::max(L.max_tiles, 1) * 8);
  L.ntiles = off; off = align256(off + 8);
  L.eorder = off; off = align256(off + (size_t)(E + 1) * 4);
  L.dl_row = off; off = align256(off + (size_t)std::max<int64_t>(R, 1) * 4);
  L.dwg_items = off; off = align256(off + (size_t)std::max(L.dwg_max_items, 1) * 16);
  L.dwg_estart = off; off = align256(off + (size_t)(E + 1) * 4);
  L.dwg_part = off; off = align256(off + (size_t)std::max(L.dwg_max_items, 1) * H * 4);
  // the products with a bf16 store epilogue (down, dxd) split the tiles of a
  // partial last wave along K: at most 256 partial tiles, and at most eight
  // per tile the problem can have
  L.tail_items = (int)std::min<int64_t>(256, (int64_t)8 * L.max_tiles * ((H + 255) / 256));
  L.gemm_part = off; off = align256(off + (size_t)std::max(L.tail_items, 1) * 256 * 256 * 4);
  L.route_groups = (int)((S + 31) / 32);
  const bool tiled = route_tiled(S, E, dtype == MOE_BF16);
  L.route_parts = dtype == MOE_BF16 && !tiled ? route_parts(S, H, L.epad) : 1;
  L.route_part = off;
  if (tiled) {
    const int P = route_tiled_parts(S, H, E);
    off = align256(off + (P > 1 ? (size_t)P * S * E * 4 : 4));
  } else {
    off = align256(off + (L.route_parts > 1 ? (size_t)L.route_groups * L.route_parts * 32 * L.epad * 4 : 4));
  }
  L.route_tickets = off; off = align256(off + (size_t)std::max(L.route_groups, 1) * 4);
  L.route_logits = off;
  if (route_tiled(S, E, dtype == MOE_BF16)) off = align256(off + (size_t)S * E * 4);
  // raw softmax gates only: token-slice partials of the dense dWg
  L.dwg_dense_part = off;
  if (!(flags & MOE_F_RENORM))
    off = align256(off + (size_t)dwg_dense_splits(S, H, L.epad) * H * L.epad * 4);
  L.total = off;
  return L;
}

// -------------------------------------------------------------- validation --
static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status_t check_dims(const moe_dims_t* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (d->S < 0 || d->H <= 0 || d->Hf <= 0 || d->E <= 0 || d->K <= 0) return MOE_ERR_SHAPE;
  if (d->E > 1024 || d->K > 16 || d->K > d->E) return MOE_ERR_UNSUPPORTED;
  if (d->H % 128 || d->Hf % 128 || d->H > 65536 || d->Hf > 65536) return MOE_ERR_UNSUPPORTED;
  if (d->S * (int64_t)d->K >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  if (d->S * (int64_t)std::max(d->H, d->Hf) >= (int64_t(1) << 30)) return MOE_ERR_SHAPE;
  if ((int64_t)d->H * d->Hf >= (int64_t(1) << 30)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

moe_status_t check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return MOE_ERR_NULL;
  for (const void* p : ps)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

static moe_status_t check_ws(const moe_dims_t* d, const void* ws, size_t ws_bytes) {
  if (!ws) return MOE_ERR_NULL;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  if (ws_bytes < ws_layout(d->S, d->H, d->Hf, d->E, d->K, d->dtype, d->flags).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

static moe_status_t launched() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

#define MOE_TRY(expr)                 \
  do {                                \
    moe_status_t st_ = (expr);        \
    if (st_ != MOE_OK) return st_;    \
  } while (0)

extern "C" {

size_t moe_workspace_bytes(const moe_dims_t* d) {
  if (check_dims(d) != MOE_OK) return 0;
  return ws_layout(d->S, d->H, d->Hf, d->E, d->K, d->dtype, d->flags).total;
}

const char* moe_status_string(moe_status_t st) {
  // a C caller may pass any int: read the bits, not an enum value outside the
  // enumerators' range (undefined in C++)
  int32_t code;
  memcpy(&code, &st, sizeof code);
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "invalid shape";
    case MOE_ERR_DTYPE: return "invalid dtype";
    case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or mode";
    case MOE_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

moe_status_t moe_clear_status(void* ws, void* stream) {
  MOE_TRY(check_ptrs({ws}));
  launch_fill_i32(reinterpret_cast<int32_t*>(ws), 0, 1, reinterpret_cast<hipStream_t>(stream));
  return launched();
}

moe_status_t moe_read_status(const void* ws, uint32_t* status, void* stream) {
  MOE_TRY(check_ptrs({ws}));
  if (!status) return MOE_ERR_NULL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(status, ws, 4, hipMemcpyDeviceToHost, s) != hipSuccess) return MOE_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status_t moe_route(const moe_dims_t* d, const void* x, const void* Wg, const float* bias,
                       float* logits, int32_t* topk_idx, float* gates, int32_t* counts, void* ws,
                       size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  if (d->S == 0) {  // no tokens: only the counts are written (zeros)
    MOE_TRY(check_ptrs({counts}));
    launch_fill_i32(counts, 0, d->E, reinterpret_cast<hipStream_t>(stream));
    return launched();
  }
  MOE_TRY(check_ptrs({x, Wg, topk_idx, gates, counts}));
  if ((bias && !aligned16(bias)) || (logits && !aligned16(logits))) return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(d, ws, ws_bytes));
  const WsLayout L = ws_layout(d->S, d->H, d->Hf, d->E, d->K, d->dtype, d->flags);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = reinterpret_cast<char*>(ws);
  const bool bf16 = d->dtype == MOE_BF16;
  if (route_tiled(d->S, d->E, bf16)) {  // its GEMM launch also zeroes the counts
    float* lg = logits ? logits : reinterpret_cast<float*>(w + L.route_logits);
    launch_route_tiled(x, Wg, bias, lg, topk_idx, gates, counts,
                       reinterpret_cast<uint32_t*>(w + L.status), d->S, d->H, d->E, L.epad, d->K,
                       (d->flags & MOE_F_RENORM) != 0, reinterpret_cast<float*>(w + L.route_part),
                       s);
    return launched();
  }
  launch_fill_i32(counts, 0, d->E, s);
  int32_t* tickets = reinterpret_cast<int32_t*>(w + L.route_tickets);
  launch_transpose_wg(Wg, w + L.wgT, d->H, d->E, L.epad, bf16, bf16, tickets, L.route_groups,
                      s);
  launch_route(x, w + L.wgT, bias, logits, topk_idx, gates, counts,
               reinterpret_cast<uint32_t*>(w + L.status), d->S, d->H, d->E, L.epad, d->K,
               (d->flags & MOE_F_RENORM) != 0, bf16, L.route_parts,
               reinterpret_cast<float*>(w + L.route_part), tickets, s);
  return launched();
}

moe_status_t moe_load_stats(int32_t E, const int32_t* counts, float* stats, void* stream) {
  if (E < 1 || E > 1024) return MOE_ERR_SHAPE;
  if (!counts || !stats) return MOE_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(counts) & 3u) || (reinterpret_cast<uintptr_t>(stats) & 3u))
    return MOE_ERR_ALIGN;
  launch_load_stats(counts, E, stats, reinterpret_cast<hipStream_t>(stream));
  return launched();
}

moe_status_t moe_dispatch(const moe_dims_t* d, const void* x, const int32_t* topk_idx,
                          int32_t* cu_seqlens, int32_t* row_of, int32_t* tok_of, void* xd,
                          void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  if (d->S == 0) MOE_TRY(check_ptrs({cu_seqlens}));  // only cu_seqlens (all zeros) is written
  else MOE_TRY(check_ptrs({x, topk_idx, cu_seqlens, row_of, tok_of, xd}));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  const WsLayout L = ws_layout(d->S, d->H, d->Hf, d->E, d->K, d->dtype, d->flags);
  char* w = reinterpret_cast<char*>(ws);
  launch_dispatch(x, topk_idx, cu_seqlens, row_of, tok_of, xd, L, w,
                  reinterpret_cast<uint32_t*>(w + L.status), d->S, d->H, d->E, d->K,
                  d->dtype == MOE_BF16, reinterpret_cast<hipStream_t>(stream));
  return launched();
}

moe_status_t moe_ffn_up(const moe_dims_t* d, const void* xd, const int32_t* cu, const void* W1,
                        const void* W3, void* h1, void* h3, void* a, void* ws, size_t ws_bytes,
                        void* stream) {
  MOE_TRY(check_dims(d));
  if (d->S == 0) return MOE_OK;
  const bool keep_h = (d->flags & MOE_F_RECOMPUTE) == 0;
  MOE_TRY(check_ptrs({xd, cu, W1, W3, a}));
  if (keep_h) MOE_TRY(check_ptrs({h1, h3}));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  const WsLayout L = ws_layout(d->S, d->H, d->Hf, d->E, d->K, d->dtype, d->flags);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = reinterpret_cast<char*>(ws);
  const int64_t R = d->S * d->K;
  if (R > 0) {
    launch_tile_table(cu, d->E, L, w, false, s);
    launch_ffn_up(xd, cu, W1, W3, keep_h ? h1 : nullptr, keep_h ? h3 : nullptr, a, R, d->H, d->Hf,
                  d->E, L, w, d->dtype == MOE_BF16, s);
  }
  return launched();
}

moe_status_t moe_ffn_down(const moe_dims_t* d, const void* a, const int32_t* cu, const void* W2,
                          void* y, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  if (d->S == 0) return MOE_OK;
  MOE_TRY(check_ptrs({a, cu, W2, y}));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  const WsLayout L = ws_layout(d->S, d->H, d->Hf, d->E, d->K, d->dtype, d->flags);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = reinterpret_cast<char*>(ws);
  const int64_t R = d->S * d->K;
  if (R > 0) {
    launch_tile_table(cu, d->E, L, w, false, s);
    launch_ffn_down(a, cu, W2, y, R, d->H, d->Hf, d->E, L, w, d->dtype == MOE_BF16, s);
  }
  return launched();
}

moe_status_t moe_grouped_ffn(const moe_dims_t* d, const void* xd, const int32_t* cu,
                             const void* W1, const void* W3, const void* W2, void* h1, void* h3,
                             void* a, void* y, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  if (d->S == 0) return MOE_OK;
  const bool keep_h = (d->flags & MOE_F_RECOMPUTE) == 0;
  MOE_TRY(check_ptrs({xd, cu, W1, W3, W2, a, y}));
  if (keep_h) MOE_TRY(check_ptrs({h1, h3}));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  const WsLayout L = ws_layout(d->S, d->H, d->Hf, d->E, d->K, d->dtype, d->flags);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = reinterpret_cast<char*>(ws);
  const bool bf16 = d->dtype == MOE_BF16;
  const int64_t R = d->S * d->K;
  if (R > 0) {
    launch_tile_table(cu, d->E, L, w, false, s);
    launch_ffn_up(xd, cu, W1, W3, keep_h ? h1 : nullptr, keep_h ? h3 : nullptr, a, R, d->H, d->Hf,
                  d->E, L, w, bf16, s);
    launch_ffn_down(a, cu, W2, y, R, d->H, d->Hf, d->E, L, w, bf16, s);
  }
  return launched();
}

moe_status_t moe_combine(const moe_dims_t* d, const void* y, const int32_t* row_of,
                         const float* gates, void* out, void* stream) {
  MOE_TRY(check_dims(d));
  if (d->S == 0) return MOE_OK;
  MOE_TRY(check_ptrs({y, row_of, gates, out}));
  launch_combine(y, row_of, gates, out, d->S, d->H, d->K, d->S * d->K, d->dtype == MOE_BF16,
                 reinterpret_cast<hipStream_t>(stream));
  return launched();
}

moe_status_t moe_backward(const moe_dims_t* d, const moe_saved_t* sv, const void* dout, void* dx,
                          float* dWg, float* dW1, float* dW3, float* dW2, const moe_bwd_bufs_t* b,
                          void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  if (!sv || !b) return MOE_ERR_NULL;
  const bool raw = (d->flags & MOE_F_RENORM) == 0;
  if (d->S == 0) {  // no tokens: the weight gradients are zero (or unchanged when accumulating)
    MOE_TRY(check_ptrs({sv->cu_seqlens, dWg, dW1, dW3, dW2}));
    MOE_TRY(check_ws(d, ws, ws_bytes));
    const WsLayout L = ws_layout(0, d->H, d->Hf, d->E, d->K, d->dtype, d->flags);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool bf16 = d->dtype == MOE_BF16, accum = (d->flags & MOE_F_ACCUM_GRAD) != 0;
    launch_bwd_dw2(nullptr, nullptr, sv->cu_seqlens, nullptr, dW2, 0, d->H, d->Hf, d->E, accum,
                   bf16, s);
    launch_bwd_dw13(nullptr, nullptr, nullptr, sv->cu_seqlens, nullptr, dW1, dW3, 0, d->H, d->Hf, d->E,
                    accum, bf16, s);
    launch_dwg(nullptr, nullptr, 0, sv->cu_seqlens, nullptr, dWg, L, reinterpret_cast<char*>(ws), 0,
               d->H, d->E, accum, bf16, s);
    return launched();
  }
  const bool recompute = (d->flags & MOE_F_RECOMPUTE) != 0;
  MOE_TRY(check_ptrs({sv->x, sv->Wg, sv->W1, sv->W3, sv->W2, sv->xd, sv->a, sv->y, sv->topk_idx,
                      sv->gates, sv->cu_seqlens, sv->row_of, sv->tok_of}));
  if (!recompute) MOE_TRY(check_ptrs({sv->h1, sv->h3}));
  MOE_TRY(check_ptrs({dout, dx, dWg, dW1, dW3, dW2, b->dy, b->dh1, b->dh3, b->dxd, b->dgates,
                      b->dlogits}));
  if (raw) MOE_TRY(check_ptrs({sv->logits}));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  const WsLayout L = ws_layout(d->S, d->H, d->Hf, d->E, d->K, d->dtype, d->flags);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = reinterpret_cast<char*>(ws);
  const bool bf16 = d->dtype == MOE_BF16;
  const bool accum = (d->flags & MOE_F_ACCUM_GRAD) != 0;
  const int64_t R = d->S * d->K;
  const int H = d->H, Hf = d->Hf, E = d->E, K = d->K;
  float* dl_row = reinterpret_cast<float*>(w + L.dl_row);

  launch_combine_bwd(dout, sv->y, sv->row_of, sv->topk_idx, sv->gates, raw ? sv->logits : nullptr,
                     b->dy, b->dgates, b->dlogits, dl_row, d->S, H, E, K, R, bf16, s);
  if (R > 0) {
    launch_tile_table(sv->cu_seqlens, E, L, w, true, s);
    const void* h1 = sv->h1;
    const void* h3 = sv->h3;
    if (recompute) {
      // h1, h3 again from xd, straight into the dh1, dh3 buffers; the dA
      // epilogue then reads each tile's h1, h3 before writing its dh1, dh3 at
      // the same place (every element is read and written by one tile only)
      launch_ffn_up(sv->xd, sv->cu_seqlens, sv->W1, sv->W3, b->dh1, b->dh3, nullptr, R, H, Hf, E, L,
                    w, bf16, s);
      h1 = b->dh1;
      h3 = b->dh3;
    }
    launch_bwd_da(b->dy, sv->cu_seqlens, sv->W2, h1, h3, b->dh1, b->dh3, R, H, Hf, E, L, w, bf16, s);
  }
  // experts by descending row count (written by the tile table above)
  const int32_t* eorder = R > 0 ? reinterpret_cast<const int32_t*>(w + L.eorder) : nullptr;
  launch_bwd_dw2(sv->a, b->dy, sv->cu_seqlens, eorder, dW2, R, H, Hf, E, accum, bf16, s);
  if (R > 0)
    launch_bwd_dxd(b->dh1, b->dh3, sv->cu_seqlens, sv->W1, sv->W3, b->dxd, R, H, Hf, E, L, w, bf16,
                   s);
  launch_bwd_dw13(sv->xd, b->dh1, b->dh3, sv->cu_seqlens, eorder, dW1, dW3, R, H, Hf, E, accum,
                  bf16, s);
  launch_transpose_wg(sv->Wg, w + L.wgT, H, E, L.epad, bf16, false, nullptr, 0, s);
  if (raw) {
    launch_dx_dense(b->dxd, sv->row_of, b->dlogits, w + L.wgT, dx, d->S, H, E, K, R, bf16, s);
    launch_dwg_dense(sv->x, b->dlogits, dWg, L, w, d->S, H, E, accum, bf16, s);
  } else {
    launch_dx(b->dxd, sv->row_of, sv->topk_idx, b->dlogits, w + L.wgT, dx, d->S, H, E, K, R, bf16,
              s);
    launch_dwg(sv->x, sv->tok_of, d->S, sv->cu_seqlens, dl_row, dWg, L, w, R, H, E, accum, bf16, s);
  }
  return launched();
}

// ------------------------------------------------------------------- MoD --
static moe_status_t check_mod(int32_t B, int32_t T, int32_t C, int32_t H, int32_t dtype) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (B < 1 || T < 1 || C < 0 || H <= 0) return MOE_ERR_SHAPE;
  if (T > 8192 || C > T || H % 128) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)B * T * H >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

size_t moe_mod_workspace_bytes(int32_t H) {
  if (H <= 0) return 0;
  return (size_t)kModSplitsHost * H * 4;
}

moe_status_t moe_mod_select(int32_t B, int32_t T, int32_t C, int32_t H, int32_t dtype,
                            const void* x, const void* w_r, float* r, int32_t* keep_idx, void* xk,
                            void* stream) {
  MOE_TRY(check_mod(B, T, C, H, dtype));
  MOE_TRY(check_ptrs({x, w_r, r}));
  if (C > 0) MOE_TRY(check_ptrs({keep_idx, xk}));
  launch_mod_select(B, T, C, H, dtype == MOE_BF16, x, w_r, r, keep_idx, xk,
                    reinterpret_cast<hipStream_t>(stream));
  return launched();
}

moe_status_t moe_mod_merge(int32_t B, int32_t T, int32_t C, int32_t H, int32_t dtype,
                           const void* x, const float* r, const int32_t* keep_idx, const void* m,
                           void* out, void* stream) {
  MOE_TRY(check_mod(B, T, C, H, dtype));
  MOE_TRY(check_ptrs({x, r, out}));
  if (C > 0) MOE_TRY(check_ptrs({keep_idx, m}));
  launch_mod_merge(B, T, C, H, dtype == MOE_BF16, x, r, keep_idx, m, out,
                   reinterpret_cast<hipStream_t>(stream));
  return launched();
}

moe_status_t moe_mod_backward(int32_t B, int32_t T, int32_t C, int32_t H, int32_t dtype,
                              uint32_t flags, const void* x, const void* w_r, const float* r,
                              const int32_t* keep_idx, const void* m, const void* dout,
                              const void* dxk, void* dm, float* dr, void* dx, float* dw_r,
                              void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_mod(B, T, C, H, dtype));
  MOE_TRY(check_ptrs({x, w_r, r, dout}));
  if (C > 0) MOE_TRY(check_ptrs({keep_idx, m, dr}));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!dxk) {
    if (C > 0) MOE_TRY(check_ptrs({dm}));
    launch_mod_backward(B, T, C, H, dtype == MOE_BF16, false, x, w_r, r, keep_idx, m, dout, nullptr,
                        dm, dr, nullptr, nullptr, nullptr, s);
    return launched();
  }
  MOE_TRY(check_ptrs({dx, dw_r, ws}));
  if (ws_bytes < moe_mod_workspace_bytes(H)) return MOE_ERR_WORKSPACE;
  launch_mod_backward(B, T, C, H, dtype == MOE_BF16, (flags & MOE_F_ACCUM_GRAD) != 0, x, w_r, r,
                      keep_idx, m, dout, dxk, dm, dr, dx, dw_r, reinterpret_cast<float*>(ws), s);
  return launched();
}

// ------------------------------------------------------------------ timer --
void moe_timer_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timer_on = on != 0;
}

void moe_timer_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto& r : g_recs) {
    hipEventSynchronize(r.b);
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
}

int moe_timer_read(const char** names, double* total_ms, int64_t* launches, int cap) {
  std::lock_guard<std::mutex> lk(g_tmu);
  std::map<std::string, std::pair<double, int64_t>> acc;
  std::map<std::string, const char*> nm;
  for (auto& r : g_recs) {
    hipEventSynchronize(r.b);
    float ms = 0.f;
    hipEventElapsedTime(&ms, r.a, r.b);
    auto& v = acc[r.name];
    v.first += ms;
    v.second += 1;
    nm[r.name] = r.name;
  }
  int i = 0;
  for (auto& kv : acc) {
    if (i < cap) {
      if (names) names[i] = nm[kv.first];
      if (total_ms) total_ms[i] = kv.second.first;
      if (launches) launches[i] = kv.second.second;
    }
    ++i;
  }
  return i;
}

}  // extern "C"

// Internal host-side launch interface between the C ABI (api.hip) and the
// kernel translation units.  Not exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

#include "moe.h"

namespace moe {

// Host-side argument checks shared by the entry points (api.hip): the size
// contract of include/moe.h, and non-null 16-byte-aligned pointers.
moe_status_t check_dims(const moe_dims_t* d);
moe_status_t check_ptrs(std::initializer_list<const void*> ps);

// Kernel timer hook: when the library timer is on, launches are bracketed by
// events recorded on the launch stream.
struct TimedLaunch {
  TimedLaunch(const char* name, hipStream_t s);
  ~TimedLaunch();
  const char* name_;
  hipStream_t stream_;
  void* slot_;
};

// Workspace layout (bytes from the start of ws).  Every region is 256-byte aligned.
struct WsLayout {
  size_t status;      // uint32 device status word
  size_t wgT;         // [Epad, H] router weight transposed (dtype)
  size_t bits;        // dispatch: [nb, E, 8] uint32 token bitmaps (256 tokens per block)
  size_t hist;        // dispatch: [nb, E] int32 per-block counts
  size_t base;        // dispatch: [nb, E] int32 first row of each (block, expert)
  size_t tiles;       // grouped GEMM: [max_tiles] int2 (expert, first row) per M tile
  size_t ntiles;      // int32 number of valid M tiles, then int32 log2 of the M tiles per
                      // tile group of the M-grouped products (0, 1 or 2)
  size_t eorder;      // [E + 1] int32 experts by descending row count (ties: lower index
                      // first), then the count of them the weight gradients split by XCD
  size_t dl_row;      // [R] fp32 dlogit of each dispatched row
  size_t dwg_items;   // [dwg_max_items] int4 (expert, first row, rows, 0) row items of dWg
  size_t dwg_estart;  // [E+1] int32 first item of each expert (exclusive scan)
  size_t dwg_part;    // [dwg_max_items, H] fp32 partial router-weight gradient per item
  size_t gemm_part;   // [tail_items, 256 * 256] fp32 K-split partial tiles of the last GEMM wave
  size_t route_part;  // fp32 partial logits of a split router: [groups, route_parts, 32, epad]
                      // (fused), or [route_tiled_parts, S, E] (tiled)
  size_t route_tickets; // [groups] int32 parts finished per 32-token group
  size_t route_logits;  // [S, E] fp32 logits of the tiled router when the caller keeps none
  size_t dwg_dense_part; // [splits, H, epad] fp32 token-slice partials of the dense dWg (raw gates)
  size_t total;
  int nb;             // dispatch blocks of 256 tokens
  int epad;           // E rounded up to 16
  int max_tiles;      // upper bound on M tiles over all experts
  int bm;             // rows per M tile of the grouped GEMMs (kGemmBM or kGemmBMFew)
  int dwg_rb;         // rows per dWg item (a power of two, 16..256)
  int dwg_max_items;  // upper bound on dWg items over all experts
  int tail_items;     // capacity of gemm_part in partial tiles
  int route_groups;   // 32-token groups of the router
  int route_parts;    // K parts per group (1: no split)
};
// the layout depends on the flags: raw softmax gates add the dense dWg partials
WsLayout ws_layout(int64_t S, int H, int Hf, int E, int K, int dtype, uint32_t flags);

constexpr int kGemmBM = 256;   // M tile of the grouped GEMMs (rows per tile)
constexpr int kGemmBMFew = 64; // M tile when experts average at most kFewRows rows (bf16)
constexpr int kFewRows = 32;

void launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s);
void launch_fill_f32(float* p, float v, int64_t n, hipStream_t s);
// blocked: the bf16 router's K-blocked layout [H / 32][epad][32]; else [epad][H]
void launch_transpose_wg(const void* Wg, void* wgT, int H, int E, int epad, bool bf16,
                         bool blocked, int32_t* tickets, int ntickets, hipStream_t s);
// K parts per 32-token group of the bf16 router (1: no split)
int route_parts(int64_t S, int H, int epad);
// many experts and tokens: the router as a tiled GEMM into fp32 logits (the
// caller's, or the workspace's route_logits) plus a top-K launch; it reads Wg
// in its [H][E] layout (no transposed copy)
bool route_tiled(int64_t S, int E, bool bf16);
int route_tiled_parts(int64_t S, int H, int E);
// part: [route_tiled_parts, S, E] fp32 partial logits (used when there are
// several parts; null: one part)
void launch_route_tiled(const void* x, const void* Wg, const float* bias, float* logits,
                        int32_t* idx, float* gates, int32_t* counts, uint32_t* status, int64_t S,
                        int H, int E, int epad, int K, bool renorm, float* part, hipStream_t s);
void launch_route(const void* x, const void* wgT, const float* bias, float* logits, int32_t* idx,
                  float* gates, int32_t* counts, uint32_t* status, int64_t S, int H, int E, int epad,
                  int K, bool renorm, bool bf16, int nparts, float* rpart, int32_t* tickets,
                  hipStream_t s);

void launch_load_stats(const int32_t* counts, int E, float* stats, hipStream_t s);

// status: where the kernels OR their anomaly bits (the workspace's status word,
// or the caller's word for the allocation-free entry point)
void launch_dispatch(const void* x, const int32_t* idx, int32_t* cu, int32_t* row_of,
                     int32_t* tok_of, void* xd, const WsLayout& L, char* ws, uint32_t* status,
                     int64_t S, int H, int E, int K, bool bf16, hipStream_t s);
constexpr int kDispatchTokens = 256;  // tokens per dispatch bitmap block

// M tiles of every expert; with expert_order also the experts by descending
// row count into the eorder region (used by the weight-gradient products)
void launch_tile_table(const int32_t* cu, int E, const WsLayout& L, char* ws, bool expert_order,
                       hipStream_t s);

// Grouped GEMMs (see gemm.hip for the operand layouts).
void launch_ffn_up(const void* xd, const int32_t* cu, const void* W1, const void* W3, void* h1,
                   void* h3, void* a, int64_t R, int H, int Hf, int E, const WsLayout& L, char* ws,
                   bool bf16, hipStream_t s);
void launch_ffn_down(const void* a, const int32_t* cu, const void* W2, void* y, int64_t R, int H,
                     int Hf, int E, const WsLayout& L, char* ws, bool bf16, hipStream_t s);
void launch_bwd_da(const void* dy, const int32_t* cu, const void* W2, const void* h1,
                   const void* h3, void* dh1, void* dh3, int64_t R, int H, int Hf, int E,
                   const WsLayout& L, char* ws, bool bf16, hipStream_t s);
void launch_bwd_dxd(const void* dh1, const void* dh3, const int32_t* cu, const void* W1,
                    const void* W3, void* dxd, int64_t R, int H, int Hf, int E, const WsLayout& L,
                    char* ws, bool bf16, hipStream_t s);
// eorder: the experts in the order their tiles are dealt (the tile table's
// longest-first order), or nullptr for index order
void launch_bwd_dw2(const void* a, const void* dy, const int32_t* cu, const int32_t* eorder,
                    float* dW2, int64_t R, int H, int Hf, int E, bool accum, bool bf16,
                    hipStream_t s);
void launch_bwd_dw13(const void* xd, const void* dh1, const void* dh3, const int32_t* cu,
                     const int32_t* eorder, float* dW1, float* dW3, int64_t R, int H, int Hf,
                     int E, bool accum, bool bf16, hipStream_t s);

void launch_combine(const void* y, const int32_t* row_of, const float* gates, void* out, int64_t S,
                    int H, int K, int64_t R, bool bf16, hipStream_t s);
// logits [S, E] given: raw softmax gates (dlogits dense over all experts);
// nullptr: gates renormalised over the K chosen
void launch_combine_bwd(const void* dout, const void* y, const int32_t* row_of,
                        const int32_t* idx, const float* gates, const float* logits, void* dy,
                        float* dgates, float* dlogits, float* dl_row, int64_t S, int H, int E,
                        int K, int64_t R, bool bf16, hipStream_t s);
void launch_dx(const void* dxd, const int32_t* row_of, const int32_t* idx, const float* dlogits,
               const void* wgT, void* dx, int64_t S, int H, int E, int K, int64_t R, bool bf16,
               hipStream_t s);
// raw softmax gates: the router terms are dense over all experts
void launch_dx_dense(const void* dxd, const int32_t* row_of, const float* dlogits,
                     const void* wgT, void* dx, int64_t S, int H, int E, int K, int64_t R,
                     bool bf16, hipStream_t s);
int dwg_dense_splits(int64_t S, int H, int epad);
void launch_dwg_dense(const void* x, const float* dlogits, float* dWg, const WsLayout& L,
                      char* ws, int64_t S, int H, int E, bool accum, bool bf16, hipStream_t s);
void launch_dwg(const void* x, const int32_t* tok_of, int64_t S, const int32_t* cu,
                const float* dl_row, float* dWg,
                const WsLayout& L, char* ws, int64_t R, int H, int E, bool accum, bool bf16,
                hipStream_t s);

void launch_mod_select(int B, int T, int C, int H, bool bf16, const void* x, const void* w_r,
                       float* r, int32_t* keep, void* xk, hipStream_t s);
void launch_mod_merge(int B, int T, int C, int H, bool bf16, const void* x, const float* r,
                      const int32_t* keep, const void* m, void* out, hipStream_t s);
void launch_mod_backward(int B, int T, int C, int H, bool bf16, bool accum, const void* x,
                         const void* w_r, const float* r, const int32_t* keep, const void* m,
                         const void* dout, const void* dxk, void* dm, float* dr, void* dx,
                         float* dw_r, float* part, hipStream_t s);
constexpr int kModSplitsHost = 128;  // row splits of the MoD score-weight gradient

}  // namespace moe

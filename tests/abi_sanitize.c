/* Host driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of
   the library's C ABI (built and run by tests/test_abi_sanitize.py, CPU only).

   Every call here fails host-side validation before anything is launched,
   so no GPU is needed: invalid dims, null and misaligned pointers, short
   workspaces, sizes past the allocation-free dispatch's scratch, and the
   workspace sizing over random dims around every documented limit (its
   64-bit layout arithmetic is where overflow would show).  Exits non-zero on
   the first mismatch with the documented status; the sanitizers abort on any
   memory or undefined-behaviour error. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "moe.h"

static int fails = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "line %d: expectation failed: %s\n", __LINE__, #cond); \
      ++fails;                                                        \
    }                                                                 \
  } while (0)

#define FAKE ((void*)((uintptr_t)1 << 20))        /* aligned, never dereferenced */
#define MIS ((void*)(((uintptr_t)1 << 20) + 4))

static uint64_t rng_state = 11;
static uint64_t rng(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 2685821657736338717ull;
}

static moe_dims_t dims(int64_t S, int H, int Hf, int E, int K, int dtype, uint32_t flags) {
  moe_dims_t d;
  d.S = S; d.H = H; d.Hf = Hf; d.E = E; d.K = K; d.dtype = dtype; d.flags = flags;
  return d;
}

/* the size contract of include/moe.h */
static int expected(int64_t S, int64_t H, int64_t Hf, int64_t E, int64_t K, int dtype) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (S < 0 || H <= 0 || Hf <= 0 || E <= 0 || K <= 0) return MOE_ERR_SHAPE;
  if (E > 1024 || K > 16 || K > E) return MOE_ERR_UNSUPPORTED;
  if (H % 128 || Hf % 128 || H > 65536 || Hf > 65536) return MOE_ERR_UNSUPPORTED;
  const int64_t mx = H > Hf ? H : Hf;
  if (S * K >= ((int64_t)1 << 31) || S * mx >= ((int64_t)1 << 30) || H * Hf >= ((int64_t)1 << 30))
    return MOE_ERR_SHAPE;
  return MOE_OK;
}

int main(void) {
  // status strings
  for (int c = 0; c <= 8; ++c) EXPECT(moe_status_string((moe_status_t)c) != NULL);

  // route
  moe_dims_t d = dims(64, 128, 256, 8, 2, MOE_F32, MOE_F_RENORM);
  const size_t ws = moe_workspace_bytes(&d);
  EXPECT(ws > 0 && ws % 256 == 0);
  EXPECT(moe_route(&d, NULL, FAKE, NULL, NULL, FAKE, FAKE, FAKE, FAKE, ws, NULL) == MOE_ERR_NULL);
  EXPECT(moe_route(&d, FAKE, FAKE, NULL, NULL, MIS, FAKE, FAKE, FAKE, ws, NULL) == MOE_ERR_ALIGN);
  EXPECT(moe_route(&d, FAKE, FAKE, NULL, NULL, FAKE, FAKE, FAKE, FAKE, ws - 256, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_route(NULL, FAKE, FAKE, NULL, NULL, FAKE, FAKE, FAKE, FAKE, ws, NULL) == MOE_ERR_NULL);
  moe_dims_t dk = dims(64, 128, 256, 2, 3, MOE_F32, MOE_F_RENORM);
  EXPECT(moe_route(&dk, FAKE, FAKE, NULL, NULL, FAKE, FAKE, FAKE, FAKE, ws, NULL) == MOE_ERR_UNSUPPORTED);

  // dispatch, ffn, combine, backward
  moe_dims_t db = dims(64, 128, 256, 8, 2, MOE_BF16, MOE_F_RENORM);
  const size_t wsb = moe_workspace_bytes(&db);
  EXPECT(moe_dispatch(&db, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, wsb, NULL) == MOE_ERR_NULL);
  EXPECT(moe_grouped_ffn(&db, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, NULL) ==
         MOE_ERR_WORKSPACE);
  EXPECT(moe_ffn_up(&db, FAKE, FAKE, MIS, FAKE, FAKE, FAKE, FAKE, FAKE, wsb, NULL) == MOE_ERR_ALIGN);
  EXPECT(moe_ffn_down(&db, FAKE, NULL, FAKE, FAKE, FAKE, wsb, NULL) == MOE_ERR_NULL);
  EXPECT(moe_combine(&db, FAKE, FAKE, NULL, FAKE, NULL) == MOE_ERR_NULL);
  moe_saved_t sv;
  sv.x = sv.Wg = sv.W1 = sv.W3 = sv.W2 = sv.xd = sv.h1 = sv.h3 = sv.a = sv.y = FAKE;
  sv.topk_idx = sv.cu_seqlens = sv.row_of = sv.tok_of = (const int32_t*)FAKE;
  sv.gates = (const float*)FAKE;
  sv.logits = NULL;
  moe_bwd_bufs_t bb;
  bb.dy = bb.dh1 = bb.dh3 = bb.dxd = FAKE;
  bb.dgates = bb.dlogits = (float*)FAKE;
  float* F = (float*)FAKE;
  moe_dims_t draw = dims(64, 128, 256, 8, 2, MOE_BF16, 0);
  EXPECT(moe_backward(&draw, &sv, FAKE, FAKE, F, F, F, F, &bb, FAKE, wsb, NULL) == MOE_ERR_NULL);
  EXPECT(moe_backward(&db, NULL, FAKE, FAKE, F, F, F, F, &bb, FAKE, wsb, NULL) == MOE_ERR_NULL);
  EXPECT(moe_backward(&db, &sv, FAKE, FAKE, F, F, F, F, NULL, FAKE, wsb, NULL) == MOE_ERR_NULL);
  EXPECT(moe_backward(&db, &sv, FAKE, FAKE, F, F, F, F, &bb, FAKE, 16, NULL) == MOE_ERR_WORKSPACE);

  // load statistics, MoD
  EXPECT(moe_load_stats(0, NULL, NULL, NULL) == MOE_ERR_SHAPE);
  EXPECT(moe_load_stats(8, NULL, F, NULL) == MOE_ERR_NULL);
  EXPECT(moe_mod_select(4, 2048, 3000, 4096, 1, FAKE, FAKE, F, NULL, FAKE, NULL) ==
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_mod_merge(0, 2048, 1024, 4096, 1, FAKE, F, NULL, FAKE, FAKE, NULL) == MOE_ERR_SHAPE);
  EXPECT(moe_mod_backward(4, 2048, 1024, 4096, 1, 0, FAKE, FAKE, F, (const int32_t*)FAKE, FAKE, FAKE,
                          FAKE, FAKE, F, FAKE, F, FAKE, 16, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_mod_backward(4, 2048, 1024, 4096, 1, 0, FAKE, FAKE, F, NULL, FAKE, FAKE, FAKE, FAKE, F,
                          FAKE, F, FAKE, 1 << 30, NULL) == MOE_ERR_NULL);
  EXPECT(moe_mod_workspace_bytes(4096) > 0 && moe_mod_workspace_bytes(-1) == 0);

  // allocation-free dispatch: sizes past its scratch are refused before any device work
  moe_dims_t big = dims(26113, 128, 128, 1024, 2, MOE_BF16, MOE_F_RENORM);
  EXPECT(moe_dispatch_noalloc(&big, FAKE, FAKE, (int32_t*)FAKE,
                              (int32_t*)FAKE, (int32_t*)FAKE, FAKE,
                              NULL, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_dispatch_noalloc(&big, FAKE, NULL, NULL, NULL, NULL, FAKE, NULL, NULL) ==
         MOE_ERR_NULL);

  // random dims around every limit: workspace sizing and the documented status
    const int64_t Ss[] = {0, 1, 63, 8192, 1 << 20, 1 << 27, (int64_t)1 << 33, -1};
  const int Hs[] = {128, 256, 4096, 7168, 65536, 65536 + 128, 100, 0, -128};
  const int Hfs[] = {128, 1408, 2048, 14336, 65536, 131072, 200, 0};
  const int Es[] = {1, 8, 384, 1024, 1025, 0, -3};
  const int Ks[] = {1, 2, 8, 16, 17, 0};
  const int dts[] = {0, 1, 2, -1};
  const uint32_t fls[] = {MOE_F_RENORM, 0, MOE_F_RENORM | MOE_F_ACCUM_GRAD | MOE_F_RECOMPUTE};
  for (int it = 0; it < 4000; ++it) {
    moe_dims_t r = dims(Ss[rng() % 8], Hs[rng() % 9], Hfs[rng() % 8], Es[rng() % 7], Ks[rng() % 6],
                        dts[rng() % 4], fls[rng() % 3]);
    const int want = expected(r.S, r.H, r.Hf, r.E, r.K, r.dtype);
    const size_t nb = moe_workspace_bytes(&r);
    if (want == MOE_OK) {
      EXPECT(nb > 0 && nb % 256 == 0);
      EXPECT(moe_route(&r, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                       NULL) == MOE_ERR_NULL);
      EXPECT(moe_dispatch_noalloc(&r, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                  NULL) == MOE_ERR_NULL);
    } else {
      EXPECT(nb == 0);
      EXPECT(moe_route(&r, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                       NULL) == want);
      EXPECT(moe_combine(&r, NULL, NULL, NULL, NULL, NULL) == want);
      EXPECT(moe_backward(&r, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                          NULL, 0, NULL) == want);
    }
    if (fails > 20) break;
  }
  if (fails) {
    fprintf(stderr, "%d expectation(s) failed\n", fails);
    return 1;
  }
  printf("abi_sanitize: ok\n");
  return 0;
}

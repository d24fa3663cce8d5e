/*
 * moe.h - C ABI of the MI355X (gfx950) MoE-layer hot path.
 *
 * The layer: out[s] = sum_k g[s,k] * FFN_{idx[s,k]}(x[s]) with a softmax
 * router, top-K gating, dispatch of every (token, k) pair into contiguous
 * per-expert rows, a grouped SwiGLU FFN over one contiguous weight tensor per
 * projection, a gate-weighted combine, and the backward of all of it.
 *
 * Sources (the pages the method is described on):
 *   [FW]  "PyTorch MoE/MoD Training Framework: custom CUDA kernels, DeepSpeed
 *         and a 7x speed-up on T4" (ai-manual.ru)
 *   [MEP] "Moonshot AI opened MoonEP: training Mixture of Experts without GPU
 *         idling" (dzen.guru)
 *   [T4]  "MoE on T4: how to find and remove the bottlenecks" (ai-manual.ru)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a DEVICE pointer, row-major, densely packed,
 *    16-byte aligned.  The caller owns and allocates every buffer; the library
 *    never allocates or frees device memory and keeps no pointer after a call
 *    returns.  Buffers must stay alive until the work on `stream` completes.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues kernels on it; no call synchronises the device or the host.
 *  - The return value reports host-side argument validation (done before any
 *    launch: a call that returns an error has enqueued nothing) and launch
 *    errors (MOE_ERR_HIP).  Data-dependent anomalies found on the device
 *    (non-finite router logits, expert indices outside [0,E), an expert chosen
 *    twice by one token) are OR-ed into the 32-bit status word at the start
 *    of the workspace: read it with moe_read_status after synchronising.
 *  - Activations and weights are bf16 (MOE_BF16) or fp32 (MOE_F32); all
 *    accumulation is fp32; router logits, gates, their gradients and weight
 *    gradients are always fp32.  fp32 -> bf16 rounding is to nearest even.
 *  - Sizes: 1 <= K <= min(E, 16), 1 <= E <= 1024, 0 <= S, S*K < 2^31,
 *    H and Hf multiples of 128 (at most 65536), S*max(H,Hf) < 2^30 and
 *    H*Hf < 2^30 (each expert's rows and weights fit a 32-bit byte range).  Anything else returns
 *    MOE_ERR_UNSUPPORTED or MOE_ERR_SHAPE.  S = 0 is valid and enqueues only
 *    the work that clears outputs.
 *  - Thread safety: no mutable global state except the optional kernel timer
 *    (moe_timer_*) and idempotent per-device caches (the compute-unit count,
 *    kernel attributes).  Concurrent calls on different streams must use
 *    different workspaces.
 *  - Reproducibility: every reduction runs in a fixed order, so repeated
 *    calls on the same device give bit-identical results.  The products
 *    with a plain store epilogue (y of the expert FFN, dxd of its backward)
 *    split the tiles of a partial last wave of GEMM tiles along K and sum
 *    the fp32 parts in part order; the split depends on the device's
 *    compute-unit count, so devices of another size may round those
 *    outputs differently (fp32 summation order only).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be, or overflows */
  MOE_ERR_DTYPE = 3,       /* dtype is not MOE_F32 or MOE_BF16 */
  MOE_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = 5,   /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_UNSUPPORTED = 6, /* a size outside the supported range (see above) */
  MOE_ERR_HIP = 7          /* a kernel launch failed */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* dims.flags */
enum {
  MOE_F_RENORM = 1u << 0,     /* gates renormalised over the K chosen experts (Mixtral block) */
  MOE_F_ACCUM_GRAD = 1u << 1, /* weight gradients are added to (not written over) dW, dWg */
  MOE_F_RECOMPUTE = 1u << 3   /* h1, h3 are not kept: the forward writes only a, the backward
                                 recomputes h1, h3 into its dh1, dh3 buffers (see moe_backward) */
};

/* Device-side status bits (OR-ed into the workspace status word). */
enum {
  MOE_DEV_NONFINITE_LOGIT = 1u << 0, /* a router logit was NaN or infinite */
  MOE_DEV_BAD_EXPERT = 1u << 1,      /* a topk_idx entry was outside [0, E) */
  MOE_DEV_DUP_EXPERT = 1u << 2       /* a token listed the same expert twice */
};

typedef struct {
  int64_t S;     /* tokens entering the layer */
  int32_t H;     /* hidden size */
  int32_t Hf;    /* expert intermediate size (H' on the pages) */
  int32_t E;     /* experts, all resident on this GPU */
  int32_t K;     /* experts per token */
  int32_t dtype; /* moe_dtype_t of activations and weights */
  uint32_t flags;
} moe_dims_t;

/* Bytes of workspace every call with these dims needs (the same for all
 * entry points; dims.flags included: raw softmax gates need more for the
 * backward, so size with the flags the calls will carry).  Returns 0 for
 * invalid dims.  Its first 4 bytes are the
 * device status word, which accumulates across calls until cleared with
 * moe_clear_status (clear it once for a new workspace); the rest needs no
 * initialisation. */
size_t moe_workspace_bytes(const moe_dims_t* dims);

/* Enqueue a clear of the workspace status word on `stream`. */
moe_status_t moe_clear_status(void* ws, void* stream);

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status_t st);

/* Copy the device status word from `ws` into *status (synchronous on `stream`). */
moe_status_t moe_read_status(const void* ws, uint32_t* status, void* stream);

/*
 * moe_route - router projection, softmax and top-K gating.
 * [FW] "What's in the box", routing/gating item (softmax over the experts and
 * the top-k pick done in a single launch) and "Comparison with alternatives"
 * (wavefront-level primitives for top-k); [T4] "The router is the main
 * culprit" (fused softmax + top-k; keep the routing sparse).
 * Fewer than 256 experts, fp32, or E not a multiple of 8: one fused launch.
 * Otherwise a tiled GEMM writes fp32 logits (the H reduction cut into parts,
 * summed in a fixed order, when the tokens are few) and one launch does the
 * softmax, top-K, gates and counts.  Both give the same results to rounding
 * of the fp32 logits.
 *
 *   x        [S, H]   activations (dtype)
 *   Wg       [H, E]   router weight (dtype)
 *   bias     [E]      fp32 constant added to the logits before selection and
 *                     gates (no gradient); may be NULL
 *   logits   [S, E]   fp32 output, x*Wg + bias; may be NULL (not stored)
 *   topk_idx [S, K]   int32 output: chosen experts, best first; order key is
 *                     (fp32 logit descending, expert index ascending), -0 == +0,
 *                     NaN ranks last
 *   gates    [S, K]   fp32 output: softmax probability of each chosen expert,
 *                     divided by their sum when MOE_F_RENORM is set
 *   counts   [E]      int32 output: (token, k) pairs per expert (overwritten)
 */
moe_status_t moe_route(const moe_dims_t* dims, const void* x, const void* Wg, const float* bias,
                       float* logits, int32_t* topk_idx, float* gates, int32_t* counts,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * moe_dispatch - permute the (token, k) pairs into contiguous per-expert rows.
 * [MEP] guide: the fixed S*K-rows contract, and dispatch returning cu_seqlens
 * (offsets of each expert's active rows) with tokens written straight to
 * their final positions; [FW] "What's in the box", dispatch/combine item.
 *
 *   topk_idx   [S, K]  int32 input (from moe_route or the caller)
 *   cu_seqlens [E+1]   int32 output: cu[0]=0, cu[e+1]=cu[e]+count[e], cu[E]=S*K
 *   row_of     [S*K]   int32 output: row of pair p = s*K+k
 *   tok_of     [S*K]   int32 output: token of each row
 *   xd         [S*K,H] output (dtype): xd[row_of[s*K+k]] = x[s], bit for bit
 * Rows of one expert are in ascending token order (a stable counting sort),
 * so the permutation is unique.  Pairs with an expert outside [0,E) get
 * row_of = -1 and set MOE_DEV_BAD_EXPERT.
 */
moe_status_t moe_dispatch(const moe_dims_t* dims, const void* x, const int32_t* topk_idx,
                          int32_t* cu_seqlens, int32_t* row_of, int32_t* tok_of, void* xd,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * moe_dispatch_noalloc - moe_dispatch without a workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same inputs, outputs and results
 * (bit for bit) as moe_dispatch; the dispatch kernels' per-block bitmaps,
 * counts and bases live in a scratch array the library holds on each GPU it
 * runs on (MOE_DISPATCH_NOALLOC_SCRATCH_BYTES, kept until the process ends).
 * The call allocates nothing.
 *   status  optional device uint32: the MOE_DEV_* anomaly bits are OR-ed into
 *           it (it accumulates until the caller clears it); NULL: not reported
 * Limit: 256 + 40 * ceil(S / 256) * E bytes (each region rounded up to 256)
 * must fit the scratch, i.e. about ceil(S / 256) * E <= 104 800 (S up to
 * 26 112 at E = 1024, 69 888 at E = 384); larger sizes return
 * MOE_ERR_WORKSPACE before anything is launched.  Every call on one GPU reuses that GPU's
 * scratch: calls that overlap on one GPU (different streams or threads) race
 * and must be serialised by the caller.
 */
#define MOE_DISPATCH_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status_t moe_dispatch_noalloc(const moe_dims_t* dims, const void* x, const int32_t* topk_idx,
                                  int32_t* cu_seqlens, int32_t* row_of, int32_t* tok_of, void* xd,
                                  uint32_t* status, void* stream);

/*
 * moe_grouped_ffn - the grouped SwiGLU expert FFN over all experts' rows.
 * [T4] "RMSNorm, RoPE, SwiGLU" table, SwiGLU row (three matrix products);
 * [MEP] guide, weights step (one contiguous [E, H, H'] tensor per projection;
 * the grouped GEMM finds an expert's weights from its index alone).
 *
 *   xd         [R, H]      dispatched rows, R = S*K (dtype)
 *   cu_seqlens [E+1]       int32 row offsets (from moe_dispatch)
 *   W1, W3     [E, H, Hf]  gate and up projections (dtype)
 *   W2         [E, Hf, H]  down projection (dtype)
 *   h1, h3     [R, Hf]     outputs: xd*W1[e], xd*W3[e] (dtype; saved for backward);
 *                          not written, and may be NULL, under MOE_F_RECOMPUTE
 *   a          [R, Hf]     output: silu(h1)*h3, from the fp32 values (dtype)
 *   y          [R, H]      output: a*W2[e] (dtype)
 * Equivalent to moe_ffn_up followed by moe_ffn_down.
 */
moe_status_t moe_grouped_ffn(const moe_dims_t* dims, const void* xd, const int32_t* cu_seqlens,
                             const void* W1, const void* W3, const void* W2, void* h1, void* h3,
                             void* a, void* y, void* ws, size_t ws_bytes, void* stream);

/* The two halves of moe_grouped_ffn, for per-kernel measurement. */
moe_status_t moe_ffn_up(const moe_dims_t* dims, const void* xd, const int32_t* cu_seqlens,
                        const void* W1, const void* W3, void* h1, void* h3, void* a, void* ws,
                        size_t ws_bytes, void* stream);
moe_status_t moe_ffn_down(const moe_dims_t* dims, const void* a, const int32_t* cu_seqlens,
                          const void* W2, void* y, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine - gate-weighted sum of each token's K expert rows.
 * [FW] "What's in the box", dispatch/combine item.
 *   out[s] = sum over k = 0..K-1 (in that order, fp32) of gates[s,k]*y[row_of[s*K+k]]
 *   y [R, H] (dtype), row_of [S*K], gates [S, K] fp32, out [S, H] (dtype).
 */
moe_status_t moe_combine(const moe_dims_t* dims, const void* y, const int32_t* row_of,
                         const float* gates, void* out, void* stream);

/* Tensors saved by the forward that the backward reads (all device pointers). */
typedef struct {
  const void* x;            /* [S, H] */
  const void* Wg;           /* [H, E] */
  const void* W1;           /* [E, H, Hf] */
  const void* W3;           /* [E, H, Hf] */
  const void* W2;           /* [E, Hf, H] */
  const void* xd;           /* [R, H] */
  const void* h1;           /* [R, Hf] */
  const void* h3;           /* [R, Hf] */
  const void* a;            /* [R, Hf] */
  const void* y;            /* [R, H] */
  const int32_t* topk_idx;  /* [S, K] */
  const float* gates;       /* [S, K] */
  const int32_t* cu_seqlens;/* [E+1] */
  const int32_t* row_of;    /* [S*K] */
  const int32_t* tok_of;    /* [S*K] */
  const float* logits;      /* [S, E] router logits (moe_route's output); required without
                               MOE_F_RENORM, unused with it (may be NULL) */
} moe_saved_t;

/* Intermediate gradients the backward writes (caller-owned, all required). */
typedef struct {
  void* dy;        /* [R, H]  dtype: gates[s,k]*dout[s] at each row */
  void* dh1;       /* [R, Hf] dtype */
  void* dh3;       /* [R, Hf] dtype */
  void* dxd;       /* [R, H]  dtype */
  float* dgates;   /* [S, K]  <dout[s], y[row]> */
  float* dlogits;  /* [S, E]  gradient at the router logits (zero off the chosen experts
                               under MOE_F_RENORM, dense without it) */
} moe_bwd_bufs_t;

/*
 * moe_backward - the whole layer backward given dout = d(loss)/d(out).
 * [FW] "What's in the box", sparse-backward item (gating and dispatch
 * gradients in one kernel, nothing extra saved); [MEP] guide, gradient step
 * (an fp32 gradient buffer shaped like each projection tensor).
 *
 *   dout [S, H] (dtype)
 *   dx   [S, H] output (dtype): through dispatch and through the router
 *   dWg  [H, E] fp32 output: x^T * dlogits (the bias gets no gradient)
 *   dW1, dW3 [E, H, Hf], dW2 [E, Hf, H] fp32 outputs: experts with no rows
 *   get zeros (or are left unchanged under MOE_F_ACCUM_GRAD).
 * The selection itself has no gradient.  With MOE_F_RENORM the gates are
 * the softmax renormalised over the K chosen experts, so dlogits is zero off
 * them and the router terms of dx and dWg touch K experts per token.
 * Without it (raw gates, the chosen entries of the softmax over all E
 * experts; [FW] "What's in the box", routing/gating item read literally)
 * dlogits[s, e] = p_e (dp_e - sum_k g_k dg_k) is dense over all experts,
 * saved->logits is required (MOE_ERR_NULL otherwise), and dx's router term
 * and dWg are dense products over all E.
 * With MOE_F_RECOMPUTE the forward did not keep h1, h3 (saved->h1, h3 may be
 * NULL): the backward recomputes them from xd into bufs->dh1, dh3 (one more
 * up-projection GEMM) and the SwiGLU backward overwrites them there in
 * place; results are bitwise those of the saving mode ([FW] "What's in the
 * box", sparse-backward item: gradients without saving intermediates).
 */
moe_status_t moe_backward(const moe_dims_t* dims, const moe_saved_t* saved, const void* dout,
                          void* dx, float* dWg, float* dW1, float* dW3, float* dW2,
                          const moe_bwd_bufs_t* bufs, void* ws, size_t ws_bytes, void* stream);

/*
 * Mixture-of-Depths step around the MoE layer (config with B sequences of T
 * tokens, C kept per sequence).  [FW] "Comparison with alternatives" (MoD: a
 * share of the tokens skips the layer; custom kernels at 50% sparsity) and
 * "Who the framework saves" (MoE combined with MoD).
 *
 * moe_mod_select: r[s] = <x[s], w_r> (fp32); per sequence keep the C tokens
 *   of largest r (ties to the lower position), listed in ascending position
 *   as global indices b*T+t in keep_idx [B*C]; xk [B*C, H] = x[keep_idx].
 * moe_mod_merge: out = x; out[keep_idx[j]] += r[keep_idx[j]] * m[j].
 * moe_mod_backward: dm[j] = r[s] dout[s]; dr[j] = <dout[s], m[j]>;
 *   dx = dout + scatter over kept s of (dxk[j] + dr[j] w_r); dw_r = sum dr[j] x[s]
 *   (dw_r written over, or added to under MOE_F_ACCUM_GRAD).  Two phases:
 *   call with dxk = NULL to get dm and dr before the MoE backward, then with
 *   dxk (the MoE backward's dx) to get dx and dw_r.
 * Sizes: B >= 1, 1 <= T <= 8192, 0 <= C <= T, B*T*H < 2^31, H a multiple of
 * 128.  moe_mod_backward needs moe_mod_workspace_bytes(H) bytes of `ws`.
 */
size_t moe_mod_workspace_bytes(int32_t H);
moe_status_t moe_mod_select(int32_t B, int32_t T, int32_t C, int32_t H, int32_t dtype,
                            const void* x, const void* w_r, float* r, int32_t* keep_idx, void* xk,
                            void* stream);
moe_status_t moe_mod_merge(int32_t B, int32_t T, int32_t C, int32_t H, int32_t dtype,
                           const void* x, const float* r, const int32_t* keep_idx, const void* m,
                           void* out, void* stream);
moe_status_t moe_mod_backward(int32_t B, int32_t T, int32_t C, int32_t H, int32_t dtype,
                              uint32_t flags, const void* x, const void* w_r, const float* r,
                              const int32_t* keep_idx, const void* m, const void* dout,
                              const void* dxk, void* dm, float* dr, void* dx, float* dw_r,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * moe_load_stats - load statistics of a routing histogram ([MEP] "Which
 * problem MoonEP solves": maxvio, the most loaded expert's load over the
 * mean load, minus one).
 *   counts [E] int32 device (moe_route's per-expert counts)
 *   stats  [2] fp32 device output: stats[0] = maxvio = max_e c_e / mean_e c_e - 1,
 *          stats[1] = load entropy = -sum_e f_e ln f_e over f_e = c_e / sum c > 0
 *          (ln E when balanced, 0 when one expert takes every pair); both 0
 *          when every count is 0.
 * 1 <= E <= 1024.  Asynchronous on `stream`; no workspace.
 */
moe_status_t moe_load_stats(int32_t E, const int32_t* counts, float* stats, void* stream);

/*
 * Optional per-kernel timer (measurement only).  When enabled, every kernel
 * the library launches is bracketed by a pair of hipEvents recorded on the
 * stream it is launched on; moe_timer_read sums the elapsed milliseconds and
 * launch counts per kernel name since the last reset (it synchronises those
 * events).  This is process-global state: enable it only from one thread.
 */
void moe_timer_enable(int on);
void moe_timer_reset(void);
/* Fills up to `cap` entries; returns the number of distinct kernel names. */
int moe_timer_read(const char** names, double* total_ms, int64_t* launches, int cap);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */

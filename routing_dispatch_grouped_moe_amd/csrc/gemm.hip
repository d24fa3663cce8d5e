// Grouped GEMMs of the expert FFN and its backward (SwiGLU row of the T4
// tuning page's "RMSNorm, RoPE, SwiGLU" table: three matrix products per
// expert; MoonEP page, weights step: one contiguous tensor per projection,
// the grouped GEMM reaching expert e's weights from e alone; MoonEP page,
// gradient step: an fp32 gradient buffer shaped like the weights).
//
// Two grouping kinds over the expert row offsets cu[E+1]:
//   M-grouped  C[rows of e, N] = A[rows of e, K] * B_e[K, N]      (fwd, dA, dxd)
//   K-grouped  C_e[M, N] = A[rows of e, M]^T * B[rows of e, N]    (dW1, dW3, dW2)
//
// gfx950 design.  A block computes a 128x128 tile (per B operand) with four
// wavefronts as 2x2, each 64x64 on v_mfma_f32_32x32x16_bf16, fp32
// accumulation.  Every operand tile is staged in LDS as rows of 64
// K-contiguous bf16 (128 B) with the 16-byte chunk index XOR-ed by (row & 7),
// so the MFMA fragment reads (8 rows x 16 B per quarter-wave) and the stage
// writes are free of bank conflicts.  Operands stored K-contiguous in HBM are
// copied chunk for chunk; operands stored with M or N contiguous (weights
// [H, H'] in the forward, activations in the weight gradients) are read as
// 8x8 bf16 blocks (eight 16-byte rows) and transposed in registers with
// v_perm before the LDS write.  Global reads go through raw buffer
// resources bounded to the expert's rows, so ragged tiles read zeros without
// branches.  The next K step is prefetched into registers while the current
// one runs on MFMA (two LDS stages, one barrier per step).  M tiles come
// from a device-built table (expert, first row), so there is no host sync.
//
// The fp32 storage type (the tiny fp32 workload) uses a plain FMA kernel
// with the same tile decomposition and epilogues.
#include "dev_common.h"
#include "launch.h"

namespace moe {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kGroupM = 8;  // M tiles walked together (n fastest inside a group of 8 M tiles)

enum { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2, EPI_F32 = 3 };

struct GemmArgs {
  const int32_t* cu;      // [E+1] row offsets of the experts
  const int2* tiles;      // M-grouped: (expert, first row inside the expert) of each M tile
  const int32_t* ntiles;  // M-grouped: number of valid M tiles
  int E, M, N, K;         // M-grouped: N and K (K per segment); K-grouped: M and N
  int mtn, ntn;           // tiles along M (K-grouped) / along N
  const void* A0;         // row-indexed operand (second K segment in A1)
  const void* A1;
  int64_t lda;
  const void* B0;         // second B operand in B1 (dual) or second K segment (two-segment)
  const void* B1;
  int64_t ldb;
  int64_t sBe;            // per-expert stride of B (weights); 0 when B is row-indexed
  void* C0;
  void* C1;
  void* C2;
  int64_t ldc;
  int64_t sCe;            // per-expert stride of C (weight gradients)
  const void* X0;         // h1, h3 for the SwiGLU backward epilogue
  const void* X1;
  int accum;
};

// ------------------------------------------------------------- epilogue --
template <int EPI, bool BF16, bool DUAL>
__device__ __forceinline__ void epilogue(const GemmArgs& p, int e, int64_t row, int col, float v0,
                                         float v1) {
  const int64_t o = row * p.ldc + col;
  if constexpr (EPI == EPI_STORE) {
    store1<BF16>(p.C0, o, v0);
  } else if constexpr (EPI == EPI_SWIGLU_FWD) {
    store1<BF16>(p.C0, o, v0);
    store1<BF16>(p.C1, o, v1);
    store1<BF16>(p.C2, o, silu_f(v0) * v1);
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    const float z = load1<BF16>(p.X0, o), u = load1<BF16>(p.X1, o);
    const float sg = sigmoid_f(z);
    store1<BF16>(p.C0, o, v0 * u * sg * (1.0f + z * (1.0f - sg)));
    store1<BF16>(p.C1, o, v0 * z * sg);
  } else {
    float* c0 = reinterpret_cast<float*>(p.C0) + (int64_t)e * p.sCe + o;
    *c0 = p.accum ? *c0 + v0 : v0;
    if constexpr (DUAL) {
      float* c1 = reinterpret_cast<float*>(p.C1) + (int64_t)e * p.sCe + o;
      *c1 = p.accum ? *c1 + v1 : v1;
    }
  }
}

// Tile coordinates of a block.  Returns false when the block has no tile.
template <bool KGROUP, int BN>
__device__ __forceinline__ bool tile_of(const GemmArgs& p, int bid, int& e, int64_t& row0,
                                        int& valid, int& m0, int& n0) {
  if constexpr (KGROUP) {
    const int per_e = p.mtn * p.ntn;
    e = bid / per_e;
    const int rem = bid - e * per_e;
    m0 = (rem / p.ntn) * kBM;
    n0 = (rem % p.ntn) * BN;
    row0 = p.cu[e];
    valid = max(0, p.cu[e + 1] - p.cu[e]);  // the reduction length
    return true;
  } else {
    const int per_group = kGroupM * p.ntn;
    const int g = bid / per_group, r = bid - g * per_group;
    const int mt = g * kGroupM + r % kGroupM;
    n0 = (r / kGroupM) * BN;
    if (mt >= *p.ntiles) return false;
    const int2 t = p.tiles[mt];
    e = t.x;
    row0 = (int64_t)p.cu[e] + t.y;
    valid = min(kBM, p.cu[e + 1] - (int)row0);
    m0 = 0;
    return true;
  }
}

// -------------------------------------------------------- LDS addressing --
__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  return (uint32_t)row * 128u + ((uint32_t)(chunk ^ (row & 7)) << 4);
}

// 8x8 bf16 transpose: in[j] holds 8 consecutive-MN values at k = j; out[m]
// holds the 8 k values (k pairs packed per dword) of MN index m.
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      out[m][q] = __builtin_amdgcn_perm(in[2 * q + 1][m >> 1], in[2 * q][m >> 1],
                                        (m & 1) ? 0x07060302u : 0x05040100u);
}

// One operand tile of ROWS x 64 (rows = M or N index, 64 = K step) staged via
// registers.  KC: stored [rows][K] in HBM (K contiguous); otherwise [K][rows].
template <bool KC, int ROWS, int NOPS>
struct OperandStage {
  static constexpr int kItems = NOPS * (KC ? ROWS * 8 : ROWS);  // 16-B chunks or 8x8 blocks
  static constexpr int kSlots = (kItems + 255) / 256;
  static constexpr int kRegs = KC ? kSlots : kSlots * 8;
  u32x4 r[kRegs];

  // rs[op]: resource of operand op; off0: byte offset of (row 0 or k 0) of this K step.
  // For KC, element (row, k) is at (row*ld + k); otherwise at (k*ld + row).
  __device__ __forceinline__ void load(const __amdgpu_buffer_rsrc_t (&rs)[NOPS], int64_t ld,
                                       int row_base, int k0, int tid) {
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int it = tid + 256 * sl;
      if (it >= kItems) break;
      const int op = NOPS == 1 ? 0 : it / (kItems / NOPS);
      const int li = NOPS == 1 ? it : it - op * (kItems / NOPS);
      if constexpr (KC) {
        const int row = li >> 3, c = li & 7;
        r[sl] = buf_load16(rs[op], (uint32_t)(((int64_t)(row_base + row) * ld + k0 + c * 8) * 2));
      } else {
        const int kg = li & 7, mg = li >> 3;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          r[sl * 8 + j] = buf_load16(
              rs[op], (uint32_t)(((int64_t)(k0 + kg * 8 + j) * ld + row_base + mg * 8) * 2));
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) {
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int it = tid + 256 * sl;
      if (it >= kItems) break;
      const int op = NOPS == 1 ? 0 : it / (kItems / NOPS);
      const int li = NOPS == 1 ? it : it - op * (kItems / NOPS);
      char* t = lds + op * (ROWS * 128);
      if constexpr (KC) {
        const int row = li >> 3, c = li & 7;
        *reinterpret_cast<u32x4*>(t + lds_off(row, c)) = r[sl];
      } else {
        const int kg = li & 7, mg = li >> 3;
        u32x4 in[8], out[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) in[j] = r[sl * 8 + j];
        transpose8x8(in, out);
#pragma unroll
        for (int m = 0; m < 8; ++m) *reinterpret_cast<u32x4*>(t + lds_off(mg * 8 + m, kg)) = out[m];
      }
    }
  }
};

template <bool A_KC, bool B_KC, bool DUAL, bool TWOSEG, bool KGROUP, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int kTileA = kBM * 128, kTileB = kBN * 128;  // bytes per stage
  constexpr int kStage = kTileA + NB * kTileB;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  int e, valid, m0, n0;
  int64_t row0;
  if (!tile_of<KGROUP, kBN>(p, blockIdx.x, e, row0, valid, m0, n0)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;

  // Resources and tile origins.
  __amdgpu_buffer_rsrc_t ra[TWOSEG ? 2 : 1];
  __amdgpu_buffer_rsrc_t rb[TWOSEG ? 2 : NB];
  int a_base, b_base;  // row (KC) or column (not KC) origin inside the resource
  int nk;
  const int nk_seg = KGROUP ? 0 : p.K / kBK;
  if constexpr (KGROUP) {
    // A: [rows][M] of expert e; B: [rows][N]; reduction over the expert's rows.
    if (valid == 0) {
      if (!p.accum) {
        for (int i = tid; i < kBM * kBN; i += 256) {
          const int r = i / kBN, c = i % kBN;
          epilogue<EPI, true, DUAL>(p, e, m0 + r, n0 + c, 0.f, 0.f);
        }
      }
      return;
    }
    const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A0) + row0 * p.lda;
    ra[0] = make_rsrc(A, (uint32_t)((int64_t)valid * p.lda * 2));
    const uint16_t* B0 = reinterpret_cast<const uint16_t*>(p.B0) + row0 * p.ldb;
    rb[0] = make_rsrc(B0, (uint32_t)((int64_t)valid * p.ldb * 2));
    if constexpr (DUAL) {
      const uint16_t* B1 = reinterpret_cast<const uint16_t*>(p.B1) + row0 * p.ldb;
      rb[1] = make_rsrc(B1, (uint32_t)((int64_t)valid * p.ldb * 2));
    }
    a_base = m0;
    b_base = n0;
    nk = (valid + kBK - 1) / kBK;
  } else {
    const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A0) + row0 * p.lda;
    ra[0] = make_rsrc(A, (uint32_t)((int64_t)valid * p.lda * 2));
    if constexpr (TWOSEG) {
      const uint16_t* A1 = reinterpret_cast<const uint16_t*>(p.A1) + row0 * p.lda;
      ra[1] = make_rsrc(A1, (uint32_t)((int64_t)valid * p.lda * 2));
    }
    const uint32_t wbytes = (uint32_t)((int64_t)p.N * p.K * 2);
    rb[0] = make_rsrc(reinterpret_cast<const uint16_t*>(p.B0) + (int64_t)e * p.sBe, wbytes);
    if constexpr (DUAL || TWOSEG)
      rb[1] = make_rsrc(reinterpret_cast<const uint16_t*>(p.B1) + (int64_t)e * p.sBe, wbytes);
    a_base = 0;
    b_base = n0;
    nk = TWOSEG ? 2 * nk_seg : nk_seg;
  }

  OperandStage<A_KC, kBM, 1> sa;
  OperandStage<B_KC, kBN, NB> sb;
  auto load_step = [&](int kt) {
    int seg = 0, k0 = kt * kBK;
    if constexpr (TWOSEG) {
      seg = kt >= nk_seg ? 1 : 0;
      k0 = (kt - seg * nk_seg) * kBK;
    }
    __amdgpu_buffer_rsrc_t rA[1] = {ra[TWOSEG ? seg : 0]};
    sa.load(rA, p.lda, a_base, k0, tid);
    if constexpr (TWOSEG) {
      __amdgpu_buffer_rsrc_t rB[1] = {rb[seg]};
      sb.load(rB, p.ldb, b_base, k0, tid);
    } else {
      sb.load(rb, p.ldb, b_base, k0, tid);
    }
  };

  f32x16 acc[NB][2][2];
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][i][j][v] = 0.f;

  load_step(0);
  sa.store(smem, tid);
  sb.store(smem + kTileA, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * kStage;
    if (kt + 1 < nk) load_step(kt + 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int chunk = kk * 2 + (lane >> 5);
      u32x4 af[2], bfr[NB][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(cur + lds_off(wm * 64 + i * 32 + (lane & 31), chunk));
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bfr[q][j] = *reinterpret_cast<const u32x4*>(cur + kTileA + q * kTileB +
                                                      lds_off(wn * 64 + j * 32 + (lane & 31), chunk));
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[q][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, af[i]), __builtin_bit_cast(bf16x8, bfr[q][j]),
                acc[q][i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      char* nxt = smem + ((kt + 1) & 1) * kStage;
      sa.store(nxt, tid);
      sb.store(nxt + kTileA, tid);
    }
    __syncthreads();
  }

  // 32x32 MFMA result: lane holds column (lane % 32), rows 8*(v/4) + 4*(lane/32) + v%4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int c = n0 + wn * 64 + j * 32 + (lane & 31);
        const float v1 = DUAL ? acc[NB - 1][i][j][v] : 0.f;
        if constexpr (KGROUP) {
          epilogue<EPI, true, DUAL>(p, e, m0 + r, c, acc[0][i][j][v], v1);
        } else {
          if (r < valid) epilogue<EPI, true, DUAL>(p, e, row0 + r, c, acc[0][i][j][v], v1);
        }
      }
}

// ---------------------------------------------------------- fp32 kernel --
// Tile 128 (M) x 32 (N); thread (tid % 32) owns a column, rows tid/32 + 8 i.
constexpr int kBNf = 32;

template <bool A_KC, bool B_KC, bool DUAL, bool TWOSEG, bool KGROUP, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p) {
  int e, valid, m0, n0;
  int64_t row0;
  if (!tile_of<KGROUP, kBNf>(p, blockIdx.x, e, row0, valid, m0, n0)) return;
  const int tid = threadIdx.x;
  const int col = n0 + (tid & 31);
  const float* A0 = reinterpret_cast<const float*>(p.A0);
  const float* A1 = reinterpret_cast<const float*>(p.A1);
  const float* B0 = reinterpret_cast<const float*>(p.B0);
  const float* B1 = reinterpret_cast<const float*>(p.B1);
  for (int i = 0; i < kBM / 8; ++i) {
    const int r = (tid >> 5) + 8 * i;
    float acc0 = 0.f, acc1 = 0.f;
    if constexpr (KGROUP) {
      // C_e[m0+r, col] = sum over the expert's rows k of A[k, m0+r] * B[k, col]
      for (int k = 0; k < valid; ++k) {
        const int64_t gr = row0 + k;
        const float a = A0[gr * p.lda + m0 + r];
        acc0 = fmaf(a, B0[gr * p.ldb + col], acc0);
        if constexpr (DUAL) acc1 = fmaf(a, B1[gr * p.ldb + col], acc1);
      }
      if (valid > 0 || !p.accum) epilogue<EPI, false, DUAL>(p, e, m0 + r, col, acc0, acc1);
    } else {
      if (r >= valid) continue;
      const int64_t gr = row0 + r;
      for (int seg = 0; seg < (TWOSEG ? 2 : 1); ++seg) {
        const float* A = seg ? A1 : A0;
        const float* Bw = (seg ? B1 : B0) + (int64_t)e * p.sBe;
        const float* Bw1 = B1 + (int64_t)e * p.sBe;
        for (int k = 0; k < p.K; ++k) {
          const float a = A[gr * p.lda + k];
          const float b0 = B_KC ? Bw[(int64_t)col * p.ldb + k] : Bw[(int64_t)k * p.ldb + col];
          acc0 = fmaf(a, b0, acc0);
          if constexpr (DUAL) acc1 = fmaf(a, Bw1[(int64_t)k * p.ldb + col], acc1);
        }
      }
      epilogue<EPI, false, DUAL>(p, e, gr, col, acc0, acc1);
    }
  }
}

// ------------------------------------------------------------ tile table --
__device__ int block_exclusive_scan_1024_g(int v, int* sh, int* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int incl = sh[tid];
  *total = sh[1023];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ cu, int E,
                                                          int max_tiles, int2* __restrict__ tiles,
                                                          int32_t* __restrict__ ntiles) {
  __shared__ int sh[1024];
  const int e = threadIdx.x;
  // A malformed cu (not monotone) yields no tiles for that expert rather than
  // a table overflow.
  const int c = e < E ? max(0, cu[e + 1] - cu[e]) : 0;
  const int nt = (c + kBM - 1) / kBM;
  int total;
  const int start = block_exclusive_scan_1024_g(nt, sh, &total);
  for (int t = 0; t < nt && start + t < max_tiles; ++t) tiles[start + t] = make_int2(e, t * kBM);
  if (e == 0) *ntiles = min(total, max_tiles);
}

void launch_tile_table(const int32_t* cu, int E, const WsLayout& L, char* ws, hipStream_t s) {
  TimedLaunch tl("gemm_tile_table", s);
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, s, cu, E, L.max_tiles,
                     reinterpret_cast<int2*>(ws + L.tiles), reinterpret_cast<int32_t*>(ws + L.ntiles));
}

// -------------------------------------------------------------- launches --
template <bool A_KC, bool B_KC, bool DUAL, bool TWOSEG, bool KGROUP, int EPI>
static void gemm_launch(const char* name, GemmArgs p, int max_mtiles, bool bf16, hipStream_t s) {
  const int bn = bf16 ? kBN : kBNf;
  p.ntn = p.N / bn;
  int blocks;
  if (KGROUP) {
    p.mtn = p.M / kBM;
    blocks = p.E * p.mtn * p.ntn;
  } else {
    const int groups = (max_mtiles + kGroupM - 1) / kGroupM;
    blocks = groups * kGroupM * p.ntn;
  }
  if (blocks <= 0) return;
  TimedLaunch tl(name, s);
  if (bf16) {
    auto kern = gemm_bf16_kernel<A_KC, B_KC, DUAL, TWOSEG, KGROUP, EPI>;
    constexpr int lds = 2 * (kBM * 128 + (DUAL ? 2 : 1) * kBN * 128);
    static bool attr = false;
    if (!attr) {
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      attr = true;
    }
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), lds, s, p);
  } else {
    hipLaunchKernelGGL((gemm_f32_kernel<A_KC, B_KC, DUAL, TWOSEG, KGROUP, EPI>), dim3(blocks),
                       dim3(256), 0, s, p);
  }
}

static GemmArgs base_args(const int32_t* cu, const WsLayout& L, char* ws, int E) {
  GemmArgs p{};
  p.cu = cu;
  p.tiles = reinterpret_cast<const int2*>(ws + L.tiles);
  p.ntiles = reinterpret_cast<const int32_t*>(ws + L.ntiles);
  p.E = E;
  return p;
}

void launch_ffn_up(const void* xd, const int32_t* cu, const void* W1, const void* W3, void* h1,
                   void* h3, void* a, int64_t R, int H, int Hf, int E, const WsLayout& L, char* ws,
                   bool bf16, hipStream_t s) {
  (void)R;
  GemmArgs p = base_args(cu, L, ws, E);
  p.N = Hf; p.K = H;
  p.A0 = xd; p.lda = H;
  p.B0 = W1; p.B1 = W3; p.ldb = Hf; p.sBe = (int64_t)H * Hf;
  p.C0 = h1; p.C1 = h3; p.C2 = a; p.ldc = Hf;
  gemm_launch<true, false, true, false, false, EPI_SWIGLU_FWD>("ffn_up", p, L.max_tiles, bf16, s);
}

void launch_ffn_down(const void* a, const int32_t* cu, const void* W2, void* y, int64_t R, int H,
                     int Hf, int E, const WsLayout& L, char* ws, bool bf16, hipStream_t s) {
  (void)R;
  GemmArgs p = base_args(cu, L, ws, E);
  p.N = H; p.K = Hf;
  p.A0 = a; p.lda = Hf;
  p.B0 = W2; p.ldb = H; p.sBe = (int64_t)Hf * H;
  p.C0 = y; p.ldc = H;
  gemm_launch<true, false, false, false, false, EPI_STORE>("ffn_down", p, L.max_tiles, bf16, s);
}

void launch_bwd_da(const void* dy, const int32_t* cu, const void* W2, const void* h1,
                   const void* h3, void* dh1, void* dh3, int64_t R, int H, int Hf, int E,
                   const WsLayout& L, char* ws, bool bf16, hipStream_t s) {
  (void)R;
  // da[rows, Hf] = dy[rows, H] * W2[e]^T; W2[e] is [Hf][H] = [N][K], K contiguous.
  GemmArgs p = base_args(cu, L, ws, E);
  p.N = Hf; p.K = H;
  p.A0 = dy; p.lda = H;
  p.B0 = W2; p.ldb = H; p.sBe = (int64_t)Hf * H;
  p.C0 = dh1; p.C1 = dh3; p.ldc = Hf;
  p.X0 = h1; p.X1 = h3;
  gemm_launch<true, true, false, false, false, EPI_SWIGLU_BWD>("bwd_dA", p, L.max_tiles, bf16, s);
}

void launch_bwd_dxd(const void* dh1, const void* dh3, const int32_t* cu, const void* W1,
                    const void* W3, void* dxd, int64_t R, int H, int Hf, int E, const WsLayout& L,
                    char* ws, bool bf16, hipStream_t s) {
  (void)R;
  // dxd[rows, H] = dh1 * W1[e]^T + dh3 * W3[e]^T; W1[e] is [H][Hf] = [N][K].
  GemmArgs p = base_args(cu, L, ws, E);
  p.N = H; p.K = Hf;
  p.A0 = dh1; p.A1 = dh3; p.lda = Hf;
  p.B0 = W1; p.B1 = W3; p.ldb = Hf; p.sBe = (int64_t)H * Hf;
  p.C0 = dxd; p.ldc = H;
  gemm_launch<true, true, false, true, false, EPI_STORE>("bwd_dxd", p, L.max_tiles, bf16, s);
}

void launch_bwd_dw2(const void* a, const void* dy, const int32_t* cu, float* dW2, int64_t R, int H,
                    int Hf, int E, bool accum, bool bf16, hipStream_t s) {
  (void)R;
  // dW2[e][Hf, H] = a[rows, Hf]^T * dy[rows, H]
  GemmArgs p{};
  p.cu = cu; p.E = E; p.M = Hf; p.N = H;
  p.A0 = a; p.lda = Hf;
  p.B0 = dy; p.ldb = H;
  p.C0 = dW2; p.ldc = H; p.sCe = (int64_t)Hf * H;
  p.accum = accum;
  gemm_launch<false, false, false, false, true, EPI_F32>("bwd_dW2", p, 0, bf16, s);
}

void launch_bwd_dw13(const void* xd, const void* dh1, const void* dh3, const int32_t* cu,
                     float* dW1, float* dW3, int64_t R, int H, int Hf, int E, bool accum,
                     bool bf16, hipStream_t s) {
  (void)R;
  // dW1[e][H, Hf] = xd[rows, H]^T * dh1[rows, Hf]; dW3 likewise with dh3.
  GemmArgs p{};
  p.cu = cu; p.E = E; p.M = H; p.N = Hf;
  p.A0 = xd; p.lda = H;
  p.B0 = dh1; p.B1 = dh3; p.ldb = Hf;
  p.C0 = dW1; p.C1 = dW3; p.ldc = Hf; p.sCe = (int64_t)H * Hf;
  p.accum = accum;
  gemm_launch<false, false, true, false, true, EPI_F32>("bwd_dW13", p, 0, bf16, s);
}

}  // namespace moe

// Tile machinery shared by the MFMA kernels (the grouped GEMMs and the
// router GEMM): XCD-contiguous block numbering, the XOR-swizzled LDS tile
// layouts, MFMA operand fragment reads (plain and transposing), and direct
// global -> LDS operand loads.  Internal to the library.
#pragma once

#include "dev_common.h"

namespace moe {

constexpr int kBK = 64;  // K extent of one operand tile (one K step)

// Blocks are handed to the eight XCDs round-robin (block b runs on XCD b % 8),
// and each XCD has its own L2.  Renumber so that XCD x runs one contiguous
// range of tile ids: the blocks an XCD holds at once then cover a compact
// patch of tiles that share operand tiles in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int x = b & 7, q = nb >> 3, r = nb & 7;
  return x * q + min(x, r) + (b >> 3);
}

// ------------------------------------------------------ LDS tile layouts --
// K-contiguous tile [rows][64]: 128 B a row, chunk c (8 k values) stored at
// c ^ ((row >> 1) & 7): the sixteen rows (same chunk) one read cycle touches
// land on sixteen distinct 16-byte bank groups.
__device__ __forceinline__ uint32_t kc_off(int row, int c) {
  return (uint32_t)row * 128u + ((uint32_t)(c ^ ((row >> 1) & 7)) << 4);
}
// K-major tile [64][cols]: row k holds cols values, chunk c stored at
// c ^ (4 (k & 3) ^ 2 ((k >> 3) & 1)): the 4 rows x 64 B that 32 lanes of a
// transpose load read (k0..k0+3, four aligned chunks) cover all sixteen
// 16-byte bank groups, and rows k and k+8 (the other half of the wave) are
// shifted against each other.
template <int COLS>
__device__ __forceinline__ uint32_t km_off(int k, int c) {
  // the swizzle moves a chunk by up to 14 places: rows of at least 16 chunks
  static_assert(COLS >= 128, "K-major tiles need at least 128 columns");
  return (uint32_t)k * (COLS * 2) + ((uint32_t)(c ^ (4 * (k & 3)) ^ (2 * ((k >> 3) & 1))) << 4);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ u32x4 lds_read16(const char* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

// MFMA 32x32x16 operand fragment (8 k values of one M/N index per lane, lane
// l: index l % 32, k = 8 (l / 32) + 0..7) from a K-contiguous tile.
__device__ __forceinline__ u32x4 frag_kc(const char* tile, int row_base, int kk, int lane) {
  const int row = row_base + (lane & 31);
  return lds_read16(tile, kc_off(row, 2 * kk + (lane >> 5)));
}
// The same fragment from a K-major tile, with two transpose loads: in each
// 16-lane group, lane s reads four values of row k0 + s/4 at column
// 4*(s%4); lane i then holds column i of rows k0..k0+3.
template <int COLS>
__device__ __forceinline__ u32x4 frag_km(const char* tile, int col_base, int kk, int lane) {
  const int col = col_base + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int kb = 16 * kk + 8 * (lane >> 5) + ((lane & 15) >> 2);
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = kb + 4 * h;
    const uint32_t off = km_off<COLS>(k, col >> 3) + (col & 7) * 2;
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)((__attribute__((address_space(3))) char*)(tile) + off));
    const u32x2 u = __builtin_bit_cast(u32x2, v);
    r[2 * h] = u[0];
    r[2 * h + 1] = u[1];
  }
  return r;
}
// The swizzle term of km_off depends on k only through k & 3 and
// (k >> 3) & 1, which for the rows a lane reads are fixed by the lane; so a
// fragment's two transpose loads for any K16 slice kk are at
// base + kk * 16 rows + h * 4 rows, with one per-lane base per fragment.
template <int COLS>
__device__ __forceinline__ uint32_t frag_km_base(int col_base, int lane) {
  return km_off<COLS>(8 * (lane >> 5) + ((lane & 15) >> 2),
                      (col_base + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) >> 3) +
         (4 * (lane & 3) & 7) * 2;
}
template <int COLS>
__device__ __forceinline__ u32x4 frag_km_at(const char* tile, uint32_t base, int kk) {
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t off = base + (uint32_t)(16 * kk + 4 * h) * (COLS * 2);
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)((__attribute__((address_space(3))) char*)(tile) + off));
    const u32x2 u = __builtin_bit_cast(u32x2, v);
    r[2 * h] = u[0];
    r[2 * h + 1] = u[1];
  }
  return r;
}

// Direct global -> LDS staging of one operand tile per K step with
// buffer_load ... lds: each wave instruction moves 1 KB, lane l's 16 bytes
// landing at +16 l, so the swizzled LDS layouts above are produced by
// choosing which global chunk each lane fetches.  Lane offsets are for K
// step 0 and loop invariant; a step's K offset moves the buffer descriptor's
// base instead (scalar work), and the descriptor's range still bounds every
// read (past the end reads zero).
//   KC:  stored [rows][K] in HBM, LDS tile [ROWS][kBK]
//   !KC: stored [K][cols] in HBM, LDS tile [kBK][ROWS]

template <bool KC, int ROWS, int NOPS, int WAVES>
struct DmaOperand {
  static constexpr int kInstr = NOPS * ROWS * kBK * 2 / 1024;  // 1-KB wave instructions per step
  static constexpr int kPer = kInstr / WAVES;                  // per wavefront
  static_assert(kInstr % (WAVES * NOPS) == 0, "operand tile not a multiple of the waves");
  uint32_t voff[kPer];

  __device__ __forceinline__ void init(int64_t ld, int base, int w, int lane) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ins = w * kPer + i;
      const int op = ins / (kInstr / NOPS);
      const int P = (ins - op * (kInstr / NOPS)) * 64 + lane;  // physical 16-byte chunk
      int64_t el;
      if constexpr (KC) {
        constexpr int cpr = kBK / 8;
        const int row = P / cpr;
        el = (int64_t)(base + row) * ld + ((P % cpr) ^ ((row >> 1) & 7)) * 8;
      } else {
        constexpr int cpr = ROWS / 8;
        const int k = P / cpr;
        el = (int64_t)k * ld + base + ((P % cpr) ^ (4 * (k & 3)) ^ (2 * ((k >> 3) & 1))) * 8;
      }
      voff[i] = (uint32_t)(el * 2);
    }
  }
  // Instruction i of this wavefront's loads of the step whose descriptors
  // are rsrc[]: issued from inline assembly, so the compiler does not treat
  // it as an LDS store and never makes LDS reads wait for it; the kernel
  // waits for these loads explicitly (vmcnt) before the barrier that
  // publishes their stage, and only ever targets a stage nobody reads.
  __device__ __forceinline__ void issue_one(int i, const u32x4 (&rsrc)[NOPS], char* lds, int w) const {
    const int ins = w * kPer + i;
    const int op = ins / (kInstr / NOPS);
    char* dst = lds + (ins - op * (kInstr / NOPS)) * 1024 + op * (ROWS * kBK * 2);
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)dst;
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff[i]), "s"(rsrc[op]), "s"(m0) : "m0");
  }
  // descriptor words of operand op for the K step at element offset k0
  __device__ __forceinline__ void rsrc_for(const uint16_t* const (&base)[NOPS], uint32_t bytes,
                                           int64_t ld, int k0, u32x4 (&rsrc)[NOPS]) const {
    const uint32_t kadd = KC ? (uint32_t)k0 * 2u : (uint32_t)((int64_t)k0 * ld * 2);
    const uint32_t left = __builtin_amdgcn_readfirstlane(bytes - min(kadd, bytes));
#pragma unroll
    for (int op = 0; op < NOPS; ++op) {
      const uint64_t a = (uint64_t)(uintptr_t)(reinterpret_cast<const char*>(base[op]) + kadd);
      rsrc[op][0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
      rsrc[op][1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
      rsrc[op][2] = left;
      rsrc[op][3] = 0x00020000u;
    }
  }
};

}  // namespace moe

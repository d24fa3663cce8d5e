// Device helpers shared by the gfx950 kernels of the MoE hot path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ----------------------------------------------------------------- bf16 --
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> two bf16 in one word (lo in bits 0..15), round to nearest even,
// NaN stays NaN: one gfx950 v_cvt_pk_bf16_f32 per pair.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// Load / store 8 consecutive elements as fp32, from bf16 or fp32 storage.
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&v)[8]) {
  if constexpr (BF16) {
    u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(w[i]); v[2 * i + 1] = bf16_hi(w[i]); }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}
template <bool BF16>
__device__ __forceinline__ void store8(void* base, int64_t elem, const float (&v)[8]) {
  if constexpr (BF16) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(base) + elem) = w;
  } else {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + elem);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}
template <bool BF16>
__device__ __forceinline__ float load1(const void* base, int64_t elem) {
  if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[elem]);
  else return reinterpret_cast<const float*>(base)[elem];
}
template <bool BF16>
__device__ __forceinline__ void store1(void* base, int64_t elem, float v) {
  if constexpr (BF16) reinterpret_cast<uint16_t*>(base)[elem] = uint16_t(f32_to_bf16_bits(v));
  else reinterpret_cast<float*>(base)[elem] = v;
}

// Four fp32 values as four consecutive bf16 elements (8 bytes, 8-byte aligned).
__device__ __forceinline__ void store4_bf16(void* base, int64_t elem, const float (&v)[4]) {
  u32x2 w;
  w[0] = pack_bf16x2(v[0], v[1]);
  w[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + elem) = w;
}

// -------------------------------------------------------- buffer loads --
// A raw buffer resource clamps every access to [0, bytes): reads past the end
// return zero, which is how ragged tiles are padded without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Descriptor words (uniform, for an "s" operand of inline assembly) of the
// byte range [base, base + bytes): reads past it return zero.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}
// Direct global -> LDS loads: lane l reads 4 (dma4) or 16 (dma16) bytes at
// byte offset voff of the descriptor's range and writes them to LDS at
// dst + 4 l (16 l).  Issued from inline assembly: the compiler neither
// treats them as LDS stores nor makes LDS reads wait on them, so the caller
// waits for them (vmcnt) before the barrier that publishes the data, and
// only ever targets LDS that no wavefront is reading.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}
__device__ __forceinline__ void dma4(const u32x4& rsrc, uint32_t voff, const void* dst) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds_addr(dst)) : "m0");
}
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t voff, const void* dst) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds_addr(dst)) : "m0");
}

// ------------------------------------------------------- wave reductions --
// Cross-lane steps on DPP (VALU lane moves, no LDS round trip): butterfly
// within each 16-lane row (quad swaps, then the half-row and row mirrors),
// then the rows combined through the broadcasts of lanes 15 and 31, so that
// lane 63 holds the reduction of the whole wavefront; it is then read out
// to every lane.  Lanes of rows a step leaves out get `old`.  The whole
// wavefront must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xf, false);
}
constexpr int kDppXor1 = 0xb1, kDppXor2 = 0x4e, kDppHalfMirror = 0x141, kDppMirror = 0x140,
              kDppBcast15 = 0x142, kDppBcast31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __uint_as_float(dpp_mov<CTRL, ROWS>(0u, __float_as_uint(v)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<kDppXor1, 0xf>(v);
  v = dpp_add<kDppXor2, 0xf>(v);
  v = dpp_add<kDppHalfMirror, 0xf>(v);
  v = dpp_add<kDppMirror, 0xf>(v);
  v = dpp_add<kDppBcast15, 0xa>(v);
  v = dpp_add<kDppBcast31, 0xc>(v);
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}

// Largest value over the wavefront, to every lane (lanes a step leaves out
// keep their own value).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_fmax(float v) {
  const uint32_t b = __float_as_uint(v);
  return fmaxf(v, __uint_as_float(dpp_mov<CTRL, ROWS>(b, b)));
}
__device__ __forceinline__ float wave_max_f32(float v) {
  v = dpp_fmax<kDppXor1, 0xf>(v);
  v = dpp_fmax<kDppXor2, 0xf>(v);
  v = dpp_fmax<kDppHalfMirror, 0xf>(v);
  v = dpp_fmax<kDppMirror, 0xf>(v);
  v = dpp_fmax<kDppBcast15, 0xa>(v);
  v = dpp_fmax<kDppBcast31, 0xc>(v);
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_max(uint64_t v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const uint64_t o = ((uint64_t)dpp_mov<CTRL, ROWS>(hi, hi) << 32) | dpp_mov<CTRL, ROWS>(lo, lo);
  return o > v ? o : v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max<kDppXor1, 0xf>(v);
  v = dpp_max<kDppXor2, 0xf>(v);
  v = dpp_max<kDppHalfMirror, 0xf>(v);
  v = dpp_max<kDppMirror, 0xf>(v);
  v = dpp_max<kDppBcast15, 0xa>(v);
  v = dpp_max<kDppBcast31, 0xc>(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------- top-K order keys --
// Maps a float to a uint32 whose unsigned order is the float order, with
// -0 == +0 and NaN below -inf.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;   // NaN
  if (u == 0x80000000u) u = 0u;                      // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Larger key = better expert: logit descending, then expert index ascending.
__device__ __forceinline__ uint64_t topk_key(float logit, int e) {
  return (uint64_t(ordered_bits(logit)) << 32) | uint64_t(~uint32_t(e));
}
__device__ __forceinline__ int key_expert(uint64_t key) { return int(~uint32_t(key)); }

// Logistic sigmoid from the hardware base-2 exponential and reciprocal
// (v_exp_f32, v_rcp_f32; about 1 ulp each, far below the bf16 rounding of
// every SwiGLU output): e^-z = 2^(-z log2 e).  Both ends saturate exactly:
// z -> -inf gives rcp(inf) = 0, z -> +inf gives rcp(1) = 1.  Four
// instructions instead of a range-reduced expf and an IEEE division, which
// matters in GEMM epilogues that evaluate it for every output element.
__device__ __forceinline__ float sigmoid_f(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

}  // namespace moe

// MFMA operand policies for gfx950 (CDNA4) used by the chunked prefill.
//
// Every product runs as 16x16 output tiles.  A lane l holds output column
// l % 16 and rows 4q..4q+3, q = l / 16; its MFMA operand slots for a 32-deep
// step are the logical contraction indices {4q..4q+3, 16+4q..16+4q+3}
// (two consecutive 16-row accumulator tiles), so an accumulator tile pair can
// be fed back as an operand without moving data between lanes.  Operands
// kept in LDS are stored with the matching permutation (kperm) so the eight
// values are one contiguous read.  A 16-deep step uses the slots 4q..4q+3.
//
// Policies:
//   PolBF16x3 : bf16 MFMA; each fp32 operand x is split into hi = bf16(x) and
//               lo = bf16(x - hi); a product is hi*hi + hi*lo + lo*hi with
//               fp32 accumulation (~16 significant bits per operand).
//   PolF32    : fp32 MFMA (v_mfma_f32_16x16x4_f32), operands unrounded.
// mma_part(acc, a, b, p) issues part p < kParts of one 32-deep step; issuing a
// part over many independent accumulators before the next part keeps the MFMA
// pipe full (a dependent 16x16x32 bf16 MFMA waits ~44 cycles, an independent
// one issues every ~16-19).
#pragma once

#include "kda_common.hpp"

namespace kda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Position of logical index x inside its 32-block so that lane group q's
// eight contraction slots {4q..4q+3, 16+4q..16+4q+3} are contiguous.
__host__ __device__ constexpr int kperm(int x) {
  return (x & ~31) + (((x & 15) >> 2) << 3) + (x & 3) + (((x & 31) >> 4) << 2);
}

// Orders LDS traffic of one wave against itself (no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct PolBF16x3 {
  static constexpr int kPlanes = 2;  // hi plane, lo plane
  static constexpr int kElem = 2;    // bytes per element per plane
  static constexpr int kParts = 3;
  static constexpr int kParts16 = 3;
  struct Frag {
    bf16x8_t hi, lo;
  };
  struct Frag16 {
    s16x4_t hi, lo;
  };
  // x = hi + lo with hi = bf16(x), lo = bf16(x - hi): two values per call,
  // packed as two bf16 halves of a 32-bit word (v_cvt_pk_bf16_f32).
  __device__ __forceinline__ static void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const bf16x2_t h = {(__bf16)a, (__bf16)b};
    const uint32_t hw = __builtin_bit_cast(uint32_t, h);
    const float ra = a - __uint_as_float(hw << 16);
    const float rb = b - __uint_as_float(hw & 0xFFFF0000u);
    const bf16x2_t l = {(__bf16)ra, (__bf16)rb};
    hi = hw;
    lo = __builtin_bit_cast(uint32_t, l);
  }
  __device__ __forceinline__ static void store4(char* base, int plane, int off, const float v[4]) {
    uint32_t h0, l0, h1, l1;
    split2(v[0], v[1], h0, l0);
    split2(v[2], v[3], h1, l1);
    *reinterpret_cast<uint2*>(base + off) = make_uint2(h0, h1);
    *reinterpret_cast<uint2*>(base + plane + off) = make_uint2(l0, l1);
  }
  __device__ __forceinline__ static void store2(char* base, int plane, int off, float a, float b) {
    uint32_t h, l;
    split2(a, b, h, l);
    *reinterpret_cast<uint32_t*>(base + off) = h;
    *reinterpret_cast<uint32_t*>(base + plane + off) = l;
  }
  __device__ __forceinline__ static void store1(char* base, int plane, int off, float v) {
    const __bf16 h = (__bf16)v;
    const __bf16 l = (__bf16)(v - (float)h);
    *reinterpret_cast<__bf16*>(base + off) = h;
    *reinterpret_cast<__bf16*>(base + plane + off) = l;
  }
  __device__ __forceinline__ static Frag load(const char* base, int plane, int off) {
    Frag f;
    f.hi = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(base + off));
    f.lo = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(base + plane + off));
    return f;
  }
  __device__ __forceinline__ static Frag16 load16(const char* base, int plane, int off) {
    Frag16 f;
    f.hi = __builtin_bit_cast(s16x4_t, *reinterpret_cast<const u32x2_t*>(base + off));
    f.lo = __builtin_bit_cast(s16x4_t, *reinterpret_cast<const u32x2_t*>(base + plane + off));
    return f;
  }
  __device__ __forceinline__ static Frag make(const float v[8]) {
    u32x4_t hw, lw;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t h, l;
      split2(v[2 * e], v[2 * e + 1], h, l);
      hw[e] = h;
      lw[e] = l;
    }
    Frag f;
    f.hi = __builtin_bit_cast(bf16x8_t, hw);
    f.lo = __builtin_bit_cast(bf16x8_t, lw);
    return f;
  }
  __device__ __forceinline__ static Frag16 make16(const float v[4]) {
    u32x2_t hw, lw;
    uint32_t h, l;
    split2(v[0], v[1], h, l);
    hw[0] = h; lw[0] = l;
    split2(v[2], v[3], h, l);
    hw[1] = h; lw[1] = l;
    Frag16 f;
    f.hi = __builtin_bit_cast(s16x4_t, hw);
    f.lo = __builtin_bit_cast(s16x4_t, lw);
    return f;
  }
  __device__ __forceinline__ static void mma_part(f32x4_t& acc, const Frag& a, const Frag& b, int p) {
    if (p == 0) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    else if (p == 1) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    else acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void mma16_part(f32x4_t& acc, const Frag16& a, const Frag16& b, int p) {
    if (p == 0) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, acc, 0, 0, 0);
    else if (p == 1) acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, acc, 0, 0, 0);
    else acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, acc, 0, 0, 0);
  }
};

struct PolF32 {
  static constexpr int kPlanes = 1;
  static constexpr int kElem = 4;
  static constexpr int kParts = 8;
  static constexpr int kParts16 = 4;
  struct Frag {
    float v[8];
  };
  struct Frag16 {
    float v[4];
  };
  __device__ __forceinline__ static void store4(char* base, int, int off, const float v[4]) {
    *reinterpret_cast<float4*>(base + off) = make_float4(v[0], v[1], v[2], v[3]);
  }
  __device__ __forceinline__ static void store2(char* base, int, int off, float a, float b) {
    *reinterpret_cast<float2*>(base + off) = make_float2(a, b);
  }
  __device__ __forceinline__ static void store1(char* base, int, int off, float v) {
    *reinterpret_cast<float*>(base + off) = v;
  }
  __device__ __forceinline__ static Frag load(const char* base, int, int off) {
    Frag f;
    const float4 a = *reinterpret_cast<const float4*>(base + off);
    const float4 b = *reinterpret_cast<const float4*>(base + off + 16);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
  __device__ __forceinline__ static Frag16 load16(const char* base, int, int off) {
    Frag16 f;
    const float4 a = *reinterpret_cast<const float4*>(base + off);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    return f;
  }
  __device__ __forceinline__ static Frag make(const float v[8]) {
    Frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = v[e];
    return f;
  }
  __device__ __forceinline__ static Frag16 make16(const float v[4]) {
    Frag16 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) f.v[e] = v[e];
    return f;
  }
  __device__ __forceinline__ static void mma_part(f32x4_t& acc, const Frag& a, const Frag& b, int p) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[p], b.v[p], acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void mma16_part(f32x4_t& acc, const Frag16& a, const Frag16& b, int p) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[p], b.v[p], acc, 0, 0, 0);
  }
};

}  // namespace kda

// Shared device helpers for the KDA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kD = 128;  // d_k = d_v handled by every kernel

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (bf16 held as raw 16-bit patterns)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest, ties to even, two values per instruction
// (gfx950 v_cvt_pk_bf16_f32; NaN stays NaN).  a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) { return pack_bf16x2(x, 0.0f) & 0xFFFFu; }

// Raw buffer resource over [base, base + bytes) (gfx9 word 3: 32-bit data
// format).  A raw buffer access takes a 32-bit per-lane offset, so a batch of
// stores at constant distances needs one address register, not a 64-bit
// pointer per store.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// ---------------------------------------------------------------------------
// Element-type traits for q/k/v/o.
// ---------------------------------------------------------------------------
struct BF16 {
  using storage = uint16_t;
  using raw4 = uint2;      // 4 packed elements as loaded
  using raw1 = uint32_t;   // 1 element (low 16 bits)
  __device__ __forceinline__ static raw4 load4raw(const void* base, int64_t idx) {
    return *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + idx);
  }
  __device__ __forceinline__ static void unpack4(raw4 w, float out[4]) {
    out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x);
    out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
  }
  __device__ __forceinline__ static raw1 load1raw(const void* base, int64_t idx) {
    return reinterpret_cast<const uint16_t*>(base)[idx];
  }
  __device__ __forceinline__ static float unpack1(raw1 w) { return __uint_as_float(w << 16); }
  // load 4 consecutive elements as floats (8-byte aligned)
  __device__ __forceinline__ static void load4(const void* base, int64_t idx, float out[4]) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + idx);
    out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x);
    out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
  }
  __device__ __forceinline__ static void store4(void* base, int64_t idx, const float in[4]) {
    uint2 w;
    w.x = pack_bf16x2(in[0], in[1]);
    w.y = pack_bf16x2(in[2], in[3]);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + idx) = w;
  }
  __device__ __forceinline__ static float load1(const void* base, int64_t idx) {
    return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(base)[idx]) << 16);
  }
  __device__ __forceinline__ static void store1(void* base, int64_t idx, float x) {
    reinterpret_cast<uint16_t*>(base)[idx] = uint16_t(f32_to_bf16_rne(x));
  }
  // one element at byte offset off of a buffer resource (dropped past its range)
  __device__ __forceinline__ static void bstore1(__amdgpu_buffer_rsrc_t rs, int off, float x) {
    __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f32_to_bf16_rne(x)), rs, off, 0, 0);
  }
};

struct F32 {
  using storage = float;
  using raw4 = float4;
  using raw1 = float;
  __device__ __forceinline__ static raw4 load4raw(const void* base, int64_t idx) {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
  }
  __device__ __forceinline__ static void unpack4(raw4 w, float out[4]) {
    out[0] = w.x; out[1] = w.y; out[2] = w.z; out[3] = w.w;
  }
  __device__ __forceinline__ static raw1 load1raw(const void* base, int64_t idx) {
    return reinterpret_cast<const float*>(base)[idx];
  }
  __device__ __forceinline__ static float unpack1(raw1 w) { return w; }
  __device__ __forceinline__ static void load4(const void* base, int64_t idx, float out[4]) {
    const float4 w = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    out[0] = w.x; out[1] = w.y; out[2] = w.z; out[3] = w.w;
  }
  __device__ __forceinline__ static void store4(void* base, int64_t idx, const float in[4]) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx) = make_float4(in[0], in[1], in[2], in[3]);
  }
  __device__ __forceinline__ static float load1(const void* base, int64_t idx) {
    return reinterpret_cast<const float*>(base)[idx];
  }
  __device__ __forceinline__ static void store1(void* base, int64_t idx, float x) {
    reinterpret_cast<float*>(base)[idx] = x;
  }
  __device__ __forceinline__ static void bstore1(__amdgpu_buffer_rsrc_t rs, int off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, off, 0, 0);
  }
};

__device__ __forceinline__ float4 ld_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st_f4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

}  // namespace kda

// Device-side types and helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kGroup = 32;        // K elements per scale
constexpr int kChunk = 128;       // K elements per packed chunk (4 scale groups)
constexpr int kRowTile = 16;      // weight rows per MFMA tile
constexpr int kWave = 64;

// Constants the dequantiser combines with one v_and_or_b32 per pair of codes.
// VOP3 encodings on gfx950 take no 32-bit literal, so the masks are pinned in
// VGPRs once per thread (an opaque v_mov keeps the compiler from folding them
// back into two-instruction AND + OR forms).
struct DequantMasks {
  uint32_t lo, hi, magic;
};

__device__ __forceinline__ uint32_t pin_vgpr(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

__device__ __forceinline__ DequantMasks make_dequant_masks() {
  return DequantMasks{pin_vgpr(0x000F000Fu), pin_vgpr(0x00F000F0u), pin_vgpr(0x64006400u)};
}

// Dequantise the 8 INT4 codes of one packed word into the bf16 MFMA operand
// fragment, value e = bf16_rne((q_e - 8) * s).
//
// Subtract-then-scale with one BF16 rounding (Chord W4A16 MoE post, section
// "H200 and Blackwell indexed decode": the fused dequant keeps the unfused
// BF16 rounding order).  Code e sits at bit 4*(e/2) + 16*(e%2) of the word, so
// one AND-OR turns two codes into the fp16 values 1024 + q (low nibble of a
// half) or 1024 + 16 q (high nibble); v_fma_mix_f32 then forms, exactly,
//   (1024 + q) * s - 1032 s  =  (q - 8) s
//   (1024 + 16 q) * (s / 16) - 72 s  =  (q - 8) s
// (the fma rounds once and (q - 8) s fits fp32 exactly: a 4-bit integer times
// an 8-bit significand), and v_cvt_pk_bf16_f32 rounds that to bf16, nearest
// even.  c0 = -1032 s, s16 = s / 16, c1 = -72 s are exact for any scale with
// 2^-100 < |s| < 2^100.  Cost per 8 codes: 1 shift, 4 AND-OR, 8 fma_mix,
// 4 cvt_pk.
__device__ __forceinline__ bf16x8_t dequant8(uint32_t d, float s, float c0, float s16, float c1,
                                             const DequantMasks& m) {
  const uint32_t d8 = d >> 8;
  const f16x2_t h0 = __builtin_bit_cast(f16x2_t, (d & m.lo) | m.magic);
  const f16x2_t h1 = __builtin_bit_cast(f16x2_t, (d & m.hi) | m.magic);
  const f16x2_t h2 = __builtin_bit_cast(f16x2_t, (d8 & m.lo) | m.magic);
  const f16x2_t h3 = __builtin_bit_cast(f16x2_t, (d8 & m.hi) | m.magic);
  bf16x8_t r;
  r[0] = (__bf16)__builtin_fmaf((float)h0.x, s, c0);
  r[1] = (__bf16)__builtin_fmaf((float)h0.y, s, c0);
  r[2] = (__bf16)__builtin_fmaf((float)h1.x, s16, c1);
  r[3] = (__bf16)__builtin_fmaf((float)h1.y, s16, c1);
  r[4] = (__bf16)__builtin_fmaf((float)h2.x, s, c0);
  r[5] = (__bf16)__builtin_fmaf((float)h2.y, s, c0);
  r[6] = (__bf16)__builtin_fmaf((float)h3.x, s16, c1);
  r[7] = (__bf16)__builtin_fmaf((float)h3.y, s16, c1);
  return r;
}

// Source row of row i of packed tile `tile`: with gate_up, packed tile 2t is
// gate tile t (rows 16t..) and packed tile 2t + 1 up tile t (rows N/2 + 16t..)
// (both weight packers)
__device__ __forceinline__ int source_row(int tile, int i, int N, int gate_up) {
  const int t = gate_up ? (tile & 1 ? N / 32 + (tile >> 1) : tile >> 1) : tile;
  return t * kRowTile + i;
}

// Global-memory byte pointer (address space 1: loads through it are
// global_load, never flat_load).
typedef const char __attribute__((address_space(1)))* gptr_t;

// A pointer the caller knows to be the same in every lane, moved to SGPRs so
// address arithmetic on it stays scalar.
template <typename T>
__device__ __forceinline__ gptr_t uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<gptr_t>(((uint64_t)hi << 32) | lo);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t gload_u32x4(gptr_t p) {
  return *reinterpret_cast<const u32x4_t __attribute__((address_space(1)))*>(p);
}

__device__ __forceinline__ uint32_t gload_u32(gptr_t p) {
  return *reinterpret_cast<const uint32_t __attribute__((address_space(1)))*>(p);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
  return __builtin_bit_cast(float, b16 << 16);
}

// Two fp32 -> packed bf16x2 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace w4a16

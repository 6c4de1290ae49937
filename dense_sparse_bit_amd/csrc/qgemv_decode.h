// qgemv_decode.h -- gfx950 device helpers: code unpacking into FP16 pairs,
// LUT lookups through v_perm_b32, fp16x2 -> fp32 dot products, wave64 sums.
//
// The slot layouts decoded here are the ones written by the repacker (see
// qgemv_layout.h).  Every helper is used both by the product kernels and by
// the debug code-unpack kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

namespace qgemv_dev {

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

// v_perm_b32: byte k of the result is byte sel[k] of the 8-byte pool {hi4:lo4};
// selector bytes >= 13 give 0xFF.
__device__ __forceinline__ uint32_t perm(uint32_t hi4, uint32_t lo4, uint32_t sel) {
  return __builtin_amdgcn_perm(hi4, lo4, sel);
}

// fp32 += a.x*b.x + a.y*b.y (v_dot2_f32_f16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// FP16 1024.0 in both halves: OR-ing a value v < 1024 into the mantissa gives 1024 + v exactly.
constexpr uint32_t kMagic = 0x64006400u;

// ---- uniform codes: FP16 pairs (1024 + k*q) per slot -----------------------
// U4: 4 slots per dword, scale k = 1, 16, 1, 16.
__device__ __forceinline__ void u4_slots(uint32_t w, uint32_t h[4]) {
  const uint32_t w8 = w >> 8;
  h[0] = (w & 0x000F000Fu) | kMagic;
  h[1] = (w & 0x00F000F0u) | kMagic;
  h[2] = (w8 & 0x000F000Fu) | kMagic;
  h[3] = (w8 & 0x00F000F0u) | kMagic;
}
// U3: 5 slots per dword (k = 1, 8, 64, 1, 8) and one pair spread over bit 9/25 of 3 dwords (k = 1).
__device__ __forceinline__ void u3_slots(uint32_t w, uint32_t h[5]) {
  const uint32_t w10 = w >> 10;
  h[0] = (w & 0x00070007u) | kMagic;
  h[1] = (w & 0x00380038u) | kMagic;
  h[2] = (w & 0x01C001C0u) | kMagic;
  h[3] = (w10 & 0x00070007u) | kMagic;
  h[4] = (w10 & 0x00380038u) | kMagic;
}
__device__ __forceinline__ uint32_t u3_spare(uint32_t w0, uint32_t w1, uint32_t w2) {
  return ((w0 >> 9) & 0x00010001u) | ((w1 >> 8) & 0x00020002u) | ((w2 >> 7) & 0x00040004u) | kMagic;
}

// ---- LUT codes: v_perm selectors ------------------------------------------
// L4: selector bytes for the A codes (bits 0-2 + flag bit 6) and the B codes
// (bits 3-5 + flag bit 7 moved to bit 4).  A flag sends the byte past index 12,
// so the lookup in the wrong half of the table yields 0xFF.
__device__ __forceinline__ void l4_sel(uint32_t w, uint32_t& sa, uint32_t& sb) {
  sa = w & 0x47474747u;
  sb = (w >> 3) & 0x17171717u;
}
// L3: 8 selectors (4 codes each) from the 3 dwords of a chunk.
__device__ __forceinline__ void l3_sel(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t s[8]) {
  s[0] = w0 & 0x07070707u;
  s[1] = (w0 >> 3) & 0x07070707u;
  s[2] = w1 & 0x07070707u;
  s[3] = (w1 >> 3) & 0x07070707u;
  s[4] = w2 & 0x07070707u;
  s[5] = (w2 >> 3) & 0x07070707u;
  s[6] = ((w0 >> 6) & 0x03030303u) | ((w2 >> 4) & 0x04040404u);
  s[7] = ((w1 >> 6) & 0x03030303u) | ((w2 >> 5) & 0x04040404u);
}

// 16-entry table in byte planes t[0..3] = lo bytes (e0-3, e4-7, e8-11, e12-15),
// t[4..7] = hi bytes.  Returns the FP16 pairs for bytes (0,1) and (2,3) of sel.
__device__ __forceinline__ void l4_lookup(const uint32_t t[8], uint32_t sel, uint32_t flag,
                                          uint32_t& p01, uint32_t& p23) {
  const uint32_t seln = sel ^ flag;
  const uint32_t lo = perm(t[1], t[0], sel) & perm(t[3], t[2], seln);
  const uint32_t hi = perm(t[5], t[4], sel) & perm(t[7], t[6], seln);
  p01 = perm(hi, lo, 0x05010400u);
  p23 = perm(hi, lo, 0x07030602u);
}
// 8-entry table t[0..1] = lo bytes (e0-3, e4-7), t[2..3] = hi bytes.
__device__ __forceinline__ void l3_lookup(const uint32_t t[4], uint32_t sel, uint32_t& p01, uint32_t& p23) {
  const uint32_t lo = perm(t[1], t[0], sel);
  const uint32_t hi = perm(t[3], t[2], sel);
  p01 = perm(hi, lo, 0x05010400u);
  p23 = perm(hi, lo, 0x07030602u);
}

// ---- wave64 reduction (DPP), result valid in every lane --------------------
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_mov<0x140, 0xF>(v);  // row_mirror
  v += dpp_mov<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_mov<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

}  // namespace qgemv_dev

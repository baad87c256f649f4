// codec_dev.h -- device-side bit manipulation for rebuilding BF16 values from a compressed
// tile (codec of the page "GAAC: Lossless KV Compression ...", §3.1: exponent = calibrated
// base + offset, sign and mantissa stored unchanged; §3.2: values are rebuilt on chip).
//
// The rebuild works on one group of 16 tokens of one channel at a time, four tokens per
// 32-bit word ("SWAR"): the 3-bit codes arrive one per byte lane, the escape planes are
// spread to bit 3+p of each byte, the base is added to all four bytes at once (no carry can
// cross a byte since every exponent is <= 255), and two v_perm/v_bfi steps interleave the
// exponent bytes with the stored sign/mantissa bytes into two BF16 pairs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
__device__ __forceinline__ uint32_t bitsel(uint32_t mask, uint32_t a, uint32_t b) { return (a & mask) | (b & ~mask); }

// Codes of slot S (0..7) of a 32-element CODE unit: one 3-bit code per byte lane.  Lane k's
// 24-bit stream holds slot s at bits 3s..3s+2; stream byte w of lane k is byte k of word w.
template <int S>
__device__ __forceinline__ uint32_t code_slot(uint32_t W0, uint32_t W1, uint32_t W2) {
  constexpr int x = 3 * S, w = x / 8, b = x % 8;
  const uint32_t lo = (w == 0 ? W0 : (w == 1 ? W1 : W2));
  if constexpr (b <= 5) {
    return (lo >> b) & 0x07070707u;
  } else if constexpr (b == 6) {
    const uint32_t hi = (w == 0 ? W1 : W2);
    return ((lo >> 6) & 0x03030303u) | ((hi << 2) & 0x04040404u);
  } else {
    const uint32_t hi = (w == 0 ? W1 : W2);
    return ((lo >> 7) & 0x01010101u) | ((hi << 1) & 0x06060606u);
  }
}

// Four bits -> bit 0 of four bytes.
__device__ __forceinline__ uint32_t spread4(uint32_t nib) { return __umul24(nib, 0x00204081u) & 0x01010101u; }

// Rebuild the 16 BF16 values of group GI (0 or 1) of a pair.
//   sm[4]   : the group's sign/mantissa bytes, word j = tokens 4j..4j+3
//   W0..W2  : the pair's CODE unit
//   base    : exponent base of the group's mode (b3, b4 or 0)
//   plane0  : first escape plane (0 for narrow groups); pl[0..3] further planes of a raw group
//   nextra  : number of further planes (0, or 4 for a BF16 raw group)
// Output word j: o02 = BF16 of tokens (4j, 4j+2), o13 = tokens (4j+1, 4j+3), low half first.
template <int GI>
__device__ __forceinline__ void rebuild_group(const uint32_t sm[4], uint32_t W0, uint32_t W1, uint32_t W2,
                                              uint32_t base, uint32_t plane0, const uint32_t pl[4], int nextra,
                                              uint32_t o02[4], uint32_t o13[4]) {
  const uint32_t H = base * 0x01010101u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t cs;
    if (j == 0) cs = code_slot<4 * GI + 0>(W0, W1, W2);
    else if (j == 1) cs = code_slot<4 * GI + 1>(W0, W1, W2);
    else if (j == 2) cs = code_slot<4 * GI + 2>(W0, W1, W2);
    else cs = code_slot<4 * GI + 3>(W0, W1, W2);
    uint32_t esc = spread4((plane0 >> (4 * j)) & 0xFu) << 3;
    if (nextra) {
#pragma unroll
      for (int p = 0; p < 4; ++p) esc |= spread4((pl[p] >> (4 * j)) & 0xFu) << (4 + p);
    }
    const uint32_t E = H + cs + esc;
    const uint32_t s = sm[j];
    o02[j] = bitsel(0x7F807F80u, E << 7, perm_b32(s, s, 0x02020000u));
    o13[j] = bitsel(0x7F807F80u, E >> 1, perm_b32(s, s, 0x03030101u));
  }
}

// Exclusive prefix of escape planes before group q given the tag words holding q (q even
// or odd) and the plane count of all earlier words.  BF16: a wide group has 1 plane, a raw
// group 5 (= 1 + 4).
__device__ __forceinline__ uint32_t planes_before(uint32_t Ew, uint32_t Rw, uint32_t Pw, int bit) {
  const uint32_t below = (bit == 0) ? 0u : (0xFFFFFFFFu >> (32 - bit));
  return Pw + __popc(Ew & below) + 4u * __popc(Rw & below);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace kvc

// codec_dev.h -- device-side bit manipulation for rebuilding BF16 values from a compressed
// tile (codec of the page "GAAC: Lossless KV Compression ...", §3.1: exponent = calibrated
// base + offset, sign and mantissa stored unchanged; §3.2: values are rebuilt on chip).
//
// The rebuild works on one exponent group (16 or 8 tokens of one channel) at a time, four tokens per
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

// Codes of slot S (0..7) of a 32-element CODE unit: one 3-bit code per byte lane, at bits
// SH..SH+2 of the lane (SH <= 3; every other bit is zero).  Lane k's 24-bit stream holds slot s
// at bits 3s..3s+2; stream byte w of lane k is byte k of word w.
template <int S, int SH = 0>
__device__ __forceinline__ uint32_t code_slot(uint32_t W0, uint32_t W1, uint32_t W2) {
  constexpr int x = 3 * S, w = x / 8, b = x % 8;
  const uint32_t lo = (w == 0 ? W0 : (w == 1 ? W1 : W2));
  if constexpr (b <= 5 && b >= SH) {
    return (lo >> (b - SH)) & (0x07070707u << SH);
  } else if constexpr (b <= 5) {
    return (lo << (SH - b)) & (0x07070707u << SH);
  } else if constexpr (b == 6) {
    const uint32_t hi = (w == 0 ? W1 : W2);
    return ((lo >> (6 - SH)) & (0x03030303u << SH)) | ((hi << (2 + SH)) & (0x04040404u << SH));
  } else {
    const uint32_t hi = (w == 0 ? W1 : W2);
    return ((lo >> (7 - SH)) & (0x01010101u << SH)) | ((hi << (1 + SH)) & (0x06060606u << SH));
  }
}

// (a & mask) | (b & ~mask) as one v_bfi_b32.  Written as asm: given chains of constant-mask
// selects the compiler splits them into separate ANDs and an OR3 (two more instructions each).
// The mask goes in a scalar register: it must be the same for every lane (a constant).
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(mask), "v"(a), "v"(b));
  return r;
}

// Sign and mantissa of the E5M2 elements of slot S of an SM unit (3-bit fields sign:mantissa,
// laid out like the exponent codes) at their FP8 bit positions: sign at bit 7, mantissa at bits
// 0..1 of each byte lane (bits 2..6 undefined).
template <int S>
__device__ __forceinline__ uint32_t e5m2_sign_mant(uint32_t W0, uint32_t W1, uint32_t W2) {
  constexpr int x = 3 * S, w = x / 8, b = x % 8;
  const uint32_t lo = (w == 0 ? W0 : (w == 1 ? W1 : W2));
  if constexpr (b <= 5) {
    return bfi(0x80808080u, lo << (5 - b), lo >> b);
  } else {
    const uint32_t hi = (w == 0 ? W1 : W2);
    if constexpr (b == 6) return bfi(0x80808080u, hi << 7, lo >> 6);
    else return bfi(0x80808080u, hi << 6, bfi(0x02020202u, hi << 1, lo >> 7));
  }
}

// Sign and mantissa of four E4M3 elements from y = bytes (a, a, b, b) of an SM word (4-bit
// fields sign:mantissa, low nibble first): elements (a.lo, a.hi, b.lo, b.hi) with the sign at
// bit 7 and the mantissa at bits 0..2 of their byte lanes (bits 3..6 undefined).  Lanes 0 and 1
// (2 and 3) hold the same byte, so y >> 4 brings each low nibble's sign to bit 7 of lane 0 (2)
// and each high nibble's mantissa down to bits 0..2 of lane 1 (3); the other bits are already
// in place in y.
__device__ __forceinline__ uint32_t e4m3_sign_mant(uint32_t y) { return bfi(0x07800780u, y >> 4, y); }

// 24-bit multiply (v_mul_u32_u24, full rate): the low 32 bits of the product of the operands' low
// 24 bits, so both operands must be below 2^24.  Written as asm so that the compiler cannot fold a
// following shift into the constant and fall back to the quarter-rate 32-bit multiply.
__device__ __forceinline__ uint32_t mul_u24(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_mul_u32_u24 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Four bits -> bit 0 of four bytes.
__device__ __forceinline__ uint32_t spread4(uint32_t nib) { return mul_u24(nib, 0x00204081u) & 0x01010101u; }

// Offset bits 4..7 of tokens 4q..4q+3 of a raw group, one per byte lane (bits 4..7 of each
// byte), from the 16-bit escape unit holding their four 4-bit fields (token 4q in the low nibble).
__device__ __forceinline__ uint32_t raw_high_nibbles(uint32_t u16) {
  const uint32_t y = perm_b32(u16, u16, 0x01010000u);
  return ((y << 4) & 0x00F000F0u) | (y & 0xF000F000u);
}

// Rebuild the 16 BF16 values of group GI (0 or 1) of a pair.
//   sm[4]   : the group's sign/mantissa bytes, word q = tokens 4q..4q+3
//   W0..W2  : the pair's CODE unit
//   base    : exponent base of the group's mode (b3, b4 or 0)
//   plane0  : escape plane of offset bit 3 (0 for narrow groups)
//   X[4]    : offset bits 4..7 per byte lane (raw groups), else 0
// Output word q: o02 = BF16 of tokens (4q, 4q+2), o13 = tokens (4q+1, 4q+3), low half first.
template <int GI>
__device__ __forceinline__ void rebuild_group(const uint32_t sm[4], uint32_t W0, uint32_t W1, uint32_t W2,
                                              uint32_t base, uint32_t plane0, const uint32_t X[4],
                                              uint32_t o02[4], uint32_t o13[4]) {
  const uint32_t H = perm_b32(base, base, 0u);  // base in all four bytes
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t cs;
    if (q == 0) cs = code_slot<4 * GI + 0>(W0, W1, W2);
    else if (q == 1) cs = code_slot<4 * GI + 1>(W0, W1, W2);
    else if (q == 2) cs = code_slot<4 * GI + 2>(W0, W1, W2);
    else cs = code_slot<4 * GI + 3>(W0, W1, W2);
    const uint32_t esc = spread4((plane0 >> (4 * q)) & 0xFu);
    const uint32_t E = H + cs + (esc << 3) + X[q];
    const uint32_t s = sm[q];
    o02[q] = bitsel(0x7F807F80u, E << 7, perm_b32(s, s, 0x02020000u));
    o13[q] = bitsel(0x7F807F80u, E >> 1, perm_b32(s, s, 0x03030101u));
  }
}

// Exclusive prefix of escape planes before group q given the tag words holding q (q even
// or odd) and the plane count of all earlier words.  BF16: a wide group has 1 plane, a raw
// group 5 (= 1 + 4).
__device__ __forceinline__ uint32_t planes_before(uint32_t Ew, uint32_t Rw, uint32_t Pw, int bit) {
  const uint32_t below = (bit == 0) ? 0u : (0xFFFFFFFFu >> (32 - bit));
  return Pw + __popc(Ew & below) + 4u * __popc(Rw & below);
}

// Escape units (16-bit units of the tile's escape area) of the split attention's rebuild: a wide
// group holds one, a raw group RU = F - 3.  For group 2n + gi of a tag word (E, R planes Ew, Rw)
// whose earlier words hold Pw units: below = (1 << 2n) - 1, e2 / r2 = bits 2n, 2n+1 of Ew / Rw.
// Returns the unit where the group's escape starts (its planes are units P .. P + RU - 1).
__host__ __device__ inline uint32_t esc_unit_of_group(uint32_t Ew, uint32_t Rw, uint32_t Pw, uint32_t below, uint32_t e2,
                                                      uint32_t r2, int gi, int RU) {
  const uint32_t P0 = Pw + (uint32_t)__builtin_popcount(Ew & below) + (uint32_t)(RU - 1) * (uint32_t)__builtin_popcount(Rw & below);
  return gi ? P0 + (e2 & 1u) + (uint32_t)(RU - 1) * (r2 & 1u) : P0;
}

// Whether the groups of a tag word may read their escape: units_through is the escape units of
// this word and every earlier word of the tile (16 tokens per group; a wide group 1, a raw group
// RU), esc_pieces the 16-byte pieces (8 units each) the tile's table entry says are stored.  A
// word that does not fit (corrupt tags) is rebuilt as narrow; by esc_unit_of_group every group
// of a word that fits ends at or before units_through, inside the stored pieces.
__host__ __device__ inline bool esc_tags_fit(uint32_t units_through, uint32_t esc_pieces) {
  return units_through <= 8u * esc_pieces;
}

// 8-token groups (escape units are bytes).  Whether the groups of a tag word may read their
// escape: bytes_through = escape bytes of this word and every earlier word, esc_pieces = the
// 16-byte pieces staged.
__host__ __device__ inline bool esc_bytes_fit(uint32_t bytes_through, uint32_t esc_pieces) {
  return bytes_through <= 16u * esc_pieces;
}

// 8-token groups: escape byte where the first group of the four-group CODE unit at nibble k
// (0..7) of a tag word starts (E, R planes Ew, Rw; Pw = escape bytes of the earlier words; a
// wide group holds 1 byte, a raw group RU).
__host__ __device__ inline uint32_t g8_unit_escape(uint32_t Ew, uint32_t Rw, uint32_t Pw, int k, int RU) {
  const uint32_t below = (1u << (4 * k)) - 1u;
  return Pw + (uint32_t)__builtin_popcount(Ew & below) + (uint32_t)(RU - 1) * (uint32_t)__builtin_popcount(Rw & below);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace kvc

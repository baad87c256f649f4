// attention_kernels.hip -- split-K decode attention over the paged KV cache and the
// log-sum-exp merge of the splits.
//
// Method: page "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal
// Devices", §3.2 -- the kernel reads compressed tiles and rebuilds only the values attention
// needs on chip (no decompressed copy of the cache in HBM); compressed blocks, raw blocks and
// the uncompressed tail share one softmax normalisation.  The split kernels cover the finished
// blocks; the merge kernel adds the tail.
//
// Work decomposition (one 64-lane wave per workgroup):
//   grid = (split, kv-head, sequence).  A split walks a contiguous range of 64-token
//   super-blocks.  Lane l = n + 16j: j (0..3) selects the 16-token group t0+16j..t0+16j+15 of the
//   super-block, n (0..15) a query head (QK output), a channel pair (rebuild, PV) or an MFMA row.
//   QK   : v_mfma_f32_16x16x32_bf16 with A = K rows (16 tokens x 32 channels) and B = the g query
//          heads (columns n < g used).  Row m of MFMA rb is token 16(m/4) + 4rb + m%4, so lane
//          n + 16j ends up holding the scores of head n for its own token group j.
//   PV   : the same MFMA with A = P (rows = heads, k = 8 tokens of group j per lane) and B = V
//          (k = the same 8 tokens, columns = 16 channels).  A group owner's rebuilt V values are
//          already B operands, so V never touches LDS; P is split into a bf16 high part and a bf16
//          low part (two MFMAs) so the probabilities keep ~16 mantissa bits.
//   K    : group owners rebuild 16 tokens x 2 channels and write them to an XOR-swizzled LDS
//          tile [64 tokens][D] (16-byte chunks, chunk ^ ((row & 3) | ((row >> 2) & 4))) that the
//          QK A-operand reads without bank conflicts.
//   Pipeline: the V bytes of super-block i load while its K is rebuilt and scored, and the K
//          bytes of super-block i+1 load while its V is rebuilt and accumulated, so one half
//          super-block of HBM reads is always in flight per wave.
//   Softmax: online, fp32, base-2 (scores pre-multiplied by scale*log2(e)); per-split outputs
//          (acc, max, sum) go to the workspace and combine_kernel merges them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <math.h>
#include <mutex>
#include <stdint.h>

#include <type_traits>

#include "codec_dev.h"
#include "kvc.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kSB = 64;  // tokens per super-block

enum : int { SRC_COMP = 0, SRC_RAW = 1, SRC_NONE = 2 };

struct AttnArgs {
  Geo G;
  DevBufs B;
  const uint16_t* q;
  float* ws_acc;
  float* ws_ml;
  float sl2;  // scale * log2(e)
  int n_splits;
  const uint8_t* k_new;  // decode step: the new tokens, [n][Hkv][D] elements (else null)
  const uint8_t* v_new;
  // blockIdx.z -> {sequence index i (row of q, k_new, v_new and the workspace), sequence id,
  // tokens in finished blocks, tail position of the new token}; longest sequences first, so the
  // workgroups with the most blocks are dispatched first.  One scalar load per workgroup.
  int4 zrow[kMaxSeqsPerLaunch];
};


// Element format: 0 BF16, 1 FP8 E5M2, 2 FP8 E4M3 (kvc_dtype).
template <int FMT>
struct FmtT {
  static constexpr int F = FMT == 0 ? 8 : (FMT == 1 ? 5 : 4);   // exponent bits
  static constexpr int MB = FMT == 0 ? 7 : (FMT == 1 ? 2 : 3);  // mantissa bits
  static constexpr int EB = FMT == 0 ? 2 : 1;                   // bytes per element
  static constexpr int SMW = FMT == 0 ? 8 : (FMT == 1 ? 3 : 4); // SM words per pair of groups
  // FP8 exponents are rebuilt in place, at bit MB of their byte lane (bases, codes and escape
  // bits all pre-shifted), so that the element byte is one bit-select away; BF16 at bit 0.
  static constexpr int XS = FMT == 0 ? 0 : MB;
  static constexpr uint32_t XMASK = FMT == 0 ? 0xFFFFFFFFu : ((1u << F) - 1u) * (0x01010101u << MB);
  // Rebuilt words of four tokens 4q..4q+3: BF16 pairs (4q, 4q+2), (4q+1, 4q+3) [interleaved];
  // FP8 (converted to BF16) pairs (4q, 4q+1), (4q+2, 4q+3) [natural].
  static constexpr bool NATURAL = FMT != 0;
};

// Compile-time geometry of a compressed tile (FORMAT v1) for head_dim 32*NR, T = TT tokens and
// element format FMT.
// Decode step: the first split of each (sequence, KV head) stores the sequence's new token into
// the tail (K row t, V column t) once its own work is done; the merge kernel that follows reads
// it there.
template <int FMT>
__device__ __forceinline__ void store_new_token(const AttnArgs& a, int si, int seq, int t, int h) {
  constexpr int EB = FmtT<FMT>::EB;
  const Geo& G = a.G;
  uint8_t* tk = reinterpret_cast<uint8_t*>(a.B.tail) + tail_offset(G, seq, 0, h) * EB;
  uint8_t* tv = reinterpret_cast<uint8_t*>(a.B.tail) + tail_offset(G, seq, 1, h) * EB;
  const uint8_t* kn = a.k_new + ((size_t)si * G.Hkv + h) * G.D * EB;
  const uint8_t* vn = a.v_new + ((size_t)si * G.Hkv + h) * G.D * EB;
  for (int c = threadIdx.x; c < G.D; c += blockDim.x) {
    if constexpr (EB == 2) {
      reinterpret_cast<uint16_t*>(tk)[(size_t)t * G.D + c] = reinterpret_cast<const uint16_t*>(kn)[c];
      reinterpret_cast<uint16_t*>(tv)[(size_t)c * G.T + t] = reinterpret_cast<const uint16_t*>(vn)[c];
    } else {
      tk[(size_t)t * G.D + c] = kn[c];
      tv[(size_t)c * G.T + t] = vn[c];
    }
  }
}

template <int NR, int TT, int FMT>
struct TG {
  static constexpr int D = 32 * NR;
  static constexpr int NT = TT / 16;
  static constexpr int NG = NT * D;
  static constexpr int PW = NG / 32;
  static constexpr int CODE_OFF = (2 * PW * 4 + 15) / 16 * 16;
  static constexpr int SM_OFF = CODE_OFF + (TT * D * 3 / 8 + 15) / 16 * 16;
  static constexpr int ESC_OFF = SM_OFF + (TT * D * (1 + FmtT<FMT>::MB) / 8 + 15) / 16 * 16;
  static constexpr int RAW = TT * D;  // elements of a raw tile
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two FP8 values (bytes 2*HI, 2*HI+1 of x) -> two BF16 (low half = the lower byte); exact.
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t x) {
  if constexpr (FMT == 1) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(x, 1.0f, HI));
  else return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI));
}

// Eight FP8 values (tokens or channels in order) -> an MFMA operand of eight BF16.
template <int FMT>
__device__ __forceinline__ uint4 fp8x8_to_operand(uint2 v) {
  return make_uint4(fp8x2_to_bf16x2<FMT, false>(v.x), fp8x2_to_bf16x2<FMT, true>(v.x),
                    fp8x2_to_bf16x2<FMT, false>(v.y), fp8x2_to_bf16x2<FMT, true>(v.y));
}

__device__ __forceinline__ uint2 ld64(const void* p) { return *reinterpret_cast<const uint2*>(p); }

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack2(float a, float b) { return bf16_bits(a) | (bf16_bits(b) << 16); }
__device__ __forceinline__ float bf16_round(float f) { return (float)(__bf16)f; }

__device__ __forceinline__ uint4 ld128(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t ld32(const void* p) { return *reinterpret_cast<const uint32_t*>(p); }

__device__ __forceinline__ int swz(int row) { return (row & 3) | ((row >> 2) & 4); }

// Inclusive prefix sum over the 16 lanes of a DPP row.
__device__ __forceinline__ uint32_t row_scan16(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  return v;
}

// Where the 16-token group starting at token t of one (sequence, K|V, head) lives.
struct TileRef {
  int kind;              // bits 0..1: SRC_COMP, SRC_RAW (raw tile), SRC_NONE; above them (compressed
                         // tiles) the offset of the tile's base version in the packed LDS bases
  int tg;                // token group inside the tile
  int escu;              // escape bytes / 16 (compressed)
  const uint8_t* p;      // the compressed or raw tile; for SRC_NONE a dummy tile-sized area (the
                         // tail buffer), so every load a kernel issues from it stays in bounds
  __device__ __forceinline__ int src() const { return kind & 3; }
  __device__ __forceinline__ int bo() const { return kind >> 2; }
  __device__ __forceinline__ int valid() const { return src() == SRC_NONE ? 0 : 16; }
};

// L here is the token count of the finished blocks (a multiple of T): the tail is merged in
// by combine_kernel.
template <int TT>
__device__ __forceinline__ uint32_t load_entry(const AttnArgs& a, int seq, int L, int t, int kv, int h) {
  if (t >= L) return kUnallocated;
  return a.B.table[table_index(a.G, seq, t / TT, kv, h)];
}

// Status bit 4 if any lane's group inside the finished blocks has no table entry.  Called in
// wave-uniform control flow; the result is wave-uniform (kept in a scalar register).
__device__ __forceinline__ uint32_t missing_flag(int L, int t, uint32_t entry) {
  return __builtin_amdgcn_ballot_w64(t < L && entry == kUnallocated) ? 4u : 0u;
}

template <int NR, int TT, int FMT>
__device__ __forceinline__ TileRef tile_ref(const AttnArgs& a, int seq, int L, int t, int kv, int h, uint32_t entry) {
  TileRef r;
  r.kind = SRC_NONE;
  r.tg = (t % TT) >> 4;
  r.escu = 0;
  r.p = reinterpret_cast<const uint8_t*>(a.B.tail);
  if (t >= L || entry == kUnallocated) {  // past the finished blocks, or missing (missing_flag)
    r.tg = 0;
    return r;
  }
  const uint32_t slot = entry_slot(entry);
  if (entry & kRawTile) {
    r.kind = SRC_RAW;
    r.p = reinterpret_cast<const uint8_t*>(a.B.raw_pool) + (size_t)slot * TG<NR, TT, FMT>::RAW * FmtT<FMT>::EB;
  } else {
    r.kind = SRC_COMP | (entry_version(entry) * (2 * NR * 16)) << 2;  // and the bases it was encoded with
    r.p = a.B.comp_pool + (size_t)slot * (uint32_t)a.G.stride;
    r.escu = min(entry_esc_units(entry), a.G.esc_cap >> 4);  // never past the slot's escape area
  }
  return r;
}

// Compressed bytes of one tile (K or V) held by one lane: tag words (lanes n < PW), escape
// bytes (lanes n < escu, two 16-byte pieces), and sign/mantissa + code words of its NR pairs
// (SM: 32 bytes per pair for BF16, 12 for E5M2, 16 for E4M3).
template <int NR, int FMT>
struct SmRegs {
  uint32_t w[NR][FmtT<FMT>::SMW];
};
template <int NR>
struct SmRegs<NR, 0> {  // BF16: two 16-byte pieces per pair (one per group)
  uint4 v[NR][2];
};

template <int NR, int FMT>
struct CRegs {
  uint32_t tE, tR;
  uint4 esc0, esc1;
  SmRegs<NR, FMT> sm;
  uint32_t cd[NR][3];
};

// esc_loader: this lane's group stages the tile's escape bytes (with 64-token blocks the four
// lane groups hold the same tile and group 0 stages them for all).
template <int NR, int TT, int FMT>
__device__ __forceinline__ void load_tile(const TileRef& r, int n, CRegs<NR, FMT>& c, bool esc_loader) {
  using Q = TG<NR, TT, FMT>;
  const uint8_t* t = r.p;  // a raw or dummy tile is large enough for every load below
  c.tE = c.tR = 0;
  if (n < Q::PW) {
    c.tE = ld32(t + 4 * n);
    c.tR = ld32(t + 4 * (Q::PW + n));
  }
  c.esc0 = c.esc1 = make_uint4(0, 0, 0, 0);
  if (esc_loader && n < r.escu) c.esc0 = ld128(t + Q::ESC_OFF + 16 * n);
  if (esc_loader && n + 16 < r.escu) c.esc1 = ld128(t + Q::ESC_OFF + 16 * (n + 16));
  // one base per section for this lane's first pair; round i adds 16 pairs (immediate offsets)
  const uint32_t pr0 = (uint32_t)(r.tg * (Q::D / 2) + n);
  const uint8_t* smb = t + Q::SM_OFF + (FMT == 0 ? 32u : FMT == 1 ? 12u : 16u) * pr0;
  const uint8_t* cpb = t + Q::CODE_OFF + 12u * pr0;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if constexpr (FMT == 0) {
      c.sm.v[i][0] = ld128(smb + 32 * 16 * i);
      c.sm.v[i][1] = ld128(smb + 32 * 16 * i + 16);
    } else if constexpr (FMT == 1) {
      const uint8_t* sp = smb + 12 * 16 * i;
      c.sm.w[i][0] = ld32(sp); c.sm.w[i][1] = ld32(sp + 4); c.sm.w[i][2] = ld32(sp + 8);
    } else {
      const uint4 a = ld128(smb + 16 * 16 * i);
      c.sm.w[i][0] = a.x; c.sm.w[i][1] = a.y; c.sm.w[i][2] = a.z; c.sm.w[i][3] = a.w;
    }
    const uint8_t* cp = cpb + 12 * 16 * i;
    c.cd[i][0] = ld32(cp);
    c.cd[i][1] = ld32(cp + 4);
    c.cd[i][2] = ld32(cp + 8);
  }
}

// Stage the escape bytes of this lane group's tile into its LDS area; return the exclusive
// escape-unit prefix of tag word n (a wide group has 1 unit, a raw group F - 3).  A tag word
// whose groups would end past the escape units the table entry staged (corrupt tags) is
// flagged (bad) and cleared, prefix 0: its groups rebuild as narrow and read unit 0 only.  The
// prefix grows with n, so every later word of that tile is cleared too, and the words kept
// read only staged units.
template <int NR, int FMT>
__device__ __forceinline__ uint32_t stage_escape(CRegs<NR, FMT>& c, const TileRef& r, int n, uint8_t* esc_lds,
                                                 bool esc_loader, uint32_t& bad) {
  if (esc_loader && r.src() == SRC_COMP) {
    if (n < r.escu) *reinterpret_cast<uint4*>(esc_lds + 16 * n) = c.esc0;
    if (n + 16 < r.escu) *reinterpret_cast<uint4*>(esc_lds + 16 * (n + 16)) = c.esc1;
  }
  // escape units per group: wide 1, raw F - 3 (the E plane counts 1 for both)
  const uint32_t cnt = __popc(c.tE) + (uint32_t)(FmtT<FMT>::F - 4) * __popc(c.tR);
  const uint32_t incl = row_scan16(cnt);
  if (r.src() == SRC_COMP && !esc_tags_fit(incl, (uint32_t)r.escu)) {
    bad |= 1u;
    c.tE = c.tR = 0u;
    return 0u;
  }
  return incl - cnt;
}

// Escape spread table: entry v holds exponent bit 3 set in byte k for every set bit k of v (the
// plane bits of four tokens moved to exponent bit 3 of their byte lanes; for FP8 the exponent
// sits at bit MB of the lane).  Lives at LDS offset 0 of every attention workgroup.
__shared__ uint32_t esc_lut[16];

template <int FMT>
__device__ __forceinline__ void init_esc_lut() {
  if (threadIdx.x < 16) esc_lut[threadIdx.x] = spread4(threadIdx.x) << (3 + FmtT<FMT>::XS);
}


// Rebuild the two groups of round i for lane n of lane group j.  bases packs b3[c0], b3[c1],
// b4[c0], b4[c1]; below = (1 << 2n) - 1.  Output, low half first: BF16 o[gi][0][q] = tokens
// (4q, 4q+2), o[gi][1][q] = (4q+1, 4q+3); FP8 (converted exactly to BF16) o[gi][0][q] = tokens
// (4q, 4q+1), o[gi][1][q] = (4q+2, 4q+3).
// The tag words E, R and escape prefix P of round i's pair, for every round of a tile, fetched
// together (the cross-lane reads of all rounds are in flight at once).
template <int NR, int FMT>
__device__ __forceinline__ void fetch_tags(const CRegs<NR, FMT>& c, int j, int tg, uint32_t pfx, uint32_t t[NR][3]) {
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int w = tg * NR + i;
    t[i][0] = (uint32_t)__shfl((int)c.tE, 16 * j + w);
    t[i][1] = (uint32_t)__shfl((int)c.tR, 16 * j + w);
    t[i][2] = (uint32_t)__shfl((int)pfx, 16 * j + w);
  }
}

template <int NR, int FMT>
__device__ __forceinline__ void rebuild_round(const CRegs<NR, FMT>& c, int i, int j, int n, const uint32_t tw[3],
                                              uint32_t bases, const uint16_t* esc16, uint32_t below, uint32_t& bad,
                                              uint32_t o[2][2][4]) {
  constexpr int RU = FmtT<FMT>::F - 3;  // escape units of a raw group
  const uint32_t Ew = tw[0], Rw = tw[1], Pw = tw[2];
  bad |= Rw & ~Ew;
  if constexpr (FMT == 2) bad |= Ew & ~Rw;  // no wide mode in a 4-bit exponent field
  const uint32_t e2 = __builtin_amdgcn_ubfe(Ew, 2 * n, 2), r2 = __builtin_amdgcn_ubfe(Rw, 2 * n, 2);
  const uint32_t W0 = c.cd[i][0], W1 = c.cd[i][1], W2 = c.cd[i][2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const uint32_t E = (e2 >> gi) & 1u, R = (r2 >> gi) & 1u;
    const uint32_t P = esc_unit_of_group(Ew, Rw, Pw, below, e2, r2, gi, RU);
    // base in all four bytes: byte gi (b3) or 2 + gi (b4) of `bases`, 0 for a raw group
    const uint32_t sel = R ? 0x0C0C0C0Cu : E * 0x02020202u + (uint32_t)gi * 0x01010101u;
    const uint32_t H = perm_b32(0u, bases, sel);
    const uint32_t pw = esc16[P];                                             // read always,
    const uint32_t plane0 = E ? pw : 0u;                                      // keep if escaped
    uint32_t Evq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int slot = 4 * gi + q;
      constexpr int XS = FmtT<FMT>::XS;
      const uint32_t cs = slot == 0 ? code_slot<0, XS>(W0, W1, W2) : slot == 1 ? code_slot<1, XS>(W0, W1, W2)
                        : slot == 2 ? code_slot<2, XS>(W0, W1, W2) : slot == 3 ? code_slot<3, XS>(W0, W1, W2)
                        : slot == 4 ? code_slot<4, XS>(W0, W1, W2) : slot == 5 ? code_slot<5, XS>(W0, W1, W2)
                        : slot == 6 ? code_slot<6, XS>(W0, W1, W2) : code_slot<7, XS>(W0, W1, W2);
      Evq[q] = H + cs + esc_lut[(plane0 >> (4 * q)) & 0xFu];
    }
    if constexpr (FMT == 0) {
      if (R) {  // raw group (rare): base 0; offset bits 4..7 of each token go into its exponent byte
        // four 16-bit units P+1 .. P+4 (only 2-byte aligned in general: read one by one)
        const uint32_t hx = (uint32_t)esc16[P + 1] | ((uint32_t)esc16[P + 2] << 16);
        const uint32_t hy = (uint32_t)esc16[P + 3] | ((uint32_t)esc16[P + 4] << 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t u = q < 2 ? hx : hy;
          const uint32_t y = perm_b32(u, u, (q & 1) ? 0x03030202u : 0x01010000u);
          Evq[q] += ((y << 4) & 0x00F000F0u) | (y & 0xF000F000u);
        }
      }
    } else if constexpr (FMT == 1) {
      if (R) {  // raw group (rare): offset bit 4 of each token from unit P+1
        const uint32_t u = esc16[P + 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) Evq[q] += esc_lut[(u >> (4 * q)) & 0xFu] << 1;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int slot = 4 * gi + q;
      const uint32_t Ev = Evq[q];
      if constexpr (FMT == 0) {
        const uint4 s4 = c.sm.v[i][gi];
        const uint32_t sv = q == 0 ? s4.x : q == 1 ? s4.y : q == 2 ? s4.z : s4.w;
        o[gi][0][q] = bitsel(0x7F807F80u, Ev << 7, perm_b32(sv, sv, 0x02020000u));
        o[gi][1][q] = bitsel(0x7F807F80u, Ev >> 1, perm_b32(sv, sv, 0x03030101u));
      } else {
        uint32_t g;  // sign at bit 7, mantissa at bits 0..MB-1 of each byte lane
        if constexpr (FMT == 1) {
          const uint32_t S0 = c.sm.w[i][0], S1 = c.sm.w[i][1], S2 = c.sm.w[i][2];
          g = slot == 0 ? e5m2_sign_mant<0>(S0, S1, S2) : slot == 1 ? e5m2_sign_mant<1>(S0, S1, S2)
            : slot == 2 ? e5m2_sign_mant<2>(S0, S1, S2) : slot == 3 ? e5m2_sign_mant<3>(S0, S1, S2)
            : slot == 4 ? e5m2_sign_mant<4>(S0, S1, S2) : slot == 5 ? e5m2_sign_mant<5>(S0, S1, S2)
            : slot == 6 ? e5m2_sign_mant<6>(S0, S1, S2) : e5m2_sign_mant<7>(S0, S1, S2);
        } else {
          const uint32_t sw = c.sm.w[i][2 * gi + (q >> 1)];
          g = e4m3_sign_mant(perm_b32(sw, sw, (q & 1) ? 0x03030202u : 0x01010000u));
        }
        const uint32_t B = bfi(FmtT<FMT>::XMASK, Ev, g);  // the four FP8 bytes
        o[gi][0][q] = fp8x2_to_bf16x2<FMT, false>(B);
        o[gi][1][q] = fp8x2_to_bf16x2<FMT, true>(B);
      }
    }
  }
}

// Online-softmax state update for one super-block.  s[16]: this lane's 16 scores (already in
// base-2 units, masked to -inf); they are replaced by probabilities; returns the rescale factor.
__device__ __forceinline__ float softmax_update(float s[16], float& m, float& l) {
  float mx = s[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) mx = fmaxf(mx, s[k]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m, mx);
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m - m_use);
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    s[k] = __builtin_amdgcn_exp2f(s[k] - m_use);
    sum += s[k];
  }
  l = l * alpha + sum;
  m = m_new;
  return alpha;
}

template <int NR>
__device__ __forceinline__ void rescale_acc(f32x4_t acc[NR][2], float alpha, int j) {
  // lane 16j + n takes the factors of query heads 4j .. 4j+3 (lanes 4j + r): byte addresses
  // (lane & 48) + 4r.  Formed here, on this rarely taken path, behind a volatile asm so that
  // they are not hoisted out of the loop and kept live across it.
  (void)j;
  uint32_t base;
  asm volatile("v_and_b32 %0, 48, %1" : "=v"(base) : "v"((uint32_t)threadIdx.x));
  float a[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    a[r] = __int_as_float(__builtin_amdgcn_ds_bpermute((int)(base + 4 * r), __float_as_int(alpha)));
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][x][r] *= a[r];
}

// P as MFMA A operands (high and low bf16 parts).  INTERLEAVED: token order (0,2,1,3,4,6,5,7)
// matching the rebuilt V words; otherwise natural order.  Two values per conversion: the high
// part is the round-to-nearest-even BF16 pair, the low part the BF16 pair of the exact
// remainders.
template <bool INTERLEAVED>
__device__ __forceinline__ void pack_p(const float p[16], uint4 hi[2], uint4 lo[2]) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const int k0 = 2 * k2, k1 = 2 * k2 + 1;
      const int s0 = INTERLEAVED ? ((k0 & 4) | ((k0 & 1) << 1) | ((k0 >> 1) & 1)) : k0;
      const int s1 = INTERLEAVED ? ((k1 & 4) | ((k1 & 1) << 1) | ((k1 >> 1) & 1)) : k1;
      const float a = p[8 * e + s0], b = p[8 * e + s1];
      h[k2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
      const float al = a - __uint_as_float(h[k2] << 16), bl = b - __uint_as_float(h[k2] & 0xFFFF0000u);
      l[k2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){al, bl}, bf16x2_t));
    }
    hi[e] = make_uint4(h[0], h[1], h[2], h[3]);
    lo[e] = make_uint4(l[0], l[1], l[2], l[3]);
  }
}

template <int NR>
__device__ __forceinline__ void write_partial(const AttnArgs& a, int si, int h, int split, float m, float l,
                                              f32x4_t acc[NR][2]) {
  const int lane = threadIdx.x, n = lane & 15, j = lane >> 4;
  const Geo& G = a.G;
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  const int S = a.n_splits;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int head = 4 * j + r;
    if (head < G.g) {
      float* dst = a.ws_acc + (((size_t)si * G.Hq + h * G.g + head) * S + split) * (32 * NR);
#pragma unroll
      for (int i = 0; i < NR; ++i)
        *reinterpret_cast<float2*>(dst + 32 * i + 2 * n) = make_float2(acc[i][0][r], acc[i][1][r]);
    }
  }
  if (j == 0 && n < G.g) {
    float* ml = a.ws_ml + (((size_t)si * G.Hq + h * G.g + n) * S + split) * 2;
    ml[0] = m;
    ml[1] = lt;
  }
}

// Zero the bf16 lanes of a natural-order 8-token V operand past `keep` valid tokens.
__device__ __forceinline__ uint4 mask_tokens(uint4 v, int keep) {
  if (keep >= 8) return v;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t m = (2 * k < keep ? 0x0000FFFFu : 0u) | (2 * k + 1 < keep ? 0xFFFF0000u : 0u);
    w[k] &= m;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Super-blocks [sb0, sb1) of split `split` (L = tokens of the finished blocks): the full 64-token
// super-blocks are dealt out as evenly as possible (the first nfull % n_splits splits take one
// more), and the last split also takes the partial last super-block, if any (blocks of T < 64
// tokens that do not fill one).  Its share of full ones is never above the others',
// so a length just past a multiple of 64 * n_splits puts one extra super-block on a few splits
// instead of on all of them.
__device__ __forceinline__ void split_range(int L, int n_splits, int split, int& sb0, int& sb1) {
  const int nfull = L / kSB, base = nfull / n_splits, rem = nfull % n_splits;
  sb0 = split * base + min(split, rem);
  sb1 = sb0 + base + (split < rem ? 1 : 0);
  if (split == n_splits - 1 && (L % kSB)) sb1 += 1;
}

// Visit order of a split's super-blocks: the split holding the partial last super-block takes
// it first, while its first full super-block's bytes are still in flight, instead of adding it
// to the end of the kernel's longest split.
struct SbOrder {
  int sb0, cnt, rot;
  __device__ __forceinline__ SbOrder(int L, int n_splits, int split) {
    int sb1;
    split_range(L, n_splits, split, sb0, sb1);
    cnt = sb1 - sb0;
    rot = (split == n_splits - 1 && (L % kSB) && cnt > 1) ? cnt - 1 : 0;
  }
  __device__ __forceinline__ int at(int it) const {
    int x = it + rot;
    if (x >= cnt) x -= cnt;
    return sb0 + x;
  }
};

// First token of lane group j's 16-token group in super-block sb.
__device__ __forceinline__ int group_token(int sb, int j) { return sb * kSB + 16 * j; }

// Co-resident waves of a SIMD issue in age order when their priorities are equal, so the wave
// dispatched first runs ahead and the later one finishes alone, at a fraction of the SIMD's
// issue rate.  Each wave lowers its priority as its remaining work shrinks (rp = K and V phases
// left, the current one included): the wave that is behind wins the issue slot, and waves that
// share a SIMD finish together.
__device__ __forceinline__ void phase_priority(int rp) {
  if (rp >= 6) __builtin_amdgcn_s_setprio(3);
  else if (rp >= 4) __builtin_amdgcn_s_setprio(2);
  else if (rp >= 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// ------------------------------------------------------------------------------------------
// b3[c0], b3[c0+1], b4[c0], b4[c0+1] of base version ver for packed-bases slot k = (K|V, round i,
// lane n): c0 = 32i + 2n, one byte each.
template <int NR, int FMT>
__device__ __forceinline__ uint32_t packed_bases(const Geo& G, const uint8_t* bases, int ver, int k, int h) {
  const int kv = k / (NR * 16), i = (k / 16) % NR, nn = k % 16, c0 = 32 * i + 2 * nn;
  const uint8_t* b3 = bases_of(G, bases, ver, 3, kv, h);
  const uint8_t* b4 = bases_of(G, bases, ver, 4, kv, h);
  const uint32_t w = b3[c0] | (b3[c0 + 1] << 8) | (b4[c0] << 16) | (b4[c0 + 1] << 24);
  return w << FmtT<FMT>::XS;  // FP8 bases are < 32: each byte stays in its lane
}

// Compressed cache.
template <int NR, int TT, int FMT>
__global__ void __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_comp_kernel(AttnArgs a) {
  using Q = TG<NR, TT, FMT>;
  constexpr bool NAT = FmtT<FMT>::NATURAL;
  constexpr int D = Q::D;
  extern __shared__ uint4 lds4[];
  const Geo& G = a.G;
  const int esc_room = max(G.esc_cap, 16);
  uint8_t* klds = reinterpret_cast<uint8_t*>(lds4);              // [64][D] bf16, swizzled
  // escape staging: one area per lane group; with 64-token blocks the four lane groups hold the
  // same tile (one block per super-block) and share one copy
  constexpr int kEscAreas = TT == kSB ? 1 : 4;
  uint8_t* esc_base = klds + kSB * D * 2;                         // [kEscAreas][esc_room]
  uint4* qlds = reinterpret_cast<uint4*>(esc_base + kEscAreas * esc_room);  // [g][D/8] query chunks
  uint32_t* blds = reinterpret_cast<uint32_t*>(qlds + G.g * (D / 8));  // [version][2][NR][16] packed bases
  const int lane = threadIdx.x, n = lane & 15, j = lane >> 4;
  const int split = blockIdx.x, h = blockIdx.y;
  const int4 z = a.zrow[blockIdx.z];
  const int si = z.x, seq = z.y, L = z.z;
  const SbOrder ord(L, a.n_splits, split);
  uint8_t* esc_lds = esc_base + (kEscAreas == 1 ? 0 : j * esc_room);
  const bool esc_loader = kEscAreas > 1 || j == 0;  // the lanes that load and stage escape bytes
  const uint16_t* esc16 = reinterpret_cast<const uint16_t*>(esc_lds);
  const uint32_t below = (1u << (2 * n)) - 1u;
  uint32_t flags = 0, bad = 0;
  init_esc_lut<FMT>();

  // Prologue: one memory round trip before the first tile loads.  The first super-block's
  // table entries, the query heads h*g .. h*g+g-1 (g * D/8 <= 256 chunks: at most four per lane)
  // and the calibrated bases of every lane's channel pairs are all requested together; the
  // query and the bases go to LDS (keeping the per-lane register budget at two waves per SIMD)
  // only after the first tiles' loads are in flight.
  uint32_t eK = kUnallocated, eV = kUnallocated;
  if (ord.cnt > 0) {
    eK = load_entry<TT>(a, seq, L, group_token(ord.at(0), j), 0, h);
    eV = load_entry<TT>(a, seq, L, group_token(ord.at(0), j), 1, h);
  }
  uint4 qr[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int k = lane + kWave * u;
    qr[u] = k < G.g * (D / 8) ? ld128(a.q + ((size_t)si * G.Hq + h * G.g) * D + 8 * k) : make_uint4(0, 0, 0, 0);
  }
  // the packed bases of base version 0 (every cache has it)
  constexpr int BU = 2 * NR * 16 / kWave;
  uint32_t br[BU];
#pragma unroll
  for (int u = 0; u < BU; ++u) br[u] = packed_bases<NR, FMT>(G, a.B.bases, 0, lane + kWave * u, h);

  float m = -INFINITY, l = 0.0f;
  f32x4_t acc[NR][2];
#pragma unroll
  for (int i = 0; i < NR; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  CRegs<NR, FMT> cK, cV;
  TileRef rK, rV;
  if (ord.cnt > 0) {
    rK = tile_ref<NR, TT, FMT>(a, seq, L, group_token(ord.at(0), j), 0, h, eK);
    flags |= missing_flag(L, group_token(ord.at(0), j), eK);
    load_tile<NR, TT, FMT>(rK, n, cK, esc_loader);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (lane + kWave * u < G.g * (D / 8)) qlds[lane + kWave * u] = qr[u];
#pragma unroll
  for (int u = 0; u < BU; ++u) blds[lane + kWave * u] = br[u];
  // further base versions (a recalibrated cache), after the first tile loads are in flight
  for (int v = 1; v < G.n_versions; ++v)
#pragma unroll
    for (int u = 0; u < BU; ++u) blds[v * 2 * NR * 16 + lane + kWave * u] = packed_bases<NR, FMT>(G, a.B.bases, v, lane + kWave * u, h);

  if (ord.cnt > 0) {
    for (int it = 0; it < ord.cnt; ++it) {
      phase_priority(2 * (ord.cnt - it));
      const int sb = ord.at(it);
      // V bytes of this super-block load while K is rebuilt and scored
      rV = tile_ref<NR, TT, FMT>(a, seq, L, group_token(sb, j), 1, h, eV);
      flags |= missing_flag(L, group_token(sb, j), eV);
      load_tile<NR, TT, FMT>(rV, n, cV, esc_loader);
      if (it + 1 < ord.cnt) {
        eK = load_entry<TT>(a, seq, L, group_token(ord.at(it + 1), j), 0, h);
        eV = load_entry<TT>(a, seq, L, group_token(ord.at(it + 1), j), 1, h);
      }

      // ---- K: rebuild into the LDS tile ----
      __syncthreads();
      const uint32_t pfxK = stage_escape<NR, FMT>(cK, rK, n, esc_lds, esc_loader, bad);
      __syncthreads();
      if (rK.src() == SRC_COMP) {
        uint32_t tags[NR][3];
        // the tile's base version: one per wave with 64-token blocks (a scalar), else per lane group
        const int boK = kEscAreas == 1 ? __builtin_amdgcn_readfirstlane(rK.bo()) : rK.bo();
        fetch_tags<NR, FMT>(cK, j, rK.tg, pfxK, tags);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          uint32_t o[2][2][4];
          rebuild_round<NR, FMT>(cK, i, j, n, tags[i], blds[boK + i * 16 + n], esc16, below, bad, o);
          // transpose to token-major rows: token 16j + 4q + k gets the (c0, c0+1) word, taken
          // from one half of each of the two channels' token-pair words (BF16: word k & 1, half
          // k >> 1; FP8: word k >> 1, half k & 1)
          const int chunk = 4 * i + (n >> 2), off = 4 * (n & 3);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int rk = 16 * j + k;  // row of quad 0; quad q adds 4q rows (same swizzle)
            uint8_t* p = klds + rk * 2 * D + ((chunk ^ swz(rk)) << 4) + off;
            const int wi = NAT ? (k >> 1) : (k & 1);
            const uint32_t sel = (NAT ? (k & 1) : (k >> 1)) ? 0x07060302u : 0x05040100u;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<uint32_t*>(p + q * 4 * 2 * D) = perm_b32(o[1][wi][q], o[0][wi][q], sel);
          }
        }
      }
      // Raw K groups (raw tiles).  BF16: straight from memory into their LDS rows with
      // LDS-DMA loads: one instruction fills RPI whole rows (64 lanes x 16 bytes), each lane
      // fetching the row piece whose swizzled position is its own, so a group costs one memory
      // round trip and no registers.  FP8: eight-element pieces through registers, converted
      // to BF16 on the way.  Rows past the valid tokens hold stale but finite-or-not data;
      // their scores are masked before the softmax.
      if constexpr (FMT != 0) {
        if (rK.src() == SRC_RAW) {
          constexpr int NCH = D / 8;  // 8-element pieces per row; lane n takes pieces n, n+16, ...
#pragma unroll
          for (int m0 = 0; m0 < NCH; m0 += 4) {
            uint2 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int k = n + 16 * (m0 + u), rr = k / NCH, chunk = k % NCH;
              v[u] = ld64(rK.p + (size_t)(rK.tg * 16 + rr) * D + 8 * chunk);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int k = n + 16 * (m0 + u), rr = k / NCH, chunk = k % NCH, row = 16 * j + rr;
              *reinterpret_cast<uint4*>(klds + row * 2 * D + ((chunk ^ swz(row)) << 4)) = fp8x8_to_operand<FMT>(v[u]);
            }
          }
        }
      } else {
        constexpr int RPI = 512 / D;  // rows per instruction
        constexpr int LPR = D / 8;    // lanes (16-byte pieces) per row
        bool dma = false;
#pragma unroll 1
        for (int g = 0; g < 4; ++g) {
          if ((__builtin_amdgcn_readlane(rK.kind, 16 * g) & 3) != SRC_RAW) continue;
          const uint64_t rp = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)((uintptr_t)rK.p >> 32), 16 * g) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)(uintptr_t)rK.p, 16 * g);
          const int tg_g = __builtin_amdgcn_readlane(rK.tg, 16 * g);
          const uint16_t* raw_g = reinterpret_cast<const uint16_t*>(rp) + (size_t)tg_g * 16 * D;
#pragma unroll 1
          for (int i = 0; i < 16 / RPI; ++i) {
            const int row = 16 * g + RPI * i + lane / LPR, pos = lane % LPR;
            const int chunk = pos ^ swz(row);
            __builtin_amdgcn_global_load_lds(raw_g + (size_t)(row - 16 * g) * D + 8 * chunk,
                                             (__attribute__((address_space(3))) void*)(klds + (16 * g + RPI * i) * 2 * D),
                                             16, 0, 0);
          }
          dma = true;
        }
        if (dma) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the DMA has landed in LDS
      }
      __syncthreads();

      // ---- QK and softmax ----
      const int valid = min(rK.valid(), rV.valid());
      f32x4_t cc[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) cc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NR; ++ks) {
        uint4 qv = qlds[min(n, G.g - 1) * (D / 8) + 4 * ks + j];
        if (n >= G.g) qv = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int row = 16 * (n >> 2) + 4 * rb + (n & 3);
          const uint4 av = *reinterpret_cast<const uint4*>(klds + row * 2 * D + (((4 * ks + j) ^ swz(row)) << 4));
          cc[rb] = mfma16(av, qv, cc[rb]);
        }
      }
      float s[16];
      if (__builtin_amdgcn_ballot_w64(valid < 16)) {  // a group past the finished blocks (T < 64)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[4 * rb + r] = (4 * rb + r < valid) ? cc[rb][r] * a.sl2 : -INFINITY;
      } else {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[4 * rb + r] = cc[rb][r] * a.sl2;
      }
      const float alpha = softmax_update(s, m, l);
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) rescale_acc<NR>(acc, alpha, j);  // a running max moved
      uint4 phi[2], plo[2];
      pack_p<!NAT>(s, phi, plo);

      // K bytes of the next super-block load while V is rebuilt and accumulated
      if (it + 1 < ord.cnt) {
        rK = tile_ref<NR, TT, FMT>(a, seq, L, group_token(ord.at(it + 1), j), 0, h, eK);
        flags |= missing_flag(L, group_token(ord.at(it + 1), j), eK);
        load_tile<NR, TT, FMT>(rK, n, cK, esc_loader);
      }

      phase_priority(2 * (ord.cnt - it) - 1);
      // ---- V: rebuild straight into B operands ----
      __syncthreads();
      const uint32_t pfxV = stage_escape<NR, FMT>(cV, rV, n, esc_lds, esc_loader, bad);
      __syncthreads();
      uint32_t tagsV[NR][3];
      const int boV = kEscAreas == 1 ? __builtin_amdgcn_readfirstlane(rV.bo()) : rV.bo();
      fetch_tags<NR, FMT>(cV, j, rV.tg, pfxV, tagsV);
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        uint4 bv[2][2];
        if (rV.src() == SRC_COMP) {
          uint32_t o[2][2][4];
          rebuild_round<NR, FMT>(cV, i, j, n, tagsV[i], blds[boV + (NR + i) * 16 + n], esc16, below, bad, o);
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            bv[x][0] = make_uint4(o[x][0][0], o[x][1][0], o[x][0][1], o[x][1][1]);
            bv[x][1] = make_uint4(o[x][0][2], o[x][1][2], o[x][0][3], o[x][1][3]);
          }
        } else if (rV.src() == SRC_RAW) {
#pragma unroll
          for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int ch = 32 * i + 2 * n + x;
              const size_t off = (size_t)ch * TT + rV.tg * 16 + 8 * e;  // elements
              if constexpr (FMT == 0) {  // natural order -> the interleaved order of P
                const uint4 v = mask_tokens(ld128(reinterpret_cast<const uint16_t*>(rV.p) + off), rV.valid() - 8 * e);
                bv[x][e] = make_uint4(perm_b32(v.y, v.x, 0x05040100u), perm_b32(v.y, v.x, 0x07060302u),
                                      perm_b32(v.w, v.z, 0x05040100u), perm_b32(v.w, v.z, 0x07060302u));
              } else {
                bv[x][e] = mask_tokens(fp8x8_to_operand<FMT>(ld64(rV.p + off)), rV.valid() - 8 * e);
              }
            }
        } else {
#pragma unroll
          for (int x = 0; x < 2; ++x) bv[x][0] = bv[x][1] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            acc[i][x] = mfma16(phi[e], bv[x][e], acc[i][x]);
            acc[i][x] = mfma16(plo[e], bv[x][e], acc[i][x]);
          }
      }
    }
  }
  if (bad) flags |= 8u;
  if (flags) atomicOr(&a.B.counters->status, flags);
  write_partial<NR>(a, si, h, split, m, l, acc);
  if (a.k_new != nullptr && split == 0) store_new_token<FMT>(a, si, seq, z.w, h);
}

// ------------------------------------------------------------------------------------------
// Compressed caches with 8-token groups (FORMAT v1, 64-token blocks; GAAC page §3.1 codes the
// exponents of small groups of eight values of one channel): the same split-K structure,
// phase pipelining and rebuild-in-registers as attn_comp_kernel, with a lane layout made for
// 8-token groups.  A CODE unit of an 8-token-group tile is 4 consecutive channels x the 8 tokens
// of one token group (one group per channel), so each lane rebuilds whole units, four tokens per
// 32-bit word:
//   V    : lane n + 16j takes, for each 32-token half h of the block and each 64-channel slice r,
//          the unit of token group 4h + j and channels 64r + 4n .. 64r + 4n + 3.  Its four
//          channels' 8 tokens are PV B operands as rebuilt: MFMA column n of accumulator (r, m)
//          is channel 64r + 4n + m, and k-group j of half h is tokens 32h + 8j .. 32h + 8j + 7.
//   K    : lane n + 16j takes token group 2s + (j >> 1), slice j & 1 (one slice: 4s + j) for its
//          unit s, so the 32 lanes of one LDS store pass cover both halves of a row's banks.
//          Token t = 32h + 8j' + u is stored in LDS row 16j' + 8h + u: the QK A-operand reads
//          (unchanged from attn_comp_kernel) then leave lane n + 16j with the scores of head n for
//          tokens 32h + 8j + u in s[8h + u] -- exactly its P operand for half h.
//   Escapes are bytes: a wide group one 8-bit plane, a raw group one more (E5M2) or four more
//          bytes of 4-bit fields (BF16); tag words and the escape prefix of every word are shared
//          across the wave by lane shuffles, as in attn_comp_kernel.
template <int NH, int FMT>
struct TG8 {
  static constexpr int D = 64 * NH;
  static constexpr int PW = D / 4;   // tag words per plane: 8 token groups x D groups / 32
  static constexpr int US = 2 * NH;  // CODE units a lane holds per tile
  static constexpr int CODE_OFF = (8 * PW + 15) / 16 * 16;
  static constexpr int SM_OFF = CODE_OFF + 24 * D;  // 64 x D codes of 3 bits
  static constexpr int ESC_OFF = SM_OFF + 64 * D * (1 + FmtT<FMT>::MB) / 8;
  static constexpr int SMB = 32 * (1 + FmtT<FMT>::MB) / 8;  // sign/mantissa bytes of one unit
  static constexpr int SMW = SMB / 4;
};

// LDS row of token t of a 64-token block (see above).
__device__ __forceinline__ int g8_krow(int t) { return 16 * ((t >> 3) & 3) + 8 * (t >> 5) + (t & 7); }

// Token group and 64-channel slice of a lane's unit s: K or V assignment (above).
template <int NH, bool ISK>
__device__ __forceinline__ void g8_unit(int s, int j, int& tg, int& r) {
  if constexpr (ISK) {
    if constexpr (NH == 2) { tg = 2 * s + (j >> 1); r = j & 1; }
    else { tg = 4 * s + j; r = 0; }
  } else {
    tg = 4 * (s / NH) + j;
    r = s % NH;
  }
}

// Compressed bytes of one tile held by one lane: tag words `lane` of both planes (lanes < PW),
// escape piece `lane` (lanes below the staged pieces), and the code and sign/mantissa words of
// its units.
template <int NH, int FMT>
struct C8Regs {
  uint32_t tE, tR;
  uint4 esc;
  uint32_t sm[TG8<NH, FMT>::US][TG8<NH, FMT>::SMW];
  uint32_t cd[TG8<NH, FMT>::US][3];
};

template <int NH, int FMT, bool ISK>
__device__ __forceinline__ void g8_load_tile(const TileRef& rf, int lane, C8Regs<NH, FMT>& c) {
  using Q = TG8<NH, FMT>;
  const uint8_t* t = rf.p;  // a raw or dummy tile is large enough for every load below
  const int n = lane & 15, j = lane >> 4;
  c.tE = c.tR = 0;
  if (lane < Q::PW) {
    c.tE = ld32(t + 4 * lane);
    c.tR = ld32(t + 4 * (Q::PW + lane));
  }
  c.esc = make_uint4(0, 0, 0, 0);
  if (lane < rf.escu) c.esc = ld128(t + Q::ESC_OFF + 16 * lane);
#pragma unroll
  for (int s = 0; s < Q::US; ++s) {
    int tg, r;
    g8_unit<NH, ISK>(s, j, tg, r);
    const int u = tg * (Q::D / 4) + 16 * r + n;
    const uint8_t* sp = t + Q::SM_OFF + Q::SMB * u;
    if constexpr (Q::SMW == 8) {
      const uint4 a = ld128(sp), b = ld128(sp + 16);
      c.sm[s][0] = a.x; c.sm[s][1] = a.y; c.sm[s][2] = a.z; c.sm[s][3] = a.w;
      c.sm[s][4] = b.x; c.sm[s][5] = b.y; c.sm[s][6] = b.z; c.sm[s][7] = b.w;
    } else if constexpr (Q::SMW == 4) {
      const uint4 a = ld128(sp);
      c.sm[s][0] = a.x; c.sm[s][1] = a.y; c.sm[s][2] = a.z; c.sm[s][3] = a.w;
    } else {
      c.sm[s][0] = ld32(sp); c.sm[s][1] = ld32(sp + 4); c.sm[s][2] = ld32(sp + 8);
    }
    const uint8_t* cp = t + Q::CODE_OFF + 12 * u;
    c.cd[s][0] = ld32(cp);
    c.cd[s][1] = ld32(cp + 4);
    c.cd[s][2] = ld32(cp + 8);
  }
}

// Stage the tile's escape pieces into LDS; return the escape bytes before tag word `lane`
// (lanes < PW).  A word whose groups would end past the staged bytes (corrupt tags) is flagged
// and cleared, as in stage_escape.
template <int NH, int FMT>
__device__ __forceinline__ uint32_t g8_stage_escape(C8Regs<NH, FMT>& c, const TileRef& rf, int lane, uint8_t* esc_lds,
                                                    uint32_t& bad) {
  if (rf.src() == SRC_COMP && lane < rf.escu) *reinterpret_cast<uint4*>(esc_lds + 16 * lane) = c.esc;
  const uint32_t cnt = __popc(c.tE) + (uint32_t)(FmtT<FMT>::F - 4) * __popc(c.tR);  // wide 1 byte, raw F - 3
  uint32_t incl = row_scan16(cnt);
  if constexpr (TG8<NH, FMT>::PW > 16)
    incl += lane >= 16 ? (uint32_t)__builtin_amdgcn_readlane((int)incl, 15) : 0u;
  if (rf.src() == SRC_COMP && !esc_bytes_fit(incl, (uint32_t)rf.escu)) {
    bad |= 1u;
    c.tE = c.tR = 0u;
    return 0u;
  }
  return incl - cnt;
}

// Codes of slot S (a value the unrolled loops make constant) of a CODE unit.
template <int XS>
__device__ __forceinline__ uint32_t code_slot_of(int S, uint32_t W0, uint32_t W1, uint32_t W2) {
  switch (S) {
    case 0: return code_slot<0, XS>(W0, W1, W2);
    case 1: return code_slot<1, XS>(W0, W1, W2);
    case 2: return code_slot<2, XS>(W0, W1, W2);
    case 3: return code_slot<3, XS>(W0, W1, W2);
    case 4: return code_slot<4, XS>(W0, W1, W2);
    case 5: return code_slot<5, XS>(W0, W1, W2);
    case 6: return code_slot<6, XS>(W0, W1, W2);
    default: return code_slot<7, XS>(W0, W1, W2);
  }
}
__device__ __forceinline__ uint32_t e5m2_sign_mant_of(int S, uint32_t W0, uint32_t W1, uint32_t W2) {
  switch (S) {
    case 0: return e5m2_sign_mant<0>(W0, W1, W2);
    case 1: return e5m2_sign_mant<1>(W0, W1, W2);
    case 2: return e5m2_sign_mant<2>(W0, W1, W2);
    case 3: return e5m2_sign_mant<3>(W0, W1, W2);
    case 4: return e5m2_sign_mant<4>(W0, W1, W2);
    case 5: return e5m2_sign_mant<5>(W0, W1, W2);
    case 6: return e5m2_sign_mant<6>(W0, W1, W2);
    default: return e5m2_sign_mant<7>(W0, W1, W2);
  }
}

// Unit s of lane n as one word: bits 0..3 its groups' E bits, 4..7 their R bits, 8.. the escape
// bytes before its first group, from the tag words and escape prefix of the lane holding its tag
// word (cross-lane reads).  A raw group without an E bit is flagged (bad).
template <int NH, int FMT, bool ISK>
__device__ __forceinline__ uint32_t g8_unit_tags(const C8Regs<NH, FMT>& c, int s, int j, int n, uint32_t pfx,
                                                 uint32_t& bad) {
  constexpr int RU = FmtT<FMT>::F - 3;  // escape bytes of a raw group
  int tg, r;
  g8_unit<NH, ISK>(s, j, tg, r);
  const int w = tg * (TG8<NH, FMT>::D / 32) + 2 * r + (n >> 3);  // unit tg * D/4 + 16r + n, 8 units a word
  const uint32_t Ew = (uint32_t)__shfl((int)c.tE, w), Rw = (uint32_t)__shfl((int)c.tR, w), Pw = (uint32_t)__shfl((int)pfx, w);
  const int bit = 4 * (n & 7);
  const uint32_t e4 = __builtin_amdgcn_ubfe(Ew, bit, 4), r4 = __builtin_amdgcn_ubfe(Rw, bit, 4);
  bad |= r4 & ~e4;
  if constexpr (FMT == 2) bad |= e4 & ~r4;  // no wide mode in a 4-bit exponent field
  return e4 | (r4 << 4) | (g8_unit_escape(Ew, Rw, Pw, n & 7, RU) << 8);
}

// Element words of quad qq of group gi of unit s from its rebuilt exponents Ev (four byte lanes) and
// its stored sign/mantissa fields (layout of g8_rebuild_unit's output).
template <int NH, int FMT>
__device__ __forceinline__ void g8_assemble(const C8Regs<NH, FMT>& c, int s, int gi, int qq, uint32_t Ev,
                                            uint32_t o[4][2][2]) {
  const int slot = 2 * gi + qq;
  if constexpr (FMT == 0) {
    const uint32_t sv = c.sm[s][slot];
    o[gi][0][qq] = bitsel(0x7F807F80u, Ev << 7, perm_b32(sv, sv, 0x02020000u));
    o[gi][1][qq] = bitsel(0x7F807F80u, Ev >> 1, perm_b32(sv, sv, 0x03030101u));
  } else {
    uint32_t g;  // sign at bit 7, mantissa at bits 0..MB-1 of each byte lane
    if constexpr (FMT == 1) {
      g = e5m2_sign_mant_of(slot, c.sm[s][0], c.sm[s][1], c.sm[s][2]);
    } else {
      const uint32_t sw = c.sm[s][gi];
      g = e4m3_sign_mant(perm_b32(sw, sw, qq ? 0x03030202u : 0x01010000u));
    }
    const uint32_t B = bfi(FmtT<FMT>::XMASK, Ev, g);  // the four FP8 bytes
    o[gi][0][qq] = fp8x2_to_bf16x2<FMT, false>(B);
    o[gi][1][qq] = fp8x2_to_bf16x2<FMT, true>(B);
  }
}

// Rebuild unit s of lane n: channels gi = 0..3 x 8 tokens.  ut = the unit's tags and escape
// offset (g8_unit_tags); bw = b3 (x) and b4 (y) of the four
// channels, one byte each (FP8: pre-shifted to the exponent position).  Output, low half first:
// BF16 o[gi][0][qq] = tokens (4qq, 4qq+2), o[gi][1][qq] = (4qq+1, 4qq+3); FP8 (converted exactly
// to BF16) o[gi][0][qq] = (4qq, 4qq+1), o[gi][1][qq] = (4qq+2, 4qq+3).
template <int NH, int FMT>
__device__ __forceinline__ void g8_rebuild_unit(const C8Regs<NH, FMT>& c, int s, uint32_t ut, uint2 bw,
                                                const uint8_t* esc8, uint32_t o[4][2][2]) {
  constexpr int RU = FmtT<FMT>::F - 3;  // escape bytes of a raw group
  constexpr int XS = FmtT<FMT>::XS;
  const uint32_t e4 = ut & 0xFu, r4 = (ut >> 4) & 0xFu;
  uint32_t P = ut >> 8;
  const uint32_t W0 = c.cd[s][0], W1 = c.cd[s][1], W2 = c.cd[s][2];
  // byte g of Hw: the base of group g's mode, b4 where the group escapes (wide or raw), else b3;
  // a raw group's base is 0, which its rare path below restores by taking b4 back off
  const uint32_t e1 = spread4(e4);        // bit 0 of byte g = group g escapes
  const uint32_t mE = (e1 << 8) - e1;     // x 255 (exact mod 2^32): byte g all ones where it escapes
  const uint32_t Hw = (bw.y & mE) | (bw.x & ~mE);  // per-lane mask: not bfi(), which takes a uniform one
  // Every LDS read of the unit first (escape planes, then their spread words), so that they are in
  // flight together; the rare raw groups afterwards, behind one branch for the unit.
  uint32_t Pg[4], Ev[4][2];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    Pg[gi] = P;
    P += ((e4 >> gi) & 1u) + (uint32_t)(RU - 1) * ((r4 >> gi) & 1u);
  }
  uint32_t plane[4];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) plane[gi] = esc8[Pg[gi]] & (0u - ((e4 >> gi) & 1u));  // read always, keep if escaped
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    const uint32_t H = perm_b32(0u, Hw, (uint32_t)gi * 0x01010101u);  // the group's base in all four bytes
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
      Ev[gi][qq] = H + code_slot_of<XS>(2 * gi + qq, W0, W1, W2) + esc_lut[(plane[gi] >> (4 * qq)) & 0xFu];
  }
  if (r4) {  // a raw group (rare): base 0 (b4 taken back off) and the offset bits above bit 3
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      if ((r4 >> gi) & 1u) {
        const uint32_t H = perm_b32(0u, Hw, (uint32_t)gi * 0x01010101u);
        Ev[gi][0] -= H;
        Ev[gi][1] -= H;
        if constexpr (FMT == 0) {  // four bytes of 4-bit fields at P + 1 (any alignment): two aligned words
          const uint32_t a0 = Pg[gi] + 1u;
          const uint32_t* e32 = reinterpret_cast<const uint32_t*>(esc8);
          const uint32_t hi = __builtin_amdgcn_alignbyte(e32[(a0 >> 2) + 1], e32[a0 >> 2], a0 & 3u);
          Ev[gi][0] += raw_high_nibbles(hi & 0xFFFFu);
          Ev[gi][1] += raw_high_nibbles(hi >> 16);
        } else if constexpr (FMT == 1) {  // the bit-4 plane
          const uint32_t u = esc8[Pg[gi] + 1];
          Ev[gi][0] += esc_lut[u & 0xFu] << 1;
          Ev[gi][1] += esc_lut[(u >> 4) & 0xFu] << 1;
        }
      }
    }
  }
#pragma unroll
  for (int gi = 0; gi < 4; ++gi)
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) g8_assemble<NH, FMT>(c, s, gi, qq, Ev[gi][qq], o);
}

// b3 (even k) or b4 (odd k) of the four channels 64r + 4nn .. +3 of base version ver, for packed
// slot k = ((kv * NH + r) * 16 + nn) * 2 + which.
template <int NH, int FMT>
__device__ __forceinline__ uint32_t g8_packed_bases(const Geo& G, const uint8_t* bases, int ver, int k, int h) {
  const int kv = k / (32 * NH), r = (k / 32) % NH, nn = (k / 2) % 16, which = k & 1;
  return ld32(bases_of(G, bases, ver, 3 + which, kv, h) + 64 * r + 4 * nn) << FmtT<FMT>::XS;
}

// Scale accumulators of heads 4j .. 4j+3 (row r of lane 16j + n) by their heads' factors.
template <int N>
__device__ __forceinline__ void rescale_rows(f32x4_t (&acc)[N], float alpha) {
  uint32_t base;
  asm volatile("v_and_b32 %0, 48, %1" : "=v"(base) : "v"((uint32_t)threadIdx.x));
  float a[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    a[r] = __int_as_float(__builtin_amdgcn_ds_bpermute((int)(base + 4 * r), __float_as_int(alpha)));
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[i][r] *= a[r];
}

template <int NH, int FMT>
__global__ void __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_g8_kernel(AttnArgs a) {
  using Q = TG8<NH, FMT>;
  constexpr int NR = 2 * NH;  // 32-channel rounds (tile_ref geometry)
  constexpr bool NAT = FmtT<FMT>::NATURAL;
  constexpr int D = Q::D;
  extern __shared__ uint4 lds4[];
  const Geo& G = a.G;
  const int esc_room = (max(G.esc_cap, 16) + 15) / 16 * 16;
  uint8_t* klds = reinterpret_cast<uint8_t*>(lds4);                         // [64][D] bf16, swizzled
  uint8_t* esc_lds = klds + kSB * D * 2;                                      // esc_room + 16 bytes
  uint4* qlds = reinterpret_cast<uint4*>(esc_lds + esc_room + 16);            // [g][D/8]
  uint32_t* blds = reinterpret_cast<uint32_t*>(qlds + G.g * (D / 8));         // [version][K|V][NH][16][2]
  const int lane = threadIdx.x, n = lane & 15, j = lane >> 4;
  const int split = blockIdx.x, h = blockIdx.y;
  const int4 z = a.zrow[blockIdx.z];
  const int si = z.x, seq = z.y, L = z.z;
  const SbOrder ord(L, a.n_splits, split);
  uint32_t flags = 0, bad = 0;
  init_esc_lut<FMT>();

  uint32_t eK = kUnallocated, eV = kUnallocated;
  if (ord.cnt > 0) {
    eK = load_entry<kSB>(a, seq, L, ord.at(0) * kSB, 0, h);
    eV = load_entry<kSB>(a, seq, L, ord.at(0) * kSB, 1, h);
  }
  uint4 qr[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int k = lane + kWave * u;
    qr[u] = k < G.g * (D / 8) ? ld128(a.q + ((size_t)si * G.Hq + h * G.g) * D + 8 * k) : make_uint4(0, 0, 0, 0);
  }
  constexpr int BU = 64 * NH / kWave;  // packed base words per lane and version
  uint32_t br[BU];
#pragma unroll
  for (int u = 0; u < BU; ++u) br[u] = g8_packed_bases<NH, FMT>(G, a.B.bases, 0, lane + kWave * u, h);

  float m = -INFINITY, l = 0.0f;
  f32x4_t acc[NH * 4];  // accumulator r * 4 + gi: MFMA column n = channel 64r + 4n + gi
#pragma unroll
  for (int i = 0; i < NH * 4; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  C8Regs<NH, FMT> cK, cV;
  TileRef rK, rV;
  if (ord.cnt > 0) {
    rK = tile_ref<NR, kSB, FMT>(a, seq, L, ord.at(0) * kSB, 0, h, eK);
    flags |= missing_flag(L, ord.at(0) * kSB, eK);
    g8_load_tile<NH, FMT, true>(rK, lane, cK);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (lane + kWave * u < G.g * (D / 8)) qlds[lane + kWave * u] = qr[u];
#pragma unroll
  for (int u = 0; u < BU; ++u) blds[lane + kWave * u] = br[u];
  for (int v = 1; v < G.n_versions; ++v)
#pragma unroll
    for (int u = 0; u < BU; ++u) blds[v * 64 * NH + lane + kWave * u] = g8_packed_bases<NH, FMT>(G, a.B.bases, v, lane + kWave * u, h);

  for (int it = 0; it < ord.cnt; ++it) {
    phase_priority(2 * (ord.cnt - it));
    const int sb = ord.at(it);
    rV = tile_ref<NR, kSB, FMT>(a, seq, L, sb * kSB, 1, h, eV);
    flags |= missing_flag(L, sb * kSB, eV);
    g8_load_tile<NH, FMT, false>(rV, lane, cV);
    if (it + 1 < ord.cnt) {
      eK = load_entry<kSB>(a, seq, L, ord.at(it + 1) * kSB, 0, h);
      eV = load_entry<kSB>(a, seq, L, ord.at(it + 1) * kSB, 1, h);
    }

    // ---- K: rebuild into the LDS tile ----
    __syncthreads();
    const uint32_t pfxK = g8_stage_escape<NH, FMT>(cK, rK, lane, esc_lds, bad);
    __syncthreads();
    const int kind = __builtin_amdgcn_readfirstlane(rK.kind);
    if ((kind & 3) == SRC_COMP) {
      const int boK = kind >> 2;
      uint32_t ut[Q::US];  // every unit's tags first: their cross-lane reads are in flight together
#pragma unroll
      for (int s = 0; s < Q::US; ++s) ut[s] = g8_unit_tags<NH, FMT, true>(cK, s, j, n, pfxK, bad);
#pragma unroll
      for (int s = 0; s < Q::US; ++s) {
        int tg, r;
        g8_unit<NH, true>(s, j, tg, r);
        const uint2 bw = *reinterpret_cast<const uint2*>(blds + boK + ((0 * NH + r) * 16 + n) * 2);
        uint32_t o[4][2][2];
        g8_rebuild_unit<NH, FMT>(cK, s, ut[s], bw, esc_lds, o);
        // token 8tg + 4qq + k: channels 64r + 4n .. +3 as one 8-byte store (BF16: word k & 1,
        // half k >> 1; FP8: word k >> 1, half k & 1)
        const int chunk = 8 * r + (n >> 1), off = 8 * (n & 1);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int row = 16 * (tg & 3) + 8 * (tg >> 2) + 4 * qq + k;
            const int wi = NAT ? (k >> 1) : (k & 1);
            const uint32_t sel = (NAT ? (k & 1) : (k >> 1)) ? 0x07060302u : 0x05040100u;
            const uint32_t w01 = perm_b32(o[1][wi][qq], o[0][wi][qq], sel);
            const uint32_t w23 = perm_b32(o[3][wi][qq], o[2][wi][qq], sel);
            *reinterpret_cast<uint2*>(klds + row * 2 * D + ((chunk ^ swz(row)) << 4) + off) = make_uint2(w01, w23);
          }
      }
    } else if ((kind & 3) == SRC_RAW) {
      // a raw tile: token rows straight into their LDS rows (BF16 by LDS-DMA, FP8 through
      // registers, converted to BF16)
      const uint64_t rp = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)((uintptr_t)rK.p >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)rK.p);
      if constexpr (FMT == 0) {
        constexpr int RPI = 512 / D;  // rows per instruction
        constexpr int LPR = D / 8;    // lanes (16-byte pieces) per row
        const uint16_t* raw = reinterpret_cast<const uint16_t*>(rp);
#pragma unroll 1
        for (int i = 0; i < kSB / RPI; ++i) {
          const int row = RPI * i + lane / LPR, pos = lane % LPR;
          const int tok = 32 * ((row & 15) >> 3) + 8 * (row >> 4) + (row & 7);  // the token of LDS row `row`
          __builtin_amdgcn_global_load_lds(raw + (size_t)tok * D + 8 * (pos ^ swz(row)),
                                           (__attribute__((address_space(3))) void*)(klds + RPI * i * 2 * D), 16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the DMA has landed in LDS
      } else {
        const uint8_t* raw = reinterpret_cast<const uint8_t*>(rp);
        constexpr int NCH = D / 8;  // 8-element pieces per row; lane group j fills LDS rows 16j .. 16j+15
#pragma unroll
        for (int m0 = 0; m0 < NCH; m0 += 4) {
          uint2 v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int k = n + 16 * (m0 + u), row = 16 * j + k / NCH, chunk = k % NCH;
            const int tok = 32 * ((row & 15) >> 3) + 8 * (row >> 4) + (row & 7);
            v[u] = ld64(raw + (size_t)tok * D + 8 * chunk);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int k = n + 16 * (m0 + u), row = 16 * j + k / NCH, chunk = k % NCH;
            *reinterpret_cast<uint4*>(klds + row * 2 * D + ((chunk ^ swz(row)) << 4)) = fp8x8_to_operand<FMT>(v[u]);
          }
        }
      }
    }
    __syncthreads();

    // ---- QK and softmax: s[8h + u] = head n, token 32h + 8j + u ----
    const int valid = min(rK.valid(), rV.valid());
    f32x4_t cc[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) cc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NR; ++ks) {
      uint4 qv = qlds[min(n, G.g - 1) * (D / 8) + 4 * ks + j];
      if (n >= G.g) qv = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int row = 16 * (n >> 2) + 4 * rb + (n & 3);
        const uint4 av = *reinterpret_cast<const uint4*>(klds + row * 2 * D + (((4 * ks + j) ^ swz(row)) << 4));
        cc[rb] = mfma16(av, qv, cc[rb]);
      }
    }
    float s[16];
    if (__builtin_amdgcn_ballot_w64(valid == 0)) {  // a block missing from the table (status bit 4)
#pragma unroll
      for (int k = 0; k < 16; ++k) s[k] = -INFINITY;
    } else {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[4 * rb + r] = cc[rb][r] * a.sl2;
    }
    const float alpha = softmax_update(s, m, l);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) rescale_rows<NH * 4>(acc, alpha);
    uint4 phi[2], plo[2];
    pack_p<!NAT>(s, phi, plo);

    if (it + 1 < ord.cnt) {
      rK = tile_ref<NR, kSB, FMT>(a, seq, L, ord.at(it + 1) * kSB, 0, h, eK);
      flags |= missing_flag(L, ord.at(it + 1) * kSB, eK);
      g8_load_tile<NH, FMT, true>(rK, lane, cK);
    }

    phase_priority(2 * (ord.cnt - it) - 1);
    // ---- V: rebuild straight into B operands ----
    __syncthreads();
    const uint32_t pfxV = g8_stage_escape<NH, FMT>(cV, rV, lane, esc_lds, bad);
    __syncthreads();
    const int kindV = __builtin_amdgcn_readfirstlane(rV.kind);
    const int boV = kindV >> 2;
    uint32_t utV[Q::US];
    if ((kindV & 3) == SRC_COMP) {
#pragma unroll
      for (int s = 0; s < Q::US; ++s) utV[s] = g8_unit_tags<NH, FMT, false>(cV, s, j, n, pfxV, bad);
    }
#pragma unroll
    for (int s = 0; s < Q::US; ++s) {
      int tg, r;
      g8_unit<NH, false>(s, j, tg, r);
      const int hh = s / NH;  // the 32-token half
      uint4 bv[4];
      if ((kindV & 3) == SRC_COMP) {
        const uint2 bw = *reinterpret_cast<const uint2*>(blds + boV + ((NH + r) * 16 + n) * 2);
        uint32_t o[4][2][2];
        g8_rebuild_unit<NH, FMT>(cV, s, utV[s], bw, esc_lds, o);
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) bv[gi] = make_uint4(o[gi][0][0], o[gi][1][0], o[gi][0][1], o[gi][1][1]);
      } else if ((kindV & 3) == SRC_RAW) {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const size_t off = (size_t)(64 * r + 4 * n + gi) * kSB + 32 * hh + 8 * j;  // elements
          if constexpr (FMT == 0) {  // natural order -> the interleaved order of P
            const uint4 v = ld128(reinterpret_cast<const uint16_t*>(rV.p) + off);
            bv[gi] = make_uint4(perm_b32(v.y, v.x, 0x05040100u), perm_b32(v.y, v.x, 0x07060302u),
                                perm_b32(v.w, v.z, 0x05040100u), perm_b32(v.w, v.z, 0x07060302u));
          } else {
            bv[gi] = fp8x8_to_operand<FMT>(ld64(rV.p + off));
          }
        }
      } else {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) bv[gi] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        acc[4 * r + gi] = mfma16(phi[hh], bv[gi], acc[4 * r + gi]);
        acc[4 * r + gi] = mfma16(plo[hh], bv[gi], acc[4 * r + gi]);
      }
    }
  }
  if (bad) flags |= 8u;
  if (flags) atomicOr(&a.B.counters->status, flags);
  // partials: head 4j + i, channels 64r + 4n .. +3 from accumulators 4r .. 4r+3
  {
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    const int S = a.n_splits;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = 4 * j + i;
      if (head < G.g) {
        float* dst = a.ws_acc + (((size_t)si * G.Hq + h * G.g + head) * S + split) * D;
#pragma unroll
        for (int r = 0; r < NH; ++r)
          *reinterpret_cast<float4*>(dst + 64 * r + 4 * n) =
              make_float4(acc[4 * r][i], acc[4 * r + 1][i], acc[4 * r + 2][i], acc[4 * r + 3][i]);
      }
    }
    if (j == 0 && n < G.g) {
      float* ml = a.ws_ml + (((size_t)si * G.Hq + h * G.g + n) * S + split) * 2;
      ml[0] = m;
      ml[1] = lt;
    }
  }
  if (a.k_new != nullptr && split == 0) store_new_token<FMT>(a, si, seq, z.w, h);
}

// ------------------------------------------------------------------------------------------
// Uncompressed cache (every tile raw): the speedup baseline.  K rows are loaded straight into
// QK A operands and V straight into PV B operands (no LDS), with the same K/V phase pipelining.
// Operand pieces as loaded: eight BF16 (uint4) or eight FP8 (uint2, converted at use).
template <int FMT>
using Piece = typename std::conditional<FMT == 0, uint4, uint2>::type;

template <int FMT>
__device__ __forceinline__ Piece<FMT> ld_piece(const uint8_t* base, size_t elem) {
  if constexpr (FMT == 0) return ld128(reinterpret_cast<const uint16_t*>(base) + elem);
  else return ld64(base + elem);
}
template <int FMT>
__device__ __forceinline__ uint4 operand(const Piece<FMT>& v) {
  if constexpr (FMT == 0) return v;
  else return fp8x8_to_operand<FMT>(v);
}

template <int NR, int FMT>
struct RawK {
  Piece<FMT> ka[4][NR];
};
template <int NR, int FMT>
struct RawV {
  Piece<FMT> vb[NR][2][2];
};

template <int NR, int TT, int FMT>
__device__ __forceinline__ void raw_load_k(const TileRef& r, int n, int j, RawK<NR, FMT>& k) {
  constexpr int D = 32 * NR;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int rr = 4 * rb + (n & 3);
#pragma unroll
    for (int ks = 0; ks < NR; ++ks) k.ka[rb][ks] = ld_piece<FMT>(r.p, (size_t)(r.tg * 16 + rr) * D + 32 * ks + 8 * j);
  }
}

template <int NR, int TT, int FMT>
__device__ __forceinline__ void raw_load_v(const TileRef& r, int n, RawV<NR, FMT>& v) {
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        v.vb[i][x][e] = ld_piece<FMT>(r.p, (size_t)(32 * i + 2 * n + x) * TT + r.tg * 16 + 8 * e);
}

template <int NR, int TT, int FMT>
__global__ void __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_raw_kernel(AttnArgs a) {
  constexpr int D = 32 * NR;
  const Geo& G = a.G;
  const int lane = threadIdx.x, n = lane & 15, j = lane >> 4;
  const int split = blockIdx.x, h = blockIdx.y;
  const int4 z = a.zrow[blockIdx.z];
  const int si = z.x, seq = z.y, L = z.z;
  const SbOrder ord(L, a.n_splits, split);
  uint32_t flags = 0;

  uint4 qb[NR];
#pragma unroll
  for (int ks = 0; ks < NR; ++ks)
    qb[ks] = (n < G.g) ? ld128(a.q + ((size_t)si * G.Hq + h * G.g + n) * D + 32 * ks + 8 * j) : make_uint4(0, 0, 0, 0);

  float m = -INFINITY, l = 0.0f;
  f32x4_t acc[NR][2];
#pragma unroll
  for (int i = 0; i < NR; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (ord.cnt > 0) {
    RawK<NR, FMT> ck;
    RawV<NR, FMT> cv;
    const int jr = n >> 2;  // token group of this lane's QK A-operand rows
    uint32_t eK = load_entry<TT>(a, seq, L, group_token(ord.at(0), jr), 0, h);
    uint32_t eV = load_entry<TT>(a, seq, L, group_token(ord.at(0), j), 1, h);
    TileRef rK = tile_ref<NR, TT, FMT>(a, seq, L, group_token(ord.at(0), jr), 0, h, eK);
    flags |= missing_flag(L, group_token(ord.at(0), jr), eK);
    raw_load_k<NR, TT, FMT>(rK, n, j, ck);
    for (int it = 0; it < ord.cnt; ++it) {
      phase_priority(2 * (ord.cnt - it));
      const int sb = ord.at(it);
      const TileRef rV = tile_ref<NR, TT, FMT>(a, seq, L, group_token(sb, j), 1, h, eV);
      flags |= missing_flag(L, group_token(sb, j), eV);
      raw_load_v<NR, TT, FMT>(rV, n, cv);
      if (it + 1 < ord.cnt) {
        eK = load_entry<TT>(a, seq, L, group_token(ord.at(it + 1), jr), 0, h);
        eV = load_entry<TT>(a, seq, L, group_token(ord.at(it + 1), j), 1, h);
      }
      // scores of this lane belong to token group j: its K validity comes from lane 4j
      const int validKj = __shfl(rK.valid(), 4 * j);
      const int valid = min(validKj, rV.valid());
      float s[16];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        f32x4_t cc = {0.f, 0.f, 0.f, 0.f};
        const bool rowok = 4 * rb + (n & 3) < rK.valid();
#pragma unroll
        for (int ks = 0; ks < NR; ++ks)
          cc = mfma16(rowok ? operand<FMT>(ck.ka[rb][ks]) : make_uint4(0, 0, 0, 0), qb[ks], cc);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[4 * rb + r] = (4 * rb + r < valid) ? cc[r] * a.sl2 : -INFINITY;
      }
      const float alpha = softmax_update(s, m, l);
      rescale_acc<NR>(acc, alpha, j);
      uint4 phi[2], plo[2];
      pack_p<false>(s, phi, plo);
      if (it + 1 < ord.cnt) {
        rK = tile_ref<NR, TT, FMT>(a, seq, L, group_token(ord.at(it + 1), jr), 0, h, eK);
        flags |= missing_flag(L, group_token(ord.at(it + 1), jr), eK);
        raw_load_k<NR, TT, FMT>(rK, n, j, ck);
      }
      phase_priority(2 * (ord.cnt - it) - 1);
#pragma unroll
      for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint4 v = mask_tokens(operand<FMT>(cv.vb[i][x][e]), rV.valid() - 8 * e);
            acc[i][x] = mfma16(phi[e], v, acc[i][x]);
            acc[i][x] = mfma16(plo[e], v, acc[i][x]);
          }
    }
  }
  if (flags) atomicOr(&a.B.counters->status, flags);
  write_partial<NR>(a, si, h, split, m, l, acc);
  if (a.k_new != nullptr && split == 0) store_new_token<FMT>(a, si, seq, z.w, h);
}

// Log-sum-exp merge of the splits, with the tail.  The split kernels cover the finished blocks;
// the unfinished block (the tail, fewer than T tokens, stored raw) is attended here as one more
// term of the same normalisation, so no split carries a partial block.  One 256-thread block per
// (CH-channel slice, query head, sequence): CH = 16 when there are many splits to read (the
// reads spread over D/16 blocks per head), CH = D when there are few (one block per head, so the
// tail is scored once per head).
//   * Every load is issued first, unconditionally (indices clamped into their buffers, unused
//     values masked afterwards by selects) -- the splits' (max, sum) pairs, this slice's partial
//     outputs, the tail's K rows and the query, the tail's V values for the slice -- so the block
//     waits on one memory round trip.
//   * Tail scores: thread (token tid/4, channel quarter tid%4) takes a 4-lane dot product, in
//     fp32, of the BF16 query with the token's K row, pre-multiplied by scale*log2(e).
//   * M = the largest of the split maxima (splits that saw a token) and the tail scores; the
//     weights exp2(m_s - M), exp2(s_t - M) go to LDS; den = sum_s w_s l_s + sum_t w_t.
//   * out = (sum_s w_s acc_s + sum_t w_t v_t) / den, rounded to BF16.
// In a decode step the newest token is already in the tail: the split kernel that ran before
// this one stored it there (store_new_token).
constexpr int kCombineThreads = 256;
constexpr int kMaxSplits = 1024;
constexpr int kTailTok = 64;        // tail tokens a block can hold (T <= 64)

struct CombineArgs {
  Geo G;
  SeqList S;
  const uint8_t* tail;
  const uint16_t* q;
  const float* ws_acc;
  const float* ws_ml;
  uint16_t* out;
  float sl2;
  int n_splits;
};

// Cross-lane moves inside a 16-lane row by DPP, without an LDS round trip: xor 1 and xor 2 as
// quad permutations, the half-row and row mirrors (lane i with 7 - i and with 15 - i) and row
// rotations by 4 and 8.  Once every lane of a quad holds the quad's total, the half-row mirror
// pairs whole quads and the row mirror whole half-rows, so four steps reduce a row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kDppRor4 = 0x124, kDppRor8 = 0x128;

// every lane of each aligned group of N lanes (N a power of two <= 16) gets the group's sum
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N >= 1 && N <= 16 && (N & (N - 1)) == 0, "group of 1 to 16 lanes");
  if constexpr (N >= 2) v += dpp<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  // the wave: each row by DPP, then the four rows' results (read as scalars)
  v = is_max ? fmaxf(v, dpp<kDppXor1>(v)) : v + dpp<kDppXor1>(v);
  v = is_max ? fmaxf(v, dpp<kDppXor2>(v)) : v + dpp<kDppXor2>(v);
  v = is_max ? fmaxf(v, dpp<kDppHalfMirror>(v)) : v + dpp<kDppHalfMirror>(v);
  v = is_max ? fmaxf(v, dpp<kDppMirror>(v)) : v + dpp<kDppMirror>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  v = is_max ? fmaxf(fmaxf(r0, r1), fmaxf(r2, r3)) : (r0 + r1) + (r2 + r3);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kCombineThreads / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight consecutive tail elements as four BF16 pairs (BF16: 16 bytes; FP8: 8 bytes, converted).
template <int FMT>
__device__ __forceinline__ uint4 tail_oct(const uint8_t* p) {
  if constexpr (FMT == 0) return *reinterpret_cast<const uint4*>(p);
  else return fp8x8_to_operand<FMT>(*reinterpret_cast<const uint2*>(p));
}
// Four consecutive tail elements as two BF16 pairs.
template <int FMT>
__device__ __forceinline__ uint2 tail_quad(const uint8_t* p) {
  if constexpr (FMT == 0) return *reinterpret_cast<const uint2*>(p);
  else {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(p);
    return make_uint2(fp8x2_to_bf16x2<FMT, false>(x), fp8x2_to_bf16x2<FMT, true>(x));
  }
}

__device__ __forceinline__ float dot8(uint4 k, uint4 q) {
  float d = bf16_lo(k.x) * bf16_lo(q.x) + bf16_hi(k.x) * bf16_hi(q.x);
  d += bf16_lo(k.y) * bf16_lo(q.y) + bf16_hi(k.y) * bf16_hi(q.y);
  d += bf16_lo(k.z) * bf16_lo(q.z) + bf16_hi(k.z) * bf16_hi(q.z);
  d += bf16_lo(k.w) * bf16_lo(q.w) + bf16_hi(k.w) * bf16_hi(q.w);
  return d;
}

// NR: head_dim / 32; CH: channels per block; UPT: partial outputs per thread (the launch picks
// UPT * 1024 / CH >= n_splits).
template <int NR, int FMT, int CH, int UPT>
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(CombineArgs a) {
  constexpr int D = 32 * NR, EB = FmtT<FMT>::EB;
  constexpr int NQ = CH / 4;                      // channel quads per block
  constexpr int NSL = kCombineThreads / NQ;       // split slices
  constexpr int MLPT = (UPT * NSL + kCombineThreads - 1) / kCombineThreads;  // (max, sum) pairs per thread
  constexpr int KPL = D / 4;                      // tail K channels per lane (4 lanes per token)
  constexpr int TPC = kCombineThreads / CH;       // tail V: threads per channel
  constexpr int QPT = (kTailTok / 4) / TPC;       // tail V: token quads per thread
  static_assert(NQ <= 32 && TPC <= 16 && QPT >= 1, "combine geometry");
  __shared__ float w[UPT * NSL];
  __shared__ float pt[kTailTok];
  __shared__ float red[kCombineThreads / 64];
  __shared__ float part[kCombineThreads / 64 * CH];
  __shared__ float tsum[CH];
  const Geo& G = a.G;
  const int cb = blockIdx.x, hq = blockIdx.y, si = blockIdx.z, tid = threadIdx.x;
  const int S = a.n_splits, T = G.T;
  const int seq = a.S.ids[si], L = a.S.lens[si], ntail = L % T, h = hq / G.g;
  const float* ml = a.ws_ml + ((size_t)si * G.Hq + hq) * S * 2;
  const float* acc = a.ws_acc + ((size_t)si * G.Hq + hq) * S * D + cb * CH;
  const int quad = tid % NQ, slice = tid / NQ;    // partial outputs: channels 4*quad.., splits slice + NSL*u
  const int tk = tid >> 2, kq4 = tid & 3;         // tail K: token tk, channels KPL*kq4 ..
  const int cv = tid / TPC, tq0 = (tid % TPC) * QPT;  // tail V: channel cb*CH + cv, token quads tq0 ..

  // ---- loads ----
  float2 mv[MLPT];
#pragma unroll
  for (int u = 0; u < MLPT; ++u)
    mv[u] = *reinterpret_cast<const float2*>(ml + 2 * min(tid + kCombineThreads * u, S - 1));
  float4 av[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u)
    av[u] = *reinterpret_cast<const float4*>(acc + (size_t)min(slice + NSL * u, S - 1) * D + 4 * quad);
  const uint8_t* tk_base = a.tail + tail_offset(G, seq, 0, h) * EB;  // K tail [t][c]
  const uint8_t* tv_base = a.tail + tail_offset(G, seq, 1, h) * EB;  // V tail [c][t]
  const uint16_t* qrow = a.q + ((size_t)si * G.Hq + hq) * D + KPL * kq4;
  const int tkc = min(tk, T - 1);
  const uint8_t* krow = tk_base + (size_t)tkc * D * EB;
  uint4 kk[KPL / 8], qq[KPL / 8];
#pragma unroll
  for (int p = 0; p < KPL / 8; ++p) {
    kk[p] = tail_oct<FMT>(krow + (KPL * kq4 + 8 * p) * EB);
    qq[p] = *reinterpret_cast<const uint4*>(qrow + 8 * p);
  }
  uint2 vv[QPT];
#pragma unroll
  for (int u = 0; u < QPT; ++u)
    vv[u] = tail_quad<FMT>(tv_base + ((size_t)(cb * CH + cv) * T + min(4 * (tq0 + u), T - 4)) * EB);

  // ---- maximum ----
  float dot = 0.0f;
#pragma unroll
  for (int p = 0; p < KPL / 8; ++p) dot += dot8(kk[p], qq[p]);
  dot = group_sum<4>(dot);
  const bool kok = tk < ntail;
  const float st = kok ? dot * a.sl2 : -INFINITY;
  float mx = st;
#pragma unroll
  for (int u = 0; u < MLPT; ++u)
    if (tid + kCombineThreads * u < S && mv[u].y > 0.0f) mx = fmaxf(mx, mv[u].x);
  const float M = block_reduce(mx, red, true);

  // ---- weights and denominator ----
  float den = 0.0f;
#pragma unroll
  for (int u = 0; u < MLPT; ++u) {
    const int s = tid + kCombineThreads * u;
    const bool ok = s < S && mv[u].y > 0.0f;
    const float ws = ok ? exp2f(mv[u].x - M) : 0.0f;
    if (s < UPT * NSL) w[s] = ws;
    den += ok ? ws * mv[u].y : 0.0f;
  }
  if (kq4 == 0) {
    const float p = kok ? exp2f(st - M) : 0.0f;
    pt[tk] = p;
    den += p;
  }
  den = block_reduce(den, red, false);  // its barriers also publish w[] and pt[]

  // ---- weighted sums ----
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int s = slice + NSL * u;
    const float ws = s < S ? w[s] : 0.0f;
    sum.x += s < S ? ws * av[u].x : 0.0f;
    sum.y += s < S ? ws * av[u].y : 0.0f;
    sum.z += s < S ? ws * av[u].z : 0.0f;
    sum.w += s < S ? ws * av[u].w : 0.0f;
  }
  int o0 = NQ;  // add the slices of this wave
  if constexpr (NQ == 4) {  // the four lanes of a row with this lane's quad: two rotations
    sum.x += dpp<kDppRor4>(sum.x); sum.y += dpp<kDppRor4>(sum.y);
    sum.z += dpp<kDppRor4>(sum.z); sum.w += dpp<kDppRor4>(sum.w);
    sum.x += dpp<kDppRor8>(sum.x); sum.y += dpp<kDppRor8>(sum.y);
    sum.z += dpp<kDppRor8>(sum.z); sum.w += dpp<kDppRor8>(sum.w);
    o0 = 16;
  }
  for (int o = o0; o < 64; o <<= 1) {
    sum.x += __shfl_xor(sum.x, o);
    sum.y += __shfl_xor(sum.y, o);
    sum.z += __shfl_xor(sum.z, o);
    sum.w += __shfl_xor(sum.w, o);
  }
  float tv = 0.0f;
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int t0 = 4 * (tq0 + u);
    const float v4[4] = {bf16_lo(vv[u].x), bf16_hi(vv[u].x), bf16_lo(vv[u].y), bf16_hi(vv[u].y)};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      tv += (t0 + k < ntail) ? pt[min(t0 + k, kTailTok - 1)] * v4[k] : 0.0f;
    }
  }
  tv = group_sum<TPC>(tv);
  const int lane = tid & 63, wv = tid >> 6;
  if (lane < NQ) *reinterpret_cast<float4*>(part + wv * CH + 4 * lane) = sum;
  if (tid % TPC == 0) tsum[cv] = tv;
  __syncthreads();
  if (tid < CH) {
    float t = tsum[tid];
#pragma unroll
    for (int i = 0; i < kCombineThreads / 64; ++i) t += part[i * CH + tid];
    a.out[((size_t)si * G.Hq + hq) * D + cb * CH + tid] = f32_to_bf16_rne(t / den);
  }
}

template <int NR, int TT, int FMT>
int launch_attn(const AttnArgs& a, int n_seqs, void* stream) {
  const dim3 grid(a.n_splits, a.G.Hkv, n_seqs);
  if (a.G.compressed) {
    // K tile, escape staging (one shared area for 64-token blocks), query, bases per version
    const size_t lds = (size_t)kSB * (32 * NR) * 2 + (size_t)(TT == kSB ? 1 : 4) * max(a.G.esc_cap, 16) +
                       (size_t)a.G.g * (32 * NR) * 2 + (size_t)a.G.n_versions * 2 * NR * 16 * 4;
    hipLaunchKernelGGL((attn_comp_kernel<NR, TT, FMT>), grid, dim3(kWave), lds, (hipStream_t)stream, a);
  } else {
    hipLaunchKernelGGL((attn_raw_kernel<NR, TT, FMT>), grid, dim3(kWave), 0, (hipStream_t)stream, a);
  }
  return (int)hipGetLastError();
}

template <int NR, int FMT>
int launch_attn_t(const AttnArgs& a, int n_seqs, void* stream) {
  switch (a.G.T) {
    case 16: return launch_attn<NR, 16, FMT>(a, n_seqs, stream);
    case 32: return launch_attn<NR, 32, FMT>(a, n_seqs, stream);
    case 64: return launch_attn<NR, 64, FMT>(a, n_seqs, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

// 8-token groups: 64-token blocks only, and the tile offsets this kernel is compiled for.
template <int NH, int FMT>
int launch_attn_g8(const AttnArgs& a, int n_seqs, void* stream) {
  using Q = TG8<NH, FMT>;
  const Geo& G = a.G;
  if (G.T != kSB || G.GT != 8 || G.mode_set != 0 || G.code_off != Q::CODE_OFF || G.sm_off != Q::SM_OFF ||
      G.esc_off != Q::ESC_OFF || G.PW != Q::PW || G.esc_cap > 512)
    return (int)hipErrorInvalidValue;
  const dim3 grid(a.n_splits, G.Hkv, n_seqs);
  // K tile, escape staging (+16 bytes that the byte reads may touch past the last piece), query,
  // bases per version
  const size_t lds = (size_t)kSB * Q::D * 2 + (size_t)((max(G.esc_cap, 16) + 15) / 16 * 16 + 16) +
                     (size_t)G.g * Q::D * 2 + (size_t)G.n_versions * 64 * NH * 4;
  hipLaunchKernelGGL((attn_g8_kernel<NH, FMT>), grid, dim3(kWave), lds, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

template <int FMT>
int launch_attn_f(const AttnArgs& a, int n_seqs, void* stream) {
  if (a.G.compressed && a.G.GT == 8)
    return (a.G.D == 128) ? launch_attn_g8<2, FMT>(a, n_seqs, stream) : launch_attn_g8<1, FMT>(a, n_seqs, stream);
  return (a.G.D == 128) ? launch_attn_t<4, FMT>(a, n_seqs, stream) : launch_attn_t<2, FMT>(a, n_seqs, stream);
}

}  // namespace

int launch_attention_partials(const Geo& G, const DevBufs& B, const SeqList& S, const uint16_t* q, float scale,
                              int n_splits, float* ws_acc, float* ws_ml, const void* k_new, const void* v_new,
                              const int* new_pos, void* stream) {
  AttnArgs a;
  a.k_new = reinterpret_cast<const uint8_t*>(k_new);
  a.v_new = reinterpret_cast<const uint8_t*>(v_new);
  // longest first (stable): with the same split count for every sequence, a long sequence's
  // workgroups carry the most blocks, and dispatching them first shortens the kernel's tail
  int order[kMaxSeqsPerLaunch];
  for (int i = 0; i < S.n; ++i) order[i] = i;
  std::stable_sort(order, order + S.n, [&](int x, int y) { return S.lens[x] > S.lens[y]; });
  for (int z = 0; z < kMaxSeqsPerLaunch; ++z) {
    const int i = z < S.n ? order[z] : 0;
    a.zrow[z] = z < S.n ? make_int4(i, S.ids[i], S.lens[i], k_new ? new_pos[i] : 0) : make_int4(0, 0, 0, 0);
  }
  a.G = G;
  a.B = B;
  a.q = q;
  a.ws_acc = ws_acc;
  a.ws_ml = ws_ml;
  a.sl2 = scale * 1.4426950408889634f;
  a.n_splits = n_splits;
  switch (G.fmt) {
    case 0: return launch_attn_f<0>(a, S.n, stream);
    case 1: return launch_attn_f<1>(a, S.n, stream);
    case 2: return launch_attn_f<2>(a, S.n, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

template <int NR, int FMT>
void (*pick_combine(int n_splits))(CombineArgs) {
  constexpr int D = 32 * NR;
  if constexpr (D <= 128)  // one block per head (a 256-channel head always takes 16-channel slices)
    if (n_splits <= 4 * (kCombineThreads / (D / 4))) return combine_kernel<NR, FMT, D, 4>;
  if (n_splits <= 4 * (kCombineThreads / 4)) return combine_kernel<NR, FMT, 16, 4>;
  return combine_kernel<NR, FMT, 16, 16>;
}

int launch_combine(const Geo& G, const DevBufs& B, const SeqList& S, const uint16_t* q, float scale, int n_splits,
                   const float* ws_acc, const float* ws_ml, uint16_t* out, void* stream) {
  CombineArgs a;
  a.G = G;
  a.S = S;
  a.tail = reinterpret_cast<const uint8_t*>(B.tail);
  a.q = q;
  a.ws_acc = ws_acc;
  a.ws_ml = ws_ml;
  a.out = out;
  a.sl2 = scale * 1.4426950408889634f;
  a.n_splits = n_splits;
  if (n_splits < 1 || n_splits > kMaxSplits || G.T > kTailTok || G.T < 4) return (int)hipErrorInvalidValue;
  void (*k)(CombineArgs) = nullptr;
  const bool d128 = G.D == 128, d256 = G.D == 256;
  switch (G.fmt) {
    case 0: k = d256 ? pick_combine<8, 0>(n_splits) : d128 ? pick_combine<4, 0>(n_splits) : pick_combine<2, 0>(n_splits); break;
    case 1: k = d256 ? pick_combine<8, 1>(n_splits) : d128 ? pick_combine<4, 1>(n_splits) : pick_combine<2, 1>(n_splits); break;
    case 2: k = d256 ? pick_combine<8, 2>(n_splits) : d128 ? pick_combine<4, 2>(n_splits) : pick_combine<2, 2>(n_splits); break;
    default: return (int)hipErrorInvalidValue;
  }
  const int ch = (G.D <= 128 && n_splits <= 4 * (kCombineThreads / (G.D / 4))) ? G.D : 16;
  hipLaunchKernelGGL(k, dim3(G.D / ch, G.Hq, S.n), dim3(kCombineThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

// ---- the split workspace of kv_decode_attention_noalloc -----------------------------------
// A fixed array of device memory for callers that cannot allocate.  Each GPU the library runs
// on holds its own copy (at its own address) until the process ends.  In host code the name
// `scratch` is only a host-side stand-in: its device address comes from hipGetSymbolAddress,
// resolved once per device with that device current, and only that address is ever passed on.
static __device__ __align__(256) uint8_t scratch[KVC_NOALLOC_WS_BYTES];

int noalloc_workspace(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

}  // namespace kvc

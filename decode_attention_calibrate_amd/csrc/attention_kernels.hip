// attention_kernels.hip -- split-K decode attention over the paged KV cache and the
// log-sum-exp merge of the splits.
//
// Method: page "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal
// Devices", §3.2 -- the kernel reads compressed tiles and rebuilds only the values attention
// needs on chip (no decompressed copy of the cache in HBM); compressed blocks, raw blocks and
// the uncompressed tail share one softmax normalisation.
//
// Work decomposition (one 64-lane wave per workgroup):
//   grid = (split, kv-head, sequence).  A split walks a contiguous range of 64-token
//   super-blocks.  Lane l = n + 16j: j (0..3) selects the 16-token group t0+16j..t0+16j+15 of the
//   super-block, n (0..15) a query head (QK output), a channel pair (rebuild, PV) or an MFMA row.
//   QK   : v_mfma_f32_16x16x32_bf16 with A = K rows from LDS (16 tokens x 32 channels) and
//          B = the g query heads (columns n < g used).  Row m of MFMA rb is token
//          16(m/4) + 4rb + m%4, so lane n + 16j ends up holding the scores of head n for its own
//          token group j.
//   PV   : the same MFMA with A = P (rows = heads, k = 8 tokens of group j per lane) and B = V
//          (k = the same 8 tokens, columns = 16 channels).  A group owner's rebuilt V values are
//          already B operands, so V never touches LDS; P is split into a bf16 high part and a bf16
//          low part (two MFMAs) so the probabilities keep ~16 mantissa bits.
//   K    : group owners rebuild 16 tokens x 2 channels and write them to an XOR-swizzled LDS
//          tile [64 tokens][D] (16-byte chunks, chunk ^ ((row & 3) | ((row >> 2) & 4))) that the
//          QK A-operand reads conflict-free.
//   Softmax: online, fp32, base-2 (scores pre-multiplied by scale*log2(e)); per-split outputs
//          (acc, max, sum) go to the workspace and combine_kernel merges them.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "codec_dev.h"
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
  SeqList S;
  const uint16_t* q;
  float* ws_acc;
  float* ws_ml;
  float sl2;  // scale * log2(e)
  int n_splits;
};

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

// Where the 16-token group starting at token t of one (sequence, K|V, head) lives.
struct Src {
  int kind;              // SRC_COMP, SRC_RAW (raw tile or tail), SRC_NONE
  int tg;                // token group inside the tile
  int valid;             // valid tokens in the group (0..16)
  uint32_t esc_units;    // escape bytes / 16 (compressed)
  const uint8_t* comp;   // compressed tile (never null: clamped to slot 0 when unused)
  const uint16_t* raw;   // raw tile or tail tile
};

__device__ __forceinline__ Src resolve(const Geo& G, const DevBufs& B, int seq, int L, int t, int kv, int h,
                                       uint32_t entry) {
  Src s;
  s.kind = SRC_NONE;
  s.tg = 0;
  s.valid = 0;
  s.esc_units = 0;
  s.comp = B.comp_pool;
  s.raw = B.tail;
  const int n_full = L / G.T;
  if (t >= L) return s;
  if (t < n_full * G.T) {
    s.tg = (t % G.T) >> 4;
    if (entry == kUnallocated) {
      atomicOr(&B.counters->status, 4u);
      return s;
    }
    const uint32_t slot = entry & 0x00FFFFFFu;
    s.valid = 16;
    if (entry & 0x80000000u) {
      s.kind = SRC_RAW;
      s.raw = B.raw_pool + (size_t)slot * G.raw_elems;
    } else {
      s.kind = SRC_COMP;
      s.comp = B.comp_pool + (size_t)slot * G.stride;
      s.esc_units = (entry >> 24) & 0x7Fu;
    }
  } else {
    s.kind = SRC_RAW;
    s.tg = (t - n_full * G.T) >> 4;
    s.valid = min(16, L - t);
    s.raw = B.tail + tail_offset(G, seq, kv, h);
  }
  return s;
}

__device__ __forceinline__ uint32_t load_entry(const Geo& G, const DevBufs& B, int seq, int L, int t, int kv, int h) {
  const int n_full = L / G.T;
  if (t >= L || t >= n_full * G.T) return kUnallocated;
  return B.table[table_index(G, seq, t / G.T, kv, h)];
}

// Compressed-tile registers of one lane for one super-block: tag words, escape bytes,
// sign/mantissa and code words of its NR group pairs.
template <int NR>
struct CompRegs {
  uint32_t tE, tR;
  uint4 esc0, esc1;
  uint4 sm[NR][2];
  uint32_t cd[NR][3];
};

template <int NR>
__device__ __forceinline__ void load_comp(const Geo& G, const Src& s, int n, CompRegs<NR>& r) {
  const uint8_t* t = s.comp;
  r.tE = 0;
  r.tR = 0;
  if (n < G.PW) {
    r.tE = ld32(t + G.tag_off + 4 * n);
    r.tR = ld32(t + G.tag_off + 4 * (G.PW + n));
  }
  r.esc0 = make_uint4(0, 0, 0, 0);
  r.esc1 = make_uint4(0, 0, 0, 0);
  if (n < (int)s.esc_units) r.esc0 = ld128(t + G.esc_off + 16 * n);
  if (n + 16 < (int)s.esc_units) r.esc1 = ld128(t + G.esc_off + 16 * (n + 16));
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int pr = s.tg * (G.D / 2) + 16 * i + n;
    r.sm[i][0] = ld128(t + G.sm_off + 32 * pr);
    r.sm[i][1] = ld128(t + G.sm_off + 32 * pr + 16);
    const uint8_t* c = t + G.code_off + 12 * pr;
    r.cd[i][0] = ld32(c);
    r.cd[i][1] = ld32(c + 4);
    r.cd[i][2] = ld32(c + 8);
  }
}

// Stage the escape bytes of lane group j into LDS and compute the exclusive plane prefix of
// each tag word (held by lane 16j + w).
template <int NR>
__device__ __forceinline__ uint32_t stage_escape(const CompRegs<NR>& r, const Src& s, int n, uint8_t* esc_lds) {
  if (s.kind == SRC_COMP) {
    if (n < (int)s.esc_units) *reinterpret_cast<uint4*>(esc_lds + 16 * n) = r.esc0;
    if (n + 16 < (int)s.esc_units) *reinterpret_cast<uint4*>(esc_lds + 16 * (n + 16)) = r.esc1;
  }
  const uint32_t cnt = __popc(r.tE) + 4u * __popc(r.tR);
  uint32_t incl = cnt;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    const uint32_t v = __shfl_up(incl, o, 16);
    if (n >= o) incl += v;
  }
  return incl - cnt;
}

// Rebuild the pair of round i for lane n of lane group j.  bases: b3[c0], b3[c1], b4[c0], b4[c1].
template <int NR>
__device__ __forceinline__ void rebuild_pair(const Geo& G, const CompRegs<NR>& r, int i, int j, int tg, uint32_t pfx,
                                             uint32_t bases, const uint16_t* esc16, int max_plane, uint32_t* status,
                                             uint32_t outs[2][2][4]) {
  const int w = tg * (G.D / 32) + i;            // tag word of this pair (same word for both groups)
  const int bit = (2 * (16 * i + (threadIdx.x & 15))) & 31;
  const uint32_t Ew = __shfl(r.tE, 16 * j + w);
  const uint32_t Rw = __shfl(r.tR, 16 * j + w);
  const uint32_t Pw = __shfl(pfx, 16 * j + w);
  uint32_t P = planes_before(Ew, Rw, Pw, bit);
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const uint32_t E = (Ew >> (bit + gi)) & 1u, R = (Rw >> (bit + gi)) & 1u;
    if (R && !E) atomicOr(status, 8u);
    const uint32_t b3 = (bases >> (8 * gi)) & 0xFFu, b4 = (bases >> (16 + 8 * gi)) & 0xFFu;
    const uint32_t base = R ? 0u : (E ? b4 : b3);
    const int p0 = min((int)P, max_plane);
    const uint32_t plane0 = E ? (uint32_t)esc16[p0] : 0u;
    uint32_t pl[4] = {0u, 0u, 0u, 0u};
    int nextra = 0;
    if (R) {
      nextra = 4;
#pragma unroll
      for (int p = 0; p < 4; ++p) pl[p] = esc16[min((int)P + 1 + p, max_plane)];
    }
    const uint4 sv = r.sm[i][gi];
    const uint32_t smv[4] = {sv.x, sv.y, sv.z, sv.w};
    if (gi == 0) rebuild_group<0>(smv, r.cd[i][0], r.cd[i][1], r.cd[i][2], base, plane0, pl, nextra, outs[0][0], outs[0][1]);
    else rebuild_group<1>(smv, r.cd[i][0], r.cd[i][1], r.cd[i][2], base, plane0, pl, nextra, outs[1][0], outs[1][1]);
    P += E + 4u * R;
  }
}

// Online-softmax state update for one super-block.  s[16]: this lane's 16 scores (already in
// base-2 units, masked to -inf); returns the probabilities in p and the rescale factor.
__device__ __forceinline__ float softmax_update(float s[16], float& m, float& l) {
  float mx = s[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) mx = fmaxf(mx, s[k]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m, mx);
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  const float alpha = exp2f(m - m_use);
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    s[k] = exp2f(s[k] - m_use);
    sum += s[k];
  }
  l = l * alpha + sum;
  m = m_new;
  return alpha;
}

template <int NR>
__device__ __forceinline__ void rescale_acc(f32x4_t acc[NR][2], float alpha, int j) {
  float a[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) a[r] = __shfl(alpha, 4 * j + r);
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][x][r] *= a[r];
}

// P as MFMA A operands (high and low bf16 parts).  INTERLEAVED: token order (0,2,1,3,4,6,5,7)
// matching the rebuilt V words; otherwise natural order.
template <bool INTERLEAVED>
__device__ __forceinline__ void pack_p(const float p[16], uint4 hi[2], uint4 lo[2]) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    float v[8], w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int src = INTERLEAVED ? ((k & 4) | ((k & 1) << 1) | ((k >> 1) & 1)) : k;
      v[k] = p[8 * e + src];
      w[k] = v[k] - bf16_round(v[k]);
    }
    hi[e] = make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
    lo[e] = make_uint4(pack2(w[0], w[1]), pack2(w[2], w[3]), pack2(w[4], w[5]), pack2(w[6], w[7]));
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
      float* dst = a.ws_acc + (((size_t)si * G.Hq + h * G.g + head) * S + split) * G.D;
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

// Natural-order raw V words for channel c and tokens tg*16 + 8e .. +8 (masked past valid).
__device__ __forceinline__ uint4 raw_v_operand(const Geo& G, const Src& s, int c, int e) {
  uint4 v = ld128(s.raw + (size_t)c * G.T + s.tg * 16 + 8 * e);
  const int keep = s.valid - 8 * e;  // tokens of this 8-token half still valid
  if (keep < 8) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t m = (2 * k < keep ? 0x0000FFFFu : 0u) | (2 * k + 1 < keep ? 0xFFFF0000u : 0u);
      w[k] &= m;
    }
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return v;
}

// ------------------------------------------------------------------------------------------
// Compressed cache.
template <int NR>
__global__ void __launch_bounds__(kWave) attn_comp_kernel(AttnArgs a) {
  constexpr int D = 32 * NR;
  extern __shared__ uint4 lds4[];
  uint8_t* klds = reinterpret_cast<uint8_t*>(lds4);              // [64][D] bf16, swizzled
  uint8_t* esc_base = klds + kSB * D * 2;                         // [4][esc_cap]
  const Geo& G = a.G;
  const DevBufs& B = a.B;
  const int lane = threadIdx.x, n = lane & 15, j = lane >> 4;
  const int split = blockIdx.x, h = blockIdx.y, si = blockIdx.z;
  const int seq = a.S.ids[si], L = a.S.lens[si];
  const int nsb = (L + kSB - 1) / kSB;
  const int per = (nsb + a.n_splits - 1) / a.n_splits;
  const int sb0 = split * per, sb1 = min(nsb, sb0 + per);
  const int esc_room = max(G.esc_cap, 16);                        // LDS bytes per lane group
  uint8_t* esc_lds = esc_base + j * esc_room;
  const uint16_t* esc16 = reinterpret_cast<const uint16_t*>(esc_lds);
  const int max_plane = esc_room / 2 - 1;

  // query heads h*g + n as B operands: channels 32ks + 8j .. +8
  uint4 qb[NR];
#pragma unroll
  for (int ks = 0; ks < NR; ++ks)
    qb[ks] = (n < G.g) ? ld128(a.q + ((size_t)si * G.Hq + h * G.g + n) * D + 32 * ks + 8 * j) : make_uint4(0, 0, 0, 0);
  // calibrated bases of this lane's channel pairs (c0 = 32i + 2n), K and V
  uint32_t kbase[NR], vbase[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int c0 = 32 * i + 2 * n;
    const uint8_t* bk = B.bases + (size_t)h * D;
    const uint8_t* bv = B.bases + ((size_t)2 * G.Hkv + h) * D;
    const size_t wide = (size_t)G.Hkv * D;
    kbase[i] = bk[c0] | (bk[c0 + 1] << 8) | (bk[wide + c0] << 16) | (bk[wide + c0 + 1] << 24);
    vbase[i] = bv[c0] | (bv[c0 + 1] << 8) | (bv[wide + c0] << 16) | (bv[wide + c0 + 1] << 24);
  }

  float m = -INFINITY, l = 0.0f;
  f32x4_t acc[NR][2];
#pragma unroll
  for (int i = 0; i < NR; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint32_t eK = 0, eV = 0;
  if (sb0 < sb1) {
    eK = load_entry(G, B, seq, L, sb0 * kSB + 16 * j, 0, h);
    eV = load_entry(G, B, seq, L, sb0 * kSB + 16 * j, 1, h);
  }
  for (int sb = sb0; sb < sb1; ++sb) {
    const int t_j = sb * kSB + 16 * j;
    const Src sK = resolve(G, B, seq, L, t_j, 0, h, eK);
    const Src sV = resolve(G, B, seq, L, t_j, 1, h, eV);
    CompRegs<NR> rK, rV;
    load_comp<NR>(G, sK, n, rK);
    load_comp<NR>(G, sV, n, rV);
    if (sb + 1 < sb1) {
      eK = load_entry(G, B, seq, L, t_j + kSB, 0, h);
      eV = load_entry(G, B, seq, L, t_j + kSB, 1, h);
    }

    // ---- K: rebuild into the LDS tile ----
    __syncthreads();
    const uint32_t pfxK = stage_escape<NR>(rK, sK, n, esc_lds);
    __syncthreads();
    if (sK.kind == SRC_COMP) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        uint32_t o[2][2][4];
        rebuild_pair<NR>(G, rK, i, j, sK.tg, pfxK, kbase[i], esc16, max_plane, &B.counters->status, o);
        const int chunk = 4 * i + (n >> 2), off = 4 * (n & 3);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r0 = 16 * j + 4 * jj;
          const uint32_t w0 = perm_b32(o[1][0][jj], o[0][0][jj], 0x05040100u);
          const uint32_t w2 = perm_b32(o[1][0][jj], o[0][0][jj], 0x07060302u);
          const uint32_t w1 = perm_b32(o[1][1][jj], o[0][1][jj], 0x05040100u);
          const uint32_t w3 = perm_b32(o[1][1][jj], o[0][1][jj], 0x07060302u);
          *reinterpret_cast<uint32_t*>(klds + (r0 + 0) * 2 * D + ((chunk ^ swz(r0 + 0)) << 4) + off) = w0;
          *reinterpret_cast<uint32_t*>(klds + (r0 + 1) * 2 * D + ((chunk ^ swz(r0 + 1)) << 4) + off) = w1;
          *reinterpret_cast<uint32_t*>(klds + (r0 + 2) * 2 * D + ((chunk ^ swz(r0 + 2)) << 4) + off) = w2;
          *reinterpret_cast<uint32_t*>(klds + (r0 + 3) * 2 * D + ((chunk ^ swz(r0 + 3)) << 4) + off) = w3;
        }
      }
    } else if (sK.kind == SRC_RAW) {
      // raw K tile / tail: token-major rows, copied 16 bytes at a time
      for (int k = n; k < 16 * (D / 8); k += 16) {
        const int rr = k / (D / 8), chunk = k % (D / 8), row = 16 * j + rr;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (rr < sK.valid) v = ld128(sK.raw + (size_t)(sK.tg * 16 + rr) * D + 8 * chunk);
        *reinterpret_cast<uint4*>(klds + row * 2 * D + ((chunk ^ swz(row)) << 4)) = v;
      }
    }
    __syncthreads();

    // ---- QK ----
    float s[16];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
      const int row = 16 * (n >> 2) + 4 * rb + (n & 3);
#pragma unroll
      for (int ks = 0; ks < NR; ++ks) {
        const uint4 av = *reinterpret_cast<const uint4*>(klds + row * 2 * D + (((4 * ks + j) ^ swz(row)) << 4));
        c = mfma16(av, qb[ks], c);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s[4 * rb + r] = (4 * rb + r < sK.valid && 4 * rb + r < sV.valid) ? c[r] * a.sl2 : -INFINITY;
    }
    const float alpha = softmax_update(s, m, l);
    rescale_acc<NR>(acc, alpha, j);
    uint4 phi[2], plo[2];
    pack_p<true>(s, phi, plo);

    // ---- V: rebuild straight into B operands ----
    __syncthreads();
    const uint32_t pfxV = stage_escape<NR>(rV, sV, n, esc_lds);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      uint4 bv[2][2];
      if (sV.kind == SRC_COMP) {
        uint32_t o[2][2][4];
        rebuild_pair<NR>(G, rV, i, j, sV.tg, pfxV, vbase[i], esc16, max_plane, &B.counters->status, o);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          bv[x][0] = make_uint4(o[x][0][0], o[x][1][0], o[x][0][1], o[x][1][1]);
          bv[x][1] = make_uint4(o[x][0][2], o[x][1][2], o[x][0][3], o[x][1][3]);
        }
      } else if (sV.kind == SRC_RAW) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint4 v = raw_v_operand(G, sV, 32 * i + 2 * n + x, e);
            bv[x][e] = make_uint4(perm_b32(v.y, v.x, 0x05040100u), perm_b32(v.y, v.x, 0x07060302u),
                                  perm_b32(v.w, v.z, 0x05040100u), perm_b32(v.w, v.z, 0x07060302u));
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
  write_partial<NR>(a, si, h, split, m, l, acc);
}

// ------------------------------------------------------------------------------------------
// Uncompressed cache (every tile raw): the speedup baseline.  K rows are loaded straight into
// QK A operands and V straight into PV B operands; no LDS.
template <int NR>
__global__ void __launch_bounds__(kWave) attn_raw_kernel(AttnArgs a) {
  constexpr int D = 32 * NR;
  const Geo& G = a.G;
  const DevBufs& B = a.B;
  const int lane = threadIdx.x, n = lane & 15, j = lane >> 4;
  const int split = blockIdx.x, h = blockIdx.y, si = blockIdx.z;
  const int seq = a.S.ids[si], L = a.S.lens[si];
  const int nsb = (L + kSB - 1) / kSB;
  const int per = (nsb + a.n_splits - 1) / a.n_splits;
  const int sb0 = split * per, sb1 = min(nsb, sb0 + per);

  uint4 qb[NR];
#pragma unroll
  for (int ks = 0; ks < NR; ++ks)
    qb[ks] = (n < G.g) ? ld128(a.q + ((size_t)si * G.Hq + h * G.g + n) * D + 32 * ks + 8 * j) : make_uint4(0, 0, 0, 0);

  float m = -INFINITY, l = 0.0f;
  f32x4_t acc[NR][2];
#pragma unroll
  for (int i = 0; i < NR; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint32_t eK = 0, eV = 0;
  if (sb0 < sb1) {
    eK = load_entry(G, B, seq, L, sb0 * kSB + 16 * j, 0, h);
    eV = load_entry(G, B, seq, L, sb0 * kSB + 16 * j, 1, h);
  }
  for (int sb = sb0; sb < sb1; ++sb) {
    const int t_j = sb * kSB + 16 * j;
    const Src sK = resolve(G, B, seq, L, t_j, 0, h, eK);
    const Src sV = resolve(G, B, seq, L, t_j, 1, h, eV);
    // K source of the token group this lane's MFMA rows come from (group n / 4)
    const int jr = n >> 2;
    const int kindR = __shfl(sK.kind, 16 * jr), tgR = __shfl(sK.tg, 16 * jr), validR = __shfl(sK.valid, 16 * jr);
    const uint16_t* rawR = reinterpret_cast<const uint16_t*>(
        __shfl((unsigned long long)reinterpret_cast<uintptr_t>(sK.raw), 16 * jr));
    uint4 ka[4][NR];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int rr = 4 * rb + (n & 3);
#pragma unroll
      for (int ks = 0; ks < NR; ++ks)
        ka[rb][ks] = (kindR == SRC_RAW && rr < validR) ? ld128(rawR + (size_t)(tgR * 16 + rr) * D + 32 * ks + 8 * j)
                                                        : make_uint4(0, 0, 0, 0);
    }
    uint4 vb[NR][2][2];
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          vb[i][x][e] = (sV.kind == SRC_RAW) ? raw_v_operand(G, sV, 32 * i + 2 * n + x, e) : make_uint4(0, 0, 0, 0);
    if (sb + 1 < sb1) {
      eK = load_entry(G, B, seq, L, t_j + kSB, 0, h);
      eV = load_entry(G, B, seq, L, t_j + kSB, 1, h);
    }

    float s[16];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NR; ++ks) c = mfma16(ka[rb][ks], qb[ks], c);
#pragma unroll
      for (int r = 0; r < 4; ++r) s[4 * rb + r] = (4 * rb + r < sK.valid && 4 * rb + r < sV.valid) ? c[r] * a.sl2 : -INFINITY;
    }
    const float alpha = softmax_update(s, m, l);
    rescale_acc<NR>(acc, alpha, j);
    uint4 phi[2], plo[2];
    pack_p<false>(s, phi, plo);
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          acc[i][x] = mfma16(phi[e], vb[i][x][e], acc[i][x]);
          acc[i][x] = mfma16(plo[e], vb[i][x][e], acc[i][x]);
        }
  }
  write_partial<NR>(a, si, h, split, m, l, acc);
}

// Log-sum-exp merge of the splits: one block per (query head, sequence), one thread per channel.
__global__ void combine_kernel(int Hq, int D, int S, const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
                               uint16_t* __restrict__ out) {
  const int hq = blockIdx.x, si = blockIdx.y, c = threadIdx.x;
  if (c >= D) return;
  const float* ml = ws_ml + ((size_t)si * Hq + hq) * S * 2;
  const float* acc = ws_acc + ((size_t)si * Hq + hq) * S * D;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s)
    if (ml[2 * s + 1] > 0.0f) M = fmaxf(M, ml[2 * s]);
  float num = 0.0f, den = 0.0f;
  for (int s = 0; s < S; ++s) {
    const float ls = ml[2 * s + 1];
    if (ls > 0.0f) {
      const float w = exp2f(ml[2 * s] - M);
      num += w * acc[(size_t)s * D + c];
      den += w * ls;
    }
  }
  out[((size_t)si * Hq + hq) * D + c] = f32_to_bf16_rne(num / den);
}

template <int NR>
int launch_attn_nr(const AttnArgs& a, int n_seqs, void* stream) {
  const dim3 grid(a.n_splits, a.G.Hkv, n_seqs);
  if (a.G.compressed) {
    const size_t lds = (size_t)kSB * (32 * NR) * 2 + (size_t)4 * max(a.G.esc_cap, 16);
    hipLaunchKernelGGL(attn_comp_kernel<NR>, grid, dim3(kWave), lds, (hipStream_t)stream, a);
  } else {
    hipLaunchKernelGGL(attn_raw_kernel<NR>, grid, dim3(kWave), 0, (hipStream_t)stream, a);
  }
  return (int)hipGetLastError();
}

}  // namespace

int launch_attention_partials(const Geo& G, const DevBufs& B, const SeqList& S, const uint16_t* q, float scale,
                              int n_splits, float* ws_acc, float* ws_ml, void* stream) {
  AttnArgs a;
  a.G = G;
  a.B = B;
  a.S = S;
  a.q = q;
  a.ws_acc = ws_acc;
  a.ws_ml = ws_ml;
  a.sl2 = scale * 1.4426950408889634f;
  a.n_splits = n_splits;
  return (G.D == 128) ? launch_attn_nr<4>(a, S.n, stream) : launch_attn_nr<2>(a, S.n, stream);
}

int launch_combine(const Geo& G, int n_seqs, int n_splits, const float* ws_acc, const float* ws_ml, uint16_t* out,
                   void* stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(G.Hq, n_seqs), dim3(G.D), 0, (hipStream_t)stream, G.Hq, G.D, n_splits,
                     ws_acc, ws_ml, out);
  return (int)hipGetLastError();
}

}  // namespace kvc

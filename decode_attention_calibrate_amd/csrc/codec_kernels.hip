// codec_kernels.hip -- cache initialisation, window calibration, block encode (append), tail
// update, slot release and block decode for the lossless KV codec of the page "GAAC: Lossless
// KV Compression for Bandwidth-Efficient LLM Inference on Personal Devices" (§3.1 codec,
// §3.3 fill-then-finalize blocks in fixed-capacity slots with a block table).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec_dev.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int kThreads = 256;

// Element bits at index i of a BF16 (EB = 2) or FP8 (EB = 1) element array.
__device__ __forceinline__ uint32_t elem_at(const void* p, size_t i, int EB) {
  return EB == 2 ? (uint32_t)reinterpret_cast<const uint16_t*>(p)[i] : (uint32_t)reinterpret_cast<const uint8_t*>(p)[i];
}
__device__ __forceinline__ void elem_put(void* p, size_t i, int EB, uint32_t x) {
  if (EB == 2) reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)x;
  else reinterpret_cast<uint8_t*>(p)[i] = (uint8_t)x;
}
__device__ __forceinline__ uint32_t exp_of(const Geo& G, uint32_t x) { return (x >> G.MB) & ((1u << G.F) - 1u); }
// (sign << MB) | mantissa
__device__ __forceinline__ uint32_t sm_of(const Geo& G, uint32_t x) {
  return ((x >> (G.MB + G.F)) << G.MB) | (x & ((1u << G.MB) - 1u));
}

__device__ __forceinline__ int block_sum(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  int s = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  return s;
}

__device__ __forceinline__ int block_max(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  int s = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) s = max(s, red[i]);
  return s;
}

// Exclusive prefix sum over the block (thread order); *total receives the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) red[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
    if (i < w) before += red[i];
    all += red[i];
  }
  *total = all;
  return before + incl - v;
}

__global__ void init_kernel(Geo G, DevBufs B) {
  const size_t n_table = (size_t)G.max_seqs * G.max_blocks * 2 * G.Hkv;
  const size_t n_bases = (size_t)G.n_versions * G.ver_bytes;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_table; i += stride) B.table[i] = kUnallocated;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_bases; i += stride) B.bases[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x < kPoolStripes) {
    Counters* c = B.counters;
    c->comp_top[threadIdx.x].n = G.compressed ? pool_stripe_size(G.n_comp, threadIdx.x) : 0;
    c->raw_top[threadIdx.x].n = pool_stripe_size(G.n_raw, threadIdx.x);
    if (threadIdx.x == 0) c->status = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x < kStatStripes) {
    StatStripe& st = B.counters->stat[threadIdx.x];
    st.raw_tiles = 0;
    st.groups[0] = st.groups[1] = st.groups[2] = st.groups[3] = 0;
    st.esc_bytes = 0;
  }
}

// One block per (channel, kv-head, K|V): histogram of the F-bit exponent field over the
// calibration tokens, then the 8- and 16-wide windows with the largest count (ties: lower median
// start).  A format whose exponent field is only 4 bits wide (E4M3) has no 16-wide window; its
// b4 stays 0.  Mode set 1 (a 2-bit mode) also takes the 4-wide window, stored after b3 and b4.
// The bases go to base version G.cur_ver.
__global__ void calibrate_kernel(Geo G, DevBufs B, const void* __restrict__ k, const void* __restrict__ v, int n) {
  __shared__ int hist[256];
  __shared__ int red[8];
  const int c = blockIdx.x, h = blockIdx.y, kv = blockIdx.z, tid = threadIdx.x;
  hist[tid] = 0;
  __syncthreads();
  const void* src = kv ? v : k;
  for (int t = tid; t < n; t += kThreads) atomicAdd(&hist[exp_of(G, elem_at(src, ((size_t)t * G.Hkv + h) * G.D + c, G.EB))], 1);
  __syncthreads();
  for (int w = G.mode_set == 1 ? 2 : 3; w <= 4 && w < G.F; ++w) {
    const int width = 1 << w, nb = (1 << G.F) - width + 1;
    int cov = -1;
    if (tid < nb) {
      cov = 0;
      for (int e = tid; e < tid + width; ++e) cov += hist[e];
    }
    const int best = block_max(cov, red);
    const int flag = (tid < nb && cov == best) ? 1 : 0;
    int count;
    const int rank = block_exclusive_scan(flag, red, &count);
    if (flag && rank == (count - 1) / 2) {
      B.bases[bases_at(G, G.cur_ver, w, kv, h) + c] = (uint8_t)tid;
    }
    __syncthreads();
  }
}

// Element format constants (kvc_dtype: 0 BF16, 1 FP8 E5M2, 2 FP8 E4M3).
template <int FMT>
struct EncFmt {
  static constexpr int F = FMT == 0 ? 8 : (FMT == 1 ? 5 : 4);
  static constexpr int MB = FMT == 0 ? 7 : (FMT == 1 ? 2 : 3);
  static constexpr int EB = FMT == 0 ? 2 : 1;
};

// Mode of a group from its exponent range and the channel's bases: 0 narrow, 1 wide, 2 raw.
__device__ __forceinline__ int choose_mode(uint32_t mn, uint32_t mx, uint32_t b3, uint32_t b4, bool has_wide) {
  if (b3 <= mn && mx <= b3 + 7) return 0;
  if (has_wide && b4 <= mn && mx <= b4 + 15) return 1;
  return 2;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

struct PairInfo {
  int mode[2];
  uint32_t base[2];
};

// Modes and bases of a pair of groups (channels c0, c0 + 1 of one token group) from its 16 words
// held in registers (token tau: channel c0 in the low half, c0 + 1 in the high half) and the two
// channels' bases.
template <int FMT>
__device__ __forceinline__ PairInfo pair_info_regs(const uint32_t pw[kGroup], uint32_t b3a, uint32_t b3b,
                                                   uint32_t b4a, uint32_t b4b) {
  using EF = EncFmt<FMT>;
  // both channels' exponents in 16-bit lanes, packed 16-bit min and max over the 16 tokens
  u16x2 lo = {0xFFFFu, 0xFFFFu}, hi = {0u, 0u};
#pragma unroll
  for (int tau = 0; tau < kGroup; ++tau) {
    const u16x2 e = __builtin_bit_cast(u16x2, (pw[tau] >> EF::MB) & (((1u << EF::F) - 1u) * 0x00010001u));
    lo = __builtin_elementwise_min(lo, e);
    hi = __builtin_elementwise_max(hi, e);
  }
  const uint32_t mn[2] = {lo.x, lo.y}, mx[2] = {hi.x, hi.y};
  PairInfo P;
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const uint32_t b3 = gi ? b3b : b3a, b4 = gi ? b4b : b4a;
    P.mode[gi] = choose_mode(mn[gi], mx[gi], b3, b4, EF::F > 4);
    P.base[gi] = P.mode[gi] == 0 ? b3 : (P.mode[gi] == 1 ? b4 : 0u);
  }
  return P;
}

// GT-bit escape units of a group: none (narrow), one plane (wide), F - 3 units (raw: bit 3,
// then BF16 bits 4..7 as four units of nibbles, E5M2 bit 4 as one more plane).
__device__ __forceinline__ int mode_planes(const Geo& G, int m) { return m == 0 ? 0 : (m == 1 ? 1 : G.F - 3); }

// The 16 bytes x (8 BF16 or 16 FP8 elements, in order) as consecutive 16-bit LDS elements at
// dst (16-byte aligned): one or two 16-byte stores.
template <int EB>
__device__ __forceinline__ void store_elems(uint16_t* dst, uint4 x) {
  if constexpr (EB == 2) {
    *reinterpret_cast<uint4*>(dst) = x;
  } else {  // FP8 bytes widened to 16 bits: bytes (b0, b1) of a word -> (b0, 0, b1, 0)
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t y[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      y[2 * k] = perm_b32(0u, w[k], 0x0C010C00u);
      y[2 * k + 1] = perm_b32(0u, w[k], 0x0C030C02u);
    }
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(y[0], y[1], y[2], y[3]);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(y[4], y[5], y[6], y[7]);
  }
}

// Gathers block b's T tokens into the LDS tile [T][D] with 16-byte loads along each source's
// contiguous axis: tokens still in the old tail (K token-major, V channel-major), then the
// appended tokens (token-major input, 16-byte aligned).  Unrolled so a thread's loads are in
// flight together.
template <int EB>
__device__ __forceinline__ void gather_block(const Geo& G, const uint8_t* tail, const void* in, int si, int h, int kv,
                                             int b, int L0, int n_tok, int tail_base, uint16_t* tile) {
  const int tid = threadIdx.x, D = G.D, T = G.T;
  constexpr int VE = 16 / EB;  // elements per 16-byte vector
  const int n_tail = min(max(L0 - b * T, 0), T);  // tokens of this block taken from the tail
  const int tt0 = b * T - tail_base;              // tail position of the block's first token
  const int nvpc = (n_tail + VE - 1) / VE;  // V: vectors per channel (the last one may be partial)
  const int nvt = kv ? D * nvpc : n_tail * (D / VE);
  const int nvi = (T - n_tail) * (D / VE);  // vectors of the appended tokens
#pragma unroll 4
  for (int v = tid; v < nvt; v += kThreads) {
    int t, c, st, sc;  // first element (t, c) and the element step along the vector
    const uint8_t* src;
    if (kv) { c = v / nvpc; t = (v % nvpc) * VE; src = tail + ((size_t)c * T + tt0 + t) * EB; st = 1; sc = 0; }
    else { t = v / (D / VE); c = (v % (D / VE)) * VE; src = tail + ((size_t)(tt0 + t) * D + c) * EB; st = 0; sc = 1; }
    const int ne = kv ? min(VE, n_tail - t) : VE;  // elements of this vector inside the tail
    uint4 x;
    if (ne == VE) {
      x = *reinterpret_cast<const uint4*>(src);
    } else {  // the ragged end of a V channel: element by element
      uint32_t w4[4] = {0u, 0u, 0u, 0u};
      for (int e = 0; e < ne; ++e)
        w4[e / (4 / EB)] |= elem_at(src, e, EB) << (8 * EB * (e % (4 / EB)));
      x = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    if (!kv) {  // K: the vector is VE consecutive channels of one token, whole
      store_elems<EB>(tile + t * D + c, x);
      continue;
    }
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const uint32_t val = EB == 2 ? (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu : (w[e >> 2] >> (8 * (e & 3))) & 0xFFu;
      if (e < ne) tile[(t + st * e) * D + c + sc * e] = (uint16_t)val;
    }
  }
#pragma unroll 4
  for (int v = tid; v < nvi; v += kThreads) {
    const int t = n_tail + v / (D / VE), c = (v % (D / VE)) * VE, p = b * T + t;
    const uint8_t* src = reinterpret_cast<const uint8_t*>(in) +
                         ((((size_t)si * n_tok + (p - L0)) * G.Hkv + h) * D + c) * EB;
    store_elems<EB>(tile + t * D + c, *reinterpret_cast<const uint4*>(src));
  }
}

// Pops a slot for one tile (raw or compressed, falling back to raw when the compressed pool is
// empty) and adds the tile to the statistics.  Thread 0 only; returns the slot (-1: both pools
// empty) and sets *raw.
// Pops a slot from one pool's sub-stacks, starting at sub-stack s0; -1 when all are empty.
__device__ int pop_from(PoolTop* top, const int32_t* stack, int s0) {
  for (int k = 0; k < kPoolStripes; ++k) {
    const int s = (s0 + k) % kPoolStripes;
    const int idx = atomicSub(&top[s].n, 1) - 1;
    if (idx >= 0) return stack[kPoolStripes * idx + s];
    atomicAdd(&top[s].n, 1);
  }
  return -1;
}

__device__ int pop_slot(const DevBufs& B, int want_raw, const unsigned long long modes[4], int esc_bytes, int* raw_out) {
  Counters* C = B.counters;
  const int h = blockIdx.x + 7 * blockIdx.y + 3 * blockIdx.z;  // spreads workgroups over the stripes
  int slot = -1, raw = want_raw;
  if (!raw) {
    slot = pop_from(C->comp_top, B.comp_free, h % kPoolStripes);
    if (slot < 0) {
      atomicOr(&C->status, 1u);
      raw = 1;
    }
  }
  if (raw) {
    slot = pop_from(C->raw_top, B.raw_free, h % kPoolStripes);
    if (slot < 0) atomicOr(&C->status, 2u);
  }
  if (slot >= 0) {
    StatStripe& st = C->stat[h % kStatStripes];
    if (raw) {
      atomicAdd(&st.raw_tiles, 1ull);
    } else {
      atomicAdd(&st.groups[0], modes[0]);
      atomicAdd(&st.groups[1], modes[1]);
      atomicAdd(&st.groups[2], modes[2]);
      if (modes[3]) atomicAdd(&st.groups[3], modes[3]);
      atomicAdd(&st.esc_bytes, (unsigned long long)esc_bytes);
    }
  }
  *raw_out = raw;
  return slot;
}

// Stores the LDS tile [T][D] as a raw tile (K token-major, V channel-major) and its table entry.
__device__ void store_raw_tile(const Geo& G, const DevBufs& B, int slot, int kv, const uint16_t* tile, size_t entry_idx) {
  const int D = G.D, T = G.T;
  uint8_t* dst = reinterpret_cast<uint8_t*>(B.raw_pool) + (size_t)slot * G.raw_elems * G.EB;
  for (int i = threadIdx.x; i < G.raw_elems; i += blockDim.x) {
    if (kv) {
      const int c = i / T, t = i % T;
      elem_put(dst, i, G.EB, tile[t * D + c]);
    } else {
      elem_put(dst, i, G.EB, tile[i]);
    }
  }
  if (threadIdx.x == 0) B.table[entry_idx] = (uint32_t)slot | kRawTile;
}

// One block per newly full block of one (sequence, K|V, head): gathers its T tokens from the
// old tail and the appended tokens, encodes it (or stores it raw), pops a slot and writes the
// block-table entry.

// Place the four 3-bit fields of slot s (one per byte lane, bits 0..2) at bits 3s..3s+2 of
// the byte lanes' 24-bit streams held in W[0..2] (byte lane k of word w = stream bits 8w..8w+7).
template <int SL>
__device__ __forceinline__ void place_slot(uint32_t W[3], uint32_t f) {
  constexpr int x = 3 * SL, w = x >> 3, b = x & 7;
  if constexpr (b <= 5) {
    W[w] |= f << b;  // fields < 8: no bit leaves its byte lane
  } else {
    W[w] |= (f << b) & (b == 6 ? 0xC0C0C0C0u : 0x80808080u);
    W[w + 1] |= (f >> (8 - b)) & (b == 6 ? 0x01010101u : 0x03030303u);
  }
}

template <int FMT>
__global__ void __launch_bounds__(kThreads) encode_kernel(Geo G, DevBufs B, SeqList S, const void* __restrict__ kin,
                                                          const void* __restrict__ vin, int n_tok) {
  using EF = EncFmt<FMT>;
  extern __shared__ uint4 smem4[];                                      // 16-byte aligned
  uint32_t* smem = reinterpret_cast<uint32_t*>(smem4);
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);                  // [T][D] logical
  uint32_t* tagw = smem + (G.raw_elems / 2);                            // [2][PW]
  __shared__ int red[8];
  __shared__ int sh_slot, sh_raw;
  __shared__ unsigned long long sh_modes[4];

  const int si = blockIdx.y, kv = blockIdx.z / G.Hkv, h = blockIdx.z % G.Hkv;
  const int seq = S.ids[si], L0 = S.lens[si];
  const int first_blk = L0 / G.T, last_full = (L0 + n_tok) / G.T;
  const int b = first_blk + blockIdx.x;
  if (b >= last_full) return;
  const int tid = threadIdx.x, D = G.D, T = G.T;
  const void* in = kv ? vin : kin;
  const uint8_t* tail = reinterpret_cast<const uint8_t*>(B.tail) + tail_offset(G, seq, kv, h) * G.EB;
  const int tail_base = first_blk * T;

  gather_block<EF::EB>(G, tail, in, si, h, kv, b, L0, n_tok, tail_base, tile);
  for (int i = tid; i < 2 * G.PW; i += kThreads) tagw[i] = 0;
  if (tid < 3) sh_modes[tid] = 0;
  __syncthreads();

  const size_t entry_idx = table_index(G, seq, b, kv, h);
  int is_raw = 1, total = 0;
  const uint8_t* b3 = bases_of(G, B.bases, G.cur_ver, 3, kv, h);  // blocks are encoded with the current bases
  const uint8_t* b4 = bases_of(G, B.bases, G.cur_ver, 4, kv, h);
  // One pair of groups per thread (G.NP <= 256 for T <= 64, D <= 128): channels c0, c0 + 1 of
  // token group tg, read from LDS once as 16 words (token tau: channel c0 in the low half).
  const int pr = tid, q0 = 2 * pr, tg = q0 / D, c0 = q0 % D;
  const bool has_pair = pr < G.NP;
  uint32_t pw[kGroup];
#pragma unroll
  for (int tau = 0; tau < kGroup; ++tau)
    pw[tau] = has_pair ? *reinterpret_cast<const uint32_t*>(tile + (tg * kGroup + tau) * D + c0) : 0u;
  PairInfo PI = {{0, 0}, {0u, 0u}};
  int my_before = 0;
  if (G.compressed) {
    // one block scan of three packed counts: escape units (bits 0..11; at most 256 pairs x 10),
    // wide groups (12..21) and raw groups (22..31; at most 512 each)
    int packed = 0;
    if (has_pair) {
      PI = pair_info_regs<FMT>(pw, b3[c0], b3[c0 + 1], b4[c0], b4[c0 + 1]);
      packed = mode_planes(G, PI.mode[0]) + mode_planes(G, PI.mode[1]) + ((PI.mode[0] == 1) + (PI.mode[1] == 1)) * (1 << 12) +
               ((PI.mode[0] == 2) + (PI.mode[1] == 2)) * (1 << 22);
    }
    int all = 0;
    my_before = block_exclusive_scan(packed, red, &all) & 0xFFF;
    total = all & 0xFFF;
    is_raw = (2 * total > G.esc_cap) ? 1 : 0;
    if (tid == 0) {
      const int wide = (all >> 12) & 0x3FF, rawg = (int)((unsigned)all >> 22);
      sh_modes[0] = (unsigned long long)(2 * G.NP - wide - rawg);
      sh_modes[1] = (unsigned long long)wide;
      sh_modes[2] = (unsigned long long)rawg;
      sh_modes[3] = 0;
    }
  }

  // BF16: the pair's fields are packed in registers while thread 0 pops the slot (its atomics'
  // round trips overlap the other waves' packing); stored once the slot is known.
  uint32_t W[3] = {0u, 0u, 0u}, smb[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  uint32_t units[2][5] = {{0u, 0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u, 0u}};
  if (FMT == 0 && has_pair && !is_raw) {
    // BF16, four tokens per word for both channels at once: word k of a quad holds channel c0 in
    // its low half; shifted right by 7 its bytes 0 and 2 are the two exponents, and one bit-select
    // puts each channel's sign/mantissa byte (sign << 7 | mantissa) in the same bytes.  v_perm then
    // gathers each channel's four bytes into one word (token 4 t4 + k in byte lane k).
    const uint32_t base2 = PI.base[0] | (PI.base[1] << 16);
    const uint32_t B0 = PI.base[0] * 0x01010101u, B1 = PI.base[1] * 0x01010101u;
    const bool any_raw = PI.mode[0] == 2 || PI.mode[1] == 2;
    uint32_t pl = 0;  // offset bit 3 of token tau at bit tau of each 16-bit half (the escape planes)
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      uint32_t ex[4], sx[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = pw[4 * t4 + k];
        ex[k] = w >> 7;
        sx[k] = bfi(0x00800080u, w >> 8, w);
        pl |= ((((ex[k] & 0x00FF00FFu) - base2) >> 3) & 0x00010001u) << (4 * t4 + k);
      }
      const uint32_t A = perm_b32(ex[1], ex[0], 0x06020400u), Bq = perm_b32(ex[3], ex[2], 0x06020400u);
      const uint32_t o0 = perm_b32(Bq, A, 0x05040100u) - B0, o1 = perm_b32(Bq, A, 0x07060302u) - B1;
      const uint32_t SA = perm_b32(sx[1], sx[0], 0x06020400u), SB = perm_b32(sx[3], sx[2], 0x06020400u);
      smb[t4] = perm_b32(SB, SA, 0x05040100u);
      smb[4 + t4] = perm_b32(SB, SA, 0x07060302u);
      switch (t4) {
        case 0: place_slot<0>(W, o0 & 0x07070707u); place_slot<4>(W, o1 & 0x07070707u); break;
        case 1: place_slot<1>(W, o0 & 0x07070707u); place_slot<5>(W, o1 & 0x07070707u); break;
        case 2: place_slot<2>(W, o0 & 0x07070707u); place_slot<6>(W, o1 & 0x07070707u); break;
        default: place_slot<3>(W, o0 & 0x07070707u); place_slot<7>(W, o1 & 0x07070707u); break;
      }
      if (any_raw) {  // offset bits 4..7, token 4 t4 + k at bits 4k of unit 1 + t4
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          const uint32_t t = ((gi ? o1 : o0) >> 4) & 0x0F0F0F0Fu;
          const uint32_t u = t | (t >> 4);
          units[gi][1 + t4] = (u & 0xFFu) | ((u >> 8) & 0xFF00u);
        }
      }
    }
    units[0][0] = pl & 0xFFFFu;
    units[1][0] = pl >> 16;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int q = q0 + gi;
      if (PI.mode[gi] >= 1) atomicOr(&tagw[q >> 5], 1u << (q & 31));
      if (PI.mode[gi] == 2) atomicOr(&tagw[G.PW + (q >> 5)], 1u << (q & 31));
    }
  }

  if (tid == 0) sh_slot = pop_slot(B, is_raw, sh_modes, 2 * total, &sh_raw);
  __syncthreads();
  const int slot = sh_slot, raw = sh_raw;
  if (slot < 0) {
    if (tid == 0) B.table[entry_idx] = kUnallocated;
    return;
  }

  if (raw) {
    store_raw_tile(G, B, slot, kv, tile, entry_idx);
    return;
  }

  uint8_t* dst = B.comp_pool + (size_t)slot * G.stride;
  int P = my_before;
  if (has_pair && FMT == 0) {
    uint16_t* esc16 = reinterpret_cast<uint16_t*>(dst + G.esc_off);
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int np = mode_planes(G, PI.mode[gi]);
      for (int p = 0; p < np; ++p) esc16[P + p] = (uint16_t)units[gi][p];
      P += np;
    }
    uint32_t* code = reinterpret_cast<uint32_t*>(dst + G.code_off + 12 * pr);
    code[0] = W[0];
    code[1] = W[1];
    code[2] = W[2];
    uint4* smd = reinterpret_cast<uint4*>(dst + G.sm_off + 32 * pr);
    smd[0] = make_uint4(smb[0], smb[1], smb[2], smb[3]);
    smd[1] = make_uint4(smb[4], smb[5], smb[6], smb[7]);
  } else if (has_pair) {  // FP8: element by element
    uint32_t W[3] = {0u, 0u, 0u};
    uint32_t SM[4] = {0u, 0u, 0u, 0u};  // E5M2: 3 words in the CODE unit layout; E4M3: 4 words of nibbles
    uint32_t smb[8];                      // BF16: the 8 SM words (one byte per element)
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int q = q0 + gi;
      const uint32_t base = PI.base[gi];
      // escape units: [0] = plane of offset bit 3; a raw BF16 group adds [1..4] = 4-bit fields
      // of offset bits 4..7 (token tau at bits 4*(tau%4) of unit 1 + tau/4), a raw E5M2 group
      // adds [1] = plane of offset bit 4
      uint32_t units[5] = {0u, 0u, 0u, 0u, 0u};
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        uint32_t cf = 0, sf = 0;  // this slot's code / sign-mantissa fields, one per byte lane
#pragma unroll
        for (int lk = 0; lk < 4; ++lk) {
          const int tau = 4 * t4 + lk;
          const uint32_t x = (pw[tau] >> (16 * gi)) & 0xFFFFu;
          const uint32_t o = ((x >> EF::MB) & ((1u << EF::F) - 1u)) - base;
          const uint32_t f = ((x >> (EF::MB + EF::F)) << EF::MB) | (x & ((1u << EF::MB) - 1u));
          cf |= (o & 7u) << (8 * lk);
          sf |= f << (8 * lk);
          units[0] |= ((o >> 3) & 1u) << tau;
          if constexpr (EF::F == 8) units[1 + t4] |= ((o >> 4) & 0xFu) << (4 * lk);
          if constexpr (EF::F == 5) units[1] |= ((o >> 4) & 1u) << tau;
        }
        const int sl = 4 * gi + t4;  // slot of the unit (elements 4*sl .. 4*sl+3)
        switch (sl) {
          case 0: place_slot<0>(W, cf); if constexpr (FMT == 1) place_slot<0>(SM, sf); break;
          case 1: place_slot<1>(W, cf); if constexpr (FMT == 1) place_slot<1>(SM, sf); break;
          case 2: place_slot<2>(W, cf); if constexpr (FMT == 1) place_slot<2>(SM, sf); break;
          case 3: place_slot<3>(W, cf); if constexpr (FMT == 1) place_slot<3>(SM, sf); break;
          case 4: place_slot<4>(W, cf); if constexpr (FMT == 1) place_slot<4>(SM, sf); break;
          case 5: place_slot<5>(W, cf); if constexpr (FMT == 1) place_slot<5>(SM, sf); break;
          case 6: place_slot<6>(W, cf); if constexpr (FMT == 1) place_slot<6>(SM, sf); break;
          default: place_slot<7>(W, cf); if constexpr (FMT == 1) place_slot<7>(SM, sf); break;
        }
        if constexpr (FMT == 0) smb[sl] = sf;
        if constexpr (FMT == 2) {  // four nibbles: element 4sl + lk at bits 4*(4*(sl%2) + lk) of word sl/2
          const uint32_t t = sf | (sf >> 4);
          const uint32_t nib16 = (t & 0xFFu) | ((t >> 8) & 0xFF00u);
          SM[sl >> 1] |= nib16 << (16 * (sl & 1));
        }
      }
      const int np = mode_planes(G, PI.mode[gi]);
      uint16_t* esc16 = reinterpret_cast<uint16_t*>(dst + G.esc_off);
      for (int p = 0; p < np; ++p) esc16[P + p] = (uint16_t)units[p];
      P += np;
      if (PI.mode[gi] >= 1) atomicOr(&tagw[q >> 5], 1u << (q & 31));
      if (PI.mode[gi] == 2) atomicOr(&tagw[G.PW + (q >> 5)], 1u << (q & 31));
    }
    uint32_t* code = reinterpret_cast<uint32_t*>(dst + G.code_off + 12 * pr);
    code[0] = W[0];
    code[1] = W[1];
    code[2] = W[2];
    uint32_t* smd = reinterpret_cast<uint32_t*>(dst + G.sm_off + G.sm_pair * pr);
    if constexpr (FMT == 0) {
      *reinterpret_cast<uint4*>(smd) = make_uint4(smb[0], smb[1], smb[2], smb[3]);
      *reinterpret_cast<uint4*>(smd + 4) = make_uint4(smb[4], smb[5], smb[6], smb[7]);
    } else if constexpr (FMT == 1) {
      smd[0] = SM[0]; smd[1] = SM[1]; smd[2] = SM[2];
    } else {
      *reinterpret_cast<uint4*>(smd) = make_uint4(SM[0], SM[1], SM[2], SM[3]);
    }
  }
  // zero the unused escape bytes [2*total, esc_cap)
  {
    const int used = 2 * total;
    if ((used & 3) && tid == 0) reinterpret_cast<uint16_t*>(dst + G.esc_off)[total] = 0;
    const int w0 = (used + 3) >> 2;
    uint32_t* esc32 = reinterpret_cast<uint32_t*>(dst + G.esc_off);
    for (int i = w0 + tid; i < (G.esc_cap >> 2); i += kThreads) esc32[i] = 0;
  }
  __syncthreads();
  for (int i = tid; i < 2 * G.PW; i += kThreads) reinterpret_cast<uint32_t*>(dst + G.tag_off)[i] = tagw[i];
  if (tid == 0) {
    const uint32_t units = (uint32_t)((2 * total + 15) >> 4);
    B.table[entry_idx] = comp_entry((uint32_t)slot, units, G.cur_ver);
  }
}

// BF16 tiles with 8-token groups (FORMAT v1): one thread per CODE unit (channels c0 .. c0+3 of one
// token group, 8 tokens each, read from LDS as 8 words of channels c0, c0+1 and 8 of c0+2, c0+3),
// fields packed four tokens per word as in encode_kernel.  Escape units are single bytes: an 8-bit
// plane per escaped group, then four bytes of 4-bit fields for a raw group.
__global__ void __launch_bounds__(kThreads) encode_g8_kernel(Geo G, DevBufs B, SeqList S, const void* __restrict__ kin,
                                                             const void* __restrict__ vin, int n_tok) {
  extern __shared__ uint4 smem4[];                                      // 16-byte aligned
  uint32_t* smem = reinterpret_cast<uint32_t*>(smem4);
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);                  // [T][D] logical
  uint32_t* tagw = smem + (G.raw_elems / 2);                            // [2][PW]
  __shared__ int red[8];
  __shared__ int sh_slot, sh_raw;
  __shared__ unsigned long long sh_modes[4];

  const int si = blockIdx.y, kv = blockIdx.z / G.Hkv, h = blockIdx.z % G.Hkv;
  const int seq = S.ids[si], L0 = S.lens[si];
  const int first_blk = L0 / G.T, last_full = (L0 + n_tok) / G.T;
  const int b = first_blk + blockIdx.x;
  if (b >= last_full) return;
  const int tid = threadIdx.x, D = G.D;
  const uint8_t* tail = reinterpret_cast<const uint8_t*>(B.tail) + tail_offset(G, seq, kv, h) * 2;
  gather_block<2>(G, tail, kv ? vin : kin, si, h, kv, b, L0, n_tok, first_blk * G.T, tile);
  for (int i = tid; i < 2 * G.PW; i += kThreads) tagw[i] = 0;
  if (tid < 4) sh_modes[tid] = 0;
  __syncthreads();

  const size_t entry_idx = table_index(G, seq, b, kv, h);
  const uint8_t* b3 = bases_of(G, B.bases, G.cur_ver, 3, kv, h);  // blocks are encoded with the current bases
  const uint8_t* b4 = bases_of(G, B.bases, G.cur_ver, 4, kv, h);
  // one CODE unit per thread (T * D / 32 <= 256 units for T <= 64, D <= 128)
  const int u = tid, q0 = 4 * u, tg = q0 / D, c0 = q0 % D;
  const bool has_unit = u < G.raw_elems / 32;
  uint32_t A[8], Bw[8];  // token tau: channels c0 (low half), c0+1 / c0+2 (low half), c0+3
#pragma unroll
  for (int tau = 0; tau < 8; ++tau) {
    const uint2 x = has_unit ? *reinterpret_cast<const uint2*>(tile + (tg * 8 + tau) * D + c0) : make_uint2(0u, 0u);
    A[tau] = x.x;
    Bw[tau] = x.y;
  }
  int mode[4] = {0, 0, 0, 0};
  uint32_t base[4] = {0u, 0u, 0u, 0u};
  int packed = 0;  // escape bytes of the unit (bits 0..15), escaped groups (16..)
  if (G.compressed && has_unit) {
    u16x2 loA = {0xFFFFu, 0xFFFFu}, hiA = {0u, 0u}, loB = {0xFFFFu, 0xFFFFu}, hiB = {0u, 0u};
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
      const u16x2 ea = __builtin_bit_cast(u16x2, (A[tau] >> 7) & 0x00FF00FFu);
      const u16x2 eb = __builtin_bit_cast(u16x2, (Bw[tau] >> 7) & 0x00FF00FFu);
      loA = __builtin_elementwise_min(loA, ea);
      hiA = __builtin_elementwise_max(hiA, ea);
      loB = __builtin_elementwise_min(loB, eb);
      hiB = __builtin_elementwise_max(hiB, eb);
    }
    const uint32_t mn[4] = {loA.x, loA.y, loB.x, loB.y}, mx[4] = {hiA.x, hiA.y, hiB.x, hiB.y};
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      mode[gi] = choose_mode(mn[gi], mx[gi], b3[c0 + gi], b4[c0 + gi], true);
      base[gi] = mode[gi] == 0 ? b3[c0 + gi] : (mode[gi] == 1 ? b4[c0 + gi] : 0u);
      packed += mode[gi] == 0 ? 0 : (mode[gi] == 1 ? 1 + (1 << 16) : 5 + (1 << 16));
    }
  }
  int all = 0;
  const int my_before = block_exclusive_scan(packed, red, &all) & 0xFFFF;
  const int used = all & 0xFFFF, n_esc = all >> 16;  // escape bytes; wide + raw groups
  const int is_raw = (!G.compressed || used > G.esc_cap) ? 1 : 0;
  if (tid == 0 && G.compressed) {
    const int rawg = (used - n_esc) / 4;  // a raw group's escape is 5 bytes, a wide group's 1
    sh_modes[0] = (unsigned long long)(G.NG - n_esc);
    sh_modes[1] = (unsigned long long)(n_esc - rawg);
    sh_modes[2] = (unsigned long long)rawg;
  }

  // the unit's fields, packed in registers while thread 0 pops the slot
  uint32_t W[3] = {0u, 0u, 0u}, smb[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u}, plane[4] = {0u, 0u, 0u, 0u};
  uint32_t hin[4] = {0u, 0u, 0u, 0u};  // raw groups: token tau's offset bits 4..7 at bits 4 tau
  if (has_unit && !is_raw) {
    const uint32_t base2A = base[0] | (base[1] << 16), base2B = base[2] | (base[3] << 16);
    const bool any_raw = (mode[0] | mode[1] | mode[2] | mode[3]) & 2;
    uint32_t plA = 0, plB = 0;  // offset bit 3 of token tau at bit tau of each 16-bit half
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      uint32_t exA[4], exB[4], sxA[4], sxB[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t wa = A[4 * qq + k], wb = Bw[4 * qq + k];
        exA[k] = wa >> 7;
        exB[k] = wb >> 7;
        sxA[k] = bfi(0x00800080u, wa >> 8, wa);
        sxB[k] = bfi(0x00800080u, wb >> 8, wb);
        plA |= ((((exA[k] & 0x00FF00FFu) - base2A) >> 3) & 0x00010001u) << (4 * qq + k);
        plB |= ((((exB[k] & 0x00FF00FFu) - base2B) >> 3) & 0x00010001u) << (4 * qq + k);
      }
      const uint32_t aA = perm_b32(exA[1], exA[0], 0x06020400u), bA = perm_b32(exA[3], exA[2], 0x06020400u);
      const uint32_t aB = perm_b32(exB[1], exB[0], 0x06020400u), bB = perm_b32(exB[3], exB[2], 0x06020400u);
      const uint32_t o[4] = {perm_b32(bA, aA, 0x05040100u) - base[0] * 0x01010101u,
                             perm_b32(bA, aA, 0x07060302u) - base[1] * 0x01010101u,
                             perm_b32(bB, aB, 0x05040100u) - base[2] * 0x01010101u,
                             perm_b32(bB, aB, 0x07060302u) - base[3] * 0x01010101u};
      const uint32_t sA = perm_b32(sxA[1], sxA[0], 0x06020400u), tA = perm_b32(sxA[3], sxA[2], 0x06020400u);
      const uint32_t sB = perm_b32(sxB[1], sxB[0], 0x06020400u), tB = perm_b32(sxB[3], sxB[2], 0x06020400u);
      smb[0 + qq] = perm_b32(tA, sA, 0x05040100u);  // element 8 gi + 4 qq + k: word 2 gi + qq
      smb[2 + qq] = perm_b32(tA, sA, 0x07060302u);
      smb[4 + qq] = perm_b32(tB, sB, 0x05040100u);
      smb[6 + qq] = perm_b32(tB, sB, 0x07060302u);
      if (qq == 0) {
        place_slot<0>(W, o[0] & 0x07070707u); place_slot<2>(W, o[1] & 0x07070707u);
        place_slot<4>(W, o[2] & 0x07070707u); place_slot<6>(W, o[3] & 0x07070707u);
      } else {
        place_slot<1>(W, o[0] & 0x07070707u); place_slot<3>(W, o[1] & 0x07070707u);
        place_slot<5>(W, o[2] & 0x07070707u); place_slot<7>(W, o[3] & 0x07070707u);
      }
      if (any_raw) {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const uint32_t t = (o[gi] >> 4) & 0x0F0F0F0Fu;
          const uint32_t v = t | (t >> 4);
          hin[gi] |= ((v & 0xFFu) | ((v >> 8) & 0xFF00u)) << (16 * qq);
        }
      }
    }
    plane[0] = plA & 0xFFu;
    plane[1] = (plA >> 16) & 0xFFu;
    plane[2] = plB & 0xFFu;
    plane[3] = (plB >> 16) & 0xFFu;
    uint32_t e4 = 0, r4 = 0;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      e4 |= (mode[gi] >= 1 ? 1u : 0u) << gi;
      r4 |= (mode[gi] == 2 ? 1u : 0u) << gi;
    }
    if (e4) atomicOr(&tagw[q0 >> 5], e4 << (q0 & 31));
    if (r4) atomicOr(&tagw[G.PW + (q0 >> 5)], r4 << (q0 & 31));
  }

  if (tid == 0) sh_slot = pop_slot(B, is_raw, sh_modes, used, &sh_raw);
  __syncthreads();
  const int slot = sh_slot, raw = sh_raw;
  if (slot < 0) {
    if (tid == 0) B.table[entry_idx] = kUnallocated;
    return;
  }
  if (raw) {
    store_raw_tile(G, B, slot, kv, tile, entry_idx);
    return;
  }
  uint8_t* dst = B.comp_pool + (size_t)slot * G.stride;
  if (has_unit) {
    uint8_t* esc = dst + G.esc_off;
    int P = my_before;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      if (mode[gi] >= 1) esc[P++] = (uint8_t)plane[gi];
      if (mode[gi] == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) esc[P + k] = (uint8_t)(hin[gi] >> (8 * k));
        P += 4;
      }
    }
    uint32_t* code = reinterpret_cast<uint32_t*>(dst + G.code_off + 12 * u);
    code[0] = W[0];
    code[1] = W[1];
    code[2] = W[2];
    uint4* smd = reinterpret_cast<uint4*>(dst + G.sm_off + 32 * u);
    smd[0] = make_uint4(smb[0], smb[1], smb[2], smb[3]);
    smd[1] = make_uint4(smb[4], smb[5], smb[6], smb[7]);
  }
  // zero the unused escape bytes [used, esc_cap)
  {
    uint8_t* esc = dst + G.esc_off;
    if (tid < ((4 - (used & 3)) & 3)) esc[used + tid] = 0;
    const int w0 = (used + 3) >> 2;
    uint32_t* esc32 = reinterpret_cast<uint32_t*>(esc);
    for (int i = w0 + tid; i < (G.esc_cap >> 2); i += kThreads) esc32[i] = 0;
  }
  __syncthreads();
  for (int i = tid; i < 2 * G.PW; i += kThreads) reinterpret_cast<uint32_t*>(dst + G.tag_off)[i] = tagw[i];
  if (tid == 0) B.table[entry_idx] = comp_entry((uint32_t)slot, (uint32_t)((used + 15) >> 4), G.cur_ver);
}

// Any group size (8-token groups; 16 works too): the slot is assembled in LDS by OR-ing every
// field into zeroed words at the bit positions FORMAT v1 gives it, then copied out whole.
// One 256-thread workgroup per new tile, as encode_kernel.
// ORs the low nbits (<= 32) of val into an LSB-first bit stream of LDS words at bit bp.
__device__ __forceinline__ void or_bits(uint32_t* words, int bp, uint32_t val, int nbits) {
  const int w = bp >> 5, sh = bp & 31;
  atomicOr(&words[w], val << sh);
  if (sh + nbits > 32) atomicOr(&words[w + 1], val >> (32 - sh));
}

template <int FMT>
__global__ void __launch_bounds__(kThreads) encode_any_kernel(Geo G, DevBufs B, SeqList S, const void* __restrict__ kin,
                                                              const void* __restrict__ vin, int n_tok) {
  using EF = EncFmt<FMT>;
  extern __shared__ uint32_t smem[];
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);                        // [T][D] logical
  uint32_t* slotw = smem + G.raw_elems / 2;                                   // the slot, stride bytes
  uint16_t* gP = reinterpret_cast<uint16_t*>(slotw + G.stride / 4);           // [NG] escape units before q
  uint8_t* gm = reinterpret_cast<uint8_t*>(gP + G.NG);                        // [NG] group modes
  __shared__ int red[8];
  __shared__ int sh_slot, sh_raw;
  __shared__ unsigned long long sh_modes[4];

  const int si = blockIdx.y, kv = blockIdx.z / G.Hkv, h = blockIdx.z % G.Hkv;
  const int seq = S.ids[si], L0 = S.lens[si];
  const int first_blk = L0 / G.T, last_full = (L0 + n_tok) / G.T;
  const int b = first_blk + blockIdx.x;
  if (b >= last_full) return;
  const int tid = threadIdx.x, D = G.D, GT = G.GT, NG = G.NG;
  const uint8_t* tail = reinterpret_cast<const uint8_t*>(B.tail) + tail_offset(G, seq, kv, h) * G.EB;
  gather_block<EF::EB>(G, tail, kv ? vin : kin, si, h, kv, b, L0, n_tok, first_blk * G.T, tile);
  for (int i = tid; i < G.stride / 4; i += kThreads) slotw[i] = 0u;
  __syncthreads();

  const uint8_t* b3 = bases_of(G, B.bases, G.cur_ver, 3, kv, h);  // blocks are encoded with the current bases
  const uint8_t* b4 = bases_of(G, B.bases, G.cur_ver, 4, kv, h);
  // modes; each thread takes consecutive groups, so a block scan gives every group's escape offset
  const int per = (NG + kThreads - 1) / kThreads, q0 = min(NG, tid * per), q1 = min(NG, q0 + per);
  int units = 0, cnt[3] = {0, 0, 0};
  if (G.compressed) {
    for (int q = q0; q < q1; ++q) {
      const int tg = q / D, c = q % D;
      uint32_t mn = 255, mx = 0;
      for (int tau = 0; tau < GT; ++tau) {
        const uint32_t e = exp_of(G, tile[(tg * GT + tau) * D + c]);
        mn = min(mn, e);
        mx = max(mx, e);
      }
      const int m = choose_mode(mn, mx, b3[c], b4[c], EF::F > 4);
      gm[q] = (uint8_t)m;
      cnt[m]++;
      units += mode_planes(G, m);
    }
  }
  int total;
  int P = block_exclusive_scan(units, red, &total);
  for (int q = q0; q < q1 && G.compressed; ++q) {
    gP[q] = (uint16_t)P;
    P += mode_planes(G, gm[q]);
  }
  const int esc_bytes = (total * GT + 7) / 8;
  for (int m = 0; m < 3; ++m) {
    const int sm = block_sum(cnt[m], red);
    if (tid == 0) sh_modes[m] = (unsigned long long)sm;
  }
  if (tid == 0) sh_modes[3] = 0;
  if (tid == 0) sh_slot = pop_slot(B, (!G.compressed || esc_bytes > G.esc_cap) ? 1 : 0, sh_modes, esc_bytes, &sh_raw);
  __syncthreads();
  const int slot = sh_slot, raw = sh_raw;
  const size_t entry_idx = table_index(G, seq, b, kv, h);
  if (slot < 0) {
    if (tid == 0) B.table[entry_idx] = kUnallocated;
    return;
  }
  if (raw) {
    store_raw_tile(G, B, slot, kv, tile, entry_idx);
    return;
  }

  // one element quad per step: elements n0 .. n0+3 = tokens tau0 .. tau0+3 of group q
  const int esc_bit0 = 8 * G.esc_off;
  for (int k = tid; k < G.raw_elems / 4; k += kThreads) {
    const int n0 = 4 * k, q = n0 / GT, tau0 = n0 % GT, tg = q / D, c = q % D;
    const int m = gm[q];
    const uint32_t base = m == 0 ? b3[c] : (m == 1 ? b4[c] : 0u);
    uint32_t cf = 0, sf = 0, e3 = 0, hi = 0;
#pragma unroll
    for (int lk = 0; lk < 4; ++lk) {
      const uint32_t x = tile[(tg * GT + tau0 + lk) * D + c];
      const uint32_t o = exp_of(G, x) - base;
      cf |= (o & 7u) << (8 * lk);
      sf |= sm_of(G, x) << (8 * lk);
      e3 |= ((o >> 3) & 1u) << lk;
      if constexpr (EF::F == 8) hi |= ((o >> 4) & 0xFu) << (4 * lk);
      if constexpr (EF::F == 5) hi |= ((o >> 4) & 1u) << lk;
    }
    // CODE (and the E5M2 SM fields): slot s of 32-element unit u
    const int u = n0 >> 5, sl = (n0 & 31) >> 2;
    uint32_t W[3] = {0u, 0u, 0u}, SMW[3] = {0u, 0u, 0u};
    switch (sl) {
      case 0: place_slot<0>(W, cf); if constexpr (FMT == 1) place_slot<0>(SMW, sf); break;
      case 1: place_slot<1>(W, cf); if constexpr (FMT == 1) place_slot<1>(SMW, sf); break;
      case 2: place_slot<2>(W, cf); if constexpr (FMT == 1) place_slot<2>(SMW, sf); break;
      case 3: place_slot<3>(W, cf); if constexpr (FMT == 1) place_slot<3>(SMW, sf); break;
      case 4: place_slot<4>(W, cf); if constexpr (FMT == 1) place_slot<4>(SMW, sf); break;
      case 5: place_slot<5>(W, cf); if constexpr (FMT == 1) place_slot<5>(SMW, sf); break;
      case 6: place_slot<6>(W, cf); if constexpr (FMT == 1) place_slot<6>(SMW, sf); break;
      default: place_slot<7>(W, cf); if constexpr (FMT == 1) place_slot<7>(SMW, sf); break;
    }
    uint32_t* cw = slotw + (G.code_off + 12 * u) / 4;
#pragma unroll
    for (int w = 0; w < 3; ++w)
      if (W[w]) atomicOr(&cw[w], W[w]);
    if constexpr (FMT == 0) {
      slotw[(G.sm_off + n0) / 4] = sf;  // one byte per element: this quad owns the word
    } else if constexpr (FMT == 1) {
      uint32_t* sw = slotw + (G.sm_off + 12 * u) / 4;
#pragma unroll
      for (int w = 0; w < 3; ++w)
        if (SMW[w]) atomicOr(&sw[w], SMW[w]);
    } else {  // 4-bit fields, element n at bits 4n..4n+3
      const uint32_t t2 = sf | (sf >> 4);
      const uint32_t nib16 = (t2 & 0xFFu) | ((t2 >> 8) & 0xFF00u);
      atomicOr(&slotw[G.sm_off / 4 + (n0 >> 3)], nib16 << (16 * (k & 1)));
    }
    if (m >= 1) {  // escape planes: bit 3 of the offsets, then the raw group's high bits
      const int P0 = gP[q];
      or_bits(slotw, esc_bit0 + P0 * GT + tau0, e3, 4);
      if (m == 2) {
        if constexpr (EF::F == 8) or_bits(slotw, esc_bit0 + (P0 + 1) * GT + 4 * tau0, hi, 16);
        else if constexpr (EF::F == 5) or_bits(slotw, esc_bit0 + (P0 + 1) * GT + tau0, hi, 4);
      }
    }
    if (tau0 == 0) {  // the group's tag bits
      if (m >= 1) atomicOr(&slotw[G.tag_off / 4 + (q >> 5)], 1u << (q & 31));
      if (m == 2) atomicOr(&slotw[G.tag_off / 4 + G.PW + (q >> 5)], 1u << (q & 31));
    }
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(B.comp_pool + (size_t)slot * G.stride);
  const uint4* src = reinterpret_cast<const uint4*>(slotw);
  for (int i = tid; i < G.stride / 16; i += kThreads) dst[i] = src[i];
  if (tid == 0) B.table[entry_idx] = comp_entry((uint32_t)slot, (uint32_t)((esc_bytes + 15) >> 4), G.cur_ver);
}

// FORMAT v2 (the nested precision modes of GAAC page §4.7.2; BF16): one 256-thread workgroup per
// new tile, as encode_any_kernel.  Each group takes the first mode of the set whose calibrated
// window holds its exponents; a block scan of the groups' code bits gives every group's offset
// in the CODES stream; the slot is assembled in LDS (TAG planes = bits 0 and 1 of the mode
// index, SM bytes, the codes of four tokens at a time OR-ed in at their stream position), then
// copied out whole.  A tile whose codes exceed the capacity is stored raw.
__device__ __forceinline__ uint32_t v2_base(const Geo& G, int k, const uint8_t* b2, const uint8_t* b3,
                                            const uint8_t* b4, int c) {
  const int w = G.mw[k];
  return k == G.n_modes - 1 ? 0u : (w == 2 ? b2[c] : (w == 3 ? b3[c] : b4[c]));
}

__global__ void __launch_bounds__(kThreads) encode_v2_kernel(Geo G, DevBufs B, SeqList S, const void* __restrict__ kin,
                                                             const void* __restrict__ vin, int n_tok) {
  extern __shared__ uint32_t smem[];
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);                  // [T][D] logical
  uint32_t* slotw = smem + G.raw_elems / 2;                             // the slot, stride bytes
  uint32_t* gO = slotw + G.stride / 4;                                  // [NG] code bit offset of q
  uint8_t* gk = reinterpret_cast<uint8_t*>(gO + G.NG);                  // [NG] mode index of q
  __shared__ int red[8];
  __shared__ int sh_slot, sh_raw;
  __shared__ unsigned long long sh_modes[4];

  const int si = blockIdx.y, kv = blockIdx.z / G.Hkv, h = blockIdx.z % G.Hkv;
  const int seq = S.ids[si], L0 = S.lens[si];
  const int first_blk = L0 / G.T, last_full = (L0 + n_tok) / G.T;
  const int b = first_blk + blockIdx.x;
  if (b >= last_full) return;
  const int tid = threadIdx.x, D = G.D, GT = G.GT, NG = G.NG;
  const uint8_t* tail = reinterpret_cast<const uint8_t*>(B.tail) + tail_offset(G, seq, kv, h) * 2;
  gather_block<2>(G, tail, kv ? vin : kin, si, h, kv, b, L0, n_tok, first_blk * G.T, tile);
  for (int i = tid; i < G.stride / 4; i += kThreads) slotw[i] = 0u;
  __syncthreads();

  const uint8_t* b3 = bases_of(G, B.bases, G.cur_ver, 3, kv, h);  // blocks are encoded with the current bases
  const uint8_t* b4 = bases_of(G, B.bases, G.cur_ver, 4, kv, h);
  const uint8_t* b2 = bases_of(G, B.bases, G.cur_ver, 2, kv, h);  // mode set 1 only
  const int per = (NG + kThreads - 1) / kThreads, q0 = min(NG, tid * per), q1 = min(NG, q0 + per);
  int bits = 0, cnt[4] = {0, 0, 0, 0};
  if (G.compressed) {
    for (int q = q0; q < q1; ++q) {
      const int tg = q / D, c = q % D;
      uint32_t mn = 255, mx = 0;
      for (int tau = 0; tau < GT; ++tau) {
        const uint32_t e = exp_of(G, tile[(tg * GT + tau) * D + c]);
        mn = min(mn, e);
        mx = max(mx, e);
      }
      int k = G.n_modes - 1;
      for (int j = 0; j < G.n_modes - 1; ++j) {
        const uint32_t base = v2_base(G, j, b2, b3, b4, c);
        if (base <= mn && mx <= base + (1u << G.mw[j]) - 1u) { k = j; break; }
      }
      gk[q] = (uint8_t)k;
      cnt[k]++;
      bits += GT * G.mw[k];
    }
  }
  int total;
  int O = block_exclusive_scan(bits, red, &total);
  for (int q = q0; q < q1 && G.compressed; ++q) {
    gO[q] = (uint32_t)O;
    O += GT * G.mw[gk[q]];
  }
  const int used = (total + 7) / 8;
  for (int m = 0; m < 4; ++m) {
    const int sm = block_sum(cnt[m], red);
    if (tid == 0) sh_modes[m] = (unsigned long long)sm;
  }
  if (tid == 0) sh_slot = pop_slot(B, (!G.compressed || used > G.code_cap) ? 1 : 0, sh_modes, used, &sh_raw);
  __syncthreads();
  const int slot = sh_slot, raw = sh_raw;
  const size_t entry_idx = table_index(G, seq, b, kv, h);
  if (slot < 0) {
    if (tid == 0) B.table[entry_idx] = kUnallocated;
    return;
  }
  if (raw) {
    store_raw_tile(G, B, slot, kv, tile, entry_idx);
    return;
  }
  // four consecutive tokens of one group per step: their codes are 4w consecutive stream bits
  const int code_bit0 = 8 * G.code_off;
  for (int k4 = tid; k4 < G.raw_elems / 4; k4 += kThreads) {
    const int n0 = 4 * k4, q = n0 / GT, tau0 = n0 % GT, tg = q / D, c = q % D;
    const int k = gk[q], w = G.mw[k];
    const uint32_t base = v2_base(G, k, b2, b3, b4, c);
    uint32_t cf = 0, sf = 0;
#pragma unroll
    for (int lk = 0; lk < 4; ++lk) {
      const uint32_t x = tile[(tg * GT + tau0 + lk) * D + c];
      cf |= (exp_of(G, x) - base) << (w * lk);
      sf |= sm_of(G, x) << (8 * lk);
    }
    or_bits(slotw, code_bit0 + (int)gO[q] + tau0 * w, cf, 4 * w);
    slotw[(G.sm_off + n0) / 4] = sf;
    if (tau0 == 0) {
      if (k & 1) atomicOr(&slotw[G.tag_off / 4 + (q >> 5)], 1u << (q & 31));
      if (k & 2) atomicOr(&slotw[G.tag_off / 4 + G.PW + (q >> 5)], 1u << (q & 31));
    }
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(B.comp_pool + (size_t)slot * G.stride);
  const uint4* src = reinterpret_cast<const uint4*>(slotw);
  for (int i = tid; i < G.stride / 16; i += kThreads) dst[i] = src[i];
  if (tid == 0) B.table[entry_idx] = comp_entry((uint32_t)slot, 0u, G.cur_ver);
}

// Storage statistics of finished tiles from their table entries and stored tag planes (the
// positional-drift study of GAAC page App. C reads these per segment): one thread per tile;
// out[i][7] = {state (0 compressed, 1 raw, -1 unallocated), bytes (FORMAT v1: the escape bytes
// the tags call for; FORMAT v2: the code bytes), groups per mode index [4], base version (-1
// unless compressed)}.  A raw bit without its escape bit (FORMAT v1, corrupt) counts as raw.
__global__ void tile_stats_kernel(Geo G, DevBufs B, int seq, int first, int n, int32_t* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * 2 * G.Hkv) return;
  const int bi = i / (2 * G.Hkv), kv = (i / G.Hkv) % 2, h = i % G.Hkv;
  const uint32_t e = B.table[table_index(G, seq, first + bi, kv, h)];
  int32_t* o = out + (size_t)i * 7;
  int c[4] = {0, 0, 0, 0}, state = 0, ver = -1;
  long bits = 0;
  if (e == kUnallocated) {
    state = -1;
  } else if (e & kRawTile) {
    state = 1;
  } else {
    ver = entry_version(e);
    const uint32_t* tag0 = reinterpret_cast<const uint32_t*>(B.comp_pool + (size_t)entry_slot(e) * G.stride + G.tag_off);
    const uint32_t* tag1 = tag0 + G.PW;
    for (int w = 0; w < G.PW; ++w) {
      const uint32_t valid = (w == G.PW - 1 && (G.NG & 31)) ? ((1u << (G.NG & 31)) - 1u) : 0xFFFFFFFFu;
      const uint32_t a = tag0[w] & valid, b = tag1[w] & valid;
      if (G.mode_set == 0) {  // planes E (mode >= wide) and R (raw)
        c[2] += __popc(b);
        c[1] += __popc(a & ~b);
      } else {                // bits 0 and 1 of the mode index
        c[1] += __popc(a & ~b);
        c[2] += __popc(~a & b);
        c[3] += __popc(a & b);
      }
    }
    c[0] = G.NG - c[1] - c[2] - c[3];
    if (G.mode_set == 0) bits = (long)G.GT * (c[1] + (long)(G.F - 3) * c[2]);
    else for (int k = 0; k < G.n_modes; ++k) bits += (long)G.GT * G.mw[k] * c[k];
  }
  o[0] = state;
  o[1] = (int32_t)((bits + 7) / 8);
  for (int k = 0; k < 4; ++k) o[2 + k] = c[k];
  o[6] = ver;
}

// Exponent concentration (GAAC page §3.1: most exponents of a head-channel lie in a few
// consecutive values): one block per (channel, kv-head), the largest number of the n tokens'
// exponents inside any window of w consecutive exponent values.  x: [n][Hkv][D] elements.
// Block b takes head b % Hkv: workgroups are dealt to the eight XCDs round robin, so with 8
// (or a divisor of 8) heads all channels of a head run on one XCD and share its L2 copy of the
// head's token rows instead of every XCD fetching every row.
__global__ void coverage_kernel(Geo G, const void* __restrict__ x, int n, int w, int32_t* __restrict__ out) {
  __shared__ int hist[256];
  __shared__ int red[8];
  const int c = blockIdx.x / G.Hkv, h = blockIdx.x % G.Hkv, tid = threadIdx.x;
  hist[tid] = 0;
  __syncthreads();
  for (int t = tid; t < n; t += kThreads) atomicAdd(&hist[exp_of(G, elem_at(x, ((size_t)t * G.Hkv + h) * G.D + c, G.EB))], 1);
  __syncthreads();
  const int nb = (1 << G.F) - w + 1;
  int cov = 0;
  if (tid < nb)
    for (int e = tid; e < tid + w; ++e) cov += hist[e];
  const int best = block_max(cov, red);
  if (tid == 0) out[(size_t)h * G.D + c] = best;
}

// Streaming-read probe: one 64-lane wave per workgroup (the split attention kernels' shape);
// wave w reads n16 16-byte words from src + w * n16 with eight 16-byte loads per lane per batch,
// the next batch in flight while the current one is folded into a checksum, and writes one
// checksum word per lane (so no load is dead).  n16 is a multiple of 512.
__global__ void __launch_bounds__(64) read_probe_kernel(const uint4* __restrict__ src, size_t n16,
                                                        uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  const uint4* p = src + (size_t)blockIdx.x * n16 + threadIdx.x;
  const size_t nb = n16 / (64 * U);
  uint4 a[U], b[U];
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) a[u] = p[64 * u];
  for (size_t i = 0; i < nb; ++i) {
    if (i + 1 < nb) {
#pragma unroll
      for (int u = 0; u < U; ++u) b[u] = p[(i + 1) * 64 * U + 64 * u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = acc * 31u + (a[u].x ^ a[u].y ^ a[u].z ^ a[u].w);
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = b[u];
  }
  sink[(size_t)blockIdx.x * 64 + threadIdx.x] = acc;
}

// Writes the appended tokens that do not complete a block into the sequence's tail.
__global__ void tail_kernel(Geo G, DevBufs B, SeqList S, const void* __restrict__ kin, const void* __restrict__ vin,
                            int n_tok) {
  const int si = blockIdx.x, kv = blockIdx.y / G.Hkv, h = blockIdx.y % G.Hkv;
  const int seq = S.ids[si], L0 = S.lens[si];
  const int new_full = (L0 + n_tok) / G.T;
  const int p0 = max(L0, new_full * G.T), p1 = L0 + n_tok;
  const int D = G.D, T = G.T;
  const void* in = kv ? vin : kin;
  uint8_t* tail = reinterpret_cast<uint8_t*>(B.tail) + tail_offset(G, seq, kv, h) * G.EB;
  for (int i = threadIdx.x; i < (p1 - p0) * D; i += blockDim.x) {
    const int p = p0 + i / D, c = i % D, tt = p - new_full * T;
    const uint32_t x = elem_at(in, (((size_t)si * n_tok + (p - L0)) * G.Hkv + h) * D + c, G.EB);
    elem_put(tail, kv ? (size_t)c * T + tt : (size_t)tt * D + c, G.EB, x);
  }
}

__global__ void release_kernel(Geo G, DevBufs B, int seq, int n_blocks) {
  const int n = n_blocks * 2 * G.Hkv;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const size_t idx = (size_t)seq * G.max_blocks * 2 * G.Hkv + i;
    const uint32_t e = B.table[idx];
    if (e == kUnallocated) continue;
    const int slot = (int)entry_slot(e);
    const int s = slot % kPoolStripes;  // back to the sub-stack the slot belongs to
    if (e & kRawTile) {
      const int t = atomicAdd(&B.counters->raw_top[s].n, 1);
      B.raw_free[kPoolStripes * t + s] = slot;
    } else {
      const int t = atomicAdd(&B.counters->comp_top[s].n, 1);
      B.comp_free[kPoolStripes * t + s] = slot;
    }
    B.table[idx] = kUnallocated;
  }
}

// FORMAT v2 tile (BF16), one element at a time: every group's mode index from the two tag
// planes and, by a block scan of their code bits, its offset in the CODES stream (in LDS); then
// each thread rebuilds elements from their w-bit code and sign/mantissa byte and hands element
// (t, c) to put(t, c, bits).  Corrupt tiles (a mode index outside the set, codes past the
// capacity, an exponent past 8 bits) set status bit 8; every read stays inside the slot: the
// mode index is clamped to the set and code reads past the capacity return 0.
template <class Put>
__device__ void decode_tile_v2(const Geo& G, const DevBufs& B, const uint8_t* tile, const uint8_t* b2,
                               const uint8_t* b3, const uint8_t* b4, Put put) {
  __shared__ uint32_t gO[1024];
  __shared__ uint8_t gk[1024];
  __shared__ int red[8];
  const int tid = threadIdx.x, D = G.D, GT = G.GT;
  const uint32_t* tag0 = reinterpret_cast<const uint32_t*>(tile + G.tag_off);
  const uint32_t* tag1 = tag0 + G.PW;
  const int per = (G.NG + kThreads - 1) / kThreads, q0 = min(G.NG, tid * per), q1 = min(G.NG, q0 + per);
  int bits = 0;
  bool bad = false;
  for (int q = q0; q < q1; ++q) {
    int k = (int)(((tag0[q >> 5] >> (q & 31)) & 1u) | (((tag1[q >> 5] >> (q & 31)) & 1u) << 1));
    if (k >= G.n_modes) {
      bad = true;
      k = G.n_modes - 1;
    }
    gk[q] = (uint8_t)k;
    bits += GT * G.mw[k];
  }
  int total;
  int O = block_exclusive_scan(bits, red, &total);
  for (int q = q0; q < q1; ++q) {
    gO[q] = (uint32_t)O;
    O += GT * G.mw[gk[q]];
  }
  if (tid == 0 && total > 8 * G.code_cap) bad = true;  // codes past the capacity
  __syncthreads();
  // one group per thread and pass: its code bits (at most GT * 8 = 128, plus up to 31 bits of
  // word offset: five words) in registers from aligned word loads, clamped to the slot's code
  // area; its GT sign/mantissa bytes in one 8- or 16-byte load; its base once
  const uint32_t* code32 = reinterpret_cast<const uint32_t*>(tile + G.code_off);
  const int n_words = (G.code_cap + 15) / 16 * 4;  // the code area (16-byte aligned) in words
  for (int q = tid; q < G.NG; q += kThreads) {
    const int k = gk[q], w = G.mw[k];
    const int tg = q / D, c = q % D;
    const uint32_t base = v2_base(G, k, b2, b3, b4, c);
    const int O = (int)gO[q], w0 = O >> 5, sh = O & 31;
    uint32_t cw[5];
#pragma unroll
    for (int u = 0; u < 5; ++u) cw[u] = (w0 + u < n_words && (u == 0 || 32 * u < sh + GT * w)) ? code32[w0 + u] : 0u;
    uint32_t smw[4];
    if (GT == 16) {
      const uint4 v = *reinterpret_cast<const uint4*>(tile + G.sm_off + (size_t)q * 16);
      smw[0] = v.x; smw[1] = v.y; smw[2] = v.z; smw[3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(tile + G.sm_off + (size_t)q * 8);
      smw[0] = v.x; smw[1] = v.y; smw[2] = smw[3] = 0u;
    }
    const uint32_t mask = (1u << w) - 1u;
    for (int tau = 0; tau < GT; ++tau) {
      const int bp = sh + tau * w, wi = bp >> 5, bs = bp & 31;
      const uint32_t lo = cw[0], hi = cw[1];
      uint32_t a0 = wi == 0 ? lo : wi == 1 ? hi : wi == 2 ? cw[2] : wi == 3 ? cw[3] : cw[4];
      uint32_t a1 = wi == 0 ? hi : wi == 1 ? cw[2] : wi == 2 ? cw[3] : wi == 3 ? cw[4] : 0u;
      const uint32_t o = (uint32_t)(((((uint64_t)a1 << 32) | a0) >> bs) & mask);
      const uint32_t e = base + o;
      bad |= e > 255u;
      const uint32_t s8 = (smw[tau >> 2] >> (8 * (tau & 3))) & 0xFFu;
      put(tg * GT + tau, c, ((s8 >> 7) << 15) | ((e & 0xFFu) << 7) | (s8 & 0x7Fu));
    }
  }
  if (bad) atomicOr(&B.counters->status, 8u);
}

// A compressed tile's tag planes and escape area in LDS, loaded by the whole workgroup in one
// coalesced pass, with the escape units before every tag word (a wide or raw group has E set;
// a raw BF16 group adds four more units).  Decoding threads then read only LDS.
constexpr int kMaxTagWords = 64 * 128 / 8 / 32;  // T <= 64, D <= 128, groups of >= 8 tokens
struct TileMeta {
  uint32_t tag[2 * kMaxTagWords];  // plane E, then plane R
  uint32_t pre[kMaxTagWords];
  uint32_t esc[512 / 4];           // esc_cap <= 512
};
// tl / nt: this thread's index among the nt threads staging the tile (the whole block, or one
// half of it when two tiles are staged at once); every thread of the block reaches the
// barriers, `active` false for threads with no tile to stage.
// A tile whose tags claim more escape bits than the escape capacity holds is corrupt: flagged
// (status bit 8); its reads past the capacity are clamped by the decoders.
__device__ void stage_tile_meta(const Geo& G, const DevBufs& B, const uint8_t* tile, TileMeta& m, int tl, int nt,
                                bool active) {
  const uint32_t* tag_g = reinterpret_cast<const uint32_t*>(tile + G.tag_off);
  const uint32_t* esc_g = reinterpret_cast<const uint32_t*>(tile + G.esc_off);
  if (active) {
    for (int i = tl; i < 2 * G.PW; i += nt) m.tag[i] = tag_g[i];
    for (int i = tl; i < G.esc_cap / 4; i += nt) m.esc[i] = esc_g[i];
  }
  __syncthreads();
  // escape units before each tag word: an exclusive scan over the PW <= 32 words by the first
  // wave of the staging threads (nt >= 128 threads: tl < 64 is one whole wave)
  if (active && tl < 64) {
    const uint32_t cnt = tl < G.PW ? __popc(m.tag[tl]) + (uint32_t)(G.F - 4) * __popc(m.tag[G.PW + tl]) : 0u;
    uint32_t inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = (uint32_t)__shfl_up((int)inc, o);
      if (tl >= o) inc += t;
    }
    if (tl < G.PW) m.pre[tl] = inc - cnt;
    if (tl == 63 && inc * (uint32_t)G.GT > 8u * (uint32_t)G.esc_cap) atomicOr(&B.counters->status, 8u);  // escape overrun
  }
  __syncthreads();
}

// Codes of slot s (0..7, a run-time value) of a CODE unit, one 3-bit code per byte lane.
__device__ __forceinline__ uint32_t code_slot_rt(uint32_t W0, uint32_t W1, uint32_t W2, int s) {
  switch (s) {
    case 0: return code_slot<0>(W0, W1, W2);
    case 1: return code_slot<1>(W0, W1, W2);
    case 2: return code_slot<2>(W0, W1, W2);
    case 3: return code_slot<3>(W0, W1, W2);
    case 4: return code_slot<4>(W0, W1, W2);
    case 5: return code_slot<5>(W0, W1, W2);
    case 6: return code_slot<6>(W0, W1, W2);
    default: return code_slot<7>(W0, W1, W2);
  }
}

// BF16 tiles with 8-token groups, four tokens per 32-bit word as the 16-token path: one thread
// per CODE unit (32 elements = channels c0..c0+3 x tokens 8tg..8tg+7, one group per channel).
// Escape units are single bytes (an 8-bit plane per escaped group; a raw group adds four bytes
// of offset bits 4..7, token tau's nibble at bits 4*tau).
// put4(t, c0, w) receives BF16 channels c0..c0+3 of token t (w.x: c0, c0+1; w.y: c0+2, c0+3);
// with by_cols, put8(tg, c, w) instead receives tokens 8tg..8tg+7 of channel c in order (two per
// word, the earlier token in the low half).
// tl, nt, active: as stage_tile_meta (every thread of the block calls it).
template <class Put4, class Put8>
__device__ void decode_bf16_g8_tile(const Geo& G, const DevBufs& B, const uint8_t* tile, const uint8_t* b3,
                                    const uint8_t* b4, TileMeta& m, Put4 put4, Put8 put8, bool by_cols, int tl, int nt,
                                    bool active) {
  const int D = G.D;
  const int n_units = active ? G.raw_elems / 32 : 0;
  stage_tile_meta(G, B, tile, m, tl, nt, active);
  const uint8_t* esc = reinterpret_cast<const uint8_t*>(m.esc);
  for (int u = tl; u < n_units; u += nt) {
    const int q0 = 4 * u, w = q0 >> 5, bit = q0 & 31, tg = q0 / D, c0 = q0 % D;
    uint32_t P = m.pre[w];  // escape bytes before group q0
    const uint32_t Ew = m.tag[w], Rw = m.tag[G.PW + w];
    const uint32_t below = bit == 0 ? 0u : (0xFFFFFFFFu >> (32 - bit));
    P += __popc(Ew & below) + 4u * __popc(Rw & below);
    const uint32_t* cw = reinterpret_cast<const uint32_t*>(tile + G.code_off + 12 * u);
    const uint32_t W0 = cw[0], W1 = cw[1], W2 = cw[2];
    const uint4 s4[2] = {*reinterpret_cast<const uint4*>(tile + G.sm_off + 32 * u),
                         *reinterpret_cast<const uint4*>(tile + G.sm_off + 32 * u + 16)};
    const uint32_t smw[8] = {s4[0].x, s4[0].y, s4[0].z, s4[0].w, s4[1].x, s4[1].y, s4[1].z, s4[1].w};
    uint32_t o02[4][2], o13[4][2];  // [channel][token quad]
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const uint32_t E = (Ew >> (bit + gi)) & 1u, R = (Rw >> (bit + gi)) & 1u;
      if (R && !E) atomicOr(&B.counters->status, 8u);
      const int c = c0 + gi;
      const uint32_t base = R ? 0u : (E ? b4[c] : b3[c]);
      const uint32_t H = perm_b32(base, base, 0u);
      uint32_t plane = 0, hi = 0;
      if (E && (int)P < G.esc_cap) plane = esc[P];
      if (R) {  // four bytes at P + 1 (not word aligned in general): byte by byte
        for (int k = 0; k < 4; ++k) hi |= ((int)P + 1 + k < G.esc_cap ? (uint32_t)esc[P + 1 + k] : 0u) << (8 * k);
      }
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const uint32_t cs = code_slot_rt(W0, W1, W2, 2 * gi + qq);
        const uint32_t e3 = spread4((plane >> (4 * qq)) & 0xFu) << 3;
        const uint32_t X = R ? raw_high_nibbles((hi >> (16 * qq)) & 0xFFFFu) : 0u;
        const uint32_t Ev = H + cs + e3 + X;
        const uint32_t sv = smw[2 * gi + qq];
        o02[gi][qq] = bitsel(0x7F807F80u, Ev << 7, perm_b32(sv, sv, 0x02020000u));
        o13[gi][qq] = bitsel(0x7F807F80u, Ev >> 1, perm_b32(sv, sv, 0x03030101u));
      }
      P += E + 4u * R;
    }
    if (by_cols) {  // channel c0+gi: tokens 4qq+{0,1} are the low halves of o02, o13; 4qq+{2,3} the high
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
        put8(tg, c0 + gi, make_uint4(perm_b32(o13[gi][0], o02[gi][0], 0x05040100u), perm_b32(o13[gi][0], o02[gi][0], 0x07060302u),
                                     perm_b32(o13[gi][1], o02[gi][1], 0x05040100u), perm_b32(o13[gi][1], o02[gi][1], 0x07060302u)));
      continue;
    }
    // token t = 8tg + 4qq + k: channels c0..c0+3 as one 8-byte store
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t sel = (k >> 1) ? 0x07060302u : 0x05040100u;  // tokens 4qq+{0,1}: low halves
        const uint32_t w01 = (k & 1) ? perm_b32(o13[1][qq], o13[0][qq], sel) : perm_b32(o02[1][qq], o02[0][qq], sel);
        const uint32_t w23 = (k & 1) ? perm_b32(o13[3][qq], o13[2][qq], sel) : perm_b32(o02[3][qq], o02[2][qq], sel);
        put4(8 * tg + 4 * qq + k, c0, make_uint2(w01, w23));
      }
  }
}
template <class Put4>
__device__ void decode_bf16_g8_tile(const Geo& G, const DevBufs& B, const uint8_t* tile, const uint8_t* b3,
                                    const uint8_t* b4, TileMeta& m, Put4 put4, int tl, int nt, bool active) {
  decode_bf16_g8_tile(G, B, tile, b3, b4, m, put4, [](int, int, uint4) {}, false, tl, nt, active);
}

// Four FP8 values (bytes of w, in order) -> four BF16 values (two per word, in order), exactly.
template <int FMT>
__device__ __forceinline__ uint2 fp8x4_bf16(uint32_t w) {
  if constexpr (FMT == 1)
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true)));
  else
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)));
}

// BF16 tiles with 16-token groups: one thread per pair of groups (channels c0, c0+1 x 16 tokens,
// one 32-element CODE unit), the four-token SWAR rebuild of rebuild_group.  put2(t, c0, w)
// receives BF16 channels c0, c0+1 of token t (low half c0); with by_cols, put_col(t0, c, w)
// instead receives tokens t0 .. t0+3 of channel c (two per word, the earlier token in the low
// half).  tl, nt, active: as stage_tile_meta.
template <class Put2, class PutCol>
__device__ __forceinline__ void decode_bf16_g16_tile(const Geo& G, const DevBufs& B, const uint8_t* tile, const uint8_t* b3,
                                     const uint8_t* b4, TileMeta& m, Put2 put2, PutCol put_col, bool by_cols, int tl,
                                     int nt, bool active) {
  const int D = G.D;
  stage_tile_meta(G, B, tile, m, tl, nt, active);
  const uint16_t* esc16 = reinterpret_cast<const uint16_t*>(m.esc);
  const int max_plane = G.esc_cap / 2;
  const int n_pairs = active ? G.NP : 0;
  for (int pr = tl; pr < n_pairs; pr += nt) {
    const int q0 = 2 * pr, w = q0 >> 5, bit = q0 & 31;
    const uint32_t Ew = m.tag[w], Rw = m.tag[G.PW + w];
    uint32_t P = planes_before(Ew, Rw, m.pre[w], bit);
    const uint4 s0 = *reinterpret_cast<const uint4*>(tile + G.sm_off + 32 * pr);
    const uint4 s1 = *reinterpret_cast<const uint4*>(tile + G.sm_off + 32 * pr + 16);
    const uint32_t* cw = reinterpret_cast<const uint32_t*>(tile + G.code_off + 12 * pr);
    const uint32_t W0 = cw[0], W1 = cw[1], W2 = cw[2];
    const int tg = q0 / D, c0 = q0 % D;
    uint32_t outs[2][2][4];  // [channel][o02 | o13][token quad]
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const uint32_t E = (Ew >> (bit + gi)) & 1u, R = (Rw >> (bit + gi)) & 1u;
      if (R && !E) atomicOr(&B.counters->status, 8u);
      const int mode = (int)(E + R);
      const int c = c0 + gi;
      const uint32_t base = mode == 0 ? b3[c] : (mode == 1 ? b4[c] : 0u);
      uint32_t plane0 = 0, X[4] = {0u, 0u, 0u, 0u};
      if (E && (int)P < max_plane) plane0 = esc16[P];
      if (R) {
        for (int qq = 0; qq < 4; ++qq) X[qq] = ((int)P + 1 + qq < max_plane) ? raw_high_nibbles(esc16[P + 1 + qq]) : 0u;
      }
      const uint32_t smv[4] = {gi ? s1.x : s0.x, gi ? s1.y : s0.y, gi ? s1.z : s0.z, gi ? s1.w : s0.w};
      if (gi == 0) rebuild_group<0>(smv, W0, W1, W2, base, plane0, X, outs[0][0], outs[0][1]);
      else rebuild_group<1>(smv, W0, W1, W2, base, plane0, X, outs[1][0], outs[1][1]);
      P += E + 4u * R;
    }
    if (by_cols) {  // channel c0+gi, tokens 4j..4j+3: the low halves of o02, o13, then the high halves
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          put_col(tg * kGroup + 4 * j, c0 + gi,
                  make_uint2(perm_b32(outs[gi][1][j], outs[gi][0][j], 0x05040100u),
                             perm_b32(outs[gi][1][j], outs[gi][0][j], 0x07060302u)));
      continue;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tg * kGroup + 4 * j;
      // (c0, c1) pairs per token
      put2(t + 0, c0, perm_b32(outs[1][0][j], outs[0][0][j], 0x05040100u));
      put2(t + 2, c0, perm_b32(outs[1][0][j], outs[0][0][j], 0x07060302u));
      put2(t + 1, c0, perm_b32(outs[1][1][j], outs[0][1][j], 0x05040100u));
      put2(t + 3, c0, perm_b32(outs[1][1][j], outs[0][1][j], 0x07060302u));
    }
  }
}

// FP8 tiles (E5M2, E4M3) with 16- or 8-token groups, four tokens per 32-bit word: one thread
// per CODE unit (32 elements: 32/GT channels x GT tokens, one group per channel).  Each 4-token
// slot's exponents are base (b3 narrow, b4 wide, 0 raw) + 3-bit code + escape bits (plane bit 3
// for wide and raw groups; E5M2 raw groups a second plane for bit 4; escape units of GT bits),
// then assembled with the sign/mantissa fields into the four FP8 bytes (E5M2: 3-bit fields laid
// out like the codes; E4M3: a nibble per element, low nibble first).  Corrupt tags (raw without
// escape, E4M3 wide, exponent sums past the field) set status bit 8; escape reads stay inside
// the staged capacity.
// put_tok(t, c0, w) receives the FP8 bytes of channels c0 .. c0 + 32/GT - 1 of token t (byte i:
// channel c0 + i); with by_cols, put_col(t0, c, w) instead receives tokens t0 .. t0 + 3 of
// channel c (byte k: token t0 + k).  tl, nt, active: as stage_tile_meta.
template <int FMT, int GT, class PutTok, class PutCol>
__device__ __forceinline__ void decode_fp8_tile(const Geo& G, const DevBufs& B, const uint8_t* tile, const uint8_t* b3,
                                const uint8_t* b4, TileMeta& m, PutTok put_tok, PutCol put_col, bool by_cols, int tl,
                                int nt, bool active) {
  constexpr int F = FMT == 1 ? 5 : 4, MB = 7 - F;
  constexpr int GPU = 32 / GT;  // groups (channels) per unit
  constexpr int SPG = GT / 4;   // 4-token slots per group
  constexpr uint32_t EMAX = ((1u << F) - 1u) * 0x01010101u;
  const int D = G.D;
  stage_tile_meta(G, B, tile, m, tl, nt, active);
  const uint8_t* esc8 = reinterpret_cast<const uint8_t*>(m.esc);
  const uint16_t* esc16 = reinterpret_cast<const uint16_t*>(m.esc);
  const int max_unit = GT == 8 ? G.esc_cap : G.esc_cap / 2;
  auto esc_unit = [&](uint32_t P) -> uint32_t { return (int)P < max_unit ? (GT == 8 ? esc8[P] : esc16[P]) : 0u; };
  const int n_units = active ? G.raw_elems / 32 : 0;
  for (int u = tl; u < n_units; u += nt) {
    const int q0 = GPU * u, w = q0 >> 5, bit = q0 & 31, tg = q0 / D, c0 = q0 % D;
    const uint32_t Ew = m.tag[w], Rw = m.tag[G.PW + w];
    const uint32_t below = bit == 0 ? 0u : (0xFFFFFFFFu >> (32 - bit));
    uint32_t P = m.pre[w] + __popc(Ew & below) + (uint32_t)(F - 4) * __popc(Rw & below);
    const uint32_t* cw = reinterpret_cast<const uint32_t*>(tile + G.code_off + 12 * u);
    const uint32_t W0 = cw[0], W1 = cw[1], W2 = cw[2];
    uint32_t S[4];
    if constexpr (FMT == 1) {
      const uint32_t* sw = reinterpret_cast<const uint32_t*>(tile + G.sm_off + 12 * u);
      S[0] = sw[0], S[1] = sw[1], S[2] = sw[2], S[3] = 0u;
    } else {
      const uint4 s4 = *reinterpret_cast<const uint4*>(tile + G.sm_off + 16 * u);
      S[0] = s4.x, S[1] = s4.y, S[2] = s4.z, S[3] = s4.w;
    }
    uint32_t bytes[GPU][SPG];
    uint32_t over = 0;
#pragma unroll
    for (int gi = 0; gi < GPU; ++gi) {
      const uint32_t E = (Ew >> (bit + gi)) & 1u, R = (Rw >> (bit + gi)) & 1u;
      if ((R && !E) || (FMT == 2 && E && !R)) atomicOr(&B.counters->status, 8u);
      const int c = c0 + gi;
      const uint32_t H = (R ? 0u : (E ? b4[c] : b3[c])) * 0x01010101u;
      const uint32_t plane = E ? esc_unit(P) : 0u;
      const uint32_t hip = (FMT == 1 && R) ? esc_unit(P + 1) : 0u;
#pragma unroll
      for (int q = 0; q < SPG; ++q) {
        const int slot = SPG * gi + q;
        const uint32_t cs = code_slot_rt(W0, W1, W2, slot);
        uint32_t e = H + cs + (spread4((plane >> (4 * q)) & 0xFu) << 3);
        if constexpr (FMT == 1) e += spread4((hip >> (4 * q)) & 0xFu) << 4;
        over |= (e + (0x80u - (1u << F)) * 0x01010101u) & 0x80808080u;  // a lane at or past 2^F
        e &= EMAX;
        uint32_t g;  // sign at bit 7, mantissa at bits 0..MB-1
        if constexpr (FMT == 1) {
          g = slot == 0 ? e5m2_sign_mant<0>(S[0], S[1], S[2]) : slot == 1 ? e5m2_sign_mant<1>(S[0], S[1], S[2])
            : slot == 2 ? e5m2_sign_mant<2>(S[0], S[1], S[2]) : slot == 3 ? e5m2_sign_mant<3>(S[0], S[1], S[2])
            : slot == 4 ? e5m2_sign_mant<4>(S[0], S[1], S[2]) : slot == 5 ? e5m2_sign_mant<5>(S[0], S[1], S[2])
            : slot == 6 ? e5m2_sign_mant<6>(S[0], S[1], S[2]) : e5m2_sign_mant<7>(S[0], S[1], S[2]);
        } else {
          const uint32_t sw = S[slot >> 1];
          g = e4m3_sign_mant(perm_b32(sw, sw, (slot & 1) ? 0x03030202u : 0x01010000u));
        }
        bytes[gi][q] = bfi(EMAX << MB, e << MB, g);
      }
      P += E + (uint32_t)(F - 4) * R;
    }
    if (over) atomicOr(&B.counters->status, 8u);
    if (by_cols) {
#pragma unroll
      for (int gi = 0; gi < GPU; ++gi)
#pragma unroll
        for (int q = 0; q < SPG; ++q) put_col(GT * tg + 4 * q, c0 + gi, bytes[gi][q]);
      continue;
    }
#pragma unroll
    for (int q = 0; q < SPG; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t sel = 0x0C0C0000u | ((4u + k) << 8) | (uint32_t)k;  // byte k of the low, then the high word
        uint32_t wd = perm_b32(bytes[1][q], bytes[0][q], sel);
        if constexpr (GPU == 4) wd |= perm_b32(bytes[3][q], bytes[2][q], sel) << 16;
        put_tok(GT * tg + 4 * q + k, c0, wd);
      }
  }
}

// One block per (block, K|V, head): rebuilds the tile into [n*T][Hkv][D].
__global__ void __launch_bounds__(kThreads) decode_blocks_kernel(Geo G, DevBufs B, int seq, int first,
                                                                  void* __restrict__ kout, void* __restrict__ vout) {
  const int bi = blockIdx.x, kv = blockIdx.y / G.Hkv, h = blockIdx.y % G.Hkv;
  const int b = first + bi, D = G.D, T = G.T, tid = threadIdx.x;
  void* outv = kv ? vout : kout;
  const uint32_t e = B.table[table_index(G, seq, b, kv, h)];
  auto out_idx = [&](int t, int c) -> size_t { return (((size_t)bi * T + t) * G.Hkv + h) * D + c; };
  if (e == kUnallocated) {
    for (int i = tid; i < G.raw_elems; i += kThreads) elem_put(outv, out_idx(i / D, i % D), G.EB, 0u);
    if (tid == 0) atomicOr(&B.counters->status, 4u);
    return;
  }
  const int slot = (int)entry_slot(e);
  if (e & kRawTile) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(B.raw_pool) + (size_t)slot * G.raw_elems * G.EB;
    for (int i = tid; i < G.raw_elems; i += kThreads) {
      const int t = i / D, c = i % D;
      elem_put(outv, out_idx(t, c), G.EB, elem_at(src, kv ? (size_t)c * T + t : (size_t)i, G.EB));
    }
    return;
  }
  const uint8_t* tile = B.comp_pool + (size_t)slot * G.stride;
  const int ver = entry_version(e);  // the base version this tile was encoded with
  const uint8_t* b3 = bases_of(G, B.bases, ver, 3, kv, h);
  const uint8_t* b4 = bases_of(G, B.bases, ver, 4, kv, h);
  __shared__ TileMeta meta;
  if (G.mode_set != 0) {
    decode_tile_v2(G, B, tile, bases_of(G, B.bases, ver, 2, kv, h), b3, b4,
                   [&](int t, int c, uint32_t x) { elem_put(outv, out_idx(t, c), 2, x); });
    return;
  }
  const int row = G.Hkv * D;  // elements between consecutive tokens of the output
  if (G.EB == 2 && G.GT == 8) {
    uint16_t* o16 = reinterpret_cast<uint16_t*>(outv) + out_idx(0, 0);
    decode_bf16_g8_tile(G, B, tile, b3, b4, meta,
                        [&](int t, int c0, uint2 w) { *reinterpret_cast<uint2*>(o16 + t * row + c0) = w; },
                        tid, kThreads, true);
    return;
  }
  if (G.EB == 1) {  // FP8: the bytes of two (16-token groups) or four (8-token groups) channels per token
    uint8_t* o8 = reinterpret_cast<uint8_t*>(outv) + out_idx(0, 0);
    auto put_tok = [&](int t, int c0, uint32_t w) {
      if (G.GT == 8) *reinterpret_cast<uint32_t*>(o8 + t * row + c0) = w;
      else *reinterpret_cast<uint16_t*>(o8 + t * row + c0) = (uint16_t)w;
    };
    auto no_col = [](int, int, uint32_t) {};
    if (G.fmt == 1) {
      if (G.GT == 8) decode_fp8_tile<1, 8>(G, B, tile, b3, b4, meta, put_tok, no_col, false, tid, kThreads, true);
      else decode_fp8_tile<1, 16>(G, B, tile, b3, b4, meta, put_tok, no_col, false, tid, kThreads, true);
    } else {
      if (G.GT == 8) decode_fp8_tile<2, 8>(G, B, tile, b3, b4, meta, put_tok, no_col, false, tid, kThreads, true);
      else decode_fp8_tile<2, 16>(G, B, tile, b3, b4, meta, put_tok, no_col, false, tid, kThreads, true);
    }
    return;
  }
  uint16_t* out0 = reinterpret_cast<uint16_t*>(outv) + out_idx(0, 0);
  decode_bf16_g16_tile(G, B, tile, b3, b4, meta,
                       [&](int t, int c0, uint32_t w) { *reinterpret_cast<uint32_t*>(out0 + t * row + c0) = w; },
                       [](int, int, uint2) {}, false, tid, kThreads, true);
}


// ------------------------------------------------------------------------------------------
// Decode attention over compressed caches with 8-token groups (the split kernels of the
// attention library rebuild 16-token groups only).  Method as there (GAAC page §3.2): each
// workgroup covers a contiguous range of finished blocks of one (sequence, KV head), rebuilds
// every block's K and V tile on chip, into LDS (the cache is never decompressed to HBM), and
// keeps an fp32 online softmax for each query head of the GQA group; the partial results (acc,
// and max and sum in base-2 units) go to the same workspace, for the same merge kernel.  The
// rebuilt tiles go to LDS as BF16 (FP8 converted exactly; K as rows, V transposed, rows padded
// to an odd number of 16-byte units); scores and PV run on v_mfma_f32_16x16x32_bf16 with the
// query heads as the 16 rows (zero past the GQA group): wave w scores tokens 16w..16w+15, the
// block's maximum per head meets in LDS, the probabilities go to LDS as a BF16 high part plus
// remainder (~16 mantissa bits), and wave w accumulates channels (D/4)w .. (D/4)(w+1)-1.
struct AnyAttnArgs {
  Geo G;
  DevBufs B;
  const uint16_t* q;
  float* ws_acc;
  float* ws_ml;
  float sl2;  // scale * log2(e)
  int n_splits;
  const uint8_t* k_new;  // decode step: the new tokens, [n][Hkv][D] elements (else null)
  const uint8_t* v_new;
  int4 zrow[kMaxSeqsPerLaunch];  // blockIdx.z -> {sequence index, sequence id, tokens in finished
                                 // blocks, tail position of the new token}
};

constexpr int kAnyMaxG = 16;   // query heads per KV head
constexpr int kAnyMaxTD = 64 * 128;

// Element bits -> value, exactly: FMT 0 BF16, 1 OCP E5M2, 2 OCP E4M3 (FN).
template <int FMT>
__device__ __forceinline__ float elem_value(uint32_t x) {
  if constexpr (FMT == 0) {
    return __uint_as_float(x << 16);
  } else {
    constexpr int F = FMT == 1 ? 5 : 4, MB = 7 - F, bias = FMT == 1 ? 15 : 7;
    const uint32_t e = (x >> MB) & ((1u << F) - 1u), m = x & ((1u << MB) - 1u);
    float v;
    if (FMT == 1 && e == 31) v = m ? __uint_as_float(0x7FC00000u) : __uint_as_float(0x7F800000u);
    else if (FMT == 2 && e == 15 && m == 7) v = __uint_as_float(0x7FC00000u);
    else if (e == 0) v = ldexpf((float)m, 1 - bias - MB);
    else v = ldexpf((float)((1u << MB) | m), (int)e - bias - MB);
    return (x >> 7) ? -v : v;
  }
}

// Sum / maximum over aligned segments of W lanes (W = 16, 32 or 64 divides the wave).
__device__ __forceinline__ float seg_sum(float v, int W) {
  for (int o = 1; o < W; o <<= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float seg_max(float v, int W) {
  for (int o = 1; o < W; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Element bits -> BF16 bits, exactly (every FP8 value is a BF16 value).
template <int FMT>
__device__ __forceinline__ uint16_t elem_bf16(uint32_t x) {
  if constexpr (FMT == 0) return (uint16_t)x;
  else return (uint16_t)(__float_as_uint(elem_value<FMT>(x)) >> 16);
}

typedef __bf16 any_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float any_f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ any_f32x4_t any_mfma(const uint4& a, const uint4& b, any_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(any_bf16x8_t, a), __builtin_bit_cast(any_bf16x8_t, b),
                                                 c, 0, 0, 0);
}
// Maximum / sum over each row of 16 lanes (DPP: quad swaps, then the half-row and row mirrors),
// the same value in all 16 lanes.
template <int CTRL>
__device__ __forceinline__ float any_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, any_dpp<0xB1>(v));
  v = fmaxf(v, any_dpp<0x4E>(v));
  v = fmaxf(v, any_dpp<0x141>(v));
  return fmaxf(v, any_dpp<0x140>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += any_dpp<0xB1>(v);
  v += any_dpp<0x4E>(v);
  v += any_dpp<0x141>(v);
  return v + any_dpp<0x140>(v);
}

template <int FMT>
__global__ void __launch_bounds__(kThreads) attn_any_kernel(AnyAttnArgs a) {
  constexpr int KS = 128 + 8;  // K rows [t][KS], BF16 bits
  constexpr int VS = 64 + 8;   // V transposed [c][VS]; P [head][VS]
  const Geo& G = a.G;
  const int D = G.D, T = G.T, g = G.g, S = a.n_splits, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, col = lane & 15, kq = lane >> 4;
  const int split = blockIdx.x, h = blockIdx.y;
  const int4 z = a.zrow[blockIdx.z];
  const int si = z.x, seq = z.y, L = z.z;
  __shared__ __align__(16) uint16_t kt[64 * KS];
  __shared__ __align__(16) uint16_t vt[128 * VS];
  __shared__ __align__(16) uint16_t pl[2][16 * VS];  // probabilities, BF16 high part and remainder
  __shared__ float wmx[4][16], wsm[4][16];            // per wave: maximum and sum of each head's row
  __shared__ float mh[16], lh[16];                    // running maximum and sum per head (row)
  __shared__ TileMeta meta[2];
  // blocks [b0, b1): the finished blocks dealt out as evenly as possible
  const int nb = L / T, per = nb / S, rem = nb % S;
  const int b0 = split * per + min(split, rem), b1 = b0 + per + (split < rem ? 1 : 0);
  // zeros where a 16-token block leaves the MFMA's 32-token K steps short (tokens 16..31 of P and
  // V are never written then)
  for (int i = tid; i < 128 * VS / 8; i += kThreads) reinterpret_cast<uint4*>(vt)[i] = make_uint4(0, 0, 0, 0);
  for (int i = tid; i < 2 * 16 * VS / 8; i += kThreads) reinterpret_cast<uint4*>(pl)[i] = make_uint4(0, 0, 0, 0);
  if (tid < 16) {
    mh[tid] = -INFINITY;
    lh[tid] = 0.0f;
  }
  // this lane's query operands: head col (zero past the group), channels 32i + 8kq .. +7
  uint4 qa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    qa[i] = (col < g && 32 * i < D) ? *reinterpret_cast<const uint4*>(a.q + ((size_t)si * G.Hq + h * g + col) * D + 32 * i + 8 * kq)
                                    : make_uint4(0, 0, 0, 0);
  const int CTW = D / 64;  // 16-channel output tiles per wave
  any_f32x4_t o[2];
  o[0] = o[1] = any_f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t flags = 0;
  __syncthreads();
  auto entry = [&](int b, int kv) -> uint32_t { return a.B.table[table_index(G, seq, b, kv, h)]; };
  // rebuilt element (t, c) of the K (kv 0) or V (kv 1) tile, as BF16 bits, to LDS
  auto put = [&](int kv, int t, int c, uint32_t x) {
    if (kv) vt[c * VS + t] = elem_bf16<FMT>(x);
    else kt[t * KS + c] = elem_bf16<FMT>(x);
  };
  uint32_t eK = b0 < b1 ? entry(b0, 0) : kUnallocated, eV = b0 < b1 ? entry(b0, 1) : kUnallocated;
  for (int b = b0; b < b1; ++b) {
    // the next block's table entries load while this block is rebuilt
    uint32_t nK = kUnallocated, nV = kUnallocated;
    if (b + 1 < b1) {
      nK = entry(b + 1, 0);
      nV = entry(b + 1, 1);
    }
    if (G.mode_set == 0) {
      // FORMAT v1: the K tile by threads 0..127 and the V tile by 128..255 at once (BF16 with
      // 8-token groups, or FP8), K as rows, V as transposed columns
      const int kv = tid >> 7, tl = tid & 127;
      const uint32_t e = kv ? eV : eK, slot = entry_slot(e);
      const bool comp = e != kUnallocated && !(e & kRawTile);
      const int ver = comp ? entry_version(e) : 0;
      if (e == kUnallocated) {  // missing: zeros, reported
        for (int i = tl; i < T * D; i += kThreads / 2) put(kv, i / D, i % D, 0u);
        flags |= 4u;
      } else if (!comp) {  // raw tile: K [t][c], V [c][t]
        const uint8_t* src = reinterpret_cast<const uint8_t*>(a.B.raw_pool) + (size_t)slot * G.raw_elems * G.EB;
        for (int i = tl; i < T * D; i += kThreads / 2)
          put(kv, i / D, i % D, elem_at(src, kv ? (size_t)(i % D) * T + i / D : (size_t)i, G.EB));
      }
      const uint8_t* tile = a.B.comp_pool + (comp ? (size_t)slot * G.stride : 0);
      const uint8_t* b3 = bases_of(G, a.B.bases, ver, 3, kv, h);
      const uint8_t* b4 = bases_of(G, a.B.bases, ver, 4, kv, h);
      if constexpr (FMT == 0) {
        decode_bf16_g8_tile(G, a.B, tile, b3, b4, meta[kv],
                            [&](int t, int c0, uint2 w) { *reinterpret_cast<uint2*>(kt + t * KS + c0) = w; },
                            [&](int tg, int c, uint4 w) { *reinterpret_cast<uint4*>(vt + c * VS + 8 * tg) = w; }, kv == 1,
                            tl, kThreads / 2, comp);
      } else {
        auto put_tok = [&](int t, int c0, uint32_t w) {
          if (G.GT == 8) *reinterpret_cast<uint2*>(kt + t * KS + c0) = fp8x4_bf16<FMT>(w);
          else *reinterpret_cast<uint32_t*>(kt + t * KS + c0) = fp8x4_bf16<FMT>(w).x;
        };
        auto put_col = [&](int t0, int c, uint32_t w) { *reinterpret_cast<uint2*>(vt + c * VS + t0) = fp8x4_bf16<FMT>(w); };
        if (G.GT == 8) decode_fp8_tile<FMT, 8>(G, a.B, tile, b3, b4, meta[kv], put_tok, put_col, kv == 1, tl, kThreads / 2, comp);
        else decode_fp8_tile<FMT, 16>(G, a.B, tile, b3, b4, meta[kv], put_tok, put_col, kv == 1, tl, kThreads / 2, comp);
      }
      __syncthreads();
    } else {
      for (int kv = 0; kv < 2; ++kv) {
        const uint32_t e = kv ? eV : eK, slot = entry_slot(e);
        const int ver = entry_version(e);
        if (e == kUnallocated) {  // missing: zeros, reported
          for (int i = tid; i < T * D; i += kThreads) put(kv, i / D, i % D, 0u);
          flags |= 4u;
        } else if (e & kRawTile) {  // raw tile: K [t][c], V [c][t]
          const uint8_t* src = reinterpret_cast<const uint8_t*>(a.B.raw_pool) + (size_t)slot * G.raw_elems * G.EB;
          for (int i = tid; i < T * D; i += kThreads) {
            const int t = i / D, c = i % D;
            put(kv, t, c, elem_at(src, kv ? (size_t)c * T + t : (size_t)i, G.EB));
          }
        } else {  // FORMAT v2 (nested precision modes, BF16)
          decode_tile_v2(G, a.B, a.B.comp_pool + (size_t)slot * G.stride, bases_of(G, a.B.bases, ver, 2, kv, h),
                         bases_of(G, a.B.bases, ver, 3, kv, h), bases_of(G, a.B.bases, ver, 4, kv, h),
                         [&](int t, int c, uint32_t x) { put(kv, t, c, x); });
        }
        __syncthreads();
      }
    }
    eK = nK;
    eV = nV;
    // ---- scores: wave w takes tokens 16w .. 16w+15; lane holds heads 4kq+r of token 16w+col ----
    float sc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (16 * wv < T) {
      any_f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (32 * i < D) acc = any_mfma(qa[i], *reinterpret_cast<const uint4*>(kt + (16 * wv + col) * KS + 32 * i + 8 * kq), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = acc[r] * a.sl2;
        const float mx = row16_max(sc[r]);
        if (col == 0) wmx[wv][4 * kq + r] = mx;
      }
    }
    __syncthreads();
    // ---- the block's maximum per head, probabilities, rescale factors ----
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hd = 4 * kq + r;
      float mb = wmx[0][hd];
      for (int w = 1; w < T / 16; ++w) mb = fmaxf(mb, wmx[w][hd]);
      const float m_old = mh[hd], m_new = fmaxf(m_old, mb);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      alpha[r] = exp2f(m_old - m_use);
      if (16 * wv < T) {
        const float p = exp2f(sc[r] - m_use);
        const float hi = (float)(__bf16)p;
        pl[0][hd * VS + 16 * wv + col] = __builtin_bit_cast(uint16_t, (__bf16)p);
        pl[1][hd * VS + 16 * wv + col] = __builtin_bit_cast(uint16_t, (__bf16)(p - hi));
        const float sm = row16_sum(p);
        if (col == 0) wsm[wv][hd] = sm;
      }
    }
    __syncthreads();
    // ---- PV: wave w accumulates channel tiles CTW*w .. ; the running state moves on ----
    for (int u = 0; u < CTW; ++u) {
      const int ct = CTW * wv + u;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[u][r] *= alpha[r];
      for (int j = 0; 32 * j < T; ++j) {
        const uint4 vb = *reinterpret_cast<const uint4*>(vt + (16 * ct + col) * VS + 32 * j + 8 * kq);
        o[u] = any_mfma(*reinterpret_cast<const uint4*>(pl[0] + col * VS + 32 * j + 8 * kq), vb, o[u]);
        o[u] = any_mfma(*reinterpret_cast<const uint4*>(pl[1] + col * VS + 32 * j + 8 * kq), vb, o[u]);
      }
    }
    if (tid < 16) {  // the running maximum and sum of head (row) tid, as every lane rescaled above
      float mb = wmx[0][tid], sum = wsm[0][tid];
      for (int w = 1; w < T / 16; ++w) mb = fmaxf(mb, wmx[w][tid]), sum += wsm[w][tid];
      const float m_old = mh[tid], m_new = fmaxf(m_old, mb);
      lh[tid] = lh[tid] * exp2f(m_old - (m_new == -INFINITY ? 0.0f : m_new)) + sum;
      mh[tid] = m_new;
    }
    __syncthreads();  // before the next block overwrites the tiles, the probabilities and the state
  }
  // ---- partial results: heads 4kq+r, channels 16ct + col ----
  for (int u = 0; u < CTW; ++u) {
    const int ct = CTW * wv + u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hd = 4 * kq + r;
      if (hd < g) a.ws_acc[(((size_t)si * G.Hq + h * g + hd) * S + split) * D + 16 * ct + col] = o[u][r];
    }
  }
  if (tid < g) {
    float* ml = a.ws_ml + (((size_t)si * G.Hq + h * g + tid) * S + split) * 2;
    ml[0] = mh[tid];
    ml[1] = lh[tid];
  }
  if (flags && (tid & (kThreads / 2 - 1)) == 0) atomicOr(&a.B.counters->status, flags);  // either half may see a gap
  // decode step: the first split stores the sequence's new token into the tail (K row t, V
  // column t); the merge kernel that follows reads it there
  if (a.k_new != nullptr && split == 0) {
    const int t = z.w;
    void* tail = a.B.tail;
    const size_t ko = tail_offset(G, seq, 0, h), vo = tail_offset(G, seq, 1, h);
    const size_t src = ((size_t)si * G.Hkv + h) * D;
    for (int c = tid; c < D; c += kThreads) {
      elem_put(tail, ko + (size_t)t * D + c, G.EB, elem_at(a.k_new, src + c, G.EB));
      elem_put(tail, vo + (size_t)c * T + t, G.EB, elem_at(a.v_new, src + c, G.EB));
    }
  }
}
// ------------------------------------------------------------------------------------------
// Decode attention over 256-channel heads, stored as two 128-channel half-heads (GAAC page App.
// D): a head's score needs both halves, so one workgroup takes both.  Per block the four
// half-tiles (K and V of both halves) are rebuilt at once, one per wave, into LDS as BF16 (K as
// rows, V transposed; the SWAR decoders of every format and group size); scores and PV then run
// on v_mfma_f32_16x16x32_bf16 as in the 8-token-group kernel (query heads as the 16 rows, eight
// 32-channel K steps over both halves, wave w accumulating channels 64w .. 64w+63).  The last
// split also attends the tail (the merge kernel then merges splits only).
struct HalfAttnArgs {
  Geo G;  // the half-head geometry the cache stores (D = 128, Hkv and Hq doubled)
  DevBufs B;
  const uint16_t* q;  // [n][Hq][256]
  float* ws_acc;
  float* ws_ml;
  float sl2;
  int n_splits;
  int4 zrow[kMaxSeqsPerLaunch];  // {sequence index, sequence id, tokens in finished blocks, tail tokens}
};

template <int FMT>
__global__ void __launch_bounds__(kThreads) attn_half_kernel(HalfAttnArgs a) {
  constexpr int DH = 128, DR = 256;  // half-head and head channels
  constexpr int KS = DH + 8;         // K half-tile rows [t][KS], BF16 bits
  constexpr int VS = 64 + 8;         // V transposed [c][VS] (c over the whole head); P [head][VS]
  const Geo& G = a.G;
  const int T = G.T, g = G.g, S = a.n_splits, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, col = lane & 15, kq = lane >> 4;
  const int Hq = G.Hq / 2;
  const int split = blockIdx.x, h = blockIdx.y;
  const int4 z = a.zrow[blockIdx.z];
  const int si = z.x, seq = z.y, L = z.z, ntail = z.w;
  __shared__ __align__(16) uint16_t kt[2][64 * KS];
  __shared__ __align__(16) uint16_t vt[DR * VS];
  __shared__ __align__(16) uint16_t pl[2][16 * VS];  // probabilities, BF16 high part and remainder
  __shared__ float wmx[4][16], wsm[4][16];            // per wave: maximum and sum of each head's row
  __shared__ float mh[16], lh[16];                    // running maximum and sum per head (row)
  __shared__ TileMeta meta[4];
  const int nb = L / T, per = nb / S, rem = nb % S;
  const int b0 = split * per + min(split, rem), b1 = b0 + per + (split < rem ? 1 : 0);
  const int bend = b1 + ((split == S - 1 && ntail > 0) ? 1 : 0);  // block b1 = the tail
  // zeros where a 16-token block leaves the MFMA's 32-token K steps short
  for (int i = tid; i < DR * VS / 8; i += kThreads) reinterpret_cast<uint4*>(vt)[i] = make_uint4(0, 0, 0, 0);
  for (int i = tid; i < 2 * 16 * VS / 8; i += kThreads) reinterpret_cast<uint4*>(pl)[i] = make_uint4(0, 0, 0, 0);
  if (tid < 16) {
    mh[tid] = -INFINITY;
    lh[tid] = 0.0f;
  }
  // this lane's query operands: head col (zero past the group), channels 32i + 8kq .. +7
  uint4 qa[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    qa[i] = col < g ? *reinterpret_cast<const uint4*>(a.q + ((size_t)si * Hq + h * g + col) * DR + 32 * i + 8 * kq)
                    : make_uint4(0, 0, 0, 0);
  any_f32x4_t o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = any_f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t flags = 0;
  __syncthreads();
  for (int b = b0; b < bend; ++b) {
    const bool tailblk = b == b1;
    const int nvalid = tailblk ? ntail : T;
    // ---- the four half-tiles at once, one per wave: wave w fills (K|V) w >> 1 of half-head w & 1 ----
    {
      const int kv = wv >> 1, hf = wv & 1, hh = 2 * h + hf;
      const uint32_t e = tailblk ? 0u : a.B.table[table_index(G, seq, b, kv, hh)];
      const uint32_t slot = entry_slot(e);
      const bool comp = !tailblk && e != kUnallocated && !(e & kRawTile);
      const int ver = comp ? entry_version(e) : 0;
      uint16_t* krow = kt[hf];
      uint16_t* vcol = vt + (size_t)DH * hf * VS;
      if (!comp) {  // tail, raw tile (K [t][c], V [c][t]) or missing (zeros, reported)
        const uint8_t* src = nullptr;
        if (tailblk) src = reinterpret_cast<const uint8_t*>(a.B.tail) + tail_offset(G, seq, kv, hh) * G.EB;
        else if (e != kUnallocated) src = reinterpret_cast<const uint8_t*>(a.B.raw_pool) + (size_t)slot * G.raw_elems * G.EB;
        else flags |= 4u;
        // 8-element pieces in the stored orientation, which is the LDS one (K rows, V columns);
        // tokens at or past nvalid (a tail's unused columns) are zeros
        const int per_line = kv ? T / 8 : DH / 8;
        for (int p = lane; p < T * DH / 8; p += 64) {
          const int r = p / per_line, x0 = 8 * (p % per_line);  // K: token r, channels x0..; V: channel r, tokens x0..
          uint4 v8 = make_uint4(0, 0, 0, 0);
          if (src) {
            const size_t off = (size_t)r * (kv ? T : DH) + x0;
            if constexpr (FMT == 0) {
              v8 = *reinterpret_cast<const uint4*>(src + 2 * off);
            } else {
              const uint2 b8 = *reinterpret_cast<const uint2*>(src + off);
              const uint2 lo = fp8x4_bf16<FMT>(b8.x), hi = fp8x4_bf16<FMT>(b8.y);
              v8 = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
          }
          uint32_t wds[4] = {v8.x, v8.y, v8.z, v8.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {  // invalid tokens: a whole K row, or single V column entries
            const int t_lo = kv ? x0 + 2 * k : r, t_hi = kv ? x0 + 2 * k + 1 : r;
            if (t_lo >= nvalid) wds[k] &= 0xFFFF0000u;
            if (t_hi >= nvalid) wds[k] &= 0x0000FFFFu;
          }
          v8 = make_uint4(wds[0], wds[1], wds[2], wds[3]);
          if (kv) *reinterpret_cast<uint4*>(vcol + r * VS + x0) = v8;
          else *reinterpret_cast<uint4*>(krow + r * KS + x0) = v8;
        }
      }
      const uint8_t* b3 = bases_of(G, a.B.bases, ver, 3, kv, hh);
      const uint8_t* b4 = bases_of(G, a.B.bases, ver, 4, kv, hh);
      const uint8_t* tile = a.B.comp_pool + (comp ? (size_t)slot * G.stride : 0);
      // every thread reaches its decoder's barriers (active only for a compressed tile)
      if constexpr (FMT == 0) {
        if (G.GT == 8)
          decode_bf16_g8_tile(G, a.B, tile, b3, b4, meta[wv],
                              [&](int t, int c0, uint2 w) { *reinterpret_cast<uint2*>(krow + t * KS + c0) = w; },
                              [&](int tg, int c, uint4 w) { *reinterpret_cast<uint4*>(vcol + c * VS + 8 * tg) = w; },
                              kv == 1, lane, 64, comp);
        else
          decode_bf16_g16_tile(G, a.B, tile, b3, b4, meta[wv],
                               [&](int t, int c0, uint32_t w) { *reinterpret_cast<uint32_t*>(krow + t * KS + c0) = w; },
                               [&](int t0, int c, uint2 w) { *reinterpret_cast<uint2*>(vcol + c * VS + t0) = w; },
                               kv == 1, lane, 64, comp);
      } else {
        auto put_tok = [&](int t, int c0, uint32_t w) {
          if (G.GT == 8) *reinterpret_cast<uint2*>(krow + t * KS + c0) = fp8x4_bf16<FMT>(w);
          else *reinterpret_cast<uint32_t*>(krow + t * KS + c0) = fp8x4_bf16<FMT>(w).x;
        };
        auto put_col = [&](int t0, int c, uint32_t w) { *reinterpret_cast<uint2*>(vcol + c * VS + t0) = fp8x4_bf16<FMT>(w); };
        if (G.GT == 8) decode_fp8_tile<FMT, 8>(G, a.B, tile, b3, b4, meta[wv], put_tok, put_col, kv == 1, lane, 64, comp);
        else decode_fp8_tile<FMT, 16>(G, a.B, tile, b3, b4, meta[wv], put_tok, put_col, kv == 1, lane, 64, comp);
      }
    }
    __syncthreads();
    // ---- scores: wave w takes tokens 16w .. 16w+15 over the 256 channels of both halves ----
    float sc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (16 * wv < T) {
      any_f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc = any_mfma(qa[i], *reinterpret_cast<const uint4*>(kt[i >> 2] + (16 * wv + col) * KS + 32 * (i & 3) + 8 * kq), acc);
      const bool tok_ok = 16 * wv + col < nvalid;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = tok_ok ? acc[r] * a.sl2 : -INFINITY;
        const float mx = row16_max(sc[r]);
        if (col == 0) wmx[wv][4 * kq + r] = mx;
      }
    }
    __syncthreads();
    // ---- the block's maximum per head, probabilities, rescale factors ----
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hd = 4 * kq + r;
      float mb = wmx[0][hd];
      for (int w = 1; w < T / 16; ++w) mb = fmaxf(mb, wmx[w][hd]);
      const float m_old = mh[hd], m_new = fmaxf(m_old, mb);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      alpha[r] = exp2f(m_old - m_use);
      if (16 * wv < T) {
        const float p = exp2f(sc[r] - m_use);
        const float hi = (float)(__bf16)p;
        pl[0][hd * VS + 16 * wv + col] = __builtin_bit_cast(uint16_t, (__bf16)p);
        pl[1][hd * VS + 16 * wv + col] = __builtin_bit_cast(uint16_t, (__bf16)(p - hi));
        const float sm = row16_sum(p);
        if (col == 0) wsm[wv][hd] = sm;
      }
    }
    __syncthreads();
    // ---- PV: wave w accumulates channels 64w .. 64w+63 (four 16-channel tiles) ----
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ct = 4 * wv + u;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[u][r] *= alpha[r];
      for (int j = 0; 32 * j < T; ++j) {
        const uint4 vb = *reinterpret_cast<const uint4*>(vt + (16 * ct + col) * VS + 32 * j + 8 * kq);
        o[u] = any_mfma(*reinterpret_cast<const uint4*>(pl[0] + col * VS + 32 * j + 8 * kq), vb, o[u]);
        o[u] = any_mfma(*reinterpret_cast<const uint4*>(pl[1] + col * VS + 32 * j + 8 * kq), vb, o[u]);
      }
    }
    if (tid < 16) {  // the running maximum and sum of head (row) tid, as every lane rescaled above
      float mb = wmx[0][tid], sum = wsm[0][tid];
      for (int w = 1; w < T / 16; ++w) mb = fmaxf(mb, wmx[w][tid]), sum += wsm[w][tid];
      const float m_old = mh[tid], m_new = fmaxf(m_old, mb);
      lh[tid] = lh[tid] * exp2f(m_old - (m_new == -INFINITY ? 0.0f : m_new)) + sum;
      mh[tid] = m_new;
    }
    __syncthreads();  // before the next block overwrites the tiles, the probabilities and the state
  }
  // ---- partial results: heads 4kq+r, channels 16ct + col ----
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int ct = 4 * wv + u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hd = 4 * kq + r;
      if (hd < g) a.ws_acc[(((size_t)si * Hq + h * g + hd) * S + split) * DR + 16 * ct + col] = o[u][r];
    }
  }
  if (tid < g) {
    float* ml = a.ws_ml + (((size_t)si * Hq + h * g + tid) * S + split) * 2;
    ml[0] = mh[tid];
    ml[1] = lh[tid];
  }
  if (flags) atomicOr(&a.B.counters->status, flags);
}

// ------------------------------------------------------------------------------------------
// Prefill attention over blocks rebuilt by the block decoder (GAAC page §3.3 encodes a prompt's
// complete blocks during prefill and says nothing about how prefill attention reads them; this
// library runs standard causal attention on the rebuilt blocks).  Causal: query i of n_q (token
// position n_kv - n_q + i) attends tokens 0 .. its own position.  One 256-thread workgroup per
// (64 queries, query head), 16 queries per wave; key blocks of KB tokens (64, or 32 for
// 256-channel heads) go to double-buffered LDS as BF16 (K as rows, V transposed); the scores
// are computed transposed, S^T = K Q^T, and the output as O^T = V^T P^T on
// v_mfma_f32_16x16x32_bf16, so each lane holds one query's scores and they serve directly as
// its PV operand (P as a BF16 high part plus remainder, ~16 mantissa bits), with an online
// softmax per query in between.
struct PrefillArgs {
  Geo G;               // the cache's geometry (format; D and heads in the real head layout)
  const uint8_t* k;    // [n_kv][Hkv][D] elements
  const uint8_t* v;
  const uint16_t* q;   // [n_q][Hq][D] BF16
  uint16_t* out;       // [n_q][Hq][D] BF16
  int n_kv, n_q;
  float sl2;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
// Element bits -> BF16 bits (exact: every FP8 value is a BF16 value).
template <int FMT>
__device__ __forceinline__ uint16_t bf16_of(uint32_t x) {
  if constexpr (FMT == 0) return (uint16_t)x;
  else return (uint16_t)(__float_as_uint(elem_value<FMT>(x)) >> 16);
}
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// An 8-element piece of one token's channels as stored (BF16: 16 bytes; FP8: 8 bytes).
template <int FMT> struct PrefillPiece { typedef uint4 type; };
template <> struct PrefillPiece<1> { typedef uint2 type; };
template <> struct PrefillPiece<2> { typedef uint2 type; };

// The piece as eight BF16 values in natural order (FP8 converted exactly).
template <int FMT>
__device__ __forceinline__ uint4 piece_bf16(const typename PrefillPiece<FMT>::type& x) {
  if constexpr (FMT == 0) {
    return x;
  } else {
    const uint32_t w[2] = {x.x, x.y};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t b = w[k >> 1] >> (16 * (k & 1));
      o[k] = (uint32_t)bf16_of<FMT>(b & 0xFFu) | ((uint32_t)bf16_of<FMT>((b >> 8) & 0xFFu) << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// D: head channels (64, 128 or 256).
template <int FMT, int D>
__global__ void __launch_bounds__(kThreads) prefill_kernel(PrefillArgs a) {
  constexpr int QW = 16;           // queries per wave
  constexpr int QT = 4 * QW;       // queries per workgroup
  using Piece = typename PrefillPiece<FMT>::type;
  const Geo& G = a.G;
  const int Hkv = G.Hkv, Hq = G.Hq, g = G.g, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, col = lane & 15, kq = lane >> 4;
  constexpr int KB = D > 128 ? 32 : 64;  // keys per block in LDS
  // LDS row strides, each an odd number of 16-byte units, so that the 16 rows an MFMA operand
  // read touches (and the rows the fill writes at once) fall in different bank groups
  constexpr int KS = D + 8, VS = KB + 8;
  constexpr int C8 = D / 8, TO = KB / 8;  // 8-channel pieces per token, 8-token octets per block
  // the last query tiles attend the most keys: they go first (longest processing time first);
  // heads are the fastest grid dimension, so every head's longest tiles precede all shorter ones
  const int q0 = (gridDim.y - 1 - blockIdx.y) * QT, hq = blockIdx.x, h = hq / g;
  const int pos0 = a.n_kv - a.n_q;   // position of query 0
  const int nq = min(QT, a.n_q - q0);
  // two buffers: the next key block is stored while the current one is attended
  __shared__ __align__(16) uint16_t klb[2][64 * 136];   // key block, BF16 bits, [t][KS]
  __shared__ __align__(16) uint16_t vtlb[2][256 * 40];  // value block transposed, BF16 bits, [c][VS]
  // this wave's queries as QK A operands (rows = queries, k = channels), zero past n_q
  const int qw0 = q0 + QW * wv;                        // first query of this wave
  uint4 qa[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qa[ks] = make_uint4(0, 0, 0, 0);
    if (32 * ks < D && qw0 + col < a.n_q)
      qa[ks] = *reinterpret_cast<const uint4*>(a.q + ((size_t)(qw0 + col) * Hq + hq) * D + 32 * ks + 8 * kq);
  }
  // the online softmax of query qw0 + col (every lane of a column holds the same state)
  float m = -INFINITY, l = 0.0f;
  f32x4_t o[16];  // O^T: lane holds channels 16s + 4kq + i of query qw0 + col
#pragma unroll
  for (int s = 0; s < 16; ++s) o[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int last = pos0 + q0 + nq - 1;       // the last key any query of this workgroup sees
  const int wlast = pos0 + qw0 + QW - 1;     // ... of this wave (clamped below by the data)

  // The fill: threads 0..127 carry K pieces (piece p = tid + 128u: token p / C8, channels
  // 8 (p % C8) ..), threads 128..255 an 8-token x 8-channel block of V each, transposed in
  // registers so that two 8-byte stores write 8 tokens of one channel (in each 32-token chunk
  // the tokens sit in the order of the PV operand, see below).  The 16 lanes of each
  // V store phase cover 8 token octets x 2 channel parities (4 x 4 for 32-key blocks), which
  // puts their rows in distinct bank groups.  A block's pieces load into registers while the
  // previous block is being attended.
  const bool kthr = tid < 128;
  const int vt = tid - 128, v16 = vt & 15;
  const int vj = v16 % TO, vc8 = (16 / TO) * (vt >> 4) + v16 / TO;  // V: token octet, channel piece
  const bool vok = !kthr && vc8 < C8;
  Piece pc[8];
  auto load_block = [&](int kb) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      int t, c8;
      bool ok;
      if (kthr) {
        const int p = tid + 128 * u;
        t = p / C8;
        c8 = p % C8;
        ok = p < KB * C8;
      } else {
        t = 8 * vj + u;
        c8 = vc8;
        ok = vok;
      }
      const int tok = kb + t;
      Piece x;
      if constexpr (FMT == 0) x = make_uint4(0, 0, 0, 0);
      else x = make_uint2(0, 0);
      if (ok && tok <= last) {
        const uint8_t* src = (kthr ? a.k : a.v) + (((size_t)tok * Hkv + h) * D + 8 * c8) * (FMT == 0 ? 2 : 1);
        x = *reinterpret_cast<const Piece*>(src);
      }
      pc[u] = x;
    }
  };
  auto store_block = [&](int buf) {
    uint16_t* kl = klb[buf];
    uint16_t* vtl = vtlb[buf];
    if (kthr) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int p = tid + 128 * u;
        if (p < KB * C8) *reinterpret_cast<uint4*>(kl + (p / C8) * KS + 8 * (p % C8)) = piece_bf16<FMT>(pc[u]);
      }
    } else if (vok) {
      uint32_t x[8][4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint4 b = piece_bf16<FMT>(pc[u]);
        x[u][0] = b.x; x[u][1] = b.y; x[u][2] = b.z; x[u][3] = b.w;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {  // channel 8 vc8 + k: tokens 8 vj .. 8 vj + 7
        const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
        const int w = k >> 1;
        const uint4 y = make_uint4(perm_b32(x[1][w], x[0][w], sel), perm_b32(x[3][w], x[2][w], sel),
                                   perm_b32(x[5][w], x[4][w], sel), perm_b32(x[7][w], x[6][w], sel));
        // tokens in each 32-token chunk stored in the order the PV operand reads them: position
        // 8kq + j holds token 4kq + j (j < 4), then token 16 + 4kq + j - 4; quad q = 2 (vj % 4)
        const int qa = 2 * (vj & 3), cb = 32 * (vj >> 2);
        const int pa = cb + (qa < 4 ? 8 * qa : 8 * (qa - 4) + 4), pb = cb + (qa + 1 < 4 ? 8 * (qa + 1) : 8 * (qa - 3) + 4);
        *reinterpret_cast<uint2*>(vtl + (8 * vc8 + k) * VS + pa) = make_uint2(y.x, y.y);
        *reinterpret_cast<uint2*>(vtl + (8 * vc8 + k) * VS + pb) = make_uint2(y.z, y.w);
      }
    }
  };
  load_block(0);
  store_block(0);
  __syncthreads();
  if (KB <= last) load_block(KB);
  for (int kb0 = 0, buf = 0; kb0 <= last; kb0 += KB, buf ^= 1) {
    const uint16_t* kl = klb[buf];
    const uint16_t* vtl = vtlb[buf];
    if (kb0 <= wlast && qw0 < a.n_q) {
      // S^T = K Q^T: sub-block sb = keys kb0+16sb..; lane holds keys kb0+16sb+4kq+i of query col
      f32x4_t sc[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        sc[sb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (16 * sb < KB) {
#pragma unroll
          for (int ks = 0; ks < 8; ++ks)
            if (32 * ks < D)
              sc[sb] = mfma_bf16(*reinterpret_cast<const uint4*>(kl + (16 * sb + col) * KS + 32 * ks + 8 * kq), qa[ks], sc[sb]);
        }
      }
      const int qpos = pos0 + qw0 + col;
      const bool qok = qw0 + col < a.n_q;
      float rmax = -INFINITY;
      // the causal mask and the query count matter only on the blocks that reach past this
      // wave's first query or hold the last queries; elsewhere every score is kept
      if (kb0 + KB - 1 <= pos0 + qw0 && qw0 + QW <= a.n_q) {
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sc[sb][i] = 16 * sb < KB ? sc[sb][i] * a.sl2 : -INFINITY;
            rmax = fmaxf(rmax, sc[sb][i]);
          }
      } else {
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = kb0 + 16 * sb + 4 * kq + i;
            const bool ok = 16 * sb < KB && tok <= qpos && qok;
            sc[sb][i] = ok ? sc[sb][i] * a.sl2 : -INFINITY;
            rmax = fmaxf(rmax, sc[sb][i]);
          }
      }
      rmax = fmaxf(rmax, __shfl_xor(rmax, 16));  // the query's other keys sit in lanes col + 16 kq
      rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
      const float m_new = fmaxf(m, rmax);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      // exponents are <= 0 here: the hardware exp2 (results below 2^-126 flush to 0)
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      float sum = 0.0f;
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[sb][i] = __builtin_amdgcn_exp2f(sc[sb][i] - m_use);
          sum += sc[sb][i];
        }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      l = l * alpha + sum;
      // the running output needs rescaling only where a query's maximum moved (alpha < 1); once
      // the maxima settle, whole blocks skip it
      if (__any(m_new != m)) {
#pragma unroll
        for (int s = 0; s < 16; ++s)
          if (16 * s < D)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[s][i] *= alpha;
      }
      m = m_new;
      // O^T += V^T P^T over 32-key chunks (sub-blocks 2kc, 2kc+1).  Inside a chunk the MFMA's
      // k slots 8kq+j and 8kq+4+j stand for keys 16(2kc)+4kq+j and 16(2kc+1)+4kq+j, so each
      // lane's own probabilities are its P^T operand (as a BF16 high part plus remainder) and
      // the V^T operand reads the same keys, which the fill stored in that order: one 16-byte
      // piece of a channel row.
      for (int kc = 0; kc < KB / 32; ++kc) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = sc[2 * kc + (e >> 1)][2 * (e & 1)], p1 = sc[2 * kc + (e >> 1)][2 * (e & 1) + 1];
          hi[e] = bf16_pair(p0, p1);
          lo[e] = bf16_pair(p0 - __uint_as_float(hi[e] << 16), p1 - __uint_as_float(hi[e] & 0xFFFF0000u));
        }
        const uint4 ph = make_uint4(hi[0], hi[1], hi[2], hi[3]), plo = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          if (16 * s < D) {
            const uint4 va = *reinterpret_cast<const uint4*>(vtl + (16 * s + col) * VS + 32 * kc + 8 * kq);
            o[s] = mfma_bf16(va, ph, o[s]);
            o[s] = mfma_bf16(va, plo, o[s]);
          }
        }
      }
    }
    // the next block (loaded during the previous block's math) into the other buffer, then one
    // barrier: this block's reads are done and the next block's stores are visible
    if (kb0 + KB <= last) store_block(buf ^ 1);
    __syncthreads();
    if (kb0 + 2 * KB <= last) load_block(kb0 + 2 * KB);
  }
  // out: lane holds channels 16s + 4kq .. 16s + 4kq + 3 of query qw0 + col
  const int qi = qw0 + col;
  if (qi < a.n_q) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (16 * s < D) {
        uint16_t* dst = a.out + ((size_t)qi * Hq + hq) * D + 16 * s + 4 * kq;
        *reinterpret_cast<uint2*>(dst) = make_uint2(bf16_pair(o[s][0] * inv, o[s][1] * inv), bf16_pair(o[s][2] * inv, o[s][3] * inv));
      }
  }
}

}  // namespace

int launch_init(const Geo& G, const DevBufs& B, const int32_t*, const int32_t*, void* stream) {
  hipLaunchKernelGGL(init_kernel, dim3(256), dim3(256), 0, (hipStream_t)stream, G, B);
  return (int)hipGetLastError();
}

int launch_calibrate(const Geo& G, const DevBufs& B, const void* k, const void* v, int n, void* stream) {
  hipLaunchKernelGGL(calibrate_kernel, dim3(G.D, G.Hkv, 2), dim3(kThreads), 0, (hipStream_t)stream, G, B, k, v, n);
  return (int)hipGetLastError();
}

int launch_append(const Geo& G, const DevBufs& B, const SeqList& S, const void* k, const void* v, int n_tokens,
                  int max_new_blocks, void* stream) {
  if (max_new_blocks > 0 && G.mode_set != 0) {  // FORMAT v2: the nested-mode encoder
    const size_t lds = (size_t)G.raw_elems * 2 + (size_t)G.stride + (size_t)(5 * G.NG + 3) / 4 * 4;
    hipLaunchKernelGGL(encode_v2_kernel, dim3(max_new_blocks, S.n, 2 * G.Hkv), dim3(kThreads), lds,
                       (hipStream_t)stream, G, B, S, k, v, n_tokens);
    const int err = (int)hipGetLastError();
    if (err) return err;
  } else if (max_new_blocks > 0) {
    // 8-token groups: BF16 by the unit-per-thread encoder, FP8 by the bit-assembling one
    const bool any = G.GT != kGroup && G.fmt != 0;
    const size_t lds = any ? (size_t)G.raw_elems * 2 + (size_t)G.stride + (size_t)(3 * G.NG + 3) / 4 * 4
                           : (size_t)G.raw_elems * 2 + (size_t)2 * G.PW * 4;
    void (*kern)(Geo, DevBufs, SeqList, const void*, const void*, int) =
        any ? (G.fmt == 1 ? encode_any_kernel<1> : encode_any_kernel<2>)
            : G.GT != kGroup ? encode_g8_kernel
                             : (G.fmt == 0 ? encode_kernel<0> : (G.fmt == 1 ? encode_kernel<1> : encode_kernel<2>));
    hipLaunchKernelGGL(kern, dim3(max_new_blocks, S.n, 2 * G.Hkv), dim3(kThreads), lds, (hipStream_t)stream, G, B,
                       S, k, v, n_tokens);
    const int err = (int)hipGetLastError();
    if (err) return err;
  }
  // the tokens past the last finished block go to the tail; when every sequence's appended tokens
  // end exactly on a block boundary (a decode step's block-completing token) there are none
  bool any_tail = false;
  for (int i = 0; i < S.n; ++i) any_tail |= (S.lens[i] + n_tokens) % G.T != 0;
  if (!any_tail) return (int)hipGetLastError();
  hipLaunchKernelGGL(tail_kernel, dim3(S.n, 2 * G.Hkv), dim3(256), 0, (hipStream_t)stream, G, B, S, k, v, n_tokens);
  return (int)hipGetLastError();
}

int launch_tile_stats(const Geo& G, const DevBufs& B, int seq, int first, int n, int32_t* out, void* stream) {
  const int tiles = n * 2 * G.Hkv;
  hipLaunchKernelGGL(tile_stats_kernel, dim3((tiles + 255) / 256), dim3(256), 0, (hipStream_t)stream, G, B, seq, first, n,
                     out);
  return (int)hipGetLastError();
}

int launch_coverage(const Geo& G, const void* x, int n, int w, int32_t* out, void* stream) {
  hipLaunchKernelGGL(coverage_kernel, dim3(G.D * G.Hkv), dim3(kThreads), 0, (hipStream_t)stream, G, x, n, w, out);
  return (int)hipGetLastError();
}

int launch_read_probe(const void* src, size_t bytes_per_wave, int waves, uint32_t* sink, void* stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(waves), dim3(64), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(src), bytes_per_wave / 16, sink);
  return (int)hipGetLastError();
}

int launch_release(const Geo& G, const DevBufs& B, int seq, int n_blocks, void* stream) {
  if (n_blocks <= 0) return 0;
  const int n = n_blocks * 2 * G.Hkv;
  hipLaunchKernelGGL(release_kernel, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, G, B, seq, n_blocks);
  return (int)hipGetLastError();
}

int launch_decode_blocks(const Geo& G, const DevBufs& B, int seq, int first, int n, void* k_out, void* v_out,
                         void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(decode_blocks_kernel, dim3(n, 2 * G.Hkv), dim3(kThreads), 0, (hipStream_t)stream, G, B, seq,
                     first, k_out, v_out);
  return (int)hipGetLastError();
}

int launch_attention_any(const Geo& G, const DevBufs& B, const SeqList& S, const uint16_t* q, float scale,
                         int n_splits, float* ws_acc, float* ws_ml, const void* k_new, const void* v_new,
                         const int* new_pos, void* stream) {
  // shapes the LDS arrays hold: T <= 64 tokens, D <= 128 channels (a power of two), g <= 16
  if (G.T > 64 || G.D > 128 || G.g > kAnyMaxG || (G.D & (G.D - 1))) return (int)hipErrorInvalidValue;
  AnyAttnArgs a;
  a.G = G;
  a.B = B;
  a.q = q;
  a.ws_acc = ws_acc;
  a.ws_ml = ws_ml;
  a.sl2 = scale * 1.4426950408889634f;
  a.n_splits = n_splits;
  a.k_new = reinterpret_cast<const uint8_t*>(k_new);
  a.v_new = reinterpret_cast<const uint8_t*>(v_new);
  for (int z = 0; z < kMaxSeqsPerLaunch; ++z)
    a.zrow[z] = z < S.n ? make_int4(z, S.ids[z], S.lens[z], k_new ? new_pos[z] : 0) : make_int4(0, 0, 0, 0);
  auto k = G.fmt == 0 ? attn_any_kernel<0> : G.fmt == 1 ? attn_any_kernel<1> : attn_any_kernel<2>;
  hipLaunchKernelGGL(k, dim3(n_splits, G.Hkv, S.n), dim3(kThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_attention_half(const Geo& G, const DevBufs& B, const SeqList& S, const int* ntail, const uint16_t* q,
                          float scale, int n_splits, float* ws_acc, float* ws_ml, void* stream) {
  if (G.D != 128 || G.T > 64 || G.g > kAnyMaxG || (G.Hkv & 1)) return (int)hipErrorInvalidValue;
  HalfAttnArgs a;
  a.G = G;
  a.B = B;
  a.q = q;
  a.ws_acc = ws_acc;
  a.ws_ml = ws_ml;
  a.sl2 = scale * 1.4426950408889634f;
  a.n_splits = n_splits;
  for (int z = 0; z < kMaxSeqsPerLaunch; ++z)
    a.zrow[z] = z < S.n ? make_int4(z, S.ids[z], S.lens[z], ntail[z]) : make_int4(0, 0, 0, 0);
  auto k = G.fmt == 0 ? attn_half_kernel<0> : G.fmt == 1 ? attn_half_kernel<1> : attn_half_kernel<2>;
  hipLaunchKernelGGL(k, dim3(n_splits, G.Hkv / 2, S.n), dim3(kThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_prefill(const Geo& G, const void* k, const void* v, int n_kv, const uint16_t* q, int n_q, float scale,
                   uint16_t* out, void* stream) {
  if (G.D > 256 || (G.D & (G.D - 1)) || n_q < 1 || n_q > n_kv) return (int)hipErrorInvalidValue;
  PrefillArgs a;
  a.G = G;
  a.k = reinterpret_cast<const uint8_t*>(k);
  a.v = reinterpret_cast<const uint8_t*>(v);
  a.q = q;
  a.out = out;
  a.n_kv = n_kv;
  a.n_q = n_q;
  a.sl2 = scale * 1.4426950408889634f;
  if (G.D != 64 && G.D != 128 && G.D != 256) return (int)hipErrorInvalidValue;
  void (*kern)(PrefillArgs);
  if (G.D == 64) kern = G.fmt == 0 ? prefill_kernel<0, 64> : G.fmt == 1 ? prefill_kernel<1, 64> : prefill_kernel<2, 64>;
  else if (G.D == 128) kern = G.fmt == 0 ? prefill_kernel<0, 128> : G.fmt == 1 ? prefill_kernel<1, 128> : prefill_kernel<2, 128>;
  else kern = G.fmt == 0 ? prefill_kernel<0, 256> : G.fmt == 1 ? prefill_kernel<1, 256> : prefill_kernel<2, 256>;
  hipLaunchKernelGGL(kern, dim3(G.Hq, (n_q + 63) / 64), dim3(kThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace kvc

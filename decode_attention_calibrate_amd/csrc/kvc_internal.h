// kvc_internal.h -- geometry, kernel argument blocks and launcher declarations shared by the
// C-ABI host code (api.cpp) and the HIP kernels.  Not part of the public ABI.
//
// Compressed tile layout (FORMAT v1, this library's byte layout for the codec of the page
// "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference on Personal Devices",
// §3.1 codec, App. D stored pieces).  One tile = T tokens x D channels of one (K|V, kv-head):
//   group q = tg*D + c = tokens tg*GT .. tg*GT+GT-1 of channel c (GT = 16 or 8 tokens);
//          element n = GT*q + tau;
//   TAG  : plane E (mode >= 1) then plane R (mode == 2), PW = NG/32 little-endian words each;
//   CODE : 3-bit offset codes; 12-byte units of 32 elements (32/GT groups); element
//          r of a unit lives in byte lane r%4, slot r/4 of a 24-bit lane stream spread over
//          the unit's three words (byte lane k of word w = stream bits 8w..8w+7);
//   SM   : sign/mantissa field (s << MB) | m per element, element order: BF16 one byte each;
//          E5M2 3-bit fields in the CODE unit layout (12 bytes per 32 elements); E4M3 4-bit
//          fields, element n at bits 4n..4n+3 (16 bytes per 32 elements);
//   ESC  : an LSB-first bit stream; for every group with mode >= 1, in q order: a GT-bit
//          plane with bit 3 of the GT offsets (bit tau = token tau); a raw BF16 group then
//          adds the offset bits 4..7 as one 4-bit field per token (4 more GT-bit units), a raw
//          E5M2 group one more plane (bit 4); zero up to esc_cap;
//   RAW  : tiles that overflow esc_cap (and every tile of an uncompressed cache) are stored
//          as native elements, K token-major [t][c], V channel-major [c][t].
// FORMAT v2 (the nested precision modes, BF16; Geo::mode_set != 0): TAG (two planes holding bit
// 0 and bit 1 of each group's mode index) | SM (one byte per element) | CODES: one LSB-first
// stream with each group's offsets, in group order, at its mode's width; a tile whose codes
// exceed the capacity is stored RAW.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace kvc {

constexpr int kGroup = 16;          // group size of the SWAR paths (attention, fast encode/decode)
constexpr int kMaxSeqsPerLaunch = 64;
constexpr uint32_t kUnallocated = 0xFFFFFFFFu;

struct Geo {
  int fmt;                          // 0 BF16, 1 FP8 E5M2, 2 FP8 E4M3 (kvc_dtype)
  int F, MB, EB;                    // exponent bits, mantissa bits, bytes per element
  int sm_pair;                      // SM bytes per pair of groups (32 elements)
  int T, D, Hkv, Hq, g;             // block tokens, head dim, KV heads, query heads, Hq/Hkv
  int GT;                           // tokens per exponent group (16, or 8)
  int NT, NG, NP, PW;               // token groups per tile, groups, group pairs, tag words
  int tag_off, code_off, sm_off, esc_off, stride;  // compressed tile offsets (bytes)
  int esc_cap;                      // escape capacity (bytes)
  int raw_elems;                    // T*D (a raw tile or tail tile holds raw_elems * EB bytes)
  int max_seqs, max_blocks;
  int n_comp, n_raw;
  int compressed;
  // FORMAT v2 (nested precision modes, BF16): mode_set 0 = FORMAT v1; 1, 2, 3 = the mode widths
  // mw[0..n_modes) = {2,3,4,8}, {4,8}, {3,4,8} (raw last).  A v2 slot is TAG | SM | CODES:
  // sm_off, code_off (the stream start) and code_cap (its capacity in bytes) above; esc_cap
  // stays the escape allowance the capacity includes.
  int mode_set, n_modes, mw[4], code_cap;
  // base versions: n_versions calibrated base sets (1..4) of ver_bytes each in the bases
  // buffer; cur_ver is the set blocks are encoded with now.  Each compressed tile's table entry
  // names the set it was encoded with (entry_version).
  int n_versions, cur_ver, ver_bytes;
};

// counters buffer (12,416 bytes).  Atomics to one 128-byte line are performed one after
// another, and a bulk append encodes thousands of tiles at once, so every hot word has a line
// of its own:
//   * each free stack is kPoolStripes interleaved sub-stacks: sub-stack s holds the slots
//     s, s + 16, s + 32, ... (a seeded permutation of them), its element k at index 16k + s of
//     the stack array, with its own top; a tile pops from a preferred sub-stack and moves on
//     to the next ones when it is empty; a released slot goes back to sub-stack slot % 16;
//   * the statistics are kStatStripes copies (one chosen per encoding workgroup), which
//     readers add; compressed tiles are not counted separately (each adds exactly NG groups).
constexpr int kPoolStripes = 16;
constexpr int kStatStripes = 64;
struct alignas(128) PoolTop {
  int32_t n;  // slots in this sub-stack
};
struct alignas(128) StatStripe {
  unsigned long long raw_tiles, groups[4], esc_bytes;  // groups per mode index; FORMAT v2: code bytes
};
struct Counters {
  PoolTop comp_top[kPoolStripes];
  PoolTop raw_top[kPoolStripes];
  alignas(128) uint32_t status;
  StatStripe stat[kStatStripes];
};
constexpr size_t kCountersBytes = 128 * (2 * kPoolStripes + 1 + kStatStripes);
static_assert(sizeof(Counters) == kCountersBytes, "counters buffer");
// slots of sub-stack s in a pool of n slots
__host__ __device__ inline int pool_stripe_size(int n, int s) { return n > s ? (n - s + kPoolStripes - 1) / kPoolStripes : 0; }

struct DevBufs {
  uint8_t* comp_pool;
  uint16_t* raw_pool;    // element storage: 16-bit words (BF16) or bytes (FP8, cast to uint8_t*)
  uint16_t* tail;        // same
  uint8_t* bases;        // [version][K|V][b3|b4][Hkv][D], then (mode set 1) [K|V][Hkv][D] of b2 per version
  uint32_t* table;       // [max_seqs][max_blocks][2][Hkv]
  int32_t* comp_free;
  int32_t* raw_free;
  Counters* counters;
};

struct SeqList {
  int n;
  int ids[kMaxSeqsPerLaunch];
  int lens[kMaxSeqsPerLaunch];     // token count (attention) or token count before append
};

// Table entry of one (sequence, block, K|V, kv-head): kUnallocated, or bit 31 = raw tile,
// bits 29..30 = the base version a compressed tile was encoded with, bits 23..28 = the escape
// bytes a FORMAT v1 tile uses in 16-byte units (<= 63, i.e. <= 1,008 bytes), bits 0..22 = slot.
constexpr uint32_t kRawTile = 0x80000000u;
constexpr uint32_t kSlotMask = 0x007FFFFFu;
constexpr int kMaxSlots = 1 << 23;
constexpr int kMaxVersions = 4;
__host__ __device__ inline uint32_t entry_slot(uint32_t e) { return e & kSlotMask; }
__host__ __device__ inline int entry_esc_units(uint32_t e) { return (int)((e >> 23) & 0x3Fu); }
__host__ __device__ inline int entry_version(uint32_t e) { return (int)((e >> 29) & 3u); }
__host__ __device__ inline uint32_t comp_entry(uint32_t slot, uint32_t esc_units, int ver) {
  return slot | (esc_units << 23) | ((uint32_t)ver << 29);
}
// Calibrated bases of version ver, K|V kv, kv-head h: w = 3 (8-exponent window), 4 (16) or 2
// (4-exponent window, FORMAT v2 mode set 1); D bytes, one per channel.
__host__ __device__ inline size_t bases_at(const Geo& G, int ver, int w, int kv, int h) {
  const size_t v0 = (size_t)ver * G.ver_bytes;
  if (w == 2) return v0 + (size_t)4 * G.Hkv * G.D + ((size_t)kv * G.Hkv + h) * G.D;
  return v0 + ((size_t)(2 * kv + (w - 3)) * G.Hkv + h) * G.D;
}
__host__ __device__ inline const uint8_t* bases_of(const Geo& G, const uint8_t* bases, int ver, int w, int kv, int h) {
  return bases + bases_at(G, ver, w, kv, h);
}

__host__ __device__ inline size_t table_index(const Geo& G, int seq, int blk, int kv, int h) {
  return (((size_t)seq * G.max_blocks + blk) * 2 + kv) * G.Hkv + h;
}
__host__ __device__ inline size_t tail_offset(const Geo& G, int seq, int kv, int h) {
  return (((size_t)seq * 2 + kv) * G.Hkv + h) * (size_t)G.raw_elems;
}

// ---- launchers (defined in the .hip files; return hipError_t as int) ----
int launch_init(const Geo& G, const DevBufs& B, const int32_t* comp_perm_dev, const int32_t* raw_perm_dev,
                void* stream);
int launch_calibrate(const Geo& G, const DevBufs& B, const void* k, const void* v, int n_tokens, void* stream);
int launch_append(const Geo& G, const DevBufs& B, const SeqList& seqs, const void* k, const void* v, int n_tokens,
                  int max_new_blocks, void* stream);
int launch_release(const Geo& G, const DevBufs& B, int seq, int n_blocks, void* stream);
int launch_decode_blocks(const Geo& G, const DevBufs& B, int seq, int first, int n, void* k_out, void* v_out,
                         void* stream);
// seqs.lens: tokens of the finished blocks (partials) or of the whole sequence (combine).
// k_new / v_new (a decode step, else null): each sequence's new token, [n][Hkv][D] elements,
// which the split kernel's first split of every (sequence, head) stores at tail position
// new_pos[i] while the blocks are attended (the split kernel never reads the tail).
int launch_attention_partials(const Geo& G, const DevBufs& B, const SeqList& seqs, const uint16_t* q, float scale,
                              int n_splits, float* ws_acc, float* ws_ml, const void* k_new, const void* v_new,
                              const int* new_pos, void* stream);
// (Compressed caches with 8-token groups in 64-token blocks take a register-rebuild kernel of
// their own.)  The same partials for compressed caches with 8-token groups in other block sizes
// and for FORMAT v2 (any format), from blocks rebuilt into LDS; same workspace layout and
// decode-step tail store.
int launch_attention_any(const Geo& G, const DevBufs& B, const SeqList& seqs, const uint16_t* q, float scale,
                         int n_splits, float* ws_acc, float* ws_ml, const void* k_new, const void* v_new,
                         const int* new_pos, void* stream);
// Partials for 256-channel heads stored as two half-heads: seqs.lens are the finished tokens and
// ntail[i] the tail tokens, which the last split attends (the merge then merges splits only).
// Workspace and q in the real head geometry ([..][Hq/2 of G][256]).
int launch_attention_half(const Geo& G, const DevBufs& B, const SeqList& seqs, const int* ntail, const uint16_t* q,
                          float scale, int n_splits, float* ws_acc, float* ws_ml, void* stream);
// Causal prefill attention over decoded K/V ([n_kv][Hkv][D]) for the last n_q positions; G in the
// real head layout (D up to 256).
int launch_prefill(const Geo& G, const void* k, const void* v, int n_kv, const uint16_t* q, int n_q, float scale,
                   uint16_t* out, void* stream);
int launch_combine(const Geo& G, const DevBufs& B, const SeqList& seqs, const uint16_t* q, float scale, int n_splits,
                   const float* ws_acc, const float* ws_ml, uint16_t* out, void* stream);
int launch_tile_stats(const Geo& G, const DevBufs& B, int seq, int first, int n, int32_t* out, void* stream);
int launch_coverage(const Geo& G, const void* x, int n, int w, int32_t* out, void* stream);
int launch_read_probe(const void* src, size_t bytes_per_wave, int waves, uint32_t* sink, void* stream);
// Device address of the current device's KVC_NOALLOC_WS_BYTES split workspace (resolved once per
// device; later calls only look it up).  Returns a hipError_t as int.
int noalloc_workspace(void** ptr);

}  // namespace kvc

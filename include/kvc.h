/*
 * kvc.h -- C ABI of a lossless compressed-KV decode-attention library for AMD MI355X (gfx950).
 *
 * The method is the one of the page "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM
 * Inference on Personal Devices" (paperlayer.ai summary of arXiv:2610.38210v1):
 *   - §3.1: BF16 (or FP8, App. B) exponents are stored as a calibrated per-(head, channel)
 *     base plus a small offset; each group of tokens of one channel picks a 3-bit, 4-bit or raw
 *     exponent mode; values outside the window widen the whole group; sign and mantissa bits
 *     are stored unchanged, so every value is rebuilt bit for bit.
 *   - §3.2: decode attention reads the compressed tiles and rebuilds them on chip, with the
 *     compressed blocks, the raw blocks and the uncompressed tail in one softmax.
 *   - §3.3 / Figure 3: new tokens accumulate in an uncompressed tail; a full block is encoded
 *     once into a fixed-capacity slot, or kept raw if its encoding does not fit; a block table
 *     records each block's storage mode and location.
 * The byte layout of a compressed tile ("FORMAT v1") is this library's own; the page prints none.
 *
 * Conventions for every entry point:
 *   - Plain C: no C++ types or exceptions cross this boundary.  Every call returns KVC_OK (0)
 *     or a negative KVC_E* code and never aborts; kv_last_error() gives a message.
 *   - "dev" pointers are device memory owned by the caller (e.g. torch tensors on one GPU).
 *     The library never allocates or frees device memory; it allocates only the small host
 *     object behind kvc_cache.
 *   - "stream" is a hipStream_t passed as void* (NULL = the default stream).  Work is only
 *     enqueued; nothing synchronises except kv_cache_create and kv_get_status.
 *   - Argument errors are found on the host before anything is enqueued.  Conditions found on
 *     the device (a pool ran out, a missing block) set sticky bits read by kv_get_status.
 *   - One kvc_cache is one layer of KV cache, used from one host thread and one stream at a time.
 *   - Element tensors hold raw bit patterns: BF16 as 16-bit words, FP8 as bytes.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KVC_BF16 = 0, KVC_FP8_E5M2 = 1, KVC_FP8_E4M3 = 2 } kvc_dtype;

enum {
  KVC_OK = 0,
  KVC_EINVAL = -1,        /* bad argument                                               */
  KVC_ENOSLOT = -2,       /* not enough free slots / table room for the request         */
  KVC_EUNSUPPORTED = -3,  /* valid request the library's kernels do not implement      */
  KVC_EHIP = -4,          /* a HIP runtime call failed                                  */
  KVC_ECORRUPT = -5,      /* corrupt stored data (reserved tag, escape overrun)         */
  KVC_ESTATE = -6,        /* call not valid in the cache's current state                */
  KVC_ESMALLWS = -7       /* workspace smaller than kv_attention_workspace_bytes()      */
};

/* Sticky device status bits (kv_get_status). */
enum {
  KVC_STATUS_COMP_EXHAUSTED = 1u << 0, /* a compressed slot was needed and none was free     */
  KVC_STATUS_RAW_EXHAUSTED = 1u << 1,  /* a raw slot was needed and none was free            */
  KVC_STATUS_MISSING_BLOCK = 1u << 2,  /* attention met an unallocated block (skipped)       */
  KVC_STATUS_CORRUPT = 1u << 3         /* a reserved tag pair was met while decoding         */
};

typedef struct {
  int32_t dtype;              /* kvc_dtype                                                   */
  int32_t num_kv_heads;       /* Hkv                                                         */
  int32_t num_q_heads;        /* Hq; Hq % Hkv == 0, Hq / Hkv <= 16 (query head hq reads KV
                                 head hq / (Hq / Hkv))                                       */
  int32_t head_dim;           /* D in {64, 128, 256}.  A 256-channel head is stored as two
                                 128-channel half-heads (GAAC page App. D): the tiles, tails,
                                 bases and table rows of [..][Hkv][256] data are those of
                                 [..][2 Hkv][128], the same memory (a block takes 2 x 2 Hkv
                                 slots); calibration, encode, decode, statistics and decode
                                 attention (both halves of a head in one softmax, through a
                                 simpler LDS-rebuild kernel) work on it                      */
  int32_t block_tokens;       /* T: tokens per block/tile: a multiple of 16 is valid; the
                                 kernels implement 16, 32 and 64 (others: KVC_EUNSUPPORTED)  */
  int32_t group_tokens;       /* G: tokens per exponent group, 16 or 8 (GAAC
                                 page §3.1 groups the exponents of a few tokens of one
                                 channel).  Decode attention over a compressed cache
                                 rebuilds tiles in registers: a kernel for G = 16 (the tuned
                                 path) and one for G = 8 in 64-token blocks; a G = 8 cache in
                                 16- or 32-token blocks is attended by rebuilding each block's
                                 tiles into LDS (correct for every format, not tuned)        */
  int32_t esc_cap_bytes;      /* escape capacity per tile, multiple of 16, <= 2032 (the
                                 kernels implement <= 512); < 0 selects T*D/16               */
  int32_t compressed;         /* 1: blocks are encoded; 0: every block is stored raw (the
                                 uncompressed baseline cache, same table and layout)         */
  int32_t max_seqs;           /* sequence ids are 0 .. max_seqs-1                            */
  int32_t max_blocks_per_seq; /* finished blocks a sequence may hold                         */
  int32_t num_comp_slots;     /* compressed slot pool size (ignored when compressed == 0)    */
  int32_t num_raw_slots;      /* raw slot pool size                                          */
  int32_t mode_set;           /* exponent modes (GAAC page §4.7.2, nested precision modes):
                                 0 = 3-bit, 4-bit and raw in FORMAT v1 (the tuned path);
                                 FORMAT v2, each group's offsets at its own mode's width in
                                 one stream: 1 = 2-, 3-, 4-bit and raw (a 2-bit mode added),
                                 2 = 4-bit and raw (no 3-bit mode), 3 = 3-, 4-bit and raw.
                                 FORMAT v2 needs BF16 and head_dim <= 128
                                 (KVC_EUNSUPPORTED otherwise); its caches are decoded and
                                 attended by the element-wise LDS-rebuild kernels           */
  int32_t base_versions;      /* calibrated base sets the cache can hold at once, 1..4 (0
                                 means 1): kv_recalibrate switches later blocks to a new set
                                 while every stored tile keeps decoding with the set it was
                                 encoded with (GAAC page App. C: windows calibrated near the
                                 start of a context drift away from rotated keys)           */
} kvc_params;

/* Device buffers, all owned by the caller; sizes from kv_buffer_sizes (same order). */
typedef struct {
  void* comp_pool;   /* [num_comp_slots][slot_stride] bytes: compressed tiles               */
  void* raw_pool;    /* [num_raw_slots][T*D] elements: raw tiles, K token-major [t][c],
                        V channel-major [c][t]                                              */
  void* tail;        /* [max_seqs][2 (K,V)][Hkv][T*D] elements, raw-tile layout             */
  void* bases;       /* per base version (base_versions of them, version-major):
                        [2 (K,V)][2 (narrow b3, wide b4)][Hkv][D] uint8 calibrated bases;
                        mode_set 1 adds [2 (K,V)][Hkv][D] 2-bit-window bases b2 after them  */
  void* block_table; /* [max_seqs][max_blocks_per_seq][2 (K,V)][Hkv] uint32 entries:
                        0xFFFFFFFF = unallocated; else bit 31 = raw, bits 29..30 = the base
                        version a compressed tile was encoded with, bits 23..28 = escape
                        bytes used in 16-byte units (0 in FORMAT v2), bits 0..22 = slot
                        (slot counts < 2^23)                                                */
  void* comp_free;   /* [num_comp_slots] int32 free stack of compressed slots: 16
                        interleaved sub-stacks (sub-stack s = the slots equal to s mod 16,
                        its element k at index 16k + s), popped from a preferred sub-stack
                        first                                                              */
  void* raw_free;    /* [num_raw_slots] int32 free stack of raw slots, the same layout      */
  void* counters;    /* 12,416 B: the 32 sub-stack tops, the status word and 64 stripes of
                        uint64 statistics, each on its own 128-byte line                   */
} kvc_buffers;

#define KVC_NUM_BUFFERS 8

typedef struct {
  uint64_t comp_tiles;    /* tiles stored compressed                                        */
  uint64_t raw_tiles;     /* tiles stored raw (escape overflow or compressed == 0)          */
  uint64_t groups[4];     /* groups per mode index (compressed tiles only): FORMAT v1 narrow,
                             wide, raw, 0; FORMAT v2 the modes of the set in width order     */
  uint64_t esc_bytes;     /* escape bytes used by compressed tiles (FORMAT v2: code bytes)  */
  int32_t comp_free;      /* free compressed slots                                          */
  int32_t raw_free;       /* free raw slots                                                 */
} kvc_stats;

typedef struct kvc_cache kvc_cache; /* opaque host object */

/* Byte size of every kvc_buffers field for these parameters (out_bytes[KVC_NUM_BUFFERS]),
 * plus the compressed slot stride.  Host only; no GPU needed. */
int kv_buffer_sizes(const kvc_params* params, size_t* out_bytes, size_t* slot_stride);

/* Validates the parameters and buffers, initialises the block table (all unallocated), the
 * free stacks (a permutation of the slot ids seeded by perm_seed, dealt to the sub-stacks in
 * that order), the counters and the bases
 * (zero), then synchronises the stream.  *out receives a host object the caller frees with
 * kv_cache_destroy.  The buffers must stay valid for the cache's lifetime. */
int kv_cache_create(const kvc_params* params, const kvc_buffers* buffers, uint64_t perm_seed, void* stream,
                    kvc_cache** out);
void kv_cache_destroy(kvc_cache* cache);

/* Window calibration (GAAC page §3.1: per-head-channel windows of 8 and 16 exponents chosen
 * from calibration data).  k_dev, v_dev: [n_tokens][Hkv][D] elements (typically the first
 * tokens of one sequence).  For each (K|V, head, channel) the narrow base b3 is the start of
 * the 8-wide exponent window holding the most calibration exponents and b4 the same for the
 * 16-wide window; ties take the lower median of the tied starts.  The bases go to base
 * version 0, which blocks are then encoded with.  Must precede the first block encode
 * (KVC_ESTATE otherwise) and may not be repeated once blocks exist. */
int kv_calibrate(kvc_cache* cache, const void* k_dev, const void* v_dev, int32_t n_tokens, void* stream);

/* Recalibration of a live cache (GAAC page App. C: exponent windows calibrated near the start
 * of a context drift away from RoPE-rotated keys further on).  Calibrates a new base version
 * from k_dev, v_dev ([n_tokens][Hkv][D] elements, as kv_calibrate) and encodes every block
 * finished after this call with it; blocks already stored keep the version they were encoded
 * with (tiles are never re-encoded), and every decoder reads a tile's version from its table
 * entry.  The new version is the first of the cache's base_versions, after the current one,
 * that holds no live block (blocks of released sequences do not count).  KVC_ESTATE if
 * kv_calibrate has not run, or if every other version still holds live blocks (base_versions
 * = 1 always); KVC_EINVAL for NULL or empty inputs.  Enqueued on stream; host bookkeeping
 * only otherwise. */
int kv_recalibrate(kvc_cache* cache, const void* k_dev, const void* v_dev, int32_t n_tokens, void* stream);

/* Appends n_tokens tokens to each listed sequence (GAAC page §3.3, fill-then-finalize).
 * k_dev, v_dev: [n_seqs][n_tokens][Hkv][D] elements, 16-byte aligned (KVC_EINVAL otherwise).
 * Tokens go to the sequence's tail; each
 * block that becomes full is encoded once into a compressed slot, or stored raw when its
 * escape planes exceed the capacity (or when compressed == 0), and its table entry is written.
 * n_tokens == 1 is a decode step; larger values are a bulk (prefill) append.  seq_ids_host:
 * host array of n_seqs distinct ids.  KVC_ENOSLOT if a sequence would exceed
 * max_blocks_per_seq; pool exhaustion is detected on the device (status bits). */
int kv_encode_append(kvc_cache* cache, const int32_t* seq_ids_host, int32_t n_seqs, const void* k_dev,
                     const void* v_dev, int32_t n_tokens, void* stream);

/* Rebuilds finished blocks first_block .. first_block+n_blocks-1 of one sequence into plain
 * element tensors k_out_dev, v_out_dev: [n_blocks*T][Hkv][D], 16-byte aligned (GAAC page §3.2
 * reconstruction, bit for bit).  Unallocated blocks come out as zeros and set
 * KVC_STATUS_MISSING_BLOCK. */
int kv_decode_blocks(kvc_cache* cache, int32_t seq, int32_t first_block, int32_t n_blocks, void* k_out_dev,
                     void* v_out_dev, void* stream);

/* Causal prefill attention over K/V in plain element tensors, e.g. the blocks kv_decode_blocks
 * rebuilt.  GAAC page §3.3 encodes a prompt's complete blocks during prefill and leaves the
 * incomplete suffix uncompressed; it does not say how prefill attention reads them.  This
 * library's reading: standard causal attention over the rebuilt blocks.  k_dev, v_dev:
 * [n_kv][Hkv][D] elements of the cache's format (the sequence's first n_kv tokens); q_dev:
 * [n_q][Hq][D] BF16, the queries of positions n_kv - n_q .. n_kv - 1; out_dev: [n_q][Hq][D] BF16
 * (round-to-nearest-even of an fp32 result).  Query i attends tokens 0 .. n_kv - n_q + i with
 * softmax(scale * q . k); query head hq reads KV head hq / (Hq / Hkv).  1 <= n_q <= n_kv; every
 * pointer 16-byte aligned (KVC_EINVAL otherwise).  The cache handle supplies the format and the
 * head geometry only.  Correct for every format and head_dim; not tuned. */
int kv_prefill_attention(kvc_cache* cache, const void* k_dev, const void* v_dev, int32_t n_kv, const void* q_dev,
                         int32_t n_q, float scale, void* out_dev, void* stream);

/* Bytes of workspace kv_decode_attention needs for n_seqs sequences and n_splits splits:
 * fp32 partial outputs [n_seqs][Hq][n_splits][D] and (max, sum) pairs [n_seqs][Hq][n_splits][2]. */
size_t kv_attention_workspace_bytes(const kvc_params* params, int32_t n_seqs, int32_t n_splits);

/* One decode-attention step (GAAC page §3.2) for each listed sequence:
 *   out[s][hq][c] = sum_t softmax_t(scale * q[s][hq] . k_t) v_t[c]
 * over every token of the sequence (finished blocks, compressed or raw, and the tail), with
 * query head hq reading KV head hq / (Hq / Hkv).  q_dev: [n_seqs][Hq][D] BF16; out_dev:
 * [n_seqs][Hq][D] BF16 (round-to-nearest-even of an fp32 result); q, out and the workspace
 * 16-byte aligned (KVC_EINVAL otherwise).  The finished blocks of each
 * sequence are split into n_splits contiguous ranges (of 64-token super-blocks; of blocks for
 * a compressed cache with 8-token groups in 16- or 32-token blocks) processed in parallel
 * (1 <= n_splits <= 1024); their
 * partial results and the tail are merged by log-sum-exp.  Every listed sequence must hold at
 * least one token (KVC_EINVAL otherwise).  With head_dim 256 the split kernel's last split
 * attends the tail and the merge kernel merges the splits only; kv_decode_step then runs as
 * the append followed by this attention. */
int kv_decode_attention(kvc_cache* cache, const int32_t* seq_ids_host, int32_t n_seqs, const void* q_dev,
                        float scale, int32_t n_splits, void* ws_dev, size_t ws_bytes, void* out_dev, void* stream);

/* The two halves of kv_decode_attention, for callers that schedule or time them apart:
 * kv_attention_partials runs the split kernel over the finished blocks and leaves, for every
 * (sequence, query head, split), the unnormalised partial output, the running maximum
 * (base-2 units) and the sum of weights in the workspace; kv_attention_combine attends the
 * tail of each sequence (its tokens not yet in a finished block) and merges it with the splits
 * (log-sum-exp) into out.  Both take the arguments and checks of kv_decode_attention; the
 * sequences, query, scale, split count and workspace must be the same in the two calls, with
 * no append to those sequences between them. */
int kv_attention_partials(kvc_cache* cache, const int32_t* seq_ids_host, int32_t n_seqs, const void* q_dev,
                          float scale, int32_t n_splits, void* ws_dev, size_t ws_bytes, void* stream);
int kv_attention_combine(kvc_cache* cache, const int32_t* seq_ids_host, int32_t n_seqs, const void* q_dev,
                         float scale, int32_t n_splits, const void* ws_dev, size_t ws_bytes, void* out_dev,
                         void* stream);

/* One decode step for each listed sequence: appends its new token (k_new_dev, v_new_dev:
 * [n_seqs][Hkv][D] elements, 16-byte aligned) and evaluates kv_decode_attention over all of its
 * tokens including the new one (GAAC page §3.2 with §3.3's fill-then-finalize), with the result
 * of kv_encode_append(.., n_tokens = 1) followed by kv_decode_attention, bit for bit.  When no
 * listed sequence's new token completes a block, the split kernel stores the new token into the
 * tail while it attends the finished blocks, and the merge kernel attends the tail with it (no
 * separate append launch); otherwise the step is exactly that append (which encodes the
 * finished block) and that attention.  Arguments and checks as kv_encode_append and
 * kv_decode_attention, all made before anything runs. */
int kv_decode_step(kvc_cache* cache, const int32_t* seq_ids_host, int32_t n_seqs, const void* k_new_dev,
                   const void* v_new_dev, const void* q_dev, float scale, int32_t n_splits, void* ws_dev,
                   size_t ws_bytes, void* out_dev, void* stream);

/* Bytes of the fixed split workspace of kv_decode_attention_noalloc (per GPU). */
#define KVC_NOALLOC_WS_BYTES (16u << 20)

/* kv_decode_attention without a caller workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, checks and results as kv_decode_attention (bit for bit: the same kernels), except
 * that the split partials go to a fixed array of KVC_NOALLOC_WS_BYTES inside the library; each
 * GPU the library runs on holds its own copy until the process ends.  Returns KVC_ESMALLWS,
 * with nothing enqueued, when kv_attention_workspace_bytes(params, n_seqs, n_splits) exceeds
 * KVC_NOALLOC_WS_BYTES (with 32 query heads of 128 channels: n_seqs * n_splits <= 1008).  It
 * calls no allocating routine; the array's device address is resolved by kv_cache_create on
 * the device current at that time.  Every call on one GPU shares that GPU's array, which keeps
 * the last call's partials (each call writes every entry it reads, so nothing is cleared):
 * calls ordered on one stream are safe, calls that overlap on one GPU (other streams or host
 * threads without ordering between them) race and give wrong results. */
int kv_decode_attention_noalloc(kvc_cache* cache, const int32_t* seq_ids_host, int32_t n_seqs, const void* q_dev,
                                float scale, int32_t n_splits, void* out_dev, void* stream);

/* Storage statistics of finished blocks first_block .. first_block+n_blocks-1 of one sequence,
 * read on the device from the table entries and the stored tag planes (GAAC page App. C studies
 * escape bytes per tile and raw fallbacks along the context).  out_dev: [n_blocks][2 (K,V)][Hkv]
 * [7] int32 (2 Hkv rows for head_dim 256: one per stored half-head), 4-byte aligned: {state: 0 compressed, 1 raw, -1 unallocated; bytes: FORMAT v1 the
 * escape bytes the tile's tags call for, FORMAT v2 its code bytes, 0 for raw tiles; groups per
 * mode index [4] (compressed tiles); the base version of a compressed tile, else -1}.
 * Enqueued; KVC_EINVAL for blocks past the finished ones. */
int kv_tile_stats(kvc_cache* cache, int32_t seq, int32_t first_block, int32_t n_blocks, int32_t* out_dev,
                  void* stream);

/* Exponent concentration (GAAC page §3.1: most exponents of a head-channel lie in a few
 * consecutive values): for each (kv-head h, channel c) of x_dev [n_tokens][Hkv][D] elements of
 * the cache's format, out_dev[h][c] (int32) = the largest number of its n_tokens exponents
 * inside any window of `window` consecutive exponent values.  1 <= window <= 2^(exponent bits)
 * (KVC_EINVAL otherwise).  Enqueued; the cache supplies the format and geometry only. */
int kv_window_coverage(kvc_cache* cache, const void* x_dev, int32_t n_tokens, int32_t window, int32_t* out_dev,
                       void* stream);

/* Equal-memory admission (GAAC page §4.5: more sequences in the same KV memory): plans the slot
 * pools one layer's budget_bytes buys for caches of these parameters (their slot counts are
 * ignored) and admits requests first come, first served.  A compressed cache spends raw_share
 * of the budget on raw-fallback slots (whole raw tiles) and the rest on compressed slots (slot
 * stride each); an uncompressed cache spends all of it on raw slots.  Requests of
 * lengths_host[0 .. n_requests) tokens are admitted in order while the main pool still holds
 * each one's finished blocks plus one spare block (2 * Hkv slots per block); the first that does
 * not fit stops admission.  Outputs the admitted count and the two pool sizes.  Host only; the
 * budget pays for slots only (tables, tails and counters are not counted). */
int kv_admit_fcfs(const kvc_params* params, uint64_t budget_bytes, double raw_share, const int32_t* lengths_host,
                  int32_t n_requests, int32_t* n_admitted, int32_t* num_comp_slots, int32_t* num_raw_slots);

/* Streaming-read probe, a measurement aid rather than an operation of the page (its case for
 * compressing the cache, GAAC page §1 and §3.2, is that decode attention is bound by reading
 * it): `waves` workgroups of one 64-lane wave, the split attention kernels' launch shape; wave w
 * reads bytes_per_wave contiguous bytes of src_dev from offset w * bytes_per_wave with 16-byte
 * loads, the next 8 KiB batch in flight while the current one is consumed, and writes one
 * checksum word per lane to sink_dev[w * 64 + lane].  Reads waves * bytes_per_wave bytes of
 * src_dev (caller-owned, 16-byte aligned) and writes waves * 64 uint32 words of sink_dev
 * (caller-owned, 4-byte aligned).  bytes_per_wave must be a positive multiple of
 * KVC_READ_PROBE_UNIT and 1 <= waves <= 2^20, else KVC_EINVAL.  Enqueued on stream; time it
 * with events to get the attainable read rate the attention kernels are measured against. */
#define KVC_READ_PROBE_UNIT 8192u
int kv_read_probe(const void* src_dev, uint64_t bytes_per_wave, int32_t waves, uint32_t* sink_dev, void* stream);

/* Returns every slot of a sequence to the free stacks and empties it (enqueued). */
int kv_release_seq(kvc_cache* cache, int32_t seq, void* stream);

/* Current token count of a sequence (host mirror; no GPU access). */
int kv_seq_length(const kvc_cache* cache, int32_t seq, int32_t* length);

/* Synchronises the stream, then reports the sticky status bits and statistics.  Either output
 * pointer may be NULL. */
int kv_get_status(kvc_cache* cache, uint32_t* flags, kvc_stats* stats, void* stream);

/* Message of the calling thread's last failed call ("" if none). */
const char* kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */

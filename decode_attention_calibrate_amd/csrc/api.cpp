// api.cpp -- the C ABI declared in include/kvc.h: argument validation, the host mirror of
// sequence lengths, and kernel launches.  No compute happens here and there is no CPU path:
// every step of the method runs in the HIP kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <array>
#include <new>
#include <string>
#include <vector>

#include "kvc.h"
#include "kvc_internal.h"

using kvc::DevBufs;
using kvc::Geo;
using kvc::SeqList;

struct kvc_cache {
  kvc_params p;
  Geo G;
  DevBufs B;
  std::vector<int32_t> len;  // tokens per sequence (host mirror)
  bool calibrated = false;
  long long blocks = 0;      // finished blocks over all sequences
  // finished blocks per base version, over all sequences and per sequence (a version holding
  // none may be recalibrated); G.cur_ver is the version new blocks are encoded with
  std::array<long long, kvc::kMaxVersions> ver_blocks{};
  std::vector<std::array<long long, kvc::kMaxVersions>> seq_ver_blocks;
  void* noalloc_ws = nullptr;  // this device's fixed split workspace (kv_decode_attention_noalloc)
};

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(int err, const char* what) {
  if (err == 0) return KVC_OK;
  g_err = std::string(what) + ": " + hipGetErrorString((hipError_t)err);
  return KVC_EHIP;
}

// Channels of one stored tile: a 256-channel head is stored as two 128-channel half-heads.
int tile_channels(const kvc_params& p) { return p.head_dim == 256 ? 128 : p.head_dim; }
int esc_cap_of(const kvc_params& p) { return p.esc_cap_bytes < 0 ? p.block_tokens * tile_channels(p) / 16 : p.esc_cap_bytes; }

int check_params(const kvc_params* p) {
  if (!p) return fail(KVC_EINVAL, "params is NULL");
  if (p->dtype < 0 || p->dtype > 2) return fail(KVC_EINVAL, "dtype must be KVC_BF16, KVC_FP8_E5M2 or KVC_FP8_E4M3");
  if (p->num_kv_heads < 1 || p->num_q_heads < 1) return fail(KVC_EINVAL, "head counts must be >= 1");
  if (p->num_q_heads % p->num_kv_heads != 0) return fail(KVC_EINVAL, "num_q_heads must be a multiple of num_kv_heads");
  if (p->num_q_heads / p->num_kv_heads > 16) return fail(KVC_EINVAL, "at most 16 query heads per KV head");
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256)
    return fail(KVC_EINVAL, "head_dim must be 64, 128 or 256");
  if (p->block_tokens < 16 || p->block_tokens % 16 != 0) return fail(KVC_EINVAL, "block_tokens must be a multiple of 16");
  if (p->group_tokens < 1 || p->block_tokens % p->group_tokens != 0)
    return fail(KVC_EINVAL, "group_tokens must divide block_tokens");
  const int cap = esc_cap_of(*p);
  if (cap < 0 || cap % 16 != 0 || cap > 2032) return fail(KVC_EINVAL, "esc_cap_bytes must be a multiple of 16, <= 2032");
  if (p->compressed != 0 && p->compressed != 1) return fail(KVC_EINVAL, "compressed must be 0 or 1");
  if (p->max_seqs < 1 || p->max_blocks_per_seq < 1) return fail(KVC_EINVAL, "max_seqs and max_blocks_per_seq >= 1");
  if (p->num_raw_slots < 0 || p->num_comp_slots < 0) return fail(KVC_EINVAL, "slot counts must be >= 0");
  if (p->num_raw_slots >= kvc::kMaxSlots || p->num_comp_slots >= kvc::kMaxSlots) return fail(KVC_EINVAL, "slot counts < 2^23");
  if (p->base_versions < 0 || p->base_versions > kvc::kMaxVersions) return fail(KVC_EINVAL, "base_versions must be 0 .. 4");
  if (p->compressed && p->num_comp_slots < 1) return fail(KVC_EINVAL, "a compressed cache needs compressed slots");
  if (!p->compressed && p->num_raw_slots < 1) return fail(KVC_EINVAL, "an uncompressed cache needs raw slots");
  // valid requests the library's kernels do not implement
  if (p->group_tokens != 16 && p->group_tokens != 8)
    return fail(KVC_EUNSUPPORTED, "these kernels implement 16- and 8-token groups");
  if (p->block_tokens != 16 && p->block_tokens != 32 && p->block_tokens != 64)
    return fail(KVC_EUNSUPPORTED, "these kernels implement block_tokens 16, 32 or 64");
  // (the table entry's 6-bit escape-length field holds up to 1,008 bytes)
  if (cap > 512) return fail(KVC_EUNSUPPORTED, "these kernels implement esc_cap_bytes <= 512");
  if (p->mode_set < 0 || p->mode_set > 3) return fail(KVC_EINVAL, "mode_set must be 0, 1, 2 or 3");
  if (p->mode_set != 0 && (p->dtype != KVC_BF16 || p->head_dim > 128))
    return fail(KVC_EUNSUPPORTED, "FORMAT v2 mode sets are implemented for BF16 caches with head_dim <= 128");
  return KVC_OK;
}

int align16(int x) { return (x + 15) / 16 * 16; }

Geo make_geo(const kvc_params& p) {
  Geo G;
  memset(&G, 0, sizeof(G));
  G.fmt = p.dtype;
  G.F = p.dtype == KVC_BF16 ? 8 : (p.dtype == KVC_FP8_E5M2 ? 5 : 4);
  G.MB = p.dtype == KVC_BF16 ? 7 : (p.dtype == KVC_FP8_E5M2 ? 2 : 3);
  G.EB = p.dtype == KVC_BF16 ? 2 : 1;
  G.sm_pair = 4 * (1 + G.MB);
  G.T = p.block_tokens;
  // a 256-channel head is stored as two 128-channel half-heads: the same memory as
  // [..][2 Hkv][128], so every kernel sees half-heads
  const int halves = p.head_dim / tile_channels(p);
  G.D = tile_channels(p);
  G.Hkv = p.num_kv_heads * halves;
  G.Hq = p.num_q_heads * halves;
  G.g = p.num_q_heads / p.num_kv_heads;
  G.GT = p.group_tokens;
  G.NT = G.T / G.GT;
  G.NG = G.NT * G.D;
  G.NP = G.NG / 2;
  G.PW = (G.NG + 31) / 32;
  G.tag_off = 0;
  G.code_off = align16(2 * G.PW * 4);
  G.sm_off = G.code_off + align16(G.T * G.D * 3 / 8);
  G.esc_off = G.sm_off + align16(G.T * G.D * (1 + G.MB) / 8);
  G.esc_cap = esc_cap_of(p);
  G.stride = G.esc_off + G.esc_cap;
  G.raw_elems = G.T * G.D;
  G.max_seqs = p.max_seqs;
  G.max_blocks = p.max_blocks_per_seq;
  G.n_comp = p.compressed ? p.num_comp_slots : 0;
  G.n_raw = p.num_raw_slots;
  G.compressed = p.compressed;
  G.mode_set = p.mode_set;
  if (p.mode_set != 0) {  // FORMAT v2: TAG | SM | CODES (each group's offsets at its mode's width)
    static const int widths[4][4] = {{3, 4, 8, 0}, {2, 3, 4, 8}, {4, 8, 0, 0}, {3, 4, 8, 0}};
    static const int counts[4] = {3, 4, 2, 3};
    G.n_modes = counts[p.mode_set];
    for (int k = 0; k < 4; ++k) G.mw[k] = widths[p.mode_set][k];
    G.sm_off = align16(2 * G.PW * 4);
    G.code_off = G.sm_off + align16(G.T * G.D);
    G.code_cap = G.T * G.D * std::max(3, G.mw[0]) / 8 + G.esc_cap;
    G.stride = G.code_off + align16(G.code_cap);
    G.esc_off = G.code_off;
  }
  G.n_versions = std::max(1, p.base_versions);
  G.cur_ver = 0;
  G.ver_bytes = (p.mode_set == 1 ? 6 : 4) * G.Hkv * G.D;
  return G;
}

void sizes_of(const kvc_params& p, const Geo& G, size_t out[KVC_NUM_BUFFERS]) {
  out[0] = (size_t)G.n_comp * G.stride;
  out[1] = (size_t)G.n_raw * G.raw_elems * G.EB;
  out[2] = (size_t)p.max_seqs * 2 * G.Hkv * G.raw_elems * G.EB;
  out[3] = (size_t)G.n_versions * G.ver_bytes;
  out[4] = (size_t)p.max_seqs * p.max_blocks_per_seq * 2 * G.Hkv * 4;
  out[5] = (size_t)G.n_comp * 4;
  out[6] = (size_t)G.n_raw * 4;
  out[7] = kvc::kCountersBytes;
}

uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

std::vector<int32_t> permutation(int n, uint64_t seed) {
  std::vector<int32_t> v(n);
  for (int i = 0; i < n; ++i) v[i] = i;
  uint64_t s = seed;
  for (int i = n - 1; i > 0; --i) {
    const int k = (int)(splitmix64(s) % (uint64_t)(i + 1));
    std::swap(v[i], v[k]);
  }
  return v;
}

// The free-stack array for a permuted pool: the slots of sub-stack s (those equal to s modulo
// kPoolStripes) keep their order in perm and go to indices s, s + 16, s + 32, ...
std::vector<int32_t> stack_layout(const std::vector<int32_t>& perm) {
  std::vector<int32_t> out(perm.size());
  int next[kvc::kPoolStripes] = {};
  for (int32_t slot : perm) {
    const int s = slot % kvc::kPoolStripes;
    out[(size_t)kvc::kPoolStripes * next[s]++ + s] = slot;
  }
  return out;
}

int check_seq_ids(const kvc_cache* c, const int32_t* ids, int n) {
  if (!ids || n < 1) return fail(KVC_EINVAL, "seq_ids must list at least one sequence");
  std::vector<char> seen(c->p.max_seqs, 0);
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= c->p.max_seqs) return fail(KVC_EINVAL, "sequence id out of range");
    if (seen[ids[i]]) return fail(KVC_EINVAL, "sequence ids must be distinct");
    seen[ids[i]] = 1;
  }
  return KVC_OK;
}

}  // namespace

extern "C" {

int kv_buffer_sizes(const kvc_params* params, size_t* out_bytes, size_t* slot_stride) {
  const int rc = check_params(params);
  if (rc != KVC_OK) return rc;
  if (!out_bytes) return fail(KVC_EINVAL, "out_bytes is NULL");
  const Geo G = make_geo(*params);
  sizes_of(*params, G, out_bytes);
  if (slot_stride) *slot_stride = (size_t)G.stride;
  return KVC_OK;
}

int kv_cache_create(const kvc_params* params, const kvc_buffers* buffers, uint64_t perm_seed, void* stream,
                    kvc_cache** out) {
  int rc = check_params(params);
  if (rc != KVC_OK) return rc;
  if (!buffers || !out) return fail(KVC_EINVAL, "buffers and out must not be NULL");
  *out = nullptr;
  const Geo G = make_geo(*params);
  size_t sz[KVC_NUM_BUFFERS];
  sizes_of(*params, G, sz);
  void* const ptrs[KVC_NUM_BUFFERS] = {buffers->comp_pool, buffers->raw_pool, buffers->tail, buffers->bases,
                                       buffers->block_table, buffers->comp_free, buffers->raw_free,
                                       buffers->counters};
  for (int i = 0; i < KVC_NUM_BUFFERS; ++i) {
    if (sz[i] > 0 && !ptrs[i]) return fail(KVC_EINVAL, "a required device buffer is NULL");
    if (ptrs[i] && ((uintptr_t)ptrs[i] & 15u)) return fail(KVC_EINVAL, "device buffers must be 16-byte aligned");
  }
  kvc_cache* c = new (std::nothrow) kvc_cache;
  if (!c) return fail(KVC_EINVAL, "out of host memory");
  c->p = *params;
  c->G = G;
  c->B.comp_pool = (uint8_t*)buffers->comp_pool;
  c->B.raw_pool = (uint16_t*)buffers->raw_pool;
  c->B.tail = (uint16_t*)buffers->tail;
  c->B.bases = (uint8_t*)buffers->bases;
  c->B.table = (uint32_t*)buffers->block_table;
  c->B.comp_free = (int32_t*)buffers->comp_free;
  c->B.raw_free = (int32_t*)buffers->raw_free;
  c->B.counters = (kvc::Counters*)buffers->counters;
  c->len.assign(params->max_seqs, 0);
  c->seq_ver_blocks.assign(params->max_seqs, std::array<long long, kvc::kMaxVersions>{});
  hipStream_t st = (hipStream_t)stream;
  if (G.n_comp > 0) {
    const std::vector<int32_t> perm = stack_layout(permutation(G.n_comp, perm_seed));
    rc = hip_fail((int)hipMemcpyAsync(c->B.comp_free, perm.data(), perm.size() * 4, hipMemcpyHostToDevice, st),
                  "copy compressed free stack");
    if (rc == KVC_OK) rc = hip_fail((int)hipStreamSynchronize(st), "synchronise");
  }
  if (rc == KVC_OK && G.n_raw > 0) {
    const std::vector<int32_t> perm = stack_layout(permutation(G.n_raw, perm_seed ^ 0x5A5A5A5A5A5A5A5Aull));
    rc = hip_fail((int)hipMemcpyAsync(c->B.raw_free, perm.data(), perm.size() * 4, hipMemcpyHostToDevice, st),
                  "copy raw free stack");
    if (rc == KVC_OK) rc = hip_fail((int)hipStreamSynchronize(st), "synchronise");
  }
  if (rc == KVC_OK) rc = hip_fail(kvc::launch_init(G, c->B, nullptr, nullptr, stream), "launch init");
  if (rc == KVC_OK) rc = hip_fail((int)hipStreamSynchronize(st), "synchronise");
  // the fixed workspace of kv_decode_attention_noalloc on this (the current) device; a failure
  // here is reported by that entry point, which resolves it again
  if (rc == KVC_OK && kvc::noalloc_workspace(&c->noalloc_ws) != 0) c->noalloc_ws = nullptr;
  if (rc != KVC_OK) {
    delete c;
    return rc;
  }
  *out = c;
  return KVC_OK;
}

void kv_cache_destroy(kvc_cache* cache) { delete cache; }

int kv_calibrate(kvc_cache* c, const void* k_dev, const void* v_dev, int32_t n_tokens, void* stream) {
  if (!c) return fail(KVC_EINVAL, "cache is NULL");
  if (!k_dev || !v_dev || n_tokens < 1) return fail(KVC_EINVAL, "calibration needs K and V with n_tokens >= 1");
  if (c->blocks > 0) return fail(KVC_ESTATE, "calibration must precede the first finished block");
  c->G.cur_ver = 0;
  const int rc = hip_fail(kvc::launch_calibrate(c->G, c->B, k_dev, v_dev, n_tokens, stream),
                          "launch calibrate");
  if (rc == KVC_OK) c->calibrated = true;
  return rc;
}

int kv_recalibrate(kvc_cache* c, const void* k_dev, const void* v_dev, int32_t n_tokens, void* stream) {
  if (!c) return fail(KVC_EINVAL, "cache is NULL");
  if (!k_dev || !v_dev || n_tokens < 1) return fail(KVC_EINVAL, "recalibration needs K and V with n_tokens >= 1");
  if (!c->calibrated) return fail(KVC_ESTATE, "kv_calibrate must run before kv_recalibrate");
  int next = -1;
  for (int d = 1; d < c->G.n_versions && next < 0; ++d) {
    const int v = (c->G.cur_ver + d) % c->G.n_versions;
    if (c->ver_blocks[v] == 0) next = v;
  }
  if (next < 0)
    return fail(KVC_ESTATE, c->G.n_versions == 1 ? "the cache holds one base version (base_versions = 1)"
                                                  : "every other base version still holds live blocks");
  Geo G = c->G;
  G.cur_ver = next;
  const int rc = hip_fail(kvc::launch_calibrate(G, c->B, k_dev, v_dev, n_tokens, stream), "launch calibrate");
  if (rc == KVC_OK) c->G.cur_ver = next;
  return rc;
}

int kv_encode_append(kvc_cache* c, const int32_t* seq_ids_host, int32_t n_seqs, const void* k_dev, const void* v_dev,
                     int32_t n_tokens, void* stream) {
  if (!c) return fail(KVC_EINVAL, "cache is NULL");
  int rc = check_seq_ids(c, seq_ids_host, n_seqs);
  if (rc != KVC_OK) return rc;
  if (!k_dev || !v_dev || n_tokens < 1) return fail(KVC_EINVAL, "append needs K and V with n_tokens >= 1");
  if (((uintptr_t)k_dev & 15u) || ((uintptr_t)v_dev & 15u)) return fail(KVC_EINVAL, "K and V must be 16-byte aligned");
  const int T = c->G.T;
  long long new_blocks = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const long long L1 = (long long)c->len[seq_ids_host[i]] + n_tokens;
    if (L1 / T > c->p.max_blocks_per_seq) return fail(KVC_ENOSLOT, "sequence would exceed max_blocks_per_seq");
    if (L1 > INT32_MAX) return fail(KVC_EINVAL, "sequence too long");
    new_blocks += L1 / T - c->len[seq_ids_host[i]] / T;
  }
  if (new_blocks > 0 && c->p.compressed && !c->calibrated)
    return fail(KVC_ESTATE, "kv_calibrate must run before the first block is encoded");
  const size_t row = (size_t)c->G.Hkv * c->G.D;
  for (int s0 = 0; s0 < n_seqs; s0 += kvc::kMaxSeqsPerLaunch) {
    SeqList S;
    S.n = std::min(kvc::kMaxSeqsPerLaunch, n_seqs - s0);
    int max_new = 0;
    for (int i = 0; i < S.n; ++i) {
      const int id = seq_ids_host[s0 + i];
      S.ids[i] = id;
      S.lens[i] = c->len[id];
      max_new = std::max(max_new, (c->len[id] + n_tokens) / T - c->len[id] / T);
    }
    const uint8_t* k = (const uint8_t*)k_dev + (size_t)s0 * n_tokens * row * c->G.EB;
    const uint8_t* v = (const uint8_t*)v_dev + (size_t)s0 * n_tokens * row * c->G.EB;
    rc = hip_fail(kvc::launch_append(c->G, c->B, S, k, v, n_tokens, max_new, stream), "launch append");
    if (rc != KVC_OK) return rc;
  }
  for (int i = 0; i < n_seqs; ++i) {
    const int id = seq_ids_host[i];
    const long long nb = ((long long)c->len[id] + n_tokens) / T - c->len[id] / T;
    c->seq_ver_blocks[id][c->G.cur_ver] += nb;
    c->ver_blocks[c->G.cur_ver] += nb;
    c->len[id] += n_tokens;
  }
  c->blocks += new_blocks;
  return KVC_OK;
}

int kv_decode_blocks(kvc_cache* c, int32_t seq, int32_t first_block, int32_t n_blocks, void* k_out_dev,
                     void* v_out_dev, void* stream) {
  if (!c) return fail(KVC_EINVAL, "cache is NULL");
  if (seq < 0 || seq >= c->p.max_seqs) return fail(KVC_EINVAL, "sequence id out of range");
  if (!k_out_dev || !v_out_dev || first_block < 0 || n_blocks < 1) return fail(KVC_EINVAL, "bad block range");
  if (first_block + n_blocks > c->len[seq] / c->G.T) return fail(KVC_EINVAL, "blocks past the finished blocks");
  if (((uintptr_t)k_out_dev & 15u) || ((uintptr_t)v_out_dev & 15u))
    return fail(KVC_EINVAL, "k_out and v_out must be 16-byte aligned");
  return hip_fail(kvc::launch_decode_blocks(c->G, c->B, seq, first_block, n_blocks, k_out_dev, v_out_dev, stream),
                  "launch decode_blocks");
}

int kv_prefill_attention(kvc_cache* c, const void* k_dev, const void* v_dev, int32_t n_kv, const void* q_dev,
                         int32_t n_q, float scale, void* out_dev, void* stream) {
  if (!c) return fail(KVC_EINVAL, "cache is NULL");
  if (!k_dev || !v_dev || !q_dev || !out_dev) return fail(KVC_EINVAL, "k, v, q and out must not be NULL");
  if (n_q < 1 || n_q > n_kv) return fail(KVC_EINVAL, "need 1 <= n_q <= n_kv");
  for (const void* p : {k_dev, v_dev, q_dev, (const void*)out_dev})
    if ((uintptr_t)p & 15u) return fail(KVC_EINVAL, "k, v, q and out must be 16-byte aligned");
  Geo G = c->G;  // the real head layout (a 256-channel head is not split here)
  G.D = c->p.head_dim;
  G.Hkv = c->p.num_kv_heads;
  G.Hq = c->p.num_q_heads;
  return hip_fail(kvc::launch_prefill(G, k_dev, v_dev, n_kv, (const uint16_t*)q_dev, n_q, scale, (uint16_t*)out_dev,
                                      stream),
                  "launch prefill attention");
}

size_t kv_attention_workspace_bytes(const kvc_params* p, int32_t n_seqs, int32_t n_splits) {
  if (!p || n_seqs < 1 || n_splits < 1) return 0;
  return (size_t)n_seqs * p->num_q_heads * n_splits * ((size_t)p->head_dim + 2) * 4;
}

// Shared argument checks of the attention calls.
static int check_attention_args(kvc_cache* c, const int32_t* seq_ids_host, int32_t n_seqs, const void* q_dev,
                                int32_t n_splits, const void* ws_dev, size_t ws_bytes) {
  if (!c) return fail(KVC_EINVAL, "cache is NULL");
  int rc = check_seq_ids(c, seq_ids_host, n_seqs);
  if (rc != KVC_OK) return rc;
  if (!q_dev || !ws_dev) return fail(KVC_EINVAL, "q and workspace must not be NULL");
  if (n_splits < 1 || n_splits > 1024) return fail(KVC_EINVAL, "n_splits must be in 1..1024");
  if (ws_bytes < kv_attention_workspace_bytes(&c->p, n_seqs, n_splits))
    return fail(KVC_ESMALLWS, "workspace smaller than kv_attention_workspace_bytes()");
  if (((uintptr_t)ws_dev & 15u) || ((uintptr_t)q_dev & 15u)) return fail(KVC_EINVAL, "q and workspace must be 16-byte aligned");
  for (int i = 0; i < n_seqs; ++i)
    if (c->len[seq_ids_host[i]] < 1) return fail(KVC_EINVAL, "every listed sequence needs at least one token");
  return KVC_OK;
}

static int check_out(const void* out_dev) {
  if (!out_dev) return fail(KVC_EINVAL, "out must not be NULL");
  if ((uintptr_t)out_dev & 15u) return fail(KVC_EINVAL, "out must be 16-byte aligned");
  return KVC_OK;
}

// The split kernel over the finished blocks of every listed sequence (argument checks done by the
// caller).  k_new / v_new (a decode step, else null): the new token of each sequence, already
// counted in c->len, which the kernel stores into the tail.
static int run_partials(kvc_cache* c, const int32_t* seq_ids_host, int32_t n_seqs, const void* q_dev, float scale,
                        int32_t n_splits, void* ws_dev, const void* k_new_dev, const void* v_new_dev, void* stream) {
  int rc = KVC_OK;
  const Geo& G = c->G;
  const size_t row = (size_t)G.Hkv * G.D * G.EB;  // bytes of one token of all KV heads
  const size_t hq = c->p.num_q_heads;             // query heads (G.Hq counts half-heads)
  float* acc = (float*)ws_dev;
  float* ml = acc + (size_t)n_seqs * G.Hq * n_splits * G.D;
  for (int s0 = 0; s0 < n_seqs; s0 += kvc::kMaxSeqsPerLaunch) {
    SeqList S;
    int new_pos[kvc::kMaxSeqsPerLaunch];
    S.n = std::min(kvc::kMaxSeqsPerLaunch, n_seqs - s0);
    for (int i = 0; i < S.n; ++i) {
      S.ids[i] = seq_ids_host[s0 + i];
      S.lens[i] = c->len[S.ids[i]] / G.T * G.T;  // the finished blocks; the merge adds the tail
      new_pos[i] = c->len[S.ids[i]] % G.T - 1;   // a decode step's token: the tail's last position
    }
    if (c->p.head_dim == 256) {  // half-head pairs; the kernel attends the tail too
      int ntail[kvc::kMaxSeqsPerLaunch];
      for (int i = 0; i < S.n; ++i) ntail[i] = c->len[S.ids[i]] % G.T;
      rc = hip_fail(kvc::launch_attention_half(G, c->B, S, ntail, (const uint16_t*)q_dev + (size_t)s0 * G.Hq * G.D, scale,
                                               n_splits, acc + (size_t)s0 * G.Hq * n_splits * G.D,
                                               ml + (size_t)s0 * hq * n_splits * 2, stream),
                    "launch attention");
      if (rc != KVC_OK) return rc;
      continue;
    }
    // compressed caches in FORMAT v2, or with 8-token groups in blocks other than 64 tokens, take
    // the LDS-rebuild kernel; everything else the register-rebuild split kernels
    auto launch = (G.compressed && (G.mode_set != 0 || (G.GT != kvc::kGroup && G.T != 64)))
                      ? kvc::launch_attention_any
                      : kvc::launch_attention_partials;
    rc = hip_fail(launch(G, c->B, S, (const uint16_t*)q_dev + (size_t)s0 * G.Hq * G.D, scale, n_splits,
                         acc + (size_t)s0 * G.Hq * n_splits * G.D, ml + (size_t)s0 * hq * n_splits * 2,
                         k_new_dev ? (const uint8_t*)k_new_dev + (size_t)s0 * row : nullptr,
                         v_new_dev ? (const uint8_t*)v_new_dev + (size_t)s0 * row : nullptr, new_pos, stream),
                  "launch attention");
    if (rc != KVC_OK) return rc;
  }
  return KVC_OK;
}

int kv_attention_partials(kvc_cache* c, const int32_t* seq_ids_host, int32_t n_seqs, const void* q_dev, float scale,
                          int32_t n_splits, void* ws_dev, size_t ws_bytes, void* stream) {
  int rc = check_attention_args(c, seq_ids_host, n_seqs, q_dev, n_splits, ws_dev, ws_bytes);
  if (rc != KVC_OK) return rc;
  return run_partials(c, seq_ids_host, n_seqs, q_dev, scale, n_splits, ws_dev, nullptr, nullptr, stream);
}

int kv_attention_combine(kvc_cache* c, const int32_t* seq_ids_host, int32_t n_seqs, const void* q_dev, float scale,
                         int32_t n_splits, const void* ws_dev, size_t ws_bytes, void* out_dev, void* stream) {
  int rc = check_attention_args(c, seq_ids_host, n_seqs, q_dev, n_splits, ws_dev, ws_bytes);
  if (rc != KVC_OK) return rc;
  rc = check_out(out_dev);
  if (rc != KVC_OK) return rc;
  // 256-channel heads: the real head geometry, and no tail (the split kernel attended it)
  const bool wide = c->p.head_dim == 256;
  Geo G = c->G;
  if (wide) {
    G.D = 256;
    G.Hkv = c->p.num_kv_heads;
    G.Hq = c->p.num_q_heads;
    G.raw_elems = G.T * G.D;
  }
  const float* acc = (const float*)ws_dev;
  const float* ml = acc + (size_t)n_seqs * G.Hq * n_splits * G.D;
  for (int s0 = 0; s0 < n_seqs; s0 += kvc::kMaxSeqsPerLaunch) {
    SeqList S;
    S.n = std::min(kvc::kMaxSeqsPerLaunch, n_seqs - s0);
    for (int i = 0; i < S.n; ++i) {
      S.ids[i] = seq_ids_host[s0 + i];
      S.lens[i] = wide ? c->len[S.ids[i]] / G.T * G.T : c->len[S.ids[i]];
    }
    rc = hip_fail(kvc::launch_combine(G, c->B, S, (const uint16_t*)q_dev + (size_t)s0 * G.Hq * G.D, scale, n_splits,
                                      acc + (size_t)s0 * G.Hq * n_splits * G.D, ml + (size_t)s0 * G.Hq * n_splits * 2,
                                      (uint16_t*)out_dev + (size_t)s0 * G.Hq * G.D, stream),
                  "launch combine");
    if (rc != KVC_OK) return rc;
  }
  return KVC_OK;
}

int kv_decode_attention(kvc_cache* c, const int32_t* seq_ids_host, int32_t n_seqs, const void* q_dev, float scale,
                        int32_t n_splits, void* ws_dev, size_t ws_bytes, void* out_dev, void* stream) {
  if (check_out(out_dev) != KVC_OK) return KVC_EINVAL;
  const int rc = kv_attention_partials(c, seq_ids_host, n_seqs, q_dev, scale, n_splits, ws_dev, ws_bytes, stream);
  if (rc != KVC_OK) return rc;
  return kv_attention_combine(c, seq_ids_host, n_seqs, q_dev, scale, n_splits, ws_dev, ws_bytes, out_dev, stream);
}

int kv_decode_attention_noalloc(kvc_cache* c, const int32_t* seq_ids_host, int32_t n_seqs, const void* q_dev,
                                float scale, int32_t n_splits, void* out_dev, void* stream) {
  if (!c) return fail(KVC_EINVAL, "cache is NULL");
  if (n_seqs < 1 || n_splits < 1) return fail(KVC_EINVAL, "n_seqs and n_splits must be >= 1");
  if (kv_attention_workspace_bytes(&c->p, n_seqs, n_splits) > (size_t)KVC_NOALLOC_WS_BYTES)
    return fail(KVC_ESMALLWS, "n_seqs x n_splits needs more workspace than the fixed " +
                                  std::to_string(KVC_NOALLOC_WS_BYTES) + " bytes of kv_decode_attention_noalloc");
  if (!c->noalloc_ws) {
    const int rc = hip_fail(kvc::noalloc_workspace(&c->noalloc_ws), "resolve the fixed workspace");
    if (rc != KVC_OK) return rc;
  }
  return kv_decode_attention(c, seq_ids_host, n_seqs, q_dev, scale, n_splits, c->noalloc_ws, KVC_NOALLOC_WS_BYTES,
                             out_dev, stream);
}

int kv_decode_step(kvc_cache* c, const int32_t* seq_ids_host, int32_t n_seqs, const void* k_new_dev,
                   const void* v_new_dev, const void* q_dev, float scale, int32_t n_splits, void* ws_dev, size_t ws_bytes,
                   void* out_dev, void* stream) {
  if (!c) return fail(KVC_EINVAL, "cache is NULL");
  int rc = check_seq_ids(c, seq_ids_host, n_seqs);
  if (rc != KVC_OK) return rc;
  if (!k_new_dev || !v_new_dev) return fail(KVC_EINVAL, "k_new and v_new must not be NULL");
  rc = check_out(out_dev);
  if (rc != KVC_OK) return rc;
  if (((uintptr_t)k_new_dev & 15u) || ((uintptr_t)v_new_dev & 15u))
    return fail(KVC_EINVAL, "k_new and v_new must be 16-byte aligned");
  const Geo& G = c->G;
  for (int i = 0; i < n_seqs; ++i)
    if (c->len[seq_ids_host[i]] >= INT32_MAX - 1) return fail(KVC_EINVAL, "sequence too long");
  // the attention arguments are checked against the lengths after the append, before anything runs
  for (int i = 0; i < n_seqs; ++i) c->len[seq_ids_host[i]] += 1;
  rc = check_attention_args(c, seq_ids_host, n_seqs, q_dev, n_splits, ws_dev, ws_bytes);
  for (int i = 0; i < n_seqs; ++i) c->len[seq_ids_host[i]] -= 1;
  if (rc != KVC_OK) return rc;
  // does this token finish a block of some listed sequence?  (256-channel heads: the kernel
  // that attends them reads the tail itself, so the token is always appended first)
  bool completes = c->p.head_dim == 256;
  for (int i = 0; i < n_seqs; ++i) completes |= (c->len[seq_ids_host[i]] + 1) % G.T == 0;
  if (completes) {  // the block must be encoded first: the append, then both attention halves
    rc = kv_encode_append(c, seq_ids_host, n_seqs, k_new_dev, v_new_dev, 1, stream);
    if (rc != KVC_OK) return rc;
    return kv_decode_attention(c, seq_ids_host, n_seqs, q_dev, scale, n_splits, ws_dev, ws_bytes, out_dev, stream);
  }
  // the finished blocks do not change: the split kernel attends them as they are and stores the
  // new token into the tail; the merge then attends the tail with the new token in it
  for (int i = 0; i < n_seqs; ++i) c->len[seq_ids_host[i]] += 1;
  rc = run_partials(c, seq_ids_host, n_seqs, q_dev, scale, n_splits, ws_dev, k_new_dev, v_new_dev, stream);
  if (rc == KVC_OK) rc = kv_attention_combine(c, seq_ids_host, n_seqs, q_dev, scale, n_splits, ws_dev, ws_bytes, out_dev, stream);
  if (rc != KVC_OK)
    for (int i = 0; i < n_seqs; ++i) c->len[seq_ids_host[i]] -= 1;
  return rc;
}

int kv_tile_stats(kvc_cache* c, int32_t seq, int32_t first_block, int32_t n_blocks, int32_t* out_dev, void* stream) {
  if (!c) return fail(KVC_EINVAL, "cache is NULL");
  if (seq < 0 || seq >= c->p.max_seqs) return fail(KVC_EINVAL, "sequence id out of range");
  if (!out_dev || first_block < 0 || n_blocks < 1) return fail(KVC_EINVAL, "bad block range");
  if (first_block + n_blocks > c->len[seq] / c->G.T) return fail(KVC_EINVAL, "blocks past the finished blocks");
  if ((uintptr_t)out_dev & 3u) return fail(KVC_EINVAL, "out must be 4-byte aligned");
  return hip_fail(kvc::launch_tile_stats(c->G, c->B, seq, first_block, n_blocks, out_dev, stream), "launch tile stats");
}

int kv_window_coverage(kvc_cache* c, const void* x_dev, int32_t n_tokens, int32_t window, int32_t* out_dev,
                       void* stream) {
  if (!c) return fail(KVC_EINVAL, "cache is NULL");
  if (!x_dev || !out_dev || n_tokens < 1) return fail(KVC_EINVAL, "coverage needs x, out and n_tokens >= 1");
  if (window < 1 || window > (1 << c->G.F)) return fail(KVC_EINVAL, "window must be in 1 .. 2^(exponent bits)");
  if ((uintptr_t)out_dev & 3u) return fail(KVC_EINVAL, "out must be 4-byte aligned");
  return hip_fail(kvc::launch_coverage(c->G, x_dev, n_tokens, window, out_dev, stream), "launch coverage");
}

int kv_read_probe(const void* src_dev, uint64_t bytes_per_wave, int32_t waves, uint32_t* sink_dev, void* stream) {
  if (!src_dev || !sink_dev) return fail(KVC_EINVAL, "read probe needs src and sink");
  if (((uintptr_t)src_dev & 15u) || ((uintptr_t)sink_dev & 3u)) return fail(KVC_EINVAL, "src must be 16-byte, sink 4-byte aligned");
  if (bytes_per_wave == 0 || bytes_per_wave % KVC_READ_PROBE_UNIT) return fail(KVC_EINVAL, "bytes_per_wave must be a positive multiple of 8192");
  if (waves < 1 || waves > (1 << 20)) return fail(KVC_EINVAL, "waves must be in 1 .. 2^20");
  return hip_fail(kvc::launch_read_probe(src_dev, (size_t)bytes_per_wave, waves, sink_dev, stream), "launch read probe");
}

int kv_admit_fcfs(const kvc_params* params, uint64_t budget_bytes, double raw_share, const int32_t* lengths_host,
                  int32_t n_requests, int32_t* n_admitted, int32_t* num_comp_slots, int32_t* num_raw_slots) {
  if (!params || !n_admitted || !num_comp_slots || !num_raw_slots) return fail(KVC_EINVAL, "NULL argument");
  if (n_requests < 0 || (n_requests > 0 && !lengths_host)) return fail(KVC_EINVAL, "bad request list");
  if (!(raw_share >= 0.0 && raw_share <= 1.0)) return fail(KVC_EINVAL, "raw_share must be in [0, 1]");
  kvc_params p = *params;  // slot counts are what this call plans: any valid value passes the checks
  p.num_comp_slots = p.num_raw_slots = 1;
  const int rc = check_params(&p);
  if (rc != KVC_OK) return rc;
  const Geo G = make_geo(p);
  const uint64_t raw_tile = (uint64_t)G.raw_elems * G.EB, tiles_per_block = 2ull * G.Hkv;
  uint64_t n_raw, n_comp;
  if (p.compressed) {
    n_raw = (uint64_t)((double)budget_bytes * raw_share) / raw_tile;
    n_comp = (budget_bytes - n_raw * raw_tile) / (uint64_t)G.stride;
  } else {
    n_raw = budget_bytes / raw_tile;
    n_comp = 0;
  }
  if (n_raw >= (uint64_t)kvc::kMaxSlots || n_comp >= (uint64_t)kvc::kMaxSlots) return fail(KVC_EINVAL, "budget exceeds 2^23 slots per pool");
  uint64_t free_slots = p.compressed ? n_comp : n_raw;
  int admitted = 0;
  for (; admitted < n_requests; ++admitted) {
    const int32_t L = lengths_host[admitted];
    if (L < 1) return fail(KVC_EINVAL, "request lengths must be >= 1");
    const uint64_t need = ((uint64_t)L / G.T + 1) * tiles_per_block;  // its finished blocks + one spare block
    if (need > free_slots) break;                                     // first come, first served: stop here
    free_slots -= need;
  }
  *n_admitted = admitted;
  *num_comp_slots = (int32_t)n_comp;
  *num_raw_slots = (int32_t)n_raw;
  return KVC_OK;
}

int kv_release_seq(kvc_cache* c, int32_t seq, void* stream) {
  if (!c) return fail(KVC_EINVAL, "cache is NULL");
  if (seq < 0 || seq >= c->p.max_seqs) return fail(KVC_EINVAL, "sequence id out of range");
  const int nb = c->len[seq] / c->G.T;
  const int rc = hip_fail(kvc::launch_release(c->G, c->B, seq, nb, stream), "launch release");
  if (rc == KVC_OK) {
    c->blocks -= nb;
    c->len[seq] = 0;
    for (int v = 0; v < kvc::kMaxVersions; ++v) {
      c->ver_blocks[v] -= c->seq_ver_blocks[seq][v];
      c->seq_ver_blocks[seq][v] = 0;
    }
  }
  return rc;
}

int kv_seq_length(const kvc_cache* c, int32_t seq, int32_t* length) {
  if (!c || !length) return fail(KVC_EINVAL, "cache and length must not be NULL");
  if (seq < 0 || seq >= c->p.max_seqs) return fail(KVC_EINVAL, "sequence id out of range");
  *length = c->len[seq];
  return KVC_OK;
}

int kv_get_status(kvc_cache* c, uint32_t* flags, kvc_stats* stats, void* stream) {
  if (!c) return fail(KVC_EINVAL, "cache is NULL");
  kvc::Counters h;
  hipStream_t st = (hipStream_t)stream;
  int rc = hip_fail((int)hipMemcpyAsync(&h, c->B.counters, sizeof(h), hipMemcpyDeviceToHost, st), "read counters");
  if (rc == KVC_OK) rc = hip_fail((int)hipStreamSynchronize(st), "synchronise");
  if (rc != KVC_OK) return rc;
  if (flags) *flags = h.status;
  if (stats) {
    *stats = kvc_stats{};
    for (const kvc::StatStripe& st : h.stat) {
      stats->raw_tiles += st.raw_tiles;
      for (int i = 0; i < 4; ++i) stats->groups[i] += st.groups[i];
      stats->esc_bytes += st.esc_bytes;
    }
    // every compressed tile adds exactly NG groups
    stats->comp_tiles = (stats->groups[0] + stats->groups[1] + stats->groups[2] + stats->groups[3]) / (uint64_t)c->G.NG;
    stats->comp_free = stats->raw_free = 0;
    for (int s = 0; s < kvc::kPoolStripes; ++s) {
      stats->comp_free += h.comp_top[s].n;
      stats->raw_free += h.raw_top[s].n;
    }
  }
  return KVC_OK;
}

const char* kv_last_error(void) { return g_err.c_str(); }

}  // extern "C"

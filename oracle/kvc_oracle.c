/*
 * kvc_oracle.c -- plain CPU oracle for the lossless KV-cache codec and for exact decode
 * attention.  TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg are the only code allowed to load it.  It shares no code, header, table
 * or helper with the HIP library, and the HIP library never calls it.
 *
 * Method followed (page "GAAC: Lossless KV Compression for Bandwidth-Efficient LLM Inference
 * on Personal Devices", paperlayer.ai summary of arXiv:2610.38210v1):
 *   - §3.1: exponents are coded as calibrated per-(head, channel) base plus offset over
 *     contiguous windows of 8 and 16 values; each small group picks a 3-bit, 4-bit or raw
 *     exponent mode according to whether its offsets fit; a value outside the window widens
 *     the whole group (no per-value exceptions); sign and mantissa bits are kept unchanged.
 *   - §3.3 / Figure 3: a finished block is encoded once into a fixed-capacity slot; a block
 *     whose encoding does not fit stays in its native (uncompressed) form.
 *   - App. D: the stored pieces are 3-bit exponent codes, 2-bit mode tags, escape bytes held
 *     in a fixed-capacity escape area, and block-table entries.
 *   - App. B: the same codec applies to FP8 E5M2 / E4M3 caches.
 * The pages print no byte layout.  The layout below ("FORMAT v1") is this library's reading;
 * every choice is stated below.  The oracle writes each field bit by bit at the
 * position the format defines, with no blocking or fusion, so it can be checked by eye.
 *
 * FORMAT v1 for one tile = T tokens x D channels of one (K|V, kv-head), element = F exponent
 * bits, MB mantissa bits, 1 sign bit:
 *   groups      q = tg*D + c covers tokens tg*G .. tg*G+G-1 of channel c (tg < T/G);
 *               element (q, tau) is token tg*G+tau, channel c, element index n = q*G + tau.
 *   modes       0 narrow (width 3, base b3[c]); 1 wide (width 4, base b4[c]; only if F > 4);
 *               2 raw (width F, base 0).  Offset o = e - base; code = o & 7.
 *   TAG         two bit planes of N_G bits (plane E: mode >= 1, plane R: mode == 2), each
 *               padded to whole 32-bit words; (E=0, R=1) is invalid.
 *   CODE        3-bit code of every element.  Units of 32 elements (12 bytes): element
 *               n = 32u + r sits in byte-lane k = r % 4 at slot s = r / 4; bit b of its field
 *               is bit x = 3s + b of lane k's 24-bit stream, stored in byte 4*(x/8) + k of the
 *               unit, bit x % 8.
 *   SM          sign and mantissa, (1+MB)-bit field (s << MB) | m per element:
 *               BF16 one byte per element; E5M2 3-bit fields in the CODE unit layout;
 *               E4M3 4-bit fields, element n in bits 4n..4n+3 (LSB-first).
 *   ESC         for each group with mode >= 1 in increasing q, in an LSB-first bit stream:
 *               first one bit plane of G bits holding bit 3 of every offset (bit tau = token
 *               tau); then, for a raw group, the remaining F-4 bits of each offset: for BF16
 *               (F = 8) as one 4-bit field per element (offset bits 4..7 of token tau at
 *               bits 4*tau .. 4*tau+3), for F = 5 as one more plane (bit 4).  A group thus
 *               uses (w - 3) * G bits.  Unused bytes up to esc_cap are zero.
 *   sections    TAG | CODE | SM | ESC, each starting 16-byte aligned; slot stride = sum of
 *               the four 16-aligned section sizes (ESC counted at esc_cap).
 *   fallback    if the escape planes need more than esc_cap bytes, the tile is RAW: native
 *               elements, K tiles token-major [t][c], V tiles channel-major [c][t].
 *
 * FORMAT v2 ("orc_v2_*", BF16 only) -- the nested precision modes of §4.7.2 / Table 4: other
 * sets of exponent modes, each group storing its offsets at its own mode's width:
 *   mode sets   1: widths {2, 3, 4, 8} (a 2-bit mode added), 2: {4, 8} (no 3-bit mode),
 *               3: {3, 4, 8} (the v1 modes in the v2 layout).  Mode k has width W[k] and base
 *               b_W[c] (a calibrated window of 2^W exponents), the last mode is raw (base 0).
 *               A group takes the first mode whose window holds all its exponents.
 *   TAG         two bit planes of N_G bits: plane 0 bit 0 of k, plane 1 bit 1 of k (words).
 *   SM          one byte (s << 7) | m per element, as v1.
 *   CODES       one LSB-first bit stream: the groups in q order, each holding its G offsets in
 *               token order at W_q bits each (element tau of group q at bit O_q + tau * W_q,
 *               O_q = G * sum of W over the earlier groups).  Capacity: every offset at
 *               max(3, narrowest width) bits plus esc_cap bytes (v1's CODE plus ESC bytes for
 *               the sets with a 3-bit mode); unused bytes up to it are zero.
 *   sections    TAG | SM | CODES, each starting 16-byte aligned; slot stride = their sum.
 *   fallback    codes needing more than the capacity: the tile is RAW as in v1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_BF16 = 0, ORC_E5M2 = 1, ORC_E4M3 = 2 };
enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ECORRUPT = -5 };
enum { MODE_NARROW = 0, MODE_WIDE = 1, MODE_RAW = 2 };

typedef struct {
  int32_t fmt, T, D, G, esc_cap;
} orc_params;

typedef struct {
  int32_t F, MB, EB, has_wide;
  int32_t n_groups, plane_bytes;
  int32_t tag_bytes, code_bytes, sm_bytes;
  int32_t tag_off, code_off, sm_off, esc_off, stride, raw_bytes;
} orc_layout;

static int32_t align16(int32_t x) { return (x + 15) / 16 * 16; }

int orc_layout_of(const orc_params* p, orc_layout* L) {
  memset(L, 0, sizeof(*L));
  if (p->fmt == ORC_BF16) { L->F = 8; L->MB = 7; L->EB = 16; }
  else if (p->fmt == ORC_E5M2) { L->F = 5; L->MB = 2; L->EB = 8; }
  else if (p->fmt == ORC_E4M3) { L->F = 4; L->MB = 3; L->EB = 8; }
  else return ORC_EINVAL;
  if (p->T <= 0 || p->D <= 0 || p->G <= 0 || p->T % p->G != 0) return ORC_EINVAL;
  if ((p->T * p->D) % 32 != 0) return ORC_EINVAL;
  if (p->esc_cap < 0 || p->esc_cap % 16 != 0) return ORC_EINVAL;
  L->has_wide = L->F > 4;
  L->n_groups = (p->T / p->G) * p->D;
  L->plane_bytes = (L->n_groups + 31) / 32 * 4;
  L->tag_bytes = 2 * L->plane_bytes;
  L->code_bytes = p->T * p->D * 3 / 8;
  L->sm_bytes = p->T * p->D * (1 + L->MB) / 8;
  L->tag_off = 0;
  L->code_off = L->tag_off + align16(L->tag_bytes);
  L->sm_off = L->code_off + align16(L->code_bytes);
  L->esc_off = L->sm_off + align16(L->sm_bytes);
  L->stride = L->esc_off + p->esc_cap;
  L->raw_bytes = p->T * p->D * L->EB / 8;
  return ORC_OK;
}

/* ---- element fields ---------------------------------------------------------------- */

static uint32_t f_sign(const orc_layout* L, uint32_t x) { return (x >> (L->MB + L->F)) & 1u; }
static uint32_t f_exp(const orc_layout* L, uint32_t x) { return (x >> L->MB) & ((1u << L->F) - 1u); }
static uint32_t f_man(const orc_layout* L, uint32_t x) { return x & ((1u << L->MB) - 1u); }
static uint32_t f_join(const orc_layout* L, uint32_t s, uint32_t e, uint32_t m) {
  return (s << (L->MB + L->F)) | (e << L->MB) | m;
}

/* ---- LSB-first bit streams ------------------------------------------------------------ */

static void put_bit(uint8_t* buf, long bit, uint32_t v) {
  if (v & 1u) buf[bit >> 3] |= (uint8_t)(1u << (bit & 7));
}
static uint32_t get_bit(const uint8_t* buf, long bit) { return (buf[bit >> 3] >> (bit & 7)) & 1u; }

/* Bit position, inside a section, of bit b of the W-bit field of element n in the
 * 32-element unit layout (used by CODE, W = 3, and by the E5M2 SM section, W = 3). */
static long unit_bit(long n, int W, int b) {
  long u = n / 32;
  int r = (int)(n % 32);
  int k = r % 4, s = r / 4;
  int x = W * s + b;
  long byte = u * (4L * W) + 4L * (x / 8) + k;
  return 8L * byte + (x % 8);
}

static void put_sm(const orc_layout* L, uint8_t* sec, long n, uint32_t field) {
  int W = 1 + L->MB;
  for (int b = 0; b < W; ++b) {
    long bit = (W == 8) ? 8L * n + b : (W == 3) ? unit_bit(n, 3, b) : 4L * n + b;
    put_bit(sec, bit, field >> b);
  }
}
static uint32_t get_sm(const orc_layout* L, const uint8_t* sec, long n) {
  int W = 1 + L->MB;
  uint32_t field = 0;
  for (int b = 0; b < W; ++b) {
    long bit = (W == 8) ? 8L * n + b : (W == 3) ? unit_bit(n, 3, b) : 4L * n + b;
    field |= get_bit(sec, bit) << b;
  }
  return field;
}

/* ---- calibration (§3.1: windows of 8 and 16 consecutive exponents per head-channel) ---- */

/* Window start with the largest count of calibration exponents inside [b, b + 2^w - 1];
 * among equally good starts, the lower median in ascending order. */
static int pick_window(const long* hist, int F, int w) {
  int nb = (1 << F) - (1 << w) + 1;
  long best = -1;
  long* cov = (long*)malloc(sizeof(long) * (size_t)nb);
  for (int b = 0; b < nb; ++b) {
    long s = 0;
    for (int e = b; e < b + (1 << w); ++e) s += hist[e];
    cov[b] = s;
    if (s > best) best = s;
  }
  int ties = 0;
  for (int b = 0; b < nb; ++b) ties += (cov[b] == best);
  int want = (ties - 1) / 2, seen = 0, pick = 0;
  for (int b = 0; b < nb; ++b) {
    if (cov[b] != best) continue;
    if (seen == want) { pick = b; break; }
    ++seen;
  }
  free(cov);
  return pick;
}

/* x: [n_tokens][D] element bits of one (K|V, head).  Writes b3[D], b4[D] (b4 = 0 if the
 * format has no wide mode). */
int orc_calibrate(const orc_params* p, const uint16_t* x, int32_t n_tokens, uint8_t* b3, uint8_t* b4) {
  orc_layout L;
  if (orc_layout_of(p, &L) != ORC_OK || n_tokens < 0) return ORC_EINVAL;
  long hist[256];
  for (int c = 0; c < p->D; ++c) {
    for (int e = 0; e < 256; ++e) hist[e] = 0;
    for (int t = 0; t < n_tokens; ++t) hist[f_exp(&L, x[(long)t * p->D + c])] += 1;
    b3[c] = (uint8_t)pick_window(hist, L.F, 3);
    b4[c] = L.has_wide ? (uint8_t)pick_window(hist, L.F, 4) : 0;
  }
  return ORC_OK;
}

/* Exponent concentration (§3.1: most exponents of a head-channel fall in a few consecutive
 * values): for each channel of x [n_tokens][D], the largest number of its exponents inside any
 * window of w consecutive exponent values [b, b + w - 1], 0 <= b <= 2^F - w. */
int orc_window_coverage(const orc_params* p, const uint16_t* x, int32_t n_tokens, int32_t w, int32_t* out) {
  orc_layout L;
  if (orc_layout_of(p, &L) != ORC_OK || n_tokens < 0 || w < 1 || w > (1 << L.F)) return ORC_EINVAL;
  long hist[256];
  for (int c = 0; c < p->D; ++c) {
    for (int e = 0; e < 256; ++e) hist[e] = 0;
    for (int t = 0; t < n_tokens; ++t) hist[f_exp(&L, x[(long)t * p->D + c])] += 1;
    long best = 0;
    for (int b = 0; b + w <= (1 << L.F); ++b) {
      long s = 0;
      for (int e = b; e < b + w; ++e) s += hist[e];
      if (s > best) best = s;
    }
    out[c] = (int32_t)best;
  }
  return ORC_OK;
}

/* ---- encode / decode of one tile ---------------------------------------------------- */

static int group_mode(const orc_layout* L, uint32_t mn, uint32_t mx, uint32_t b3, uint32_t b4) {
  if (b3 <= mn && mx <= b3 + 7) return MODE_NARROW;
  if (L->has_wide && b4 <= mn && mx <= b4 + 15) return MODE_WIDE;
  return MODE_RAW;
}
static int mode_width(const orc_layout* L, int mode) { return mode == MODE_NARROW ? 3 : mode == MODE_WIDE ? 4 : L->F; }
static uint32_t mode_base(int mode, uint32_t b3, uint32_t b4) { return mode == MODE_NARROW ? b3 : mode == MODE_WIDE ? b4 : 0; }

static void write_raw(const orc_params* p, const orc_layout* L, const uint16_t* x, int is_v, uint8_t* out) {
  for (int t = 0; t < p->T; ++t)
    for (int c = 0; c < p->D; ++c) {
      long pos = is_v ? (long)c * p->T + t : (long)t * p->D + c;
      uint32_t v = x[(long)t * p->D + c];
      if (L->EB == 16) { out[2 * pos] = (uint8_t)(v & 0xFF); out[2 * pos + 1] = (uint8_t)(v >> 8); }
      else out[pos] = (uint8_t)(v & 0xFF);
    }
}

/* x: logical tile [T][D] of element bits.  out: at least max(stride, raw_bytes) bytes.
 * Returns 0; *is_raw says which form was written; *esc_used = escape bytes used
 * (compressed tiles), mode_counts[3] = groups per mode (as chosen before any fallback). */
int orc_encode_tile(const orc_params* p, const uint16_t* x, const uint8_t* b3, const uint8_t* b4, int32_t is_v,
                    uint8_t* out, int32_t* is_raw, int32_t* esc_used, int32_t* mode_counts) {
  orc_layout L;
  if (orc_layout_of(p, &L) != ORC_OK) return ORC_EINVAL;
  int NG = L.n_groups, G = p->G, D = p->D;
  int* mode = (int*)malloc(sizeof(int) * (size_t)NG);
  long planes = 0;
  mode_counts[0] = mode_counts[1] = mode_counts[2] = 0;
  for (int q = 0; q < NG; ++q) {
    int tg = q / D, c = q % D;
    uint32_t mn = 0xFFFFFFFFu, mx = 0;
    for (int tau = 0; tau < G; ++tau) {
      uint32_t e = f_exp(&L, x[(long)(tg * G + tau) * D + c]);
      if (e < mn) mn = e;
      if (e > mx) mx = e;
    }
    mode[q] = group_mode(&L, mn, mx, b3[c], b4[c]);
    mode_counts[mode[q]] += 1;
    planes += mode_width(&L, mode[q]) - 3;
  }
  long esc_bytes = (planes * G + 7) / 8;
  long total = L.stride > L.raw_bytes ? L.stride : L.raw_bytes;
  memset(out, 0, (size_t)total);
  if (esc_bytes > p->esc_cap) {
    write_raw(p, &L, x, is_v, out);
    *is_raw = 1;
    *esc_used = 0;
    free(mode);
    return ORC_OK;
  }
  uint8_t* tagE = out + L.tag_off;
  uint8_t* tagR = out + L.tag_off + L.plane_bytes;
  uint8_t* code = out + L.code_off;
  uint8_t* sm = out + L.sm_off;
  uint8_t* esc = out + L.esc_off;
  long P = 0;
  for (int q = 0; q < NG; ++q) {
    int tg = q / D, c = q % D;
    int w = mode_width(&L, mode[q]);
    uint32_t base = mode_base(mode[q], b3[c], b4[c]);
    put_bit(tagE, q, mode[q] >= MODE_WIDE);
    put_bit(tagR, q, mode[q] == MODE_RAW);
    for (int tau = 0; tau < G; ++tau) {
      uint32_t v = x[(long)(tg * G + tau) * D + c];
      long n = (long)q * G + tau;
      uint32_t o = f_exp(&L, v) - base;
      for (int b = 0; b < 3; ++b) put_bit(code, unit_bit(n, 3, b), (o & 7u) >> b);
      put_sm(&L, sm, n, (f_sign(&L, v) << L.MB) | f_man(&L, v));
      if (w > 3) put_bit(esc, P * G + tau, o >> 3);
      if (w == 8) {
        for (int b = 0; b < 4; ++b) put_bit(esc, (P + 1) * G + 4L * tau + b, o >> (4 + b));
      } else if (w == 5) {
        put_bit(esc, (P + 1) * G + tau, o >> 4);
      }
    }
    P += w - 3;
  }
  *is_raw = 0;
  *esc_used = (int32_t)esc_bytes;
  free(mode);
  return ORC_OK;
}

/* Inverse of orc_encode_tile.  x: [T][D] element bits.  Rejects the invalid tag pair, a
 * wide tag in a format without wide mode, and escape planes that run past esc_cap. */
int orc_decode_tile(const orc_params* p, const uint8_t* in, int32_t is_raw, int32_t is_v, const uint8_t* b3,
                    const uint8_t* b4, uint16_t* x) {
  orc_layout L;
  if (orc_layout_of(p, &L) != ORC_OK) return ORC_EINVAL;
  int NG = L.n_groups, G = p->G, D = p->D;
  if (is_raw) {
    for (int t = 0; t < p->T; ++t)
      for (int c = 0; c < D; ++c) {
        long pos = is_v ? (long)c * p->T + t : (long)t * D + c;
        x[(long)t * D + c] = (L.EB == 16) ? (uint16_t)(in[2 * pos] | (in[2 * pos + 1] << 8)) : (uint16_t)in[pos];
      }
    return ORC_OK;
  }
  const uint8_t* tagE = in + L.tag_off;
  const uint8_t* tagR = in + L.tag_off + L.plane_bytes;
  const uint8_t* code = in + L.code_off;
  const uint8_t* sm = in + L.sm_off;
  const uint8_t* esc = in + L.esc_off;
  long P = 0;
  for (int q = 0; q < NG; ++q) {
    int tg = q / D, c = q % D;
    uint32_t E = get_bit(tagE, q), R = get_bit(tagR, q);
    if (!E && R) return ORC_ECORRUPT;
    int mode = (int)(E + R);
    if (mode == MODE_WIDE && !L.has_wide) return ORC_ECORRUPT;
    int w = mode_width(&L, mode);
    if ((P + (w - 3)) * G > 8L * p->esc_cap) return ORC_ECORRUPT;
    uint32_t base = mode_base(mode, b3[c], b4[c]);
    for (int tau = 0; tau < G; ++tau) {
      long n = (long)q * G + tau;
      uint32_t o = 0;
      for (int b = 0; b < 3; ++b) o |= get_bit(code, unit_bit(n, 3, b)) << b;
      if (w > 3) o |= get_bit(esc, P * G + tau) << 3;
      if (w == 8) {
        for (int b = 0; b < 4; ++b) o |= get_bit(esc, (P + 1) * G + 4L * tau + b) << (4 + b);
      } else if (w == 5) {
        o |= get_bit(esc, (P + 1) * G + tau) << 4;
      }
      uint32_t e = base + o;
      if (e >= (1u << L.F)) return ORC_ECORRUPT;
      uint32_t field = get_sm(&L, sm, n);
      x[(long)(tg * G + tau) * D + c] = (uint16_t)f_join(&L, field >> L.MB, e, field & ((1u << L.MB) - 1u));
    }
    P += w - 3;
  }
  return ORC_OK;
}

/* ---- batches (OpenMP over independent tiles only) -------------------------------------- */

int orc_encode_batch(const orc_params* p, int32_t n, const uint16_t* x, const uint8_t* b3, const uint8_t* b4,
                     const int32_t* is_v, uint8_t* out, int64_t out_stride, int32_t* is_raw, int32_t* esc_used,
                     int32_t* mode_counts, int32_t nthreads) {
  orc_layout L;
  if (orc_layout_of(p, &L) != ORC_OK) return ORC_EINVAL;
  if (out_stride < L.stride || out_stride < L.raw_bytes) return ORC_EINVAL;
  long td = (long)p->T * p->D;
  int rc = ORC_OK;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(min : rc)
  for (int i = 0; i < n; ++i) {
    int r = orc_encode_tile(p, x + i * td, b3 + (long)i * p->D, b4 + (long)i * p->D, is_v[i], out + i * out_stride,
                            is_raw + i, esc_used + i, mode_counts + 3L * i);
    if (r < rc) rc = r;
  }
  return rc;
}

int orc_decode_batch(const orc_params* p, int32_t n, const uint8_t* in, int64_t in_stride, const int32_t* is_raw,
                     const int32_t* is_v, const uint8_t* b3, const uint8_t* b4, uint16_t* x, int32_t* status,
                     int32_t nthreads) {
  orc_layout L;
  if (orc_layout_of(p, &L) != ORC_OK) return ORC_EINVAL;
  long td = (long)p->T * p->D;
#pragma omp parallel for schedule(static) num_threads(nthreads)
  for (int i = 0; i < n; ++i)
    status[i] = orc_decode_tile(p, in + i * in_stride, is_raw[i], is_v[i], b3 + (long)i * p->D, b4 + (long)i * p->D,
                                x + i * td);
  return ORC_OK;
}

/* ---- element values -------------------------------------------------------------------- */

/* Exact value of one stored element, by the definition of its format: BF16 (IEEE-style,
 * bias 127), OCP FP8 E5M2 (bias 15, IEEE-style Inf/NaN), OCP FP8 E4M3FN (bias 7, no Inf,
 * S.1111.111 is NaN). */
double orc_value(int32_t fmt, uint32_t bits) {
  int F, MB;
  if (fmt == ORC_BF16) { F = 8; MB = 7; }
  else if (fmt == ORC_E5M2) { F = 5; MB = 2; }
  else { F = 4; MB = 3; }
  uint32_t s = (bits >> (F + MB)) & 1u, e = (bits >> MB) & ((1u << F) - 1u), m = bits & ((1u << MB) - 1u);
  int bias = (1 << (F - 1)) - 1;
  uint32_t emax = (1u << F) - 1u;
  double sign = s ? -1.0 : 1.0;
  if (fmt == ORC_E4M3) {
    if (e == emax && m == (1u << MB) - 1u) return NAN;
  } else if (e == emax) {
    return m == 0 ? sign * INFINITY : NAN;
  }
  if (e == 0) return sign * ldexp((double)m, 1 - bias - MB);
  return sign * ldexp((double)((1u << MB) | m), (int)e - bias - MB);
}

/* ---- exact decode attention ------------------------------------------------------------ */

/* One decode step for one sequence.  q: [Hq][D] BF16 bits; k, v: [L][Hkv][D] element bits of
 * format fmt; out: [Hq][D] fp64.  Query head hq reads KV head hq / (Hq / Hkv).
 * s_t = scale * sum_c q_c k_tc;  out = sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s).
 * Every token attends (no mask), all in fp64. */
int orc_attention(int32_t fmt, const uint16_t* q, const uint16_t* k, const uint16_t* v, int32_t L, int32_t Hq,
                  int32_t Hkv, int32_t D, double scale, double* out, int32_t nthreads) {
  if (L <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0) return ORC_EINVAL;
  int g = Hq / Hkv;
  int rc = ORC_OK;
#pragma omp parallel for schedule(dynamic) num_threads(nthreads)
  for (int hq = 0; hq < Hq; ++hq) {
    int h = hq / g;
    double* s = (double*)malloc(sizeof(double) * (size_t)L);
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    for (int c = 0; c < D; ++c) qd[c] = orc_value(ORC_BF16, q[(long)hq * D + c]);
    double mx = -INFINITY;
    for (int t = 0; t < L; ++t) {
      double acc = 0.0;
      for (int c = 0; c < D; ++c) acc += qd[c] * orc_value(fmt, k[((long)t * Hkv + h) * D + c]);
      s[t] = scale * acc;
      if (s[t] > mx) mx = s[t];
    }
    double den = 0.0;
    for (int t = 0; t < L; ++t) {
      s[t] = exp(s[t] - mx);
      den += s[t];
    }
    for (int c = 0; c < D; ++c) {
      double num = 0.0;
      for (int t = 0; t < L; ++t) num += s[t] * orc_value(fmt, v[((long)t * Hkv + h) * D + c]);
      out[(long)hq * D + c] = num / den;
    }
    free(s);
    free(qd);
  }
  return rc;
}

/* ---- FORMAT v2: nested precision modes (BF16) ------------------------------------------ */

typedef struct {
  int32_t n_modes, width[4];
  int32_t n_groups, plane_bytes, tag_bytes, sm_bytes, code_cap;
  int32_t tag_off, sm_off, code_off, stride, raw_bytes;
} orc_v2_layout;

int orc_v2_layout_of(const orc_params* p, int32_t mode_set, orc_v2_layout* L) {
  memset(L, 0, sizeof(*L));
  if (p->fmt != ORC_BF16) return ORC_EINVAL;
  if (p->T <= 0 || p->D <= 0 || p->G <= 0 || p->T % p->G != 0 || (p->T * p->D) % 32 != 0) return ORC_EINVAL;
  if (p->esc_cap < 0 || p->esc_cap % 16 != 0) return ORC_EINVAL;
  if (mode_set == 1) { L->n_modes = 4; L->width[0] = 2; L->width[1] = 3; L->width[2] = 4; L->width[3] = 8; }
  else if (mode_set == 2) { L->n_modes = 2; L->width[0] = 4; L->width[1] = 8; }
  else if (mode_set == 3) { L->n_modes = 3; L->width[0] = 3; L->width[1] = 4; L->width[2] = 8; }
  else return ORC_EINVAL;
  L->n_groups = (p->T / p->G) * p->D;
  L->plane_bytes = (L->n_groups + 31) / 32 * 4;
  L->tag_bytes = 2 * L->plane_bytes;
  L->sm_bytes = p->T * p->D;
  L->code_cap = p->T * p->D * (L->width[0] < 3 ? 3 : L->width[0]) / 8 + p->esc_cap;
  L->tag_off = 0;
  L->sm_off = align16(L->tag_bytes);
  L->code_off = L->sm_off + align16(L->sm_bytes);
  L->stride = L->code_off + align16(L->code_cap);
  L->raw_bytes = p->T * p->D * 2;
  return ORC_OK;
}

/* Calibrated start of the window of 2^w exponents (same objective and tie-break as v1). */
int orc_v2_calibrate(const orc_params* p, const uint16_t* x, int32_t n_tokens, int32_t w, uint8_t* b) {
  orc_layout L;
  if (orc_layout_of(p, &L) != ORC_OK || n_tokens < 0 || w < 1 || w >= L.F) return ORC_EINVAL;
  long hist[256];
  for (int c = 0; c < p->D; ++c) {
    for (int e = 0; e < 256; ++e) hist[e] = 0;
    for (int t = 0; t < n_tokens; ++t) hist[f_exp(&L, x[(long)t * p->D + c])] += 1;
    b[c] = (uint8_t)pick_window(hist, L.F, w);
  }
  return ORC_OK;
}

/* base of mode width w for channel c: bases[0] = b2, bases[1] = b3, bases[2] = b4 */
static uint32_t v2_base(int w, const uint8_t* const bases[3], int c) { return w >= 8 ? 0u : bases[w - 2][c]; }

/* x: [T][D] BF16 bits.  b2, b3, b4: per-channel bases (unused ones may be any array).  out:
 * at least max(stride, raw_bytes) bytes.  *code_bytes = used CODES bytes; mode_counts[4] =
 * groups per mode index (as chosen before any fallback). */
int orc_v2_encode_tile(const orc_params* p, int32_t mode_set, const uint16_t* x, const uint8_t* b2, const uint8_t* b3,
                       const uint8_t* b4, int32_t is_v, uint8_t* out, int32_t* is_raw, int32_t* code_bytes,
                       int32_t* mode_counts) {
  orc_v2_layout L;
  orc_layout L1;
  if (orc_v2_layout_of(p, mode_set, &L) != ORC_OK || orc_layout_of(p, &L1) != ORC_OK) return ORC_EINVAL;
  const uint8_t* bases[3] = {b2, b3, b4};
  int NG = L.n_groups, G = p->G, D = p->D;
  int* mode = (int*)malloc(sizeof(int) * (size_t)NG);
  long bits = 0;
  for (int k = 0; k < 4; ++k) mode_counts[k] = 0;
  for (int q = 0; q < NG; ++q) {
    int tg = q / D, c = q % D;
    uint32_t mn = 0xFFFFFFFFu, mx = 0;
    for (int tau = 0; tau < G; ++tau) {
      uint32_t e = f_exp(&L1, x[(long)(tg * G + tau) * D + c]);
      if (e < mn) mn = e;
      if (e > mx) mx = e;
    }
    int k = L.n_modes - 1;  /* raw unless a window holds the group */
    for (int j = 0; j < L.n_modes - 1; ++j) {
      uint32_t b = v2_base(L.width[j], bases, c);
      if (b <= mn && mx <= b + (1u << L.width[j]) - 1u) { k = j; break; }
    }
    mode[q] = k;
    mode_counts[k] += 1;
    bits += (long)G * L.width[k];
  }
  long used = (bits + 7) / 8;
  long total = L.stride > L.raw_bytes ? L.stride : L.raw_bytes;
  memset(out, 0, (size_t)total);
  if (used > L.code_cap) {
    write_raw(p, &L1, x, is_v, out);
    *is_raw = 1;
    *code_bytes = 0;
    free(mode);
    return ORC_OK;
  }
  uint8_t* tag0 = out + L.tag_off;
  uint8_t* tag1 = out + L.tag_off + L.plane_bytes;
  uint8_t* sm = out + L.sm_off;
  uint8_t* code = out + L.code_off;
  long O = 0;
  for (int q = 0; q < NG; ++q) {
    int tg = q / D, c = q % D, k = mode[q], w = L.width[k];
    uint32_t base = v2_base(w, bases, c);
    put_bit(tag0, q, (uint32_t)k & 1u);
    put_bit(tag1, q, ((uint32_t)k >> 1) & 1u);
    for (int tau = 0; tau < G; ++tau) {
      uint32_t v = x[(long)(tg * G + tau) * D + c];
      long n = (long)q * G + tau;
      uint32_t o = f_exp(&L1, v) - base;
      for (int b = 0; b < w; ++b) put_bit(code, O + (long)tau * w + b, o >> b);
      sm[n] = (uint8_t)((f_sign(&L1, v) << 7) | f_man(&L1, v));
    }
    O += (long)G * w;
  }
  *is_raw = 0;
  *code_bytes = (int32_t)used;
  free(mode);
  return ORC_OK;
}

/* Inverse of orc_v2_encode_tile.  Rejects a mode index outside the set, codes that run past
 * the capacity, and exponents past the 8-bit field. */
int orc_v2_decode_tile(const orc_params* p, int32_t mode_set, const uint8_t* in, int32_t is_raw, int32_t is_v,
                       const uint8_t* b2, const uint8_t* b3, const uint8_t* b4, uint16_t* x) {
  orc_v2_layout L;
  orc_layout L1;
  if (orc_v2_layout_of(p, mode_set, &L) != ORC_OK || orc_layout_of(p, &L1) != ORC_OK) return ORC_EINVAL;
  if (is_raw) return orc_decode_tile(p, in, 1, is_v, b3, b4, x);
  const uint8_t* bases[3] = {b2, b3, b4};
  int NG = L.n_groups, G = p->G, D = p->D;
  const uint8_t* tag0 = in + L.tag_off;
  const uint8_t* tag1 = in + L.tag_off + L.plane_bytes;
  const uint8_t* sm = in + L.sm_off;
  const uint8_t* code = in + L.code_off;
  long O = 0;
  for (int q = 0; q < NG; ++q) {
    int tg = q / D, c = q % D;
    int k = (int)(get_bit(tag0, q) | (get_bit(tag1, q) << 1));
    if (k >= L.n_modes) return ORC_ECORRUPT;
    int w = L.width[k];
    if (O + (long)G * w > 8L * L.code_cap) return ORC_ECORRUPT;
    uint32_t base = v2_base(w, bases, c);
    for (int tau = 0; tau < G; ++tau) {
      long n = (long)q * G + tau;
      uint32_t o = 0;
      for (int b = 0; b < w; ++b) o |= get_bit(code, O + (long)tau * w + b) << b;
      uint32_t e = base + o;
      if (e >= 256u) return ORC_ECORRUPT;
      x[(long)(tg * G + tau) * D + c] = (uint16_t)f_join(&L1, (uint32_t)sm[n] >> 7, e, sm[n] & 0x7Fu);
    }
    O += (long)G * w;
  }
  return ORC_OK;
}

int orc_v2_encode_batch(const orc_params* p, int32_t mode_set, int32_t n, const uint16_t* x, const uint8_t* b2,
                        const uint8_t* b3, const uint8_t* b4, const int32_t* is_v, uint8_t* out, int64_t out_stride,
                        int32_t* is_raw, int32_t* code_bytes, int32_t* mode_counts, int32_t nthreads) {
  orc_v2_layout L;
  if (orc_v2_layout_of(p, mode_set, &L) != ORC_OK) return ORC_EINVAL;
  if (out_stride < L.stride || out_stride < L.raw_bytes) return ORC_EINVAL;
  long td = (long)p->T * p->D;
  int rc = ORC_OK;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(min : rc)
  for (int i = 0; i < n; ++i) {
    int r = orc_v2_encode_tile(p, mode_set, x + i * td, b2 + (long)i * p->D, b3 + (long)i * p->D, b4 + (long)i * p->D,
                               is_v[i], out + i * out_stride, is_raw + i, code_bytes + i, mode_counts + 4L * i);
    if (r < rc) rc = r;
  }
  return rc;
}

int orc_v2_decode_batch(const orc_params* p, int32_t mode_set, int32_t n, const uint8_t* in, int64_t in_stride,
                        const int32_t* is_raw, const int32_t* is_v, const uint8_t* b2, const uint8_t* b3,
                        const uint8_t* b4, uint16_t* x, int32_t* status, int32_t nthreads) {
  orc_v2_layout L;
  if (orc_v2_layout_of(p, mode_set, &L) != ORC_OK) return ORC_EINVAL;
  long td = (long)p->T * p->D;
#pragma omp parallel for schedule(static) num_threads(nthreads)
  for (int i = 0; i < n; ++i)
    status[i] = orc_v2_decode_tile(p, mode_set, in + i * in_stride, is_raw[i], is_v[i], b2 + (long)i * p->D,
                                   b3 + (long)i * p->D, b4 + (long)i * p->D, x + i * td);
  return ORC_OK;
}


// escape_bounds.cpp -- host check of the escape indexing of the split attention's tile rebuild.
// Built host-only from the kernel's own helpers (codec_dev.h: esc_unit_of_group, esc_tags_fit)
// and run by tests/test_escape_bounds.py.  For random, all-wide, all-raw and corrupt tag words
// (a raw bit without its escape bit) and every count of stored 16-byte escape pieces, it walks
// the per-lane steps of the rebuild -- tag-word prefix, the fit check that clears a word, the
// unit index of each group -- and checks:
//   (1) a kept word's groups start where the format puts them: after all escape units of the
//       tile's earlier groups (wide 1 unit, raw F - 3);
//   (2) every escape unit that feeds a rebuilt value of a kept word lies inside the stored
//       pieces (index < 8 * pieces), so corrupt tags never read another tile's escape bytes;
//   (3) every escape read at all (the unconditional plane read, the raw path of a corrupt
//       raw-without-escape group) has index <= 8 * pieces: at most one unit past the stored
//       pieces, inside the workgroup's LDS, and never used.
// The same walk for the 8-token-group kernel (escape units of one byte; esc_bytes_fit,
// g8_unit_escape; four groups per CODE unit, eight units per tag word), where a raw BF16 group's
// four bytes of 4-bit fields are read as the two aligned words around them: every byte read lies
// below 16 * pieces + 16 (the staging area is the escape room plus 16 bytes), every byte used by
// a kept word below 16 * pieces.
// Prints "ok <cases>" or the first failing case, and exits non-zero on a failure.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "codec_dev.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next32() {  // splitmix64
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)(z ^ (z >> 31));
}

static int check_tile(const uint32_t* E0, const uint32_t* R0, int PW, int RU, uint32_t pieces, long* cases) {
  uint32_t E[16], R[16], P[16];
  uint32_t incl = 0;
  bool cleared[16];
  for (int w = 0; w < PW; ++w) {  // stage_escape: inclusive prefix per tag word, then the fit check
    const uint32_t cnt = (uint32_t)__builtin_popcount(E0[w]) + (uint32_t)(RU - 1) * (uint32_t)__builtin_popcount(R0[w]);
    incl += cnt;
    cleared[w] = !kvc::esc_tags_fit(incl, pieces);
    E[w] = cleared[w] ? 0u : E0[w];
    R[w] = cleared[w] ? 0u : R0[w];
    P[w] = cleared[w] ? 0u : incl - cnt;
  }
  // words are cleared from the first one that does not fit onwards
  for (int w = 1; w < PW; ++w)
    if (cleared[w - 1] && !cleared[w]) { printf("FAIL: word %d kept after a cleared word\n", w); return 1; }
  const uint32_t limit = 8u * pieces;
  uint32_t before = 0;  // format position: units of all earlier groups of the tile (original tags)
  for (int w = 0; w < PW; ++w) {
    for (int n = 0; n < 16; ++n) {
      const uint32_t below = (1u << (2 * n)) - 1u;
      const uint32_t e2 = (E[w] >> (2 * n)) & 3u, r2 = (R[w] >> (2 * n)) & 3u;
      for (int gi = 0; gi < 2; ++gi) {
        ++*cases;
        const uint32_t p = kvc::esc_unit_of_group(E[w], R[w], P[w], below, e2, r2, gi, RU);
        const uint32_t e = (e2 >> gi) & 1u, r = (r2 >> gi) & 1u;
        const uint32_t e_orig = (E0[w] >> (2 * n + gi)) & 1u, r_orig = (R0[w] >> (2 * n + gi)) & 1u;
        if (!cleared[w] && p != before) {
          printf("FAIL (1): word %d group %d at unit %u, format says %u\n", w, 2 * n + gi, p, before);
          return 1;
        }
        // reads: the plane (unit p, read always), and for a raw group units p+1 .. p+RU-1
        const uint32_t last = r ? p + (uint32_t)(RU - 1) : p;
        if (last > limit) {
          printf("FAIL (3): word %d group %d reads unit %u, %u stored\n", w, 2 * n + gi, last, limit);
          return 1;
        }
        if (!cleared[w] && e && last >= limit) {
          printf("FAIL (2): word %d group %d uses unit %u, %u stored\n", w, 2 * n + gi, last, limit);
          return 1;
        }
        before += e_orig + (uint32_t)(RU - 1) * r_orig;
      }
    }
  }
  return 0;
}

static int check_tile_g8(const uint32_t* E0, const uint32_t* R0, int PW, int RU, uint32_t pieces, long* cases) {
  uint32_t E[32], R[32], P[32];
  uint32_t incl = 0;
  bool cleared[32];
  for (int w = 0; w < PW; ++w) {  // g8_stage_escape: inclusive byte prefix per tag word, then the fit check
    const uint32_t cnt = (uint32_t)__builtin_popcount(E0[w]) + (uint32_t)(RU - 1) * (uint32_t)__builtin_popcount(R0[w]);
    incl += cnt;
    cleared[w] = !kvc::esc_bytes_fit(incl, pieces);
    E[w] = cleared[w] ? 0u : E0[w];
    R[w] = cleared[w] ? 0u : R0[w];
    P[w] = cleared[w] ? 0u : incl - cnt;
  }
  for (int w = 1; w < PW; ++w)
    if (cleared[w - 1] && !cleared[w]) { printf("FAIL g8: word %d kept after a cleared word\n", w); return 1; }
  const uint32_t limit = 16u * pieces, room = 16u * pieces + 16u;
  uint32_t before = 0;
  for (int w = 0; w < PW; ++w)
    for (int k = 0; k < 8; ++k) {  // the unit at nibble k
      uint32_t p = kvc::g8_unit_escape(E[w], R[w], P[w], k, RU);
      for (int gi = 0; gi < 4; ++gi) {
        ++*cases;
        const uint32_t e = (E[w] >> (4 * k + gi)) & 1u, r = (R[w] >> (4 * k + gi)) & 1u;
        const uint32_t e_orig = (E0[w] >> (4 * k + gi)) & 1u, r_orig = (R0[w] >> (4 * k + gi)) & 1u;
        if (!cleared[w] && p != before) {
          printf("FAIL g8 (1): word %d group %d at byte %u, format says %u\n", w, 4 * k + gi, p, before);
          return 1;
        }
        uint32_t last_read = p, last_used = p;  // the plane byte, read always
        if (r) {
          if (RU == 5) {  // bytes p+1 .. p+4, read as the aligned words at (p+1) & ~3 and the next one
            last_read = ((p + 1u) & ~3u) + 7u;
            last_used = p + 4u;
          } else if (RU == 2) {
            last_read = last_used = p + 1u;
          }
        }
        if (last_read >= room) {
          printf("FAIL g8 (3): word %d group %d reads byte %u, room %u\n", w, 4 * k + gi, last_read, room);
          return 1;
        }
        if (!cleared[w] && e && last_used >= limit) {
          printf("FAIL g8 (2): word %d group %d uses byte %u, %u stored\n", w, 4 * k + gi, last_used, limit);
          return 1;
        }
        p += e + (uint32_t)(RU - 1) * r;
        before += e_orig + (uint32_t)(RU - 1) * r_orig;
      }
    }
  return 0;
}

int main() {
  long cases = 0;
  const int RUs[3] = {5, 2, 1};  // BF16, E5M2, E4M3 raw groups
  const int PWs[3] = {4, 8, 16};  // tag words per tile: T = 16, 32, 64 at D = 128
  for (int f = 0; f < 3; ++f)
    for (int pw = 0; pw < 3; ++pw)
      for (uint32_t pieces = 0; pieces <= 32; ++pieces)
        for (int trial = 0; trial < 300; ++trial) {
          uint32_t E[16], R[16];
          const int kind = trial % 6;
          for (int w = 0; w < PWs[pw]; ++w) {
            const uint32_t a = next32(), b = next32(), c = next32();
            switch (kind) {
              case 0: E[w] = a & b & c; R[w] = E[w] & next32() & next32(); break;  // sparse, valid pairs
              case 1: E[w] = a; R[w] = a & b; break;                                // dense, valid pairs
              case 2: E[w] = 0xFFFFFFFFu; R[w] = 0xFFFFFFFFu; break;                // every group raw
              case 3: E[w] = 0xFFFFFFFFu; R[w] = 0; break;                          // every group wide
              case 4: E[w] = a & b; R[w] = c; break;                                // raw without escape bits
              default: E[w] = (trial & 1) ? 0 : a; R[w] = ~a & b; break;            // corrupt pairs only
            }
          }
          if (check_tile(E, R, PWs[pw], RUs[f], pieces, &cases)) {
            printf("case: format %d, %d tag words, %u pieces, trial %d\n", f, PWs[pw], pieces, trial);
            return 1;
          }
        }
  const int PW8[3] = {8, 16, 32};  // tag words per tile with 8-token groups: T = 16, 32, 64 at D = 128
  for (int f = 0; f < 3; ++f)
    for (int pw = 0; pw < 3; ++pw)
      for (uint32_t pieces = 0; pieces <= 32; ++pieces)
        for (int trial = 0; trial < 200; ++trial) {
          uint32_t E[32], R[32];
          const int kind = trial % 6;
          for (int w = 0; w < PW8[pw]; ++w) {
            const uint32_t a = next32(), b = next32(), c = next32();
            switch (kind) {
              case 0: E[w] = a & b & c; R[w] = E[w] & next32() & next32(); break;
              case 1: E[w] = a; R[w] = a & b; break;
              case 2: E[w] = 0xFFFFFFFFu; R[w] = 0xFFFFFFFFu; break;
              case 3: E[w] = 0xFFFFFFFFu; R[w] = 0; break;
              case 4: E[w] = a & b; R[w] = c; break;
              default: E[w] = (trial & 1) ? 0 : a; R[w] = ~a & b; break;
            }
          }
          if (check_tile_g8(E, R, PW8[pw], RUs[f], pieces, &cases)) {
            printf("case g8: format %d, %d tag words, %u pieces, trial %d\n", f, PW8[pw], pieces, trial);
            return 1;
          }
        }
  printf("ok %ld\n", cases);
  return 0;
}

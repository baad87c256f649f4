/* oracle_check.c -- drives the C oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built by tests/test_sanitizers.py): round trips of random tiles in every format, group size
 * and FORMAT v2 mode set, random bytes through every decoder (which must answer OK or CORRUPT
 * and never read or write out of bounds), calibration, window coverage and attention. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct { int32_t fmt, T, D, G, esc_cap; } orc_params;
int orc_calibrate(const orc_params*, const uint16_t*, int32_t, uint8_t*, uint8_t*);
int orc_encode_tile(const orc_params*, const uint16_t*, const uint8_t*, const uint8_t*, int32_t, uint8_t*, int32_t*,
                    int32_t*, int32_t*);
int orc_decode_tile(const orc_params*, const uint8_t*, int32_t, int32_t, const uint8_t*, const uint8_t*, uint16_t*);
int orc_v2_calibrate(const orc_params*, const uint16_t*, int32_t, int32_t, uint8_t*);
int orc_v2_encode_tile(const orc_params*, int32_t, const uint16_t*, const uint8_t*, const uint8_t*, const uint8_t*,
                       int32_t, uint8_t*, int32_t*, int32_t*, int32_t*);
int orc_v2_decode_tile(const orc_params*, int32_t, const uint8_t*, int32_t, int32_t, const uint8_t*, const uint8_t*,
                       const uint8_t*, uint16_t*);
int orc_window_coverage(const orc_params*, const uint16_t*, int32_t, int32_t, int32_t*);
int orc_attention(int32_t, const uint16_t*, const uint16_t*, const uint16_t*, int32_t, int32_t, int32_t, int32_t, double,
                  double*, int32_t);

static uint64_t s = 88172645463325252ull;
static uint32_t rnd(void) { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return (uint32_t)s; }

int main(void) {
  const int fmts[3] = {0, 1, 2}, EB[3] = {16, 8, 8}, MB[3] = {7, 2, 3};
  long cases = 0;
  for (int fi = 0; fi < 3; ++fi)
    for (int Gi = 0; Gi < 2; ++Gi)
      for (int Ti = 0; Ti < 2; ++Ti) {
        orc_params p = {fmts[fi], Ti ? 64 : 16, 64, Gi ? 16 : 8, Ti ? 256 : 64};
        const int n = p.T * p.D, F = (EB[fi] == 16) ? 8 : (fi == 1 ? 5 : 4);
        uint16_t* x = malloc(sizeof(uint16_t) * n);
        uint16_t* y = malloc(sizeof(uint16_t) * n);
        uint8_t b2[64], b3[64], b4[64];
        uint8_t* out = malloc(32768);
        for (int trial = 0; trial < 60; ++trial) {
          const int spread = 1 + (int)(rnd() % (trial % 3 == 0 ? 3 : 40));
          for (int i = 0; i < n; ++i) {
            uint32_t e = (uint32_t)((100 % (1 << F)) + rnd() % spread) & ((1u << F) - 1u);
            x[i] = (uint16_t)(((rnd() & 1u) << (F + MB[fi])) | (e << MB[fi]) | (rnd() & ((1u << MB[fi]) - 1u)));
          }
          if (orc_calibrate(&p, x, p.T, b3, b4)) return 1;
          int32_t raw, esc, modes[4], st;
          if (orc_encode_tile(&p, x, b3, b4, trial & 1, out, &raw, &esc, modes)) return 2;
          if (orc_decode_tile(&p, out, raw, trial & 1, b3, b4, y) || memcmp(x, y, sizeof(uint16_t) * n)) return 3;
          for (int i = 0; i < 11904 && i < 32768; ++i) out[i] = (uint8_t)rnd();  /* random bytes: OK or CORRUPT */
          st = orc_decode_tile(&p, out, 0, trial & 1, b3, b4, y);
          if (st != 0 && st != -5) return 4;
          if (fi == 0)
            for (int ms = 1; ms <= 3; ++ms) {
              if (orc_v2_calibrate(&p, x, p.T, 2, b2) || orc_v2_calibrate(&p, x, p.T, 3, b3) ||
                  orc_v2_calibrate(&p, x, p.T, 4, b4))
                return 5;
              if (orc_v2_encode_tile(&p, ms, x, b2, b3, b4, trial & 1, out, &raw, &esc, modes)) return 6;
              if (orc_v2_decode_tile(&p, ms, out, raw, trial & 1, b2, b3, b4, y) || memcmp(x, y, sizeof(uint16_t) * n))
                return 7;
              for (int i = 0; i < 12928; ++i) out[i] = (uint8_t)rnd();
              st = orc_v2_decode_tile(&p, ms, out, 0, trial & 1, b2, b3, b4, y);
              if (st != 0 && st != -5) return 8;
              ++cases;
            }
          int32_t cov[64];
          if (orc_window_coverage(&p, x, p.T, 6, cov)) return 9;
          ++cases;
        }
        free(x); free(y); free(out);
      }
  uint16_t q[4 * 64], k[33 * 2 * 64], v[33 * 2 * 64];
  for (int i = 0; i < 4 * 64; ++i) q[i] = (uint16_t)(0x3F00 | (rnd() & 0x80FF));
  for (int i = 0; i < 33 * 2 * 64; ++i) { k[i] = (uint16_t)(0x3C00 | (rnd() & 0x83FF)); v[i] = (uint16_t)(0x3C00 | (rnd() & 0x83FF)); }
  double o[4 * 64];
  if (orc_attention(0, q, k, v, 33, 4, 2, 64, 0.125, o, 1)) return 10;
  printf("ok %ld\n", cases);
  return 0;
}

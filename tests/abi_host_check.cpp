// abi_host_check.cpp -- drives the host half of the C ABI (api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, built by tests/test_sanitizers.py with the kernel launchers stubbed
// out: parameter validation and buffer sizes for every format, group size, block size, head size
// and mode set; the admission planner; and NULL, misaligned and out-of-range arguments to every
// entry point.  No call here reaches the HIP runtime.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvc.h"

static int expect(int got, int want, const char* what) {
  if (got != want) {
    printf("FAIL %s: %d (want %d): %s\n", what, got, want, kv_last_error());
    return 1;
  }
  return 0;
}

int main() {
  int bad = 0;
  long cases = 0;
  const int dts[3] = {KVC_BF16, KVC_FP8_E5M2, KVC_FP8_E4M3};
  const int Ds[4] = {64, 128, 256, 96}, Ts[5] = {16, 32, 64, 48, 8}, Gs[3] = {8, 16, 4};
  for (int dt : dts)
    for (int D : Ds)
      for (int T : Ts)
        for (int G : Gs)
          for (int ms = -1; ms <= 4; ++ms)
            for (int comp = 0; comp <= 1; ++comp) {
              const int nv = (int)(cases % 7) - 1;  // base versions -1 .. 5 across the cases
              kvc_params p = {dt, 8, 32, D, T, G, -1, comp, 4, 100, 1000, 100, ms, nv};
              size_t sz[KVC_NUM_BUFFERS], stride = 0;
              const int rc = kv_buffer_sizes(&p, sz, &stride);
              const bool valid = (D == 64 || D == 128 || D == 256) && (T == 16 || T == 32 || T == 64) && (G == 8 || G == 16) &&
                                 ms >= 0 && ms <= 3 && (ms == 0 || (dt == KVC_BF16 && D <= 128)) && nv >= 0 && nv <= 4;
              if (valid != (rc == KVC_OK)) {
                printf("FAIL sizes dt=%d D=%d T=%d G=%d ms=%d: rc %d\n", dt, D, T, G, ms, rc);
                bad = 1;
              }
              if (rc == KVC_OK && (stride == 0 || stride % 16 || sz[7] != 12416)) bad = 1;
              // the bases buffer holds one calibrated set per base version
              if (rc == KVC_OK && sz[3] != (size_t)(nv < 1 ? 1 : nv) * (ms == 1 ? 6 : 4) * 8 * D) bad = 1;
              int32_t lens[5] = {4096, 8000, 100, 32768, 1};
              int32_t n = -1, nc = -1, nr = -1;
              const int ra = kv_admit_fcfs(&p, 1ull << 30, 1.0 / 64, lens, 5, &n, &nc, &nr);
              if ((ra == KVC_OK) != valid) bad = 1;
              ++cases;
            }
  kvc_params p = {KVC_BF16, 8, 32, 128, 64, 16, -1, 1, 2, 10, 100, 10, 0};
  bad |= expect(kv_buffer_sizes(nullptr, nullptr, nullptr), KVC_EINVAL, "sizes NULL");
  bad |= expect(kv_cache_create(&p, nullptr, 0, nullptr, nullptr), KVC_EINVAL, "create NULL buffers");
  kvc_buffers b;
  memset(&b, 0, sizeof(b));
  kvc_cache* c = nullptr;
  bad |= expect(kv_cache_create(&p, &b, 0, nullptr, &c), KVC_EINVAL, "create NULL device buffers");
  alignas(16) static uint8_t fake[64];
  void* odd = fake + 1;
  b = {odd, odd, odd, odd, odd, odd, odd, odd};
  bad |= expect(kv_cache_create(&p, &b, 0, nullptr, &c), KVC_EINVAL, "create misaligned buffers");
  int32_t ids[1] = {0};
  uint32_t flags;
  int32_t len;
  bad |= expect(kv_calibrate(nullptr, fake, fake, 1, nullptr), KVC_EINVAL, "calibrate NULL cache");
  bad |= expect(kv_recalibrate(nullptr, fake, fake, 1, nullptr), KVC_EINVAL, "recalibrate NULL cache");
  bad |= expect(kv_encode_append(nullptr, ids, 1, fake, fake, 1, nullptr), KVC_EINVAL, "append NULL cache");
  bad |= expect(kv_decode_blocks(nullptr, 0, 0, 1, fake, fake, nullptr), KVC_EINVAL, "decode NULL cache");
  bad |= expect(kv_decode_attention(nullptr, ids, 1, fake, 1.f, 1, fake, 64, fake, nullptr), KVC_EINVAL, "attn NULL");
  bad |= expect(kv_decode_attention_noalloc(nullptr, ids, 1, fake, 1.f, 1, fake, nullptr), KVC_EINVAL, "noalloc NULL");
  bad |= expect(kv_decode_step(nullptr, ids, 1, fake, fake, fake, 1.f, 1, fake, 64, fake, nullptr), KVC_EINVAL, "step");
  bad |= expect(kv_prefill_attention(nullptr, fake, fake, 1, fake, 1, 1.f, fake, nullptr), KVC_EINVAL, "prefill");
  bad |= expect(kv_tile_stats(nullptr, 0, 0, 1, (int32_t*)fake, nullptr), KVC_EINVAL, "tile stats");
  bad |= expect(kv_window_coverage(nullptr, fake, 1, 6, (int32_t*)fake, nullptr), KVC_EINVAL, "coverage");
  bad |= expect(kv_read_probe(nullptr, 8192, 1, (uint32_t*)fake, nullptr), KVC_EINVAL, "probe NULL src");
  bad |= expect(kv_read_probe(fake, 8192, 1, nullptr, nullptr), KVC_EINVAL, "probe NULL sink");
  bad |= expect(kv_read_probe(odd, 8192, 1, (uint32_t*)fake, nullptr), KVC_EINVAL, "probe misaligned src");
  bad |= expect(kv_read_probe(fake, 4096, 1, (uint32_t*)fake, nullptr), KVC_EINVAL, "probe ragged bytes");
  bad |= expect(kv_read_probe(fake, 0, 1, (uint32_t*)fake, nullptr), KVC_EINVAL, "probe zero bytes");
  bad |= expect(kv_read_probe(fake, 8192, 0, (uint32_t*)fake, nullptr), KVC_EINVAL, "probe zero waves");
  bad |= expect(kv_release_seq(nullptr, 0, nullptr), KVC_EINVAL, "release");
  bad |= expect(kv_seq_length(nullptr, 0, &len), KVC_EINVAL, "length");
  bad |= expect(kv_get_status(nullptr, &flags, nullptr, nullptr), KVC_EINVAL, "status");
  bad |= expect(kv_admit_fcfs(&p, 1ull << 30, 2.0, nullptr, 0, &len, &len, &len), KVC_EINVAL, "admit share");
  int32_t zero[2] = {5, 0};
  bad |= expect(kv_admit_fcfs(&p, 1ull << 30, 0.0, zero, 2, &len, &len, &len), KVC_EINVAL, "admit length 0");
  if (kv_attention_workspace_bytes(nullptr, 1, 1) != 0 || kv_attention_workspace_bytes(&p, 0, 1) != 0) bad = 1;
  if (strlen(kv_last_error()) == 0) bad = 1;
  if (bad) return 1;
  printf("ok %ld\n", cases);
  return 0;
}

// abi_launch_stubs.cpp -- stand-ins for the kernel launchers, so the host half of the C ABI
// (api.cpp) links without device code for the sanitizer build of tests/test_sanitizers.py.
// Every launcher reports "no device" (hipErrorNoDevice = 100); the checks driven there return
// before any launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_internal.h"

namespace kvc {
static const int kNoDevice = 100;
int launch_init(const Geo&, const DevBufs&, const int32_t*, const int32_t*, void*) { return kNoDevice; }
int launch_calibrate(const Geo&, const DevBufs&, const void*, const void*, int, void*) { return kNoDevice; }
int launch_append(const Geo&, const DevBufs&, const SeqList&, const void*, const void*, int, int, void*) { return kNoDevice; }
int launch_release(const Geo&, const DevBufs&, int, int, void*) { return kNoDevice; }
int launch_decode_blocks(const Geo&, const DevBufs&, int, int, int, void*, void*, void*) { return kNoDevice; }
int launch_attention_partials(const Geo&, const DevBufs&, const SeqList&, const uint16_t*, float, int, float*, float*,
                              const void*, const void*, const int*, void*) { return kNoDevice; }
int launch_attention_any(const Geo&, const DevBufs&, const SeqList&, const uint16_t*, float, int, float*, float*,
                         const void*, const void*, const int*, void*) { return kNoDevice; }
int launch_attention_half(const Geo&, const DevBufs&, const SeqList&, const int*, const uint16_t*, float, int, float*,
                          float*, void*) { return kNoDevice; }
int launch_prefill(const Geo&, const void*, const void*, int, const uint16_t*, int, float, uint16_t*, void*) {
  return kNoDevice;
}
int launch_combine(const Geo&, const DevBufs&, const SeqList&, const uint16_t*, float, int, const float*, const float*,
                   uint16_t*, void*) { return kNoDevice; }
int launch_tile_stats(const Geo&, const DevBufs&, int, int, int, int32_t*, void*) { return kNoDevice; }
int launch_coverage(const Geo&, const void*, int, int, int32_t*, void*) { return kNoDevice; }
int launch_read_probe(const void*, size_t, int, uint32_t*, void*) { return kNoDevice; }
int noalloc_workspace(void** ptr) { *ptr = nullptr; return kNoDevice; }
}  // namespace kvc

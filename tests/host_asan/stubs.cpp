// Host-only stand-ins for a sanitizer build of libkvc's host code.
//
// The entry points (api.hip, compiled for the host only), the block pool and
// the budget schedules are linked against these instead of the kernels and the
// HIP runtime. Every launcher records its call and succeeds without touching
// memory, so the entry points' validation, workspace layout and overlap checks
// run on the CPU under AddressSanitizer and UndefinedBehaviorSanitizer.
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "kvc_internal.h"

extern "C" int kvc_stub_launches = 0;

namespace kvc {
namespace {
hipError_t launched() {
  ++kvc_stub_launches;
  return hipSuccess;
}
}  // namespace

hipError_t launch_quant_append(const kvc_cache_t&, const __half*, const __half*, int, float*, hipStream_t) {
  return launched();
}
hipError_t launch_decode_attn(const AttnLaunch&, hipStream_t) { return launched(); }
hipError_t launch_attn_split(const AttnLaunch&, hipStream_t) { return launched(); }
hipError_t launch_attn_merge(const AttnLaunch&, hipStream_t) { return launched(); }
hipError_t launch_select(const kvc_cache_t&, const float*, int, int, int, uint8_t*, int32_t*, int, hipStream_t) {
  return launched();
}
bool evict_fits_one_launch(int max_len, int n_sink, int n_recent) {
  return (long long)max_len - n_sink - n_recent <= 8192;
}
bool evict_can_merge(int num_q_heads, int num_kv_heads, int splits) {
  return num_q_heads / num_kv_heads <= kEvictMaxMergeHeads && splits <= kEvictMaxSplits;
}
hipError_t launch_evict(const EvictArgs&, hipStream_t) { return launched(); }
hipError_t launch_evict_inplace(const EvictArgs&, hipStream_t) { return launched(); }
hipError_t launch_compact(const kvc_cache_t&, const float*, const uint8_t*, const kvc_cache_t&, float*, int32_t*, int,
                          hipStream_t) {
  return launched();
}
hipError_t launch_compact_gather(const kvc_cache_t&, const float*, const int32_t*, int, const kvc_cache_t&, float*,
                                 hipStream_t) {
  return launched();
}
size_t block_evict_lds_bytes(int max_blocks_per_seq) { return (size_t)max_blocks_per_seq * 8; }
hipError_t launch_block_evict(const kvc_cache_t&, const float*, double, const kvc_cache_t&, float*, int32_t*,
                              int32_t*, float*, int, hipStream_t) {
  return launched();
}
hipError_t launch_fill_zero(float*, long long, hipStream_t) { return launched(); }
hipError_t launch_kvsep_gather(const KvsepArgs&, hipStream_t) { return launched(); }
int bw_probe_workgroups() { return 4096; }
hipError_t launch_bw_probe(const void*, size_t, unsigned*, hipStream_t) { return launched(); }
}  // namespace kvc

// The HIP runtime calls of the entry points.
alignas(256) static char g_scratch_stand_in[256];
extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** p, const void*) {
  *p = g_scratch_stand_in;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipHostGetDevicePointer(void** dev, void* host, unsigned int) {
  *dev = host;
  return hipSuccess;
}
// Registration of device code: a host-only build embeds none.
void** __hipRegisterFatBinary(const void*) { return nullptr; }
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterVar(void**, void*, char*, const char*, int, size_t, int, int) {}
}
// The host-only object refers to its (absent) device image by this name.
#ifdef KVC_FATBIN_SYMBOL
extern "C" const char KVC_FATBIN_SYMBOL[1] = {0};
#endif

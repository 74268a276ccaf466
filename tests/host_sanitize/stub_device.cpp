// Host stand-ins for the device side of the library (lf_kernel.hip,
// lf_prefill.hip), so that the host runtime lf_host.cpp builds with g++ and
// runs under AddressSanitizer / UndefinedBehaviorSanitizer without a GPU:
// "device" buffers are host memory, copies are memcpy, launches are recorded.
#include <cstring>
#include <vector>

#include "../../kv_cache_eviction_lf_amd/csrc/lf_internal.h"
#include "stub_device.h"

namespace stub {
std::vector<lf::StepArgs> steps;
std::vector<lf::PrefillArgs> prefills;
int fail_copies = 0;  // > 0: the next copies fail (error paths)
alignas(256) unsigned char prefill_scratch_mem[1 << 16];
}  // namespace stub

namespace lf {

// Tile height of the kernels: 16 rows per wave for bf16 (4 waves), 4 row loads
// of 64 / (d / 4) rows per wave for fp32.
int tile_rows(int dtype, int head_dim, int group) {
  if (group < 1 || group > 8 || (head_dim != 64 && head_dim != 128)) return 0;
  return dtype == 1 ? 64 : kThreads / 64 * (64 / (head_dim / 4)) * 4;
}

int launch_step(int, int, int, const StepArgs& a, void*, char*, size_t) {
  stub::steps.push_back(a);
  return 0;
}

int launch_prefill(int, int, const PrefillArgs& a, int, void*, char*, size_t) {
  stub::prefills.push_back(a);
  return 0;
}

int prefill_scratch(void** ptr, char*, size_t) {
  *ptr = stub::prefill_scratch_mem;
  return 0;
}

int copy_rows_and_wait(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t rows, bool,
                       void*, char* err, size_t errlen) {
  if (stub::fail_copies > 0) {
    --stub::fail_copies;
    std::snprintf(err, errlen, "stub copy failure");
    return 1;
  }
  for (size_t r = 0; r < rows; ++r)
    std::memcpy(static_cast<char*>(dst) + r * dpitch, static_cast<const char*>(src) + r * spitch, width);
  return 0;
}

int upload_and_wait(void* dst, const void* src, size_t bytes, void* stream, char* err, size_t errlen) {
  return copy_rows_and_wait(dst, bytes, src, bytes, bytes, 1, true, stream, err, errlen);
}

int download_and_wait(void* dst, const void* src, size_t bytes, void* stream, char* err, size_t errlen) {
  return copy_rows_and_wait(dst, bytes, src, bytes, bytes, 1, false, stream, err, errlen);
}

}  // namespace lf

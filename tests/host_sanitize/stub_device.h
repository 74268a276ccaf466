// What the host stand-ins of the device side record (stub_device.cpp).
#pragma once
#include <cstdio>
#include <vector>

#include "../../kv_cache_eviction_lf_amd/csrc/lf_internal.h"

namespace stub {
extern std::vector<lf::StepArgs> steps;       // every launch_step, in order
extern std::vector<lf::PrefillArgs> prefills;  // every launch_prefill
extern int fail_copies;                        // > 0: that many next copies fail
extern unsigned char prefill_scratch_mem[1 << 16];
}  // namespace stub

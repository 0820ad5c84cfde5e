// Internal declarations shared by the host entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "submconv.h"

namespace submconv {

// Status plus message; the C entry points turn it into an int and a thread-local string.
struct Status {
  int code = SUBM_OK;
  std::string msg;
  bool ok() const { return code == SUBM_OK; }
};

Status make_status(int code, std::string msg);
Status hip_status(hipError_t e, const char* what);

#define SUBM_HIP_TRY(expr)                                       \
  do {                                                           \
    hipError_t _e = (expr);                                      \
    if (_e != hipSuccess) return ::submconv::hip_status(_e, #expr); \
  } while (0)

// Stream-ordered device allocation from the per-device pool (see allocator in submconv_api.hip).
Status device_alloc(void** ptr, size_t bytes, hipStream_t stream);
void device_free(void* ptr, hipStream_t stream);

// Device-side statistics written by the map build.
struct BuildStats {
  int32_t mn[4];                     // per-column minimum of (b, z, y, x)
  int32_t mx[4];                     // per-column maximum
  uint32_t flags;                    // kFlag* bits
  uint32_t pad;
  unsigned long long pairs;          // total nbr entries >= 0
  unsigned long long per_tap[27];    // entries >= 0 per tap
};

constexpr uint32_t kFlagDuplicate = 1u;
constexpr uint32_t kFlagBatchRange = 2u;
constexpr uint32_t kFlagProbeOverflow = 4u;

// Map handle contents.
struct MapData {
  int device = 0;
  int64_t n = 0;
  int64_t pairs = 0;
  int64_t per_tap[27] = {};
  int32_t* nbr = nullptr;   // device [n, 27], input row order
};

// Launchers (indice_map.hip).  All enqueue on `stream`; none synchronises.
// Builds nbr[n,27] and fills *stats (device).  `table_slots` is the hash capacity, `table`
// a device buffer of table_slots 16-byte slots, `partials` a device buffer of
// map_partial_count() * 27 uint32 for per-block pair counts.
int64_t map_table_slots(int64_t n);
int map_partial_blocks(int64_t n);
hipError_t launch_map_build(const int32_t* coords, int64_t n, void* table, int64_t table_slots,
                            uint32_t* partials, int partial_blocks, int32_t* nbr,
                            BuildStats* stats, hipStream_t stream);

// Convolution launcher (conv.hip).  Arguments already validated by the caller.
hipError_t launch_subm_conv(const MapData* map, int64_t n, int ksize, int cin, int cout,
                            int dtype, const void* feats, const void* weight, const void* bias,
                            void* out, hipStream_t stream);

}  // namespace submconv

// The opaque handle type of the C ABI.
struct submconv_map {
  submconv::MapData d;
};

// C ABI entry points: argument validation, status codes, device memory, the map handle.
// Every check that does not need the GPU runs before any HIP call, so invalid arguments are
// rejected identically on a machine without a GPU.
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "internal.h"

namespace submconv {

namespace {
thread_local std::string g_last_error;
}  // namespace

void clear_error() { g_last_error.clear(); }
int fail(const Status& s) {
  g_last_error = s.msg;
  return s.code;
}
int fail(int code, const char* msg) {
  g_last_error = msg;
  return code;
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_pool_mu;
bool g_pool_ready[kMaxDevices] = {};

// Keep freed blocks in the device's default pool (no release back to the driver at every
// synchronisation), so repeated builds and frees cost no driver allocations after warm-up.
Status ensure_pool(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return make_status(SUBM_ERR_HIP, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (g_pool_ready[dev]) return Status{};
  hipMemPool_t pool;
  SUBM_HIP_TRY(hipDeviceGetDefaultMemPool(&pool, dev));
  uint64_t threshold = UINT64_MAX;
  SUBM_HIP_TRY(hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &threshold));
  g_pool_ready[dev] = true;
  return Status{};
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

Pinned pinned_block(int dev) {
  thread_local Pinned bufs[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return Pinned{};
  if (bufs[dev].host == nullptr) {
    void* p = nullptr;
    void* d = nullptr;
    if (hipHostMalloc(&p, kPinnedBytes, hipHostMallocDefault) != hipSuccess) return Pinned{};
    if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess) {
      (void)hipHostFree(p);
      return Pinned{};
    }
    bufs[dev].host = p;
    bufs[dev].dev = d;
  }
  return bufs[dev];
}

Status make_status(int code, std::string msg) {
  Status s;
  s.code = code;
  s.msg = std::move(msg);
  return s;
}

Status hip_status(hipError_t e, const char* what) {
  const int code = (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) ? SUBM_ERR_OUT_OF_MEMORY : SUBM_ERR_HIP;
  return make_status(code, std::string(what) + ": " + hipGetErrorString(e));
}

Status device_alloc(void** ptr, size_t bytes, hipStream_t stream) {
  int dev = 0;
  SUBM_HIP_TRY(hipGetDevice(&dev));
  Status s = ensure_pool(dev);
  if (!s.ok()) return s;
  *ptr = nullptr;
  SUBM_HIP_TRY(hipMallocAsync(ptr, bytes, stream));
  return Status{};
}

void device_free(void* ptr, hipStream_t stream) {
  if (ptr != nullptr) (void)hipFreeAsync(ptr, stream);
}

}  // namespace submconv

using namespace submconv;

extern "C" const char* subm_status_string(int status) {
  switch (status) {
    case SUBM_OK: return "SUBM_OK";
    case SUBM_ERR_INVALID_ARG: return "SUBM_ERR_INVALID_ARG";
    case SUBM_ERR_DUPLICATE_COORD: return "SUBM_ERR_DUPLICATE_COORD";
    case SUBM_ERR_COORD_RANGE: return "SUBM_ERR_COORD_RANGE";
    case SUBM_ERR_SHAPE_MISMATCH: return "SUBM_ERR_SHAPE_MISMATCH";
    case SUBM_ERR_UNSUPPORTED: return "SUBM_ERR_UNSUPPORTED";
    case SUBM_ERR_OUT_OF_MEMORY: return "SUBM_ERR_OUT_OF_MEMORY";
    case SUBM_ERR_HIP: return "SUBM_ERR_HIP";
    default: return "unknown status";
  }
}

extern "C" const char* subm_last_error(void) { return g_last_error.c_str(); }

namespace {

// Build workspace (hash table or dense grid, bounds partials, statistics): one grow-only device
// buffer per GPU, held under a mutex for the whole build.  A build ends with a stream
// synchronisation, so the buffer is idle when the next build takes it; builds on one GPU from
// several threads are serialised by the mutex.
struct Workspace {
  std::mutex mu;
  void* ptr = nullptr;
  size_t bytes = 0;
  // Recorded after the last kernel of the latest build: a build returns once its insert kernel
  // is done, so the next build's kernels wait for this event (on the device) before they touch
  // the shared structure.
  hipEvent_t last = nullptr;
};
Workspace g_workspace[kMaxDevices];

// Per-thread, per-device event recorded after the insert kernel; the build waits for it.
hipEvent_t inserted_event(int dev) {
  thread_local hipEvent_t ev[kMaxDevices] = {};
  if (ev[dev] == nullptr && hipEventCreateWithFlags(&ev[dev], hipEventDisableTiming) != hipSuccess) ev[dev] = nullptr;
  return ev[dev];
}

// Layout: [statistics | bounds partials | table area].  The table area is all 0xFF bytes
// whenever no build is running (each build resets what it wrote), so a new allocation is filled.
constexpr size_t kStatsBytes = 4096;
constexpr size_t kPartialsBytes = 65536;
static_assert(sizeof(MapStats) <= kStatsBytes, "statistics block");

Status workspace_reserve(Workspace& ws, size_t table_bytes, hipStream_t stream) {
  const size_t bytes = kStatsBytes + kPartialsBytes + table_bytes;
  if (ws.bytes >= bytes) return Status{};
  if (ws.ptr != nullptr) {
    SUBM_HIP_TRY(hipFree(ws.ptr));
    ws.ptr = nullptr;
    ws.bytes = 0;
  }
  const size_t grain = size_t(64) << 20;
  const size_t want = (bytes + grain - 1) / grain * grain;
  SUBM_HIP_TRY(hipMalloc(&ws.ptr, want));
  ws.bytes = want;
  // Statistics and partials start zeroed (the plan's completion counter lives there); the table
  // area starts empty.
  SUBM_HIP_TRY(launch_fill(ws.ptr, kStatsBytes + kPartialsBytes, 0u, stream));
  SUBM_HIP_TRY(launch_fill(static_cast<unsigned char*>(ws.ptr) + kStatsBytes + kPartialsBytes,
                           want - kStatsBytes - kPartialsBytes, 0xFFFFFFFFu, stream));
  return Status{};
}

// The plan's flags and mode and the insert's error flags arrive in the calling thread's pinned
// block for the device (a thread runs one build at a time): the kernels write them through its
// device address, so the build needs no copy command.
static_assert(sizeof(MapHostFlags) <= kPinnedBytes, "host flags fit the pinned block");

void release_map(submconv_map* m, hipStream_t stream) {
  if (m->d.ready != nullptr) {
    (void)hipEventSynchronize(m->d.ready);  // the build's own kernels write the map memory
    (void)hipEventDestroy(m->d.ready);
  }
  device_free(m->d.nbr, stream);
  device_free(m->d.pair_out, stream);
  delete m;
}

}  // namespace

extern "C" int sparse_indice_map_build_ex(const int32_t* coords, int64_t n, int mode, hipStream_t stream,
                                          submconv_map_t* out_map) {
  clear_error();
  if (out_map == nullptr) return fail(SUBM_ERR_INVALID_ARG, "out_map is NULL");
  *out_map = nullptr;
  if (mode != SUBM_MAP_AUTO && mode != SUBM_MAP_HASH && mode != SUBM_MAP_GRID)
    return fail(SUBM_ERR_INVALID_ARG, "mode must be SUBM_MAP_AUTO, SUBM_MAP_HASH or SUBM_MAP_GRID");
  if (n < 0) return fail(SUBM_ERR_INVALID_ARG, "n is negative");
  if (n > INT32_MAX) return fail(SUBM_ERR_INVALID_ARG, "n exceeds 2^31 - 1 (rows are int32)");
  if (n > 0 && coords == nullptr) return fail(SUBM_ERR_INVALID_ARG, "coords is NULL");
  if ((reinterpret_cast<uintptr_t>(coords) & 15u) != 0) return fail(SUBM_ERR_INVALID_ARG, "coords is not 16-byte aligned");

  submconv_map* m = new (std::nothrow) submconv_map;
  if (m == nullptr) return fail(SUBM_ERR_OUT_OF_MEMORY, "host allocation of the map handle failed");
  if (hipGetDevice(&m->d.device) != hipSuccess) {
    delete m;
    return fail(SUBM_ERR_HIP, "hipGetDevice failed");
  }
  m->d.n = n;
  m->d.mode = kModeHash;
  if (n == 0) {
    *out_map = m;
    return SUBM_OK;
  }
  if (m->d.device < 0 || m->d.device >= kMaxDevices) {
    delete m;
    return fail(SUBM_ERR_HIP, "device ordinal out of range");
  }
  const Pinned pinned = pinned_block(m->d.device);
  const hipEvent_t inserted = inserted_event(m->d.device);
  if (pinned.host == nullptr || inserted == nullptr) {
    delete m;
    return fail(SUBM_ERR_OUT_OF_MEMORY, "pinned host flags or build event");
  }
  volatile MapHostFlags* host = static_cast<volatile MapHostFlags*>(pinned.host);

  const size_t table_bytes = round_up(map_table_bytes(n), 256);
  if (map_partials_bytes(n) > kPartialsBytes) {
    delete m;
    return fail(SUBM_ERR_HIP, "internal error: bounds partials exceed their workspace block");
  }

  Workspace& ws = g_workspace[m->d.device];
  std::lock_guard<std::mutex> lock(ws.mu);
  hipError_t e = ws.last == nullptr ? hipEventCreateWithFlags(&ws.last, hipEventDisableTiming)
                                    : hipStreamWaitEvent(stream, ws.last, 0);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&m->d.ready, hipEventDisableTiming);
  if (e != hipSuccess) {
    if (m->d.ready != nullptr) (void)hipEventDestroy(m->d.ready);
    delete m;
    return fail(hip_status(e, "build events"));
  }
  void* nbr = nullptr;
  Status s = workspace_reserve(ws, table_bytes, stream);
  // nbr [n, 27], masks [n], counts [27]
  if (s.ok()) s = device_alloc(&nbr, (size_t)n * 28 * sizeof(int32_t) + 128, stream);
  if (!s.ok()) {
    device_free(nbr, stream);
    (void)hipEventDestroy(m->d.ready);
    delete m;
    return fail(s);
  }
  unsigned char* base = static_cast<unsigned char*>(ws.ptr);
  MapStats* dstats = reinterpret_cast<MapStats*>(base);
  void* partials = base + kStatsBytes;
  void* table = base + kStatsBytes + kPartialsBytes;

  m->d.nbr = static_cast<int32_t*>(nbr);
  m->d.masks = reinterpret_cast<uint32_t*>(m->d.nbr + (size_t)n * 27);
  m->d.dev_counts = m->d.masks + n;
  host->flags = 0;
  host->mode = kModeNone;
  host->duplicate = 0;
  host->overflow = 0;
  e = launch_map_build(coords, n, mode, table, partials, m->d.nbr, m->d.masks, m->d.dev_counts, dstats,
                       static_cast<MapHostFlags*>(pinned.dev), inserted, stream);
  if (e == hipSuccess) e = hipEventRecord(m->d.ready, stream);
  if (e == hipSuccess) e = hipEventRecord(ws.last, stream);
  // (Spinning on a host word that the lookup kernel stores as it starts measured slower than
  // this event wait.)
  if (e == hipSuccess) e = hipEventSynchronize(inserted);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(stream);
    release_map(m, stream);
    return fail(hip_status(e, "indice map build"));
  }
  const uint32_t flags = host->flags;
  int code = SUBM_OK;
  const char* msg = "";
  if (flags & kFlagBatchRange) {
    code = SUBM_ERR_COORD_RANGE;
    msg = "batch index outside [0, 65534]";
  } else if (flags & kFlagExtentRange) {
    code = SUBM_ERR_COORD_RANGE;
    msg = "extent (max - min) of z, y or x exceeds 65534";
  } else if (host->duplicate) {
    code = SUBM_ERR_DUPLICATE_COORD;
    msg = "two rows share the same (b, z, y, x)";
  } else if (host->overflow) {
    code = SUBM_ERR_HIP;
    msg = "internal error: hash table full";
  }
  if (code != SUBM_OK) {
    release_map(m, stream);
    return fail(code, msg);
  }
  m->d.mode = host->mode;
  *out_map = m;
  return SUBM_OK;
}

extern "C" int sparse_indice_map_build(const int32_t* coords, int64_t n, hipStream_t stream,
                                       submconv_map_t* out_map) {
  return sparse_indice_map_build_ex(coords, n, SUBM_MAP_AUTO, stream, out_map);
}

extern "C" int sparse_indice_map_mode(submconv_map_t map, int* mode) {
  clear_error();
  if (map == nullptr) return fail(SUBM_ERR_INVALID_ARG, "map is NULL");
  if (mode == nullptr) return fail(SUBM_ERR_INVALID_ARG, "mode is NULL");
  *mode = map->d.mode == kModeGrid ? SUBM_MAP_GRID : map->d.mode == kModeSubdivided ? SUBM_MAP_SUBDIVIDED : SUBM_MAP_HASH;
  return SUBM_OK;
}

Status submconv::map_counts(submconv_map* map) {
  std::lock_guard<std::mutex> lock(map->mu);
  if (map->d.counts_ready) return Status{};
  uint32_t c[27] = {};
  if (map->d.n > 0) {
    DeviceGuard guard(map->d.device);
    if (map->d.ready != nullptr) SUBM_HIP_TRY(hipEventSynchronize(map->d.ready));
    SUBM_HIP_TRY(hipMemcpy(c, map->d.dev_counts, sizeof(c), hipMemcpyDeviceToHost));
  }
  int64_t total = 0;
  for (int k = 0; k < 27; ++k) {
    map->d.per_tap[k] = c[k];
    total += c[k];
  }
  map->d.pairs = total;
  map->d.counts_ready = true;
  return Status{};
}

extern "C" int sparse_indice_map_free(submconv_map_t map) {
  clear_error();
  if (map == nullptr) return SUBM_OK;
  DeviceGuard guard(map->d.device);
  release_map(map, nullptr);
  return SUBM_OK;
}

extern "C" int sparse_indice_map_info(submconv_map_t map, int64_t* n, int64_t* pairs) {
  clear_error();
  if (map == nullptr) return fail(SUBM_ERR_INVALID_ARG, "map is NULL");
  if (n != nullptr) *n = map->d.n;
  if (pairs != nullptr) {
    Status s = map_counts(map);
    if (!s.ok()) return fail(s);
    *pairs = map->d.pairs;
  }
  return SUBM_OK;
}

extern "C" int sparse_indice_map_offset_counts(submconv_map_t map, int64_t* counts) {
  clear_error();
  if (map == nullptr) return fail(SUBM_ERR_INVALID_ARG, "map is NULL");
  if (counts == nullptr) return fail(SUBM_ERR_INVALID_ARG, "counts is NULL");
  Status s = map_counts(map);
  if (!s.ok()) return fail(s);
  std::memcpy(counts, map->d.per_tap, sizeof(map->d.per_tap));
  return SUBM_OK;
}

extern "C" int sparse_indice_map_copy_nbr(submconv_map_t map, int32_t* nbr, hipStream_t stream) {
  clear_error();
  if (map == nullptr) return fail(SUBM_ERR_INVALID_ARG, "map is NULL");
  if (map->d.n == 0) return SUBM_OK;
  if (nbr == nullptr) return fail(SUBM_ERR_INVALID_ARG, "nbr is NULL");
  hipError_t e = hipMemcpyAsync(nbr, map->d.nbr, (size_t)map->d.n * 27 * sizeof(int32_t), hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return fail(hip_status(e, "copy of nbr"));
  return SUBM_OK;
}

Status submconv::check_conv(submconv_map_t map, int64_t n, int ksize, int cin, int cout, int dtype, const void* feats,
                            const void* weight, const void* bias, const void* out) {
  if (ksize != 1 && ksize != 3) return make_status(SUBM_ERR_UNSUPPORTED, "ksize must be 1 or 3");
  if (dtype != SUBM_F32 && dtype != SUBM_F16 && dtype != SUBM_BF16)
    return make_status(SUBM_ERR_UNSUPPORTED, "dtype must be SUBM_F32, SUBM_F16 or SUBM_BF16");
  if (n < 0) return make_status(SUBM_ERR_INVALID_ARG, "n is negative");
  if (cin < 1 || cout < 1) return make_status(SUBM_ERR_INVALID_ARG, "cin and cout must be >= 1");
  if (cin > (1 << 24) || cout > (1 << 24)) return make_status(SUBM_ERR_INVALID_ARG, "cin / cout above 2^24");
  if (ksize == 3 && map == nullptr) return make_status(SUBM_ERR_INVALID_ARG, "map is NULL but ksize == 3");
  if (map != nullptr && map->d.n != n) return make_status(SUBM_ERR_SHAPE_MISMATCH, "n differs from the map's voxel count");
  if (n > INT32_MAX) return make_status(SUBM_ERR_INVALID_ARG, "n exceeds 2^31 - 1");
  if (n == 0) return Status{};
  if (feats == nullptr || weight == nullptr || out == nullptr)
    return make_status(SUBM_ERR_INVALID_ARG, "feats, weight or out is NULL");
  if (out == feats) return make_status(SUBM_ERR_INVALID_ARG, "out must not alias feats");
  const uintptr_t elem = dtype == SUBM_F32 ? 4 : 2;
  if ((reinterpret_cast<uintptr_t>(feats) | reinterpret_cast<uintptr_t>(weight) | reinterpret_cast<uintptr_t>(out) |
       reinterpret_cast<uintptr_t>(bias)) % elem != 0)
    return make_status(SUBM_ERR_INVALID_ARG, "a pointer is not aligned to the element size");
  if (map != nullptr) {
    int dev = -1;
    SUBM_HIP_TRY(hipGetDevice(&dev));
    if (dev != map->d.device) return make_status(SUBM_ERR_INVALID_ARG, "the map was built on another device");
  }
  return Status{};
}

extern "C" int subm_conv3d_forward(submconv_map_t map, int64_t n, int ksize, int cin, int cout, int dtype,
                                   const void* feats, const void* weight, const void* bias, void* out,
                                   hipStream_t stream) {
  clear_error();
  Status s = check_conv(map, n, ksize, cin, cout, dtype, feats, weight, bias, out);
  if (!s.ok()) return fail(s);
  if (n == 0) return SUBM_OK;
  hipError_t e = launch_subm_conv(map == nullptr ? nullptr : &map->d, n, ksize, cin, cout, dtype, feats, weight, bias, out, stream);
  if (e != hipSuccess) return fail(hip_status(e, "subm_conv3d_forward launch"));
  return SUBM_OK;
}

extern "C" int subm_conv3d_forward_per_offset(submconv_map_t map, int64_t n, int cin, int cout, int dtype,
                                              const void* feats, const void* weight, const void* bias, void* out,
                                              hipStream_t stream) {
  clear_error();
  if (map == nullptr) return fail(SUBM_ERR_INVALID_ARG, "map is NULL");
  if (dtype != SUBM_F16 && dtype != SUBM_BF16) return fail(SUBM_ERR_UNSUPPORTED, "dtype must be SUBM_F16 or SUBM_BF16");
  if (n < 0) return fail(SUBM_ERR_INVALID_ARG, "n is negative");
  if (cin < 1 || cout < 1) return fail(SUBM_ERR_INVALID_ARG, "cin and cout must be >= 1");
  if (cin % 8 != 0 || cout % 4 != 0) return fail(SUBM_ERR_UNSUPPORTED, "cin must be a multiple of 8 and cout of 4");
  if (map->d.n != n) return fail(SUBM_ERR_SHAPE_MISMATCH, "n differs from the map's voxel count");
  if ((uint64_t)n * (uint64_t)cin >= (1ull << 30) || (uint64_t)cout * 27u * (uint64_t)cin >= (1ull << 30))
    return fail(SUBM_ERR_UNSUPPORTED, "feats or weight exceed 2^30 elements");
  if (n == 0) return SUBM_OK;
  if (feats == nullptr || weight == nullptr || out == nullptr) return fail(SUBM_ERR_INVALID_ARG, "feats, weight or out is NULL");
  if (out == feats) return fail(SUBM_ERR_INVALID_ARG, "out must not alias feats");
  if (((reinterpret_cast<uintptr_t>(feats) | reinterpret_cast<uintptr_t>(weight)) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(out) & 7u) != 0 || (reinterpret_cast<uintptr_t>(bias) & 1u) != 0)
    return fail(SUBM_ERR_UNSUPPORTED, "feats / weight must be 16-byte aligned, out 8-byte, bias 2-byte");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(hip_status(e, "hipGetDevice"));
  if (dev != map->d.device) return fail(SUBM_ERR_INVALID_ARG, "the map was built on another device");
  {
    Status cs = map_counts(map);
    if (!cs.ok()) return fail(cs);
    std::lock_guard<std::mutex> lock(map->mu);
    const int64_t off_centre = map->d.pairs - map->d.per_tap[13];
    if (map->d.pair_out == nullptr && off_centre > 0) {
      void* pairs = nullptr;
      void* scratch = nullptr;
      Status s = device_alloc(&pairs, (size_t)off_centre * 2 * sizeof(int32_t), stream);
      if (s.ok()) s = device_alloc(&scratch, pair_scratch_ints(n) * sizeof(int32_t), stream);
      if (!s.ok()) {
        device_free(pairs, stream);
        return fail(s);
      }
      int32_t* po = static_cast<int32_t*>(pairs);
      e = launch_pair_lists(map->d, po, po + off_centre, static_cast<int32_t*>(scratch), stream);
      device_free(scratch, stream);
      if (e == hipSuccess) e = hipStreamSynchronize(stream);
      if (e != hipSuccess) {
        device_free(pairs, stream);
        return fail(hip_status(e, "pair lists"));
      }
      int64_t run = 0;
      for (int k = 0; k < 27; ++k) {
        map->d.pair_off[k] = run;
        if (k != 13) run += map->d.per_tap[k];
      }
      map->d.pair_in = po + off_centre;
      map->d.pair_out = po;
    }
  }
  void* acc = nullptr;
  Status s = device_alloc(&acc, (size_t)n * cout * sizeof(float), stream);
  if (!s.ok()) return fail(s);
  e = launch_subm_conv_per_offset(map->d, cin, cout, dtype, feats, weight, bias, out, static_cast<float*>(acc), stream);
  device_free(acc, stream);
  if (e != hipSuccess) return fail(hip_status(e, "subm_conv3d_forward_per_offset launch"));
  return SUBM_OK;
}

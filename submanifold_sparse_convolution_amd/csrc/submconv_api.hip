// C ABI entry points: argument validation, status codes, device memory, the map handle.
// Every check that does not need the GPU runs before any HIP call, so invalid arguments are
// rejected identically on a machine without a GPU.
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

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

namespace submconv {
namespace {
thread_local TimingEvents g_timing;
}  // namespace
TimingEvents take_timing_events() {
  const TimingEvents t = g_timing;
  g_timing = TimingEvents{};
  return t;
}
}  // namespace submconv

extern "C" int subm_timing_events(hipEvent_t start, hipEvent_t stop) {
  submconv::clear_error();
  submconv::g_timing.start = start;
  submconv::g_timing.stop = stop;
  return SUBM_OK;
}

namespace {

// Build workspace (statistics, bounds partials, the hash table area, the dense grid area): one
// grow-only device buffer per GPU, held under a mutex while a build is enqueued; builds on one GPU
// from several threads are serialised by the mutex.
struct Workspace {
  std::mutex mu;
  void* ptr = nullptr;
  size_t bytes = 0;
  size_t hash_cap = 0;     // bytes of the hash table area
  size_t grid_cap = 0;     // bytes of the grid area
  int64_t prev_n = 0;      // rows of the latest build on it (0: nothing to put back)
  uint32_t tag = 0;        // grid tag of the next build: every grid cell is all-ones or below it
  // The latest build's `ready` event (a pooled event, never destroyed): a build returns before
  // its last kernel has run, so the next build's kernels wait for it (on the device) before
  // they touch the shared structure.
  hipEvent_t last = nullptr;
};
Workspace g_workspace[kMaxDevices];

// Pool of flag slots per device: pinned pages of 16-byte slots, each with its event, created on
// demand with the device current and kept until the process ends.
struct SlotPool {
  std::mutex mu;
  std::vector<FlagSlot> free;
};
SlotPool g_slots[kMaxDevices];
constexpr size_t kSlotPage = 4096;

Status take_flag_slot(int dev, FlagSlot* out) {
  SlotPool& pool = g_slots[dev];
  std::lock_guard<std::mutex> lock(pool.mu);
  if (pool.free.empty()) {
    void* host = nullptr;
    void* devp = nullptr;
    SUBM_HIP_TRY(hipHostMalloc(&host, kSlotPage, hipHostMallocDefault));
    if (hipHostGetDevicePointer(&devp, host, 0) != hipSuccess) {
      (void)hipHostFree(host);
      return make_status(SUBM_ERR_HIP, "hipHostGetDevicePointer of the build flags");
    }
    for (size_t i = 0; i < kSlotPage / sizeof(MapHostFlags); ++i) {
      FlagSlot slot;
      slot.host = static_cast<MapHostFlags*>(host) + i;
      slot.dev = static_cast<MapHostFlags*>(devp) + i;
      pool.free.push_back(slot);
    }
  }
  FlagSlot& top = pool.free.back();
  // (kernel-completion events of hipExtLaunchKernel: created with timing)
  if (top.ready == nullptr) SUBM_HIP_TRY(hipEventCreate(&top.ready));
  *out = top;
  pool.free.pop_back();
  return Status{};
}

void give_flag_slot(int dev, FlagSlot& slot) {
  if (slot.host == nullptr) return;
  SlotPool& pool = g_slots[dev];
  std::lock_guard<std::mutex> lock(pool.mu);
  pool.free.push_back(slot);
  slot = FlagSlot{};
}

// The build's coordinate status from its flags (valid once the lookup kernel has completed).
Status read_flags(MapData& d) {
  const volatile MapHostFlags* host = d.slot.host;
  const uint32_t flags = host->flags;
  if (flags & kFlagBatchRange) return make_status(SUBM_ERR_COORD_RANGE, "batch index outside [0, 65534]");
  if (flags & kFlagExtentRange)
    return make_status(SUBM_ERR_COORD_RANGE, "extent (max - min) of z, y or x exceeds 65534");
  if (host->duplicate) return make_status(SUBM_ERR_DUPLICATE_COORD, "two rows share the same (b, z, y, x)");
  if (host->overflow) return make_status(SUBM_ERR_HIP, "internal error: hash table full");
  d.mode = host->mode;
  return Status{};
}

// Waits for the build's last kernel and reads the flags (caller holds the map's mutex or owns the
// map alone).
Status check_locked(MapData& d) {
  if (d.checked) return d.check;
  DeviceGuard guard(d.device);
  const hipError_t e = hipEventSynchronize(d.check_event);
  d.check = e != hipSuccess ? hip_status(e, "indice map build") : read_flags(d);
  d.checked = true;
  return d.check;
}

// Layout: [statistics | bounds partials | hash table area | grid area].  A new allocation has
// zeroed statistics (they say "nothing to put back"), both table areas all 0xFF bytes and tag 0.
constexpr size_t kStatsBytes = 4096;
constexpr size_t kPartialsBytes = 65536;
static_assert(sizeof(MapStats) <= kStatsBytes, "statistics block");

Status workspace_reserve(Workspace& ws, size_t hash_bytes, size_t grid_bytes, hipStream_t stream) {
  if (ws.hash_cap >= hash_bytes && ws.grid_cap >= grid_bytes) return Status{};
  if (ws.ptr != nullptr) {
    SUBM_HIP_TRY(hipFree(ws.ptr));  // waits for the device, so no build still uses it
    ws.ptr = nullptr;
    ws.bytes = 0;
  }
  const size_t head = kStatsBytes + kPartialsBytes;
  const size_t hash = hash_bytes > ws.hash_cap ? hash_bytes : ws.hash_cap;
  const size_t grid = grid_bytes > ws.grid_cap ? grid_bytes : ws.grid_cap;
  const size_t grain = size_t(64) << 20;
  const size_t want = (head + hash + grid + grain - 1) / grain * grain;
  SUBM_HIP_TRY(hipMalloc(&ws.ptr, want));
  ws.bytes = want;
  ws.hash_cap = hash;
  ws.grid_cap = want - head - hash;
  ws.prev_n = 0;
  ws.tag = 0;
  SUBM_HIP_TRY(launch_fill(ws.ptr, head, 0u, stream));
  SUBM_HIP_TRY(launch_fill(static_cast<unsigned char*>(ws.ptr) + head, want - head, 0xFFFFFFFFu, stream));
  return Status{};
}

// Largest tag + n a grid build may reach before the grid area is refilled (2^32 - 1, so that an
// all-ones cell is never an entry); SUBMCONV_GRID_TAG_LIMIT lowers it, so that tests reach the
// refill with small sets.
uint64_t grid_tag_limit() {
  const char* v = std::getenv("SUBMCONV_GRID_TAG_LIMIT");
  if (v != nullptr && *v != '\0') {
    const unsigned long long x = std::strtoull(v, nullptr, 10);
    if (x > 0 && x < 0xFFFFFFFFull) return x;
  }
  return 0xFFFFFFFFull;
}

static_assert(sizeof(MapHostFlags) == 16 && kSlotPage % sizeof(MapHostFlags) == 0, "flag slots tile a page");

// Rulebook (and neighbour-pool plan) blocks of freed maps, per device, for the next build (plan)
// on the same stream.  Returning a
// block to the stream-ordered pool and allocating it again each enqueue a marker packet (~3 us of
// idle GPU between two kernels, measured); a cached block costs nothing.  A block is cached only
// when every use of its map was on the map's own stream, so a later build on that stream writes
// it after all of them in stream order.  At most kCachedBlocks per device, kept until a build
// takes them (or the process ends): a block that does not fit goes back to the pool in order
// after the work on its stream.  Nothing is ever freed on a stream other than the block's own,
// whose work may still be running (a stream that is not synchronised with the null stream would
// not order such a free).
struct CachedBlock {
  void* ptr = nullptr;
  size_t bytes = 0;
  hipStream_t stream = nullptr;
};
struct BlockCache {
  std::mutex mu;
  std::vector<CachedBlock> blocks;
};
BlockCache g_blocks[kMaxDevices];
constexpr size_t kCachedBlocks = 8;
constexpr size_t kCachedBlockBytes = size_t(1) << 30;  // and at most 1 GiB of them per device

void release_map(submconv_map* m) {
  if (m->d.ready != nullptr) {
    (void)hipEventSynchronize(m->d.ready);  // the build's own kernels write the map memory
    if (m->d.slot.host == nullptr) (void)hipEventDestroy(m->d.ready);  // a derived map's own event
  }
  give_flag_slot(m->d.device, m->d.slot);
  if (m->d.pool_slot.ready != nullptr) (void)hipEventSynchronize(m->d.pool_slot.ready);  // the plan kernel
  give_flag_slot(m->d.device, m->d.pool_slot);
  map_memory_give(m->d.device, m->d.nbr, m->d.nbr_bytes, m->d.home,
                  !m->other_streams.load(std::memory_order_relaxed));
  device_free(m->d.pair_out, m->d.home);  // (work on other streams has completed: the free rules)
  // the plan block goes to the cache when the plan and every use of the map ran on the map's stream
  map_memory_give(m->d.device, m->d.pool_plan, m->d.pool_plan_bytes, m->d.home,
                  !m->other_streams.load(std::memory_order_relaxed) && m->d.pool_stream == m->d.home);
  device_free(m->d.order_block, m->d.order_stream);  // (in order after the calls that used it)
  delete m;
}

}  // namespace

namespace {
// Per-(device, stream) scratch buffers (packed weights of the neighbour-pool convolution): at
// most kScratchStreams per device; the oldest goes back to the pool, in order after the work on
// its own stream, when a new stream needs one.
struct ScratchEntry {
  hipStream_t stream = nullptr;
  void* ptr = nullptr;
  size_t bytes = 0;
};
struct ScratchCache {
  std::mutex mu;
  std::vector<ScratchEntry> entries;
};
ScratchCache g_scratch[kMaxDevices];
constexpr size_t kScratchStreams = 16;
}  // namespace

Status submconv::stream_scratch(int dev, hipStream_t stream, size_t bytes, void** ptr) {
  *ptr = nullptr;
  if (dev < 0 || dev >= kMaxDevices) return make_status(SUBM_ERR_HIP, "device ordinal out of range");
  ScratchCache& c = g_scratch[dev];
  std::lock_guard<std::mutex> lock(c.mu);
  for (size_t i = 0; i < c.entries.size(); ++i) {
    ScratchEntry& e = c.entries[i];
    if (e.stream != stream) continue;
    if (e.bytes >= bytes) {
      *ptr = e.ptr;
      return Status{};
    }
    device_free(e.ptr, e.stream);  // in order after this stream's earlier work
    c.entries.erase(c.entries.begin() + i);
    break;
  }
  if (c.entries.size() >= kScratchStreams) {
    device_free(c.entries.front().ptr, c.entries.front().stream);
    c.entries.erase(c.entries.begin());
  }
  const size_t want = round_up(bytes, size_t(1) << 20);
  void* p = nullptr;
  Status s = device_alloc(&p, want, stream);
  if (!s.ok()) return s;
  ScratchEntry e;
  e.stream = stream;
  e.ptr = p;
  e.bytes = want;
  c.entries.push_back(e);
  *ptr = p;
  return Status{};
}

Status submconv::map_memory_take(int dev, size_t bytes, hipStream_t stream, void** ptr, size_t* got) {
  *ptr = nullptr;
  *got = 0;
  if (dev >= 0 && dev < kMaxDevices) {
    BlockCache& cache = g_blocks[dev];
    std::lock_guard<std::mutex> lock(cache.mu);
    int best = -1;
    for (size_t i = 0; i < cache.blocks.size(); ++i) {
      const CachedBlock& b = cache.blocks[i];
      // (at most twice the size asked for, so a small map does not hold a large block)
      if (b.stream == stream && b.bytes >= bytes && b.bytes / 2 <= bytes &&
          (best < 0 || b.bytes < cache.blocks[best].bytes))
        best = (int)i;
    }
    if (best >= 0) {
      *ptr = cache.blocks[best].ptr;
      *got = cache.blocks[best].bytes;
      cache.blocks.erase(cache.blocks.begin() + best);
      return Status{};
    }
  }
  Status s = device_alloc(ptr, bytes, stream);
  if (s.ok()) *got = bytes;
  return s;
}

void submconv::map_memory_give(int dev, void* ptr, size_t bytes, hipStream_t stream, bool reusable) {
  if (ptr == nullptr) return;
  if (reusable && dev >= 0 && dev < kMaxDevices) {
    BlockCache& cache = g_blocks[dev];
    std::lock_guard<std::mutex> lock(cache.mu);
    size_t held = 0;
    for (const CachedBlock& b : cache.blocks) held += b.bytes;
    if (cache.blocks.size() < kCachedBlocks && held + bytes <= kCachedBlockBytes) {
      CachedBlock b;
      b.ptr = ptr;
      b.bytes = bytes;
      b.stream = stream;
      cache.blocks.push_back(b);
      return;
    }
  }
  device_free(ptr, stream);
}

namespace {

// Shared by the synchronous and asynchronous builds; `wait` selects whether the coordinate
// check happens before returning.
int build_map(const int32_t* coords, int64_t n, int mode, hipStream_t stream, submconv_map_t* out_map, bool wait) {
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
  const size_t hash_bytes = round_up(map_hash_bytes(n), 256);
  const size_t grid_bytes = round_up(map_grid_bytes(n), 256);
  if (map_partials_bytes(n) > kPartialsBytes) {
    delete m;
    return fail(SUBM_ERR_HIP, "internal error: bounds partials exceed their workspace block");
  }
  Status s = take_flag_slot(m->d.device, &m->d.slot);
  if (!s.ok()) {
    delete m;
    return fail(s);
  }
  m->d.checked = false;
  volatile MapHostFlags* host = m->d.slot.host;

  Workspace& ws = g_workspace[m->d.device];
  std::lock_guard<std::mutex> lock(ws.mu);
  // (an event already complete needs no wait packet on the stream)
  hipError_t e = ws.last == nullptr || hipEventQuery(ws.last) == hipSuccess ? hipSuccess
                                                                            : hipStreamWaitEvent(stream, ws.last, 0);
  if (e != hipSuccess) {
    release_map(m);
    return fail(hip_status(e, "build events"));
  }
  void* nbr = nullptr;
  size_t nbr_bytes = 0;
  s = workspace_reserve(ws, hash_bytes, grid_bytes, stream);
  if (s.ok() && (uint64_t)ws.tag + (uint64_t)n > grid_tag_limit()) {
    // The grid's tags would run out: back to all-ones (once per ~2^32 / n builds).
    const hipError_t fe = launch_fill(static_cast<unsigned char*>(ws.ptr) + kStatsBytes + kPartialsBytes + ws.hash_cap,
                                      ws.grid_cap, 0xFFFFFFFFu, stream);
    if (fe != hipSuccess) s = hip_status(fe, "grid refill");
    ws.tag = 0;
  }
  // nbr [n, 27], masks [n], counter banks [kTapBanks, 27]
  if (s.ok())
    s = map_memory_take(m->d.device, (size_t)n * 28 * sizeof(int32_t) + kTapBanks * 27 * sizeof(uint32_t), stream,
                        &nbr, &nbr_bytes);
  if (!s.ok()) {
    release_map(m);
    return fail(s);
  }
  unsigned char* base = static_cast<unsigned char*>(ws.ptr);
  MapStats* dstats = reinterpret_cast<MapStats*>(base);
  void* partials = base + kStatsBytes;
  void* hash_table = base + kStatsBytes + kPartialsBytes;
  int32_t* grid = reinterpret_cast<int32_t*>(base + kStatsBytes + kPartialsBytes + ws.hash_cap);

  m->d.nbr = static_cast<int32_t*>(nbr);
  m->d.nbr_bytes = nbr_bytes;
  m->d.home = stream;
  m->d.masks = reinterpret_cast<uint32_t*>(m->d.nbr + (size_t)n * 27);
  m->d.dev_banks = m->d.masks + n;
  host->flags = 0;
  host->mode = kModeNone;
  host->duplicate = 0;
  host->overflow = 0;
  m->d.ready = m->d.slot.ready;
  m->d.check_event = m->d.ready;
  e = launch_map_build(coords, n, mode, hash_table, grid, ws.tag, partials, ws.prev_n, m->d.nbr, m->d.masks,
                       m->d.dev_banks, dstats, m->d.slot.dev, m->d.ready, stream);
  ws.prev_n = n;  // from here on the tables hold this build's entries (or the launch failed)
  ws.tag += (uint32_t)n;
  if (e == hipSuccess) ws.last = m->d.ready;
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(stream);
    release_map(m);
    return fail(hip_status(e, "indice map build"));
  }
  if (wait) {
    // (Spinning on a host word that the lookup kernel stores as it starts measured slower than
    // this event wait.)
    s = check_locked(m->d);
    if (!s.ok()) {
      release_map(m);
      return fail(s);
    }
  }
  *out_map = m;
  return SUBM_OK;
}

}  // namespace

extern "C" int sparse_indice_map_build_ex(const int32_t* coords, int64_t n, int mode, hipStream_t stream,
                                          submconv_map_t* out_map) {
  return build_map(coords, n, mode, stream, out_map, true);
}

extern "C" int sparse_indice_map_build_async(const int32_t* coords, int64_t n, int mode, hipStream_t stream,
                                             submconv_map_t* out_map) {
  return build_map(coords, n, mode, stream, out_map, false);
}

extern "C" int sparse_indice_map_status(submconv_map_t map) {
  clear_error();
  if (map == nullptr) return fail(SUBM_ERR_INVALID_ARG, "map is NULL");
  const Status s = map_check(map);
  return s.ok() ? SUBM_OK : fail(s);
}

extern "C" int sparse_indice_map_build(const int32_t* coords, int64_t n, hipStream_t stream,
                                       submconv_map_t* out_map) {
  return sparse_indice_map_build_ex(coords, n, SUBM_MAP_AUTO, stream, out_map);
}

extern "C" int sparse_indice_map_mode(submconv_map_t map, int* mode) {
  clear_error();
  if (map == nullptr) return fail(SUBM_ERR_INVALID_ARG, "map is NULL");
  if (mode == nullptr) return fail(SUBM_ERR_INVALID_ARG, "mode is NULL");
  const Status s = map_check(map);
  if (!s.ok()) return fail(s);
  *mode = map->d.mode == kModeGrid ? SUBM_MAP_GRID : map->d.mode == kModeSubdivided ? SUBM_MAP_SUBDIVIDED : SUBM_MAP_HASH;
  return SUBM_OK;
}

Status submconv::map_check(submconv_map* map) {
  std::lock_guard<std::mutex> lock(map->mu);
  return check_locked(map->d);
}

Status submconv::map_counts(submconv_map* map) {
  std::lock_guard<std::mutex> lock(map->mu);
  const Status cs = check_locked(map->d);
  if (!cs.ok()) return cs;
  if (map->d.counts_ready) return Status{};
  uint32_t banks[kTapBanks][27] = {};
  if (map->d.n > 0) {
    DeviceGuard guard(map->d.device);
    if (map->d.ready != nullptr) SUBM_HIP_TRY(hipEventSynchronize(map->d.ready));
    SUBM_HIP_TRY(hipMemcpy(banks, map->d.dev_banks, sizeof(banks), hipMemcpyDeviceToHost));
  }
  int64_t total = 0;
  for (int k = 0; k < 27; ++k) {
    int64_t c = 0;
    for (int b = 0; b < kTapBanks; ++b) c += banks[b][k];
    map->d.per_tap[k] = c;
    total += c;
  }
  map->d.pairs = total;
  map->d.counts_ready = true;
  return Status{};
}

extern "C" int sparse_indice_map_free(submconv_map_t map) {
  clear_error();
  if (map == nullptr) return SUBM_OK;
  DeviceGuard guard(map->d.device);
  release_map(map);
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
  const Status s = map_check(map);
  if (!s.ok()) return fail(s);
  map_note_use(map, stream);
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

namespace {

// Whether a convolution takes the neighbour-pool kernel (conv_pool.hip): k = 3, 16-bit storage,
// 128 output channels, cin a multiple of 32, 16-byte aligned tensors, features within 31-bit
// offsets, enough rows for one full tile per compute unit, and a plan that did not overflow.
// SUBMCONV_POOL=0 or a forced conv.hip tile (SUBMCONV_TILE) keep the conv.hip kernels.
bool pool_eligible(const submconv_map* map, int64_t n, int ksize, int cin, int cout, int dtype, const void* feats,
                   const void* weight, const void* out) {
  if (map == nullptr || ksize != 3 || cout != 128 || (dtype != SUBM_BF16 && dtype != SUBM_F16)) return false;
  if (cin < 32 || cin % 32 != 0 || map->d.pool_state == 3) return false;
  if (((reinterpret_cast<uintptr_t>(feats) | reinterpret_cast<uintptr_t>(weight) | reinterpret_cast<uintptr_t>(out) |
        reinterpret_cast<uintptr_t>(map->d.nbr)) & 15u) != 0)
    return false;
  if ((uint64_t)n * (uint64_t)cin * 2u >= 0x7FFFF000ull) return false;
  const char* v = std::getenv("SUBMCONV_POOL");
  if ((v != nullptr && v[0] == '0') || std::getenv("SUBMCONV_TILE") != nullptr) return false;
  PoolTiling t;
  return pool_tiling(n, &t);
}

// Builds the map's plan on first use (enqueued on `stream`; the overflow flag arrives in the
// plan's pinned word) and reads the flag once the plan kernel has completed.  Returns the
// map's pool_state (1: built, flag not read yet; 2: usable; 3: overflowed).
Status pool_prepare(submconv_map* map, hipStream_t stream, int* state) {
  std::lock_guard<std::mutex> lock(map->mu);
  MapData& d = map->d;
  if (d.pool_state == 0) {
    PoolTiling t;
    if (!pool_tiling(d.n, &t)) return make_status(SUBM_ERR_HIP, "internal error: no neighbour-pool tiling");
    Status s = take_flag_slot(d.device, &d.pool_slot);
    if (!s.ok()) return s;
    d.pool_slot.host->flags = 0u;
    // (a block of a freed map's plan on this stream when one fits: no allocator packet between the
    // build's kernels and the plan kernel)
    s = map_memory_take(d.device, pool_plan_bytes(t), stream, &d.pool_plan, &d.pool_plan_bytes);
    if (!s.ok()) {
      give_flag_slot(d.device, d.pool_slot);
      return s;
    }
    const hipError_t e = launch_pool_plan(d.nbr, d.n, t, d.pool_plan, &d.pool_slot.dev->flags, d.pool_slot.ready, stream);
    if (e != hipSuccess) return hip_status(e, "neighbour-pool plan");
    d.pool_tiling = t;
    d.pool_state = 1;
    d.pool_stream = stream;
  }
  if (d.pool_state == 1 && hipEventQuery(d.pool_slot.ready) == hipSuccess)
    d.pool_state = reinterpret_cast<volatile MapHostFlags*>(d.pool_slot.host)->flags != 0u ? 3 : 2;
  // work on another stream than the plan's waits for the plan kernel
  if (d.pool_state == 1 && stream != d.pool_stream) SUBM_HIP_TRY(hipStreamWaitEvent(stream, d.pool_slot.ready, 0));
  *state = d.pool_state;
  return Status{};
}

}  // namespace

extern "C" int subm_release_cached_memory(void) {
  clear_error();
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(SUBM_ERR_HIP, "subm_release_cached_memory: no current device");
  Workspace& ws = g_workspace[dev];
  BlockCache& cache = g_blocks[dev];
  ScratchCache& sc = g_scratch[dev];
  // hold every cache while the device drains, so that nothing new is enqueued on their memory
  std::lock_guard<std::mutex> l1(ws.mu);
  std::lock_guard<std::mutex> l2(cache.mu);
  std::lock_guard<std::mutex> l3(sc.mu);
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(hip_status(e, "subm_release_cached_memory"));
  if (ws.ptr != nullptr) {
    e = hipFree(ws.ptr);
    ws.ptr = nullptr;
    ws.bytes = 0;
    ws.hash_cap = 0;
    ws.grid_cap = 0;
    ws.prev_n = 0;
    ws.tag = 0;
    if (e != hipSuccess) return fail(hip_status(e, "subm_release_cached_memory workspace"));
  }
  for (const CachedBlock& b : cache.blocks) device_free(b.ptr, b.stream);
  cache.blocks.clear();
  for (const ScratchEntry& x : sc.entries) device_free(x.ptr, x.stream);
  sc.entries.clear();
  e = hipDeviceSynchronize();  // (the stream-ordered frees above)
  if (e != hipSuccess) return fail(hip_status(e, "subm_release_cached_memory"));
  return SUBM_OK;
}

extern "C" int sparse_indice_map_plan_state(submconv_map_t map, int* state) {
  clear_error();
  if (map == nullptr) return fail(SUBM_ERR_INVALID_ARG, "map is NULL");
  if (state == nullptr) return fail(SUBM_ERR_INVALID_ARG, "state is NULL");
  std::lock_guard<std::mutex> lock(map->mu);
  MapData& d = map->d;
  if (d.pool_state == 1 && hipEventQuery(d.pool_slot.ready) == hipSuccess)
    d.pool_state = reinterpret_cast<volatile MapHostFlags*>(d.pool_slot.host)->flags != 0u ? 3 : 2;
  *state = d.pool_state;
  return SUBM_OK;
}

extern "C" int sparse_indice_map_row_order_state(submconv_map_t map, int* state) {
  clear_error();
  if (map == nullptr) return fail(SUBM_ERR_INVALID_ARG, "map is NULL");
  if (state == nullptr) return fail(SUBM_ERR_INVALID_ARG, "state is NULL");
  std::lock_guard<std::mutex> lock(map->mu);
  const MapData& d = map->d;
  if (d.order_block == nullptr) {
    *state = SUBM_ORDER_NONE;
    return SUBM_OK;
  }
  uint32_t gate = 0;
  hipError_t e = hipMemcpyAsync(&gate, order_view(d.order_block, d.n).gate, sizeof(gate), hipMemcpyDeviceToHost,
                                d.order_stream);
  if (e == hipSuccess) e = hipStreamSynchronize(d.order_stream);
  if (e != hipSuccess) return fail(hip_status(e, "row order gate read"));
  *state = gate != 0u ? SUBM_ORDER_ON : SUBM_ORDER_OFF;
  return SUBM_OK;
}

namespace {
// SUBMCONV_ROW_ORDER=0 keeps every map in its input row order (timing and tests).
bool row_order_enabled() {
  const char* v = std::getenv("SUBMCONV_ROW_ORDER");
  return v == nullptr || v[0] != '0';
}
}  // namespace

extern "C" int subm_conv3d_forward(submconv_map_t map, int64_t n, int ksize, int cin, int cout, int dtype,
                                   const void* feats, const void* weight, const void* bias, void* out,
                                   hipStream_t stream) {
  clear_error();
  Status s = check_conv(map, n, ksize, cin, cout, dtype, feats, weight, bias, out);
  if (!s.ok()) return fail(s);
  if (n == 0) return SUBM_OK;
  map_note_use(map, stream);
  if (pool_eligible(map, n, ksize, cin, cout, dtype, feats, weight, out)) {
    // (the plan needs no coordinate check first: every rulebook entry is -1 or a row of the set,
    // whatever the coordinates were)
    int state = 0;
    s = pool_prepare(map, stream, &state);
    if (!s.ok()) return fail(s);
    if (state != 3) {
      void* wpk = nullptr;
      s = stream_scratch(map->d.device, stream, pool_weight_bytes(cin), &wpk);
      if (!s.ok()) return fail(s);
      // state 1: the plan's flags are not known on the host yet, so the conv.hip kernel is launched
      // behind the pool kernel and each of the two runs only if the tile flags say it should
      const uint32_t* gate = state == 1 ? pool_tile_flags(map->d.pool_tiling, map->d.pool_plan) : nullptr;
      hipError_t e = launch_pool_conv(map->d.pool_tiling, map->d.pool_plan, gate, n, cin, dtype, feats, weight, bias, out,
                                      wpk, stream);
      if (e == hipSuccess && gate != nullptr)
        e = launch_subm_conv(&map->d, n, ksize, cin, cout, dtype, feats, weight, bias, out, stream, gate,
                             pool_flag_count(map->d.pool_tiling));
      if (e != hipSuccess) return fail(hip_status(e, "subm_conv3d_forward launch"));
      return SUBM_OK;
    }
  }
  // A large map's second convolution on the matrix-core walk enqueues its sparse-row order (built
  // only where rows have few neighbours, decided on the device; row_order.hip).
  std::unique_lock<std::mutex> order_lock;
  if (map != nullptr) order_lock = std::unique_lock<std::mutex>(map->mu);
  if (ksize == 3 && n >= kOrderMinRows && dtype != SUBM_F32 && cout > 32 && map->d.order_block == nullptr &&
      stream == map->d.home && !map->other_streams.load(std::memory_order_relaxed) && row_order_enabled() &&
      ++map->d.order_calls == 2) {
    void* blk = nullptr;
    void* scr = nullptr;
    hipError_t e = hipMallocAsync(&blk, order_block_bytes(n), stream);
    if (e != hipSuccess) return fail(hip_status(e, "row order allocation"));
    s = stream_scratch(map->d.device, stream, order_scratch_bytes(n), &scr);
    if (!s.ok()) {
      device_free(blk, stream);
      return fail(s);
    }
    e = launch_row_order(&map->d, blk, scr, stream);
    if (e != hipSuccess) {
      device_free(blk, stream);
      return fail(hip_status(e, "row order launch"));
    }
    map->d.order_block = blk;
    map->d.order_stream = stream;
  }
  hipError_t e = launch_subm_conv(map == nullptr ? nullptr : &map->d, n, ksize, cin, cout, dtype, feats, weight, bias, out, stream);
  if (e != hipSuccess) return fail(hip_status(e, "subm_conv3d_forward launch"));
  return SUBM_OK;
}

// ---------------------------------------------------------------------------------------------
// subm_conv3d_forward_noalloc: subm_conv3d_forward without any device allocation.  The one
// scratch buffer of the convolution (the packed weights of the neighbour-pool kernel) is this
// file-scope array; each device holds its own copy until the process ends, and its device
// address is looked up once per device (host code never passes the array's name to a kernel).
namespace {
constexpr size_t kNoAllocScratchBytes = (size_t)27 * 128 * 256 * 2;  // packed weights, cin <= 256
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};

Status noalloc_scratch(int dev, void** ptr) {
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (g_noalloc_ptr[dev] == nullptr) {
    void* p = nullptr;
    SUBM_HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr) return make_status(SUBM_ERR_HIP, "hipGetSymbolAddress returned no address for the scratch array");
    g_noalloc_ptr[dev] = p;
  }
  *ptr = g_noalloc_ptr[dev];
  return Status{};
}
}  // namespace

extern "C" int subm_conv3d_forward_noalloc(submconv_map_t map, int64_t n, int ksize, int cin, int cout, int dtype,
                                           const void* feats, const void* weight, const void* bias, void* out,
                                           hipStream_t stream) {
  clear_error();
  Status s = check_conv(map, n, ksize, cin, cout, dtype, feats, weight, bias, out);
  if (!s.ok()) return fail(s);
  if (n == 0) return SUBM_OK;
  map_note_use(map, stream);
  if (pool_eligible(map, n, ksize, cin, cout, dtype, feats, weight, out)) {
    int state = 0;
    {
      std::lock_guard<std::mutex> lock(map->mu);
      MapData& d = map->d;
      if (d.pool_state == 1 && hipEventQuery(d.pool_slot.ready) == hipSuccess)
        d.pool_state = reinterpret_cast<volatile MapHostFlags*>(d.pool_slot.host)->flags != 0u ? 3 : 2;
      if (d.pool_state == 1 && stream != d.pool_stream) {
        const hipError_t we = hipStreamWaitEvent(stream, d.pool_slot.ready, 0);
        if (we != hipSuccess) return fail(hip_status(we, "subm_conv3d_forward_noalloc stream wait"));
      }
      state = d.pool_state;
    }
    // (no plan yet: building one allocates, so the general kernels run instead)
    if (state == 1 || state == 2) {
      if (pool_weight_bytes(cin) > kNoAllocScratchBytes)
        return fail(SUBM_ERR_UNSUPPORTED, "subm_conv3d_forward_noalloc: cin above 256 needs more packed-weight "
                                          "workspace than its static 1.7 MB");
      int dev = -1;
      if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(SUBM_ERR_HIP, "subm_conv3d_forward_noalloc: no current device");
      void* wpk = nullptr;
      s = noalloc_scratch(dev, &wpk);
      if (!s.ok()) return fail(s);
      const uint32_t* gate = state == 1 ? pool_tile_flags(map->d.pool_tiling, map->d.pool_plan) : nullptr;
      hipError_t e = launch_pool_conv(map->d.pool_tiling, map->d.pool_plan, gate, n, cin, dtype, feats, weight, bias, out,
                                      wpk, stream);
      if (e == hipSuccess && gate != nullptr)
        e = launch_subm_conv(&map->d, n, ksize, cin, cout, dtype, feats, weight, bias, out, stream, gate,
                             pool_flag_count(map->d.pool_tiling));
      if (e != hipSuccess) return fail(hip_status(e, "subm_conv3d_forward_noalloc launch"));
      return SUBM_OK;
    }
  }
  hipError_t e = launch_subm_conv(map == nullptr ? nullptr : &map->d, n, ksize, cin, cout, dtype, feats, weight, bias, out, stream);
  if (e != hipSuccess) return fail(hip_status(e, "subm_conv3d_forward_noalloc launch"));
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
  map_note_use(map, stream);
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

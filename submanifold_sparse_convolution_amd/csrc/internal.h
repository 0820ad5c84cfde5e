// Internal declarations shared by the host entry points and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
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

#define SUBM_HIP_TRY(expr)                                          \
  do {                                                              \
    hipError_t _e = (expr);                                         \
    if (_e != hipSuccess) return ::submconv::hip_status(_e, #expr); \
  } while (0)

// Stream-ordered device allocation from the per-device pool (submconv_api.hip).
Status device_alloc(void** ptr, size_t bytes, hipStream_t stream);
void device_free(void* ptr, hipStream_t stream);

// Thread-local error detail of the C entry points (submconv_api.hip): clear_error() at entry,
// fail() stores the message and returns the code.
void clear_error();
int fail(const Status& s);
int fail(int code, const char* msg);

// Per-thread, per-device pinned host block of kPinnedBytes that the device can write (for the
// few words a build reads back after its synchronisation).  host == nullptr on failure.
constexpr size_t kPinnedBytes = 4096;
struct Pinned {
  void* host = nullptr;
  void* dev = nullptr;
};
Pinned pinned_block(int dev);

// Restores the caller's current device on scope exit.
struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// Measurement hook (subm_timing_events): the events that this thread's next convolution kernel
// records (its own start and completion, bound to its dispatch); take_timing_events() returns
// them and clears the request.
struct TimingEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
TimingEvents take_timing_events();
// Launches kernel(a) on `stream`, binding a pending timing request to it.
template <typename F, typename A>
inline void launch_kernel_timed(F kernel, dim3 grid, dim3 block, hipStream_t stream, const A& a) {
  const TimingEvents te = take_timing_events();
  if (te.start == nullptr && te.stop == nullptr) kernel<<<grid, block, 0, stream>>>(a);
  else hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, te.start, te.stop, 0u, a);
}

// Map build constants.
constexpr int kTapBanks = 16;               // tap hit counters are spread over banks of 27
constexpr int64_t kGridCellsPerVoxel = 128;       // dense grid allowed up to this many cells per voxel
constexpr int64_t kGridMaxCells = int64_t(1) << 29;  // ... and at most 2 GiB of int32 cells
constexpr int kModeNone = -1;               // coordinates out of range: nothing built
constexpr int kModeHash = 0;
constexpr int kModeGrid = 1;
constexpr int kModeSubdivided = 2;           // derived from a parent map, no structure

constexpr uint32_t kFlagDuplicate = 1u;
constexpr uint32_t kFlagBatchRange = 2u;
constexpr uint32_t kFlagProbeOverflow = 4u;
constexpr uint32_t kFlagExtentRange = 8u;

// Words the build's kernels (the insert kernel's plan and hash inserts, the lookup kernel's grid
// duplicate check) write straight into pinned host memory; the host reads them once the lookup
// kernel has completed.
struct MapHostFlags {
  uint32_t flags;      // kFlag* range bits of the plan
  int32_t mode;        // kMode* of the plan
  uint32_t duplicate;  // 1: a cell or key was taken twice
  uint32_t overflow;   // 1: the hash probe ran out of slots
};

// Device-side plan of the latest build on a workspace, published by the insert kernel's block 0
// for the lookup kernel and for the next build's first kernel (which puts a hash build's slots
// back).
struct MapStats {
  int32_t mn[4];       // per-column minimum of (b, z, y, x)
  int32_t mx[4];       // per-column maximum
  uint32_t flags;      // kFlag* bits of the plan (coordinate ranges)
  uint32_t err_flags;  // kFlag* bits raised while inserting (duplicates, probe overflow)
  int32_t mode;        // kMode*
  uint32_t pad;
  int64_t cells;       // GRID: number of cells
  int64_t slots;       // HASH: number of slots
  int64_t sy, sz, sb;  // GRID strides of y, z and the batch slab (x stride is 1)
};

// Where a build's flags arrive: a 16-byte slot of pinned host memory that the kernels write
// through its device address, and an event recorded after the build's last kernel.  Slots come from a
// per-device pool (submconv_api.hip) and go back once the map has been checked or freed, so
// several asynchronous builds can be in flight at once.
struct FlagSlot {
  MapHostFlags* host = nullptr;
  MapHostFlags* dev = nullptr;
  hipEvent_t ready = nullptr;     // recorded after the build's last kernel
};

// Tiling of the neighbour-pool convolution (conv_pool.hip): tile t covers row blocks of 32
// [t nb / ntiles, (t + 1) nb / ntiles) (16 or 17 blocks; e = 1 when some tile has 17), workgroup
// v takes tiles [v per_wg, (v + 1) per_wg).
struct PoolTiling {
  int nb = 0;
  int ntiles = 0;
  int per_wg = 0;
  int e = 0;
};

// Map handle contents.
struct MapData {
  int device = 0;
  int mode = kModeHash;
  int64_t n = 0;
  // Pair counts: valid once counts_ready (the build's lookup may still run when it returns; the
  // counts arrive in dev_banks and are read on first use, see map_counts()).
  bool counts_ready = false;
  int64_t pairs = 0;
  int64_t per_tap[27] = {};
  int32_t* nbr = nullptr;     // device [n, 27], input row order
  size_t nbr_bytes = 0;       // bytes of the allocation that starts at nbr
  hipStream_t home = nullptr;  // the stream whose build wrote nbr / masks
  uint32_t* masks = nullptr;  // device [n]: bit k set when nbr[i, k] >= 0 (same allocation as nbr)
  uint32_t* dev_banks = nullptr;   // device [kTapBanks][27] per-tap pair counts, summed on the host
                                   // (same allocation as nbr)
  hipEvent_t ready = nullptr;      // recorded after the build's last kernel (the slot's event for
                                   // a built map, the map's own for a derived one)
  // Coordinate check of the build (range, duplicates): `checked` once its flags have been read
  // (a synchronous build reads them before it returns, an asynchronous one on first use, see
  // map_check()); `check` is the result; `slot` is held until the map is freed.
  bool checked = true;
  Status check;
  FlagSlot slot;
  hipEvent_t check_event = nullptr;  // the event whose completion makes the flags valid
  // Per-tap pair lists of the per-offset convolution, built on first use: the pairs of tap k
  // (k != 13) are pair_out / pair_in [pair_off[k] .. pair_off[k] + per_tap[k]), output row
  // ascending.  One allocation, pair_out first.
  int32_t* pair_out = nullptr;
  int32_t* pair_in = nullptr;
  int64_t pair_off[27] = {};
  // Neighbour-pool plan of the 128-channel convolution (conv_pool.hip), built by the first
  // convolution that takes that path.  pool_state: 0 not built, 1 built but its overflow flag
  // not read yet, 2 usable, 3 a sub-pool overflowed (that map keeps the conv.hip kernels).
  int pool_state = 0;
  PoolTiling pool_tiling;
  void* pool_plan = nullptr;
  size_t pool_plan_bytes = 0;  // bytes of the block that starts at pool_plan
  hipStream_t pool_stream = nullptr;  // the stream the plan kernel ran on
  FlagSlot pool_slot;  // .host->flags / .dev: the overflow flag; .ready: the plan kernel's completion
  // Row order of the persistent 27-tap convolution (row_order.hip), enqueued by the map's second
  // convolution on that path when the set is large enough; used by the calls on order_stream.
  int order_calls = 0;
  void* order_block = nullptr;
  hipStream_t order_stream = nullptr;
};

// Map build (indice_map.hip).  Enqueues on `stream`; does not synchronise.  `hash_table` holds
// map_hash_bytes(n) and is all 0xFF bytes except for the slots of the previous build on this
// workspace if that was a hash build (the first kernel puts those back); `grid` holds
// map_grid_bytes(n) int32 cells, each either 0xFFFFFFFF or tag' + row of an earlier build with
// tag' + its n <= `tag`, and tag + n <= 2^32 - 1.  `stats` (one MapStats, device) still describes the
// previous build on this workspace (all zero for none; `prev_n` is its row count, 0 for none).
// `partials` holds map_partials_bytes(n).  `host_flags` (device address of pinned host memory,
// zeroed by the caller) holds the plan's flags and mode and the duplicate / overflow flags, and
// the per-tap counts reach `banks` (device [kTapBanks][27], to be summed), once `ready` (the
// lookup kernel's completion; it must allow timing) has completed.
int64_t map_hash_slots(int64_t n);
int64_t map_grid_budget_cells(int64_t n);
int map_bounds_blocks(int64_t n);
size_t map_hash_bytes(int64_t n);
size_t map_grid_bytes(int64_t n);
size_t map_partials_bytes(int64_t n);
hipError_t launch_map_build(const int32_t* coords, int64_t n, int mode_request, void* hash_table, int32_t* grid,
                            uint32_t tag, void* partials, int64_t prev_n, int32_t* nbr, uint32_t* masks,
                            uint32_t* banks, MapStats* stats, MapHostFlags* host_flags, hipEvent_t ready,
                            hipStream_t stream);
// Fill `bytes` bytes at `p` (16-byte aligned, bytes a multiple of 16) with `value` (each 32-bit
// word).
hipError_t launch_fill(void* p, size_t bytes, uint32_t value, hipStream_t stream);

// Prefix sum of n int32 (sort_scan.hip): out[i] = in[0] + ... + in[i] (inclusive) or the sum
// before i (exclusive); out may equal in; both 16-byte aligned.  scratch: scan_scratch_bytes(n).
// A non-null `gate` makes every kernel of the call return at once when *gate is zero (the same
// for the sort below).
size_t scan_scratch_bytes(int64_t n);
hipError_t launch_scan(const int32_t* in, int32_t* out, int64_t n, bool exclusive, void* scratch, hipStream_t stream,
                       const uint32_t* gate = nullptr);
// Stable LSD radix sort of n (key, value) pairs by key bits [0, bits), digits of at most 9 bits
// (as few passes as that allows), ping-pong
// between (keys, vals) and (keys_alt, vals_alt): *result_in_alt says which pair holds the sorted
// result (the other is overwritten).  scratch: radix_sort_scratch_bytes(n).  K: uint32_t or
// uint64_t.
size_t radix_sort_scratch_bytes(int64_t n);
template <typename K>
hipError_t launch_radix_sort_pairs(K* keys, int32_t* vals, K* keys_alt, int32_t* vals_alt, int64_t n, int bits,
                                   void* scratch, hipStream_t stream, bool* result_in_alt,
                                   const uint32_t* gate = nullptr);

// Row order of a sparse map (row_order.hip).  The block (order_block_bytes(n)) holds the gate
// (device flag: 1 when the order was built, 0 when the map is too dense for it to pay), the input
// row at each position, and the rulebook rows and masks in that order.
struct OrderView {
  uint32_t* gate;
  int32_t* rows;
  int32_t* nbr;
  uint32_t* masks;
};
OrderView order_view(void* block, int64_t n);
size_t order_block_bytes(int64_t n);
size_t order_scratch_bytes(int64_t n);
// Enqueues the gate, the sort and the permuted copy (reads d->nbr, d->masks, d->dev_banks).
hipError_t launch_row_order(const MapData* d, void* block, void* scratch, hipStream_t stream);
constexpr int64_t kOrderMinRows = 65536;  // smaller sets keep the input order

// Child map of a subdivide (structure.hip): nbr [8 np, 27] and masks [8 np] from the parent
// rulebook [np, 27].
hipError_t launch_child_map(const int32_t* parent_nbr, int64_t np, int32_t* nbr, uint32_t* masks,
                            hipStream_t stream);

// Per-offset convolution (conv_offsets.hip).  launch_pair_lists fills pair_out / pair_in of a
// map (sizes pairs - n) using pair_scratch_ints(n) int32 of scratch; launch_subm_conv_per_offset
// needs the pair lists, 16-bit storage, cin % 8 == 0, cout % 4 == 0 and acc = float32 [n, cout].
hipError_t launch_pair_lists(const MapData& m, int32_t* pair_out, int32_t* pair_in, int32_t* scratch,
                             hipStream_t stream);
size_t pair_scratch_ints(int64_t n);
hipError_t launch_subm_conv_per_offset(const MapData& m, int cin, int cout, int dtype, const void* feats,
                                       const void* weight, const void* bias, void* out, float* acc,
                                       hipStream_t stream);

// Convolution whose epilogue also stores group-norm partials per (row tile, group) (conv.hip):
// hipErrorNotSupported (nothing launched) when the shape does not take that path.
hipError_t launch_subm_conv_gn_partials(const MapData* map, int64_t n, int ksize, int cin, int cout, int dtype,
                                        const void* feats, const void* weight, const void* bias, void* out,
                                        float2* part, int cpg, int groups, int* tile_rows, hipStream_t stream);

// Convolution launcher (conv.hip).  Arguments already validated by the caller.  gate != null:
// flags [gate_n]; the launched kernels do nothing unless one of them is set (the fallback of a
// neighbour-pool launch whose plan may have overflowed; only the 16-bit k = 3 path above 64
// output channels takes it).
hipError_t launch_subm_conv(const MapData* map, int64_t n, int ksize, int cin, int cout, int dtype,
                            const void* feats, const void* weight, const void* bias, void* out,
                            hipStream_t stream, const uint32_t* gate = nullptr, int gate_n = 0);


// Neighbour-pool convolution (conv_pool.hip): k = 3, 16-bit storage, cout == 128, cin % 32 == 0.
// pool_tiling: false when n is too small (fewer than one full tile per compute unit) or the plan
// would exceed 31-bit offsets.  launch_pool_plan writes the plan of map rows nbr [n, 27] (plan:
// pool_plan_bytes(t)): the tile records and the overflow flags of every (tile, dz)
// (pool_tile_flags, pool_flag_count(t) of them), and stores 1 into *host_flag (pinned, zeroed by
// the caller) when a sub-pool does not fit; `done` records its completion.  launch_pool_conv
// packs the weights into wpk (pool_weight_bytes(cin)) and runs the convolution; gate != null:
// the flags, the kernel does nothing if one is set.
bool pool_tiling(int64_t n, PoolTiling* t);
int pool_flag_count(const PoolTiling& t);
size_t pool_plan_bytes(const PoolTiling& t);
uint32_t* pool_tile_flags(const PoolTiling& t, void* plan);
size_t pool_weight_bytes(int cin);
hipError_t launch_pool_plan(const int32_t* nbr, int64_t n, const PoolTiling& t, void* plan, uint32_t* host_flag,
                            hipEvent_t done, hipStream_t stream);
hipError_t launch_pool_conv(const PoolTiling& t, const void* plan, const uint32_t* gate, int64_t n, int cin, int dtype,
                            const void* feats, const void* weight, const void* bias, void* out, void* wpk,
                            hipStream_t stream);

// Per-(device, stream) scratch of at least `bytes`, reused by every call on that stream (work on
// one stream is ordered, so a later call cannot overwrite it while an earlier one still reads
// it); grows by a stream-ordered free and allocation (submconv_api.hip).
Status stream_scratch(int dev, hipStream_t stream, size_t bytes, void** ptr);

}  // namespace submconv

namespace submconv {
// Subdivision handle contents (structure.hip): one coarse / fine relation, all arrays in one
// device allocation owned by the handle.
struct SubdivData {
  int device = 0;
  int kind = 0;                  // subm_subdivision_kind_t
  int64_t n_coarse = 0;
  int64_t n_fine = 0;
  void* block = nullptr;         // the allocation holding the arrays below
  int32_t* coarse = nullptr;     // [n_coarse, 4]
  int32_t* fine = nullptr;       // [n_fine, 4]
  int32_t* parent = nullptr;     // [n_fine]
  int32_t* seg_off = nullptr;    // [n_coarse + 1]: members of coarse row m are positions seg_off[m] ..
  int32_t* seg_rows = nullptr;   // ... seg_off[m+1] - 1 of seg_rows [n_fine] (null: position = fine row)
};
}  // namespace submconv

// The opaque handle types of the C ABI.
struct submconv_map {
  submconv::MapData d;
  std::mutex mu;  // guards the lazy reads of the counts and the lazy build of the pair lists
  std::atomic<bool> other_streams{false};  // work reading the map was enqueued off d.home
};

namespace submconv {
// Waits for an asynchronous build's insert kernel on first use and returns the build's coordinate
// status (SUBM_OK at once for a checked map).
Status map_check(submconv_map* map);
// Makes map->d.pairs / per_tap valid (waits for the build's last kernel on first use); fails with
// the build's coordinate status.
Status map_counts(submconv_map* map);
// Records that work reading the map's memory is enqueued on `stream` (every entry point that
// reads a map calls it before enqueuing); a map used only on the stream of its build gives its
// memory back to the per-device block cache when freed (map_memory_give).
// Work enqueued on another stream than the build's is also ordered after the build: the stream
// waits for the build's last kernel unless it has already completed.
inline void map_note_use(submconv_map* map, hipStream_t stream) {
  if (map != nullptr && stream != map->d.home) {
    map->other_streams.store(true, std::memory_order_relaxed);
    if (map->d.ready != nullptr && hipEventQuery(map->d.ready) != hipSuccess)
      (void)hipStreamWaitEvent(stream, map->d.ready, 0);
  }
}
// Memory for a map's rulebook on device `dev`: a cached block of a freed map that was built and
// used only on `stream` when one fits (no allocator call, so nothing is enqueued), else a new
// stream-ordered allocation.  *got receives the block's size.
Status map_memory_take(int dev, size_t bytes, hipStream_t stream, void** ptr, size_t* got);
// Gives a map's rulebook memory back: into the device's cache, tagged with `stream`, when
// `reusable` (all work on it was on that stream) and the cache has room, else back to the pool in
// order after the work on `stream`.
void map_memory_give(int dev, void* ptr, size_t bytes, hipStream_t stream, bool reusable);
// Host-side checks of a convolution call (subm_conv3d_forward's rules).
Status check_conv(submconv_map_t map, int64_t n, int ksize, int cin, int cout, int dtype, const void* feats,
                  const void* weight, const void* bias, const void* out);
}  // namespace submconv
struct sparse_subdivision {
  submconv::SubdivData d;
};

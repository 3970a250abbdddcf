// Host side of libmk: the C ABI declared in include/mk.h.
//
// A handle owns a control block (tickets, counters, error record), per-chunk
// ready flags with self-resetting arrival counters, and an on-demand
// workspace.  Each operation validates its arguments, classifies every peer
// pointer (device memory or pinned host memory read/written over PCIe),
// chooses the tile shape and role counts, advances the handle's epoch and
// makes exactly one persistent kernel launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "mk_params.h"

namespace mk {
hipError_t launch_ag(const AgParams &p, int bm, int bn, int grid, hipStream_t s);
hipError_t launch_rs(const RsParams &p, int bm, int grid, hipStream_t s);
hipError_t launch_ar(const ArParams &p, int bm, int grid, hipStream_t s);
hipError_t launch_moe(const MoeParams &p, int bm, int grid, hipStream_t s);
hipError_t occupancy(int op, int bm, int bn, int *blocks_per_cu);
hipError_t occupancy_moe(int bm, int *blocks_per_cu);
hipError_t launch_attn(const AttnParams &p, int grid, hipStream_t s);
hipError_t occupancy_attn(int *blocks_per_cu);
hipError_t launch_mfma_loop(int grid, int iters, float *sink, hipStream_t s);
}  // namespace mk

struct mk_ctx {
  int device = 0;
  int cu_count = 0;
  int timeout_ms = 2000;
  uint64_t timeout_ticks = 0;
  int force_tile = 0;  // MK_TILE env: 128 or 256 forces the tile edge
  bool no_slabs = true;   // MK_NO_SLABS=0 env: cut AllGather land blocks into K-slabs
  int ring_splits = 0;  // MK_RING_SPLITS=1: one task per (head, query tile) (0: library choice)
  int tile_map = -1;  // MK_TILE_MAP env: 0 global m-major order, 1 XCD blocks, 2 XCD strided, 3 XCD rounds (-1: per op)
  int item_kib = 512;  // MK_ITEM_KIB env: target size of one AllGather land item
  int item_kib_first = 512;  // MK_ITEM_KIB_FIRST env: the same for the shards landed at the start
  int help_every = 0;  // MK_HELP_EVERY env: 1 in this many compute workgroups helps land (0: automatic)
  int help_eager = -1;  // MK_HELP_EAGER env: helpers land until the queue is empty (-1: automatic)
  int land_split = 1;  // MK_LAND_SPLIT env: land first-round chunks at the start, the rest between tiles
  int moe_withhold = -1;  // MK_TEST_MOE_WITHHOLD env (failure tests only): the MoE land queue skips this unit
  mk::Ctrl *ctrl = nullptr;
  uint32_t *flags = nullptr;
  uint32_t *cnt = nullptr;
  uint32_t epoch = 0;
  int max_flags = mk::kMaxFlags;  // flags (and arrival counters) the control memory holds
  bool scratch = false;           // control memory is the library's per-device array (no handle)
  mk_roles roles[MK_OP_COUNT];
  mk_roles last[MK_OP_COUNT];
  int last_grid[MK_OP_COUNT] = {0, 0, 0, 0};
  bool launched[MK_OP_COUNT] = {false, false, false, false};
  int occ[MK_OP_COUNT][3] = {};  // blocks per CU: [256x256, 128x128, 256x224]
  void *ws = nullptr;
  size_t ws_bytes = 0;
  std::string err;
};

namespace {

struct DeviceGuard {
  int old = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&old) != hipSuccess) old = -1;
    if (old != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (old >= 0) (void)hipSetDevice(old);
  }
};

mk_status fail(mk_ctx *h, mk_status st, const std::string &msg) {
  if (h) h->err = msg;
  return st;
}

mk_status hip_fail(mk_ctx *h, hipError_t e, const char *what) {
  std::string m = std::string(what) + ": " + hipGetErrorString(e);
  (void)hipGetLastError();
  return fail(h, MK_ERR_HIP, m);
}

inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Workspace of a handle when mk_config.workspace_bytes is 0: enough for every
// operation at the library's reference workloads (the largest user is the
// GEMM+AllReduce reduce role, [2048, 8192] fp32 = 64 MiB).
constexpr size_t kDefaultWorkspace = (size_t)128 << 20;

// A buffer of `bytes` bytes at p must end inside the allocation that holds p.
// The runtime knows the extent of device and pinned host allocations; where
// it reports none, nothing is checked.  A caching allocator's blocks sit
// inside larger runtime allocations, so this catches a short buffer only
// near the end of such an allocation.
mk_status check_extent(mk_ctx *h, const void *p, size_t bytes, const char *what) {
  void *base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void *>(p)) != hipSuccess || !base || !size) {
    (void)hipGetLastError();
    return MK_OK;
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
  if (q < b || q - b >= size) return MK_OK;  // not the allocation p lies in
  const size_t left = size - (q - b);
  if (bytes > left)
    return fail(h, MK_ERR_INVALID, std::string(what) + " is smaller than its shape: " + std::to_string(bytes) +
                                       " bytes needed, " + std::to_string(left) + " left in its allocation");
  return MK_OK;
}

// Resolve a pointer the kernel will dereference, for a buffer of `bytes`
// bytes.  Device memory must belong to the handle's device; pinned host
// memory is accepted when allow_host and replaced by its device-side address.
mk_status resolve(mk_ctx *h, const void *p, size_t bytes, bool allow_host, const void **out, const char *what) {
  if (p == nullptr) return fail(h, MK_ERR_INVALID, std::string(what) + " is NULL");
  if (reinterpret_cast<uintptr_t>(p) & 15u)
    return fail(h, MK_ERR_INVALID, std::string(what) + " is not 16-byte aligned");
  hipPointerAttribute_t a;
  std::memset(&a, 0, sizeof(a));
  hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(h, MK_ERR_INVALID, std::string(what) + " is not HIP-allocated memory (pageable host memory?)");
  }
  if (mk_status st = check_extent(h, p, bytes, what)) return st;
  switch (a.type) {
    case hipMemoryTypeDevice:
      if (a.device != h->device)
        return fail(h, MK_ERR_INVALID, std::string(what) + " lives on another device");
      *out = p;
      return MK_OK;
    case hipMemoryTypeHost:
      if (!allow_host) return fail(h, MK_ERR_INVALID, std::string(what) + " must be device memory");
      *out = a.devicePointer ? a.devicePointer : p;
      return MK_OK;
    case hipMemoryTypeManaged:
    case hipMemoryTypeUnified:
      *out = p;
      return MK_OK;
    default:
      return fail(h, MK_ERR_INVALID, std::string(what) + " is not device or pinned host memory");
  }
}

mk::Sync make_sync(mk_ctx *h, uint32_t n_flags) {
  // the per-device array is cleared before every launch (which a captured
  // graph replays too), so its launches all use epoch 1
  if (h->scratch) h->epoch = 1;
  else if (++h->epoch == 0) h->epoch = 1;
  mk::Sync s;
  s.ctrl = h->ctrl;
  s.flags = h->flags;
  s.cnt = h->cnt;
  s.epoch = h->epoch;
  s.n_flags = n_flags;
  s.timeout_ticks = h->timeout_ticks;
  return s;
}

// Workgroups resident at once for a kernel instantiation.
int max_grid(mk_ctx *h, int op, int bm, int bn = 0) {
  if (bn == 0) bn = bm;
  int &o = h->occ[op][bm != 256 ? 1 : bn == 224 ? 2 : 0];
  if (o == 0) {
    int b = 0;
    hipError_t e = op == MK_OP_MOE ? mk::occupancy_moe(bm, &b)
                   : op == MK_OP_RING_ATTN ? mk::occupancy_attn(&b)
                                           : mk::occupancy(op, bm, bn, &b);
    if (e != hipSuccess || b < 1) {
      (void)hipGetLastError();
      b = 1;
    }
    o = b;
  }
  return std::max(1, o * h->cu_count);
}

int pick_tile(mk_ctx *h, long tiles256) {
  if (h->force_tile == 128 || h->force_tile == 256 || h->force_tile == 224)
    return h->force_tile == 224 ? 256 : h->force_tile;
  return tiles256 * 2 >= h->cu_count ? 256 : 128;
}

// Column edge of the 256-row AllGather tiles: 224 when its rounds of
// resident tiles cost less (an N of 7 x 512 = 3584 gives 512 tiles of
// 256x224 = two full rounds on 256 CUs instead of 448 of 256x256 = 1.75).
int pick_tile_n(mk_ctx *h, int tiles_m, int n, int gmax) {
  if (h->force_tile == 224) return 224;
  if (h->force_tile != 0) return 256;
  auto cost = [&](int bn) {
    const long tiles = (long)tiles_m * ((n + bn - 1) / bn);
    return ((tiles + gmax - 1) / gmax) * bn;
  };
  return cost(224) < cost(256) ? 224 : 256;
}

// Group and sub-block shape of the kMapRounds order: a group is the m-blocks
// one round of `grid` workgroups covers; the 8 XCDs split it into
// split_m x (8 / split_m) sub-blocks, picked to minimise the A + B rows that
// one XCD's tiles of a round read per K step.
void rounds_order(int tiles_m, int tiles_n, int grid, int bm, int bn, int *group_m, int *split_m) {
  const int G = std::max(1, std::min(tiles_m, grid / std::max(1, tiles_n)));
  int best = 1;
  long best_cost = -1;
  for (int am = 1; am <= 8; am *= 2) {
    const int bx = 8 / am;
    const long cost = (long)cdiv(G, am) * bm + (long)cdiv(tiles_n, bx) * bn +
                      (am > G || bx > tiles_n ? 1L << 40 : 0);  // an XCD with no tiles
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = am;
    }
  }
  *group_m = G;
  *split_m = best;
}

// Apply the user's role settings to the defaults.  `want_land` / `want_reduce`
// are the defaults; compute fills the rest of the resident grid (capped by
// the tile count).  Grid = the sum; at least one workgroup.
void choose_roles(mk_ctx *h, mk_op op, int gmax, int want_land, int n_tiles, int *land, int *compute) {
  const mk_roles &r = h->roles[op];
  int l = r.n_land >= 0 ? r.n_land : want_land;
  l = std::max(0, std::min(l, 4 * gmax));
  int c;
  if (r.n_compute >= 0) c = std::min(r.n_compute, 4 * gmax);
  else c = std::max(1, std::min(n_tiles, gmax - l));
  *land = l;
  *compute = std::max(0, c);
}

void record(mk_ctx *h, mk_op op, int land, int compute, int reduce, int grid) {
  h->last[op].n_land = land;
  h->last[op].n_compute = compute;
  h->last[op].n_reduce = reduce;
  h->last_grid[op] = grid;
  h->launched[op] = true;
}

// Roles of a GEMM+ReduceScatter / GEMM+AllReduce launch.
//   compute  workgroups that run tiles (0: transfer alone)
//   reduce   workgroups that take reduce items first (they take the first
//            tickets); by default none: the tile epilogues read the peers'
//            partials themselves
//   items    the fused launch has reduce items (reduce > 0 and something to
//            reduce)
//   xfer     transfer alone: reduce workgroups move the operation's
//            reduce and scatter bytes, nothing is computed
//   joins    reduce workgroups run tiles once every item is claimed
struct Roles {
  int compute = 0, reduce = 0;
  bool items = false, xfer = false;
  int joins = 0;
};

mk_status choose_reduce_roles(mk_ctx *h, mk_op op, int gmax, int n_tiles, bool has_peers, unsigned flags,
                              Roles *out) {
  const mk_roles &r = h->roles[op];
  if (r.n_land > 0) return fail(h, MK_ERR_INVALID, "this operation has no land role");
  Roles ro;
  if (r.n_compute == 0) {  // transfer alone
    if (flags & MK_F_NO_PEERS)
      return fail(h, MK_ERR_INVALID, "transfer alone (n_compute = 0) with MK_F_NO_PEERS moves nothing");
    ro.xfer = true;
    ro.reduce = std::max(1, std::min(r.n_reduce > 0 ? r.n_reduce : gmax, 4 * gmax));
    *out = ro;
    return MK_OK;
  }
  ro.reduce = r.n_reduce > 0 ? std::min(r.n_reduce, 4 * gmax) : 0;
  if (r.n_compute > 0) ro.compute = std::min(r.n_compute, 4 * gmax);
  else ro.compute = std::max(1, std::min(n_tiles, gmax - ro.reduce));
  ro.items = ro.reduce > 0 && has_peers;
  ro.joins = (flags & MK_F_STATIC_ROLES) ? 0 : 1;
  *out = ro;
  return MK_OK;
}

mk_status check_common(mk_ctx *h, int world, int rank) {
  if (!h) return MK_ERR_INVALID;
  h->err.clear();
  if (world < 1 || world > MK_MAX_WORLD) return fail(h, MK_ERR_INVALID, "world out of range");
  if (rank < 0 || rank >= world) return fail(h, MK_ERR_INVALID, "rank out of range");
  return MK_OK;
}

mk_status check_gemm_shape(mk_ctx *h, long m, long n, long k) {
  if (m < 1 || n < 8 || k < 8) return fail(h, MK_ERR_INVALID, "GEMM dimensions too small");
  if (n % 8 || k % 8) return fail(h, MK_ERR_INVALID, "n and k must be multiples of 8");
  if (k > (1 << 20) || n > (1 << 22) || m > (1L << 28))
    return fail(h, MK_ERR_UNSUPPORTED, "GEMM dimensions beyond the supported range");
  if ((long)256 * k * 2 >= 0x80000000L) return fail(h, MK_ERR_UNSUPPORTED, "k too large");
  return MK_OK;
}

// The workspace is allocated by mk_create (mk_config.workspace_bytes) and
// never grown by a call: an operation that needs more refuses before
// launching, so no call allocates, frees or synchronises.
mk_status need_ws(mk_ctx *h, size_t bytes, const char *what) {
  if (bytes <= h->ws_bytes) return MK_OK;
  return fail(h, MK_ERR_INVALID, std::string(what) + " needs a workspace of " + std::to_string(bytes) +
                                     " bytes; the handle has " + std::to_string(h->ws_bytes) +
                                     " (mk_config.workspace_bytes)");
}

// ---------------------------------------------------------------- per-device control memory
//
// mk_ag_gemm_noalloc runs without a handle: its control block, ready flags
// and arrival counters live in `scratch`, a fixed array that each GPU the
// library runs on holds until the process ends.  In host code `scratch` is
// a host-side stand-in; the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// ever passed to a kernel.  Every call clears the control block and its
// flags first (with a kernel, so a captured graph replays the clear too) and
// uses epoch 1; calls that overlap on one GPU share the array and race.

constexpr int kScratchFlags = 2048;
constexpr size_t kScratchCtrlBytes = (sizeof(mk::Ctrl) + 255) & ~(size_t)255;
constexpr size_t kScratchFlagBytes = (size_t)kScratchFlags * mk::kFlagStride * sizeof(uint32_t);
constexpr size_t kScratchBytes = kScratchCtrlBytes + 2 * kScratchFlagBytes;  // 260 KiB
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Zero the control block and the first n_flags flags and arrival counters.
__global__ void scratch_clear_kernel(uint32_t *ctrl_words, uint32_t n_ctrl_words, uint32_t *flags,
                                     uint32_t *cnt, uint32_t n_flags) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_ctrl_words) ctrl_words[i] = 0u;
  if (i < n_flags) {
    flags[(size_t)i * mk::kFlagStride] = 0u;
    cnt[(size_t)i * mk::kFlagStride] = 0u;
  }
}

// status[0] = the launch's error code (0 = MK_OK), status[1] = its detail.
__global__ void scratch_report_kernel(const mk::Ctrl *ctrl, int32_t *status) {
  if (threadIdx.x == 0) {
    status[0] = (int32_t)(ctrl->err_code == mk::kErrInternal ? (uint32_t)MK_ERR_HIP : ctrl->err_code);
    status[1] = (int32_t)ctrl->err_info;
  }
}

hipError_t scratch_clear(mk_ctx *h, uint32_t n_flags, hipStream_t s) {
  const uint32_t words = (uint32_t)(sizeof(mk::Ctrl) / sizeof(uint32_t));
  const uint32_t n = std::max(words, n_flags);
  hipLaunchKernelGGL(scratch_clear_kernel, dim3((n + 255) / 256), dim3(256), 0, s,
                     reinterpret_cast<uint32_t *>(h->ctrl), words, h->flags, h->cnt, n_flags);
  return hipGetLastError();
}

hipError_t scratch_report(mk_ctx *h, int32_t *status, hipStream_t s) {
  hipLaunchKernelGGL(scratch_report_kernel, dim3(1), dim3(64), 0, s, h->ctrl, status);
  return hipGetLastError();
}

struct ScratchDevice {
  std::once_flag once;
  mk_ctx *ctx = nullptr;
  mk_status st = MK_OK;
};
ScratchDevice g_scratch[kMaxDevices];

// The per-device context of mk_ag_gemm_noalloc for the current device, set
// up on the device's first call: gfx950 check, the array's device address,
// the library's default schedule (no environment knobs).  Nothing is
// allocated on the device.
mk_status scratch_ctx(mk_ctx **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return MK_ERR_INVALID;
  }
  ScratchDevice &sd = g_scratch[dev];
  std::call_once(sd.once, [&] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      sd.st = MK_ERR_HIP;
      return;
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      sd.st = MK_ERR_UNSUPPORTED;
      return;
    }
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      sd.st = MK_ERR_HIP;
      return;
    }
    mk_ctx *h = new mk_ctx();
    h->device = dev;
    h->cu_count = prop.multiProcessorCount;
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) khz = 100000;
    h->timeout_ticks = (uint64_t)khz * (uint64_t)h->timeout_ms;
    for (int i = 0; i < MK_OP_COUNT; ++i) h->roles[i] = mk_roles{-1, -1, -1};
    char *base = static_cast<char *>(ptr);
    h->ctrl = reinterpret_cast<mk::Ctrl *>(base);
    h->flags = reinterpret_cast<uint32_t *>(base + kScratchCtrlBytes);
    h->cnt = reinterpret_cast<uint32_t *>(base + kScratchCtrlBytes + kScratchFlagBytes);
    h->max_flags = kScratchFlags;
    h->scratch = true;
    sd.ctx = h;
  });
  if (sd.st != MK_OK) return sd.st;
  *out = sd.ctx;
  return MK_OK;
}

}  // namespace

extern "C" {

const char *mk_status_string(mk_status s) {
  switch (s) {
    case MK_OK: return "MK_OK";
    case MK_ERR_INVALID: return "MK_ERR_INVALID: invalid argument";
    case MK_ERR_UNSUPPORTED: return "MK_ERR_UNSUPPORTED: unsupported device or shape";
    case MK_ERR_OOM: return "MK_ERR_OOM: device allocation failed";
    case MK_ERR_HIP: return "MK_ERR_HIP: HIP runtime error";
    case MK_ERR_TIMEOUT: return "MK_ERR_TIMEOUT: an in-kernel wait expired";
  }
  return "unknown mk_status";
}

const char *mk_last_error(mk_handle h) { return h ? h->err.c_str() : ""; }

mk_status mk_create(mk_handle *out, const mk_config *cfg) {
  if (!out || !cfg) return MK_ERR_INVALID;
  if (cfg->flags != 0) return MK_ERR_INVALID;
  if (cfg->workspace_bytes > ((size_t)1 << 40)) return MK_ERR_INVALID;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device < 0 || cfg->device >= ndev) {
    (void)hipGetLastError();
    return MK_ERR_INVALID;
  }
  DeviceGuard g(cfg->device);
  if (!g.ok) return MK_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, cfg->device) != hipSuccess) return MK_ERR_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MK_ERR_UNSUPPORTED;
  mk_ctx *h = new mk_ctx();
  h->device = cfg->device;
  h->cu_count = prop.multiProcessorCount;
  h->timeout_ms = cfg->spin_timeout_ms > 0 ? cfg->spin_timeout_ms : 2000;
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, cfg->device) != hipSuccess || khz <= 0)
    khz = 100000;
  h->timeout_ticks = (uint64_t)khz * (uint64_t)h->timeout_ms;
  if (const char *t = std::getenv("MK_TILE")) h->force_tile = std::atoi(t);
  if (const char *t = std::getenv("MK_NO_SLABS")) h->no_slabs = std::atoi(t) != 0;
  if (const char *t = std::getenv("MK_RING_SPLITS")) h->ring_splits = std::atoi(t) == 1 ? 1 : 0;
  if (const char *t = std::getenv("MK_TILE_MAP")) h->tile_map = std::min(3, std::max(0, std::atoi(t)));
  if (const char *t = std::getenv("MK_ITEM_KIB")) h->item_kib = std::min(4096, std::max(4, std::atoi(t)));
  if (const char *t = std::getenv("MK_ITEM_KIB_FIRST")) h->item_kib_first = std::min(4096, std::max(4, std::atoi(t)));
  if (const char *t = std::getenv("MK_HELP_EVERY")) h->help_every = std::max(1, std::atoi(t));
  if (const char *t = std::getenv("MK_HELP_EAGER")) h->help_eager = std::atoi(t) != 0 ? 1 : 0;
  if (const char *t = std::getenv("MK_LAND_SPLIT")) h->land_split = std::atoi(t) != 0 ? 1 : 0;
  if (const char *t = std::getenv("MK_TEST_MOE_WITHHOLD")) h->moe_withhold = std::atoi(t);
  for (int i = 0; i < MK_OP_COUNT; ++i) h->roles[i] = mk_roles{-1, -1, -1};
  if (const char *r = std::getenv("MK_ROLES")) {
    int l = -1, c = -1, d = -1;
    if (std::sscanf(r, "%d,%d,%d", &l, &c, &d) >= 1)
      for (int i = 0; i < MK_OP_COUNT; ++i) {
        const bool red = i == MK_OP_GEMM_RS || i == MK_OP_GEMM_AR;  // a reduce role, no land role
        h->roles[i] = mk_roles{red ? -1 : l, c, red ? d : -1};
      }
  }
  const size_t flag_bytes = (size_t)mk::kMaxFlags * mk::kFlagStride * sizeof(uint32_t);
  hipError_t e = hipMalloc(reinterpret_cast<void **>(&h->ctrl), sizeof(mk::Ctrl));
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&h->flags), flag_bytes);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&h->cnt), flag_bytes);
  h->ws_bytes = cfg->workspace_bytes ? cfg->workspace_bytes : kDefaultWorkspace;
  if (e == hipSuccess) e = hipMalloc(&h->ws, h->ws_bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    mk_destroy(h);
    return MK_ERR_OOM;
  }
  e = hipMemset(h->ctrl, 0, sizeof(mk::Ctrl));
  if (e == hipSuccess) e = hipMemset(h->flags, 0, flag_bytes);
  if (e == hipSuccess) e = hipMemset(h->cnt, 0, flag_bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipGetLastError();
    mk_destroy(h);
    return MK_ERR_HIP;
  }
  *out = h;
  return MK_OK;
}

mk_status mk_destroy(mk_handle h) {
  if (!h) return MK_ERR_INVALID;
  DeviceGuard g(h->device);
  if (h->ctrl) (void)hipFree(h->ctrl);
  if (h->flags) (void)hipFree(h->flags);
  if (h->cnt) (void)hipFree(h->cnt);
  if (h->ws) (void)hipFree(h->ws);
  delete h;
  return MK_OK;
}

mk_status mk_set_roles(mk_handle h, mk_op op, const mk_roles *roles) {
  if (!h || !roles || op < 0 || op >= MK_OP_COUNT) return MK_ERR_INVALID;
  h->err.clear();
  if (roles->n_reduce > 0 && op != MK_OP_GEMM_RS && op != MK_OP_GEMM_AR)
    return fail(h, MK_ERR_INVALID, "only GEMM+ReduceScatter and GEMM+AllReduce have a reduce role");
  h->roles[op] = *roles;
  return MK_OK;
}

mk_status mk_get_roles(mk_handle h, mk_op op, mk_roles *roles) {
  if (!h || !roles || op < 0 || op >= MK_OP_COUNT) return MK_ERR_INVALID;
  *roles = h->roles[op];
  return MK_OK;
}

mk_status mk_last_launch(mk_handle h, mk_op op, mk_roles *roles, int *grid) {
  if (!h || op < 0 || op >= MK_OP_COUNT || !h->launched[op]) return MK_ERR_INVALID;
  if (roles) *roles = h->last[op];
  if (grid) *grid = h->last_grid[op];
  return MK_OK;
}

mk_status mk_sync(mk_handle h, mk_stream stream) {
  if (!h) return MK_ERR_INVALID;
  DeviceGuard g(h->device);
  hipError_t e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(h, e, "hipStreamSynchronize");
  uint32_t rec[3] = {0, 0, 0};
  e = hipMemcpy(rec, &h->ctrl->err_code, sizeof(rec), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(h, e, "reading the error record");
  if (rec[0] != 0) {
    const uint32_t zero = 0;
    e = hipMemcpy(&h->ctrl->err_code, &zero, sizeof(zero), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(h, e, "clearing the error record");
    char buf[160];
    if (rec[0] == MK_ERR_TIMEOUT)
      std::snprintf(buf, sizeof(buf), "in-kernel wait timed out (wait id 0x%08x, epoch %u)",
                    rec[1], rec[2]);
    else
      std::snprintf(buf, sizeof(buf), "in-kernel index check failed (code %u, info 0x%08x, epoch %u)",
                    rec[0], rec[1], rec[2]);
    h->err = buf;
    return rec[0] == MK_ERR_TIMEOUT ? MK_ERR_TIMEOUT : MK_ERR_HIP;
  }
  return MK_OK;
}

// ---------------------------------------------------------------- AllGather + GEMM

// mk_ag_gemm on a handle, or (h->scratch) on the per-device array of
// mk_ag_gemm_noalloc, whose launch is bracketed by a clear of the array and
// an optional status report.
static mk_status ag_gemm_impl(mk_handle h, mk_stream stream, int world, int rank,
                              const mk_bf16 *const *a_shards, const mk_bf16 *bt, mk_bf16 *c,
                              mk_bf16 *a_gathered, int m_s, int n, int k, unsigned flags,
                              int32_t *status) {
  mk_status st = check_common(h, world, rank);
  if (st != MK_OK) return st;
  if (flags & ~(MK_F_PRELANDED | MK_F_STATIC_ROLES)) return fail(h, MK_ERR_INVALID, "unknown flag bits");
  if (!a_shards) return fail(h, MK_ERR_INVALID, "a_shards is NULL");
  if (m_s < 1) return fail(h, MK_ERR_INVALID, "m_s < 1");
  st = check_gemm_shape(h, (long)world * m_s, n, k);
  if (st != MK_OK) return st;
  DeviceGuard g(h->device);
  const bool pre = (flags & MK_F_PRELANDED) != 0;
  mk::AgParams p;
  std::memset(&p, 0, sizeof(p));
  const void *dp;
  for (int q = 0; q < world; ++q) {
    if (pre && q != rank) continue;  // peers are not read when pre-landed
    char what[32];
    std::snprintf(what, sizeof(what), "a_shards[%d]", q);
    if ((st = resolve(h, a_shards[q], (size_t)m_s * k * 2, q != rank, &dp, what)) != MK_OK) return st;
    p.shard[q] = static_cast<const uint16_t *>(dp);
  }
  if ((st = resolve(h, bt, (size_t)n * k * 2, false, &dp, "bt")) != MK_OK) return st;
  p.bt = static_cast<const uint16_t *>(dp);
  if ((st = resolve(h, c, (size_t)world * m_s * n * 2, true, &dp, "c")) != MK_OK) return st;
  p.c = static_cast<uint16_t *>(const_cast<void *>(dp));
  if ((st = resolve(h, a_gathered, (size_t)world * m_s * k * 2, false, &dp, "a_gathered")) != MK_OK) return st;
  p.ag = static_cast<uint16_t *>(const_cast<void *>(dp));

  const int M = world * m_s;
  const int bm = pick_tile(h, (long)cdiv(M, 256) * cdiv(n, 256));
  const int bn = bm == 256 ? pick_tile_n(h, cdiv(M, 256), n, max_grid(h, MK_OP_AG_GEMM, 256, 256)) : bm;
  p.world = world;
  p.rank = rank;
  p.m_s = m_s;
  p.n = n;
  p.k = k;
  p.tiles_m = cdiv(M, bm);
  p.tiles_n = cdiv(n, bn);
  p.n_tiles = p.tiles_m * p.tiles_n;
  p.mb0 = (rank * m_s) / bm;
  // AllGather tiles share A and B slabs best per XCD; the reduce epilogues
  // balance better in the global order (own slice first)
  p.tile_map = h->tile_map >= 0 ? h->tile_map : mk::kMapStrided;
  // landing geometry: one flag per lb_rows rows of a shard and K-slab,
  // items of about item_kib KiB (512 by default).  Shards are cut into K-slabs (about 8, of at least
  // 256 columns) when every slab of every row starts on a 128-byte line, so
  // that tiles can start once their first slab has landed; otherwise one
  // slab spans K.
  const bool base_aligned = reinterpret_cast<uintptr_t>(p.ag) % 128 == 0;
  p.n_slabs = 1;
  p.slab_k = k;
  if (!pre && base_aligned && k % 64 == 0 && k >= 2048 && !h->no_slabs) {
    p.slab_k = std::max(256, (int)((cdiv(k, 8) + 63) / 64 * 64));
    p.n_slabs = cdiv(k, p.slab_k);
  }
  p.slab_stages = p.n_slabs > 1 ? p.slab_k / 64 : 0;
  p.lb_rows = bm;
  while ((long)world * cdiv(m_s, p.lb_rows) * p.n_slabs > h->max_flags) p.lb_rows *= 2;
  if ((long)world * cdiv(m_s, p.lb_rows) * p.n_slabs > h->max_flags)
    return fail(h, MK_ERR_UNSUPPORTED, "more landing flags than the control memory holds");
  p.blocks_per_chunk = cdiv(m_s, p.lb_rows);
  p.item_rows = std::max(1, std::min(p.lb_rows, (h->item_kib * 1024) / (p.slab_k * 2)));
  p.items_per_block = cdiv(p.lb_rows, p.item_rows);
  const int items_per_chunk = p.blocks_per_chunk * p.n_slabs * p.items_per_block;
  p.n_items = world * items_per_chunk;
  p.n_peer_items = (world - 1) * items_per_chunk;
  p.prelanded = pre ? 1 : 0;

  const int gmax = max_grid(h, MK_OP_AG_GEMM, bm, bn);
  const bool dynamic = (flags & MK_F_STATIC_ROLES) == 0;
  // Landing costs workgroup time.  When the tiles leave part of the last
  // round of resident workgroups idle, land workgroups fit there (they run
  // one tile fewer) and every second waiting workgroup helps with the first
  // chunks.  When the tiles fill whole rounds, either every waiting
  // workgroup lands until the queue is empty (all landing at the start), or
  // (split) the chunks of first-round tiles land at the start and every
  // workgroup lands its share of the rest after each tile, just before the
  // tiles that need it; the split needs the global tile order, whose first
  // round covers the fewest chunks.
  const int want_land0 = pre ? 0 : std::max(1, std::min(std::min(p.n_items, gmax / 8), 32));
  const bool fills = p.n_tiles % gmax == 0 || gmax - p.n_tiles % gmax < want_land0;
  const bool split = !pre && dynamic && fills && h->land_split > 0 && h->roles[MK_OP_AG_GEMM].n_land < 0;
  if (split && h->tile_map < 0) p.tile_map = mk::kMapRounds;
  int land = 0, compute = 0;
  choose_roles(h, MK_OP_AG_GEMM, gmax, split ? 0 : want_land0, p.n_tiles, &land, &compute);
  if (pre) land = 0;
  p.n_land = land;
  p.n_compute = compute;
  p.land_joins_compute = (dynamic && compute > 0) ? 1 : 0;
  p.help_land = (dynamic && !pre) ? 1 : 0;
  // land blocks on 128-byte boundaries of a_gathered allow the light acquire
  const bool aligned = base_aligned && ((size_t)p.lb_rows * k * 2) % 128 == 0 &&
                       ((size_t)m_s * k * 2) % 128 == 0;
  p.light_acquire = aligned ? 1 : 0;
  // in-loop slab checks rely on the light acquire, and on land workgroups
  // that finish the queue without ever waiting on a tile (a tile inside its
  // K loop cannot help land)
  if (!aligned || land == 0) p.slab_stages = 0;
  // peers whose chunk has tiles in the first round of tiles (in the global
  // order the local chunk's tiles run first; every workgroup ends up
  // running tiles)
  const int grid_all = std::max(1, land + compute);
  {
    const long tiles_per_chunk = (long)cdiv(m_s, bm) * p.tiles_n;
    const long room = (long)grid_all - tiles_per_chunk;
    const long first = room <= 0 ? 1 : (room + tiles_per_chunk - 1) / tiles_per_chunk;
    p.first_peers = (int)std::max(0L, std::min((long)(world - 1), first));
    // the other XCD maps start tiles of every chunk at once; the rounds map
    // keeps the global order's rounds
    if (p.tile_map != mk::kMapGlobal && p.tile_map != mk::kMapRounds) p.first_peers = world - 1;
  }
  // the first group's items: under the split schedule every workgroup lands
  // them at once at the start, so they are cut small enough (item_kib_first)
  // for all workgroups to take part; the later ones stay large
  {
    const int kib_first = split ? h->item_kib_first : h->item_kib;
    p.item_rows_first = std::max(1, std::min(p.lb_rows, (kib_first * 1024) / (p.slab_k * 2)));
    p.items_per_block_first = cdiv(p.lb_rows, p.item_rows_first);
    const int items_per_chunk_first = p.blocks_per_chunk * p.n_slabs * p.items_per_block_first;
    p.n_first_items = p.first_peers * items_per_chunk_first;
    p.n_peer_items = p.n_first_items + (world - 1 - p.first_peers) * items_per_chunk;
    p.n_items = p.n_peer_items + items_per_chunk;
  }
  rounds_order(p.tiles_m, p.tiles_n, grid_all, bm, bn, &p.tile_group_m, &p.tile_split_m);
  if (split) {
    p.help_eager = 1;
    p.eager_items = p.n_first_items;
    p.land_between = (p.n_peer_items - p.eager_items + grid_all - 1) / grid_all;
    p.help_every = 1;
  } else {
    p.help_eager = h->help_eager >= 0 ? h->help_eager : (fills ? 1 : 0);
    p.eager_items = p.n_items;
    p.land_between = 0;
    p.help_every = h->help_every > 0 ? h->help_every : (p.help_eager ? 1 : 2);
  }
  const int grid = std::max(1, land + compute);
  p.sync = make_sync(h, (uint32_t)(world * p.blocks_per_chunk * p.n_slabs));
  hipError_t e = hipSuccess;
  if (h->scratch) e = scratch_clear(h, p.sync.n_flags, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(h, e, "launching the control-memory clear");
  e = mk::launch_ag(p, bm, bn, grid, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(h, e, "launching the AllGather+GEMM kernel");
  if (h->scratch && status) e = scratch_report(h, status, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(h, e, "launching the status report");
  record(h, MK_OP_AG_GEMM, land, compute, 0, grid);
  return MK_OK;
}

mk_status mk_ag_gemm(mk_handle h, mk_stream stream, int world, int rank,
                     const mk_bf16 *const *a_shards, const mk_bf16 *bt, mk_bf16 *c,
                     mk_bf16 *a_gathered, int m_s, int n, int k, unsigned flags) {
  if (h && h->scratch) return MK_ERR_INVALID;
  return ag_gemm_impl(h, stream, world, rank, a_shards, bt, c, a_gathered, m_s, n, k, flags, nullptr);
}

mk_status mk_ag_gemm_noalloc(mk_stream stream, int world, int rank, const mk_bf16 *const *a_shards,
                             const mk_bf16 *bt, mk_bf16 *c, mk_bf16 *a_gathered, int m_s, int n, int k,
                             unsigned flags, int32_t *status) {
  mk_ctx *h = nullptr;
  mk_status st = scratch_ctx(&h);
  if (st != MK_OK) return st;
  if (status) {
    const void *dp;
    if ((st = resolve(h, status, sizeof(int32_t) * 2, false, &dp, "status")) != MK_OK) return st;
    status = static_cast<int32_t *>(const_cast<void *>(dp));
  }
  return ag_gemm_impl(h, stream, world, rank, a_shards, bt, c, a_gathered, m_s, n, k, flags, status);
}

// ---------------------------------------------------------------- GEMM + ReduceScatter

mk_status mk_gemm_rs(mk_handle h, mk_stream stream, int world, int rank, const mk_bf16 *a,
                     const mk_bf16 *bt, const float *const *peer_part, mk_bf16 *c_own,
                     mk_bf16 *const *outbox, int m, int n, int k, unsigned flags) {
  mk_status st = check_common(h, world, rank);
  if (st != MK_OK) return st;
  if (flags & ~(MK_F_NO_PEERS | MK_F_STATIC_ROLES)) return fail(h, MK_ERR_INVALID, "unknown flag bits");
  if (world > 1 && (!peer_part || !outbox)) return fail(h, MK_ERR_INVALID, "peer_part / outbox is NULL");
  st = check_gemm_shape(h, m, n, k);
  if (st != MK_OK) return st;
  if (m % world) return fail(h, MK_ERR_INVALID, "m must be a multiple of world");
  DeviceGuard g(h->device);
  const bool no_peers = (flags & MK_F_NO_PEERS) != 0;
  mk::RsParams p;
  std::memset(&p, 0, sizeof(p));
  const void *dp;
  if ((st = resolve(h, a, (size_t)m * k * 2, false, &dp, "a")) != MK_OK) return st;
  p.a = static_cast<const uint16_t *>(dp);
  if ((st = resolve(h, bt, (size_t)n * k * 2, false, &dp, "bt")) != MK_OK) return st;
  p.bt = static_cast<const uint16_t *>(dp);
  if ((st = resolve(h, c_own, (size_t)(m / world) * n * 2, true, &dp, "c_own")) != MK_OK) return st;
  p.c_own = static_cast<uint16_t *>(const_cast<void *>(dp));
  for (int q = 0; q < world; ++q) {
    if (q == rank) continue;
    char what[32];
    if (!no_peers) {  // compute alone reads no partial
      std::snprintf(what, sizeof(what), "peer_part[%d]", q);
      if ((st = resolve(h, peer_part[q], (size_t)(m / world) * n * 4, true, &dp, what)) != MK_OK) return st;
      p.peer_c[q < rank ? q : q - 1] = static_cast<const float *>(dp);
    }
    std::snprintf(what, sizeof(what), "outbox[%d]", q);
    if ((st = resolve(h, outbox[q], (size_t)(m / world) * n * 2, true, &dp, what)) != MK_OK) return st;
    p.outbox[q] = static_cast<uint16_t *>(const_cast<void *>(dp));
  }
  const int bm = pick_tile(h, (long)cdiv(m, 256) * cdiv(n, 256));
  p.world = world;
  p.rank = rank;
  p.m = m;
  p.n = n;
  p.k = k;
  p.ms = m / world;
  p.no_peers = no_peers ? 1 : 0;
  p.tiles_m = cdiv(m, bm);
  p.tiles_n = cdiv(n, bm);
  p.n_tiles = p.tiles_m * p.tiles_n;
  p.tile_map = h->tile_map >= 0 ? h->tile_map : mk::kMapRounds;
  const int gmax = max_grid(h, MK_OP_GEMM_RS, bm);
  const int lo = rank * p.ms, hi = lo + p.ms;
  const int mb_lo = lo / bm, mb_hi = (hi - 1) / bm;
  Roles ro;
  if ((st = choose_reduce_roles(h, MK_OP_GEMM_RS, gmax, p.n_tiles, world > 1 && !no_peers, flags, &ro)) != MK_OK)
    return st;
  p.n_compute = ro.compute;
  p.red.n_reduce = ro.reduce;
  p.red.xfer_only = ro.xfer;
  p.red.joins_compute = ro.joins;
  if (ro.xfer) {  // transfer alone: every tile's rows, no flags
    p.red.mb_lo = 0;
    p.red.mbs = p.tiles_m;
    p.red.n_items = p.n_tiles;
  } else if (ro.items) {  // the own slice's tiles
    p.red.mb_lo = mb_lo;
    p.red.mbs = mb_hi - mb_lo + 1;
    p.red.n_items = p.red.mbs * p.tiles_n;
    if (p.red.n_items > mk::kMaxFlags) return fail(h, MK_ERR_UNSUPPORTED, "too many reduce items for the flags");
    if ((st = need_ws(h, (size_t)p.ms * n * 4, "the GEMM+ReduceScatter reduce role")) != MK_OK) return st;
    p.red.ws = static_cast<float *>(h->ws);
    p.red.light_acquire = n % 32 == 0 ? 1 : 0;
  }
  // tile order: the own slice first (its epilogue reads the peers' partials,
  // the heaviest), or last when the reduce role sums the partials meanwhile
  p.mb0 = p.red.n_items > 0 && !ro.xfer ? (mb_hi + 1) % p.tiles_m : mb_lo;
  const int grid = std::max(1, ro.reduce + ro.compute);
  rounds_order(p.tiles_m, p.tiles_n, grid, bm, bm, &p.tile_group_m, &p.tile_split_m);
  p.sync = make_sync(h, ro.xfer ? 0u : (uint32_t)p.red.n_items);
  hipError_t e = mk::launch_rs(p, bm, grid, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(h, e, "launching the GEMM+ReduceScatter kernel");
  record(h, MK_OP_GEMM_RS, 0, ro.compute, ro.reduce, grid);
  return MK_OK;
}

// ---------------------------------------------------------------- GEMM + AllReduce

mk_status mk_gemm_ar(mk_handle h, mk_stream stream, int world, int rank, const mk_bf16 *a,
                     const mk_bf16 *bt, const float *const *peer_part, mk_bf16 *c,
                     mk_bf16 *const *bcast, int n_bcast, int m, int n, int k, unsigned flags) {
  mk_status st = check_common(h, world, rank);
  if (st != MK_OK) return st;
  if (flags & ~(MK_F_NO_PEERS | MK_F_STATIC_ROLES)) return fail(h, MK_ERR_INVALID, "unknown flag bits");
  if (n_bcast < 0 || n_bcast > MK_MAX_WORLD) return fail(h, MK_ERR_INVALID, "n_bcast out of range");
  if (world > 1 && !peer_part) return fail(h, MK_ERR_INVALID, "peer_part is NULL");
  if (n_bcast > 0 && !bcast) return fail(h, MK_ERR_INVALID, "bcast is NULL");
  st = check_gemm_shape(h, m, n, k);
  if (st != MK_OK) return st;
  DeviceGuard g(h->device);
  const bool no_peers = (flags & MK_F_NO_PEERS) != 0;
  mk::ArParams p;
  std::memset(&p, 0, sizeof(p));
  const void *dp;
  if ((st = resolve(h, a, (size_t)m * k * 2, false, &dp, "a")) != MK_OK) return st;
  p.a = static_cast<const uint16_t *>(dp);
  if ((st = resolve(h, bt, (size_t)n * k * 2, false, &dp, "bt")) != MK_OK) return st;
  p.bt = static_cast<const uint16_t *>(dp);
  if ((st = resolve(h, c, (size_t)m * n * 2, true, &dp, "c")) != MK_OK) return st;
  p.c = static_cast<uint16_t *>(const_cast<void *>(dp));
  for (int q = 0; q < world && !no_peers; ++q) {
    if (q == rank) continue;
    char what[32];
    std::snprintf(what, sizeof(what), "peer_part[%d]", q);
    if ((st = resolve(h, peer_part[q], (size_t)m * n * 4, true, &dp, what)) != MK_OK) return st;
    p.peer_c[q < rank ? q : q - 1] = static_cast<const float *>(dp);
  }
  for (int b = 0; b < n_bcast; ++b) {
    char what[32];
    std::snprintf(what, sizeof(what), "bcast[%d]", b);
    if ((st = resolve(h, bcast[b], (size_t)m * n * 2, true, &dp, what)) != MK_OK) return st;
    p.bcast[b] = static_cast<uint16_t *>(const_cast<void *>(dp));
  }
  const int bm = pick_tile(h, (long)cdiv(m, 256) * cdiv(n, 256));
  p.world = world;
  p.rank = rank;
  p.n_bcast = n_bcast;
  p.m = m;
  p.n = n;
  p.k = k;
  p.no_peers = no_peers ? 1 : 0;
  p.tiles_m = cdiv(m, bm);
  p.tiles_n = cdiv(n, bm);
  p.n_tiles = p.tiles_m * p.tiles_n;
  p.tile_map = h->tile_map >= 0 ? h->tile_map : mk::kMapGlobal;
  const int gmax = max_grid(h, MK_OP_GEMM_AR, bm);
  Roles ro;
  if ((st = choose_reduce_roles(h, MK_OP_GEMM_AR, gmax, p.n_tiles, world > 1 && !no_peers, flags, &ro)) != MK_OK)
    return st;
  p.n_compute = ro.compute;
  p.red.n_reduce = ro.reduce;
  p.red.xfer_only = ro.xfer;
  p.red.joins_compute = ro.joins;
  if (ro.xfer || ro.items) {  // every tile is a reduce item
    p.red.mb_lo = 0;
    p.red.mbs = p.tiles_m;
    p.red.n_items = p.n_tiles;
  }
  if (ro.items && !ro.xfer) {
    if (p.red.n_items > mk::kMaxFlags) return fail(h, MK_ERR_UNSUPPORTED, "too many reduce items for the flags");
    if ((st = need_ws(h, (size_t)m * n * 4, "the GEMM+AllReduce reduce role")) != MK_OK) return st;
    p.red.ws = static_cast<float *>(h->ws);
    p.red.light_acquire = n % 32 == 0 ? 1 : 0;
  }
  const int grid = std::max(1, ro.reduce + ro.compute);
  rounds_order(p.tiles_m, p.tiles_n, grid, bm, bm, &p.tile_group_m, &p.tile_split_m);
  p.sync = make_sync(h, ro.xfer ? 0u : (uint32_t)p.red.n_items);
  hipError_t e = mk::launch_ar(p, bm, grid, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(h, e, "launching the GEMM+AllReduce kernel");
  record(h, MK_OP_GEMM_AR, 0, ro.compute, ro.reduce, grid);
  return MK_OK;
}

// ---------------------------------------------------------------- MoE dispatch + grouped GEMM

// Shared by mk_moe_dispatch_gemm and mk_moe_dispatch_gemm_combine; the
// combine arguments are NULL for the former.
static mk_status moe_launch(mk_handle h, mk_stream stream, int n_src, int rank,
                            const mk_bf16 *const *x_src, const float *const *logits_src,
                            const mk_bf16 *wt, int T, int H, int N, int E, int E_loc, int top_k,
                            mk_bf16 *y, int32_t *topk_idx, float *topk_gate, int32_t *slot_token,
                            int32_t *expert_offsets, int32_t *chunk_offsets, mk_bf16 *x_slots,
                            int cap, bool combine, const mk_bf16 *y_peer, mk_bf16 *const *ret,
                            mk_bf16 *out, unsigned flags) {
  if (!h) return MK_ERR_INVALID;
  h->err.clear();
  if (n_src < 1 || n_src > MK_MAX_WORLD) return fail(h, MK_ERR_INVALID, "n_src out of range");
  if (flags & ~(MK_F_NO_GATE | MK_F_STATIC_ROLES)) return fail(h, MK_ERR_INVALID, "unknown flag bits");
  if (!x_src || !logits_src) return fail(h, MK_ERR_INVALID, "x_src / logits_src is NULL");
  if (T < 1 || H < 8 || N < 8 || H % 8 || N % 8) return fail(h, MK_ERR_INVALID, "bad T / H / N");
  if (top_k < 1 || top_k > 8 || E < top_k || E > 256) return fail(h, MK_ERR_INVALID, "bad E / top_k");
  if (E_loc < 1 || E_loc > mk::kMaxLocalExperts || rank < 0 || (long)(rank + 1) * E_loc > E)
    return fail(h, MK_ERR_INVALID, "bad E_loc / rank");
  const long need = (long)n_src * T * std::min(top_k, E_loc);
  if (cap < need) return fail(h, MK_ERR_INVALID, "cap < n_src*T*min(top_k, E_loc)");
  if (cap >= (1 << 23) || (long)n_src * T * top_k >= (1L << 30) || H > (1 << 20))
    return fail(h, MK_ERR_UNSUPPORTED, "MoE sizes beyond the supported range");
  DeviceGuard g(h->device);
  mk::MoeParams p;
  std::memset(&p, 0, sizeof(p));
  const void *dp;
  mk_status st;
  for (int s = 0; s < n_src; ++s) {
    char what[32];
    std::snprintf(what, sizeof(what), "x_src[%d]", s);
    if ((st = resolve(h, x_src[s], (size_t)T * H * 2, s != rank, &dp, what)) != MK_OK) return st;
    p.x[s] = static_cast<const uint16_t *>(dp);
    std::snprintf(what, sizeof(what), "logits_src[%d]", s);
    if ((st = resolve(h, logits_src[s], (size_t)T * E * 4, true, &dp, what)) != MK_OK) return st;
    p.logits[s] = static_cast<const float *>(dp);
  }
  if ((st = resolve(h, wt, (size_t)E_loc * N * H * 2, false, &dp, "wt")) != MK_OK) return st;
  p.wt = static_cast<const uint16_t *>(dp);
  if ((st = resolve(h, y, (size_t)cap * N * 2, true, &dp, "y")) != MK_OK) return st;
  p.y = static_cast<uint16_t *>(const_cast<void *>(dp));
  if ((st = resolve(h, topk_idx, (size_t)n_src * T * top_k * 4, true, &dp, "topk_idx")) != MK_OK) return st;
  p.topk_idx = static_cast<int32_t *>(const_cast<void *>(dp));
  if ((st = resolve(h, topk_gate, (size_t)n_src * T * top_k * 4, true, &dp, "topk_gate")) != MK_OK) return st;
  p.topk_gate = static_cast<float *>(const_cast<void *>(dp));
  if ((st = resolve(h, slot_token, (size_t)cap * 4, true, &dp, "slot_token")) != MK_OK) return st;
  p.slot_token = static_cast<int32_t *>(const_cast<void *>(dp));
  if ((st = resolve(h, expert_offsets, (size_t)(E_loc + 1) * 4, true, &dp, "expert_offsets")) != MK_OK) return st;
  p.expert_offsets = static_cast<int32_t *>(const_cast<void *>(dp));
  if ((st = resolve(h, chunk_offsets, (size_t)E_loc * (n_src + 1) * 4, true, &dp, "chunk_offsets")) != MK_OK) return st;
  p.chunk_offsets = static_cast<int32_t *>(const_cast<void *>(dp));
  if ((st = resolve(h, x_slots, (size_t)cap * H * 2, false, &dp, "x_slots")) != MK_OK) return st;
  p.x_slots = static_cast<uint16_t *>(const_cast<void *>(dp));
  if (combine) {
    if (flags & MK_F_NO_GATE) return fail(h, MK_ERR_INVALID, "the combine sums gated rows: MK_F_NO_GATE");
    if (rank >= n_src) return fail(h, MK_ERR_INVALID, "the combine sums this rank's own tokens: rank >= n_src");
    if (n_src > 1 && !ret) return fail(h, MK_ERR_INVALID, "ret is NULL");
    if ((st = resolve(h, y_peer, (size_t)T * top_k * N * 2, true, &dp, "y_peer")) != MK_OK) return st;
    p.y_peer = static_cast<const uint16_t *>(dp);
    if ((st = resolve(h, out, (size_t)T * N * 2, true, &dp, "out")) != MK_OK) return st;
    p.out = static_cast<uint16_t *>(const_cast<void *>(dp));
    for (int s = 0; s < n_src; ++s) {
      if (s == rank) continue;
      char what[32];
      std::snprintf(what, sizeof(what), "ret[%d]", s);
      if ((st = resolve(h, ret[s], (size_t)T * top_k * N * 2, true, &dp, what)) != MK_OK) return st;
      p.ret[s] = static_cast<uint16_t *>(const_cast<void *>(dp));
    }
    p.combine = 1;
  }

  p.S = n_src;
  p.T = T;
  p.H = H;
  p.N = N;
  p.E = E;
  p.E_loc = E_loc;
  p.top_k = top_k;
  p.rank = rank;
  p.cap = cap;
  p.items_per_src = cdiv(T, mk::kRouteTokens);
  p.n_items = n_src * p.items_per_src;
  if (p.n_items > mk::kMaxFlags) return fail(h, MK_ERR_UNSUPPORTED, "too many route items");
  p.no_gate = (flags & MK_F_NO_GATE) ? 1 : 0;
  p.static_roles = (flags & MK_F_STATIC_ROLES) ? 1 : 0;
  p.withhold = h->moe_withhold;

  // expected routed rows decide the tile edge
  const long exp_rows = (long)n_src * T * top_k * E_loc / E;
  const int bm = pick_tile(h, (long)(cdiv((int)std::max(1L, exp_rows), 256) + E_loc) * cdiv(N, 256));
  p.tiles_n = cdiv(N, bm);
  p.tile_map = h->tile_map >= 0 ? h->tile_map : mk::kMapBlocks;
  const long max_row_tiles = cdiv(cap, bm) + E_loc;

  // workspace: item_cnt, item_base, tok_rank, slot_gate, slot_ret
  const size_t sz_items = (size_t)p.n_items * E_loc * sizeof(int32_t);
  const size_t sz_rank = (size_t)n_src * T * top_k * sizeof(int32_t);
  const size_t sz_gate = (size_t)cap * sizeof(float);
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t total = al(sz_items) * 2 + al(sz_rank) + al(sz_gate) * 2;
  if ((st = need_ws(h, total, "the MoE dispatch")) != MK_OK) return st;
  char *w = static_cast<char *>(h->ws);
  p.item_cnt = reinterpret_cast<int32_t *>(w);
  w += al(sz_items);
  p.item_base = reinterpret_cast<int32_t *>(w);
  w += al(sz_items);
  p.tok_rank = reinterpret_cast<int32_t *>(w);
  w += al(sz_rank);
  p.slot_gate = reinterpret_cast<float *>(w);
  w += al(sz_gate);
  p.slot_ret = reinterpret_cast<int32_t *>(w);

  const int gmax = max_grid(h, MK_OP_MOE, bm);
  const mk_roles &r = h->roles[MK_OP_MOE];
  // compute workgroups land while their rows are missing, so a small land
  // role suffices (1/16 of the grid measured 1-3% faster than 1/8)
  int land = r.n_land >= 0 ? r.n_land : std::max(1, std::min(p.n_items, gmax / 16));
  land = std::max(1, std::min(land, 4 * gmax));  // landing cannot be switched off: compute depends on it
  int compute = r.n_compute >= 0 ? std::min(r.n_compute, 4 * gmax)
                                 : (int)std::max(1L, std::min(max_row_tiles * p.tiles_n, (long)gmax - land));
  if (combine && p.static_roles) {
    // With static roles the land workgroups wait for the last tile before
    // they combine without taking tiles, so at least one compute workgroup
    // must be resident besides them: keep the grid within one residency.
    land = std::min(land, std::max(1, gmax - 1));
    compute = std::max(1, std::min(compute, gmax - land));
  }
  p.n_land = land;
  p.n_compute = compute;
  const int grid = land + compute;
  p.sync = make_sync(h, (uint32_t)p.n_items);
  hipError_t e = mk::launch_moe(p, bm, grid, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(h, e, "launching the MoE dispatch kernel");
  record(h, MK_OP_MOE, land, compute, 0, grid);
  return MK_OK;
}

mk_status mk_moe_dispatch_gemm(mk_handle h, mk_stream stream, int n_src, int rank,
                               const mk_bf16 *const *x_src, const float *const *logits_src,
                               const mk_bf16 *wt, int T, int H, int N, int E, int E_loc,
                               int top_k, mk_bf16 *y, int32_t *topk_idx, float *topk_gate,
                               int32_t *slot_token, int32_t *expert_offsets,
                               int32_t *chunk_offsets, mk_bf16 *x_slots, int cap,
                               unsigned flags) {
  return moe_launch(h, stream, n_src, rank, x_src, logits_src, wt, T, H, N, E, E_loc, top_k, y,
                    topk_idx, topk_gate, slot_token, expert_offsets, chunk_offsets, x_slots, cap,
                    false, nullptr, nullptr, nullptr, flags);
}

mk_status mk_moe_dispatch_gemm_combine(mk_handle h, mk_stream stream, int n_src, int rank,
                                       const mk_bf16 *const *x_src, const float *const *logits_src,
                                       const mk_bf16 *wt, int T, int H, int N, int E, int E_loc,
                                       int top_k, mk_bf16 *y, int32_t *topk_idx, float *topk_gate,
                                       int32_t *slot_token, int32_t *expert_offsets,
                                       int32_t *chunk_offsets, mk_bf16 *x_slots, int cap,
                                       const mk_bf16 *y_peer, mk_bf16 *const *ret, mk_bf16 *out,
                                       unsigned flags) {
  return moe_launch(h, stream, n_src, rank, x_src, logits_src, wt, T, H, N, E, E_loc, top_k, y,
                    topk_idx, topk_gate, slot_token, expert_offsets, chunk_offsets, x_slots, cap,
                    true, y_peer, ret, out, flags);
}

// ---------------------------------------------------------------- ring attention

mk_status mk_ring_attention(mk_handle h, mk_stream stream, int world, int rank, const mk_bf16 *q,
                            const mk_bf16 *const *k_src, const mk_bf16 *const *v_src, int BH,
                            int S_q, int S_kv, int D, float scale, mk_bf16 *o, float *lse,
                            mk_bf16 *k_recv, mk_bf16 *vt_recv, unsigned flags) {
  if (!h) return MK_ERR_INVALID;
  h->err.clear();
  if (world < 1 || world > MK_MAX_WORLD || rank < 0 || rank >= world)
    return fail(h, MK_ERR_INVALID, "bad world / rank");
  if (flags & ~MK_F_PRELANDED) return fail(h, MK_ERR_INVALID, "unknown flag bits");
  const bool pre = (flags & MK_F_PRELANDED) != 0;
  if (!pre && (!k_src || !v_src)) return fail(h, MK_ERR_INVALID, "k_src / v_src is NULL");
  if (BH < 1 || S_q < 1 || S_kv < 1) return fail(h, MK_ERR_INVALID, "bad BH / S_q / S_kv");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(h, MK_ERR_INVALID, "scale must be positive and finite");
  if (D != mk::kAttnD || S_kv % 64 != 0)
    return fail(h, MK_ERR_UNSUPPORTED, "ring attention needs D = 128 and S_kv a multiple of 64");
  if ((long)BH * S_q * D >= (1L << 31) || (long)world * BH * S_kv * D >= (1L << 34))
    return fail(h, MK_ERR_UNSUPPORTED, "ring attention sizes beyond the supported range");
  DeviceGuard g(h->device);
  mk::AttnParams p;
  std::memset(&p, 0, sizeof(p));
  const void *dp;
  mk_status st;
  if ((st = resolve(h, q, (size_t)BH * S_q * D * 2, false, &dp, "q")) != MK_OK) return st;
  p.q = static_cast<const uint16_t *>(dp);
  for (int r = 0; r < world && !pre; ++r) {
    char what[32];
    std::snprintf(what, sizeof(what), "k_src[%d]", r);
    if ((st = resolve(h, k_src[r], (size_t)BH * S_kv * D * 2, r != rank, &dp, what)) != MK_OK) return st;
    p.k_src[r] = static_cast<const uint16_t *>(dp);
    std::snprintf(what, sizeof(what), "v_src[%d]", r);
    if ((st = resolve(h, v_src[r], (size_t)BH * S_kv * D * 2, r != rank, &dp, what)) != MK_OK) return st;
    p.v_src[r] = static_cast<const uint16_t *>(dp);
  }
  if ((st = resolve(h, o, (size_t)BH * S_q * D * 2, false, &dp, "o")) != MK_OK) return st;
  p.o = static_cast<uint16_t *>(const_cast<void *>(dp));
  if ((st = resolve(h, lse, (size_t)BH * S_q * 4, false, &dp, "lse")) != MK_OK) return st;
  p.lse = static_cast<float *>(const_cast<void *>(dp));
  if ((st = resolve(h, k_recv, (size_t)world * BH * S_kv * D * 2, false, &dp, "k_recv")) != MK_OK) return st;
  p.k_recv = static_cast<uint16_t *>(const_cast<void *>(dp));
  if ((st = resolve(h, vt_recv, (size_t)world * BH * S_kv * D * 2, false, &dp, "vt_recv")) != MK_OK) return st;
  p.vt_recv = static_cast<uint16_t *>(const_cast<void *>(dp));

  p.world = world;
  p.rank = rank;
  p.BH = BH;
  p.S_q = S_q;
  p.S_kv = S_kv;
  p.scale_log2 = scale * 1.44269504088896340736f;
  // landing chunks: 256 keys (64 KB of K, 64 KB of V), larger while the flags
  // would not fit
  p.chunk_keys = 256;
  while ((long)world * BH * cdiv(S_kv, p.chunk_keys) > mk::kMaxFlags) p.chunk_keys *= 2;
  p.chunks = cdiv(S_kv, p.chunk_keys);
  p.n_items = world * BH * p.chunks;
  p.q_tiles = cdiv(S_q, 128);
  p.n_pairs = BH * p.q_tiles;
  if (p.n_pairs >= (1 << 29)) return fail(h, MK_ERR_UNSUPPORTED, "too many attention tasks");
  // two tasks per (bh, q-tile), one per half of the ring's key tiles, when
  // there are two tiles and flags for the pairs: smaller tasks balance the
  // workgroups that join after landing
  const long n_tiles = (long)world * (S_kv / 64);
  p.splits = (h->ring_splits != 1 && n_tiles >= 2 && (long)p.n_items + p.n_pairs <= mk::kMaxFlags) ? 2 : 1;
  p.n_tasks = p.splits * p.n_pairs;
  p.tile_map = h->tile_map >= 0 ? h->tile_map : mk::kMapBlocks;
  if (p.tile_map == mk::kMapRounds) p.tile_map = mk::kMapBlocks;  // no rounds order for tasks
  p.merge_flag0 = (uint32_t)p.n_items;
  if (p.splits == 2) {
    const size_t slot = (size_t)(128 * 128 + 2 * 128) * sizeof(float);
    if ((st = need_ws(h, slot * p.n_pairs, "ring attention")) != MK_OK) return st;
    p.ws = static_cast<float *>(h->ws);
  }
  // chunks of both receive buffers start and end on 128-byte lines
  p.light_acquire = ((reinterpret_cast<uintptr_t>(p.k_recv) | reinterpret_cast<uintptr_t>(p.vt_recv)) & 127u) == 0 ? 1 : 0;

  const int gmax = max_grid(h, MK_OP_RING_ATTN, 256);
  const mk_roles &r = h->roles[MK_OP_RING_ATTN];
  // every workgroup waits for land workgroups, so all must be resident at once
  // the blocks are as large as the queries' share of the work is small:
  // a quarter of the grid lands (then computes), which keeps every ring step
  // landed ahead of the tasks that consume it (3/16 and 1/2 were slower)
  int land = r.n_land >= 0 ? r.n_land : std::min(p.n_items, std::max(1, gmax / 4));
  land = pre ? 0 : std::max(1, std::min(land, gmax));
  p.prelanded = pre ? 1 : 0;
  int compute = r.n_compute >= 0 ? r.n_compute : std::min(p.n_tasks, gmax - land);
  compute = std::max(0, std::min(compute, gmax - land));
  p.n_land = land;
  p.n_compute = compute;
  const int grid = std::max(1, land + compute);
  p.sync = make_sync(h, (uint32_t)(p.n_items + (p.splits == 2 ? p.n_pairs : 0)));
  hipError_t e = mk::launch_attn(p, grid, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(h, e, "launching the ring attention kernel");
  record(h, MK_OP_RING_ATTN, land, compute, 0, grid);
  return MK_OK;
}

// ---------------------------------------------------------------- measurement aid

mk_status mk_mfma_ceiling(mk_handle h, mk_stream stream, int iters, float *sink) {
  if (!h) return MK_ERR_INVALID;
  h->err.clear();
  if (iters < 1 || iters > (1 << 24)) return fail(h, MK_ERR_INVALID, "iters out of range");
  DeviceGuard g(h->device);
  const void *dp;
  mk_status st;
  if ((st = resolve(h, sink, 256 * sizeof(float), false, &dp, "sink")) != MK_OK) return st;
  // two 256-thread workgroups per CU: 2 waves per SIMD
  hipError_t e = mk::launch_mfma_loop(2 * h->cu_count, iters, static_cast<float *>(const_cast<void *>(dp)),
                                      reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(h, e, "launching the MFMA loop");
  return MK_OK;
}

}  // extern "C"

// Device-side building blocks of the persistent fused kernels (gfx950 only).
//
//  * control block, per-chunk flags and arrival counters
//  * release / acquire flag protocol with bounded waits
//  * a bf16 MFMA GEMM tile engine with a double-buffered LDS pipeline fed by
//    direct global->LDS buffer loads
//
// The operations follow the mKernel articles: [P1] German article
// (chatgpz.de), section "Was mKernel macht" (persistent kernel, CTAs assign
// themselves compute / communication roles, tile/chunk-granular overlap).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mk.h"

namespace mk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kMaxWaves = 8;      // workgroups have up to 8 waves of 64 lanes
constexpr int kBK = 64;           // K elements per pipeline stage (128 bytes of bf16 per row)
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset that always fails the range check -> 0
constexpr int kFlagStride = 16;   // uint32 words between flags (64 bytes)
constexpr int kMaxFlags = 8192;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format, gfx9 family

// Error codes recorded on the device (match mk_status values).
constexpr uint32_t kErrTimeout = MK_ERR_TIMEOUT;
constexpr uint32_t kErrInternal = 100;  // an index check failed; reported as MK_ERR_HIP

// One control block per handle.  Every counter lives on its own 64-byte line.
struct Ctrl {
  uint32_t ticket;      uint32_t _p0[15];
  uint32_t tile_ctr;    uint32_t _p1[15];
  uint32_t land_ctr;    uint32_t _p2[15];
  uint32_t reduce_ctr;  uint32_t _p3[15];
  uint32_t done;        uint32_t _p4[15];
  uint32_t abort_epoch; uint32_t _p5[15];
  uint32_t err_code;    uint32_t err_info; uint32_t err_epoch; uint32_t _p6[13];
  uint32_t route_ctr;   uint32_t _p7[15];
  uint32_t route_done;  uint32_t _p8[15];
  uint32_t scan_ready;  uint32_t _p9[15];
  uint32_t xq[8 * 16];  // per-XCD tile queue counters, one 64-byte line each
  uint32_t tiles_done;  uint32_t _p10[15];
  uint32_t combine_ctr; uint32_t _p11[15];
};

// Per-launch synchronisation state passed to every kernel.
struct Sync {
  Ctrl *ctrl;
  uint32_t *flags;   // kMaxFlags flags, kFlagStride words apart, value = epoch when ready
  uint32_t *cnt;     // arrival counters, same layout; self-resetting
  uint32_t epoch;    // this launch's epoch (never 0)
  uint32_t n_flags;  // flags/counters this launch uses (cleared after an abort)
  uint64_t timeout_ticks;  // bound on every wait, in s_memrealtime ticks
};

// ---------------------------------------------------------------- atomics

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_acq_rel(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_relaxed(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A store that the writer's L2 writes through to memory (device scope, the
// sc1 bit): once the thread's stores are complete it is visible to every
// XCD, and publishing it needs no write-back of the L2.
template <class T>
__device__ __forceinline__ void st_through(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}
__device__ __forceinline__ void fence_release() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}

__device__ __forceinline__ uint32_t *flag_ptr(const Sync &s, uint32_t i) {
  return s.flags + (size_t)i * kFlagStride;
}
__device__ __forceinline__ uint32_t *cnt_ptr(const Sync &s, uint32_t i) {
  return s.cnt + (size_t)i * kFlagStride;
}

__device__ __forceinline__ bool aborted(const Sync &s) {
  return ld_relaxed(&s.ctrl->abort_epoch) == s.epoch;
}

// Record a failure (first one wins) and tell every workgroup of this launch to stop.
__device__ __forceinline__ void raise_error(const Sync &s, uint32_t code, uint32_t info) {
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(&s.ctrl->err_code, &expected, code, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    st_relaxed(&s.ctrl->err_info, info);
    st_relaxed(&s.ctrl->err_epoch, s.epoch);
  }
  st_relaxed(&s.ctrl->abort_epoch, s.epoch);
}

// Spin (one thread) until *p == want.  Returns false on timeout or abort.
// The caller issues the acquire fence after a successful wait.
__device__ __forceinline__ bool spin_until_eq(const Sync &s, const uint32_t *p, uint32_t want,
                                           uint32_t info) {
  if (ld_relaxed(p) == want) return true;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    __builtin_amdgcn_s_sleep(2);
    if (ld_relaxed(p) == want) return true;
    if (aborted(s)) return false;
    if (__builtin_amdgcn_s_memrealtime() - t0 > s.timeout_ticks) {
      raise_error(s, kErrTimeout, info);
      return false;
    }
  }
}

// Spin (one thread) until *p >= want (a monotone counter within one launch).
__device__ __forceinline__ bool spin_until_ge(const Sync &s, const uint32_t *p, uint32_t want,
                                           uint32_t info) {
  if (ld_relaxed(p) >= want) return true;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    __builtin_amdgcn_s_sleep(2);
    if (ld_relaxed(p) >= want) return true;
    if (aborted(s)) return false;
    if (__builtin_amdgcn_s_memrealtime() - t0 > s.timeout_ticks) {
      raise_error(s, kErrTimeout, info);
      return false;
    }
  }
}

// Every lane of one wave: spin until *p == want in every lane whose `need`
// is set (lanes may watch different words).  The exit conditions are
// wave-uniform (a ballot, the scalar clock, lane 0's view of the abort word),
// so the wave leaves together.  Returns false on timeout or abort.
__device__ __forceinline__ bool wave_spin_all_eq(const Sync &s, const uint32_t *p, bool need, uint32_t want,
                                                 uint32_t info) {
  bool pending = need && ld_relaxed(p) != want;
  if (__ballot(pending) == 0) return true;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    __builtin_amdgcn_s_sleep(2);
    if (pending) pending = ld_relaxed(p) != want;
    if (__ballot(pending) == 0) return true;
    if (__builtin_amdgcn_readfirstlane((int)aborted(s))) return false;
    if (__builtin_amdgcn_s_memrealtime() - t0 > s.timeout_ticks) {
      if ((threadIdx.x & 63) == 0) raise_error(s, kErrTimeout, info);
      return false;
    }
  }
}

// Arrival of one work item of flag `f`, which completes after `target` items.
// Called by one thread after every thread of the workgroup has waited for
// its own stores (wait_stores) and the workgroup has passed a barrier: the
// release fence writes this XCD's L2 back, so the item's data is in memory
// before the count moves.  The last arrival acquires the other arrivals'
// releases, resets the counter and publishes the flag.
__device__ __forceinline__ void arrive(const Sync &s, uint32_t f, uint32_t target) {
  fence_release();
  const uint32_t old = add_relaxed(cnt_ptr(s, f), 1u);
  if (old + 1 == target) {
    fence_acquire();
    st_relaxed(cnt_ptr(s, f), 0u);
    st_release(flag_ptr(s, f), s.epoch);
  }
}

// Arrival of one work item whose stores were written through to memory
// (kStoreWriteThrough): every thread of the workgroup has waited for its
// own stores (wait_stores) and passed a barrier, so the item's data is in
// memory already and the count moves without the L2 write-back that
// arrive() pays for (a write-back of the whole XCD's L2, whose cost grows
// with every other workgroup's dirty lines).  The last arrival publishes the
// flag as arrive() does.
__device__ __forceinline__ void arrive_written_through(const Sync &s, uint32_t f, uint32_t target) {
  const uint32_t old = add_relaxed(cnt_ptr(s, f), 1u);
  if (old + 1 == target) {
    fence_acquire();
    st_relaxed(cnt_ptr(s, f), 0u);
    st_release(flag_ptr(s, f), s.epoch);
  }
}

// Wait for this thread's outstanding global stores (and loads).
__device__ __forceinline__ void wait_stores() {
  __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));  // vmcnt(0)
}

// Values that thread 0 broadcasts through LDS are identical in every lane,
// but the compiler cannot know that; without readfirstlane it treats loops
// and branches on them as divergent.
__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Every single-thread region (if (threadIdx.x == 0) ...) is bracketed by
// barriers: two such regions with no barrier between them (say, the arrival
// at the end of one loop iteration and the counter fetch at the start of the
// next) can be merged by the compiler into a lane-0-only path out of the
// loop, leaving the other lanes to meet the loop's barriers without lane 0.

// Take this workgroup's role ticket (all threads get the value).
__device__ __forceinline__ uint32_t take_ticket(const Sync &s, uint32_t *lds_word) {
  __syncthreads();
  if (threadIdx.x == 0) *lds_word = add_relaxed(&s.ctrl->ticket, 1u);
  __syncthreads();
  return uniform(*lds_word);
}

// Copy a kernel's parameter block to LDS, one word per thread (the caller's
// next barrier publishes it).
template <class P>
__device__ __forceinline__ void copy_params(P *dst, const P &src) {
  static_assert(sizeof(P) % 4 == 0, "parameters copy as words");
  for (int i = (int)threadIdx.x; i < (int)(sizeof(P) / 4); i += (int)blockDim.x)
    reinterpret_cast<uint32_t *>(dst)[i] = reinterpret_cast<const uint32_t *>(&src)[i];
}

// Fetch the next index from a device counter (all threads get the value).
__device__ __forceinline__ uint32_t next_index(uint32_t *ctr, uint32_t *lds_word) {
  __syncthreads();
  if (threadIdx.x == 0) *lds_word = add_relaxed(ctr, 1u);
  __syncthreads();
  return uniform(*lds_word);
}

// XCD (accelerator die) the workgroup runs on: hardware register XCC_ID,
// bits 3:0.  Each XCD has its own L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (kXcds - 1);
}

// Tile order of a tiles_m x tiles_n grid.  map selects it:
//   kMapGlobal  one queue, m-major (every n-block of m-block 0, then 1, ...)
//   kMapBlocks  XCD x owns m-blocks [x tiles_m / 8, (x+1) tiles_m / 8)
//   kMapStrided XCD x owns m-blocks x, x + 8, x + 16, ...
//   kMapRounds  the m-blocks form groups of group_m (one round of the grid in
//               the global order, so round r still covers the same rows);
//               each group is cut into split_m x (8 / split_m) sub-blocks and
//               XCD x owns sub-block (x % split_m, x / split_m) of every
//               group, the groups in order
// With an XCD map, every owned m-block of n-block 0 comes first, then of
// n-block 1, ..., so the tiles one XCD runs at a time share a few A and B
// slabs in its L2 (the stride also spreads neighbouring m-blocks, which may
// cost alike, over the XCDs); a workgroup drains its own XCD's queue first,
// then the others in turn.
constexpr int kMapGlobal = 0, kMapBlocks = 1, kMapStrided = 2, kMapRounds = 3;
struct TileOrder {
  int map;
  int group_m;  // kMapRounds: m-blocks per group (>= 1)
  int split_m;  // kMapRounds: 1, 2, 4 or 8
};

// Next tile as mi * tiles_n + nb, or -1 when none is left (all threads get
// the value).
__device__ __forceinline__ int next_tile(const Sync &s, int tiles_m, int tiles_n, int xcd,
                                         TileOrder ord, uint32_t *lds_word) {
  const int map = ord.map;
  __syncthreads();
  if (threadIdx.x == 0) {
    int r = -1;
    if (map == kMapGlobal) {
      const uint32_t i = add_relaxed(&s.ctrl->xq[0], 1u);
      if (i < (uint32_t)(tiles_m * tiles_n)) r = (int)i;
    } else if (map == kMapRounds) {
      const int G = ord.group_m, am = ord.split_m, bx = kXcds / am;
      const int nfull = tiles_m / G, gl = tiles_m - nfull * G;  // gl: rows of the last, partial group
      for (int k = 0; k < kXcds && r < 0; ++k) {
        const int x = (xcd + k) & (kXcds - 1);
        const int xa = x % am, xb = x / am;
        const int n_lo = xb * tiles_n / bx, nc = (xb + 1) * tiles_n / bx - n_lo;
        const int m_lo = xa * G / am, mc = (xa + 1) * G / am - m_lo;
        const int ml_lo = xa * gl / am, mlc = (xa + 1) * gl / am - ml_lo;
        const uint32_t cf = (uint32_t)(mc * nc);
        const uint32_t size = (uint32_t)nfull * cf + (uint32_t)(mlc * nc);
        uint32_t *q = &s.ctrl->xq[x * 16];
        if (size == 0 || ld_relaxed(q) >= size) continue;
        const uint32_t i = add_relaxed(q, 1u);
        if (i < size) {
          int g, j, mcc, mlo;
          if (i < (uint32_t)nfull * cf) {
            g = (int)(i / cf); j = (int)(i % cf); mcc = mc; mlo = m_lo;
          } else {
            g = nfull; j = (int)(i - (uint32_t)nfull * cf); mcc = mlc; mlo = ml_lo;
          }
          r = (g * G + mlo + j % mcc) * tiles_n + n_lo + j / mcc;
        }
      }
    } else {
      for (int k = 0; k < kXcds && r < 0; ++k) {
        const int x = (xcd + k) & (kXcds - 1);
        int lo, mc;
        if (map == kMapBlocks) {
          lo = x * tiles_m / kXcds;
          mc = (x + 1) * tiles_m / kXcds - lo;
        } else {
          lo = x;
          mc = x < tiles_m ? (tiles_m - x + kXcds - 1) / kXcds : 0;
        }
        const uint32_t size = (uint32_t)(mc * tiles_n);
        uint32_t *q = &s.ctrl->xq[x * 16];
        if (size == 0 || ld_relaxed(q) >= size) continue;
        const uint32_t i = add_relaxed(q, 1u);
        if (i < size) {
          const int mi = (int)(i % (uint32_t)mc);
          r = (map == kMapBlocks ? lo + mi : x + kXcds * mi) * tiles_n + (int)(i / (uint32_t)mc);
        }
      }
    }
    *lds_word = (uint32_t)r;
  }
  __syncthreads();
  return (int)uniform(*lds_word);
}

// Every workgroup calls this once, last.  The final workgroup of the launch
// resets the launch-scoped counters for the next call on this handle; after
// an abort it also clears the arrival counters, which may be partial.
__device__ __forceinline__ void finish_launch(const Sync &s) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    uint32_t d = add_acq_rel(&s.ctrl->done, 1u);
    if (d + 1 == gridDim.x) {
      Ctrl *c = s.ctrl;
      st_relaxed(&c->ticket, 0u);
      st_relaxed(&c->tile_ctr, 0u);
      st_relaxed(&c->land_ctr, 0u);
      st_relaxed(&c->reduce_ctr, 0u);
      st_relaxed(&c->route_ctr, 0u);
      st_relaxed(&c->route_done, 0u);
      for (int x = 0; x < 8; ++x) st_relaxed(&c->xq[x * 16], 0u);
      st_relaxed(&c->tiles_done, 0u);
      st_relaxed(&c->combine_ctr, 0u);
      if (ld_relaxed(&c->abort_epoch) == s.epoch) {
        for (uint32_t i = 0; i < s.n_flags; ++i) st_relaxed(cnt_ptr(s, i), 0u);
      }
      st_relaxed(&c->done, 0u);
      __threadfence();
    }
  }
}

// Broadcast a wait result from thread 0 to the workgroup; on success every
// thread's later loads observe the data published before the flag.
//
// heavy_acquire = false skips the agent-scope acquire (an invalidate of this
// XCD's whole L2) and is used only for data that no workgroup of this launch
// can have cached before it was published: a landing buffer whose land
// blocks start and end on 128-byte cache-line boundaries and which is only
// read after its flags are seen.  Each launch starts with the caches
// invalidated, so no line of such a block can be in any L1/L2 before the
// block lands, and the writer's release already wrote it back to memory.
__device__ __forceinline__ bool wg_sync_ok(bool ok_thread0, uint32_t *lds_word,
                                           bool heavy_acquire = true) {
  __syncthreads();
  if (threadIdx.x == 0) {
    if (ok_thread0 && heavy_acquire) fence_acquire();
    *lds_word = ok_thread0 ? 1u : 0u;
  }
  __syncthreads();
  return uniform(*lds_word) != 0;
}

// Broadcast a flag value of thread 0 without any memory ordering.
__device__ __forceinline__ bool wg_broadcast(bool v_thread0, uint32_t *lds_word) {
  __syncthreads();
  if (threadIdx.x == 0) *lds_word = v_thread0 ? 1u : 0u;
  __syncthreads();
  return uniform(*lds_word) != 0;
}

// ---------------------------------------------------------------- data movement

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           (int)kRsrcWord3);
}

// Copy `bytes` (a multiple of 16) from src to dst with the whole workgroup,
// 16-byte vectors, several loads in flight per thread.
__device__ __forceinline__ void wg_copy16(void *__restrict__ dst, const void *__restrict__ src,
                                          size_t bytes) {
  const u32x4_t *s = reinterpret_cast<const u32x4_t *>(src);
  u32x4_t *d = reinterpret_cast<u32x4_t *>(dst);
  const size_t n = bytes >> 4;
  const size_t nt = blockDim.x;
  constexpr int U = 8;
  size_t i = threadIdx.x;
  for (; i + (size_t)(U - 1) * nt < n; i += (size_t)U * nt) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&s[i + (size_t)u * nt]);
#pragma unroll
    for (int u = 0; u < U; ++u) d[i + (size_t)u * nt] = v[u];
  }
  for (; i < n; i += nt) d[i] = __builtin_nontemporal_load(&s[i]);
}

// Copy a rows x row_bytes block (row_bytes a multiple of 16) between two
// matrices of row pitch pitch_bytes with the whole workgroup, 16-byte
// vectors.  Thread i moves the vectors at positions i, i + nt, i + 2 nt, ...
// of the block (nt threads, upr vectors per row).  When the rows are dense
// or nt is a multiple of upr, those vectors lie a fixed stride apart: the
// thread's offset stays in one register and the stride steps go in the
// buffer instructions' scalar offset.  Full batches of U move with the
// loads of batch b + 1 issued before the stores of batch b, so a thread
// always has loads in flight and never waits for its own stores.  Other
// shapes take a plain loop.  The block spans less than 2 GiB.
// U = 4 batches of 16-byte vectors per thread: deeper batches hold more
// registers in the out-of-line copy, and an 8-deep build placed a spilled
// descriptor's restore next to an LDS DMA of the fused kernels.  AUX: the
// stores' cache-policy bits (kStoreWriteThrough for landing copies).
template <int U = 4, int AUX = 0>
__device__ __forceinline__ void wg_copy2d(void *__restrict__ dst, const void *__restrict__ src,
                                          int rows, int row_bytes, size_t pitch_bytes) {
  const int nt = blockDim.x, tid = threadIdx.x;
  const int upr = row_bytes >> 4;
  const int n = rows * upr;
  const bool dense = (size_t)row_bytes == pitch_bytes;
  const uint32_t span = (uint32_t)((size_t)(rows - 1) * pitch_bytes + row_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, span), rd = make_rsrc(dst, span);
  if (!dense && nt % upr != 0) {
    for (int p = tid; p < n; p += nt) {
      const uint32_t o = (uint32_t)((size_t)(p / upr) * pitch_bytes + (size_t)(p % upr) * 16);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0), rd, o, 0, AUX);
    }
    return;
  }
  const uint32_t stride = (uint32_t)(dense ? (size_t)nt * 16 : (size_t)(nt / upr) * pitch_bytes);
  const uint32_t o0 = (uint32_t)(dense ? (size_t)tid * 16
                                       : (size_t)(tid / upr) * pitch_bytes + (size_t)(tid % upr) * 16);
  const int batches = (n / nt) / U;  // full batches every thread has
  u32x4_t v0[U], v1[U];
  auto load = [&](u32x4_t (&v)[U], int b) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, o0, (b * U + u) * stride, 0);
  };
  auto store = [&](const u32x4_t (&v)[U], int b) {
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, o0, (b * U + u) * stride, AUX);
  };
  if (batches > 0) {
    load(v0, 0);
    int b = 0;
    for (;;) {
      if (b + 1 >= batches) { store(v0, b); break; }
      load(v1, b + 1);
      store(v0, b);
      ++b;
      if (b + 1 >= batches) { store(v1, b); break; }
      load(v0, b + 1);
      store(v1, b);
      ++b;
    }
  }
  // the rest: fewer than U + 1 vectors per thread
  for (int p = tid + batches * U * nt, j = batches * U; p < n; p += nt, ++j) {
    const uint32_t so = j * stride;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_amdgcn_raw_buffer_load_b128(rs, o0, so, 0), rd, o0, so, AUX);
  }
}

// The same copy as an out-of-line call: a kernel that also runs the GEMM
// loop keeps the copy's registers out of the loop's allocation.  Arguments
// of a call arrive in vector registers; they are uniform, and reading them
// through readfirstlane says so (the buffer descriptors need scalars).
__device__ __forceinline__ const void *uniform_ptr(const void *p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo);
}
// Landing copies store with the system-coherence bits (sc0 sc1): the L2 of
// the writer's XCD writes them through to memory, so once a thread's stores
// are complete (vmcnt) they are visible to every XCD and the arrival needs
// no write-back of the L2 (see arrive_written_through).
constexpr int kStoreWriteThrough = 0x11;  // cache-policy bits sc0 | sc1

__device__ __attribute__((noinline)) void wg_copy2d_call(void *dst, const void *src, int rows,
                                                         int row_bytes, size_t pitch_bytes) {
  const uint64_t pb = reinterpret_cast<uint64_t>(uniform_ptr(reinterpret_cast<const void *>(pitch_bytes)));
  wg_copy2d<4, kStoreWriteThrough>(const_cast<void *>(uniform_ptr(dst)), uniform_ptr(src),
                                   __builtin_amdgcn_readfirstlane(rows),
                                   __builtin_amdgcn_readfirstlane(row_bytes), (size_t)pb);
}

// ---------------------------------------------------------------- GEMM tile engine
//
// C_tile[BM x BN] = A[m0:m0+BM, :] @ Bt[n0:n0+BN, :]^T with fp32 accumulation.
// Each wave owns a block of the tile built from E x E bf16 MFMA blocks
// (TileCfg: E = 16, 16x16x32 MFMAs, for the 8-wave 256-row tiles; E = 32,
// 32x32x16 MFMAs, for the 4-wave 128-row tiles).  The MFMA is issued with
// the B^T fragment as its first operand and the A fragment as its second, so
// the accumulator holds C^T blocks: lane l holds row (l % E) of its block and
// groups of four consecutive columns (acc_pos), which the epilogues store as
// 8-byte bf16 / 16-byte fp32 vectors.
//
// LDS layout of one operand stage: row r occupies 128 bytes (64 bf16 of K);
// its eight 16-byte chunks are stored at position p = c ^ ((r >> 1) & 7) for
// logical chunk c.  A fragment read serves 16 lanes (16 rows, 256 bytes) per
// LDS cycle; with a 128-byte row pitch, rows r and r+1 already fall in
// different halves of the 64 banks, and the (r >> 1) swizzle spreads the 8
// even (and the 8 odd) rows over distinct 16-byte bank groups, so the 16
// reads hit 16 distinct groups.  Stages are filled by buffer_load ... lds
// (16 bytes per lane, the lane's destination fixed at base + 16*lane); the
// swizzle is realised by choosing which global chunk each lane fetches.  Rows
// past the matrix or chunks past K use an out-of-range offset and read as
// zero.

template <int BM, int BN>
struct TileCfg {
  // 256-row tiles run 8 waves (2 per SIMD) in a 4 x 2 grid of 16x16x32
  // MFMA blocks: 64x64 per wave for 256x256 tiles, 64x112 for 256x224 (an N
  // of 7 x 512 splits into 2^k x 224 columns), whose B stage keeps 256 rows
  // of LDS, the last 32 filled with zeros.  (32x32x16 MFMAs in a 2 x 4 grid
  // of 128x64 blocks measured 5-8% slower for the 256x256 tiles.)  Smaller
  // tiles run 4 waves in a 2 x 2 grid of 32x32x16 MFMA blocks.
  static constexpr bool N224 = (BM == 256 && BN == 224);
  static constexpr bool M16 = (BM == 256);  // 16x16x32 MFMAs
  static constexpr int MFMA = M16 ? 16 : 32;                 // MFMA output edge
  static constexpr int SUBSTEPS = M16 ? 2 : 4;               // MFMA K steps per 64-wide stage
  static constexpr int GROUPS = M16 ? 1 : 4;                 // 4-column groups per accumulator
  using Acc = std::conditional_t<M16, f32x4_t, f32x16_t>;
  static constexpr int WAVES_M = M16 ? 4 : 2;
  static constexpr int WAVES_N = 2;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / MFMA, FN = WN / MFMA;
  static constexpr int BN_LDS = N224 ? 256 : BN;              // B rows held per stage
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN_LDS * 128;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int FLAG_SLOT = 2 * STAGE_BYTES;  // 256 bytes: a flag word fetched by DMA
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES + 256;
  static constexpr int LOADS_A = BM / (8 * WAVES);  // buffer loads per wave per stage
  static constexpr int LOADS_B = BN_LDS / (8 * WAVES);
  static constexpr int LOADS = LOADS_A + LOADS_B;
  static_assert(WM % MFMA == 0 && WN % MFMA == 0, "wave blocks are built from whole MFMAs");
  static_assert(BM % (8 * WAVES) == 0 && BN_LDS % (8 * WAVES) == 0, "stage rows split over waves");
};

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource (V#) as four SGPRs: base, stride 0, num_records, word3.
__device__ __forceinline__ i32x4_t make_vdesc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32) & 0xFFFF);
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  r[3] = (int32_t)kRsrcWord3;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// One 16-byte-per-lane global->LDS DMA: lane l's 16 bytes at buffer offset
// voff land at LDS byte address m0_base + 16*l.  Issued as inline assembly so
// the compiler does not treat every later LDS read as aliasing the DMA (it
// would wait for the prefetch before each read); completion is waited for
// explicitly with wait_vmcnt.
//
// The compiler's hazard checks do not look at the operands of inline
// assembly.  An LDS DMA needs 1 wait state after an SALU write of M0, which
// the asm's s_nop 0 provides.  A vector memory instruction that reads an
// SGPR written by a VALU instruction (for instance a descriptor reloaded from
// a spill with v_readlane) needs 5; the library's build is checked for that
// pattern instead (an s_nop 4 here slows the MFMA stream the DMAs are
// interleaved with).
// PAD: 5 wait states in front instead of 1, for DMAs outside the MFMA
// loop, where the compiler may restore a spilled descriptor SGPR with
// v_readlane right before the asm (a vector memory read of a VALU-written
// SGPR needs 5 wait states, and the compiler does not see asm operands).
template <bool PAD = false>
__device__ __forceinline__ void dma16(i32x4_t vdesc, uint32_t m0_base, uint32_t voff) {
  if constexpr (PAD)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(vdesc), "{m0}"(m0_base)
                 : "memory");
  else
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(vdesc), "{m0}"(m0_base)
                 : "memory");
}

// One 4-byte-per-lane global->LDS DMA (lane l's word lands at m0_base + 4 l).
// Issued once per K-slab, so it always carries the 5 wait states a
// descriptor restored from a spill would need.
__device__ __forceinline__ void dma4(i32x4_t vdesc, uint32_t m0_base, uint32_t voff) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(vdesc), "{m0}"(m0_base)
               : "memory");
}

template <int ROWS, int WAVES>
__device__ __forceinline__ void stage_operand(i32x4_t vdesc, uint32_t lds, int ld_bytes, int k0,
                                              int K, int wave, int lane) {
  constexpr int PER_WAVE = ROWS / (8 * WAVES);
  const int rsub = lane >> 3;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int j = wave * PER_WAVE + i;        // 8-row group filled by this instruction
    const int row = j * 8 + rsub;
    const int c = (lane & 7) ^ ((row >> 1) & 7);  // logical chunk stored at this lane's slot
    const int kk = k0 + c * 8;
    const uint32_t off = (kk < K) ? (uint32_t)(row * ld_bytes + kk * 2) : kOOB;
    dma16(vdesc, __builtin_amdgcn_readfirstlane(lds + j * 1024), off);
  }
}

// Workgroup barrier without the memory fence __syncthreads() implies: the
// fence would wait for every outstanding global load, including the
// prefetch of the next stage.  LDS reads before it are complete because
// their results feed MFMAs issued before it; LDS-DMA completion is waited
// for explicitly with wait_vmcnt.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt simm16 (gfx9): vmcnt[3:0], expcnt[6:4]=7, lgkmcnt[11:8]=15, vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One K-substep of fragments for a wave (16 K values for 32x32 MFMAs, 32
// for 16x16): FM A row-blocks and FN B^T row-blocks, one 16-byte LDS read
// each.  Lane l reads row l % MFMA of its block and 8 consecutive K values
// starting at 8 (l / MFMA) of the substep.
template <int BM, int BN>
struct Frags {
  bf16x8_t a[TileCfg<BM, BN>::FM];
  bf16x8_t b[TileCfg<BM, BN>::FN];
};

template <int BM, int BN>
__device__ __forceinline__ void load_frags(Frags<BM, BN> &f, const char *stage, int ks, int wm,
                                           int wn, int lane) {
  using C = TileCfg<BM, BN>;
  constexpr int E = C::MFMA;
  const int r = lane & (E - 1);
  const int c = ks * (64 / 8 / C::SUBSTEPS) + lane / E;  // logical 16-byte chunk of the 128-byte row
  // every block starts on a multiple of 16 rows, so the swizzle term of
  // row (block start + r) is (r >> 1) & 7 = (lane >> 1) & 7
  const int coff = ((c ^ ((lane >> 1) & 7)) << 4);
  const char *pa = stage + (wm * C::WM + r) * 128 + coff;
  const char *pb = stage + C::A_BYTES + (wn * C::WN + r) * 128 + coff;
  // issue order = first use in mma_frags (i outer, j inner): a[0] and every
  // b[j] are needed by the first FN MFMAs, a[i] only at MFMA i*FN
  f.a[0] = *reinterpret_cast<const bf16x8_t *>(pa);
#pragma unroll
  for (int j = 0; j < C::FN; ++j) f.b[j] = *reinterpret_cast<const bf16x8_t *>(pb + j * E * 128);
#pragma unroll
  for (int i = 1; i < C::FM; ++i) f.a[i] = *reinterpret_cast<const bf16x8_t *>(pa + i * E * 128);
}

// acc += B^T-block x A-block^T: the accumulator holds C^T blocks (see above).
template <int BM, int BN>
__device__ __forceinline__ typename TileCfg<BM, BN>::Acc mma(const bf16x8_t &b, const bf16x8_t &a,
                                                             const typename TileCfg<BM, BN>::Acc &acc) {
  if constexpr (TileCfg<BM, BN>::MFMA == 16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc, 0, 0, 0);
}

template <int BM, int BN>
using AccTile = typename TileCfg<BM, BN>::Acc[TileCfg<BM, BN>::FM][TileCfg<BM, BN>::FN];

template <int BM, int BN>
__device__ __forceinline__ void mma_frags(const Frags<BM, BN> &f, AccTile<BM, BN> &acc) {
  using C = TileCfg<BM, BN>;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = mma<BM, BN>(f.b[j], f.a[i], acc[i][j]);
}

// Interleave the next substep's LDS reads with this substep's MFMAs: one
// read, then MFMAs, repeated, so the reads' latency hides under the MFMAs.
template <int BM, int BN>
__device__ __forceinline__ void interleave_reads_and_mfmas() {
  using C = TileCfg<BM, BN>;
  constexpr int R = C::FM + C::FN, M = C::FM * C::FN;
  constexpr int per = M / R > 0 ? M / R : 1;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 DS read
    __builtin_amdgcn_sched_group_barrier(0x008, per, 0); // MFMAs
  }
  __builtin_amdgcn_sched_group_barrier(0x008, M - per * R > 0 ? M - per * R : 0, 0);
}

// Run the K loop of one tile with every wave doing both jobs (tiles of
// four waves, one per SIMD).  va covers rows [m0, m0 + valid_m) of A, vb
// rows [n0, n0 + valid_n) of Bt; both hold K-contiguous rows of pitch
// ld_bytes.  smem holds two stages.  On return the accumulators hold the
// tile and smem is free.
//
// Pipeline (per 64-wide K stage kb, 4 substeps of 16):
//   substeps 0..2: read the next substep's fragments, MFMAs of this one
//   then: wait for this wave's DMA of stage kb+1, barrier (every wave's DMA
//   landed; every wave's reads of stage kb done), start the DMA of stage
//   kb+2 into stage kb's buffer, read stage kb+1's first fragments, MFMAs of
//   substep 3.
// The fragment stream never drains and each DMA has a full stage of MFMAs
// to land.
template <int BM, int BN>
__device__ __forceinline__ void gemm_tile_interleaved(
    char *smem, i32x4_t va, i32x4_t vb, int ld_bytes, int K, AccTile<BM, BN> &acc) {
  using C = TileCfg<BM, BN>;
  static_assert(C::MFMA == 32, "substep pipeline of the 32x32 MFMA tiles");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16_t{};

  const uint32_t base = lds_addr(smem);
  const int nk = (K + kBK - 1) / kBK;
  stage_operand<BM, C::WAVES>(va, base, ld_bytes, 0, K, wave, lane);
  stage_operand<BN, C::WAVES>(vb, base + C::A_BYTES, ld_bytes, 0, K, wave, lane);
  if (nk > 1) {
    stage_operand<BM, C::WAVES>(va, base + C::STAGE_BYTES, ld_bytes, kBK, K, wave, lane);
    stage_operand<BN, C::WAVES>(vb, base + C::STAGE_BYTES + C::A_BYTES, ld_bytes, kBK, K, wave, lane);
    wait_vmcnt<C::LOADS>();
  } else {
    wait_vmcnt<0>();
  }
  wg_barrier();
  // f0 / f1 alternate so no fragment set is ever copied; at the loop head f0
  // holds substep 0 of stage kb.  The last stage's final read of the other
  // buffer is harmless (its data is not used).
  Frags<BM, BN> f0, f1;
  load_frags<BM, BN>(f0, smem, 0, wm, wn, lane);
  for (int kb = 0; kb < nk; ++kb) {
    const char *st = smem + (kb & 1) * C::STAGE_BYTES;
    load_frags<BM, BN>(f1, st, 1, wm, wn, lane);
    mma_frags<BM, BN>(f0, acc);
    interleave_reads_and_mfmas<BM, BN>();
    load_frags<BM, BN>(f0, st, 2, wm, wn, lane);
    mma_frags<BM, BN>(f1, acc);
    interleave_reads_and_mfmas<BM, BN>();
    load_frags<BM, BN>(f1, st, 3, wm, wn, lane);
    mma_frags<BM, BN>(f0, acc);
    interleave_reads_and_mfmas<BM, BN>();
    // every LDS read of stage kb has returned (substep 3's fragments are in
    // registers) and this wave's DMA of stage kb+1 has landed
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (0 << 8));  // vmcnt(0) lgkmcnt(0)
    wg_barrier();
    if (kb + 2 < nk) {
      const uint32_t dst = base + (kb & 1) * C::STAGE_BYTES;
      stage_operand<BM, C::WAVES>(va, dst, ld_bytes, (kb + 2) * kBK, K, wave, lane);
      stage_operand<BN, C::WAVES>(vb, dst + C::A_BYTES, ld_bytes, (kb + 2) * kBK, K, wave, lane);
    }
    load_frags<BM, BN>(f0, smem + ((kb + 1) & 1) * C::STAGE_BYTES, 0, wm, wn, lane);
    mma_frags<BM, BN>(f1, acc);
    interleave_reads_and_mfmas<BM, BN>();
  }
  wg_barrier();  // every wave is done reading; the caller may refill either stage
}

// Barrier that is also a scheduling fence: no instruction moves across it,
// so a phase's MFMAs stay between the barriers that delimit the phase.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Per-lane part of a stage DMA's buffer offset.  Instruction g fetches rows
// 8g .. 8g+7; lane l serves row 8g + (l >> 3), logical K chunk
// c = (l & 7) ^ ((row >> 1) & 7).  Since (row >> 1) & 7 = 4 (g & 1) + (l >> 4),
// c depends on g only through its parity, so two per-lane offsets cover
// every instruction; the row-group and K parts are uniform and added per
// instruction, which keeps no per-instruction value alive across the loop.
__device__ __forceinline__ int dma_chunk(int lane, int par) { return (lane & 7) ^ (par * 4 + (lane >> 4)); }

// One DMA instruction: row group g of an operand (buffer descriptor vdesc,
// row pitch ld_bytes), K values [k0, k0 + 64), into LDS at lds_rows (the
// operand's region of a stage plus 1024 g).  lane_off is the lane's offset
// for g's parity; chunks at or past K and rows past the descriptor's range
// read as zero.  k0 >= K fetches zeros only (no memory is touched).
__device__ __forceinline__ uint32_t dma_row_offset(uint32_t lane_off, int lane_c8, int ld_bytes, int k0, int K,
                                                   int g) {
  const uint32_t uni = (uint32_t)__builtin_amdgcn_readfirstlane(g * 8 * ld_bytes + k0 * 2);
  return lane_c8 < K - k0 ? lane_off + uni : kOOB;
}
template <bool PAD = false>
__device__ __forceinline__ void dma_row_group(i32x4_t vdesc, uint32_t lds_rows, uint32_t lane_off,
                                              int lane_c8, int ld_bytes, int k0, int K, int g) {
  dma16<PAD>(vdesc, __builtin_amdgcn_readfirstlane(lds_rows), dma_row_offset(lane_off, lane_c8, ld_bytes, k0, K, g));
}

// Gate of a tile whose A rows arrive during the K loop in K-slabs of
// `stages` stages, slab s being published by flag flag0 + s (an epoch-valued
// flag of `sync`).  Slab 0 has been waited for before the tile starts; the
// K loop checks each later slab before it fetches the slab's first A stage.
// stages == 0: nothing to check.
struct SlabGate {
  const Sync *sync;
  uint32_t flag0;
  int stages;
};

// K loop of the 8-wave 256x256 tile as two groups that take turns
// ("ping-pong").  Waves w and w + 4 share a SIMD; waves 0..3 (tile rows
// 0..127) form group 0, waves 4..7 (rows 128..255) group 1.  Every wave
// alternates a MEMORY phase (read all fragments of one 64-wide stage from
// LDS into registers) and a COMPUTE phase (the stage's 32 MFMAs, from
// registers only).  Group 1 runs one phase behind group 0, so in every
// phase one wave of each SIMD feeds the matrix core while its partner waits
// on LDS.  Workgroup barriers delimit the phases; barriers match by count,
// so the groups' extra barriers at the start and the end pair up.
//
//   phase 2t   : group 0 MEMORY(t)   group 1 COMPUTE(t-1)
//   phase 2t+1 : group 0 COMPUTE(t)  group 1 MEMORY(t)
//
// Refills are spread over every phase, 4 DMA instructions per wave each,
// because issuing a whole stage at once stalls the issuing wave for as long
// as the address unit takes to accept it.  Wave (group q, index i) owns row
// groups 16 q + 4 i .. +3 (8 rows each) of both operands and fetches them
// for every stage: its "own" operand (A for group 0, whose rows it alone
// reads; B for group 1) in COMPUTE(t) for stage t+2, the other one in
// MEMORY(t) for stage t+1.  Stage s lives in buffer s & 1.
//   phase 2t   G0 MEMORY(t):  B rows 0..127, stage t+1.  The buffer's last
//                             reads were in phases 2t-2 and 2t-1.
//   phase 2t   G1 COMPUTE(t-1): B rows 128..255, stage t+1.  Same buffer.
//   phase 2t+1 G0 COMPUTE(t): A rows 0..127, stage t+2.  Last read by G0 in
//                             phase 2t.
//   phase 2t+1 G1 MEMORY(t):  A rows 128..255, stage t+1.  Last read by G1
//                             in phase 2t-1.
// Every stage-t+1 part is read from phase 2t+2 on (A rows 128..255 from
// 2t+3), and its issuer waits for it before the barrier that opens that
// phase: G0 at the end of COMPUTE(t) (B; A top of t+1 was issued a phase
// earlier still), G1 at the end of MEMORY(t) (B) and of COMPUTE(t) (A).
// Each such wait is vmcnt(4): only the 4 instructions issued since may be
// in flight.  Refills of stages past the last are zero fills (offset out of
// range) of buffers nothing reads again, so the counts are the same in
// every iteration; they are drained at the end.
template <int BM, int BN>
__device__ __forceinline__ void gemm_tile_pingpong(
    char *smem, i32x4_t va, i32x4_t vb, int ld_bytes, int K, AccTile<BM, BN> &acc,
    const SlabGate &gate) {
  using C = TileCfg<BM, BN>;
  constexpr int G = 4;                                // waves per group
  static_assert(BM == 256 && C::WAVES == 2 * G && (G / C::WAVES_N) * C::WM == BM / 2,
                "two groups of four waves, one group per half of the A rows");
  constexpr int R = 4;                                // row groups per wave and operand
  constexpr int MFMAS = C::SUBSTEPS * C::FM * C::FN;  // per stage (32 or 56)
  constexpr int DMA_EVERY = MFMAS / R;                // MFMAs between refill instructions
  static_assert(BM / 8 == 2 * G * R && C::BN_LDS / 8 == 2 * G * R, "row groups per wave");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int group = wave / G;
  const bool g0 = group == 0;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = typename C::Acc{};

  const uint32_t base = lds_addr(smem);
  const int nk = (K + kBK - 1) / kBK;
  const int ld = ld_bytes;
  const int rg = wave * R;   // first owned row group (= 16 group + 4 index)
  const uint32_t lane_off[2] = {(uint32_t)((lane >> 3) * ld + dma_chunk(lane, 0) * 16),
                                (uint32_t)((lane >> 3) * ld + dma_chunk(lane, 1) * 16)};
  const int lane_c8[2] = {dma_chunk(lane, 0) * 8, dma_chunk(lane, 1) * 8};
  // own operand (fetched in COMPUTE) and other operand (fetched in MEMORY)
  const i32x4_t v_own = g0 ? va : vb, v_oth = g0 ? vb : va;
  const uint32_t lds_own = base + (g0 ? 0u : (uint32_t)C::A_BYTES) + rg * 1024;
  const uint32_t lds_oth = base + (g0 ? (uint32_t)C::A_BYTES : 0u) + rg * 1024;
  auto fetch = [&](bool own, int stage, int d) {
    dma_row_group(own ? v_own : v_oth,
                  (own ? lds_own : lds_oth) + (stage & 1) * C::STAGE_BYTES + d * 1024,
                  lane_off[d & 1], lane_c8[d & 1], ld, stage * kBK, K, rg + d);
  };
  // the own operand's offsets for stage t+2 are computed in MEMORY(t), which
  // has time to spare, so COMPUTE(t) issues its refills without address
  // arithmetic between the MFMAs
  auto own_offset = [&](int stage, int d) {
    return dma_row_offset(lane_off[d & 1], lane_c8[d & 1], ld, stage * kBK, K, rg + d);
  };
  auto fetch_own = [&](int stage, int d, uint32_t off) {
    dma16(v_own, __builtin_amdgcn_readfirstlane(lds_own + (stage & 1) * C::STAGE_BYTES + d * 1024), off);
  };
  auto fetch_padded = [&](bool own, int stage, int d) {  // prologue: see dma16
    dma_row_group<true>(own ? v_own : v_oth,
                        (own ? lds_own : lds_oth) + (stage & 1) * C::STAGE_BYTES + d * 1024,
                        lane_off[d & 1], lane_c8[d & 1], ld, stage * kBK, K, rg + d);
  };
  // slab gate: wave 0 fetches the flag of the slab starting at stage u into
  // an LDS slot in MEMORY(u-3) (completed by its wait at the end of
  // COMPUTE(u-3)) and reads it in MEMORY(u-2), before the barrier after
  // which A rows of stage u are first fetched (group 0, COMPUTE(u-2)); if
  // the flag is not yet set there it waits for it.  Slabs span at least
  // four stages, so the slot is never refilled before it is read.
  // (gate values are uniform; readfirstlane keeps them scalar even when the
  // caller read them from memory into vector registers)
  const int S = __builtin_amdgcn_readfirstlane(gate.stages);  // 0: no gate
  const uint32_t flag0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)gate.flag0);
  const bool gated = S > 0 && wave == 0;
  i32x4_t fdesc{};
  uint32_t epoch = 0;
  if (gated) {
    fdesc = make_vdesc(gate.sync->flags, gate.sync->n_flags * kFlagStride * 4u);
    epoch = (uint32_t)__builtin_amdgcn_readfirstlane((int)gate.sync->epoch);
  }
  // prologue, in the order the loop's waits expect: own 0, other 0, own 1
#pragma unroll
  for (int d = 0; d < R; ++d) fetch_padded(true, 0, d);
#pragma unroll
  for (int d = 0; d < R; ++d) fetch_padded(false, 0, d);
#pragma unroll
  for (int d = 0; d < R; ++d) fetch_padded(true, 1, d);
  wait_vmcnt<R>();                    // stage 0 landed
  phase_barrier();
  if (!g0) phase_barrier();           // group 1 starts one phase late
  Frags<BM, BN> f[C::SUBSTEPS];
  int chk_t = S - 2, pf_t = S - 3;  // first stages t with (t + 2) % S == 0, (t + 3) % S == 0
  uint32_t chk_slab = 1, pf_slab = 1;
  for (int t = 0; t < nk; ++t) {
    // MEMORY(t): fragments of stage t, then the other operand of stage t+1
    const char *st = smem + (t & 1) * C::STAGE_BYTES;
#pragma unroll
    for (int ks = 0; ks < C::SUBSTEPS; ++ks) load_frags<BM, BN>(f[ks], st, ks, wm, wn, lane);
#pragma unroll
    for (int d = 0; d < R; ++d) fetch(false, t + 1, d);
    uint32_t own_off[R];
#pragma unroll
    for (int d = 0; d < R; ++d) own_off[d] = own_offset(t + 2, d);
    if (gated) {
      // stage t + 2 starts slab chk_slab when t == chk_t; stage t + 3 starts
      // slab pf_slab when t == pf_t (counters, not a division per stage)
      if (t == chk_t) {
        chk_t += S;
        if (t + 2 < nk) {
          const uint32_t seen = uniform(*reinterpret_cast<volatile uint32_t *>(smem + C::FLAG_SLOT));
          if (seen != epoch && lane == 0) {
            // on timeout or abort the error is recorded; the tile completes
            // with undefined values and the caller stops at its next wait
            (void)spin_until_eq(*gate.sync, flag_ptr(*gate.sync, flag0 + chk_slab), epoch,
                                0x51000000u | (flag0 + chk_slab));
          }
        }
        ++chk_slab;
      }
      if (t == pf_t) {
        pf_t += S;
        if (t + 3 < nk)
          dma4(fdesc, __builtin_amdgcn_readfirstlane(lds_addr(smem + C::FLAG_SLOT)),
               (flag0 + pf_slab) * kFlagStride * 4u);
        ++pf_slab;
      }
    }
    if (g0)
      __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    else  // B rows 128..255 of stage t+1
      __builtin_amdgcn_s_waitcnt(R | (7 << 4) | (0 << 8));               // vmcnt(4) lgkmcnt(0)
    phase_barrier();
    // COMPUTE(t): MFMAs from registers; the own operand of stage t+2
    // between them
#pragma unroll
    for (int m = 0; m < MFMAS; ++m) {
      const int ks = m / (C::FM * C::FN), i = (m / C::FN) % C::FM, j = m % C::FN;
      acc[i][j] = mma<BM, BN>(f[ks].b[j], f[ks].a[i], acc[i][j]);
      if (m % DMA_EVERY == 0 && m / DMA_EVERY < R) fetch_own(t + 2, m / DMA_EVERY, own_off[m / DMA_EVERY]);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<R>();  // G0: B rows 0..127 and A rows 0..127 of t+1; G1: A rows 128..255 of t+1
    phase_barrier();
  }
  if (g0) phase_barrier();            // pairs with group 1's last barrier
  wait_vmcnt<0>();                    // the zero fills past the last stage
  wg_barrier();  // every wave is done reading; the caller may refill either stage
}

// A tile's K loop over K-contiguous operand rows of pitch ld_bytes (A and
// Bt both hold K bf16 values per row).  gate applies to the 8-wave tile
// only; a caller using the 4-wave tile waits for all of its A rows before
// calling.
template <int BM, int BN>
__device__ __forceinline__ void gemm_tile(char *smem, i32x4_t va, i32x4_t vb, int ld_bytes, int K,
                                          AccTile<BM, BN> &acc,
                                          const SlabGate &gate = SlabGate{nullptr, 0u, 0}) {
  if constexpr (TileCfg<BM, BN>::WAVES == 8)
    gemm_tile_pingpong<BM, BN>(smem, va, vb, ld_bytes, K, acc, gate);
  else
    gemm_tile_interleaved<BM, BN>(smem, va, vb, ld_bytes, K, acc);
}

// Position of accumulator group g (4 consecutive columns) of block (i, j).
template <int BM, int BN>
struct AccPos {
  int row;  // row within the tile
  int col;  // first of 4 columns within the tile
};

template <int BM, int BN>
__device__ __forceinline__ AccPos<BM, BN> acc_pos(int i, int j, int g) {
  using C = TileCfg<BM, BN>;
  constexpr int E = C::MFMA;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  AccPos<BM, BN> p;
  p.row = wm * C::WM + i * E + (lane & (E - 1));
  p.col = wn * C::WN + j * E + g * 8 + (lane / E) * 4;
  return p;
}

// The 4 values of accumulator group g (the columns acc_pos gives).
template <class A>
__device__ __forceinline__ f32x4_t acc_group(const A &v, int g) {
  return f32x4_t{v[g * 4 + 0], v[g * 4 + 1], v[g * 4 + 2], v[g * 4 + 3]};
}

// Epilogue through LDS.  Block b holds accumulator row-block b of every
// wave: E = MFMA rows (32 or 16) from each of the WAVES_M wave rows,
// EpiCfg::ROWS in all (LDS row E u + l is tile row u WM + E b + l).  Every
// thread then takes 4 consecutive columns of an LDS row, so each wave
// instruction covers whole rows (1 KiB of fp32 for BN = 256) and the
// epilogue's global loads and stores are fully contiguous.  Indexing blocks
// by the accumulator index keeps every LDS write at one per-lane base plus
// an immediate offset and lets each block's accumulators die once written,
// so nothing is spilled.  LDS rows are padded by 16 bytes so the rows one
// accumulator write spans fall in distinct bank groups.  f(row, col, v) is
// called for every 4-column group (row, col relative to the tile) of the
// tile, each exactly once.
template <int BM, int BN>
struct EpiCfg {
  using C = TileCfg<BM, BN>;
  static constexpr int ROWS = C::WAVES_M * C::MFMA;  // LDS rows per block
  static constexpr int PITCH = BN * 4 + 16;
  static constexpr int CHUNKS = ROWS * (BN / 4);
};

// Accumulator row-block b of this wave into the LDS block at wp (the
// lane's position, set up by the staged epilogues).
template <int BM, int BN>
__device__ __forceinline__ void epi_write_block(const AccTile<BM, BN> &acc, int b, char *wp) {
  using C = TileCfg<BM, BN>;
#pragma unroll
  for (int j = 0; j < C::FN; ++j)
#pragma unroll
    for (int g = 0; g < C::GROUPS; ++g)
      *reinterpret_cast<f32x4_t *>(wp + (j * C::MFMA + g * 8) * 4) = acc_group(acc[b][j], g);
}

template <int BM, int BN>
__device__ __forceinline__ char *epi_lane_pos(char *smem) {
  using C = TileCfg<BM, BN>;
  using E = EpiCfg<BM, BN>;
  static_assert(E::ROWS * E::PITCH <= 2 * C::STAGE_BYTES, "epilogue block must fit the LDS stages");
  static_assert(E::CHUNKS % C::THREADS == 0, "chunks split evenly over threads");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  // the lane's accumulator row and first column (see acc_pos)
  return smem + (wm * C::MFMA + (lane & (C::MFMA - 1))) * E::PITCH +
         (wn * C::WN + (lane / C::MFMA) * 4) * 4;
}

template <int BM, int BN, class F>
__device__ __forceinline__ void staged_epilogue(const AccTile<BM, BN> &acc, char *smem, F &&f) {
  using C = TileCfg<BM, BN>;
  using E = EpiCfg<BM, BN>;
  char *wp = epi_lane_pos<BM, BN>(smem);
#pragma unroll
  for (int b = 0; b < C::FM; ++b) {
    wg_barrier();  // the previous block's reads (or the K loop's) are done
    epi_write_block<BM, BN>(acc, b, wp);
    wg_barrier();
    // kept rolled: f is inlined once per block, so the epilogue stays small
    // enough for the instruction cache
#pragma unroll 1
    for (int k = 0; k < E::CHUNKS / C::THREADS; ++k) {
      const int idx = (int)threadIdx.x + k * C::THREADS;
      const int rr = idx / (BN / 4), c4 = idx % (BN / 4);
      const f32x4_t v = *reinterpret_cast<const f32x4_t *>(smem + rr * E::PITCH + c4 * 16);
      f((rr / C::MFMA) * C::WM + b * C::MFMA + rr % C::MFMA, c4 * 4, v);
    }
  }
  wg_barrier();  // LDS is free again for the next tile's stages
}

// The staged epilogue for epilogues that read global memory per 4-column
// group: pre(row, col) issues those loads and returns their registers,
// f(row, col, v, loaded) finishes the group.  The loads of the next group
// are issued before the current group's stores: on gfx9 a wait for a load
// also waits for every store issued before it, so loading after storing
// would cost one memory round trip per group.
template <int BM, int BN, class Pre, class F>
__device__ __forceinline__ void staged_epilogue_pf(const AccTile<BM, BN> &acc, char *smem, Pre &&pre,
                                                   F &&f) {
  using C = TileCfg<BM, BN>;
  using E = EpiCfg<BM, BN>;
  constexpr int NK = E::CHUNKS / C::THREADS;
  static_assert(NK % 2 == 0, "column groups are taken in pairs");
  static_assert(C::THREADS % (BN / 4) == 0, "a thread keeps one column group");
  char *wp = epi_lane_pos<BM, BN>(smem);
  // THREADS is a multiple of BN / 4: a thread keeps its column group
  const int c4 = (int)threadIdx.x % (BN / 4);
  const int rr0 = (int)threadIdx.x / (BN / 4);
  constexpr int RSTEP = C::THREADS / (BN / 4);
#pragma unroll
  for (int b = 0; b < C::FM; ++b) {
    wg_barrier();
    epi_write_block<BM, BN>(acc, b, wp);
    wg_barrier();
    auto row_of = [&](int rr) { return (rr / C::MFMA) * C::WM + b * C::MFMA + rr % C::MFMA; };
    auto lds_val = [&](int rr) { return *reinterpret_cast<const f32x4_t *>(smem + rr * E::PITCH + c4 * 16); };
    // two register sets in turn, never copied (a copy of registers a load
    // is still filling waits for that load); the prefetch past the block's
    // last group asks for rows past the tile, which pre() does not load
    auto ra = pre(row_of(rr0), c4 * 4);
#pragma unroll 1
    for (int k = 0; k < NK; k += 2) {
      const int rr = rr0 + k * RSTEP;
      auto rb = pre(row_of(rr + RSTEP), c4 * 4);
      f(row_of(rr), c4 * 4, lds_val(rr), ra);
      ra = pre(k + 2 < NK ? row_of(rr + 2 * RSTEP) : BM, c4 * 4);
      f(row_of(rr + RSTEP), c4 * 4, lds_val(rr + RSTEP), rb);
    }
  }
  wg_barrier();
}

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  bf16x4_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  v[2] = (__bf16)c;
  v[3] = (__bf16)d;
  return *reinterpret_cast<uint2 *>(&v);
}

}  // namespace mk

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

constexpr int kThreads = 256;     // 4 waves of 64 lanes
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

// Arrival of one work item of flag `f`, which completes after `target` items.
// Called by one thread after the whole workgroup's stores are fenced and
// barriered.  The last arrival resets the counter and publishes the flag.
__device__ __forceinline__ void arrive(const Sync &s, uint32_t f, uint32_t target) {
  uint32_t old = add_acq_rel(cnt_ptr(s, f), 1u);
  if (old + 1 == target) {
    st_relaxed(cnt_ptr(s, f), 0u);
    st_release(flag_ptr(s, f), s.epoch);
  }
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

// Fetch the next index from a device counter (all threads get the value).
__device__ __forceinline__ uint32_t next_index(uint32_t *ctr, uint32_t *lds_word) {
  __syncthreads();
  if (threadIdx.x == 0) *lds_word = add_relaxed(ctr, 1u);
  __syncthreads();
  return uniform(*lds_word);
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
__device__ __forceinline__ bool wg_sync_ok(bool ok_thread0, uint32_t *lds_word) {
  __syncthreads();
  if (threadIdx.x == 0) {
    if (ok_thread0) fence_acquire();
    *lds_word = ok_thread0 ? 1u : 0u;
  }
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
  constexpr int U = 8;
  size_t i = threadIdx.x;
  for (; i + (size_t)(U - 1) * kThreads < n; i += (size_t)U * kThreads) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&s[i + (size_t)u * kThreads]);
#pragma unroll
    for (int u = 0; u < U; ++u) d[i + (size_t)u * kThreads] = v[u];
  }
  for (; i < n; i += kThreads) d[i] = __builtin_nontemporal_load(&s[i]);
}

// ---------------------------------------------------------------- GEMM tile engine
//
// C_tile[BM x BN] = A[m0:m0+BM, :] @ Bt[n0:n0+BN, :]^T with fp32 accumulation.
// 4 waves in a 2 x 2 grid; each wave owns a (BM/2) x (BN/2) block built from
// 32x32x16 bf16 MFMAs.  The MFMA is issued with the B^T fragment as its first
// operand and the A fragment as its second, so the accumulator holds C^T
// blocks: lane l holds row (l % 32) of its 32x32 block and, for v = 0..15,
// column 8*(v/4) + 4*(l/32) + v%4 -- four consecutive columns per group,
// which the epilogues store as 8-byte bf16 / 16-byte fp32 vectors.
//
// LDS layout of one operand stage: row r occupies 128 bytes (64 bf16 of K);
// its eight 16-byte chunks are stored at position p = c ^ (r & 7) for logical
// chunk c, so the 32 rows read by one MFMA fragment load hit distinct banks.
// Stages are filled by buffer_load ... lds (16 bytes per lane, the lane's
// destination fixed at base + 16*lane); the swizzle is realised by choosing
// which global chunk each lane fetches.  Rows past the matrix or chunks past
// K use an out-of-range offset and read as zero.

template <int BM, int BN>
struct TileCfg {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int LOADS_A = BM / 32;  // buffer loads per wave per stage
  static constexpr int LOADS_B = BN / 32;
  static constexpr int LOADS = LOADS_A + LOADS_B;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile must split into 2x2 waves of 32x32 blocks");
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
__device__ __forceinline__ void dma16(i32x4_t vdesc, uint32_t m0_base, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(vdesc), "{m0}"(m0_base)
               : "memory");
}

template <int ROWS>
__device__ __forceinline__ void stage_operand(i32x4_t vdesc, uint32_t lds, int ld_bytes, int k0,
                                              int K, int wave, int lane) {
  constexpr int PER_WAVE = ROWS / 32;
  const int rsub = lane >> 3;
  const int c = (lane & 7) ^ rsub;
  const int kk = k0 + c * 8;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int j = wave * PER_WAVE + i;        // 8-row group filled by this instruction
    const int row = j * 8 + rsub;
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

template <int BM, int BN>
__device__ __forceinline__ void mma_stage(const char *ldsA, const char *ldsB,
                                          f32x16_t (&acc)[TileCfg<BM, BN>::FM][TileCfg<BM, BN>::FN],
                                          int wm, int wn, int lane) {
  using C = TileCfg<BM, BN>;
  const int r32 = lane & 31;
  const int sw = lane & 7;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c = ks * 2 + (lane >> 5);
    const int coff = ((c ^ sw) << 4);
    bf16x8_t a[C::FM], b[C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
      a[i] = *reinterpret_cast<const bf16x8_t *>(ldsA + (wm * C::WM + i * 32 + r32) * 128 + coff);
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      b[j] = *reinterpret_cast<const bf16x8_t *>(ldsB + (wn * C::WN + j * 32 + r32) * 128 + coff);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
  }
}

// Run the K loop of one tile.  va covers rows [m0, m0 + valid_m) of A with
// row pitch lda_bytes; vb rows [n0, n0 + valid_n) of Bt.  smem holds two
// stages.  On return the accumulators hold the tile and smem is free.
template <int BM, int BN>
__device__ __forceinline__ void gemm_tile(char *smem, i32x4_t va, int lda_bytes, i32x4_t vb,
                                          int ldb_bytes, int K,
                                          f32x16_t (&acc)[TileCfg<BM, BN>::FM][TileCfg<BM, BN>::FN]) {
  using C = TileCfg<BM, BN>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16_t{};

  const uint32_t base = lds_addr(smem);
  const int nk = (K + kBK - 1) / kBK;
  stage_operand<BM>(va, base, lda_bytes, 0, K, wave, lane);
  stage_operand<BN>(vb, base + C::A_BYTES, ldb_bytes, 0, K, wave, lane);
  for (int kb = 0; kb < nk; ++kb) {
    // This wave's loads of stage kb are done; after the barrier every wave's
    // are, and every wave has finished reading the other stage's buffer,
    // which the prefetch of stage kb+1 overwrites.
    wait_vmcnt<0>();
    wg_barrier();
    if (kb + 1 < nk) {
      const uint32_t nxt = base + ((kb + 1) & 1) * C::STAGE_BYTES;
      stage_operand<BM>(va, nxt, lda_bytes, (kb + 1) * kBK, K, wave, lane);
      stage_operand<BN>(vb, nxt + C::A_BYTES, ldb_bytes, (kb + 1) * kBK, K, wave, lane);
    }
    const char *cur = smem + (kb & 1) * C::STAGE_BYTES;
    mma_stage<BM, BN>(cur, cur + C::A_BYTES, acc, wm, wn, lane);
  }
  wg_barrier();  // every wave is done reading; the caller may refill either stage
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
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  AccPos<BM, BN> p;
  p.row = wm * C::WM + i * 32 + (lane & 31);
  p.col = wn * C::WN + j * 32 + g * 8 + (lane >> 5) * 4;
  return p;
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

// Persistent fused kernels: AllGather+GEMM, GEMM+ReduceScatter, GEMM+AllReduce.
//
// [P1] German article on mKernel (chatgpz.de), table "Die fuenf
// verschmolzenen Kerne": AllGather + GEMM (the local GEMM consumes tiles of
// the peers' shards as they arrive), GEMM + AllReduce (output tiles enter the
// reduction the moment they are produced) and GEMM + ReduceScatter (each
// output tile is reduced and forwarded to its owning rank as soon as it is
// produced).  Section "Was mKernel macht": one persistent kernel whose CTAs
// assign themselves roles, with tunable counts per role.
//
// One launch = one call.  Every workgroup takes a ticket; tickets
// [0, n_land) land chunks, the next n_compute run GEMM tiles.  Land
// workgroups take tickets first, so every flag a compute workgroup waits on
// is owned by a workgroup that is already running.
#include "mk_params.h"

namespace mk {

// 4 bf16 values (8 bytes) stored with a non-temporal hint: outputs the
// kernel never reads again.
__device__ __forceinline__ void store_nt(uint16_t *dst, const uint2 &o) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(u32x2_t{o.x, o.y}, reinterpret_cast<u32x2_t *>(dst));
}

// ---------------------------------------------------------------- AllGather + GEMM

__device__ __forceinline__ uint32_t ag_flag(const AgParams &p, int q, int j, int s) {
  return (uint32_t)((q * p.blocks_per_chunk + j) * p.n_slabs + s);
}

// Where land item `it` (numbering in AgParams) lives: shard q, land block j,
// slab s; rows [r0, r1) of the shard, columns [c0, c1).
struct AgItem {
  int q, j, s, r0, r1, c0, c1;
  int per_block;  // items per land block (and slab) of this item's shard: its flag's arrivals
};

__device__ __forceinline__ AgItem ag_item(const AgParams &p, uint32_t it) {
  int q, s, item_rows;
  uint32_t rem, per_block;
  if (it < (uint32_t)p.n_peer_items) {
    // two groups of peers in landing order, each slab-major: the first
    // first_peers peers (items of item_rows_first rows), then the others
    const bool first = it < (uint32_t)p.n_first_items;
    per_block = (uint32_t)(first ? p.items_per_block_first : p.items_per_block);
    item_rows = first ? p.item_rows_first : p.item_rows;
    const uint32_t per_chunk_slab = (uint32_t)p.blocks_per_chunk * per_block;
    const int pos0 = first ? 0 : p.first_peers;
    const uint32_t np = (uint32_t)(first ? p.first_peers : p.world - 1 - p.first_peers);
    const uint32_t ig = first ? it : it - (uint32_t)p.n_first_items;
    const uint32_t per_slab = np * per_chunk_slab;
    s = (int)(ig / per_slab);
    rem = ig % per_slab;
    q = (p.rank + 1 + pos0 + (int)(rem / per_chunk_slab)) % p.world;
    rem %= per_chunk_slab;
  } else {
    per_block = (uint32_t)p.items_per_block;
    item_rows = p.item_rows;
    const uint32_t per_chunk_slab = (uint32_t)p.blocks_per_chunk * per_block;
    const uint32_t il = it - (uint32_t)p.n_peer_items;
    s = (int)(il / per_chunk_slab);
    rem = il % per_chunk_slab;
    q = p.rank;
  }
  AgItem r;
  r.q = q;
  r.s = s;
  r.per_block = (int)per_block;
  r.j = (int)(rem / per_block);
  const int ii = (int)(rem % per_block);
  r.r0 = r.j * p.lb_rows + ii * item_rows;
  r.r1 = min(r.r0 + item_rows, min((r.j + 1) * p.lb_rows, p.m_s));
  r.c0 = s * p.slab_k;
  r.c1 = min(r.c0 + p.slab_k, p.k);
  return r;
}

// Land item `it`.  Peers land in the order rank+1, rank+2, ...; every thread
// copies its share, waits for its stores, and thread 0 records the arrival
// after the barrier.
__device__ __forceinline__ void ag_land_item(const AgParams &p, uint32_t it) {
  const AgItem g = ag_item(p, it);
  if (g.r1 > g.r0)
    wg_copy2d_call(p.ag + ((size_t)g.q * p.m_s + g.r0) * p.k + g.c0, p.shard[g.q] + (size_t)g.r0 * p.k + g.c0,
                   g.r1 - g.r0, (g.c1 - g.c0) * 2, (size_t)p.k * 2);
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) arrive_written_through(p.sync, ag_flag(p, g.q, g.j, g.s), (uint32_t)g.per_block);
}

__device__ __forceinline__ void ag_land(const AgParams &p, uint32_t *s_word) {
  for (;;) {
    const uint32_t it = next_index(&p.sync.ctrl->land_ctr, s_word);
    if (it >= (uint32_t)p.n_items) break;
    ag_land_item(p, it);
  }
}

// Thread 0: are slabs [s0, s1) of all land blocks overlapping gathered rows
// [m0, m1) ready?
__device__ __forceinline__ bool ag_rows_ready(const AgParams &p, int m0, int m1, int s0, int s1) {
  int r = m0;
  while (r < m1) {
    const int q = r / p.m_s, lr = r - q * p.m_s;
    const int j = lr / p.lb_rows;
    for (int s = s0; s < s1; ++s)
      if (ld_relaxed(flag_ptr(p.sync, ag_flag(p, q, j, s))) != p.sync.epoch) return false;
    r = q * p.m_s + min((j + 1) * p.lb_rows, p.m_s);
  }
  return true;
}

// Thread 0: wait for slabs [s0, s1) of every land block overlapping
// gathered rows [m0, m1).
__device__ __forceinline__ bool ag_wait_rows(const AgParams &p, int m0, int m1, int s0, int s1) {
  int r = m0;
  while (r < m1) {
    const int q = r / p.m_s, lr = r - q * p.m_s;
    const int j = lr / p.lb_rows;
    for (int s = s0; s < s1; ++s)
      if (!spin_until_eq(p.sync, flag_ptr(p.sync, ag_flag(p, q, j, s)), p.sync.epoch,
                         (uint32_t)((q << 16) | (j << 8) | s)))
        return false;
    r = q * p.m_s + min((j + 1) * p.lb_rows, p.m_s);
  }
  return true;
}

// Make slabs [s0, s1) of gathered rows [m0, m1) available to the workgroup.
// While they are missing, the workgroup lands the next unlanded items
// itself (slab-major landing order matches what tiles need first); once
// nothing is left to land it waits.  Returns false on timeout / abort.
__device__ __forceinline__ bool ag_acquire_rows(const AgParams &p, int m0, int m1, int s0, int s1,
                                                bool helper, uint32_t *s_word) {
  for (;;) {
    // the barrier closes the previous item's single-thread arrival (see uniform())
    __syncthreads();
    bool ready = false;
    if (threadIdx.x == 0) ready = ag_rows_ready(p, m0, m1, s0, s1);
    if (wg_broadcast(ready, s_word)) break;
    if (!helper) break;
    const uint32_t it = next_index(&p.sync.ctrl->land_ctr, s_word);
    if (it >= (uint32_t)p.n_items) break;
    ag_land_item(p, it);
    if (p.help_eager) {  // keep landing while items below eager_items are unclaimed
      for (;;) {
        __syncthreads();
        bool more = false;
        if (threadIdx.x == 0) more = ld_relaxed(&p.sync.ctrl->land_ctr) < (uint32_t)p.eager_items;
        if (!wg_broadcast(more, s_word)) break;
        const uint32_t jt = next_index(&p.sync.ctrl->land_ctr, s_word);
        if (jt >= (uint32_t)p.n_items) break;
        ag_land_item(p, jt);
      }
      break;
    }
  }
  bool ok0 = true;
  if (threadIdx.x == 0) ok0 = ag_wait_rows(p, m0, m1, s0, s1);
  return wg_sync_ok(ok0, s_word, !p.light_acquire);
}

template <int BM, int BN, bool PRE>
__device__ __forceinline__ void ag_compute(const AgParams &p, char *smem, uint32_t *s_word,
                                           uint32_t ticket) {
  // compute workgroups that land items while their rows are missing
  const bool helper = p.help_land && ticket % (uint32_t)p.help_every == 0;
  using C = TileCfg<BM, BN>;
  const int xcd = xcd_id();
  const int M = p.world * p.m_s;
  const int loc0 = p.rank * p.m_s, loc1 = loc0 + p.m_s;
  const int ldb = p.k * 2;
  for (;;) {
    const int t = next_tile(p.sync, p.tiles_m, p.tiles_n, xcd, TileOrder{p.tile_map, p.tile_group_m, p.tile_split_m}, s_word);
    if (t < 0) break;
    const int mi = t / p.tiles_n, nb = t % p.tiles_n;
    const int mb = (mi + p.mb0) % p.tiles_m;   // local rows first, then peers in landing order
    const int m0 = mb * BM, n0 = nb * BN;
    const int m1 = min(m0 + BM, M);
    const uint16_t *abase;
    SlabGate gate{&p.sync, 0u, 0};
    bool gated = false;
    if (!PRE && m0 >= loc0 && m1 <= loc1) {
      abase = p.shard[p.rank] + (size_t)(m0 - loc0) * p.k;
    } else {
      abase = p.ag + (size_t)m0 * p.k;
      if (!PRE) {
        // rows inside one land block: the 8-wave K loop checks slabs 1.. as
        // it reaches them; otherwise every slab is waited for here
        const int q0 = m0 / p.m_s, j0 = (m0 - q0 * p.m_s) / p.lb_rows;
        const int q1 = (m1 - 1) / p.m_s, j1 = (m1 - 1 - q1 * p.m_s) / p.lb_rows;
        const bool in_loop = C::WAVES == 8 && p.slab_stages > 0 && q0 == q1 && j0 == j1;
        if (!ag_acquire_rows(p, m0, m1, 0, in_loop ? 1 : p.n_slabs, helper, s_word)) break;
        if (in_loop) gate = SlabGate{&p.sync, ag_flag(p, q0, j0, 0), p.slab_stages};
        gated = in_loop;
      }
    }
    const int valid_n = min(BN, p.n - n0);
    const i32x4_t ra = make_vdesc(abase, (uint32_t)((m1 - m0) * ldb));
    const i32x4_t rb = make_vdesc(p.bt + (size_t)n0 * p.k, (uint32_t)(valid_n * ldb));
    AccTile<BM, BN> acc;
    // two instantiations of the K loop: with a gate it is longer and holds
    // more registers, so tiles that need no in-loop check run the plain one
    if (gated)
      gemm_tile<BM, BN>(smem, ra, rb, ldb, p.k, acc, gate);
    else
      gemm_tile<BM, BN>(smem, ra, rb, ldb, p.k, acc);
    staged_epilogue<BM, BN>(acc, smem, [&](int r, int cc, const f32x4_t &v) {
      const int row = m0 + r, col = n0 + cc;
      if (row < m1 && col < p.n) store_nt(p.c + (size_t)row * p.n + col, pack_bf16x4(v[0], v[1], v[2], v[3]));
    });
    // this workgroup's share of the items later tiles need
    if constexpr (!PRE) {
      for (int i = 0; i < p.land_between; ++i) {
        const uint32_t it = next_index(&p.sync.ctrl->land_ctr, s_word);
        if (it >= (uint32_t)p.n_items) break;
        ag_land_item(p, it);
      }
    }
  }
}

// MODE selects one of three instantiations so that profiles tell them apart:
//   kAgFused      land + compute (the fused operation)
//   kAgGemmOnly   A already gathered (MK_F_PRELANDED): compute only
//   kAgLandOnly   n_compute = 0: landing only (transfer alone)
constexpr int kAgFused = 0, kAgGemmOnly = 1, kAgLandOnly = 2;

template <int BM, int BN, int MODE>
__global__ __launch_bounds__((TileCfg<BM, BN>::THREADS), 1) void ag_gemm_kernel(AgParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[TileCfg<BM, BN>::LDS_BYTES];
  __shared__ uint32_t s_word;
  // The 4-wave tile's loop reads its parameters from an LDS copy: LDS reads
  // are reloaded where they are used (the K loop's asm may write memory), so
  // no parameter stays live in scalar registers across its K loop, where
  // spilled ones were restored with v_readlane every iteration.  (The 8-wave
  // tile's fused loop measured slower that way and keeps the kernel
  // arguments.)
  __shared__ AgParams s_prm;
  constexpr bool kLdsParams = TileCfg<BM, BN>::WAVES == 4;
  if (kLdsParams) copy_params(&s_prm, p);  // take_ticket's barrier publishes the copy
  const AgParams &q = kLdsParams ? s_prm : p;
  const uint32_t ticket = take_ticket(p.sync, &s_word);
  if (MODE == kAgLandOnly) {
    if (ticket < (uint32_t)p.n_land) ag_land(p, &s_word);
  } else if (MODE == kAgGemmOnly) {
    if (ticket < (uint32_t)p.n_compute) ag_compute<BM, BN, true>(q, smem, &s_word, ticket);
  } else if (ticket < (uint32_t)p.n_land) {
    ag_land(p, &s_word);
    if (p.land_joins_compute) ag_compute<BM, BN, false>(q, smem, &s_word, ticket);
  } else if (ticket < (uint32_t)(p.n_land + p.n_compute)) {
    ag_compute<BM, BN, false>(q, smem, &s_word, ticket);
    // with dynamic roles nobody may have been assigned the items no tile
    // waits for (the local shard's copy is landed last): drain the queue
    if (p.help_land) ag_land(p, &s_word);
  }
  finish_launch(p.sync);
}

// ---------------------------------------------------------------- peer partials

// One 4-column group of each of the np peers' fp32 partials (the compact
// list, ascending rank).
struct PeerRow {
  f32x4_t v[MK_MAX_WORLD - 1];
};

__device__ __forceinline__ void load_peers(PeerRow &pr, const float *const *pc, int np, size_t off) {
#pragma unroll
  for (int i = 0; i < MK_MAX_WORLD - 1; ++i)
    if (i < np) pr.v[i] = *reinterpret_cast<const f32x4_t *>(pc[i] + off);
}

// v + the peers' partials, in rank order.
__device__ __forceinline__ f32x4_t sum_peers(const f32x4_t &v, const PeerRow &pr, int np) {
  f32x4_t x = v;
#pragma unroll
  for (int i = 0; i < MK_MAX_WORLD - 1; ++i)
    if (i < np) x += pr.v[i];
  return x;
}

// The pointer tables of a launch, copied to LDS once and read where they are
// used.  Taken from the kernel arguments instead, they are loaded into SGPRs
// at the start and held through the K loop, which then spills its buffer
// descriptors to VGPR lanes; a descriptor restored right before an LDS DMA
// violates the 5-wait-state rule for VALU-written SGPRs.
//   peer  the peers' fp32 partials (compact list, ascending rank)
//   epi   what a tile's epilogue adds to its accumulators: the peers, the
//         reduce workspace (one entry), or nothing (compute alone)
//   dst   RS outboxes by rank, or AR broadcast buffers
struct PtrTable {
  const float *peer[MK_MAX_WORLD];
  const float *epi[MK_MAX_WORLD];
  uint16_t *dst[MK_MAX_WORLD];
};

// Which list the tile epilogues add.
constexpr int kEpiNone = 0, kEpiWs = 1, kEpiPeers = 2;

__device__ __forceinline__ void fill_table(PtrTable *t, const float *const *peer, uint16_t *const *dst,
                                           const float *ws, int epi) {
  if (threadIdx.x < MK_MAX_WORLD) {
    t->peer[threadIdx.x] = peer[threadIdx.x];
    t->dst[threadIdx.x] = dst[threadIdx.x];
    t->epi[threadIdx.x] = epi == kEpiPeers ? peer[threadIdx.x] : threadIdx.x == 0 && epi == kEpiWs ? ws : nullptr;
  }
  __syncthreads();
}

// A table entry as a uniform (scalar) pointer: every lane reads the same slot.
template <class T>
__device__ __forceinline__ T *table_ptr(T *const &slot) {
  return static_cast<T *>(const_cast<void *>(uniform_ptr(slot)));
}

// load_peers / sum_peers for a peer count known at compile time, from the
// compact list (ascending rank).  Every load is unconditional: loads behind uniform
// branches leave the compiler unable to count them, and it then waits for
// all memory traffic, the previous group's stores included, before using
// any of them.
template <int NP>
struct PeerVals {
  f32x4_t v[NP];
};

template <>
struct PeerVals<0> {};

// The partials are read once: non-temporal loads keep them from displacing
// cached data.
template <int NP>
__device__ __forceinline__ PeerVals<NP> load_peer_vals(const float *const *pc, size_t off) {
  PeerVals<NP> r;
  if constexpr (NP > 0) {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      r.v[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(pc[i] + off));
  }
  return r;
}


template <int NP>
__device__ __forceinline__ f32x4_t add_peer_vals(const f32x4_t &v, const PeerVals<NP> &pv) {
  f32x4_t x = v;
  if constexpr (NP > 0) {
#pragma unroll
    for (int i = 0; i < NP; ++i) x += pv.v[i];
  }
  return x;
}

// body(std::integral_constant<int, NP>) for the peer counts with a
// specialised epilogue (world 8, 4, 2 and 1); false for any other count.
template <class Body>
__device__ __forceinline__ bool with_peer_count(int np, Body &&body) {
  switch (np) {
    case 0: body(std::integral_constant<int, 0>{}); return true;
    case 7: body(std::integral_constant<int, 7>{}); return true;
    case 3: body(std::integral_constant<int, 3>{}); return true;
    case 1: body(std::integral_constant<int, 1>{}); return true;
    default: return false;
  }
}

// ---------------------------------------------------------------- reduce role

constexpr int kRedToWs = 0, kRedToOut = 1, kRedZero = 2;

// The four-column groups of rows [r0, r0 + rows) x columns [c0, c0 + cols)
// of a row-major layout of row pitch n (cols a multiple of 4), with the whole
// workgroup.  kRedToWs: the fp32 sum of the np partials pc[] (ascending
// rank) goes to ws; kRedToOut: the sum, rounded to bf16, goes to d0 and to
// every extra[0..n_extra); kRedZero: bf16 zeros go there and nothing is
// read.  d0, ws and the partials share the layout.  With a peer count known
// at compile time each thread issues the loads of its next group before it
// stores the current one (group indices past the end load a group of the
// region and store nothing, so no load needs a branch).
template <int MODE>
__device__ __forceinline__ void reduce_region(const float *const *pc, int np, float *ws, uint16_t *d0,
                                              uint16_t *const *extra, int n_extra, size_t r0, int rows,
                                              int c0, int cols, size_t n) {
  const int cg = cols >> 2;
  const int G = rows * cg;
  const int nt = blockDim.x;
  if (G <= 0) return;
  auto off = [&](int g) {
    g = min(g, G - 1);
    return (r0 + (size_t)(g / cg)) * n + (size_t)c0 + (size_t)(g % cg) * 4;
  };
  auto put = [&](int g, const f32x4_t &x) {
    if (g >= G) return;
    const size_t o = off(g);
    if constexpr (MODE == kRedToWs) {
      *reinterpret_cast<f32x4_t *>(ws + o) = x;
    } else {
      const uint2 b = MODE == kRedZero ? make_uint2(0u, 0u) : pack_bf16x4(x[0], x[1], x[2], x[3]);
      store_nt(d0 + o, b);
      for (int i = 0; i < n_extra; ++i) store_nt(table_ptr(extra[i]) + o, b);
    }
  };
  if constexpr (MODE == kRedZero) {
    for (int g = (int)threadIdx.x; g < G; g += nt) put(g, f32x4_t{});
    return;
  } else {
    if (!with_peer_count(np, [&](auto npc) {
          constexpr int NP = decltype(npc)::value;
          const float *p[NP > 0 ? NP : 1];
#pragma unroll
          for (int i = 0; i < NP; ++i) p[i] = table_ptr(pc[i]);
          int g = (int)threadIdx.x;
          auto va = load_peer_vals<NP>(p, off(g));
#pragma unroll 1
          for (; g < G; g += 2 * nt) {
            auto vb = load_peer_vals<NP>(p, off(g + nt));
            put(g, add_peer_vals<NP>(f32x4_t{}, va));
            va = load_peer_vals<NP>(p, off(g + 2 * nt));
            put(g + nt, add_peer_vals<NP>(f32x4_t{}, vb));
          }
        })) {
      for (int g = (int)threadIdx.x; g < G; g += nt) {
        PeerRow pr;
        load_peers(pr, pc, np, off(g));
        put(g, sum_peers(f32x4_t{}, pr, np));
      }
    }
  }
}

// Release reduce item `it` (flag index = item) after the workgroup's stores
// of it: every thread waits for its own stores, then one release fence
// writes this XCD's L2 back before the flag moves.
__device__ __forceinline__ void red_release(const Sync &s, uint32_t it) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    fence_release();
    st_release(flag_ptr(s, it), s.epoch);
  }
  __syncthreads();
}

// Claim and process reduce items until none is left.  release: each item's
// flag is released after its stores.
template <class Item>
__device__ __forceinline__ void red_loop(const Sync &s, int n_items, bool release, Item &&item,
                                         uint32_t *s_word) {
  for (;;) {
    const uint32_t it = next_index(&s.ctrl->reduce_ctr, s_word);
    if (it >= (uint32_t)n_items) break;
    item((int)it);
    if (release) red_release(s, it);
  }
}

// After the K loop of a tile whose epilogue needs reduce item `it`: wait for
// the item (thread 0) and acquire it.  Compute workgroups never reduce items
// themselves: every item is taken by a reduce workgroup, and those took the
// first tickets and wait for nothing, so every item a tile waits for is done
// by a running workgroup.
__device__ __forceinline__ bool red_wait(const Sync &s, uint32_t it, bool light, uint32_t *s_word) {
  bool ok0 = true;
  if (threadIdx.x == 0) ok0 = spin_until_eq(s, flag_ptr(s, it), s.epoch, 0x52000000u | it);
  return wg_sync_ok(ok0, s_word, !light);
}

// ---------------------------------------------------------------- GEMM + ReduceScatter

// Reduce item `it`: the own-slice rows of tile (mb_lo + it / tiles_n,
// it % tiles_n) -- or, with no compute, every row of that tile, whose own
// rows get bf16 of the peers' sum and whose other rows get zeros in their
// outbox.
template <int BM, int BN>
__device__ __forceinline__ void rs_reduce_item(const RsParams &p, const PtrTable &tab, int it) {
  const int mb = p.red.mb_lo + it / p.tiles_n, nb = it % p.tiles_n;
  const int c0 = nb * BN, cols = min(BN, p.n - c0);
  int r0 = mb * BM;
  const int r1 = min(r0 + BM, p.m);
  const int lo = p.rank * p.ms;
  if (!p.red.xfer_only) {
    const int a = max(r0, lo), b = min(r1, lo + p.ms);
    reduce_region<kRedToWs>(tab.peer, p.world - 1, p.red.ws, nullptr, nullptr, 0, (size_t)(a - lo), b - a,
                            c0, cols, (size_t)p.n);
    return;
  }
  while (r0 < r1) {  // rows of one slice at a time
    const int q = r0 / p.ms, b = min(r1, (q + 1) * p.ms);
    if (q == p.rank)
      reduce_region<kRedToOut>(tab.peer, p.world - 1, nullptr, p.c_own, nullptr, 0, (size_t)(r0 - lo),
                               b - r0, c0, cols, (size_t)p.n);
    else
      reduce_region<kRedZero>(nullptr, 0, nullptr, table_ptr(tab.dst[q]), nullptr, 0,
                              (size_t)(r0 - q * p.ms), b - r0, c0, cols, (size_t)p.n);
    r0 = b;
  }
}

template <int BM, int BN>
__device__ __forceinline__ void rs_compute(const RsParams &p, const PtrTable &tab, char *smem,
                                           uint32_t *s_word) {
  const int xcd = xcd_id();
  const int lda = p.k * 2;
  // what the epilogues add to the own slice: the peers' partials, or their
  // sum from the reduce role's workspace, or nothing (compute alone)
  const bool red = p.red.n_items > 0;
  const int enp = red ? 1 : p.no_peers ? 0 : p.world - 1;
  const int lo = p.rank * p.ms, hi = lo + p.ms;
  for (;;) {
    const int t = next_tile(p.sync, p.tiles_m, p.tiles_n, xcd, TileOrder{p.tile_map, p.tile_group_m, p.tile_split_m}, s_word);
    if (t < 0) break;
    const int mi = t / p.tiles_n, nb = t % p.tiles_n;
    const int mb = (mi + p.mb0) % p.tiles_m;   // tile order: see the launcher
    const int m0 = mb * BM, n0 = nb * BN;
    const int m1 = min(m0 + BM, p.m);
    const int valid_n = min(BN, p.n - n0);
    const i32x4_t ra = make_vdesc(p.a + (size_t)m0 * p.k, (uint32_t)((m1 - m0) * lda));
    const i32x4_t rb = make_vdesc(p.bt + (size_t)n0 * p.k, (uint32_t)(valid_n * lda));
    AccTile<BM, BN> acc;
    gemm_tile<BM, BN>(smem, ra, rb, lda, p.k, acc);
    // the reduce item of this tile's own-slice rows (worked out after the K
    // loop: values held across it cost registers the loop needs)
    if (red && m0 < hi && m1 > lo &&
        !red_wait(p.sync, (uint32_t)((m0 / BM - p.red.mb_lo) * p.tiles_n + n0 / BN), p.red.light_acquire != 0,
                  s_word))
      break;
    const int cols = min(BN, p.n - n0);
    // Row r of slice q: the own slice adds the epilogue list and goes to
    // c_own, any other slice to outbox[q].
    auto epi_row = [&](int row, int cc, const f32x4_t &v, int q, uint16_t *d) {
      const size_t off = (size_t)(row - q * p.ms) * p.n + n0 + cc;
      f32x4_t x = v;
      if (q == p.rank) {
        PeerRow pr;  // all loads are issued before any is used
        load_peers(pr, tab.epi, enp, off);
        x = sum_peers(v, pr, enp);
      }
      store_nt(d + off, pack_bf16x4(x[0], x[1], x[2], x[3]));
    };
    // A tile inside one slice (every tile when the slice height is a
    // multiple of BM) reads its destination once; only a tile that straddles
    // slices picks one per row (from the LDS table: a per-row pick from the
    // kernel arguments compiles to a vector load of the pointer, whose wait
    // also waits for every store before it).
    const int q0 = m0 / p.ms;
    if ((m1 - 1) / p.ms == q0 && q0 == p.rank) {
      // own slice: the partials of the next column group are loaded before
      // this one is stored
      const int r0 = m0 - q0 * p.ms, rows = m1 - m0;
      auto put = [&](int r, int cc, const f32x4_t &x) {
        if (r < rows && cc < cols)
          store_nt(p.c_own + (size_t)(r0 + r) * p.n + n0 + cc, pack_bf16x4(x[0], x[1], x[2], x[3]));
      };
      // addresses clamped into the tile: a group past its edge loads an
      // element of the tile that it does not use, so no load needs a branch
      auto off_in = [&](int r, int cc) { return (size_t)(r0 + min(r, rows - 1)) * p.n + n0 + min(cc, cols - 4); };
      if (!with_peer_count(enp, [&](auto np) {
            constexpr int NP = decltype(np)::value;
            const float *pc[NP > 0 ? NP : 1];
#pragma unroll
            for (int i = 0; i < NP; ++i) pc[i] = table_ptr(tab.epi[i]);
            staged_epilogue_pf<BM, BN>(
                acc, smem, [&](int r, int cc) { return load_peer_vals<NP>(pc, off_in(r, cc)); },
                [&](int r, int cc, const f32x4_t &v, const PeerVals<NP> &pv) { put(r, cc, add_peer_vals<NP>(v, pv)); });
          }))
        staged_epilogue<BM, BN>(acc, smem, [&](int r, int cc, const f32x4_t &v) {
          if (r < rows && cc < cols) {
            PeerRow pr;
            load_peers(pr, tab.epi, enp, off_in(r, cc));
            put(r, cc, sum_peers(v, pr, enp));
          }
        });
    } else if ((m1 - 1) / p.ms == q0) {
      uint16_t *d0 = table_ptr(tab.dst[q0]);
      staged_epilogue<BM, BN>(acc, smem, [&](int r, int cc, const f32x4_t &v) {
        if (r < m1 - m0 && cc < cols) epi_row(m0 + r, cc, v, q0, d0);
      });
    } else {
      staged_epilogue<BM, BN>(acc, smem, [&](int r, int cc, const f32x4_t &v) {
        const int row = m0 + r;
        if (row >= m1 || cc >= cols) return;
        const int q = row / p.ms;
        epi_row(row, cc, v, q, q == p.rank ? p.c_own : tab.dst[q]);
      });
    }
  }
}

template <int BM, int BN>
__global__ __launch_bounds__((TileCfg<BM, BN>::THREADS), 1) void gemm_rs_kernel(RsParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[TileCfg<BM, BN>::LDS_BYTES];
  __shared__ uint32_t s_word;
  __shared__ PtrTable s_tab;
  // the tile loop reads its parameters from an LDS copy: LDS reads are
  // reloaded where they are used (the K loop's asm may write memory), so
  // fewer parameters stay live in (spilled) scalar registers around it
  __shared__ RsParams s_prm;
  copy_params(&s_prm, p);  // take_ticket's barrier publishes the copy
  fill_table(&s_tab, p.peer_c, p.outbox, p.red.ws,
             p.red.n_items > 0 && !p.red.xfer_only ? kEpiWs : p.no_peers ? kEpiNone : kEpiPeers);
  // reduce workgroups take the first tickets: every item a tile waits for
  // belongs to a workgroup that is already running
  const uint32_t ticket = take_ticket(p.sync, &s_word);
  const uint32_t nr = (uint32_t)p.red.n_reduce;
  if (ticket < nr) {
    red_loop(p.sync, p.red.n_items, !p.red.xfer_only, [&](int it) { rs_reduce_item<BM, BN>(p, s_tab, it); },
             &s_word);
    if (p.red.joins_compute) rs_compute<BM, BN>(s_prm, s_tab, smem, &s_word);
  } else if (ticket < nr + (uint32_t)p.n_compute) {
    rs_compute<BM, BN>(s_prm, s_tab, smem, &s_word);
  }
  finish_launch(p.sync);
}

// ---------------------------------------------------------------- GEMM + AllReduce

// Reduce item `it` = tile it: the peers' sum into the workspace, or, with no
// compute, bf16 of it to c and every broadcast buffer.
template <int BM, int BN>
__device__ __forceinline__ void ar_reduce_item(const ArParams &p, const PtrTable &tab, int it) {
  const int mb = it / p.tiles_n, nb = it % p.tiles_n;
  const int c0 = nb * BN, cols = min(BN, p.n - c0);
  const int r0 = mb * BM, rows = min(BM, p.m - r0);
  if (!p.red.xfer_only)
    reduce_region<kRedToWs>(tab.peer, p.world - 1, p.red.ws, nullptr, nullptr, 0, (size_t)r0, rows, c0,
                            cols, (size_t)p.n);
  else
    reduce_region<kRedToOut>(tab.peer, p.world - 1, nullptr, p.c, tab.dst, p.n_bcast, (size_t)r0, rows, c0,
                             cols, (size_t)p.n);
}

template <int BM, int BN>
__device__ __forceinline__ void ar_compute(const ArParams &p, const PtrTable &tab, char *smem,
                                           uint32_t *s_word) {
  const int xcd = xcd_id();
  const int lda = p.k * 2;
  const bool red = p.red.n_items > 0;
  const int enp = red ? 1 : p.no_peers ? 0 : p.world - 1;
  for (;;) {
    const int t = next_tile(p.sync, p.tiles_m, p.tiles_n, xcd, TileOrder{p.tile_map, p.tile_group_m, p.tile_split_m}, s_word);
    if (t < 0) break;
    const int mb = t / p.tiles_n, nb = t % p.tiles_n;
    const int m0 = mb * BM, n0 = nb * BN;
    const int m1 = min(m0 + BM, p.m);
    const int valid_n = min(BN, p.n - n0);
    const i32x4_t ra = make_vdesc(p.a + (size_t)m0 * p.k, (uint32_t)((m1 - m0) * lda));
    const i32x4_t rb = make_vdesc(p.bt + (size_t)n0 * p.k, (uint32_t)(valid_n * lda));
    AccTile<BM, BN> acc;
    gemm_tile<BM, BN>(smem, ra, rb, lda, p.k, acc);
    if (red && !red_wait(p.sync, (uint32_t)((m0 / BM) * p.tiles_n + n0 / BN), p.red.light_acquire != 0, s_word))
      break;
    const int cols = min(BN, p.n - n0);
    // the partials of the next column group are loaded before this one is
    // stored
    const int rows = m1 - m0;
    uint16_t *bc[MK_MAX_WORLD];
#pragma unroll
    for (int b = 0; b < MK_MAX_WORLD; ++b)
      if (b < p.n_bcast) bc[b] = table_ptr(tab.dst[b]);
    auto put = [&](int r, int cc, const f32x4_t &x) {
      if (r >= rows || cc >= cols) return;
      const size_t off = (size_t)(m0 + r) * p.n + n0 + cc;
      const uint2 o = pack_bf16x4(x[0], x[1], x[2], x[3]);
      store_nt(p.c + off, o);
#pragma unroll
      for (int b = 0; b < MK_MAX_WORLD; ++b)
        if (b < p.n_bcast) store_nt(bc[b] + off, o);
    };
    // addresses clamped into the tile (see the ReduceScatter epilogue)
    auto off_in = [&](int r, int cc) { return (size_t)(m0 + min(r, rows - 1)) * p.n + n0 + min(cc, cols - 4); };
    if (!with_peer_count(enp, [&](auto np) {
          constexpr int NP = decltype(np)::value;
          const float *pc[NP > 0 ? NP : 1];
#pragma unroll
          for (int i = 0; i < NP; ++i) pc[i] = table_ptr(tab.epi[i]);
          staged_epilogue_pf<BM, BN>(
              acc, smem, [&](int r, int cc) { return load_peer_vals<NP>(pc, off_in(r, cc)); },
              [&](int r, int cc, const f32x4_t &v, const PeerVals<NP> &pv) { put(r, cc, add_peer_vals<NP>(v, pv)); });
        }))
      staged_epilogue<BM, BN>(acc, smem, [&](int r, int cc, const f32x4_t &v) {
        if (r < rows && cc < cols) {
          PeerRow pr;
          load_peers(pr, tab.epi, enp, off_in(r, cc));
          put(r, cc, sum_peers(v, pr, enp));
        }
      });
  }
}

template <int BM, int BN>
__global__ __launch_bounds__((TileCfg<BM, BN>::THREADS), 1) void gemm_ar_kernel(ArParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[TileCfg<BM, BN>::LDS_BYTES];
  __shared__ uint32_t s_word;
  __shared__ PtrTable s_tab;
  // the tile loop reads its parameters from an LDS copy: LDS reads are
  // reloaded where they are used (the K loop's asm may write memory), so
  // fewer parameters stay live in (spilled) scalar registers around it
  __shared__ ArParams s_prm;
  copy_params(&s_prm, p);  // take_ticket's barrier publishes the copy
  fill_table(&s_tab, p.peer_c, p.bcast, p.red.ws,
             p.red.n_items > 0 && !p.red.xfer_only ? kEpiWs : p.no_peers ? kEpiNone : kEpiPeers);
  const uint32_t ticket = take_ticket(p.sync, &s_word);
  const uint32_t nr = (uint32_t)p.red.n_reduce;
  if (ticket < nr) {
    red_loop(p.sync, p.red.n_items, !p.red.xfer_only, [&](int it) { ar_reduce_item<BM, BN>(p, s_tab, it); },
             &s_word);
    if (p.red.joins_compute) ar_compute<BM, BN>(s_prm, s_tab, smem, &s_word);
  } else if (ticket < nr + (uint32_t)p.n_compute) {
    ar_compute<BM, BN>(s_prm, s_tab, smem, &s_word);
  }
  finish_launch(p.sync);
}

// ---------------------------------------------------------------- launchers

template <typename K, typename P>
static hipError_t launch(K kernel, int threads, int grid, hipStream_t stream, const P &params) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, stream, params);
  return hipGetLastError();
}

using Big = TileCfg<256, 256>;
using Small = TileCfg<128, 128>;

template <int BM, int BN>
static hipError_t launch_ag_tile(const AgParams &p, int grid, hipStream_t s) {
  constexpr int T = TileCfg<BM, BN>::THREADS;
  if (p.prelanded) return launch(ag_gemm_kernel<BM, BN, kAgGemmOnly>, T, grid, s, p);
  if (p.n_compute == 0) return launch(ag_gemm_kernel<BM, BN, kAgLandOnly>, T, grid, s, p);
  return launch(ag_gemm_kernel<BM, BN, kAgFused>, T, grid, s, p);
}

hipError_t launch_ag(const AgParams &p, int bm, int bn, int grid, hipStream_t s) {
  if (bm == 256 && bn == 224) return launch_ag_tile<256, 224>(p, grid, s);
  if (bm == 256) return launch_ag_tile<256, 256>(p, grid, s);
  return launch_ag_tile<128, 128>(p, grid, s);
}
hipError_t launch_rs(const RsParams &p, int bm, int grid, hipStream_t s) {
  if (bm == 256) return launch(gemm_rs_kernel<256, 256>, Big::THREADS, grid, s, p);
  return launch(gemm_rs_kernel<128, 128>, Small::THREADS, grid, s, p);
}
hipError_t launch_ar(const ArParams &p, int bm, int grid, hipStream_t s) {
  if (bm == 256) return launch(gemm_ar_kernel<256, 256>, Big::THREADS, grid, s, p);
  return launch(gemm_ar_kernel<128, 128>, Small::THREADS, grid, s, p);
}

// Resident workgroups per CU of each instantiation (queried once per handle).
hipError_t occupancy(int op, int bm, int bn, int *blocks_per_cu) {
  const void *f = nullptr;
  switch (op) {
    case MK_OP_AG_GEMM:
      f = bm != 256 ? (const void *)ag_gemm_kernel<128, 128, kAgFused>
          : bn == 224 ? (const void *)ag_gemm_kernel<256, 224, kAgFused>
                      : (const void *)ag_gemm_kernel<256, 256, kAgFused>;
      break;
    case MK_OP_GEMM_RS:
      f = bm == 256 ? (const void *)gemm_rs_kernel<256, 256> : (const void *)gemm_rs_kernel<128, 128>;
      break;
    case MK_OP_GEMM_AR:
      f = bm == 256 ? (const void *)gemm_ar_kernel<256, 256> : (const void *)gemm_ar_kernel<128, 128>;
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, f,
                                                      bm == 256 ? Big::THREADS : Small::THREADS, 0);
  static_assert(TileCfg<256, 224>::THREADS == Big::THREADS, "256-row tiles run 8 waves");
}

}  // namespace mk

// Kernel parameter blocks shared by the host launcher and the kernels.
#pragma once

#include <stdint.h>

#include "../../include/mk.h"
#include "mk_device.h"

namespace mk {

// AllGather + GEMM.  Landing unit: a "land block" of lb_rows rows of one
// shard and one K-slab of slab_k columns (one ready flag each), copied as
// items_per_block items of item_rows rows (items_per_block_first items of
// item_rows_first rows for the first group's shards, which every workgroup
// lands at once at the start).  Flag of block j of shard q, slab s:
// (q * blocks_per_chunk + j) * n_slabs + s.  Items are numbered peers first,
// in two groups: the first_peers peers (in landing order rank+1, rank+2,
// ...) whose tiles run in the first round of tiles (n_first_items items),
// then the others; each group slab-major (every peer's slab 0, then slab 1,
// ...).  The local shard's items come last.
struct AgParams {
  Sync sync;
  const uint16_t *shard[MK_MAX_WORLD];
  const uint16_t *bt;
  uint16_t *c;
  uint16_t *ag;
  int world, rank, m_s, n, k;
  int n_land, n_compute;
  int tiles_m, tiles_n, n_tiles, mb0, tile_map, tile_group_m, tile_split_m;
  int lb_rows, blocks_per_chunk, item_rows, items_per_block, n_items, n_peer_items;
  int item_rows_first, items_per_block_first, n_first_items;
  int first_peers;
  int n_slabs, slab_k;
  int slab_stages;         // slab_k / 64 when tiles may start before their later slabs land, else 0
  int prelanded;
  int land_joins_compute;  // land workgroups run tiles once nothing is left to land
  int help_land;           // compute workgroups land items while their rows are missing
  int help_every;          // ... only every help_every-th compute workgroup (by ticket)
  int help_eager;          // a helping workgroup lands every item below eager_items, not only until its rows are ready
  int eager_items;
  int land_between;        // items every compute workgroup lands after each tile
  int light_acquire;       // land blocks are cache-line aligned (see wg_sync_ok)
};

// Reduce role of GEMM+ReduceScatter and GEMM+AllReduce.  A reduce item is
// the part of one output tile (tile grid of the GEMM, m-blocks
// [mb_lo, mb_lo + mbs) x every n-block) whose rows need the peers' partials:
// RS rows of this rank's slice, AR every row.  In the fused launch a reduce
// workgroup sums the peers' fp32 partials of an item into the workspace
// (same layout as the partials) and releases the item's flag (flag index =
// item); the tile's epilogue then adds the workspace instead of the peers.
// Transfer alone (no compute workgroups): items cover every tile and write
// the outputs themselves -- bf16 of the peers' sum where the rows need it,
// zeros to the RS outboxes -- so the same bytes move as in the fused call.
struct RedParams {
  float *ws;
  int n_reduce;
  int mb_lo, mbs, n_items;
  int light_acquire;     // item regions start and end on 128-byte lines of ws
  int xfer_only;         // no compute: items write the outputs
  int joins_compute;     // reduce workgroups run tiles once every item is claimed
};

// GEMM + ReduceScatter.
struct RsParams {
  Sync sync;
  const uint16_t *a;
  const uint16_t *bt;
  const float *peer_c[MK_MAX_WORLD];  // the world - 1 peers' partials, ascending rank
  uint16_t *c_own;
  uint16_t *outbox[MK_MAX_WORLD];
  int world, rank, m, n, k, ms;
  int n_compute;
  int no_peers;                       // compute alone: epilogues leave out the peers' partials
  int tiles_m, tiles_n, n_tiles, mb0, tile_map, tile_group_m, tile_split_m;
  RedParams red;
};

// GEMM + AllReduce.
struct ArParams {
  Sync sync;
  const uint16_t *a;
  const uint16_t *bt;
  const float *peer_c[MK_MAX_WORLD];  // the world - 1 peers' partials, ascending rank
  uint16_t *c;
  uint16_t *bcast[MK_MAX_WORLD];
  int world, rank, n_bcast, m, n, k;
  int n_compute;
  int no_peers;
  int tiles_m, tiles_n, n_tiles, tile_map, tile_group_m, tile_split_m;
  RedParams red;
};

// Ring attention.  Receive buffers are indexed by source rank: k_recv
// [W][BH][S_kv][D], vt_recv [W][BH][D][S_kv] (V transposed).
constexpr int kAttnD = 128;
struct AttnParams {
  Sync sync;
  const uint16_t *q;                      // [BH][S_q][D]
  const uint16_t *k_src[MK_MAX_WORLD];    // [BH][S_kv][D] of rank r
  const uint16_t *v_src[MK_MAX_WORLD];
  uint16_t *o;                            // [BH][S_q][D]
  float *lse;                             // [BH][S_q]
  uint16_t *k_recv;
  uint16_t *vt_recv;
  int world, rank, BH, S_q, S_kv;
  float scale_log2;                       // scale * log2(e)
  int n_land, n_compute;
  int chunk_keys, chunks;                 // keys per landing chunk, chunks per block
  int q_tiles, n_tasks, n_items;
  int light_acquire;
  int prelanded;                          // receive buffers already hold every block
  int splits, n_pairs;                    // tasks per (bh, q-tile) pair: 1, or 2 ring halves
  uint32_t merge_flag0;                   // flag / counter of pair i: merge_flag0 + i
  float *ws;                              // splits == 2: one combine slot per pair
  int tile_map;                           // task order: kMapGlobal, or an XCD map over heads
};

// MoE dispatch + grouped GEMM.  Route items are blocks of kRouteTokens
// tokens of one source; an item's flag says all of its local tokens landed.
// An item lands as kLandParts parts (the item's tokens t with t % kLandParts
// == part), each a unit of the land queue; the item's flag completes after
// kLandParts arrivals.
constexpr int kRouteTokens = 256;
constexpr int kLandParts = 2;
constexpr int kMaxLocalExperts = 32;

struct MoeParams {
  Sync sync;
  const uint16_t *x[MK_MAX_WORLD];
  const float *logits[MK_MAX_WORLD];
  const uint16_t *wt;
  uint16_t *y;
  int32_t *topk_idx;
  float *topk_gate;
  int32_t *slot_token;
  int32_t *expert_offsets;
  int32_t *chunk_offsets;
  uint16_t *x_slots;
  // workspace
  int32_t *item_cnt;    // [n_items, E_loc] tokens of item routed to local expert e
  int32_t *item_base;   // [n_items, E_loc] first slot of (item, e) (written for the combine)
  int32_t *tok_rank;    // [S*T, top_k] rank of the token within (item, e); -1 if not local
  float *slot_gate;     // [cap]
  int32_t *slot_ret;    // [cap] return position (s*T + t)*top_k + k of every slot (combine)
  // combine (when `combine`): rows of this rank's experts return to ret[s]
  // ([T, top_k, N] per source s != rank); this rank's tokens sum their rows
  // from y (local experts) and y_peer ([T, top_k, N], remote experts) into out
  const uint16_t *y_peer;
  uint16_t *ret[MK_MAX_WORLD];
  uint16_t *out;
  int combine;
  int S, T, H, N, E, E_loc, top_k, rank, cap;
  int items_per_src, n_items;
  int n_land, n_compute;
  int tiles_n;
  int tile_map;         // kMapBlocks: XCD x takes the row tiles of a block of local experts
  int no_gate;
  int static_roles;     // land workgroups do not take tiles
  int withhold;         // failure tests: land unit never landed (-1: none), so its waiters time out
};

}  // namespace mk

// Persistent fused MoE dispatch + grouped GEMM.
//
// [P1] German article on mKernel (chatgpz.de), table "Die fuenf
// verschmolzenen Kerne", row "MoE-Versand + GEMM": tokens are routed to the
// ranks that own their experts and each expert's GEMM runs in the same kernel
// on the tokens as soon as they land, with no staging-buffer round trip.
//
// Phases inside one launch, chained by flags:
//   route  (every workgroup)   top-k over the logits, softmax gates, and per
//                              (route item, local expert) counts and ranks
//   offsets (every workgroup)  once every item is routed: each workgroup sums
//                              the counts itself into its LDS (expert totals
//                              and offsets, first row tile of each expert;
//                              a route item's slot bases when it needs them),
//                              so no workgroup waits for another's scan
//   scan   (ticket-0 workgroup) the slot offsets as outputs (expert_offsets,
//                              chunk_offsets) and the per-item bases the
//                              combine reads; publishes scan_ready
//   land   (every workgroup)   copies each routed token row straight into its
//                              expert slot and releases that route item's flag
//                              (a workgroup copies at a few tens of GB/s, so
//                              landing needs the whole grid)
//   compute (compute workgroups) grouped-GEMM tiles over the expert slots; a
//                              tile waits for the flags of the route items whose
//                              tokens fill its rows (one wave checks them in
//                              parallel); y = bf16(gate * acc)
//   combine (every workgroup, when requested) each finished row also returns
//                              to its source (ret[s] at (token, k)); once every
//                              tile is done, this rank's tokens sum their k rows
//                              (local experts from y, remote ones from what
//                              their owners returned) into out
// A route item is kRouteTokens consecutive tokens of one source rank.
//
// Everything one workgroup publishes to others (routing outputs, the scan,
// slot metadata, landed rows) is stored write-through (device scope), so a
// publish is: every thread waits for its stores, a barrier, then one
// counter add or flag store -- no write-back of the XCD's L2, whose cost
// grows with every other workgroup's dirty lines.  Readers acquire with an
// L2 invalidate before they read.
#include "mk_params.h"

namespace mk {

struct MoeShared {
  // a copy of the parameters that the tile loop reads: LDS reads are
  // reloaded where they are used (the K loop's asm may write memory), so no
  // parameter stays live in scalar registers across the K loop, where
  // spilled registers would be restored right before its DMAs
  MoeParams prm;
  uint32_t word;
  int32_t wave_cnt[kMaxWaves][kMaxLocalExperts];
  int32_t list_tok[kRouteTokens * 8];  // (slot << 8 | token in item) of the unit's rows
  int32_t n_list;
  int32_t tile_base[kMaxLocalExperts + 1];   // first row tile of each expert; [E_loc]: row tiles
  int32_t expert_off[kMaxLocalExperts + 1];   // first slot of each expert; [E_loc]: slots
  int32_t expert_tot[kMaxLocalExperts];
  int32_t unit_base[kMaxLocalExperts];        // first slot of (land item, expert)
  float tile_gate[256];      // gate of each row of the current tile
  int32_t tile_ret_src[256]; // source its row returns to (combine), -1: none
  uint32_t tile_ret_row[256];
  uint16_t *ret_ptr[MK_MAX_WORLD];
};

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---------------------------------------------------------------- route

// Route item `item` with two lanes per token (E = 64, top-2, 512 threads):
// lane h of token tt reads logits 32h .. 32h+31 and keeps its top-2; the
// pair merges the two lists (both lanes get the same result, the order of
// (logit descending, expert ascending) being strict) and adds its softmax
// sums; lane h then owns selection h -- its expert, gate and rank -- so
// every routing output is one store per lane.  Half the loads, compares and
// exponentials per lane of the one-lane-per-token form.
__device__ __forceinline__ void moe_route_item_pairs(const MoeParams &p, int item, MoeShared &sh) {
  const int s = item / p.items_per_src, b = item % p.items_per_src;
  const int tt = (int)threadIdx.x >> 1, h = (int)threadIdx.x & 1;
  const int t = b * kRouteTokens + tt;
  const bool valid = t < p.T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr float kLog2e = 1.4426950408889634f;
  f32x4_t l[8];
  int i0 = -1, i1 = -1;
  float v0 = 0.f, v1 = 0.f;
  if (valid) {
    const f32x4_t *lg = reinterpret_cast<const f32x4_t *>(p.logits[s] + (size_t)t * 64 + h * 32);
#pragma unroll
    for (int q = 0; q < 8; ++q) l[q] = lg[q];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float v = l[q][u];
        const int e = h * 32 + q * 4 + u;
        if (i0 < 0 || v > v0) {
          i1 = i0; v1 = v0;
          i0 = e; v0 = v;
        } else if (i1 < 0 || v > v1) {
          i1 = e; v1 = v;
        }
      }
  }
  // merge with the partner lane's list (every lane takes part in the shuffles)
  const float pv0 = __shfl_xor(v0, 1, 64), pv1 = __shfl_xor(v1, 1, 64);
  const int pi0 = __shfl_xor(i0, 1, 64), pi1 = __shfl_xor(i1, 1, 64);
  auto better = [](float va, int ia, float vb, int ib) { return va > vb || (va == vb && ia < ib); };
  int s0, s1;
  float w0, w1;
  if (better(v0, i0, pv0, pi0)) {
    s0 = i0; w0 = v0;
    if (better(v1, i1, pv0, pi0)) { s1 = i1; w1 = v1; } else { s1 = pi0; w1 = pv0; }
  } else {
    s0 = pi0; w0 = pv0;
    if (better(v0, i0, pv1, pi1)) { s1 = i0; w1 = v0; } else { s1 = pi1; w1 = pv1; }
  }
  // softmax terms as exp2(l log2(e) - max log2(e)): one fma and one
  // v_exp_f32 each; the pair adds its two partial sums
  const float mxl = w0 * kLog2e;
  float sum = 0.f;
  if (valid) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int u = 0; u < 4; ++u) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(l[q][u], kLog2e, -mxl));
  }
  sum += __shfl_xor(sum, 1, 64);
  const int my_e = h == 0 ? s0 : s1;
  const float my_gate = __builtin_amdgcn_exp2f(__builtin_fmaf(h == 0 ? w0 : w1, kLog2e, -mxl)) / sum;
  // per local expert: count and rank of this item's tokens (token order:
  // lanes are token-major, and a token's two lanes never share an expert)
  const int e_lo = p.rank * p.E_loc;
  int my_rank = -1;
  for (int e = 0; e < p.E_loc; ++e) {
    const bool mine = valid && my_e == e_lo + e;
    const uint64_t m = __ballot(mine);
    if (mine) my_rank = __popcll(m & lanemask_lt());
    if (lane == 0) sh.wave_cnt[wave][e] = __popcll(m);
  }
  __syncthreads();
  if (my_rank >= 0) {
    const int e = my_e - e_lo;
    int before = 0;
    for (int w = 0; w < wave; ++w) before += sh.wave_cnt[w][e];
    my_rank += before;
  }
  // every routing output in one batch of write-through stores
  if (valid) {
    const size_t o = ((size_t)s * p.T + t) * 2 + h;
    st_through(&p.topk_idx[o], (int32_t)my_e);
    st_through(&p.topk_gate[o], my_gate);
    st_through(&p.tok_rank[o], (int32_t)my_rank);
  }
  if (threadIdx.x < (unsigned)p.E_loc) {
    int tot = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += sh.wave_cnt[w][threadIdx.x];
    st_through(&p.item_cnt[(size_t)item * p.E_loc + threadIdx.x], (int32_t)tot);
  }
  __syncthreads();
}

__device__ __forceinline__ void moe_route_item(const MoeParams &p, int item, MoeShared &sh) {
  if (p.E == 64 && p.top_k == 2 && blockDim.x == 2 * kRouteTokens) {
    moe_route_item_pairs(p, item, sh);
    return;
  }
  const int s = item / p.items_per_src, b = item % p.items_per_src;
  // one token per thread; threads past kRouteTokens only join the counts
  const int t = b * kRouteTokens + (int)threadIdx.x;
  const bool valid = threadIdx.x < (unsigned)kRouteTokens && t < p.T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // top-k by value, descending, kept sorted in sel/selv (fixed-size,
  // fully unrolled so the arrays stay in registers).  A new expert goes
  // before the first kept entry it is strictly larger than, so equal logits
  // keep the lower expert id first.
  int sel[8];
  float selv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { sel[j] = -1; selv[j] = 0.f; }
  auto insert = [&](int e, float v) {
#pragma unroll
    for (int j = 7; j >= 0; --j) {
      if (j >= p.top_k) continue;
      const bool here = sel[j] < 0 || v > selv[j];
      const bool above = j > 0 && (sel[j - 1] < 0 || v > selv[j - 1]);
      if (here) {
        if (above) { sel[j] = sel[j - 1]; selv[j] = selv[j - 1]; }
        else { sel[j] = e; selv[j] = v; }
      }
    }
  };
  // softmax terms exp(l - max) as exp2(l log2(e) - max log2(e)): one fma
  // and one v_exp_f32 each (relative error ~1e-6 for the logit ranges of
  // a router, against the 1e-5 the gates are held to)
  constexpr float kLog2e = 1.4426950408889634f;
  float gate[8];
  if (valid) {
    const float *lg = p.logits[s] + (size_t)t * p.E;
    float sum = 0.f;
    if (p.E == 64) {
      // the token's 64 logits in 16 vector loads issued together, then the
      // top-k and the softmax sum from registers (one load per logit in a
      // loop leaves every iteration waiting for its load)
      f32x4_t l[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) l[q] = reinterpret_cast<const f32x4_t *>(lg)[q];
      if (p.top_k == 2) {
        // the same selection as insert() for two slots, without the general
        // slot loop
#pragma unroll
        for (int q = 0; q < 16; ++q)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float v = l[q][u];
            const int e = q * 4 + u;
            if (sel[0] < 0 || v > selv[0]) {
              sel[1] = sel[0]; selv[1] = selv[0];
              sel[0] = e; selv[0] = v;
            } else if (sel[1] < 0 || v > selv[1]) {
              sel[1] = e; selv[1] = v;
            }
          }
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q)
#pragma unroll
          for (int u = 0; u < 4; ++u) insert(q * 4 + u, l[q][u]);
      }
      const float mxl = selv[0] * kLog2e;
#pragma unroll
      for (int q = 0; q < 16; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(l[q][u], kLog2e, -mxl));
    } else {
      for (int e = 0; e < p.E; ++e) insert(e, lg[e]);
      const float mxl = selv[0] * kLog2e;
      for (int e = 0; e < p.E; ++e) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(lg[e], kLog2e, -mxl));
    }
    const float mxl = selv[0] * kLog2e;
#pragma unroll
    for (int j = 0; j < 8; ++j) gate[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(selv[j], kLog2e, -mxl)) / sum;
  }
  // per local expert: count and rank of this item's tokens (token order)
  const int e_lo = p.rank * p.E_loc;
  int my_rank[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) my_rank[j] = -1;
  for (int e = 0; e < p.E_loc; ++e) {
    bool mine = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) mine |= (j < p.top_k) && valid && sel[j] == e_lo + e;
    const uint64_t m = __ballot(mine);
    const int r = __popcll(m & lanemask_lt());
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < p.top_k && valid && sel[j] == e_lo + e) my_rank[j] = r;
    if (lane == 0) sh.wave_cnt[wave][e] = __popcll(m);
  }
  __syncthreads();
  for (int e = 0; e < p.E_loc; ++e) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += sh.wave_cnt[w][e];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < p.top_k && valid && sel[j] == e_lo + e) my_rank[j] += before;
  }
  // every routing output in one batch of write-through stores, so the
  // caller's wait for them is one round trip
  if (valid) {
    const size_t o = ((size_t)s * p.T + t) * p.top_k;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= p.top_k) continue;
      st_through(&p.topk_idx[o + j], (int32_t)sel[j]);
      st_through(&p.topk_gate[o + j], gate[j]);
      st_through(&p.tok_rank[o + j], (int32_t)my_rank[j]);
    }
  }
  if (threadIdx.x < (unsigned)p.E_loc) {
    int tot = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += sh.wave_cnt[w][threadIdx.x];
    st_through(&p.item_cnt[(size_t)item * p.E_loc + threadIdx.x], (int32_t)tot);
  }
  __syncthreads();
}

// ---------------------------------------------------------------- scan

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t y = __shfl_up(v, d, 64);
    if (lane >= d) v += y;
  }
  return v;
}

// Every workgroup, once every route item is counted: slots are ordered
// (expert, source, token), so expert e's slots start at the sum of the
// earlier experts' totals and its row tiles after theirs.  Each wave sums
// whole experts; integer sums are exact in any order, so every workgroup gets
// the same offsets.
template <int BM>
__device__ __forceinline__ void moe_offsets(const MoeParams &p, MoeShared &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int e = wave; e < p.E_loc; e += nw) {
    int32_t tot = 0;
    for (int i = lane; i < p.n_items; i += 64) tot += p.item_cnt[(size_t)i * p.E_loc + e];
    tot = wave_inclusive_scan(tot);
    if (lane == 63) sh.expert_tot[e] = tot;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t off = 0, tiles = 0;
    for (int e = 0; e < p.E_loc; ++e) {
      sh.expert_off[e] = off;
      sh.tile_base[e] = tiles;
      off += sh.expert_tot[e];
      tiles += (sh.expert_tot[e] + BM - 1) / BM;
    }
    sh.expert_off[p.E_loc] = off;
    sh.tile_base[p.E_loc] = tiles;
  }
  __syncthreads();
}

// First slot of every local expert's tokens of route item `item`
// (sh.unit_base): the expert's offset plus its counts in the earlier items.
__device__ __forceinline__ void moe_unit_bases(const MoeParams &p, int item, MoeShared &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int e = wave; e < p.E_loc; e += nw) {
    int32_t before = 0;
    for (int i = lane; i < item; i += 64) before += p.item_cnt[(size_t)i * p.E_loc + e];
    before = wave_inclusive_scan(before);
    if (lane == 63) sh.unit_base[e] = sh.expert_off[e] + before;
  }
  __syncthreads();
}

// The ticket-0 workgroup: the slot offsets as outputs -- expert_offsets, each
// source's first slot per expert (chunk_offsets) and, for the combine, each
// item's base (item_base).  Each wave scans whole experts over the items.
__device__ __forceinline__ void moe_scan(const MoeParams &p, MoeShared &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (threadIdx.x <= (unsigned)p.E_loc) st_through(&p.expert_offsets[threadIdx.x], sh.expert_off[threadIdx.x]);
  for (int e = wave; e < p.E_loc; e += nw) {
    int32_t carry = sh.expert_off[e];
    for (int i0 = 0; i0 < p.n_items; i0 += 64) {
      const int i = i0 + lane;
      const int32_t v = i < p.n_items ? p.item_cnt[(size_t)i * p.E_loc + e] : 0;
      const int32_t incl = wave_inclusive_scan(v);
      const int32_t base = carry + incl - v;
      if (i < p.n_items) {
        if (p.combine) st_through(&p.item_base[(size_t)i * p.E_loc + e], base);
        if (i % p.items_per_src == 0) st_through(&p.chunk_offsets[e * (p.S + 1) + i / p.items_per_src], base);
      }
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) st_through(&p.chunk_offsets[e * (p.S + 1) + p.S], carry);
  }
}

// ---------------------------------------------------------------- land

// Copy every listed row (n rows in sh.list_tok, of route item `item`) from
// its token's row of x to its slot's row of x_slots.  The stores are
// device-scope 8-byte stores, which write through the L2.
//
// A step is 8 rows x 128 8-byte units per row of one wave (two units per
// lane and row); a wave's steps run in a two-deep pipeline: the loads of
// step i + 1 are issued before the stores of step i, so a wait for them
// leaves the stores in flight (a wait for a load also waits for every store
// issued before it).  Row addresses stay in vector registers.  Steps have no
// branches, so the compiler's waits count exactly: the rows past the last
// of a partial group repeat the last row and units past a row's end repeat
// its last unit (the same bytes stored twice to the same place).
__device__ __forceinline__ void moe_copy_rows(const MoeParams &p, const MoeShared &sh, int n, int item) {
  constexpr int RB = 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int sr = item / p.items_per_src;
  const uint64_t *xs = reinterpret_cast<const uint64_t *>(p.x[sr]);
  uint64_t *xd = reinterpret_cast<uint64_t *>(p.x_slots);
  const int t0 = (item - sr * p.items_per_src) * kRouteTokens;
  const int nu = p.H / 4;                     // 8-byte units per row
  const int chunks = (nu + 127) / 128;        // steps per row group
  const int groups = (n + RB - 1) / RB;
  const int steps = groups * chunks;
  const size_t rw = (size_t)p.H / 4;          // units per row
  struct Step {
    const uint64_t *src[RB];
    uint64_t *dst[RB];
    uint64_t a[RB][2];
    int u0, u1;
  };
  auto issue = [&](int st, Step &q) {
    const int g = st / chunks, c = st - g * chunks;
    const int r0 = g * RB;
    q.u0 = min(c * 128 + lane, nu - 1);
    q.u1 = min(c * 128 + 64 + lane, nu - 1);
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int r = min(r0 + j, n - 1);
      const int v = sh.list_tok[r];
      q.src[j] = xs + (size_t)(t0 + (v & 255)) * rw;
      q.dst[j] = xd + (size_t)(v >> 8) * rw;
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      q.a[j][0] = q.src[j][q.u0];
      q.a[j][1] = q.src[j][q.u1];
    }
  };
  auto drain = [&](const Step &q) {
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      st_through(q.dst[j] + q.u0, q.a[j][0]);
      st_through(q.dst[j] + q.u1, q.a[j][1]);
    }
  };
  // this wave's steps are wave + k * nw, k < my; the loop body has no
  // branches (the compiler's waits then leave one step's loads and the
  // previous step's stores in flight), the last one or two steps follow it
  const int my = wave < steps ? (steps - wave + nw - 1) / nw : 0;
  if (my == 0) return;
  Step qa, qb;
  issue(wave, qa);
  int k = 0;
  for (; k + 2 < my; k += 2) {
    issue(wave + (k + 1) * nw, qb);
    drain(qa);
    issue(wave + (k + 2) * nw, qa);
    drain(qb);
  }
  if (k + 1 < my) {
    issue(wave + (k + 1) * nw, qb);
    drain(qa);
    drain(qb);
  } else {
    drain(qa);
  }
}

// Land part `part` of route item `item`: the rows of the item's tokens t
// with t % kLandParts == part that chose local experts and their slot
// metadata, all stored write-through.
__device__ __forceinline__ void moe_land_item(const MoeParams &p, int item, int part, MoeShared &sh) {
  const int s = item / p.items_per_src, b = item % p.items_per_src;
  const int t = b * kRouteTokens + (int)threadIdx.x;
  const int e_lo = p.rank * p.E_loc;
  if (threadIdx.x == 0) sh.n_list = 0;
  moe_unit_bases(p, item, sh);  // ends with a barrier
  if (threadIdx.x < (unsigned)kRouteTokens && t < p.T && (int)threadIdx.x % kLandParts == part) {
    const size_t o = ((size_t)s * p.T + t) * p.top_k;
    for (int j = 0; j < p.top_k; ++j) {
      const int e = p.topk_idx[o + j] - e_lo;
      if (e >= 0 && e < p.E_loc) {
        const int slot = sh.unit_base[e] + p.tok_rank[o + j];
        if (slot < 0 || slot >= p.cap) {  // cannot happen when routing and scan agree
          raise_error(p.sync, kErrInternal, (uint32_t)item);
          continue;
        }
        st_through(&p.slot_token[slot], (int32_t)(s * p.T + t));
        st_through(&p.slot_gate[slot], p.topk_gate[o + j]);
        if (p.combine) st_through(&p.slot_ret[slot], (int32_t)((size_t)(s * p.T + t) * p.top_k + j));
        const int k = atomicAdd(&sh.n_list, 1);
        sh.list_tok[k] = (slot << 8) | (int)threadIdx.x;
      }
    }
  }
  __syncthreads();
  const int n = (int)uniform((uint32_t)sh.n_list);
  moe_copy_rows(p, sh, n, item);
}

// ---------------------------------------------------------------- compute

// Wave 0, every lane: wait for every route item that holds tokens of local
// expert e in slots [slot0, slot1) (expert e's slots start at e_off).  Lane l
// takes items l, l + 64, ...: the wave scans the items' counts of e into
// their slot ranges and each lane whose item's range overlaps the tile's rows
// watches that item's flag; the wave loops until no lane has an item
// pending, so a wait costs one round trip per 64 items rather than one per
// item.
__device__ __forceinline__ bool moe_wait_rows(const MoeParams &p, int e, int e_off, int slot0, int slot1) {
  const int lane = threadIdx.x & 63;
  int32_t carry = e_off;
  for (int i0 = 0; i0 < p.n_items; i0 += 64) {
    const int i = i0 + lane;
    const int32_t cnt = i < p.n_items ? p.item_cnt[(size_t)i * p.E_loc + e] : 0;
    const int32_t incl = wave_inclusive_scan(cnt);
    const int32_t base = carry + incl - cnt;
    carry += __shfl(incl, 63, 64);
    const bool need = cnt > 0 && base < slot1 && base + cnt > slot0;
    const uint32_t *f = flag_ptr(p.sync, (uint32_t)(need ? i : 0));
    if (!wave_spin_all_eq(p.sync, f, need, p.sync.epoch, (uint32_t)i0)) return false;
  }
  return true;
}

// Land unit w of the land queue (route item w / kLandParts, part
// w % kLandParts) and record its arrival: every thread waits for its own
// (write-through) stores, then after the barrier one counter add; the last
// part of the item publishes its flag.
__device__ __forceinline__ void moe_land_and_release(const MoeParams &p, uint32_t w, MoeShared &sh) {
  const uint32_t it = w / kLandParts;
  moe_land_item(p, (int)it, (int)(w % kLandParts), sh);
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) arrive_written_through(p.sync, it, (uint32_t)kLandParts);
}

// Land units of the land queue until none is left.
__device__ __forceinline__ void moe_land_queue(const MoeParams &p, MoeShared &sh) {
  for (;;) {
    const uint32_t it = next_index(&p.sync.ctrl->land_ctr, &sh.word);
    if (it >= (uint32_t)(p.n_items * kLandParts)) break;
    if ((int)it == p.withhold) continue;  // failure tests only
    moe_land_and_release(p, it, sh);
  }
}

// Next grouped-GEMM tile as rt * tiles_n + nb, or -1 when none is left (all
// threads get the value).  XCD x owns the row tiles of local experts
// [x E_loc / 8, (x+1) E_loc / 8), so the tiles one XCD runs at once share
// their expert's weights in its L2; within an XCD every owned row tile of
// n-block 0 comes first, then n-block 1, ...  A workgroup drains its own
// XCD's queue first, then the others in turn.
__device__ __forceinline__ int moe_next_tile(const MoeParams &p, const MoeShared &sh, int xcd, uint32_t *lds_word) {
  __syncthreads();
  if (threadIdx.x == 0) {
    int r = -1;
    for (int k = 0; k < kXcds && r < 0; ++k) {
      const int x = (xcd + k) & (kXcds - 1);
      const int lo = sh.tile_base[x * p.E_loc / kXcds], mc = sh.tile_base[(x + 1) * p.E_loc / kXcds] - lo;
      const uint32_t size = (uint32_t)(mc * p.tiles_n);
      uint32_t *ctr = &p.sync.ctrl->xq[x * 16];
      if (size == 0 || ld_relaxed(ctr) >= size) continue;
      const uint32_t i = add_relaxed(ctr, 1u);
      if (i < size) r = (lo + (int)(i % (uint32_t)mc)) * p.tiles_n + (int)(i / (uint32_t)mc);
    }
    *lds_word = (uint32_t)r;
  }
  __syncthreads();
  return (int)uniform(*lds_word);
}

template <int BM, int BN>
__device__ __forceinline__ void moe_compute(const MoeParams &p, char *smem, MoeShared &sh) {
  if (threadIdx.x < (unsigned)MK_MAX_WORLD) sh.ret_ptr[threadIdx.x] = p.ret[threadIdx.x];
  __syncthreads();
  const int n_row_tiles = (int)uniform((uint32_t)sh.tile_base[p.E_loc]);
  const int ld = p.H * 2;
  const int xcd = xcd_id();
  for (;;) {
    const int t = p.tile_map == kMapBlocks ? moe_next_tile(p, sh, xcd, &sh.word)
                                           : next_tile(p.sync, n_row_tiles, p.tiles_n, xcd, TileOrder{p.tile_map, 1, 1}, &sh.word);
    if (t < 0) break;
    const int rt = (int)t / p.tiles_n, nb = (int)t % p.tiles_n;
    // row tile rt is tile mt of the last expert e whose first row tile is <= rt
    int e = 0;
    for (int x = 1; x < p.E_loc; ++x)
      if ((int)uniform((uint32_t)sh.tile_base[x]) <= rt) e = x;
    const int mt = rt - (int)uniform((uint32_t)sh.tile_base[e]);
    const int slot0 = (int)uniform((uint32_t)sh.expert_off[e]) + mt * BM;
    const int slot1 = min(slot0 + BM, (int)uniform((uint32_t)sh.expert_off[e + 1]));
    if (e >= p.E_loc || slot0 < 0 || slot1 > p.cap || slot1 <= slot0) {
      if (threadIdx.x == 0) raise_error(p.sync, kErrInternal, t);
      break;
    }
    const int n0 = nb * BN;
    bool ok0 = true;
    if (threadIdx.x < 64) ok0 = moe_wait_rows(p, e, (int)uniform((uint32_t)sh.expert_off[e]), slot0, slot1);
    if (!wg_sync_ok(ok0, &sh.word)) break;
    const int valid_n = min(BN, p.N - n0);
    const i32x4_t ra = make_vdesc(p.x_slots + (size_t)slot0 * p.H, (uint32_t)((slot1 - slot0) * ld));
    const i32x4_t rb = make_vdesc(p.wt + ((size_t)e * p.N + n0) * p.H, (uint32_t)(valid_n * ld));
    // the tile's row gates and return positions, for the epilogue
    if (threadIdx.x < (unsigned)BM) {
      const int slot = slot0 + (int)threadIdx.x;
      float g = 1.f;
      int src = -1;
      uint32_t rrow = 0;
      if (slot < slot1) {
        if (!p.no_gate) g = p.slot_gate[slot];
        if (p.combine) {
          const size_t rp = (size_t)p.slot_ret[slot];
          const size_t per_src = (size_t)p.T * p.top_k;
          src = (int)(rp / per_src);
          rrow = (uint32_t)(rp - (size_t)src * per_src);
          if (src == p.rank) src = -1;  // this rank's own tokens stay in y
        }
      }
      sh.tile_gate[threadIdx.x] = g;
      sh.tile_ret_src[threadIdx.x] = src;
      sh.tile_ret_row[threadIdx.x] = rrow;
    }
    AccTile<BM, BN> acc;
    gemm_tile<BM, BN>(smem, ra, rb, ld, p.H, acc);
    // y = bf16(gate * acc) row by row through LDS (whole-row stores); a row
    // of a remote token is also stored to its source's return buffer
    const int rows = slot1 - slot0;
    staged_epilogue<BM, BN>(acc, smem, [&](int r, int cc, const f32x4_t &v) {
      const int col = n0 + cc;
      if (r >= rows || col >= p.N) return;
      const float g = sh.tile_gate[r];
      const uint2 o = p.no_gate ? pack_bf16x4(v[0], v[1], v[2], v[3])
                                : pack_bf16x4(v[0] * g, v[1] * g, v[2] * g, v[3] * g);
      *reinterpret_cast<uint2 *>(p.y + (size_t)(slot0 + r) * p.N + col) = o;
      const int src = sh.tile_ret_src[r];
      if (src >= 0) *reinterpret_cast<uint2 *>(sh.ret_ptr[src] + (size_t)sh.tile_ret_row[r] * p.N + col) = o;
    });
    if (p.combine) {  // count the finished tile for the combine (release of its rows)
      wait_stores();
      __syncthreads();
      if (threadIdx.x == 0) {
        fence_release();
        add_relaxed(&p.sync.ctrl->tiles_done, 1u);
      }
    }
  }
}

// ---------------------------------------------------------------- combine

constexpr int kCombineTokens = 16;  // tokens per combine item
static_assert(kCombineTokens * 8 <= TileCfg<128, 128>::THREADS, "one thread per (token, k) row");
static_assert(kCombineTokens * 8 * sizeof(void *) <= TileCfg<128, 128>::LDS_BYTES, "row table fits");

// Combine tokens [c*16, c*16+16) of the local source: out[t] = bf16(sum over
// k of row k), row k from y when the token's k-th expert is local and from
// y_peer otherwise.  The rows' addresses go to LDS first (rows[t][k]); then
// every thread takes 8 columns of a token and issues its top_k loads together.
__device__ __forceinline__ void moe_combine_item(const MoeParams &p, int c, char *smem) {
  const uint16_t **rows = reinterpret_cast<const uint16_t **>(smem);
  const int t0 = c * kCombineTokens, nt = min(kCombineTokens, p.T - t0);
  const int K = p.top_k;
  const int i = (int)threadIdx.x;
  if (i < nt * K) {
    const int t = t0 + i / K, k = i % K;
    const size_t o = ((size_t)p.rank * p.T + t) * K + k;
    const int e = p.topk_idx[o] - p.rank * p.E_loc;
    if (e >= 0 && e < p.E_loc) {
      const int item = p.rank * p.items_per_src + t / kRouteTokens;
      const int slot = p.item_base[(size_t)item * p.E_loc + e] + p.tok_rank[o];
      rows[i] = p.y + (size_t)slot * p.N;
    } else {
      rows[i] = p.y_peer + ((size_t)t * K + k) * p.N;
    }
  }
  __syncthreads();
  const int vpr = p.N / 8;  // 16-byte vectors per row
  for (int idx = i; idx < nt * vpr; idx += blockDim.x) {
    const int tl = idx / vpr, cv = idx - tl * vpr;
    u32x4_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < K) v[k] = *reinterpret_cast<const u32x4_t *>(rows[tl * K + k] + cv * 8);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k >= K) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += __uint_as_float(v[k][q] << 16);
        acc[2 * q + 1] += __uint_as_float(v[k][q] & 0xFFFF0000u);
      }
    }
    uint4 r;
    const uint2 lo = pack_bf16x4(acc[0], acc[1], acc[2], acc[3]);
    const uint2 hi = pack_bf16x4(acc[4], acc[5], acc[6], acc[7]);
    r.x = lo.x; r.y = lo.y; r.z = hi.x; r.w = hi.y;
    *reinterpret_cast<uint4 *>(p.out + (size_t)(t0 + tl) * p.N + cv * 8) = r;
  }
  __syncthreads();  // rows[] is rewritten by the next item
}

// Every workgroup, after its other roles: wait until every tile is done,
// then combine token chunks of the local source until none are left.  The
// GEMM staging area is free by then and holds the row addresses.
__device__ __forceinline__ void moe_combine(const MoeParams &p, MoeShared &sh, char *smem) {
  Ctrl *ctrl = p.sync.ctrl;
  const uint32_t n_items = (uint32_t)((p.T + kCombineTokens - 1) / kCombineTokens);
  bool waited = false;
  for (;;) {
    const uint32_t c = next_index(&ctrl->combine_ctr, &sh.word);
    if (c >= n_items) break;
    if (!waited) {
      bool ok0 = true;
      if (threadIdx.x == 0) {
        // every tile's rows, and the ticket-0 workgroup's item bases
        const uint32_t n_tiles = (uint32_t)sh.tile_base[p.E_loc] * (uint32_t)p.tiles_n;
        ok0 = spin_until_ge(p.sync, &ctrl->tiles_done, n_tiles, 0xFFFF0003u) &&
              spin_until_eq(p.sync, &ctrl->scan_ready, p.sync.epoch, 0xFFFF0002u);
      }
      if (!wg_sync_ok(ok0, &sh.word)) break;  // full acquire: rows of every tile are visible
      waited = true;
    }
    moe_combine_item(p, (int)c, smem);
  }
}

// ---------------------------------------------------------------- kernel

template <int BM, int BN>
__global__ __launch_bounds__((TileCfg<BM, BN>::THREADS), 1) void moe_kernel(MoeParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[TileCfg<BM, BN>::LDS_BYTES];
  __shared__ MoeShared sh;
  const uint32_t ticket = take_ticket(p.sync, &sh.word);
  Ctrl *ctrl = p.sync.ctrl;
  copy_params(&sh.prm, p);

  // route: every workgroup takes route items until none are left
  for (;;) {
    const uint32_t it = next_index(&ctrl->route_ctr, &sh.word);
    if (it >= (uint32_t)p.n_items) break;
    moe_route_item(p, (int)it, sh);
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) add_relaxed(&ctrl->route_done, 1u);  // the outputs were written through
  }

  // every workgroup: wait until every route item is counted, then the
  // offsets into LDS
  bool ok0 = true;
  if (threadIdx.x == 0) ok0 = spin_until_ge(p.sync, &ctrl->route_done, (uint32_t)p.n_items, 0xFFFF0001u);
  const bool ok = wg_sync_ok(ok0, &sh.word);
  if (ok) moe_offsets<BM>(p, sh);
  if (ok && ticket == 0) {
    moe_scan(p, sh);
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) st_through(&ctrl->scan_ready, p.sync.epoch);
  }
  if (ok && ticket < (uint32_t)(p.n_land + p.n_compute)) {
    // Every workgroup lands route items until none is left, then takes
    // tiles until none is left (land workgroups too, unless the roles are
    // static), then combines.  A workgroup waiting in the combine has seen
    // the tile queue empty, so every tile belongs to a running workgroup:
    // the combine's wait needs no co-residency.
    moe_land_queue(p, sh);
    if (ticket >= (uint32_t)p.n_land || !p.static_roles) moe_compute<BM, BN>(sh.prm, smem, sh);
    if (p.combine) moe_combine(p, sh, smem);
  }
  finish_launch(p.sync);
}

hipError_t launch_moe(const MoeParams &p, int bm, int grid, hipStream_t s) {
  if (bm == 256)
    hipLaunchKernelGGL((moe_kernel<256, 256>), dim3(grid), dim3(TileCfg<256, 256>::THREADS), 0, s, p);
  else
    hipLaunchKernelGGL((moe_kernel<128, 128>), dim3(grid), dim3(TileCfg<128, 128>::THREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t occupancy_moe(int bm, int *blocks_per_cu) {
  const void *f = bm == 256 ? (const void *)moe_kernel<256, 256> : (const void *)moe_kernel<128, 128>;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
      blocks_per_cu, f, bm == 256 ? TileCfg<256, 256>::THREADS : TileCfg<128, 128>::THREADS, 0);
}

}  // namespace mk

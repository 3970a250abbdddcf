/*
 * mk.h -- C ABI of libmk, persistent fused communication + GEMM kernels for
 * AMD Instinct MI355X (gfx950).
 *
 * What the operations compute follows the mKernel articles:
 *   [P1] German article on mKernel (chatgpz.de), table "Die fuenf
 *        verschmolzenen Kerne" (the five fused kernels), and section "Was
 *        mKernel macht" (persistent kernel whose CTAs assign themselves
 *        roles; compute and communication overlap at tile/chunk granularity).
 *   [P3] Romanian article (world.tibi.club), section "Cum functioneaza? O
 *        privire sub capota" (reduce, broadcast and scatter in one kernel).
 *
 * Scope.  Each call runs ONE GPU's share of a collective-fused GEMM.  The
 * other ranks are emulated: their contributions are buffers that already
 * exist, either in device memory (a separate HBM region) or in pinned host
 * memory (hipHostMalloc) that the kernel reads or writes over PCIe.  Every
 * pointer argument may be either kind unless stated; the library classifies
 * each one with hipPointerGetAttributes.  Pageable host memory is rejected.
 *
 * Execution model.  Every operation is ONE persistent kernel launch on the
 * caller's stream.  Each workgroup takes a ticket from a device counter and
 * becomes a LAND workgroup (copies incoming chunks, then release-stores a
 * per-chunk ready flag), a COMPUTE workgroup (bf16 MFMA GEMM tiles, started
 * as soon as the flags of their rows are seen with acquire semantics), or
 * (GEMM+RS and GEMM+AR) a REDUCE workgroup (sums the peers' partials of a
 * tile into the workspace and release-stores the tile's flag; the tile's
 * epilogue adds that sum).  Role counts are tunable per operation
 * (mk_set_roles).  Every in-kernel wait is bounded by
 * mk_config.spin_timeout_ms; on expiry the kernel records MK_ERR_TIMEOUT,
 * every workgroup leaves its loop and the launch completes.
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as pointers to their 16-bit patterns (mk_bf16);
 *     fp32 tensors as float*.  All matrices are row-major and contiguous.
 *   - Matrix B of a GEMM C = A @ B is passed TRANSPOSED as bt = B^T, shape
 *     [N, K], K contiguous (the layout of a linear layer's weight).
 *   - K and N must be multiples of 8 and every pointer 16-byte aligned.
 *   - Accumulation is fp32; outputs are rounded to bf16 to nearest even.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronise the device.  Buffers must stay valid
 *     until the stream's work completes.  The caller owns every buffer it
 *     passes; the library owns only what mk_create allocates.
 *   - One handle serves one stream at a time: its flags and counters are
 *     per handle, so calls on one handle must be stream-ordered.
 *   - Argument errors return MK_ERR_INVALID / MK_ERR_UNSUPPORTED before
 *     anything is launched.  Launch failures return MK_ERR_HIP.  Device-side
 *     timeouts are reported by mk_sync as MK_ERR_TIMEOUT.
 *   - Every buffer is checked for being non-NULL, 16-byte aligned, on the
 *     handle's device (or pinned host memory where allowed), and for ending
 *     inside the runtime allocation it starts in, given the byte size its
 *     shape implies (MK_ERR_INVALID otherwise; mk_last_error names it).  A
 *     caching allocator's blocks are sub-ranges of larger allocations, so a
 *     buffer that is too short but ends inside such an allocation is not
 *     detected: sizes remain the caller's responsibility.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mk_ctx *mk_handle;
typedef uint16_t mk_bf16; /* bit pattern of a bfloat16 value */
typedef void *mk_stream;  /* hipStream_t */

#define MK_MAX_WORLD 16

typedef enum {
  MK_OK = 0,
  MK_ERR_INVALID = 1,     /* bad argument; nothing launched */
  MK_ERR_UNSUPPORTED = 2, /* device is not gfx950, or a shape the kernels do not support */
  MK_ERR_OOM = 3,         /* device allocation failed */
  MK_ERR_HIP = 4,         /* a HIP runtime call failed (see mk_last_error) */
  MK_ERR_TIMEOUT = 5      /* an in-kernel wait expired; outputs of that call are undefined */
} mk_status;

typedef enum {
  MK_OP_AG_GEMM = 0,
  MK_OP_GEMM_RS = 1,
  MK_OP_GEMM_AR = 2,
  MK_OP_MOE = 3,
  MK_OP_RING_ATTN = 4,
  MK_OP_COUNT = 5
} mk_op;

typedef struct {
  int device;             /* HIP device ordinal the handle is bound to */
  int spin_timeout_ms;    /* bound on every in-kernel wait; <= 0 selects 2000 ms */
  unsigned flags;         /* reserved, must be 0 */
  size_t workspace_bytes; /* device workspace the handle owns, allocated by mk_create and
                             never grown by a call; 0 selects 128 MiB.  Users: the MoE
                             dispatch (about 16 bytes per routed slot plus 8 per
                             (token, k) pair), ring attention (66.5 KiB per (head,
                             128-query tile) pair), the GEMM+RS reduce role ([m/W, n]
                             fp32) and the GEMM+AR reduce role ([m, n] fp32).  A call
                             that needs more returns MK_ERR_INVALID before launching. */
} mk_config;

/* Workgroup role counts of one persistent launch.  A negative value selects
 * the library's default for that role; n_compute = 0 runs only the data
 * movement (transfer alone: the outputs then do not hold the operation's
 * result).
 *   n_land    AG+GEMM, MoE and ring attention: workgroups that copy incoming
 *             chunks (the AG, MoE and ring attention launches also let
 *             compute workgroups land while their rows are missing)
 *   n_reduce  GEMM+RS and GEMM+AR only (MK_ERR_INVALID elsewhere):
 *             workgroups that sum the peers' partials of the rows the tiles
 *             reduce into the workspace, one tile-sized item at a time, each
 *             released by a flag; a tile's epilogue then adds that sum
 *             instead of reading every peer.  Reduce workgroups run tiles
 *             once every item is claimed (not with MK_F_STATIC_ROLES).
 *             Default 0: the tile epilogues read the peers themselves.
 *             With n_compute = 0 the reduce workgroups (default: the whole
 *             grid) move the reduce and scatter bytes alone: bf16 of the
 *             peers' sum to c_own / c and the broadcast buffers, zeros to
 *             the RS outboxes. */
typedef struct {
  int n_land;
  int n_compute;
  int n_reduce;
} mk_roles;

/* Per-call option bits. */
#define MK_F_PRELANDED 0x1u /* AG: a_gathered already holds the gathered A; ring attention: the
                               receive buffers hold every block; skip landing (compute alone) */
#define MK_F_NO_GATE 0x2u   /* MoE: store x @ W_e without the gate factor */
#define MK_F_STATIC_ROLES 0x4u /* AG, RS, AR, MoE: every workgroup keeps its ticket role for the
                                 whole launch (by default AG compute workgroups land chunks while
                                 their rows are missing, and land and reduce workgroups run
                                 tiles once their queue is empty) */
#define MK_F_NO_PEERS 0x8u     /* RS, AR: compute alone -- the epilogues leave out the peers'
                                 partials (c_own = bf16 of this rank's own rows, c = bf16(A @ B));
                                 peer_part is not read and may hold NULL entries.  For timing
                                 the GEMM with its output traffic. */

/* Create a handle on cfg->device: checks the device is gfx950, allocates the
 * control block (tickets, counters, per-chunk flags, error record) and the
 * workspace (cfg->workspace_bytes).  No kernel runs.  This is the only call
 * that allocates device memory (mk_destroy frees it).  *out is set only on
 * MK_OK; MK_ERR_OOM if an allocation fails. */
mk_status mk_create(mk_handle *out, const mk_config *cfg);

/* Free everything mk_create allocated.  The caller must have synchronised
 * every stream the handle was used on. */
mk_status mk_destroy(mk_handle h);

/* Set / query the role counts used by later calls of operation `op`.
 * mk_get_roles reports the values as set (negative = default). */
mk_status mk_set_roles(mk_handle h, mk_op op, const mk_roles *roles);
mk_status mk_get_roles(mk_handle h, mk_op op, mk_roles *roles);

/* Roles the last launch of `op` actually used (after defaults and clamping),
 * and its grid size.  MK_ERR_INVALID if `op` was never launched. */
mk_status mk_last_launch(mk_handle h, mk_op op, mk_roles *roles, int *grid);

/* Synchronise `stream`, then read and clear the device error record.
 * Returns MK_ERR_TIMEOUT if a launch since the previous mk_sync timed out. */
mk_status mk_sync(mk_handle h, mk_stream stream);

const char *mk_status_string(mk_status s);
/* Text of the last host-side error on this handle ("" if none). */
const char *mk_last_error(mk_handle h);

/*
 * AllGather + GEMM  [P1, row "AllGather + GEMM"]:
 *   every rank holds a shard of A; the shards are gathered and
 *   C = concat_rows(shard_0, ..., shard_{W-1}) @ B.
 *
 *   world      W, 1 <= W <= MK_MAX_WORLD;  rank: this rank, 0 <= rank < W
 *   a_shards   host array of W pointers; a_shards[q] is shard q, [m_s, k] bf16.
 *              a_shards[rank] is local device memory; the others are the
 *              emulated peers (device or pinned host memory).
 *   bt         B^T, [n, k] bf16, device memory
 *   c          output [W*m_s, n] bf16; row block q is shard q's product
 *   a_gathered output [W*m_s, k] bf16, device memory: the gathered A (the
 *              landing buffer).  With MK_F_PRELANDED it is an input instead.
 *   m_s >= 1, n >= 8, k >= 8.
 */
mk_status mk_ag_gemm(mk_handle h, mk_stream stream, int world, int rank,
                     const mk_bf16 *const *a_shards, const mk_bf16 *bt, mk_bf16 *c,
                     mk_bf16 *a_gathered, int m_s, int n, int k, unsigned flags);

/*
 * AllGather + GEMM that allocates nothing -- for callers that cannot call
 * hipMalloc: code under HIP graph capture, tight serving loops, harnesses
 * that forbid device allocation.  Computes exactly what mk_ag_gemm computes
 * (same arguments, same outputs, same kernels) with the library's default
 * schedule, but needs no handle: the control block, ready flags and arrival
 * counters live in one fixed array of the library on each device (260 KiB,
 * held by every GPU the library runs on until the process ends; 2048 ready
 * flags, the landing blocks are made coarser until they fit).  The caller
 * passes inputs and outputs only.
 *
 *   Runs on the current device (hipSetDevice) and on `stream`: a small
 *   kernel clears the array's control block and this call's flags, then the
 *   fused kernel runs, then (status != NULL) a one-thread kernel writes
 *   status[0] = the launch's result (MK_OK, or MK_ERR_TIMEOUT when an
 *   in-kernel wait expired) and status[1] = its detail.  No call allocates
 *   or frees memory or synchronises; the device's first call looks up the
 *   array's address.
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents: calls that overlap on one GPU (two streams, or two host
 *   threads) race and give undefined results -- order them on one stream.
 *   status   optional device memory, int32[2], 16-byte aligned
 *   flags    MK_F_PRELANDED, MK_F_STATIC_ROLES
 *   Errors as mk_ag_gemm (MK_ERR_INVALID / MK_ERR_UNSUPPORTED before
 *   anything is launched; MK_ERR_UNSUPPORTED also for a device that is not
 *   gfx950); there is no handle, so no error text.
 */
mk_status mk_ag_gemm_noalloc(mk_stream stream, int world, int rank, const mk_bf16 *const *a_shards,
                             const mk_bf16 *bt, mk_bf16 *c, mk_bf16 *a_gathered, int m_s, int n, int k,
                             unsigned flags, int32_t *status);

/*
 * GEMM + ReduceScatter  [P1, row "GEMM + ReduceScatter"]:
 *   P = A @ B ([m, n] fp32); with slices of ms = m / W rows, this rank keeps
 *   c_own = bf16(P[slice rank] + sum over q != rank of peer_part[q]) and
 *   forwards outbox[q] = bf16(P[slice q]) for every q != rank.
 *
 *   a          [m, k] bf16 device memory;  bt: [n, k] bf16 device memory
 *   peer_part  host array of W pointers; peer_part[q] (q != rank) is rank q's
 *              fp32 partial of THIS rank's slice, [ms, n]; entry [rank] ignored
 *   c_own      output [ms, n] bf16
 *   outbox     host array of W pointers; outbox[q] (q != rank) receives
 *              [ms, n] bf16; entry [rank] ignored
 *   m must be a multiple of W.
 *   flags: MK_F_NO_PEERS (compute alone), MK_F_STATIC_ROLES.
 *   Reduce role (mk_set_roles n_reduce > 0): needs [m/W, n] fp32 of workspace.
 */
mk_status mk_gemm_rs(mk_handle h, mk_stream stream, int world, int rank, const mk_bf16 *a,
                     const mk_bf16 *bt, const float *const *peer_part, mk_bf16 *c_own,
                     mk_bf16 *const *outbox, int m, int n, int k, unsigned flags);

/*
 * GEMM + AllReduce  [P1, row "GEMM + AllReduce"; P3, reduce + broadcast]:
 *   c = bf16(A @ B + sum over q != rank of peer_part[q]) (fp32 sums), written
 *   to c and to every broadcast buffer bcast[0..n_bcast-1] (bit-identical).
 *
 *   peer_part  host array of W pointers, each [m, n] fp32; entry [rank] ignored
 *   c          output [m, n] bf16;  bcast: host array of n_bcast pointers,
 *              each [m, n] bf16;  0 <= n_bcast <= MK_MAX_WORLD
 *   flags: MK_F_NO_PEERS (compute alone), MK_F_STATIC_ROLES.
 *   Reduce role (mk_set_roles n_reduce > 0): needs [m, n] fp32 of workspace.
 */
mk_status mk_gemm_ar(mk_handle h, mk_stream stream, int world, int rank, const mk_bf16 *a,
                     const mk_bf16 *bt, const float *const *peer_part, mk_bf16 *c,
                     mk_bf16 *const *bcast, int n_bcast, int m, int n, int k, unsigned flags);

/*
 * MoE dispatch + grouped GEMM  [P1, row "MoE-Versand + GEMM"]:
 *   tokens of every source rank are routed to their top_k experts; those
 *   routed to this rank's experts land directly in per-expert slots and are
 *   multiplied by their expert's weight as they land.
 *
 *   Routing (per token, bit-exact): the top_k experts by logit, descending,
 *   the lower expert id first among equal logits; gate = softmax over all E
 *   logits (fp32) at that expert, not renormalised.  This rank owns experts
 *   rank*E_loc .. rank*E_loc+E_loc-1.  Slots are ordered by (local expert,
 *   source, token); nothing is dropped.
 *
 *   n_src      S source ranks (1..MK_MAX_WORLD); x_src[s]: [T, H] bf16 tokens of
 *              source s (s = rank is local, the others emulated peers)
 *   logits_src host array of S pointers, each [T, E] fp32
 *   wt         expert weights transposed, [E_loc, N, H] bf16 device memory
 *              (wt[e] = W_e^T for W_e of shape [H, N])
 *   y          output [cap, N] bf16; rows [0, n_slots) are
 *              bf16(gate * (x_slot @ W_e)) (no gate with MK_F_NO_GATE)
 *   topk_idx   output [S*T, top_k] int32 (global expert ids); row s*T + t
 *   topk_gate  output [S*T, top_k] fp32
 *   slot_token output [cap] int32: s*T + t of every slot
 *   expert_offsets output [E_loc+1] int32: first slot of each local expert;
 *              expert_offsets[E_loc] = n_slots
 *   chunk_offsets  output [E_loc, S+1] int32: first slot of source s within
 *              expert e; chunk_offsets[e][S] = expert_offsets[e+1]
 *   x_slots    output [cap, H] bf16 device memory: the landed token rows
 *   cap        rows of y, slot_token and x_slots; must be >= S*T*min(top_k, E_loc)
 *   flags      MK_F_NO_GATE, MK_F_STATIC_ROLES (land workgroups do not take
 *              tiles; by default every workgroup lands, then takes tiles)
 *   1 <= top_k <= 8, top_k <= E <= 256, E_loc >= 1, rank*E_loc + E_loc <= E,
 *   H and N multiples of 8.
 */
mk_status mk_moe_dispatch_gemm(mk_handle h, mk_stream stream, int n_src, int rank,
                               const mk_bf16 *const *x_src, const float *const *logits_src,
                               const mk_bf16 *wt, int T, int H, int N, int E, int E_loc,
                               int top_k, mk_bf16 *y, int32_t *topk_idx, float *topk_gate,
                               int32_t *slot_token, int32_t *expert_offsets,
                               int32_t *chunk_offsets, mk_bf16 *x_slots, int cap,
                               unsigned flags);

/*
 * MoE dispatch + grouped GEMM + combine  [P1, row "MoE-Versand + GEMM"; the
 * return trip is this library's reading, the pages name only the dispatch]:
 *   everything mk_moe_dispatch_gemm does (same arguments, same outputs), and
 *   in the same launch:
 *   - return: every finished row y[slot] whose token came from a source
 *     s != rank is also written to ret[s] at row (t * top_k + k), k being the
 *     place of the slot's expert in token t's top-k list (bit-identical to
 *     y[slot]); other rows of ret[s] are left untouched;
 *   - combine: once every tile is done, for this rank's own tokens
 *     out[t] = bf16(sum over k of v_k) with fp32 sums, v_k = y[slot] when
 *     expert k of token t is local and y_peer[t * top_k + k] otherwise.
 *
 *   y_peer  [T * top_k, N] bf16: the rows the owners of this rank's remote
 *           experts returned (rows of local experts are not read)
 *   ret     host array of S pointers; ret[s] (s != rank) is source s's
 *           return buffer, [T * top_k, N] bf16; entry [rank] ignored; may be
 *           NULL when S == 1
 *   out     output [T, N] bf16
 *   rank < n_src (source `rank` holds this rank's own tokens).
 *   MK_F_NO_GATE is rejected (MK_ERR_INVALID): the combine sums gated rows.
 *   The grid is capped at what is resident at once, since every workgroup
 *   waits for the last tile before it combines.
 */
mk_status mk_moe_dispatch_gemm_combine(mk_handle h, mk_stream stream, int n_src, int rank,
                                       const mk_bf16 *const *x_src, const float *const *logits_src,
                                       const mk_bf16 *wt, int T, int H, int N, int E, int E_loc,
                                       int top_k, mk_bf16 *y, int32_t *topk_idx, float *topk_gate,
                                       int32_t *slot_token, int32_t *expert_offsets,
                                       int32_t *chunk_offsets, mk_bf16 *x_slots, int cap,
                                       const mk_bf16 *y_peer, mk_bf16 *const *ret, mk_bf16 *out,
                                       unsigned flags);

/*
 * Ring attention  [P1, table "Die fuenf verschmolzenen Kerne", ring attention
 * row: the ring KV exchange and the local attention in one persistent kernel]:
 *   this rank's queries attend to the keys and values of every rank's block,
 *   the blocks taken in ring order (step s: the block of rank (rank - s) mod
 *   W), with softmax over all W * S_kv keys (no causal mask):
 *     o   = bf16(softmax(q k^T * scale) v)      fp32 accumulation, online softmax
 *     lse = max + log(sum exp(s - max))         natural log, fp32, per query row
 *   The land role copies every block into the receive buffers, K as is and V
 *   transposed, and releases one flag per chunk of keys; attention tiles start
 *   as soon as their chunk has landed.
 *
 *   q        [B*H, S_q, D] bf16 device memory (D = 128)
 *   k_src    host array of W pointers, each [B*H, S_kv, D] bf16: rank r's keys
 *            (r = rank local; the others emulated peers, device or pinned host)
 *   v_src    the same for the values
 *   o        output [B*H, S_q, D] bf16;  lse: output [B*H, S_q] fp32
 *   k_recv   output [W, B*H, S_kv, D] bf16 device memory: every block by source
 *            rank, as received
 *   vt_recv  output [W, B*H, D, S_kv] bf16 device memory: every value block,
 *            transposed
 *   scale    score factor (1/sqrt(D) is the usual choice)
 *   Supported: D = 128, S_kv a multiple of 64, S_q >= 1, B*H >= 1.  Other
 *   shapes return MK_ERR_UNSUPPORTED.
 *   MK_F_PRELANDED: k_recv / vt_recv already hold every block (attention
 *   alone); k_src / v_src are not read and may be NULL.
 */
mk_status mk_ring_attention(mk_handle h, mk_stream stream, int world, int rank, const mk_bf16 *q,
                            const mk_bf16 *const *k_src, const mk_bf16 *const *v_src, int BH,
                            int S_q, int S_kv, int D, float scale, mk_bf16 *o, float *lse,
                            mk_bf16 *k_recv, mk_bf16 *vt_recv, unsigned flags);

/*
 * Measurement aid (not part of the fused path): a loop of independent bf16
 * 32x32x16 MFMAs with no memory traffic on 2 workgroups of 256 threads per CU,
 * 8 accumulators per wave, iters rounds of 8 MFMAs (32768 FLOP each) per wave:
 * 2 * cu_count * 4 waves * iters * 8 * 32768 FLOP in all.  Timing it gives the
 * practical dense bf16 MFMA ceiling the fused kernels are compared with.
 *   sink   device memory of at least 256 floats (written, values meaningless)
 *   1 <= iters <= 2^24
 */
mk_status mk_mfma_ceiling(mk_handle h, mk_stream stream, int iters, float *sink);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */

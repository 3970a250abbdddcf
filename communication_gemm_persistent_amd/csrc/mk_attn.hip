// Persistent fused ring attention: the ring KV exchange and a
// FlashAttention-style online-softmax attention in one launch.
//
// [P1] German article on mKernel (chatgpz.de), table "Die fuenf
// verschmolzenen Kerne", ring attention row: sequence-parallel attention in
// which, at every step, a KV block moves one rank along the ring while the
// local attention consumes the block received before; compute and the ring
// transfer run at the same time inside one persistent kernel.
//
// Roles (atomic tickets):
//   land     copies every rank's KV block into this rank's receive buffers in
//            ring order (at step s the block of rank (rank - s) mod W), a
//            chunk of keys at a time: K as it is, V transposed (keys
//            contiguous, the layout the P V product reads); then releases
//            the chunk's flag.  Land workgroups run tasks when done (unless
//            the launch only lands).
//   compute  takes (batch*head, 128-query tile) tasks.  For every ring step
//            and every 64-key tile of that step's block it waits for the
//            tile's chunk, stages K and V^T in LDS (DMA, double-buffered) and
//            runs S = Q K^T, the online softmax and O += P V on the matrix
//            cores; O is divided by the softmax denominator at the end and
//            stored with each row's log-sum-exp.
//
// Every wave owns 32 query rows (two 16-row blocks) and all 128 columns of
// the head.  S comes out of the 16x16x32 MFMA with each lane holding 4
// S columns of one query row (LDS K rows 16 kb + 4 g .. +3); the P V product
// takes P from those registers directly: within every 32-row step, lane
// group g supplies LDS rows 4g..4g+3 and 16+4g..16+4g+3 as its 8 K slots.
// The K tile is staged with its keys permuted so that those 8 rows hold 8
// consecutive keys (LDS row 32 kk + 16 h + 4 g + s holds key
// 32 kk + 8 g + 4 h + s): the matching V^T values are then one 16-byte LDS
// read, and the sum over K slots is the sum over keys.
#include "mk_params.h"

namespace mk {

constexpr int kAttnQ = 128;        // query rows per task
constexpr int kAttnKT = 64;        // keys per tile
constexpr int kAttnThreads = 256;  // 4 waves
// LDS stage: the K tile as two halves [64 keys x 64 d] (8 KB each), then the
// V^T tile [128 d x 64 keys] (16 KB); 128-byte rows whose 16-byte chunks are
// XOR-swizzled by (row >> 1) & 7, as in the GEMM tiles.
constexpr int kAttnKHalf = kAttnKT * 128;
constexpr int kAttnVOff = 2 * kAttnKHalf;
constexpr int kAttnStage = kAttnVOff + kAttnD * 128;
constexpr int kAttnLds = 2 * kAttnStage;
// workspace slot of a (bh, qt) pair: unnormalised O [128][128], row max, row sum
constexpr int kAttnSlot = kAttnQ * kAttnD + 2 * kAttnQ;
static_assert(kAttnD == 128, "the task layout assumes 128-wide heads");


// ---------------------------------------------------------------- land

// Land item i: ring step s = i / (BH * chunks), source rank (rank - s) mod W,
// then (batch*head, chunk).  Returns the flag index of the chunk.
__device__ __forceinline__ uint32_t attn_flag(const AttnParams &p, int src, int bh, int c) {
  return (uint32_t)((src * p.BH + bh) * p.chunks + c);
}

__device__ __forceinline__ void attn_land_item(const AttnParams &p, int item) {
  const int per_step = p.BH * p.chunks;
  const int s = item / per_step, rem = item % per_step;
  const int src = (p.rank - s + p.world) % p.world;
  const int bh = rem / p.chunks, c = rem % p.chunks;
  const int key0 = c * p.chunk_keys, nk = min(p.chunk_keys, p.S_kv - key0);
  const int tid = threadIdx.x;
  // K: the chunk's rows are contiguous in both buffers
  {
    const u32x4_t *sp = reinterpret_cast<const u32x4_t *>(p.k_src[src] + ((size_t)bh * p.S_kv + key0) * kAttnD);
    u32x4_t *dp = reinterpret_cast<u32x4_t *>(p.k_recv + (((size_t)src * p.BH + bh) * p.S_kv + key0) * kAttnD);
    const int n16 = nk * (kAttnD / 8);
    int i = tid;
    for (; i + 3 * kAttnThreads < n16; i += 4 * kAttnThreads) {
      const u32x4_t a0 = sp[i], a1 = sp[i + kAttnThreads], a2 = sp[i + 2 * kAttnThreads],
                    a3 = sp[i + 3 * kAttnThreads];
      dp[i] = a0; dp[i + kAttnThreads] = a1; dp[i + 2 * kAttnThreads] = a2; dp[i + 3 * kAttnThreads] = a3;
    }
    for (; i < n16; i += kAttnThreads) dp[i] = sp[i];
  }
  // V: transposed in registers, one 8-key x 8-d block per thread and step:
  // eight 16-byte loads (one key's 8 d values each, 16 threads per 256-byte
  // key row) become eight 16-byte rows of V^T (8 keys each) by byte
  // permutes -- the low halves of two keys' words form one d row, the high
  // halves the next
  const uint16_t *vsrc = p.v_src[src] + ((size_t)bh * p.S_kv + key0) * kAttnD;
  uint16_t *vdst = p.vt_recv + ((size_t)src * p.BH + bh) * kAttnD * p.S_kv + key0;
  const int nblk = (nk / 8) * (kAttnD / 8);
#pragma unroll 2
  for (int b = tid; b < nblk; b += kAttnThreads) {
    const int kg = b / (kAttnD / 8), dg = b % (kAttnD / 8);
    u32x4_t in[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      in[i] = *reinterpret_cast<const u32x4_t *>(vsrc + (size_t)(kg * 8 + i) * kAttnD + dg * 8);
#pragma unroll
    for (int cw = 0; cw < 4; ++cw) {  // word cw holds d = 8 dg + 2 cw (low half) and + 1 (high half)
      u32x4_t lo, hi;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lo[q] = __builtin_amdgcn_perm(in[2 * q + 1][cw], in[2 * q][cw], 0x05040100u);
        hi[q] = __builtin_amdgcn_perm(in[2 * q + 1][cw], in[2 * q][cw], 0x07060302u);
      }
      *reinterpret_cast<u32x4_t *>(vdst + (size_t)(dg * 8 + 2 * cw) * p.S_kv + kg * 8) = lo;
      *reinterpret_cast<u32x4_t *>(vdst + (size_t)(dg * 8 + 2 * cw + 1) * p.S_kv + kg * 8) = hi;
    }
  }
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) st_release(flag_ptr(p.sync, attn_flag(p, src, bh, c)), p.sync.epoch);
}

// ---------------------------------------------------------------- compute

__device__ __forceinline__ float xor_max(float v, int m) {
  return fmaxf(v, __shfl_xor(v, m, 64));
}

__device__ __forceinline__ bf16x8_t pack_p(const f32x4_t &a, const f32x4_t &b) {
  const uint2 lo = pack_bf16x4(a[0], a[1], a[2], a[3]);
  const uint2 hi = pack_bf16x4(b[0], b[1], b[2], b[3]);
  u32x4_t w;
  w[0] = lo.x; w[1] = lo.y; w[2] = hi.x; w[3] = hi.y;
  return __builtin_bit_cast(bf16x8_t, w);
}

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t &a, const bf16x8_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One task: query tile qt of batch*head bh over ring tiles [j0, j1) (tile j:
// ring step j / tiles-per-block, key tile j % tiles-per-block).  With one
// split the task covers the whole ring and stores o and lse; with two, the
// halves of a (bh, qt) pair combine through the workspace (attn_merge).
__device__ __forceinline__ bool attn_task(const AttnParams &p, int bh, int qt, int j0, int j1,
                                          char *smem, uint32_t *s_word) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int row0 = qt * kAttnQ + wave * 32;  // this wave's first query row
  const int tpb = p.S_kv / kAttnKT;          // tiles per block
  const uint32_t base = lds_addr(smem);
  const int ldk = kAttnD * 2, ldv = p.S_kv * 2;

  // Q fragments (kept for the whole task): rows r16 of each 16-row block,
  // d = 32 ks + 8 g .. +7; rows past S_q are zeros
  bf16x8_t qf[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int row = row0 + mb * 16 + r16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row < p.S_q)
        v = *reinterpret_cast<const u32x4_t *>(p.q + ((size_t)bh * p.S_q + row) * kAttnD + ks * 32 + g * 8);
      qf[mb][ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // O in oacc[mb][0..7]; oacc[mb][8] is the P row sum: the P V product's
  // ninth d-block multiplies P by a block of ones, so the sum comes out of the
  // matrix core (of the bf16 P the O rows are built from), is rescaled with
  // O, and every lane holds its query row's sum
  f32x4_t oacc[2][9];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int db = 0; db < 9; ++db) oacc[mb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY};  // running row max (log2 domain)
  const bf16x8_t ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};

  // DMA lane offsets (8-row groups, 64-wide rows, swizzled as the GEMM tiles).
  // K: LDS row 8 gl + rs (rs = lane >> 3) holds key kperm(gl) + 8 (rs >> 2) + (rs & 3)
  // (the permutation above); the swizzle follows the LDS row
  const int rs = lane >> 3;
  const uint32_t lane_off_k[2] = {(uint32_t)((8 * (rs >> 2) + (rs & 3)) * ldk + dma_chunk(lane, 0) * 16),
                                  (uint32_t)((8 * (rs >> 2) + (rs & 3)) * ldk + dma_chunk(lane, 1) * 16)};
  auto kperm = [](int gl) { return 32 * (gl >> 2) + 16 * (gl & 1) + 4 * ((gl >> 1) & 1); };
  const uint32_t lane_off_v[2] = {(uint32_t)((lane >> 3) * ldv + dma_chunk(lane, 0) * 16),
                                  (uint32_t)((lane >> 3) * ldv + dma_chunk(lane, 1) * 16)};
  const int lane_c8[2] = {dma_chunk(lane, 0) * 8, dma_chunk(lane, 1) * 8};
  // this wave's DMAs of a tile: K half (wave >> 1), row groups 4 (wave & 1) ..
  // +3; V^T row groups 4 wave .. +3.  K and V^T of tile t go to the K and V
  // parts of stage t & 1, K one tile ahead of V (see the loop below).
  // Ring position of a tile, advanced tile by tile so the loop divides
  // nothing: tile j is key tile kt = j % tpb of ring step j / tpb, whose
  // source rank is (rank - step) mod W; landing chunk c = kt / tpc holds it
  // (tile kc = kt % tpc of the chunk)
  const int tpc = p.chunk_keys / kAttnKT;
  struct Pos {
    int kt, c, kc;
    int src;
  };
  auto pos_of = [&](int j) {
    Pos q;
    const int step = j / tpb;
    q.kt = j - step * tpb;
    q.c = q.kt / tpc;
    q.kc = q.kt - q.c * tpc;
    q.src = p.rank - step < 0 ? p.rank - step + p.world : p.rank - step;
    return q;
  };
  auto advance = [&](Pos &q) {
    ++q.kt;
    if (++q.kc == tpc) {
      q.kc = 0;
      ++q.c;
    }
    if (q.kt == tpb) {  // next ring step: the previous rank's block
      q.kt = q.c = q.kc = 0;
      q.src = q.src == 0 ? p.world - 1 : q.src - 1;
    }
  };
  const size_t blk_k = (size_t)p.S_kv * kAttnD;  // elements of one (rank, bh) block
  auto stage_k = [&](const Pos &q, int buf) {
    const i32x4_t vk = make_vdesc(p.k_recv + ((size_t)q.src * p.BH + bh) * blk_k, (uint32_t)(p.S_kv * ldk));
    const uint32_t st = base + buf * kAttnStage;
    const int half = wave >> 1;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int gl = 4 * (wave & 1) + d;  // row group within the tile
      const uint32_t uni = (uint32_t)__builtin_amdgcn_readfirstlane((q.kt * kAttnKT + kperm(gl)) * ldk + half * 128);
      dma16(vk, __builtin_amdgcn_readfirstlane(st + half * kAttnKHalf + gl * 1024), lane_off_k[gl & 1] + uni);
    }
  };
  auto stage_v = [&](const Pos &q, int buf) {
    const i32x4_t vv = make_vdesc(p.vt_recv + ((size_t)q.src * p.BH + bh) * blk_k, (uint32_t)(kAttnD * ldv));
    const uint32_t st = base + buf * kAttnStage;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int gl = 4 * wave + d;
      dma_row_group(vv, st + kAttnVOff + gl * 1024, lane_off_v[gl & 1], lane_c8[gl & 1], ldv,
                    q.kt * kAttnKT, p.S_kv, gl);
    }
  };
  // wait for the chunk holding a tile (once per chunk)
  int have = -1;
  auto acquire = [&](const Pos &q) -> bool {
    const int id = q.src * p.chunks + q.c;
    if (id == have || p.prelanded) return true;
    have = id;
    bool ok0 = true;
    const uint32_t f = attn_flag(p, q.src, bh, q.c);
    if (threadIdx.x == 0) ok0 = spin_until_eq(p.sync, flag_ptr(p.sync, f), p.sync.epoch, f);
    return wg_sync_ok(ok0, s_word, !p.light_acquire);
  };
  // S = Q K^T of the K tile in stage buf: s[mb][kb] lane (g, r16): query
  // 16 mb + r16, LDS K rows 16 kb + 4 g + 0..3
  auto qk = [&](f32x4_t (&s)[2][4], int buf) {
    const char *st = smem + buf * kAttnStage;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[mb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = (ks & 1) * 4 + g;  // logical chunk of the 128-byte row
      const char *kh = st + (ks >> 1) * kAttnKHalf + ((c ^ ((lane >> 1) & 7)) << 4);
      bf16x8_t kf[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kf[kb] = *reinterpret_cast<const bf16x8_t *>(kh + (kb * 16 + r16) * 128);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) s[mb][kb] = mfma16(kf[kb], qf[mb][ks], s[mb][kb]);
    }
  };

  // row max of S (log2 domain) over the wave's 4 lane groups: the scale is
  // positive, so the max is taken over the raw scores and scaled once
  const float c = p.scale_log2;
  auto row_max = [&](const f32x4_t (&s)[2][4], float (&m)[2]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[mb][kb][r]);
      m[mb] = xor_max(xor_max(mx, 16), 32) * c;
    }
  };

  // Software pipeline: iteration j computes S of tile j + 1 while it runs
  // the exponentials of tile j (the MFMAs of one and the vector instructions
  // of the other interleave), then O += P V of tile j while it takes the row
  // max of tile j + 1.  LDS holds K(j+1) and V(j) during iteration j, while
  // K(j+2) and V(j+1) land.  The acquires come before any DMA of the
  // iteration is issued, so a failed wait returns with nothing in flight.
  Pos p1 = pos_of(j0), p2 = p1;
  advance(p2);
  if (!acquire(p1)) return false;
  if (j0 + 1 < j1 && !acquire(p2)) return false;
  stage_k(p1, j0 & 1);
  stage_v(p1, j0 & 1);
  if (j0 + 1 < j1) stage_k(p2, (j0 + 1) & 1);
  advance(p1);  // from here on, in iteration j: p1 is tile j + 1, p2 tile j + 2
  advance(p2);
  wait_vmcnt<0>();
  wg_barrier();
  f32x4_t sacc[2][4];
  float tmax[2];  // row max of the tile in sacc
  qk(sacc, j0 & 1);
  row_max(sacc, tmax);
  for (int j = j0; j < j1; ++j) {
    // every wave is done with K(j) (read for S(j)) and V(j - 1); this wave's
    // DMAs of K(j+1) and V(j) have landed (waited for below, or in the prologue)
    wg_barrier();
    if (j + 2 < j1) {
      if (!acquire(p2)) return false;
      stage_k(p2, j & 1);
    }
    if (j + 1 < j1) stage_v(p1, (j + 1) & 1);
    advance(p1);
    advance(p2);
    // the running max; when no row's max grows, alpha is exactly 1 for every
    // row of the wave and the rescale of O is skipped (the same bits)
    float mnew[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const float mold = mrow[mb];
      mnew[mb] = fmaxf(mold, tmax[mb]);
      mrow[mb] = mnew[mb];
      if (__any(mnew[mb] > mold)) {
        const float alpha = __builtin_amdgcn_exp2f(mold - mnew[mb]);
#pragma unroll
        for (int db = 0; db < 9; ++db) {
          oacc[mb][db][0] *= alpha; oacc[mb][db][1] *= alpha;
          oacc[mb][db][2] *= alpha; oacc[mb][db][3] *= alpha;
        }
      }
    }
    // S of tile j + 1 (in the last iteration a product of stale LDS data,
    // never used: the stage is in-bounds and nothing is landing in it) and
    // P = exp2(s scale_log2 - m) of tile j: one fma and one exp2 per score
    f32x4_t snext[2][4];
    qk(snext, (j + 1) & 1);
    bf16x8_t pf[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[mb][kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mb][kb][r], c, -mnew[mb]));
      pf[mb][0] = pack_p(sacc[mb][0], sacc[mb][1]);
      pf[mb][1] = pack_p(sacc[mb][2], sacc[mb][3]);
    }
    // O += P V: V^T row d = 16 db + r16, K slots = keys 32 kk + 8 g .. +7
    // (16-byte chunk 4 kk + g of the row); then the row max of tile j + 1
    const char *vt = smem + (j & 1) * kAttnStage + kAttnVOff;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const char *vrow = vt + (db * 16 + r16) * 128;
      const int swz = (lane >> 1) & 7;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8_t vf = *reinterpret_cast<const bf16x8_t *>(vrow + (((4 * kk + g) ^ swz) << 4));
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) oacc[mb][db] = mfma16(vf, pf[mb][kk], oacc[mb][db]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) oacc[mb][8] = mfma16(ones, pf[mb][kk], oacc[mb][8]);
    row_max(snext, tmax);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sacc[mb][kb] = snext[mb][kb];
    wait_vmcnt<0>();  // this wave's DMAs of K(j+2) and V(j+1)
  }
  wg_barrier();  // both buffers are free for the next task
  // the row sums (every lane holds its row's); then store, or combine with
  // the other half
  float lrow[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) lrow[mb] = oacc[mb][8][0];
  if (p.splits == 2) {
    // (bh, qt) pair: the first half to finish writes its unnormalised O, row
    // max and row sum and releases the pair's flag; the second combines.
    const uint32_t pair = (uint32_t)(qt * p.BH + bh);
    const uint32_t f = p.merge_flag0 + pair;
    float *slot = p.ws + (size_t)pair * kAttnSlot;
    bool first = false;
    if (threadIdx.x == 0) first = add_acq_rel(cnt_ptr(p.sync, f), 1u) == 0u;
    first = wg_broadcast(first, s_word);
    if (first) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int lr = wave * 32 + mb * 16 + r16;  // row within the tile
#pragma unroll
        for (int db = 0; db < 8; ++db)
          *reinterpret_cast<f32x4_t *>(slot + lr * kAttnD + db * 16 + 4 * g) = oacc[mb][db];
        if (g == 0) {
          slot[kAttnQ * kAttnD + lr] = mrow[mb];
          slot[kAttnQ * kAttnD + kAttnQ + lr] = lrow[mb];
        }
      }
      wait_stores();
      __syncthreads();
      if (threadIdx.x == 0) st_release(flag_ptr(p.sync, f), p.sync.epoch);
      return true;
    }
    bool ok0 = true;
    if (threadIdx.x == 0) {
      st_relaxed(cnt_ptr(p.sync, f), 0u);  // for the next launch
      ok0 = spin_until_eq(p.sync, flag_ptr(p.sync, f), p.sync.epoch, f);
    }
    if (!wg_sync_ok(ok0, s_word, !p.light_acquire)) return false;
    // combine: the same operations whichever half finished first (products
    // then one commutative add, no contraction into fma), so the bits do not
    // depend on the order
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma clang fp contract(off)
      const int lr = wave * 32 + mb * 16 + r16;
      const float mo = slot[kAttnQ * kAttnD + lr], lo = slot[kAttnQ * kAttnD + kAttnQ + lr];
      const float m = fmaxf(mrow[mb], mo);
      const float a = __builtin_amdgcn_exp2f(mrow[mb] - m), b = __builtin_amdgcn_exp2f(mo - m);
      const float l = lrow[mb] * a + lo * b;
      const float inv = 1.f / l;
      const int row = qt * kAttnQ + lr;
      if (row < p.S_q) {
        uint16_t *orow = p.o + ((size_t)bh * p.S_q + row) * kAttnD;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const f32x4_t w = *reinterpret_cast<const f32x4_t *>(slot + lr * kAttnD + db * 16 + 4 * g);
          const f32x4_t v = oacc[mb][db];
          float x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = (v[r] * a + w[r] * b) * inv;
          *reinterpret_cast<uint2 *>(orow + db * 16 + 4 * g) = pack_bf16x4(x[0], x[1], x[2], x[3]);
        }
        if (g == 0) p.lse[(size_t)bh * p.S_q + row] = (m + __log2f(l)) * 0.69314718055994530942f;
      }
    }
    return true;
  }
  // O / l, lse = (m + log2 l) ln 2
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const float l = lrow[mb];
    const float inv = 1.f / l;
    const int row = row0 + mb * 16 + r16;
    if (row < p.S_q) {
      uint16_t *orow = p.o + ((size_t)bh * p.S_q + row) * kAttnD;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const f32x4_t v = oacc[mb][db];
        *reinterpret_cast<uint2 *>(orow + db * 16 + 4 * g) = pack_bf16x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      }
      if (g == 0) p.lse[(size_t)bh * p.S_q + row] = (mrow[mb] + __log2f(l)) * 0.69314718055994530942f;
    }
  }
  return true;
}

// Next task of the XCD-blocked order as (bh, half, qt), or bh = -1 when none
// is left (all threads get the value).  XCD x owns heads [x BH / 8,
// (x+1) BH / 8); its queue runs half by half, and within a half head by
// head with the query tiles of a head consecutive, so the tasks an XCD runs
// at once share the fewest K and V^T streams in its L2.  A workgroup drains
// its own XCD's queue first, then the others in turn.
__device__ __forceinline__ int attn_next_task(const AttnParams &q, int xcd, uint32_t *lds_word, int *half,
                                              int *qt) {
  __syncthreads();
  if (threadIdx.x == 0) {
    int r = -1;
    for (int k = 0; k < kXcds && r < 0; ++k) {
      const int x = (xcd + k) & (kXcds - 1);
      const int lo = x * q.BH / kXcds, mc = (x + 1) * q.BH / kXcds - lo;
      const uint32_t size = (uint32_t)(mc * q.splits * q.q_tiles);
      uint32_t *ctr = &q.sync.ctrl->xq[x * 16];
      if (size == 0 || ld_relaxed(ctr) >= size) continue;
      const uint32_t i = add_relaxed(ctr, 1u);
      if (i < size) {
        const int per_half = mc * q.q_tiles;
        const int hf = (int)i / per_half, rem = (int)i % per_half;
        r = ((lo + rem / q.q_tiles) * q.splits + hf) * q.q_tiles + rem % q.q_tiles;
      }
    }
    *lds_word = (uint32_t)r;
  }
  __syncthreads();
  const int r = (int)uniform(*lds_word);
  if (r >= 0) {
    *qt = r % q.q_tiles;
    *half = (r / q.q_tiles) % q.splits;
  }
  return r < 0 ? -1 : r / (q.q_tiles * q.splits);
}

template <int DUMMY>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[kAttnLds];
  __shared__ uint32_t s_word;
  // the task loop reads its parameters from an LDS copy: LDS reads are
  // reloaded where they are used, so no parameter stays live in (spilled)
  // scalar registers around the tile loop's DMAs
  __shared__ AttnParams s_prm;
  copy_params(&s_prm, p);  // take_ticket's barrier publishes the copy
  const uint32_t ticket = take_ticket(p.sync, &s_word);
  Ctrl *ctrl = p.sync.ctrl;
  if (ticket < (uint32_t)p.n_land) {
    for (;;) {
      const uint32_t it = next_index(&ctrl->land_ctr, &s_word);
      if (it >= (uint32_t)p.n_items) break;
      attn_land_item(p, (int)it);
    }
  }
  // land workgroups join once landing is done, unless the launch lands only
  const AttnParams &q = s_prm;
  if (ticket < (uint32_t)q.n_compute + (q.n_compute > 0 ? (uint32_t)q.n_land : 0u)) {
    for (;;) {
      // Every first half before any second half: the first round covers the
      // early ring steps, and the late steps have longer to land; the tasks
      // running together consume the ring's blocks in the order they land.
      // By default each XCD takes a block of heads and runs a head's query
      // tiles together (attn_next_task), so they stream the same K and V^T
      // tiles through one L2; the global order (MK_TILE_MAP=0) runs the
      // query tiles of every head at once over the whole chip.
      int bh, qt, half;
      if (q.tile_map == kMapGlobal) {
        const uint32_t t = next_index(&q.sync.ctrl->tile_ctr, &s_word);
        if (t >= (uint32_t)q.n_tasks) break;
        half = (int)(t / (uint32_t)q.n_pairs);
        const int pair = (int)(t % (uint32_t)q.n_pairs);
        bh = pair % q.BH;
        qt = pair / q.BH;
      } else {
        bh = attn_next_task(q, xcd_id(), &s_word, &half, &qt);
        if (bh < 0) break;
      }
      const int n_tiles = q.world * (q.S_kv / kAttnKT);
      const int j0 = half * n_tiles / q.splits, j1 = (half + 1) * n_tiles / q.splits;
      if (!attn_task(p, bh, qt, j0, j1, smem, &s_word)) break;
    }
  }
  finish_launch(p.sync);
}

hipError_t launch_attn(const AttnParams &p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_kernel<0>), dim3(grid), dim3(kAttnThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t occupancy_attn(int *blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, attn_kernel<0>, kAttnThreads, 0);
}

}  // namespace mk

// One ring step of the forward pass, bf16 inputs, fp32 accumulation, head dim 128, on the
// gfx950 matrix cores.
//
// What one step computes (page 1, "Blockwise Attention and Online Softmax Formulations";
// page 4, "Incremental Blockwise Attention"): for every query row of the resident shard,
// softmax attention against the keys of ONE KV shard, keeping a running maximum m, a
// running sum l and an unnormalised output O while walking the shard's keys tile by tile,
// then O / l and LSE = m + ln l.  The epilogue either writes that partial or merges it into
// the running (O, LSE) of earlier ring steps (page 2, "FlashAttention Integration").
//
// Mapping onto CDNA4:
//  * On gfx950 the vector unit of a SIMD runs one wave's softmax while the matrix unit runs
//    another wave's products.  A wave's own independent vector instructions also run under
//    its matrix instructions, but its softmax is a chain of dependent instructions whose
//    stalls only another wave can fill; measured, whole alternating phases take fewer
//    cycles per tile than each wave interleaving its own softmax with its products.  So a
//    workgroup is 8 wave64s, two per SIMD, in two groups that swap roles every half step (a
//    "ping-pong"): while group 0 issues its matrix phase (P V of the previous key tile and
//    Q K^T of the current one), group 1 runs the softmax of its current tile, and the other
//    way round in the next half step.  A workgroup barrier separates the half steps.
//  * Each wave owns 32 query rows of one head; the workgroup's waves share one KV head.
//    With grouped-query attention the query heads of a KV group go to different waves
//    (page 3, section 2: several query heads share one KV group), so every K/V tile staged
//    in LDS feeds up to 4 heads.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (A = K rows
//    from LDS, B = Q^T held in VGPRs for the whole kernel).  In the 32x32 accumulator layout
//    lane l then holds 16 keys of ONE query (column l % 32), so the row max and row sum are
//    per-lane reductions plus one exchange with lane l ^ 32 (v_permlane32_swap).
//  * The probabilities never leave registers: the score accumulator, rounded to bf16, is
//    exactly the B operand (P^T) of the second product O^T += V^T P^T, because the order
//    in which the contraction visits keys is free as long as A and B agree.
//  * Online softmax in base 2 with scale * log2(e) folded into one FMA per score.  The
//    running maximum m only has to keep the weights 2^(s - m) finite, not at most 1: the
//    final O / l is the same in exact arithmetic for any m.  So most tiles exponentiate
//    against m as it stands, without computing their own maximum, and check afterwards
//    that the tile's weights stayed small (row-sum share <= 2^24); only a tile that fails
//    the check, or a row without a maximum yet, takes the maximum and rescales, and then
//    lazily: m moves only when the new maximum exceeds it by more than TAU = 8.  The
//    softmax is the vector-unit bound of the kernel (the SIMD's vector issue is shared
//    with the matrix instructions of the other wave), so every instruction saved counts.
//  * Causal masking (page 1, "Causal Masking Dynamics"): with positions increasing inside
//    every shard, the allowed keys of a row are a prefix [0, limit) of the KV shard, so a
//    wave skips every key tile at or beyond its largest limit, runs maskless below its
//    smallest limit, and masks only the diagonal tiles in between.
//  * Key tiles of 64 keys (96 for long shards) rotate through three LDS stages each and are
//    staged by DMA (buffer_load ... lds): no VGPRs and no vector instructions.  Each wave's
//    share of a tile is BN/16 loads of 1 KB (group 0 V tiles, group 1 K tiles): half at the
//    start of its softmax phase and half at the start of its next matrix phase, which
//    balances the two phases; it waits for them at the end of the softmax phase after that.
//    V is stored row-major and read with the gfx950 transposing LDS load, which yields the
//    V^T operand directly.
//  * Workgroups are launched heaviest query block first (causal work grows with the query
//    position), with the KV head as the fastest-varying index so that neighbouring
//    workgroups, dispatched round-robin over the 8 XCDs, put each KV head's tiles into
//    one XCD's L2.
#include <atomic>
#include <algorithm>
#include <functional>
#include <mutex>
#include <queue>
#include <type_traits>
#include <vector>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;            // head dimension
// Keys per tile: 64, or 96 for long shards.  A wider tile spreads each phase's fixed costs
// (barriers, ballots, the first operand reads, dependency gaps) over more keys but costs 24
// more VGPRs and 48 KB more LDS (144 KB in all), and rounds short causal shards' work up to
// coarser tiles: measured on MI355X, 96 keys are 0.5-0.6 % faster per ring pass at L = 32768,
// equal at L = 8192 and 1-3 % slower at L <= 4096.
constexpr int BN_SHORT = 64;
constexpr int BN_LONG = 96;
constexpr int LONG_TILES_MIN_L = 16384;
constexpr int QW = 32;            // query rows per wave
constexpr int WAVES = 8;          // two per SIMD
constexpr int THREADS = 64 * WAVES;
constexpr int ROW_BYTES = D * 2;  // one key's K or V row: 256 B, sixteen 16-byte chunks
constexpr float TAU = 8.0f;       // lazy-rescale threshold, log2 units
constexpr int PREFETCH = 2;       // matrix-phase operand slots read ahead

template <int S>
struct Stage {
  static constexpr int value = S;
};
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float lane_pair_max(float x) {
  // max of this lane's value and lane (l ^ 32)'s value, in every lane
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lane_pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier without a memory fence: the compiler may not move memory operations
// across it, but no wait for outstanding loads is emitted.  Every LDS read issued before
// it has been consumed by a matrix instruction (so has completed), and DMA writes into
// LDS are waited for explicitly by the waves that issued them.
__device__ __forceinline__ void barrier_no_fence() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// BATCH: the workgroup walks the KV shards of `sb` one after the other (several ring steps in
// one launch), carrying its online-softmax state (m, l, O) from one shard's keys to the next,
// and merges or writes once at the end.  Otherwise the one KV shard of `a`.
template <int MODE, int BN, bool BATCH>
__global__ __launch_bounds__(THREADS, 1) void step_fwd_bf16_kernel(StepArgs a, int heads_per_wg,
                                                                  int n_qb, int inner_count, SplitPlan plan,
                                                                  ShardBatch sb) {
  static_assert(BN % 32 == 0 && BN >= 64, "tiles of whole 32-key blocks, at least two");
  constexpr int NB = BN / 32;       // 32-key blocks per tile: score accumulators
  constexpr int NCH = BN / 16;      // 16-key chunks per tile: P operands of P V
  constexpr int SLOTS = BN / 4;     // matrix-phase slots of two products (NCH x 4 = NB x 8)
  constexpr int LOADS_W = BN / 16;  // 1 KB DMA loads per wave and tile (BN / 4 over 4 waves)
  constexpr int LOADS_HALF = LOADS_W / 2;   // issued in the softmax phase; the rest in the next matrix phase
  constexpr int TILE_BYTES = BN * ROW_BYTES;   // written by BN / 4 DMA loads of 1 KB
  __shared__ __attribute__((aligned(1024))) char k_lds[3][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds[3][TILE_BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int group = wave >> 2;                                  // 0 or 1
  const int lane = tid & 63;
  const int lq = lane & 31;   // query column of the 32x32 accumulators
  const int lg = lane >> 5;   // which half of the accumulator's key rows

  const int L = a.L;
  const int G = a.h / a.n_kv;
  const int Hw = heads_per_wg;          // heads per workgroup (4, 2 or 1)
  const int PB = WAVES / Hw;            // 32-row query blocks per workgroup
  const int inner = blockIdx.x % inner_count;
  const int item = blockIdx.x / inner_count;
  int qb, part;                         // heaviest query block first
  split_item(plan, n_qb, item, qb, part);
  const bool split_blk = qb >= plan.split_from;
  const int g = inner % a.n_kv;
  const int bi = (inner / a.n_kv) % a.b;
  const int hs = inner / (a.n_kv * a.b);
  const int hq = g * G + hs * Hw + (wave % Hw);
  const int t0_wg = qb * QW * PB;
  const int t0 = t0_wg + (wave / Hw) * QW;
  const int t = t0 + lq;                // this lane's query row

  const __bf16* qp = (const __bf16*)a.q;
  const int64_t kv_base = ((int64_t)bi * L * a.n_kv + g) * D;
  const int n_shards = BATCH ? sb.n : 1;

  // ---- key ranges and tile ranges of a KV shard ----------------------------------------
  // Row t may attend to the keys [lo, hi) of the KV shard (a prefix when documents are
  // not packed).  Both bounds are nondecreasing in t, so a wave's tile range comes from its
  // first and last valid rows: tiles before wave_first or from wave_tiles on are skipped,
  // tiles in [full_begin, full_end) need no mask, the rest are masked.
  const bool packed = a.doc_begin != nullptr;
  int kv_shard = a.kv_shard;
  auto range = [&](int row) {
    int64_t db = 0, de = 0;
    if (packed) {
      db = a.doc_begin[(int64_t)bi * L + row];
      de = a.doc_end[(int64_t)bi * L + row];
    }
    return key_range(a.causal, a.layout, a.N, L, a.q_shard, kv_shard, row, packed, db, de);
  };
  int lim = 0, lo = 0, wave_first = 0, wave_tiles = 0, full_begin = 0, full_end = 0;
  int j_begin = 0, n_tiles = 0;     // the workgroup's key tiles: [j_begin, n_tiles)
  // the workgroup's tile range in shard s (with a split block: this item's half of it)
  auto wg_tiles = [&](int s) {
    int tg = t0_wg;
    if (BATCH) {
      kv_shard = ((a.q_shard - (sb.k_first + s)) % a.N + a.N) % a.N;
      __asm__ volatile("" : "+s"(tg));
    }
    j_begin = n_tiles = 0;
    if (tg < L) {
      j_begin = range(tg).lo / BN;
      n_tiles = (range(min(tg + QW * PB - 1, L - 1)).hi + BN - 1) / BN;
    }
    j_begin = __builtin_amdgcn_readfirstlane(j_begin);
    n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);
    if (split_blk) {
      const int j_mid = j_begin + (n_tiles - j_begin + 1) / 2;
      if (part == 0) n_tiles = j_mid;
      else j_begin = j_mid;
    }
  };
  // the rest of shard s's ranges: this lane's keys and this wave's tile classes.  In a batch
  // the rows pass through an empty asm, so that nothing of the range computation is hoisted
  // out of the shard loop into registers held through the tile loop.
  auto row_tiles = [&]() {
    int tl = t, tw = t0;
    if (BATCH) __asm__ volatile("" : "+v"(tl), "+s"(tw));
    const KeyRange rr = tl < L ? range(tl) : KeyRange{0, 0};
    lim = rr.hi;
    lo = rr.lo;
    wave_first = wave_tiles = full_begin = full_end = 0;
    if (tw < L) {
      const KeyRange r0 = range(tw), r1 = range(min(tw + QW - 1, L - 1));
      wave_first = r0.lo / BN;
      wave_tiles = (r1.hi + BN - 1) / BN;
      full_begin = (r1.lo + BN - 1) / BN;
      full_end = r0.hi / BN;
    }
    wave_first = __builtin_amdgcn_readfirstlane(wave_first);
    wave_tiles = __builtin_amdgcn_readfirstlane(wave_tiles);
    full_begin = __builtin_amdgcn_readfirstlane(full_begin);
    full_end = __builtin_amdgcn_readfirstlane(full_end);
    if (split_blk) {
      wave_first = max(wave_first, j_begin);
      wave_tiles = min(wave_tiles, n_tiles);
    }
  };
  bool any_tiles = false;
  int anchor_tile = -1;             // (batch) the wave's first tile of a shard after the first
  if (BATCH) {
    for (int s = 0; s < n_shards; ++s) {
      wg_tiles(s);
      any_tiles = any_tiles || n_tiles > j_begin;
    }
  } else {
    wg_tiles(0);
    row_tiles();
    any_tiles = n_tiles > j_begin;
  }
  // the accumulator this item writes, and (first step only) the second accumulator's LSE
  // where no second item covers the rows: chosen here, so only these stay live in the loop
  float* const o_dst = part ? a.o2 : a.o;
  float* const l_dst = part ? a.lse2 : a.lse;
  float* const l2_empty = (MODE == MODE_PART && !split_blk) ? a.lse2 : nullptr;
  // This lane's half of row t, head hq: elements 32 e + 8 ib + 4 lg + x.  On the last step
  // of a pass (o_out set) the rows go to the output instead of the accumulator, rounded to
  // nearest even, and rows this step leaves alone are copied over, cast.
  auto row_offset = [&]() { return (((int64_t)bi * L + t) * a.h + hq) * D + 4 * lg; };
  auto cast_row = [&](int64_t off, int e, int ib, const f32x4& v) __attribute__((always_inline)) {
    *(bf16x4*)(a.o_out + off + 32 * e + 8 * ib) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  };
  // no row of the workgroup sees a key of the shard(s): merging would leave (O, LSE) as it is
  if (MODE == MODE_MERGE && !any_tiles) {
    if (a.o_out && t < L) {
      const int64_t off = row_offset();
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) cast_row(off, e, ib, *(const f32x4*)(o_dst + off + 32 * e + 8 * ib));
    }
    return;
  }

  // ---- Q^T operand, resident for the whole kernel -------------------------------------
  // Rows past the shard end read row L-1 instead: they are never stored, and their key
  // limit of 0 masks every score.  (All global loads of this kernel are branch-free.)
  bf16x8 qop[D / 16];
  {
    const __bf16* row = qp + (((int64_t)bi * L + min(t, L - 1)) * a.h + hq) * D + lg * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qop[kk] = *(const bf16x8*)(row + kk * 16);
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e) acc[e] = f32x16{};
  f32x16 sc[NB];
  bf16x8 pb[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) pb[c] = bf16x8{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.scale * LOG2E;

  // ---- tile staging: global -> LDS by DMA (buffer_load ... lds, 16 B per lane) -----------
  // A K or V tile is BN rows of 256 B; DMA load i (1 KB) fills rows 4i..4i+3, lane l
  // writing slot l: row 4i + l/16, slot position l%16.  Each lane picks which global
  // 16-byte chunk lands in its slot, which gives the swizzles the readers need:
  //   K: chunk c of row r sits at position c ^ (r & 15)   (16 rows, same chunk: 16 banks)
  //   V: chunk c of row r sits at position c ^ 4 (r & 3)  (transposed reads, see below)
  // Wave w of a group issues loads i = w, w+4, w+8, ... of a tile, so the row bits
  // that enter the swizzle are fixed per lane and the lane's byte offset is one register.
  // The buffer descriptor covers exactly rows 0..L-1 of this (batch, KV head), so rows
  // past the shard end fail the hardware range check and arrive as zeros (always masked).
  const unsigned row_stride = (unsigned)a.n_kv * D * 2;   // bytes between keys in HBM
  const int num_records = (int)((unsigned)(L - 1) * row_stride + ROW_BYTES);
  dma_rsrc k_rsrc = make_dma_rsrc((const __bf16*)(BATCH ? sb.k : a.k) + kv_base, (unsigned)num_records);
  dma_rsrc v_rsrc = make_dma_rsrc((const __bf16*)(BATCH ? sb.v : a.v) + kv_base, (unsigned)num_records);
  const int ws = wave & 3;
  const unsigned lrow = lane >> 4;                       // row within a 1 KB load
  const unsigned k_dma_off = lrow * row_stride + (unsigned)((lane & 15) ^ ((4 * ws + lrow) & 15)) * 16;
  const unsigned v_dma_off = lrow * row_stride + (unsigned)((lane & 15) ^ (4 * lrow)) * 16;
  auto issue_tile_dma = [&](dma_rsrc rsrc, unsigned dst, unsigned off, int j) {
#pragma unroll
    for (int t = 0; t < LOADS_W; ++t) {
      const int i = ws + 4 * t;
      dma16_to_lds(rsrc, dst + 1024 * i, off, (unsigned)(j * BN + 4 * i) * row_stride);
    }
  };
  // In the main loop each wave issues the first half of its share of a tile at the start of
  // its softmax phase and the second half at the start of its next matrix phase (an LDS-DMA
  // load costs the issuing wave ~45-55 cycles in either phase; the split balances them:
  // -2 % cycles per tile against all four in the softmax phase).  (Measured against this:
  // the loads between the exponential chains, 11 % slower; all four in the matrix phase,
  // 4 % slower.)  Group 0 stages V tiles, group 1 K tiles.  Loads of tiles past the wave's
  // last one point beyond the buffer (zeros, no memory traffic) into a stage nobody reads
  // again, so every phase issues exactly LOADS_HALF loads and the waits can count them.
  dma_rsrc my_rsrc = group ? k_rsrc : v_rsrc;
  const unsigned my_dma_off = group ? k_dma_off : v_dma_off;
  const unsigned my_lds = group ? RA_LDS_ADDR(k_lds) : RA_LDS_ADDR(v_lds);
  auto issue_one = [&](int tile, int stage, int t) {
    const int i = ws + 4 * t;
    const unsigned soff = tile < n_tiles ? (unsigned)(tile * BN + 4 * i) * row_stride : 0x80000000u;
    dma16_to_lds(my_rsrc, my_lds + (unsigned)(stage * TILE_BYTES + 1024 * i), my_dma_off, soff);
  };

  // ---- the two phases of one wave ------------------------------------------------------
  // K operand of d-step kk, key sub-tile jj: row 32jj + lq, chunk 2kk + lg (16 B).  The
  // swizzled position depends on kk and the lane only, so the eight offsets are kept.
  unsigned k_off[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    k_off[kk] = (unsigned)lq * ROW_BYTES + (unsigned)(((2 * kk + lg) ^ (lq & 15)) * 16);
  auto k_operand = [&](const char* kt, int kk, int jj) {
    return *(const bf16x8*)(kt + k_off[kk] + jj * 32 * ROW_BYTES);
  };
  // V^T operand of key chunk c (16 keys) and d-tile e, read with ds_read_b64_tr_b16: in
  // each 16-lane group the lanes' 8-byte pieces form a 4 x 16 array whose column i goes
  // to lane i.  Lane j of a group points at row k0 + j/4, d = d0 + 4 (j%4); lane i then
  // receives V[k0 .. k0+3][d0 + i], i.e. four consecutive keys of one d, which is the A
  // operand of O^T = V^T P^T (m = d, k = key).  Two reads give the lane's eight keys,
  // 16c + 4lg + {0..3} and 16c + 8 + 4lg + {0..3}: the same key order as the lane's P
  // values in the score accumulator.  With the V swizzle the 16-lane group's four rows
  // (r & 3 = j/4) land in disjoint bank ranges.
  const int g16 = lane >> 4, j16 = lane & 15, jq = j16 >> 2;
  unsigned v_off[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e) {
    const int low = 2 * (g16 & 1) + ((j16 & 3) >> 1);            // chunk within the 4 of tile e
    v_off[e] = (unsigned)(4 * lg + jq) * ROW_BYTES + (unsigned)((4 * (e ^ jq) + low) * 16) +
               (unsigned)((j16 & 1) * 8);
  }
  auto v_operand = [&](const char* vt, int c, int e) {
    const char* base = vt + v_off[e] + 16 * c * ROW_BYTES;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4*)(base));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4*)(base + 8 * ROW_BYTES));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // Matrix phase of step j: O^T += V(j-1)^T P(j-1)^T and S^T(j) = K(j) Q^T, interleaved one
  // MFMA of each per slot (6 independent accumulators), each slot's two LDS operands
  // fetched two slots ahead.  The same code runs at every step so that the accumulators
  // keep one home: where the wave has no tile j-1, P is zero (the V buffer holds finite
  // data: a real tile, or zeros before the first); where it has no tile j, the scores
  // are computed from whatever K buffer is there and never used.
  auto matrix_phase = [&](int j, auto stage_c) __attribute__((always_inline)) {
    constexpr int stage = decltype(stage_c)::value;     // compile-time: LDS addresses fold
    // the second half of the tile whose first half the previous softmax phase loaded:
    // group 0 V(j) into this step's stage, group 1 K(j+2) into the stage of K(j-1)
    const bool dma_now = j > j_begin;
    const int dma_tile_idx = group ? j + 2 : j;
    constexpr int dma_stage_g0 = stage, dma_stage_g1 = (stage + 2) % 3;
    const char* vt = v_lds[(stage + 2) % 3];            // V(j-1)
    const char* kt = k_lds[stage];                      // K(j)
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) sc[jj] = f32x16{};
    bf16x8 va[PREFETCH + 1], ka[PREFETCH + 1];
#pragma unroll
    for (int x = 0; x < PREFETCH; ++x) {
      va[x] = v_operand(vt, x >> 2, x & 3);
      ka[x] = k_operand(kt, x / NB, x % NB);
    }
    // Scheduling fences keep the program order: slot x first issues the reads of slot
    // x + PREFETCH, then its two products, whose operands were read PREFETCH slots
    // earlier, so the LDS latency hides behind 2 PREFETCH products.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < SLOTS; ++x) {
      if (x + PREFETCH < SLOTS) {
        va[(x + PREFETCH) % (PREFETCH + 1)] = v_operand(vt, (x + PREFETCH) >> 2, (x + PREFETCH) & 3);
        ka[(x + PREFETCH) % (PREFETCH + 1)] = k_operand(kt, (x + PREFETCH) / NB, (x + PREFETCH) % NB);
      }
      acc[x & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[x % (PREFETCH + 1)], pb[x >> 2], acc[x & 3], 0, 0, 0);
      sc[x % NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[x % (PREFETCH + 1)], qop[x / NB], sc[x % NB], 0, 0, 0);
      if (x < LOADS_W - LOADS_HALF && dma_now)
        issue_one(dma_tile_idx, group ? dma_stage_g1 : dma_stage_g0, LOADS_HALF + x);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Softmax phase of step j: mask, running max, lazy rescale, P = exp2(S c - m), row sum.
  // P = exp2(S c2 - m) into pb (rounded to bf16: the B operand of the next P V), and this
  // lane's share of the row sum, taken in fp32 from the unrounded weights (the LSE keeps
  // fp32 accuracy).  The scores in sc are left intact.
  auto exponentiate = [&](float neg_m) __attribute__((always_inline)) {
    float r[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[c >> 1][8 * (c & 1) + x], c2, neg_m));
        pb[c][x] = (__bf16)p;
        r[c] = x == 0 ? p : r[c] + p;     // each chain starts at its first weight
      }
    float sum = (r[0] + r[1]) + (r[2] + r[3]);
#pragma unroll
    for (int c = 4; c < NCH; c += 2) sum += r[c] + r[c + 1];
    return sum;
  };
  // Softmax phase of step j: mask, P = exp2(S c2 - m), row sum.  Fast path: exponentiate
  // against the running maximum as it stands, without computing this tile's maximum; it
  // stands as long as no weight gets large (this lane's tile sum <= 2^24, which bounds
  // every weight, keeps P and O finite and is checked together with inf and NaN).
  // Otherwise, and while a row has no maximum yet, take the tile's maximum and rescale
  // lazily: the maximum moves only when the new one exceeds it by more than TAU.
  auto softmax_phase = [&](int j, int stage) __attribute__((always_inline)) {
    // this wave's loads: group 0 V(j+1) into the stage of V(j-2), group 1 K(j+3) into the
    // stage of K(j); both stages were last read in interval 2j
    const int dma_tile_idx = group ? j + 3 : j + 1;
    const int dma_stage = group ? stage : (stage == 2 ? 0 : stage + 1);
#pragma unroll
    for (int t = 0; t < LOADS_HALF; ++t) issue_one(dma_tile_idx, dma_stage, t);   // the rest: next matrix phase
    if (j >= wave_tiles || j < wave_first) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) pb[c] = bf16x8{};
      return;
    }
    if (j < full_begin || j >= full_end) {
      // keep this a real (scalar) branch: only diagonal, boundary and ragged tiles pay for
      // the mask
      __asm__ volatile("" ::: "memory");
      // allowed key offsets of this row: [thr_lo, thr), thr_lo <= thr; one unsigned compare
      // per score, fenced in groups of four so that the compiler keeps each compare next to
      // its select instead of holding all the lane masks in scalar registers
      const int thr_lo = lo - (j * BN + 4 * lg);
      const unsigned width = (unsigned)(lim - lo);
#pragma unroll
      for (int jj = 0; jj < NB; ++jj)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int x = 32 * jj + 8 * (i >> 2) + (i & 3);
          if (!((unsigned)(x - thr_lo) < width)) sc[jj][i] = -INFINITY;
          if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
    }
    // (in a batch, the first tile of every shard after the first re-anchors m, as a launch
    // of its own would: see below)
    const bool anchor = BATCH && j == anchor_tile;
    bool full_path = anchor || __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
    float rs = 0.f;
    if (!full_path) {
      rs = exponentiate(-m_run);
      full_path = __builtin_amdgcn_ballot_w64(!(rs <= 0x1p24f)) != 0;
    }
    if (full_path) {
      float mx;
      {
        float xm[NB];
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
          xm[jj] = fmaxf(fmaxf(sc[jj][0], sc[jj][1]), sc[jj][2]);
#pragma unroll
          for (int i = 3; i < 15; i += 2) xm[jj] = fmaxf(fmaxf(xm[jj], sc[jj][i]), sc[jj][i + 1]);
        }
        float x0 = fmaxf(fmaxf(xm[0], sc[0][15]), xm[1]);
        x0 = fmaxf(x0, sc[1][15]);
#pragma unroll
        for (int jj = 2; jj < NB; ++jj) x0 = fmaxf(fmaxf(x0, xm[jj]), sc[jj][15]);
        mx = lane_pair_max(x0) * c2;
      }
      // Rescale when the maximum has grown by more than TAU, or (anchor) re-anchor m on this
      // tile's maximum, up or down, as a launch of this shard alone would start: the tile's
      // largest weight is then exactly 1 and carries no bf16 rounding into P V, which matters
      // where a few keys dominate a row (with m carried over from an earlier shard it would
      // be 2^f, rounded, for some f in (-TAU, TAU]).  In re-anchoring, a lane whose tile holds
      // no key, or whose maximum lies more than 32 below m (the rescale would grow O and l by
      // more than 2^32), keeps its m.
      if (anchor || __builtin_amdgcn_ballot_w64(mx > m_run + TAU) != 0) {
        const float m_new = !anchor ? fmaxf(m_run, mx) : (mx == -INFINITY || mx < m_run - 32.f) ? m_run : mx;
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < D / 32; ++e) acc[e] *= alpha;
        m_run = m_new;
      }
      rs = exponentiate(m_run == -INFINITY ? 0.f : -m_run);
    }
    l_run += rs;
  };
  // ---- main loop -------------------------------------------------------------------------
  // Every wave runs the same sequence: matrix phase of step j, barrier, softmax phase of
  // step j, barrier.  Group 1 executes one extra barrier before the loop and group 0 one
  // after it, so group 1 runs half a step behind group 0 and the two waves of each SIMD
  // alternate between matrix and vector work.  Numbering the intervals between barriers,
  // interval 2j+1 holds group 0's matrix phase j and group 1's softmax phase j-1, interval
  // 2j+2 group 0's softmax phase j and group 1's matrix phase j.  K(j) is read in
  // intervals 2j+1 and 2j+2, V(j) in 2j+3 and 2j+4; tile j lives in stage (j - j_begin) % 3
  // (j_begin: the workgroup's first key tile; the steps below count from it).
  // Staging: group 0 loads V(j+1) in halves, at the start of its softmax phase j
  // (interval 2j+2) and of its matrix phase j+1 (interval 2j+3), into the stage of V(j-2)
  // (last read in interval 2j); first read in interval 2j+5.  Group 1 loads K(j+3) in
  // halves in its softmax phase j (interval 2j+3) and matrix phase j+1 (interval 2j+4),
  // into the stage of K(j) (last read in interval 2j+2); first read in interval 2j+7.  Each
  // wave waits at the end of its softmax phase j+1 (vmcnt(LOADS_HALF): only the loads that
  // phase just issued may still be in flight), before the barrier that opens the first interval
  // reading the tile.  The prologue loads the first two K tiles and the first V tile
  // completely and starts the third K tile, which group 1's first wait covers; the first
  // matrix phase issues no loads.
  for (int s = 0; s < n_shards; ++s) {
  if (BATCH) {
    // the next shard with a key for this workgroup: its ranges and K/V descriptors
    wg_tiles(s);
    if (n_tiles <= j_begin) continue;
    row_tiles();
    anchor_tile = s > 0 ? wave_first : -1;
    k_rsrc = make_dma_rsrc((const __bf16*)((const char*)sb.k + s * sb.stride) + kv_base, (unsigned)num_records);
    v_rsrc = make_dma_rsrc((const __bf16*)((const char*)sb.v + s * sb.stride) + kv_base, (unsigned)num_records);
    my_rsrc = group ? k_rsrc : v_rsrc;
#pragma unroll
    for (int c = 0; c < NCH; ++c) pb[c] = bf16x8{};
  }
  {
    u32x4* z = (u32x4*)v_lds[2];        // read by the (zero-P) PV of step 0
    for (int i = tid; i < TILE_BYTES / 16; i += THREADS) z[i] = u32x4{};
  }
  if (group == 1) {
    issue_tile_dma(k_rsrc, RA_LDS_ADDR(k_lds[0]), k_dma_off, j_begin);   // rows past L arrive as zeros
    issue_tile_dma(k_rsrc, RA_LDS_ADDR(k_lds[1]), k_dma_off, j_begin + 1);
  } else {
    issue_tile_dma(v_rsrc, RA_LDS_ADDR(v_lds[0]), v_dma_off, j_begin);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): Q, K(0), K(1), V(0) are in place
  __syncthreads();
  if (group == 1) {
    issue_tile_dma(k_rsrc, RA_LDS_ADDR(k_lds[2]), k_dma_off, j_begin + 2);
    barrier_no_fence();
  }
  auto step = [&](int j, auto stage_c) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);        // matrix phase first in the SIMD's issue arbitration
    matrix_phase(j, stage_c);
    __builtin_amdgcn_s_setprio(0);
    barrier_no_fence();
    softmax_phase(j, decltype(stage_c)::value);
    // vmcnt(LOADS_HALF): everything but the loads this softmax phase just issued has landed,
    // i.e. the tile split over the previous softmax phase and this step's matrix phase
    __builtin_amdgcn_s_waitcnt(0x0F70 | LOADS_HALF);
    barrier_no_fence();
  };
  // unrolled by the three stages so that every LDS address in the matrix phase is a
  // per-lane base plus an immediate; tile j lives in stage (j - j_begin) % 3
  for (int j = j_begin; j <= n_tiles; j += 3) {
    step(j, Stage<0>{});
    if (j + 1 > n_tiles) break;
    step(j + 1, Stage<1>{});
    if (j + 2 > n_tiles) break;
    step(j + 2, Stage<2>{});
  }
  if (group == 0) barrier_no_fence();
  __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): no load into LDS outlives the loop
  // before the next shard's prologue writes the stages: every wave's loads have landed
  // (loads past a wave's last tile still write zeros into a stage) and its reads are done
  if (BATCH) __syncthreads();
  }   // shard

  // ---- epilogue ------------------------------------------------------------------------
  const float l_tot = lane_pair_sum(l_run);
  if (t >= L) return;
  const bool any = l_tot > 0.f;
  const float lse_new = any ? (m_run + __log2f(l_tot)) * LN2 : -INFINITY;
  const float inv = any ? 1.f / l_tot : 0.f;
  const int64_t lse_idx = ((int64_t)bi * a.h + hq) * L + t;
  const int64_t row_off = row_offset();   // (formed here: not held through the loop)
  float* lse_p = l_dst + lse_idx;
  // the row's final values are formed in acc, then stored once
  if (MODE == MODE_PART) {
    // rows of an unsplit block have no second partial in this step: mark it empty (a later
    // step may split the block and merge into it)
    if (l2_empty && lg == 0) l2_empty[lse_idx] = -INFINITY;
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[e][i] *= inv;
    if (lg == 0) *lse_p = lse_new;
  } else if (!any) {   // nothing allowed in this step: the accumulator is unchanged
    if (!a.o_out) return;
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const f32x4 old = *(const f32x4*)(o_dst + row_off + 32 * e + 8 * ib);
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[e][4 * ib + x] = old[x];
      }
  } else {
    const float lse_old = *lse_p;
    const float M = fmaxf(lse_old, lse_new);
    const float wa = __builtin_amdgcn_exp2f((lse_old - M) * LOG2E);
    const float wb = __builtin_amdgcn_exp2f((lse_new - M) * LOG2E);
    const float tot = wa + wb;
    const float fa = wa / tot, fb = wb * inv / tot;
    auto merge_rows = [&](auto may_be_empty) __attribute__((always_inline)) {
      // an empty row of the second accumulator is not read: its O is undefined
      const bool have_old = !decltype(may_be_empty)::value || lse_old > -INFINITY;
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          const f32x4 old = have_old ? *(const f32x4*)(o_dst + row_off + 32 * e + 8 * ib) : f32x4{};
#pragma unroll
          for (int x = 0; x < 4; ++x) acc[e][4 * ib + x] = __builtin_fmaf(fb, acc[e][4 * ib + x], fa * old[x]);
        }
    };
    if (part) merge_rows(std::true_type{});
    else merge_rows(std::false_type{});   // the first accumulator: every row was written in the first step
    if (lg == 0) *lse_p = M + __logf(tot);
  }
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const f32x4 v = {acc[e][4 * ib], acc[e][4 * ib + 1], acc[e][4 * ib + 2], acc[e][4 * ib + 3]};
      if (a.o_out) cast_row(row_off, e, ib, v);
      else *(f32x4*)(o_dst + row_off + 32 * e + 8 * ib) = v;
    }
}

}  // namespace

namespace {
// Compute units of the current device (looked up once per device).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace

StepGeometry step_geometry_bf16(const StepArgs& a) {
  StepGeometry g;
  const int G = a.h / a.n_kv;
  g.Hw = (G % 4 == 0) ? 4 : ((G % 2 == 0) ? 2 : 1);
  g.PB = WAVES / g.Hw;
  g.rows_wg = QW * g.PB;
  g.n_qb = (a.L + g.rows_wg - 1) / g.rows_wg;
  g.inner = a.n_kv * a.b * (G / g.Hw);
  return g;
}

// Which query blocks of a step run as two work items, and the launch order.
//
// One workgroup per compute unit fits (its LDS).  When a step has fewer query blocks than the
// chip has units for them (short shards: n_qb blocks per KV head and batch row), units sit
// idle and the longest block sets the step time; splitting a block's key range over two
// workgroups halves its length, the second half merging into a second accumulator (no two
// workgroups write one row) that the pass folds into the first at the end.  Measured on
// MI355X: that pays only while it puts idle units to work.  Balancing a grid that already
// fills the chip does not: the units whose blocks finish early let the clock of the busy ones
// rise (the chip is power-limited under full load), and every extra workgroup adds its fixed
// cost.  So the split is taken only when n_qb is below the units per (KV head, batch row),
// with at most one item per unit; among those plans it takes the one with the shortest
// longest item (a block's work: its key tiles plus a fixed cost; blocks s and up are split,
// the tile counts grow with the block index), the fewest splits on a tie, and only if the
// longest item shrinks by a tenth.  The host knows every block's tile count from the scalar
// key limit (not with packed documents, whose bounds live on the device).  Items go out
// heaviest first (ties: unsplit blocks first).
// Blocks [s, n_qb) split: merge the unsplit blocks (s-1 .. 0) and the parts (2 per block,
// n_qb-1 .. s), both already in nonincreasing cost, into one nonincreasing launch order.
SplitPlan order_items(const int* w, const int* wp, int n_qb, int s, int fixed) {
  SplitPlan pl{};
  int u = s - 1, m = 0, item = 0;
  const int n_parts = 2 * (n_qb - s);
  while (u >= 0 || m < n_parts) {
    const int cu = u >= 0 ? w[u] + fixed : -1;
    const int cp = m < n_parts ? wp[n_qb - 1 - m / 2] + fixed : -1;
    if (cu >= cp) {
      pl.order[item >> 5] |= 1u << (item & 31);
      --u;
    } else {
      ++m;
    }
    ++item;
  }
  pl.split_from = s;
  return pl;
}

// Longest load of `units` compute units that take the items in launch order, each the next
// item when it frees up (how the hardware hands out workgroups): blocks [0, s) whole, blocks
// [s, n_qb) as two parts, in the nonincreasing order order_items launches them.
int list_makespan(const int* w, const int* wp, int n_qb, int s, int units, int fixed) {
  std::priority_queue<int, std::vector<int>, std::greater<int>> load;   // free-up times
  int u = s - 1, m = 0, longest = 0, started = 0;
  const int n_parts = 2 * (n_qb - s);
  while (u >= 0 || m < n_parts) {
    const int cu = u >= 0 ? w[u] + fixed : -1;
    const int cp = m < n_parts ? wp[n_qb - 1 - m / 2] + fixed : -1;
    int c;
    if (cu >= cp) {
      c = cu;
      --u;
    } else {
      c = cp;
      ++m;
    }
    int t0 = 0;
    if (started < units) {
      ++started;
    } else {
      t0 = load.top();
      load.pop();
    }
    load.push(t0 + c);
    longest = max(longest, t0 + c);
  }
  return longest;
}

// The plan from each block's cost in tiles: w[qb] tiles whole, wp[qb] tiles for the longer of
// its two parts.  by_makespan: choose by the list-scheduling makespan, also when there are
// more items than units (launches of several ring steps, whose workgroups are long next to
// their fixed costs); otherwise only plans with at most one item per unit, by the longest item.
SplitPlan plan_from_costs(const int* w, const int* wp, int n_qb, int units, bool by_makespan = false) {
  SplitPlan pl{};
  pl.split_from = n_qb;
  constexpr int FIXED = 3;              // per-workgroup cost in tile times (Q load, pipeline fill, epilogue)
  if (by_makespan) {
    // every split point by its list schedule: the shortest, fewest splits on a tie, taken if
    // it beats no split by a tenth
    if (units < 1) return pl;
    const int none = list_makespan(w, wp, n_qb, n_qb, units, FIXED);
    int best = n_qb, best_len = none;
    for (int s = n_qb - 1; s >= 0; --s) {
      const int len = list_makespan(w, wp, n_qb, s, units, FIXED);
      if (len < best_len) {
        best_len = len;
        best = s;
      }
    }
    if (best == n_qb || 10 * best_len > 9 * none) return pl;
    return order_items(w, wp, n_qb, best, FIXED);
  }
  if (n_qb >= units) return pl;         // the grid fills the chip already
  int pre_max[kSplitMaxBlocks + 1], suf_max[kSplitMaxBlocks + 1];
  pre_max[0] = 0;
  for (int qb = 0; qb < n_qb; ++qb) pre_max[qb + 1] = max(pre_max[qb], w[qb] + FIXED);
  suf_max[n_qb] = 0;
  for (int qb = n_qb - 1; qb >= 0; --qb) suf_max[qb] = max(suf_max[qb + 1], wp[qb] + FIXED);
  const int none = pre_max[n_qb];
  int best = n_qb, best_len = none;
  for (int s = n_qb - 1; s >= max(0, 2 * n_qb - units); --s) {   // s + 2 (n_qb - s) items <= units
    const int len = max(pre_max[s], suf_max[s]);
    if (len < best_len) {
      best_len = len;
      best = s;
    }
  }
  if (best == n_qb || 10 * best_len > 9 * none) return pl;
  return order_items(w, wp, n_qb, best, FIXED);
}

// Tiles of block qb in KV shard ks (no packed documents: the keys of a row are a prefix).
int block_tiles(const StepArgs& a, const StepGeometry& g, int ks, int qb) {
  const int last = min((qb + 1) * g.rows_wg, a.L) - 1;
  return (kv_limit(a.causal, a.layout, a.N, a.L, a.q_shard, ks, last) + BN_SHORT - 1) / BN_SHORT;
}

SplitPlan plan_split(const StepArgs& a, const StepGeometry& g, int n_cu) {
  SplitPlan pl{};
  pl.split_from = g.n_qb;
  if (a.doc_begin || g.n_qb < 1 || g.n_qb > kSplitMaxBlocks || n_cu < 1) return pl;
  int w[kSplitMaxBlocks], wp[kSplitMaxBlocks];
  for (int qb = 0; qb < g.n_qb; ++qb) {
    w[qb] = block_tiles(a, g, a.kv_shard, qb);
    wp[qb] = (w[qb] + 1) / 2;
  }
  return plan_from_costs(w, wp, g.n_qb, n_cu / g.inner);
}

// A launch of several ring steps splits a block's key range in every one of its KV shards: a
// part's cost is the sum of its halves (the first part takes the odd tile).  Its workgroups
// are long next to their fixed costs, so here the plan also balances a grid that fills the
// chip: it takes the split point whose list schedule over the units (in launch order) is
// shortest.  Measured on MI355X, striped causal h = 32, n_kv = 8, L = 2048, N = 8 (32 blocks
// per KV head on 32 units, the heaviest twice the mean): 0.368 -> 0.324 ms per batched pass.
SplitPlan plan_split_batch(const StepArgs& a, const ShardBatch& sb, const StepGeometry& g, int n_cu) {
  SplitPlan pl{};
  pl.split_from = g.n_qb;
  if (a.doc_begin || g.n_qb < 1 || g.n_qb > kSplitMaxBlocks || n_cu < 1 || sb.n < 1) return pl;
  // The search runs a list schedule per split point (up to 65 of up to 128 items), so the
  // plans of recent batch shapes are kept: a pass asks for each launch's plan twice, and a
  // caller's passes repeat the same shapes.
  struct Entry {
    int key[10];
    SplitPlan plan;
  };
  static std::mutex mu;
  static Entry cache[32];
  static int n_cached = 0, next_slot = 0;
  const int key[10] = {a.causal, a.layout, a.N, a.L, a.q_shard, sb.k_first, sb.n, g.rows_wg, g.n_qb,
                       n_cu / g.inner};
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_cached; ++i)
      if (std::equal(key, key + 10, cache[i].key)) return cache[i].plan;
  }
  int w[kSplitMaxBlocks], wp[kSplitMaxBlocks];
  for (int qb = 0; qb < g.n_qb; ++qb) {
    w[qb] = wp[qb] = 0;
    for (int s = 0; s < sb.n; ++s) {
      const int ks = ((a.q_shard - (sb.k_first + s)) % a.N + a.N) % a.N;
      const int t = block_tiles(a, g, ks, qb);
      w[qb] += t;
      wp[qb] += (t + 1) / 2;
    }
  }
  pl = plan_from_costs(w, wp, g.n_qb, n_cu / g.inner, true);
  std::lock_guard<std::mutex> lock(mu);
  Entry& e = cache[next_slot];
  std::copy(key, key + 10, e.key);
  e.plan = pl;
  next_slot = (next_slot + 1) % 32;
  if (n_cached < 32) ++n_cached;
  return pl;
}

bool step_splits_bf16(const StepArgs& a) {
  const StepGeometry g = step_geometry_bf16(a);
  return plan_split(a, g, cu_count()).split_from < g.n_qb;
}

template <bool BATCH>
hipError_t launch_fwd(const StepArgs& a, const ShardBatch& sb, const SplitPlan& plan, const StepGeometry& g,
                      int mode, hipStream_t stream) {
  const int n_items = plan.split_from + 2 * (g.n_qb - plan.split_from);
  const int64_t grid = (int64_t)n_items * g.inner;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  // (the split plan counts tiles of BN_SHORT keys; it is only taken for L <= kSplitMaxL)
  static_assert(kSplitMaxL < LONG_TILES_MIN_L, "split shards use the short tiles");
  const bool long_tiles = a.L >= LONG_TILES_MIN_L;
  if (mode == MODE_PART) {
    if (long_tiles)
      hipLaunchKernelGGL((step_fwd_bf16_kernel<MODE_PART, BN_LONG, BATCH>), dim3((unsigned)grid), dim3(THREADS), 0,
                         stream, a, g.Hw, g.n_qb, g.inner, plan, sb);
    else
      hipLaunchKernelGGL((step_fwd_bf16_kernel<MODE_PART, BN_SHORT, BATCH>), dim3((unsigned)grid), dim3(THREADS), 0,
                         stream, a, g.Hw, g.n_qb, g.inner, plan, sb);
  } else {
    if (long_tiles)
      hipLaunchKernelGGL((step_fwd_bf16_kernel<MODE_MERGE, BN_LONG, BATCH>), dim3((unsigned)grid), dim3(THREADS), 0,
                         stream, a, g.Hw, g.n_qb, g.inner, plan, sb);
    else
      hipLaunchKernelGGL((step_fwd_bf16_kernel<MODE_MERGE, BN_SHORT, BATCH>), dim3((unsigned)grid), dim3(THREADS), 0,
                         stream, a, g.Hw, g.n_qb, g.inner, plan, sb);
  }
  return hipGetLastError();
}

hipError_t launch_step_bf16(const StepArgs& a, int mode, hipStream_t stream) {
  const StepGeometry g = step_geometry_bf16(a);
  SplitPlan plan{};
  plan.split_from = g.n_qb;
  if (a.o_out && a.o2) return hipErrorInvalidValue;   // a split pass ends with the fold instead
  if (a.o2 && a.lse2) plan = plan_split(a, g, cu_count());
  return launch_fwd<false>(a, ShardBatch{}, plan, g, mode, stream);
}

hipError_t launch_steps_bf16(const StepArgs& a, const ShardBatch& sb, int mode, hipStream_t stream) {
  if (sb.n < 1 || sb.n > kMaxBatch || !sb.k || !sb.v || !a.o2 != !a.lse2) return hipErrorInvalidValue;
  if (a.o_out && a.o2) return hipErrorInvalidValue;   // a split pass ends with the fold instead
  if (a.o2 && mode != MODE_MERGE) return hipErrorInvalidValue;   // the parts merge into (o2, lse2)
  const StepGeometry g = step_geometry_bf16(a);
  SplitPlan plan{};
  plan.split_from = g.n_qb;
  if (a.o2) plan = plan_split_batch(a, sb, g, cu_count());
  return launch_fwd<true>(a, sb, plan, g, mode, stream);
}

bool steps_split_bf16(const StepArgs& a, const ShardBatch& sb) {
  const StepGeometry g = step_geometry_bf16(a);
  return plan_split_batch(a, sb, g, cu_count()).split_from < g.n_qb;
}

}  // namespace ra

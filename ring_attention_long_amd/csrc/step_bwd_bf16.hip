// One ring step of the backward pass, bf16 inputs, fp32 accumulation, head dim 128.
//
// The pages say what flows where (page 1, "The Backward Pass and Gradient Exchange";
// page 4, "The Backward Pass: Symmetric Ring Operation"): P is recomputed from the saved
// statistics, dQ accumulates on the query's device while K/V pass by, and dK/dV
// accumulate for each KV block.  The gradients themselves are the textbook ones of softmax
// attention: with P = exp(s - LSE) (0 where masked) and D = rowsum(dO * O),
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q,
// summed over the query heads of each KV group for dK and dV.
//
// Two kernels per step, each keeping one lane layout end to end:
//  * dQ kernel (query-major, like the forward): S^T = K Q^T and dP^T = V dO^T with Q^T and
//    dO^T resident in VGPRs; lane l holds one query's scores, so LSE and D are one value
//    per lane; dQ^T += K^T dS^T with K^T read by the transposing LDS load.  Eight waves in
//    the forward's ping-pong.
//  * dK/dV kernel (key-major): each wave keeps the K rows of 32 keys in VGPRs (their V rows
//    in LDS) and walks the query tiles of every head of its KV group; S = Q K^T and
//    dP = dO V^T put one key per lane, and dV^T += dO^T P, dK^T += Q^T dS take dO^T and
//    Q^T from transposing LDS loads.  No atomics: every workgroup owns its keys.
// Recomputing S and dP in both kernels costs two extra products per pair (7 instead of 5)
// and buys two independent kernels with no transposes of dS.
//
// LDS tiles (K, V, Q, dO) are 64 rows x 256 B filled by DMA (buffer_load ... lds); the
// 16-byte chunk c of row r sits at position c ^ (4 (r & 3) + ((r >> 2) & 3)), which keeps
// both the 16-row ds_read_b128 pattern and the transposing-read pattern free of bank
// conflicts.
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int ROW_BYTES = D * 2;
constexpr int TILE_ROWS = 64;
constexpr int TILE_BYTES = TILE_ROWS * ROW_BYTES;   // 16 KB, 16 DMA loads of 1 KB
constexpr float LOG2E = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// DMA of one 64-row tile: load i (1 KB) fills rows 4i..4i+3, lane l writes slot l (row
// 4i + l/16, position l%16) with the global chunk (l%16) ^ swz(row).  Wave w issues loads
// i = w, w+4, w+8, w+12, so swz(row) = 4 (l/16) + w is fixed per lane.
__device__ __forceinline__ unsigned dma_lane_offset(unsigned row_stride, int lane, int w) {
  const int lrow = lane >> 4;
  return (unsigned)lrow * row_stride + (unsigned)((lane & 15) ^ (4 * lrow + w)) * 16;
}
__device__ __forceinline__ void dma_tile(dma_rsrc rsrc, unsigned dst, unsigned lane_off, unsigned row0_off,
                                         unsigned row_stride, int w) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = w + 4 * t;
    dma16_to_lds(rsrc, dst + 1024u * i, lane_off, row0_off + (unsigned)(4 * i) * row_stride);
  }
}
// Buffer descriptor covering rows 0..rows-1 (row_stride bytes apart, 256 B each) from base;
// reads beyond return zeros.
__device__ __forceinline__ dma_rsrc rows_rsrc(const void* base, int rows, unsigned row_stride) {
  const unsigned n = rows > 0 ? (unsigned)(rows - 1) * row_stride + ROW_BYTES : 0u;
  return make_dma_rsrc(base, n);
}
// Row read: 16 B of row r, chunk c.
__device__ __forceinline__ bf16x8 row_chunk(const char* tile, int r, int c) {
  return *(const bf16x8*)(tile + r * ROW_BYTES + ((c ^ swz(r)) * 16));
}
// Transposing read: the A operand [m = column d][k = 8 rows] of a product contracting
// over rows.  Lane (g16, j) of a 16-lane group points at row k0 + j/4, column
// d0 + 4 (j%4) with d0 = 32e + 16 (g16 & 1) and k0 = 16c + 4 lg (+8 for the second half);
// each lane then receives 4 consecutive rows of its column d = 32e + l%32.  The row order
// 16c + 4lg + {0..3}, 16c + 8 + 4lg + {0..3} matches the register order of the 32x32
// accumulator that supplies the other operand.
__device__ __forceinline__ bf16x8 rows_transposed(const char* tile, int lane, int c, int e) {
  const int g16 = lane >> 4, j = lane & 15, lg = lane >> 5;
  bf16x4 part[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 16 * c + 8 * h + 4 * lg + (j >> 2);
    const int d = 32 * e + 16 * (g16 & 1) + 4 * (j & 3);
    const int chunk = d >> 3;
    const char* p = tile + r * ROW_BYTES + ((chunk ^ swz(r)) * 16) + (d & 7) * 2;
    part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)p);
  }
  return bf16x8{part[0][0], part[0][1], part[0][2], part[0][3],
                part[1][0], part[1][1], part[1][2], part[1][3]};
}

// ------------------------------------------------------------------------------------------
// D[b][h][t] = sum_d dO[b][t][h][d] * O[b][t][h][d]   (16 lanes per row, 8 elements each)
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const __bf16* __restrict__ o,
                                                             const __bf16* __restrict__ dout,
                                                             float* __restrict__ delta, int L,
                                                             int h, int64_t rows) {
  const int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int part = threadIdx.x & 15;
  float s = 0.f;
  if (row < rows) {
    const bf16x8 a = *(const bf16x8*)(o + row * D + part * 8);
    const bf16x8 b = *(const bf16x8*)(dout + row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)a[e] * (float)b[e];
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 16);
  if (row < rows && part == 0) {
    const int hq = (int)(row % h);
    const int64_t bt = row / h;
    const int t = (int)(bt % L);
    const int64_t bi = bt / L;
    delta[(bi * h + hq) * L + t] = s;
  }
}

// ------------------------------------------------------------------------------------------
// dK/dV kernel: workgroup = 8 waves on 128 keys of one KV head, walking the 64-row query
// tiles of every head of the KV group.
//
// Wave w owns keys 32 (w % 4) .. +31 of the workgroup and rows 32 (w / 4) .. +31 of each
// query tile, so the two waves on a SIMD share their keys and split the rows.  Per tile a
// wave runs a matrix phase (dV^T += dO^T P and dK^T += Q^T dS of the previous tile, then
// S = Q K^T and dP = dO V^T of this tile: 32 products, plus 2 that subtract the row's
// LSE / scale and D, see xq_lds) and a vector phase (P, dS of this tile, no memory reads
// outside diagonal tiles).  The two groups (w / 4 = 0, 1) run half a tile apart, separated
// by workgroup barriers, so that while one wave of a SIMD issues products the other does
// its vector work.  The two row halves' dK and dV are summed through LDS at the end.
// K rows stay in VGPRs; V rows of the 128 keys stay in LDS.  Q and dO tiles rotate
// through three LDS stages (a tile is read during four consecutive half steps and loaded
// during the two before).
// ------------------------------------------------------------------------------------------
constexpr int KV_THREADS = 512;

constexpr int KB = 128;                                // keys per workgroup
constexpr int STAGE_BYTES = 2 * TILE_BYTES;            // Q tile, then dO tile
constexpr int N_STAGE = 3;
constexpr int V_OFF = N_STAGE * STAGE_BYTES;           // 96 KB
constexpr int SMEM_BYTES = V_OFF + KB * ROW_BYTES;     // + 32 KB of V rows

// Workgroup barrier without a memory fence: memory operations may not move across it,
// but no wait for outstanding loads is emitted (each wave waits for its own DMA).
__device__ __forceinline__ void barrier_no_fence() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__global__ __launch_bounds__(KV_THREADS, 1) void bwd_dkdv_kernel(StepArgs a, const __bf16* __restrict__ dout,
                                                                 const float* __restrict__ lse,
                                                                 const float* __restrict__ delta,
                                                                 float* __restrict__ dk, float* __restrict__ dv,
                                                                 KvForm kf, int set_out, SplitPlan plan,
                                                                 float* __restrict__ dk2, float* __restrict__ dv2) {
  __shared__ __attribute__((aligned(1024))) char smem[SMEM_BYTES];
  // Per row of a staged tile, one more 16-wide k-step for the products S = Q K^T and
  // dP = dO V^T: columns 0 and 1 hold the bf16 pair (hi, lo) of -LSE / scale (S) or -D (dP),
  // the other columns zeros, and the matching K^T / V^T rows are ones.  The products then
  // come out as S - LSE / scale and dP - D, so the vector phase reads no statistics.
  __shared__ __attribute__((aligned(16))) __bf16 xq_lds[N_STAGE][TILE_ROWS][16];
  __shared__ __attribute__((aligned(16))) __bf16 xo_lds[N_STAGE][TILE_ROWS][16];
  __shared__ __attribute__((aligned(16))) int lo_lds[N_STAGE][TILE_ROWS];   // allowed keys [lo, hi)
  __shared__ __attribute__((aligned(16))) int hi_lds[N_STAGE][TILE_ROWS];
  // per stage and 32-row half: the key bounds of the half's first and last row inside the
  // shard, (lo_first, hi_first, lo_last, hi_last)
  __shared__ __attribute__((aligned(16))) int cls_lds[N_STAGE][2][4];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wave & 3, grp = wave >> 2;
  const int lane = tid & 63, lk = lane & 31, lg = lane >> 5;
  const int L = a.L;
  const int G = a.h / a.n_kv;
  // key blocks heaviest first (keys early in the shard see more queries); a split block runs
  // the first half of its (head, query tile) iterations as part 0 and the rest as part 1,
  // which writes its dK, dV into the second buffers
  const int n_kb = (L + KB - 1) / KB;
  int kbp, part;
  split_item(plan, n_kb, (int)(blockIdx.x / (a.n_kv * a.b)), kbp, part);
  const int kb = n_kb - 1 - kbp;
  const bool split_blk = kbp >= plan.split_from;
  if (part) {
    dk = dk2;
    dv = dv2;
  }
  const int g = blockIdx.x % a.n_kv;
  const int bi = (blockIdx.x / a.n_kv) % a.b;
  const int u0 = kb * KB;
  const int uw = u0 + 32 * slot;            // this wave's first key
  const int u = uw + lk;                    // this lane's key
  // allowed keys of query row t: [lo, hi), both nondecreasing in t (see key_range)
  const bool packed = a.doc_begin != nullptr;
  auto range_of = [&](int row, int64_t db, int64_t de) {
    // the shard indices pass through an empty asm so that what is derived from them is
    // recomputed here rather than kept in registers through the main loop
    int qs = a.q_shard, ks = a.kv_shard;
    __asm__ volatile("" : "+s"(qs), "+s"(ks));
    return key_range(a.causal, a.layout, a.N, L, qs, ks, row, packed, db, de);
  };
  auto range = [&](int row) {
    int64_t db = 0, de = 0;
    if (packed) {
      db = a.doc_begin[(int64_t)bi * L + row];
      de = a.doc_end[(int64_t)bi * L + row];
    }
    return range_of(row, db, de);
  };

  // the query rows that may see keys [u0, u0 + KB): from the first with hi > u0 to the last
  // with lo < u0 + KB
  int t_lo = 0, t_hi = L;
  while (t_lo < t_hi) {
    const int mid = (t_lo + t_hi) >> 1;
    if (range(mid).hi > u0) t_hi = mid;
    else t_lo = mid + 1;
  }
  int t_stop = t_lo, t_top = L;
  while (t_stop < t_top) {
    const int mid = (t_stop + t_top) >> 1;
    if (range(mid).lo >= u0 + KB) t_top = mid;
    else t_stop = mid + 1;
  }
  const int qt_first = t_lo / TILE_ROWS;
  const int t_end = (t_stop + TILE_ROWS - 1) / TILE_ROWS * TILE_ROWS;
  const int n_qt_r = t_end / TILE_ROWS - qt_first;           // query tiles of the range
  const int n_iter_all = n_qt_r * G;                         // (head, query tile) pairs
  const int half = (n_iter_all + 1) / 2;
  const int i_first = split_blk && part ? half : 0;          // this workgroup's iterations
  const int n_iter = split_blk ? (part ? n_iter_all - half : half) : n_iter_all;
  if (t_lo >= t_stop || n_iter <= 0) {     // no query of this step (or part) sees these keys
    if (set_out && grp == 0 && u < L) {     // their gradients are zero
      float* kz = dk + (((int64_t)bi * L + u) * a.n_kv + g) * D + 4 * lg;
      float* vz = dv + (((int64_t)bi * L + u) * a.n_kv + g) * D + 4 * lg;
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          *(f32x4*)(kz + 32 * e + 8 * ib) = f32x4{};
          *(f32x4*)(vz + 32 * e + 8 * ib) = f32x4{};
        }
    }
    return;
  }

  // resident K rows of this lane's key (B operand [k = d][n = key])
  const int64_t krow = (((int64_t)bi * L + min(u, L - 1)) * a.n_kv + g) * D + lg * 8;
  bf16x8 kop[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) kop[kk] = *(const bf16x8*)((const __bf16*)a.k + krow + kk * 16);

  const float c2 = a.scale * LOG2E;
  const unsigned q_stride = (unsigned)a.h * D * 2;
  const unsigned kv_stride = (unsigned)a.n_kv * D * 2;
  const int wq = wave & 3;                                    // DMA lane pattern of this wave
  const unsigned q_lane_off = dma_lane_offset(q_stride, lane, wq);

  // LDS read offsets.  Row reads (A operand [m = row][k = d], also the V rows as B
  // operand): row lk of a 32-row block, chunk (2 kk + lg) ^ swz(lk), i.e. byte offset
  // r_base ^ 32 kk.  Transposing reads (A operand [m = d][k = row]) of rows
  // 16c + 8h + 4lg + {0..3} of a 32-row block, d = 32e + lane % 32 (see rows_transposed):
  // byte offset t_base[h] ^ 64 e, plus 16c rows.  The bases stay in three VGPRs and the
  // offsets are formed next to their reads.
  const unsigned r_base = (unsigned)lk * ROW_BYTES + (unsigned)((lg ^ swz(lk)) * 16);
  const int g16 = lane >> 4, j16 = lane & 15, jq = j16 >> 2;
  const int low = 2 * (g16 & 1) + ((j16 & 3) >> 1);
  unsigned t_base[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    t_base[h] = (unsigned)(8 * h + 4 * lg + jq) * ROW_BYTES +
                (unsigned)((4 * jq + (low ^ ((2 * h + lg) & 3))) * 16) + (unsigned)((j16 & 1) * 8);

  f32x16 dka[D / 32], dva[D / 32], sc, dp;
#pragma unroll
  for (int e = 0; e < D / 32; ++e) {
    dka[e] = f32x16{};
    dva[e] = f32x16{};
  }
  bf16x8 pb[2] = {bf16x8{}, bf16x8{}}, ds[2] = {bf16x8{}, bf16x8{}};

  // (head, first row) of a query tile index, advanced one tile at a time
  struct Cursor {
    int hq, tq0;
  };
  auto advance = [&](Cursor& c) {
    c.tq0 += TILE_ROWS;
    if (c.tq0 >= t_end) {
      c.tq0 = qt_first * TILE_ROWS;
      ++c.hq;
    }
  };
  const Cursor first = {g * G + i_first / n_qt_r, (qt_first + i_first % n_qt_r) * TILE_ROWS};
  // Q and dO rows of batch bi: one descriptor each over its L rows of all heads, so that
  // rows past the shard end read zeros; the head and row go into the scalar offset.
  const dma_rsrc q_rsrc = make_dma_rsrc((const __bf16*)a.q + (int64_t)bi * L * a.h * D, (unsigned)L * q_stride);
  const dma_rsrc o_rsrc = make_dma_rsrc(dout + (int64_t)bi * L * a.h * D, (unsigned)L * q_stride);
  // Load k (0..7) of this wave's share of a tile: k < 4 the Q rows, k >= 4 the dO rows;
  // load i = wq + 4 (k % 4) of the 16 that fill a tile (see dma_tile).
  auto stage_dma_one = [&](const Cursor& c, int buf, int k) __attribute__((always_inline)) {
    const int i = wq + 4 * (k & 3);
    const unsigned dst = RA_LDS_ADDR(smem) + (unsigned)(buf * STAGE_BYTES + (k >> 2) * TILE_BYTES + 1024 * i);
    dma16_to_lds(k < 4 ? q_rsrc : o_rsrc, dst, q_lane_off,
                 (unsigned)c.hq * ROW_BYTES + (unsigned)(c.tq0 + 4 * i) * q_stride);
  };
  auto stage_dma = [&](const Cursor& c, int buf) {   // group 1: all eight
#pragma unroll
    for (int k = 0; k < 8; ++k) stage_dma_one(c, buf, k);
  };
  auto doc_index = [&](const Cursor& c) { return (int64_t)bi * L + min(c.tq0 + lane, L - 1); };
  // The statistics of a tile are written by three waves of group 0 (whose vector phase is
  // the short one), one part each: wave 0 the LSE pairs, wave 1 the D pairs and, with packed
  // documents, wave 2 the key bounds.  `x` is the wave's value for this lane's row.
  const int stat_waves = packed ? 3 : 2;
  auto stats_store = [&](const Cursor& c, int buf, float x, int db, int de) {
    // the lane index passes through an empty asm so that the LDS addresses below are formed
    // here instead of being kept (and spilled) through the main loop
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    const int row = c.tq0 + ln;
    if (wave < 2) {
      // exp2(c2 (S + hi + lo)) = exp(scale S - LSE) with hi + lo = -LSE / scale to about 16
      // bits; rows past the shard end, or with no key anywhere, get -1e30 (weights 0).
      // dP - D the same way with hi + lo = -D.
      // 1 / scale from the hardware reciprocal (within an ulp, far inside the pair's 16
      // bits), formed here: the empty asm keeps it from being hoisted into a register held
      // (and spilled) through the main loop
      float s_ = a.scale;
      __asm__ volatile("" : "+v"(s_));
      const float inv_scale = __builtin_amdgcn_rcpf(s_);
      const float xv = wave == 1 ? -x : (row < L && x > -INFINITY) ? -x * inv_scale : -1e30f;
      const __bf16 x_hi = (__bf16)xv;
      bf16x8 pair = {};
      pair[0] = x_hi;
      pair[1] = (__bf16)(xv - (float)x_hi);
      __bf16* dst = wave == 0 ? &xq_lds[buf][ln][0] : &xo_lds[buf][ln][0];
      *(bf16x8*)dst = pair;
      *(bf16x8*)(dst + 8) = bf16x8{};
      return;
    }
    const KeyRange r = row < L ? range_of(row, db, de) : KeyRange{0, 0};
    lo_lds[buf][ln] = r.lo;
    hi_lds[buf][ln] = r.hi;
    const int half = ln >> 5;
    if ((ln & 31) == 0) {
      cls_lds[buf][half][0] = r.lo;
      cls_lds[buf][half][1] = r.hi;
    }
    if (ln == min(32 * half + 31, L - 1 - c.tq0)) {   // the half's last row in the shard
      cls_lds[buf][half][2] = r.lo;
      cls_lds[buf][half][3] = r.hi;
    }
  };
  auto doc_b = [&](const Cursor& c) { return packed ? a.doc_begin[doc_index(c)] : 0; };
  auto doc_e = [&](const Cursor& c) { return packed ? a.doc_end[doc_index(c)] : 0; };

  // ---- prologue: V rows, tile 0 (and its statistics and those of tile 1) in place ----------
  {
    const int64_t kv_base = ((int64_t)bi * L * a.n_kv + g) * D;
    const dma_rsrc vr = rows_rsrc((const __bf16*)a.v + kv_base, L, kv_stride);
    const unsigned v_lane_off = dma_lane_offset(kv_stride, lane, wave & 3);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = wave + 8 * t;            // i % 4 == wave % 4
      dma16_to_lds(vr, RA_LDS_ADDR(smem) + (unsigned)(V_OFF + 1024 * i), v_lane_off, (unsigned)(u0 + 4 * i) * kv_stride);
    }
    u32x4* z = (u32x4*)(smem + 2 * STAGE_BYTES);   // stage 2 is read (with P = 0) before its first tile
    for (int i = tid; i < STAGE_BYTES / 16; i += KV_THREADS) z[i] = u32x4{};
  }
  Cursor cc = first;                          // tile of the current step
  Cursor cs = first;                          // next tile to stage
  if (grp == 1) stage_dma(cs, 0);
  // this wave's part of the statistics of a tile (waves 0 and 1: LSE and D of the lane's row),
  // addressed by a 32-bit offset from the batch's [h][L] slice (h L < 2^23 for the backward)
  const float* stat_src = (wave == 0 ? lse : delta) + (int64_t)bi * a.h * L;
  auto stat_value = [&](const Cursor& c) {
    return stat_src[(unsigned)(min(c.hq, a.h - 1) * L + min(c.tq0 + lane, L - 1))];
  };
  if (wave < stat_waves) {                  // tiles 0 and 1
    stats_store(cs, 0, stat_value(cs), doc_b(cs), doc_e(cs));
    Cursor c1 = cs;
    advance(c1);
    if (n_iter > 1) stats_store(c1, 1, stat_value(c1), doc_b(c1), doc_e(c1));
  }
  advance(cs);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): V rows and tile 0 are in place
  __syncthreads();

  // ---- main loop ---------------------------------------------------------------------------
  // Every wave runs: matrix phase j, barrier, vector phase j, barrier.  Group 1 executes one
  // extra barrier before the loop and group 0 one after it, so that between barriers 2j and
  // 2j+1 group 0 runs matrix phase j and group 1 vector phase j-1, and between 2j+1 and
  // 2j+2 group 0 runs vector phase j and group 1 matrix phase j.  Tile j (stage j % 3) is
  // read from interval 2j+1 to 2j+4.  Group 1 starts the DMA of tile j in its vector phase
  // j-2 (interval 2j-1; the stage last held tile j-3, read up to interval 2j-2) and waits for
  // it at the end of its matrix phase j-1 (interval 2j), one interval before tile j is first
  // read.  Waves 0-2 load the tile's statistics and store them in their vector phase j-1
  // (interval 2j; first read in interval 2j+1).
  // Matrix phase of tile j (stage BCUR; the previous tile is in stage (BCUR + 2) % 3): 16
  // slots of two products, first dV^T += dO^T P and dK^T += Q^T dS of tile j - 1, then
  // S = Q K^T and dP = dO V^T of tile j.  Slot x issues the LDS reads of slot x + 2, then
  // its products; scheduling fences keep that order so the LDS latency hides behind four
  // products.  The LDS offsets are rebuilt from three base registers each phase (keeping
  // all of them live would not fit the 256 VGPRs of two waves per SIMD).
  // The B operand [k][n = key] of the extra k-step: ones in rows 0 and 1 (and in rows 8 and
  // 9, which meet the zero columns 8 and 9 of the A operand: one constant for every lane).
  // Built where it is used: volatile moves are not hoisted, so the constant does not hold
  // four VGPRs through the loop.
  auto ones_op = []() __attribute__((always_inline)) {
    unsigned w0, w1, w2, w3;
    __asm__ volatile("v_mov_b32 %0, 0x3f803f80" : "=v"(w0));
    __asm__ volatile("v_mov_b32 %0, 0" : "=v"(w1));
    __asm__ volatile("v_mov_b32 %0, 0" : "=v"(w2));
    __asm__ volatile("v_mov_b32 %0, 0" : "=v"(w3));
    return __builtin_bit_cast(bf16x8, u32x4{w0, w1, w2, w3});
  };
  const unsigned x_off = (unsigned)lk * 32 + (unsigned)lg * 16;   // row lk, columns 8 lg ..
  i32x4 cls_v = {};                                               // key bounds of the tile's half
  auto matrix_phase = [&](int bcur) __attribute__((always_inline)) {
    const int bprev = bcur == 0 ? 2 : bcur - 1;
    unsigned rb = r_base, tb0 = t_base[0], tb1 = t_base[1];
    __asm__ volatile("" : "+v"(rb), "+v"(tb0), "+v"(tb1));   // keep the offsets next to their reads
    auto row_op = [&](const char* blk, int kk) { return *(const bf16x8*)(blk + (rb ^ (32u * kk))); };
    auto tr_op = [&](const char* blk, int c, int e) {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(blk + c * 16 * ROW_BYTES + (tb0 ^ (64u * e))));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(blk + c * 16 * ROW_BYTES + (tb1 ^ (64u * e))));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    const char* qc = smem + bcur * STAGE_BYTES + grp * 32 * ROW_BYTES;    // this wave's rows
    const char* oc = qc + TILE_BYTES;
    const char* qp = smem + bprev * STAGE_BYTES + grp * 32 * ROW_BYTES;
    const char* op = qp + TILE_BYTES;
    const char* vt = smem + V_OFF + slot * 32 * ROW_BYTES;
    const char* xq = (const char*)&xq_lds[bcur][32 * grp][0] + x_off;
    const char* xo = (const char*)&xo_lds[bcur][32 * grp][0] + x_off;
    bf16x8 ra[3], rbv[3], rv[3];
    auto load = [&](int y) {
      if (y < 8) {
        ra[y % 3] = tr_op(op, y >> 2, y & 3);
        rbv[y % 3] = tr_op(qp, y >> 2, y & 3);
      } else if (y < 16) {
        ra[y % 3] = row_op(qc, y - 8);
        rbv[y % 3] = row_op(oc, y - 8);
        rv[y % 3] = row_op(vt, y - 8);
      } else {
        ra[y % 3] = *(const bf16x8*)xq;
        rbv[y % 3] = *(const bf16x8*)xo;
      }
    };
    load(0);
    load(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < 17; ++x) {
      if (x + 2 < 17) load(x + 2);
      if (x < 8) {
        dva[x & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[x % 3], pb[x >> 2], dva[x & 3], 0, 0, 0);
        dka[x & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rbv[x % 3], ds[x >> 2], dka[x & 3], 0, 0, 0);
      } else if (x == 8) {
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[x % 3], kop[0], f32x16{}, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rbv[x % 3], rv[x % 3], f32x16{}, 0, 0, 0);
      } else if (x < 16) {
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[x % 3], kop[x - 8], sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rbv[x % 3], rv[x % 3], dp, 0, 0, 0);
      } else {                                // S - LSE / scale, dP - D
        const bf16x8 ones = ones_op();
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[x % 3], ones, sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rbv[x % 3], ones, dp, 0, 0, 0);
      }
      // the tile's key bounds for the vector phase, read once the operand ring drains
      if (x == 15) cls_v = *(const i32x4*)&cls_lds[bcur][grp][0];
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // accumulator layout: lane = key u, register i = row 8 (i / 4) + 4 lg + (i % 4) of the
  // wave's 32-row half.  sc and dp arrive as S - LSE / scale and dP - D.  `stage` (loads for a
  // later tile) goes first so that its copies start early; `mid` runs after the
  // exponentials, by when those loads have had time to land.
  auto vector_phase = [&](int j, int bcur, auto&& stage, auto&& mid) __attribute__((always_inline)) {
    stage();
    __builtin_amdgcn_sched_barrier(0);
    const int r0 = cc.tq0 + 32 * grp;
    // key bounds of the half's first and last row inside the shard: from the two-piece
    // limit on the scalar unit, or with packed documents from the record of the tile
    int lo_first = 0, hi_first, lo_last = 0, hi_last;
    if (packed) {
      lo_first = __builtin_amdgcn_readfirstlane(cls_v[0]);
      hi_first = __builtin_amdgcn_readfirstlane(cls_v[1]);
      lo_last = __builtin_amdgcn_readfirstlane(cls_v[2]);
      hi_last = __builtin_amdgcn_readfirstlane(cls_v[3]);
    } else {
      hi_first = kv_form_eval(kf, r0);
      hi_last = kv_form_eval(kf, min(r0 + 31, L - 1));
    }
    const bool skip = j >= n_iter || r0 >= L || hi_last <= uw || lo_first >= uw + 32;
    const bool full = hi_first >= uw + 32 && lo_last <= uw;   // rows past the shard end have weight 0
    if (!skip) {
      // all products first (in place), then the exponentials: sixteen independent
      // transcendental ops instead of product-exponential pairs through one temporary
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] *= c2;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(sc[i]);
        sc[i] = p;
        dp[i] = p * dp[i];
      }
    }
    mid();                                  // one call site, on every path
    if (skip) {
      pb[0] = pb[1] = ds[0] = ds[1] = bf16x8{};
      return;
    }
    if (!full) {
      // keep this a real (scalar) branch: only diagonal and boundary tiles pay for the mask
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int rr = 32 * grp + 8 * q4 + 4 * lg;
        i32x4 lo4 = {}, hi4;
        if (packed) {
          lo4 = *(const i32x4*)&lo_lds[bcur][rr];
          hi4 = *(const i32x4*)&hi_lds[bcur][rr];
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) hi4[x] = kv_form_eval(kf, cc.tq0 + rr + x);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int i = 4 * q4 + x;
          if (u >= hi4[x] || u < lo4[x] || cc.tq0 + rr + x >= L) {
            sc[i] = 0.f;
            dp[i] = 0.f;
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        pb[c][x] = (__bf16)sc[8 * c + x];
        ds[c][x] = (__bf16)dp[8 * c + x];
      }
  };

  if (grp == 1) {
    if (n_iter > 1) stage_dma(cs, 1);
    barrier_no_fence();
  }
  int bcur = 0;
  for (int j = 0; j <= n_iter; ++j) {
    const int bnext = bcur == 2 ? 0 : bcur + 1;
    const int bnext2 = bcur == 0 ? 2 : bcur - 1;   // stage of tile j + 2 (held tile j - 1)
    __builtin_amdgcn_s_setprio(1);          // matrix phase first in the SIMD's issue arbitration
    matrix_phase(bcur);
    __builtin_amdgcn_s_setprio(0);
    if (grp == 1) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads for tile j + 1 landed
    barrier_no_fence();
    // Group 1 starts the loads of tile j + 2 first in its vector phase.  Waves 0 and 1 (and 2
    // with packed documents) load their part of the statistics of tile j + 1 at the start of
    // theirs and store it after the exponentials (first read after the next barrier; the
    // stage held tile j - 2, whose last reader finished at least two barriers earlier).  The
    // values live only within the phase, so no register carries them across the loop.
    const bool stat_tile = wave < stat_waves && j >= 1 && j + 1 < n_iter;
    Cursor c1 = cc;
    advance(c1);
    // (left unset on the other paths: an initialiser there would make the compiler wait for
    // every outstanding load before writing these registers)
    float st_x;
    int st_b, st_e;
    vector_phase(
        j, bcur,
        [&]() __attribute__((always_inline)) {
          if (grp == 1) {
            if (j + 2 < n_iter) {
              advance(cs);                  // cs: tile j + 2
              stage_dma(cs, bnext2);
            }
          } else {
            st_x = stat_value(c1);
            if (packed) {
              st_b = a.doc_begin[doc_index(c1)];
              st_e = a.doc_end[doc_index(c1)];
            }
          }
        },
        [&]() __attribute__((always_inline)) {
          if (stat_tile) stats_store(c1, bnext, st_x, st_b, st_e);
        });
    if (wave < stat_waves) __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): visible after the barrier
    advance(cc);
    bcur = bnext;
    barrier_no_fence();
  }
  if (grp == 0) barrier_no_fence();

  // ---- the two row halves' dK and dV meet in LDS; group 0 writes ---------------------------
  __syncthreads();
  f32x4* red = (f32x4*)(smem + slot * 32768);   // 2 x 16 x 64 x 16 B per key slot
  if (grp == 1) {
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        red[((0 * 4 + e) * 4 + ib) * 64 + lane] =
            f32x4{dka[e][4 * ib], dka[e][4 * ib + 1], dka[e][4 * ib + 2], dka[e][4 * ib + 3]};
        red[((1 * 4 + e) * 4 + ib) * 64 + lane] =
            f32x4{dva[e][4 * ib], dva[e][4 * ib + 1], dva[e][4 * ib + 2], dva[e][4 * ib + 3]};
      }
  }
  __syncthreads();
  if (grp == 1 || u >= L) return;
  // lane holds dK^T / dV^T [d = 32e + 8 (i/4) + 4 lg + i%4][key u]
  float* krow_out = dk + (((int64_t)bi * L + u) * a.n_kv + g) * D + 4 * lg;
  float* vrow_out = dv + (((int64_t)bi * L + u) * a.n_kv + g) * D + 4 * lg;
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const f32x4 ok = red[((0 * 4 + e) * 4 + ib) * 64 + lane];
      const f32x4 ov = red[((1 * 4 + e) * 4 + ib) * 64 + lane];
      f32x4* pk = (f32x4*)(krow_out + 32 * e + 8 * ib);
      f32x4* pv = (f32x4*)(vrow_out + 32 * e + 8 * ib);
      f32x4 vk = {}, vv = {};
      if (!set_out) {
        vk = *pk;
        vv = *pv;
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        vk[x] += a.scale * (dka[e][4 * ib + x] + ok[x]);
        vv[x] += dva[e][4 * ib + x] + ov[x];
      }
      *pk = vk;
      *pv = vv;
    }
}

// ------------------------------------------------------------------------------------------
// dQ kernel: workgroup = 8 waves x 32 query rows (query heads of one KV group first, as in the
// forward), walking the 64-key tiles of the KV shard.
//
// Wave w holds Q^T and dO^T of its 32 rows in VGPRs; per key tile it computes
// S^T = K Q^T and dP^T = V dO^T (lane = query, so LSE and D are one value per lane),
// dS = P * (dP - D) with P = exp2(S c2 - LSE log2 e), and dQ^T += K^T dS^T (K^T from the
// transposing LDS read).  Ping-pong as in the forward: matrix phase j = dQ of tile j-1
// (16 products) and S, dP of tile j (32 products); vector phase j = dS of tile j.  K tiles
// rotate through four LDS stages (read in matrix phases j and j+1), V tiles through three.
// In its vector phase j group 0 loads V(j+2) and group 1 loads K(j+3), four loads per
// wave, and each wave waits for them at the end of its next vector phase.
// ------------------------------------------------------------------------------------------
constexpr int DQ_THREADS = 512;
constexpr int K_STAGES = 4;
constexpr int V_STAGES = 3;

__global__ __launch_bounds__(DQ_THREADS, 1) void bwd_dq_kernel(StepArgs a, const __bf16* __restrict__ dout,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ delta,
                                                               float* __restrict__ dq, int heads_per_wg,
                                                               int n_qb, int inner_count, int set_out) {
  __shared__ __attribute__((aligned(1024))) char k_lds[K_STAGES][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds[V_STAGES][TILE_BYTES];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int lane = tid & 63, lq = lane & 31, lg = lane >> 5;
  const int L = a.L;
  const int G = a.h / a.n_kv;
  const int Hw = heads_per_wg, PB = 8 / Hw;
  const int inner = blockIdx.x % inner_count;
  const int qb = n_qb - 1 - blockIdx.x / inner_count;   // heaviest query block first
  const int g = inner % a.n_kv;
  const int bi = (inner / a.n_kv) % a.b;
  const int hs = inner / (a.n_kv * a.b);
  const int hq = g * G + hs * Hw + (wave % Hw);
  const int t0_wg = qb * 32 * PB;
  const int t0 = t0_wg + (wave / Hw) * 32;
  const int t = t0 + lq;
  const int tc = min(t, L - 1);
  // allowed keys of row t: [lo, hi), both nondecreasing in t (see key_range); tile classes
  // as in the forward step kernel
  const bool packed = a.doc_begin != nullptr;
  auto range = [&](int row) {
    int64_t db = 0, de = 0;
    if (packed) {
      db = a.doc_begin[(int64_t)bi * L + row];
      de = a.doc_end[(int64_t)bi * L + row];
    }
    return key_range(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, row, packed, db, de);
  };
  const KeyRange rr = t < L ? range(t) : KeyRange{0, 0};
  const int lim = rr.hi, lo = rr.lo;
  int wave_first = 0, wave_tiles = 0, full_begin = 0, full_end = 0, j_begin = 0, n_tiles = 0;
  if (t0 < L) {
    const KeyRange r0 = range(t0), r1 = range(min(t0 + 31, L - 1));
    wave_first = r0.lo / 64;
    wave_tiles = (r1.hi + 63) / 64;
    full_begin = (r1.lo + 63) / 64;
    full_end = r0.hi / 64;
  }
  if (t0_wg < L) {
    j_begin = range(t0_wg).lo / 64;
    n_tiles = (range(min(t0_wg + 32 * PB - 1, L - 1)).hi + 63) / 64;
  }
  wave_first = __builtin_amdgcn_readfirstlane(wave_first);
  wave_tiles = __builtin_amdgcn_readfirstlane(wave_tiles);
  full_begin = __builtin_amdgcn_readfirstlane(full_begin);
  full_end = __builtin_amdgcn_readfirstlane(full_end);
  j_begin = __builtin_amdgcn_readfirstlane(j_begin);
  n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);
  if (n_tiles <= j_begin) {   // uniform over the workgroup: no key of this step is allowed
    if (set_out && t < L) {    // the rows' gradients are zero
      float* zr = dq + (((int64_t)bi * L + t) * a.h + hq) * D + 4 * lg;
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) *(f32x4*)(zr + 32 * e + 8 * ib) = f32x4{};
    }
    return;
  }

  // resident operands: Q^T and dO^T of this lane's query, one row per lane
  const int64_t qrow = (((int64_t)bi * L + tc) * a.h + hq) * D + lg * 8;
  bf16x8 qop[D / 16], dop[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qop[kk] = *(const bf16x8*)((const __bf16*)a.q + qrow + kk * 16);
    dop[kk] = *(const bf16x8*)(dout + qrow + kk * 16);
  }
  const float lse_t = lse[((int64_t)bi * a.h + hq) * L + tc];
  const float neg_lse2 = lse_t > -INFINITY ? -lse_t * LOG2E : -INFINITY;   // empty row: P = 0
  const float dlt = delta[((int64_t)bi * a.h + hq) * L + tc];
  const float c2 = a.scale * LOG2E;

  const unsigned row_stride = (unsigned)a.n_kv * D * 2;
  const int64_t kv_base = ((int64_t)bi * L * a.n_kv + g) * D;
  const dma_rsrc k_rsrc = rows_rsrc((const __bf16*)a.k + kv_base, L, row_stride);
  const dma_rsrc v_rsrc = rows_rsrc((const __bf16*)a.v + kv_base, L, row_stride);
  const unsigned lane_off = dma_lane_offset(row_stride, lane, wave & 3);
  // tile `tile` of K or V into an LDS stage (this wave's four loads); tiles past the last
  // point beyond the buffer: zeros, no memory traffic, into a stage nobody reads again
  auto tile_dma = [&](const dma_rsrc& r, unsigned dst, int tile) {
    dma_tile(r, dst, lane_off, tile < n_tiles ? (unsigned)(tile * 64) * row_stride : 0x80000000u,
             row_stride, wave & 3);
  };

  // LDS read offsets (see the dK/dV kernel): row reads at r_base ^ 32 kk (+ 32 rows per
  // jj), transposing reads at t_base[h] ^ 64 e (+ 16 rows per c)
  const unsigned r_base = (unsigned)lq * ROW_BYTES + (unsigned)((lg ^ swz(lq)) * 16);
  const int g16 = lane >> 4, j16 = lane & 15, jq = j16 >> 2;
  const int low = 2 * (g16 & 1) + ((j16 & 3) >> 1);
  unsigned t_base[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    t_base[h] = (unsigned)(8 * h + 4 * lg + jq) * ROW_BYTES +
                (unsigned)((4 * jq + (low ^ ((2 * h + lg) & 3))) * 16) + (unsigned)((j16 & 1) * 8);

  f32x16 acc[D / 32], sc[2], dp[2];
#pragma unroll
  for (int e = 0; e < D / 32; ++e) acc[e] = f32x16{};
  bf16x8 ds[4] = {bf16x8{}, bf16x8{}, bf16x8{}, bf16x8{}};

  // Matrix phase j: dQ^T += K(j-1)^T dS(j-1)^T (8 slots), then S^T(j) and dP^T(j) (16 slots);
  // slot x issues the reads of slot x + 2, then its two products (scheduling fences).
  auto matrix_phase = [&](int ks, int kp, int vs) __attribute__((always_inline)) {
    unsigned rb = r_base, tb0 = t_base[0], tb1 = t_base[1];
    __asm__ volatile("" : "+v"(rb), "+v"(tb0), "+v"(tb1));   // keep the offsets next to their reads
    const char* kc = k_lds[ks];
    const char* kprev = k_lds[kp];
    const char* vc = v_lds[vs];
    auto row_op = [&](const char* blk, int jj, int kk) {
      return *(const bf16x8*)(blk + jj * 32 * ROW_BYTES + (rb ^ (32u * kk)));
    };
    auto tr_op = [&](const char* blk, int c, int e) {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(blk + c * 16 * ROW_BYTES + (tb0 ^ (64u * e))));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(blk + c * 16 * ROW_BYTES + (tb1 ^ (64u * e))));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    bf16x8 r0[3], r1[3];
    auto load = [&](int y) {
      if (y < 8) {                      // dQ slot: c = y / 2, d-tiles e = 2 (y % 2) + {0, 1}
        r0[y % 3] = tr_op(kprev, y >> 1, 2 * (y & 1));
        r1[y % 3] = tr_op(kprev, y >> 1, 2 * (y & 1) + 1);
      } else {                          // S/dP slot: kk = (y - 8) / 2, jj = (y - 8) % 2
        r0[y % 3] = row_op(kc, (y - 8) & 1, (y - 8) >> 1);
        r1[y % 3] = row_op(vc, (y - 8) & 1, (y - 8) >> 1);
      }
    };
    load(0);
    load(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < 24; ++x) {
      if (x + 2 < 24) load(x + 2);
      if (x < 8) {
        const int c = x >> 1, e = 2 * (x & 1);
        acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r0[x % 3], ds[c], acc[e], 0, 0, 0);
        acc[e + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r1[x % 3], ds[c], acc[e + 1], 0, 0, 0);
      } else {
        const int kk = (x - 8) >> 1, jj = (x - 8) & 1;
        sc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r0[x % 3], qop[kk], kk == 0 ? f32x16{} : sc[jj], 0, 0, 0);
        dp[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r1[x % 3], dop[kk], kk == 0 ? f32x16{} : dp[jj], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Vector phase j: this wave's loads, then dS of tile j (zero where the wave has no tile).
  // Accumulator layout: lane = query, register i of block jj = key
  // 64 j + 32 jj + 8 (i / 4) + 4 lg + (i % 4).
  auto vector_phase = [&](int j, int vs2, int ks3) __attribute__((always_inline)) {
    if (grp == 0) tile_dma(v_rsrc, RA_LDS_ADDR(v_lds) + (unsigned)(vs2 * TILE_BYTES), j + 2);
    else tile_dma(k_rsrc, RA_LDS_ADDR(k_lds) + (unsigned)(ks3 * TILE_BYTES), j + 3);
    if (j >= wave_tiles || j < wave_first) {
#pragma unroll
      for (int c = 0; c < 4; ++c) ds[c] = bf16x8{};
      return;
    }
    if (j < full_begin || j >= full_end) {
      // keep this a real (scalar) branch: only diagonal, boundary and ragged tiles pay for
      // the mask
      __asm__ volatile("" ::: "memory");
      const int thr = lim - (j * 64 + 4 * lg);       // first masked key offset of this row
      const int thr_lo = lo - (j * 64 + 4 * lg);     // first allowed key offset of this row
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int x = 32 * jj + 8 * (i >> 2) + (i & 3);
          if (x >= thr || x < thr_lo) sc[jj][i] = -INFINITY;
        }
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[jj][i], c2, neg_lse2));
        ds[2 * jj + (i >> 3)][i & 7] = (__bf16)(p * (dp[jj][i] - dlt));
      }
  };

  // ---- prologue: K(0), K(1), V(0), V(1) in place, K(2) in flight ----------------------------
  {
    u32x4* z = (u32x4*)k_lds[K_STAGES - 1];   // K(-1): read (with dS = 0) by matrix phase 0
    for (int i = tid; i < TILE_BYTES / 16; i += DQ_THREADS) z[i] = u32x4{};
  }
  if (grp == 1) {
    tile_dma(k_rsrc, RA_LDS_ADDR(k_lds[0]), j_begin);
    tile_dma(k_rsrc, RA_LDS_ADDR(k_lds[1]), j_begin + 1);
  } else {
    tile_dma(v_rsrc, RA_LDS_ADDR(v_lds[0]), j_begin);
    tile_dma(v_rsrc, RA_LDS_ADDR(v_lds[1]), j_begin + 1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  // Intervals between barriers: 2j+1 holds group 0's matrix phase j and group 1's vector
  // phase j-1; 2j+2 group 0's vector phase j and group 1's matrix phase j.  K(j) is read in
  // intervals 2j+1 .. 2j+4, V(j) in 2j+1, 2j+2.  Group 0 loads V(j+2) in interval 2j+2 into
  // the stage of V(j-1) and has it by the end of 2j+4; group 1 loads K(j+3) in 2j+3 into the
  // stage of K(j-1) and has it by the end of 2j+5.
  if (grp == 1) {
    tile_dma(k_rsrc, RA_LDS_ADDR(k_lds[2]), j_begin + 2);
    barrier_no_fence();
  }
  int ks = 0, vs = 0;                     // stages of tile j: counted from j_begin
  for (int j = j_begin; j <= n_tiles; ++j) {
    const int kp = ks == 0 ? K_STAGES - 1 : ks - 1;
    const int ks3 = kp;                               // stage of K(j+3) (held K(j-1))
    const int vs2 = vs == 0 ? V_STAGES - 1 : vs - 1;  // stage of V(j+2) (held V(j-1))
    __builtin_amdgcn_s_setprio(1);        // matrix phase first in the SIMD's issue arbitration
    matrix_phase(ks, kp, vs);
    __builtin_amdgcn_s_setprio(0);
    barrier_no_fence();
    vector_phase(j, vs2, ks3);
    __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4): this wave's loads of its previous vector phase landed
    ks = ks == K_STAGES - 1 ? 0 : ks + 1;
    vs = vs == V_STAGES - 1 ? 0 : vs + 1;
    barrier_no_fence();
  }
  if (grp == 0) barrier_no_fence();
  __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): no load into LDS outlives the loop

  if (t >= L) return;
  float* row = dq + (((int64_t)bi * L + t) * a.h + hq) * D + 4 * lg;
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4* p = (f32x4*)(row + 32 * e + 8 * ib);
      f32x4 v = {};
      if (!set_out) v = *p;
#pragma unroll
      for (int x = 0; x < 4; ++x) v[x] += a.scale * acc[e][4 * ib + x];
      *p = v;
    }
}

// dk[bi][u] += dk2[bi][u] and dv likewise for keys u < rows of every batch row (the second
// halves of split key blocks, which are the first key blocks of the shard); 4 floats a thread.
__global__ __launch_bounds__(256) void add_second_kernel(float* __restrict__ dk, float* __restrict__ dv,
                                                        const float* __restrict__ dk2, const float* __restrict__ dv2,
                                                        int64_t row_floats, int64_t batch_floats, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const int64_t per_b = row_floats / 4;
  const int64_t off = (i / per_b) * batch_floats + (i % per_b) * 4;
  f32x4 a = *(const f32x4*)(dk + off), b = *(const f32x4*)(dk2 + off);
  *(f32x4*)(dk + off) = a + b;
  a = *(const f32x4*)(dv + off);
  b = *(const f32x4*)(dv2 + off);
  *(f32x4*)(dv + off) = a + b;
}

}  // namespace

hipError_t launch_bwd_preprocess(const void* o, const void* dout, float* delta, int b, int L, int h,
                                 hipStream_t s) {
  const int64_t rows = (int64_t)b * L * h;
  const int64_t threads = rows * 16;
  hipLaunchKernelGGL(bwd_preprocess_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     (const __bf16*)o, (const __bf16*)dout, delta, L, h, rows);
  return hipGetLastError();
}

hipError_t launch_step_bwd_bf16(const StepArgs& a, const void* dout, const float* lse,
                                const float* delta, float* dq, float* dk, float* dv, hipStream_t s,
                                bool set_dq, bool set_dkdv, float* dk2, float* dv2) {
  const int G = a.h / a.n_kv;
  const int Hw = (G % 4 == 0) ? 4 : ((G % 2 == 0) ? 2 : 1);
  const int PB = 8 / Hw;
  const int n_qb = (a.L + 32 * PB - 1) / (32 * PB);
  const int inner = a.n_kv * a.b * (G / Hw);
  const int64_t grid_q = (int64_t)n_qb * inner;
  const int n_kb = (a.L + KB - 1) / KB;
  const int64_t grid_k = (int64_t)n_kb * a.n_kv * a.b;
  if (grid_q > 0x7fffffff || grid_k > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)grid_q), dim3(DQ_THREADS), 0, s, a,
                     (const __bf16*)dout, lse, delta, dq, Hw, n_qb, inner, (int)set_dq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const KvForm kf = make_kv_form(a.causal, a.layout, a.N, a.L, a.q_shard, a.kv_shard);
  // Key blocks whose (head, query tile) iterations run as two workgroups: only while the key
  // blocks leave compute units idle (as the forward's steps), from their iteration counts (the
  // query tiles from the first row that sees the block to the shard end, times G: no packed
  // documents here, so every row's keys are a prefix).  Item i of the plan's order is key block
  // n_kb - 1 - (its block index): the heaviest blocks are the first keys.
  SplitPlan plan{};
  plan.split_from = n_kb;
  if (dk2 && dv2 && set_dkdv && !a.doc_begin && n_kb <= kSplitMaxBlocks) {
    int w[kSplitMaxBlocks], wp[kSplitMaxBlocks];
    const int n_qt = (a.L + TILE_ROWS - 1) / TILE_ROWS;
    for (int kbp = 0; kbp < n_kb; ++kbp) {
      const int u0 = (n_kb - 1 - kbp) * KB;
      int lo = 0, hi = a.L;             // first row whose key limit passes u0
      while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (kv_limit(a.causal, a.layout, a.N, a.L, a.q_shard, a.kv_shard, mid) > u0) hi = mid;
        else lo = mid + 1;
      }
      w[kbp] = lo < a.L ? (n_qt - lo / TILE_ROWS) * G : 0;
      wp[kbp] = (w[kbp] + 1) / 2;
    }
    plan = plan_from_costs(w, wp, n_kb, device_cu_count() / (a.n_kv * a.b), false);
  }
  const int64_t grid_kp = (int64_t)(plan.split_from + 2 * (n_kb - plan.split_from)) * a.n_kv * a.b;
  if (grid_kp > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)grid_kp), dim3(KV_THREADS), 0, s, a,
                     (const __bf16*)dout, lse, delta, dk, dv, kf, (int)set_dkdv, plan, dk2, dv2);
  if ((e = hipGetLastError()) != hipSuccess || plan.split_from >= n_kb) return e;
  const int rows = min(a.L, (n_kb - plan.split_from) * KB);      // keys of the split blocks
  const int64_t row_floats = (int64_t)rows * a.n_kv * D, n4 = (int64_t)a.b * row_floats / 4;
  hipLaunchKernelGGL(add_second_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, dk, dv, dk2, dv2,
                     row_floats, (int64_t)a.L * a.n_kv * D, n4);
  return hipGetLastError();
}

}  // namespace ra

// Internal declarations shared by the HIP sources of libra.  Not part of the C-ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra.h"

namespace ra {

// ---------------------------------------------------------------------------------------
// Global position of local token t of shard p (page 1, "Causal Masking Dynamics: Striped
// Attention and Zig-Zag Topologies"; page 3, section 6):
//   contiguous: shard p holds the consecutive tokens [pL, pL + L)
//   striped:    token g lives on shard g mod N, so local t of shard p is global tN + p
//   zigzag:     2N chunks of C = L/2 tokens; shard p holds chunk p, then chunk 2N-1-p
// In every layout a shard's positions increase with t.
// ---------------------------------------------------------------------------------------
__host__ __device__ inline int64_t global_pos(int layout, int N, int L, int p, int t) {
  if (layout == RA_LAYOUT_STRIPED) return (int64_t)t * N + p;
  if (layout == RA_LAYOUT_ZIGZAG) {
    const int C = L / 2;
    return t < C ? (int64_t)p * C + t : (int64_t)(2 * N - 1 - p) * C + (t - C);
  }
  return (int64_t)p * L + t;
}

// Inverse of global_pos: the shard j and local index t holding global position P
// (0 <= P < N L).
__host__ __device__ inline void owner_of(int layout, int N, int L, int64_t P, int& j, int& t) {
  if (layout == RA_LAYOUT_STRIPED) {
    j = (int)(P % N);
    t = (int)(P / N);
  } else if (layout == RA_LAYOUT_ZIGZAG) {
    const int C = L / 2;
    const int c = (int)(P / C);
    const int off = (int)(P - (int64_t)c * C);
    if (c < N) {
      j = c;
      t = off;
    } else {
      j = 2 * N - 1 - c;
      t = C + off;
    }
  } else {
    j = (int)(P / L);
    t = (int)(P - (int64_t)j * L);
  }
}

__host__ __device__ inline int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// ---------------------------------------------------------------------------------------
// Key limit of query row t of shard qs against KV shard ks.
//
// The causal mask allows key u of shard ks for query t of shard qs iff
// pos(ks, u) <= pos(qs, t) (inclusive; page 1, a token attends to positions j <= i).
// Because positions increase with the local index in every layout, the allowed keys of a
// row always form a prefix [0, limit) of the KV shard.  The mask of a whole (q-tile,
// k-tile) pair therefore reduces to integer comparisons of key indices against per-row
// limits: a k-tile is skipped when it starts at or beyond the largest limit of the
// q-tile, needs no mask when it ends at or below the smallest one, and is masked only in
// between (the diagonal).  Non-causal: every key is allowed.
// ---------------------------------------------------------------------------------------
__host__ __device__ inline int kv_limit(int causal, int layout, int N, int L, int qs, int ks,
                                        int t) {
  if (!causal) return L;
  if (layout == RA_LAYOUT_STRIPED) {
    // keys of shard ks sit at uN + ks and query t at tN + qs; since |qs - ks| < N,
    // uN + ks <= tN + qs holds exactly for u <= t when ks <= qs and for u < t otherwise
    const int lim = t + (qs >= ks ? 1 : 0);
    return lim < 0 ? 0 : (lim > L ? L : lim);
  }
  const int64_t P = global_pos(layout, N, L, qs, t);
  if (layout == RA_LAYOUT_ZIGZAG) {
    const int C = L / 2;
    const int64_t a = clamp64(P - (int64_t)ks * C + 1, 0, C);
    const int64_t b = clamp64(P - (int64_t)(2 * N - 1 - ks) * C + 1, 0, C);
    return (int)(a + b);
  }
  return (int)clamp64(P - (int64_t)ks * L + 1, 0, L);
}

// The same limit as two clamped linear pieces, for kernels that evaluate it per tile on the
// scalar unit: kv_limit(t) = clamp(t + o1, 0, c1) + clamp(t + o2, 0, c2), with (o1, o2) =
// (o1a, o2a) for t < split and (o1b, o2b) otherwise.  Zigzag needs both pieces (the shard's
// two chunks, split at L/2); the other layouts one.  Offsets are clamped to [-(L+2), L+2],
// which leaves every clamp of t + o for 0 <= t < L unchanged.
struct KvForm {
  int split, o1a, o2a, o1b, o2b, c1, c2;
};
inline KvForm make_kv_form(int causal, int layout, int N, int L, int qs, int ks) {
  auto c = [&](int64_t o) { return (int)clamp64(o, -(int64_t)L - 2, (int64_t)L + 2); };
  if (!causal) return KvForm{0, 0, 0, L, 0, L, 0};
  if (layout == RA_LAYOUT_STRIPED) {
    const int o = qs >= ks ? 1 : 0;
    return KvForm{0, o, 0, o, 0, L, 0};
  }
  if (layout == RA_LAYOUT_ZIGZAG) {
    const int64_t C = L / 2;
    return KvForm{(int)C,
                  c((int64_t)(qs - ks) * C + 1), c((int64_t)(qs + ks - 2 * N + 1) * C + 1),
                  c((int64_t)(2 * N - 2 - qs - ks) * C + 1), c((int64_t)(ks - qs - 1) * C + 1),
                  (int)C, (int)C};
  }
  const int o = c((int64_t)(qs - ks) * L + 1);
  return KvForm{0, o, 0, o, 0, L, 0};
}
__host__ __device__ inline int kv_form_eval(const KvForm& f, int t) {
  const bool lo = t < f.split;
  const int a = t + (lo ? f.o1a : f.o1b), b = t + (lo ? f.o2a : f.o2b);
  return (a < 0 ? 0 : (a > f.c1 ? f.c1 : a)) + (b < 0 ? 0 : (b > f.c2 ? f.c2 : b));
}

// ---------------------------------------------------------------------------------------
// Asynchronous global -> LDS copy (buffer_load_dwordx4 ... lds): every lane moves the 16
// bytes at voffset + soffset of the buffer to LDS address lds_base + 16 * lane.  Reads at
// or past the descriptor's num_records bytes return zeros.  The copy is issued through
// inline assembly, so the compiler does not track it: it would otherwise wait for every
// outstanding copy before each later LDS read, including reads of other buffers.  The
// caller owns the wait: s_waitcnt vmcnt before any wave reads the destination, then a
// barrier, and the destination must not be read or written between the call and that
// wait.  M0 carries the LDS base; no compiler-generated code in these kernels uses M0.
// ---------------------------------------------------------------------------------------
typedef int dma_rsrc __attribute__((ext_vector_type(4)));

__device__ __forceinline__ dma_rsrc make_dma_rsrc(const void* base, unsigned num_records) {
  const uint64_t b = (uint64_t)base;
  return dma_rsrc{(int)__builtin_amdgcn_readfirstlane((unsigned)b),
                  (int)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32) & 0xFFFFu),
                  (int)__builtin_amdgcn_readfirstlane(num_records), 0x00020000};
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 32-bit LDS byte address of a __shared__ object: taken from the object itself (a link-time
// constant), so that stage and slot offsets stay plain scalar integer arithmetic instead of
// generic-pointer arithmetic with its null checks.
#define RA_LDS_ADDR(obj) ((unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)(obj))

// One 1 KB LDS-DMA load: 16 bytes per lane from the buffer at voffset + soffset into LDS at
// lds_addr + 16 lane (lds_addr is wave-uniform).
__device__ __forceinline__ void dma16_to_lds(dma_rsrc rsrc, unsigned lds_addr, unsigned voffset,
                                             unsigned soffset) {
  // s_nop: one wait state between writing M0 and an LDS-DMA load that reads it.  No memory
  // clobber: the destination is never read before the caller's wait and barrier, and the
  // compiler may keep scheduling LDS reads of other buffers around the load.
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voffset), "s"(rsrc),
                     "s"(__builtin_amdgcn_readfirstlane(soffset))
                   : "m0");
}
#pragma clang diagnostic pop

// ---------------------------------------------------------------------------------------
// Number of keys of shard ks whose global position is < X (X may lie anywhere; the count is
// clamped to [0, L]).  Positions increase with the local index, so these keys are a prefix.
// ---------------------------------------------------------------------------------------
__host__ __device__ inline int count_below(int layout, int N, int L, int ks, int64_t X) {
  if (layout == RA_LAYOUT_STRIPED) {
    // keys at uN + ks < X  <=>  u < (X - ks) / N, rounded up
    if (X <= ks) return 0;
    return (int)clamp64((X - ks + N - 1) / N, 0, L);
  }
  if (layout == RA_LAYOUT_ZIGZAG) {
    const int C = L / 2;
    const int64_t a = clamp64(X - (int64_t)ks * C, 0, C);
    const int64_t b = clamp64(X - (int64_t)(2 * N - 1 - ks) * C, 0, C);
    return (int)(a + b);
  }
  return (int)clamp64(X - (int64_t)ks * L, 0, L);
}

// ---------------------------------------------------------------------------------------
// Allowed keys of query row t (shard qs) in KV shard ks: the local index range [lo, hi).
// Without packed documents lo = 0 and hi = kv_limit.  With them (page 3, section 5:
// documents packed into one window, no attention across documents) the row may only see
// positions in [doc_begin, doc_end) of its own document, intersected with the causal rule;
// since positions increase with the local index this is again one index range.
// doc_begin / doc_end hold the row's document bounds (global positions) for this batch row.
// ---------------------------------------------------------------------------------------
struct KeyRange {
  int lo, hi;
};
__host__ __device__ inline KeyRange key_range(int causal, int layout, int N, int L, int qs, int ks,
                                              int t, bool packed, int64_t doc_begin, int64_t doc_end) {
  if (!packed) return KeyRange{0, kv_limit(causal, layout, N, L, qs, ks, t)};
  int64_t end = doc_end;
  if (causal) {
    const int64_t P = global_pos(layout, N, L, qs, t);
    end = end < P + 1 ? end : P + 1;
  }
  const int lo = count_below(layout, N, L, ks, doc_begin);
  const int hi = count_below(layout, N, L, ks, end);
  return KeyRange{lo, hi > lo ? hi : lo};
}

// Epilogue of a forward step kernel.
enum StepMode : int {
  MODE_PART = 0,   // write this step's normalised (O, LSE) partial
  MODE_MERGE = 1,  // merge this step's partial into (O_acc, LSE_acc) in place
};

struct StepArgs {
  const void* q;       // [b][L][h][d]
  const void* k;       // [b][L][n_kv][d]
  const void* v;       // [b][L][n_kv][d]
  float* o;            // [b][L][h][d] fp32: partial (MODE_PART) or accumulator (MODE_MERGE)
  float* lse;          // [b][h][L]    fp32
  int b, L, h, n_kv, d, N;
  int causal, layout;
  int q_shard, kv_shard;
  float scale;         // softmax scale on q.k
  const int32_t* doc_begin;   // [b][L] packed-document bounds of each query row, or null
  const int32_t* doc_end;
  // Second accumulator of a forward pass, [b][L][h][d] and [b][h][L] fp32 (bf16 step kernel
  // only; null: none).  With it the step kernel may run the key range of its heaviest query
  // blocks as two work items, the second one writing (MODE_PART) or merging (MODE_MERGE) its
  // partial here; MODE_PART also sets lse2 to -inf on every row no second item covers, so
  // after the first step of a pass every row of (o2, lse2) is a valid partial or empty.
  // Rows with lse2 = -inf may hold anything in o2.
  float* o2 = nullptr;
  float* lse2 = nullptr;
  // Last step of a forward pass (bf16 step kernel, MODE_PART or MODE_MERGE, no second
  // accumulator): the merged rows, and the accumulator rows this step does not change, are
  // written here as bf16 [b][L][h][d] (rounded to nearest even) instead of to `o`; lse still
  // receives the final LSE.  Null: write `o`.
  __bf16* o_out = nullptr;
};

// Several consecutive ring steps in one launch of the bf16 step kernel: steps k_first ..
// k_first + n - 1 of the pass of a.q_shard, i.e. KV shards (q_shard - k) mod N, whose K and V
// sit at k + i stride and v + i stride bytes (i = k - k_first), each laid out as StepArgs::k
// and ::v.  a.k, a.v and a.kv_shard are not used.
struct ShardBatch {
  const void* k = nullptr;
  const void* v = nullptr;
  int64_t stride = 0;
  int k_first = 0;
  int n = 0;
};
constexpr int kMaxBatch = 128;
hipError_t launch_step_bf16(const StepArgs& a, int mode, hipStream_t s);
hipError_t launch_steps_bf16(const StepArgs& a, const ShardBatch& sb, int mode, hipStream_t s);
hipError_t launch_step_f32(const StepArgs& a, int mode, hipStream_t s);
hipError_t launch_merge(float* o_acc, float* lse_acc, const float* o_part,
                        const float* lse_part, int b, int L, int h, int d, hipStream_t s);
hipError_t launch_finalize(const float* o_acc, void* o, int dtype, int64_t n_elems,
                           hipStream_t s);
hipError_t launch_fill_lse(float* lse, int64_t n, float value, hipStream_t s);
// The ring's K/V receive for steps k0 .. k0 + n_steps - 1 of device qs, in one launch: step
// k copies K and V of shard (qs - k) mod N from k_all, v_all ([N] shards of shard_bytes,
// a multiple of 16) to kdst and vdst + (k - k0) stride.
hipError_t launch_stage_kv(char* kdst, char* vdst, const void* k_all, const void* v_all, int64_t shard_bytes,
                           int64_t stride, int N, int qs, int k0, int n_steps, hipStream_t s);
// Fold the second accumulator (o2, lse2) of a forward pass into (o, lse), row by row (rows
// with lse2 = -inf keep (o, lse) and never read o2).  With out null, o is updated in place in
// fp32; otherwise the folded rows (and the untouched ones) are written to out in bf16 and o is
// only read.  lse is updated in place either way.
hipError_t launch_fold_second(float* o, float* lse, const float* o2, const float* lse2, void* out, int b, int L,
                              int h, int d, hipStream_t s);

// Work items of a bf16 forward step whose heaviest query blocks are split over two
// workgroups: blocks [split_from, n_qb) run as two items each, part 0 on the first half of
// the block's key tiles (rounded up) and part 1 on the rest.  Item i (launch order) is an
// unsplit block when bit i of `order` is set: the k-th such item is block split_from - 1 - k;
// otherwise the m-th part item is part m % 2 of block n_qb - 1 - m / 2.  Any bit pattern with
// split_from ones among the first split_from + 2 (n_qb - split_from) bits maps the items one
// to one onto the (block, part) pairs; the host picks one that launches the heaviest first.
// With split_from = n_qb nothing is split and item i is block n_qb - 1 - i.
struct SplitPlan {
  uint32_t order[4];   // up to 128 items
  int split_from;
};
constexpr int kSplitMaxBlocks = 64;
__host__ __device__ inline void split_item(const SplitPlan& pl, int n_qb, int item, int& qb, int& part) {
  part = 0;
  if (pl.split_from >= n_qb) {
    qb = n_qb - 1 - item;
    return;
  }
  const int word = item >> 5;
  const uint32_t w = word == 0 ? pl.order[0] : word == 1 ? pl.order[1] : word == 2 ? pl.order[2] : pl.order[3];
  int before = __builtin_popcount(w & ((1u << (item & 31)) - 1u));
  if (word > 0) before += __builtin_popcount(pl.order[0]);
  if (word > 1) before += __builtin_popcount(pl.order[1]);
  if (word > 2) before += __builtin_popcount(pl.order[2]);
  if ((w >> (item & 31)) & 1u) {
    qb = pl.split_from - 1 - before;
  } else {
    const int m = item - before;
    qb = n_qb - 1 - (m >> 1);
    part = m & 1;
  }
}
// The plan of one step (host), for a pass with a second accumulator: geometry as
// launch_step_bf16 uses it, n_cu compute units.
struct StepGeometry {
  int Hw, PB, n_qb, inner, rows_wg;
};
StepGeometry step_geometry_bf16(const StepArgs& a);
SplitPlan plan_split(const StepArgs& a, const StepGeometry& g, int n_cu);
// The plan from per-block costs in tiles (w whole, wp the longer part; both nondecreasing in
// the block index): with by_makespan the split point of the shortest list schedule over the
// units, else only while the blocks leave units idle (at most one item per unit).
SplitPlan plan_from_costs(const int* w, const int* wp, int n_qb, int units, bool by_makespan);
// Compute units of the current device (looked up once per device; 256 if the query fails).
inline int device_cu_count() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
  }
  return n;
}
// The same for a launch of several ring steps (launch_steps_bf16 with a second accumulator):
// a split block runs each of its KV shards' key ranges as two halves, one per part.
SplitPlan plan_split_batch(const StepArgs& a, const ShardBatch& sb, const StepGeometry& g, int n_cu);
// Whether launch_step_bf16 would split any query block of this step (given a second
// accumulator) on the current device.
bool step_splits_bf16(const StepArgs& a);
// Whether launch_steps_bf16 would split any query block of this batch (given a second
// accumulator) on the current device.
bool steps_split_bf16(const StepArgs& a, const ShardBatch& sb);

// Largest shard length for which a forward pass keeps a second accumulator, so that its steps
// can split the key ranges of their heaviest query blocks (below it a step has too few
// workgroups to fill the chip, or the causal imbalance between query blocks is not evened
// out by running several blocks per compute unit).
constexpr int kSplitMaxL = 4096;

// (O, LSE) of two partials over disjoint key sets, merged (page 2, "FlashAttention
// Integration": each partial is rescaled by its share of the combined denominator).  One
// definition for every kernel that merges a second accumulator, so that all paths round the
// same way: explicit FMA, no contraction left to the compiler.
struct MergeWeights {
  float f1, f2, lse;
};
__device__ __forceinline__ MergeWeights merge_weights(float l1, float l2) {
  const float M = fmaxf(l1, l2);
  const float w1 = __builtin_amdgcn_exp2f((l1 - M) * 1.4426950408889634f);
  const float w2 = __builtin_amdgcn_exp2f((l2 - M) * 1.4426950408889634f);
  const float tot = w1 + w2;
  return MergeWeights{w1 / tot, w2 / tot, M + __logf(tot)};
}
__device__ __forceinline__ float merge_value(const MergeWeights& m, float o1, float o2) {
  return __builtin_fmaf(m.f1, o1, m.f2 * o2);
}
// Head-group exchange of the all-to-all sequence-parallel scheme, one device's side.
// Gather: rows [b][S][Hg][d] (element bytes es) of heads head0 .. head0+Hg-1, in global
// position order, from the N shards src_all [N][b][L][H][d] in their own layout order.
hipError_t launch_ulysses_gather(void* dst, const void* src_all, int b, int L, int N, int layout,
                                 int H, int Hg, int head0, int d, int es, hipStream_t s);
// Scatter: fp32 rows [b][S][Hg][d] back to heads head0 .. of the shards' dst_all
// [N][b][L][H][d] (converted to dtype), and LSE [b][Hg][S] to lse_all [N][b][H][L].
hipError_t launch_ulysses_scatter(void* dst_all, float* lse_all, const float* o, const float* lse,
                                  int b, int L, int N, int layout, int H, int Hg, int head0, int d,
                                  int dtype, hipStream_t s);
// Per-row statistics [N][b][H][L] (heads head0 ..) -> [b][Hg][S] in global position order.
hipError_t launch_ulysses_gather_rows(float* dst, const float* src_all, int b, int L, int N, int layout, int H,
                                      int Hg, int head0, hipStream_t s);
// Rows [b][S][Hg][d] fp32 -> heads head0 .. of dst_all [N][b][L][H][d] (converted to dtype).
hipError_t launch_ulysses_scatter_rows(void* dst_all, const float* src, int b, int L, int N, int layout, int H,
                                       int Hg, int head0, int d, int dtype, hipStream_t s);
hipError_t launch_bwd_preprocess(const void* o, const void* dout, float* delta, int b, int L, int h,
                                 hipStream_t s);
// Adds this step's contributions to dq [b][L][h][d], dk and dv [b][L][n_kv][d] (fp32), or,
// with set_dq / set_dkdv, stores them there in place of what the buffer held (every row of
// the shard is written, zeros where the step contributes nothing).
// With dk2, dv2 ([b][L][n_kv][d] fp32, any contents; only with set_dkdv and no packed
// documents) the dK/dV kernel may run the query tiles of a key block as two workgroups when
// the key blocks leave compute units idle: the second half's dK, dV go to dk2, dv2 and are
// added into dk, dv after the kernel.
hipError_t launch_step_bwd_bf16(const StepArgs& a, const void* dout, const float* lse,
                                const float* delta, float* dq, float* dk, float* dv, hipStream_t s,
                                bool set_dq = false, bool set_dkdv = false, float* dk2 = nullptr,
                                float* dv2 = nullptr);

}  // namespace ra

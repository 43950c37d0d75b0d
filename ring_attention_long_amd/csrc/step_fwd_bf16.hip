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
//  * On gfx950 a wave's vector instructions do not run underneath its own matrix
//    instructions, but the vector unit of a SIMD does run one wave's softmax while the
//    matrix unit runs another wave's products.  So a workgroup is 8 wave64s, two per SIMD,
//    in two groups that swap roles every half step (a "ping-pong"): while group 0 issues
//    its matrix phase (P V of the previous key tile and Q K^T of the current one), group 1
//    runs the softmax of its current tile, and the other way round in the next half step.
//    A workgroup barrier separates the half steps.
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
//    in which the contraction visits keys is free as long as A and B agree.  V is staged
//    into LDS transposed (Vt[d][key]) so its A operand is two 8-byte LDS reads.
//  * Online softmax in base 2 with scale * log2(e) folded into one FMA per score, and a
//    lazy rescale: the running maximum used for exponentiation moves only when a row's new
//    maximum exceeds it by more than TAU (= 8, so P <= 2^8); the final O / l is unchanged
//    in exact arithmetic, and most tiles skip the O *= alpha pass.
//  * Causal masking (page 1, "Causal Masking Dynamics"): with positions increasing inside
//    every shard, the allowed keys of a row are a prefix [0, limit) of the KV shard, so a
//    wave skips every key tile at or beyond its largest limit, runs maskless below its
//    smallest limit, and masks only the diagonal tiles in between.
//  * K/V tiles are double-buffered in LDS and staged during the softmax halves: group 0
//    writes K tiles, group 1 writes V tiles (transposed), each into the buffer the other
//    group has finished reading, and each then issues the global loads of its next tile a
//    full step before that tile is written.
//  * Workgroups are launched heaviest query block first (causal work grows with the query
//    position), with the KV head as the fastest-varying index so that neighbouring
//    workgroups, dispatched round-robin over the 8 XCDs, put each KV head's tiles into
//    one XCD's L2.
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;            // head dimension
constexpr int BN = 64;            // keys per tile
constexpr int QW = 32;            // query rows per wave
constexpr int WAVES = 8;          // two per SIMD
constexpr int THREADS = 64 * WAVES;
constexpr int STAGERS = 256;      // threads per group; each group stages one of K, V
constexpr int KPITCH = D + 8;     // bf16 per K row in LDS: 272 B, rows shift by 4 banks
constexpr int VPITCH = BN + 4;    // bf16 per Vt row in LDS: 136 B, rows shift by 2 banks
constexpr int K_TILE = BN * KPITCH;
constexpr int V_TILE = D * VPITCH;
constexpr float TAU = 8.0f;       // lazy-rescale threshold, log2 units
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

__device__ __forceinline__ u32x4 load16(const __bf16* p) { return *(const u32x4*)p; }

template <int MODE>
__global__ __launch_bounds__(THREADS, 1) void step_fwd_bf16_kernel(StepArgs a, int heads_per_wg,
                                                                  int n_qb, int inner_count) {
  __shared__ __bf16 k_lds[2][K_TILE];
  __shared__ __bf16 vt_lds[2][V_TILE];

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
  const int qb = n_qb - 1 - blockIdx.x / inner_count;   // heaviest query block first
  const int g = inner % a.n_kv;
  const int bi = (inner / a.n_kv) % a.b;
  const int hs = inner / (a.n_kv * a.b);
  const int hq = g * G + hs * Hw + (wave % Hw);
  const int t0_wg = qb * QW * PB;
  const int t0 = t0_wg + (wave / Hw) * QW;
  const int t = t0 + lq;                // this lane's query row

  const __bf16* qp = (const __bf16*)a.q;
  const __bf16* kp = (const __bf16*)a.k;
  const __bf16* vp = (const __bf16*)a.v;
  const int64_t kv_row = (int64_t)a.n_kv * D;          // elements between keys
  const int64_t kv_base = ((int64_t)bi * L * a.n_kv + g) * D;

  // ---- key limits and tile ranges ---------------------------------------------------
  const int lim = t < L ? kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, t) : 0;
  int wave_tiles = 0, wave_full = 0;
  if (t0 < L) {
    const int t_last = min(t0 + QW - 1, L - 1);
    wave_tiles = (kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, t_last) + BN - 1) / BN;
    wave_full = kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, t0) / BN;
  }
  wave_tiles = __builtin_amdgcn_readfirstlane(wave_tiles);
  wave_full = __builtin_amdgcn_readfirstlane(wave_full);
  int n_tiles = 0;
  if (t0_wg < L) {
    const int t_last = min(t0_wg + QW * PB - 1, L - 1);
    n_tiles = (kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, t_last) + BN - 1) / BN;
  }
  n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);

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
  f32x16 sc[2];
  bf16x8 pb[4];
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.scale * LOG2E;

  // ---- tile staging: global -> registers -> LDS ----------------------------------------
  // Group 0 stages K tiles: 64 keys x 16 chunks of 16 B, a straight copy.  Group 1 stages
  // V tiles: thread (kq, dc) loads 4 keys x 8 d and writes 8 transposed 8-byte rows
  // Vt[d][4 keys].  Each group keeps one tile in flight in `sreg`.
  const int st = tid & (STAGERS - 1);
  const int kq = st & 15, dc = st >> 4;
  u32x4 sreg[4];
  // Rows past the shard end are clamped to row L-1: those keys are always masked, so any
  // finite values will do, and the loads need no per-lane guard.
  auto load_tile = [&](int j) {
    if (group == 0) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int u = min(j * BN + (st >> 4) + 16 * it, L - 1);
        sreg[it] = load16(kp + kv_base + (int64_t)u * kv_row + (st & 15) * 8);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = min(j * BN + kq * 4 + r, L - 1);
        sreg[r] = load16(vp + kv_base + (int64_t)u * kv_row + dc * 8);
      }
    }
  };
  auto store_tile = [&](int buf) {
    if (group == 0) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int idx = st + STAGERS * it;
        *(u32x4*)&k_lds[buf][(idx >> 4) * KPITCH + (idx & 15) * 8] = sreg[it];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int w = i >> 1;
        unsigned lo, hi;
        if (i & 1) {
          lo = (sreg[0][w] >> 16) | (sreg[1][w] & 0xffff0000u);
          hi = (sreg[2][w] >> 16) | (sreg[3][w] & 0xffff0000u);
        } else {
          lo = (sreg[0][w] & 0xffffu) | (sreg[1][w] << 16);
          hi = (sreg[2][w] & 0xffffu) | (sreg[3][w] << 16);
        }
        *(u32x2*)&vt_lds[buf][(dc * 8 + i) * VPITCH + kq * 4] = u32x2{lo, hi};
      }
    }
  };

  // ---- the two phases of one wave ------------------------------------------------------
  // Operands of the two products, read from LDS.  V^T operand of chunk c (16 keys), d-tile
  // e: Vt[32e + lq][16c + 4lg .. +4] and [.. + 8 .. +4].  K operand of d-step kk, key
  // sub-tile jj: K[32jj + lq][16kk + 8lg .. +8].
  auto v_operand = [&](const __bf16* vt, int c, int e) {
    const __bf16* vr = vt + (32 * e + lq) * VPITCH + 16 * c + 4 * lg;
    const u32x2 lo = *(const u32x2*)vr;
    const u32x2 hi = *(const u32x2*)(vr + 8);
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
  };
  auto k_operand = [&](const __bf16* kt, int kk, int jj) {
    return *(const bf16x8*)(kt + (32 * jj + lq) * KPITCH + kk * 16 + lg * 8);
  };
  // Matrix phase of step j: O^T += V(j-1)^T P(j-1)^T and S^T(j) = K(j) Q^T.  In the steady
  // state both run interleaved, one MFMA of each per slot (6 independent accumulators),
  // with each slot's two LDS operands fetched two slots ahead.
  auto matrix_phase = [&](int j) {
    const bool do_pv = j >= 1 && j - 1 < wave_tiles;
    const bool do_qk = j < wave_tiles;
    const __bf16* vt = vt_lds[(j - 1) & 1];
    const __bf16* kt = k_lds[j & 1];
    if (do_pv && do_qk) {
      sc[0] = f32x16{};
      sc[1] = f32x16{};
      bf16x8 va[3], ka[3];
      va[0] = v_operand(vt, 0, 0);
      ka[0] = k_operand(kt, 0, 0);
      va[1] = v_operand(vt, 0, 1);
      ka[1] = k_operand(kt, 0, 1);
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        if (x + 2 < 16) {
          va[(x + 2) % 3] = v_operand(vt, (x + 2) >> 2, (x + 2) & 3);
          ka[(x + 2) % 3] = k_operand(kt, (x + 2) >> 1, (x + 2) & 1);
        }
        acc[x & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[x % 3], pb[x >> 2], acc[x & 3], 0, 0, 0);
        sc[x & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[x % 3], qop[x >> 1], sc[x & 1], 0, 0, 0);
      }
#pragma unroll
      for (int x = 0; x < 14; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // the next slot's LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // this slot's two MFMAs
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      return;
    }
    if (do_pv) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < D / 32; ++e)
          acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(vt, c, e), pb[c], acc[e], 0, 0, 0);
    }
    if (do_qk) {
      sc[0] = f32x16{};
      sc[1] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          sc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(kt, kk, jj), qop[kk], sc[jj], 0, 0, 0);
    }
  };
  // Softmax phase of step j: mask, running max, lazy rescale, P = exp2(S c - m), row sum.
  auto softmax_phase = [&](int j) {
    if (j < 0 || j >= wave_tiles) return;
    if (j >= wave_full) {
      // keep this a real (scalar) branch: only diagonal and ragged tiles pay for the mask
      __asm__ volatile("" ::: "memory");
      const int thr = lim - (j * BN + 4 * lg);       // first masked key offset of this row
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * jj + 8 * (i >> 2) + (i & 3) >= thr) sc[jj][i] = -INFINITY;
    }
    float mx;
    {
      float x0 = fmaxf(fmaxf(sc[0][0], sc[0][1]), sc[0][2]);
      float x1 = fmaxf(fmaxf(sc[1][0], sc[1][1]), sc[1][2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) {
        x0 = fmaxf(fmaxf(x0, sc[0][i]), sc[0][i + 1]);
        x1 = fmaxf(fmaxf(x1, sc[1][i]), sc[1][i + 1]);
      }
      x0 = fmaxf(fmaxf(x0, sc[0][15]), x1);
      x0 = fmaxf(x0, sc[1][15]);
      mx = lane_pair_max(x0) * c2;
    }
    if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < D / 32; ++e) acc[e] *= alpha;
      m_run = m_new;
    }
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[0][i], c2, neg_m));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[1][i], c2, neg_m));
      sc[0][i] = p0;
      sc[1][i] = p1;
      rs0 += p0;
      rs1 += p1;
    }
    l_run += rs0 + rs1;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int x = 0; x < 8; ++x) pb[c][x] = (__bf16)sc[c >> 1][8 * (c & 1) + x];
  };
  // ---- main loop -------------------------------------------------------------------------
  // Every wave runs the same sequence: matrix phase of step j, barrier, softmax phase of
  // step j (plus its share of the staging: group 0 writes K(j+1), group 1 writes V(j+1),
  // each then fetching the tile after), barrier.  Group 1 executes one extra barrier before
  // the loop and group 0 one after it, so group 1 runs half a step behind group 0 and the
  // two groups of each SIMD alternate between matrix and vector work.  Buffer lifetimes,
  // counted in half steps h (group 0 runs phase h, group 1 phase h - 1):
  //   K(j) is read at h = 2j, 2j+1 and written (by group 0) at h = 2j-1;
  //   V(j) is read at h = 2j+2, 2j+3 and written (by group 1) at h = 2j;
  // so a write never touches the buffer of the other parity being read.
  if (n_tiles > 0) {          // prologue: K(0) and V(0) in LDS, K(1) and V(1) in flight
    load_tile(0);
    store_tile(0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): Q is in registers before the loop
  if (n_tiles > 1) load_tile(1);
  __syncthreads();
  if (group == 1) __syncthreads();
  for (int j = 0; j <= n_tiles; ++j) {
    matrix_phase(j);
    __syncthreads();
    softmax_phase(j);
    if (j + 1 < n_tiles) {
      store_tile((j + 1) & 1);
      if (j + 2 < n_tiles) load_tile(j + 2);
    }
    __syncthreads();
  }
  if (group == 0) __syncthreads();

  // ---- epilogue ------------------------------------------------------------------------
  const float l_tot = lane_pair_sum(l_run);
  if (t >= L) return;
  const bool any = l_tot > 0.f;
  const float lse_new = any ? (m_run + __log2f(l_tot)) * LN2 : -INFINITY;
  const float inv = any ? 1.f / l_tot : 0.f;
  float* orow = a.o + (((int64_t)bi * L + t) * a.h + hq) * D + 4 * lg;
  float* lse_p = a.lse + ((int64_t)bi * a.h + hq) * L + t;
  if (MODE == MODE_PART) {
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4 v = {acc[e][4 * ib] * inv, acc[e][4 * ib + 1] * inv, acc[e][4 * ib + 2] * inv,
                   acc[e][4 * ib + 3] * inv};
        *(f32x4*)(orow + 32 * e + 8 * ib) = v;
      }
    if (lg == 0) *lse_p = lse_new;
  } else {
    if (!any) return;   // nothing allowed in this step: the accumulator is unchanged
    const float lse_old = *lse_p;
    const float M = fmaxf(lse_old, lse_new);
    const float wa = __builtin_amdgcn_exp2f((lse_old - M) * LOG2E);
    const float wb = __builtin_amdgcn_exp2f((lse_new - M) * LOG2E);
    const float tot = wa + wb;
    const float fa = wa / tot, fb = wb * inv / tot;
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4* dst = (f32x4*)(orow + 32 * e + 8 * ib);
        const f32x4 old = *dst;
        f32x4 v;
#pragma unroll
        for (int x = 0; x < 4; ++x) v[x] = fa * old[x] + fb * acc[e][4 * ib + x];
        *dst = v;
      }
    if (lg == 0) *lse_p = M + __logf(tot);
  }
}

}  // namespace

hipError_t launch_step_bf16(const StepArgs& a, int mode, hipStream_t stream) {
  const int G = a.h / a.n_kv;
  const int Hw = (G % 4 == 0) ? 4 : ((G % 2 == 0) ? 2 : 1);
  const int PB = WAVES / Hw;
  const int n_qb = (a.L + QW * PB - 1) / (QW * PB);
  const int inner = a.n_kv * a.b * (G / Hw);
  const int64_t grid = (int64_t)n_qb * inner;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (mode == MODE_PART)
    hipLaunchKernelGGL(step_fwd_bf16_kernel<MODE_PART>, dim3((unsigned)grid), dim3(THREADS), 0,
                       stream, a, Hw, n_qb, inner);
  else
    hipLaunchKernelGGL(step_fwd_bf16_kernel<MODE_MERGE>, dim3((unsigned)grid), dim3(THREADS), 0,
                       stream, a, Hw, n_qb, inner);
  return hipGetLastError();
}

}  // namespace ra

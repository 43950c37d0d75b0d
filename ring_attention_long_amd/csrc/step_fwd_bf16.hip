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
//  * A workgroup is 4 wave64s that share one KV head.  With grouped-query attention the
//    query heads of one KV group go to different waves (page 3, section 2: several query
//    heads share one KV group), so every K/V tile staged in LDS feeds up to 4 heads.
//  * Each wave owns 64 query rows = two 32-row sub-tiles.  Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T held in VGPRs
//    for the whole kernel).  In the 32x32 accumulator layout lane l then holds 16 keys of
//    ONE query (column l % 32), so the row max and row sum are plain per-lane reductions
//    plus one exchange with lane l ^ 32 (v_permlane32_swap); no reductions over 32 lanes.
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
//  * K/V tiles are double-buffered in LDS: the global loads of tile j+1 are issued before
//    the matrix work on tile j and written to LDS after it, one barrier per tile.
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
constexpr int QW = 64;            // query rows per wave
constexpr int THREADS = 256;      // 4 waves
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
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;   // query column inside a 32-row sub-tile
  const int lg = lane >> 5;   // which half of the key rows of the accumulator

  const int L = a.L;
  const int G = a.h / a.n_kv;
  const int Hw = heads_per_wg;          // heads handled by this workgroup (1, 2 or 4)
  const int P = 4 / Hw;                 // 64-row query blocks handled by this workgroup
  const int inner = blockIdx.x % inner_count;
  const int qb = n_qb - 1 - blockIdx.x / inner_count;   // heaviest query block first
  const int g = inner % a.n_kv;
  const int bi = (inner / a.n_kv) % a.b;
  const int hs = inner / (a.n_kv * a.b);
  const int hq = g * G + hs * Hw + (wave % Hw);
  const int t0_wg = qb * QW * P;
  const int t0 = t0_wg + (wave / Hw) * QW;

  const __bf16* qp = (const __bf16*)a.q;
  const __bf16* kp = (const __bf16*)a.k;
  const __bf16* vp = (const __bf16*)a.v;
  const int64_t kv_row = (int64_t)a.n_kv * D;          // elements between keys
  const int64_t kv_base = ((int64_t)bi * L * a.n_kv + g) * D;

  // ---- per-row key limits and tile ranges -------------------------------------------
  int lim[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int t = t0 + 32 * s + lq;
    lim[s] = t < L ? kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, t) : 0;
  }
  int wave_tiles = 0, wave_full = 0;
  if (t0 < L) {
    const int t_last = min(t0 + QW - 1, L - 1);
    wave_tiles = (kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, t_last) + BN - 1) / BN;
    wave_full = kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, t0) / BN;
  }
  int n_tiles = 0;
  {
    const int t_last = min(t0_wg + QW * P - 1, L - 1);
    if (t0_wg < L)
      n_tiles = (kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, t_last) + BN - 1) / BN;
  }

  // ---- Q^T operands, resident for the whole kernel -----------------------------------
  bf16x8 qop[2][D / 16];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int t = t0 + 32 * s + lq;
    const __bf16* row = qp + (((int64_t)bi * L + t) * a.h + hq) * D + lg * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (t < L) qop[s][kk] = *(const bf16x8*)(row + kk * 16);
      else qop[s][kk] = bf16x8{};
    }
  }

  f32x16 acc[D / 32][2];
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int s = 0; s < 2; ++s) acc[e][s] = f32x16{};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  const float c2 = a.scale * LOG2E;

  // ---- tile staging: global -> registers -> LDS ---------------------------------------
  // K: 64 keys x 16 chunks of 16 B, straight copy.  V: thread (kq, dc) loads 4 keys x 8 d
  // and writes 8 transposed 8-byte rows Vt[d][4 keys].
  const int kq = tid & 15, dc = tid >> 4;
  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int j) {
    const int kv0 = j * BN;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = tid + THREADS * it;
      const int u = kv0 + (idx >> 4);
      kreg[it] = u < L ? load16(kp + kv_base + (int64_t)u * kv_row + (idx & 15) * 8) : u32x4{};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int u = kv0 + kq * 4 + r;
      vreg[r] = u < L ? load16(vp + kv_base + (int64_t)u * kv_row + dc * 8) : u32x4{};
    }
  };
  auto store_tile = [&](int st) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = tid + THREADS * it;
      *(u32x4*)&k_lds[st][(idx >> 4) * KPITCH + (idx & 15) * 8] = kreg[it];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int w = i >> 1;
      unsigned lo, hi;
      if (i & 1) {
        lo = (vreg[0][w] >> 16) | (vreg[1][w] & 0xffff0000u);
        hi = (vreg[2][w] >> 16) | (vreg[3][w] & 0xffff0000u);
      } else {
        lo = (vreg[0][w] & 0xffffu) | (vreg[1][w] << 16);
        hi = (vreg[2][w] & 0xffffu) | (vreg[3][w] << 16);
      }
      *(u32x2*)&vt_lds[st][(dc * 8 + i) * VPITCH + kq * 4] = u32x2{lo, hi};
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int st = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1);

    if (j < wave_tiles) {
      const int kv0 = j * BN;
      // ---- S^T = K Q^T --------------------------------------------------------------
      f32x16 sc[2][2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int s = 0; s < 2; ++s) sc[jj][s] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const bf16x8 ka = *(const bf16x8*)&k_lds[st][(32 * jj + lq) * KPITCH + kk * 16 + lg * 8];
#pragma unroll
          for (int s = 0; s < 2; ++s)
            sc[jj][s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[s][kk], sc[jj][s], 0, 0, 0);
        }
      }
      // ---- diagonal / ragged tiles: mask keys at or beyond each row's limit -----------
      if (j >= wave_full) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kv0 + 32 * jj + 8 * (i >> 2) + 4 * lg + (i & 3);
              if (key >= lim[s]) sc[jj][s][i] = -INFINITY;
            }
      }
      // ---- online softmax --------------------------------------------------------------
      float mx[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float x = sc[0][s][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) x = fmaxf(x, sc[0][s][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) x = fmaxf(x, sc[1][s][i]);
        mx[s] = lane_pair_max(x) * c2;
      }
      const bool grow = (mx[0] > m_run[0] + TAU) || (mx[1] > m_run[1] + TAU);
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const float m_new = fmaxf(m_run[s], mx[s]);
          const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[s] - m_new);
          l_run[s] *= alpha;
#pragma unroll
          for (int e = 0; e < D / 32; ++e) acc[e][s] *= alpha;
          m_run[s] = m_new;
        }
      }
      bf16x8 pb[4][2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const float neg_m = m_run[s] == -INFINITY ? 0.f : -m_run[s];
        float rs = 0.f;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[jj][s][i], c2, neg_m));
            sc[jj][s][i] = p;
            rs += p;
          }
        l_run[s] += rs;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int t = 0; t < 8; ++t) pb[c][s][t] = (__bf16)sc[c >> 1][s][8 * (c & 1) + t];
      }
      // ---- O^T += V^T P^T ---------------------------------------------------------------
#pragma unroll
      for (int e = 0; e < D / 32; ++e) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const __bf16* vr = &vt_lds[st][(32 * e + lq) * VPITCH + 16 * c + 4 * lg];
          const u32x2 lo = *(const u32x2*)vr;
          const u32x2 hi = *(const u32x2*)(vr + 8);
          const u32x4 w = u32x4{lo[0], lo[1], hi[0], hi[1]};
          const bf16x8 va = __builtin_bit_cast(bf16x8, w);
#pragma unroll
          for (int s = 0; s < 2; ++s)
            acc[e][s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c][s], acc[e][s], 0, 0, 0);
        }
      }
    }

    if (j + 1 < n_tiles) store_tile(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------------------
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int t = t0 + 32 * s + lq;
    const float l_tot = lane_pair_sum(l_run[s]);
    if (t >= L) continue;
    const bool any = l_tot > 0.f;
    const float lse_new = any ? (m_run[s] + __log2f(l_tot)) * LN2 : -INFINITY;
    const float inv = any ? 1.f / l_tot : 0.f;
    float* orow = a.o + (((int64_t)bi * L + t) * a.h + hq) * D + 4 * lg;
    float* lse_p = a.lse + ((int64_t)bi * a.h + hq) * L + t;
    if (MODE == MODE_PART) {
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          f32x4 v = {acc[e][s][4 * ib] * inv, acc[e][s][4 * ib + 1] * inv,
                     acc[e][s][4 * ib + 2] * inv, acc[e][s][4 * ib + 3] * inv};
          *(f32x4*)(orow + 32 * e + 8 * ib) = v;
        }
      if (lg == 0) *lse_p = lse_new;
    } else {
      if (!any) continue;   // nothing allowed in this step: the accumulator is unchanged
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
          for (int x = 0; x < 4; ++x) v[x] = fa * old[x] + fb * acc[e][s][4 * ib + x];
          *dst = v;
        }
      if (lg == 0) *lse_p = M + __logf(tot);
    }
  }
}

}  // namespace

hipError_t launch_step_bf16(const StepArgs& a, int mode, hipStream_t stream) {
  const int G = a.h / a.n_kv;
  const int Hw = (G % 4 == 0) ? 4 : ((G % 2 == 0) ? 2 : 1);
  const int P = 4 / Hw;
  const int n_qb = (a.L + QW * P - 1) / (QW * P);
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

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
//    per lane; dQ^T += K^T dS^T with K^T read by the transposing LDS load.
//  * dK/dV kernel (key-major): each wave keeps K and V rows of 32 keys in VGPRs and walks
//    the query tiles of every head of its KV group; S = Q K^T and dP = dO V^T put one key
//    per lane, and dV^T += dO^T P, dK^T += Q^T dS take dO^T and Q^T from transposing LDS
//    loads.  No atomics: every workgroup owns its keys.
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
constexpr int THREADS = 256;
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
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rsrc, char* dst, unsigned lane_off,
                                         unsigned row0_off, unsigned row_stride, int w) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = w + 4 * t;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + 1024 * i), 16, lane_off,
                                             row0_off + (unsigned)(4 * i) * row_stride, 0, 0);
  }
}
// Buffer descriptor covering rows 0..rows-1 (row_stride bytes apart, 256 B each) from base;
// reads beyond return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int rows,
                                                            unsigned row_stride) {
  const int n = rows > 0 ? (int)((unsigned)(rows - 1) * row_stride + ROW_BYTES) : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, n, 0x00020000);
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
// dQ kernel: workgroup = 4 waves x 32 query rows (heads of one KV group first), 64-key tiles.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(THREADS, 1) void bwd_dq_kernel(StepArgs a, const __bf16* __restrict__ dout,
                                                            const float* __restrict__ lse,
                                                            const float* __restrict__ delta,
                                                            float* __restrict__ dq, int heads_per_wg,
                                                            int n_qb, int inner_count) {
  __shared__ __attribute__((aligned(1024))) char k_lds[2][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds[2][TILE_BYTES];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lq = lane & 31, lg = lane >> 5;
  const int L = a.L;
  const int G = a.h / a.n_kv;
  const int Hw = heads_per_wg, PB = 4 / Hw;
  const int inner = blockIdx.x % inner_count;
  const int qb = n_qb - 1 - blockIdx.x / inner_count;
  const int g = inner % a.n_kv;
  const int bi = (inner / a.n_kv) % a.b;
  const int hs = inner / (a.n_kv * a.b);
  const int hq = g * G + hs * Hw + (wave % Hw);
  const int t0_wg = qb * 32 * PB;
  const int t0 = t0_wg + (wave / Hw) * 32;
  const int t = t0 + lq;
  const int tc = min(t, L - 1);

  const int lim = t < L ? kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, t) : 0;
  int wave_tiles = 0, wave_full = 0, n_tiles = 0;
  if (t0 < L) {
    wave_tiles = (kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, min(t0 + 31, L - 1)) + 63) / 64;
    wave_full = kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, t0) / 64;
  }
  if (t0_wg < L)
    n_tiles = (kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, min(t0_wg + 32 * PB - 1, L - 1)) + 63) / 64;
  wave_tiles = __builtin_amdgcn_readfirstlane(wave_tiles);
  wave_full = __builtin_amdgcn_readfirstlane(wave_full);
  n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);

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
  const __amdgpu_buffer_rsrc_t k_rsrc = rows_rsrc((const __bf16*)a.k + kv_base, L, row_stride);
  const __amdgpu_buffer_rsrc_t v_rsrc = rows_rsrc((const __bf16*)a.v + kv_base, L, row_stride);
  const unsigned lane_off = dma_lane_offset(row_stride, lane, wave);

  f32x16 acc[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e) acc[e] = f32x16{};

  if (n_tiles > 0) {
    dma_tile(k_rsrc, k_lds[0], lane_off, 0, row_stride, wave);
    dma_tile(v_rsrc, v_lds[0], lane_off, 0, row_stride, wave);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) {
      dma_tile(k_rsrc, k_lds[buf ^ 1], lane_off, (unsigned)((j + 1) * 64) * row_stride, row_stride, wave);
      dma_tile(v_rsrc, v_lds[buf ^ 1], lane_off, (unsigned)((j + 1) * 64) * row_stride, row_stride, wave);
    }
    if (j < wave_tiles) {
      const char* kt = k_lds[buf];
      const char* vt = v_lds[buf];
      f32x16 sc[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          sc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_chunk(kt, 32 * jj + lq, 2 * kk + lg),
                                                           qop[kk], sc[jj], 0, 0, 0);
          dp[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_chunk(vt, 32 * jj + lq, 2 * kk + lg),
                                                           dop[kk], dp[jj], 0, 0, 0);
        }
      const bool masked = j >= wave_full;
      bf16x8 ds[4];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j * 64 + 32 * jj + 8 * (i >> 2) + 4 * lg + (i & 3);
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[jj][i], c2, neg_lse2));
          if (masked && key >= lim) p = 0.f;
          const float v = p * (dp[jj][i] - dlt);
          ds[2 * jj + (i >> 3)][i & 7] = (__bf16)v;
        }
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < D / 32; ++e)
          acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rows_transposed(kt, lane, c, e), ds[c], acc[e], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  if (t >= L) return;
  float* row = dq + (((int64_t)bi * L + t) * a.h + hq) * D + 4 * lg;
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4* p = (f32x4*)(row + 32 * e + 8 * ib);
      f32x4 v = *p;
#pragma unroll
      for (int x = 0; x < 4; ++x) v[x] += a.scale * acc[e][4 * ib + x];
      *p = v;
    }
}

// ------------------------------------------------------------------------------------------
// dK/dV kernel: workgroup = 4 waves x 32 keys of one KV head; loops over the query tiles
// (64 rows) of every head of the KV group.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(THREADS, 1) void bwd_dkdv_kernel(StepArgs a, const __bf16* __restrict__ dout,
                                                              const float* __restrict__ lse,
                                                              const float* __restrict__ delta,
                                                              float* __restrict__ dk, float* __restrict__ dv,
                                                              int n_kb) {
  __shared__ __attribute__((aligned(1024))) char q_lds[2][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char o_lds[2][TILE_BYTES];   // dO tiles
  __shared__ float lse_lds[2][TILE_ROWS];
  __shared__ float dlt_lds[2][TILE_ROWS];
  __shared__ int lim_lds[2][TILE_ROWS];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lk = lane & 31, lg = lane >> 5;
  const int L = a.L;
  const int G = a.h / a.n_kv;
  const int kb = (int)(blockIdx.x / (a.n_kv * a.b));   // keys early in the shard see more queries: first
  const int g = blockIdx.x % a.n_kv;
  const int bi = (blockIdx.x / a.n_kv) % a.b;
  const int u0 = kb * 128;
  const int uw = u0 + 32 * wave;            // this wave's first key
  const int u = uw + lk;                    // this lane's key
  const int uc = min(u, L - 1);

  // resident K and V rows of this lane's key (B operands [k = d][n = key])
  const int64_t krow = (((int64_t)bi * L + uc) * a.n_kv + g) * D + lg * 8;
  bf16x8 kop[D / 16], vop[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    kop[kk] = *(const bf16x8*)((const __bf16*)a.k + krow + kk * 16);
    vop[kk] = *(const bf16x8*)((const __bf16*)a.v + krow + kk * 16);
  }
  // first query row that may see key u0 (limits are nondecreasing in the query index)
  int t_lo = 0, t_hi = L;
  while (t_lo < t_hi) {
    const int mid = (t_lo + t_hi) >> 1;
    if (kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, mid) > u0) t_hi = mid;
    else t_lo = mid + 1;
  }
  const int qt_first = t_lo / TILE_ROWS;
  const int n_qt = (L + TILE_ROWS - 1) / TILE_ROWS - qt_first;   // query tiles per head
  const int n_iter = n_qt > 0 ? n_qt * G : 0;
  const float c2 = a.scale * LOG2E;
  const unsigned q_stride = (unsigned)a.h * D * 2;
  const unsigned lane_off = dma_lane_offset(q_stride, lane, wave);

  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e) {
    dka[e] = f32x16{};
    dva[e] = f32x16{};
  }

  // stage query tile `it` (head g*G + it / n_qt, tile qt_first + it % n_qt)
  auto stage = [&](int it, int buf) {
    const int hq = g * G + it / n_qt;
    const int tq0 = (qt_first + it % n_qt) * TILE_ROWS;
    const int64_t base = ((int64_t)bi * L * a.h + hq) * D;
    const __amdgpu_buffer_rsrc_t qr = rows_rsrc((const __bf16*)a.q + base, L, q_stride);
    const __amdgpu_buffer_rsrc_t orr = rows_rsrc(dout + base, L, q_stride);
    dma_tile(qr, q_lds[buf], lane_off, (unsigned)tq0 * q_stride, q_stride, wave);
    dma_tile(orr, o_lds[buf], lane_off, (unsigned)tq0 * q_stride, q_stride, wave);
    if (tid < TILE_ROWS) {
      const int tq = tq0 + tid;
      const int64_t li = ((int64_t)bi * a.h + hq) * L + min(tq, L - 1);
      const float l = lse[li];
      lse_lds[buf][tid] = l > -INFINITY ? -l * LOG2E : -INFINITY;   // stored negated, base 2
      dlt_lds[buf][tid] = delta[li];
      lim_lds[buf][tid] = tq < L ? kv_limit(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, tq) : 0;
    }
  };

  if (n_iter > 0) stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    if (it + 1 < n_iter) stage(it + 1, buf ^ 1);
    const int tq0 = (qt_first + it % n_qt) * TILE_ROWS;
    // skip when no query of the tile may see this wave's keys (limits grow with the
    // query index; rows past the shard end have limit 0)
    const int lim_last = lim_lds[buf][min(TILE_ROWS - 1, L - 1 - tq0)];
    if (__builtin_amdgcn_readfirstlane(lim_last) > uw) {
      const char* qt = q_lds[buf];
      const char* ot = o_lds[buf];
      f32x16 sc[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          sc[qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_chunk(qt, 32 * qs + lk, 2 * kk + lg),
                                                           kop[kk], sc[qs], 0, 0, 0);
          dp[qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_chunk(ot, 32 * qs + lk, 2 * kk + lg),
                                                           vop[kk], dp[qs], 0, 0, 0);
        }
      // accumulator layout: lane = key u, register i of block qs = query
      // tq0 + 32 qs + 8 (i/4) + 4 lg + (i%4)
      bf16x8 pb[4], ds[4];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int r0 = 32 * qs + 8 * q4 + 4 * lg;
          const f32x4 l4 = *(const f32x4*)&lse_lds[buf][r0];
          const f32x4 d4 = *(const f32x4*)&dlt_lds[buf][r0];
          const i32x4 m4 = *(const i32x4*)&lim_lds[buf][r0];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int i = 4 * q4 + x;
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qs][i], c2, l4[x]));
            if (u >= m4[x]) p = 0.f;
            const float s = p * (dp[qs][i] - d4[x]);
            pb[2 * qs + (i >> 3)][i & 7] = (__bf16)p;
            ds[2 * qs + (i >> 3)][i & 7] = (__bf16)s;
          }
        }
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < D / 32; ++e) {
          dva[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rows_transposed(ot, lane, c, e), pb[c], dva[e], 0, 0, 0);
          dka[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rows_transposed(qt, lane, c, e), ds[c], dka[e], 0, 0, 0);
        }
    }
    (void)tq0;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }
  if (u >= L) return;
  // lane holds dK^T / dV^T [d = 32e + 8 (i/4) + 4 lg + i%4][key u]
  float* krow_out = dk + (((int64_t)bi * L + u) * a.n_kv + g) * D + 4 * lg;
  float* vrow_out = dv + (((int64_t)bi * L + u) * a.n_kv + g) * D + 4 * lg;
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4* pk = (f32x4*)(krow_out + 32 * e + 8 * ib);
      f32x4* pv = (f32x4*)(vrow_out + 32 * e + 8 * ib);
      f32x4 vk = *pk, vv = *pv;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        vk[x] += a.scale * dka[e][4 * ib + x];
        vv[x] += dva[e][4 * ib + x];
      }
      *pk = vk;
      *pv = vv;
    }
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
                                const float* delta, float* dq, float* dk, float* dv, hipStream_t s) {
  const int G = a.h / a.n_kv;
  const int Hw = (G % 4 == 0) ? 4 : ((G % 2 == 0) ? 2 : 1);
  const int PB = 4 / Hw;
  const int n_qb = (a.L + 32 * PB - 1) / (32 * PB);
  const int inner = a.n_kv * a.b * (G / Hw);
  const int64_t grid_q = (int64_t)n_qb * inner;
  const int n_kb = (a.L + 127) / 128;
  const int64_t grid_k = (int64_t)n_kb * a.n_kv * a.b;
  if (grid_q > 0x7fffffff || grid_k > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)grid_q), dim3(THREADS), 0, s, a,
                     (const __bf16*)dout, lse, delta, dq, Hw, n_qb, inner);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)grid_k), dim3(THREADS), 0, s, a,
                     (const __bf16*)dout, lse, delta, dk, dv, n_kb);
  return hipGetLastError();
}

}  // namespace ra

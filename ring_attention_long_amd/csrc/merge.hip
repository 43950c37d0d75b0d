// Bandwidth-bound kernels around the ring: the (O, LSE) merge of two partial results, the
// final cast of the fp32 accumulator to the output type, and the fold of a pass's second
// accumulator (the split key ranges of short shards) into the first.
//
// Merge (page 2, "FlashAttention Integration"; page 3, section 3): the two partials are
// normalised outputs over disjoint key sets with denominators exp(lse_acc) and
// exp(lse_part).  Around M = max(lse_acc, lse_part) the weights are
// wa = exp(lse_acc - M), wb = exp(lse_part - M); the merged row is (wa O_acc + wb O_part)
// / (wa + wb) with LSE M + ln(wa + wb).  (0, -inf) is the identity and a pair of empty
// rows stays (0, -inf).
//
// Each thread owns 4 consecutive floats (16-byte loads and stores); the d/4 threads of a
// row sit in one wave, so every lane reads the row's old LSE before the lane holding the
// row's first column overwrites it.
#include <algorithm>

#include "ra_internal.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void merge_kernel(float* __restrict__ o_acc,
                                                    float* __restrict__ lse_acc,
                                                    const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part,
                                                    int L, int h, int d4, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const int64_t row = i / d4;                 // row = (bi * L + t) * h + hq
  const int col4 = (int)(i - row * d4);
  const int hq = (int)(row % h);
  const int64_t bt = row / h;
  const int t = (int)(bt % L);
  const int64_t bi = bt / L;
  const int64_t li = (bi * h + hq) * L + t;
  const float la = lse_acc[li], lb = lse_part[li];
  const float M = fmaxf(la, lb);
  f32x4 out = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (M != -INFINITY) {
    const float wa = expf(la - M), wb = expf(lb - M);
    const float tot = wa + wb;
    const float fa = wa / tot, fb = wb / tot;
    const f32x4 x = ((const f32x4*)o_acc)[i];
    const f32x4 y = ((const f32x4*)o_part)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = fa * x[e] + fb * y[e];
    lse = M + logf(tot);
  }
  ((f32x4*)o_acc)[i] = out;
  if (col4 == 0) lse_acc[li] = lse;
}

__global__ __launch_bounds__(256) void finalize_bf16_kernel(const float* __restrict__ src,
                                                            __bf16* __restrict__ dst,
                                                            int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = ((const f32x4*)src)[2 * i];
  const f32x4 b = ((const f32x4*)src)[2 * i + 1];
  __bf16 r[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (__bf16)a[e];       // round to nearest even
    r[4 + e] = (__bf16)b[e];
  }
  ((u32x4*)dst)[i] = __builtin_bit_cast(u32x4, r);
}

// Fold of a forward pass's second accumulator (see launch_fold_second): one thread per 8
// consecutive floats of a row, the d/8 threads of a row in one wave (every lane reads the
// row's LSE before the lane holding the row's first columns overwrites it).
template <bool TO_BF16>
__global__ __launch_bounds__(256) void fold_second_kernel(float* __restrict__ o, float* __restrict__ lse,
                                                          const float* __restrict__ o2,
                                                          const float* __restrict__ lse2,
                                                          __bf16* __restrict__ out, int L, int h, int d8,
                                                          int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const int64_t row = i / d8;                 // row = (bi * L + t) * h + hq
  const int col8 = (int)(i - row * d8);
  const int hq = (int)(row % h);
  const int64_t bt = row / h;
  const int t = (int)(bt % L);
  const int64_t bi = bt / L;
  const int64_t li = (bi * h + hq) * L + t;
  const float l2 = lse2[li];
  f32x4 a = ((const f32x4*)o)[2 * i];
  f32x4 b = ((const f32x4*)o)[2 * i + 1];
  if (l2 > -INFINITY) {                       // otherwise o2's row is undefined and not read
    const MergeWeights m = merge_weights(lse[li], l2);
    const f32x4 c = ((const f32x4*)o2)[2 * i];
    const f32x4 e = ((const f32x4*)o2)[2 * i + 1];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      a[x] = merge_value(m, a[x], c[x]);
      b[x] = merge_value(m, b[x], e[x]);
    }
    if (!TO_BF16) {
      ((f32x4*)o)[2 * i] = a;
      ((f32x4*)o)[2 * i + 1] = b;
    }
    if (col8 == 0) lse[li] = m.lse;
  }
  if (TO_BF16) {
    __bf16 r[8];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      r[x] = (__bf16)a[x];       // round to nearest even
      r[4 + x] = (__bf16)b[x];
    }
    ((u32x4*)out)[i] = __builtin_bit_cast(u32x4, r);
  }
}

__global__ __launch_bounds__(256) void copy_f32_kernel(const float* __restrict__ src,
                                                       float* __restrict__ dst, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) ((f32x4*)dst)[i] = ((const f32x4*)src)[i];
}

// The K/V receive of ring steps k0 .. k0 + gridDim.y - 1 of device qs: step k gets the shard
// of device (qs - k) mod N, K into kdst + (k - k0) stride and V into vdst + (k - k0) stride.
// blockIdx.y: the step, blockIdx.z: K (0) or V (1); 16 bytes per thread and iteration.
__global__ __launch_bounds__(256) void stage_kv_kernel(char* __restrict__ kdst, char* __restrict__ vdst,
                                                       const char* __restrict__ k_all,
                                                       const char* __restrict__ v_all, int64_t shard_bytes,
                                                       int64_t stride, int N, int qs, int k0) {
  const int k = k0 + (int)blockIdx.y;
  const int src = ((qs - k) % N + N) % N;
  const u32x4* from = (const u32x4*)((blockIdx.z ? v_all : k_all) + (int64_t)src * shard_bytes);
  u32x4* to = (u32x4*)((blockIdx.z ? vdst : kdst) + (int64_t)blockIdx.y * stride);
  const int64_t n16 = shard_bytes / 16;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    to[i] = from[i];
}

__global__ __launch_bounds__(256) void fill_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                        int b, int L, int h, int d, hipStream_t s) {
  const int64_t n4 = (int64_t)b * L * h * d / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(blocks_for(n4)), dim3(256), 0, s, o_acc, lse_acc, o_part,
                     lse_part, L, h, d / 4, n4);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* o_acc, void* o, int dtype, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (dtype == RA_BF16) {
    hipLaunchKernelGGL(finalize_bf16_kernel, dim3(blocks_for(n / 8)), dim3(256), 0, s, o_acc,
                       (__bf16*)o, n / 8);
  } else {
    if ((const void*)o_acc == o) return hipSuccess;
    hipLaunchKernelGGL(copy_f32_kernel, dim3(blocks_for(n / 4)), dim3(256), 0, s, o_acc,
                       (float*)o, n / 4);
  }
  return hipGetLastError();
}

hipError_t launch_fold_second(float* o, float* lse, const float* o2, const float* lse2, void* out, int b, int L,
                              int h, int d, hipStream_t s) {
  const int64_t n8 = (int64_t)b * L * h * d / 8;
  if (n8 == 0) return hipSuccess;
  if (d % 8) return hipErrorInvalidValue;
  if (out)
    hipLaunchKernelGGL(fold_second_kernel<true>, dim3(blocks_for(n8)), dim3(256), 0, s, o, lse, o2, lse2,
                       (__bf16*)out, L, h, d / 8, n8);
  else
    hipLaunchKernelGGL(fold_second_kernel<false>, dim3(blocks_for(n8)), dim3(256), 0, s, o, lse, o2, lse2,
                       (__bf16*)nullptr, L, h, d / 8, n8);
  return hipGetLastError();
}

hipError_t launch_stage_kv(char* kdst, char* vdst, const void* k_all, const void* v_all, int64_t shard_bytes,
                           int64_t stride, int N, int qs, int k0, int n_steps, hipStream_t s) {
  if (n_steps <= 0 || shard_bytes <= 0) return hipSuccess;
  if (shard_bytes % 16 || n_steps > 65535) return hipErrorInvalidValue;
  // 64 workgroups per shard and tensor: the copy runs beside step kernels that fill every
  // compute unit, and wider grids slowed them (measured on MI355X)
  const int64_t blocks = std::min<int64_t>((shard_bytes / 16 + 255) / 256, 64);
  hipLaunchKernelGGL(stage_kv_kernel, dim3((unsigned)blocks, (unsigned)n_steps, 2), dim3(256), 0, s, kdst, vdst,
                     (const char*)k_all, (const char*)v_all, shard_bytes, stride, N, qs, k0);
  return hipGetLastError();
}

hipError_t launch_fill_lse(float* lse, int64_t n, float value, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(blocks_for(n)), dim3(256), 0, s, lse, n, value);
  return hipGetLastError();
}

}  // namespace ra

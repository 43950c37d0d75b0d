// The two head-group exchanges of all-to-all sequence parallelism (page 3, sections 4.2 and
// 7): before attention each device trades "its slice of the sequence, every head" for "the
// whole sequence, its share of the heads"; after attention the outputs go back the same
// way.  On one GPU the N devices' shards are resident buffers and one device's side of each
// exchange is a copy kernel: the gather builds the whole sequence of the device's heads in
// global position order (so the attention that follows masks by position alone), the
// scatter writes the device's heads of every shard's output and LSE.  The backward uses
// the same exchanges for O, dO and the LSE on the way in and the gradients on the way
// out.  All are plain HBM-bound copies, 16 bytes per thread on the wide side.
#include "ra_internal.h"

namespace ra {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// One thread per 16-byte chunk of a destination row; blockIdx.y = batch row.
__global__ __launch_bounds__(256) void ulysses_gather_kernel(char* __restrict__ dst, const char* __restrict__ src,
                                                             int b, int L, int N, int layout, int H, int Hg,
                                                             int head0, int chunks_per_head) {
  const int bi = blockIdx.y;
  const int64_t S = (int64_t)N * L;
  const int W = Hg * chunks_per_head;                 // chunks per position
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= S * W) return;
  const int64_t P = idx / W;
  const int w = (int)(idx - P * W);
  const int hh = w / chunks_per_head, c = w - hh * chunks_per_head;
  int j, t;
  owner_of(layout, N, L, P, j, t);
  const int64_t head_bytes = (int64_t)chunks_per_head * 16;
  const char* s = src + ((((int64_t)j * b + bi) * L + t) * H + head0 + hh) * head_bytes + (int64_t)c * 16;
  char* d = dst + (((int64_t)bi * S + P) * Hg + hh) * head_bytes + (int64_t)c * 16;
  *(u32x4*)d = *(const u32x4*)s;
}

// Output rows: one thread per 8 (bf16) or 4 (fp32) elements of a destination row.
template <int DTYPE>
__global__ __launch_bounds__(256) void ulysses_scatter_o_kernel(void* __restrict__ dst, const float* __restrict__ src,
                                                                int b, int L, int N, int layout, int H, int Hg,
                                                                int head0, int d) {
  constexpr int E = DTYPE == RA_BF16 ? 8 : 4;
  const int bi = blockIdx.y;
  const int64_t S = (int64_t)N * L;
  const int per_head = d / E;
  const int W = Hg * per_head;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= S * W) return;
  const int64_t P = idx / W;
  const int w = (int)(idx - P * W);
  const int hh = w / per_head, c = w - hh * per_head;
  int j, t;
  owner_of(layout, N, L, P, j, t);
  const float* s = src + (((int64_t)bi * S + P) * Hg + hh) * d + (int64_t)c * E;
  const int64_t o = ((((int64_t)j * b + bi) * L + t) * H + head0 + hh) * d + (int64_t)c * E;
  if constexpr (DTYPE == RA_BF16) {
    const f32x4 lo = *(const f32x4*)s, hi = *(const f32x4*)(s + 4);
    bf16x8 v;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      v[x] = (__bf16)lo[x];        // round to nearest even
      v[x + 4] = (__bf16)hi[x];
    }
    *(bf16x8*)((__bf16*)dst + o) = v;
  } else {
    *(f32x4*)((float*)dst + o) = *(const f32x4*)s;
  }
}

// LSE: one thread per (head, position); reads run along the sequence.
__global__ __launch_bounds__(256) void ulysses_scatter_lse_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                                  int b, int L, int N, int layout, int H, int Hg,
                                                                  int head0) {
  const int bi = blockIdx.y;
  const int64_t S = (int64_t)N * L;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= S * Hg) return;
  const int hh = (int)(idx / S);
  const int64_t P = idx - (int64_t)hh * S;
  int j, t;
  owner_of(layout, N, L, P, j, t);
  dst[(((int64_t)j * b + bi) * H + head0 + hh) * L + t] = src[((int64_t)bi * Hg + hh) * S + P];
}

// Per-row statistics the other way: src [N][b][H][L] (fp32) -> dst [b][Hg][S].
__global__ __launch_bounds__(256) void ulysses_gather_rows_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                                  int b, int L, int N, int layout, int H, int Hg,
                                                                  int head0) {
  const int bi = blockIdx.y;
  const int64_t S = (int64_t)N * L;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= S * Hg) return;
  const int hh = (int)(idx / S);
  const int64_t P = idx - (int64_t)hh * S;
  int j, t;
  owner_of(layout, N, L, P, j, t);
  dst[((int64_t)bi * Hg + hh) * S + P] = src[(((int64_t)j * b + bi) * H + head0 + hh) * L + t];
}

dim3 grid_for(int64_t threads, int b) { return dim3((unsigned)((threads + 255) / 256), (unsigned)b); }

}  // namespace

hipError_t launch_ulysses_gather(void* dst, const void* src_all, int b, int L, int N, int layout,
                                 int H, int Hg, int head0, int d, int es, hipStream_t s) {
  const int chunks = d * es / 16;
  const int64_t threads = (int64_t)N * L * Hg * chunks;
  if ((threads + 255) / 256 > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(ulysses_gather_kernel, grid_for(threads, b), dim3(256), 0, s, (char*)dst,
                     (const char*)src_all, b, L, N, layout, H, Hg, head0, chunks);
  return hipGetLastError();
}

hipError_t launch_ulysses_gather_rows(float* dst, const float* src_all, int b, int L, int N, int layout, int H,
                                      int Hg, int head0, hipStream_t s) {
  const int64_t threads = (int64_t)N * L * Hg;
  if ((threads + 255) / 256 > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(ulysses_gather_rows_kernel, grid_for(threads, b), dim3(256), 0, s, dst, src_all, b, L, N,
                     layout, H, Hg, head0);
  return hipGetLastError();
}

hipError_t launch_ulysses_scatter_rows(void* dst_all, const float* src, int b, int L, int N, int layout, int H,
                                       int Hg, int head0, int d, int dtype, hipStream_t s) {
  const int E = dtype == RA_BF16 ? 8 : 4;
  const int64_t threads = (int64_t)N * L * Hg * (d / E);
  if ((threads + 255) / 256 > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (dtype == RA_BF16)
    hipLaunchKernelGGL(ulysses_scatter_o_kernel<RA_BF16>, grid_for(threads, b), dim3(256), 0, s, dst_all, src, b, L,
                       N, layout, H, Hg, head0, d);
  else
    hipLaunchKernelGGL(ulysses_scatter_o_kernel<RA_F32>, grid_for(threads, b), dim3(256), 0, s, dst_all, src, b, L,
                       N, layout, H, Hg, head0, d);
  return hipGetLastError();
}

hipError_t launch_ulysses_scatter(void* dst_all, float* lse_all, const float* o, const float* lse,
                                  int b, int L, int N, int layout, int H, int Hg, int head0, int d,
                                  int dtype, hipStream_t s) {
  const int64_t lse_threads = (int64_t)N * L * Hg;
  hipError_t e = launch_ulysses_scatter_rows(dst_all, o, b, L, N, layout, H, Hg, head0, d, dtype, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ulysses_scatter_lse_kernel, grid_for(lse_threads, b), dim3(256), 0, s, lse_all, lse, b, L, N,
                     layout, H, Hg, head0);
  return hipGetLastError();
}

}  // namespace ra

// One ring step of the forward pass in fp32 (head dim 64 or 128), on the vector ALUs.
//
// Same step as the bf16 kernel (page 1, "Blockwise Attention and Online Softmax
// Formulations"), kept plain for full fp32 accuracy: one thread owns one query row, the
// workgroup's 64 rows share K/V tiles of 32 keys staged in LDS (every lane reads the same
// key, an LDS broadcast), and the running maximum is refreshed exactly on every tile.
// Causal and packed-document masking use the same per-row key range as the bf16 kernel.
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int ROWS = 64;   // query rows (threads) per workgroup
constexpr int KT = 32;     // keys per tile

template <int D, int MODE>
__global__ __launch_bounds__(ROWS) void step_fwd_f32_kernel(StepArgs a, int n_qb) {
  __shared__ float k_lds[KT][D];
  __shared__ float v_lds[KT][D];
  const int L = a.L;
  const int G = a.h / a.n_kv;
  const int qb = n_qb - 1 - (int)(blockIdx.x % n_qb);
  const int hq = (blockIdx.x / n_qb) % a.h;
  const int bi = blockIdx.x / (n_qb * a.h);
  const int g = hq / G;
  const int t = qb * ROWS + threadIdx.x;
  const int t_last = min(qb * ROWS + ROWS - 1, L - 1);
  // allowed keys of a row: [lo, hi), nondecreasing in the row (see key_range)
  const bool packed = a.doc_begin != nullptr;
  auto range = [&](int row) {
    int64_t db = 0, de = 0;
    if (packed) {
      db = a.doc_begin[(int64_t)bi * L + row];
      de = a.doc_end[(int64_t)bi * L + row];
    }
    return key_range(a.causal, a.layout, a.N, L, a.q_shard, a.kv_shard, row, packed, db, de);
  };
  const int j_begin = range(qb * ROWS).lo / KT;
  const int n_tiles = (range(t_last).hi + KT - 1) / KT;
  const KeyRange rr = t < L ? range(t) : KeyRange{0, 0};
  const int lim = rr.hi, lo = rr.lo;

  const float* qp = (const float*)a.q + (((int64_t)bi * L + min(t, L - 1)) * a.h + hq) * D;
  const float* kp = (const float*)a.k + ((int64_t)bi * L * a.n_kv + g) * D;
  const float* vp = (const float*)a.v + ((int64_t)bi * L * a.n_kv + g) * D;
  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = t < L ? qp[e] * a.scale : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int j = j_begin; j < n_tiles; ++j) {
    const int kv0 = j * KT;
    __syncthreads();
    for (int idx = threadIdx.x; idx < KT * D; idx += ROWS) {
      const int r = idx / D, e = idx % D, u = kv0 + r;
      k_lds[r][e] = u < L ? kp[(int64_t)u * a.n_kv * D + e] : 0.f;
      v_lds[r][e] = u < L ? vp[(int64_t)u * a.n_kv * D + e] : 0.f;
    }
    __syncthreads();
    float s[KT];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < KT; ++r) {
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) x = fmaf(q[e], k_lds[r][e], x);
      s[r] = (kv0 + r < lim && kv0 + r >= lo) ? x : -INFINITY;
      mt = fmaxf(mt, s[r]);
    }
    const float m_new = fmaxf(m, mt);
    if (m_new == -INFINITY) continue;                 // nothing allowed yet for this row
    const float alpha = expf(m - m_new);              // 0 when m was -inf
    l *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] *= alpha;
    m = m_new;
#pragma unroll
    for (int r = 0; r < KT; ++r) {
      const float p = expf(s[r] - m);
      l += p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = fmaf(p, v_lds[r][e], o[e]);
    }
  }
  if (t >= L) return;
  const bool any = l > 0.f;
  const float lse_new = any ? m + logf(l) : -INFINITY;
  const float inv = any ? 1.f / l : 0.f;
  float* orow = a.o + (((int64_t)bi * L + t) * a.h + hq) * D;
  float* lse_p = a.lse + ((int64_t)bi * a.h + hq) * L + t;
  if (MODE == MODE_PART) {
#pragma unroll
    for (int e = 0; e < D; ++e) orow[e] = o[e] * inv;
    *lse_p = lse_new;
  } else {
    if (!any) return;
    const float lse_old = *lse_p;
    const float M = fmaxf(lse_old, lse_new);
    const float wa = expf(lse_old - M), wb = expf(lse_new - M);
    const float tot = wa + wb;
    const float fa = wa / tot, fb = wb * inv / tot;
#pragma unroll
    for (int e = 0; e < D; ++e) orow[e] = fa * orow[e] + fb * o[e];
    *lse_p = M + logf(tot);
  }
}

template <int D>
hipError_t launch_d(const StepArgs& a, int mode, hipStream_t stream) {
  const int n_qb = (a.L + ROWS - 1) / ROWS;
  const int64_t grid = (int64_t)n_qb * a.h * a.b;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (mode == MODE_PART)
    hipLaunchKernelGGL((step_fwd_f32_kernel<D, MODE_PART>), dim3((unsigned)grid), dim3(ROWS), 0,
                       stream, a, n_qb);
  else
    hipLaunchKernelGGL((step_fwd_f32_kernel<D, MODE_MERGE>), dim3((unsigned)grid), dim3(ROWS), 0,
                       stream, a, n_qb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_f32(const StepArgs& a, int mode, hipStream_t stream) {
  if (a.d == 64) return launch_d<64>(a, mode, stream);
  if (a.d == 128) return launch_d<128>(a, mode, stream);
  return hipErrorInvalidValue;
}

}  // namespace ra

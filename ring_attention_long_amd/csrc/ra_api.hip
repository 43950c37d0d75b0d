// C-ABI of libra (declared in include/ra.h): argument validation, kernel launches and the
// ring driver.
//
// The ring driver (page 1, "The Ring Attention Protocol and Overlapped Communication";
// page 4, "The Ring Communication Protocol"): at step k device i attends its resident
// queries to the KV shard of device (i - k) mod N and folds the partial into its running
// (O, LSE).  On one GPU the other devices' shards are resident buffers and the receive
// from the upstream neighbour is a device-to-device copy on a second stream into the idle
// half of a double buffer (page 1, "Practical Implementation Patterns": a current and an
// incoming KV buffer), overlapped with the current step's kernel.  Events order the two
// streams: the copy that fills a buffer waits for the step that last read it, and a step
// waits for the copy that filled its buffer.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "ra_internal.h"

namespace {

thread_local std::string g_last_error;

ra_status fail(ra_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ra_status fail(ra_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

ra_status hip_fail(hipError_t e, const char* what) {
  return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

float effective_scale(const ra_problem* p) {
  return p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->d);
}

constexpr int kMaxRing = 128;   // largest N the ring driver accepts

// Shape and enum checks that do not depend on which kernels exist.
ra_status check_shape(const ra_problem* p) {
  if (!p) return fail(RA_ERR_INVALID_ARG, "problem is NULL");
  if (p->b < 1 || p->L < 1 || p->h < 1 || p->n_kv < 1 || p->d < 1 || p->N < 1)
    return fail(RA_ERR_INVALID_ARG, "sizes must be >= 1 (b=%d L=%d h=%d n_kv=%d d=%d N=%d)", p->b,
                p->L, p->h, p->n_kv, p->d, p->N);
  if (p->h % p->n_kv) return fail(RA_ERR_INVALID_ARG, "h=%d is not a multiple of n_kv=%d", p->h, p->n_kv);
  if (p->causal != 0 && p->causal != 1) return fail(RA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->layout < RA_LAYOUT_CONTIGUOUS || p->layout > RA_LAYOUT_ZIGZAG)
    return fail(RA_ERR_INVALID_ARG, "unknown layout %d", p->layout);
  if (p->dtype != RA_F32 && p->dtype != RA_BF16) return fail(RA_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (p->layout == RA_LAYOUT_ZIGZAG && (p->L % 2))
    return fail(RA_ERR_INVALID_ARG, "zigzag layout needs an even L (got %d)", p->L);
  if (isnan(p->scale) || isinf(p->scale)) return fail(RA_ERR_INVALID_ARG, "scale is not finite");
  if (p->steps_per_launch < 0)
    return fail(RA_ERR_INVALID_ARG, "steps_per_launch must be >= 0 (got %d)", p->steps_per_launch);
  const int64_t seq = (int64_t)p->N * p->L;
  const int64_t q_elems = (int64_t)p->b * p->L * p->h * p->d;
  if (seq > (int64_t)1 << 31 || q_elems > (int64_t)1 << 40)
    return fail(RA_ERR_INVALID_ARG, "problem too large (S=%lld)", (long long)seq);
  return RA_OK;
}

ra_status check_problem(const ra_problem* p) {
  const ra_status s = check_shape(p);
  if (s != RA_OK) return s;
  if ((p->doc_begin == nullptr) != (p->doc_end == nullptr))
    return fail(RA_ERR_INVALID_ARG, "doc_begin and doc_end must both be set or both be NULL");
  if (p->doc_begin && (!aligned(p->doc_begin, 4) || !aligned(p->doc_end, 4)))
    return fail(RA_ERR_INVALID_ARG, "doc_begin / doc_end are not 4-byte aligned");
  if (p->dtype == RA_BF16 && p->d != 128)
    return fail(RA_ERR_UNSUPPORTED, "bf16 kernels support d = 128 only (got %d)", p->d);
  // the bf16 kernels stage K/V rows by DMA through a buffer range of 32-bit byte offsets
  // that must stay below 2^31 (larger offsets mark loads past the shard end)
  if (p->dtype == RA_BF16 && (int64_t)p->L * p->n_kv * p->d * 2 >= ((int64_t)1 << 31))
    return fail(RA_ERR_UNSUPPORTED, "one (batch, KV head) slice of K or V (L*n_kv*d*2 = %lld bytes) must stay below 2 GiB",
                (long long)p->L * p->n_kv * p->d * 2);
  if (p->dtype == RA_F32 && p->d != 64 && p->d != 128)
    return fail(RA_ERR_UNSUPPORTED, "fp32 kernels support d = 64 or 128 (got %d)", p->d);
  return RA_OK;
}

ra_status check_shard(const ra_problem* p, int32_t s, const char* name) {
  if (s < 0 || s >= p->N) return fail(RA_ERR_INVALID_ARG, "%s=%d outside [0, N=%d)", name, s, p->N);
  return RA_OK;
}

ra_status check_ptr(const void* ptr, const char* name, size_t align) {
  if (!ptr) return fail(RA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(ptr, align)) return fail(RA_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return RA_OK;
}

#define RA_TRY(x)                   \
  do {                              \
    const ra_status _s = (x);       \
    if (_s != RA_OK) return _s;     \
  } while (0)

size_t elem_size(const ra_problem* p) { return p->dtype == RA_BF16 ? 2 : 4; }

ra::StepArgs step_args(const ra_problem* p, int32_t qs, int32_t ks, const void* q, const void* k,
                       const void* v, float* o, float* lse) {
  ra::StepArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.b = p->b;
  a.L = p->L;
  a.h = p->h;
  a.n_kv = p->n_kv;
  a.d = p->d;
  a.N = p->N;
  a.causal = p->causal;
  a.layout = p->layout;
  a.q_shard = qs;
  a.kv_shard = ks;
  a.scale = effective_scale(p);
  a.doc_begin = p->doc_begin;
  a.doc_end = p->doc_end;
  return a;
}

hipError_t launch_step(const ra_problem* p, const ra::StepArgs& a, int mode, hipStream_t s) {
  return p->dtype == RA_BF16 ? ra::launch_step_bf16(a, mode, s) : ra::launch_step_f32(a, mode, s);
}

bool step_is_live(const ra_problem* p, int32_t qs, int32_t ks) {
  return ra::kv_limit(p->causal, p->layout, p->N, p->L, qs, ks, p->L - 1) > 0;
}

// Debugging aid: with RA_POISON_STAGING=1 in the environment, each KV staging buffer is
// filled with NaN on the copy stream as soon as the step that read it has finished, so a
// step that read a buffer outside its staged..consumed window would produce NaN.  Off by
// default; read on every call.
bool poison_staging() {
  const char* v = getenv("RA_POISON_STAGING");
  return v && v[0] == '1';
}

// After step k consumed `bytes` at buf (both multiples of 4): make the copy stream wait for the
// step, then fill the buffer with all-ones bit patterns (NaN in fp32 and in bf16).
hipError_t poison_after(void* buf, size_t bytes, hipEvent_t consumed, hipStream_t ps, bool split) {
  hipError_t e;
  if (split && (e = hipStreamWaitEvent(ps, consumed, 0)) != hipSuccess) return e;
  uint32_t bits = 0xFFFFFFFFu;
  float nan_all_ones;
  memcpy(&nan_all_ones, &bits, 4);
  return ra::launch_fill_lse((float*)buf, (int64_t)(bytes / 4), nan_all_ones, ps);
}

// Event set of one ring pass; destroyed on every exit path.
struct Events {
  // a pass makes at most entry, done, staged and consumed per step, four timing events per
  // step (timed passes have N <= RA_MAX_TIMED_STEPS); a full set is an error, not an overrun
  static constexpr int kCap = 2 + 2 * kMaxRing + 4 * RA_MAX_TIMED_STEPS;
  hipEvent_t e[kCap] = {};
  int n = 0;
  ~Events() {
    for (int i = 0; i < n; ++i)
      if (e[i]) (void)hipEventDestroy(e[i]);
  }
  hipError_t make(hipEvent_t* out, bool timing) {
    if (n >= kCap) return hipErrorOutOfMemory;
    hipEvent_t ev = nullptr;
    const hipError_t r = hipEventCreateWithFlags(&ev, timing ? hipEventDefault : hipEventDisableTiming);
    if (r == hipSuccess) {
      e[n++] = ev;
      *out = ev;
    }
    return r;
  }
};

// The KV staging double buffer of a forward or backward ring pass: K and V of two shards.
size_t staging_bytes(const ra_problem* p) {
  return 4 * align_up((size_t)p->b * p->L * p->n_kv * p->d * elem_size(p), 256);
}

// A forward pass keeps a second accumulator (bf16 path, short shards, no packed documents),
// so that its steps may split the key ranges of their heaviest query blocks over two
// workgroups (see plan_split).  Its bytes: fp32 [b][L][h][d] and LSE [b][h][L].
bool fwd_split(const ra_problem* p) {
  return p->dtype == RA_BF16 && !p->doc_begin && p->L <= ra::kSplitMaxL;
}
size_t second_o_bytes(const ra_problem* p) { return align_up((size_t)p->b * p->L * p->h * p->d * 4, 256); }
size_t second_lse_bytes(const ra_problem* p) { return align_up((size_t)p->b * p->h * p->L * 4, 256); }
size_t second_acc_bytes(const ra_problem* p) {
  return fwd_split(p) ? second_o_bytes(p) + second_lse_bytes(p) : 0;
}
// ra_ring_fwd's workspace without the second accumulator: the KV double buffer and (not for
// fp32) the fp32 accumulator.
size_t ring_fwd_base_workspace(const ra_problem* p) {
  const size_t shard_bytes = (size_t)p->b * p->L * p->n_kv * p->d * elem_size(p);
  size_t n = 4 * align_up(shard_bytes, 256);
  if (p->dtype != RA_F32) n += align_up((size_t)p->b * p->L * p->h * p->d * 4, 256);
  return n;
}

// Ring steps per launch of a forward pass (ra_problem.steps_per_launch; bf16 only): with
// m >= 2 the steps after the first run m at a time, each workgroup walking those KV shards
// in ring order with its softmax state in registers and merging once, instead of paying its
// Q load, the fp32 accumulator's read-modify-write and a launch for every step; the staging
// then gives every remote shard a slot of its own instead of the double buffer.
// The library's choice (0), from measurement on MI355X (h = 32, n_kv = 8, N = 8, L = 1024 ..
// 32768): all N - 1 remote steps in one launch while a step is short (b h L^2 <= 2^33, i.e.
// L <= 16384 at b = 1, h = 32) or with packed documents, else at most kDefaultStepsPerLaunch.
// Short steps: one launch and one wait instead of two took 7 % less time at L = 1024, 4-6 %
// at 2048 and up to 2 % at 4096-16384 (every layout).  Long steps
// (L = 32768) measured alike with 4 and 7 per launch (within 0.3 %), and with a causal mask
// the query blocks of a launch do unequal work per shard, so the workgroups sharing an XCD's
// L2 drift apart over the shards and stop sharing K/V tiles: seven steps per launch fetched
// 3x the bytes of four there (33 against 11 GB per pass); four keep the traffic down.
// Packed documents bound each block's keys per shard, and there all remote steps in one
// launch took 4 % less time than four at L = 32768.
constexpr int kDefaultStepsPerLaunch = 4;
int fwd_steps_per_launch(const ra_problem* p) {
  if (p->dtype != RA_BF16 || p->N < 3) return 1;
  int m = p->steps_per_launch;
  if (m == 0) {
    const double work = (double)p->b * p->h * (double)p->L * p->L;
    m = (p->doc_begin || work <= 8589934592.0) ? p->N - 1 : kDefaultStepsPerLaunch;
  }
  return m < p->N - 1 ? m : p->N - 1;
}
size_t batch_workspace(const ra_problem* p) {
  const size_t A = align_up((size_t)p->b * p->L * p->n_kv * p->d * elem_size(p), 256);
  return 2 * (size_t)(p->N - 1) * A + align_up((size_t)p->b * p->L * p->h * p->d * 4, 256);
}

// Events of one forward pass made ahead of time (the allocation-free entry point keeps one
// set per device); without one, ring_fwd_impl creates its own for the call.
struct RingEvents {
  hipEvent_t entry = nullptr;
  hipEvent_t staged[kMaxRing] = {};
  hipEvent_t consumed[kMaxRing] = {};
};

// The ring's K/V receive for ring steps k0 .. k0 + n - 1 of device qs on stream ps: K and V of
// shard (qs - k) mod N into kdst, vdst + (k - k0) stride.  Small shards in one launch of the
// staging kernel (16-byte accesses: sizes and addresses aligned to 16); from
// kStageKernelMaxBytes of K and V per shard, or unaligned, two runtime copies per shard.  Below
// the threshold the runtime copies' fixed cost left the first launches of short shards waiting
// for their data (L = 1024 passes 12-20 % faster with the kernel); above it the two measured
// alike.
constexpr size_t kStageKernelMaxBytes = (size_t)16 << 20;
hipError_t stage_kv(char* kdst, char* vdst, const void* k_all, const void* v_all, size_t shard_bytes, size_t stride,
                    int N, int qs, int k0, int n, hipStream_t ps) {
  const uintptr_t align = (uintptr_t)kdst | (uintptr_t)vdst | (uintptr_t)k_all | (uintptr_t)v_all |
                          (uintptr_t)shard_bytes | (uintptr_t)stride;
  if (2 * shard_bytes < kStageKernelMaxBytes && align % 16 == 0)
    return ra::launch_stage_kv(kdst, vdst, k_all, v_all, (int64_t)shard_bytes, (int64_t)stride, N, qs, k0, n, ps);
  hipError_t e;
  for (int i = 0; i < n; ++i) {
    const int src = ((qs - (k0 + i)) % N + N) % N;
    if ((e = hipMemcpyAsync(kdst + (size_t)i * stride, (const char*)k_all + (size_t)src * shard_bytes, shard_bytes,
                            hipMemcpyDeviceToDevice, ps)) != hipSuccess ||
        (e = hipMemcpyAsync(vdst + (size_t)i * stride, (const char*)v_all + (size_t)src * shard_bytes, shard_bytes,
                            hipMemcpyDeviceToDevice, ps)) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

// The forward pass in batched launches (see fwd_steps_per_launch): step 0 on the local shard
// while the copy stream stages the N - 1 remote shards in ring order, each into its own slot;
// then the remaining steps, m at a time, each launch after the copies of its shards.  The
// last launch with a live step writes the bf16 output.  Arguments as ring_fwd_impl's, checked;
// tm: per-launch and per-copy timings (N <= RA_MAX_TIMED_STEPS), or null.
// With (o2, lse2), the second accumulator (short shards whose launches leave compute units
// idle): step 0 and the batched launches may split the key ranges of their query blocks over
// two workgroups, the second merging into (o2, lse2), and the pass ends by folding it into
// the output instead of the last launch writing it.
ra_status ring_fwd_batched(const ra_problem* p, int32_t qs, const void* q, const void* k_all,
                           const void* v_all, void* o, float* lse, void* ws, hipStream_t cs, hipStream_t ps,
                           const RingEvents* pre, int m, ra_ring_timing* tm, float* o2, float* lse2) {
  const int N = p->N;
  const size_t shard_bytes = (size_t)p->b * p->L * p->n_kv * p->d * elem_size(p);
  const size_t A = align_up(shard_bytes, 256);
  char* wsc = (char*)ws;
  char* kslot = wsc;                              // slot k - 1 holds the K of ring step k
  char* vslot = wsc + (size_t)(N - 1) * A;
  float* o_acc = (float*)(wsc + 2 * (size_t)(N - 1) * A);
  const bool split = ps != cs;
  const bool poison = poison_staging();
  const bool timing = tm != nullptr;
  Events ev;
  hipEvent_t entry, staged[kMaxRing], consumed[kMaxRing];
  hipEvent_t t_sb[RA_MAX_TIMED_STEPS], t_se[RA_MAX_TIMED_STEPS], t_cb[RA_MAX_TIMED_STEPS],
      t_ce[RA_MAX_TIMED_STEPS];
  hipError_t e;
  if (pre) {
    entry = pre->entry;
    for (int k = 0; k < N; ++k) {
      staged[k] = pre->staged[k];
      consumed[k] = pre->consumed[k];
    }
  } else {
    if ((e = ev.make(&entry, timing)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    for (int k = 0; k < N; ++k) {
      if ((e = ev.make(&staged[k], false)) != hipSuccess) return hip_fail(e, "hipEventCreate");
      if ((e = ev.make(&consumed[k], false)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
  }
  if (timing) {
    tm->n_steps = N;
    for (int k = 0; k < N; ++k) {
      tm->step_begin_ms[k] = tm->step_end_ms[k] = tm->copy_begin_ms[k] = tm->copy_end_ms[k] = -1.f;
      tm->launch_steps[k] = 0;
      if ((e = ev.make(&t_sb[k], true)) != hipSuccess || (e = ev.make(&t_se[k], true)) != hipSuccess ||
          (e = ev.make(&t_cb[k], true)) != hipSuccess || (e = ev.make(&t_ce[k], true)) != hipSuccess)
        return hip_fail(e, "hipEventCreate");
    }
  }
  // launches: [0], then [k0, k1) groups of live steps; the last live group writes o
  int g_first[kMaxRing], g_end[kMaxRing], n_groups = 0;
  g_first[0] = 0;
  g_end[0] = 1;
  n_groups = 1;
  for (int k = 1; k < N; k += m) {
    const int k1 = k + m < N ? k + m : N;
    bool live = false;
    for (int j = k; j < k1; ++j) live = live || step_is_live(p, qs, ((qs - j) % N + N) % N);
    if (!live) continue;
    g_first[n_groups] = k;
    g_end[n_groups] = k1;
    ++n_groups;
  }
  // The copy stream must not read k_all / v_all before work the caller queued on `compute`.
  if ((e = hipEventRecord(entry, cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (split && (e = hipStreamWaitEvent(ps, entry, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  const char* kc = (const char*)k_all;
  const char* vc = (const char*)v_all;
  // the copies of every remote shard, in ring order, queued right after step 0's launch (which
  // reads the local shard in place) so that the compute stream does not wait for the host
  // (per group of m steps, dead groups included: the ring still passes their shards on; small
  // shards in one staging launch per group, large ones shard by shard with an event after
  // each, which measured 1-2 % faster at L = 4096 and 8192 than one event per group)
  const int stage_n = 2 * shard_bytes < kStageKernelMaxBytes ? m : 1;
  auto stage_all = [&]() -> ra_status {
    for (int k = 1; k < N; k += m) {
      const int k1 = k + m < N ? k + m : N;
      if (timing && (e = hipEventRecord(t_cb[k], ps)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      for (int j = k; j < k1; j += stage_n) {
        const int n = k1 - j < stage_n ? k1 - j : stage_n;
        if ((e = stage_kv(kslot + (size_t)(j - 1) * A, vslot + (size_t)(j - 1) * A, k_all, v_all, shard_bytes, A,
                          N, qs, j, n, ps)) != hipSuccess)
          return hip_fail(e, "staging copy");
        if ((e = hipEventRecord(staged[j + n - 1], ps)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      }
      if (timing && (e = hipEventRecord(t_ce[k], ps)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    return RA_OK;
  };
  for (int gi = 0; gi < n_groups; ++gi) {
    const int k0 = g_first[gi], k1 = g_end[gi];
    const bool last = gi == n_groups - 1;
    ra::StepArgs a;
    if (k0 > 0 && split && (e = hipStreamWaitEvent(cs, staged[k1 - 1], 0)) != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent");   // copies run in ring order: the last covers the others
    if (timing && (e = hipEventRecord(t_sb[k0], cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if (k0 == 0) {
      a = step_args(p, qs, qs, q, kc + (size_t)qs * shard_bytes, vc + (size_t)qs * shard_bytes, o_acc, lse);
      a.o2 = o2;
      a.lse2 = lse2;
      if (last && !o2) a.o_out = (__bf16*)o;
      if ((e = ra::launch_step_bf16(a, ra::MODE_PART, cs)) != hipSuccess) return hip_fail(e, "step kernel launch");
    } else {
      a = step_args(p, qs, qs, q, nullptr, nullptr, o_acc, lse);
      a.o2 = o2;
      a.lse2 = lse2;
      if (last && !o2) a.o_out = (__bf16*)o;
      ra::ShardBatch sb;
      sb.k = kslot + (size_t)(k0 - 1) * A;
      sb.v = vslot + (size_t)(k0 - 1) * A;
      sb.stride = (int64_t)A;
      sb.k_first = k0;
      sb.n = k1 - k0;
      if ((e = ra::launch_steps_bf16(a, sb, ra::MODE_MERGE, cs)) != hipSuccess)
        return hip_fail(e, "step kernel launch");
      if (poison) {
        if ((e = hipEventRecord(consumed[k0], cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
        for (int k = k0; k < k1; ++k)
          if ((e = poison_after(kslot + (size_t)(k - 1) * A, shard_bytes, consumed[k0], ps, split)) != hipSuccess ||
              (e = poison_after(vslot + (size_t)(k - 1) * A, shard_bytes, consumed[k0], ps, split)) != hipSuccess)
            return hip_fail(e, "staging poison");
      }
    }
    if (timing) {
      if ((e = hipEventRecord(t_se[k0], cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      tm->launch_steps[k0] = k1 - k0;
    }
    if (k0 == 0) RA_TRY(stage_all());
  }
  if (o2 && (e = ra::launch_fold_second(o_acc, lse, o2, lse2, o, p->b, p->L, p->h, p->d, cs)) != hipSuccess)
    return hip_fail(e, "fold kernel launch");
  // Work the caller queues on `compute` after this call must not overtake the copy stream,
  // which still writes the workspace when the last live group ends before the last copy (or
  // when poisoning): join it back.
  if (split) {
    if ((e = hipEventRecord(consumed[0], ps)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(cs, consumed[0], 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  if (timing) {
    hipEvent_t done;
    if ((e = ev.make(&done, true)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    if ((e = hipEventRecord(done, cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipEventSynchronize(done)) != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    (void)hipEventElapsedTime(&tm->total_ms, entry, done);
    for (int k = 0; k < N; ++k) {
      if (tm->launch_steps[k] > 0) {
        (void)hipEventElapsedTime(&tm->step_begin_ms[k], entry, t_sb[k]);
        (void)hipEventElapsedTime(&tm->step_end_ms[k], entry, t_se[k]);
      }
      if (k >= 1) {   // the staging launch of the group holding step k
        const int g = 1 + (k - 1) / m * m;
        (void)hipEventElapsedTime(&tm->copy_begin_ms[k], entry, t_cb[g]);
        (void)hipEventElapsedTime(&tm->copy_end_ms[k], entry, t_ce[g]);
      }
    }
  }
  return RA_OK;
}

// Whether any launch of a batched pass (step 0, then live groups of m ring steps) would split a
// query block, given a second accumulator.
bool batched_splits(const ra_problem* p, int32_t qs, int m) {
  const int N = p->N;
  if (ra::step_splits_bf16(step_args(p, qs, qs, nullptr, nullptr, nullptr, nullptr, nullptr))) return true;
  for (int k = 1; k < N; k += m) {
    const int k1 = k + m < N ? k + m : N;
    bool live = false;
    for (int j = k; j < k1; ++j) live = live || step_is_live(p, qs, ((qs - j) % N + N) % N);
    if (!live) continue;
    ra::ShardBatch sb;
    sb.k_first = k;
    sb.n = k1 - k;
    if (ra::steps_split_bf16(step_args(p, qs, qs, nullptr, nullptr, nullptr, nullptr, nullptr), sb)) return true;
  }
  return false;
}

ra_status ring_fwd_impl(const ra_problem* p, int32_t qs, const void* q, const void* k_all,
                        const void* v_all, void* o, float* lse, void* ws, size_t ws_bytes,
                        ra_stream compute, ra_stream copy, ra_ring_timing* tm,
                        const RingEvents* pre = nullptr, float* o_acc_ext = nullptr, float* o2_ext = nullptr,
                        float* lse2_ext = nullptr) {
  // o_acc_ext: leave the merged fp32 result there (no cast to p->dtype, o unused) and use
  // the workspace for the staging buffers only; the second accumulator (when the problem
  // keeps one) is then (o2_ext, lse2_ext).
  RA_TRY(check_problem(p));
  // before either path: both keep per-step events in arrays of kMaxRing
  if (p->N > kMaxRing) return fail(RA_ERR_UNSUPPORTED, "ring size N=%d above %d", p->N, kMaxRing);
  RA_TRY(check_shard(p, qs, "q_shard"));
  RA_TRY(check_ptr(q, "q", 16));
  RA_TRY(check_ptr(k_all, "k_all", 16));
  RA_TRY(check_ptr(v_all, "v_all", 16));
  if (!o_acc_ext) RA_TRY(check_ptr(o, "o", 16));
  RA_TRY(check_ptr(lse, "lse", 4));
  RA_TRY(check_ptr(ws, "ws", 16));
  const size_t need = o_acc_ext ? staging_bytes(p) : ring_fwd_base_workspace(p);
  if (ws_bytes < need)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  const int m = o_acc_ext ? 1 : fwd_steps_per_launch(p);
  if (m >= 2) {
    if (tm && p->N > RA_MAX_TIMED_STEPS)
      return fail(RA_ERR_INVALID_ARG, "timed ring needs N <= %d", RA_MAX_TIMED_STEPS);
    if (ws_bytes >= batch_workspace(p)) {
      float* o2 = nullptr;
      float* lse2 = nullptr;
      if (fwd_split(p) && ws_bytes >= batch_workspace(p) + second_acc_bytes(p) && batched_splits(p, qs, m)) {
        o2 = (float*)((char*)ws + batch_workspace(p));
        lse2 = (float*)((char*)o2 + second_o_bytes(p));
      }
      return ring_fwd_batched(p, qs, q, k_all, v_all, o, lse, ws, (hipStream_t)compute,
                              copy ? (hipStream_t)copy : (hipStream_t)compute, pre, m, tm, o2, lse2);
    }
    if (p->steps_per_launch != 0)   // asked for explicitly: the workspace must hold the slots
      return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed for %d steps per launch", ws_bytes,
                  batch_workspace(p), m);
  }
  // the second accumulator: the caller's (o_acc_ext), or after the rest when the workspace
  // has room for it
  bool second = fwd_split(p) && (o_acc_ext ? (o2_ext && lse2_ext) : ws_bytes >= need + second_acc_bytes(p));
  if (second) {   // ... and only if some step splits a query block (else the plain finalize)
    bool any_split = false;
    for (int k = 0; k < p->N && !any_split; ++k) {
      const int src = ((qs - k) % p->N + p->N) % p->N;
      if (!step_is_live(p, qs, src)) continue;
      const ra::StepArgs a = step_args(p, qs, src, nullptr, nullptr, nullptr, nullptr, nullptr);
      any_split = ra::step_splits_bf16(a);
    }
    second = any_split;
  }
  const int N = p->N;
  if (tm && N > RA_MAX_TIMED_STEPS)
    return fail(RA_ERR_INVALID_ARG, "timed ring needs N <= %d", RA_MAX_TIMED_STEPS);

  const size_t shard_bytes = (size_t)p->b * p->L * p->n_kv * p->d * elem_size(p);
  const size_t A = align_up(shard_bytes, 256);
  char* wsc = (char*)ws;
  char* kbuf[2] = {wsc, wsc + 2 * A};
  char* vbuf[2] = {wsc + A, wsc + 3 * A};
  float* o_acc = o_acc_ext ? o_acc_ext : p->dtype == RA_F32 ? (float*)o : (float*)(wsc + 4 * A);
  float* lse_acc = lse;
  float* o2 = nullptr;
  float* lse2 = nullptr;
  if (second) {
    if (o_acc_ext) {
      o2 = o2_ext;
      lse2 = lse2_ext;
    } else {   // after the staging buffers and the (bf16 path) accumulator
      o2 = (float*)(wsc + 4 * A + align_up((size_t)p->b * p->L * p->h * p->d * 4, 256));
      lse2 = (float*)((char*)o2 + second_o_bytes(p));
    }
  }
  const hipStream_t cs = (hipStream_t)compute;
  const hipStream_t ps = copy ? (hipStream_t)copy : cs;
  const bool split = ps != cs;
  const bool timing = tm != nullptr;
  const bool poison = poison_staging();

  Events ev;
  hipEvent_t entry, staged[kMaxRing], consumed[kMaxRing];
  hipEvent_t t_sb[RA_MAX_TIMED_STEPS], t_se[RA_MAX_TIMED_STEPS], t_cb[RA_MAX_TIMED_STEPS],
      t_ce[RA_MAX_TIMED_STEPS];
  hipError_t e;
  if (pre) {
    entry = pre->entry;
    for (int k = 0; k < N; ++k) {
      staged[k] = pre->staged[k];
      consumed[k] = pre->consumed[k];
    }
  } else {
    if ((e = ev.make(&entry, timing)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    for (int k = 0; k < N; ++k) {
      if ((e = ev.make(&staged[k], false)) != hipSuccess) return hip_fail(e, "hipEventCreate");
      if ((e = ev.make(&consumed[k], false)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
  }
  if (timing) {
    tm->n_steps = N;
    for (int k = 0; k < N; ++k) {
      tm->step_begin_ms[k] = tm->step_end_ms[k] = tm->copy_begin_ms[k] = tm->copy_end_ms[k] = -1.f;
      tm->launch_steps[k] = 0;
      if ((e = ev.make(&t_sb[k], true)) != hipSuccess || (e = ev.make(&t_se[k], true)) != hipSuccess ||
          (e = ev.make(&t_cb[k], true)) != hipSuccess || (e = ev.make(&t_ce[k], true)) != hipSuccess)
        return hip_fail(e, "hipEventCreate");
    }
  }
  bool live[kMaxRing];
  // The last live step of a bf16 pass without the second accumulator writes the output
  // itself (merged rows cast to bf16), so no separate finalize pass reads the accumulator.
  int k_final = -1;
  if (!o_acc_ext && p->dtype == RA_BF16 && !second)
    for (int k = 0; k < N; ++k)
      if (step_is_live(p, qs, ((qs - k) % N + N) % N)) k_final = k;

  // The copy stream must not read k_all / v_all before work the caller queued on `compute`.
  if ((e = hipEventRecord(entry, cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (split && (e = hipStreamWaitEvent(ps, entry, 0)) != hipSuccess)
    return hip_fail(e, "hipStreamWaitEvent");

  bool have_acc = false;
  const char* kc = (const char*)k_all;
  const char* vc = (const char*)v_all;
  for (int k = 0; k < N; ++k) {
    // Stage the KV shard of step k+1 into buffer (k+1) % 2, last read by step k-1.
    if (k + 1 < N) {
      const int dst = (k + 1) & 1;
      if (split && k - 1 >= 1 && (e = hipStreamWaitEvent(ps, consumed[k - 1], 0)) != hipSuccess)
        return hip_fail(e, "hipStreamWaitEvent");
      if (timing && (e = hipEventRecord(t_cb[k + 1], ps)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      if ((e = stage_kv(kbuf[dst], vbuf[dst], k_all, v_all, shard_bytes, 0, N, qs, k + 1, 1, ps)) != hipSuccess)
        return hip_fail(e, "staging copy");
      if (timing && (e = hipEventRecord(t_ce[k + 1], ps)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      if ((e = hipEventRecord(staged[k + 1], ps)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    // Step k on the shard of device (qs - k) mod N.
    if (split && k >= 1 && (e = hipStreamWaitEvent(cs, staged[k], 0)) != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent");
    const int src = ((qs - k) % N + N) % N;
    const void* kp = k == 0 ? (const void*)(kc + (size_t)qs * shard_bytes) : (const void*)kbuf[k & 1];
    const void* vp = k == 0 ? (const void*)(vc + (size_t)qs * shard_bytes) : (const void*)vbuf[k & 1];
    live[k] = step_is_live(p, qs, src);
    if (live[k]) {
      if (timing && (e = hipEventRecord(t_sb[k], cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      ra::StepArgs a = step_args(p, qs, src, q, kp, vp, o_acc, lse_acc);
      a.o2 = o2;
      a.lse2 = lse2;
      if (k == k_final) a.o_out = (__bf16*)o;
      if ((e = launch_step(p, a, have_acc ? ra::MODE_MERGE : ra::MODE_PART, cs)) != hipSuccess)
        return hip_fail(e, "step kernel launch");
      have_acc = true;
      if (timing && (e = hipEventRecord(t_se[k], cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    if ((e = hipEventRecord(consumed[k], cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if (poison && k >= 1 &&
        ((e = poison_after(kbuf[k & 1], shard_bytes, consumed[k], ps, split)) != hipSuccess ||
         (e = poison_after(vbuf[k & 1], shard_bytes, consumed[k], ps, split)) != hipSuccess))
      return hip_fail(e, "staging poison");
  }
  const int64_t n_out = (int64_t)p->b * p->L * p->h * p->d;
  if (!have_acc) {
    // unreachable for valid problems (a shard always sees itself), kept for completeness
    if ((e = ra::launch_fill_lse(o_acc, n_out, 0.f, cs)) != hipSuccess) return hip_fail(e, "fill kernel launch");
    if ((e = ra::launch_fill_lse(lse_acc, (int64_t)p->b * p->h * p->L, -INFINITY, cs)) != hipSuccess)
      return hip_fail(e, "fill kernel launch");
  }
  if (second && have_acc) {
    // fold the second accumulator in: into the bf16 output, or in place for o_acc_ext
    if ((e = ra::launch_fold_second(o_acc, lse_acc, o2, lse2, o_acc_ext ? nullptr : o, p->b, p->L, p->h, p->d,
                                    cs)) != hipSuccess)
      return hip_fail(e, "fold kernel launch");
  } else if (!o_acc_ext && p->dtype != RA_F32 && k_final < 0 &&
             (e = ra::launch_finalize(o_acc, o, p->dtype, n_out, cs)) != hipSuccess) {
    return hip_fail(e, "finalize kernel launch");
  }

  if (timing) {
    hipEvent_t done;
    if ((e = ev.make(&done, true)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    if ((e = hipEventRecord(done, cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipEventSynchronize(done)) != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    (void)hipEventElapsedTime(&tm->total_ms, entry, done);
    for (int k = 0; k < N; ++k) {
      if (live[k]) {
        (void)hipEventElapsedTime(&tm->step_begin_ms[k], entry, t_sb[k]);
        (void)hipEventElapsedTime(&tm->step_end_ms[k], entry, t_se[k]);
        tm->launch_steps[k] = 1;
      }
      if (k >= 1) {
        (void)hipEventElapsedTime(&tm->copy_begin_ms[k], entry, t_cb[k]);
        (void)hipEventElapsedTime(&tm->copy_end_ms[k], entry, t_ce[k]);
      }
    }
  }
  return RA_OK;
}

// ---- all-to-all sequence parallelism (page 3, sections 4.2 and 7) -----------------------
// Device g of N holds, after the first exchange, the whole sequence (S = N L tokens) of
// query heads [g h/N, (g+1) h/N) and KV heads [g n_kv/N, (g+1) n_kv/N): the same query
// head to KV head map as the full problem, since h/N over n_kv/N is h / n_kv.  It runs one
// attention over the whole sequence in global position order, then sends each shard's rows
// of its heads back.
ra_status check_ulysses(const ra_problem* p) {
  RA_TRY(check_problem(p));
  if (p->doc_begin) return fail(RA_ERR_UNSUPPORTED, "packed documents are not supported by the all-to-all path");
  if (p->h % p->N || p->n_kv % p->N)
    return fail(RA_ERR_INVALID_ARG, "the all-to-all path splits heads over the N devices: h=%d and n_kv=%d must be "
                "multiples of N=%d", p->h, p->n_kv, p->N);
  if (p->b > 65535) return fail(RA_ERR_UNSUPPORTED, "batch %d above 65535", p->b);
  return RA_OK;
}

// The attention problem one device solves after the first exchange.
ra_problem ulysses_local(const ra_problem* p) {
  ra_problem q = *p;
  q.L = p->N * p->L;
  q.h = p->h / p->N;
  q.n_kv = p->n_kv / p->N;
  q.N = 1;
  q.layout = RA_LAYOUT_CONTIGUOUS;
  q.scale = effective_scale(p);
  q.doc_begin = q.doc_end = nullptr;
  return q;
}

struct UlyssesWs {
  size_t q, kv, o, lse, second, total;
};
UlyssesWs ulysses_ws(const ra_problem* p) {
  const size_t S = (size_t)p->N * p->L, es = elem_size(p);
  UlyssesWs w;
  w.q = align_up((size_t)p->b * S * (p->h / p->N) * p->d * es, 256);
  w.kv = align_up((size_t)p->b * S * (p->n_kv / p->N) * p->d * es, 256);
  w.o = align_up((size_t)p->b * S * (p->h / p->N) * p->d * 4, 256);
  w.lse = align_up((size_t)p->b * (p->h / p->N) * S * 4, 256);
  const ra_problem lp = ulysses_local(p);
  w.second = second_acc_bytes(&lp);
  w.total = w.q + 2 * w.kv + w.o + w.lse + w.second;
  return w;
}

ra_status ulysses_fwd_impl(const ra_problem* p, int32_t group, const void* q_all, const void* k_all,
                           const void* v_all, void* o_all, float* lse_all, void* ws, size_t ws_bytes,
                           ra_stream stream, ra_ulysses_timing* tm) {
  RA_TRY(check_ulysses(p));
  RA_TRY(check_shard(p, group, "head_group"));
  const ra_problem lp = ulysses_local(p);
  RA_TRY(check_problem(&lp));
  RA_TRY(check_ptr(q_all, "q_all", 16));
  RA_TRY(check_ptr(k_all, "k_all", 16));
  RA_TRY(check_ptr(v_all, "v_all", 16));
  RA_TRY(check_ptr(o_all, "o_all", 16));
  RA_TRY(check_ptr(lse_all, "lse_all", 4));
  RA_TRY(check_ptr(ws, "ws", 16));
  const UlyssesWs w = ulysses_ws(p);
  if (ws_bytes < w.total - w.second)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, w.total - w.second);
  // room for the second accumulator, and a query block that the step splits
  const bool second = w.second && ws_bytes >= w.total &&
                      ra::step_splits_bf16(step_args(&lp, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr));

  char* base = (char*)ws;
  void* q_g = base;
  void* k_g = base + w.q;
  void* v_g = base + w.q + w.kv;
  float* o_g = (float*)(base + w.q + 2 * w.kv);
  float* lse_g = (float*)(base + w.q + 2 * w.kv + w.o);
  const hipStream_t s = (hipStream_t)stream;
  const int Hg = p->h / p->N, Kg = p->n_kv / p->N, es = (int)elem_size(p);

  Events ev;
  hipEvent_t t0 = nullptr, t1 = nullptr, t2 = nullptr, t3 = nullptr;
  hipError_t e;
  if (tm) {
    if ((e = ev.make(&t0, true)) != hipSuccess || (e = ev.make(&t1, true)) != hipSuccess ||
        (e = ev.make(&t2, true)) != hipSuccess || (e = ev.make(&t3, true)) != hipSuccess)
      return hip_fail(e, "hipEventCreate");
    if ((e = hipEventRecord(t0, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  if ((e = ra::launch_ulysses_gather(q_g, q_all, p->b, p->L, p->N, p->layout, p->h, Hg, group * Hg, p->d, es, s)) !=
          hipSuccess ||
      (e = ra::launch_ulysses_gather(k_g, k_all, p->b, p->L, p->N, p->layout, p->n_kv, Kg, group * Kg, p->d, es, s)) !=
          hipSuccess ||
      (e = ra::launch_ulysses_gather(v_g, v_all, p->b, p->L, p->N, p->layout, p->n_kv, Kg, group * Kg, p->d, es, s)) !=
          hipSuccess)
    return hip_fail(e, "gather kernel launch");
  if (tm && (e = hipEventRecord(t1, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  ra::StepArgs a = step_args(&lp, 0, 0, q_g, k_g, v_g, o_g, lse_g);
  if (second) {
    a.o2 = (float*)(base + w.q + 2 * w.kv + w.o + w.lse);
    a.lse2 = (float*)((char*)a.o2 + second_o_bytes(&lp));
  }
  if ((e = launch_step(&lp, a, ra::MODE_PART, s)) != hipSuccess) return hip_fail(e, "step kernel launch");
  if (second && (e = ra::launch_fold_second(o_g, lse_g, a.o2, a.lse2, nullptr, lp.b, lp.L, lp.h, lp.d, s)) !=
                      hipSuccess)
    return hip_fail(e, "fold kernel launch");
  if (tm && (e = hipEventRecord(t2, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if ((e = ra::launch_ulysses_scatter(o_all, lse_all, o_g, lse_g, p->b, p->L, p->N, p->layout, p->h, Hg, group * Hg,
                                      p->d, p->dtype, s)) != hipSuccess)
    return hip_fail(e, "scatter kernel launch");
  if (tm) {
    if ((e = hipEventRecord(t3, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipEventSynchronize(t3)) != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    (void)hipEventElapsedTime(&tm->gather_ms, t0, t1);
    (void)hipEventElapsedTime(&tm->attend_ms, t1, t2);
    (void)hipEventElapsedTime(&tm->scatter_ms, t2, t3);
    (void)hipEventElapsedTime(&tm->total_ms, t0, t3);
  }
  return RA_OK;
}

// ---- two-dimensional arrangement: head groups x sequence ring (page 3, sections 7, 8) ----
// N = N_h * N_s devices.  The sequence is cut into N_s ring shards of N_h L tokens under
// p->layout; ring shard r is split into N_h consecutive pieces of L tokens and device
// r N_h + g holds piece g for every head.  Device (g, r) trades pieces with the other N_h - 1
// devices of ring shard r (first exchange) for the whole ring shard of its head group (h/N_h
// query heads, n_kv/N_h KV heads), runs the ring over the N_s ring shards with the devices of
// its head group, and sends each piece's rows back (second exchange).
ra_status check_usp(const ra_problem* p, int32_t n_hg) {
  if (!p) return fail(RA_ERR_INVALID_ARG, "problem is NULL");
  // the layout cuts ring shards of n_hg L tokens (checked on the ring problem), not pieces
  ra_problem pieces = *p;
  if (pieces.layout == RA_LAYOUT_ZIGZAG) pieces.layout = RA_LAYOUT_CONTIGUOUS;
  RA_TRY(check_problem(&pieces));
  if (p->doc_begin) return fail(RA_ERR_UNSUPPORTED, "packed documents are not supported by the two-dimensional path");
  if (n_hg < 1 || p->N % n_hg)
    return fail(RA_ERR_INVALID_ARG, "n_head_groups=%d must divide the device count N=%d", n_hg, p->N);
  if (p->h % n_hg || p->n_kv % n_hg)
    return fail(RA_ERR_INVALID_ARG, "the two-dimensional path splits heads over n_head_groups=%d: h=%d and n_kv=%d "
                "must be multiples of it", n_hg, p->h, p->n_kv);
  if (p->b > 65535) return fail(RA_ERR_UNSUPPORTED, "batch %d above 65535", p->b);
  return RA_OK;
}

// The ring problem one device runs after the first exchange.
ra_problem usp_ring_problem(const ra_problem* p, int32_t n_hg) {
  ra_problem r = *p;
  r.L = p->L * n_hg;
  r.h = p->h / n_hg;
  r.n_kv = p->n_kv / n_hg;
  r.N = p->N / n_hg;
  r.scale = effective_scale(p);
  r.doc_begin = r.doc_end = nullptr;
  return r;
}

struct UspWs {
  size_t q, kv, o, lse, staging, second, total;
};
UspWs usp_ws(const ra_problem* rp) {
  const size_t es = elem_size(rp);
  UspWs w;
  w.q = align_up((size_t)rp->b * rp->L * rp->h * rp->d * es, 256);
  w.kv = align_up((size_t)rp->N * rp->b * rp->L * rp->n_kv * rp->d * es, 256);   // every ring shard's K (or V)
  w.o = align_up((size_t)rp->b * rp->L * rp->h * rp->d * 4, 256);
  w.lse = align_up((size_t)rp->b * rp->h * rp->L * 4, 256);
  w.staging = staging_bytes(rp);
  w.second = second_acc_bytes(rp);
  w.total = w.q + 2 * w.kv + w.o + w.lse + w.staging + w.second;
  return w;
}

ra_status usp_fwd_impl(const ra_problem* p, int32_t n_hg, int32_t g, int32_t r, const void* q_all,
                       const void* k_all, const void* v_all, void* o_all, float* lse_all, void* ws, size_t ws_bytes,
                       ra_stream compute, ra_stream copy, ra_usp_timing* tm) {
  RA_TRY(check_usp(p, n_hg));
  const ra_problem rp = usp_ring_problem(p, n_hg);
  RA_TRY(check_problem(&rp));
  if (g < 0 || g >= n_hg) return fail(RA_ERR_INVALID_ARG, "head_group=%d outside [0, %d)", g, n_hg);
  RA_TRY(check_shard(&rp, r, "ring_rank"));
  RA_TRY(check_ptr(q_all, "q_all", 16));
  RA_TRY(check_ptr(k_all, "k_all", 16));
  RA_TRY(check_ptr(v_all, "v_all", 16));
  RA_TRY(check_ptr(o_all, "o_all", 16));
  RA_TRY(check_ptr(lse_all, "lse_all", 4));
  RA_TRY(check_ptr(ws, "ws", 16));
  const UspWs w = usp_ws(&rp);
  if (ws_bytes < w.total - w.second)
    return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, w.total - w.second);
  const bool second = w.second && ws_bytes >= w.total;   // room for the second accumulator
  if (rp.N > kMaxRing) return fail(RA_ERR_UNSUPPORTED, "ring size N_s=%d above %d", rp.N, kMaxRing);

  char* base = (char*)ws;
  char* q_g = base;
  char* k_ring = base + w.q;
  char* v_ring = k_ring + w.kv;
  float* o_g = (float*)(v_ring + w.kv);
  float* lse_g = (float*)((char*)o_g + w.o);
  char* staging = (char*)lse_g + w.lse;
  const hipStream_t s = (hipStream_t)compute;
  const int es = (int)elem_size(p), Hg = rp.h, Kg = rp.n_kv, N_s = rp.N;
  // bytes of one device's shard of q (all heads) and of k (all KV heads)
  const size_t dev_q = (size_t)p->b * p->L * p->h * p->d * es, dev_kv = (size_t)p->b * p->L * p->n_kv * p->d * es;
  const size_t ring_kv = (size_t)rp.b * rp.L * Kg * p->d * es;   // one ring shard's K of the head group
  const char* qc = (const char*)q_all;
  const char* kc = (const char*)k_all;
  const char* vc = (const char*)v_all;

  Events ev;
  hipEvent_t t0 = nullptr, t1 = nullptr, t2 = nullptr, t3 = nullptr, t4 = nullptr;
  hipError_t e;
  if (tm && ((e = ev.make(&t0, true)) != hipSuccess || (e = ev.make(&t1, true)) != hipSuccess ||
             (e = ev.make(&t2, true)) != hipSuccess || (e = ev.make(&t3, true)) != hipSuccess ||
             (e = ev.make(&t4, true)) != hipSuccess))
    return hip_fail(e, "hipEventCreate");
  auto gather_kv = [&](int rr) -> hipError_t {
    hipError_t x = ra::launch_ulysses_gather(k_ring + (size_t)rr * ring_kv, kc + (size_t)rr * n_hg * dev_kv, p->b,
                                             p->L, n_hg, RA_LAYOUT_CONTIGUOUS, p->n_kv, Kg, g * Kg, p->d, es, s);
    if (x != hipSuccess) return x;
    return ra::launch_ulysses_gather(v_ring + (size_t)rr * ring_kv, vc + (size_t)rr * n_hg * dev_kv, p->b, p->L,
                                     n_hg, RA_LAYOUT_CONTIGUOUS, p->n_kv, Kg, g * Kg, p->d, es, s);
  };
  // The first exchanges of the other ring shards: what the other devices of head group g
  // gather for themselves; on a real machine the ring below receives them from those devices.
  if (tm && (e = hipEventRecord(t0, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  for (int rr = 0; rr < N_s; ++rr)
    if (rr != r && (e = gather_kv(rr)) != hipSuccess) return hip_fail(e, "gather kernel launch");
  // This device's first exchange: Q, K and V of head group g for the whole ring shard r.
  if (tm && (e = hipEventRecord(t1, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if ((e = ra::launch_ulysses_gather(q_g, qc + (size_t)r * n_hg * dev_q, p->b, p->L, n_hg, RA_LAYOUT_CONTIGUOUS, p->h,
                                     Hg, g * Hg, p->d, es, s)) != hipSuccess ||
      (e = gather_kv(r)) != hipSuccess)
    return hip_fail(e, "gather kernel launch");
  if (tm && (e = hipEventRecord(t2, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  // The ring over the N_s ring shards, the merged fp32 result left in o_g.
  float* o2 = second ? (float*)(staging + w.staging) : nullptr;
  float* lse2 = second ? (float*)((char*)o2 + second_o_bytes(&rp)) : nullptr;
  RA_TRY(ring_fwd_impl(&rp, r, q_g, k_ring, v_ring, nullptr, lse_g, staging, w.staging, compute, copy, nullptr,
                       nullptr, o_g, o2, lse2));
  if (tm && (e = hipEventRecord(t3, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  // Second exchange: rows [g' L, (g'+1) L) of the ring shard go back to device r N_h + g'.
  if ((e = ra::launch_ulysses_scatter((char*)o_all + (size_t)r * n_hg * dev_q,
                                      lse_all + (size_t)r * n_hg * p->b * p->h * p->L, o_g, lse_g, p->b, p->L, n_hg,
                                      RA_LAYOUT_CONTIGUOUS, p->h, Hg, g * Hg, p->d, p->dtype, s)) != hipSuccess)
    return hip_fail(e, "scatter kernel launch");
  if (tm) {
    if ((e = hipEventRecord(t4, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipEventSynchronize(t4)) != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    (void)hipEventElapsedTime(&tm->others_gather_ms, t0, t1);
    (void)hipEventElapsedTime(&tm->gather_ms, t1, t2);
    (void)hipEventElapsedTime(&tm->ring_ms, t2, t3);
    (void)hipEventElapsedTime(&tm->scatter_ms, t3, t4);
    tm->total_ms = tm->gather_ms + tm->ring_ms + tm->scatter_ms;
  }
  return RA_OK;
}

ra_status check_bwd_problem(const ra_problem* p);

// Backward of the all-to-all path: the head group's Q, K, V, O, dO (dtype) and LSE, D (fp32)
// of the whole sequence, and its fp32 dQ, dK, dV.
struct UlyssesBwdWs {
  size_t q, kv, lse, dq, dkv, total;
};
UlyssesBwdWs ulysses_bwd_ws(const ra_problem* p) {
  const size_t S = (size_t)p->N * p->L, es = elem_size(p);
  const size_t Hg = p->h / p->N, Kg = p->n_kv / p->N;
  UlyssesBwdWs w;
  w.q = align_up((size_t)p->b * S * Hg * p->d * es, 256);
  w.kv = align_up((size_t)p->b * S * Kg * p->d * es, 256);
  w.lse = align_up((size_t)p->b * Hg * S * 4, 256);
  w.dq = align_up((size_t)p->b * S * Hg * p->d * 4, 256);
  w.dkv = align_up((size_t)p->b * S * Kg * p->d * 4, 256);
  w.total = 3 * w.q + 2 * w.kv + 2 * w.lse + w.dq + 2 * w.dkv;   // q, o, dO; k, v; lse, D; dq; dk, dv
  return w;
}

ra_status check_bwd_problem(const ra_problem* p) {
  RA_TRY(check_problem(p));
  if (p->dtype != RA_BF16 || p->d != 128)
    return fail(RA_ERR_UNSUPPORTED, "the backward supports bf16 with d = 128 only");
  if ((int64_t)p->L * p->h * p->d * 2 >= ((int64_t)1 << 31) ||
      (int64_t)p->L * p->n_kv * p->d * 2 >= ((int64_t)1 << 31))
    return fail(RA_ERR_UNSUPPORTED, "one (batch, head) slice must stay below 2 GiB");
  return RA_OK;
}

// Staging buffers of the key/value-stationary backward: per buffer one query shard's Q and
// dO (dtype) and its LSE and D (fp32).
struct QStage {
  size_t q, lse, one, total;
};
QStage qstage_ws(const ra_problem* p) {
  QStage w;
  w.q = align_up((size_t)p->b * p->L * p->h * p->d * elem_size(p), 256);
  w.lse = align_up((size_t)p->b * p->h * p->L * 4, 256);
  w.one = 2 * w.q + 2 * w.lse;
  w.total = 2 * w.one;
  return w;
}

// Smallest workspace of the backward ring pass: two K/V staging buffers and D.
size_t ring_bwd_workspace_min(const ra_problem* p) {
  const size_t shard_bytes = (size_t)p->b * p->L * p->n_kv * p->d * elem_size(p);
  return 4 * align_up(shard_bytes, 256) + align_up((size_t)p->b * p->h * p->L * 4, 256);
}
// Short shards (no packed documents): second dK, dV buffers, so that the dK/dV kernel may split
// the query tiles of its key blocks over two workgroups when the blocks leave units idle.
bool bwd_split(const ra_problem* p) { return !p->doc_begin && p->L <= ra::kSplitMaxL; }
size_t bwd_second_bytes(const ra_problem* p) {
  return bwd_split(p) ? 2 * align_up((size_t)p->b * p->L * p->n_kv * p->d * 4, 256) : 0;
}
size_t ring_bwd_workspace(const ra_problem* p) { return ring_bwd_workspace_min(p) + bwd_second_bytes(p); }

// The backward ring pass (ra_ring_bwd), optionally timed per step as ra_ring_fwd_timed.
ra_status ring_bwd_impl(const ra_problem* p, int32_t qs, const void* q, const void* k_all, const void* v_all,
                        const void* o, const void* dout, const float* lse, float* dq, float* dk_all, float* dv_all,
                        void* ws, size_t ws_bytes, ra_stream compute, ra_stream copy, ra_ring_timing* tm) {
  RA_TRY(check_bwd_problem(p));
  RA_TRY(check_shard(p, qs, "q_shard"));
  RA_TRY(check_ptr(q, "q", 16));
  RA_TRY(check_ptr(k_all, "k_all", 16));
  RA_TRY(check_ptr(v_all, "v_all", 16));
  RA_TRY(check_ptr(o, "o", 16));
  RA_TRY(check_ptr(dout, "dout", 16));
  RA_TRY(check_ptr(lse, "lse", 4));
  RA_TRY(check_ptr(dq, "dq", 16));
  RA_TRY(check_ptr(dk_all, "dk_all", 16));
  RA_TRY(check_ptr(dv_all, "dv_all", 16));
  RA_TRY(check_ptr(ws, "ws", 16));
  const size_t need = ring_bwd_workspace_min(p);
  if (ws_bytes < need) return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  const int N = p->N;
  if (N > kMaxRing) return fail(RA_ERR_UNSUPPORTED, "ring size N=%d above %d", N, kMaxRing);
  if (tm && N > RA_MAX_TIMED_STEPS)
    return fail(RA_ERR_INVALID_ARG, "timed ring needs N <= %d", RA_MAX_TIMED_STEPS);
  const bool timing = tm != nullptr;
  // the second dK, dV buffers after the minimum, when the workspace holds them
  float* dk2 = nullptr;
  float* dv2 = nullptr;
  if (bwd_split(p) && ws_bytes >= need + bwd_second_bytes(p)) {
    dk2 = (float*)((char*)ws + need);
    dv2 = (float*)((char*)dk2 + bwd_second_bytes(p) / 2);
  }

  const size_t shard_elems = (size_t)p->b * p->L * p->n_kv * p->d;
  const size_t shard_bytes = shard_elems * elem_size(p);
  const size_t A = align_up(shard_bytes, 256);
  char* wsc = (char*)ws;
  char* kbuf[2] = {wsc, wsc + 2 * A};
  char* vbuf[2] = {wsc + A, wsc + 3 * A};
  float* delta = (float*)(wsc + 4 * A);
  const hipStream_t cs = (hipStream_t)compute;
  const hipStream_t ps = copy ? (hipStream_t)copy : cs;
  const bool split = ps != cs;
  const bool poison = poison_staging();

  Events ev;
  hipEvent_t entry, staged[kMaxRing], consumed[kMaxRing];
  hipEvent_t t_sb[RA_MAX_TIMED_STEPS], t_se[RA_MAX_TIMED_STEPS], t_cb[RA_MAX_TIMED_STEPS],
      t_ce[RA_MAX_TIMED_STEPS];
  hipError_t e;
  if ((e = ev.make(&entry, timing)) != hipSuccess) return hip_fail(e, "hipEventCreate");
  for (int k = 0; k < N; ++k) {
    if ((e = ev.make(&staged[k], false)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    if ((e = ev.make(&consumed[k], false)) != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  bool live[kMaxRing];
  int dq_first = -1;                          // the first live step: it stores dQ, later ones add
  for (int k = 0; k < N; ++k) {
    live[k] = step_is_live(p, qs, ((qs - k) % N + N) % N);
    if (live[k] && dq_first < 0) dq_first = k;
  }
  if (timing) {
    tm->n_steps = N;
    for (int k = 0; k < N; ++k) {
      tm->step_begin_ms[k] = tm->step_end_ms[k] = tm->copy_begin_ms[k] = tm->copy_end_ms[k] = -1.f;
      tm->launch_steps[k] = 0;
      if ((e = ev.make(&t_sb[k], true)) != hipSuccess || (e = ev.make(&t_se[k], true)) != hipSuccess ||
          (e = ev.make(&t_cb[k], true)) != hipSuccess || (e = ev.make(&t_ce[k], true)) != hipSuccess)
        return hip_fail(e, "hipEventCreate");
    }
  }
  // The gradient outputs are written, not accumulated into: each KV shard gets the
  // contributions of exactly one ring step, whose launch stores dK and dV (zeros for keys no
  // query sees), and the first live step stores dQ; only what no launch stores is zero-filled
  // (the shards of dead steps, dQ if no step is live).  Then D = rowsum(dO * O).
  if (dq_first < 0 && (e = ra::launch_fill_lse(dq, (int64_t)p->b * p->L * p->h * p->d, 0.f, cs)) != hipSuccess)
    return hip_fail(e, "fill kernel launch");
  for (int k = 0; k < N; ++k) {
    if (live[k]) continue;
    const size_t src = (size_t)(((qs - k) % N + N) % N);
    if ((e = ra::launch_fill_lse(dk_all + src * shard_elems, (int64_t)shard_elems, 0.f, cs)) != hipSuccess ||
        (e = ra::launch_fill_lse(dv_all + src * shard_elems, (int64_t)shard_elems, 0.f, cs)) != hipSuccess)
      return hip_fail(e, "fill kernel launch");
  }
  if ((e = ra::launch_bwd_preprocess(o, dout, delta, p->b, p->L, p->h, cs)) != hipSuccess)
    return hip_fail(e, "preprocess kernel launch");
  if ((e = hipEventRecord(entry, cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (split && (e = hipStreamWaitEvent(ps, entry, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");

  const char* kc = (const char*)k_all;
  const char* vc = (const char*)v_all;
  for (int k = 0; k < N; ++k) {
    if (k + 1 < N) {
      const int dst = (k + 1) & 1;
      if (split && k - 1 >= 1 && (e = hipStreamWaitEvent(ps, consumed[k - 1], 0)) != hipSuccess)
        return hip_fail(e, "hipStreamWaitEvent");
      if (timing && (e = hipEventRecord(t_cb[k + 1], ps)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      if ((e = stage_kv(kbuf[dst], vbuf[dst], k_all, v_all, shard_bytes, 0, N, qs, k + 1, 1, ps)) != hipSuccess)
        return hip_fail(e, "staging copy");
      if (timing && (e = hipEventRecord(t_ce[k + 1], ps)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      if ((e = hipEventRecord(staged[k + 1], ps)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    if (split && k >= 1 && (e = hipStreamWaitEvent(cs, staged[k], 0)) != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent");
    const int src = ((qs - k) % N + N) % N;
    const void* kp = k == 0 ? (const void*)(kc + (size_t)qs * shard_bytes) : (const void*)kbuf[k & 1];
    const void* vp = k == 0 ? (const void*)(vc + (size_t)qs * shard_bytes) : (const void*)vbuf[k & 1];
    if (live[k]) {
      if (timing && (e = hipEventRecord(t_sb[k], cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      const ra::StepArgs a = step_args(p, qs, src, q, kp, vp, nullptr, nullptr);
      if ((e = ra::launch_step_bwd_bf16(a, dout, lse, delta, dq, dk_all + (size_t)src * shard_elems,
                                        dv_all + (size_t)src * shard_elems, cs, k == dq_first, true, dk2, dv2)) !=
          hipSuccess)
        return hip_fail(e, "backward step kernel launch");
      if (timing && (e = hipEventRecord(t_se[k], cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    if ((e = hipEventRecord(consumed[k], cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if (poison && k >= 1 &&
        ((e = poison_after(kbuf[k & 1], shard_bytes, consumed[k], ps, split)) != hipSuccess ||
         (e = poison_after(vbuf[k & 1], shard_bytes, consumed[k], ps, split)) != hipSuccess))
      return hip_fail(e, "staging poison");
  }
  if (timing) {
    hipEvent_t done;
    if ((e = ev.make(&done, true)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    if ((e = hipEventRecord(done, cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipEventSynchronize(done)) != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    (void)hipEventElapsedTime(&tm->total_ms, entry, done);
    for (int k = 0; k < N; ++k) {
      if (live[k]) {
        (void)hipEventElapsedTime(&tm->step_begin_ms[k], entry, t_sb[k]);
        (void)hipEventElapsedTime(&tm->step_end_ms[k], entry, t_se[k]);
        tm->launch_steps[k] = 1;
      }
      if (k >= 1) {
        (void)hipEventElapsedTime(&tm->copy_begin_ms[k], entry, t_cb[k]);
        (void)hipEventElapsedTime(&tm->copy_end_ms[k], entry, t_ce[k]);
      }
    }
  }
  return RA_OK;
}

// ---- allocation-free forward pass --------------------------------------------------------
// For callers that cannot allocate device memory: the staging double buffer and the fp32
// accumulator of ra_ring_fwd live in this fixed device array instead of a caller workspace.
// Host code never passes `scratch` itself to a kernel or a copy (on the host it only names the
// symbol); it uses the device address that hipGetSymbolAddress returns, looked up once per
// device with that device current and kept in g_scratch.
__device__ __align__(256) unsigned char scratch[RA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchDevice {
  void* ptr = nullptr;   // this device's address of `scratch`
  RingEvents events;     // made once, reused by every call on the device
  bool ready = false;
};
std::mutex g_scratch_mu;
ScratchDevice g_scratch[kMaxDevices];

// Set-up on the first call on the current device: the array's address and the events.
ra_status scratch_for_current_device(const ScratchDevice** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(RA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchDevice& s = g_scratch[dev];
  if (!s.ready) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
      return hip_fail(e, "hipGetSymbolAddress(scratch)");
    RingEvents ev;
    hipEvent_t* all[1 + 2 * kMaxRing];
    int n = 0;
    all[n++] = &ev.entry;
    for (int k = 0; k < kMaxRing; ++k) {
      all[n++] = &ev.staged[k];
      all[n++] = &ev.consumed[k];
    }
    for (int i = 0; i < n; ++i) {
      if ((e = hipEventCreateWithFlags(all[i], hipEventDisableTiming)) != hipSuccess) {
        for (int j = 0; j < i; ++j) (void)hipEventDestroy(*all[j]);
        return hip_fail(e, "hipEventCreate");
      }
    }
    s.ptr = ptr;
    s.events = ev;
    s.ready = true;
  }
  *out = &s;
  return RA_OK;
}

}  // namespace

extern "C" {

const char* ra_status_string(ra_status s) {
  switch (s) {
    case RA_OK: return "ok";
    case RA_ERR_INVALID_ARG: return "invalid argument";
    case RA_ERR_UNSUPPORTED: return "unsupported problem";
    case RA_ERR_WORKSPACE: return "workspace too small";
    case RA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* ra_last_error(void) { return g_last_error.c_str(); }

ra_status ra_step_fwd(const ra_problem* p, int32_t q_shard, int32_t kv_shard, const void* q,
                      const void* k, const void* v, float* o_part, float* lse_part, ra_stream stream) {
  RA_TRY(check_problem(p));
  RA_TRY(check_shard(p, q_shard, "q_shard"));
  RA_TRY(check_shard(p, kv_shard, "kv_shard"));
  RA_TRY(check_ptr(q, "q", 16));
  RA_TRY(check_ptr(k, "k", 16));
  RA_TRY(check_ptr(v, "v", 16));
  RA_TRY(check_ptr(o_part, "o_part", 16));
  RA_TRY(check_ptr(lse_part, "lse_part", 4));
  const ra::StepArgs a = step_args(p, q_shard, kv_shard, q, k, v, o_part, lse_part);
  const hipError_t e = launch_step(p, a, ra::MODE_PART, (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "step kernel launch");
}

ra_status ra_merge_lse(const ra_problem* p, float* o_acc, float* lse_acc, const float* o_part,
                       const float* lse_part, ra_stream stream) {
  RA_TRY(check_problem(p));
  RA_TRY(check_ptr(o_acc, "o_acc", 16));
  RA_TRY(check_ptr(lse_acc, "lse_acc", 4));
  RA_TRY(check_ptr(o_part, "o_part", 16));
  RA_TRY(check_ptr(lse_part, "lse_part", 4));
  const hipError_t e =
      ra::launch_merge(o_acc, lse_acc, o_part, lse_part, p->b, p->L, p->h, p->d, (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "merge kernel launch");
}

ra_status ra_finalize(const ra_problem* p, const float* o_acc, void* o, ra_stream stream) {
  RA_TRY(check_problem(p));
  RA_TRY(check_ptr(o_acc, "o_acc", 16));
  RA_TRY(check_ptr(o, "o", 16));
  const hipError_t e = ra::launch_finalize(o_acc, o, p->dtype, (int64_t)p->b * p->L * p->h * p->d,
                                           (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "finalize kernel launch");
}

ra_status ra_fwd_step_plan(const ra_problem* p, int32_t q_shard, int32_t kv_shard, int32_t n_cu, int32_t* block,
                           int32_t* part, int32_t max_items, int32_t* n_items, int32_t* block_rows) {
  RA_TRY(check_problem(p));
  RA_TRY(check_shard(p, q_shard, "q_shard"));
  RA_TRY(check_shard(p, kv_shard, "kv_shard"));
  if (!n_items || !block_rows || (max_items > 0 && (!block || !part)))
    return fail(RA_ERR_INVALID_ARG, "output pointer is NULL");
  if (p->dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "the step plan describes the bf16 kernel");
  if (n_cu < 1) return fail(RA_ERR_INVALID_ARG, "n_cu=%d must be positive", n_cu);
  const ra::StepArgs a = step_args(p, q_shard, kv_shard, nullptr, nullptr, nullptr, nullptr, nullptr);
  const ra::StepGeometry g = ra::step_geometry_bf16(a);
  ra::SplitPlan pl{};
  pl.split_from = g.n_qb;
  if (fwd_split(p)) pl = ra::plan_split(a, g, n_cu);
  const int n = pl.split_from + 2 * (g.n_qb - pl.split_from);
  *n_items = n;
  *block_rows = g.rows_wg;
  for (int i = 0; i < n && i < max_items; ++i) {
    int qb, pt;
    ra::split_item(pl, g.n_qb, i, qb, pt);
    block[i] = qb;
    part[i] = qb >= pl.split_from ? pt : -1;
  }
  return RA_OK;
}

size_t ra_ring_fwd_workspace(const ra_problem* p) {
  if (check_problem(p) != RA_OK) return 0;
  return (fwd_steps_per_launch(p) >= 2 ? batch_workspace(p) : ring_fwd_base_workspace(p)) + second_acc_bytes(p);
}

ra_status ra_ring_fwd(const ra_problem* p, int32_t q_shard, const void* q, const void* k_all,
                      const void* v_all, void* o, float* lse, void* ws, size_t ws_bytes,
                      ra_stream compute, ra_stream copy) {
  return ring_fwd_impl(p, q_shard, q, k_all, v_all, o, lse, ws, ws_bytes, compute, copy, nullptr);
}

ra_status ra_ring_fwd_timed(const ra_problem* p, int32_t q_shard, const void* q,
                            const void* k_all, const void* v_all, void* o, float* lse, void* ws,
                            size_t ws_bytes, ra_stream compute, ra_stream copy, ra_ring_timing* t) {
  if (!t) return fail(RA_ERR_INVALID_ARG, "timing output is NULL");
  return ring_fwd_impl(p, q_shard, q, k_all, v_all, o, lse, ws, ws_bytes, compute, copy, t);
}

ra_status ra_ring_fwd_noalloc(const ra_problem* p, int32_t q_shard, const void* q, const void* k_all,
                              const void* v_all, void* o, float* lse, ra_stream compute, ra_stream copy) {
  RA_TRY(check_problem(p));
  RA_TRY(check_shard(p, q_shard, "q_shard"));
  RA_TRY(check_ptr(q, "q", 16));
  RA_TRY(check_ptr(k_all, "k_all", 16));
  RA_TRY(check_ptr(v_all, "v_all", 16));
  RA_TRY(check_ptr(o, "o", 16));
  RA_TRY(check_ptr(lse, "lse", 4));
  const size_t need = ring_fwd_base_workspace(p);   // with the second accumulator only if it fits too
  if (need > RA_NOALLOC_SCRATCH_BYTES)
    return fail(RA_ERR_WORKSPACE, "this problem needs %zu bytes of scratch; the allocation-free entry point holds %zu",
                need, (size_t)RA_NOALLOC_SCRATCH_BYTES);
  if (p->N > kMaxRing) return fail(RA_ERR_UNSUPPORTED, "ring size N=%d above %d", p->N, kMaxRing);
  const ScratchDevice* s = nullptr;
  RA_TRY(scratch_for_current_device(&s));
  return ring_fwd_impl(p, q_shard, q, k_all, v_all, o, lse, s->ptr, RA_NOALLOC_SCRATCH_BYTES, compute, copy,
                       nullptr, &s->events);
}

ra_status ra_bwd_preprocess(const ra_problem* p, const void* o, const void* dout, float* delta,
                            ra_stream stream) {
  RA_TRY(check_bwd_problem(p));
  RA_TRY(check_ptr(o, "o", 16));
  RA_TRY(check_ptr(dout, "dout", 16));
  RA_TRY(check_ptr(delta, "delta", 4));
  const hipError_t e = ra::launch_bwd_preprocess(o, dout, delta, p->b, p->L, p->h, (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "preprocess kernel launch");
}

ra_status ra_step_bwd(const ra_problem* p, int32_t q_shard, int32_t kv_shard, const void* q,
                      const void* k, const void* v, const void* dout, const float* lse,
                      const float* delta, float* dq_acc, float* dk_acc, float* dv_acc,
                      ra_stream stream) {
  RA_TRY(check_bwd_problem(p));
  RA_TRY(check_shard(p, q_shard, "q_shard"));
  RA_TRY(check_shard(p, kv_shard, "kv_shard"));
  RA_TRY(check_ptr(q, "q", 16));
  RA_TRY(check_ptr(k, "k", 16));
  RA_TRY(check_ptr(v, "v", 16));
  RA_TRY(check_ptr(dout, "dout", 16));
  RA_TRY(check_ptr(lse, "lse", 4));
  RA_TRY(check_ptr(delta, "delta", 4));
  RA_TRY(check_ptr(dq_acc, "dq_acc", 16));
  RA_TRY(check_ptr(dk_acc, "dk_acc", 16));
  RA_TRY(check_ptr(dv_acc, "dv_acc", 16));
  const ra::StepArgs a = step_args(p, q_shard, kv_shard, q, k, v, nullptr, nullptr);
  const hipError_t e = ra::launch_step_bwd_bf16(a, dout, lse, delta, dq_acc, dk_acc, dv_acc,
                                                (hipStream_t)stream);
  return e == hipSuccess ? RA_OK : hip_fail(e, "backward step kernel launch");
}

size_t ra_ring_bwd_workspace(const ra_problem* p) {
  if (check_bwd_problem(p) != RA_OK) return 0;
  return ring_bwd_workspace(p);
}

size_t ra_ring_bwd_workspace_min(const ra_problem* p) {
  if (check_bwd_problem(p) != RA_OK) return 0;
  return ring_bwd_workspace_min(p);
}

ra_status ra_ring_bwd(const ra_problem* p, int32_t qs, const void* q, const void* k_all,
                      const void* v_all, const void* o, const void* dout, const float* lse,
                      float* dq, float* dk_all, float* dv_all, void* ws, size_t ws_bytes,
                      ra_stream compute, ra_stream copy) {
  return ring_bwd_impl(p, qs, q, k_all, v_all, o, dout, lse, dq, dk_all, dv_all, ws, ws_bytes, compute, copy,
                       nullptr);
}

ra_status ra_ring_bwd_timed(const ra_problem* p, int32_t qs, const void* q, const void* k_all,
                            const void* v_all, const void* o, const void* dout, const float* lse,
                            float* dq, float* dk_all, float* dv_all, void* ws, size_t ws_bytes,
                            ra_stream compute, ra_stream copy, ra_ring_timing* t) {
  if (!t) return fail(RA_ERR_INVALID_ARG, "timing output is NULL");
  return ring_bwd_impl(p, qs, q, k_all, v_all, o, dout, lse, dq, dk_all, dv_all, ws, ws_bytes, compute, copy, t);
}

size_t ra_ring_bwd_kv_stationary_workspace(const ra_problem* p) {
  if (check_bwd_problem(p) != RA_OK || p->doc_begin) return 0;
  return qstage_ws(p).total;
}

ra_status ra_ring_bwd_kv_stationary(const ra_problem* p, int32_t ks, const void* k_home, const void* v_home,
                                    const void* q_all, const void* dout_all, const float* lse_all,
                                    const float* delta_all, float* dq_all, float* dk, float* dv, void* ws,
                                    size_t ws_bytes, ra_stream compute, ra_stream copy) {
  RA_TRY(check_bwd_problem(p));
  if (p->doc_begin)   // the bounds describe one query shard's rows; here every step has another
    return fail(RA_ERR_UNSUPPORTED, "packed documents are not supported with stationary keys and values");
  RA_TRY(check_shard(p, ks, "kv_shard"));
  RA_TRY(check_ptr(k_home, "k", 16));
  RA_TRY(check_ptr(v_home, "v", 16));
  RA_TRY(check_ptr(q_all, "q_all", 16));
  RA_TRY(check_ptr(dout_all, "dout_all", 16));
  RA_TRY(check_ptr(lse_all, "lse_all", 4));
  RA_TRY(check_ptr(delta_all, "delta_all", 4));
  RA_TRY(check_ptr(dq_all, "dq_all", 16));
  RA_TRY(check_ptr(dk, "dk", 16));
  RA_TRY(check_ptr(dv, "dv", 16));
  RA_TRY(check_ptr(ws, "ws", 16));
  const QStage w = qstage_ws(p);
  if (ws_bytes < w.total) return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, w.total);
  const int N = p->N;
  if (N > kMaxRing) return fail(RA_ERR_UNSUPPORTED, "ring size N=%d above %d", N, kMaxRing);

  const size_t q_elems = (size_t)p->b * p->L * p->h * p->d;
  const size_t q_bytes = q_elems * elem_size(p);
  const size_t row_elems = (size_t)p->b * p->h * p->L;
  const size_t kv_elems = (size_t)p->b * p->L * p->n_kv * p->d;
  char* buf[2] = {(char*)ws, (char*)ws + w.one};
  const hipStream_t cs = (hipStream_t)compute;
  const hipStream_t ps = copy ? (hipStream_t)copy : cs;
  const bool split = ps != cs;
  const bool poison = poison_staging();

  Events ev;
  hipEvent_t entry, staged[kMaxRing], consumed[kMaxRing];
  hipError_t e;
  if ((e = ev.make(&entry, false)) != hipSuccess) return hip_fail(e, "hipEventCreate");
  for (int k = 0; k < N; ++k) {
    if ((e = ev.make(&staged[k], false)) != hipSuccess) return hip_fail(e, "hipEventCreate");
    if ((e = ev.make(&consumed[k], false)) != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  if ((e = ra::launch_fill_lse(dq_all, (int64_t)(q_elems * N), 0.f, cs)) != hipSuccess ||
      (e = ra::launch_fill_lse(dk, (int64_t)kv_elems, 0.f, cs)) != hipSuccess ||
      (e = ra::launch_fill_lse(dv, (int64_t)kv_elems, 0.f, cs)) != hipSuccess)
    return hip_fail(e, "fill kernel launch");
  if ((e = hipEventRecord(entry, cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (split && (e = hipStreamWaitEvent(ps, entry, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");

  const char* qc = (const char*)q_all;
  const char* oc = (const char*)dout_all;
  auto shard_of = [&](int step) { return (ks + step) % N; };   // query shard held at this step
  for (int k = 0; k < N; ++k) {
    if (k + 1 < N) {
      // stage query shard (ks + k + 1) mod N into buffer (k + 1) % 2, last read by step k - 1
      const int i = shard_of(k + 1);
      char* dst = buf[(k + 1) & 1];
      if (split && k - 1 >= 1 && (e = hipStreamWaitEvent(ps, consumed[k - 1], 0)) != hipSuccess)
        return hip_fail(e, "hipStreamWaitEvent");
      if ((e = hipMemcpyAsync(dst, qc + (size_t)i * q_bytes, q_bytes, hipMemcpyDeviceToDevice, ps)) != hipSuccess ||
          (e = hipMemcpyAsync(dst + w.q, oc + (size_t)i * q_bytes, q_bytes, hipMemcpyDeviceToDevice, ps)) !=
              hipSuccess ||
          (e = hipMemcpyAsync(dst + 2 * w.q, lse_all + (size_t)i * row_elems, row_elems * 4, hipMemcpyDeviceToDevice,
                              ps)) != hipSuccess ||
          (e = hipMemcpyAsync(dst + 2 * w.q + w.lse, delta_all + (size_t)i * row_elems, row_elems * 4,
                              hipMemcpyDeviceToDevice, ps)) != hipSuccess)
        return hip_fail(e, "hipMemcpyAsync(query shard)");
      if ((e = hipEventRecord(staged[k + 1], ps)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    if (split && k >= 1 && (e = hipStreamWaitEvent(cs, staged[k], 0)) != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent");
    const int i = shard_of(k);
    const char* b = buf[k & 1];
    const void* qp = k == 0 ? (const void*)(qc + (size_t)i * q_bytes) : (const void*)b;
    const void* op = k == 0 ? (const void*)(oc + (size_t)i * q_bytes) : (const void*)(b + w.q);
    const float* lp = k == 0 ? lse_all + (size_t)i * row_elems : (const float*)(b + 2 * w.q);
    const float* dp = k == 0 ? delta_all + (size_t)i * row_elems : (const float*)(b + 2 * w.q + w.lse);
    if (step_is_live(p, i, ks)) {
      const ra::StepArgs a = step_args(p, i, ks, qp, k_home, v_home, nullptr, nullptr);
      if ((e = ra::launch_step_bwd_bf16(a, op, lp, dp, dq_all + (size_t)i * q_elems, dk, dv, cs)) != hipSuccess)
        return hip_fail(e, "backward step kernel launch");
    }
    if ((e = hipEventRecord(consumed[k], cs)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if (poison && k >= 1 && (e = poison_after(buf[k & 1], w.one, consumed[k], ps, split)) != hipSuccess)
      return hip_fail(e, "staging poison");
  }
  return RA_OK;
}

int64_t ra_allowed_pairs(const ra_problem* p, int32_t q_shard, int32_t kv_shard) {
  if (check_shape(p) != RA_OK) return -1;
  if (q_shard < 0 || q_shard >= p->N || kv_shard < -1 || kv_shard >= p->N) return -1;
  int64_t total = 0;
  for (int ks = 0; ks < p->N; ++ks) {
    if (kv_shard >= 0 && ks != kv_shard) continue;
    for (int t = 0; t < p->L; ++t) total += ra::kv_limit(p->causal, p->layout, p->N, p->L, q_shard, ks, t);
  }
  return total * p->b;
}

int64_t ra_allowed_pairs_packed(const ra_problem* p, int32_t q_shard, int32_t kv_shard,
                                const int32_t* doc_begin_host, const int32_t* doc_end_host) {
  if (check_shape(p) != RA_OK) return -1;
  if (q_shard < 0 || q_shard >= p->N || kv_shard < -1 || kv_shard >= p->N) return -1;
  if (!doc_begin_host || !doc_end_host) return -1;
  int64_t total = 0;
  for (int bi = 0; bi < p->b; ++bi)
    for (int ks = 0; ks < p->N; ++ks) {
      if (kv_shard >= 0 && ks != kv_shard) continue;
      for (int t = 0; t < p->L; ++t) {
        const int64_t i = (int64_t)bi * p->L + t;
        const ra::KeyRange r = ra::key_range(p->causal, p->layout, p->N, p->L, q_shard, ks, t, true,
                                             doc_begin_host[i], doc_end_host[i]);
        total += r.hi - r.lo;
      }
    }
  return total;
}

size_t ra_usp_fwd_workspace(const ra_problem* p, int32_t n_head_groups) {
  if (check_usp(p, n_head_groups) != RA_OK) return 0;
  const ra_problem rp = usp_ring_problem(p, n_head_groups);
  if (check_problem(&rp) != RA_OK) return 0;
  return usp_ws(&rp).total;
}

ra_status ra_usp_fwd(const ra_problem* p, int32_t n_head_groups, int32_t head_group, int32_t ring_rank,
                     const void* q_all, const void* k_all, const void* v_all, void* o_all, float* lse_all, void* ws,
                     size_t ws_bytes, ra_stream compute, ra_stream copy) {
  return usp_fwd_impl(p, n_head_groups, head_group, ring_rank, q_all, k_all, v_all, o_all, lse_all, ws, ws_bytes,
                      compute, copy, nullptr);
}

ra_status ra_usp_fwd_timed(const ra_problem* p, int32_t n_head_groups, int32_t head_group, int32_t ring_rank,
                           const void* q_all, const void* k_all, const void* v_all, void* o_all, float* lse_all,
                           void* ws, size_t ws_bytes, ra_stream compute, ra_stream copy, ra_usp_timing* t) {
  if (!t) return fail(RA_ERR_INVALID_ARG, "timing output is NULL");
  return usp_fwd_impl(p, n_head_groups, head_group, ring_rank, q_all, k_all, v_all, o_all, lse_all, ws, ws_bytes,
                      compute, copy, t);
}

size_t ra_ulysses_bwd_workspace(const ra_problem* p) {
  if (check_ulysses(p) != RA_OK) return 0;
  const ra_problem lp = ulysses_local(p);
  if (check_bwd_problem(&lp) != RA_OK) return 0;
  return ulysses_bwd_ws(p).total;
}

ra_status ra_ulysses_bwd(const ra_problem* p, int32_t group, const void* q_all, const void* k_all,
                         const void* v_all, const void* o_all, const void* dout_all, const float* lse_all,
                         float* dq_all, float* dk_all, float* dv_all, void* ws, size_t ws_bytes, ra_stream stream) {
  RA_TRY(check_ulysses(p));
  RA_TRY(check_shard(p, group, "head_group"));
  const ra_problem lp = ulysses_local(p);
  RA_TRY(check_bwd_problem(&lp));
  RA_TRY(check_ptr(q_all, "q_all", 16));
  RA_TRY(check_ptr(k_all, "k_all", 16));
  RA_TRY(check_ptr(v_all, "v_all", 16));
  RA_TRY(check_ptr(o_all, "o_all", 16));
  RA_TRY(check_ptr(dout_all, "dout_all", 16));
  RA_TRY(check_ptr(lse_all, "lse_all", 4));
  RA_TRY(check_ptr(dq_all, "dq_all", 16));
  RA_TRY(check_ptr(dk_all, "dk_all", 16));
  RA_TRY(check_ptr(dv_all, "dv_all", 16));
  RA_TRY(check_ptr(ws, "ws", 16));
  const UlyssesBwdWs w = ulysses_bwd_ws(p);
  if (ws_bytes < w.total) return fail(RA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, w.total);

  char* c = (char*)ws;
  void* q_g = c;
  void* o_g = c + w.q;
  void* do_g = c + 2 * w.q;
  void* k_g = c + 3 * w.q;
  void* v_g = c + 3 * w.q + w.kv;
  float* lse_g = (float*)(c + 3 * w.q + 2 * w.kv);
  float* dl_g = (float*)(c + 3 * w.q + 2 * w.kv + w.lse);
  float* dq_g = (float*)(c + 3 * w.q + 2 * w.kv + 2 * w.lse);
  float* dk_g = (float*)(c + 3 * w.q + 2 * w.kv + 2 * w.lse + w.dq);
  float* dv_g = (float*)(c + 3 * w.q + 2 * w.kv + 2 * w.lse + w.dq + w.dkv);
  const hipStream_t s = (hipStream_t)stream;
  const int Hg = p->h / p->N, Kg = p->n_kv / p->N, es = (int)elem_size(p);
  const int64_t S = (int64_t)p->N * p->L;
  hipError_t e;
  // first exchange: the head group's inputs of the whole sequence
  if ((e = ra::launch_ulysses_gather(q_g, q_all, p->b, p->L, p->N, p->layout, p->h, Hg, group * Hg, p->d, es, s)) !=
          hipSuccess ||
      (e = ra::launch_ulysses_gather(o_g, o_all, p->b, p->L, p->N, p->layout, p->h, Hg, group * Hg, p->d, es, s)) !=
          hipSuccess ||
      (e = ra::launch_ulysses_gather(do_g, dout_all, p->b, p->L, p->N, p->layout, p->h, Hg, group * Hg, p->d, es,
                                     s)) != hipSuccess ||
      (e = ra::launch_ulysses_gather(k_g, k_all, p->b, p->L, p->N, p->layout, p->n_kv, Kg, group * Kg, p->d, es, s)) !=
          hipSuccess ||
      (e = ra::launch_ulysses_gather(v_g, v_all, p->b, p->L, p->N, p->layout, p->n_kv, Kg, group * Kg, p->d, es, s)) !=
          hipSuccess ||
      (e = ra::launch_ulysses_gather_rows(lse_g, lse_all, p->b, p->L, p->N, p->layout, p->h, Hg, group * Hg, s)) !=
          hipSuccess)
    return hip_fail(e, "gather kernel launch");
  // the backward of the whole-sequence attention
  if ((e = ra::launch_bwd_preprocess(o_g, do_g, dl_g, p->b, (int)S, Hg, s)) != hipSuccess)
    return hip_fail(e, "preprocess kernel launch");
  if ((e = ra::launch_fill_lse(dq_g, (int64_t)p->b * S * Hg * p->d, 0.f, s)) != hipSuccess ||
      (e = ra::launch_fill_lse(dk_g, (int64_t)p->b * S * Kg * p->d, 0.f, s)) != hipSuccess ||
      (e = ra::launch_fill_lse(dv_g, (int64_t)p->b * S * Kg * p->d, 0.f, s)) != hipSuccess)
    return hip_fail(e, "fill kernel launch");
  const ra::StepArgs a = step_args(&lp, 0, 0, q_g, k_g, v_g, nullptr, nullptr);
  if ((e = ra::launch_step_bwd_bf16(a, do_g, lse_g, dl_g, dq_g, dk_g, dv_g, s)) != hipSuccess)
    return hip_fail(e, "backward step kernel launch");
  // second exchange: the gradients back to the shards
  if ((e = ra::launch_ulysses_scatter_rows(dq_all, dq_g, p->b, p->L, p->N, p->layout, p->h, Hg, group * Hg, p->d,
                                           RA_F32, s)) != hipSuccess ||
      (e = ra::launch_ulysses_scatter_rows(dk_all, dk_g, p->b, p->L, p->N, p->layout, p->n_kv, Kg, group * Kg, p->d,
                                           RA_F32, s)) != hipSuccess ||
      (e = ra::launch_ulysses_scatter_rows(dv_all, dv_g, p->b, p->L, p->N, p->layout, p->n_kv, Kg, group * Kg, p->d,
                                           RA_F32, s)) != hipSuccess)
    return hip_fail(e, "scatter kernel launch");
  return RA_OK;
}

size_t ra_ulysses_fwd_workspace(const ra_problem* p) {
  if (check_ulysses(p) != RA_OK) return 0;
  const ra_problem lp = ulysses_local(p);
  if (check_problem(&lp) != RA_OK) return 0;
  return ulysses_ws(p).total;
}

ra_status ra_ulysses_fwd(const ra_problem* p, int32_t head_group, const void* q_all, const void* k_all,
                         const void* v_all, void* o_all, float* lse_all, void* ws, size_t ws_bytes,
                         ra_stream stream) {
  return ulysses_fwd_impl(p, head_group, q_all, k_all, v_all, o_all, lse_all, ws, ws_bytes, stream, nullptr);
}

ra_status ra_ulysses_fwd_timed(const ra_problem* p, int32_t head_group, const void* q_all, const void* k_all,
                               const void* v_all, void* o_all, float* lse_all, void* ws, size_t ws_bytes,
                               ra_stream stream, ra_ulysses_timing* t) {
  if (!t) return fail(RA_ERR_INVALID_ARG, "timing is NULL");
  return ulysses_fwd_impl(p, head_group, q_all, k_all, v_all, o_all, lse_all, ws, ws_bytes, stream, t);
}

ra_status ra_document_ranges(const ra_problem* p, int32_t shard, const int32_t* bounds,
                             int32_t n_docs, int32_t* begin_out, int32_t* end_out) {
  RA_TRY(check_shape(p));
  RA_TRY(check_shard(p, shard, "shard"));
  if (!bounds || !begin_out || !end_out) return fail(RA_ERR_INVALID_ARG, "NULL array");
  const int64_t S = (int64_t)p->N * p->L;
  if (n_docs < 1 || bounds[0] != 0 || bounds[n_docs] != S)
    return fail(RA_ERR_INVALID_ARG, "bounds must run from 0 to S=%lld over n_docs >= 1 documents",
                (long long)S);
  for (int i = 0; i < n_docs; ++i)
    if (bounds[i + 1] <= bounds[i]) return fail(RA_ERR_INVALID_ARG, "bounds not strictly increasing at %d", i);
  for (int t = 0; t < p->L; ++t) {
    const int64_t P = ra::global_pos(p->layout, p->N, p->L, shard, t);
    int lo = 0, hi = n_docs;                   // largest i with bounds[i] <= P
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (bounds[mid] <= P) lo = mid;
      else hi = mid;
    }
    begin_out[t] = bounds[lo];
    end_out[t] = bounds[lo + 1];
  }
  return RA_OK;
}

}  // extern "C"

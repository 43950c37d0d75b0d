// Host-side exercise of the C-ABI for an AddressSanitizer / UndefinedBehaviorSanitizer build of
// the library's host code: every entry point is called with arguments that validation must
// refuse before any HIP call (so no device is touched), and the host-only helpers run on valid
// inputs.  Prints "checks failures" and exits non-zero on any wrong status; a sanitizer report
// aborts the process.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "ra.h"

static long n_checks = 0, n_fail = 0;
// The second accumulator that ra_ring_fwd_workspace includes for short bf16 shards; a
// workspace without it is accepted.
static size_t al256(size_t x) { return (x + 255) / 256 * 256; }
static size_t second_acc(size_t b, size_t L, size_t h, size_t d) { return al256(b * L * h * d * 4) + al256(b * h * L * 4); }
static void expect(bool ok, const char* what) {
  ++n_checks;
  if (!ok) {
    ++n_fail;
    fprintf(stderr, "FAILED: %s (last error: %s)\n", what, ra_last_error());
  }
}

int main() {
  void* F = (void*)0x10000;   // aligned, never dereferenced: validation fails before any use
  float* Ff = (float*)F;
  void* mis = (void*)0x10002;
  ra_problem p = {1, 128, 4, 2, 128, 4, 1, RA_LAYOUT_STRIPED, RA_BF16, 0.f, nullptr, nullptr};

  // problems refused by every entry point
  ra_problem bad[6] = {p, p, p, p, p, p};
  bad[0].h = 3;                       // not a multiple of n_kv
  bad[1].L = 0;
  bad[2].layout = 7;
  bad[3].d = 64;                      // bf16 supports d = 128 only
  bad[4].layout = RA_LAYOUT_ZIGZAG;
  bad[4].L = 127;                     // zigzag needs an even L
  bad[5].scale = 1.0f / 0.0f;
  for (const ra_problem& b : bad) {
    expect(ra_step_fwd(&b, 0, 0, F, F, F, Ff, Ff, nullptr) < 0, "step_fwd bad problem");
    expect(ra_ring_fwd(&b, 0, F, F, F, F, Ff, F, 1u << 30, nullptr, nullptr) < 0, "ring_fwd bad problem");
    expect(ra_ring_fwd_noalloc(&b, 0, F, F, F, F, Ff, nullptr, nullptr) < 0, "ring_fwd_noalloc bad problem");
    expect(ra_step_bwd(&b, 0, 0, F, F, F, F, Ff, Ff, Ff, Ff, Ff, nullptr) < 0, "step_bwd bad problem");
    expect(ra_ring_bwd(&b, 0, F, F, F, F, F, Ff, Ff, Ff, Ff, F, 1u << 30, nullptr, nullptr) < 0, "ring_bwd bad problem");
    expect(ra_ring_bwd_kv_stationary(&b, 0, F, F, F, F, Ff, Ff, Ff, Ff, Ff, F, 1u << 30, nullptr, nullptr) < 0,
           "kv_stationary bad problem");
    expect(ra_ulysses_fwd(&b, 0, F, F, F, F, Ff, F, 1u << 30, nullptr) < 0, "ulysses_fwd bad problem");
    expect(ra_ulysses_bwd(&b, 0, F, F, F, F, F, Ff, Ff, Ff, Ff, F, 1u << 30, nullptr) < 0, "ulysses_bwd bad problem");
    expect(ra_ring_fwd_workspace(&b) == 0, "ring_fwd_workspace bad problem");
    // pair counting depends on shapes and positions only, not on d
    expect((ra_allowed_pairs(&b, 0, -1) == -1) == (&b != &bad[3]), "allowed_pairs bad problem");
  }
  // null problem
  expect(ra_step_fwd(nullptr, 0, 0, F, F, F, Ff, Ff, nullptr) == RA_ERR_INVALID_ARG, "step_fwd null problem");
  expect(ra_merge_lse(nullptr, Ff, Ff, Ff, Ff, nullptr) == RA_ERR_INVALID_ARG, "merge null problem");
  expect(ra_finalize(nullptr, Ff, F, nullptr) == RA_ERR_INVALID_ARG, "finalize null problem");
  expect(ra_bwd_preprocess(nullptr, F, F, Ff, nullptr) == RA_ERR_INVALID_ARG, "preprocess null problem");
  expect(ra_ring_fwd_workspace(nullptr) == 0 && ra_ring_bwd_workspace(nullptr) == 0 &&
             ra_ring_bwd_workspace_min(nullptr) == 0 &&
             ra_ring_bwd_kv_stationary_workspace(nullptr) == 0 && ra_ulysses_fwd_workspace(nullptr) == 0 &&
             ra_ulysses_bwd_workspace(nullptr) == 0,
         "workspace of null problem");
  // bad shard indices, null and misaligned pointers, short workspaces
  expect(ra_step_fwd(&p, 4, 0, F, F, F, Ff, Ff, nullptr) == RA_ERR_INVALID_ARG, "step_fwd shard");
  expect(ra_step_fwd(&p, 0, -1, F, F, F, Ff, Ff, nullptr) == RA_ERR_INVALID_ARG, "step_fwd kv shard");
  expect(ra_step_fwd(&p, 0, 0, nullptr, F, F, Ff, Ff, nullptr) == RA_ERR_INVALID_ARG, "step_fwd null q");
  expect(ra_step_fwd(&p, 0, 0, F, mis, F, Ff, Ff, nullptr) == RA_ERR_INVALID_ARG, "step_fwd misaligned k");
  expect(ra_merge_lse(&p, Ff, nullptr, Ff, Ff, nullptr) == RA_ERR_INVALID_ARG, "merge null lse");
  expect(ra_finalize(&p, Ff, nullptr, nullptr) == RA_ERR_INVALID_ARG, "finalize null o");
  const size_t ws = ra_ring_fwd_workspace(&p);
  expect(ws > second_acc(p.b, p.L, p.h, p.d), "ring_fwd_workspace");
  ra_problem p1 = p;   // the smallest workspace: one launch per step, no second accumulator
  p1.steps_per_launch = 1;
  const size_t ws_min = ra_ring_fwd_workspace(&p1) - second_acc(p.b, p.L, p.h, p.d);
  expect(ws_min < ws, "ring_fwd minimum workspace");
  expect(ra_ring_fwd(&p, 0, F, F, F, F, Ff, F, ws_min - 1, nullptr, nullptr) == RA_ERR_WORKSPACE, "ring_fwd workspace");
  ra_ring_timing tm;
  expect(ra_ring_fwd_timed(&p, 0, F, F, F, F, Ff, F, ws_min - 1, nullptr, nullptr, &tm) == RA_ERR_WORKSPACE,
         "ring_fwd_timed workspace");
  // the step plan: validation, then valid plans (host only) that cover every block once
  {
    int32_t blk[256], part[256], n = 0, rows = 0;
    expect(ra_fwd_step_plan(nullptr, 0, 0, 256, blk, part, 256, &n, &rows) < 0, "plan null problem");
    expect(ra_fwd_step_plan(&p, 4, 0, 256, blk, part, 256, &n, &rows) == RA_ERR_INVALID_ARG, "plan shard");
    expect(ra_fwd_step_plan(&p, 0, 0, 0, blk, part, 256, &n, &rows) == RA_ERR_INVALID_ARG, "plan n_cu");
    expect(ra_fwd_step_plan(&p, 0, 0, 256, nullptr, part, 256, &n, &rows) == RA_ERR_INVALID_ARG, "plan null block");
    ra_problem f = p;
    f.dtype = RA_F32;
    f.d = 64;
    expect(ra_fwd_step_plan(&f, 0, 0, 256, blk, part, 256, &n, &rows) == RA_ERR_UNSUPPORTED, "plan fp32");
    for (int L : {64, 1000, 2048, 4096, 4098, 8192})
      for (int causal = 0; causal < 2; ++causal)
        for (int cu : {1, 80, 256, 100000}) {
          ra_problem q = p;
          q.L = L;
          q.h = 32;
          q.n_kv = 8;
          q.causal = causal;
          q.layout = causal ? RA_LAYOUT_ZIGZAG : RA_LAYOUT_CONTIGUOUS;
          const bool ok = ra_fwd_step_plan(&q, 1, 3, cu, blk, part, 256, &n, &rows) == RA_OK;
          expect(ok && rows > 0 && n > 0 && n <= 256, "plan valid");
          if (!ok || n > 256 || rows <= 0) continue;
          const int n_qb = (L + rows - 1) / rows;
          std::vector<int> seen(n_qb, 0);
          bool cover = true;
          for (int i = 0; i < n; ++i) {
            if (blk[i] < 0 || blk[i] >= n_qb || part[i] < -1 || part[i] > 1) {
              cover = false;
              continue;
            }
            seen[blk[i]] += part[i] < 0 ? 3 : (part[i] == 0 ? 1 : 2);
          }
          for (int v : seen) cover = cover && v == 3;
          expect(cover, "plan covers every block once");
        }
  }
  expect(ra_ring_fwd_timed(&p, 0, F, F, F, F, Ff, F, ws, nullptr, nullptr, nullptr) == RA_ERR_INVALID_ARG,
         "ring_fwd_timed null timing");
  expect(ra_ring_fwd_noalloc(&p, 4, F, F, F, F, Ff, nullptr, nullptr) == RA_ERR_INVALID_ARG, "noalloc shard");
  expect(ra_ring_fwd_noalloc(&p, 0, F, F, F, nullptr, Ff, nullptr, nullptr) == RA_ERR_INVALID_ARG, "noalloc null o");
  ra_problem big = p;
  big.L = 8192;
  big.h = 32;
  big.n_kv = 8;
  big.N = 2;
  expect(ra_ring_fwd_workspace(&big) > RA_NOALLOC_SCRATCH_BYTES, "big workspace");
  expect(ra_ring_fwd_noalloc(&big, 0, F, F, F, F, Ff, nullptr, nullptr) == RA_ERR_WORKSPACE, "noalloc oversized");
  const size_t bws = ra_ring_bwd_workspace_min(&p);
  expect(ra_ring_bwd_workspace(&p) > bws, "ring_bwd workspace with the second dK, dV buffers");
  expect(ra_ring_bwd(&p, 0, F, F, F, F, F, Ff, Ff, Ff, Ff, F, bws - 1, nullptr, nullptr) == RA_ERR_WORKSPACE,
         "ring_bwd workspace");
  expect(ra_ring_bwd_timed(&p, 0, F, F, F, F, F, Ff, Ff, Ff, Ff, F, bws, nullptr, nullptr, nullptr) ==
             RA_ERR_INVALID_ARG,
         "ring_bwd_timed null timing");
  expect(ra_ring_bwd(&p, 0, F, F, F, F, nullptr, Ff, Ff, Ff, Ff, F, bws, nullptr, nullptr) == RA_ERR_INVALID_ARG,
         "ring_bwd null dout");
  const size_t sws = ra_ring_bwd_kv_stationary_workspace(&p);
  expect(ra_ring_bwd_kv_stationary(&p, 0, F, F, F, F, Ff, Ff, Ff, Ff, Ff, F, sws - 1, nullptr, nullptr) ==
             RA_ERR_WORKSPACE,
         "kv_stationary workspace");
  ra_problem ul = p;
  ul.h = 6;
  ul.n_kv = 3;
  ul.N = 4;   // heads not a multiple of N
  expect(ra_ulysses_fwd(&ul, 0, F, F, F, F, Ff, F, 1u << 30, nullptr) == RA_ERR_INVALID_ARG, "ulysses divisibility");
  expect(ra_ulysses_fwd_workspace(&ul) == 0, "ulysses workspace of invalid problem");
  ra_ulysses_timing ut;
  ra_problem u2 = p;
  u2.N = 2;
  const size_t uws = ra_ulysses_fwd_workspace(&u2);
  const size_t u_second = second_acc(u2.b, (size_t)u2.N * u2.L, u2.h / u2.N, u2.d);   // the whole-sequence problem
  expect(uws > u_second, "ulysses workspace");
  expect(ra_ulysses_fwd_timed(&u2, 0, F, F, F, F, Ff, F, uws - u_second - 1, nullptr, &ut) == RA_ERR_WORKSPACE,
         "ulysses_fwd_timed workspace");
  expect(ra_ulysses_bwd(&p, 4, F, F, F, F, F, Ff, Ff, Ff, Ff, F, 1u << 30, nullptr) == RA_ERR_INVALID_ARG,
         "ulysses_bwd group");
  // packed documents: both or neither
  ra_problem half = p;
  half.doc_begin = (const int32_t*)F;
  expect(ra_step_fwd(&half, 0, 0, F, F, F, Ff, Ff, nullptr) == RA_ERR_INVALID_ARG, "doc bounds both or neither");

  // host-only helpers on valid inputs: pairs sum to S(S+1)/2 over the shards (causal), every
  // layout; document ranges of a three-document window
  for (int layout = 0; layout < 3; ++layout) {
    ra_problem c = p;
    c.layout = layout;
    int64_t total = 0;
    for (int s = 0; s < c.N; ++s) total += ra_allowed_pairs(&c, s, -1);
    const int64_t S = (int64_t)c.N * c.L;
    expect(total == S * (S + 1) / 2, "causal pairs sum");
    const int32_t bounds[4] = {0, 100, 301, (int32_t)S};
    std::vector<int32_t> b0(c.L), e0(c.L);
    for (int s = 0; s < c.N; ++s) {
      expect(ra_document_ranges(&c, s, bounds, 3, b0.data(), e0.data()) == RA_OK, "document ranges");
      for (int t = 0; t < c.L; ++t) expect(b0[t] < e0[t] && b0[t] >= 0 && e0[t] <= S, "range order");
      const int64_t pk = ra_allowed_pairs_packed(&c, s, -1, b0.data(), e0.data());
      expect(pk > 0 && pk <= ra_allowed_pairs(&c, s, -1), "packed pairs");
    }
    const int32_t unsorted[4] = {0, 300, 200, (int32_t)S};
    expect(ra_document_ranges(&c, 0, unsorted, 3, b0.data(), e0.data()) == RA_ERR_INVALID_ARG, "unsorted bounds");
  }
  for (int s = -5; s <= 1; ++s) expect(ra_status_string(s) != nullptr && strlen(ra_status_string(s)) > 0, "status");
  printf("%ld %ld\n", n_checks, n_fail);
  return n_fail != 0;
}

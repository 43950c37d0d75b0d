// Host check of the split plans of batched forward launches (ra::plan_split_batch, linked from
// libra.so): for every shape below, the items of the plan map one to one onto the query blocks
// (a block whole, or its two parts once each), there are at most 128 of them, they launch in
// nonincreasing cost, and the plan splits where a list schedule gains and not where the blocks
// are equal and already fill the units.  Prints "<cases> <failures>".
#include <cstdio>

#include "ra_internal.h"

static int n_cases = 0, n_bad = 0;
static void expect(bool ok, const char* what, int L, int h, int n_kv, int layout, int causal, int N) {
  ++n_cases;
  if (!ok) {
    ++n_bad;
    fprintf(stderr, "FAILED: %s (L=%d h=%d n_kv=%d layout=%d causal=%d N=%d)\n", what, L, h, n_kv, layout, causal, N);
  }
}

// tiles of block qb in shard ks: the same prefix rule the kernels use
static int tiles(const ra::StepArgs& a, int rows_wg, int ks, int qb) {
  const int last = (qb + 1) * rows_wg < a.L ? (qb + 1) * rows_wg - 1 : a.L - 1;
  return (ra::kv_limit(a.causal, a.layout, a.N, a.L, a.q_shard, ks, last) + 63) / 64;
}

int main() {
  for (int N : {3, 5, 8})
    for (int L : {200, 1024, 2048, 4096})
      for (int hk : {0, 1, 2})
        for (int layout = 0; layout < 3; ++layout)
          for (int causal = 0; causal < 2; ++causal)
            for (int k_first : {1, 2}) {
              const int h = hk == 0 ? 32 : hk == 1 ? 8 : 6, n_kv = hk == 0 ? 8 : 2;
              ra::StepArgs a{};
              a.b = 1; a.L = L; a.h = h; a.n_kv = n_kv; a.d = 128; a.N = N; a.causal = causal; a.layout = layout;
              a.q_shard = N - 1; a.kv_shard = 0;
              const ra::StepGeometry g = ra::step_geometry_bf16(a);
              if (g.n_qb > ra::kSplitMaxBlocks) continue;
              ra::ShardBatch sb;
              sb.k_first = k_first;
              sb.n = N - k_first;
              const ra::SplitPlan p = ra::plan_split_batch(a, sb, g, 256);
              const ra::SplitPlan p2 = ra::plan_split_batch(a, sb, g, 256);   // from the cache
              bool same = p.split_from == p2.split_from;
              for (int w = 0; w < 4; ++w) same = same && p.order[w] == p2.order[w];
              expect(same, "cached plan differs", L, h, n_kv, layout, causal, N);
              const int items = p.split_from + 2 * (g.n_qb - p.split_from);
              expect(p.split_from >= 0 && p.split_from <= g.n_qb && items <= 128, "item count", L, h, n_kv, layout, causal, N);
              int seen[64][3] = {};
              long long prev = -1;
              bool order_ok = true;
              for (int i = 0; i < items; ++i) {
                int qb, part;
                ra::split_item(p, g.n_qb, i, qb, part);
                if (qb < 0 || qb >= g.n_qb) {
                  expect(false, "block index", L, h, n_kv, layout, causal, N);
                  continue;
                }
                const bool split = qb >= p.split_from;
                ++seen[qb][split ? part : 2];
                long long c = 0;
                for (int s = 0; s < sb.n; ++s) {
                  const int ks = ((a.q_shard - (k_first + s)) % N + N) % N;
                  const int t = tiles(a, g.rows_wg, ks, qb);
                  c += split ? (t + 1) / 2 : t;
                }
                if (prev >= 0 && c > prev + 0) order_ok = order_ok && false;
                prev = c;
              }
              for (int qb = 0; qb < g.n_qb; ++qb) {
                const bool split = qb >= p.split_from;
                const bool ok = split ? (seen[qb][0] == 1 && seen[qb][1] == 1 && seen[qb][2] == 0)
                                      : (seen[qb][2] == 1 && seen[qb][0] == 0 && seen[qb][1] == 0);
                expect(ok, "block covered once", L, h, n_kv, layout, causal, N);
              }
              expect(order_ok, "launch order nonincreasing in cost", L, h, n_kv, layout, causal, N);
              const int units = 256 / g.inner;
              // equal blocks that already fill the units: nothing to balance
              if (!causal && g.n_qb % units == 0 && g.n_qb >= units)
                expect(p.split_from == g.n_qb, "equal blocks on full units stay whole", L, h, n_kv, layout, causal, N);
              // striped causal, 32 blocks per KV head on 32 units: the heaviest twice the mean
              if (causal && layout == 1 && L == 2048 && h == 32 && N == 8 && k_first == 1)
                expect(p.split_from < g.n_qb, "imbalanced full grid splits", L, h, n_kv, layout, causal, N);
              // fewer blocks than units: some block splits
              if (g.n_qb * 2 <= units && g.n_qb >= 2)
                expect(p.split_from < g.n_qb, "idle units are used", L, h, n_kv, layout, causal, N);
            }
  // packed documents: no plan (the costs live in device memory)
  {
    ra::StepArgs a{};
    a.b = 1; a.L = 1024; a.h = 32; a.n_kv = 8; a.d = 128; a.N = 8; a.causal = 1; a.layout = 1;
    const int32_t fake = 0;
    a.doc_begin = &fake;
    a.doc_end = &fake;
    const ra::StepGeometry g = ra::step_geometry_bf16(a);
    ra::ShardBatch sb;
    sb.k_first = 1;
    sb.n = 7;
    expect(ra::plan_split_batch(a, sb, g, 256).split_from == g.n_qb, "packed documents: whole blocks", 1024, 32, 8, 1, 1, 8);
  }
  printf("%d %d\n", n_cases, n_bad);
  return n_bad ? 1 : 0;
}

// Host check: the two-piece key-limit form used by the dK/dV kernel (make_kv_form and
// kv_form_eval in ra_internal.h) equals kv_limit for every layout, shard pair and row on
// small shapes, and at the edge rows of a large one.  Prints the count of mismatches.
#include <stdio.h>
#include "ra_internal.h"

int main() {
  long bad = 0, n = 0;
  for (int causal = 0; causal < 2; ++causal)
    for (int layout = 0; layout < 3; ++layout)
      for (int N = 1; N <= 6; ++N)
        for (int L = 2; L <= 40; L += 2)
          for (int qs = 0; qs < N; ++qs)
            for (int ks = 0; ks < N; ++ks) {
              const ra::KvForm f = ra::make_kv_form(causal, layout, N, L, qs, ks);
              for (int t = 0; t < L; ++t, ++n)
                if (ra::kv_limit(causal, layout, N, L, qs, ks, t) != ra::kv_form_eval(f, t)) ++bad;
            }
  const int N = 8, L = 1 << 20;
  for (int layout = 0; layout < 3; ++layout)
    for (int qs = 0; qs < N; ++qs)
      for (int ks = 0; ks < N; ++ks) {
        const ra::KvForm f = ra::make_kv_form(1, layout, N, L, qs, ks);
        for (int t : {0, 1, 2, L / 2 - 1, L / 2, L / 2 + 1, L - 2, L - 1}) {
          ++n;
          if (ra::kv_limit(1, layout, N, L, qs, ks, t) != ra::kv_form_eval(f, t)) ++bad;
        }
      }
  printf("%ld %ld\n", n, bad);
  return bad != 0;
}

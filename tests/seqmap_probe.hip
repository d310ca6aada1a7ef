// Host-side probe of the clamped sequence layout the prefill kernels use
// (gdn_seqmap.h): reads cases from stdin -- "N T seq_len use_cu C" then
// N+1 offsets when use_cu -- and prints, per case, the N ranges and the
// N+1 chunk-slot prefixes on one line.  Built and run by
// tests/test_seqmap.py on the CPU.
#include <stdio.h>
#include <vector>

#include "../gated_deltanet_recurrence_delta_amd/csrc/gdn_seqmap.h"

int main() {
  int N, use_cu, C;
  long long T;
  int seq_len;
  while (scanf("%d %lld %d %d %d", &N, &T, &seq_len, &use_cu, &C) == 5) {
    std::vector<int32_t> cu(N + 1), beg(N), end(N), prefix(N + 1);
    if (use_cu)
      for (int i = 0; i <= N; ++i) scanf("%d", &cu[i]);
    gdn::seq_layout(use_cu ? cu.data() : nullptr, N, seq_len, T, C, beg.data(),
                    end.data(), prefix.data());
    for (int i = 0; i < N; ++i) printf("%d %d ", beg[i], end[i]);
    for (int i = 0; i <= N; ++i) printf("%d ", prefix[i]);
    // the per-sequence (unordered) bounds as well
    for (int i = 0; i < N; ++i) {
      int64_t b, e;
      gdn::seq_bounds(use_cu ? cu.data() : nullptr, i, seq_len, T, b, e);
      printf("%lld %lld ", (long long)b, (long long)e);
    }
    printf("\n");
  }
  return 0;
}

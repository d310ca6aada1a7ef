// gdn_seqmap.h -- token ranges of packed sequences read from device
// cu_seqlens, clamped so that no kernel indexes outside the sizes the host
// validated.  The host checks only what it can see (num_seqs, total_tokens
// and, when given, a host copy of the offsets); the device array itself may
// disagree with them.  Every prefill kernel therefore takes its sequence
// ranges from these functions, never from cu_seqlens directly.
//
// Well-formed offsets (cu[0] = 0, non-decreasing, cu[N] = T) pass through
// unchanged.  The functions are plain host/device code so that the same
// index logic is unit-tested on the CPU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

__host__ __device__ inline int64_t clamp_i64(int64_t x, int64_t lo,
                                             int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// [beg, end) of sequence n on its own: 0 <= beg <= end <= T.  cu == NULL
// means N equal sequences of seq_len tokens.  Ranges of different sequences
// may overlap when the offsets are malformed; each stays inside [0, T].
__host__ __device__ inline void seq_bounds(const int32_t* cu, int n,
                                           int32_t seq_len, int64_t T,
                                           int64_t& beg, int64_t& end) {
  if (cu) {
    beg = clamp_i64(cu[n], 0, T);
    end = clamp_i64(cu[n + 1], beg, T);
  } else {
    beg = clamp_i64((int64_t)n * seq_len, 0, T);
    end = clamp_i64(beg + seq_len, beg, T);
  }
}

// Disjoint, ordered ranges of all N sequences and the first chunk slot of
// each, walking the sequences in order: beg_n = clamp(cu[n], end_{n-1}, T)
// (end_{-1} = 0), end_n = clamp(cu[n+1], beg_n, T), prefix[n] = sum over
// m < n of ceil((end_m - beg_m) / C), prefix[N] the total.  Because the
// ranges are disjoint inside [0, T], the total is at most T / C + N (each
// sequence adds at most one partial chunk), the number of chunk slots the
// workspace holds.
__host__ __device__ inline void seq_layout(const int32_t* cu, int N,
                                           int32_t seq_len, int64_t T, int C,
                                           int32_t* beg, int32_t* end,
                                           int32_t* prefix) {
  int64_t prev_end = 0;
  int32_t acc = 0;
  for (int n = 0; n < N; ++n) {
    int64_t b, e;
    if (cu) {
      b = clamp_i64(cu[n], prev_end, T);
      e = clamp_i64(cu[n + 1], b, T);
    } else {
      b = clamp_i64((int64_t)n * seq_len, prev_end, T);
      e = clamp_i64(b + seq_len, b, T);
    }
    beg[n] = (int32_t)b;
    end[n] = (int32_t)e;
    prefix[n] = acc;
    acc += (int32_t)((e - b + C - 1) / C);
    prev_end = e;
  }
  prefix[N] = acc;
}

}  // namespace gdn

// Accepted prefix of a verified block from the verification's partial
// argmax keys (LongSpark paper page, Fig. 2 (a): the target verifies the
// drafted block; Table 1: accepted length tau).
//
// The partial keys of row i of sequence c are the nkeys 64-bit keys
// part[(c (B+1) + i) nkeys ..], whose unsigned maximum holds ~g_i in its low
// word (g_i = the row's argmax, lowest index on ties).  M = longest prefix
// with draft[c, i] == g_i and tau = M + 1.
#pragma once

#include "common.hpp"

namespace ls {

// The nkeys partial keys of a row are reduced by kLanesPerRow lanes of one
// wave: lane s takes keys s, s + kLanesPerRow, ..., then a max across the lanes.
constexpr int kLanesPerRow = 16;
__device__ __forceinline__ uint64_t row_key(const uint64_t* __restrict__ p, int nkeys, int sub) {
  uint64_t k = 0;
  for (int s = sub; s < nkeys; s += kLanesPerRow) k = p[s] > k ? p[s] : k;
#pragma unroll
  for (int o = kLanesPerRow / 2; o >= 1; o >>= 1) {
    const uint64_t other = shfl_xor_u64(k, o);
    k = other > k ? other : k;
  }
  return k;
}

// First half, before a workgroup barrier: the rows' argmax tokens g_i into
// g[0..B] (LDS), kLanesPerRow lanes per row over the workgroup's kThreads
// threads, and into target_tok when it is not null.  Every thread must call
// it (it holds no barrier itself).
template <int kThreads>
__device__ __forceinline__ void accept_rows(const uint64_t* __restrict__ part, int nkeys, int c,
                                            int B, int32_t* g, int32_t* __restrict__ target_tok) {
  static_assert(kThreads % kLanesPerRow == 0, "whole lane groups per row");
  const int tid = threadIdx.x, sub = tid % kLanesPerRow;
  for (int row = tid / kLanesPerRow; row <= B; row += kThreads / kLanesPerRow) {
    const uint64_t k = row_key(part + (int64_t(c) * (B + 1) + row) * nkeys, nkeys, sub);
    if (sub == 0) {
      const int32_t gi = int32_t(~uint32_t(k));
      g[row] = gi;
      if (target_tok) target_tok[int64_t(c) * (B + 1) + row] = gi;
    }
  }
}

// Second half, after the barrier, in any wave with all 64 lanes active:
// dj = draft[c, lane] for lane < B (loaded early by the caller).  One
// ballot of mismatches; bit B stands for "all B drafts accepted".  Every
// lane returns tau (1 <= tau <= B + 1).
__device__ __forceinline__ int accept_tau(const int32_t* g, int32_t dj, int B) {
  const int lane = threadIdx.x & 63;
  const uint64_t miss = __ballot(lane < B && dj != g[lane]) | (uint64_t(1) << B);
  return int(__builtin_ctzll(miss)) + 1;
}

}  // namespace ls

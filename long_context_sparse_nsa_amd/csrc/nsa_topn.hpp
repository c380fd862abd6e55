// Block-wide top-n block selection for one (query, KV group), 256 threads.
//
// Candidates are blocks 0..J with group scores S[j] >= 0 (in LDS).  Block 0
// (force_initial) and the n_local trailing blocks J, J-1, ... are always taken
// and count toward n; the other n - |F| slots go to the highest scores, equal
// scores to the lower block id; with J+1 <= n every block is taken.  Source:
// lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc), section
// "NSA: три ветви", selection paragraph (16 best blocks, always including the
// initial block and two local ones).
//
// Method: a 4-pass, 8-bit MSB-first radix select over the float bit patterns
// (non-negative floats order like their unsigned bits) finds the value T of the
// last routed pick and how many candidates equal to T are still needed; a
// block-wide prefix count over candidates in index order then takes the
// lowest-index ties.  Every step is a count, so the result is deterministic.
#pragma once
#include "nsa_device.hpp"

namespace nsa {

struct TopnSmem {
  int hist[256];
  int scratch[8];
  int pick[2];
};

// flag: LDS byte per candidate (>= J+1 entries).  Writes the ascending list to
// out[0..n) (padded with -1) and, if out2 != null, to out2 as well.
__device__ void block_topn(const float* S, int J, int n, int nloc, int finit, uint8_t* flag, TopnSmem& sm,
                           int32_t* out, int32_t* out2) {
  const int tid = threadIdx.x;
  const int ncand = J + 1;
  for (int j = tid; j < ncand; j += 256) flag[j] = (ncand <= n) ? 1 : 0;
  __syncthreads();
  if (ncand > n) {
    if (tid == 0) {
      if (finit) flag[0] = 2;
      for (int r = 0; r < nloc; ++r)
        if (J - r >= 0) flag[J - r] = 2;
    }
    // forced count: the n_local trailing blocks (clipped at 0) plus block 0 if
    // it is not already one of them
    const int nl = nloc < ncand ? nloc : ncand;
    const int nf = nl + ((finit && J - nloc + 1 > 0) ? 1 : 0);
    int rem = n - nf;
    __syncthreads();
    if (rem > 0) {
      uint32_t prefix = 0, pmask = 0;
      for (int shift = 24; shift >= 0; shift -= 8) {
        sm.hist[tid] = 0;
        __syncthreads();
        for (int j = tid; j < ncand; j += 256) {
          if (flag[j] == 0) {
            const uint32_t u = __float_as_uint(S[j]);
            if ((u & pmask) == prefix) atomicAdd(&sm.hist[(u >> shift) & 255u], 1);
          }
        }
        __syncthreads();
        if (tid < 64) {
          const int lane = tid;
          const int c0 = sm.hist[4 * lane], c1 = sm.hist[4 * lane + 1], c2 = sm.hist[4 * lane + 2],
                    c3 = sm.hist[4 * lane + 3];
          const int tot = c0 + c1 + c2 + c3;
          int suf = tot;  // inclusive suffix sum over lanes >= lane
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            int y = __shfl_down(suf, o);
            if (lane + o < 64) suf += y;
          }
          const int above = suf - tot;  // candidates in higher bins of other lanes
          const int g3 = above + c3, g2 = g3 + c2, g1 = g2 + c1, g0 = g1 + c0;
          // chosen bin b: (# >= b) >= rem and (# > b) < rem
          if (g3 >= rem && above < rem) { sm.pick[0] = 4 * lane + 3; sm.pick[1] = above; }
          if (g2 >= rem && g3 < rem)    { sm.pick[0] = 4 * lane + 2; sm.pick[1] = g3; }
          if (g1 >= rem && g2 < rem)    { sm.pick[0] = 4 * lane + 1; sm.pick[1] = g2; }
          if (g0 >= rem && g1 < rem)    { sm.pick[0] = 4 * lane + 0; sm.pick[1] = g1; }
        }
        __syncthreads();
        const uint32_t bin = (uint32_t)sm.pick[0];
        rem -= sm.pick[1];
        prefix |= bin << shift;
        pmask |= 255u << shift;
        __syncthreads();
      }
      // take every candidate above the threshold, and the `rem` lowest-index ties
      const int R = (ncand + 255) / 256;
      const int j0 = tid * R, j1 = min(j0 + R, ncand);
      int eq = 0;
      for (int j = j0; j < j1; ++j)
        if (flag[j] == 0 && __float_as_uint(S[j]) == prefix) ++eq;
      int total;
      int base = block_scan_256(eq, sm.scratch, &total);
      for (int j = j0; j < j1; ++j) {
        if (flag[j] != 0) continue;
        const uint32_t u = __float_as_uint(S[j]);
        if (u > prefix) flag[j] = 1;
        else if (u == prefix) {
          if (base < rem) flag[j] = 1;
          ++base;
        }
      }
    }
    __syncthreads();
  }
  // ascending compaction of the taken blocks
  const int R = (ncand + 255) / 256;
  const int j0 = tid * R, j1 = min(j0 + R, ncand);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += flag[j] != 0;
  int total;
  int pos = block_scan_256(cnt, sm.scratch, &total);
  for (int j = j0; j < j1; ++j) {
    if (flag[j] != 0 && pos < n) {
      out[pos] = j;
      if (out2) out2[pos] = j;
      ++pos;
    }
  }
  for (int r = total + tid; r < n; r += 256) {
    out[r] = -1;
    if (out2) out2[r] = -1;
  }
}

}  // namespace nsa

// Block-wide top-n block selection for one (query, KV group), NT threads.
//
// Candidates are blocks 0..J with group scores S[j] >= 0 (in LDS).  Block 0
// (force_initial) and the n_local trailing blocks J, J-1, ... are always taken
// and count toward n; the other n - |F| slots go to the highest scores, equal
// scores to the lower block id; with J+1 <= n every block is taken.  Source:
// lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc), section
// "NSA: три ветви", selection paragraph (16 best blocks, always including the
// initial block and two local ones).
//
// Method: every candidate gets the unique 64-bit key
//   (bits of S[j]) << 32 | (0xFFFFFFFF - j)
// (non-negative floats order like their bit patterns, and the low word prefers
// the lower block id on equal scores), so "best" is simply the largest key.
// Each wave extracts the n_r largest keys of its share of the candidates by n_r
// rounds of a wave-wide max (DPP row operations, no LDS atomics); wave 0 then extracts
// the n_r largest of the waves' winners the same way.  The final ascending list
// is formed by lane-parallel ranking.  Fully deterministic.
#pragma once
#include "nsa_device.hpp"

namespace nsa {

constexpr int kTopnMaxRouted = 64;

struct TopnSmem {
  uint64_t wbest[16 * kTopnMaxRouted];  // per-wave winners
};

// Wave-wide maximum of an unsigned value with DPP row shifts and row broadcasts
// (lane 63 accumulates the maximum of all lanes), then broadcast from lane 63.
// Lanes whose DPP source is out of range read 0, the identity of the maximum.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false));  // row_shr:1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false));  // row_shr:2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false));  // row_shr:4
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false));  // row_shr:8
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Extract the `rounds` (<= 64) largest of the keys held in k[0..K) over the
// wave; returns the r-th winner in lane r (0 when none is left).  A key is
// compared by its high word (score bits) and then its low word (inverted id).
template <int K>
__device__ __forceinline__ uint64_t wave_extract(uint64_t (&k)[K], int rounds) {
  const int lane = threadIdx.x & 63;
  uint64_t mine_win = 0;
  for (int r = 0; r < rounds; ++r) {
    uint64_t mine = k[0];
#pragma unroll
    for (int q = 1; q < K; ++q) mine = k[q] > mine ? k[q] : mine;
    const uint32_t hi = (uint32_t)(mine >> 32), lo = (uint32_t)mine;
    const uint32_t Mh = wave_max_u32(hi);
    // the index word only needs a second reduction when several lanes hold the
    // top score; otherwise the single holder's word is read directly
    const uint64_t holders = __ballot(hi == Mh);
    const uint32_t Ml = __popcll(holders) == 1
                            ? (uint32_t)__builtin_amdgcn_readlane((int)lo, (int)__ffsll((unsigned long long)holders) - 1)
                            : wave_max_u32(hi == Mh ? lo : 0u);
    const uint64_t best = ((uint64_t)Mh << 32) | Ml;
    if (best == 0) break;  // nothing left anywhere in the wave (uniform)
#pragma unroll
    for (int q = 0; q < K; ++q)
      if (k[q] == best) k[q] = 0;  // keys are unique: exactly one lane holds it
    if (lane == r) mine_win = best;
  }
  return mine_win;
}

// Candidates with key 0 are excluded.  MAXC bounds the candidates per lane:
// ceil(ceil((J+1)/(NT/64)) / 64) <= MAXC.
template <int NT, int MAXC>
__device__ void block_topn(const float* S, int J, int n, int nloc, int finit, TopnSmem& sm, int32_t* out,
                           int32_t* out2) {
  static_assert(NT % 64 == 0 && NT <= 1024, "block size");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ncand = J + 1;
  if (ncand <= n) {  // every candidate is taken
    for (int r = tid; r < n; r += NT) {
      const int v = r < ncand ? r : -1;
      out[r] = v;
      if (out2) out2[r] = v;
    }
    return;
  }
  const int lo_local = J - nloc + 1 > 0 ? J - nloc + 1 : 0;  // local blocks are [lo_local, J]
  const bool f0 = finit && lo_local > 0;                      // block 0 forced separately
  const int nf = (J - lo_local + 1) + (f0 ? 1 : 0);
  const int nr = n - nf;                                      // routed picks (uniform)
  if (nr > 0) {
    // ---- per-wave extraction over a contiguous share of the candidates; the
    // number of key slots per lane is picked from the actual candidate count
    const int per_wave = (ncand + NW - 1) / NW;
    const int c0 = wave * per_wave;
    auto key = [&](int q) -> uint64_t {
      const int j = c0 + lane + 64 * q;
      const bool ok = q * 64 + lane < per_wave && j < lo_local && !(f0 && j == 0);
      return ok ? ((uint64_t)__float_as_uint(S[j]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j) : 0ull;
    };
    uint64_t w;
    if (per_wave <= 128 || MAXC <= 2) {
      uint64_t k[2] = {key(0), key(1)};
      w = wave_extract<2>(k, nr);
    } else if (per_wave <= 512 || MAXC <= 8) {
      uint64_t k[8 < MAXC ? 8 : MAXC];
#pragma unroll
      for (int q = 0; q < (8 < MAXC ? 8 : MAXC); ++q) k[q] = key(q);
      w = wave_extract<(8 < MAXC ? 8 : MAXC)>(k, nr);
    } else {
      uint64_t k[MAXC];
#pragma unroll
      for (int q = 0; q < MAXC; ++q) k[q] = key(q);
      w = wave_extract<MAXC>(k, nr);
    }
    sm.wbest[wave * kTopnMaxRouted + lane] = w;
    __syncthreads();
  }
  if (wave == 0) {
    // ---- wave 0: merge the waves' winners, add the forced blocks, rank
    int v = INT32_MAX;
    if (nr > 0) {
      uint64_t k2[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) k2[w] = lane < nr ? sm.wbest[w * kTopnMaxRouted + lane] : 0ull;
      const uint64_t best = wave_extract<NW>(k2, nr);
      if (lane < nr) v = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
    }
    if (lane >= nr && lane < n) {
      const int i = lane - nr;  // forced block i
      v = f0 ? (i == 0 ? 0 : lo_local + i - 1) : lo_local + i;
    }
    int rank = 0;
    for (int q = 0; q < n; ++q) rank += __builtin_amdgcn_readlane(v, q) < v;
    if (lane < n) {
      out[rank] = v;
      if (out2) out2[rank] = v;
    }
  }
}

// Single-wave variant for one (query, KV group): candidates 0..J with scores
// S[j] >= 0, at most 64 * MAXC of them.  Writes the n ids ascending to out
// (-1 fills the tail when fewer than n candidates exist).  No LDS, no barrier.
template <int MAXC>
__device__ void wave_topn(const float* S, int J, int n, int nloc, int finit, int32_t* out) {
  const int lane = threadIdx.x & 63;
  const int ncand = J + 1;
  if (ncand <= n) {
    for (int r = lane; r < n; r += 64) out[r] = r < ncand ? r : -1;
    return;
  }
  const int lo_local = J - nloc + 1 > 0 ? J - nloc + 1 : 0;
  const bool f0 = finit && lo_local > 0;
  const int nf = (J - lo_local + 1) + (f0 ? 1 : 0);
  const int nr = n - nf;
  int v = INT32_MAX;
  if (nr > 0) {
    uint64_t k[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int j = lane + 64 * c;
      const bool ok = j < lo_local && !(f0 && j == 0);
      k[c] = ok ? ((uint64_t)__float_as_uint(S[j]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j) : 0ull;
    }
    const uint64_t best = wave_extract<MAXC>(k, nr);
    if (lane < nr) v = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
  }
  if (lane >= nr && lane < n) {
    const int i = lane - nr;
    v = f0 ? (i == 0 ? 0 : lo_local + i - 1) : lo_local + i;
  }
  int rank = 0;
  for (int q = 0; q < n; ++q) rank += __builtin_amdgcn_readlane(v, q) < v;
  if (lane < n) out[rank] = v;
}

}  // namespace nsa

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
__device__ __forceinline__ void block_topn(const float* S, int J, int n, int nloc, int finit, TopnSmem& sm, int32_t* out,
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
    lds_barrier();
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

// ---------------------------------------------------------------------------
// Rank-based block top-n (the fast path for up to 8 candidates per thread and
// nr <= 64 routed picks).  Keys as above (unique, 0 = no candidate).
//  1. every lane takes the maximum of its keys; the nr-th largest lane maximum
//     of the wave is a threshold tau: every key among the wave's nr largest is
//     >= tau (otherwise nr lane maxima would exceed it), and at most K*nr keys
//     are >= tau (they lie in the <= nr lanes whose maximum is >= tau);
//  2. the survivors (>= tau) are compacted in LDS and each is ranked by
//     counting the survivors above it (broadcast LDS reads); ranks < nr are the
//     wave's winners, stored in rank order;
//  3. one wave ranks the waves' winners the same way.
// Every step is exact and deterministic.
template <int NW>
struct __attribute__((aligned(16))) TopnFastSmem {
  __attribute__((aligned(16))) uint64_t lmax[NW][64];
  __attribute__((aligned(16))) uint64_t surv[NW][144];  // <= 128 survivors, zero padded to a multiple of 16
  __attribute__((aligned(16))) uint64_t best[NW * kTopnMaxRouted + 16];  // the waves' winners: wave w at [w*nr, (w+1)*nr)
  __attribute__((aligned(16))) int ids[64];
  int fail;
};

typedef unsigned long long u64x2_t __attribute__((ext_vector_type(2)));

// Number of keys greater than x among v[0 .. 16*nb) (16-byte aligned, padded
// with zeros, which never count).  Each batch issues eight 16-byte broadcast
// reads at once, so the LDS latency is paid once per 16 keys.
__device__ __forceinline__ int count_greater(const uint64_t* v, int nb, uint64_t x) {
  int c = 0;
  for (int b = 0; b < nb; ++b) {
    u64x2_t a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const u64x2_t*>(v + 16 * b + 2 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) c += (a[i].x > x ? 1 : 0) + (a[i].y > x ? 1 : 0);
  }
  return c;
}

__device__ __forceinline__ void wave_lds_sync() {  // LDS writes of this wave visible to all its lanes
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Ranks the T (<= 64 * SL) keys in surv (zero padded to a multiple of 16) and
// writes those with rank < nr to dst[rank]; dst[T .. nr) are set to 0.
template <int SL = 2>
__device__ __forceinline__ void rank_into(const uint64_t* surv, int T, int nr, uint64_t* dst) {
  const int lane = threadIdx.x & 63;
  const int nb = (T + 15) >> 4;
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    const int idx = lane + 64 * s;
    if (idx < T) {
      const uint64_t x = surv[idx];
      const int rk = count_greater(surv, nb, x);
      if (rk < nr) dst[rk] = x;
    } else if (idx < nr) {
      dst[idx] = 0ull;
    }
  }
}

// Zero entries [T, roundup16(T)) of a list of at most 128 keys.
__device__ __forceinline__ void pad16(uint64_t* v, int T) {
  const int lane = threadIdx.x & 63;
  const int end = (T + 15) & ~15;
  if (T + lane < end) v[T + lane] = 0ull;
}

// Returns false (for the whole wave) when more than 128 keys survive.
template <int K>
__device__ __forceinline__ bool wave_rank_topn(const uint64_t (&k)[K], int nr, uint64_t* lmax, uint64_t* surv,
                                               uint64_t* dst) {
  const int lane = threadIdx.x & 63;
  uint64_t km = k[0];
#pragma unroll
  for (int c = 1; c < K; ++c) km = k[c] > km ? k[c] : km;
  lmax[lane] = km;
  wave_lds_sync();
  const int r = count_greater(lmax, 4, km);
  const uint64_t at = __ballot(km != 0ull && r == nr - 1);
  uint64_t tau = 0ull;
  if (at != 0ull) {
    const int src = __ffsll((unsigned long long)at) - 1;
    tau = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(km >> 32), src) << 32) |
          (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)km, src);
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int c = 0; c < K; ++c) {
    const bool sv = k[c] != 0ull && k[c] >= tau;
    const uint64_t m = __ballot(sv);
    const int pos = base + __popcll(m & lt);
    if (sv && pos < 128) surv[pos] = k[c];
    base += __popcll(m);
  }
  if (base > 128) return false;
  pad16(surv, base);
  wave_lds_sync();
  rank_into(surv, base, nr, dst);
  wave_lds_sync();
  return true;
}

// Block top-n with the rank-based fast path; falls back to block_topn (which
// reads S again) when a wave has more than 128 survivors, more than K
// candidates per thread are needed, or nr > 64.
template <int NT, int K, int MAXC>
__device__ __forceinline__ void block_topn_fast(const float* S, int J, int n, int nloc, int finit, TopnFastSmem<NT / 64>& fs,
                                TopnSmem& sm, int32_t* out, int32_t* out2) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ncand = J + 1;
  const int lo_local = J - nloc + 1 > 0 ? J - nloc + 1 : 0;
  const bool f0 = finit && lo_local > 0;
  const int nf = (J - lo_local + 1) + (f0 ? 1 : 0);
  const int nr = n - nf;
  if (ncand <= n || nr <= 0 || nr > kTopnMaxRouted || ncand > NT * K) {
    block_topn<NT, MAXC>(S, J, n, nloc, finit, sm, out, out2);
    return;
  }
  uint64_t k[K];
#pragma unroll
  for (int c = 0; c < K; ++c) {
    const int j = tid + NT * c;
    const bool ok = j < lo_local && !(f0 && j == 0);
    k[c] = ok ? ((uint64_t)__float_as_uint(S[j]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j) : 0ull;
  }
  if (tid == 0) fs.fail = 0;
  lds_barrier();
  const bool ok = wave_rank_topn<K>(k, nr, fs.lmax[wave], fs.surv[wave], fs.best + wave * nr);
  if (!ok && lane == 0) fs.fail = 1;
  lds_barrier();
  if (fs.fail) {
    lds_barrier();
    block_topn<NT, MAXC>(S, J, n, nloc, finit, sm, out, out2);
    return;
  }
  if (wave == 0) {
    // the waves' winners: NW contiguous lists of nr (zero padded); rank them together
    const int T = NW * nr;
    pad16(fs.best, T);
    wave_lds_sync();
    uint64_t* win = fs.surv[0];
    if (T <= 128) rank_into<2>(fs.best, T, nr, win);
    else rank_into<4>(fs.best, T, nr, win);
    wave_lds_sync();
    int v = INT32_MAX;
    if (lane < nr) v = (int)(0xFFFFFFFFu - (uint32_t)(win[lane] & 0xFFFFFFFFull));
    if (lane >= nr && lane < n) {
      const int i = lane - nr;  // forced block i
      v = f0 ? (i == 0 ? 0 : lo_local + i - 1) : lo_local + i;
    }
    // ascending order: the rank of each id among the n (distinct) ids
    fs.ids[lane] = v;
    wave_lds_sync();
    int rank = 0;
    for (int q0 = 0; q0 < n; q0 += 16) {
      int4 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const int4*>(fs.ids + q0 + 4 * i);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rank += (a[i].x < v) + (a[i].y < v) + (a[i].z < v) + (a[i].w < v);
    }
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
__device__ __forceinline__ void wave_topn(const float* S, int J, int n, int nloc, int finit, int32_t* out) {
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

// Wave-wide minimum of an unsigned value (DPP row shifts and broadcasts as in
// wave_max_u32, on the complement).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return 0xFFFFFFFFu - wave_max_u32(0xFFFFFFFFu - x); }

// Top-n for one (query, KV group) by one wave, without sorting networks:
// candidates 0..J (J + 1 <= 16 * K) with group scores S[j] >= 0 in LDS, lane l
// holding j = 256*c + 4*l + e (c < K/4, e < 4).
//  1. threshold: with v_0 >= v_1 >= ... the lanes' maximum scores (32-bit, ties
//     allowed), tau = v_{nr-1} is found as the minimum over the lanes whose
//     maximum is exceeded by fewer than nr others (counted with broadcast LDS
//     reads); every score among the nr largest is >= tau, and only the nr
//     lanes whose maximum is >= tau can hold such scores;
//  2. the survivors (score >= tau, usually about nr + a few) are compacted by
//     ballot into LDS as 64-bit keys (score bits << 32 | ~j, so equal scores
//     prefer the lower id) and ranked exactly by counting larger keys;
//  3. the routed picks and the forced blocks are put in ascending order by
//     counting smaller ids.
// Writes the ids ascending to items[0 .. count) (LDS) and, when sel_out is not
// null, to sel_out[0 .. n) padded with -1; returns count (wave-uniform).
// scratch: LDS of at least 416 64-bit words.  Exact and deterministic; more
// than 256 survivors (possible only with many equal scores) take the one-by-one
// extraction instead.
template <int K>
__device__ __forceinline__ int wave_topn_fast(const float* S, int J, int n, int nloc, int finit, uint64_t* scratch,
                                              int* items, int32_t* sel_out) {
  static_assert(K % 4 == 0 && K <= 32, "candidates per lane");
  const int lane = threadIdx.x & 63;
  const int ncand = J + 1;
  if (ncand <= n) {
    for (int r = lane; r < n; r += 64) {
      if (r < ncand) items[r] = r;
      if (sel_out) sel_out[r] = r < ncand ? r : -1;
    }
    return ncand;
  }
  const int lo_local = J - nloc + 1 > 0 ? J - nloc + 1 : 0;  // local blocks are [lo_local, J]
  const bool f0 = finit && lo_local > 0;
  const int nf = (J - lo_local + 1) + (f0 ? 1 : 0);
  const int nr = n - nf;
  uint32_t* lmax = reinterpret_cast<uint32_t*>(scratch);      // 64 words (as 32 64-bit words)
  uint64_t* surv = scratch + 32;                              // up to 256 keys + 16 of padding
  uint64_t* win = scratch + 32 + 272;                         // nr <= 64 winners
  int* ids = reinterpret_cast<int*>(scratch + 32 + 272 + 64);  // n <= 64 ids (32 words)
  int myid = INT32_MAX;
  if (nr > 0) {
    // ---- scores as 32-bit keys: bits + 1 (0 = not a candidate)
    uint32_t k[K];
#pragma unroll
    for (int c = 0; c < K / 4; ++c) {
      const int j0 = 256 * c + 4 * lane;
      float4 s4 = {0.f, 0.f, 0.f, 0.f};
      if (j0 < ncand) s4 = *reinterpret_cast<const float4*>(S + j0);  // S is padded to a multiple of 4
      const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + e;
        const bool ok = j < lo_local && !(f0 && j == 0);
        k[4 * c + e] = ok ? __float_as_uint(sv[e]) + 1u : 0u;
      }
    }
    // ---- 1. threshold
    uint32_t km = k[0];
#pragma unroll
    for (int c = 1; c < K; ++c) km = max(km, k[c]);
    lmax[lane] = km;
    wave_lds_sync();
    int above = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint4 a = reinterpret_cast<const uint4*>(lmax)[q];
      above += (a.x > km) + (a.y > km) + (a.z > km) + (a.w > km);
    }
    uint32_t tau = wave_min_u32(above < nr ? km : 0xFFFFFFFFu);
    if (tau == 0u) tau = 1u;  // fewer than nr lanes hold candidates: all of them survive
    // ---- 2. survivors, compacted by ballot, then ranked exactly
    const uint64_t below = (1ull << lane) - 1ull;
    int T = 0;
#pragma unroll
    for (int c = 0; c < K; ++c) {
      const bool sv = k[c] >= tau;
      const uint64_t m = __ballot(sv);
      const int pos = T + __popcll(m & below);
      if (sv && pos < 256) {
        const uint32_t j = (uint32_t)(256 * (c >> 2) + 4 * lane + (c & 3));
        surv[pos] = ((uint64_t)(k[c] - 1u) << 32) | (uint64_t)(0xFFFFFFFFu - j);
      }
      T += __popcll(m);
    }
    if (T <= 256) {
      pad16(surv, T);
      wave_lds_sync();
      rank_into<4>(surv, T, nr, win);
      wave_lds_sync();
      if (lane < nr) myid = (int)(0xFFFFFFFFu - (uint32_t)win[lane]);
    } else {  // many equal scores: extract the maxima one by one from 64-bit keys
      uint64_t kk[K];
#pragma unroll
      for (int c = 0; c < K; ++c) {
        const uint32_t j = (uint32_t)(256 * (c >> 2) + 4 * lane + (c & 3));
        kk[c] = k[c] ? ((uint64_t)(k[c] - 1u) << 32) | (uint64_t)(0xFFFFFFFFu - j) : 0ull;
      }
      const uint64_t w = wave_extract<K>(kk, nr);
      if (lane < nr) myid = (int)(0xFFFFFFFFu - (uint32_t)w);
    }
  }
  const int nrp = nr > 0 ? nr : 0;
  if (lane >= nrp && lane < nrp + nf) {
    const int i = lane - nrp;  // forced block i
    myid = f0 ? (i == 0 ? 0 : lo_local + i - 1) : lo_local + i;
  }
  // ---- 3. ascending order: the rank of each id among the cnt (distinct) ids
  const int cnt = nrp + nf < n ? nrp + nf : n;
  ids[lane] = myid;
  wave_lds_sync();
  int rk = 0;
  for (int q0 = 0; q0 < cnt; q0 += 16) {
    int4 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = reinterpret_cast<const int4*>(ids)[q0 / 4 + i];
#pragma unroll
    for (int i = 0; i < 4; ++i) rk += (a[i].x < myid) + (a[i].y < myid) + (a[i].z < myid) + (a[i].w < myid);
  }
  if (lane < cnt) {
    items[rk] = myid;
    if (sel_out) sel_out[rk] = myid;
  }
  if (sel_out && lane >= cnt && lane < n) sel_out[lane] = -1;
  return cnt;
}

}  // namespace nsa

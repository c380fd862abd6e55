// DeepSeek Sparse Attention (DSA) decode step on gfx950: lightning indexer,
// token top-k, and MQA attention over the selected tokens' shared latents.
//
// Source: lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc),
// section "DSA: молниеносный индексатор": the indexer scores every past token
// s of query t as I = sum_j w_j * ReLU(qI_j . kI_s) with a few small FP8 heads
// and no softmax; the 2048 tokens with the largest I are kept per query; MLA
// then runs in MQA mode over them (all heads share one contiguous 576-number
// latent per token).  The practice spec of that lesson fixes the selection
// rules: only keys j <= i, and all of them when there are fewer than k.
//
// Four launches per step (one query per sequence, t = seq_lens[b] - 1):
//  1. dsa_index_kernel   about one workgroup per compute unit; each wave scores
//     16-token tiles with v_mfma_f32_16x16x32_fp8_fp8 (indexer heads x tokens),
//     ReLU, the weighted head sum, and writes fp32 scores.  Tile loads run a
//     batch of eight tiles ahead of the compute.
//  2. dsa_topk_kernel    exact top-k by radix select on order-preserving integer
//     keys of the scores, one workgroup per 4096-score chunk: a sampled
//     histogram bounds the k-th key between two bins, each chunk marks its keys
//     above the bound and lists those within it, and the last workgroup of the
//     sequence finds the k-th key among the listed ones (or, when the bound did
//     not hold, over every score), takes ties at it from the lowest positions
//     and writes the positions ascending.
//  3. dsa_attn_kernel    workgroup = (sequence, 64 heads -- 32 when the head
//     count is not a multiple of 64 --, token split of at most 128 tokens); the
//     split's 32-token tiles of latents are all gathered into LDS at once with
//     the direct global->LDS copy, and every wave reads each tile for its own 16
//     heads: logits of every tile first (exact maximum per head), then the
//     probabilities and the values, with no exchange between waves; the tile's
//     latents are gathered once per 64 heads.
//  4. dsa_combine_kernel merges the token-split partials exactly and writes bf16
//     (one wave per (sequence, head), 16-byte loads of 8 channels per lane).
#include <hip/hip_runtime.h>

#include "nsa_device.hpp"
#include "nsa_internal.hpp"
#include "nsa_stage.hpp"
#include "nsa_tiles.hpp"

namespace nsa {

namespace {

// Per (head, split) partial: m and l (fp32), 6 floats of padding, then the split's
// output divided by its own l as 512 fp16 values (weighted averages of bf16
// values: fp16's 11-bit significand adds about 2^-12 relative error, well below
// the bf16 rounding of the result, at half the bytes of fp32).
constexpr int kPartStride = 8 + 512 / 2;  // floats
constexpr int kPartOut = 8;

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
}
__device__ __forceinline__ f32x2_t unpack_f16x2(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
}

__device__ __forceinline__ f32x4_t mfma_fp8(long a, long b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// 1. indexer scores
template <int HI, int DI>
__global__ __launch_bounds__(256) void dsa_index_kernel(DsaParams p) {
  constexpr int RT = HI / 16, KS = DI / 32, BPL = DI / 4, LV = BPL / 16, NT = 8;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int b = blockIdx.x / p.nseg, sg = blockIdx.x - b * p.nseg;
  if (sg == 0 && tid < 4) p.cnt[4 * b + tid] = 0u;  // the top-k launch's arrival counters
  const int64_t L = p.seq_lens[b];
  const int64_t n = L < p.cap ? L : p.cap;
  const int64_t s0 = (int64_t)sg * p.seg;
  if (s0 >= n) return;
  const int64_t s1 = s0 + p.seg < n ? s0 + p.seg : n;

  // A operand: head 16*rt + lr, k-step ks holds bytes lg*BPL + 8*ks .. +8 (the
  // B operand pairs the same bytes of each token row)
  long qa[RT][KS];
  float wv[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const uint8_t* qrow = p.qi + ((size_t)b * HI + 16 * rt + lr) * DI + lg * BPL;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[rt][ks] = *reinterpret_cast<const long*>(qrow + 8 * ks);
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[rt][i] = p.wi[(size_t)b * HI + 16 * rt + 4 * lg + i];
  }
  const uint8_t* kb = p.ki + (size_t)b * p.cap * DI + lg * BPL;
  float* sc = p.scores + (size_t)b * p.sstride;
  const int ntile = (int)((s1 - s0 + 15) / 16);
  const int nvw = ntile > wave ? (ntile - wave + 3) / 4 : 0;  // this wave's tiles: wave, wave+4, ...

  u32x4_t ba[NT][LV], bb[NT][LV];
  auto load = [&](u32x4_t (&buf)[NT][LV], int v0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      int64_t tok = s0 + 16 * (int64_t)(wave + 4 * (v0 + t)) + lr;
      tok = tok < s1 ? tok : s1 - 1;  // past the end: a valid row, never stored
      const uint8_t* src = kb + tok * DI;
#pragma unroll
      for (int l = 0; l < LV; ++l) buf[t][l] = *reinterpret_cast<const u32x4_t*>(src + 16 * l);
    }
  };
  auto compute = [&](const u32x4_t (&buf)[NT][LV], int v0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (v0 + t >= nvw) break;  // wave-uniform
      f32x4_t acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t& x = buf[t][ks >> 1];
        const long kv = (long)(((uint64_t)x[2 * (ks & 1) + 1] << 32) | x[2 * (ks & 1)]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma_fp8(qa[rt][ks], kv, acc[rt]);
      }
      float part = 0.f;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) part = fmaf(wv[rt][i], fmaxf(acc[rt][i], 0.f), part);
      const float s = sum_over_groups_swap(part);  // all heads, token lr of the tile
      const int64_t tok = s0 + 16 * (int64_t)(wave + 4 * (v0 + t)) + lr;
      if (lg == 0 && tok < s1) sc[tok] = s;
    }
  };
  load(ba, 0);
  for (int v0 = 0; v0 < nvw; v0 += 2 * NT) {
    load(bb, v0 + NT);
    compute(ba, v0);
    load(ba, v0 + 2 * NT);
    compute(bb, v0 + NT);
  }
  wait_vmem();  // the last prefetch is never used
}

// ---------------------------------------------------------------------------
// 2. exact top-k of the scores: 4096-score chunks, one 256-thread workgroup each
//
// Radix select on order-preserving integer keys (a larger float gives a larger
// key), in three steps that keep every workgroup's work per key small:
//  - bound: every workgroup of a sequence builds the same histogram of the first
//    digit (top 13 bits) over a fixed sample of the sequence's scores (16
//    evenly spaced runs of 256) and takes the bins of two sample ranks around
//    the expected rank of the k-th key, a margin of four standard deviations
//    and 16 apart: lo is the lower bin's first key, hi the upper bin's last;
//  - chunk pass: each workgroup marks its keys above hi in the position bitmap,
//    copies its keys in [lo, hi] with their positions to its slice of the
//    candidate list, and stores both counts (agent-scope stores);
//  - the last workgroup of the sequence (an arrival counter, zeroed by the
//    indexer launch) checks that the bound held -- fewer than k keys above hi,
//    at least k above or at lo, and the candidates fit in LDS -- and finds the
//    k-th key among the candidates (digits of the key relative to lo, 11 bits
//    at a time); keys above it are taken, and the rest from the keys equal to
//    it, lowest positions first; the positions are written ascending from the
//    bitmap.  When the bound did not hold, that workgroup runs the select over
//    every score of the sequence instead (three digit histograms, 13, 13 and
//    6 bits), which is slower but exact.
// Coherence across XCDs as in the decode selection: agent-scope atomic stores
// and loads, the writers wait for their stores before the arrival increment.

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkPer = kDsaChunk / kTopkThreads;         // keys per thread in a chunk (4)
constexpr int kTopkRun = 256;                              // sample run length
constexpr int kTopkRuns = 16;                              // sample runs
constexpr int kTopkSamples = kTopkRun * kTopkRuns / kTopkThreads;  // sampled keys per thread (4)
constexpr int kTopkCandLds = 4096;                         // candidates the last workgroup holds
constexpr int kTopkWpt = kDsaMaxLen / 32 / kTopkThreads;   // bitmap words per thread at the end

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // larger float -> larger key
}

// Every score's key is raised to at least 2^19 (only NaNs with the sign bit set
// have smaller keys; they tie there), so bin 0 holds no key and key 0 can stand
// for "no key".
__device__ __forceinline__ uint32_t score_key(float f) { return max(order_key(f), 1u << 19); }

// Exclusive prefix over the workgroup's threads; *total gets the sum.  T is
// int, or uint32_t for sums taken modulo 2^32 (packed fields).
template <class T>
__device__ __forceinline__ T scan_wg(T v, T* s_w, T* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  T base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const T s = s_w[w];
    base += w < wave ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// In the NB-bin histogram h, the bins holding the ra-th and rb-th largest
// keys (ranks from 1) to s_out[0] and s_out[2], the counts of keys in higher
// bins to s_out[1] and s_out[3].  With `sampled` the ranks come from the
// histogram's total instead: the expected rank of the k-th key of n among the
// sample, minus and plus four standard deviations and 16, clamped to
// [1, total]; s_out[4] gets the total.  Thread t sums bins [kPer*(NT-1-t),
// +kPer) (thread 0 the highest) from a rotated start, so that the lanes of a
// wave read different LDS banks; only threads whose bins hold a rank walk them.
template <int NB = kDsaBins>
__device__ __forceinline__ void find_bins(const uint32_t* h, int ra, int rb, bool sampled, int k, int n, int* s_w,
                                          int* s_out) {
  constexpr int kPer = NB / kTopkThreads;
  const int tid = (int)threadIdx.x, g0 = kPer * (kTopkThreads - 1 - tid);
  int sum = 0;
  for (int e = 0; e < kPer; ++e) sum += (int)h[g0 + ((e + tid) & (kPer - 1))];
  int total;
  const int above = scan_wg(sum, s_w, &total);
  if (sampled) {  // a heuristic bound (the result does not depend on it)
    const float kp = (float)k * (float)total * __builtin_amdgcn_rcpf((float)n);
    const float d = 4.f * __builtin_amdgcn_sqrtf(kp) + 16.f;
    ra = max(1, (int)(kp - d));
    rb = min(total, (int)(kp + d) + 1);
    if (tid == 0) s_out[4] = total;
  }
  for (int j = 0; j < 2; ++j) {
    const int need = j == 0 ? ra : rb;
    if (above < need && above + sum >= need) {  // one thread: its bins read at once, then walked
      uint32_t hv[kPer];
#pragma unroll
      for (int e = 0; e < kPer; ++e) hv[e] = h[g0 + e];
      int acc = above, bin = g0, acc_at = above;
      bool found = false;
#pragma unroll
      for (int e = kPer - 1; e >= 0; --e) {
        if (!found && acc + (int)hv[e] >= need) {
          found = true;
          bin = g0 + e;
          acc_at = acc;
        }
        acc += (int)hv[e];
      }
      s_out[2 * j] = bin;
      s_out[2 * j + 1] = acc_at;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void zero_hist(uint32_t* h) {
  for (int i = threadIdx.x; i < kDsaBins; i += kTopkThreads) h[i] = 0u;
}

__global__ __launch_bounds__(kTopkThreads) void dsa_topk_kernel(DsaParams p) {
  __shared__ uint32_t h[kDsaBins];
  __shared__ uint32_t s_sb[kDsaMaxLen / 32], s_tb[kDsaMaxLen / 32];  // selected / tied positions
  __shared__ uint64_t s_cand[kTopkCandLds];                          // (key << 32) | position
  __shared__ int s_w[kTopkWaves];
  __shared__ uint32_t s_wu[kTopkWaves];
  __shared__ int s_out[5];
  __shared__ uint32_t s_coff[kDsaMaxLen / kDsaChunk + 1];
  __shared__ uint32_t s_small[64];  // the boundary bin's keys, once at most 64
  __shared__ int s_last, s_nb;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / p.nchunk, ch = blockIdx.x - b * p.nchunk;
  clk_stamp(p.clk, 0);
  const int64_t L = p.seq_lens[b];
  const int n = (int)(L < p.cap ? L : p.cap);
  const int k = p.topk;
  int32_t* out = p.sel + (size_t)b * k;
  if (n <= k) {  // every past token
    if (ch == 0)
      for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* sc = p.scores + (size_t)b * p.sstride;
  const int c0 = ch * kDsaChunk;
  uint32_t* bits = p.bits + (size_t)b * p.nchunk * (kDsaChunk / 32);
  uint64_t* cand = p.cand + (size_t)b * p.nchunk * kDsaChunk;  // chunk ch: entries [c0, c0 + its count)
  uint32_t* counts = p.cnt + (size_t)p.B * 4 + (size_t)b * p.nchunk * 2;  // per chunk: above, candidates
  uint32_t* arrive = p.cnt + 4 * b;

  // ---- loads, all issued at once: the sample (run r starts at r*n/16; sample
  // s = t + NT*j is score s % 256 of run s / 256) and this chunk (key (i, e) is
  // position c0 + 4*(t + NT*i) + e: 1 KB of consecutive scores per wave and load)
  float sv[kTopkSamples];
#pragma unroll
  for (int j = 0; j < kTopkSamples; ++j) {
    const int s = tid + kTopkThreads * j, run = s / kTopkRun;
    const int pos = (int)(((int64_t)run * n) / kTopkRuns) + (s - run * kTopkRun);
    sv[j] = sc[pos < n ? pos : n - 1];
  }
  f32x4_t cv[kTopkPer / 4];
  const int last = (int)p.sstride - 4;
#pragma unroll
  for (int i = 0; i < kTopkPer / 4; ++i) {
    const int pos = c0 + 4 * (tid + kTopkThreads * i);
    cv[i] = c0 < n ? *reinterpret_cast<const f32x4_t*>(sc + (pos < last ? pos : last)) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  zero_hist(h);
  if (tid < kDsaChunk / 32) s_sb[tid] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kTopkSamples; ++j) atomicAdd(&h[score_key(sv[j]) >> 19], 1u);
  __syncthreads();
  find_bins(h, 0, 0, true, k, n, s_w, s_out);
  const uint32_t lo = (uint32_t)s_out[2] << 19, hi = ((uint32_t)s_out[0] << 19) | 0x7FFFFu;
  clk_stamp(p.clk, 1);

  // ---- chunk pass
  int above = 0, nc = 0;
  uint32_t ck[kTopkPer];  // this thread's keys (0 past n)
#pragma unroll
  for (int i = 0; i < kTopkPer / 4; ++i) {
    uint32_t ns = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = c0 + 4 * (tid + kTopkThreads * i) + e;
      const uint32_t kk = pos < n ? score_key(cv[i][e]) : 0u;
      ck[4 * i + e] = kk;
      ns |= kk > hi ? 1u << e : 0u;
      nc += kk - lo <= hi - lo ? 1 : 0;
    }
    above += __popc(ns);
    if (ns) atomicOr(&s_sb[(tid + kTopkThreads * i) >> 3], ns << (4 * (tid & 7)));
  }
  // one scan for both counts, packed as above << 16 | candidates (each at most
  // 4096 per chunk); its barriers also order the bitmap's atomics before its
  // store below
  uint32_t ptot;
  const uint32_t cpfx = scan_wg<uint32_t>(((uint32_t)above << 16) | (uint32_t)nc, s_wu, &ptot);
  int slot = (int)(cpfx & 0xFFFFu);  // this thread's first candidate slot in the chunk's slice
  const int ntot = (int)(ptot & 0xFFFFu), atot = (int)(ptot >> 16);
#pragma unroll
  for (int i = 0; i < kTopkPer; ++i) {
    if (ck[i] - lo <= hi - lo) {
      const uint32_t pos = (uint32_t)(c0 + 4 * (tid + kTopkThreads * (i >> 2)) + (i & 3));
      __hip_atomic_store(cand + c0 + slot, ((uint64_t)ck[i] << 32) | pos, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ++slot;
    }
  }
  if (tid < kDsaChunk / 32)
    __hip_atomic_store(bits + ch * (kDsaChunk / 32) + tid, s_sb[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) {
    __hip_atomic_store(counts + 2 * ch, (uint32_t)atot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(counts + 2 * ch + 1, (uint32_t)ntot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Hand-off to the last workgroup of the sequence without a release / acquire
  // pair: the stores above are agent-scope atomic stores, written through to
  // the device-coherent level; each thread waits until its stores are
  // acknowledged (asm with a memory clobber, so the compiler keeps them before
  // it) and only then is the arrival counter incremented; the last workgroup
  // issues its agent-scope atomic loads only after the counter's value has
  // returned.  A fence pair would write back and invalidate the whole L2 of
  // the XCD for every workgroup.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(p.nchunk - 1);
  __syncthreads();
  clk_stamp(p.clk, 2);
  if (!s_last) return;

  // ---- last workgroup of the sequence.  One round of loads before any wait:
  // the chunks' counts, the first kPre candidates of every chunk (64 threads per
  // chunk; entries past a chunk's count are read but never used) and the
  // position bitmap.
  constexpr int kPre = 4 * 64;
  const int nch = (n + kDsaChunk - 1) / kDsaChunk;  // chunks holding positions < n
  const int cc = tid >> 6, j0 = tid & 63;           // this thread's chunk and first entry
  uint64_t pre[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    pre[u] = cc < nch ? __hip_atomic_load(cand + cc * kDsaChunk + j0 + 64 * u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                      : 0ull;
  const int nw = (n + 31) / 32;
  uint32_t wv[kTopkWpt];
#pragma unroll
  for (int u = 0; u < kTopkWpt; ++u) {
    const int i = tid + kTopkThreads * u;
    wv[u] = i < nw ? __hip_atomic_load(bits + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
  }
  if (tid <= nch) {
    uint32_t a = 0u, m = 0u;
    if (tid < nch) {
      a = __hip_atomic_load(counts + 2 * tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      m = __hip_atomic_load(counts + 2 * tid + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s_coff[tid] = m;
    h[tid] = a;  // scratch for the totals
  }
  __syncthreads();
  if (tid == 0) {  // candidate counts -> offsets; totals
    uint32_t acc = 0u, asum = 0u;
    for (int c = 0; c < nch; ++c) {
      const uint32_t m = s_coff[c];
      s_coff[c] = acc;
      acc += m;
      asum += h[c];
    }
    s_coff[nch] = acc;
    s_out[0] = (int)asum;
  }
  __syncthreads();
  const int A = s_out[0], M = (int)s_coff[nch];
  const bool exact = A < k && A + M >= k && M <= kTopkCandLds;  // workgroup-uniform
  int need;
  uint32_t prefix;
  __syncthreads();  // s_out is rewritten below
  if (exact) {
    {
      const int cnt_c = cc < nch ? (int)(s_coff[cc + 1] - s_coff[cc]) : 0, off = cc < nch ? (int)s_coff[cc] : 0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j0 + 64 * u < cnt_c) s_cand[off + j0 + 64 * u] = pre[u];
      for (int j = j0 + kPre; j < cnt_c; j += 64)  // chunks with more than kPre candidates
        s_cand[off + j] = __hip_atomic_load(cand + cc * kDsaChunk + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int u = 0; u < kTopkWpt; ++u) {
        s_sb[tid + kTopkThreads * u] = wv[u];
        s_tb[tid + kTopkThreads * u] = 0u;
      }
    }
    clk_stamp(p.clk, 3);
    // The k-th key among the candidates, digit by digit on the key relative to
    // lo (below 2^hb): 11 bits at a time from the top (2048-bin histograms).
    // Once the boundary bin holds at most 64 candidates, one wave ranks them
    // directly instead of another histogram pass.
    constexpr int kCB = 11, kCBins = 1 << kCB;
    need = k - A;
    int hb = 32 - __clz(hi - lo);
    int shift = hb > kCB ? hb - kCB : 0;
    uint32_t pm = 0u, pf = 0u;  // relative-key bits found so far: mask and value
    bool ranked = false;
    while (true) {  // workgroup-uniform
      const uint32_t dm = (1u << (hb - shift)) - 1u;  // hb - shift <= kCB
      for (int i = tid; i < kCBins; i += kTopkThreads) h[i] = 0u;
      __syncthreads();
      for (int i = tid; i < M; i += kTopkThreads) {
        const uint32_t r = (uint32_t)(s_cand[i] >> 32) - lo;
        if ((r & pm) == pf) atomicAdd(&h[(r >> shift) & dm], 1u);
      }
      __syncthreads();
      find_bins<kCBins>(h, need, need, false, 0, 0, s_w, s_out);
      const int cb = (int)h[s_out[0]];  // candidates in the boundary bin
      pf |= (uint32_t)s_out[0] << shift;
      pm |= dm << shift;
      need -= s_out[1];
      __syncthreads();  // s_out and h are rewritten below
      if (shift == 0) break;
      if (cb <= 64) {  // workgroup-uniform
        if (tid == 0) s_nb = 0;
        __syncthreads();
        for (int i = tid; i < M; i += kTopkThreads) {
          const uint32_t kc = (uint32_t)(s_cand[i] >> 32);
          if (((kc - lo) & pm) == pf) s_small[atomicAdd(&s_nb, 1)] = kc;
        }
        __syncthreads();
        if (tid < cb) {  // the need-th largest key: fewer than need above it, need at or above
          const uint32_t kc = s_small[tid];
          int gt = 0, ge = 0;
          for (int j = 0; j < cb; ++j) {
            const uint32_t v = s_small[j];
            gt += v > kc ? 1 : 0;
            ge += v >= kc ? 1 : 0;
          }
          if (gt < need && need <= ge) {  // every lane holding that key writes the same
            s_out[0] = (int)kc;
            s_out[1] = gt;
          }
        }
        __syncthreads();
        ranked = true;
        break;
      }
      hb = shift;
      shift = hb > kCB ? hb - kCB : 0;
    }
    if (ranked) {
      prefix = (uint32_t)s_out[0];
      need -= s_out[1];
    } else {
      prefix = lo + pf;
    }
    for (int i = tid; i < M; i += kTopkThreads) {
      const uint64_t c = s_cand[i];
      const uint32_t kc = (uint32_t)(c >> 32), pos = (uint32_t)c;
      if (kc > prefix) atomicOr(&s_sb[pos >> 5], 1u << (pos & 31));
      else if (kc == prefix) atomicOr(&s_tb[pos >> 5], 1u << (pos & 31));
    }
  } else {
    // The bound did not hold: three digit histograms (13, 13, 6 bits) over
    // every score of the sequence, read from the score row in rolled loops.
    for (int u = 0; u < kTopkWpt; ++u) {
      s_sb[tid + kTopkThreads * u] = 0u;
      s_tb[tid + kTopkThreads * u] = 0u;
    }
    need = k;
    prefix = 0u;
    uint32_t pmask = 0u;
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 19 : (pass == 1 ? 6 : 0);
      const uint32_t dmask = pass == 2 ? 0x3Fu : 0x1FFFu;
      zero_hist(h);
      __syncthreads();
      for (int pos = tid; pos < n; pos += kTopkThreads) {
        const uint32_t kk = score_key(sc[pos]);
        if ((kk & pmask) == prefix) atomicAdd(&h[(kk >> shift) & dmask], 1u);
      }
      __syncthreads();
      find_bins(h, need, need, false, 0, 0, s_w, s_out);
      prefix |= (uint32_t)s_out[0] << shift;
      pmask |= dmask << shift;
      need -= s_out[1];
      __syncthreads();
    }
    for (int pos = tid; pos < n; pos += kTopkThreads) {
      const uint32_t kk = score_key(sc[pos]);
      if (kk > prefix) atomicOr(&s_sb[pos >> 5], 1u << (pos & 31));
      else if (kk == prefix) atomicOr(&s_tb[pos >> 5], 1u << (pos & 31));
    }
  }
  // prefix is the k-th largest key: the keys above it are marked in s_sb, and
  // `need` of the keys equal to it (s_tb) are taken, the lowest positions first
  __syncthreads();
  clk_stamp(p.clk, 4);
  // Thread t owns words [kTopkWpt*t, +kTopkWpt).  One scan gives both the
  // marked positions (above the k-th key) and the ties before this thread,
  // packed as ties << 16 | marked: the marked total is below k <= 4096, so the
  // low field never carries, and a prefix of ties is below 2^16.  The first
  // `need` ties in position order are taken, so the ties taken before this
  // thread are min(need, its tie prefix), and its output offset follows.
  const int w0 = kTopkWpt * tid;
  uint32_t marked = 0u, ties = 0u;
  for (int e = 0; e < kTopkWpt; ++e) {
    marked += w0 + e < nw ? (uint32_t)__popc(s_sb[w0 + e]) : 0u;
    ties += w0 + e < nw ? (uint32_t)__popc(s_tb[w0 + e]) : 0u;
  }
  uint32_t ptotal;
  const uint32_t pfx = scan_wg<uint32_t>((ties << 16) | marked, s_wu, &ptotal);
  const int tb0 = (int)(pfx >> 16);
  int take = need - tb0;
  take = take < 0 ? 0 : (take > (int)ties ? (int)ties : take);
  int o = (int)(pfx & 0xFFFFu) + (tb0 < need ? tb0 : need);
  uint32_t word[kTopkWpt];
#pragma unroll
  for (int e = 0; e < kTopkWpt; ++e) {
    uint32_t s_ = w0 + e < nw ? s_sb[w0 + e] : 0u, t_ = w0 + e < nw ? s_tb[w0 + e] : 0u;
    while (t_ != 0u && take > 0) {  // lowest tie positions first
      const uint32_t low = t_ & (~t_ + 1u);
      s_ |= low;
      t_ ^= low;
      --take;
    }
    word[e] = s_;
  }
#pragma unroll
  for (int e = 0; e < kTopkWpt; ++e) {
    uint32_t s_ = word[e];
    while (s_ != 0u) {
      const int bit = __builtin_ctz(s_);
      s_ &= s_ - 1u;
      if (o < k) out[o++] = 32 * (w0 + e) + bit;
    }
  }
  clk_stamp(p.clk, exact ? 5 : 6);
}

// ---------------------------------------------------------------------------
// 3. attention over the selected tokens

constexpr int kTileTok = 32, kKt = kDsaDqk / 32;   // 18 fragments of 32 dims per 16-row group
constexpr int kFrag = (kTileTok / 16) * kKt;         // 36 fragments of 1 KB per tile
constexpr int kTileBytes = kTileTok * kDsaDqk * 2;   // 36 KB
constexpr int kNbuf = 4;                             // tiles of a split, all in flight at once
constexpr int kMaxSplit = kNbuf * kTileTok;          // selected tokens per workgroup (host plan: 128)

template <int NW>  // waves per workgroup; each owns 16 heads over every token of the split
__global__ __launch_bounds__(64 * NW, 1) void dsa_attn_kernel(DsaParams p) {
  constexpr int NT = 64 * NW, HPG = 16 * NW, NCP = kFrag / NW;  // threads, heads, copies per wave per tile
  static_assert(kFrag % NW == 0, "whole fragments per wave");
  __shared__ __attribute__((aligned(1024))) char s_buf[kNbuf][kTileBytes];
  __shared__ int s_rows[kMaxSplit];
  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ngrp = p.H / HPG, per_b = ngrp * p.ts;
  const int b = blockIdx.x / per_b, r = blockIdx.x - b * per_b;
  const int hg = r / p.ts, sp = r - hg * p.ts;
  uint64_t* clk = p.clk ? p.clk + (size_t)kClkMaxGroups * kClkSlots : nullptr;
  clk_stamp(clk, 0);
  const int64_t L = p.seq_lens[b];
  const int n = (int)(L < p.cap ? L : p.cap);
  const int nsel = n < p.topk ? n : p.topk;
  const int per = ((nsel + p.ts - 1) / p.ts + kTileTok - 1) / kTileTok * kTileTok;
  const int t0 = sp * per, t1 = t0 + per < nsel ? t0 + per : nsel;
  float* part = p.part + ((size_t)(b * ngrp + hg) * p.ts + sp) * HPG * kPartStride;
  if (t0 >= t1) {  // empty split
    if (tid < HPG) {
      part[tid * kPartStride] = -INFINITY;
      part[tid * kPartStride + 1] = 0.f;
    }
    return;
  }
  const int ntl = (t1 - t0 + kTileTok - 1) / kTileTok;  // <= kMaxSplit / kTileTok (host plan)
  const int32_t* sel = p.sel + (size_t)b * p.topk;
  const uint16_t* cb = p.c + (size_t)b * p.cap * kDsaDqk;

  // the split's selected positions, in LDS (rows past the end repeat the last one)
  for (int i = tid; i < ntl * kTileTok; i += NT) s_rows[i] = sel[t0 + i < t1 ? t0 + i : t1 - 1];
  // q fragments of this wave's 16 heads: B operand, head lr, dims 32*ks + 8*lg .. +8
  u32x4_t qf[kKt];
  {
    const uint16_t* qrow = p.q + ((size_t)b * p.H + HPG * hg + 16 * wave + lr) * kDsaDqk + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < kKt; ++ks) qf[ks] = ld16(qrow + 32 * ks);
  }
  __syncthreads();
  clk_stamp(clk, 1);
  // Fragment f = m*18 + ks holds the 16-byte chunks (dims 32*ks + 8*g .. of row
  // 16*m + R) for g < 4, R < 16 in the 64 slots of 1 KB, chunk (g, R) at slot
  // swz(g, R, ks) = (16*g + R) ^ ((2*g + ks) & 7): the S^T reads (lane (g, R))
  // stay a permutation of the slots, and the V reads -- 16 lanes on one row
  // across 16 chunks -- spread over the LDS banks (two lanes per bank group
  // instead of sixteen).  The copy writes lane i's chunk at slot i, so lane i
  // fetches the chunk that belongs there.  Wave w copies fragments w, w+NW, ...
  auto stage = [&](int it) {
    char* dst = s_buf[it % kNbuf];
#pragma unroll
    for (int ii = 0; ii < NCP; ++ii) {
      const int f = wave + NW * ii;
      const int m = f / kKt, ks = f - m * kKt;
      const int R = lr ^ ((2 * lg + ks) & 7);
      const int row = s_rows[kTileTok * it + 16 * m + R];
      copy16_to_lds(cb + (size_t)row * kDsaDqk + 32 * ks + 8 * lg, dst + f * 1024);
    }
  };

  // Every tile of the split is in flight at once (a split holds at most kNbuf
  // tiles), so no buffer is reused and the logits of all tiles fit in
  // registers: pass 1 computes them as the tiles land and takes the exact
  // maximum per head; pass 2 forms P = 2^(z - max) and O^T += V^T P^T.  With the
  // maximum known there is no rescaling of the accumulators, which then stay
  // in the matrix unit's registers, and the query fragments are dead in pass 2.
  for (int it = 0; it < ntl; ++it) stage(it);
  const float sc = p.scale_log2;
  float z[kNbuf][2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int it = 0; it < kNbuf; ++it) {
    if (it >= ntl) break;  // workgroup-uniform
    const int ahead = ntl - 1 - it;  // tiles issued after this one
    if (ahead >= 3) wait_vmem_le<3 * NCP>();
    else if (ahead == 2) wait_vmem_le<2 * NCP>();
    else if (ahead == 1) wait_vmem_le<NCP>();
    else wait_vmem();
    lds_barrier();  // every wave's copies of tile it have landed
    if (it == 0) clk_stamp(clk, 2);
    const char* kt = s_buf[it];
    // S^T for the tile's 32 tokens (row groups 0 and 1) and this wave's 16 heads
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKt; ++ks)
        s = mfma_bf16(*reinterpret_cast<const u32x4_t*>(kt + ((mm * kKt + ks) * 64 + (lane ^ ((2 * lg + ks) & 7))) * 16),
                      qf[ks], s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = kTileTok * it + 16 * mm + 4 * lg + i;  // token index within the split
        z[it][mm][i] = t0 + tt < t1 ? s[i] * sc : -INFINITY;
        mx = fmaxf(mx, z[it][mm][i]);
      }
    }
  }
  mx = max_over_groups_swap(mx);  // head lr over every token of the split (finite: the split is not empty)

  f32x4_t acc[4][8];  // dim block db (128 dims), operand jj: O^T[128*db + 8*(4lg+i) + jj][head lr]
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[db][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
#pragma unroll
  for (int it = 0; it < kNbuf; ++it) {
    if (it >= ntl) break;  // workgroup-uniform
    const char* kt = s_buf[it];
    float e[2][4];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[mm][i] = z[it][mm][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[it][mm][i] - mx);
        lsum += e[mm][i];
      }
    const u32x4_t pb = pack_probs(e[0], e[1]);
    // O^T += V^T P^T: the values are the first 512 latent dims; lane (lg, lr) reads
    // the 8 rows of its k-slots, 8 dims 128*db + 8*lr .. of each, from the fragments
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      uint32_t vr[8][4];
      const int c = 16 * db + lr, ks = c >> 2, lgc = c & 3;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int R = step_key(lg, rr);
        const int slot = (lgc * 16 + (R & 15)) ^ ((2 * lgc + ks) & 7);
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(kt + (((R >> 4) * kKt + ks) * 64 + slot) * 16);
        vr[rr][0] = x[0];
        vr[rr][1] = x[1];
        vr[rr][2] = x[2];
        vr[rr][3] = x[3];
      }
      pv_step<128>(vr, pb, acc[db]);
    }
  }
  clk_stamp(clk, 3);
  lsum = sum_over_groups_swap(lsum);
  // this wave's 16 heads: (m, l, O / l) to the partial
  float* dst = part + (size_t)(16 * wave + lr) * kPartStride;
  if (lg == 0) {
    dst[0] = mx;
    dst[1] = lsum;
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  // The output rows go through LDS (the tiles are dead once every wave is past
  // its value products), so that each store writes one head's 1 KB row:
  // row 16*wave + lr at byte kOutRow*(16*wave + lr), padded so that the 16 rows
  // a wave writes at once fall on different LDS banks.
  constexpr int kOutRow = 1024 + 16;
  __syncthreads();
  char* so = &s_buf[0][0];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // 8 consecutive channels 128*db + 8*(4lg+i) ..
      const f32x4_t* a = &acc[db][0];
      *reinterpret_cast<u32x4_t*>(so + (16 * wave + lr) * kOutRow + 2 * (128 * db + acc_channel<128>(lg, i, 0))) =
          u32x4_t{pack_f16x2(a[0][i] * inv, a[1][i] * inv), pack_f16x2(a[2][i] * inv, a[3][i] * inv),
                  pack_f16x2(a[4][i] * inv, a[5][i] * inv), pack_f16x2(a[6][i] * inv, a[7][i] * inv)};
    }
  lds_barrier();  // this wave's rows (each wave stores only the rows it wrote)
  float* wdst = part + (size_t)(16 * wave) * kPartStride;
#pragma unroll
  for (int hh = 0; hh < 16; ++hh) {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(so + (16 * wave + hh) * kOutRow + 16 * lane);
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(wdst + (size_t)hh * kPartStride + kPartOut) + 8 * lane) = x;
  }
  clk_stamp(clk, 4);
}

// ---------------------------------------------------------------------------
// 4. exact merge of the token splits: one wave per (sequence, head), 8 channels per lane
__global__ __launch_bounds__(256) void dsa_combine_kernel(DsaParams p) {
  constexpr int MS = 16;  // splits held in registers; more are merged in a second loop
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int bh = 4 * blockIdx.x + wave;
  if (bh >= p.B * p.H) return;
  const int b = bh / p.H, h = bh - b * p.H;
  const int ngrp = p.H / p.hpg, hg = h / p.hpg, hl = h - hg * p.hpg;
  const float* src = p.part + ((size_t)(b * ngrp + hg) * p.ts * p.hpg + hl) * kPartStride;
  const size_t sstep = (size_t)p.hpg * kPartStride;
  const int c = 8 * lane;  // this lane's 8 channels
  float m[MS], l[MS];
  u32x4_t v[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s) {  // every load issued before any is used
    const bool in = s < p.ts;
    m[s] = in ? src[s * sstep] : -INFINITY;
    l[s] = in ? src[s * sstep + 1] : 0.f;
    v[s] = in ? *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(src + s * sstep + kPartOut) + c)
              : u32x4_t{0u, 0u, 0u, 0u};
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MS; ++s) M = fmaxf(M, m[s]);
  for (int s = MS; s < p.ts; ++s) M = fmaxf(M, src[s * sstep]);
  float Ls = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](float ms, float ls, u32x4_t w) {
    if (ms == -INFINITY) return;
    const float a = __builtin_amdgcn_exp2f(ms - M) * ls;  // the split's weight: exp(m - M) * l
    Ls += a;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x2_t x = unpack_f16x2(w[q]);
      o[2 * q] += a * x[0];
      o[2 * q + 1] += a * x[1];
    }
  };
#pragma unroll
  for (int s = 0; s < MS; ++s) add(m[s], l[s], v[s]);
  for (int s = MS; s < p.ts; ++s)
    add(src[s * sstep], src[s * sstep + 1],
        *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(src + s * sstep + kPartOut) + c));
  const float inv = Ls > 0.f ? 1.0f / Ls : 0.f;
  u32x4_t w;
#pragma unroll
  for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(o[2 * q] * inv, o[2 * q + 1] * inv);
  *reinterpret_cast<u32x4_t*>(p.out + ((size_t)b * p.H + h) * kDsaDv + c) = w;
}

template <int HI, int DI>
hipError_t launch_dsa_t(const DsaParams& p, hipStream_t s, const PhaseEvents* ev) {
  if (ev) (void)hipEventRecord(ev->ev[0], s);
  hipLaunchKernelGGL((dsa_index_kernel<HI, DI>), dim3((unsigned)(p.B * p.nseg)), dim3(256), 0, s, p);
  if (ev) (void)hipEventRecord(ev->ev[1], s);
  hipLaunchKernelGGL(dsa_topk_kernel, dim3((unsigned)(p.B * p.nchunk)), dim3(kTopkThreads), 0, s, p);
  if (ev) (void)hipEventRecord(ev->ev[2], s);
  if (p.hpg == 64)
    hipLaunchKernelGGL((dsa_attn_kernel<4>), dim3((unsigned)(p.B * (p.H / 64) * p.ts)), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((dsa_attn_kernel<2>), dim3((unsigned)(p.B * (p.H / 32) * p.ts)), dim3(128), 0, s, p);
  hipLaunchKernelGGL(dsa_combine_kernel, dim3((unsigned)((p.B * p.H + 3) / 4)), dim3(256), 0, s, p);
  if (ev) (void)hipEventRecord(ev->ev[3], s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dsa_decode(const DsaParams& p, hipStream_t s, const PhaseEvents* ev) {
  if (p.HI == 16 && p.DI == 128) return launch_dsa_t<16, 128>(p, s, ev);
  if (p.HI == 16 && p.DI == 64) return launch_dsa_t<16, 64>(p, s, ev);
  if (p.HI == 32 && p.DI == 128) return launch_dsa_t<32, 128>(p, s, ev);
  if (p.HI == 32 && p.DI == 64) return launch_dsa_t<32, 64>(p, s, ev);
  if (p.HI == 64 && p.DI == 128) return launch_dsa_t<64, 128>(p, s, ev);
  if (p.HI == 64 && p.DI == 64) return launch_dsa_t<64, 64>(p, s, ev);
  return hipErrorInvalidValue;
}

}  // namespace nsa

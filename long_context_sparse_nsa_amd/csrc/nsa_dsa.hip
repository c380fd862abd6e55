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
//  2. exact top-k by radix select on order-preserving integer keys of the
//     scores, over 4096-score chunks: dsa_hist_kernel sums the top-13-bit
//     histogram of every chunk into one per sequence (zeroed by the indexer
//     launch); dsa_select_kernel marks the positions above the boundary bin in a
//     bitmap and collects the boundary bin's scores, and the last workgroup of
//     the sequence finishes the select on those candidates (13 + 6 more bits),
//     takes ties at the threshold from the lowest positions and writes the
//     positions ascending.
//  3. dsa_attn_kernel    workgroup = (sequence, 64 heads -- 32 when the head
//     count is not a multiple of 64 --, token split); 32-token tiles of latents
//     are gathered into LDS with the direct global->LDS copy, four buffers
//     (three tiles in flight), and every wave reads each tile for its own 16
//     heads: one online softmax per wave, no exchange between waves, and the
//     tile's latents are gathered once per 64 heads.
//  4. dsa_combine_kernel merges the token-split partials exactly and writes bf16.
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
  if (sg == 0) {  // the selection's histogram and counters start at zero (used by the next launches)
    for (int i = tid; i < kDsaBins; i += 256) p.hist[(size_t)b * kDsaBins + i] = 0u;
    if (tid < 4) p.cnt[4 * b + tid] = 0u;
  }
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
// 2. exact top-k of the scores

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // larger float -> larger key
}

// Exclusive prefix over the 256 threads of a selection workgroup.
__device__ __forceinline__ int scan256(int v, int* s_w, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int s = s_w[w];
    base += w < wave ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// The 16 order keys of this thread's positions c0 + 16*tid .. +15 (0 past n):
// four 16-byte loads, addresses clamped inside the score row.
__device__ __forceinline__ void load_keys16(const DsaParams& p, int b, int c0, int n, uint32_t (&key)[16], int& nv) {
  const float* sc = p.scores + (size_t)b * p.sstride;
  const int base = c0 + 16 * (int)threadIdx.x, last = (int)p.sstride - 4;
  f32x4_t v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const f32x4_t*>(sc + (base + 4 * q < last ? base + 4 * q : last));
  nv = n - base;
  nv = nv < 0 ? 0 : (nv > 16 ? 16 : nv);
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) key[4 * q + e] = 4 * q + e < nv ? order_key(v[q][e]) : 0u;
}

// In a histogram of `nb` bins (nb / 256 per thread, a power of two; the highest
// bins to thread 0), the bin holding the need-th largest key and the count of
// keys above it.  Each thread sums its bins starting at a rotated offset, so the
// lanes of a wave read different LDS banks; only the thread whose segment holds
// the boundary walks it in order.
__device__ __forceinline__ void find_bin(const uint32_t* h, int nb, int need, int* s_w, int* s_found) {
  const int tid = (int)threadIdx.x, per = nb / 256, g0 = per * (255 - tid);
  int sum = 0;
#pragma unroll 8
  for (int e = 0; e < per; ++e) sum += (int)h[g0 + ((e + tid) & (per - 1))];
  int total;
  const int above = scan256(sum, s_w, &total);
  if (above < need && above + sum >= need) {
    int acc = above;
    for (int e = per - 1; e >= 0; --e) {
      const int c = (int)h[g0 + e];
      if (acc + c >= need) {
        s_found[0] = g0 + e;
        s_found[1] = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

// 2a. first-digit histogram of every score, summed over the workgroups of a sequence
__global__ __launch_bounds__(256) void dsa_hist_kernel(DsaParams p) {
  __shared__ uint32_t h[kDsaBins];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / p.nchunk, ch = blockIdx.x - b * p.nchunk;
  const int64_t L = p.seq_lens[b];
  const int n = (int)(L < p.cap ? L : p.cap);
  const int c0 = ch * kDsaChunk;
  if (n <= p.topk || c0 >= n) return;  // workgroup-uniform
  for (int i = tid; i < kDsaBins; i += 256) h[i] = 0u;
  uint32_t key[16];
  int nv;
  load_keys16(p, b, c0, n, key, nv);
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (k < nv) atomicAdd(&h[key[k] >> 19], 1u);
  __syncthreads();
  uint32_t* gh = p.hist + (size_t)b * kDsaBins;
  for (int i = tid; i < kDsaBins; i += 256) {
    const uint32_t c = h[i];
    if (c) atomicAdd(gh + i, c);
  }
}

// 2b. every workgroup finds the first digit's boundary bin, marks the positions
// above it in the bitmap and writes the boundary bin's scores into its own slice
// of the candidate list; the last workgroup of the sequence resolves the
// candidates exactly (two more digits, ties to the lower position) and writes
// the positions ascending.  Bitmap words, candidates and counts are stored with
// agent-scope atomic stores and read with agent-scope atomic loads after the
// arrival count (the workgroups of a sequence may sit on different XCDs, whose
// L2s are not coherent for plain stores).
constexpr int kCandLds = 4096;  // candidates the last workgroup holds in LDS
constexpr int kCandPer = 4;     // candidate loads per thread in flight at once

__global__ __launch_bounds__(256) void dsa_select_kernel(DsaParams p) {
  __shared__ uint32_t h[kDsaBins];
  __shared__ uint32_t s_bits[2 * kDsaMaxLen / 32];  // this chunk's words; later selected + tie words
  __shared__ uint64_t s_cand[kCandLds];
  __shared__ int s_w[4];
  __shared__ int s_found[2];
  __shared__ int s_last, s_nc;
  __shared__ uint32_t s_coff[kDsaMaxLen / kDsaChunk + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int b = blockIdx.x / p.nchunk, ch = blockIdx.x - b * p.nchunk;
  const int64_t L = p.seq_lens[b];
  const int n = (int)(L < p.cap ? L : p.cap);
  int32_t* out = p.sel + (size_t)b * p.topk;
  if (n <= p.topk) {  // every past token
    if (ch == 0)
      for (int i = tid; i < p.topk; i += 256) out[i] = i < n ? i : -1;
    return;
  }
  const int c0 = ch * kDsaChunk;
  uint32_t* bits = p.bits + (size_t)b * p.nchunk * 128;
  uint64_t* cand = p.cand + (size_t)b * p.cap;       // chunk ch writes entries [c0, c0 + its count)
  uint32_t* ccount = p.cnt + (size_t)p.B * 4 + (size_t)b * p.nchunk;  // per-chunk candidate counts
  uint32_t* arrive = p.cnt + 4 * b + 1;

  // the first digit's histogram into LDS (eight 16-byte loads per thread, all in flight)
  {
    const u32x4_t* gh = reinterpret_cast<const u32x4_t*>(p.hist + (size_t)b * kDsaBins);
    u32x4_t v[kDsaBins / 4 / 256];
#pragma unroll
    for (int q = 0; q < kDsaBins / 4 / 256; ++q) v[q] = gh[tid + 256 * q];
#pragma unroll
    for (int q = 0; q < kDsaBins / 4 / 256; ++q) reinterpret_cast<u32x4_t*>(h)[tid + 256 * q] = v[q];
  }
  if (tid == 0) s_nc = 0;
  __syncthreads();
  find_bin(h, kDsaBins, p.topk, s_w, s_found);
  const uint32_t T0 = (uint32_t)s_found[0];
  const int above0 = s_found[1];
  if (c0 < n) {
    uint32_t key[16];
    int nv;
    load_keys16(p, b, c0, n, key, nv);
    if (tid < 128) s_bits[tid] = 0u;
    __syncthreads();
    uint32_t w = 0u;  // this thread's 16 positions: half of bitmap word tid / 2
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t bin = key[k] >> 19;
      const bool valid = k < nv;
      if (valid && bin > T0) w |= 1u << (16 * (tid & 1) + k);
      const bool cd = valid && bin == T0;
      const uint64_t m = __ballot(cd);
      if (m != 0ull) {  // wave-aggregated slot in this chunk's slice
        const int first = __builtin_ctzll(m);
        int slot0 = 0;
        if (lane == first) slot0 = atomicAdd(&s_nc, __popcll(m));
        slot0 = __shfl(slot0, first);
        if (cd) {
          const int slot = slot0 + __popcll(m & ((1ull << lane) - 1ull));
          __hip_atomic_store(cand + c0 + slot, ((uint64_t)key[k] << 32) | (uint32_t)(c0 + 16 * tid + k),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    atomicOr(&s_bits[tid >> 1], w);
    __syncthreads();
    if (tid < 128) __hip_atomic_store(bits + ch * 128 + tid, s_bits[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid == 0) __hip_atomic_store(ccount + ch, (uint32_t)s_nc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(p.nchunk - 1);
  __syncthreads();
  if (!s_last) return;

  // ---- last workgroup.  Candidate offsets per chunk, then every candidate and
  // bitmap word loaded in one round trip.
  if (tid < p.nchunk) s_coff[tid + 1] = __hip_atomic_load(ccount + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (tid == 0) {  // counts -> offsets (at most 16 chunks)
    uint32_t acc = 0u;
    s_coff[0] = 0u;
    for (int c = 1; c <= p.nchunk; ++c) {
      acc += s_coff[c];
      s_coff[c] = acc;
    }
  }
  __syncthreads();
  const int nc = (int)s_coff[p.nchunk];
  const bool in_lds = nc <= kCandLds;
  // candidate e lives in chunk c (s_coff[c] <= e < s_coff[c+1]) at slot e - s_coff[c]
  auto cand_at = [&](int e) -> const uint64_t* {
    int c = 0;
    while (c + 1 < p.nchunk && (int)s_coff[c + 1] <= e) ++c;
    return cand + c * kDsaChunk + (e - (int)s_coff[c]);
  };
  if (in_lds) {  // chunk c's slice is copied by threads 16c .. 16c + 15, four loads in flight each
    const int c = tid >> 4, j = tid & 15;
    if (c < p.nchunk) {
      const int cnt_c = (int)(s_coff[c + 1] - s_coff[c]), off = (int)s_coff[c];
      for (int i0 = j; i0 < cnt_c; i0 += 16 * kCandPer) {
        uint64_t v[kCandPer];
#pragma unroll
        for (int u = 0; u < kCandPer; ++u) {
          const int i = i0 + 16 * u;
          v[u] = i < cnt_c ? __hip_atomic_load(cand + c * kDsaChunk + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0ull;
        }
#pragma unroll
        for (int u = 0; u < kCandPer; ++u)
          if (i0 + 16 * u < cnt_c) s_cand[off + i0 + 16 * u] = v[u];
      }
    }
  }
  auto cand_get = [&](int e) -> uint64_t {
    return in_lds ? s_cand[e] : __hip_atomic_load(cand_at(e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  int need = p.topk - above0;
  uint32_t prefix = T0 << 19, pmask = 0xFFF80000u;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 6 : 0;
    const uint32_t dmask = pass == 0 ? 0x1FFFu : 0x3Fu;
    __syncthreads();
    for (int i = tid; i < kDsaBins; i += 256) h[i] = 0u;
    __syncthreads();
    for (int i = tid; i < nc; i += 256) {
      const uint32_t k = (uint32_t)(cand_get(i) >> 32);
      if ((k & pmask) == prefix) atomicAdd(&h[(k >> shift) & dmask], 1u);
    }
    __syncthreads();
    find_bin(h, pass == 0 ? kDsaBins : 256, need, s_w, s_found);
    prefix |= (uint32_t)s_found[0] << shift;
    pmask |= dmask << shift;
    need -= s_found[1];
    __syncthreads();
  }
  // prefix is the k-th largest key: keys above it are in; `need` ties at it go to
  // the lowest positions
  const int nw = (n + 31) / 32;
  constexpr int WPT = kDsaMaxLen / 32 / 256;
  uint32_t* sb = s_bits;
  uint32_t* tb = s_bits + kDsaMaxLen / 32;
  {
    uint32_t v[WPT];
#pragma unroll
    for (int e = 0; e < WPT; ++e) {
      const int i = tid + 256 * e;
      v[e] = i < nw ? __hip_atomic_load(bits + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    }
#pragma unroll
    for (int e = 0; e < WPT; ++e) {
      sb[tid + 256 * e] = v[e];
      tb[tid + 256 * e] = 0u;
    }
  }
  __syncthreads();
  for (int i = tid; i < nc; i += 256) {
    const uint64_t e = cand_get(i);
    const uint32_t k = (uint32_t)(e >> 32), pos = (uint32_t)e;
    if (k > prefix) atomicOr(&sb[pos >> 5], 1u << (pos & 31));
    else if (k == prefix) atomicOr(&tb[pos >> 5], 1u << (pos & 31));
  }
  __syncthreads();
  // thread t owns words [WPT*t, WPT*t + WPT): ties taken in position order, then
  // the selected positions written ascending
  const int w0 = WPT * tid;
  int ties = 0;
#pragma unroll
  for (int e = 0; e < WPT; ++e) ties += w0 + e < nw ? __popc(tb[w0 + e]) : 0;
  int total;
  int tb0 = scan256(ties, s_w, &total);
  int take = need - tb0;
  take = take < 0 ? 0 : (take > ties ? ties : take);
  int cntsel = 0;
  uint32_t word[WPT];
#pragma unroll
  for (int e = 0; e < WPT; ++e) {
    uint32_t s_ = w0 + e < nw ? sb[w0 + e] : 0u, t_ = w0 + e < nw ? tb[w0 + e] : 0u;
    while (t_ != 0u && take > 0) {  // lowest tie positions first
      const uint32_t low = t_ & (~t_ + 1u);
      s_ |= low;
      t_ ^= low;
      --take;
    }
    word[e] = s_;
    cntsel += __popc(s_);
  }
  int o = scan256(cntsel, s_w, &total);
#pragma unroll
  for (int e = 0; e < WPT; ++e) {
    uint32_t s_ = word[e];
    while (s_ != 0u) {
      const int bit = __builtin_ctz(s_);
      s_ &= s_ - 1u;
      if (o < p.topk) out[o++] = 32 * (w0 + e) + bit;
    }
  }
}

// ---------------------------------------------------------------------------
// 3. attention over the selected tokens

constexpr int kTileTok = 32, kKt = kDsaDqk / 32;   // 18 fragments of 32 dims per 16-row group
constexpr int kFrag = (kTileTok / 16) * kKt;         // 36 fragments of 1 KB per tile
constexpr int kTileBytes = kTileTok * kDsaDqk * 2;   // 36 KB
constexpr int kNbuf = 4;                             // three tiles in flight while one is used
constexpr int kMaxSplit = 512;                       // selected tokens per workgroup (host plan)
constexpr int kCopies = kFrag / 4;                   // copy instructions per wave per tile

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

  f32x4_t acc[4][8];  // dim block db (128 dims), operand jj: O^T[128*db + 8*(4lg+i) + jj][head lr]
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[db][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mref = -INFINITY, lsum = 0.f;
  const float sc = p.scale_log2;

  for (int it = 0; it < kNbuf - 1 && it < ntl; ++it) stage(it);
  for (int it = 0; it < ntl; ++it) {
    if (it + kNbuf - 1 < ntl) stage(it + kNbuf - 1);
    const int ahead = ntl - 1 - it < kNbuf - 1 ? ntl - 1 - it : kNbuf - 1;  // tiles issued after this one
    if (ahead >= 3) wait_vmem_le<3 * NCP>();
    else if (ahead == 2) wait_vmem_le<2 * NCP>();
    else if (ahead == 1) wait_vmem_le<NCP>();
    else wait_vmem();
    lds_barrier();
    const char* kt = s_buf[it % kNbuf];
    // S^T for the tile's 32 tokens (row groups 0 and 1) and this wave's 16 heads
    f32x4_t s[2];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      s[mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKt; ++ks)
        s[mm] = mfma_bf16(*reinterpret_cast<const u32x4_t*>(kt + ((mm * kKt + ks) * 64 + (lane ^ ((2 * lg + ks) & 7))) * 16),
                          qf[ks], s[mm]);
    }
    float z[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = kTileTok * it + 16 * mm + 4 * lg + i;  // token index within the split
        z[mm][i] = t0 + tt < t1 ? s[mm][i] * sc : -INFINITY;
        mx = fmaxf(mx, z[mm][i]);
      }
    mx = max_over_groups_swap(mx);  // head lr over the tile's 32 tokens
    if (mx > mref + 8.f || (mref == -INFINITY && mx > -INFINITY)) {  // move the reference (lazily)
      const float f = mref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref - mx);
      lsum *= f;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc[db][jj] *= f;
      mref = mx;
    }
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[mm][i] = z[mm][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[mm][i] - mref);
        lsum += z[mm][i];
      }
    const u32x4_t pb = pack_probs(z[0], z[1]);
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
    lds_barrier();  // every wave is done with this buffer before it is refilled
  }
  lsum = sum_over_groups_swap(lsum);
  // this wave's 16 heads: (m, l, O / l) to the partial
  float* dst = part + (size_t)(16 * wave + lr) * kPartStride;
  if (lg == 0) {
    dst[0] = mref;
    dst[1] = lsum;
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  uint16_t* oh = reinterpret_cast<uint16_t*>(dst + kPartOut);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // 8 consecutive channels 128*db + 8*(4lg+i) .. in one 16-byte store
      const f32x4_t* a = &acc[db][0];
      *reinterpret_cast<u32x4_t*>(oh + 128 * db + acc_channel<128>(lg, i, 0)) =
          u32x4_t{pack_f16x2(a[0][i] * inv, a[1][i] * inv), pack_f16x2(a[2][i] * inv, a[3][i] * inv),
                  pack_f16x2(a[4][i] * inv, a[5][i] * inv), pack_f16x2(a[6][i] * inv, a[7][i] * inv)};
    }
}

// ---------------------------------------------------------------------------
// 4. exact merge of the token splits: workgroup per (sequence, head), 4 channels per thread
__global__ __launch_bounds__(128) void dsa_combine_kernel(DsaParams p) {
  constexpr int MS = 16;  // splits held in registers; more are merged in a second loop
  const int bh = blockIdx.x, b = bh / p.H, h = bh - b * p.H;
  const int ngrp = p.H / p.hpg, hg = h / p.hpg, hl = h - hg * p.hpg;
  const float* src = p.part + ((size_t)(b * ngrp + hg) * p.ts * p.hpg + hl) * kPartStride;
  const size_t sstep = (size_t)p.hpg * kPartStride;
  const int c = 4 * threadIdx.x;  // this thread's 4 channels
  float m[MS], l[MS];
  u32x2_t v[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s) {  // every load issued before any is used
    const bool in = s < p.ts;
    m[s] = in ? src[s * sstep] : -INFINITY;
    l[s] = in ? src[s * sstep + 1] : 0.f;
    v[s] = in ? *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const uint16_t*>(src + s * sstep + kPartOut) + c)
              : u32x2_t{0u, 0u};
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MS; ++s) M = fmaxf(M, m[s]);
  for (int s = MS; s < p.ts; ++s) M = fmaxf(M, src[s * sstep]);
  float Ls = 0.f;
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
  auto add = [&](float ms, float ls, u32x2_t w) {
    if (ms == -INFINITY) return;
    const float a = __builtin_amdgcn_exp2f(ms - M) * ls;  // the split's weight: exp(m - M) * l
    const f32x2_t x0 = unpack_f16x2(w[0]), x1 = unpack_f16x2(w[1]);
    Ls += a;
    o = f32x4_t{o[0] + a * x0[0], o[1] + a * x0[1], o[2] + a * x1[0], o[3] + a * x1[1]};
  };
#pragma unroll
  for (int s = 0; s < MS; ++s) add(m[s], l[s], v[s]);
  for (int s = MS; s < p.ts; ++s)
    add(src[s * sstep], src[s * sstep + 1],
        *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const uint16_t*>(src + s * sstep + kPartOut) + c));
  const float inv = Ls > 0.f ? 1.0f / Ls : 0.f;
  u32x2_t w;
  w[0] = pack_bf16x2(o[0] * inv, o[1] * inv);
  w[1] = pack_bf16x2(o[2] * inv, o[3] * inv);
  *reinterpret_cast<u32x2_t*>(p.out + ((size_t)b * p.H + h) * kDsaDv + c) = w;
}

template <int HI, int DI>
hipError_t launch_dsa_t(const DsaParams& p, hipStream_t s, const PhaseEvents* ev) {
  if (ev) (void)hipEventRecord(ev->ev[0], s);
  hipLaunchKernelGGL((dsa_index_kernel<HI, DI>), dim3((unsigned)(p.B * p.nseg)), dim3(256), 0, s, p);
  if (ev) (void)hipEventRecord(ev->ev[1], s);
  hipLaunchKernelGGL(dsa_hist_kernel, dim3((unsigned)(p.B * p.nchunk)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(dsa_select_kernel, dim3((unsigned)(p.B * p.nchunk)), dim3(256), 0, s, p);
  if (ev) (void)hipEventRecord(ev->ev[2], s);
  if (p.hpg == 64)
    hipLaunchKernelGGL((dsa_attn_kernel<4>), dim3((unsigned)(p.B * (p.H / 64) * p.ts)), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((dsa_attn_kernel<2>), dim3((unsigned)(p.B * (p.H / 32) * p.ts)), dim3(128), 0, s, p);
  hipLaunchKernelGGL(dsa_combine_kernel, dim3((unsigned)(p.B * p.H)), dim3(128), 0, s, p);
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

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
//  2. dsa_select_kernel  one 1024-thread workgroup per sequence holds the
//     scores as order-preserving integer keys in registers and finds the k-th
//     largest exactly by radix select (12 + 12 + 8 bits, LDS histograms; a
//     wave whose active lanes share a digit adds once); ties at the threshold
//     go to the lower positions; the ids are written ascending.
//  3. dsa_attn_kernel    workgroup = (sequence, 32 heads, token split); 64-token
//     tiles of latents are gathered into LDS with the direct global->LDS copy
//     (two buffers).  Wave (head tile, token half) keeps its own online softmax
//     over its 32 tokens of each tile, so no per-tile exchange is needed; the
//     two halves merge through LDS at the end into one partial per workgroup.
//  4. dsa_combine_kernel merges the token-split partials exactly and writes bf16.
#include <hip/hip_runtime.h>

#include "nsa_device.hpp"
#include "nsa_internal.hpp"
#include "nsa_stage.hpp"
#include "nsa_tiles.hpp"

namespace nsa {

namespace {

constexpr int kPartStride = 520;  // floats per (head) partial: m, l, 6 pad, 512 outputs
constexpr int kPartOut = 8;

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

// Exclusive prefix over the 1024 threads of the workgroup (16 waves).
__device__ __forceinline__ int scan1024(int v, int* s_w, int* total) {
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
  for (int w = 0; w < 16; ++w) {
    const int s = s_w[w];
    base += w < wave ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__global__ __launch_bounds__(kDsaSelThreads) void dsa_select_kernel(DsaParams p) {
  constexpr int KPT = kDsaKeysPerThread;
  __shared__ uint32_t hist[4096];
  __shared__ int s_w[16];
  __shared__ int s_found[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int b = blockIdx.x;
  const int64_t L = p.seq_lens[b];
  const int n = (int)(L < p.cap ? L : p.cap);
  int32_t* out = p.sel + (size_t)b * p.topk;
  if (n <= p.topk) {  // every past token
    for (int i = tid; i < p.topk; i += kDsaSelThreads) out[i] = i < n ? i : -1;
    return;
  }
  const int base = tid * KPT;  // this thread's positions: base .. base + KPT - 1
  const float* sc = p.scores + (size_t)b * p.sstride;
  uint32_t key[KPT];
#pragma unroll
  for (int k4 = 0; k4 < KPT / 4; ++k4) {
    const int i0 = base + 4 * k4;
    if (i0 + 3 < n) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(sc + i0);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[4 * k4 + e] = order_key(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) key[4 * k4 + e] = i0 + e < n ? order_key(sc[i0 + e]) : 0u;
    }
  }
  int nvalid = n - base;
  nvalid = nvalid < 0 ? 0 : (nvalid > KPT ? KPT : nvalid);

  uint32_t prefix = 0u, pmask = 0u;
  int need = p.topk;  // still to take among the keys that match the prefix
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const uint32_t dmask = pass == 2 ? 0xFFu : 0xFFFu;
    for (int i = tid; i < 4096; i += kDsaSelThreads) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const bool act = k < nvalid && (key[k] & pmask) == prefix;
      const uint32_t d = (key[k] >> shift) & dmask;
      const uint64_t am = __ballot(act);
      if (am != 0ull) {
        const int first = __builtin_ctzll(am);
        const uint32_t d0 = (uint32_t)__shfl((int)d, first);
        const uint64_t same = __ballot(act && d == d0);
        if (same == am) {
          if (lane == first) atomicAdd(&hist[d0], (uint32_t)__popcll(am));
        } else if (act) {
          atomicAdd(&hist[d], 1u);
        }
      }
    }
    __syncthreads();
    // bins 4*(1023 - tid) .. +3 per thread: the prefix over threads is the count above
    const int g0 = 4 * (kDsaSelThreads - 1 - tid);
    const uint32_t h0 = hist[g0], h1 = hist[g0 + 1], h2 = hist[g0 + 2], h3 = hist[g0 + 3];
    int total;
    const int above = scan1024((int)(h0 + h1 + h2 + h3), s_w, &total);
    int acc = above;
    const uint32_t hv[4] = {h3, h2, h1, h0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // bins from the highest down
      const int c = (int)hv[e];
      if (acc < need && acc + c >= need) {
        s_found[0] = g0 + 3 - e;
        s_found[1] = acc;
      }
      acc += c;
    }
    __syncthreads();
    prefix |= (uint32_t)s_found[0] << shift;
    pmask |= dmask << shift;
    need -= s_found[1];
    __syncthreads();
  }
  // prefix is the k-th largest key; take every larger key and the first `need`
  // equal ones by position
  int gt = 0, eq = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    gt += (k < nvalid && key[k] > prefix) ? 1 : 0;
    eq += (k < nvalid && key[k] == prefix) ? 1 : 0;
  }
  int total;
  const int eb = scan1024(eq, s_w, &total);
  int take = need - eb;
  take = take < 0 ? 0 : (take > eq ? eq : take);
  int o = scan1024(gt + take, s_w, &total);
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    if (k < nvalid) {
      const bool sel = key[k] > prefix || (key[k] == prefix && take > 0);
      if (key[k] == prefix && take > 0) --take;
      if (sel && o < p.topk) out[o++] = base + k;  // o < topk always; the test keeps a bad count in bounds
    }
  }
}

// ---------------------------------------------------------------------------
// 3. attention over the selected tokens

constexpr int kTileTok = 64, kKt = kDsaDqk / 32;  // 18 fragments of 32 dims per 16-row group
constexpr int kTileBytes = kTileTok * kDsaDqk * 2;  // 72 KB
constexpr int kMaxTilesPerSplit = 8;

__global__ __launch_bounds__(256, 1) void dsa_attn_kernel(DsaParams p) {
  __shared__ __attribute__((aligned(1024))) char s_buf[2][kTileBytes];
  __shared__ int s_rows[kMaxTilesPerSplit * kTileTok];
  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jt = wave >> 1, hh = wave & 1;  // head tile, token half
  const int ngrp = p.H / 32, per_b = ngrp * p.ts;
  const int b = blockIdx.x / per_b, r = blockIdx.x - b * per_b;
  const int hg = r / p.ts, sp = r - hg * p.ts;
  const int64_t L = p.seq_lens[b];
  const int n = (int)(L < p.cap ? L : p.cap);
  const int nsel = n < p.topk ? n : p.topk;
  const int per = ((nsel + p.ts - 1) / p.ts + kTileTok - 1) / kTileTok * kTileTok;
  const int t0 = sp * per, t1 = t0 + per < nsel ? t0 + per : nsel;
  float* part = p.part + ((size_t)(b * ngrp + hg) * p.ts + sp) * 32 * kPartStride;
  if (t0 >= t1) {  // empty split
    if (tid < 32) {
      part[tid * kPartStride] = -INFINITY;
      part[tid * kPartStride + 1] = 0.f;
    }
    return;
  }
  const int ntl = (t1 - t0 + kTileTok - 1) / kTileTok;  // <= kMaxTilesPerSplit (host plan)
  const int32_t* sel = p.sel + (size_t)b * p.topk;
  const uint16_t* cb = p.c + (size_t)b * p.cap * kDsaDqk;

  // the split's selected positions, in LDS (rows past the end repeat the last one)
  for (int i = tid; i < ntl * kTileTok; i += 256) s_rows[i] = sel[t0 + i < t1 ? t0 + i : t1 - 1];
  // q fragments of this wave's 16 heads: B operand, head lr, dims 32*ks + 8*lg .. +8
  u32x4_t qf[kKt];
  {
    const uint16_t* qrow = p.q + ((size_t)b * p.H + 32 * hg + 16 * jt + lr) * kDsaDqk + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < kKt; ++ks) qf[ks] = ld16(qrow + 32 * ks);
  }
  // 72 fragments of 1 KB per tile; wave w copies fragments w, w+4, ... (18 each):
  // fragment f = m*18 + ks holds, at 16*lane, dims 32*ks + 8*lg .. of row 16*m + lr
  __syncthreads();
  auto stage = [&](int it, int buf) {
#pragma unroll
    for (int ii = 0; ii < kKt; ++ii) {
      const int f = wave + 4 * ii;
      const int m = f / kKt, ks = f - m * kKt;
      const int row = s_rows[kTileTok * it + 16 * m + lr];
      copy16_to_lds(cb + (size_t)row * kDsaDqk + 32 * ks + 8 * lg, s_buf[buf] + f * 1024);
    }
  };

  f32x4_t acc[4][8];  // dim block db (128 dims), tile jj: O^T[128*db + 8*(4lg+i) + jj][head lr]
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[db][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mref = -INFINITY, lsum = 0.f;
  const float sc = p.scale_log2;

  stage(0, 0);
  for (int it = 0; it < ntl; ++it) {
    if (it + 1 < ntl) {
      stage(it + 1, (it + 1) & 1);
      wait_vmem_le<kKt>();
    } else {
      wait_vmem();
    }
    lds_barrier();
    const char* kt = s_buf[it & 1];
    // S^T for this wave's 32 tokens (row groups 2hh, 2hh+1) and 16 heads
    f32x4_t s[2];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      s[mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKt; ++ks) s[mm] = mfma_bf16(lds_k<kDsaDqk>(kt, 2 * hh + mm, ks, lane), qf[ks], s[mm]);
    }
    float z[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = kTileTok * it + 32 * hh + 16 * mm + 4 * lg + i;  // token index within the split
        z[mm][i] = t0 + tt < t1 ? s[mm][i] * sc : -INFINITY;
        mx = fmaxf(mx, z[mm][i]);
      }
    mx = max_over_groups_swap(mx);  // head lr over the wave's 32 tokens
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
        const int R = 32 * hh + step_key(lg, rr);
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(kt + (((R >> 4) * kKt + ks) * 64 + lgc * 16 + (R & 15)) * 16);
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

  // merge the two token halves of each head tile through LDS, write the partial
  float* xm = reinterpret_cast<float*>(s_buf[0]) + jt * (16 * 514);  // [16 heads][m, l, 512]
  if (hh == 1) {
    if (lg == 0) {
      xm[lr * 514] = mref;
      xm[lr * 514 + 1] = lsum;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
#pragma unroll
        for (int i = 0; i < 4; ++i) xm[lr * 514 + 2 + 128 * db + acc_channel<128>(lg, i, jj)] = acc[db][jj][i];
  }
  lds_barrier();
  if (hh == 0) {
    const float m1 = xm[lr * 514], l1 = xm[lr * 514 + 1];
    const float M = fmaxf(mref, m1);
    const float a0 = mref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref - M);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
    float* dst = part + (size_t)(16 * jt + lr) * kPartStride;
    if (lg == 0) {
      dst[0] = M;
      dst[1] = a0 * lsum + a1 * l1;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int ch = 128 * db + acc_channel<128>(lg, i, jj);
          v[jj] = a0 * acc[db][jj][i] + a1 * xm[lr * 514 + 2 + ch];
        }
        float* o = dst + kPartOut + 128 * db + acc_channel<128>(lg, i, 0);  // 8 consecutive channels
        *reinterpret_cast<f32x4_t*>(o) = f32x4_t{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4_t*>(o + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
      }
  }
}

// ---------------------------------------------------------------------------
// 4. exact merge of the token splits: workgroup per (sequence, head), 4 channels per thread
__global__ __launch_bounds__(128) void dsa_combine_kernel(DsaParams p) {
  const int bh = blockIdx.x, b = bh / p.H, h = bh - b * p.H;
  const int ngrp = p.H / 32, hg = h >> 5, hl = h & 31;
  const float* src = p.part + ((size_t)(b * ngrp + hg) * p.ts * 32 + hl) * kPartStride;
  const size_t sstep = (size_t)32 * kPartStride;
  float M = -INFINITY;
  for (int s = 0; s < p.ts; ++s) M = fmaxf(M, src[s * sstep]);
  float Ls = 0.f;
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
  const int c = 4 * threadIdx.x;
  for (int s = 0; s < p.ts; ++s) {
    const float m = src[s * sstep];
    if (m == -INFINITY) continue;
    const float a = __builtin_amdgcn_exp2f(m - M);
    Ls += a * src[s * sstep + 1];
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src + s * sstep + kPartOut + c);
    o = f32x4_t{o[0] + a * v[0], o[1] + a * v[1], o[2] + a * v[2], o[3] + a * v[3]};
  }
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
  hipLaunchKernelGGL(dsa_select_kernel, dim3((unsigned)p.B), dim3(kDsaSelThreads), 0, s, p);
  if (ev) (void)hipEventRecord(ev->ev[2], s);
  hipLaunchKernelGGL(dsa_attn_kernel, dim3((unsigned)(p.B * (p.H / 32) * p.ts)), dim3(256), 0, s, p);
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

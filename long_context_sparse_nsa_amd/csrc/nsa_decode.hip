// NSA decode step on gfx950: two launches per step.
//
// Pass 1 (decode_cmp_kernel): the compressed branch, split over chunks of 256
//   compressed keys per (sequence, KV group).  Each workgroup streams its chunk
//   of the compressed cache once, computes the 16-head logits with MFMA, the
//   chunk-local softmax statistics, the partial output, and the per-head
//   probabilities folded onto selection blocks.  The last workgroup of a
//   (sequence, group) — found with a device-scope counter — merges the chunks
//   exactly (per-head max / sum rescaling), writes the gated compressed output,
//   sums the folded scores over the group's heads and runs the top-n.
// Pass 2 (decode_sw_kernel): the selected blocks and the window blocks, as one
//   sorted union so every token is read once; each token's logit feeds the
//   selected-branch softmax if its block was selected and the window softmax if
//   it lies in the last w tokens.  The last workgroup merges the partials and
//   writes out = g_cmp*o_cmp + g_slc*o_slc + g_win*o_win in bf16.
//
// Sources: lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc),
// section "NSA: три ветви" (output equation; compressed branch l=32, d=16;
// selection of n l'-blocks re-using the compressed-branch weights, shared by a
// GQA group so each KV block is read once per group; window of w tokens) and
// section "Сколько это экономит" (decode is bound by reading the KV cache).
#include <hip/hip_runtime.h>

#include "nsa_device.hpp"
#include "nsa_internal.hpp"
#include "nsa_tiles.hpp"
#include "nsa_topn.hpp"

namespace nsa {

namespace {

__device__ __forceinline__ int64_t raw_row0(const DecodeParams& p, int b, int g) {
  if (p.cu) {
    const int64_t c0 = p.cu[b], c1 = p.cu[b + 1];
    return (int64_t)p.H * c0 + (int64_t)g * (c1 - c0);
  }
  return ((int64_t)b * p.H + g) * p.cap;
}

__device__ __forceinline__ int64_t cmp_row0(const DecodeParams& p, int b, int g) {
  if (p.cuc) {
    const int64_t c0 = p.cuc[b], c1 = p.cuc[b + 1];
    return (int64_t)p.H * c0 + (int64_t)g * (c1 - c0);
  }
  return ((int64_t)b * p.H + g) * p.ccap;
}

// Tokens present in sequence b, clamped to [1, capacity] so that inconsistent
// device-side lengths can never move an access outside the caller's buffers.
__device__ __forceinline__ int seq_len_clamped(const DecodeParams& p, int b) {
  int64_t cap = p.cap;
  if (p.cu) {
    const int64_t c = p.cu[b + 1] - p.cu[b];
    if (c < cap) cap = c;
  }
  int64_t L = p.seq_lens[b];
  if (L > cap) L = cap;
  if (L < 1) L = 1;
  return (int)L;
}

// Complete compressed blocks among L tokens, clamped to the compressed capacity.
__device__ __forceinline__ int n_visible(const DecodeParams& p, int b, int L) {
  int64_t nv = L >= p.l ? (L - p.l) / p.d + 1 : 0;
  const int64_t ccap = p.cuc ? p.cuc[b + 1] - p.cuc[b] : p.ccap;
  return (int)(nv < ccap ? nv : ccap);
}

// LDS budget of pass 1, in floats (compute phase and merge phase share it).
template <int DV>
struct K1Smem {
  static constexpr int kP = 16 * (kChunk + 4);          // probabilities for the fold
  static constexpr int kAcc = 4 * 16 * (DV + 1);        // per-wave partial outputs
  static constexpr int kRed = 128;                      // per-wave max / sum
  static constexpr int kCompute = kP + kAcc + kRed;
  static constexpr int kMerge = kMaxBlocks + kMaxChunks * 16 + kMaxBlocks / 4 + sizeof(TopnSmem) / 4 + 8;
  static constexpr int kFloats = kCompute > kMerge ? kCompute : kMerge;
};

}  // namespace

template <int DK, int DV>
__global__ __launch_bounds__(256) void decode_cmp_kernel(DecodeParams p) {
  constexpr int KT = DK / 32, VC = DV / 16, VW = DV / 32;
  using SM = K1Smem<DV>;
  __shared__ float smem[SM::kFloats];
  __shared__ int s_last;

  const int nch = p.nch;
  const int c = blockIdx.x % nch;
  const int bg = blockIdx.x / nch;
  const int g = bg % p.H, b = bg / p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;

  const int L = seq_len_clamped(p, b);
  const int nvis = n_visible(p, b, L);  // complete compressed blocks
  const int nch_b = (nvis + kChunk - 1) / kChunk;

  if (c < nch_b) {
    float* s_p = smem;
    float* s_acc = smem + SM::kP;
    float* s_red = s_acc + SM::kAcc;
    const int64_t crow = cmp_row0(p, b, g);
    const uint16_t* kc = p.kc + crow * DK;
    const uint16_t* vc = p.vc + crow * DV;
    const int key0 = c * kChunk + wave * 64;

    u32x4_t qf[KT];
    load_q_frags<DK>(p.q + ((int64_t)b * p.Hq + (int64_t)g * p.G) * DK, p.G, lg, lr, qf);
    u32x4_t kf[4][KT];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) load_k_tile<DK>(kc, key0 + 16 * tt + lr, nvis, lg, kf[tt]);
    uint32_t vr[2][8][VW];
#pragma unroll
    for (int s = 0; s < 2; ++s) load_v_step<DV>(vc, key0 + 32 * s, nvis, lg, lr, vr[s]);

    float z[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const f32x4_t st = qk_tile<DK>(kf[tt], qf);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + 16 * tt + 4 * lg + i;
        const float v = key < nvis ? st[i] * p.scale_log2 : -INFINITY;
        z[tt][i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = max_over_groups(mx);
    if (lg == 0) s_red[wave * 16 + lr] = mx;
    __syncthreads();
    // chunk max per head; finite because key c*kChunk (wave 0) is visible
    const float m = fmaxf(fmaxf(s_red[lr], s_red[16 + lr]), fmaxf(s_red[32 + lr], s_red[48 + lr]));
    float ls = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp2f(z[tt][i] - m);
        z[tt][i] = e;
        ls += e;
        s_p[lr * (kChunk + 4) + wave * 64 + 16 * tt + 4 * lg + i] = e;
      }
    ls = sum_over_groups(ls);
    if (lg == 0) s_red[64 + wave * 16 + lr] = ls;

    f32x4_t acc[VC];
#pragma unroll
    for (int j = 0; j < VC; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) pv_step<DV>(vr[s], pack_probs(z[2 * s], z[2 * s + 1]), acc);
#pragma unroll
    for (int j = 0; j < VC; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_acc[(wave * 16 + lr) * (DV + 1) + acc_channel<DV>(lg, i, j)] = acc[j][i];
    __syncthreads();

    // chunk partial output [16][DV] (sum over the 4 waves, same reference max)
    float* O = p.o1 + ((size_t)bg * nch + c) * 16 * DV;
    for (int e = tid; e < 16 * DV; e += 256) {
      const int h = e / DV, ch = e - h * DV;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v += s_acc[(w * 16 + h) * (DV + 1) + ch];
      O[e] = v;
    }
    if (tid < 16) {
      p.m1[((size_t)bg * nch + c) * 16 + tid] = m;
      p.l1[((size_t)bg * nch + c) * 16 + tid] =
          s_red[64 + tid] + s_red[80 + tid] + s_red[96 + tid] + s_red[112 + tid];
    }
    // per-head scores of the selection blocks this chunk touches:
    // slot jj is block jb0 + jj; slot nbo receives the overhang of the last keys.
    const int nbo = p.nbo, slots = nbo + 1;
    const int64_t jb0 = (int64_t)c * kChunk * p.d / p.lsel;
    const int kc0 = c * kChunk, kc1 = min(kc0 + kChunk, nvis);
    float* SC = p.sc1 + ((size_t)bg * nch + c) * 16 * slots;
    const float inv_l = 1.0f / (float)p.l;
    for (int e = tid; e < 16 * slots; e += 256) {
      const int h = e / slots, jj = e - h * slots;
      const int64_t j = jb0 + jj;
      const int64_t lo_tok = j * p.lsel, hi_tok = lo_tok + p.lsel;  // block j = [lo, hi)
      const int64_t a = lo_tok - p.l;
      int64_t ilo = a < 0 ? 0 : a / p.d + 1;  // first key with i*d + l > lo
      if (ilo < kc0) ilo = kc0;
      int64_t ihi = (hi_tok - 1) / p.d;       // last key with i*d < hi
      if (ihi > kc1 - 1) ihi = kc1 - 1;
      float s = 0.f;
      for (int64_t i = ilo; i <= ihi; ++i) {
        const int64_t x0 = i * p.d;
        const int64_t ov = min(x0 + p.l, hi_tok) - max(x0, lo_tok);
        s += (float)ov * s_p[h * (kChunk + 4) + (int)(i - kc0)];
      }
      SC[e] = s * inv_l;
    }
  }

  // ---- last workgroup of this (sequence, group) merges the chunks
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&p.cnt1[bg], 1u) == (unsigned)(nch - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (tid == 0) p.cnt1[bg] = 0u;

  float* S = smem;
  float* f = S + kMaxBlocks;
  uint8_t* flag = reinterpret_cast<uint8_t*>(f + kMaxChunks * 16);
  TopnSmem& tsm = *reinterpret_cast<TopnSmem*>(flag + kMaxBlocks);

  const int t = L - 1;
  const int J = t / p.lsel;
  const size_t cbase = (size_t)bg * nch;
  if (tid < 16) {
    float M = -INFINITY;
    for (int cc = 0; cc < nch_b; ++cc) M = fmaxf(M, p.m1[(cbase + cc) * 16 + tid]);
    float Ls = 0.f;
    for (int cc = 0; cc < nch_b; ++cc) Ls += p.l1[(cbase + cc) * 16 + tid] * exp2f(p.m1[(cbase + cc) * 16 + tid] - M);
    const float inv = Ls > 0.f ? 1.0f / Ls : 0.f;
    for (int cc = 0; cc < nch_b; ++cc)
      f[cc * 16 + tid] = tid < p.G ? exp2f(p.m1[(cbase + cc) * 16 + tid] - M) * inv : 0.f;
  }
  __syncthreads();
  // gated compressed-branch output (zero when no block is complete yet)
  float* oc = p.ocmp + (size_t)bg * 16 * DV;
  for (int e = tid; e < 16 * DV; e += 256) {
    const int h = e / DV;
    float a = 0.f;
    for (int cc = 0; cc < nch_b; ++cc) a += f[cc * 16 + h] * p.o1[(cbase + cc) * 16 * DV + e];
    const float gt = h < p.G ? p.gates[((int64_t)b * p.Hq + (int64_t)g * p.G + h) * 3 + 0] : 0.f;
    oc[e] = gt * a;
  }
  // group scores of candidate blocks 0..J
  const int nbo = p.nbo, slots = nbo + 1;
  for (int j = tid; j <= J; j += 256) {
    const int cc = j / nbo, jj = j - cc * nbo;
    float s = 0.f;
    if (cc < nch_b) {
      const float* SC = p.sc1 + (cbase + cc) * 16 * slots;
      for (int h = 0; h < p.G; ++h) s += f[cc * 16 + h] * SC[h * slots + jj];
    }
    if (jj == 0 && cc >= 1 && cc - 1 < nch_b) {
      const float* SC = p.sc1 + (cbase + cc - 1) * 16 * slots;
      for (int h = 0; h < p.G; ++h) s += f[(cc - 1) * 16 + h] * SC[h * slots + nbo];
    }
    S[j] = s;
  }
  __syncthreads();
  block_topn(S, J, p.n, p.nloc, p.finit, flag, tsm, p.sel + (size_t)bg * p.n,
             p.sel_out ? p.sel_out + (size_t)bg * p.n : nullptr);
}

// LDS budget of pass 2 in floats.
template <int DV>
struct K2Smem {
  static constexpr int kAcc = 4 * 16 * (DV + 1);
  static constexpr int kStat = 4 * 4 * 16;  // [grp m/l][wave][head]
  static constexpr int kFac = 2 * 64 * 16;  // final merge factors
  static constexpr int kFloats = (kAcc + kStat) > kFac ? (kAcc + kStat) : kFac;
};

template <int DK, int DV, int LSEL>
__global__ __launch_bounds__(256) void decode_sw_kernel(DecodeParams p) {
  constexpr int KT = DK / 32, VC = DV / 16, VW = DV / 32;
  constexpr int NT = LSEL / 16, NS = (NT + 1) / 2;
  constexpr int PSTRIDE = 32 + 16 * DV;  // one branch partial: m[16], l[16], o[16][DV]
  using SM = K2Smem<DV>;
  __shared__ float smem[SM::kFloats];
  __shared__ int s_items[kMaxUnion];
  __shared__ uint8_t s_insel[kMaxUnion];
  __shared__ int s_nitems;
  __shared__ int s_last;

  const int nw2 = p.nw2;
  const int wg = blockIdx.x % nw2;
  const int bg = blockIdx.x / nw2;
  const int g = bg % p.H, b = bg / p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;

  const int L = seq_len_clamped(p, b);
  const int t = L - 1;
  const int J = t / LSEL;
  const int wlo = t - p.w + 1 > 0 ? t - p.w + 1 : 0;  // first window token
  const int jw0 = wlo / LSEL;

  if (tid == 0) {  // sorted union of the selected blocks and the window blocks
    const int32_t* sel = p.sel + (size_t)bg * p.n;
    int a = 0, cnt = 0, jw = jw0;
    while (true) {
      const int sa = (a < p.n && sel[a] >= 0) ? sel[a] : INT32_MAX;
      const int sb = jw <= J ? jw : INT32_MAX;
      if (sa == INT32_MAX && sb == INT32_MAX) break;
      const int j = sa < sb ? sa : sb;
      if (cnt < kMaxUnion) {
        s_items[cnt] = j;
        s_insel[cnt] = (uint8_t)(sa == j);
      }
      ++cnt;
      if (sa == j) ++a;
      if (sb == j) ++jw;
    }
    s_nitems = cnt < kMaxUnion ? cnt : kMaxUnion;
  }
  __syncthreads();

  float m_s = -INFINITY, l_s = 0.f, m_w = -INFINITY, l_w = 0.f;
  f32x4_t accS[VC], accW[VC];
#pragma unroll
  for (int j = 0; j < VC; ++j) accS[j] = accW[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int item = wg * 4 + wave;
  if (item < s_nitems) {
    const int jblk = s_items[item];
    const bool insel = s_insel[item] != 0;
    const int64_t x0 = (int64_t)jblk * LSEL;
    const int64_t row = raw_row0(p, b, g);
    const uint16_t* kb = p.k + row * DK;
    const uint16_t* vb = p.v + row * DV;
    const int64_t nval = min((int64_t)L, x0 + LSEL);  // tokens of this block that exist
    const bool anyW = x0 + LSEL - 1 >= wlo;

    u32x4_t qf[KT];
    load_q_frags<DK>(p.q + ((int64_t)b * p.Hq + (int64_t)g * p.G) * DK, p.G, lg, lr, qf);
    u32x4_t kf[NT][KT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) load_k_tile<DK>(kb, x0 + 16 * tt + lr, nval, lg, kf[tt]);
    uint32_t vr[NS][8][VW];
#pragma unroll
    for (int s = 0; s < NS; ++s) load_v_step<DV>(vb, x0 + 32 * s, nval, lg, lr, vr[s]);

    float zs[2 * NS][4], zw[2 * NS][4];
    float mxs = -INFINITY, mxw = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2 * NS; ++tt) {
      f32x4_t st = {0.f, 0.f, 0.f, 0.f};
      if (tt < NT) st = qk_tile<DK>(kf[tt < NT ? tt : 0], qf);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t x = x0 + 16 * tt + 4 * lg + i;
        const bool valid = tt < NT && x <= t;
        const float z = st[i] * p.scale_log2;
        zs[tt][i] = (valid && insel) ? z : -INFINITY;
        zw[tt][i] = (valid && x >= wlo) ? z : -INFINITY;
        mxs = fmaxf(mxs, zs[tt][i]);
        mxw = fmaxf(mxw, zw[tt][i]);
      }
    }
    m_s = max_over_groups(mxs);
    m_w = max_over_groups(mxw);
    if (insel) {
#pragma unroll
      for (int tt = 0; tt < 2 * NS; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = exp2f(zs[tt][i] - m_s);
          zs[tt][i] = e;
          l_s += e;
        }
      l_s = sum_over_groups(l_s);
#pragma unroll
      for (int s = 0; s < NS; ++s) pv_step<DV>(vr[s], pack_probs(zs[2 * s], zs[2 * s + 1]), accS);
    }
    if (anyW) {
#pragma unroll
      for (int tt = 0; tt < 2 * NS; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = exp2f(zw[tt][i] - m_w);
          zw[tt][i] = e;
          l_w += e;
        }
      l_w = sum_over_groups(l_w);
#pragma unroll
      for (int s = 0; s < NS; ++s) pv_step<DV>(vr[s], pack_probs(zw[2 * s], zw[2 * s + 1]), accW);
    }
  }

  // ---- workgroup merge of the 4 waves, per branch, then the partial to memory
  float* s_acc = smem;
  float* s_st = smem + SM::kAcc;  // [grp*2 + (0:m,1:l)][wave][16]
  if (lg == 0) {
    s_st[(0 * 4 + wave) * 16 + lr] = m_s;
    s_st[(1 * 4 + wave) * 16 + lr] = l_s;
    s_st[(2 * 4 + wave) * 16 + lr] = m_w;
    s_st[(3 * 4 + wave) * 16 + lr] = l_w;
  }
  float* part = p.part2 + ((size_t)bg * nw2 + wg) * 2 * PSTRIDE;
  for (int grp = 0; grp < 2; ++grp) {
#pragma unroll
    for (int j = 0; j < VC; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s_acc[(wave * 16 + lr) * (DV + 1) + acc_channel<DV>(lg, i, j)] = grp == 0 ? accS[j][i] : accW[j][i];
    __syncthreads();
    float* pp = part + grp * PSTRIDE;
    for (int e = tid; e < 16 * DV; e += 256) {
      const int h = e / DV, ch = e - h * DV;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, s_st[(grp * 2 * 4 + w) * 16 + h]);
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = s_st[(grp * 2 * 4 + w) * 16 + h];
        if (mw != -INFINITY) v += exp2f(mw - M) * s_acc[(w * 16 + h) * (DV + 1) + ch];
      }
      pp[32 + e] = v;
    }
    if (tid < 16) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, s_st[(grp * 2 * 4 + w) * 16 + tid]);
      float ls = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = s_st[(grp * 2 * 4 + w) * 16 + tid];
        if (mw != -INFINITY) ls += exp2f(mw - M) * s_st[((grp * 2 + 1) * 4 + w) * 16 + tid];
      }
      pp[tid] = M;
      pp[16 + tid] = ls;
    }
    __syncthreads();
  }

  // ---- last workgroup: merge all partials and apply the gates
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&p.cnt2[bg], 1u) == (unsigned)(nw2 - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (tid == 0) p.cnt2[bg] = 0u;

  float* fac = smem;  // [grp][wg][16]
  const float* pall = p.part2 + (size_t)bg * nw2 * 2 * PSTRIDE;
  if (tid < 32) {
    const int grp = tid >> 4, h = tid & 15;
    float M = -INFINITY;
    for (int w2 = 0; w2 < nw2; ++w2) M = fmaxf(M, pall[(w2 * 2 + grp) * PSTRIDE + h]);
    float ls = 0.f;
    for (int w2 = 0; w2 < nw2; ++w2) {
      const float mw = pall[(w2 * 2 + grp) * PSTRIDE + h];
      if (mw != -INFINITY) ls += exp2f(mw - M) * pall[(w2 * 2 + grp) * PSTRIDE + 16 + h];
    }
    const float inv = ls > 0.f ? 1.0f / ls : 0.f;
    for (int w2 = 0; w2 < nw2; ++w2) {
      const float mw = pall[(w2 * 2 + grp) * PSTRIDE + h];
      fac[(grp * nw2 + w2) * 16 + h] = mw != -INFINITY ? exp2f(mw - M) * inv : 0.f;
    }
  }
  __syncthreads();
  const float* oc = p.ocmp + (size_t)bg * 16 * DV;
  for (int e = tid; e < p.G * DV; e += 256) {
    const int h = e / DV;
    float os = 0.f, ow = 0.f;
    for (int w2 = 0; w2 < nw2; ++w2) {
      os += fac[(0 * nw2 + w2) * 16 + h] * pall[(w2 * 2 + 0) * PSTRIDE + 32 + e];
      ow += fac[(1 * nw2 + w2) * 16 + h] * pall[(w2 * 2 + 1) * PSTRIDE + 32 + e];
    }
    const int64_t qh = (int64_t)b * p.Hq + (int64_t)g * p.G + h;
    const float r = oc[e] + p.gates[qh * 3 + 1] * os + p.gates[qh * 3 + 2] * ow;
    p.out[qh * DV + (e - h * DV)] = (uint16_t)f32_to_bf16(r);
  }
}

// ---------------------------------------------------------------- host side

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeLayout decode_layout(int B, int H, int DV, int l, int d, int lsel, int n, int w, int64_t max_len) {
  DecodeLayout lay{};
  const int64_t nc = max_len >= l ? (max_len - l) / d + 1 : 0;
  lay.nch = (int)((nc + kChunk - 1) / kChunk);
  if (lay.nch < 1) lay.nch = 1;
  lay.nbo = (int)((int64_t)kChunk * d / lsel);
  const int umax = n + (w + lsel - 1) / lsel + 1;
  lay.nw2 = (umax + 3) / 4;
  const size_t BH = (size_t)B * H;
  size_t off = 0;
  lay.off_cnt1 = off; off = align256(off + BH * 4);
  lay.off_cnt2 = off; off = align256(off + BH * 4);
  lay.off_m1 = off;   off = align256(off + BH * lay.nch * 16 * 4);
  lay.off_l1 = off;   off = align256(off + BH * lay.nch * 16 * 4);
  lay.off_o1 = off;   off = align256(off + BH * lay.nch * 16 * (size_t)DV * 4);
  lay.off_sc1 = off;  off = align256(off + BH * lay.nch * 16 * (size_t)(lay.nbo + 1) * 4);
  lay.off_ocmp = off; off = align256(off + BH * 16 * (size_t)DV * 4);
  lay.off_sel = off;  off = align256(off + BH * (size_t)n * 4);
  lay.off_part2 = off; off = align256(off + BH * lay.nw2 * 2 * (32 + 16 * (size_t)DV) * 4);
  lay.total = off;
  return lay;
}

template <int DK, int DV>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
  const dim3 blk(256);
  hipLaunchKernelGGL((decode_cmp_kernel<DK, DV>), dim3((unsigned)(p.B * p.H * p.nch)), blk, 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2((unsigned)(p.B * p.H * p.nw2));
  switch (p.lsel) {
    case 16: hipLaunchKernelGGL((decode_sw_kernel<DK, DV, 16>), g2, blk, 0, s, p); break;
    case 32: hipLaunchKernelGGL((decode_sw_kernel<DK, DV, 32>), g2, blk, 0, s, p); break;
    case 64: hipLaunchKernelGGL((decode_sw_kernel<DK, DV, 64>), g2, blk, 0, s, p); break;
    case 128: hipLaunchKernelGGL((decode_sw_kernel<DK, DV, 128>), g2, blk, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int DK, int DV, hipStream_t s) {
  if (DK == 192 && DV == 128) return launch_decode_t<192, 128>(p, s);
  if (DK == 128 && DV == 128) return launch_decode_t<128, 128>(p, s);
  if (DK == 64 && DV == 64) return launch_decode_t<64, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace nsa

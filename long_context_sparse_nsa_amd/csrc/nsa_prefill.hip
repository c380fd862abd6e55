// NSA causal prefill on gfx950: one workgroup per (sequence, position t, KV group).
//
// Compressed branch in two exact passes over the blocks visible at t:
//   pass 1: logits (MFMA) -> per-head running max / sum -> exact normaliser;
//   pass 2: logits again -> normalised probabilities p -> o_cmp += p.Vc and the
//           probabilities summed over the group's heads and folded onto
//           selection blocks (token overlap / l), kept per 64-key slice in LDS
//           and added up in slice order (deterministic).
// Then the block-wide top-n, and the selected and window branches over the
// sorted union of their blocks (each token's logit feeds the branch softmaxes it
// belongs to), and the gated sum written in bf16.
//
// Sources: lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc),
// section "NSA: три ветви" (output equation, the three branches, selection per
// GQA group); lesson "Native Sparse Attention (DeepSeek NSA)" (AI Engineering
// from Scratch, phase 10 · 17), "Build it" steps 2-5.
#include <hip/hip_runtime.h>

#include "nsa_device.hpp"
#include "nsa_internal.hpp"
#include "nsa_tiles.hpp"
#include "nsa_topn.hpp"

namespace nsa {

// Prefill limits (checked by the host): slices of 64 compressed keys, per-slice
// fold slots, candidate blocks.
constexpr int kPfMaxSlices = 64;     // Nc <= 4096
constexpr int kPfMaxSlots = 72;      // selection blocks touched by one 64-key slice
constexpr int kPfMaxBlocks = 4096;   // J+1

template <int DV>
struct PfSmem {
  static constexpr int kStage = 4 * 16 * 65;                 // per-wave p staging [wave][h][64(+1)]
  static constexpr int kPsum = 4 * 64;
  static constexpr int kFold = kPfMaxSlices * kPfMaxSlots;   // per-slice block contributions
  static constexpr int kS = kPfMaxBlocks;
  static constexpr int kFlag = kPfMaxBlocks / 4;
  static constexpr int kTopn = sizeof(TopnSmem) / 4 + 4;
  static constexpr int kStat = 4 * 4 * 16;
  static constexpr int kPhaseA = kStage + kPsum + kFold + kS + kFlag + kTopn + kStat;
  static constexpr int kAcc = 4 * 16 * (DV + 1);
  static constexpr int kFloats = kPhaseA > kAcc + kStat ? kPhaseA : kAcc + kStat;
};

template <int DK, int DV, int LSEL>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams p) {
  constexpr int KT = DK / 32, VC = DV / 16, VW = DV / 32;
  constexpr int NT = LSEL / 16, NS = (NT + 1) / 2;
  using SM = PfSmem<DV>;
  __shared__ float smem[SM::kFloats];
  __shared__ int s_sel[kMaxSel];
  __shared__ int s_items[kMaxUnion];
  __shared__ uint8_t s_insel[kMaxUnion];
  __shared__ int s_nitems;

  // grid order: (b, g) outer, t inner, so workgroups running together share the
  // group's compressed cache and window in L2
  const int64_t bid = blockIdx.x;
  const int t = (int)(bid % p.T);
  const int bg = (int)(bid / p.T);
  const int g = bg % p.H, b = bg / p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;

  float* s_stage = smem;
  float* s_psum = s_stage + SM::kStage;
  float* s_fold = s_psum + SM::kPsum;
  float* S = s_fold + SM::kFold;
  uint8_t* flag = reinterpret_cast<uint8_t*>(S + SM::kS);
  TopnSmem& tsm = *reinterpret_cast<TopnSmem*>(S + SM::kS + SM::kFlag);
  float* s_stat = S + SM::kS + SM::kFlag + SM::kTopn;  // [4][4][16]

  const int64_t qrow = ((int64_t)b * p.T + t) * p.Hq + (int64_t)g * p.G;
  u32x4_t qf[KT];
  load_q_frags<DK>(p.q + qrow * DK, p.G, lg, lr, qf);

  const int nvis = t + 1 >= p.l ? (t + 1 - p.l) / p.d + 1 : 0;
  const int nsl = (nvis + 63) / 64;
  const int rounds = (nsl + 3) / 4;
  const int64_t crow = ((int64_t)b * p.H + g) * p.nc;
  const uint16_t* kc = p.kc + crow * DK;
  const uint16_t* vc = p.vc + crow * DV;

  // ---- pass 1: exact per-head normaliser of the compressed branch
  float m_run = -INFINITY, l_run = 0.f;
  for (int r = 0; r < rounds; ++r) {
    const int sl = 4 * r + wave;
    if (sl < nsl) {
      const int key0 = sl * 64;
      u32x4_t kf[4][KT];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) load_k_tile<DK>(kc, key0 + 16 * tt + lr, nvis, lg, kf[tt]);
      float z[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const f32x4_t st = qk_tile<DK>(kf[tt], qf);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 16 * tt + 4 * lg + i;
          z[tt][i] = key < nvis ? st[i] * p.scale_log2 : -INFINITY;
          mx = fmaxf(mx, z[tt][i]);
        }
      }
      mx = max_over_groups(mx);
      const float mn = fmaxf(m_run, mx);
      float ls = 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) ls += exp2f(z[tt][i] - mn);
      ls = sum_over_groups(ls);
      l_run = (m_run == -INFINITY ? 0.f : l_run * exp2f(m_run - mn)) + ls;
      m_run = mn;
    }
  }
  if (lg == 0) {
    s_stat[(0 * 4 + wave) * 16 + lr] = m_run;
    s_stat[(1 * 4 + wave) * 16 + lr] = l_run;
  }
  __syncthreads();
  float Mh = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) Mh = fmaxf(Mh, s_stat[(0 * 4 + w) * 16 + lr]);
  float Lh = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = s_stat[(0 * 4 + w) * 16 + lr];
    if (mw != -INFINITY) Lh += exp2f(mw - Mh) * s_stat[(1 * 4 + w) * 16 + lr];
  }
  const float invL = Lh > 0.f ? 1.0f / Lh : 0.f;
  __syncthreads();

  // ---- pass 2: normalised probabilities, o_cmp, folded group scores per slice
  const int nbs = (63 * p.d + p.l - 1) / p.lsel + 2;  // slots per slice (host checks <= kPfMaxSlots)
  f32x4_t accC[VC];
#pragma unroll
  for (int j = 0; j < VC; ++j) accC[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float* stg = s_stage + wave * 16 * 65;
  float* psum = s_psum + wave * 64;
  for (int r = 0; r < rounds; ++r) {
    const int sl = 4 * r + wave;
    if (sl < nsl) {
      const int key0 = sl * 64;
      u32x4_t kf[4][KT];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) load_k_tile<DK>(kc, key0 + 16 * tt + lr, nvis, lg, kf[tt]);
      uint32_t vr[2][8][VW];
#pragma unroll
      for (int s = 0; s < 2; ++s) load_v_step<DV>(vc, key0 + 32 * s, nvis, lg, lr, vr[s]);
      float z[4][4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const f32x4_t st = qk_tile<DK>(kf[tt], qf);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 16 * tt + 4 * lg + i;
          const float e = key < nvis ? exp2f(st[i] * p.scale_log2 - Mh) * invL : 0.f;
          z[tt][i] = e;
          stg[lr * 65 + 16 * tt + 4 * lg + i] = e;
        }
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) pv_step<DV>(vr[s], pack_probs(z[2 * s], z[2 * s + 1]), accC);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      {  // sum over the group's heads, one key per lane
        float sum = 0.f;
        for (int h = 0; h < p.G; ++h) sum += stg[h * 65 + lane];
        psum[lane] = sum;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      {  // fold onto the selection blocks this slice touches (units of the stride d:
         // key i covers [i, i+q), block j covers [j*r, (j+1)*r))
        const int q = p.l / p.d, r = p.lsel / p.d;
        const int jlo = key0 / r;
        const int kend = min(key0 + 64, nvis);
        if (lane < nbs) {
          const int lo = (jlo + lane) * r, hi = lo + r;
          const int ilo = max(key0, lo - q + 1), ihi = min(kend - 1, hi - 1);
          float s = 0.f;
          for (int i = ilo; i <= ihi; ++i) s += (float)(min(i + q, hi) - max(i, lo)) * psum[i - key0];
          s_fold[sl * kPfMaxSlots + lane] = s * (1.0f / (float)q);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  __syncthreads();

  // ---- group scores of candidates 0..J (slice contributions added in slice order)
  const int J = t / LSEL;
  {
    const int q = p.l / p.d, r = p.lsel / p.d;
    for (int j = tid; j <= J; j += 256) {
      float s = 0.f;
      const int ilo = max(0, j * r - q + 1), ihi = min(nvis - 1, (j + 1) * r - 1);
      if (ilo <= ihi) {
        for (int sl = ilo / 64; sl <= ihi / 64; ++sl) s += s_fold[sl * kPfMaxSlots + (j - sl * 64 / r)];
      }
      S[j] = s;
    }
  }
  __syncthreads();
  int32_t* selg = p.sel_out ? p.sel_out + (((int64_t)b * p.T + t) * p.H + g) * p.n : nullptr;
  block_topn<256, 16>(S, J, p.n, p.nloc, p.finit, tsm, s_sel, selg);
  __syncthreads();

  // ---- selected and window branches over the sorted union of their blocks
  const int wlo = t - p.w + 1 > 0 ? t - p.w + 1 : 0;
  const int jw0 = wlo / LSEL;
  if (tid == 0) {
    int a = 0, cnt = 0, jw = jw0;
    while (true) {
      const int sa = (a < p.n && s_sel[a] >= 0) ? s_sel[a] : INT32_MAX;
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

  const int64_t row = ((int64_t)b * p.H + g) * p.T;
  const uint16_t* kb = p.k + row * DK;
  const uint16_t* vb = p.v + row * DV;
  float m_s = -INFINITY, l_s = 0.f, m_w = -INFINITY, l_w = 0.f;
  f32x4_t accS[VC], accW[VC];
#pragma unroll
  for (int j = 0; j < VC; ++j) accS[j] = accW[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = wave; it < s_nitems; it += 4) {
    const int jblk = s_items[it];
    const bool insel = s_insel[it] != 0;
    const int64_t x0 = (int64_t)jblk * LSEL;
    const int64_t nval = min((int64_t)t + 1, x0 + LSEL);
    const bool anyW = x0 + LSEL - 1 >= wlo;
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
    if (insel) {
      mxs = max_over_groups(mxs);
      const float mn = fmaxf(m_s, mxs);
      const float alpha = m_s == -INFINITY ? 0.f : exp2f(m_s - mn);
      float ls = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2 * NS; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = exp2f(zs[tt][i] - mn);
          zs[tt][i] = e;
          ls += e;
        }
      ls = sum_over_groups(ls);
      l_s = l_s * alpha + ls;
      m_s = mn;
#pragma unroll
      for (int j = 0; j < VC; ++j) accS[j] *= alpha;
#pragma unroll
      for (int s = 0; s < NS; ++s) pv_step<DV>(vr[s], pack_probs(zs[2 * s], zs[2 * s + 1]), accS);
    }
    if (anyW) {
      mxw = max_over_groups(mxw);
      const float mn = fmaxf(m_w, mxw);
      const float alpha = m_w == -INFINITY ? 0.f : exp2f(m_w - mn);
      float ls = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2 * NS; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = exp2f(zw[tt][i] - mn);
          zw[tt][i] = e;
          ls += e;
        }
      ls = sum_over_groups(ls);
      l_w = l_w * alpha + ls;
      m_w = mn;
#pragma unroll
      for (int j = 0; j < VC; ++j) accW[j] *= alpha;
#pragma unroll
      for (int s = 0; s < NS; ++s) pv_step<DV>(vr[s], pack_probs(zw[2 * s], zw[2 * s + 1]), accW);
    }
  }

  // ---- merge the 4 waves and write the gated sum
  __syncthreads();  // LDS of phase A is reused below
  float* s_acc = smem;
  float* st2 = smem + SM::kAcc;  // [grp*2 + (m,l)][wave][16]
  if (lg == 0) {
    st2[(0 * 4 + wave) * 16 + lr] = m_s;
    st2[(1 * 4 + wave) * 16 + lr] = l_s;
    st2[(2 * 4 + wave) * 16 + lr] = m_w;
    st2[(3 * 4 + wave) * 16 + lr] = l_w;
  }
  // o_cmp: sum of the waves' exact partials
#pragma unroll
  for (int j = 0; j < VC; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_acc[(wave * 16 + lr) * (DV + 1) + acc_channel<DV>(lg, i, j)] = accC[j][i];
  __syncthreads();
  float res[(16 * DV + 255) / 256];
  {
    int q = 0;
    for (int e = tid; e < 16 * DV; e += 256, ++q) {
      const int h = e / DV, ch = e - h * DV;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v += s_acc[(w * 16 + h) * (DV + 1) + ch];
      const float gt = h < p.G ? p.gates[(((int64_t)b * p.T + t) * p.Hq + (int64_t)g * p.G + h) * 3 + 0] : 0.f;
      res[q] = gt * v;
    }
  }
  for (int grp = 0; grp < 2; ++grp) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < VC; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s_acc[(wave * 16 + lr) * (DV + 1) + acc_channel<DV>(lg, i, j)] = grp == 0 ? accS[j][i] : accW[j][i];
    __syncthreads();
    int q = 0;
    for (int e = tid; e < 16 * DV; e += 256, ++q) {
      const int h = e / DV, ch = e - h * DV;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, st2[(grp * 2 * 4 + w) * 16 + h]);
      float v = 0.f, ls = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = st2[(grp * 2 * 4 + w) * 16 + h];
        if (mw != -INFINITY) {
          const float a = exp2f(mw - M);
          v += a * s_acc[(w * 16 + h) * (DV + 1) + ch];
          ls += a * st2[((grp * 2 + 1) * 4 + w) * 16 + h];
        }
      }
      const float gt = h < p.G ? p.gates[(((int64_t)b * p.T + t) * p.Hq + (int64_t)g * p.G + h) * 3 + 1 + grp] : 0.f;
      res[q] += ls > 0.f ? gt * v / ls : 0.f;
    }
  }
  {
    int q = 0;
    for (int e = tid; e < 16 * DV; e += 256, ++q) {
      const int h = e / DV, ch = e - h * DV;
      if (h < p.G) p.out[(qrow + h) * DV + ch] = (uint16_t)f32_to_bf16(res[q]);
    }
  }
}

template <int DK, int DV>
static hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)p.B * p.H * p.T)), blk(256);
  switch (p.lsel) {
    case 16: hipLaunchKernelGGL((prefill_kernel<DK, DV, 16>), grid, blk, 0, s, p); break;
    case 32: hipLaunchKernelGGL((prefill_kernel<DK, DV, 32>), grid, blk, 0, s, p); break;
    case 64: hipLaunchKernelGGL((prefill_kernel<DK, DV, 64>), grid, blk, 0, s, p); break;
    case 128: hipLaunchKernelGGL((prefill_kernel<DK, DV, 128>), grid, blk, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int DK, int DV, hipStream_t s) {
  if (DK == 192 && DV == 128) return launch_prefill_t<192, 128>(p, s);
  if (DK == 128 && DV == 128) return launch_prefill_t<128, 128>(p, s);
  if (DK == 64 && DV == 64) return launch_prefill_t<64, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace nsa

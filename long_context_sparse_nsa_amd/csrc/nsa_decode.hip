// NSA decode step on gfx950: three launches per step; kernel boundaries are the
// only cross-workgroup synchronisation (no device-scope fences, no counters).
//
// 1. decode_cmp_kernel, two kinds of workgroups in one launch:
//    - chunk workgroups: the compressed branch, split over chunks of compressed
//      keys per (sequence, KV group).  Each streams its chunk of the compressed
//      cache once, computes the 16-head logits with MFMA, the chunk-local
//      softmax statistics, the partial output, and the per-head probabilities
//      folded onto selection blocks;
//    - window workgroups: the window branch, which does not depend on the
//      selection, as 32-token steps over the window's blocks.
// 2. decode_finish_kernel: several workgroups per (sequence, group), each
//    computing the exact per-head normalisers from the chunk statistics, the
//    group scores and the top-n, then attending its share of the selected
//    blocks (one 32-token step per wave).
// 3. decode_combine_kernel: per query head, the exact merge of every partial and
//    out = g_cmp*o_cmp + g_slc*o_slc + g_win*o_win in bf16.
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

// LDS budget of the compressed pass, in floats.
template <int DV>
struct K1Smem {
  static constexpr int kP = 16 * (kChunk + 4);             // probabilities for the fold
  static constexpr int kAcc = kCmpWaves * 16 * (DV + 1);   // per-wave partial outputs
  static constexpr int kRed = 2 * kCmpWaves * 16;          // per-wave max / sum
  static constexpr int kFloats = kP + kAcc + kRed;
};

// One 32-token step [x0, x0 + 32) of the raw cache for the group's heads.
template <int DK, int DV>
struct Step {
  u32x4_t kf[2][DK / 32];
  uint32_t vr[8][DV / 32];
};

// Tokens x < nval exist (nval already bounds x <= t and the block end).
template <int DK, int DV>
__device__ __forceinline__ void step_load(Step<DK, DV>& st, const uint16_t* kb, const uint16_t* vb, int64_t x0,
                                          int64_t nval, int lg, int lr) {
  load_k_tile<DK>(kb, x0 + lr, nval, lg, st.kf[0]);
  load_k_tile<DK>(kb, x0 + 16 + lr, nval, lg, st.kf[1]);
  load_v_step<DV>(vb, x0, nval, lg, lr, st.vr);
}

// Online-softmax state of one branch for the wave's 16 heads (head = lane % 16).
template <int DV>
struct Branch {
  float m, l;
  f32x4_t acc[DV / 16];
  __device__ __forceinline__ void init() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int j = 0; j < DV / 16; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // Fold in the step's tokens whose mask bit is set (z = -inf elsewhere).
  __device__ __forceinline__ void update(float (&z)[2][4], const uint32_t (&vr)[8][DV / 32]) {
    float mx = fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                     fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
    mx = max_over_groups(mx);
    const float mn = fmaxf(m, mx);
    const float alpha = m == -INFINITY ? 0.f : exp2f(m - mn);
    float ls = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp2f(z[tt][i] - mn);
        z[tt][i] = e;
        ls += e;
      }
    l = l * alpha + sum_over_groups(ls);
    m = mn;
#pragma unroll
    for (int j = 0; j < DV / 16; ++j) acc[j] *= alpha;
    pv_step<DV>(vr, pack_probs(z[0], z[1]), acc);
  }
};

// Logits of a step, scaled to log2 units; element (tt, i) is token x0 + 16*tt + 4*lg + i.
template <int DK, int DV>
__device__ __forceinline__ void step_logits(const Step<DK, DV>& st, const u32x4_t (&qf)[DK / 32], float scale,
                                            float (&z)[2][4]) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const f32x4_t sv = qk_tile<DK>(st.kf[tt], qf);
#pragma unroll
    for (int i = 0; i < 4; ++i) z[tt][i] = sv[i] * scale;
  }
}

// Workgroup merge of 4 waves' branch states into one partial
// (m[16], l[16], o[16][DV]) written to `dst`; `buf`/`st` are LDS scratch.
template <int DV, int NWV>
__device__ __forceinline__ void merge_waves_to(const Branch<DV>& br, float* dst, float* buf, float* st) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  constexpr int NTH = 64 * NWV;
  if (lg == 0) {
    st[wave * 16 + lr] = br.m;
    st[(NWV + wave) * 16 + lr] = br.l;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NWV; ++w) M = fmaxf(M, st[w * 16 + lr]);
  const float alpha = br.m == -INFINITY ? 0.f : exp2f(br.m - M);
#pragma unroll
  for (int j = 0; j < DV / 16; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) buf[(wave * 16 + lr) * (DV + 1) + acc_channel<DV>(lg, i, j)] = alpha * br.acc[j][i];
  __syncthreads();
  for (int e = tid; e < 16 * DV; e += NTH) {
    const int h = e / DV, ch = e - h * DV;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) v += buf[(w * 16 + h) * (DV + 1) + ch];
    dst[32 + e] = v;
  }
  if (tid < 16) {
    float Mh = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) Mh = fmaxf(Mh, st[w * 16 + tid]);
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float mw = st[w * 16 + tid];
      if (mw != -INFINITY) ls += exp2f(mw - Mh) * st[(NWV + w) * 16 + tid];
    }
    dst[tid] = Mh;
    dst[16 + tid] = ls;
  }
  __syncthreads();
}



}  // namespace

// Window workgroup wi of a (sequence, group): one 32-token step per wave over
// the window's blocks [wlo / l', J] (steps wi*4 .. wi*4+3); writes one partial
// (m[16], l[16], o[16][DV]) of the window branch.
template <int DK, int DV, int LSEL>
__device__ __forceinline__ void window_work(const DecodeParams& p, int b, int g, int bg, int wi, float* smem) {
  constexpr int KT = DK / 32, NWV = kCmpWaves;
  constexpr int SPB = LSEL >= 32 ? LSEL / 32 : 1;
  constexpr int PSTRIDE = 32 + 16 * DV;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int L = seq_len_clamped(p, b);
  const int t = L - 1;
  const int wlo = t - p.w + 1 > 0 ? t - p.w + 1 : 0;
  const int jw0 = wlo / LSEL, J = t / LSEL;
  const int nsteps = (J - jw0 + 1) * SPB;
  Branch<DV> bw;
  bw.init();
  const int si = wi * NWV + wave;
  if (si < nsteps) {
    const int it = si / SPB, half = si - it * SPB;
    const int64_t xb = (int64_t)(jw0 + it) * LSEL;
    const int64_t x0 = xb + 32 * half;
    const int64_t nv = min((int64_t)L, xb + LSEL);
    const int64_t row = raw_row0(p, b, g);
    u32x4_t qf[KT];
    load_q_frags<DK>(p.q + ((int64_t)b * p.Hq + (int64_t)g * p.G) * DK, p.G, lg, lr, qf);
    Step<DK, DV> st;
    step_load<DK, DV>(st, p.k + row * DK, p.v + row * DV, x0, nv, lg, lr);
    if (x0 < nv && x0 + 31 >= wlo) {
      float z[2][4];
      step_logits<DK, DV>(st, qf, p.scale_log2, z);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t x = x0 + 16 * tt + 4 * lg + i;
          if (!(x < nv && x >= wlo)) z[tt][i] = -INFINITY;
        }
      bw.update(z, st.vr);
    }
  }
  float* buf = smem;
  float* stt = smem + NWV * 16 * (DV + 1);
  merge_waves_to<DV, NWV>(bw, p.wpart + ((size_t)bg * p.nwin + wi) * PSTRIDE, buf, stt);
}

template <int DK, int DV, int LSEL>
__global__ __launch_bounds__(64 * kCmpWaves, 3) void decode_cmp_kernel(DecodeParams p) {
  constexpr int KT = DK / 32, VC = DV / 16, VW = DV / 32;
  constexpr int NWV = kCmpWaves, KPW = kCmpKeysPerWave, NTH = 64 * NWV;
  constexpr int TPW = KPW / 16, SPW = KPW / 32;  // 16-key tiles and 32-key steps per wave
  using SM = K1Smem<DV>;
  __shared__ float smem[SM::kFloats];

  // workgroups [0, B*H*nwin) are window workgroups (scheduled first), the rest chunks
  const int nwg_win = p.B * p.H * p.nwin;
  if ((int)blockIdx.x < nwg_win) {
    const int bgw = blockIdx.x / p.nwin;
    window_work<DK, DV, LSEL>(p, bgw / p.H, bgw % p.H, bgw, blockIdx.x - bgw * p.nwin, smem);
    return;
  }
  const int nch = p.nch;
  const int cid = blockIdx.x - nwg_win;
  const int c = cid % nch;
  const int bg = cid / nch;
  const int g = bg % p.H, b = bg / p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;

  const int L = seq_len_clamped(p, b);
  const int nvis = n_visible(p, b, L);  // complete compressed blocks
  const int nch_b = (nvis + kChunk - 1) / kChunk;
  if (c >= nch_b) return;  // uniform over the workgroup

  float* s_p = smem;
  float* s_acc = smem + SM::kP;
  float* s_red = s_acc + SM::kAcc;  // [0, NWV*16): max; [NWV*16, 2*NWV*16): sum
  const int64_t crow = cmp_row0(p, b, g);
  const uint16_t* kc = p.kc + crow * DK;
  const uint16_t* vc = p.vc + crow * DV;
  const int key0 = c * kChunk + wave * KPW;

  u32x4_t qf[KT];
  load_q_frags<DK>(p.q + ((int64_t)b * p.Hq + (int64_t)g * p.G) * DK, p.G, lg, lr, qf);
  u32x4_t kf[TPW][KT];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) load_k_tile<DK>(kc, key0 + 16 * tt + lr, nvis, lg, kf[tt]);

  float z[TPW][4];
  float mx = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
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
  float m = s_red[lr];
#pragma unroll
  for (int w = 1; w < NWV; ++w) m = fmaxf(m, s_red[w * 16 + lr]);
  float ls = 0.f;
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = exp2f(z[tt][i] - m);
      z[tt][i] = e;
      ls += e;
      s_p[lr * (kChunk + 4) + wave * KPW + 16 * tt + 4 * lg + i] = e;
    }
  ls = sum_over_groups(ls);
  if (lg == 0) s_red[(NWV + wave) * 16 + lr] = ls;

  // values are loaded after the logits (the key registers are free by then), which
  // keeps the kernel at three workgroups per CU; the other resident workgroups
  // cover the latency
  uint32_t vr[SPW][8][VW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) load_v_step<DV>(vc, key0 + 32 * s, nvis, lg, lr, vr[s]);
  f32x4_t acc[VC];
#pragma unroll
  for (int j = 0; j < VC; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < SPW; ++s) pv_step<DV>(vr[s], pack_probs(z[2 * s], z[2 * s + 1]), acc);
#pragma unroll
  for (int j = 0; j < VC; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_acc[(wave * 16 + lr) * (DV + 1) + acc_channel<DV>(lg, i, j)] = acc[j][i];
  __syncthreads();

  // chunk partial output [16][DV] (sum over the waves, same reference max)
  float* O = p.o1 + ((size_t)bg * nch + c) * 16 * DV;
  for (int e = tid; e < 16 * DV; e += NTH) {
    const int h = e / DV, ch = e - h * DV;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) v += s_acc[(w * 16 + h) * (DV + 1) + ch];
    O[e] = v;
  }
  if (tid < 16) {
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) lsum += s_red[(NWV + w) * 16 + tid];
    p.m1[((size_t)bg * nch + c) * 16 + tid] = m;
    p.l1[((size_t)bg * nch + c) * 16 + tid] = lsum;
  }
  // per-head scores of the selection blocks this chunk touches, in units of the
  // stride d (d divides l and l'): key i covers units [i, i+q), block j covers
  // [j*r, (j+1)*r) with q = l/d, r = l'/d, and the overlap share is (units)/q.
  // Slot jj is block jb0 + jj; slot nbo receives the overhang of the last keys.
  const int nbo = p.nbo, slots = nbo + 1;
  const int q = p.l / p.d, r = p.lsel / p.d;
  const int jb0 = c * kChunk / r;
  const int kc0 = c * kChunk, kc1 = min(kc0 + kChunk, nvis);
  float* SC = p.sc1 + ((size_t)bg * nch + c) * 16 * slots;
  const float inv_q = 1.0f / (float)q;
  for (int e = tid; e < 16 * slots; e += NTH) {
    const int h = e / slots, jj = e - h * slots;
    const int lo = (jb0 + jj) * r, hi = lo + r;      // block j in units
    const int ilo = max(kc0, lo - q + 1), ihi = min(kc1 - 1, hi - 1);
    const float* ps = s_p + h * (kChunk + 4) - kc0;
    float sacc = 0.f;
    for (int i = ilo; i <= ihi; ++i) sacc += (float)(min(i + q, hi) - max(i, lo)) * ps[i];
    SC[e] = sacc * inv_q;
  }
}

// Finish: nfin workgroups of 4 waves per (sequence, group).  Every one of them
// computes the exact per-head normalisers of the compressed branch, the group
// scores and the top-n (identical results, so no exchange is needed); then
// workgroup k attends the selected steps [4k, 4k+4) (one 32-token step per
// wave, over all selected blocks in ascending order) and writes one partial.
// Spreading the selected blocks over many workgroups lets their loads use many
// CUs' memory pipelines instead of one.
template <int DK, int DV, int LSEL>
__global__ __launch_bounds__(256) void decode_finish_kernel(DecodeParams p) {
  constexpr int NTH = 256, NWV = 4;
  constexpr int KT = DK / 32;
  constexpr int SPB = LSEL >= 32 ? LSEL / 32 : 1;   // 32-token steps per selection block
  constexpr int PSTRIDE = 32 + 16 * DV;
  __shared__ float S[kMaxBlocks];
  __shared__ float f[kMaxChunks * 16];
  __shared__ float s_stat[2 * kMaxChunks * 16];    // chunk m / l staging, then wave merge scratch
  __shared__ float s_ov[kMaxChunks * 16];          // overhang score slot of each chunk, per head
  __shared__ float s_buf[NWV * 16 * (DV + 1)];
  __shared__ TopnSmem tsm;
  __shared__ TopnFastSmem<NWV> tfs;
  __shared__ int s_sel[kMaxSel];
  __shared__ int s_items[kMaxSel];
  __shared__ int s_nitems;

  const int bg = blockIdx.x / p.nfin, kfin = blockIdx.x - bg * p.nfin;
  const int g = bg % p.H, b = bg / p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int nch = p.nch;
  const int L = seq_len_clamped(p, b);
  const int nvis = n_visible(p, b, L);
  const int nch_b = (nvis + kChunk - 1) / kChunk;
  const int t = L - 1;
  const int J = t / LSEL;
  const size_t cbase = (size_t)bg * nch;
  float* s_m = s_stat;
  float* s_l = s_stat + kMaxChunks * 16;

  // ---- one round of independent loads: chunk statistics, overhang slots, scores
  const int nbo = p.nbo, slots = nbo + 1;
  for (int idx = tid; idx < nch_b * 16; idx += NTH) {
    s_m[idx] = p.m1[cbase * 16 + idx];
    s_l[idx] = p.l1[cbase * 16 + idx];
    const int cc = idx >> 4, h = idx & 15;
    s_ov[idx] = h < p.G ? p.sc1[((cbase + cc) * 16 + h) * slots + nbo] : 0.f;
  }
  constexpr int RPT = 4;  // candidate blocks per thread and load round
  float vv[RPT][16];
  auto load_scores = [&](int j0) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int j = j0 + tid + NTH * r;
      const int cc = j / nbo, jj = j - cc * nbo;
      const bool ok = j <= J && cc < nch_b;
      const float* SC = p.sc1 + (cbase + (ok ? cc : 0)) * 16 * slots + jj;
#pragma unroll
      for (int h = 0; h < 16; ++h) vv[r][h] = (ok && h < p.G) ? SC[h * slots] : 0.f;
    }
  };
  load_scores(0);
  __syncthreads();
  // ---- exact per-head normalisers: thread (c, h) = (tid / 16, tid % 16), passes of
  // 32 chunks; reductions over c by shuffles in a wave and through LDS across waves
  {
    float* red = s_buf;  // [wave][16] scratch
    const int h = tid & 15, cw = tid >> 4;
    float M = -INFINITY;
    for (int c0 = 0; c0 < nch_b; c0 += NTH / 16) {
      const int c = c0 + cw;
      float m = c < nch_b ? s_m[c * 16 + h] : -INFINITY;
      m = max_over_groups(m);
      if (lg == 0) red[wave * 16 + h] = m;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < NWV; ++w) M = fmaxf(M, red[w * 16 + h]);
      __syncthreads();
    }
    float Ls = 0.f;
    for (int c0 = 0; c0 < nch_b; c0 += NTH / 16) {
      const int c = c0 + cw;
      float e = c < nch_b ? s_l[c * 16 + h] * exp2f(s_m[c * 16 + h] - M) : 0.f;
      e = sum_over_groups(e);
      if (lg == 0) red[wave * 16 + h] = e;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < NWV; ++w) Ls += red[w * 16 + h];
      __syncthreads();
    }
    const float inv = Ls > 0.f ? 1.0f / Ls : 0.f;
    for (int c = cw; c < nch_b; c += NTH / 16) {
      const float fc = h < p.G ? exp2f(s_m[c * 16 + h] - M) * inv : 0.f;
      f[c * 16 + h] = fc;
      if (kfin == 0) p.fcmp[(cbase + c) * 16 + h] = fc;  // for the combine kernel
    }
  }
  __syncthreads();

  // ---- group scores of candidate blocks 0..J, top-n
  for (int j0 = 0; j0 <= J; j0 += NTH * RPT) {
    if (j0 > 0) load_scores(j0);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int j = j0 + tid + NTH * r;
      if (j > J) continue;
      const int cc = j / nbo, jj = j - cc * nbo;
      float sc = 0.f;
      if (cc < nch_b) {
#pragma unroll
        for (int h = 0; h < 16; ++h) sc += f[cc * 16 + h] * vv[r][h];
      }
      if (jj == 0 && cc >= 1 && cc - 1 < nch_b) {  // overhang of the previous chunk
#pragma unroll
        for (int h = 0; h < 16; ++h) sc += f[(cc - 1) * 16 + h] * s_ov[(cc - 1) * 16 + h];
      }
      S[j] = sc;
    }
  }
  __syncthreads();
  block_topn_fast<NTH, 8, kMaxBlocks / NTH>(S, J, p.n, p.nloc, p.finit, tfs, tsm, s_sel,
                                            (p.sel_out && kfin == 0) ? p.sel_out + (size_t)bg * p.n : nullptr);
  __syncthreads();
  if (wave == 0) {  // the selected blocks, ascending (the list ends at the first -1)
    const int j = lane < p.n ? s_sel[lane] : -1;
    const uint64_t m = __ballot(j >= 0);
    if (j >= 0) s_items[__popcll(m & ((1ull << lane) - 1ull))] = j;
    if (lane == 0) s_nitems = __popcll(m);
  }
  __syncthreads();

  // ---- this workgroup's share of the selected steps: one 32-token step per wave
  Branch<DV> br;
  br.init();
  const int si = kfin * NWV + wave;
  if (si < s_nitems * SPB) {
    const int it = si / SPB, half = si - it * SPB;
    const int64_t xb = (int64_t)s_items[it] * LSEL;
    const int64_t x0 = xb + 32 * half;
    const int64_t nv = min((int64_t)L, xb + LSEL);
    const int64_t row = raw_row0(p, b, g);
    u32x4_t qf[KT];
    load_q_frags<DK>(p.q + ((int64_t)b * p.Hq + (int64_t)g * p.G) * DK, p.G, lg, lr, qf);
    Step<DK, DV> st;
    step_load<DK, DV>(st, p.k + row * DK, p.v + row * DV, x0, nv, lg, lr);
    if (x0 < nv) {
      float z[2][4];
      step_logits<DK, DV>(st, qf, p.scale_log2, z);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (x0 + 16 * tt + 4 * lg + i >= nv) z[tt][i] = -INFINITY;
      br.update(z, st.vr);
    }
  }
  merge_waves_to<DV, NWV>(br, p.rpart + ((size_t)bg * p.nfin + kfin) * PSTRIDE, s_buf, s_stat);
}

// Combine: one workgroup per query head, one thread per output channel.
//   o_cmp = sum_c f[c] * O_c (f from the finish kernel: exact normalised factors)
//   o_slc = exact merge of the finish workgroups' partials
//   o_win = exact merge of the window partials
//   out   = g_cmp*o_cmp + g_slc*o_slc + g_win*o_win  (bf16)
// Every partial up to the launch bounds is loaded in one round (entries beyond
// the sequence's own count are discarded by selects, never multiplied in).
template <int DV>
__global__ __launch_bounds__(DV) void decode_combine_kernel(DecodeParams p) {
  constexpr int PSTRIDE = 32 + 16 * DV;
  constexpr int kBatch = 16;
  __shared__ float s_f[kMaxChunks];
  __shared__ float s_pm[kMaxFinish], s_pl[kMaxFinish], s_wm[kMaxWindow], s_wl[kMaxWindow];
  const int qh = blockIdx.x;
  const int b = qh / p.Hq, hq = qh - b * p.Hq;
  const int g = hq / p.G, h = hq - g * p.G;
  const int bg = b * p.H + g;
  const int ch = threadIdx.x;
  const int nch = p.nch, nfin = p.nfin, nwin = p.nwin;
  const size_t cbase = (size_t)bg * nch;
  const float* wp = p.wpart + (size_t)bg * nwin * PSTRIDE;
  const float* rp = p.rpart + (size_t)bg * nfin * PSTRIDE;

  // ---- one round of loads
  const int L = seq_len_clamped(p, b);
  for (int c = ch; c < nch; c += DV) s_f[c] = p.fcmp[(cbase + c) * 16 + h];
  if (ch < nfin) {
    s_pm[ch] = rp[(size_t)ch * PSTRIDE + h];
    s_pl[ch] = rp[(size_t)ch * PSTRIDE + 16 + h];
  } else if (ch >= 32 && ch < 32 + nwin) {
    const int wi = ch - 32;
    s_wm[wi] = wp[(size_t)wi * PSTRIDE + h];
    s_wl[wi] = wp[(size_t)wi * PSTRIDE + 16 + h];
  }
  float vo[kBatch], vr[kMaxFinish], vw[kMaxWindow];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) vo[u] = u < nch ? p.o1[((cbase + u) * 16 + h) * DV + ch] : 0.f;
#pragma unroll
  for (int k = 0; k < kMaxFinish; ++k) vr[k] = k < nfin ? rp[(size_t)k * PSTRIDE + 32 + h * DV + ch] : 0.f;
#pragma unroll
  for (int k = 0; k < kMaxWindow; ++k) vw[k] = k < nwin ? wp[(size_t)k * PSTRIDE + 32 + h * DV + ch] : 0.f;
  const float* gt = p.gates + (size_t)qh * 3;
  const float g0 = gt[0], g1 = gt[1], g2 = gt[2];
  const int nvis = n_visible(p, b, L);
  const int nch_b = (nvis + kChunk - 1) / kChunk;
  __syncthreads();

  // ---- compressed branch
  float oc = 0.f;
#pragma unroll
  for (int u = 0; u < kBatch; ++u) oc += u < nch_b ? s_f[u] * vo[u] : 0.f;
  for (int c0 = kBatch; c0 < nch_b; c0 += kBatch) {  // long contexts: remaining chunks
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = c0 + u < nch_b ? p.o1[((cbase + c0 + u) * 16 + h) * DV + ch] : 0.f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) oc += c0 + u < nch_b ? s_f[c0 + u] * v[u] : 0.f;
  }
  // ---- selected branch: the finish workgroups' partials
  float M = -INFINITY;
  for (int k = 0; k < nfin; ++k) M = fmaxf(M, s_pm[k]);
  float vs = 0.f, ls = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxFinish; ++k) {
    if (k < nfin && s_pm[k] != -INFINITY) {
      const float a = exp2f(s_pm[k] - M);
      vs += a * vr[k];
      ls += a * s_pl[k];
    }
  }
  // ---- window branch
  float Mw = -INFINITY;
  for (int k = 0; k < nwin; ++k) Mw = fmaxf(Mw, s_wm[k]);
  float vwin = 0.f, lwin = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxWindow; ++k) {
    if (k < nwin && s_wm[k] != -INFINITY) {
      const float a = exp2f(s_wm[k] - Mw);
      vwin += a * vw[k];
      lwin += a * s_wl[k];
    }
  }
  const float os = ls > 0.f ? vs / ls : 0.f;
  const float ow = lwin > 0.f ? vwin / lwin : 0.f;
  p.out[(size_t)qh * DV + ch] = (uint16_t)f32_to_bf16(g0 * oc + g1 * os + g2 * ow);
}

// ---------------------------------------------------------------- host side

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeLayout decode_layout(int B, int H, int DV, int l, int d, int lsel, int n, int nloc, int w, int64_t max_len) {
  (void)nloc;  // the always-taken blocks are part of the n selected blocks
  DecodeLayout lay{};
  const int64_t nc = max_len >= l ? (max_len - l) / d + 1 : 0;
  lay.nch = (int)((nc + kChunk - 1) / kChunk);
  if (lay.nch < 1) lay.nch = 1;
  lay.nbo = (int)((int64_t)kChunk * d / lsel);
  const size_t BH = (size_t)B * H;
  size_t off = 0;
  lay.off_m1 = off;   off = align256(off + BH * lay.nch * 16 * 4);
  lay.off_l1 = off;   off = align256(off + BH * lay.nch * 16 * 4);
  lay.off_o1 = off;   off = align256(off + BH * lay.nch * 16 * (size_t)DV * 4);
  lay.off_sc1 = off;  off = align256(off + BH * lay.nch * 16 * (size_t)(lay.nbo + 1) * 4);
  // window workgroups: one 32-token step per wave over the window's blocks (at
  // most ceil(w/l')+1 of them); one partial each
  const int spb = lsel >= 32 ? lsel / 32 : 1;
  const int wsteps = ((w + lsel - 1) / lsel + 1) * spb;
  lay.nwin = (wsteps + kCmpWaves - 1) / kCmpWaves;
  lay.off_wpart = off; off = align256(off + BH * lay.nwin * (32 + 16 * (size_t)DV) * 4);
  // finish workgroups (4 waves, one step each): one partial each; normalised
  // compressed-branch factors
  lay.nfin = (n * spb + 3) / 4;
  lay.off_rpart = off; off = align256(off + BH * lay.nfin * (32 + 16 * (size_t)DV) * 4);
  lay.off_fcmp = off; off = align256(off + BH * lay.nch * 16 * 4);
  lay.total = off;
  return lay;
}

template <int DK, int DV>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s, const PhaseEvents* ev) {
  hipError_t e;
  if (ev && (e = hipEventRecord(ev->ev[0], s)) != hipSuccess) return e;
  const dim3 g1((unsigned)(p.B * p.H * (p.nch + p.nwin))), b1(64 * kCmpWaves);
  switch (p.lsel) {
    case 16: hipLaunchKernelGGL((decode_cmp_kernel<DK, DV, 16>), g1, b1, 0, s, p); break;
    case 32: hipLaunchKernelGGL((decode_cmp_kernel<DK, DV, 32>), g1, b1, 0, s, p); break;
    case 64: hipLaunchKernelGGL((decode_cmp_kernel<DK, DV, 64>), g1, b1, 0, s, p); break;
    case 128: hipLaunchKernelGGL((decode_cmp_kernel<DK, DV, 128>), g1, b1, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev->ev[1], s)) != hipSuccess) return e;
  const dim3 g2((unsigned)(p.B * p.H * p.nfin)), blk(256);
  switch (p.lsel) {
    case 16: hipLaunchKernelGGL((decode_finish_kernel<DK, DV, 16>), g2, blk, 0, s, p); break;
    case 32: hipLaunchKernelGGL((decode_finish_kernel<DK, DV, 32>), g2, blk, 0, s, p); break;
    case 64: hipLaunchKernelGGL((decode_finish_kernel<DK, DV, 64>), g2, blk, 0, s, p); break;
    case 128: hipLaunchKernelGGL((decode_finish_kernel<DK, DV, 128>), g2, blk, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev->ev[2], s)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<DV>), dim3((unsigned)(p.B * p.Hq)), dim3(DV), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev->ev[3], s)) != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, int DK, int DV, hipStream_t s, const PhaseEvents* ev) {
  if (DK == 192 && DV == 128) return launch_decode_t<192, 128>(p, s, ev);
  if (DK == 128 && DV == 128) return launch_decode_t<128, 128>(p, s, ev);
  if (DK == 64 && DV == 64) return launch_decode_t<64, 64>(p, s, ev);
  return hipErrorInvalidValue;
}

}  // namespace nsa

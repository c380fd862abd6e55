// NSA decode step on gfx950: two launches per step.  Between them the kernel
// boundary is the synchronisation; inside the second, one device-scope counter
// per (sequence, group) finds the workgroup that finishes last.
//
// 1. decode_stream_kernel, about one workgroup per compute unit, two kinds:
//    - segment workgroups: the compressed branch, split over segments of
//      compressed keys per (sequence, KV group).  Each streams its segment of
//      the compressed cache once into registers, computes the 16-head logits with
//      MFMA, the segment's softmax statistics and partial output, and the
//      per-head probabilities folded onto selection blocks;
//    - window workgroups: the window branch, which does not depend on the
//      selection, streamed the same way over the window's raw tokens.
// 2. decode_finish_kernel: several workgroups per (sequence, group), each
//    computing the exact per-head normalisers from the segment statistics, the
//    group scores and the top-n, a slice of the compressed-branch output, and
//    its share of the selected blocks (one 32-token step per wave); the last
//    of them to finish merges the partials and applies the gates:
//    out = g_cmp*o_cmp + g_slc*o_slc + g_win*o_win in bf16.
//
// Sources: lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc),
// section "NSA: три ветви" (output equation; compressed branch l=32, d=16;
// selection of n l'-blocks re-using the compressed-branch weights, shared by a
// GQA group so each KV block is read once per group; window of w tokens) and
// section "Сколько это экономит" (decode is bound by reading the KV cache).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "nsa_device.hpp"
#include "nsa_internal.hpp"
#include "nsa_tiles.hpp"
#include "nsa_topn.hpp"

namespace nsa {

namespace {

// Wave-uniform reads of the read-only length arrays through the scalar data
// cache: waiting for them does not wait for outstanding vector loads.
template <class T>
__device__ __forceinline__ T ld_scalar(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

__device__ __forceinline__ int64_t raw_row0(const DecodeParams& p, int b, int g) {
  if (p.cu) {
    const int64_t c0 = ld_scalar(p.cu + b), c1 = ld_scalar(p.cu + b + 1);
    return (int64_t)p.H * c0 + (int64_t)g * (c1 - c0);
  }
  return ((int64_t)b * p.H + g) * p.cap;
}

__device__ __forceinline__ int64_t cmp_row0(const DecodeParams& p, int b, int g) {
  if (p.cuc) {
    const int64_t c0 = ld_scalar(p.cuc + b), c1 = ld_scalar(p.cuc + b + 1);
    return (int64_t)p.H * c0 + (int64_t)g * (c1 - c0);
  }
  return ((int64_t)b * p.H + g) * p.ccap;
}

// Tokens present in sequence b, clamped to [1, capacity] so that inconsistent
// device-side lengths can never move an access outside the caller's buffers.
__device__ __forceinline__ int seq_len_clamped(const DecodeParams& p, int b) {
  int64_t cap = p.cap;
  if (p.cu) {
    const int64_t c = ld_scalar(p.cu + b + 1) - ld_scalar(p.cu + b);
    if (c < cap) cap = c;
  }
  int64_t L = ld_scalar(p.seq_lens + b);
  if (L > cap) L = cap;
  if (L < 1) L = 1;
  return (int)L;
}

// Complete compressed blocks among L tokens, clamped to the compressed capacity.
__device__ __forceinline__ int n_visible(const DecodeParams& p, int b, int L) {
  int64_t nv = L >= p.l ? (L - p.l) / p.d + 1 : 0;
  const int64_t ccap = p.cuc ? ld_scalar(p.cuc + b + 1) - ld_scalar(p.cuc + b) : p.ccap;
  return (int)(nv < ccap ? nv : ccap);
}

// Stores and loads that are coherent across the whole device without cache
// maintenance (relaxed atomics at agent scope): the finish workgroups of one
// (sequence, group) hand their partials to the last of them this way.
__device__ __forceinline__ void st_shared_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_shared_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2_t ld2_shared_dev(const float* p) {  // p 8-byte aligned
  const uint64_t u = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x2_t{__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32))};
}

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
template <int DV, int NWV, bool DEV_SHARED = false>
__device__ __forceinline__ void merge_waves_to(const Branch<DV>& br, float* dst, float* buf, float* st) {
  auto put = [&](float* q, float v) {
    if constexpr (DEV_SHARED) st_shared_dev(q, v);
    else *q = v;
  };
  auto put2 = [&](float* q, float v0, float v1) {  // q 8-byte aligned
    if constexpr (DEV_SHARED) {
      const uint64_t u = (uint64_t)__float_as_uint(v0) | ((uint64_t)__float_as_uint(v1) << 32);
      __hip_atomic_store(reinterpret_cast<uint64_t*>(q), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      q[0] = v0;
      q[1] = v1;
    }
  };
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  constexpr int NTH = 64 * NWV;
  if (lg == 0) {
    st[wave * 16 + lr] = br.m;
    st[(NWV + wave) * 16 + lr] = br.l;
  }
  lds_barrier();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NWV; ++w) M = fmaxf(M, st[w * 16 + lr]);
  const float alpha = br.m == -INFINITY ? 0.f : exp2f(br.m - M);
#pragma unroll
  for (int j = 0; j < DV / 16; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) buf[(wave * 16 + lr) * (DV + 1) + acc_channel<DV>(lg, i, j)] = alpha * br.acc[j][i];
  lds_barrier();
  for (int e = 2 * tid; e < 16 * DV; e += 2 * NTH) {  // two outputs per thread and pass
    const int h = e / DV, ch = e - h * DV;
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      v0 += buf[(w * 16 + h) * (DV + 1) + ch];
      v1 += buf[(w * 16 + h) * (DV + 1) + ch + 1];
    }
    put2(dst + 32 + e, v0, v1);
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
    put(dst + tid, Mh);
    put(dst + 16 + tid, ls);
  }
  lds_barrier();
}



}  // namespace

// ---------------------------------------------------------------- streaming pass

// Smallest row stride >= n that is 4 mod 16: the four lane groups of a wave then
// address disjoint LDS banks when they add into four different head rows.
__host__ __device__ constexpr int score_stride(int n) { return n + ((20 - n % 16) % 16); }

// The 16 rows of a 64-row tile that one wave owns, held in registers in MFMA
// operand order: K row lr, dims 32*ks + 8*lg .. (A operand of S^T), and V rows
// 4*lg + e, channels (DV/16)*lr .. (the values its P^T k-slots pair with).
template <int DK, int DV>
struct WaveTile {
  u32x4_t k[DK / 32];
  uint32_t v[4][DV / 32];
};

// A wave-uniform pointer moved into scalar registers, so that loads address it
// as scalar base + 32-bit lane offset + immediate.  The result is typed as a
// global-memory pointer: through a generic pointer the loads would be flat
// loads, which also count against the LDS counter, so every LDS wait of the
// pipeline would also wait for the tiles in flight.
typedef const __attribute__((address_space(1))) char* gchar_ptr;
__device__ __forceinline__ gchar_ptr scalar_ptr(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return (gchar_ptr)(((uint64_t)hi << 32) | lo);
}
template <class T>
__device__ __forceinline__ T ld_global(gchar_ptr p) {
  return *(const __attribute__((address_space(1))) T*)p;
}

// Rows row0 .. row0+15 (row0 wave-uniform); rows past rowmax read row rowmax
// (their logits are masked by the caller).  koff / voff are the lane's byte
// offsets within a full tile slice: (lr*DK + 8*lg)*2 and (4*lg*DV + (DV/16)*lr)*2.
template <int DK, int DV>
__device__ __forceinline__ void load_wave_tile(WaveTile<DK, DV>& T, const uint16_t* kb, const uint16_t* vb,
                                               int64_t row0, int64_t rowmax, uint32_t koff, uint32_t voff,
                                               int lg, int lr) {
  constexpr int CPL = DV / 16;  // channels per lane and row
  auto put_v = [&](int e, gchar_ptr src) {
    if constexpr (CPL == 8) {
      const u32x4_t x = ld_global<u32x4_t>(src);
      T.v[e][0] = x[0]; T.v[e][1] = x[1]; T.v[e][2] = x[2]; T.v[e][3] = x[3];
    } else {
      const u32x2_t x = ld_global<u32x2_t>(src);
      T.v[e][0] = x[0]; T.v[e][1] = x[1];
    }
  };
  if (row0 + 15 <= rowmax) {  // wave-uniform: all 16 rows exist
    const gchar_ptr kp = scalar_ptr(kb + row0 * DK) + koff;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) T.k[ks] = ld_global<u32x4_t>(kp + 64 * ks);
    const gchar_ptr vp = scalar_ptr(vb + row0 * DV) + voff;
#pragma unroll
    for (int e = 0; e < 4; ++e) put_v(e, vp + e * DV * 2);
  } else {
    const int64_t rk = min(row0 + lr, rowmax);
    const gchar_ptr kp = (gchar_ptr)(kb + rk * DK + 8 * lg);
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) T.k[ks] = ld_global<u32x4_t>(kp + 64 * ks);
#pragma unroll
    for (int e = 0; e < 4; ++e) put_v(e, (gchar_ptr)(vb + min(row0 + 4 * lg + e, rowmax) * DV + CPL * lr));
  }
}

// Workgroup of the streaming pass: kStreamWaves waves stream the rows of a
// segment of the compressed cache (or of part of the window of the raw cache)
// as 64-row tiles; wave w owns rows 16w .. 16w+15 of every tile and loads them
// straight into registers, kDepth - 1 tiles ahead of the one it computes:
//   logits  S^T = K . q^T                      (16x16x32 MFMA, d_k/32 k-steps)
//   values  O^T += V^T . P^T                   (16x16x16 MFMA; P^T is the logit tile)
//   scores  F^T  = Omega^T . P^T (P as bf16 hi + lo) (16x16x16 MFMA), added into the
//           per-head score rows of the segment's selection blocks in LDS, in a
//           fixed order, so repeated calls give identical results
// Omega[key][block] is the number of stride units key and block share (an exact
// small integer; divided by l/d when the scores are written out).  The four
// waves keep one softmax reference per head: each tile's per-wave maxima are
// exchanged through LDS (the only barrier of a tile), and the reference moves
// (rescaling the outputs, the sums and the scores) only when a tile maximum
// exceeds it by kLazy.
//
// Outputs per compressed segment: the reference m, the sum l of exp2(z - m), the
// unnormalised output sum, and the selection-block scores (slot nbo is the
// overhang into the first block of the next segment).  Per window workgroup:
// the same (m, l, o) triple over its window tokens.
template <int DK, int DV>
__global__ __launch_bounds__(64 * kStreamWaves, 1) void decode_stream_kernel(DecodeParams p) {
  constexpr int NW = kStreamWaves, NTH = 64 * NW, KT = DK / 32, VC = DV / 16;
#ifndef NSA_STREAM_DEPTH
#define NSA_STREAM_DEPTH 3
#endif
  constexpr int kDepth = NSA_STREAM_DEPTH;  // register tiles per wave (kDepth in flight while one is awaited)
  constexpr int PSTRIDE = 32 + 16 * DV;
  constexpr float kLazy = 8.0f, kNegBig = -1e30f;
  __shared__ float s_sc[16 * kScStrideMax];
  __shared__ float s_o[NW][16][DV + 1];
  __shared__ __attribute__((aligned(16))) float s_fw[2][NW][16][16];  // per-wave fold results [head][block row]
  __shared__ float s_tmax[2][NW][16];
  __shared__ float s_alpha[16];
  __shared__ float s_l[NW][16];

  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per = p.nch + p.nwin;
  const int bg = blockIdx.x / per, c = blockIdx.x - bg * per;
  const int g = bg % p.H, b = bg / p.H;
  const bool fold = c < p.nch;  // workgroup-uniform: compressed segment, else window part
  const uint32_t koff = (uint32_t)((lr * DK + 8 * lg) * 2), voff = (uint32_t)((4 * lg * DV + VC * lr) * 2);
  u32x4_t qf[KT];
  WaveTile<DK, DV> tb[kDepth];
  auto load_q = [&]() { load_q_frags<DK>(p.q + ((int64_t)b * p.Hq + (int64_t)g * p.G) * DK, p.G, lg, lr, qf); };

  // rows [r0, r0 + 64*nt) are streamed; keys outside [vlo, vhi] are masked
  int64_t r0, rowmax;
  int nt, vlo, vhi;
  const uint16_t *kb, *vb;
  int L;
  if (fold) {
    // A segment's rows and its slot's capacity do not depend on the sequence
    // length, so the first tiles are requested while the length is read; rows
    // past the length are masked (their values are zeroed before use).
    const int k0 = c * p.seg;
    const int64_t ccap_b = p.cuc ? ld_scalar(p.cuc + b + 1) - ld_scalar(p.cuc + b) : p.ccap;
    if (k0 >= ccap_b) return;  // beyond the slot: never read by the later kernels
    const int64_t rpre = min((int64_t)k0 + p.seg, ccap_b) - 1;
    const int64_t crow = cmp_row0(p, b, g);
    kb = p.kc + crow * DK;
    vb = p.vc + crow * DV;
    L = seq_len_clamped(p, b);
    load_q();
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d)
      load_wave_tile<DK, DV>(tb[d], kb, vb, (int64_t)k0 + 64 * d + 16 * wave, rpre, koff, voff, lg, lr);
    const int nvis = n_visible(p, b, L);
    if (k0 >= nvis) {  // empty segment: never read by the later kernels
      wait_vmem();
      return;
    }
    const int k1 = min(k0 + p.seg, nvis);
    r0 = k0;
    nt = (k1 - k0 + 63) >> 6;
    vlo = k0;
    vhi = k1 - 1;
    rowmax = nvis - 1;
  } else {
    const int wi = c - p.nch;
    if (wi == 0 && tid == 0) p.cnt[bg] = 0u;  // arrival counter of the finish workgroups
    L = seq_len_clamped(p, b);
    const int t = L - 1;
    const int wlo = t - p.w + 1 > 0 ? t - p.w + 1 : 0;
    const int T0 = (wlo >> 6) + wi * p.wtiles, T1 = min((wlo >> 6) + (wi + 1) * p.wtiles, (t >> 6) + 1);
    r0 = (int64_t)T0 * 64;
    nt = T1 - T0;
    vlo = wlo;
    vhi = t;
    rowmax = t;
    const int64_t row = raw_row0(p, b, g);
    kb = p.k + row * DK;
    vb = p.v + row * DV;
    if (nt <= 0) {  // nothing of the window falls to this workgroup: empty partial
      float* dst = p.wpart + ((size_t)bg * p.nwin + wi) * PSTRIDE;
      for (int e = tid; e < PSTRIDE; e += NTH) dst[e] = e < 16 ? -INFINITY : 0.f;
      return;
    }
    load_q();
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d)
      load_wave_tile<DK, DV>(tb[d], kb, vb, r0 + 64 * d + 16 * wave, min(rowmax, r0 + 64 * (int64_t)nt - 1), koff,
                             voff, lg, lr);
  }

  // Loads never read past the workgroup's own last row: requests for tiles
  // beyond the range (issued so that every pipeline step has the same loads in
  // flight) re-read that row from cache.
  const int64_t rlast = min(rowmax, r0 + 64 * (int64_t)nt - 1);

  const int qd = p.l / p.d, rd = p.lsel / p.d;  // key and block lengths in stride units
  const int rsh = __builtin_ctz(rd);            // rd is a power of two
  const int jseg0 = fold ? (int)(r0 >> rsh) : 0;
  const int sstride = score_stride(p.nbo + 1);
  if (fold)
    for (int e = tid; e < 16 * sstride; e += NTH) s_sc[e] = 0.f;

  // Adds tile i's fold results into the score rows: entry (head h, block j) is
  // the sum over the waves, in wave order, of the rows their keys give block j
  // (so the scores do not depend on wave timing).
  auto fold_flush = [&](int i) {
    const int kt0 = (int)(r0 + 64 * i);
    const int jT0 = kt0 >> rsh;
    const int nr = ((kt0 + 63 + qd - 1) >> rsh) - jT0 + 1;  // blocks the tile's keys touch
    const float(*fw)[16][16] = s_fw[i & 1];
    for (int e = tid; e < 16 * nr; e += NTH) {
      const int h = e & 15, j = jT0 + (e >> 4);
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int kw = kt0 + 16 * w, j0w = kw >> rsh;
        const int nrw = ((kw + 15 + qd - 1) >> rsh) - j0w + 1;
        const int row = j - j0w;
        if (row >= 0 && row < nrw) v += fw[w][h][row];
      }
      s_sc[h * sstride + (j - jseg0)] += v;
    }
  };

  f32x4_t acc[VC];
#pragma unroll
  for (int j = 0; j < VC; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f, mref = kNegBig;
  const float sc = p.scale_log2;

  auto process = [&](int i, const WaveTile<DK, DV>& T) {
    const int64_t k0 = r0 + 64 * i + 16 * wave;  // the wave's first row
    // ---- logits of the wave's 16 rows; element e is row k0 + 4lg + e, head lr
    f32x4_t sv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KT; ++ks) sv = mfma_bf16(T.k[ks], qf[ks], sv);
    float z[4];
    if (k0 >= vlo && k0 + 15 <= vhi) {  // wave-uniform
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = sv[e] * sc;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t x = k0 + 4 * lg + e;
        z[e] = (x >= vlo && x <= vhi) ? sv[e] * sc : -INFINITY;
      }
    }
    float mw = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mw = max_over_groups_swap(mw);
    if (lg == 0) s_tmax[i & 1][wave][lr] = mw;
    lds_barrier();  // the tile's maxima, and the previous tile's fold results, are complete
    if (fold && i > 0) fold_flush(i - 1);
    float mt = s_tmax[i & 1][0][lr];
#pragma unroll
    for (int w = 1; w < NW; ++w) mt = fmaxf(mt, s_tmax[i & 1][w][lr]);

    // ---- lazy reference move (identical decision in every wave)
    const bool move = mt > mref + kLazy;
    if (__ballot(move) != 0ull) {
      const float mn = move ? mt : mref;
      const float alpha = __builtin_amdgcn_exp2f(mref - mn);
#pragma unroll
      for (int j = 0; j < VC; ++j) acc[j] *= alpha;
      lsum *= alpha;
      mref = mn;
      if (fold && i > 0) {
        if (wave == 0 && lg == 0) s_alpha[lr] = alpha;
        lds_barrier();  // also orders every thread's flush before the scaling
        for (int e = tid; e < 16 * sstride; e += NTH) s_sc[e] *= s_alpha[e / sstride];
        lds_barrier();
      }
    }

    // ---- probabilities, values (rows past rlast may hold values of rows past the
    // sequence, which are zeroed: their weight is 0 but their bits are arbitrary)
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = __builtin_amdgcn_exp2f(z[e] - mref);
    lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const u32x2_t ph = {pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
    const bool vall = k0 + 15 <= rlast;  // wave-uniform
    const uint32_t vm01 = (k0 + 4 * lg <= rlast ? 0x0000FFFFu : 0u) | (k0 + 4 * lg + 1 <= rlast ? 0xFFFF0000u : 0u);
    const uint32_t vm23 = (k0 + 4 * lg + 2 <= rlast ? 0x0000FFFFu : 0u) | (k0 + 4 * lg + 3 <= rlast ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int j = 0; j < VC; ++j) {
      const int wd = j >> 1, h = j & 1;
      u32x2_t va = {pack_halves(T.v[0][wd], T.v[1][wd], h), pack_halves(T.v[2][wd], T.v[3][wd], h)};
      if (!vall) va = u32x2_t{va[0] & vm01, va[1] & vm23};
      acc[j] = mfma16_bf16(va, ph, acc[j]);
    }

    // ---- fold onto selection blocks: rows of Omega^T are blocks j0 + lr
    if (fold) {
      const int phi = (int)k0 & (rd - 1);  // offset of the first key in its block
      float ov[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int u0 = phi + 4 * lg + e;  // key's first unit, relative to block j0
        const int o = min(u0 + qd, (lr + 1) * rd) - max(u0, lr * rd);
        ov[e] = (float)(o > 0 ? o : 0);
      }
      const u32x2_t om = {pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
      float lo[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        lo[2 * e] = pr[2 * e] - bf16_lo(ph[e]);
        lo[2 * e + 1] = pr[2 * e + 1] - bf16_hi(ph[e]);
      }
      const u32x2_t pl = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3])};
      f32x4_t f = mfma16_bf16(om, ph, f32x4_t{0.f, 0.f, 0.f, 0.f});
      f = mfma16_bf16(om, pl, f);
      // element e: block j0 + 4lg + e, head lr
      *reinterpret_cast<f32x4_t*>(&s_fw[i & 1][wave][lr][4 * lg]) = f;
    }
  };

  // ---- the pipeline: tile i+kDepth-1 is requested before tile i is computed.
  // Every step of the main loop issues the same loads, so the compiler's wait
  // before a tile's first use leaves the later tiles in flight; the last
  // (nt mod kDepth) tiles were requested by the main loop and need no loads.
  int i0 = 0;
  for (; i0 + kDepth <= nt; i0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      load_wave_tile<DK, DV>(tb[(u + kDepth - 1) % kDepth], kb, vb, r0 + 64 * (i0 + u + kDepth - 1) + 16 * wave,
                             rlast, koff, voff, lg, lr);
      process(i0 + u, tb[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < kDepth - 1; ++u)
    if (i0 + u < nt) process(i0 + u, tb[u]);  // workgroup-uniform

  // ---- workgroup merge: all waves share mref, so outputs and sums just add
  lsum = sum_over_groups_swap(lsum);
  if (lg == 0) s_l[wave][lr] = lsum;
#pragma unroll
  for (int j = 0; j < VC; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_o[wave][lr][acc_channel<DV>(lg, e, j)] = acc[j][e];
  lds_barrier();
  if (fold) {
    fold_flush(nt - 1);
    lds_barrier();
  }
  float *dm, *dl, *dox;
  if (fold) {
    const size_t slot = (size_t)bg * p.nch + c;
    dm = p.m1 + slot * 16;
    dl = p.l1 + slot * 16;
    dox = p.o1 + slot * 16 * DV;
  } else {
    float* dst = p.wpart + ((size_t)bg * p.nwin + (c - p.nch)) * PSTRIDE;
    dm = dst;
    dl = dst + 16;
    dox = dst + 32;
  }
#pragma unroll
  for (int hh = 0; hh < 16 / NW; ++hh)
#pragma unroll
    for (int cc = 0; cc < DV / 64; ++cc) {
      const int h = wave + NW * hh, ch = lane + 64 * cc;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += s_o[w][h][ch];
      dox[h * DV + ch] = v;
    }
  if (tid < 16) {  // lane tid holds head tid's reference
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) ls += s_l[w][tid];
    dl[tid] = ls;
    dm[tid] = mref;
  }
  if (fold) {
    const int slots = p.nbo + 1;
    const float invq = 1.0f / (float)qd;
    float* SC = p.sc1 + ((size_t)bg * p.nch + c) * slots * 16;  // [slot][head]
    for (int e0 = tid; e0 < 16 * slots; e0 += 4 * NTH) {  // four entries per thread and pass
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + NTH * u;
        v[u] = e < 16 * slots ? s_sc[(e & 15) * sstride + (e >> 4)] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e0 + NTH * u < 16 * slots) SC[e0 + NTH * u] = v[u] * invq;
    }
  }
}

// Finish: nfin workgroups of 4 waves per (sequence, group).  Every one of them
// computes the exact per-head normalisers of the compressed branch, the group
// scores and the top-n (identical results, so no exchange is needed); then
// workgroup k
//   - sums its slice of the normalised compressed-branch output over the
//     segments (the loads are issued before the normalisers are known),
//   - attends the selected steps [4k, 4k+4) (one 32-token step per wave, over
//     all selected blocks in ascending order) and writes one partial.
// The last of the nfin workgroups to finish (a device-scope counter, cleared
// by the streaming pass) merges the selected-branch partials and the window
// partials and writes out = g_cmp*o_cmp + g_slc*o_slc + g_win*o_win in bf16.
template <int DK, int DV, int LSEL>
#ifndef NSA_FIN_WAVES
#define NSA_FIN_WAVES 4
#endif
__global__ __launch_bounds__(64 * NSA_FIN_WAVES) void decode_finish_kernel(DecodeParams p) {
  constexpr int NWV = NSA_FIN_WAVES, NTH = 64 * NWV;
  constexpr int KT = DK / 32;
  constexpr int SPB = LSEL >= 32 ? LSEL / 32 : 1;   // 32-token steps per selection block
  constexpr int PSTRIDE = 32 + 16 * DV;
  constexpr int RPT = 4;                             // candidate blocks per thread and load round
  constexpr int OB = 8;                              // segments per compressed-output load batch
  __shared__ float S[kMaxBlocks];
  __shared__ float s_f[kMaxChunks * 16];
  __shared__ float s_ml[2 * kMaxChunks * 16];       // segment m / l, then wave-merge scratch
  __shared__ float s_ov[kMaxChunks * 16];           // overhang score slot of each segment, per head
  __shared__ float s_buf[NWV * 16 * (DV + 1)];
  __shared__ TopnSmem tsm;
  __shared__ TopnFastSmem<NWV> tfs;
  __shared__ int s_sel[kMaxSel];
  __shared__ int s_items[kMaxSel];
  __shared__ int s_nitems;
  __shared__ int s_last;
  __shared__ float s_pf[kMaxFinish][16], s_wf[kMaxWindow][16];
  __shared__ float s_gate[16][3];

  // Workgroups are dealt to the 8 XCDs round-robin by id; when the sizes allow,
  // the nfin workgroups of one (sequence, group) get ids on the same XCD, so the
  // partials they hand over stay in that XCD's L2.  Only speed depends on this.
  int bg, kfin;
  if ((p.B * p.H) % 8 == 0) {
    const int w = blockIdx.x, xcd = w & 7, r = w >> 3;
    bg = xcd + 8 * (r / p.nfin);
    kfin = r - (r / p.nfin) * p.nfin;
  } else {
    bg = blockIdx.x / p.nfin;
    kfin = blockIdx.x - bg * p.nfin;
  }
  const int g = bg % p.H, b = bg / p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int nch = p.nch, nbo = p.nbo, slots = nbo + 1;
  const size_t cbase = (size_t)bg * nch;
  float* s_m = s_ml;
  float* s_l = s_ml + kMaxChunks * 16;

  // ---- one round of loads (all issued before any is waited for): the sequence
  // length, segment statistics and overhang slots of the first 16 segment slots,
  // the first round of candidate scores ([segment][slot][16 heads]), this
  // workgroup's first batch of compressed-branch outputs, the query fragments
  const int L = seq_len_clamped(p, b);
  float pm = 0.f, pl = 0.f, pov = 0.f;
  if (tid < nch * 16) {
    pm = p.m1[cbase * 16 + tid];
    pl = p.l1[cbase * 16 + tid];
    pov = p.sc1[((cbase + (tid >> 4)) * slots + nbo) * 16 + (tid & 15)];
  }
  f32x4_t vv[RPT][4];
  auto load_scores = [&](int j0) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int j = j0 + tid + NTH * r;
      int cc = j / nbo, jj = j - cc * nbo;
      if (cc >= nch) cc = nch - 1, jj = 0;  // beyond every sequence: read in bounds, discarded
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(p.sc1 + ((cbase + cc) * slots + jj) * 16);
#pragma unroll
      for (int u = 0; u < 4; ++u) vv[r][u] = src[u];
    }
  };
  load_scores(0);
  // compressed-branch output slice of this workgroup: outputs [e0, e1) of the
  // group's 16 x DV, one per thread and pass
  const int per = (16 * DV + p.nfin - 1) / p.nfin;
  const int e0 = kfin * per, e1 = min(e0 + per, 16 * DV);
  float vo[OB];
  {
    const int e = e0 + tid;
    const int ee = e < e1 ? e : e0;
#pragma unroll
    for (int u = 0; u < OB; ++u) vo[u] = p.o1[(cbase + min(u, nch - 1)) * 16 * DV + ee];
  }
  u32x4_t qf[KT];
  load_q_frags<DK>(p.q + ((int64_t)b * p.Hq + (int64_t)g * p.G) * DK, p.G, lg, lr, qf);
  if (p.wgate) {  // gate network: 3 G dot products of the query with a weight row, four lanes each
    for (int e0 = 0; e0 < 12 * p.G; e0 += NTH) {  // one pass when NTH >= 12 G
      const int pr = (e0 + tid) >> 2, pt = tid & 3;
      const int pc = pr < 3 * p.G ? pr : 0;
      const int hq = g * p.G + pc / 3, br = pc % 3;
      float z = gate_dot_quarter<DK>(p.q + ((size_t)b * p.Hq + hq) * DK, p.wgate + ((size_t)hq * 3 + br) * DK, pt);
      z += __shfl_xor(z, 1);
      z += __shfl_xor(z, 2);
      if (pr < 3 * p.G && pt == 0) s_gate[pr / 3][br] = gate_sigmoid(z + (p.bgate ? p.bgate[hq * 3 + br] : 0.f));
    }
  } else {
    const float gv = tid < 3 * p.G ? p.gates[((size_t)b * p.Hq + (size_t)g * p.G) * 3 + tid] : 0.f;
    if (tid < 3 * p.G) s_gate[tid / 3][tid % 3] = gv;
  }
  if (tid < nch * 16) {
    s_m[tid] = pm;
    s_l[tid] = pl;
    s_ov[tid] = pov;
  }
  for (int idx = tid + NTH; idx < nch * 16; idx += NTH) {  // more than 16 segments
    s_m[idx] = p.m1[cbase * 16 + idx];
    s_l[idx] = p.l1[cbase * 16 + idx];
    s_ov[idx] = p.sc1[((cbase + (idx >> 4)) * slots + nbo) * 16 + (idx & 15)];
  }
  const int nvis = n_visible(p, b, L);
  const int nch_b = (nvis + p.seg - 1) / p.seg;
  const int t = L - 1;
  const int J = t / LSEL;
  lds_barrier();

  // ---- exact per-head normalisers (wave 0: lane = head + 16 * segment phase)
  if (wave == 0) {
    const int h = lr;
    float M = -INFINITY;
    for (int c = lg; c < nch_b; c += 4) M = fmaxf(M, s_m[c * 16 + h]);
    M = max_over_groups_swap(M);
    float Ls = 0.f;
    for (int c = lg; c < nch_b; c += 4) Ls += s_l[c * 16 + h] * __builtin_amdgcn_exp2f(s_m[c * 16 + h] - M);
    Ls = sum_over_groups_swap(Ls);
    const float inv = Ls > 0.f ? 1.0f / Ls : 0.f;
    for (int c = lg; c < nch_b; c += 4) s_f[c * 16 + h] = h < p.G ? __builtin_amdgcn_exp2f(s_m[c * 16 + h] - M) * inv : 0.f;
  }
  lds_barrier();

  // ---- this workgroup's slice of the compressed-branch output.  The first
  // output of each thread is kept in a register and stored with the partial
  // below: a store issued here would make the top-n wait for its completion
  // (stores are counted with the loads, and its registers get reused).
  float oc_first = 0.f;
  for (int e = e0 + tid; e < e1; e += NTH) {
    const int h = e / DV;
    float oc = 0.f;
    if (e == e0 + tid) {
#pragma unroll
      for (int u = 0; u < OB; ++u) oc += u < nch_b ? s_f[u * 16 + h] * vo[u] : 0.f;
    } else {
      for (int c = 0; c < min(nch_b, OB); ++c) oc += s_f[c * 16 + h] * p.o1[(cbase + c) * 16 * DV + e];
    }
    for (int c = OB; c < nch_b; ++c) oc += s_f[c * 16 + h] * p.o1[(cbase + c) * 16 * DV + e];
    if (e == e0 + tid) oc_first = oc;
    else st_shared_dev(p.ocmp + (size_t)bg * 16 * DV + e, oc);
  }

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
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) sc += s_f[cc * 16 + 4 * u + e] * vv[r][u][e];
      }
      if (jj == 0 && cc >= 1 && cc - 1 < nch_b) {  // overhang of the previous segment
#pragma unroll
        for (int h = 0; h < 16; ++h) sc += s_f[(cc - 1) * 16 + h] * s_ov[(cc - 1) * 16 + h];
      }
      S[j] = sc;
    }
  }
  lds_barrier();
  {
    int32_t* so = (p.sel_out && kfin == 0) ? p.sel_out + (size_t)bg * p.n : nullptr;
    if (J + 1 <= 4 * NTH) block_topn_fast<NTH, 4, kMaxBlocks / NTH>(S, J, p.n, p.nloc, p.finit, tfs, tsm, s_sel, so);
    else block_topn_fast<NTH, 8, kMaxBlocks / NTH>(S, J, p.n, p.nloc, p.finit, tfs, tsm, s_sel, so);
  }
  lds_barrier();
  if (wave == 0) {  // the selected blocks, ascending (the list ends at the first -1)
    const int j = lane < p.n ? s_sel[lane] : -1;
    const uint64_t m = __ballot(j >= 0);
    if (j >= 0) s_items[__popcll(m & ((1ull << lane) - 1ull))] = j;
    if (lane == 0) s_nitems = __popcll(m);
  }
  lds_barrier();

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
  float* rp = p.rpart + (size_t)bg * p.nfin * PSTRIDE;
  if (e0 + tid < e1) st_shared_dev(p.ocmp + (size_t)bg * 16 * DV + e0 + tid, oc_first);
  merge_waves_to<DV, NWV, true>(br, rp + (size_t)kfin * PSTRIDE, s_buf, s_ml);

  // ---- the last workgroup of this (sequence, group) applies the gates.  The
  // partial and the output slice were stored coherently; once every thread's
  // stores have completed, the counter is incremented, and the workgroup that
  // sees the final count reads the others' results with coherent loads.
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(p.cnt + bg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (unsigned)(p.nfin - 1);
  lds_barrier();
  if (!s_last) return;
  const float* wp = p.wpart + (size_t)bg * p.nwin * PSTRIDE;
  const float* oc_src = p.ocmp + (size_t)bg * 16 * DV;
  constexpr int FF = 8, FW = 2, NP = 16 * DV / 2 / NTH;  // fast-path partial counts; output pairs per thread
  const bool fast = p.nfin <= FF && p.nwin <= FW;        // workgroup-uniform
  f32x2_t ro[NP][FF], rw[NP][FW], rc[NP];
  float fm[FF], fl[FF], wm[FW], wl[FW];
  if (fast) {  // every load of the merge in flight at once
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int e2 = 2 * (tid + NTH * u);
      rc[u] = ld2_shared_dev(oc_src + e2);
#pragma unroll
      for (int k = 0; k < FF; ++k) ro[u][k] = k < p.nfin ? ld2_shared_dev(rp + (size_t)k * PSTRIDE + 32 + e2) : f32x2_t{0.f, 0.f};
#pragma unroll
      for (int k = 0; k < FW; ++k) {
        const float* src = wp + (size_t)k * PSTRIDE + 32 + e2;
        rw[u][k] = k < p.nwin ? f32x2_t{src[0], src[1]} : f32x2_t{0.f, 0.f};
      }
    }
    if (tid < 16) {
#pragma unroll
      for (int k = 0; k < FF; ++k) {
        fm[k] = k < p.nfin ? ld_shared_dev(rp + (size_t)k * PSTRIDE + tid) : -INFINITY;
        fl[k] = k < p.nfin ? ld_shared_dev(rp + (size_t)k * PSTRIDE + 16 + tid) : 0.f;
      }
#pragma unroll
      for (int k = 0; k < FW; ++k) {
        wm[k] = k < p.nwin ? wp[(size_t)k * PSTRIDE + tid] : -INFINITY;
        wl[k] = k < p.nwin ? wp[(size_t)k * PSTRIDE + 16 + tid] : 0.f;
      }
    }
  }
  if (tid < 16) {  // per-head merge factors of the selected and window partials
    const int h = tid;
    float ls = 0.f, lw = 0.f;
    if (fast) {  // static indexing only: the loaded values stay in registers
      float M = -INFINITY, Mw = -INFINITY;
#pragma unroll
      for (int k = 0; k < FF; ++k) M = fmaxf(M, fm[k]);
#pragma unroll
      for (int k = 0; k < FW; ++k) Mw = fmaxf(Mw, wm[k]);
#pragma unroll
      for (int k = 0; k < FF; ++k) {
        const float a = fm[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fm[k] - M);
        s_pf[k][h] = a;
        ls += a * fl[k];
      }
#pragma unroll
      for (int k = 0; k < FW; ++k) {
        const float a = wm[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(wm[k] - Mw);
        s_wf[k][h] = a;
        lw += a * wl[k];
      }
    } else {
      float M = -INFINITY, Mw = -INFINITY;
      for (int k = 0; k < p.nfin; ++k) M = fmaxf(M, ld_shared_dev(rp + (size_t)k * PSTRIDE + h));
      for (int k = 0; k < p.nwin; ++k) Mw = fmaxf(Mw, wp[(size_t)k * PSTRIDE + h]);
      for (int k = 0; k < p.nfin; ++k) {
        const float mk = ld_shared_dev(rp + (size_t)k * PSTRIDE + h);
        const float a = mk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mk - M);
        s_pf[k][h] = a;
        ls += a * ld_shared_dev(rp + (size_t)k * PSTRIDE + 16 + h);
      }
      for (int k = 0; k < p.nwin; ++k) {
        const float mk = wp[(size_t)k * PSTRIDE + h];
        const float a = mk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mk - Mw);
        s_wf[k][h] = a;
        lw += a * wp[(size_t)k * PSTRIDE + 16 + h];
      }
    }
    const float is = ls > 0.f ? 1.0f / ls : 0.f, iw = lw > 0.f ? 1.0f / lw : 0.f;
    for (int k = 0; k < p.nfin; ++k) s_pf[k][h] *= is;
    for (int k = 0; k < p.nwin; ++k) s_wf[k][h] *= iw;
  }
  lds_barrier();
  auto emit = [&](int e, float oc, float os, float ow) {  // output e of the group's 16 x DV
    const int h = e / DV;
    if (h >= p.G) return;
    const int hq = g * p.G + h;
    p.out[((size_t)b * p.Hq + hq) * DV + (e - h * DV)] =
        (uint16_t)f32_to_bf16(s_gate[h][0] * oc + s_gate[h][1] * os + s_gate[h][2] * ow);
  };
  if (fast) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int e2 = 2 * (tid + NTH * u), h = e2 / DV;
      float os0 = 0.f, os1 = 0.f, ow0 = 0.f, ow1 = 0.f;
#pragma unroll
      for (int k = 0; k < FF; ++k) {
        const float a = k < p.nfin ? s_pf[k][h] : 0.f;
        os0 += a * ro[u][k][0];
        os1 += a * ro[u][k][1];
      }
#pragma unroll
      for (int k = 0; k < FW; ++k) {
        const float a = k < p.nwin ? s_wf[k][h] : 0.f;
        ow0 += a * rw[u][k][0];
        ow1 += a * rw[u][k][1];
      }
      emit(e2, rc[u][0], os0, ow0);
      emit(e2 + 1, rc[u][1], os1, ow1);
    }
  } else {
    for (int e = tid; e < p.G * DV; e += NTH) {
      const int h = e / DV;
      float os = 0.f, ow = 0.f;
      for (int k = 0; k < p.nfin; ++k) os += s_pf[k][h] * ld_shared_dev(rp + (size_t)k * PSTRIDE + 32 + e);
      for (int k = 0; k < p.nwin; ++k) ow += s_wf[k][h] * wp[(size_t)k * PSTRIDE + 32 + e];
      emit(e, ld_shared_dev(oc_src + e), os, ow);
    }
  }
}

// ---------------------------------------------------------------- host side

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeLayout decode_layout(int B, int H, int DV, int l, int d, int lsel, int n, int nloc, int w, int64_t max_len) {
  (void)nloc;  // the always-taken blocks are part of the n selected blocks
  DecodeLayout lay{};
  const int64_t nc = max_len >= l ? (max_len - l) / d + 1 : 0;
  const int r = lsel / d;
  const int64_t gran = r > 64 ? r : 64;  // segments hold whole tiles and whole selection blocks
  auto up = [&](int64_t x) { return (x + gran - 1) / gran * gran; };
  // Rows per (sequence, group): the compressed keys plus the window's tiles,
  // spread over about kStreamSlots / (B*H) workgroups (at least one segment and
  // one window workgroup).
  const int64_t win_tiles = (w + 63) / 64 + 1;
  const int64_t bh = (int64_t)B * H;
  const int64_t per_bg = bh >= kStreamSlots / 2 ? 2 : kStreamSlots / bh;
  int64_t seg = up((nc + 64 * win_tiles + per_bg - 1) / per_bg);
  const int64_t seg_min = up((nc + kMaxChunks - 1) / kMaxChunks);
  const int64_t seg_max = (int64_t)(kScStrideMax - 4) * r / gran * gran;  // score rows fit the LDS table
  if (seg < seg_min) seg = seg_min;
  if (seg > seg_max) seg = seg_max;  // the host rejects seg_min > seg_max
  if (seg < gran) seg = gran;
  lay.seg = (int)seg;
  lay.nch = (int)((nc + seg - 1) / seg);
  if (lay.nch < 1) lay.nch = 1;
  lay.nbo = (int)(seg / r);
  int64_t wt = seg / 64;
  if (wt * kMaxWindow < win_tiles) wt = (win_tiles + kMaxWindow - 1) / kMaxWindow;
  lay.wtiles = (int)wt;
  lay.nwin = (int)((win_tiles + wt - 1) / wt);
  const size_t BH = (size_t)B * H;
  size_t off = 0;
  lay.off_m1 = off;   off = align256(off + BH * lay.nch * 16 * 4);
  lay.off_l1 = off;   off = align256(off + BH * lay.nch * 16 * 4);
  lay.off_o1 = off;   off = align256(off + BH * lay.nch * 16 * (size_t)DV * 4);
  lay.off_sc1 = off;  off = align256(off + BH * lay.nch * 16 * (size_t)(lay.nbo + 1) * 4);
  lay.off_wpart = off; off = align256(off + BH * lay.nwin * (32 + 16 * (size_t)DV) * 4);
  // finish workgroups (4 waves, one 32-token step each): one partial each; the
  // normalised compressed-branch output; the arrival counters
  const int spb = lsel >= 32 ? lsel / 32 : 1;
  lay.nfin = (n * spb + NSA_FIN_WAVES - 1) / NSA_FIN_WAVES;
  lay.off_rpart = off; off = align256(off + BH * lay.nfin * (32 + 16 * (size_t)DV) * 4);
  lay.off_ocmp = off; off = align256(off + BH * 16 * (size_t)DV * 4);
  lay.off_cnt = off; off = align256(off + BH * 4);
  lay.total = off;
  return lay;
}

// With events, each kernel is launched with its start / stop events attached
// to the dispatch (ev[0], ev[1]: streaming kernel; ev[2], ev[3]: finish kernel),
// so their elapsed times are the kernels' own execution times.
template <int DK, int DV>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s, const PhaseEvents* ev) {
  hipEvent_t e0 = ev ? ev->ev[0] : nullptr, e1 = ev ? ev->ev[1] : nullptr;
  hipEvent_t e2 = ev ? ev->ev[2] : nullptr, e3 = ev ? ev->ev[3] : nullptr;
  hipExtLaunchKernelGGL((decode_stream_kernel<DK, DV>), dim3((unsigned)(p.B * p.H * (p.nch + p.nwin))),
                        dim3(64 * kStreamWaves), 0, s, e0, e1, 0, p);
  hipError_t e;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 g2((unsigned)(p.B * p.H * p.nfin)), blk(64 * NSA_FIN_WAVES);
  switch (p.lsel) {
    case 16: hipExtLaunchKernelGGL((decode_finish_kernel<DK, DV, 16>), g2, blk, 0, s, e2, e3, 0, p); break;
    case 32: hipExtLaunchKernelGGL((decode_finish_kernel<DK, DV, 32>), g2, blk, 0, s, e2, e3, 0, p); break;
    case 64: hipExtLaunchKernelGGL((decode_finish_kernel<DK, DV, 64>), g2, blk, 0, s, e2, e3, 0, p); break;
    case 128: hipExtLaunchKernelGGL((decode_finish_kernel<DK, DV, 128>), g2, blk, 0, s, e2, e3, 0, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int DK, int DV, hipStream_t s, const PhaseEvents* ev) {
  if (DK == 192 && DV == 128) return launch_decode_t<192, 128>(p, s, ev);
  if (DK == 128 && DV == 128) return launch_decode_t<128, 128>(p, s, ev);
  if (DK == 64 && DV == 64) return launch_decode_t<64, 64>(p, s, ev);
  return hipErrorInvalidValue;
}

}  // namespace nsa

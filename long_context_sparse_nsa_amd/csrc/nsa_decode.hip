// NSA decode step on gfx950: two launches per step.  Between them the kernel
// boundary is the synchronisation; inside the second, one device-scope counter
// per (sequence, group) finds the workgroup that finishes last.
//
// 1. decode_stream_kernel, about one workgroup per compute unit, two kinds:
//    - segment workgroups: the compressed branch, split over segments of
//      compressed keys per (sequence, KV group).  Each streams its segment of
//      the compressed cache once into registers, computes the 16-head logits
//      with MFMA, the segment's softmax statistics and partial output, and the
//      per-head probabilities folded onto selection blocks;
//    - window workgroups: the window branch, which does not depend on the
//      selection, streamed the same way over the window's raw tokens.
//    The segments are planned on the host from the longest length, or, when
//    that plan needs more workgroups than compute units (a ragged batch of
//    many long slots), on the device from the actual lengths (balanced plan).
// 2. decode_finish_kernel: several workgroups of 4 waves (8 when 4-wave ones
//    would be more than one per compute unit) per (sequence, group), each
//    computing the exact per-head normalisers from the segment statistics, the
//    group scores and the top-n (one wave), a slice of the compressed-branch
//    output, and its share of the selected blocks (one 32-token step per
//    wave); the last of them to finish merges the partials and applies the
//    gates: out = g_cmp*o_cmp + g_slc*o_slc + g_win*o_win in bf16.
//
// Sources: lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc),
// section "NSA: три ветви" (output equation; compressed branch l=32, d=16;
// selection of n l'-blocks re-using the compressed-branch weights, shared by a
// GQA group so each KV block is read once per group; window of w tokens) and
// section "Сколько это экономит" (decode is bound by reading the KV cache).
#include <algorithm>

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

// ---- balanced plan of a ragged batch (p.bal): every compressed segment holds
// T tiles of kStreamTile keys (a sequence's last one fewer), with T chosen from
// the actual lengths so that the segments of all units fill about p.bal_fill
// slots.  Sequence b has tiles_b = ceil(n_visible / kStreamTile) tiles and
// c_b = ceil(tiles_b / T) segments per group; unit (b, g) owns the slots
// [base_b + g*c_b, base_b + (g+1)*c_b), base_b = H * sum over b' < b of c_b'.
// The helpers are wave-wide (every lane of the calling wave takes part; the
// results are wave-uniform) and read the lengths with one vector load per lane
// and 64 sequences.
__device__ __forceinline__ int lane_tiles(const DecodeParams& p, int b) {
  int64_t cap = p.cap, ccap = p.ccap;
  if (p.cu) {
    const int64_t c = p.cu[b + 1] - p.cu[b];
    if (c < cap) cap = c;
  }
  if (p.cuc) ccap = p.cuc[b + 1] - p.cuc[b];
  int64_t L = p.seq_lens[b];
  if (L > cap) L = cap;
  if (L < 1) L = 1;
  int64_t nv = L >= p.l ? (L - p.l) / p.d + 1 : 0;
  if (nv > ccap) nv = ccap;
  return (int)((nv + kStreamTile - 1) / kStreamTile);
}
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}
// T, or 0 when even segments of tcap tiles would not fit in about one round
// (every sequence long): then the fixed plan is used.  With at most 64
// sequences, *tl gets the lane's own sequence's tiles, so that the calls below
// need no second round of loads.
__device__ __forceinline__ int bal_tiles_per_segment(const DecodeParams& p, int* tl) {
  const int lane = threadIdx.x & 63;
  int tot = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int x = b0 + lane < p.B ? lane_tiles(p, b0 + lane) : 0;
    tot += wave_sum_int(x);
    *tl = x;
  }
  int T = (p.H * tot + p.bal_fill - 1) / p.bal_fill;
  if (T < p.tmin) T = p.tmin;
  if (T > p.tcap) T = 0;
  return __builtin_amdgcn_readfirstlane(T);
}
// The unit and segment of compressed slot s; false for a slot past every unit's segments.
__device__ __forceinline__ bool bal_slot(const DecodeParams& p, int T, int tl, int s, int& b, int& g, int& k) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int bb = b0 + lane;
    const int cb = bb < p.B ? ((p.B <= 64 ? tl : lane_tiles(p, bb)) + T - 1) / T : 0;
    const int incl = wave_incl_scan(p.H * cb);
    const int excl = incl - p.H * cb;
    const uint64_t hit = __ballot(cb > 0 && s >= base + excl && s < base + incl);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      const int c = __builtin_amdgcn_readlane(cb, src);
      const int off = s - base - __builtin_amdgcn_readlane(excl, src);
      b = b0 + src;
      g = off / c;
      k = off - g * c;
      return true;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  return false;
}
// The first slot and the number of segments of unit (b, g).
__device__ __forceinline__ void bal_unit(const DecodeParams& p, int T, int tl, int b, int g, int& first, int& count) {
  const int lane = threadIdx.x & 63;
  int base = 0, cnt = 0;
  for (int b0 = 0; b0 <= b; b0 += 64) {
    const int bb = b0 + lane;
    const int cb = bb < p.B ? ((p.B <= 64 ? tl : lane_tiles(p, bb)) + T - 1) / T : 0;
    base += wave_sum_int(bb < b ? p.H * cb : 0);
    if (b < b0 + 64) cnt = __builtin_amdgcn_readlane(cb, b - b0);
  }
  first = __builtin_amdgcn_readfirstlane(base + g * cnt);
  count = __builtin_amdgcn_readfirstlane(cnt);
}

// Stores and loads that are coherent across the whole device without cache
// maintenance (relaxed atomics at agent scope): the selection workgroups of one
// (sequence, group) hand their partials to the last of them this way.
//
// Why relaxed atomics and a wait are enough here.  The partials are written
// with agent-scope atomic stores, which the hardware writes through to the
// device-coherent level (they are never held dirty in an XCD's L2); the writer
// then waits until all of its stores are acknowledged (s_waitcnt vmcnt(0),
// written as asm with a memory clobber, so the compiler keeps every store
// before it) and only then increments the arrival counter.  The workgroup that
// sees the final count issues its loads only after the counter's value has
// returned, and reads with agent-scope atomic loads, which bypass the
// non-coherent caches.  So every partial is in memory before its writer's
// increment and is read from memory after the last increment.  A release /
// acquire pair would instead write back and invalidate the whole L2 of the
// XCD per workgroup, which costs far more than this hand-off.
__device__ __forceinline__ void wait_stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The same device-coherent accesses 16 bytes at a time, through a buffer
// resource: cache policy sc1 is what the compiler emits for the agent-scope
// relaxed atomics above (checked in the generated code), which it offers only
// up to 8 bytes.  Offsets are in bytes; accesses past `bytes` read 0 and are
// dropped by the hardware's range check.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kCoherent = 16;  // cache-policy operand: sc1
__device__ __forceinline__ rsrc_t coherent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4_t ld4_coherent(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoherent));
}
__device__ __forceinline__ float ld1_coherent(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kCoherent));
}
__device__ __forceinline__ void st4_coherent(rsrc_t r, uint32_t off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)off, 0, kCoherent);
}
__device__ __forceinline__ void st1_coherent(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, kCoherent);
}
// The selected-branch partials keep o / l as fp16: weighted averages of bf16
// values, so fp16's 11-bit significand adds about 2^-12 relative error, well
// below the bf16 rounding of the result, at half the bytes of fp32.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
}
__device__ __forceinline__ f32x2_t unpack_f16x2(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
}
__device__ __forceinline__ void st8_coherent(rsrc_t r, uint32_t off, u32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kCoherent);
}
__device__ __forceinline__ u32x4_t ld16_coherent(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoherent);
}
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

}  // namespace

// ---------------------------------------------------------------- streaming pass

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

// A whole 32-token step [x0, x0 + 32) of the raw cache (every row exists) in
// the Step layout, addressed as scalar base + this lane's 32-bit offsets:
// koff = (lr*DK + 8*lg)*2 and voff = (4*lg*DV + (DV/16)*lr)*2 bytes.
template <int DK, int DV>
__device__ __forceinline__ void step_load_full(Step<DK, DV>& st, const uint16_t* kb, const uint16_t* vb, int64_t x0,
                                               uint32_t koff, uint32_t voff) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const gchar_ptr kp = scalar_ptr(kb + (x0 + 16 * tt) * DK) + koff;
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) st.kf[tt][kk] = ld_global<u32x4_t>(kp + 64 * kk);
  }
  const gchar_ptr vp = scalar_ptr(vb + x0 * DV) + voff;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int key = r < 4 ? r : 12 + r;  // step_key(lg, r) - 4*lg
    if constexpr (DV / 32 == 4) {
      const u32x4_t x = ld_global<u32x4_t>(vp + key * DV * 2);
      st.vr[r][0] = x[0]; st.vr[r][1] = x[1]; st.vr[r][2] = x[2]; st.vr[r][3] = x[3];
    } else {
      const u32x2_t x = ld_global<u32x2_t>(vp + key * DV * 2);
      st.vr[r][0] = x[0]; st.vr[r][1] = x[1];
    }
  }
}

// Workgroup of the streaming pass: kStreamWaves waves stream the rows of a
// segment of the compressed cache (or of part of the window of the raw cache)
// as kStreamTile-row tiles; wave w owns rows 16w .. 16w+15 of every tile and loads them
// straight into registers, kDepth - 1 tiles ahead of the one it computes:
//   logits  S^T = K . q^T                      (16x16x32 MFMA, d_k/32 k-steps)
//   values  O^T += V^T . P^T                   (16x16x16 MFMA; P^T is the logit tile)
//   scores  F^T  = Omega^T . P^T (P as bf16 hi + lo) (16x16x16 MFMA), added into the
//           per-head score rows of the segment's selection blocks in LDS, in a
//           fixed order, so repeated calls give identical results
// Omega[key][block] is the number of stride units key and block share (an exact
// small integer; divided by l/d when the scores are written out).  Each wave
// keeps its own softmax reference per head, moved (rescaling its outputs and
// sums) only when a tile maximum exceeds it by kLazy, so the tile loop has no
// barrier and the waves stream independently.  A wave's fold rows of every tile
// are kept in LDS with the reference they were computed against; at the end the
// workgroup merges the waves' (m, l, o) and sums each block's fold rows, scaled
// to the common reference, in tile and wave order, so repeated calls give
// identical results.
//
// Outputs per compressed segment: the reference m, the sum l of exp2(z - m), the
// unnormalised output sum, and the selection-block scores (slot nbo is the
// overhang into the first block of the next segment).  Per window workgroup:
// the same (m, l, o) triple over its window tokens.
template <int DK, int DV>
__global__ __launch_bounds__(64 * kStreamWaves, 1) void decode_stream_kernel(DecodeParams p) {
  constexpr int NW = kStreamWaves, NTH = 64 * NW, KT = DK / 32, VC = DV / 16;
  constexpr int TR = kStreamTile;  // rows per tile
  constexpr int kDepth = 2;        // register tiles per wave (two waves per SIMD: one in flight while one is computed)
  constexpr int PSTRIDE = 32 + 16 * DV;
  constexpr float kLazy = 8.0f, kNegBig = -1e30f;
  __shared__ float s_o[NW][16][DV + 1];
  constexpr int FWP = 20;  // each head's fold rows padded: distinct LDS banks for the 16 heads
  __shared__ __attribute__((aligned(16))) float s_fw[kSegTiles][NW][16][FWP];  // fold rows [tile][wave][head][block row]
  __shared__ float s_fm[kSegTiles][NW][16];  // the reference each tile's fold rows are relative to
  __shared__ float s_l[NW][16], s_m[NW][16], s_fac[NW][16];

  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> unit bg and compressed segment (c < nch: keys [k0, k0 + seg) into
  // output slot `slot`) or window part c - nch
  int bg, c, seg, k0 = 0, slot = 0;
  int tl = 0;
  const int T = p.bal ? bal_tiles_per_segment(p, &tl) : 0;
  if (T == 0) {  // the fixed plan
    const int per = p.nch + p.nwin;
    bg = blockIdx.x / per;
    if (bg >= p.B * p.H) return;  // the launch is sized for either plan
    c = blockIdx.x - bg * per;
    seg = p.seg;
    k0 = c * seg;
    slot = bg * p.nch + c;
  } else if ((int)blockIdx.x < p.B * p.H * p.nwin) {  // window parts first
    bg = blockIdx.x / p.nwin;
    c = p.nch + (blockIdx.x - bg * p.nwin);
    seg = 0;
  } else {
    slot = blockIdx.x - p.B * p.H * p.nwin;
    int sb, sg, sk;
    if (!bal_slot(p, T, tl, slot, sb, sg, sk)) return;  // a slot past every unit's segments
    bg = sb * p.H + sg;
    c = 0;
    seg = T * kStreamTile;
    k0 = sk * seg;
  }
  const int g = bg % p.H, b = bg / p.H;
  const bool fold = c < p.nch;  // workgroup-uniform: compressed segment, else window part
  clk_stamp(p.clk, 0);
  const uint32_t koff = (uint32_t)((lr * DK + 8 * lg) * 2), voff = (uint32_t)((4 * lg * DV + VC * lr) * 2);
  u32x4_t qf[KT];
  WaveTile<DK, DV> tb[kDepth];
  auto load_q = [&]() { load_q_frags<DK>(p.q + ((int64_t)b * p.Hq + (int64_t)g * p.G) * DK, p.G, lg, lr, qf); };

  // rows [r0, r0 + TR*nt) are streamed; keys outside [vlo, vhi] are masked
  int64_t r0, rowmax;
  int nt, vlo, vhi;
  const uint16_t *kb, *vb;
  int L;
  if (fold) {
    // A segment's rows and its slot's capacity do not depend on the sequence
    // length, so the first tiles are requested while the length is read; rows
    // past the length are masked (their values are zeroed before use).
    const int64_t ccap_b = p.cuc ? ld_scalar(p.cuc + b + 1) - ld_scalar(p.cuc + b) : p.ccap;
    if (k0 >= ccap_b) return;  // beyond the slot: never read by the selection kernel
    const int64_t rpre = min((int64_t)k0 + seg, ccap_b) - 1;
    const int64_t crow = cmp_row0(p, b, g);
    kb = p.kc + crow * DK;
    vb = p.vc + crow * DV;
    L = seq_len_clamped(p, b);
    load_q();
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d)
      load_wave_tile<DK, DV>(tb[d], kb, vb, (int64_t)k0 + TR * d + 16 * wave, rpre, koff, voff, lg, lr);
    const int nvis = n_visible(p, b, L);
    if (k0 >= nvis) {  // empty segment: never read by the selection kernel
      wait_vmem();
      return;
    }
    const int k1 = min(k0 + seg, nvis);
    r0 = k0;
    nt = (k1 - k0 + TR - 1) / TR;
    vlo = k0;
    vhi = k1 - 1;
    rowmax = nvis - 1;
  } else {
    const int wi = c - p.nch;
    if (wi == 0 && tid == 0) p.cnt[bg] = 0u;  // arrival counter of the selection workgroups
    L = seq_len_clamped(p, b);
    const int t = L - 1;
    const int wlo = t - p.w + 1 > 0 ? t - p.w + 1 : 0;
    const int T0 = wlo / TR + wi * p.wtiles, T1 = min(wlo / TR + (wi + 1) * p.wtiles, t / TR + 1);
    r0 = (int64_t)T0 * TR;
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
      load_wave_tile<DK, DV>(tb[d], kb, vb, r0 + TR * d + 16 * wave, min(rowmax, r0 + TR * (int64_t)nt - 1), koff,
                             voff, lg, lr);
  }

  // Loads never read past the workgroup's own last row: requests for tiles
  // beyond the range (issued so that every pipeline step has the same loads in
  // flight) re-read that row from cache.
  const int64_t rlast = min(rowmax, r0 + TR * (int64_t)nt - 1);

  const int qd = p.l / p.d, rd = p.lsel / p.d;  // key and block lengths in stride units
  const int rsh = __builtin_ctz(rd);            // rd is a power of two
  const int jseg0 = fold ? (int)(r0 >> rsh) : 0;
  f32x4_t acc[VC];
#pragma unroll
  for (int j = 0; j < VC; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f, mref = kNegBig;
  const float sc = p.scale_log2;

  auto process = [&](int i, const WaveTile<DK, DV>& T) {
    const int64_t k0 = r0 + TR * i + 16 * wave;  // the wave's first row
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
    float mt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mt = max_over_groups_swap(mt);  // head lr's maximum over the wave's 16 rows

    // ---- lazy move of this wave's reference
    const bool move = mt > mref + kLazy;
    if (__ballot(move) != 0ull) {
      const float mn = move ? mt : mref;
      const float alpha = __builtin_amdgcn_exp2f(mref - mn);
#pragma unroll
      for (int j = 0; j < VC; ++j) acc[j] *= alpha;
      lsum *= alpha;
      mref = mn;
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
      *reinterpret_cast<f32x4_t*>(&s_fw[i][wave][lr][4 * lg]) = f;
      if (lg == 0) s_fm[i][wave][lr] = mref;
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
      load_wave_tile<DK, DV>(tb[(u + kDepth - 1) % kDepth], kb, vb, r0 + TR * (i0 + u + kDepth - 1) + 16 * wave,
                             rlast, koff, voff, lg, lr);
      process(i0 + u, tb[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < kDepth - 1; ++u)
    if (i0 + u < nt) process(i0 + u, tb[u]);  // workgroup-uniform
  clk_stamp(p.clk, 1);

  // ---- workgroup merge: the waves' (m, l, o) to the common reference M (per head)
  lsum = sum_over_groups_swap(lsum);
  if (lg == 0) {
    s_l[wave][lr] = lsum;
    s_m[wave][lr] = mref;
  }
#pragma unroll
  for (int j = 0; j < VC; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_o[wave][lr][acc_channel<DV>(lg, e, j)] = acc[j][e];
  lds_barrier();
  float Mh = s_m[0][lr];
#pragma unroll
  for (int w = 1; w < NW; ++w) Mh = fmaxf(Mh, s_m[w][lr]);  // lane lr: head lr
  if (tid < 16 * NW) s_fac[tid >> 4][lr] = __builtin_amdgcn_exp2f(s_m[tid >> 4][lr] - Mh);  // (wave, head)
  if (fold) {  // the fold rows' references become their factors to M (entry e: head e mod 16 = lr)
    float* fm = &s_fm[0][0][0];
    for (int e = tid; e < NW * nt * 16; e += NTH) fm[e] = __builtin_amdgcn_exp2f(fm[e] - Mh);
  }
  clk_stamp(p.clk, 3);
  lds_barrier();
  float *dm, *dl, *dox;
  if (fold) {
    dm = p.m1 + (size_t)slot * 16;
    dl = p.l1 + (size_t)slot * 16;
    dox = p.o1 + (size_t)slot * 16 * DV;
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
      for (int w = 0; w < NW; ++w) v += s_fac[w][h] * s_o[w][h][ch];
      dox[h * DV + ch] = v;
    }
  clk_stamp(p.clk, 4);
  if (tid < 16) {  // lane tid: head tid (Mh of lane tid is head tid's)
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) ls += s_fac[w][tid] * s_l[w][tid];
    dl[tid] = ls;
    dm[tid] = Mh;
  }
  if (fold) {
    // Scores of the segment's blocks jseg0 .. jseg0 + nbo (slot nbo is the
    // overhang into the next segment's first block): block J sums the fold rows
    // J - j0 of the wave-tiles whose keys reach into it, each scaled from its
    // own reference to M, in tile and wave order.
    const int slots = seg / rd + 1;  // the segment's blocks and the overhang
    const float invq = 1.0f / (float)qd;
    float* SC = p.sc1 + (size_t)slot * p.scs * 16;  // [slot][head]
    const float(*fm)[16] = reinterpret_cast<const float(*)[16]>(&s_fm[0][0][0]);        // [u][head]
    const float(*fw)[16][FWP] = reinterpret_cast<const float(*)[16][FWP]>(&s_fw[0][0][0][0]);  // [u][head][row]
    // With l <= l' (qd <= rd) and rd <= 16, every wave-tile starts on a block
    // boundary, own = 16/rd blocks apart, and at most two wave-tiles reach a
    // block: slot s = u*own + k takes row k of wave-tile u and row k + own of
    // wave-tile u - 1 (rows past the keys' reach are exact zeros).  Four entries
    // per thread and pass, all their reads issued before any is used; the two
    // terms are added in wave-tile order.
    if (rd <= 16) {
      const int osh = 4 - rsh, own = 1 << osh, nu = NW * nt;
      constexpr int EB = 4;
      for (int e0 = tid; e0 < 16 * slots; e0 += EB * NTH) {
        float x0[EB], x1[EB];
#pragma unroll
        for (int q = 0; q < EB; ++q) {
          const int e = e0 + q * NTH;
          const int sl = e >> 4, u = sl >> osh, k = sl & (own - 1);
          const bool in = e < 16 * slots;
          const bool ok0 = in && u < nu;
          const bool ok1 = in && u >= 1 && u - 1 < nu && k + own < 16;
          const int ua = ok0 ? u : 0, ka = ok0 ? k : 0, ub = ok1 ? u - 1 : 0, kb = ok1 ? k + own : 0;
          const float a = fm[ua][lr] * fw[ua][lr][ka];
          const float c = fm[ub][lr] * fw[ub][lr][kb];
          x0[q] = ok0 ? a : 0.f;
          x1[q] = ok1 ? c : 0.f;
        }
#pragma unroll
        for (int q = 0; q < EB; ++q) {
          const int e = e0 + q * NTH;
          if (e < 16 * slots) SC[e] = (x1[q] + x0[q]) * invq;
        }
      }
    } else {
      for (int e = tid; e < 16 * slots; e += NTH) {  // head e mod 16 = lr
        const int J = jseg0 + (e >> 4);
        // wave-tiles u = NW*i + w start at key r0 + 16u; their keys [K, K + 15 + qd - 1]
        // (stride units) reach block J iff K <= J*rd + rd - 1 and K + 15 + qd - 1 >= J*rd
        const int klo = J * rd - (15 + qd - 1) - (int)r0, khi = J * rd + rd - 1 - (int)r0;
        const int ulo = klo > 0 ? (klo + 15) >> 4 : 0;
        const int uhi = khi >= 0 ? min(khi >> 4, NW * nt - 1) : -1;
        float v = 0.f;
        for (int u = ulo; u <= uhi; ++u) {
          const int row = J - (((int)r0 + 16 * u) >> rsh);
          if (row >= 0 && row < 16) v += fm[u][lr] * fw[u][lr][row];
        }
        SC[e] = v * invq;
      }
    }
  }
  clk_stamp(p.clk, 2);
}

// Merges the NWV waves' selected-branch states into one partial and stores it
// device-coherently at byte offset `off` of r: m[16], l[16] (fp32) and the
// output divided by l, o[16][DV] (fp16, from byte 128; the last workgroup
// weights it by its share of the total).  buf holds NWV*16*(DV+1) floats,
// st 2*NWV*16.
template <int DV, int NWV>
__device__ __forceinline__ void merge_store(const Branch<DV>& a, float* buf, float* st, rsrc_t r, uint32_t off) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  constexpr int NTH = 64 * NWV, RS = NWV * 16;
  if (lg == 0) {
    st[wave * 16 + lr] = a.m;
    st[RS + wave * 16 + lr] = a.l;
  }
  lds_barrier();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NWV; ++w) M = fmaxf(M, st[w * 16 + lr]);
  const float fa = a.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(a.m - M);
#pragma unroll
  for (int j = 0; j < DV / 16; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) buf[(wave * 16 + lr) * (DV + 1) + acc_channel<DV>(lg, i, j)] = fa * a.acc[j][i];
  lds_barrier();
  // four consecutive outputs of one head per thread and pass
  for (int e = 4 * tid; e < 16 * DV; e += 4 * NTH) {
    const int h = e / DV, ch = e - h * DV;
    float Mh = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) Mh = fmaxf(Mh, st[w * 16 + h]);
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float mw = st[w * 16 + h];
      if (mw != -INFINITY) ls += __builtin_amdgcn_exp2f(mw - Mh) * st[RS + w * 16 + h];
    }
    const float inv = ls > 0.f ? 1.0f / ls : 0.f;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NWV; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += buf[(w * 16 + h) * (DV + 1) + ch + i];
    v *= inv;
    st8_coherent(r, off + 128 + (uint32_t)e * 2, u32x2_t{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])});
  }
  if (tid < 16) {
    float Mh = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) Mh = fmaxf(Mh, st[w * 16 + tid]);
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float mw = st[w * 16 + tid];
      if (mw != -INFINITY) ls += __builtin_amdgcn_exp2f(mw - Mh) * st[RS + w * 16 + tid];
    }
    st1_coherent(r, off + (uint32_t)tid * 4, Mh);
    st1_coherent(r, off + (uint32_t)(16 + tid) * 4, ls);
  }
}

// Finish: nfin workgroups of NWV waves per (sequence, group) (NWV = 4, or 8
// when 4-wave workgroups would be more than one per compute unit: fewer
// workgroups then read the group scores again).  Every one
// of them computes the exact per-head normalisers of the compressed branch,
// the group scores and the top-n (one wave; identical results in every
// workgroup, so no exchange is needed); then workgroup k
//   - sums its slice of the normalised compressed-branch output over the
//     segments (the loads are issued before the normalisers are known),
//   - attends the selected steps [4k, 4k+4) (one 32-token step per wave, over
//     all selected blocks in ascending order) and stores one partial.
// The last of the nfin workgroups to finish (a device-scope counter, cleared
// by the streaming pass) merges the selected-branch partials and the window
// partials and writes out = g_cmp*o_cmp + g_slc*o_slc + g_win*o_win in bf16.
template <int DK, int DV, int LSEL, int NWV>
__global__ __launch_bounds__(64 * NWV) void decode_finish_kernel(DecodeParams p) {
  constexpr int NTH = 64 * NWV;
  constexpr int KT = DK / 32;
  constexpr int SPB = LSEL >= 32 ? LSEL / 32 : 1;   // 32-token steps per selection block
  constexpr int WSTRIDE = 32 + 16 * DV;              // window partial (fp32 m, l, o), floats
  constexpr int RSTRIDE = 32 + 8 * DV;               // selected partial (m, l fp32; o / l fp16), in floats
  constexpr int RPT = 4;                             // candidate blocks per thread and load round
  constexpr int OB = 8;                              // segments per compressed-output load batch
  // The candidates' scores (until the top-n) share their LDS with the wave-merge
  // buffer (after the selected steps), and the two top-n paths share theirs, so
  // that two workgroups fit on a compute unit.
  constexpr int MB = NWV * 16 * (DV + 1);
  __shared__ __attribute__((aligned(16))) float s_big[MB > kMaxBlocks + 64 ? MB : kMaxBlocks + 64];
  __shared__ float s_f[kMaxChunks * 16];
  __shared__ float s_ml[2 * kMaxChunks * 16];       // segment m / l, then wave-merge scratch
  __shared__ float s_ov[kMaxChunks * 16];           // overhang score slot of each segment, per head
  struct TopnBlock {
    TopnSmem tsm;
    TopnFastSmem<NWV> tfs;
  };
  __shared__ union TopnLds {
    TopnBlock blk;                                  // the workgroup's top-n (more than 2048 candidates)
    uint64_t tw[416];                               // the single-wave top-n
  } s_topn;
  float* S = s_big;
  float* s_buf = s_big;
  TopnSmem& tsm = s_topn.blk.tsm;
  TopnFastSmem<NWV>& tfs = s_topn.blk.tfs;
  uint64_t* s_tw = s_topn.tw;
  __shared__ int s_sel[kMaxSel];
  __shared__ int s_items[kMaxSel];
  __shared__ int s_nitems;
  __shared__ int s_last;
  __shared__ float s_pf[kMaxFinish][16], s_wf[kMaxWindow][16];
  __shared__ float s_gate[16][3];

  // Workgroups are dealt to the 8 XCDs round-robin by id; when the sizes allow,
  // the nfin workgroups of one (sequence, group) get ids on the same XCD, so the
  // partials they hand over stay close.  Only speed depends on this.
  int bg, kfin;
  if ((p.B * p.H) % 8 == 0) {
    const int w = blockIdx.x, xcd = w & 7, r = w >> 3;
    bg = xcd + 8 * (r / p.nfin);
    kfin = r - (r / p.nfin) * p.nfin;
  } else {
    bg = blockIdx.x / p.nfin;
    kfin = blockIdx.x - bg * p.nfin;
  }
  uint64_t* clk = p.clk ? p.clk + (size_t)kClkMaxGroups * kClkSlots : nullptr;
  clk_stamp(clk, 0);
  const int g = bg % p.H, b = bg / p.H;
  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the unit's segment slots: nch segments of segk keys from slot cbase, nbo
  // selection blocks each, score rows `slots` apart
  int nch = p.nch, nbo = p.nbo, segk = p.seg;
  size_t cbase = (size_t)bg * nch;
  int tl = 0;
  const int T = p.bal ? bal_tiles_per_segment(p, &tl) : 0;
  if (T > 0) {  // from the balanced plan (every wave computes the same)
    int first, count;
    bal_unit(p, T, tl, b, g, first, count);
    nch = count;
    cbase = count > 0 ? (size_t)first : 0;  // no compressed block yet: nothing is read
    segk = T * kStreamTile;
    nbo = segk / (LSEL / p.d);
  }
  const int nchr = nch > 0 ? nch : 1;  // in-bounds clamp of the discarded loads
  const int slots = p.scs, nfin = p.nfin;
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
      if (cc >= nchr) cc = nchr - 1, jj = 0;  // beyond every sequence: read in bounds, discarded
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(p.sc1 + ((cbase + cc) * slots + jj) * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) vv[r][q] = src[q];
    }
  };
  load_scores(0);
  // compressed-branch output slice of this workgroup: outputs [e0, e1) of the
  // group's 16 x DV, one per thread and pass
  const int per = (16 * DV + nfin - 1) / nfin;
  const int e0 = kfin * per, e1 = min(e0 + per, 16 * DV);
  float vo[OB];
  {
    const int e = e0 + tid;
    const int ee = e < e1 ? e : e0;
#pragma unroll
    for (int q = 0; q < OB; ++q) vo[q] = p.o1[(cbase + min(q, nchr - 1)) * 16 * DV + ee];
  }
  u32x4_t qf[KT];
  load_q_frags<DK>(p.q + ((int64_t)b * p.Hq + (int64_t)g * p.G) * DK, p.G, lg, lr, qf);
  if (p.wgate) {  // gate network: 3 G dot products of the query with a weight row, four lanes each
    for (int f0 = 0; f0 < 12 * p.G; f0 += NTH) {  // one pass when NTH >= 12 G
      const int pr = (f0 + tid) >> 2, pt = tid & 3;
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
  const int nch_b = (nvis + segk - 1) / segk;
  const int t = L - 1;
  const int J = t / LSEL;
  lds_barrier();
  clk_stamp(clk, 1);

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
      for (int q = 0; q < OB; ++q) oc += q < nch_b ? s_f[q * 16 + h] * vo[q] : 0.f;
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
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) sc += s_f[cc * 16 + 4 * q + e] * vv[r][q][e];
      }
      if (jj == 0 && cc >= 1 && cc - 1 < nch_b) {  // overhang of the previous segment
#pragma unroll
        for (int h = 0; h < 16; ++h) sc += s_f[(cc - 1) * 16 + h] * s_ov[(cc - 1) * 16 + h];
      }
      S[j] = sc;
    }
  }
  lds_barrier();
  clk_stamp(clk, 2);
  {
    int32_t* so = (p.sel_out && kfin == 0) ? p.sel_out + (size_t)bg * p.n : nullptr;
    if (J + 1 <= 2048) {  // workgroup-uniform: one wave ranks, the others wait
      if (wave == 0) {
        const int cnt = J + 1 <= 1024 ? wave_topn_fast<16>(S, J, p.n, p.nloc, p.finit, s_tw, s_items, so)
                                      : wave_topn_fast<32>(S, J, p.n, p.nloc, p.finit, s_tw, s_items, so);
        if (lane == 0) s_nitems = cnt;
      }
    } else {
      block_topn_fast<NTH, 8, kMaxBlocks / NTH>(S, J, p.n, p.nloc, p.finit, tfs, tsm, s_sel, so);
      lds_barrier();
      if (wave == 0) {  // the selected blocks, ascending (the list ends at the first -1)
        const int j = lane < p.n ? s_sel[lane] : -1;
        const uint64_t m = __ballot(j >= 0);
        if (j >= 0) s_items[__popcll(m & ((1ull << lane) - 1ull))] = j;
        if (lane == 0) s_nitems = __popcll(m);
      }
    }
  }
  lds_barrier();
  clk_stamp(clk, 3);

  // ---- this workgroup's share of the selected steps: one 32-token step per
  // wave.  A full step reads its 32 rows through a scalar base; a step that
  // ends past the sequence is shifted back to end at its last token (the
  // earlier rows are masked), so no row past the length is read.
  Branch<DV> br;
  br.init();
  const int si = kfin * NWV + wave;
  const int nss = s_nitems * SPB;
  if (si < nss) {
    const int it = si / SPB, half = si - it * SPB;
    const int xb = s_items[it] * LSEL;
    const int x0 = xb + 32 * half;
    const int nv = min(L, xb + LSEL);
    if (x0 < nv) {  // wave-uniform
      const int64_t row = raw_row0(p, b, g);
      const uint16_t* kraw = p.k + row * DK;
      const uint16_t* vraw = p.v + row * DV;
      Step<DK, DV> st;
      int xs = x0;
      if (L >= 32) {
        xs = max(0, min(x0, nv - 32));
        step_load_full<DK, DV>(st, kraw, vraw, xs, (uint32_t)((lr * DK + 8 * lg) * 2),
                               (uint32_t)((4 * lg * DV + (DV / 16) * lr) * 2));
      } else {
        step_load<DK, DV>(st, kraw, vraw, x0, nv, lg, lr);
      }
      float z[2][4];
      step_logits<DK, DV>(st, qf, p.scale_log2, z);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int x = xs + 16 * tt + 4 * lg + e;
          if (x < x0 || x >= nv) z[tt][e] = -INFINITY;
        }
      br.update(z, st.vr);
    }
  }
  clk_stamp(clk, 4);
  float* rp = p.rpart + (size_t)bg * nfin * RSTRIDE;
  const rsrc_t rr = coherent_rsrc(rp, (uint32_t)(nfin * RSTRIDE * 4));
  if (e0 + tid < e1) st_shared_dev(p.ocmp + (size_t)bg * 16 * DV + e0 + tid, oc_first);
  const int nsp = min(nfin, (nss + NWV - 1) / NWV);  // partials that hold a step
  if (kfin < nsp) merge_store<DV, NWV>(br, s_buf, s_ml, rr, (uint32_t)kfin * RSTRIDE * 4);

  // ---- the last workgroup of this (sequence, group) applies the gates (the
  // hand-off is explained at wait_stores_done)
  wait_stores_done();
  lds_barrier();
  clk_stamp(clk, 5);
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(p.cnt + bg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (unsigned)(nfin - 1);
  lds_barrier();
  if (!s_last) return;
  clk_stamp(clk, 6);
  const rsrc_t ro = coherent_rsrc(p.ocmp + (size_t)bg * 16 * DV, 16 * DV * 4);
  const float* wp = p.wpart + (size_t)bg * p.nwin * WSTRIDE;
  const int nwin = p.nwin;
  // eight consecutive outputs e8 .. e8+7 of one head per thread (16*DV/8 threads)
  constexpr int NO = 16 * DV / 8;
  constexpr int FF = 8, FW = 2;                // fast-path partial counts
  const bool fast = nfin <= FF && nwin <= FW;  // workgroup-uniform
  const int e8 = 8 * (tid < NO ? tid : 0), h8 = e8 / DV;
  u32x4_t ro8[FF];
  f32x4_t rw8[FW][2], rc8[2];
  float fm[FF], fl[FF], wm[FW], wl[FW];
  if (fast) {  // every load of the merge in flight at once
    rc8[0] = ld4_coherent(ro, (uint32_t)e8 * 4);
    rc8[1] = ld4_coherent(ro, (uint32_t)(e8 + 4) * 4);
#pragma unroll
    for (int k = 0; k < FF; ++k)
      ro8[k] = k < nsp ? ld16_coherent(rr, (uint32_t)(k * RSTRIDE * 4 + 128 + e8 * 2)) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < FW; ++k)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        rw8[k][u] = k < nwin ? *reinterpret_cast<const f32x4_t*>(wp + (size_t)k * WSTRIDE + 32 + e8 + 4 * u)
                             : f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (tid < 16) {
#pragma unroll
      for (int k = 0; k < FF; ++k) {
        fm[k] = k < nsp ? ld1_coherent(rr, (uint32_t)(k * RSTRIDE + tid) * 4) : -INFINITY;
        fl[k] = k < nsp ? ld1_coherent(rr, (uint32_t)(k * RSTRIDE + 16 + tid) * 4) : 0.f;
      }
#pragma unroll
      for (int k = 0; k < FW; ++k) {
        wm[k] = k < nwin ? wp[(size_t)k * WSTRIDE + tid] : -INFINITY;
        wl[k] = k < nwin ? wp[(size_t)k * WSTRIDE + 16 + tid] : 0.f;
      }
    }
  }
  if (tid < 16) {  // per-head merge factors: selected partials (outputs already divided by their l)
    const int h = tid;
    float ls = 0.f, lw = 0.f;
    float M = -INFINITY, Mw = -INFINITY;
    if (fast) {  // static indexing only: the loaded values stay in registers
#pragma unroll
      for (int k = 0; k < FF; ++k) M = fmaxf(M, fm[k]);
#pragma unroll
      for (int k = 0; k < FW; ++k) Mw = fmaxf(Mw, wm[k]);
#pragma unroll
      for (int k = 0; k < FF; ++k) {
        const float a = fm[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fm[k] - M) * fl[k];
        s_pf[k][h] = a;
        ls += a;
      }
#pragma unroll
      for (int k = 0; k < FW; ++k) {
        const float a = wm[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(wm[k] - Mw);
        s_wf[k][h] = a;
        lw += a * wl[k];
      }
    } else {
      for (int k = 0; k < nsp; ++k) M = fmaxf(M, ld1_coherent(rr, (uint32_t)(k * RSTRIDE + h) * 4));
      for (int k = 0; k < nwin; ++k) Mw = fmaxf(Mw, wp[(size_t)k * WSTRIDE + h]);
      for (int k = 0; k < nsp; ++k) {
        const float mk = ld1_coherent(rr, (uint32_t)(k * RSTRIDE + h) * 4);
        const float a = mk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mk - M) * ld1_coherent(rr, (uint32_t)(k * RSTRIDE + 16 + h) * 4);
        s_pf[k][h] = a;
        ls += a;
      }
      for (int k = 0; k < nwin; ++k) {
        const float mk = wp[(size_t)k * WSTRIDE + h];
        const float a = mk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mk - Mw);
        s_wf[k][h] = a;
        lw += a * wp[(size_t)k * WSTRIDE + 16 + h];
      }
    }
    const float is = ls > 0.f ? 1.0f / ls : 0.f, iw = lw > 0.f ? 1.0f / lw : 0.f;
    for (int k = 0; k < nsp; ++k) s_pf[k][h] *= is;
    for (int k = 0; k < nwin; ++k) s_wf[k][h] *= iw;
  }
  lds_barrier();
  if (tid < NO && h8 < p.G) {
    float os[8], ow[8], oc[8];
    for (int i = 0; i < 8; ++i) os[i] = ow[i] = 0.f;
    if (fast) {
#pragma unroll
      for (int k = 0; k < FF; ++k) {
        const float a = k < nsp ? s_pf[k][h8] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x2_t x = unpack_f16x2(ro8[k][i]);
          os[2 * i] += a * x[0];
          os[2 * i + 1] += a * x[1];
        }
      }
#pragma unroll
      for (int k = 0; k < FW; ++k) {
        const float a = k < nwin ? s_wf[k][h8] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ow[i] += a * rw8[k][0][i];
          ow[4 + i] += a * rw8[k][1][i];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        oc[i] = rc8[0][i];
        oc[4 + i] = rc8[1][i];
      }
    } else {
      for (int k = 0; k < nsp; ++k) {
        const u32x4_t x = ld16_coherent(rr, (uint32_t)(k * RSTRIDE * 4 + 128 + e8 * 2));
        const float a = s_pf[k][h8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x2_t y = unpack_f16x2(x[i]);
          os[2 * i] += a * y[0];
          os[2 * i + 1] += a * y[1];
        }
      }
      for (int k = 0; k < nwin; ++k) {
        const float a = s_wf[k][h8];
        for (int i = 0; i < 8; ++i) ow[i] += a * wp[(size_t)k * WSTRIDE + 32 + e8 + i];
      }
      const f32x4_t c0 = ld4_coherent(ro, (uint32_t)e8 * 4), c1 = ld4_coherent(ro, (uint32_t)(e8 + 4) * 4);
      for (int i = 0; i < 4; ++i) {
        oc[i] = c0[i];
        oc[4 + i] = c1[i];
      }
    }
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = s_gate[h8][0] * oc[i] + s_gate[h8][1] * os[i] + s_gate[h8][2] * ow[i];
    *reinterpret_cast<u32x4_t*>(p.out + ((size_t)b * p.Hq + (size_t)g * p.G + h8) * DV + (e8 - h8 * DV)) =
        u32x4_t{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]), pack_bf16x2(r[6], r[7])};
  }
  clk_stamp(clk, 7);
}

// ---------------------------------------------------------------- host side

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeLayout decode_layout(int B, int H, int DV, int l, int d, int lsel, int n, int nloc, int w, int64_t max_len) {
  (void)nloc;  // the always-taken blocks are part of the n selected blocks
  DecodeLayout lay{};
  const int64_t nc = max_len >= l ? (max_len - l) / d + 1 : 0;
  const int r = lsel / d;
  const int64_t gran = r > kStreamTile ? r : kStreamTile;  // segments hold whole tiles and whole selection blocks
  auto up = [&](int64_t x) { return (x + gran - 1) / gran * gran; };
  // Rows per (sequence, group): the compressed keys plus the window's tiles,
  // spread over about kStreamSlots / (B*H) workgroups (at least one segment and
  // one window workgroup).
  const int64_t win_tiles = (w + kStreamTile - 1) / kStreamTile + 1;
  const int64_t bh = (int64_t)B * H;
  // At least about one workgroup per compute unit, and segments of at most
  // kSegRows keys, so that the longest sequence of a ragged batch does not set
  // a long critical path (segments past a shorter sequence end at once).
  const int64_t rows = nc + kStreamTile * win_tiles;
  int64_t per_bg = bh >= kStreamSlots / 2 ? 2 : kStreamSlots / bh;
  if (per_bg < (rows + kSegRows - 1) / kSegRows) per_bg = (rows + kSegRows - 1) / kSegRows;
  int64_t seg = up((rows + per_bg - 1) / per_bg);
  const int64_t seg_min = up((nc + kMaxChunks - 1) / kMaxChunks);
  const int64_t seg_max = (int64_t)(kScStrideMax - 4) * r / gran * gran;  // score slots per segment
  if (seg < seg_min) seg = seg_min;
  if (seg > seg_max) seg = seg_max;  // the host rejects seg_min > seg_max
  if (seg < gran) seg = gran;
  lay.seg = (int)seg;
  lay.nch = (int)((nc + seg - 1) / seg);
  if (lay.nch < 1) lay.nch = 1;
  lay.nbo = (int)(seg / r);
  int64_t wt = seg / kStreamTile;
  if (wt * kMaxWindow < win_tiles) wt = (win_tiles + kMaxWindow - 1) / kMaxWindow;
  lay.wtiles = (int)wt;
  lay.nwin = (int)((win_tiles + wt - 1) / wt);
  lay.scs = lay.nbo + 1;
  const size_t BH = (size_t)B * H;
  size_t nslots = BH * lay.nch;
  // A plan that needs more than one round of workgroups (a batch longer than
  // the compute units can stream at once) is balanced on the device instead:
  // the fixed plan cuts every sequence as if it had the longest length, so in a
  // ragged batch the long sequences' segments run a second round while the
  // short ones' slots sit empty.  Balanced segments of T tiles are cut from the
  // actual lengths so that all of them fill about one round.
  lay.bal = 0;
  if ((int64_t)BH * (lay.nch + lay.nwin) > kStreamSlots) {
    const int64_t tiles_max = (nc + kStreamTile - 1) / kStreamTile;
    const int64_t tcap = std::min<int64_t>(kBalTiles, (int64_t)(kScStrideMax - 4) * r / kStreamTile);
    const int64_t tmin = std::max<int64_t>(1, (tiles_max + kMaxChunks - 1) / kMaxChunks);
    if (tmin <= tcap) {  // the device falls back to the fixed plan when T would exceed tcap
      lay.bal = 1;
      lay.tcap = (int)tcap;
      lay.tmin = (int)tmin;
      lay.bal_fill = (int)std::max<int64_t>(kStreamSlots - (int64_t)BH * lay.nwin, (int64_t)BH);
      lay.nslot = lay.bal_fill + (int)BH;
      lay.scs = std::max(lay.scs, (int)(tcap * kStreamTile / r) + 1);
      nslots = std::max(nslots, (size_t)lay.nslot);
    }
  }
  size_t off = 0;
  lay.off_m1 = off;   off = align256(off + nslots * 16 * 4);
  lay.off_l1 = off;   off = align256(off + nslots * 16 * 4);
  lay.off_o1 = off;   off = align256(off + nslots * 16 * (size_t)DV * 4);
  lay.off_sc1 = off;  off = align256(off + nslots * 16 * (size_t)lay.scs * 4);
  lay.off_wpart = off; off = align256(off + BH * lay.nwin * (32 + 16 * (size_t)DV) * 4);
  // finish workgroups (finw waves, one 32-token step each): one partial each
  // (m, l and the output divided by l); the normalised compressed-branch output;
  // the arrival counters.  Four waves, or eight when 4-wave workgroups would be
  // more than one per compute unit (each of them reads all the group scores).
  const int spb = lsel >= 32 ? lsel / 32 : 1;
  lay.finw = (int64_t)BH * ((n * spb + 3) / 4) > kStreamSlots ? 8 : 4;
  lay.nfin = (n * spb + lay.finw - 1) / lay.finw;
  lay.off_rpart = off; off = align256(off + BH * lay.nfin * (32 + 8 * (size_t)DV) * 4);
  lay.off_ocmp = off; off = align256(off + BH * 16 * (size_t)DV * 4);
  lay.off_cnt = off; off = align256(off + BH * 4);
  lay.total = off;
  return lay;
}

template <int DK, int DV, int NWV>
static hipError_t launch_finish(const DecodeParams& p, hipStream_t s, hipEvent_t e2, hipEvent_t e3) {
  const dim3 g2((unsigned)(p.B * p.H * p.nfin)), blk(64 * NWV);
  switch (p.lsel) {
    case 16: hipExtLaunchKernelGGL((decode_finish_kernel<DK, DV, 16, NWV>), g2, blk, 0, s, e2, e3, 0, p); break;
    case 32: hipExtLaunchKernelGGL((decode_finish_kernel<DK, DV, 32, NWV>), g2, blk, 0, s, e2, e3, 0, p); break;
    case 64: hipExtLaunchKernelGGL((decode_finish_kernel<DK, DV, 64, NWV>), g2, blk, 0, s, e2, e3, 0, p); break;
    case 128: hipExtLaunchKernelGGL((decode_finish_kernel<DK, DV, 128, NWV>), g2, blk, 0, s, e2, e3, 0, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// With events, each kernel is launched with its start / stop events attached
// to the dispatch (ev[0], ev[1]: streaming kernel; ev[2], ev[3]: finish
// kernel), so their elapsed times are the kernels' own execution times.
template <int DK, int DV>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s, const PhaseEvents* ev) {
  hipEvent_t e0 = ev ? ev->ev[0] : nullptr, e1 = ev ? ev->ev[1] : nullptr;
  hipEvent_t e2 = ev ? ev->ev[2] : nullptr, e3 = ev ? ev->ev[3] : nullptr;
  const unsigned g1 = (unsigned)std::max(p.B * p.H * (p.nch + p.nwin), p.bal ? p.B * p.H * p.nwin + p.nslot : 0);
  hipExtLaunchKernelGGL((decode_stream_kernel<DK, DV>), dim3(g1), dim3(64 * kStreamWaves), 0, s, e0, e1, 0, p);
  hipError_t e;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.finw == 8) return launch_finish<DK, DV, 8>(p, s, e2, e3);
  return launch_finish<DK, DV, 4>(p, s, e2, e3);
}

hipError_t launch_decode(const DecodeParams& p, int DK, int DV, hipStream_t s, const PhaseEvents* ev) {
  if (DK == 192 && DV == 128) return launch_decode_t<192, 128>(p, s, ev);
  if (DK == 128 && DV == 128) return launch_decode_t<128, 128>(p, s, ev);
  if (DK == 64 && DV == 64) return launch_decode_t<64, 64>(p, s, ev);
  return hipErrorInvalidValue;
}

}  // namespace nsa

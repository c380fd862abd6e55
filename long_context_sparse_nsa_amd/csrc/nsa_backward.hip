// NSA backward of the causal prefill: gradients of the three-branch output with
// respect to the queries, the raw keys and values, the compressed cache and the
// gates, for training.
//
// Sources: "Native Sparse Attention (DeepSeek NSA)" lesson (AI Engineering from
// Scratch, phase 10 · 17), the section on native trainability: the top-n choice
// only decides which blocks are read and is not part of the differentiated graph;
// the gradient reaches the compressed cache through the compressed branch and the
// raw keys and values through the selected and window branches.  Lesson 5.5/02
// "Разреженное внимание — NSA и DSA", section "NSA: три ветви": out = sum_c g_c o_c.
//
// Per branch c with o_c = softmax(s q K_c^T) V_c, output gradient dO and gate g_c:
//   dg_c = dO . o_c,   D_c = g_c (dO . o_c),
//   P = exp(s q.k - lse_c),   dS = P (g_c dO.v - D_c),
//   dq = s sum_c sum_k dS k,   dk = s sum_q dS q,   dv = sum_q g_c P dO.
//
// Kernels (launch order):
//   bwd_bitmap_kernel   inverts the selection: bit t of row (b, g, block j) is set
//                       when position t selected block j.
//   bwd_query_kernel    one wave per (b, t, g): recomputes every branch's softmax
//                       (lse, D, dg) and then accumulates dq over all branches.
//   bwd_kv_kernel<WIN>  one wave per 16 raw keys: the window queries; stores dk, dv.
//   bwd_kv_kernel<SLC>  one wave per 16 raw keys and a range of positions: the
//                       queries that selected the keys' block; adds into dk, dv.
//   bwd_kv_kernel<CMP>  one wave per 16 compressed keys and a range of positions:
//                       adds into dk_cmp, dv_cmp.
// Products are bf16 MFMA (P and dS rounded to bf16 as operands) with fp32 sums.
#include <algorithm>

#include "nsa_train.hpp"
#include "nsa_tiles.hpp"

namespace nsa {
namespace {

constexpr int kCmp = 0, kSlc = 1, kWin = 2;  // branch ids (gate and lse slot order)
constexpr int kBwdWaves = 4;                 // waves per workgroup
constexpr float kNegInf = -__builtin_inff();

// Row pieces for a product whose contraction runs over 8 rows: lane lr holds the
// D/16 contiguous channels starting at (D/16)*lr of row `row` (zeros if !ok).
template <int D>
__device__ __forceinline__ void load_piece(const uint16_t* row, bool ok, int lr, uint32_t (&w)[D / 32]) {
  static_assert(D == 64 || D == 128 || D == 192, "row width");
  if (!ok) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) w[i] = 0u;
    return;
  }
  const uint16_t* p = row + (D / 16) * lr;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {  // 8-byte loads: (D/16)*lr elements is 8-byte aligned for every D here
    const u32x2_t x = ld8(p + 4 * i);
    w[2 * i] = x[0];
    w[2 * i + 1] = x[1];
  }
}

__device__ __forceinline__ int n_visible(int t, int l, int d, int nc) {
  return t >= l - 1 ? min(nc, (t - l + 1) / d + 1) : 0;
}

// ---------------------------------------------------------------------------
// Query side.

// One key range [s0, s1) of a branch, forward recompute: online softmax state
// (m in log2 units, l) and O^T accumulators (layout of pv_step).
template <int DK, int DV>
__device__ __forceinline__ void fwd_range(const uint16_t* kb, const uint16_t* vb, int s0, int s1,
                                          const u32x4_t (&qf)[DK / 32], float sl2, int lg, int lr, float& m,
                                          float& l, f32x4_t (&acc)[DV / 16]) {
  for (int k0 = s0; k0 < s1; k0 += 32) {
    u32x4_t kf0[DK / 32], kf1[DK / 32];
    load_k_tile<DK>(kb, k0 + lr, s1, lg, kf0);
    load_k_tile<DK>(kb, k0 + 16 + lr, s1, lg, kf1);
    uint32_t vr[8][DV / 32];
    load_v_step<DV>(vb, k0, s1, lg, lr, vr);
    const f32x4_t a = qk_tile<DK>(kf0, qf), c = qk_tile<DK>(kf1, qf);
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = (k0 + 4 * lg + i < s1) ? a[i] * sl2 : kNegInf;
      z[4 + i] = (k0 + 16 + 4 * lg + i < s1) ? c[i] * sl2 : kNegInf;
    }
    float mx = z[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmaxf(mx, z[r]);
    mx = max_over_groups(mx);
    const float mn = fmaxf(m, mx);  // finite: key k0 < s1 is always valid
    const float al = __builtin_amdgcn_exp2f(m - mn);
    float pr[8], ps = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      pr[r] = __builtin_amdgcn_exp2f(z[r] - mn);
      ps += pr[r];
    }
    ps = sum_over_groups(ps);
    l = l * al + ps;
    m = mn;
#pragma unroll
    for (int j = 0; j < DV / 16; ++j) acc[j] *= al;
    const float lo[4] = {pr[0], pr[1], pr[2], pr[3]}, hi[4] = {pr[4], pr[5], pr[6], pr[7]};
    pv_step<DV>(vr, pack_probs(lo, hi), acc);
  }
}

// One key range of a branch, gradient pass: dq^T += K^T dS^T.
template <int DK, int DV>
__device__ __forceinline__ void dq_range(const uint16_t* kb, const uint16_t* vb, int s0, int s1,
                                         const u32x4_t (&qf)[DK / 32], const u32x4_t (&of)[DV / 32], float sl2,
                                         float lse2, float gate, float dc, int lg, int lr, f32x4_t (&dqa)[DK / 16]) {
  for (int k0 = s0; k0 < s1; k0 += 32) {
    u32x4_t kf0[DK / 32], kf1[DK / 32], vf0[DV / 32], vf1[DV / 32];
    load_k_tile<DK>(kb, k0 + lr, s1, lg, kf0);
    load_k_tile<DK>(kb, k0 + 16 + lr, s1, lg, kf1);
    load_k_tile<DV>(vb, k0 + lr, s1, lg, vf0);
    load_k_tile<DV>(vb, k0 + 16 + lr, s1, lg, vf1);
    uint32_t kr[8][DK / 32];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int key = k0 + step_key(lg, r);
      load_piece<DK>(kb + (int64_t)key * DK, key < s1, lr, kr[r]);
    }
    const f32x4_t a = qk_tile<DK>(kf0, qf), c = qk_tile<DK>(kf1, qf);
    const f32x4_t pa = qk_tile<DV>(vf0, of), pc = qk_tile<DV>(vf1, of);
    float lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = (k0 + 4 * lg + i < s1) ? __builtin_amdgcn_exp2f(a[i] * sl2 - lse2) : 0.f;
      const float p1 = (k0 + 16 + 4 * lg + i < s1) ? __builtin_amdgcn_exp2f(c[i] * sl2 - lse2) : 0.f;
      lo[i] = p0 * (gate * pa[i] - dc);
      hi[i] = p1 * (gate * pc[i] - dc);
    }
    pv_step<DK>(kr, pack_probs(lo, hi), dqa);
  }
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void bwd_query_kernel(BwdParams p) {
  const int lane = threadIdx.x & 63, lg = lane >> 4, lr = lane & 15;
  const int wave = threadIdx.x >> 6;
  // Consecutive workgroups cycle through the (b, g) pairs; latest positions first.
  const int nbg = p.B * p.H;
  const int bid = (int)blockIdx.x;
  const int tile = p.nqt - 1 - bid / nbg;
  const int bg = bid - (bid / nbg) * nbg;
  const int b = bg / p.H, g = bg - (bg / p.H) * p.H;
  const int t = tile * kBwdWaves + wave;
  if (t >= p.T) return;
  const int T = p.T, G = p.G, Hq = p.Hq;
  const int64_t bgl = (int64_t)b * p.H + g;
  const uint16_t* kraw = p.k + bgl * T * DK;
  const uint16_t* vraw = p.v + bgl * T * DV;
  const uint16_t* kcmp = p.kc + bgl * p.nc * DK;
  const uint16_t* vcmp = p.vc + bgl * p.nc * DV;
  const int64_t qrow = ((int64_t)b * T + t) * Hq + (int64_t)g * G;  // the group's first head
  const bool hv = lr < G;

  u32x4_t qf[DK / 32], of[DV / 32];
  load_q_frags<DK>(p.q + qrow * DK, G, lg, lr, qf);
  load_q_frags<DV>(p.dout + qrow * DV, G, lg, lr, of);
  float gt[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) gt[c] = hv ? p.gates[(qrow + lr) * 3 + c] : 0.f;
  // dO channels of this lane in the O^T accumulator layout: (DV/16)*(4lg+i) + j.
  float dov[4][DV / 16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w[DV / 32];
    const uint16_t* src = p.dout + (qrow + lr) * DV + (DV / 16) * (4 * lg + i);
#pragma unroll
    for (int u = 0; u < DV / 64; ++u) {
      const u32x2_t x = hv ? ld8(src + 4 * u) : u32x2_t{0u, 0u};
      w[2 * u] = x[0];
      w[2 * u + 1] = x[1];
    }
#pragma unroll
    for (int u = 0; u < DV / 32; ++u) {
      dov[i][2 * u] = bf16_lo(w[u]);
      dov[i][2 * u + 1] = bf16_hi(w[u]);
    }
  }

  const int nvis = n_visible(t, p.l, p.d, p.nc);
  const int32_t* selrow = p.sel + (((int64_t)b * T + t) * p.H + g) * p.n;
  const int wlo = max(0, t - p.w + 1);
  const float sl2 = p.scale_log2;

  // Pass 1: per-branch softmax statistics and outputs.
  float lse2[3], dcs[3];
#pragma unroll 1
  for (int c = 0; c < 3; ++c) {
    float m = kNegInf, l = 0.f;
    f32x4_t acc[DV / 16];
#pragma unroll
    for (int j = 0; j < DV / 16; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (c == kCmp) {
      if (nvis > 0) fwd_range<DK, DV>(kcmp, vcmp, 0, nvis, qf, sl2, lg, lr, m, l, acc);
    } else if (c == kWin) {
      fwd_range<DK, DV>(kraw, vraw, wlo, t + 1, qf, sl2, lg, lr, m, l, acc);
    } else {
      for (int s = 0; s < p.n; ++s) {
        const int j = selrow[s];
        if (j < 0) break;
        const int s0 = j * p.lsel, s1 = min(s0 + p.lsel, t + 1);
        if (s0 < s1) fwd_range<DK, DV>(kraw, vraw, s0, s1, qf, sl2, lg, lr, m, l, acc);
      }
    }
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < DV / 16; ++j) dot = fmaf(acc[j][i], dov[i][j], dot);
    dot = sum_over_groups(dot);
    const bool any = l > 0.f;
    dot = any ? dot / l : 0.f;  // dO . o_c
    lse2[c] = any ? m + __log2f(l) : 0.f;
    dcs[c] = gt[c] * dot;
    if (lg == 0) {  // statistics record of (c, b, t, g): lse[16] | D[16] | gate[16], zeros past G
      float* rec = p.stat + ((((int64_t)c * p.B + b) * T + t) * p.H + g) * kStatFloats;
      rec[lr] = hv ? lse2[c] : 0.f;
      rec[16 + lr] = hv ? dcs[c] : 0.f;
      rec[32 + lr] = gt[c];
      if (hv) p.dgates[(qrow + lr) * 3 + c] = dot;
    }
  }

  // Pass 2: dq over the same key ranges.
  f32x4_t dqa[DK / 16];
#pragma unroll
  for (int j = 0; j < DK / 16; ++j) dqa[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (nvis > 0) dq_range<DK, DV>(kcmp, vcmp, 0, nvis, qf, of, sl2, lse2[kCmp], gt[kCmp], dcs[kCmp], lg, lr, dqa);
  dq_range<DK, DV>(kraw, vraw, wlo, t + 1, qf, of, sl2, lse2[kWin], gt[kWin], dcs[kWin], lg, lr, dqa);
  for (int s = 0; s < p.n; ++s) {
    const int j = selrow[s];
    if (j < 0) break;
    const int s0 = j * p.lsel, s1 = min(s0 + p.lsel, t + 1);
    if (s0 < s1) dq_range<DK, DV>(kraw, vraw, s0, s1, qf, of, sl2, lse2[kSlc], gt[kSlc], dcs[kSlc], lg, lr, dqa);
  }
  if (hv) {
    float* dst = p.dq + (qrow + lr) * DK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j4 = 0; j4 < DK / 64; ++j4) {
        const int j = 4 * j4;
        *reinterpret_cast<f32x4_t*>(dst + (DK / 16) * (4 * lg + i) + j) =
            f32x4_t{dqa[j][i], dqa[j + 1][i], dqa[j + 2][i], dqa[j + 3][i]} * p.scale;
      }
  }
}

// ---------------------------------------------------------------------------
// Key side.  A workgroup owns 64 keys, a wave 16 of them (the MFMA columns,
// K and V fragments held in registers).  The queries that see those keys are
// taken two at a time: the 32 rows (query, head) of a pair form the contraction
// of dV^T += dout^T (g P) and dK^T += Q^T dS.  Each pair's Q rows, dout rows and
// statistics records are copied global -> LDS directly by all four waves,
// kKvBuf buffers deep; within a row the 16-byte chunks are XOR-swizzled with the
// row index so that the MFMA operand reads (16 rows at one column) spread over
// the LDS banks.

constexpr int kKvBuf = 3;

template <int DK, int DV>
struct KvShape {
  static constexpr int kQ = 32 * DK;  // bf16 elements of a pair's Q rows
  static constexpr int kO = 32 * DV;
  static constexpr int kBuf = 2 * kQ + 2 * kO + 2 * kStatFloats * 4;  // bytes per buffer
  static constexpr int kCpQ = 32 * DK / 8 / 256;                       // copies per wave
  static constexpr int kCpO = 32 * DV / 8 / 256;
  static constexpr int kCopies = kCpQ + kCpO + 1;
  static_assert(32 * DK % 2048 == 0 && 32 * DV % 2048 == 0, "whole copy instructions per wave");
};

// Byte offset in LDS of channel e (a multiple of 4) of row r of a block of D-wide rows.
template <int D>
__device__ __forceinline__ int sw_off(int r, int e) {
  return r * D * 2 + ((((e >> 3) ^ (r & 7))) << 4) + ((e & 7) << 1);
}

template <int D>
__device__ __forceinline__ u32x4_t lds_frag(const char* blk, int r, int e) {  // 8 channels, e % 8 == 0
  return *reinterpret_cast<const u32x4_t*>(blk + sw_off<D>(r, e));
}

template <int D>
__device__ __forceinline__ void lds_piece(const char* blk, int r, int lr, uint32_t (&w)[D / 32]) {
#pragma unroll
  for (int u = 0; u < D / 64; ++u) {
    const u32x2_t x = *reinterpret_cast<const u32x2_t*>(blk + sw_off<D>(r, (D / 16) * lr + 4 * u));
    w[2 * u] = x[0];
    w[2 * u + 1] = x[1];
  }
}

template <int DK, int DV, int MODE>
__global__ __launch_bounds__(256) void bwd_kv_kernel(BwdParams p) {
  using SH = KvShape<DK, DV>;
  __shared__ __attribute__((aligned(1024))) char s_buf[kKvBuf][SH::kBuf];
  __shared__ int32_t s_list[MODE == kSlc ? 32 * kBwdQWordsMax : 1];
  __shared__ int s_scan[4];

  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nbg = p.B * p.H;
  const int bid = (int)blockIdx.x;
  const int kt = bid / nbg;
  const int bg = bid - kt * nbg;
  const int b = bg / p.H, g = bg - (bg / p.H) * p.H;
  const int kw0 = kt * 64;  // the workgroup's first key
  const int nkeys = MODE == kCmp ? p.nc : p.T;
  if (kw0 >= nkeys) return;
  const int T = p.T, G = p.G, Hq = p.Hq;
  const int k0 = kw0 + 16 * wave;
  const int key = k0 + lr;
  const int64_t bgl = (int64_t)b * p.H + g;

  // Positions visited by the workgroup.
  int tlo, npos;
  if constexpr (MODE == kWin) {
    tlo = kw0;
    npos = min(T - 1, kw0 + 63 + p.w - 1) - tlo + 1;
  } else if constexpr (MODE == kCmp) {
    tlo = kw0 * p.d + p.l - 1 + (int)blockIdx.y * p.qchunk;
    npos = min(T - 1, tlo + p.qchunk - 1) - tlo + 1;
    if (npos <= 0) return;
  } else {
    // The positions that chose one of the workgroup's blocks, from the bitmap
    // rows, in order; bit 24 + w of an entry: wave w's block was chosen.
    const int jw[4] = {kw0 / p.lsel, (kw0 + 16) / p.lsel, (kw0 + 32) / p.lsel, (kw0 + 48) / p.lsel};
    const int first = (kw0 / p.lsel) * p.lsel;  // no earlier position can choose these blocks
    const int wlo = max(first >> 5, (int)blockIdx.y * p.qwords);
    const int whi = min(p.nwords, ((int)blockIdx.y + 1) * p.qwords);
    if (wlo >= whi) return;
    const uint32_t* rows = p.bits + bgl * p.nblk * p.nwords;
    const int wi = wlo + tid;
    uint32_t m[4] = {0u, 0u, 0u, 0u};
    if (tid < p.qwords && wi < whi) {
#pragma unroll
      for (int w = 0; w < 4; ++w) m[w] = jw[w] < p.nblk ? rows[(int64_t)jw[w] * p.nwords + wi] : 0u;
    }
    const uint32_t any = m[0] | m[1] | m[2] | m[3];
    int tot;
    int off = block_scan<256>(__builtin_popcount(any), s_scan, &tot);
    uint32_t x = any;
    while (x) {
      const int bit = __builtin_ctz(x);
      x &= x - 1;
      int mask = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) mask |= (int)((m[w] >> bit) & 1u) << w;
      s_list[off++] = (32 * wi + bit) | (mask << 24);
    }
    __syncthreads();
    tlo = 0;
    npos = tot;
    if (npos == 0) return;
  }
  const int npair = (npos + 1) / 2;

  // Position of entry i and the waves it concerns (all for window / compressed).
  auto entry = [&](int i, int& t, int& mask) {
    if (i >= npos) { t = -1; mask = 0; return; }
    if constexpr (MODE == kSlc) {
      const int e = s_list[i];
      t = e & 0xFFFFFF;
      mask = e >> 24;
    } else {
      t = tlo + i;
      mask = 0xF;
    }
  };

  // Copies of pair i into buffer i % kKvBuf (the same number of instructions in every wave).
  auto issue = [&](int i) {
    int tA, mA, tB, mB;
    entry(2 * i, tA, mA);
    entry(2 * i + 1, tB, mB);
    if (tB < 0) tB = tA;  // a duplicate, masked out in the compute
    char* buf = s_buf[i % kKvBuf];
#pragma unroll
    for (int j = 0; j < SH::kCpQ; ++j) {
      const int pch = (wave * SH::kCpQ + j) * 64 + lane;  // LDS chunk: row r, slot s
      const int r = pch / (DK / 8), sl = pch - r * (DK / 8);
      const int c = sl ^ (r & 7);
      const int tt = r < 16 ? tA : tB, h = min(r & 15, G - 1);
      const uint16_t* src = p.q + (((int64_t)b * T + tt) * Hq + (int64_t)g * G + h) * DK + 8 * c;
      copy16_to_lds(src, buf + (wave * SH::kCpQ + j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < SH::kCpO; ++j) {
      const int pch = (wave * SH::kCpO + j) * 64 + lane;
      const int r = pch / (DV / 8), sl = pch - r * (DV / 8);
      const int c = sl ^ (r & 7);
      const int tt = r < 16 ? tA : tB, h = min(r & 15, G - 1);
      const uint16_t* src = p.dout + (((int64_t)b * T + tt) * Hq + (int64_t)g * G + h) * DV + 8 * c;
      copy16_to_lds(src, buf + 2 * SH::kQ + (wave * SH::kCpO + j) * 1024);
    }
    // statistics: 2 records x 12 chunks, 6 lanes per wave
    if (lane < 6) {
      const int ch = wave * 6 + lane, x = ch / 12, cc = ch - x * 12;
      const int tt = x == 0 ? tA : tB;
      const float* src = p.stat + ((((int64_t)MODE * p.B + b) * T + tt) * p.H + g) * kStatFloats + 4 * cc;
      copy16_to_lds(src, buf + 2 * SH::kQ + 2 * SH::kO + wave * 96);
    }
  };

  u32x4_t kf[DK / 32], vf[DV / 32];
  const uint16_t* kb = MODE == kCmp ? p.kc + bgl * p.nc * DK : p.k + bgl * T * DK;
  const uint16_t* vb = MODE == kCmp ? p.vc + bgl * p.nc * DV : p.v + bgl * T * DV;
  load_k_tile<DK>(kb, key, nkeys, lg, kf);
  load_k_tile<DV>(vb, key, nkeys, lg, vf);
  f32x4_t dka[DK / 16], dva[DV / 16];
#pragma unroll
  for (int j = 0; j < DK / 16; ++j) dka[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < DV / 16; ++j) dva[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  wait_vmem();

  auto visible = [&](int t) {
    if (key >= nkeys) return false;
    if constexpr (MODE == kWin) return key <= t && key > t - p.w;
    if constexpr (MODE == kSlc) return key <= t;
    return key * p.d + p.l - 1 <= t;
  };

  issue(0);
  if (npair > 1) issue(1);
  for (int i = 0; i < npair; ++i) {
    if (i + 1 < npair) wait_vmem_le<SH::kCopies>(); else wait_vmem();
    lds_barrier();
    if (i + 2 < npair) issue(i + 2);
    const char* buf = s_buf[i % kKvBuf];
    const char* bq = buf;
    const char* bo = buf + 2 * SH::kQ;
    const float* bs = reinterpret_cast<const float*>(buf + 2 * SH::kQ + 2 * SH::kO);
    float pg[2][4], ds[2][4];
#pragma unroll
    for (int X = 0; X < 2; ++X) {
      int t, mask;
      entry(2 * i + X, t, mask);
      const int r = 16 * X + lr;
      u32x4_t qa[DK / 32], oa[DV / 32];
#pragma unroll
      for (int kk = 0; kk < DK / 32; ++kk) qa[kk] = lds_frag<DK>(bq, r, 8 * lg + 32 * kk);
#pragma unroll
      for (int kk = 0; kk < DV / 32; ++kk) oa[kk] = lds_frag<DV>(bo, r, 8 * lg + 32 * kk);
      const f32x4_t s = qk_tile<DK>(qa, kf);   // S[head 4lg+i][key lr]
      const f32x4_t dp = qk_tile<DV>(oa, vf);  // dout . v
      const f32x4_t lse = *reinterpret_cast<const f32x4_t*>(bs + X * kStatFloats + 4 * lg);
      const f32x4_t dc = *reinterpret_cast<const f32x4_t*>(bs + X * kStatFloats + 16 + 4 * lg);
      const f32x4_t gt = *reinterpret_cast<const f32x4_t*>(bs + X * kStatFloats + 32 + 4 * lg);
      const bool vis = t >= 0 && ((mask >> wave) & 1) && visible(t);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = vis && 4 * lg + e < G;
        const float pr = ok ? __builtin_amdgcn_exp2f(s[e] * p.scale_log2 - lse[e]) : 0.f;
        pg[X][e] = pr * gt[e];
        ds[X][e] = pr * (gt[e] * dp[e] - dc[e]);
      }
    }
    uint32_t orow[8][DV / 32];
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) lds_piece<DV>(bo, (r8 < 4 ? 0 : 16) + 4 * lg + (r8 & 3), lr, orow[r8]);
    pv_step<DV>(orow, pack_probs(pg[0], pg[1]), dva);
    uint32_t qrow[8][DK / 32];
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) lds_piece<DK>(bq, (r8 < 4 ? 0 : 16) + 4 * lg + (r8 & 3), lr, qrow[r8]);
    pv_step<DK>(qrow, pack_probs(ds[0], ds[1]), dka);
  }

  if (key >= nkeys) return;
  float* dk = (MODE == kCmp ? p.dkc + bgl * p.nc * DK : p.dk + bgl * T * DK) + (int64_t)key * DK;
  float* dv = (MODE == kCmp ? p.dvc + bgl * p.nc * DV : p.dv + bgl * T * DV) + (int64_t)key * DV;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < DK / 16; ++j) {
      const float x = dka[j][i] * p.scale;
      float* a = dk + (DK / 16) * (4 * lg + i) + j;
      if constexpr (MODE == kWin) *a = x; else unsafeAtomicAdd(a, x);
    }
#pragma unroll
    for (int j = 0; j < DV / 16; ++j) {
      const float x = dva[j][i];
      float* a = dv + (DV / 16) * (4 * lg + i) + j;
      if constexpr (MODE == kWin) *a = x; else unsafeAtomicAdd(a, x);
    }
  }
}

__global__ __launch_bounds__(256) void bwd_bitmap_kernel(BwdParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.T * p.H * p.n;
  if (i >= total) return;
  const int j = p.sel[i];
  if (j < 0 || j >= p.nblk) return;
  int64_t r = i / p.n;
  const int g = (int)(r % p.H);
  r /= p.H;
  const int t = (int)(r % p.T);
  const int b = (int)(r / p.T);
  atomicOr(p.bits + (((int64_t)b * p.H + g) * p.nblk + j) * p.nwords + (t >> 5), 1u << (t & 31));
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(uint32_t* a, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) a[i] = 0u;
}

hipError_t zero_words(void* a, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint32_t*>(a), n);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s, const PhaseEvents* ev) {
  const int nbg = p.B * p.H;
  hipError_t e;
  if ((e = zero_words(p.bits, (int64_t)nbg * p.nblk * p.nwords, s)) != hipSuccess) return e;
  if ((e = zero_words(p.dkc, (int64_t)nbg * p.nc * DK, s)) != hipSuccess) return e;
  if ((e = zero_words(p.dvc, (int64_t)nbg * p.nc * DV, s)) != hipSuccess) return e;
  const int64_t nsel = (int64_t)p.B * p.T * p.H * p.n;
  hipLaunchKernelGGL(bwd_bitmap_kernel, dim3((unsigned)((nsel + 255) / 256)), dim3(256), 0, s, p);
  if (ev) hipEventRecord(ev->ev[0], s);
  hipLaunchKernelGGL((bwd_query_kernel<DK, DV>), dim3((unsigned)(nbg * p.nqt)), dim3(256), 0, s, p);
  if (ev) hipEventRecord(ev->ev[1], s);
  const int kraw = (p.T + 63) / 64, kcmp = (p.nc + 63) / 64;
  hipLaunchKernelGGL((bwd_kv_kernel<DK, DV, kWin>), dim3((unsigned)(nbg * kraw)), dim3(256), 0, s, p);
  hipLaunchKernelGGL((bwd_kv_kernel<DK, DV, kSlc>), dim3((unsigned)(nbg * kraw), (unsigned)p.nqw), dim3(256), 0, s,
                     p);
  if (ev) hipEventRecord(ev->ev[2], s);
  if (p.nc > 0)
    hipLaunchKernelGGL((bwd_kv_kernel<DK, DV, kCmp>), dim3((unsigned)(nbg * kcmp), (unsigned)p.ncq), dim3(256), 0,
                       s, p);
  if (ev) hipEventRecord(ev->ev[3], s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bwd(const BwdParams& p, int DK, int DV, hipStream_t s, const PhaseEvents* ev) {
  if (DK == 192 && DV == 128) return launch_bwd_t<192, 128>(p, s, ev);
  if (DK == 128 && DV == 128) return launch_bwd_t<128, 128>(p, s, ev);
  if (DK == 64 && DV == 64) return launch_bwd_t<64, 64>(p, s, ev);
  return hipErrorInvalidValue;
}

}  // namespace nsa

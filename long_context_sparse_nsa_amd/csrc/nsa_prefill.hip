// NSA causal prefill on gfx950, tiled over query positions.
//
// Kernel 1 runs one workgroup (8 waves, two per SIMD) per (sequence, KV group,
// tile of 16 consecutive positions t0 .. t0+15), kernel 2 one workgroup of 4
// waves per 8 positions.  Wave w owns two consecutive positions and keeps, for
// each, the group's query fragments and a 16-head x d_v fp32 accumulator in
// registers.  Key/value rows are copied straight from global memory into LDS
// (no register round trip), several steps ahead, and each staged tile serves
// every position of the workgroup that needs it.
//
// Kernel 1 (compressed + window branches, group scores, selection):
//   W   sliding window (t - w, t] over the raw keys, online softmax; the
//       accumulator is then scaled to g_win * o_win;
//   C1  compressed keys visible at t: logits only, exact per-head max and sum;
//   C2  the same keys again: normalised probabilities p, accumulator += g_cmp *
//       p . Vc, and p folded onto selection blocks by token overlap (an MFMA
//       with the overlap counts) and summed over the group's heads into the
//       position's score row in LDS;
//   top-n per position (initial and local blocks forced) -> selected ids;
//   the accumulator (g_win o_win + g_cmp o_cmp, fp32) goes to the workspace.
// Kernel 2 (selected branch): the union of the 8 positions' selected blocks is
// staged 32 rows at a time; each wave runs the online softmax for those of its
// positions that chose the block, then writes bf16(acc + g_slc o_slc).
//
// Sources: lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc),
// section "NSA: три ветви" (output equation, the three branches, blockwise
// selection shared by the GQA group); lesson "Native Sparse Attention (DeepSeek
// NSA)" (AI Engineering from Scratch, phase 10 · 17), "Build it" steps 2-5.
#include <hip/hip_runtime.h>

#include "nsa_device.hpp"
#include "nsa_internal.hpp"
#include "nsa_stage.hpp"
#include "nsa_tiles.hpp"
#include "nsa_topn.hpp"

namespace nsa {

namespace {

constexpr int kTileQ = 16;               // positions per workgroup
constexpr int kWaves = 8;                // waves per workgroup (two per SIMD)
constexpr int kWaveQ = kTileQ / kWaves;  // positions per wave
constexpr int kThreads = 64 * kWaves;
constexpr float kNegBig = -1e30f;        // running-reference start: finite, so exp2 never sees inf - inf
constexpr float kLazy = 8.0f;            // the softmax reference moves only when exceeded by this (log2 units)
constexpr float kLn2 = 0.6931471805599453f;  // log-sum-exp outputs: log2 units to natural log
constexpr int kReadAhead = 2;  // k-steps of K operand reads issued ahead of their MFMAs

template <int DK, int DV>
struct PfShape {
  static constexpr int KT = DK / 32;           // MFMA k-steps of a logit tile
  static constexpr int VC = DV / 16;           // MFMAs per 32-key value step
  static constexpr int kKBytes = 64 * DK * 2;  // 64-key K tile, MFMA fragment order
  static constexpr int kVBytes = 64 * DV * 2;  // 64-key V tile, row-major
  static constexpr int kBuf = kKBytes + kVBytes;
};

// A operand with row 0 all ones (bf16 1.0) and zeros elsewhere: MFMA'd with a
// P^T operand it adds, in row 0 (lane lr = head, element 0), the step's sum of
// the bf16 probabilities -- the softmax denominator of exactly the weights the
// value product used.
__device__ __forceinline__ u32x4_t ones_row_operand(int lr) {
  const uint32_t v = lr == 0 ? 0x3F803F80u : 0u;
  return u32x4_t{v, v, v, v};
}

// Online softmax with a lazily moved reference m (scaled log2 units): m only
// moves when the block maximum ms exceeds it by more than kLazy, so exp2(z - m)
// stays below 2^kLazy and the accumulators are rescaled rarely.  The final
// division by the sum taken against the same reference makes the result
// independent of m.  ms is equal on the 4 lanes of a head.
template <int VC>
__device__ __forceinline__ void lazy_rescale(float ms, float& m, f32x4_t (&acc)[VC], f32x4_t& lsum) {
  const bool move = ms > m + kLazy;
  if (__ballot(move) != 0ull) {  // wave-uniform
    const float mn = move ? ms : m;
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
    for (int j = 0; j < VC; ++j) acc[j] *= alpha;
    lsum *= alpha;
    m = mn;
  }
}

// The V rows of a step, staged row-major with the 16-byte pieces of row r
// XOR-permuted by f(r) (a permutation inside the row), and read back as V^T
// MFMA operands with the LDS transpose read: the 16 lanes of a lane group point
// at 4 rows x 16 channels (4 lanes per row, 4 channels each) and lane i receives
// channel i of the 4 rows.  f spreads the 32 lanes of each half-wave over all 16
// bank groups of 16 bytes.
template <int DV>
struct VSwizzle {
  static_assert(DV == 64 || DV == 128, "transposed V reads are laid out for d_v = 64 or 128");
  static constexpr int PR = DV / 8;  // 16-byte pieces per row
  __device__ static int f(int r) { return DV == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }
  // lane's byte offset of its piece in copy c's 1 KB (full tiles): depends on c
  // only through c mod 2, so one value serves all copies of a wave when NW is even
  __device__ static uint32_t copy_offset(int c, int lane) {
    const int r = (64 * c + lane) / PR;
    return 16u * (uint32_t)((lane - lane % PR) + ((lane % PR) ^ f(r)));
  }
};

template <int DV, int ROWS, int NW>
__device__ __forceinline__ void stage_v_swizzled(const uint16_t* base, int64_t row0, int64_t rowmax, uint32_t dst,
                                                 int wave, int lane, uint32_t voff) {
  using VS = VSwizzle<DV>;
  constexpr int NI = ROWS * VS::PR / 64, PW = (NI + NW - 1) / NW;
  static_assert(NW % 2 == 0, "one copy offset per wave");
  if (row0 + ROWS - 1 <= rowmax) {  // wave-uniform
    const char* tile = reinterpret_cast<const char*>(base + row0 * DV);
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int c = wave + NW * k;
      if (NI % NW != 0 && c >= NI) break;
      copy16_sb_at(tile + 1024 * c, voff, dst + 1024 * c);
    }
  } else {
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int c = wave + NW * k;
      if (NI % NW != 0 && c >= NI) break;
      const int sl = 64 * c + lane, r = sl / VS::PR;
      int64_t row = row0 + r;
      row = row < rowmax ? row : rowmax;
      copy16_to_lds_at(base + row * DV + 8 * ((sl % VS::PR) ^ VS::f(r)), dst + 1024 * c);
    }
  }
}

// This lane's part of the transposed-read addresses: row 4*lg + lr/4 of a
// 16-row half, 8 bytes at channel 4*(lr%4) of a 16-channel block, before the
// block index j is XOR-ed into bits 5.. (32*j).
template <int DV>
__device__ __forceinline__ uint32_t vt_lane_offset(int lg, int lr) {
  const int r = 4 * lg + lr / 4;
  return (uint32_t)(r * DV * 2 + 16 * (VSwizzle<DV>::f(r) + (lr % 4) / 2) + 8 * (lr % 2));
}

// V^T operand of channels 16j .. 16j+15 for the 32-key step at row 32*ks of the
// staged tile: element e of lane (lg, lr) is channel 16j + lr of key
// step_key(lg, e).
template <int DV>
__device__ __forceinline__ u32x4_t lds_vt_operand(const char* vt, int ks, int j, uint32_t vlane) {
  typedef short v4i16_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16_t* lds_v4_t;
  const char* pa = vt + 32 * ks * DV * 2 + (vlane ^ (32u * (uint32_t)j));
  const v4i16_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_t)(pa));
  const v4i16_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_t)(pa + 16 * DV * 2));
  const u32x2_t ua = __builtin_bit_cast(u32x2_t, a), ub = __builtin_bit_cast(u32x2_t, b);
  return u32x4_t{ua[0], ua[1], ub[0], ub[1]};
}

// acc[q] += V^T . P_q^T over the 32-key step `ks` of the staged V tile (rows
// swizzled as above), for the wave's positions; each V^T operand is read once
// and used for all of them.  acc[q][j] element i is channel 16j + 4*lg + i.
template <int DV, int NQ>
__device__ __forceinline__ void pv_half(const char* vt, int ks, uint32_t vlane, const u32x4_t (&pk)[NQ],
                                        f32x4_t (&acc)[NQ][DV / 16]) {
#pragma unroll
  for (int j = 0; j < DV / 16; ++j) {
    const u32x4_t va = lds_vt_operand<DV>(vt, ks, j, vlane);
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q][j] = mfma_bf16(va, pk[q], acc[q][j]);
  }
}

// The 8 logits of a 32-key half (keys x0 + step rows) with keys outside
// (lo, hi] replaced by -inf; the test is skipped when the whole half is inside.
__device__ __forceinline__ void mask_range(const f32x4_t (&sv)[2], int x0, int lo, int hi, int lg,
                                           float (&z)[2][4]) {
  if (x0 > lo && x0 + 31 <= hi) {  // wave-uniform
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int i = 0; i < 4; ++i) z[mm][i] = sv[mm][i];
  } else {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = x0 + 16 * mm + 4 * lg + i;
        z[mm][i] = (x > lo && x <= hi) ? sv[mm][i] : -INFINITY;
      }
  }
}

// exp2(z * sc + nm) of a half's 8 logits, packed as the P^T operand.
__device__ __forceinline__ u32x4_t exp_pack(const float (&z)[2][4], float sc, float nm) {
  float e[2][4];
#pragma unroll
  for (int mm = 0; mm < 2; ++mm)
#pragma unroll
    for (int i = 0; i < 4; ++i) e[mm][i] = __builtin_amdgcn_exp2f(fmaf(z[mm][i], sc, nm));
  return pack_probs(e[0], e[1]);
}

// lazy_rescale for several positions at once (one wave-uniform branch).
template <int VC, int NQ>
__device__ __forceinline__ void lazy_rescale_n(const float (&ms)[NQ], float (&m)[NQ], f32x4_t (&acc)[NQ][VC],
                                               f32x4_t (&lsum)[NQ]) {
  bool any = false;
#pragma unroll
  for (int q = 0; q < NQ; ++q) any = any || (ms[q] > m[q] + kLazy);
  if (__ballot(any) != 0ull) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const float mn = ms[q] > m[q] + kLazy ? ms[q] : m[q];
      const float alpha = __builtin_amdgcn_exp2f(m[q] - mn);
#pragma unroll
      for (int j = 0; j < VC; ++j) acc[q][j] *= alpha;
      lsum[q] *= alpha;
      m[q] = mn;
    }
  }
}

__device__ __forceinline__ int n_visible(int t, int l, int d) { return t + 1 >= l ? (t + 1 - l) / d + 1 : 0; }

__device__ __forceinline__ float max8(const float (&z)[2][4]) {
  return fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
               fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
}

// Workgroup -> (sequence b, group g, tile).  Tiles are issued latest first (they
// carry the most compressed keys); consecutive workgroup ids cycle through the
// (b, g) pairs, so with 4 groups each XCD keeps seeing one group's keys.
struct TileId {
  int b, g, t0;
};
__device__ __forceinline__ TileId tile_id(const PrefillParams& p) {
  const int nbg = p.B * p.H;
  const int bid = (int)blockIdx.x;
  const int tile = p.ntile - 1 - bid / nbg;
  const int bg = bid - (bid / nbg) * nbg;
  return TileId{bg / p.H, bg - (bg / p.H) * p.H, tile * kTileQ};
}

}  // namespace

// ---------------------------------------------------------------------------
// Kernel 1: window + compressed branches, group scores, top-n.
// NBUF key-tile buffers (NBUF - 1 tiles in flight); MAXB score slots per position.
template <int DK, int DV, int NBUF, int MAXB>
__global__ __launch_bounds__(kThreads, 1) void pf_cmp_win_kernel(PrefillParams p) {
  using SH = PfShape<DK, DV>;
  constexpr int KT = SH::KT, VC = SH::VC;
  using SO = StageOffsets<DK, DV, 64, kWaves>;
  constexpr int NLD_K = SO::kMinCopiesK, NLD_KV = SO::kMinCopiesKV;
  __shared__ __attribute__((aligned(1024))) char s_buf[NBUF][SH::kBuf];
  __shared__ float s_score[kTileQ][MAXB];
  __shared__ float s_gnet[kTileQ][2][16];  // gate network: (g_cmp, g_win) per position and head

  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const TileId ti = tile_id(p);
  const int b = ti.b, g = ti.g, t0 = ti.t0;
  const int T = p.T;
  const int tlast = min(t0 + kTileQ - 1, T - 1);
  const int64_t bg = (int64_t)b * p.H + g;
  const uint16_t* kraw = p.k + bg * T * DK;
  const uint16_t* vraw = p.v + bg * T * DV;
  const uint16_t* kcmp = p.kc + bg * p.nc * DK;
  const uint16_t* vcmp = p.vc + bg * p.nc * DV;

  // chunk plan: window rows, then the compressed rows twice
  const int xlo = max(0, t0 - p.w + 1);
  const int nW = (tlast - xlo + 1 + 63) / 64;
  const int ncT = n_visible(tlast, p.l, p.d);
  const int nC = (ncT + 63) / 64;
  const int nch = nW + 2 * nC;
  const int Jtile = tlast / p.lsel;

  for (int e = tid; e < kTileQ * (Jtile + 1); e += kThreads) s_score[e / (Jtile + 1)][e % (Jtile + 1)] = 0.f;

  const SO so(lane);
  const uint32_t vcopy = VSwizzle<DV>::copy_offset(wave, lane);
  const uint32_t vlane = vt_lane_offset<DV>(lg, lr);
  const uint32_t lds_buf0 = lds_addr_of(&s_buf[0][0]);
  auto stage = [&](int c, int buf) {
    const uint32_t kt = lds_buf0 + (uint32_t)(buf * SH::kBuf);
    const uint32_t vt = kt + SH::kKBytes;
    // rows past the tile's needs but inside the arrays are copied and masked
    if (c < nW) {
      const int64_t r0 = xlo + 64 * c;
      stage_k(kraw, r0, T - 1, kt, wave, lane, so);
      stage_v_swizzled<DV, 64, kWaves>(vraw, r0, T - 1, vt, wave, lane, vcopy);
    } else if (c < nW + nC) {
      stage_k(kcmp, 64 * (c - nW), p.nc - 1, kt, wave, lane, so);
    } else {
      const int64_t r0 = 64 * (c - nW - nC);
      stage_k(kcmp, r0, p.nc - 1, kt, wave, lane, so);
      stage_v_swizzled<DV, 64, kWaves>(vcmp, r0, p.nc - 1, vt, wave, lane, vcopy);
    }
  };

  // per-position state (positions t0 + kWaveQ*wave + q; the scalars are wave-uniform)
  int tq[kWaveQ], nvq[kWaveQ];
  bool act[kWaveQ];
  u32x4_t qf[kWaveQ][KT];
  f32x4_t acc[kWaveQ][VC];
  f32x4_t lsum[kWaveQ];
  float mref[kWaveQ];
#pragma unroll
  for (int q = 0; q < kWaveQ; ++q) {
    tq[q] = t0 + kWaveQ * wave + q;
    act[q] = tq[q] < T;
    nvq[q] = act[q] ? n_visible(tq[q], p.l, p.d) : 0;
    const int tt = act[q] ? tq[q] : T - 1;
    load_q_frags<DK>(p.q + (((int64_t)b * T + tt) * p.Hq + (int64_t)g * p.G) * DK, p.G, lg, lr, qf[q]);
#pragma unroll
    for (int j = 0; j < VC; ++j) acc[q][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lsum[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    mref[q] = kNegBig;
  }
  // gate network (when given): this lane's head lr, both positions, branches cmp
  // and win, computed before the pipeline starts and kept in LDS (this wave's rows)
  if (p.wgate) {
    const int hq = g * p.G + (lr < p.G ? lr : 0);
#pragma unroll
    for (int q = 0; q < kWaveQ; ++q) {
      const int tt = act[q] ? tq[q] : T - 1;
      const uint16_t* qrow = p.q + (((int64_t)b * T + tt) * p.Hq + hq) * DK;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int br = 2 * c;
        const float z = sum_over_groups_swap(gate_dot_quarter<DK>(qrow, p.wgate + ((size_t)hq * 3 + br) * DK, lg));
        if (lg == 0) s_gnet[kWaveQ * wave + q][c][lr] = gate_sigmoid(z + (p.bgate ? p.bgate[hq * 3 + br] : 0.f));
      }
    }
  }
  auto gate = [&](int q, int br) -> float {
    if (!act[q] || lr >= p.G) return 0.f;
    if (p.wgate) return s_gnet[kWaveQ * wave + q][br == 2 ? 1 : 0][lr];
    return p.gates[(((int64_t)b * T + tq[q]) * p.Hq + (int64_t)g * p.G + lr) * 3 + br];
  };
  const float sc = p.scale_log2;
  const int qd = p.l / p.d, rd = p.lsel / p.d;  // key and block lengths in stride units
  const float invq = 1.0f / (float)qd;
  const u32x4_t ones_a = ones_row_operand(lr);

  // One pipeline over all chunks (window, then C1, then C2): chunks c+1 ..
  // c+NBUF-1 are in flight while chunk c is computed.  Copies complete in issue
  // order, so chunk c has landed once at most the later chunks' copies remain.
  auto nld = [&](int c) -> int { return c >= nch ? 0 : ((c >= nW && c < nW + nC) ? NLD_K : NLD_KV); };
  auto begin_chunk = [&](int c) -> const char* {
    if constexpr (NBUF == 3) {
      const int later = nld(c + 1);
      if (later == 0) wait_vmem_le<0>();
      else if (later == NLD_K) wait_vmem_le<NLD_K>();
      else wait_vmem_le<NLD_KV>();
    } else {
      wait_vmem_le<0>();
    }
    lds_barrier();
    if (c + NBUF - 1 < nch) stage(c + NBUF - 1, (c + NBUF - 1) % NBUF);
    return s_buf[c % NBUF];
  };
  // logits of one 32-key half of the staged chunk for the wave's positions
  // (each K fragment read once from LDS and used for all of them)
  // Both halves at once, k-step by k-step over the four 16-key row blocks (eight
  // independent MFMA chains), with the reads of the next KD k-steps in flight.
  auto logits = [&](const char* kt, f32x4_t (&s0)[kWaveQ][2], f32x4_t (&s1)[kWaveQ][2]) {
#pragma unroll
    for (int q = 0; q < kWaveQ; ++q) s0[q][0] = s0[q][1] = s1[q][0] = s1[q][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KT; ++ks)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const u32x4_t a = lds_k<DK>(kt, m, ks, lane);
#pragma unroll
        for (int q = 0; q < kWaveQ; ++q) {
          f32x4_t& d = m < 2 ? s0[q][m] : s1[q][m - 2];
          d = mfma_bf16(a, qf[q][ks], d);
        }
      }
    constexpr int KD = 1;  // registers are nearly all taken by the two positions' state
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * KD, 0);
#pragma unroll
    for (int ks = 0; ks < KT; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * kWaveQ, 0);
      if (ks + KD < KT) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
  };

  // The query fragments must have arrived before the tile copies are queued: the
  // compiler does not count those copies, so a wait it placed for the fragments
  // inside the loop would also drain them.
  wait_vmem_le<0>();
  __syncthreads();  // score rows zeroed (each wave reads only its own rows, zeroed by all)
#pragma unroll
  for (int c0 = 0; c0 < NBUF - 1; ++c0)
    if (c0 < nch) stage(c0, c0);
  int c = 0;

  // Each chunk is processed as two 32-key halves whose logits are issued
  // together, so the exponentials of one half can overlap the other half's MFMAs.

  // ---- W: window (t - w, t], online softmax into acc
  for (int cw = 0; cw < nW; ++cw, ++c) {
    const char* kt = begin_chunk(c);
    const char* vt = kt + SH::kKBytes;
    f32x4_t s0[kWaveQ][2], s1[kWaveQ][2];
    logits(kt, s0, s1);
    const int x0 = xlo + 64 * cw;
    float z0[kWaveQ][2][4], z1[kWaveQ][2][4], ms[kWaveQ];
#pragma unroll
    for (int q = 0; q < kWaveQ; ++q) {
      // keys x with xlo_q < x <= xhi are in the window (none for padding positions)
      const int xhi = act[q] ? tq[q] : -1, xlo_q = tq[q] - p.w;
      mask_range(s0[q], x0, xlo_q, xhi, lg, z0[q]);
      mask_range(s1[q], x0 + 32, xlo_q, xhi, lg, z1[q]);
      ms[q] = max_over_groups_swap(fmaxf(max8(z0[q]), max8(z1[q]))) * sc;
    }
    lazy_rescale_n(ms, mref, acc, lsum);
    u32x4_t pk[kWaveQ];
#pragma unroll
    for (int q = 0; q < kWaveQ; ++q) pk[q] = exp_pack(z0[q], sc, -mref[q]);
    pv_half<DV>(vt, 0, vlane, pk, acc);
#pragma unroll
    for (int q = 0; q < kWaveQ; ++q) lsum[q] = mfma_bf16(ones_a, pk[q], lsum[q]);
#pragma unroll
    for (int q = 0; q < kWaveQ; ++q) pk[q] = exp_pack(z1[q], sc, -mref[q]);
    pv_half<DV>(vt, 1, vlane, pk, acc);
#pragma unroll
    for (int q = 0; q < kWaveQ; ++q) lsum[q] = mfma_bf16(ones_a, pk[q], lsum[q]);
  }
  // acc <- g_win * o_win (the denominator of head lr sits in lane lr, element 0)
#pragma unroll
  for (int q = 0; q < kWaveQ; ++q) {
    const float lt = __shfl(lsum[q][0], lr);
    const float f = lt > 0.f ? gate(q, 2) / lt : 0.f;
#pragma unroll
    for (int j = 0; j < VC; ++j) acc[q][j] *= f;
    if (p.lse && act[q] && lg == 0 && lr < p.G)  // window log-sum-exp (natural log)
      p.lse[(((int64_t)b * T + tq[q]) * p.Hq + (int64_t)g * p.G + lr) * 3 + 2] =
          lt > 0.f ? (mref[q] + __builtin_log2f(lt)) * kLn2 : -INFINITY;
  }

  // ---- C1: exact per-head max and sum over the visible compressed keys
  float lc[kWaveQ];
#pragma unroll
  for (int q = 0; q < kWaveQ; ++q) {
    mref[q] = kNegBig;
    lc[q] = 0.f;
  }
  for (int c1 = 0; c1 < nC; ++c1, ++c) {
    const char* kt = begin_chunk(c);
    f32x4_t s0[kWaveQ][2], s1[kWaveQ][2];
    logits(kt, s0, s1);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int i0 = 64 * c1 + 32 * hh;
#pragma unroll
      for (int q = 0; q < kWaveQ; ++q) {
        float z[2][4];
        mask_range(hh ? s1[q] : s0[q], i0, -1, nvq[q] - 1, lg, z);
        const float mn = fmaxf(mref[q], max_over_groups_swap(max8(z)) * sc);
        float ls = 0.f;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int i = 0; i < 4; ++i) ls += __builtin_amdgcn_exp2f(fmaf(z[mm][i], sc, -mn));
        lc[q] = lc[q] * __builtin_amdgcn_exp2f(mref[q] - mn) + ls;
        mref[q] = mn;
      }
    }
  }
  // p = exp2(s*sc - bias) is the normalised probability; bias = +inf zeroes the
  // padding heads and positions without visible compressed keys
  float bias[kWaveQ], gC[kWaveQ];
#pragma unroll
  for (int q = 0; q < kWaveQ; ++q) {
    const float L = sum_over_groups_swap(lc[q]);
    bias[q] = (L > 0.f && lr < p.G) ? mref[q] + __builtin_log2f(L) : INFINITY;
    gC[q] = gate(q, 0);
    if (p.lse && act[q] && lg == 0 && lr < p.G)  // compressed-branch log-sum-exp (natural log)
      p.lse[(((int64_t)b * T + tq[q]) * p.Hq + (int64_t)g * p.G + lr) * 3] =
          L > 0.f ? (mref[q] + __builtin_log2f(L)) * kLn2 : -INFINITY;
  }

  // The value products of the second pass take the bf16 p the fold uses: acc
  // (g_win o_win so far) is divided by g_cmp of head lr first and multiplied by
  // it afterwards, so acc = g_win o_win + g_cmp o_cmp.  A head whose g_cmp is
  // zero or below 2^-60 takes no compressed-branch values (its contribution is
  // below any bf16 output's resolution).
  bool gz[kWaveQ];
#pragma unroll
  for (int q = 0; q < kWaveQ; ++q) {
    gz[q] = !(gC[q] >= 0x1p-60f);
    const float r = gz[q] ? 1.0f : 1.0f / gC[q];
#pragma unroll
    for (int j = 0; j < VC; ++j) acc[q][j] *= r;
  }

  // ---- C2: normalised p; acc += g_cmp p.Vc; fold p onto selection blocks.
  // Fold: key i covers stride units [i, i+qd), block j covers [j*rd, (j+1)*rd).
  // F[head][block] = sum over a 32-key step of p * overlap (the overlap counts are
  // small integers, exact in bf16; p enters as bf16 hi + lo parts), then summed
  // over the heads into the position's score row.  The overlap operand depends
  // on the step only through i0 mod rd, so for rd <= 32 it is built once.
  auto fold_operand = [&](int i0, int rt) -> u32x4_t {
    const int jb = i0 / rd;
    const int ublo = (jb + 16 * rt + lr) * rd, ubhi = ublo + rd;
    uint32_t ow[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      uint32_t bits[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int key = i0 + step_key(lg, 2 * h + e);
        const int ov = min(key + qd, ubhi) - max(key, ublo);
        bits[e] = __float_as_uint((float)(ov > 0 ? ov : 0)) >> 16;
      }
      ow[h] = bits[0] | (bits[1] << 16);
    }
    return u32x4_t{ow[0], ow[1], ow[2], ow[3]};
  };
  const bool om_const = 32 % rd == 0;
  const u32x4_t om_c0 = fold_operand(0, 0), om_c1 = fold_operand(0, 1);
  for (int c2 = 0; c2 < nC; ++c2, ++c) {
    const char* kt = begin_chunk(c);
    const char* vt = kt + SH::kKBytes;
    f32x4_t s0[kWaveQ][2], s1[kWaveQ][2];
    logits(kt, s0, s1);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int i0 = 64 * c2 + 32 * hh;
      u32x4_t pg[kWaveQ], ph[kWaveQ], pl[kWaveQ];
#pragma unroll
      for (int q = 0; q < kWaveQ; ++q) {
        float a[2][4];
        mask_range(hh ? s1[q] : s0[q], i0, -1, nvq[q] - 1, lg, a);
        const float nb = -bias[q];
        float ra[2][4];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int i = 0; i < 4; ++i) a[mm][i] = __builtin_amdgcn_exp2f(fmaf(a[mm][i], sc, nb));
        ph[q] = pack_probs(a[0], a[1]);
        pg[q] = gz[q] ? u32x4_t{0u, 0u, 0u, 0u} : ph[q];  // B operand: this lane's elements are head lr's
        // rounding residual, so that hi + lo carries p to about 16 bits
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t w = ph[q][2 * mm + (i >> 1)];
            ra[mm][i] = a[mm][i] - ((i & 1) ? bf16_hi(w) : bf16_lo(w));
          }
        pl[q] = pack_probs(ra[0], ra[1]);
      }
      pv_half<DV>(vt, hh, vlane, pg, acc);
      const int jb = i0 / rd;
      const int nrows = (i0 - jb * rd + 31 + qd - 1) / rd + 1;  // blocks the step touches (<= 32)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        if (16 * rt >= nrows) break;
        const u32x4_t om = om_const ? (rt ? om_c1 : om_c0) : fold_operand(i0, rt);
        const int j = jb + 16 * rt + lr;
#pragma unroll
        for (int q = 0; q < kWaveQ; ++q) {
          // F[head 4lg+i][block lr]: the P operand doubles as the A operand (rows = heads)
          f32x4_t F = mfma_bf16(ph[q], om, f32x4_t{0.f, 0.f, 0.f, 0.f});
          F = mfma_bf16(pl[q], om, F);
          const float v = sum_over_groups_swap((F[0] + F[1]) + (F[2] + F[3]));
          const int Jq = act[q] ? tq[q] / p.lsel : -1;
          if (lg == 0 && 16 * rt + lr < nrows && j <= Jq) s_score[kWaveQ * wave + q][j] += v * invq;
        }
      }
    }
  }

#pragma unroll
  for (int q = 0; q < kWaveQ; ++q) {
    const float f = gz[q] ? 1.0f : gC[q];
#pragma unroll
    for (int j = 0; j < VC; ++j) acc[q][j] *= f;
  }

  // ---- top-n per position
#pragma unroll
  for (int q = 0; q < kWaveQ; ++q) {
    if (!act[q]) continue;
    const int J = tq[q] / p.lsel;
    int32_t* out = p.sel + (((int64_t)b * T + tq[q]) * p.H + g) * p.n;
    const float* S = s_score[kWaveQ * wave + q];
    if (J < 128) wave_topn<2>(S, J, p.n, p.nloc, p.finit, out);
    else if (J < 256) wave_topn<4>(S, J, p.n, p.nloc, p.finit, out);
    else if (MAXB <= 512 || J < 512) wave_topn<8>(S, J, p.n, p.nloc, p.finit, out);
    else wave_topn<MAXB / 64>(S, J, p.n, p.nloc, p.finit, out);
  }

  // ---- accumulator (g_win o_win + g_cmp o_cmp) to the workspace
#pragma unroll
  for (int q = 0; q < kWaveQ; ++q) {
    if (!act[q] || lr >= p.G) continue;
    float* dst = p.acc + (((int64_t)b * T + tq[q]) * p.Hq + (int64_t)g * p.G + lr) * DV + 4 * lg;
#pragma unroll
    for (int j = 0; j < VC; ++j) *reinterpret_cast<f32x4_t*>(dst + 16 * j) = acc[q][j];
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: selected branch over the union of the tile's selected blocks.
// ROWS = 32 keys are used per step (a block of l' > 32 takes several steps; for
// l' = 16 the block plus 16 masked rows).
//
// A step's work usually falls on one or two positions, so within a workgroup the
// step's critical path is one wave's chain of LDS reads, MFMAs and softmax while
// the other waves wait at the step's barrier.  The workgroup is therefore small
// (8 positions, 4 waves of two positions each, 68 KB of LDS) so that two of them
// share a compute unit and each fills the other's waits; each position's logits
// run k-step by k-step over the 16-key row blocks (independent MFMA chains),
// with the operand reads of the next k-steps in flight.
constexpr int kSelTile = 8;                  // positions per selected-branch workgroup
constexpr int kSelWaves = 4;                 // waves of the selected-branch workgroup
constexpr int kSelRows = 32;                 // keys per step
constexpr int kSelQ = kSelTile / kSelWaves;  // positions per wave
static_assert(kSelTile <= 16 && kSelQ * kSelWaves == kSelTile, "position masks are 16 bits");
constexpr int kSelThreads = 64 * kSelWaves;

// The K rows of a step are staged row-major (DK*2 bytes per row) by copies that
// each read 1 KB of contiguous source, so every 128-byte line is fetched whole
// by 8 lanes of one instruction.  Row-major MFMA operand reads (16 rows x 16
// bytes per lane group) would hit the same LDS banks, so inside each 128-byte
// line the 16-byte pieces of row r are XOR-permuted by r mod 8: tile piece P
// sits at slot (P & ~7) | ((P & 7) ^ ((P / R) & 7)).  The map is its own
// inverse, so lane i of copy c loads the piece that belongs in slot 64c + i;
// any 8 consecutive lanes of an operand read (8 rows, one piece each) then hit
// 8 different bank groups, and whole 16-row blocks keep the permutation, so the
// operand (m, ks) of a lane sits at its (0, ks) offset + 256*R*m bytes.
template <int DK>
struct SelSwizzle {
  static constexpr int R = DK / 8;  // 16-byte pieces per row
  static_assert(R % 8 == 0, "rows of whole 128-byte lines");
  __device__ static int slot(int P) { return (P & ~7) | ((P & 7) ^ ((P / R) & 7)); }
};

// Stages K rows [row0, row0 + ROWS) as above.  Wave w issues copies c = w,
// w + NW, ...; kcopy[k] is this lane's source byte offset within copy w + NW*k.
// Rows past rowmax are replaced by row rowmax.
template <int DK, int ROWS, int NW>
struct SelKCopies {
  static constexpr int NI = ROWS * SelSwizzle<DK>::R / 64, PW = (NI + NW - 1) / NW;
};
template <int DK, int ROWS, int NW>
__device__ __forceinline__ void stage_k_rowmajor(const uint16_t* base, int64_t row0, int64_t rowmax, uint32_t dst,
                                                 int wave, int lane, const uint32_t (&kcopy)[SelKCopies<DK, ROWS, NW>::PW]) {
  using SW = SelSwizzle<DK>;
  constexpr int NI = SelKCopies<DK, ROWS, NW>::NI, PW = SelKCopies<DK, ROWS, NW>::PW;
  if (row0 + ROWS - 1 <= rowmax) {  // wave-uniform
    const char* tile = reinterpret_cast<const char*>(base + row0 * DK);
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int c = wave + NW * k;
      if (NI % NW != 0 && c >= NI) break;
      copy16_sb_at(tile + 1024 * c, kcopy[k], dst + 1024 * c);
    }
  } else {
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int c = wave + NW * k;
      if (NI % NW != 0 && c >= NI) break;
      const int P = SW::slot(64 * c + lane);
      int64_t row = row0 + P / SW::R;
      row = row < rowmax ? row : rowmax;
      copy16_to_lds_at(base + row * DK + 8 * (P % SW::R), dst + 1024 * c);
    }
  }
}

template <int DK, int DV, int LSEL>
__global__ __launch_bounds__(kSelThreads, 2) void pf_sel_kernel(PrefillParams p) {
  using SH = PfShape<DK, DV>;
  using SW = SelSwizzle<DK>;
  constexpr int KT = SH::KT, VC = SH::VC;
  constexpr int ROWS = kSelRows;
  constexpr int MT = ROWS / 16, NKS = ROWS / 32, SPB = LSEL > ROWS ? LSEL / ROWS : 1;
  constexpr int NBUF = 3;                     // NBUF - 1 steps in flight
  using SO = StageOffsets<DK, DV, ROWS, kSelWaves>;
  constexpr int NLD = SO::kMinCopiesKV;       // copies per wave per step (K and V), at least
  constexpr int kStepBytes = SO::kKBytes + SO::kVBytes;
  __shared__ __attribute__((aligned(1024))) char s_buf[NBUF][kStepBytes];
  __shared__ uint32_t s_mask[kPfMaxBlocks];  // per block: bit q set if position t0+q chose it
  __shared__ uint32_t s_list[kPfMaxBlocks];  // the union, ascending: block id << 16 | mask
  __shared__ int s_scan[kSelWaves];
  __shared__ int s_nu;

  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T;
  const int nbg = p.B * p.H, bid = (int)blockIdx.x;
  const int bgi = bid % nbg;
  const int b = bgi / p.H, g = bgi % p.H;
  const int t0 = ((T + kSelTile - 1) / kSelTile - 1 - bid / nbg) * kSelTile;  // latest tiles first
  const int tlast = min(t0 + kSelTile - 1, T - 1);
  const int Jtile = tlast / LSEL;
  const int64_t bg = (int64_t)b * p.H + g;
  const uint16_t* kraw = p.k + bg * T * DK;
  const uint16_t* vraw = p.v + bg * T * DV;

  // ---- g_slc from the gate network (when given) for this lane's head lr and
  // the wave's positions, before any other load
  float gsl[kSelQ];
  if (p.wgate) {
    const int hq = g * p.G + (lr < p.G ? lr : 0);
    const uint16_t* wrow = p.wgate + ((size_t)hq * 3 + 1) * DK;
#pragma unroll
    for (int q = 0; q < kSelQ; ++q) {
      const int tt = min(t0 + kSelQ * wave + q, T - 1);
      const float z = sum_over_groups_swap(
          gate_dot_quarter<DK>(p.q + (((int64_t)b * T + tt) * p.Hq + hq) * DK, wrow, lg));
      gsl[q] = gate_sigmoid(z + (p.bgate ? p.bgate[hq * 3 + 1] : 0.f));
    }
  }

  // ---- union of the tile's selections
  for (int j = tid; j <= Jtile; j += kSelThreads) s_mask[j] = 0u;
  __syncthreads();
  for (int e = tid; e < kSelTile * p.n; e += kSelThreads) {
    const int q = e / p.n;
    if (t0 + q < T) {
      const int j = p.sel[(((int64_t)b * T + t0 + q) * p.H + g) * p.n + (e - q * p.n)];
      if (j >= 0 && j <= Jtile) atomicOr(&s_mask[j], 1u << q);
    }
  }
  __syncthreads();
  {
    constexpr int PER = kPfMaxBlocks / kSelThreads;
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int j = tid * PER + k;
      cnt += (j <= Jtile && s_mask[j] != 0u) ? 1 : 0;
    }
    int total;
    int pos = block_scan<kSelThreads>(cnt, s_scan, &total);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int j = tid * PER + k;
      if (j <= Jtile && s_mask[j] != 0u) s_list[pos++] = ((uint32_t)j << 16) | s_mask[j];
    }
    if (tid == 0) s_nu = total;
  }
  __syncthreads();
  const int nsteps = s_nu * SPB;

  int tq[kSelQ];
  bool act[kSelQ];
  u32x4_t qf[kSelQ][KT];
  f32x4_t acc[kSelQ][VC];
  f32x4_t lsum[kSelQ];
  float mref[kSelQ];
#pragma unroll
  for (int q = 0; q < kSelQ; ++q) {
    tq[q] = t0 + kSelQ * wave + q;
    act[q] = tq[q] < T;
    const int tt = act[q] ? tq[q] : T - 1;
    load_q_frags<DK>(p.q + (((int64_t)b * T + tt) * p.Hq + (int64_t)g * p.G) * DK, p.G, lg, lr, qf[q]);
#pragma unroll
    for (int j = 0; j < VC; ++j) acc[q][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lsum[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    mref[q] = kNegBig;
  }
  const float sc = p.scale_log2;
  const u32x4_t ones_a = ones_row_operand(lr);

  // this lane's byte offsets of its K operands (m = 0) in a staged step, and of
  // its K copies' source pieces
  uint32_t koff[KT];
#pragma unroll
  for (int ks = 0; ks < KT; ++ks) koff[ks] = 16u * (uint32_t)SW::slot(SW::R * lr + 4 * ks + lg);
  constexpr int KPW = SelKCopies<DK, ROWS, kSelWaves>::PW;
  uint32_t kcopy[KPW];
#pragma unroll
  for (int k = 0; k < KPW; ++k) {
    const int c = wave + kSelWaves * k;
    kcopy[k] = 16u * (uint32_t)SW::slot(64 * c + lane) - 1024u * (uint32_t)c;
  }
  const uint32_t vcopy = VSwizzle<DV>::copy_offset(wave, lane);
  const uint32_t vlane = vt_lane_offset<DV>(lg, lr);

  const uint32_t lds_buf0 = lds_addr_of(&s_buf[0][0]);
  auto step_row0 = [&](int st) -> int64_t {
    const int u = st / SPB;
    return (int64_t)(s_list[u] >> 16) * LSEL + (int64_t)(st - u * SPB) * ROWS;
  };
  auto stage = [&](int st, int buf) {
    const int64_t r0 = (int64_t)__builtin_amdgcn_readfirstlane((int)step_row0(st));
    const uint32_t kt = lds_buf0 + (uint32_t)(buf * kStepBytes);
    stage_k_rowmajor<DK, ROWS, kSelWaves>(kraw, r0, T - 1, kt, wave, lane, kcopy);
    stage_v_swizzled<DV, ROWS, kSelWaves>(vraw, r0, T - 1, kt + SO::kKBytes, wave, lane, vcopy);
  };

  wait_vmem_le<0>();  // query fragments in (see the compressed-branch kernel)
#pragma unroll
  for (int s0 = 0; s0 < NBUF - 1; ++s0)
    if (s0 < nsteps) stage(s0, s0);
  for (int st = 0; st < nsteps; ++st) {
    // step st has landed once at most the later step's copies are outstanding
    if (st + 1 < nsteps) wait_vmem_le<NLD>();
    else wait_vmem_le<0>();
    lds_barrier();
    if (st + NBUF - 1 < nsteps) stage(st + NBUF - 1, (st + NBUF - 1) % NBUF);
    const uint32_t ent = (uint32_t)__builtin_amdgcn_readfirstlane((int)s_list[st / SPB]);
    const uint32_t mine = (ent >> (kSelQ * wave)) & ((1u << kSelQ) - 1u);
    if (mine == 0u) continue;
    const char* kt = s_buf[st % NBUF];
    const char* vt = s_buf[st % NBUF] + SO::kKBytes;
    const int jblk = (int)(ent >> 16);
    const int x0 = jblk * LSEL + (st % SPB) * ROWS;
    const int xend = (jblk + 1) * LSEL;  // first row past the block

#pragma unroll
    for (int q = 0; q < kSelQ; ++q) {
      if (!((mine >> q) & 1u)) continue;
      f32x4_t s[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) s[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KT; ++ks)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          s[m] = mfma_bf16(*reinterpret_cast<const u32x4_t*>(kt + koff[ks] + 256 * SW::R * m), qf[q][ks], s[m]);
      // the V^T operands of the first 32 keys, in flight during the softmax
      u32x4_t vop[VC];
#pragma unroll
      for (int j = 0; j < VC; ++j) vop[j] = lds_vt_operand<DV>(vt, 0, j, vlane);
      // Instruction order: the K operands of the first KD k-steps, then each
      // k-step's MFMAs followed by the reads of the k-step KD later, then the V
      // reads -- so about KD k-steps of operand reads are always in flight.
      {
        constexpr int KD = KT < kReadAhead ? KT : kReadAhead;
        __builtin_amdgcn_sched_group_barrier(0x100, MT * KD, 0);
#pragma unroll
        for (int ks = 0; ks < KT; ++ks) {
          __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);
          if (ks + KD < KT) __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, VC * 2, 0);
      }
      float z[MT][4];
      if (x0 + ROWS - 1 <= tq[q] && x0 + ROWS <= xend) {  // wave-uniform: no row masked
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) z[m][i] = s[m][i];
      } else {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int x = x0 + 16 * m + 4 * lg + i;
            z[m][i] = (x <= tq[q] && x < xend) ? s[m][i] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[m][i]);
      mx = max_over_groups_swap(mx);
      lazy_rescale(mx * sc, mref[q], acc[q], lsum[q]);
      const float nm = -mref[q];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[m][i] = __builtin_amdgcn_exp2f(fmaf(z[m][i], sc, nm));
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4_t pk = pack_probs(z[2 * ks], z[2 * ks + 1]);
        if (ks > 0) {
#pragma unroll
          for (int j = 0; j < VC; ++j) vop[j] = lds_vt_operand<DV>(vt, ks, j, vlane);
        }
#pragma unroll
        for (int j = 0; j < VC; ++j) acc[q][j] = mfma_bf16(vop[j], pk, acc[q][j]);
        lsum[q] = mfma_bf16(ones_a, pk, lsum[q]);
      }
    }
  }

  // ---- out = bf16(acc_in + g_slc * o_slc); acc[q][j] element i is channel
  // 16j + 4*lg + i of head lr
#pragma unroll
  for (int q = 0; q < kSelQ; ++q) {
    const float lt = __shfl(lsum[q][0], lr);
    if (!act[q] || lr >= p.G) continue;
    const int64_t hrow = ((int64_t)b * T + tq[q]) * p.Hq + (int64_t)g * p.G + lr;
    const float f = lt > 0.f ? (p.wgate ? gsl[q] : p.gates[hrow * 3 + 1]) / lt : 0.f;
    if (p.lse && lg == 0)  // selected-branch log-sum-exp (natural log)
      p.lse[hrow * 3 + 1] = lt > 0.f ? (mref[q] + __builtin_log2f(lt)) * kLn2 : -INFINITY;
    const float* src = p.acc + hrow * DV + 4 * lg;
    uint16_t* dst = p.out + hrow * DV + 4 * lg;
#pragma unroll
    for (int j = 0; j < VC; ++j) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(src + 16 * j);
      *reinterpret_cast<u32x2_t*>(dst + 16 * j) =
          u32x2_t{pack_bf16x2(a[0] + f * acc[q][j][0], a[1] + f * acc[q][j][1]),
                  pack_bf16x2(a[2] + f * acc[q][j][2], a[3] + f * acc[q][j][3])};
    }
  }
}

template <int DK, int DV>
static hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t s, const PhaseEvents* ev) {
  const dim3 grid((unsigned)((int64_t)p.B * p.H * p.ntile)), blk(kThreads);
  // up to 512 candidate blocks the score rows leave room for a third key buffer
  if ((p.T - 1) / p.lsel < 512) hipLaunchKernelGGL((pf_cmp_win_kernel<DK, DV, 3, 512>), grid, blk, 0, s, p);
  else hipLaunchKernelGGL((pf_cmp_win_kernel<DK, DV, 2, kPfMaxBlocks>), grid, blk, 0, s, p);
  if (ev) hipEventRecord(ev->ev[2], s);
  const dim3 sgrid((unsigned)((int64_t)p.B * p.H * ((p.T + kSelTile - 1) / kSelTile))), sblk(kSelThreads);
  switch (p.lsel) {
    case 16: hipLaunchKernelGGL((pf_sel_kernel<DK, DV, 16>), sgrid, sblk, 0, s, p); break;
    case 32: hipLaunchKernelGGL((pf_sel_kernel<DK, DV, 32>), sgrid, sblk, 0, s, p); break;
    case 64: hipLaunchKernelGGL((pf_sel_kernel<DK, DV, 64>), sgrid, sblk, 0, s, p); break;
    case 128: hipLaunchKernelGGL((pf_sel_kernel<DK, DV, 128>), sgrid, sblk, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  if (ev) hipEventRecord(ev->ev[3], s);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int DK, int DV, hipStream_t s, const PhaseEvents* ev) {
  if (DK == 192 && DV == 128) return launch_prefill_t<192, 128>(p, s, ev);
  if (DK == 128 && DV == 128) return launch_prefill_t<128, 128>(p, s, ev);
  if (DK == 64 && DV == 64) return launch_prefill_t<64, 64>(p, s, ev);
  return hipErrorInvalidValue;
}

}  // namespace nsa

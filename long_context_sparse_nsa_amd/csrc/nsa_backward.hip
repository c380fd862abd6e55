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
//   bwd_kv_kernel<SLC>  one wave per 16 raw keys and up to kSlcSplit of the
//                       positions that selected the keys' block (counted and split by
//                       bwd_slc_count_kernel / bwd_slc_scan_kernel); partial sums per split.
//   bwd_kv_kernel<CMP>  one wave per 16 compressed keys and a range of positions;
//                       partial sums per range.
//   bwd_kv_reduce_kernel  adds the selected partials to dk, dv and sums the
//                       compressed ones into dk_cmp, dv_cmp, in a fixed order.
// Products are bf16 MFMA (P and dS rounded to bf16 as operands) with fp32 sums;
// no atomics on gradients, so results repeat bit for bit.
#include <algorithm>

#include "nsa_train.hpp"
#include "nsa_tiles.hpp"

namespace nsa {
namespace {

constexpr int kCmp = 0, kSlc = 1, kWin = 2;  // branch ids (gate and lse slot order)
constexpr int kBwdWaves = 4;                 // waves per workgroup
constexpr float kNegInf = -__builtin_inff();

// Wait until this wave's copies of at most `later` subsequent steps (C copy
// instructions each, LATER at most) are still in flight; copies complete in
// issue order.
template <int C, int LATER>
__device__ __forceinline__ void wait_steps(int later) {
  static_assert(LATER >= 1 && LATER <= 4 && C * LATER < 64, "vmcnt range");
  if (later >= 4 && LATER >= 4) wait_vmem_le<C * (LATER >= 4 ? 4 : 0)>();
  else if (later >= 3 && LATER >= 3) wait_vmem_le<C * (LATER >= 3 ? 3 : 0)>();
  else if (later >= 2 && LATER >= 2) wait_vmem_le<C * (LATER >= 2 ? 2 : 0)>();
  else if (later >= 1) wait_vmem_le<C>();
  else wait_vmem();
}

__device__ __forceinline__ int n_visible(int t, int l, int d, int nc) {
  return t >= l - 1 ? min(nc, (t - l + 1) / d + 1) : 0;
}

// ---------------------------------------------------------------------------
// LDS blocks of D-wide bf16 rows: the 16-byte chunk c of row r sits at slot
// c ^ (r & 7), so that MFMA operand reads of 16 rows at one column spread over
// the LDS banks.

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

// ---------------------------------------------------------------------------
// Query side.  A workgroup owns 4 consecutive positions of one (b, g); a wave one
// position, its 16 heads the MFMA columns.  The 32-key tiles of the three
// branches are copied once into LDS for the four waves, kQtBuf buffers deep:
// the compressed blocks [0, nvis) and the window's union are contiguous ranges,
// the selected branch walks the union of the four positions' blocks, each block
// marked with the waves that chose it.  Pass 1 recomputes every branch's online
// softmax (statistics record, dgates); pass 2 stages the same tiles again and
// accumulates dq^T += K^T dS^T.

constexpr int kQtBuf = 3;

template <int DK, int DV>
struct QtShape {
  static constexpr int kK = 32 * DK, kV = 32 * DV;  // bf16 elements of a 32-key tile
  static constexpr int kBuf = 2 * kK + 2 * kV;        // bytes per buffer
  static constexpr int kCpK = 32 * DK / 8 / 256, kCpV = 32 * DV / 8 / 256;  // copies per wave
  static constexpr int kCopies = kCpK + kCpV;
};

// lds_rows_product with two products sharing the row pieces: acc1 += rows^T pb1,
// acc2 += rows^T pb2.
template <int D>
__device__ __forceinline__ void lds_rows_product2(const char* blk, const int (&rows)[8], int lr, const u32x4_t& pb1,
                                                  f32x4_t (&acc1)[D / 16], const u32x4_t& pb2,
                                                  f32x4_t (&acc2)[D / 16]) {
#pragma unroll
  for (int u = 0; u < D / 64; ++u) {
    uint32_t w[8][2];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const u32x2_t x = *reinterpret_cast<const u32x2_t*>(blk + sw_off<D>(rows[r], (D / 16) * lr + 4 * u));
      w[r][0] = x[0];
      w[r][1] = x[1];
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int wd = jj >> 1, h = jj & 1;
      const u32x4_t va = {pack_halves(w[0][wd], w[1][wd], h), pack_halves(w[2][wd], w[3][wd], h),
                          pack_halves(w[4][wd], w[5][wd], h), pack_halves(w[6][wd], w[7][wd], h)};
      acc1[4 * u + jj] = mfma_bf16(va, pb1, acc1[4 * u + jj]);
      acc2[4 * u + jj] = mfma_bf16(va, pb2, acc2[4 * u + jj]);
    }
  }
}

// ONEPASS: the forward's per-branch log-sum-exp is given (p.lse_in), so one walk
// over the tiles suffices: with P = exp(s q.k - lse) known, D_c = g_c sum_k P dP
// accumulates beside dq = s (sum_k g_c P dP k - sum_c D_c sum_{k in c} P k); the
// second sum is kept per branch and folded in when the branch's tiles end.
template <int DK, int DV, bool ONEPASS>
__global__ __launch_bounds__(256, 2) void bwd_query_kernel(BwdParams p) {
  using SH = QtShape<DK, DV>;
  __shared__ __attribute__((aligned(1024))) char s_buf[kQtBuf][SH::kBuf];
  __shared__ uint32_t s_bm[4][kPfMaxBlocks / 32];  // each wave's selected blocks
  __shared__ int32_t s_sel[kPfMaxBlocks];          // union, ascending: block | wave mask << 16
  __shared__ int s_scan[4];
  const uint32_t lds0 = lds_addr_of(&s_buf[0][0]);

  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Consecutive workgroups cycle through the (b, g) pairs; latest positions first.
  const int nbg = p.B * p.H;
  const int bid = (int)blockIdx.x;
  const int tile = p.nqt - 1 - bid / nbg;
  const int bg = bid - (bid / nbg) * nbg;
  const int b = bg / p.H, g = bg - (bg / p.H) * p.H;
  const int T = p.T, G = p.G, Hq = p.Hq, nc = p.nc;
  const int t0 = tile * kBwdWaves, t = t0 + wave, tl = min(t0 + kBwdWaves - 1, T - 1);
  const bool tv = t < T;
  const int64_t bgl = (int64_t)b * p.H + g;
  const uint16_t* kraw = p.k + bgl * T * DK;
  const uint16_t* vraw = p.v + bgl * T * DV;
  const uint16_t* kcmp = p.kc + bgl * nc * DK;
  const uint16_t* vcmp = p.vc + bgl * nc * DV;
  const int64_t qrow = ((int64_t)b * T + (tv ? t : tl)) * Hq + (int64_t)g * G;  // the group's first head
  const bool hv = lr < G;

  // Union of the four positions' selected blocks.
  for (int i = tid; i < 4 * (kPfMaxBlocks / 32); i += 256) (&s_bm[0][0])[i] = 0u;
  __syncthreads();
  if (tv) {
    for (int s = lane; s < p.n; s += 64) {
      const int j = p.sel[(((int64_t)b * T + t) * p.H + g) * p.n + s];
      if (j >= 0 && j < p.nblk) atomicOr(&s_bm[wave][j >> 5], 1u << (j & 31));
    }
  }
  __syncthreads();
  uint32_t mw[4] = {0u, 0u, 0u, 0u}, un = 0u;
  if (tid < kPfMaxBlocks / 32) {
#pragma unroll
    for (int w = 0; w < 4; ++w) mw[w] = s_bm[w][tid];
    un = mw[0] | mw[1] | mw[2] | mw[3];
  }
  int nsel;
  int off = block_scan<256>(__builtin_popcount(un), s_scan, &nsel);
  while (un) {
    const int bit = __builtin_ctz(un);
    un &= un - 1;
    int mask = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) mask |= (int)((mw[w] >> bit) & 1u) << w;
    s_sel[off++] = (32 * tid + bit) | (mask << 16);
  }
  __syncthreads();

  // The workgroup's tiles: compressed, selected, window; pass 2 repeats them.
  const int ncmp = (n_visible(tl, p.l, p.d, nc) + 31) / 32;
  const int tps = max(1, p.lsel / 32);  // tiles per selected block
  const int nslc = nsel * tps;
  const int wlo = max(0, t0 - p.w + 1);
  const int nwin = (tl - wlo) / 32 + 1;
  const int ntile = ncmp + nslc + nwin, nstep = ONEPASS ? ntile : 2 * ntile;

  auto desc = [&](int i, int& br, int& k0, int& wm, int& kend) {
    const int u = i < ntile ? i : i - ntile;
    if (u < ncmp) {
      br = kCmp; k0 = 32 * u; wm = 0xF; kend = nc;
    } else if (u < ncmp + nslc) {
      const int e = s_sel[(u - ncmp) / tps], j = e & 0xFFFF;
      br = kSlc; k0 = j * p.lsel + 32 * ((u - ncmp) % tps); wm = e >> 16; kend = min(j * p.lsel + p.lsel, T);
    } else {
      br = kWin; k0 = wlo + 32 * (u - ncmp - nslc); wm = 0xF; kend = T;
    }
  };

  // This lane's share of a tile's copies, computed once: row r (bits 0..7) and the
  // byte offset of global chunk (slot ^ (r & 7)) within the row (bits 8..).
  uint32_t cpk[SH::kCpK], cpv[SH::kCpV];
#pragma unroll
  for (int j = 0; j < SH::kCpK; ++j) {
    const int pch = (wave * SH::kCpK + j) * 64 + lane;
    const int r = pch / (DK / 8), sl = pch - r * (DK / 8);
    cpk[j] = (uint32_t)r | ((uint32_t)(16 * (sl ^ (r & 7))) << 8);
  }
#pragma unroll
  for (int j = 0; j < SH::kCpV; ++j) {
    const int pch = (wave * SH::kCpV + j) * 64 + lane;
    const int r = pch / (DV / 8), sl = pch - r * (DV / 8);
    cpv[j] = (uint32_t)r | ((uint32_t)(16 * (sl ^ (r & 7))) << 8);
  }
  auto issue = [&](int i) {
    int br, k0, wm, kend;
    desc(i, br, k0, wm, kend);
    const int nk = br == kCmp ? nc : T;
    const uint16_t* kb = (br == kCmp ? kcmp : kraw) + (int64_t)k0 * DK;  // the tile's first row
    const uint16_t* vb = (br == kCmp ? vcmp : vraw) + (int64_t)k0 * DV;
    const uint32_t lim = (uint32_t)(nk - 1 - k0);  // rows past the end read the last row (masked later)
    const uint32_t buf = lds0 + (uint32_t)((i % kQtBuf) * SH::kBuf);
#pragma unroll
    for (int j = 0; j < SH::kCpK; ++j)
      copy16_sb_at(kb, min(cpk[j] & 0xFFu, lim) * (uint32_t)(DK * 2) + (cpk[j] >> 8),
                   buf + (wave * SH::kCpK + j) * 1024);
#pragma unroll
    for (int j = 0; j < SH::kCpV; ++j)
      copy16_sb_at(vb, min(cpv[j] & 0xFFu, lim) * (uint32_t)(DV * 2) + (cpv[j] >> 8),
                   buf + 2 * SH::kK + (wave * SH::kCpV + j) * 1024);
  };

  u32x4_t qf[DK / 32], of[DV / 32];
  load_q_frags<DK>(p.q + qrow * DK, tv ? G : 0, lg, lr, qf);
  load_q_frags<DV>(p.dout + qrow * DV, tv ? G : 0, lg, lr, of);
  float gt[3];
  if (p.wgate) {  // gate network: sigmoid(w_gate[h, c] . q_h + b_gate[h, c]), lane parts in the q-fragment layout
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      float z = 0.f;
      if (tv && hv) {
        const uint16_t* wr = p.wgate + ((int64_t)(g * G + lr) * 3 + c) * DK + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
          const u32x4_t wv = ld16(wr + 32 * kk);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            z = fmaf(bf16_lo(wv[u]), bf16_lo(qf[kk][u]), z);
            z = fmaf(bf16_hi(wv[u]), bf16_hi(qf[kk][u]), z);
          }
        }
      }
      z = sum_over_groups(z);
      if (p.bgate && hv) z += p.bgate[(g * G + lr) * 3 + c];
      gt[c] = (tv && hv) ? gate_sigmoid(z) : 0.f;
    }
  } else {
#pragma unroll
    for (int c = 0; c < 3; ++c) gt[c] = (tv && hv) ? p.gates[(qrow + lr) * 3 + c] : 0.f;
  }
  const int nvis = tv ? n_visible(t, p.l, p.d, nc) : 0;
  const float sl2 = p.scale_log2;
  wait_vmem();

  // One pipeline step: wait for tile i, hand the next buffer to the copies.
  auto step_begin = [&](int i) {
    wait_steps<SH::kCopies, kQtBuf - 2>(min(nstep - 1 - i, kQtBuf - 2));
    lds_barrier();
    if (i + kQtBuf - 1 < nstep) issue(i + kQtBuf - 1);
  };
  // This wave's valid keys of step i's tile: [klo, khi).
  auto key_range = [&](int br, int k0, int wm, int kend, int& klo, int& khi) {
    klo = 0;
    khi = 0;
    if (tv && ((wm >> wave) & 1)) {
      if (br == kCmp) khi = nvis;
      else if (br == kSlc) khi = min(kend, t + 1);
      else { klo = t - p.w + 1; khi = t + 1; }
    }
    klo = max(klo, k0);
    khi = min(khi, k0 + 32);
  };
  // dq store (scaled), plus the gate network's path.
  auto store_dq = [&](const f32x4_t (&dqa)[DK / 16], const float (&dg_c)[3]) {
    if (!(tv && hv)) return;
    float* dst = p.dq + (qrow + lr) * DK;
    float dz[3];  // gate network: dq_h += sum_c dz_c w_gate[h, c], dz_c = dgates_c g_c (1 - g_c)
#pragma unroll
    for (int c = 0; c < 3; ++c) dz[c] = dg_c[c] * gt[c] * (1.f - gt[c]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j4 = 0; j4 < DK / 64; ++j4) {
        const int j = 4 * j4, ch = (DK / 16) * (4 * lg + i) + j;
        f32x4_t v = f32x4_t{dqa[j][i], dqa[j + 1][i], dqa[j + 2][i], dqa[j + 3][i]} * p.scale;
        if (p.wgate) {
#pragma unroll
          for (int c = 0; c < 3; ++c) {
            const u32x2_t w = ld8(p.wgate + ((int64_t)(g * G + lr) * 3 + c) * DK + ch);
            v += f32x4_t{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])} * dz[c];
          }
        }
        *reinterpret_cast<f32x4_t*>(dst + ch) = v;
      }
  };

  if constexpr (ONEPASS) {
    float ls2[3], dg_c[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 3; ++c) ls2[c] = (tv && hv) ? p.lse_in[(qrow + lr) * 3 + c] * kLog2e : 0.f;
    f32x4_t dqa[DK / 16], bv[DK / 16];
#pragma unroll
    for (int j = 0; j < DK / 16; ++j) {
      dqa[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      bv[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    float dsum = 0.f;  // this lane's part of sum_k P dP over the current branch
    int cur = 0;
    auto close_branch = [&](const int c) {
      const float ds = sum_over_groups(dsum);  // dout . o_c
      const float gc = c == kCmp ? gt[0] : (c == kSlc ? gt[1] : gt[2]);
      const float D = gc * ds;
#pragma unroll
      for (int j = 0; j < DK / 16; ++j) {
        dqa[j] -= bv[j] * D;
        bv[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      if (c == kCmp) dg_c[0] = ds; else if (c == kSlc) dg_c[1] = ds; else dg_c[2] = ds;
      if (tv && lg == 0) {
        float* rec = p.stat + ((((int64_t)c * p.B + b) * T + t) * p.H + g) * kStatFloats;
        const float lsc = c == kCmp ? ls2[0] : (c == kSlc ? ls2[1] : ls2[2]);
        rec[lr] = hv ? lsc : 0.f;
        rec[16 + lr] = hv ? D : 0.f;
        rec[32 + lr] = gc;
        if (hv) p.dgates[(qrow + lr) * 3 + c] = ds;
      }
      dsum = 0.f;
    };
    for (int i = 0; i < kQtBuf - 1 && i < nstep; ++i) issue(i);
    for (int i = 0; i < nstep; ++i) {
      step_begin(i);
      int br, k0, wm, kend, klo, khi;
      desc(i, br, k0, wm, kend);
      if (cur < br) {
        while (cur < br) close_branch(cur++);
        wait_vmem();  // keep the copy count exact for the next wait
      }
      key_range(br, k0, wm, kend, klo, khi);
      if (klo >= khi) continue;
      const char* kt = s_buf[i % kQtBuf];
      const char* vt = kt + 2 * SH::kK;
      const float ls = br == kCmp ? ls2[0] : (br == kSlc ? ls2[1] : ls2[2]);
      const float gc = br == kCmp ? gt[0] : (br == kSlc ? gt[1] : gt[2]);
      // Two 16-key halves: logits and dout.v (16x16x32), then both sums over the
      // half's keys with 16x16x16 products whose B operand is the half's P tile as
      // it stands (lane: head lr, keys 4lg .. 4lg+3).
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4_t kf[DK / 32], vf[DV / 32];
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) kf[kk] = lds_frag<DK>(kt, 16 * hh + lr, 8 * lg + 32 * kk);
#pragma unroll
        for (int kk = 0; kk < DV / 32; ++kk) vf[kk] = lds_frag<DV>(vt, 16 * hh + lr, 8 * lg + 32 * kk);
        const f32x4_t sv = qk_tile<DK>(kf, qf), dp = qk_tile<DV>(vf, of);
        float pa[4], pb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int x = k0 + 16 * hh + 4 * lg + e;
          const float pr = (x >= klo && x < khi) ? __builtin_amdgcn_exp2f(sv[e] * sl2 - ls) : 0.f;
          dsum = fmaf(pr, dp[e], dsum);
          pa[e] = pr * gc * dp[e];
          pb[e] = pr;
        }
        // g P dP as bf16 high + low parts (about 16 significant bits): the two sums
        // cancel in dq = s (A - D Bv), and with one key per branch (P rounds to
        // exactly 1) the difference is 0, so A's rounding must stay well below it.
        // P <= 1 itself enters as one bf16, like the probabilities of the other products.
        u32x2_t opa, opal, opb;
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          opa[w2] = pack_bf16x2(pa[2 * w2], pa[2 * w2 + 1]);
          opb[w2] = pack_bf16x2(pb[2 * w2], pb[2 * w2 + 1]);
          opal[w2] = pack_bf16x2(pa[2 * w2] - bf16_lo(opa[w2]), pa[2 * w2 + 1] - bf16_hi(opa[w2]));
        }
#pragma unroll
        for (int u = 0; u < DK / 64; ++u) {  // channels (DK/16)*lr + 4u .. +3 of keys 16hh + 4lg + r
          uint32_t w[4][2];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const u32x2_t x2 =
                *reinterpret_cast<const u32x2_t*>(kt + sw_off<DK>(16 * hh + 4 * lg + r, (DK / 16) * lr + 4 * u));
            w[r][0] = x2[0];
            w[r][1] = x2[1];
          }
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int wd = jj >> 1, h = jj & 1;
            const u32x2_t va = {pack_halves(w[0][wd], w[1][wd], h), pack_halves(w[2][wd], w[3][wd], h)};
            dqa[4 * u + jj] = mfma16_bf16(va, opa, dqa[4 * u + jj]);
            dqa[4 * u + jj] = mfma16_bf16(va, opal, dqa[4 * u + jj]);
            bv[4 * u + jj] = mfma16_bf16(va, opb, bv[4 * u + jj]);
          }
        }
      }
    }
    while (cur < 3) close_branch(cur++);
    store_dq(dqa, dg_c);
    return;
  }

  // Pass-1 state of the current branch, and the finished branches' statistics.
  float m = kNegInf, l = 0.f;
  f32x4_t acc[DV / 16];
#pragma unroll
  for (int j = 0; j < DV / 16; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float lse_c[3] = {0.f, 0.f, 0.f}, dc_c[3] = {0.f, 0.f, 0.f}, dg_c[3] = {0.f, 0.f, 0.f};
  int fin = 0;
  auto finalize = [&](const int c) {
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t* src = p.dout + (qrow + lr) * DV + (DV / 16) * (4 * lg + i);
#pragma unroll
      for (int u = 0; u < DV / 64; ++u) {
        const u32x2_t x = (tv && hv) ? ld8(src + 4 * u) : u32x2_t{0u, 0u};
        dot = fmaf(acc[4 * u][i], bf16_lo(x[0]), dot);
        dot = fmaf(acc[4 * u + 1][i], bf16_hi(x[0]), dot);
        dot = fmaf(acc[4 * u + 2][i], bf16_lo(x[1]), dot);
        dot = fmaf(acc[4 * u + 3][i], bf16_hi(x[1]), dot);
      }
    }
    dot = sum_over_groups(dot);
    const bool any = l > 0.f;
    dot = any ? dot / l : 0.f;  // dout . o_c
    const float gc = c == kCmp ? gt[0] : (c == kSlc ? gt[1] : gt[2]);
    const float ls = any ? m + __log2f(l) : 0.f, dcv = gc * dot;
    if (c == kCmp) { lse_c[0] = ls; dc_c[0] = dcv; dg_c[0] = dot; }
    else if (c == kSlc) { lse_c[1] = ls; dc_c[1] = dcv; dg_c[1] = dot; }
    else { lse_c[2] = ls; dc_c[2] = dcv; dg_c[2] = dot; }
    if (tv && lg == 0) {  // statistics record of (c, b, t, g): lse[16] | D[16] | gate[16], zeros past G
      float* rec = p.stat + ((((int64_t)c * p.B + b) * T + t) * p.H + g) * kStatFloats;
      rec[lr] = hv ? ls : 0.f;
      rec[16 + lr] = hv ? dcv : 0.f;
      rec[32 + lr] = gc;
      if (hv) p.dgates[(qrow + lr) * 3 + c] = dot;
    }
    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int j = 0; j < DV / 16; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  for (int i = 0; i < kQtBuf - 1 && i < nstep; ++i) issue(i);
  // Pass 1: each branch's online softmax.
  for (int i = 0; i < ntile; ++i) {
    step_begin(i);
    int br, k0, wm, kend, klo, khi;
    desc(i, br, k0, wm, kend);
    if (fin < br) {
      while (fin < br) finalize(fin++);
      wait_vmem();  // keep the copy count exact for the next wait
    }
    key_range(br, k0, wm, kend, klo, khi);
    if (klo >= khi) continue;
    const char* kt = s_buf[i % kQtBuf];
    const char* vt = kt + 2 * SH::kK;
    u32x4_t kf0[DK / 32], kf1[DK / 32];
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) {
      kf0[kk] = lds_frag<DK>(kt, lr, 8 * lg + 32 * kk);
      kf1[kk] = lds_frag<DK>(kt, 16 + lr, 8 * lg + 32 * kk);
    }
    uint32_t vr[8][DV / 32];
#pragma unroll
    for (int r = 0; r < 8; ++r) lds_piece<DV>(vt, step_key(lg, r), lr, vr[r]);
    const f32x4_t a = qk_tile<DK>(kf0, qf), c = qk_tile<DK>(kf1, qf);
    float z[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x0 = k0 + 4 * lg + e, x1 = x0 + 16;
      z[e] = (x0 >= klo && x0 < khi) ? a[e] * sl2 : kNegInf;
      z[4 + e] = (x1 >= klo && x1 < khi) ? c[e] * sl2 : kNegInf;
    }
    float mx = z[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmaxf(mx, z[r]);
    mx = max_over_groups(mx);
    const float mn = fmaxf(m, mx);  // finite: the tile holds a valid key of this wave
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
  while (fin < 3) finalize(fin++);
  wait_vmem();

  // Pass 2: dq over the same tiles.
  f32x4_t dqa[DK / 16];
#pragma unroll
  for (int j = 0; j < DK / 16; ++j) dqa[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int i = ntile; i < nstep; ++i) {
    step_begin(i);
    int br, k0, wm, kend, klo, khi;
    desc(i, br, k0, wm, kend);
    key_range(br, k0, wm, kend, klo, khi);
    if (klo >= khi) continue;
    const char* kt = s_buf[i % kQtBuf];
    const char* vt = kt + 2 * SH::kK;
    const float ls = br == kCmp ? lse_c[0] : (br == kSlc ? lse_c[1] : lse_c[2]);
    const float dc = br == kCmp ? dc_c[0] : (br == kSlc ? dc_c[1] : dc_c[2]);
    const float gc = br == kCmp ? gt[0] : (br == kSlc ? gt[1] : gt[2]);
    u32x4_t kf0[DK / 32], kf1[DK / 32];
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) {
      kf0[kk] = lds_frag<DK>(kt, lr, 8 * lg + 32 * kk);
      kf1[kk] = lds_frag<DK>(kt, 16 + lr, 8 * lg + 32 * kk);
    }
    const f32x4_t a = qk_tile<DK>(kf0, qf), c = qk_tile<DK>(kf1, qf);
    u32x4_t vf0[DV / 32], vf1[DV / 32];
#pragma unroll
    for (int kk = 0; kk < DV / 32; ++kk) {
      vf0[kk] = lds_frag<DV>(vt, lr, 8 * lg + 32 * kk);
      vf1[kk] = lds_frag<DV>(vt, 16 + lr, 8 * lg + 32 * kk);
    }
    const f32x4_t pa = qk_tile<DV>(vf0, of), pc = qk_tile<DV>(vf1, of);
    float lo[4], hi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x0 = k0 + 4 * lg + e, x1 = x0 + 16;
      const float p0 = (x0 >= klo && x0 < khi) ? __builtin_amdgcn_exp2f(a[e] * sl2 - ls) : 0.f;
      const float p1 = (x1 >= klo && x1 < khi) ? __builtin_amdgcn_exp2f(c[e] * sl2 - ls) : 0.f;
      lo[e] = p0 * (gc * pa[e] - dc);
      hi[e] = p1 * (gc * pc[e] - dc);
    }
    uint32_t kr[8][DK / 32];
#pragma unroll
    for (int r = 0; r < 8; ++r) lds_piece<DK>(kt, step_key(lg, r), lr, kr[r]);
    pv_step<DK>(kr, pack_probs(lo, hi), dqa);
  }

  store_dq(dqa, dg_c);
}

// Gate-network gradients, partial sums over position range blockIdx.y of the
// B*T positions for query head blockIdx.x: thread ch < DK sums dz_c q[ch] for
// c = 0..2 (dw_gate), thread DK sums dz_c (db_gate); dz_c = dgates_c g_c (1 - g_c)
// with the gates kept in the statistics records.
template <int DK>
__global__ __launch_bounds__(256) void bwd_gate_part_kernel(BwdParams p) {
  static_assert(DK < 256, "one thread per channel plus one");
  const int h = blockIdx.x, ck = blockIdx.y, ch = threadIdx.x;
  const int g = h / p.G, hl = h - g * p.G;
  const int64_t P = (int64_t)p.B * p.T, per = (P + kGateChunks - 1) / kGateChunks;
  const int64_t r0 = ck * per, r1 = min(P, r0 + per);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f;
  for (int64_t pos = r0; pos < r1; ++pos) {
    const int64_t b = pos / p.T, t = pos - b * p.T;
    const float* dg = p.dgates + (pos * p.Hq + h) * 3;
    float dz[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const float gc = p.stat[((((int64_t)c * p.B + b) * p.T + t) * p.H + g) * kStatFloats + 32 + hl];
      dz[c] = dg[c] * gc * (1.f - gc);
    }
    const float x = ch < DK ? bf16_to_f32(p.q[(pos * p.Hq + h) * DK + ch]) : 1.f;
    a0 = fmaf(dz[0], x, a0);
    a1 = fmaf(dz[1], x, a1);
    a2 = fmaf(dz[2], x, a2);
  }
  if (ch <= DK) {
    float* dst = p.gpart + ((int64_t)ck * p.Hq + h) * 3 * (DK + 1);
    dst[ch] = a0;
    dst[(DK + 1) + ch] = a1;
    dst[2 * (DK + 1) + ch] = a2;
  }
}

// dw_gate, db_gate = sum of the partials in range order.
template <int DK>
__global__ __launch_bounds__(256) void bwd_gate_sum_kernel(BwdParams p) {
  const int64_t n = (int64_t)p.Hq * 3 * (DK + 1);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int ck = 0; ck < kGateChunks; ++ck) s += p.gpart[ck * n + i];
  const int64_t hc = i / (DK + 1);
  const int ch = (int)(i - hc * (DK + 1));
  if (ch < DK) p.dwgate[hc * DK + ch] = s;
  else if (p.dbgate) p.dbgate[hc] = s;
}

// ---------------------------------------------------------------------------
// Key side.  A workgroup owns 64 keys, a wave 16 of them (the MFMA columns,
// K and V fragments held in registers).  The queries that see those keys are
// taken two at a time: the 32 rows (query, head) of a pair form the contraction
// of dV^T += dout^T (g P) and dK^T += Q^T dS.  Each pair's Q rows, dout rows and
// statistics records are copied global -> LDS directly by all four waves,
// kKvBuf buffers deep (kKvBuf - 1 pairs in flight); within a row the 16-byte chunks are XOR-swizzled with the
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

// acc^T += rows^T . pb for 8 rows of an LDS block (the pv_step product), the row
// pieces read in 8-byte slices: slice u feeds the four MFMAs of output channels
// (D/16)*m + 4u .. 4u+3, so only 8 x 2 words are live at a time.
template <int D>
__device__ __forceinline__ void lds_rows_product(const char* blk, const int (&rows)[8], int lr, const u32x4_t& pb,
                                                 f32x4_t (&acc)[D / 16]) {
#pragma unroll
  for (int u = 0; u < D / 64; ++u) {
    uint32_t w[8][2];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const u32x2_t x = *reinterpret_cast<const u32x2_t*>(blk + sw_off<D>(rows[r], (D / 16) * lr + 4 * u));
      w[r][0] = x[0];
      w[r][1] = x[1];
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int wd = jj >> 1, h = jj & 1;
      const u32x4_t va = {pack_halves(w[0][wd], w[1][wd], h), pack_halves(w[2][wd], w[3][wd], h),
                          pack_halves(w[4][wd], w[5][wd], h), pack_halves(w[6][wd], w[7][wd], h)};
      acc[4 * u + jj] = mfma_bf16(va, pb, acc[4 * u + jj]);
    }
  }
}

template <int DK, int DV, int MODE>
__global__ __launch_bounds__(256, 2) void bwd_kv_kernel(BwdParams p) {
  using SH = KvShape<DK, DV>;
  __shared__ __attribute__((aligned(1024))) char s_buf[kKvBuf][SH::kBuf];
  __shared__ int32_t s_list[MODE == kSlc ? kSlcSplit : 1];
  __shared__ int s_scan[4];
  __shared__ int s_kt;
  const uint32_t lds0 = lds_addr_of(&s_buf[0][0]);

  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nbg = p.B * p.H;
  int kt, bg, split = 0;
  if constexpr (MODE == kSlc) {
    // Slot blockIdx.x of sequence-group blockIdx.y: key tile kt with
    // off[kt] <= slot < off[kt + 1], its split slot - off[kt].
    bg = (int)blockIdx.y;
    const int32_t* off = p.slc_off + (int64_t)bg * (p.kraw + 1);
    const int slot = (int)blockIdx.x;
    if (slot >= off[p.kraw]) return;
    if (tid == 0) {
      int lo = 0, hi = p.kraw;  // off[lo] <= slot < off[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= slot) lo = mid; else hi = mid;
      }
      s_kt = lo;
    }
    __syncthreads();
    kt = s_kt;
    split = slot - off[kt];
  } else {
    const int bid = (int)blockIdx.x;
    kt = bid / nbg;
    bg = bid - kt * nbg;
  }
  const int b = bg / p.H, g = bg - (bg / p.H) * p.H;
  const int kw0 = kt * 64;  // the workgroup's first key
  const int nkeys = MODE == kCmp ? p.nc : p.T;
  if (kw0 >= nkeys) return;
  const int T = p.T, G = p.G, Hq = p.Hq;
  const int k0 = kw0 + 16 * wave;
  const int key = k0 + lr;
  const int64_t bgl = (int64_t)b * p.H + g;

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

  // This lane's copy offsets within a pair (bytes from the first position's
  // rows; bit 31: the row belongs to the second position).  LDS chunk pch of a
  // block holds row r = pch / (D/8), slot sl, i.e. global chunk sl ^ (r & 7).
  uint32_t offq[SH::kCpQ], offo[SH::kCpO], offs;
#pragma unroll
  for (int j = 0; j < SH::kCpQ; ++j) {
    const int pch = (wave * SH::kCpQ + j) * 64 + lane;
    const int r = pch / (DK / 8), sl = pch - r * (DK / 8), h = min(r & 15, G - 1);
    offq[j] = (uint32_t)((((g * G + h) * DK) + 8 * (sl ^ (r & 7))) * 2) | (r >= 16 ? 0x80000000u : 0u);
  }
#pragma unroll
  for (int j = 0; j < SH::kCpO; ++j) {
    const int pch = (wave * SH::kCpO + j) * 64 + lane;
    const int r = pch / (DV / 8), sl = pch - r * (DV / 8), h = min(r & 15, G - 1);
    offo[j] = (uint32_t)((((g * G + h) * DV) + 8 * (sl ^ (r & 7))) * 2) | (r >= 16 ? 0x80000000u : 0u);
  }
  {
    const int ch = wave * 6 + min(lane, 5), x = ch / 12, cc = ch - x * 12;
    offs = (uint32_t)(16 * cc) | (x ? 0x80000000u : 0u);
  }

  // The workgroup's positions come in segments (one for the window and the
  // compressed branch; one per 128-word slice of the bitmap for the selected).
  {
    int tlo = 0, npos = 0;
    if constexpr (MODE == kWin) {
      tlo = kw0;
      npos = min(T - 1, kw0 + 63 + p.w - 1) - tlo + 1;
    } else if constexpr (MODE == kCmp) {
      tlo = kw0 * p.d + p.l - 1 + (int)blockIdx.y * p.qchunk;
      npos = max(0, min(T - 1, tlo + p.qchunk - 1) - tlo + 1);
    } else {
      // This split's positions: ranks [split * kSlcSplit, (split + 1) * kSlcSplit)
      // among the positions that chose one of the workgroup's blocks, in order;
      // bit 24 + w of an entry: wave w's block was chosen.
      int jw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) jw[w] = (kw0 + 16 * w) / p.lsel;
      const int wfirst = (jw[0] * p.lsel) >> 5;  // no earlier position can choose these blocks
      const int nw = p.nwords - wfirst, per = (nw + 255) / 256;
      const int w0 = wfirst + tid * per, w1 = min(p.nwords, w0 + per);
      const uint32_t* rows = p.bits + bgl * p.nblk * p.nwords;
      auto word = [&](int wi, uint32_t (&m)[4]) {
#pragma unroll
        for (int w = 0; w < 4; ++w) m[w] = jw[w] < p.nblk ? rows[(int64_t)jw[w] * p.nwords + wi] : 0u;
        return m[0] | m[1] | m[2] | m[3];
      };
      int cnt = 0;
      for (int wi = w0; wi < w1; ++wi) {
        uint32_t m[4];
        cnt += __builtin_popcount(word(wi, m));
      }
      int total;
      int rank = block_scan<256>(cnt, s_scan, &total);
      const int lo = split * kSlcSplit;
      npos = min(kSlcSplit, total - lo);
      if (rank < lo + kSlcSplit && rank + cnt > lo) {
        for (int wi = w0; wi < w1; ++wi) {
          uint32_t m[4];
          uint32_t x = word(wi, m);
          while (x) {
            const int bit = __builtin_ctz(x);
            x &= x - 1;
            if (rank >= lo && rank < lo + kSlcSplit) {
              int mask = 0;
#pragma unroll
              for (int w = 0; w < 4; ++w) mask |= (int)((m[w] >> bit) & 1u) << w;
              s_list[rank - lo] = (32 * wi + bit) | (mask << 24);
            }
            ++rank;
          }
        }
      }
      __syncthreads();
    }
    const int npair = (max(npos, 0) + 1) / 2;

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

    // Copies of pair i into buffer i % kKvBuf (the same number of instructions in
    // every wave): from the first position's rows plus this lane's offset, which
    // adds the distance to the second position's rows when its flag bit is set.
    auto issue = [&](int i) {
      int tA, mA, tB, mB;
      entry(2 * i, tA, mA);
      entry(2 * i + 1, tB, mB);
      if (tB < 0) tB = tA;  // a duplicate, masked out in the compute
      const uint32_t buf = lds0 + (uint32_t)((i % kKvBuf) * SH::kBuf);
      const uint16_t* qA = p.q + ((int64_t)b * T + tA) * Hq * DK;
      const uint16_t* oA = p.dout + ((int64_t)b * T + tA) * Hq * DV;
      const uint32_t dq = (uint32_t)(tB - tA) * (uint32_t)(Hq * DK * 2);
      const uint32_t dov = (uint32_t)(tB - tA) * (uint32_t)(Hq * DV * 2);
#pragma unroll
      for (int j = 0; j < SH::kCpQ; ++j)
        copy16_sb_at(qA, (offq[j] & 0x7FFFFFFFu) + ((offq[j] >> 31) ? dq : 0u), buf + (wave * SH::kCpQ + j) * 1024);
#pragma unroll
      for (int j = 0; j < SH::kCpO; ++j)
        copy16_sb_at(oA, (offo[j] & 0x7FFFFFFFu) + ((offo[j] >> 31) ? dov : 0u),
                     buf + 2 * SH::kQ + (wave * SH::kCpO + j) * 1024);
      if (lane < 6) {  // statistics: 2 records x 12 chunks, 6 lanes per wave
        const float* sA = p.stat + ((((int64_t)MODE * p.B + b) * T + tA) * p.H + g) * kStatFloats;
        const uint32_t ds = (uint32_t)(tB - tA) * (uint32_t)(p.H * kStatFloats * 4);
        copy16_sb_at(sA, (offs & 0x7FFFFFFFu) + ((offs >> 31) ? ds : 0u), buf + 2 * SH::kQ + 2 * SH::kO + wave * 96);
      }
    };

    for (int i = 0; i < kKvBuf - 1 && i < npair; ++i) issue(i);
    for (int i = 0; i < npair; ++i) {
      wait_steps<SH::kCopies, kKvBuf - 2>(min(npair - 1 - i, kKvBuf - 2));
      lds_barrier();
      if (i + kKvBuf - 1 < npair) issue(i + kKvBuf - 1);
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
        const f32x4_t sc = qk_tile<DK>(qa, kf);  // S[head 4lg+i][key lr]
        const f32x4_t dp = qk_tile<DV>(oa, vf);  // dout . v
        const f32x4_t lse = *reinterpret_cast<const f32x4_t*>(bs + X * kStatFloats + 4 * lg);
        const f32x4_t dc = *reinterpret_cast<const f32x4_t*>(bs + X * kStatFloats + 16 + 4 * lg);
        const f32x4_t gt = *reinterpret_cast<const f32x4_t*>(bs + X * kStatFloats + 32 + 4 * lg);
        const bool vis = t >= 0 && ((mask >> wave) & 1) && visible(t);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = vis && 4 * lg + e < G;
          const float pr = ok ? __builtin_amdgcn_exp2f(sc[e] * p.scale_log2 - lse[e]) : 0.f;
          pg[X][e] = pr * gt[e];
          ds[X][e] = pr * (gt[e] * dp[e] - dc[e]);
        }
      }
      int rows[8];
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8) rows[r8] = (r8 < 4 ? 0 : 16) + 4 * lg + (r8 & 3);
      lds_rows_product<DV>(bo, rows, lr, pack_probs(pg[0], pg[1]), dva);
      lds_rows_product<DK>(bq, rows, lr, pack_probs(ds[0], ds[1]), dka);
    }
  }

  if (key >= nkeys) return;
  // Window: the owner stores dk, dv.  Selected / compressed: this workgroup's
  // partial sums go to its slice of the workspace (zeros when it saw no
  // position), summed by bwd_kv_reduce_kernel in a fixed order.
  float* dk;
  float* dv;
  int stride;
  if constexpr (MODE == kWin) {
    dk = p.dk + (bgl * T + key) * DK;
    dv = p.dv + (bgl * T + key) * DV;
    stride = 1;
  } else {
    const int64_t row = MODE == kSlc
                            ? ((int64_t)bg * p.slots_max + blockIdx.x) * 64 + (key - kw0)
                            : (int64_t)blockIdx.y * nbg * p.nc + bgl * nkeys + key;
    float* base = (MODE == kSlc ? p.part_slc : p.part_cmp) + row * (DK + DV);
    dk = base;
    dv = base + DK;
    stride = 1;
  }
  (void)stride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j4 = 0; j4 < DK / 64; ++j4) {
      const int j = 4 * j4;
      *reinterpret_cast<f32x4_t*>(dk + (DK / 16) * (4 * lg + i) + j) =
          f32x4_t{dka[j][i], dka[j + 1][i], dka[j + 2][i], dka[j + 3][i]} * p.scale;
    }
#pragma unroll
    for (int j4 = 0; j4 < DV / 64; ++j4) {
      const int j = 4 * j4;
      *reinterpret_cast<f32x4_t*>(dv + (DV / 16) * (4 * lg + i) + j) =
          f32x4_t{dva[j][i], dva[j + 1][i], dva[j + 2][i], dva[j + 3][i]};
    }
  }
}

// Sum of the key-side partials in a fixed order: selected -> dk, dv += sum;
// compressed -> dk_cmp, dv_cmp = sum.  One thread per 4 channels of a key row.
template <int DK, int DV, int MODE>
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(BwdParams p) {
  constexpr int W = DK + DV;
  const int nbg = p.B * p.H;
  const int64_t nrow = (int64_t)nbg * (MODE == kSlc ? p.T : p.nc);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nrow * (W / 4)) return;
  const int64_t row = idx / (W / 4);
  const int c4 = (int)(idx - row * (W / 4)) * 4;
  f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (MODE == kSlc) {  // the key tile's split slots, in order
    const int64_t bgr = row / p.T;
    const int key = (int)(row - bgr * p.T), kt = key >> 6;
    const int32_t* off = p.slc_off + bgr * (p.kraw + 1);
    for (int sl = off[kt]; sl < off[kt + 1]; ++sl)
      s += *reinterpret_cast<const f32x4_t*>(p.part_slc + ((bgr * p.slots_max + sl) * 64 + (key & 63)) * W + c4);
  } else {
    const float* src = p.part_cmp + row * W + c4;
    for (int c = 0; c < p.ncq; ++c) s += *reinterpret_cast<const f32x4_t*>(src + (int64_t)c * nrow * W);
  }
  if constexpr (MODE == kSlc) {
    float* dst = c4 < DK ? p.dk + row * DK + c4 : p.dv + row * DV + (c4 - DK);
    *reinterpret_cast<f32x4_t*>(dst) += s;
  } else {
    float* dst = c4 < DK ? p.dkc + row * DK + c4 : p.dvc + row * DV + (c4 - DK);
    *reinterpret_cast<f32x4_t*>(dst) = s;
  }
}

// Selected branch, per (sequence-group, 64-key tile): the number of positions
// that chose one of the tile's blocks (the union of its bitmap rows).
__global__ __launch_bounds__(256) void bwd_slc_count_kernel(BwdParams p) {
  __shared__ int s_scan[4];
  const int nbg = p.B * p.H;
  const int bg = (int)blockIdx.x % nbg, kt = (int)blockIdx.x / nbg;
  const int kw0 = kt * 64;
  int jw[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) jw[w] = (kw0 + 16 * w) / p.lsel;
  const uint32_t* rows = p.bits + (int64_t)bg * p.nblk * p.nwords;
  int cnt = 0;
  for (int wi = ((jw[0] * p.lsel) >> 5) + (int)threadIdx.x; wi < p.nwords; wi += 256) {
    uint32_t u = 0u;
#pragma unroll
    for (int w = 0; w < 4; ++w) u |= jw[w] < p.nblk ? rows[(int64_t)jw[w] * p.nwords + wi] : 0u;  // as the list
    cnt += __builtin_popcount(u);
  }
  int total;
  block_scan<256>(cnt, s_scan, &total);
  if (threadIdx.x == 0) p.slc_cnt[(int64_t)bg * p.kraw + kt] = total;
}

// Per sequence-group: split slots of each key tile, ceil(count / kSlcSplit),
// as an exclusive prefix off[0 .. kraw] (off[kraw] = the slots used).
__global__ __launch_bounds__(256) void bwd_slc_scan_kernel(BwdParams p) {
  __shared__ int s_scan[4];
  const int bg = (int)blockIdx.x;
  const int32_t* cnt = p.slc_cnt + (int64_t)bg * p.kraw;
  int32_t* off = p.slc_off + (int64_t)bg * (p.kraw + 1);
  int base = 0;
  for (int k0 = 0; k0 < p.kraw; k0 += 256) {
    const int kt = k0 + (int)threadIdx.x;
    const int ns = kt < p.kraw ? (cnt[kt] + kSlcSplit - 1) / kSlcSplit : 0;
    int tot;
    const int ex = block_scan<256>(ns, s_scan, &tot);
    if (kt < p.kraw) off[kt] = base + ex;
    base += tot;
  }
  if (threadIdx.x == 0) off[p.kraw] = base;
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
  const int64_t nsel = (int64_t)p.B * p.T * p.H * p.n;
  hipLaunchKernelGGL(bwd_bitmap_kernel, dim3((unsigned)((nsel + 255) / 256)), dim3(256), 0, s, p);
  if (ev) hipEventRecord(ev->ev[0], s);
  if (p.lse_in)
    hipLaunchKernelGGL((bwd_query_kernel<DK, DV, true>), dim3((unsigned)(nbg * p.nqt)), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_query_kernel<DK, DV, false>), dim3((unsigned)(nbg * p.nqt)), dim3(256), 0, s, p);
  if (p.wgate) {
    hipLaunchKernelGGL((bwd_gate_part_kernel<DK>), dim3((unsigned)p.Hq, kGateChunks), dim3(256), 0, s, p);
    const int64_t ng = (int64_t)p.Hq * 3 * (DK + 1);
    hipLaunchKernelGGL((bwd_gate_sum_kernel<DK>), dim3((unsigned)((ng + 255) / 256)), dim3(256), 0, s, p);
  }
  if (ev) hipEventRecord(ev->ev[1], s);
  const int kraw = (p.T + 63) / 64, kcmp = (p.nc + 63) / 64;
  constexpr int W4 = (DK + DV) / 4;
  hipLaunchKernelGGL((bwd_kv_kernel<DK, DV, kWin>), dim3((unsigned)(nbg * kraw)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(bwd_slc_count_kernel, dim3((unsigned)(nbg * kraw)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(bwd_slc_scan_kernel, dim3((unsigned)nbg), dim3(256), 0, s, p);
  hipLaunchKernelGGL((bwd_kv_kernel<DK, DV, kSlc>), dim3((unsigned)p.slots_max, (unsigned)nbg), dim3(256), 0, s, p);
  const int64_t rraw = (int64_t)nbg * p.T * W4;
  hipLaunchKernelGGL((bwd_kv_reduce_kernel<DK, DV, kSlc>), dim3((unsigned)((rraw + 255) / 256)), dim3(256), 0, s, p);
  if (ev) hipEventRecord(ev->ev[2], s);
  if (p.nc > 0) {
    hipLaunchKernelGGL((bwd_kv_kernel<DK, DV, kCmp>), dim3((unsigned)(nbg * kcmp), (unsigned)p.ncq), dim3(256), 0,
                       s, p);
    const int64_t rcmp = (int64_t)nbg * p.nc * W4;
    hipLaunchKernelGGL((bwd_kv_reduce_kernel<DK, DV, kCmp>), dim3((unsigned)((rcmp + 255) / 256)), dim3(256), 0, s,
                       p);
  }
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

// Streaming compression for decode on gfx950: after a step has written token
// t = seq_lens[b] - 1 into the cache, every sequence whose t is the last token
// of a compression block (t = i*d + l - 1) gets block i's compressed key and
// value, for all of its KV heads:
//
//   y_i = flatten(X[i*d : i*d+l] + PE) . W,   W: [l*D, D], flatten token-major
//
// Source: lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc),
// section "NSA: три ветви", compressed-branch paragraph (blocks of l tokens with
// stride d, each folded into one key and one value by a learned MLP; about t/d
// of them exist at position t, so decode adds one every d tokens).  The MLP is
// read as in full compression: one bias-free linear layer plus a learned
// intra-block position embedding.
//
// The product has one row per (sequence, KV head) whose block is due, K = l*D
// and N = D.  Its bytes are almost all W, which every row shares, so the K
// dimension is split into chunks of 256 elements: workgroup (chunk, 64-channel
// slice) multiplies all rows of a 64-row tile by its 256 x 64 piece of W and of
// the position-embedding term, and writes an fp32 partial.  A second kernel
// adds the partials of each output in chunk order and rounds to bf16 (round to
// nearest even), so the result does not depend on timing and the call needs
// neither atomics nor zeroed memory.
#include <hip/hip_runtime.h>

#include "nsa_device.hpp"
#include "nsa_internal.hpp"

namespace nsa {

namespace {

struct DueRow {
  bool due;
  int64_t xrow;  // cache row of the block's first token
  int64_t crow;  // compressed-cache row that receives the block
};

// Row r = b * H + g of the product: is a block of (b, g) completed by the
// newest token, and where do its tokens and its summary live?
__device__ __forceinline__ DueRow due_row(const AppendParams& p, int r) {
  DueRow d{false, 0, 0};
  if (r >= p.B * p.H) return d;
  const int b = r / p.H, g = r - b * p.H;
  int64_t row0, cap_b;
  if (p.cu) {
    const int64_t a = p.cu[b], e = p.cu[b + 1];
    cap_b = e - a;
    row0 = (int64_t)p.H * a + (int64_t)g * cap_b;
  } else {
    cap_b = p.cap;
    row0 = ((int64_t)b * p.H + g) * p.cap;
  }
  const int64_t L = p.seq_lens[b];
  if (L < p.l || L > cap_b || (L - p.l) % p.d != 0) return d;
  const int64_t i = (L - p.l) / p.d;
  int64_t crow0, ccap_b;
  if (p.cuc) {
    const int64_t a = p.cuc[b], e = p.cuc[b + 1];
    ccap_b = e - a;
    crow0 = (int64_t)p.H * a + (int64_t)g * ccap_b;
  } else {
    ccap_b = p.ccap;
    crow0 = ((int64_t)b * p.H + g) * p.ccap;
  }
  if (i >= ccap_b) return d;
  d.due = true;
  d.xrow = row0 + i * p.d;
  d.crow = crow0 + i;
  return d;
}

// LDS of one partial workgroup: each wave's 64 x 64 product and its share of
// the position-embedding term, summed across waves in wave order.
struct AppendSmem {
  f32x4_t part[4][64][16];  // [wave][row][channel quad]
  float bias[4][64];        // [wave][channel]
};

// One 256-element chunk of K (eight 32-wide k-steps) for one 64-channel slice
// and one 64-row tile.  Wave w takes k-steps 2w and 2w+1 for all four 16-row
// MFMA tiles, so every wave reads a different quarter of the chunk's W.  Operand layouts follow the full compression kernel: lane (lg, lr) holds
// A row lr (eight k-slots of group lg) and four W channels c0 + 4*lr .. +3 of
// eight k-rows, transposed in registers into the B operands of four column
// tiles (tile j holds channel 4*lr + j).  The length lookups are issued first,
// then the W loads, then (once the due rows are known) the token loads, so the
// chunk costs about two memory round trips, the second overlapping W.  k-steps
// past the end of a short last chunk reload a valid step and multiply zeros.
template <int D>
__device__ __forceinline__ void append_chunk(const AppendParams& p, const uint16_t* x, const uint16_t* w,
                                             const uint16_t* pe, int kc, int c0, int col0, int rt,
                                             AppendSmem& sm) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int K = p.l * D;
  const int k_begin = kc * 256;
  const int nks = (K - k_begin) / 32 < 8 ? (K - k_begin) / 32 : 8;  // K is a multiple of 64: nks >= 2

  const DueRow mine = due_row(p, rt * 64 + lane);  // lane l: row l of the tile

  uint32_t wr[2][8][2];
  u32x4_t pv[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int s = 2 * wave + h;
    const int k0 = k_begin + 32 * (s < nks ? s : nks - 1);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const u32x2_t v = ld8(w + (size_t)(k0 + 8 * lg + r) * D + c0 + 4 * lr);
      wr[h][r][0] = v[0];
      wr[h][r][1] = v[1];
    }
    pv[h] = ld16(pe + k0 + 8 * lg);  // every A row of the position term equals the flattened PE
  }

  const uint64_t due_mask = __ballot(mine.due);  // the same in every wave
  if (due_mask == 0) {  // uniform over the workgroup (and over all chunks of the tile)
    wait_vmem();
    return;
  }
  // token loads: MFMA tile t, row 16t + lr; its cache row comes from lane 16t + lr
  u32x4_t a[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int src = 16 * t + lr;
    const int lo = __shfl((int)(uint32_t)(uint64_t)mine.xrow, src);
    const int hi = __shfl((int)(uint32_t)((uint64_t)mine.xrow >> 32), src);
    const int64_t xr = (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
    const bool due = (due_mask >> src) & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int s = 2 * wave + h;
      a[t][h] = due ? ld16(x + xr * D + k_begin + 32 * (s < nks ? s : nks - 1) + 8 * lg) : u32x4_t{0, 0, 0, 0};
    }
  }

  f32x4_t acc[4][4], accb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    accb[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bool live = 2 * wave + h < nks;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int wd = j >> 1, hh = j & 1;
      const u32x4_t bj{pack_halves(wr[h][0][wd], wr[h][1][wd], hh), pack_halves(wr[h][2][wd], wr[h][3][wd], hh),
                       pack_halves(wr[h][4][wd], wr[h][5][wd], hh), pack_halves(wr[h][6][wd], wr[h][7][wd], hh)};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if ((due_mask >> (16 * t)) & 0xFFFFull)  // tile with a due row (uniform)
          acc[t][j] = mfma_bf16(live ? a[t][h] : u32x4_t{0, 0, 0, 0}, bj, acc[t][j]);
      }
      accb[j] = mfma_bf16(live ? pv[h] : u32x4_t{0, 0, 0, 0}, bj, accb[j]);
    }
  }
  // D element i of tile t, column tile j: row 16t + 4*lg + i, channel 4*lr + j
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sm.part[wave][16 * t + 4 * lg + i][lr] = f32x4_t{acc[t][0][i], acc[t][1][i], acc[t][2][i], acc[t][3][i]};
  if (lg == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) sm.bias[wave][4 * lr + j] = accb[j][0];
  }
  __syncthreads();
  // thread -> (row, channel quad), four rows apart per pass
  const int q = tid & 15, row_base = tid >> 4;
  const int C = p.DK + p.DV;
  f32x4_t bias;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ch = 4 * q + j;
    bias[j] = ((sm.bias[0][ch] + sm.bias[1][ch]) + sm.bias[2][ch]) + sm.bias[3][ch];
  }
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int row = row_base + 16 * pass;
    if ((due_mask >> row) & 1) {
      const f32x4_t s0 = sm.part[0][row][q], s1 = sm.part[1][row][q], s2 = sm.part[2][row][q], s3 = sm.part[3][row][q];
      f32x4_t v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (((s0[j] + s1[j]) + s2[j]) + s3[j]) + bias[j];
      *reinterpret_cast<f32x4_t*>(p.part + ((size_t)kc * p.rows_pad + rt * 64 + row) * C + col0 + 4 * q) = v;
    }
  }
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void append_partial_kernel(AppendParams p) {
  __shared__ AppendSmem sm;
  const int x = blockIdx.x, rt = blockIdx.y;
  const int nk = (DK / 64) * p.nck_k;
  if (x < nk) {
    const int slice = x / p.nck_k, kc = x - slice * p.nck_k;
    append_chunk<DK>(p, p.k, p.wk, p.pek, kc, 64 * slice, 64 * slice, rt, sm);
  } else {
    const int y = x - nk;
    const int slice = y / p.nck_v, kc = y - slice * p.nck_v;
    append_chunk<DV>(p, p.v, p.wv, p.pev, kc, 64 * slice, DK + 64 * slice, rt, sm);
  }
}

// Eight threads per (row, 4 channels): thread e sums chunks e, e+8, e+16, ...
// (its loads all issued before the sums); the eight sums are then added in a
// fixed tree over lane offsets 4, 2, 1.  The result is rounded and stored.
template <int DK, int DV>
__global__ __launch_bounds__(256) void append_reduce_kernel(AppendParams p) {
  constexpr int C = DK + DV, C4 = C / 4, MAXPER = 12;  // up to 96 chunks per output
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int e = gid & 7, idx = gid >> 3;
  const int r = idx / C4, c = (idx - r * C4) * 4;
  const bool in = r < p.B * p.H;
  const bool isk = c < DK;
  const int nck = isk ? p.nck_k : p.nck_v;
  const float* src = p.part + (size_t)(in ? r : 0) * C + c;
  const size_t stride = (size_t)p.rows_pad * C;
  f32x4_t v[MAXPER];
#pragma unroll
  for (int m = 0; m < MAXPER; ++m) {
    const int kc = e + 8 * m;
    v[m] = (in && kc < nck) ? *reinterpret_cast<const f32x4_t*>(src + kc * stride) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const DueRow dr = due_row(p, in ? r : p.B * p.H);
  f32x4_t s = v[0];
#pragma unroll
  for (int m = 1; m < MAXPER; ++m) s = f32x4_t{s[0] + v[m][0], s[1] + v[m][1], s[2] + v[m][2], s[3] + v[m][3]};
#pragma unroll
  for (int o = 4; o >= 1; o >>= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] += __shfl_xor(s[j], o);
  }
  if (!dr.due || e != 0) return;
  u32x2_t o;
  o[0] = pack_bf16x2(s[0], s[1]);
  o[1] = pack_bf16x2(s[2], s[3]);
  uint16_t* dst = isk ? p.kc + dr.crow * DK + c : p.vc + dr.crow * DV + (c - DK);
  *reinterpret_cast<u32x2_t*>(dst) = o;
}

template <int DK, int DV>
hipError_t launch_append_t(const AppendParams& p, hipStream_t s) {
  const dim3 g1((unsigned)((DK / 64) * p.nck_k + (DV / 64) * p.nck_v), (unsigned)(p.rows_pad / 64)), blk(256);
  hipLaunchKernelGGL((append_partial_kernel<DK, DV>), g1, blk, 0, s, p);
  const int64_t threads = (int64_t)p.B * p.H * ((DK + DV) / 4) * 8;
  const dim3 g2((unsigned)((threads + 255) / 256));
  hipLaunchKernelGGL((append_reduce_kernel<DK, DV>), g2, blk, 0, s, p);
  return hipGetLastError();
}

}  // namespace

int append_chunks(int l, int D) { return (l * D + 255) / 256; }

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  if (p.DK == 64 && p.DV == 64) return launch_append_t<64, 64>(p, s);
  if (p.DK == 128 && p.DV == 128) return launch_append_t<128, 128>(p, s);
  if (p.DK == 192 && p.DV == 128) return launch_append_t<192, 128>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace nsa

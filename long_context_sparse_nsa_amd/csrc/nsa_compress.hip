// Token-block compression on gfx950 (MFMA GEMM over overlapping blocks).
//
//   y_i = flatten(X[i*d : i*d+l] + PE) . W,   W: [l*D, D], flatten token-major
//
// Source: lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc),
// section "NSA: три ветви", compressed-branch paragraph (blocks of l tokens with
// stride d, each folded into one key and one value by a learned MLP); the MLP
// is read as one bias-free linear layer with a learned intra-block position
// embedding.
//
// Row i of the GEMM's A operand is the contiguous run X[i*d*D, i*d*D + l*D), so
// overlapping blocks need no copy: consecutive rows start d*D elements apart.
// By linearity y_i = X_i . W + PE . W; the second term is the same for every
// block and is computed with the same MFMAs (an A tile whose rows all equal the
// flattened PE), split over the 4 waves by k-step and summed in fixed order.
// Every product is bf16 x bf16 accumulated in fp32; the result is rounded to bf16.
#include <hip/hip_runtime.h>

#include "nsa_device.hpp"
#include "nsa_internal.hpp"

namespace nsa {

template <int D>
__global__ __launch_bounds__(256) void compress_kernel(CompressParams p) {
  __shared__ float s_bias[4][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int bgi = blockIdx.z;
  const int g = bgi % p.H, b = bgi / p.H;
  const int c0 = blockIdx.y * 64;

  int64_t row0, cap_b;
  if (p.cu) {
    const int64_t a = p.cu[b], e = p.cu[b + 1];
    cap_b = e - a;
    row0 = (int64_t)p.H * a + (int64_t)g * cap_b;
  } else {
    cap_b = p.cap;
    row0 = ((int64_t)b * p.H + g) * p.cap;
  }
  const int64_t L = p.seq_lens ? (int64_t)p.seq_lens[b] : cap_b;
  const int64_t nc = L >= p.l ? (L - p.l) / p.d + 1 : 0;
  int64_t crow0, ccap_b;
  if (p.cuc) {
    const int64_t a = p.cuc[b], e = p.cuc[b + 1];
    ccap_b = e - a;
    crow0 = (int64_t)p.H * a + (int64_t)g * ccap_b;
  } else {
    ccap_b = p.ccap;
    crow0 = ((int64_t)b * p.H + g) * p.ccap;
  }
  const int64_t nwrite = nc < ccap_b ? nc : ccap_b;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  if (i0 >= nwrite) return;  // whole workgroup idle (uniform)

  const int64_t irow = i0 + wave * 16 + lr;        // this lane's A row (block)
  const bool arow_ok = irow < nwrite;
  const uint16_t* xrow = p.x + (row0 + irow * p.d) * D + 8 * lg;
  const int K = p.l * D;

  f32x4_t acc[4], accb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = accb[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0, ks = 0; k0 < K; k0 += 32, ++ks) {
    u32x4_t a = arow_ok ? ld16(xrow + k0) : u32x4_t{0, 0, 0, 0};
    uint32_t wr[8][2];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const u32x2_t x = ld8(p.w + (size_t)(k0 + 8 * lg + r) * D + c0 + 4 * lr);
      wr[r][0] = x[0];
      wr[r][1] = x[1];
    }
    u32x4_t bj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int wd = j >> 1, h = j & 1;
      bj[j] = u32x4_t{pack_halves(wr[0][wd], wr[1][wd], h), pack_halves(wr[2][wd], wr[3][wd], h),
                      pack_halves(wr[4][wd], wr[5][wd], h), pack_halves(wr[6][wd], wr[7][wd], h)};
      acc[j] = mfma_bf16(a, bj[j], acc[j]);
    }
    if ((ks & 3) == wave) {
      const u32x4_t pe = ld16(p.pe + k0 + 8 * lg);
#pragma unroll
      for (int j = 0; j < 4; ++j) accb[j] = mfma_bf16(pe, bj[j], accb[j]);
    }
  }
  // bias: every row of the PE tile is identical; row 0 (lg == 0, i == 0) suffices
  if (lg == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) s_bias[wave][4 * lr + j] = accb[j][0];
  }
  __syncthreads();
  float bias[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ch = 4 * lr + j;
    bias[j] = ((s_bias[0][ch] + s_bias[1][ch]) + s_bias[2][ch]) + s_bias[3][ch];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t orow = i0 + wave * 16 + 4 * lg + i;
    if (orow < nwrite) {
      u32x2_t v;
      v[0] = pack_bf16x2(acc[0][i] + bias[0], acc[1][i] + bias[1]);
      v[1] = pack_bf16x2(acc[2][i] + bias[2], acc[3][i] + bias[3]);
      *reinterpret_cast<u32x2_t*>(p.y + (crow0 + orow) * D + c0 + 4 * lr) = v;
    }
  }
}

hipError_t launch_compress(const CompressParams& p, hipStream_t s) {
  if (p.max_nc <= 0) return hipSuccess;
  const dim3 grid((unsigned)((p.max_nc + 63) / 64), (unsigned)(p.D / 64), (unsigned)(p.B * p.H)), blk(256);
  switch (p.D) {
    case 64: hipLaunchKernelGGL(compress_kernel<64>, grid, blk, 0, s, p); break;
    case 128: hipLaunchKernelGGL(compress_kernel<128>, grid, blk, 0, s, p); break;
    case 192: hipLaunchKernelGGL(compress_kernel<192>, grid, blk, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nsa

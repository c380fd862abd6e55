// Backward of the token-block compression (training): given the gradient dY of
// the compressed rows, the gradients of the raw rows, the weight and the
// intra-block position encoding.
//
// Source: lesson 5.5/02 "Разреженное внимание — NSA и DSA", section "NSA: три
// ветви", compressed branch (a learnable MLP with an intra-block position
// encoding maps each block of l tokens to one key / value), and the "Native Sparse
// Attention (DeepSeek NSA)" lesson ("Build it" step 1): block i covers tokens
// [i*d, i*d + l) and Y_i = X_i W with X_i = (x[i*d : i*d+l] + PE) flattened.
//
// With that forward, summing over every sequence, head and block:
//   dX_i   = dY_i W^T
//   dx[t] += sum over the blocks i that cover t of dX_i[t - i*d]   (fused: no dX)
//   dW     = sum_i X_i^T dY_i = sum_i x-rows^T dY_i + PE (x) s,  s = sum_i dY_i
//   dPE    = sum_i dX_i = s W^T
// The two products run on bf16 MFMAs, dY entering as bf16 high + low parts (x and
// W are bf16 already), with fp32 accumulation.  All sums run in a fixed order (no
// atomics), so results are reproducible.
#include "nsa_train.hpp"
#include "nsa_device.hpp"

namespace nsa {
namespace {

// fp32 values to bf16 high and low parts: hi = bf16(v), lo = bf16(v - hi).  Two
// MFMAs against the same bf16 operand then give the fp32 product to about 2^-16
// relative, in fp32 accumulation.
__device__ __forceinline__ void split8(const f32x4_t& v0, const f32x4_t& v1, u32x4_t& hi, u32x4_t& lo) {
  const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    hi[e] = h;
    lo[e] = pack_bf16x2(v[2 * e] - bf16_lo(h), v[2 * e + 1] - bf16_hi(h));
  }
}

// dx = the compression's input gradient, accumulated into dx.  Token t = a*d + j
// (0 <= j < d) lies in the blocks a - u, u = 0 .. R-1 (R = l/d), at in-block row
// j + u*d, so for one j the tokens a*d + j are the rows of one product over
// (u, o):   dx[a*d + j][c] += sum_u sum_o dY[a - u][o] W[(j + u*d)*D + c][o].
// Workgroup: one (bh, j), 4 waves x 32 rows a, all D columns.  A = dY rows
// (high + low bf16 parts), B = rows of W, contiguous in o.
template <int D>
__global__ __launch_bounds__(256) void cbwd_dx_kernel(const float* dy, const uint16_t* w, float* dx, int64_t T, int d,
                                                      int R, int nc, int na) {
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63, lg = lane >> 4, lr = lane & 15, wave = threadIdx.x >> 6;
  const int j = blockIdx.y;
  const int64_t bh = blockIdx.z;
  const int a0 = blockIdx.x * 128 + wave * 32;
  const float* dyb = dy + bh * nc * D;
  f32x4_t acc[2][NT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int u = 0; u < R; ++u) {
    const uint16_t* wr = w + (int64_t)(j + u * d) * D * D;
    for (int o0 = 0; o0 < D; o0 += 32) {
      u32x4_t ahi[2], alo[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int i = a0 + 16 * rt + lr - u;  // this lane's row's block
        f32x4_t v0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, v1 = v0;
        if (i >= 0 && i < nc) {
          const f32x4_t* src = reinterpret_cast<const f32x4_t*>(dyb + (int64_t)i * D + o0 + 8 * lg);
          v0 = src[0];
          v1 = src[1];
        }
        split8(v0, v1, ahi[rt], alo[rt]);
      }
      u32x4_t bw[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) bw[ct] = ld16(wr + (int64_t)(16 * ct + lr) * D + o0 + 8 * lg);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          acc[rt][ct] = mfma_bf16(ahi[rt], bw[ct], acc[rt][ct]);
          acc[rt][ct] = mfma_bf16(alo[rt], bw[ct], acc[rt][ct]);
        }
    }
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = a0 + 16 * rt + 4 * lg + i;
      const int64_t t = (int64_t)a * d + j;
      if (a >= na || t >= T) continue;
      float* dst = dx + (bh * T + t) * D + lr;
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) dst[16 * ct] += acc[rt][ct][i];
    }
}

// dW without the position-encoding term, per in-block row r:
//   dW[r*D + c][o] = sum over (bh, i) of x[bh][i*d + r][c] dY[bh][i][o],
// a product whose contraction runs over rows of both operands.  Workgroup: one
// r and one of the split contraction ranges (blockIdx.y), written to its own
// partial.  Each 32-row chunk is staged in LDS transposed (channel-major, 40
// elements per channel row, so the 16-byte operand reads of 16 lanes hit
// distinct banks): x as bf16, dY as bf16 high and low parts.  Wave w owns
// channel tiles CT*w .. CT*w + CT-1 and every o tile.
constexpr int kXS = 40;  // LDS row stride of the transposed chunks (elements)
template <int D>
__global__ __launch_bounds__(256) void cbwd_dw_kernel(const uint16_t* x, const float* dy, float* part, int64_t T,
                                                      int d, int nc, int64_t K, int64_t kz) {
  constexpr int NO = D / 16, CT = NO / 4;
  constexpr int XC = 32 * D / 8 / 256, YC = 32 * D / 4 / 256;  // 16-byte chunks per thread
  static_assert(XC * 256 * 8 == 32 * D && YC * 256 * 4 == 32 * D, "chunks per thread");
  __shared__ __attribute__((aligned(16))) uint16_t xt[D * kXS];
  __shared__ __attribute__((aligned(16))) uint16_t yh[D * kXS];
  __shared__ __attribute__((aligned(16))) uint16_t yl[D * kXS];
  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, lr = lane & 15, wave = tid >> 6;
  const int r = blockIdx.x;
  const int64_t kb = (int64_t)blockIdx.y * kz, ke = std::min<int64_t>(K, kb + kz);
  u32x4_t xr[XC];
  f32x4_t yr[YC];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int q = 0; q < XC; ++q) {
      const int e = tid + 256 * q, kk = e / (D / 8), cc = (e - kk * (D / 8)) * 8;
      const int64_t k = k0 + kk;
      xr[q] = u32x4_t{0u, 0u, 0u, 0u};
      if (k < ke) {
        const int64_t bh = k / nc, i = k - bh * nc;
        xr[q] = ld16(x + (bh * T + i * d + r) * D + cc);
      }
    }
#pragma unroll
    for (int q = 0; q < YC; ++q) {
      const int e = tid + 256 * q, kk = e / (D / 4), oo = (e - kk * (D / 4)) * 4;
      const int64_t k = k0 + kk;
      yr[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (k < ke) yr[q] = *reinterpret_cast<const f32x4_t*>(dy + k * D + oo);
    }
  };
  f32x4_t acc[CT][NO];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int o = 0; o < NO; ++o) acc[c][o] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (kb < ke) load(kb);
  for (int64_t k0 = kb; k0 < ke; k0 += 32) {
    __syncthreads();  // the previous chunk's operand reads are done
#pragma unroll
    for (int q = 0; q < XC; ++q) {
      const int e = tid + 256 * q, kk = e / (D / 8), cc = (e - kk * (D / 8)) * 8;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        xt[(cc + 2 * m) * kXS + kk] = (uint16_t)(xr[q][m] & 0xFFFFu);
        xt[(cc + 2 * m + 1) * kXS + kk] = (uint16_t)(xr[q][m] >> 16);
      }
    }
#pragma unroll
    for (int q = 0; q < YC; ++q) {
      const int e = tid + 256 * q, kk = e / (D / 4), oo = (e - kk * (D / 4)) * 4;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float v = yr[q][m];
        const uint32_t h = f32_to_bf16(v);
        yh[(oo + m) * kXS + kk] = (uint16_t)h;
        yl[(oo + m) * kXS + kk] = (uint16_t)f32_to_bf16(v - __uint_as_float(h << 16));
      }
    }
    __syncthreads();
    if (k0 + 32 < ke) load(k0 + 32);  // next chunk in flight during the products
    u32x4_t af[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
      af[c] = *reinterpret_cast<const u32x4_t*>(xt + (16 * (CT * wave + c) + lr) * kXS + 8 * lg);
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      const u32x4_t yhi = *reinterpret_cast<const u32x4_t*>(yh + (16 * o + lr) * kXS + 8 * lg);
      const u32x4_t ylo = *reinterpret_cast<const u32x4_t*>(yl + (16 * o + lr) * kXS + 8 * lg);
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        acc[c][o] = mfma_bf16(af[c], yhi, acc[c][o]);
        acc[c][o] = mfma_bf16(af[c], ylo, acc[c][o]);
      }
    }
  }
  float* dst = part + (int64_t)blockIdx.y * ((int64_t)gridDim.x * D * D) + (int64_t)r * D * D;
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = 16 * (CT * wave + c) + 4 * lg + i;
#pragma unroll
      for (int o = 0; o < NO; ++o) dst[(int64_t)ch * D + 16 * o + lr] = acc[c][o][i];
    }
}

// dw = sum of the split-contraction partials, in order.
__global__ __launch_bounds__(256) void cbwd_sum_parts_kernel(const float* part, int nparts, int64_t n, float* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = part[i];
  for (int z = 1; z < nparts; ++z) s += part[(int64_t)z * n + i];
  out[i] = s;
}

// Column sums of dY [rows x D], stage 1: partial sums of row chunks.
constexpr int kSumChunks = 64;
__global__ __launch_bounds__(256) void cbwd_colsum_part_kernel(const float* dy, int64_t rows, int D, float* part) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= D) return;
  const int64_t per = (rows + kSumChunks - 1) / kSumChunks;
  const int64_t r0 = (int64_t)blockIdx.y * per, r1 = std::min<int64_t>(rows, r0 + per);
  float s = 0.f;
  for (int64_t r = r0; r < r1; ++r) s += dy[r * D + c];
  part[(int64_t)blockIdx.y * D + c] = s;
}

// Stage 2 and the position-encoding terms: s = sum of the partials, then per
// flattened row m = (j, c) of W:  dPE[m] = s . W[m],  dW[m][:] += PE[m] s.
__global__ __launch_bounds__(256) void cbwd_pe_kernel(const float* part, const uint16_t* w, const uint16_t* pe,
                                                      int lD, int D, float* dw, float* dpe) {
  __shared__ float s[256];
  for (int c = threadIdx.x; c < D; c += 256) {
    float x = 0.f;
    for (int r = 0; r < kSumChunks; ++r) x += part[(int64_t)r * D + c];
    s[c] = x;
  }
  __syncthreads();
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= lD) return;
  const float pm = bf16_to_f32(pe[m]);
  float acc = 0.f;
  for (int o = 0; o < D; ++o) {
    const float so = s[o];
    acc = fmaf(so, bf16_to_f32(w[(int64_t)m * D + o]), acc);
    dw[(int64_t)m * D + o] += pm * so;
  }
  dpe[m] = acc;
}

}  // namespace

template <int D>
static void launch_cbwd_t(const CompressBwdParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.BH * p.nc;
  if (rows > 0) {
    const int R = p.l / p.d, na = p.nc + R - 1;
    hipLaunchKernelGGL(cbwd_dx_kernel<D>, dim3((unsigned)((na + 127) / 128), (unsigned)p.d, (unsigned)p.BH), dim3(256),
                       0, s, p.dy, p.w, p.dx, p.T, p.d, R, p.nc, na);
  }
  // kCbwdSplit contraction ranges of whole 32-row chunks (an empty range writes zeros)
  const int64_t kz = std::max<int64_t>(32, ((rows + kCbwdSplit - 1) / kCbwdSplit + 31) / 32 * 32);
  hipLaunchKernelGGL(cbwd_dw_kernel<D>, dim3((unsigned)p.l, kCbwdSplit), dim3(256), 0, s, p.x, p.dy, p.dwpart, p.T,
                     p.d, p.nc > 0 ? p.nc : 1, rows, kz);
}

hipError_t launch_compress_bwd(const CompressBwdParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.BH * p.nc;
  const int lD = p.l * p.D;
  hipLaunchKernelGGL(cbwd_colsum_part_kernel, dim3((unsigned)((p.D + 255) / 256), kSumChunks), dim3(256), 0, s, p.dy,
                     rows, p.D, p.part);
  switch (p.D) {
    case 64: launch_cbwd_t<64>(p, s); break;
    case 128: launch_cbwd_t<128>(p, s); break;
    case 192: launch_cbwd_t<192>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  // dW = sum of the split partials, in order, then the position-encoding terms
  const int64_t nw = (int64_t)lD * p.D;
  hipLaunchKernelGGL(cbwd_sum_parts_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, p.dwpart,
                     kCbwdSplit, nw, p.dw);
  hipLaunchKernelGGL(cbwd_pe_kernel, dim3((unsigned)((lD + 255) / 256)), dim3(256), 0, s, p.part, p.w, p.pe, lD, p.D,
                     p.dw, p.dpe);
  return hipGetLastError();
}

}  // namespace nsa

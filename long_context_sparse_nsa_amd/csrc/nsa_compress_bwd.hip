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
//   dX_i   = dY_i W^T                                (one fp32 GEMM)
//   dx[t] += sum over the blocks i that cover t of dX_i[t - i*d]
//   dW     = sum_i X_i^T dY_i = sum_i x-rows^T dY_i + PE (x) s,  s = sum_i dY_i
//   dPE    = sum_i dX_i = s W^T
// All sums run in fp32 in a fixed order (no atomics), so results are reproducible.
#include "nsa_train.hpp"
#include "nsa_device.hpp"

namespace nsa {
namespace {

constexpr int kGT = 64;  // output tile edge
constexpr int kGK = 16;  // contraction chunk

// Operand views for the two GEMMs.  at(m, k) / at(k, n) give an element; kContig
// says whether consecutive k are adjacent in memory (it picks the load order).
struct DyRowsA {  // A(m = (bh, i), k = o) = dY[m][o]
  const float* p;
  int D;
  static constexpr bool kContig = true;
  __device__ float at(int64_t m, int64_t k) const { return p[m * D + k]; }
};
struct WRowsB {  // B(k = o, n = (j, c)) = W[(j, c)][o]
  const uint16_t* p;
  int D;
  static constexpr bool kContig = true;
  __device__ float at(int64_t k, int64_t n) const { return bf16_to_f32(p[n * D + k]); }
};
struct XBlocksA {  // A(m = (j, c), k = (bh, i)) = x[bh][i*d + j][c]
  const uint16_t* p;
  int64_t T;
  int D, d, nc;
  static constexpr bool kContig = false;
  __device__ float at(int64_t m, int64_t k) const {
    const int64_t bh = k / nc, i = k - bh * nc;
    return bf16_to_f32(p[(bh * T + i * d) * D + m]);
  }
};
struct DyColsB {  // B(k = (bh, i), n = o) = dY[k][o]
  const float* p;
  int D;
  static constexpr bool kContig = false;
  __device__ float at(int64_t k, int64_t n) const { return p[k * D + n]; }
};

// C[M x N] = A . B (fp32), 64 x 64 tiles, 4 x 4 outputs per thread.  With
// gridDim.z > 1 each z takes the contraction range [z*kz, (z+1)*kz) and writes
// its partial product to C + z*cz.
template <class OA, class OB>
__global__ __launch_bounds__(256) void cbwd_gemm_kernel(int64_t M, int64_t N, int64_t K, OA a, OB bm, float* C,
                                                        int64_t ldc, int64_t kz, int64_t cz) {
  __shared__ float As[kGK][kGT + 4];
  __shared__ float Bs[kGK][kGT + 4];
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * kGT, n0 = (int64_t)blockIdx.x * kGT;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t kb = (int64_t)blockIdx.z * kz, ke = std::min<int64_t>(K, kb + kz);
  C += (int64_t)blockIdx.z * cz;
  float acc[4][4] = {};
  for (int64_t k0 = kb; k0 < ke; k0 += kGK) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int mm, kk;
      if (OA::kContig) { mm = tid >> 2; kk = (tid & 3) * 4 + r; } else { mm = tid & 63; kk = (tid >> 6) + 4 * r; }
      const int64_t m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < M && k < ke) ? a.at(m, k) : 0.f;
      int nn, kb2;
      if (OB::kContig) { nn = tid >> 2; kb2 = (tid & 3) * 4 + r; } else { nn = tid & 63; kb2 = (tid >> 6) + 4 * r; }
      const int64_t n = n0 + nn, k2 = k0 + kb2;
      Bs[kb2][nn] = (n < N && k2 < ke) ? bm.at(k2, n) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        av[u] = As[kk][ty * 4 + u];
        bv[u] = Bs[kk][tx * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(av[u], bv[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t m = m0 + ty * 4 + u;
    if (m >= M) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t n = n0 + tx * 4 + v;
      if (n < N) C[m * ldc + n] = acc[u][v];
    }
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

// dx[bh][t][c] += sum over covering blocks i of dX[bh*nc + i][(t - i*d)*D + c].
__global__ __launch_bounds__(256) void cbwd_fold_kernel(const float* dX, float* dx, int64_t BH, int64_t T, int D,
                                                        int l, int d, int nc) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= BH * T * D) return;
  const int c = (int)(idx % D);
  const int64_t r = idx / D;
  const int t = (int)(r % T);
  const int64_t bh = r / T;
  const int ilo = t >= l ? (t - l) / d + 1 : 0;  // first block with i*d + l > t
  const int ihi = std::min(nc - 1, t / d);
  float s = 0.f;
  for (int i = ilo; i <= ihi; ++i) s += dX[(bh * nc + i) * (int64_t)l * D + (int64_t)(t - i * d) * D + c];
  dx[idx] += s;
}

}  // namespace

hipError_t launch_compress_bwd(const CompressBwdParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.BH * p.nc;
  const int lD = p.l * p.D;
  if (rows > 0) {
    hipLaunchKernelGGL(cbwd_colsum_part_kernel, dim3((unsigned)((p.D + 255) / 256), kSumChunks), dim3(256), 0, s,
                       p.dy, rows, p.D, p.part);
    // dX = dY W^T  [rows x lD]
    hipLaunchKernelGGL((cbwd_gemm_kernel<DyRowsA, WRowsB>),
                       dim3((unsigned)((lD + kGT - 1) / kGT), (unsigned)((rows + kGT - 1) / kGT)), dim3(256), 0, s,
                       rows, (int64_t)lD, (int64_t)p.D, DyRowsA{p.dy, p.D}, WRowsB{p.w, p.D}, p.dX, (int64_t)lD,
                       (int64_t)p.D, (int64_t)0);
    const int64_t nfold = (int64_t)p.BH * p.T * p.D;
    hipLaunchKernelGGL(cbwd_fold_kernel, dim3((unsigned)((nfold + 255) / 256)), dim3(256), 0, s, p.dX, p.dx,
                       (int64_t)p.BH, p.T, p.D, p.l, p.d, p.nc);
  } else {
    hipLaunchKernelGGL(cbwd_colsum_part_kernel, dim3((unsigned)((p.D + 255) / 256), kSumChunks), dim3(256), 0, s,
                       p.dy, (int64_t)0, p.D, p.part);
  }
  // dW = sum x-rows^T dY  [lD x D]  (zero when there is no block): kCbwdSplit
  // contraction ranges of whole 16-row chunks, then their sum in order.
  const int64_t kz = ((rows + kCbwdSplit - 1) / kCbwdSplit + kGK - 1) / kGK * kGK;
  const int64_t nw = (int64_t)lD * p.D;
  hipLaunchKernelGGL((cbwd_gemm_kernel<XBlocksA, DyColsB>),
                     dim3((unsigned)((p.D + kGT - 1) / kGT), (unsigned)((lD + kGT - 1) / kGT), kCbwdSplit), dim3(256),
                     0, s, (int64_t)lD, (int64_t)p.D, rows, XBlocksA{p.x, p.T, p.D, p.d, p.nc > 0 ? p.nc : 1},
                     DyColsB{p.dy, p.D}, p.dwpart, (int64_t)p.D, kz > 0 ? kz : (int64_t)kGK, nw);
  hipLaunchKernelGGL(cbwd_sum_parts_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, p.dwpart,
                     kCbwdSplit, nw, p.dw);
  hipLaunchKernelGGL(cbwd_pe_kernel, dim3((unsigned)((lD + 255) / 256)), dim3(256), 0, s, p.part, p.w, p.pe, lD, p.D,
                     p.dw, p.dpe);
  return hipGetLastError();
}

}  // namespace nsa

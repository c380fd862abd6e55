// Wave-level attention tiles for one KV group: the G (<= 16) query heads of the
// group form the 16 columns of every MFMA, keys form the rows.
//
//   S^T tile  = K[16 keys x d_k] . q^T[d_k x 16 heads]     (A = keys, B = queries)
//   O^T      += V^T[d_v x 32 keys] . P^T[32 keys x 16 heads] (A = values, B = probs)
//
// In the S^T result lane (lg, lr) holds keys 4*lg + i (i = 0..3) of the tile for
// head lr.  Two consecutive S^T tiles (keys 0..15 and 16..31 of a 32-key step)
// therefore give lane (lg, lr) the eight keys {4lg+i, 16+4lg+i}; these are the
// lane's eight k-slots of the P^T operand, and the V^T operand is built with the
// same key order.  V rows are loaded as contiguous d_v/16-element pieces (lane lr
// reads channels (d_v/16)*lr ...) and transposed in registers, so MFMA number j
// of a step covers output channels (d_v/16)*m + j, m = 0..15.  All per-head
// softmax bookkeeping is then lane-local plus a reduction over the 4 lane groups.
#pragma once
#include "nsa_device.hpp"

namespace nsa {

// q fragments of the group's heads (B operand of S^T).  qg points at the first
// head of the group; rows are DK apart.  Heads >= G read as zero.
template <int DK>
__device__ __forceinline__ void load_q_frags(const uint16_t* qg, int G, int lg, int lr, u32x4_t (&qf)[DK / 32]) {
#pragma unroll
  for (int kk = 0; kk < DK / 32; ++kk) qf[kk] = u32x4_t{0, 0, 0, 0};
  if (lr < G) {
    const uint16_t* qp = qg + (size_t)lr * DK + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) qf[kk] = ld16(qp + 32 * kk);
  }
}

// A-operand fragments of one 16-key tile: this lane's key row is `key`
// (valid iff 0 <= key < nvalid); kbase points at key row 0.
template <int DK>
__device__ __forceinline__ void load_k_tile(const uint16_t* kbase, int64_t key, int64_t nvalid, int lg,
                                            u32x4_t (&kf)[DK / 32]) {
  if (key >= 0 && key < nvalid) {
    const uint16_t* kp = kbase + key * DK + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) kf[kk] = ld16(kp + 32 * kk);
  } else {
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) kf[kk] = u32x4_t{0, 0, 0, 0};
  }
}

template <int DK>
__device__ __forceinline__ f32x4_t qk_tile(const u32x4_t (&kf)[DK / 32], const u32x4_t (&qf)[DK / 32]) {
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < DK / 32; ++kk) s = mfma_bf16(kf[kk], qf[kk], s);
  return s;
}

// Key offset (within a 32-key step) of k-slot r of lane group lg.
__device__ __forceinline__ int step_key(int lg, int r) { return r < 4 ? 4 * lg + r : 16 + 4 * lg + (r - 4); }

// V rows of one 32-key step starting at key `k0` (rows valid iff < nvalid), the
// DV/16 channels starting at (DV/16)*lr of each row.
template <int DV>
__device__ __forceinline__ void load_v_step(const uint16_t* vbase, int64_t k0, int64_t nvalid, int lg, int lr,
                                            uint32_t (&vr)[8][DV / 32]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int64_t key = k0 + step_key(lg, r);
    if (key >= 0 && key < nvalid) {
      const uint16_t* vp = vbase + key * DV + (DV / 16) * lr;
      if constexpr (DV / 32 == 4) {
        u32x4_t x = ld16(vp);
        vr[r][0] = x[0]; vr[r][1] = x[1]; vr[r][2] = x[2]; vr[r][3] = x[3];
      } else {
        u32x2_t x = ld8(vp);
        vr[r][0] = x[0]; vr[r][1] = x[1];
      }
    } else {
#pragma unroll
      for (int q = 0; q < DV / 32; ++q) vr[r][q] = 0u;
    }
  }
}

// P^T operand from the probabilities of the two tiles of a step.
__device__ __forceinline__ u32x4_t pack_probs(const float (&a)[4], const float (&b)[4]) {
  return u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
}

// acc[j] element i = O^T[channel (DV/16)*(4*lg+i) + j][head lr].
template <int DV>
__device__ __forceinline__ void pv_step(const uint32_t (&vr)[8][DV / 32], const u32x4_t& pb, f32x4_t (&acc)[DV / 16]) {
#pragma unroll
  for (int j = 0; j < DV / 16; ++j) {
    const int wd = j >> 1, h = j & 1;
    u32x4_t va = {pack_halves(vr[0][wd], vr[1][wd], h), pack_halves(vr[2][wd], vr[3][wd], h),
                  pack_halves(vr[4][wd], vr[5][wd], h), pack_halves(vr[6][wd], vr[7][wd], h)};
    acc[j] = mfma_bf16(va, pb, acc[j]);
  }
}

// Channel held by acc[j][i] of lane group lg.
template <int DV>
__device__ __forceinline__ int acc_channel(int lg, int i, int j) { return (DV / 16) * (4 * lg + i) + j; }

}  // namespace nsa

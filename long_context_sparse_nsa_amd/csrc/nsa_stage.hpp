// Staging of K/V row tiles from HBM into LDS with the direct global->LDS copy,
// shared by the workgroups of the prefill and decode kernels, and the LDS
// operand reads that go with the staged layout.
//
// A tile is ROWS rows [row0, row0 + ROWS) of a row-major bf16 array; rows past
// rowmax are replaced by row rowmax (the caller masks their logits).  The NW
// waves of a workgroup share the copy (the wave index is wave-uniform) and
// each issues at least SO::kMinCopies copy instructions for K (+ V), so that
// waiting until at most that many copies are outstanding covers every earlier
// tile.
//
// K tile in fragment order: fragment f = m*KT + ks holds, at 16*lane, the eight
// dims 32*ks + 8*(lane/16) .. of row 16*m + lane%16 -- the A operand of the S^T
// MFMA, so a wave reads one contiguous KB per fragment.  V tile row-major
// (DV*2 bytes per row), copied in 1 KB pieces.  Wave w copies fragments
// w, w + NW, ... and pieces likewise; their per-lane byte offsets within the
// tile are fixed, so they are computed once.
#pragma once
#include "nsa_device.hpp"
#include "nsa_tiles.hpp"

namespace nsa {

template <int DK_, int DV_, int ROWS_, int NW_>
struct StageOffsets {
  static constexpr int DK = DK_, DV = DV_, ROWS = ROWS_, NW = NW_;
  static constexpr int KT = DK / 32, NF = (ROWS / 16) * KT, NI = ROWS * DV * 2 / 1024;
  static constexpr int FK = (NF + NW - 1) / NW, FV = (NI + NW - 1) / NW;
  static constexpr int kMinCopiesK = NF / NW, kMinCopiesKV = NF / NW + NI / NW;
  static constexpr int kKBytes = ROWS * DK * 2, kVBytes = ROWS * DV * 2;
  uint32_t k, v;  // lane parts of the byte offsets; the fragment/piece parts are uniform
  __device__ StageOffsets(int lane)
      : k((uint32_t)(((lane & 15) * DK + 8 * (lane >> 4)) * 2)), v((uint32_t)(lane * 16)) {}
};

template <class SO>
__device__ __forceinline__ void stage_k(const uint16_t* base, int64_t row0, int64_t rowmax, uint32_t dst, int wave,
                                        int lane, const SO& so) {
  constexpr int DK = SO::DK, KT = SO::KT, NF = SO::NF, NW = SO::NW, ROWS = SO::ROWS;
  if (row0 + ROWS - 1 <= rowmax) {  // wave-uniform: the whole tile lies inside the array
    const uint16_t* tile = base + row0 * DK;
#pragma unroll
    for (int ii = 0; ii < SO::FK; ++ii) {
      const int f = wave + NW * ii;
      if (NF % NW != 0 && f >= NF) break;
      const int m = f / KT, ks = f - m * KT;
      copy16_sb_at(tile + 16 * m * DK + 32 * ks, so.k, dst + f * 1024);
    }
  } else {
#pragma unroll
    for (int ii = 0; ii < SO::FK; ++ii) {
      const int f = wave + NW * ii;
      if (NF % NW != 0 && f >= NF) break;
      const int m = f / KT, ks = f - m * KT;
      int64_t row = row0 + 16 * m + (lane & 15);
      row = row < rowmax ? row : rowmax;
      copy16_to_lds_at(base + row * DK + 32 * ks + 8 * (lane >> 4), dst + f * 1024);
    }
  }
}

template <class SO>
__device__ __forceinline__ void stage_v(const uint16_t* base, int64_t row0, int64_t rowmax, uint32_t dst, int wave,
                                        int lane, const SO& so) {
  constexpr int NI = SO::NI, RB = SO::DV * 2, NW = SO::NW, ROWS = SO::ROWS;
  const char* bb = reinterpret_cast<const char*>(base);
  if (row0 + ROWS - 1 <= rowmax) {  // wave-uniform
    const char* tile = bb + row0 * RB;
#pragma unroll
    for (int ii = 0; ii < SO::FV; ++ii) {
      const int i = wave + NW * ii;
      if (NI % NW != 0 && i >= NI) break;
      copy16_sb_at(tile + i * 1024, so.v, dst + i * 1024);
    }
  } else {
#pragma unroll
    for (int ii = 0; ii < SO::FV; ++ii) {
      const int i = wave + NW * ii;
      if (NI % NW != 0 && i >= NI) break;
      const int off = i * 1024 + lane * 16;
      int64_t row = row0 + off / RB;
      row = row < rowmax ? row : rowmax;
      copy16_to_lds_at(bb + row * RB + (off % RB), dst + i * 1024);
    }
  }
}

// ---- LDS operand reads

template <int DK>
__device__ __forceinline__ u32x4_t lds_k(const char* kt, int m, int ks, int lane) {
  return *reinterpret_cast<const u32x4_t*>(kt + ((m * (DK / 32) + ks) * 64 + lane) * 16);
}

// The eight V rows of 32-key step ks that pair with this lane's P^T k-slots,
// channels (DV/16)*lr .. of each.
template <int DV>
__device__ __forceinline__ void lds_v_step(const char* vt, int ks, int lg, int lr, uint32_t (&vr)[8][DV / 32]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const char* src = vt + (32 * ks + step_key(lg, r)) * (DV * 2) + (DV / 16) * lr * 2;
    if constexpr (DV / 32 == 4) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(src);
      vr[r][0] = x[0]; vr[r][1] = x[1]; vr[r][2] = x[2]; vr[r][3] = x[3];
    } else {
      const u32x2_t x = *reinterpret_cast<const u32x2_t*>(src);
      vr[r][0] = x[0]; vr[r][1] = x[1];
    }
  }
}

// V^T operand j of a step (channels (DV/16)*m + j), from the rows read above.
template <int DV>
__device__ __forceinline__ u32x4_t v_operand(const uint32_t (&vr)[8][DV / 32], int j) {
  const int wd = j >> 1, h = j & 1;
  return u32x4_t{pack_halves(vr[0][wd], vr[1][wd], h), pack_halves(vr[2][wd], vr[3][wd], h),
                 pack_halves(vr[4][wd], vr[5][wd], h), pack_halves(vr[6][wd], vr[7][wd], h)};
}

}  // namespace nsa

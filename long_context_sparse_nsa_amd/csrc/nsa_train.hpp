// Parameters and launchers of the training kernels: the prefill backward and
// the compression backward.
#pragma once
#include "nsa_internal.hpp"

namespace nsa {

constexpr int kStatFloats = 48;      // statistics record of one (branch, position, group)
constexpr int kSlcSplit = 512;       // selected-branch key side: positions per workgroup
constexpr int kCbwdSplit = 8;
constexpr int kGateChunks = 64;      // gate-network gradients: position ranges summed in order        // compression backward: contraction ranges of the dW product

// Prefill backward (gradients of the three-branch output).
struct BwdParams {
  int B, T, Hq, H, G;
  int l, d, lsel, n, w;
  float scale, scale_log2;           // softmax scale and scale * log2(e)
  int nc;                            // compressed blocks per sequence
  int nqt;                           // query workgroups per (b, g): ceil(T / 4)
  int nblk, nwords;                  // selection blocks ceil(T / lsel); 32-position words ceil(T / 32)
  int qchunk, ncq;                   // compressed-branch key side: positions per workgroup, workgroups per tile
  const uint16_t* q;                 // [B, T, Hq, DK]
  const uint16_t* k;                 // [B, H, T, DK]
  const uint16_t* v;                 // [B, H, T, DV]
  const uint16_t* kc;                // [B, H, nc, DK]
  const uint16_t* vc;                // [B, H, nc, DV]
  const float* gates;                // [B, T, Hq, 3], or null with the gate network
  const float* lse_in;               // [B, T, Hq, 3] the forward's per-branch log-sum-exp, or null
  const uint16_t* wgate;             // gate network [Hq, 3, DK] (null: gates are given)
  const float* bgate;                // [Hq, 3] or null
  float* dwgate;                     // [Hq, 3, DK] (gate network only)
  float* dbgate;                     // [Hq, 3] or null
  float* gpart;                      // workspace [kGateChunks, Hq, 3, DK + 1]: gate-gradient partials
  const int32_t* sel;                // [B, T, H, n] the forward's selected block ids
  const uint16_t* dout;              // [B, T, Hq, DV]
  float* dq;                         // [B, T, Hq, DK]
  float* dk;                         // [B, H, T, DK]
  float* dv;                         // [B, H, T, DV]
  float* dkc;                        // [B, H, nc, DK]
  float* dvc;                        // [B, H, nc, DV]
  float* dgates;                     // [B, T, Hq, 3]
  float* stat;                       // workspace [3, B, T, H, kStatFloats]: per branch and group, the
                                     // heads' lse (log2 units) [16] | g_c (dO . o_c) [16] | g_c [16]
  uint32_t* bits;                    // workspace [B, H, nblk, nwords]: position t selected block j
  float* part_slc;                   // workspace [B*H, slots_max, 64, DK + DV]: selected-branch partials
  int kraw, slots_max;               // 64-key tiles per sequence; selected-branch split slots per (b, g)
  int32_t* slc_cnt;                  // workspace [B*H, kraw]: positions per key tile
  int32_t* slc_off;                  // workspace [B*H, kraw + 1]: first split slot per key tile
  float* part_cmp;                   // workspace [ncq, B, H, nc, DK + DV]: compressed-branch partials
};

// Compression backward of one compressed cache (keys or values).
struct CompressBwdParams {
  int BH, D, l, d, nc;
  int64_t T;
  const uint16_t* x;                 // raw rows [BH, T, D]
  const uint16_t* w;                 // [l*D, D]
  const uint16_t* pe;                // [l, D]
  const float* dy;                   // [BH, nc, D]
  float* dx;                         // [BH, T, D], accumulated
  float* dw;                         // [l*D, D]
  float* dpe;                        // [l, D]
  float* part;                       // workspace [64, D]
  float* dwpart;                     // workspace [kCbwdSplit, l*D, D]
};
hipError_t launch_compress_bwd(const CompressBwdParams& p, hipStream_t s);
hipError_t launch_prefill_bwd(const BwdParams& p, int DK, int DV, hipStream_t s, const PhaseEvents* ev);

}  // namespace nsa

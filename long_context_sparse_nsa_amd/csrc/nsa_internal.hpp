// Internal interface between the C ABI (nsa_api.cpp) and the kernel files.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace nsa {

// Compressed keys handled by one decode workgroup (4 waves x 64 keys).
constexpr int kChunk = 256;
// Limits of the on-chip tables (checked by the host before any launch).
constexpr int kMaxChunks = 128;      // chunks per sequence in decode  (Nc <= 32768)
constexpr int kMaxBlocks = 8192;     // selection candidates J+1
constexpr int kMaxSel = 64;          // n_sel
constexpr int kMaxUnion = 256;       // selected + window blocks per query
constexpr int kGPad = 16;            // query heads per group, padded to one MFMA tile

// Everything the decode kernels need; plain values and device pointers.
struct DecodeParams {
  int B, Hq, H, G;                   // batch, q heads, kv heads, heads per group
  int l, d, lsel, n, nloc, finit, w;
  float scale_log2;                  // softmax scale * log2(e)
  const uint16_t* q;                 // [B, Hq, DK]
  const uint16_t* k;                 // raw cache rows
  const uint16_t* v;
  const uint16_t* kc;                // compressed cache rows
  const uint16_t* vc;
  const int32_t* seq_lens;           // [B]
  const int64_t* cu;                 // [B+1] or null
  const int64_t* cuc;                // [B+1] or null
  int64_t cap;                       // uniform capacity when cu == null
  int64_t ccap;                      // uniform compressed capacity when cuc == null
  const float* gates;                // [B, Hq, 3]
  uint16_t* out;                     // [B, Hq, DV]
  int32_t* sel_out;                  // [B, H, n] or null
  // workspace
  uint32_t* cnt1;                    // [B*H]
  uint32_t* cnt2;                    // [B*H]
  float* m1;                         // [B*H, nch, 16]
  float* l1;                         // [B*H, nch, 16]
  float* o1;                         // [B*H, nch, 16, DV]
  float* sc1;                        // [B*H, nch, 16, nbo+1]
  float* ocmp;                       // [B*H, 16, DV] gated compressed-branch output
  int32_t* sel;                      // [B*H, n]
  float* part2;                      // [B*H, nw2, 2, 32 + 16*DV]
  int nch;                           // launch width of the compressed pass
  int nbo;                           // selection blocks owned by one chunk = kChunk*d/lsel
  int nw2;                           // launch width of the selected/window pass
};

struct DecodeLayout {
  size_t off_cnt1, off_cnt2, off_m1, off_l1, off_o1, off_sc1, off_ocmp, off_sel, off_part2, total;
  int nch, nbo, nw2;
};

// Parameters of the per-query prefill kernel and the compression kernel.
struct PrefillParams {
  int B, T, Hq, H, G;
  int l, d, lsel, n, nloc, finit, w;
  float scale_log2;
  int nc;                            // compressed blocks per sequence: floor((T-l)/d)+1
  const uint16_t* q;                 // [B, T, Hq, DK]
  const uint16_t* k;                 // [B, H, T, DK]
  const uint16_t* v;
  const uint16_t* kc;                // [B, H, nc, DK]
  const uint16_t* vc;
  const float* gates;                // [B, T, Hq, 3]
  uint16_t* out;                     // [B, T, Hq, DV]
  int32_t* sel_out;                  // [B, T, H, n] or null
};

struct CompressParams {
  int B, H, D, l, d;
  const uint16_t* x;                 // raw rows (layout as nsa_compress_kv)
  const int64_t* cu;                 // or null
  const int32_t* seq_lens;           // or null
  int64_t cap;                       // uniform capacity when cu == null
  const uint16_t* w;                 // [l*D, D]
  const uint16_t* pe;                // [l, D]
  uint16_t* y;                       // compressed rows
  const int64_t* cuc;                // or null
  int64_t ccap;                      // uniform compressed capacity when cuc == null
  int max_nc;                        // launch bound on blocks per sequence
};

DecodeLayout decode_layout(int B, int H, int DV, int l, int d, int lsel, int n, int w, int64_t max_len);

hipError_t launch_decode(const DecodeParams& p, int DK, int DV, hipStream_t s);
hipError_t launch_prefill(const PrefillParams& p, int DK, int DV, hipStream_t s);
hipError_t launch_compress(const CompressParams& p, hipStream_t s);

}  // namespace nsa

// Internal interface between the C ABI (nsa_api.cpp) and the kernel files.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace nsa {

// Decode streaming pass: workgroups of kStreamWaves waves stream kStreamTile-row tiles
// of one segment of the compressed cache (or of the window); the segment
// length is chosen so that one launch has about kStreamSlots workgroups (one
// per compute unit of an MI355X).
constexpr int kStreamWaves = 8;
constexpr int kStreamSlots = 256;
constexpr int kStreamTile = 16 * kStreamWaves;  // rows per streamed tile (16 per wave)
constexpr int kScStrideMax = 548;     // selection blocks per decode segment + 4, at most
// Limits of the on-chip tables (checked by the host before any launch).
constexpr int kMaxCompressed = 32768;                 // compressed blocks per sequence in decode
constexpr int kMaxChunks = 64;                        // compressed segments per sequence in decode
constexpr int kSegRows = 640;                         // compressed keys per decode segment, at most (fixed plan)
constexpr int kBalTiles = 8;                          // streamed tiles per segment, at most (balanced plan)
constexpr int kSegTiles = kBalTiles;                  // streamed tiles per segment, at most (LDS fold rows)
constexpr int kMaxBlocks = 8192;     // selection candidates J+1
constexpr int kMaxSel = 64;          // n_sel
constexpr int kMaxUnion = 256;       // selected + window blocks per query
constexpr int kGPad = 16;            // query heads per group, padded to one MFMA tile
constexpr int kMaxFinish = 16;       // decode selection workgroups per (sequence, group)
constexpr int kMaxWindow = 16;       // decode window workgroups per (sequence, group)

// Profiling hook: with a phase-clock buffer, thread 0 of every workgroup of the
// decode kernels (and of the DSA top-k and attention kernels) records the 100 MHz constant clock at kClkSlots numbered
// points; kernel k's workgroup w uses entries [(k*kClkMaxGroups + w)*kClkSlots, +kClkSlots).
constexpr int kClkSlots = 16;
constexpr int kClkMaxGroups = 4096;

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
  const float* gates;                // [B, Hq, 3], or null with the gate network below
  const uint16_t* wgate;             // gate network [Hq, 3, DK] (null: gates are given)
  const float* bgate;                // [Hq, 3] or null
  uint16_t* out;                     // [B, Hq, DV]
  int32_t* sel_out;                  // [B, H, n] or null
  // workspace (contents on entry are irrelevant)
  float* m1;                         // [segment slot, 16]: B*H*nch slots (fixed plan) or nslot (balanced)
  float* l1;                         // [segment slot, 16]
  float* o1;                         // [segment slot, 16, DV]
  float* sc1;                        // [segment slot, scs, 16] selection-block scores per head
  float* wpart;                      // [B*H, nwin, 32 + 16*DV] window-workgroup partials (m, l, o)
  float* rpart;                      // [B*H, nfin, 32 + 8*DV] selected partials (m, l fp32; o / l fp16)
  float* ocmp;                       // [B*H, 16, DV] normalised compressed-branch output
  uint32_t* cnt;                     // [B*H] selection-workgroup arrival counters
  uint64_t* clk;                     // phase clock (profiling) or null
  int nch;                           // compressed segments per (sequence, group)
  int seg;                           // compressed keys per segment (multiple of 64 and of lsel/d)
  int nbo;                           // selection blocks owned by one segment = seg*d/lsel
  int nfin;                          // selection workgroups per (sequence, group)
  int finw;                          // waves per selection workgroup (4 or 8)
  int wtiles;                        // 64-token window tiles per window workgroup
  int nwin;                          // window workgroups per (sequence, group)
  // Balanced plan (bal = 1; ragged batches whose fixed plan needs more than one
  // round of workgroups): the window workgroups come first, then nslot
  // compressed slots; the segments hold T tiles, T chosen on the device from
  // the actual lengths to fill about bal_fill slots, at least tmin; when T
  // would exceed tcap the device keeps the fixed plan (the launch and the
  // buffers are sized for either).
  int bal, nslot, bal_fill, tmin, tcap;
  int scs;                           // score slots per segment in sc1 (stride): nbo + 1, or the balanced maximum
};

struct DecodeLayout {
  size_t off_m1, off_l1, off_o1, off_sc1, off_wpart, off_rpart, off_ocmp, off_cnt, total;
  int nch, seg, nbo, nfin, nwin, wtiles, finw;
  int bal, nslot, bal_fill, tmin, tcap, scs;
};

// Parameters of the prefill kernels and the compression kernel.
constexpr int kPfMaxBlocks = 1024;   // prefill selection candidates per position (J+1)

struct PrefillParams {
  int B, T, Hq, H, G;
  int l, d, lsel, n, nloc, finit, w;
  float scale_log2;
  int nc;                            // compressed blocks per sequence: floor((T-l)/d)+1
  int ntile;                         // position tiles per sequence: ceil(T/16)
  const uint16_t* q;                 // [B, T, Hq, DK]
  const uint16_t* k;                 // [B, H, T, DK]
  const uint16_t* v;
  const uint16_t* kc;                // [B, H, nc, DK]
  const uint16_t* vc;
  const float* gates;                // [B, T, Hq, 3], or null with the gate network below
  const uint16_t* wgate;             // gate network [Hq, 3, DK] (null: gates are given)
  const float* bgate;                // [Hq, 3] or null
  uint16_t* out;                     // [B, T, Hq, DV]
  int32_t* sel;                      // [B, T, H, n] selected block ids (caller's or workspace)
  float* acc;                        // [B, T, Hq, DV] workspace: g_win o_win + g_cmp o_cmp
  float* lse;                        // [B, T, Hq, 3] per-branch log-sum-exp (natural log), or null
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

// Streaming compression (one new block per sequence and KV head when due).
struct AppendParams {
  int B, H, DK, DV, l, d;
  const uint16_t* k;                 // raw caches (layout as nsa_compress_kv)
  const uint16_t* v;
  const int64_t* cu;                 // or null
  const int32_t* seq_lens;           // current lengths (the newest token is seq_lens[b] - 1)
  int64_t cap;                       // uniform capacity when cu == null
  const uint16_t* wk;                // [l*DK, DK]
  const uint16_t* pek;               // [l, DK]
  const uint16_t* wv;                // [l*DV, DV]
  const uint16_t* pev;               // [l, DV]
  uint16_t* kc;                      // compressed caches
  uint16_t* vc;
  const int64_t* cuc;                // or null
  int64_t ccap;                      // uniform compressed capacity when cuc == null
  float* part;                       // fp32 partials [max(nck_k, nck_v)][rows_pad][DK + DV]
  int rows_pad;                      // B*H rounded up to a multiple of 64
  int nck_k, nck_v;                  // 256-element chunks of l*DK and l*DV
};
int append_chunks(int l, int D);
hipError_t launch_append(const AppendParams& p, hipStream_t s);

// DeepSeek Sparse Attention decode step (lightning indexer + token top-k +
// MQA attention over one shared latent per token).
constexpr int kDsaDqk = 576, kDsaDv = 512, kDsaMaxLen = 65536, kDsaMaxTopk = 4096;
constexpr int kDsaChunk = 4096;     // scores per top-k workgroup
constexpr int kDsaBins = 8192;      // radix digit histograms of the top-k: 13 bits
struct DsaParams {
  int B, H, HI, DI, topk;
  float scale_log2;
  int64_t cap;                       // tokens per sequence in the caches
  const uint16_t* q;                 // [B, H, 576] bf16
  const uint8_t* qi;                 // [B, HI, DI] fp8 e4m3
  const float* wi;                   // [B, HI]
  const uint16_t* c;                 // [B, cap, 576] bf16 latent cache
  const uint8_t* ki;                 // [B, cap, DI] fp8 e4m3 indexer keys
  const int32_t* seq_lens;           // [B]
  uint16_t* out;                     // [B, H, 512] bf16
  float* scores;                     // workspace [B, sstride]
  int64_t sstride;                   // cap rounded up to a multiple of 4
  int32_t* sel;                      // [B, topk] (caller's or workspace), ascending, -1 padded
  float* part;                       // workspace [B, H/hpg, ts, hpg, 264]: m, l, pad, 512 fp16 outputs / l
  int seg;                           // indexer tokens per workgroup (multiple of 512)
  int nseg;                          // indexer workgroups per sequence
  int ts;                            // attention token splits per (sequence, head group)
  int hpg;                           // heads per attention workgroup: 64, or 32 when H % 64 != 0
  int nchunk;                        // top-k workgroups per sequence: ceil(cap / kDsaChunk)
  uint32_t* cnt;                     // workspace [B, 4] arrival counters (zeroed by the indexer launch),
                                     // then [B, nchunk, 2] per-chunk counts
  uint32_t* bits;                    // workspace [B, nchunk * kDsaChunk / 32]: positions above the bound
  uint64_t* cand;                    // workspace [B, nchunk * kDsaChunk]: (key << 32 | position) candidates
  uint64_t* clk;                     // phase clock (null = off): top-k kernel, then attention kernel
};

DecodeLayout decode_layout(int B, int H, int DV, int l, int d, int lsel, int n, int nloc, int w, int64_t max_len);

// Optional events recorded between the kernels of one call (null = none).
struct PhaseEvents {
  hipEvent_t ev[4];
};

hipError_t launch_decode(const DecodeParams& p, int DK, int DV, hipStream_t s, const PhaseEvents* ev);

// The allocation-free decode entry point keeps its workspace in one fixed
// device array per GPU (nsa_noalloc.hip); noalloc_scratch returns its device
// address on the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_dsa_decode(const DsaParams& p, hipStream_t s, const PhaseEvents* ev);
// With events, ev[2] is recorded after the first prefill kernel and ev[3] after
// the second (the caller records ev[0] and ev[1] around the compression).
hipError_t launch_prefill(const PrefillParams& p, int DK, int DV, hipStream_t s, const PhaseEvents* ev);
hipError_t launch_compress(const CompressParams& p, hipStream_t s);

}  // namespace nsa

// C ABI of the NSA forward pass: argument validation (host only, before any
// HIP call), workspace planning and kernel launches on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include <hip/hip_runtime.h>

#include "nsa.h"
#include "nsa_train.hpp"

namespace {

thread_local std::string g_last_error;
thread_local nsa::PhaseEvents g_phase_events{};
thread_local bool g_phase_on = false;
thread_local uint64_t* g_clk = nullptr;
thread_local size_t g_clk_bytes = 0;

nsa_status_t fail(nsa_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
nsa_status_t fail(nsa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

nsa_status_t ok() {
  g_last_error.clear();
  return NSA_SUCCESS;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int64_t n_compressed(int64_t L, int l, int d) { return L >= l ? (L - l) / d + 1 : 0; }

// Checks shared by every entry point.
nsa_status_t check_common(const nsa_dims_t* dims, const nsa_config_t* cfg, bool need_cfg) {
  if (!dims) return fail(NSA_ERROR_INVALID_VALUE, "dims is NULL");
  if (need_cfg && !cfg) return fail(NSA_ERROR_INVALID_VALUE, "cfg is NULL");
  if (dims->batch < 1 || dims->num_q_heads < 1 || dims->num_kv_heads < 1 || dims->d_k < 1 || dims->d_v < 1)
    return fail(NSA_ERROR_INVALID_VALUE, "dims must be positive (batch=%d, q_heads=%d, kv_heads=%d, d_k=%d, d_v=%d)",
                dims->batch, dims->num_q_heads, dims->num_kv_heads, dims->d_k, dims->d_v);
  if (dims->num_q_heads % dims->num_kv_heads != 0)
    return fail(NSA_ERROR_INVALID_VALUE, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                dims->num_q_heads, dims->num_kv_heads);
  const int G = dims->num_q_heads / dims->num_kv_heads;
  if (G > nsa::kGPad) return fail(NSA_ERROR_UNSUPPORTED, "group size %d > 16 query heads per KV head", G);
  const int dk = dims->d_k, dv = dims->d_v;
  if (!((dk == 64 && dv == 64) || (dk == 128 && dv == 128) || (dk == 192 && dv == 128)))
    return fail(NSA_ERROR_UNSUPPORTED, "(d_k, d_v) = (%d, %d) not in {(64,64), (128,128), (192,128)}", dk, dv);
  if (!cfg) return NSA_SUCCESS;
  if (cfg->l < 1 || cfg->d < 1 || cfg->l_sel < 1 || cfg->n_sel < 1 || cfg->n_local < 0 ||
      (cfg->force_initial != 0 && cfg->force_initial != 1) || cfg->w < 1)
    return fail(NSA_ERROR_INVALID_VALUE,
                "bad NSA parameters (l=%d, d=%d, l_sel=%d, n_sel=%d, n_local=%d, force_initial=%d, w=%d)", cfg->l,
                cfg->d, cfg->l_sel, cfg->n_sel, cfg->n_local, cfg->force_initial, cfg->w);
  if (!(cfg->softmax_scale >= 0.f) || !std::isfinite(cfg->softmax_scale))
    return fail(NSA_ERROR_INVALID_VALUE, "softmax_scale must be finite and >= 0");
  if (cfg->l % cfg->d != 0 || cfg->l_sel % cfg->d != 0 || cfg->l > cfg->l_sel || !is_pow2(cfg->l_sel / cfg->d))
    return fail(NSA_ERROR_UNSUPPORTED, "need d | l, d | l_sel, l <= l_sel and l_sel/d a power of two (l=%d d=%d l_sel=%d)",
                cfg->l, cfg->d, cfg->l_sel);
  if (cfg->l_sel != 16 && cfg->l_sel != 32 && cfg->l_sel != 64 && cfg->l_sel != 128)
    return fail(NSA_ERROR_UNSUPPORTED, "l_sel=%d not in {16, 32, 64, 128}", cfg->l_sel);
  if (cfg->n_sel > nsa::kMaxSel) return fail(NSA_ERROR_UNSUPPORTED, "n_sel=%d > %d", cfg->n_sel, nsa::kMaxSel);
  if (cfg->n_local + cfg->force_initial > cfg->n_sel)
    return fail(NSA_ERROR_UNSUPPORTED, "n_local + force_initial (%d) > n_sel (%d)", cfg->n_local + cfg->force_initial,
                cfg->n_sel);
  if ((int64_t)cfg->n_sel + (cfg->w + cfg->l_sel - 1) / cfg->l_sel + 1 > nsa::kMaxUnion)
    return fail(NSA_ERROR_UNSUPPORTED, "n_sel + window blocks exceeds %d", nsa::kMaxUnion);
  return NSA_SUCCESS;
}

float scale_log2(const nsa_dims_t* dims, const nsa_config_t* cfg) {
  const float s = cfg->softmax_scale > 0.f ? cfg->softmax_scale : 1.0f / std::sqrt((float)dims->d_k);
  return s * 1.4426950408889634f;
}

nsa_status_t check_decode_sizes(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t max_seq_len) {
  if (max_seq_len < 1) return fail(NSA_ERROR_INVALID_VALUE, "max_seq_len must be >= 1");
  if ((max_seq_len - 1) / cfg->l_sel + 1 > nsa::kMaxBlocks)
    return fail(NSA_ERROR_UNSUPPORTED, "max_seq_len %lld gives more than %d selection blocks", (long long)max_seq_len,
                nsa::kMaxBlocks);
  const int64_t nc = n_compressed(max_seq_len, cfg->l, cfg->d);
  if (nc > nsa::kMaxCompressed)
    return fail(NSA_ERROR_UNSUPPORTED, "max_seq_len %lld gives more than %d compressed blocks", (long long)max_seq_len,
                nsa::kMaxCompressed);
  const nsa::DecodeLayout lay = nsa::decode_layout(dims->batch, dims->num_kv_heads, dims->d_v, cfg->l, cfg->d,
                                                   cfg->l_sel, cfg->n_sel, cfg->n_local, cfg->w, max_seq_len);
  if ((int64_t)dims->batch * dims->num_kv_heads * (lay.nch + lay.nwin + lay.nfin) > (int64_t)INT32_MAX / 2)
    return fail(NSA_ERROR_UNSUPPORTED, "launch too large");
  if ((int64_t)lay.nch * lay.seg < nc || lay.nch > nsa::kMaxChunks || lay.nbo + 1 > nsa::kScStrideMax - 3 ||
      lay.seg > nsa::kSegRows)
    return fail(NSA_ERROR_UNSUPPORTED, "no segment plan for %lld compressed blocks with l_sel/d=%d", (long long)nc,
                cfg->l_sel / cfg->d);
  if (lay.nwin > nsa::kMaxWindow)
    return fail(NSA_ERROR_UNSUPPORTED, "w=%d with l_sel=%d needs more than %d window workgroups", cfg->w, cfg->l_sel,
                nsa::kMaxWindow);
  if (lay.nfin > nsa::kMaxFinish)
    return fail(NSA_ERROR_UNSUPPORTED, "n_sel=%d with l_sel=%d needs more than %d selection workgroups", cfg->n_sel,
                cfg->l_sel, nsa::kMaxFinish);

  return NSA_SUCCESS;
}

nsa_status_t check_prefill_sizes(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t T) {
  if (T < 1) return fail(NSA_ERROR_INVALID_VALUE, "seq_len must be >= 1");
  if ((T - 1) / cfg->l_sel + 1 > nsa::kPfMaxBlocks)
    return fail(NSA_ERROR_UNSUPPORTED, "prefill supports at most %d selection blocks (seq_len %lld, l_sel %d)",
                nsa::kPfMaxBlocks, (long long)T, cfg->l_sel);
  if ((int64_t)dims->batch * dims->num_kv_heads * ((T + 15) / 16) > (int64_t)INT32_MAX / 2)
    return fail(NSA_ERROR_UNSUPPORTED, "batch * kv_heads * seq_len too large");
  return NSA_SUCCESS;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Exactly one gate source: given values, or the gate network's weights (bias optional).
nsa_status_t check_gates(const float* gates, const uint16_t* w_gate, const float* b_gate) {
  if (!gates && !w_gate) return fail(NSA_ERROR_INVALID_VALUE, "give gates or the gate network's w_gate");
  if (gates && (w_gate || b_gate))
    return fail(NSA_ERROR_INVALID_VALUE, "gates and the gate network (w_gate / b_gate) are exclusive");
  return NSA_SUCCESS;
}

// Prefill workspace: [compressed K | compressed V] (in-call compression only),
// then the fp32 accumulator [B, T, Hq, d_v], then the selection buffer
// [B, T, Hkv, n_sel] (always reserved; unused when the caller passes sel_idx_out).
struct PrefillWs {
  size_t off_kc, off_vc, off_acc, off_sel, total;
};
PrefillWs prefill_ws(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t T, bool compress) {
  PrefillWs w{};
  const int64_t nc = n_compressed(T, cfg->l, cfg->d);
  const size_t rows = compress ? (size_t)dims->batch * dims->num_kv_heads * (size_t)nc : 0;
  w.off_kc = 0;
  w.off_vc = align256(rows * dims->d_k * 2);
  w.off_acc = w.off_vc + align256(rows * dims->d_v * 2);
  w.off_sel = w.off_acc + align256((size_t)dims->batch * T * dims->num_q_heads * dims->d_v * 4);
  w.total = w.off_sel + align256((size_t)dims->batch * T * dims->num_kv_heads * cfg->n_sel * 4);
  return w;
}

// Streaming-compression workspace: fp32 chunk partials
// [max(chunks_k, chunks_v)][B*Hkv rounded up to 64][d_k + d_v].
size_t append_ws_bytes(const nsa_dims_t* dims, const nsa_config_t* cfg) {
  const size_t rows_pad = ((size_t)dims->batch * dims->num_kv_heads + 63) / 64 * 64;
  const int ck = nsa::append_chunks(cfg->l, dims->d_k), cv = nsa::append_chunks(cfg->l, dims->d_v);
  return align256((size_t)(ck > cv ? ck : cv) * rows_pad * (dims->d_k + dims->d_v) * 4);
}

// DSA decode: supported shapes and the launch plan.
nsa_status_t check_dsa(const nsa_dsa_dims_t* dims, int32_t top_k, int64_t cache_len) {
  if (!dims) return fail(NSA_ERROR_INVALID_VALUE, "dims is NULL");
  if (dims->batch < 1 || dims->num_heads < 1 || dims->d_qk < 1 || dims->d_v < 1 || dims->idx_heads < 1 ||
      dims->idx_dim < 1)
    return fail(NSA_ERROR_INVALID_VALUE, "DSA dims must be positive");
  if (top_k < 1 || cache_len < 1) return fail(NSA_ERROR_INVALID_VALUE, "top_k and cache_len must be >= 1");
  if (dims->d_qk != nsa::kDsaDqk || dims->d_v != nsa::kDsaDv)
    return fail(NSA_ERROR_UNSUPPORTED, "(d_qk, d_v) = (%d, %d), only (576, 512)", dims->d_qk, dims->d_v);
  if (dims->num_heads % 32 != 0 || dims->num_heads > 256)
    return fail(NSA_ERROR_UNSUPPORTED, "num_heads=%d: a multiple of 32, at most 256", dims->num_heads);
  if (!(dims->idx_heads == 16 || dims->idx_heads == 32 || dims->idx_heads == 64) ||
      !(dims->idx_dim == 64 || dims->idx_dim == 128))
    return fail(NSA_ERROR_UNSUPPORTED, "indexer heads %d x dim %d: heads in {16, 32, 64}, dim in {64, 128}",
                dims->idx_heads, dims->idx_dim);
  if (top_k > nsa::kDsaMaxTopk) return fail(NSA_ERROR_UNSUPPORTED, "top_k=%d > %d", top_k, nsa::kDsaMaxTopk);
  if (cache_len > nsa::kDsaMaxLen)
    return fail(NSA_ERROR_UNSUPPORTED, "cache_len %lld > %d", (long long)cache_len, nsa::kDsaMaxLen);
  return NSA_SUCCESS;
}

struct DsaPlan {
  int seg, nseg, ts, hpg, nchunk;
  int64_t sstride;
  size_t off_scores, off_sel, off_part, off_cnt, off_bits, off_cand, total;
};
DsaPlan dsa_plan(const nsa_dsa_dims_t* dims, int32_t top_k, int64_t cap) {
  DsaPlan pl{};
  const int B = dims->batch, hpg = dims->num_heads % 64 == 0 ? 64 : 32, ngrp = dims->num_heads / hpg;
  pl.hpg = hpg;
  // indexer: about 256 workgroups, segments of whole 512-token batches
  const int want = B >= 256 ? 1 : 256 / B;
  int64_t seg = (cap + want - 1) / want;
  seg = (seg + 511) / 512 * 512;
  pl.seg = (int)seg;
  pl.nseg = (int)((cap + seg - 1) / seg);
  // attention: at most 128 selected tokens per workgroup (the kernel holds all
  // of a split's tiles at once), about 256 workgroups (more splits add partial
  // traffic faster than they add parallelism)
  const int tmin = (top_k + 127) / 128, tmax = (top_k + 63) / 64;
  int ts = 256 / (B * ngrp);
  ts = ts < tmin ? tmin : ts;
  ts = ts > tmax ? tmax : ts;
  pl.ts = ts;
  pl.sstride = (cap + 3) / 4 * 4;
  pl.off_scores = 0;
  pl.off_sel = align256((size_t)B * pl.sstride * 4);
  pl.off_part = pl.off_sel + align256((size_t)B * top_k * 4);
  pl.nchunk = (int)((cap + nsa::kDsaChunk - 1) / nsa::kDsaChunk);
  pl.off_cnt = pl.off_part + align256((size_t)B * ngrp * ts * hpg * (8 + 256) * 4);
  pl.off_bits = pl.off_cnt + align256((size_t)B * (4 + 2 * pl.nchunk) * 4);
  pl.off_cand = pl.off_bits + align256((size_t)B * pl.nchunk * (nsa::kDsaChunk / 32) * 4);
  pl.total = pl.off_cand + align256((size_t)B * pl.nchunk * nsa::kDsaChunk * 8);
  return pl;
}

nsa_status_t hip_fail(hipError_t e, const char* what) {
  return fail(NSA_ERROR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* nsa_status_string(nsa_status_t s) {
  switch (s) {
    case NSA_SUCCESS: return "NSA_SUCCESS";
    case NSA_ERROR_INVALID_VALUE: return "NSA_ERROR_INVALID_VALUE";
    case NSA_ERROR_UNSUPPORTED: return "NSA_ERROR_UNSUPPORTED";
    case NSA_ERROR_WORKSPACE: return "NSA_ERROR_WORKSPACE";
    case NSA_ERROR_HIP: return "NSA_ERROR_HIP";
  }
  return "NSA_UNKNOWN_STATUS";
}

const char* nsa_last_error(void) { return g_last_error.c_str(); }

nsa_status_t nsa_set_phase_events(void* const* events, int32_t count) {
  if (count == 0) {
    g_phase_on = false;
    return ok();
  }
  if (count != 4 || !events) return fail(NSA_ERROR_INVALID_VALUE, "give 4 events (or count 0)");
  for (int i = 0; i < 4; ++i) {
    if (!events[i]) return fail(NSA_ERROR_INVALID_VALUE, "phase event %d is NULL", i);
    g_phase_events.ev[i] = static_cast<hipEvent_t>(events[i]);
  }
  g_phase_on = true;
  return ok();
}

nsa_status_t nsa_set_phase_clock(void* buffer, size_t bytes) {
  if (!buffer || bytes == 0) {
    g_clk = nullptr;
    g_clk_bytes = 0;
    return ok();
  }
  const size_t need = (size_t)2 * nsa::kClkMaxGroups * nsa::kClkSlots * sizeof(uint64_t);
  if (bytes < need) return fail(NSA_ERROR_WORKSPACE, "phase clock buffer of %zu bytes needed, %zu given", need, bytes);
  g_clk = static_cast<uint64_t*>(buffer);
  g_clk_bytes = bytes;
  return ok();
}

nsa_status_t nsa_decode_workspace_size(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t max_seq_len,
                                       size_t* bytes) {
  nsa_status_t st = check_common(dims, cfg, true);
  if (st != NSA_SUCCESS) return st;
  if (!bytes) return fail(NSA_ERROR_INVALID_VALUE, "bytes is NULL");
  if ((st = check_decode_sizes(dims, cfg, max_seq_len)) != NSA_SUCCESS) return st;
  *bytes = nsa::decode_layout(dims->batch, dims->num_kv_heads, dims->d_v, cfg->l, cfg->d, cfg->l_sel, cfg->n_sel,
                              cfg->n_local, cfg->w, max_seq_len)
               .total;
  return ok();
}

nsa_status_t nsa_prefill_workspace_size(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t seq_len,
                                        int32_t compress_in_call, size_t* bytes) {
  nsa_status_t st = check_common(dims, cfg, true);
  if (st != NSA_SUCCESS) return st;
  if (!bytes) return fail(NSA_ERROR_INVALID_VALUE, "bytes is NULL");
  if ((st = check_prefill_sizes(dims, cfg, seq_len)) != NSA_SUCCESS) return st;
  *bytes = prefill_ws(dims, cfg, seq_len, compress_in_call != 0).total;
  return ok();
}

nsa_status_t nsa_compress_kv(const nsa_dims_t* dims, const nsa_config_t* cfg, const uint16_t* k, const uint16_t* v,
                             const int64_t* cu_seqlens, const int32_t* seq_lens, int64_t max_len,
                             const uint16_t* w_k, const uint16_t* pe_k, const uint16_t* w_v, const uint16_t* pe_v,
                             uint16_t* k_cmp, uint16_t* v_cmp, const int64_t* cu_cmp, void* stream) {
  nsa_status_t st = check_common(dims, cfg, true);
  if (st != NSA_SUCCESS) return st;
  if (!k || !v || !w_k || !pe_k || !w_v || !pe_v || !k_cmp || !v_cmp)
    return fail(NSA_ERROR_INVALID_VALUE, "a tensor pointer is NULL");
  if (max_len < 1) return fail(NSA_ERROR_INVALID_VALUE, "max_len must be >= 1");
  const int64_t nc = n_compressed(max_len, cfg->l, cfg->d);
  if ((nc + 63) / 64 > 65535 || (int64_t)dims->batch * dims->num_kv_heads > 65535)
    return fail(NSA_ERROR_UNSUPPORTED, "compression launch too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int which = 0; which < 2; ++which) {
    nsa::CompressParams p{};
    p.B = dims->batch;
    p.H = dims->num_kv_heads;
    p.D = which == 0 ? dims->d_k : dims->d_v;
    p.l = cfg->l;
    p.d = cfg->d;
    p.x = which == 0 ? k : v;
    p.cu = cu_seqlens;
    p.seq_lens = seq_lens;
    p.cap = max_len;
    p.w = which == 0 ? w_k : w_v;
    p.pe = which == 0 ? pe_k : pe_v;
    p.y = which == 0 ? k_cmp : v_cmp;
    p.cuc = cu_cmp;
    p.ccap = nc;
    p.max_nc = (int)nc;
    hipError_t e = nsa::launch_compress(p, s);
    if (e != hipSuccess) return hip_fail(e, "compression launch");
  }
  return ok();
}

nsa_status_t nsa_compress_append_workspace_size(const nsa_dims_t* dims, const nsa_config_t* cfg, size_t* bytes) {
  nsa_status_t st = check_common(dims, cfg, true);
  if (st != NSA_SUCCESS) return st;
  if (!bytes) return fail(NSA_ERROR_INVALID_VALUE, "bytes is NULL");
  *bytes = append_ws_bytes(dims, cfg);
  return ok();
}

nsa_status_t nsa_compress_append(const nsa_dims_t* dims, const nsa_config_t* cfg, const uint16_t* k,
                                 const uint16_t* v, const int64_t* cu_seqlens, const int32_t* seq_lens,
                                 int64_t max_len, const uint16_t* w_k, const uint16_t* pe_k, const uint16_t* w_v,
                                 const uint16_t* pe_v, uint16_t* k_cmp, uint16_t* v_cmp, const int64_t* cu_cmp,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  nsa_status_t st = check_common(dims, cfg, true);
  if (st != NSA_SUCCESS) return st;
  if (!k || !v || !seq_lens || !w_k || !pe_k || !w_v || !pe_v || !k_cmp || !v_cmp)
    return fail(NSA_ERROR_INVALID_VALUE, "a tensor pointer is NULL");
  if (max_len < 1) return fail(NSA_ERROR_INVALID_VALUE, "max_len must be >= 1");
  const int64_t rows = (int64_t)dims->batch * dims->num_kv_heads;
  if ((rows + 63) / 64 > 65535 || rows * (dims->d_k + dims->d_v) / 4 * 8 > (int64_t)INT32_MAX)
    return fail(NSA_ERROR_UNSUPPORTED, "batch * kv_heads too large");
  if (nsa::append_chunks(cfg->l, dims->d_k) > 96 || nsa::append_chunks(cfg->l, dims->d_v) > 96)
    return fail(NSA_ERROR_UNSUPPORTED, "l * d_k above 96 * 256");
  const size_t need = append_ws_bytes(dims, cfg);
  if (!workspace || workspace_bytes < need)
    return fail(NSA_ERROR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  nsa::AppendParams p{};
  p.B = dims->batch;
  p.H = dims->num_kv_heads;
  p.DK = dims->d_k;
  p.DV = dims->d_v;
  p.l = cfg->l;
  p.d = cfg->d;
  p.k = k;
  p.v = v;
  p.cu = cu_seqlens;
  p.seq_lens = seq_lens;
  p.cap = max_len;
  p.wk = w_k;
  p.pek = pe_k;
  p.wv = w_v;
  p.pev = pe_v;
  p.kc = k_cmp;
  p.vc = v_cmp;
  p.cuc = cu_cmp;
  p.ccap = n_compressed(max_len, cfg->l, cfg->d);
  p.part = static_cast<float*>(workspace);
  p.rows_pad = (int)((rows + 63) / 64 * 64);
  p.nck_k = nsa::append_chunks(cfg->l, dims->d_k);
  p.nck_v = nsa::append_chunks(cfg->l, dims->d_v);
  if (p.ccap == 0) return ok();  // no sequence can hold a complete block
  hipError_t e = nsa::launch_append(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

namespace {

// Checks of a decode call that do not depend on where its workspace lives.
nsa_status_t check_decode_call(const nsa_dims_t* dims, const nsa_config_t* cfg, const uint16_t* q,
                               const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_cmp_cache,
                               const uint16_t* v_cmp_cache, const int32_t* seq_lens, int64_t max_seq_len,
                               const float* gates, const uint16_t* w_gate, const float* b_gate,
                               const uint16_t* out) {
  nsa_status_t st = check_common(dims, cfg, true);
  if (st != NSA_SUCCESS) return st;
  if (!q || !k_cache || !v_cache || !k_cmp_cache || !v_cmp_cache || !seq_lens || !out)
    return fail(NSA_ERROR_INVALID_VALUE, "a tensor pointer is NULL");
  if ((st = check_gates(gates, w_gate, b_gate)) != NSA_SUCCESS) return st;
  return check_decode_sizes(dims, cfg, max_seq_len);
}

// Launches a validated decode step with the workspace at `workspace`.
nsa_status_t decode_launch(const nsa_dims_t* dims, const nsa_config_t* cfg, const uint16_t* q,
                           const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_cmp_cache,
                           const uint16_t* v_cmp_cache, const int32_t* seq_lens, const int64_t* cu_seqlens,
                           const int64_t* cu_cmp, int64_t max_seq_len, const float* gates,
                           const uint16_t* w_gate, const float* b_gate, uint16_t* out, int32_t* sel_idx_out,
                           const nsa::DecodeLayout& lay, void* workspace, void* stream) {
  char* ws = static_cast<char*>(workspace);
  nsa::DecodeParams p{};
  p.B = dims->batch;
  p.Hq = dims->num_q_heads;
  p.H = dims->num_kv_heads;
  p.G = p.Hq / p.H;
  p.l = cfg->l;
  p.d = cfg->d;
  p.lsel = cfg->l_sel;
  p.n = cfg->n_sel;
  p.nloc = cfg->n_local;
  p.finit = cfg->force_initial;
  p.w = cfg->w;
  p.scale_log2 = scale_log2(dims, cfg);
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.kc = k_cmp_cache;
  p.vc = v_cmp_cache;
  p.seq_lens = seq_lens;
  p.cu = cu_seqlens;
  p.cuc = cu_cmp;
  p.cap = max_seq_len;
  p.ccap = n_compressed(max_seq_len, cfg->l, cfg->d);
  p.gates = gates;
  p.wgate = w_gate;
  p.bgate = b_gate;
  p.out = out;
  p.sel_out = sel_idx_out;
  p.m1 = reinterpret_cast<float*>(ws + lay.off_m1);
  p.l1 = reinterpret_cast<float*>(ws + lay.off_l1);
  p.o1 = reinterpret_cast<float*>(ws + lay.off_o1);
  p.sc1 = reinterpret_cast<float*>(ws + lay.off_sc1);
  p.wpart = reinterpret_cast<float*>(ws + lay.off_wpart);
  p.nwin = lay.nwin;
  p.wtiles = lay.wtiles;
  p.rpart = reinterpret_cast<float*>(ws + lay.off_rpart);
  p.ocmp = reinterpret_cast<float*>(ws + lay.off_ocmp);
  p.cnt = reinterpret_cast<uint32_t*>(ws + lay.off_cnt);
  p.nfin = lay.nfin;
  p.finw = lay.finw;
  p.nch = lay.nch;
  p.seg = lay.seg;
  p.nbo = lay.nbo;
  p.bal = lay.bal;
  p.nslot = lay.nslot;
  p.bal_fill = lay.bal_fill;
  p.tmin = lay.tmin;
  p.tcap = lay.tcap;
  p.scs = lay.scs;
  const int64_t g1 = std::max<int64_t>((int64_t)p.B * p.H * (p.nch + p.nwin),
                                       lay.bal ? (int64_t)p.B * p.H * p.nwin + p.nslot : 0);
  if (g_clk && std::max<int64_t>(g1, (int64_t)p.B * p.H * p.nfin) <= nsa::kClkMaxGroups) p.clk = g_clk;
  const nsa::PhaseEvents* ev = g_phase_on ? &g_phase_events : nullptr;
  hipError_t e = nsa::launch_decode(p, dims->d_k, dims->d_v, static_cast<hipStream_t>(stream), ev);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

}  // namespace

nsa_status_t nsa_decode_fwd(const nsa_dims_t* dims, const nsa_config_t* cfg, const uint16_t* q,
                            const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_cmp_cache,
                            const uint16_t* v_cmp_cache, const int32_t* seq_lens, const int64_t* cu_seqlens,
                            const int64_t* cu_cmp, int64_t max_seq_len, const float* gates,
                            const uint16_t* w_gate, const float* b_gate, uint16_t* out,
                            int32_t* sel_idx_out, void* workspace, size_t workspace_bytes, void* stream) {
  nsa_status_t st = check_decode_call(dims, cfg, q, k_cache, v_cache, k_cmp_cache, v_cmp_cache, seq_lens, max_seq_len,
                                      gates, w_gate, b_gate, out);
  if (st != NSA_SUCCESS) return st;
  const nsa::DecodeLayout lay = nsa::decode_layout(dims->batch, dims->num_kv_heads, dims->d_v, cfg->l, cfg->d,
                                                   cfg->l_sel, cfg->n_sel, cfg->n_local, cfg->w, max_seq_len);
  if (!workspace || workspace_bytes < lay.total)
    return fail(NSA_ERROR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total,
                workspace ? workspace_bytes : (size_t)0);
  return decode_launch(dims, cfg, q, k_cache, v_cache, k_cmp_cache, v_cmp_cache, seq_lens, cu_seqlens, cu_cmp,
                       max_seq_len, gates, w_gate, b_gate, out, sel_idx_out, lay, workspace, stream);
}

nsa_status_t nsa_decode_fwd_noalloc(const nsa_dims_t* dims, const nsa_config_t* cfg, const uint16_t* q,
                                    const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_cmp_cache,
                                    const uint16_t* v_cmp_cache, const int32_t* seq_lens, const int64_t* cu_seqlens,
                                    const int64_t* cu_cmp, int64_t max_seq_len, const float* gates,
                                    const uint16_t* w_gate, const float* b_gate, uint16_t* out,
                                    int32_t* sel_idx_out, void* stream) {
  nsa_status_t st = check_decode_call(dims, cfg, q, k_cache, v_cache, k_cmp_cache, v_cmp_cache, seq_lens, max_seq_len,
                                      gates, w_gate, b_gate, out);
  if (st != NSA_SUCCESS) return st;
  const nsa::DecodeLayout lay = nsa::decode_layout(dims->batch, dims->num_kv_heads, dims->d_v, cfg->l, cfg->d,
                                                   cfg->l_sel, cfg->n_sel, cfg->n_local, cfg->w, max_seq_len);
  if (lay.total > nsa::kNoAllocScratchBytes)
    return fail(NSA_ERROR_UNSUPPORTED,
                "this decode step needs %zu bytes of scratch; the allocation-free entry point holds %zu "
                "(use nsa_decode_fwd with a workspace)",
                lay.total, nsa::kNoAllocScratchBytes);
  void* ws = nullptr;
  const hipError_t e = nsa::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "locating the scratch array");
  return decode_launch(dims, cfg, q, k_cache, v_cache, k_cmp_cache, v_cmp_cache, seq_lens, cu_seqlens, cu_cmp,
                       max_seq_len, gates, w_gate, b_gate, out, sel_idx_out, lay, ws, stream);
}

nsa_status_t nsa_dsa_decode_workspace_size(const nsa_dsa_dims_t* dims, int32_t top_k, int64_t cache_len,
                                           size_t* bytes) {
  nsa_status_t st = check_dsa(dims, top_k, cache_len);
  if (st != NSA_SUCCESS) return st;
  if (!bytes) return fail(NSA_ERROR_INVALID_VALUE, "bytes is NULL");
  *bytes = dsa_plan(dims, top_k, cache_len).total;
  return ok();
}

nsa_status_t nsa_dsa_decode_fwd(const nsa_dsa_dims_t* dims, int32_t top_k, float softmax_scale, const uint16_t* q,
                                const uint8_t* q_idx, const float* w_idx, const uint16_t* latent,
                                const uint8_t* k_idx, const int32_t* seq_lens, int64_t cache_len, uint16_t* out,
                                int32_t* sel_idx_out, void* workspace, size_t workspace_bytes, void* stream) {
  nsa_status_t st = check_dsa(dims, top_k, cache_len);
  if (st != NSA_SUCCESS) return st;
  if (!q || !q_idx || !w_idx || !latent || !k_idx || !seq_lens || !out)
    return fail(NSA_ERROR_INVALID_VALUE, "a tensor pointer is NULL");
  if (!(softmax_scale >= 0.f) || !std::isfinite(softmax_scale))
    return fail(NSA_ERROR_INVALID_VALUE, "softmax_scale must be finite and >= 0");
  const DsaPlan plan = dsa_plan(dims, top_k, cache_len);
  if (!workspace || workspace_bytes < plan.total)
    return fail(NSA_ERROR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.total,
                workspace ? workspace_bytes : (size_t)0);
  char* ws = static_cast<char*>(workspace);
  nsa::DsaParams p{};
  p.B = dims->batch;
  p.H = dims->num_heads;
  p.HI = dims->idx_heads;
  p.DI = dims->idx_dim;
  p.topk = top_k;
  const float sc = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)dims->d_qk);
  p.scale_log2 = sc * 1.4426950408889634f;
  p.cap = cache_len;
  p.q = q;
  p.qi = q_idx;
  p.wi = w_idx;
  p.c = latent;
  p.ki = k_idx;
  p.seq_lens = seq_lens;
  p.out = out;
  p.scores = reinterpret_cast<float*>(ws + plan.off_scores);
  p.sstride = plan.sstride;
  p.sel = sel_idx_out ? sel_idx_out : reinterpret_cast<int32_t*>(ws + plan.off_sel);
  p.part = reinterpret_cast<float*>(ws + plan.off_part);
  p.seg = plan.seg;
  p.nseg = plan.nseg;
  p.ts = plan.ts;
  p.hpg = plan.hpg;
  p.nchunk = plan.nchunk;
  p.cnt = reinterpret_cast<uint32_t*>(ws + plan.off_cnt);
  p.bits = reinterpret_cast<uint32_t*>(ws + plan.off_bits);
  p.cand = reinterpret_cast<uint64_t*>(ws + plan.off_cand);
  if (g_clk && (int64_t)p.B * (p.H / p.hpg) * p.ts <= nsa::kClkMaxGroups &&
      (int64_t)p.B * p.nchunk <= nsa::kClkMaxGroups)
    p.clk = g_clk;
  const nsa::PhaseEvents* ev = g_phase_on ? &g_phase_events : nullptr;
  hipError_t e = nsa::launch_dsa_decode(p, static_cast<hipStream_t>(stream), ev);
  if (e != hipSuccess) return hip_fail(e, "DSA decode launch");
  return ok();
}

nsa_status_t nsa_prefill_fwd(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t seq_len, const uint16_t* q,
                             const uint16_t* k, const uint16_t* v, const uint16_t* k_cmp, const uint16_t* v_cmp,
                             const uint16_t* w_k, const uint16_t* pe_k, const uint16_t* w_v, const uint16_t* pe_v,
                             const float* gates, const uint16_t* w_gate, const float* b_gate, uint16_t* out,
                             int32_t* sel_idx_out, float* lse_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  nsa_status_t st = check_common(dims, cfg, true);
  if (st != NSA_SUCCESS) return st;
  if (!q || !k || !v || !out) return fail(NSA_ERROR_INVALID_VALUE, "a tensor pointer is NULL");
  if ((st = check_gates(gates, w_gate, b_gate)) != NSA_SUCCESS) return st;
  if ((k_cmp == nullptr) != (v_cmp == nullptr))
    return fail(NSA_ERROR_INVALID_VALUE, "k_cmp and v_cmp must both be given or both be NULL");
  const bool compress = k_cmp == nullptr;
  if (compress && (!w_k || !pe_k || !w_v || !pe_v))
    return fail(NSA_ERROR_INVALID_VALUE, "compression weights are NULL and no compressed cache was given");
  if ((st = check_prefill_sizes(dims, cfg, seq_len)) != NSA_SUCCESS) return st;
  const PrefillWs lay = prefill_ws(dims, cfg, seq_len, compress);
  if (!workspace || workspace_bytes < lay.total)
    return fail(NSA_ERROR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total,
                workspace ? workspace_bytes : (size_t)0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const nsa::PhaseEvents* ev = g_phase_on ? &g_phase_events : nullptr;
  if (ev) hipEventRecord(ev->ev[0], s);
  const int64_t nc = n_compressed(seq_len, cfg->l, cfg->d);
  if (compress && nc == 0) {
    k_cmp = k;  // no complete compressed block exists; the cache is never read
    v_cmp = v;
  } else if (compress) {
    uint16_t* kcw = reinterpret_cast<uint16_t*>(ws + lay.off_kc);
    uint16_t* vcw = reinterpret_cast<uint16_t*>(ws + lay.off_vc);
    st = nsa_compress_kv(dims, cfg, k, v, nullptr, nullptr, seq_len, w_k, pe_k, w_v, pe_v, kcw, vcw, nullptr, stream);
    if (st != NSA_SUCCESS) return st;
    k_cmp = kcw;
    v_cmp = vcw;
  }
  if (ev) hipEventRecord(ev->ev[1], s);
  nsa::PrefillParams p{};
  p.B = dims->batch;
  p.T = (int)seq_len;
  p.Hq = dims->num_q_heads;
  p.H = dims->num_kv_heads;
  p.G = p.Hq / p.H;
  p.l = cfg->l;
  p.d = cfg->d;
  p.lsel = cfg->l_sel;
  p.n = cfg->n_sel;
  p.nloc = cfg->n_local;
  p.finit = cfg->force_initial;
  p.w = cfg->w;
  p.scale_log2 = scale_log2(dims, cfg);
  p.nc = (int)nc;
  p.ntile = (int)((seq_len + 15) / 16);
  p.q = q;
  p.k = k;
  p.v = v;
  p.kc = k_cmp;
  p.vc = v_cmp;
  p.gates = gates;
  p.wgate = w_gate;
  p.bgate = b_gate;
  p.out = out;
  p.sel = sel_idx_out ? sel_idx_out : reinterpret_cast<int32_t*>(ws + lay.off_sel);
  p.acc = reinterpret_cast<float*>(ws + lay.off_acc);
  p.lse = lse_out;
  hipError_t e = nsa::launch_prefill(p, dims->d_k, dims->d_v, s, ev);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward (training).

namespace {

// Prefill-backward plan of the key side.  Selected branch: each 64-key tile's
// positions are split into workgroups of kSlcSplit; slots_max bounds the splits
// of one (sequence, group): every selection lands in at most max(1, l_sel/64)
// tiles.  Compressed branch: ranges of at least 1024 positions, at most 32.
struct BwdPlan {
  int kraw, slots_max, qchunk, ncq;
};
BwdPlan bwd_plan(const nsa_config_t* cfg, int64_t T) {
  BwdPlan pl{};
  pl.kraw = (int)((T + 63) / 64);
  const int64_t sel = T * cfg->n_sel * std::max(1, cfg->l_sel / 64);
  pl.slots_max = pl.kraw + (int)((sel + nsa::kSlcSplit - 1) / nsa::kSlcSplit);
  pl.qchunk = (int)std::max<int64_t>(1024, (T + 31) / 32);
  pl.qchunk += pl.qchunk & 1;
  pl.ncq = (int)((T + pl.qchunk - 1) / pl.qchunk);
  return pl;
}

// Prefill-backward workspace: per-branch statistics records [3, B, T, Hkv, 48]
// fp32, the selection bitmap [B, Hkv, ceil(T / l_sel), ceil(T / 32)] uint32, the
// key side's partial sums: selected [B*Hkv, slots_max, 64, d_k + d_v] and
// compressed [ncq, B, Hkv, nc, d_k + d_v] fp32, the selected branch's counts
// [B*Hkv, kraw] and slot offsets [B*Hkv, kraw + 1] int32, and the gate-network
// gradient partials [64, Hq, 3, d_k + 1] fp32.
struct BwdWs {
  size_t off_stat, off_bits, off_pslc, off_pcmp, off_cnt, off_soff, off_gpart, total;
};
BwdWs bwd_ws(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t T) {
  BwdWs w{};
  const BwdPlan pl = bwd_plan(cfg, T);
  const size_t bh = (size_t)dims->batch * dims->num_kv_heads, wd = (size_t)(dims->d_k + dims->d_v);
  const size_t recs = (size_t)3 * bh * (size_t)T;
  const size_t nblk = (size_t)((T + cfg->l_sel - 1) / cfg->l_sel), nwords = (size_t)((T + 31) / 32);
  const size_t nc = (size_t)n_compressed(T, cfg->l, cfg->d);
  w.off_stat = 0;
  w.off_bits = align256(recs * nsa::kStatFloats * 4);
  w.off_pslc = w.off_bits + align256(bh * nblk * nwords * 4);
  w.off_pcmp = w.off_pslc + align256(bh * (size_t)pl.slots_max * 64 * wd * 4);
  w.off_cnt = w.off_pcmp + align256((size_t)pl.ncq * bh * nc * wd * 4);
  w.off_soff = w.off_cnt + align256(bh * (size_t)pl.kraw * 4);
  w.off_gpart = w.off_soff + align256(bh * (size_t)(pl.kraw + 1) * 4);
  w.total = w.off_gpart + align256((size_t)nsa::kGateChunks * dims->num_q_heads * 3 * (dims->d_k + 1) * 4);
  return w;
}

// Compression-backward workspace: 64 column-sum partials [64, D], then the dW
// product's split partials [8, l*D, D].
size_t cbwd_ws(const nsa_config_t* cfg, int D) {
  return align256((size_t)64 * D * 4) + align256((size_t)nsa::kCbwdSplit * cfg->l * D * D * 4);
}

nsa_status_t check_cbwd(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t T, int32_t which) {
  nsa_status_t st = check_common(dims, cfg, true);
  if (st != NSA_SUCCESS) return st;
  if (which != 0 && which != 1) return fail(NSA_ERROR_INVALID_VALUE, "which must be 0 (keys) or 1 (values)");
  if (T < 1) return fail(NSA_ERROR_INVALID_VALUE, "seq_len must be >= 1");
  if ((int64_t)dims->batch * dims->num_kv_heads > 65535 ||
      (int64_t)dims->batch * dims->num_kv_heads * n_compressed(T, cfg->l, cfg->d) > INT32_MAX)
    return fail(NSA_ERROR_UNSUPPORTED, "compression backward launch too large");
  return NSA_SUCCESS;
}

}  // namespace

extern "C" {

nsa_status_t nsa_prefill_bwd_workspace_size(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t seq_len,
                                            size_t* bytes) {
  nsa_status_t st = check_common(dims, cfg, true);
  if (st != NSA_SUCCESS) return st;
  if (!bytes) return fail(NSA_ERROR_INVALID_VALUE, "bytes is NULL");
  if ((st = check_prefill_sizes(dims, cfg, seq_len)) != NSA_SUCCESS) return st;
  *bytes = bwd_ws(dims, cfg, seq_len).total;
  return ok();
}

nsa_status_t nsa_prefill_bwd(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t seq_len, const uint16_t* q,
                             const uint16_t* k, const uint16_t* v, const uint16_t* k_cmp, const uint16_t* v_cmp,
                             const float* gates, const uint16_t* w_gate, const float* b_gate, const int32_t* sel_idx,
                             const float* lse, const uint16_t* dout, float* dq, float* dk, float* dv, float* dk_cmp, float* dv_cmp,
                             float* dgates, float* dw_gate, float* db_gate, void* workspace, size_t workspace_bytes,
                             void* stream) {
  nsa_status_t st = check_common(dims, cfg, true);
  if (st != NSA_SUCCESS) return st;
  if ((st = check_prefill_sizes(dims, cfg, seq_len)) != NSA_SUCCESS) return st;
  if (!q || !k || !v || !sel_idx || !dout || !dq || !dk || !dv || !dgates)
    return fail(NSA_ERROR_INVALID_VALUE, "a tensor pointer is NULL");
  if ((st = check_gates(gates, w_gate, b_gate)) != NSA_SUCCESS) return st;
  if (w_gate && (!dw_gate || (b_gate && !db_gate)))
    return fail(NSA_ERROR_INVALID_VALUE, "the gate network needs dw_gate (and db_gate with b_gate)");
  if ((int64_t)dims->batch * dims->num_kv_heads > 65535)
    return fail(NSA_ERROR_UNSUPPORTED, "batch * num_kv_heads above 65535");
  if (seq_len * dims->num_q_heads * (int64_t)std::max(dims->d_k, dims->d_v) * 2 >= ((int64_t)1 << 32))
    return fail(NSA_ERROR_UNSUPPORTED, "seq_len * num_q_heads * max(d_k, d_v) * 2 must stay below 2^32 bytes");
  const int64_t nc = n_compressed(seq_len, cfg->l, cfg->d);
  if (nc > 0 && (!k_cmp || !v_cmp || !dk_cmp || !dv_cmp))
    return fail(NSA_ERROR_INVALID_VALUE, "the compressed cache and its gradient buffers are required (%lld blocks)",
                (long long)nc);
  const BwdWs lay = bwd_ws(dims, cfg, seq_len);
  if (!workspace || workspace_bytes < lay.total)
    return fail(NSA_ERROR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total,
                workspace ? workspace_bytes : (size_t)0);
  char* ws = static_cast<char*>(workspace);
  nsa::BwdParams p{};
  p.B = dims->batch;
  p.T = (int)seq_len;
  p.Hq = dims->num_q_heads;
  p.H = dims->num_kv_heads;
  p.G = p.Hq / p.H;
  p.l = cfg->l;
  p.d = cfg->d;
  p.lsel = cfg->l_sel;
  p.n = cfg->n_sel;
  p.w = cfg->w;
  p.scale_log2 = scale_log2(dims, cfg);
  p.scale = p.scale_log2 / 1.4426950408889634f;
  p.nc = (int)nc;
  p.nqt = (int)((seq_len + 3) / 4);
  p.nblk = (int)((seq_len + cfg->l_sel - 1) / cfg->l_sel);
  p.nwords = (int)((seq_len + 31) / 32);
  const BwdPlan pl = bwd_plan(cfg, seq_len);
  p.kraw = pl.kraw;
  p.slots_max = pl.slots_max;
  p.qchunk = pl.qchunk;
  p.ncq = pl.ncq;
  p.q = q;
  p.k = k;
  p.v = v;
  p.kc = nc > 0 ? k_cmp : k;  // never read without a compressed block
  p.vc = nc > 0 ? v_cmp : v;
  p.gates = gates;
  p.wgate = w_gate;
  p.bgate = b_gate;
  p.dwgate = dw_gate;
  p.dbgate = b_gate ? db_gate : nullptr;
  p.lse_in = lse;
  p.gpart = reinterpret_cast<float*>(ws + lay.off_gpart);
  p.sel = sel_idx;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dkc = dk_cmp;
  p.dvc = dv_cmp;
  p.dgates = dgates;
  p.stat = reinterpret_cast<float*>(ws + lay.off_stat);
  p.bits = reinterpret_cast<uint32_t*>(ws + lay.off_bits);
  p.part_slc = reinterpret_cast<float*>(ws + lay.off_pslc);
  p.part_cmp = reinterpret_cast<float*>(ws + lay.off_pcmp);
  p.slc_cnt = reinterpret_cast<int32_t*>(ws + lay.off_cnt);
  p.slc_off = reinterpret_cast<int32_t*>(ws + lay.off_soff);
  const nsa::PhaseEvents* ev = g_phase_on ? &g_phase_events : nullptr;
  hipError_t e = nsa::launch_prefill_bwd(p, dims->d_k, dims->d_v, static_cast<hipStream_t>(stream), ev);
  if (e != hipSuccess) return hip_fail(e, "prefill backward launch");
  return ok();
}

nsa_status_t nsa_compress_bwd_workspace_size(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t seq_len,
                                             int32_t which, size_t* bytes) {
  nsa_status_t st = check_cbwd(dims, cfg, seq_len, which);
  if (st != NSA_SUCCESS) return st;
  if (!bytes) return fail(NSA_ERROR_INVALID_VALUE, "bytes is NULL");
  *bytes = cbwd_ws(cfg, which == 0 ? dims->d_k : dims->d_v);
  return ok();
}

nsa_status_t nsa_compress_bwd(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t seq_len, int32_t which,
                              const uint16_t* x, const uint16_t* w, const uint16_t* pe, const float* dy, float* dx,
                              float* dw, float* dpe, void* workspace, size_t workspace_bytes, void* stream) {
  nsa_status_t st = check_cbwd(dims, cfg, seq_len, which);
  if (st != NSA_SUCCESS) return st;
  const int64_t nc = n_compressed(seq_len, cfg->l, cfg->d);
  if (!x || !w || !pe || !dx || !dw || !dpe || (nc > 0 && !dy))
    return fail(NSA_ERROR_INVALID_VALUE, "a tensor pointer is NULL");
  const int D = which == 0 ? dims->d_k : dims->d_v;
  const size_t need = cbwd_ws(cfg, D);
  if (!workspace || workspace_bytes < need)
    return fail(NSA_ERROR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  char* ws = static_cast<char*>(workspace);
  nsa::CompressBwdParams p{};
  p.BH = dims->batch * dims->num_kv_heads;
  p.D = D;
  p.l = cfg->l;
  p.d = cfg->d;
  p.nc = (int)nc;
  p.T = seq_len;
  p.x = x;
  p.w = w;
  p.pe = pe;
  p.dy = dy;
  p.dx = dx;
  p.dw = dw;
  p.dpe = dpe;
  p.part = reinterpret_cast<float*>(ws);
  p.dwpart = reinterpret_cast<float*>(ws + align256((size_t)64 * D * 4));
  hipError_t e = nsa::launch_compress_bwd(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "compression backward launch");
  return ok();
}

}  // extern "C"

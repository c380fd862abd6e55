/*
 * nsa.h — C ABI of the MI355X (gfx950) Native Sparse Attention forward pass.
 *
 * Native Sparse Attention runs three attention branches per query over one KV
 * cache and mixes them with per-head gates:
 *
 *   o_t = g_cmp * Attn(q_t, compressed K/V) + g_slc * Attn(q_t, selected K/V)
 *       + g_win * Attn(q_t, window K/V)
 *
 * Sources: lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc),
 * section "NSA: три ветви" (the output equation and the paragraphs on the
 * compressed branch, the selection branch and the sliding window); lesson
 * "Native Sparse Attention (DeepSeek NSA)" (AI Engineering from Scratch, phase
 * 10 · 17), sections "Concept — three parallel branches" and "Build it".
 *
 * Conventions shared by every entry point
 *  - bf16 tensors are passed as uint16_t bit patterns; gates are float32.
 *  - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *    never allocates or frees device memory and never synchronises; all work is
 *    enqueued on `stream` (a hipStream_t; NULL means the default stream) and the
 *    pointers must stay valid until that work has finished.
 *  - Arguments are validated on the host before anything is enqueued.  On any
 *    error nothing is launched, outputs are untouched, and nsa_last_error()
 *    (thread-local) describes the problem.  Device faults surface at the
 *    caller's next synchronisation.
 *  - Workspace: a caller-provided device buffer of at least the size the
 *    matching *_workspace_size query returns; its contents on entry do not
 *    matter.  Calls that share a workspace must not overlap in time.
 *  - Query head h belongs to KV group g = h / G with G = num_q_heads /
 *    num_kv_heads; all heads of a group select the same blocks (selection
 *    paragraph of "NSA: три ветви").
 *  - Supported set: (d_k, d_v) in {(64,64), (128,128), (192,128)}; 1 <= G <= 16;
 *    d divides l and l'; l <= l'; l'/d a power of two; l' in {16,32,64,128};
 *    1 <= n_sel <= 64; n_local + force_initial <= n_sel.  Anything else returns
 *    NSA_ERROR_UNSUPPORTED.
 */
#ifndef NSA_H_
#define NSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NSA_SUCCESS = 0,
  NSA_ERROR_INVALID_VALUE = 1, /* null pointer, non-positive size, inconsistent shape */
  NSA_ERROR_UNSUPPORTED = 2,   /* valid but outside the supported set above */
  NSA_ERROR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  NSA_ERROR_HIP = 4            /* a HIP launch failed; message in nsa_last_error() */
} nsa_status_t;

/* NSA parameters ("NSA: три ветви": l=32, d=16, l'=64, n=16 incl. the initial
 * and two local blocks, w=512). */
typedef struct {
  int32_t l;             /* compression block length (tokens per compressed key) */
  int32_t d;             /* compression stride; blocks overlap when d < l */
  int32_t l_sel;         /* selection block length l' */
  int32_t n_sel;         /* blocks selected per (query, KV group), forced ones included */
  int32_t n_local;       /* trailing blocks (the query's own and the ones before) always selected */
  int32_t force_initial; /* 1: block 0 is always selected */
  int32_t w;             /* sliding-window length: keys x with t - w < x <= t */
  float softmax_scale;   /* 0 selects 1/sqrt(d_k) for all three branches */
} nsa_config_t;

typedef struct {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t d_k;
  int32_t d_v;
} nsa_dims_t;

/*
 * nsa_compress_kv — token-block compression ("NSA: три ветви", compressed
 * branch: blocks of l tokens with stride d, each folded by a learned MLP into
 * one key and one value).  The MLP is one bias-free linear layer on the block
 * plus a learned intra-block position embedding, flattened token-major:
 *
 *   k_cmp[i] = sum_{j<l} (K[i*d + j] + pe_k[j]) . w_k[j*d_k : (j+1)*d_k, :]
 *
 * and likewise for values with (w_v, pe_v).  Accumulates in fp32 and rounds the
 * result to bf16 (round to nearest even).
 *
 *   k, v        bf16 caches.  Token x of sequence b, KV head g is row
 *               Hkv*cu_seqlens[b] + g*cap_b + x of a [rows, d_k] (resp. d_v)
 *               row-major array, cap_b = cu_seqlens[b+1] - cu_seqlens[b].
 *               cu_seqlens == NULL means cap_b = max_len for every b
 *               (i.e. the dense layout [B, Hkv, max_len, D]).
 *   seq_lens    int32 [B] tokens present per sequence (device); NULL = cap_b.
 *   max_len     host upper bound of every seq_lens[b] (and of cap_b).
 *   w_k [l*d_k, d_k], pe_k [l, d_k], w_v [l*d_v, d_v], pe_v [l, d_v]: bf16.
 *   k_cmp, v_cmp  outputs; block i of (b, g) is row Hkv*cu_cmp[b] + g*ccap_b + i,
 *               ccap_b = cu_cmp[b+1] - cu_cmp[b]; cu_cmp == NULL means
 *               ccap_b = floor((max_len - l)/d) + 1.  Blocks i < floor((L_b-l)/d)+1
 *               (and i < ccap_b) are written; other rows are untouched.
 */
nsa_status_t nsa_compress_kv(const nsa_dims_t* dims, const nsa_config_t* cfg,
                             const uint16_t* k, const uint16_t* v,
                             const int64_t* cu_seqlens, const int32_t* seq_lens, int64_t max_len,
                             const uint16_t* w_k, const uint16_t* pe_k,
                             const uint16_t* w_v, const uint16_t* pe_v,
                             uint16_t* k_cmp, uint16_t* v_cmp, const int64_t* cu_cmp,
                             void* stream);

/*
 * nsa_compress_append — streaming compression for decode ("NSA: три ветви",
 * compressed branch: a block of l tokens with stride d is complete once its
 * last token exists, so decode gains one compressed key/value every d tokens).
 * Call it after token t = seq_lens[b] - 1 has been written into k/v and before
 * nsa_decode_fwd for that step: for every sequence b with t = i*d + l - 1
 * (seq_lens[b] >= l, (seq_lens[b] - l) divisible by d) and i < ccap_b, block i
 * of each KV head is computed exactly as nsa_compress_kv computes it and stored
 * at compressed row i; every other row, and every other sequence, is left
 * untouched.  The sum over the l*D inputs is taken in a different order than
 * in nsa_compress_kv (fp32 chunk partials added in a fixed order), so the two
 * may differ in the last bf16 bit; repeated calls give identical bits.
 *
 *   k, v, cu_seqlens, max_len, w_k, pe_k, w_v, pe_v, k_cmp, v_cmp, cu_cmp:
 *               as for nsa_compress_kv.
 *   seq_lens    int32 [B] on the device, required (the current lengths);
 *               a length above cap_b is treated as having no due block.
 *   workspace   at least nsa_compress_append_workspace_size bytes of device
 *               memory (fp32 partial sums); contents on entry do not matter.
 */
nsa_status_t nsa_compress_append(const nsa_dims_t* dims, const nsa_config_t* cfg,
                                 const uint16_t* k, const uint16_t* v,
                                 const int64_t* cu_seqlens, const int32_t* seq_lens, int64_t max_len,
                                 const uint16_t* w_k, const uint16_t* pe_k,
                                 const uint16_t* w_v, const uint16_t* pe_v,
                                 uint16_t* k_cmp, uint16_t* v_cmp, const int64_t* cu_cmp,
                                 void* workspace, size_t workspace_bytes, void* stream);
/* Workspace bytes for nsa_compress_append (host-only): max(ceil(l*d_k/256),
 * ceil(l*d_v/256)) * (batch*num_kv_heads rounded up to 64) * (d_k + d_v) * 4. */
nsa_status_t nsa_compress_append_workspace_size(const nsa_dims_t* dims, const nsa_config_t* cfg,
                                                size_t* bytes);
/*
 * nsa_decode_fwd — one decode step: each sequence b has one query at position
 * t = seq_lens[b] - 1 whose key/value are already in the cache.
 *
 *   q         bf16 [B, Hq, d_k]
 *   k_cache, v_cache      bf16, layout of nsa_compress_kv's k/v (cu_seqlens,
 *                         NULL = dense with capacity max_seq_len).
 *   k_cmp_cache, v_cmp_cache  bf16 compressed cache, layout of nsa_compress_kv's
 *                         outputs (cu_cmp); must hold the floor((L_b-l)/d)+1
 *                         complete blocks of each sequence.
 *   seq_lens  int32 [B] on the device, 1 <= seq_lens[b] <= cap_b.
 *   max_seq_len  host upper bound of seq_lens (sizes the launch).
 *   gates     float32 [B, Hq, 3] = (g_cmp, g_slc, g_win), used as given; or
 *             NULL when the gate network computes them (see w_gate).
 *   w_gate, b_gate  the gate network, or both NULL when gates are given.  Read
 *             as one linear layer and a sigmoid on each query head's vector
 *             ("Native Sparse Attention" lesson, "Build it" step 5: a small MLP
 *             on the query yields the three gate weights; "NSA: три ветви": the
 *             gates lie in [0, 1], from a small network with a sigmoid):
 *               gate[b, h, c] = sigmoid(w_gate[h, c, :] . q[b, h, :] + b_gate[h, c])
 *             w_gate bf16 [Hq, 3, d_k] (c = cmp, slc, win); b_gate float32
 *             [Hq, 3] or NULL (no bias).  Computed in fp32 inside the kernels
 *             that apply the gates.  Giving both gates and w_gate/b_gate is
 *             NSA_ERROR_INVALID_VALUE.
 *   out       bf16 [B, Hq, d_v].
 *   sel_idx_out  nullable int32 [B, Hkv, n_sel]: the selected block ids,
 *             ascending, padded with -1 when fewer than n_sel blocks exist.
 *
 * Selection: candidates are blocks 0..J, J = floor(t/l'); block 0 (if
 * force_initial) and J, J-1, ... (n_local of them) are always taken and count
 * toward n_sel; the remaining slots take the highest group scores (compressed-
 * branch probabilities folded onto l'-blocks by token overlap / l and summed
 * over the group's heads), equal scores to the lower block id; if J+1 <= n_sel
 * all candidates are taken.
 */
nsa_status_t nsa_decode_fwd(const nsa_dims_t* dims, const nsa_config_t* cfg,
                            const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                            const uint16_t* k_cmp_cache, const uint16_t* v_cmp_cache,
                            const int32_t* seq_lens, const int64_t* cu_seqlens, const int64_t* cu_cmp,
                            int64_t max_seq_len, const float* gates,
                            const uint16_t* w_gate, const float* b_gate, uint16_t* out,
                            int32_t* sel_idx_out, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * nsa_decode_fwd_noalloc — nsa_decode_fwd without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Arguments, layouts,
 * validation and results are those of nsa_decode_fwd (the same kernels run);
 * the workspace is instead a fixed array of 32 MiB that the library holds in
 * device memory, one copy per GPU, until the process ends.  The call allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine).
 *
 * A step whose workspace (nsa_decode_workspace_size) exceeds 32 MiB returns
 * NSA_ERROR_UNSUPPORTED with the sizes in nsa_last_error(); the 64k / batch 8,
 * 128k / batch 4 and ragged 16-sequence workloads need 5.5, 4.5 and 19.6 MiB.
 * Every call on a GPU shares that GPU's array and nothing in it needs to start
 * at a particular value, but calls that overlap in time on one GPU (other
 * streams, other threads) race on it: order them on one stream.
 */
nsa_status_t nsa_decode_fwd_noalloc(const nsa_dims_t* dims, const nsa_config_t* cfg,
                                    const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                    const uint16_t* k_cmp_cache, const uint16_t* v_cmp_cache,
                                    const int32_t* seq_lens, const int64_t* cu_seqlens, const int64_t* cu_cmp,
                                    int64_t max_seq_len, const float* gates,
                                    const uint16_t* w_gate, const float* b_gate, uint16_t* out,
                                    int32_t* sel_idx_out, void* stream);

/*
 * nsa_prefill_fwd — causal prefill of B sequences of seq_len tokens each: every
 * position t attends per the three branches (compressed blocks whose last token
 * is <= t; the selected blocks' tokens <= t; the window t-w < x <= t).
 *
 *   q      bf16 [B, T, Hq, d_k]
 *   k, v   bf16 [B, Hkv, T, d_k] and [B, Hkv, T, d_v]
 *   k_cmp, v_cmp  bf16 [B, Hkv, floor((T-l)/d)+1, D] precomputed compressed
 *          cache, or both NULL to compress in the call from (w_k, pe_k, w_v,
 *          pe_v) into the workspace (the weights are ignored otherwise).
 *   gates  float32 [B, T, Hq, 3], or NULL with the gate network
 *   w_gate, b_gate  the gate network as for nsa_decode_fwd (q is [B, T, Hq, d_k]
 *          here, and the gates of position t come from q[b, t, h, :])
 *   out    bf16 [B, T, Hq, d_v]
 *   sel_idx_out  nullable int32 [B, T, Hkv, n_sel], ascending, -1 padded.
 *   lse_out  nullable float32 [B, T, Hq, 3]: each branch's log-sum-exp of its
 *          scaled logits, natural log, c = cmp, slc, win (what a training step
 *          keeps from the forward); -inf for a branch with no key (the
 *          compressed branch before the first complete block).  The window and
 *          selected sums are those of the bf16 probabilities the value products
 *          use, the compressed sum is fp32.
 */
nsa_status_t nsa_prefill_fwd(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t seq_len,
                             const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const uint16_t* k_cmp, const uint16_t* v_cmp,
                             const uint16_t* w_k, const uint16_t* pe_k,
                             const uint16_t* w_v, const uint16_t* pe_v,
                             const float* gates, const uint16_t* w_gate, const float* b_gate,
                             uint16_t* out, int32_t* sel_idx_out, float* lse_out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * DeepSeek Sparse Attention (DSA) decode step — lesson 5.5/02 "Разреженное
 * внимание — NSA и DSA" (ai.flicky.cc), section "DSA: молниеносный индексатор",
 * and the selection rules of its practice spec (topk_mask: only past keys, all
 * of them when fewer than k).  For each sequence b, with t = seq_lens[b] - 1:
 *
 *   indexer   I[s] = sum_j w_idx[b, j] * ReLU(q_idx[b, j] . k_idx[b, s]),  s <= t
 *             (idx_heads small heads of idx_dim FP8 numbers, no softmax);
 *   selection the top_k positions with the largest I (ties to the lower
 *             position); every position 0..t when t + 1 <= top_k;
 *   attention MLA in MQA mode: every query head h attends the selected
 *             positions' shared latent vectors c[s] (d_qk numbers):
 *             out[b, h] = softmax_s(scale * q[b, h] . c[s]) . c[s][0 : d_v].
 *
 * Supported: d_qk = 576, d_v = 512 (the 576-number latent, its first 512 numbers
 * the values); num_heads a multiple of 32 up to 256; idx_heads in {16, 32, 64};
 * idx_dim in {64, 128}; 1 <= top_k <= 4096; 1 <= cache_len <= 65536.
 *
 *   q         bf16 [B, num_heads, d_qk]
 *   q_idx     FP8 E4M3 (OCP: bias 7, no infinities, max 448) [B, idx_heads, idx_dim]
 *   w_idx     float32 [B, idx_heads]
 *   latent    bf16 [B, cache_len, d_qk]      (token-major: each token contiguous)
 *   k_idx     FP8 E4M3 [B, cache_len, idx_dim]
 *   seq_lens  int32 [B] on the device, 1 <= seq_lens[b] <= cache_len
 *   softmax_scale  0 selects 1/sqrt(d_qk)
 *   out       bf16 [B, num_heads, d_v]
 *   sel_idx_out    nullable int32 [B, top_k]: the selected positions, ascending,
 *             -1 padded when t + 1 < top_k.
 * Indexer scores are fp32 (exact FP8 products, fp32 sums); attention is bf16
 * MFMA with fp32 accumulation.  With nsa_set_phase_events, events[0..3] are
 * recorded before the indexer, after it, after the selection and at the end.
 */
typedef struct {
  int32_t batch;
  int32_t num_heads;   /* query heads, all sharing one latent per token */
  int32_t d_qk;        /* latent length: the logit dims */
  int32_t d_v;         /* value dims: the first d_v latent numbers */
  int32_t idx_heads;   /* indexer heads */
  int32_t idx_dim;     /* indexer query / key length */
} nsa_dsa_dims_t;
nsa_status_t nsa_dsa_decode_fwd(const nsa_dsa_dims_t* dims, int32_t top_k, float softmax_scale,
                                const uint16_t* q, const uint8_t* q_idx, const float* w_idx,
                                const uint16_t* latent, const uint8_t* k_idx,
                                const int32_t* seq_lens, int64_t cache_len,
                                uint16_t* out, int32_t* sel_idx_out,
                                void* workspace, size_t workspace_bytes, void* stream);
/* Workspace bytes for nsa_dsa_decode_fwd (host-only): fp32 scores [B, cache_len]
 * (row stride cache_len rounded up to 4, at offset 0), a selection buffer
 * [B, top_k], the attention partials, and the top-k's counters, position
 * bitmap and candidate list.  Its contents on entry do not matter. */
nsa_status_t nsa_dsa_decode_workspace_size(const nsa_dsa_dims_t* dims, int32_t top_k, int64_t cache_len,
                                           size_t* bytes);

/* Workspace bytes needed by nsa_decode_fwd / nsa_prefill_fwd for these sizes
 * (host-only; no device call).  `compress_in_call` = 1 when k_cmp/v_cmp will be
 * NULL.  Returns NSA_SUCCESS and writes *bytes, or a validation error.  Prefill
 * always needs a workspace: it holds the fp32 partial output [B, T, Hq, d_v] of
 * the compressed and window branches, a selection buffer [B, T, Hkv, n_sel] and,
 * with in-call compression, the compressed cache.  Prefill supports at most
 * 1024 selection blocks per sequence ((seq_len - 1) / l' + 1 <= 1024). */
nsa_status_t nsa_decode_workspace_size(const nsa_dims_t* dims, const nsa_config_t* cfg,
                                       int64_t max_seq_len, size_t* bytes);
nsa_status_t nsa_prefill_workspace_size(const nsa_dims_t* dims, const nsa_config_t* cfg,
                                        int64_t seq_len, int32_t compress_in_call, size_t* bytes);

/*
 * nsa_prefill_bwd — gradients of the causal prefill for training.  The pages fix
 * what flows where ("Native Sparse Attention (DeepSeek NSA)" lesson, the section
 * on native trainability): the top-n choice only picks which blocks are read and
 * is held constant, the compressed branch passes gradient to the compressed
 * cache, the selected and window branches to the raw keys and values; the
 * output is sum_c g_c o_c ("NSA: три ветви").  For every position t, head h
 * and branch c (softmax o_c over the branch's keys, lse_c its log-sum-exp):
 *   dgates[t, h, c] = dout . o_c
 *   dq    = s sum_c sum_k P (g_c dout.v_k - g_c dout.o_c) k
 *   dk, dv (raw) from the selected and window branches; dk_cmp, dv_cmp from the
 *   compressed branch (feed them to nsa_compress_bwd for the compression MLP).
 * The branch statistics (lse_c, D_c = g_c dout . o_c) are kept in the workspace
 * for the key-side kernels.  With nsa_set_phase_events
 * the events mark: before the query-side kernel, after it, after the raw-key
 * kernels, after the compressed-key kernel.
 *
 *   q, k, v, k_cmp, v_cmp  as for nsa_prefill_fwd; the compressed cache is the
 *          one the forward used (required when seq_len >= l).
 *   gates  float32 [B, T, Hq, 3] the forward's gate values, or NULL with
 *   w_gate, b_gate  the forward's gate network (as for nsa_prefill_fwd): the
 *          gates are recomputed, dq gains the gates' path sum_c dz_c w_gate[h, c]
 *          with dz_c = dgates_c g_c (1 - g_c), and dw_gate = sum_t dz q,
 *          db_gate = sum_t dz are written.  Exactly one gate source.
 *   sel_idx  int32 [B, T, Hkv, n_sel]: the forward's sel_idx_out (ascending,
 *          -1 padded; any other content gives undefined gradients).
 *   lse    nullable float32 [B, T, Hq, 3]: the forward's lse_out.  Given, the
 *          query side walks the key tiles once (P = exp(s q.k - lse); D_c =
 *          g_c sum P dP accumulates beside dq); NULL recomputes each branch's
 *          softmax in a first pass.
 *   dout   bf16 [B, T, Hq, d_v] gradient of the output.
 *   dq     float32 [B, T, Hq, d_k]             (written)
 *   dk, dv float32 [B, Hkv, T, d_k / d_v]       (written)
 *   dk_cmp, dv_cmp  float32 [B, Hkv, nc, d_k / d_v], nc = floor((T-l)/d)+1
 *          (written; may be NULL when T < l)
 *   dgates float32 [B, T, Hq, 3]               (written; the gradient of the gate values)
 *   dw_gate, db_gate  float32 [Hq, 3, d_k] and [Hq, 3] (written; required with
 *          w_gate, db_gate with b_gate; ignored otherwise)
 * Supported: the shapes of nsa_prefill_fwd with seq_len * Hq * max(d_k, d_v) * 2
 * below 2^32 (one sequence's query rows addressable with 32-bit offsets).
 * Products are bf16 MFMA with fp32 sums (probabilities and dS rounded to bf16
 * as operands).  Partial sums are combined in a fixed order (no atomics), so
 * repeated calls give identical bits.
 */
nsa_status_t nsa_prefill_bwd(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t seq_len,
                             const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const uint16_t* k_cmp, const uint16_t* v_cmp,
                             const float* gates, const uint16_t* w_gate, const float* b_gate,
                             const int32_t* sel_idx, const float* lse, const uint16_t* dout,
                             float* dq, float* dk, float* dv, float* dk_cmp, float* dv_cmp,
                             float* dgates, float* dw_gate, float* db_gate,
                             void* workspace, size_t workspace_bytes, void* stream);
/* Workspace bytes for nsa_prefill_bwd (host-only): per (branch, position, KV
 * group) a record of 48 fp32 (the heads' log-sum-exp, D and gate, padded to 16
 * heads), [3, B, T, Hkv, 48]; a selection bitmap [B, Hkv, ceil(T/l_sel),
 * ceil(T/32)] uint32; the key side's fp32 partial sums: [B*Hkv, S, 64, d_k + d_v]
 * for the selected branch with S = ceil(T/64) + ceil(T * n_sel * max(1, l_sel/64)
 * / 512) (one slot per 512 positions of a 64-key tile), and [P_c, B, Hkv, nc,
 * d_k + d_v] for the compressed branch, P_c = ceil(T / q), q = max(1024,
 * ceil(T/32)) rounded up to even (at most 32); per-tile counts [B*Hkv,
 * ceil(T/64)] and slot offsets [B*Hkv, ceil(T/64) + 1] int32; and the gate
 * network's gradient partials [64, Hq, 3, d_k + 1].  Each part is rounded up
 * to 256 bytes.  Contents on entry do not matter. */
nsa_status_t nsa_prefill_bwd_workspace_size(const nsa_dims_t* dims, const nsa_config_t* cfg,
                                            int64_t seq_len, size_t* bytes);

/*
 * nsa_compress_bwd — backward of nsa_compress_kv for one cache (which = 0:
 * keys with w_k, pe_k, d_k; which = 1: values with w_v, pe_v, d_v), dense layout
 * of nsa_prefill_fwd ([B, Hkv, T, D] raw rows, [B, Hkv, nc, D] compressed rows).
 * With X_i = (x[i*d : i*d+l] + pe) flattened and y_i = X_i w ("NSA: три ветви",
 * compressed branch; "Build it" step 1 of the NSA lesson):
 *   dx[t] += sum over the blocks i covering t of (dy_i w^T)[t - i*d]   (added)
 *   dw     = sum_i X_i^T dy_i                                           (written)
 *   dpe    = sum_i dy_i w^T                                             (written)
 * summed over all sequences and heads with fp32 accumulation in a fixed order
 * (run-to-run identical); in the products dy enters as bf16 high + low parts
 * (about 2^-16 relative).  The bf16 rounding of the forward's compressed rows is
 * taken as the identity.
 *   x      bf16 raw rows; w bf16 [l*D, D]; pe bf16 [l, D]
 *   dy     float32 [B, Hkv, nc, D] (e.g. nsa_prefill_bwd's dk_cmp); may be NULL when T < l
 *   dx     float32 [B, Hkv, T, D], accumulated into (e.g. nsa_prefill_bwd's dk)
 *   dw     float32 [l*D, D]; dpe float32 [l, D]
 */
nsa_status_t nsa_compress_bwd(const nsa_dims_t* dims, const nsa_config_t* cfg, int64_t seq_len,
                              int32_t which, const uint16_t* x, const uint16_t* w, const uint16_t* pe,
                              const float* dy, float* dx, float* dw, float* dpe,
                              void* workspace, size_t workspace_bytes, void* stream);
/* Workspace bytes for nsa_compress_bwd (host-only): 64 x D fp32 partial column
 * sums and 8 partial products [8, l*D, D] fp32 of dw, each part rounded up to
 * 256 bytes (independent of seq_len). */
nsa_status_t nsa_compress_bwd_workspace_size(const nsa_dims_t* dims, const nsa_config_t* cfg,
                                             int64_t seq_len, int32_t which, size_t* bytes);

/* Profiling hook: until called again on this thread, every nsa_decode_fwd,
 * nsa_prefill_fwd and nsa_prefill_bwd on this thread records the caller-owned hipEvent_t handles
 * events[0..3] on the call's stream between its kernels, so a caller can time
 * each kernel with hipEventElapsedTime:
 *   decode:  events[0] / events[1] are the start / stop events of the
 *            streaming kernel's dispatch (compressed branch with the folded
 *            selection scores, and the window branch), events[2] / events[3]
 *            those of the selection kernel (top-n, the selected blocks, the
 *            exact merge and the gated sum), so each pair times one kernel;
 *   prefill: before the in-call compression, after it (or right away when the
 *            cache is given), after the compressed + window + top-n kernel, after
 *            the selected-branch kernel (which writes the gated sum);
 *   prefill backward: before the query-side kernel (dq and the branch
 *            statistics), after it, after the raw-key kernels (window and
 *            selected branches), after the compressed-key kernel.
 * count = 0 (the default) records nothing; any count other than 0 or 4, or a
 * NULL handle, is NSA_ERROR_INVALID_VALUE.  The array is copied; the events are
 * not. */
nsa_status_t nsa_set_phase_events(void* const* events, int32_t count);

/*
 * nsa_set_phase_clock — profiling hook for this thread's nsa_decode_fwd and
 * nsa_dsa_decode_fwd calls: thread 0 of every workgroup of two of a step's
 * kernels writes the device's constant 100 MHz clock (uint64 ticks) at
 * numbered points of the kernel into `buffer` (device memory, at least
 * 2 * 4096 * 16 * 8 = 1 MiB): kernel k's workgroup w writes entries
 * [(k * 4096 + w) * 16, ... + 16).  For the NSA decode step:
 *   kernel 0 (compressed stream): 0 start, 1 last tile computed (wave 0), 3 every wave done,
 *   4 outputs merged, 2 outputs stored;
 *   kernel 1 (selection): 0 start, 1 first loads arrived, 2 group scores ready,
 *            3 top-n done, 4 selected and window steps computed, 5 partials
 *            stored, 6 (last workgroup of a (sequence, group) only) merge
 *            begins, 7 output written;
 * and of the DSA step:
 *   kernel 0 (top-k, one workgroup per 4096-score chunk): 0 start,
 *            1 sampled bound found, 2 chunk counted and arrived; the last
 *            workgroup of a sequence: 3 candidates loaded (bounded path),
 *            4 position bitmaps built, 5 positions written (bounded path) or
 *            6 (select over every score); 1..6 only when the sequence has more
 *            than top_k positions;
 *   kernel 1 (attention): 0 start, 1 positions and queries loaded, 2 first
 *            tile staged, 3 every tile done, 4 partial stored.
 * Entries of workgroups that end early are not written.  Nothing is recorded
 * when a kernel has more than 4096 workgroups.  buffer NULL or bytes 0
 * disables it (the default); a smaller buffer is NSA_ERROR_WORKSPACE.  The
 * buffer is borrowed until the last recording call has finished on its stream.
 */
nsa_status_t nsa_set_phase_clock(void* buffer, size_t bytes);

/* Human-readable name of a status code (static storage). */
const char* nsa_status_string(nsa_status_t status);
/* Message of the last failed call on this thread ("" if none). */
const char* nsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NSA_H_ */

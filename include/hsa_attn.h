/*
 * hsa_attn.h - C ABI of the gfx950 (MI355X) hierarchical sparse attention
 * forward library, libhsa_attn.so.
 *
 * The method (sources are web pages, cited by title and section):
 *  [HSA]  "Understanding and Improving Length Generalization in Hierarchical
 *         Sparse Attention Models" (ai.info summary of arXiv 2510.17196),
 *         Methodology: the sequence is split into chunks of S tokens, each
 *         chunk gets a landmark vector, and each query retrieves the top-K
 *         chunks (S = 64, K = 8 by default).
 *  [HiLS] mlsift "length extrapolation" page, HiLS abstract: the query
 *         attends independently inside each retrieved chunk and the chunk
 *         outputs are fused according to the chunk retrieval scores.
 *  [DHSA] pith.science review of arXiv 2510.24606, "What carries the
 *         argument" and Referee report (Eq. 4, tiling rule, Algorithm 1):
 *         variable-length chunks, sqrt|C|-scaled mean pooling of queries and
 *         keys, chunk similarity S_c, tiled to a token map S_t, top-N_b
 *         preceding keys per query, masked softmax attention.
 *
 * Conventions shared by every entry point
 *  - Device pointers unless stated otherwise.  Tensors are contiguous and
 *    head-major: Q [B,Hq,L,d], K and V [B,Hkv,L,d].  Query head h belongs to
 *    KV group g = h / (Hq/Hkv); Hq must be a multiple of Hkv.
 *  - dtype is HSA_DTYPE_BF16 or HSA_DTYPE_F32 for Q, K, V and the output;
 *    landmarks are always fp32; indices are int32.  Head dim d is 64 or 128.
 *  - A landmark is (sum of the chunk's S keys) / sqrt(S), the sqrt(S)-scaled
 *    mean.  Retrieval scores and in-chunk logits both scale by 1/sqrt(d).
 *  - Chunk c is available to query position t when (c+1)*S <= t (all of its
 *    tokens precede t).  A trailing partial chunk is never available.  A
 *    query with no available chunk outputs zeros.
 *  - The selection of a KV group is shared by its query heads and ranks the
 *    sum of their per-head scores; ties go to the lower chunk index.  Each
 *    head fuses the chunk outputs with a softmax over its own per-head scores
 *    of the selected chunks.
 *  - Ownership: the caller allocates and frees every buffer, the workspace
 *    included.  The library allocates no device memory and keeps no global
 *    mutable state, except the fixed scratch array of hsa_decode_noalloc.  A workspace's contents on entry do not matter: each
 *    call clears, in its own launches, whatever it accumulates into, and
 *    results repeat bit for bit from call to call (the backward above 4096
 *    chunks excepted; see there).  All work is enqueued asynchronously on `stream` (a
 *    hipStream_t, NULL = default stream); the library never synchronises.
 *  - Errors: arguments are validated on the host before anything is
 *    enqueued, so any status other than HSA_OK / HSA_ERR_HIP means nothing
 *    was launched.  HSA_ERR_HIP reports a failed launch; the HIP message is
 *    kept for the calling thread (hsa_last_error_message).  No C++ exception
 *    crosses this boundary.
 */
#ifndef HSA_ATTN_H
#define HSA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hsa_stream_t; /* the same handle as hipStream_t */

typedef enum {
  HSA_OK = 0,
  HSA_ERR_INVALID_ARGUMENT = 1,    /* bad size, null required pointer, ... */
  HSA_ERR_UNSUPPORTED = 2,         /* valid request this build does not run */
  HSA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the *_size value */
  HSA_ERR_HIP = 4,                 /* a HIP call failed */
} hsa_status_t;

typedef enum {
  HSA_DTYPE_F32 = 0,
  HSA_DTYPE_BF16 = 1,
} hsa_dtype_t;

/* Static description of a status code. */
const char* hsa_status_string(hsa_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* hsa_last_error_message(void);

/*
 * Landmark pooling ([HSA] Methodology; sqrt-scaled mean as in [DHSA] Eq. 4).
 *   K    [B,Hkv,L,d] dtype, read only.
 *   lmk  [B,Hkv,L/S,d] fp32, written for chunks chunk_begin .. chunk_end-1
 *        only (0 <= chunk_begin <= chunk_end <= L/S), so a decode cache can
 *        append landmarks as chunks complete.
 * lmk[b,g,c,:] = sum_{j<S} K[b,g,c*S+j,:] / sqrt(S).
 */
hsa_status_t hsa_build_landmarks(const void* K, float* lmk, int B, int Hkv, int64_t L, int d,
                                 int S, int64_t chunk_begin, int64_t chunk_end,
                                 hsa_dtype_t dtype, hsa_stream_t stream);

/*
 * HSA prefill (every query position of the sequence).  [HSA] Methodology,
 * [HiLS] abstract.
 *   Q [B,Hq,L,d], K, V [B,Hkv,L,d]: dtype, read only.
 *   lmk     fp32 [B,Hkv,L/S,d] landmarks, or NULL to build them in the
 *           workspace from K.
 *   O       [B,Hq,L,d] dtype, written.
 *   sel_idx int32 [B,Hkv,L,topk] or NULL: selected chunks of each query in
 *           rank order (score desc, index asc), -1 padded.
 *   sel_w   fp32 [B,Hq,L,topk] or NULL: fusion weights in the same order,
 *           0 padded.
 *   workspace of at least hsa_prefill_workspace_size(...) bytes, 256-byte
 *   aligned; its contents on entry do not matter.
 * Limits: 1 <= S <= 1024, 1 <= topk <= 32, B*Hq*L*topk < 2^31, L < 2^26,
 * Hq/Hkv <= 32.
 */
size_t hsa_prefill_workspace_size(int B, int64_t L, int Hq, int Hkv, int d, int S, int topk,
                                  hsa_dtype_t dtype);
hsa_status_t hsa_prefill(const void* Q, const void* K, const void* V, const float* lmk,
                         void* O, int32_t* sel_idx, float* sel_w, int B, int64_t L, int Hq,
                         int Hkv, int d, int S, int topk, hsa_dtype_t dtype, void* workspace,
                         size_t workspace_bytes, hsa_stream_t stream);

/*
 * HSA prefill with retrieval every R tokens ([HSA] Key Contributions 4,
 * Main Findings: per-token vs per-8-token retrieval).  Token t reuses the
 * chunk selection made at the first token of its block, t0 = floor(t/R)*R:
 * the chunks fully before t0, ranked by the group sum of q_t0 . lmk / sqrt(d)
 * (ties: lower index).  Each token then attends inside those chunks with its
 * own query and fuses the chunk outputs by a softmax over its own per-head
 * scores, as in hsa_prefill; R = 1 is hsa_prefill.
 *   sel_idx int32 [B,Hkv,ceil(L/R),topk] or NULL: the selection of each
 *          block (rank order, -1 padded).
 *   sel_w  fp32 [B,Hq,L,topk] or NULL: each token's fusion weights.
 * Other arguments, limits and errors as hsa_prefill; interval >= 1.
 */
size_t hsa_prefill_interval_workspace_size(int B, int64_t L, int Hq, int Hkv, int d, int S,
                                           int topk, int interval, hsa_dtype_t dtype);
hsa_status_t hsa_prefill_interval(const void* Q, const void* K, const void* V, const float* lmk,
                                  void* O, int32_t* sel_idx, float* sel_w, int B, int64_t L,
                                  int Hq, int Hkv, int d, int S, int topk, int interval,
                                  hsa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                  hsa_stream_t stream);

/*
 * HSA prefill backward ([HiLS] abstract: retrieval learned end to end, the
 * gradient reaching the retrieval scores through the fusion weights).
 * Gradients of sum(dO * O), O the output of hsa_prefill on the same inputs,
 * with respect to Q, K and V.  The top-K selection is piecewise constant in
 * the inputs and is held fixed; every other step is differentiated: the
 * fusion softmax, the attention inside each chunk, the retrieval scores
 * q . lambda_c / sqrt(d) and the landmark pooling lambda_c = sum_j k_j /
 * sqrt(S).
 *   Q, dO [B,Hq,L,d], K, V [B,Hkv,L,d] bf16, read only.
 *   lmk   fp32 [B,Hkv,L/S,d] landmarks of K, or NULL to build them.
 *   dQ [B,Hq,L,d], dK, dV [B,Hkv,L,d] bf16, written.
 *   workspace of at least hsa_prefill_backward_workspace_size(...) bytes.
 * Limits: as hsa_prefill, plus bf16 only and S <= 64 (HSA_ERR_UNSUPPORTED
 * otherwise).  Gradients are accumulated in fp32 in a fixed order (each
 * chunk's rows in token order), so they repeat bit for bit; above 4096
 * chunks (L / S > 4096) a chunk's rows follow atomic arrival instead, and
 * dK, dV may then differ from run to run in their last bits.
 */
size_t hsa_prefill_backward_workspace_size(int B, int64_t L, int Hq, int Hkv, int d, int S,
                                           int topk, hsa_dtype_t dtype);
hsa_status_t hsa_prefill_backward(const void* Q, const void* K, const void* V, const void* dO,
                                  const float* lmk, void* dQ, void* dK, void* dV, int B,
                                  int64_t L, int Hq, int Hkv, int d, int S, int topk,
                                  hsa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                  hsa_stream_t stream);

/*
 * HSA decode: one new query per sequence at position n_ctx, attending a KV
 * cache of capacity n_max tokens whose first n_ctx are valid.  All
 * floor(n_ctx/S) complete chunks are available.
 *   q      [B,Hq,d] dtype.
 *   Kc, Vc [B,Hkv,n_max,d] dtype (64-bit addressing: a group's slab may
 *          exceed 4 GiB).
 *   lmk    fp32 [B,Hkv,n_max/S,d]; entries of the first floor(n_ctx/S)
 *          chunks are read (see hsa_build_landmarks).
 *   o      [B,Hq,d] dtype, written.
 *   sel_idx int32 [B,Hkv,topk] or NULL, sel_w fp32 [B,Hq,topk] or NULL, as
 *          in hsa_prefill.
 * Limits: 1 <= S <= 1024, 1 <= topk <= 32, n_ctx <= n_max, Hq/Hkv <= 32.
 */
size_t hsa_decode_workspace_size(int B, int Hq, int Hkv, int d, int S, int topk,
                                 int64_t n_ctx);
hsa_status_t hsa_decode(const void* q, const void* Kc, const void* Vc, const float* lmk,
                        int64_t n_ctx, int64_t n_max, void* o, int32_t* sel_idx, float* sel_w,
                        int B, int Hq, int Hkv, int d, int S, int topk, hsa_dtype_t dtype,
                        void* workspace, size_t workspace_bytes, hsa_stream_t stream);

/*
 * hsa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * arguments and results are hsa_decode's (the same kernels run); instead of
 * a caller workspace the call uses a fixed scratch array of
 * HSA_DECODE_NOALLOC_SCRATCH_BYTES in device memory that each GPU holds
 * from the first call on it until the process ends.  The scratch of the
 * current device is used, so `stream` must belong to the current device.
 * The call allocates and frees nothing (no hipMalloc, no library
 * allocation); the first call on a device looks up the array's address.
 *  - A shape whose hsa_decode_workspace_size exceeds the scratch size is
 *    rejected with HSA_ERR_UNSUPPORTED before anything is enqueued (16 MiB
 *    covers, e.g., batch 32 x 32/8 heads x 131,072 tokens at topk 8, which
 *    needs 4.4 MB, and batch 1 x 16/4 heads x 16M tokens at topk 16).
 *  - Every call on a GPU shares that GPU's array, and the array keeps the
 *    last call's contents (which no result depends on).  Calls that overlap
 *    on one GPU (two streams, two threads) race on it: serialise them.
 */
#define HSA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
hsa_status_t hsa_decode_noalloc(const void* q, const void* Kc, const void* Vc, const float* lmk,
                                int64_t n_ctx, int64_t n_max, void* o, int32_t* sel_idx,
                                float* sel_w, int B, int Hq, int Hkv, int d, int S, int topk,
                                hsa_dtype_t dtype, hsa_stream_t stream);

/*
 * DHSA prefill ([DHSA] "What carries the argument", Eq. 4, tiling rule,
 * Algorithm 1 top-N_b preceding keys).
 *   Q, K, V  [B,H,L,d] dtype (F32 or BF16; fp32 runs on the VALU in fp32,
 *            bf16 on the bf16 MFMA with fp32 accumulation).
 *   offsets  HOST int32 [n_chunks+1], 0 = b_0 < b_1 < ... < b_n = L: chunk l
 *            holds tokens b_l .. b_{l+1}-1; the same boundaries for every
 *            batch entry and head.
 *   budget   N_b >= 1 keys kept per query.
 *   O        [B,H,L,d] dtype, written.
 *   mask_bits  uint32 [B,H,L,ceil(L/32)] or NULL: bit j of row i set when
 *            key j is kept for query i (debug output; L*L/8 bytes per head).
 *   chunk_order int32 [B,H,n_chunks,n_chunks] or NULL: row l lists the key
 *            chunks 0..l by (S_c[l,k] desc, k asc), -1 padded.
 * Per query i in chunk l: q_hat_l = sum_{i in C_l} q_i / sqrt|C_l| (same for
 * k_hat), S_c[l,k] = q_hat_l . k_hat_k, every key j <= i scores
 * S_c[l, chunk(j)], the first min(N_b, i+1) keys in (score desc, j asc)
 * order are kept, and softmax(q.k/sqrt d) attention runs over them.
 * Limits: n_chunks <= 4096, B*H*n_chunks*n_chunks < 2^31.
 * The offsets are validated on the host and copied into the workspace on
 * `stream` from pageable memory: the call cannot be captured in a HIP graph
 * (dhsa_decode and dhsa_build_chunk_keys likewise).
 */
size_t dhsa_prefill_workspace_size(int B, int64_t L, int H, int d, int n_chunks,
                                   hsa_dtype_t dtype);
hsa_status_t dhsa_prefill(const void* Q, const void* K, const void* V, const int32_t* offsets,
                          int n_chunks, int64_t budget, void* O, uint32_t* mask_bits,
                          int32_t* chunk_order, int B, int64_t L, int H, int d,
                          hsa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                          hsa_stream_t stream);

/*
 * DHSA decode, pooled chunk keys ([DHSA] "What carries the argument", Eq. 4):
 * khat[b,h,k] = (sum of the keys of chunk k) / sqrt|C_k| for the complete
 * chunks k in [chunk_begin, chunk_end), the cache dhsa_decode scores the new
 * query against.  Append a chunk when it completes.
 *   K        [B,H,n_max,d] dtype key cache.
 *   khat     fp32 [B,H,n_cap,d], rows chunk_begin..chunk_end-1 written.
 *   offsets  HOST int32 [n_chunks+1]: 0 = b_0 < ... < b_n <= n_max.
 * The workspace (dhsa_chunk_keys_workspace_size(chunk_end - chunk_begin)
 * bytes) receives the boundaries of the range.
 */
size_t dhsa_chunk_keys_workspace_size(int n_chunks);
hsa_status_t dhsa_build_chunk_keys(const void* K, float* khat, const int32_t* offsets,
                                   int n_chunks, int chunk_begin, int chunk_end, int B, int H,
                                   int64_t n_max, int d, int n_cap, hsa_dtype_t dtype,
                                   void* workspace, size_t workspace_bytes, hsa_stream_t stream);

/*
 * DHSA decode ([DHSA] Referee report, minor comment on Algorithm 2: the
 * decode-time update in which the last chunk holds the current query): the
 * new query i = b_n + m - 1 sits in the current, partial chunk [b_n, i].
 * That chunk is pooled like any chunk over the tokens it holds so far:
 * q_hat = (sum of its m queries) / sqrt(m), k_hat likewise over keys b_n..i.
 * The n complete chunks (pooled keys from khat) and the current one are
 * scored by S_c = q_hat . k_hat, every key j <= i takes the score of its
 * chunk, the first min(N_b, i+1) keys in (score desc, j asc) order are kept
 * and softmax(q_i . k / sqrt d) attention runs over them; the result equals
 * dhsa_prefill's row i on the sequence cut at i+1.
 *   q_cur    [B,H,m,d] dtype: the current chunk's queries, the new one last.
 *   Kc, Vc   [B,H,n_max,d] dtype caches holding tokens 0..i (the new key and
 *            value included).
 *   khat     fp32 [B,H,n_cap,d] from dhsa_build_chunk_keys (rows 0..n-1).
 *   offsets  HOST int32 [n_chunks+1]: boundaries of the complete chunks.
 *   o        [B,H,d] dtype, written.
 *   chunk_order int32 [B,H,n_chunks+1] or NULL: the chunks by (S_c desc,
 *            index asc); index n_chunks is the current chunk.
 * Limits: n_chunks + 1 <= 4096, n_max < 2^31.  The workspace size depends on
 * the budget and the cache capacity n_max as passed to dhsa_decode.
 */
size_t dhsa_decode_workspace_size(int B, int H, int d, int n_chunks, int64_t budget,
                                  int64_t n_max);
hsa_status_t dhsa_decode(const void* q_cur, int m, const void* Kc, const void* Vc,
                         int64_t n_max, const float* khat, int n_cap, const int32_t* offsets,
                         int n_chunks, int64_t budget, void* o, int32_t* chunk_order, int B,
                         int H, int d, hsa_dtype_t dtype, void* workspace,
                         size_t workspace_bytes, hsa_stream_t stream);

/*
 * Sliding-window attention, the local attention of the upper layers ([HSA]
 * Methodology: upper layers pair local self-attention with the HSA module;
 * 512-token sliding windows by default).  A query at position t attends the
 * keys max(0, t-W+1) .. t of its KV head (query head h uses KV head
 * h / (Hq/Hkv)): o_t = softmax(q_t . k_j / sqrt d) v_j over that window.
 * The pages give no formula for how the layer merges this output with the
 * HSA output, so the two come from separate calls and the model combines
 * them (residual sum, the bypassing path, gating).
 *
 * swa_prefill: every position of the sequence.
 *   Q [B,Hq,L,d], K, V [B,Hkv,L,d] dtype, read only; O [B,Hq,L,d] written.
 *   W = window >= 1 (W >= L gives dense causal attention).
 * swa_decode: one new query per sequence at position pos (the position
 *   hsa_decode calls n_ctx).
 *   q [B,Hq,d]; Kc, Vc [B,Hkv,n_max,d] caches holding tokens 0..pos (the new
 *   key and value included); o [B,Hq,d] written.
 * Device pointers, row-major, caller-owned; no workspace.  Limits: d in
 * {64, 128}, Hq % Hkv == 0, B*Hq*L < 2^31 (prefill), 0 <= pos < n_max
 * (decode).  Invalid arguments return an error before anything is enqueued.
 * With profiling on, each call records one stage (0 attend).
 */
hsa_status_t swa_prefill(const void* Q, const void* K, const void* V, void* O, int B, int64_t L,
                         int Hq, int Hkv, int d, int64_t window, hsa_dtype_t dtype,
                         hsa_stream_t stream);
hsa_status_t swa_decode(const void* q, const void* Kc, const void* Vc, int64_t pos,
                        int64_t n_max, int64_t window, void* o, int B, int Hq, int Hkv, int d,
                        hsa_dtype_t dtype, hsa_stream_t stream);

/*
 * The upper layers' two attentions over a whole sequence ([HSA]
 * Methodology: upper layers pair local sliding-window self-attention, 512
 * tokens by default, with the HSA module): hsa_prefill's output O_hsa and
 * swa_prefill's output O_swa of the same Q, K, V.  After HSA's landmark,
 * selection and list stages, one launch runs both HSA's chunk attention and
 * the sliding-window attention (the HSA blocks move partial outputs and
 * gathered query rows; the window blocks are bound by MFMA issue and softmax
 * arithmetic; sharing the launch overlaps the two); then HSA's fusion.  The
 * combination of the two outputs is the caller's (the pages give no formula).
 *   Arguments as hsa_prefill plus window (>= 1) and O_swa [B,Hq,L,d];
 *   workspace of hsa_prefill_workspace_size(...) bytes.
 * The single launch needs bf16 and S <= 64; otherwise the two attentions run
 * as consecutive launches (same results).  Profiling stages: 0 landmarks,
 * 1 select, 2 invert, 3 attend (both), 4 fuse.
 */
hsa_status_t hsa_swa_prefill(const void* Q, const void* K, const void* V, const float* lmk,
                             int64_t window, void* O_hsa, void* O_swa, int32_t* sel_idx,
                             float* sel_w, int B, int64_t L, int Hq, int Hkv, int d, int S,
                             int topk, hsa_dtype_t dtype, void* workspace,
                             size_t workspace_bytes, hsa_stream_t stream);

/*
 * The upper layers' two attentions of one new query in one pass ([HSA]
 * Methodology: upper layers pair local sliding-window self-attention with
 * the HSA module): HSA decode (as hsa_decode: the query at position n_ctx
 * retrieves among the floor(n_ctx/S) complete chunks) and sliding-window
 * attention over the cache keys max(0, n_ctx-W+1) .. n_ctx (as swa_decode
 * with pos = n_ctx), written to two outputs.  The window's 64-key pieces
 * run as blocks of the same attention launch as the selected chunks (they
 * need no selection, so they start at once), and the fusion launch also
 * merges the pieces; the combination of the two outputs is the caller's
 * (the pages give no formula for it).
 *   q [B,Hq,d]; Kc, Vc [B,Hkv,n_max,d] holding tokens 0..n_ctx (n_ctx <
 *   n_max); lmk fp32 [B,Hkv,n_max/S,d]; o_hsa, o_swa [B,Hq,d] written;
 *   sel_idx, sel_w as in hsa_decode.
 * Limits: as hsa_decode, plus S <= 64 and min(window, n_ctx+1) <= 4096
 * (HSA_ERR_UNSUPPORTED otherwise).  Profiling stages: 0 scan, 1 attend
 * (chunks and window pieces), 2 fuse (both outputs).
 */
size_t hsa_swa_decode_workspace_size(int B, int Hq, int Hkv, int d, int S, int topk,
                                     int64_t n_ctx, int64_t window);
hsa_status_t hsa_swa_decode(const void* q, const void* Kc, const void* Vc, const float* lmk,
                            int64_t n_ctx, int64_t n_max, int64_t window, void* o_hsa,
                            void* o_swa, int32_t* sel_idx, float* sel_w, int B, int Hq, int Hkv,
                            int d, int S, int topk, hsa_dtype_t dtype, void* workspace,
                            size_t workspace_bytes, hsa_stream_t stream);

/*
 * Profiling aid (not part of the method).  While enabled on the calling
 * thread, each call of the entry points below records a HIP
 * event on its stream before each of its stages and one after the last:
 *   hsa_prefill : 0 landmarks, 1 select, 2 invert, 3 attend, 4 fuse
 *   hsa_decode  : 0 scan (landmark stream, per-slice top-K), 1 attend (merge
 *                 of the slices' candidates, one block per selected chunk),
 *                 2 fuse (softmax over the retrieval scores, weighted sum;
 *                 for chunks of at most 64 keys it runs inside the attend
 *                 launch, and this stage is empty)
 *   dhsa_prefill: 0 pool, 1 rank (S_c rows and their ranking), 2 attend,
 *                 3 mask
 *   dhsa_decode : 0 score (pooling, S_c, rank, cut), 1 attend, 2 combine
 *   swa_prefill, swa_decode: 0 attend
 *   hsa_prefill_backward: 0 landmarks, 1 select, 2 invert, 3 weights (fusion
 *                 weights), 4 score (log-sum-exp, dO . o_k, dQ pieces), 5 rows
 *                 (retrieval-score gradients), 6 kv (dK, dV), 7 finish (dQ)
 * hsa_profile_read waits for the recorded events, adds the elapsed
 * milliseconds of stage s summed over all recorded calls into stage_ms[s]
 * (s < max_stages; the caller zeroes the array), releases the events and
 * returns the number of calls; *n_stages receives the stage count.  The
 * events are host-side runtime objects; no device memory is allocated.
 */
hsa_status_t hsa_profile_enable(int enable);
int hsa_profile_read(double* stage_ms, int max_stages, int* n_stages);

/*
 * Debugging aids (not part of the method).
 *
 * HSA_ATTN_LOG set to a non-zero value in the environment (read once per
 * process): every entry point prints a line with its name and shapes to
 * stderr, every kernel launch a line with the kernel's name and template
 * arguments, grid, block and dynamic LDS bytes, and every rejected call its
 * status and message.
 *
 * The debug library (libhsa_attn_debug.so, built beside the release one with
 * device checks compiled in; the Python binding loads it when HSA_ATTN_DEBUG
 * is 1) checks the kernels' gather indices against the buffers they address:
 * a failed check is counted and the kernel carries on.  Each entry point of
 * that library then synchronises its stream and returns HSA_ERR_HIP with the
 * source file and line of the first failed check (the counters are cleared),
 * so it is for testing, not for capture into a graph.
 *
 * hsa_device_checks_enabled returns 1 in the debug library, 0 otherwise.
 * hsa_device_checks_selftest launches a one-thread kernel whose single check
 * fails when fail_check is non-zero (it touches no memory); the debug
 * library then returns HSA_ERR_HIP, the release library HSA_ERR_UNSUPPORTED.
 */
int hsa_device_checks_enabled(void);
hsa_status_t hsa_device_checks_selftest(int fail_check, hsa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HSA_ATTN_H */

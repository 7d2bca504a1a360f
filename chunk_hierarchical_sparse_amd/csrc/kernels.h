// kernels.h - host-side launchers of the gfx950 kernels (internal to
// libhsa_attn; the public interface is include/hsa_attn.h).
//
// Every launcher enqueues on `stream` and returns the hipError_t of the
// launch; argument validation has already happened in api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsa {

// Input element types.
enum : int { kF32 = 0, kBF16 = 1 };

// ---- shared ----------------------------------------------------------------
// HSA_ATTN_LOG set to a non-zero value in the environment: every entry point
// prints its shapes and every kernel launch its instantiated name, grid,
// block and dynamic LDS bytes to stderr (api.cpp).
bool launch_log_enabled();
void log_launch(const void* kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream);

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t stream);

// Device checks of the debug library (built with HSA_DEVICE_CHECKS=1, loaded
// when HSA_ATTN_DEBUG=1): each translation unit registers readers of its own
// check counters at load time, and each source file with checks its tag and
// path (hsa_common.h); after an entry point's launches the library
// synchronises the stream and reports the first failed check (api.cpp).  In
// the release library nothing registers.
typedef hipError_t (*CheckRead)(uint32_t counters[3]);  // failures, line, source tag
typedef hipError_t (*CheckClear)();
bool register_device_checks(CheckRead read, CheckClear clear);
bool register_check_source(uint32_t tag, const char* path);
// A one-block kernel whose single check fails when `fail` is non-zero
// (landmarks.hip); the debug library's self-test.
hipError_t launch_check_selftest(int fail, hipStream_t stream);

// Records `message` as the calling thread's last error (hsa_last_error_message)
// and returns `status` (an hsa_status_t value).
int api_error(int status, const char* message);

// ---- landmarks (landmarks.hip) ---------------------------------------------
// lmk[bh, c, :] = sum of rows c*S .. c*S+S-1 of K[bh] / sqrt(S), for chunks
// c0 <= c < c1.  K row stride is d; a (b,h) slab holds `slab_tokens` rows and
// lmk holds `lmk_chunks` chunks per (b,h).
hipError_t launch_landmarks(const void* K, int dtype, float* lmk, int64_t BH, int64_t slab_tokens,
                            int64_t lmk_chunks, int d, int S, int64_t c0, int64_t c1,
                            hipStream_t stream);

// ---- HSA prefill (prefill.hip) ---------------------------------------------
struct PrefillArgs {
  const void* Q;
  const void* K;
  const void* V;
  const float* lmk;   // [B,Hkv,n,d]
  void* O;            // [B,Hq,L,d]
  int32_t* idx;       // [B,Hkv,nq,topk]: selection of each selection row
  float* sel_w;       // [B,Hq,L,topk] or null
  int32_t* counts;    // [B*Hkv, n]
  int32_t* cursor;    // [B*Hkv, n]
  int32_t* blockbase; // [B*Hkv, ceil(L/kInvertTokens), n] when n <= kInvertDetBins: each
                      // counting block's per-chunk counts (ordered lists only)
  int32_t* offs;      // [B*Hkv, n+1]
  int32_t* tile_off;  // [B*Hkv, n+1]
  int32_t* tile_chunk;  // [B*Hkv, tiles_ub]: chunk of each attention work unit
  int32_t* list;      // [B*Hkv, L*topk]
  int32_t* entry_pos; // [B*Hkv, L*topk]: list position of selection (token, slot)
  void* partial;      // [B*Hkv, L*topk, G, d] in list order (bf16 or fp32 like the inputs)
  float* part_score;  // [B*Hkv, L*topk, G] in list order
  int B, Hq, Hkv, d, S, topk, dtype;
  int64_t L, n;
  int entries_per_tile;  // selection entries (token, slot) per attention work unit
  int64_t tiles_ub;      // upper bound of work units per (b, group)
  int log2G;             // log2(Hq/Hkv) when it is a power of two, else -1
  int interval;          // retrieval interval R: token t uses selection row t / R
  int64_t nq;            // selection rows, ceil(L / R)
  int ordered;           // build each chunk's list in token order (when n <= kInvertDetBins)
};
// A selection entry of the per-chunk lists: token << kSlotBits | slot.
constexpr int kSlotBits = 5;  // topk <= 32
// The per-chunk lists are built over blocks of kInvertTokens tokens.  The
// order inside a list follows atomic arrival, which no forward result
// depends on (every row is computed on its own).  With `ordered` set (the
// backward, whose dK and dV sum over a chunk's list) and up to
// kInvertDetBins chunks, the lists are in token order instead, so those
// sums run in a fixed order.
constexpr int kInvertTokens = 512;
constexpr int kInvertDetBins = 4096;
// prefill_select also clears counts and cursor; prefill_invert relies on
// that, so it runs right after prefill_select on the same stream.
hipError_t prefill_select(const PrefillArgs& a, hipStream_t stream);
hipError_t prefill_invert(const PrefillArgs& a, hipStream_t stream);
hipError_t prefill_attend(const PrefillArgs& a, hipStream_t stream);
hipError_t prefill_fuse(const PrefillArgs& a, hipStream_t stream);
int prefill_entries_per_tile(int dtype, int G, int S);
// Retrieval every R tokens with R * G == 32 (bf16, topk <= 8, S <= 64):
// the query-major path (prefill_qmajor.hip) replaces the invert, the
// chunk-major attention and the fusion.  `scratch` holds the landmarks split
// into three bf16 parts, prefill_query_major_scratch bytes.
bool prefill_query_major(const PrefillArgs& a);
size_t prefill_query_major_scratch(int64_t BHkv, int64_t n, int d);
hipError_t prefill_attend_query_major(const PrefillArgs& a, void* scratch, hipStream_t stream);

// ---- HSA decode (decode.hip) -----------------------------------------------
struct DecodeArgs {
  const void* q;       // [B,Hq,d]
  const void* Kc;      // [B,Hkv,n_max,d]
  const void* Vc;
  const float* lmk;    // [B,Hkv,n_max/S,d]
  void* o;             // [B,Hq,d]
  int32_t* sel;        // [B,Hkv,topk]
  float* sel_w;        // [B,Hq,topk] or null
  uint64_t* cand;      // [B*Hkv, n_slices, topk]
  uint64_t* cand_mm;   // [B*Hkv, n_slices, 2]: largest, smallest kept key (0 if not full)
  float* part_o;       // [B,Hq,topk,d]
  float* part_s;       // [B,Hq,topk]
  int B, Hq, Hkv, d, S, topk, dtype;
  int64_t n_ctx, n_max, n_avail, lmk_chunks;
  int n_slices, slice;
  // sliding-window attention of the same query in the same launches (0
  // pieces: none): keys [swa_lo, swa_hi) of the cache in pieces of 64
  int swa_pieces;
  int64_t swa_lo, swa_hi;
  void* o_swa;         // [B,Hq,d]
  float* sw_o;         // [B,Hq,swa_pieces,d]: each piece's normalised output
  float* sw_lse;       // [B,Hq,swa_pieces]: natural log-sum-exp of its logits
  // the decode with the fusion folded into the attention (decode_fused_*):
  // per (b, group), the attention blocks done (cleared by the scan)
  uint32_t* sync;      // [B*Hkv] or null
};
void decode_plan(int64_t n_avail, int topk, int64_t BHkv, int* n_slices, int* slice);
// Whether the folded decode takes these arguments (chunks of at most 64
// keys, some chunk available, a.sync set).
bool decode_fused_ok(const DecodeArgs& a);
// stages: 0 scan (also clears a.sync); 1 merge + attention, the last block
// of each (b, group) fusing its chunk outputs
constexpr int kDecodeFusedStages = 2;
hipError_t decode_fused_stage(const DecodeArgs& a, int stage, hipStream_t stream);
// stages: 0 scan (landmark stream + per-slice top-K), 1 attend (merge of the
// slices' candidates, then one block per selected chunk; with swa_pieces
// also one block per window piece), 2 fuse (softmax over the chunks'
// retrieval scores, weighted sum of the chunk outputs; the window pieces'
// softmax merge)
constexpr int kDecodeStages = 3;
hipError_t decode_stage(const DecodeArgs& a, int stage, hipStream_t stream);
int64_t decode_max_chunks(int topk);

// ---- DHSA prefill (dhsa.hip) -----------------------------------------------
struct DhsaArgs {
  const void* Q;          // [B,H,L,d]
  const void* K;
  const void* V;
  void* O;
  const int32_t* offs;    // device [nc+1]
  float* qh;              // [B,H,nc,d]
  float* kh;              // [B,H,nc,d]
  int32_t* order;         // [B,H,nc,nc]
  int32_t* cumlen;        // [B,H,nc,nc+1]
  int32_t* diag_pos;      // [B,H,nc]
  int32_t* ranked;        // [B,H,nc,nc,2]: (first key, length) of the chunk at each rank
  uint32_t* mask_bits;    // [B,H,L,ceil(L/32)] or null
  int B, H, d, dtype, nc, tiles_per_chunk;
  int64_t L, budget;
};
// stages: 0 pool, 1 rank (S_c rows and their ranking), 2 attend, 3 mask
// (only with mask_bits)
constexpr int kDhsaStages = 4;
hipError_t dhsa_stage(const DhsaArgs& a, int stage, hipStream_t stream);
int dhsa_max_chunks();

// ---- DHSA decode (dhsa_decode.hip) -----------------------------------------
struct DhsaDecodeArgs {
  const void* qcur;     // [B,H,m,d]: queries of the current chunk, last = new query
  const void* Kc;       // [B,H,n_max,d]
  const void* Vc;
  const float* khat;    // [B,H,n_cap,d]: pooled keys of the complete chunks
  void* o;              // [B,H,d]
  int32_t* chunk_order; // [B,H,n+1] or null
  const int32_t* offs;  // [n+1] device copy of the complete chunks' boundaries
  int32_t* plan;        // [B*H, max_pieces, 2]: (first token, count <= 64) of each piece
  int32_t* n_plan;      // [B*H]: pieces in use
  float* part;          // [B*H, max_pieces, d+2]: (max, sum, weighted values) per piece
  int B, H, d, dtype, n, n_cap, m, P, max_pieces;
  int64_t n_max, pos, budget;
};
// stages: 0 score (pooling, S_c, rank, cut), 1 attend, 2 combine
constexpr int kDhsaDecodeStages = 3;
// pieces of at most 64 keys the kept keys can need
int64_t dhsa_decode_max_pieces(int64_t keep_max, int n_chunks);
hipError_t dhsa_decode_stage(const DhsaDecodeArgs& a, int stage, hipStream_t stream);
hipError_t launch_dhsa_chunk_keys(const void* K, float* khat, const int32_t* offs, int dtype,
                                  int64_t BH, int64_t n_max, int d, int n_cap, int chunk_begin,
                                  int chunk_end, hipStream_t stream);

// ---- HSA prefill backward (prefill_bwd.hip) ---------------------------------
// Reuses the forward's work list (select + invert outputs in p), built with
// one work unit per chunk.  Per-row values live in list order at
// partial_row(); p.partial (bf16) receives each (row, slot)'s dQ piece.
struct PrefillBwdArgs {
  PrefillArgs p;
  const void* dO;   // [B,Hq,L,d]
  float* lse2;      // list order: log2-sum-exp2 of the row's chunk logits (log2 units)
  float* dw;        // list order: dO . o_k, the gradient of the row's fusion weight
  float* wk;        // list order: fusion weight w_k
  float* ds;        // list order: gradient of the row's retrieval score
  void* dQ;         // [B,Hq,L,d] outputs, dtype of the inputs
  void* dK;         // [B,Hkv,L,d]
  void* dV;
};
// stages after landmarks / select / invert: weights (wk), score (lse2, dw, dQ
// pieces), rows (ds), kv (dK, dV of every selected chunk, zero elsewhere),
// finish (dQ gather)
hipError_t prefill_bwd_weights(const PrefillBwdArgs& a, hipStream_t stream);
hipError_t prefill_bwd_score(const PrefillBwdArgs& a, hipStream_t stream);
hipError_t prefill_bwd_rows(const PrefillBwdArgs& a, hipStream_t stream);
hipError_t prefill_bwd_kv(const PrefillBwdArgs& a, hipStream_t stream);
hipError_t prefill_bwd_finish(const PrefillBwdArgs& a, hipStream_t stream);

// ---- sliding-window attention (swa.hip) ------------------------------------
struct SwaArgs {
  const void* Q;   // prefill [B,Hq,L,d]; decode [B,Hq,d]
  const void* K;   // [B,Hkv,L,d] (decode: the cache, L = its capacity)
  const void* V;
  void* O;         // like Q
  int B, Hq, Hkv, d, dtype;
  int64_t L;       // prefill: sequence length; decode: cache capacity n_max
  int64_t window;  // W >= 1: a query at t attends keys max(0, t-W+1) .. t
  int64_t n_ctx;   // decode: tokens in the cache, the new one at n_ctx - 1
};
hipError_t launch_swa_prefill(const SwaArgs& a, hipStream_t stream);
hipError_t launch_swa_decode(const SwaArgs& a, hipStream_t stream);

// ---- upper layers: HSA chunk attention and sliding-window prefill in one
// launch (upper.hip); bf16, chunks of at most 64 keys, the same Q/K/V -------
hipError_t launch_upper_attend(const PrefillArgs& pa, const SwaArgs& sa, hipStream_t stream);

}  // namespace hsa

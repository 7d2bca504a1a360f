// api.cpp - the C ABI of libhsa_attn (declared in include/hsa_attn.h):
// host-side argument validation, workspace carving, launch sequencing.
// Nothing is enqueued until every argument has been checked.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cxxabi.h>

#include <string>
#include <utility>
#include <vector>

#include "hsa_attn.h"
#include "kernels.h"

namespace hsa {

// Translation units of the debug library register their check counters,
// and source files with checks their tags, during static initialisation
// (hsa_common.h).
struct CheckSource {
  CheckRead read;
  CheckClear clear;
};

std::vector<CheckSource>& check_sources() {
  static std::vector<CheckSource> v;
  return v;
}

std::vector<std::pair<uint32_t, std::string>>& check_paths() {
  static std::vector<std::pair<uint32_t, std::string>> v;
  return v;
}

bool register_device_checks(CheckRead read, CheckClear clear) {
  check_sources().push_back({read, clear});
  return true;
}

bool register_check_source(uint32_t tag, const char* path) {
  check_paths().emplace_back(tag, path);
  return true;
}

std::string check_source_path(uint32_t tag) {
  for (const auto& p : check_paths())
    if (p.first == tag) {
      const size_t slash = p.second.rfind('/');
      return slash == std::string::npos ? p.second : p.second.substr(slash + 1);
    }
  return "unknown source";
}

}  // namespace hsa

namespace {

thread_local std::string g_err;

// Optional per-stage event timing of the calling thread (profiling aid).
struct Profile {
  bool on = false;
  std::vector<std::vector<hipEvent_t>> calls;
};
thread_local Profile g_prof;

// Records an event before each stage of one call and one after the last.
struct StageMarks {
  hipStream_t st;
  std::vector<hipEvent_t> ev;
  explicit StageMarks(hipStream_t s) : st(s) {}
  void mark() {
    if (!g_prof.on) return;
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return;
    if (hipEventRecord(e, st) != hipSuccess) {
      (void)hipEventDestroy(e);
      return;
    }
    ev.push_back(e);
  }
  ~StageMarks() {
    if (!ev.empty()) g_prof.calls.push_back(std::move(ev));
  }
};

// One line to stderr per entry-point call (its name and shapes) when
// HSA_ATTN_LOG is set; the kernels' launch lines follow it.
void log_call(const char* fmt, ...) {
  if (!hsa::launch_log_enabled()) return;
  char line[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof line, fmt, ap);
  va_end(ap);
  fprintf(stderr, "hsa_attn: %s\n", line);
}

hsa_status_t fail(hsa_status_t s, const std::string& msg) {
  g_err = msg;
  if (hsa::launch_log_enabled()) fprintf(stderr, "hsa_attn:   status %d: %s\n", (int)s, msg.c_str());
  return s;
}

hsa_status_t hip_fail(hipError_t e, const char* where) {
  return fail(HSA_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

// The end of every entry point that launched work.  In the debug library
// (device checks registered) the stream is synchronised and every kernel
// source's check counters are read; the first failure becomes HSA_ERR_HIP
// and the counters are cleared.  Otherwise HSA_OK.
hsa_status_t finish(hipStream_t stream) {
  if (hsa::check_sources().empty()) return HSA_OK;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "device checks: stream synchronise");
  std::string report;
  for (const auto& src : hsa::check_sources()) {
    uint32_t c[3] = {0u, 0u, 0u};
    if ((e = src.read(c)) != hipSuccess) return hip_fail(e, "device checks: read");
    if (c[0] == 0u) continue;
    if ((e = src.clear()) != hipSuccess) return hip_fail(e, "device checks: clear");
    if (report.empty())
      report = "device check failed at " + hsa::check_source_path(c[2]) + ":" +
               std::to_string(c[1]) + " (" + std::to_string(c[0]) + " failures)";
  }
  return report.empty() ? HSA_OK : fail(HSA_ERR_HIP, report);
}

bool dtype_ok(hsa_dtype_t dt) { return dt == HSA_DTYPE_F32 || dt == HSA_DTYPE_BF16; }
int elem_bytes(hsa_dtype_t dt) { return dt == HSA_DTYPE_F32 ? 4 : 2; }
int dt_code(hsa_dtype_t dt) { return dt == HSA_DTYPE_F32 ? hsa::kF32 : hsa::kBF16; }

constexpr size_t kAlign = 256;

// Carves aligned sub-buffers out of a workspace; with base == nullptr it
// only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

// Total (token, slot) selections of one (b, group) in prefill.
int64_t prefill_entries(int64_t L, int S, int topk) {
  const int64_t n = L / S;
  int64_t e = 0;
  for (int64_t c = 0; c < n; ++c) e += (int64_t)S * (c < topk ? c : topk);
  e += (L - n * S) * (n < topk ? n : topk);
  return e;
}

hsa_status_t check_prefill(int B, int64_t L, int Hq, int Hkv, int d, int S, int topk,
                           hsa_dtype_t dt) {
  if (!dtype_ok(dt)) return fail(HSA_ERR_UNSUPPORTED, "dtype must be F32 or BF16");
  if (B < 0 || L < 0) return fail(HSA_ERR_INVALID_ARGUMENT, "B and L must be >= 0");
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(HSA_ERR_INVALID_ARGUMENT, "Hq and Hkv must be positive with Hq % Hkv == 0");
  if (Hq / Hkv > 32) return fail(HSA_ERR_UNSUPPORTED, "Hq / Hkv must be <= 32");
  if (d != 64 && d != 128) return fail(HSA_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (S < 1 || S > 1024) return fail(HSA_ERR_INVALID_ARGUMENT, "chunk size S must be in [1, 1024]");
  if (topk < 1 || topk > 32) return fail(HSA_ERR_INVALID_ARGUMENT, "topk must be in [1, 32]");
  if ((int64_t)B * Hkv * L * topk >= (int64_t)1 << 31 ||
      (int64_t)B * Hq * L * topk >= (int64_t)1 << 31)
    return fail(HSA_ERR_UNSUPPORTED, "B*H*L*topk must be < 2^31");
  if (L >= ((int64_t)1 << 26)) return fail(HSA_ERR_UNSUPPORTED, "L must be < 2^26");
  return HSA_OK;
}

struct PrefillLayout {
  float* lmk;
  int32_t* idx;
  int32_t *counts, *cursor, *blockbase, *offs, *tile_off, *tile_chunk, *list, *entry_pos;
  int entries_per_tile;
  int64_t tiles_ub;
  void* partial;
  float* part_score;
  size_t bytes;
};

// entries_per_unit > 0 overrides the attention work-unit size (selection
// entries per unit).
PrefillLayout prefill_layout(void* ws, int B, int64_t L, int Hq, int Hkv, int d, int S,
                             int topk, hsa_dtype_t dt, int interval = 1,
                             int entries_per_unit = 0) {
  Carver cv(ws);
  PrefillLayout p;
  const int64_t n = L / S;
  const int64_t BG = (int64_t)B * Hkv;
  const int64_t nq = (L + interval - 1) / interval;
  p.lmk = cv.take<float>((size_t)(BG * n * d));
  p.idx = cv.take<int32_t>((size_t)(BG * nq * topk));
  p.counts = cv.take<int32_t>((size_t)(BG * n));
  p.cursor = cv.take<int32_t>((size_t)(BG * n));
  const int64_t inv_blocks = (L + hsa::kInvertTokens - 1) / hsa::kInvertTokens;
  p.blockbase = cv.take<int32_t>(n <= hsa::kInvertDetBins ? (size_t)(BG * inv_blocks * n) : 1);
  p.offs = cv.take<int32_t>((size_t)(BG * (n + 1)));
  p.tile_off = cv.take<int32_t>((size_t)(BG * (n + 1)));
  p.entries_per_tile = entries_per_unit > 0
                           ? entries_per_unit
                           : hsa::prefill_entries_per_tile(dt_code(dt), Hq / Hkv, S);
  p.tiles_ub = prefill_entries(L, S, topk) / p.entries_per_tile + n + 1;
  p.tile_chunk = cv.take<int32_t>((size_t)(BG * p.tiles_ub));
  p.list = cv.take<int32_t>((size_t)(BG * L * topk));
  p.entry_pos = cv.take<int32_t>((size_t)(BG * L * topk));
  p.partial = cv.take<char>((size_t)((int64_t)B * Hq * L * topk * d * elem_bytes(dt)));
  p.part_score = cv.take<float>((size_t)((int64_t)B * Hq * L * topk));
  p.bytes = cv.off + kAlign;
  return p;
}

// The backward's workspace: the forward's work list with one work unit per
// chunk (so a chunk's dK and dV are summed inside one block) and per-row
// values in list order.
struct BackwardLayout {
  PrefillLayout fwd;
  float *lse2, *dw, *wk, *ds;
  size_t bytes;
};

BackwardLayout backward_layout(void* ws, int B, int64_t L, int Hq, int Hkv, int d, int S,
                               int topk) {
  BackwardLayout p;
  // a token selects a chunk at most once: a chunk's list has at most L entries
  p.fwd = prefill_layout(ws, B, L, Hq, Hkv, d, S, topk, HSA_DTYPE_BF16, 1, (int)(L > 0 ? L : 1));
  Carver cv(ws);
  cv.off = p.fwd.bytes;
  const size_t rows = (size_t)B * Hq * L * topk;
  p.lse2 = cv.take<float>(rows);
  p.dw = cv.take<float>(rows);
  p.wk = cv.take<float>(rows);
  p.ds = cv.take<float>(rows);
  p.bytes = cv.off + kAlign;
  return p;
}

hsa_status_t check_decode(int B, int Hq, int Hkv, int d, int S, int topk, int64_t n_ctx,
                          int64_t n_max, hsa_dtype_t dt) {
  hsa_status_t s = check_prefill(B, 1, Hq, Hkv, d, S, topk, dt);
  if (s != HSA_OK) return s;
  if (n_ctx < 0 || n_max < n_ctx)
    return fail(HSA_ERR_INVALID_ARGUMENT, "need 0 <= n_ctx <= n_max");
  if (n_ctx / S > hsa::decode_max_chunks(topk))
    return fail(HSA_ERR_UNSUPPORTED, "too many chunks in the context for this topk");
  return HSA_OK;
}

struct DecodeLayout {
  uint64_t* cand;
  uint64_t* cand_mm;
  int32_t* sel;
  float* part_o;
  float* part_s;
  float* sw_o;
  float* sw_lse;
  uint32_t* sync;
  int n_slices, slice;
  size_t bytes;
};

// swa_pieces > 0: room for the window pieces of hsa_swa_decode as well.
DecodeLayout decode_layout(void* ws, int B, int Hq, int Hkv, int d, int S, int topk,
                           int64_t n_ctx, int swa_pieces = 0) {
  DecodeLayout p;
  hsa::decode_plan(n_ctx / S, topk, (int64_t)B * Hkv, &p.n_slices, &p.slice);
  Carver cv(ws);
  p.cand = cv.take<uint64_t>((size_t)B * Hkv * p.n_slices * topk);
  p.cand_mm = cv.take<uint64_t>((size_t)B * Hkv * p.n_slices * 2);
  p.sel = cv.take<int32_t>((size_t)B * Hkv * topk);
  p.part_o = cv.take<float>((size_t)B * Hq * topk * d);
  p.part_s = cv.take<float>((size_t)B * Hq * topk);
  p.sw_o = swa_pieces ? cv.take<float>((size_t)B * Hq * swa_pieces * d) : nullptr;
  p.sw_lse = swa_pieces ? cv.take<float>((size_t)B * Hq * swa_pieces) : nullptr;
  // per (b, group), the attention blocks done (the fusion's counter)
  p.sync = cv.take<uint32_t>((size_t)B * Hkv);
  p.bytes = cv.off + kAlign;
  return p;
}

constexpr int kSwaPieceKeys = 64;
constexpr int kSwaMaxPieces = 64;  // window of at most 4096 keys in the fused decode

int swa_decode_pieces(int64_t n_ctx, int64_t window) {
  const int64_t w = window < n_ctx + 1 ? window : n_ctx + 1;
  return (int)((w + kSwaPieceKeys - 1) / kSwaPieceKeys);
}

struct DhsaLayout {
  int32_t* offs;
  float *qh, *kh;
  int32_t *order, *cumlen, *diag_pos, *ranked;
  size_t bytes;
};

DhsaLayout dhsa_layout(void* ws, int B, int H, int d, int nc) {
  Carver cv(ws);
  DhsaLayout p;
  const int64_t BH = (int64_t)B * H;
  p.offs = cv.take<int32_t>((size_t)nc + 1);
  p.qh = cv.take<float>((size_t)(BH * nc * d));
  p.kh = cv.take<float>((size_t)(BH * nc * d));
  p.order = cv.take<int32_t>((size_t)(BH * nc * nc));
  p.cumlen = cv.take<int32_t>((size_t)(BH * nc * (nc + 1)));
  p.diag_pos = cv.take<int32_t>((size_t)(BH * nc));
  p.ranked = cv.take<int32_t>((size_t)(BH * nc * nc * 2));
  p.bytes = cv.off + kAlign;
  return p;
}

struct DhsaDecodeLayout {
  int32_t* offs;
  int32_t* plan;
  int32_t* n_plan;
  float* part;
  size_t bytes;
};

DhsaDecodeLayout dhsa_decode_layout(void* ws, int B, int H, int d, int n_chunks,
                                    int64_t max_pieces) {
  Carver cv(ws);
  DhsaDecodeLayout p;
  const int64_t BH = (int64_t)B * H, nc = (int64_t)n_chunks + 1;
  p.offs = cv.take<int32_t>((size_t)nc);
  p.plan = cv.take<int32_t>((size_t)(BH * max_pieces * 2));
  p.n_plan = cv.take<int32_t>((size_t)BH);
  p.part = cv.take<float>((size_t)(BH * max_pieces * (d + 2)));
  p.bytes = cv.off + kAlign;
  return p;
}

int64_t dhsa_decode_pieces(int n_chunks, int64_t budget, int64_t n_max) {
  return hsa::dhsa_decode_max_pieces(budget < n_max ? budget : n_max, n_chunks);
}

// Complete chunks 0..n-1: offsets[0] = 0, strictly increasing, ending at or
// before `limit`.
hsa_status_t check_chunk_offsets(const int32_t* offsets, int n, int64_t limit) {
  if (!offsets) return fail(HSA_ERR_INVALID_ARGUMENT, "offsets must not be NULL");
  if (offsets[0] != 0) return fail(HSA_ERR_INVALID_ARGUMENT, "offsets must start at 0");
  for (int k = 0; k < n; ++k)
    if (offsets[k + 1] <= offsets[k])
      return fail(HSA_ERR_INVALID_ARGUMENT, "offsets must be strictly increasing");
  if (offsets[n] > limit) return fail(HSA_ERR_INVALID_ARGUMENT, "offsets run past the cache");
  return HSA_OK;
}

void* align_ws(void* ws) {
  return (void*)(((uintptr_t)ws + kAlign - 1) / kAlign * kAlign);
}

}  // namespace

namespace hsa {

int api_error(int status, const char* message) {
  g_err = message;
  return status;
}

bool launch_log_enabled() {
  static const bool on = [] {
    const char* v = getenv("HSA_ATTN_LOG");
    return v != nullptr && *v != '\0' && strcmp(v, "0") != 0;
  }();
  return on;
}

void log_launch(const void* kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream) {
  // the kernel's symbol, demangled: "void hsa::(anonymous namespace)::name<args>(params)"
  const char* sym = hipKernelNameRefByPtr(kernel, stream);
  int status = -1;
  char* dem = sym ? abi::__cxa_demangle(sym, nullptr, nullptr, &status) : nullptr;
  std::string k = status == 0 && dem ? dem : (sym ? sym : "?");
  free(dem);
  if (k.compare(0, 5, "void ") == 0) k.erase(0, 5);
  for (const char* ns : {"hsa::(anonymous namespace)::", "hsa::"})
    if (k.compare(0, strlen(ns), ns) == 0) k.erase(0, strlen(ns));
  const size_t paren = k.rfind('(');
  if (paren != std::string::npos && paren > 0) k.erase(paren);
  fprintf(stderr, "hsa_attn:   launch %s grid (%u, %u, %u) block (%u, %u, %u) lds %zu B\n",
          k.c_str(), grid.x, grid.y, grid.z, block.x, block.y, block.z, lds);
}

}  // namespace hsa

extern "C" {

const char* hsa_status_string(hsa_status_t status) {
  switch (status) {
    case HSA_OK: return "HSA_OK: success";
    case HSA_ERR_INVALID_ARGUMENT: return "HSA_ERR_INVALID_ARGUMENT: invalid argument";
    case HSA_ERR_UNSUPPORTED: return "HSA_ERR_UNSUPPORTED: request not supported by this build";
    case HSA_ERR_WORKSPACE_TOO_SMALL: return "HSA_ERR_WORKSPACE_TOO_SMALL: workspace too small";
    case HSA_ERR_HIP: return "HSA_ERR_HIP: a HIP call failed";
  }
  return "unknown hsa_status_t";
}

const char* hsa_last_error_message(void) { return g_err.c_str(); }

hsa_status_t hsa_build_landmarks(const void* K, float* lmk, int B, int Hkv, int64_t L, int d,
                                 int S, int64_t chunk_begin, int64_t chunk_end,
                                 hsa_dtype_t dtype, hsa_stream_t stream) {
  g_err.clear();
  log_call("hsa_build_landmarks B=%d Hkv=%d L=%lld d=%d S=%d chunks [%lld, %lld) dtype=%d", B, Hkv,
           (long long)L, d, S, (long long)chunk_begin, (long long)chunk_end, (int)dtype);
  if (!dtype_ok(dtype)) return fail(HSA_ERR_UNSUPPORTED, "dtype must be F32 or BF16");
  if (B < 0 || Hkv <= 0 || L < 0) return fail(HSA_ERR_INVALID_ARGUMENT, "bad B, Hkv or L");
  if (d != 64 && d != 128) return fail(HSA_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (S < 1 || S > 1024) return fail(HSA_ERR_INVALID_ARGUMENT, "chunk size S must be in [1, 1024]");
  const int64_t n = L / S;
  if (chunk_begin < 0 || chunk_end < chunk_begin || chunk_end > n)
    return fail(HSA_ERR_INVALID_ARGUMENT, "need 0 <= chunk_begin <= chunk_end <= L/S");
  if ((int64_t)B * Hkv * (chunk_end - chunk_begin) >= ((int64_t)1 << 31))
    return fail(HSA_ERR_UNSUPPORTED, "too many chunks for one launch");
  if (B == 0 || chunk_end == chunk_begin) return HSA_OK;
  if (!K || !lmk) return fail(HSA_ERR_INVALID_ARGUMENT, "K and lmk must not be NULL");
  hipError_t e = hsa::launch_landmarks(K, dt_code(dtype), lmk, (int64_t)B * Hkv, L, n, d, S,
                                       chunk_begin, chunk_end, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hsa_build_landmarks launch");
  return finish((hipStream_t)stream);
}

size_t hsa_prefill_workspace_size(int B, int64_t L, int Hq, int Hkv, int d, int S, int topk,
                                  hsa_dtype_t dtype) {
  if (check_prefill(B, L, Hq, Hkv, d, S, topk, dtype) != HSA_OK) return 0;
  return prefill_layout(nullptr, B, L, Hq, Hkv, d, S, topk, dtype).bytes;
}

}  // extern "C"

namespace {

// The forward's kernel arguments over a carved workspace.
hsa::PrefillArgs prefill_args(const PrefillLayout& lay, const void* Q, const void* K,
                              const void* V, const float* lmk, void* O, int32_t* sel_idx,
                              float* sel_w, int B, int64_t L, int Hq, int Hkv, int d, int S,
                              int topk, int interval, hsa_dtype_t dtype) {
  const int G = Hq / Hkv;
  hsa::PrefillArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.lmk = lmk ? lmk : lay.lmk;
  a.idx = sel_idx ? sel_idx : lay.idx;
  a.sel_w = sel_w;
  a.counts = lay.counts;
  a.cursor = lay.cursor;
  a.blockbase = lay.blockbase;
  a.ordered = 0;
  a.offs = lay.offs;
  a.tile_off = lay.tile_off;
  a.tile_chunk = lay.tile_chunk;
  a.list = lay.list;
  a.entry_pos = lay.entry_pos;
  a.partial = lay.partial;
  a.part_score = lay.part_score;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.S = S;
  a.topk = topk;
  a.dtype = dt_code(dtype);
  a.L = L;
  a.n = L / S;
  a.entries_per_tile = lay.entries_per_tile;
  a.log2G = -1;
  for (int k = 0; k < 6; ++k)
    if ((1 << k) == G) a.log2G = k;
  a.interval = interval;
  a.nq = (L + interval - 1) / interval;
  a.tiles_ub = lay.tiles_ub;
  return a;
}

hsa_status_t prefill_impl(const void* Q, const void* K, const void* V, const float* lmk,
                          void* O, int32_t* sel_idx, float* sel_w, int B, int64_t L, int Hq,
                          int Hkv, int d, int S, int topk, int interval, hsa_dtype_t dtype,
                          void* workspace, size_t workspace_bytes, hsa_stream_t stream) {
  g_err.clear();
  log_call("%s B=%d L=%lld Hq=%d Hkv=%d d=%d S=%d topk=%d dtype=%d",
           interval > 1 ? "hsa_prefill_interval" : "hsa_prefill", B, (long long)L, Hq, Hkv, d, S,
           topk, (int)dtype);
  hsa_status_t s = check_prefill(B, L, Hq, Hkv, d, S, topk, dtype);
  if (s != HSA_OK) return s;
  if (interval < 1) return fail(HSA_ERR_INVALID_ARGUMENT, "the retrieval interval must be >= 1");
  if (B == 0 || L == 0) return HSA_OK;
  if (!Q || !K || !V || !O) return fail(HSA_ERR_INVALID_ARGUMENT, "Q, K, V and O must not be NULL");
  const size_t need = prefill_layout(nullptr, B, L, Hq, Hkv, d, S, topk, dtype, interval).bytes;
  if (!workspace || workspace_bytes < need)
    return fail(HSA_ERR_WORKSPACE_TOO_SMALL,
                "workspace needs " + std::to_string(need) + " bytes");
  PrefillLayout lay =
      prefill_layout(align_ws(workspace), B, L, Hq, Hkv, d, S, topk, dtype, interval);
  const hipStream_t st = (hipStream_t)stream;
  const int64_t n = L / S;
  hsa::PrefillArgs a = prefill_args(lay, Q, K, V, lmk, O, sel_idx, sel_w, B, L, Hq, Hkv, d, S,
                                    topk, interval, dtype);
  if ((int64_t)B * Hkv * a.tiles_ub >= ((int64_t)1 << 31))
    return fail(HSA_ERR_UNSUPPORTED, "too many attention tiles for one launch");
  hipError_t e;
  StageMarks pm(st);
  pm.mark();
  if (!lmk && n > 0) {
    e = hsa::launch_landmarks(K, a.dtype, lay.lmk, (int64_t)B * Hkv, L, n, d, S, 0, n, st);
    if (e != hipSuccess) return hip_fail(e, "landmarks");
  }
  pm.mark();
  if ((e = hsa::prefill_select(a, st)) != hipSuccess) return hip_fail(e, "select");
  // the split landmarks of the query-major path use the partials' buffer
  const size_t partial_bytes = (size_t)((int64_t)B * Hq * L * topk * d * elem_bytes(dtype));
  if (hsa::prefill_query_major(a) &&
      hsa::prefill_query_major_scratch((int64_t)B * Hkv, n, d) <= partial_bytes) {
    // one selection row per wave, fused in registers: no invert, no partial
    // outputs, no fusion pass (their stage marks stay, with nothing between)
    pm.mark();
    pm.mark();
    if ((e = hsa::prefill_attend_query_major(a, lay.partial, st)) != hipSuccess)
      return hip_fail(e, "attend");
    pm.mark();
    pm.mark();
    return finish(st);
  }
  pm.mark();
  if ((e = hsa::prefill_invert(a, st)) != hipSuccess) return hip_fail(e, "invert");
  pm.mark();
  if ((e = hsa::prefill_attend(a, st)) != hipSuccess) return hip_fail(e, "attend");
  pm.mark();
  if ((e = hsa::prefill_fuse(a, st)) != hipSuccess) return hip_fail(e, "fuse");
  pm.mark();
  return finish(st);
}

}  // namespace

extern "C" {

hsa_status_t hsa_prefill(const void* Q, const void* K, const void* V, const float* lmk,
                         void* O, int32_t* sel_idx, float* sel_w, int B, int64_t L, int Hq,
                         int Hkv, int d, int S, int topk, hsa_dtype_t dtype, void* workspace,
                         size_t workspace_bytes, hsa_stream_t stream) {
  return prefill_impl(Q, K, V, lmk, O, sel_idx, sel_w, B, L, Hq, Hkv, d, S, topk, 1, dtype,
                      workspace, workspace_bytes, stream);
}

size_t hsa_prefill_backward_workspace_size(int B, int64_t L, int Hq, int Hkv, int d, int S,
                                           int topk, hsa_dtype_t dtype) {
  if (dtype != HSA_DTYPE_BF16 || S > 64 || check_prefill(B, L, Hq, Hkv, d, S, topk, dtype) != HSA_OK)
    return 0;
  return backward_layout(nullptr, B, L, Hq, Hkv, d, S, topk).bytes;
}

hsa_status_t hsa_prefill_backward(const void* Q, const void* K, const void* V, const void* dO,
                                  const float* lmk, void* dQ, void* dK, void* dV, int B,
                                  int64_t L, int Hq, int Hkv, int d, int S, int topk,
                                  hsa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                  hsa_stream_t stream) {
  g_err.clear();
  log_call("hsa_prefill_backward B=%d L=%lld Hq=%d Hkv=%d d=%d S=%d topk=%d dtype=%d", B,
           (long long)L, Hq, Hkv, d, S, topk, (int)dtype);
  hsa_status_t s = check_prefill(B, L, Hq, Hkv, d, S, topk, dtype);
  if (s != HSA_OK) return s;
  if (dtype != HSA_DTYPE_BF16) return fail(HSA_ERR_UNSUPPORTED, "the backward runs bf16 only");
  if (S > 64) return fail(HSA_ERR_UNSUPPORTED, "the backward needs chunk size S <= 64");
  if (B == 0 || L == 0) return HSA_OK;
  if (!Q || !K || !V || !dO || !dQ || !dK || !dV)
    return fail(HSA_ERR_INVALID_ARGUMENT, "Q, K, V, dO, dQ, dK and dV must not be NULL");
  const size_t need = backward_layout(nullptr, B, L, Hq, Hkv, d, S, topk).bytes;
  if (!workspace || workspace_bytes < need)
    return fail(HSA_ERR_WORKSPACE_TOO_SMALL,
                "workspace needs " + std::to_string(need) + " bytes");
  BackwardLayout lay = backward_layout(align_ws(workspace), B, L, Hq, Hkv, d, S, topk);
  const hipStream_t st = (hipStream_t)stream;
  const int64_t n = L / S;
  hsa::PrefillBwdArgs ba;
  ba.p = prefill_args(lay.fwd, Q, K, V, lmk, nullptr, nullptr, nullptr, B, L, Hq, Hkv, d, S,
                      topk, 1, dtype);
  if ((int64_t)B * Hkv * ba.p.tiles_ub >= ((int64_t)1 << 31))
    return fail(HSA_ERR_UNSUPPORTED, "too many attention tiles for one launch");
  ba.p.ordered = 1;  // dK and dV sum over each chunk's list: keep it in token order
  ba.dO = dO;
  ba.lse2 = lay.lse2;
  ba.dw = lay.dw;
  ba.wk = lay.wk;
  ba.ds = lay.ds;
  ba.dQ = dQ;
  ba.dK = dK;
  ba.dV = dV;
  hipError_t e;
  StageMarks pm(st);
  pm.mark();
  if (!lmk && n > 0) {
    e = hsa::launch_landmarks(K, ba.p.dtype, lay.fwd.lmk, (int64_t)B * Hkv, L, n, d, S, 0, n, st);
    if (e != hipSuccess) return hip_fail(e, "landmarks");
  }
  pm.mark();
  if ((e = hsa::prefill_select(ba.p, st)) != hipSuccess) return hip_fail(e, "select");
  pm.mark();
  if ((e = hsa::prefill_invert(ba.p, st)) != hipSuccess) return hip_fail(e, "invert");
  pm.mark();
  if ((e = hsa::prefill_bwd_weights(ba, st)) != hipSuccess)
    return hip_fail(e, "backward weights");
  pm.mark();
  if ((e = hsa::prefill_bwd_score(ba, st)) != hipSuccess) return hip_fail(e, "backward score");
  pm.mark();
  if ((e = hsa::prefill_bwd_rows(ba, st)) != hipSuccess) return hip_fail(e, "backward rows");
  pm.mark();
  if ((e = hsa::prefill_bwd_kv(ba, st)) != hipSuccess) return hip_fail(e, "backward kv");
  pm.mark();
  if ((e = hsa::prefill_bwd_finish(ba, st)) != hipSuccess) return hip_fail(e, "backward finish");
  pm.mark();
  return finish(st);
}

size_t hsa_prefill_interval_workspace_size(int B, int64_t L, int Hq, int Hkv, int d, int S,
                                           int topk, int interval, hsa_dtype_t dtype) {
  if (interval < 1 || check_prefill(B, L, Hq, Hkv, d, S, topk, dtype) != HSA_OK) return 0;
  return prefill_layout(nullptr, B, L, Hq, Hkv, d, S, topk, dtype, interval).bytes;
}

hsa_status_t hsa_prefill_interval(const void* Q, const void* K, const void* V, const float* lmk,
                                  void* O, int32_t* sel_idx, float* sel_w, int B, int64_t L,
                                  int Hq, int Hkv, int d, int S, int topk, int interval,
                                  hsa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                  hsa_stream_t stream) {
  return prefill_impl(Q, K, V, lmk, O, sel_idx, sel_w, B, L, Hq, Hkv, d, S, topk, interval,
                      dtype, workspace, workspace_bytes, stream);
}

size_t hsa_decode_workspace_size(int B, int Hq, int Hkv, int d, int S, int topk,
                                 int64_t n_ctx) {
  if (check_decode(B, Hq, Hkv, d, S, topk, n_ctx, n_ctx, HSA_DTYPE_BF16) != HSA_OK) return 0;
  return decode_layout(nullptr, B, Hq, Hkv, d, S, topk, n_ctx).bytes;
}

hsa_status_t hsa_decode(const void* q, const void* Kc, const void* Vc, const float* lmk,
                        int64_t n_ctx, int64_t n_max, void* o, int32_t* sel_idx, float* sel_w,
                        int B, int Hq, int Hkv, int d, int S, int topk, hsa_dtype_t dtype,
                        void* workspace, size_t workspace_bytes, hsa_stream_t stream) {
  g_err.clear();
  log_call("hsa_decode B=%d n_ctx=%lld n_max=%lld Hq=%d Hkv=%d d=%d S=%d topk=%d dtype=%d", B,
           (long long)n_ctx, (long long)n_max, Hq, Hkv, d, S, topk, (int)dtype);
  hsa_status_t s = check_decode(B, Hq, Hkv, d, S, topk, n_ctx, n_max, dtype);
  if (s != HSA_OK) return s;
  if (B == 0) return HSA_OK;
  if (!q || !o) return fail(HSA_ERR_INVALID_ARGUMENT, "q and o must not be NULL");
  if (n_ctx / S > 0 && (!Kc || !Vc || !lmk))
    return fail(HSA_ERR_INVALID_ARGUMENT, "Kc, Vc and lmk must not be NULL");
  const size_t need = decode_layout(nullptr, B, Hq, Hkv, d, S, topk, n_ctx).bytes;
  if (!workspace || workspace_bytes < need)
    return fail(HSA_ERR_WORKSPACE_TOO_SMALL,
                "workspace needs " + std::to_string(need) + " bytes");
  DecodeLayout lay = decode_layout(align_ws(workspace), B, Hq, Hkv, d, S, topk, n_ctx);
  hsa::DecodeArgs a;
  a.q = q;
  a.Kc = Kc;
  a.Vc = Vc;
  a.lmk = lmk;
  a.o = o;
  a.sel = sel_idx ? sel_idx : lay.sel;
  a.sel_w = sel_w;
  a.cand = lay.cand;
  a.cand_mm = lay.cand_mm;
  a.part_o = lay.part_o;
  a.part_s = lay.part_s;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.S = S;
  a.topk = topk;
  a.dtype = dt_code(dtype);
  a.n_ctx = n_ctx;
  a.n_max = n_max;
  a.n_avail = n_ctx / S;
  a.lmk_chunks = n_max / S;
  a.n_slices = lay.n_slices;
  a.slice = lay.slice;
  a.swa_pieces = 0;
  a.swa_lo = a.swa_hi = 0;
  a.o_swa = nullptr;
  a.sw_o = a.sw_lse = nullptr;
  a.sync = lay.sync;
  const hipStream_t st = (hipStream_t)stream;
  StageMarks pm(st);
  if (hsa::decode_fused_ok(a)) {
    // scan, then attention with the fusion folded in (the fusion's stage
    // mark stays, with nothing between)
    for (int stage = 0; stage < hsa::kDecodeFusedStages; ++stage) {
      pm.mark();
      hipError_t e = hsa::decode_fused_stage(a, stage, st);
      if (e != hipSuccess) return hip_fail(e, "decode");
    }
    pm.mark();
    pm.mark();
    return finish(st);
  }
  for (int stage = 0; stage < hsa::kDecodeStages; ++stage) {
    pm.mark();
    hipError_t e = hsa::decode_stage(a, stage, st);
    if (e != hipSuccess) return hip_fail(e, "decode");
  }
  pm.mark();
  return finish(st);
}

size_t hsa_swa_decode_workspace_size(int B, int Hq, int Hkv, int d, int S, int topk,
                                     int64_t n_ctx, int64_t window) {
  if (check_decode(B, Hq, Hkv, d, S, topk, n_ctx, n_ctx, HSA_DTYPE_BF16) != HSA_OK) return 0;
  if (window < 1) return 0;
  return decode_layout(nullptr, B, Hq, Hkv, d, S, topk, n_ctx, swa_decode_pieces(n_ctx, window))
      .bytes;
}

hsa_status_t hsa_swa_decode(const void* q, const void* Kc, const void* Vc, const float* lmk,
                            int64_t n_ctx, int64_t n_max, int64_t window, void* o_hsa,
                            void* o_swa, int32_t* sel_idx, float* sel_w, int B, int Hq, int Hkv,
                            int d, int S, int topk, hsa_dtype_t dtype, void* workspace,
                            size_t workspace_bytes, hsa_stream_t stream) {
  g_err.clear();
  log_call("hsa_swa_decode B=%d n_ctx=%lld n_max=%lld window=%lld Hq=%d Hkv=%d d=%d S=%d topk=%d "
           "dtype=%d", B, (long long)n_ctx, (long long)n_max, (long long)window, Hq, Hkv, d, S,
           topk, (int)dtype);
  hsa_status_t s = check_decode(B, Hq, Hkv, d, S, topk, n_ctx, n_max, dtype);
  if (s != HSA_OK) return s;
  if (n_ctx >= n_max)
    return fail(HSA_ERR_INVALID_ARGUMENT,
                "need n_ctx < n_max: the new token (position n_ctx) is in the cache");
  if (window < 1) return fail(HSA_ERR_INVALID_ARGUMENT, "window must be >= 1");
  if (S > kSwaPieceKeys) return fail(HSA_ERR_UNSUPPORTED, "hsa_swa_decode needs S <= 64");
  const int pieces = swa_decode_pieces(n_ctx, window);
  if (pieces > kSwaMaxPieces)
    return fail(HSA_ERR_UNSUPPORTED, "hsa_swa_decode needs min(window, n_ctx + 1) <= 4096");
  if (B == 0) return HSA_OK;
  if (!q || !Kc || !Vc || !o_hsa || !o_swa)
    return fail(HSA_ERR_INVALID_ARGUMENT, "q, Kc, Vc, o_hsa and o_swa must not be NULL");
  if (n_ctx / S > 0 && !lmk) return fail(HSA_ERR_INVALID_ARGUMENT, "lmk must not be NULL");
  if ((int64_t)B * Hkv * n_max >= (int64_t(1) << 40))
    return fail(HSA_ERR_UNSUPPORTED, "B*Hkv*n_max must be < 2^40");
  const size_t need = decode_layout(nullptr, B, Hq, Hkv, d, S, topk, n_ctx, pieces).bytes;
  if (!workspace || workspace_bytes < need)
    return fail(HSA_ERR_WORKSPACE_TOO_SMALL,
                "workspace needs " + std::to_string(need) + " bytes");
  DecodeLayout lay = decode_layout(align_ws(workspace), B, Hq, Hkv, d, S, topk, n_ctx, pieces);
  hsa::DecodeArgs a;
  a.q = q;
  a.Kc = Kc;
  a.Vc = Vc;
  a.lmk = lmk;
  a.o = o_hsa;
  a.sel = sel_idx ? sel_idx : lay.sel;
  a.sel_w = sel_w;
  a.cand = lay.cand;
  a.cand_mm = lay.cand_mm;
  a.part_o = lay.part_o;
  a.part_s = lay.part_s;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.S = S;
  a.topk = topk;
  a.dtype = dt_code(dtype);
  a.n_ctx = n_ctx;
  a.n_max = n_max;
  a.n_avail = n_ctx / S;
  a.lmk_chunks = n_max / S;
  a.n_slices = lay.n_slices;
  a.slice = lay.slice;
  a.swa_pieces = pieces;
  a.swa_hi = n_ctx + 1;
  a.swa_lo = a.swa_hi - (window < n_ctx + 1 ? window : n_ctx + 1);
  a.o_swa = o_swa;
  a.sw_o = lay.sw_o;
  a.sync = nullptr;  // the fusion and the window's merge run as their own launch
  a.sw_lse = lay.sw_lse;
  const hipStream_t st = (hipStream_t)stream;
  StageMarks pm(st);
  for (int stage = 0; stage < hsa::kDecodeStages; ++stage) {
    pm.mark();
    hipError_t e = hsa::decode_stage(a, stage, st);
    if (e != hipSuccess) return hip_fail(e, "hsa_swa_decode");
  }
  pm.mark();
  return finish(st);
}

size_t dhsa_prefill_workspace_size(int B, int64_t L, int H, int d, int n_chunks,
                                   hsa_dtype_t dtype) {
  (void)L;
  if (!dtype_ok(dtype) || B < 0 || H <= 0 || n_chunks < 1 || n_chunks > hsa::dhsa_max_chunks())
    return 0;
  if (d != 64 && d != 128) return 0;
  return dhsa_layout(nullptr, B, H, d, n_chunks).bytes;
}

hsa_status_t dhsa_prefill(const void* Q, const void* K, const void* V, const int32_t* offsets,
                          int n_chunks, int64_t budget, void* O, uint32_t* mask_bits,
                          int32_t* chunk_order, int B, int64_t L, int H, int d,
                          hsa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                          hsa_stream_t stream) {
  g_err.clear();
  log_call("dhsa_prefill B=%d L=%lld H=%d d=%d chunks=%d budget=%lld dtype=%d", B, (long long)L, H,
           d, n_chunks, (long long)budget, (int)dtype);
  if (!dtype_ok(dtype)) return fail(HSA_ERR_UNSUPPORTED, "dtype must be F32 or BF16");
  if (B < 0 || L < 1 || H <= 0) return fail(HSA_ERR_INVALID_ARGUMENT, "need B >= 0, L >= 1, H >= 1");
  if (d != 64 && d != 128) return fail(HSA_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (budget < 1) return fail(HSA_ERR_INVALID_ARGUMENT, "budget N_b must be >= 1");
  if (!offsets) return fail(HSA_ERR_INVALID_ARGUMENT, "offsets must not be NULL");
  if (n_chunks < 1) return fail(HSA_ERR_INVALID_ARGUMENT, "n_chunks must be >= 1");
  if (n_chunks > hsa::dhsa_max_chunks())
    return fail(HSA_ERR_UNSUPPORTED, "n_chunks must be <= 4096");
  if (L >= ((int64_t)1 << 31)) return fail(HSA_ERR_UNSUPPORTED, "L must be < 2^31");
  if ((int64_t)B * H * n_chunks * (n_chunks + 1) >= ((int64_t)1 << 31))
    return fail(HSA_ERR_UNSUPPORTED, "B*H*n_chunks^2 must be < 2^31");
  if (offsets[0] != 0 || offsets[n_chunks] != L)
    return fail(HSA_ERR_INVALID_ARGUMENT, "offsets must start at 0 and end at L");
  int max_len = 0;
  for (int l = 0; l < n_chunks; ++l) {
    const int len = offsets[l + 1] - offsets[l];
    if (len <= 0) return fail(HSA_ERR_INVALID_ARGUMENT, "offsets must be strictly increasing");
    if (len > max_len) max_len = len;
  }
  if (B == 0) return HSA_OK;
  if (!Q || !K || !V || !O) return fail(HSA_ERR_INVALID_ARGUMENT, "Q, K, V and O must not be NULL");
  const size_t need = dhsa_layout(nullptr, B, H, d, n_chunks).bytes;
  if (!workspace || workspace_bytes < need)
    return fail(HSA_ERR_WORKSPACE_TOO_SMALL,
                "workspace needs " + std::to_string(need) + " bytes");
  DhsaLayout lay = dhsa_layout(align_ws(workspace), B, H, d, n_chunks);
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(lay.offs, offsets, sizeof(int32_t) * (n_chunks + 1),
                                hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "offsets upload");
  hsa::DhsaArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.offs = lay.offs;
  a.qh = lay.qh;
  a.kh = lay.kh;
  a.order = chunk_order ? chunk_order : lay.order;
  a.cumlen = lay.cumlen;
  a.diag_pos = lay.diag_pos;
  a.ranked = lay.ranked;
  a.mask_bits = mask_bits;
  a.B = B;
  a.H = H;
  a.d = d;
  a.dtype = dt_code(dtype);
  a.nc = n_chunks;
  a.tiles_per_chunk = (max_len + 127) / 128;
  a.L = L;
  a.budget = budget;
  // the bf16 attention launches up to four blocks per 128-row tile
  if ((int64_t)B * H * n_chunks * a.tiles_per_chunk * 4 >= ((int64_t)1 << 31))
    return fail(HSA_ERR_UNSUPPORTED, "too many attention tiles for one launch");
  StageMarks pm(st);
  for (int stage = 0; stage < hsa::kDhsaStages; ++stage) {
    pm.mark();
    e = hsa::dhsa_stage(a, stage, st);
    if (e != hipSuccess) return hip_fail(e, "dhsa");
  }
  pm.mark();
  return finish(st);
}

size_t dhsa_chunk_keys_workspace_size(int n_chunks) {
  if (n_chunks < 0) return 0;
  return ((size_t)n_chunks + 1) * sizeof(int32_t) + kAlign;
}

hsa_status_t dhsa_build_chunk_keys(const void* K, float* khat, const int32_t* offsets,
                                   int n_chunks, int chunk_begin, int chunk_end, int B, int H,
                                   int64_t n_max, int d, int n_cap, hsa_dtype_t dtype,
                                   void* workspace, size_t workspace_bytes, hsa_stream_t stream) {
  g_err.clear();
  log_call("dhsa_build_chunk_keys B=%d H=%d n_max=%lld d=%d chunks [%d, %d) dtype=%d", B, H,
           (long long)n_max, d, chunk_begin, chunk_end, (int)dtype);
  if (!dtype_ok(dtype)) return fail(HSA_ERR_UNSUPPORTED, "dtype must be F32 or BF16");
  if (d != 64 && d != 128) return fail(HSA_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (B < 0 || H <= 0 || n_max < 0 || n_chunks < 0 || n_cap < n_chunks)
    return fail(HSA_ERR_INVALID_ARGUMENT, "need B >= 0, H >= 1, 0 <= n_chunks <= n_cap");
  if (chunk_begin < 0 || chunk_end < chunk_begin || chunk_end > n_chunks)
    return fail(HSA_ERR_INVALID_ARGUMENT, "need 0 <= chunk_begin <= chunk_end <= n_chunks");
  hsa_status_t s = check_chunk_offsets(offsets, n_chunks, n_max);
  if (s != HSA_OK) return s;
  if ((int64_t)B * H * (chunk_end - chunk_begin) >= ((int64_t)1 << 31))
    return fail(HSA_ERR_UNSUPPORTED, "too many chunks for one launch");
  if (B == 0 || chunk_end == chunk_begin) return HSA_OK;
  if (!K || !khat) return fail(HSA_ERR_INVALID_ARGUMENT, "K and khat must not be NULL");
  const int cnt = chunk_end - chunk_begin;
  if (!workspace || workspace_bytes < dhsa_chunk_keys_workspace_size(cnt))
    return fail(HSA_ERR_WORKSPACE_TOO_SMALL,
                "workspace needs " + std::to_string(dhsa_chunk_keys_workspace_size(cnt)) +
                    " bytes");
  int32_t* offs = (int32_t*)align_ws(workspace);
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(offs, offsets + chunk_begin, sizeof(int32_t) * (cnt + 1),
                                hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "offsets upload");
  e = hsa::launch_dhsa_chunk_keys(K, khat, offs, dt_code(dtype), (int64_t)B * H, n_max, d, n_cap,
                                  chunk_begin, chunk_end, st);
  return e == hipSuccess ? finish(st) : hip_fail(e, "dhsa_build_chunk_keys launch");
}

size_t dhsa_decode_workspace_size(int B, int H, int d, int n_chunks, int64_t budget,
                                  int64_t n_max) {
  if (B < 0 || H <= 0 || n_chunks < 0 || n_chunks + 1 > hsa::dhsa_max_chunks()) return 0;
  if (d != 64 && d != 128) return 0;
  if (budget < 1 || n_max < 1) return 0;
  return dhsa_decode_layout(nullptr, B, H, d, n_chunks, dhsa_decode_pieces(n_chunks, budget, n_max))
      .bytes;
}

hsa_status_t dhsa_decode(const void* q_cur, int m, const void* Kc, const void* Vc,
                         int64_t n_max, const float* khat, int n_cap, const int32_t* offsets,
                         int n_chunks, int64_t budget, void* o, int32_t* chunk_order, int B,
                         int H, int d, hsa_dtype_t dtype, void* workspace,
                         size_t workspace_bytes, hsa_stream_t stream) {
  g_err.clear();
  log_call("dhsa_decode B=%d H=%d m=%d n_max=%lld d=%d chunks=%d budget=%lld dtype=%d", B, H, m,
           (long long)n_max, d, n_chunks, (long long)budget, (int)dtype);
  if (!dtype_ok(dtype)) return fail(HSA_ERR_UNSUPPORTED, "dtype must be F32 or BF16");
  if (d != 64 && d != 128) return fail(HSA_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (B < 0 || H <= 0) return fail(HSA_ERR_INVALID_ARGUMENT, "need B >= 0 and H >= 1");
  if (m < 1) return fail(HSA_ERR_INVALID_ARGUMENT, "the current chunk needs m >= 1 queries");
  if (n_chunks < 0 || n_chunks > n_cap)
    return fail(HSA_ERR_INVALID_ARGUMENT, "need 0 <= n_chunks <= n_cap");
  if (n_chunks + 1 > hsa::dhsa_max_chunks())
    return fail(HSA_ERR_UNSUPPORTED, "n_chunks + 1 must be <= 4096");
  if (budget < 1) return fail(HSA_ERR_INVALID_ARGUMENT, "budget N_b must be >= 1");
  if (n_max >= ((int64_t)1 << 31)) return fail(HSA_ERR_UNSUPPORTED, "n_max must be < 2^31");
  hsa_status_t s = check_chunk_offsets(offsets, n_chunks, n_max);
  if (s != HSA_OK) return s;
  const int64_t pos = (int64_t)offsets[n_chunks] + m - 1;
  if (pos >= n_max) return fail(HSA_ERR_INVALID_ARGUMENT, "the new query lies past the cache");
  const int64_t pieces = dhsa_decode_pieces(n_chunks, budget, n_max);
  if ((int64_t)B * H * pieces * (d + 2) >= ((int64_t)1 << 31))
    return fail(HSA_ERR_UNSUPPORTED, "B*H*(min(budget, n_max)/64 + n_chunks + 2)*(d+2) must be < 2^31");
  if (B == 0) return HSA_OK;
  if (!q_cur || !Kc || !Vc || !o || (n_chunks > 0 && !khat))
    return fail(HSA_ERR_INVALID_ARGUMENT, "q_cur, Kc, Vc, o (and khat) must not be NULL");
  const size_t need = dhsa_decode_layout(nullptr, B, H, d, n_chunks, pieces).bytes;
  if (!workspace || workspace_bytes < need)
    return fail(HSA_ERR_WORKSPACE_TOO_SMALL,
                "workspace needs " + std::to_string(need) + " bytes");
  DhsaDecodeLayout lay = dhsa_decode_layout(align_ws(workspace), B, H, d, n_chunks, pieces);
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(lay.offs, offsets, sizeof(int32_t) * (n_chunks + 1),
                                hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "offsets upload");
  hsa::DhsaDecodeArgs a;
  a.qcur = q_cur;
  a.Kc = Kc;
  a.Vc = Vc;
  a.khat = khat;
  a.o = o;
  a.chunk_order = chunk_order;
  a.offs = lay.offs;
  a.plan = lay.plan;
  a.n_plan = lay.n_plan;
  a.part = lay.part;
  a.B = B;
  a.H = H;
  a.d = d;
  a.dtype = dt_code(dtype);
  a.n = n_chunks;
  a.n_cap = n_cap;
  a.m = m;
  a.P = 1;
  while (a.P < n_chunks + 1) a.P <<= 1;
  a.max_pieces = (int)pieces;
  a.n_max = n_max;
  a.pos = pos;
  a.budget = budget;
  StageMarks pm(st);
  for (int stage = 0; stage < hsa::kDhsaDecodeStages; ++stage) {
    pm.mark();
    e = hsa::dhsa_decode_stage(a, stage, st);
    if (e != hipSuccess) return hip_fail(e, "dhsa_decode");
  }
  pm.mark();
  return finish(st);
}

}  // extern "C"

namespace {

hsa_status_t check_swa(int B, int Hq, int Hkv, int d, int64_t window, hsa_dtype_t dtype) {
  if (!dtype_ok(dtype)) return fail(HSA_ERR_UNSUPPORTED, "dtype must be F32 or BF16");
  if (B < 0 || Hq <= 0 || Hkv <= 0)
    return fail(HSA_ERR_INVALID_ARGUMENT, "need B >= 0, Hq >= 1, Hkv >= 1");
  if (Hq % Hkv != 0) return fail(HSA_ERR_INVALID_ARGUMENT, "Hq must be a multiple of Hkv");
  if (d != 64 && d != 128) return fail(HSA_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (window < 1) return fail(HSA_ERR_INVALID_ARGUMENT, "window must be >= 1");
  return HSA_OK;
}

}  // namespace

extern "C" {

hsa_status_t swa_prefill(const void* Q, const void* K, const void* V, void* O, int B, int64_t L,
                         int Hq, int Hkv, int d, int64_t window, hsa_dtype_t dtype,
                         hsa_stream_t stream) {
  g_err.clear();
  log_call("swa_prefill B=%d L=%lld Hq=%d Hkv=%d d=%d window=%lld dtype=%d", B, (long long)L, Hq,
           Hkv, d, (long long)window, (int)dtype);
  hsa_status_t s = check_swa(B, Hq, Hkv, d, window, dtype);
  if (s != HSA_OK) return s;
  if (L < 0) return fail(HSA_ERR_INVALID_ARGUMENT, "need L >= 0");
  if ((int64_t)B * Hq * L >= (int64_t(1) << 31))
    return fail(HSA_ERR_UNSUPPORTED, "B*Hq*L must be < 2^31");
  if (B == 0 || L == 0) return HSA_OK;
  if (!Q || !K || !V || !O)
    return fail(HSA_ERR_INVALID_ARGUMENT, "Q, K, V and O must not be NULL");
  hsa::SwaArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.dtype = dt_code(dtype);
  a.L = L;
  a.window = window;
  a.n_ctx = 0;
  const hipStream_t st = (hipStream_t)stream;
  StageMarks pm(st);
  pm.mark();
  hipError_t e = hsa::launch_swa_prefill(a, st);
  if (e != hipSuccess) return hip_fail(e, "swa_prefill");
  pm.mark();
  return finish(st);
}

hsa_status_t hsa_swa_prefill(const void* Q, const void* K, const void* V, const float* lmk,
                             int64_t window, void* O_hsa, void* O_swa, int32_t* sel_idx,
                             float* sel_w, int B, int64_t L, int Hq, int Hkv, int d, int S,
                             int topk, hsa_dtype_t dtype, void* workspace,
                             size_t workspace_bytes, hsa_stream_t stream) {
  g_err.clear();
  log_call("hsa_swa_prefill B=%d L=%lld Hq=%d Hkv=%d d=%d S=%d topk=%d window=%lld dtype=%d", B,
           (long long)L, Hq, Hkv, d, S, topk, (long long)window, (int)dtype);
  hsa_status_t s = check_prefill(B, L, Hq, Hkv, d, S, topk, dtype);
  if (s != HSA_OK) return s;
  if ((s = check_swa(B, Hq, Hkv, d, window, dtype)) != HSA_OK) return s;
  if ((int64_t)B * Hq * L >= (int64_t(1) << 31))
    return fail(HSA_ERR_UNSUPPORTED, "B*Hq*L must be < 2^31");
  if (B == 0 || L == 0) return HSA_OK;
  if (!Q || !K || !V || !O_hsa || !O_swa)
    return fail(HSA_ERR_INVALID_ARGUMENT, "Q, K, V, O_hsa and O_swa must not be NULL");
  const size_t need = prefill_layout(nullptr, B, L, Hq, Hkv, d, S, topk, dtype).bytes;
  if (!workspace || workspace_bytes < need)
    return fail(HSA_ERR_WORKSPACE_TOO_SMALL,
                "workspace needs " + std::to_string(need) + " bytes");
  PrefillLayout lay = prefill_layout(align_ws(workspace), B, L, Hq, Hkv, d, S, topk, dtype);
  const hipStream_t st = (hipStream_t)stream;
  const int64_t n = L / S;
  hsa::PrefillArgs a = prefill_args(lay, Q, K, V, lmk, O_hsa, sel_idx, sel_w, B, L, Hq, Hkv, d,
                                    S, topk, 1, dtype);
  if ((int64_t)B * Hkv * a.tiles_ub >= ((int64_t)1 << 31))
    return fail(HSA_ERR_UNSUPPORTED, "too many attention tiles for one launch");
  hsa::SwaArgs w;
  w.Q = Q;
  w.K = K;
  w.V = V;
  w.O = O_swa;
  w.B = B;
  w.Hq = Hq;
  w.Hkv = Hkv;
  w.d = d;
  w.dtype = dt_code(dtype);
  w.L = L;
  w.window = window;
  w.n_ctx = 0;
  // one launch for both attentions: bf16 with chunks of at most 64 keys;
  // otherwise the two run as consecutive launches
  const bool fused = dtype == HSA_DTYPE_BF16 && S <= 64;
  hipError_t e;
  StageMarks pm(st);
  pm.mark();
  if (!lmk && n > 0) {
    e = hsa::launch_landmarks(K, a.dtype, lay.lmk, (int64_t)B * Hkv, L, n, d, S, 0, n, st);
    if (e != hipSuccess) return hip_fail(e, "landmarks");
  }
  pm.mark();
  if ((e = hsa::prefill_select(a, st)) != hipSuccess) return hip_fail(e, "select");
  pm.mark();
  if ((e = hsa::prefill_invert(a, st)) != hipSuccess) return hip_fail(e, "invert");
  pm.mark();
  if (fused) {
    if ((e = hsa::launch_upper_attend(a, w, st)) != hipSuccess) return hip_fail(e, "attend");
  } else {
    if ((e = hsa::prefill_attend(a, st)) != hipSuccess) return hip_fail(e, "attend");
    if ((e = hsa::launch_swa_prefill(w, st)) != hipSuccess) return hip_fail(e, "swa");
  }
  pm.mark();
  if ((e = hsa::prefill_fuse(a, st)) != hipSuccess) return hip_fail(e, "fuse");
  pm.mark();
  return finish(st);
}

hsa_status_t swa_decode(const void* q, const void* Kc, const void* Vc, int64_t pos,
                        int64_t n_max, int64_t window, void* o, int B, int Hq, int Hkv, int d,
                        hsa_dtype_t dtype, hsa_stream_t stream) {
  g_err.clear();
  log_call("swa_decode B=%d pos=%lld n_max=%lld Hq=%d Hkv=%d d=%d window=%lld dtype=%d", B,
           (long long)pos, (long long)n_max, Hq, Hkv, d, (long long)window, (int)dtype);
  hsa_status_t s = check_swa(B, Hq, Hkv, d, window, dtype);
  if (s != HSA_OK) return s;
  if (pos < 0 || pos >= n_max)
    return fail(HSA_ERR_INVALID_ARGUMENT, "need 0 <= pos < n_max (the new token is cached)");
  if (B == 0) return HSA_OK;
  if ((int64_t)B * Hkv * n_max >= (int64_t(1) << 40))
    return fail(HSA_ERR_UNSUPPORTED, "B*Hkv*n_max must be < 2^40");
  if (!q || !Kc || !Vc || !o)
    return fail(HSA_ERR_INVALID_ARGUMENT, "q, Kc, Vc and o must not be NULL");
  hsa::SwaArgs a;
  a.Q = q;
  a.K = Kc;
  a.V = Vc;
  a.O = o;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.dtype = dt_code(dtype);
  a.L = n_max;
  a.window = window;
  a.n_ctx = pos + 1;
  const hipStream_t st = (hipStream_t)stream;
  StageMarks pm(st);
  pm.mark();
  hipError_t e = hsa::launch_swa_decode(a, st);
  if (e != hipSuccess) return hip_fail(e, "swa_decode");
  pm.mark();
  return finish(st);
}

int hsa_device_checks_enabled(void) { return hsa::check_sources().empty() ? 0 : 1; }

hsa_status_t hsa_device_checks_selftest(int fail_check, hsa_stream_t stream) {
  g_err.clear();
  log_call("hsa_device_checks_selftest fail=%d", fail_check);
  if (hsa::check_sources().empty())
    return ::fail(HSA_ERR_UNSUPPORTED, "device checks are compiled into the debug library only");
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e = hsa::launch_check_selftest(fail_check, st);
  if (e != hipSuccess) return hip_fail(e, "hsa_device_checks_selftest launch");
  return finish(st);
}

hsa_status_t hsa_profile_enable(int enable) {
  g_err.clear();
  g_prof.on = enable != 0;
  return HSA_OK;
}

int hsa_profile_read(double* stage_ms, int max_stages, int* n_stages) {
  g_err.clear();
  int stages = 0;
  for (auto& ev : g_prof.calls) {
    if (ev.empty()) continue;
    if (hipEventSynchronize(ev.back()) != hipSuccess) continue;
    const int ns = (int)ev.size() - 1;
    if (ns > stages) stages = ns;
    for (int s = 0; s < ns && s < max_stages; ++s) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, ev[s], ev[s + 1]) == hipSuccess && stage_ms) stage_ms[s] += ms;
    }
  }
  const int calls = (int)g_prof.calls.size();
  for (auto& ev : g_prof.calls)
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  g_prof.calls.clear();
  if (n_stages) *n_stages = stages;
  return calls;
}

}  // extern "C"

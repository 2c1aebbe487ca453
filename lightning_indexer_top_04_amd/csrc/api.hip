// C ABI of liblsi: argument validation (before anything is enqueued),
// workspace carving and the launch sequences of each entry point.
#include <mutex>
#include <string>

#include "lsi_internal.hpp"

namespace lsi {

namespace {
thread_local std::string g_last_error;
// profiling marks of the calling thread (lsi_profile_events)
struct ProfState {
  hipEvent_t* ev = nullptr;
  const char** names = nullptr;
  int cap = 0;
  int used = 0;
};
thread_local ProfState g_prof;
}

bool prof_next(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  ProfState& p = g_prof;
  if (p.ev == nullptr || p.used + 2 > p.cap) return false;
  *start = p.ev[p.used];
  *stop = p.ev[p.used + 1];
  if (p.names) p.names[p.used / 2] = name;
  p.used += 2;
  return true;
}

void set_error(const std::string& msg) { g_last_error = msg; }

int32_t fail(int32_t status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int32_t check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(LSI_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return LSI_OK;
}

int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev] = v;
  }
  return cache[dev];
}

namespace {

constexpr size_t kWsAlign = 256;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define LSI_REQUIRE(cond, msg)                                   \
  do {                                                           \
    if (!(cond)) return fail(LSI_ERR_INVALID_ARG, (msg));        \
  } while (0)
#define LSI_SUPPORT(cond, msg)                                   \
  do {                                                           \
    if (!(cond)) return fail(LSI_ERR_UNSUPPORTED, (msg));        \
  } while (0)
#define LSI_TRY(expr)                                            \
  do {                                                           \
    const int32_t _st = (expr);                                  \
    if (_st != LSI_OK) return _st;                               \
  } while (0)
// A launcher's status (it returns hipGetLastError(), which also clears the
// error): the first failure ends the call before anything else is enqueued.
#define LSI_LAUNCH(expr, what)                                                         \
  do {                                                                                 \
    const hipError_t _le = (expr);                                                     \
    if (_le != hipSuccess)                                                             \
      return fail(LSI_ERR_HIP, std::string(what) + ": " + hipGetErrorString(_le));     \
  } while (0)

int32_t check_batch(const lsi_batch* b, bool need_pages) {
  LSI_REQUIRE(b != nullptr, "batch is NULL");
  LSI_REQUIRE(b->num_req >= 1, "batch->num_req must be >= 1");
  LSI_REQUIRE(b->max_seq_len >= 0, "batch->max_seq_len must be >= 0");
  LSI_REQUIRE(b->reserved == 0, "batch->reserved must be 0");
  LSI_REQUIRE(b->seq_lens != nullptr, "batch->seq_lens is NULL");
  if (need_pages) {
    LSI_REQUIRE(b->page_table != nullptr, "batch->page_table is NULL");
    LSI_REQUIRE(b->max_pages >= 1, "batch->max_pages must be >= 1");
  }
  return LSI_OK;
}

int32_t check_cache(const lsi_paged_cache* c, const lsi_batch* b, const char* name) {
  const std::string n(name);
  LSI_REQUIRE(c != nullptr, n + " is NULL");
  LSI_REQUIRE(c->data != nullptr, n + "->data is NULL");
  LSI_REQUIRE(c->page_size >= 1, n + "->page_size must be >= 1");
  LSI_REQUIRE(c->num_pages >= 1, n + "->num_pages must be >= 1");
  LSI_REQUIRE(c->dim >= 1, n + "->dim must be >= 1");
  LSI_REQUIRE((int64_t)c->num_pages * c->page_size <= INT32_MAX,
              n + ": num_pages * page_size exceeds 2^31-1 tokens");
  LSI_REQUIRE((int64_t)b->max_pages * c->page_size >= b->max_seq_len,
              n + ": batch->max_seq_len exceeds max_pages * page_size");
  LSI_REQUIRE(aligned(c->data, 16), n + "->data must be 16-byte aligned");
  switch (c->dtype) {
    case LSI_F32:
    case LSI_BF16:
      LSI_REQUIRE(c->scale == nullptr, n + "->scale must be NULL for f32/bf16 caches");
      break;
    case LSI_FP8_E4M3:
    case LSI_INT4:
      LSI_REQUIRE(c->scale != nullptr, n + "->scale is required for fp8/int4 caches");
      break;
    default:
      return fail(LSI_ERR_INVALID_ARG, n + "->dtype is not an LSI element type");
  }
  return LSI_OK;
}

int32_t check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return LSI_OK;
  if (ws == nullptr) return fail(LSI_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, kWsAlign)) return fail(LSI_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need)
    return fail(LSI_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                       " bytes, have " + std::to_string(have));
  return LSI_OK;
}

// ---- indexer scan ----------------------------------------------------------
// scores == nullptr with ld == 0 means the caller keeps scores internally
int32_t validate_index(const lsi_paged_cache* ikeys, const lsi_batch* batch, const void* q,
                       int32_t n_heads, int32_t dim, const float* w, const float* scores,
                       int64_t ld, bool internal_scores = false) {
  LSI_TRY(check_batch(batch, true));
  LSI_TRY(check_cache(ikeys, batch, "ikeys"));
  LSI_REQUIRE(q != nullptr && w != nullptr, "q and w must be non-NULL");
  if (!internal_scores) {
    LSI_REQUIRE(scores != nullptr, "scores must be non-NULL");
    LSI_REQUIRE(ld >= batch->max_seq_len && ld >= 1, "ld must be >= max(1, batch->max_seq_len)");
  }
  LSI_REQUIRE(dim == ikeys->dim, "dim must equal ikeys->dim");
  LSI_REQUIRE(n_heads >= 1, "n_heads must be >= 1");
  if (ikeys->dtype == LSI_FP8_E4M3 || ikeys->dtype == LSI_INT4) {
    LSI_SUPPORT(dim == 128 && n_heads == 64, "fp8/int4 indexer keys need 64 heads of dim 128");
    LSI_SUPPORT(is_pow2(ikeys->page_size) && ikeys->page_size % 32 == 0,
                "fp8/int4 indexer keys need a power-of-two page_size that is a multiple of 32");
    LSI_REQUIRE(aligned(q, 16), "q must be 16-byte aligned");
  } else if (ikeys->dtype == LSI_F32) {
    LSI_SUPPORT(dim <= 256 && (int64_t)n_heads * dim <= 8192,
                "f32 indexer keys support dim <= 256 and n_heads*dim <= 8192");
  } else {
    return fail(LSI_ERR_UNSUPPORTED, "indexer keys must be fp8, int4 or f32");
  }
  return LSI_OK;
}

ScanArgs scan_args(const lsi_paged_cache* ikeys, const lsi_batch* batch, const void* q,
                   int32_t n_heads, int32_t dim, const float* w, float* scores, int64_t ld) {
  ScanArgs a;
  a.keys = ikeys->data;
  a.kscale = ikeys->scale;
  a.num_pages = ikeys->num_pages;
  a.page_size = ikeys->page_size;
  a.seq_lens = batch->seq_lens;
  a.page_table = batch->page_table;
  a.max_pages = batch->max_pages;
  a.max_seq_len = batch->max_seq_len;
  a.num_req = batch->num_req;
  a.q = q;
  a.w = w;
  a.scores = scores;
  a.ld = ld;
  a.n_heads = n_heads;
  a.dim = dim;
  return a;
}

hipError_t run_scan(int dtype, const ScanArgs& a, hipStream_t s) {
  switch (dtype) {
    case LSI_FP8_E4M3: return launch_scan_fp8(a, s);
    case LSI_INT4: return launch_scan_int4(a, s);
    default: return launch_scan_f32(a, s);
  }
}

// ---- top-k -----------------------------------------------------------------
int32_t validate_topk(const float* scores, int64_t ld, const lsi_batch* batch, int32_t k,
                      const int32_t* idx, const int32_t* count) {
  LSI_TRY(check_batch(batch, false));
  LSI_REQUIRE(scores != nullptr && idx != nullptr && count != nullptr,
              "scores, idx and count must be non-NULL");
  LSI_REQUIRE(ld >= batch->max_seq_len && ld >= 1, "ld must be >= max(1, batch->max_seq_len)");
  LSI_REQUIRE(k >= 1 && k <= 65536, "k must be in [1, 65536]");
  return LSI_OK;
}

// ---- attention -------------------------------------------------------------
int32_t validate_attn(const lsi_paged_cache* kv, const lsi_paged_cache* v, const lsi_batch* batch,
                      const void* q, int32_t n_heads, int32_t dk, int32_t dv, const int32_t* idx,
                      int32_t k, float sm_scale, const void* out, const float* lse) {
  LSI_TRY(check_batch(batch, true));
  LSI_TRY(check_cache(kv, batch, "kv"));
  LSI_REQUIRE(q != nullptr && idx != nullptr && out != nullptr && lse != nullptr,
              "q, idx, out and lse must be non-NULL");
  LSI_REQUIRE(k >= 1 && k <= 65536, "k must be in [1, 65536]");
  LSI_REQUIRE(n_heads >= 1, "n_heads must be >= 1");
  LSI_REQUIRE(sm_scale == sm_scale && sm_scale > 0.f, "sm_scale must be a positive number");
  LSI_REQUIRE(dk == kv->dim, "dk must equal kv->dim");
  if (kv->dtype == LSI_BF16) {
    LSI_SUPPORT(dk == 576 && dv == 512, "bf16 latent attention needs dk = 576 and dv = 512");
    LSI_SUPPORT(n_heads % 16 == 0, "bf16 latent attention needs n_heads a multiple of 16");
    LSI_REQUIRE(v == nullptr, "bf16 latent attention reads V from kv; v must be NULL");
    LSI_REQUIRE(aligned(q, 16) && aligned(out, 16), "q and out must be 16-byte aligned");
  } else if (kv->dtype == LSI_F32) {
    LSI_SUPPORT(dk <= 256 && dv >= 1 && dv <= 256, "f32 attention supports dk, dv <= 256");
    LSI_SUPPORT(n_heads <= 65535, "f32 attention supports n_heads <= 65535");
    LSI_REQUIRE(v != nullptr, "f32 attention needs a separate value cache v");
    LSI_TRY(check_cache(v, batch, "v"));
    LSI_REQUIRE(v->dtype == LSI_F32 && v->dim == dv, "v must be f32 with dim == dv");
    LSI_REQUIRE(v->page_size == kv->page_size && v->num_pages == kv->num_pages,
                "v must share kv's page geometry");
  } else {
    return fail(LSI_ERR_UNSUPPORTED, "attention caches must be bf16 (latent) or f32");
  }
  return LSI_OK;
}

AttnArgs attn_args(const lsi_paged_cache* kv, const lsi_paged_cache* v, const lsi_batch* batch,
                   const void* q, int32_t n_heads, int32_t dk, int32_t dv, const int32_t* idx,
                   int32_t k, float sm_scale, void* out, float* lse, void* ws) {
  AttnArgs a;
  a.kv = kv->data;
  a.v = v ? v->data : nullptr;
  a.num_pages = kv->num_pages;
  a.page_size = kv->page_size;
  a.seq_lens = batch->seq_lens;
  a.page_table = batch->page_table;
  a.max_pages = batch->max_pages;
  a.max_seq_len = batch->max_seq_len;
  a.num_req = batch->num_req;
  a.q = q;
  a.n_heads = n_heads;
  a.dk = dk;
  a.dv = dv;
  a.idx = idx;
  a.k = k;
  a.sm_scale = sm_scale;
  a.out = out;
  a.lse = lse;
  a.ws = ws;
  return a;
}

size_t attn_ws(int dtype, int num_req, int n_heads, int dv, int k) {
  return dtype == LSI_BF16 ? mla_ws_bytes(num_req, n_heads, dv, k) : 0;
}

hipError_t run_attn(int dtype, const AttnArgs& a, hipStream_t s) {
  return dtype == LSI_BF16 ? launch_mla_bf16(a, s) : launch_attn_f32(a, s);
}

int64_t scores_ld(int max_seq_len) { return std::max<int64_t>(64, ceil_div(max_seq_len, 64) * 64); }

// ---- prefill events ----------------------------------------------------------
struct PrefillEvents {
  hipEvent_t start = nullptr, copied[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr};
  bool ready = false;
};
std::mutex g_ev_mu;
PrefillEvents g_ev[64];

// A pointer kernels may read: device memory as it is, pinned host memory
// through the device address of its mapping (the same allocation seen from
// the GPU; reads cross the host bus).  Pageable host memory is rejected.
int32_t device_view(const void* p, const void** out, const char* what) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();   // the failed query must not read as a launch error later
    return fail(LSI_ERR_INVALID_ARG, std::string(what) + " is neither device memory nor pinned host memory");
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
    *out = p;
    return LSI_OK;
  }
  if (at.type == hipMemoryTypeHost && at.devicePointer != nullptr) {
    // the offset of p inside the allocation carries over to its device address
    const ptrdiff_t off = at.hostPointer ? static_cast<const char*>(p) - static_cast<const char*>(at.hostPointer) : 0;
    *out = static_cast<const char*>(at.devicePointer) + off;
    return LSI_OK;
  }
  return fail(LSI_ERR_INVALID_ARG, std::string(what) + " is neither device memory nor pinned host memory");
}

// ---- pieces shared by the single- and multi-layer decode steps ---------------
// scan of every cached token (which also clears the top-k counters that the
// selection uses next), then the top-k that also returns the physical rows
int32_t enqueue_select(const lsi_paged_cache* ikeys, const lsi_paged_cache* kv,
                       const lsi_batch* batch, const void* q_idx, int32_t n_idx_heads,
                       int32_t idx_dim, const float* w, int32_t k, int32_t* idx, int32_t* count,
                       float* scores, int64_t ld, void* topk_ws, int32_t* phys, hipStream_t stream,
                       const char* what, bool defer = false, uint32_t* hist_rep = nullptr) {
  ScanArgs sa = scan_args(ikeys, batch, q_idx, n_idx_heads, idx_dim, w, scores, ld);
  sa.zero_ptr = static_cast<uint32_t*>(topk_ws);
  sa.zero_words = topk_zero_words(batch->num_req);
  sa.hist_rep = hist_rep;
  LSI_LAUNCH(run_scan(ikeys->dtype, sa, stream), std::string(what) + " (scan)");

  TopkArgs t;
  t.scores = scores;
  t.ld = ld;
  t.seq_lens = batch->seq_lens;
  t.num_req = batch->num_req;
  t.max_len = batch->max_seq_len;
  t.k = k;
  t.idx = idx;
  t.count = count;
  t.ws = topk_ws;
  t.phys = phys;
  t.page_table = batch->page_table;
  t.max_pages = batch->max_pages;
  t.page_size = kv->page_size;
  t.num_pages = kv->num_pages;
  t.defer = defer ? 1 : 0;
  t.hist_rep = hist_rep;
  LSI_LAUNCH(launch_topk(t, 1, stream), std::string(what) + " (top-k)");
  return LSI_OK;
}

// attention over a selection whose physical rows the top-k already wrote
int32_t enqueue_attend(const lsi_paged_cache* kv, const lsi_paged_cache* v, const lsi_batch* batch,
                       const void* q_attn, int32_t n_heads, int32_t dk, int32_t dv,
                       const int32_t* idx, int32_t k, float sm_scale, void* out, float* lse,
                       void* attn_wsp, const int32_t* phys, hipStream_t stream, const char* what,
                       void* deferred_topk_ws = nullptr, int32_t* idx_out = nullptr,
                       uint32_t* zero_ptr = nullptr, int64_t zero_words = 0) {
  AttnArgs a = attn_args(kv, v, batch, q_attn, n_heads, dk, dv, idx, k, sm_scale, out, lse, attn_wsp);
  a.phys = phys;
  a.tk_ws = deferred_topk_ws;
  a.tk_max_len = batch->max_seq_len;
  a.idx_out = idx_out;
  a.phys_out = deferred_topk_ws ? const_cast<int32_t*>(phys) : nullptr;
  a.zero_ptr = zero_ptr;
  a.zero_words = zero_words;
  LSI_LAUNCH(run_attn(kv->dtype, a, stream), std::string(what) + " (attention)");
  return LSI_OK;
}

// ---- multi-layer events --------------------------------------------------------
constexpr int kMaxLayers = 4096;
struct LayerEvents {
  hipEvent_t attn_done = nullptr, selected = nullptr;
  bool ready = false;
};
std::mutex g_ml_mu;
LayerEvents g_ml_ev[64];

}  // namespace
}  // namespace lsi

using namespace lsi;

extern "C" {

int32_t lsi_version(void) { return 101; }

const char* lsi_status_string(int32_t status) {
  switch (status) {
    case LSI_OK: return "ok";
    case LSI_ERR_INVALID_ARG: return "invalid argument";
    case LSI_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case LSI_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case LSI_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* lsi_last_error(void) { return g_last_error.c_str(); }
const char* lsi_last_error_detail(void) { return g_last_error.c_str(); }

int32_t lsi_profile_events(hipEvent_t* events, const char** names, int32_t capacity) {
  const int32_t recorded = g_prof.used;
  if (events == nullptr || capacity <= 0) {
    g_prof = ProfState{};
  } else {
    g_prof.ev = events;
    g_prof.names = names;
    g_prof.cap = capacity;
    g_prof.used = 0;
  }
  return recorded;
}

int32_t lsi_index_scores(const lsi_paged_cache* ikeys, const lsi_batch* batch, const void* q,
                         int32_t n_heads, int32_t dim, const float* w, float* scores, int64_t ld,
                         hipStream_t stream) {
  LSI_TRY(validate_index(ikeys, batch, q, n_heads, dim, w, scores, ld));
  const ScanArgs a = scan_args(ikeys, batch, q, n_heads, dim, w, scores, ld);
  LSI_LAUNCH(run_scan(ikeys->dtype, a, stream), "lsi_index_scores");
  return check_launch("lsi_index_scores");
}

size_t lsi_topk_workspace_bytes(int32_t num_req, int32_t max_seq_len, int32_t k) {
  (void)k;
  if (num_req < 1 || max_seq_len < 0) return 0;
  return topk_ws_bytes(num_req, max_seq_len);
}

int32_t lsi_topk(const float* scores, int64_t ld, const lsi_batch* batch, int32_t k, int32_t* idx,
                 int32_t* count, void* workspace, size_t ws_bytes, hipStream_t stream) {
  LSI_TRY(validate_topk(scores, ld, batch, k, idx, count));
  LSI_TRY(check_ws(workspace, ws_bytes, topk_ws_bytes(batch->num_req, batch->max_seq_len)));
  TopkArgs t;
  t.scores = scores;
  t.ld = ld;
  t.seq_lens = batch->seq_lens;
  t.num_req = batch->num_req;
  t.max_len = batch->max_seq_len;
  t.k = k;
  t.idx = idx;
  t.count = count;
  t.ws = workspace;
  LSI_LAUNCH(launch_topk(t, 0, stream), "lsi_topk");
  return check_launch("lsi_topk");
}

size_t lsi_sparse_mla_workspace_bytes(int32_t num_req, int32_t n_heads, int32_t dv, int32_t k) {
  if (num_req < 1 || n_heads < 1 || dv < 1 || k < 1) return 0;
  // the bf16 latent path is the only one with scratch
  if (n_heads % 16 != 0 || dv != 512) return 0;
  return mla_ws_bytes(num_req, n_heads, dv, k);
}

int32_t lsi_sparse_mla_decode(const lsi_paged_cache* kv, const lsi_paged_cache* v,
                              const lsi_batch* batch, const void* q, int32_t n_heads, int32_t dk,
                              int32_t dv, const int32_t* idx, int32_t k, float sm_scale, void* out,
                              float* lse, void* workspace, size_t ws_bytes, hipStream_t stream) {
  LSI_TRY(validate_attn(kv, v, batch, q, n_heads, dk, dv, idx, k, sm_scale, out, lse));
  LSI_TRY(check_ws(workspace, ws_bytes, attn_ws(kv->dtype, batch->num_req, n_heads, dv, k)));
  const AttnArgs a = attn_args(kv, v, batch, q, n_heads, dk, dv, idx, k, sm_scale, out, lse, workspace);
  LSI_LAUNCH(run_attn(kv->dtype, a, stream), "lsi_sparse_mla_decode");
  return check_launch("lsi_sparse_mla_decode");
}

size_t lsi_decode_step_state_bytes(int32_t num_req) {
  if (num_req < 1) return 0;
  return align_up((size_t)num_req * kHistReps * kHistWords * sizeof(uint32_t), kWsAlign);
}

size_t lsi_decode_step_workspace_bytes(int32_t num_req, int32_t max_seq_len, int32_t k,
                                       int32_t n_heads, int32_t dv) {
  if (num_req < 1 || max_seq_len < 0 || k < 1 || n_heads < 1) return 0;
  const size_t st = lsi_decode_step_state_bytes(num_req);
  const size_t sc = align_up((size_t)num_req * scores_ld(max_seq_len) * sizeof(float), kWsAlign);
  const size_t tk = topk_ws_bytes(num_req, max_seq_len);
  const size_t ph = align_up((size_t)num_req * k * sizeof(int32_t), kWsAlign);
  const size_t at = (n_heads % 16 == 0 && dv == 512) ? mla_ws_bytes(num_req, n_heads, dv, k) : 0;
  return st + sc + tk + ph + at;
}

}  // extern "C"

namespace lsi {
namespace {

int32_t validate_decode_step(const lsi_paged_cache* ikeys, const lsi_paged_cache* kv,
                             const lsi_paged_cache* v, const lsi_batch* batch, const void* q_idx,
                             int32_t n_idx_heads, int32_t idx_dim, const float* w,
                             const void* q_attn, int32_t n_heads, int32_t dk, int32_t dv,
                             float sm_scale, int32_t k, const int32_t* idx, const int32_t* count,
                             const void* out, const float* lse) {
  LSI_TRY(check_batch(batch, true));
  LSI_TRY(validate_index(ikeys, batch, q_idx, n_idx_heads, idx_dim, w, nullptr, 0, true));
  LSI_REQUIRE(ikeys->page_size == kv->page_size, "ikeys and kv must share the page size");
  LSI_REQUIRE(k >= 1 && k <= 65536, "k must be in [1, 65536]");
  LSI_REQUIRE(idx != nullptr && count != nullptr, "idx and count must be non-NULL");
  LSI_TRY(validate_attn(kv, v, batch, q_attn, n_heads, dk, dv, idx, k, sm_scale, out, lse));
  return LSI_OK;
}

// The launches of one decode step over a validated call and a workspace of
// at least lsi_decode_step_workspace_bytes().
int32_t enqueue_decode_step(const lsi_paged_cache* ikeys, const lsi_paged_cache* kv,
                            const lsi_paged_cache* v, const lsi_batch* batch, const void* q_idx,
                            int32_t n_idx_heads, int32_t idx_dim, const float* w,
                            const void* q_attn, int32_t n_heads, int32_t dk, int32_t dv,
                            float sm_scale, int32_t k, int32_t* idx, int32_t* count, void* out,
                            float* lse, void* workspace, hipStream_t stream, const char* what) {
  const int64_t ld = scores_ld(batch->max_seq_len);
  char* ws = static_cast<char*>(workspace);
  // state kept between calls (zero on entry and on return): the replicated
  // histograms the scan builds for the top-k
  uint32_t* hist_rep = reinterpret_cast<uint32_t*>(ws);
  ws += lsi_decode_step_state_bytes(batch->num_req);
  float* scores = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)batch->num_req * ld * sizeof(float), kWsAlign);
  void* topk_ws = ws;
  ws += topk_ws_bytes(batch->num_req, batch->max_seq_len);
  int32_t* phys = reinterpret_cast<int32_t*>(ws);   // physical rows of the selection
  ws += align_up((size_t)batch->num_req * k * sizeof(int32_t), kWsAlign);
  void* attn_wsp = ws;

  // The threshold bin of long rows is left to the attention kernel when the
  // 16-head latent kernel runs (one launch fewer): it resolves the slots it
  // reads from the top-k workspace and writes their positions to idx.
  const bool defer = kv->dtype == LSI_BF16 && mla_resolves(batch->num_req, n_heads, k) &&
                     topk_can_defer(batch->num_req, batch->max_seq_len);
  // One request with fp8 keys: the scan also builds the top-k's histograms
  // (no histogram launch); the attention clears them again afterwards.
  const bool scan_hist = defer && ikeys->dtype == LSI_FP8_E4M3 &&
                         scan_builds_hist(batch->num_req, batch->max_seq_len, ikeys->page_size);
  LSI_TRY(enqueue_select(ikeys, kv, batch, q_idx, n_idx_heads, idx_dim, w, k, idx, count, scores,
                         ld, topk_ws, phys, stream, what, defer, scan_hist ? hist_rep : nullptr));
  LSI_TRY(enqueue_attend(kv, v, batch, q_attn, n_heads, dk, dv, idx, k, sm_scale, out, lse,
                         attn_wsp, phys, stream, what, defer ? topk_ws : nullptr, defer ? idx : nullptr,
                         scan_hist ? hist_rep : nullptr,
                         scan_hist ? (int64_t)batch->num_req * kHistReps * kHistWords : 0));
  return check_launch(what);
}

// Library-owned scratch of lsi_decode_step_noalloc: one copy of this array
// per GPU, which holds it until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol); it uses the device address that hipGetSymbolAddress returns for
// the current device, looked up once per device.
constexpr size_t kNoAllocScratch = LSI_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kNoAllocScratch];
std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {};

int32_t scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(LSI_ERR_HIP, "lsi_decode_step_noalloc: no current device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(LSI_ERR_HIP, std::string("lsi_decode_step_noalloc: scratch address: ") + hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return LSI_OK;
}

}  // namespace
}  // namespace lsi

extern "C" {

int32_t lsi_decode_step(const lsi_paged_cache* ikeys, const lsi_paged_cache* kv,
                        const lsi_paged_cache* v, const lsi_batch* batch, const void* q_idx,
                        int32_t n_idx_heads, int32_t idx_dim, const float* w, const void* q_attn,
                        int32_t n_heads, int32_t dk, int32_t dv, float sm_scale, int32_t k,
                        int32_t* idx, int32_t* count, void* out, float* lse, void* workspace,
                        size_t ws_bytes, hipStream_t stream) {
  LSI_TRY(validate_decode_step(ikeys, kv, v, batch, q_idx, n_idx_heads, idx_dim, w, q_attn, n_heads,
                               dk, dv, sm_scale, k, idx, count, out, lse));
  const size_t need = lsi_decode_step_workspace_bytes(batch->num_req, batch->max_seq_len, k, n_heads, dv);
  LSI_TRY(check_ws(workspace, ws_bytes, need));
  return enqueue_decode_step(ikeys, kv, v, batch, q_idx, n_idx_heads, idx_dim, w, q_attn, n_heads, dk,
                             dv, sm_scale, k, idx, count, out, lse, workspace, stream,
                             "lsi_decode_step");
}

int32_t lsi_decode_step_noalloc(const lsi_paged_cache* ikeys, const lsi_paged_cache* kv,
                                const lsi_paged_cache* v, const lsi_batch* batch,
                                const void* q_idx, int32_t n_idx_heads, int32_t idx_dim,
                                const float* w, const void* q_attn, int32_t n_heads, int32_t dk,
                                int32_t dv, float sm_scale, int32_t k, int32_t* idx,
                                int32_t* count, void* out, float* lse, hipStream_t stream) {
  LSI_TRY(validate_decode_step(ikeys, kv, v, batch, q_idx, n_idx_heads, idx_dim, w, q_attn, n_heads,
                               dk, dv, sm_scale, k, idx, count, out, lse));
  const size_t need = lsi_decode_step_workspace_bytes(batch->num_req, batch->max_seq_len, k, n_heads, dv);
  if (need > kNoAllocScratch)
    return fail(LSI_ERR_WORKSPACE, "lsi_decode_step_noalloc: the call needs " + std::to_string(need) +
                                       " bytes of scratch; the library's fixed scratch holds " +
                                       std::to_string(kNoAllocScratch));
  void* ws = nullptr;
  LSI_TRY(scratch_for_current_device(&ws));
  return enqueue_decode_step(ikeys, kv, v, batch, q_idx, n_idx_heads, idx_dim, w, q_attn, n_heads, dk,
                             dv, sm_scale, k, idx, count, out, lse, ws, stream,
                             "lsi_decode_step_noalloc");
}

size_t lsi_multilayer_workspace_bytes(int32_t num_req, int32_t max_seq_len, int32_t k,
                                      int32_t n_heads, int32_t dv) {
  if (num_req < 1 || max_seq_len < 0 || k < 1 || n_heads < 1) return 0;
  const size_t st = lsi_decode_step_state_bytes(num_req);
  const size_t sc = align_up((size_t)num_req * scores_ld(max_seq_len) * sizeof(float), kWsAlign);
  const size_t tk = topk_ws_bytes(num_req, max_seq_len);
  const size_t ph = align_up((size_t)num_req * k * sizeof(int32_t), kWsAlign);
  const size_t at = (n_heads % 16 == 0 && dv == 512) ? mla_ws_bytes(num_req, n_heads, dv, k) : 0;
  return 2 * st + sc + 2 * tk + 2 * ph + at;
}

int32_t lsi_multilayer_decode(int32_t n_layers, int32_t retention, int32_t schedule,
                              const lsi_paged_cache* ikeys, const lsi_paged_cache* kv,
                              const lsi_batch* batch, const void* const* q_idx,
                              int32_t n_idx_heads, int32_t idx_dim, const float* const* w,
                              const void* const* q_attn, int32_t n_heads, int32_t dk, int32_t dv,
                              float sm_scale, int32_t k, int32_t* const* idx,
                              int32_t* const* count, void* const* out, float* const* lse,
                              void* workspace, size_t ws_bytes, hipStream_t stream,
                              hipStream_t s_index) {
  LSI_REQUIRE(n_layers >= 1 && n_layers <= kMaxLayers, "n_layers must be in [1, 4096]");
  LSI_REQUIRE(retention >= 1 && retention <= n_layers, "retention must be in [1, n_layers]");
  LSI_REQUIRE(schedule == LSI_SCHED_SERIAL || schedule == LSI_SCHED_MLI, "unknown schedule");
  LSI_REQUIRE(ikeys != nullptr && kv != nullptr && q_idx != nullptr && w != nullptr &&
                  q_attn != nullptr && idx != nullptr && count != nullptr && out != nullptr &&
                  lse != nullptr,
              "the per-layer host arrays must be non-NULL");
  LSI_TRY(check_batch(batch, true));
  LSI_REQUIRE(k >= 1 && k <= 65536, "k must be in [1, 65536]");
  const int64_t ld = scores_ld(batch->max_seq_len);
  for (int l = 0; l < n_layers; ++l) {
    const std::string at = "layer " + std::to_string(l) + ": ";
    if (l % retention == 0) {
      const int32_t st = validate_index(&ikeys[l], batch, q_idx[l], n_idx_heads, idx_dim, w[l],
                                        nullptr, 0, true);
      if (st != LSI_OK) return fail(st, at + g_last_error);
      LSI_REQUIRE(ikeys[l].page_size == kv[l].page_size, at + "ikeys and kv must share the page size");
      LSI_REQUIRE(idx[l / retention] != nullptr && count[l / retention] != nullptr,
                  at + "idx and count must be non-NULL");
    }
    LSI_SUPPORT(kv[l].dtype == LSI_BF16, at + "the multi-layer step needs the bf16 latent cache");
    LSI_REQUIRE(kv[l].num_pages == kv[0].num_pages && kv[l].page_size == kv[0].page_size,
                at + "every layer's cache must have the shape of layer 0's");
    const int32_t st = validate_attn(&kv[l], nullptr, batch, q_attn[l], n_heads, dk, dv,
                                     idx[(l / retention)], k, sm_scale, out[l], lse[l]);
    if (st != LSI_OK) return fail(st, at + g_last_error);
  }
  const size_t need = lsi_multilayer_workspace_bytes(batch->num_req, batch->max_seq_len, k, n_heads, dv);
  LSI_TRY(check_ws(workspace, ws_bytes, need));

  // Per selection slot parity: the scan-built histograms (state kept between
  // calls, zero on entry and on return), the top-k workspace and the
  // physical rows, so that the attention reading slot s - 1 (and resolving
  // its threshold bin) never shares them with the indexer filling slot s.
  char* ws = static_cast<char*>(workspace);
  uint32_t* state[2];
  const size_t st_bytes = lsi_decode_step_state_bytes(batch->num_req);
  for (int i = 0; i < 2; ++i) {
    state[i] = reinterpret_cast<uint32_t*>(ws);
    ws += st_bytes;
  }
  float* scores = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)batch->num_req * ld * sizeof(float), kWsAlign);
  void* topk_ws[2];
  for (int i = 0; i < 2; ++i) {
    topk_ws[i] = ws;
    ws += topk_ws_bytes(batch->num_req, batch->max_seq_len);
  }
  int32_t* phys[2];
  for (int i = 0; i < 2; ++i) {
    phys[i] = reinterpret_cast<int32_t*>(ws);
    ws += align_up((size_t)batch->num_req * k * sizeof(int32_t), kWsAlign);
  }
  void* attn_wsp = ws;
  // the one-layer step's launches: the threshold bin left to the attention,
  // and (fp8 keys, one request) the histograms built by the scan
  const bool defer = mla_resolves(batch->num_req, n_heads, k) &&
                     topk_can_defer(batch->num_req, batch->max_seq_len);
  bool scan_hist = defer;
  for (int l = 0; l < n_layers && scan_hist; l += retention)
    scan_hist = ikeys[l].dtype == LSI_FP8_E4M3 &&
                scan_builds_hist(batch->num_req, batch->max_seq_len, ikeys[l].page_size);
  const int64_t st_words = (int64_t)batch->num_req * kHistReps * kHistWords;

  const bool mli = schedule == LSI_SCHED_MLI;
  const bool split = mli && s_index != nullptr && s_index != stream;
  hipStream_t si = split ? s_index : stream;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(LSI_ERR_HIP, "lsi_multilayer_decode: no current device");
  std::lock_guard<std::mutex> lock(g_ml_mu);
  LayerEvents& ev = g_ml_ev[dev];
  if (split && !ev.ready) {
    hipError_t e = hipEventCreateWithFlags(&ev.attn_done, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev.selected, hipEventDisableTiming);
    if (e != hipSuccess) return fail(LSI_ERR_HIP, std::string("event create: ") + hipGetErrorString(e));
    ev.ready = true;
  }
#define LSI_HIP(expr)                                                                     \
  do {                                                                                    \
    const hipError_t _e = (expr);                                                         \
    if (_e != hipSuccess)                                                                 \
      return fail(LSI_ERR_HIP, std::string("lsi_multilayer_decode: ") + hipGetErrorString(_e)); \
  } while (0)
  // `pending`: a selection made on si that `stream` has not waited for yet.
  // There is at most one: the next layer that reads it waits before the next
  // indexer records the event again.
  // MLI: when the last layer has an indexer, no attention of this call reads
  // the last selection, so nothing would resolve a threshold bin left open:
  // that selection is finished by the top-k itself
  const int last_slot = (n_layers - 1) / retention;
  const bool last_unread = mli && (n_layers - 1) % retention == 0 && last_slot >= 1;
  bool pending = false;
  for (int l = 0; l < n_layers; ++l) {
    const int slot = l / retention;
    const bool indexer = l % retention == 0;
    const bool fin = last_unread && slot == last_slot;
    if (pending) {
      LSI_HIP(hipStreamWaitEvent(stream, ev.selected, 0));
      pending = false;
    }
    int src = slot;   // the selection this layer attends
    if (indexer && mli && l > 0) {
      // the indexer of layer l starts once layer l-1 is done (in a model its
      // query comes from that layer's output) and runs beside the attention
      // of layer l, which reads the previous indexer layer's selection
      src = slot - 1;
      if (split) {
        LSI_HIP(hipEventRecord(ev.attn_done, stream));
        LSI_HIP(hipStreamWaitEvent(si, ev.attn_done, 0));
      }
      LSI_TRY(enqueue_select(&ikeys[l], &kv[l], batch, q_idx[l], n_idx_heads, idx_dim, w[l], k,
                             idx[slot], count[slot], scores, ld, topk_ws[slot & 1], phys[slot & 1], si,
                             "lsi_multilayer_decode", defer && !fin,
                             scan_hist && !fin ? state[slot & 1] : nullptr));
      if (split) {
        LSI_HIP(hipEventRecord(ev.selected, si));
        pending = true;   // the next layer waits for it; this one does not
      }
    } else if (indexer) {
      LSI_TRY(enqueue_select(&ikeys[l], &kv[l], batch, q_idx[l], n_idx_heads, idx_dim, w[l], k,
                             idx[slot], count[slot], scores, ld, topk_ws[slot & 1], phys[slot & 1],
                             stream, "lsi_multilayer_decode", defer,
                             scan_hist ? state[slot & 1] : nullptr));
    }
    // The first attention after a selection was made clears that
    // selection's histograms (its top-k has read them): the layer's own
    // (serial, and layer 0) or the previous slot's (an MLI indexer layer,
    // whose own top-k may still be reading its own).
    uint32_t* clear = nullptr;
    if (scan_hist && indexer) clear = state[src & 1];
    LSI_TRY(enqueue_attend(&kv[l], nullptr, batch, q_attn[l], n_heads, dk, dv, idx[src], k,
                           sm_scale, out[l], lse[l], attn_wsp, phys[src & 1], stream,
                           "lsi_multilayer_decode", defer ? topk_ws[src & 1] : nullptr,
                           defer ? idx[src] : nullptr, clear, clear ? st_words : 0));
  }
  if (pending) LSI_HIP(hipStreamWaitEvent(stream, ev.selected, 0));
  // MLI: the last selection's histograms (when the scan built them) were
  // read by its top-k but cleared by no attention
  if (scan_hist && mli && last_slot >= 1 && !last_unread)
    LSI_HIP(launch_zero(state[last_slot & 1], st_words, stream));
#undef LSI_HIP
  return check_launch("lsi_multilayer_decode");
}

size_t lsi_two_stage_workspace_bytes(int32_t num_req, int32_t max_seq_len, int32_t n_cand,
                                     int32_t k) {
  if (num_req < 1 || max_seq_len < 0 || n_cand < 1 || k < 1) return 0;
  (void)k;
  // one request: the state words of the compact scan's histograms first
  const size_t st = num_req == 1 ? lsi_decode_step_state_bytes(1) : 0;
  const size_t s4 = align_up((size_t)num_req * scores_ld(max_seq_len) * 4, kWsAlign);
  const size_t rg = align_up((size_t)kMaxRangeSlots * 16, kWsAlign);
  const size_t t1 = topk_ws_bytes(num_req, max_seq_len);
  const size_t cand = align_up((size_t)num_req * n_cand * 4, kWsAlign);
  const size_t ccount = align_up((size_t)num_req * 4, kWsAlign);
  const size_t s8 = align_up((size_t)num_req * n_cand * 4, kWsAlign);
  const size_t t2 = topk_ws_bytes(num_req, n_cand);
  return st + s4 + rg + t1 + cand + ccount + s8 + t2;
}

int32_t lsi_two_stage_topk(const lsi_paged_cache* ikeys4, const lsi_paged_cache* ikeys8,
                           const lsi_batch* batch, const void* q, int32_t n_heads, int32_t dim,
                           const float* w, int32_t n_cand, int32_t k, int32_t* idx,
                           int32_t* count, int32_t* cand, void* workspace, size_t ws_bytes,
                           hipStream_t stream) {
  LSI_TRY(check_batch(batch, true));
  const int64_t ld = scores_ld(batch->max_seq_len);
  LSI_TRY(validate_index(ikeys4, batch, q, n_heads, dim, w, nullptr, 0, true));
  LSI_TRY(validate_index(ikeys8, batch, q, n_heads, dim, w, nullptr, 0, true));
  LSI_REQUIRE(ikeys4->dtype == LSI_INT4, "ikeys4 must be LSI_INT4");
  LSI_REQUIRE(ikeys8->dtype == LSI_FP8_E4M3, "ikeys8 must be LSI_FP8_E4M3");
  LSI_REQUIRE(ikeys4->page_size == ikeys8->page_size && ikeys4->num_pages == ikeys8->num_pages,
              "ikeys4 and ikeys8 must share the page geometry");
  LSI_REQUIRE(k >= 1 && n_cand >= k && n_cand <= 65536, "need 1 <= k <= n_cand <= 65536");
  LSI_REQUIRE(idx != nullptr && count != nullptr, "idx and count must be non-NULL");
  LSI_TRY(check_ws(workspace, ws_bytes,
                   lsi_two_stage_workspace_bytes(batch->num_req, batch->max_seq_len, n_cand, k)));
  // the original keys may live in pinned host memory: the rescoring reads
  // only the candidates' rows, over the host bus
  lsi_paged_cache k8 = *ikeys8;
  LSI_TRY(device_view(ikeys8->data, &k8.data, "ikeys8->data"));
  const void* sc8 = nullptr;
  LSI_TRY(device_view(ikeys8->scale, &sc8, "ikeys8->scale"));
  k8.scale = static_cast<const float*>(sc8);
  const int B = batch->num_req;
  char* ws = static_cast<char*>(workspace);
  // One request: the compact scan also builds the first top-k's histograms
  // (fixed 12- and 6-bit key digits, no histogram launch) in the state words
  // at the start of the workspace, which the exact scan clears again.
  uint32_t* hist_rep = reinterpret_cast<uint32_t*>(ws);
  const bool scan_hist = B == 1 && scan_builds_hist(1, batch->max_seq_len, ikeys4->page_size);
  if (B == 1) ws += lsi_decode_step_state_bytes(1);
  void* t2 = ws;               // the second top-k's workspace (counters first)
  ws += topk_ws_bytes(B, n_cand);
  float* s4 = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)B * ld * 4, kWsAlign);
  uint4* rslots = reinterpret_cast<uint4*>(ws);   // the int4 scan's per-workgroup key ranges
  ws += align_up((size_t)kMaxRangeSlots * 16, kWsAlign);
  void* t1 = ws;
  ws += topk_ws_bytes(B, batch->max_seq_len);
  int32_t* cl = reinterpret_cast<int32_t*>(ws);
  ws += align_up((size_t)B * n_cand * 4, kWsAlign);
  int32_t* cc = reinterpret_cast<int32_t*>(ws);
  ws += align_up((size_t)B * 4, kWsAlign);
  float* s8 = reinterpret_cast<float*>(ws);

  // stage 1: compact keys over every token, keep n_cand.  The scan clears
  // the top-k's counters and either builds its histograms (one request) or
  // records each workgroup's key range, so that the histogram launch's first
  // digit spans the row's range (the compact scores crowd into a few
  // binades: with the fixed digit the threshold bin holds ~2% of a row,
  // which the refinement's second digit splits).
  ScanArgs a4 = scan_args(ikeys4, batch, q, n_heads, dim, w, s4, ld);
  a4.zero_ptr = static_cast<uint32_t*>(t1);
  a4.zero_words = topk_zero_words(B);
  a4.range_slots = scan_hist ? nullptr : rslots;
  a4.hist_rep = scan_hist ? hist_rep : nullptr;
  int nslots = 0;
  LSI_LAUNCH(launch_scan_int4(a4, stream, &nslots), "lsi_two_stage_topk (compact scan)");
  TopkArgs ta;
  ta.scores = s4;
  ta.range_slots = nslots > 0 ? rslots : nullptr;
  ta.range_nslots = nslots;
  ta.hist_rep = a4.hist_rep;
  ta.ld = ld;
  ta.seq_lens = batch->seq_lens;
  ta.num_req = B;
  ta.max_len = batch->max_seq_len;
  ta.k = n_cand;
  ta.idx = cl;
  ta.count = cc;
  ta.ws = t1;
  LSI_LAUNCH(launch_topk(ta, 1, stream), "lsi_two_stage_topk (first top-k)");

  // stage 2: exact fp8 scores of the candidates only, keep k
  ScanArgs a8 = scan_args(&k8, batch, q, n_heads, dim, w, s8, n_cand);
  a8.positions = cl;
  a8.n_pos = n_cand;
  // (it clears the second top-k's counters and, after the first top-k has
  // read them, the histogram state words just before them)
  a8.zero_ptr = scan_hist ? hist_rep : static_cast<uint32_t*>(t2);
  a8.zero_words = topk_zero_words(B) + (scan_hist ? (int64_t)(static_cast<char*>(t2) - reinterpret_cast<char*>(hist_rep)) / 4 : 0);
  LSI_LAUNCH(launch_scan_fp8(a8, stream), "lsi_two_stage_topk (exact scan)");
  TopkArgs tb;
  tb.scores = s8;
  tb.ld = n_cand;
  tb.seq_lens = cc;          // row length = number of stage-1 candidates
  tb.num_req = B;
  tb.max_len = n_cand;
  tb.k = k;
  tb.map = cl;               // slot -> position
  tb.map_ld = n_cand;
  tb.idx = idx;
  tb.count = count;
  tb.ws = t2;
  LSI_LAUNCH(launch_topk(tb, 1, stream), "lsi_two_stage_topk (second top-k)");
  if (cand) {
    const hipError_t e = hipMemcpyAsync(cand, cl, (size_t)B * n_cand * 4, hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return fail(LSI_ERR_HIP, std::string("lsi_two_stage_topk: ") + hipGetErrorString(e));
  }
  return check_launch("lsi_two_stage_topk");
}

size_t lsi_prefill_workspace_bytes(int32_t hist_len, int32_t T, int32_t dim, int32_t block_tokens,
                                   int32_t k, int32_t scores_external) {
  (void)hist_len;
  (void)scores_external;   // the scores are never stored in the workspace
  if (hist_len < 0 || T < 1 || dim < 1 || block_tokens < 1 || k < 1 || k > 65536) return 0;
  const size_t bufk = align_up((size_t)block_tokens * dim, kWsAlign);
  const size_t bufs = align_up((size_t)block_tokens * 4, kWsAlign);
  const size_t cand = align_up((size_t)T * prefill_cand_cap(k) * 8, kWsAlign);
  const size_t state = align_up((size_t)T * 8, kWsAlign);
  return 2 * (bufk + bufs) + cand + state;
}

int32_t lsi_prefill_index_topk(const uint8_t* hist_keys, const float* hist_scale, int32_t hist_len,
                               const uint8_t* chunk_keys, const float* chunk_scale, int32_t T,
                               const void* q, int32_t n_heads, int32_t dim, const float* w,
                               int32_t k, int32_t block_tokens, int32_t* idx, int32_t* count,
                               float* scores, void* workspace, size_t ws_bytes,
                               hipStream_t s_compute, hipStream_t s_copy) {
  LSI_REQUIRE(hist_len >= 0 && T >= 1, "need hist_len >= 0 and T >= 1");
  LSI_REQUIRE((int64_t)hist_len + T <= INT32_MAX / 2, "hist_len + T too large");
  LSI_REQUIRE(hist_len == 0 || (hist_keys != nullptr && hist_scale != nullptr),
              "hist_keys and hist_scale are required when hist_len > 0");
  LSI_REQUIRE(chunk_keys != nullptr && chunk_scale != nullptr, "chunk_keys and chunk_scale are required");
  LSI_REQUIRE(q != nullptr && w != nullptr && idx != nullptr && count != nullptr,
              "q, w, idx and count must be non-NULL");
  LSI_SUPPORT(n_heads == 64 && dim == 128, "the prefill indexer needs 64 heads of dim 128");
  LSI_REQUIRE(k >= 1 && k <= 65536, "k must be in [1, 65536]");
  LSI_REQUIRE(block_tokens >= 32 && block_tokens % 32 == 0, "block_tokens must be a positive multiple of 32");
  LSI_REQUIRE(aligned(q, 16) && aligned(chunk_keys, 16), "q and chunk_keys must be 16-byte aligned");
  const size_t need = lsi_prefill_workspace_bytes(hist_len, T, dim, block_tokens, k, scores != nullptr);
  LSI_TRY(check_ws(workspace, ws_bytes, need));
  if (s_copy == nullptr) s_copy = s_compute;

  const int64_t ld = (int64_t)hist_len + T;
  char* ws = static_cast<char*>(workspace);
  uint8_t* bufk[2];
  float* bufs[2];
  for (int i = 0; i < 2; ++i) {
    bufk[i] = reinterpret_cast<uint8_t*>(ws);
    ws += align_up((size_t)block_tokens * dim, kWsAlign);
    bufs[i] = reinterpret_cast<float*>(ws);
    ws += align_up((size_t)block_tokens * 4, kWsAlign);
  }
  const int cap = prefill_cand_cap(k);
  uint2* cand = reinterpret_cast<uint2*>(ws);          // [T][cap] running candidates
  ws += align_up((size_t)T * cap * 8, kWsAlign);
  uint32_t* state = reinterpret_cast<uint32_t*>(ws);   // [T][2] count, entry threshold

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(LSI_ERR_HIP, "lsi_prefill_index_topk: no current device");
  std::lock_guard<std::mutex> lock(g_ev_mu);
  PrefillEvents& ev = g_ev[dev];
  if (!ev.ready) {
    hipError_t e = hipEventCreateWithFlags(&ev.start, hipEventDisableTiming);
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
      e = hipEventCreateWithFlags(&ev.copied[i], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&ev.done[i], hipEventDisableTiming);
    }
    if (e != hipSuccess) return fail(LSI_ERR_HIP, std::string("event create: ") + hipGetErrorString(e));
    ev.ready = true;
  }

#define LSI_HIP(expr)                                                                     \
  do {                                                                                    \
    const hipError_t _e = (expr);                                                         \
    if (_e != hipSuccess)                                                                 \
      return fail(LSI_ERR_HIP, std::string("lsi_prefill_index_topk: ") + hipGetErrorString(_e)); \
  } while (0)
  LSI_HIP(launch_zero(state, 2 * (int64_t)T, s_compute));
  // the copy stream must not overwrite buffers a previous call still reads
  LSI_HIP(hipEventRecord(ev.start, s_compute));
  LSI_HIP(hipStreamWaitEvent(s_copy, ev.start, 0));
  PrefillScanArgs pa;
  pa.q = q;
  pa.w = w;
  pa.T = T;
  pa.hist_len = hist_len;
  pa.scores = scores;
  pa.ld = ld;
  pa.cand = cand;
  pa.state = state;
  pa.cap = cap;
  pa.k = k;
  pa.idx = idx;
  pa.count = count;
  const int nblk = (int)ceil_div(hist_len, block_tokens);
  for (int blk = 0; blk < nblk; ++blk) {
    const int j = blk & 1;
    const int tok0 = blk * block_tokens;
    const int n = std::min(block_tokens, hist_len - tok0);
    if (blk >= 2) LSI_HIP(hipStreamWaitEvent(s_copy, ev.done[j], 0));
    LSI_HIP(hipMemcpyAsync(bufk[j], hist_keys + (size_t)tok0 * dim, (size_t)n * dim, hipMemcpyDefault, s_copy));
    LSI_HIP(hipMemcpyAsync(bufs[j], hist_scale + tok0, (size_t)n * 4, hipMemcpyDefault, s_copy));
    LSI_HIP(hipEventRecord(ev.copied[j], s_copy));
    LSI_HIP(hipStreamWaitEvent(s_compute, ev.copied[j], 0));
    pa.keys = bufk[j];
    pa.kscale = bufs[j];
    pa.tok0 = tok0;
    pa.n_tok = n;
    LSI_HIP(launch_prefill_scan(pa, s_compute));
    LSI_HIP(hipEventRecord(ev.done[j], s_compute));
  }
  pa.keys = chunk_keys;
  pa.kscale = chunk_scale;
  pa.tok0 = hist_len;
  pa.n_tok = T;
  pa.final_block = 1;   // the chunk's own keys come last: selection written here
  LSI_HIP(launch_prefill_scan(pa, s_compute));
#undef LSI_HIP
  return check_launch("lsi_prefill_index_topk");
}

}  // extern "C"

extern "C" size_t lsi_workspace_bytes(int32_t op, const lsi_ws_query* q) {
  if (q == nullptr) return 0;
  switch (op) {
    case LSI_OP_TOPK: return lsi_topk_workspace_bytes(q->num_req, q->max_seq_len, q->k);
    case LSI_OP_SPARSE_MLA: return lsi_sparse_mla_workspace_bytes(q->num_req, q->n_heads, q->dv, q->k);
    case LSI_OP_DECODE_STEP:
      return lsi_decode_step_workspace_bytes(q->num_req, q->max_seq_len, q->k, q->n_heads, q->dv);
    case LSI_OP_MULTILAYER:
      return lsi_multilayer_workspace_bytes(q->num_req, q->max_seq_len, q->k, q->n_heads, q->dv);
    case LSI_OP_TWO_STAGE: return lsi_two_stage_workspace_bytes(q->num_req, q->max_seq_len, q->n_cand, q->k);
    case LSI_OP_PREFILL:
      return lsi_prefill_workspace_bytes(q->max_seq_len, q->num_req, q->dim, q->block_tokens, q->k,
                                         q->scores_external);
    default: return 0;
  }
}

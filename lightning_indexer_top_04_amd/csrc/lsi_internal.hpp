// Internal launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include "lsi_common.hpp"

namespace lsi {

// Arguments of an indexer scan over a paged cache.  In gather mode
// (positions != nullptr) item i of request b is logical position
// positions[b * n_pos + i] and its score goes to scores[b * ld + i];
// otherwise item i is position i.
struct ScanArgs {
  const void* keys = nullptr;       // [num_pages][page_size][row bytes]
  const float* kscale = nullptr;    // [num_pages][page_size]
  int num_pages = 0;
  int page_size = 0;
  const int32_t* seq_lens = nullptr;
  const int32_t* page_table = nullptr;
  int max_pages = 0;
  int max_seq_len = 0;
  int num_req = 0;
  const void* q = nullptr;          // [num_req][H][d]
  const float* w = nullptr;         // [num_req][H]
  float* scores = nullptr;
  int64_t ld = 0;
  const int32_t* positions = nullptr;
  int n_pos = 0;
  int n_heads = 0;
  int dim = 0;
  // optional: clear this many uint32 words at zero_ptr (grid-stride), so a
  // top-k that follows finds its counters at zero without another launch
  uint32_t* zero_ptr = nullptr;
  int64_t zero_words = 0;
  // optional (fp8 keys, contiguous walk, one request, slices of at most
  // 4096 positions: scan_builds_hist): every workgroup adds the histogram of
  // its scores' top 12 key bits (and of their top 6 bits) into replica
  // blockIdx % kHistReps of the row's replicated histogram, which must be
  // zero when the scan starts ([num_req][kHistReps][kHistWords] words)
  uint32_t* hist_rep = nullptr;
  // optional (contiguous walk): every workgroup stores {request, ~lowest
  // key, highest key, 0} of the scores it wrote (request ~0u when it wrote
  // none) at range_slots[its linear index] (the key ranges for the top-k's
  // digits, TopkArgs::range_slots); plain stores, nothing to clear
  uint4* range_slots = nullptr;
};
// most workgroups a scan that records key ranges may use (its slots)
constexpr int kMaxRangeSlots = 8192;
constexpr int kHistReps = 8;
constexpr int kHistWords = 4096 + 64;     // 12-bit digits, then 6-bit digits
// whether a scan of this shape can build the replicated histogram
bool scan_builds_hist(int num_req, int max_seq_len, int page_size);

hipError_t launch_scan_fp8(const ScanArgs& a, hipStream_t s);
hipError_t launch_scan_int4(const ScanArgs& a, hipStream_t s, int* nslots = nullptr);
hipError_t launch_scan_f32(const ScanArgs& a, hipStream_t s);

// ---- top-k ----------------------------------------------------------------
struct TopkArgs {
  const float* scores = nullptr;   // [num_req][ld]
  int64_t ld = 0;
  const int32_t* seq_lens = nullptr;  // per-row length (clamped to max_len)
  int lens_const = -1;             // if >= 0: every row has this length
  int causal_base = -1;            // if >= 0: row r has length causal_base+r+1
  // optional [R][2]: ~(min key), max key of row r, recorded by the producer
  // of the scores; the one-workgroup path's first digit then spans it
  const uint32_t* range = nullptr;
  // optional: the scan's per-workgroup key ranges (ScanArgs::range_slots,
  // range_nslots of them); the multi-workgroup path's histogram launch
  // reduces a row's slots and its digits span the row's key range
  const uint4* range_slots = nullptr;
  int range_nslots = 0;
  int num_req = 0;
  int max_len = 0;
  int k = 0;
  const int32_t* map = nullptr;    // optional: output map[r*map_ld + slot]
  int64_t map_ld = 0;
  int32_t* idx = nullptr;          // [num_req][k]
  int32_t* count = nullptr;        // [num_req]
  void* ws = nullptr;              // workspace (topk_ws_bytes)
  // optional: also write the physical cache row of every kept position
  // (page_table[r][pos / page_size] * page_size + pos % page_size, or -1)
  int32_t* phys = nullptr;         // [num_req][k]
  const int32_t* page_table = nullptr;
  int max_pages = 0;
  int page_size = 1;
  int num_pages = 0;
  // Long rows only (several workgroups per row), with phys: leave the
  // threshold bin to the attention that reads the selection.  When every
  // member of the bin is kept the select writes them itself; otherwise it
  // writes kUnresolvedRow into phys[r][better .. k) and no refinement runs:
  // the attention resolves those slots (resolve_members) and writes idx.
  int defer = 0;
  // optional: the row histograms were built by the scan (ScanArgs::hist_rep,
  // the same array): no histogram launch; the select reads them and places
  // its outputs with one returning atomic per workgroup
  const uint32_t* hist_rep = nullptr;
};
constexpr int32_t kUnresolvedRow = -2;
size_t topk_ws_bytes(int num_req, int max_len);
// words of the workspace that must be zero when the top-k starts
int64_t topk_zero_words(int num_req);
// ws_state: 0 = counters not cleared (clear them first), 1 = already cleared
hipError_t launch_topk(const TopkArgs& a, int ws_state, hipStream_t s);
hipError_t launch_zero(uint32_t* p, int64_t words, hipStream_t s);
// whether launch_topk takes the path that honours TopkArgs::defer
bool topk_can_defer(int num_req, int max_len);

// ---- attention -------------------------------------------------------------
struct AttnArgs {
  const void* kv = nullptr;        // [num_pages][page_size][dk]
  const void* v = nullptr;         // f32 only: [num_pages][page_size][dv]
  int num_pages = 0;
  int page_size = 0;
  const int32_t* seq_lens = nullptr;
  const int32_t* page_table = nullptr;
  int max_pages = 0;
  int max_seq_len = 0;
  int num_req = 0;
  const void* q = nullptr;         // [num_req][H][dk]
  int n_heads = 0;
  int dk = 0;
  int dv = 0;
  const int32_t* idx = nullptr;    // [num_req][k]
  const int32_t* phys = nullptr;   // optional [num_req][k] physical rows of idx (-1 = skip)
  int k = 0;
  float sm_scale = 0.f;
  void* out = nullptr;             // [num_req][H][dv]
  float* lse = nullptr;            // [num_req][H]
  void* ws = nullptr;
  // optional: the top-k workspace of a selection made with TopkArgs::defer
  // (phys rows equal to kUnresolvedRow are resolved from it, and their
  // positions written to idx), and that top-k's max_len
  void* tk_ws = nullptr;
  int tk_max_len = 0;
  int32_t* idx_out = nullptr;      // [num_req][k], receives the resolved positions
  // optional [num_req][k] (the phys array itself): receives the resolved
  // physical rows, so that later attentions over the same selection find no
  // slot left to resolve
  int32_t* phys_out = nullptr;
  // optional: clear this many uint32 words at zero_ptr (grid-stride; the
  // scan-built histograms, once the selection has read them)
  uint32_t* zero_ptr = nullptr;
  int64_t zero_words = 0;
};
size_t mla_ws_bytes(int num_req, int n_heads, int dv, int k);
// whether launch_mla_bf16 resolves deferred selections (AttnArgs::tk_ws) for
// this shape (the 16-head kernel does; the 32-head batch kernel does not)
bool mla_resolves(int num_req, int n_heads, int k);
hipError_t launch_mla_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

// ---- prefill ---------------------------------------------------------------
struct PrefillScanArgs {
  const uint8_t* keys = nullptr;   // [n_tok][128] fp8 codes of this block
  const float* kscale = nullptr;   // [n_tok]
  int tok0 = 0;                    // position of the block's first token
  int n_tok = 0;
  const void* q = nullptr;         // [T][64][128] bf16
  const float* w = nullptr;        // [T][64]
  int T = 0;
  int hist_len = 0;                // query i sits at hist_len + i
  float* scores = nullptr;         // optional [T][ld]: every visible score as well
  int64_t ld = 0;
  // the running selection: per query a candidate buffer [T][cap] of (score
  // key, position) and a state [T][2] (count, entry threshold key; zero
  // before the first block); the last block writes idx [T][k] and count [T]
  uint2* cand = nullptr;
  uint32_t* state = nullptr;
  int cap = 0;
  int k = 0;
  int final_block = 0;
  int32_t* idx = nullptr;
  int32_t* count = nullptr;
};
// candidate capacity per query for a selection of k (>= 2k + 8 tiles of 64)
inline int prefill_cand_cap(int k) { return (int)(((int64_t)2 * k + 512 + 63) / 64 * 64); }
hipError_t launch_prefill_scan(const PrefillScanArgs& a, hipStream_t s);

}  // namespace lsi

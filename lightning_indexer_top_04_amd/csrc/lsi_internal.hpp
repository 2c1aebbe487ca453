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
};

hipError_t launch_scan_fp8(const ScanArgs& a, hipStream_t s);
hipError_t launch_scan_int4(const ScanArgs& a, hipStream_t s);
hipError_t launch_scan_f32(const ScanArgs& a, hipStream_t s);

// ---- top-k ----------------------------------------------------------------
struct TopkArgs {
  const float* scores = nullptr;   // [num_req][ld]
  int64_t ld = 0;
  const int32_t* seq_lens = nullptr;  // per-row length (clamped to max_len)
  int lens_const = -1;             // if >= 0: every row has this length
  int causal_base = -1;            // if >= 0: row r has length causal_base+r+1
  const uint32_t* range = nullptr; // optional [R][2]: ~(min key), max key of row r
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
};
size_t topk_ws_bytes(int num_req, int max_len);
// words of the workspace that must be zero when the top-k starts
int64_t topk_zero_words(int num_req);
// ws_state: 0 = counters not cleared (clear them first), 1 = already cleared
hipError_t launch_topk(const TopkArgs& a, int ws_state, hipStream_t s);
hipError_t launch_zero(uint32_t* p, int64_t words, hipStream_t s);

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
};
size_t mla_ws_bytes(int num_req, int n_heads, int dv, int k);
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
  float* scores = nullptr;         // [T][ld]
  int64_t ld = 0;
  // optional [T][2]: per query row, atomic maxima of ~key and key over the
  // scores written (zero before the first block), i.e. the row's key range
  uint32_t* range = nullptr;
};
hipError_t launch_prefill_scan(const PrefillScanArgs& a, hipStream_t s);

}  // namespace lsi

/*
 * lsi.h - C ABI of the MI355X (gfx950) lightning-indexer sparse-attention
 * decode library (liblsi.so).
 *
 * What is computed (sources: "Multi-layer Indexer" abstract on
 * zhuanzhiai.com, first paragraph - in DeepSeek Sparse Attention a lightning
 * indexer scores the whole cache of a layer and keeps the k=2048 best tokens,
 * which the layer then attends; "LeanSparse: Shrinking GPU Memory for
 * Sparse-Attention LLM Serving" episode notes on radioguide.fm - indexer keys
 * stay on the GPU, decode can search compact keys and rank a short list of
 * originals exactly, prefill streams history through two alternating GPU
 * buffers):
 *
 *   indexer score   I_s = sigma_s * sum_j w_j * max(0, q_j . k_s)
 *                   (k_s the decoded key code, sigma_s its per-token scale;
 *                   because sigma_s > 0 and ReLU is positively homogeneous
 *                   this equals sum_j w_j * ReLU(q_j . (sigma_s k_s)))
 *   selection       the k highest scores of each request (all tokens when
 *                   fewer than k exist)
 *   attention       softmax(sm_scale * q_h . K_sel) V_sel for every query head
 *                   h, with one key/value head shared by all query heads
 *                   (MLA: K is the whole latent row, V its first dv entries)
 *
 * Conventions for every call
 *   - All pointers are DEVICE pointers unless marked (host).  The caller owns
 *     every buffer; the library never allocates device memory.  Scratch comes
 *     in as `workspace` (256-byte aligned) of at least the size the matching
 *     *_workspace_bytes() function returns; its contents on entry do not
 *     matter and on return are unspecified, except for the leading state
 *     words of lsi_decode_step, lsi_multilayer_decode and (one request)
 *     lsi_two_stage_topk, whose rules are given with those calls.
 *   - Work is enqueued on the caller's stream; no call synchronises the host.
 *     Arguments are validated on the host BEFORE anything is enqueued:
 *     LSI_ERR_INVALID_ARG, LSI_ERR_UNSUPPORTED and LSI_ERR_WORKSPACE mean
 *     nothing was enqueued.  LSI_ERR_HIP (a launch or runtime call failed)
 *     can come after some of a call's kernels or copies were already
 *     enqueued: the call's outputs (and the workspace state words of the
 *     calls that keep them) are then undefined.  lsi_last_error_detail() gives a
 *     per-thread message.
 *   - Paged caches: token s of request b lives in physical page
 *     page_table[b][s / page_size], slot s % page_size.  Indexer keys and
 *     attention KV use the same page table and page size.  A page id outside
 *     [0, num_pages) is never dereferenced: its tokens score -inf and are
 *     never attended.  seq_lens[b] is clamped on the device to
 *     [0, max_seq_len].
 *   - Token indices are logical positions in [0, seq_len).  Index lists are
 *     [num_req][k] int32, padded with -1 after `count` valid entries; their
 *     order is unspecified (set semantics).  Among tokens whose scores are
 *     exactly equal at the k-th place, the lower positions are kept.
 *   - Scores order as IEEE floats with -0 == +0; NaN scores order below -inf.
 *   - Not thread-safe per stream; calls on one stream may not overlap in
 *     their use of one workspace.
 */
#ifndef LSI_H
#define LSI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
enum {
  LSI_OK = 0,
  LSI_ERR_INVALID_ARG = 1,   /* null pointer, bad size, inconsistent shape   */
  LSI_ERR_UNSUPPORTED = 2,   /* valid but not implemented (dtype/head shape) */
  LSI_ERR_WORKSPACE = 3,     /* workspace missing, misaligned or too small   */
  LSI_ERR_HIP = 4            /* a HIP runtime call or launch failed          */
};

/* ---- element types ------------------------------------------------------ */
enum {
  LSI_F32 = 0,       /* IEEE binary32                                          */
  LSI_BF16 = 1,      /* bfloat16                                               */
  LSI_FP8_E4M3 = 2,  /* OCP FP8 E4M3FN (bias 7, max 448, 0x7F/0xFF NaN)       */
  LSI_INT4 = 3       /* two's-complement nibbles in [-7,7], two per byte,
                        element 2i in the low nibble of byte i                */
};

/* A paged per-token cache.
 *   data  [num_pages][page_size][row] with row = dim elements of `dtype`
 *         (dim/2 bytes for LSI_INT4), rows densely packed.
 *   scale [num_pages][page_size] float per-token scale; required for
 *         LSI_FP8_E4M3 and LSI_INT4, must be NULL for LSI_F32 / LSI_BF16. */
typedef struct {
  int32_t dtype;
  int32_t page_size;
  int32_t num_pages;
  int32_t dim;
  const void* data;
  const float* scale;
} lsi_paged_cache;

/* A ragged batch of requests sharing one physical page pool.
 *   num_req, max_pages, max_seq_len are host integers; max_seq_len bounds
 *   every seq_lens[b] and sizes grids and workspaces (it must not exceed
 *   max_pages * page_size).
 *   seq_lens   [num_req] int32 (device)
 *   page_table [num_req][max_pages] int32 (device); may be NULL for calls
 *              that do not read caches (lsi_topk). */
typedef struct {
  int32_t num_req;
  int32_t max_pages;
  int32_t max_seq_len;
  int32_t reserved;        /* must be 0 */
  const int32_t* seq_lens;
  const int32_t* page_table;
} lsi_batch;

/* ---- indexer scan --------------------------------------------------------
 * Scores every cached token of every request (MLI abstract: the indexer
 * scores the whole cache).
 *   ikeys   indexer-key cache: LSI_FP8_E4M3 with dim 128 and page_size a
 *           multiple of 32, or LSI_F32 (dim <= 256, any page_size).
 *   q       [num_req][n_heads][dim]; bf16 for fp8 keys, f32 for f32 keys.
 *           fp8 keys need n_heads == 64; f32 keys n_heads*dim <= 8192.
 *   w       [num_req][n_heads] float head weights (any sign).
 *   scores  [num_req][ld] float, ld >= max_seq_len; entries at positions
 *           >= seq_lens[b] are not written.
 * Accumulation is fp32 over exact products (fp8 -> bf16 is exact). */
int32_t lsi_index_scores(const lsi_paged_cache* ikeys, const lsi_batch* batch,
                         const void* q, int32_t n_heads, int32_t dim,
                         const float* w, float* scores, int64_t ld,
                         hipStream_t stream);

/* ---- top-k selection -----------------------------------------------------
 * For each request the k largest of scores[b][0 .. seq_lens[b]) (MLI
 * abstract: keep the k=2048 highest-scoring tokens).  Radix select, not a
 * sort.
 *   scores [num_req][ld] float; batch->page_table may be NULL.
 *   idx    [num_req][k] int32 positions, -1 padded; count [num_req] int32
 *          = min(k, seq_lens[b]).
 *   1 <= k <= 65536. */
size_t lsi_topk_workspace_bytes(int32_t num_req, int32_t max_seq_len,
                                int32_t k);
int32_t lsi_topk(const float* scores, int64_t ld, const lsi_batch* batch,
                 int32_t k, int32_t* idx, int32_t* count, void* workspace,
                 size_t ws_bytes, hipStream_t stream);

/* ---- sparse attention over the selection ---------------------------------
 * Attention of every query head over the selected tokens only (MLI abstract:
 * the layer attends the selection).
 *   kv   LSI_BF16 latent cache with dim == dk == 576, dv == 512,
 *        n_heads a multiple of 16 (V = first dv entries of each row, v must
 *        be NULL); or LSI_F32 key cache with dk <= 256 plus a separate LSI_F32
 *        value cache v with dim == dv <= 256 (any n_heads <= 1024).
 *   q    [num_req][n_heads][dk], same dtype as kv.
 *   idx  [num_req][k] int32 positions; entries outside [0, seq_lens[b]) are
 *        skipped (so -1 padding is fine).
 *   out  [num_req][n_heads][dv], same dtype as kv (bf16 rounded from fp32).
 *   lse  [num_req][n_heads] float, natural log of the softmax normaliser of
 *        the scaled logits; -inf (and out = 0) when no entry is valid. */
size_t lsi_sparse_mla_workspace_bytes(int32_t num_req, int32_t n_heads,
                                      int32_t dv, int32_t k);
int32_t lsi_sparse_mla_decode(const lsi_paged_cache* kv,
                              const lsi_paged_cache* v,
                              const lsi_batch* batch, const void* q,
                              int32_t n_heads, int32_t dk, int32_t dv,
                              const int32_t* idx, int32_t k, float sm_scale,
                              void* out, float* lse, void* workspace,
                              size_t ws_bytes, hipStream_t stream);

/* ---- fused decode step ---------------------------------------------------
 * lsi_index_scores -> lsi_topk -> lsi_sparse_mla_decode for one layer, on
 * one stream, with the scores kept in the workspace.  Arguments have the
 * meanings given above; idx/count receive the selection.
 * Workspace state: unlike the other calls' scratch, the first
 * lsi_decode_step_state_bytes(num_req) bytes of this call's workspace carry
 * state from one call to the next.  They must be zero when a workspace is
 * first used (allocate it zero-filled, or clear it once); every call that
 * returns LSI_OK leaves them zero again, so a workspace can be reused call
 * after call with no clearing.  After a call that returned an error, or if
 * the buffer was used for anything else in between, clear them again.
 * (One-request steps build the top-k's histograms inside the scan, which
 * adds into these words; the attention kernel clears them afterwards.) */
size_t lsi_decode_step_state_bytes(int32_t num_req);
size_t lsi_decode_step_workspace_bytes(int32_t num_req, int32_t max_seq_len,
                                       int32_t k, int32_t n_heads,
                                       int32_t dv);
int32_t lsi_decode_step(const lsi_paged_cache* ikeys,
                        const lsi_paged_cache* kv, const lsi_paged_cache* v,
                        const lsi_batch* batch, const void* q_idx,
                        int32_t n_idx_heads, int32_t idx_dim, const float* w,
                        const void* q_attn, int32_t n_heads, int32_t dk,
                        int32_t dv, float sm_scale, int32_t k, int32_t* idx,
                        int32_t* count, void* out, float* lse,
                        void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- fused decode step without allocation ---------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc.  Computes
 * exactly what lsi_decode_step computes, with the same arguments except the
 * workspace: its scratch is a library-owned device array of
 * LSI_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, allocated with the library's
 * code on that GPU and held until the process ends.  The call allocates and
 * frees nothing.  A call that needs more scratch than that
 * (lsi_decode_step_workspace_bytes() above the limit) returns
 * LSI_ERR_WORKSPACE before anything is enqueued.  The array starts zeroed,
 * which is the state lsi_decode_step's workspace needs, and every successful
 * call leaves its state words zero again.  Every call on one GPU uses
 * the same array: calls that overlap on one GPU (on different streams, or
 * from different threads without ordering) race and give undefined results;
 * calls ordered on one stream are safe. */
#define LSI_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int32_t lsi_decode_step_noalloc(const lsi_paged_cache* ikeys,
                                const lsi_paged_cache* kv,
                                const lsi_paged_cache* v,
                                const lsi_batch* batch, const void* q_idx,
                                int32_t n_idx_heads, int32_t idx_dim,
                                const float* w, const void* q_attn,
                                int32_t n_heads, int32_t dk, int32_t dv,
                                float sm_scale, int32_t k, int32_t* idx,
                                int32_t* count, void* out, float* lse,
                                hipStream_t stream);

/* ---- several layers of one decode step ------------------------------------
 * MLI abstract: neighbouring layers select nearly the same tokens, so a layer
 * may attend the selection of the previous indexer layer instead of its own;
 * the indexer of a layer then no longer has to finish before that layer's
 * attention and runs beside it.  The same paragraph describes IndexCache,
 * which keeps an indexer in only a fraction 1/retention of the layers; the
 * others reuse the latest selection.
 *
 * Layer l (0 <= l < n_layers) has its own caches and queries; all layers
 * share `batch` (one page table, as the caches of one model's layers do).
 * Layer l has an indexer when l % retention == 0; its selection goes to
 * slot l / retention.  The selection layer l attends:
 *   LSI_SCHED_SERIAL  that of the latest indexer layer j <= l (its own when
 *                     it has an indexer): with retention 1 this is
 *                     lsi_decode_step once per layer.
 *   LSI_SCHED_MLI     that of the latest indexer layer j < l; layer 0 has
 *                     none before it and attends its own.
 * Arguments (per-layer arrays are HOST arrays of n_layers entries, or of
 * n_slots = ceil(n_layers / retention) entries for idx and count):
 *   ikeys[l]            LSI_FP8_E4M3 or LSI_F32 indexer cache (read for
 *                       indexer layers only; the other entries are ignored)
 *   kv[l]               LSI_BF16 latent cache, dk 576, dv 512; every layer's
 *                       with the page size and page count of layer 0's
 *   q_idx[l], w[l]      as for lsi_index_scores (indexer layers only)
 *   q_attn[l], out[l], lse[l]   as for lsi_sparse_mla_decode
 *   idx[slot] [num_req][k], count[slot] [num_req]: the selections
 * Streams: LSI_SCHED_SERIAL enqueues everything on `stream`.  LSI_SCHED_MLI
 * with a distinct s_index enqueues the indexer (scan and top-k) of layer l on
 * s_index after layer l-1's attention (a model's indexer query comes from
 * the previous layer's output) and the attention of layer l on `stream`; a
 * layer's attention waits only for the selection it reads.  `stream`
 * carries the final dependency.  With s_index NULL or equal to `stream`
 * LSI_SCHED_MLI runs the same work in order on `stream`.  Calls on one
 * device are serialised by a lock while they enqueue (they share two
 * events).  1 <= retention <= n_layers <= 4096.
 * Each indexer layer runs the launches of lsi_decode_step (the scan builds
 * the top-k's histograms, the attention resolves the threshold bin), with
 * two sets of that state alternating between selection slots.  Workspace
 * state: its first 2 * lsi_decode_step_state_bytes(num_req) bytes must be
 * zero the first time it is used; every successful call leaves them zero. */
enum { LSI_SCHED_SERIAL = 0, LSI_SCHED_MLI = 1 };
size_t lsi_multilayer_workspace_bytes(int32_t num_req, int32_t max_seq_len,
                                      int32_t k, int32_t n_heads, int32_t dv);
int32_t lsi_multilayer_decode(int32_t n_layers, int32_t retention,
                              int32_t schedule, const lsi_paged_cache* ikeys,
                              const lsi_paged_cache* kv,
                              const lsi_batch* batch,
                              const void* const* q_idx, int32_t n_idx_heads,
                              int32_t idx_dim, const float* const* w,
                              const void* const* q_attn, int32_t n_heads,
                              int32_t dk, int32_t dv, float sm_scale,
                              int32_t k, int32_t* const* idx,
                              int32_t* const* count, void* const* out,
                              float* const* lse, void* workspace,
                              size_t ws_bytes, hipStream_t stream,
                              hipStream_t s_index);

/* ---- two-stage compact-key search ----------------------------------------
 * LeanSparse episode notes: decode searches compact indexer keys, then ranks
 * a short list of the original keys exactly.  Stage 1 scores every token with
 * the int4 keys (ikeys4: LSI_INT4, dim 128) and keeps the n_cand best; stage 2
 * re-scores only those with the fp8 keys (ikeys8: LSI_FP8_E4M3, dim 128) and
 * keeps the k best.  Both caches use batch's page table.
 *   q [num_req][64][128] bf16, w [num_req][64] float.
 *   idx [num_req][k], count [num_req] as for lsi_topk.
 *   cand (optional, may be NULL) [num_req][n_cand] receives the stage-1
 *   candidates (-1 padded).  k <= n_cand <= 65536.
 * ikeys8->data and ->scale may be pinned host memory (hipHostMalloc) instead
 * of device memory (LeanSparse: only the compact keys need to stay in GPU
 * memory, the short list of originals is fetched from the host): stage 2
 * then reads the candidates' rows across the host bus.  Pageable host
 * memory returns LSI_ERR_INVALID_ARG.
 * Workspace state (num_req == 1 only): the first
 * lsi_decode_step_state_bytes(1) bytes carry state from one call to the
 * next, with the rules of lsi_decode_step's: zero when a workspace is first
 * used, left zero by every call that returns LSI_OK.  (The compact scan
 * builds the first top-k's histograms there; the exact scan clears them.)
 * With num_req > 1 the workspace holds no state. */
size_t lsi_two_stage_workspace_bytes(int32_t num_req, int32_t max_seq_len,
                                     int32_t n_cand, int32_t k);
int32_t lsi_two_stage_topk(const lsi_paged_cache* ikeys4,
                           const lsi_paged_cache* ikeys8,
                           const lsi_batch* batch, const void* q,
                           int32_t n_heads, int32_t dim, const float* w,
                           int32_t n_cand, int32_t k, int32_t* idx,
                           int32_t* count, int32_t* cand, void* workspace,
                           size_t ws_bytes, hipStream_t stream);

/* ---- prefill indexer chunk -----------------------------------------------
 * T new queries at positions hist_len .. hist_len+T-1; query i scores the
 * positions 0 .. hist_len+i (causal, itself included) and keeps the k best.
 * The history (LeanSparse notes: streamed through two alternating GPU
 * buffers) is copied block by block, block_tokens at a time, on s_copy into
 * two workspace buffers while s_compute scores the previous block.
 *   hist_keys  [hist_len][dim] uint8 fp8 codes, hist_scale [hist_len] float:
 *              pinned host memory (or device memory).
 *   chunk_keys [T][dim] uint8, chunk_scale [T] float: device.
 *   q [T][n_heads][dim] bf16 (n_heads 64, dim 128), w [T][n_heads] float.
 *   idx [T][k] int32 positions (the k best in ascending position order,
 *   then -1 padding), count [T] int32 = min(k, hist_len + i + 1).
 *   scores (optional, may be NULL) [T][hist_len+T] float receives the scores
 *   of visible positions (a debugging aid: the selection never needs them).
 * Ranking: score descending, equal scores by position ascending.  No score
 * matrix is kept: each query holds a running candidate buffer of
 * 2k + 512 (rounded up to 64) entries of 8 bytes, pruned to about its k
 * best whenever it could fill up, so the workspace is O(T k) plus the two
 * copy buffers; scores_external no longer changes the size.
 * s_copy may equal s_compute (then nothing overlaps).  The call returns once
 * everything is enqueued; s_compute carries the final dependency. */
size_t lsi_prefill_workspace_bytes(int32_t hist_len, int32_t T, int32_t dim,
                                   int32_t block_tokens, int32_t k,
                                   int32_t scores_external);
int32_t lsi_prefill_index_topk(const uint8_t* hist_keys,
                               const float* hist_scale, int32_t hist_len,
                               const uint8_t* chunk_keys,
                               const float* chunk_scale, int32_t T,
                               const void* q, int32_t n_heads, int32_t dim,
                               const float* w, int32_t k,
                               int32_t block_tokens, int32_t* idx,
                               int32_t* count, float* scores, void* workspace,
                               size_t ws_bytes, hipStream_t s_compute,
                               hipStream_t s_copy);

/* ---- workspace sizes through one call -------------------------------------
 * The same figures as the *_workspace_bytes functions above, selected by op.
 * Fields that an op does not use are ignored.  For LSI_OP_PREFILL, num_req
 * is T (the chunk's queries) and max_seq_len is hist_len.  Returns 0 for an
 * unknown op or invalid sizes. */
enum {
  LSI_OP_TOPK = 1, LSI_OP_SPARSE_MLA = 2, LSI_OP_DECODE_STEP = 3,
  LSI_OP_MULTILAYER = 4, LSI_OP_TWO_STAGE = 5, LSI_OP_PREFILL = 6
};
typedef struct {
  int32_t num_req, max_seq_len, k, n_heads, dv;  /* decode-side calls          */
  int32_t n_cand;                                /* LSI_OP_TWO_STAGE           */
  int32_t dim, block_tokens, scores_external;    /* LSI_OP_PREFILL             */
} lsi_ws_query;
size_t lsi_workspace_bytes(int32_t op, const lsi_ws_query* q);

/* ---- kernel timing ---------------------------------------------------------
 * Profiling aid for the calling host thread.  With events != NULL, every
 * kernel that later calls from this thread launch takes the next two caller
 * events (created with timing enabled) as its start and stop events, given
 * to the dispatch itself (hipExtLaunchKernel), and names[i] (host array of
 * capacity / 2 entries, may be NULL) receives a static string naming the
 * kernel of pair i = (events[2i], events[2i+1]), until `capacity` events are
 * used.  The elapsed time of a pair is that kernel's duration; nothing extra
 * is enqueued.  lsi_profile_events(NULL, NULL, 0) stops.  Returns the number
 * of events used since the previous call. */
int32_t lsi_profile_events(hipEvent_t* events, const char** names,
                           int32_t capacity);

/* ---- diagnostics ---------------------------------------------------------*/
const char* lsi_status_string(int32_t status);   /* static string          */
const char* lsi_last_error_detail(void);         /* per-thread detail of the
                                                    last failure            */
const char* lsi_last_error(void);                /* the same string         */
int32_t lsi_version(void);                       /* major*10000+minor*100+patch */

#ifdef __cplusplus
}
#endif
#endif /* LSI_H */

// Top-k selection per row: the k largest scores (the "Multi-layer Indexer"
// abstract: keep the k=2048 highest-scoring tokens of the whole cache).
//
// Radix select over the order-preserving 32-bit key of each score, never a
// sort.  Three launches, handing over only at kernel boundaries (on this
// GPU an agent-scope fence in hundreds of workgroups costs tens of
// microseconds, so no workgroup waits for or signals another one):
//   1. topk_hist: each workgroup builds an LDS histogram of the top 12 key
//      bits of its slice and adds the non-empty bins to the row's global
//      histogram (a few dozen atomics per hot bin).
//   2. topk_select: each workgroup reads the row histogram, finds the bin
//      that holds the k-th largest key, writes the keys above it straight to
//      the output and collects the bin's members; slots come from a block
//      scan and one atomic per workgroup and counter.
//   3. topk_refine: one workgroup per row refines the candidates in LDS:
//      12 more key bits, the last 8 key bits, then positions (ascending) for
//      exact ties; each stage is a 4096-bin LDS histogram and an ordered
//      in-place compaction.  It also writes the padding and the count.
#include "lsi_internal.hpp"
#include "topk_common.hpp"

namespace lsi {
namespace {

using namespace topk;

constexpr int kBlock = 512;
constexpr int kPer = 8;                  // elements per thread in topk_select
constexpr int kSelChunk = kBlock * kPer;  // 4096
constexpr int kLdsCand = 4096;           // candidates refined in LDS

__device__ __forceinline__ int row_len(const TopkArgs& a, int r) {
  int L;
  if (a.lens_const >= 0) L = a.lens_const;
  else if (a.causal_base >= 0) L = a.causal_base + r + 1;
  else L = a.seq_lens[r];
  return min(max(L, 0), a.max_len);
}

__device__ __forceinline__ int out_value(const TopkArgs& a, int r, int slot) {
  return a.map ? a.map[(int64_t)r * a.map_ld + slot] : slot;
}

// Write kept position `pos` at output slot `o` of row r (and its physical
// cache row when requested).
__device__ __forceinline__ void emit(const TopkArgs& a, int r, int o, int pos) {
  a.idx[(int64_t)r * a.k + o] = pos;
  if (a.phys) {
    int row = -1;
    if (pos >= 0) {
      const int page = a.page_table[(int64_t)r * a.max_pages + pos / a.page_size];
      if ((unsigned)page < (unsigned)a.num_pages) row = page * a.page_size + pos % a.page_size;
    }
    a.phys[(int64_t)r * a.k + o] = row;
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void zero_kernel(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

__global__ __launch_bounds__(kBlock) void topk_hist_kernel(TopkArgs a, int chunk) {
  __shared__ uint32_t hist[kBins];
  const int r = blockIdx.y;
  const int L = row_len(a, r);
  if (L <= a.k) return;
  const int begin = blockIdx.x * chunk;
  if (begin >= L) return;
  const int end = min(begin + chunk, L);
  for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = 0u;
  __syncthreads();
  const float* row = a.scores + (int64_t)r * a.ld;
  for (int i = begin + threadIdx.x; i < end; i += kBlock)
    atomicAdd(&hist[float_key(row[i]) >> 20], 1u);
  __syncthreads();
  uint32_t* gh = carve(a.ws, a.num_req).hist + (size_t)r * kBins;
  for (int i = threadIdx.x; i < kBins; i += kBlock)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// The single-workgroup refinement of a row's candidate list.
__device__ void refine_row(const TopkArgs& a, int r, const Ws& ws, uint32_t* st, uint32_t* hist,
                           uint32_t* tmp, uint32_t* lkey, int32_t* lslot) {
  const float* row = a.scores + (int64_t)r * a.ld;
  int32_t* list = ws.cand + (size_t)r * a.max_len;
  uint32_t n = st[ST_CAND];
  uint32_t need = st[ST_NEED];
  uint32_t out_pos = st[ST_OUT];
  bool in_lds = false;
  // stages: key bits [19:8], key bits [7:0], then position bits
  // [31:20], [19:8], [7:0] ascending
  for (int stage = 0; stage < 5 && need > 0 && n > 0; ++stage) {
    if (n <= need) break;
    if (!in_lds && n <= (uint32_t)kLdsCand) {
      for (uint32_t i = threadIdx.x; i < n; i += kBlock) {
        const int slot = list[i];
        lslot[i] = slot;
        lkey[i] = float_key(row[slot]);
      }
      in_lds = true;
      __syncthreads();
    }
    const bool by_key = stage < 2;
    const int shift = stage == 0 ? 8 : stage == 1 ? 0 : stage == 2 ? 20 : stage == 3 ? 8 : 0;
    const uint32_t mask = (stage == 1 || stage == 4) ? 0xFFu : 0xFFFu;
    auto value = [&](uint32_t i, int& slot) -> uint32_t {
      slot = in_lds ? lslot[i] : list[i];
      if (!by_key) return (uint32_t)out_value(a, r, slot);
      return in_lds ? lkey[i] : float_key(row[slot]);
    };
    for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = 0u;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n; i += kBlock) {
      int slot;
      const uint32_t v = value(i, slot);
      atomicAdd(&hist[(v >> shift) & mask], 1u);
    }
    __syncthreads();
    uint32_t better;
    const int bin = find_threshold<kBlock>(hist, need, by_key, tmp, &better);
    // ordered pass: winners (better than bin) go out, equal ones stay
    uint32_t keep = 0;
    for (uint32_t base = 0; base < n; base += kBlock) {
      const uint32_t i = base + threadIdx.x;
      int slot = -1;
      uint32_t v = 0, flag_win = 0, flag_eq = 0;
      if (i < n) {
        v = value(i, slot);
        const int d = (int)((v >> shift) & mask);
        flag_eq = d == bin;
        flag_win = by_key ? (d > bin) : (d < bin);
      }
      uint32_t tot;
      const uint32_t pre = block_excl_scan<kBlock>(flag_win | (flag_eq << 16), tmp, &tot);
      if (flag_win && out_pos + (pre & 0xFFFF) < (uint32_t)a.k)
        emit(a, r, out_pos + (pre & 0xFFFF), out_value(a, r, slot));
      if (flag_eq) {
        const uint32_t j = keep + (pre >> 16);
        if (in_lds) {
          lslot[j] = slot;
          if (by_key) lkey[j] = v;
        } else {
          list[j] = slot;
        }
      }
      out_pos += tot & 0xFFFF;
      keep += tot >> 16;
      __syncthreads();
    }
    need -= better;
    n = keep;
  }
  // whatever remains is taken whole (n <= need here)
  const uint32_t take = min(n, need);
  for (uint32_t i = threadIdx.x; i < take && out_pos + i < (uint32_t)a.k; i += kBlock)
    emit(a, r, out_pos + i, out_value(a, r, in_lds ? lslot[i] : list[i]));
  out_pos += take;
  __syncthreads();
  for (int i = (int)out_pos + threadIdx.x; i < a.k; i += kBlock) emit(a, r, i, -1);
  if (threadIdx.x == 0) a.count[r] = (int32_t)min(out_pos, (uint32_t)a.k);
}

__global__ __launch_bounds__(kBlock) void topk_select_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t tmp[32];
  __shared__ uint32_t bases[2];
  const int r = blockIdx.y;
  const int L = row_len(a, r);
  const int begin = blockIdx.x * kSelChunk;
  if (begin >= max(L, 1)) return;
  const int end = min(begin + kSelChunk, L);
  if (L <= a.k) {
    // every element is kept; workgroup 0 also pads and counts
    for (int i = begin + threadIdx.x; i < end; i += kBlock) emit(a, r, i, out_value(a, r, i));
    if (blockIdx.x == 0) {
      for (int i = L + threadIdx.x; i < a.k; i += kBlock) emit(a, r, i, -1);
      if (threadIdx.x == 0) a.count[r] = L;
    }
    return;
  }
  const Ws ws = carve(a.ws, a.num_req);
  uint32_t* st = ws.state + (size_t)r * kState;
  const uint32_t* gh = ws.hist + (size_t)r * kBins;
  for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = gh[i];
  __syncthreads();
  uint32_t better;
  const uint32_t digit = (uint32_t)find_threshold<kBlock>(hist, (uint32_t)a.k, true, tmp, &better);
  if (blockIdx.x == 0 && threadIdx.x == 0) st[ST_NEED] = (uint32_t)a.k - better;
  const float* row = a.scores + (int64_t)r * a.ld;
  int32_t* list = ws.cand + (size_t)r * a.max_len;
  // thread t owns elements begin + t*kPer .. +kPer (contiguous, 32 bytes)
  const int i0 = begin + threadIdx.x * kPer;
  uint32_t win = 0, eq = 0;      // bit masks over the kPer elements
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = i0 + j;
    if (i < end) {
      const uint32_t d = float_key(row[i]) >> 20;
      win |= (uint32_t)(d > digit) << j;
      eq |= (uint32_t)(d == digit) << j;
    }
  }
  uint32_t tot;
  const uint32_t pre = block_excl_scan<kBlock>(__popc(win) | (__popc(eq) << 16), tmp, &tot);
  if (threadIdx.x == 0) {
    bases[0] = (tot & 0xFFFF) ? atomicAdd(&st[ST_OUT], tot & 0xFFFF) : 0u;
    bases[1] = (tot >> 16) ? atomicAdd(&st[ST_CAND], tot >> 16) : 0u;
  }
  __syncthreads();
  uint32_t ow = bases[0] + (pre & 0xFFFF);
  uint32_t oc = bases[1] + (pre >> 16);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if ((win >> j) & 1u) {
      if (ow < (uint32_t)a.k) emit(a, r, ow, out_value(a, r, i0 + j));
      ++ow;
    }
    if ((eq >> j) & 1u) {
      if (oc < (uint32_t)a.max_len) list[oc] = i0 + j;
      ++oc;
    }
  }
}

__global__ __launch_bounds__(kBlock) void topk_refine_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t lkey[kLdsCand];
  __shared__ int32_t lslot[kLdsCand];
  __shared__ uint32_t tmp[32];
  const int r = blockIdx.x;
  const int L = row_len(a, r);
  if (L <= a.k) return;
  const Ws ws = carve(a.ws, a.num_req);
  refine_row(a, r, ws, ws.state + (size_t)r * kState, hist, tmp, lkey, lslot);
}

// a few dozen workgroups per row at most, so a hot bin sees few atomics
int pick_hist_chunk(int64_t rows, int64_t max_len) {
  const int64_t target = (int64_t)num_cus() * 4;
  int64_t c = ceil_div(rows * max_len, target);
  c = std::max<int64_t>(c, ceil_div(max_len, 32));
  c = ceil_div(c, kBlock) * kBlock;
  if (c < 4096) c = 4096;
  if (c > 65536) c = 65536;
  return (int)c;
}

}  // namespace

size_t topk_ws_bytes(int num_req, int max_len) {
  return align_up(((size_t)num_req * (kBins + kState) + (size_t)num_req * max_len) * 4, 256);
}

int64_t topk_zero_words(int num_req) { return (int64_t)num_req * (kBins + kState); }

hipError_t launch_zero(uint32_t* p, int64_t n, hipStream_t s) {
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(n, kBlock * 4), 1024));
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(kBlock), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, int ws_state, hipStream_t s) {
  if (ws_state == 0) launch_zero(static_cast<uint32_t*>(a.ws), topk_zero_words(a.num_req), s);
  const int chunk = pick_hist_chunk(a.num_req, a.max_len);
  dim3 hgrid((unsigned)std::max<int64_t>(1, ceil_div(a.max_len, chunk)), (unsigned)a.num_req);
  hipLaunchKernelGGL(topk_hist_kernel, hgrid, dim3(kBlock), 0, s, a, chunk);
  dim3 sgrid((unsigned)std::max<int64_t>(1, ceil_div(a.max_len, kSelChunk)), (unsigned)a.num_req);
  hipLaunchKernelGGL(topk_select_kernel, sgrid, dim3(kBlock), 0, s, a);
  hipLaunchKernelGGL(topk_refine_kernel, dim3(a.num_req), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace lsi

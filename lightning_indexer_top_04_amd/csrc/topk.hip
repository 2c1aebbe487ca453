// Top-k selection per row: the k largest scores (the "Multi-layer Indexer"
// abstract: keep the k=2048 highest-scoring tokens of the whole cache).
//
// Radix select over the order-preserving 32-bit key of each score, never a
// sort.  Two launches over the data:
//   1. topk_hist: every workgroup builds an LDS histogram of the top 12 key
//      bits of its slice and adds the non-empty bins to the row's global
//      histogram.  The last workgroup of a row (arrival counter) finds the
//      bin that holds the k-th largest key.
//   2. topk_select: every workgroup appends keys above that bin straight to
//      the output and keys inside it to a candidate list (wave ballot +
//      popcount, one atomic per wave).  The last workgroup of the row refines
//      the candidates alone: 12 more key bits, the last 8 key bits, then the
//      position (ascending) for exact ties, each a 4096-bin LDS histogram and
//      an in-place ordered compaction.
#include "lsi_internal.hpp"

namespace lsi {
namespace {

constexpr int kBins = 4096;
constexpr int kBlock = 512;
constexpr int kState = 16;

// state words per row
enum {
  ST_HIST_DONE = 0,
  ST_SEL_DONE = 1,
  ST_DIGIT = 2,
  ST_NEED = 3,
  ST_OUT = 4,
  ST_CAND = 5,
  ST_MODE = 6,   // 0: select, 1: keep every element
  ST_K = 7
};

struct TopkWs {
  uint32_t* hist;    // [R][kBins]
  uint32_t* state;   // [R][kState]
  int32_t* cand;     // [R][max_len]
};

__host__ __device__ inline TopkWs carve(void* ws, int R) {
  TopkWs w;
  w.hist = static_cast<uint32_t*>(ws);
  w.state = w.hist + (size_t)R * kBins;
  w.cand = reinterpret_cast<int32_t*>(w.state + (size_t)R * kState);
  return w;
}

__device__ __forceinline__ int row_len(const TopkArgs& a, int r) {
  int L;
  if (a.lens_const >= 0) L = a.lens_const;
  else if (a.causal_base >= 0) L = a.causal_base + r + 1;
  else L = a.seq_lens[r];
  return min(max(L, 0), a.max_len);
}

__device__ __forceinline__ uint32_t atomic_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-wide exclusive scan of one uint32 per thread (kBlock threads).
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kBlock / 64; ++i) {
    const uint32_t t = tmp[i];
    if (i < wave) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Find, in priority order (descending bins when desc, else ascending), the
// bin at which the running count first reaches `need` (1 <= need <= total).
// Returns the bin and, in *better, the count of all bins before it.
__device__ int find_threshold(const uint32_t* cnt, uint32_t need, bool desc,
                              uint32_t* tmp, uint32_t* better) {
  constexpr int per = kBins / kBlock;   // 8
  const int t = threadIdx.x;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int q = t * per + i;
    local += cnt[desc ? kBins - 1 - q : q];
  }
  uint32_t tot;
  const uint32_t excl = block_excl_scan(local, tmp, &tot);
  if (excl < need && excl + local >= need) {
    uint32_t acc = excl;
    for (int i = 0; i < per; ++i) {
      const int q = t * per + i;
      const int bin = desc ? kBins - 1 - q : q;
      if (acc + cnt[bin] >= need) {
        tmp[16] = (uint32_t)bin;
        tmp[17] = acc;
        break;
      }
      acc += cnt[bin];
    }
  }
  __syncthreads();
  const int bin = (int)tmp[16];
  *better = tmp[17];
  __syncthreads();
  return bin;
}

// Wave-aggregated append: returns the slot of this lane (if flag) after one
// atomic per wave on *counter.  Every lane of the wave must call it.
__device__ __forceinline__ int wave_append(bool flag, uint32_t* counter) {
  const int lane = threadIdx.x & 63;
  const uint64_t mask = __ballot(flag);
  const int cnt = __popcll(mask);
  uint32_t base = 0;
  if (lane == 0 && cnt) base = atomicAdd(counter, (uint32_t)cnt);
  base = __shfl(base, 0);
  const int off = __popcll(mask & ((1ull << lane) - 1ull));
  return flag ? (int)base + off : -1;
}

__device__ __forceinline__ int out_value(const TopkArgs& a, int r, int slot) {
  return a.map ? a.map[(int64_t)r * a.map_ld + slot] : slot;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void topk_zero_kernel(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

__global__ __launch_bounds__(kBlock) void topk_hist_kernel(TopkArgs a, int chunk) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t tmp[32];
  __shared__ int is_last;
  const int r = blockIdx.y;
  const int L = row_len(a, r);
  const int nchunks = max(1, (L + chunk - 1) / chunk);
  if ((int)blockIdx.x >= nchunks) return;
  TopkWs ws = carve(a.ws, a.num_req);
  uint32_t* st = ws.state + (size_t)r * kState;
  if (L > a.k) {
    for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = 0u;
    __syncthreads();
    const int begin = blockIdx.x * chunk;
    const int end = min(begin + chunk, L);
    const float* row = a.scores + (int64_t)r * a.ld;
    for (int i = begin + threadIdx.x; i < end; i += kBlock)
      atomicAdd(&hist[float_key(row[i]) >> 20], 1u);
    __syncthreads();
    uint32_t* gh = ws.hist + (size_t)r * kBins;
    for (int i = threadIdx.x; i < kBins; i += kBlock)
      if (hist[i]) atomicAdd(&gh[i], hist[i]);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0)
    is_last = (atomicAdd(&st[ST_HIST_DONE], 1u) == (uint32_t)(nchunks - 1));
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  if (L <= a.k) {
    if (threadIdx.x == 0) {
      st[ST_MODE] = 1u;
      st[ST_K] = (uint32_t)L;
    }
    return;
  }
  const uint32_t* gh = ws.hist + (size_t)r * kBins;
  for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = atomic_load(gh + i);
  __syncthreads();
  uint32_t better;
  const int bin = find_threshold(hist, (uint32_t)a.k, true, tmp, &better);
  if (threadIdx.x == 0) {
    st[ST_MODE] = 0u;
    st[ST_DIGIT] = (uint32_t)bin;
    st[ST_NEED] = (uint32_t)a.k - better;
    st[ST_K] = (uint32_t)a.k;
  }
}

// The single-workgroup refinement of a row's candidate list.
__device__ void refine_row(const TopkArgs& a, int r, TopkWs ws, uint32_t* st,
                           uint32_t* hist, uint32_t* tmp) {
  const float* row = a.scores + (int64_t)r * a.ld;
  int32_t* list = ws.cand + (size_t)r * a.max_len;
  int32_t* out = a.idx + (int64_t)r * a.k;
  uint32_t n = atomic_load(st + ST_CAND);
  uint32_t need = atomic_load(st + ST_NEED);
  uint32_t out_pos = atomic_load(st + ST_OUT);
  // stages: key bits [19:8], key bits [7:0], then position bits
  // [31:20], [19:8], [7:0] ascending
  for (int stage = 0; stage < 5 && need > 0 && n > 0; ++stage) {
    if (n <= need) break;
    const bool by_key = stage < 2;
    const int shift = stage == 0 ? 8 : stage == 1 ? 0 : stage == 2 ? 20 : stage == 3 ? 8 : 0;
    const uint32_t mask = (stage == 1 || stage == 4) ? 0xFFu : 0xFFFu;
    for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = 0u;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n; i += kBlock) {
      const int slot = list[i];
      const uint32_t v = by_key ? float_key(row[slot]) : (uint32_t)out_value(a, r, slot);
      atomicAdd(&hist[(v >> shift) & mask], 1u);
    }
    __syncthreads();
    uint32_t better;
    const int bin = find_threshold(hist, need, by_key, tmp, &better);
    // ordered pass: winners (better than bin) go out, equal ones stay
    uint32_t keep = 0;
    for (uint32_t base = 0; base < n; base += kBlock) {
      const uint32_t i = base + threadIdx.x;
      int slot = -1;
      uint32_t flag_win = 0, flag_eq = 0;
      if (i < n) {
        slot = list[i];
        const uint32_t v = by_key ? float_key(row[slot]) : (uint32_t)out_value(a, r, slot);
        const int d = (int)((v >> shift) & mask);
        flag_eq = d == bin;
        flag_win = by_key ? (d > bin) : (d < bin);
      }
      uint32_t tot;
      const uint32_t pre = block_excl_scan(flag_win | (flag_eq << 16), tmp, &tot);
      if (flag_win && out_pos + (pre & 0xFFFF) < (uint32_t)a.k)
        out[out_pos + (pre & 0xFFFF)] = out_value(a, r, slot);
      if (flag_eq) list[keep + (pre >> 16)] = slot;
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
    out[out_pos + i] = out_value(a, r, list[i]);
  out_pos += take;
  __syncthreads();
  for (int i = (int)out_pos + threadIdx.x; i < a.k; i += kBlock) out[i] = -1;
  if (threadIdx.x == 0) a.count[r] = (int32_t)min(out_pos, (uint32_t)a.k);
}

__global__ __launch_bounds__(kBlock) void topk_select_kernel(TopkArgs a, int chunk) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t tmp[32];
  __shared__ int is_last;
  const int r = blockIdx.y;
  const int L = row_len(a, r);
  const int nchunks = max(1, (L + chunk - 1) / chunk);
  if ((int)blockIdx.x >= nchunks) return;
  TopkWs ws = carve(a.ws, a.num_req);
  uint32_t* st = ws.state + (size_t)r * kState;
  const int mode = (int)st[ST_MODE];
  const int begin = blockIdx.x * chunk;
  const int end = min(begin + chunk, L);
  int32_t* out = a.idx + (int64_t)r * a.k;
  if (mode == 1) {
    for (int i = begin + threadIdx.x; i < end && i < a.k; i += kBlock) out[i] = out_value(a, r, i);
  } else {
    const uint32_t digit = st[ST_DIGIT];
    const float* row = a.scores + (int64_t)r * a.ld;
    int32_t* list = ws.cand + (size_t)r * a.max_len;
    for (int base = begin; base < end; base += kBlock) {
      const int i = base + threadIdx.x;
      uint32_t d = 0;
      if (i < end) d = float_key(row[i]) >> 20;
      const bool in = i < end;
      const int ws_ = wave_append(in && d > digit, st + ST_OUT);
      if (ws_ >= 0 && ws_ < a.k) out[ws_] = out_value(a, r, i);
      const int cs = wave_append(in && d == digit, st + ST_CAND);
      if (cs >= 0 && cs < a.max_len) list[cs] = i;
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0)
    is_last = (atomicAdd(&st[ST_SEL_DONE], 1u) == (uint32_t)(nchunks - 1));
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  if (mode == 1) {
    for (int i = L + threadIdx.x; i < a.k; i += kBlock) out[i] = -1;
    if (threadIdx.x == 0) a.count[r] = L;
    return;
  }
  refine_row(a, r, ws, st, hist, tmp);
}

int pick_chunk(int64_t rows, int64_t max_len) {
  const int64_t target = (int64_t)num_cus() * 4;
  int64_t c = ceil_div(rows * max_len, target);
  c = ceil_div(c, kBlock) * kBlock;
  if (c < 2048) c = 2048;
  if (c > 65536) c = 65536;
  return (int)c;
}

}  // namespace

size_t topk_ws_bytes(int num_req, int max_len) {
  return align_up(((size_t)num_req * (kBins + kState) + (size_t)num_req * max_len) * 4, 256);
}

int64_t topk_zero_words(int num_req) { return (int64_t)num_req * (kBins + kState); }

hipError_t launch_topk(const TopkArgs& a, bool ws_already_zero, hipStream_t s) {
  if (!ws_already_zero) {
    const int64_t n = topk_zero_words(a.num_req);
    const int blocks = (int)std::min<int64_t>(ceil_div(n, kBlock), 1024);
    hipLaunchKernelGGL(topk_zero_kernel, dim3(blocks), dim3(kBlock), 0, s,
                       static_cast<uint32_t*>(a.ws), n);
  }
  const int chunk = pick_chunk(a.num_req, a.max_len);
  dim3 grid((unsigned)std::max<int64_t>(1, ceil_div(a.max_len, chunk)), (unsigned)a.num_req);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kBlock), 0, s, a, chunk);
  hipLaunchKernelGGL(topk_select_kernel, grid, dim3(kBlock), 0, s, a, chunk);
  return hipGetLastError();
}

}  // namespace lsi

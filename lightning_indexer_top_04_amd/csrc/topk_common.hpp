// Device pieces of the radix top-k shared by the top-k kernels and the
// indexer scan (which builds the first-digit histogram of its own scores).
#pragma once

#include "lsi_common.hpp"

namespace lsi {
namespace topk {

constexpr int kBins = 4096;      // 12-bit digits
constexpr int kState = 16;       // state words per row

// state words per row
enum {
  ST_HIST_DONE = 0,   // arrivals of the histogram producers
  ST_SEL_DONE = 1,    // arrivals of the select workgroups
  ST_DIGIT = 2,       // top 12 key bits of the k-th largest key
  ST_NEED = 3,        // how many of that bin still need to be taken
  ST_OUT = 4,         // winners written so far
  ST_CAND = 5,        // candidates collected so far
  ST_MODE = 6,        // 0: select, 1: keep every element
  ST_K = 7
};

struct Ws {
  uint32_t* hist;    // [R][kBins]
  uint32_t* state;   // [R][kState]
  int32_t* cand;     // [R][max_len]
};

__host__ __device__ inline Ws carve(void* ws, int R) {
  Ws w;
  w.hist = static_cast<uint32_t*>(ws);
  w.state = w.hist + (size_t)R * kBins;
  w.cand = reinterpret_cast<int32_t*>(w.state + (size_t)R * kState);
  return w;
}

__device__ __forceinline__ uint32_t atomic_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-wide exclusive scan of one uint32 per thread (NT threads).
template <int NT>
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
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t t = tmp[i];
    if (i < wave) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// In priority order (descending bins when desc, else ascending), the bin at
// which the running count first reaches need (1 <= need <= total); *better
// receives the count of all bins before it.  tmp needs 32 words.
template <int NT>
__device__ int find_threshold(const uint32_t* cnt, uint32_t need, bool desc, uint32_t* tmp,
                              uint32_t* better) {
  constexpr int per = kBins / NT;
  const int t = threadIdx.x;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int q = t * per + i;
    local += cnt[desc ? kBins - 1 - q : q];
  }
  uint32_t tot;
  const uint32_t excl = block_excl_scan<NT>(local, tmp, &tot);
  if (excl < need && excl + local >= need) {
    uint32_t acc = excl;
    for (int i = 0; i < per; ++i) {
      const int q = t * per + i;
      const int bin = desc ? kBins - 1 - q : q;
      if (acc + cnt[bin] >= need) {
        tmp[24] = (uint32_t)bin;
        tmp[25] = acc;
        break;
      }
      acc += cnt[bin];
    }
  }
  __syncthreads();
  const int bin = (int)tmp[24];
  *better = tmp[25];
  __syncthreads();
  return bin;
}

// End of a histogram producer for row r: add the workgroup's LDS histogram
// `h` to the row's global histogram, count the arrival, and let the last of
// the row's `nprod` producers decide the first digit (or "keep all" when the
// row has at most k elements).  Every thread of the block must call it.
template <int NT>
__device__ void hist_flush_and_decide(const Ws& ws, int r, int L, int k, int nprod,
                                      uint32_t* h, uint32_t* tmp, int* flag) {
  __syncthreads();
  uint32_t* gh = ws.hist + (size_t)r * kBins;
  uint32_t* st = ws.state + (size_t)r * kState;
  if (L > k) {
    for (int i = threadIdx.x; i < kBins; i += NT)
      if (h[i]) atomicAdd(&gh[i], h[i]);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) *flag = (atomicAdd(&st[ST_HIST_DONE], 1u) == (uint32_t)(nprod - 1));
  __syncthreads();
  if (!*flag) return;
  __threadfence();
  if (L <= k) {
    if (threadIdx.x == 0) {
      st[ST_MODE] = 1u;
      st[ST_K] = (uint32_t)L;
    }
    return;
  }
  for (int i = threadIdx.x; i < kBins; i += NT) h[i] = atomic_load(gh + i);
  __syncthreads();
  uint32_t better;
  const int bin = find_threshold<NT>(h, (uint32_t)k, true, tmp, &better);
  if (threadIdx.x == 0) {
    st[ST_MODE] = 0u;
    st[ST_DIGIT] = (uint32_t)bin;
    st[ST_NEED] = (uint32_t)k - better;
    st[ST_K] = (uint32_t)k;
  }
}

}  // namespace topk
}  // namespace lsi

// Device pieces of the radix top-k shared by its kernels and by the kernels
// that prepare a top-k workspace.
#pragma once

#include "lsi_common.hpp"

namespace lsi {
namespace topk {

constexpr int kBins = 4096;      // 12-bit digits
constexpr int kState = 16;       // state words per row

// state words per row
enum {
  ST_NEED = 0,        // how many of the threshold bin still need to be taken
  ST_OUT = 1,         // winners written so far
  ST_CAND = 2,        // candidates collected so far
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

}  // namespace topk
}  // namespace lsi

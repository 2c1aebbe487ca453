// Device pieces of the radix top-k shared by its kernels and by the kernels
// that prepare a top-k workspace.
#pragma once

#include "lsi_common.hpp"

namespace lsi {
namespace topk {

constexpr int kBins = 4096;      // 12-bit digits
constexpr int kMinChunk = 1024;  // smallest chunk of positions per workgroup
constexpr int kMaxChunk = 8192;  // largest

// Per-row workspace of the multi-workgroup top-k.  Only hist and h2 must be
// zero when a call starts (they are adjacent); every other word is written
// before it is read.
struct Ws {
  uint32_t* hist;    // [R][kBins] histogram of the top 12 key bits
  uint32_t* h2;      // [R][kBins] threshold-bin members by key bits [19:8]
  uint16_t* suf;     // [R][nchunk][kBins] per chunk: elements with digit >= bin
  int2* cand;        // [R][max_len] threshold-bin members (slot, key), in chunk order
  int32_t* list;     // [R][max_len] their slots, compacted (when too many for LDS)
  uint32_t* rec;     // [R][4] threshold bin, count above it, count in it
  int nchunk;        // chunks per row at the smallest chunk size
};

__host__ __device__ inline int max_chunks(int max_len) { return (max_len + kMinChunk - 1) / kMinChunk; }

__host__ __device__ inline Ws carve(void* ws, int R, int max_len) {
  Ws w;
  w.nchunk = max_chunks(max_len);
  w.hist = static_cast<uint32_t*>(ws);
  w.h2 = w.hist + (size_t)R * kBins;
  w.suf = reinterpret_cast<uint16_t*>(w.h2 + (size_t)R * kBins);
  w.cand = reinterpret_cast<int2*>(w.suf + (size_t)R * w.nchunk * kBins);
  w.list = reinterpret_cast<int32_t*>(w.cand + (size_t)R * max_len);
  w.rec = reinterpret_cast<uint32_t*>(w.list + (size_t)R * max_len);
  return w;
}

// Workgroup barrier.  With lds_only it orders LDS traffic only: a plain
// __syncthreads also waits for this wave's global stores to complete, which
// in a loop that writes results as it goes costs a memory round trip per
// iteration.
__device__ __forceinline__ void wg_sync(bool lds_only) {
  if (lds_only) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else __syncthreads();
}

// Block-wide exclusive scan of one value per thread (NT threads); T is
// uint32_t or uint64_t (two 32-bit counts packed, each summed on its own as
// long as neither overflows).  tmp needs NT/64 values of T.
template <int NT, class T>
__device__ T block_excl_scan(T v, T* tmp, T* total, bool lds_only = false) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  T inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) tmp[wave] = inc;
  wg_sync(lds_only);
  T base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const T t = tmp[i];
    if (i < wave) base += t;
    tot += t;
  }
  wg_sync(lds_only);
  *total = tot;
  return base + inc - v;
}

// In priority order (descending bins when desc, else ascending), the bin at
// which the running count first reaches need (1 <= need <= total); *better
// receives the count of all bins before it.  tmp needs 32 words.
template <int NT>
__device__ int find_threshold(const uint32_t* cnt, uint32_t need, bool desc, uint32_t* tmp,
                              uint32_t* better, bool lds_only = false) {
  constexpr int per = kBins / NT;
  const int t = threadIdx.x;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int q = t * per + i;
    local += cnt[desc ? kBins - 1 - q : q];
  }
  uint32_t tot;
  const uint32_t excl = block_excl_scan<NT>(local, tmp, &tot, lds_only);
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
  wg_sync(lds_only);
  const int bin = (int)tmp[24];
  *better = tmp[25];
  wg_sync(lds_only);
  return bin;
}

}  // namespace topk
}  // namespace lsi

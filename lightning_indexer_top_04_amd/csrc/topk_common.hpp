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
  int32_t* crow;     // [R][max_len] physical row of each candidate (deferred selections only)
  uint32_t* rng;     // [R][2] the row's key range as reduced by the histogram launch
  int nchunk;        // chunks per row at the smallest chunk size
};

__host__ __device__ inline int max_chunks(int max_len) {
  return (int)(((int64_t)max_len + kMinChunk - 1) / kMinChunk);
}

__host__ __device__ inline Ws carve(void* ws, int R, int max_len) {
  Ws w;
  w.nchunk = max_chunks(max_len);
  w.hist = static_cast<uint32_t*>(ws);
  w.h2 = w.hist + (size_t)R * kBins;
  w.suf = reinterpret_cast<uint16_t*>(w.h2 + (size_t)R * kBins);
  w.cand = reinterpret_cast<int2*>(w.suf + (size_t)R * w.nchunk * kBins);
  w.list = reinterpret_cast<int32_t*>(w.cand + (size_t)R * max_len);
  w.rec = reinterpret_cast<uint32_t*>(w.list + (size_t)R * max_len);
  w.crow = reinterpret_cast<int32_t*>(w.rec + (size_t)R * 4);
  w.rng = reinterpret_cast<uint32_t*>(w.crow + (size_t)R * max_len);
  return w;
}

// The multi-workgroup top-k's digits of a row's keys: level 1 is
// (key - base) >> sh1 (12 bits), level 2 ((key - base) >> sh2) & 4095 over
// the level-1 bin's members, and the sh2 bits below it come last.  Without
// a recorded key range these are the top 12, the next 12 and the last 8 key
// bits.  With one ([~lowest key, highest key] of the row, written by the
// producer of the scores) the range fills the 4096 level-1 bins, so scores
// crowded into a few binades still spread over many bins and the threshold
// bin keeps few members.  Keys outside a recorded range (none, when the
// producer is right) are clamped into the end bins, never out of bounds.
struct Digits {
  uint32_t base = 0u;
  int sh1 = 20;
  int sh2 = 8;
  __device__ uint32_t d1(uint32_t key) const {
    return key < base ? 0u : min((key - base) >> sh1, (uint32_t)kBins - 1u);
  }
  __device__ uint32_t d2(uint32_t key) const { return ((key - base) >> sh2) & (uint32_t)(kBins - 1); }
};
__device__ inline Digits row_digits(const uint32_t* range, int r) {
  Digits g;
  if (range != nullptr) {
    const uint32_t lo = ~range[2 * (size_t)r];
    const uint32_t hi = range[2 * (size_t)r + 1];
    if (hi >= lo) {
      const uint32_t span = hi - lo;
      const int bits = span ? 32 - __clz((int)span) : 0;
      g.base = lo;
      g.sh1 = bits > 12 ? bits - 12 : 0;
      g.sh2 = g.sh1 > 12 ? g.sh1 - 12 : 0;
    }
  }
  return g;
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
  T inc;
  if constexpr (sizeof(T) == 4) {
    inc = (T)wave_incl_sum((uint32_t)v);
  } else {
    inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const T t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
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

// ---------------------------------------------------------------------------
// The threshold bin of a row whose selection was left unfinished (TopkArgs::
// defer): the row's `members` candidates sit in ws.cand (in chunk order), the
// second histogram (key bits [19:8] of the members) in ws.h2, and the record
// {threshold bin, count above it, members} in ws.rec.  The kept members are,
// in candidate-list order, those whose key bits [19:8] exceed the second
// threshold bin, then, inside that bin, those whose key bits [7:0] exceed the
// third, then, among exact ties, the lowest positions: the same set as the
// one-workgroup refinement keeps.  The i-th kept member takes output slot
// better + i.  Every workgroup that calls this computes the same thresholds
// and the same order; put(slot, position, physical row) is called for the
// slots in [lo, hi).  better and members are the record's (read by the
// caller with its other first loads).  NT threads; hist (kBins words) and tmp
// (32 words) are LDS.
// ---------------------------------------------------------------------------
template <int NT, class Put>
__device__ void resolve_members(const Ws& ws, int r, int max_len, int k, uint32_t better, uint32_t members,
                                uint32_t* hist, uint32_t* tmp, int lo, int hi, Put&& put) {
  constexpr int E = 8;                       // candidates per thread and batch
  constexpr int NB = 2;                      // batches held in registers
  constexpr int kHeld = NB * NT * E;         // candidates held (the rest streamed)
  constexpr int per = kBins / NT;            // level-2 bins per thread
  static_assert(per % 4 == 0 && kHeld < 65536, "register layout");
  const int tid = threadIdx.x;
  const int2* cand = ws.cand + (size_t)r * max_len;
  const int32_t* crow = ws.crow + (size_t)r * max_len;
  const uint32_t* g2 = ws.h2 + (size_t)r * kBins;
  const uint32_t need = (uint32_t)k - better;
  // one round trip: the first kHeld candidates with their rows (thread t
  // holds E consecutive ones per batch) and the second histogram (thread t
  // the per bins kBins - per (t + 1) .. kBins - per t - 1, which it takes in
  // descending order)
  int2 e[NB][E];
  int32_t rw[NB][E];
  uint4 hq[per / 4];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint32_t i0 = b * NT * E + tid * E;
    if (i0 + E <= (uint32_t)max_len && ((reinterpret_cast<uintptr_t>(cand) | reinterpret_cast<uintptr_t>(crow)) & 15) == 0) {
      // whole 16-byte loads (inside the row's lists, aligned), masked below
      const int4* c4 = reinterpret_cast<const int4*>(cand + i0);
      const int4* r4 = reinterpret_cast<const int4*>(crow + i0);
#pragma unroll
      for (int u = 0; u < E / 2; ++u) {
        const int4 x = c4[u];
        e[b][2 * u] = make_int2(x.x, x.y);
        e[b][2 * u + 1] = make_int2(x.z, x.w);
      }
#pragma unroll
      for (int u = 0; u < E / 4; ++u) {
        const int4 x = r4[u];
        rw[b][4 * u] = x.x;
        rw[b][4 * u + 1] = x.y;
        rw[b][4 * u + 2] = x.z;
        rw[b][4 * u + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < E; ++u) {
        const uint32_t i = i0 + u;
        e[b][u] = i < members ? cand[i] : make_int2(-1, 0);
        rw[b][u] = i < members ? crow[i] : -1;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < per / 4; ++j) hq[j] = reinterpret_cast<const uint4*>(g2 + kBins - per * (tid + 1))[j];
  __builtin_amdgcn_sched_barrier(0);
  uint32_t hv[per];    // hv[i]: count of bin kBins - 1 - (per t + i)
#pragma unroll
  for (int j = 0; j < per / 4; ++j) {
    hv[per - 1 - 4 * j] = hq[j].x;
    hv[per - 2 - 4 * j] = hq[j].y;
    hv[per - 3 - 4 * j] = hq[j].z;
    hv[per - 4 - 4 * j] = hq[j].w;
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int u = 0; u < E; ++u)
      if (b * NT * E + tid * E + u >= members) e[b][u] = make_int2(-1, 0);
  // f(pos, key) over every candidate: the held batches, then the rest
  auto pass = [&](auto&& f) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int u = 0; u < E; ++u)
        if (e[b][u].x >= 0) f(e[b][u].x, (uint32_t)e[b][u].y);
    for (uint32_t base = kHeld; base < members; base += NT * E) {
      int2 x[E];
#pragma unroll
      for (int u = 0; u < E; ++u) {
        const uint32_t i = base + tid * E + u;
        x[u] = i < members ? cand[i] : make_int2(-1, 0);
      }
#pragma unroll
      for (int u = 0; u < E; ++u)
        if (x[u].x >= 0) f(x[u].x, (uint32_t)x[u].y);
    }
  };
  // level 2: key bits [19:8], histogram built by the select; the threshold
  // bin (descending) from the per-thread sums, then in registers
  uint32_t bin2, better2, n2;
  {
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) local += hv[i];
    uint32_t tot;
    const uint32_t excl = block_excl_scan<NT>(local, tmp, &tot);
    // branch-free walk of the thread's bins: the first whose running count
    // reaches need
    uint32_t acc = excl;
    int fi = -1;
    uint32_t fb = 0, fn = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const bool hit = fi < 0 && acc + hv[i] >= need;
      fi = hit ? i : fi;
      fb = hit ? acc : fb;
      fn = hit ? hv[i] : fn;
      acc += hv[i];
    }
    if (excl < need && fi >= 0) {
      tmp[24] = (uint32_t)(kBins - 1 - (per * tid + fi));
      tmp[25] = fb;
      tmp[26] = fn;
    }
    __syncthreads();
    bin2 = tmp[24];
    better2 = tmp[25];
    n2 = tmp[26];
    __syncthreads();
  }
  const bool take2 = n2 <= need - better2;
  // level 3: key bits [7:0] of the members in bin2
  uint32_t bin3 = 0, take3 = 1, pos_t = 0;
  if (!take2) {
    const uint32_t need_b = need - better2;
    for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
    __syncthreads();
    pass([&](int, uint32_t key) {
      if (((key >> 8) & (kBins - 1)) == bin2) atomicAdd(&hist[key & 255u], 1u);
    });
    __syncthreads();
    uint32_t better3;
    bin3 = (uint32_t)find_threshold<NT>(hist, need_b, true, tmp, &better3);
    const uint32_t n3 = hist[bin3];
    take3 = n3 <= need_b - better3;
    if (!take3) {
      // exact ties (the same key): the need_c lowest positions, by a radix
      // select over position bits [30:20], [19:9], [8:0] (ascending)
      uint32_t need_c = need_b - better3;
      uint32_t prefix = 0;
      const int shifts[3] = {20, 9, 0};
      const int widths[3] = {11, 11, 9};
      for (int lv = 0; lv < 3; ++lv) {
        const int sh = shifts[lv];
        const uint32_t mask = (1u << widths[lv]) - 1u;
        __syncthreads();
        for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
        __syncthreads();
        pass([&](int pos, uint32_t key) {
          if (((key >> 8) & (kBins - 1)) == bin2 && (key & 255u) == bin3 &&
              (lv == 0 || ((uint32_t)pos >> (sh + widths[lv])) == prefix))
            atomicAdd(&hist[((uint32_t)pos >> sh) & mask], 1u);
        });
        __syncthreads();
        uint32_t below;
        const uint32_t bin = (uint32_t)find_threshold<NT>(hist, need_c, false, tmp, &below);
        prefix = (prefix << widths[lv]) | bin;
        need_c -= below;
      }
      pos_t = prefix;   // the need_c-th smallest tied position: keep positions <= pos_t
    }
  }
  // the ordered pass: kept members in list order, slots better + running index
  // (branch-free: a branchy test costs more than the loads it follows)
  auto kept = [&](int pos, uint32_t key) -> bool {
    const uint32_t d2 = (key >> 8) & (kBins - 1);
    const uint32_t d3 = key & 255u;
    const bool in3 = (d3 > bin3) | ((d3 == bin3) & ((take3 != 0u) | ((uint32_t)pos <= pos_t)));
    return (d2 > bin2) | ((d2 == bin2) & (take2 | in3));
  };
  // the held batches: one scan of both counts (16 bits each)
  uint32_t m[NB] = {0u, 0u};
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int u = 0; u < E; ++u)
      m[b] |= (uint32_t)((e[b][u].x >= 0) & kept(e[b][u].x, (uint32_t)e[b][u].y)) << u;
  uint32_t tot;
  const uint32_t ex = block_excl_scan<NT>((uint32_t)__popc(m[0]) | ((uint32_t)__popc(m[1]) << 16), tmp, &tot);
  const uint32_t tot0 = tot & 0xFFFFu;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    uint32_t o = better + (b == 0 ? (ex & 0xFFFFu) : tot0 + (ex >> 16));
#pragma unroll
    for (int u = 0; u < E; ++u) {
      if ((m[b] >> u) & 1u) {
        if (o >= (uint32_t)lo && o < (uint32_t)hi) put((int)o, e[b][u].x, rw[b][u]);
        ++o;
      }
    }
  }
  uint32_t run = tot0 + (tot >> 16);
  for (uint32_t base = kHeld; base < members && better + run < (uint32_t)hi; base += NT * E) {
    int2 x[E];
    int32_t xr[E];
    uint32_t mm = 0;
#pragma unroll
    for (int u = 0; u < E; ++u) {
      const uint32_t i = base + tid * E + u;
      x[u] = i < members ? cand[i] : make_int2(-1, 0);
      xr[u] = i < members ? crow[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < E; ++u)
      if (x[u].x >= 0 && kept(x[u].x, (uint32_t)x[u].y)) mm |= 1u << u;
    uint32_t t2;
    uint32_t o = run + block_excl_scan<NT>((uint32_t)__popc(mm), tmp, &t2) + better;
#pragma unroll
    for (int u = 0; u < E; ++u) {
      if ((mm >> u) & 1u) {
        if (o >= (uint32_t)lo && o < (uint32_t)hi) put((int)o, x[u].x, xr[u]);
        ++o;
      }
    }
    run += t2;
  }
}

}  // namespace topk
}  // namespace lsi

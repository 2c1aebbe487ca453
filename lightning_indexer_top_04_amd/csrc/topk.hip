// Top-k selection per row: the k largest scores (the "Multi-layer Indexer"
// abstract: keep the k=2048 highest-scoring tokens of the whole cache).
//
// Radix select over the order-preserving 32-bit key of each score, never a
// sort.  Long rows take three launches, handing over only at kernel
// boundaries (on this GPU an agent-scope fence in hundreds of workgroups
// costs tens of microseconds, so no workgroup waits for or signals another):
//   1. topk_hist: each workgroup builds an LDS histogram of the top 12 key
//      bits of its 4096-position chunk, stores the chunk's suffix counts
//      (elements at or above each bin) and adds the non-empty bins to the
//      row's global histogram.
//   2. topk_select: each workgroup reads the row histogram, finds the bin
//      that holds the k-th largest key, and learns from the earlier chunks'
//      suffix counts where its own winners (keys above that bin) and
//      candidates (keys in it) start; it writes its winners straight to the
//      output, with their physical rows, and its candidates (slot, key) to
//      the row's candidate list.  No atomics, nothing to wait for.
//   3. topk_refine: one workgroup per row finds the threshold bin again,
//      loads the candidates into LDS and refines them: 12 more key bits,
//      the last 8 key bits, then positions (ascending) for exact ties; each
//      stage is a 4096-bin LDS histogram and an ordered compaction.  It also
//      writes the padding and the count.
// Batches of rows (as many as compute units) and short rows take one launch
// of one workgroup per row instead (topk_row).
#include "lsi_internal.hpp"
#include "topk_common.hpp"

namespace lsi {
namespace {

using namespace topk;

constexpr int kBlock = 512;
constexpr int kLdsCand = 16384;          // candidates refined in LDS
constexpr int kBatch = 8;                // loads in flight per thread in a streaming pass
constexpr int kRefPer = 8;               // candidates per thread in a refinement pass
constexpr int kRefBatch = 4096;          // members per batch of the level-2 pass
constexpr int kRefThreads = 1024;        // threads of the one-workgroup refinement
constexpr int kSelPages = 520;           // page ids a select workgroup stages (8192 positions
                                         // over pages of 16 or more tokens)

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

// Page and in-page offset of position pos >= 0 (shifts for the usual
// power-of-two page sizes: a 32-bit division is dozens of instructions).
__device__ __forceinline__ void split_pos(int pos, int ps, int& page, int& off) {
  if ((ps & (ps - 1)) == 0) {
    page = pos >> (__ffs(ps) - 1);
    off = pos & (ps - 1);
  } else {
    page = pos / ps;
    off = pos - page * ps;
  }
}

// Physical cache row of logical position pos of row r (-1 for none).
__device__ __forceinline__ int phys_of(const TopkArgs& a, int r, int pos) {
  if (pos < 0) return -1;
  int pg, off;
  split_pos(pos, a.page_size, pg, off);
  const int page = a.page_table[(int64_t)r * a.max_pages + pg];
  return (unsigned)page < (unsigned)a.num_pages ? page * a.page_size + off : -1;
}

// Write kept position `pos` at output slot `o` of row r (and its physical
// cache row when requested).
__device__ __forceinline__ void emit(const TopkArgs& a, int r, int o, int pos) {
  a.idx[(int64_t)r * a.k + o] = pos;
  if (a.phys) a.phys[(int64_t)r * a.k + o] = phys_of(a, r, pos);
}

// Output slots o0 .. o0+n-1 of row r receive out_value(get(i)) (get returns
// a slot index, or -1 for padding).  The loads of kGather slots per thread
// are all issued before the first store, so a batch costs one round trip
// per dependent load instead of one per element.
constexpr int kGather = 4;
template <int NT, class Get>
__device__ void emit_range(const TopkArgs& a, int r, uint32_t o0, uint32_t n, Get get) {
  for (uint32_t b = threadIdx.x; b < n; b += NT * kGather) {
    int v[kGather];
#pragma unroll
    for (int u = 0; u < kGather; ++u) {
      const uint32_t i = b + u * NT;
      v[u] = i < n ? get(i) : -1;
    }
#pragma unroll
    for (int u = 0; u < kGather; ++u) v[u] = v[u] >= 0 ? out_value(a, r, v[u]) : -1;
    int pr[kGather];
#pragma unroll
    for (int u = 0; u < kGather; ++u) pr[u] = a.phys ? phys_of(a, r, v[u]) : -1;
#pragma unroll
    for (int u = 0; u < kGather; ++u) {
      const uint32_t i = b + u * NT;
      if (i < n && o0 + i < (uint32_t)a.k) {
        a.idx[(int64_t)r * a.k + o0 + i] = v[u];
        if (a.phys) a.phys[(int64_t)r * a.k + o0 + i] = pr[u];
      }
    }
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void zero_kernel(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

static_assert(kBins == 8 * kBlock, "tiling");

// PER positions per thread: chunks of PER * kBlock positions
// Element j of this thread in a chunk of PER * kBlock scores: thread t
// takes runs of VW consecutive scores, VW * kBlock apart, so that a load is
// VW scores wide (VW = 1 where rows are not 16-byte aligned).
template <int VW>
__device__ __forceinline__ int chunk_pos(int begin, int j) {
  return begin + VW * ((int)threadIdx.x + (j / VW) * kBlock) + j % VW;
}
// The chunk's PER keys of this thread, every load issued before the first
// use; positions past `end` read the last score (and are not counted).
// Keeps the scheduler from moving anything across this point.  Loads are
// issued above it and their values used below it: without it the compiler,
// short of registers, pairs each load with its use, and a batch of loads
// becomes a chain of round trips.
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

template <int PER, int VW>
__device__ __forceinline__ void load_keys(const float* row, int begin, int end, uint32_t (&key)[PER]) {
  static_assert(PER % VW == 0, "runs tile the chunk");
  float x[PER];
#pragma unroll
  for (int q = 0; q < PER / VW; ++q) {
    const int p = chunk_pos<VW>(begin, q * VW);
    if constexpr (VW == 4) {
      if (p + 4 <= end) {
        const float4 v = *reinterpret_cast<const float4*>(row + p);
        x[4 * q] = v.x;
        x[4 * q + 1] = v.y;
        x[4 * q + 2] = v.z;
        x[4 * q + 3] = v.w;
        continue;
      }
    } else if constexpr (VW == 2) {
      if (p + 2 <= end) {
        const float2 v = *reinterpret_cast<const float2*>(row + p);
        x[2 * q] = v.x;
        x[2 * q + 1] = v.y;
        continue;
      }
    }
#pragma unroll
    for (int e = 0; e < VW; ++e) x[q * VW + e] = row[min(p + e, end - 1)];
  }
  issue_fence();
#pragma unroll
  for (int j = 0; j < PER; ++j) key[j] = float_key(x[j]);
}

// Histogram counters in REPS replicas of each bin (lane % REPS picks one):
// with several scores per thread, the lanes of a wave that hit one bin, as
// most do when the scores crowd into a few bins, serialise REPS times less
// on the LDS atomic.  Bins b and b + 2048 (a positive and a negative score
// bin) share the 32-bit words of replica set b % 2048 as low and high
// halves; a replica counts at most kBlock / REPS * PER < 2^16 elements.
template <int PER>
constexpr int hist_reps() { return PER >= 8 ? 4 : 1; }
template <int REPS>
__device__ __forceinline__ uint32_t hist_count(const uint32_t* h, int bin) {
  const int sh = 16 * (bin >> 11);
  if constexpr (REPS == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(h + 4 * (bin & 2047));
    return ((v.x >> sh) & 0xFFFFu) + ((v.y >> sh) & 0xFFFFu) + ((v.z >> sh) & 0xFFFFu) + ((v.w >> sh) & 0xFFFFu);
  } else {
    static_assert(REPS == 1, "one or four replicas");
    return (h[bin & 2047] >> sh) & 0xFFFFu;
  }
}

template <int PER, int VW>
__global__ __launch_bounds__(kBlock) void topk_hist_kernel(TopkArgs a) {
  constexpr int kReps = hist_reps<PER>();
  static_assert(kBlock / kReps * PER < 65536, "16-bit replica counters");
  constexpr int kChunk = PER * kBlock;
  __shared__ __attribute__((aligned(16))) uint32_t hist[kReps * kBins / 2];
  __shared__ uint32_t tmp[32];
  __shared__ uint32_t rr[2];
  const int r = blockIdx.x;   // rows fastest: every row's early (full) chunks
  const int c = blockIdx.y;   // are dispatched before the empty tails
  const int L = row_len(a, r);
  if (L <= a.k) return;
  const int begin = c * kChunk;
  if (begin >= L) return;
  const int end = min(begin + kChunk, L);
  const float* row = a.scores + (int64_t)r * a.ld;
  // the row's key range from the scan's per-workgroup slots (when it
  // recorded them), reduced by every workgroup and stored by the first for
  // the launches that follow
  uint32_t nlo = 0u, hi = 0u;
  if (a.range_slots != nullptr) {
    if (threadIdx.x < 2) rr[threadIdx.x] = 0u;
    for (int i = threadIdx.x; i < a.range_nslots; i += kBlock) {
      const uint4 v = a.range_slots[i];
      if (v.x == (uint32_t)r) {
        nlo = max(nlo, v.y);
        hi = max(hi, v.z);
      }
    }
  }
  // the chunk's loads go out first, so they cost one round trip
  uint32_t d[PER];
  load_keys<PER, VW>(row, begin, end, d);
  for (int i = threadIdx.x; i < kReps * kBins / 2; i += kBlock) hist[i] = 0u;
  __syncthreads();
  Digits dg = row_digits(a.range, r);
  const Ws ws = carve(a.ws, a.num_req, a.max_len);
  if (a.range_slots != nullptr) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      nlo = max(nlo, (uint32_t)__shfl_xor((int)nlo, o));
      hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
    }
    if ((threadIdx.x & 63) == 0) {
      atomicMax(&rr[0], nlo);
      atomicMax(&rr[1], hi);
    }
    __syncthreads();
    dg = row_digits(rr, 0);
    if (c == 0 && threadIdx.x < 2) ws.rng[2 * (size_t)r + threadIdx.x] = rr[threadIdx.x];
  }
  const int rep = threadIdx.x & (kReps - 1);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t bin = dg.d1(d[j]);
    const uint32_t one = chunk_pos<VW>(begin, j) < end ? 1u : 0u;
    atomicAdd(&hist[kReps * (bin & 2047) + rep], one << (16 * (bin >> 11)));
  }
  __syncthreads();
  // the chunk's suffix counts: thread t owns bins 4095-8t down to 4088-8t
  uint32_t v[8], run = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = hist_count<kReps>(hist, kBins - 1 - (8 * (int)threadIdx.x + i));
    run += v[i];
  }
  uint32_t tot;
  uint32_t acc = block_excl_scan<kBlock>(run, tmp, &tot);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc += v[i];
    v[i] = acc;
  }
  // bins 4088-8t .. 4095-8t ascending, 16-bit counts, one 16-byte store
  uint4* suf = reinterpret_cast<uint4*>(ws.suf + ((size_t)r * ws.nchunk + c) * kBins + kBins - 8 - 8 * (int)threadIdx.x);
  *suf = make_uint4(v[7] | (v[6] << 16), v[5] | (v[4] << 16), v[3] | (v[2] << 16), v[1] | (v[0] << 16));
  // and the row's histogram: the non-empty bins, consecutive bins in
  // consecutive lanes (the few hot bins share a cache line, which then takes
  // one atomic request per wave instead of one per lane group)
  uint32_t* gh = ws.hist + (size_t)r * kBins;
  for (int i = threadIdx.x; i < kBins; i += kBlock) {
    const uint32_t n = hist_count<kReps>(hist, i);
    if (n) atomicAdd(&gh[i], n);
  }
}

// The single-workgroup refinement of a row's candidate list: n candidates
// (positions in `list`, or already in LDS as (key, position) pairs), of which
// `need` are still to be taken, after out_pos winners already written.
// The candidates share every key bit above the lowest key_bits of
// (key - kbase); lkey holds (key - kbase) when they sit in LDS.
template <int NT, int CAP>
__device__ void refine_cands(const TopkArgs& a, int r, uint32_t n, uint32_t need, uint32_t out_pos,
                             int32_t* list, bool in_lds, uint32_t* hist, uint32_t* tmp,
                             uint32_t* lkey, int32_t* lslot, int key_bits, uint32_t kbase) {
  const float* row = a.scores + (int64_t)r * a.ld;
  // stages: the unresolved key bits, at most 12 at a time (two stages for up
  // to 24 bits), then position bits [31:20], [19:8], [7:0] ascending
  const int kb_hi = key_bits > 12 ? 12 : key_bits;
  const int kb_lo = key_bits > 12 ? key_bits - 12 : 0;
  if (need > 0 && n > need && n <= 64) {
    // few candidates: the first wave ranks each one against all of them (key
    // descending, then position ascending) and writes the `need` best; no
    // histogram stages and no workgroup barriers
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      uint32_t key = 0u;
      int pos = 0x7FFFFFFF;
      if (lane < (int)n) {
        const int slot = in_lds ? lslot[lane] : list[lane];
        key = in_lds ? lkey[lane] : float_key(row[slot]) - kbase;
        pos = out_value(a, r, slot);
      }
      uint32_t rank = 0;
      for (int j = 0; j < (int)n; ++j) {
        const uint32_t kj = (uint32_t)__shfl((int)key, j);
        const int pj = __shfl(pos, j);
        rank += (kj > key || (kj == key && pj < pos)) ? 1u : 0u;
      }
      const bool take = lane < (int)n && rank < need;
      const uint64_t m = __ballot(take);
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      const uint32_t o = out_pos + (uint32_t)__popcll(m & below);
      if (take && o < (uint32_t)a.k) emit(a, r, (int)o, pos);
    }
    out_pos += need;
    need = 0;
    n = 0;
  }
  for (int stage = 0; stage < 5 && need > 0 && n > 0; ++stage) {
    if (n <= need) break;
    const bool by_key = stage < 2;
    const int nbits = stage == 0 ? kb_hi : stage == 1 ? kb_lo : stage == 4 ? 8 : 12;
    if (nbits == 0) continue;
    if (!in_lds && n <= (uint32_t)CAP) {
      for (uint32_t i = threadIdx.x; i < n; i += NT) {
        const int slot = list[i];
        lslot[i] = slot;
        lkey[i] = float_key(row[slot]) - kbase;
      }
      in_lds = true;
      __syncthreads();   // (the list was written by other threads)
    }
    const int shift = stage == 0 ? kb_lo : stage == 1 ? 0 : stage == 2 ? 20 : stage == 3 ? 8 : 0;
    const uint32_t mask = (1u << nbits) - 1u;
    if (in_lds) {
      // Candidates in LDS: each thread holds up to CAP / NT of them in
      // registers for the whole stage (wave w takes a contiguous run, its
      // lanes interleaved), so the stage needs two count exchanges instead of
      // a block scan per NT candidates.  The kept ones are written back in
      // wave order, not position order: later stages select by value and by
      // position bits, never by list order.
      constexpr int kPer = CAP / NT;
      constexpr int kNW = NT / 64;
      static_assert(kNW <= 16, "per-wave counts fit the 32-word scratch");
      const int lane = threadIdx.x & 63;
      const int w = threadIdx.x >> 6;
      uint32_t v[kPer];
      int sl[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const uint32_t i = (uint32_t)(w * 64 * kPer + j * 64 + lane);
        sl[j] = -1;
        v[j] = 0;
        if (i < n) {
          sl[j] = lslot[i];
          v[j] = by_key ? lkey[i] : (uint32_t)out_value(a, r, sl[j]);
        }
      }
      for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0u;
      wg_sync(true);
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (sl[j] >= 0) atomicAdd(&hist[(v[j] >> shift) & mask], 1u);
      wg_sync(true);
      uint32_t better;
      const int bin = find_threshold<NT>(hist, need, by_key, tmp, &better, true);
      // this thread's winners and kept ones as bit masks over j; the wave's
      // counts by a lane sum (ballots here would be kept live, per j, into
      // the write pass below)
      uint32_t winm = 0, eqm = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int d = (int)((v[j] >> shift) & mask);
        if (sl[j] >= 0) {
          winm |= (uint32_t)(by_key ? d > bin : d < bin) << j;
          eqm |= (uint32_t)(d == bin) << j;
        }
      }
      uint32_t cnt = (uint32_t)__popc(winm) | ((uint32_t)__popc(eqm) << 16);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
      if (lane == 0) {
        tmp[w] = cnt & 0xFFFFu;
        tmp[16 + w] = cnt >> 16;
      }
      wg_sync(true);
      uint32_t ow = out_pos, oe = 0, tw = 0, te = 0;
#pragma unroll
      for (int x = 0; x < kNW; ++x) {
        const uint32_t a0 = tmp[x], a1 = tmp[16 + x];
        if (x < w) {
          ow += a0;
          oe += a1;
        }
        tw += a0;
        te += a1;
      }
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const bool win = (winm >> j) & 1u;
        const bool eq = (eqm >> j) & 1u;
        const uint64_t bw = __ballot(win);
        const uint64_t be = __ballot(eq);
        // winners are staged behind the kept ones (te + tw <= n <= CAP) and
        // written out below in batches: an output row that needs a page-table
        // load would otherwise cost one round trip per j
        if (win) {
          const uint32_t o = ow + (uint32_t)__popcll(bw & below);
          if (o < (uint32_t)a.k) lslot[te + (o - out_pos)] = sl[j];
        }
        if (eq) {
          const uint32_t o = oe + (uint32_t)__popcll(be & below);
          lslot[o] = sl[j];
          if (by_key) lkey[o] = v[j];
        }
        ow += (uint32_t)__popcll(bw);
        oe += (uint32_t)__popcll(be);
      }
      wg_sync(true);
      if (out_pos < (uint32_t)a.k)
        emit_range<NT>(a, r, out_pos, min(tw, (uint32_t)a.k - out_pos),
                       [&](uint32_t i) { return lslot[te + i]; });
      out_pos += tw;
      need -= better;
      n = te;
      continue;
    }
    auto value = [&](uint32_t i, int& slot) -> uint32_t {
      slot = in_lds ? lslot[i] : list[i];
      if (!by_key) return (uint32_t)out_value(a, r, slot);
      return in_lds ? lkey[i] : float_key(row[slot]) - kbase;
    };
    // with the candidates in LDS only LDS traffic needs ordering: the winners
    // written to the output are never read back here
    for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0u;
    wg_sync(in_lds);
    for (uint32_t i = threadIdx.x; i < n; i += NT) {
      int slot;
      const uint32_t v = value(i, slot);
      atomicAdd(&hist[(v >> shift) & mask], 1u);
    }
    wg_sync(in_lds);
    uint32_t better;
    const int bin = find_threshold<NT>(hist, need, by_key, tmp, &better, in_lds);
    // ordered pass: winners (better than bin) go out, equal ones stay; a
    // thread takes kRefPer consecutive candidates, so one block scan orders
    // NT * kRefPer of them (all reads of a batch precede its writes, which
    // land at or below the positions read)
    uint32_t keep = 0;
    for (uint32_t base = 0; base < n; base += NT * kRefPer) {
      const uint32_t i0 = base + threadIdx.x * kRefPer;
      int slot[kRefPer];
      uint32_t v[kRefPer], win = 0, eq = 0;
#pragma unroll
      for (int j = 0; j < kRefPer; ++j) {
        slot[j] = -1;
        v[j] = 0;
        if (i0 + j < n) {
          v[j] = value(i0 + j, slot[j]);
          const int d = (int)((v[j] >> shift) & mask);
          eq |= (uint32_t)(d == bin) << j;
          win |= (uint32_t)(by_key ? (d > bin) : (d < bin)) << j;
        }
      }
      uint32_t tot;
      const uint32_t pre = block_excl_scan<NT>((uint32_t)(__popc(win) | (__popc(eq) << 16)), tmp, &tot, in_lds);
      uint32_t ow = out_pos + (pre & 0xFFFF);
      uint32_t oe = keep + (pre >> 16);
#pragma unroll
      for (int j = 0; j < kRefPer; ++j) {
        if ((win >> j) & 1u) {
          if (ow < (uint32_t)a.k) emit(a, r, ow, out_value(a, r, slot[j]));
          ++ow;
        }
        if ((eq >> j) & 1u) {
          if (in_lds) {
            lslot[oe] = slot[j];
            if (by_key) lkey[oe] = v[j];
          } else {
            list[oe] = slot[j];
          }
          ++oe;
        }
      }
      out_pos += tot & 0xFFFF;
      keep += tot >> 16;
      wg_sync(in_lds);
    }
    need -= better;
    n = keep;
  }
  // whatever remains is taken whole (n <= need here)
  const uint32_t take = min(n, need);
  emit_range<NT>(a, r, out_pos, take, [&](uint32_t i) { return in_lds ? lslot[i] : list[i]; });
  out_pos += take;
  if (out_pos < (uint32_t)a.k) emit_range<NT>(a, r, out_pos, (uint32_t)a.k - out_pos, [](uint32_t) { return -1; });
  if (threadIdx.x == 0) a.count[r] = (int32_t)min(out_pos, (uint32_t)a.k);
}

// Lane t of a wave holds the count of priority position t (t = 0 first).
// Returns the position at which the running count first reaches need
// (1 <= need <= total) and, in *before, the count of the positions ahead of
// it; every lane gets both.
__device__ __forceinline__ int wave_threshold64(uint32_t cnt, uint32_t need, uint32_t* before) {
  const uint32_t inc = wave_incl_sum(cnt);
  const uint64_t m = __ballot(inc >= need);
  const int p = m ? __ffsll((unsigned long long)m) - 1 : 63;
  *before = __shfl(inc - cnt, p);
  return p;
}

// MAPPED: outputs go through the slot map (their pages are looked up per
// winner); otherwise the chunk's page-table entries are staged in LDS
template <int PER, bool MAPPED, int VW>
__global__ __launch_bounds__(kBlock, 8) void topk_select_kernel(TopkArgs a) {
  constexpr int kChunk = PER * kBlock;
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
  __shared__ uint32_t tmp[32];
  __shared__ uint32_t before[2];
  __shared__ uint32_t thr[4];
  __shared__ int pages[MAPPED ? 1 : kSelPages];
  const int r = blockIdx.x;   // rows fastest: every row's early (full) chunks
  const int c = blockIdx.y;   // are dispatched before the empty tails
  const int L = row_len(a, r);
  const int begin = c * kChunk;
  if (begin >= max(L, 1)) return;
  const int end = min(begin + kChunk, L);
  if (L <= a.k) {
    // every element is kept; workgroup 0 also pads and counts
    emit_range<kBlock>(a, r, begin, end - begin, [&](uint32_t i) { return begin + (int)i; });
    if (c == 0) {
      if (L < a.k) emit_range<kBlock>(a, r, L, a.k - L, [](uint32_t) { return -1; });
      if (threadIdx.x == 0) a.count[r] = L;
    }
    return;
  }
  const Ws ws = carve(a.ws, a.num_req, a.max_len);
  const float* row = a.scores + (int64_t)r * a.ld;
  // one round trip for the chunk's keys (the same elements per thread as in
  // the histogram pass), the row histogram and the chunk's page-table
  // entries (so winners leave with their physical rows; with a slot map the
  // pages are only known per winner)
  uint32_t key[PER];
  const Digits dg = row_digits(a.range_slots ? ws.rng : a.range, r);
  load_keys<PER, VW>(row, begin, end, key);
  const uint32_t* gh = ws.hist + (size_t)r * kBins;
  // scan-built histograms: kHistReps replicas of [4096 12-bit | 64 6-bit] bins
  const uint32_t* hr = a.hist_rep ? a.hist_rep + (size_t)r * kHistReps * kHistWords : nullptr;
  constexpr int kRepPer = kHistReps * 64 / kBlock;   // replica bins per thread and level
  static_assert(kRepPer >= 1 && kRepPer * kBlock == kHistReps * 64, "replica bins tile the workgroup");
  if (hr == nullptr) {
    uint32_t hv[kBins / kBlock];
#pragma unroll
    for (int m = 0; m < kBins / kBlock; ++m) hv[m] = gh[threadIdx.x + m * kBlock];
    issue_fence();
#pragma unroll
    for (int m = 0; m < kBins / kBlock; ++m) hist[threadIdx.x + m * kBlock] = hv[m];
  } else {
    uint32_t cv[kRepPer];
#pragma unroll
    for (int m = 0; m < kRepPer; ++m) {
      const int e = threadIdx.x + m * kBlock;
      cv[m] = hr[(e >> 6) * kHistWords + 4096 + (e & 63)];
    }
    issue_fence();
#pragma unroll
    for (int m = 0; m < kRepPer; ++m) hist[threadIdx.x + m * kBlock] = cv[m];
  }
  bool lds_pages = !MAPPED && a.phys;
  int pg0 = 0, off;
  if (lds_pages) {
    int pg1;
    split_pos(begin, a.page_size, pg0, off);
    split_pos(end - 1, a.page_size, pg1, off);
    const int npg = pg1 - pg0 + 1;
    lds_pages = npg <= kSelPages;   // else (tiny pages) each winner looks its page up
    if (lds_pages) {
      const int* pt = a.page_table + (int64_t)r * a.max_pages + pg0;
      static_assert(kSelPages <= 2 * kBlock, "two page ids per thread");
      const int t = threadIdx.x;
      const int p0 = t < npg ? pt[t] : 0;
      const int p1 = t + kBlock < npg ? pt[t + kBlock] : 0;
      issue_fence();
      if (t < npg) pages[t] = p0;
      if (t + kBlock < npg) pages[t + kBlock] = p1;
    }
  }
  if (threadIdx.x < 2) before[threadIdx.x] = 0u;
  __syncthreads();
  uint32_t better, digit, members;   // threshold bin of the whole row, count above it, in it
  if (hr == nullptr) {
    digit = (uint32_t)find_threshold<kBlock>(hist, (uint32_t)a.k, true, tmp, &better);
    members = hist[digit];
  } else {
    // the 6-bit digit first (one wave, lane t = super-bin 63 - t), then the
    // 64 12-bit bins inside the threshold super-bin
    if (threadIdx.x < 64) {
      uint32_t c = 0;
#pragma unroll
      for (int rep = 0; rep < kHistReps; ++rep) c += hist[rep * 64 + 63 - threadIdx.x];
      uint32_t bs;
      const int p = wave_threshold64(c, (uint32_t)a.k, &bs);
      if (threadIdx.x == 0) {
        thr[0] = 63u - (uint32_t)p;
        thr[1] = bs;
      }
    }
    __syncthreads();
    const uint32_t sb = thr[0];
    uint32_t fv[kRepPer];
#pragma unroll
    for (int m = 0; m < kRepPer; ++m) {
      const int e = threadIdx.x + m * kBlock;
      fv[m] = hr[(e >> 6) * kHistWords + 64 * sb + (e & 63)];
    }
    issue_fence();
#pragma unroll
    for (int m = 0; m < kRepPer; ++m) hist[kHistReps * 64 + threadIdx.x + m * kBlock] = fv[m];
    __syncthreads();
    if (threadIdx.x < 64) {
      uint32_t c = 0;
#pragma unroll
      for (int rep = 0; rep < kHistReps; ++rep) c += hist[kHistReps * 64 + rep * 64 + 63 - threadIdx.x];
      uint32_t b2;
      const int p = wave_threshold64(c, (uint32_t)a.k - thr[1], &b2);
      if (threadIdx.x == (unsigned)p) {
        thr[2] = 64u * sb + 63u - (uint32_t)p;
        thr[3] = c;
      }
      if (threadIdx.x == 0) before[0] = thr[1] + b2;   // (read below, before being reset)
    }
    __syncthreads();
    digit = thr[2];
    members = thr[3];
    better = before[0];
    __syncthreads();
    if (threadIdx.x < 2) before[threadIdx.x] = 0u;
  }
  // better < k <= better + members: every member is kept exactly when
  // members == k - better; with `defer` the members then leave with the
  // winners, and otherwise their slots are left to the attention
  const bool members_out = a.defer && members <= (uint32_t)a.k - better;
  if (c == 0 && threadIdx.x == 0) {
    uint32_t* rec = ws.rec + (size_t)r * 4;
    rec[0] = digit;
    rec[1] = better;
    rec[2] = members;
  }
  if (a.defer && c == 0) {
    if (threadIdx.x == 0) a.count[r] = a.k;
    if (!members_out)
      for (int i = (int)better + (int)threadIdx.x; i < a.k; i += kBlock) a.phys[(int64_t)r * a.k + i] = kUnresolvedRow;
  }
  // winners and threshold-bin members of the chunks before this one, from
  // their suffix counts (one load pair per earlier chunk)
  // (summed per wave first: LDS atomics on one address serialise per lane)
  if (hr == nullptr && (int)(threadIdx.x & ~63u) < c) {
    uint32_t nw = 0, ne = 0;
    for (int c2 = threadIdx.x; c2 < c; c2 += kBlock) {
      const uint16_t* sf = ws.suf + ((size_t)r * ws.nchunk + c2) * kBins;
      const uint32_t ge = sf[digit];
      const uint32_t gt = digit + 1 < (uint32_t)kBins ? sf[digit + 1] : 0u;
      nw += gt;
      ne += ge - gt;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      nw += __shfl_xor(nw, o);
      ne += __shfl_xor(ne, o);
    }
    if ((threadIdx.x & 63) == 0) {
      atomicAdd(&before[0], nw);
      atomicAdd(&before[1], ne);
    }
  }
  uint32_t win = 0, eq = 0;      // bit masks over the PER elements
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (chunk_pos<VW>(begin, j) < end) {
      const uint32_t dj = dg.d1(key[j]);
      win |= (uint32_t)(dj > digit) << j;
      eq |= (uint32_t)(dj == digit) << j;
    }
  }
  uint32_t tot;
  const uint32_t pre = block_excl_scan<kBlock>((uint32_t)(__popc(win) | (__popc(eq) << 16)), tmp, &tot);
  if (hr != nullptr) {
    // no per-chunk counts: the chunk's winners and members take their place
    // in the row's output with one returning atomic (the row's first two
    // histogram words, cleared by the scan, serve as the counter pair)
    if (threadIdx.x == 0) {
      unsigned long long* ctr = reinterpret_cast<unsigned long long*>(ws.hist + (size_t)r * kBins);
      const unsigned long long old =
          atomicAdd(ctr, ((unsigned long long)(tot >> 16) << 32) | (unsigned long long)(tot & 0xFFFFu));
      before[0] = (uint32_t)old;
      before[1] = (uint32_t)(old >> 32);
    }
    __syncthreads();
  }
  uint32_t ow = before[0] + (pre & 0xFFFF);
  uint32_t oc = before[1] + (pre >> 16);
  // threshold-bin members first (their keys are then dead), then the
  // winners in groups of eight (fewer live registers: four workgroups fit
  // per compute unit)
  int2* cand = ws.cand + (size_t)r * a.max_len;
  uint32_t om = better + oc;        // output slot of this workgroup's first member
  if (!members_out) {
    int32_t* crow = ws.crow + (size_t)r * a.max_len;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if ((eq >> j) & 1u) {
        const int pos = chunk_pos<VW>(begin, j);
        if (a.defer) {
          // the member's physical row, for the attention that resolves it
          int row;
          if (lds_pages) {
            int pg, po;
            split_pos(pos, a.page_size, pg, po);
            const int page = pages[pg - pg0];
            row = (unsigned)page < (unsigned)a.num_pages ? page * a.page_size + po : -1;
          } else {
            row = phys_of(a, r, pos);
          }
          crow[oc] = row;
        }
        cand[oc++] = make_int2(pos, (int)key[j]);
      }
    }
  }
  // the members' next 12 key bits go into the row's second histogram, so the
  // refinement starts from it: counted in LDS first (the level-1 histogram
  // there is no longer read), then one global add per non-empty bin
  // (not needed when every member is kept)
  // (the member whose LDS add opens a bin adds that bin's final count: no
  // pass over the 4096 bins)
  if ((tot >> 16) != 0u && members > (uint32_t)a.k - better) {   // uniform
    for (int i = threadIdx.x; i < kBins / 4; i += kBlock) reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    uint32_t opened = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if ((eq >> j) & 1u) opened |= (atomicAdd(&hist[dg.d2(key[j])], 1u) == 0u ? 1u : 0u) << j;
    __syncthreads();
    uint32_t* g2 = ws.h2 + (size_t)r * kBins;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if ((opened >> j) & 1u) {
        const uint32_t d2 = dg.d2(key[j]);
        atomicAdd(&g2[d2], hist[d2]);
      }
  }
  // with members_out the members are emitted like winners, at slots after
  // every winner of the row
  const uint32_t emit = members_out ? (win | eq) : win;
  constexpr int G = PER < 8 ? PER : 8;
#pragma unroll
  for (int g0 = 0; g0 < PER; g0 += G) {
    int wv[G], wp[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int j = g0 + u;
      const int i = chunk_pos<VW>(begin, j);
      wv[u] = ((emit >> j) & 1u) ? (MAPPED ? out_value(a, r, i) : i) : -1;
    }
    if (lds_pages) {
      // every page read first, then the rows (non-winners read a valid dummy)
      int pg[G], po[G], page[G];
#pragma unroll
      for (int u = 0; u < G; ++u) split_pos(max(wv[u], begin), a.page_size, pg[u], po[u]);
#pragma unroll
      for (int u = 0; u < G; ++u) page[u] = pages[pg[u] - pg0];
#pragma unroll
      for (int u = 0; u < G; ++u)
        wp[u] = (wv[u] >= 0 && (unsigned)page[u] < (unsigned)a.num_pages) ? page[u] * a.page_size + po[u] : -1;
    } else {
#pragma unroll
      for (int u = 0; u < G; ++u) wp[u] = a.phys ? phys_of(a, r, wv[u]) : -1;
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if ((win >> (g0 + u)) & 1u) {
        if (ow < (uint32_t)a.k) {
          a.idx[(int64_t)r * a.k + ow] = wv[u];
          if (a.phys) a.phys[(int64_t)r * a.k + ow] = wp[u];
        }
        ++ow;
      } else if (members_out && ((eq >> (g0 + u)) & 1u)) {
        if (om < (uint32_t)a.k) {
          a.idx[(int64_t)r * a.k + om] = wv[u];
          a.phys[(int64_t)r * a.k + om] = wp[u];
        }
        ++om;
      }
    }
  }
}

__global__ __launch_bounds__(kRefThreads) void topk_refine_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t lkey[kLdsCand];
  __shared__ int32_t lslot[kLdsCand];
  __shared__ uint32_t tmp[32];
  const int r = blockIdx.x;
  const int L = row_len(a, r);
  if (L <= a.k) return;
  const Ws ws = carve(a.ws, a.num_req, a.max_len);
  const Digits dg = row_digits(a.range_slots ? ws.rng : a.range, r);
  // the threshold bin's members are the candidates (everything above it has
  // been written already); their second histogram (level-2 digits) was
  // built by the select, so one ordered pass over them settles 12 more bits.
  // The histogram, the record and the first batch of members are loaded
  // together.
  constexpr int kU = kRefBatch / kRefThreads;
  const uint32_t* rec = ws.rec + (size_t)r * 4;
  const int2* cand = ws.cand + (size_t)r * a.max_len;
  const uint32_t* g2 = ws.h2 + (size_t)r * kBins;
  const int tid = threadIdx.x;
  uint32_t hv[kBins / kRefThreads];
  int2 e[kU];
#pragma unroll
  for (int m = 0; m < kBins / kRefThreads; ++m) hv[m] = g2[tid + m * kRefThreads];
#pragma unroll
  for (int u = 0; u < kU; ++u) e[u] = cand[min(tid + u * kRefThreads, a.max_len - 1)];
  const uint32_t better = rec[1];
  const uint32_t n = rec[2];
  issue_fence();
#pragma unroll
  for (int m = 0; m < kBins / kRefThreads; ++m) hist[tid + m * kRefThreads] = hv[m];
  const uint32_t need = (uint32_t)a.k - better;
  if (n <= need) {
    // every member is kept (then n == need): written out directly, every
    // output row (and its page) looked up before any store
    for (uint32_t base = 0; base < n; base += kRefBatch) {
      if (base > 0) {
#pragma unroll
        for (int u = 0; u < kU; ++u) e[u] = cand[min(base + tid + u * kRefThreads, n - 1)];
      }
      int wv[kU], wp[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) wv[u] = base + tid + u * kRefThreads < n ? out_value(a, r, e[u].x) : -1;
#pragma unroll
      for (int u = 0; u < kU; ++u) wp[u] = a.phys ? phys_of(a, r, wv[u]) : -1;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t i = base + tid + u * kRefThreads;
        if (i < n) {
          a.idx[(int64_t)r * a.k + better + i] = wv[u];
          if (a.phys) a.phys[(int64_t)r * a.k + better + i] = wp[u];
        }
      }
    }
    if (tid == 0) a.count[r] = (int32_t)(better + n);
    return;
  }
  wg_sync(true);
  uint32_t better2;
  const uint32_t bin2 = (uint32_t)find_threshold<kRefThreads>(hist, need, true, tmp, &better2, true);
  const uint32_t n2 = hist[bin2];
  // when the second threshold bin's members are all kept (the usual case:
  // one or two of them) they leave in the pass below with the winners
  const bool take_eq = n2 <= need - better2;
  const bool in_lds = n2 <= (uint32_t)kLdsCand;
  int32_t* list = ws.list + (size_t)r * a.max_len;
  uint32_t ow = better, oe = 0;
  // The first batch (loaded with the histogram) is waited for here, by a
  // wait the compiler can see: otherwise it counts those loads as pending
  // inside the loop and waits for every store of the previous batch before
  // reusing their registers.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  // Two copies of the pass: positions leaving as they are (no slot map, no
  // physical rows), and with their lookups.  A lookup load that is issued
  // and used only under a condition still counts as pending where the loop
  // starts again, and the compiler then waits for every outstanding store
  // before reusing its register: one loop with both cases ran its stores
  // one round trip at a time.
  auto pass = [&](auto plain_tag) {
    constexpr bool kPlain = decltype(plain_tag)::value;
    for (uint32_t base = 0; base < n; base += kRefBatch) {
      if (base > 0) {
#pragma unroll
        for (int u = 0; u < kU; ++u) e[u] = cand[min(base + tid + u * kRefThreads, n - 1)];
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the batch, before any branch uses it
      }
      uint32_t win = 0, eq = 0;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (base + tid + u * kRefThreads < n) {
          const uint32_t d = dg.d2((uint32_t)e[u].y);
          win |= (uint32_t)(d > bin2 || (take_eq && d == bin2)) << u;
          eq |= (uint32_t)(!take_eq && d == bin2) << u;
        }
      }
      uint32_t tot;
      const uint32_t pre = block_excl_scan<kRefThreads>((uint32_t)(__popc(win) | (__popc(eq) << 16)), tmp, &tot, true);
      uint32_t o = ow + (pre & 0xFFFF);
      uint32_t q = oe + (pre >> 16);
      // winners: every output row (and its page) is looked up before any store
      // (the lookups load for every element, at clamped indexes, and are
      // masked afterwards: loads under a per-element condition were each
      // waited for on their own)
      int wv[kU], wp[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        wv[u] = e[u].x;
        wp[u] = -1;
      }
      if constexpr (!kPlain) {
        if (a.map) {
#pragma unroll
          for (int u = 0; u < kU; ++u)
            wv[u] = a.map[(int64_t)r * a.map_ld + (((win >> u) & 1u) ? e[u].x : 0)];
        }
        // non-winners (possibly unwritten words past the row's members) look
        // up position 0
#pragma unroll
        for (int u = 0; u < kU; ++u) wv[u] = ((win >> u) & 1u) ? wv[u] : -1;
        if (a.phys) {
          int pg[kU], off[kU];
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            split_pos(max(wv[u], 0), a.page_size, pg[u], off[u]);
            wp[u] = a.page_table[(int64_t)r * a.max_pages + pg[u]];
          }
#pragma unroll
          for (int u = 0; u < kU; ++u)
            wp[u] = wv[u] >= 0 && (unsigned)wp[u] < (unsigned)a.num_pages ? wp[u] * a.page_size + off[u] : -1;
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if ((win >> u) & 1u) {
          if (o < (uint32_t)a.k) {
            a.idx[(int64_t)r * a.k + o] = wv[u];
            if (!kPlain && a.phys) a.phys[(int64_t)r * a.k + o] = wp[u];
          }
          ++o;
        }
        if ((eq >> u) & 1u) {
          if (in_lds) {
            lslot[q] = e[u].x;
            lkey[q] = (uint32_t)e[u].y - dg.base;
          } else {
            list[q] = e[u].x;
          }
          ++q;
        }
      }
      ow += tot & 0xFFFF;
      oe += tot >> 16;
    }
  };
  if (a.map == nullptr && a.phys == nullptr) {
    pass(std::true_type{});
  } else {
    pass(std::false_type{});
  }
  if (take_eq) {
    if (tid == 0) a.count[r] = (int32_t)min(better + better2 + n2, (uint32_t)a.k);
    return;
  }
  wg_sync(in_lds);
  // the members that share the level-2 digit: the key bits below it, then
  // positions
  refine_cands<kRefThreads, kLdsCand>(a, r, n2, need - better2, better + better2, list, in_lds, hist,
                                      tmp, lkey, lslot, dg.sh2, dg.base);
}

// ---------------------------------------------------------------------------
// One workgroup per row, for batches of rows and short rows.  Scores gather
// in a few binades, so the top bits of the key would put most of a row into a
// handful of histogram bins (and the LDS atomics on them in line); the first
// digit is instead (key - row minimum) >> shift, with shift chosen so that the
// row's key range fills the 4096 bins.  That is monotone in the key, so the
// select stays exact; the refinement resolves the `shift` bits below it.
//   pass 0: row minimum and maximum key (no atomics)
//   pass 1: LDS histogram of the first digit
//   pass 2: keys above the threshold bin go straight out, the bin's members
//           are collected in LDS (slots from wave-aggregated LDS counters)
//   then the refinement in LDS.  No global atomics, no state to clear.
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 1024;
constexpr int kRowCap = 8192;     // candidates held in LDS

// NB batches of kRowThreads * kBatch scores stay in registers for all three
// passes (a row of up to NB batches is read from memory once); batches past
// them are streamed again by every pass.  One resident batch: holding whole
// 64K-score rows (NB = 9, 72 registers of keys) spills at 128 VGPRs and ran
// slower than streaming them three times.
// LOOKUP: the row has a slot map or physical rows to look up per winner.
// Without it the select pass loads nothing: a load there is waited for with
// vmcnt(0), which also waits for every earlier batch's winner stores.
template <int NB, bool LOOKUP>
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t lkey[kRowCap];
  __shared__ int32_t lslot[kRowCap];
  __shared__ uint32_t tmp[32];
  __shared__ uint32_t cnt[2];
  __shared__ uint32_t red[2][kRowThreads / 64];
  const int r = blockIdx.x;
  const int L = row_len(a, r);
  const float* row = a.scores + (int64_t)r * a.ld;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (L <= a.k) {
    emit_range<kRowThreads>(a, r, 0, L, [](uint32_t i) { return (int)i; });
    if (L < a.k) emit_range<kRowThreads>(a, r, L, a.k - L, [](uint32_t) { return -1; });
    if (tid == 0) a.count[r] = L;
    return;
  }
  // pass 0: key range of the row
  // (each streaming batch issues kBatch loads per thread before using any;
  // indexes past the end are clamped to the last element, which is harmless
  // for the minimum and maximum and not counted elsewhere)
  constexpr int kStride = kRowThreads * kBatch;
  const int nbat = (L + kStride - 1) / kStride;
  uint32_t kr[NB][kBatch];
  // the resident batches' slot-map entries come in with their scores (a
  // winner's output value is then in a register, not one more round trip)
  int mv[NB][kBatch];
  const bool pre_map = LOOKUP && a.map != nullptr;
  {
    float x[NB][kBatch];
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = min(tid + bi * kStride + j * kRowThreads, L - 1);
        x[bi][j] = bi < nbat ? row[i] : 0.f;
        mv[bi][j] = pre_map && bi < nbat ? a.map[(int64_t)r * a.map_ld + i] : 0;
      }
    issue_fence();
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int j = 0; j < kBatch; ++j) kr[bi][j] = bi < nbat ? float_key(x[bi][j]) : 0u;
  }
  // f(b, keys, map entries or nullptr) for every batch b of this thread, the
  // resident ones first
  auto for_batches = [&](auto&& f) {
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
      if (bi < nbat) f(tid + bi * kStride, kr[bi], pre_map ? mv[bi] : nullptr);
    for (int b = tid + NB * kStride; b < L; b += kStride) {
      float x[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) x[j] = row[min(b + j * kRowThreads, L - 1)];
      issue_fence();
      uint32_t kk[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) kk[j] = float_key(x[j]);
      f(b, kk, static_cast<const int*>(nullptr));
    }
  };
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  if (a.range) {
    // the producer recorded the row's key range (the same keys)
    kmin = ~a.range[2 * (int64_t)r];
    kmax = a.range[2 * (int64_t)r + 1];
  } else {
    for_batches([&](int, const uint32_t (&kk)[kBatch], const int*) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        kmin = min(kmin, kk[j]);
        kmax = max(kmax, kk[j]);
      }
    });
  }
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  }
  if (lane == 0) {
    red[0][wave] = kmin;
    red[1][wave] = kmax;
  }
  for (int i = tid; i < kBins; i += kRowThreads) hist[i] = 0u;
  if (tid < 2) cnt[tid] = 0u;
  __syncthreads();
#pragma unroll
  for (int wv = 0; wv < kRowThreads / 64; ++wv) {
    kmin = min(kmin, red[0][wv]);
    kmax = max(kmax, red[1][wv]);
  }
  const uint32_t range = kmax - kmin;
  const int span = range ? 32 - __clz(range) : 0;      // bits of the range
  const int shift = span > 12 ? span - 12 : 0;
  // pass 1
  for_batches([&](int b, const uint32_t (&kk)[kBatch], const int*) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) atomicAdd(&hist[(kk[j] - kmin) >> shift], b + j * kRowThreads < L ? 1u : 0u);
  });
  __syncthreads();
  uint32_t better;
  const uint32_t digit = (uint32_t)find_threshold<kRowThreads>(hist, (uint32_t)a.k, true, tmp, &better);
  int32_t* list = carve(a.ws, a.num_req, a.max_len).list + (size_t)r * a.max_len;
  // pass 2.  Resident batches (a uniform loop): flags per thread, one block
  // scan of the winner and member counts, then every thread writes its own
  // (a ballot pair per element, as below, is about 3 us of issue at 1024
  // threads).  Streamed batches: per-wave ballots and LDS counters.
#pragma unroll
  for (int bi = 0; bi < NB; ++bi) {
    if (bi < nbat) {
      const int b = tid + bi * kStride;
      uint32_t win = 0, eq = 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const bool in = b + j * kRowThreads < L;
        const uint32_t d = (kr[bi][j] - kmin) >> shift;
        win |= (uint32_t)(in && d > digit) << j;
        eq |= (uint32_t)(in && d == digit) << j;
      }
      const uint32_t base_w = cnt[0], base_e = cnt[1];   // read before the scan's barriers
      uint32_t tot;
      const uint32_t pre =
          block_excl_scan<kRowThreads>((uint32_t)__popc(win) | ((uint32_t)__popc(eq) << 16), tmp, &tot, true);
      uint32_t ow = base_w + (pre & 0xFFFFu), oe = base_e + (pre >> 16);
      int wv[kBatch], wp[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = b + j * kRowThreads;
        wv[j] = ((win >> j) & 1u) ? (LOOKUP ? (pre_map ? mv[bi][j] : out_value(a, r, i)) : i) : -1;
      }
      if constexpr (LOOKUP) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) wp[j] = a.phys ? phys_of(a, r, wv[j]) : -1;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if ((win >> j) & 1u) {
          a.idx[(int64_t)r * a.k + ow] = wv[j];
          if (LOOKUP && a.phys) a.phys[(int64_t)r * a.k + ow] = wp[j];
          ++ow;
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if ((eq >> j) & 1u) {
          const int i = b + j * kRowThreads;
          if (oe < (uint32_t)kRowCap) {
            lkey[oe] = kr[bi][j] - kmin;
            lslot[oe] = i;
          }
          if (oe < (uint32_t)a.max_len) list[oe] = i;
          ++oe;
        }
      }
      if (tid == 0) {
        cnt[0] = base_w + (tot & 0xFFFFu);
        cnt[1] = base_e + (tot >> 16);
      }
      wg_sync(true);
    }
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  auto for_streamed = [&](auto&& f) {
    for (int b = tid + NB * kStride; b < L; b += kStride) {
      float x[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) x[j] = row[min(b + j * kRowThreads, L - 1)];
      issue_fence();
      uint32_t kk[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) kk[j] = float_key(x[j]);
      f(b, kk, static_cast<const int*>(nullptr));
    }
  };
  for_streamed([&](int b, const uint32_t (&kk)[kBatch], const int* pm) {
    uint32_t rel[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) rel[j] = kk[j] - kmin;
    uint64_t bw[kBatch], be[kBatch];
    uint32_t nw = 0, ne = 0;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool in = b + j * kRowThreads < L;
      const uint32_t d = rel[j] >> shift;
      bw[j] = __ballot(in && d > digit);
      be[j] = __ballot(in && d == digit);
      nw += (uint32_t)__popcll(bw[j]);
      ne += (uint32_t)__popcll(be[j]);
    }
    // one LDS counter update per wave and batch
    uint32_t wb = 0, eb = 0;
    if (lane == 0) {
      if (nw) wb = atomicAdd(&cnt[0], nw);
      if (ne) eb = atomicAdd(&cnt[1], ne);
    }
    wb = __shfl(wb, 0);
    eb = __shfl(eb, 0);
    // winners: all value and page loads first, then the stores
    int wv[kBatch], wp[kBatch];
    uint32_t wo[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      wo[j] = wb + (uint32_t)__popcll(bw[j] & below);
      wb += (uint32_t)__popcll(bw[j]);
      const int i = b + j * kRowThreads;
      wv[j] = ((bw[j] >> lane) & 1ull) ? (LOOKUP ? (pm ? pm[j] : out_value(a, r, i)) : i) : -1;
    }
    if constexpr (LOOKUP) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) wp[j] = a.phys ? phys_of(a, r, wv[j]) : -1;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if ((bw[j] >> lane) & 1ull) {
        a.idx[(int64_t)r * a.k + wo[j]] = wv[j];
        if (LOOKUP && a.phys) a.phys[(int64_t)r * a.k + wo[j]] = wp[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = b + j * kRowThreads;
      if ((be[j] >> lane) & 1ull) {
        const uint32_t c = eb + (uint32_t)__popcll(be[j] & below);
        if (c < (uint32_t)kRowCap) {
          lkey[c] = rel[j];
          lslot[c] = i;
        }
        if (c < (uint32_t)a.max_len) list[c] = i;
      }
      eb += (uint32_t)__popcll(be[j]);
    }
  });
  __syncthreads();
  const uint32_t n = cnt[1];
  refine_cands<kRowThreads, kRowCap>(a, r, n, (uint32_t)a.k - better, better, list, n <= (uint32_t)kRowCap,
                                     hist, tmp, lkey, lslot, shift, kmin);
}

}  // namespace

size_t topk_ws_bytes(int num_req, int max_len) {
  const size_t R = (size_t)num_req;
  return align_up(2 * R * kBins * 4 + R * max_chunks(max_len) * kBins * 2 + (4 * R * max_len + 6 * R) * 4, 256);
}

int64_t topk_zero_words(int num_req) { return (int64_t)num_req * 2 * kBins; }

hipError_t launch_zero(uint32_t* p, int64_t n, hipStream_t s) {
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(n, kBlock * 4), 1024));
  launch(zero_kernel, dim3(blocks), dim3(kBlock), 0, s, "zero_kernel", p, n);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, int ws_state, hipStream_t s) {
  // rows enough to fill every compute unit, or short ones: one workgroup per
  // row is enough parallelism and needs no hand-over between workgroups
  if (a.num_req >= num_cus() || a.max_len <= 32768) {
    if (a.map != nullptr || a.phys != nullptr)
      launch((topk_row_kernel<1, true>), dim3(a.num_req), dim3(kRowThreads), 0, s, "topk_row_kernel", a);
    else
      launch((topk_row_kernel<1, false>), dim3(a.num_req), dim3(kRowThreads), 0, s, "topk_row_kernel", a);
    return hipGetLastError();
  }
  if (ws_state == 0) {
    const hipError_t e = launch_zero(static_cast<uint32_t*>(a.ws), topk_zero_words(a.num_req), s);
    if (e != hipSuccess) return e;
  }
  // chunks sized for about two workgroups per compute unit, and at most 256
  // chunks per row: every chunk adds to the row histogram's few hot bins,
  // whose atomics serialise (a 524288-score row in 512 chunks spent 10 us
  // in the histogram launch, 4 us less in 128).  With scan-built histograms
  // every chunk places its output with one returning atomic on the row's
  // counter pair, and those serialise too (~12 ns each: 128 chunks of a
  // 131072-score row spread their placements over 1.5 us): chunks of 2048
  // scores (64 chunks of a 131072-score row: 0.2 us faster than 128; 32:
  // 0.4 us slower), and for
  // longer rows 128 chunks (a 524288-score row whose threshold bin holds
  // ~10,000 members: 7.8 us in 128 chunks, 10.1 in 64).
  const int64_t want = a.hist_rep != nullptr ? std::max<int64_t>(2048, ceil_div(a.max_len, 128))
                                             : ceil_div((int64_t)a.num_req * a.max_len, 2 * (int64_t)num_cus());
  int per = kMinChunk / kBlock;
  while (per * kBlock < kMaxChunk && (per * kBlock < want || ceil_div(a.max_len, per * kBlock) > 256)) per *= 2;
  dim3 grid((unsigned)a.num_req, (unsigned)std::max<int64_t>(1, ceil_div(a.max_len, per * kBlock)));
  const bool mapped = a.map != nullptr;
  // rows that start on 16-byte boundaries are read 4 (or 2) scores per load
  const bool vec = reinterpret_cast<uintptr_t>(a.scores) % 16 == 0 && a.ld % 4 == 0;
  switch (per * (vec ? 1 : -1)) {
#define LSI_TOPK_PER(P, VW)                                                                           \
  case (VW == 1 ? -P : P):                                                                            \
    if (a.hist_rep == nullptr) {                                                                      \
      launch((topk_hist_kernel<P, VW>), grid, dim3(kBlock), 0, s, "topk_hist_kernel", a);                                                               \
    }                                                                                                 \
    if (mapped) launch((topk_select_kernel<P, true, VW>), grid, dim3(kBlock), 0, s, "topk_select_kernel", a); \
    else launch((topk_select_kernel<P, false, VW>), grid, dim3(kBlock), 0, s, "topk_select_kernel", a);                                                               \
    break;
    LSI_TOPK_PER(2, 2)
    LSI_TOPK_PER(4, 4)
    LSI_TOPK_PER(8, 4)
    LSI_TOPK_PER(16, 4)
    LSI_TOPK_PER(2, 1)
    LSI_TOPK_PER(4, 1)
    LSI_TOPK_PER(8, 1)
    LSI_TOPK_PER(16, 1)
#undef LSI_TOPK_PER
    default: return hipErrorInvalidValue;
  }
  if (!a.defer) {
    launch(topk_refine_kernel, dim3(a.num_req), dim3(kRefThreads), 0, s, "topk_refine_kernel", a);
  }
  return hipGetLastError();
}

bool topk_can_defer(int num_req, int max_len) {
  // the multi-workgroup path (the only one that defers)
  return !(num_req >= num_cus() || max_len <= 32768);
}

}  // namespace lsi

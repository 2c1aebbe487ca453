// Indexer scores of a prefill chunk against one block of keys (history block
// or the chunk itself), causal: query i sits at position hist_len + i and
// scores positions <= hist_len + i, and the running selection of the k best
// of them.  (LeanSparse episode notes: prefill streams a layer's history
// through two alternating GPU buffers, which keeps its workspace small; the
// host side of the streaming lives with the C ABI, this file is the compute.)
//
// A workgroup holds eight queries (one per wave, each wave keeps its query's
// 64x128 bf16 operand in registers) and walks every 64-token tile of the
// block.  A tile's fp8 codes are fetched once per workgroup (16 bytes per
// thread), converted exactly to bf16 into one of two LDS buffers and
// consumed by all eight waves: while the waves compute tile i from one
// buffer, tile i + 1 is converted into the other and tile i + 2 is on its
// way from memory, so a tile costs one barrier.  The score math is the one
// of the decode scan: v_mfma_f32_32x32x16_bf16 over 32 heads x 32 tokens
// per K-step, ReLU and head weights in registers.
//
// No score matrix: each query keeps a buffer of candidates (order-preserving
// score key, position) of capacity cap >= 2k + 512 and an entry threshold.
// A score enters only if its key exceeds the threshold.  Every 8 tiles a
// wave whose buffer could overflow before the next check prunes it on its
// own (radix digits of the keys over the buffer's key range, in a private
// LDS histogram), keeping at least k and at most k + 64 candidates in
// position order, and raises the threshold to the smallest kept key.  At
// least k kept candidates beat any later token whose key is at or below it
// (equal keys rank by position, and a later token has a higher one), so
// nothing that could still be selected is dropped.  A query belongs to the
// same wave and workgroup index in every launch, so its buffer and state are
// never shared.  The launch over the last block reduces each buffer to
// exactly its k best and writes their positions in ascending order.
// Workspace: T x cap x 8 bytes, O(T k).
#include "lsi_internal.hpp"

namespace lsi {
namespace {

constexpr int kTile = 64;      // tokens per tile
constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kStride = 136;   // bf16 per LDS key row (padding vs bank conflicts)
constexpr int kQPerWg = 8;     // queries per workgroup, one per wave
constexpr int kThreads = 64 * kQPerWg;
static_assert(kTile * kDim == 16 * kThreads, "one 16-byte piece of a tile per thread");
constexpr int kCheckTiles = 8;  // tiles between capacity checks of the candidate buffers

constexpr int kWBins = 2048;    // bins of a wave's private LDS histogram (11-bit digits)
constexpr uint32_t kSlack = 64; // entries a pruning may keep beyond k
constexpr int kGroup = 8;       // 128-entry chunks a pruning pass loads at once

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int) { return wave_incl_sum(v); }

// Over the wave's histogram h (kWBins words) in descending bin order, the
// bin where the running count first reaches need (1 <= need <= total), the
// count of the bins above it and its own count.  Lane l sums bins
// 2047 - 32 l - 31 .. 2047 - 32 l; the lane where the count is reached then
// splits its 32 bins over 32 lanes.
__device__ __forceinline__ void wave_threshold(const uint32_t* h, uint32_t need, int lane, uint32_t& bin,
                                               uint32_t& above, uint32_t& members) {
  const uint4* p = reinterpret_cast<const uint4*>(h + kWBins - 32 - 32 * lane);
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 v = p[i];
    sum += v.x + v.y + v.z + v.w;
  }
  const uint32_t incl = wave_incl_scan(sum, lane);
  const int L = min((int)__builtin_ctzll(__ballot(incl >= need)), 63);
  const uint32_t before = (uint32_t)__shfl((int)(incl - sum), L);
  const uint32_t c = lane < 32 ? h[kWBins - 1 - 32 * L - lane] : 0u;
  const uint32_t ci = wave_incl_scan(c, lane) + before;
  const int j = min((int)__builtin_ctzll(__ballot(lane < 32 && ci >= need)), 31);
  bin = (uint32_t)(kWBins - 1 - 32 * L - j);
  members = (uint32_t)__shfl((int)c, j);
  above = (uint32_t)__shfl((int)ci, j) - members;
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Pruning of one query's candidate buffer by its own wave (no workgroup
// barrier; the other waves keep scanning).  buf holds n entries (key,
// position) in position order (capacity cap, even); every pass reads them
// 1024 at a time, two consecutive entries per lane and chunk of 128.  The rank order is key descending, then
// position ascending.  The bound is found digit by digit: 11-bit digits of
// key - (smallest key) over the buffer's own key range, in the wave's LDS
// histogram wh.  A level ends the search when its threshold bin can be kept
// whole: exactly (the k-th entry closes the bin), or, when not final, with
// at most `limit` entries in all (k <= limit); a single key value left over keeps its
// lowest positions, which come first in the buffer.  The kept entries are
// packed in order: into buf (returns their count; tau receives their
// smallest key, the next entry threshold, since at least k entries beat
// anything at or below it that comes later) or, when final, their positions
// into idx_row followed by -1 up to k (returns the count).
__device__ uint32_t wave_prune(uint2* buf, uint32_t n, uint32_t cap, uint32_t k, uint32_t limit, bool final_pass,
                               uint32_t* wh, int lane, int32_t* idx_row, uint32_t& tau) {
  constexpr uint32_t kNone = 0xFFFFFFFFu;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  // f(e0, e1) for entries i, i + 1 (i even; position kNone past the end),
  // every lane's pair of a chunk of 128 in order, kGroup chunks loaded
  // before any is used (addresses clamped into the buffer, which holds cap
  // entries; values past n are ignored)
  auto pass = [&](auto&& f) {
    for (uint32_t g0 = 0; g0 < n; g0 += 128 * kGroup) {
      uint4 v[kGroup];
#pragma unroll
      for (int c = 0; c < kGroup; ++c) {
        const uint32_t i = min(g0 + 128 * c + 2 * lane, cap - 2);
        v[c] = *reinterpret_cast<const uint4*>(buf + i);
      }
#pragma unroll
      for (int c = 0; c < kGroup; ++c) {
        const uint32_t i = g0 + 128 * c + 2 * lane;
        f(make_uint2(v[c].x, i < n ? v[c].y : kNone), make_uint2(v[c].z, i + 1 < n ? v[c].w : kNone));
      }
    }
  };
  // kept: key > K, or key == K and among the first need_tie such entries
  uint32_t K = 0u, need_tie = kNone;
  if (n > k) {
    uint32_t mn = kNone, mx = 0u;
    pass([&](uint2 e0, uint2 e1) {
      if (e0.y != kNone) { mn = min(mn, e0.x); mx = max(mx, e0.x); }
      if (e1.y != kNone) { mn = min(mn, e1.x); mx = max(mx, e1.x); }
    });
    mn = wave_min(mn);
    mx = wave_max(mx);
    const uint32_t span = (mx - mn) >> 11;
    int sh = span ? 32 - __clz((int)span) : 0;      // (mx - mn) >> sh < kWBins
    int w = 32;                                       // the current bin: keys base .. base + 2^w - 1
    uint32_t base = mn;
    uint32_t kept_above = 0;                          // entries above the current bin
    for (;;) {
      uint4* z = reinterpret_cast<uint4*>(wh);
#pragma unroll
      for (int i = 0; i < kWBins / 256; ++i) z[lane + 64 * i] = make_uint4(0u, 0u, 0u, 0u);
      pass([&](uint2 e0, uint2 e1) {
        const uint32_t d0 = e0.x - base, d1 = e1.x - base;
        if (e0.y != kNone && e0.x >= base && ((uint64_t)d0 >> w) == 0) atomicAdd(&wh[d0 >> sh], 1u);
        if (e1.y != kNone && e1.x >= base && ((uint64_t)d1 >> w) == 0) atomicAdd(&wh[d1 >> sh], 1u);
      });
      uint32_t b, above, members;
      wave_threshold(wh, k - kept_above, lane, b, above, members);
      kept_above += above;
      const uint32_t lo = base + (b << sh);
      const uint32_t need = k - kept_above;
      if (members == need || (!final_pass && kept_above + members <= limit)) {
        K = lo - 1u;   // every key >= lo (lo > the entry threshold >= 0)
        need_tie = 0u;
        break;
      }
      if (sh == 0) {   // one key value: its first `need` entries
        K = lo;
        need_tie = need;
        break;
      }
      base = lo;
      w = sh;
      sh = sh > 11 ? sh - 11 : 0;
    }
  }
  uint32_t out = 0, seen_tie = 0, kmin = kNone;
  // in place: a chunk's kept entries go below its end, and every chunk of
  // a group is read before any of them is written
  pass([&](uint2 e0, uint2 e1) {
    const bool v0 = e0.y != kNone, v1 = e1.y != kNone;
    const bool t0 = v0 && e0.x == K, t1 = v1 && e1.x == K;
    const uint64_t bt0 = __ballot(t0), bt1 = __ballot(t1);
    const uint32_t r0 = seen_tie + (uint32_t)(__popcll(bt0 & below) + __popcll(bt1 & below));
    const uint32_t r1 = r0 + (t0 ? 1u : 0u);
    seen_tie += (uint32_t)(__popcll(bt0) + __popcll(bt1));
    const bool k0 = v0 && (e0.x > K || (t0 && r0 < need_tie));
    const bool k1 = v1 && (e1.x > K || (t1 && r1 < need_tie));
    const uint64_t m0 = __ballot(k0), m1 = __ballot(k1);
    const uint32_t o0 = out + (uint32_t)(__popcll(m0 & below) + __popcll(m1 & below));
    const uint32_t o1 = o0 + (k0 ? 1u : 0u);
    if (k0) {
      if (final_pass) idx_row[o0] = (int32_t)e0.y;
      else buf[o0] = e0;
      kmin = min(kmin, e0.x);
    }
    if (k1) {
      if (final_pass) idx_row[o1] = (int32_t)e1.y;
      else buf[o1] = e1;
      kmin = min(kmin, e1.x);
    }
    out += (uint32_t)(__popcll(m0) + __popcll(m1));
  });
  if (final_pass)
    for (uint32_t i = out + lane; i < k; i += 64) idx_row[i] = -1;
  tau = wave_min(kmin);
  return out;
}

__global__ __launch_bounds__(kThreads, 2) void prefill_scan_kernel(PrefillScanArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 kt[2][kTile * kStride];
  __shared__ float ksc[2][kTile];
  __shared__ __attribute__((aligned(16))) uint32_t whist[kQPerWg][kWBins];   // one per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 31;
  const int h = lane >> 5;
  const int q0 = blockIdx.x * kQPerWg;
  const int qi = q0 + wave;
  const bool active = qi < a.T;
  const int q_last = min(q0 + kQPerWg - 1, a.T - 1);
  // tokens of this block visible to the last query of the workgroup
  const int n_eff = min(a.n_tok, a.hist_len + q_last + 1 - a.tok0);
  if (n_eff <= 0 && !a.final_block) return;
  const int ntile = n_eff > 0 ? (n_eff + kTile - 1) / kTile : 0;
  const int my_last = active ? a.hist_len + qi : -1;   // last visible position
  // this wave's query: candidate count and entry threshold (a key)
  uint32_t cnt_r = 0, tau_r = 0;
  if (active) {
    cnt_r = a.state[2 * (int64_t)qi];
    tau_r = a.state[2 * (int64_t)qi + 1];
  }
  uint2* cbuf = a.cand + (size_t)(active ? qi : 0) * a.cap;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));

  // cooperative tile fetch: thread -> token tid/8, bytes (tid%8)*16 .. +16
  const int ft = tid >> 3;
  const int fb = (tid & 7) * 16;
  auto fetch = [&](int tile, u32x4& raw, float& sc) {
    const int s = tile * kTile + ft;
    if (s < a.n_tok) {
      raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.keys + (int64_t)s * kDim + fb));
      sc = a.kscale[s];
    } else {
      raw = u32x4{0, 0, 0, 0};
      sc = 0.f;
    }
  };
  auto stage = [&](int buf, const u32x4& raw, float sc) {
    const u32x2 c0 = fp8x4_to_bf16x4(raw.x);
    const u32x2 c1 = fp8x4_to_bf16x4(raw.y);
    const u32x2 c2 = fp8x4_to_bf16x4(raw.z);
    const u32x2 c3 = fp8x4_to_bf16x4(raw.w);
    u32x4* dst = reinterpret_cast<u32x4*>(&kt[buf][ft * kStride + fb]);
    dst[0] = u32x4{c0.x, c0.y, c1.x, c1.y};
    dst[1] = u32x4{c2.x, c2.y, c3.x, c3.y};
    if ((tid & 7) == 0) ksc[buf][ft] = sc;
  };
  u32x4 raw;
  float sc;
  fetch(0, raw, sc);

  bf16x8 qa[2][8];
  float wv[2][16];
  if (active) {
    const __bf16* qb = static_cast<const __bf16*>(a.q) + (int64_t)qi * kHeads * kDim;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        qa[mt][t] = *reinterpret_cast<const bf16x8*>(qb + (32 * mt + m) * kDim + 64 * h + 8 * t);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        wv[mt][r] = a.w[(int64_t)qi * kHeads + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3)];
  }
  stage(0, raw, sc);
  if (ntile > 1) fetch(1, raw, sc);
  __syncthreads();

  int32_t* idx_row = a.idx ? a.idx + (int64_t)(active ? qi : 0) * a.k : nullptr;
  // a pruning may keep a few more than k, as long as the next 8 tiles fit
  const uint32_t keep_limit = min((uint32_t)a.k + kSlack, (uint32_t)(a.cap - kCheckTiles * kTile));

  for (int tile = 0; tile < ntile; ++tile) {
    const int cur = tile & 1;
    // could the buffer fill up before the next check (64 entries per tile)?
    if (tile % kCheckTiles == 0 && active && cnt_r + kCheckTiles * kTile > (uint32_t)a.cap)
      cnt_r = wave_prune(cbuf, cnt_r, (uint32_t)a.cap, (uint32_t)a.k, keep_limit, false, whist[wave], lane, idx_row, tau_r);
    // the next tile into the other buffer (its readers passed the last
    // barrier), then the one after it from memory
    if (tile + 1 < ntile) {
      stage(cur ^ 1, raw, sc);
      if (tile + 2 < ntile) fetch(tile + 2, raw, sc);
    }
    const int s0 = a.tok0 + tile * kTile;   // position of the tile's first token
    if (active && s0 <= my_last) {
#pragma unroll
      for (int half = 0; half < kTile / 32; ++half) {
        if (s0 + 32 * half > my_last) break;
        f32x16 acc0 = {};
        f32x16 acc1 = {};
        const __bf16* krow = &kt[cur][(32 * half + m) * kStride + 64 * h];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bf16x8 kb = *reinterpret_cast<const bf16x8*>(krow + 8 * t);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][t], kb, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][t], kb, acc1, 0, 0, 0);
        }
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          part += wv[0][r] * fmaxf(acc0[r], 0.f);
          part += wv[1][r] * fmaxf(acc1[r], 0.f);
        }
        const float total = half_swap_sum(part);
        const int local = tile * kTile + 32 * half + m;
        const int pos = a.tok0 + local;
        const bool valid = h == 0 && local < a.n_tok && pos <= my_last;
        const float v = total * ksc[cur][32 * half + m];
        if (valid && a.scores) a.scores[(int64_t)qi * a.ld + pos] = v;
        // candidates: scores above the entry threshold, appended in lane order
        const uint32_t key = float_key(v);
        const bool enter = valid && key > tau_r;
        const uint64_t mk = __ballot(enter);
        if (enter) cbuf[cnt_r + (uint32_t)__popcll(mk & below)] = make_uint2(key, (uint32_t)pos);
        cnt_r += (uint32_t)__popcll(mk);
      }
    }
    __syncthreads();
  }
  if (a.final_block) {
    // the query's k best (all of its candidates when it has fewer)
    if (active) {
      uint32_t t;
      const uint32_t c = wave_prune(cbuf, cnt_r, (uint32_t)a.cap, (uint32_t)a.k, (uint32_t)a.k, true, whist[wave], lane, idx_row, t);
      if (lane == 0) a.count[qi] = (int32_t)c;
    }
  } else if (active && lane == 0) {
    a.state[2 * (int64_t)qi] = cnt_r;
    a.state[2 * (int64_t)qi + 1] = tau_r;
  }
}

}  // namespace

hipError_t launch_prefill_scan(const PrefillScanArgs& a, hipStream_t s) {
  dim3 grid((unsigned)ceil_div(a.T, kQPerWg));
  launch(prefill_scan_kernel, grid, dim3(kThreads), 0, s, "prefill_scan_kernel", a);
  return hipGetLastError();
}

}  // namespace lsi

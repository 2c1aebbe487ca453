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
// A score enters only if its key exceeds the threshold.  The threshold is
// the key of the k-th best candidate after the last compaction, a lower
// bound of the final k-th score, and a later token equal to it ranks below
// every kept candidate (ties keep the lower positions, and every later token
// has a higher position), so nothing that could still be selected is
// dropped.  Every 8 tiles the workgroup compacts the buffers that could
// overflow before the next check: an exact top-k of the buffer (key bits
// 31..20, 19..8, 7..0, then positions ascending, by LDS histograms) keeps k
// candidates and raises the threshold.  A query belongs to the same wave and
// workgroup index in every launch, so its buffer and state are never shared.
// The launch over the last block reduces each buffer to its k best and
// writes the selection.  Workspace: T x cap x 8 bytes, O(T k).
#include "lsi_internal.hpp"
#include "topk_common.hpp"

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
constexpr int kCE = 8;          // candidates per thread and batch in a compaction

// Exact top-k of the candidate buffer of query qi (n = st[0] entries, ranked
// by key descending, position ascending) by the whole workgroup.  Non-final:
// the k best stay at the front of the buffer, st = {k, key of the k-th};
// final: their positions go to idx (padded with -1) and count.  hist (4096
// words) and tmp (32 words) are LDS; st is LDS.
__device__ void compact_candidates(const PrefillScanArgs& a, int qi, uint32_t* st, uint32_t* hist,
                                   uint32_t* tmp, bool final_pass) {
  using namespace topk;
  const int tid = threadIdx.x;
  const uint32_t n = st[0];
  const uint32_t k = (uint32_t)a.k;
  uint2* buf = a.cand + (size_t)qi * a.cap;
  if (n <= k && !final_pass) return;
  // The kept set, narrowed level by level: a candidate is kept when its
  // digit at the deciding level beats the threshold bin, or it sits in every
  // threshold bin down to a level where the whole bin is kept.
  // lv 0..2: key bits [31:20], [19:8], [7:0] (descending); lv 3..5: position
  // bits [30:20], [19:9], [8:0] (ascending).
  int deciding = -1;          // level whose threshold bin is kept whole (-1: all kept)
  uint32_t bins[6] = {0, 0, 0, 0, 0, 0};
  auto digit = [](int lv, uint32_t key, uint32_t pos) -> uint32_t {
    switch (lv) {
      case 0: return key >> 20;
      case 1: return (key >> 8) & 4095u;
      case 2: return key & 255u;
      case 3: return (pos >> 20) & 2047u;
      case 4: return (pos >> 9) & 2047u;
      default: return pos & 511u;
    }
  };
  auto in_bins = [&](int upto, uint32_t key, uint32_t pos) {   // in the threshold bin of levels < upto
    for (int l = 0; l < upto; ++l)
      if (digit(l, key, pos) != bins[l]) return false;
    return true;
  };
  auto kept = [&](uint32_t key, uint32_t pos) -> bool {
    if (deciding < 0) return true;
    for (int l = 0; l <= deciding; ++l) {
      const uint32_t d = digit(l, key, pos);
      if (d != bins[l]) return l < 3 ? d > bins[l] : d < bins[l];
    }
    return true;   // in every threshold bin down to the deciding level
  };
  auto pass = [&](auto&& f) {
    for (uint32_t base = 0; base < n; base += kThreads * kCE) {
      uint2 e[kCE];
#pragma unroll
      for (int u = 0; u < kCE; ++u) {
        const uint32_t i = base + u * kThreads + tid;
        e[u] = i < n ? buf[i] : make_uint2(0u, 0xFFFFFFFFu);
      }
#pragma unroll
      for (int u = 0; u < kCE; ++u)
        if (e[u].y != 0xFFFFFFFFu) f(e[u].x, e[u].y);
    }
  };
  if (n > k) {
    uint32_t need = k;
    for (int lv = 0; lv < 6; ++lv) {
      __syncthreads();
      for (int i = tid; i < kBins; i += kThreads) hist[i] = 0u;
      __syncthreads();
      pass([&](uint32_t key, uint32_t pos) {
        if (in_bins(lv, key, pos)) atomicAdd(&hist[digit(lv, key, pos)], 1u);
      });
      __syncthreads();
      uint32_t before;
      bins[lv] = (uint32_t)find_threshold<kThreads>(hist, need, lv < 3, tmp, &before);
      const uint32_t members = hist[bins[lv]];
      need -= before;
      deciding = lv;
      if (members == need) break;   // the whole threshold bin is kept
    }
  }
  // write-back (or the selection): the kept candidates, packed in place
  // (a batch is read whole before any of it is written, and its outputs go
  // below its end); the smallest kept key becomes the new entry threshold
  if (tid == 0) tmp[30] = 0xFFFFFFFFu;
  __syncthreads();
  uint32_t out = 0;
  uint32_t kmin = 0xFFFFFFFFu;
  for (uint32_t base = 0; base < n; base += kThreads * kCE) {
    uint2 e[kCE];
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < kCE; ++u) {
      const uint32_t i = base + u * kThreads + tid;
      e[u] = i < n ? buf[i] : make_uint2(0u, 0xFFFFFFFFu);
      if (e[u].y != 0xFFFFFFFFu && kept(e[u].x, e[u].y)) m |= 1u << u;
    }
    uint32_t tot;
    uint32_t o = out + block_excl_scan<kThreads>((uint32_t)__popc(m), tmp, &tot);
#pragma unroll
    for (int u = 0; u < kCE; ++u) {
      if ((m >> u) & 1u) {
        if (final_pass) a.idx[(int64_t)qi * a.k + o] = (int32_t)e[u].y;
        else buf[o] = e[u];
        kmin = min(kmin, e[u].x);
        ++o;
      }
    }
    out += tot;
  }
  atomicMin(&tmp[30], kmin);
  __syncthreads();
  if (final_pass) {
    for (uint32_t i = out + tid; i < k; i += kThreads) a.idx[(int64_t)qi * a.k + i] = -1;
    if (tid == 0) a.count[qi] = (int32_t)out;
  } else if (tid == 0) {
    st[0] = out;
    st[1] = tmp[30];
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads, 2) void prefill_scan_kernel(PrefillScanArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 kt[2][kTile * kStride];
  __shared__ float ksc[2][kTile];
  __shared__ uint32_t hist[topk::kBins];
  __shared__ uint32_t tmp[32];
  __shared__ uint32_t qst[kQPerWg][2];    // count and entry threshold of each wave's query
  __shared__ int qflag[kQPerWg];
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

  // The workgroup compacts the buffers of its queries listed in qflag.
  auto compact_flagged = [&](bool final_pass) {
    for (int j = 0; j < kQPerWg; ++j) {
      if (qflag[j] == 0) continue;                 // uniform (LDS after a barrier)
      if (wave == j && lane == 0) {
        qst[j][0] = cnt_r;
        qst[j][1] = tau_r;
      }
      __syncthreads();
      compact_candidates(a, q0 + j, qst[j], hist, tmp, final_pass);
      if (wave == j) {
        cnt_r = qst[j][0];
        tau_r = qst[j][1];
      }
    }
  };

  for (int tile = 0; tile < ntile; ++tile) {
    const int cur = tile & 1;
    if (tile % kCheckTiles == 0) {
      // could a buffer fill up before the next check (64 entries per tile)?
      if (lane == 0) qflag[wave] = active && cnt_r + kCheckTiles * kTile > (uint32_t)a.cap;
      __syncthreads();
      compact_flagged(false);
    }
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
    // every query's k best (all of its candidates when it has fewer)
    if (lane == 0) qflag[wave] = active;
    __syncthreads();
    compact_flagged(true);
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

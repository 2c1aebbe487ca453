// Indexer scores of a prefill chunk against one block of keys (history block
// or the chunk itself), causal: query i sits at position hist_len + i and
// scores positions <= hist_len + i.  (LeanSparse episode notes: prefill
// streams a layer's history through two alternating GPU buffers; the host
// side of that lives with the C ABI, this file is the compute.)
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

__global__ __launch_bounds__(kThreads, 2) void prefill_scan_kernel(PrefillScanArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 kt[2][kTile * kStride];
  __shared__ float ksc[2][kTile];
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
  if (n_eff <= 0) return;
  const int ntile = (n_eff + kTile - 1) / kTile;
  const int my_last = active ? a.hist_len + qi : -1;   // last visible position

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
  // key range of the scores this wave writes (the row top-k's first digit
  // spans it; recording it here spares that kernel a pass over the row)
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;

  for (int tile = 0; tile < ntile; ++tile) {
    const int cur = tile & 1;
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
        if (h == 0 && local < a.n_tok && pos <= my_last) {
          const float v = total * ksc[cur][32 * half + m];
          a.scores[(int64_t)qi * a.ld + pos] = v;
          const uint32_t key = float_key(v);
          kmin = min(kmin, key);
          kmax = max(kmax, key);
        }
      }
    }
    __syncthreads();
  }
  if (a.range && active) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    }
    if (lane == 0 && kmax >= kmin) {
      atomicMax(&a.range[2 * (int64_t)qi], ~kmin);
      atomicMax(&a.range[2 * (int64_t)qi + 1], kmax);
    }
  }
}

}  // namespace

hipError_t launch_prefill_scan(const PrefillScanArgs& a, hipStream_t s) {
  dim3 grid((unsigned)ceil_div(a.T, kQPerWg));
  launch(prefill_scan_kernel, grid, dim3(kThreads), 0, s, "prefill_scan_kernel", a);
  return hipGetLastError();
}

}  // namespace lsi

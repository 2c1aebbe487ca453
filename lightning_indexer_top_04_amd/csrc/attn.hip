// Sparse attention over the selected tokens (the "Multi-layer Indexer"
// abstract: the layer attends only the k tokens its indexer kept).
//
// bf16 latent MLA (dk = 576 = 512 latent + 64 rope, dv = 512, one latent row
// shared by all heads): a workgroup owns 64 heads of one request and one slice
// of the selection, with 8 waves: wave (g4, half) owns heads 16*g4 .. +15;
// for the scores it takes tile rows 16*half .. +15, for the output it takes
// value dims 256*half .. +255, so each wave holds a 16 x 256 fp32 output (64
// registers) and two waves fit per SIMD.  Per 32-row tile the selected rows
// are gathered through the page table into LDS twice: row-major (K) and
// transposed for the first 512 columns (V^T).
//   S^T = K Q^T       v_mfma_f32_16x16x32_bf16, rows on M, heads on N
//   logits -> LDS     both waves of a head group then read all 32 rows,
//                     so each computes the same max, probabilities and sum
//   O^T += V^T P^T    16 M-tiles of 16 value dims, one K-step over 32 rows
// Softmax runs online in the log2 domain with lazy rescaling.  Splits of the
// selection are merged with their log-sum-exp by a small combine kernel.
#include "lsi_internal.hpp"

namespace lsi {
namespace {

constexpr int kD = 576;
constexpr int kDV = 512;
constexpr int kRows = 32;        // rows per tile
constexpr int kKStride = 584;    // bf16 elements per LDS row of the K tile
constexpr int kVStride = 40;     // bf16 per LDS row of the V^T tile (32 rows + pad)
constexpr int kLStride = 36;     // floats per LDS row of the logits tile
constexpr int kHeadsPerWg = 64;
constexpr int kMlaThreads = 512;
constexpr int kMaxSplitRows = 1024;  // selection rows one workgroup handles (k <= 65536 with <= 64 splits)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(kMlaThreads, 1) void mla_bf16_kernel(AttnArgs a, int rows_per_split,
                                                                  int nsplit, float* part_o,
                                                                  float* part_lse) {
  __shared__ __attribute__((aligned(16))) __bf16 Ks[kRows * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kDV * kVStride];
  __shared__ __attribute__((aligned(16))) float Lg[kHeadsPerWg * kLStride];
  __shared__ int rowidx[kRows];
  __shared__ int rows_all[kMaxSplitRows];

  const int n_hg = a.n_heads / kHeadsPerWg;
  const int bid = blockIdx.x;
  const int split = bid % nsplit;
  const int hg = (bid / nsplit) % n_hg;
  const int b = bid / (nsplit * n_hg);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = wave >> 1;          // head group of 16 inside the workgroup
  const int half = wave & 1;         // score rows / value dims half
  const int n = lane & 15;
  const int g = lane >> 4;
  const int hl = 16 * g4 + n;        // head inside the workgroup
  const int head = hg * kHeadsPerWg + hl;
  const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int r0 = split * rows_per_split;
  const int r1 = min(r0 + rows_per_split, a.k);

  // query operand: lane holds Q[head][32u + 8g .. 32u + 8g + 7]
  const __bf16* qh = static_cast<const __bf16*>(a.q) + ((int64_t)b * a.n_heads + head) * kD;
  bf16x8 qr[kD / 32];
#pragma unroll
  for (int u = 0; u < kD / 32; ++u) qr[u] = *reinterpret_cast<const bf16x8*>(qh + 32 * u + 8 * g);

  f32x4 o[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c = a.sm_scale * kLog2e;
  const __bf16* kvb = static_cast<const __bf16*>(a.kv);
  const int32_t* idxb = a.idx + (int64_t)b * a.k;

  // Physical rows of the whole slice, resolved once: given by the selection
  // (phys) or looked up through the page table.
  const int n_rows_pool = a.num_pages * a.page_size;
  for (int e = tid; e < r1 - r0; e += kMlaThreads) {
    int row = -1;
    if (a.phys) {
      row = a.phys[(int64_t)b * a.k + r0 + e];
      if (row >= n_rows_pool) row = -1;
    } else {
      const int pos = idxb[r0 + e];
      if (pos >= 0 && pos < L) {
        const int page = a.page_table[(int64_t)b * a.max_pages + pos / a.page_size];
        if ((unsigned)page < (unsigned)a.num_pages) row = page * a.page_size + pos % a.page_size;
      }
    }
    rows_all[e] = row < 0 ? -1 : row;
  }
  __syncthreads();

  // Gather of one 32-row tile into registers: thread tid owns tile row
  // tid % 32 and the 16-byte column chunks tid / 32 + 16*it (it = 0..4; the
  // fifth exists for threads below 256), so the lanes of a half-wave hold 32
  // different rows of one column and the transposed V writes spread over the
  // LDS banks.
  constexpr int kChunks = 5;
  const int my_row = tid & (kRows - 1);
  const int my_col0 = tid >> 5;                      // 0..15
  struct Pre {
    u32x4 v[kChunks];
    int row;
  };
  auto row_of = [&](int e) -> int { return e < r1 ? rows_all[e - r0] : -1; };
  auto prefetch = [&](int base) {
    Pre p;
    p.row = row_of(base + my_row);
    const __bf16* src = kvb + (int64_t)(p.row < 0 ? 0 : p.row) * kD;
#pragma unroll
    for (int it = 0; it < kChunks; ++it) {
      const int col = my_col0 + 16 * it;
      p.v[it] = (p.row >= 0 && col < kD / 8) ? *reinterpret_cast<const u32x4*>(src + col * 8)
                                              : u32x4{0, 0, 0, 0};
    }
    return p;
  };
  // two tiles in flight: the current one and the next
  Pre pa = prefetch(r0), pb = prefetch(r0 + kRows);

  for (int base = r0; base < r1; base += kRows) {
    const Pre cur = pa;
    pa = pb;
    if (tid < kRows) rowidx[tid] = cur.row;
#pragma unroll
    for (int it = 0; it < kChunks; ++it) {
      const int col = my_col0 + 16 * it;
      if (col < kD / 8) {
        const u32x4 v = cur.v[it];
        *reinterpret_cast<u32x4*>(&Ks[my_row * kKStride + col * 8]) = v;
        if (col < kDV / 8) {
          uint16_t* dst = Vt + (col * 8) * kVStride + my_row;
          dst[0 * kVStride] = (uint16_t)(v.x & 0xFFFF);
          dst[1 * kVStride] = (uint16_t)(v.x >> 16);
          dst[2 * kVStride] = (uint16_t)(v.y & 0xFFFF);
          dst[3 * kVStride] = (uint16_t)(v.y >> 16);
          dst[4 * kVStride] = (uint16_t)(v.z & 0xFFFF);
          dst[5 * kVStride] = (uint16_t)(v.z >> 16);
          dst[6 * kVStride] = (uint16_t)(v.w & 0xFFFF);
          dst[7 * kVStride] = (uint16_t)(v.w >> 16);
        }
      }
    }
    __syncthreads();
    pb = prefetch(base + 2 * kRows);

    // S^T for tile rows 16*half .. +15, this wave's 16 heads
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    const __bf16* krow = &Ks[(16 * half + n) * kKStride + 8 * g];
#pragma unroll
    for (int u = 0; u < kD / 32; ++u) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(krow + 32 * u);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qr[u], sacc, 0, 0, 0);
    }
    // logits of rows 16*half + 4g + r for head hl -> LDS
    {
      f32x4 xl;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        xl[r] = rowidx[16 * half + 4 * g + r] >= 0 ? sacc[r] * c : -INFINITY;
      *reinterpret_cast<f32x4*>(&Lg[hl * kLStride + 16 * half + 4 * g]) = xl;
    }
    __syncthreads();
    // every wave of the head group reads rows 8g .. 8g+7 of its heads
    float x[8];
    {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(&Lg[hl * kLStride + 8 * g]);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(&Lg[hl * kLStride + 8 * g + 4]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = x0[r];
        x[4 + r] = x1[r];
      }
    }
    float tmax = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, x[i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // Lazy rescaling: the reference max only moves when the tile max exceeds
    // it by more than 8 (log2 units); probabilities then stay below 2^8.
    const bool first = m_run == -INFINITY;
    const float m_new = (first || tmax > m_run + 8.f) ? fmaxf(m_run, tmax) : m_run;
    float p[8];
    float alpha = 1.f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = 0.f;
    } else {
      if (!first) alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = exp2f(x[i] - m_new);
    }
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) psum += p[i];
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int j = 0; j < 16; ++j) o[j] *= alpha;
    }
    const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7])};
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
    // O^T[dims 256*half + 16j + ..][head] += V^T P^T over the 32 rows
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bf16x8 av =
          *reinterpret_cast<const bf16x8*>(&Vt[(256 * half + 16 * j + n) * kVStride + 8 * g]);
      o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, o[j], 0, 0, 0);
    }
    __syncthreads();
  }

  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse2 = l_run > 0.f ? m_run + log2f(l_run) : -INFINITY;
  const int64_t bh = (int64_t)b * a.n_heads + head;
  // lane holds O[head][256*half + 16j + 4g + r]
  if (nsplit == 1) {
    __bf16* ob = static_cast<__bf16*>(a.out) + bh * kDV + 256 * half;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      u32x2 w2 = {pack_bf16x2(o[j][0] * inv, o[j][1] * inv), pack_bf16x2(o[j][2] * inv, o[j][3] * inv)};
      *reinterpret_cast<u32x2*>(ob + 16 * j + 4 * g) = w2;
    }
    if (g == 0 && half == 0) a.lse[bh] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  } else {
    float* po = part_o + (bh * nsplit + split) * kDV + 256 * half;
#pragma unroll
    for (int j = 0; j < 16; ++j) *reinterpret_cast<f32x4*>(po + 16 * j + 4 * g) = o[j] * inv;
    if (g == 0 && half == 0) part_lse[bh * nsplit + split] = lse2;
  }
}

// Merge split partials: out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M).
// One workgroup of 128 threads per (request, head), 4 value dims per thread.
__global__ __launch_bounds__(128) void mla_combine_kernel(AttnArgs a, int nsplit,
                                                           const float* part_o,
                                                           const float* part_lse) {
  constexpr int kMaxSplit = 64;
  __shared__ float wts[kMaxSplit];
  __shared__ float stat[2];
  const int64_t bh = blockIdx.x;
  const float* pl = part_lse + bh * nsplit;
  if (threadIdx.x < 64) {
    const float ls = threadIdx.x < nsplit ? pl[threadIdx.x] : -INFINITY;
    float M = ls;
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float wgt = (M == -INFINITY || ls == -INFINITY) ? 0.f : exp2f(ls - M);
    float sum = wgt;
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    if (threadIdx.x < kMaxSplit) wts[threadIdx.x] = wgt;
    if (threadIdx.x == 0) {
      stat[0] = M;
      stat[1] = sum;
    }
  }
  __syncthreads();
  const float M = stat[0];
  const float wsum = stat[1];
  const int d0 = threadIdx.x * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part_o + (bh * nsplit + s) * kDV + d0);
    acc += wts[s] * v;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  __bf16* ob = static_cast<__bf16*>(a.out) + bh * kDV;
  u32x2 w2 = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  *reinterpret_cast<u32x2*>(ob + d0) = w2;
  if (threadIdx.x == 0) a.lse[bh] = wsum > 0.f ? (M + log2f(wsum)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// fp32 generic path: separate K and V caches, one K/V head, any head count.
// One workgroup per (request, head); rows in blocks of 256, online softmax.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  extern __shared__ float sm[];
  float* qs = sm;                    // [dk]
  float* ps = sm + a.dk;             // [256]
  int* rows = reinterpret_cast<int*>(ps + 256);   // [256]
  float* red = reinterpret_cast<float*>(rows + 256);  // [8]
  const int head = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t bh = (int64_t)b * a.n_heads + head;
  const float* qg = static_cast<const float*>(a.q) + bh * a.dk;
  for (int i = tid; i < a.dk; i += 256) qs[i] = qg[i];
  __syncthreads();
  const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const float* K = static_cast<const float*>(a.kv);
  const float* V = static_cast<const float*>(a.v);
  float m_run = -INFINITY, l_run = 0.f, o = 0.f;
  for (int base = 0; base < a.k; base += 256) {
    const int e = base + tid;
    int row = -1;
    if (e < a.k) {
      const int pos = a.idx[(int64_t)b * a.k + e];
      if (pos >= 0 && pos < L) {
        const int page = a.page_table[(int64_t)b * a.max_pages + pos / a.page_size];
        if ((unsigned)page < (unsigned)a.num_pages) row = page * a.page_size + pos % a.page_size;
      }
    }
    float logit = -INFINITY;
    if (row >= 0) {
      const float* kr = K + (int64_t)row * a.dk;
      float dot = 0.f;
      for (int i = 0; i < a.dk; ++i) dot = fmaf(qs[i], kr[i], dot);
      logit = dot * a.sm_scale;
    }
    rows[tid] = row;
    float mx = wave_max(logit);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float m_new = fmaxf(m_run, mx);
    float p = 0.f, alpha = 1.f;
    if (m_new != -INFINITY) {
      alpha = expf(m_run - m_new);
      p = row >= 0 ? expf(logit - m_new) : 0.f;
    }
    ps[tid] = p;
    float sum = wave_sum(p);
    __syncthreads();
    if (lane == 0) red[4 + wave] = sum;
    __syncthreads();
    sum = red[4] + red[5] + red[6] + red[7];
    l_run = l_run * alpha + sum;
    m_run = m_new;
    if (tid < a.dv) {
      o *= alpha;
      for (int r = 0; r < 256; ++r) {
        const int rw = rows[r];
        if (rw >= 0) o = fmaf(ps[r], V[(int64_t)rw * a.dv + tid], o);
      }
    }
    __syncthreads();
  }
  if (tid < a.dv) static_cast<float*>(a.out)[bh * a.dv + tid] = l_run > 0.f ? o / l_run : 0.f;
  if (tid == 0) a.lse[bh] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

int pick_nsplit(int num_req, int n_heads, int k) {
  const int groups = num_req * (n_heads / kHeadsPerWg);
  const int tiles = (k + kRows - 1) / kRows;
  // ~2 workgroups per CU, at least 4 tiles per split
  int ns = (int)ceil_div((int64_t)num_cus() * 2, std::max(groups, 1));
  ns = std::min(ns, std::max(1, tiles / 2));
  ns = std::max(ns, (int)ceil_div(tiles, kMaxSplitRows / kRows));
  return std::min(std::max(ns, 1), 64);
}

}  // namespace

size_t mla_ws_bytes(int num_req, int n_heads, int dv, int k) {
  const int ns = pick_nsplit(num_req, n_heads, k);
  if (ns == 1) return 0;
  return align_up((size_t)num_req * n_heads * ns * (dv + 1) * sizeof(float), 256);
}

hipError_t launch_mla_bf16(const AttnArgs& a, hipStream_t s) {
  const int ns = pick_nsplit(a.num_req, a.n_heads, a.k);
  const int tiles = (a.k + kRows - 1) / kRows;
  const int rows_per_split = (int)ceil_div(tiles, ns) * kRows;
  const int nsplit = (int)ceil_div(a.k, rows_per_split);
  float* part_o = static_cast<float*>(a.ws);
  float* part_lse = part_o ? part_o + (size_t)a.num_req * a.n_heads * nsplit * kDV : nullptr;
  const int grid = a.num_req * (a.n_heads / kHeadsPerWg) * nsplit;
  hipLaunchKernelGGL(mla_bf16_kernel, dim3(grid), dim3(kMlaThreads), 0, s, a, rows_per_split, nsplit,
                     part_o, part_lse);
  if (nsplit > 1)
    hipLaunchKernelGGL(mla_combine_kernel, dim3(a.num_req * a.n_heads), dim3(kDV / 4), 0, s, a,
                       nsplit, part_o, part_lse);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  const size_t smem = sizeof(float) * (a.dk + 256 + 256 + 8);
  hipLaunchKernelGGL(attn_f32_kernel, dim3(a.n_heads, a.num_req), dim3(256), smem, s, a);
  return hipGetLastError();
}

}  // namespace lsi

// Sparse attention over the selected tokens (the "Multi-layer Indexer"
// abstract: the layer attends only the k tokens its indexer kept).
//
// bf16 latent MLA (dk = 576 = 512 latent + 64 rope, dv = 512, one latent row
// shared by all heads).  A workgroup of 4 waves owns 16 heads of one request
// and one slice of the selection, taken in blocks of 64 rows:
//   gather    the block's rows go from the pool straight into LDS by DMA
//             (global_load_lds_dwordx4): one 1 KB instruction per row for the
//             512 latent dims, one per 8 rows for the 64 rope dims.  Chunk c
//             (16 bytes) of row r is stored at position c ^ (r % 16) (rope:
//             c ^ (r % 8)), so the MFMA-layout reads below hit distinct banks.
//   S^T = K Q^T        v_mfma_f32_16x16x32_bf16, wave w takes rows 16w..+15
//                      (M), the 16 heads on N, the query in registers
//   softmax            online over blocks in the log2 domain; block max and
//                      sum per head are exchanged through LDS
//   O = P V            wave w takes value dims 128w..+127: P (bf16) from LDS,
//                      V read with ds_read_b64_tr_b16, which hands each lane
//                      four rows of one value dim straight from the row-major
//                      rows in LDS
// Every LDS operand of a block is read before the block's first MFMA (an
// MFMA waiting on its own read pays the LDS latency once per MFMA).
// The workgroups of one slice (all head groups) are given block ids that are
// equal modulo 8, so they run on one XCD and share its L2 for the rows.
// Splits of the selection are merged with their log-sum-exp by a small
// combine kernel, from bf16 partials of the normalised outputs.
#include "lsi_internal.hpp"
#include "topk_common.hpp"

namespace lsi {
namespace {

constexpr int kD = 576;
constexpr int kDV = 512;
constexpr int kMH = 16;                       // heads per workgroup
constexpr int kMBlk = 64;                     // selection rows per block
constexpr int kMThreads = 256;
constexpr int kVRow = 1024;                   // LDS bytes of a row's 512 latent dims
constexpr int kRopeOff = kMBlk * kVRow;       // rope dims: 8 rows per 1 KB
constexpr int kKvBytes = kRopeOff + kMBlk * 128;
constexpr int kPStride = 72;                  // bf16 per LDS row of P (64 rows + pad)
constexpr int kMaxSplitRows = 1024;           // selection rows one workgroup handles
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(4))) short s16x4;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int OFF>
__device__ __forceinline__ void dma_row16(uint8_t* lds, const uint8_t* g) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, OFF, 0);
}

// Max and sum over the four 16-lane rows of the wave (lanes n, n+16, n+32,
// n+48) with the row-swap permutes: two VALU swaps instead of two LDS
// round trips of a shuffle.
__device__ __forceinline__ float max4rows(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum4rows(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS reads and
// writes, not for its block DMAs still in flight (__syncthreads would).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
// Nine 16-byte LDS reads (half a row tile of S), complete when the statement
// ends.  Written out so that the compiler, which cannot tell these rows from
// a block DMA still in flight into the other buffer, does not wait for that
// DMA first.
__device__ __forceinline__ void lds_read_b128x9(u32x4* o, const uint32_t* ad) {
  asm volatile(
      "ds_read_b128 %0, %9\n\t"
      "ds_read_b128 %1, %10\n\t"
      "ds_read_b128 %2, %11\n\t"
      "ds_read_b128 %3, %12\n\t"
      "ds_read_b128 %4, %13\n\t"
      "ds_read_b128 %5, %14\n\t"
      "ds_read_b128 %6, %15\n\t"
      "ds_read_b128 %7, %16\n\t"
      "ds_read_b128 %8, %17\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]),
        "=&v"(o[7]), "=&v"(o[8])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]),
        "v"(ad[8])
      : "memory");
}
// One 8-byte LDS write (same reason); the next barrier waits for it.
__device__ __forceinline__ void lds_write_b64(uint32_t a, u32x2 v) {
  asm volatile("ds_write_b64 %0, %1" : : "v"(a), "v"(v) : "memory");
}
// Two 16-byte and eight transposing 8-byte LDS reads, complete when the
// statement ends (same reason as above).
__device__ __forceinline__ void lds_read_p2_tr8(u32x4 (&p)[2], s16x4 (&o)[8], uint32_t pa0, uint32_t pa1,
                                                const uint32_t (&ad)[8]) {
  asm volatile(
      "ds_read_b128 %0, %10\n\t"
      "ds_read_b128 %1, %11\n\t"
      "ds_read_b64_tr_b16 %2, %12\n\t"
      "ds_read_b64_tr_b16 %3, %13\n\t"
      "ds_read_b64_tr_b16 %4, %14\n\t"
      "ds_read_b64_tr_b16 %5, %15\n\t"
      "ds_read_b64_tr_b16 %6, %16\n\t"
      "ds_read_b64_tr_b16 %7, %17\n\t"
      "ds_read_b64_tr_b16 %8, %18\n\t"
      "ds_read_b64_tr_b16 %9, %19\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(p[0]), "=&v"(p[1]), "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]),
        "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(pa0), "v"(pa1), "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]),
        "v"(ad[6]), "v"(ad[7])
      : "memory");
}
// LDS transpose read: within each 16-lane group, lane 4a + c receives element
// c of the 8-byte chunks addressed by lanes a, a + 4, a + 8 and a + 12.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<uint8_t*>(p)));
}

__global__ __launch_bounds__(kMThreads, 1) void mla_bf16_kernel(AttnArgs a, int rows_per_split,
                                                                int nsplit, int units, __bf16* part_o,
                                                                float* part_lse) {
  __shared__ __attribute__((aligned(1024))) uint8_t kvs[kKvBytes];
  __shared__ __attribute__((aligned(16))) __bf16 Pl[kMH * kPStride];
  __shared__ float red_m[4][kMH];
  __shared__ float red_l[4][kMH];
  __shared__ float alpha_s[kMH];
  __shared__ __attribute__((aligned(16))) int rows_all[kMaxSplitRows];
  // the 16 heads' query rows (16 x 1152 bytes), moved in once per workgroup:
  // chunk j (16 bytes) of head n at position 72 n + ((j & ~7) | ((j ^ n) & 7)),
  // so that the 16 heads' reads of one chunk spread over the banks
  __shared__ __attribute__((aligned(1024))) uint8_t qlds[kMH * kD * 2];
  __shared__ uint32_t rtmp[32];

  // Block ids map to XCDs round-robin (bid % 8).  Every head group of one
  // (request, slice) unit runs on the XCD of that unit, so each selected row
  // is fetched from memory into one L2 and read there by the 8 head groups;
  // the partials, 16 KB of bf16 per workgroup, are what crosses XCDs instead
  // (written through to memory, sc1).
  if (a.zero_ptr) {
    // clear the scan-built histograms the selection has read (they must be
    // zero when the next scan starts)
    const int64_t nthreads = (int64_t)gridDim.x * kMThreads;
    for (int64_t i = (int64_t)blockIdx.x * kMThreads + threadIdx.x; i < a.zero_words; i += nthreads)
      a.zero_ptr[i] = 0u;
  }
  const int n_hg = a.n_heads / kMH;
  const int bid = blockIdx.x;
  // unit u = (request, split) on XCD u % 8 with all its head groups
  const int u = (bid / (8 * n_hg)) * 8 + (bid & 7);
  const int hg = (bid >> 3) % n_hg;
  if (u >= units) return;
  const int b = u / nsplit;
  const int split = u % nsplit;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  // The 16 heads' query rows go into qlds by DMA first (18 DMAs of 1 KB;
  // wave w issues numbers w, w + 4, ...): they arrive with the row ids, and
  // the waves read them into registers while the first block's rows are on
  // their way, so that S reads only the rows from LDS.
  const uint8_t* qg = reinterpret_cast<const uint8_t*>(static_cast<const __bf16*>(a.q) +
                                                       ((int64_t)b * a.n_heads + hg * kMH) * kD);
  for (int i = w; i < kMH * kD * 2 / 1024; i += 4) {
    const int p = 64 * i + lane;                        // 16-byte position in qlds
    const int hn = p / 72, jj = p - 72 * hn;
    const int j = (jj & ~7) | ((jj ^ hn) & 7);          // global chunk stored there
    dma_row16<0>(qlds + 1024 * i, qg + hn * (kD * 2) + 16 * j);
  }
  const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int r0 = split * rows_per_split;
  const int r1 = min(r0 + rows_per_split, a.k);
  const int nr = max(0, r1 - r0);

  // physical rows of the slice, resolved once (given by the selection, or
  // looked up through the page table); -1 = skip
  constexpr int kRowsPerThread = kMaxSplitRows / kMThreads;
  const int n_rows_pool = a.num_pages * a.page_size;
  // a deferred selection's record (count above the threshold bin, members),
  // loaded by the last thread together with the row ids (one round trip for
  // both; a load by one lane is not made uniform and waited for at once)
  // and handed over through LDS
  uint32_t rec_v[2] = {0u, 0u};
  if (a.tk_ws != nullptr && tid == kMThreads - 1) {
    const uint32_t* rec = topk::carve(a.tk_ws, a.num_req, a.tk_max_len).rec + (size_t)b * 4;
    rec_v[0] = rec[1];
    rec_v[1] = rec[2];
  }
  int prow[kRowsPerThread];
  if (a.phys) {
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const int e = tid + i * kMThreads;
      prow[i] = e < nr ? a.phys[(int64_t)b * a.k + r0 + e] : -1;
    }
  } else {
    // every position load first, then every page-table load (at clamped,
    // in-bounds indexes, masked afterwards): two round trips, where loads
    // under per-element conditions were issued and waited for one by one
    int pos[kRowsPerThread], pg[kRowsPerThread];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const int e = tid + i * kMThreads;
      pos[i] = a.idx[(int64_t)b * a.k + min(r0 + min(e, max(nr - 1, 0)), a.k - 1)];
    }
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const int e = tid + i * kMThreads;
      if (e >= nr || pos[i] < 0 || pos[i] >= L) pos[i] = -1;
      pg[i] = a.page_table[(int64_t)b * a.max_pages + (pos[i] >= 0 ? pos[i] / a.page_size : 0)];
    }
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i)
      prow[i] = pos[i] >= 0 && (unsigned)pg[i] < (unsigned)a.num_pages ? pg[i] * a.page_size + pos[i] % a.page_size : -1;
  }
  bool unresolved = false;
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int e = tid + i * kMThreads;
    if (e < nr) rows_all[e] = (prow[i] < 0 || prow[i] >= n_rows_pool) ? -1 : prow[i];
    unresolved |= e < nr && prow[i] == kUnresolvedRow;
  }
  if (tid == kMThreads - 1) {
    rtmp[30] = rec_v[0];
    rtmp[31] = rec_v[1];
  }
  if (a.tk_ws != nullptr && __syncthreads_or(unresolved)) {
    // Part of this slice lies in a threshold bin that the top-k left open:
    // work out the kept members (every workgroup that needs them reaches the
    // same set and order) and take the rows of this slice's slots.  The
    // block buffer is free until the gather below.
    const topk::Ws tw = topk::carve(a.tk_ws, a.num_req, a.tk_max_len);
    const uint32_t rec_better = rtmp[30], rec_members = rtmp[31];
    lds_barrier();   // rtmp is the resolve's scratch from here on
    topk::resolve_members<kMThreads>(tw, b, a.tk_max_len, a.k, rec_better, rec_members,
                                     reinterpret_cast<uint32_t*>(kvs), rtmp, r0, r1,
                                     [&](int slot, int pos, int row) {
                                       rows_all[slot - r0] = (row < 0 || row >= n_rows_pool) ? -1 : row;
                                       if (hg == 0) {
                                         a.idx_out[(int64_t)b * a.k + slot] = pos;
                                         if (a.phys_out) a.phys_out[(int64_t)b * a.k + slot] = row;
                                       }
                                     });
  }
  // every wave's query DMAs have landed (vmcnt counts loads to LDS) before
  // the barrier after which any wave reads qlds
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // query operand of S^T = K Q^T: lane (n, g) holds Q[head n][32t + 8g .. +7]
  // (one DMA of the group's rows per workgroup instead of a load per wave,
  // which doubled the gather's L2 requests)
  bf16x8 qr[kD / 32];

  const uint8_t* kvb = static_cast<const uint8_t*>(a.kv);
  const float c = a.sm_scale * kLog2e;
  f32x4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // per head n (S layout), the same in every wave
  float l_run = 0.f;

  for (int base = 0; base < nr; base += kMBlk) {
    const int nb = min(kMBlk, nr - base);
    // ---- gather: wave w moves rows 16w .. 16w+15 of the block
    {
      const int rl = 16 * w + (lane & 15);
      const int myrow = rl < nb ? rows_all[base + rl] : -1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rw = __builtin_amdgcn_readlane(myrow, i);
        const uint8_t* src = kvb + (int64_t)(rw < 0 ? 0 : rw) * (kD * 2) + 16 * (lane ^ ((16 * w + i) & 15));
        dma_row16<0>(kvs + (16 * w + i) * kVRow, src);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int rr = 8 * t + (lane >> 3);                 // row inside the wave's 16
        const int rw = __shfl(myrow, rr);
        const int p = lane & 7;
        const uint8_t* src = kvb + (int64_t)(rw < 0 ? 0 : rw) * (kD * 2) + 2 * kDV + 16 * (p ^ (rr & 7));
        dma_row16<0>(kvs + kRopeOff + (2 * w + t) * 1024, src);
      }
    }
    if (base == 0) {
      // the query rows landed before the barrier above: read them while this
      // block's rows are on their way
#pragma unroll
      for (int t = 0; t < kD / 32; ++t) {
        const int j = 4 * t + g;
        qr[t] = *reinterpret_cast<const bf16x8*>(qlds + 16 * (72 * n + ((j & ~7) | ((j ^ n) & 7))));
      }
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // ---- S^T for rows 16w + (0..15): A = K rows from LDS, B = Q^T.  Every
    // LDS read is issued before the first MFMA (an MFMA waiting on its own
    // read pays the LDS latency 18 times), two accumulators halve the chain.
    f32x4 sacc;
    {
      const int row = 16 * w + n;                  // A-operand row of this lane
      const uint8_t* vrow = kvs + row * kVRow;
      const uint8_t* rrow = kvs + kRopeOff + (row >> 3) * 1024 + (row & 7) * 128;
      bf16x8 av[kD / 32];
#pragma unroll
      for (int t = 0; t < kD / 32; ++t) {
        if (t < 16) {
          av[t] = *reinterpret_cast<const bf16x8*>(vrow + 16 * ((4 * t + g) ^ (row & 15)));
        } else {
          av[t] = *reinterpret_cast<const bf16x8*>(rrow + 16 * ((4 * (t - 16) + g) ^ (row & 7)));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < kD / 32; t += 2) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[t], qr[t], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[t + 1], qr[t + 1], s1, 0, 0, 0);
      }
      sacc = s0 + s1;
    }
    // lane (n, g) holds S^T[row 16w + 4g + r][head n]
    float x[4];
    {
      const int4 rv = *reinterpret_cast<const int4*>(&rows_all[base + 16 * w + 4 * g]);
      const int rr[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = 16 * w + 4 * g + r < nb && rr[r] >= 0;
        x[r] = ok ? sacc[r] * c : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = max4rows(mx);
    if (g == 0) red_m[w][n] = mx;
    __syncthreads();
    const float bmax = fmaxf(fmaxf(red_m[0][n], red_m[1][n]), fmaxf(red_m[2][n], red_m[3][n]));
    // Lazy rescaling: the reference max only moves when the block max exceeds
    // it by more than 8 (log2 units); probabilities then stay below 2^8.
    const bool first = m_run == -INFINITY;
    const float m_new = (first || bmax > m_run + 8.f) ? fmaxf(m_run, bmax) : m_run;
    const float alpha = (first || m_new == m_run) ? (first ? 0.f : 1.f) : exp2f(m_run - m_new);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = m_new == -INFINITY ? 0.f : exp2f(x[r] - m_new);
    float ps = (p[0] + p[1]) + (p[2] + p[3]);
    ps = sum4rows(ps);
    if (g == 0) red_l[w][n] = ps;
    {
      const u32x2 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      *reinterpret_cast<u32x2*>(&Pl[n * kPStride + 16 * w + 4 * g]) = pw;
    }
    if (w == 0 && g == 0) alpha_s[n] = alpha;
    __syncthreads();
    l_run = l_run * (first ? 0.f : alpha) + ((red_l[0][n] + red_l[1][n]) + (red_l[2][n] + red_l[3][n]));
    m_run = m_new;

    // ---- O[heads][dims 128w ..] += P V; lane (dim n, g) holds heads 4g + r
    {
      f32x4 al;
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] = alpha_s[4 * g + r];
      if (al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f) {
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t] *= al;
      }
    }
    const int s16 = lane & 15;                 // source lane of the transpose reads
    const int ja = s16 >> 2;                   // row offset within the group of 4
    const int aa = s16 & 3;                    // 4-dim column group
    {
      // all LDS reads of the block first, then the 16 MFMAs
      bf16x8 pa[2];
      s16x4 v0[2][8], v1[2][8];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        pa[kk] = *reinterpret_cast<const bf16x8*>(&Pl[n * kPStride + 32 * kk + 8 * g]);
        const int ra = 32 * kk + 8 * g + ja;     // rows ra and ra + 4
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int ch = (128 * w + 16 * t + 4 * aa) >> 3;    // 16-byte chunk of the dim group
          const int hb = 8 * (aa & 1);
          v0[kk][t] = lds_read_tr16(kvs + ra * kVRow + 16 * (ch ^ (ra & 15)) + hb);
          v1[kk][t] = lds_read_tr16(kvs + (ra + 4) * kVRow + 16 * (ch ^ ((ra + 4) & 15)) + hb);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const short vv[8] = {v0[kk][t][0], v0[kk][t][1], v0[kk][t][2], v0[kk][t][3],
                               v1[kk][t][0], v1[kk][t][1], v1[kk][t][2], v1[kk][t][3]};
          bf16x8 vb;
#pragma unroll
          for (int e = 0; e < 8; ++e) vb[e] = __builtin_bit_cast(__bf16, vv[e]);
          o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[kk], vb, o[t], 0, 0, 0);
        }
      }
    }
    __syncthreads();   // the block's LDS is refilled next
  }

  // ---- results: the per-head statistics (every wave holds head n's in
  // lanes n, n + 16, ...) moved to the output layout by lane shuffles
  const int dim0 = 128 * w + n;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hl = 4 * g + r;
    const float lr = __shfl(l_run, hl);
    const float mr = __shfl(m_run, hl);
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    const float lse2 = lr > 0.f ? mr + log2f(lr) : -INFINITY;
    const int64_t bh = (int64_t)b * a.n_heads + hg * kMH + hl;
    if (nsplit == 1) {
      __bf16* ob = static_cast<__bf16*>(a.out) + bh * kDV + dim0;
#pragma unroll
      for (int t = 0; t < 8; ++t) ob[16 * t] = (__bf16)(o[t][r] * inv);
      if (w == 0 && n == 0) a.lse[bh] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
    } else {
      // bf16 partial, dims in lane order (dim 128w + 16t + n at 128w + 8n + t):
      // one 16-byte store per head, written through to memory for the
      // combine, which reads it from another XCD
      u32x4 v;
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = pack_bf16x2(o[2 * t][r] * inv, o[2 * t + 1][r] * inv);
      __bf16* po = part_o + (bh * nsplit + split) * kDV + 128 * w + 8 * n;
      asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(po), "v"(v) : "memory");
      if (w == 0 && n == 0) part_lse[bh * nsplit + split] = lse2;
    }
  }
}

// ---------------------------------------------------------------------------
// Batches: 32 heads per workgroup of 8 waves, one workgroup per CU, the next
// 64-row block gathered while the current one is computed.  Half the head
// groups of the 16-head kernel, so each selected row is moved into LDS half
// as often, and the gather latency hides behind compute instead of behind a
// second workgroup.  Wave w = (rt, ht) computes S^T for rows 16rt..+15 and
// heads 16ht..+15 of the group (its query tile in registers); the softmax of
// a head meets the four row tiles through LDS; for O = P V wave w owns value
// dims 64w..+63 of all 32 heads.
// ---------------------------------------------------------------------------
constexpr int kWH = 32;                       // heads per workgroup
constexpr int kWThreads = 512;
constexpr int kWMaxRows = 2048;               // selection rows one workgroup handles
constexpr int kWDmaPerBlock = 9;              // DMA instructions per wave per block
                                              // (the vmcnt(9) waits below)
static_assert(kWDmaPerBlock == kMBlk / (kWThreads / 64) + 1, "a DMA per row of the wave, one for their rope dims");

__global__ __launch_bounds__(kWThreads, 1) void mla_bf16_wide_kernel(AttnArgs a, int rows_per_split,
                                                                    int nsplit, int units, float* part_o,
                                                                    float* part_lse) {
  __shared__ __attribute__((aligned(1024))) uint8_t kvs0[kKvBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t kvs1[kKvBytes];
  __shared__ __attribute__((aligned(16))) __bf16 Pl[kWH * kPStride];
  __shared__ __attribute__((aligned(16))) float red_m[kWH][4];   // [head][row tile]
  __shared__ __attribute__((aligned(16))) float red_l[kWH][4];
  __shared__ __attribute__((aligned(16))) int rows_all[kWMaxRows];

  const int n_hg = a.n_heads / kWH;
  const int bid = blockIdx.x;
  const int u = (bid / (8 * n_hg)) * 8 + (bid & 7);
  const int hg = (bid >> 3) % n_hg;
  if (u >= units) return;
  const int b = u / nsplit;
  const int split = u % nsplit;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = w & 3;                        // row tile of S
  const int ht = w >> 2;                       // head tile of S
  const int n = lane & 15;
  const int g = lane >> 4;
  const int hh = 16 * ht + n;                  // this lane's head (S layout) within the group
  const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int r0 = split * rows_per_split;
  const int r1 = min(r0 + rows_per_split, a.k);
  const int nr = max(0, r1 - r0);

  // query operand of S^T = K Q^T: lane (n, g) holds Q[head][32t + 8g .. +7]
  const __bf16* qh = static_cast<const __bf16*>(a.q) + ((int64_t)b * a.n_heads + hg * kWH + hh) * kD;
  bf16x8 qr[kD / 32];
#pragma unroll
  for (int t = 0; t < kD / 32; ++t) qr[t] = *reinterpret_cast<const bf16x8*>(qh + 32 * t + 8 * g);
  // physical rows of the slice (-1 = skip): every id load of the thread is
  // issued before the first is used (then the page-table loads), so the
  // slice costs one or two round trips, not one per 512 rows
  const int n_rows_pool = a.num_pages * a.page_size;
  {
    constexpr int kPer = kWMaxRows / kWThreads;
    int v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid + i * kWThreads;
      v[i] = e < nr ? (a.phys ? a.phys[(int64_t)b * a.k + r0 + e] : a.idx[(int64_t)b * a.k + r0 + e]) : -1;
    }
    if (!a.phys) {
      int pg[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const bool in = v[i] >= 0 && v[i] < L;
        pg[i] = a.page_table[(int64_t)b * a.max_pages + (in ? v[i] / a.page_size : 0)];
        pg[i] = in ? pg[i] : -1;
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        v[i] = (unsigned)pg[i] < (unsigned)a.num_pages ? pg[i] * a.page_size + v[i] % a.page_size : -1;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid + i * kWThreads;
      if (e < nr) rows_all[e] = (v[i] < 0 || v[i] >= n_rows_pool) ? -1 : v[i];
    }
  }
  // the query and row loads are complete here (ordinary loads are not left
  // in flight under the block DMAs, whose waits are counted by hand below)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  const uint8_t* kvb = static_cast<const uint8_t*>(a.kv);
  // wave w moves rows 8w..8w+7 of a block: one 1 KB DMA per row for the
  // latent dims (chunk c of row r at c ^ (r % 16)), one for their rope dims
  // (c ^ (r % 8)) -- kWDmaPerBlock instructions, every wave, every block
  auto gather = [&](int blk, uint8_t* buf) {
    const int base = blk * kMBlk;
    const int nb = min(kMBlk, nr - base);
    const int rl = 8 * w + (lane & 7);
    const int myrow = rl < nb ? rows_all[base + rl] : -1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rw = __builtin_amdgcn_readlane(myrow, i);
      const uint8_t* src = kvb + (int64_t)(rw < 0 ? 0 : rw) * (kD * 2) + 16 * (lane ^ ((8 * w + i) & 15));
      dma_row16<0>(buf + (8 * w + i) * kVRow, src);
    }
    const int rr = lane >> 3;
    const int rw = __shfl(myrow, rr);
    const uint8_t* src = kvb + (int64_t)(rw < 0 ? 0 : rw) * (kD * 2) + 2 * kDV + 16 * ((lane & 7) ^ rr);
    dma_row16<0>(buf + kRopeOff + w * 1024, src);
  };

  const float c = a.sm_scale * kLog2e;
  f32x4 o[2][4];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int t = 0; t < 4; ++t) o[h2][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Running maxima (log2 units).  Every wave holds the same values: for head
  // hh (its S tile), for head lane % 32 (the vote below) and for the heads
  // 16 h2 + 4 g + r of its O rows.  A head's running maximum moves only when
  // a block's maximum passes it by more than 8 (the first finite score
  // always does); until then the block's P is taken against the old value,
  // at most 2^8, so most blocks need no exchange of maxima before P.
  float m_s = -INFINITY;
  float m_v = -INFINITY;
  float m_o[2][4];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int r = 0; r < 4; ++r) m_o[h2][r] = -INFINITY;
  float l_w = 0.f;   // this wave's rows' share of the softmax sum of head hh
  auto bump = [](float m, float bm) { return bm > m + 8.f ? fmaxf(m, bm) : m; };
  auto hmax = [&](int head) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(&red_m[head][0]);
    return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
  };

  const int nblk = (nr + kMBlk - 1) / kMBlk;
  auto step = [&](int blk, const uint8_t* kv, uint8_t* next) {
    const int base = blk * kMBlk;
    const int nb = min(kMBlk, nr - base);
    // the next block goes out first; then this block's DMAs (the ones before
    // the last kWDmaPerBlock) must have landed, in every wave
    if (blk + 1 < nblk) {
      gather(blk + 1, next);
      asm volatile("s_waitcnt vmcnt(9)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    // ---- S^T for rows 16rt + (0..15) and heads 16ht + (0..15), nine reads
    // at a time
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    {
      const int row = 16 * rt + n;
      const uint32_t vrow = lds_addr(kv) + row * kVRow;
      const uint32_t rrow = lds_addr(kv) + kRopeOff + (row >> 3) * 1024 + (row & 7) * 128;
      uint32_t ad[kD / 32];
#pragma unroll
      for (int t = 0; t < kD / 32; ++t)
        ad[t] = t < 16 ? vrow + 16 * ((4 * t + g) ^ (row & 15)) : rrow + 16 * ((4 * (t - 16) + g) ^ (row & 7));
#pragma unroll
      for (int t0 = 0; t0 < kD / 32; t0 += 9) {
        u32x4 av[9];
        lds_read_b128x9(av, ad + t0);
#pragma unroll
        for (int i = 0; i < 9; ++i)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[i]), qr[t0 + i], sacc, 0, 0, 0);
      }
    }
    // lane (n, g) holds S^T[row 16rt + 4g + r][head hh]; the four rows'
    // physical ids in one read
    const int4 rv = *reinterpret_cast<const int4*>(&rows_all[base + 16 * rt + 4 * g]);
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = 16 * rt + 4 * g + r;
      const int id = r == 0 ? rv.x : r == 1 ? rv.y : r == 2 ? rv.z : rv.w;
      x[r] = rl < nb && id >= 0 ? sacc[r] * c : -INFINITY;
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = max4rows(mx);
    auto write_p = [&](float m, float (&p)[4]) {
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = m == -INFINITY ? 0.f : exp2f(x[r] - m);
      const u32x2 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      lds_write_b64(lds_addr(&Pl[hh * kPStride + 16 * rt + 4 * g]), pw);
    };
    float p[4];
    write_p(m_s, p);
    if (g == 0) red_m[hh][rt] = mx;
    lds_barrier();
    // Vote (the same in every wave): does any head's block maximum pass its
    // running maximum by more than 8?
    if (__ballot(hmax(lane & 31) > m_v + 8.f) != 0) {
      const float ms_new = bump(m_s, hmax(hh));
      const float a_s = ms_new == m_s ? 1.f : (m_s == -INFINITY ? 0.f : exp2f(m_s - ms_new));
      write_p(ms_new, p);
      l_w = l_w * a_s + sum4rows((p[0] + p[1]) + (p[2] + p[3]));
      m_s = ms_new;
      m_v = bump(m_v, hmax(lane & 31));
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        f32x4 al;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float mn = bump(m_o[h2][r], hmax(16 * h2 + 4 * g + r));
          al[r] = mn == m_o[h2][r] ? 1.f : (m_o[h2][r] == -INFINITY ? 0.f : exp2f(m_o[h2][r] - mn));
          m_o[h2][r] = mn;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) o[h2][t] *= al;
      }
      lds_barrier();   // the rewritten P
    } else {
      l_w += sum4rows((p[0] + p[1]) + (p[2] + p[3]));
    }

    // ---- O[32 heads][dims 64w ..] += P V; lane (dim n, g) holds heads 16h2 + 4g + r
    const int s16 = lane & 15;
    const int ja = s16 >> 2;
    const int aa = s16 & 3;
#pragma unroll 1
    for (int kk = 0; kk < 2; ++kk) {
      const int ra = 32 * kk + 8 * g + ja;
      uint32_t ad[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int ch = (64 * w + 16 * t + 4 * aa) >> 3;
        const int hb = 8 * (aa & 1);
        ad[2 * t] = lds_addr(kv) + ra * kVRow + 16 * (ch ^ (ra & 15)) + hb;
        ad[2 * t + 1] = lds_addr(kv) + (ra + 4) * kVRow + 16 * (ch ^ ((ra + 4) & 15)) + hb;
      }
      u32x4 pr[2];
      s16x4 vt[8];
      lds_read_p2_tr8(pr, vt, lds_addr(&Pl[n * kPStride + 32 * kk + 8 * g]),
                      lds_addr(&Pl[(16 + n) * kPStride + 32 * kk + 8 * g]), ad);
      const bf16x8 pa[2] = {__builtin_bit_cast(bf16x8, pr[0]), __builtin_bit_cast(bf16x8, pr[1])};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const s16x4 v0 = vt[2 * t];
        const s16x4 v1 = vt[2 * t + 1];
        const short vv[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        bf16x8 vb;
#pragma unroll
        for (int e = 0; e < 8; ++e) vb[e] = __builtin_bit_cast(__bf16, vv[e]);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) o[h2][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[h2], vb, o[h2][t], 0, 0, 0);
      }
    }
    lds_barrier();   // this block's buffer is refilled by the next step
  };
  if (nblk > 0) gather(0, kvs0);
  for (int blk = 0; blk < nblk; blk += 2) {
    step(blk, kvs0, kvs1);
    if (blk + 1 < nblk) step(blk + 1, kvs1, kvs0);
  }

  // ---- results: the four row tiles' shares of each head's sum
  if (g == 0) red_l[hh][rt] = l_w;
  __syncthreads();
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hl = 16 * h2 + 4 * g + r;
      const f32x4 lv = *reinterpret_cast<const f32x4*>(&red_l[hl][0]);
      const float lr = (lv[0] + lv[1]) + (lv[2] + lv[3]);
      const float mr = m_o[h2][r];
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
      const float lse2 = lr > 0.f ? mr + log2f(lr) : -INFINITY;
      const int64_t bh = (int64_t)b * a.n_heads + hg * kWH + hl;
      const int dim0 = 64 * w + n;
      if (nsplit == 1) {
        __bf16* ob = static_cast<__bf16*>(a.out) + bh * kDV + dim0;
#pragma unroll
        for (int t = 0; t < 4; ++t) ob[16 * t] = (__bf16)(o[h2][t][r] * inv);
        if (w == 0 && n == 0) a.lse[bh] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
      } else {
        float* po = part_o + (bh * nsplit + split) * kDV + dim0;
#pragma unroll
        for (int t = 0; t < 4; ++t) po[16 * t] = o[h2][t][r] * inv;
        if (w == 0 && n == 0) part_lse[bh * nsplit + split] = lse2;
      }
    }
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
  // (request, head) of this block: head group instance bh / 16 sits on XCD
  // (bh / 16) % 8, the XCD whose workgroups wrote its partials
  const int jx = blockIdx.x >> 3;
  const int64_t bh = 16 * (8 * (int64_t)(jx / 16) + (blockIdx.x & 7)) + jx % 16;
  if (bh >= (int64_t)a.num_req * a.n_heads) return;
  const float* pl = part_lse + bh * nsplit;
  const int d0 = threadIdx.x * 4;
  // The first kFirst partials are loaded together with the log-sum-exps
  // (they do not depend on the weights): one round trip instead of one per
  // group of loads.  Indexes past nsplit read the last partial again and get
  // weight 0.
  constexpr int kFirst = 32;
  const float ls_raw = (int)threadIdx.x < nsplit ? pl[threadIdx.x & (kMaxSplit - 1)] : -INFINITY;
  f32x4 v[kFirst];
#pragma unroll
  for (int s = 0; s < kFirst; ++s)
    v[s] = *reinterpret_cast<const f32x4*>(part_o + (bh * nsplit + min(s, nsplit - 1)) * kDV + d0);
  __builtin_amdgcn_sched_barrier(0);
  if (threadIdx.x < 64) {
    const float ls = ls_raw;
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
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kFirst; ++s) acc += wts[s] * v[s];
  for (int s = kFirst; s < nsplit; ++s) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(part_o + (bh * nsplit + s) * kDV + d0);
    acc += wts[s] * x;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  __bf16* ob = static_cast<__bf16*>(a.out) + bh * kDV;
  u32x2 w2 = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  *reinterpret_cast<u32x2*>(ob + d0) = w2;
  if (threadIdx.x == 0) a.lse[bh] = wsum > 0.f ? (M + log2f(wsum)) * kLn2 : -INFINITY;
}

// Merge of the 16-head kernel's bf16 partials (dims in lane order: dim
// 128w + 16t + n stored at 128w + 8n + t): out = sum_s 2^(lse_s - M) o_s /
// sum_s 2^(lse_s - M).  One workgroup of four waves per (request, head), two
// stored dims per thread (more loads in flight than two waves with four
// dims); every wave works out the split weights itself and broadcasts them
// from the lanes that hold them.
__global__ __launch_bounds__(256) void mla_combine_bf16_kernel(AttnArgs a, int nsplit,
                                                                const __bf16* part_o,
                                                                const float* part_lse) {
  constexpr int kBatch = 32;     // splits loaded before any is used
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const float* pl = part_lse + bh * nsplit;
  const __bf16* pb = part_o + bh * nsplit * kDV + 2 * tid;
  // nsplit <= 64: lane s holds split s's log-sum-exp
  const float ls = lane < nsplit ? pl[lane] : -INFINITY;
  float acc[2] = {0.f, 0.f};
  float M = -INFINITY, wgt = 0.f, wsum = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
    const int nb = min(kBatch, nsplit - s0);
    uint32_t v[kBatch];
#pragma unroll
    for (int s = 0; s < kBatch; ++s) v[s] = *reinterpret_cast<const uint32_t*>(pb + (int64_t)(s0 + min(s, nb - 1)) * kDV);
    __builtin_amdgcn_sched_barrier(0);
    if (s0 == 0) {
      M = ls;
      for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
      wgt = (M == -INFINITY || ls == -INFINITY) ? 0.f : exp2f(ls - M);
      wsum = wgt;
      for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o);
    }
#pragma unroll
    for (int s = 0; s < kBatch; ++s) {
      if (s < nb) {
        const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), s0 + s));
        acc[0] += ws * __uint_as_float(v[s] << 16);
        acc[1] += ws * __uint_as_float(v[s] & 0xFFFF0000u);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  // stored dims 2 tid, 2 tid + 1 = 128w + 8n + t0 + i hold dims 128w + 16 (t0 + i) + n
  const int w = tid >> 6, n = (tid & 63) >> 2, t0 = 2 * (tid & 3);
  __bf16* ob = static_cast<__bf16*>(a.out) + bh * kDV + 128 * w + 16 * t0 + n;
#pragma unroll
  for (int i = 0; i < 2; ++i) ob[16 * i] = (__bf16)(acc[i] * inv);
  if (tid == 0) a.lse[bh] = wsum > 0.f ? (M + log2f(wsum)) * kLn2 : -INFINITY;
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

// Kernel and split of the selection for a launch.  The 32-head kernel takes
// batches (enough workgroups to fill the chip at one per CU); the 16-head
// kernel, with twice the workgroups per request, takes few requests.
struct MlaPlan {
  bool wide;
  int nsplit;
  int rows_per_split;
};

constexpr int kWideMinReq = 4;

MlaPlan plan_mla(int num_req, int n_heads, int k) {
  const int blocks = (k + kMBlk - 1) / kMBlk;
  const bool wide = n_heads % kWH == 0 && num_req >= kWideMinReq;
  const int groups = num_req * (n_heads / (wide ? kWH : kMH));
  const int max_rows = wide ? kWMaxRows : kMaxSplitRows;
  // about one workgroup per CU (both kernels' LDS allows one), at least one
  // block per split, at most max_rows rows per workgroup
  int ns = (int)ceil_div((int64_t)num_cus(), std::max(groups, 1));
  ns = std::min(ns, std::max(1, blocks));
  ns = std::max(ns, (int)ceil_div(blocks, max_rows / kMBlk));
  ns = std::min(std::max(ns, 1), 64);
  const int rows_per_split = (int)ceil_div(blocks, ns) * kMBlk;
  return {wide, (int)ceil_div(std::max(k, 1), rows_per_split), rows_per_split};
}

}  // namespace

bool mla_resolves(int num_req, int n_heads, int k) { return !plan_mla(num_req, n_heads, k).wide; }

size_t mla_ws_bytes(int num_req, int n_heads, int dv, int k) {
  const MlaPlan p = plan_mla(num_req, n_heads, k);
  if (p.nsplit == 1) return 0;
  return align_up((size_t)num_req * n_heads * p.nsplit * (dv + 1) * sizeof(float), 256);
}

hipError_t launch_mla_bf16(const AttnArgs& a, hipStream_t s) {
  const MlaPlan p = plan_mla(a.num_req, a.n_heads, a.k);
  const int nsplit = p.nsplit;
  const int rows_per_split = p.rows_per_split;
  // partials: [num_req * n_heads][nsplit][dv] (fp32 for the 32-head kernel,
  // bf16 for the 16-head one), then the [num_req * n_heads][nsplit] log-sum-exps
  float* part_o = static_cast<float*>(a.ws);
  float* part_lse = part_o ? part_o + (size_t)a.num_req * a.n_heads * nsplit * kDV : nullptr;
  const int units = a.num_req * nsplit;
  if (p.wide) {
    const int grid = (int)ceil_div(units, 8) * 8 * (a.n_heads / kWH);
    launch(mla_bf16_wide_kernel, dim3(grid), dim3(kWThreads), 0, s, "mla_bf16_wide_kernel", a, rows_per_split, nsplit,
                       units, part_o, part_lse);
    if (nsplit > 1) {
      // one block per (request, head), laid out so that head group instance
      // i (16 heads) lands on XCD i % 8
      const int64_t inst = (int64_t)a.num_req * (a.n_heads / kMH);
      launch(mla_combine_kernel, dim3((unsigned)(8 * 16 * ceil_div(inst, 8))), dim3(kDV / 4), 0, s,
             "mla_combine_kernel", a, nsplit, part_o, part_lse);
    }
  } else {
    // 8 XCDs x (units per XCD) x head groups: unit u with all its head groups
    // on XCD u % 8
    const int grid = (int)(8 * ceil_div(units, 8) * (a.n_heads / kMH));
    __bf16* part_b = reinterpret_cast<__bf16*>(part_o);
    launch(mla_bf16_kernel, dim3(grid), dim3(kMThreads), 0, s, "mla_bf16_kernel", a, rows_per_split, nsplit, units,
           part_b, part_lse);
    if (nsplit > 1)
      launch(mla_combine_bf16_kernel, dim3((unsigned)(a.num_req * a.n_heads)), dim3(256), 0, s,
             "mla_combine_bf16_kernel", a, nsplit, part_b, part_lse);
  }
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  const size_t smem = sizeof(float) * (a.dk + 256 + 256 + 8);
  launch(attn_f32_kernel, dim3(a.n_heads, a.num_req), dim3(256), smem, s, "attn_f32_kernel", a);
  return hipGetLastError();
}

}  // namespace lsi

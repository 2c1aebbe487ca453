// Indexer scan kernels: I_s = sigma_s * sum_j w_j * max(0, q_j . k_s) for every
// cached token (the lightning indexer of the "Multi-layer Indexer" abstract
// scores the whole cache of a layer).
//
// fp8 keys: the contraction [64 heads x 128] x [128 x 32 tokens] runs on the
// fp8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales), heads on
// the accumulator rows, tokens on the lanes, with the key bytes fed to the
// MFMA as stored (no conversion instruction).  The bf16 query is split
// exactly into two fp8 parts: per head a power of two 2^E puts the largest
// |q| in [128, 256), hi = RNE_e4m3(q 2^E) and lo = e4m3(q 2^E - hi).  A bf16
// value has 8 significant bits and hi carries the top 4 (with rounding), so
// the remainder has at most 4 and lo holds it exactly whenever the scaled
// value is at least 2^-2 (the lowest e4m3 binade with a 2^-9 step); smaller
// elements, below 2^-10 of their head's largest, keep an error under 2^-10
// in scaled units.  acc += hi.k + lo.k, and the head weight absorbs 2^-E.
// int4 keys (compact keys of the two-stage search) use v_mfma_f32_32x32x16_f16
// on an exact nibble-to-fp16 conversion (below).  ReLU, the head weights and
// the head sum stay in registers: a lane sums the 32 heads it holds and one
// cross-half swap adds the other 32.
//
// Memory paths: a contiguous page walk (every cached token of a request)
// streams 32-token tiles from the pages into an LDS ring by global->LDS DMA
// (scan_dma_kernel); gathered positions (the exact rescoring of the two-stage
// search) load each lane's own key row into registers (scan_gather_kernel).
#include "lsi_internal.hpp"

namespace lsi {
namespace {

constexpr int kTile = 32;        // tokens per MFMA tile
constexpr int kWaves = 4;        // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kMaxChunk = 8192;  // tokens per workgroup (contiguous mode, one request per grid row)
constexpr int kMaxBalChunk = 32768;   // tokens per workgroup (contiguous mode, balanced slices)
constexpr int kMaxChunkPages = 512;   // page ids a workgroup stages (two per thread)
static_assert(kMaxChunkPages <= 2 * 256, "two page ids per thread");
constexpr int KIND_FP8 = 0;
constexpr int KIND_INT4 = 1;

// Bits of the scale word that mark a gathered row as absent (a NaN, which no
// valid per-token scale is).
constexpr uint32_t kAbsent = 0xFFFFFFFFu;

struct TileFetch {
  u32x4 raw[4];   // the lane's key half (fp8: 64 bytes, int4: raw[0..1] = 32 bytes)
  float scale;    // kAbsent when the position or page is invalid
};

// ---------------------------------------------------------------------------
// int4 keys (compact keys of the two-stage search) run on fp16 MFMA.
// A nibble n in [-7,7] becomes the fp16 value n exactly: (n ^ 8) | 0x6400 is
// the fp16 number 1032 + n, and one packed fp16 add of -1032 leaves n.
// The bf16 query is scaled per head by a power of two 2^E_j that puts its
// largest element in [2^14, 2^15), which makes it exact in fp16; the head
// weight absorbs 2^-E_j.  Pairs are extracted as dims (0,4),(1,5),(2,6),(3,7)
// of each 8-dim group; the query uses the same order.
// ---------------------------------------------------------------------------
// The second nibble of each byte is taken in place: (x & 0x00F000F0) |
// 0x64006400 is the fp16 number 1024 + 16 n' (exact), and one packed fma
// with 1/16 and -72 leaves n' - 8 = n exactly; the upper byte's nibbles
// after one shift by 8.  Ten instructions per eight values instead of twelve.
__device__ __forceinline__ f16x8 int4x8_to_f16x8(uint32_t d) {
  const uint32_t x = d ^ 0x88888888u;
  const uint32_t y = x >> 8;
  const f16x2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2 bias_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
  f16x2 p0 = __builtin_bit_cast(f16x2, (x & 0x000F000Fu) | 0x64006400u) + bias;
  f16x2 p1 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, (x & 0x00F000F0u) | 0x64006400u), sixteenth, bias_hi);
  f16x2 p2 = __builtin_bit_cast(f16x2, (y & 0x000F000Fu) | 0x64006400u) + bias;
  f16x2 p3 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, (y & 0x00F000F0u) | 0x64006400u), sixteenth, bias_hi);
  f16x8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

template <int KIND>
struct QOp {
  using T = typename std::conditional<KIND == KIND_FP8, bf16x8, f16x8>::type;
};

// Gathered positions: lane (m, h) loads half h of the key row of position
// m of its tile (64 bytes fp8, 32 int4) straight into registers; two tiles
// per wave in flight.
template <int KIND>
__global__ __launch_bounds__(kThreads, 2) void scan_gather_kernel(ScanArgs a, int chunk, int page_shift) {
  constexpr int ROW = KIND == KIND_FP8 ? kDim : kDim / 2;   // key bytes per token
  using QT = typename QOp<KIND>::T;
  constexpr int kRing = 2;                                  // tiles in the prefetch ring
  __shared__ float inv_scale[kWaves * kHeads];
  __shared__ __attribute__((aligned(16))) float wl[kWaves * kHeads];   // w_j * 2^-E_j

  if (a.zero_ptr) {
    const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * kThreads;
    for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kThreads + threadIdx.x;
         i < a.zero_words; i += nthreads)
      a.zero_ptr[i] = 0u;
  }
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 31;
  const int h = lane >> 5;
  const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int n_items = a.n_pos;
  const int nprod = max(1, (n_items + chunk - 1) / chunk);
  if ((int)blockIdx.x >= nprod) return;
  const int begin = blockIdx.x * chunk;
  const int end = min(begin + chunk, n_items);
  const int ntile = max(0, (end - begin + kTile - 1) / kTile);
  // the slice item of lane m in tile tile_in (clamped to the slice)
  auto tile_item = [&](int tile_in) {
    const int tile = min(tile_in, ntile - 1);
    return min(begin + tile * kTile + m, end - 1);
  };
  // the positions of the wave's first two tiles are loaded before the query
  // is prepared (their round trip overlaps that work); ntile >= 1 here, so
  // the loads are unconditional and in bounds
  const int pos_first0 = a.positions[(int64_t)b * a.n_pos + tile_item(wave)];
  const int pos_first1 = a.positions[(int64_t)b * a.n_pos + tile_item(wave + kWaves)];

  // query operand: lane (m, h) holds head 32*mt+m, dims 64h+8t .. 64h+8t+7
  const __bf16* qb = static_cast<const __bf16*>(a.q) + (int64_t)b * kHeads * kDim;
  QT qa[2][8];
  // fp8 path: qs[mt][part*2 + s] = 32 fp8 bytes (dims 64h + 32s ..) of the hi
  // (part 0) or lo (part 1) split of head 32*mt + m
  i32x8 qs[2][4];
  if constexpr (KIND == KIND_FP8) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int head = 32 * mt + m;
      bf16x8 raw[8];
      float amax = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        raw[t] = *reinterpret_cast<const bf16x8*>(qb + head * kDim + 64 * h + 8 * t);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)raw[t][e]));
      }
      {
        const uint32_t u = __float_as_uint(amax);
        auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        amax = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      int e2 = 0;
      if (amax > 0.f) (void)frexpf(amax, &e2);
      const int E = (amax > 0.f) ? 8 - e2 : 0;
      const float sc = ldexpf(1.0f, E);
      if (h == 0) inv_scale[wave * kHeads + head] = ldexpf(1.0f, -E);
#pragma unroll
      for (int sI = 0; sI < 2; ++sI) {
        i32x8 hi, lo;
#pragma unroll
        for (int d = 0; d < 8; ++d) {          // dword d: dims 64h + 32 sI + 4d .. +3
          const int t = sI * 4 + (d >> 1);
          const int e0 = (d & 1) * 4;
          float x[4], rem[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) x[j] = (float)raw[t][e0 + j] * sc;
          int ph = 0;
          ph = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], ph, false);
          ph = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], ph, true);
          const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(ph, false);
          const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(ph, true);
          rem[0] = x[0] - h01[0];
          rem[1] = x[1] - h01[1];
          rem[2] = x[2] - h23[0];
          rem[3] = x[3] - h23[1];
          int pl = 0;
          pl = __builtin_amdgcn_cvt_pk_fp8_f32(rem[0], rem[1], pl, false);
          pl = __builtin_amdgcn_cvt_pk_fp8_f32(rem[2], rem[3], pl, true);
          hi[d] = ph;
          lo[d] = pl;
        }
        qs[mt][sI] = hi;
        qs[mt][2 + sI] = lo;
      }
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int head = 32 * mt + m;
      bf16x8 raw[8];
      float amax = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        raw[t] = *reinterpret_cast<const bf16x8*>(qb + head * kDim + 64 * h + 8 * t);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)raw[t][e]));
      }
      {
        const uint32_t u = __float_as_uint(amax);
        auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        amax = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      int e2 = 0;
      if (amax > 0.f) (void)frexpf(amax, &e2);
      const int E = (amax > 0.f) ? 15 - e2 : 0;
      const float sc = ldexpf(1.0f, E);
      if (h == 0) inv_scale[wave * kHeads + head] = ldexpf(1.0f, -E);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        constexpr int order[8] = {0, 4, 1, 5, 2, 6, 3, 7};
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (_Float16)((float)raw[t][order[e]] * sc);
        qa[mt][t] = v;
      }
    }
  }
  __syncthreads();

  // head weights (with the query scale folded in), read per tile from LDS:
  // the accumulator row of register r in a 32x32 tile is 8*(r/4) + 4*h + r%4,
  // so each group of four registers needs four consecutive weights
  if (lane < kHeads) wl[wave * kHeads + lane] = a.w[(int64_t)b * kHeads + lane] * inv_scale[wave * kHeads + lane];
  __builtin_amdgcn_wave_barrier();
  const f32x4* wl4 = reinterpret_cast<const f32x4*>(wl + wave * kHeads + 4 * h);

  // Every load below is unconditional and in bounds by construction, so the
  // compiler can keep all tiles of the ring in flight (a conditional load at a
  // join point makes it drain every outstanding load): the tile index is
  // clamped to the last tile of the slice, an out-of-range page or position
  // reads row 0 of the pool and is reported as -inf, and tokens past the end of
  // a request still lie inside their allocated page and are never stored.
  auto fetch_at = [&](int pos) {
    TileFetch f;
    const bool in = pos >= 0 && pos < L;
    const int page = a.page_table[(int64_t)b * a.max_pages + ((in ? pos : 0) >> page_shift)];
    const bool ok = in && page >= 0 && page < a.num_pages;
    const int64_t row = ok ? (int64_t)page * a.page_size + (pos & (a.page_size - 1)) : 0;
    const u32x4* kp = reinterpret_cast<const u32x4*>(
        static_cast<const uint8_t*>(a.keys) + row * ROW + h * (ROW / 2));
#pragma unroll
    for (int i = 0; i < ROW / 32; ++i) f.raw[i] = kp[i];
    const float sc = a.kscale[row];
    f.scale = ok ? sc : __uint_as_float(kAbsent);
    return f;
  };
  auto fetch = [&](int tile_in) { return fetch_at(a.positions[(int64_t)b * a.n_pos + tile_item(tile_in)]); };

  // Consume tile `tile` held in f, refill f with the tile two wave-steps
  // ahead, then compute and store.  Two TileFetch registers form a ring that
  // the loop below walks with static names, so two tiles stay in flight.
  auto consume = [&](TileFetch& f, int tile) {
    u32x4 kr[ROW / 32];
#pragma unroll
    for (int i = 0; i < ROW / 32; ++i) kr[i] = f.raw[i];
    const float scale = f.scale;
    const int item = begin + tile * kTile + m;
    const bool valid = item < end;
    const bool ok = __float_as_uint(scale) != kAbsent;
    f = fetch(tile + kRing * kWaves);   // clamped at the end of the slice
    f32x16 acc0 = {};
    f32x16 acc1 = {};
    if constexpr (KIND == KIND_FP8) {
#pragma unroll
      for (int sI = 0; sI < 2; ++sI) {
        const u32x4 k0 = kr[2 * sI];
        const u32x4 k1 = kr[2 * sI + 1];
        const i32x8 kb = {(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w,
                          (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qs[0][part * 2 + sI], kb, acc0,
                                                                 0, 0, 0, 127, 0, 127);
          acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qs[1][part * 2 + sI], kb, acc1,
                                                                 0, 0, 0, 127, 0, 127);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if constexpr (KIND == KIND_FP8) {
      } else {
        const u32x4 r4 = kr[t >> 2];
        const uint32_t d = (t & 3) == 0 ? r4.x : (t & 3) == 1 ? r4.y : (t & 3) == 2 ? r4.z : r4.w;
        const f16x8 kb = int4x8_to_f16x8(d);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[0][t], kb, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[1][t], kb, acc1, 0, 0, 0);
      }
    }
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 w0 = wl4[2 * q];        // heads 8q + 4h + 0..3
      const f32x4 w1 = wl4[8 + 2 * q];    // heads 32 + 8q + 4h + 0..3
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        part += w0[j] * fmaxf(acc0[4 * q + j], 0.f);
        part += w1[j] * fmaxf(acc1[4 * q + j], 0.f);
      }
    }
    const float total = half_swap_sum(part);
    if (h == 0 && valid) a.scores[(int64_t)b * a.ld + item] = ok ? total * scale : -INFINITY;
  };

  if (wave < ntile) {
    TileFetch f0 = fetch_at(pos_first0);
    TileFetch f1 = fetch_at(pos_first1);
    for (int tile = wave; tile < ntile; tile += 2 * kWaves) {
      consume(f0, tile);
      if (tile + kWaves >= ntile) break;
      consume(f1, tile + kWaves);
    }
  }
}

// ---------------------------------------------------------------------------
// Contiguous page walk (fp8 or int4 keys): the prefetch ring lives in LDS and
// is filled by global->LDS DMA (global_load_lds_dwordx4), so no VGPRs hold
// tiles in flight and no instruction copies them into LDS.  Each DMA
// instruction moves 1 KB (8 fp8 or 16 int4 token rows) contiguously; a
// lane's 16 bytes land at base + 16*lane, so the lane fetches the chunk that
// belongs at that LDS position (the chunk order within a row is permuted per
// row, see goff/rd below), which spreads the per-lane 16-byte reads of the
// MFMA layout over all bank groups.  The query operand (hi/lo fp8 split, or
// exact fp16) is computed once per workgroup, 16 heads per wave, and handed
// to every wave through LDS.
// ---------------------------------------------------------------------------
// Per key kind: bytes per token row, per tile, and the DMA operations that
// fill one ring slot (1 KB code moves plus one move of the 32 scales).
template <int KIND>
struct DmaTile {
  static constexpr int kRow = KIND == KIND_FP8 ? kDim : kDim / 2;
  static constexpr int kBytes = kTile * kRow;           // fp8 4 KB, int4 2 KB
  static constexpr int kSlot = kBytes + 256;            // codes + the 32 scales, twice
  static constexpr int kMoves = kBytes / 1024;
  static constexpr int kOps = kMoves + 1;
};
constexpr int kFlushTiles = 32;             // tiles of scores staged per wave (4 KB)

// Key tiles are read once: the non-temporal hint keeps them from evicting the
// freshly written scores from L2, whose write-back would otherwise interleave
// with the key stream in HBM.
constexpr int kNonTemporal = 2;

template <int OFF>
__device__ __forceinline__ void lds_dma16(uint8_t* lds, const uint8_t* g) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, OFF, kNonTemporal);
}
// The four 16-byte reads of a lane's key half, with their wait in the same
// statement.  Written out because the compiler, not knowing which DMA wrote
// which ring position, would otherwise wait for every DMA in flight first.
__device__ __forceinline__ void lds_read_tile(u32x4 (&kr)[4], const uint8_t* slot, const uint32_t (&rd)[4]) {
  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)slot;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3])
      : "v"(base + rd[0]), "v"(base + rd[1]), "v"(base + rd[2]), "v"(base + rd[3])
      : "memory");
}
// Workgroup barrier for LDS data only.  __syncthreads() also releases global
// memory, which waits for every DMA in flight; here only LDS writes need to
// be visible to the other waves.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// The tile reads plus one float at byte offset `so` of the slot (its scale),
// all complete when the statement ends: the slot may be refilled right after.
__device__ __forceinline__ void lds_read_tile_scale(u32x4 (&kr)[4], float& sc, const uint8_t* slot,
                                                    const uint32_t (&rd)[4], uint32_t so) {
  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)slot;
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b128 %1, %6\n\t"
      "ds_read_b128 %2, %7\n\t"
      "ds_read_b128 %3, %8\n\t"
      "ds_read_b32 %4, %9\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3]), "=&v"(sc)
      : "v"(base + rd[0]), "v"(base + rd[1]), "v"(base + rd[2]), "v"(base + rd[3]), "v"(base + so)
      : "memory");
}
__device__ __forceinline__ float lds_read_f32(const uint8_t* p) {
  const uint32_t addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
  float v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ void lds_dma4(uint8_t* lds, const float* g) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 4, 0, kNonTemporal);
}

// LDS accesses to the ring's memory once no DMA is in flight (the
// histogram), written out for the same reason as the tile reads: the
// compiler would wait for every vector-memory operation first, the score
// stores included.  Each statement completes its own accesses.
__device__ __forceinline__ uint32_t lds_u32_addr(const uint32_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint32_t*)p;
}
__device__ __forceinline__ void lds_zero16(uint32_t* p) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  asm volatile("ds_write_b128 %0, %1" : : "v"(lds_u32_addr(p)), "v"(z) : "memory");
}
// two LDS increments; returns the counts they found
__device__ __forceinline__ void lds_inc2_rtn(uint32_t* p0, uint32_t* p1, uint32_t& r0, uint32_t& r1) {
  asm volatile(
      "ds_add_rtn_u32 %0, %2, %4\n\t"
      "ds_add_rtn_u32 %1, %3, %4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1)
      : "v"(lds_u32_addr(p0)), "v"(lds_u32_addr(p1)), "v"(1u)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_read_u32(const uint32_t* p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_u32_addr(p)) : "memory");
  return v;
}

// The lane's 32 bytes of an int4 key row (two 16-byte reads) and the tile's
// scale word, complete when the statement ends.
__device__ __forceinline__ void lds_read_tile2_scale(u32x4 (&kr)[2], float& sc, const uint8_t* slot,
                                                     const uint32_t (&rd)[2], uint32_t so) {
  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)slot;
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %4\n\t"
      "ds_read_b32 %2, %5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(sc)
      : "v"(base + rd[0]), "v"(base + rd[1]), "v"(base + so)
      : "memory");
}

// Wait until the tile issued RING - 1 refills ago has landed: every refill
// is OPS vector-memory operations.  Why a count suffices (AMD's CDNA3
// Instruction Set Architecture reference guide, "Data Dependency
// Resolution" and the s_waitcnt description; the CDNA4 guide keeps the
// rule): VM_CNT counts the wave's vector-memory instructions that have not
// completed, and vector-memory loads complete in the order they were
// issued, so waiting until VM_CNT <= n means every load but the last n has
// completed.  A global load with the LDS modifier (global_load_lds_dwordx4,
// the "load to LDS" form of the buffer/global instructions) is such a load:
// it increments VM_CNT at issue and decrements it once its data are
// written to LDS.  The score stores a wave issues between refills are
// vector-memory operations too; they only add to the count behind the
// tile's loads, which makes the wait stricter, never looser.
template <int RING, int OPS>
__device__ __forceinline__ void wait_ring_tile() {
  static_assert(RING == 2 && (OPS == 5 || OPS == 3), "two-slot ring of fp8 or int4 tiles");
  if constexpr (OPS == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  if constexpr (OPS == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
}

template <int KIND, int RING>
__global__ __launch_bounds__(kThreads, 3) void scan_dma_kernel(ScanArgs a, int chunk, int page_shift, int bal_n, int bal_sp) {
  using TL = DmaTile<KIND>;
  constexpr int kSlotBytes = TL::kSlot;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[RING][kWaves * kSlotBytes];
  __shared__ int pages[kMaxChunkPages];
  __shared__ __attribute__((aligned(16))) float wl[kHeads];   // w_j * 2^-E_j
  __shared__ __attribute__((aligned(16))) float sbuf[kWaves][kFlushTiles * kTile];

  if (a.zero_ptr) {
    const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * kThreads;
    for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kThreads + threadIdx.x;
         i < a.zero_words; i += nthreads)
      a.zero_ptr[i] = 0u;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31;
  const int h = lane >> 5;
  uint8_t* slot[RING];
#pragma unroll
  for (int r = 0; r < RING; ++r) slot[r] = &ring[r][0] + wv * kSlotBytes;
  uint8_t* qraw = reinterpret_cast<uint8_t*>(&sbuf[wv][0]);
  static_assert(sizeof(sbuf[0]) == 16 * kDim * 2, "a wave's staging buffer holds its 16 query rows");

  // The workgroup's slice: request b, positions [begin, begin + span).
  int b = 0, begin = 0, span = 0, Lraw = 0;
  int npg_max = 0, page_in0 = -1, page_in1 = -1;
  // One round trip for the slice's page ids (as far as the longest request
  // reaches; the request's own length only trims them), the request length
  // (with_len) and the query rows and head weights.  The query split is
  // computed while the first key tiles are on their way.  The query rows of
  // the wave's 16 heads (4 KB) and the 64 head weights come in by DMA, into
  // the wave's part of the score staging buffer (its query split is written
  // over them once read) and the start of its slot in the last ring
  // position (filled with a tile only after the split): an ordinary load
  // issued ahead of the tile DMAs would be waited for with every DMA behind
  // it.  (The page ids and the length are such loads; their wait covers
  // these DMAs too, which is what the prologue wants.)  Issue order after
  // that wait: tiles 0 .. RING-2; the last ring position gets its tile once
  // the split is done.
  auto prologue = [&](bool with_len) {
    npg_max = max(0, (min(begin + span, a.max_seq_len) - begin + a.page_size - 1) >> page_shift);
    const int32_t* pt = a.page_table + (int64_t)b * a.max_pages + (begin >> page_shift);
    page_in0 = tid < npg_max ? pt[tid] : -1;
    page_in1 = tid + kThreads < npg_max ? pt[tid + kThreads] : -1;
    if (with_len) Lraw = a.seq_lens[b];
    const uint8_t* qg = reinterpret_cast<const uint8_t*>(static_cast<const __bf16*>(a.q) +
                                                        ((int64_t)b * kHeads + 16 * wv) * kDim) + 16 * lane;
    asm volatile("" ::: "memory");
    lds_dma16<0>(qraw, qg);
    lds_dma16<1024>(qraw, qg);
    lds_dma16<2048>(qraw, qg);
    lds_dma16<3072>(qraw, qg);
    lds_dma4(slot[RING - 1], a.w + (int64_t)b * kHeads + lane);
  };
  if (bal_n > 0) {
    // The slice the grid would have if every request had the longest
    // length (bal_n slices of bal_sp positions per request) is loaded
    // while the real one is worked out, and loaded again only if it differs.
    const int gb = (int)blockIdx.x / bal_n;
    const int gbegin = ((int)blockIdx.x % bal_n) * bal_sp;
    b = gb;
    begin = gbegin;
    span = bal_sp;
    if (gb < a.num_req) prologue(false);
    // Balanced slices over a one-dimensional grid of G workgroups (at most
    // kThreads requests): request r of length L_r gets slices of
    // ceil(L_r / n_r) positions rounded up to a multiple of `chunk`, with
    // n_r = ceil(L_r * G' / T) for T the batch's tokens and G' the largest
    // of eight values from G down to G - R whose slices fit in the grid (at
    // G - R they always do).  Workgroups take the slices in request order;
    // the rest retire here.
    constexpr int kCand = 8;
    __shared__ int64_t bal_sum[kWaves];
    __shared__ int bal_cnt[kWaves][kCand];
    __shared__ int bal_scan[kWaves];
    __shared__ int bal_own[4];
    const int R = a.num_req;
    const int64_t G = gridDim.x;
    const int Lr = tid < R ? min(max(a.seq_lens[tid], 0), a.max_seq_len) : 0;
    int64_t t = Lr;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const int lo = __shfl_xor((int)(uint32_t)t, o);
      const int hi = __shfl_xor((int)(t >> 32), o);
      t += (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
    }
    if (lane == 0) bal_sum[wv] = t;
    if (tid == 0) bal_own[0] = -1;
    __syncthreads();
    int64_t T = 0;
#pragma unroll
    for (int x = 0; x < kWaves; ++x) T += bal_sum[x];
    const bool uniform = T == (int64_t)R * a.max_seq_len;   // every request at the longest length
    // x / y rounded up for 0 <= x < 2^53, y > 0: a double quotient, then
    // corrected (a 64-bit integer division is a long software sequence)
    auto cdiv = [](int64_t x, int64_t y) -> int64_t {
      int64_t q = (int64_t)__builtin_ceil((double)x / (double)y);
      if (q * y < x) ++q;
      else if (q > 0 && (q - 1) * y >= x) --q;
      return q;
    };
    auto slices = [&](int i, int& sp) -> int {   // slices of this thread's request at G'_i
      sp = 0;
      if (Lr == 0) return 0;
      const int64_t Gi = G - ((int64_t)R * i + kCand - 2) / (kCand - 1);
      const int nr = (int)max((int64_t)1, cdiv((int64_t)Lr * Gi, T));
      sp = (int)(cdiv(cdiv(Lr, nr), chunk) * chunk);
      return (int)cdiv(Lr, sp);
    };
    if (!uniform) {
      // G' = G first; the seven smaller values only when that does not fit
      int pick = 0;
      {
        int sp;
        int c = slices(0, sp);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
        if (lane == 0) bal_cnt[wv][0] = c;
      }
      __syncthreads();
      {
        int c = 0;
#pragma unroll
        for (int x = 0; x < kWaves; ++x) c += bal_cnt[x][0];
        if (c > G) pick = -1;
      }
      if (pick < 0) {
        for (int i = 1; i < kCand; ++i) {
          int sp;
          int c = slices(i, sp);
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
          if (lane == 0) bal_cnt[wv][i] = c;
        }
        __syncthreads();
        pick = kCand - 1;
        for (int i = kCand - 1; i >= 1; --i) {
          int c = 0;
#pragma unroll
          for (int x = 0; x < kWaves; ++x) c += bal_cnt[x][i];
          if (c <= G) pick = i;
        }
      }
      int sp;
      const int used = slices(pick, sp);
      int inc = used;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o);
        if (lane >= o) inc += v;
      }
      if (lane == 63) bal_scan[wv] = inc;
      __syncthreads();
      int pre = inc - used;
#pragma unroll
      for (int x = 0; x < kWaves; ++x)
        if (x < wv) pre += bal_scan[x];
      const int me = (int)blockIdx.x;
      if (used > 0 && me >= pre && me < pre + used) {
        bal_own[0] = tid;
        bal_own[1] = (me - pre) * sp;
        bal_own[2] = sp;
        bal_own[3] = Lr;
      }
      __syncthreads();
      b = bal_own[0];
      begin = bal_own[1];
      span = bal_own[2];
      Lraw = bal_own[3];
    } else {
      // every request has the longest length: the slicing is the one
      // loaded above
      b = gb < R ? gb : -1;
      Lraw = a.max_seq_len;
    }
    if (b < 0) {             // no slice for this workgroup
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (a.range_slots != nullptr && tid == 0)
        a.range_slots[blockIdx.y * gridDim.x + blockIdx.x] = make_uint4(~0u, 0u, 0u, 0u);
      return;
    }
    if (b != gb || begin != gbegin || span != bal_sp) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      prologue(false);
    }
  } else {
    b = blockIdx.y;
    begin = blockIdx.x * chunk;
    span = chunk;
    prologue(true);
  }
  const int L = min(max(Lraw, 0), a.max_seq_len);
  if (begin > 0 && begin >= L) {
    // nothing of this request here; no DMA may still be writing the LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (a.range_slots != nullptr && tid == 0)
      a.range_slots[blockIdx.y * gridDim.x + blockIdx.x] = make_uint4(~0u, 0u, 0u, 0u);
    return;
  }
  if (tid < npg_max) pages[tid] = page_in0;
  if (tid + kThreads < npg_max) pages[tid + kThreads] = page_in1;
  lds_barrier();   // the page ids only: the query DMAs are waited for below
  const int end = min(begin + span, L);
  const int ntile = max(0, (end - begin + kTile - 1) / kTile);

  // A wave takes a contiguous run of the slice's tiles, so its scores form
  // one contiguous range.
  const int per = (ntile + kWaves - 1) / kWaves;
  const int my0 = wv * per;
  const int myn = max(0, min(ntile - my0, per));
  // fp8: a 1 KB move covers 8 rows of 128 bytes, chunk j of row r stored at
  // j ^ (r % 8); int4: 16 rows of 64 bytes, chunk j of row r at j ^ f(r),
  // f(r) = (r ^ (r / 4)) % 4, which puts the 16-byte reads of 8 consecutive
  // rows at one chunk into 8 different bank groups
  uint32_t goff;
  uint32_t rd[KIND == KIND_FP8 ? 4 : 2];
  if constexpr (KIND == KIND_FP8) {
    const int r8 = lane >> 3;
    goff = 128 * r8 + 16 * ((lane & 7) ^ r8);
#pragma unroll
    for (int i = 0; i < 4; ++i) rd[i] = m * 128 + 16 * ((4 * h + i) ^ (m & 7));
  } else {
    const int r16 = lane >> 2;
    goff = 64 * r16 + 16 * ((lane & 3) ^ ((r16 ^ (r16 >> 2)) & 3));
#pragma unroll
    for (int i = 0; i < 2; ++i) rd[i] = m * 64 + 16 * ((2 * h + i) ^ ((m ^ (m >> 2)) & 3));
  }
  const uint8_t* keys = static_cast<const uint8_t*>(a.keys);

  // Tiles 0 .. RING - 1 are always issued (the query split's wait counts
  // on them); a refill j + RING only when that tile exists.  So while a
  // later tile has been issued, RING - 1 later tiles of TL::kOps DMAs each
  // (four (fp8) or two (int4) 1 KB key moves and one for the 32 scales,
  // which lanes 32..63 copy a second time) follow a tile's DMAs, and
  // waiting until at most that many vector-memory operations are
  // outstanding means the tile has landed in LDS (loads complete in issue
  // order); the wave's last tile, with nothing issued after it, waits for
  // all of them.  The initial fills past a short run (and every fill of a
  // wave without tiles) read pool row 0, which all of them share in L2, into
  // a slot that is never consumed; they are the only DMAs that can still be
  // in flight once the run is done (when it has fewer than RING tiles).  A
  // slot is refilled only after every read of it has completed (its reads
  // end with their own wait).
  auto issue = [&](int j, uint8_t* slot) {
    int64_t row0 = 0;
    if (j < myn) {
      const int t0 = (my0 + j) * kTile;
      const int page = __builtin_amdgcn_readfirstlane(pages[t0 >> page_shift]);
      if (page >= 0 && page < a.num_pages)
        row0 = (int64_t)page * a.page_size + ((begin + t0) & (a.page_size - 1));
    }
    const uint8_t* g = keys + row0 * TL::kRow + goff;
    asm volatile("" ::: "memory");
    lds_dma16<0>(slot, g);
    lds_dma16<1024>(slot, g);
    if constexpr (TL::kMoves == 4) {
      lds_dma16<2048>(slot, g);
      lds_dma16<3072>(slot, g);
    }
    lds_dma4(slot + TL::kBytes, a.kscale + row0 + m);
  };

#pragma unroll
  for (int r = 0; r + 1 < RING; ++r) issue(r, slot[r]);
  wait_ring_tile<RING, TL::kOps>();   // the query DMAs, RING - 1 tile groups ago
  const int qhead = 16 * wv + (lane >> 2);
  const int d0 = 32 * (lane & 3);
  bf16x8 raw[4];
  float wq;
  {
    u32x4 qr[4];
    uint32_t qoff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) qoff[t] = (lane >> 2) * 2 * kDim + 2 * d0 + 16 * t;
    lds_read_tile(qr, qraw, qoff);
#pragma unroll
    for (int t = 0; t < 4; ++t) raw[t] = __builtin_bit_cast(bf16x8, qr[t]);
    wq = lds_read_f32(slot[RING - 1] + 4 * qhead);
  }

  // Query operand in the score staging buffer (free until the first tile is
  // scored).  fp8: row `head` holds 16 chunks of 16 bytes, hi dims then lo
  // dims; int4: 16 chunks of 8 fp16, dims 8c..8c+7 in the order
  // (0,4,1,5,2,6,3,7) that the nibble conversion produces.  Chunk c is stored
  // at position c ^ (head % 16) so that the reads below, 16 rows at a time at
  // one logical chunk, spread over all banks.  A wave writes only the rows of
  // its own 16 heads, over its own raw query rows, which it has read.
  uint8_t* qx = reinterpret_cast<uint8_t*>(&sbuf[0][0]);
  static_assert(sizeof(sbuf) == kHeads * 2 * kDim, "query operand fills the staging buffer");
  {
    float amax = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)raw[t][e]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    int e2 = 0;
    if (amax > 0.f) (void)frexpf(amax, &e2);
    uint8_t* row = qx + qhead * 2 * kDim;
    const int sw = qhead & 15;
    if constexpr (KIND == KIND_FP8) {
      const int E = (amax > 0.f) ? 8 - e2 : 0;
      const float sc = ldexpf(1.0f, E);
      if ((lane & 3) == 0) wl[qhead] = wq * ldexpf(1.0f, -E);
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) {              // dword d: dims d0 + 4d .. +3
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (float)raw[d >> 1][(d & 1) * 4 + j] * sc;
        int ph = 0;
        ph = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], ph, false);
        ph = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], ph, true);
        const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(ph, false);
        const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(ph, true);
        int pl = 0;
        pl = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] - h01[0], x[1] - h01[1], pl, false);
        pl = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] - h23[0], x[3] - h23[1], pl, true);
        hi[d] = (uint32_t)ph;
        lo[d] = (uint32_t)pl;
      }
      const int c0 = d0 / 16;
      *reinterpret_cast<u32x4*>(row + 16 * (c0 ^ sw)) = u32x4{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<u32x4*>(row + 16 * ((c0 + 1) ^ sw)) = u32x4{hi[4], hi[5], hi[6], hi[7]};
      *reinterpret_cast<u32x4*>(row + 16 * ((8 + c0) ^ sw)) = u32x4{lo[0], lo[1], lo[2], lo[3]};
      *reinterpret_cast<u32x4*>(row + 16 * ((9 + c0) ^ sw)) = u32x4{lo[4], lo[5], lo[6], lo[7]};
    } else {
      // the largest |q| of the head scaled into [2^14, 2^15): exact in fp16
      const int E = (amax > 0.f) ? 15 - e2 : 0;
      const float sc = ldexpf(1.0f, E);
      if ((lane & 3) == 0) wl[qhead] = wq * ldexpf(1.0f, -E);
      constexpr int order[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
      for (int t = 0; t < 4; ++t) {            // chunk d0 / 8 + t: dims d0 + 8t .. +7
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (_Float16)((float)raw[t][order[e]] * sc);
        *reinterpret_cast<f16x8*>(row + 16 * ((d0 / 8 + t) ^ sw)) = v;
      }
    }
  }
  lds_barrier();
  // fp8: qs[mt][part*2 + sI] = 32 bytes (dims 64h + 32 sI ..) of part `part`
  // of head 32 mt + m; int4: qa[mt][t] = fp16 dims 64h + 8t .. of that head
  i32x8 qs[2][4];
  f16x8 qa[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int head = 32 * mt + m;
    const uint8_t* row = qx + head * 2 * kDim;
    if constexpr (KIND == KIND_FP8) {
#pragma unroll
      for (int part = 0; part < 2; ++part)
#pragma unroll
        for (int sI = 0; sI < 2; ++sI) {
          const int c = part * 8 + 4 * h + 2 * sI;
          const u32x4 v0 = *reinterpret_cast<const u32x4*>(row + 16 * (c ^ (head & 15)));
          const u32x4 v1 = *reinterpret_cast<const u32x4*>(row + 16 * ((c + 1) ^ (head & 15)));
          qs[mt][part * 2 + sI] = i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                                        (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
        }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        qa[mt][t] = *reinterpret_cast<const f16x8*>(row + 16 * ((8 * h + t) ^ (head & 15)));
    }
  }
  lds_barrier();   // the staging buffer takes scores from here on
  const f32x4* wl4 = reinterpret_cast<const f32x4*>(wl + 4 * h);
  issue(RING - 1, slot[RING - 1]);    // the query rows are no longer needed

  // Score of token m of the wave's j-th tile (the same in lanes m and m + 32).
  const int nissued = max(myn, RING);   // tiles whose DMAs are issued
  auto consume = [&](int j, uint8_t* slot) -> float {
    if (j + 1 < nissued) wait_ring_tile<RING, TL::kOps>();
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    float scale;
    f32x16 acc0 = {};
    f32x16 acc1 = {};
    if constexpr (KIND == KIND_FP8) {
      u32x4 kr[4];
      lds_read_tile_scale(kr, scale, slot, rd, TL::kBytes + 4 * lane);
#pragma unroll
      for (int sI = 0; sI < 2; ++sI) {
        const u32x4 k0 = kr[2 * sI];
        const u32x4 k1 = kr[2 * sI + 1];
        const i32x8 kb = {(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w,
                          (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qs[0][part * 2 + sI], kb, acc0,
                                                                 0, 0, 0, 127, 0, 127);
          acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qs[1][part * 2 + sI], kb, acc1,
                                                                 0, 0, 0, 127, 0, 127);
        }
      }
    } else {
      u32x4 kr[2];
      lds_read_tile2_scale(kr, scale, slot, rd, TL::kBytes + 4 * lane);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x4 r4 = kr[t >> 2];
        const uint32_t d = (t & 3) == 0 ? r4.x : (t & 3) == 1 ? r4.y : (t & 3) == 2 ? r4.z : r4.w;
        const f16x8 kb = int4x8_to_f16x8(d);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[0][t], kb, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[1][t], kb, acc1, 0, 0, 0);
      }
    }
    const int page = pages[((my0 + j) * kTile) >> page_shift];
    const bool ok = page >= 0 && page < a.num_pages;
    // the slot's reads are complete (the MFMAs consumed them): refill it
    if (j + RING < myn) issue(j + RING, slot);
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 w0 = wl4[2 * q];        // heads 8q + 4h + 0..3
      const f32x4 w1 = wl4[8 + 2 * q];    // heads 32 + 8q + 4h + 0..3
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        part += w0[jj] * fmaxf(acc0[4 * q + jj], 0.f);
        part += w1[jj] * fmaxf(acc1[4 * q + jj], 0.f);
      }
    }
    const float total = half_swap_sum(part);
    return ok ? total * scale : -INFINITY;
  };

  // Scores are staged per wave in LDS and written kFlushTiles tiles (4 KB)
  // at a time: a trickle of small score stores from every wave, each to its
  // own DRAM row, slows the key stream far beyond the bytes it adds.
  float* out = a.scores + (int64_t)b * a.ld + begin;
  float* stage = sbuf[wv];
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;   // key range of this lane's scores (range_slots)
  auto stage_score = [&](int j, float v) {
    if (h == 0) {
      stage[(j % kFlushTiles) * kTile + m] = v;
      if (a.range_slots != nullptr && (my0 + j) * kTile + m < end - begin) {
        const uint32_t kk = float_key(v);
        kmn = min(kmn, kk);
        kmx = max(kmx, kk);
      }
    }
  };
  auto flush = [&](int j) {                  // after tile j, the last of its group
    const int first = j - j % kFlushTiles;
    const int pos0 = (my0 + first) * kTile;
    const int n = min((j - first + 1) * kTile, (end - begin) - pos0);
    __builtin_amdgcn_wave_barrier();
    for (int i = 4 * lane; i < n; i += 4 * 64) {
      if (i + 4 <= n) {
        // written through to memory (sc1): the top-k that follows reads the
        // scores from other XCDs, and lines left dirty in L2 would be
        // written back at the end of the launch, after the last workgroup
        const f32x4 v = *reinterpret_cast<const f32x4*>(stage + i);
        asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(out + pos0 + i), "v"(v) : "memory");
      } else {
        for (int k = i; k < n; ++k) out[pos0 + k] = stage[k];
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  for (int j = 0; j < myn; j += RING) {
    {
      // Issue priority falls as the run nears its end.  Three workgroups
      // share a CU and the oldest waves otherwise win every arbitration, so
      // the first-dispatched finish far ahead of the last and the CU ends
      // its work under-occupied; this keeps co-resident runs in step.
      const int p = (6 * (myn - j)) / (myn + 1);
      if (p >= 3) __builtin_amdgcn_s_setprio(3);
      else if (p == 2) __builtin_amdgcn_s_setprio(2);
      else if (p == 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int jr = j + r;
      if (jr >= myn) break;
      stage_score(jr, consume(jr, slot[r]));
      if (jr + 1 == myn || (jr + 1) % kFlushTiles == 0) flush(jr);
    }
  }
  // No DMA may still be writing this workgroup's LDS when it retires or
  // when the ring holds the histogram below.  A run of RING or more tiles
  // has none left (its last tile waited for all); the score stores are not
  // waited for (the barriers below are LDS-only).
  if (myn < RING) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (a.range_slots != nullptr) {
    // the workgroup's key range (waves combined in LDS) into its slot: plain
    // stores (atomics from every workgroup on one row's pair of words
    // serialise, several microseconds at 512 workgroups)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, o));
      kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, o));
    }
    uint32_t* lr = reinterpret_cast<uint32_t*>(&ring[0][0]);
    __syncthreads();
    if (tid < 2) lr[tid] = 0u;
    __syncthreads();
    if (lane == 0 && kmx >= kmn) {
      atomicMax(&lr[0], ~kmn);
      atomicMax(&lr[1], kmx);
    }
    __syncthreads();
    if (tid == 0)
      a.range_slots[blockIdx.y * gridDim.x + blockIdx.x] = make_uint4(lr[1] != 0u ? (uint32_t)b : ~0u, lr[0], lr[1], 0u);
  }
  if (a.hist_rep != nullptr) {
    // The histogram of this workgroup's scores for the top-k that follows:
    // 12-bit and 6-bit top key digits, counted in the ring's LDS (no DMA is
    // in flight any more; the barriers wait for LDS operations only, so the
    // score stores stay in flight) and added to one of the row's replicas (workgroups
    // spread over kHistReps copies, so that the few hot bins take a sixteenth
    // of the atomics each).  Every score of the wave is still in its staging
    // buffer: the host enables this for slices of at most 32 tiles per wave.
    // Cleared with 16-byte stores; the lane whose LDS add finds a bin empty
    // adds that bin's final count to the replica (one global add per
    // non-empty bin, no pass over all 4160 bins).
    uint32_t* lh = reinterpret_cast<uint32_t*>(&ring[0][0]);
    static_assert(sizeof(ring) >= kHistWords * 4 && kHistWords % 4 == 0, "the ring holds the histogram");
    lds_barrier();   // every wave is done with the ring
    for (int i = tid; i < kHistWords / 4; i += kThreads) lds_zero16(lh + 4 * i);
    lds_barrier();
    const int nsc = myn > 0 ? min(myn * kTile, (end - begin) - my0 * kTile) : 0;
    uint32_t* gh = a.hist_rep + ((size_t)b * kHistReps + blockIdx.x % kHistReps) * kHistWords;
    constexpr int kMaxPer = kFlushTiles * kTile / 64;   // scores per lane at most (the staging buffer)
    uint32_t first = 0u;                                 // bit 2u: 12-bit bin new, 2u + 1: 6-bit bin new
    uint32_t bins[kMaxPer][2];
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
      const int i = lane + 64 * u;
      bins[u][0] = bins[u][1] = 0u;
      if (i < nsc) {
        const uint32_t key = float_key(stage[i]);
        bins[u][0] = key >> 20;
        bins[u][1] = 4096 + (key >> 26);
        uint32_t c0, c1;
        lds_inc2_rtn(&lh[bins[u][0]], &lh[bins[u][1]], c0, c1);
        first |= (c0 == 0u ? 1u : 0u) << (2 * u);
        first |= (c1 == 0u ? 1u : 0u) << (2 * u + 1);
      }
      if (64 * (u + 1) >= nsc) break;
    }
    lds_barrier();   // every count is in
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
        if ((first >> (2 * u + e)) & 1u) atomicAdd(&gh[bins[u][e]], lds_read_u32(&lh[bins[u][e]]));
      if (64 * (u + 1) >= nsc) break;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 keys (small generic case): one thread per token, fp32 FMAs in order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scan_f32_kernel(ScanArgs a) {
  extern __shared__ float smem[];
  if (a.zero_ptr) {
    const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * blockDim.x;
    for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
         i < a.zero_words; i += nthreads)
      a.zero_ptr[i] = 0u;
  }
  const int H = a.n_heads;
  const int d = a.dim;
  float* qs = smem;           // [H][d]
  float* ws = smem + H * d;   // [H]
  const int b = blockIdx.y;
  const float* qg = static_cast<const float*>(a.q) + (int64_t)b * H * d;
  for (int i = threadIdx.x; i < H * d; i += blockDim.x) qs[i] = qg[i];
  for (int i = threadIdx.x; i < H; i += blockDim.x) ws[i] = a.w[(int64_t)b * H + i];
  __syncthreads();
  const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= L) return;
  const int page = a.page_table[(int64_t)b * a.max_pages + s / a.page_size];
  if ((unsigned)page >= (unsigned)a.num_pages) {
    a.scores[(int64_t)b * a.ld + s] = -INFINITY;
    return;
  }
  const float* kr = static_cast<const float*>(a.keys) +
                    ((int64_t)page * a.page_size + s % a.page_size) * d;
  float total = 0.f;
  for (int j = 0; j < H; ++j) {
    float dot = 0.f;
    for (int i = 0; i < d; ++i) dot = fmaf(qs[j * d + i], kr[i], dot);
    total = fmaf(ws[j], fmaxf(dot, 0.f), total);
  }
  a.scores[(int64_t)b * a.ld + s] = total;
}

}  // namespace

int pick_chunk(int64_t num_req, int64_t max_items, int page_size, bool gather, int wg_per_cu) {
  // aim at one wave of resident workgroups over the whole batch
  const int64_t target = (int64_t)num_cus() * wg_per_cu;
  const int64_t unit = std::max<int64_t>(kTile * kWaves, gather ? 1 : page_size);
  int64_t chunk = ceil_div(num_req * max_items, target);
  chunk = ceil_div(std::max<int64_t>(chunk, 256), unit) * unit;
  if (!gather) chunk = std::min<int64_t>(chunk, std::max<int64_t>(kMaxChunk, unit));
  return (int)std::min<int64_t>(chunk, 1 << 24);
}

bool scan_builds_hist(int num_req, int max_seq_len, int page_size) {
  // one request walks the contiguous path; each wave's run must fit its
  // staging buffer (32 tiles: slices of at most 4096 positions)
  return num_req == 1 && pick_chunk(1, max_seq_len, page_size, false, 3) <= kWaves * kFlushTiles * kTile;
}

namespace {

template <int KIND>
hipError_t launch_mfma_scan(const ScanArgs& a_in, hipStream_t s, int* nslots) {
  // key ranges only when every workgroup has a slot
  ScanArgs a = a_in;
  auto slots = [&](int64_t g) {
    if (a.range_slots != nullptr && g > kMaxRangeSlots) a.range_slots = nullptr;
    if (nslots) *nslots = a.range_slots != nullptr ? (int)g : 0;
  };
  const bool gather = a.positions != nullptr;
  const int max_items = gather ? a.n_pos : a.max_seq_len;
  constexpr int kRingTiles = 2;
  const int ps = ilog2(a.page_size);
  if (!gather) {
    // Batches: one wave of resident workgroups over balanced slices, sized
    // on the device from the request lengths (a grid of one row per request
    // would leave the slices of ragged requests to a partial second wave).
    // Two per CU, although three fit: with three, the 32 x 131072-token
    // scan took 113-114 us on some devices against 95 on others; with two it
    // takes 93-95 us on both, and the 64-request ragged scan is faster too.
    const int64_t G = (int64_t)num_cus() * 2;
    const int64_t unit = std::max<int64_t>(kTile * kWaves, a.page_size);
    const int64_t work = (int64_t)a.num_req * a.max_seq_len;
    if (a.num_req >= 2 && a.num_req <= kThreads && 4 * (int64_t)a.num_req <= G &&
        a.max_seq_len <= (1 << 30) && work >= G * unit) {
      const int64_t span = ceil_div(ceil_div(work, G - a.num_req), unit) * unit;
      if (span <= kMaxBalChunk && ceil_div(span, (int64_t)a.page_size) <= kMaxChunkPages) {
        // the device's slicing when every request has the longest length:
        // the workgroups load that slice while they work out their own
        const int64_t R = a.num_req, Lm = a.max_seq_len, T = R * Lm;
        int64_t n_u = 0, sp_u = 0;
        for (int i = 0; i < 8; ++i) {
          const int64_t Gi = G - (R * i + 6) / 7;
          const int64_t nr = std::max<int64_t>(1, (Lm * Gi + T - 1) / T);
          const int64_t sp = ceil_div(ceil_div(Lm, nr), unit) * unit;
          const int64_t used = ceil_div(Lm, sp);
          if (R * used <= G || i == 7) {
            n_u = used;
            sp_u = sp;
            break;
          }
        }
        slots(G);
        launch((scan_dma_kernel<KIND, kRingTiles>), dim3((unsigned)G), dim3(kThreads), 0, s, KIND == KIND_FP8 ? "scan_dma_kernel<fp8>" : "scan_dma_kernel<int4>", a,
                           (int)unit, ps, (int)n_u, (int)sp_u);
        return hipGetLastError();
      }
    }
  }
  const int chunk = pick_chunk(a.num_req, max_items, a.page_size, gather, gather ? 2 : 3);
  // the DMA scan stages a slice's page ids, two per thread
  if (!gather && (chunk + a.page_size - 1) / a.page_size > kMaxChunkPages) return hipErrorInvalidValue;
  dim3 grid((unsigned)std::max<int64_t>(1, ceil_div(max_items, chunk)), (unsigned)a.num_req);
  if (gather) a.range_slots = nullptr;   // the contiguous walk only
  slots((int64_t)grid.x * grid.y);
  if (!gather) {
    launch((scan_dma_kernel<KIND, kRingTiles>), grid, dim3(kThreads), 0, s, KIND == KIND_FP8 ? "scan_dma_kernel<fp8>" : "scan_dma_kernel<int4>", a, chunk, ps, 0, 0);
  } else {
    launch(scan_gather_kernel<KIND>, grid, dim3(kThreads), 0, s, KIND == KIND_FP8 ? "scan_gather_kernel<fp8>" : "scan_gather_kernel<int4>", a, chunk, ps);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_fp8(const ScanArgs& a, hipStream_t s) { return launch_mfma_scan<KIND_FP8>(a, s, nullptr); }
hipError_t launch_scan_int4(const ScanArgs& a, hipStream_t s, int* nslots) {
  return launch_mfma_scan<KIND_INT4>(a, s, nslots);
}

hipError_t launch_scan_f32(const ScanArgs& a, hipStream_t s) {
  dim3 grid((unsigned)std::max<int64_t>(1, ceil_div(a.max_seq_len, 256)), (unsigned)a.num_req);
  const size_t smem = sizeof(float) * ((size_t)a.n_heads * a.dim + a.n_heads);
  launch(scan_f32_kernel, grid, dim3(256), smem, s, "scan_f32_kernel", a);
  return hipGetLastError();
}

}  // namespace lsi

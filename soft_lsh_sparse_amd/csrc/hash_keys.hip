// Prefill hashing: bucket ids of every key in L tables of P hyperplane sign
// bits, and the Euclidean norm of every value row.
//
// Step 1 of the soft-LSH mechanism of SOCKET (page "Resumen Técnico: SOCKET -
// Estimador de Núcleo de Colisión Suave para Atención Escasa", section
// "Mecanismo Central: LSH Suave", item 1; German page "SOCKET: SOft Collision
// Kernel EsTimator for Sparse Attention", Kernmechanismus, Vorverarbeitung):
// keys are hashed into L independent tables with random projections, one
// bucket per key and table, and the value norms are cached.
//
// bf16 path (the large prefill), three launches:
//
//  1. prep: R [d, C] is transposed to R^T [rows, d] (zero rows past C) in the
//     workspace, and the fix-up counter is cleared.
//  2. main: a persistent grid of two 4-wave blocks per CU. Every block walks
//     32-key tiles; the K and V rows of the next three tiles are in flight
//     into a 4-slot LDS ring (64 KB per block) through direct-to-LDS loads
//     (global_load_lds_dwordx4, no registers held), so each CU keeps about
//     100 KB of loads in flight while it computes. The projection y = K R runs
//     on the matrix cores (v_mfma_f32_32x32x16_bf16, float32 accumulation of
//     the exact bf16 products): every wave keeps up to 128 hyperplane
//     columns of R^T in registers as the stationary A operand and reads the
//     tile's K rows from LDS as the B operand (XOR-swizzled so the 8 lanes
//     the LDS serves together hit 8 bank groups), so one lane ends with 16
//     projections of one key. Their sign bits are packed with one funnel
//     shift each; the A rows are permuted so that a lane's 16 bits are 16
//     consecutive hyperplanes and one exchange between the two lane halves
//     yields a 32-bit word of 32 consecutive sign bits. With P = 8 that word
//     is four id bytes, stored directly. The value norms of the same tile are
//     reduced from the V rows in LDS (bf16 dot2).
//  3. fix-up: a sign is certified when |y| exceeds the worst-case float32
//     summation error 2*d*2^-24*|k|*max|r| (plus a floor for flushed
//     denormals). Uncertain projections (about 1.5e-4 of them for random
//     data) are appended by the main kernel to a per-wave list in the
//     workspace (one entry per key and 16-column group, with a mask; slots
//     from ballot prefix counts) with their float32 sign written; the fix-up
//     kernel recomputes each one from
//     the bf16 inputs (float64 sum of exact products, certified, with a
//     double-double fallback) and sets or clears that one bit with an atomic
//     AND/OR. A block with an overflowing list (or any block with an uncertain
//     sign when id rows are not whole 4-byte words) has all its tiles
//     re-hashed exactly by a fourth kernel (float64 / double-double, one
//     thread per key and table), which exits at once when nothing
//     overflowed. Either way the bucket ids are those of the exact dot
//     products.
//
// f32 path (small inputs): one thread per key, float64 dot products with the
// same certification and a serial double-double fallback.

#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace socket_lsh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define SOCKET_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kTileKeys = 32;
constexpr int kHashWaves = 4;        // one wave per SIMD; two blocks per CU
constexpr int kHashThreads = kHashWaves * 64;
constexpr int kRing = 4;              // LDS slots per block: one tile computed, three in flight
constexpr int kBlocksPerCU = 2;
constexpr int kMaxTilesPerWave = 4;   // 4 x 32 hyperplane columns per wave
constexpr int kMaxColWords = 16;      // L*P <= 512 bits per key
constexpr int kRtRows = kHashWaves * kMaxTilesPerWave * 32;
constexpr float kAbsFloor = 0x1p-100f;  // covers flushed float32 denormals
// fix-up entry: (row << 21) | (16-column group << 16) | mask of its columns
constexpr int kEntryRowShift = 21;

template <int D>
struct HashGeom {
  static constexpr int S = D / 16;                        // MFMA k-steps of 16
  static constexpr int CH = D / 8;                        // 16-byte chunks per row
  static constexpr int kTileBytes = kTileKeys * D * 2;    // one matrix of a tile
  static constexpr int kSlotBytes = 2 * kTileBytes;       // K then V
  static constexpr int kSegs = kSlotBytes / 1024;         // 1 KB load segments per slot
  static constexpr int kDmaPerWave = kSegs / kHashWaves;  // loads per wave per tile
  static_assert(kSegs % kHashWaves == 0, "every wave issues the same number of loads");
};

struct HashArgs {
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* R;   // [d, C]
  const uint16_t* RT;  // [kRtRows, d], zero past C
  int64_t n_keys, stride;
  int tph, n_tiles;  // tiles per head, tiles in total (< 2^31)
  int L, P, C;
  uint8_t* ids;
  float* vnorm;
  unsigned long long* fix_list;  // [grid * kHashWaves][fix_cap] entries, one region per wave
  uint32_t* fix_count;           // [grid * kHashWaves] entries each wave appended
  uint32_t fix_cap;  // per wave; 0: the block is re-hashed exactly when any sign is uncertain
};

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Block barrier that orders LDS only: the wave's LDS operations complete,
// then all waves meet. (__syncthreads would also drain every outstanding
// global load, which is exactly what the ring keeps in flight.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16-byte LDS reads and their completion in one asm block: the ring is
// filled by direct-to-LDS loads whose progress the compiler cannot see, so
// the kernel orders these reads itself (wait + barrier before them).
__device__ __forceinline__ void lds_read4(const uint32_t (&addr)[4], u32x4_t (&o)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3])
      : "memory");
}

__device__ __forceinline__ u32x4_t lds_read1(uint32_t addr) {
  u32x4_t o;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(o) : "v"(addr) : "memory");
  return o;
}

// Byte offset of a pointer into LDS, as DS instructions address it.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  typedef __attribute__((address_space(3))) const unsigned char lds_uchar;
  return (uint32_t)(uintptr_t)(lds_uchar*)p;
}

__device__ __forceinline__ float sumsq_bf16x2(uint32_t w, float acc) {
  const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

__device__ __forceinline__ float sumsq_bf16x8(const u32x4_t w, float acc) {
  const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
  acc = sumsq_bf16x2(w0, acc);
  acc = sumsq_bf16x2(w1, acc);
  acc = sumsq_bf16x2(w2, acc);
  return sumsq_bf16x2(w3, acc);
}

// P bits starting at bit `off` of a per-key bit vector.
__device__ __forceinline__ uint32_t extract_bits(const uint32_t* row, int off, int P) {
  const int w = off >> 5, b = off & 31;
  uint64_t x = row[w];
  if (b + P > 32) x |= (uint64_t)row[w + 1] << 32;
  return (uint32_t)(x >> b) & ((1u << P) - 1u);
}

// A row m of a 32-column MFMA tile holds hyperplane column jmap(m) of the
// tile. With the D layout (lane (n, h) holds rows (v/4)*8 + h*4 + v%4,
// v = 0..15) this gives lane half h the 16 consecutive columns h*16 + v.
__device__ __forceinline__ int jmap(int m) {
  return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3);
}

// K and V rows of tile `tile` into one ring slot (K at byte 0, V at
// kTileBytes). Wave w loads the 1 KB segments w, w + kHashWaves, ... of
// each matrix; lane i fills 16-byte position i of a segment. K rows are
// stored XOR-swizzled: position q of row r holds chunk q ^ (r & 7).
template <int D>
struct DmaLane {
  static constexpr int kSegsPerMatrix = HashGeom<D>::kDmaPerWave / 2;
  // rows between a wave's consecutive segments (a multiple of 8, so the
  // XOR swizzle of a position is the same in all of them)
  static constexpr int kRowStep = kHashWaves * 64 / HashGeom<D>::CH;
  static_assert(kSegsPerMatrix == 1 || kRowStep % 8 == 0, "swizzle period");
  int r0;    // row of this lane's position in the wave's first segment
  int koff;  // element offset of that position's K chunk in a full tile

  __device__ __forceinline__ DmaLane(int wave, int lane) {
    using G = HashGeom<D>;
    const int p = wave * 64 + lane;
    const int q = p % G::CH;
    r0 = p / G::CH;
    koff = r0 * D + (q ^ (r0 & 7)) * 8;
  }
};

template <int D>
__device__ __forceinline__ void dma_tile(const HashArgs& a, int tile, unsigned char* slot,
                                         const DmaLane<D>& dl, int wave) {
  using G = HashGeom<D>;
  const int head = tile / a.tph;
  const int64_t row0 = (int64_t)(tile - head * a.tph) * kTileKeys;
  const int rows = (int)min<int64_t>(kTileKeys, a.n_keys - row0);
  const uint16_t* kb = a.K + ((int64_t)head * a.stride + row0) * D;
  const uint16_t* vb = a.V + ((int64_t)head * a.stride + row0) * D;
  const int voff = (wave * 64 + (threadIdx.x & 63)) * 8;  // V is stored unswizzled
  if (rows == kTileKeys) {
#pragma unroll
    for (int j = 0; j < DmaLane<D>::kSegsPerMatrix; ++j) {
      const int g = wave + j * kHashWaves;
      const int step = j * DmaLane<D>::kRowStep * D;
      __builtin_amdgcn_global_load_lds((const void*)(kb + dl.koff + step),
                                       SOCKET_LDS(slot + g * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vb + voff + step),
                                       SOCKET_LDS(slot + G::kTileBytes + g * 1024), 16, 0, 0);
    }
  } else {
    // last tile of a head: rows past the end re-read row 0 (same count of
    // loads, so the wait counts stay exact)
#pragma unroll
    for (int j = 0; j < DmaLane<D>::kSegsPerMatrix; ++j) {
      const int g = wave + j * kHashWaves;
      const int r = dl.r0 + j * DmaLane<D>::kRowStep;
      const int step = j * DmaLane<D>::kRowStep * D;
      const int back = r < rows ? 0 : r * D;  // row r -> row 0
      __builtin_amdgcn_global_load_lds((const void*)(kb + dl.koff + step - back),
                                       SOCKET_LDS(slot + g * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vb + voff + step - back),
                                       SOCKET_LDS(slot + G::kTileBytes + g * 1024), 16, 0, 0);
    }
  }
}

struct TileRows {
  int64_t grow0;  // global row (head * stride + row) of key 0 of the tile
  int rows;       // keys of the tile (32 except at the end of a head)
};

__device__ __forceinline__ TileRows tile_rows(const HashArgs& a, int tile) {
  const int head = tile / a.tph;
  const int64_t row0 = (int64_t)(tile - head * a.tph) * kTileKeys;
  return {(int64_t)head * a.stride + row0, (int)min<int64_t>(kTileKeys, a.n_keys - row0)};
}

// One 32-key tile from its ring slot: projections on the matrix cores, the
// certified sign bits and the ids, the key norms (from the B operand already
// in registers) and the value norms.
template <int D, int TPW, bool kWordIds>
__device__ __forceinline__ void hash_tile(const HashArgs& a, int tile, const unsigned char* slot,
                                          const bf16x8_t (&ra)[TPW][HashGeom<D>::S],
                                          const float (&rmax)[TPW], uint32_t* bitvec,
                                          uint32_t& fix_n, unsigned long long* fix_list,
                                          int wave, int lane) {
  using G = HashGeom<D>;
  constexpr int S = G::S;
  constexpr float kGamma = 2.0f * D * 0x1p-24f;
  const int kn = lane & 31, kh = lane >> 5;
  const uint32_t sbase = lds_offset(slot);
  const TileRows tr = tile_rows(a, tile);
  const int CT = (a.C + 31) >> 5;

  // value norms: wave w takes keys w*8 .. w*8+7, 8 lanes per key
  {
    const int vkey = wave * 8 + (lane >> 3);
    u32x4_t vw[G::CH / 8];
    if constexpr (G::CH / 8 == 2) {
      const uint32_t addr[4] = {
          sbase + G::kTileBytes + vkey * (D * 2) + ((lane & 7) << 4),
          sbase + G::kTileBytes + vkey * (D * 2) + (((lane & 7) + 8) << 4),
          sbase + G::kTileBytes + vkey * (D * 2) + ((lane & 7) << 4),
          sbase + G::kTileBytes + vkey * (D * 2) + (((lane & 7) + 8) << 4)};
      u32x4_t t4[4];
      lds_read4(addr, t4);
      vw[0] = t4[0];
      vw[1] = t4[1];
    } else {
      vw[0] = lds_read1(sbase + G::kTileBytes + vkey * (D * 2) + ((lane & 7) << 4));
    }
    float vs = 0.f;
#pragma unroll
    for (int j = 0; j < G::CH / 8; ++j) vs = sumsq_bf16x8(vw[j], vs);
    vs += dpp_f32<0xB1>(vs);   // lanes i ^ 1
    vs += dpp_f32<0x4E>(vs);   // lanes i ^ 2
    vs += dpp_f32<0x141>(vs);  // the other quad of the half-row
    if ((lane & 7) == 0 && vkey < tr.rows)
      a.vnorm[tr.grow0 + vkey] = __builtin_amdgcn_sqrtf(vs);
  }

  // Column tiles in pairs (two accumulators live at a time): the B operand
  // (chunks kh*S + s of key row kn; the A rows use the same map) is read
  // four k-steps at a time, again for every pair. The first pass also sums
  // the squared key entries. (Column tiles past C multiply zero rows of
  // R^T; their bits are dropped.)
  const bool row_ok = kn < tr.rows;
  uint32_t word[TPW];  // 32 consecutive sign bits, in both lanes of a key
  float ksq = 0.f, thr_k = 0.f;
#pragma unroll
  for (int tp = 0; tp < TPW; tp += 2) {
    f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int s0 = 0; s0 < S; s0 += 4) {
      uint32_t addr[4];
      u32x4_t kw[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        addr[s] = sbase + kn * (D * 2) + (((kh * S + s0 + s) ^ (kn & 7)) << 4);
      lds_read4(addr, kw);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          if (tp + i < TPW)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                ra[tp + i][s0 + s], __builtin_bit_cast(bf16x8_t, kw[s]), acc[i], 0, 0, 0);
        if (tp == 0) ksq = sumsq_bf16x8(kw[s], ksq);
      }
    }
    if (tp == 0) {
      ksq += __builtin_bit_cast(float, xor32_u32(__builtin_bit_cast(uint32_t, ksq)));
      // an upper bound is enough: the hardware square root (1 ulp) rounded up
      thr_k = kGamma * 1.000001f * __builtin_amdgcn_sqrtf(ksq);
    }

    // sign bits, certification, uncertain signs
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = tp + i;
      if (t >= TPW) break;
      const int ct = wave * TPW + t;
      float mn = fabsf(acc[i][0]);
#pragma unroll
      for (int v = 1; v < 16; ++v) mn = fminf(mn, fabsf(acc[i][v]));
      uint32_t h = 0;
#pragma unroll
      for (int v = 15; v >= 0; --v)
        h = __builtin_amdgcn_alignbit(h, __float_as_uint(acc[i][v]), 31);
      h = ~h & 0xffffu;  // bit v: projection onto column ct*32 + kh*16 + v is > 0
      const float thr = thr_k * rmax[t] + kAbsFloor;
      // Rare: some lanes hold projections too close to zero for their float32
      // sign. Each such key lists its group of 16 columns with the mask of
      // uncertain ones (float32 signs stay in h) in the wave's own region:
      // slots from a ballot prefix count, no atomics. The count runs on past
      // the capacity, which marks the block for the exact re-hash.
      const bool cand = row_ok && ct < CT && mn <= thr;
      if (__ballot(cand) != 0) {
        const int c0 = ct * 32 + kh * 16;
        uint32_t fm = 0;
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (fabsf(acc[i][v]) <= thr) fm |= 1u << v;
        const int valid = min(max(a.C - c0, 0), 16);  // columns of this lane below C
        fm &= valid >= 16 ? 0xffffu : (1u << valid) - 1u;
        if (!cand) fm = 0;
        const uint64_t bal = __ballot(fm != 0);
        const uint32_t pos =
            fix_n + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (fm != 0 && pos < a.fix_cap)
          fix_list[pos] = ((unsigned long long)(tr.grow0 + kn) << kEntryRowShift) |
                          ((unsigned long long)(c0 >> 4) << 16) | fm;
        fix_n += (uint32_t)__popcll(bal);
      }
      const uint32_t o = xor32_u32(h);
      word[t] = kh ? (o | (h << 16)) : (h | (o << 16));
    }
  }
  if constexpr (kWordIds) {
    // P == 8: word ct holds the id bytes of tables 4ct .. 4ct+3
    if (row_ok) {
      uint32_t* orow = reinterpret_cast<uint32_t*>(a.ids + (tr.grow0 + kn) * a.L);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int ct = wave * TPW + t;
        if ((TPW == 1 ? 0 : (t & 1)) == kh && ct < CT) orow[ct] = word[t];
      }
    }
  } else {
    if (kh == 0) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int ct = wave * TPW + t;
        if (ct < CT) bitvec[kn * kMaxColWords + ct] = word[t];
      }
    }
    lds_barrier();
    uint8_t* obase = a.ids + tr.grow0 * a.L;
    const int tid = wave * 64 + lane;
    for (int q = tid; q < kTileKeys * a.L; q += kHashThreads) {
      const int r = q / a.L, l = q - r * a.L;
      if (r < tr.rows)
        obase[(int64_t)r * a.L + l] =
            (uint8_t)extract_bits(bitvec + r * kMaxColWords, l * a.P, a.P);
    }
    // the next writer of bitvec is past another barrier
  }
}

template <int D, int TPW, bool kWordIds>
__global__ __launch_bounds__(kHashThreads, kBlocksPerCU) void hash_keys_bf16_kernel(HashArgs a) {
  using G = HashGeom<D>;
  constexpr int S = G::S;
  constexpr int kWaitSteady = (kRing - 2) * G::kDmaPerWave;
  __shared__ __align__(16) unsigned char ring[kRing * G::kSlotBytes];
  __shared__ uint32_t bitvec[kWordIds ? 1 : kTileKeys * kMaxColWords];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kn = lane & 31, kh = lane >> 5;
  const int nb = gridDim.x;
  const int b = blockIdx.x;
  if (b >= a.n_tiles) return;
  const int iters = (a.n_tiles - b + nb - 1) / nb;  // tiles b, b + nb, ...
  const int part = b * kHashWaves + wave;  // this wave's list region
  unsigned long long* const fix_list = a.fix_list + (size_t)part * a.fix_cap;
  uint32_t fix_n = 0;  // wave-uniform count of listed entries

  // stationary A operand: R^T rows of this wave's column tiles
  bf16x8_t ra[TPW][S];
  float rmax[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int col = (wave * TPW + t) * 32 + jmap(kn);
    const uint4* src = reinterpret_cast<const uint4*>(a.RT + (int64_t)col * D);
    float sq = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint4 w = src[kh * S + s];
      const u32x4_t wv = {w.x, w.y, w.z, w.w};
      sq = sumsq_bf16x8(wv, sq);
      ra[t][s] = __builtin_bit_cast(bf16x8_t, wv);
    }
    sq += __shfl_xor(sq, 32, kWave);
    // the bound takes the largest column norm of the tile, rounded up
    rmax[t] = sqrtf(group_max<64>(sq)) * (1.0f + 0x1p-20f);
  }

  const DmaLane<D> dl(wave, lane);
#pragma unroll
  for (int j = 0; j < kRing - 1; ++j)
    if (j < iters) dma_tile<D>(a, b + j * nb, ring + j * G::kSlotBytes, dl, wave);

  for (int it = 0; it < iters; ++it) {
    // this wave's loads into the slot of tile `it` are done once at most the
    // loads of the later tiles are outstanding; the barrier then makes every
    // wave's part visible and frees the slot computed last round
    if (it + kRing - 2 < iters)
      wait_vmcnt<kWaitSteady>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    if (it + kRing - 1 < iters)
      dma_tile<D>(a, b + (it + kRing - 1) * nb,
                  ring + ((it + kRing - 1) % kRing) * G::kSlotBytes, dl, wave);
    hash_tile<D, TPW, kWordIds>(a, b + it * nb, ring + (it % kRing) * G::kSlotBytes, ra, rmax,
                                bitvec, fix_n, fix_list, wave, lane);
  }
  if (lane == 0) a.fix_count[part] = fix_n;
}

// R [d, C] -> R^T [kRtRows, d] with zero rows past C.
__global__ __launch_bounds__(256) void hash_prep_kernel(const uint16_t* __restrict__ R, int C,
                                                        int D, uint16_t* __restrict__ RT) {
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)kRtRows * D;
  for (int64_t i = i0; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i / D), d = (int)(i % D);
    RT[i] = c < C ? R[(int64_t)d * C + c] : (uint16_t)0;
  }
}

// Settles the listed uncertain projections. An entry names a key row, a
// group of 16 hyperplane columns and the mask of its uncertain columns.
// Blocks (blk, j) take the list regions of the waves of main-kernel block
// `blk`, kFixBlocksPerPart blocks per main block; 16 lanes per entry, which go
// through the masked columns one by one: each lane takes D/16 exact
// products of the key row and the R^T row (one contiguous load each), the
// float64 sum of the group decides the sign unless it is within the
// rounding bound of the sum of |products| (then double-double decides).
// The bit is set or cleared with an atomic on its 32-bit word.
constexpr int kFixBlocksPerPart = 16;

template <int D>
__global__ __launch_bounds__(256) void hash_fixup_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ RT, int C, int L, int P,
    uint8_t* __restrict__ ids, const unsigned long long* __restrict__ list,
    const uint32_t* __restrict__ count, uint32_t cap) {
  constexpr int kPer = D / 16;  // dims per lane: 8 (one 16-byte load) or 4
  const int blk = blockIdx.x / kFixBlocksPerPart;
  const int j = blockIdx.x % kFixBlocksPerPart;
  const int sub = threadIdx.x & 15;
  const uint32_t groups = blockDim.x / 16;
  // the block's regions back to back as one index range
  uint32_t n[kHashWaves], total = 0;
#pragma unroll
  for (int w = 0; w < kHashWaves; ++w) {
    n[w] = min(count[blk * kHashWaves + w], cap);
    total += n[w];
  }
  for (uint32_t e = j * groups + threadIdx.x / 16; e < total; e += kFixBlocksPerPart * groups) {
    uint32_t idx = e;
    int part = blk * kHashWaves;
#pragma unroll
    for (int w = 0; w < kHashWaves - 1; ++w)
      if (idx >= n[w] && part == blk * kHashWaves + w) {
        idx -= n[w];
        ++part;
      }
    const unsigned long long ent = list[(size_t)part * cap + idx];
    const int64_t row = (int64_t)(ent >> kEntryRowShift);
    const int c0 = (int)((ent >> 16) & 31u) * 16;
    uint32_t mask = (uint32_t)(ent & 0xffffu);
    uint16_t kv[kPer];
    if constexpr (kPer == 8)
      *reinterpret_cast<uint4*>(kv) = *reinterpret_cast<const uint4*>(K + row * D + sub * 8);
    else
      *reinterpret_cast<uint2*>(kv) = *reinterpret_cast<const uint2*>(K + row * D + sub * 4);
    while (mask != 0) {  // same mask in the 16 lanes: uniform
      const int col = c0 + __ffs(mask) - 1;
      mask &= mask - 1;
      uint16_t rv[kPer];
      if constexpr (kPer == 8)
        *reinterpret_cast<uint4*>(rv) = *reinterpret_cast<const uint4*>(RT + col * D + sub * 8);
      else
        *reinterpret_cast<uint2*>(rv) = *reinterpret_cast<const uint2*>(RT + col * D + sub * 4);
      double p[kPer];
      double s = 0.0, sa = 0.0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        p[i] = (double)bf16_bits_to_f32(kv[i]) * (double)bf16_bits_to_f32(rv[i]);
        s += p[i];
        sa += fabs(p[i]);
      }
      // identical sums in all 16 lanes, so the branch below is uniform
      s = sum16_f64(s);
      sa = sum16_f64(sa);
      bool pos;
      if (fabs(s) > (double)D * 0x1p-52 * sa) {
        pos = s > 0.0;
      } else {
        double h = 0.0, l = 0.0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) dd_add(h, l, p[i], 0.0, h, l);
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) {
          const double oh = __shfl_xor(h, m, kWave), ol = __shfl_xor(l, m, kWave);
          dd_add(h, l, oh, ol, h, l);
        }
        pos = h > 0.0;
      }
      if (sub == 0) {
        const uint64_t byte = (uint64_t)row * L + (uint64_t)(col / P);
        uint32_t* word = reinterpret_cast<uint32_t*>(ids + (byte & ~(uint64_t)3));
        const uint32_t bit = 1u << ((byte & 3) * 8 + col % P);
        if (pos)
          atomicOr(word, bit);
        else
          atomicAnd(word, ~bit);
      }
    }
  }
}

// Exact re-hash of the tiles of every main-kernel block whose list
// overflowed (count above the capacity; with capacity 0, any uncertain
// sign): one thread per (key, table) recomputes the table's P projections
// from the bf16 inputs in float64 (exact products; the sum of |products|
// bounds the rounding) or, when that cannot decide, in double-double, and
// rewrites the id byte. Blocks of parts without overflow exit at once.
template <int D>
__global__ __launch_bounds__(256) void hash_redo_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ R, int64_t n_keys,
    int64_t stride, int tph, int n_tiles, int nb, int L, int P, uint8_t* __restrict__ ids,
    const uint32_t* __restrict__ count, uint32_t cap) {
  const int blk = blockIdx.x;
  bool over = false;
  for (int w = 0; w < kHashWaves; ++w) over |= count[blk * kHashWaves + w] > cap;
  if (!over) return;
  const int C = L * P;
  for (int tile = blk; tile < n_tiles; tile += nb) {
    const int head = tile / tph;
    const int64_t row0 = (int64_t)(tile - head * tph) * kTileKeys;
    const int rows = (int)min<int64_t>(kTileKeys, n_keys - row0);
    const int64_t grow0 = (int64_t)head * stride + row0;
    for (int q = threadIdx.x; q < rows * L; q += blockDim.x) {
      const int r = q / L, l = q - r * L;
      const uint16_t* krow = K + (grow0 + r) * D;
      uint32_t id = 0;
      for (int j = 0; j < P; ++j) {
        const int col = l * P + j;
        double y = 0.0, mag = 0.0;
        for (int i = 0; i < D; ++i) {
          const double p = (double)bf16_bits_to_f32(krow[i]) *
                           (double)bf16_bits_to_f32(R[(int64_t)i * C + col]);
          y += p;
          mag += fabs(p);
        }
        if (fabs(y) <= (double)D * 0x1p-52 * mag) {
          double h = 0.0, lo = 0.0;
          for (int i = 0; i < D; ++i)
            dd_add(h, lo,
                   (double)bf16_bits_to_f32(krow[i]) *
                       (double)bf16_bits_to_f32(R[(int64_t)i * C + col]),
                   0.0, h, lo);
          y = h;
        }
        if (y > 0.0) id |= 1u << j;
      }
      ids[(grow0 + r) * L + l] = (uint8_t)id;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void hash_keys_f32_kernel(
    const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ R, int64_t n_heads, int64_t n_keys,
    int64_t stride, int L, int P, uint8_t* __restrict__ ids,
    float* __restrict__ vnorm) {
  const int64_t gidx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gidx >= n_heads * n_keys) return;
  const int64_t head = gidx / n_keys, row = gidx % n_keys;
  const int64_t off = head * stride + row;
  const int C = L * P;
  constexpr double kBound = 2.0 * D * 0x1p-53;

  float kr[D];
  double vs = 0.0;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    kr[i] = K[off * D + i];
    const double v = V[off * D + i];
    vs += v * v;
  }
  vnorm[off] = (float)sqrt(vs);

  for (int l = 0; l < L; ++l) {
    uint32_t id = 0;
    for (int j = 0; j < P; ++j) {
      const int c = l * P + j;
      double y = 0.0, mag = 0.0;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        const double p = (double)kr[i] * (double)R[(int64_t)i * C + c];
        y += p;
        mag += fabs(p);
      }
      if (fabs(y) <= kBound * mag) {
        double h = 0.0, lo = 0.0;
        for (int i = 0; i < D; ++i)
          dd_add(h, lo, (double)kr[i] * (double)R[(int64_t)i * C + c], 0.0, h,
                 lo);
        y = h;
      }
      if (y > 0.0) id |= 1u << j;
    }
    ids[off * L + l] = (uint8_t)id;
  }
}

// --------------------------------------------------------------- launchers

constexpr int kMaxHashBlocks = 256 * kBlocksPerCU;

struct HashWs {
  uint16_t* rt;
  uint32_t* count;            // [kMaxHashBlocks * kHashWaves]
  unsigned long long* list;   // [kMaxHashBlocks * kHashWaves][cap]
  uint32_t cap;               // entries per block
};

HashWs hash_ws_layout(void* ws, int64_t n_total, int d, int C) {
  HashWs w{};
  unsigned char* p = static_cast<unsigned char*>(ws);
  size_t off = 0;
  w.rt = reinterpret_cast<uint16_t*>(p + off);
  off = align256(off + (size_t)kRtRows * d * sizeof(uint16_t));
  w.count = reinterpret_cast<uint32_t*>(p + off);
  off = align256(off + kMaxHashBlocks * kHashWaves * sizeof(uint32_t));
  w.list = reinterpret_cast<unsigned long long*>(p + off);
  w.cap = hash_fix_capacity(n_total, C) / (kMaxHashBlocks * kHashWaves);
  return w;
}

template <int D, int TPW, bool kWordIds>
void launch_main(const HashArgs& a, hipStream_t stream) {
  // two blocks per CU (each ring takes 64 KB of the 160 KB of LDS)
  const int grid = std::min(a.n_tiles, kMaxHashBlocks);
  launch_kernel((hash_keys_bf16_kernel<D, TPW, kWordIds>), dim3(grid), dim3(kHashThreads), 0,
                stream, a);
}

template <int D>
void launch_main_d(const HashArgs& a, int tpw, bool word_ids, hipStream_t stream) {
  switch (tpw * 2 + (word_ids ? 1 : 0)) {
#define SOCKET_HASH_CASE(t)                                            \
  case 2 * t: launch_main<D, t, false>(a, stream); break;              \
  case 2 * t + 1: launch_main<D, t, true>(a, stream); break;
    SOCKET_HASH_CASE(1)
    SOCKET_HASH_CASE(2)
    SOCKET_HASH_CASE(3)
    SOCKET_HASH_CASE(4)
#undef SOCKET_HASH_CASE
    default: break;
  }
}

}  // namespace

uint32_t hash_fix_capacity(int64_t n_total, int C) {
  const int64_t want = n_total * C / 512;
  return (uint32_t)std::max<int64_t>(65536, std::min<int64_t>(want, (int64_t)1 << 26));
}

size_t hash_keys_bf16_workspace_bytes(int64_t n_total, int d, int C) {
  size_t off = align256((size_t)kRtRows * d * sizeof(uint16_t));
  off = align256(off + kMaxHashBlocks * kHashWaves * sizeof(uint32_t));
  const size_t parts = (size_t)kMaxHashBlocks * kHashWaves;
  return off + (hash_fix_capacity(n_total, C) / parts) * parts * sizeof(unsigned long long);
}

hipError_t launch_hash_keys_bf16(const uint16_t* K, const uint16_t* V,
                                 const uint16_t* R, int64_t n_heads,
                                 int64_t n_keys, int64_t stride, int d, int L,
                                 int P, uint8_t* ids, float* vnorm, void* ws,
                                 hipStream_t stream) {
  if (n_heads == 0 || n_keys == 0) return hipSuccess;
  const int C = L * P;
  const int64_t tph = (n_keys + kTileKeys - 1) / kTileKeys;
  if (n_heads * tph >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const HashWs w = hash_ws_layout(ws, n_heads * n_keys, d, C);
  // the fix-up patches bits through 4-byte words inside id rows
  const bool word_rows = (L % 4 == 0) && (reinterpret_cast<uintptr_t>(ids) & 3) == 0;
  HashArgs a{};
  a.K = K;
  a.V = V;
  a.R = R;
  a.RT = w.rt;
  a.n_keys = n_keys;
  a.stride = stride;
  a.tph = (int)tph;
  a.n_tiles = (int)(n_heads * tph);
  a.L = L;
  a.P = P;
  a.C = C;
  a.ids = ids;
  a.vnorm = vnorm;
  a.fix_list = w.list;
  a.fix_count = w.count;
  a.fix_cap = word_rows ? w.cap : 0u;

  launch_kernel(hash_prep_kernel, dim3(64), dim3(256), 0, stream, R, C, d, w.rt);
  const int CT = (C + 31) / 32;
  const int tpw = (CT + kHashWaves - 1) / kHashWaves;
  const bool word_ids = P == 8 && word_rows;
  if (d == 128)
    launch_main_d<128>(a, tpw, word_ids, stream);
  else
    launch_main_d<64>(a, tpw, word_ids, stream);
  const int blocks = std::min(a.n_tiles, kMaxHashBlocks);
  if (a.fix_cap != 0) {
    const dim3 fgrid(blocks * kFixBlocksPerPart);
    if (d == 128)
      launch_kernel(hash_fixup_kernel<128>, fgrid, dim3(256), 0, stream, K, w.rt, C, L, P,
                    ids, w.list, w.count, a.fix_cap);
    else
      launch_kernel(hash_fixup_kernel<64>, fgrid, dim3(256), 0, stream, K, w.rt, C, L, P,
                    ids, w.list, w.count, a.fix_cap);
  }
  if (d == 128)
    launch_kernel(hash_redo_kernel<128>, dim3(blocks), dim3(256), 0, stream, K, R, n_keys,
                  stride, a.tph, a.n_tiles, blocks, L, P, ids, w.count, a.fix_cap);
  else
    launch_kernel(hash_redo_kernel<64>, dim3(blocks), dim3(256), 0, stream, K, R, n_keys,
                  stride, a.tph, a.n_tiles, blocks, L, P, ids, w.count, a.fix_cap);
  return hipGetLastError();
}

hipError_t launch_hash_keys_f32(const float* K, const float* V, const float* R,
                                int64_t n_heads, int64_t n_keys,
                                int64_t stride, int d, int L, int P,
                                uint8_t* ids, float* vnorm,
                                hipStream_t stream) {
  const int64_t total = n_heads * n_keys;
  if (total == 0) return hipSuccess;
  const int grid = (int)((total + 255) / 256);
  if (d == 128)
    launch_kernel(hash_keys_f32_kernel<128>, dim3(grid), dim3(256), 0,
                  stream, K, V, R, n_heads, n_keys, stride, L, P, ids, vnorm);
  else
    launch_kernel(hash_keys_f32_kernel<64>, dim3(grid), dim3(256), 0,
                  stream, K, V, R, n_heads, n_keys, stride, L, P, ids, vnorm);
  return hipGetLastError();
}

}  // namespace socket_lsh

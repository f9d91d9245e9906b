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
//     workspace, and written again in the main kernel's fragment order.
//  2. main: one block of 8 waves per CU (two per SIMD). R^T of all the
//     hyperplane columns sits in LDS in the order the MFMA A operand reads
//     it (fragment (column tile, k-step) = 1 KB, conflict-free 16-byte
//     reads); every wave owns its own 32-key tiles and loads their K and V
//     rows straight into registers, each lane every other 16-byte chunk of
//     one row (the next tile's K while the current one is computed, the
//     current tile's V for its value norms at the end), so no wave waits
//     for another after the set-up. The projection y = K R runs on the
//     matrix cores (v_mfma_f32_32x32x16_bf16, float32 accumulation of the
//     exact bf16 products), one 32-column tile at a time, and the sign work
//     of the previous column tile sits between its k-steps. One lane ends with 16 projections of one key; their sign
//     bits are packed with one funnel shift each; the A rows are permuted so
//     that a lane's 16 bits are 16 consecutive hyperplanes and one exchange
//     between the two lane halves yields a 32-bit word of 32 consecutive
//     sign bits. With P = 8 that word is four id bytes, stored directly.
//  3. settle: a sign is certified when |y| exceeds the worst-case float32
//     summation error 2*d*2^-24*|k|*max|r| (plus a floor for flushed
//     denormals). Uncertain projections (about 1.5e-4 of them for random
//     data) are appended by the main kernel to a per-wave list in the
//     workspace (one entry per key and 16-column group, with a mask; slots
//     from ballot prefix counts) with their float32 sign written; the
//     blocks of a settling kernel recompute each one from the bf16 inputs
//     (float64 sum of exact products, certified, with a double-double
//     fallback) and set or clear that one bit with an atomic AND/OR. A
//     wave with an overflowing list (or any wave with an uncertain sign
//     when id rows are not whole 4-byte words) has all its tiles re-hashed
//     exactly by the other blocks of the same launch (float64 /
//     double-double, one thread per key and table; its list is left
//     alone), which go on at once when nothing overflowed. Either way the
//     bucket ids are those of the exact dot products.
//
// f32 path: one thread per key, float64 dot products with the same
// certification and a serial double-double fallback. bf16 inputs of at most
// 32 keys (the keys a decode step appends) take one launch of one block per
// key and one thread per hyperplane column, with the same arithmetic.

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
constexpr int kHashWaves = 8;         // two waves per SIMD, one block per CU
constexpr int kHashThreads = kHashWaves * 64;
constexpr int kMaxColWords = 16;      // L*P <= 512 bits per key
constexpr int kRtRows = kMaxColWords * 32;
constexpr float kAbsFloor = 0x1p-100f;  // covers flushed float32 denormals
// fix-up entry: (row << 21) | (16-column group << 16) | mask of its columns
constexpr int kEntryRowShift = 21;

struct HashArgs {
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* R;   // [d, C]
  const uint16_t* RT;  // [kRtRows, d], zero past C
  const uint4* RTF;    // R^T in the order of the MFMA A fragments (see the main kernel)
  int64_t n_keys, stride;
  int tph, n_tiles;  // 32-key tiles per head, tiles in total (< 2^31)
  int L, P, C;
  uint8_t* ids;
  float* vnorm;
  unsigned long long* fix_list;  // [grid * kHashWaves][fix_cap] entries, one region per wave
  uint32_t* fix_count;           // [grid * kHashWaves] entries each wave appended
  uint32_t fix_cap;  // per wave; 0: the wave's tiles are re-hashed exactly when any sign is uncertain
  int* owner;           // [n_tiles] the wave (list region) that hashed the tile
};

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

// Row m of a 32-column MFMA tile holds hyperplane column
// ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3) of the tile. With the D
// layout (lane (n, h) holds rows (v/4)*8 + h*4 + v%4, v = 0..15) this gives
// lane half h the 16 consecutive columns h*16 + v. jmap: the column of row
// m; jmap_inv: the row of column j.
__device__ __forceinline__ int jmap(int m) {
  return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3);
}
__device__ __forceinline__ int jmap_inv(int j) {
  return (((j >> 2) & 3) << 3) | (((j >> 4) & 1) << 2) | (j & 3);
}

typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4_t;

// Byte offset of a pointer into LDS, as DS instructions address it.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  typedef __attribute__((address_space(3))) const unsigned char lds_uchar;
  return (uint32_t)(uintptr_t)(lds_uchar*)p;
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

// Half-rows of one lane for a 32-key tile: lane (kn, kh) holds the 16-byte
// chunks 2s + kh (s = 0..S-1: the B operand of k-step s) of row kn of K, or
// of V (rows past the end of the head repeat its last row). The two lanes
// of a key read neighbouring chunks, so each load instruction touches 32
// rows in 32-byte runs.
template <int D>
struct HalfRows {
  u32x4_t q[D / 16];
};

template <int D>
__device__ __forceinline__ void load_half_rows(const HashArgs& a, const uint16_t* base, int tile,
                                               HalfRows<D>& r, int lane) {
  const int kn = lane & 31, kh = lane >> 5;
  const TileRows tr = tile_rows(a, tile);
  const int64_t row = tr.grow0 + min(kn, tr.rows - 1);
  const uint4* p = reinterpret_cast<const uint4*>(base + row * D) + kh;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const uint4 x = p[2 * s];
    r.q[s] = u32x4_t{x.x, x.y, x.z, x.w};
  }
}

// Sign bits and the certification test of a column tile's projections
// (acc, lane (kn, kh): the 16 columns ct*32 + kh*16 + v of key kn), in S
// steps of 16 / S projections each, so that every step fits beside one
// k-step of the next column tile's MFMAs: word collects the sign bits
// (complemented at the end) and mn the smallest magnitude.
struct ColSigns {
  uint32_t word;
  float mn;
};

template <int S>
__device__ __forceinline__ void col_signs_step(const f32x16_t& acc, int s, ColSigns& cs) {
  constexpr int kPer = 16 / S;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int v = 15 - (s * kPer + i);
    const float m = fabsf(acc[v]);
    cs.mn = (s == 0 && i == 0) ? m : fminf(cs.mn, m);
    cs.word = __builtin_amdgcn_alignbit((s == 0 && i == 0) ? 0u : cs.word, __float_as_uint(acc[v]), 31);
  }
  // done here, beside this k-step (not gathered after the loop)
  asm volatile("" : "+v"(cs.word), "+v"(cs.mn));
}

// The certification of column tile ct of a tile: rarely, list entries for
// uncertain signs (see the file comment). Returns h, the tile's 16 sign
// bits of the lane (bit v: projection onto column ct*32 + kh*16 + v > 0).
__device__ __forceinline__ uint32_t col_finish(const HashArgs& a, const f32x16_t& acc,
                                               const ColSigns& cs, int ct, float thr,
                                               bool row_ok, int64_t grow, int CT,
                                               uint32_t& fix_n, unsigned long long* fix_list,
                                               int lane) {
  const int kh = lane >> 5;
  const bool cand = row_ok && ct < CT && cs.mn <= thr;
  // Rare: some lanes hold projections too close to zero for their float32
  // sign. Each such key lists its group of 16 columns with the mask of
  // uncertain ones (float32 signs stay in the ids) in the wave's own
  // region: slots from a ballot prefix count, no atomics. The count runs on
  // past the capacity, which marks the wave for the exact re-hash.
  if (__ballot(cand) != 0) {
    // (values the compiler would otherwise compute once for every column
    // tile ahead of the loop and keep in registers)
    int C = a.C, khl = kh;
    asm volatile("" : "+s"(C), "+v"(khl));
    const int c0 = ct * 32 + khl * 16;
    uint32_t fm = 0;  // (built by shifts: no mask constants held in registers)
#pragma unroll
    for (int v = 15; v >= 0; --v) fm = (fm << 1) | (fabsf(acc[v]) <= thr ? 1u : 0u);
    const int valid = min(max(C - c0, 0), 16);  // columns of this lane below C
    fm &= valid >= 16 ? 0xffffu : (1u << valid) - 1u;
    if (!cand) fm = 0;
    const uint64_t bal = __ballot(fm != 0);
    const uint32_t pos =
        fix_n + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (fm != 0 && pos < a.fix_cap)
      fix_list[pos] = ((unsigned long long)grow << kEntryRowShift) |
                      ((unsigned long long)(c0 >> 4) << 16) | fm;
    fix_n += (uint32_t)__popcll(bal);
  }
  return ~cs.word & 0xffffu;
}

// The 32-bit sign words of column tiles ct (h0) and ct + 1 (h1), ct even,
// from the lane halves' 16 bits: one swap of the halves (lanes 32-63 of the
// first operand trade places with lanes 0-31 of the second) leaves the word
// of ct in lanes 0-31 and the word of ct + 1 in lanes 32-63.
__device__ __forceinline__ uint32_t pair_words(uint32_t h0, uint32_t h1) {
  const auto r = __builtin_amdgcn_permlane32_swap(h0, h1, false, false);
  // lanes 0-31: r[0] = own bits of ct, r[1] = the partner's bits of ct;
  // lanes 32-63: r[0] = the partner's bits of ct + 1, r[1] = own bits of ct + 1
  return r[0] | (r[1] << 16);
}

// Main kernel: one block of 8 waves per CU. R^T of all NCT column tiles
// sits in LDS in the order the A operand is read (fragment (ct, s) = 1 KB,
// lane l at 16*l: conflict-free 16-byte reads). Block b hashes the 32-key
// tiles b, b + grid, ...; its waves take them one at a time (the first two
// each fixed, then from a counter in LDS) and need no other wave after the
// set-up: the next tile's K half-rows are in flight into registers while
// the current one is computed; the two waves of a SIMD take turns on its
// matrix core. Per tile: the key norms, then for every column tile the S
// k-steps on the matrix cores interleaved with the sign work of the
// previous column tile, then the value norms. A wave's uncertain signs go
// to its own list region (part = block * 8 + wave); owner records the part
// of every tile for the exact re-hash.
template <int D, int NCT, bool kWordIds>
__global__ __launch_bounds__(kHashThreads, 1) void hash_keys_bf16_kernel(HashArgs a) {
  constexpr int S = D / 16;
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr float kGamma = 2.0f * D * 0x1p-24f;
  __shared__ u32x4_t frag[NCT * S * 64];
  __shared__ float rmax_s[NCT];
  __shared__ uint32_t bitvec[kWordIds ? 1 : kHashWaves * kTileKeys * kMaxColWords];
  __shared__ uint32_t tiles_taken;  // the block's tiles handed out past the first two per wave

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kn = lane & 31, kh = lane >> 5;
  const int CT = (a.C + 31) >> 5;
  const int part = blockIdx.x * kHashWaves + wave;  // this wave's list region
  // the block's tiles: blockIdx.x + j * gridDim.x, j < nblk
  const int nblk = (a.n_tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  auto block_tile = [&](int j) { return j < nblk ? (int)blockIdx.x + j * (int)gridDim.x : a.n_tiles; };
  unsigned long long* const fix_list = a.fix_list + (size_t)part * a.fix_cap;
  uint32_t fix_n = 0;  // wave-uniform count of listed entries

  // the first tile's key rows are in flight during the set-up
  HalfRows<D> ka, kb;
  load_half_rows<D>(a, a.K, min(block_tile(wave), a.n_tiles - 1), ka, lane);
  if (threadIdx.x == 0) tiles_taken = 0;

  // set-up: the fragments into LDS (a plain copy), then thread t takes the
  // squared norm of hyperplane column t; the largest of each column tile
  // (rounded up) bounds the projection errors
  for (int q = threadIdx.x; q < NCT * S * 64; q += kHashThreads) {
    const uint4 x = a.RTF[q];
    frag[q] = u32x4_t{x.x, x.y, x.z, x.w};
  }
  __syncthreads();
  for (int r = threadIdx.x; r < NCT * 32; r += kHashThreads) {
    const int ct = r >> 5, m = jmap_inv(r & 31);
    float sq = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) sq = sumsq_bf16x8(frag[(ct * S + c % S) * 64 + (c / S) * 32 + m], sq);
    const float mx = group_max<32>(sq);  // the 32 columns of the tile are 32 aligned lanes
    if ((r & 31) == 0) rmax_s[ct] = sqrtf(mx) * (1.0f + 0x1p-20f);
  }
  __syncthreads();
  const u32x4_t* const fl0 = frag + lane;

  // The ids and the value norm of a finished tile, stored in the middle of
  // the next one: a store still in flight at a wave's next wait for its
  // loads would be waited for too.
  struct Pending {
    uint32_t words[NCT / 2];
    float vn;
    int64_t grow;
    bool ok;
  } pend;
  pend.ok = false;
  auto flush = [&]() {
    if (pend.ok) {
      if (kh == 0) a.vnorm[pend.grow] = pend.vn;
      if constexpr (kWordIds) {
        // P == 8: word ct holds the id bytes of tables 4ct .. 4ct+3
        uint32_t* orow = reinterpret_cast<uint32_t*>(a.ids + pend.grow * a.L);
#pragma unroll
        for (int i = 0; i < NCT / 2; ++i) {
          const int ct = 2 * i + kh;
          if (ct < CT) orow[ct] = pend.words[i];
        }
      }
    }
    pend.ok = false;
  };

  // Tiles: the wave's first two are the block's tiles wave and wave + 8,
  // later ones are handed out by the block's counter in LDS, which balances
  // the two waves of a SIMD (the hardware serves the older one first). A
  // request is sent a tile ahead of the one whose rows it names.
  auto grab = [&]() {
    uint32_t t = 0;
    if (lane == 0) t = atomicAdd(&tiles_taken, 1u);
    return t;  // in lane 0
  };
  auto tile_of = [&](uint32_t t) {
    t = (uint32_t)__builtin_amdgcn_readfirstlane((int)t);
    return block_tile((int)min<uint32_t>(2u * kHashWaves + t, (uint32_t)nblk));
  };

  // One tile with its key rows in cur, while the key rows of tile `next`
  // load into nxt (the last tile's rows again when there is none) and the
  // tile's value rows arrive for its value norms at the end.
  auto step = [&](const HalfRows<D>& cur, HalfRows<D>& nxt, int tile, int next) {
    HalfRows<D> vr;
    load_half_rows<D>(a, a.V, tile, vr, lane);
    load_half_rows<D>(a, a.K, min(next, a.n_tiles - 1), nxt, lane);
    if (lane == 0) a.owner[tile] = part;
    const TileRows tr = tile_rows(a, tile);
    const bool row_ok = kn < tr.rows;
    const int64_t grow = tr.grow0 + kn;
    // the fragments are read again for every tile (not hoisted out of the
    // loop into registers)
    uint32_t flo = lds_offset(fl0);
    asm volatile("" : "+v"(flo));
    const lds_u32x4_t* fl = reinterpret_cast<const lds_u32x4_t*>((uintptr_t)flo);

    // key norm (each lane half holds half of the row); an upper bound is
    // enough: the hardware square root (1 ulp) rounded up
    float ks = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) ks = sumsq_bf16x8(cur.q[s], ks);
    ks += __builtin_bit_cast(float, xor32_u32(__builtin_bit_cast(uint32_t, ks)));
    const float thr_k = kGamma * 1.000001f * __builtin_amdgcn_sqrtf(ks);

    // column tiles: the k-steps of ct on the matrix cores while the signs
    // of ct - 1 are packed
    uint32_t words[NCT / 2];  // lane half kh: the words of column tiles 2i + kh
    uint32_t h_even = 0;      // sign bits of the last even column tile
    f32x16_t prev = {};
    // A fragments kAhead k-steps ahead of their MFMA (LDS latency)
    constexpr int kAhead = 3, kSteps = NCT * S;
    u32x4_t fr[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) fr[i] = fl[i * 64];
#pragma unroll
    for (int ct = 0; ct <= NCT; ++ct) {
      f32x16_t acc = {};
      ColSigns cs;
      const float rm = ct > 0 ? rmax_s[ct - 1] : 0.f;  // read early, used at the end
      if (ct == NCT / 2) flush();
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int i = ct * S + s;
        if (ct < NCT) {
          if (i + kAhead < kSteps) fr[(i + kAhead) % (kAhead + 1)] = fl[(i + kAhead) * 64];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, fr[i % (kAhead + 1)]),
              __builtin_bit_cast(bf16x8_t, cur.q[s]), acc, 0, 0, 0);
        }
        if (ct > 0) col_signs_step<S>(prev, s, cs);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ct > 0) {
        const int pc = ct - 1;
        const uint32_t h = col_finish(a, prev, cs, pc, thr_k * rm + kAbsFloor, row_ok, grow,
                                      CT, fix_n, fix_list, lane);
        if (pc % 2 == 0)
          h_even = h;
        else
          words[pc / 2] = pair_words(h_even, h);
      }
      prev = acc;
    }

    float vs = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) vs = sumsq_bf16x8(vr.q[s], vs);
    vs += __builtin_bit_cast(float, xor32_u32(__builtin_bit_cast(uint32_t, vs)));
    pend.vn = __builtin_amdgcn_sqrtf(vs);
    pend.grow = grow;
    pend.ok = row_ok;
#pragma unroll
    for (int i = 0; i < NCT / 2; ++i) pend.words[i] = words[i];

    if constexpr (!kWordIds) {
      // any P: the words through this wave's LDS rows, then id bytes
      uint32_t* bv = bitvec + wave * kTileKeys * kMaxColWords;
#pragma unroll
      for (int i = 0; i < NCT / 2; ++i) bv[kn * kMaxColWords + 2 * i + kh] = words[i];
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();
      uint8_t* obase = a.ids + tr.grow0 * a.L;
      for (int q = lane; q < kTileKeys * a.L; q += 64) {
        const int r = q / a.L, l = q - r * a.L;
        if (r < tr.rows)
          obase[(int64_t)r * a.L + l] = (uint8_t)extract_bits(bv + r * kMaxColWords, l * a.P, a.P);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
  };

  // tiles in pairs, so that the two row buffers swap roles without copies
  int t0 = block_tile(wave), t1 = block_tile(wave + kHashWaves);
  uint32_t r2 = grab();  // the tile after t1
  while (t0 < a.n_tiles) {
    step(ka, kb, t0, t1);
    t0 = t1; t1 = tile_of(r2); r2 = grab();
    if (t0 >= a.n_tiles) break;
    step(kb, ka, t0, t1);
    t0 = t1; t1 = tile_of(r2); r2 = grab();
  }
  flush();
  if (lane == 0) a.fix_count[part] = fix_n;
}

// R [d, C] -> R^T [kRtRows, d] with zero rows past C, and the same in the
// order of the main kernel's A fragments: 16-byte chunk q holds, for
// f = q / 64 = ct * S + st and l = q % 64 = h * 32 + m, elements
// (2 * st + h) * 8 .. + 7 of R^T row ct * 32 + jmap(m) (S = D / 16), the
// chunk the B operand of k-step st holds in lane half h.
__global__ __launch_bounds__(256) void hash_prep_kernel(const uint16_t* __restrict__ R, int C,
                                                        int D, uint16_t* __restrict__ RT,
                                                        uint16_t* __restrict__ RTF) {
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t total = (int64_t)kRtRows * D;
  for (int64_t i = i0; i < total; i += stride) {
    const int c = (int)(i / D), d = (int)(i % D);
    RT[i] = c < C ? R[(int64_t)d * C + c] : (uint16_t)0;
  }
  const int S = D / 16;
  for (int64_t i = i0; i < total; i += stride) {
    const int64_t q = i / 8;
    const int e = (int)(i % 8);
    const int f = (int)(q / 64), l = (int)(q % 64);
    const int ct = f / S, st = f % S, h = l / 32, m = l % 32;
    const int r = ct * 32 + jmap(m), d = (2 * st + h) * 8 + e;
    RTF[i] = r < C ? R[(int64_t)d * C + r] : (uint16_t)0;
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
constexpr int kFixBlocksPerPart = 8;

template <int D>
__device__ __forceinline__ void hash_fixup_block(
    int bid, const uint16_t* __restrict__ K, const uint16_t* __restrict__ RT, int C, int L,
    int P, uint8_t* __restrict__ ids, const unsigned long long* __restrict__ list,
    const uint32_t* __restrict__ count, uint32_t cap) {
  constexpr int kPer = D / 16;  // dims per lane: 8 (one 16-byte load) or 4
  const int blk = bid / kFixBlocksPerPart;
  const int j = bid % kFixBlocksPerPart;
  const int sub = threadIdx.x & 15;
  const uint32_t groups = blockDim.x / 16;
  // the block's regions back to back as one index range
  uint32_t n[kHashWaves], total = 0;
#pragma unroll
  for (int w = 0; w < kHashWaves; ++w) {
    // a wave whose list overflowed has all its tiles hashed again exactly
    // (below), so its entries are left alone
    const uint32_t c = count[blk * kHashWaves + w];
    n[w] = c > cap ? 0u : c;
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

// Exact re-hash of the tiles of every main-kernel wave whose list
// overflowed (count above the capacity; with capacity 0, any uncertain
// sign): one thread per (key, table) recomputes the table's P projections
// from the bf16 inputs in float64 (exact products; the sum of |products|
// bounds the rounding) or, when that cannot decide, in double-double, and
// rewrites the id byte. Each block checks 256 tiles at a time (owner: the
// wave that hashed the tile) and goes on at once when none needs it.
template <int D>
__device__ __forceinline__ void hash_redo_block(
    int bid, int nblocks, const uint16_t* __restrict__ K, const uint16_t* __restrict__ R,
    int64_t n_keys, int64_t stride, int tph, int n_tiles, int parts, int L, int P,
    uint8_t* __restrict__ ids, const uint32_t* __restrict__ count, const int* __restrict__ owner,
    uint32_t cap) {
  __shared__ int list[256];
  __shared__ int nlist;
  const int C = L * P;
  for (int64_t base = (int64_t)bid * 256; base < n_tiles; base += (int64_t)nblocks * 256) {
    const int64_t t = base + threadIdx.x;
    // (an owner outside the waves of the main kernel cannot occur; it is
    // not used as an index then)
    const int o = t < n_tiles ? owner[t] : -1;
    const bool need = (unsigned)o < (unsigned)parts && count[o] > cap;
    if (!__syncthreads_or(need)) continue;
    if (threadIdx.x == 0) nlist = 0;
    __syncthreads();
    if (need) list[atomicAdd(&nlist, 1)] = (int)t;
    __syncthreads();
    for (int e = 0; e < nlist; ++e) {
    const int tile = list[e];
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
    __syncthreads();
  }
}

// The fix-up and the exact re-hash in one launch: blocks 0 .. fix_blocks-1
// settle the listed signs, the next redo_blocks check the tiles for waves
// whose list overflowed (disjoint rows: a tile belongs to one wave).
template <int D>
__global__ __launch_bounds__(256, 8) void hash_settle_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ R,
    const uint16_t* __restrict__ RT, int64_t n_keys, int64_t stride, int tph, int n_tiles,
    int parts, int L, int P, uint8_t* __restrict__ ids,
    const unsigned long long* __restrict__ list, const uint32_t* __restrict__ count,
    const int* __restrict__ owner, uint32_t cap, int fix_blocks, int redo_blocks) {
  const int bid = (int)blockIdx.x;  // block-uniform roles
  if (bid < fix_blocks)
    hash_fixup_block<D>(bid, K, RT, L * P, L, P, ids, list, count, cap);
  else
    hash_redo_block<D>(bid - fix_blocks, redo_blocks, K, R, n_keys, stride, tph, n_tiles, parts,
                       L, P, ids, count, owner, cap);
}

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }

// The f32 path: one thread per key.
template <int D, typename T>
__global__ __launch_bounds__(256) void hash_keys_direct_kernel(
    const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ R, int64_t n_heads, int64_t n_keys,
    int64_t stride, int L, int P, uint8_t* __restrict__ ids,
    float* __restrict__ vnorm) {
  const int64_t gidx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gidx >= n_heads * n_keys) return;
  const int64_t head = gidx / n_keys, row = gidx % n_keys;
  const int64_t off = head * stride + row;
  const int C = L * P;
  constexpr double kBound = 2.0 * D * 0x1p-53;

  float kr[D];
#pragma unroll
  for (int i = 0; i < D; ++i) kr[i] = load_elem(K, off * D + i);
  double vs = 0.0;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const double v = load_elem(V, off * D + i);
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
        const double p = (double)kr[i] * (double)load_elem(R, (int64_t)i * C + c);
        y += p;
        mag += fabs(p);
      }
      if (fabs(y) <= kBound * mag) {
        double h = 0.0, lo = 0.0;
        for (int i = 0; i < D; ++i)
          dd_add(h, lo, (double)kr[i] * (double)load_elem(R, (int64_t)i * C + c), 0.0, h,
                 lo);
        y = h;
      }
      if (y > 0.0) id |= 1u << j;
    }
    ids[off * L + l] = (uint8_t)id;
  }
}

// A few bf16 keys (a decode step's appended ones): one block per key, one
// thread per hyperplane column (a second pass for C > 256). Each projection
// is the float64 sum of the exact products over the key row (staged in
// LDS) and column c of R (consecutive threads read consecutive columns),
// certified against the rounding bound of the sum of |products|, else
// recomputed in double-double; the sign bits meet in LDS and threads
// l < L write the id bytes. The value norm follows the main kernel's
// arithmetic exactly (bf16 dot2 steps over the even and over the odd
// 16-byte chunks of the row, then the two sums).
template <int D>
__global__ __launch_bounds__(256) void hash_keys_small_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ R, int64_t n_keys, int64_t stride, int L, int P,
    uint8_t* __restrict__ ids, float* __restrict__ vnorm) {
  __shared__ float kr[D];
  __shared__ uint32_t bits[kMaxColWords];
  const int64_t key = blockIdx.x;
  const int64_t off = (key / n_keys) * stride + key % n_keys;
  const int C = L * P;
  constexpr double kBound = 2.0 * D * 0x1p-53;
  const int t = threadIdx.x;
  if (t < D) kr[t] = bf16_bits_to_f32(K[off * D + t]);
  if (t < kMaxColWords) bits[t] = 0u;
  if (t == 0) {
    const u32x4_t* vrow = reinterpret_cast<const u32x4_t*>(V + off * D);
    float half[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      half[h] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) half[h] = sumsq_bf16x8(vrow[2 * c + h], half[h]);
    }
    vnorm[off] = __builtin_amdgcn_sqrtf(half[0] + half[1]);
  }
  __syncthreads();
  for (int c = t; c < C; c += blockDim.x) {
    double y = 0.0, mag = 0.0;
#pragma unroll 8
    for (int i = 0; i < D; ++i) {
      const double p = (double)kr[i] * (double)bf16_bits_to_f32(R[(int64_t)i * C + c]);
      y += p;
      mag += fabs(p);
    }
    if (fabs(y) <= kBound * mag) {
      double h = 0.0, lo = 0.0;
      for (int i = 0; i < D; ++i)
        dd_add(h, lo, (double)kr[i] * (double)bf16_bits_to_f32(R[(int64_t)i * C + c]), 0.0, h,
               lo);
      y = h;
    }
    if (y > 0.0) atomicOr(&bits[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  for (int l = t; l < L; l += blockDim.x)
    ids[off * L + l] = (uint8_t)extract_bits(bits, l * P, P);
}

// --------------------------------------------------------------- launchers

constexpr int kMaxHashBlocks = 256;  // one per CU
// bf16 inputs of at most this many keys (the keys a decode step appends,
// one per KV head) go to the one-launch direct kernel
constexpr int64_t kDirectMaxKeys = 32;

struct HashWs {
  uint16_t* rt;
  uint16_t* rtf;              // R^T in fragment order
  uint32_t* count;            // [kMaxHashBlocks * kHashWaves]
  int* owner;                 // [n_tiles]
  unsigned long long* list;   // [kMaxHashBlocks * kHashWaves][cap]
  uint32_t cap;               // entries per wave
};

int64_t hash_tiles(int64_t n_heads, int64_t n_keys) {
  return n_heads * ((n_keys + kTileKeys - 1) / kTileKeys);
}

HashWs hash_ws_layout(void* ws, int64_t n_heads, int64_t n_keys, int d, int C) {
  HashWs w{};
  unsigned char* p = static_cast<unsigned char*>(ws);
  size_t off = 0;
  w.rt = reinterpret_cast<uint16_t*>(p + off);
  off = align256(off + (size_t)kRtRows * d * sizeof(uint16_t));
  w.rtf = reinterpret_cast<uint16_t*>(p + off);
  off = align256(off + (size_t)kRtRows * d * sizeof(uint16_t));
  w.count = reinterpret_cast<uint32_t*>(p + off);
  off = align256(off + kMaxHashBlocks * kHashWaves * sizeof(uint32_t));
  w.owner = reinterpret_cast<int*>(p + off);
  off = align256(off + (size_t)hash_tiles(n_heads, n_keys) * sizeof(int));
  w.list = reinterpret_cast<unsigned long long*>(p + off);
  w.cap = hash_fix_capacity(n_heads * n_keys, C) / (kMaxHashBlocks * kHashWaves);
  return w;
}

template <int D, int NCT, bool kWordIds>
void launch_main(const HashArgs& a, int grid, hipStream_t stream) {
  launch_kernel((hash_keys_bf16_kernel<D, NCT, kWordIds>), dim3(grid), dim3(kHashThreads), 0,
                stream, a);
}

template <int D>
void launch_main_d(const HashArgs& a, int grid, bool word_ids, hipStream_t stream) {
  const int CT = (a.C + 31) / 32;
  if (CT <= 8) {
    if (word_ids) launch_main<D, 8, true>(a, grid, stream);
    else launch_main<D, 8, false>(a, grid, stream);
  } else {
    if (word_ids) launch_main<D, 16, true>(a, grid, stream);
    else launch_main<D, 16, false>(a, grid, stream);
  }
}

}  // namespace

uint32_t hash_fix_capacity(int64_t n_total, int C) {
  const int64_t want = n_total * C / 512;
  return (uint32_t)std::max<int64_t>(65536, std::min<int64_t>(want, (int64_t)1 << 26));
}

size_t hash_keys_bf16_workspace_bytes(int64_t n_heads, int64_t n_keys, int d, int C) {
  size_t off = align256((size_t)kRtRows * d * sizeof(uint16_t));
  off = align256(off + (size_t)kRtRows * d * sizeof(uint16_t));
  off = align256(off + kMaxHashBlocks * kHashWaves * sizeof(uint32_t));
  off = align256(off + (size_t)hash_tiles(n_heads, n_keys) * sizeof(int));
  const size_t parts = (size_t)kMaxHashBlocks * kHashWaves;
  return off + (hash_fix_capacity(n_heads * n_keys, C) / parts) * parts * sizeof(unsigned long long);
}

hipError_t launch_hash_keys_bf16(const uint16_t* K, const uint16_t* V,
                                 const uint16_t* R, int64_t n_heads,
                                 int64_t n_keys, int64_t stride, int d, int L,
                                 int P, uint8_t* ids, float* vnorm, void* ws,
                                 hipStream_t stream) {
  if (n_heads == 0 || n_keys == 0) return hipSuccess;
  if (n_heads * n_keys <= kDirectMaxKeys) {
    const dim3 grid((unsigned)(n_heads * n_keys));
    if (d == 128)
      launch_kernel(hash_keys_small_kernel<128>, grid, dim3(256), 0, stream, K, V, R, n_keys,
                    stride, L, P, ids, vnorm);
    else
      launch_kernel(hash_keys_small_kernel<64>, grid, dim3(256), 0, stream, K, V, R, n_keys,
                    stride, L, P, ids, vnorm);
    return hipGetLastError();
  }
  const int C = L * P;
  const int64_t tph = (n_keys + kTileKeys - 1) / kTileKeys;
  if (n_heads * tph >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const HashWs w = hash_ws_layout(ws, n_heads, n_keys, d, C);
  // the fix-up patches bits through 4-byte words inside id rows
  const bool word_rows = (L % 4 == 0) && (reinterpret_cast<uintptr_t>(ids) & 3) == 0;
  HashArgs a{};
  a.K = K;
  a.V = V;
  a.R = R;
  a.RT = w.rt;
  a.RTF = reinterpret_cast<const uint4*>(w.rtf);
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
  a.owner = w.owner;

  launch_kernel(hash_prep_kernel, dim3(256), dim3(256), 0, stream, R, C, d, w.rt, w.rtf);
  const bool word_ids = P == 8 && word_rows;
  // enough 8-wave blocks that every wave has a tile, at most one per CU
  const int blocks = (int)std::min<int64_t>((a.n_tiles + kHashWaves - 1) / kHashWaves,
                                            kMaxHashBlocks);
  if (d == 128)
    launch_main_d<128>(a, blocks, word_ids, stream);
  else
    launch_main_d<64>(a, blocks, word_ids, stream);
  // listed signs (none with a capacity of 0) and overflowed waves, one launch
  const int fix_blocks = a.fix_cap != 0 ? blocks * kFixBlocksPerPart : 0;
  const dim3 sgrid(fix_blocks + kMaxHashBlocks);
  if (d == 128)
    launch_kernel(hash_settle_kernel<128>, sgrid, dim3(256), 0, stream, K, R, w.rt, n_keys, stride,
                  a.tph, a.n_tiles, blocks * kHashWaves, L, P, ids, w.list, w.count, w.owner,
                  a.fix_cap, fix_blocks, kMaxHashBlocks);
  else
    launch_kernel(hash_settle_kernel<64>, sgrid, dim3(256), 0, stream, K, R, w.rt, n_keys, stride,
                  a.tph, a.n_tiles, blocks * kHashWaves, L, P, ids, w.list, w.count, w.owner,
                  a.fix_cap, fix_blocks, kMaxHashBlocks);
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
    launch_kernel(hash_keys_direct_kernel<128, float>, dim3(grid), dim3(256), 0,
                  stream, K, V, R, n_heads, n_keys, stride, L, P, ids, vnorm);
  else
    launch_kernel(hash_keys_direct_kernel<64, float>, dim3(grid), dim3(256), 0,
                  stream, K, V, R, n_heads, n_keys, stride, L, P, ids, vnorm);
  return hipGetLastError();
}

}  // namespace socket_lsh

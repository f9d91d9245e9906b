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
// bf16 path (the large prefill): the projection y = K R is a GEMM on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, float32 accumulation of the
// exact bf16 products). Each wave keeps 128 hyperplane columns of R^T in
// registers as the stationary A operand; a 32-key tile of K is staged once
// in LDS and read by every wave as the B operand, so D = y^T lands with one
// key per lane column. The sign of a projection is certified when |y| is
// larger than the worst-case float32 summation error 2*d*2^-24*|k|*|r|;
// otherwise the wave recomputes that projection cooperatively in
// double-double arithmetic from the bf16 inputs (exact products), so the
// bucket ids equal those of the exact dot products. Sign bits are packed
// with one cross-lane exchange, assembled per key in LDS and written as
// bytes. The value rows of the same tile stream through registers for the
// norms.
//
// f32 path (small inputs): one thread per key, float64 dot products with the
// same certification and a serial double-double fallback.

#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace socket_lsh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTileKeys = 32;
constexpr int kTilesPerWave = 4;    // 4 x 32 = 128 hyperplane columns per wave
constexpr int kMaxColWords = 16;    // L*P <= 512 bits per key
constexpr float kAbsFloor = 0x1p-100f;  // covers flushed float32 denormals

template <int D>
struct HashGeom {
  static constexpr int S = D / 16;              // MFMA k-steps of 16
  static constexpr int chunks = D / 8;          // 16-byte chunks per bf16 row
  static constexpr int lds_stride = 2 * D + 16; // padded LDS row (bank spread)
};

__device__ __forceinline__ float sumsq8_bf16(const uint4& w) {
  float f[8];
  unpack8_bf16(w, f);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fmaf(f[i], f[i], s);
  return s;
}

// P bits starting at bit `off` of a per-key bit vector.
__device__ __forceinline__ uint32_t extract_bits(const uint32_t* row, int off,
                                                 int P) {
  const int w = off >> 5, b = off & 31;
  uint64_t x = row[w];
  if (b + P > 32) x |= (uint64_t)row[w + 1] << 32;
  return (uint32_t)(x >> b) & ((1u << P) - 1u);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void hash_keys_bf16_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ R, int64_t n_keys, int64_t stride, int L,
    int P, uint8_t* __restrict__ ids, float* __restrict__ vnorm,
    int64_t n_tiles, int64_t tiles_per_head, int word_store) {
  using Geo = HashGeom<D>;
  constexpr int NT = NW * 64;
  constexpr int S = Geo::S;
  constexpr int CH = Geo::chunks;
  constexpr int TILE_CHUNKS = kTileKeys * CH;
  constexpr int PER = (TILE_CHUNKS + NT - 1) / NT;
  constexpr float kGamma = 2.0f * D * 0x1p-24f;

  __shared__ __align__(16) unsigned char ktile[kTileKeys * Geo::lds_stride];
  __shared__ uint32_t bitvec[kTileKeys * kMaxColWords];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kn = lane & 31;  // key (B column) / hyperplane (A row) of this lane
  const int kh = lane >> 5;  // which half of the reduction dimension
  const int C = L * P;
  const int CT = (C + 31) >> 5;

  // Stationary A operand: R^T columns (wave*4 + t)*32 + kn. The reduction
  // index of k-step s, lane half kh, element e is d = (kh*S + s)*8 + e; the
  // B operand below uses the same map, so the product is the plain dot.
  bf16x8_t ra[kTilesPerWave][S];
  float rmax[kTilesPerWave];
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    const int col = (wave * kTilesPerWave + t) * 32 + kn;
    float sq = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int dd = (kh * S + s) * 8 + e;
        uint32_t lo = col < C ? R[(int64_t)dd * C + col] : 0u;
        uint32_t hi = col < C ? R[(int64_t)(dd + 1) * C + col] : 0u;
        float flo = bf16_bits_to_f32(lo), fhi = bf16_bits_to_f32(hi);
        sq = fmaf(flo, flo, sq);
        sq = fmaf(fhi, fhi, sq);
        w[e >> 1] = lo | (hi << 16);
      }
      u32x4_t v = {w[0], w[1], w[2], w[3]};
      ra[t][s] = __builtin_bit_cast(bf16x8_t, v);
    }
    sq += __shfl_xor(sq, 32, kWave);
    rmax[t] = sqrtf(group_max<64>(sq));
  }

  uint4 kreg[PER], vreg[PER];
  auto load_tile = [&](int64_t tile) {
    const int64_t head = tile / tiles_per_head;
    const int64_t row0 = (tile % tiles_per_head) * kTileKeys;
    const int rows = (int)min<int64_t>(kTileKeys, n_keys - row0);
    const uint16_t* kb = K + (head * stride + row0) * D;
    const uint16_t* vb = V + (head * stride + row0) * D;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int q = tid + p * NT;
      const int r = q / CH, c = q % CH;
      const bool ok = q < TILE_CHUNKS && r < rows;
      kreg[p] = ok ? *reinterpret_cast<const uint4*>(kb + r * D + c * 8)
                   : make_uint4(0, 0, 0, 0);
      vreg[p] = ok ? *reinterpret_cast<const uint4*>(vb + r * D + c * 8)
                   : make_uint4(0, 0, 0, 0);
    }
  };

  int64_t tile = blockIdx.x;
  if (tile >= n_tiles) return;
  load_tile(tile);

  for (; tile < n_tiles; tile += gridDim.x) {
    const int64_t head = tile / tiles_per_head;
    const int64_t row0 = (tile % tiles_per_head) * kTileKeys;
    const int rows = (int)min<int64_t>(kTileKeys, n_keys - row0);

    // Stage K in LDS; reduce the value norms of the tile.
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int q = tid + p * NT;
      const int r = q / CH, c = q % CH;
      float s = group_sum<CH>(sumsq8_bf16(vreg[p]));
      if (q < TILE_CHUNKS) {
        *reinterpret_cast<uint4*>(ktile + r * Geo::lds_stride + c * 16) = kreg[p];
        if (c == 0 && r < rows) vnorm[head * stride + row0 + r] = sqrtf(s);
      }
    }
    __syncthreads();

    const int64_t next = tile + gridDim.x;
    if (next < n_tiles) load_tile(next);

    f32x16_t acc[kTilesPerWave];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) acc[t] = f32x16_t{};
    float ksq = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint4 kb = *reinterpret_cast<const uint4*>(
          ktile + kn * Geo::lds_stride + (kh * S + s) * 16);
      ksq += sumsq8_bf16(kb);
      u32x4_t kv = {kb.x, kb.y, kb.z, kb.w};
      const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, kv);
#pragma unroll
      for (int t = 0; t < kTilesPerWave; ++t) {
        if (wave * kTilesPerWave + t < CT)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[t][s], bop,
                                                           acc[t], 0, 0, 0);
      }
    }
    ksq += __shfl_xor(ksq, 32, kWave);
    const float thr_k = kGamma * sqrtf(ksq);
    const bool row_ok = kn < rows;

#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int ct = wave * kTilesPerWave + t;
      if (ct >= CT) break;
      // D layout: lane (kn, kh), register v holds hyperplane row
      // (v/4)*8 + kh*4 + v%4 of the tile for key kn.
      const float thr = thr_k * rmax[t] + kAbsFloor;
      // only real keys and real hyperplane columns (padding columns are zero)
      uint32_t fm = 0;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int colv = ct * 32 + (v >> 2) * 8 + kh * 4 + (v & 3);
        if (row_ok && colv < C && fabsf(acc[t][v]) <= thr) fm |= 1u << v;
      }
      // Re-evaluate uncertain signs, one projection per wave iteration.
      while (true) {
        const uint64_t act = __ballot(fm != 0);
        if (act == 0) break;
        const int src = __ffsll((unsigned long long)act) - 1;
        const uint32_t sfm = __shfl(fm, src, kWave);
        const int vsel = __ffs(sfm) - 1;
        const int en = src & 31, eh = src >> 5;
        const int col = ct * 32 + (vsel >> 2) * 8 + eh * 4 + (vsel & 3);
        double h = 0.0, l = 0.0;
        for (int i = lane; i < D; i += kWave) {
          const uint16_t kb16 = *reinterpret_cast<const uint16_t*>(
              ktile + en * Geo::lds_stride + i * 2);
          const double prod = (double)bf16_bits_to_f32(kb16) *
                              (double)bf16_bits_to_f32(R[(int64_t)i * C + col]);
          dd_add(h, l, prod, 0.0, h, l);
        }
        const double y = wave_sum_dd(h, l);
        if (lane == src) {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (v == vsel) acc[t][v] = y > 0.0 ? 1.0f : -1.0f;
          fm &= ~(1u << vsel);
        }
      }
      uint32_t word = 0;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        word |= (acc[t][v] > 0.f ? 1u : 0u) << ((v >> 2) * 8 + kh * 4 + (v & 3));
      word |= __shfl_xor(word, 32, kWave);
      if (kh == 0) bitvec[kn * kMaxColWords + ct] = word;
    }
    __syncthreads();

    // Bucket ids: bits [l*P, l*P + P) of each key's bit vector.
    uint8_t* obase = ids + (head * stride + row0) * L;
    if (word_store) {
      const int wpk = L >> 2;
      for (int q = tid; q < kTileKeys * wpk; q += NT) {
        const int r = q / wpk, w4 = q % wpk;
        if (r >= rows) continue;
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          packed |= extract_bits(bitvec + r * kMaxColWords, (w4 * 4 + e) * P, P)
                    << (8 * e);
        *reinterpret_cast<uint32_t*>(obase + (int64_t)r * L + w4 * 4) = packed;
      }
    } else {
      for (int q = tid; q < kTileKeys * L; q += NT) {
        const int r = q / L, l = q % L;
        if (r >= rows) continue;
        obase[(int64_t)r * L + l] =
            (uint8_t)extract_bits(bitvec + r * kMaxColWords, l * P, P);
      }
    }
    __syncthreads();
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

template <int D, int NW>
hipError_t launch_bf16_nw(const uint16_t* K, const uint16_t* V,
                          const uint16_t* R, int64_t n_keys, int64_t stride,
                          int L, int P, uint8_t* ids, float* vnorm,
                          int64_t n_tiles, int64_t tph, int word_store,
                          hipStream_t stream) {
  // about 8 waves per CU on 256 CUs; each block loops over tiles
  const int64_t cap = (int64_t)256 * 8 / NW;
  const int grid = (int)std::min<int64_t>(n_tiles, cap);
  launch_kernel((hash_keys_bf16_kernel<D, NW>), dim3(grid), dim3(NW * 64),
                     0, stream, K, V, R, n_keys, stride, L, P, ids, vnorm,
                     n_tiles, tph, word_store);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_d(const uint16_t* K, const uint16_t* V,
                         const uint16_t* R, int64_t n_keys, int64_t stride,
                         int L, int P, uint8_t* ids, float* vnorm,
                         int64_t n_tiles, int64_t tph, int word_store,
                         hipStream_t stream) {
  const int CT = (L * P + 31) / 32;
  const int NW = (CT + kTilesPerWave - 1) / kTilesPerWave;
  switch (NW) {
#define SOCKET_NW_CASE(n)                                                    \
  case n:                                                                    \
    return launch_bf16_nw<D, n>(K, V, R, n_keys, stride, L, P, ids, vnorm,   \
                                n_tiles, tph, word_store, stream);
    SOCKET_NW_CASE(1)
    SOCKET_NW_CASE(2)
    SOCKET_NW_CASE(3)
    SOCKET_NW_CASE(4)
#undef SOCKET_NW_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_hash_keys_bf16(const uint16_t* K, const uint16_t* V,
                                 const uint16_t* R, int64_t n_heads,
                                 int64_t n_keys, int64_t stride, int d, int L,
                                 int P, uint8_t* ids, float* vnorm,
                                 hipStream_t stream) {
  if (n_heads == 0 || n_keys == 0) return hipSuccess;
  const int64_t tph = (n_keys + kTileKeys - 1) / kTileKeys;
  const int64_t n_tiles = n_heads * tph;
  const int word_store =
      (L % 4 == 0 && (reinterpret_cast<uintptr_t>(ids) & 3) == 0) ? 1 : 0;
  if (d == 128)
    return launch_bf16_d<128>(K, V, R, n_keys, stride, L, P, ids, vnorm,
                              n_tiles, tph, word_store, stream);
  return launch_bf16_d<64>(K, V, R, n_keys, stride, L, P, ids, vnorm, n_tiles,
                           tph, word_store, stream);
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
                       stream, K, V, R, n_heads, n_keys, stride, L, P, ids,
                       vnorm);
  else
    launch_kernel(hash_keys_f32_kernel<64>, dim3(grid), dim3(256), 0,
                       stream, K, V, R, n_heads, n_keys, stride, L, P, ids,
                       vnorm);
  return hipGetLastError();
}

}  // namespace socket_lsh

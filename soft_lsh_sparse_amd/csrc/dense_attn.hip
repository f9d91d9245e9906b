// Dense flash-decode attention: the baseline SOCKET is compared against.
//
// SOCKET's speed-up is stated against dense FlashAttention decoding (page
// "Resumen Técnico: SOCKET - Estimador de Núcleo de Colisión Suave para
// Atención Escasa", section "Resultados Experimentales", item Eficiencia;
// German page "SOCKET: SOft Collision Kernel EsTimator for Sparse
// Attention", section "Experimentelle Ergebnisse"): every query attends to
// all n cached keys with the exact softmax. This kernel computes that on
// the same GPU and data layout as the sparse path, so both are timed on one
// harness.
//
// Split-k decoding with the GQA group shared: each block takes one KV head
// (b, g) and a chunk of consecutive keys for all G query heads of the group,
// so every K and V row is read from memory once per group (the sparse path
// reads the rows each query head selected). Each of the 4 waves streams
// its share of the chunk with 16-byte loads (one row per LPR lanes, whole
// 1 KB runs of consecutive rows per load instruction, the next batch in
// flight while one is used), keeps a running softmax per head, and the
// block merges its waves in LDS. The chunk partials (m, l, acc[d]) of each
// query row are merged by the sparse path's merge kernel, in chunk order.
// Everything accumulates in float32 in a fixed order.

#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace socket_lsh {
namespace {

constexpr int kDenseThreads = 256;
constexpr int kDenseWaves = kDenseThreads / 64;
constexpr int kDenseKeysPerWave = 256;
constexpr int kDenseChunk = kDenseKeysPerWave * kDenseWaves;

template <typename T>
__device__ __forceinline__ void unpack16d(const uint4& w, float* f);
template <>
__device__ __forceinline__ void unpack16d<BF16>(const uint4& w, float* f) {
  unpack8_bf16(w, f);
}
template <>
__device__ __forceinline__ void unpack16d<F32>(const uint4& w, float* f) {
  unpack4_f32(w, f);
}

// G query heads per KV head; IT loads per tensor and batch. INDEXED: the n
// keys of KV head gi are the rows idx[gi * n + i] (a shared index set of the
// group, each in [0, stride)) instead of rows 0..n-1.
template <typename T, int D, int G, int IT, bool INDEXED>
__global__ __launch_bounds__(kDenseThreads) void dense_attn_kernel(
    const typename T::storage* __restrict__ Q, const typename T::storage* __restrict__ K,
    const typename T::storage* __restrict__ V, int Hq, int Hkv, int64_t stride, int64_t n,
    int chunks, const int32_t* __restrict__ idx, float* __restrict__ partial) {
  constexpr int EPL = 16 / T::bytes;  // elements per 16-byte load
  constexpr int LPR = D / EPL;        // lanes per key row
  constexpr int KPI = 64 / LPR;       // key rows per wave-wide load
  constexpr int KPB = IT * KPI;       // keys per batch
  constexpr int NB = kDenseKeysPerWave / KPB;
  static_assert(NB * KPB == kDenseKeysPerWave, "keys per wave");
  __shared__ float sm_m[G][kDenseWaves], sm_l[G][kDenseWaves];
  __shared__ float sm_acc[G][kDenseWaves][D];

  const int gi = blockIdx.x / chunks, chunk = blockIdx.x % chunks;  // gi = b * Hkv + g
  const int b = gi / Hkv, g = gi % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / LPR, sub = lane % LPR;
  const float scale = 1.0f / sqrtf((float)D);

  float qf[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int64_t row = (int64_t)b * Hq + g * G + j;
    const uint4 w = *reinterpret_cast<const uint4*>(Q + row * D + sub * EPL);
    unpack16d<T>(w, qf[j]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[j][e] *= scale;
  }

  const typename T::storage* Kh = K + (int64_t)gi * stride * D + sub * EPL;
  const typename T::storage* Vh = V + (int64_t)gi * stride * D + sub * EPL;
  const int64_t wbeg = (int64_t)chunk * kDenseChunk + wave * kDenseKeysPerWave;
  // INDEXED: the wave's key rows, one position per lane and register
  // (positions past n repeat the last one; rows are clamped into the head)
  constexpr int NREG = kDenseKeysPerWave / 64;
  int ireg[NREG];
  if constexpr (INDEXED) {
    const int32_t* irow = idx + (int64_t)gi * n;
#pragma unroll
    for (int r = 0; r < NREG; ++r) {
      const int64_t p = min<int64_t>(wbeg + r * 64 + lane, n - 1);
      ireg[r] = (int)min<int64_t>(max(irow[p], 0), stride - 1);
    }
  }
  auto row_of = [&](int bt, int it) -> int64_t {
    if constexpr (INDEXED) {
      const int p = bt * KPB + it * KPI + grp;  // position within the wave
      return __shfl(ireg[p >> 6], p & 63, kWave);
    } else {
      return min<int64_t>(wbeg + bt * KPB + it * KPI + grp, n - 1);
    }
  };

  // Batches of KPB consecutive keys, double-buffered. Keys past n are
  // loaded as row n - 1 (inside the head) and get weight 0.
  uint4 kr[2][IT], vr[2][IT];
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
  }
  auto issue = [&](int bt) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int64_t key = row_of(bt, it);
      kr[bt & 1][it] = *reinterpret_cast<const uint4*>(Kh + key * D);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int64_t key = row_of(bt, it);
      vr[bt & 1][it] = *reinterpret_cast<const uint4*>(Vh + key * D);
    }
  };

  if (wbeg < n) {
    issue(0);
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) {
      if (bt + 1 < NB) issue(bt + 1);
      if (wbeg + bt * KPB >= n) continue;  // wave-uniform: past the last key
      float s[G][IT];
      float mb[G];
#pragma unroll
      for (int j = 0; j < G; ++j) mb[j] = -INFINITY;
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        float f[EPL];
        unpack16d<T>(kr[bt & 1][it], f);
        const bool valid = wbeg + bt * KPB + it * KPI + grp < n;
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float dot = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) dot = fmaf(qf[j][e], f[e], dot);
          dot = lane_group_sum<LPR>(dot);
          s[j][it] = valid ? dot : -INFINITY;
          mb[j] = fmaxf(mb[j], s[j][it]);
        }
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        // the key groups of the wave hold different keys: combine across them
        if constexpr (LPR <= 8) mb[j] = fmaxf(mb[j], xor_lanes<8>(mb[j]));
        if constexpr (LPR <= 16) mb[j] = fmaxf(mb[j], xor_lanes<16>(mb[j]));
        if constexpr (LPR <= 32) mb[j] = fmaxf(mb[j], xor_lanes<32>(mb[j]));
        const float mn = fmaxf(m[j], mb[j]);
        const float c = m[j] == -INFINITY ? 0.f : __expf(m[j] - mn);
        l[j] *= c;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] *= c;
        m[j] = mn;
      }
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        float f[EPL];
        unpack16d<T>(vr[bt & 1][it], f);
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float p = s[j][it] == -INFINITY ? 0.f : __expf(s[j][it] - m[j]);
          l[j] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(p, f[e], acc[j][e]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    if constexpr (LPR <= 8) {
      l[j] += xor_lanes<8>(l[j]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] += xor_lanes<8>(acc[j][e]);
    }
    if constexpr (LPR <= 16) {
      l[j] += xor_lanes<16>(l[j]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] += xor_lanes<16>(acc[j][e]);
    }
    if constexpr (LPR <= 32) {
      l[j] += xor_lanes<32>(l[j]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] += xor_lanes<32>(acc[j][e]);
    }
    if (lane == 0) {
      sm_m[j][wave] = m[j];
      sm_l[j][wave] = l[j];
    }
    if (grp == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[j][wave][sub * EPL + e] = acc[j][e];
    }
  }
  __syncthreads();

  for (int q = threadIdx.x; q < G * D; q += kDenseThreads) {
    const int j = q / D, t = q % D;
    const int64_t row = (int64_t)b * Hq + g * G + j;
    float* out = partial + (row * chunks + chunk) * (D + 2);
    float mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDenseWaves; ++w) mt = fmaxf(mt, sm_m[j][w]);
    float lt = 0.f, at = 0.f;
#pragma unroll
    for (int w = 0; w < kDenseWaves; ++w) {
      const float c = sm_m[j][w] == -INFINITY ? 0.f : expf(sm_m[j][w] - mt);
      lt = fmaf(c, sm_l[j][w], lt);
      at = fmaf(c, sm_acc[j][w][t], at);
    }
    out[t] = at;
    if (t == 0) {
      out[D] = mt;
      out[D + 1] = lt;
    }
  }
}

typedef __bf16 bf16x8_d __attribute__((ext_vector_type(8)));
typedef float f32x4_d __attribute__((ext_vector_type(4)));

// Maximum over each aligned row of 16 lanes, in every lane of the row
// (quad swaps, then the half-row and row mirrors).
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
  return v;
}

// bf16 variant on the matrix cores. Each wave takes its keys in tiles of
// 16: the scores of the tile are one v_mfma_f32_16x16x32_bf16 chain over
// D/32 slabs of the dimension, A = the group's query rows (rows G..15 zero),
// B = the tile's key rows, loaded 16 bytes per lane straight into the B
// layout (lane i: key i mod 16, dimensions 8 (i / 16) .. + 7 of the slab).
// Lane i then holds the score of key i mod 16 for heads 4 (i / 16) + r,
// r = 0..3, in its four accumulators. The running softmax is updated once
// per tile (row maxima by DPP); the value rows are read 16 bytes per lane
// as in the float path, and each lane fetches the weight of its key from
// the lane that holds it (one shuffle per head and load), so the weighted
// sum of the values stays in float32. Products of bf16 values are exact in
// float32, so the scores differ from the float path's only in the order of
// the float32 additions.
template <int D, int G, bool INDEXED>
__global__ __launch_bounds__(kDenseThreads, 2) void dense_mfma_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int Hq, int Hkv, int64_t stride, int64_t n, int chunks,
    const int32_t* __restrict__ idx, float* __restrict__ partial, int jobs) {
  static_assert(G <= 8, "two rows of 16 lanes hold the heads");
  constexpr int SL = D / 32;            // slabs of the score product
  constexpr int LPR = D / 8;            // lanes per value row
  constexpr int KPI = 64 / LPR;         // value rows per load
  constexpr int VIT = 16 / KPI;         // value loads per tile
  constexpr int NTILE = kDenseKeysPerWave / 16;
  __shared__ float sm_m[G][kDenseWaves], sm_l[G][kDenseWaves];
  __shared__ float sm_acc[G][kDenseWaves][D];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // persistent blocks: block i takes the jobs (KV head, chunk) i, i + grid, ...
  for (int job = blockIdx.x; job < jobs; job += gridDim.x) {  // block-uniform
  const int gi = job / chunks, chunk = job % chunks;  // gi = b * Hkv + g
  const int b = gi / Hkv, g = gi % Hkv;
  const int col = lane & 15, quarter = lane >> 4;   // score layout
  const int grp = lane / LPR, sub = lane % LPR;     // value layout
  const float scale = 1.0f / sqrtf((float)D);

  // A operand: row `col` = query head col of the group (zero past G),
  // dimensions 32 s + 8 quarter .. + 7
  bf16x8_d qa[SL];
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (col < G)
      w = *reinterpret_cast<const uint4*>(Q + ((int64_t)b * Hq + g * G + col) * D + s * 32 +
                                          quarter * 8);
    qa[s] = __builtin_bit_cast(bf16x8_d, w);
  }

  const uint16_t* Kh = K + (int64_t)gi * stride * D;
  const uint16_t* Vh = V + (int64_t)gi * stride * D;
  // Key positions: tile t of wave w of chunk c holds positions
  // ((t * 4 + w) * chunks + c) * 16 + 0..15, so the blocks working on a head
  // at the same time read neighbouring 4 KB pieces of its rows (contiguous
  // chunks per block read a quarter slower). Every position of the head
  // belongs to exactly one (chunk, wave, tile); softmax partials do not
  // depend on which keys a chunk holds.
  // (32-bit: n <= 2^20)
  const int pbase = (wave * chunks + chunk) * 16, tstride = kDenseWaves * chunks * 16;
  auto pos_of = [&](int p) -> int {  // p = t * 16 + e, the wave's own
    return pbase + (p >> 4) * tstride + (p & 15);
  };
  const int nlast = (int)n - 1;
  constexpr int NREG = kDenseKeysPerWave / 64;
  int ireg[NREG];
  if constexpr (INDEXED) {
    const int32_t* irow = idx + (int64_t)gi * n;
#pragma unroll
    for (int r = 0; r < NREG; ++r) {
      const int p = min(pos_of(r * 64 + lane), nlast);
      ireg[r] = (int)min<int64_t>(max(irow[p], 0), stride - 1);
    }
  }
  // row of the key at wave position p (< 256); positions past n read row
  // n - 1 (inside the head) and weigh nothing
  auto row_of = [&](int p) -> int64_t {
    if constexpr (INDEXED) return __shfl(ireg[p >> 6], p & 63, kWave);
    else return min(pos_of(p), nlast);
  };

  // two buffers, the next tile in flight while one is used; the tile loop
  // is unrolled, so every buffer index is a constant (registers, not
  // scratch) and the loop has no branch at which the compiler would wait
  // for every load in flight
  uint4 kb[2][SL], vb[2][VIT];
  auto issue = [&](int t, uint4 (&kb)[SL], uint4 (&vb)[VIT]) {
    const int64_t kr = row_of(t * 16 + col);
#pragma unroll
    for (int s = 0; s < SL; ++s)
      kb[s] = *reinterpret_cast<const uint4*>(Kh + kr * D + s * 32 + quarter * 8);
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int64_t vr = row_of(t * 16 + it * KPI + grp);
      vb[it] = *reinterpret_cast<const uint4*>(Vh + vr * D + sub * 8);
    }
  };

  float m[G], lp[4], acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) lp[r] = 0.f;  // this lane's share of l, head 4 quarter + r

  auto tile = [&](int t, const uint4 (&kb)[SL], const uint4 (&vb)[VIT]) {
    f32x4_d c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SL; ++s)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], __builtin_bit_cast(bf16x8_d, kb[s]), c,
                                                0, 0, 0);
    const bool valid = pos_of(t * 16 + col) < n;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = valid ? c[r] * scale : -INFINITY;
    // tile maxima of the heads (rows of 16 lanes), then the running state
    float mrow[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) mrow[r] = max16(sc[r]);
    float cf[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mb = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mrow[j & 3]), (j >> 2) * 16));
      const float mn = fmaxf(m[j], mb);
      cf[j] = m[j] == -INFINITY ? 0.f : __expf(m[j] - mn);
      m[j] = mn;
    }
    // weights of this lane's four scores (heads 4 quarter + r)
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = quarter * 4 + r;
      float mj = m[0], cj = cf[0];
#pragma unroll
      for (int jj = 1; jj < G; ++jj)
        if (j == jj) {
          mj = m[jj];
          cj = cf[jj];
        }
      pr[r] = (j < G && sc[r] != -INFINITY) ? __expf(sc[r] - mj) : 0.f;
      lp[r] = lp[r] * cj + pr[r];
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] *= cf[j];
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      float f[8];
      unpack8_bf16(vb[it], f);
      const int key = it * KPI + grp;  // in the tile
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float p = __shfl(pr[j & 3], (j >> 2) * 16 + key, kWave);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(p, f[e], acc[j][e]);
      }
    }
  };

  if (pbase < (int)n) {  // wave-uniform: else every position of the wave is past n
    issue(0, kb[0], vb[0]);
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      if (t + 1 < NTILE) issue(t + 1, kb[(t + 1) % 2], vb[(t + 1) % 2]);
      tile(t, kb[t % 2], vb[t % 2]);
    }
  }
  // l of every head: the lanes of its row hold the parts
  float lsum[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float part = lane_group_sum<16>(lp[j & 3]);
    lsum[j] = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, part), (j >> 2) * 16));
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    if constexpr (LPR <= 8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] += xor_lanes<8>(acc[j][e]);
    }
    if constexpr (LPR <= 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] += xor_lanes<16>(acc[j][e]);
    }
    if constexpr (LPR <= 32) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] += xor_lanes<32>(acc[j][e]);
    }
    if (lane == 0) {
      sm_m[j][wave] = m[j];
      sm_l[j][wave] = lsum[j];
    }
    if (grp == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[j][wave][sub * 8 + e] = acc[j][e];
    }
  }
  __syncthreads();

  for (int q = threadIdx.x; q < G * D; q += kDenseThreads) {
    const int j = q / D, tt = q % D;
    const int64_t row = (int64_t)b * Hq + g * G + j;
    float* out = partial + (row * chunks + chunk) * (D + 2);
    float mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDenseWaves; ++w) mt = fmaxf(mt, sm_m[j][w]);
    float lt = 0.f, at = 0.f;
#pragma unroll
    for (int w = 0; w < kDenseWaves; ++w) {
      const float c = sm_m[j][w] == -INFINITY ? 0.f : expf(sm_m[j][w] - mt);
      lt = fmaf(c, sm_l[j][w], lt);
      at = fmaf(c, sm_acc[j][w][tt], at);
    }
    out[tt] = at;
    if (tt == 0) {
      out[D] = mt;
      out[D + 1] = lt;
    }
  }
  __syncthreads();  // the LDS partials are read before the next job writes them
  }
}

template <typename T, int D, int G>
hipError_t launch_dense_g(const void* Q, const void* K, const void* V, const DensePlan& p,
                          int64_t stride, const int32_t* idx, void* out, float* partial,
                          hipStream_t stream) {
  using S = typename T::storage;
  constexpr int IT = G >= 4 ? 4 : 8;
  if constexpr (T::bytes == 2) {
    // as many blocks as the CUs hold at once (two per CU)
    const int jobs = p.B * p.Hkv * p.chunks;
    const int grid = std::min(jobs, 256 * 2);
    if (idx != nullptr)
      launch_kernel((dense_mfma_kernel<D, G, true>), dim3(grid), dim3(kDenseThreads), 0, stream,
                    (const S*)Q, (const S*)K, (const S*)V, p.Hq, p.Hkv, stride, p.n, p.chunks,
                    idx, partial, jobs);
    else
      launch_kernel((dense_mfma_kernel<D, G, false>), dim3(grid), dim3(kDenseThreads), 0, stream,
                    (const S*)Q, (const S*)K, (const S*)V, p.Hq, p.Hkv, stride, p.n, p.chunks,
                    idx, partial, jobs);
  } else if (idx != nullptr)
    launch_kernel((dense_attn_kernel<T, D, G, IT, true>), dim3(p.B * p.Hkv * p.chunks),
                  dim3(kDenseThreads), 0, stream, (const S*)Q, (const S*)K, (const S*)V, p.Hq,
                  p.Hkv, stride, p.n, p.chunks, idx, partial);
  else
    launch_kernel((dense_attn_kernel<T, D, G, IT, false>), dim3(p.B * p.Hkv * p.chunks),
                  dim3(kDenseThreads), 0, stream, (const S*)Q, (const S*)K, (const S*)V, p.Hq,
                  p.Hkv, stride, p.n, p.chunks, idx, partial);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_attn_merge(partial, p.B * p.Hq, p.chunks, p.d, T::bytes == 2, out, stream);
}

template <typename T, int D>
hipError_t launch_dense_d(const void* Q, const void* K, const void* V, const DensePlan& p,
                          int64_t stride, const int32_t* idx, void* out, float* partial,
                          hipStream_t stream) {
  switch (p.Hq / p.Hkv) {
    case 1: return launch_dense_g<T, D, 1>(Q, K, V, p, stride, idx, out, partial, stream);
    case 2: return launch_dense_g<T, D, 2>(Q, K, V, p, stride, idx, out, partial, stream);
    case 4: return launch_dense_g<T, D, 4>(Q, K, V, p, stride, idx, out, partial, stream);
    default: return launch_dense_g<T, D, 8>(Q, K, V, p, stride, idx, out, partial, stream);
  }
}

}  // namespace

DensePlan plan_dense(int B, int Hq, int Hkv, int d, int64_t n) {
  DensePlan p{};
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.d = d;
  p.n = n;
  p.chunks = (int)std::max<int64_t>(1, (n + kDenseChunk - 1) / kDenseChunk);
  p.partial_bytes = (size_t)B * Hq * p.chunks * (d + 2) * sizeof(float);
  return p;
}

hipError_t launch_dense_attn(const void* Q, const void* K, const void* V, bool bf16,
                             const DensePlan& p, int64_t stride, const int32_t* idx, void* out,
                             float* partial, hipStream_t stream) {
  if (p.B == 0 || p.Hq == 0) return hipSuccess;
  if (bf16) {
    if (p.d == 128)
      return launch_dense_d<BF16, 128>(Q, K, V, p, stride, idx, out, partial, stream);
    return launch_dense_d<BF16, 64>(Q, K, V, p, stride, idx, out, partial, stream);
  }
  if (p.d == 128) return launch_dense_d<F32, 128>(Q, K, V, p, stride, idx, out, partial, stream);
  return launch_dense_d<F32, 64>(Q, K, V, p, stride, idx, out, partial, stream);
}

}  // namespace socket_lsh

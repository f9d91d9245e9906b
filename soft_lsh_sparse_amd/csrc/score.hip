// Soft collision scores.
//
// Step 3 of the soft-LSH mechanism of SOCKET (page "Resumen Técnico: SOCKET -
// Estimador de Núcleo de Colisión Suave para Atención Escasa", section
// "Mecanismo Central: LSH Suave", item 3; German page "SOCKET: SOft Collision
// Kernel EsTimator for Sparse Attention", Kernmechanismus, Bewertung): every
// key is scored by the probability mass the query puts on the key's own
// bucket, summed over the L tables and weighted by the key's value norm.
//
// One block owns one (batch, KV head) and a contiguous range of keys. It
// stages that head's probability table [2^P][L][G] (float32) in LDS, then
// streams the bucket-id rows (L bytes per key, coalesced across lanes) and
// the value norms from HBM. Each id byte is looked up once for the whole GQA
// group: the G probabilities of the group sit in one 16-byte LDS slot.
//
// Bank spread: with the [u][l][G] layout and L a multiple of 16, the LDS bank
// of slot (u, l) depends only on l mod 16. Lane i walks the tables in the
// rotated order l = (t + n) mod L for its key n (n mod 16 = i mod 16), so the
// 16 lanes served together hit 16 different bank groups whatever buckets the
// keys fall in. The rotation is applied to the id bytes in registers once
// per key. The L probabilities are summed in float32 in that fixed order and
// multiplied by the value norm.
//
// Optionally the kernel also counts every score in a 2048-bin histogram of
// the top 11 bits of its order key (the first pass of the top-k radix
// select): per-block counts are kept in LDS as packed 16-bit pairs (a block
// never scores more than 32768 keys per row) and added to the per-row global
// histogram with integer atomics, which makes the result order-independent.

#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace socket_lsh {
namespace {

constexpr int kScoreThreads = 512;
constexpr int64_t kMaxSegForHist = 32768;

// Rotate the NB-byte array held in NW 32-bit words left by r bytes
// (0 <= r < 16): byte i of the result is byte (i + r) mod NB of the input.
template <int NW>
__device__ __forceinline__ void rotate_bytes(uint32_t (&w)[NW], int r) {
  const int rw = r >> 2, rb = r & 3;
  uint32_t t[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) t[i] = (rw & 1) ? w[(i + 1) % NW] : w[i];
#pragma unroll
  for (int i = 0; i < NW; ++i) w[i] = (rw & 2) ? t[(i + 2) % NW] : t[i];
#pragma unroll
  for (int i = 0; i < NW; ++i)
    t[i] = __builtin_amdgcn_alignbyte(w[(i + 1) % NW], w[i], rb);
#pragma unroll
  for (int i = 0; i < NW; ++i) w[i] = t[i];
}

template <int G>
__device__ __forceinline__ void lds_load_group(const float* p, float (&o)[G]) {
  if constexpr (G == 4) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
  } else if constexpr (G == 8) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    const float4 y = *reinterpret_cast<const float4*>(p + 4);
    o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
    o[4] = y.x; o[5] = y.y; o[6] = y.z; o[7] = y.w;
  } else if constexpr (G == 2) {
    const float2 x = *reinterpret_cast<const float2*>(p);
    o[0] = x.x; o[1] = x.y;
  } else {
    o[0] = p[0];
  }
}

// Block -> (batch*KV head, key segment), placing all segments of one head
// on the same XCD (blocks are dealt to the 8 XCDs round-robin) so the head's
// probability table is fetched into that XCD's L2 once.
__device__ __forceinline__ bool score_block_coords(int bhkv, int segs, int& bg,
                                                   int& seg) {
  const int total = bhkv * segs;
  const int per_xcd = (total + 7) / 8;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int li = xcd * per_xcd + slot;
  if (slot >= per_xcd || li >= total) return false;
  bg = li / segs;
  seg = li % segs;
  return true;
}

// Shared tail of both kernels: store the G scores of key n and count them.
template <int G>
__device__ __forceinline__ void emit_scores(const float (&acc)[G], float vn,
                                            int64_t n, int64_t n_keys,
                                            float* srow, uint32_t* hloc) {
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float s = vn * acc[j];
    srow[(int64_t)j * n_keys + n] = s;
    if (hloc) {
      const uint32_t bin = float_order_key(s) >> 21;
      atomicAdd(hloc + j * (kHistBins / 2) + (bin >> 1), 1u << ((bin & 1) * 16));
    }
  }
}

template <int G>
__device__ __forceinline__ void flush_hist(const uint32_t* hloc, uint32_t* hrow) {
  for (int i = threadIdx.x; i < G * kHistBins; i += blockDim.x) {
    const int j = i / kHistBins, bin = i % kHistBins;
    const uint32_t v = (hloc[j * (kHistBins / 2) + (bin >> 1)] >> ((bin & 1) * 16)) & 0xffffu;
    if (v) atomicAdd(hrow + (int64_t)j * kHistBins + bin, v);
  }
}

// Fast path: L a multiple of 16 (LW = L/4 words of ids per key).
template <int G, int LW>
__global__ __launch_bounds__(kScoreThreads) void score_kernel_rot(
    const float* __restrict__ table, const uint8_t* __restrict__ ids,
    const float* __restrict__ vnorm, int Hq, int Hkv, int bhkv,
    int64_t n_keys, int64_t stride, int P, int segs, int64_t seg_len,
    float* __restrict__ scores, uint32_t* __restrict__ hist) {
  constexpr int L = LW * 4;
  extern __shared__ __align__(16) float tab[];
  int bg, seg;
  if (!score_block_coords(bhkv, segs, bg, seg)) return;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tsize = (1 << P) * L * G;
  uint32_t* hloc = hist ? reinterpret_cast<uint32_t*>(tab + tsize) : nullptr;

  {
    const float4* src = reinterpret_cast<const float4*>(table + (int64_t)bg * tsize);
    float4* dst = reinterpret_cast<float4*>(tab);
    for (int i = threadIdx.x; i < tsize / 4; i += kScoreThreads) dst[i] = src[i];
    if (hloc)
      for (int i = threadIdx.x; i < G * kHistBins / 2; i += kScoreThreads) hloc[i] = 0u;
  }
  __syncthreads();

  const int64_t n0 = seg * seg_len;
  const int64_t n1 = min(n_keys, n0 + seg_len);
  const uint8_t* idrow = ids + (int64_t)bg * stride * L;
  const float* vrow = vnorm + (int64_t)bg * stride;
  float* srow = scores + ((int64_t)b * Hq + (int64_t)g * G) * n_keys;
  const uint32_t umask = (1u << P) - 1u;  // ids are < 2^P; never index past the table

  // ids and norm of the next key are loaded while the current one is scored
  uint4 nxt[LW / 4];
  float nxt_vn = 0.f;
  int64_t n = n0 + threadIdx.x;
  if (n < n1) {
    const uint4* src = reinterpret_cast<const uint4*>(idrow + n * L);
#pragma unroll
    for (int i = 0; i < LW / 4; ++i) nxt[i] = src[i];
    nxt_vn = vrow[n];
  }
  for (; n < n1; n += kScoreThreads) {
    uint32_t w[LW];
#pragma unroll
    for (int i = 0; i < LW / 4; ++i) {
      w[4 * i] = nxt[i].x; w[4 * i + 1] = nxt[i].y;
      w[4 * i + 2] = nxt[i].z; w[4 * i + 3] = nxt[i].w;
    }
    const float vn = nxt_vn;
    const int64_t n2 = n + kScoreThreads;
    if (n2 < n1) {
      const uint4* src = reinterpret_cast<const uint4*>(idrow + n2 * L);
#pragma unroll
      for (int i = 0; i < LW / 4; ++i) nxt[i] = src[i];
      nxt_vn = vrow[n2];
    }
    const int r = (int)(n & 15);
    rotate_bytes<LW>(w, r);
    float acc[G];
#pragma unroll
    for (int j = 0; j < G; ++j) acc[j] = 0.f;
#pragma unroll
    for (int t = 0; t < L; ++t) {
      const uint32_t u = (w[t >> 2] >> ((t & 3) * 8)) & umask;
      const int l = (t + r) & (L - 1);
      float pr[G];
      lds_load_group<G>(tab + ((int)u * L + l) * G, pr);
#pragma unroll
      for (int j = 0; j < G; ++j) acc[j] += pr[j];
    }
    emit_scores<G>(acc, vn, n, n_keys, srow, hloc);
  }
  if (hloc) {
    __syncthreads();
    flush_hist<G>(hloc, hist + ((int64_t)b * Hq + (int64_t)g * G) * kHistBins);
  }
}

// General path: any L (no bank rotation, byte loads of the ids).
template <int G>
__global__ __launch_bounds__(kScoreThreads) void score_kernel_generic(
    const float* __restrict__ table, const uint8_t* __restrict__ ids,
    const float* __restrict__ vnorm, int Hq, int Hkv, int bhkv,
    int64_t n_keys, int64_t stride, int L, int P, int segs, int64_t seg_len,
    float* __restrict__ scores, uint32_t* __restrict__ hist) {
  extern __shared__ __align__(16) float tab[];
  int bg, seg;
  if (!score_block_coords(bhkv, segs, bg, seg)) return;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tsize = (1 << P) * L * G;
  uint32_t* hloc = hist ? reinterpret_cast<uint32_t*>(tab + tsize) : nullptr;
  for (int i = threadIdx.x; i < tsize; i += kScoreThreads)
    tab[i] = table[(int64_t)bg * tsize + i];
  if (hloc)
    for (int i = threadIdx.x; i < G * kHistBins / 2; i += kScoreThreads) hloc[i] = 0u;
  __syncthreads();

  const int64_t n0 = seg * seg_len;
  const int64_t n1 = min(n_keys, n0 + seg_len);
  const uint8_t* idrow = ids + (int64_t)bg * stride * L;
  const float* vrow = vnorm + (int64_t)bg * stride;
  float* srow = scores + ((int64_t)b * Hq + (int64_t)g * G) * n_keys;
  for (int64_t n = n0 + threadIdx.x; n < n1; n += kScoreThreads) {
    float acc[G];
#pragma unroll
    for (int j = 0; j < G; ++j) acc[j] = 0.f;
    for (int l = 0; l < L; ++l) {
      const int u = idrow[n * L + l] & ((1 << P) - 1);
      float pr[G];
#pragma unroll
      for (int j = 0; j < G; ++j) pr[j] = tab[(u * L + l) * G + j];
#pragma unroll
      for (int j = 0; j < G; ++j) acc[j] += pr[j];
    }
    emit_scores<G>(acc, vrow[n], n, n_keys, srow, hloc);
  }
  if (hloc) {
    __syncthreads();
    flush_hist<G>(hloc, hist + ((int64_t)b * Hq + (int64_t)g * G) * kHistBins);
  }
}

template <int G>
hipError_t launch_score_g(const float* table, const uint8_t* ids,
                          const float* vnorm, int B, int Hq, int Hkv,
                          int64_t n_keys, int64_t stride, int L, int P,
                          float* scores, uint32_t* hist, hipStream_t stream) {
  const int bhkv = B * Hkv;
  const size_t lds = score_lds_bytes(L, P, G, hist != nullptr);
  // blocks resident per CU as limited by the 160 KB of LDS
  const int per_cu = (int)std::max<size_t>(1, std::min<size_t>(2, (160 * 1024) / lds));
  const int64_t target = (int64_t)256 * per_cu;
  int64_t segs = (target + bhkv - 1) / bhkv;
  segs = std::max<int64_t>(1, std::min<int64_t>(segs, (n_keys + 2047) / 2048));
  if (hist) segs = std::max<int64_t>(segs, (n_keys + kMaxSegForHist - 1) / kMaxSegForHist);
  int64_t seg_len = (n_keys + segs - 1) / segs;
  seg_len = (seg_len + 1023) / 1024 * 1024;
  if (hist && seg_len > kMaxSegForHist) seg_len = kMaxSegForHist;
  segs = (n_keys + seg_len - 1) / seg_len;
  const int total = (int)(bhkv * segs);
  const int grid = ((total + 7) / 8) * 8;
  static bool attr_set = false;
  if (!attr_set) {
    // allow up to the full 160 KB of LDS for the staged table
    const int max_lds = 160 * 1024;
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&score_kernel_rot<G, 8>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&score_kernel_rot<G, 16>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&score_kernel_rot<G, 4>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&score_kernel_generic<G>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    attr_set = true;
  }
  const bool aligned = (reinterpret_cast<uintptr_t>(ids) % 16 == 0) &&
                       ((stride * L) % 16 == 0);
  if (aligned && L == 32) {
    hipLaunchKernelGGL((score_kernel_rot<G, 8>), dim3(grid), dim3(kScoreThreads),
                       lds, stream, table, ids, vnorm, Hq, Hkv, bhkv, n_keys,
                       stride, P, (int)segs, seg_len, scores, hist);
    trace_mark(stream);
  } else if (aligned && L == 64) {
    hipLaunchKernelGGL((score_kernel_rot<G, 16>), dim3(grid), dim3(kScoreThreads),
                       lds, stream, table, ids, vnorm, Hq, Hkv, bhkv, n_keys,
                       stride, P, (int)segs, seg_len, scores, hist);
    trace_mark(stream);
  } else if (aligned && L == 16) {
    hipLaunchKernelGGL((score_kernel_rot<G, 4>), dim3(grid), dim3(kScoreThreads),
                       lds, stream, table, ids, vnorm, Hq, Hkv, bhkv, n_keys,
                       stride, P, (int)segs, seg_len, scores, hist);
    trace_mark(stream);
  } else {
    hipLaunchKernelGGL((score_kernel_generic<G>), dim3(grid), dim3(kScoreThreads),
                       lds, stream, table, ids, vnorm, Hq, Hkv, bhkv, n_keys,
                       stride, L, P, (int)segs, seg_len, scores, hist);
    trace_mark(stream);
  }
  return hipGetLastError();
}

}  // namespace

size_t score_lds_bytes(int L, int P, int G, bool with_hist) {
  return (size_t)(1 << P) * L * G * sizeof(float) +
         (with_hist ? (size_t)G * kHistBins / 2 * sizeof(uint32_t) : 0);
}

hipError_t launch_score(const float* table, const uint8_t* ids,
                        const float* vnorm, int B, int Hq, int Hkv,
                        int64_t n_keys, int64_t stride, int L, int P,
                        float* scores, uint32_t* hist, hipStream_t stream) {
  if (n_keys == 0) return hipSuccess;
  switch (Hq / Hkv) {
    case 1:
      return launch_score_g<1>(table, ids, vnorm, B, Hq, Hkv, n_keys, stride,
                               L, P, scores, hist, stream);
    case 2:
      return launch_score_g<2>(table, ids, vnorm, B, Hq, Hkv, n_keys, stride,
                               L, P, scores, hist, stream);
    case 4:
      return launch_score_g<4>(table, ids, vnorm, B, Hq, Hkv, n_keys, stride,
                               L, P, scores, hist, stream);
    case 8:
      return launch_score_g<8>(table, ids, vnorm, B, Hq, Hkv, n_keys, stride,
                               L, P, scores, hist, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace socket_lsh

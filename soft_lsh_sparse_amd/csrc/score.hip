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
// copies that head's probability table [2^P][L][G] (float32, from the bucket
// kernel) into LDS, then streams the bucket-id rows (L bytes per key,
// coalesced across lanes) and the value norms from HBM, several iterations
// ahead in registers so that enough bytes are in flight to cover the memory
// latency. Each id byte is looked up once for the whole GQA group: the G
// probabilities of the group sit in one 16-byte LDS slot.
//
// Bank spread: with the [u][l][G] layout and L a multiple of 16, the LDS bank
// group of slot (u, l) depends only on l mod 8 (32 banks of 4 bytes, 16-byte
// slots). Lane i walks the tables in the rotated order l = (t + n) mod L for
// its key n (n mod 8 = i mod 8), so the 8 lanes the LDS serves together hit 8
// different bank groups whatever buckets the keys fall in. The rotation is
// applied to the id bytes in registers once per key; the slot offset of step
// t is a per-lane base (two candidates, before and after the wrap) plus a
// compile-time immediate. The L probabilities are summed in float32 in that
// fixed order and multiplied by the value norm.
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

constexpr int kScoreThreads = 512;  // generic path
// Rotated-path blocks: 16 waves, the most one CU holds at <= 128 VGPRs,
// with two iterations of ids and norms in flight per thread.
constexpr int kRotThreads = 1024;
constexpr int kPrefetch = 2;
constexpr int64_t kMaxSegForHist = 32768;
// keeps every per-thread byte offset of a segment (key * L, L <= 1024) in 31 bits
constexpr int64_t kMaxSeg = 1 << 20;

// v_cndmask_b32 with an explicit lane mask: b where the lane's mask bit is
// set, a elsewhere. Written out so the compiler keeps one select per word
// instead of rewriting the rotation below as a dynamically indexed array.
__device__ __forceinline__ uint32_t select_lanes(uint32_t a, uint32_t b, uint64_t mask) {
  uint32_t out;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(out) : "v"(a), "v"(b), "s"(mask));
  return out;
}

// Rotate the NB-byte array held in NW 32-bit words left by r bytes
// (0 <= r < 8): byte i of the result is byte (i + r) mod NB of the input.
// One word-select stage (lanes whose bit is set in by_word: r >= 4) and one
// byte funnel shift per word.
template <int NW>
__device__ __forceinline__ void rotate_bytes(uint32_t (&w)[NW], uint64_t by_word, int rb) {
  uint32_t t[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) t[i] = select_lanes(w[i], w[(i + 1) % NW], by_word);
#pragma unroll
  for (int i = 0; i < NW; ++i)
    w[i] = __builtin_amdgcn_alignbyte(t[(i + 1) % NW], t[i], rb);
}

// Ties the next ids to the running sums (empty asm, no instruction): every
// sum is complete before this point, and the words w[k0 .. k1) cannot be
// used, hence no lookup of theirs issued, before it. Keeps the compiler
// from issuing all lookups of a key at once and from deferring the sums,
// either of which holds one register per looked-up float.
template <int G, int LW>
__device__ __forceinline__ void fence_chunk(float (&acc)[G], uint32_t (&w)[LW], int k0,
                                            int k1) {
#pragma unroll
  for (int j = 0; j < G; ++j) asm volatile("" : "+v"(acc[j]), "+v"(w[k0]));
#pragma unroll
  for (int k = k0 + 1; k < k1; ++k) asm volatile("" : "+v"(w[k]) : "v"(w[k0]));
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

// The table of batch*KV head bg into LDS, and the packed histogram cleared.
template <int G>
__device__ __forceinline__ void stage_table(float* tab, const float* table, int bg,
                                            int L, int P, uint32_t* hloc) {
  const int tsize = (1 << P) * L * G;
  if (tsize % 4 == 0) {  // every head's table then starts 16-byte aligned
    const float4* src = reinterpret_cast<const float4*>(table + (int64_t)bg * tsize);
    float4* dst = reinterpret_cast<float4*>(tab);
    for (int i = threadIdx.x; i < tsize / 4; i += blockDim.x) dst[i] = src[i];
  } else {
    for (int i = threadIdx.x; i < tsize; i += blockDim.x)
      tab[i] = table[(int64_t)bg * tsize + i];
  }
  if (hloc)
    for (int i = threadIdx.x; i < G * kHistBins / 2; i += blockDim.x) hloc[i] = 0u;
}

// Shared tail: store the G scores of key n and count them.
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

struct ScoreArgs {
  const float* table;  // [bhkv][2^P][L][G]
  const uint8_t* ids;
  const float* vnorm;
  int Hq, Hkv, bhkv, P, segs;
  int64_t n_keys, stride, seg_len;
  float* scores;
  uint32_t* hist;
};

// Fast path: L a multiple of 16 (LW = L/4 words of ids per key).
template <int G, int LW>
__global__ __launch_bounds__(kRotThreads) void score_kernel_rot(ScoreArgs a) {
  constexpr int kThreads = kRotThreads;
  constexpr int L = LW * 4;
  constexpr int kChunk = 64 / G;  // lookups per dependency step (a multiple of 4)
  extern __shared__ __align__(16) float tab[];
  int bg, seg;
  if (!score_block_coords(a.bhkv, a.segs, bg, seg)) return;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int P = a.P;
  const int tsize = (1 << P) * L * G;
  uint32_t* hloc = a.hist ? reinterpret_cast<uint32_t*>(tab + tsize) : nullptr;

  // block-uniform bases of this segment; per-thread offsets stay 32-bit
  const int64_t n0 = seg * a.seg_len;
  const int cnt = (int)(min(a.n_keys, n0 + a.seg_len) - n0);
  const uint8_t* idseg = a.ids + ((int64_t)bg * a.stride + n0) * L;
  const float* vseg = a.vnorm + (int64_t)bg * a.stride + n0;
  float* sseg = a.scores + ((int64_t)b * a.Hq + (int64_t)g * G) * a.n_keys + n0;

  // the first kPrefetch iterations of ids and norms go in flight before the
  // table is staged
  uint4 pf[kPrefetch][LW / 4];
  float pf_vn[kPrefetch];
  const int first = threadIdx.x;
#pragma unroll
  for (int q = 0; q < kPrefetch; ++q) {
    const int i = first + q * kThreads;
    pf_vn[q] = 0.f;
    if (i < cnt) {
      const uint4* src = reinterpret_cast<const uint4*>(idseg + i * L);
#pragma unroll
      for (int k = 0; k < LW / 4; ++k) pf[q][k] = src[k];
      pf_vn[q] = vseg[i];
    }
  }
  stage_table<G>(tab, a.table, bg, L, P, hloc);
  __syncthreads();

  // n0 and the thread stride are multiples of 8, so every key of this
  // thread has the same rotation r = key index mod 8 and the same two bases
  const int r = first & 7;
  const uint64_t by_word = __ballot(r >= 4);
  const int rb = r & 3;
  const int base_nowrap = r * G;        // slot offset of step t: t*G + base
  const int base_wrap = (r - L) * G;    // ... once t + r >= L
  for (int bi = first; bi < cnt; bi += kPrefetch * kThreads) {
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q) {
      const int i = bi + q * kThreads;
      if (i < cnt) {
        uint32_t w[LW];
#pragma unroll
        for (int k = 0; k < LW / 4; ++k) {
          w[4 * k] = pf[q][k].x; w[4 * k + 1] = pf[q][k].y;
          w[4 * k + 2] = pf[q][k].z; w[4 * k + 3] = pf[q][k].w;
        }
        const float vn = pf_vn[q];
        const int ii = i + kPrefetch * kThreads;
        if (ii < cnt) {
          const uint4* src = reinterpret_cast<const uint4*>(idseg + ii * L);
#pragma unroll
          for (int k = 0; k < LW / 4; ++k) pf[q][k] = src[k];
          pf_vn[q] = vseg[ii];
        }
        rotate_bytes<LW>(w, by_word, rb);
        float acc[G];
#pragma unroll
        for (int t = 0; t < L; ++t) {
          // P bits of byte t: ids are < 2^P, so this never leaves the table
          const uint32_t u = __builtin_amdgcn_ubfe(w[t >> 2], (t & 3) * 8, P);
          const int base = (t + 7 < L) ? base_nowrap
                                       : (t + r < L ? base_nowrap : base_wrap);
          float pr[G];
          lds_load_group<G>(tab + (int)u * (L * G) + base + t * G, pr);
#pragma unroll
          for (int j = 0; j < G; ++j) acc[j] = t == 0 ? pr[j] : acc[j] + pr[j];
          // the next kChunk lookups wait for these sums: at most 64 floats
          // of lookups in flight per lane, which bounds the registers
          if ((t + 1) % kChunk == 0 && t + 1 < L)
            fence_chunk<G, LW>(acc, w, (t + 1) / 4, std::min(LW, (t + 1 + kChunk) / 4));
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float sc = vn * acc[j];
          sseg[(int64_t)j * a.n_keys + i] = sc;
          if (hloc) {
            const uint32_t bin = float_order_key(sc) >> 21;
            atomicAdd(hloc + j * (kHistBins / 2) + (bin >> 1), 1u << ((bin & 1) * 16));
          }
        }
      }
    }
  }
  if (hloc) {
    __syncthreads();
    flush_hist<G>(hloc, a.hist + ((int64_t)b * a.Hq + (int64_t)g * G) * kHistBins);
  }
}

// General path: any L (no bank rotation, byte loads of the ids).
template <int G>
__global__ __launch_bounds__(kScoreThreads) void score_kernel_generic(ScoreArgs a, int L) {
  extern __shared__ __align__(16) float tab[];
  int bg, seg;
  if (!score_block_coords(a.bhkv, a.segs, bg, seg)) return;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int P = a.P;
  const int tsize = (1 << P) * L * G;
  uint32_t* hloc = a.hist ? reinterpret_cast<uint32_t*>(tab + tsize) : nullptr;
  stage_table<G>(tab, a.table, bg, L, P, hloc);
  __syncthreads();

  const int64_t n0 = seg * a.seg_len;
  const int64_t n1 = min(a.n_keys, n0 + a.seg_len);
  const uint8_t* idrow = a.ids + (int64_t)bg * a.stride * L;
  const float* vrow = a.vnorm + (int64_t)bg * a.stride;
  float* srow = a.scores + ((int64_t)b * a.Hq + (int64_t)g * G) * a.n_keys;
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
    emit_scores<G>(acc, vrow[n], n, a.n_keys, srow, hloc);
  }
  if (hloc) {
    __syncthreads();
    flush_hist<G>(hloc, a.hist + ((int64_t)b * a.Hq + (int64_t)g * G) * kHistBins);
  }
}

template <int G>
void set_lds_attributes() {
  static bool done = false;
  if (done) return;
  const int max_lds = (int)kLdsBytesPerCU;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&score_kernel_rot<G, 8>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&score_kernel_rot<G, 16>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&score_kernel_rot<G, 4>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&score_kernel_generic<G>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
  done = true;
}

template <int G>
hipError_t launch_score_g(ScoreArgs a, int L, hipStream_t stream) {
  const size_t lds = score_lds_bytes(L, a.P, G, a.hist != nullptr);
  // blocks resident per CU as limited by the 160 KB of LDS
  const int per_cu = (int)std::max<size_t>(1, std::min<size_t>(2, kLdsBytesPerCU / lds));
  const int64_t target = (int64_t)256 * per_cu;
  const int64_t n_keys = a.n_keys;
  int64_t segs = (target + a.bhkv - 1) / a.bhkv;
  segs = std::max<int64_t>(1, std::min<int64_t>(segs, (n_keys + 2047) / 2048));
  if (a.hist) segs = std::max<int64_t>(segs, (n_keys + kMaxSegForHist - 1) / kMaxSegForHist);
  int64_t seg_len = (n_keys + segs - 1) / segs;
  seg_len = (seg_len + 1023) / 1024 * 1024;
  if (a.hist && seg_len > kMaxSegForHist) seg_len = kMaxSegForHist;
  if (seg_len > kMaxSeg) seg_len = kMaxSeg;
  segs = (n_keys + seg_len - 1) / seg_len;
  a.segs = (int)segs;
  a.seg_len = seg_len;
  const int total = (int)(a.bhkv * segs);
  const int grid = ((total + 7) / 8) * 8;
  set_lds_attributes<G>();
  const bool aligned = (reinterpret_cast<uintptr_t>(a.ids) % 16 == 0) &&
                       ((a.stride * L) % 16 == 0);
  if (aligned && L == 32) {
    launch_kernel((score_kernel_rot<G, 8>), dim3(grid), dim3(kRotThreads), lds,
                       stream, a);
  } else if (aligned && L == 64) {
    launch_kernel((score_kernel_rot<G, 16>), dim3(grid), dim3(kRotThreads), lds,
                       stream, a);
  } else if (aligned && L == 16) {
    launch_kernel((score_kernel_rot<G, 4>), dim3(grid), dim3(kRotThreads), lds,
                       stream, a);
  } else {
    launch_kernel((score_kernel_generic<G>), dim3(grid), dim3(kScoreThreads), lds,
                       stream, a, L);
  }
  return hipGetLastError();
}

}  // namespace

size_t score_lds_bytes(int L, int P, int G, bool with_hist) {
  return (size_t)(1 << P) * L * G * sizeof(float) +
         (with_hist ? (size_t)G * kHistBins / 2 * sizeof(uint32_t) : 0);
}

hipError_t launch_score(const float* table, const uint8_t* ids, const float* vnorm,
                        int B, int Hq, int Hkv, int64_t n_keys, int64_t stride,
                        int L, int P, float* scores, uint32_t* hist,
                        hipStream_t stream) {
  if (n_keys == 0) return hipSuccess;
  ScoreArgs a{};
  a.table = table;
  a.ids = ids;
  a.vnorm = vnorm;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.bhkv = B * Hkv;
  a.P = P;
  a.n_keys = n_keys;
  a.stride = stride;
  a.scores = scores;
  a.hist = hist;
  switch (Hq / Hkv) {
    case 1: return launch_score_g<1>(a, L, stream);
    case 2: return launch_score_g<2>(a, L, stream);
    case 4: return launch_score_g<4>(a, L, stream);
    case 8: return launch_score_g<8>(a, L, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace socket_lsh
